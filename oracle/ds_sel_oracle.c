/*
 * ds_sel_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, single-threaded CPU definition of compressed-attention block
 * selection.  Only the test-suite, the package smoke check and the
 * benchmark's CPU-baseline leg may load it.  The GPU library neither links
 * nor calls it, and the two share no source, header, table or helper.
 *
 * What it computes (the pages give the problem, not the formula):
 *   Page "DeepSeek V4.1F Q4 on M3 Ultra with native DSpark MTP (40tps /
 *   800tps)", paragraph "Decode at depth": in each layer the compressed
 *   attention keeps 512 compressed blocks chosen from the whole context;
 *   a block is a candidate only if the layer's mask lets it through; the
 *   admitted index is built per query row; the 512 best candidates are kept.
 *   The same fact appears on page "DeepSeek V4.1 Flash on M3 Ultra nearly
 *   doubles decode to 31 t/s with first public DSpark Metal port",
 *   paragraph "Key techniques".
 *
 * Readings taken where the pages are silent (each is also listed with the
 * other readings in the design notes):
 *   - score(b) = sum over heads h of w[h] * (q[h] . K[b]), every operation
 *     an fp32 IEEE round-to-nearest-even operation, in the fixed order
 *     written in score_fp32() below;
 *   - admitted(b) = (no mask, or mask bit b set) and b < clamp(limit, 0, N);
 *   - "best" is the total order: higher score first, equal scores broken by
 *     the lower block index;
 *   - the output holds the first min(k, admitted) blocks of that order, then
 *     padding (index -1, score -inf); count = min(k, admitted).
 *
 * This is the plain definition: build the admitted list, score every member,
 * sort with the C library's qsort, keep the head.  No blocking, no fusion,
 * no radix passes.  Build with -O2 -ffp-contract=off and without fast-math
 * so that every fp32 operation is a separately rounded IEEE operation.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_OK 0
#define ORACLE_E_INVALID (-1)
#define ORACLE_E_NONFINITE (-2)
#define ORACLE_E_NOMEM (-3)

/* bf16 is the top half of an IEEE binary32, so widening is exact. */
static float bf16_bits_to_float(uint16_t bits) {
  uint32_t u = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return f;
}

/* Mask bit b of one (layer, row): bit (b mod 32) of 32-bit word floor(b/32),
 * least significant bit first. */
static int mask_bit(const uint32_t* row_words, int64_t b) {
  return (int)((row_words[b >> 5] >> (uint32_t)(b & 31)) & 1u);
}

/* The per-row causal limit, clamped to [0, N]; no limit array admits all. */
static int64_t clamped_limit(const int32_t* limit, int64_t lr, int64_t n_blocks) {
  if (!limit) return n_blocks;
  int64_t v = limit[lr];
  if (v < 0) v = 0;
  if (v > n_blocks) v = n_blocks;
  return v;
}

/* The score of one block for one (layer, row), in the fixed fp32 order:
 *   s = +0
 *   for h = 0..H-1:
 *     dot = +0;  for i = 0..d-1: dot = dot + q[h][i]*K[i]
 *     t = w[h]*dot;  s = s + t
 * The bf16 x bf16 products are exact in fp32, the sums and w*dot are rounded.
 * The canonical zero is +0 (adding +0 turns a -0 into +0). */
static float score_fp32(const uint16_t* q_row, const uint16_t* w_row, const uint16_t* key,
                        int heads, int dim) {
  float s = 0.0f;
  for (int h = 0; h < heads; ++h) {
    const uint16_t* qh = q_row + (int64_t)h * dim;
    float dot = 0.0f;
    for (int i = 0; i < dim; ++i) {
      float prod = bf16_bits_to_float(qh[i]) * bf16_bits_to_float(key[i]);
      dot = dot + prod;
    }
    float t = bf16_bits_to_float(w_row[h]) * dot;
    s = s + t;
  }
  return s + 0.0f;
}

typedef struct {
  float score;
  int32_t block;
} scored_block;

/* Total order: higher score first; equal scores by lower block index. */
static int by_score_desc_then_index(const void* pa, const void* pb) {
  const scored_block* a = (const scored_block*)pa;
  const scored_block* b = (const scored_block*)pb;
  if (a->score > b->score) return -1;
  if (a->score < b->score) return 1;
  if (a->block < b->block) return -1;
  if (a->block > b->block) return 1;
  return 0;
}

static int inputs_finite(int64_t n, const uint16_t* bits, int64_t stride_rows, int64_t row_len) {
  for (int64_t r = 0; r < n; ++r)
    for (int64_t i = 0; i < row_len; ++i)
      if ((bits[r * stride_rows + i] & 0x7F80u) == 0x7F80u) return 0;
  return 1;
}

/*
 * Top-k block selection for every (layer, row).
 *
 * q      bf16 bits [layers][rows][heads][dim]            (contiguous)
 * w      bf16 bits [layers][rows][heads]                 (contiguous)
 * keys   bf16 bits; block b of layer l starts at keys + l*key_layer_stride + b*ldk
 * mask   NULL, or u32 words; (l, r) row starts at mask + l*mask_layer_stride
 *        + r*mask_row_stride and holds at least ceil(blocks/32) words
 * limit  NULL, or int32 [layers][rows]
 * out_idx   int32 [layers][rows][k]
 * out_score float [layers][rows][k]
 * out_count int32 [layers][rows] (may be NULL)
 *
 * Returns 0, or a negative code: -1 bad argument, -2 a non-finite bf16
 * input, -3 out of host memory.
 */
int ds_sel_oracle_select(int32_t layers, int32_t rows, int32_t heads, int32_t dim, int64_t blocks,
                         int32_t k, const uint16_t* q, const uint16_t* w, const uint16_t* keys,
                         int64_t ldk, int64_t key_layer_stride, const uint32_t* mask,
                         int64_t mask_row_stride, int64_t mask_layer_stride, const int32_t* limit,
                         int32_t* out_idx, float* out_score, int32_t* out_count) {
  if (layers < 1 || rows < 1 || heads < 1 || dim < 1 || blocks < 0 || k < 1) return ORACLE_E_INVALID;
  if (ldk < dim || !q || !w || !out_idx || !out_score) return ORACLE_E_INVALID;
  if (blocks > 0 && !keys) return ORACLE_E_INVALID;
  if (blocks > 0x7FFFFFFFLL) return ORACLE_E_INVALID;

  if (!inputs_finite((int64_t)layers * rows * heads, q, dim, dim)) return ORACLE_E_NONFINITE;
  if (!inputs_finite((int64_t)layers * rows, w, heads, heads)) return ORACLE_E_NONFINITE;
  for (int32_t l = 0; l < layers; ++l)
    if (blocks > 0 && !inputs_finite(blocks, keys + l * key_layer_stride, ldk, dim))
      return ORACLE_E_NONFINITE;

  scored_block* list = NULL;
  if (blocks > 0) {
    list = (scored_block*)malloc((size_t)blocks * sizeof *list);
    if (!list) return ORACLE_E_NOMEM;
  }

  for (int32_t l = 0; l < layers; ++l) {
    const uint16_t* layer_keys = keys ? keys + l * key_layer_stride : NULL;
    for (int32_t r = 0; r < rows; ++r) {
      int64_t lr = (int64_t)l * rows + r;
      const uint16_t* q_row = q + lr * heads * dim;
      const uint16_t* w_row = w + lr * heads;
      const uint32_t* mrow = mask ? mask + l * mask_layer_stride + r * mask_row_stride : NULL;
      int64_t lim = clamped_limit(limit, lr, blocks);

      /* 1. The admitted list, ascending in block index. */
      int64_t n = 0;
      for (int64_t b = 0; b < lim; ++b) {
        if (mrow && !mask_bit(mrow, b)) continue;
        list[n].block = (int32_t)b;
        ++n;
      }
      /* 2. Score every admitted block. */
      for (int64_t j = 0; j < n; ++j)
        list[j].score = score_fp32(q_row, w_row, layer_keys + (int64_t)list[j].block * ldk, heads, dim);
      /* 3. Sort by the total order and keep the first min(k, n). */
      if (n > 1) qsort(list, (size_t)n, sizeof *list, by_score_desc_then_index);
      int64_t m = n < k ? n : k;
      int32_t* oi = out_idx + lr * k;
      float* os = out_score + lr * k;
      for (int64_t j = 0; j < k; ++j) {
        if (j < m) {
          oi[j] = list[j].block;
          os[j] = list[j].score;
        } else {
          oi[j] = -1;
          os[j] = -INFINITY;
        }
      }
      if (out_count) out_count[lr] = (int32_t)m;
    }
  }
  free(list);
  return ORACLE_OK;
}

/*
 * The fp32 score (same order as above) of each listed block for one
 * (layer, row), admitted or not.  Used to judge a GPU-selected block that the
 * oracle itself did not select.  Returns 0 or -1 for a bad argument.
 */
int ds_sel_oracle_score_blocks(int32_t layers, int32_t rows, int32_t heads, int32_t dim,
                               int64_t blocks, const uint16_t* q, const uint16_t* w,
                               const uint16_t* keys, int64_t ldk, int64_t key_layer_stride,
                               int32_t layer, int32_t row, int64_t n_list, const int32_t* list,
                               float* out) {
  if (layer < 0 || layer >= layers || row < 0 || row >= rows || n_list < 0) return ORACLE_E_INVALID;
  if (heads < 1 || dim < 1 || ldk < dim) return ORACLE_E_INVALID;
  int64_t lr = (int64_t)layer * rows + row;
  for (int64_t j = 0; j < n_list; ++j) {
    if (list[j] < 0 || list[j] >= blocks) return ORACLE_E_INVALID;
    out[j] = score_fp32(q + lr * heads * dim, w + lr * heads,
                        keys + layer * key_layer_stride + (int64_t)list[j] * ldk, heads, dim);
  }
  return ORACLE_OK;
}

/*
 * The per-head ReLU score (a non-linear variant).
 *
 * The pages give no score formula (page "DeepSeek V4.1F Q4 on M3 Ultra with
 * native DSpark MTP (40tps / 800tps)", paragraph "Decode at depth": blocks
 * are scored and the best kept).  This variant clamps each head's dot product
 * at zero before weighting:
 *   score(b) = sum over heads h of w[h] * max(q[h] . K[b], 0)
 * so the heads can no longer be folded into one query vector.  Same fixed
 * fp32 order as score_fp32():
 *   s = +0
 *   for h = 0..H-1:
 *     dot = +0;  for i = 0..d-1: dot = dot + q[h][i]*K[i]
 *     r = dot if dot > 0, else +0
 *     t = w[h]*r;  s = s + t
 * Admission, order, output and padding are those of ds_sel_oracle_select.
 */
static float score_relu_fp32(const uint16_t* q_row, const uint16_t* w_row, const uint16_t* key,
                             int heads, int dim) {
  float s = 0.0f;
  for (int h = 0; h < heads; ++h) {
    const uint16_t* qh = q_row + (int64_t)h * dim;
    float dot = 0.0f;
    for (int i = 0; i < dim; ++i) {
      float prod = bf16_bits_to_float(qh[i]) * bf16_bits_to_float(key[i]);
      dot = dot + prod;
    }
    float r = dot > 0.0f ? dot : 0.0f;
    float t = bf16_bits_to_float(w_row[h]) * r;
    s = s + t;
  }
  return s + 0.0f;
}

/* Top-k selection under the per-head ReLU score; arguments and returns as
 * ds_sel_oracle_select. */
int ds_sel_oracle_select_relu(int32_t layers, int32_t rows, int32_t heads, int32_t dim,
                              int64_t blocks, int32_t k, const uint16_t* q, const uint16_t* w,
                              const uint16_t* keys, int64_t ldk, int64_t key_layer_stride,
                              const uint32_t* mask, int64_t mask_row_stride,
                              int64_t mask_layer_stride, const int32_t* limit, int32_t* out_idx,
                              float* out_score, int32_t* out_count) {
  if (layers < 1 || rows < 1 || heads < 1 || dim < 1 || blocks < 0 || k < 1) return ORACLE_E_INVALID;
  if (ldk < dim || !q || !w || !out_idx || !out_score) return ORACLE_E_INVALID;
  if (blocks > 0 && !keys) return ORACLE_E_INVALID;
  if (blocks > 0x7FFFFFFFLL) return ORACLE_E_INVALID;
  if (!inputs_finite((int64_t)layers * rows * heads, q, dim, dim)) return ORACLE_E_NONFINITE;
  if (!inputs_finite((int64_t)layers * rows, w, heads, heads)) return ORACLE_E_NONFINITE;
  for (int32_t l = 0; l < layers; ++l)
    if (blocks > 0 && !inputs_finite(blocks, keys + l * key_layer_stride, ldk, dim))
      return ORACLE_E_NONFINITE;

  scored_block* list = NULL;
  if (blocks > 0) {
    list = (scored_block*)malloc((size_t)blocks * sizeof *list);
    if (!list) return ORACLE_E_NOMEM;
  }
  for (int32_t l = 0; l < layers; ++l) {
    const uint16_t* layer_keys = keys ? keys + l * key_layer_stride : NULL;
    for (int32_t r = 0; r < rows; ++r) {
      int64_t lr = (int64_t)l * rows + r;
      const uint16_t* q_row = q + lr * heads * dim;
      const uint16_t* w_row = w + lr * heads;
      const uint32_t* mrow = mask ? mask + l * mask_layer_stride + r * mask_row_stride : NULL;
      int64_t lim = clamped_limit(limit, lr, blocks);
      int64_t n = 0;
      for (int64_t b = 0; b < lim; ++b) {
        if (mrow && !mask_bit(mrow, b)) continue;
        list[n].block = (int32_t)b;
        ++n;
      }
      for (int64_t j = 0; j < n; ++j)
        list[j].score = score_relu_fp32(q_row, w_row, layer_keys + (int64_t)list[j].block * ldk,
                                        heads, dim);
      if (n > 1) qsort(list, (size_t)n, sizeof *list, by_score_desc_then_index);
      int64_t m = n < k ? n : k;
      int32_t* oi = out_idx + lr * k;
      float* os = out_score + lr * k;
      for (int64_t j = 0; j < k; ++j) {
        oi[j] = j < m ? list[j].block : -1;
        os[j] = j < m ? list[j].score : -INFINITY;
      }
      if (out_count) out_count[lr] = (int32_t)m;
    }
  }
  free(list);
  return ORACLE_OK;
}

/* The per-head ReLU score of each listed block for one (layer, row), as
 * ds_sel_oracle_score_blocks. */
int ds_sel_oracle_score_blocks_relu(int32_t layers, int32_t rows, int32_t heads, int32_t dim,
                                    int64_t blocks, const uint16_t* q, const uint16_t* w,
                                    const uint16_t* keys, int64_t ldk, int64_t key_layer_stride,
                                    int32_t layer, int32_t row, int64_t n_list, const int32_t* list,
                                    float* out) {
  if (layer < 0 || layer >= layers || row < 0 || row >= rows || n_list < 0) return ORACLE_E_INVALID;
  if (heads < 1 || dim < 1 || ldk < dim) return ORACLE_E_INVALID;
  int64_t lr = (int64_t)layer * rows + row;
  for (int64_t j = 0; j < n_list; ++j) {
    if (list[j] < 0 || list[j] >= blocks) return ORACLE_E_INVALID;
    out[j] = score_relu_fp32(q + lr * heads * dim, w + lr * heads,
                             keys + layer * key_layer_stride + (int64_t)list[j] * ldk, heads, dim);
  }
  return ORACLE_OK;
}

/*
 * The 8-bit compressed-key stream.
 *
 * Page "DeepSeek V4.1F Q4 on M3 Ultra with native DSpark MTP (40tps /
 * 800tps)", paragraph "DSpark": the verify rows share one stream of Q8 data.
 * The pages apply Q8 to weights; this library reads it for the block keys:
 * a key row of d values is stored as d/32 groups, each of 32 signed 8-bit
 * codes c and one fp16 scale s, and stands for the values K[i] = s * c[i]
 * (the scale of the group holding column i).  The score is the same
 * definition as for bf16 keys, on those values:
 *   score(b) = sum_h w[h] * (q[h] . K[b]),   K[b][i] = s[b][i/32] * c[b][i]
 * every operation an fp32 round-to-nearest-even operation in the order
 * written in score_q8_fp32(): the value s*c is exact in fp32 (an 11-bit
 * significand times a 7-bit integer), each q*K product and each sum rounded.
 *
 * Quantising a bf16 key row (the encoding, done when a block is written):
 * per group, amax = max |x|; if amax == 0 the scale and codes are 0;
 * otherwise scale = fp16(amax / 127) (fp32 division, then rounded to fp16,
 * nearest-even), and if that scale is 0 the codes are 0; otherwise
 * code = clamp(round-half-away-from-zero(x / scale), -127, 127), the division
 * in fp32.
 */

/* fp16 bits -> fp32 (exact). */
static float half_bits_to_float(uint16_t h) {
  uint32_t sign = (uint32_t)(h >> 15) << 31;
  uint32_t exp = (h >> 10) & 0x1Fu, man = h & 0x3FFu;
  uint32_t u;
  if (exp == 0) {
    if (man == 0) {
      u = sign;
    } else { /* subnormal: man * 2^-24 */
      float f = (float)man * 5.9604644775390625e-08f;
      memcpy(&u, &f, sizeof u);
      u |= sign;
    }
  } else if (exp == 31) {
    u = sign | 0x7F800000u | (man << 13);
  } else {
    u = sign | ((exp + 112u) << 23) | (man << 13);
  }
  float f;
  memcpy(&f, &u, sizeof f);
  return f;
}

/* fp32 -> fp16 bits, round to nearest, ties to even (finite inputs; values
 * beyond the fp16 range become infinity, tiny ones subnormals or zero). */
static uint16_t float_to_half_bits(float f) {
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  uint32_t sign = (u >> 16) & 0x8000u;
  uint32_t a = u & 0x7FFFFFFFu;
  if (a >= 0x47800000u) return (uint16_t)(sign | 0x7C00u); /* >= 65536: overflow */
  if (a < 0x38800000u) {                                 /* below 2^-14: subnormal range */
    /* value = a_float; subnormal half = round(value / 2^-24) */
    float v;
    memcpy(&v, &a, sizeof v);
    float scaled = v * 16777216.0f; /* exact: a power of two */
    /* round half to even on the scaled value (an integer grid) */
    float fl = floorf(scaled);
    float frac = scaled - fl;
    uint32_t m = (uint32_t)fl;
    if (frac > 0.5f || (frac == 0.5f && (m & 1u))) m += 1u;
    return (uint16_t)(sign | m); /* m == 1024 carries into the exponent field correctly */
  }
  uint32_t exp = (a >> 23) - 112u; /* rebias 127 -> 15 */
  uint32_t man = a & 0x7FFFFFu;
  uint32_t h = (exp << 10) | (man >> 13);
  uint32_t rest = man & 0x1FFFu;
  if (rest > 0x1000u || (rest == 0x1000u && (h & 1u))) h += 1u; /* carry may reach infinity */
  return (uint16_t)(sign | h);
}

/*
 * Quantise key rows.  keys bf16 bits, block b of layer l at keys +
 * l*key_layer_stride + b*ldk; codes int8 at codes + l*code_layer_stride +
 * b*ldc; scales fp16 bits at scales + l*scale_layer_stride + b*lds (d/32 per
 * row).  dim must be a multiple of 32.  Returns 0 or -1 for a bad argument.
 */
int ds_sel_oracle_quantize_q8(int32_t layers, int64_t blocks, int32_t dim, const uint16_t* keys,
                              int64_t ldk, int64_t key_layer_stride, int8_t* codes, int64_t ldc,
                              int64_t code_layer_stride, uint16_t* scales, int64_t lds,
                              int64_t scale_layer_stride) {
  if (layers < 1 || blocks < 0 || dim < 32 || dim % 32 != 0 || ldk < dim || ldc < dim ||
      lds < dim / 32)
    return ORACLE_E_INVALID;
  for (int32_t l = 0; l < layers; ++l) {
    for (int64_t b = 0; b < blocks; ++b) {
      const uint16_t* x = keys + l * key_layer_stride + b * ldk;
      int8_t* c = codes + l * code_layer_stride + b * ldc;
      uint16_t* sc = scales + l * scale_layer_stride + b * lds;
      for (int32_t g = 0; g < dim / 32; ++g) {
        float amax = 0.0f;
        for (int i = 0; i < 32; ++i) {
          float v = fabsf(bf16_bits_to_float(x[32 * g + i]));
          if (v > amax) amax = v;
        }
        uint16_t hs = amax == 0.0f ? 0 : float_to_half_bits(amax / 127.0f);
        float s = half_bits_to_float(hs);
        sc[g] = hs;
        for (int i = 0; i < 32; ++i) {
          int code = 0;
          if (s != 0.0f) {
            float r = roundf(bf16_bits_to_float(x[32 * g + i]) / s);
            if (r > 127.0f) r = 127.0f;
            if (r < -127.0f) r = -127.0f;
            code = (int)r;
          }
          c[32 * g + i] = (int8_t)code;
        }
      }
    }
  }
  return ORACLE_OK;
}

/* The score of one block from its 8-bit key row, in the fixed fp32 order:
 *   s = +0
 *   for h = 0..H-1:
 *     dot = +0;  for i = 0..d-1: dot = dot + q[h][i]*(scale[i/32]*code[i])
 *     t = w[h]*dot;  s = s + t                                             */
static float score_q8_fp32(const uint16_t* q_row, const uint16_t* w_row, const int8_t* code,
                           const uint16_t* scale, int heads, int dim) {
  float s = 0.0f;
  for (int h = 0; h < heads; ++h) {
    const uint16_t* qh = q_row + (int64_t)h * dim;
    float dot = 0.0f;
    for (int i = 0; i < dim; ++i) {
      float k = half_bits_to_float(scale[i / 32]) * (float)code[i];
      float prod = bf16_bits_to_float(qh[i]) * k;
      dot = dot + prod;
    }
    float t = bf16_bits_to_float(w_row[h]) * dot;
    s = s + t;
  }
  return s + 0.0f;
}

/*
 * Top-k block selection on the 8-bit key stream: the same admission, order
 * and output as ds_sel_oracle_select, with the score of score_q8_fp32.
 * Scales must be finite.  Returns 0, or -1 bad argument, -2 non-finite input,
 * -3 out of host memory.
 */
int ds_sel_oracle_select_q8(int32_t layers, int32_t rows, int32_t heads, int32_t dim, int64_t blocks,
                            int32_t k, const uint16_t* q, const uint16_t* w, const int8_t* codes,
                            int64_t ldc, int64_t code_layer_stride, const uint16_t* scales,
                            int64_t lds, int64_t scale_layer_stride, const uint32_t* mask,
                            int64_t mask_row_stride, int64_t mask_layer_stride, const int32_t* limit,
                            int32_t* out_idx, float* out_score, int32_t* out_count) {
  if (layers < 1 || rows < 1 || heads < 1 || dim < 32 || dim % 32 != 0 || blocks < 0 || k < 1)
    return ORACLE_E_INVALID;
  if (ldc < dim || lds < dim / 32 || !q || !w || !out_idx || !out_score) return ORACLE_E_INVALID;
  if (blocks > 0 && (!codes || !scales)) return ORACLE_E_INVALID;
  if (blocks > 0x7FFFFFFFLL) return ORACLE_E_INVALID;
  if (!inputs_finite((int64_t)layers * rows * heads, q, dim, dim)) return ORACLE_E_NONFINITE;
  if (!inputs_finite((int64_t)layers * rows, w, heads, heads)) return ORACLE_E_NONFINITE;
  for (int32_t l = 0; l < layers; ++l)
    for (int64_t b = 0; b < blocks; ++b)
      for (int32_t g = 0; g < dim / 32; ++g)
        if ((scales[l * scale_layer_stride + b * lds + g] & 0x7C00u) == 0x7C00u) return ORACLE_E_NONFINITE;

  scored_block* list = NULL;
  if (blocks > 0) {
    list = (scored_block*)malloc((size_t)blocks * sizeof *list);
    if (!list) return ORACLE_E_NOMEM;
  }
  for (int32_t l = 0; l < layers; ++l) {
    for (int32_t r = 0; r < rows; ++r) {
      int64_t lr = (int64_t)l * rows + r;
      const uint16_t* q_row = q + lr * heads * dim;
      const uint16_t* w_row = w + lr * heads;
      const uint32_t* mrow = mask ? mask + l * mask_layer_stride + r * mask_row_stride : NULL;
      int64_t lim = clamped_limit(limit, lr, blocks);
      int64_t n = 0;
      for (int64_t b = 0; b < lim; ++b) {
        if (mrow && !mask_bit(mrow, b)) continue;
        list[n].block = (int32_t)b;
        ++n;
      }
      for (int64_t j = 0; j < n; ++j) {
        int64_t b = list[j].block;
        list[j].score = score_q8_fp32(q_row, w_row, codes + l * code_layer_stride + b * ldc,
                                      scales + l * scale_layer_stride + b * lds, heads, dim);
      }
      if (n > 1) qsort(list, (size_t)n, sizeof *list, by_score_desc_then_index);
      int64_t m = n < k ? n : k;
      int32_t* oi = out_idx + lr * k;
      float* os = out_score + lr * k;
      for (int64_t j = 0; j < k; ++j) {
        if (j < m) {
          oi[j] = list[j].block;
          os[j] = list[j].score;
        } else {
          oi[j] = -1;
          os[j] = -INFINITY;
        }
      }
      if (out_count) out_count[lr] = (int32_t)m;
    }
  }
  free(list);
  return ORACLE_OK;
}

/* The q8 score (same order) of each listed block for one (layer, row). */
int ds_sel_oracle_score_blocks_q8(int32_t layers, int32_t rows, int32_t heads, int32_t dim,
                                  int64_t blocks, const uint16_t* q, const uint16_t* w,
                                  const int8_t* codes, int64_t ldc, int64_t code_layer_stride,
                                  const uint16_t* scales, int64_t lds, int64_t scale_layer_stride,
                                  int32_t layer, int32_t row, int64_t n_list, const int32_t* list,
                                  float* out) {
  if (layer < 0 || layer >= layers || row < 0 || row >= rows || n_list < 0) return ORACLE_E_INVALID;
  if (heads < 1 || dim < 32 || dim % 32 != 0 || ldc < dim || lds < dim / 32) return ORACLE_E_INVALID;
  int64_t lr = (int64_t)layer * rows + row;
  for (int64_t j = 0; j < n_list; ++j) {
    if (list[j] < 0 || list[j] >= blocks) return ORACLE_E_INVALID;
    out[j] = score_q8_fp32(q + lr * heads * dim, w + lr * heads,
                           codes + layer * code_layer_stride + (int64_t)list[j] * ldc,
                           scales + layer * scale_layer_stride + (int64_t)list[j] * lds, heads, dim);
  }
  return ORACLE_OK;
}

/*
 * Attention over the selected blocks -- the step that consumes the selection.
 *
 * Page "DeepSeek V4.1F Q4 on M3 Ultra with native DSpark MTP (40tps /
 * 800tps)", paragraph "Decode at depth": the compressed attention of a layer
 * attends to the 512 blocks the selection keeps.  The pages give no formula;
 * the reading taken here is ordinary scaled-dot-product attention over the
 * selected blocks, with the block key K[b] (the same key the selection
 * scores) and a block value V[b]:
 *   for each layer l, row r and attention head h, with c = count[l][r],
 *     s_j = scale * (qa[l][r][h] . K[l][idx[l][r][j]])         j < c
 *     o[l][r][h] = sum_j exp(s_j - max_i s_i) V[l][idx_j] / sum_j exp(s_j - max_i s_i)
 *   and o = 0 when c = 0.
 * Everything runs in double precision (bf16 inputs widen exactly); entries of
 * idx at or past count are not read.  Returns ORACLE_E_INVALID when a read
 * index lies outside [0, N).
 */
int ds_sel_oracle_attend(int32_t layers, int32_t rows, int32_t heads, int32_t dim, int64_t blocks,
                         int32_t k, const uint16_t* qa, const uint16_t* keys, int64_t ldk,
                         int64_t key_layer_stride, const uint16_t* values, int64_t ldv,
                         int64_t value_layer_stride, const int32_t* idx, const int32_t* count,
                         double scale, double* out) {
  if (layers < 1 || rows < 1 || heads < 1 || dim < 1 || blocks < 0 || k < 1 || !qa || !idx ||
      !count || !out || ldk < dim || ldv < dim)
    return ORACLE_E_INVALID;
  double* s = (double*)malloc(sizeof(double) * (size_t)k);
  if (!s) return ORACLE_E_NOMEM;
  for (int32_t l = 0; l < layers; ++l) {
    const uint16_t* K = keys + (int64_t)l * key_layer_stride;
    const uint16_t* V = values + (int64_t)l * value_layer_stride;
    for (int32_t r = 0; r < rows; ++r) {
      const int64_t lr = (int64_t)l * rows + r;
      const int32_t* sel = idx + lr * k;
      int32_t c = count[lr];
      if (c < 0 || c > k) {
        free(s);
        return ORACLE_E_INVALID;
      }
      for (int32_t j = 0; j < c; ++j) {
        if (sel[j] < 0 || (int64_t)sel[j] >= blocks) {
          free(s);
          return ORACLE_E_INVALID;
        }
      }
      for (int32_t h = 0; h < heads; ++h) {
        const uint16_t* qh = qa + (lr * heads + h) * (int64_t)dim;
        double* oh = out + (lr * heads + h) * (int64_t)dim;
        for (int32_t i = 0; i < dim; ++i) oh[i] = 0.0;
        if (c == 0) continue;
        double smax = -INFINITY;
        for (int32_t j = 0; j < c; ++j) {
          const uint16_t* kb = K + (int64_t)sel[j] * ldk;
          double dot = 0.0;
          for (int32_t i = 0; i < dim; ++i)
            dot += (double)bf16_bits_to_float(qh[i]) * (double)bf16_bits_to_float(kb[i]);
          s[j] = scale * dot;
          if (s[j] > smax) smax = s[j];
        }
        double z = 0.0;
        for (int32_t j = 0; j < c; ++j) {
          const double p = exp(s[j] - smax);
          const uint16_t* vb = V + (int64_t)sel[j] * ldv;
          for (int32_t i = 0; i < dim; ++i) oh[i] += p * (double)bf16_bits_to_float(vb[i]);
          z += p;
        }
        for (int32_t i = 0; i < dim; ++i) oh[i] /= z;
      }
    }
  }
  free(s);
  return ORACLE_OK;
}
