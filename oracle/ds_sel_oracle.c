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
