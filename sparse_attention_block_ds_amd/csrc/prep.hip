// prep: per layer, the admitted counts, the compacted admitted index, the
// head-weight fold and the candidate floors.
//
// Admission and compaction (page "DeepSeek V4.1F Q4 on M3 Ultra with native
// DSpark MTP (40tps / 800tps)", paragraph "Decode at depth": only blocks the
// mask admits are scored, and the admitted index is compacted once per row).
// A block is admitted for row r if its mask bit is set (when there is a mask)
// and it lies below the row's causal limit.  The layer's union over rows is
// compacted into one ascending index; when all rows share one mask row, each
// row's own list is a prefix of it (the rows differ only by their limits), so
// only the row's length is kept.  Without a mask the index is the identity and
// nothing is built.  The block axis is cut into tiles of 2048 blocks (64 mask
// words); workgroup x >= 1 of a layer expands tiles [16 (x-1), 16 x): it first
// counts the admitted blocks of all earlier tiles (a workgroup sum over their
// mask words), then each wave takes one tile: a wave prefix sum over its
// words' popcounts places every admitted block, the wave writes them into LDS
// in order and copies the tile's run to the global index in coalesced stores.
//
// Fold (workgroup 0 of each layer): score = sum_h w_h (q_h . K_b) =
// (sum_h w_h q_h) . K_b, so each row's H query heads collapse into one fp32
// vector q~ before the key stream (the products w_h q_hi are bf16 x bf16 and
// exact in fp32; the sum runs in ascending h).  For the matrix cores q~ is
// also split into three bf16 parts, hi = bf16(q~), mid = bf16(q~ - hi),
// lo = bf16(q~ - hi - mid), with hi + mid + lo == q~ exactly whenever
// |q~_i| >= 2^-110 (the lowest of q~'s 24 bits is then at or above bf16's
// least subnormal 2^-133); below that lo drops bits and the parts sum to q~
// within 2^-133, far below any score tolerance.
//
// Candidate floors (workgroup 0): the key stream writes only keys that can
// still be among a row's best k, i.e. keys at or above the row's floor.  The
// floor comes from 512 blocks spread evenly over [0, N), scored on the
// matrix cores: per row, the floor is the sampled key of rank about three
// times more selective than k would suggest (3 k n_sample / n_admitted, plus
// 8), found by a bitwise search over the wave's ballots.  Any floor is safe:
// the candidate lists have room for every position, and the select rescores
// the row exactly when fewer than min(k, admitted) candidates came through.
// The floor only decides how few keys are written; at 512 samples and 75000
// admitted blocks the expected sample count above the k-th key is 3.5 and the
// rank taken is 19, so a rescore is a ~1e-8 event.
#include "device_util.h"
#include "dssel_internal.h"
#include "relu_heads.h"

namespace dssel {
namespace {

constexpr int kPrepWaves = kPrepThreads / kWave;

// Sum over the wave, uniform result: DPP sums within each row of 16 lanes,
// then the four row sums read out to scalars.
__device__ __forceinline__ int wave_sum(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false);   // lane ^ 1
  v += __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false);   // lane ^ 2
  v += __builtin_amdgcn_update_dpp(0, v, 0x141, 0xF, 0xF, false);  // other quad of 8
  v += __builtin_amdgcn_update_dpp(0, v, 0x140, 0xF, 0xF, false);  // other half of 16
  return __builtin_amdgcn_readlane(v, 0) + __builtin_amdgcn_readlane(v, 16) +
         __builtin_amdgcn_readlane(v, 32) + __builtin_amdgcn_readlane(v, 48);
}

struct Limits {
  int64_t lim[kMaxRows];
  int64_t maxlim;
};

// The layer's R limits, clamped to [0, N]: R independent loads, then the clamps.
template <int R>
__device__ __forceinline__ Limits layer_limits(const Call& c, int l) {
  Limits s;
  int64_t raw[R];
#pragma unroll
  for (int r = 0; r < R; ++r) raw[r] = c.blocks;
  if (c.limit) {
#pragma unroll
    for (int r = 0; r < R; ++r) raw[r] = c.limit[(int64_t)l * R + r];
  }
  s.maxlim = 0;
#pragma unroll
  for (int r = 0; r < kMaxRows; ++r) {
    const int64_t v = r < R ? raw[r < R ? r : 0] : 0;
    s.lim[r] = v < 0 ? 0 : (v > c.blocks ? c.blocks : v);
    s.maxlim = s.lim[r] > s.maxlim ? s.lim[r] : s.maxlim;
  }
  return s;
}

// Union of the rows' admitted blocks in mask word j (blocks 32 j .. 32 j + 31).
template <int R>
__device__ __forceinline__ uint32_t union_word(const Call& c, const uint32_t* mask_l, const Limits& s,
                                               int64_t j) {
  if (c.mode == kSharedMask) return mask_l[j] & below_limit_bits(j, s.maxlim);
  uint32_t w[R];
#pragma unroll
  for (int r = 0; r < R; ++r) w[r] = mask_l[r * c.mask_row_stride + j];
  uint32_t u = 0;
#pragma unroll
  for (int r = 0; r < R; ++r) u |= w[r] & below_limit_bits(j, s.lim[r]);
  return u;
}

// Row r's admitted blocks in mask word j.
__device__ __forceinline__ uint32_t row_word(const Call& c, const uint32_t* mask_l, const Limits& s,
                                             int r, int64_t j) {
  const uint32_t m = c.mode == kSharedMask ? mask_l[j] : mask_l[r * c.mask_row_stride + j];
  return m & below_limit_bits(j, s.lim[r]);
}

// LDS of the fold workgroup and of the expanding workgroups (never both).
struct FoldShared {
  union {
    float part[kPrepThreads * 8];          // fold partial sums, [head slice][r * d + i]
    uint32_t relu[kReluStageBytes / 4];    // per-head ReLU score: the layer's q heads and w
  };
  float q[kMaxRows][256];                  // folded query rows
  uint32_t skey[kMaxRows][kSampleSlots];   // sample keys (0: not admitted by the row)
  int64_t lim[kMaxRows];                   // the rows' limits, clamped to [0, N]
  int acc[kMaxRows + 1];
};

struct ExpandShared {
  int32_t stage[kPrepWaves][kTileBlocks];  // one tile's compacted run per wave
  int tile_cnt[kPrepWaves];
  int scan[kPrepWaves + 1];
  int before;
};

union PrepShared {
  FoldShared f;
  ExpandShared e;
};

// Block of sample slot j: (2 j + 1) * N / (2 S) with S = min(512, N), i.e. the
// middle of the j-th of S equal stretches of [0, N).
__device__ __forceinline__ int64_t sample_block(int j, int64_t n) {
  return n >= kSampleSlots ? ((2 * (int64_t)j + 1) * n) >> 10 : j;
}
static_assert(kSampleSlots == 512, "sample_block divides by 2 * 512 with a shift");

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kSampleGroups = kSampleSlots / 16;                // 16 sampled blocks per MFMA
constexpr int kGroupsPerWave = kSampleGroups / (kPrepThreads / kWave);  // 2

// Sampled keys on the matrix cores.  A floor only has to be a reasonable
// guess (any floor is exact, see above), so the sampled scores use q~
// rounded to bf16: one v_mfma_f32_16x16x32_bf16 per 32 columns gives 16
// sampled blocks (B columns, block = lane % 16) against query rows 0-7 (A rows,
// row = lane % 16, rows >= R zero).  Lane l then holds rows 4 (l / 16) + i of
// block l % 16.  Each wave takes groups wave and wave + 16 of 16 slots.
template <int R, int D>
struct SampleMfma {
  static constexpr bool kFold = true;  // scores on the folded query
  static constexpr int KC = D / 32;
  u32x4_t kb[kGroupsPerWave][KC];
  uint32_t mw[kGroupsPerWave][4];  // mask words of rows 4 (lane / 16) + i at the lane's block

  __device__ void issue(const Call& c, int l, int64_t n, const uint32_t* mask_l, int S) {
    const int lane = lane_id(), wave = threadIdx.x / kWave;
    const uint16_t* K = c.keys + (int64_t)l * c.key_layer_stride;
#pragma unroll
    for (int g = 0; g < kGroupsPerWave; ++g) {
      const int j = (wave + g * (kPrepThreads / kWave)) * 16 + (lane & 15);
#pragma unroll
      for (int cc = 0; cc < KC; ++cc) kb[g][cc] = u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
      for (int i = 0; i < 4; ++i) mw[g][i] = 0xFFFFFFFFu;
      if (j < S) {
        const int64_t b = sample_block(j, n);
        const uint16_t* row = K + b * c.ldk + 8 * (lane >> 4);
#pragma unroll
        for (int cc = 0; cc < KC; ++cc) kb[g][cc] = *reinterpret_cast<const u32x4_t*>(row + 32 * cc);
        if (c.mode == kSharedMask) {
          const uint32_t w = mask_l[b >> 5];
#pragma unroll
          for (int i = 0; i < 4; ++i) mw[g][i] = w;
        } else if (c.mode == kRowMask) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int r = 4 * (lane >> 4) + i;
            if (r < R) mw[g][i] = mask_l[r * c.mask_row_stride + (b >> 5)];
          }
        }
      }
    }
  }

  __device__ void stage(const Call&, int, FoldShared&) {}

  __device__ void finish(int64_t n, int S, FoldShared& sh) {
    const int lane = lane_id(), wave = threadIdx.x / kWave;
    const int m = lane & 15;
    bf16x8_t a[KC];
#pragma unroll
    for (int cc = 0; cc < KC; ++cc) {
      u32x4_t v = {0u, 0u, 0u, 0u};
      if (m < R) {
        const float* qr = &sh.q[m < R ? m : 0][32 * cc + 8 * (lane >> 4)];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          v[e] = (uint32_t)f32_to_bf16_rne(qr[2 * e]) | ((uint32_t)f32_to_bf16_rne(qr[2 * e + 1]) << 16);
      }
      a[cc] = __builtin_bit_cast(bf16x8_t, v);
    }
#pragma unroll
    for (int g = 0; g < kGroupsPerWave; ++g) {
      const int j = (wave + g * (kPrepThreads / kWave)) * 16 + (lane & 15);
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int cc = 0; cc < KC; ++cc)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[cc], __builtin_bit_cast(bf16x8_t, kb[g][cc]), acc,
                                                      0, 0, 0);
      if (j < S) {
        const int64_t b = sample_block(j, n);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 4 * (lane >> 4) + i;
          if (r < R && b < sh.lim[r] && ((mw[g][i] >> (b & 31)) & 1u))
            sh.skey[r][j] = score_to_key(acc[i]);
        }
      }
    }
  }
};

// The same sampled scores on 8-bit keys: each 32-column group is one MFMA
// with its own accumulation (codes widened exactly to bf16), scaled by the
// block's group scale and summed in fp32.
template <int R, int D>
struct SampleMfmaQ8 {
  static constexpr bool kFold = true;
  static constexpr int KC = D / 32;
  uint2 kb[kGroupsPerWave][KC];
  uint16_t ks[kGroupsPerWave][KC];
  uint32_t mw[kGroupsPerWave][4];

  __device__ void issue(const Call& c, int l, int64_t n, const uint32_t* mask_l, int S) {
    const int lane = lane_id(), wave = threadIdx.x / kWave;
    const int8_t* codes = c.codes + (int64_t)l * c.code_layer_stride;
    const uint16_t* scales = c.scales + (int64_t)l * c.scale_layer_stride;
#pragma unroll
    for (int g = 0; g < kGroupsPerWave; ++g) {
      const int j = (wave + g * (kPrepThreads / kWave)) * 16 + (lane & 15);
#pragma unroll
      for (int cc = 0; cc < KC; ++cc) {
        kb[g][cc] = make_uint2(0u, 0u);
        ks[g][cc] = 0;
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) mw[g][i] = 0xFFFFFFFFu;
      if (j < S) {
        const int64_t b = sample_block(j, n);
        const int8_t* row = codes + b * c.ldc + 8 * (lane >> 4);
#pragma unroll
        for (int cc = 0; cc < KC; ++cc) {
          kb[g][cc] = *reinterpret_cast<const uint2*>(row + 32 * cc);
          ks[g][cc] = scales[b * c.lds + cc];
        }
        if (c.mode == kSharedMask) {
          const uint32_t w = mask_l[b >> 5];
#pragma unroll
          for (int i = 0; i < 4; ++i) mw[g][i] = w;
        } else if (c.mode == kRowMask) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int r = 4 * (lane >> 4) + i;
            if (r < R) mw[g][i] = mask_l[r * c.mask_row_stride + (b >> 5)];
          }
        }
      }
    }
  }

  __device__ void stage(const Call&, int, FoldShared&) {}

  __device__ void finish(int64_t n, int S, FoldShared& sh) {
    const int lane = lane_id(), wave = threadIdx.x / kWave;
    const int m = lane & 15;
    bf16x8_t a[KC];
#pragma unroll
    for (int cc = 0; cc < KC; ++cc) {
      u32x4_t v = {0u, 0u, 0u, 0u};
      if (m < R) {
        const float* qr = &sh.q[m < R ? m : 0][32 * cc + 8 * (lane >> 4)];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          v[e] = (uint32_t)f32_to_bf16_rne(qr[2 * e]) | ((uint32_t)f32_to_bf16_rne(qr[2 * e + 1]) << 16);
      }
      a[cc] = __builtin_bit_cast(bf16x8_t, v);
    }
#pragma unroll
    for (int g = 0; g < kGroupsPerWave; ++g) {
      const int j = (wave + g * (kPrepThreads / kWave)) * 16 + (lane & 15);
      float sc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int cc = 0; cc < KC; ++cc) {
        const u32x4_t bv = {bf16_pair_of_codes(kb[g][cc].x, 0), bf16_pair_of_codes(kb[g][cc].x, 16),
                            bf16_pair_of_codes(kb[g][cc].y, 0), bf16_pair_of_codes(kb[g][cc].y, 16)};
        const f32x4_t acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            a[cc], __builtin_bit_cast(bf16x8_t, bv), f32x4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
        const float scale = half_bits_to_f32(ks[g][cc]);
#pragma unroll
        for (int i = 0; i < 4; ++i) sc[i] += scale * acc[i];
      }
      if (j < S) {
        const int64_t b = sample_block(j, n);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 4 * (lane >> 4) + i;
          if (r < R && b < sh.lim[r] && ((mw[g][i] >> (b & 31)) & 1u)) sh.skey[r][j] = score_to_key(sc[i]);
        }
      }
    }
  }
};

// Sampled keys under the per-head ReLU score: the same sampled blocks and
// mask words as SampleMfma, scored against every (row, head) pair on the
// matrix cores (relu_heads.h) with the layer's heads staged in LDS; no fold.
template <int R, int D>
struct SampleRelu {
  static constexpr bool kFold = false;
  static constexpr int KC = D / 32;
  relu_u32x4_t kb[kGroupsPerWave][KC];
  uint32_t mw[kGroupsPerWave][4];
  ReluStage st;

  __device__ void issue(const Call& c, int l, int64_t n, const uint32_t* mask_l, int S) {
    const int lane = lane_id(), wave = threadIdx.x / kWave;
    const uint16_t* K = c.keys + (int64_t)l * c.key_layer_stride;
#pragma unroll
    for (int g = 0; g < kGroupsPerWave; ++g) {
      const int j = (wave + g * (kPrepThreads / kWave)) * 16 + (lane & 15);
#pragma unroll
      for (int cc = 0; cc < KC; ++cc) kb[g][cc] = relu_u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
      for (int i = 0; i < 4; ++i) mw[g][i] = 0xFFFFFFFFu;
      if (j < S) {
        const int64_t b = sample_block(j, n);
        const uint16_t* row = K + b * c.ldk + 8 * (lane >> 4);
#pragma unroll
        for (int cc = 0; cc < KC; ++cc) kb[g][cc] = *reinterpret_cast<const relu_u32x4_t*>(row + 32 * cc);
        if (c.mode == kSharedMask) {
          const uint32_t w = mask_l[b >> 5];
#pragma unroll
          for (int i = 0; i < 4; ++i) mw[g][i] = w;
        } else if (c.mode == kRowMask) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int r = 4 * (lane >> 4) + i;
            if (r < R) mw[g][i] = mask_l[r * c.mask_row_stride + (b >> 5)];
          }
        }
      }
    }
  }

  __device__ void stage(const Call& c, int l, FoldShared& sh) {
    st = relu_stage_heads<R, D>(c, l, sh.relu, threadIdx.x, kPrepThreads);
  }

  // Row r's score of a sampled block is complete in all four lanes of its
  // column; the lanes of group r / 4 hold row r's mask word and store it.
  __device__ void finish(int64_t n, int S, FoldShared& sh) {
    const int lane = lane_id(), wave = threadIdx.x / kWave;
    float all[R][kGroupsPerWave];
#pragma unroll
    for (int g = 0; g < kGroupsPerWave; ++g) {  // one group at a time: 128 registers
      float one[R][1];
      relu_all_rows<R, D, 1, false>(st, reinterpret_cast<const relu_u32x4_t(&)[1][KC]>(kb[g]), one);
#pragma unroll
      for (int r = 0; r < R; ++r) all[r][g] = one[r][0];
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const float (&sc)[kGroupsPerWave] = all[r];
#pragma unroll
      for (int g = 0; g < kGroupsPerWave; ++g) {
        const int j = (wave + g * (kPrepThreads / kWave)) * 16 + (lane & 15);
        if ((lane >> 4) == r / 4 && j < S) {
          const int64_t b = sample_block(j, n);
          if (b < sh.lim[r] && ((mw[g][r % 4] >> (b & 31)) & 1u)) sh.skey[r][j] = score_to_key(sc[g]);
        }
      }
    }
  }
};

// A floor for the j-th largest of the 512 keys a wave holds (8 per lane): the
// largest x with at least j keys >= x, built bit by bit from the top, over
// the top 16 bits only (sign, exponent and 7 mantissa bits of the score).
// It is at most the j-th largest key and lets through at most the keys that
// share its 16-bit prefix besides.
__device__ __forceinline__ uint32_t wave_jth_largest(const uint32_t (&v)[kSampleSlots / kWave], int j) {
  uint32_t x = 0;
#pragma unroll 1
  for (int bit = 31; bit >= 16; --bit) {
    const uint32_t t = x | (1u << bit);
    int n = 0;
#pragma unroll
    for (int i = 0; i < kSampleSlots / kWave; ++i) n += __popcll(__ballot(v[i] >= t));
    if (n >= j) x = t;
  }
  return x;
}

// Workgroup 0 of layer l: counts, fold, floors.  Every global load the
// workgroup needs (sampled key rows and their mask words, the query heads and
// weights, the mask words to count) is issued before any of them is used.
template <int R, int D, class Sampler>
__device__ void fold_count_floor(const Call& c, int l, FoldShared& sh) {
  const int H = c.heads;
  const int tid = threadIdx.x, lane = lane_id(), wave = tid / kWave;
  const Limits s = layer_limits<R>(c, l);
  const uint32_t* mask_l = c.mask ? c.mask + (int64_t)l * c.mask_layer_stride : nullptr;
  int32_t* counts = c.counts + (int64_t)l * kCountStride;

  // Sampled key rows: spread over [0, N), so that their addresses wait for
  // nothing (samples at or past a row's limit are simply not admitted).
  const int64_t N = c.blocks;
  const int S = N < kSampleSlots ? (int)N : kSampleSlots;
  Sampler smp;
  smp.issue(c, l, N, mask_l, S);

  // The mask words to count, when every row shares one mask row (all words
  // below N: the limits are applied when counting).
  constexpr int kCountWords = 4;  // per thread in flight: masks up to 131072 blocks
  const int64_t all_words = (N + 31) / 32;
  uint32_t cw[kCountWords];
#pragma unroll
  for (int i = 0; i < kCountWords; ++i) {
    const int64_t j = tid + (int64_t)i * kPrepThreads;
    cw[i] = (c.mode == kSharedMask && j < all_words) ? mask_l[j] : 0u;
  }
  for (int i = tid; i < kMaxRows * kSampleSlots; i += kPrepThreads) (&sh.skey[0][0])[i] = 0u;

  // fold, first half: thread (slice hs, chunk) sums w_h q_h[i0 .. i0 + 8) over
  // its slice of heads, ascending h, eight heads' loads at a time.  The
  // per-head ReLU score has no fold: its sampler stages the heads instead.
  const int chunks = R * D / 8;
  const int slices = kPrepThreads / chunks;  // >= 4
  const int hper = (H + slices - 1) / slices;
  if constexpr (!Sampler::kFold) smp.stage(c, l, sh);
  if (Sampler::kFold && tid < chunks * slices) {
    const int ch = tid % chunks, hs = tid / chunks;
    const int r = ch / (D / 8), i0 = (ch % (D / 8)) * 8;
    const int64_t lr = (int64_t)l * R + r;
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.0f;
    const int h0 = hs * hper, h1 = h0 + hper < H ? h0 + hper : H;
    for (int hb = h0; hb < h1; hb += 8) {
      uint4 qv[8];
      float wv[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int h = hb + u < h1 ? hb + u : h1 - 1;  // repeated loads past h1 are not summed
        qv[u] = *reinterpret_cast<const uint4*>(c.q + (lr * H + h) * D + i0);
        wv[u] = bf16_to_f32(c.w[lr * H + h]);
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (hb + u >= h1) break;
        const uint32_t q4[4] = {qv[u].x, qv[u].y, qv[u].z, qv[u].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc[2 * e] = fmaf(wv[u], bf16_lo(q4[e]), acc[2 * e]);
          acc[2 * e + 1] = fmaf(wv[u], bf16_hi(q4[e]), acc[2 * e + 1]);
        }
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) sh.part[hs * R * D + r * D + i0 + e] = acc[e];
  }

  if (tid <= kMaxRows) sh.acc[tid] = 0;
  if (tid == 0) {
#pragma unroll
    for (int r = 0; r < kMaxRows; ++r) sh.lim[r] = s.lim[r];
  }

  // admitted counts per row and for the union
  __syncthreads();
  const int64_t words = (s.maxlim + 31) / 32;
  if (c.mode == kNoMask) {
    if (tid < R) sh.acc[tid] = (int)sh.lim[tid];
    if (tid == 0) sh.acc[kMaxRows] = (int)s.maxlim;
  } else {
    int rc[kMaxRows + 1];
#pragma unroll
    for (int r = 0; r <= kMaxRows; ++r) rc[r] = 0;
    int64_t j0 = tid;
    if (c.mode == kSharedMask) {
#pragma unroll
      for (int i = 0; i < kCountWords; ++i) {
        const int64_t j = tid + (int64_t)i * kPrepThreads;
        if (j < words) {
          rc[kMaxRows] += __popc(cw[i] & below_limit_bits(j, s.maxlim));
#pragma unroll
          for (int r = 0; r < R; ++r) rc[r] += __popc(cw[i] & below_limit_bits(j, s.lim[r]));
        }
      }
      j0 = tid + (int64_t)kCountWords * kPrepThreads;
    }
    for (int64_t j = j0; j < words; j += kPrepThreads) {
      rc[kMaxRows] += __popc(union_word<R>(c, mask_l, s, j));
#pragma unroll
      for (int r = 0; r < R; ++r) rc[r] += __popc(row_word(c, mask_l, s, r, j));
    }
#pragma unroll
    for (int r = 0; r <= kMaxRows; ++r) {
      if (r < R || r == kMaxRows) {
        const int v = wave_sum(rc[r]);
        if (lane == 0 && v) atomicAdd(&sh.acc[r], v);
      }
    }
  }

  // fold, second half: the slices' partial sums in ascending slice order; the
  // three-way bf16 split (exact for |q~_i| >= 2^-110)
  for (int o = tid; Sampler::kFold && o < R * D; o += kPrepThreads) {
    const int r = o / D, i = o % D;
    const int64_t lr = (int64_t)l * R + r;
    float acc = 0.0f;
    for (int hs = 0; hs < slices; ++hs) acc += sh.part[hs * R * D + o];
    sh.q[r][i] = acc;
    c.qt[lr * D + i] = acc;
    const uint16_t hi = f32_to_bf16_rne(acc);
    const float r1 = acc - bf16_to_f32(hi);   // exact: acc minus its own rounding
    const uint16_t mid = f32_to_bf16_rne(r1);
    const float r2 = r1 - bf16_to_f32(mid);   // exact for the same reason
    const uint16_t lo = f32_to_bf16_rne(r2);
    uint16_t* parts = c.qparts + ((int64_t)l * 3 * R + r) * D + i;
    parts[0] = hi;
    parts[(int64_t)R * D] = mid;
    parts[(int64_t)2 * R * D] = lo;
  }
  __syncthreads();
  if (tid <= kMaxRows && (tid < R || tid == kMaxRows)) counts[tid] = sh.acc[tid];

  // sample keys
  smp.finish(N, S, sh);
  __syncthreads();

  // floors: wave r finds row r's jth largest sample key
  if (wave < R) {
    const int r = wave;
    uint32_t v[kSampleSlots / kWave];
    int sr = 0;  // admitted samples: the non-zero keys
#pragma unroll
    for (int i = 0; i < kSampleSlots / kWave; ++i) {
      v[i] = sh.skey[r][i * kWave + lane];
      sr += __popcll(__ballot(v[i] != 0u));
    }
    const int64_t n = sh.acc[r];
    const int64_t m = n < c.k ? n : c.k;
    uint32_t floor = 0;
    if (sr > 0 && n > 3 * m) {
      const int64_t jth = (3 * m * sr + n - 1) / n + 8;
      if (jth <= sr) floor = wave_jth_largest(v, (int)jth);
    }
    if (lane == 0) {
      c.floor_key[(int64_t)l * R + r] = floor;
      c.cand_count[((int64_t)l * R + r) * kCountPad] = 0;
    }
  }
}

// Workgroup x >= 1 of layer l: expand tiles [16 (x-1), 16 x) of the union.
template <int R>
__device__ void expand_tiles(const Call& c, int l, int x, ExpandShared& sh) {
  const int tid = threadIdx.x, lane = lane_id(), wave = tid / kWave;
  const Limits s = layer_limits<R>(c, l);
  const uint32_t* mask_l = c.mask + (int64_t)l * c.mask_layer_stride;
  const int64_t words = (s.maxlim + 31) / 32;
  const int t0 = (x - 1) * kPrepTilesPerWg;

  // this wave's tile word (loaded alongside the earlier tiles' words)
  const int t = t0 + wave;
  const int64_t j = (int64_t)t * kTileWords + lane;
  const uint32_t u = (t < c.ntiles && j < words) ? union_word<R>(c, mask_l, s, j) : 0u;

  // admitted blocks of all earlier tiles
  int before = 0;
  const int64_t w_end = (int64_t)t0 * kTileWords < words ? (int64_t)t0 * kTileWords : words;
  for (int64_t jj = tid; jj < w_end; jj += kPrepThreads) before += __popc(union_word<R>(c, mask_l, s, jj));
  if (tid == 0) sh.before = 0;
  __syncthreads();
  before = wave_sum(before);
  if (lane == 0 && before) atomicAdd(&sh.before, before);

  // place the tile's admitted blocks in order: lane i's k-th set bit goes to
  // its exclusive prefix + k.  Each lane walks its 32 bits starting at bit
  // i % 32, so at every step the lanes write to different LDS banks.
  const int cnt = __popc(u);
  const int in_tile = wave_inclusive_scan(cnt) - cnt;
  const int tile_total = __shfl(in_tile + cnt, kWave - 1, kWave);
  if (lane == 0) sh.tile_cnt[wave] = tile_total;
  const int32_t b0 = (int32_t)(j * 32);
  for (int step = 0; step < 32; ++step) {
    const int bit = (step + lane) & 31;
    if ((u >> bit) & 1u) sh.stage[wave][in_tile + __popc(u & ((1u << bit) - 1u))] = b0 + bit;
  }
  __syncthreads();
  int total = 0;
  const int mine = tid < kPrepWaves ? sh.tile_cnt[tid] : 0;
  const int excl = block_exclusive_scan<kPrepThreads>(mine, &total, sh.scan);
  if (tid < kPrepWaves) sh.tile_cnt[tid] = excl;
  __syncthreads();
  int32_t* out = c.list + (int64_t)l * c.blocks + sh.before + sh.tile_cnt[wave];
  for (int i = lane; i < tile_total; i += kWave) out[i] = sh.stage[wave][i];
}

template <int R, int D, class Sampler>
__global__ __launch_bounds__(kPrepThreads) void prep_kernel(Call c) {
  __shared__ PrepShared sh;
  // blockIdx.x is the layer, so that consecutive workgroups (which the
  // dispatcher deals out to the XCDs in turn) belong to different layers and
  // the layers' fold workgroups spread over every XCD.
  if (blockIdx.y == 0) fold_count_floor<R, D, Sampler>(c, blockIdx.x, sh.f);
  else expand_tiles<R>(c, blockIdx.x, blockIdx.y, sh.e);
}

template <int R, int D>
void launch_rd(const Call& c, dim3 grid, hipStream_t stream) {
  if (c.fmt == kKeysQ8)
    hipLaunchKernelGGL((prep_kernel<R, D, SampleMfmaQ8<R, D>>), grid, dim3(kPrepThreads), 0, stream, c);
  else if (c.score_kind == kScoreHeadRelu)
    hipLaunchKernelGGL((prep_kernel<R, D, SampleRelu<R, D>>), grid, dim3(kPrepThreads), 0, stream, c);
  else
    hipLaunchKernelGGL((prep_kernel<R, D, SampleMfma<R, D>>), grid, dim3(kPrepThreads), 0, stream, c);
}

template <int R>
hipError_t launch_r(const Call& c, dim3 grid, hipStream_t stream) {
  switch (c.dim) {
    case 32: launch_rd<R, 32>(c, grid, stream); break;
    case 64: launch_rd<R, 64>(c, grid, stream); break;
    case 128: launch_rd<R, 128>(c, grid, stream); break;
    case 256: launch_rd<R, 256>(c, grid, stream); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prep(const Call& c, hipStream_t stream) {
  const int expanders = c.mode == kNoMask ? 0 : (c.ntiles + kPrepTilesPerWg - 1) / kPrepTilesPerWg;
  dim3 grid(c.layers, 1 + expanders);
  switch (c.rows) {
    case 1: return launch_r<1>(c, grid, stream);
    case 2: return launch_r<2>(c, grid, stream);
    case 3: return launch_r<3>(c, grid, stream);
    case 4: return launch_r<4>(c, grid, stream);
    case 5: return launch_r<5>(c, grid, stream);
    case 6: return launch_r<6>(c, grid, stream);
    case 7: return launch_r<7>(c, grid, stream);
    case 8: return launch_r<8>(c, grid, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace dssel
