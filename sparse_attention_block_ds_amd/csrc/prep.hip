// prep: per layer, the admitted counts, the compacted admitted index, the
// head-weight fold and the candidate floors.
//
// Admission and compaction (page "DeepSeek V4.1F Q4 on M3 Ultra with native
// DSpark MTP (40tps / 800tps)", paragraph "Decode at depth": only blocks the
// mask admits are scored, and the admitted index is compacted once per row). A
// block is admitted for row r if its mask bit is set (when there is a mask) and
// it lies below the row's causal limit.  The layer's union over rows is
// compacted into one ascending index; when all rows share one mask row, each
// row's own list is a prefix of it (the rows differ only by their limits), so
// only the row's length is kept.  Without a mask the index is the identity and
// nothing is built.  The block axis is cut into tiles of 2048 blocks (64 mask
// words); expanding workgroup x >= 1 of a layer (grid row R + x - 1) expands
// tiles [16 (x-1), 16 x): it first counts the admitted blocks of all earlier
// tiles (a workgroup sum over their mask words), then each wave takes one tile:
// a wave prefix sum over its words' popcounts places every admitted block, the
// wave writes them into LDS in order and copies the tile's run to the global
// index in coalesced stores.
//
// Fold (workgroup r < R of each layer, one per row): score = sum_h w_h (q_h .
// K_b) = (sum_h w_h q_h) . K_b, so each row's H query heads collapse into one
// fp32 vector q~ before the key stream (the products w_h q_hi are bf16 x bf16
// and exact in fp32; the sum runs in ascending h).  For the matrix cores q~ is
// also split into three bf16 parts, hi = bf16(q~), mid = bf16(q~ - hi), lo =
// bf16(q~ - hi - mid), with hi + mid + lo == q~ exactly whenever |q~_i| >=
// 2^-110 (the lowest of q~'s 24 bits is then at or above bf16's least subnormal
// 2^-133); below that lo drops bits and the parts sum to q~ within 2^-133, far
// below any score tolerance.
//
// Candidate floors (the same row workgroups): the key stream writes only keys
// that can still be among a row's best k, i.e. keys at or above the row's
// floor.  The floor comes from 512 blocks (256 on a one-layer call) spread
// evenly over [0, N), scored on the matrix cores: per row, the floor is the
// sampled key of rank about three times more selective than k would suggest
// (3 k n_sample / n_admitted, plus 8), found by a bitwise search over the
// wave's ballots.  Any floor is safe:
// the candidate lists have room for every position, and the select rescores the
// row exactly when fewer than min(k, admitted) candidates came through. The
// floor only decides how few keys are written; at 75000 admitted blocks the
// expected sample count above the k-th key is 3.5 with 512 samples (rank taken
// 19) and 1.75 with 256 (rank 14), so a rescore is a ~1e-8 event either way.
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

// Head slices of the fold: each of the row's d / 8 column chunks is summed
// over kFoldSlices slices of the heads, then the slices in order.
constexpr int kFoldSlices = 16;
constexpr int kFoldBatch = 4;  // heads loaded per step of a fold thread

// LDS of a row workgroup (StageWords: the per-head ReLU score's staged heads
// and weights of the row, 0 for the folded scores).
template <int StageWords>
struct FoldShared {
  union {
    float part[kFoldSlices * 256];                    // fold partial sums, [head slice][i]
    uint32_t relu[StageWords > 0 ? StageWords : 1];   // the row's q heads and w
  };
  float q[256];                            // the folded query row
  uint32_t skey[kSampleSlots];             // sample keys (0: not admitted by the row)
  int acc[2];                              // admitted count of the row, of the union
};

// LDS of an expanding workgroup: each wave's tile run as offsets from the
// tile's first block (a tile has 2048 blocks, so 16 bits suffice).
struct ExpandShared {
  uint16_t stage[kPrepWaves][kTileBlocks];
  int tile_cnt[kPrepWaves];
  int scan[kPrepWaves + 1];
  int before;
};

// A workgroup is either a row workgroup or an expanding one.
template <class Fold>
union PrepShared {
  Fold f;
  ExpandShared e;
};

// Block of sample slot j of NS: (2 j + 1) * N / (2 NS) when N >= NS, i.e. the
// middle of the j-th of NS equal stretches of [0, N), else block j.
template <int NS>
__device__ __forceinline__ int64_t sample_block(int j, int64_t n) {
  constexpr int kShift = __builtin_ctz(2 * NS);
  static_assert((1 << kShift) == 2 * NS, "sample_block divides by 2 NS with a shift");
  return n >= NS ? ((2 * (int64_t)j + 1) * n) >> kShift : j;
}

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// Sampled blocks per row: 512 on batched calls, where a tighter floor saves
// the key stream and the select more than the samples cost; 256 on one-layer
// calls, where the row workgroup's sample loads are on the critical path
// (measured on gfx950: prep 2.7 us shorter, the whole call 1.7-2.7 us).
constexpr int kSamplesBatched = kSampleSlots;  // 512: the LDS holds this many keys
constexpr int kSamplesOneLayer = 256;
// Groups of 16 sampled blocks (one MFMA each) per wave.
template <int NS>
constexpr int kGroupsPerWave = NS / 16 / (kPrepThreads / kWave);

// Sampled keys of one row on the matrix cores.  A floor only has to be a
// reasonable guess (any floor is exact, see above), so the sampled scores use
// q~ rounded to bf16: one v_mfma_f32_16x16x32_bf16 per 32 columns gives 16
// sampled blocks (B columns, block = lane % 16) against the row (A row 0, the
// other 15 A rows zero); lanes 0-15 then hold the row's 16 scores.  Each wave
// takes groups wave, wave + 16, ... of 16 slots (G of them).  Loads are unconditional when
// there are blocks (slots past S re-read slot 0 and are not admitted), so no
// branch waits on them; nothing is read when there are none (S = 0).
template <int D, int NS>
struct SampleMfma {
  static constexpr int kSamples = NS;
  static constexpr int G = kGroupsPerWave<NS>;
  static constexpr bool kFold = true;  // scores on the folded query
  using Shared = FoldShared<0>;
  static constexpr int KC = D / 32;
  u32x4_t kb[G][KC];
  uint32_t mw[G];  // the row's mask word at the lane's block

  // mrow: the row's mask words, or null when there is no mask.
  __device__ void issue(const Call& c, int l, int64_t n, const uint32_t* mrow, int S) {
    const int lane = lane_id(), wave = threadIdx.x / kWave;
    const uint16_t* K = c.keys + (int64_t)l * c.key_layer_stride;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const int j = (wave + g * (kPrepThreads / kWave)) * 16 + (lane & 15);
      if (S == 0) {
#pragma unroll
        for (int cc = 0; cc < KC; ++cc) kb[g][cc] = {};
        mw[g] = 0u;
        continue;
      }
      const int64_t b = sample_block<NS>(j < S ? j : 0, n);
      const uint16_t* row = K + b * c.ldk + 8 * (lane >> 4);
#pragma unroll
      for (int cc = 0; cc < KC; ++cc) kb[g][cc] = *reinterpret_cast<const u32x4_t*>(row + 32 * cc);
      mw[g] = mrow ? mrow[b >> 5] : 0xFFFFFFFFu;
      if (j >= S) mw[g] = 0u;
    }
  }

  __device__ void stage(const Call&, int64_t, Shared&) {}

  // One 32-column chunk at a time over both groups, so that each chunk's A
  // operand and B operands are dead once its MFMAs are issued.
  __device__ void finish(int64_t n, int S, int64_t lim, Shared& sh) {
    const int lane = lane_id(), wave = threadIdx.x / kWave;
    f32x4_t acc[G];
#pragma unroll
    for (int g = 0; g < G; ++g) acc[g] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int cc = 0; cc < KC; ++cc) {
      u32x4_t v = {0u, 0u, 0u, 0u};
      if ((lane & 15) == 0) {
        const float* qr = &sh.q[32 * cc + 8 * (lane >> 4)];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          v[e] = (uint32_t)f32_to_bf16_rne(qr[2 * e]) | ((uint32_t)f32_to_bf16_rne(qr[2 * e + 1]) << 16);
      }
      const bf16x8_t a = __builtin_bit_cast(bf16x8_t, v);
#pragma unroll
      for (int g = 0; g < G; ++g)
        acc[g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(bf16x8_t, kb[g][cc]), acc[g],
                                                         0, 0, 0);
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const int j = (wave + g * (kPrepThreads / kWave)) * 16 + (lane & 15);
      if (lane < 16 && j < S) {
        const int64_t b = sample_block<NS>(j, n);
        if (b < lim && ((mw[g] >> (b & 31)) & 1u)) sh.skey[j] = score_to_key(acc[g][0]);
      }
    }
  }
};

// The same sampled scores on 8-bit keys: each 32-column group is one MFMA
// with its own accumulation (codes widened exactly to bf16), scaled by the
// block's group scale and summed in fp32.
template <int D, int NS>
struct SampleMfmaQ8 {
  static constexpr int kSamples = NS;
  static constexpr int G = kGroupsPerWave<NS>;
  static constexpr bool kFold = true;
  using Shared = FoldShared<0>;
  static constexpr int KC = D / 32;
  uint2 kb[G][KC];
  uint16_t ks[G][KC];
  uint32_t mw[G];

  __device__ void issue(const Call& c, int l, int64_t n, const uint32_t* mrow, int S) {
    const int lane = lane_id(), wave = threadIdx.x / kWave;
    const int8_t* codes = c.codes + (int64_t)l * c.code_layer_stride;
    const uint16_t* scales = c.scales + (int64_t)l * c.scale_layer_stride;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const int j = (wave + g * (kPrepThreads / kWave)) * 16 + (lane & 15);
      if (S == 0) {
#pragma unroll
        for (int cc = 0; cc < KC; ++cc) {
          kb[g][cc] = {};
          ks[g][cc] = 0;
        }
        mw[g] = 0u;
        continue;
      }
      const int64_t b = sample_block<NS>(j < S ? j : 0, n);
      const int8_t* row = codes + b * c.ldc + 8 * (lane >> 4);
#pragma unroll
      for (int cc = 0; cc < KC; ++cc) {
        kb[g][cc] = *reinterpret_cast<const uint2*>(row + 32 * cc);
        ks[g][cc] = scales[b * c.lds + cc];
      }
      mw[g] = mrow ? mrow[b >> 5] : 0xFFFFFFFFu;
      if (j >= S) mw[g] = 0u;
    }
  }

  __device__ void stage(const Call&, int64_t, Shared&) {}

  // One 32-column group at a time over both sample groups, so that each
  // group's A operand, codes and scales are dead once its MFMAs are issued.
  __device__ void finish(int64_t n, int S, int64_t lim, Shared& sh) {
    const int lane = lane_id(), wave = threadIdx.x / kWave;
    float sc[G];
#pragma unroll
    for (int g = 0; g < G; ++g) sc[g] = 0.f;
#pragma unroll
    for (int cc = 0; cc < KC; ++cc) {
      u32x4_t v = {0u, 0u, 0u, 0u};
      if ((lane & 15) == 0) {
        const float* qr = &sh.q[32 * cc + 8 * (lane >> 4)];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          v[e] = (uint32_t)f32_to_bf16_rne(qr[2 * e]) | ((uint32_t)f32_to_bf16_rne(qr[2 * e + 1]) << 16);
      }
      const bf16x8_t a = __builtin_bit_cast(bf16x8_t, v);
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const u32x4_t bv = {bf16_pair_of_codes(kb[g][cc].x, 0), bf16_pair_of_codes(kb[g][cc].x, 16),
                            bf16_pair_of_codes(kb[g][cc].y, 0), bf16_pair_of_codes(kb[g][cc].y, 16)};
        const f32x4_t acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            a, __builtin_bit_cast(bf16x8_t, bv), f32x4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
        sc[g] += half_bits_to_f32(ks[g][cc]) * acc[0];
      }
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const int j = (wave + g * (kPrepThreads / kWave)) * 16 + (lane & 15);
      if (lane < 16 && j < S) {
        const int64_t b = sample_block<NS>(j, n);
        if (b < lim && ((mw[g] >> (b & 31)) & 1u)) sh.skey[j] = score_to_key(sc[g]);
      }
    }
  }
};

// Sampled keys of one row under the per-head ReLU score: the same sampled
// blocks and mask words as SampleMfma, scored against every head of the row
// on the matrix cores (relu_heads.h) with the row's heads staged in LDS; no
// fold.
template <int D, int NS>
struct SampleRelu {
  static constexpr int kSamples = NS;
  static constexpr int G = kGroupsPerWave<NS>;
  static constexpr bool kFold = false;
  using Shared = FoldShared<kReluStageBytes / 4>;
  static constexpr int KC = D / 32;
  relu_u32x4_t kb[G][KC];
  uint32_t mw[G];
  ReluStage st;

  __device__ void issue(const Call& c, int l, int64_t n, const uint32_t* mrow, int S) {
    const int lane = lane_id(), wave = threadIdx.x / kWave;
    const uint16_t* K = c.keys + (int64_t)l * c.key_layer_stride;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const int j = (wave + g * (kPrepThreads / kWave)) * 16 + (lane & 15);
      if (S == 0) {
#pragma unroll
        for (int cc = 0; cc < KC; ++cc) kb[g][cc] = {};
        mw[g] = 0u;
        continue;
      }
      const int64_t b = sample_block<NS>(j < S ? j : 0, n);
      const uint16_t* row = K + b * c.ldk + 8 * (lane >> 4);
#pragma unroll
      for (int cc = 0; cc < KC; ++cc) kb[g][cc] = *reinterpret_cast<const relu_u32x4_t*>(row + 32 * cc);
      mw[g] = mrow ? mrow[b >> 5] : 0xFFFFFFFFu;
      if (j >= S) mw[g] = 0u;
    }
  }

  __device__ void stage(const Call& c, int64_t lr, Shared& sh) {
    st = relu_stage_heads<1, D>(c, lr, sh.relu, threadIdx.x, kPrepThreads);
  }

  // The row's score of a sampled block is complete in all four lanes of its
  // column; lanes 0-15 store it.
  __device__ void finish(int64_t n, int S, int64_t lim, Shared& sh) {
    const int lane = lane_id(), wave = threadIdx.x / kWave;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float one[1][1];
      relu_all_rows<1, D, 1, false>(st, reinterpret_cast<const relu_u32x4_t(&)[1][KC]>(kb[g]), one);
      const int j = (wave + g * (kPrepThreads / kWave)) * 16 + (lane & 15);
      if (lane < 16 && j < S) {
        const int64_t b = sample_block<NS>(j, n);
        if (b < lim && ((mw[g] >> (b & 31)) & 1u)) sh.skey[j] = score_to_key(one[0][0]);
      }
    }
  }
};

// A floor for the j-th largest of the NS keys a wave holds (NS / 64 per lane):
// the largest x with at least j keys >= x, built bit by bit from the top, over
// the top 16 bits only (sign, exponent and 7 mantissa bits of the score).
// It is at most the j-th largest key and lets through at most the keys that
// share its 16-bit prefix besides.
template <int NS>
__device__ __forceinline__ uint32_t wave_jth_largest(const uint32_t (&v)[NS / kWave], int j) {
  uint32_t x = 0;
#pragma unroll 1
  for (int bit = 31; bit >= 16; --bit) {
    const uint32_t t = x | (1u << bit);
    int n = 0;
#pragma unroll
    for (int i = 0; i < NS / kWave; ++i) n += __popcll(__ballot(v[i] >= t));
    if (n >= j) x = t;
  }
  return x;
}

// Row r's limit, clamped to [0, N].
__device__ __forceinline__ int64_t row_limit(const Call& c, int l, int r) {
  const int64_t v = c.limit ? (int64_t)c.limit[(int64_t)l * c.rows + r] : c.blocks;
  return v < 0 ? 0 : (v > c.blocks ? c.blocks : v);
}

// Workgroup r < R of layer l: row r's admitted count, fold and floor (and,
// in workgroup 0, the union's count).  The sampled key rows and the row's
// mask words at them are issued first, then the row's query heads and
// weights, then the mask words to count.  One workgroup per row keeps the
// bytes each compute unit pulls in small: the row's heads (H d bf16) and the
// sampled key rows.
template <int R, int D, class Sampler>
__device__ void row_tile(const Call& c, int l, int r, typename Sampler::Shared& sh) {
  const int H = c.heads;
  const int tid = threadIdx.x, lane = lane_id();
  const int64_t lr = (int64_t)l * R + r;
  const int64_t lim = row_limit(c, l, r);
  const uint32_t* mask_l = c.mask ? c.mask + (int64_t)l * c.mask_layer_stride : nullptr;
  const uint32_t* mrow = c.mode == kRowMask ? mask_l + (int64_t)r * c.mask_row_stride : mask_l;
  int32_t* counts = c.counts + (int64_t)l * kCountStride;

  // Sampled key rows: spread over [0, N), so that their addresses wait for
  // nothing (samples at or past the row's limit are simply not admitted).
  const int64_t N = c.blocks;
  const int S = N < Sampler::kSamples ? (int)N : Sampler::kSamples;
  Sampler smp;
  smp.issue(c, l, N, mrow, S);
  for (int i = tid; i < Sampler::kSamples; i += kPrepThreads) sh.skey[i] = 0u;

  // fold, first half: thread (slice hs, chunk) sums w_h q_h[i0 .. i0 + 4) over
  // its slice of heads, ascending h, four heads' loads at a time.  Four
  // columns and four heads per step keep the workgroup within 64 VGPRs at
  // d <= 128 while the sampled rows are in flight, so that two workgroups fit
  // on a compute unit.  The per-head ReLU score has no fold: its sampler
  // stages the row's heads instead.
  constexpr int chunks = D / 4;
  constexpr int slices = kFoldSlices;
  const int hper = (H + slices - 1) / slices;
  if constexpr (!Sampler::kFold) smp.stage(c, lr, sh);
  if (Sampler::kFold && tid < chunks * slices) {
    const int ch = tid % chunks, hs = tid / chunks;
    const int i0 = ch * 4;
    float acc[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] = 0.0f;
    const int h0 = hs * hper, h1 = h0 + hper < H ? h0 + hper : H;
    for (int hb = h0; hb < h1; hb += kFoldBatch) {
      uint2 qv[kFoldBatch];
      float wv[kFoldBatch];
#pragma unroll
      for (int u = 0; u < kFoldBatch; ++u) {
        const int h = hb + u < h1 ? hb + u : h1 - 1;  // repeated loads past h1 are not summed
        qv[u] = *reinterpret_cast<const uint2*>(c.q + (lr * H + h) * D + i0);
        wv[u] = bf16_to_f32(c.w[lr * H + h]);
      }
#pragma unroll
      for (int u = 0; u < kFoldBatch; ++u) {
        if (hb + u >= h1) break;
        acc[0] = fmaf(wv[u], bf16_lo(qv[u].x), acc[0]);
        acc[1] = fmaf(wv[u], bf16_hi(qv[u].x), acc[1]);
        acc[2] = fmaf(wv[u], bf16_lo(qv[u].y), acc[2]);
        acc[3] = fmaf(wv[u], bf16_hi(qv[u].y), acc[3]);
      }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) sh.part[hs * D + i0 + e] = acc[e];
  }
  if (tid < 2) sh.acc[tid] = 0;

  // The row's mask words to count (all words below N: the limit is applied
  // when counting), issued once the fold's loads are consumed.
  constexpr int kCountWords = 4;  // per thread in flight: masks up to 131072 blocks
  const int64_t all_words = (N + 31) / 32;
  uint32_t cw[kCountWords];
#pragma unroll
  for (int i = 0; i < kCountWords; ++i) {
    const int64_t j = tid + (int64_t)i * kPrepThreads;
    cw[i] = (mrow && j < all_words) ? mrow[j] : 0u;
  }

  __syncthreads();
  // fold, second half: the slices' partial sums in ascending slice order; the
  // three-way bf16 split (exact for |q~_i| >= 2^-110)
  for (int i = tid; Sampler::kFold && i < D; i += kPrepThreads) {
    float acc = 0.0f;
#pragma unroll
    for (int hs = 0; hs < slices; ++hs) acc += sh.part[hs * D + i];
    sh.q[i] = acc;
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

  // sample keys (the sampled rows' registers are free afterwards)
  smp.finish(N, S, lim, sh);

  // admitted counts: the row's, and in workgroup 0 the union's
  if (c.mode == kNoMask) {
    if (tid == 0) {
      sh.acc[0] = (int)lim;
      if (r == 0) {
        const Limits s = layer_limits<R>(c, l);
        sh.acc[1] = (int)s.maxlim;
      }
    }
  } else {
    const int64_t words = (lim + 31) / 32;
    int rc = 0;
#pragma unroll
    for (int i = 0; i < kCountWords; ++i) {
      const int64_t j = tid + (int64_t)i * kPrepThreads;
      if (j < words) rc += __popc(cw[i] & below_limit_bits(j, lim));
    }
    for (int64_t j = tid + (int64_t)kCountWords * kPrepThreads; j < words; j += kPrepThreads)
      rc += __popc(mrow[j] & below_limit_bits(j, lim));
    rc = wave_sum(rc);
    if (lane == 0 && rc) atomicAdd(&sh.acc[0], rc);
    if (r == 0) {
      const Limits s = layer_limits<R>(c, l);
      const int64_t uwords = (s.maxlim + 31) / 32;
      int uc = 0;
      int64_t j0 = tid;
      if (c.mode == kSharedMask) {
#pragma unroll
        for (int i = 0; i < kCountWords; ++i) {
          const int64_t j = tid + (int64_t)i * kPrepThreads;
          if (j < uwords) uc += __popc(cw[i] & below_limit_bits(j, s.maxlim));
        }
        j0 = tid + (int64_t)kCountWords * kPrepThreads;
      }
      for (int64_t j = j0; j < uwords; j += kPrepThreads) uc += __popc(union_word<R>(c, mask_l, s, j));
      uc = wave_sum(uc);
      if (lane == 0 && uc) atomicAdd(&sh.acc[1], uc);
    }
  }

  __syncthreads();
  if (tid == 0) counts[r] = sh.acc[0];
  if (tid == 1 && r == 0) counts[kMaxRows] = sh.acc[1];

  // floor: wave 0 finds the row's jth largest sample key
  if (tid < kWave) {
    constexpr int NS = Sampler::kSamples;
    uint32_t v[NS / kWave];
    int sr = 0;  // admitted samples: the non-zero keys
#pragma unroll
    for (int i = 0; i < NS / kWave; ++i) {
      v[i] = sh.skey[i * kWave + lane];
      sr += __popcll(__ballot(v[i] != 0u));
    }
    const int64_t n = sh.acc[0];
    const int64_t m = n < c.k ? n : c.k;
    uint32_t floor = 0;
    if (sr > 0 && n > 3 * m) {
      const int64_t jth = (3 * m * sr + n - 1) / n + 8;
      if (jth <= sr) floor = wave_jth_largest<NS>(v, (int)jth);
    }
    if (lane == 0) {
      c.floor_key[lr] = floor;
      c.cand_count[lr * kCountPad] = 0;
    }
  }
}

// Expanding workgroups per layer: one per 16 tiles, at most kMaxExpanders.
// Expander x (1-based) takes the contiguous tiles [(x-1) tpe, x tpe), tpe
// the tiles per expander rounded up to a multiple of 16, in rounds of 16 (one
// tile per wave).  Each expander counts the admitted blocks of every tile
// before its own, so each mask word is read at most kMaxExpanders times and
// the work stays linear in N.
constexpr int kMaxExpanders = 64;
__host__ __device__ __forceinline__ int prep_expanders(int ntiles) {
  const int e = (ntiles + kPrepTilesPerWg - 1) / kPrepTilesPerWg;
  return e < kMaxExpanders ? e : kMaxExpanders;
}
__host__ __device__ __forceinline__ int expander_tiles(int ntiles, int expanders) {
  const int per = (ntiles + expanders - 1) / expanders;
  return (per + kPrepTilesPerWg - 1) / kPrepTilesPerWg * kPrepTilesPerWg;
}

// Expanding workgroup x >= 1 of layer l: its tiles of the union, in order.
template <int R>
__device__ void expand_tiles(const Call& c, int l, int x, ExpandShared& sh) {
  const int tid = threadIdx.x, lane = lane_id(), wave = tid / kWave;
  const int tpe = expander_tiles(c.ntiles, prep_expanders(c.ntiles));
  const int t_begin = (x - 1) * tpe;
  if (t_begin >= c.ntiles) return;  // uniform: nothing left for this expander
  const int t_end = t_begin + tpe < c.ntiles ? t_begin + tpe : c.ntiles;
  const Limits s = layer_limits<R>(c, l);
  const uint32_t* mask_l = c.mask + (int64_t)l * c.mask_layer_stride;
  const int64_t words = (s.maxlim + 31) / 32;

  // the first round's tile word (loaded alongside the earlier tiles' words)
  int t = t_begin + wave;
  int64_t j = (int64_t)t * kTileWords + lane;
  uint32_t u = (t < t_end && j < words) ? union_word<R>(c, mask_l, s, j) : 0u;

  // admitted blocks of all earlier tiles
  int before = 0;
  const int64_t w_end = (int64_t)t_begin * kTileWords < words ? (int64_t)t_begin * kTileWords : words;
  for (int64_t jj = tid; jj < w_end; jj += kPrepThreads) before += __popc(union_word<R>(c, mask_l, s, jj));
  if (tid == 0) sh.before = 0;
  __syncthreads();
  before = wave_sum(before);
  if (lane == 0 && before) atomicAdd(&sh.before, before);

  for (int t0 = t_begin; t0 < t_end; t0 += kPrepTilesPerWg) {
    if (t0 != t_begin) {
      t = t0 + wave;
      j = (int64_t)t * kTileWords + lane;
      u = (t < t_end && j < words) ? union_word<R>(c, mask_l, s, j) : 0u;
    }
    // place the tile's admitted blocks in order: lane i's k-th set bit goes to
    // its exclusive prefix + k.  Each lane walks its 32 bits starting at bit
    // i % 32, so at every step the lanes write to different LDS banks.
    const int cnt = __popc(u);
    const int in_tile = wave_inclusive_scan(cnt) - cnt;
    const int tile_total = __shfl(in_tile + cnt, kWave - 1, kWave);
    if (lane == 0) sh.tile_cnt[wave] = tile_total;
    const int32_t b0 = (int32_t)(j * 32);
    const int32_t tb = t * kTileBlocks;  // the tile's first block
#pragma unroll 1  // unrolled, the 32 placements need more than 128 VGPRs
    for (int step = 0; step < 32; ++step) {
      const int bit = (step + lane) & 31;
      if ((u >> bit) & 1u) sh.stage[wave][in_tile + __popc(u & ((1u << bit) - 1u))] = (uint16_t)(b0 + bit - tb);
    }
    __syncthreads();
    int total = 0;
    const int mine = tid < kPrepWaves ? sh.tile_cnt[tid] : 0;
    const int excl = block_exclusive_scan<kPrepThreads>(mine, &total, sh.scan);
    if (tid < kPrepWaves) sh.tile_cnt[tid] = excl;
    __syncthreads();
    int32_t* out = c.list + (int64_t)l * c.blocks + sh.before + sh.tile_cnt[wave];
    for (int i = lane; i < tile_total; i += kWave) out[i] = tb + (int32_t)sh.stage[wave][i];
    __syncthreads();  // the round's counts and runs are read before the next round rewrites them
    if (tid == 0) sh.before += total;
  }
}

// At most 80 SGPRs: measured on gfx950, a 1024-thread workgroup whose waves
// hold 96 or more SGPRs leaves no room for a second one on its compute unit
// (and a few SGPRs then spill into VGPR lanes instead), while at 80 two row
// or expanding workgroups share a unit, which the layers' R + E workgroups
// per layer need once they outnumber the units.
template <int R, int D, class Sampler>
__global__ __launch_bounds__(kPrepThreads) __attribute__((amdgpu_num_sgpr(80))) void prep_kernel(Call c) {
  __shared__ PrepShared<typename Sampler::Shared> sh;
  // blockIdx.x is the layer, so that consecutive workgroups (which the
  // dispatcher deals out to the XCDs in turn) belong to different layers and
  // the layers' row workgroups spread over every XCD.
  if ((int)blockIdx.y < R) row_tile<R, D, Sampler>(c, blockIdx.x, blockIdx.y, sh.f);
  else expand_tiles<R>(c, blockIdx.x, blockIdx.y - R + 1, sh.e);
}

template <int R, int D, int NS>
void launch_rdn(const Call& c, dim3 grid, hipStream_t stream) {
  if (c.fmt == kKeysQ8)
    hipLaunchKernelGGL((prep_kernel<R, D, SampleMfmaQ8<D, NS>>), grid, dim3(kPrepThreads), 0, stream, c);
  else if (c.score_kind == kScoreHeadRelu)
    hipLaunchKernelGGL((prep_kernel<R, D, SampleRelu<D, NS>>), grid, dim3(kPrepThreads), 0, stream, c);
  else
    hipLaunchKernelGGL((prep_kernel<R, D, SampleMfma<D, NS>>), grid, dim3(kPrepThreads), 0, stream, c);
}

template <int R, int D>
void launch_rd(const Call& c, dim3 grid, hipStream_t stream) {
  if (c.layers == 1) launch_rdn<R, D, kSamplesOneLayer>(c, grid, stream);
  else launch_rdn<R, D, kSamplesBatched>(c, grid, stream);
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
  const int expanders = c.mode == kNoMask ? 0 : prep_expanders(c.ntiles);
  dim3 grid(c.layers, c.rows + expanders);
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
