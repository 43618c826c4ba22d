// score: one pass over the admitted block keys of a layer, shared by all of
// its query rows, writing each row's order-preserving radix key at the
// block's compacted position and counting the keys' first radix digit.
//
// Page "DeepSeek V4.1F Q4 on M3 Ultra with native DSpark MTP (40tps /
// 800tps)": paragraph "Decode at depth" -- only admitted blocks are scored;
// paragraph "DSpark" -- the rows of a speculative verify share one stream of
// data, here the key stream: each admitted K row is read from HBM once and
// dotted with every row's folded query.
//
// Layout (VALU path): a K row of d bf16 values is d/8 lanes x 16 bytes, so a
// wave reads 64/(d/8) whole rows per 16-byte load (1 KB, fully coalesced).
// Each lane multiplies its 8 values by the matching 8 values of every row's
// fp32 q~ (kept in registers), the d/8 partial sums of a K row are added with
// a butterfly across its lanes, and lane r of the group finishes row r:
// radix key -> keys[l][r][pos], and a workgroup-local LDS histogram of the
// first digit, added to the layer's global histogram at the end.
#include "device_util.h"
#include "dssel_internal.h"

namespace dssel {
namespace {

template <int LPR, int R>
__global__ __launch_bounds__(kScoreThreads) void score_kernel(Call c) {
  constexpr int D = LPR * 8;
  constexpr int GROUPS = kWave / LPR;  // K rows per wave per load
  constexpr int UNROLL = 4;
  constexpr int WAVES = kScoreThreads / kWave;
  __shared__ uint32_t hist[R * kHistBins];

  const int l = blockIdx.y;
  const int32_t* counts = c.counts + (int64_t)l * kCountStride;
  const int n_union = counts[kMaxRows];
  const int p0 = blockIdx.x * kScoreChunk;
  if (p0 >= n_union) return;  // uniform for the workgroup
  const int p1 = min(p0 + kScoreChunk, n_union);
  const int64_t N = c.blocks;

  int P[R];  // positions [0, P[r]) hold row r's keys
#pragma unroll
  for (int r = 0; r < R; ++r) P[r] = (c.mode == kRowMask) ? n_union : counts[r];

  for (int i = threadIdx.x; i < R * kHistBins; i += kScoreThreads) hist[i] = 0u;

  const int lane = lane_id();
  const int wave = threadIdx.x / kWave;
  const int slice = lane % LPR;
  const int grp = lane / LPR;

  float qv[R][8];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const float* qt = c.qt + ((int64_t)l * R + r) * D + slice * 8;
#pragma unroll
    for (int e = 0; e < 8; ++e) qv[r][e] = qt[e];
  }
  // Per-row mask state (only for kRowMask).
  const uint32_t* mask_l = c.mask ? c.mask + (int64_t)l * c.mask_layer_stride : nullptr;
  int64_t lim[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    int64_t v = c.limit ? (int64_t)c.limit[(int64_t)l * R + r] : N;
    lim[r] = v < 0 ? 0 : (v > N ? N : v);
  }
  __syncthreads();

  const uint16_t* K = c.keys + (int64_t)l * c.key_layer_stride;
  const int32_t* list = c.list + (int64_t)l * N;
  uint32_t* skeys = c.skeys + (int64_t)l * R * N;

  for (int base = p0 + wave * GROUPS * UNROLL; base < p1; base += WAVES * GROUPS * UNROLL) {
    uint4 kv[UNROLL];
    int pos[UNROLL];
    int blk[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      pos[u] = base + u * GROUPS + grp;
      blk[u] = 0;
      kv[u] = make_uint4(0u, 0u, 0u, 0u);
      if (pos[u] < p1) {
        blk[u] = (c.mode == kNoMask) ? pos[u] : list[pos[u]];
        kv[u] = *reinterpret_cast<const uint4*>(K + (int64_t)blk[u] * c.ldk + slice * 8);
      }
    }
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const uint32_t kw[4] = {kv[u].x, kv[u].y, kv[u].z, kv[u].w};
      float acc[R];
#pragma unroll
      for (int r = 0; r < R; ++r) acc[r] = 0.0f;
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) {
        const float x0 = bf16_lo(kw[e2]);
        const float x1 = bf16_hi(kw[e2]);
#pragma unroll
        for (int r = 0; r < R; ++r) {
          acc[r] = fmaf(qv[r][2 * e2], x0, acc[r]);
          acc[r] = fmaf(qv[r][2 * e2 + 1], x1, acc[r]);
        }
      }
#pragma unroll
      for (int m = 1; m < LPR; m <<= 1) {
#pragma unroll
        for (int r = 0; r < R; ++r) acc[r] += __shfl_xor(acc[r], m, kWave);
      }
      if (pos[u] < p1) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
          if (r % LPR != slice || pos[u] >= P[r]) continue;
          bool admitted = true;
          if (c.mode == kRowMask) {
            const int b = blk[u];
            const uint32_t word = mask_l[r * c.mask_row_stride + (b >> 5)];
            admitted = ((word >> (b & 31)) & 1u) && (int64_t)b < lim[r];
          }
          const uint32_t key = admitted ? score_to_key(acc[r]) : 0u;
          skeys[(int64_t)r * N + pos[u]] = key;
          if (admitted) atomicAdd(&hist[r * kHistBins + (key >> kDigit1Shift)], 1u);
        }
      }
    }
  }
  __syncthreads();
  uint32_t* ghist = c.hist + (int64_t)l * R * kHistBins;
  for (int i = threadIdx.x; i < R * kHistBins; i += kScoreThreads) {
    const uint32_t v = hist[i];
    if (v) atomicAdd(&ghist[i], v);
  }
}

template <int LPR>
hipError_t launch_rows(const Call& c, dim3 grid, hipStream_t s) {
  switch (c.rows) {
#define DSSEL_ROWS_CASE(RR) \
  case RR: hipLaunchKernelGGL((score_kernel<LPR, RR>), grid, dim3(kScoreThreads), 0, s, c); break;
    DSSEL_ROWS_CASE(1)
    DSSEL_ROWS_CASE(2)
    DSSEL_ROWS_CASE(3)
    DSSEL_ROWS_CASE(4)
    DSSEL_ROWS_CASE(5)
    DSSEL_ROWS_CASE(6)
    DSSEL_ROWS_CASE(7)
    DSSEL_ROWS_CASE(8)
#undef DSSEL_ROWS_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_score(const Call& c, hipStream_t stream) {
  if (c.blocks == 0) return hipSuccess;
  const int64_t chunks = (c.blocks + kScoreChunk - 1) / kScoreChunk;
  dim3 grid((unsigned)chunks, c.layers);
  switch (c.dim) {
    case 32: return launch_rows<4>(c, grid, stream);
    case 64: return launch_rows<8>(c, grid, stream);
    case 128: return launch_rows<16>(c, grid, stream);
    case 256: return launch_rows<32>(c, grid, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace dssel
