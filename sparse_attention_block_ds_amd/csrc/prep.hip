// prep: admission + compaction of the admitted index, the head-weight fold,
// and clearing of the first-digit histograms, for every layer of one call.
//
// Compaction (page "DeepSeek V4.1F Q4 on M3 Ultra with native DSpark MTP
// (40tps / 800tps)", paragraph "Decode at depth": the admitted index is
// compacted once per row, so no later stage tests the mask again).  One
// workgroup per layer walks the mask words in order: each thread takes a run
// of words, ANDs them with the causal limits, popcounts them, a workgroup
// prefix sum turns the counts into write offsets, and each thread expands its
// words' set bits into ascending block indices.  When all rows of a layer share
// one mask row, the rows' lists are prefixes of that one list (they differ only
// by their limits), so the list is written once and each row keeps its length.
// Without a mask the compacted index is the identity and nothing is written.
//
// Fold: score = sum_h w_h (q_h . K_b) = (sum_h w_h q_h) . K_b, so each row's
// H query heads collapse into one fp32 vector q~ before the key stream.  The
// products w_h q_hi are bf16 x bf16 and exact in fp32; the sum over h runs in
// ascending h.  q~ stays fp32 (never rounded back to bf16).
#include "device_util.h"
#include "dssel_internal.h"

namespace dssel {
namespace {

__device__ __forceinline__ int64_t clamp_limit(const int32_t* limit, int64_t idx, int64_t n) {
  if (!limit) return n;
  int64_t v = limit[idx];
  return v < 0 ? 0 : (v > n ? n : v);
}

// Bits of mask word j (blocks 32j .. 32j+31) that lie below `lim`.
__device__ __forceinline__ uint32_t below_limit_bits(int64_t j, int64_t lim) {
  const int64_t lo = j * 32;
  if (lim >= lo + 32) return 0xFFFFFFFFu;
  if (lim <= lo) return 0u;
  return (1u << (uint32_t)(lim - lo)) - 1u;
}

__device__ void compact_layer(const Call& c, int l) {
  __shared__ int scan_scratch[kPrepThreads / kWave + 1];
  __shared__ int row_totals[kMaxRows];
  const int R = c.rows;
  const int64_t N = c.blocks;
  const int tid = threadIdx.x;

  int64_t lim[kMaxRows];
  int64_t maxlim = 0;
#pragma unroll
  for (int r = 0; r < kMaxRows; ++r) {
    lim[r] = r < R ? clamp_limit(c.limit, (int64_t)l * R + r, N) : 0;
    maxlim = lim[r] > maxlim ? lim[r] : maxlim;
  }
  int32_t* counts = c.counts + (int64_t)l * kCountStride;

  if (c.mode == kNoMask) {
    if (tid < R) counts[tid] = (int32_t)lim[tid];
    if (tid == 0) counts[kMaxRows] = (int32_t)maxlim;
    return;
  }

  if (tid < kMaxRows) row_totals[tid] = 0;
  const int64_t words = (maxlim + 31) / 32;
  const uint32_t* mrow0 = c.mask + (int64_t)l * c.mask_layer_stride;
  int32_t* list = c.list + (int64_t)l * N;
  int row_count[kMaxRows];
#pragma unroll
  for (int r = 0; r < kMaxRows; ++r) row_count[r] = 0;

  int64_t base = 0;
  constexpr int V = kPrepWordsPerThread;
  for (int64_t chunk = 0; chunk < words; chunk += (int64_t)kPrepThreads * V) {
    uint32_t uw[V];
    int mine = 0;
    const int64_t j0 = chunk + (int64_t)tid * V;
#pragma unroll
    for (int v = 0; v < V; ++v) {
      const int64_t j = j0 + v;
      uint32_t u = 0;
      if (j < words) {
        if (c.mode == kSharedMask) {
          u = mrow0[j] & below_limit_bits(j, maxlim);
#pragma unroll
          for (int r = 0; r < kMaxRows; ++r)
            if (r < R) row_count[r] += __popc(u & below_limit_bits(j, lim[r]));
        } else {
#pragma unroll
          for (int r = 0; r < kMaxRows; ++r) {
            if (r < R) {
              const uint32_t mr = mrow0[r * c.mask_row_stride + j] & below_limit_bits(j, lim[r]);
              row_count[r] += __popc(mr);
              u |= mr;
            }
          }
        }
      }
      uw[v] = u;
      mine += __popc(u);
    }
    int total = 0;
    const int excl = block_exclusive_scan<kPrepThreads>(mine, &total, scan_scratch);
    int64_t pos = base + excl;
#pragma unroll
    for (int v = 0; v < V; ++v) {
      uint32_t u = uw[v];
      const int32_t b0 = (int32_t)((j0 + v) * 32);
      while (u) {
        const int bit = __ffs(u) - 1;
        list[pos++] = b0 + bit;
        u &= u - 1;
      }
    }
    base += total;
  }
#pragma unroll
  for (int r = 0; r < kMaxRows; ++r)
    if (r < R && row_count[r]) atomicAdd(&row_totals[r], row_count[r]);
  __syncthreads();
  if (tid < R) counts[tid] = row_totals[tid];
  if (tid == 0) counts[kMaxRows] = (int32_t)base;
}

__device__ void fold_row(const Call& c, int l, int r) {
  const int H = c.heads, D = c.dim;
  const int64_t lr = (int64_t)l * c.rows + r;
  const uint16_t* qrow = c.q + lr * H * D;
  const uint16_t* wrow = c.w + lr * H;
  for (int i = threadIdx.x; i < D; i += kPrepThreads) {
    float acc = 0.0f;
    for (int h = 0; h < H; ++h) {
      const float wh = __uint_as_float((uint32_t)wrow[h] << 16);
      const float qi = __uint_as_float((uint32_t)qrow[(int64_t)h * D + i] << 16);
      acc = fmaf(wh, qi, acc);  // the product is exact, so this equals mul + add
    }
    c.qt[lr * D + i] = acc;
  }
}

__global__ __launch_bounds__(kPrepThreads) void prep_kernel(Call c) {
  const int l = blockIdx.y;
  if (blockIdx.x == 0) {
    uint32_t* h = c.hist + (int64_t)l * c.rows * kHistBins;
    for (int i = threadIdx.x; i < c.rows * kHistBins; i += kPrepThreads) h[i] = 0u;
    compact_layer(c, l);
  } else {
    fold_row(c, l, blockIdx.x - 1);
  }
}

}  // namespace

hipError_t launch_prep(const Call& c, hipStream_t stream) {
  dim3 grid(1 + c.rows, c.layers);
  hipLaunchKernelGGL(prep_kernel, grid, dim3(kPrepThreads), 0, stream, c);
  return hipGetLastError();
}

}  // namespace dssel
