// prep: the admission directory, the head-weight fold, and clearing of the
// first-digit histograms, for every layer of one call.
//
// Admission directory (page "DeepSeek V4.1F Q4 on M3 Ultra with native DSpark
// MTP (40tps / 800tps)", paragraph "Decode at depth": the admitted index is
// compacted once per row).  The block axis is cut into tiles of 2048 blocks
// (64 mask words).  One workgroup per layer reads the mask words coalesced,
// one wave per tile: each lane ANDs its word with the causal limits and
// popcounts it, a wave prefix sum places the word inside its tile, a workgroup
// prefix sum over the tiles places the tile, and each lane writes its word's
// admitted block indices at their compacted positions: the compacted index is
// built in one pass, in ascending order.  When all rows share one mask row, the
// rows' lists are prefixes of one list (they differ only by their limits): each
// row keeps only its length.  Without a mask the compacted index is the
// identity and nothing is built.
//
// Fold: score = sum_h w_h (q_h . K_b) = (sum_h w_h q_h) . K_b, so each row's
// H query heads collapse into one fp32 vector q~ before the key stream.  The
// products w_h q_hi are bf16 x bf16 and exact in fp32.  Thread (g, i) of the
// fold workgroup sums head group g of column i in ascending h, and the groups
// are added in a fixed tree, so the result is the same on every run.  For the
// matrix cores q~ is also split exactly into three bf16 parts, hi = bf16(q~),
// mid = bf16(q~ - hi), lo = bf16(q~ - hi - mid), with hi + mid + lo == q~
// (each step keeps 8 more significant bits of the 24).
#include "device_util.h"
#include "dssel_internal.h"

namespace dssel {
namespace {

constexpr int kPrepWaves = kPrepThreads / kWave;

__device__ __forceinline__ int64_t clamp_limit(const int32_t* limit, int64_t idx, int64_t n) {
  if (!limit) return n;
  int64_t v = limit[idx];
  return v < 0 ? 0 : (v > n ? n : v);
}

__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
  for (int off = kWave / 2; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

__device__ void tile_directory(const Call& c, int l) {
  __shared__ int scan_scratch[kPrepWaves + 1];
  __shared__ int tile_cnt[kPrepWaves];
  __shared__ int row_totals[kMaxRows];
  const int R = c.rows;
  const int64_t N = c.blocks;
  const int tid = threadIdx.x, lane = lane_id(), wave = tid / kWave;

  int64_t lim[kMaxRows];
  int64_t maxlim = 0;
#pragma unroll
  for (int r = 0; r < kMaxRows; ++r) {
    lim[r] = r < R ? clamp_limit(c.limit, (int64_t)l * R + r, N) : 0;
    maxlim = lim[r] > maxlim ? lim[r] : maxlim;
  }
  int32_t* counts = c.counts + (int64_t)l * kCountStride;
  if (c.mode == kNoMask) {
#pragma unroll
    for (int r = 0; r < kMaxRows; ++r)
      if (tid == r && r < R) counts[r] = (int32_t)lim[r];
    if (tid == 0) counts[kMaxRows] = (int32_t)maxlim;
    return;
  }

  if (tid < kMaxRows) row_totals[tid] = 0;
  const int64_t words = (maxlim + 31) / 32;
  const uint32_t* mrow0 = c.mask + (int64_t)l * c.mask_layer_stride;
  int32_t* tile_off = c.tile_off + (int64_t)l * (c.ntiles + 1);
  int32_t* list = c.list + (int64_t)l * N;
  int row_count[kMaxRows];
#pragma unroll
  for (int r = 0; r < kMaxRows; ++r) row_count[r] = 0;

  int base = 0;
  // kPrepWaves tiles per pass: wave w takes tile t0 + w, lane = its word
  for (int t0 = 0; t0 < c.ntiles; t0 += kPrepWaves) {
    const int t = t0 + wave;
    const int64_t j = (int64_t)t * kTileWords + lane;
    uint32_t u = 0;
    if (t < c.ntiles && j < words) {
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
    const int cnt = __popc(u);
    const int in_tile = wave_inclusive_scan(cnt) - cnt;  // this word's offset in its tile
    if (lane == kWave - 1) tile_cnt[wave] = in_tile + cnt;
    __syncthreads();
    int total = 0;
    const int mine = tid < kPrepWaves ? tile_cnt[tid] : 0;
    const int excl = block_exclusive_scan<kPrepThreads>(mine, &total, scan_scratch);
    if (tid < kPrepWaves) tile_cnt[tid] = excl;  // tile offsets within this pass
    if (tid < kPrepWaves && t0 + tid < c.ntiles) tile_off[t0 + tid] = base + excl;
    __syncthreads();
    // expand the word's admitted blocks at their compacted positions, in order
    int pos = base + tile_cnt[wave] + in_tile;
    const int32_t b0 = (int32_t)(j * 32);
    while (u) {
      list[pos++] = b0 + (__ffs(u) - 1);
      u &= u - 1u;
    }
    base += total;
    __syncthreads();
  }
#pragma unroll
  for (int r = 0; r < kMaxRows; ++r) {
    const int v = wave_sum(row_count[r]);
    if (r < R && lane == 0 && v) atomicAdd(&row_totals[r], v);
  }
  __syncthreads();
  if (tid < R) counts[tid] = row_totals[tid];
  if (tid == 0) {
    counts[kMaxRows] = base;
    tile_off[c.ntiles] = base;
  }
}

__device__ void fold_row(const Call& c, int l, int r) {
  __shared__ float partial[kPrepThreads];
  const int H = c.heads, D = c.dim, R = c.rows;
  const int groups = kPrepThreads / D;          // 4 .. 32 head groups
  const int per = (H + groups - 1) / groups;
  const int i = threadIdx.x % D, g = threadIdx.x / D;
  const int64_t lr = (int64_t)l * R + r;
  const uint16_t* qrow = c.q + lr * H * D;
  const uint16_t* wrow = c.w + lr * H;
  const int h0 = g * per, h1 = h0 + per < H ? h0 + per : H;
  float acc = 0.0f;
#pragma unroll 8
  for (int h = h0; h < h1; ++h)
    acc = fmaf(bf16_to_f32(wrow[h]), bf16_to_f32(qrow[(int64_t)h * D + i]), acc);
  partial[threadIdx.x] = acc;
  __syncthreads();
  // fixed pairwise tree over the head groups
  for (int s = groups / 2; s > 0; s >>= 1) {
    if (g < s) partial[threadIdx.x] = partial[threadIdx.x] + partial[threadIdx.x + s * D];
    __syncthreads();
  }
  if (g == 0) {
    const float q = partial[i];
    c.qt[lr * D + i] = q;
    const uint16_t hi = f32_to_bf16_rne(q);
    const float r1 = q - bf16_to_f32(hi);   // exact: q minus its own rounding
    const uint16_t mid = f32_to_bf16_rne(r1);
    const float r2 = r1 - bf16_to_f32(mid);  // exact for the same reason
    const uint16_t lo = f32_to_bf16_rne(r2);
    uint16_t* parts = c.qparts + ((int64_t)l * 3 * R + r) * D + i;
    parts[0] = hi;
    parts[(int64_t)R * D] = mid;
    parts[(int64_t)2 * R * D] = lo;
  }
}

__global__ __launch_bounds__(kPrepThreads) void prep_kernel(Call c) {
  const int l = blockIdx.y;
  if (blockIdx.x == 0) {
    uint32_t* h = c.hist + (int64_t)l * c.rows * kHistBins;
    for (int i = threadIdx.x; i < c.rows * kHistBins; i += kPrepThreads) h[i] = 0u;
    tile_directory(c, l);
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
