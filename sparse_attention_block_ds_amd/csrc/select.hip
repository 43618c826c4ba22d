// select: the bounded radix select of the best k keys of every (layer, row),
// with ties broken by the lower block index, and the ordered output.
//
// Page "DeepSeek V4.1F Q4 on M3 Ultra with native DSpark MTP (40tps /
// 800tps)", paragraph "Decode at depth": the top 512 are taken with a radix
// select of bounded depth.  Here the depth is at most three digits of the
// 32-bit key (11 + 11 + 10 bits), each resolved with one LDS histogram, so the
// work is a fixed number of passes over the row's keys whatever the data.
//
// One workgroup per (layer, row):
//  1. From the first-digit histogram the score kernel built, find the
//     boundary bin B1: the highest bin whose keys, with every key above it,
//     number at least m = min(k, admitted).
//  2. If the keys in bins >= B1 fit the LDS buffer (the usual case: a few
//     hundred keys sit in B1), gather them as (key, position) pairs, sort
//     them by (key desc, position asc) with an LDS bitonic network, and keep
//     the first m.  Positions ascend with block index, so this is the
//     lower-index tie rule.
//  3. Otherwise (a huge run of near-equal scores), resolve digits 2 and 3 with
//     two more histogram passes to the exact k-th key T, gather every key
//     above T, add the ties at T in position order until m are taken (an
//     ordered fill with a workgroup prefix sum), and sort those m.
// Output: block indices and fp32 scores (recovered exactly from the keys),
// then padding (-1, -inf) up to k, and the count m.
#include "device_util.h"
#include "dssel_internal.h"

namespace dssel {
namespace {

constexpr int NT = kSelectThreads;

// Largest bin B in [0, nbins) with (keys in bins >= B) >= need, and the
// number of keys in bins > B.  nbins is 1024 or 2048; the histogram is in LDS.
__device__ void find_boundary(const uint32_t* hist, int nbins, int need, int* out_bin,
                              int* out_above, int* scan_scratch) {
  const int per = nbins / NT;  // 1 or 2 bins per thread, in descending bin order
  const int hi = nbins - 1 - threadIdx.x * per;
  int c_hi = (int)hist[hi];
  int c_lo = per == 2 ? (int)hist[hi - 1] : 0;
  int total = 0;
  const int excl = block_exclusive_scan<NT>(c_hi + c_lo, &total, scan_scratch);
  if (excl < need && excl + c_hi + c_lo >= need) {
    if (excl + c_hi >= need) {
      *out_bin = hi;
      *out_above = excl;
    } else {
      *out_bin = hi - 1;
      *out_above = excl + c_hi;
    }
  }
  __syncthreads();
}

__device__ __forceinline__ bool before(uint32_t ka, int pa, uint32_t kb, int pb) {
  return ka > kb || (ka == kb && pa < pb);
}

// Sort sk/sp[0, n) (n a power of two) by (key desc, pos asc) in LDS.
__device__ void bitonic_sort(uint32_t* sk, int32_t* sp, int n) {
  for (int size = 2; size <= n; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int t = threadIdx.x; t < (n >> 1); t += NT) {
        const int i = 2 * t - (t & (stride - 1));
        const int j = i + stride;
        const bool up = (i & size) == 0;  // this run ends in "before" order
        const uint32_t ki = sk[i], kj = sk[j];
        const int32_t pi = sp[i], pj = sp[j];
        const bool swap = up ? before(kj, pj, ki, pi) : before(ki, pi, kj, pj);
        if (swap) {
          sk[i] = kj; sk[j] = ki;
          sp[i] = pj; sp[j] = pi;
        }
      }
      __syncthreads();
    }
  }
}

__global__ __launch_bounds__(NT) void select_kernel(Call c) {
  __shared__ uint32_t hist[kHistBins];
  __shared__ uint32_t sk[kSelectBuf];
  __shared__ int32_t sp[kSelectBuf];
  __shared__ int scan_scratch[NT / kWave + 1];
  __shared__ int sh_bin, sh_above, sh_count;

  const int l = blockIdx.y, r = blockIdx.x;
  const int R = c.rows, k = c.k;
  const int64_t lr = (int64_t)l * R + r;
  const int64_t N = c.blocks;
  const int32_t* counts = c.counts + (int64_t)l * kCountStride;
  const int n_adm = N ? counts[r] : 0;
  const int m = n_adm < k ? n_adm : k;
  const int P = (c.mode == kRowMask) ? (N ? counts[kMaxRows] : 0) : n_adm;
  const uint32_t* keys = c.skeys + (int64_t)l * R * N + (int64_t)r * N;
  const int32_t* list = c.list + (int64_t)l * N;
  int32_t* oi = c.out_idx + lr * k;
  float* os = c.out_score + lr * k;
  const int tid = threadIdx.x;

  if (m > 0) {
    for (int i = tid; i < kHistBins; i += NT) hist[i] = c.hist[lr * kHistBins + i];
    if (tid == 0) {
      sh_count = 0;
      sh_bin = 0;
      sh_above = 0;
    }
    __syncthreads();
    find_boundary(hist, kHistBins, m, &sh_bin, &sh_above, scan_scratch);
    const uint32_t B1 = (uint32_t)sh_bin;
    const int above1 = sh_above;
    const int gathered = above1 + (int)hist[B1];

    if (gathered <= kSelectBuf) {
      // 2. gather every key whose first digit is >= B1
      for (int p0 = 0; p0 < P; p0 += NT) {
        const int p = p0 + tid;
        uint32_t key = 0;
        if (p < P) key = keys[p];
        const bool want = p < P && key != 0u && (key >> kDigit1Shift) >= B1;
        const int slot = wave_append(want, &sh_count);
        if (want && slot < kSelectBuf) {
          sk[slot] = key;
          sp[slot] = p;
        }
      }
      __syncthreads();
      int n = 1;
      while (n < gathered) n <<= 1;
      for (int i = gathered + tid; i < n; i += NT) {
        sk[i] = 0u;
        sp[i] = 0x7FFFFFFF;
      }
      __syncthreads();
      bitonic_sort(sk, sp, n);
    } else {
      // 3. bounded fallback: two more digits, then an ordered fill of the ties
      int need = m - above1;
      for (int i = tid; i < kHistBins; i += NT) hist[i] = 0u;
      __syncthreads();
      for (int p = tid; p < P; p += NT) {
        const uint32_t key = keys[p];
        if (key != 0u && (key >> kDigit1Shift) == B1)
          atomicAdd(&hist[(key >> kDigit2Shift) & (kHistBins - 1)], 1u);
      }
      __syncthreads();
      find_boundary(hist, kHistBins, need, &sh_bin, &sh_above, scan_scratch);
      const uint32_t prefix2 = (B1 << 11) | (uint32_t)sh_bin;
      need -= sh_above;
      for (int i = tid; i < kHistBins; i += NT) hist[i] = 0u;
      __syncthreads();
      for (int p = tid; p < P; p += NT) {
        const uint32_t key = keys[p];
        if (key != 0u && (key >> kDigit2Shift) == prefix2)
          atomicAdd(&hist[key & (kDigit3Bins - 1)], 1u);
      }
      __syncthreads();
      find_boundary(hist, kDigit3Bins, need, &sh_bin, &sh_above, scan_scratch);
      const uint32_t T = (prefix2 << 10) | (uint32_t)sh_bin;
      need -= sh_above;            // ties at T still to take, >= 1
      const int strict = m - need; // keys > T, all of them selected
      // every key above T (order restored by the sort)
      for (int p0 = 0; p0 < P; p0 += NT) {
        const int p = p0 + tid;
        const uint32_t key = p < P ? keys[p] : 0u;
        const bool want = key > T;
        const int slot = wave_append(want, &sh_count);
        if (want && slot < kSelectBuf) {
          sk[slot] = key;
          sp[slot] = p;
        }
      }
      // the first `need` ties at T in position order
      int taken = 0;
      for (int p0 = 0; p0 < P && taken < need; p0 += NT) {
        const int p = p0 + tid;
        const bool tie = p < P && keys[p] == T;
        int chunk_total = 0;
        const int rank = taken + block_exclusive_scan<NT>(tie ? 1 : 0, &chunk_total, scan_scratch);
        if (tie && rank < need) {
          sk[strict + rank] = T;
          sp[strict + rank] = p;
        }
        taken += chunk_total;
      }
      __syncthreads();
      int n = 1;
      while (n < m) n <<= 1;
      for (int i = m + tid; i < n; i += NT) {
        sk[i] = 0u;
        sp[i] = 0x7FFFFFFF;
      }
      __syncthreads();
      bitonic_sort(sk, sp, n);
    }
  }

  for (int j = tid; j < k; j += NT) {
    if (j < m) {
      const int p = sp[j];
      oi[j] = (c.mode == kNoMask) ? p : list[p];
      os[j] = key_to_score(sk[j]);
    } else {
      oi[j] = -1;
      os[j] = -__builtin_inff();
    }
  }
  if (tid == 0 && c.out_count) c.out_count[lr] = m;
}

}  // namespace

hipError_t launch_select(const Call& c, hipStream_t stream) {
  dim3 grid(c.rows, c.layers);
  hipLaunchKernelGGL(select_kernel, grid, dim3(kSelectThreads), 0, stream, c);
  return hipGetLastError();
}

}  // namespace dssel
