// select: the bounded radix select of the best k keys of every (layer, row),
// with ties broken by the lower block index, and the ordered output.
//
// Page "DeepSeek V4.1F Q4 on M3 Ultra with native DSpark MTP (40tps /
// 800tps)", paragraph "Decode at depth": the top 512 are taken with a radix
// select of bounded depth.  Here the depth is at most three digits of the
// 32-bit key (11 + 11 + 10 bits), each resolved with one LDS histogram, so the
// work is a fixed number of passes over the row's keys whatever the data.
//
// A candidate is the 64-bit word (key << 32) | ~position: a larger word is a
// higher score, or an equal score at a lower position.  Positions ascend with
// block index, so one unsigned compare is the whole output order, ties to the
// lower block index included.
//
// One workgroup per (layer, row):
//  1. From the first-digit histogram the score kernel built, find the
//     boundary bin B1: the highest bin whose keys, with every key above it,
//     number at least m = min(k, admitted).
//  2. If the keys in bins >= B1 fit the LDS buffer (the usual case: a few
//     hundred keys sit in B1), gather them with 16-byte loads, sort them
//     descending with an LDS bitonic network, and keep the first m.
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
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint64_t pack(uint32_t key, int pos) {
  return ((uint64_t)key << 32) | (uint32_t)~(uint32_t)pos;
}
__device__ __forceinline__ uint32_t key_of(uint64_t e) { return (uint32_t)(e >> 32); }
__device__ __forceinline__ int pos_of(uint64_t e) { return (int)~(uint32_t)e; }

// Largest bin B in [0, nbins) with (keys in bins >= B) >= need, and the
// number of keys in bins > B.  nbins is 1024 or 2048; the histogram is in LDS.
__device__ void find_boundary(const uint32_t* hist, int nbins, int need, int* out_bin,
                              int* out_above, int* scan_scratch) {
  const int per = nbins / NT;  // 1 or 2 bins per thread, in descending bin order
  const int hi = nbins - 1 - threadIdx.x * per;
  const int c_hi = (int)hist[hi];
  const int c_lo = per == 2 ? (int)hist[hi - 1] : 0;
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

// Order this wave's earlier LDS writes before its later LDS reads.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Sort se[0, n) (n a power of two) descending in LDS.  Thread t handles the
// compare-exchange pairs t, t + NT, ...; for strides <= 64 the pairs of wave w
// stay inside its own 128-element spans, so only stages whose neighbours cross
// waves need a workgroup barrier.
__device__ void bitonic_sort_desc(uint64_t* se, int n) {
  for (int size = 2; size <= n; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int t = threadIdx.x; t < (n >> 1); t += NT) {
        const int i = 2 * t - (t & (stride - 1));
        const int j = i + stride;
        const bool desc = (i & size) == 0;
        const uint64_t ei = se[i], ej = se[j];
        if (desc ? ei < ej : ei > ej) {
          se[i] = ej;
          se[j] = ei;
        }
      }
      const int next = stride > 1 ? (stride >> 1) : size;
      if (stride > 64 || next > 64) __syncthreads();
      else wave_lds_sync();
    }
  }
  __syncthreads();
}

// Zero-fill se[count, n) for the smallest power of two n >= count.
__device__ int pad_pow2(uint64_t* se, int count) {
  int n = 1;
  while (n < count) n <<= 1;
  for (int i = count + threadIdx.x; i < n; i += NT) se[i] = 0ull;
  __syncthreads();
  return n;
}

__global__ __launch_bounds__(NT) void select_kernel(Call c) {
  __shared__ uint32_t hist[kHistBins];
  __shared__ uint64_t se[kSelectBuf];
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
  const uint32_t* keys = c.skeys + lr * c.key_row;  // 16-byte aligned rows
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
    int n = 0;

    if (gathered <= kSelectBuf) {
      // 2. gather every key whose first digit is >= B1, four keys per load
      constexpr int kBatch = 4;
      const u32x4_t* k4 = reinterpret_cast<const u32x4_t*>(keys);
      const int chunks = (P + 3) >> 2;
      for (int c0 = 0; c0 < chunks; c0 += NT * kBatch) {
        u32x4_t v[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
          const int ci = c0 + u * NT + tid;
          v[u] = ci < chunks ? k4[ci] : u32x4_t{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int p = 4 * (c0 + u * NT + tid) + e;
            const uint32_t key = v[u][e];
            const bool want = p < P && key != 0u && (key >> kDigit1Shift) >= B1;
            const int slot = wave_append(want, &sh_count);
            if (want && slot < kSelectBuf) se[slot] = pack(key, p);
          }
        }
      }
      __syncthreads();
      n = pad_pow2(se, gathered);
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
      need -= sh_above;             // ties at T still to take, >= 1
      const int strict = m - need;  // keys > T, all of them selected
      for (int p0 = 0; p0 < P; p0 += NT) {
        const int p = p0 + tid;
        const uint32_t key = p < P ? keys[p] : 0u;
        const bool want = key > T;
        const int slot = wave_append(want, &sh_count);
        if (want && slot < kSelectBuf) se[slot] = pack(key, p);
      }
      int taken = 0;
      for (int p0 = 0; p0 < P && taken < need; p0 += NT) {
        const int p = p0 + tid;
        const bool tie = p < P && keys[p] == T;
        int chunk_total = 0;
        const int rank = taken + block_exclusive_scan<NT>(tie ? 1 : 0, &chunk_total, scan_scratch);
        if (tie && rank < need) se[strict + rank] = pack(T, p);
        taken += chunk_total;
      }
      __syncthreads();
      n = pad_pow2(se, m);
    }
    bitonic_sort_desc(se, n);
  }

  for (int j = tid; j < k; j += NT) {
    if (j < m) {
      const uint64_t e = se[j];
      int p = pos_of(e);
      p = p < 0 ? 0 : (p >= P ? P - 1 : p);  // in range by construction; never index past it
      oi[j] = (c.mode == kNoMask) ? p : list[p];
      os[j] = key_to_score(key_of(e));
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
