// Device helpers shared by the libdssel kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dssel {

constexpr int kWave = 64;

// Order-preserving map from an fp32 score to a uint32 radix key: a larger
// score gives a larger key, and the map is a bijection on bit patterns once
// -0 has been folded onto +0 (so the score is recovered from its key).
__device__ __forceinline__ uint32_t score_to_key(float s) {
  uint32_t u = __float_as_uint(s);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float key_to_score(uint32_t key) {
  uint32_t u = (key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key;
  return __uint_as_float(u);
}

// bf16 halves of a 32-bit word, widened exactly to fp32.
__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }

__device__ __forceinline__ float bf16_to_f32(uint16_t v) { return __uint_as_float((uint32_t)v << 16); }

// Round a finite fp32 value to bf16, nearest with ties to even.
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float x) {
  const uint32_t u = __float_as_uint(x);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

// Bits of mask word j (blocks 32j .. 32j+31) that lie below `lim`.
__device__ __forceinline__ uint32_t below_limit_bits(int64_t j, int64_t lim) {
  const int64_t lo = j * 32;
  if (lim >= lo + 32) return 0xFFFFFFFFu;
  if (lim <= lo) return 0u;
  return (1u << (uint32_t)(lim - lo)) - 1u;
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// Inclusive prefix sum across the 64 lanes of a wave.
__device__ __forceinline__ int wave_inclusive_scan(int v) {
  const int lane = lane_id();
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    int t = __shfl_up(v, off, kWave);
    if (lane >= off) v += t;
  }
  return v;
}

// Exclusive prefix sum across a workgroup of NT threads (NT a multiple of 64,
// at most 64 waves).  `scratch` must hold NT/64 + 1 ints of LDS.  Every thread
// of the workgroup must call it; it contains two barriers and leaves the
// scratch reusable after the final barrier.
template <int NT>
__device__ __forceinline__ int block_exclusive_scan(int v, int* total, int* scratch) {
  constexpr int kWaves = NT / kWave;
  const int lane = lane_id();
  const int wave = threadIdx.x / kWave;
  const int incl = wave_inclusive_scan(v);
  if (lane == kWave - 1) scratch[wave] = incl;
  __syncthreads();
  if (wave == 0) {
    int x = lane < kWaves ? scratch[lane] : 0;
    int xi = wave_inclusive_scan(x);
    if (lane < kWaves) scratch[lane] = xi - x;
    if (lane == kWaves - 1) scratch[kWaves] = xi;
  }
  __syncthreads();
  const int result = scratch[wave] + incl - v;
  *total = scratch[kWaves];
  __syncthreads();
  return result;
}

// Append the calling lane's item to an LDS list with one atomic per wave.
// Returns the slot index for lanes with `want`, -1 otherwise.  Must be
// called by every active lane of the wave (uniform control flow).
__device__ __forceinline__ int wave_append(bool want, int* counter) {
  const uint64_t ballot = __ballot(want);
  if (ballot == 0) return -1;
  const int leader = __ffsll((long long)ballot) - 1;
  const int lane = lane_id();
  const int n = __popcll(ballot);
  int base = 0;
  if (lane == leader) base = atomicAdd(counter, n);
  base = __shfl(base, leader, kWave);
  const uint64_t below = ballot & ((lane == 0) ? 0ull : (~0ull >> (kWave - lane)));
  return want ? base + __popcll(below) : -1;
}

// Order this wave's earlier LDS writes before its later LDS reads (the lanes
// of one wave execute together; this only stops the compiler reordering).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int mask) {
  const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)v, mask, kWave);
  const uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(v >> 32), mask, kWave);
  return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ uint32_t shfl_xor_u32(uint32_t v, int mask) {
  return (uint32_t)__shfl_xor((int)v, mask, kWave);
}

// One compare-exchange step of a descending bitonic network on element e
// (value v, partner value p): block size k, distance j.
template <typename T>
__device__ __forceinline__ T bitonic_keep(T v, T p, int e, int k, int j) {
  const bool desc = (e & k) == 0;
  const bool low = (e & j) == 0;
  const bool take_max = desc == low;
  return take_max ? (v > p ? v : p) : (v < p ? v : p);
}

// Sort the 64 * EPL values held by one wave in descending order, in registers.
// Element e = i * 64 + lane lives in v[i] of that lane; distances below 64
// exchange across lanes, larger ones between the lane's own registers.
template <int EPL, typename T>
__device__ __forceinline__ void wave_sort_desc(T (&v)[EPL]) {
  const int lane = lane_id();
#pragma unroll
  for (int k = 2; k <= 64 * EPL; k <<= 1) {
#pragma unroll
    for (int j = k >> 1; j > 0; j >>= 1) {
      T nv[EPL];
#pragma unroll
      for (int i = 0; i < EPL; ++i) {
        T p;
        if (j < 64) {
          if constexpr (sizeof(T) == 8) p = shfl_xor_u64(v[i], j);
          else p = shfl_xor_u32(v[i], j);
        } else {
          p = v[i ^ (j >> 6)];
        }
        nv[i] = bitonic_keep(v[i], p, i * 64 + lane, k, j);
      }
#pragma unroll
      for (int i = 0; i < EPL; ++i) v[i] = nv[i];
    }
  }
}

}  // namespace dssel
