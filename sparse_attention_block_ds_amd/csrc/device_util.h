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

// 8-bit keys: eight signed codes (two 32-bit words) as eight bf16 values,
// exactly (|code| <= 128 has at most 8 significant bits): each code widens to
// fp32 and keeps its top 16 bits.
__device__ __forceinline__ uint32_t bf16_pair_of_codes(uint32_t w, int shift) {
  const float a = (float)(int8_t)(w >> shift);
  const float b = (float)(int8_t)(w >> (shift + 8));
  return (__float_as_uint(a) >> 16) | (__float_as_uint(b) & 0xFFFF0000u);
}

// fp16 bits widened to fp32 (exact).
__device__ __forceinline__ float half_bits_to_f32(uint16_t h) {
  return (float)__builtin_bit_cast(_Float16, h);
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

// Sum of v over aligned groups of `width` lanes (4, 8, 16 or 32), left in
// every lane of the group.  Within a row of 16 lanes the exchanges are DPP
// moves on the vector ALU (swap neighbours, swap pairs, mirror the half row,
// mirror the row); only the step across rows goes through the LDS crossbar.
template <int kCtrl>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kCtrl, 0xF, 0xF, false));
}

__device__ __forceinline__ float group_sum(float v, int width) {
  v += dpp_f32<0xB1>(v);                 // quad_perm [1, 0, 3, 2]: lane ^ 1
  v += dpp_f32<0x4E>(v);                 // quad_perm [2, 3, 0, 1]: lane ^ 2
  if (width >= 8) v += dpp_f32<0x141>(v);   // row_half_mirror: the other quad of 8
  if (width >= 16) v += dpp_f32<0x140>(v);  // row_mirror: the other half of 16
  if (width >= 32) v += __shfl_xor(v, 16, kWave);
  return v;
}

// Order this wave's earlier LDS writes before its later LDS reads (the lanes
// of one wave execute together; this only stops the compiler reordering).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

}  // namespace dssel
