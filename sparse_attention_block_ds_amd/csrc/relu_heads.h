// The per-head ReLU score on the matrix cores, shared by the sampled floors
// (prep) and the key stream (score).
//
// score(b) = sum_h w_h max(q_h . K_b, 0): the heads cannot be folded into one
// query vector, so every (row, head) pair meets every key.  Per 16 blocks and
// row r, v_mfma_f32_16x16x32_bf16 takes 16 heads as the A rows (head
// 16 t + lane % 16, staged in LDS) against the 16 blocks' keys as the B
// columns (block lane % 16, held in registers), d / 32 MFMAs per head tile.
// Lane l then holds the dot products of heads 16 t + 4 (l / 16) + i (i < 4)
// with its block; it clamps each at zero, weights it and adds the four into
// its partial sum, over every head tile; two cross-lane adds (lanes l ^ 16,
// l ^ 32) leave the full sum in all four lanes of the block.
#pragma once

#include "device_util.h"
#include "dssel_internal.h"

namespace dssel {

typedef __bf16 relu_bf16x8_t __attribute__((ext_vector_type(8)));
typedef float relu_f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t relu_u32x4_t __attribute__((ext_vector_type(4)));

struct ReluStage {
  const uint16_t* q;  // [R][Hp][D + 8]
  const float* w;     // [R][Hp]
  int hp;             // heads rounded up to 16
};

template <int D>
__device__ __forceinline__ int relu_w_offset_words(int rows, int hp) {
  return (rows * hp * (D + 8) * 2 + 15) / 16 * 4;  // 16-byte aligned, in 32-bit words
}

// Cooperative copy of the query heads and weights of R consecutive rows, from
// (layer, row) index lr0 on, into the stage (all threads of the workgroup call
// it; the caller synchronises afterwards).
template <int R, int D>
__device__ __forceinline__ ReluStage relu_stage_heads(const Call& c, int64_t lr0, uint32_t* lds, int tid,
                                                      int nthreads) {
  const int H = c.heads, hp = (H + 15) / 16 * 16;
  constexpr int QS = D + 8;
  uint16_t* qs = reinterpret_cast<uint16_t*>(lds);
  float* ws = reinterpret_cast<float*>(lds + relu_w_offset_words<D>(R, hp));
  const int chunks = R * hp * (D / 8);
  for (int x = tid; x < chunks; x += nthreads) {
    const int c8 = x % (D / 8), rh = x / (D / 8);
    const int r = rh / hp, h = rh % hp;
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (h < H) v = *reinterpret_cast<const uint4*>(c.q + ((lr0 + r) * H + h) * D + 8 * c8);
    *reinterpret_cast<uint4*>(qs + (int64_t)rh * QS + 8 * c8) = v;
  }
  for (int x = tid; x < R * hp; x += nthreads) {
    const int r = x / hp, h = x % hp;
    ws[x] = h < H ? bf16_to_f32(c.w[(lr0 + r) * H + h]) : 0.0f;
  }
  return ReluStage{qs, ws, hp};
}

template <int D>
__device__ __forceinline__ ReluStage relu_stage_view(const Call& c, const uint32_t* lds, int rows) {
  const int hp = (c.heads + 15) / 16 * 16;
  return ReluStage{reinterpret_cast<const uint16_t*>(lds),
                   reinterpret_cast<const float*>(lds + relu_w_offset_words<D>(rows, hp)), hp};
}

// Row r's per-head ReLU score of NG groups of 16 blocks (B operands kb[g]),
// summed over every head and complete in every lane of each block.
template <int D, int NG>
__device__ __forceinline__ void relu_row_scores(const ReluStage& st, int r,
                                                const relu_u32x4_t (&kb)[NG][D / 32], float (&out)[NG]) {
  constexpr int KC = D / 32, QS = D + 8;
  const int lane = lane_id();
  const int m = lane & 15, g = lane >> 4;
  float part[NG];
#pragma unroll
  for (int n = 0; n < NG; ++n) part[n] = 0.0f;
  const uint16_t* qrow = st.q + ((int64_t)r * st.hp + m) * QS + 8 * g;
  const float* wrow = st.w + r * st.hp + 4 * g;
  for (int t = 0; t < st.hp; t += 16) {
    relu_f32x4_t acc[NG];
#pragma unroll
    for (int n = 0; n < NG; ++n) acc[n] = relu_f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int cc = 0; cc < KC; ++cc) {
      const relu_u32x4_t a = *reinterpret_cast<const relu_u32x4_t*>(qrow + (int64_t)t * QS + 32 * cc);
#pragma unroll
      for (int n = 0; n < NG; ++n)
        acc[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(relu_bf16x8_t, a),
                                                         __builtin_bit_cast(relu_bf16x8_t, kb[n][cc]),
                                                         acc[n], 0, 0, 0);
    }
    const float4 w4 = *reinterpret_cast<const float4*>(wrow + t);
#pragma unroll
    for (int n = 0; n < NG; ++n) {
      part[n] += w4.x * fmaxf(acc[n][0], 0.0f);
      part[n] += w4.y * fmaxf(acc[n][1], 0.0f);
      part[n] += w4.z * fmaxf(acc[n][2], 0.0f);
      part[n] += w4.w * fmaxf(acc[n][3], 0.0f);
    }
  }
#pragma unroll
  for (int n = 0; n < NG; ++n) {
    float v = part[n];
    v += __shfl_xor(v, 16, kWave);
    v += __shfl_xor(v, 32, kWave);
    out[n] = v;
  }
}

// Every row's score of NG groups of 16 blocks at once: head tiles outside,
// rows inside, so that each tile issues R x NG independent MFMA chains.  The
// A fragments (R x d/32 LDS reads) of tile t + 16 are read while tile t's
// MFMAs run, and tile t's clamp and weighting run after both are issued, so
// neither the LDS latency nor the MFMA latency is waited out per instruction.
template <int R, int D>
__device__ __forceinline__ void relu_read_tile(const uint16_t* qbase, int hp, int t,
                                               relu_u32x4_t (&a)[R][D / 32]) {
  constexpr int KC = D / 32, QS = D + 8;
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int cc = 0; cc < KC; ++cc)
      a[r][cc] = *reinterpret_cast<const relu_u32x4_t*>(qbase + ((int64_t)r * hp + t) * QS + 32 * cc);
}

__device__ __forceinline__ float relu_clamp(float x) {
  return __builtin_amdgcn_fmed3f(x, 0.0f, __builtin_huge_valf());  // max(x, 0) for finite x
}

// PIPE = false: the fragments are read inside the tile (no prefetch registers),
// for kernels held to 128 registers whose other waves hide the latency.
template <int R, int D, int NG, bool PIPE = true>
__device__ __forceinline__ void relu_all_rows(const ReluStage& st, const relu_u32x4_t (&kb)[NG][D / 32],
                                              float (&out)[R][NG]) {
  constexpr int KC = D / 32, QS = D + 8;
  const int lane = lane_id();
  const int m = lane & 15, g = lane >> 4;
  float part[R][NG];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int n = 0; n < NG; ++n) part[r][n] = 0.0f;
  const uint16_t* qbase = st.q + (int64_t)m * QS + 8 * g;
  const float* wbase = st.w + 4 * g;
  relu_u32x4_t a[PIPE ? R : 1][KC];
  if constexpr (PIPE) relu_read_tile<R, D>(qbase, st.hp, 0, a);
  for (int t = 0; t < st.hp; t += 16) {
    relu_f32x4_t acc[R][NG];
    if constexpr (!PIPE) {
#pragma unroll
      for (int r = 0; r < R; ++r) {
#pragma unroll
        for (int cc = 0; cc < KC; ++cc) {
          const relu_u32x4_t x =
              *reinterpret_cast<const relu_u32x4_t*>(qbase + ((int64_t)r * st.hp + t) * QS + 32 * cc);
#pragma unroll
          for (int n = 0; n < NG; ++n)
            acc[r][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                __builtin_bit_cast(relu_bf16x8_t, x), __builtin_bit_cast(relu_bf16x8_t, kb[n][cc]),
                cc == 0 ? relu_f32x4_t{0.f, 0.f, 0.f, 0.f} : acc[r][n], 0, 0, 0);
        }
      }
    } else {
#pragma unroll
      for (int cc = 0; cc < KC; ++cc)
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
          for (int n = 0; n < NG; ++n)
            acc[r][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                __builtin_bit_cast(relu_bf16x8_t, a[PIPE ? r : 0][cc]),
                __builtin_bit_cast(relu_bf16x8_t, kb[n][cc]),
                cc == 0 ? relu_f32x4_t{0.f, 0.f, 0.f, 0.f} : acc[r][n], 0, 0, 0);
    }
    float4 w4[R];
#pragma unroll
    for (int r = 0; r < R; ++r) w4[r] = *reinterpret_cast<const float4*>(wbase + r * st.hp + t);
    if constexpr (PIPE) {
      if (t + 16 < st.hp) relu_read_tile<R, D>(qbase, st.hp, t + 16, a);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int n = 0; n < NG; ++n) {
        part[r][n] += w4[r].x * relu_clamp(acc[r][n][0]);
        part[r][n] += w4[r].y * relu_clamp(acc[r][n][1]);
        part[r][n] += w4[r].z * relu_clamp(acc[r][n][2]);
        part[r][n] += w4[r].w * relu_clamp(acc[r][n][3]);
      }
  }
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int n = 0; n < NG; ++n) {
      float v = part[r][n];
      v += __shfl_xor(v, 16, kWave);
      v += __shfl_xor(v, 32, kWave);
      out[r][n] = v;
    }
}

}  // namespace dssel
