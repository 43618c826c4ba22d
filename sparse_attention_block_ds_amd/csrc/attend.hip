// attend: attention over the selected blocks -- the step that consumes the
// selection.
//
// Page "DeepSeek V4.1F Q4 on M3 Ultra with native DSpark MTP (40tps /
// 800tps)", paragraph "Decode at depth": each layer's compressed attention
// works on the 512 blocks the selection keeps; the paragraph on prefill names
// this attention core as the kernel its gain came from.  The pages give no
// formula; the reading is ordinary scaled-dot-product attention over the
// selected blocks with the block key K[b] and a block value V[b]: per layer
// l, row r and attention head h, with c = count[l][r],
//   o[l][r][h] = sum_{j<c} softmax_j(scale * (q[l][r][h] . K[idx_j])) V[idx_j],
// accumulated in fp32, and o = 0 when no block is selected.
//
// attend_partial_kernel: one workgroup per (64-head tile, split, row, layer);
// wave w owns heads 16 w .. 16 w + 15 of the tile.  A split takes a
// contiguous range of 64-block chunks of the selection:
//  1. the chunk's K rows (row-major) and V rows (transposed, dim-major) are
//     gathered into LDS with 16-byte loads; the next chunk's loads are in
//     flight while this chunk is computed;
//  2. S = Q K^T on v_mfma_f32_16x16x32_bf16 (the wave's 16 query heads against
//     four 16-block tiles); bf16 x bf16 products are exact in fp32;
//  3. online softmax per head (running maximum and sum, the partial output
//     rescaled when the maximum grows), in base-2 units; reductions over the
//     16 lanes that hold one head use DPP;
//  4. O += P V on the matrix cores, P entering as two bf16 parts
//     (hi = bf16(p), lo = bf16(p - hi)), which carries p to about 2^-17.
// With one split the workgroup normalises and writes o; with several, each
// split writes its (maximum, sum, unnormalised o) and attend_combine_kernel
// merges the splits of a head.
//
// Slots at or past count and indices outside [0, N) are masked: their rows
// are not read and their weight is zero.
#include "device_util.h"
#include "dssel_internal.h"

namespace dssel {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kThreads = kAttendThreads;  // 4 waves
constexpr int kChunk = kAttendChunk;      // selected blocks per step
constexpr float kLog2e = 1.4426950408889634f;

template <int D>
struct AttendShared {
  static constexpr int kRowK = D + 8;       // halves per K row (16-byte pad: no bank conflicts)
  static constexpr int kRowV = kChunk + 8;  // halves per transposed V row
  static constexpr int kRowP = kChunk + 4;  // floats per weight row
  alignas(16) uint16_t k[kChunk * kRowK];
  alignas(16) uint16_t vt[D * kRowV];
  alignas(16) float p[kThreads / kWave][16 * kRowP];  // per wave: its heads' weights for the chunk
  int32_t blk[kAttendMaxK];                 // the split's block indices, -1 where masked
};

__device__ __forceinline__ float row_max16(float v) {
  v = fmaxf(v, dpp_f32<0xB1>(v));   // lane ^ 1
  v = fmaxf(v, dpp_f32<0x4E>(v));   // lane ^ 2
  v = fmaxf(v, dpp_f32<0x141>(v));  // the other quad of 8
  return fmaxf(v, dpp_f32<0x140>(v));  // the other half of 16
}

// The chunk's rows in flight: K as 16-byte row segments, V as pairs of rows
// at one 16-byte segment (so the transposed LDS writes pack two blocks).
template <int D>
struct ChunkRegs {
  static constexpr int kSegs = D / 8;
  static constexpr int kKTasks = kChunk * kSegs;             // (row, segment)
  static constexpr int kVTasks = kChunk / 2 * kSegs;         // (row pair, segment)
  static constexpr int kKPer = (kKTasks + kThreads - 1) / kThreads;
  static constexpr int kVPer = (kVTasks + kThreads - 1) / kThreads;
  u32x4_t kv[kKPer];
  u32x4_t va[kVPer], vb[kVPer];

  __device__ __forceinline__ void load(const AttendCall& c, const uint16_t* K, const uint16_t* V,
                                       const int32_t* blk, int tid) {
#pragma unroll
    for (int t = 0; t < kKPer; ++t) {
      const int u = tid + t * kThreads;
      kv[t] = u32x4_t{0u, 0u, 0u, 0u};
      if (u < kKTasks) {
        const int b = blk[u / kSegs];
        if (b >= 0) kv[t] = *reinterpret_cast<const u32x4_t*>(K + (int64_t)b * c.ldk + (u % kSegs) * 8);
      }
    }
#pragma unroll
    for (int t = 0; t < kVPer; ++t) {
      const int u = tid + t * kThreads;
      va[t] = vb[t] = u32x4_t{0u, 0u, 0u, 0u};
      if (u < kVTasks) {
        const int rp = u % (kChunk / 2), seg = u / (kChunk / 2);
        const int b0 = blk[2 * rp], b1 = blk[2 * rp + 1];
        if (b0 >= 0) va[t] = *reinterpret_cast<const u32x4_t*>(V + (int64_t)b0 * c.ldv + seg * 8);
        if (b1 >= 0) vb[t] = *reinterpret_cast<const u32x4_t*>(V + (int64_t)b1 * c.ldv + seg * 8);
      }
    }
  }

  __device__ __forceinline__ void store(AttendShared<D>& sh, int tid) const {
    using S = AttendShared<D>;
#pragma unroll
    for (int t = 0; t < kKPer; ++t) {
      const int u = tid + t * kThreads;
      if (u < kKTasks)
        *static_cast<u32x4_t*>(__builtin_assume_aligned(&sh.k[(u / kSegs) * S::kRowK + (u % kSegs) * 8], 16)) =
            kv[t];
    }
#pragma unroll
    for (int t = 0; t < kVPer; ++t) {
      const int u = tid + t * kThreads;
      if (u < kVTasks) {
        const int rp = u % (kChunk / 2), seg = u / (kChunk / 2);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          // dims seg*8 + 2e and + 1: (row 2rp, row 2rp+1) packed into one word each
          const uint32_t lo = (va[t][e] & 0xFFFFu) | (vb[t][e] << 16);
          const uint32_t hi = (va[t][e] >> 16) | (vb[t][e] & 0xFFFF0000u);
          *reinterpret_cast<uint32_t*>(&sh.vt[(seg * 8 + 2 * e) * S::kRowV + 2 * rp]) = lo;
          *reinterpret_cast<uint32_t*>(&sh.vt[(seg * 8 + 2 * e + 1) * S::kRowV + 2 * rp]) = hi;
        }
      }
    }
  }
};

template <int D>
__global__ __launch_bounds__(kThreads) void attend_partial_kernel(AttendCall c) {
  using S = AttendShared<D>;
  constexpr int KC = D / 32;  // 32-wide k chunks of the head dimension
  constexpr int NT = D / 16;  // 16-wide output tiles
  __shared__ S sh;
  const int tid = threadIdx.x, lane = lane_id(), wave = tid / kWave;
  const int tile = blockIdx.x % c.head_tiles, split = blockIdx.x / c.head_tiles;
  const int r = blockIdx.y, l = blockIdx.z;
  const int64_t lr = (int64_t)l * c.rows + r;
  const int h0 = tile * kAttendHeadTile + wave * 16;  // this wave's first head
  int m = c.count ? c.count[lr] : c.k;
  m = m < 0 ? 0 : (m > c.k ? c.k : m);
  const int j_begin = split * c.chunks_per_split * kChunk;
  int j_end = j_begin + c.chunks_per_split * kChunk;
  j_end = j_end < m ? j_end : m;
  const int nchunks = j_end > j_begin ? (j_end - j_begin + kChunk - 1) / kChunk : 0;
  const uint16_t* K = c.keys + (int64_t)l * c.key_layer_stride;
  const uint16_t* V = c.values + (int64_t)l * c.value_layer_stride;

  // the split's block indices (validated) into LDS
  {
    const int32_t* sel = c.idx + lr * c.k;
    for (int x = tid; x < nchunks * kChunk; x += kThreads) {
      const int j = j_begin + x;
      const int b = j < j_end ? sel[j] : -1;
      sh.blk[x] = (b >= 0 && (int64_t)b < c.blocks) ? b : -1;
    }
  }

  // A operand of S = Q K^T: head h0 + lane % 16, dims 32 cc + 8 (lane / 16) .. + 8
  bf16x8_t qa[KC];
  {
    const int h = h0 + (lane & 15);
#pragma unroll
    for (int cc = 0; cc < KC; ++cc) {
      u32x4_t v = {0u, 0u, 0u, 0u};
      if (h < c.heads)
        v = *reinterpret_cast<const u32x4_t*>(c.q + (lr * c.heads + h) * D + 32 * cc + 8 * (lane >> 4));
      qa[cc] = __builtin_bit_cast(bf16x8_t, v);
    }
  }

  // per head i of the lane's four (heads h0 + 4 (lane / 16) + i): running max and sum
  float mrun[4], lsum[4];
  f32x4_t o[NT];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    mrun[i] = -__builtin_inff();
    lsum[i] = 0.0f;
  }
#pragma unroll
  for (int n = 0; n < NT; ++n) o[n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const float s2 = c.scale * kLog2e;  // scores in base-2 units
  float* pw = sh.p[wave];

  __syncthreads();
  ChunkRegs<D> regs;
  if (nchunks > 0) regs.load(c, K, V, sh.blk, tid);

  for (int ch = 0; ch < nchunks; ++ch) {
    const int32_t* blk = sh.blk + ch * kChunk;
    __syncthreads();  // every wave is done with the previous chunk's LDS
    regs.store(sh, tid);
    __syncthreads();
    if (ch + 1 < nchunks) regs.load(c, K, V, blk + kChunk, tid);

    // S for the wave's 16 heads x 64 blocks (four 16-block tiles)
    f32x4_t s[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      s[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int cc = 0; cc < KC; ++cc) {
        const u32x4_t kb = *static_cast<const u32x4_t*>(__builtin_assume_aligned(
            &sh.k[(16 * t + (lane & 15)) * S::kRowK + 32 * cc + 8 * (lane >> 4)], 16));
        s[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[cc], __builtin_bit_cast(bf16x8_t, kb), s[t],
                                                       0, 0, 0);
      }
    }

    // online softmax: lane holds heads 4 (lane / 16) + i and blocks 16 t + lane % 16
    bool ok[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) ok[t] = blk[16 * t + (lane & 15)] >= 0;
    float alpha[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float cmax = -__builtin_inff();
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        s[t][i] = ok[t] ? s[t][i] * s2 : -__builtin_inff();
        cmax = fmaxf(cmax, s[t][i]);
      }
      cmax = row_max16(cmax);
      const float mnew = fmaxf(mrun[i], cmax);
      const bool none = mnew == -__builtin_inff();  // nothing admitted yet: weights stay 0
      alpha[i] = none ? 1.0f : exp2f(mrun[i] - mnew);
      float psum = 0.0f;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const float pv = none ? 0.0f : exp2f(s[t][i] - mnew);
        psum += pv;
        pw[(4 * (lane >> 4) + i) * S::kRowP + 16 * t + (lane & 15)] = pv;
      }
      lsum[i] = lsum[i] * alpha[i] + group_sum(psum, 16);
      mrun[i] = mnew;
    }
#pragma unroll
    for (int n = 0; n < NT; ++n)
#pragma unroll
      for (int i = 0; i < 4; ++i) o[n][i] *= alpha[i];
    wave_lds_sync();

    // O += P V: A = P (head lane % 16, blocks 32 kk + 8 (lane / 16) .. + 8) as hi + lo
#pragma unroll
    for (int kk = 0; kk < kChunk / 32; ++kk) {
      const float* pr = pw + (lane & 15) * S::kRowP + 32 * kk + 8 * (lane >> 4);
      const f32x4_t p0 = *static_cast<const f32x4_t*>(__builtin_assume_aligned(pr, 16));
      const f32x4_t p1 = *static_cast<const f32x4_t*>(__builtin_assume_aligned(pr + 4, 16));
      const float pe[8] = {p0[0], p0[1], p0[2], p0[3], p1[0], p1[1], p1[2], p1[3]};
      u32x4_t hi, lo;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint16_t ha = f32_to_bf16_rne(pe[2 * e]), hb = f32_to_bf16_rne(pe[2 * e + 1]);
        const uint16_t la = f32_to_bf16_rne(pe[2 * e] - bf16_to_f32(ha));
        const uint16_t lb = f32_to_bf16_rne(pe[2 * e + 1] - bf16_to_f32(hb));
        hi[e] = (uint32_t)ha | ((uint32_t)hb << 16);
        lo[e] = (uint32_t)la | ((uint32_t)lb << 16);
      }
      const bf16x8_t ahi = __builtin_bit_cast(bf16x8_t, hi), alo = __builtin_bit_cast(bf16x8_t, lo);
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        const u32x4_t vbits = *static_cast<const u32x4_t*>(__builtin_assume_aligned(
            &sh.vt[(16 * n + (lane & 15)) * S::kRowV + 32 * kk + 8 * (lane >> 4)], 16));
        const bf16x8_t bv = __builtin_bit_cast(bf16x8_t, vbits);
        o[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ahi, bv, o[n], 0, 0, 0);
        o[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(alo, bv, o[n], 0, 0, 0);
      }
    }
    wave_lds_sync();  // the weights are rewritten by the next chunk
  }

  // lane holds heads h0 + 4 (lane / 16) + i, dims 16 n + lane % 16
  if (c.splits == 1) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int h = h0 + 4 * (lane >> 4) + i;
      if (h >= c.heads) continue;
      const float inv = lsum[i] > 0.0f ? 1.0f / lsum[i] : 0.0f;
      float* oh = c.out + (lr * c.heads + h) * D;
#pragma unroll
      for (int n = 0; n < NT; ++n) oh[16 * n + (lane & 15)] = o[n][i] * inv;
    }
  } else {
    // partial record of this (layer, row, tile, split): max and sum per head, then o
    const int64_t rec = ((lr * c.head_tiles + tile) * c.splits + split) * kAttendHeadTile;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int hl = wave * 16 + 4 * (lane >> 4) + i;  // head within the tile
      if ((lane & 15) == 0) {
        c.part_ml[2 * (rec + hl)] = mrun[i];
        c.part_ml[2 * (rec + hl) + 1] = lsum[i];
      }
      float* oh = c.part_o + (rec + hl) * D;
#pragma unroll
      for (int n = 0; n < NT; ++n) oh[16 * n + (lane & 15)] = o[n][i];
    }
  }
}

// Merge the splits of each head: with M = max_s m_s,
//   o = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s,
// summed in ascending split order.  64 threads per head (dims t, t + 64, ...),
// four heads per workgroup; the split records are read in batches whose loads
// do not wait on each other.
constexpr int kCombineHeads = kThreads / kWave;  // heads per combine workgroup

template <int D>
__global__ __launch_bounds__(kThreads) void attend_combine_kernel(AttendCall c) {
  constexpr int kPer = (D + kWave - 1) / kWave;  // dims per thread
  constexpr int kB = 4;                          // split records per batch
  const int tile = blockIdx.x / (kAttendHeadTile / kCombineHeads);
  const int hl = (blockIdx.x % (kAttendHeadTile / kCombineHeads)) * kCombineHeads + threadIdx.x / kWave;
  const int h = tile * kAttendHeadTile + hl;
  if (h >= c.heads) return;  // a whole wave (no barriers below)
  const int t = threadIdx.x % kWave;
  const int r = blockIdx.y, l = blockIdx.z;
  const int64_t lr = (int64_t)l * c.rows + r;
  const int64_t rec0 = (lr * c.head_tiles + tile) * c.splits * kAttendHeadTile + hl;  // split s: + s * 64
  float mx = -__builtin_inff();
  for (int s0 = 0; s0 < c.splits; s0 += kB) {
    float mv[kB];
#pragma unroll
    for (int b = 0; b < kB; ++b)
      mv[b] = s0 + b < c.splits ? c.part_ml[2 * (rec0 + (int64_t)(s0 + b) * kAttendHeadTile)] : -__builtin_inff();
#pragma unroll
    for (int b = 0; b < kB; ++b) mx = fmaxf(mx, mv[b]);
  }
  float z = 0.0f, acc[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) acc[i] = 0.0f;
  if (mx != -__builtin_inff()) {
    for (int s0 = 0; s0 < c.splits; s0 += kB) {
      float ms[kB], ls[kB], ov[kB][kPer];
#pragma unroll
      for (int b = 0; b < kB; ++b) {
        const bool ok = s0 + b < c.splits;
        const int64_t rec = rec0 + (int64_t)(s0 + b) * kAttendHeadTile;
        ms[b] = ok ? c.part_ml[2 * rec] : -__builtin_inff();
        ls[b] = ok ? c.part_ml[2 * rec + 1] : 0.0f;
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
          const int dim = t + kWave * i;
          ov[b][i] = (ok && dim < D) ? c.part_o[rec * D + dim] : 0.0f;
        }
      }
#pragma unroll
      for (int b = 0; b < kB; ++b) {
        if (ms[b] == -__builtin_inff()) continue;
        const float f = exp2f(ms[b] - mx);
        z += f * ls[b];
#pragma unroll
        for (int i = 0; i < kPer; ++i) acc[i] += f * ov[b][i];
      }
    }
  }
  float* oh = c.out + (lr * c.heads + h) * D;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int dim = t + kWave * i;
    if (dim < D) oh[dim] = z > 0.0f ? acc[i] / z : 0.0f;
  }
}

template <int D>
hipError_t launch_attend_d(const AttendCall& c, hipStream_t stream) {
  const dim3 grid(c.head_tiles * c.splits, c.rows, c.layers);
  hipLaunchKernelGGL(attend_partial_kernel<D>, grid, dim3(kThreads), 0, stream, c);
  if (c.splits > 1) {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(attend_combine_kernel<D>,
                       dim3(c.head_tiles * (kAttendHeadTile / kCombineHeads), c.rows, c.layers), dim3(kThreads),
                       0, stream, c);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attend(const AttendCall& c, hipStream_t stream) {
  switch (c.dim) {
    case 32: return launch_attend_d<32>(c, stream);
    case 64: return launch_attend_d<64>(c, stream);
    case 128: return launch_attend_d<128>(c, stream);
    case 256: return launch_attend_d<256>(c, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace dssel
