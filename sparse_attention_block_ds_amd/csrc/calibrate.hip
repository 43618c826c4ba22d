// Calibration kernels: the floors and ceilings the selection chain is measured
// against -- an empty launch, a plain read of every key row, and a gather of
// exactly the admitted key rows with the addressing the key stream uses.  They
// compute nothing of the method; each XOR-folds what it reads into one word
// per workgroup so that no load can be dropped.
#include "device_util.h"
#include "dssel_internal.h"

namespace dssel {
namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kCalThreads = 256;
constexpr int kCalWaves = kCalThreads / kWave;
constexpr int kCalUnroll = 8;  // independent 16-byte loads in flight per thread

__global__ __launch_bounds__(kCalThreads) void calib_empty_kernel() {}

__device__ __forceinline__ uint32_t fold4(u32x4_t v) { return v[0] ^ v[1] ^ v[2] ^ v[3]; }

// Every key row of every layer as one contiguous array (the host checks that
// the rows are packed): workgroup g reads 16-byte pieces [g P / G, (g+1) P / G)
// of the P pieces, eight loads in flight per thread.
__global__ __launch_bounds__(kCalThreads) void calib_read_kernel(CalibCall c) {
  const int64_t total = (int64_t)c.layers * c.blocks * (c.dim / 8);
  const int64_t p0 = total * blockIdx.x / gridDim.x, p1 = total * (blockIdx.x + 1) / gridDim.x;
  const u32x4_t* src = reinterpret_cast<const u32x4_t*>(c.keys);
  uint32_t acc = 0;
  for (int64_t i0 = p0 + threadIdx.x; i0 < p1; i0 += kCalUnroll * kCalThreads) {
    u32x4_t v[kCalUnroll];
#pragma unroll
    for (int u = 0; u < kCalUnroll; ++u) {
      const int64_t i = i0 + (int64_t)u * kCalThreads;
      v[u] = i < p1 ? src[i] : u32x4_t{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < kCalUnroll; ++u) acc ^= fold4(v[u]);
  }
  for (int off = 32; off > 0; off >>= 1) acc ^= __shfl_xor(acc, off, kWave);
  if (lane_id() == 0) atomicXor(&c.sink[blockIdx.x], acc);
}

// The admitted key rows only, with the key stream's addressing: workgroup g
// streams the flattened (layer, block) range [ranges[g], ranges[g + 1]) (the
// host balances the ranges by admitted count) 2048 blocks at a time.  Wave 0
// lists the tile's admitted blocks in LDS (a prefix sum of its mask words'
// popcounts places every set bit), then each wave takes groups of 16 listed
// rows, lane i loading 16 bytes of row i % 16 at column 8 (i / 16) + 32 c,
// two groups ahead of their use.
template <int D>
__global__ __launch_bounds__(kCalThreads) void calib_gather_kernel(CalibCall c) {
  constexpr int KC = D / 32;
  __shared__ int32_t list[kTileBlocks];
  __shared__ int ntile;
  const int lane = lane_id(), wave = threadIdx.x / kWave;
  const int64_t g0 = c.ranges[blockIdx.x], g1 = c.ranges[blockIdx.x + 1];
  uint32_t acc = 0;
  for (int64_t t0 = g0; t0 < g1;) {
    const int64_t l = t0 / c.blocks;
    const int64_t b0 = t0 % c.blocks;
    int64_t b1 = b0 + kTileBlocks;
    b1 = b1 < c.blocks ? b1 : c.blocks;
    b1 = b1 < b0 + (g1 - t0) ? b1 : b0 + (g1 - t0);
    if (wave == 0) {
      const int64_t b = b0 + 32 * lane;  // b0 is a multiple of 32 (the host aligns the ranges)
      uint32_t word = 0;
      if (b < b1) {
        word = c.mask ? c.mask[l * c.mask_layer_stride + (b >> 5)] : 0xFFFFFFFFu;
        const int64_t hi = b1 - b;  // keep the bits of blocks below b1
        if (hi < 32) word &= (1u << hi) - 1u;
      }
      const int cnt = __popc(word);
      const int before = wave_inclusive_scan(cnt) - cnt;
      for (int s = 0; s < 32; ++s) {
        const int bit = (s + lane) & 31;
        if ((word >> bit) & 1u) list[before + __popc(word & ((1u << bit) - 1u))] = (int32_t)(b + bit);
      }
      if (lane == kWave - 1) ntile = before + cnt;
    }
    __syncthreads();
    const int n = ntile;
    const uint16_t* K = c.keys + l * c.key_layer_stride;
    auto load = [&](u32x4_t (&buf)[KC], int g) {
      const int e = g + (lane & 15);
#pragma unroll
      for (int cc = 0; cc < KC; ++cc) buf[cc] = u32x4_t{0u, 0u, 0u, 0u};
      if (e < n) {
        const uint16_t* row = K + (int64_t)list[e] * c.ldk + 8 * (lane >> 4);
#pragma unroll
        for (int cc = 0; cc < KC; ++cc) buf[cc] = *reinterpret_cast<const u32x4_t*>(row + 32 * cc);
      }
    };
    auto fold = [&](const u32x4_t (&buf)[KC]) {
#pragma unroll
      for (int cc = 0; cc < KC; ++cc) acc ^= fold4(buf[cc]);
    };
    constexpr int step = kCalWaves * 16;
    u32x4_t r0[KC], r1[KC], r2[KC];
    int g = wave * 16;
    load(r0, g);
    load(r1, g + step);
    for (; g < n; g += 3 * step) {
      load(r2, g + 2 * step);
      fold(r0);
      load(r0, g + 3 * step);
      fold(r1);
      load(r1, g + 4 * step);
      fold(r2);
    }
    __syncthreads();
    t0 += b1 - b0;
  }
  for (int off = 32; off > 0; off >>= 1) acc ^= __shfl_xor(acc, off, kWave);
  if (lane == 0) atomicXor(&c.sink[blockIdx.x], acc);
}

}  // namespace

hipError_t launch_calibrate(const CalibCall& c, hipStream_t stream) {
  dim3 grid((unsigned)c.workgroups);
  switch (c.kind) {
    case kCalibEmpty: hipLaunchKernelGGL(calib_empty_kernel, grid, dim3(kCalThreads), 0, stream); break;
    case kCalibRead: hipLaunchKernelGGL(calib_read_kernel, grid, dim3(kCalThreads), 0, stream, c); break;
    case kCalibGather:
      switch (c.dim) {
        case 32: hipLaunchKernelGGL(calib_gather_kernel<32>, grid, dim3(kCalThreads), 0, stream, c); break;
        case 64: hipLaunchKernelGGL(calib_gather_kernel<64>, grid, dim3(kCalThreads), 0, stream, c); break;
        case 128: hipLaunchKernelGGL(calib_gather_kernel<128>, grid, dim3(kCalThreads), 0, stream, c); break;
        case 256: hipLaunchKernelGGL(calib_gather_kernel<256>, grid, dim3(kCalThreads), 0, stream, c); break;
        default: return hipErrorInvalidValue;
      }
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace dssel
