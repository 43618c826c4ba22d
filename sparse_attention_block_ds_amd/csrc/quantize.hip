// Quantising bf16 key rows into the 8-bit key stream (the encoding the 8-bit
// variant of the selection reads; done when a block's key is written).
//
// Page "DeepSeek V4.1F Q4 on M3 Ultra with native DSpark MTP (40tps /
// 800tps)", paragraph "DSpark": the verify rows share one stream of Q8 data.
// Here a key row of d values is stored as d/32 groups of 32 signed 8-bit codes
// with one fp16 scale each.  Per group: amax = max |x|; scale =
// fp16(amax / 127) (an fp32 division rounded to nearest, then rounded to fp16,
// nearest-even); code = clamp(round-half-away(x / scale), -127, 127) with the
// division in fp32; an all-zero group, or one whose scale rounds to 0, gets
// scale 0 and codes 0.
//
// One thread per group: four 16-byte loads of the 32 bf16 values, two 16-byte
// stores of the codes, one 2-byte store of the scale.
#include "device_util.h"
#include "dssel_internal.h"

namespace dssel {
namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
constexpr int kQuantThreads = 256;

__global__ __launch_bounds__(kQuantThreads) void quantize_kernel(QuantizeCall c) {
  const int64_t groups_per_row = c.dim / 32;
  const int64_t total = (int64_t)c.layers * c.blocks * groups_per_row;
  const int64_t t = (int64_t)blockIdx.x * kQuantThreads + threadIdx.x;
  if (t >= total) return;
  const int64_t g = t % groups_per_row;
  const int64_t row = t / groups_per_row;
  const int64_t l = row / c.blocks, b = row % c.blocks;
  const uint16_t* x = c.keys + l * c.key_layer_stride + b * c.ldk + 32 * g;
  u32x4_t v[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = *reinterpret_cast<const u32x4_t*>(x + 8 * i);
  float f[32];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      f[8 * i + 2 * e] = bf16_lo(v[i][e]);
      f[8 * i + 2 * e + 1] = bf16_hi(v[i][e]);
    }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(f[i]));
  uint16_t hs = 0;
  if (amax != 0.0f) hs = __builtin_bit_cast(uint16_t, (_Float16)__fdiv_rn(amax, 127.0f));
  const float s = half_bits_to_f32(hs);
  uint32_t packed[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    uint32_t w = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      int code = 0;
      if (s != 0.0f) {
        float r = roundf(__fdiv_rn(f[4 * i + e], s));
        r = fminf(fmaxf(r, -127.0f), 127.0f);
        code = (int)r;
      }
      w |= ((uint32_t)code & 0xFFu) << (8 * e);
    }
    packed[i] = w;
  }
  int8_t* out = c.codes + l * c.code_layer_stride + b * c.ldc + 32 * g;
  *reinterpret_cast<u32x4_t*>(out) = u32x4_t{packed[0], packed[1], packed[2], packed[3]};
  *reinterpret_cast<u32x4_t*>(out + 16) = u32x4_t{packed[4], packed[5], packed[6], packed[7]};
  c.scales[l * c.scale_layer_stride + b * c.lds + g] = hs;
}

}  // namespace

hipError_t launch_quantize(const QuantizeCall& c, hipStream_t stream) {
  const int64_t total = (int64_t)c.layers * c.blocks * (c.dim / 32);
  if (total == 0) return hipSuccess;
  const int64_t wgs = (total + kQuantThreads - 1) / kQuantThreads;
  if (wgs > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL(quantize_kernel, dim3((unsigned)wgs), dim3(kQuantThreads), 0, stream, c);
  return hipGetLastError();
}

}  // namespace dssel
