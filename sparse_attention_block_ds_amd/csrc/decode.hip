// The step between two layers of a serial decode.
//
// Page "DeepSeek V4.1F Q4 on M3 Ultra with native DSpark MTP (40tps /
// 800tps)", paragraph "Decode": decode runs the layers one after another and
// the cost to avoid is the per-dispatch overhead.  The layers are linked by
// the model, which is outside this library; its stand-in makes layer l + 1's
// query depend on layer l's selection: row r's query heads are rotated by the
// index of the row's best block,
//   q_{l+1}[r][h] = q[l+1][r][(h + s) mod H],  s = idx_l[r][0] mod H
// (s = 0 when the row selected nothing, idx = -1).  A pure data movement, so
// a serial run stays exactly reproducible.  One thread per 16-byte chunk.
#include "device_util.h"
#include "dssel_internal.h"

namespace dssel {
namespace {

constexpr int kRotateThreads = 256;

__global__ __launch_bounds__(kRotateThreads) void rotate_query_kernel(RotateCall c) {
  const int64_t chunks = (int64_t)c.rows * c.heads * (c.dim / 8);
  const int64_t x = (int64_t)blockIdx.x * kRotateThreads + threadIdx.x;
  if (x >= chunks) return;
  const int c8 = (int)(x % (c.dim / 8));
  const int64_t rh = x / (c.dim / 8);
  const int r = (int)(rh / c.heads), h = (int)(rh % c.heads);
  const int32_t best = c.idx[(int64_t)r * c.k];
  const int s = best >= 0 ? best % c.heads : 0;
  const int src = h + s < c.heads ? h + s : h + s - c.heads;
  const uint4 v = *reinterpret_cast<const uint4*>(c.q_next + ((int64_t)r * c.heads + src) * c.dim + 8 * c8);
  *reinterpret_cast<uint4*>(c.q_out + rh * c.dim + 8 * c8) = v;
}

}  // namespace

hipError_t launch_rotate(const RotateCall& c, hipStream_t stream) {
  const int64_t chunks = (int64_t)c.rows * c.heads * (c.dim / 8);
  if (chunks == 0) return hipSuccess;
  const int64_t wgs = (chunks + kRotateThreads - 1) / kRotateThreads;
  hipLaunchKernelGGL(rotate_query_kernel, dim3((unsigned)wgs), dim3(kRotateThreads), 0, stream, c);
  return hipGetLastError();
}

}  // namespace dssel
