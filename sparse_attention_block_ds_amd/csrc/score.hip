// score: the compacted admitted index and one pass over the admitted block
// keys shared by all query rows of a layer, writing the rows' order-preserving
// radix keys at the compacted positions and counting their first radix digit.
//
// Page "DeepSeek V4.1F Q4 on M3 Ultra with native DSpark MTP (40tps /
// 800tps)": paragraph "Decode at depth" -- only admitted blocks are scored,
// and the admitted index is compacted once per row; paragraph "DSpark" -- the
// rows of a speculative verify share one stream of data, here the key stream:
// each admitted K row is read from HBM once and dotted with every row's query.
//
// Work split: workgroup (l, j) takes positions [j * piece, (j + 1) * piece) of
// layer l's compacted admitted index, so the workgroups stream equal numbers of
// key rows whatever the masks look like (`piece` is chosen on the host so that
// a full-size call fills the chip with one round of resident workgroups, and a
// single layer still spreads over hundreds of them); workgroups past a layer's
// admitted positions exit at once.  A workgroup:
//  1. Set-up, one round of independent loads: the layer's counts and limits,
//     the piece's slice of the compacted index (built by prep) into LDS, and
//     the folded query.
//  2. Key stream: each wave takes 16 consecutive compacted entries at a time
//     and loads their K rows with 16-byte loads (each instruction reads 16 rows
//     x 64 contiguous bytes), two steps ahead of the arithmetic.
//       MFMA engine: v_mfma_f32_16x16x32_bf16 with the fp32 q~ entering as
//       three exact bf16 parts (hi + mid + lo == q~) along the M dimension
//       (row m = 4 * (query row % 4) + part), so the bf16 keys feed the
//       matrix cores directly: no vector-ALU conversion, no cross-lane sum.
//       VALU engine: d/8 lanes per key row, 8 fp32 FMAs per lane and row, a
//       butterfly across the row's lanes.
//  3. Epilogue per (row, entry): radix key -> keys[l][r][pos]; the first digit
//     is counted in an LDS histogram (two 16-bit counters per word), added to
//     the layer's global histogram at the end.
#include "device_util.h"
#include "dssel_internal.h"

namespace dssel {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kGroup = 16;                     // compacted entries per wave step
constexpr int kWaves = kScoreThreads / kWave;  // 4
constexpr int kPiece = kScorePieceMax;         // largest piece one workgroup compacts and streams

__device__ __forceinline__ u32x4_t load16(const uint16_t* p) {
  return *reinterpret_cast<const u32x4_t*>(p);
}

template <int R>
struct PieceCtx {
  int64_t key_row;
  int off, cnt;                // positions [off, off + cnt) of the current layer
  int mode;
  const int32_t* sh_list;      // block index of each entry of the piece
  const int* sh_P;             // positions [0, P[r]) hold row r's keys
  const int64_t* sh_lim;       // clamped causal limits of the layer's rows
  uint32_t* sh_hist;           // [R][kHistBins / 2], two 16-bit counters per word
  uint32_t* skeys_l;           // keys of this layer: [R][key_row]
  const uint32_t* mask_l;      // the layer's mask rows (kRowMask)
  int64_t mask_row_stride;

  // Finish one (row, entry): key to HBM, first digit to the LDS histogram.
  __device__ __forceinline__ void emit(int r, int e, float s) const {
    const int pos = off + e;
    if (pos >= sh_P[r]) return;
    bool admitted = true;
    if (mode == kRowMask) {  // the union list also holds blocks other rows admit
      const int b = sh_list[e];
      const uint32_t word = mask_l[r * mask_row_stride + (b >> 5)];
      admitted = ((word >> (b & 31)) & 1u) && (int64_t)b < sh_lim[r];
    }
    const uint32_t key = admitted ? score_to_key(s) : 0u;
    skeys_l[(int64_t)r * key_row + pos] = key;
    if (admitted)
      atomicAdd(&sh_hist[r * (kHistBins / 2) + (key >> (kDigit1Shift + 1))],
                1u << (16u * ((key >> kDigit1Shift) & 1u)));
  }

  __device__ __forceinline__ int block_of(int e) const {
    return mode == kNoMask ? off + e : sh_list[e];
  }
};

// ---------------------------------------------------------------- MFMA engine
// The three bf16 parts of q~ share one MFMA: output row m = 4*(r % 4) + p
// holds part p (0 hi, 1 mid, 2 lo; 3 unused) of query row r, so rows 0-3 go
// through one MFMA per 32 key columns and rows 4-7 through a second one, and
// lane l ends up owning the three part-sums of row 4*s + l/16 for block l%16.
template <int R, int D, int NBUF>
struct MfmaEngine {
  static constexpr int kRows = R, kBuffers = NBUF;
  static constexpr int KC = D / 32;       // 32-column chunks of a key row
  static constexpr int S = (R + 3) / 4;   // MFMA row sets
  bf16x8_t a[S][KC];                      // A operand: q~ parts (row m = lane % 16)
  u32x4_t buf[NBUF][KC];                  // B operand: K rows (block = lane % 16)

  __device__ void init(const Call& c, int l) {
    const int lane = lane_id();
    const int m = lane & 15, g = lane >> 4;
    const int p = m & 3;
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const int r = 4 * s + (m >> 2);
#pragma unroll
      for (int cc = 0; cc < KC; ++cc) {
        u32x4_t v = {0u, 0u, 0u, 0u};
        if (p < 3 && r < R)
          v = load16(c.qparts + (((int64_t)l * 3 + p) * R + r) * D + 32 * cc + 8 * g);
        a[s][cc] = __builtin_bit_cast(bf16x8_t, v);
      }
    }
  }

  template <int B>
  __device__ __forceinline__ void load(const PieceCtx<R>& t, const uint16_t* K, int64_t ldk, int g0) {
    const int lane = lane_id();
    const int e = g0 + (lane & 15);
    if (e < t.cnt) {
      const uint16_t* row = K + (int64_t)t.block_of(e) * ldk + 8 * (lane >> 4);
#pragma unroll
      for (int cc = 0; cc < KC; ++cc) buf[B][cc] = load16(row + 32 * cc);
    } else {
#pragma unroll
      for (int cc = 0; cc < KC; ++cc) buf[B][cc] = u32x4_t{0u, 0u, 0u, 0u};
    }
  }

  template <int B>
  __device__ __forceinline__ void compute_emit(const PieceCtx<R>& t, int g0) {
    f32x4_t acc[S];
#pragma unroll
    for (int s = 0; s < S; ++s) {
      acc[s] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int cc = 0; cc < KC; ++cc)
        acc[s] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            a[s][cc], __builtin_bit_cast(bf16x8_t, buf[B][cc]), acc[s], 0, 0, 0);
    }
    const int lane = lane_id();
    const int e = g0 + (lane & 15);
    if (e >= t.cnt) return;
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const int r = 4 * s + (lane >> 4);
      if (r < R) t.emit(r, e, (acc[s][0] + acc[s][1]) + acc[s][2]);
    }
  }
};

// ---------------------------------------------------------------- VALU engine
template <int R, int D, int NBUF>
struct ValuEngine {
  static constexpr int kRows = R, kBuffers = NBUF;
  static constexpr int LPR = D / 8;        // lanes per key row
  static constexpr int RPI = kWave / LPR;  // key rows per load instruction
  static constexpr int U = kGroup / RPI;   // load instructions per group
  float qv[R][8];
  u32x4_t buf[NBUF][U];

  __device__ void init(const Call& c, int l) {
    const int slice = lane_id() % LPR;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const float* qt = c.qt + ((int64_t)l * R + r) * D + slice * 8;
#pragma unroll
      for (int e = 0; e < 8; ++e) qv[r][e] = qt[e];
    }
  }

  template <int B>
  __device__ __forceinline__ void load(const PieceCtx<R>& t, const uint16_t* K, int64_t ldk, int g0) {
    const int lane = lane_id();
    const int slice = lane % LPR, rr = lane / LPR;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int e = g0 + u * RPI + rr;
      buf[B][u] = u32x4_t{0u, 0u, 0u, 0u};
      if (e < t.cnt) buf[B][u] = load16(K + (int64_t)t.block_of(e) * ldk + slice * 8);
    }
  }

  template <int B>
  __device__ __forceinline__ void compute_emit(const PieceCtx<R>& t, int g0) {
    const int lane = lane_id();
    const int slice = lane % LPR, rr = lane / LPR;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t kw[4] = {buf[B][u][0], buf[B][u][1], buf[B][u][2], buf[B][u][3]};
      float acc[R];
#pragma unroll
      for (int r = 0; r < R; ++r) acc[r] = 0.0f;
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) {
        const float x0 = bf16_lo(kw[e2]), x1 = bf16_hi(kw[e2]);
#pragma unroll
        for (int r = 0; r < R; ++r) {
          acc[r] = fmaf(qv[r][2 * e2], x0, acc[r]);
          acc[r] = fmaf(qv[r][2 * e2 + 1], x1, acc[r]);
        }
      }
#pragma unroll
      for (int m = 1; m < LPR; m <<= 1)
#pragma unroll
        for (int r = 0; r < R; ++r) acc[r] += __shfl_xor(acc[r], m, kWave);
      const int e = g0 + u * RPI + rr;
      if (e < t.cnt) {
#pragma unroll
        for (int r = 0; r < R; ++r)
          if (r % LPR == slice) t.emit(r, e, acc[r]);
      }
    }
  }
};

// Runs the wave's groups g0, g0 + step, ... < cnt through a ring of NBUF load
// buffers: the loads for group j + NBUF - 1 are issued before group j is
// computed, so NBUF - 1 groups of key rows are in flight behind the arithmetic.
template <int NBUF, class Engine, int J>
__device__ __forceinline__ void ring_step(Engine& eng, const PieceCtx<Engine::kRows>& pc,
                                          const uint16_t* K, int64_t ldk, int g, int step) {
  if constexpr (J < NBUF) {
    const int gj = g + J * step;
    if (gj >= pc.cnt) return;
    const int gl = gj + (NBUF - 1) * step;
    if (gl < pc.cnt) eng.template load<(J + NBUF - 1) % NBUF>(pc, K, ldk, gl);
    eng.template compute_emit<J>(pc, gj);
    ring_step<NBUF, Engine, J + 1>(eng, pc, K, ldk, g, step);
  }
}

template <int NBUF, class Engine, int J>
__device__ __forceinline__ void ring_prologue(Engine& eng, const PieceCtx<Engine::kRows>& pc,
                                              const uint16_t* K, int64_t ldk, int g0, int step) {
  if constexpr (J < NBUF - 1) {
    const int gj = g0 + J * step;
    if (gj < pc.cnt) eng.template load<J>(pc, K, ldk, gj);
    ring_prologue<NBUF, Engine, J + 1>(eng, pc, K, ldk, g0, step);
  }
}

template <int NBUF, class Engine>
__device__ __forceinline__ void stream_piece(Engine& eng, const PieceCtx<Engine::kRows>& pc,
                                             const uint16_t* K, int64_t ldk, int g0, int step) {
  ring_prologue<NBUF, Engine, 0>(eng, pc, K, ldk, g0, step);
  for (int g = g0; g < pc.cnt; g += NBUF * step) ring_step<NBUF, Engine, 0>(eng, pc, K, ldk, g, step);
}

// Everything a workgroup keeps in LDS.
template <int R>
struct ScoreShared {
  int32_t list[kPiece];
  uint32_t hist[R * (kHistBins / 2)];
  int P[kMaxRows];
  int64_t lim[kMaxRows];
};

template <int R>
__device__ void flush_hist(ScoreShared<R>& sh, uint32_t* gh) {
  __syncthreads();
  for (int i = threadIdx.x; i < R * (kHistBins / 2); i += kScoreThreads) {
    const uint32_t v = sh.hist[i];
    if (v & 0xFFFFu) atomicAdd(&gh[2 * i], v & 0xFFFFu);
    if (v >> 16) atomicAdd(&gh[2 * i + 1], v >> 16);
    sh.hist[i] = 0u;
  }
  __syncthreads();
}

template <int R, int D, class Engine>
__device__ __forceinline__ void score_body(const Call& c) {
  __shared__ ScoreShared<R> sh;
  const int tid = threadIdx.x;
  const int64_t N = c.blocks;
  const int PS = c.piece;
  const int pieces_per_layer = (int)((N + PS - 1) / PS);
  const int sl = blockIdx.x / pieces_per_layer;
  const int s0 = (blockIdx.x % pieces_per_layer) * PS;

  // Set-up: one round of independent loads -- the layer's counts and limits,
  // this piece's slice of the compacted index, and (in the engine) q~.
  const int32_t* counts = c.counts + (int64_t)sl * kCountStride;
  const int nl = counts[kMaxRows];
  if (s0 >= nl) return;  // past the layer's admitted positions: uniform for the workgroup
  const int s1 = s0 + PS < nl ? s0 + PS : nl;
  if (c.mode != kNoMask) {
    const int32_t* list = c.list + (int64_t)sl * N + s0;
    for (int i = tid; i < s1 - s0; i += kScoreThreads) sh.list[i] = list[i];
  }
  for (int i = tid; i < R * (kHistBins / 2); i += kScoreThreads) sh.hist[i] = 0u;
  if (tid < kMaxRows) sh.P[tid] = tid < R ? (c.mode == kRowMask ? nl : counts[tid]) : 0;
  if (tid < R) {
    const int64_t v = c.limit ? (int64_t)c.limit[(int64_t)sl * R + tid] : N;
    sh.lim[tid] = v < 0 ? 0 : (v > N ? N : v);
  }
  Engine eng;
  eng.init(c, sl);
  __syncthreads();

  // The key stream over positions [s0, s1).
  PieceCtx<R> pc;
  pc.key_row = c.key_row;
  pc.off = s0;
  pc.cnt = s1 - s0;
  pc.mode = c.mode;
  pc.sh_list = sh.list;
  pc.sh_P = sh.P;
  pc.sh_lim = sh.lim;
  pc.sh_hist = sh.hist;
  pc.skeys_l = c.skeys + (int64_t)sl * R * c.key_row;
  pc.mask_l = c.mask ? c.mask + (int64_t)sl * c.mask_layer_stride : nullptr;
  pc.mask_row_stride = c.mask_row_stride;
  stream_piece<Engine::kBuffers>(eng, pc, c.keys + (int64_t)sl * c.key_layer_stride, c.ldk,
                                 (tid / kWave) * kGroup, kWaves * kGroup);

  // This piece's first digits into the layer's histogram.
  flush_hist<R>(sh, c.hist + (int64_t)sl * R * kHistBins);
}

// The MFMA kernel is held to 128 registers (four waves per SIMD, 16 per
// compute unit: the memory parallelism the stream needs); it fits without
// spilling.  The vector-ALU kernel would spill there and is left unconstrained.
template <int R, int D, class Engine>
__global__ __launch_bounds__(kScoreThreads) __attribute__((amdgpu_waves_per_eu(4, 8)))
void score_kernel_mfma(Call c) {
  score_body<R, D, Engine>(c);
}

template <int R, int D, class Engine>
__global__ __launch_bounds__(kScoreThreads) void score_kernel_valu(Call c) {
  score_body<R, D, Engine>(c);
}

constexpr int kRing = 3;  // load buffers per wave: two groups of key rows in flight

template <int R, int D>
hipError_t launch_rd(const Call& c, dim3 grid, hipStream_t s) {
  if (c.engine == kEngineValu)
    hipLaunchKernelGGL((score_kernel_valu<R, D, ValuEngine<R, D, kRing>>), grid,
                       dim3(kScoreThreads), 0, s, c);
  else
    hipLaunchKernelGGL((score_kernel_mfma<R, D, MfmaEngine<R, D, kRing>>), grid,
                       dim3(kScoreThreads), 0, s, c);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const Call& c, dim3 grid, hipStream_t s) {
  switch (c.rows) {
    case 1: return launch_rd<1, D>(c, grid, s);
    case 2: return launch_rd<2, D>(c, grid, s);
    case 3: return launch_rd<3, D>(c, grid, s);
    case 4: return launch_rd<4, D>(c, grid, s);
    case 5: return launch_rd<5, D>(c, grid, s);
    case 6: return launch_rd<6, D>(c, grid, s);
    case 7: return launch_rd<7, D>(c, grid, s);
    case 8: return launch_rd<8, D>(c, grid, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_score(const Call& c, hipStream_t stream) {
  if (c.blocks == 0) return hipSuccess;
  // One workgroup per piece of c.piece positions of one layer; the host cannot
  // see how many positions are admitted, so the grid covers full admission and
  // the surplus workgroups exit at once.
  const int64_t per_layer = (c.blocks + c.piece - 1) / c.piece;
  dim3 grid((unsigned)(per_layer * c.layers));
  switch (c.dim) {
    case 32: return launch_d<32>(c, grid, stream);
    case 64: return launch_d<64>(c, grid, stream);
    case 128: return launch_d<128>(c, grid, stream);
    case 256: return launch_d<256>(c, grid, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace dssel
