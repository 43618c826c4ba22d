// score: one pass over the admitted block keys shared by all query rows of a
// layer; every (row, block) score at or above the row's candidate floor leaves
// as a (key, position) candidate.
//
// Page "DeepSeek V4.1F Q4 on M3 Ultra with native DSpark MTP (40tps /
// 800tps)": paragraph "Decode at depth" -- only admitted blocks are scored;
// paragraph "DSpark" -- the rows of a speculative verify share one stream of
// data, here the key stream: each admitted K row is read from HBM once and
// dotted with every row's query.
//
// Work split: the admitted positions of all layers are cut into equal pieces
// sized on the device from the admitted totals, so that one launch fills every
// resident slot (four workgroups per compute unit) and each workgroup streams
// the same number of key rows whatever the masks look like; a piece lies in
// one layer.  A workgroup:
//  0. Finds its piece from the per-layer admitted counts (wave 0).
//  1. Set-up, one round of independent loads: the layer's counts, limits and
//     floors, the piece's slice of the compacted index (built by prep) into
//     LDS, and the folded query.
//  2. Key stream: each wave takes 16 consecutive compacted entries at a time
//     and loads their K rows with 16-byte loads (each instruction reads 16 rows
//     x 64 contiguous bytes), two steps ahead of the arithmetic.
//       MFMA engine: v_mfma_f32_16x16x32_bf16 with the fp32 q~ entering as
//       three bf16 parts (hi + mid + lo == q~, exact for |q~_i| >= 2^-110)
//       along the M dimension
//       (row m = 4 * (query row % 4) + part), so the bf16 keys feed the
//       matrix cores directly: no vector-ALU conversion, no cross-lane sum.
//       VALU engine: d/8 lanes per key row, 8 fp32 FMAs per lane and row, a
//       butterfly across the row's lanes.
//  3. Epilogue: the score becomes an order-preserving radix key; keys at or
//     above the row's floor are staged in one LDS list per wave, tagged with
//     their row (one ballot per row set of the MFMA output, so a group costs
//     two ballots whatever the row count).  At the end of the piece the
//     workgroup counts its staged keys per row, reserves room in each row's
//     candidate list with one global atomic per row, and copies them out; a
//     wave whose list fills mid-piece distributes it the same way with
//     atomics of its own.  Nothing is written for the keys below the floor:
//     writing every key would add one write for every 10 to 64 bytes read,
//     and writes mixed into the read stream cost the stream far more than
//     their size.
#include "device_util.h"
#include "dssel_internal.h"
#include "relu_heads.h"

namespace dssel {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kGroup = 16;                     // compacted entries per wave step
constexpr int kWaves = kScoreThreads / kWave;  // 4
constexpr int kPiece = kScorePieceMax + 2 * kGroup;  // largest piece one workgroup streams
constexpr bool kInterleavedPieces = true;  // a piece is every P-th group of 16 positions

__device__ __forceinline__ u32x4_t load16(const uint16_t* p) {
  return *reinterpret_cast<const u32x4_t*>(p);
}

// A staged candidate: its key and its layer position, tagged with its row.
constexpr int kRowShift = kPositionBits;  // positions are below 2^26 (the block limit)
static_assert(kMaxRows <= 32, "row tag must fit above the position bits");

template <int R>
struct ScoreShared {
  int32_t list[kPiece];
  uint8_t rowbits[kPiece];  // mask row per query row: bit r = row r admits the element
  uint2 stage[kWaves][kWaveStage];  // (key, position | row << kRowShift)
  int P[kMaxRows];
  int64_t lim[kMaxRows];
  uint32_t floor[kMaxRows];
  int piece[4];
  int rowcnt[kWaves][kMaxRows];  // end of piece: each wave's staged count per row
  int base[kMaxRows];            // end of piece: the workgroup's slot in each row's list
};

// Number of lanes below this one whose bit is set in `bal`.
__device__ __forceinline__ int lanes_below(uint64_t bal) {
  return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32),
                                        __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
}

// Per-wave candidate staging and the piece's context.
template <int R>
struct PieceCtx {
  int off, cnt;                // elements [0, cnt); element e is position pos_of(e) of the layer
  int pj, pn, nl;              // interleaved: piece j of pn, layer's admitted count nl
  int mode;
  const ScoreShared<R>* sh;
  uint2* stage;                // this wave's [kWaveStage]
  int nst;                     // staged entries, the same in every lane of the wave
  int32_t* cand_count;         // [R][kCountPad] of this layer
  uint64_t* cand;              // [R][stride] of this layer
  int64_t stride;

  // Layer position of piece element e: contiguous pieces hold [off, off + cnt);
  // interleaved piece j of pn holds groups j, j + pn, j + 2 pn, ... of 16.
  __device__ __forceinline__ int pos_of(int e) const {
    return kInterleavedPieces ? ((e >> 4) * pn + pj) * kGroup + (e & (kGroup - 1)) : off + e;
  }

  __device__ __forceinline__ bool valid(int e) const { return e < cnt && pos_of(e) < nl; }

  __device__ __forceinline__ int block_of(int e) const {
    return mode == kNoMask ? pos_of(e) : sh->list[e];
  }

  // With a mask row per query row, the union list also holds blocks that row
  // r does not admit: its own bit and limit, gathered at the piece's set-up
  // (no global load inside the stream, whose loads then stay in flight).
  __device__ __forceinline__ bool row_admits(int r, int e) const {
    return (sh->rowbits[e] >> r) & 1u;
  }

  // Stage the lanes' candidates: lane i offers (key, position pos of row r)
  // when ok.  Called by every lane of the wave.
  __device__ __forceinline__ void append(bool ok, uint32_t key, int pos, int r) {
    const uint64_t bal = __ballot(ok);
    if (bal == 0) return;
    const int n = __popcll(bal);
    if (__builtin_expect(nst + n > kWaveStage, 0)) spill();
    if (ok) stage[nst + lanes_below(bal)] = make_uint2(key, (uint32_t)pos | ((uint32_t)r << kRowShift));
    nst += n;
  }

  // Lane r (< R) gets the number of staged entries of row r.
  __device__ __forceinline__ int count_rows() const {
    const int lane = lane_id();
    int mine = 0;
    for (int i0 = 0; i0 < nst; i0 += kWave) {
      const int i = i0 + lane;
      const int row = i < nst ? (int)(stage[i].y >> kRowShift) : -1;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int n = __popcll(__ballot(row == r));
        if (lane == r) mine += n;
      }
    }
    return mine;
  }

  // Copy the staged entries out; lane r (< R) holds the first slot of row r's
  // run in the row's list.  Entries keep their staging order within a row.
  __device__ __forceinline__ void write_out(int start) const {
    const int lane = lane_id();
    int run = start;  // lane r: next free slot of row r
    for (int i0 = 0; i0 < nst; i0 += kWave) {
      const int i = i0 + lane;
      const uint2 v = i < nst ? stage[i] : make_uint2(0u, 0xFFFFFFFFu);
      const int row = i < nst ? (int)(v.y >> kRowShift) : -1;
      uint64_t my = 0;
      int add = 0;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const uint64_t b = __ballot(row == r);
        if (row == r) my = b;
        if (lane == r) add = __popcll(b);
      }
      const int slot = __shfl(run, row < 0 ? 0 : row, kWave) + lanes_below(my);
      if (row >= 0 && slot < stride) {
        const uint32_t pos = v.y & ((1u << kRowShift) - 1u);
        cand[row * stride + slot] = ((uint64_t)v.x << 32) | (uint32_t)~pos;
      }
      run += add;
    }
  }

  // Mid-piece: the wave's list is full.  Distribute it with one atomic per
  // row of the wave's own (a cold path).
  __device__ void spill() {
    wave_lds_sync();
    const int lane = lane_id();
    const int n = count_rows();
    int start = 0;
    if (lane < R && n > 0) start = atomicAdd(&cand_count[lane * kCountPad], n);
    write_out(start);
    wave_lds_sync();
    nst = 0;
    // Rejoin the stream with nothing of this path in flight, so that the
    // stream's own counter waits (for its prefetched key rows) stay partial.
    __builtin_amdgcn_s_waitcnt(0);
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
  static constexpr bool kPairs = false;
  static constexpr int KC = D / 32;       // 32-column chunks of a key row
  static constexpr int S = (R + 3) / 4;   // MFMA row sets
  bf16x8_t a[S][KC];                      // A operand: q~ parts (row m = lane % 16)
  u32x4_t buf[NBUF][KC];                  // B operand: K rows (block = lane % 16)

  __device__ void init(const Call& c, int l, uint32_t*) {
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
    // Every lane loads (a lane past the piece's end re-reads the group's first
    // row, whose score it never offers), so the stream has no divergent
    // branch around its loads and the counter waits stay exact.
    const int lane = lane_id();
    const int e = g0 + (lane & 15);
    const uint16_t* row = K + (int64_t)t.block_of(t.valid(e) ? e : g0) * ldk + 8 * (lane >> 4);
#pragma unroll
    for (int cc = 0; cc < KC; ++cc) buf[B][cc] = load16(row + 32 * cc);
  }

  template <int B>
  __device__ __forceinline__ void compute_emit(PieceCtx<R>& t, int g0) {
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
    const int e = g0 + (lane & 15), g = lane >> 4;
    const int pos = t.pos_of(e);
    const bool live = e < t.cnt;
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const uint32_t key = score_to_key((acc[s][0] + acc[s][1]) + acc[s][2]);
      bool ok = live && pos < lp[s] && key >= lf[s];
      if (t.mode == kRowMask && ok) ok = t.row_admits(4 * s + g, e);
      t.append(ok, key, pos, 4 * s + g);
    }
  }

  // The lane's rows of the MFMA output (row 4 s + lane / 16 of set s): their
  // admitted counts (0 past R) and floors.
  int lp[S];
  uint32_t lf[S];
  __device__ void bind_rows(const ScoreShared<R>& sh) {
    const int g = lane_id() >> 4;
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const int r = 4 * s + g;
      lp[s] = r < R ? sh.P[r] : 0;
      lf[s] = r < R ? sh.floor[r] : 0u;
    }
  }
};

// ------------------------------------------------------- MFMA engine, 8-bit keys
// The same A operand (q~ as three bf16 parts along M) against 8-bit key
// rows: group g of a row is 32 int8 codes c with one fp16 scale s, standing
// for the values s c.  Each 32-column chunk is one group, so each chunk gets
// its own accumulation: the codes widen exactly to bf16 (B operand), one
// v_mfma_f32_16x16x32_bf16 per row set gives sum_i q~_i c_i over the group
// (exact products), and the lane adds s times that sum to its row's score.
// Each lane loads 8 codes (8 bytes) per chunk of its block and the block's
// group scales.
template <int R, int D, int NBUF>
struct MfmaQ8Engine {
  static constexpr int kRows = R, kBuffers = NBUF;
  static constexpr bool kPairs = false;
  static constexpr int KC = D / 32;       // 32-column groups of a key row
  static constexpr int S = (R + 3) / 4;   // MFMA row sets
  bf16x8_t a[S][KC];
  uint2 buf[NBUF][KC];                    // codes: 8 of the lane's block per group
  uint32_t sbuf[NBUF][(KC + 1) / 2];      // the block's group scales, two fp16 per word
  const int8_t* codes_l;
  const uint16_t* scales_l;
  int64_t ldc, lds;

  __device__ void init(const Call& c, int l, uint32_t*) {
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
    codes_l = c.codes + (int64_t)l * c.code_layer_stride;
    scales_l = c.scales + (int64_t)l * c.scale_layer_stride;
    ldc = c.ldc;
    lds = c.lds;
  }

  template <int B>
  __device__ __forceinline__ void load(const PieceCtx<R>& t, const uint16_t*, int64_t, int g0) {
    const int lane = lane_id();
    const int e = g0 + (lane & 15);
    const int64_t b = t.block_of(t.valid(e) ? e : g0);
    const int8_t* row = codes_l + b * ldc + 8 * (lane >> 4);
#pragma unroll
    for (int cc = 0; cc < KC; ++cc) buf[B][cc] = *reinterpret_cast<const uint2*>(row + 32 * cc);
    const uint16_t* sr = scales_l + b * lds;
#pragma unroll
    for (int h = 0; h < (KC + 1) / 2; ++h)
      sbuf[B][h] = (uint32_t)sr[2 * h] | (2 * h + 1 < KC ? (uint32_t)sr[2 * h + 1] << 16 : 0u);
  }

  template <int B>
  __device__ __forceinline__ void compute_emit(PieceCtx<R>& t, int g0) {
    float score[S];
#pragma unroll
    for (int s = 0; s < S; ++s) score[s] = 0.0f;
#pragma unroll
    for (int cc = 0; cc < KC; ++cc) {
      const u32x4_t bv = {bf16_pair_of_codes(buf[B][cc].x, 0), bf16_pair_of_codes(buf[B][cc].x, 16),
                          bf16_pair_of_codes(buf[B][cc].y, 0), bf16_pair_of_codes(buf[B][cc].y, 16)};
      const float scale = half_bits_to_f32((uint16_t)(sbuf[B][cc / 2] >> (16 * (cc & 1))));
#pragma unroll
      for (int s = 0; s < S; ++s) {
        const f32x4_t acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            a[s][cc], __builtin_bit_cast(bf16x8_t, bv), f32x4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
        score[s] += scale * ((acc[0] + acc[1]) + acc[2]);
      }
    }
    const int lane = lane_id();
    const int e = g0 + (lane & 15), g = lane >> 4;
    const int pos = t.pos_of(e);
    const bool live = e < t.cnt;
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const uint32_t key = score_to_key(score[s]);
      bool ok = live && pos < lp[s] && key >= lf[s];
      if (t.mode == kRowMask && ok) ok = t.row_admits(4 * s + g, e);
      t.append(ok, key, pos, 4 * s + g);
    }
  }

  int lp[S];
  uint32_t lf[S];
  __device__ void bind_rows(const ScoreShared<R>& sh) {
    const int g = lane_id() >> 4;
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const int r = 4 * s + g;
      lp[s] = r < R ? sh.P[r] : 0;
      lf[s] = r < R ? sh.floor[r] : 0u;
    }
  }
};

// ------------------------------------------------------ per-head ReLU engine
// The unfolded score sum_h w_h max(q_h . K, 0): the key rows load as for the
// MFMA engine (block = lane % 16, 16 bytes per 32 columns); each row's score
// is R x (H / 16) x (d / 32) MFMAs against the heads staged in LDS
// (relu_heads.h), complete in all four lanes of a block.  The lanes of group
// g then offer row 4 s + g of set s, as the MFMA engine's do.
template <int R, int D, int NBUF>
struct ReluEngine {
  static constexpr int kRows = R, kBuffers = NBUF;
  static constexpr bool kPairs = true;  // two groups per buffer: each LDS fragment feeds 2 MFMAs
  static constexpr int KC = D / 32;
  static constexpr int S = (R + 3) / 4;
  relu_u32x4_t buf[NBUF][2][KC];
  ReluStage st;

  __device__ void init(const Call& c, int l, uint32_t* lds) {
    st = relu_stage_heads<R, D>(c, (int64_t)l * R, lds, threadIdx.x, kScoreThreads);
  }

  // Groups ga and gb (both valid group starts) into buffer B.
  template <int B>
  __device__ __forceinline__ void load2(const PieceCtx<R>& t, const uint16_t* K, int64_t ldk, int ga, int gb) {
    const int lane = lane_id();
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int g0 = h ? gb : ga;
      const int e = g0 + (lane & 15);
      const uint16_t* row = K + (int64_t)t.block_of(t.valid(e) ? e : g0) * ldk + 8 * (lane >> 4);
#pragma unroll
      for (int cc = 0; cc < KC; ++cc) buf[B][h][cc] = load16(row + 32 * cc);
    }
  }

  template <int B>
  __device__ __forceinline__ void compute_emit2(PieceCtx<R>& t, int ga, int gb) {
    float o[R][2];
    relu_all_rows<R, D, 2, (R * KC <= 32)>(st, buf[B], o);  // prefetch while it fits
    const int lane = lane_id();
    const int g = lane >> 4;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int e = (h ? gb : ga) + (lane & 15);
      const int pos = t.pos_of(e);
      const bool live = e < t.cnt;
#pragma unroll
      for (int s = 0; s < S; ++s) {
        float v = o[0][h];
#pragma unroll
        for (int r = 1; r < R; ++r)
          if (r == 4 * s + g) v = o[r][h];
        const uint32_t key = score_to_key(v);
        bool ok = live && pos < lp[s] && key >= lf[s];
        if (t.mode == kRowMask && ok) ok = t.row_admits(4 * s + g, e);
        t.append(ok, key, pos, 4 * s + g);
      }
    }
  }

  int lp[S];
  uint32_t lf[S];
  __device__ void bind_rows(const ScoreShared<R>& sh) {
    const int g = lane_id() >> 4;
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const int r = 4 * s + g;
      lp[s] = r < R ? sh.P[r] : 0;
      lf[s] = r < R ? sh.floor[r] : 0u;
    }
  }
};

// ---------------------------------------------------------------- VALU engine
template <int R, int D, int NBUF>
struct ValuEngine {
  static constexpr int kRows = R, kBuffers = NBUF;
  static constexpr bool kPairs = false;
  static constexpr int LPR = D / 8;        // lanes per key row
  static constexpr int RPI = kWave / LPR;  // key rows per load instruction
  static constexpr int U = kGroup / RPI;   // load instructions per group
  float qv[R][8];
  u32x4_t buf[NBUF][U];

  __device__ void init(const Call& c, int l, uint32_t*) {
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
      buf[B][u] = load16(K + (int64_t)t.block_of(t.valid(e) ? e : g0) * ldk + slice * 8);
    }
  }

  template <int B>
  __device__ __forceinline__ void compute_emit(PieceCtx<R>& t, int g0) {
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
      const int pos = t.pos_of(e);
      const bool live = e < t.cnt;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const uint32_t key = score_to_key(acc[r]);
        bool ok = r % LPR == slice && live && pos < t.sh->P[r] && key >= t.sh->floor[r];
        if (t.mode == kRowMask && ok) ok = t.row_admits(r, e);
        t.append(ok, key, pos, r);
      }
    }
  }

  __device__ void bind_rows(const ScoreShared<R>&) {}
};

// Runs the wave's groups g0, g0 + step, ... < cnt through a ring of NBUF load
// buffers: the loads for group j + NBUF - 1 are issued before group j is
// computed, so NBUF - 1 groups of key rows are in flight behind the arithmetic.
// The loads are issued unconditionally (a prefetch past the last group re-reads
// the group being computed, an L2 hit): with no branch around them the
// compiler's counter waits stay exact, and a computing group waits only for
// its own rows, never for the younger groups' loads.
template <int NBUF, class Engine, int J>
__device__ __forceinline__ void ring_step(Engine& eng, PieceCtx<Engine::kRows>& pc,
                                          const uint16_t* K, int64_t ldk, int g, int step) {
  if constexpr (J < NBUF) {
    const int gj = g + J * step;
    if (gj >= pc.cnt) return;
    const int gl = gj + (NBUF - 1) * step;
    eng.template load<(J + NBUF - 1) % NBUF>(pc, K, ldk, gl < pc.cnt ? gl : gj);
    eng.template compute_emit<J>(pc, gj);
    ring_step<NBUF, Engine, J + 1>(eng, pc, K, ldk, g, step);
  }
}

template <int NBUF, class Engine, int J>
__device__ __forceinline__ void ring_prologue(Engine& eng, PieceCtx<Engine::kRows>& pc,
                                              const uint16_t* K, int64_t ldk, int g0, int step) {
  if constexpr (J < NBUF - 1) {
    const int gj = g0 + J * step;
    eng.template load<J>(pc, K, ldk, gj < pc.cnt ? gj : g0);
    ring_prologue<NBUF, Engine, J + 1>(eng, pc, K, ldk, g0, step);
  }
}

template <int NBUF, class Engine>
__device__ __forceinline__ void stream_piece(Engine& eng, PieceCtx<Engine::kRows>& pc,
                                             const uint16_t* K, int64_t ldk, int g0, int step) {
  if (g0 >= pc.cnt) return;  // this wave has no group
  ring_prologue<NBUF, Engine, 0>(eng, pc, K, ldk, g0, step);
  for (int g = g0; g < pc.cnt; g += NBUF * step) ring_step<NBUF, Engine, 0>(eng, pc, K, ldk, g, step);
}

// The same ring for an engine that takes two groups per buffer: pair p is
// groups g0 + 2 p step and g0 + (2 p + 1) step.  A group past the piece's end
// re-reads a valid group (never offered), so the loads stay unconditional.
template <int NBUF, class Engine, int J>
__device__ __forceinline__ void pair_step(Engine& eng, PieceCtx<Engine::kRows>& pc,
                                          const uint16_t* K, int64_t ldk, int g, int step) {
  if constexpr (J < NBUF) {
    const int pstep = 2 * step;
    const int gj = g + J * pstep;
    if (gj >= pc.cnt) return;
    const int gl = gj + (NBUF - 1) * pstep;
    const int la = gl < pc.cnt ? gl : gj;
    eng.template load2<(J + NBUF - 1) % NBUF>(pc, K, ldk, la, la + step < pc.cnt ? la + step : la);
    eng.template compute_emit2<J>(pc, gj, gj + step);
    pair_step<NBUF, Engine, J + 1>(eng, pc, K, ldk, g, step);
  }
}

template <int NBUF, class Engine, int J>
__device__ __forceinline__ void pair_prologue(Engine& eng, PieceCtx<Engine::kRows>& pc,
                                              const uint16_t* K, int64_t ldk, int g0, int step) {
  if constexpr (J < NBUF - 1) {
    const int ga = g0 + J * 2 * step;
    const int la = ga < pc.cnt ? ga : g0;
    eng.template load2<J>(pc, K, ldk, la, la + step < pc.cnt ? la + step : la);
    pair_prologue<NBUF, Engine, J + 1>(eng, pc, K, ldk, g0, step);
  }
}

template <int NBUF, class Engine>
__device__ __forceinline__ void stream_piece_pairs(Engine& eng, PieceCtx<Engine::kRows>& pc,
                                                   const uint16_t* K, int64_t ldk, int g0, int step) {
  if (g0 >= pc.cnt) return;
  pair_prologue<NBUF, Engine, 0>(eng, pc, K, ldk, g0, step);
  for (int g = g0; g < pc.cnt; g += NBUF * 2 * step) pair_step<NBUF, Engine, 0>(eng, pc, K, ldk, g, step);
}

// Which piece this workgroup streams.  Every layer's admitted positions are
// cut into pieces of T positions, where T = ceil(total / (slots - L)) clamped
// to [256, 2048], total is the admitted count summed over layers and slots the
// resident workgroups of the device; the layers' pieces are numbered in layer
// order and workgroup j takes piece j.  There are at most total / T + L pieces:
// no more than the slots unless T had to be clamped to 2048, and never more
// than the grid, which the host sizes for full admission at T = 2048.  So a
// usual call runs as one round of equal workgroups, and surplus ones exit.
struct Piece {
  int layer, j, pn, T;  // piece j of the pn pieces of `layer` (layer < 0: nothing to do)
};

__device__ __forceinline__ Piece find_piece(const Call& c, int* shared_out) {
  const int lane = lane_id();
  if (threadIdx.x < kWave) {
    const int L = c.layers;
    // the first 64 layers' counts stay in a register for the search below
    const int n0 = lane < L ? c.counts[(int64_t)lane * kCountStride + kMaxRows] : 0;
    int64_t total = 0;
    for (int l0 = 0; l0 < L; l0 += kWave) {
      const int l = l0 + lane;
      int64_t n = l0 == 0 ? n0 : (l < L ? c.counts[(int64_t)l * kCountStride + kMaxRows] : 0);
#pragma unroll
      for (int off = kWave / 2; off > 0; off >>= 1) n += __shfl_xor(n, off, kWave);
      total += n;
    }
    const int64_t div = (int64_t)c.score_slots - L;
    const int64_t per = div > 0 ? (total + div - 1) / div : kScorePieceMax;
    const int T = (int)(per < kScorePieceMin ? kScorePieceMin : (per > kScorePieceMax ? kScorePieceMax : per));
    const int j = blockIdx.x;
    int base = 0, layer = -1, pj = 0, pn = 0;
    for (int l0 = 0; l0 < L && layer < 0; l0 += kWave) {
      const int l = l0 + lane;
      const int n = l0 == 0 ? n0 : (l < L ? c.counts[(int64_t)l * kCountStride + kMaxRows] : 0);
      const int g = (n + T - 1) / T;
      const int incl = wave_inclusive_scan(g);
      const bool mine = j >= base + incl - g && j < base + incl;
      const uint64_t hit = __ballot(mine);
      if (hit) {
        const int src = __ffsll((long long)hit) - 1;
        layer = l0 + src;
        pj = j - (base + __shfl(incl - g, src, kWave));
        pn = __shfl(g, src, kWave);
      }
      base += __shfl(incl, kWave - 1, kWave);
    }
    if (lane == 0) {
      shared_out[0] = layer;
      shared_out[1] = pj;
      shared_out[2] = pn;
      shared_out[3] = T;
    }
  }
  __syncthreads();
  return Piece{shared_out[0], shared_out[1], shared_out[2], shared_out[3]};
}

template <int R, int D, class Engine>
__device__ __forceinline__ void score_body(const Call& c, uint32_t* relu_lds) {
  __shared__ ScoreShared<R> sh;
  const int tid = threadIdx.x, wave = tid / kWave;
  const int64_t N = c.blocks;
  const Piece pz = find_piece(c, sh.piece);
  if (pz.layer < 0) return;  // uniform for the workgroup
  const int sl = pz.layer;

  // Set-up: one round of independent loads.
  const int32_t* counts = c.counts + (int64_t)sl * kCountStride;
  const int nl = counts[kMaxRows];
  PieceCtx<R> pc;
  pc.nl = nl;
  pc.pj = pz.j;
  pc.pn = pz.pn;
  if (kInterleavedPieces) {
    const int groups = (nl + kGroup - 1) / kGroup;
    pc.off = 0;
    pc.cnt = ((groups - pz.j + pz.pn - 1) / pz.pn) * kGroup;
  } else {
    pc.off = pz.j * pz.T;
    pc.cnt = (pc.off + pz.T < nl ? pc.off + pz.T : nl) - pc.off;
  }
  if (c.mode != kNoMask) {
    // the piece's slice of the index: every load issued before any is stored
    const int32_t* list = c.list + (int64_t)sl * N;
    constexpr int kPer = (kPiece + kScoreThreads - 1) / kScoreThreads;
    int32_t v[kPer];
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int i = tid + u * kScoreThreads;
      const int pos = pc.pos_of(i);
      v[u] = (i < pc.cnt && pos < nl) ? list[pos] : 0;
    }
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int i = tid + u * kScoreThreads;
      if (i < pc.cnt) sh.list[i] = v[u];
    }
    if (c.mode == kRowMask) {
      const uint32_t* mask_l = c.mask + (int64_t)sl * c.mask_layer_stride;
      int64_t lim[R];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int64_t x = c.limit ? (int64_t)c.limit[(int64_t)sl * R + r] : N;
        lim[r] = x < 0 ? 0 : (x > N ? N : x);
      }
#pragma unroll
      for (int u = 0; u < kPer; ++u) {
        const int i = tid + u * kScoreThreads;
        if (i < pc.cnt) {
          const int b = v[u];
          uint32_t bits = 0;
#pragma unroll
          for (int r = 0; r < R; ++r) {
            const uint32_t word = mask_l[r * c.mask_row_stride + (b >> 5)];
            bits |= (((word >> (b & 31)) & 1u) && (int64_t)b < lim[r] ? 1u : 0u) << r;
          }
          sh.rowbits[i] = (uint8_t)bits;
        }
      }
    }
  }
  if (tid < kMaxRows) {
    sh.P[tid] = tid < R ? (c.mode == kRowMask ? nl : counts[tid]) : 0;
    sh.floor[tid] = tid < R ? c.floor_key[(int64_t)sl * R + tid] : 0u;
    const int64_t v = (c.limit && tid < R) ? (int64_t)c.limit[(int64_t)sl * R + tid] : N;
    sh.lim[tid] = v < 0 ? 0 : (v > N ? N : v);
  }
  Engine eng;
  eng.init(c, sl, relu_lds);
  __syncthreads();

  pc.mode = c.mode;
  pc.sh = &sh;
  pc.stage = &sh.stage[wave][0];
  pc.nst = 0;
  eng.bind_rows(sh);
  pc.cand_count = c.cand_count + (int64_t)sl * R * kCountPad;
  pc.cand = c.cand + (int64_t)sl * R * c.cand_stride;
  pc.stride = c.cand_stride;
  const uint16_t* K = c.keys ? c.keys + (int64_t)sl * c.key_layer_stride : nullptr;
  if constexpr (Engine::kPairs)
    stream_piece_pairs<Engine::kBuffers>(eng, pc, K, c.ldk, wave * kGroup, kWaves * kGroup);
  else
    stream_piece<Engine::kBuffers>(eng, pc, K, c.ldk, wave * kGroup, kWaves * kGroup);
  // End of the piece: one counter update per row for the whole workgroup.
  const int lane = lane_id();
  const int mine = pc.count_rows();  // lane r: this wave's staged entries of row r
  if (lane < R) sh.rowcnt[wave][lane] = mine;
  __syncthreads();
  if (tid < R) {
    int n = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) n += sh.rowcnt[w][tid];
    sh.base[tid] = n ? atomicAdd(&pc.cand_count[tid * kCountPad], n) : 0;
  }
  __syncthreads();
  int start = 0;
  if (lane < R) {
    start = sh.base[lane];
    for (int w = 0; w < wave; ++w) start += sh.rowcnt[w][lane];
  }
  pc.write_out(start);
}

// Load buffers per wave: two groups of key rows in flight; one at d = 256,
// where a third buffer of 16-byte bf16 chunks (32 registers) does not fit.
template <int D>
constexpr int kRing = D >= 256 ? 2 : 3;

// The MFMA kernel is held to at least W waves per SIMD: 4 (128 registers, 16
// waves per compute unit: the memory parallelism the stream needs) at
// d <= 128; at d = 256 the A operand and the ring need more, so 3 (168
// registers) up to four rows and 2 above, where the A operand alone takes 64.
// No instantiation spills.  The vector-ALU kernel is left unconstrained.
template <int R, int D, class Engine, int W>
__global__ __launch_bounds__(kScoreThreads) __attribute__((amdgpu_waves_per_eu(W, 8)))
void score_kernel_mfma(Call c) {
  score_body<R, D, Engine>(c, nullptr);
}

template <int R, int D, class Engine>
__global__ __launch_bounds__(kScoreThreads) void score_kernel_valu(Call c) {
  score_body<R, D, Engine>(c, nullptr);
}

// The per-head ReLU kernel: one workgroup per compute unit holds the layer's
// heads (up to 120 KiB of LDS), so its four waves each run one SIMD.
template <int R, int D>
__global__ __launch_bounds__(kScoreThreads) void score_kernel_relu(Call c) {
  __shared__ uint32_t relu_lds[kReluStageBytes / 4];
  score_body<R, D, ReluEngine<R, D, kRing<D>>>(c, relu_lds);
}

template <int R, int D>
hipError_t launch_rd(const Call& c, dim3 grid, hipStream_t s) {
  constexpr int kMfmaWaves = D < 256 ? 4 : (R > 4 ? 2 : 3);
  if (c.fmt == kKeysQ8)
    hipLaunchKernelGGL((score_kernel_mfma<R, D, MfmaQ8Engine<R, D, kRing<D>>, kMfmaWaves>), grid,
                       dim3(kScoreThreads), 0, s, c);
  else if (c.score_kind == kScoreHeadRelu)
    hipLaunchKernelGGL((score_kernel_relu<R, D>), grid, dim3(kScoreThreads), 0, s, c);
  else if (c.engine == kEngineValu)
    hipLaunchKernelGGL((score_kernel_valu<R, D, ValuEngine<R, D, kRing<D>>>), grid,
                       dim3(kScoreThreads), 0, s, c);
  else
    hipLaunchKernelGGL((score_kernel_mfma<R, D, MfmaEngine<R, D, kRing<D>>, kMfmaWaves>), grid,
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
  // The host cannot see how many positions are admitted: the grid is sized
  // for full admission and for every resident slot, and workgroups without a
  // piece exit at once.
  dim3 grid((unsigned)c.score_wgs);
  switch (c.dim) {
    case 32: return launch_d<32>(c, grid, stream);
    case 64: return launch_d<64>(c, grid, stream);
    case 128: return launch_d<128>(c, grid, stream);
    case 256: return launch_d<256>(c, grid, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace dssel
