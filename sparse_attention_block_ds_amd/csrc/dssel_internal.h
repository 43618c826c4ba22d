// Internal declarations shared by the host side (ds_sel.cpp) and the kernels
// of libdssel.  Not installed; the public ABI is include/ds_sel.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dssel {

// Radix key: an order-preserving uint32 image of an fp32 score.  The first
// digit is the top 11 bits (sign, 8 exponent bits, 2 mantissa bits), the
// second the next 11 bits, the third the last 10.
constexpr int kDigit1Bits = 11;
constexpr int kDigit1Shift = 21;
constexpr int kHistBins = 1 << kDigit1Bits;  // 2048
constexpr int kDigit2Shift = 10;
constexpr int kDigit3Bins = 1 << 10;

constexpr int kMaxRows = 8;
constexpr int kCountStride = kMaxRows + 1;   // per layer: n_r for r < 8, union size at [8]

// The block axis is cut into tiles of 2048 blocks (64 mask words); one wave
// expands one tile of the compacted admitted index.
constexpr int kTileBlocks = 2048;
constexpr int kTileWords = kTileBlocks / 32;

constexpr int kPrepThreads = 1024;                  // 16 waves
constexpr int kPrepTilesPerWg = kPrepThreads / 64;  // tiles expanded per prep workgroup
constexpr int kSampleSlots = 512;                   // the most blocks per row scored to place the floor

constexpr int kScoreThreads = 256;           // 4 waves
constexpr int kScorePieceMax = 2048;         // admitted positions per score workgroup: at most,
constexpr int kScorePieceMin = 256;          // and at least: on small calls fewer, longer pieces
                                             // finish sooner than one short piece per slot
constexpr int kScoreWgsPerCu = 4;            // resident score workgroups per compute unit
constexpr int kWaveStage = 512;              // per-wave candidate staging, all rows (LDS)
constexpr int kCountPad = 32;                // candidate counters sit 128 bytes apart
constexpr int kPositionBits = 26;            // staged candidates tag the row above the position

constexpr int kSelectBuf = 8192;             // candidates the select holds in registers
constexpr int kGatherSlack = 64;             // radix passes stop once m + this many words remain

enum AdmitMode : int {
  kNoMask = 0,      // admitted = b < limit: the compacted index is the identity
  kSharedMask = 1,  // one mask row per layer: every row's list is a prefix of one list
  kRowMask = 2,     // a mask row per query row: one union list, per-row admission
};

enum KeyFormat : int {
  kKeysBf16 = 0,  // bf16 key rows
  kKeysQ8 = 1,    // groups of 32 int8 codes, one fp16 scale per group
};

enum Engine : int {
  kEngineMfma = 0,  // bf16 matrix cores on a 3-way bf16 split of the fp32 q~ (exact for |q~_i| >= 2^-110)
  kEngineValu = 1,  // fp32 FMAs on the vector ALUs
};

// Everything one call needs, in element units, passed by value to kernels.
// The block score: the linear sum_h w_h (q_h . K) (folded), or the per-head
// ReLU variant sum_h w_h max(q_h . K, 0) (unfolded: every head on the matrix cores).
enum ScoreKind : int {
  kScoreLinear = 0,
  kScoreHeadRelu = 1,
};

// The per-head ReLU kernels stage a layer's query heads and weights in LDS:
// bf16 q [R][Hp][d + 8] (rows padded by 16 bytes) then fp32 w [R][Hp], with
// Hp = H rounded up to 16 and zeros past H.  The stage must fit this budget.
constexpr int kReluStageBytes = 120 * 1024;
constexpr int64_t relu_stage_bytes(int64_t rows, int64_t heads, int64_t dim) {
  return rows * ((heads + 15) / 16 * 16) * (2 * (dim + 8) + 4);
}

struct Call {
  int32_t layers, rows, heads, dim, k;
  int32_t mode, engine;
  int32_t score_kind;   // ScoreKind
  int32_t ntiles;     // ceil(N / kTileBlocks)
  int32_t score_wgs;    // score grid: >= layers + ceil(L * N / kScorePieceMax)
  int32_t score_slots;  // resident score workgroups on the device
  int64_t blocks;
  int64_t cand_stride;  // candidate slots per (layer, row): N rounded up to 4
  const uint16_t* q;
  const uint16_t* w;
  const uint16_t* keys;
  int64_t ldk, key_layer_stride;
  const uint32_t* mask;
  int64_t mask_row_stride, mask_layer_stride;
  const int32_t* limit;
  int32_t* out_idx;
  float* out_score;
  int32_t* out_count;
  // 8-bit keys (fmt == kKeysQ8): codes [L][N][ldc], fp16 scales [L][N][lds]
  int32_t fmt;
  const int8_t* codes;
  int64_t ldc, code_layer_stride;
  const uint16_t* scales;
  int64_t lds, scale_layer_stride;
  // scratch (owned by the handle), laid out with this call's dimensions
  float* qt;           // [L][R][d] folded query rows, fp32
  uint16_t* qparts;    // [L][3][R][d] bf16 hi/mid/lo parts of q~ (hi + mid + lo == q~)
  int32_t* list;       // [L][N] compacted admitted (union) index, ascending
  int32_t* counts;     // [L][kCountStride]
  uint32_t* floor_key; // [L][R] candidate floor: keys below it cannot be in the top k
  int32_t* cand_count; // [L][R][kCountPad] candidates appended (element 0 of each line)
  uint64_t* cand;      // [L][R][cand_stride] (key << 32) | ~position, unordered
};

// Attention over the selected blocks.  One workgroup of kAttendThreads per
// (head tile, split, row, layer); a split covers chunks_per_split chunks of
// kAttendChunk selected blocks.  With several splits each writes a partial
// record (max, sum, unnormalised o per head) that a second kernel merges.
constexpr int kAttendThreads = 256;
constexpr int kAttendHeadTile = 64;   // heads per workgroup, 16 per wave
constexpr int kAttendChunk = 64;
constexpr int kAttendMaxK = 2048;     // selections longer than this are not accepted
constexpr int kAttendPartialWgs = 512;  // partial records the scratch holds (per head tile)

struct AttendCall {
  int32_t layers, rows, heads, dim, k;
  int32_t head_tiles;        // ceil(heads / kAttendHeadTile)
  int32_t splits;            // workgroups per (layer, row, head tile)
  int32_t chunks_per_split;  // ceil(ceil(k / kAttendChunk) / splits)
  int64_t blocks;
  float scale;
  const uint16_t* q;         // [L][R][heads][d]
  const uint16_t* keys;
  int64_t ldk, key_layer_stride;
  const uint16_t* values;
  int64_t ldv, value_layer_stride;
  const int32_t* idx;        // [L][R][k]
  const int32_t* count;      // [L][R] or null (all k slots)
  float* out;                // [L][R][heads][d]
  float* part_ml;            // [records][kAttendHeadTile][2] (max, sum), base-2 units
  float* part_o;             // [records][kAttendHeadTile][d]
};

hipError_t launch_attend(const AttendCall& c, hipStream_t stream);

// Quantising bf16 key rows into the 8-bit stream (ds_sel_quantize_q8).
// The serial decode's step between layers: layer l + 1's query heads rotated
// by layer l's best block per row (decode.hip).
struct RotateCall {
  int32_t rows, heads, dim, k;
  const uint16_t* q_next;  // bf16 [R][H][d]: layer l + 1's base query
  const int32_t* idx;      // int32 [R][k]: layer l's selection
  uint16_t* q_out;         // bf16 [R][H][d]: layer l + 1's query
};
hipError_t launch_rotate(const RotateCall& c, hipStream_t stream);

struct QuantizeCall {
  int32_t layers, dim;
  int64_t blocks;
  const uint16_t* keys;
  int64_t ldk, key_layer_stride;
  int8_t* codes;
  int64_t ldc, code_layer_stride;
  uint16_t* scales;
  int64_t lds, scale_layer_stride;
};
hipError_t launch_quantize(const QuantizeCall& c, hipStream_t stream);

// Calibration launches (an empty kernel, a plain read of every key row, a
// gather of the admitted key rows); see ds_sel_calibrate.
enum CalibKind : int { kCalibEmpty = 0, kCalibRead = 1, kCalibGather = 2 };

struct CalibCall {
  int32_t kind, workgroups, layers, dim;
  int64_t blocks, ldk, key_layer_stride, mask_layer_stride;
  const uint16_t* keys;
  const uint32_t* mask;   // gather: one mask row per layer, or null (every block)
  const int64_t* ranges;  // gather: [workgroups + 1] flattened (layer * N + block) starts
  uint32_t* sink;         // [workgroups]
};

hipError_t launch_calibrate(const CalibCall& c, hipStream_t stream);

hipError_t launch_prep(const Call& c, hipStream_t stream);
hipError_t launch_score(const Call& c, hipStream_t stream);
hipError_t launch_select(const Call& c, hipStream_t stream);

}  // namespace dssel
