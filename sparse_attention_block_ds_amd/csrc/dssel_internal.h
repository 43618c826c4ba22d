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

constexpr int kPrepThreads = 512;
constexpr int kPrepWordsPerThread = 8;

constexpr int kScoreThreads = 256;           // 4 waves
constexpr int kScoreChunk = 2048;            // union positions per score workgroup

constexpr int kSelectThreads = 1024;         // 16 waves
constexpr int kSelectBuf = 8192;             // LDS (key, position) slots for the select

enum AdmitMode : int {
  kNoMask = 0,      // admitted = b < limit: the compacted index is the identity
  kSharedMask = 1,  // one mask row per layer: every row's list is a prefix of one list
  kRowMask = 2,     // a mask row per query row: one union list, per-row sentinels
};

// Everything one call needs, in element units, passed by value to kernels.
struct Call {
  int32_t layers, rows, heads, dim, k;
  int32_t mode;
  int64_t blocks;
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
  // scratch (owned by the handle), laid out with this call's dimensions
  float* qt;          // [L][R][d] folded query rows
  int32_t* list;      // [L][N] compacted admitted (union) index, ascending
  int32_t* counts;    // [L][kCountStride]
  uint32_t* skeys;    // [L][R][N] radix keys at compacted positions
  uint32_t* hist;     // [L][R][kHistBins] first-digit histograms
};

hipError_t launch_prep(const Call& c, hipStream_t stream);
hipError_t launch_score(const Call& c, hipStream_t stream);
hipError_t launch_select(const Call& c, hipStream_t stream);

}  // namespace dssel
