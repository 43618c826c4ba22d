// select: the bounded radix select of the best k keys of every (layer, row),
// with ties broken by the lower block index, and the ordered output.
//
// Page "DeepSeek V4.1F Q4 on M3 Ultra with native DSpark MTP (40tps /
// 800tps)", paragraph "Decode at depth": the top 512 are taken with a radix
// select of bounded depth.  Here every pass resolves 11 more bits of a 64-bit
// word with one LDS histogram, and the depth is bounded by the word's length
// (six passes; one or two in practice).

// A candidate is the 64-bit word (key << 32) | ~position: a larger word is a
// higher score, or an equal score at a lower position.  Positions ascend with
// block index, so one unsigned compare is the whole output order, ties to the
// lower block index included.
//
// One workgroup of NT threads per (layer, row), m = min(k, admitted):
//  * Usual path: the score kernel left c candidates, every key at or above the
//    row's floor.  If c >= m the best m of the row are among them (at least m
//    keys reach the floor, so the m-th best does, and so do all its ties).  A
//    radix select over the candidate words (in registers when c <= 8192, else
//    re-read from memory on each pass) narrows them to at most m + 64, whose
//    best m are placed in descending order.
//  * Exact fallback (c < m: the floor was set too high): the row is rescored
//    in fp32 over every admitted position, its words replace the candidate
//    list, and the same select runs over all of them.
// The final order: the gathered words are sorted in runs of 64 (one per wave,
// in registers), and each word's place is the number of larger words, found
// by a binary search in every run.
// Output: block indices and fp32 scores (recovered exactly from the keys),
// then padding (-1, -inf) up to k, and the count m.
#include "device_util.h"
#include "dssel_internal.h"

namespace dssel {
namespace {

__device__ __forceinline__ uint64_t pack(uint32_t key, int pos) {
  return ((uint64_t)key << 32) | (uint32_t)~(uint32_t)pos;
}
__device__ __forceinline__ uint32_t key_of(uint64_t e) { return (uint32_t)(e >> 32); }
__device__ __forceinline__ int pos_of(uint64_t e) { return (int)~(uint32_t)e; }

constexpr int kRun = kWave;  // words per sorted run: one per lane of a wave

// One compare-exchange step of a descending bitonic network on element e
// (value v, partner value p): block size k, distance j.
__device__ __forceinline__ uint64_t bitonic_keep(uint64_t v, uint64_t p, int e, int k, int j) {
  const bool desc = (e & k) == 0;
  const bool low = (e & j) == 0;
  return (desc == low) ? (v > p ? v : p) : (v < p ? v : p);
}

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int mask) {
  const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)v, mask, kWave);
  const uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(v >> 32), mask, kWave);
  return ((uint64_t)hi << 32) | lo;
}

// LDS words: the gathered words (at most 2 NT) with a run of zero padding,
// then the best m in order (m <= k <= DS_SEL_MAX_K = 2048).
constexpr int kGatherMax = 2048 + kGatherSlack;  // the most words gathered: k <= 2048, plus slack
constexpr int kGatherCap = (kGatherMax + kRun + 8 * kRun - 1) / (8 * kRun) * (8 * kRun);  // whole groups of 8 runs
constexpr int kOrderedCap = 2048;

// Everything that depends on the workgroup size NT (threads per row).
template <int NT>
struct SelectT {
  static constexpr int kWaves = NT / kWave;

struct Shared {
  uint32_t hist[kHistBins];
  uint64_t se[kGatherCap + kOrderedCap];  // [0, kGatherCap): gathered; then the best m, sorted
  float q[256];
  int scan[kWaves + 1];
  int bin, above, count;
};

// Largest bin B in [0, nbins) with (keys in bins >= B) >= need, and the
// number of keys in bins > B.  nbins is 1024 or 2048; the histogram is in LDS.
static __device__ __forceinline__ void find_boundary(const uint32_t* hist, int nbins, int need, int* out_bin,
                              int* out_above, int* scan_scratch) {
  const int per = (nbins + NT - 1) / NT;  // bins per thread, taken in descending order
  const int hi = nbins - 1 - threadIdx.x * per;  // the last threads may hold fewer (or no) bins
  int mine = 0;
  for (int i = 0; i < per && hi - i >= 0; ++i) mine += (int)hist[hi - i];
  int total = 0;
  const int excl = block_exclusive_scan<NT>(mine, &total, scan_scratch);
  if (excl < need && excl + mine >= need) {
    int above = excl;
    for (int i = 0; i < per && hi - i >= 0; ++i) {
      const int cnt = (int)hist[hi - i];
      if (above + cnt >= need) {
        *out_bin = hi - i;
        *out_above = above;
        break;
      }
      above += cnt;
    }
  }
  __syncthreads();
}

// The best m of the n distinct words se[0, n), in descending order, into
// out[0, min(n, m)).  The words are cut into runs of 64; each wave sorts runs
// in registers (a bitonic network across its lanes), and a word's place is
// the number of larger words, summed over the runs by a binary search in
// each, eight runs at a time with no branch (their loads all in flight).
// se[n, 512 * ceil(n / 512)) must hold zero words, which are never larger
// than a candidate.
static __device__ __forceinline__ void sort_place(uint64_t* se, int n, int m, uint64_t* out) {
  const int tid = threadIdx.x, lane = lane_id(), wave = tid / kWave;
  const int runs = (n + kRun - 1) / kRun;         // <= kGatherCap / 64
  const int runs8 = (runs + 7) / 8 * 8;           // the searches' runs: zero runs past `runs`
  for (int run = wave; run < runs; run += NT / kWave) {
    uint64_t v = se[run * kRun + lane];
    for (int k = 2; k <= kRun; k <<= 1)
      for (int j = k >> 1; j > 0; j >>= 1) v = bitonic_keep(v, shfl_xor_u64(v, j), lane, k, j);
    se[run * kRun + lane] = v;
  }
  __syncthreads();
  for (int idx = tid; idx < runs * kRun; idx += NT) {
    const uint64_t e = se[idx];
    if (e == 0ull) continue;  // padding
    int place = 0;
    for (int r0 = 0; r0 < runs8; r0 += 8) {  // eight runs' searches interleaved
      const uint64_t* base = se + r0 * kRun;
      int cnt[8];
#pragma unroll
      for (int t = 0; t < 8; ++t) cnt[t] = 0;
#pragma unroll
      for (int step = kRun / 2; step > 0; step >>= 1) {
#pragma unroll
        for (int t = 0; t < 8; ++t) cnt[t] += base[t * kRun + cnt[t] + step - 1] > e ? step : 0;
      }
#pragma unroll
      for (int t = 0; t < 8; ++t) place += cnt[t] + (base[t * kRun + cnt[t]] > e ? 1 : 0);
    }
    if (place < m) out[place] = e;
  }
  __syncthreads();
}

// Candidate words held in registers, at most kPer per thread (c <= kSelectBuf).
// The loads do not wait for the count: every slot below min(kSelectBuf, cap)
// lies inside the row's list (which has room for every position), and the
// slots at or past c are simply never used.
struct RegisterWords {
  static constexpr bool kInRegisters = true;
  static constexpr int kPer = (kSelectBuf + NT - 1) / NT;
  uint64_t v[kPer];
  int c = 0;
  // The first half of the slots, before the count is known (the usual lists
  // hold 2,000-4,000 words) ...
  __device__ void load_head(const uint64_t* src, int64_t cap) {
#pragma unroll
    for (int u = 0; u < kPer / 2; ++u) {
      const int i = u * NT + (int)threadIdx.x;
      v[u] = i < cap ? src[i] : 0ull;
    }
#pragma unroll
    for (int u = kPer / 2; u < kPer; ++u) v[u] = 0ull;
  }
  // ... and the rest once it is, only if it needs them.
  __device__ void load_tail(const uint64_t* src, int count) {
    if (count > (kPer / 2) * NT) {
#pragma unroll
      for (int u = kPer / 2; u < kPer; ++u) {
        const int i = u * NT + (int)threadIdx.x;
        v[u] = i < count ? src[i] : 0ull;
      }
    }
  }
  template <class F>
  __device__ __forceinline__ void each(F&& f) const {
#pragma unroll
    for (int u = 0; u < kPer; ++u) f(u * NT + (int)threadIdx.x < c, v[u]);
  }
};

// Candidate words read from global memory on every pass (any count).
struct GlobalWords {
  static constexpr bool kInRegisters = false;
  const uint64_t* p;
  int c;
  template <class F>
  __device__ __forceinline__ void each(F&& f) const {
    for (int i0 = 0; i0 < c; i0 += NT) {  // same trip count in every lane
      const int i = i0 + (int)threadIdx.x;
      const bool valid = i < c;
      f(valid, valid ? p[i] : 0ull);
    }
  }
};

// Best m of c distinct candidate words, sorted descending.  Radix select over
// the 64-bit word, 11 bits per pass from the top: each pass histograms the
// words that share the prefix fixed so far, and the boundary bin extends the
// prefix; the words above the prefix are all selected.  The passes go on
// until the selected words plus those sharing the prefix number at most
// m + kGatherSlack; then they are gathered and ordered.  The words are distinct
// (one per position), so six passes always suffice; on the usual candidate
// lists one or two are needed.
template <class Words>
static __device__ void radix_select_words(const Words& src, int c, int m, Shared& sh) {
  const int tid = threadIdx.x;
  const int gather_max = m + kGatherSlack;  // <= kGatherMax
  int pbits = 0;
  uint64_t prefix = 0;
  int above = 0, in_range = c, need = m;
  while (pbits < 64 && above + in_range > gather_max) {
    const int width = 64 - pbits < kDigit1Bits ? 64 - pbits : kDigit1Bits;
    const int shift = 64 - pbits - width;
    for (int i = tid; i < kHistBins; i += NT) sh.hist[i] = 0u;
    __syncthreads();
    if constexpr (Words::kInRegisters) {
      // The candidates all lie above the row's floor, so the first pass puts
      // nearly all of them in a few bins, where the LDS serialises the atomics:
      // a thread adds its words in the bin of its first one with one atomic.
      uint32_t lead = 0u;
      int nlead = 0;
      src.each([&](bool valid, uint64_t w) {
        if (valid && (pbits == 0 || (w >> (64 - pbits)) == prefix)) {
          const uint32_t b = (uint32_t)(w >> shift) & ((1u << width) - 1u);
          if (nlead == 0) lead = b;
          if (nlead == 0 || b == lead) ++nlead;
          else atomicAdd(&sh.hist[b], 1u);
        }
      });
      if (nlead > 0) atomicAdd(&sh.hist[lead], (uint32_t)nlead);
    } else {
      src.each([&](bool valid, uint64_t w) {
        if (valid && (pbits == 0 || (w >> (64 - pbits)) == prefix))
          atomicAdd(&sh.hist[(uint32_t)(w >> shift) & ((1u << width) - 1u)], 1u);
      });
    }
    __syncthreads();
    find_boundary(sh.hist, kHistBins, need, &sh.bin, &sh.above, sh.scan);
    const int bin = sh.bin;
    above += sh.above;
    need -= sh.above;
    in_range = (int)sh.hist[bin];
    prefix = (prefix << width) | (uint64_t)bin;
    pbits += width;
    __syncthreads();  // hist, bin and above are read before the next pass resets them
  }
  if (tid == 0) sh.count = 0;
  __syncthreads();
  const uint64_t lower = pbits == 0 ? 0ull : prefix << (64 - pbits);
  src.each([&](bool valid, uint64_t w) {
    const bool want = valid && w >= lower;
    const int slot = wave_append(want, &sh.count);
    if (want && slot < kGatherCap) sh.se[slot] = w;
  });
  int gathered = above + in_range;  // <= gather_max <= kGatherMax
  gathered = gathered < kGatherMax ? gathered : kGatherMax;
  const int padded = (gathered + 8 * kRun - 1) / (8 * kRun) * (8 * kRun);  // <= kGatherCap
  for (int i = gathered + tid; i < padded; i += NT) sh.se[i] = 0ull;
  __syncthreads();
  sort_place(sh.se, gathered, m, sh.se + kGatherCap);
}

// Exact fallback: the floor let fewer than m keys through, so row (l, r) is
// rescored in fp32 over every admitted position and its words replace the
// candidate list.
static __device__ int rescore_row(const Call& c, int l, int r, uint64_t* words, Shared& sh) {
  const int tid = threadIdx.x;
  const int R = c.rows, D = c.dim;
  const int64_t N = c.blocks, lr = (int64_t)l * R + r;
  const int P = c.mode == kRowMask ? c.counts[(int64_t)l * kCountStride + kMaxRows]
                                   : c.counts[(int64_t)l * kCountStride + r];
  const int32_t* list = c.list + (int64_t)l * N;
  const uint16_t* K = c.keys ? c.keys + (int64_t)l * c.key_layer_stride : nullptr;
  int64_t lim = c.limit ? (int64_t)c.limit[lr] : N;
  lim = lim < 0 ? 0 : (lim > N ? N : lim);
  const uint32_t* mrow =
      c.mode == kRowMask ? c.mask + (int64_t)l * c.mask_layer_stride + r * c.mask_row_stride : nullptr;

  for (int i = tid; i < D; i += NT) sh.q[i] = c.qt[lr * D + i];
  if (tid == 0) sh.count = 0;
  __syncthreads();
  for (int p0 = 0; p0 < P; p0 += NT) {
    const int p = p0 + tid;
    bool adm = p < P;
    int b = 0;
    if (adm) {
      b = c.mode == kNoMask ? p : list[p];
      if (mrow) adm = ((mrow[b >> 5] >> (b & 31)) & 1u) && (int64_t)b < lim;
    }
    uint64_t w = 0;
    if (adm && c.score_kind == kScoreHeadRelu) {
      // per-head ReLU: every head's dot product against the bf16 key row,
      // clamped at zero and weighted, heads in ascending order
      const int H = c.heads;
      const uint16_t* krow = K + (int64_t)b * c.ldk;
      const uint16_t* qrow = c.q + lr * H * D;
      const uint16_t* wrow = c.w + lr * H;
      float s = 0.0f;
      for (int h = 0; h < H; ++h) {
        float dot = 0.0f;
        for (int i = 0; i < D; i += 8) {
          const uint4 kv = *reinterpret_cast<const uint4*>(krow + i);
          const uint4 qv = *reinterpret_cast<const uint4*>(qrow + (int64_t)h * D + i);
          const uint32_t k4[4] = {kv.x, kv.y, kv.z, kv.w}, q4[4] = {qv.x, qv.y, qv.z, qv.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            dot = fmaf(bf16_lo(q4[e]), bf16_lo(k4[e]), dot);
            dot = fmaf(bf16_hi(q4[e]), bf16_hi(k4[e]), dot);
          }
        }
        s += bf16_to_f32(wrow[h]) * fmaxf(dot, 0.0f);
      }
      w = pack(score_to_key(s), p);
    } else if (adm && c.fmt == kKeysQ8) {
      // 8-bit keys: per 32-column group, sum q~_i c_i, then add scale times that
      const int8_t* crow = c.codes + (int64_t)l * c.code_layer_stride + (int64_t)b * c.ldc;
      const uint16_t* srow = c.scales + (int64_t)l * c.scale_layer_stride + (int64_t)b * c.lds;
      float dot = 0.0f;
      for (int g = 0; g < D / 32; ++g) {
        float t = 0.0f;
        for (int i = 0; i < 32; ++i) t = fmaf(sh.q[32 * g + i], (float)crow[32 * g + i], t);
        dot += half_bits_to_f32(srow[g]) * t;
      }
      w = pack(score_to_key(dot), p);
    } else if (adm) {
      const uint16_t* krow = K + (int64_t)b * c.ldk;
      float dot = 0.0f;
      for (int i = 0; i < D; i += 8) {
        const uint4 v = *reinterpret_cast<const uint4*>(krow + i);
        const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          dot = fmaf(sh.q[i + 2 * e], bf16_lo(w4[e]), dot);
          dot = fmaf(sh.q[i + 2 * e + 1], bf16_hi(w4[e]), dot);
        }
      }
      w = pack(score_to_key(dot), p);
    }
    const int slot = wave_append(adm, &sh.count);
    if (adm) words[slot] = w;
  }
  __syncthreads();  // the words are read back by other threads of the workgroup
  return sh.count;
}

static __device__ void run(const Call& c, Shared& sh) {
  const int l = blockIdx.y, r = blockIdx.x;
  const int R = c.rows, k = c.k;
  const int64_t lr = (int64_t)l * R + r;
  const int64_t N = c.blocks;
  // One round of independent loads: the counts and the candidate words.
  const int32_t* cnt_l = c.counts + (int64_t)l * kCountStride;
  const int n_adm = cnt_l[r];
  const int n_union = cnt_l[kMaxRows];
  int cands = c.cand_count[lr * kCountPad];
  uint64_t* words = c.cand + lr * c.cand_stride;
  RegisterWords rw;
  rw.load_head(words, c.cand_stride);
  const int m = n_adm < k ? n_adm : k;
  const int P = c.mode == kRowMask ? n_union : n_adm;
  int32_t* oi = c.out_idx + lr * k;
  float* os = c.out_score + lr * k;
  const int tid = threadIdx.x;

  if (m > 0) {
    if (cands < m) {
      cands = rescore_row(c, l, r, words, sh);
      rw.load_head(words, c.cand_stride);
    }
    if (cands <= kSelectBuf) {
      rw.load_tail(words, cands);
      rw.c = cands;
      radix_select_words(rw, cands, m, sh);
    } else {
      radix_select_words(GlobalWords{words, cands}, cands, m, sh);
    }
  }

  const int32_t* list = c.list + (int64_t)l * N;
  for (int j = tid; j < k; j += NT) {
    if (j < m) {
      const uint64_t e = sh.se[kGatherCap + j];
      int p = pos_of(e);
      p = p < 0 ? 0 : (p >= P ? P - 1 : p);  // in range by construction; never index past it
      oi[j] = (c.mode == kNoMask) ? p : list[p];
      os[j] = key_to_score(key_of(e));
    } else {
      oi[j] = -1;
      os[j] = -__builtin_inff();
    }
  }
  if (tid == 0 && c.out_count) c.out_count[lr] = m;
}

};

template <int NT>
__global__ __launch_bounds__(NT) void select_kernel(Call c) {
  __shared__ typename SelectT<NT>::Shared sh;
  SelectT<NT>::run(c, sh);
}

}  // namespace

hipError_t launch_select(const Call& c, hipStream_t stream) {
  // One workgroup per (layer, row).  A 1,024-thread workgroup is fastest for a
  // row, but only one is resident per compute unit (its waves hold more than
  // 80 SGPRs); when the rows outnumber the compute units, 768-thread
  // workgroups (three waves per SIMD, two per unit) keep every row in one
  // round.
  const int64_t rows = (int64_t)c.layers * c.rows;
  const int64_t cus = c.score_slots / kScoreWgsPerCu;
  dim3 grid(c.rows, c.layers);
  if (rows > cus)
    hipLaunchKernelGGL(select_kernel<768>, grid, dim3(768), 0, stream, c);
  else
    hipLaunchKernelGGL(select_kernel<1024>, grid, dim3(1024), 0, stream, c);
  return hipGetLastError();
}

}  // namespace dssel
