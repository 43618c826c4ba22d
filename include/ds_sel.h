/*
 * ds_sel.h -- compressed-attention block selection on AMD MI355X (gfx950).
 *
 * The operation (page "DeepSeek V4.1F Q4 on M3 Ultra with native DSpark MTP
 * (40tps / 800tps)", paragraph "Decode at depth"; restated on page "DeepSeek
 * V4.1 Flash on M3 Ultra nearly doubles decode to 31 t/s with first public
 * DSpark Metal port", paragraph "Key techniques"): in every layer the
 * compressed attention keeps k = 512 compressed blocks chosen from the whole
 * context.  Only blocks that a row's admission mask lets through are scored,
 * the admitted index is compacted once per row, and the best k are taken with
 * a radix select whose number of passes is bounded.  With the speculative
 * drafter on, one decode step verifies several query rows that share one
 * stream of data (same page, paragraph "DSpark"); here the rows of one layer
 * share one pass over the block keys.
 *
 * The pages give no formula.  This library defines, for layer l, row r and
 * block b (readings of this library):
 *
 *   admitted(l,r,b) = (mask == NULL or bit b of the (l,r) mask row is 1)
 *                     and b < clamp(limit[l][r], 0, N)     (limit NULL -> N)
 *   score(l,r,b)    = sum_h w[l][r][h] * (q[l][r][h][:] . K[l][b][:])
 *                     with bf16 inputs and fp32 accumulation
 *   order           = higher score first; equal scores -> lower block index
 *   result(l,r)     = the first m = min(k, #admitted) blocks in that order,
 *                     then k - m padding entries (index -1, score -inf);
 *                     count = m.
 *
 * The GPU evaluates the score as (sum_h w_h q_h) . K_b in fp32 (the sum is
 * linear, so folding the heads first is the same sum).  On inputs whose bf16
 * values are small integers every partial sum is exact and the result is
 * bit-identical to any other fp32 evaluation order; on general inputs scores
 * differ from a per-head evaluation only by fp32 rounding.  The order is taken
 * on the GPU's own fp32 scores, so the output is always consistent with the
 * scores it returns.
 *
 * Conventions for every entry point:
 *   - Integer status codes, 0 = success; no exceptions or longjmps cross the
 *     ABI.  ds_sel_status_string() names a code.
 *   - Argument, alignment and capacity checks run on the host before anything
 *     is enqueued; on DS_SEL_E_INVALID, DS_SEL_E_UNSUPPORTED or
 *     DS_SEL_E_CAPACITY nothing runs and the outputs are untouched.
 *   - All data pointers in ds_sel_args are DEVICE pointers on the handle's
 *     device, owned by the caller.  The library keeps none of them after the
 *     enqueued work completes.
 */
#ifndef DS_SEL_H
#define DS_SEL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  DS_SEL_OK = 0,
  DS_SEL_E_INVALID = 1,     /* bad argument: null, negative, misaligned, inconsistent */
  DS_SEL_E_CAPACITY = 2,    /* exceeds the capacity declared at ds_sel_create */
  DS_SEL_E_NODEVICE = 3,    /* no HIP device, or the ordinal does not exist */
  DS_SEL_E_HIP = 4,         /* a HIP runtime call or launch failed */
  DS_SEL_E_NOMEM = 5,       /* device or host allocation failed */
  DS_SEL_E_UNSUPPORTED = 6  /* valid but not built: dim outside {32, 64, 128, 256} */
};

/* Hard limits of this build (a capacity above them is DS_SEL_E_INVALID). */
#define DS_SEL_MAX_ROWS 8
#define DS_SEL_MAX_K 2048
#define DS_SEL_MAX_HEADS 1024
#define DS_SEL_MAX_DIM 256
#define DS_SEL_MAX_BLOCKS (1LL << 26)

/* Create-time flags.  The default key-stream engine feeds the bf16 keys to the
 * matrix cores (the fp32 folded query enters as three bf16 parts, whose sum
 * is the query exactly for |q~_i| >= 2^-110 and within 2^-133 below that);
 * DS_SEL_FLAG_VALU_SCORE selects fp32 FMAs on the vector ALUs instead.  Both
 * return the same selection on integer-valued inputs; on general inputs their
 * scores differ only by fp32 rounding order. */
#define DS_SEL_FLAG_VALU_SCORE 1u

/* The per-head ReLU score, a non-linear variant of the block score (the pages
 * give no formula: page "DeepSeek V4.1F Q4 on M3 Ultra with native DSpark MTP
 * (40tps / 800tps)", paragraph "Decode at depth"):
 *   score(b) = sum_h w[h] * max(q[h] . K[b], 0)     bf16 inputs, fp32 sums
 * The heads no longer fold into one query vector, so every (row, head) pair
 * meets every admitted key on the matrix cores (R x H x d multiply-adds per
 * block).  Admission, order, output and padding are unchanged.  A handle
 * created with this flag scores every call this way.  Supported with bf16
 * keys and the default engine, when one layer's heads fit the kernel's LDS
 * stage: R * ceil16(H) * (2 (d + 8) + 4) bytes <= 122,864 (e.g. R <= 6 at
 * H = 64, d = 128); otherwise a call returns DS_SEL_E_UNSUPPORTED. */
#define DS_SEL_FLAG_HEAD_RELU 2u

typedef struct ds_sel ds_sel; /* opaque handle; owns device scratch */

/* Create-time capacity.  Every call on the handle must fit inside it. */
typedef struct {
  uint32_t struct_size; /* sizeof(ds_sel_limits) */
  int32_t device;       /* HIP device ordinal the handle lives on */
  int32_t max_layers;   /* >= 1 */
  int32_t max_rows;     /* 1 .. DS_SEL_MAX_ROWS */
  int32_t max_heads;    /* 1 .. DS_SEL_MAX_HEADS */
  int32_t max_dim;      /* 1 .. DS_SEL_MAX_DIM */
  int32_t max_k;        /* 1 .. DS_SEL_MAX_K */
  int32_t flags;        /* 0, or DS_SEL_FLAG_* bits */
  int64_t max_blocks;   /* 0 .. DS_SEL_MAX_BLOCKS */
} ds_sel_limits;

/* One call: `layers` independent selection problems, each with `rows` query
 * rows that share the layer's block keys.  Element strides, not bytes. */
typedef struct {
  uint32_t struct_size; /* sizeof(ds_sel_args) */
  int32_t layers;       /* L >= 1 */
  int32_t rows;         /* R, 1 .. DS_SEL_MAX_ROWS */
  int32_t heads;        /* H >= 1 */
  int32_t dim;          /* d in {32, 64, 128, 256} */
  int32_t k;            /* 1 .. max_k; k > #admitted is allowed (padding) */
  int64_t blocks;       /* N >= 0 */
  const void* q;        /* bf16 [L][R][H][d], contiguous, 16-byte aligned */
  const void* w;        /* bf16 [L][R][H], contiguous */
  const void* keys;     /* bf16; block b of layer l at keys + l*key_layer_stride + b*ldk;
                           16-byte aligned; may be NULL only when N == 0 */
  int64_t ldk;          /* >= d, multiple of 8 */
  int64_t key_layer_stride; /* multiple of 8; >= N*ldk when L > 1 */
  const uint32_t* mask; /* NULL (admit all), or words; the (l,r) row starts at
                           mask + l*mask_layer_stride + r*mask_row_stride; bit b%32 of
                           word b/32 (LSB first); bits at b >= N are ignored */
  int64_t mask_row_stride;   /* 0 = one row shared by all rows of a layer, else >= ceil(N/32) */
  int64_t mask_layer_stride; /* >= (R-1)*mask_row_stride + ceil(N/32) when L > 1 */
  const int32_t* limit; /* NULL (limit N), or int32 [L][R]; admitted iff b < limit, and the
                           value is clamped to [0, N] on the device */
  int32_t* out_idx;     /* int32 [L][R][k] */
  float* out_score;     /* float [L][R][k] */
  int32_t* out_count;   /* int32 [L][R], or NULL */
} ds_sel_args;

/* Create a handle on lim->device with scratch for the declared capacity.
 * Returns DS_SEL_E_NODEVICE when there is no HIP device (also on a host with
 * no GPU at all), DS_SEL_E_INVALID for a bad capacity, DS_SEL_E_NOMEM when
 * the scratch cannot be allocated.  On success *out owns the handle. */
int ds_sel_create(const ds_sel_limits* lim, ds_sel** out);

/* Enqueue the whole chain for one call on `hip_stream` (a hipStream_t on the
 * handle's device; NULL = the null stream) and return without waiting.  The
 * outputs are valid once the stream reaches this point; inputs must not change
 * before then.  Calls on one handle must be ordered on one stream (they reuse
 * its scratch); the handle is not thread-safe.  DS_SEL_E_HIP means a launch
 * failed: outputs are undefined and the handle stays usable. */
int ds_sel_score_select(ds_sel* h, const ds_sel_args* a, void* hip_stream);

/* The same work as ds_sel_score_select, plus a per-dispatch ledger: the
 * four caller-created hipEvent_t in `events` are recorded on `hip_stream`
 * before the first kernel and after each of the three (prep, score, select),
 * so hipEventElapsedTime between consecutive events gives each kernel's
 * device time.  Same status codes; on an argument error no event is recorded.
 * (The pages keep a per-dispatch bandwidth ledger for the same purpose: page
 * "DeepSeek V4.1F Q4 on M3 Ultra with native DSpark MTP (40tps / 800tps)",
 * the paragraph listing what else the repository holds.) */
int ds_sel_score_select_profiled(ds_sel* h, const ds_sel_args* a, void* hip_stream,
                                 void* const events[4]);

/* The same selection as ds_sel_score_select, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  No handle is needed and nothing is
 * allocated: the chain's scratch is a static device array of 64 MiB inside the
 * library, one per GPU, held until the process ends.  `device` is the HIP
 * ordinal the pointers in `a` live on; `flags` takes DS_SEL_FLAG_* as
 * ds_sel_limits.flags does.  The arguments are checked as for
 * ds_sel_score_select against this build's hard limits; a call whose scratch
 * (ds_sel_noalloc_scratch_bytes) exceeds 64 MiB returns DS_SEL_E_CAPACITY and
 * enqueues nothing.  Every call on one GPU uses that GPU's one array, so calls
 * that overlap in time on one GPU (different streams, or different host
 * threads) race and give undefined results; calls ordered on one stream are
 * safe.  DS_SEL_E_NODEVICE when `device` does not exist. */
int ds_sel_score_select_noalloc(int32_t device, uint32_t flags, const ds_sel_args* a,
                                void* hip_stream);

/* Bytes of the static scratch ds_sel_score_select_noalloc needs for the call
 * `a` (-1 when a's sizes are invalid). */
int64_t ds_sel_noalloc_scratch_bytes(const ds_sel_args* a);

/* The 8-bit key stream (page "DeepSeek V4.1F Q4 on M3 Ultra with native
 * DSpark MTP (40tps / 800tps)", paragraph "DSpark": the repository's kernels
 * stream 8-bit weights in groups; this library reads that layout for the
 * block keys).  Each key row of d values is cut into d/32 groups of 32; group
 * g of block b holds 32 int8 codes c_i and one fp16 scale s, and stands for
 * the values s * c_i.  The selection is the one ds_sel_score_select defines,
 * with K[l][b][32 g + i] = s * c_i in place of the bf16 key; the block score
 * is summed per group in fp32 and each group's sum multiplied by s (the
 * folded query, weights and tie rule are unchanged).  Element strides. */
typedef struct {
  uint32_t struct_size;       /* sizeof(ds_sel_q8_keys) */
  int32_t reserved;           /* 0 */
  const int8_t* codes;        /* int8; block b of layer l at codes + l*code_layer_stride + b*ldc;
                                 8-byte aligned; may be NULL only when N == 0 */
  int64_t ldc;                /* >= d, multiple of 8 */
  int64_t code_layer_stride;  /* multiple of 8; >= N*ldc when L > 1 */
  const uint16_t* scales;     /* fp16 bits; block b of layer l at scales + l*scale_layer_stride
                                 + b*lds, d/32 of them; may be NULL only when N == 0 */
  int64_t lds;                /* >= d/32 */
  int64_t scale_layer_stride; /* >= N*lds when L > 1 */
} ds_sel_q8_keys;

/* ds_sel_score_select over the 8-bit key stream `k8`; a->keys must be NULL
 * (the keys come from k8), everything else of `a` and every rule of
 * ds_sel_score_select (handle, stream, status codes) applies unchanged.
 * `events` is NULL, or four hipEvent_t recorded as ds_sel_score_select_profiled
 * records them. */
int ds_sel_score_select_q8(ds_sel* h, const ds_sel_args* a, const ds_sel_q8_keys* k8,
                           void* hip_stream, void* const events[4]);

/* The host-side checks ds_sel_score_select_q8 applies, without a device. */
int ds_sel_check_args_q8(const ds_sel_limits* lim, const ds_sel_args* a, const ds_sel_q8_keys* k8);

/* Quantise bf16 keys into the 8-bit key stream, per group of 32 values x_i
 * with m = max |x_i|: s = the fp32 quotient m / 127 (correctly rounded),
 * rounded to fp16 to nearest even; c_i = the fp32 quotient x_i / s rounded
 * half away from zero and clamped to [-127, 127]; a group whose s is 0 (m = 0,
 * or m / 127 below half the least fp16 subnormal) gets s = +0 and codes 0.
 * The keys must be finite with |x| <= 127 * 65504 (larger ones give an
 * infinite scale, which ds_sel_score_select_q8 does not accept).  Asynchronous
 * on `hip_stream` on the current device; no handle.  DS_SEL_E_INVALID for bad
 * sizes, strides or alignment. */
typedef struct {
  uint32_t struct_size;       /* sizeof(ds_sel_quantize_args) */
  int32_t layers;             /* L >= 1 */
  int32_t dim;                /* d in {32, 64, 128, 256} */
  int32_t reserved;           /* 0 */
  int64_t blocks;             /* N, 0 .. DS_SEL_MAX_BLOCKS */
  const void* keys;           /* bf16, as in ds_sel_args (16-byte aligned, ldk multiple of 8) */
  int64_t ldk, key_layer_stride;
  int8_t* codes;              /* 16-byte aligned; ldc >= d and code_layer_stride both multiples of 16 */
  int64_t ldc, code_layer_stride;
  uint16_t* scales;           /* 2-byte aligned; lds >= d/32 */
  int64_t lds, scale_layer_stride;
} ds_sel_quantize_args;

int ds_sel_quantize_q8(const ds_sel_quantize_args* a, void* hip_stream);

/* Serial decode: the layers of `a` one after another, each layer's query
 * depending on the previous layer's selection (page "DeepSeek V4.1F Q4 on M3
 * Ultra with native DSpark MTP (40tps / 800tps)", paragraph "Decode": the
 * layers run one after another and the per-dispatch cost is what to remove).
 * The model that links real layers is outside this library; its stand-in is
 * a rotation of the next layer's query heads by this layer's best block:
 *   layer 0 selects with q[0]; for l >= 1, row r selects with
 *   q_l[r][h] = q[l][r][(h + s) mod H],  s = idx[l-1][r][0] mod H
 *   (s = 0 when layer l-1 selected nothing for the row, idx -1).
 * `a` is an ordinary call over L layers (same rules and capacity checks);
 * q_work is caller-owned device memory, bf16 [L][R][H][d], 16-byte aligned
 * (may be NULL when L == 1): layer l >= 1's rotated query is written to its
 * slot l and read from there; slot 0 is not touched.  Outputs are those of
 * ds_sel_score_select for every layer.  Enqueued on `hip_stream` as 4 L - 1
 * launches (the chain's three per layer and the rotation between layers). */
int ds_sel_decode(ds_sel* h, const ds_sel_args* a, void* q_work, void* hip_stream);

/* The same serial decode captured once into a HIP graph, so that a decode
 * step is one graph launch instead of 4 L - 1 kernel launches.  The plan
 * records the pointers of `a` and q_work and the handle's scratch: the caller
 * keeps them alive and unchanged in place (their contents may change between
 * launches: every launch reads them afresh), and destroys the plan before the
 * handle.  `hip_stream` must be a created stream (the legacy null stream
 * cannot be captured); nothing is executed at create.  Launches on one plan,
 * and calls on its handle, must be ordered on one stream.
 * DS_SEL_E_HIP when capture or instantiation fails (no plan is returned). */
typedef struct ds_sel_plan ds_sel_plan;
int ds_sel_decode_plan_create(ds_sel* h, const ds_sel_args* a, void* q_work, void* hip_stream,
                              ds_sel_plan** out);
int ds_sel_decode_plan_launch(ds_sel_plan* p, void* hip_stream);
void ds_sel_decode_plan_destroy(ds_sel_plan* p);  /* NULL is a no-op */

/* Attention over a selection -- the step that consumes it (page "DeepSeek
 * V4.1F Q4 on M3 Ultra with native DSpark MTP (40tps / 800tps)", paragraph
 * "Decode at depth": each layer's compressed attention works on the blocks
 * the selection keeps; paragraph "Prefill": the attention core).  The pages
 * give no formula.  This library defines, for layer l, row r and attention
 * head h, with c = clamp(count[l][r], 0, k) (count NULL -> k) and S the slots
 * j < c whose index idx[l][r][j] lies in [0, N):
 *
 *   s_j        = scale * (q[l][r][h][:] . K[l][idx_j][:])   bf16 inputs, fp32 sums
 *   out[l][r][h] = sum_{j in S} exp(s_j - max s) V[l][idx_j] / sum_{j in S} exp(s_j - max s)
 *
 * and out = 0 when S is empty.  Slots outside S are skipped, never read: the
 * padding (-1) that ds_sel_score_select writes past its count is one such
 * slot, so its outputs can be passed here unchanged.  The weights are carried
 * to about 2^-17 relative; everything else is fp32.  Element strides. */
typedef struct {
  uint32_t struct_size; /* sizeof(ds_sel_attend_args) */
  int32_t layers;       /* L >= 1 */
  int32_t rows;         /* R, 1 .. DS_SEL_MAX_ROWS */
  int32_t heads;        /* attention heads Ha, 1 .. DS_SEL_MAX_HEADS */
  int32_t dim;          /* d in {32, 64, 128, 256} */
  int32_t k;            /* slots per (l, r) in idx, 1 .. max_k */
  float scale;          /* finite; 1/sqrt(d) is the usual choice */
  int32_t reserved;     /* 0 */
  int64_t blocks;       /* N >= 0: indices at or above N are skipped */
  const void* q;        /* bf16 [L][R][Ha][d], contiguous, 16-byte aligned */
  const void* keys;     /* bf16; block b of layer l at keys + l*key_layer_stride + b*ldk;
                           16-byte aligned; may be NULL only when N == 0 */
  int64_t ldk;          /* >= d, multiple of 8 */
  int64_t key_layer_stride; /* multiple of 8; >= N*ldk when L > 1 */
  const void* values;   /* bf16, laid out like keys with ldv and value_layer_stride */
  int64_t ldv;          /* >= d, multiple of 8 */
  int64_t value_layer_stride; /* multiple of 8; >= N*ldv when L > 1 */
  const int32_t* idx;   /* int32 [L][R][k] */
  const int32_t* count; /* int32 [L][R], or NULL (all k slots) */
  float* out;           /* fp32 [L][R][Ha][d] */
} ds_sel_attend_args;

/* Enqueue attention over a selection on `hip_stream`, as ds_sel_score_select
 * does (same handle, stream rules and status codes).  The handle's capacity
 * bounds layers, rows, heads (attention heads here), dim, k and blocks.  When
 * few (layer, row) pairs are given, each pair's selection is split across
 * several workgroups, whose partial results sit in the handle's scratch and
 * are merged by a second kernel. */
int ds_sel_attend(ds_sel* h, const ds_sel_attend_args* a, void* hip_stream);

/* The host-side checks ds_sel_attend applies, without a device. */
int ds_sel_check_attend_args(const ds_sel_limits* lim, const ds_sel_attend_args* a);

/* Calibration launches: the floors and ceilings the chain is measured
 * against (the pages keep a per-dispatch bandwidth ledger for the same
 * purpose: page "DeepSeek V4.1F Q4 on M3 Ultra with native DSpark MTP (40tps
 * / 800tps)", the paragraph listing what else the repository holds).  None
 * computes anything of the selection; each XOR-folds what it reads into
 * sink[workgroup] so that no load is dropped.
 *   DS_SEL_CALIB_EMPTY   an empty kernel on `workgroups` workgroups of 256 threads;
 *   DS_SEL_CALIB_READ    reads every key row [0, N) x [0, dim) of every layer
 *                        with 16-byte loads; the rows must be packed
 *                        (ldk == dim, and key_layer_stride == N * dim when L > 1);
 *   DS_SEL_CALIB_GATHER  reads exactly the key rows whose bit is set in the
 *                        layer's mask row (all rows when mask is NULL), with the
 *                        addressing the key stream uses; workgroup g takes the
 *                        flattened (layer * N + block) range [ranges[g],
 *                        ranges[g + 1]), whose in-layer starts must be multiples
 *                        of 32 (DS_SEL_E_INVALID is not checked for this: the
 *                        ranges live in device memory).
 * Asynchronous on `hip_stream` on the current device; sink is device memory of
 * at least `workgroups` words, ranges of workgroups + 1 int64 (gather only). */
#define DS_SEL_CALIB_EMPTY 0
#define DS_SEL_CALIB_READ 1
#define DS_SEL_CALIB_GATHER 2

typedef struct {
  uint32_t struct_size;      /* sizeof(ds_sel_calib_args) */
  int32_t kind;              /* DS_SEL_CALIB_* */
  int32_t workgroups;        /* 1 .. 65535 */
  int32_t layers;            /* L >= 1 (read, gather) */
  int32_t dim;               /* d in {32, 64, 128, 256} (read, gather) */
  int32_t reserved;          /* 0 */
  int64_t blocks;            /* N >= 1 (read, gather) */
  const void* keys;          /* bf16, as in ds_sel_args */
  int64_t ldk, key_layer_stride;
  const uint32_t* mask;      /* gather: NULL, or one row of ceil(N/32) words per layer */
  int64_t mask_layer_stride; /* words */
  const int64_t* ranges;     /* gather: int64 [workgroups + 1], device memory */
  uint32_t* sink;            /* uint32 [workgroups], device memory */
} ds_sel_calib_args;

int ds_sel_calibrate(const ds_sel_calib_args* a, void* hip_stream);

/* Fill every byte of the handle's scratch with `byte` (0..255), enqueued on
 * `hip_stream` like a call.  For tests that check that no call depends on
 * what an earlier call left in the scratch; it uses hipMemsetAsync, so keep it
 * out of captured graphs.  DS_SEL_E_INVALID for a NULL handle or a byte out
 * of range. */
int ds_sel_poison_scratch(ds_sel* h, int32_t byte, void* hip_stream);

/* Free the handle and its scratch, after waiting for the handle's last
 * enqueued call to finish (only that work: other streams and handles are not
 * waited for).  Work captured into a graph is not tracked: a caller that
 * replays such a graph must finish its replays before destroying the handle.
 * NULL is a no-op. */
void ds_sel_destroy(ds_sel* h);

/* The host-side checks ds_sel_score_select applies, without a device:
 * DS_SEL_OK if `a` is acceptable for a handle created with `lim`.  Pointer
 * values are only checked for NULL and alignment, never dereferenced. */
int ds_sel_check_args(const ds_sel_limits* lim, const ds_sel_args* a);

/* Bytes of device scratch a handle with capacity `lim` allocates (0 on a bad
 * capacity).  With L, R, D, N the capacity's layers, rows, dim and blocks and
 * each part rounded up to 256 bytes: the folded query (L R D fp32), its three
 * bf16 parts (3 L R D), the compacted admitted index (L N int32), per-layer
 * counts (9 L int32), candidate floors (L R uint32), candidate counters one
 * per 128 bytes (32 L R int32), candidate lists with room for every
 * position (L R ceil4(N) uint64), and the attention's split records
 * (512 records of 64 heads, each a max and a sum plus D fp32). */
int64_t ds_sel_scratch_bytes(const ds_sel_limits* lim);

/* A static string naming a status code. */
const char* ds_sel_status_string(int status);

#ifdef __cplusplus
}
#endif
#endif /* DS_SEL_H */
