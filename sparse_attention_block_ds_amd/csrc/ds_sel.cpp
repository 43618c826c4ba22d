// libdssel host side: the C ABI of include/ds_sel.h.  Validates every call on
// the host, owns the device scratch, and enqueues the three kernels (prep ->
// score -> select) on the caller's stream without synchronising.
#include <hip/hip_runtime.h>

#include <cmath>
#include <mutex>
#include <new>

#include "ds_sel.h"
#include "dssel_internal.h"


// The select orders at most 2048 winners per row in LDS.
static_assert(DS_SEL_MAX_K <= 2048, "select kernel LDS sized for k <= 2048");
static_assert(DS_SEL_MAX_K <= dssel::kAttendMaxK, "attention kernel LDS sized for k <= kAttendMaxK");
static_assert(DS_SEL_MAX_DIM <= 256, "attention kernels built for d <= 256");
static_assert(DS_SEL_MAX_BLOCKS <= (1LL << dssel::kPositionBits),
              "the score kernel tags staged positions with their row above bit 26");

namespace {

constexpr int64_t kAlign = 256;

int64_t align_up(int64_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

struct Layout {
  int64_t qt, qparts, list, counts, floor, ccount, cand, part_ml, part_o, total;
};

// Scratch for a capacity: q~ fp32 [L][R][d] and its bf16 parts [L][3][R][d],
// compacted index int32 [L][N], counts int32 [L][9], candidate floors uint32
// [L][R], candidate counts int32 [L][R] (one per 128 bytes), and candidate words uint64
// [L][R][N rounded up to 4] (room for every position, so none is ever dropped);
// then the attention's split records: (max, sum) and o[d] fp32 per head of a
// 64-head tile, for at most kAttendPartialWgs workgroups.
Layout layout_for(const ds_sel_limits& lim, bool with_attend = true) {
  Layout s{};
  const int64_t L = lim.max_layers, R = lim.max_rows, D = lim.max_dim, N = lim.max_blocks;
  int64_t off = 0;
  s.qt = off;     off += align_up(L * R * D * 4);
  s.qparts = off; off += align_up(L * 3 * R * D * 2);
  s.list = off;   off += align_up(L * N * 4);
  s.counts = off; off += align_up(L * dssel::kCountStride * 4);
  s.floor = off;  off += align_up(L * R * 4);
  s.ccount = off; off += align_up(L * R * dssel::kCountPad * 4);
  s.cand = off;   off += align_up(L * R * ((N + 3) / 4 * 4) * 8);
  if (with_attend) {
    const int64_t recs = (int64_t)dssel::kAttendPartialWgs * dssel::kAttendHeadTile;
    s.part_ml = off; off += align_up(recs * 2 * 4);
    s.part_o = off;  off += align_up(recs * D * 4);
  }
  s.total = off;
  return s;
}

}  // namespace

struct ds_sel {
  ds_sel_limits lim;
  void* scratch = nullptr;
  int compute_units = 256;  // of the handle's device, read at create
  Layout lay{};             // offsets of the scratch parts
  hipEvent_t done = nullptr;  // recorded after each call's last launch (destroy waits on it)
};

namespace {

constexpr int32_t kKnownFlags = DS_SEL_FLAG_VALU_SCORE | DS_SEL_FLAG_HEAD_RELU;

int check_limits(const ds_sel_limits* lim) {
  if (!lim || lim->struct_size != sizeof(ds_sel_limits)) return DS_SEL_E_INVALID;
  if (lim->max_layers < 1 || lim->max_layers > 65535) return DS_SEL_E_INVALID;
  if (lim->max_rows < 1 || lim->max_rows > DS_SEL_MAX_ROWS) return DS_SEL_E_INVALID;
  if (lim->max_heads < 1 || lim->max_heads > DS_SEL_MAX_HEADS) return DS_SEL_E_INVALID;
  if (lim->max_dim < 1 || lim->max_dim > DS_SEL_MAX_DIM) return DS_SEL_E_INVALID;
  if (lim->max_k < 1 || lim->max_k > DS_SEL_MAX_K) return DS_SEL_E_INVALID;
  if (lim->max_blocks < 0 || lim->max_blocks > DS_SEL_MAX_BLOCKS) return DS_SEL_E_INVALID;
  if ((lim->flags & ~kKnownFlags) != 0 || lim->device < 0) return DS_SEL_E_INVALID;
  return DS_SEL_OK;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int check_q8_keys(const ds_sel_args* a, const ds_sel_q8_keys* k8);

int check_args(const ds_sel_limits& lim, const ds_sel_args* a, const ds_sel_q8_keys* k8 = nullptr) {
  if (!a || a->struct_size != sizeof(ds_sel_args)) return DS_SEL_E_INVALID;
  if (a->layers < 1 || a->rows < 1 || a->heads < 1 || a->dim < 1 || a->k < 1 || a->blocks < 0)
    return DS_SEL_E_INVALID;
  if (a->rows > DS_SEL_MAX_ROWS || a->k > DS_SEL_MAX_K || a->heads > DS_SEL_MAX_HEADS ||
      a->blocks > DS_SEL_MAX_BLOCKS)
    return DS_SEL_E_INVALID;
  if (a->dim != 32 && a->dim != 64 && a->dim != 128 && a->dim != 256) {
    if (a->dim % 8 != 0 || a->dim > DS_SEL_MAX_DIM) return DS_SEL_E_INVALID;
    return DS_SEL_E_UNSUPPORTED;
  }
  if (a->layers > lim.max_layers || a->rows > lim.max_rows || a->heads > lim.max_heads ||
      a->dim > lim.max_dim || a->k > lim.max_k || a->blocks > lim.max_blocks)
    return DS_SEL_E_CAPACITY;
  if (lim.flags & DS_SEL_FLAG_HEAD_RELU) {
    // the per-head ReLU score: bf16 keys on the matrix cores, heads staged in LDS
    if (k8 || (lim.flags & DS_SEL_FLAG_VALU_SCORE)) return DS_SEL_E_UNSUPPORTED;
    if (dssel::relu_stage_bytes(a->rows, a->heads, a->dim) + 16 > dssel::kReluStageBytes)
      return DS_SEL_E_UNSUPPORTED;
  }
  if (!a->q || !a->w || !a->out_idx || !a->out_score) return DS_SEL_E_INVALID;
  if (!aligned(a->q, 16) || !aligned(a->w, 2) || !aligned(a->out_idx, 4) ||
      !aligned(a->out_score, 4) || !aligned(a->out_count, 4) || !aligned(a->limit, 4) ||
      !aligned(a->mask, 4))
    return DS_SEL_E_INVALID;
  const int64_t N = a->blocks;
  if (k8) {
    if (a->keys) return DS_SEL_E_INVALID;  // the key stream comes from k8
    const int rc = check_q8_keys(a, k8);
    if (rc != DS_SEL_OK) return rc;
  } else if (N > 0) {
    if (!a->keys || !aligned(a->keys, 16)) return DS_SEL_E_INVALID;
    if (a->ldk < a->dim || a->ldk % 8 != 0) return DS_SEL_E_INVALID;
    if (a->key_layer_stride < 0 || a->key_layer_stride % 8 != 0) return DS_SEL_E_INVALID;
    if (a->layers > 1 && a->key_layer_stride < N * a->ldk) return DS_SEL_E_INVALID;
  }
  if (a->mask) {
    const int64_t words = (N + 31) / 32;
    if (a->mask_row_stride != 0 && a->mask_row_stride < words) return DS_SEL_E_INVALID;
    if (a->mask_row_stride < 0 || a->mask_layer_stride < 0) return DS_SEL_E_INVALID;
    if (a->layers > 1 && a->mask_layer_stride < (a->rows - 1) * a->mask_row_stride + words)
      return DS_SEL_E_INVALID;
  }
  return DS_SEL_OK;
}

// The 8-bit key stream of a call: codes [L][N][ldc] int8 (8-byte aligned rows),
// fp16 scales [L][N][lds] with d/32 per row.
int check_q8_keys(const ds_sel_args* a, const ds_sel_q8_keys* k8) {
  if (!k8 || k8->struct_size != sizeof(ds_sel_q8_keys) || k8->reserved != 0) return DS_SEL_E_INVALID;
  const int64_t N = a->blocks, groups = a->dim / 32;
  if (N == 0) return DS_SEL_OK;
  if (!k8->codes || !aligned(k8->codes, 8) || !k8->scales || !aligned(k8->scales, 2)) return DS_SEL_E_INVALID;
  if (k8->ldc < a->dim || k8->ldc % 8 != 0 || k8->code_layer_stride < 0 || k8->code_layer_stride % 8 != 0)
    return DS_SEL_E_INVALID;
  if (k8->lds < groups || k8->scale_layer_stride < 0) return DS_SEL_E_INVALID;
  if (a->layers > 1 && (k8->code_layer_stride < N * k8->ldc || k8->scale_layer_stride < N * k8->lds))
    return DS_SEL_E_INVALID;
  return DS_SEL_OK;
}

int check_attend_args(const ds_sel_limits& lim, const ds_sel_attend_args* a) {
  if (!a || a->struct_size != sizeof(ds_sel_attend_args) || a->reserved != 0) return DS_SEL_E_INVALID;
  if (a->layers < 1 || a->rows < 1 || a->heads < 1 || a->dim < 1 || a->k < 1 || a->blocks < 0)
    return DS_SEL_E_INVALID;
  if (a->rows > DS_SEL_MAX_ROWS || a->k > DS_SEL_MAX_K || a->heads > DS_SEL_MAX_HEADS ||
      a->blocks > DS_SEL_MAX_BLOCKS || !std::isfinite(a->scale))
    return DS_SEL_E_INVALID;
  if (a->dim != 32 && a->dim != 64 && a->dim != 128 && a->dim != 256) {
    if (a->dim % 8 != 0 || a->dim > DS_SEL_MAX_DIM) return DS_SEL_E_INVALID;
    return DS_SEL_E_UNSUPPORTED;
  }
  if (a->layers > lim.max_layers || a->rows > lim.max_rows || a->heads > lim.max_heads ||
      a->dim > lim.max_dim || a->k > lim.max_k || a->blocks > lim.max_blocks)
    return DS_SEL_E_CAPACITY;
  if (!a->q || !a->idx || !a->out) return DS_SEL_E_INVALID;
  if (!aligned(a->q, 16) || !aligned(a->idx, 4) || !aligned(a->count, 4) || !aligned(a->out, 4))
    return DS_SEL_E_INVALID;
  const int64_t N = a->blocks;
  if (N > 0) {
    if (!a->keys || !aligned(a->keys, 16) || !a->values || !aligned(a->values, 16))
      return DS_SEL_E_INVALID;
    if (a->ldk < a->dim || a->ldk % 8 != 0 || a->ldv < a->dim || a->ldv % 8 != 0)
      return DS_SEL_E_INVALID;
    if (a->key_layer_stride < 0 || a->key_layer_stride % 8 != 0 || a->value_layer_stride < 0 ||
        a->value_layer_stride % 8 != 0)
      return DS_SEL_E_INVALID;
    if (a->layers > 1 && (a->key_layer_stride < N * a->ldk || a->value_layer_stride < N * a->ldv))
      return DS_SEL_E_INVALID;
  }
  return DS_SEL_OK;
}

// Runs f with `device` current and restores the caller's device.
template <class F>
int with_device(int device, F f) {
  int prev = -1;
  if (hipGetDevice(&prev) != hipSuccess) return DS_SEL_E_HIP;
  if (prev != device && hipSetDevice(device) != hipSuccess) return DS_SEL_E_HIP;
  const int rc = f();
  if (prev != device) (void)hipSetDevice(prev);
  return rc;
}

}  // namespace

extern "C" {

const char* ds_sel_status_string(int status) {
  switch (status) {
    case DS_SEL_OK: return "ok";
    case DS_SEL_E_INVALID: return "invalid argument";
    case DS_SEL_E_CAPACITY: return "exceeds the handle's capacity";
    case DS_SEL_E_NODEVICE: return "no such HIP device";
    case DS_SEL_E_HIP: return "HIP runtime error";
    case DS_SEL_E_NOMEM: return "out of memory";
    case DS_SEL_E_UNSUPPORTED: return "unsupported dimension";
    default: return "unknown status";
  }
}

int64_t ds_sel_scratch_bytes(const ds_sel_limits* lim) {
  if (check_limits(lim) != DS_SEL_OK) return 0;
  return layout_for(*lim).total;
}

int ds_sel_check_args(const ds_sel_limits* lim, const ds_sel_args* a) {
  const int rc = check_limits(lim);
  if (rc != DS_SEL_OK) return rc;
  return check_args(*lim, a);
}

int ds_sel_create(const ds_sel_limits* lim, ds_sel** out) {
  if (!out) return DS_SEL_E_INVALID;
  *out = nullptr;
  int rc = check_limits(lim);
  if (rc != DS_SEL_OK) return rc;
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) != hipSuccess || ndev <= 0) {
    (void)hipGetLastError();
    return DS_SEL_E_NODEVICE;
  }
  if (lim->device >= ndev) return DS_SEL_E_NODEVICE;
  ds_sel* h = new (std::nothrow) ds_sel;
  if (!h) return DS_SEL_E_NOMEM;
  h->lim = *lim;
  const Layout s = layout_for(*lim);
  rc = with_device(lim->device, [&]() {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, lim->device) == hipSuccess &&
        cus > 0)
      h->compute_units = cus;
    (void)hipGetLastError();
    if (hipMalloc(&h->scratch, (size_t)s.total) != hipSuccess) {
      (void)hipGetLastError();
      h->scratch = nullptr;
      return (int)DS_SEL_E_NOMEM;
    }
    if (hipEventCreateWithFlags(&h->done, hipEventDisableTiming) != hipSuccess) {
      (void)hipGetLastError();
      (void)hipFree(h->scratch);
      h->scratch = nullptr;
      h->done = nullptr;
      return (int)DS_SEL_E_HIP;
    }
    return (int)DS_SEL_OK;
  });
  if (rc != DS_SEL_OK) {
    delete h;
    return rc;
  }
  h->lay = s;
  *out = h;
  return DS_SEL_OK;
}

void ds_sel_destroy(ds_sel* h) {
  if (!h) return;
  if (h->scratch) {
    with_device(h->lim.device, [&]() {
      // The handle's work ends with its last recorded event; wait for that
      // only (hipFree itself does not wait for kernels still using the memory).
      if (h->done) {
        (void)hipEventSynchronize(h->done);
        (void)hipEventDestroy(h->done);
      }
      (void)hipFree(h->scratch);
      return (int)DS_SEL_OK;
    });
  }
  delete h;
}

namespace {
// Where one call's scratch lives: the handle's allocation, or the static array.
struct Target {
  int device;
  int compute_units;
  int32_t flags;
  char* scratch;
  Layout lay;
  hipEvent_t done;  // the handle's completion event, or null
};

// Record the handle's completion event after a call's launches, unless the
// stream is being captured into a graph (the event would then not mark this
// call's completion).
int mark_done(hipEvent_t done, hipStream_t stream) {
  if (!done) return DS_SEL_OK;
  hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(stream, &st) != hipSuccess) {
    (void)hipGetLastError();
    return DS_SEL_OK;
  }
  if (st != hipStreamCaptureStatusNone) return DS_SEL_OK;
  return hipEventRecord(done, stream) == hipSuccess ? DS_SEL_OK : DS_SEL_E_HIP;
}
int enqueue(const Target& t, const ds_sel_args* a, void* hip_stream, void* const* events,
            const ds_sel_q8_keys* k8 = nullptr);

Target handle_target(const ds_sel* h) {
  Target t;
  t.device = h->lim.device;
  t.compute_units = h->compute_units;
  t.flags = h->lim.flags;
  t.scratch = static_cast<char*>(h->scratch);
  t.lay = h->lay;
  t.done = h->done;
  return t;
}

// ---------------------------------------------------------------------------
// The entry point that allocates nothing: its scratch is this file-scope
// device array (one copy per GPU, held until the process ends).  Host code
// never passes the array's name to a kernel or a copy: the name is a host-side
// stand-in, so the array's device address is looked up once per device with
// hipGetSymbolAddress and that pointer is used instead.
constexpr int64_t kStaticScratchBytes = 64ll << 20;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
struct StaticSlot {
  bool ready = false;
  void* ptr = nullptr;
  int compute_units = 256;
};
StaticSlot g_static[kMaxDevices];
std::mutex g_static_mu;

// The array's address and the compute-unit count on `device` (made current by
// the caller), looked up on the first call on that device.
int static_slot(int device, StaticSlot* out) {
  std::lock_guard<std::mutex> lock(g_static_mu);
  StaticSlot& s = g_static[device];
  if (!s.ready) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) {
      (void)hipGetLastError();
      return DS_SEL_E_HIP;
    }
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device) == hipSuccess &&
        cus > 0)
      s.compute_units = cus;
    (void)hipGetLastError();
    s.ptr = ptr;
    s.ready = true;
  }
  *out = s;
  return DS_SEL_OK;
}
}  // namespace

int ds_sel_score_select(ds_sel* h, const ds_sel_args* a, void* hip_stream) {
  if (!h) return DS_SEL_E_INVALID;
  const int rc = check_args(h->lim, a);
  if (rc != DS_SEL_OK) return rc;
  return enqueue(handle_target(h), a, hip_stream, nullptr);
}

int ds_sel_score_select_profiled(ds_sel* h, const ds_sel_args* a, void* hip_stream,
                                 void* const events[4]) {
  if (!events || !events[0] || !events[1] || !events[2] || !events[3]) return DS_SEL_E_INVALID;
  if (!h) return DS_SEL_E_INVALID;
  const int rc = check_args(h->lim, a);
  if (rc != DS_SEL_OK) return rc;
  return enqueue(handle_target(h), a, hip_stream, events);
}

int ds_sel_poison_scratch(ds_sel* h, int32_t byte, void* hip_stream) {
  if (!h || byte < 0 || byte > 255) return DS_SEL_E_INVALID;
  return with_device(h->lim.device, [&]() {
    const hipError_t e = hipMemsetAsync(h->scratch, byte, (size_t)h->lay.total,
                                        static_cast<hipStream_t>(hip_stream));
    if (e != hipSuccess) return (int)DS_SEL_E_HIP;
    return mark_done(h->done, static_cast<hipStream_t>(hip_stream));
  });
}

// ---------------------------------------------------------------- serial decode
namespace {

// The layers of `a` one after another, each a one-layer call of the chain,
// with the stand-in step between them writing layer l + 1's query into q_work.
int enqueue_decode(const Target& t, const ds_sel_args* a, void* q_work, hipStream_t stream) {
  const int64_t L = a->layers, R = a->rows, H = a->heads, D = a->dim, k = a->k;
  const uint16_t* q = static_cast<const uint16_t*>(a->q);
  uint16_t* qw = static_cast<uint16_t*>(q_work);
  for (int64_t l = 0; l < L; ++l) {
    ds_sel_args al = *a;
    al.layers = 1;
    al.q = l == 0 ? a->q : static_cast<const void*>(qw + l * R * H * D);
    al.w = static_cast<const uint16_t*>(a->w) + l * R * H;
    if (a->keys) al.keys = static_cast<const uint16_t*>(a->keys) + l * a->key_layer_stride;
    if (a->mask) al.mask = a->mask + l * a->mask_layer_stride;
    if (a->limit) al.limit = a->limit + l * R;
    al.out_idx = a->out_idx + l * R * k;
    al.out_score = a->out_score + l * R * k;
    if (a->out_count) al.out_count = a->out_count + l * R;
    const int rc = enqueue(t, &al, stream, nullptr);
    if (rc != DS_SEL_OK) return rc;
    if (l + 1 < L) {
      dssel::RotateCall rcall{};
      rcall.rows = (int32_t)R;
      rcall.heads = (int32_t)H;
      rcall.dim = (int32_t)D;
      rcall.k = (int32_t)k;
      rcall.q_next = q + (l + 1) * R * H * D;
      rcall.idx = al.out_idx;
      rcall.q_out = qw + (l + 1) * R * H * D;
      const int e = with_device(t.device, [&]() {
        return dssel::launch_rotate(rcall, stream) == hipSuccess ? (int)DS_SEL_OK : (int)DS_SEL_E_HIP;
      });
      if (e != DS_SEL_OK) return e;
    }
  }
  return DS_SEL_OK;
}

int check_decode(const ds_sel* h, const ds_sel_args* a, const void* q_work) {
  if (!h) return DS_SEL_E_INVALID;
  const int rc = check_args(h->lim, a);
  if (rc != DS_SEL_OK) return rc;
  if (a->layers > 1 && (!q_work || !aligned(q_work, 16))) return DS_SEL_E_INVALID;
  return DS_SEL_OK;
}

}  // namespace

struct ds_sel_plan {
  int device = 0;
  hipGraph_t graph = nullptr;
  hipGraphExec_t exec = nullptr;
  hipEvent_t done = nullptr;  // the handle's: a launch is a call on the handle
};

int ds_sel_decode(ds_sel* h, const ds_sel_args* a, void* q_work, void* hip_stream) {
  const int rc = check_decode(h, a, q_work);
  if (rc != DS_SEL_OK) return rc;
  return enqueue_decode(handle_target(h), a, q_work, static_cast<hipStream_t>(hip_stream));
}

int ds_sel_decode_plan_create(ds_sel* h, const ds_sel_args* a, void* q_work, void* hip_stream,
                              ds_sel_plan** out) {
  if (!out) return DS_SEL_E_INVALID;
  *out = nullptr;
  const int rc = check_decode(h, a, q_work);
  if (rc != DS_SEL_OK) return rc;
  if (!hip_stream) return DS_SEL_E_INVALID;  // the legacy null stream cannot be captured
  hipStream_t stream = static_cast<hipStream_t>(hip_stream);
  ds_sel_plan* p = new (std::nothrow) ds_sel_plan;
  if (!p) return DS_SEL_E_NOMEM;
  p->device = h->lim.device;
  p->done = h->done;
  const int e = with_device(p->device, [&]() {
    if (hipStreamBeginCapture(stream, hipStreamCaptureModeThreadLocal) != hipSuccess) return (int)DS_SEL_E_HIP;
    const int erc = enqueue_decode(handle_target(h), a, q_work, stream);
    hipGraph_t g = nullptr;
    const hipError_t end = hipStreamEndCapture(stream, &g);
    if (erc != DS_SEL_OK || end != hipSuccess || !g) {
      if (g) (void)hipGraphDestroy(g);
      (void)hipGetLastError();
      return erc != DS_SEL_OK ? erc : (int)DS_SEL_E_HIP;
    }
    p->graph = g;
    if (hipGraphInstantiate(&p->exec, g, nullptr, nullptr, 0) != hipSuccess) return (int)DS_SEL_E_HIP;
    return (int)DS_SEL_OK;
  });
  if (e != DS_SEL_OK) {
    ds_sel_decode_plan_destroy(p);
    return e;
  }
  *out = p;
  return DS_SEL_OK;
}

int ds_sel_decode_plan_launch(ds_sel_plan* p, void* hip_stream) {
  if (!p || !p->exec) return DS_SEL_E_INVALID;
  hipStream_t stream = static_cast<hipStream_t>(hip_stream);
  return with_device(p->device, [&]() {
    if (hipGraphLaunch(p->exec, stream) != hipSuccess) return (int)DS_SEL_E_HIP;
    return mark_done(p->done, stream);
  });
}

void ds_sel_decode_plan_destroy(ds_sel_plan* p) {
  if (!p) return;
  with_device(p->device, [&]() {
    if (p->exec) (void)hipGraphExecDestroy(p->exec);
    if (p->graph) (void)hipGraphDestroy(p->graph);
    return (int)DS_SEL_OK;
  });
  delete p;
}

int ds_sel_score_select_q8(ds_sel* h, const ds_sel_args* a, const ds_sel_q8_keys* k8, void* hip_stream,
                           void* const events[4]) {
  if (!h || !k8) return DS_SEL_E_INVALID;
  const int rc = check_args(h->lim, a, k8);
  if (rc != DS_SEL_OK) return rc;
  return enqueue(handle_target(h), a, hip_stream, events, k8);
}

int ds_sel_check_args_q8(const ds_sel_limits* lim, const ds_sel_args* a, const ds_sel_q8_keys* k8) {
  const int rc = check_limits(lim);
  if (rc != DS_SEL_OK) return rc;
  if (!k8) return DS_SEL_E_INVALID;
  return check_args(*lim, a, k8);
}

int ds_sel_quantize_q8(const ds_sel_quantize_args* a, void* hip_stream) {
  if (!a || a->struct_size != sizeof(ds_sel_quantize_args) || a->reserved != 0) return DS_SEL_E_INVALID;
  if (a->layers < 1 || a->blocks < 0 || a->blocks > DS_SEL_MAX_BLOCKS) return DS_SEL_E_INVALID;
  if (a->dim != 32 && a->dim != 64 && a->dim != 128 && a->dim != 256) return DS_SEL_E_INVALID;
  if (a->blocks > 0) {
    if (!a->keys || !aligned(a->keys, 16) || !a->codes || !aligned(a->codes, 16) || !a->scales ||
        !aligned(a->scales, 2))
      return DS_SEL_E_INVALID;
    if (a->ldk < a->dim || a->ldk % 8 != 0 || a->key_layer_stride < 0 || a->key_layer_stride % 8 != 0)
      return DS_SEL_E_INVALID;
    if (a->ldc < a->dim || a->ldc % 16 != 0 || a->code_layer_stride < 0 || a->code_layer_stride % 16 != 0)
      return DS_SEL_E_INVALID;
    if (a->lds < a->dim / 32 || a->scale_layer_stride < 0) return DS_SEL_E_INVALID;
    if (a->layers > 1 && (a->key_layer_stride < a->blocks * a->ldk ||
                          a->code_layer_stride < a->blocks * a->ldc ||
                          a->scale_layer_stride < a->blocks * a->lds))
      return DS_SEL_E_INVALID;
  }
  int current = 0;
  if (hipGetDevice(&current) != hipSuccess) return DS_SEL_E_NODEVICE;
  dssel::QuantizeCall c{};
  c.layers = a->layers;
  c.dim = a->dim;
  c.blocks = a->blocks;
  c.keys = static_cast<const uint16_t*>(a->keys);
  c.ldk = a->ldk;
  c.key_layer_stride = a->key_layer_stride;
  c.codes = a->codes;
  c.ldc = a->ldc;
  c.code_layer_stride = a->code_layer_stride;
  c.scales = a->scales;
  c.lds = a->lds;
  c.scale_layer_stride = a->scale_layer_stride;
  return dssel::launch_quantize(c, static_cast<hipStream_t>(hip_stream)) == hipSuccess ? (int)DS_SEL_OK
                                                                                      : (int)DS_SEL_E_HIP;
}

int64_t ds_sel_noalloc_scratch_bytes(const ds_sel_args* a) {
  if (!a || a->struct_size != sizeof(ds_sel_args) || a->layers < 1 || a->rows < 1 || a->dim < 1 ||
      a->blocks < 0 || a->rows > DS_SEL_MAX_ROWS || a->dim > DS_SEL_MAX_DIM ||
      a->blocks > DS_SEL_MAX_BLOCKS)
    return -1;
  ds_sel_limits lim{};
  lim.struct_size = sizeof(ds_sel_limits);
  lim.max_layers = a->layers;
  lim.max_rows = a->rows;
  lim.max_dim = a->dim;
  lim.max_blocks = a->blocks;
  return layout_for(lim, false).total;
}

int ds_sel_score_select_noalloc(int32_t device, uint32_t flags, const ds_sel_args* a,
                                void* hip_stream) {
  if (device < 0 || device >= kMaxDevices || (flags & ~(uint32_t)kKnownFlags) != 0)
    return DS_SEL_E_INVALID;
  // Checks against the build's hard limits only; the static array decides the rest.
  ds_sel_limits lim{};
  lim.struct_size = sizeof(ds_sel_limits);
  lim.device = device;
  lim.max_layers = 65535;
  lim.max_rows = DS_SEL_MAX_ROWS;
  lim.max_heads = DS_SEL_MAX_HEADS;
  lim.max_dim = DS_SEL_MAX_DIM;
  lim.max_k = DS_SEL_MAX_K;
  lim.max_blocks = DS_SEL_MAX_BLOCKS;
  lim.flags = (int32_t)flags;
  int rc = check_args(lim, a);
  if (rc != DS_SEL_OK) return rc;
  const int64_t need = ds_sel_noalloc_scratch_bytes(a);
  if (need < 0 || need > kStaticScratchBytes) return DS_SEL_E_CAPACITY;
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) != hipSuccess || ndev <= 0 || device >= ndev) {
    (void)hipGetLastError();
    return DS_SEL_E_NODEVICE;
  }
  return with_device(device, [&]() {
    StaticSlot slot;
    const int src = static_slot(device, &slot);
    if (src != DS_SEL_OK) return src;
    ds_sel_limits call_lim = lim;
    call_lim.max_layers = a->layers;
    call_lim.max_rows = a->rows;
    call_lim.max_dim = a->dim;
    call_lim.max_blocks = a->blocks;
    Target t;
    t.device = device;
    t.compute_units = slot.compute_units;
    t.flags = (int32_t)flags;
    t.scratch = static_cast<char*>(slot.ptr);
    t.lay = layout_for(call_lim, false);
    t.done = nullptr;
    return enqueue(t, a, hip_stream, nullptr);
  });
}

int ds_sel_calibrate(const ds_sel_calib_args* a, void* hip_stream) {
  if (!a || a->struct_size != sizeof(ds_sel_calib_args) || a->reserved != 0) return DS_SEL_E_INVALID;
  if (a->workgroups < 1 || a->workgroups > 65535 || !a->sink) return DS_SEL_E_INVALID;
  if (a->kind != DS_SEL_CALIB_EMPTY) {
    if (a->layers < 1 || a->blocks < 1 || !a->keys || !aligned(a->keys, 16)) return DS_SEL_E_INVALID;
    if (a->dim != 32 && a->dim != 64 && a->dim != 128 && a->dim != 256) return DS_SEL_E_INVALID;
    if (a->ldk < a->dim || a->ldk % 8 != 0 || a->key_layer_stride % 8 != 0) return DS_SEL_E_INVALID;
    if (a->layers > 1 && a->key_layer_stride < a->blocks * a->ldk) return DS_SEL_E_INVALID;
  }
  if (a->kind == DS_SEL_CALIB_READ) {
    if (a->ldk != a->dim || (a->layers > 1 && a->key_layer_stride != a->blocks * a->dim))
      return DS_SEL_E_INVALID;
  } else if (a->kind == DS_SEL_CALIB_GATHER) {
    if (!a->ranges || !aligned(a->ranges, 8) || !aligned(a->mask, 4)) return DS_SEL_E_INVALID;
    if (a->mask && a->layers > 1 && a->mask_layer_stride < (a->blocks + 31) / 32) return DS_SEL_E_INVALID;
  } else if (a->kind != DS_SEL_CALIB_EMPTY) {
    return DS_SEL_E_INVALID;
  }
  dssel::CalibCall c{};
  c.kind = a->kind;
  c.workgroups = a->workgroups;
  c.layers = a->layers;
  c.dim = a->dim;
  c.blocks = a->blocks;
  c.ldk = a->ldk;
  c.key_layer_stride = a->key_layer_stride;
  c.mask_layer_stride = a->mask_layer_stride;
  c.keys = static_cast<const uint16_t*>(a->keys);
  c.mask = a->mask;
  c.ranges = a->ranges;
  c.sink = a->sink;
  return dssel::launch_calibrate(c, static_cast<hipStream_t>(hip_stream)) == hipSuccess
             ? (int)DS_SEL_OK
             : (int)DS_SEL_E_HIP;
}

int ds_sel_check_attend_args(const ds_sel_limits* lim, const ds_sel_attend_args* a) {
  const int rc = check_limits(lim);
  if (rc != DS_SEL_OK) return rc;
  return check_attend_args(*lim, a);
}

int ds_sel_attend(ds_sel* h, const ds_sel_attend_args* a, void* hip_stream) {
  if (!h) return DS_SEL_E_INVALID;
  const int rc = check_attend_args(h->lim, a);
  if (rc != DS_SEL_OK) return rc;
  dssel::AttendCall c{};
  c.layers = a->layers;
  c.rows = a->rows;
  c.heads = a->heads;
  c.dim = a->dim;
  c.k = a->k;
  c.blocks = a->blocks;
  c.scale = a->scale;
  c.head_tiles = (a->heads + dssel::kAttendHeadTile - 1) / dssel::kAttendHeadTile;
  {
    // Split each (layer, row, tile)'s selection only while the pairs alone
    // leave compute units idle, and never past the scratch's record count.
    const int64_t chunks = (a->k + dssel::kAttendChunk - 1) / dssel::kAttendChunk;
    const int64_t base = (int64_t)a->layers * a->rows * c.head_tiles;
    int64_t splits = 1;
    if (base < h->compute_units) {
      splits = h->compute_units / base;
      const int64_t cap = dssel::kAttendPartialWgs / base;
      if (splits > cap) splits = cap;
      if (splits > chunks) splits = chunks;
      if (splits < 1) splits = 1;
    }
    c.chunks_per_split = (int32_t)((chunks + splits - 1) / splits);
    c.splits = (int32_t)((chunks + c.chunks_per_split - 1) / c.chunks_per_split);
  }
  c.q = static_cast<const uint16_t*>(a->q);
  c.keys = static_cast<const uint16_t*>(a->keys);
  c.ldk = a->ldk;
  c.key_layer_stride = a->key_layer_stride;
  c.values = static_cast<const uint16_t*>(a->values);
  c.ldv = a->ldv;
  c.value_layer_stride = a->value_layer_stride;
  c.idx = a->idx;
  c.count = a->count;
  c.out = a->out;
  char* base = static_cast<char*>(h->scratch);
  c.part_ml = reinterpret_cast<float*>(base + h->lay.part_ml);
  c.part_o = reinterpret_cast<float*>(base + h->lay.part_o);
  hipStream_t stream = static_cast<hipStream_t>(hip_stream);
  return with_device(h->lim.device, [&]() {
    if (dssel::launch_attend(c, stream) != hipSuccess) return (int)DS_SEL_E_HIP;
    return mark_done(h->done, stream);
  });
}

}  // extern "C"

namespace {
// Enqueue the chain for an already validated call on the target's scratch.
int enqueue(const Target& t, const ds_sel_args* a, void* hip_stream, void* const* events,
            const ds_sel_q8_keys* k8) {
  dssel::Call c{};
  c.layers = a->layers;
  c.rows = a->rows;
  c.heads = a->heads;
  c.dim = a->dim;
  c.k = a->k;
  c.blocks = a->blocks;
  c.q = static_cast<const uint16_t*>(a->q);
  c.w = static_cast<const uint16_t*>(a->w);
  c.keys = static_cast<const uint16_t*>(a->keys);
  c.ldk = a->ldk;
  c.key_layer_stride = a->key_layer_stride;
  c.mask = a->mask;
  c.mask_row_stride = a->mask_row_stride;
  c.mask_layer_stride = a->mask_layer_stride;
  c.limit = a->limit;
  c.mode = !a->mask ? dssel::kNoMask
                    : ((a->mask_row_stride == 0 || a->rows == 1) ? dssel::kSharedMask
                                                                 : dssel::kRowMask);
  c.engine = (t.flags & DS_SEL_FLAG_VALU_SCORE) ? dssel::kEngineValu : dssel::kEngineMfma;
  c.score_kind = (t.flags & DS_SEL_FLAG_HEAD_RELU) ? dssel::kScoreHeadRelu : dssel::kScoreLinear;
  c.fmt = k8 ? dssel::kKeysQ8 : dssel::kKeysBf16;
  if (k8) {
    c.codes = k8->codes;
    c.ldc = k8->ldc;
    c.code_layer_stride = k8->code_layer_stride;
    c.scales = k8->scales;
    c.lds = k8->lds;
    c.scale_layer_stride = k8->scale_layer_stride;
  }
  c.ntiles = (int32_t)((a->blocks + dssel::kTileBlocks - 1) / dssel::kTileBlocks);
  c.cand_stride = (a->blocks + 3) / 4 * 4;
  {
    // Score grid: every resident slot (four workgroups per compute unit), and
    // enough workgroups that a piece never exceeds kScorePieceMax positions
    // even when every block is admitted.
    const int64_t slots = (int64_t)dssel::kScoreWgsPerCu * t.compute_units;
    const int64_t need = a->layers + ((int64_t)a->layers * a->blocks + dssel::kScorePieceMax - 1) /
                                         dssel::kScorePieceMax;
    c.score_slots = (int32_t)slots;
    c.score_wgs = (int32_t)(slots > need ? slots : need);
  }
  c.out_idx = a->out_idx;
  c.out_score = a->out_score;
  c.out_count = a->out_count;
  char* base = t.scratch;
  c.qt = reinterpret_cast<float*>(base + t.lay.qt);
  c.qparts = reinterpret_cast<uint16_t*>(base + t.lay.qparts);
  c.list = reinterpret_cast<int32_t*>(base + t.lay.list);
  c.counts = reinterpret_cast<int32_t*>(base + t.lay.counts);
  c.floor_key = reinterpret_cast<uint32_t*>(base + t.lay.floor);
  c.cand_count = reinterpret_cast<int32_t*>(base + t.lay.ccount);
  c.cand = reinterpret_cast<uint64_t*>(base + t.lay.cand);

  hipStream_t stream = static_cast<hipStream_t>(hip_stream);
  auto mark = [&](int i) {
    return !events || hipEventRecord(static_cast<hipEvent_t>(events[i]), stream) == hipSuccess;
  };
  return with_device(t.device, [&]() {
    if (!mark(0)) return (int)DS_SEL_E_HIP;
    if (dssel::launch_prep(c, stream) != hipSuccess || !mark(1)) return (int)DS_SEL_E_HIP;
    if (dssel::launch_score(c, stream) != hipSuccess || !mark(2)) return (int)DS_SEL_E_HIP;
    if (dssel::launch_select(c, stream) != hipSuccess || !mark(3)) return (int)DS_SEL_E_HIP;
    return mark_done(t.done, stream);
  });
}
}  // namespace
