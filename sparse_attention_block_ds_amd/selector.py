"""ctypes binding of libdssel (include/ds_sel.h) for torch tensors.

Marshalling only: every step of the selection runs in the library's HIP
kernels.  torch provides device memory and the stream.  If the library is not
built this module raises instead of falling back to anything else.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

PKG = os.path.dirname(os.path.abspath(__file__))
LIBRARY = os.path.join(PKG, "libdssel.so")

DS_SEL_OK = 0
DS_SEL_E_INVALID = 1
DS_SEL_E_CAPACITY = 2
DS_SEL_E_NODEVICE = 3
DS_SEL_E_HIP = 4
DS_SEL_E_NOMEM = 5
DS_SEL_E_UNSUPPORTED = 6
DS_SEL_FLAG_VALU_SCORE = 1
DS_SEL_FLAG_HEAD_RELU = 2

EXPORTED = ("ds_sel_create", "ds_sel_score_select", "ds_sel_score_select_profiled",
            "ds_sel_destroy", "ds_sel_check_args", "ds_sel_scratch_bytes", "ds_sel_status_string",
            "ds_sel_attend", "ds_sel_check_attend_args", "ds_sel_calibrate",
            "ds_sel_score_select_noalloc", "ds_sel_noalloc_scratch_bytes",
            "ds_sel_score_select_q8", "ds_sel_check_args_q8", "ds_sel_quantize_q8",
            "ds_sel_poison_scratch", "ds_sel_decode", "ds_sel_decode_plan_create",
            "ds_sel_decode_plan_launch", "ds_sel_decode_plan_destroy")

DS_SEL_CALIB_EMPTY = 0
DS_SEL_CALIB_READ = 1
DS_SEL_CALIB_GATHER = 2


class Limits(ctypes.Structure):
    _fields_ = [("struct_size", ctypes.c_uint32), ("device", ctypes.c_int32),
                ("max_layers", ctypes.c_int32), ("max_rows", ctypes.c_int32),
                ("max_heads", ctypes.c_int32), ("max_dim", ctypes.c_int32),
                ("max_k", ctypes.c_int32), ("flags", ctypes.c_int32),
                ("max_blocks", ctypes.c_int64)]


class Args(ctypes.Structure):
    _fields_ = [("struct_size", ctypes.c_uint32), ("layers", ctypes.c_int32),
                ("rows", ctypes.c_int32), ("heads", ctypes.c_int32), ("dim", ctypes.c_int32),
                ("k", ctypes.c_int32), ("blocks", ctypes.c_int64),
                ("q", ctypes.c_void_p), ("w", ctypes.c_void_p), ("keys", ctypes.c_void_p),
                ("ldk", ctypes.c_int64), ("key_layer_stride", ctypes.c_int64),
                ("mask", ctypes.c_void_p), ("mask_row_stride", ctypes.c_int64),
                ("mask_layer_stride", ctypes.c_int64), ("limit", ctypes.c_void_p),
                ("out_idx", ctypes.c_void_p), ("out_score", ctypes.c_void_p),
                ("out_count", ctypes.c_void_p)]


class AttendArgs(ctypes.Structure):
    _fields_ = [("struct_size", ctypes.c_uint32), ("layers", ctypes.c_int32),
                ("rows", ctypes.c_int32), ("heads", ctypes.c_int32), ("dim", ctypes.c_int32),
                ("k", ctypes.c_int32), ("scale", ctypes.c_float), ("reserved", ctypes.c_int32),
                ("blocks", ctypes.c_int64), ("q", ctypes.c_void_p), ("keys", ctypes.c_void_p),
                ("ldk", ctypes.c_int64), ("key_layer_stride", ctypes.c_int64),
                ("values", ctypes.c_void_p), ("ldv", ctypes.c_int64),
                ("value_layer_stride", ctypes.c_int64), ("idx", ctypes.c_void_p),
                ("count", ctypes.c_void_p), ("out", ctypes.c_void_p)]


class CalibArgs(ctypes.Structure):
    _fields_ = [("struct_size", ctypes.c_uint32), ("kind", ctypes.c_int32),
                ("workgroups", ctypes.c_int32), ("layers", ctypes.c_int32),
                ("dim", ctypes.c_int32), ("reserved", ctypes.c_int32), ("blocks", ctypes.c_int64),
                ("keys", ctypes.c_void_p), ("ldk", ctypes.c_int64),
                ("key_layer_stride", ctypes.c_int64), ("mask", ctypes.c_void_p),
                ("mask_layer_stride", ctypes.c_int64), ("ranges", ctypes.c_void_p),
                ("sink", ctypes.c_void_p)]


class Q8Keys(ctypes.Structure):
    _fields_ = [("struct_size", ctypes.c_uint32), ("reserved", ctypes.c_int32),
                ("codes", ctypes.c_void_p), ("ldc", ctypes.c_int64),
                ("code_layer_stride", ctypes.c_int64), ("scales", ctypes.c_void_p),
                ("lds", ctypes.c_int64), ("scale_layer_stride", ctypes.c_int64)]


class QuantizeArgs(ctypes.Structure):
    _fields_ = [("struct_size", ctypes.c_uint32), ("layers", ctypes.c_int32),
                ("dim", ctypes.c_int32), ("reserved", ctypes.c_int32), ("blocks", ctypes.c_int64),
                ("keys", ctypes.c_void_p), ("ldk", ctypes.c_int64),
                ("key_layer_stride", ctypes.c_int64), ("codes", ctypes.c_void_p),
                ("ldc", ctypes.c_int64), ("code_layer_stride", ctypes.c_int64),
                ("scales", ctypes.c_void_p), ("lds", ctypes.c_int64),
                ("scale_layer_stride", ctypes.c_int64)]


class DsSelError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)} ({status})")


_lib = None


def load_library(path: Optional[str] = None):
    """Load libdssel.so (or the library at `path`); raises if it has not been built."""
    global _lib
    default = path is None
    path = LIBRARY if default else path
    if _lib is not None and default:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with "
                           "`python -m sparse_attention_block_ds_amd.build`")
    lib = ctypes.CDLL(path)
    P = ctypes.POINTER
    lib.ds_sel_create.argtypes = [P(Limits), P(ctypes.c_void_p)]
    lib.ds_sel_create.restype = ctypes.c_int
    lib.ds_sel_score_select.argtypes = [ctypes.c_void_p, P(Args), ctypes.c_void_p]
    lib.ds_sel_score_select.restype = ctypes.c_int
    lib.ds_sel_score_select_profiled.argtypes = [ctypes.c_void_p, P(Args), ctypes.c_void_p,
                                                 P(ctypes.c_void_p)]
    lib.ds_sel_score_select_profiled.restype = ctypes.c_int
    lib.ds_sel_destroy.argtypes = [ctypes.c_void_p]
    lib.ds_sel_destroy.restype = None
    lib.ds_sel_check_args.argtypes = [P(Limits), P(Args)]
    lib.ds_sel_check_args.restype = ctypes.c_int
    lib.ds_sel_scratch_bytes.argtypes = [P(Limits)]
    lib.ds_sel_scratch_bytes.restype = ctypes.c_int64
    lib.ds_sel_attend.argtypes = [ctypes.c_void_p, P(AttendArgs), ctypes.c_void_p]
    lib.ds_sel_attend.restype = ctypes.c_int
    lib.ds_sel_check_attend_args.argtypes = [P(Limits), P(AttendArgs)]
    lib.ds_sel_check_attend_args.restype = ctypes.c_int
    lib.ds_sel_score_select_noalloc.argtypes = [ctypes.c_int32, ctypes.c_uint32, P(Args),
                                                ctypes.c_void_p]
    lib.ds_sel_score_select_noalloc.restype = ctypes.c_int
    lib.ds_sel_noalloc_scratch_bytes.argtypes = [P(Args)]
    lib.ds_sel_noalloc_scratch_bytes.restype = ctypes.c_int64
    lib.ds_sel_calibrate.argtypes = [P(CalibArgs), ctypes.c_void_p]
    lib.ds_sel_calibrate.restype = ctypes.c_int
    lib.ds_sel_score_select_q8.argtypes = [ctypes.c_void_p, P(Args), P(Q8Keys), ctypes.c_void_p,
                                           ctypes.POINTER(ctypes.c_void_p)]
    lib.ds_sel_score_select_q8.restype = ctypes.c_int
    lib.ds_sel_check_args_q8.argtypes = [P(Limits), P(Args), P(Q8Keys)]
    lib.ds_sel_check_args_q8.restype = ctypes.c_int
    lib.ds_sel_quantize_q8.argtypes = [P(QuantizeArgs), ctypes.c_void_p]
    lib.ds_sel_quantize_q8.restype = ctypes.c_int
    lib.ds_sel_decode.argtypes = [ctypes.c_void_p, P(Args), ctypes.c_void_p, ctypes.c_void_p]
    lib.ds_sel_decode.restype = ctypes.c_int
    lib.ds_sel_decode_plan_create.argtypes = [ctypes.c_void_p, P(Args), ctypes.c_void_p, ctypes.c_void_p,
                                              P(ctypes.c_void_p)]
    lib.ds_sel_decode_plan_create.restype = ctypes.c_int
    lib.ds_sel_decode_plan_launch.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    lib.ds_sel_decode_plan_launch.restype = ctypes.c_int
    lib.ds_sel_decode_plan_destroy.argtypes = [ctypes.c_void_p]
    lib.ds_sel_decode_plan_destroy.restype = None
    lib.ds_sel_poison_scratch.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p]
    lib.ds_sel_poison_scratch.restype = ctypes.c_int
    lib.ds_sel_status_string.argtypes = [ctypes.c_int]
    lib.ds_sel_status_string.restype = ctypes.c_char_p
    if default:
        _lib = lib
    return lib


def status_string(status: int) -> str:
    try:
        return load_library().ds_sel_status_string(status).decode()
    except RuntimeError:
        return "status"


def selector_flags(engine="mfma", score="linear"):
    """DS_SEL_FLAG_* bits for a key-stream engine and a score formula."""
    if engine not in ("mfma", "valu"):
        raise ValueError("engine must be 'mfma' or 'valu'")
    if score not in ("linear", "relu"):
        raise ValueError("score must be 'linear' or 'relu'")
    return ((DS_SEL_FLAG_VALU_SCORE if engine == "valu" else 0) |
            (DS_SEL_FLAG_HEAD_RELU if score == "relu" else 0))


def make_limits(max_layers, max_rows, max_heads, max_dim, max_blocks, max_k=512, device=0,
                flags=0):
    return Limits(ctypes.sizeof(Limits), device, max_layers, max_rows, max_heads, max_dim, max_k,
                  flags, max_blocks)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _require(cond, msg):
    if not cond:
        raise ValueError(msg)


def _on(t, device, name):
    _require(t.device == device, f"{name} is on {t.device}, the handle is on {device}")


def check_select_tensors(q, w, keys, k, mask=None, limit=None, out=None, device=None):
    """Reject, before anything reaches the library, tensors whose dtype, shape,
    strides or device differ from what ds_sel_score_select reads and writes.
    Raises ValueError; returns nothing."""
    import torch
    _check_query(q, w)
    L, R, H, d = q.shape
    _require(keys.dtype == torch.bfloat16 and keys.dim() == 3 and keys.shape[0] == L and
             keys.shape[2] >= d, "keys must be a bf16 tensor [L, N, ldk] with ldk >= d")
    N = keys.shape[1]
    if N > 0:  # an empty key tensor is never read, whatever its strides
        _require(keys.stride(2) == 1, "keys must have unit stride in the last dim")
        _require(N == 1 or keys.stride(1) >= d, "keys rows overlap (stride(1) < d)")
    _check_rest(q, w, N, k, mask, limit, out, device, [(keys, "keys")])


def check_q8_tensors(codes, scales, L, d):
    """The 8-bit key stream: codes int8 [L, N, ldc] and scales float16 (the
    fp16 scale bits) [L, N, lds], unit stride in the last dim, ldc >= d and
    lds >= d/32.  Raises ValueError; returns N."""
    import torch
    _require(d % 32 == 0, "the 8-bit key stream needs d to be a multiple of 32")
    _require(codes.dtype == torch.int8 and codes.dim() == 3 and codes.shape[0] == L and
             codes.shape[2] >= d, "codes must be an int8 tensor [L, N, ldc] with ldc >= d")
    N = codes.shape[1]
    _require(scales.dtype == torch.float16 and scales.dim() == 3 and scales.shape[0] == L and
             scales.shape[1] == N and scales.shape[2] >= d // 32,
             "scales must be a float16 tensor [L, N, lds] with lds >= d/32")
    if N > 0:
        _require(codes.stride(2) == 1 and scales.stride(2) == 1,
                 "codes and scales must have unit stride in the last dim")
        _require(N == 1 or (codes.stride(1) >= d and scales.stride(1) >= d // 32),
                 "codes or scales rows overlap")
    return N


def check_select_q8_tensors(q, w, codes, scales, k, mask=None, limit=None, out=None, device=None):
    """check_select_tensors for ds_sel_score_select_q8.  Raises ValueError."""
    _check_query(q, w)
    N = check_q8_tensors(codes, scales, q.shape[0], q.shape[3])
    _check_rest(q, w, N, k, mask, limit, out, device, [(codes, "codes"), (scales, "scales")])


def _check_query(q, w):
    import torch
    _require(q.dim() == 4 and q.dtype == torch.bfloat16 and q.is_contiguous(),
             "q must be a contiguous bf16 tensor [L, R, H, d]")
    L, R, H, d = q.shape
    _require(w.dtype == torch.bfloat16 and tuple(w.shape) == (L, R, H) and w.is_contiguous(),
             "w must be a contiguous bf16 tensor [L, R, H]")


def _check_rest(q, w, N, k, mask, limit, out, device, keys_tensors):
    import torch
    _require(isinstance(k, int) and k >= 1, "k must be an int >= 1")
    device = q.device if device is None else torch.device(device)
    L, R, H, d = q.shape
    tensors = [(q, "q"), (w, "w")] + list(keys_tensors)
    if mask is not None:
        _require(mask.dtype == torch.int32 and mask.dim() == 3 and mask.shape[0] == L and
                 mask.shape[1] in (1, R) and mask.shape[2] * 32 >= N and mask.stride(2) == 1,
                 "mask must be an int32 tensor [L, R or 1, >= ceil(N/32)] with unit stride in the "
                 "last dim")
        tensors.append((mask, "mask"))
    if limit is not None:
        _require(limit.dtype == torch.int32 and tuple(limit.shape) == (L, R) and limit.is_contiguous(),
                 "limit must be a contiguous int32 tensor [L, R]")
        tensors.append((limit, "limit"))
    if out is not None:
        _require(isinstance(out, (tuple, list)) and len(out) == 3,
                 "out must be (idx, score, count) with count possibly None")
        idx, score, count = out
        _require(idx is not None and idx.dtype == torch.int32 and tuple(idx.shape) == (L, R, k) and
                 idx.is_contiguous(), "out idx must be a contiguous int32 tensor [L, R, k]")
        _require(score is not None and score.dtype == torch.float32 and
                 tuple(score.shape) == (L, R, k) and score.is_contiguous(),
                 "out score must be a contiguous float32 tensor [L, R, k]")
        tensors += [(idx, "out idx"), (score, "out score")]
        if count is not None:
            _require(count.dtype == torch.int32 and tuple(count.shape) == (L, R) and
                     count.is_contiguous(), "out count must be a contiguous int32 tensor [L, R]")
            tensors.append((count, "out count"))
    for t, name in tensors:
        _on(t, device, name)


def check_attend_tensors(qa, keys, values, idx, count, scale, out=None, device=None):
    """The same for ds_sel_attend.  Raises ValueError."""
    import math
    import torch
    _require(isinstance(scale, (int, float)) and math.isfinite(float(scale)),
             "scale must be a finite number (the library applies no default)")
    _require(qa.dim() == 4 and qa.dtype == torch.bfloat16 and qa.is_contiguous(),
             "qa must be a contiguous bf16 tensor [L, R, Ha, d]")
    device = qa.device if device is None else torch.device(device)
    L, R, Ha, d = qa.shape
    for t, name in ((keys, "keys"), (values, "values")):
        _require(t.dtype == torch.bfloat16 and t.dim() == 3 and t.shape[0] == L and
                 t.shape[2] >= d and (t.shape[1] == 0 or t.stride(2) == 1),
                 f"{name} must be a bf16 tensor [L, N, ld] with ld >= d and unit stride in the last dim")
    _require(keys.shape[1] == values.shape[1], "keys and values must hold the same number of blocks")
    _require(idx.dtype == torch.int32 and idx.dim() == 3 and tuple(idx.shape[:2]) == (L, R) and
             idx.is_contiguous(), "idx must be a contiguous int32 tensor [L, R, k]")
    tensors = [(qa, "qa"), (keys, "keys"), (values, "values"), (idx, "idx")]
    if count is not None:
        _require(count.dtype == torch.int32 and tuple(count.shape) == (L, R) and count.is_contiguous(),
                 "count must be a contiguous int32 tensor [L, R]")
        tensors.append((count, "count"))
    if out is not None:
        _require(out.dtype == torch.float32 and tuple(out.shape) == (L, R, Ha, d) and
                 out.is_contiguous(), "out must be a contiguous float32 tensor [L, R, Ha, d]")
        tensors.append((out, "out"))
    for t, name in tensors:
        _on(t, device, name)


def make_args(q, w, keys, k, mask=None, limit=None, out_idx=None, out_score=None, out_count=None,
              blocks=None):
    """Fill an Args struct from tensors already accepted by check_select_tensors
    (keys None, with `blocks` given, for the 8-bit key stream)."""
    L, R, H, d = q.shape
    N = keys.shape[1] if keys is not None else blocks
    a = Args()
    a.struct_size = ctypes.sizeof(Args)
    a.layers, a.rows, a.heads, a.dim, a.k, a.blocks = L, R, H, d, k, N
    a.q, a.w = _ptr(q), _ptr(w)
    if keys is not None:
        a.keys = _ptr(keys) if N > 0 else None
        a.ldk = keys.stride(1)
        a.key_layer_stride = keys.stride(0)
    if mask is not None:
        a.mask = _ptr(mask)
        a.mask_row_stride = 0 if mask.shape[1] == 1 else mask.stride(1)
        a.mask_layer_stride = mask.stride(0)
    a.limit = _ptr(limit)
    a.out_idx, a.out_score, a.out_count = _ptr(out_idx), _ptr(out_score), _ptr(out_count)
    return a


def make_q8_keys(codes, scales):
    """Fill a Q8Keys struct from tensors already accepted by check_q8_tensors."""
    k8 = Q8Keys()
    k8.struct_size = ctypes.sizeof(Q8Keys)
    k8.reserved = 0
    if codes.shape[1] > 0:
        k8.codes, k8.scales = _ptr(codes), _ptr(scales)
    k8.ldc, k8.code_layer_stride = codes.stride(1), codes.stride(0)
    k8.lds, k8.scale_layer_stride = scales.stride(1), scales.stride(0)
    return k8


def make_attend_args(qa, keys, values, idx, count, scale, out):
    """Fill an AttendArgs struct from tensors already accepted by check_attend_tensors."""
    L, R, H, d = qa.shape
    N = keys.shape[1]
    a = AttendArgs()
    a.struct_size = ctypes.sizeof(AttendArgs)
    a.layers, a.rows, a.heads, a.dim, a.k, a.blocks = L, R, H, d, idx.shape[2], N
    a.scale, a.reserved = float(scale), 0
    a.q = _ptr(qa)
    a.keys = _ptr(keys) if N > 0 else None
    a.ldk, a.key_layer_stride = keys.stride(1), keys.stride(0)
    a.values = _ptr(values) if N > 0 else None
    a.ldv, a.value_layer_stride = values.stride(1), values.stride(0)
    a.idx, a.count, a.out = _ptr(idx), _ptr(count), _ptr(out)
    return a


class Selector:
    """One libdssel handle: scratch sized for the given capacity on one device."""

    def __init__(self, max_layers, max_rows, max_heads, max_dim, max_blocks, max_k=512,
                 device: Optional[int] = None, engine: str = "mfma", score: str = "linear"):
        """engine "mfma" (default) or "valu" for the key stream; score "linear"
        (sum_h w_h q_h . K) or "relu" (sum_h w_h max(q_h . K, 0))."""
        import torch
        self._torch = torch
        self.lib = load_library()
        self.device = torch.cuda.current_device() if device is None else device
        self.limits = make_limits(max_layers, max_rows, max_heads, max_dim, max_blocks, max_k,
                                  self.device, selector_flags(engine, score))
        h = ctypes.c_void_p()
        rc = self.lib.ds_sel_create(ctypes.byref(self.limits), ctypes.byref(h))
        if rc != DS_SEL_OK:
            raise DsSelError(rc, "ds_sel_create")
        self.handle = h

    def close(self):
        if getattr(self, "handle", None):
            self.lib.ds_sel_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def score_select(self, q, w, keys, k, mask=None, limit=None, out=None, stream=None,
                     events=None):
        """Enqueue one call; returns (idx int32 [L,R,k], score f32 [L,R,k], count int32 [L,R]).

        q bf16 [L,R,H,d]; w bf16 [L,R,H]; keys bf16 [L,N,ldk] (unit stride in the
        last dim); mask int32 (bit patterns) [L, R or 1, words] or None; limit
        int32 [L,R] or None.  The work is asynchronous on `stream` (default:
        torch's current stream).  `events`: four torch.cuda.Event(enable_timing=True)
        recorded before prep and after prep, score and select.
        """
        torch = self._torch
        dev = torch.device("cuda", self.device)
        check_select_tensors(q, w, keys, k, mask, limit, out, dev)
        L, R = q.shape[0], q.shape[1]
        if out is None:
            out = (torch.empty((L, R, k), dtype=torch.int32, device=q.device),
                   torch.empty((L, R, k), dtype=torch.float32, device=q.device),
                   torch.empty((L, R), dtype=torch.int32, device=q.device))
        a = make_args(q, w, keys, k, mask, limit, *out)
        if stream is None:
            stream = torch.cuda.current_stream(q.device)
        handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else stream
        if events is None:
            rc = self.lib.ds_sel_score_select(self.handle, ctypes.byref(a), ctypes.c_void_p(handle))
        else:
            for e in events:  # torch creates the HIP event on its first record
                if not e.cuda_event:
                    e.record(stream)
            ev = (ctypes.c_void_p * 4)(*[e.cuda_event for e in events])
            rc = self.lib.ds_sel_score_select_profiled(self.handle, ctypes.byref(a),
                                                       ctypes.c_void_p(handle), ev)
        if rc != DS_SEL_OK:
            raise DsSelError(rc, "ds_sel_score_select")
        return out


    def poison_scratch(self, byte, stream=None):
        """Fill the handle's scratch with `byte` (a test hook: results must not
        depend on what earlier calls left there)."""
        torch = self._torch
        if stream is None:
            stream = torch.cuda.current_stream(torch.device("cuda", self.device))
        handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else stream
        rc = self.lib.ds_sel_poison_scratch(self.handle, int(byte), ctypes.c_void_p(handle))
        if rc != DS_SEL_OK:
            raise DsSelError(rc, "ds_sel_poison_scratch")

    def _decode_args(self, q, w, keys, k, mask, limit, q_work, out):
        torch = self._torch
        check_select_tensors(q, w, keys, k, mask, limit, out, torch.device("cuda", self.device))
        L, R = q.shape[0], q.shape[1]
        if out is None:
            out = (torch.empty((L, R, k), dtype=torch.int32, device=q.device),
                   torch.empty((L, R, k), dtype=torch.float32, device=q.device),
                   torch.empty((L, R), dtype=torch.int32, device=q.device))
        if q_work is None:
            q_work = torch.empty_like(q)
        _require(q_work.dtype == torch.bfloat16 and q_work.shape == q.shape and q_work.is_contiguous()
                 and q_work.device == q.device, "q_work must be a contiguous bf16 tensor shaped like q")
        return make_args(q, w, keys, k, mask, limit, *out), q_work, out

    def decode(self, q, w, keys, k, mask=None, limit=None, q_work=None, out=None, stream=None):
        """Serial decode over the L layers (ds_sel_decode): layer l >= 1 selects
        with its query heads rotated by layer l-1's best block per row; q_work
        (bf16 like q) receives those queries.  Returns (idx, score, count)."""
        torch = self._torch
        a, q_work, out = self._decode_args(q, w, keys, k, mask, limit, q_work, out)
        if stream is None:
            stream = torch.cuda.current_stream(q.device)
        handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else stream
        rc = self.lib.ds_sel_decode(self.handle, ctypes.byref(a), _ptr(q_work), ctypes.c_void_p(handle))
        if rc != DS_SEL_OK:
            raise DsSelError(rc, "ds_sel_decode")
        return out

    def decode_plan(self, q, w, keys, k, mask=None, limit=None, q_work=None, out=None, stream=None):
        """The serial decode captured into a HIP graph (ds_sel_decode_plan_create)
        on `stream` (a created torch.cuda.Stream, not the null stream).  Returns
        a DecodePlan whose launch() replays it; the tensors must stay alive."""
        torch = self._torch
        a, q_work, out = self._decode_args(q, w, keys, k, mask, limit, q_work, out)
        if stream is None:
            raise ValueError("decode_plan needs a created stream to capture on")
        handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else stream
        p = ctypes.c_void_p()
        rc = self.lib.ds_sel_decode_plan_create(self.handle, ctypes.byref(a), _ptr(q_work),
                                                ctypes.c_void_p(handle), ctypes.byref(p))
        if rc != DS_SEL_OK:
            raise DsSelError(rc, "ds_sel_decode_plan_create")
        return DecodePlan(self, p, (q, w, keys, mask, limit, q_work) + tuple(out), out)

    def score_select_q8(self, q, w, codes, scales, k, mask=None, limit=None, out=None,
                        stream=None, events=None):
        """score_select over the 8-bit key stream (ds_sel_score_select_q8):
        codes int8 [L,N,ldc] and scales float16 [L,N,lds] as quantize_q8
        returns them; every other argument (events included) and the result
        as score_select."""
        torch = self._torch
        dev = torch.device("cuda", self.device)
        check_select_q8_tensors(q, w, codes, scales, k, mask, limit, out, dev)
        L, R = q.shape[0], q.shape[1]
        if out is None:
            out = (torch.empty((L, R, k), dtype=torch.int32, device=q.device),
                   torch.empty((L, R, k), dtype=torch.float32, device=q.device),
                   torch.empty((L, R), dtype=torch.int32, device=q.device))
        a = make_args(q, w, None, k, mask, limit, *out, blocks=codes.shape[1])
        k8 = make_q8_keys(codes, scales)
        if stream is None:
            stream = torch.cuda.current_stream(q.device)
        handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else stream
        ev = None
        if events is not None:
            for e in events:  # torch creates the HIP event on its first record
                if not e.cuda_event:
                    e.record(stream)
            ev = (ctypes.c_void_p * 4)(*[e.cuda_event for e in events])
        rc = self.lib.ds_sel_score_select_q8(self.handle, ctypes.byref(a), ctypes.byref(k8),
                                             ctypes.c_void_p(handle), ev)
        if rc != DS_SEL_OK:
            raise DsSelError(rc, "ds_sel_score_select_q8")
        return out

    def attend(self, qa, keys, values, idx, count, scale, out=None, stream=None):
        """Enqueue attention over a selection; returns out f32 [L,R,Ha,d].

        qa bf16 [L,R,Ha,d]; keys, values bf16 [L,N,ld] (unit stride in the last
        dim); idx int32 [L,R,k] and count int32 [L,R] or None, as score_select
        returns them; scale is the caller's (1/sqrt(d) is the usual choice).
        Asynchronous on `stream`.
        """
        torch = self._torch
        check_attend_tensors(qa, keys, values, idx, count, scale, out,
                             torch.device("cuda", self.device))
        if out is None:
            out = torch.empty(tuple(qa.shape), dtype=torch.float32, device=qa.device)
        a = make_attend_args(qa, keys, values, idx, count, scale, out)
        if stream is None:
            stream = torch.cuda.current_stream(qa.device)
        handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else stream
        rc = self.lib.ds_sel_attend(self.handle, ctypes.byref(a), ctypes.c_void_p(handle))
        if rc != DS_SEL_OK:
            raise DsSelError(rc, "ds_sel_attend")
        return out


class DecodePlan:
    """A captured serial decode; holds its tensors so they outlive the graph."""

    def __init__(self, selector, handle, keep, out):
        self.selector, self.handle, self._keep, self.out = selector, handle, keep, out

    def launch(self, stream):
        handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else stream
        rc = self.selector.lib.ds_sel_decode_plan_launch(self.handle, ctypes.c_void_p(handle))
        if rc != DS_SEL_OK:
            raise DsSelError(rc, "ds_sel_decode_plan_launch")
        return self.out

    def close(self):
        if getattr(self, "handle", None):
            self.selector.lib.ds_sel_decode_plan_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def upload(problem, device="cuda"):
    """Copy a workloads.Problem's host arrays to device tensors (bf16 bit patterns kept)."""
    import torch

    def bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device).view(torch.bfloat16)

    q = bf16(problem.q)
    w = bf16(problem.w)
    keys = bf16(problem.keys)
    mask = None
    if problem.mask is not None:
        mask = torch.from_numpy(np.ascontiguousarray(problem.mask).view(np.int32)).to(device)
    limit = None
    if problem.limit is not None:
        limit = torch.from_numpy(np.ascontiguousarray(problem.limit, dtype=np.int32)).to(device)
    return q, w, keys, mask, limit


def calibrate(kind, workgroups, sink, keys=None, mask=None, ranges=None, stream=None):
    """Enqueue one calibration launch (ds_sel_calibrate) on `stream` (default:
    torch's current stream).  keys bf16 [L,N,ldk]; mask int32 [L,1,words] or
    None; ranges int64 [workgroups + 1] (gather); sink int32 [>= workgroups]."""
    import torch
    lib = load_library()
    a = CalibArgs()
    a.struct_size = ctypes.sizeof(CalibArgs)
    a.kind, a.workgroups, a.reserved = kind, workgroups, 0
    if keys is not None:
        a.layers, a.blocks, a.dim = keys.shape[0], keys.shape[1], keys.shape[2]
        a.keys, a.ldk, a.key_layer_stride = _ptr(keys), keys.stride(1), keys.stride(0)
    if mask is not None:
        a.mask, a.mask_layer_stride = _ptr(mask), mask.stride(0)
    a.ranges, a.sink = _ptr(ranges), _ptr(sink)
    if stream is None:
        stream = torch.cuda.current_stream()
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else stream
    rc = lib.ds_sel_calibrate(ctypes.byref(a), ctypes.c_void_p(handle))
    if rc != DS_SEL_OK:
        raise DsSelError(rc, "ds_sel_calibrate")


def score_select_noalloc(q, w, keys, k, mask, limit, out, device=None, engine="mfma", stream=None,
                         score="linear"):
    """ds_sel_score_select_noalloc: the selection on the library's static
    scratch, with caller-provided outputs (idx, score, count) and no handle.
    Calls overlapping in time on one GPU race (they share the scratch)."""
    import torch
    flags = selector_flags(engine, score)
    if out is None:
        raise ValueError("out (idx, score, count) is required: this entry point allocates nothing")
    dev = q.device if device is None else torch.device("cuda", device)
    check_select_tensors(q, w, keys, k, mask, limit, out, dev)
    lib = load_library()
    a = make_args(q, w, keys, k, mask, limit, *out)
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else stream
    rc = lib.ds_sel_score_select_noalloc(dev.index, flags, ctypes.byref(a), ctypes.c_void_p(handle))
    if rc != DS_SEL_OK:
        raise DsSelError(rc, "ds_sel_score_select_noalloc")
    return out


def quantize_q8(keys, codes=None, scales=None, stream=None):
    """ds_sel_quantize_q8: bf16 keys [L,N,ldk] (unit stride in the last dim)
    into the 8-bit key stream; returns (codes int8 [L,N,d], scales float16
    [L,N,d/32]), allocated here unless given (codes rows 16-byte aligned).
    Asynchronous on `stream` (default: torch's current stream)."""
    import torch
    _require(keys.dtype == torch.bfloat16 and keys.dim() == 3, "keys must be a bf16 tensor [L, N, d]")
    L, N, d = keys.shape
    _require(N == 0 or keys.stride(2) == 1, "keys must have unit stride in the last dim")
    if codes is None:
        codes = torch.empty((L, N, d), dtype=torch.int8, device=keys.device)
    if scales is None:
        scales = torch.empty((L, N, d // 32), dtype=torch.float16, device=keys.device)
    check_q8_tensors(codes, scales, L, d)
    _require(codes.shape[1] == N, "codes must hold one row per key block")
    for t, name in ((codes, "codes"), (scales, "scales")):
        _on(t, keys.device, name)
    lib = load_library()
    a = QuantizeArgs()
    a.struct_size = ctypes.sizeof(QuantizeArgs)
    a.layers, a.dim, a.reserved, a.blocks = L, d, 0, N
    if N > 0:
        a.keys, a.codes, a.scales = _ptr(keys), _ptr(codes), _ptr(scales)
    a.ldk, a.key_layer_stride = keys.stride(1), keys.stride(0)
    a.ldc, a.code_layer_stride = codes.stride(1), codes.stride(0)
    a.lds, a.scale_layer_stride = scales.stride(1), scales.stride(0)
    if stream is None:
        stream = torch.cuda.current_stream(keys.device)
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else stream
    rc = lib.ds_sel_quantize_q8(ctypes.byref(a), ctypes.c_void_p(handle))
    if rc != DS_SEL_OK:
        raise DsSelError(rc, "ds_sel_quantize_q8")
    return codes, scales
