"""CPU oracle for compressed-attention block selection -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The GPU library never loads it, and the
two share no code: the oracle is the plain C definition in
``ds_sel_oracle.c`` (admitted list -> fp32 scores in a fixed order -> qsort by
(score desc, block asc) -> first min(k, admitted)), compiled with gcc into
``libds_sel_oracle.so`` and driven through ctypes from here.

What it follows: page "DeepSeek V4.1F Q4 on M3 Ultra with native DSpark MTP
(40tps / 800tps)", paragraph "Decode at depth" (512 blocks per layer out of the
whole context, only mask-admitted blocks are candidates, the admitted index is
built per row, the top 512 are kept).  The score formula, the order and the
padding are readings of this library, stated in the C file's header.

``quantize_q8`` / ``select_q8`` / ``score_blocks_q8`` are the 8-bit key
stream: keys stored as groups of 32 signed 8-bit codes with one fp16 scale,
scored on their dequantised values (the C file states the reading).

``attend`` is the step after the selection, read the same way: per attention
head, the softmax over the selected blocks of scale * (q . K[b]) applied to the
blocks' values V[b], in double precision (the C file states the reading).

Every array is host numpy; bf16 values travel as their uint16 bit patterns.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "ds_sel_oracle.c")
LIBRARY = os.path.join(_HERE, "libds_sel_oracle.so")

# Flags that keep every fp32 operation a separately rounded IEEE operation.
CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared", "-Wall"]

_lib = None


def build(output: str = LIBRARY, source: str = SOURCE, extra_flags=()) -> str:
    """Compile the C oracle with gcc into ``output`` (always recompiles)."""
    tmp = output + ".tmp"
    cmd = ["gcc", *CFLAGS, *extra_flags, "-o", tmp, source, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, output)
    return output


def _declare(lib):
    i32, i64, p = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p
    lib.ds_sel_oracle_select.restype = ctypes.c_int
    lib.ds_sel_oracle_select.argtypes = [i32, i32, i32, i32, i64, i32, p, p, p, i64, i64, p, i64,
                                         i64, p, p, p, p]
    lib.ds_sel_oracle_score_blocks.restype = ctypes.c_int
    lib.ds_sel_oracle_score_blocks.argtypes = [i32, i32, i32, i32, i64, p, p, p, i64, i64, i32,
                                               i32, i64, p, p]
    lib.ds_sel_oracle_select_relu.restype = ctypes.c_int
    lib.ds_sel_oracle_select_relu.argtypes = lib.ds_sel_oracle_select.argtypes
    lib.ds_sel_oracle_score_blocks_relu.restype = ctypes.c_int
    lib.ds_sel_oracle_score_blocks_relu.argtypes = lib.ds_sel_oracle_score_blocks.argtypes
    lib.ds_sel_oracle_attend.restype = ctypes.c_int
    lib.ds_sel_oracle_quantize_q8.restype = ctypes.c_int
    lib.ds_sel_oracle_quantize_q8.argtypes = [i32, i64, i32, p, i64, i64, p, i64, i64, p, i64, i64]
    lib.ds_sel_oracle_select_q8.restype = ctypes.c_int
    lib.ds_sel_oracle_select_q8.argtypes = [i32, i32, i32, i32, i64, i32, p, p, p, i64, i64, p, i64,
                                            i64, p, i64, i64, p, p, p, p]
    lib.ds_sel_oracle_score_blocks_q8.restype = ctypes.c_int
    lib.ds_sel_oracle_score_blocks_q8.argtypes = [i32, i32, i32, i32, i64, p, p, p, i64, i64, p, i64,
                                                  i64, i32, i32, i64, p, p]
    lib.ds_sel_oracle_attend.argtypes = [i32, i32, i32, i32, i64, i32, p, p, i64, i64, p, i64, i64,
                                         p, p, ctypes.c_double, p]
    return lib


def load(path: str | None = None):
    """Load the compiled oracle (building it first if it is missing)."""
    global _lib
    if path is not None:
        return _declare(ctypes.CDLL(path))
    if _lib is None:
        if not os.path.exists(LIBRARY):
            build()
        _lib = _declare(ctypes.CDLL(LIBRARY))
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


class OracleError(RuntimeError):
    pass


def _shapes(q, w, keys, mask):
    if q.ndim != 4:
        raise ValueError("q must be [layers][rows][heads][dim]")
    layers, rows, heads, dim = q.shape
    if w.shape != (layers, rows, heads):
        raise ValueError("w must be [layers][rows][heads]")
    if keys.ndim != 3 or keys.shape[0] != layers or keys.shape[2] < dim:
        raise ValueError("keys must be [layers][blocks][ldk] with ldk >= dim")
    blocks, ldk = keys.shape[1], keys.shape[2]
    mrow = mlayer = 0
    if mask is not None:
        if mask.ndim != 3 or mask.shape[0] != layers or mask.shape[1] not in (1, rows):
            raise ValueError("mask must be [layers][rows or 1][words]")
        if mask.shape[2] * 32 < blocks:
            raise ValueError("mask rows need ceil(blocks/32) words")
        mrow = 0 if mask.shape[1] == 1 else mask.shape[2]
        mlayer = mask.shape[1] * mask.shape[2]
    return layers, rows, heads, dim, blocks, ldk, mrow, mlayer


def select(q, w, keys, k, mask=None, limit=None, lib=None, score="linear"):
    """Top-k selection for every (layer, row).

    score "linear": sum_h w_h (q_h . K); "relu": sum_h w_h max(q_h . K, 0)
    (the per-head ReLU variant, ds_sel_oracle_select_relu).

    q     uint16 [L][R][H][d]   bf16 bits
    w     uint16 [L][R][H]      bf16 bits
    keys  uint16 [L][N][ldk]    bf16 bits (ldk >= d; columns past d unused)
    mask  uint32 [L][R or 1][words] or None (one shared row when the middle
          dimension is 1)
    limit int32 [L][R] or None
    Returns (idx int32 [L][R][k], score float32 [L][R][k], count int32 [L][R]).
    """
    q, w, keys = _c(q, np.uint16), _c(w, np.uint16), _c(keys, np.uint16)
    mask, limit = _c(mask, np.uint32), _c(limit, np.int32)
    layers, rows, heads, dim, blocks, ldk, mrow, mlayer = _shapes(q, w, keys, mask)
    if limit is not None and limit.shape != (layers, rows):
        raise ValueError("limit must be [layers][rows]")
    idx = np.empty((layers, rows, k), np.int32)
    scores = np.empty((layers, rows, k), np.float32)
    count = np.empty((layers, rows), np.int32)
    lib = lib or load()
    fn = _scored(lib, "ds_sel_oracle_select", score)
    rc = fn(layers, rows, heads, dim, blocks, k, _ptr(q), _ptr(w), _ptr(keys), ldk, blocks * ldk,
            _ptr(mask), mrow, mlayer, _ptr(limit), _ptr(idx), _ptr(scores), _ptr(count))
    if rc != 0:
        raise OracleError(f"{fn.__name__} returned {rc}")
    return idx, scores, count


def decode_serial(q, w, keys, k, mask=None, limit=None, lib=None, score="linear"):
    """Serial decode over the layers (each layer's query depends on the one before).

    The pages' layers feed each other through the model (page "DeepSeek V4.1F
    Q4 on M3 Ultra with native DSpark MTP (40tps / 800tps)", paragraph
    "Decode"); the model is not part of this library, so a stand-in step links
    the layers: layer 0 selects with q[0]; for l >= 1, row r selects with its
    query heads rotated by its predecessor's best block,
        q_l[r][h] = q[l][r][(h + s) mod H],  s = idx[l-1][r][0] mod H
    (s = 0 when layer l-1 selected nothing for row r).  Inputs and outputs as
    select(); returns (idx, score, count) for every layer.
    """
    q = _c(q, np.uint16)
    L, R, H, _ = q.shape
    idx = np.empty((L, R, k), np.int32)
    scores = np.empty((L, R, k), np.float32)
    count = np.empty((L, R), np.int32)
    lib = lib or load()
    cur = q[0:1]
    for l in range(L):
        if l > 0:
            cur = np.empty_like(q[l:l + 1])
            for r in range(R):
                s = int(idx[l - 1, r, 0]) % H if count[l - 1, r] > 0 else 0
                cur[0, r] = np.roll(q[l, r], -s, axis=0)
        sl = slice(l, l + 1)
        out = select(cur, w[sl], keys[sl], k, None if mask is None else mask[sl],
                     None if limit is None else limit[sl], lib=lib, score=score)
        idx[l], scores[l], count[l] = out[0][0], out[1][0], out[2][0]
    return idx, scores, count


def _scored(lib, name, score):
    if score == "linear":
        return getattr(lib, name)
    if score == "relu":
        return getattr(lib, name + "_relu")
    raise ValueError("score must be 'linear' or 'relu'")


def score_blocks(q, w, keys, layer, row, blocks_list, lib=None, score="linear"):
    """fp32 scores (the oracle's fixed order) of the listed blocks of one (layer, row)."""
    q, w, keys = _c(q, np.uint16), _c(w, np.uint16), _c(keys, np.uint16)
    lst = _c(blocks_list, np.int32)
    layers, rows, heads, dim, blocks, ldk, _, _ = _shapes(q, w, keys, None)
    out = np.empty(lst.shape[0], np.float32)
    lib = lib or load()
    fn = _scored(lib, "ds_sel_oracle_score_blocks", score)
    rc = fn(layers, rows, heads, dim, blocks, _ptr(q), _ptr(w), _ptr(keys), ldk, blocks * ldk, layer,
            row, lst.shape[0], _ptr(lst), _ptr(out))
    if rc != 0:
        raise OracleError(f"{fn.__name__} returned {rc}")
    return out


def quantize_q8(keys, lib=None):
    """The 8-bit key stream of bf16 keys [L][N][ldk] (columns past d = ldk are
    all used: pass exactly [L][N][d]).  Returns (codes int8 [L][N][d], scales
    uint16 fp16 bits [L][N][d/32])."""
    keys = _c(keys, np.uint16)
    L, N, d = keys.shape
    codes = np.empty((L, N, d), np.int8)
    scales = np.empty((L, N, d // 32), np.uint16)
    lib = lib or load()
    rc = lib.ds_sel_oracle_quantize_q8(L, N, d, _ptr(keys), d, N * d, _ptr(codes), d, N * d,
                                       _ptr(scales), d // 32, N * (d // 32))
    if rc != 0:
        raise OracleError(f"ds_sel_oracle_quantize_q8 returned {rc}")
    return codes, scales


def _q8_shapes(q, codes, scales):
    layers, rows, heads, dim = q.shape
    if codes.ndim != 3 or codes.shape[0] != layers or codes.shape[2] != dim:
        raise ValueError("codes must be [layers][blocks][dim]")
    if scales.shape != (layers, codes.shape[1], dim // 32):
        raise ValueError("scales must be [layers][blocks][dim/32]")
    return codes.shape[1]


def select_q8(q, w, codes, scales, k, mask=None, limit=None, lib=None):
    """Top-k selection on the 8-bit key stream (codes int8 [L][N][d], scales
    fp16 bits [L][N][d/32]); otherwise as select()."""
    q, w = _c(q, np.uint16), _c(w, np.uint16)
    codes, scales = _c(codes, np.int8), _c(scales, np.uint16)
    mask, limit = _c(mask, np.uint32), _c(limit, np.int32)
    layers, rows, heads, dim = q.shape
    blocks = _q8_shapes(q, codes, scales)
    mrow = mlayer = 0
    if mask is not None:
        mrow = 0 if mask.shape[1] == 1 else mask.shape[2]
        mlayer = mask.shape[1] * mask.shape[2]
    idx = np.empty((layers, rows, k), np.int32)
    score = np.empty((layers, rows, k), np.float32)
    count = np.empty((layers, rows), np.int32)
    lib = lib or load()
    rc = lib.ds_sel_oracle_select_q8(layers, rows, heads, dim, blocks, k, _ptr(q), _ptr(w), _ptr(codes),
                                     dim, blocks * dim, _ptr(scales), dim // 32, blocks * (dim // 32),
                                     _ptr(mask), mrow, mlayer, _ptr(limit), _ptr(idx), _ptr(score),
                                     _ptr(count))
    if rc != 0:
        raise OracleError(f"ds_sel_oracle_select_q8 returned {rc}")
    return idx, score, count


def score_blocks_q8(q, w, codes, scales, layer, row, blocks_list, lib=None):
    """q8 scores (the oracle's fixed order) of the listed blocks of one (layer, row)."""
    q, w = _c(q, np.uint16), _c(w, np.uint16)
    codes, scales = _c(codes, np.int8), _c(scales, np.uint16)
    lst = _c(blocks_list, np.int32)
    layers, rows, heads, dim = q.shape
    blocks = _q8_shapes(q, codes, scales)
    out = np.empty(lst.shape[0], np.float32)
    lib = lib or load()
    rc = lib.ds_sel_oracle_score_blocks_q8(layers, rows, heads, dim, blocks, _ptr(q), _ptr(w),
                                           _ptr(codes), dim, blocks * dim, _ptr(scales), dim // 32,
                                           blocks * (dim // 32), layer, row, lst.shape[0], _ptr(lst),
                                           _ptr(out))
    if rc != 0:
        raise OracleError(f"ds_sel_oracle_score_blocks_q8 returned {rc}")
    return out


def attend(qa, keys, values, idx, count, scale, lib=None):
    """Attention over the selected blocks, in double precision.

    qa     uint16 [L][R][Ha][d]  bf16 bits (attention query heads)
    keys   uint16 [L][N][ldk]    bf16 bits (the block keys the selection scores)
    values uint16 [L][N][ldv]    bf16 bits
    idx    int32 [L][R][k]       selected blocks; entries past count are not read
    count  int32 [L][R]
    Returns out float64 [L][R][Ha][d]: per head, the softmax over the selected
    blocks of scale * (q . K[b]) applied to V[b]; zero where count is 0.
    """
    qa, keys, values = _c(qa, np.uint16), _c(keys, np.uint16), _c(values, np.uint16)
    idx, count = _c(idx, np.int32), _c(count, np.int32)
    layers, rows, heads, dim = qa.shape
    blocks, ldk, ldv, k = keys.shape[1], keys.shape[2], values.shape[2], idx.shape[2]
    if keys.shape[0] != layers or values.shape[:2] != keys.shape[:2] or idx.shape[:2] != (layers, rows):
        raise ValueError("inconsistent shapes")
    out = np.empty((layers, rows, heads, dim), np.float64)
    lib = lib or load()
    rc = lib.ds_sel_oracle_attend(layers, rows, heads, dim, blocks, k, _ptr(qa), _ptr(keys), ldk,
                                  blocks * ldk, _ptr(values), ldv, blocks * ldv, _ptr(idx),
                                  _ptr(count), float(scale), _ptr(out))
    if rc != 0:
        raise OracleError(f"ds_sel_oracle_attend returned {rc}")
    return out
