"""Seeded synthetic inputs for compressed-attention block selection.

This module only draws inputs.  It holds none of the selection arithmetic
(no admission test, no score, no ordering), so both the GPU path and the CPU
oracle can be fed from it without sharing any of the method.

The pages run whole-model decode on their own agent turns and code and print
no kernel-level inputs, so every workload here is synthetic.  The shapes come
from the pages' setting -- page "DeepSeek V4.1F Q4 on M3 Ultra with native
DSpark MTP (40tps / 800tps)": 512 blocks kept per layer ("Decode at depth"),
8k and 300k contexts (the results table), a 6-row speculative verify
("DSpark") -- with 4 tokens per compressed block, 64 index heads and
128-dimensional bf16 block keys as this library's reading.

Recipes (values are drawn in fp32 with numpy's PCG64 ``default_rng(seed)`` in
the order q, w, K, heavy-hitter set, mask, and rounded to bf16 with
round-to-nearest-even):

=========  ==  =  ==  ===  ======  =====================================================
name       L   R  H   d    N       values / admission
=========  ==  =  ==  ===  ======  =====================================================
tiny       1   1  4   64   4096    q, K, w integers uniform in [-3, 3]; limit = N
8k         1   1  64  128  2048    q, K ~ N(0,1), w ~ U(0,1); limit = N
300k       1   1  64  128  75000   as 8k; 5% of K rows (3750, without replacement) x4;
                                   Bernoulli(0.6) mask AND limit = N
verify     1   6  64  128  32768   as 8k per row; limit_r = N - 5 + r; no mask
verify_int 1   6  64  128  32768   q, K, w integers in [-3, 3]; limit_r = N - 5 + r
300k_x43   43  1  64  128  75000   43 independent layers, each drawn like 300k
sweep      43  6  64  128  75000   K, q in {-1,0,1}, w in {0,1}; layer l has one mask shared
                                   by its rows, Bernoulli(p_l), p_l = 0.1 + 0.9 l / 42;
                                   limit_r = N - 5 + r
=========  ==  =  ==  ===  ======  =====================================================

k = 512 everywhere.  Seeds: tiny 0, 8k 1, 300k 2, verify 3, verify_int 3,
sweep 4.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

BF16_ONE = 0x3F80
BF16_MINUS_ONE = 0xBF80


def f32_to_bf16_bits(x) -> np.ndarray:
    """Round finite fp32 values to bf16 (nearest, ties to even); return the bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    bias = ((u >> 16) & 1) + 0x7FFF
    return ((u + bias) >> 16).astype(np.uint16)


def bf16_bits_to_f32(bits) -> np.ndarray:
    """Widen bf16 bit patterns to fp32 values (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def small_int_bits(values) -> np.ndarray:
    """bf16 bits of small integers (|v| <= 256 are exact in bf16)."""
    return f32_to_bf16_bits(np.asarray(values, dtype=np.float32))


def pack_mask(bits_bool: np.ndarray) -> np.ndarray:
    """Pack booleans [..., N] into uint32 words [..., ceil(N/32)], bit b%32 of word b//32."""
    n = bits_bool.shape[-1]
    words = max(1, (n + 31) // 32)
    padded = np.zeros(bits_bool.shape[:-1] + (words * 32,), dtype=bool)
    padded[..., :n] = bits_bool
    packed = np.packbits(padded, axis=-1, bitorder="little")
    return np.ascontiguousarray(packed).view("<u4").astype(np.uint32)


@dataclass
class Problem:
    """One selection call's inputs (host numpy; bf16 as uint16 bits)."""

    name: str
    k: int
    q: np.ndarray                      # uint16 [L][R][H][d]
    w: np.ndarray                      # uint16 [L][R][H]
    keys: np.ndarray                   # uint16 [L][N][ldk]
    mask: Optional[np.ndarray] = None  # uint32 [L][R or 1][words]
    limit: Optional[np.ndarray] = None  # int32 [L][R]
    integer_valued: bool = False       # every bf16 value is a small integer
    meta: dict = field(default_factory=dict)

    @property
    def layers(self):
        return self.q.shape[0]

    @property
    def rows(self):
        return self.q.shape[1]

    @property
    def heads(self):
        return self.q.shape[2]

    @property
    def dim(self):
        return self.q.shape[3]

    @property
    def blocks(self):
        return self.keys.shape[1]

    @property
    def ldk(self):
        return self.keys.shape[2]


def _normal_bits(rng, shape):
    return f32_to_bf16_bits(rng.standard_normal(shape, dtype=np.float32))


def _uniform01_bits(rng, shape):
    return f32_to_bf16_bits(rng.random(shape, dtype=np.float32))


def _int_bits(rng, shape, lo, hi):
    """Uniform integers in [lo, hi] as bf16 bits, via a lookup table."""
    table = small_int_bits(np.arange(lo, hi + 1))
    return table[rng.integers(0, hi - lo + 1, size=shape, dtype=np.int16)]


def _causal_limits(layers, rows, n):
    lim = np.empty((layers, rows), np.int32)
    for r in range(rows):
        lim[:, r] = n - (rows - 1) + r
    return lim


def make(name: str, **overrides) -> Problem:
    """Build one of the named workloads (see the module docstring)."""
    name = name.lower()
    if name == "tiny":
        rng = np.random.default_rng(overrides.get("seed", 0))
        L, R, H, d, N = 1, 1, 4, 64, 4096
        q = _int_bits(rng, (L, R, H, d), -3, 3)
        w = _int_bits(rng, (L, R, H), -3, 3)
        keys = _int_bits(rng, (L, N, d), -3, 3)
        return Problem("tiny", 512, q, w, keys, None, np.full((L, R), N, np.int32), True,
                       {"seed": 0})
    if name == "8k":
        rng = np.random.default_rng(overrides.get("seed", 1))
        L, R, H, d, N = 1, 1, 64, 128, 2048
        q = _normal_bits(rng, (L, R, H, d))
        w = _uniform01_bits(rng, (L, R, H))
        keys = _normal_bits(rng, (L, N, d))
        return Problem("8k", 512, q, w, keys, None, np.full((L, R), N, np.int32), False,
                       {"seed": 1})
    if name == "300k":
        rng = np.random.default_rng(overrides.get("seed", 2))
        L, R, H, d, N = 1, 1, 64, 128, overrides.get("blocks", 75000)
        q = _normal_bits(rng, (L, R, H, d))
        w = _uniform01_bits(rng, (L, R, H))
        kf = bf16_bits_to_f32(_normal_bits(rng, (L, N, d)))
        heavy = rng.choice(N, size=int(0.05 * N), replace=False)
        kf[:, heavy, :] *= 4.0                      # power of two: exact in bf16
        keys = f32_to_bf16_bits(kf)
        mask = pack_mask((rng.random(N) < 0.6)[None, None, :])
        return Problem("300k", 512, q, w, keys, mask, np.full((L, R), N, np.int32), False,
                       {"seed": 2, "heavy": heavy.size, "p": 0.6})
    if name == "300k_x43":
        # 43 distinct 300k problems (one row each) in one call: the batched form
        # of the 300k config.  Each layer is drawn like the 300k config, all from
        # one generator: q, w, then per layer K, its heavy set and its mask.
        rng = np.random.default_rng(overrides.get("seed", 2))
        L = overrides.get("layers", 43)
        R, H, d, N = 1, 64, 128, overrides.get("blocks", 75000)
        q = _normal_bits(rng, (L, R, H, d))
        w = _uniform01_bits(rng, (L, R, H))
        keys = np.empty((L, N, d), np.uint16)
        bits = np.empty((L, 1, N), bool)
        for l in range(L):
            kf = bf16_bits_to_f32(_normal_bits(rng, (N, d)))
            kf[rng.choice(N, size=int(0.05 * N), replace=False), :] *= 4.0
            keys[l] = f32_to_bf16_bits(kf)
            bits[l, 0] = rng.random(N) < 0.6
        return Problem("300k_x43", 512, q, w, keys, pack_mask(bits), np.full((L, R), N, np.int32),
                       False, {"seed": 2, "p": 0.6})
    if name in ("verify", "verify_int"):
        rng = np.random.default_rng(overrides.get("seed", 3))
        L, R, H, d, N = 1, 6, 64, 128, 32768
        if name == "verify":
            q = _normal_bits(rng, (L, R, H, d))
            w = _uniform01_bits(rng, (L, R, H))
            keys = _normal_bits(rng, (L, N, d))
        else:
            q = _int_bits(rng, (L, R, H, d), -3, 3)
            w = _int_bits(rng, (L, R, H), -3, 3)
            keys = _int_bits(rng, (L, N, d), -3, 3)
        return Problem(name, 512, q, w, keys, None, _causal_limits(L, R, N),
                       name == "verify_int", {"seed": 3})
    if name == "sweep":
        rng = np.random.default_rng(overrides.get("seed", 4))
        L = overrides.get("layers", 43)
        R, H, d, N = 6, 64, 128, overrides.get("blocks", 75000)
        q = _int_bits(rng, (L, R, H, d), -1, 1)
        w = _int_bits(rng, (L, R, H), 0, 1)
        keys = _int_bits(rng, (L, N, d), -1, 1)
        ps = [0.1 + 0.9 * l / 42.0 for l in range(L)]
        bits = np.stack([rng.random(N) < p for p in ps])[:, None, :]
        mask = pack_mask(bits)
        return Problem("sweep", 512, q, w, keys, mask, _causal_limits(L, R, N), True,
                       {"seed": 4, "p": ps})
    raise KeyError(f"unknown workload {name!r}")


def make_custom(layers, rows, heads, dim, blocks, k, *, seed, values="normal", ldk=None,
                mask_p=None, mask_shared=True, limits=None, name="custom") -> Problem:
    """A workload of any shape for edge-case tests.

    values: "normal" (q, K ~ N(0,1), w ~ U(0,1)), "int3" (integers in [-3,3]),
            "ternary" (K, q in {-1,0,1}, w in {0,1}), "zero_keys" (K = 0) or
            "const_keys" (every K row equal).
    mask_p: None for no mask, else the Bernoulli admission probability.
    limits: None, an int for every row, or an int array [layers][rows].
    """
    rng = np.random.default_rng(seed)
    ldk = dim if ldk is None else ldk
    L, R, H, d, N = layers, rows, heads, dim, blocks
    integer = values in ("int3", "ternary", "zero_keys")
    if values == "normal":
        q = _normal_bits(rng, (L, R, H, d))
        w = _uniform01_bits(rng, (L, R, H))
        keys = _normal_bits(rng, (L, N, ldk))
    elif values == "int3":
        q = _int_bits(rng, (L, R, H, d), -3, 3)
        w = _int_bits(rng, (L, R, H), -3, 3)
        keys = _int_bits(rng, (L, N, ldk), -3, 3)
    elif values == "ternary":
        q = _int_bits(rng, (L, R, H, d), -1, 1)
        w = _int_bits(rng, (L, R, H), 0, 1)
        keys = _int_bits(rng, (L, N, ldk), -1, 1)
    elif values == "zero_keys":
        q = _int_bits(rng, (L, R, H, d), -3, 3)
        w = _int_bits(rng, (L, R, H), -3, 3)
        keys = np.zeros((L, N, ldk), np.uint16)
    elif values == "const_keys":
        q = _normal_bits(rng, (L, R, H, d))
        w = _uniform01_bits(rng, (L, R, H))
        row = _normal_bits(rng, (1, 1, ldk))
        keys = np.ascontiguousarray(np.broadcast_to(row, (L, N, ldk)))
    else:
        raise KeyError(values)
    if ldk > d:   # columns past d are never read; fill them with NaN bits to prove it
        keys[:, :, d:] = 0x7FC0
    mask = None
    if mask_p is not None:
        mrows = 1 if mask_shared else R
        mask = pack_mask(rng.random((L, mrows, N)) < mask_p)
    lim = None
    if limits is not None:
        lim = np.broadcast_to(np.asarray(limits, np.int32), (L, R)).copy()
    return Problem(name, k, q, w, keys, mask, lim, integer, {"seed": seed})


# ------------------------------------------------------------ attention over a selection
#
# The attention step reads, besides the selection and the block keys K, a
# query per attention head and a value row per block.  The pages give neither;
# this library's recipe: Ha = 64 attention heads of dimension d, the
# attention queries qa ~ N(0,1) and the values V ~ N(0,1), drawn in that order
# from default_rng(seed + 100) and rounded to bf16 (nearest, ties to even).

def random_q8_stream(layers, blocks, dim, *, seed, scale_exponents=None, scale_range=(1e-3, 0.05)):
    """A random 8-bit key stream: codes int8 [L][N][d] uniform in [-127, 127]
    and scales as fp16 bits [L][N][d/32], either 2**e with e drawn uniformly
    from the integer range `scale_exponents` (lo, hi inclusive; dequantised
    keys then exact in bf16 and every product exact) or uniform over
    `scale_range` rounded to fp16."""
    rng = np.random.default_rng(seed)
    codes = rng.integers(-127, 128, (layers, blocks, dim)).astype(np.int8)
    shape = (layers, blocks, dim // 32)
    if scale_exponents is not None:
        lo, hi = scale_exponents
        sc = (np.float32(2.0) ** rng.integers(lo, hi + 1, shape)).astype(np.float16)
    else:
        sc = rng.uniform(scale_range[0], scale_range[1], shape).astype(np.float16)
    return codes, sc.view(np.uint16)


def attend_inputs(layers, rows, heads, dim, blocks, *, seed, ldv=None):
    """(qa [L][R][Ha][d], values [L][N][ldv]) as bf16 bits; columns past d hold NaN bits."""
    rng = np.random.default_rng(seed + 100)
    ldv = dim if ldv is None else ldv
    qa = _normal_bits(rng, (layers, rows, heads, dim))
    values = _normal_bits(rng, (layers, blocks, ldv))
    if ldv > dim:
        values[:, :, dim:] = 0x7FC0
    return qa, values


def random_selection(layers, rows, blocks, k, *, seed, count=None):
    """A selection in the layout the selection returns: idx [L][R][k] int32 of
    distinct blocks in random order, -1 past count, and count [L][R] int32.
    count: None (min(k, N) everywhere), an int, or an int array [L][R]."""
    rng = np.random.default_rng(seed + 200)
    if count is None:
        count = min(k, blocks)
    cnt = np.broadcast_to(np.asarray(count, np.int32), (layers, rows)).copy()
    idx = np.full((layers, rows, k), -1, np.int32)
    for l in range(layers):
        for r in range(rows):
            c = int(cnt[l, r])
            if c > 0:
                idx[l, r, :c] = rng.choice(blocks, size=c, replace=False)
    return idx, cnt
