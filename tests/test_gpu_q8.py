"""GPU parity of the 8-bit key stream, through the C ABI, against the oracle:
the quantise kernel (codes and scales bit for bit) and the selection over
codes and scales (bit-exact where every product and partial sum is exact in
fp32; otherwise the general tolerance and set-acceptance rule of
tests/gpu_support.py, with the oracle's 8-bit per-block scores)."""
import numpy as np
import pytest

import oracle
from sparse_attention_block_ds_amd import selector as sel
from sparse_attention_block_ds_amd import workloads as wl
from tests import gpu_support as gs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def selector():
    import torch
    assert torch.cuda.is_available(), "the gpu tests need a GPU"
    s = sel.Selector(max_layers=43, max_rows=8, max_heads=64, max_dim=256, max_blocks=75000,
                     max_k=2048)
    yield s
    s.close()


def _print(name, p, extra=""):
    print(f"\n[case] q8 {name}: L={p.layers} R={p.rows} H={p.heads} d={p.dim} N={p.blocks} k={p.k} "
          f"mask={'none' if p.mask is None else p.mask.shape} {extra}", flush=True)


def quantize_gpu(keys_bits, ldk=None):
    """keys_bits uint16 [L][N][d] -> (codes int8, scales fp16 bits) from the quantise kernel;
    with ldk the keys sit in a padded [L][N][ldk] buffer."""
    import torch
    L, N, d = keys_bits.shape
    host = keys_bits
    if ldk is not None:
        host = np.zeros((L, N, ldk), np.uint16)
        host[:, :, :d] = keys_bits
    dev = torch.from_numpy(np.ascontiguousarray(host).view(np.int16)).cuda().view(torch.bfloat16)
    codes, scales = sel.quantize_q8(dev[:, :, :d])
    torch.cuda.synchronize()
    return codes.cpu().numpy(), scales.cpu().numpy().view(np.uint16)


# ------------------------------------------------------------ the quantise kernel
def _special_keys(rng, L, N, d):
    """Normal keys with planted groups: all zero, one nonzero value, a scale that
    underflows fp16, large values, values on half-integer multiples of the scale."""
    kf = rng.standard_normal((L, N, d)).astype(np.float32)
    g = d // 32
    kf[0, 0, :32] = 0.0
    kf[0, 1, :] = 0.0
    kf[0, 1, 5] = -3.5
    kf[0, 2, :32] = 1e-30                      # amax / 127 below half the least fp16 subnormal
    kf[0, 3, :] *= 1e5                         # scales near the top of fp16
    if N > 4:
        kf[0, 4, :32] = np.arange(-16, 16) * 0.5  # x / s lands near half-integers
    if N > 5 and g > 1:
        kf[0, 5, 32:64] = 127.0                # amax / 127 = 1 exactly
    return wl.f32_to_bf16_bits(kf)


@pytest.mark.parametrize("L,N,d,ldk", [(1, 3000, 64, None), (2, 4097, 128, None),
                                       (1, 700, 32, None), (2, 1500, 256, None),
                                       (1, 2048, 128, 136), (3, 1, 64, None), (1, 0, 128, None)])
def test_quantize_bit_exact(L, N, d, ldk):
    print(f"\n[case] quantize L={L} N={N} d={d} ldk={ldk}", flush=True)
    rng = np.random.default_rng(500 + N + d)
    keys = _special_keys(rng, L, N, d) if N >= 4 else wl.f32_to_bf16_bits(
        rng.standard_normal((L, N, d)).astype(np.float32))
    got_c, got_s = quantize_gpu(keys, ldk)
    exp_c, exp_s = oracle.quantize_q8(keys)
    np.testing.assert_array_equal(got_s, exp_s)
    np.testing.assert_array_equal(got_c, exp_c)


# ------------------------------------------------------------ selection, exact inputs
def _exact_case(seed, L, R, H, d, N, k, exps=(-3, 0), **kw):
    p = wl.make_custom(L, R, H, d, N, k, seed=seed, values="int3", **kw)
    codes, scales = wl.random_q8_stream(L, N, d, seed=seed + 1, scale_exponents=exps)
    # Every product q w s c is a multiple of 2^lo; all partial sums on either side are
    # bounded by M = sum_h |w_h| sum_i |q_hi| |s c_i|, so M < 2^(24 + lo) makes both exact.
    if N > 0:
        q = np.abs(wl.bf16_bits_to_f32(p.q).astype(np.float64))
        w = np.abs(wl.bf16_bits_to_f32(p.w).astype(np.float64))
        kabs = np.abs(codes.astype(np.float64)) * np.repeat(
            scales.view(np.float16).astype(np.float64), 32, axis=-1)
        M = max(float(np.max(np.einsum("lrh,lrhd,lnd->lrn", w, q, kabs))), 0.0)
        assert M < 2.0 ** (24 + exps[0]), "inputs outside the exact range"
    return p, codes, scales


EXACT = [
    dict(name="basic", args=(1, 1, 8, 64, 3000, 512)),
    dict(name="shared_mask", args=(2, 3, 16, 128, 4097, 512), kw=dict(mask_p=0.5)),
    dict(name="per_row_mask_limits", args=(1, 4, 8, 128, 5000, 300),
         kw=dict(mask_p=0.6, mask_shared=False, limits=np.array([[5000, 2500, 17, 4999]]))),
    dict(name="dim32", args=(1, 3, 8, 32, 2500, 128)),
    dict(name="dim256_r3", args=(1, 3, 8, 256, 2500, 128), exps=(-3, -1)),
    dict(name="dim256_r6", args=(1, 6, 8, 256, 2100, 100), exps=(-3, -1)),
    dict(name="n_zero", args=(2, 3, 8, 64, 0, 16)),
    dict(name="n_one", args=(1, 1, 8, 64, 1, 512)),
    dict(name="k_one", args=(2, 3, 8, 64, 3000, 1), kw=dict(mask_p=0.5)),
    dict(name="k_2048", args=(1, 2, 8, 128, 6000, 2048), kw=dict(mask_p=0.7)),
    dict(name="verify_shape", args=(1, 6, 8, 128, 32768, 512),
         kw=dict(limits=np.array([[32768 - 5 + r for r in range(6)]]))),
] + [dict(name=f"rows{r}", args=(1, r, 8, 64, 2100, 100), kw=dict(mask_p=0.8)) for r in range(1, 9)]


@pytest.mark.parametrize("case", EXACT, ids=[c["name"] for c in EXACT])
def test_q8_exact_inputs_bit_exact(selector, case):
    p, codes, scales = _exact_case(600 + EXACT.index(case), *case["args"],
                                   exps=case.get("exps", (-3, 0)), **case.get("kw", {}))
    _print(case["name"], p)
    gpu = gs.run_gpu_q8(selector, p, codes, scales)
    gs.assert_self_consistent(p, gpu)
    gs.assert_bit_exact(gpu, gs.run_oracle_q8(p, codes, scales), case["name"])


def test_q8_zero_scales_tie_on_index(selector):
    """Every scale 0: every score is 0 and the selection is the admitted blocks in index order."""
    p, codes, scales = _exact_case(650, 1, 2, 8, 64, 5000, 512, mask_p=0.9)
    scales[:] = 0
    _print("zero_scales", p)
    gpu = gs.run_gpu_q8(selector, p, codes, scales)
    gs.assert_self_consistent(p, gpu)
    gs.assert_bit_exact(gpu, gs.run_oracle_q8(p, codes, scales), "zero_scales")


def test_q8_padded_rows(selector):
    """Codes and scales rows with padding (ldc = 72, lds = 3 at d = 64); the padding is never read."""
    import torch
    p, codes, scales = _exact_case(651, 2, 3, 8, 64, 3000, 256, mask_p=0.5)
    L, N, d = codes.shape
    cpad = np.full((L, N, 72), 127, np.int8)
    cpad[:, :, :d] = codes
    spad = np.full((L, N, 3), 0x7C00, np.uint16)  # an infinite scale in the padding
    spad[:, :, :2] = scales
    q, w, _, mask, limit = sel.upload(p)
    c, s = gs.upload_q8(cpad, spad)
    _print("padded_rows", p, "ldc=72 lds=3")
    idx, sc, cnt = selector.score_select_q8(q, w, c[:, :, :d], s[:, :, :2], p.k, mask, limit)
    torch.cuda.synchronize()
    gpu = (idx.cpu().numpy(), sc.cpu().numpy(), cnt.cpu().numpy())
    gs.assert_bit_exact(gpu, gs.run_oracle_q8(p, codes, scales), "padded_rows")


# ------------------------------------------------------------ selection, general inputs
def _quantised(p):
    """The 8-bit stream of p's keys, from the kernel, checked against the oracle's."""
    codes, scales = quantize_gpu(p.keys)
    exp_c, exp_s = oracle.quantize_q8(p.keys)
    np.testing.assert_array_equal(scales, exp_s)
    np.testing.assert_array_equal(codes, exp_c)
    return codes, scales


def _scorer(p, codes, scales):
    return lambda l, r, blocks: oracle.score_blocks_q8(p.q, p.w, codes, scales, l, r, blocks)


@pytest.mark.parametrize("name", ["8k", "300k", "verify"])
def test_q8_general_workloads(selector, name):
    p = wl.make(name)
    _print(name, p)
    codes, scales = _quantised(p)
    gpu = gs.run_gpu_q8(selector, p, codes, scales)
    gs.assert_self_consistent(p, gpu)
    gs.assert_general(p, gpu, gs.run_oracle_q8(p, codes, scales), scorer=_scorer(p, codes, scales))


@pytest.mark.parametrize("kw", [dict(), dict(mask_p=0.4, mask_shared=False),
                                dict(mask_p=0.7, limits=np.array([[3000, 1200, 5, 2999]]))],
                         ids=["nomask", "per_row_mask", "shared_mask_limits"])
def test_q8_general_custom(selector, kw):
    p = wl.make_custom(1, 4, 16, 128, 3000, 256, seed=660, **kw)
    _print("general_custom", p)
    codes, scales = _quantised(p)
    gpu = gs.run_gpu_q8(selector, p, codes, scales)
    gs.assert_self_consistent(p, gpu)
    gs.assert_general(p, gpu, gs.run_oracle_q8(p, codes, scales), scorer=_scorer(p, codes, scales))


def test_q8_sweep_full_size_sampled(selector):
    """The 43 x 6 x 75000 sweep on its 8-bit stream: the stream bit-exact, the
    invariants on every selection, the general rule on a sample."""
    p = wl.make("sweep")
    _print("sweep", p)
    codes, scales = _quantised(p)
    gpu = gs.run_gpu_q8(selector, p, codes, scales)
    gs.assert_self_consistent(p, gpu)
    for l, r in [(0, 0), (0, 5), (17, 3), (42, 0), (42, 5)]:
        sub = wl.Problem("s", p.k, p.q[l:l + 1, r:r + 1], p.w[l:l + 1, r:r + 1], p.keys[l:l + 1],
                         p.mask[l:l + 1], p.limit[l:l + 1, r:r + 1])
        sc, ss = codes[l:l + 1], scales[l:l + 1]
        got = tuple(x[l:l + 1, r:r + 1] for x in gpu)
        gs.assert_general(sub, got, gs.run_oracle_q8(sub, sc, ss), scorer=_scorer(sub, sc, ss))
