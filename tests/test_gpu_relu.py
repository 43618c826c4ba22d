"""GPU parity of the per-head ReLU score, sum_h w_h max(q_h . K, 0), through
the C ABI (a handle created with DS_SEL_FLAG_HEAD_RELU) against the oracle's
ReLU selection.  Integer-valued inputs: bit-exact (every dot product, clamp,
weight and sum is an exact integer in fp32).  General inputs: the tolerance
and set-acceptance rule of tests/gpu_support.py with the oracle's ReLU
per-block scores."""
import numpy as np
import pytest

import oracle
from sparse_attention_block_ds_amd import selector as sel
from sparse_attention_block_ds_amd import workloads as wl
from tests import gpu_support as gs
from tests import test_gpu_parity as tp

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def selector():
    import torch
    assert torch.cuda.is_available(), "the gpu tests need a GPU"
    s = sel.Selector(max_layers=43, max_rows=8, max_heads=64, max_dim=256, max_blocks=75000,
                     max_k=2048, score="relu")
    yield s
    s.close()


def _print(name, p):
    print(f"\n[case] relu {name}: L={p.layers} R={p.rows} H={p.heads} d={p.dim} N={p.blocks} k={p.k} "
          f"mask={'none' if p.mask is None else p.mask.shape}", flush=True)


def _scorer(p):
    return lambda l, r, blocks: oracle.score_blocks(p.q, p.w, p.keys, l, r, blocks, score="relu")


EXACT = [
    dict(name="tiny_shape", args=(1, 1, 4, 64, 4096, 512), kw=dict(values="int3")),
    dict(name="verify_int_shape", args=(1, 6, 64, 128, 32768, 512),
         kw=dict(values="int3", limits=np.array([[32768 - 5 + r for r in range(6)]]))),
    dict(name="shared_mask", args=(2, 3, 16, 128, 4097, 512), kw=dict(values="int3", mask_p=0.5)),
    dict(name="per_row_mask", args=(2, 6, 16, 128, 9000, 512),
         kw=dict(values="int3", mask_p=0.3, mask_shared=False)),
    dict(name="ternary_ties", args=(3, 6, 64, 128, 20000, 512),
         kw=dict(values="ternary", mask_p=0.5, limits=np.array([[20000 - 5 + r for r in range(6)]]))),
    dict(name="heads_20", args=(1, 3, 20, 64, 3000, 256), kw=dict(values="int3")),
    dict(name="heads_1", args=(1, 2, 1, 128, 3000, 64), kw=dict(values="int3")),
    dict(name="dim32", args=(1, 3, 8, 32, 2500, 128), kw=dict(values="int3")),
    dict(name="dim256", args=(1, 3, 16, 256, 2500, 128), kw=dict(values="int3")),
    dict(name="k_one", args=(2, 3, 8, 64, 3000, 1), kw=dict(values="int3", mask_p=0.5)),
    dict(name="k_2048", args=(1, 2, 8, 128, 6000, 2048), kw=dict(values="int3", mask_p=0.7)),
    dict(name="n_zero", args=(2, 3, 8, 64, 0, 16), kw=dict(values="int3")),
    dict(name="n_one", args=(1, 1, 8, 64, 1, 512), kw=dict(values="int3")),
    dict(name="zero_keys", args=(1, 2, 8, 64, 5000, 512), kw=dict(values="zero_keys")),
] + [dict(name=f"rows{r}", args=(1, r, 16, 64, 2100, 100), kw=dict(values="int3", mask_p=0.8))
     for r in range(1, 9)]


@pytest.mark.parametrize("case", EXACT, ids=[c["name"] for c in EXACT])
def test_relu_integer_bit_exact(selector, case):
    p = wl.make_custom(*case["args"], seed=900 + EXACT.index(case), **case["kw"])
    _print(case["name"], p)
    gpu = gs.run_gpu(selector, p)
    gs.assert_self_consistent(p, gpu)
    gs.assert_bit_exact(gpu, gs.run_oracle(p, score="relu"), case["name"])


@pytest.mark.parametrize("name", ["8k", "300k", "verify"])
def test_relu_general_workloads(selector, name):
    p = wl.make(name)
    _print(name, p)
    gpu = gs.run_gpu(selector, p)
    gs.assert_self_consistent(p, gpu)
    gs.assert_general(p, gpu, gs.run_oracle(p, score="relu"), scorer=_scorer(p))


@pytest.mark.parametrize("kw", [dict(), dict(mask_p=0.4, mask_shared=False)], ids=["nomask", "row_mask"])
def test_relu_general_custom(selector, kw):
    p = wl.make_custom(2, 4, 32, 128, 3000, 256, seed=950, **kw)
    _print("general_custom", p)
    gpu = gs.run_gpu(selector, p)
    gs.assert_self_consistent(p, gpu)
    gs.assert_general(p, gpu, gs.run_oracle(p, score="relu"), scorer=_scorer(p))


def test_relu_rescore_when_floor_too_high(selector):
    """The sampled blocks carry the top scores, so the floor lets too few candidates
    through and the select rescores the row under the ReLU score; still exact."""
    rng = np.random.default_rng(9)
    N = 20000
    col0 = 1.0 + rng.integers(0, 128, N) / 128.0
    sampled = gs.floor_sample_blocks(N)
    col0[sampled] = 2.0 + rng.integers(0, 128, len(sampled)) / 64.0
    p = tp._column0_problem("relu_rescore", col0, N)
    _print("rescore", p)
    gs.assert_bit_exact(gs.run_gpu(selector, p), gs.run_oracle(p, score="relu"), "relu_rescore")


def test_relu_unsupported_shape_leaves_outputs(selector):
    """8 rows of 64 heads at d = 128 do not fit the LDS stage: UNSUPPORTED, nothing written."""
    import torch
    p = wl.make_custom(1, 8, 64, 128, 1000, 64, seed=960, values="int3")
    q, w, keys, mask, limit = sel.upload(p)
    out = (torch.full((1, 8, 64), 7, dtype=torch.int32, device="cuda"),
           torch.full((1, 8, 64), 7.0, device="cuda"), torch.full((1, 8), 7, dtype=torch.int32, device="cuda"))
    with pytest.raises(sel.DsSelError) as err:
        selector.score_select(q, w, keys, p.k, mask, limit, out=out)
    assert err.value.status == sel.DS_SEL_E_UNSUPPORTED
    torch.cuda.synchronize()
    assert all(bool((t == 7).all()) for t in out)


def test_relu_noalloc_matches_handle(selector):
    import torch
    p = wl.make_custom(2, 6, 64, 128, 9000, 512, seed=961, values="int3", mask_p=0.6, mask_shared=False)
    q, w, keys, mask, limit = sel.upload(p)
    ref = [t.clone() for t in selector.score_select(q, w, keys, p.k, mask, limit)]
    out = (torch.empty_like(ref[0]), torch.empty_like(ref[1]), torch.empty_like(ref[2]))
    sel.score_select_noalloc(q, w, keys, p.k, mask, limit, out, score="relu")
    torch.cuda.synchronize()
    for a, b in zip(ref, out):
        assert torch.equal(a, b)


_SWEEP = {}


def test_relu_sweep_full_size_all_pairs(selector):
    """The 43 x 6 x 75,000 sweep under the ReLU score, every selection bit-exact."""
    if "p" not in _SWEEP:
        p = wl.make("sweep")
        pairs = [(l, r) for l in range(p.layers) for r in range(p.rows)]
        _SWEEP["p"] = p
        _SWEEP["ora"] = dict(zip(pairs, gs.oracle_pairs(p, pairs, score="relu")))
    p, ora = _SWEEP["p"], _SWEEP["ora"]
    _print("sweep", p)
    gpu = gs.run_gpu(selector, p)
    gs.assert_self_consistent(p, gpu)
    for (l, r), o in ora.items():
        got = tuple(x[l:l + 1, r:r + 1] for x in gpu)
        gs.assert_bit_exact(got, o, f"relu sweep l={l} r={r}")
