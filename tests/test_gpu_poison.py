"""Poisoned workspace: no call may depend on what an earlier call left in the
handle's scratch.  Before each call the scratch is filled with 0xFF, 0x00 or
0x5A (ds_sel_poison_scratch); the three outputs must be identical, and equal
to the oracle's where the inputs are integer-valued."""
import numpy as np
import pytest

from sparse_attention_block_ds_amd import selector as sel
from sparse_attention_block_ds_amd import workloads as wl
from tests import gpu_support as gs
from tests import test_gpu_parity as tp
from tests import test_gpu_q8 as tq

pytestmark = pytest.mark.gpu

BYTES = (0xFF, 0x00, 0x5A)


@pytest.fixture(scope="module", params=["mfma", "valu"])
def selector(request):
    import torch
    assert torch.cuda.is_available(), "the gpu tests need a GPU"
    s = sel.Selector(max_layers=43, max_rows=8, max_heads=64, max_dim=256, max_blocks=75000,
                     max_k=2048, engine=request.param)
    yield s
    s.close()


def _poisoned_runs(selector, run):
    import torch
    outs = []
    for b in BYTES:
        selector.poison_scratch(b)
        outs.append(run())
        torch.cuda.synchronize()
    for o in outs[1:]:
        for x, y in zip(outs[0], o):
            np.testing.assert_array_equal(x, y)
    return outs[0]


def _cases():
    rng = np.random.default_rng(9)
    N = 20000
    col0 = 1.0 + rng.integers(0, 128, N) / 128.0
    sampled = gs.floor_sample_blocks(N)
    col0[sampled] = 2.0 + rng.integers(0, 128, len(sampled)) / 64.0
    return [
        ("tiny", wl.make("tiny")),
        ("verify_int", wl.make("verify_int")),
        ("per_row_mask", wl.make_custom(2, 6, 16, 128, 9000, 512, seed=800, values="int3", mask_p=0.3,
                                        mask_shared=False)),
        ("ternary_ties", wl.make_custom(3, 6, 64, 128, 20000, 512, seed=801, values="ternary",
                                        mask_p=0.5)),
        ("rescore", tp._column0_problem("rescore", col0, N)),
        ("n_zero", wl.make_custom(2, 3, 8, 64, 0, 16, seed=802, values="int3")),
        ("k_2048", wl.make_custom(1, 2, 8, 128, 6000, 2048, seed=803, values="int3", mask_p=0.7)),
    ]


@pytest.mark.parametrize("name,p", _cases(), ids=[c[0] for c in _cases()])
def test_selection_independent_of_scratch(selector, name, p):
    print(f"\n[case] poison {name}: L={p.layers} R={p.rows} N={p.blocks} k={p.k}", flush=True)
    got = _poisoned_runs(selector, lambda: gs.run_gpu(selector, p))
    gs.assert_bit_exact(got, gs.run_oracle(p), name)


def test_q8_selection_independent_of_scratch(selector):
    p, codes, scales = tq._exact_case(804, 2, 6, 16, 128, 9000, 512, mask_p=0.5, mask_shared=False)
    print(f"\n[case] poison q8: N={p.blocks}", flush=True)
    got = _poisoned_runs(selector, lambda: gs.run_gpu_q8(selector, p, codes, scales))
    gs.assert_bit_exact(got, gs.run_oracle_q8(p, codes, scales), "q8")


def test_attention_independent_of_scratch(selector):
    """A single-layer call splits each row's selection over workgroups whose partial
    records live in the scratch: the merged output must not depend on its old contents."""
    import torch
    p = wl.make_custom(1, 6, 8, 128, 9000, 512, seed=805, values="int3")
    q, w, keys, mask, limit = sel.upload(p)
    idx, _, count = selector.score_select(q, w, keys, p.k, mask, limit)
    g = torch.Generator(device="cuda")
    g.manual_seed(7)
    qa = torch.randn((1, 6, 64, 128), generator=g, device="cuda").to(torch.bfloat16)
    values = torch.randn((1, 9000, 128), generator=g, device="cuda").to(torch.bfloat16)
    print("\n[case] poison attend", flush=True)
    _poisoned_runs(selector, lambda: (selector.attend(qa, keys, values, idx, count, 0.125)
                                      .cpu().numpy(),))
