"""The entry point that allocates nothing (ds_sel_score_select_noalloc),
through the C ABI, against the handle entry point on the same inputs: two
calls in a row on the static scratch, the second with a smaller input, each
bit-identical to ds_sel_score_select (and, on these integer-valued inputs, to
the oracle); a call too large for the static scratch is refused untouched."""
import numpy as np
import pytest

from sparse_attention_block_ds_amd import selector as sel
from sparse_attention_block_ds_amd import workloads as wl
from tests import gpu_support as gs

pytestmark = pytest.mark.gpu


def _outs(p, torch, fill=-7):
    L, R, k = p.layers, p.rows, p.k
    return (torch.full((L, R, k), fill, dtype=torch.int32, device="cuda"),
            torch.full((L, R, k), float(fill), dtype=torch.float32, device="cuda"),
            torch.full((L, R), fill, dtype=torch.int32, device="cuda"))


@pytest.mark.parametrize("engine", ["mfma", "valu"])
def test_noalloc_matches_handle_twice(engine):
    import torch
    big = wl.make_custom(2, 6, 64, 128, 20000, 512, seed=901, values="int3", mask_p=0.6,
                         limits=np.array([[20000 - 5 + r for r in range(6)]] * 2))
    small = wl.make_custom(1, 3, 16, 64, 5000, 256, seed=902, values="ternary", mask_p=0.4,
                           mask_shared=False)
    h = sel.Selector(max_layers=2, max_rows=6, max_heads=64, max_dim=128, max_blocks=20000,
                     max_k=512, engine=engine)
    try:
        for p in (big, small):
            print(f"\n[case] noalloc {engine}: L={p.layers} R={p.rows} N={p.blocks} k={p.k}", flush=True)
            q, w, keys, mask, limit = sel.upload(p)
            want = h.score_select(q, w, keys, p.k, mask, limit)
            got = sel.score_select_noalloc(q, w, keys, p.k, mask, limit, _outs(p, torch), engine=engine)
            torch.cuda.synchronize()
            for a, b in zip(want, got):
                assert torch.equal(a, b)
            gs.assert_bit_exact(tuple(t.cpu().numpy() for t in got), gs.run_oracle(p), "noalloc")
    finally:
        h.close()


def test_noalloc_refuses_oversize_untouched():
    import torch
    p = wl.make_custom(1, 8, 4, 64, 1 << 20, 16, seed=903, values="int3")
    q, w, keys, mask, limit = sel.upload(p)
    out = _outs(p, torch, fill=7)
    with pytest.raises(sel.DsSelError) as e:
        sel.score_select_noalloc(q, w, keys, p.k, mask, limit, out)
    assert e.value.status == sel.DS_SEL_E_CAPACITY
    torch.cuda.synchronize()
    assert all(bool((t == 7).all()) for t in out)
