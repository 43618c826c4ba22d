"""Serial decode on the GPU (ds_sel_decode and its captured graph plan)
against the oracle's serial decode: 43 dependent layers, each layer's query
heads rotated by the previous layer's best block per row."""
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


def _print(name, p):
    print(f"\n[case] decode {name}: L={p.layers} R={p.rows} H={p.heads} d={p.dim} N={p.blocks} k={p.k}",
          flush=True)


def _host(out):
    return tuple(t.cpu().numpy() for t in out)


def _sweep_like(N=16384):
    L, R = 43, 6
    return wl.make_custom(L, R, 64, 128, N, 512, seed=1100, values="ternary", mask_p=0.6,
                          limits=np.array([[N - 5 + r for r in range(R)]] * L))


def test_decode_43_layers_bit_exact(selector):
    import torch
    p = _sweep_like()
    _print("sweep_like", p)
    q, w, keys, mask, limit = sel.upload(p)
    got = _host(selector.decode(q, w, keys, p.k, mask, limit))
    torch.cuda.synchronize()
    ora = oracle.decode_serial(p.q, p.w, p.keys, p.k, p.mask, p.limit)
    gs.assert_bit_exact(got, ora, "decode 43 layers")
    assert len({int(x) % p.heads for x in got[0][:-1, :, 0].ravel()}) > 1  # rotations exercised


def test_decode_general_inputs_layer_by_layer(selector):
    """300k-shaped layers with general values: each layer against the oracle
    given the GPU's own previous layer (so that a within-tolerance choice at one
    layer does not move every later one)."""
    import torch
    p = wl.make("300k_x43", blocks=20000)
    _print("300k_x43 (N=20000)", p)
    q, w, keys, mask, limit = sel.upload(p)
    idx, score, count = _host(selector.decode(q, w, keys, p.k, mask, limit))
    torch.cuda.synchronize()
    H = p.heads
    for l in range(p.layers):
        ql = p.q[l:l + 1].copy()
        if l > 0:
            for r in range(p.rows):
                s = int(idx[l - 1, r, 0]) % H if count[l - 1, r] > 0 else 0
                ql[0, r] = np.roll(p.q[l, r], -s, axis=0)
        sub = wl.Problem("layer", p.k, ql, p.w[l:l + 1], p.keys[l:l + 1], p.mask[l:l + 1],
                         p.limit[l:l + 1], False)
        ora = oracle.select(sub.q, sub.w, sub.keys, sub.k, sub.mask, sub.limit)
        gs.assert_general(sub, (idx[l:l + 1], score[l:l + 1], count[l:l + 1]), ora)


def test_decode_one_layer_is_the_selection(selector):
    import torch
    p = wl.make_custom(1, 6, 16, 128, 9000, 512, seed=1101, values="int3", mask_p=0.4,
                       mask_shared=False)
    q, w, keys, mask, limit = sel.upload(p)
    a = _host(selector.decode(q, w, keys, p.k, mask, limit))
    b = _host(selector.score_select(q, w, keys, p.k, mask, limit))
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)


def test_decode_plan_replays_match_eager(selector):
    """The captured plan, replayed three times with the program's own eager work
    and synchronisations in between, then again after the inputs change in place:
    every replay equals the eager decode of the inputs it saw."""
    import torch
    p = wl.make_custom(43, 3, 64, 128, 6000, 512, seed=1102, values="int3", mask_p=0.5,
                       mask_shared=False)
    _print("plan", p)
    q, w, keys, mask, limit = sel.upload(p)
    eager = [t.clone() for t in selector.decode(q, w, keys, p.k, mask, limit)]
    torch.cuda.synchronize()
    stream = torch.cuda.Stream()
    plan = selector.decode_plan(q, w, keys, p.k, mask, limit, stream=stream)
    other = wl.make_custom(2, 2, 8, 64, 3000, 64, seed=1103, values="int3")
    oq, ow, ok_, om, ol = sel.upload(other)
    try:
        for rep in range(3):
            for t in plan.out:
                t.fill_(-7)
            with torch.cuda.stream(stream):
                out = plan.launch(stream)
            stream.synchronize()
            for a, b in zip(eager, out):
                assert torch.equal(a, b), f"replay {rep}"
            selector.score_select(oq, ow, ok_, other.k, om, ol)  # eager work between replays
            torch.cuda.synchronize()
        # new contents in place: the plan reads them afresh
        p2 = wl.make_custom(43, 3, 64, 128, 6000, 512, seed=1104, values="int3", mask_p=0.5,
                            mask_shared=False)
        q2, w2, k2, m2, l2 = sel.upload(p2)
        q.copy_(q2), w.copy_(w2), keys.copy_(k2), mask.copy_(m2)
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            out = plan.launch(stream)
        stream.synchronize()
        got = tuple(t.cpu().numpy() for t in out)
        ora = oracle.decode_serial(p2.q, p2.w, p2.keys, p2.k, p2.mask, p2.limit)
        gs.assert_bit_exact(got, ora, "plan after in-place change")
    finally:
        plan.close()


def test_decode_empty_and_single_block(selector):
    import torch
    for N in (0, 1):
        p = wl.make_custom(5, 2, 8, 64, N, 16, seed=1105 + N, values="int3")
        q, w, keys, mask, limit = sel.upload(p)
        got = _host(selector.decode(q, w, keys, p.k, mask, limit))
        torch.cuda.synchronize()
        gs.assert_bit_exact(got, oracle.decode_serial(p.q, p.w, p.keys, p.k, p.mask, p.limit), f"N={N}")
