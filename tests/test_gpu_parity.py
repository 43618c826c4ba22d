"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Integer-valued inputs must match bit for bit; general inputs follow the
tolerance and set-acceptance rule in tests/gpu_support.py."""
import numpy as np
import pytest

from sparse_attention_block_ds_amd import selector as sel
from sparse_attention_block_ds_amd import workloads as wl
from tests import gpu_support as gs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", params=["mfma", "valu"])
def selector(request):
    import torch
    assert torch.cuda.is_available(), "the gpu tests need a GPU"
    s = sel.Selector(max_layers=43, max_rows=8, max_heads=64, max_dim=256, max_blocks=75000,
                     max_k=2048, engine=request.param)
    yield s
    s.close()


def _print_case(name, p):
    print(f"\n[case] {name}: L={p.layers} R={p.rows} H={p.heads} d={p.dim} N={p.blocks} k={p.k} "
          f"mask={'none' if p.mask is None else p.mask.shape} seed={p.meta.get('seed')}", flush=True)


# ------------------------------------------------------------ named workloads
def test_tiny_bit_exact(selector):
    p = wl.make("tiny")
    _print_case("tiny", p)
    gs.assert_bit_exact(gs.run_gpu(selector, p), gs.run_oracle(p), "tiny")


def test_verify_int_bit_exact(selector):
    p = wl.make("verify_int")
    _print_case("verify_int", p)
    gs.assert_bit_exact(gs.run_gpu(selector, p), gs.run_oracle(p), "verify_int")


@pytest.mark.parametrize("name", ["8k", "300k", "verify"])
def test_general_workloads(selector, name):
    p = wl.make(name)
    _print_case(name, p)
    gpu = gs.run_gpu(selector, p)
    gs.assert_self_consistent(p, gpu)
    gs.assert_general(p, gpu, gs.run_oracle(p))


_FULL = {}


def _full_size(name):
    """A full-size workload and the oracle's result for every (layer, row), computed
    once per module on a pool of host threads (the oracle runs without the GIL)."""
    if name not in _FULL:
        p = wl.make(name)
        pairs = [(l, r) for l in range(p.layers) for r in range(p.rows)]
        _FULL[name] = (p, dict(zip(pairs, gs.oracle_pairs(p, pairs))))
    return _FULL[name]


def test_sweep_full_size_all_pairs(selector):
    """All 43 x 6 selections of the sweep at full size, every one bit-exact."""
    p, ora = _full_size("sweep")
    _print_case("sweep", p)
    gpu = gs.run_gpu(selector, p)
    gs.assert_self_consistent(p, gpu)
    for (l, r), o in ora.items():
        got = tuple(x[l:l + 1, r:r + 1] for x in gpu)
        gs.assert_bit_exact(got, o, f"sweep l={l} r={r}")


def test_300k_x43_all_layers(selector):
    """The 300k config batched 43 layers to a call (one row each): every layer
    against the oracle under the general-input rule."""
    p, ora = _full_size("300k_x43")
    _print_case("300k_x43", p)
    gpu = gs.run_gpu(selector, p)
    gs.assert_self_consistent(p, gpu)
    for (l, r), o in ora.items():
        sub = gs.sub_problem(p, l, r)
        got = tuple(x[l:l + 1, r:r + 1] for x in gpu)
        gs.assert_general(sub, got, o)


# ------------------------------------------------------------ edge cases (integer: bit-exact)
EDGE = [
    dict(name="n_below_k", args=(1, 2, 8, 64, 300, 512), kw=dict(values="int3")),
    dict(name="n_one", args=(1, 1, 8, 64, 1, 512), kw=dict(values="int3")),
    dict(name="n_zero", args=(2, 3, 8, 64, 0, 16), kw=dict(values="int3")),
    dict(name="ragged_shared_mask", args=(2, 3, 16, 128, 4097, 512), kw=dict(values="int3", mask_p=0.5)),
    dict(name="empty_mask", args=(1, 2, 8, 64, 3000, 64), kw=dict(values="int3", mask_p=0.0)),
    dict(name="limit_zero", args=(1, 3, 8, 64, 3000, 64), kw=dict(values="int3", limits=0)),
    dict(name="limits_clamped", args=(1, 2, 8, 64, 2000, 256),
         kw=dict(values="int3", limits=np.array([[-5, 10 ** 7]]))),
    dict(name="all_equal_sort_path", args=(1, 2, 8, 64, 5000, 512), kw=dict(values="zero_keys")),
    dict(name="all_equal_fallback", args=(1, 2, 8, 64, 30000, 512),
         kw=dict(values="zero_keys", mask_p=0.9)),
    dict(name="per_row_mask", args=(2, 6, 16, 128, 9000, 512),
         kw=dict(values="int3", mask_p=0.3, mask_shared=False)),
    dict(name="per_row_mask_limits", args=(1, 4, 16, 128, 5000, 300),
         kw=dict(values="ternary", mask_p=0.6, mask_shared=False,
                 limits=np.array([[5000, 2500, 17, 4999]]))),
    dict(name="ldk_padded_nan", args=(1, 2, 8, 64, 3000, 128), kw=dict(values="int3", ldk=72)),
    dict(name="dim32", args=(1, 3, 8, 32, 2500, 128), kw=dict(values="int3")),
    dict(name="dim256", args=(1, 3, 8, 256, 2500, 128), kw=dict(values="int3")),
    dict(name="k_one", args=(2, 3, 8, 64, 3000, 1), kw=dict(values="int3", mask_p=0.5)),
    dict(name="k_2048", args=(1, 2, 8, 128, 6000, 2048), kw=dict(values="int3", mask_p=0.7)),
    dict(name="heads_one", args=(1, 2, 1, 128, 3000, 64), kw=dict(values="int3")),
    dict(name="ternary_ties", args=(3, 6, 64, 128, 20000, 512),
         kw=dict(values="ternary", mask_p=0.5, limits=np.array([[20000 - 5 + r for r in range(6)]]))),
] + [dict(name=f"rows{r}", args=(1, r, 8, 64, 2100, 100), kw=dict(values="int3", mask_p=0.8))
     for r in range(1, 9)]


@pytest.mark.parametrize("case", EDGE, ids=[c["name"] for c in EDGE])
def test_edge_cases_bit_exact(selector, case):
    p = wl.make_custom(*case["args"], seed=100 + EDGE.index(case), **case["kw"])
    _print_case(case["name"], p)
    gpu = gs.run_gpu(selector, p)
    gs.assert_self_consistent(p, gpu)
    gs.assert_bit_exact(gpu, gs.run_oracle(p), case["name"])


def test_fallback_with_distinct_keys(selector):
    """More than the LDS buffer in the boundary bin, with many distinct keys and ties:
    K[b][0] takes 128 values in [1, 2) and q~ picks only that column."""
    rng = np.random.default_rng(7)
    L, R, H, d, N, k = 1, 2, 2, 64, 40000, 512
    q = np.zeros((L, R, H, d), np.float32)
    q[:, :, 0, 0] = 1.0
    w = np.ones((L, R, H), np.float32)
    keys = np.zeros((L, N, d), np.float32)
    keys[0, :, 0] = 1.0 + rng.integers(0, 128, N) / 128.0
    p = wl.Problem("fallback", k, wl.f32_to_bf16_bits(q), wl.f32_to_bf16_bits(w),
                   wl.f32_to_bf16_bits(keys), None, None, True)
    _print_case("fallback_distinct", p)
    gs.assert_bit_exact(gs.run_gpu(selector, p), gs.run_oracle(p), "fallback_distinct")


def _column0_problem(name, col0, N, k=512, R=2):
    """q~ = e_0 for every row (one head, weight 1), so row scores are K[b][0]: exact."""
    L, H, d = 1, 1, 64
    q = np.zeros((L, R, H, d), np.float32)
    q[:, :, 0, 0] = 1.0
    w = np.ones((L, R, H), np.float32)
    keys = np.zeros((L, N, d), np.float32)
    keys[0, :, 0] = col0
    return wl.Problem(name, k, wl.f32_to_bf16_bits(q), wl.f32_to_bf16_bits(w),
                      wl.f32_to_bf16_bits(keys), None, None, True)


def test_many_candidates_with_ties(selector):
    """Four distinct scores over 40000 blocks: a quarter of the row ties at the top, so
    more candidates pass the floor than the select holds in registers (the select then
    re-reads them from memory on every radix pass) and the tie-break decides the output."""
    rng = np.random.default_rng(8)
    N = 40000
    p = _column0_problem("many_candidates", 1.0 + rng.integers(0, 4, N) / 4.0, N)
    _print_case("many_candidates", p)
    gs.assert_bit_exact(gs.run_gpu(selector, p), gs.run_oracle(p), "many_candidates")


def test_rescore_when_floor_too_high(selector):
    """The floor is placed from evenly spaced blocks, (2j+1) N / (2S) (S = 256 on this
    one-layer call).  Giving every block either sample count can pick the top scores makes
    the floor pass only a few dozen candidates, fewer than k, so the select must rescore
    the whole row; the result is still exact."""
    rng = np.random.default_rng(9)
    N = 20000
    col0 = 1.0 + rng.integers(0, 128, N) / 128.0          # [1, 2): below every sampled block
    sampled = gs.floor_sample_blocks(N)
    col0[sampled] = 2.0 + rng.integers(0, 128, len(sampled)) / 64.0  # [2, 4)
    p = _column0_problem("rescore", col0, N)
    _print_case("rescore", p)
    gs.assert_bit_exact(gs.run_gpu(selector, p), gs.run_oracle(p), "rescore")


@pytest.mark.parametrize("values,mask_p,shared", [("normal", None, True), ("normal", 0.4, True),
                                                  ("normal", 0.5, False)])
def test_general_custom(selector, values, mask_p, shared):
    p = wl.make_custom(3, 6, 64, 128, 12000, 512, seed=200, values=values, mask_p=mask_p,
                       mask_shared=shared, limits=np.array([[12000 - 5 + r for r in range(6)]]))
    _print_case(f"general_{mask_p}_{shared}", p)
    gpu = gs.run_gpu(selector, p)
    gs.assert_self_consistent(p, gpu)
    gs.assert_general(p, gpu, gs.run_oracle(p))


@pytest.mark.parametrize("k", [512, 2048])
def test_more_rows_than_compute_units(selector, k):
    """43 x 8 = 344 selections: more than one per compute unit, so the select
    runs with its smaller workgroups; large k exercises their widest order."""
    p = wl.make_custom(43, 8, 8, 64, 3000, k, seed=310 + k, values="int3", mask_p=0.7)
    _print_case(f"many_rows_k{k}", p)
    gpu = gs.run_gpu(selector, p)
    gs.assert_self_consistent(p, gpu)
    gs.assert_bit_exact(gpu, gs.run_oracle(p), f"many_rows_k{k}")


def test_more_rows_than_compute_units_every_select_path(selector):
    """43 x 8 selections with the smaller select workgroups, through the select's
    slow paths: on even layers half of the 20000 blocks tie at the top, so more
    candidates pass the floor than the registers hold; on odd layers the sampled
    blocks hold the top scores, so the floor passes fewer than k and every row
    is rescored."""
    rng = np.random.default_rng(11)
    L, R, H, d, N, k = 43, 8, 1, 64, 20000, 512
    q = np.zeros((L, R, H, d), np.float32)
    q[:, :, 0, 0] = 1.0
    w = np.ones((L, R, H), np.float32)
    keys = np.zeros((L, N, d), np.float32)
    sampled = gs.floor_sample_blocks(N)
    for l in range(L):
        if l % 2 == 0:
            keys[l, :, 0] = 1.0 + rng.integers(0, 2, N) / 2.0
        else:
            col0 = 1.0 + rng.integers(0, 128, N) / 128.0
            col0[sampled] = 2.0 + rng.integers(0, 128, len(sampled)) / 64.0
            keys[l, :, 0] = col0
    p = wl.Problem("many_rows_paths", k, wl.f32_to_bf16_bits(q), wl.f32_to_bf16_bits(w),
                   wl.f32_to_bf16_bits(keys), None, None, True)
    _print_case("many_rows_paths", p)
    gs.assert_bit_exact(gs.run_gpu(selector, p), gs.run_oracle(p), "many_rows_paths")


def test_layer_alone_equals_layer_in_batch(selector):
    """A batched call places each row's floor from 512 sampled blocks and a one-layer call
    from 256, and their key streams cut the work into different pieces.  Neither changes
    any key's score or the result: each layer selected alone is bit-identical to the same
    layer inside the batch, on general (non-integer) values too."""
    p = wl.make_custom(4, 6, 64, 128, 20000, 512, seed=330, values="normal", mask_p=0.5,
                       limits=np.array([[20000 - 5 + r for r in range(6)]] * 4))
    _print_case("alone_vs_batch", p)
    batched = gs.run_gpu(selector, p)
    for l in range(p.layers):
        one = wl.Problem(f"{p.name}[{l}]", p.k, p.q[l:l + 1], p.w[l:l + 1], p.keys[l:l + 1],
                         None if p.mask is None else p.mask[l:l + 1],
                         None if p.limit is None else p.limit[l:l + 1], p.integer_valued)
        alone = gs.run_gpu(selector, one)
        for a, b in zip(alone, batched):
            np.testing.assert_array_equal(a[0], b[l], err_msg=f"layer {l}")


def test_repeated_calls_identical(selector):
    """Atomic append order must not leak into the output (tie-heavy input)."""
    import torch
    p = wl.make_custom(2, 6, 64, 128, 20000, 512, seed=300, values="ternary", mask_p=0.7)
    q, w, keys, mask, limit = sel.upload(p)
    first = [t.clone() for t in selector.score_select(q, w, keys, p.k, mask, limit)]
    for _ in range(20):
        out = selector.score_select(q, w, keys, p.k, mask, limit)
        for a, b in zip(first, out):
            assert torch.equal(a, b)
    torch.cuda.synchronize()


def test_graph_capture_replays(selector):
    """The whole call captured once into a HIP graph (one submission for all layers)
    replays to the eager result, with other work and synchronisations in between."""
    import torch
    p = wl.make_custom(4, 6, 16, 128, 9000, 512, seed=320, values="int3", mask_p=0.6,
                       limits=np.array([[9000 - 5 + r for r in range(6)]] * 4))
    q, w, keys, mask, limit = sel.upload(p)
    eager = [t.clone() for t in selector.score_select(q, w, keys, p.k, mask, limit)]
    torch.cuda.synchronize()
    out = tuple(torch.full_like(t, -7) for t in eager)
    stream = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        selector.score_select(q, w, keys, p.k, mask, limit, out=out)
    for i in range(3):
        for t in out:
            t.fill_(-7)
        junk = torch.randn(1 << 20, device="cuda").sum()  # unrelated eager work
        graph.replay()
        torch.cuda.synchronize()
        assert float(junk) == float(junk)
        for a, b in zip(eager, out):
            assert torch.equal(a, b), f"replay {i}"
    gs.assert_bit_exact(tuple(t.cpu().numpy() for t in out), gs.run_oracle(p), "graph")


def test_capacity_error_leaves_outputs_untouched(selector):
    import torch
    p = wl.make_custom(1, 2, 8, 64, 80000, 16, seed=301, values="int3")
    q, w, keys, mask, limit = sel.upload(p)
    out = (torch.full((1, 2, 16), 7, dtype=torch.int32, device="cuda"),
           torch.full((1, 2, 16), 7.0, device="cuda"),
           torch.full((1, 2), 7, dtype=torch.int32, device="cuda"))
    with pytest.raises(sel.DsSelError) as e:
        selector.score_select(q, w, keys, 16, mask, limit, out=out)
    assert e.value.status == sel.DS_SEL_E_CAPACITY
    torch.cuda.synchronize()
    assert all(bool((t == 7).all()) for t in out)


@pytest.mark.parametrize("shared", [True, False])
def test_many_tiles_expander_rounds(shared):
    """2.3 M blocks are 1,124 tiles of 2,048: more than 64 expanding workgroups'
    worth, so each of the 64 takes 32 tiles in two rounds of 16 (and the last
    ones have none).  Bit-exact on integer inputs, shared and per-row masks."""
    import torch
    p = wl.make_custom(1, 2, 4, 32, 2_300_000, 64, seed=330 + int(shared), values="int3", mask_p=0.5,
                       mask_shared=shared, limits=np.array([[2_300_000, 1_700_003]], np.int32))
    _print_case(f"many_tiles shared={shared}", p)
    s = sel.Selector(max_layers=1, max_rows=2, max_heads=4, max_dim=32, max_blocks=p.blocks, max_k=64,
                     device=0)
    try:
        got = gs.run_gpu(s, p)
        torch.cuda.synchronize()
    finally:
        s.close()
    gs.assert_bit_exact(got, gs.run_oracle(p), f"many_tiles shared={shared}")
