"""The CPU oracle against what the mathematics fixes (no GPU needed)."""
import json
import os

import numpy as np
import pytest

import oracle
from sparse_attention_block_ds_amd import workloads as wl
from tests import pins

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden_problem(g):
    q = wl.small_int_bits(np.array(g["q"]))
    w = wl.small_int_bits(np.array(g["w"]))
    keys = wl.small_int_bits(np.array(g["keys"]))
    mask = np.array(g["mask_words"], np.uint32)
    limit = np.array(g["limit"], np.int32)
    return wl.Problem("hand", g["k"], q, w, keys, mask, limit, True)


def test_hand_worked_example(oracle_lib):
    with open(os.path.join(GOLDEN, "hand_example.json")) as f:
        g = json.load(f)
    p = _golden_problem(g)
    idx, score, count = oracle.select(p.q, p.w, p.keys, p.k, p.mask, p.limit, lib=oracle_lib)
    np.testing.assert_array_equal(idx, np.array(g["expect_idx"]))
    exp_score = np.array([[[float(v) for v in row] for row in g["expect_score"][0]]], np.float32)
    np.testing.assert_array_equal(score, exp_score)
    np.testing.assert_array_equal(count, np.array(g["expect_count"]))


def test_all_pins(oracle_lib):
    pins.all_pins(oracle_lib)


def test_tiny_workload_exact(oracle_lib):
    pins.check_exact_integer(wl.make("tiny"), oracle_lib)


def test_verify_int_workload_exact(oracle_lib):
    """Full-size integer verify: exact int64 scores, ordered by numpy's lexsort."""
    p = wl.make("verify_int")
    idx, score, count = oracle.select(p.q, p.w, p.keys, p.k, p.mask, p.limit, lib=oracle_lib)
    exact = pins.exact_int_scores(p)
    adm = pins.admitted_mask(p)
    for r in range(p.rows):
        blocks = np.flatnonzero(adm[0, r])
        s = exact[0, r, blocks]
        order = np.lexsort((blocks, -s))[:p.k]
        np.testing.assert_array_equal(idx[0, r], blocks[order])
        np.testing.assert_array_equal(score[0, r], s[order].astype(np.float32))
        assert count[0, r] == p.k


def test_8k_workload_invariants(oracle_lib):
    pins.check_invariants(wl.make("8k"), oracle_lib)


def test_bf16_rounding_matches_torch():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(5)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10.0 ** rng.integers(-30, 30, 100000),
                        np.array([0.0, -0.0, 1.0, 1.00390625, 1.01171875, -3.0, 65504.0], np.float32)])
    x = x.astype(np.float32)
    ours = wl.f32_to_bf16_bits(x)
    theirs = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, theirs)
    np.testing.assert_array_equal(wl.bf16_bits_to_f32(ours), torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_mask_packing_bit_order():
    bits = np.zeros((1, 1, 70), bool)
    bits[0, 0, [0, 5, 31, 32, 69]] = True
    words = wl.pack_mask(bits)
    assert words.shape == (1, 1, 3)
    assert words[0, 0, 0] == (1 | (1 << 5) | (1 << 31))
    assert words[0, 0, 1] == 1
    assert words[0, 0, 2] == (1 << (69 - 64))


def test_workload_shapes_and_recipes():
    p = wl.make("tiny")
    assert (p.layers, p.rows, p.heads, p.dim, p.blocks, p.k) == (1, 1, 4, 64, 4096, 512)
    vals = wl.bf16_bits_to_f32(p.keys)
    assert set(np.unique(vals)) <= set(range(-3, 4))
    p = wl.make("verify")
    assert (p.rows, p.blocks) == (6, 32768)
    np.testing.assert_array_equal(p.limit[0], [32768 - 5 + r for r in range(6)])
    p = wl.make("300k")
    assert p.mask.shape == (1, 1, (75000 + 31) // 32)
    frac = pins.admitted_mask(p).mean()
    assert abs(frac - 0.6) < 0.01


def test_oracle_rejects_bad_arguments(oracle_lib):
    p = wl.make_custom(1, 1, 4, 64, 10, 4, seed=1, values="int3")
    with pytest.raises(oracle.OracleError):
        oracle.select(p.q, p.w, p.keys, 0, lib=oracle_lib)
    bad = p.keys.copy()
    bad[0, 3, 7] = 0x7F80          # +inf
    with pytest.raises(oracle.OracleError):
        oracle.select(p.q, p.w, bad, 4, lib=oracle_lib)
