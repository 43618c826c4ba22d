"""The binding's argument checks, on CPU tensors (no library call is made):
every tensor whose dtype, shape, strides or device differs from what the C ABI
reads or writes is rejected with ValueError before anything is enqueued."""
import pytest
import torch

from sparse_attention_block_ds_amd import selector as sel

L, R, H, D, N, K = 2, 3, 4, 64, 100, 16
BF = torch.bfloat16
CPU = torch.device("cpu")


def good():
    return dict(q=torch.zeros(L, R, H, D, dtype=BF), w=torch.zeros(L, R, H, dtype=BF),
                keys=torch.zeros(L, N, D, dtype=BF), k=K,
                mask=torch.zeros(L, 1, 4, dtype=torch.int32),
                limit=torch.zeros(L, R, dtype=torch.int32),
                out=(torch.zeros(L, R, K, dtype=torch.int32), torch.zeros(L, R, K),
                     torch.zeros(L, R, dtype=torch.int32)))


def check(**kw):
    a = good()
    a.update(kw)
    sel.check_select_tensors(a["q"], a["w"], a["keys"], a["k"], a["mask"], a["limit"], a["out"], CPU)


def test_accepts_well_formed():
    check()
    check(mask=None, limit=None, out=None)
    check(keys=torch.zeros(L, N, 72, dtype=BF)[:, :, :D])          # padded rows
    check(mask=torch.zeros(L, R, 4, dtype=torch.int32))           # a mask row per query row
    o = good()["out"]
    check(out=(o[0], o[1], None))


@pytest.mark.parametrize("name,value", [
    ("q", torch.zeros(L, R, H, D)),                                   # fp32, not bf16
    ("q", torch.zeros(L, 2 * R, H, D, dtype=BF)[:, :R]),              # sliced rows: not contiguous
    ("q", torch.zeros(L, R, H * D, dtype=BF)),                        # wrong rank
    ("w", torch.zeros(L, R, H + 1, dtype=BF)),
    ("w", torch.zeros(L, R, H, dtype=torch.float16)),
    ("keys", torch.zeros(L, N, D)),
    ("keys", torch.zeros(L, N, 2 * D, dtype=BF)[:, :, ::2]),         # non-unit last stride
    ("keys", torch.zeros(L + 1, N, D, dtype=BF)),
    ("keys", torch.zeros(L, N, D - 8, dtype=BF)),                     # rows shorter than d
    ("mask", torch.zeros(L, 1, 3, dtype=torch.int32)),                # fewer than ceil(N/32) words
    ("mask", torch.zeros(L, 2, 4, dtype=torch.int32)),                # neither 1 nor R rows
    ("mask", torch.zeros(L, 1, 4, dtype=torch.int64)),
    ("limit", torch.zeros(L, R, dtype=torch.int64)),
    ("limit", torch.zeros(R, L, dtype=torch.int32)),
    ("k", 0),
    ("k", 2.0),
])
def test_rejects_input(name, value):
    with pytest.raises(ValueError):
        check(**{name: value})


def _outs(**kw):
    o = dict(zip(("idx", "score", "count"), good()["out"]))
    o.update(kw)
    return (o["idx"], o["score"], o["count"])


@pytest.mark.parametrize("out", [
    _outs(idx=torch.zeros(L, R, K - 1, dtype=torch.int32)),        # too small: would be overrun
    _outs(idx=torch.zeros(L, R, K)),                                # float, not int32
    _outs(score=torch.zeros(L, R, K, dtype=torch.float64)),
    _outs(score=torch.zeros(L, R, 2 * K)[:, :, :K]),                # not contiguous
    _outs(count=torch.zeros(L, R + 1, dtype=torch.int32)),
    (torch.zeros(L, R, K, dtype=torch.int32), torch.zeros(L, R, K)),  # not a triple
])
def test_rejects_output(out):
    with pytest.raises(ValueError):
        check(out=out)


def test_rejects_other_device():
    a = good()
    with pytest.raises(ValueError):
        sel.check_select_tensors(a["q"], a["w"], a["keys"], K, None, None, None, torch.device("meta"))
    with pytest.raises(ValueError):
        check(limit=torch.zeros(L, R, dtype=torch.int32, device="meta"))


def attend_good():
    return dict(qa=torch.zeros(L, R, H, D, dtype=BF), keys=torch.zeros(L, N, D, dtype=BF),
                values=torch.zeros(L, N, D, dtype=BF), idx=torch.zeros(L, R, K, dtype=torch.int32),
                count=torch.zeros(L, R, dtype=torch.int32), scale=0.125,
                out=torch.zeros(L, R, H, D))


def check_attend(**kw):
    a = attend_good()
    a.update(kw)
    sel.check_attend_tensors(a["qa"], a["keys"], a["values"], a["idx"], a["count"], a["scale"],
                             a["out"], CPU)


def test_attend_accepts_well_formed():
    check_attend()
    check_attend(count=None, out=None)


@pytest.mark.parametrize("name,value", [
    ("scale", None), ("scale", float("nan")), ("scale", float("inf")),
    ("qa", torch.zeros(L, R, H, D)),
    ("qa", torch.zeros(L, 2 * R, H, D, dtype=BF)[:, :R]),
    ("values", torch.zeros(L, N + 1, D, dtype=BF)),
    ("values", torch.zeros(L, N, D)),
    ("keys", torch.zeros(L, N, 2 * D, dtype=BF)[:, :, ::2]),
    ("idx", torch.zeros(L, R, K)),
    ("idx", torch.zeros(L + 1, R, K, dtype=torch.int32)),
    ("count", torch.zeros(L, R, dtype=torch.int64)),
    ("out", torch.zeros(L, R, H, D - 1)),
    ("out", torch.zeros(L, R, H, D, dtype=torch.float64)),
])
def test_attend_rejects(name, value):
    with pytest.raises(ValueError):
        check_attend(**{name: value})


def _gpu_test_problems():
    """Every problem shape the GPU parity tests feed through the binding."""
    import numpy as np
    from sparse_attention_block_ds_amd import workloads as wl
    from tests import test_gpu_parity as tg
    probs = [wl.make_custom(*c["args"], seed=100 + i, **c["kw"]) for i, c in enumerate(tg.EDGE)]
    probs += [wl.make(n) for n in ("tiny", "8k", "verify")]
    probs.append(wl.make_custom(43, 8, 8, 64, 3000, 512, seed=1, values="int3", mask_p=0.7))
    probs.append(wl.make_custom(3, 6, 64, 128, 1200, 512, seed=2, values="normal", mask_p=0.5,
                                mask_shared=False, limits=np.array([[1200 - 5 + r for r in range(6)]])))
    return probs


def test_accepts_every_gpu_test_shape():
    """The shapes the GPU tests use (empty N, padded rows, per-row masks, ...) pass
    the binding's checks as uploaded, so a GPU run is never spent on a check."""
    for p in _gpu_test_problems():
        q, w, keys, mask, limit = sel.upload(p, "cpu")
        sel.check_select_tensors(q, w, keys, p.k, mask, limit, None, CPU)
        out = (torch.empty(p.layers, p.rows, p.k, dtype=torch.int32), torch.empty(p.layers, p.rows, p.k),
               torch.empty(p.layers, p.rows, dtype=torch.int32))
        sel.check_select_tensors(q, w, keys, p.k, mask, limit, out, CPU)
        qa = torch.zeros(p.layers, p.rows, 2, p.dim, dtype=BF)
        idx = torch.zeros(p.layers, p.rows, p.k, dtype=torch.int32)
        sel.check_attend_tensors(qa, keys, keys, idx, None, 0.5, None, CPU)


# ------------------------------------------------------------ the 8-bit key stream
def q8_good():
    return dict(codes=torch.zeros(L, N, D, dtype=torch.int8),
                scales=torch.zeros(L, N, D // 32, dtype=torch.float16))


def check_q8(**kw):
    a, s = good(), q8_good()
    s.update(kw)
    sel.check_select_q8_tensors(a["q"], a["w"], s["codes"], s["scales"], a["k"], a["mask"], a["limit"],
                                a["out"], CPU)


def test_q8_accepts_well_formed():
    check_q8()
    check_q8(codes=torch.zeros(L, N, 72, dtype=torch.int8)[:, :, :D],
             scales=torch.zeros(L, N, 3, dtype=torch.float16)[:, :, :2])
    check_q8(codes=torch.zeros(L, 0, D, dtype=torch.int8),
             scales=torch.zeros(L, 0, D // 32, dtype=torch.float16), )


@pytest.mark.parametrize("name,value", [
    ("codes", torch.zeros(L, N, D, dtype=torch.uint8)),
    ("codes", torch.zeros(L, N, D, dtype=torch.int16)),
    ("codes", torch.zeros(L + 1, N, D, dtype=torch.int8)),
    ("codes", torch.zeros(L, N, D - 8, dtype=torch.int8)),              # rows shorter than d
    ("codes", torch.zeros(L, N, 2 * D, dtype=torch.int8)[:, :, ::2]),    # non-unit last stride
    ("scales", torch.zeros(L, N, D // 32)),                              # fp32, not fp16
    ("scales", torch.zeros(L, N, D // 32, dtype=BF)),
    ("scales", torch.zeros(L, N + 1, D // 32, dtype=torch.float16)),     # block counts differ
    ("scales", torch.zeros(L, N, D // 32 - 1, dtype=torch.float16)),     # fewer than d/32
])
def test_q8_rejects(name, value):
    with pytest.raises(ValueError):
        check_q8(**{name: value})


def test_quantize_rejects_before_the_library():
    with pytest.raises(ValueError):
        sel.quantize_q8(torch.zeros(L, N, D))                            # fp32 keys
    with pytest.raises(ValueError):
        sel.quantize_q8(torch.zeros(L, N, D, dtype=BF), codes=torch.zeros(L, N + 1, D, dtype=torch.int8))
    with pytest.raises(ValueError):
        sel.quantize_q8(torch.zeros(L, N, D, dtype=BF),
                        scales=torch.zeros(L, N, D // 32, dtype=torch.float16, device="meta"))


def test_q8_accepts_every_gpu_test_shape():
    """The 8-bit GPU tests' problems pass both the binding's checks and the C
    ABI's (ds_sel_check_args_q8 with the tests' handle capacity)."""
    import ctypes
    import numpy as np
    from tests import test_gpu_q8 as tq
    lib = sel.load_library()
    lim = sel.make_limits(43, 8, 64, 256, 75000, 2048)
    for i, c in enumerate(tq.EXACT):
        p, codes, scales = tq._exact_case(600 + i, *c["args"], exps=c.get("exps", (-3, 0)),
                                          **c.get("kw", {}))
        q, w, _, mask, limit = sel.upload(p, "cpu")
        ct = torch.from_numpy(codes)
        st = torch.from_numpy(scales.view(np.float16))
        out = (torch.empty(p.layers, p.rows, p.k, dtype=torch.int32), torch.empty(p.layers, p.rows, p.k),
               torch.empty(p.layers, p.rows, dtype=torch.int32))
        sel.check_select_q8_tensors(q, w, ct, st, p.k, mask, limit, out, CPU)
        a = sel.make_args(q, w, None, p.k, mask, limit, *out, blocks=p.blocks)
        k8 = sel.make_q8_keys(ct, st)
        rc = lib.ds_sel_check_args_q8(ctypes.byref(lim), ctypes.byref(a), ctypes.byref(k8))
        assert rc == sel.DS_SEL_OK, (c["name"], rc)
