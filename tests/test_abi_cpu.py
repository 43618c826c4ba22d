"""The C ABI without a GPU: exports, struct layout, host-side validation,
and the no-device path.  No compute call is made here."""
import ctypes
import os
import re
import subprocess

import pytest

from sparse_attention_block_ds_amd import selector as sel

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ds_sel.h")


@pytest.fixture(scope="module")
def lib():
    """libdssel.so; DS_SEL_TEST_LIBRARY names another build of it (the sanitizer run)."""
    path = os.environ.get("DS_SEL_TEST_LIBRARY")
    if path:
        return sel.load_library(path)
    if not os.path.exists(sel.LIBRARY):
        from sparse_attention_block_ds_amd import build
        build.build(verbose=False)
    return sel.load_library()


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[\w\s\*]+?\b(ds_sel_\w+)\s*\(", text, re.M)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ("ds_sel_create", "ds_sel_score_select", "ds_sel_destroy", "ds_sel_attend"):
        assert required in names
    assert set(names) == set(sel.EXPORTED)


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", sel.LIBRARY], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (ds_sel_\w+)", out))
    for name in declared_functions():
        assert name in exported, name
        assert hasattr(lib, name)


def test_struct_layout_matches_header(tmp_path):
    src = tmp_path / "layout.c"
    src.write_text(r"""
#include <stdio.h>
#include <stddef.h>
#include "ds_sel.h"
#define F(T, m) printf(#T "." #m " %zu\n", offsetof(T, m))
int main(void) {
  printf("ds_sel_limits %zu\nds_sel_args %zu\n", sizeof(ds_sel_limits), sizeof(ds_sel_args));
  printf("ds_sel_attend_args %zu\n", sizeof(ds_sel_attend_args));
  printf("ds_sel_q8_keys %zu\nds_sel_quantize_args %zu\n", sizeof(ds_sel_q8_keys),
         sizeof(ds_sel_quantize_args));
  F(ds_sel_q8_keys, codes); F(ds_sel_q8_keys, ldc); F(ds_sel_q8_keys, scales);
  F(ds_sel_q8_keys, scale_layer_stride);
  F(ds_sel_quantize_args, blocks); F(ds_sel_quantize_args, keys); F(ds_sel_quantize_args, codes);
  F(ds_sel_quantize_args, code_layer_stride); F(ds_sel_quantize_args, scales);
  F(ds_sel_quantize_args, scale_layer_stride);
  F(ds_sel_limits, max_blocks); F(ds_sel_args, blocks); F(ds_sel_args, q); F(ds_sel_args, ldk);
  F(ds_sel_args, mask); F(ds_sel_args, mask_layer_stride); F(ds_sel_args, limit);
  F(ds_sel_args, out_count);
  F(ds_sel_attend_args, scale); F(ds_sel_attend_args, blocks); F(ds_sel_attend_args, keys);
  F(ds_sel_attend_args, values); F(ds_sel_attend_args, value_layer_stride);
  F(ds_sel_attend_args, idx); F(ds_sel_attend_args, out);
  return 0;
}
""")
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c11", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)],
                   check=True)
    lines = dict(l.split() for l in subprocess.run([str(exe)], capture_output=True, text=True,
                                                   check=True).stdout.splitlines())
    assert int(lines["ds_sel_limits"]) == ctypes.sizeof(sel.Limits)
    assert int(lines["ds_sel_args"]) == ctypes.sizeof(sel.Args)
    assert int(lines["ds_sel_attend_args"]) == ctypes.sizeof(sel.AttendArgs)
    assert int(lines["ds_sel_q8_keys"]) == ctypes.sizeof(sel.Q8Keys)
    assert int(lines["ds_sel_quantize_args"]) == ctypes.sizeof(sel.QuantizeArgs)
    classes = {"ds_sel_limits": sel.Limits, "ds_sel_args": sel.Args,
               "ds_sel_attend_args": sel.AttendArgs, "ds_sel_q8_keys": sel.Q8Keys,
               "ds_sel_quantize_args": sel.QuantizeArgs}
    for key, value in lines.items():
        if "." in key:
            struct, field = key.split(".")
            cls = classes[struct]
            assert getattr(cls, field).offset == int(value), key


class FakeTensor:
    """Stands in for a device tensor: a pointer value that is never dereferenced."""

    def __init__(self, shape, strides=None, ptr=0x10000):
        self.shape = shape
        self._strides = strides or tuple(int(x) for x in _contig(shape))
        self._ptr = ptr

    def data_ptr(self):
        return self._ptr

    def stride(self, i):
        return self._strides[i]


def _contig(shape):
    out, acc = [], 1
    for s in reversed(shape):
        out.append(acc)
        acc *= s
    return tuple(reversed(out))


def _args(L=2, R=6, H=64, d=128, N=75000, k=512, mask_rows=1, with_limit=True, ldk=None,
          keys_ptr=0x20000):
    ldk = ldk or d
    q = FakeTensor((L, R, H, d), ptr=0x1000)
    w = FakeTensor((L, R, H), ptr=0x3000)
    keys = FakeTensor((L, N, ldk), (N * ldk, ldk, 1), ptr=keys_ptr)
    words = (N + 31) // 32
    mask = FakeTensor((L, mask_rows, words), ptr=0x40000) if mask_rows else None
    limit = FakeTensor((L, R), ptr=0x50000) if with_limit else None
    outs = (FakeTensor((L, R, k), ptr=0x60000), FakeTensor((L, R, k), ptr=0x70000),
            FakeTensor((L, R), ptr=0x80000))
    return sel.make_args(q, w, keys, k, mask, limit, *outs)


LIM = dict(max_layers=43, max_rows=6, max_heads=64, max_dim=128, max_blocks=75000, max_k=512)


def check(lib, args, **lim):
    limits = sel.make_limits(**{**LIM, **lim})
    return lib.ds_sel_check_args(ctypes.byref(limits), ctypes.byref(args))


def test_valid_arguments_pass(lib):
    assert check(lib, _args()) == sel.DS_SEL_OK
    assert check(lib, _args(mask_rows=6)) == sel.DS_SEL_OK
    assert check(lib, _args(mask_rows=0, with_limit=False)) == sel.DS_SEL_OK
    assert check(lib, _args(N=0, keys_ptr=0)) == sel.DS_SEL_OK
    assert check(lib, _args(d=64, H=4, ldk=72), max_dim=128) == sel.DS_SEL_OK


@pytest.mark.parametrize("field,value,expect", [
    ("layers", 0, sel.DS_SEL_E_INVALID),
    ("rows", 0, sel.DS_SEL_E_INVALID),
    ("rows", 9, sel.DS_SEL_E_INVALID),
    ("heads", 0, sel.DS_SEL_E_INVALID),
    ("k", 0, sel.DS_SEL_E_INVALID),
    ("k", 4096, sel.DS_SEL_E_INVALID),
    ("blocks", -1, sel.DS_SEL_E_INVALID),
    ("dim", 96, sel.DS_SEL_E_UNSUPPORTED),
    ("dim", 100, sel.DS_SEL_E_INVALID),
    ("q", None, sel.DS_SEL_E_INVALID),
    ("q", 0x1002, sel.DS_SEL_E_INVALID),            # not 16-byte aligned
    ("out_idx", None, sel.DS_SEL_E_INVALID),
    ("keys", None, sel.DS_SEL_E_INVALID),
    ("keys", 0x20008, sel.DS_SEL_E_INVALID),       # not 16-byte aligned
    ("ldk", 120, sel.DS_SEL_E_INVALID),            # ldk < d
    ("ldk", 132, sel.DS_SEL_E_INVALID),            # ldk not a multiple of 8
    ("key_layer_stride", 8, sel.DS_SEL_E_INVALID),  # layers overlap
    ("mask_row_stride", 5, sel.DS_SEL_E_INVALID),   # shorter than a mask row
    ("mask_layer_stride", 3, sel.DS_SEL_E_INVALID),
    ("limit", 0x50002, sel.DS_SEL_E_INVALID),       # misaligned int32
    ("struct_size", 8, sel.DS_SEL_E_INVALID),
])
def test_bad_arguments_rejected(lib, field, value, expect):
    a = _args()
    setattr(a, field, value)
    assert check(lib, a) == expect


@pytest.mark.parametrize("field,value", [("layers", 44), ("rows", 6), ("heads", 64), ("k", 512),
                                         ("blocks", 75000)])
def test_capacity_enforced(lib, field, value):
    a = _args(L=1)
    setattr(a, field, value + 1 if field != "rows" else 7)
    if field == "blocks":
        a.key_layer_stride = (value + 1) * 128
    assert check(lib, a) == sel.DS_SEL_E_CAPACITY


def test_bad_limits_rejected(lib):
    for field, value in [("max_rows", 9), ("max_k", 4097), ("max_layers", 0), ("max_dim", 512), ("flags", 4),
                         ("max_blocks", -1)]:
        lim = sel.make_limits(**LIM)
        setattr(lim, field, value)
        assert lib.ds_sel_scratch_bytes(ctypes.byref(lim)) == 0
        h = ctypes.c_void_p()
        assert lib.ds_sel_create(ctypes.byref(lim), ctypes.byref(h)) == sel.DS_SEL_E_INVALID


def test_scratch_bytes(lib):
    lim = sel.make_limits(**LIM)
    nbytes = lib.ds_sel_scratch_bytes(ctypes.byref(lim))
    up = lambda v: (v + 255) // 256 * 256
    L, R, D, N = 43, 6, 128, 75000
    expect = (up(L * R * D * 4) + up(3 * L * R * D * 2) + up(L * N * 4) + up(9 * L * 4)
              + up(L * R * 4) + up(L * R * 32 * 4) + up(L * R * ((N + 3) // 4 * 4) * 8)
              + up(512 * 64 * 2 * 4) + up(512 * 64 * D * 4))
    assert nbytes == expect


def test_no_device_or_create(lib):
    """Without a GPU, create reports DS_SEL_E_NODEVICE and hands back no handle."""
    lim = sel.make_limits(**LIM)
    h = ctypes.c_void_p(1234)
    rc = lib.ds_sel_create(ctypes.byref(lim), ctypes.byref(h))
    if os.path.exists("/dev/kfd"):
        pytest.skip("a GPU driver is present on this host")
    assert rc == sel.DS_SEL_E_NODEVICE
    assert not h.value


def test_destroy_null_is_noop_and_status_strings(lib):
    lib.ds_sel_destroy(None)
    assert lib.ds_sel_poison_scratch(None, 0xFF, None) == sel.DS_SEL_E_INVALID
    assert lib.ds_sel_status_string(0) == b"ok"
    assert lib.ds_sel_status_string(sel.DS_SEL_E_CAPACITY) == b"exceeds the handle's capacity"
    assert lib.ds_sel_status_string(99) == b"unknown status"


# ------------------------------------------------------------ attention over a selection
def _attend_args(L=2, R=6, H=64, d=128, N=75000, k=512, with_count=True, ldk=None, ldv=None):
    ldk, ldv = ldk or d, ldv or d
    qa = FakeTensor((L, R, H, d), ptr=0x1000)
    keys = FakeTensor((L, N, ldk), (N * ldk, ldk, 1), ptr=0x20000)
    values = FakeTensor((L, N, ldv), (N * ldv, ldv, 1), ptr=0x90000)
    idx = FakeTensor((L, R, k), ptr=0x60000)
    count = FakeTensor((L, R), ptr=0x80000) if with_count else None
    out = FakeTensor((L, R, H, d), ptr=0xA0000)
    return sel.make_attend_args(qa, keys, values, idx, count, 1.0 / d ** 0.5, out)


def check_attend(lib, args, **lim):
    limits = sel.make_limits(**{**LIM, **lim})
    return lib.ds_sel_check_attend_args(ctypes.byref(limits), ctypes.byref(args))


def test_attend_valid_arguments_pass(lib):
    assert check_attend(lib, _attend_args()) == sel.DS_SEL_OK
    assert check_attend(lib, _attend_args(with_count=False)) == sel.DS_SEL_OK
    assert check_attend(lib, _attend_args(d=64, H=20, ldk=72, ldv=80)) == sel.DS_SEL_OK
    a = _attend_args(N=0)
    a.keys = a.values = None
    assert check_attend(lib, a) == sel.DS_SEL_OK


@pytest.mark.parametrize("field,value,expect", [
    ("layers", 0, sel.DS_SEL_E_INVALID),
    ("rows", 9, sel.DS_SEL_E_INVALID),
    ("heads", 0, sel.DS_SEL_E_INVALID),
    ("k", 0, sel.DS_SEL_E_INVALID),
    ("k", 4096, sel.DS_SEL_E_INVALID),
    ("dim", 96, sel.DS_SEL_E_UNSUPPORTED),
    ("dim", 100, sel.DS_SEL_E_INVALID),
    ("scale", float("inf"), sel.DS_SEL_E_INVALID),
    ("scale", float("nan"), sel.DS_SEL_E_INVALID),
    ("reserved", 1, sel.DS_SEL_E_INVALID),
    ("q", None, sel.DS_SEL_E_INVALID),
    ("q", 0x1008, sel.DS_SEL_E_INVALID),            # not 16-byte aligned
    ("idx", None, sel.DS_SEL_E_INVALID),
    ("idx", 0x60002, sel.DS_SEL_E_INVALID),
    ("count", 0x80001, sel.DS_SEL_E_INVALID),
    ("out", None, sel.DS_SEL_E_INVALID),
    ("values", None, sel.DS_SEL_E_INVALID),
    ("values", 0x90008, sel.DS_SEL_E_INVALID),
    ("ldv", 120, sel.DS_SEL_E_INVALID),
    ("ldv", 132, sel.DS_SEL_E_INVALID),
    ("value_layer_stride", 8, sel.DS_SEL_E_INVALID),  # layers overlap
    ("key_layer_stride", 4, sel.DS_SEL_E_INVALID),
    ("struct_size", 8, sel.DS_SEL_E_INVALID),
])
def test_attend_bad_arguments_rejected(lib, field, value, expect):
    a = _attend_args()
    setattr(a, field, value)
    assert check_attend(lib, a) == expect


@pytest.mark.parametrize("field,value", [("layers", 44), ("rows", 7), ("heads", 65), ("k", 513),
                                         ("blocks", 75001)])
def test_attend_capacity_enforced(lib, field, value):
    a = _attend_args(L=1)
    setattr(a, field, value)
    assert check_attend(lib, a) == sel.DS_SEL_E_CAPACITY


def test_noalloc_checks_before_touching_a_device(lib):
    """The static-scratch entry point validates and sizes the call on the host:
    oversize calls are refused with CAPACITY, bad ones with INVALID, and only a
    well-formed call reaches the device lookup (NODEVICE here)."""
    def args(L, R, d, N, k=16):
        a = sel.Args()
        a.struct_size = ctypes.sizeof(sel.Args)
        a.layers, a.rows, a.heads, a.dim, a.k, a.blocks = L, R, 4, d, k, N
        a.q = a.w = a.keys = a.out_idx = a.out_score = ctypes.c_void_p(256)
        a.ldk, a.key_layer_stride = d, N * d
        return a
    small, big = args(1, 6, 128, 32768), args(1, 8, 128, 1 << 22)
    assert 0 < lib.ds_sel_noalloc_scratch_bytes(ctypes.byref(small)) <= 64 << 20
    assert lib.ds_sel_noalloc_scratch_bytes(ctypes.byref(big)) > 64 << 20
    assert lib.ds_sel_score_select_noalloc(0, 0, ctypes.byref(big), None) == sel.DS_SEL_E_CAPACITY
    bad = args(1, 6, 128, 32768, k=0)
    assert lib.ds_sel_score_select_noalloc(0, 0, ctypes.byref(bad), None) == sel.DS_SEL_E_INVALID
    assert lib.ds_sel_score_select_noalloc(0, 4, ctypes.byref(small), None) == sel.DS_SEL_E_INVALID
    assert lib.ds_sel_score_select_noalloc(-1, 0, ctypes.byref(small), None) == sel.DS_SEL_E_INVALID
    assert lib.ds_sel_score_select_noalloc(0, 0, ctypes.byref(small), None) == sel.DS_SEL_E_NODEVICE


# ------------------------------------------------------------ the 8-bit key stream
def _q8(L=2, N=75000, d=128, ldc=None, lds=None):
    ldc, lds = ldc or d, lds or d // 32
    codes = FakeTensor((L, N, ldc), (N * ldc, ldc, 1), ptr=0xB0000)
    scales = FakeTensor((L, N, lds), (N * lds, lds, 1), ptr=0xC0002)
    return sel.make_q8_keys(codes, scales)


def _q8_args(L=2, N=75000, d=128):
    a = _args(L=L, N=N, d=d)
    a.keys, a.ldk, a.key_layer_stride = None, 0, 0
    return a


def check_q8(lib, args, k8, **lim):
    limits = sel.make_limits(**{**LIM, **lim})
    return lib.ds_sel_check_args_q8(ctypes.byref(limits), ctypes.byref(args),
                                    ctypes.byref(k8) if k8 is not None else None)


def test_q8_valid_arguments_pass(lib):
    assert check_q8(lib, _q8_args(), _q8()) == sel.DS_SEL_OK
    assert check_q8(lib, _q8_args(d=64), _q8(d=64, ldc=72, lds=3)) == sel.DS_SEL_OK
    assert check_q8(lib, _q8_args(L=1, d=32), _q8(L=1, d=32)) == sel.DS_SEL_OK
    empty = _q8(N=0)
    empty.codes = empty.scales = None
    assert check_q8(lib, _q8_args(N=0), empty) == sel.DS_SEL_OK


@pytest.mark.parametrize("field,value", [
    ("codes", None), ("codes", 0xB0004),         # missing, or not 8-byte aligned
    ("scales", None), ("scales", 0xC0001),       # missing, or not 2-byte aligned
    ("ldc", 120), ("ldc", 132),                  # ldc < d, or not a multiple of 8
    ("code_layer_stride", 8), ("code_layer_stride", 75000 * 128 + 4),
    ("lds", 3),                                  # fewer than d/32 scales per row
    ("scale_layer_stride", 10),                  # layers overlap
    ("struct_size", 8), ("reserved", 1),
])
def test_q8_bad_keys_rejected(lib, field, value):
    k8 = _q8()
    setattr(k8, field, value)
    assert check_q8(lib, _q8_args(), k8) == sel.DS_SEL_E_INVALID


def test_q8_rejects_bf16_keys_and_missing_stream(lib):
    a = _q8_args()
    a.keys = 0x20000  # the keys come from the 8-bit stream only
    assert check_q8(lib, a, _q8()) == sel.DS_SEL_E_INVALID
    assert check_q8(lib, _q8_args(), None) == sel.DS_SEL_E_INVALID
    assert lib.ds_sel_score_select_q8(None, ctypes.byref(_q8_args()), ctypes.byref(_q8()),
                                      None, None) == sel.DS_SEL_E_INVALID


def _quant_args(L=2, N=1000, d=128, ldk=None, ldc=None, lds=None):
    ldk, ldc, lds = ldk or d, ldc or d, lds or d // 32
    a = sel.QuantizeArgs()
    a.struct_size = ctypes.sizeof(sel.QuantizeArgs)
    a.layers, a.dim, a.reserved, a.blocks = L, d, 0, N
    a.keys, a.ldk, a.key_layer_stride = 0x20000, ldk, N * ldk
    a.codes, a.ldc, a.code_layer_stride = 0xB0000, ldc, N * ldc
    a.scales, a.lds, a.scale_layer_stride = 0xC0002, lds, N * lds
    return a


@pytest.mark.parametrize("field,value", [
    ("layers", 0), ("blocks", -1), ("dim", 96), ("dim", 16), ("reserved", 1), ("struct_size", 4),
    ("keys", None), ("keys", 0x20008), ("ldk", 120), ("ldk", 132),
    ("codes", None), ("codes", 0xB0008),         # code rows are written with 16-byte stores
    ("ldc", 136), ("code_layer_stride", 1000 * 128 - 16),
    ("scales", 0xC0001), ("lds", 3), ("scale_layer_stride", 3999),
])
def test_quantize_bad_arguments_rejected(lib, field, value):
    a = _quant_args()
    setattr(a, field, value)
    assert lib.ds_sel_quantize_q8(ctypes.byref(a), None) == sel.DS_SEL_E_INVALID


def test_quantize_checks_before_touching_a_device(lib):
    if os.path.exists("/dev/kfd"):
        pytest.skip("a GPU driver is present on this host")
    assert lib.ds_sel_quantize_q8(ctypes.byref(_quant_args()), None) == sel.DS_SEL_E_NODEVICE


# ------------------------------------------------------------ the per-head ReLU score
def test_head_relu_supported_where_the_heads_fit(lib):
    relu = sel.DS_SEL_FLAG_HEAD_RELU
    lim8 = dict(max_rows=8)
    assert check(lib, _args(R=6), flags=relu) == sel.DS_SEL_OK          # 6 x 64 heads x d 128
    assert check(lib, _args(R=1, H=64, d=128), flags=relu) == sel.DS_SEL_OK
    # 8 rows x 64 heads x (2 (128 + 8) + 4) bytes = 141,312 > the stage
    assert check(lib, _args(R=8), flags=relu, **lim8) == sel.DS_SEL_E_UNSUPPORTED
    assert check(lib, _args(R=8, H=48), flags=relu, **lim8) == sel.DS_SEL_OK
    # with the vector-ALU engine, or on the 8-bit stream: not built
    assert check(lib, _args(R=6), flags=relu | sel.DS_SEL_FLAG_VALU_SCORE) == sel.DS_SEL_E_UNSUPPORTED
    limits = sel.make_limits(**{**LIM, "flags": relu})
    assert lib.ds_sel_check_args_q8(ctypes.byref(limits), ctypes.byref(_q8_args()),
                                    ctypes.byref(_q8())) == sel.DS_SEL_E_UNSUPPORTED
    assert sel.selector_flags("mfma", "relu") == relu
    with pytest.raises(ValueError):
        sel.selector_flags("mfma", "tanh")


def test_decode_entry_points_reject_without_a_handle(lib):
    a = _args()
    assert lib.ds_sel_decode(None, ctypes.byref(a), None, None) == sel.DS_SEL_E_INVALID
    p = ctypes.c_void_p(77)
    assert lib.ds_sel_decode_plan_create(None, ctypes.byref(a), None, None, ctypes.byref(p)) == \
        sel.DS_SEL_E_INVALID
    assert not p.value
    assert lib.ds_sel_decode_plan_create(None, ctypes.byref(a), None, None, None) == sel.DS_SEL_E_INVALID
    assert lib.ds_sel_decode_plan_launch(None, None) == sel.DS_SEL_E_INVALID
    lib.ds_sel_decode_plan_destroy(None)
