"""The C-ABI library loads and exports every function include/nvfp4ffn.h
declares; host-side argument checks reject bad calls before any launch.
CPU only: no call here reaches the GPU (every call fails validation or has
m == 0 / count == 0)."""

import ctypes
import os
import re

import pytest

import nvfp4_weight_dense_amd as nv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nvfp4ffn.h")


def _lib():
    if not os.path.exists(nv.LIB_PATH):
        from nvfp4_weight_dense_amd import build
        build.build()
    return nv.load_library()


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*([A-Za-z_][A-Za-z0-9_]*)\s*\(",
                       text, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_abi():
    names = _declared_functions()
    for want in ["nvfp4_gemm_w4a16", "nvfp4_gemm_w4a4", "silu_mul", "dense_ffn_forward",
                 "dense_ffn_forward_w4a4", "nvfp4_quantize_rows", "nvfp4_gate_up_silu_w4a16",
                 "nvfp4_gate_up_views", "dense_ffn_forward_fused", "nvfp4_lora_delta",
                 "dense_ffn_forward_lora", "fp8_quantize_rows", "fp8_gemm_w8a8",
                 "dense_ffn_forward_w8a8", "q2_gemm_w2a16", "dense_ffn_forward_q2",
                 "nvfp4_last_error", "nvfp4_release", "nvfp4_abi_version"]:
        assert want in names


def test_library_exports_every_declared_symbol():
    L = _lib()
    for name in _declared_functions():
        assert hasattr(L, name), name
    assert nv.nvfp4_abi_version() == 1


def _w(n=64, k=64, codes=0x10000, scales=0x20000):
    return nv._CWeight(codes, scales, 1.0, n, k)


def test_validation_rejects_bad_arguments_without_launching():
    L = _lib()
    x = ctypes.c_void_p(0x40000)
    y = ctypes.c_void_p(0x80000)
    s = ctypes.c_void_p(None)
    # null weight descriptor / pointers
    assert L.nvfp4_gemm_w4a16(x, 4, None, y, s) == nv.NVFP4_EINVAL
    assert "null weight descriptor" in nv.nvfp4_last_error()
    w = _w(codes=0)
    assert L.nvfp4_gemm_w4a16(x, 4, ctypes.byref(w), y, s) == nv.NVFP4_EINVAL
    # k not a multiple of 32
    w = _w(k=48)
    assert L.nvfp4_gemm_w4a16(x, 4, ctypes.byref(w), y, s) == nv.NVFP4_ESHAPE
    assert "multiple of 32" in nv.nvfp4_last_error()
    # n <= 0
    w = _w(n=0)
    assert L.nvfp4_gemm_w4a4(x, 4, ctypes.byref(w), y, s) == nv.NVFP4_ESHAPE
    # misaligned activation
    w = _w()
    assert L.nvfp4_gemm_w4a16(ctypes.c_void_p(0x40002), 4, ctypes.byref(w), y, s) == nv.NVFP4_EINVAL
    # negative m
    assert L.nvfp4_gemm_w4a16(x, -1, ctypes.byref(w), y, s) == nv.NVFP4_EINVAL
    # m == 0 is a no-op that succeeds
    assert L.nvfp4_gemm_w4a16(x, 0, ctypes.byref(w), y, s) == nv.NVFP4_OK
    assert L.nvfp4_gemm_w4a4(x, 0, ctypes.byref(w), y, s) == nv.NVFP4_OK
    # silu_mul
    assert L.silu_mul(x, None, y, 16, s) == nv.NVFP4_EINVAL
    assert L.silu_mul(x, x, y, -1, s) == nv.NVFP4_EINVAL
    assert L.silu_mul(x, x, y, 0, s) == nv.NVFP4_OK
    # quantizer
    assert L.nvfp4_quantize_rows(x, 2, 40, y, y, y, s) == nv.NVFP4_ESHAPE
    assert L.nvfp4_quantize_rows(x, 0, 64, y, y, y, s) == nv.NVFP4_OK


def test_ffn_shape_consistency_checks():
    L = _lib()
    x = ctypes.c_void_p(0x40000)
    out = ctypes.c_void_p(0x80000)
    s = ctypes.c_void_p(None)
    hidden, inter = 64, 96
    wg, wu, wd = _w(inter, hidden), _w(inter, hidden), _w(hidden, inter)
    args = lambda g, u, d: (x, 2, hidden, inter, ctypes.byref(g), ctypes.byref(u), ctypes.byref(d), out, s)
    for fn in (L.dense_ffn_forward, L.dense_ffn_forward_w4a4):
        assert fn(*args(wg, wu, _w(inter, hidden))) == nv.NVFP4_ESHAPE   # wd transposed
        assert "wd must be" in nv.nvfp4_last_error()
        assert fn(*args(_w(inter, 32), wu, wd)) == nv.NVFP4_ESHAPE        # wg k != hidden
        assert fn(x, 0, hidden, inter, ctypes.byref(wg), ctypes.byref(wu), ctypes.byref(wd),
                  out, s) == nv.NVFP4_OK
        assert fn(x, 2, 0, inter, ctypes.byref(wg), ctypes.byref(wu), ctypes.byref(wd),
                  out, s) == nv.NVFP4_ESHAPE
    assert L.nvfp4_gate_up_silu_w4a16(x, 2, ctypes.byref(wg), ctypes.byref(_w(inter, 32)), out, s) \
        == nv.NVFP4_ESHAPE


def test_gate_up_views_are_offsets_into_the_fused_buffer():
    """Host-only pointer arithmetic: no device memory is touched."""
    L = _lib()
    inter, hidden = 96, 64
    fused = _w(2 * inter, hidden)
    g, u = nv._CWeight(), nv._CWeight()
    assert L.nvfp4_gate_up_views(ctypes.byref(fused), ctypes.byref(g), ctypes.byref(u)) == nv.NVFP4_OK
    assert (g.codes, g.scales, g.n, g.k) == (0x10000, 0x20000, inter, hidden)
    assert (u.codes, u.scales, u.n, u.k) == (0x10000 + inter * hidden // 2,
                                             0x20000 + inter * hidden // 16, inter, hidden)
    assert g.tensor_scale == u.tensor_scale == 1.0
    # odd row count
    assert L.nvfp4_gate_up_views(ctypes.byref(_w(2 * inter + 1, hidden)), ctypes.byref(g),
                                 ctypes.byref(u)) == nv.NVFP4_ESHAPE
    # up's scale view would start 6 bytes in: not 16-byte aligned
    assert L.nvfp4_gate_up_views(ctypes.byref(_w(6, 32)), ctypes.byref(g),
                                 ctypes.byref(u)) == nv.NVFP4_EINVAL
    assert "up view" in nv.nvfp4_last_error()
    assert L.nvfp4_gate_up_views(ctypes.byref(fused), None, ctypes.byref(u)) == nv.NVFP4_EINVAL
    # fused FFN: shape checks, m == 0 succeeds without a launch
    x, out, s = ctypes.c_void_p(0x40000), ctypes.c_void_p(0x80000), ctypes.c_void_p(None)
    wd = _w(hidden, inter)
    fn = L.dense_ffn_forward_fused
    assert fn(x, 0, hidden, inter, ctypes.byref(fused), ctypes.byref(wd), out, s) == nv.NVFP4_OK
    assert fn(x, 2, hidden, inter + 16, ctypes.byref(fused), ctypes.byref(wd), out, s) \
        == nv.NVFP4_ESHAPE
    assert "wgu must be" in nv.nvfp4_last_error()
    assert fn(x, 2, hidden, inter, ctypes.byref(fused), ctypes.byref(_w(inter, hidden)), out, s) \
        == nv.NVFP4_ESHAPE


def test_lora_argument_checks():
    L = _lib()
    x, base, s = ctypes.c_void_p(0x40000), ctypes.c_void_p(0x80000), ctypes.c_void_p(None)
    P = nv._CLoraPair
    assert L.nvfp4_lora_delta(x, 2, 64, None, 32, base, s) == nv.NVFP4_EINVAL
    assert L.nvfp4_lora_delta(x, 2, 64, ctypes.byref(P(0x10000, 0x20000, 12, 1.0)), 32, base, s) \
        == nv.NVFP4_ESHAPE
    assert "multiple of 8" in nv.nvfp4_last_error()
    assert L.nvfp4_lora_delta(x, 2, 64, ctypes.byref(P(0x10000, 0x20000, 264, 1.0)), 32, base, s) \
        == nv.NVFP4_ESHAPE
    assert L.nvfp4_lora_delta(x, 2, 64, ctypes.byref(P(None, 0x20000, 16, 1.0)), 32, base, s) \
        == nv.NVFP4_EINVAL
    assert L.nvfp4_lora_delta(x, 2, 60, ctypes.byref(P(0x10000, 0x20000, 16, 1.0)), 32, base, s) \
        == nv.NVFP4_ESHAPE
    # rank 0 and m == 0 are no-ops
    assert L.nvfp4_lora_delta(x, 2, 64, ctypes.byref(P(None, None, 0, 1.0)), 32, base, s) == nv.NVFP4_OK
    assert L.nvfp4_lora_delta(x, 0, 64, ctypes.byref(P(0x10000, 0x20000, 16, 1.0)), 32, base, s) \
        == nv.NVFP4_OK
    # the FFN checks every pair before any launch
    hidden, inter = 64, 96
    wg, wu, wd = _w(inter, hidden), _w(inter, hidden), _w(hidden, inter)
    bad = nv._CLora(P(None, None, 0, 0.0), P(0x10000, 0x20000, 7, 1.0), P(None, None, 0, 0.0))
    assert L.dense_ffn_forward_lora(x, 2, hidden, inter, ctypes.byref(wg), ctypes.byref(wu),
                                    ctypes.byref(wd), ctypes.byref(bad), base, s) == nv.NVFP4_ESHAPE
    assert "lora.up" in nv.nvfp4_last_error()


def _f8(n=64, k=64, codes=0x10000, scales=0x20000):
    return nv._CFp8Weight(codes, scales, n, k)


def test_w8a8_argument_checks():
    L = _lib()
    x, y, s = ctypes.c_void_p(0x40000), ctypes.c_void_p(0x80000), ctypes.c_void_p(None)
    assert L.fp8_gemm_w8a8(x, 4, None, y, s) == nv.NVFP4_EINVAL
    assert L.fp8_gemm_w8a8(x, 4, ctypes.byref(_f8(scales=0)), y, s) == nv.NVFP4_EINVAL
    assert L.fp8_gemm_w8a8(x, 4, ctypes.byref(_f8(k=48)), y, s) == nv.NVFP4_ESHAPE
    assert "multiple of 32" in nv.nvfp4_last_error()
    assert L.fp8_gemm_w8a8(x, 4, ctypes.byref(_f8(scales=0x20002)), y, s) == nv.NVFP4_EINVAL
    assert "4-byte" in nv.nvfp4_last_error()
    # n*k codes beyond one 2 GiB buffer range
    assert L.fp8_gemm_w8a8(x, 4, ctypes.byref(_f8(n=1 << 20, k=1 << 12)), y, s) == nv.NVFP4_ESHAPE
    assert L.fp8_gemm_w8a8(x, 0, ctypes.byref(_f8()), y, s) == nv.NVFP4_OK
    assert L.fp8_quantize_rows(x, 2, 40, y, y, s) == nv.NVFP4_ESHAPE
    assert L.fp8_quantize_rows(x, 0, 64, y, y, s) == nv.NVFP4_OK
    assert L.fp8_quantize_rows(x, 2, 64, None, y, s) == nv.NVFP4_EINVAL
    hidden, inter = 64, 96
    wg, wu, wd = _f8(inter, hidden), _f8(inter, hidden), _f8(hidden, inter)
    fn = L.dense_ffn_forward_w8a8
    r = lambda g, u, d, m=2: fn(x, m, hidden, inter, ctypes.byref(g), ctypes.byref(u),
                                ctypes.byref(d), y, s)
    assert r(wg, wu, _f8(inter, hidden)) == nv.NVFP4_ESHAPE
    assert "wd must be" in nv.nvfp4_last_error()
    assert r(_f8(inter, 32), wu, wd) == nv.NVFP4_ESHAPE
    assert r(wg, wu, wd, m=0) == nv.NVFP4_OK
    assert r(wg, wu, wd, m=-1) == nv.NVFP4_EINVAL


def _q2(n=64, k=256, group=128, codes=0x10000, scales=0x20000):
    return nv._CQ2Weight(codes, scales, group, n, k)


def test_q2_argument_checks():
    L = _lib()
    x, y, s = ctypes.c_void_p(0x40000), ctypes.c_void_p(0x80000), ctypes.c_void_p(None)
    assert L.q2_gemm_w2a16(x, 4, None, y, s) == nv.NVFP4_EINVAL
    assert L.q2_gemm_w2a16(x, 4, ctypes.byref(_q2(codes=0)), y, s) == nv.NVFP4_EINVAL
    assert L.q2_gemm_w2a16(x, 4, ctypes.byref(_q2(k=240)), y, s) == nv.NVFP4_ESHAPE
    for bad_group in (0, 16, 96, 512):  # below 32, not a power of two, not dividing k
        assert L.q2_gemm_w2a16(x, 4, ctypes.byref(_q2(group=bad_group)), y, s) == nv.NVFP4_ESHAPE
        assert "group" in nv.nvfp4_last_error()
    assert L.q2_gemm_w2a16(x, 4, ctypes.byref(_q2(scales=0x20001)), y, s) == nv.NVFP4_EINVAL
    assert L.q2_gemm_w2a16(x, 0, ctypes.byref(_q2()), y, s) == nv.NVFP4_OK
    hidden, inter = 256, 384
    wg, wu, wd = _q2(inter, hidden), _q2(inter, hidden), _q2(hidden, inter)
    fn = L.dense_ffn_forward_q2
    r = lambda g, u, d, m=2: fn(x, m, hidden, inter, ctypes.byref(g), ctypes.byref(u),
                                ctypes.byref(d), y, s)
    assert r(wg, wu, _q2(inter, hidden)) == nv.NVFP4_ESHAPE
    assert "wd must be" in nv.nvfp4_last_error()
    assert r(wg, _q2(inter, hidden, group=64), wd) == nv.NVFP4_ESHAPE   # gate and up groups differ
    assert r(wg, wu, wd, m=0) == nv.NVFP4_OK


def test_binding_refuses_cpu_tensors():
    import torch
    _lib()
    x = torch.zeros((2, 64), dtype=torch.bfloat16)
    w = nv.NVFP4Weight(torch.zeros((8, 32), dtype=torch.uint8), torch.zeros((8, 4), dtype=torch.uint8))
    with pytest.raises(ValueError):
        nv.nvfp4_gemm_w4a16(x, w)


def _match(fn, *a, msg, **kw):
    with pytest.raises(ValueError, match=msg):
        fn(*a, **kw)


def test_binding_checks_shapes_before_any_launch():
    """Every shape the C ABI cannot see (tensor extents behind raw pointers)
    is checked by the binding and raises ValueError before the library is
    called.  CPU tensors: the shape checks run before the device check, so
    a wrong shape is reported as such."""
    import torch
    _lib()
    bf = torch.bfloat16
    u8 = torch.uint8
    W = lambda n, k, sk=None: nv.NVFP4Weight(torch.zeros((n, k // 2), dtype=u8),
                                             torch.zeros((n, sk if sk is not None else k // 16), dtype=u8))
    x = torch.zeros((2, 64), dtype=bf)
    # scales not [n, k/16]
    _match(nv.nvfp4_gemm_w4a16, x, W(8, 64, sk=3), msg="weight scales")
    # x columns != weight k
    _match(nv.nvfp4_gemm_w4a16, x, W(8, 128), msg="columns")
    _match(nv.nvfp4_gemm_w4a4, x, W(8, 128), msg="columns")
    # caller's output of the wrong shape, dtype or layout
    _match(nv.nvfp4_gemm_w4a16, x, W(8, 64), y=torch.zeros((2, 9), dtype=bf), msg=r"\[2, 8\]")
    _match(nv.nvfp4_gemm_w4a16, x, W(8, 64), y=torch.zeros((2, 8), dtype=torch.float32), msg="y:")
    _match(nv.nvfp4_gemm_w4a16, x, W(8, 64), y=torch.zeros((8, 2), dtype=bf).t(), msg="y:")
    # gate+up: weights of different shapes, act of the wrong shape
    _match(nv.nvfp4_gate_up_silu_w4a16, x, W(8, 64), W(16, 64), msg="differ")
    _match(nv.nvfp4_gate_up_silu_w4a16, x, W(8, 64), W(8, 64), act=torch.zeros((3, 8), dtype=bf),
           msg="act:")
    # FFN: wd not [hidden, inter], out of the wrong shape
    for fn in (nv.dense_ffn_forward, nv.dense_ffn_forward_w4a4):
        _match(fn, x, W(96, 64), W(96, 64), W(96, 64), msg="wd")
        _match(fn, x, W(96, 64), W(96, 64), W(64, 96), out=torch.zeros((2, 96), dtype=bf),
               msg="out:")
        _match(fn, torch.zeros((2, 32), dtype=bf), W(96, 64), W(96, 64), W(64, 96), msg="columns")
    # fused gate+up weight: odd rows, wd mismatch
    _match(nv.dense_ffn_forward_fused, x, W(97, 64), W(64, 48), msg="2\\*inter")
    _match(nv.dense_ffn_forward_fused, x, W(96, 64), W(64, 96), msg="wd")
    # LoRA: a not [rank, k], b not [n, rank], base rows != x rows
    P = lambda r, k, n: nv.LoraPair(torch.zeros((r, k), dtype=bf), torch.zeros((n, r), dtype=bf))
    base = torch.zeros((2, 8), dtype=bf)
    _match(nv.nvfp4_lora_delta, x, P(16, 32, 8), base, msg="lora pair")
    _match(nv.nvfp4_lora_delta, x, P(16, 64, 9), base, msg="lora pair")
    _match(nv.nvfp4_lora_delta, x, P(16, 64, 8), torch.zeros((3, 8), dtype=bf), msg="base")
    _match(nv.dense_ffn_forward_lora, x, W(96, 64), W(96, 64), W(64, 96), down=P(16, 64, 64),
           msg="lora down")
    # W8A8 and packed Q2: x columns and output shapes
    f8 = nv.FP8Weight(torch.zeros((8, 128), dtype=u8), torch.zeros((1, 1), dtype=torch.float32))
    _match(nv.fp8_gemm_w8a8, x, f8, msg="columns")
    q2 = nv.Q2Weight(torch.zeros((8, 32), dtype=u8), torch.zeros((8, 1), dtype=torch.int16), 128)
    _match(nv.q2_gemm_w2a16, x, q2, msg="columns")
    _match(nv.q2_gemm_w2a16, torch.zeros((2, 128), dtype=bf), q2,
           y=torch.zeros((2, 7), dtype=bf), msg="y:")
    # silu_mul: out of another shape
    g = torch.zeros((2, 8), dtype=bf)
    _match(nv.silu_mul, g, g, out=torch.zeros((2, 9), dtype=bf), msg="out")
    # shapes right, tensors on the CPU: refused as well
    _match(nv.nvfp4_gemm_w4a16, x, W(8, 64), msg="GPU")


def test_encode_probe_rejects_bad_arguments_without_launching():
    L = _lib()
    p = ctypes.c_void_p(0x40000)
    null = ctypes.c_void_p(None)
    f = ctypes.c_float
    assert L.nvfp4_probe_encode(null, 8, f(1.0), p, p, p, null) == nv.NVFP4_EINVAL
    assert L.nvfp4_probe_encode(p, 8, f(1.0), p, null, p, null) == nv.NVFP4_EINVAL
    assert L.nvfp4_probe_encode(p, 12, f(1.0), p, p, p, null) == nv.NVFP4_EINVAL
    assert L.nvfp4_probe_encode(p, 0, f(1.0), p, p, p, null) == nv.NVFP4_EINVAL
    assert L.nvfp4_probe_encode(p, 8, f(0.0), p, p, p, null) == nv.NVFP4_EINVAL
    assert L.nvfp4_probe_encode(p, 8, f(float("inf")), p, p, p, null) == nv.NVFP4_EINVAL
    assert L.nvfp4_probe_encode(p, 8, f(float("nan")), p, p, p, null) == nv.NVFP4_EINVAL
