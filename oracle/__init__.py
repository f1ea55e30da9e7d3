"""CPU oracle for the NVFP4-weight dense SwiGLU FFN (ctypes wrapper).

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
benchmark's CPU-baseline leg may import this package.  The product path (the
HIP library and its Python binding) never imports it and shares no code with
it.

The arithmetic lives in ``nvfp4_oracle.c`` (plain C, fp64 sums, closed-form
decoders); this module only builds that file with gcc and marshals numpy
arrays.  Arrays are host numpy arrays:

* activations / outputs: ``uint16`` bf16 bit patterns, ``[rows, cols]``;
* a weight is :class:`Weight` -- ``codes`` uint8 ``[n, k/2]`` (even k in the
  low nibble), ``scales`` uint8 ``[n, k/16]`` (E4M3), ``ts`` fp32.
"""

from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "nvfp4_oracle.c")
_HDR = os.path.join(_HERE, "nvfp4_oracle.h")
LIB_PATH = os.path.join(_HERE, "liboracle_nvfp4.so")


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (no fast-math, no FMA contraction)."""
    if not force and os.path.exists(LIB_PATH) and os.path.getmtime(LIB_PATH) >= max(
        os.path.getmtime(_SRC), os.path.getmtime(_HDR)
    ):
        return LIB_PATH
    tmp = LIB_PATH + ".tmp"
    cmd = [
        "gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
        "-fPIC", "-shared", "-Wall", "-o", tmp, _SRC, "-lm", "-lpthread",
    ]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


class _Weight(ctypes.Structure):
    _fields_ = [
        ("codes", ctypes.c_void_p),
        ("scales", ctypes.c_void_p),
        ("ts", ctypes.c_float),
        ("n", ctypes.c_int),
        ("k", ctypes.c_int),
    ]


_lib = None


def lib():
    global _lib
    if _lib is None:
        build(force=False)
        L = ctypes.CDLL(LIB_PATH)
        u8, u16, dbl = ctypes.c_uint8, ctypes.c_uint16, ctypes.c_double
        vp, ip = ctypes.c_void_p, ctypes.c_int
        L.nvo_e2m1_value.argtypes, L.nvo_e2m1_value.restype = [u8], dbl
        L.nvo_e4m3_value.argtypes, L.nvo_e4m3_value.restype = [u8], dbl
        L.nvo_bf16_value.argtypes, L.nvo_bf16_value.restype = [u16], dbl
        L.nvo_bf16_from_double.argtypes, L.nvo_bf16_from_double.restype = [dbl], u16
        L.nvo_e4m3_encode.argtypes, L.nvo_e4m3_encode.restype = [ctypes.c_float], u8
        L.nvo_e2m1_encode.argtypes, L.nvo_e2m1_encode.restype = [ctypes.c_float], u8
        L.nvo_silu.argtypes, L.nvo_silu.restype = [dbl], dbl
        for f in ("nvo_e4m3_encode_n", "nvo_e2m1_encode_n", "nvo_bf16_from_double_n"):
            getattr(L, f).argtypes = [vp, vp, ctypes.c_int64]
            getattr(L, f).restype = None
        L.nvo_dequant.argtypes, L.nvo_dequant.restype = [vp, vp], None
        for f in ("nvo_gemm_w4a16", "nvo_gemm_w4a4"):
            getattr(L, f).argtypes = [vp, ip, vp, vp, vp, ip]
            getattr(L, f).restype = ip
        L.nvo_silu_mul.argtypes = [vp, vp, vp, ctypes.c_int64]
        L.nvo_silu_mul.restype = None
        L.nvo_quantize_rows.argtypes = [vp, ip, ip, vp, vp, vp]
        L.nvo_quantize_rows.restype = ip
        for f in ("nvo_dense_ffn", "nvo_dense_ffn_w4a4"):
            getattr(L, f).argtypes = [vp, ip, ip, ip, vp, vp, vp, vp, vp, vp, vp, vp, ip]
            getattr(L, f).restype = ip
        L.nvo_lora_delta.argtypes = [vp, ip, ip, vp, ip, vp, vp]
        L.nvo_lora_delta.restype = ip
        L.nvo_dense_ffn_lora.argtypes = [vp, ip, ip, ip, vp, vp, vp, vp, vp, vp, vp, vp, vp, ip]
        L.nvo_dense_ffn_lora.restype = ip
        L.nvo_dequant_fp8.argtypes, L.nvo_dequant_fp8.restype = [vp, vp], None
        L.nvo_quantize_rows_fp8.argtypes = [vp, ip, ip, vp, vp]
        L.nvo_quantize_rows_fp8.restype = ip
        L.nvo_gemm_w8a8.argtypes = [vp, ip, vp, vp, vp, ip]
        L.nvo_gemm_w8a8.restype = ip
        L.nvo_dense_ffn_w8a8.argtypes = [vp, ip, ip, ip, vp, vp, vp, vp, vp, vp, vp, vp, ip]
        L.nvo_dense_ffn_w8a8.restype = ip
        L.nvo_fp16_value.argtypes, L.nvo_fp16_value.restype = [ctypes.c_uint16], dbl
        L.nvo_dequant_q2.argtypes, L.nvo_dequant_q2.restype = [vp, vp], None
        L.nvo_gemm_q2.argtypes = [vp, ip, vp, vp, vp, ip]
        L.nvo_gemm_q2.restype = ip
        L.nvo_dense_ffn_q2.argtypes = [vp, ip, ip, ip, vp, vp, vp, vp, vp, vp, vp, vp, ip]
        L.nvo_dense_ffn_q2.restype = ip
        _lib = L
    return _lib


@dataclass
class Weight:
    codes: np.ndarray   # uint8 [n, k/2]
    scales: np.ndarray  # uint8 [n, k/16]
    ts: float = 1.0

    @property
    def n(self) -> int:
        return int(self.codes.shape[0])

    @property
    def k(self) -> int:
        return int(self.codes.shape[1] * 2)

    def _struct(self):
        self.codes = np.ascontiguousarray(self.codes, dtype=np.uint8)
        self.scales = np.ascontiguousarray(self.scales, dtype=np.uint8)
        assert self.scales.shape == (self.n, self.k // 16)
        return _Weight(self.codes.ctypes.data, self.scales.ctypes.data,
                       float(self.ts), self.n, self.k)


def _p(a):
    return None if a is None else a.ctypes.data


def _u16(a):
    return np.ascontiguousarray(a, dtype=np.uint16)


# ---- scalar helpers ---------------------------------------------------------

def e2m1_value(code: int) -> float:
    return lib().nvo_e2m1_value(code)


def e4m3_value(byte: int) -> float:
    return lib().nvo_e4m3_value(byte)


def bf16_value(bits: int) -> float:
    return lib().nvo_bf16_value(bits)


def bf16_from_double(v: float) -> int:
    return lib().nvo_bf16_from_double(v)


def e4m3_encode(t: float) -> int:
    return lib().nvo_e4m3_encode(t)


def e2m1_encode(t: float) -> int:
    return lib().nvo_e2m1_encode(t)


def silu(t: float) -> float:
    return lib().nvo_silu(t)


# ---- array functions ----------------------------------------------------------

def e4m3_encode_array(t: np.ndarray) -> np.ndarray:
    t = np.ascontiguousarray(t, dtype=np.float32)
    out = np.empty(t.shape, dtype=np.uint8)
    lib().nvo_e4m3_encode_n(t.ctypes.data, out.ctypes.data, t.size)
    return out


def e2m1_encode_array(t: np.ndarray) -> np.ndarray:
    t = np.ascontiguousarray(t, dtype=np.float32)
    out = np.empty(t.shape, dtype=np.uint8)
    lib().nvo_e2m1_encode_n(t.ctypes.data, out.ctypes.data, t.size)
    return out


def bf16_from_double_array(v: np.ndarray) -> np.ndarray:
    v = np.ascontiguousarray(v, dtype=np.float64)
    out = np.empty(v.shape, dtype=np.uint16)
    lib().nvo_bf16_from_double_n(v.ctypes.data, out.ctypes.data, v.size)
    return out


def dequant(w: Weight) -> np.ndarray:
    out = np.empty((w.n, w.k), dtype=np.float64)
    s = w._struct()
    lib().nvo_dequant(ctypes.byref(s), out.ctypes.data)
    return out


def gemm_w4a16(x: np.ndarray, w: Weight, nthreads: int = 0):
    """Returns (y bf16 bits [m, n], y_exact float64 [m, n])."""
    x = _u16(x)
    m = x.shape[0]
    y = np.empty((m, w.n), dtype=np.uint16)
    ye = np.empty((m, w.n), dtype=np.float64)
    s = w._struct()
    rc = lib().nvo_gemm_w4a16(x.ctypes.data, m, ctypes.byref(s), y.ctypes.data,
                              ye.ctypes.data, nthreads)
    if rc != 0:
        raise ValueError("oracle gemm_w4a16: bad shape")
    return y, ye


def gemm_w4a4(x: np.ndarray, w: Weight, nthreads: int = 0):
    x = _u16(x)
    m = x.shape[0]
    y = np.empty((m, w.n), dtype=np.uint16)
    ye = np.empty((m, w.n), dtype=np.float64)
    s = w._struct()
    rc = lib().nvo_gemm_w4a4(x.ctypes.data, m, ctypes.byref(s), y.ctypes.data,
                             ye.ctypes.data, nthreads)
    if rc != 0:
        raise ValueError("oracle gemm_w4a4: bad shape")
    return y, ye


def silu_mul(g: np.ndarray, u: np.ndarray) -> np.ndarray:
    g, u = _u16(g), _u16(u)
    assert g.shape == u.shape
    out = np.empty_like(g)
    lib().nvo_silu_mul(g.ctypes.data, u.ctypes.data, out.ctypes.data, g.size)
    return out


def quantize_rows(x: np.ndarray):
    """Returns (codes uint8 [m, k/2], scales uint8 [m, k/16], row_scale f32 [m])."""
    x = _u16(x)
    m, k = x.shape
    codes = np.zeros((m, k // 2), dtype=np.uint8)
    scales = np.zeros((m, k // 16), dtype=np.uint8)
    rs = np.zeros((m,), dtype=np.float32)
    rc = lib().nvo_quantize_rows(x.ctypes.data, m, k, codes.ctypes.data,
                                 scales.ctypes.data, rs.ctypes.data)
    if rc != 0:
        raise ValueError("oracle quantize_rows: bad shape")
    return codes, scales, rs


def dense_ffn(x: np.ndarray, wg: Weight, wu: Weight, wd: Weight, w4a4: bool = False,
              nthreads: int = 0, intermediates: bool = False):
    """Returns y bf16 [m, hidden], y_exact f64 [m, hidden] (+ g, u, a)."""
    x = _u16(x)
    m, hidden = x.shape
    inter = wg.n
    y = np.empty((m, hidden), dtype=np.uint16)
    ye = np.empty((m, hidden), dtype=np.float64)
    g = u = a = None
    if intermediates:
        g = np.empty((m, inter), dtype=np.uint16)
        u = np.empty((m, inter), dtype=np.uint16)
        a = np.empty((m, inter), dtype=np.uint16)
    sg, su, sd = wg._struct(), wu._struct(), wd._struct()
    f = lib().nvo_dense_ffn_w4a4 if w4a4 else lib().nvo_dense_ffn
    rc = f(x.ctypes.data, m, hidden, inter, ctypes.byref(sg), ctypes.byref(su),
           ctypes.byref(sd), y.ctypes.data, ye.ctypes.data, _p(g), _p(u), _p(a),
           nthreads)
    if rc != 0:
        raise ValueError("oracle dense_ffn: bad shapes")
    if intermediates:
        return y, ye, g, u, a
    return y, ye


class _Lora(ctypes.Structure):
    _fields_ = [
        ("a", ctypes.c_void_p),
        ("b", ctypes.c_void_p),
        ("r", ctypes.c_int),
        ("scale", ctypes.c_float),
    ]


@dataclass
class Lora:
    """One LoRA pair: ``a`` bf16 bits [r, k], ``b`` bf16 bits [n, r]; dW = scale * B . A."""
    a: np.ndarray
    b: np.ndarray
    scale: float = 1.0

    def _struct(self) -> "_Lora":
        self.a = _u16(self.a)
        self.b = _u16(self.b)
        return _Lora(self.a.ctypes.data, self.b.ctypes.data, int(self.a.shape[0]), float(self.scale))


def _lora_ref(l):
    return None if l is None else ctypes.byref(l._struct())


def lora_delta(x: np.ndarray, l: Lora, base: np.ndarray):
    """Returns (bf16(base + dW . x) bits, the double value before rounding)."""
    x = _u16(x)
    out = _u16(base).copy()
    m, k = x.shape
    n = out.shape[1]
    ex = np.empty(out.shape, dtype=np.float64)
    s = l._struct()
    rc = lib().nvo_lora_delta(x.ctypes.data, m, k, ctypes.byref(s), n, out.ctypes.data,
                              ex.ctypes.data)
    if rc != 0:
        raise ValueError("oracle lora_delta: bad shape")
    return out, ex


def dense_ffn_lora(x: np.ndarray, wg: Weight, wu: Weight, wd: Weight, lg: Lora | None,
                   lu: Lora | None, ld: Lora | None, nthreads: int = 0,
                   intermediates: bool = False):
    """W4A16 FFN with LoRA pairs (None = absent).  Returns (y, y_exact[, a])."""
    x = _u16(x)
    m, hidden = x.shape
    inter = wg.n
    y = np.empty((m, hidden), dtype=np.uint16)
    ye = np.empty((m, hidden), dtype=np.float64)
    a = np.empty((m, inter), dtype=np.uint16)
    structs = [None if l is None else l._struct() for l in (lg, lu, ld)]
    refs = [None if s is None else ctypes.byref(s) for s in structs]
    sg, su, sd = wg._struct(), wu._struct(), wd._struct()
    rc = lib().nvo_dense_ffn_lora(x.ctypes.data, m, hidden, inter, ctypes.byref(sg),
                                  ctypes.byref(su), ctypes.byref(sd), refs[0], refs[1], refs[2],
                                  y.ctypes.data, ye.ctypes.data, a.ctypes.data, nthreads)
    if rc != 0:
        raise ValueError("oracle dense_ffn_lora: bad shapes")
    return (y, ye, a) if intermediates else (y, ye)


# ---- W8A8 fixed format --------------------------------------------------------

class _Fp8Weight(ctypes.Structure):
    _fields_ = [
        ("codes", ctypes.c_void_p),
        ("scales", ctypes.c_void_p),
        ("n", ctypes.c_int),
        ("k", ctypes.c_int),
    ]


@dataclass
class Fp8Weight:
    """Block-scaled FP8 weight: ``codes`` uint8 E4M3 ``[n, k]``, ``scales``
    float32 ``[ceil(n/128), ceil(k/128)]`` (one per 128 x 128 block)."""
    codes: np.ndarray
    scales: np.ndarray

    @property
    def n(self) -> int:
        return int(self.codes.shape[0])

    @property
    def k(self) -> int:
        return int(self.codes.shape[1])

    def _struct(self):
        self.codes = np.ascontiguousarray(self.codes, dtype=np.uint8)
        self.scales = np.ascontiguousarray(self.scales, dtype=np.float32)
        assert self.scales.shape == ((self.n + 127) // 128, (self.k + 127) // 128)
        return _Fp8Weight(self.codes.ctypes.data, self.scales.ctypes.data, self.n, self.k)


def dequant_fp8(w: Fp8Weight) -> np.ndarray:
    out = np.empty((w.n, w.k), dtype=np.float64)
    s = w._struct()
    lib().nvo_dequant_fp8(ctypes.byref(s), out.ctypes.data)
    return out


def quantize_rows_fp8(x: np.ndarray):
    """Returns (codes uint8 [m, k] E4M3, row_scale f32 [m])."""
    x = _u16(x)
    m, k = x.shape
    codes = np.zeros((m, k), dtype=np.uint8)
    rs = np.zeros((m,), dtype=np.float32)
    rc = lib().nvo_quantize_rows_fp8(x.ctypes.data, m, k, codes.ctypes.data, rs.ctypes.data)
    if rc != 0:
        raise ValueError("oracle quantize_rows_fp8: bad shape")
    return codes, rs


def gemm_w8a8(x: np.ndarray, w: Fp8Weight, nthreads: int = 0):
    """Returns (y bf16 bits [m, n], y_exact float64 [m, n])."""
    x = _u16(x)
    m = x.shape[0]
    y = np.empty((m, w.n), dtype=np.uint16)
    ye = np.empty((m, w.n), dtype=np.float64)
    s = w._struct()
    rc = lib().nvo_gemm_w8a8(x.ctypes.data, m, ctypes.byref(s), y.ctypes.data,
                             ye.ctypes.data, nthreads)
    if rc != 0:
        raise ValueError("oracle gemm_w8a8: bad shape")
    return y, ye


def dense_ffn_w8a8(x: np.ndarray, wg: Fp8Weight, wu: Fp8Weight, wd: Fp8Weight,
                   nthreads: int = 0, intermediates: bool = False):
    """W8A8 FFN.  Returns (y bf16 [m, hidden], y_exact f64[, g, u, a])."""
    x = _u16(x)
    m, hidden = x.shape
    inter = wg.n
    y = np.empty((m, hidden), dtype=np.uint16)
    ye = np.empty((m, hidden), dtype=np.float64)
    g = np.empty((m, inter), dtype=np.uint16)
    u = np.empty((m, inter), dtype=np.uint16)
    a = np.empty((m, inter), dtype=np.uint16)
    sg, su, sd = wg._struct(), wu._struct(), wd._struct()
    rc = lib().nvo_dense_ffn_w8a8(x.ctypes.data, m, hidden, inter, ctypes.byref(sg),
                                  ctypes.byref(su), ctypes.byref(sd), y.ctypes.data,
                                  ye.ctypes.data, g.ctypes.data, u.ctypes.data,
                                  a.ctypes.data, nthreads)
    if rc != 0:
        raise ValueError("oracle dense_ffn_w8a8: bad shapes")
    return (y, ye, g, u, a) if intermediates else (y, ye)


# ---- packed-Q2 weights ----------------------------------------------------------

class _Q2Weight(ctypes.Structure):
    _fields_ = [
        ("codes", ctypes.c_void_p),
        ("scales", ctypes.c_void_p),
        ("group", ctypes.c_int),
        ("n", ctypes.c_int),
        ("k", ctypes.c_int),
    ]


@dataclass
class Q2Weight:
    """Packed-Q2 weight: ``codes`` uint8 ``[n, k/4]`` (element 4j+i in bits
    2i..2i+1 of byte j), ``scales`` uint16 fp16 bits ``[n, k/group]``."""
    codes: np.ndarray
    scales: np.ndarray
    group: int = 128

    @property
    def n(self) -> int:
        return int(self.codes.shape[0])

    @property
    def k(self) -> int:
        return int(self.codes.shape[1] * 4)

    def _struct(self):
        self.codes = np.ascontiguousarray(self.codes, dtype=np.uint8)
        self.scales = np.ascontiguousarray(self.scales, dtype=np.uint16)
        assert self.scales.shape == (self.n, self.k // self.group)
        return _Q2Weight(self.codes.ctypes.data, self.scales.ctypes.data, int(self.group),
                         self.n, self.k)


def fp16_value(h: int) -> float:
    return lib().nvo_fp16_value(h)


def dequant_q2(w: Q2Weight) -> np.ndarray:
    out = np.empty((w.n, w.k), dtype=np.float64)
    s = w._struct()
    lib().nvo_dequant_q2(ctypes.byref(s), out.ctypes.data)
    return out


def gemm_q2(x: np.ndarray, w: Q2Weight, nthreads: int = 0):
    """Returns (y bf16 bits [m, n], y_exact float64 [m, n])."""
    x = _u16(x)
    m = x.shape[0]
    y = np.empty((m, w.n), dtype=np.uint16)
    ye = np.empty((m, w.n), dtype=np.float64)
    s = w._struct()
    rc = lib().nvo_gemm_q2(x.ctypes.data, m, ctypes.byref(s), y.ctypes.data, ye.ctypes.data,
                           nthreads)
    if rc != 0:
        raise ValueError("oracle gemm_q2: bad shape")
    return y, ye


def dense_ffn_q2(x: np.ndarray, wg: Q2Weight, wu: Q2Weight, wd: Q2Weight, nthreads: int = 0,
                 intermediates: bool = False):
    """Packed-Q2 FFN.  Returns (y bf16 [m, hidden], y_exact f64[, g, u, a])."""
    x = _u16(x)
    m, hidden = x.shape
    inter = wg.n
    y = np.empty((m, hidden), dtype=np.uint16)
    ye = np.empty((m, hidden), dtype=np.float64)
    g = np.empty((m, inter), dtype=np.uint16)
    u = np.empty((m, inter), dtype=np.uint16)
    a = np.empty((m, inter), dtype=np.uint16)
    sg, su, sd = wg._struct(), wu._struct(), wd._struct()
    rc = lib().nvo_dense_ffn_q2(x.ctypes.data, m, hidden, inter, ctypes.byref(sg),
                                ctypes.byref(su), ctypes.byref(sd), y.ctypes.data,
                                ye.ctypes.data, g.ctypes.data, u.ctypes.data, a.ctypes.data,
                                nthreads)
    if rc != 0:
        raise ValueError("oracle dense_ffn_q2: bad shapes")
    return (y, ye, g, u, a) if intermediates else (y, ye)
