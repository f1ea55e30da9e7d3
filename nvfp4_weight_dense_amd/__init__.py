"""Python binding of ``libnvfp4ffn.so``, the MI355X (gfx950) dense SwiGLU FFN
with NVFP4 weights.

Argument marshalling only: every step of the FFN runs in the library's HIP
kernels; PyTorch supplies device memory and the current stream.  The names
and argument order follow the C ABI in ``include/nvfp4ffn.h``.  There is no
CPU fallback: if the library is not built, importing works but every call
raises :class:`Nvfp4LibraryMissing`.

Tensors: activations are ``torch.bfloat16`` ``[rows, cols]`` contiguous on
the GPU; a weight is any object with ``codes`` (uint8 ``[n, k/2]``),
``scales`` (uint8 ``[n, k/16]``, E4M3 bits) and ``tensor_scale`` (or
``ts``) -- see :class:`NVFP4Weight`; a W8A8 weight has ``codes`` (uint8
``[n, k]``, E4M3 bits) and ``scales`` (float32 ``[ceil(n/128),
ceil(k/128)]``) -- see :class:`FP8Weight`.
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libnvfp4ffn.so")

NVFP4_OK = 0
NVFP4_EINVAL = -1
NVFP4_ESHAPE = -2
NVFP4_ENOMEM = -3
NVFP4_EHIP = -4

__all__ = [
    "NVFP4Weight", "Nvfp4Error", "Nvfp4LibraryMissing",
    "nvfp4_gemm_w4a16", "nvfp4_gemm_w4a4", "nvfp4_quantize_rows", "silu_mul",
    "dense_ffn_forward_noalloc",
    "nvfp4_gate_up_silu_w4a16", "dense_ffn_forward", "dense_ffn_forward_w4a4",
    "nvfp4_gate_up_views", "dense_ffn_forward_fused", "LoraPair", "nvfp4_lora_delta",
    "dense_ffn_forward_lora", "FP8Weight", "fp8_quantize_rows", "fp8_gemm_w8a8",
    "dense_ffn_forward_w8a8", "Q2Weight", "q2_gemm_w2a16", "dense_ffn_forward_q2",
    "nvfp4_last_error", "nvfp4_release", "nvfp4_abi_version", "load_library",
    "nvfp4_probe_mfma_bf16",
    "nvfp4_probe_read",
    "nvfp4_probe_encode",
]


class Nvfp4Error(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"nvfp4ffn error {code}: {message}")
        self.code = code


class Nvfp4LibraryMissing(RuntimeError):
    pass


class _CWeight(ctypes.Structure):
    _fields_ = [
        ("codes", ctypes.c_void_p),
        ("scales", ctypes.c_void_p),
        ("tensor_scale", ctypes.c_float),
        ("n", ctypes.c_int32),
        ("k", ctypes.c_int32),
    ]


class _CLoraPair(ctypes.Structure):
    _fields_ = [
        ("a", ctypes.c_void_p),
        ("b", ctypes.c_void_p),
        ("rank", ctypes.c_int32),
        ("scale", ctypes.c_float),
    ]


class _CLora(ctypes.Structure):
    _fields_ = [("gate", _CLoraPair), ("up", _CLoraPair), ("down", _CLoraPair)]


@dataclass
class LoraPair:
    """One LoRA pair on the GPU: dW = scale * b . a, a bf16 [rank, k], b bf16 [n, rank]."""
    a: torch.Tensor
    b: torch.Tensor
    scale: float = 1.0


@dataclass
class NVFP4Weight:
    """One NVFP4 matrix W[n][k] on the GPU."""
    codes: torch.Tensor    # uint8 [n, k/2], even k in the low nibble
    scales: torch.Tensor   # uint8 [n, k/16], E4M3FN bit patterns
    tensor_scale: float = 1.0


@dataclass
class FP8Weight:
    """One block-scaled FP8 matrix W[n][k] on the GPU."""
    codes: torch.Tensor   # uint8 [n, k], E4M3FN bit patterns
    scales: torch.Tensor  # float32 [ceil(n/128), ceil(k/128)]


class _CFp8Weight(ctypes.Structure):
    _fields_ = [
        ("codes", ctypes.c_void_p),
        ("scales", ctypes.c_void_p),
        ("n", ctypes.c_int32),
        ("k", ctypes.c_int32),
    ]


@dataclass
class Q2Weight:
    """One packed-Q2 matrix W[n][k] on the GPU."""
    codes: torch.Tensor   # uint8 [n, k/4], element 4j+i in bits 2i..2i+1 of byte j
    scales: torch.Tensor  # fp16 (or its uint16/int16 bits) [n, k/group]
    group: int = 128


class _CQ2Weight(ctypes.Structure):
    _fields_ = [
        ("codes", ctypes.c_void_p),
        ("scales", ctypes.c_void_p),
        ("group", ctypes.c_int32),
        ("n", ctypes.c_int32),
        ("k", ctypes.c_int32),
    ]


_lib = None


def load_library(path: str = LIB_PATH):
    """Load the C-ABI library and declare its signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise Nvfp4LibraryMissing(
            f"{path} is not built; run `python -m nvfp4_weight_dense_amd.build`")
    L = ctypes.CDLL(path)
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    wp = ctypes.POINTER(_CWeight)
    sig = {
        "nvfp4_gemm_w4a16": [vp, i32, wp, vp, vp],
        "nvfp4_gemm_w4a4": [vp, i32, wp, vp, vp],
        "nvfp4_quantize_rows": [vp, i32, i32, vp, vp, vp, vp],
        "silu_mul": [vp, vp, vp, i64, vp],
        "nvfp4_gate_up_silu_w4a16": [vp, i32, wp, wp, vp, vp],
        "dense_ffn_forward": [vp, i32, i32, i32, wp, wp, wp, vp, vp],
        "dense_ffn_forward_w4a4": [vp, i32, i32, i32, wp, wp, wp, vp, vp],
        "dense_ffn_forward_noalloc": [vp, i32, i32, i32, wp, wp, wp, vp, vp],
        "nvfp4_gate_up_views": [wp, wp, wp],
        "dense_ffn_forward_fused": [vp, i32, i32, i32, wp, wp, vp, vp],
        "nvfp4_lora_delta": [vp, i32, i32, ctypes.POINTER(_CLoraPair), i32, vp, vp],
        "dense_ffn_forward_lora": [vp, i32, i32, i32, wp, wp, wp, ctypes.POINTER(_CLora), vp, vp],
        "q2_gemm_w2a16": [vp, i32, ctypes.POINTER(_CQ2Weight), vp, vp],
        "dense_ffn_forward_q2": [vp, i32, i32, i32, ctypes.POINTER(_CQ2Weight),
                                 ctypes.POINTER(_CQ2Weight), ctypes.POINTER(_CQ2Weight), vp, vp],
        "fp8_quantize_rows": [vp, i32, i32, vp, vp, vp],
        "fp8_gemm_w8a8": [vp, i32, ctypes.POINTER(_CFp8Weight), vp, vp],
        "dense_ffn_forward_w8a8": [vp, i32, i32, i32, ctypes.POINTER(_CFp8Weight),
                                   ctypes.POINTER(_CFp8Weight), ctypes.POINTER(_CFp8Weight), vp, vp],
    }
    for name, args in sig.items():
        f = getattr(L, name)
        f.argtypes = args
        f.restype = ctypes.c_int
    L.nvfp4_probe_mfma_bf16.argtypes = [i32, i32, vp, vp]
    L.nvfp4_probe_mfma_bf16.restype = ctypes.c_int
    L.nvfp4_probe_read.argtypes = [vp, i64, ctypes.c_uint32, vp, vp]
    L.nvfp4_probe_read.restype = ctypes.c_int
    L.nvfp4_probe_encode.argtypes = [vp, i64, ctypes.c_float, vp, vp, vp, vp]
    L.nvfp4_probe_encode.restype = ctypes.c_int
    L.nvfp4_last_error.argtypes = []
    L.nvfp4_last_error.restype = ctypes.c_char_p
    L.nvfp4_release.argtypes = []
    L.nvfp4_release.restype = None
    L.nvfp4_abi_version.argtypes = []
    L.nvfp4_abi_version.restype = ctypes.c_int32
    _lib = L
    return L


# ---- marshalling helpers -------------------------------------------------------

def _ptr(t: torch.Tensor | None):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _check(rc: int):
    if rc != NVFP4_OK:
        raise Nvfp4Error(rc, nvfp4_last_error())


def _act(t: torch.Tensor, name: str, k: int | None = None) -> torch.Tensor:
    """A bf16 [rows, cols] activation; with k, cols must equal k."""
    if not isinstance(t, torch.Tensor) or t.dtype != torch.bfloat16 or t.dim() != 2 \
            or not t.is_contiguous():
        raise ValueError(f"{name}: expected a contiguous 2-D bfloat16 tensor")
    if k is not None and t.shape[1] != k:
        raise ValueError(f"{name}: has {t.shape[1]} columns, the weight has k={k}")
    return t


def _out(t: torch.Tensor | None, m: int, n: int, like: torch.Tensor, name: str) -> torch.Tensor:
    """A caller's bf16 [m, n] output (checked), or a new one on like's device."""
    if t is None:
        return torch.empty((m, n), dtype=torch.bfloat16, device=like.device)
    if not isinstance(t, torch.Tensor) or t.dtype != torch.bfloat16 or t.dim() != 2 \
            or tuple(t.shape) != (m, n) or not t.is_contiguous():
        got = tuple(t.shape) if isinstance(t, torch.Tensor) else type(t).__name__
        raise ValueError(f"{name}: expected a contiguous bfloat16 [{m}, {n}] tensor, got {got}")
    return t


def _gpu(first: torch.Tensor, *rest):
    """Every tensor on the GPU, on first's device (checked after the shapes)."""
    if not first.is_cuda:
        raise ValueError("expected GPU tensors")
    for t in rest:
        if t is not None and t.device != first.device:
            raise ValueError(f"tensors on {t.device} and {first.device}: expected one device")


def _cweight(w) -> _CWeight:
    codes, scales = w.codes, w.scales
    ts = getattr(w, "tensor_scale", None)
    if ts is None:
        ts = w.ts
    for t, nm in ((codes, "codes"), (scales, "scales")):
        if t.dtype != torch.uint8 or t.dim() != 2 or not t.is_contiguous():
            raise ValueError(f"weight {nm}: expected a contiguous 2-D uint8 tensor")
    n, half_k = codes.shape
    if tuple(scales.shape) != (n, (2 * half_k) // 16):
        raise ValueError(f"weight scales: expected [n={n}, k/16={(2 * half_k) // 16}], "
                         f"got {tuple(scales.shape)}")
    return _CWeight(codes.data_ptr(), scales.data_ptr(), float(ts), int(n), int(half_k * 2))


def _wt(w):
    """The weight's tensors (for the device check)."""
    return (w.codes, w.scales)


# ---- C ABI, same names --------------------------------------------------------

def nvfp4_abi_version() -> int:
    return int(load_library().nvfp4_abi_version())


def nvfp4_last_error() -> str:
    return load_library().nvfp4_last_error().decode()


def nvfp4_release() -> None:
    load_library().nvfp4_release()


def nvfp4_probe_mfma_bf16(workgroups: int, iters: int, sink: torch.Tensor, stream=None) -> None:
    """Enqueue the register-only bf16 MFMA loop (a measurement aid):
    workgroups * 4 * iters * 4 * 32768 flops; sink is a float32 GPU tensor of
    at least 256 elements."""
    L = load_library()
    if sink.dtype != torch.float32 or sink.numel() < 256 or not sink.is_cuda:
        raise ValueError("sink: expected a float32 GPU tensor of at least 256 elements")
    _check(L.nvfp4_probe_mfma_bf16(int(workgroups), int(iters), _ptr(sink), _stream(stream)))


def nvfp4_probe_read(src: torch.Tensor, nbytes: int, never: int, sink: torch.Tensor, stream=None) -> None:
    """Enqueue one streaming read of the first nbytes bytes of src (a
    measurement aid; a contiguous GPU tensor, nbytes a multiple of 16 within
    it); sink is a float32 GPU tensor of at least 256 elements, written only
    if the xor fold of the bytes equals `never`."""
    L = load_library()
    if not src.is_cuda or not src.is_contiguous() or nbytes > src.numel() * src.element_size():
        raise ValueError("src: expected a contiguous GPU tensor holding nbytes bytes")
    if sink.dtype != torch.float32 or sink.numel() < 256 or not sink.is_cuda:
        raise ValueError("sink: expected a float32 GPU tensor of at least 256 elements")
    _check(L.nvfp4_probe_read(_ptr(src), int(nbytes), int(never) & 0xFFFFFFFF, _ptr(sink), _stream(stream)))


def nvfp4_probe_encode(x: torch.Tensor, d: float, stream=None):
    """The activation quantizers' division and rounding steps on arbitrary
    values (a test aid): x a contiguous float32 GPU tensor with a multiple of
    8 elements, d a positive finite divisor.  Returns (q, e2m1, e4m3): q =
    x / d as the quantizers divide (fp32), and the E2M1 code and E4M3FN byte
    of each x (uint8), as the quantizers encode."""
    L = load_library()
    if not x.is_cuda or x.dtype != torch.float32 or not x.is_contiguous() or x.numel() % 8 != 0 \
            or x.numel() == 0:
        raise ValueError("x: expected a contiguous float32 GPU tensor, a positive multiple of 8 elements")
    q = torch.empty_like(x)
    e2m1 = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    e4m3 = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    _check(L.nvfp4_probe_encode(_ptr(x), x.numel(), float(d), _ptr(q), _ptr(e2m1), _ptr(e4m3),
                                _stream(stream)))
    return q, e2m1, e4m3


def nvfp4_gemm_w4a16(x: torch.Tensor, w, y: torch.Tensor | None = None, stream=None):
    """y = bf16(x . W^T); x [m, k] bf16 -> y [m, n] bf16."""
    L = load_library()
    cw = _cweight(w)
    x = _act(x, "x", cw.k)
    y = _out(y, x.shape[0], cw.n, x, "y")
    _gpu(x, y, *_wt(w))
    _check(L.nvfp4_gemm_w4a16(_ptr(x), x.shape[0], ctypes.byref(cw), _ptr(y), _stream(stream)))
    return y


def nvfp4_gemm_w4a4(x: torch.Tensor, w, y: torch.Tensor | None = None, stream=None):
    """W4A4 projection: x quantized per row to NVFP4, then x_q . W^T."""
    L = load_library()
    cw = _cweight(w)
    x = _act(x, "x", cw.k)
    y = _out(y, x.shape[0], cw.n, x, "y")
    _gpu(x, y, *_wt(w))
    _check(L.nvfp4_gemm_w4a4(_ptr(x), x.shape[0], ctypes.byref(cw), _ptr(y), _stream(stream)))
    return y


def nvfp4_quantize_rows(x: torch.Tensor, stream=None):
    """Per-row NVFP4 quantizer -> (codes [m, k/2], scales [m, k/16], row_scale [m])."""
    L = load_library()
    x = _act(x, "x")
    _gpu(x)
    m, k = x.shape
    codes = torch.empty((m, k // 2), dtype=torch.uint8, device=x.device)
    scales = torch.empty((m, k // 16), dtype=torch.uint8, device=x.device)
    rs = torch.empty((m,), dtype=torch.float32, device=x.device)
    _check(L.nvfp4_quantize_rows(_ptr(x), m, k, _ptr(codes), _ptr(scales), _ptr(rs),
                                 _stream(stream)))
    return codes, scales, rs


def silu_mul(gate: torch.Tensor, up: torch.Tensor, out: torch.Tensor | None = None, stream=None):
    """out = bf16(silu(gate) * up); out may be gate."""
    L = load_library()
    for t, nm in ((gate, "gate"), (up, "up")):
        if not isinstance(t, torch.Tensor) or t.dtype != torch.bfloat16 or not t.is_contiguous():
            raise ValueError(f"silu_mul: {nm} must be a contiguous bf16 tensor")
    if gate.shape != up.shape:
        raise ValueError("silu_mul: gate and up must have one shape")
    if out is None:
        out = torch.empty_like(gate)
    elif not isinstance(out, torch.Tensor) or out.dtype != torch.bfloat16 or \
            out.shape != gate.shape or not out.is_contiguous():
        raise ValueError("silu_mul: out must be a contiguous bf16 tensor of gate's shape")
    _gpu(gate, up, out)
    _check(L.silu_mul(_ptr(gate), _ptr(up), _ptr(out), gate.numel(), _stream(stream)))
    return out


def nvfp4_gate_up_silu_w4a16(x: torch.Tensor, wg, wu, act: torch.Tensor | None = None,
                             stream=None):
    """act = bf16(silu(bf16(x.Wg^T)) * bf16(x.Wu^T))."""
    L = load_library()
    cg, cu = _cweight(wg), _cweight(wu)
    if (cg.n, cg.k) != (cu.n, cu.k):
        raise ValueError(f"wg [{cg.n}, {cg.k}] and wu [{cu.n}, {cu.k}] differ")
    x = _act(x, "x", cg.k)
    act = _out(act, x.shape[0], cg.n, x, "act")
    _gpu(x, act, *_wt(wg), *_wt(wu))
    _check(L.nvfp4_gate_up_silu_w4a16(_ptr(x), x.shape[0], ctypes.byref(cg), ctypes.byref(cu),
                                      _ptr(act), _stream(stream)))
    return act


def _ffn_shapes(x, g, u, d, out):
    """Check x [m, hidden], wg/wu [inter, hidden], wd [hidden, inter] and out
    [m, hidden]; returns (x, out, m, hidden, inter)."""
    inter, hidden = g
    if u != (inter, hidden) or d != (hidden, inter):
        raise ValueError(f"wg {list(g)}, wu {list(u)}, wd {list(d)}: expected wg/wu "
                         f"[inter, hidden] and wd [hidden, inter]")
    x = _act(x, "x", hidden)
    out = _out(out, x.shape[0], hidden, x, "out")
    return x, out, x.shape[0], hidden, inter


def _ffn(fn, x, wg, wu, wd, out, stream):
    cg, cu, cd = _cweight(wg), _cweight(wu), _cweight(wd)
    x, out, m, hidden, inter = _ffn_shapes(x, (cg.n, cg.k), (cu.n, cu.k), (cd.n, cd.k), out)
    _gpu(x, out, *_wt(wg), *_wt(wu), *_wt(wd))
    _check(fn(_ptr(x), m, hidden, inter, ctypes.byref(cg), ctypes.byref(cu), ctypes.byref(cd),
              _ptr(out), _stream(stream)))
    return out


def dense_ffn_forward(x: torch.Tensor, wg, wu, wd, out: torch.Tensor | None = None, stream=None):
    """W4A16 dense SwiGLU FFN: out = (silu(x.Wg^T) * (x.Wu^T)) . Wd^T."""
    return _ffn(load_library().dense_ffn_forward, x, wg, wu, wd, out, stream)


def dense_ffn_forward_w4a4(x: torch.Tensor, wg, wu, wd, out: torch.Tensor | None = None,
                           stream=None):
    """Fixed-format W4A4 FFN (activations quantized per row before each projection)."""
    return _ffn(load_library().dense_ffn_forward_w4a4, x, wg, wu, wd, out, stream)


def dense_ffn_forward_noalloc(x: torch.Tensor, wg, wu, wd, out: torch.Tensor | None = None,
                              stream=None):
    """dense_ffn_forward with the library's fixed device scratch instead of its
    arena: the C call allocates nothing (out, when not given, is allocated
    here by torch).  Shapes whose scratch does not fit raise Nvfp4Error
    (NVFP4_ENOMEM)."""
    return _ffn(load_library().dense_ffn_forward_noalloc, x, wg, wu, wd, out, stream)


def nvfp4_gate_up_views(fused) -> tuple[NVFP4Weight, NVFP4Weight]:
    """(gate, up) views into a fused gate+up weight [2*inter, hidden]: row
    slices of the same codes/scales storage, at the offsets the C-ABI call
    reports (checked here)."""
    L = load_library()
    cf = _cweight(fused)
    cg, cu = _CWeight(), _CWeight()
    _check(L.nvfp4_gate_up_views(ctypes.byref(cf), ctypes.byref(cg), ctypes.byref(cu)))
    inter = cg.n
    ts = float(cf.tensor_scale)
    gate = NVFP4Weight(fused.codes[:inter], fused.scales[:inter], ts)
    up = NVFP4Weight(fused.codes[inter:], fused.scales[inter:], ts)
    for view, c in ((gate, cg), (up, cu)):
        assert view.codes.data_ptr() == c.codes and view.scales.data_ptr() == c.scales
    return gate, up


def dense_ffn_forward_fused(x: torch.Tensor, wgu, wd, out: torch.Tensor | None = None,
                            stream=None):
    """W4A16 dense SwiGLU FFN on a fused gate+up weight [2*inter, hidden]."""
    L = load_library()
    cgu, cd = _cweight(wgu), _cweight(wd)
    if cgu.n % 2:
        raise ValueError(f"wgu: {cgu.n} rows, expected 2*inter")
    inter = cgu.n // 2
    x, out, m, hidden, _ = _ffn_shapes(x, (inter, cgu.k), (inter, cgu.k), (cd.n, cd.k), out)
    _gpu(x, out, *_wt(wgu), *_wt(wd))
    _check(L.dense_ffn_forward_fused(_ptr(x), m, hidden, inter, ctypes.byref(cgu), ctypes.byref(cd),
                                     _ptr(out), _stream(stream)))
    return out


def _clora_pair(p: LoraPair | None, k: int, n: int, name: str) -> _CLoraPair:
    """A LoRA pair for a delta on an [m, n] output from a [m, k] input."""
    if p is None:
        return _CLoraPair(None, None, 0, 0.0)
    for t, nm in ((p.a, "a"), (p.b, "b")):
        if not isinstance(t, torch.Tensor) or t.dtype != torch.bfloat16 or t.dim() != 2 \
                or not t.is_contiguous():
            raise ValueError(f"{name} {nm}: expected a contiguous 2-D bfloat16 tensor")
    r = p.a.shape[0]
    if tuple(p.a.shape) != (r, k) or tuple(p.b.shape) != (n, r):
        raise ValueError(f"{name}: a is [rank, k={k}] and b is [n={n}, rank], got a "
                         f"{list(p.a.shape)} and b {list(p.b.shape)}")
    return _CLoraPair(p.a.data_ptr(), p.b.data_ptr(), int(r), float(p.scale))


def _lora_t(p: LoraPair | None):
    return () if p is None else (p.a, p.b)


def nvfp4_lora_delta(x: torch.Tensor, pair: LoraPair, base: torch.Tensor, stream=None):
    """base += pair.scale * (x . a^T) . b^T in place (bf16 base [m, n])."""
    L = load_library()
    x = _act(x, "x")
    base = _act(base, "base")
    m, k = x.shape
    if base.shape[0] != m:
        raise ValueError(f"base: {base.shape[0]} rows, x has {m}")
    if pair is None:
        raise ValueError("lora_delta: pair is None")
    cp = _clora_pair(pair, k, base.shape[1], "lora pair")
    _gpu(x, base, *_lora_t(pair))
    _check(L.nvfp4_lora_delta(_ptr(x), m, k, ctypes.byref(cp), base.shape[1],
                              _ptr(base), _stream(stream)))
    return base


def dense_ffn_forward_lora(x: torch.Tensor, wg, wu, wd, gate: LoraPair | None = None,
                           up: LoraPair | None = None, down: LoraPair | None = None,
                           out: torch.Tensor | None = None, stream=None):
    """W4A16 dense SwiGLU FFN with a LoRA overlay on gate, up and down."""
    L = load_library()
    cg, cu, cd = _cweight(wg), _cweight(wu), _cweight(wd)
    x, out, m, hidden, inter = _ffn_shapes(x, (cg.n, cg.k), (cu.n, cu.k), (cd.n, cd.k), out)
    cl = _CLora(_clora_pair(gate, hidden, inter, "lora gate"), _clora_pair(up, hidden, inter, "lora up"),
                _clora_pair(down, inter, hidden, "lora down"))
    _gpu(x, out, *_wt(wg), *_wt(wu), *_wt(wd), *_lora_t(gate), *_lora_t(up), *_lora_t(down))
    _check(L.dense_ffn_forward_lora(_ptr(x), m, hidden, inter, ctypes.byref(cg), ctypes.byref(cu),
                                    ctypes.byref(cd), ctypes.byref(cl), _ptr(out), _stream(stream)))
    return out


# ---- W8A8 fixed format ----------------------------------------------------------

def _cfp8(w) -> _CFp8Weight:
    if w.codes.dtype != torch.uint8 or w.codes.dim() != 2 or not w.codes.is_contiguous():
        raise ValueError("fp8 weight codes: expected a contiguous 2-D uint8 tensor")
    if w.scales.dtype != torch.float32 or not w.scales.is_contiguous():
        raise ValueError("fp8 weight scales: expected a contiguous float32 tensor")
    n, k = w.codes.shape
    if tuple(w.scales.shape) != ((n + 127) // 128, (k + 127) // 128):
        raise ValueError("fp8 weight scales: expected [ceil(n/128), ceil(k/128)]")
    return _CFp8Weight(w.codes.data_ptr(), w.scales.data_ptr(), int(n), int(k))


def fp8_quantize_rows(x: torch.Tensor, stream=None):
    """Per-row FP8 quantizer -> (codes uint8 [m, k] E4M3, row_scale float32 [m])."""
    L = load_library()
    x = _act(x, "x")
    _gpu(x)
    m, k = x.shape
    codes = torch.empty((m, k), dtype=torch.uint8, device=x.device)
    rs = torch.empty((m,), dtype=torch.float32, device=x.device)
    _check(L.fp8_quantize_rows(_ptr(x), m, k, _ptr(codes), _ptr(rs), _stream(stream)))
    return codes, rs


def fp8_gemm_w8a8(x: torch.Tensor, w, y: torch.Tensor | None = None, stream=None):
    """W8A8 projection: x quantized per row to FP8, then x_q . W^T (block-scaled W)."""
    L = load_library()
    cw = _cfp8(w)
    x = _act(x, "x", cw.k)
    y = _out(y, x.shape[0], cw.n, x, "y")
    _gpu(x, y, *_wt(w))
    _check(L.fp8_gemm_w8a8(_ptr(x), x.shape[0], ctypes.byref(cw), _ptr(y), _stream(stream)))
    return y


def dense_ffn_forward_w8a8(x: torch.Tensor, wg, wu, wd, out: torch.Tensor | None = None,
                           stream=None):
    """Fixed-format W8A8 FFN (FP8 activations per row, block-scaled FP8 weights)."""
    L = load_library()
    cg, cu, cd = _cfp8(wg), _cfp8(wu), _cfp8(wd)
    x, out, m, hidden, inter = _ffn_shapes(x, (cg.n, cg.k), (cu.n, cu.k), (cd.n, cd.k), out)
    _gpu(x, out, *_wt(wg), *_wt(wu), *_wt(wd))
    _check(L.dense_ffn_forward_w8a8(_ptr(x), m, hidden, inter, ctypes.byref(cg), ctypes.byref(cu),
                                    ctypes.byref(cd), _ptr(out), _stream(stream)))
    return out


# ---- packed-Q2 weights ------------------------------------------------------------

def _cq2(w) -> _CQ2Weight:
    if w.codes.dtype != torch.uint8 or w.codes.dim() != 2 or not w.codes.is_contiguous():
        raise ValueError("q2 weight codes: expected a contiguous 2-D uint8 tensor")
    if w.scales.element_size() != 2 or not w.scales.is_contiguous():
        raise ValueError("q2 weight scales: expected a contiguous 16-bit tensor of fp16 bits")
    n, k4 = w.codes.shape
    if int(w.group) <= 0 or tuple(w.scales.shape) != (n, (4 * k4) // int(w.group)):
        raise ValueError("q2 weight scales: expected [n, k/group]")
    return _CQ2Weight(w.codes.data_ptr(), w.scales.data_ptr(), int(w.group), int(n), int(4 * k4))


def q2_gemm_w2a16(x: torch.Tensor, w, y: torch.Tensor | None = None, stream=None):
    """y = bf16(x . W^T) with W = bf16((q - 2) * d) from a packed-Q2 weight."""
    L = load_library()
    cw = _cq2(w)
    x = _act(x, "x", cw.k)
    y = _out(y, x.shape[0], cw.n, x, "y")
    _gpu(x, y, *_wt(w))
    _check(L.q2_gemm_w2a16(_ptr(x), x.shape[0], ctypes.byref(cw), _ptr(y), _stream(stream)))
    return y


def dense_ffn_forward_q2(x: torch.Tensor, wg, wu, wd, out: torch.Tensor | None = None,
                         stream=None):
    """Dense SwiGLU FFN on packed-Q2 weights (bf16 activations)."""
    L = load_library()
    cg, cu, cd = _cq2(wg), _cq2(wu), _cq2(wd)
    x, out, m, hidden, inter = _ffn_shapes(x, (cg.n, cg.k), (cu.n, cu.k), (cd.n, cd.k), out)
    _gpu(x, out, *_wt(wg), *_wt(wu), *_wt(wd))
    _check(L.dense_ffn_forward_q2(_ptr(x), m, hidden, inter, ctypes.byref(cg), ctypes.byref(cu),
                                  ctypes.byref(cd), _ptr(out), _stream(stream)))
    return out
