"""Seeded synthetic inputs for the dense NVFP4 FFN workloads.

Shared by the tests, the benchmark and the smoke check as *inputs* only: it
holds none of the FFN's arithmetic (no NVFP4 decode, no GEMM, no quantizer).
Value distributions are drawn with torch's CPU generator and cast with torch's
own dtype conversions; no trained weights or datasets are involved.

Workloads (the pages quote no shapes for their FFN measurements, so these
stand in for them):

* ``tiny``     m=4, hidden=256, inter=768
* ``decode``   m=1, hidden=4096, inter=12288 (single-row decode)
* ``smallm``   m=64, hidden=5120, inter=17408 (deep-K down projection)
* ``prefill``  m=2048, hidden=5120, inter=17408, 1% of X entries x20
* ``w4a4``     hidden=4096, inter=14336, m in {1, 8, 64, 512} sharing rows
* ``w8a8``     the same shapes and rows, with block-scaled FP8 weights
* ``decode_tp8``, ``prefill_tp8``  one GPU's share of the decode / prefill
  FFN under 8-way tensor parallelism (inter 1536 / 2176)

Weight recipe: E2M1 codes uniform over all 16 nibbles (so -0 appears),
E4M3 block scales 2^u with u ~ U(-4, 0) cast to float8_e4m3fn by torch,
tensor scale 1.0.  X ~ N(0, 1) cast to bf16 by torch.

Packed-Q2 weight recipe: 2-bit codes uniform over 0..3, one fp16 scale per
group of 128 K elements drawn as 2^u with u ~ U(-4, 0) cast to float16 by
torch (11-bit mantissas, so the bf16 dequantization rounds).

FP8 weight recipe (W8A8): E4M3 codes uniform over the 254 non-NaN bytes (so
subnormals, -0 and +-448 appear), one fp32 scale per 128 x 128 block drawn
as 2^u with u ~ U(-10, -6) (not powers of two in general).
"""

from __future__ import annotations

from dataclasses import dataclass

import torch

WORKLOADS = {
    "tiny": dict(m=4, hidden=256, inter=768, outliers=False),
    "decode": dict(m=1, hidden=4096, inter=12288, outliers=False),
    "smallm": dict(m=64, hidden=5120, inter=17408, outliers=False),
    "prefill": dict(m=2048, hidden=5120, inter=17408, outliers=True),
    "w4a4": dict(m=512, hidden=4096, inter=14336, outliers=False),
    "w8a8": dict(m=512, hidden=4096, inter=14336, outliers=False),
    # one GPU's share under 8-way tensor parallelism (inter split 8 ways):
    # the decode and prefill shapes as each shard runs them
    "decode_tp8": dict(m=1, hidden=4096, inter=12288 // 8, outliers=False),
    "prefill_tp8": dict(m=2048, hidden=5120, inter=17408 // 8, outliers=True),
}

W4A4_ROW_COUNTS = (1, 8, 64, 512)
W8A8_ROW_COUNTS = (1, 8, 64, 512)

# stream ids under one seed
_X, _WG_C, _WG_S, _WU_C, _WU_S, _WD_C, _WD_S, _OUTLIER = range(8)
_LORA = 8  # LoRA pairs: streams 8..13
_FP8 = 16  # FP8 weights: streams 16..21 (codes, scales per matrix)
_Q2 = 24   # packed-Q2 weights: streams 24..29
Q2_GROUP = 128


def _gen(seed: int, stream: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(seed * 256 + stream)
    return g


@dataclass
class NvWeight:
    """Host (or device) tensors of one NVFP4 matrix [n, k]."""
    codes: torch.Tensor   # uint8 [n, k/2]
    scales: torch.Tensor  # uint8 [n, k/16] (E4M3 bit patterns)
    ts: float = 1.0

    @property
    def n(self) -> int:
        return int(self.codes.shape[0])

    @property
    def k(self) -> int:
        return int(self.codes.shape[1] * 2)

    def to(self, device) -> "NvWeight":
        return NvWeight(self.codes.to(device), self.scales.to(device), self.ts)


def activations(m: int, k: int, seed: int = 0, outliers: bool = False,
                stream: int = _X) -> torch.Tensor:
    """bf16 [m, k], N(0,1); with outliers, each entry x20 with p = 0.01."""
    x = torch.randn((m, k), generator=_gen(seed, stream), dtype=torch.float32)
    if outliers:
        mask = torch.rand((m, k), generator=_gen(seed, _OUTLIER)) < 0.01
        x = torch.where(mask, x * 20.0, x)
    return x.to(torch.bfloat16)


def weight(n: int, k: int, seed: int, code_stream: int, scale_stream: int,
           ts: float = 1.0) -> NvWeight:
    assert k % 32 == 0
    codes = torch.randint(0, 256, (n, k // 2), generator=_gen(seed, code_stream),
                          dtype=torch.uint8)
    u = torch.rand((n, k // 16), generator=_gen(seed, scale_stream),
                   dtype=torch.float32) * -4.0
    scales = torch.exp2(u).to(torch.float8_e4m3fn).view(torch.uint8)
    return NvWeight(codes, scales.contiguous(), ts)


def lora_pair(n: int, k: int, rank: int, seed: int = 0, which: int = 0):
    """One LoRA pair (a bf16 [rank, k] ~ N(0, 1/k), b bf16 [n, rank] ~ N(0, 1)),
    so that x . a^T has about the scale of x; ``which`` (0 gate, 1 up, 2 down)
    picks the generator streams."""
    sa, sb = _LORA + 2 * which, _LORA + 2 * which + 1
    a = torch.randn((rank, k), generator=_gen(seed, sa), dtype=torch.float32) / (k ** 0.5)
    b = torch.randn((n, rank), generator=_gen(seed, sb), dtype=torch.float32)
    return a.to(torch.bfloat16), b.to(torch.bfloat16)


def ffn_weights(hidden: int, inter: int, seed: int = 0):
    wg = weight(inter, hidden, seed, _WG_C, _WG_S)
    wu = weight(inter, hidden, seed, _WU_C, _WU_S)
    wd = weight(hidden, inter, seed, _WD_C, _WD_S)
    return wg, wu, wd


def workload(name: str, seed: int = 0, m: int | None = None):
    """(x bf16 [m, hidden], wg, wu, wd) on the CPU."""
    spec = WORKLOADS[name]
    rows = spec["m"] if m is None else m
    x = activations(rows, spec["hidden"], seed, spec["outliers"])
    return (x,) + ffn_weights(spec["hidden"], spec["inter"], seed)


def exact_case(m: int, n: int, k: int, seed: int = 0):
    """Inputs on which every fp32 partial sum is exact: X integer in [-2, 2],
    block scales powers of two in [2^-4, 1], tensor scale 1.  Any summation
    order then gives the same fp32 value."""
    x = torch.randint(-2, 3, (m, k), generator=_gen(seed, 100)).to(torch.bfloat16)
    codes = torch.randint(0, 256, (n, k // 2), generator=_gen(seed, 101),
                          dtype=torch.uint8)
    e = torch.randint(-4, 1, (n, k // 16), generator=_gen(seed, 102)).to(torch.float32)
    scales = torch.exp2(e).to(torch.float8_e4m3fn).view(torch.uint8).contiguous()
    return x, NvWeight(codes, scales, 1.0)


@dataclass
class Fp8Weight:
    """Host (or device) tensors of one block-scaled FP8 matrix [n, k]."""
    codes: torch.Tensor   # uint8 [n, k] (E4M3 bit patterns)
    scales: torch.Tensor  # float32 [ceil(n/128), ceil(k/128)]

    @property
    def n(self) -> int:
        return int(self.codes.shape[0])

    @property
    def k(self) -> int:
        return int(self.codes.shape[1])

    def to(self, device) -> "Fp8Weight":
        return Fp8Weight(self.codes.to(device), self.scales.to(device))


def fp8_weight(n: int, k: int, seed: int, which: int) -> Fp8Weight:
    """Codes uniform over the non-NaN E4M3 bytes; block scales 2^U(-10, -6)."""
    r = torch.randint(0, 254, (n, k), generator=_gen(seed, _FP8 + 2 * which),
                      dtype=torch.int32)
    codes = (r + (r >= 0x7F).to(torch.int32)).to(torch.uint8)  # skip 0x7F; max 0xFE
    u = torch.rand(((n + 127) // 128, (k + 127) // 128),
                   generator=_gen(seed, _FP8 + 2 * which + 1), dtype=torch.float32)
    scales = torch.exp2(u * 4.0 - 10.0)
    return Fp8Weight(codes.contiguous(), scales.contiguous())


def fp8_ffn_weights(hidden: int, inter: int, seed: int = 0):
    return (fp8_weight(inter, hidden, seed, 0), fp8_weight(inter, hidden, seed, 1),
            fp8_weight(hidden, inter, seed, 2))


def fp8_workload(name: str, seed: int = 0, m: int | None = None):
    """(x bf16 [m, hidden], wg, wu, wd) with FP8 weights, on the CPU; the
    shapes and X of workload ``name``."""
    spec = WORKLOADS[name]
    rows = spec["m"] if m is None else m
    x = activations(rows, spec["hidden"], seed, spec["outliers"])
    return (x,) + fp8_ffn_weights(spec["hidden"], spec["inter"], seed)


@dataclass
class Q2Weight:
    """Host (or device) tensors of one packed-Q2 matrix [n, k]."""
    codes: torch.Tensor   # uint8 [n, k/4]
    scales: torch.Tensor  # uint16 [n, k/group] (fp16 bit patterns)
    group: int = Q2_GROUP

    @property
    def n(self) -> int:
        return int(self.codes.shape[0])

    @property
    def k(self) -> int:
        return int(self.codes.shape[1] * 4)

    def to(self, device) -> "Q2Weight":
        return Q2Weight(self.codes.to(device), self.scales.to(device), self.group)


def q2_weight(n: int, k: int, seed: int, which: int, group: int = Q2_GROUP) -> Q2Weight:
    assert k % group == 0
    codes = torch.randint(0, 256, (n, k // 4), generator=_gen(seed, _Q2 + 2 * which),
                          dtype=torch.uint8)
    u = torch.rand((n, k // group), generator=_gen(seed, _Q2 + 2 * which + 1),
                   dtype=torch.float32) * -4.0
    scales = torch.exp2(u).to(torch.float16).view(torch.int16).view(torch.uint16)
    return Q2Weight(codes, scales.contiguous(), group)


def q2_ffn_weights(hidden: int, inter: int, seed: int = 0, group: int = Q2_GROUP):
    return (q2_weight(inter, hidden, seed, 0, group), q2_weight(inter, hidden, seed, 1, group),
            q2_weight(hidden, inter, seed, 2, group))


def q2_workload(name: str, seed: int = 0, m: int | None = None):
    """(x bf16 [m, hidden], wg, wu, wd) with packed-Q2 weights, on the CPU;
    the shapes and X of workload ``name``."""
    spec = WORKLOADS[name]
    rows = spec["m"] if m is None else m
    x = activations(rows, spec["hidden"], seed, spec["outliers"])
    return (x,) + q2_ffn_weights(spec["hidden"], spec["inter"], seed)
