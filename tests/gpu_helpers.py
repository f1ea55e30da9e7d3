"""Shared helpers of the GPU parity tests: moving seeded inputs to the GPU,
bf16 bit views, oracle calls and the float tolerance.

Tolerance for floating-point outputs: max |gpu - ref| <= 2e-2 * rms(ref),
with ref the oracle's fp64 result before its final bf16 rounding (the
oracle's bf16 output is itself up to half an ulp from that value).
"""

from __future__ import annotations

import numpy as np
import torch

import nvfp4_weight_dense_amd as nv
import oracle
import synthetic_inputs as si

TOL = 2e-2


def bits(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor (any device) -> uint16 numpy bit patterns."""
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def from_bits(b: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).view(torch.bfloat16)


def bf16_f64(b: np.ndarray) -> np.ndarray:
    return from_bits(b).double().numpy()


def o_weight(w: si.NvWeight, cols=None) -> oracle.Weight:
    codes, scales = w.codes.cpu().numpy(), w.scales.cpu().numpy()
    if cols is not None:
        codes, scales = codes[cols], scales[cols]
    return oracle.Weight(codes, scales, w.ts)


def g_weight(w: si.NvWeight) -> nv.NVFP4Weight:
    return nv.NVFP4Weight(w.codes.cuda().contiguous(), w.scales.cuda().contiguous(), w.ts)


def rel_err(gpu_bits: np.ndarray, ref_exact: np.ndarray) -> float:
    g = bf16_f64(gpu_bits)
    rms = float(np.sqrt(np.mean(ref_exact.astype(np.float64) ** 2)))
    return float(np.max(np.abs(g - ref_exact))) / max(rms, 1e-300)


def assert_close(gpu_bits: np.ndarray, ref_exact: np.ndarray, what: str = ""):
    assert gpu_bits.shape == ref_exact.shape, (gpu_bits.shape, ref_exact.shape)
    assert np.all(np.isfinite(bf16_f64(gpu_bits))), what + ": non-finite output"
    e = rel_err(gpu_bits, ref_exact)
    assert e <= TOL, f"{what}: max|err|/rms = {e:.4g} > {TOL}"
    return e


def assert_close_elem(gpu_bits: np.ndarray, ref: np.ndarray, what: str = ""):
    """|gpu - ref| <= 2e-2 * rms(ref) + 2^-8 * |ref| element by element.

    The second term is one bf16 ulp of the element: rounding an output to
    bf16 moves it by up to 2^-9 * |ref_i|, so an output beyond about 10 *
    rms(ref) cannot meet the plain 2e-2 * rms(ref) bound in bf16 at all;
    one more ulp covers a double rounding at a tie after an fp32 sum."""
    assert gpu_bits.shape == ref.shape, (gpu_bits.shape, ref.shape)
    g = bf16_f64(gpu_bits)
    assert np.all(np.isfinite(g)), what + ": non-finite output"
    rms = float(np.sqrt(np.mean(ref.astype(np.float64) ** 2)))
    bound = TOL * rms + 2.0 ** -8 * np.abs(ref)
    worst = float(np.max(np.abs(g - ref) / np.maximum(bound, 1e-300)))
    assert worst <= 1.0, f"{what}: max |err| / bound = {worst:.4g}"
    return worst


def sync():
    torch.cuda.synchronize()
