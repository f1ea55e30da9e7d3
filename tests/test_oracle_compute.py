"""Pins for the oracle's projections, quantizer and FFN (CPU only).

The projection is checked against a library matmul (numpy, float64) on
weights built value-first: the test picks each weight's value from the
published E2M1 table and torch's float8_e4m3fn values, derives the bytes
by inverse table lookup, and expects exactly x . W^T.  A nibble-order or
scale-index mistake, a transposed operand or a dropped tensor scale fails
these.  The quantizer is checked against a hand-derived golden row, against
brute-force nearest-value search on every element, and against properties
(power-of-two scaling, row independence).
"""

import math
import os

import numpy as np
import pytest
import torch

import oracle
import synthetic_inputs as si

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _e2m1_table():
    t = {}
    with open(os.path.join(GOLDEN, "e2m1_values.txt")) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                a, b = line.split()
                t[int(a, 16)] = float(b)
    return t


E2M1 = _e2m1_table()
E4M3_LIB = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(
    torch.float8_e4m3fn).to(torch.float64).numpy()


def _bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def _bf16_vals(bits: np.ndarray) -> np.ndarray:
    return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()


def _value_first_weight(rng, n, k, ts=1.0):
    """Random NVFP4 weight with its exact dense values computed from tables."""
    codes_nib = rng.integers(0, 16, size=(n, k))
    sc = rng.integers(0x18, 0x40, size=(n, k // 16)).astype(np.uint8)  # 2^-4 .. 1.875
    dense = np.vectorize(E2M1.get)(codes_nib) * np.repeat(E4M3_LIB[sc], 16, axis=1) * ts
    packed = (codes_nib[:, 0::2] | (codes_nib[:, 1::2] << 4)).astype(np.uint8)
    return oracle.Weight(packed, sc, ts), dense


@pytest.mark.parametrize("m,n,k,ts", [(1, 8, 32, 1.0), (3, 17, 64, 0.75), (5, 64, 96, 2.5)])
def test_gemm_w4a16_equals_library_matmul(m, n, k, ts):
    rng = np.random.default_rng(m * 100 + n)
    w, dense = _value_first_weight(rng, n, k, ts)
    x = torch.from_numpy(rng.normal(0, 1, (m, k)).astype(np.float32)).to(torch.bfloat16)
    xb = _bits(x)
    y, ye = oracle.gemm_w4a16(xb, w, nthreads=2)
    ref = _bf16_vals(xb) @ dense.T
    assert np.allclose(ye, ref, rtol=1e-12, atol=1e-12)
    assert np.array_equal(y, oracle.bf16_from_double_array(ye))
    assert np.array_equal(oracle.dequant(w), dense)


def test_gemm_single_weight_pins_nibble_order_and_scale_index():
    n, k = 4, 64
    x = torch.arange(1, k + 1, dtype=torch.float32).reshape(1, k).to(torch.bfloat16)
    for c, kk in [(0, 0), (1, 1), (2, 17), (3, 63)]:
        codes = np.zeros((n, k // 2), dtype=np.uint8)
        scales = np.full((n, k // 16), 0x38, dtype=np.uint8)   # 1.0
        nib = 0x5  # 3.0
        codes[c, kk // 2] = nib << 4 if kk % 2 else nib
        scales[c, kk // 16] = 0x30                          # 0.5 on that block only
        y, ye = oracle.gemm_w4a16(_bits(x), oracle.Weight(codes, scales, 2.0), nthreads=1)
        expect = np.zeros(n)
        expect[c] = (kk + 1) * 3.0 * 0.5 * 2.0
        assert np.array_equal(ye[0], expect), (c, kk, ye)


def test_gemm_zero_rows_and_bad_shapes():
    w = oracle.Weight(np.zeros((4, 16), np.uint8), np.zeros((4, 2), np.uint8))
    y, ye = oracle.gemm_w4a16(np.zeros((0, 32), np.uint16), w)
    assert y.shape == (0, 4)
    bad = oracle.Weight(np.zeros((4, 8), np.uint8), np.zeros((4, 1), np.uint8))  # k=16 ok
    oracle.gemm_w4a16(np.zeros((1, 16), np.uint16), bad)


def test_exact_case_is_exact_in_fp32():
    # the exact-arithmetic inputs: every partial sum is a multiple of 2^-5
    # below 2^19, so fp32 sums in any order equal the double result
    x, w = si.exact_case(3, 40, 512, seed=1)
    ow = oracle.Weight(w.codes.numpy(), w.scales.numpy(), 1.0)
    y, ye = oracle.gemm_w4a16(_bits(x), ow, nthreads=2)
    dense = oracle.dequant(ow)
    xs = _bf16_vals(_bits(x)).astype(np.float32)
    f32 = np.zeros(ye.shape, dtype=np.float32)
    for kk in range(512)[::-1]:  # a different order, in fp32
        f32 += xs[:, kk:kk + 1] * dense[:, kk].astype(np.float32)[None, :]
    assert np.array_equal(f32.astype(np.float64), ye)
    assert np.all(np.abs(ye * 32) < 2**24) and np.all(ye * 32 == np.round(ye * 32))


# ---- quantizer -------------------------------------------------------------------------

def _read_quant_golden():
    rows = []
    cur = None
    with open(os.path.join(GOLDEN, "quant_rows_example.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, *vals = line.split()
            if key == "row":
                cur = {"x": [], "codes": []}
                rows.append(cur)
            elif key == "row_scale":
                cur["row_scale"] = float(vals[0])
            elif key == "scales":
                cur["scales"] = [int(v, 16) for v in vals]
            elif key == "x":
                cur["x"] += [float(v) for v in vals]
            elif key == "codes":
                cur["codes"] += [int(v, 16) for v in vals]
    return rows


def _unpack(codes: np.ndarray) -> np.ndarray:
    out = np.empty(codes.shape[:-1] + (codes.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = codes & 15
    out[..., 1::2] = codes >> 4
    return out


def test_quantizer_hand_derived_rows():
    rows = _read_quant_golden()
    x = torch.tensor([r["x"] for r in rows], dtype=torch.float32).to(torch.bfloat16)
    assert torch.equal(x.float(), torch.tensor([r["x"] for r in rows]))  # exact inputs
    codes, scales, rs = oracle.quantize_rows(_bits(x))
    for i, r in enumerate(rows):
        assert rs[i] == np.float32(r["row_scale"])
        assert list(scales[i]) == r["scales"]
        assert list(_unpack(codes[i])) == r["codes"], i


def _brute_codes(q: np.ndarray) -> np.ndarray:
    vals = np.array([E2M1[c] for c in range(8)])
    a = np.abs(q.astype(np.float64))
    d = np.abs(a[..., None] - vals)
    best = d.min(axis=-1, keepdims=True)
    tied = d == best
    even = (np.arange(8) & 1) == 0
    idx = (tied * (1 + even)).argmax(axis=-1)
    idx = np.where(a >= 6, 7, idx)
    return (idx | np.where(np.signbit(q), 8, 0)).astype(np.uint8)


def test_quantizer_codes_are_nearest_of_fp32_quotient():
    rng = np.random.default_rng(11)
    x = rng.normal(0, 1, (16, 256)) * np.exp(rng.normal(0, 2, (16, 1)))
    x[3, :40] = 0.0
    x[4, 7] = -0.0
    x[5, 100:] *= 1e-3  # small blocks next to large ones
    xb = _bits(torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16))
    xv = _bf16_vals(xb).astype(np.float32)
    codes, scales, rs = oracle.quantize_rows(xb)
    nib = _unpack(codes)
    v = E4M3_LIB[scales].astype(np.float32)                      # [m, k/16]
    den = (np.repeat(v, 16, axis=1) * rs[:, None]).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        q = (xv / den).astype(np.float32)                       # IEEE fp32 division
    expect = _brute_codes(q)
    zero = (xv == 0) | (np.repeat(v, 16, axis=1) == 0)
    expect = np.where(zero, np.where(np.signbit(xv), 8, 0), expect)
    assert np.array_equal(nib, expect)
    # scale bytes: E4M3 of amax_b / (6 s_row), all finite and <= 448
    amax_b = np.abs(xv).reshape(16, -1, 16).max(axis=2)
    t = (amax_b / (np.float32(6.0) * rs[:, None]).astype(np.float32)).astype(np.float32)
    lib = torch.from_numpy(np.minimum(t, 448).astype(np.float32)).to(
        torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(scales, lib)
    assert np.all(E4M3_LIB[scales] <= 448)
    # the block holding the row amax gets 448 or the next value down
    for r in range(16):
        b = int(np.abs(xv[r]).argmax() // 16)
        assert scales[r, b] in (0x7E, 0x7D)
        assert rs[r] == np.float32(np.abs(xv[r]).max()) / np.float32(2688.0)


def test_quantizer_power_of_two_scaling_and_row_independence():
    rng = np.random.default_rng(12)
    x = torch.from_numpy(rng.normal(0, 1, (6, 128)).astype(np.float32)).to(torch.bfloat16)
    c1, s1, r1 = oracle.quantize_rows(_bits(x))
    c2, s2, r2 = oracle.quantize_rows(_bits((x.float() * 8).to(torch.bfloat16)))
    assert np.array_equal(c1, c2) and np.array_equal(s1, s2)
    assert np.array_equal(r2, r1 * 8)
    # row 2 alone gives the same bits as row 2 among others
    c3, s3, r3 = oracle.quantize_rows(_bits(x[2:3]))
    assert np.array_equal(c3[0], c1[2]) and np.array_equal(s3[0], s1[2]) and r3[0] == r1[2]


def test_w4a4_gemm_is_projection_of_dequantized_rows():
    rng = np.random.default_rng(13)
    w, dense = _value_first_weight(rng, 24, 128, 1.5)
    x = torch.from_numpy(rng.normal(0, 3, (5, 128)).astype(np.float32)).to(torch.bfloat16)
    codes, scales, rs = oracle.quantize_rows(_bits(x))
    xhat = np.vectorize(E2M1.get)(_unpack(codes)) * np.repeat(E4M3_LIB[scales], 16, axis=1) \
        * rs[:, None].astype(np.float64)
    y, ye = oracle.gemm_w4a4(_bits(x), w, nthreads=2)
    assert np.allclose(ye, xhat @ dense.T, rtol=1e-12, atol=1e-12)
    assert np.array_equal(y, oracle.bf16_from_double_array(ye))
    # quantization error stays within NVFP4's resolution
    ref = _bf16_vals(_bits(x)) @ dense.T
    assert np.sqrt(np.mean((ye - ref) ** 2)) < 0.2 * np.sqrt(np.mean(ref ** 2))


# ---- dense FFN ------------------------------------------------------------------------------

def _ffn_case(rng, m, hidden, inter):
    wg, dg = _value_first_weight(rng, inter, hidden, 0.5)
    wu, du = _value_first_weight(rng, inter, hidden, 1.0)
    wd, dd = _value_first_weight(rng, hidden, inter, 0.25)
    x = torch.from_numpy(rng.normal(0, 1, (m, hidden)).astype(np.float32)).to(torch.bfloat16)
    return x, (wg, wu, wd), (dg, du, dd)


def test_dense_ffn_matches_library_pipeline():
    rng = np.random.default_rng(14)
    x, (wg, wu, wd), (dg, du, dd) = _ffn_case(rng, 3, 64, 96)
    y, ye, g, u, a = oracle.dense_ffn(_bits(x), wg, wu, wd, nthreads=2, intermediates=True)
    xv = _bf16_vals(_bits(x))
    g_ref = torch.from_numpy(xv @ dg.T)
    u_ref = torch.from_numpy(xv @ du.T)
    # bf16 of the exact double sums (fp32 staging can double-round: allow 1 ulp)
    def close_bits(bits, ref):
        got = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double()
        return torch.all((got - ref).abs() <= ref.abs() * 2.0 ** -8 + 1e-30)
    assert close_bits(g, g_ref) and close_bits(u, u_ref)
    a_ref = torch.nn.functional.silu(torch.from_numpy(_bf16_vals(g))) * torch.from_numpy(_bf16_vals(u))
    assert close_bits(a, a_ref)
    y_ref = _bf16_vals(a) @ dd.T
    assert np.allclose(ye, y_ref, rtol=1e-12, atol=1e-12)


def test_dense_ffn_is_composition_of_steps():
    x, wg, wu, wd = si.workload("tiny")
    to_o = lambda w: oracle.Weight(w.codes.numpy(), w.scales.numpy(), w.ts)
    xb = _bits(x)
    y, ye, g, u, a = oracle.dense_ffn(xb, to_o(wg), to_o(wu), to_o(wd), intermediates=True)
    g2, _ = oracle.gemm_w4a16(xb, to_o(wg))
    u2, _ = oracle.gemm_w4a16(xb, to_o(wu))
    a2 = oracle.silu_mul(g2, u2)
    y2, ye2 = oracle.gemm_w4a16(a2, to_o(wd))
    assert np.array_equal(g, g2) and np.array_equal(u, u2) and np.array_equal(a, a2)
    assert np.array_equal(y, y2) and np.array_equal(ye, ye2)
    # W4A4 arm: the same pipeline with quantized activations at both projections
    y4, ye4, g4, u4, a4 = oracle.dense_ffn(xb, to_o(wg), to_o(wu), to_o(wd), w4a4=True,
                                           intermediates=True)
    g5, _ = oracle.gemm_w4a4(xb, to_o(wg))
    a5 = oracle.silu_mul(g5, oracle.gemm_w4a4(xb, to_o(wu))[0])
    assert np.array_equal(g4, g5) and np.array_equal(a4, a5)
    assert np.array_equal(y4, oracle.gemm_w4a4(a5, to_o(wd))[0])
    # the two arms agree to within NVFP4 activation error
    rel = np.sqrt(np.mean((ye4 - ye) ** 2) / np.mean(ye ** 2))
    assert rel < 0.25


def test_dense_ffn_rows_are_independent():
    x, wg, wu, wd = si.workload("tiny")
    to_o = lambda w: oracle.Weight(w.codes.numpy(), w.scales.numpy(), w.ts)
    for w4a4 in (False, True):
        y_all, _ = oracle.dense_ffn(_bits(x), to_o(wg), to_o(wu), to_o(wd), w4a4=w4a4)
        y_one, _ = oracle.dense_ffn(_bits(x[2:3]), to_o(wg), to_o(wu), to_o(wd), w4a4=w4a4)
        assert np.array_equal(y_all[2], y_one[0])
