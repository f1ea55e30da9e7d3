"""Pins for the oracle's W8A8 fixed format (CPU only): block-scaled FP8
weights, per-row FP8 activations, and the FFN built from them.

* The quantizer against a hand-derived golden example (ties, subnormals,
  saturation, signed zeros), against torch's own float8_e4m3fn cast of the
  fp32 quotient, against brute-force nearest-value search, and against
  properties (power-of-two scaling, row independence, the amax element
  lands on +-448).
* Weight decode against torch's float8 table and a block grid expanded by
  numpy; a single nonzero weight pins the scale grid's index order.
* The projection against a library matmul of those decoded operands.
* The FFN against its composition from the pinned parts.
"""

import os

import numpy as np
import pytest
import torch

import oracle
import synthetic_inputs as si

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
E4M3_LIB = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(
    torch.float8_e4m3fn).to(torch.float64).numpy()


def _bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def _bf16_vals(bits: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(
        torch.bfloat16).double().numpy()


def _ow(w: si.Fp8Weight) -> oracle.Fp8Weight:
    return oracle.Fp8Weight(w.codes.numpy(), w.scales.numpy())


def _dense(w: oracle.Fp8Weight) -> np.ndarray:
    """Weight values from torch's float8 table and the block grid."""
    grid = np.repeat(np.repeat(w.scales.astype(np.float64), 128, axis=0), 128, axis=1)
    return E4M3_LIB[w.codes] * grid[: w.n, : w.k]


def _xhat(xb: np.ndarray) -> np.ndarray:
    codes, rs = oracle.quantize_rows_fp8(xb)
    return E4M3_LIB[codes] * rs.astype(np.float64)[:, None]


def _golden_rows():
    rows, cur = [], None
    with open(os.path.join(GOLDEN, "fp8_quant_rows_example.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, *vals = line.split()
            if key == "row":
                cur = {}
                rows.append(cur)
            elif key == "row_scale":
                cur["rs"] = float(vals[0])
            elif key == "x":
                cur["x"] = [float(v) for v in vals]
            elif key == "codes":
                cur["codes"] = [int(v, 16) for v in vals]
    return rows


def test_fp8_quantizer_golden_example():
    rows = _golden_rows()
    x = torch.tensor([r["x"] for r in rows], dtype=torch.float32)
    xb = _bits(x.to(torch.bfloat16))
    assert np.array_equal(_bf16_vals(xb), x.double().numpy())  # inputs exact in bf16
    codes, rs = oracle.quantize_rows_fp8(xb)
    for i, r in enumerate(rows):
        assert rs[i] == np.float32(r["rs"]), i
        assert codes[i].tolist() == r["codes"], (i, [hex(c) for c in codes[i]])


def _random_rows(m, k, seed, outliers=True):
    x = si.activations(m, k, seed=seed, outliers=outliers)
    x[0, :] = 0.0
    x[1, ::3] = -0.0
    x[2] *= 1e-30  # subnormal quotients stay within range after the row scale
    return _bits(x)


def test_fp8_quantizer_matches_torch_cast_of_the_quotient():
    xb = _random_rows(16, 320, seed=3)
    codes, rs = oracle.quantize_rows_fp8(xb)
    xf = _bf16_vals(xb).astype(np.float32)
    amax = np.abs(xf).max(axis=1)
    s_row = np.where(amax == 0, np.float32(1.0), amax / np.float32(448.0)).astype(np.float32)
    assert np.array_equal(rs, s_row)
    q = (xf / s_row[:, None]).astype(np.float32)
    assert np.all(np.abs(q) <= np.float32(448.0) * np.float32(1 + 2 ** -22))
    lib = torch.from_numpy(q).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(codes, lib)


def test_fp8_quantizer_every_bf16_value_matches_torch_cast():
    """Every finite bf16 value with |x| <= 7 in one row holding 7.0: s_row is
    2^-6, the quotient 64 x is exact, and the codes must equal torch's own
    float8_e4m3fn cast of it (every midpoint tie, the subnormal grid, 448)."""
    allb = torch.arange(0, 1 << 16, dtype=torch.int32).to(torch.int16).view(torch.bfloat16)
    v = allb[torch.isfinite(allb) & (allb.abs() <= 7.0)]
    x = torch.cat([v, torch.tensor([7.0], dtype=torch.bfloat16)]).reshape(1, -1)
    pad = (-x.shape[1]) % 32
    x = torch.cat([x, torch.zeros((1, pad), dtype=torch.bfloat16)], dim=1)
    codes, rs = oracle.quantize_rows_fp8(_bits(x))
    assert rs[0] == np.float32(2.0 ** -6)
    q = x.float() * 64.0
    lib = q.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(codes, lib)


def test_fp8_quantizer_codes_are_nearest_grid_values():
    xb = _random_rows(6, 256, seed=4)
    codes, rs = oracle.quantize_rows_fp8(xb)
    q = (_bf16_vals(xb).astype(np.float32) / rs[:, None]).astype(np.float64)
    grid = np.array([E4M3_LIB[b] for b in range(256) if (b & 0x7F) != 0x7F])
    dec = E4M3_LIB[codes]
    best = np.abs(q[..., None] - grid[None, None, :]).min(axis=-1)
    assert np.all(np.abs(q - dec) == best)
    assert np.all(np.signbit(dec) == np.signbit(q))


def test_fp8_quantizer_properties():
    xb = _random_rows(8, 192, seed=5, outliers=False)
    codes, rs = oracle.quantize_rows_fp8(xb)
    xv = _bf16_vals(xb)
    for r in range(3, 8):  # nonzero rows: the amax element lands on +-448
        j = int(np.argmax(np.abs(xv[r])))
        assert codes[r, j] in (0x7E, 0xFE)
    # scaling a row by a power of two scales s_row and keeps every code
    for p in (-3, 5):
        c2, r2 = oracle.quantize_rows_fp8(_bits(torch.from_numpy(xv * 2.0 ** p).to(torch.bfloat16)))
        assert np.array_equal(c2[1:], codes[1:])
        assert np.array_equal(r2[1:], rs[1:] * np.float32(2.0 ** p))
    # a row's codes do not depend on the other rows
    for r in range(8):
        c1, r1 = oracle.quantize_rows_fp8(xb[r:r + 1])
        assert np.array_equal(c1[0], codes[r]) and r1[0] == rs[r]


def test_fp8_dequant_matches_torch_tables_and_block_grid():
    w = _ow(si.fp8_weight(200, 300, seed=1, which=0))  # ragged in both grid axes
    assert w.scales.shape == (2, 3)
    assert np.array_equal(oracle.dequant_fp8(w), _dense(w))


def test_single_weight_pins_scale_grid_index():
    n, k = 260, 392
    x = torch.arange(1, k + 1, dtype=torch.float32).reshape(1, k).to(torch.bfloat16)
    xb = _bits(x)
    xh = _xhat(xb)[0]
    scales = (np.arange(3 * 4, dtype=np.float32).reshape(3, 4) + 1.0) / 8.0
    for c, kk in [(0, 0), (127, 128), (128, 127), (259, 391), (200, 300)]:
        codes = np.zeros((n, k), dtype=np.uint8)
        codes[c, kk] = 0x44  # 3.0 = 1.5 * 2^1: e=8, t=4
        _, ye = oracle.gemm_w8a8(xb, oracle.Fp8Weight(codes, scales), nthreads=1)
        expect = np.zeros(n)
        expect[c] = xh[kk] * 3.0 * float(scales[c // 128, kk // 128])
        assert np.array_equal(ye[0], expect), (c, kk)


@pytest.mark.parametrize("m,n,k", [(1, 8, 128), (3, 130, 256), (5, 64, 96), (7, 257, 300)])
def test_gemm_w8a8_equals_library_matmul(m, n, k):
    w = _ow(si.fp8_weight(n, k, seed=m, which=1))
    xb = _random_rows(max(m, 3), k, seed=m + 10)[-m:]
    y, ye = oracle.gemm_w8a8(xb, w, nthreads=2)
    ref = _xhat(xb) @ _dense(w).T
    mag = np.abs(_xhat(xb)) @ np.abs(_dense(w)).T
    assert np.all(np.abs(ye - ref) <= 1e-12 * mag)
    assert np.array_equal(y, oracle.bf16_from_double_array(ye))


def test_dense_ffn_w8a8_is_its_composition():
    x, wg, wu, wd = si.fp8_workload("tiny")
    xb = _bits(x)
    WG, WU, WD = _ow(wg), _ow(wu), _ow(wd)
    y, ye, g, u, a = oracle.dense_ffn_w8a8(xb, WG, WU, WD, intermediates=True)
    xh = _xhat(xb)
    g_ref = oracle.bf16_from_double_array(xh @ _dense(WG).T)
    u_ref = oracle.bf16_from_double_array(xh @ _dense(WU).T)
    # sums in another order: equal up to a double rounding at a bf16 tie
    assert np.max(np.abs(g.astype(np.int32) - g_ref.astype(np.int32))) <= 1
    assert np.max(np.abs(u.astype(np.int32) - u_ref.astype(np.int32))) <= 1
    assert np.array_equal(a, oracle.silu_mul(g, u))
    ye_ref = _xhat(a) @ _dense(WD).T
    # double sums in another order differ by at most a few ulps of sum |terms|
    mag = np.abs(_xhat(a)) @ np.abs(_dense(WD)).T
    assert np.all(np.abs(ye - ye_ref) <= 1e-12 * mag)
    assert np.array_equal(y, oracle.bf16_from_double_array(ye))


def test_w8a8_zero_rows_and_shape_errors():
    w = _ow(si.fp8_weight(16, 128, seed=0, which=0))
    y, ye = oracle.gemm_w8a8(np.zeros((2, 128), dtype=np.uint16), w)
    assert not ye.any() and not y.any()
    with pytest.raises(ValueError):
        oracle.dense_ffn_w8a8(np.zeros((1, 64), dtype=np.uint16), w, w, w)
