"""Pins for the oracle's packed-Q2 FFN (CPU only).

* Dequantization against a hand-derived golden example (bit order, group
  index, bf16 ties), and against numpy's float16 decode with torch's bf16
  rounding on random weights.
* A single nonzero code pins the code order and the group index in the
  projection.
* The projection against a library matmul of the dequantized weight, and
  the FFN against its composition from the pinned parts.
"""

import os

import numpy as np
import pytest
import torch

import oracle
import synthetic_inputs as si

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def _oq(w: si.Q2Weight) -> oracle.Q2Weight:
    return oracle.Q2Weight(w.codes.numpy(), w.scales.view(torch.int16).numpy().view(np.uint16),
                           w.group)


def _lib_dequant(w: oracle.Q2Weight) -> np.ndarray:
    """numpy float16 decode of the scales, numpy bit unpacking of the codes,
    torch's bf16 rounding of the float32 product (exact: a small integer
    times an fp16 value)."""
    shifts = np.array([0, 2, 4, 6], dtype=np.uint8)
    q = ((w.codes[:, :, None] >> shifts[None, None, :]) & 3).reshape(w.n, w.k).astype(np.float32)
    d = np.repeat(w.scales.view(np.float16).astype(np.float32), w.group, axis=1)
    v = torch.from_numpy((q - 2.0) * d).to(torch.bfloat16)
    return v.double().numpy()


def _golden():
    g = {}
    with open(os.path.join(GOLDEN, "q2_dequant_example.txt")) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                key, *vals = line.split()
                g[key] = vals
    return g


def test_q2_dequant_golden_example():
    g = _golden()
    w = oracle.Q2Weight(np.array([[int(v, 16) for v in g["codes"]]], dtype=np.uint8),
                        np.array([[int(v, 16) for v in g["scales"]]], dtype=np.uint16),
                        int(g["group"][0]))
    got = oracle.dequant_q2(w)[0]
    assert got.tolist() == [float(v) for v in g["values"]]
    assert oracle.fp16_value(0x3C04) == 1.00390625


def test_fp16_decoder_matches_numpy():
    h = np.arange(1 << 16, dtype=np.uint16)
    ref = h.view(np.float16).astype(np.float64)
    got = np.array([oracle.fp16_value(int(b)) for b in h[::97]])
    r = ref[::97]
    fin = np.isfinite(r)
    assert np.array_equal(got[fin], r[fin])
    assert np.all(np.isnan(got[np.isnan(r)]))


@pytest.mark.parametrize("group", [32, 128])
def test_q2_dequant_matches_library_decode(group):
    w = _oq(si.q2_weight(40, 512, seed=group, which=0, group=group))
    assert np.array_equal(oracle.dequant_q2(w), _lib_dequant(w))


def test_single_code_pins_order_and_group_index():
    n, k, group = 4, 256, 32
    x = torch.arange(1, k + 1, dtype=torch.float32).reshape(1, k).to(torch.bfloat16)
    xb = _bits(x)
    for c, kk in [(0, 0), (1, 1), (2, 37), (3, 255)]:
        codes = np.full((n, k // 4), 0xAA, dtype=np.uint8)       # every code 2: value 0
        sh = 2 * (kk % 4)
        codes[c, kk // 4] = (int(codes[c, kk // 4]) & (0xFF ^ (3 << sh))) | (3 << sh)  # q=3: 1*d
        scales = np.full((n, k // group), 0x3C00, dtype=np.uint16)  # 1.0
        scales[c, kk // group] = 0x4000                              # 2.0 on that group only
        _, ye = oracle.gemm_q2(xb, oracle.Q2Weight(codes, scales, group), nthreads=1)
        expect = np.zeros(n)
        expect[c] = (kk + 1) * 2.0
        assert np.array_equal(ye[0], expect), (c, kk)


@pytest.mark.parametrize("m,n,k,group", [(1, 8, 128, 128), (3, 33, 256, 64), (5, 64, 384, 128)])
def test_gemm_q2_equals_library_matmul(m, n, k, group):
    w = _oq(si.q2_weight(n, k, seed=m, which=1, group=group))
    x = si.activations(m, k, seed=n, outliers=True)
    xb = _bits(x)
    y, ye = oracle.gemm_q2(xb, w, nthreads=2)
    xv = x.double().numpy()
    W = _lib_dequant(w)
    ref = xv @ W.T
    mag = np.abs(xv) @ np.abs(W).T
    assert np.all(np.abs(ye - ref) <= 1e-12 * mag)
    assert np.array_equal(y, oracle.bf16_from_double_array(ye))


def test_dense_ffn_q2_is_its_composition():
    x, wg, wu, wd = si.q2_workload("tiny")
    xb = _bits(x)
    G, U, D = _oq(wg), _oq(wu), _oq(wd)
    y, ye, g, u, a = oracle.dense_ffn_q2(xb, G, U, D, intermediates=True)
    assert np.array_equal(g, oracle.gemm_q2(xb, G)[0])
    assert np.array_equal(u, oracle.gemm_q2(xb, U)[0])
    assert np.array_equal(a, oracle.silu_mul(g, u))
    y2, ye2 = oracle.gemm_q2(a, D)
    assert np.array_equal(y, y2) and np.array_equal(ye, ye2)
    xv = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).double().numpy()
    assert np.allclose(ye, xv @ _lib_dequant(D).T, rtol=0, atol=1e-9 * np.abs(ye).max())


def test_q2_shape_errors():
    w = _oq(si.q2_weight(8, 256, seed=0, which=0))
    with pytest.raises(ValueError):
        oracle.dense_ffn_q2(np.zeros((1, 128), dtype=np.uint16), w, w, w)
