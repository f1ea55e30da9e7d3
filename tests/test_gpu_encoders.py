"""The activation quantizers' division and rounding steps, run on arbitrary
fp32 values through nvfp4_probe_encode, against their definitions: the E2M1
and E4M3 codes against the oracle's encoders, the quotient x / d against
IEEE fp32 division (numpy's).  The quantizers divide with a rounded
reciprocal and one FMA correction and round with the hardware conversions;
these tests are what ties those steps to the definitions beyond the
quantizer tests' own inputs."""

import numpy as np
import pytest
import torch

import nvfp4_weight_dense_amd as nv
import oracle
from gpu_helpers import sync

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


def _probe(x: np.ndarray, d: float):
    pad = (-x.size) % 8
    xp = np.concatenate([x.astype(np.float32), np.zeros(pad, np.float32)])
    q, c4, c8 = nv.nvfp4_probe_encode(torch.from_numpy(xp).cuda(), d)
    sync()
    n = x.size
    return q.cpu().numpy()[:n], c4.cpu().numpy()[:n], c8.cpu().numpy()[:n]


def _grid_values():
    """Every sign, exponent and top-11-bit mantissa of fp32, each with eight
    low-12-bit patterns: 8M values spread over the whole format, NaNs
    dropped."""
    hi = np.arange(1 << 20, dtype=np.uint32) << np.uint32(12)
    lows = np.array([0, 1, 0x7FF, 0x800, 0x801, 0xFFF, 0x5A5, 0xA5A], dtype=np.uint32)
    f = (hi[:, None] | lows[None, :]).ravel().view(np.float32)
    return f[~np.isnan(f)]


def _around(points, ulps=64):
    """Every fp32 within `ulps` units in the last place of each point, both
    signs."""
    p = np.asarray(points, dtype=np.float32).view(np.int32)
    off = np.arange(-ulps, ulps + 1, dtype=np.int32)
    u = (p[:, None] + off[None, :]).ravel()
    f = u[u >= 0].view(np.float32)
    return np.concatenate([f, -f])


def _e4m3_magnitudes():
    b = np.arange(0, 0x7F)
    e, m = b >> 3, b & 7
    return np.where(e == 0, m * 2.0 ** -9, (1 + m / 8) * 2.0 ** (e - 7))


E2M1_DECISIONS = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0]


def _decision_points():
    mags = _e4m3_magnitudes()
    mids = (mags[1:] + mags[:-1]) / 2
    return np.concatenate([E2M1_DECISIONS, mids, [448.0, 464.0, 480.0]])


def test_encoders_match_the_oracle_over_fp32():
    _say("encoders over the fp32 grid and around every decision point")
    x = np.concatenate([_grid_values(), _around(_decision_points()),
                        np.array([0.0, -0.0, np.inf, -np.inf], np.float32)])
    _, c4, c8 = _probe(x, 1.0)
    want4 = oracle.e2m1_encode_array(x)
    want8 = oracle.e4m3_encode_array(x)
    bad4 = np.nonzero(c4 != want4)[0]
    bad8 = np.nonzero(c8 != want8)[0]
    assert bad4.size == 0, f"E2M1: {bad4.size} mismatches, first x={x[bad4[0]]!r}"
    assert bad8.size == 0, f"E4M3: {bad8.size} mismatches, first x={x[bad8[0]]!r}"


# divisors: the reciprocal path over [2^-90, 2^100] (row and block scales of
# any mantissa), and the plain division outside it
DIVISORS = [1.0, 3.0, 0.1, 7.1234567e-3, 1.7e-20, 2.9e-27, 6.5e21, 1.1e30, 2.0 ** -90, 2.0 ** 100,
            2.0 ** -100, 3.3e-38, 1.2e32]


@pytest.mark.parametrize("d", DIVISORS)
def test_quotient_is_ieee_division(d):
    _say(f"quotients d={d}")
    rng = np.random.default_rng(abs(hash(d)) % (1 << 32))
    d32 = np.float32(d)
    targets = np.concatenate([_decision_points(), rng.uniform(-8, 8, 2000)]).astype(np.float32)
    near = _around((np.abs(targets) * d32).astype(np.float32), ulps=16)
    raw = (rng.integers(0, 1 << 32, 1 << 18, dtype=np.uint64)).astype(np.uint32).view(np.float32)
    raw = raw[np.isfinite(raw)]
    x = np.concatenate([near, raw, np.array([0.0, -0.0], np.float32)])
    with np.errstate(over="ignore", under="ignore"):
        want = (x / d32).astype(np.float32)
    x, want = x[np.isfinite(want)], want[np.isfinite(want)]
    q, _, _ = _probe(x, float(d32))
    # bit for bit from 2^-10 up, where every rounding decision of either
    # encoder lies; below, the reciprocal path may differ in the last bits
    # (a subnormal x or residual) but must encode the same
    big = np.abs(want) >= np.float32(2.0 ** -10)
    bad = np.nonzero(big & (q.view(np.uint32) != want.view(np.uint32)))[0]
    assert bad.size == 0, f"{bad.size} quotients differ, first x={x[bad[0]]!r}"
    sub = ~big
    assert np.array_equal(oracle.e2m1_encode_array(q[sub]), oracle.e2m1_encode_array(want[sub]))
    assert np.array_equal(oracle.e4m3_encode_array(q[sub]), oracle.e4m3_encode_array(want[sub]))
