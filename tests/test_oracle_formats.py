"""Pins for the oracle's element formats and roundings (CPU only).

Each check compares the oracle with something other than itself: the
published format tables (``tests/golden``), torch's own float8_e4m3fn and
bfloat16 casts (library routines), exact rational arithmetic, and a
brute-force nearest-value search over the decoded value set.
"""

import math
import os
import random
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_table(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            a, b = line.split()
            rows.append((int(a, 16), float(b)))
    return rows


def _same(a, b):
    if math.isnan(a) or math.isnan(b):
        return math.isnan(a) and math.isnan(b)
    return a == b and math.copysign(1, a) == math.copysign(1, b)


# ---- decoders ------------------------------------------------------------------

def test_e2m1_table_matches_standard():
    table = _read_table("e2m1_values.txt")
    assert len(table) == 16
    for code, value in table:
        assert _same(oracle.e2m1_value(code), value), hex(code)


def test_e4m3_points_match_standard():
    for byte, value in _read_table("e4m3_points.txt"):
        assert _same(oracle.e4m3_value(byte), value), hex(byte)


def test_e4m3_all_bytes_match_torch_float8():
    lib_vals = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(
        torch.float8_e4m3fn).to(torch.float64).tolist()
    for b in range(256):
        assert _same(oracle.e4m3_value(b), lib_vals[b]), hex(b)


def test_bf16_decode_matches_torch():
    bits = np.arange(65536, dtype=np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    for b in range(0, 65536, 7):
        assert _same(oracle.bf16_value(b), ref[b]), hex(b)


# ---- bf16 rounding ----------------------------------------------------------------

def _bf16_nearest_exact(v: float) -> int:
    """Brute force: nearest bf16 by exact rational distance, ties to even."""
    if v == 0:
        return 0x8000 if math.copysign(1, v) < 0 else 0
    f = np.array([v], dtype=np.float32)  # a nearby float: neighbours bracket v
    base = int(f.view(np.uint32)[0] >> 16)
    cands = set()
    for d in range(-3, 4):
        c = base + d
        if 0 <= c < 65536:
            cands.add(c)
    best = None
    target = Fraction(v)
    for c in cands:
        val = float(torch.tensor([c], dtype=torch.int32).to(torch.int16).view(torch.bfloat16).item()) \
            if c < 32768 else float(torch.tensor([c - 65536], dtype=torch.int16).view(torch.bfloat16).item())
        if math.isinf(val) or math.isnan(val):
            continue
        dist = abs(Fraction(val) - target)
        key = (dist, c & 1)
        if best is None or key < best[0]:
            best = (key, c)
    return best[1]


def test_bf16_rounding_single_rounding_of_doubles():
    rng = random.Random(1)
    vals = []
    for _ in range(400):
        e = rng.randint(-40, 40)
        vals.append(rng.uniform(-1, 1) * 2.0 ** e)
    # exact halfway points between adjacent bf16 values, and just off them
    for _ in range(200):
        b = rng.randint(0x0080, 0x7F00)
        lo = float(torch.tensor([b], dtype=torch.int16).view(torch.bfloat16).item())
        hi = float(torch.tensor([b + 1], dtype=torch.int16).view(torch.bfloat16).item())
        mid = (lo + hi) / 2
        vals += [mid, -mid, math.nextafter(mid, 0), math.nextafter(mid, math.inf)]
    for v in vals:
        assert oracle.bf16_from_double(v) == _bf16_nearest_exact(v), v


def test_bf16_rounding_matches_torch_on_floats():
    # for values exactly representable in fp32, torch's fp32->bf16 cast is a
    # single round-to-nearest-even
    rng = np.random.default_rng(2)
    raw = rng.integers(0, 2**32, size=200000, dtype=np.uint64).astype(np.uint32)
    f = raw.view(np.float32)
    f = f[np.isfinite(f)]
    ref = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oracle.bf16_from_double_array(f.astype(np.float64))
    assert np.array_equal(got, ref)


# ---- E4M3 / E2M1 encoders ----------------------------------------------------------

def _brute_encode(t: np.ndarray, codes: np.ndarray, values: np.ndarray, max_code_mag: int,
                  sign_bit: int) -> np.ndarray:
    """Nearest value by exhaustive search, ties to the even code, saturate."""
    pos = [(int(c), float(v)) for c, v in zip(codes, values) if v >= 0 and not math.isnan(v)
           and int(c) < sign_bit]
    pos_codes = np.array([c for c, _ in pos], dtype=np.int64)
    pos_vals = np.array([v for _, v in pos], dtype=np.float64)
    a = np.abs(t.astype(np.float64))
    dist = np.abs(a[:, None] - pos_vals[None, :])
    best = dist.min(axis=1, keepdims=True)
    tied = dist == best
    # among the nearest, prefer the even code
    even = (pos_codes[None, :] & 1) == 0
    pick = np.where(tied & even, 1, 0) * 2 + np.where(tied, 1, 0)
    idx = pick.argmax(axis=1)
    out = pos_codes[idx]
    out = np.where(a >= pos_vals.max(), max_code_mag, out)
    neg = np.signbit(t)
    return (out | np.where(neg, sign_bit, 0)).astype(np.uint8)


def _sweep_points(values: np.ndarray, scale_lo: float, scale_hi: float, n_rand: int, seed: int):
    """Grid points, midpoints, their fp32 neighbours, and random log-uniform values."""
    v = np.unique(np.abs(values[np.isfinite(values)]))
    mids = (v[1:] + v[:-1]) / 2
    pts = np.concatenate([v, mids, [v.max() * 1.03, v.max() * 1.07, v.max() * 4, 1e30]])
    pts = pts.astype(np.float32)
    near = [pts]
    up, down = pts, pts
    for _ in range(3):  # three fp32 ulps either side
        up = np.nextafter(up, np.float32(np.inf))
        down = np.nextafter(down, np.float32(0))
        near += [up, down]
    rng = np.random.default_rng(seed)
    rnd = (2.0 ** rng.uniform(np.log2(scale_lo), np.log2(scale_hi), n_rand)).astype(np.float32)
    allp = np.concatenate(near + [rnd])
    return np.concatenate([allp, -allp, np.array([0.0, -0.0], dtype=np.float32)])


def test_e4m3_encode_brute_force():
    codes = np.arange(128, dtype=np.int64)
    values = np.array([oracle.e4m3_value(int(c)) for c in codes])
    t = _sweep_points(values, 2.0 ** -12, 600.0, 200000, seed=3)
    got = oracle.e4m3_encode_array(t)
    ref = _brute_encode(t, codes[:127], values[:127], 0x7E, 0x80)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, [(float(t[i]), hex(got[i]), hex(ref[i])) for i in bad[:10]]


def test_e4m3_encode_matches_torch_cast_in_range():
    rng = np.random.default_rng(4)
    t = (2.0 ** rng.uniform(-12, np.log2(447.0), 300000)).astype(np.float32)
    t *= np.where(rng.random(t.size) < 0.5, -1, 1).astype(np.float32)
    ref = torch.from_numpy(t).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(oracle.e4m3_encode_array(t), ref)


def test_e4m3_encode_saturates_and_keeps_nan():
    assert oracle.e4m3_encode(1e9) == 0x7E
    assert oracle.e4m3_encode(-1e9) == 0xFE
    assert oracle.e4m3_encode(float("inf")) == 0x7E
    assert oracle.e4m3_encode(464.0) == 0x7E
    assert oracle.e4m3_encode(2.0 ** -10) == 0x00        # tie with 2^-9 -> even 0
    assert oracle.e4m3_encode(3 * 2.0 ** -10) == 0x02    # tie 1 vs 2 (x2^-9) -> 2


def test_e2m1_encode_brute_force():
    codes = np.arange(8, dtype=np.int64)
    values = np.array([oracle.e2m1_value(int(c)) for c in codes])
    t = _sweep_points(values, 2.0 ** -6, 50.0, 200000, seed=5)
    got = oracle.e2m1_encode_array(t)
    ref = _brute_encode(t, codes, values, 7, 8)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, [(float(t[i]), hex(got[i]), hex(ref[i])) for i in bad[:10]]


@pytest.mark.parametrize("t,code", [
    (0.25, 0x0), (0.75, 0x2), (1.25, 0x2), (1.75, 0x4), (2.5, 0x4),
    (3.5, 0x6), (5.0, 0x6), (6.0, 0x7), (100.0, 0x7), (-0.0, 0x8), (-0.2, 0x8),
    (-5.5, 0xF), (0.2500001, 0x1),
])
def test_e2m1_ties_and_saturation(t, code):
    assert oracle.e2m1_encode(t) == code


# ---- silu ---------------------------------------------------------------------------

def test_silu_identity_and_limits():
    rng = random.Random(6)
    for _ in range(2000):
        t = rng.uniform(-30, 30)
        assert math.isclose(oracle.silu(t) - oracle.silu(-t), t, rel_tol=1e-14, abs_tol=1e-14)
    assert oracle.silu(0.0) == 0.0
    assert oracle.silu(800.0) == 800.0
    s = oracle.silu(-800.0)
    assert s == 0.0 and math.copysign(1, s) < 0


def test_silu_matches_torch():
    t = torch.linspace(-40, 40, 10001, dtype=torch.float64)
    ref = torch.nn.functional.silu(t)
    got = torch.tensor([oracle.silu(float(v)) for v in t], dtype=torch.float64)
    assert torch.allclose(got, ref, rtol=1e-14, atol=1e-300)


def test_silu_mul_rounds_once():
    rng = np.random.default_rng(7)
    g = torch.from_numpy(rng.normal(0, 4, 5000).astype(np.float32)).to(torch.bfloat16)
    u = torch.from_numpy(rng.normal(0, 4, 5000).astype(np.float32)).to(torch.bfloat16)
    gb = g.view(torch.int16).numpy().view(np.uint16)
    ub = u.view(torch.int16).numpy().view(np.uint16)
    out = oracle.silu_mul(gb, ub)
    exact = torch.nn.functional.silu(g.double()) * u.double()
    for i in range(0, 5000, 5):
        assert out[i] == _bf16_nearest_exact(float(exact[i])) or \
            abs(float(exact[i])) < 1e-30, i
