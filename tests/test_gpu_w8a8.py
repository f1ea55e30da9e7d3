"""GPU parity of the W8A8 fixed format (block-scaled FP8 weights, per-row
FP8 activations) against the oracle, through the C-ABI.

* The per-row FP8 quantizer is bit-exact (codes and row scales).
* Projections and the FFN match the oracle's fp64 value ref element by
  element within |err_i| <= 2e-2 * rms(ref) + 2^-8 * |ref_i|, on shapes that
  span several tiles, ragged columns and K, split K, both column-tile
  widths, and the full workload (sampled rows).  The second term is one
  bf16 ulp of the element: the block-scaled FP8 weights here (codes uniform
  over every E4M3 byte, up to 448) with outlier activations give outputs
  beyond 10 * rms, whose bf16 rounding alone (up to 2^-9 * |ref_i|) exceeds
  2e-2 * rms.  Where the outputs are not that heavy-tailed (the full
  workload), the plain 2e-2 * rms bound is asserted as well.
* Batch invariance is bit-exact, GPU against GPU: rows 0..m-1 at m in
  {1, 8, 64} equal the m = 512 run, and a permutation of the rows permutes
  the output rows.
"""

import numpy as np
import pytest
import torch

import nvfp4_weight_dense_amd as nv
import oracle
import synthetic_inputs as si
from gpu_helpers import assert_close, assert_close_elem, bits, sync

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


def g8(w: si.Fp8Weight) -> nv.FP8Weight:
    return nv.FP8Weight(w.codes.cuda().contiguous(), w.scales.cuda().contiguous())


def o8(w: si.Fp8Weight) -> oracle.Fp8Weight:
    return oracle.Fp8Weight(w.codes.numpy(), w.scales.numpy())


def _rows_with_edge_cases(m, k, seed):
    x = si.activations(m, k, seed=seed, outliers=True)
    if m >= 3:
        x[1, :] = 0.0                      # all-zero row: s_row = 1
        x[2, ::2] = -0.0                   # signed zeros
    return x


@pytest.mark.parametrize("m,k", [(1, 32), (3, 96), (7, 4096), (5, 14336), (2, 17408 * 2), (64, 4096), (100, 14336)])
def test_fp8_quantizer_bit_exact(m, k):
    _say(f"fp8 quantize m={m} k={k}")
    x = _rows_with_edge_cases(m, k, seed=m + k)
    c, r = nv.fp8_quantize_rows(x.cuda())
    sync()
    co, ro = oracle.quantize_rows_fp8(bits(x))
    assert np.array_equal(c.cpu().numpy(), co)
    assert np.array_equal(r.cpu().numpy(), ro)


def test_fp8_quantizer_every_bf16_quotient():
    """Every finite bf16 value of magnitude <= 7 (both signs), in rows that
    each hold 7.0: s_row = 7/448 = 2^-6 exactly, so the quotient is 64 x and
    every E4M3 rounding decision a bf16 input can reach (ties at every
    midpoint, the subnormal grid, saturation at 448) is taken on the GPU and
    compared with the oracle bit for bit."""
    _say("fp8 quantize every bf16 value")
    allb = torch.arange(0, 1 << 16, dtype=torch.int32).to(torch.int16).view(torch.bfloat16)
    v = allb[torch.isfinite(allb) & (allb.abs() <= 7.0)]
    k = 4096
    rows = -(-v.numel() // (k - 1))
    x = torch.zeros(rows * (k - 1), dtype=torch.bfloat16)
    x[: v.numel()] = v
    x = torch.cat([x.view(rows, k - 1), torch.full((rows, 1), 7.0, dtype=torch.bfloat16)], dim=1)
    x = x.contiguous()
    c, r = nv.fp8_quantize_rows(x.cuda())
    sync()
    co, ro = oracle.quantize_rows_fp8(bits(x))
    assert np.all(ro == np.float32(2.0 ** -6))
    assert np.array_equal(r.cpu().numpy(), ro)
    assert np.array_equal(c.cpu().numpy(), co)


def test_fp8_quantizer_every_bf16_below_inexact_row_max():
    """E4M3 rounding decisions under an inexact row scale: each row's maximum
    has a random mantissa, so s_row = amax/448 is an inexact fp32, and the
    rest of the row walks every bf16 value in [amax 2^-20, amax) with random
    signs -- quotients across the whole E4M3 range, subnormals included, on
    both sides of every midpoint, for 64 row scales.  Bit for bit against
    the oracle."""
    _say("fp8 quantize every bf16 below an inexact row max")
    rng = np.random.default_rng(12)
    rows, k = 64, 4096
    xb = np.zeros((rows, k), np.uint16)
    for r in range(rows):
        amax = (int(rng.integers(127 - 40, 127 + 40)) << 7) | int(rng.integers(1, 128))
        sweep = np.arange(amax - 20 * 128, amax, dtype=np.uint16)
        sweep |= (rng.integers(0, 2, sweep.size) << 15).astype(np.uint16)
        xb[r, 0] = amax
        xb[r, 1:1 + sweep.size] = sweep
    x = torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16)
    c, rs = nv.fp8_quantize_rows(x.cuda())
    sync()
    co, ro = oracle.quantize_rows_fp8(xb)
    assert np.array_equal(rs.cpu().numpy(), ro)
    assert np.array_equal(c.cpu().numpy(), co)


# (m, n, k): ragged columns and K; n = 64, k = 4096 splits K over 4
# workgroups; n >= 16384 takes two column tiles per workgroup, 16400 with a
# last 16-column tile and a partial scale block along N and K
@pytest.mark.parametrize("m,n,k", [(1, 48, 96), (5, 300, 384), (17, 130, 224), (70, 257, 640),
                                   (3, 64, 4096), (3, 16400, 160), (64, 1000, 2048),
                                   (9, 200, 320), (2, 40, 64)])
def test_fp8_gemm_w8a8_matches_oracle(m, n, k):
    _say(f"fp8 gemm m={m} n={n} k={k}")
    x = _rows_with_edge_cases(m, k, seed=n)
    w = si.fp8_weight(n, k, seed=m, which=0)
    y = nv.fp8_gemm_w8a8(x.cuda(), g8(w))
    sync()
    _, ye = oracle.gemm_w8a8(bits(x), o8(w))
    assert_close_elem(bits(y), ye, f"gemm w8a8 m={m} n={n} k={k}")


@pytest.mark.parametrize("m,n,k", [(3, 14336, 4096), (65, 4096, 14336)])
def test_fp8_gemm_w8a8_exact_case_bit_exact(m, n, k):
    """Exact case at full projection shapes: every row holds 7 (amax), the
    rest integers in [-2, 2], so s_row = 2^-6 and every code is exact; the
    weights are E4M3 integers in [-2, 2] with block scales 1, 2 or 4.  Every
    product and every fp32 partial sum is then an integer below 2^24, so any
    summation order gives the oracle's value and the bf16 results must match
    bit for bit (a wrong block-scale index or K order cannot hide here)."""
    _say(f"fp8 gemm exact m={m} n={n} k={k}")
    g = torch.Generator().manual_seed(n + k)
    x = torch.randint(-2, 3, (m, k), generator=g).to(torch.float32)
    x[:, 0] = 7.0
    x = x.to(torch.bfloat16)
    vals = torch.tensor([0xC0, 0xB8, 0x00, 0x38, 0x40], dtype=torch.uint8)  # -2 -1 0 1 2
    codes = vals[torch.randint(0, 5, (n, k), generator=g)].contiguous()
    e = torch.randint(0, 3, ((n + 127) // 128, (k + 127) // 128), generator=g).to(torch.float32)
    w = si.Fp8Weight(codes, torch.exp2(e).contiguous())
    y = nv.fp8_gemm_w8a8(x.cuda(), g8(w))
    sync()
    yo, _ = oracle.gemm_w8a8(bits(x), o8(w))
    assert np.array_equal(bits(y), yo)


@pytest.mark.parametrize("m", [1, 4, 17, 65, 130])
def test_dense_ffn_w8a8_tiny_matches_oracle(m):
    _say(f"ffn w8a8 tiny m={m}")
    x, wg, wu, wd = si.fp8_workload("tiny", m=m)
    y = nv.dense_ffn_forward_w8a8(x.cuda(), g8(wg), g8(wu), g8(wd))
    sync()
    _, ye = oracle.dense_ffn_w8a8(bits(x), o8(wg), o8(wu), o8(wd))
    assert_close_elem(bits(y), ye, f"ffn w8a8 tiny m={m}")


def _rows(m, count, seed):
    if m <= count:
        return np.arange(m)
    rng = np.random.default_rng(seed)
    picked = set(rng.choice(m, count - 2, replace=False).tolist()) | {0, m - 1}
    return np.array(sorted(picked))


def _block_rows(m, block=64):
    """The first and last row of every `block`-row block."""
    return np.array(sorted({r for b in range(0, m, block) for r in (b, min(m, b + block) - 1)}))


@pytest.mark.parametrize("m,nrows", [(1, 1), (64, 3), (512, None)])
def test_dense_ffn_w8a8_full_workload_matches_oracle(m, nrows):
    _say(f"ffn w8a8 full m={m}")
    x, wg, wu, wd = si.fp8_workload("w8a8", m=m)
    y = nv.dense_ffn_forward_w8a8(x.cuda(), g8(wg), g8(wu), g8(wd))
    sync()
    # m = 512: one row at each end of every 64-row block
    rows = _block_rows(m) if nrows is None else _rows(m, nrows, seed=3)
    _, ye = oracle.dense_ffn_w8a8(bits(x)[rows], o8(wg), o8(wu), o8(wd))
    assert_close_elem(bits(y)[rows], ye, f"ffn w8a8 m={m}")
    assert_close(bits(y)[rows], ye, f"ffn w8a8 m={m}")


def test_dense_ffn_w8a8_batch_invariance():
    _say("ffn w8a8 invariance")
    x, wg, wu, wd = si.fp8_workload("w8a8")  # m = 512
    xd = x.cuda()
    W = [g8(w) for w in (wg, wu, wd)]
    ref = nv.dense_ffn_forward_w8a8(xd, *W)
    for m in si.W8A8_ROW_COUNTS[:-1]:
        y = nv.dense_ffn_forward_w8a8(xd[:m].contiguous(), *W)
        sync()
        assert torch.equal(y.view(torch.int16), ref[:m].view(torch.int16)), f"m={m}"
    perm = torch.randperm(512, generator=torch.Generator().manual_seed(0)).cuda()
    y = nv.dense_ffn_forward_w8a8(xd[perm].contiguous(), *W)
    sync()
    assert torch.equal(y.view(torch.int16), ref[perm].view(torch.int16))


def _by_row_blocks(fn, x, block=16):
    return torch.cat([fn(x[r:r + block].contiguous()) for r in range(0, x.shape[0], block)])


# The many-row kernel (from 65 rows) against the few-row kernel, row for row
# and bit for bit: K split over workgroups (n = 64, k = 4096; the down
# projection's 4096 x 14336), splits of two and three steps (idle classes),
# ragged rows, columns and K, a partial scale block along N and K.
@pytest.mark.parametrize("m,n,k", [(65, 64, 4096), (200, 300, 160), (130, 1000, 352), (257, 16400, 512),
                                   (129, 4096, 14336)])
def test_fp8_gemm_w8a8_many_rows_equal_few_rows(m, n, k):
    _say(f"fp8 gemm many rows vs 16-row blocks m={m} n={n} k={k}")
    x = _rows_with_edge_cases(m, k, seed=n + k).cuda()
    w = g8(si.fp8_weight(n, k, seed=m, which=1))
    y = nv.fp8_gemm_w8a8(x, w)
    ref = _by_row_blocks(lambda xb: nv.fp8_gemm_w8a8(xb, w), x)
    sync()
    assert torch.equal(y.view(torch.int16), ref.view(torch.int16))


@pytest.mark.parametrize("m", [65, 200])
def test_dense_ffn_w8a8_many_rows_equal_few_rows(m):
    _say(f"ffn w8a8 many rows vs 16-row blocks m={m}")
    x, wg, wu, wd = si.fp8_workload("tiny", m=m)
    W = [g8(w) for w in (wg, wu, wd)]
    xd = x.cuda()
    y = nv.dense_ffn_forward_w8a8(xd, *W)
    ref = _by_row_blocks(lambda xb: nv.dense_ffn_forward_w8a8(xb, *W), xd)
    sync()
    assert torch.equal(y.view(torch.int16), ref.view(torch.int16))


def test_w8a8_m_zero_and_errors_touch_nothing():
    _say("w8a8 m=0 / errors")
    x, wg, wu, wd = si.fp8_workload("tiny", m=4)
    out = torch.full((4, 256), 7.0, dtype=torch.bfloat16, device="cuda")
    nv.dense_ffn_forward_w8a8(x[:0].cuda(), g8(wg), g8(wu), g8(wd), out=out[:0])
    with pytest.raises(ValueError):
        nv.dense_ffn_forward_w8a8(x.cuda(), g8(wg), g8(wu), g8(wg), out=out)  # wd's shape: refused by the binding
    sync()
    assert bool((out == 7.0).all())
