"""GPU parity of the individual C-ABI entry points against the oracle.

Float outputs: max |gpu - oracle_exact| <= 2e-2 * rms(oracle_exact).
Integer/byte outputs (quantizer codes, scales) and the exact-arithmetic
projection: bit for bit.
"""

import numpy as np
import pytest
import torch

import nvfp4_weight_dense_amd as nv
import oracle
import synthetic_inputs as si
from gpu_helpers import assert_close, bf16_f64, bits, from_bits, g_weight, o_weight, sync

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


# ---- dequantization of every code byte and every finite scale byte ---------------

def _all_bytes_weight():
    # 256 weight rows of k = 32: row c holds code bytes 16c..16c+15 (mod 256)
    # and scale bytes 2c, 2c+1; the two NaN scale bytes are replaced.
    n, k = 256, 32
    codes = (np.arange(n * 16).reshape(n, 16) % 256).astype(np.uint8)
    scales = (np.arange(n * 2).reshape(n, 2) % 256).astype(np.uint8)
    scales[scales == 0x7F] = 0x7E
    scales[scales == 0xFF] = 0xFE
    return si.NvWeight(torch.from_numpy(codes), torch.from_numpy(scales), 1.0)


@pytest.mark.parametrize("m", [32, 96])  # 32: streaming kernel, 96: many-row kernel
def test_dequant_every_code_and_scale_exact(m):
    _say(f"dequant identity m={m}")
    w = _all_bytes_weight()
    x = torch.zeros((m, 32), dtype=torch.bfloat16)
    x[:32, :32] = torch.eye(32)
    y = nv.nvfp4_gemm_w4a16(x.cuda(), g_weight(w))
    sync()
    dense = oracle.dequant(o_weight(w))                  # [256, 32] doubles
    expect = oracle.bf16_from_double_array(dense.T)      # exact in bf16
    # a -0 weight times 1 plus +0 products sums to +0
    expect = np.where(expect == 0x8000, 0, expect).astype(np.uint16)
    got = bits(y)
    assert np.array_equal(got[:32], expect)
    assert np.all(got[32:] & 0x7FFF == 0)


@pytest.mark.parametrize("m", [8, 32, 96])  # streaming kernel; two-stage kernel: 32 rows; many-row kernel: 96
def test_w4a4_dequant_every_code_and_scale(m):
    """The fp16 dequantization of the W4A4 path (both operands NVFP4): rows
    r < 32 of x are one-hot at K = r, so each output is one product a_r *
    w[c][r] times the row scale -- exact in fp32 up to the row-scale
    multiply -- and every code byte and finite scale byte of the weight
    meets a unit activation.  Element by element within 2^-8 of the
    oracle's value (the fp32 row-scale multiply and the bf16 rounding);
    a wrong code, scale or fragment slot is off by far more."""
    _say(f"w4a4 dequant identity m={m}")
    w = _all_bytes_weight()
    x = torch.zeros((m, 32), dtype=torch.bfloat16)
    r = min(m, 32)
    x[:r, :r] = torch.eye(r)
    y = nv.nvfp4_gemm_w4a4(x.cuda(), g_weight(w))
    sync()
    _, ye = oracle.gemm_w4a4(bits(x), o_weight(w))
    got = bf16_f64(bits(y))
    assert np.all(np.abs(got - ye) <= 2.0 ** -8 * np.abs(ye)), np.max(np.abs(got - ye))
    assert np.count_nonzero(ye[:r]) > 0.75 * ye[:r].size  # most products are nonzero


# ---- W4A16 projection --------------------------------------------------------------

SHAPES = [
    (1, 16, 32), (1, 50, 96), (2, 200, 160), (4, 64, 4096), (15, 33, 128), (16, 64, 256),
    (9, 70, 224), (6, 20, 96),
    (17, 80, 384), (33, 33, 512), (48, 100, 640), (64, 130, 1024),
    # 17..64 rows: k % 64 == 0 with a partial last weight group (LDS-DMA
    # ring), and k % 64 != 0 (LDS-shared activations)
    (40, 70, 2176), (20, 64, 160), (64, 48, 96),
    # 17..64 rows, stream-K plan: one column group split over 16 workgroups,
    # many groups with two pieces each, a ragged last group and K unit
    (48, 48, 4096), (33, 3000, 320), (17, 129, 2176), (64, 200, 64),
    (65, 130, 1024), (130, 300, 416), (257, 129, 96), (200, 64, 2048),
    # many-row kernel with several tile rounds per persistent workgroup
    (600, 520, 2048), (300, 1000, 1024),
    # many-row kernel with k % 256 != 0: a partial last weight group of 1, 2
    # or 3 steps, scale rows only 4-byte aligned
    (130, 300, 448), (257, 96, 320), (300, 200, 2176), (65, 40, 64),
]


@pytest.mark.parametrize("m,n,k", SHAPES)
def test_gemm_w4a16_matches_oracle(m, n, k):
    _say(f"gemm_w4a16 m={m} n={n} k={k}")
    x = si.activations(m, k, seed=m + n)
    w = si.weight(n, k, seed=k, code_stream=1, scale_stream=2, ts=0.75)
    y = nv.nvfp4_gemm_w4a16(x.cuda(), g_weight(w))
    sync()
    _, ye = oracle.gemm_w4a16(bits(x), o_weight(w))
    assert_close(bits(y), ye, f"gemm m={m} n={n} k={k}")


EXACT_SHAPES = [
    ("decode gate", 1, 12288, 4096, None),
    ("decode down", 1, 4096, 12288, None),
    ("smallm gate", 64, 17408, 5120, 1024),
    ("smallm down", 64, 5120, 17408, 512),
    ("prefill gate", 2048, 17408, 5120, 256),
    ("prefill down", 2048, 5120, 17408, 128),
    ("prefill down, one-eighth of inter", 2048, 5120, 2176, 128),
]


@pytest.mark.parametrize("name,m,n,k,ncols", EXACT_SHAPES)
def test_exact_case_bit_exact_at_full_shape(name, m, n, k, ncols):
    """Integer X, power-of-two scales: every fp32 partial sum is exact, so the
    GPU must equal the oracle bit for bit whatever its tiling or split."""
    _say(f"exact case {name} m={m} n={n} k={k}")
    x, w = si.exact_case(m, n, k, seed=3)
    y = nv.nvfp4_gemm_w4a16(x.cuda(), g_weight(w))
    sync()
    got = bits(y)
    rng = np.random.default_rng(5)
    rows = np.arange(m) if m <= 64 else np.sort(rng.choice(m, 24, replace=False))
    cols = np.arange(n) if ncols is None else np.sort(rng.choice(n, ncols, replace=False))
    yo, _ = oracle.gemm_w4a16(bits(x)[rows], o_weight(w, cols))
    assert np.array_equal(got[np.ix_(rows, cols)], yo)


# ---- silu_mul -------------------------------------------------------------------------

@pytest.mark.parametrize("count,spread", [(1, 4), (7, 4), (8, 4), (1000, 4), (12288, 4),
                                          (64 * 17408 + 3, 4), (100000, 60)])
def test_silu_mul_within_one_ulp(count, spread):
    """spread 60 reaches gates below -88, where exp(-g) overflows fp32."""
    _say(f"silu_mul count={count} spread={spread}")
    g = (torch.randn(count, generator=torch.Generator().manual_seed(count)) * spread).to(torch.bfloat16)
    u = (torch.randn(count, generator=torch.Generator().manual_seed(count + 1)) * 4).to(torch.bfloat16)
    gd, ud = g.cuda(), u.cuda()
    out = nv.silu_mul(gd.view(1, -1), ud.view(1, -1))
    inplace = gd.clone().view(1, -1)
    nv.silu_mul(inplace, ud.view(1, -1), out=inplace)
    sync()
    ref = oracle.silu_mul(bits(g), bits(u))
    got = bits(out).reshape(-1)
    assert np.array_equal(got, bits(inplace).reshape(-1))
    d = np.abs(got.astype(np.int32) - ref.astype(np.int32))
    same_sign = (got & 0x8000) == (ref & 0x8000)
    zero_pair = ((got & 0x7FFF) == 0) & ((ref & 0x7FFF) <= 1)
    assert np.all((same_sign & (d <= 1)) | zero_pair)


# ---- per-row quantizer (bit exact) -------------------------------------------------------

def _quant_rows(m, k, seed):
    rng = np.random.default_rng(seed)
    x = rng.normal(0, 1, (m, k)) * np.exp2(rng.integers(-20, 20, (m, 1)))
    x[0] = 0.0
    if m > 2:
        x[1, : k // 2] = 0.0
        x[2] *= 1e-30           # fp32-subnormal row scale
    if m > 3:
        x[3] = rng.integers(-6, 7, k) * 0.4375 / 4  # ties on the E2M1 grid
    return torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16)


@pytest.mark.parametrize("m,k", [(1, 32), (5, 4096), (7, 14336), (512, 4096), (4, 20480), (3, 67136),
                                 (64, 4096), (100, 14336)])
def test_quantize_rows_bit_exact(m, k):
    _say(f"quantize m={m} k={k}")
    x = _quant_rows(m, k, seed=m * 7 + k)
    c, s, r = nv.nvfp4_quantize_rows(x.cuda())
    sync()
    co, so, ro = oracle.quantize_rows(bits(x))
    assert np.array_equal(s.cpu().numpy(), so)
    assert np.array_equal(r.cpu().numpy().view(np.uint32), ro.view(np.uint32))
    assert np.array_equal(c.cpu().numpy(), co)


def test_quantize_rows_every_bf16_below_block_max():
    """E2M1 rounding decisions under inexact scales.  Each row's maximum has
    a random mantissa, so s_row = amax/2688 is an inexact fp32, and each run
    of blocks shares a random block maximum M (element 0 of each block of the
    run) while the other elements walk every bf16 value in [M/32, M) in
    order, with random signs: quotients on both sides of every grid midpoint
    for a few hundred (row scale, block scale) pairs.  Bit for bit against
    the oracle."""
    _say("quantize every bf16 below the block max")
    rng = np.random.default_rng(11)
    rows, k = 64, 4096
    nblk = k // 16
    xb = np.zeros((rows, k), np.uint16)
    for r in range(rows):
        amax = (int(rng.integers(127 - 30, 127 + 30)) << 7) | int(rng.integers(0, 128))
        xb[r, 0] = amax
        b = 1
        while b < nblk:
            mb = amax - int(rng.integers(0, 6 * 128))
            sweep = np.arange(mb - 5 * 128, mb, dtype=np.uint16)
            sweep |= (rng.integers(0, 2, sweep.size) << 15).astype(np.uint16)
            for j in range(0, sweep.size, 15):
                if b >= nblk:
                    break
                part = sweep[j:j + 15]
                xb[r, 16 * b] = mb
                xb[r, 16 * b + 1:16 * b + 1 + part.size] = part
                b += 1
    x = torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16)
    c, s, rs = nv.nvfp4_quantize_rows(x.cuda())
    sync()
    co, so, ro = oracle.quantize_rows(xb)
    assert np.array_equal(rs.cpu().numpy().view(np.uint32), ro.view(np.uint32))
    assert np.array_equal(s.cpu().numpy(), so)
    assert np.array_equal(c.cpu().numpy(), co)


def test_quantize_golden_rows_on_gpu():
    import test_oracle_compute as toc
    rows = toc._read_quant_golden()
    x = torch.tensor([r["x"] for r in rows], dtype=torch.float32).to(torch.bfloat16)
    k = x.shape[1]                       # 48; the library takes k % 32 == 0
    xp = torch.zeros((x.shape[0], 64), dtype=torch.bfloat16)
    xp[:, :k] = x                        # a zero block changes no other block
    c, s, r = nv.nvfp4_quantize_rows(xp.cuda())
    sync()
    for i, row in enumerate(rows):
        assert list(s[i].cpu().numpy()[: k // 16]) == row["scales"]
        assert list(toc._unpack(c[i].cpu().numpy())[:k]) == row["codes"]
        assert float(r[i]) == row["row_scale"]


# ---- W4A4 projection ------------------------------------------------------------------------

# beyond 64 rows the kernel takes 128-row blocks: 100 and 257 rows leave a
# ragged last block, (130, 48, 4096) splits K over workgroups with it, and
# n = 16400 takes two column tiles per workgroup
@pytest.mark.parametrize("m,n,k", [(1, 16, 32), (3, 100, 160), (64, 130, 1024), (100, 64, 512),
                                   (5, 40, 96), (12, 48, 352), (130, 48, 4096), (257, 200, 320),
                                   (300, 16400, 160)])
def test_gemm_w4a4_matches_oracle(m, n, k):
    _say(f"gemm_w4a4 m={m} n={n} k={k}")
    x = si.activations(m, k, seed=m + 2 * n)
    w = si.weight(n, k, seed=k + 1, code_stream=3, scale_stream=4, ts=1.25)
    y = nv.nvfp4_gemm_w4a4(x.cuda(), g_weight(w))
    sync()
    _, ye = oracle.gemm_w4a4(bits(x), o_weight(w))
    assert_close(bits(y), ye, f"w4a4 m={m} n={n} k={k}")


def test_gemm_w4a4_rows_independent_of_m():
    _say("w4a4 gemm invariance")
    hidden, inter = 4096, 14336
    x = si.activations(512, hidden, seed=9).cuda()
    w = g_weight(si.weight(inter, hidden, seed=9, code_stream=1, scale_stream=2))
    ref = nv.nvfp4_gemm_w4a4(x, w)
    for m in si.W4A4_ROW_COUNTS[:-1]:
        y = nv.nvfp4_gemm_w4a4(x[:m].contiguous(), w)
        sync()
        assert torch.equal(y.view(torch.int16), ref[:m].view(torch.int16)), m
    # K split over four workgroups; 65 and 130 rows: ragged 128-row blocks
    w = g_weight(si.weight(64, hidden, seed=10, code_stream=1, scale_stream=2))
    ref = nv.nvfp4_gemm_w4a4(x, w)
    for m in (1, 8, 64, 65, 130, 300):
        y = nv.nvfp4_gemm_w4a4(x[:m].contiguous(), w)
        sync()
        assert torch.equal(y.view(torch.int16), ref[:m].view(torch.int16)), ("split", m)


def _by_row_blocks(fn, x, block=16):
    """fn over consecutive blocks of `block` rows (the few-row kernels),
    stacked: the reference for a many-row launch, row for row."""
    return torch.cat([fn(x[r:r + block].contiguous()) for r in range(0, x.shape[0], block)])


# The many-row fixed-format kernel (from 65 rows) walks each output's four
# step classes one after another; its rows must equal the few-row streaming
# kernel's bit for bit.  Shapes: K split over four workgroups (n = 64,
# k = 4096) and over two (the down projection's 4096 x 14336), splits of two
# and three steps (k = 160, 384: idle classes), ragged rows and columns, and
# two column tiles per workgroup on the streaming side (n = 16400).
@pytest.mark.parametrize("m,n,k", [(65, 64, 4096), (200, 300, 160), (130, 1000, 384), (257, 16400, 512),
                                   (129, 4096, 14336)])
def test_gemm_w4a4_many_rows_equal_few_rows(m, n, k):
    _say(f"w4a4 many rows vs 16-row blocks m={m} n={n} k={k}")
    x = si.activations(m, k, seed=n + k, outliers=True).cuda()
    w = g_weight(si.weight(n, k, seed=m, code_stream=5, scale_stream=6, ts=0.75))
    y = nv.nvfp4_gemm_w4a4(x, w)
    ref = _by_row_blocks(lambda xb: nv.nvfp4_gemm_w4a4(xb, w), x)
    sync()
    assert torch.equal(y.view(torch.int16), ref.view(torch.int16))


@pytest.mark.parametrize("m", [65, 200])
def test_dense_ffn_w4a4_many_rows_equal_few_rows(m):
    """gate+up+silu (two matrices per workgroup) and the down projection on
    the tiny FFN: a two-step gate+up split (two idle classes) and a six-step
    down projection."""
    _say(f"ffn w4a4 many rows vs 16-row blocks m={m}")
    x, wg, wu, wd = si.workload("tiny", m=m)
    W = [g_weight(w) for w in (wg, wu, wd)]
    xd = x.cuda()
    y = nv.dense_ffn_forward_w4a4(xd, *W)
    ref = _by_row_blocks(lambda xb: nv.dense_ffn_forward_w4a4(xb, *W), xd)
    sync()
    assert torch.equal(y.view(torch.int16), ref.view(torch.int16))


# ---- gate+up+silu entry point -----------------------------------------------------------------

@pytest.mark.parametrize("m", [1, 5, 64, 96])
def test_gate_up_silu_matches_oracle(m):
    """gate and up meet the FFN tolerance against the oracle; the fused act
    equals silu_mul of the GPU's own gate and up (same K order) within one
    bf16 ulp.  act itself is heavy-tailed (max/rms >> 5), where a
    correctly rounded bf16 value can sit more than 2e-2 rms from the exact
    product, so the rms bound is not the right yardstick for it."""
    _say(f"gate_up_silu m={m}")
    x, wg, wu, wd = si.workload("tiny", m=m)
    xd = x.cuda()
    act = nv.nvfp4_gate_up_silu_w4a16(xd, g_weight(wg), g_weight(wu))
    g = nv.nvfp4_gemm_w4a16(xd, g_weight(wg))
    u = nv.nvfp4_gemm_w4a16(xd, g_weight(wu))
    sync()
    assert_close(bits(g), oracle.gemm_w4a16(bits(x), o_weight(wg))[1], f"gate m={m}")
    assert_close(bits(u), oracle.gemm_w4a16(bits(x), o_weight(wu))[1], f"up m={m}")
    ref = oracle.silu_mul(bits(g), bits(u))
    got = bits(act)
    d = np.abs(got.astype(np.int32) - ref.astype(np.int32))
    same_sign = (got & 0x8000) == (ref & 0x8000)
    zero_pair = ((got & 0x7FFF) == 0) & ((ref & 0x7FFF) <= 1)
    assert np.all((same_sign & (d <= 1)) | zero_pair)


@pytest.mark.parametrize("m,n,k", [(17, 300, 1024), (32, 48, 4096), (40, 1000, 2176), (64, 130, 64),
                                   (64, 4100, 512)])
def test_gate_up_silu_small_m_split_groups(m, n, k):
    """17..64 rows: column groups of 64 gate + 64 up columns cut between
    workgroups (16 pieces of one group at n=48, two or more elsewhere, ragged
    n and a partial last K unit).  gate and up meet the tolerance against the
    oracle; act equals silu_mul of the GPU's own gate and up within one ulp."""
    _say(f"gate_up_silu small m={m} n={n} k={k}")
    x = si.activations(m, k, seed=m + 7)
    wg = si.weight(n, k, seed=n + 1, code_stream=1, scale_stream=2, ts=0.75)
    wu = si.weight(n, k, seed=n + 2, code_stream=3, scale_stream=4, ts=1.25)
    xd = x.cuda()
    act = nv.nvfp4_gate_up_silu_w4a16(xd, g_weight(wg), g_weight(wu))
    g = nv.nvfp4_gemm_w4a16(xd, g_weight(wg))
    u = nv.nvfp4_gemm_w4a16(xd, g_weight(wu))
    sync()
    assert_close(bits(g), oracle.gemm_w4a16(bits(x), o_weight(wg))[1], f"gate m={m} n={n} k={k}")
    assert_close(bits(u), oracle.gemm_w4a16(bits(x), o_weight(wu))[1], f"up m={m} n={n} k={k}")
    ref = oracle.silu_mul(bits(g), bits(u))
    got = bits(act)
    d = np.abs(got.astype(np.int32) - ref.astype(np.int32))
    same_sign = (got & 0x8000) == (ref & 0x8000)
    zero_pair = ((got & 0x7FFF) == 0) & ((ref & 0x7FFF) <= 1)
    assert np.all((same_sign & (d <= 1)) | zero_pair)


def test_gate_up_silu_many_rows_split_tiles():
    """300 rows, hidden 2048, inter 640: two row blocks x five column groups,
    each split over several workgroups by K steps; act must still equal
    silu_mul of the separately computed gate and up within one bf16 ulp."""
    m, hidden, inter = 300, 2048, 640
    _say(f"gate_up_silu split tiles m={m} hidden={hidden} inter={inter}")
    x = si.activations(m, hidden, seed=11)
    wg = si.weight(inter, hidden, seed=12, code_stream=1, scale_stream=2)
    wu = si.weight(inter, hidden, seed=13, code_stream=3, scale_stream=4)
    xd = x.cuda()
    act = nv.nvfp4_gate_up_silu_w4a16(xd, g_weight(wg), g_weight(wu))
    g = nv.nvfp4_gemm_w4a16(xd, g_weight(wg))
    u = nv.nvfp4_gemm_w4a16(xd, g_weight(wu))
    sync()
    assert_close(bits(g), oracle.gemm_w4a16(bits(x), o_weight(wg))[1], "gate")
    assert_close(bits(u), oracle.gemm_w4a16(bits(x), o_weight(wu))[1], "up")
    ref = oracle.silu_mul(bits(g), bits(u))
    got = bits(act)
    d = np.abs(got.astype(np.int32) - ref.astype(np.int32))
    same_sign = (got & 0x8000) == (ref & 0x8000)
    zero_pair = ((got & 0x7FFF) == 0) & ((ref & 0x7FFF) <= 1)
    assert np.all((same_sign & (d <= 1)) | zero_pair)


# ---- rows beyond m and error paths ------------------------------------------------------------

def test_rows_beyond_m_untouched_and_errors_leave_output():
    x, wg, wu, wd = si.workload("tiny")
    m, hidden = x.shape
    out = torch.full((m + 3, hidden), 7.0, dtype=torch.bfloat16, device="cuda")
    nv.dense_ffn_forward(x.cuda(), g_weight(wg), g_weight(wu), g_weight(wd), out=out[:m])
    nv.dense_ffn_forward_w4a4(x.cuda(), g_weight(wg), g_weight(wu), g_weight(wd), out=out[:m])
    sync()
    assert torch.all(out[m:] == 7.0)
    before = out.clone()
    bad = nv.NVFP4Weight(g_weight(wd).codes, g_weight(wd).scales, 1.0)  # transposed role
    # the binding refuses it before calling the library ...
    with pytest.raises(ValueError):
        nv.dense_ffn_forward(x.cuda(), g_weight(wg), bad, g_weight(wd), out=out[:m])
    # ... and so does the C ABI itself, before enqueuing anything
    import ctypes
    L = nv.load_library()
    xd = x.cuda()
    cg, cb, cd = nv._cweight(g_weight(wg)), nv._cweight(bad), nv._cweight(g_weight(wd))
    rc = L.dense_ffn_forward(ctypes.c_void_p(xd.data_ptr()), m, hidden, cg.n, ctypes.byref(cg),
                             ctypes.byref(cb), ctypes.byref(cd), ctypes.c_void_p(out.data_ptr()),
                             ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == nv.NVFP4_ESHAPE
    sync()
    assert torch.equal(out, before)


# ---- every row of the many-row kernel -----------------------------------------------------------

def _spread_cols(n, count, tail, seed):
    """`count` columns spread over [0, n) plus `tail` from the last 1024
    (where the many-row kernel's second column launch works) and n - 1."""
    rng = np.random.default_rng(seed)
    cols = set(rng.choice(n, count, replace=False).tolist())
    cols |= set(rng.choice(np.arange(max(0, n - 1024), n), tail, replace=False).tolist())
    cols |= {0, n - 1}
    return np.array(sorted(cols))


@pytest.mark.parametrize("name,m,n,k", [("prefill down", 2048, 5120, 17408),
                                        ("prefill gate", 2048, 17408, 5120)])
def test_exact_case_every_row_many_row_kernel(name, m, n, k):
    """All 2048 rows (every row tile, the partial last row block included)
    for columns of every column range, bit for bit on exact inputs."""
    _say(f"exact case, every row: {name}")
    x, w = si.exact_case(m, n, k, seed=4)
    y = nv.nvfp4_gemm_w4a16(x.cuda(), g_weight(w))
    sync()
    cols = _spread_cols(n, 48, 16, seed=6)
    yo, _ = oracle.gemm_w4a16(bits(x), o_weight(w, cols))
    assert np.array_equal(bits(y)[:, cols], yo)


@pytest.mark.parametrize("m", [2048, 64, 40])
def test_exact_case_every_row_gate_up_silu(m):
    """The fused gate+up+silu launch at the prefill shape (every row, and
    columns of both of the many-row kernel's column launches) and at the
    small-m shape (64 and 40 rows: column groups split between workgroups
    and finished by the last piece).  gate and up are exact, so act must be
    the silu_mul of the oracle's gate and up within one bf16 ulp."""
    hidden, inter = 5120, 17408
    _say(f"exact case, every row: gate+up+silu m={m}")
    x, wg = si.exact_case(m, inter, hidden, seed=7)
    _, wu = si.exact_case(1, inter, hidden, seed=8)
    act = nv.nvfp4_gate_up_silu_w4a16(x.cuda(), g_weight(wg), g_weight(wu))
    sync()
    cols = _spread_cols(inter, 40, 24, seed=9)
    go, _ = oracle.gemm_w4a16(bits(x), o_weight(wg, cols))
    uo, _ = oracle.gemm_w4a16(bits(x), o_weight(wu, cols))
    ref = oracle.silu_mul(go, uo)
    got = bits(act)[:, cols]
    d = np.abs(got.astype(np.int32) - ref.astype(np.int32))
    same_sign = (got & 0x8000) == (ref & 0x8000)
    zero_pair = ((got & 0x7FFF) == 0) & ((ref & 0x7FFF) <= 1)
    assert np.all((same_sign & (d <= 1)) | zero_pair)
