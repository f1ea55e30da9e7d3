"""GPU parity of the packed-Q2 FFN (2-bit codes, fp16 scale per group,
dequantized to bf16, bf16 activations) against the oracle, through the
C-ABI.

* Projections are within max|err| <= 2e-2 * rms(ref) of the oracle's fp64
  value on shapes that span several tiles, ragged columns and K, split K,
  both column-tile widths and group sizes 32/64/128; the FFN on the full
  workloads (sampled rows) too.  The tiny FFN's outputs reach 10 * rms,
  where the bf16 rounding of the output alone exceeds 2e-2 * rms, so it is
  held to the element-wise bound 2e-2 * rms(ref) + 2^-8 * |ref_i| (one
  bf16 ulp of the element).
* Up to 64 rows the projections stream the packed weight (k_q2); more rows
  take the pages' default leg (dequantize to bf16, then a library GEMM).
  Both are covered: tiny FFNs at m in {65, 130}, the prefill workload.
* Exact case, bit for bit at a full projection shape: integer activations
  in [-2, 2] and power-of-two scales make every dequantized weight, every
  product and every fp32 partial sum exact, so any summation order gives
  the oracle's bf16 result.
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


def gq(w: si.Q2Weight) -> nv.Q2Weight:
    return nv.Q2Weight(w.codes.cuda().contiguous(), w.scales.cuda().contiguous(), w.group)


def oq(w: si.Q2Weight) -> oracle.Q2Weight:
    return oracle.Q2Weight(w.codes.numpy(), w.scales.view(torch.int16).numpy().view(np.uint16),
                           w.group)


@pytest.mark.parametrize("m,n,k,group", [(1, 48, 128, 128), (5, 300, 384, 128), (17, 130, 224, 32),
                                         (70, 257, 640, 64), (3, 64, 4096, 128),
                                         (3, 16400, 256, 128), (64, 1000, 2048, 128),
                                         (2, 40, 512, 256), (130, 96, 768, 256),
                                         # up to 16 rows with a ragged last 128-K step
                                         (4, 72, 160, 32), (9, 33, 96, 32), (1, 16, 224, 32),
                                         # many rows: a partial last 512-K weight group (k % 512
                                         # != 0), 32-element groups, two column launches; k % 64
                                         # != 0 takes the streaming kernel with 64-row blocks
                                         (300, 200, 2176, 128), (257, 96, 320, 32), (65, 40, 64, 32),
                                         (600, 1100, 1024, 128), (100, 72, 96, 32),
                                         # 17..64 rows, k % 64 == 0 (the small-m kernel):
                                         # groups of 32 to 256, a partial last 256-K unit, one
                                         # column group split over 16 workgroups, ragged n
                                         (40, 300, 320, 32), (17, 129, 2176, 64), (64, 70, 512, 256),
                                         (48, 48, 4096, 128), (33, 1000, 1088, 32)])
def test_q2_gemm_matches_oracle(m, n, k, group):
    _say(f"q2 gemm m={m} n={n} k={k} group={group}")
    x = si.activations(m, k, seed=n, outliers=True)
    w = si.q2_weight(n, k, seed=m, which=0, group=group)
    y = nv.q2_gemm_w2a16(x.cuda(), gq(w))
    sync()
    _, ye = oracle.gemm_q2(bits(x), oq(w))
    # outlier activations make some outputs heavy-tailed: rounding v to bf16
    # moves it by up to 2^-8 |v| (half an ulp at the bottom of a binade), so
    # with outputs beyond 2e-2 / 2^-8 = 5.12 x rms(ref) even the correctly
    # rounded result can miss 2e-2 rms; the element-wise bound (one bf16 ulp
    # more) always applies, the plain one where it is attainable
    assert_close_elem(bits(y), ye, f"q2 gemm m={m} n={n} k={k}")
    if np.max(np.abs(ye)) <= 5.12 * np.sqrt(np.mean(ye ** 2)):
        assert_close(bits(y), ye, f"q2 gemm m={m} n={n} k={k}")


# m = 130 and 2048 take the many-row kernel (k = 2176: a partial last weight group)
@pytest.mark.parametrize("m,n,k", [(2, 12288, 4096), (33, 4096, 12288), (130, 4096, 12288),
                                   (2048, 512, 2176)])
def test_q2_gemm_exact_case_bit_exact(m, n, k):
    _say(f"q2 gemm exact m={m} n={n} k={k}")
    g = torch.Generator().manual_seed(n)
    x = torch.randint(-2, 3, (m, k), generator=g).to(torch.bfloat16)
    codes = torch.randint(0, 256, (n, k // 4), generator=g, dtype=torch.uint8)
    e = torch.randint(-4, 1, (n, k // 128), generator=g).to(torch.float32)
    scales = torch.exp2(e).to(torch.float16).view(torch.int16).view(torch.uint16).contiguous()
    w = si.Q2Weight(codes, scales, 128)
    y = nv.q2_gemm_w2a16(x.cuda(), gq(w))
    sync()
    yo, _ = oracle.gemm_q2(bits(x), oq(w))
    assert np.array_equal(bits(y), yo)


@pytest.mark.parametrize("m", [1, 4, 17, 65, 130])
def test_dense_ffn_q2_tiny_matches_oracle(m):
    _say(f"ffn q2 tiny m={m}")
    x, wg, wu, wd = si.q2_workload("tiny", m=m)
    y = nv.dense_ffn_forward_q2(x.cuda(), gq(wg), gq(wu), gq(wd))
    sync()
    _, ye = oracle.dense_ffn_q2(bits(x), oq(wg), oq(wu), oq(wd))
    assert_close_elem(bits(y), ye, f"ffn q2 tiny m={m}")


def _rows(m, count, seed):
    if m <= count:
        return np.arange(m)
    rng = np.random.default_rng(seed)
    picked = set(rng.choice(m, count - 2, replace=False).tolist()) | {0, m - 1}
    return np.array(sorted(picked))


@pytest.mark.parametrize("name,nrows", [("decode", 1), ("smallm", 3), ("prefill", 3)])
def test_dense_ffn_q2_full_workload_matches_oracle(name, nrows):
    _say(f"ffn q2 {name}")
    x, wg, wu, wd = si.q2_workload(name)
    y = nv.dense_ffn_forward_q2(x.cuda(), gq(wg), gq(wu), gq(wd))
    sync()
    rows = _rows(x.shape[0], nrows, seed=5)
    _, ye = oracle.dense_ffn_q2(bits(x)[rows], oq(wg), oq(wu), oq(wd))
    assert_close(bits(y)[rows], ye, f"ffn q2 {name}")


def test_q2_m_zero_and_errors_touch_nothing():
    _say("q2 m=0 / errors")
    x, wg, wu, wd = si.q2_workload("tiny", m=4)
    out = torch.full((4, 256), 7.0, dtype=torch.bfloat16, device="cuda")
    nv.dense_ffn_forward_q2(x[:0].cuda(), gq(wg), gq(wu), gq(wd), out=out[:0])
    with pytest.raises(ValueError):
        nv.dense_ffn_forward_q2(x.cuda(), gq(wg), gq(wu), gq(wg), out=out)  # wd's shape: refused by the binding
    bad = si.Q2Weight(wg.codes, wg.scales[:, :1].contiguous(), 256)  # group 256 on hidden 256: fine shape,
    with pytest.raises(nv.Nvfp4Error):                              # but gate and up groups differ
        nv.dense_ffn_forward_q2(x.cuda(), gq(bad), gq(wu), gq(wd), out=out)
    sync()
    assert bool((out == 7.0).all())
