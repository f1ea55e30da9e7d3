"""End-to-end GPU parity of dense_ffn_forward (W4A16) and
dense_ffn_forward_w4a4 against the oracle on every workload, at full size.

Rows of an FFN are independent, so at the large workloads the oracle runs
the full FFN on a sample of rows (all of hidden/inter) and the GPU output
rows are compared with it.  W4A4 batch invariance is checked GPU against
GPU: rows 0..m-1 at m in {1, 8, 64} equal the m = 512 run bit for bit.
"""

import numpy as np
import pytest
import torch

import nvfp4_weight_dense_amd as nv
import oracle
import synthetic_inputs as si
from gpu_helpers import assert_close, bits, g_weight, o_weight, sync

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


def _rows(m, count, seed):
    if m <= count:
        return np.arange(m)
    rng = np.random.default_rng(seed)
    picked = set(rng.choice(m, count - 2, replace=False).tolist()) | {0, m - 1}
    return np.array(sorted(picked))


@pytest.mark.parametrize("name,nrows", [("tiny", 4), ("decode", 1), ("smallm", 6), ("prefill", 6),
                                        ("decode_tp8", 1), ("prefill_tp8", 6)])
def test_dense_ffn_w4a16_matches_oracle(name, nrows):
    _say(f"ffn w4a16 {name}")
    x, wg, wu, wd = si.workload(name)
    y = nv.dense_ffn_forward(x.cuda(), g_weight(wg), g_weight(wu), g_weight(wd))
    sync()
    rows = _rows(x.shape[0], nrows, seed=1)
    _, ye = oracle.dense_ffn(bits(x)[rows], o_weight(wg), o_weight(wu), o_weight(wd))
    assert_close(bits(y)[rows], ye, f"ffn {name}")


@pytest.mark.parametrize("m", [2, 17, 64, 65, 130])
def test_dense_ffn_w4a16_row_counts(m):
    _say(f"ffn w4a16 tiny m={m}")
    x, wg, wu, wd = si.workload("tiny", m=m)
    y = nv.dense_ffn_forward(x.cuda(), g_weight(wg), g_weight(wu), g_weight(wd))
    sync()
    _, ye = oracle.dense_ffn(bits(x), o_weight(wg), o_weight(wu), o_weight(wd))
    assert_close(bits(y), ye, f"ffn tiny m={m}")


def _block_rows(m, block=64):
    """The first and last row of every `block`-row block."""
    return np.array(sorted({r for b in range(0, m, block) for r in (b, min(m, b + block) - 1)}))


@pytest.mark.parametrize("name,m,nrows", [("tiny", 4, 4), ("w4a4", 64, 4), ("w4a4", 512, None)])
def test_dense_ffn_w4a4_matches_oracle(name, m, nrows):
    _say(f"ffn w4a4 {name} m={m}")
    x, wg, wu, wd = si.workload(name, m=m)
    y = nv.dense_ffn_forward_w4a4(x.cuda(), g_weight(wg), g_weight(wu), g_weight(wd))
    sync()
    # m = 512: one row at each end of every 64-row block
    rows = _block_rows(m) if nrows is None else _rows(m, nrows, seed=2)
    _, ye = oracle.dense_ffn(bits(x)[rows], o_weight(wg), o_weight(wu), o_weight(wd), w4a4=True)
    assert_close(bits(y)[rows], ye, f"ffn w4a4 {name} m={m}")


def test_dense_ffn_w4a4_batch_invariance():
    _say("ffn w4a4 invariance")
    x, wg, wu, wd = si.workload("w4a4")  # m = 512
    xd = x.cuda()
    W = [g_weight(w) for w in (wg, wu, wd)]
    ref = nv.dense_ffn_forward_w4a4(xd, *W)
    for m in si.W4A4_ROW_COUNTS[:-1]:
        y = nv.dense_ffn_forward_w4a4(xd[:m].contiguous(), *W)
        sync()
        assert torch.equal(y.view(torch.int16), ref[:m].view(torch.int16)), f"m={m}"
    # a row's bits also do not depend on which other rows share the launch
    perm = torch.randperm(512, generator=torch.Generator().manual_seed(0)).cuda()
    y = nv.dense_ffn_forward_w4a4(xd[perm].contiguous(), *W)
    sync()
    assert torch.equal(y.view(torch.int16), ref[perm].view(torch.int16))


def test_w4a4_activation_codes_match_oracle_on_gpu_activations():
    """The quantizer applied to the GPU's own act matches the oracle's
    quantizer bit for bit (isolates it from ulp differences upstream)."""
    _say("w4a4 act quantizer")
    x, wg, wu, wd = si.workload("w4a4", m=8)
    act = nv.nvfp4_gate_up_silu_w4a16(x.cuda(), g_weight(wg), g_weight(wu))
    c, s, r = nv.nvfp4_quantize_rows(act)
    sync()
    co, so, ro = oracle.quantize_rows(bits(act))
    assert np.array_equal(c.cpu().numpy(), co)
    assert np.array_equal(s.cpu().numpy(), so)
    assert np.array_equal(r.cpu().numpy(), ro)


@pytest.mark.parametrize("name,m", [("tiny", 1), ("tiny", 40), ("tiny", 200), ("decode", 1)])
def test_dense_ffn_fused_gate_up_weight(name, m):
    """A [2*inter, hidden] buffer holding gate then up gives the same bits
    as the separate weights (GEMV, small-m and many-row paths; the full
    decode workload as the benchmark runs it), and the oracle's result
    within tolerance."""
    _say(f"ffn fused gate+up weight {name} m={m}")
    x, wg, wu, wd = si.workload(name, m=m)
    assert wg.ts == wu.ts
    wgu = nv.NVFP4Weight(torch.cat([wg.codes, wu.codes]).cuda(),
                         torch.cat([wg.scales, wu.scales]).cuda(), wg.ts)
    gv, uv = nv.nvfp4_gate_up_views(wgu)
    assert gv.codes.data_ptr() == wgu.codes.data_ptr()
    assert uv.scales.data_ptr() == wgu.scales.data_ptr() + wg.n * wg.k // 16
    xd, gd = x.cuda(), g_weight(wd)
    y_fused = nv.dense_ffn_forward_fused(xd, wgu, gd)
    y_sep = nv.dense_ffn_forward(xd, g_weight(wg), g_weight(wu), gd)
    sync()
    assert torch.equal(y_fused.view(torch.int16), y_sep.view(torch.int16))
    _, ye = oracle.dense_ffn(bits(x), o_weight(wg), o_weight(wu), o_weight(wd))
    assert_close(bits(y_fused), ye, f"ffn fused {name} m={m}")
