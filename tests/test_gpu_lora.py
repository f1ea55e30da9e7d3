"""GPU parity of the LoRA overlay (nvfp4_lora_delta, dense_ffn_forward_lora)
against the oracle, on seeded inputs.

The delta alone has the usual bound (max|err| <= 2e-2 * rms of the oracle's
value before its last rounding).  The FFN with the overlay rounds twice
more than the plain FFN: gate/up and the output are rounded to bf16 before
their deltas are added (the overlay updates bf16 buffers in place), and the
GPU's and the oracle's first roundings may differ by one ulp.  Its bound
adds that one rounding at the element's own magnitude:
|err_i| <= 2e-2 * rms(ref) + 2^-7 * |ref_i| (one bf16 ulp is at most
2^-7 of the value)."""

import numpy as np
import pytest
import torch

import nvfp4_weight_dense_amd as nv
import oracle
import synthetic_inputs as si
from gpu_helpers import assert_close, bf16_f64, bits, g_weight, o_weight, sync

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


def _pair(n, k, rank, which, scale, seed=0):
    a, b = si.lora_pair(n, k, rank, seed=seed, which=which)
    return (nv.LoraPair(a.cuda(), b.cuda(), scale),
            oracle.Lora(bits(a), bits(b), scale))


@pytest.mark.parametrize("m,k,n,rank", [(1, 4096, 3000, 16), (5, 512, 777, 8), (3, 12288, 4096, 64),
                                        (70, 256, 768, 256)])
def test_lora_delta_matches_oracle(m, k, n, rank):
    _say(f"lora delta m={m} k={k} n={n} rank={rank}")
    x = si.activations(m, k, seed=5)
    base = si.activations(m, n, seed=6)
    gp, op = _pair(n, k, rank, 0, 0.75)
    got = nv.nvfp4_lora_delta(x.cuda(), gp, base.cuda().clone())
    sync()
    _, exact = oracle.lora_delta(bits(x), op, bits(base))
    assert_close(bits(got), exact, "lora delta")
    # the delta part alone, against the delta the oracle adds
    d_gpu = got.cpu().double().numpy() - base.double().numpy()
    d_ref = exact - base.double().numpy()
    err = np.max(np.abs(d_gpu - d_ref)) / np.sqrt(np.mean(d_ref ** 2))
    assert err <= 2e-2, err


@pytest.mark.parametrize("name,m", [("tiny", 1), ("tiny", 4), ("tiny", 40), ("tiny", 70), ("decode", 1)])
def test_dense_ffn_lora_matches_oracle(name, m):
    _say(f"ffn lora {name} m={m}")
    x, wg, wu, wd = si.workload(name, m=m)
    hidden, inter = x.shape[1], wg.n
    pg, og = _pair(inter, hidden, 16, 0, 2.0)
    pu, ou = _pair(inter, hidden, 16, 1, -1.5)
    pd, od = _pair(hidden, inter, 16, 2, 0.5)
    y = nv.dense_ffn_forward_lora(x.cuda(), g_weight(wg), g_weight(wu), g_weight(wd), pg, pu, pd)
    sync()
    _, ye = oracle.dense_ffn_lora(bits(x), o_weight(wg), o_weight(wu), o_weight(wd), og, ou, od)
    got = bf16_f64(bits(y))
    assert np.all(np.isfinite(got))
    bound = 2e-2 * np.sqrt(np.mean(ye ** 2)) + 2.0 ** -7 * np.abs(ye)
    worst = np.max(np.abs(got - ye) / bound)
    assert worst <= 1.0, f"ffn lora {name} m={m}: max err/bound = {worst:.3f}"
    # the overlay changes the result by much more than the tolerance
    _, ye0 = oracle.dense_ffn(bits(x), o_weight(wg), o_weight(wu), o_weight(wd))
    assert np.max(np.abs(ye - ye0)) > 0.2 * np.sqrt(np.mean(ye0 ** 2))


@pytest.mark.parametrize("which", ["gate", "up", "down"])
def test_dense_ffn_lora_single_pair(which):
    """Only one of the three pairs present (the others rank 0)."""
    _say(f"ffn lora, {which} only")
    x, wg, wu, wd = si.workload("tiny", m=3)
    hidden, inter = x.shape[1], wg.n
    shapes = {"gate": (inter, hidden, 0), "up": (inter, hidden, 1), "down": (hidden, inter, 2)}
    n, k, w = shapes[which]
    gp, op = _pair(n, k, 8, w, 1.25)
    gpu = {which: gp}
    orc = {which: op}
    y = nv.dense_ffn_forward_lora(x.cuda(), g_weight(wg), g_weight(wu), g_weight(wd),
                                  gpu.get("gate"), gpu.get("up"), gpu.get("down"))
    sync()
    _, ye = oracle.dense_ffn_lora(bits(x), o_weight(wg), o_weight(wu), o_weight(wd),
                                  orc.get("gate"), orc.get("up"), orc.get("down"))
    got = bf16_f64(bits(y))
    bound = 2e-2 * np.sqrt(np.mean(ye ** 2)) + 2.0 ** -7 * np.abs(ye)
    assert np.max(np.abs(got - ye) / bound) <= 1.0


# ranks: gate and up at most 16 (their B rows are loaded with the batch's
# weights) or above it (loaded in the epilogue), mismatched either way
@pytest.mark.parametrize("m,rg,ru,rd", [(1, 16, 8, 24), (2, 16, 8, 24), (3, 16, 8, 24), (4, 16, 8, 24),
                                        (1, 32, 8, 16), (2, 24, 32, 8), (3, 8, 24, 32), (4, 32, 16, 24)])
def test_dense_ffn_lora_fused_epilogue_equals_composition(m, rg, ru, rd):
    """Up to four rows the GEMVs add the LoRA deltas in their epilogues; the
    result must equal, bit for bit, the same FFN composed from the separate
    entry points (gate and up GEMMs, LoRA deltas into the bf16 buffers,
    silu_mul, down GEMM, down delta): the same roundings in the same order."""
    _say(f"ffn lora fused vs composed m={m} ranks {rg}/{ru}/{rd}")
    x, wg, wu, wd = si.workload("tiny", m=m)
    hidden, inter = x.shape[1], wg.n
    pg, _ = _pair(inter, hidden, rg, 0, 2.0)
    pu, _ = _pair(inter, hidden, ru, 1, -1.5)
    pd, _ = _pair(hidden, inter, rd, 2, 0.5)
    xd = x.cuda()
    Wg, Wu, Wd = g_weight(wg), g_weight(wu), g_weight(wd)
    y = nv.dense_ffn_forward_lora(xd, Wg, Wu, Wd, pg, pu, pd)
    g = nv.nvfp4_lora_delta(xd, pg, nv.nvfp4_gemm_w4a16(xd, Wg))
    u = nv.nvfp4_lora_delta(xd, pu, nv.nvfp4_gemm_w4a16(xd, Wu))
    act = nv.silu_mul(g, u)
    y2 = nv.nvfp4_lora_delta(act, pd, nv.nvfp4_gemm_w4a16(act, Wd))
    sync()
    assert np.array_equal(bits(y), bits(y2))


def test_dense_ffn_lora_without_pairs_is_dense_ffn():
    _say("ffn lora, no pairs")
    x, wg, wu, wd = si.workload("tiny", m=6)
    W = [g_weight(w) for w in (wg, wu, wd)]
    y0 = nv.dense_ffn_forward(x.cuda(), *W)
    y1 = nv.dense_ffn_forward_lora(x.cuda(), *W)
    sync()
    assert torch.equal(y0.view(torch.int16), y1.view(torch.int16))
