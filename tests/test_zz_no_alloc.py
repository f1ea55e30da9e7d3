"""dense_ffn_forward_noalloc (the allocation-free FFN, through the C ABI)
gives the bits of dense_ffn_forward, on two calls in a row (the second
smaller, so the fixed scratch still holds the first call's data), and
refuses a shape whose scratch does not fit before anything is enqueued."""

import numpy as np
import pytest
import torch

import nvfp4_weight_dense_amd as nv
import synthetic_inputs as si
from gpu_helpers import g_weight, sync

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


def _pair(name, m):
    x, wg, wu, wd = si.workload(name, m=m)
    xd = x.cuda()
    W = [g_weight(w) for w in (wg, wu, wd)]
    ref = nv.dense_ffn_forward(xd, *W)
    out = torch.full_like(ref, float("nan"))
    return xd, W, ref, out


@pytest.mark.parametrize("calls", [
    # small-m kernels with split-K partials, then the single-row GEMV
    (("smallm", 64), ("decode", 1)),
    # the 16-row streaming kernel (arrival counters), then fewer rows of it
    (("tiny", 16), ("tiny", 9)),
    # the many-row kernel (act only), then the small-m kernel, tiny shapes
    (("tiny", 130), ("tiny", 48)),
])
def test_noalloc_matches_dense_ffn_forward(calls):
    for name, m in calls:
        _say(f"noalloc {name} m={m}")
        xd, W, ref, out = _pair(name, m)
        got = nv.dense_ffn_forward_noalloc(xd, *W, out=out)
        sync()
        assert got.data_ptr() == out.data_ptr()
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), f"{name} m={m}"


def test_noalloc_refuses_a_shape_beyond_its_scratch():
    _say("noalloc refusal")
    x, wg, wu, wd = si.workload("prefill")   # m = 2048: act alone is 68 MiB
    xd = x.cuda()
    W = [g_weight(w) for w in (wg, wu, wd)]
    out = torch.full((2048, 5120), 7.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(nv.Nvfp4Error) as e:
        nv.dense_ffn_forward_noalloc(xd, *W, out=out)
    assert e.value.code == nv.NVFP4_ENOMEM
    assert "fixed scratch" in str(e.value)
    sync()
    assert bool(torch.all(out == 7.0))
    # and a call after the refusal still works
    xs, Ws, ref, outs = _pair("tiny", 4)
    nv.dense_ffn_forward_noalloc(xs, *Ws, out=outs)
    sync()
    assert torch.equal(outs.view(torch.int16), ref.view(torch.int16))
