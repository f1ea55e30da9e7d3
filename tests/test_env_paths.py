"""The environment switches of the library, each in a fresh child process
(the library reads them once, at its first call):

* NVFP4_FORCE_PATH names a kernel family; a shape it cannot serve is an
  ESHAPE error, never a silent fallback (page layers/mod.rs,
  `w4a16_v2_kernel`: a requested but missing variant refuses to start).
* NVFP4_ARENA_MAX_BYTES caps the scratch arena; a call that needs more
  fails with ENOMEM before anything is enqueued, output untouched.
* NVFP4_PROFILE=1 syncs around each FFN and prints one timing line
  (page layers/dense_ffn_prefill.rs, `forward_prefill`: under the profile
  flag the prefill FFN syncs its stream and logs its time).
* NVFP4_SPLITK_MIN_K keeps projections with a shorter K from splitting K
  over workgroups; results stay within tolerance and the fixed format
  stays row-invariant.

The forced-path refusal is checked on the CPU (the check runs before any
device call); the rest need the GPU.
"""

import os
import subprocess
import sys
import textwrap

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _child(code: str, env: dict, timeout=120):
    e = dict(os.environ)
    e.update(env)
    e["PYTHONPATH"] = ROOT + os.pathsep + os.path.join(ROOT, "tests") + os.pathsep + e.get("PYTHONPATH", "")
    r = subprocess.run([sys.executable, "-c", textwrap.dedent(code)], env=e, cwd=ROOT,
                       capture_output=True, text=True, timeout=timeout)
    print(r.stdout, r.stderr, flush=True)
    return r


def test_forced_path_refuses_a_shape_it_cannot_serve_cpu():
    code = """
        import ctypes
        import nvfp4_weight_dense_amd as nv
        L = nv.load_library()
        x, y, s = ctypes.c_void_p(0x40000), ctypes.c_void_p(0x80000), ctypes.c_void_p(None)
        w = nv._CWeight(0x10000, 0x20000, 1.0, 64, 4096)
        rc = L.nvfp4_gemm_w4a16(x, 64, ctypes.byref(w), y, s)   # gemv serves m <= 4 only
        print("rc", rc, nv.nvfp4_last_error())
        assert rc == nv.NVFP4_ESHAPE and "NVFP4_FORCE_PATH=gemv" in nv.nvfp4_last_error()
        hidden, inter = 256, 768
        wg, wu, wd = (nv._CWeight(0x10000, 0x20000, 1.0, inter, hidden),
                      nv._CWeight(0x10000, 0x20000, 1.0, inter, hidden),
                      nv._CWeight(0x10000, 0x20000, 1.0, hidden, inter))
        rc = L.dense_ffn_forward(x, 8, hidden, inter, ctypes.byref(wg), ctypes.byref(wu),
                                 ctypes.byref(wd), y, s)
        assert rc == nv.NVFP4_ESHAPE, rc
        print("FORCED_OK")
    """
    r = _child(code, {"NVFP4_FORCE_PATH": "gemv"})
    assert r.returncode == 0 and "FORCED_OK" in r.stdout
    code_prefill = """
        import ctypes
        import nvfp4_weight_dense_amd as nv
        L = nv.load_library()
        x, y, s = ctypes.c_void_p(0x40000), ctypes.c_void_p(0x80000), ctypes.c_void_p(None)
        w = nv._CWeight(0x10000, 0x20000, 1.0, 64, 96)      # k % 64 != 0
        rc = L.nvfp4_gemm_w4a16(x, 300, ctypes.byref(w), y, s)
        assert rc == nv.NVFP4_ESHAPE and "prefill" in nv.nvfp4_last_error(), rc
        print("FORCED_OK")
    """
    r = _child(code_prefill, {"NVFP4_FORCE_PATH": "prefill"})
    assert r.returncode == 0 and "FORCED_OK" in r.stdout


_GPU_PRELUDE = """
    import torch
    import nvfp4_weight_dense_amd as nv
    import synthetic_inputs as si
    from gpu_helpers import g_weight
    x, wg, wu, wd = si.workload("tiny", m=M)
    xd = x.cuda()
    W = [g_weight(w) for w in (wg, wu, wd)]
"""


@pytest.mark.gpu
def test_forced_path_refusal_leaves_output_untouched():
    code = _GPU_PRELUDE.replace("M", "64") + """
    out = torch.full((64, 256), 3.0, dtype=torch.bfloat16, device="cuda")
    try:
        nv.dense_ffn_forward(xd, *W, out=out)
        raise SystemExit("no error")
    except nv.Nvfp4Error as e:
        assert e.code == nv.NVFP4_ESHAPE, e
    torch.cuda.synchronize()
    assert bool(torch.all(out == 3.0))
    print("FORCED_GPU_OK", flush=True)
    """
    r = _child(code, {"NVFP4_FORCE_PATH": "gemv"})
    assert r.returncode == 0 and "FORCED_GPU_OK" in r.stdout


@pytest.mark.gpu
def test_arena_cap_gives_enomem_with_output_untouched():
    code = _GPU_PRELUDE.replace("M", "8") + """
    out = torch.full((8, 256), 5.0, dtype=torch.bfloat16, device="cuda")
    try:
        nv.dense_ffn_forward(xd, *W, out=out)   # act alone needs 8 x 768 x 2 bytes
        raise SystemExit("no error")
    except nv.Nvfp4Error as e:
        assert e.code == nv.NVFP4_ENOMEM, e
        assert "NVFP4_ARENA_MAX_BYTES" in str(e), e
    torch.cuda.synchronize()
    assert bool(torch.all(out == 5.0))
    print("ARENA_OK", flush=True)
    """
    r = _child(code, {"NVFP4_ARENA_MAX_BYTES": "4096"})
    assert r.returncode == 0 and "ARENA_OK" in r.stdout


@pytest.mark.gpu
def test_profile_line():
    code = _GPU_PRELUDE.replace("M", "4") + """
    y = nv.dense_ffn_forward(xd, *W)
    torch.cuda.synchronize()
    print("PROFILE_RAN", flush=True)
    """
    r = _child(code, {"NVFP4_PROFILE": "1"})
    assert r.returncode == 0 and "PROFILE_RAN" in r.stdout
    import re
    assert re.search(r"FFN \[dense_total\] m=4: \d+us", r.stderr), r.stderr


@pytest.mark.gpu
def test_splitk_min_k_keeps_results_and_invariance():
    code = """
    import numpy as np
    import torch
    import nvfp4_weight_dense_amd as nv
    import oracle
    import synthetic_inputs as si
    from gpu_helpers import assert_close, bits, g_weight, o_weight
    # deep-K shapes that split by default: the small-m and streaming kernels
    for name, m in (("smallm", 40), ("decode", 8)):
        x, wg, wu, wd = si.workload(name, m=m)
        y = nv.dense_ffn_forward(x.cuda(), *[g_weight(w) for w in (wg, wu, wd)])
        torch.cuda.synchronize()
        rows = np.array([0, m - 1])
        _, ye = oracle.dense_ffn(bits(x)[rows], o_weight(wg), o_weight(wu), o_weight(wd))
        assert_close(bits(y)[rows], ye, name)
    x, wg, wu, wd = si.workload("w4a4", m=64)
    W = [g_weight(w) for w in (wg, wu, wd)]
    xd = x.cuda()
    ref = nv.dense_ffn_forward_w4a4(xd, *W)
    for m in (1, 8):
        y = nv.dense_ffn_forward_w4a4(xd[:m].contiguous(), *W)
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), ref[:m].view(torch.int16)), m
    print("SPLITK_OK", flush=True)
    """
    r = _child(code, {"NVFP4_SPLITK_MIN_K": str(1 << 30), "NVFP4_LOG": "1"})
    assert r.returncode == 0 and "SPLITK_OK" in r.stdout
