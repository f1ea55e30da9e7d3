"""Exhaustive pin of the oracle's fp32 -> E4M3 and fp32 -> E2M1 encoders (CPU).

``exhaustive_encode.c`` encodes every one of the 2^32 fp32 bit patterns with
the oracle and compares each code with the nearest entry of the format's value
set, decoded from the bit fields (E4M3 and E2M1 element encodings of the OCP
Microscaling spec that NVFP4 builds on), ties to the even code, saturation at
the largest finite value, sign kept.  A second run plants a rounding mistake
in a copy of the oracle (ties away from zero instead of to even) and checks
that the sweep reports it, so a silent checker cannot pass.
"""

import os
import re
import subprocess

import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
CHECKER = os.path.join(HERE, "exhaustive_encode.c")


def _threads():
    return max(1, min(8, len(os.sched_getaffinity(0))))


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    exe = str(tmp_path_factory.mktemp("exh") / "exhaustive_encode")
    subprocess.run(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-Wall", "-o", exe, CHECKER,
                    "-ldl", "-lpthread", "-lm"], check=True)
    return exe


def _run(exe, lib):
    r = subprocess.run([exe, lib, str(_threads())], capture_output=True, text=True, timeout=600)
    counts = dict(re.findall(r"^(e4m3|e2m1) checked=\d+ mismatches=(\d+)$", r.stdout, re.M))
    checked = re.findall(r"^(?:e4m3|e2m1) checked=(\d+)", r.stdout, re.M)
    return r, {k: int(v) for k, v in counts.items()}, [int(c) for c in checked]


def test_encoders_match_nearest_even_on_every_fp32(checker):
    r, bad, checked = _run(checker, oracle.build(force=False))
    assert checked == [2 ** 32, 2 ** 32], r.stdout + r.stderr
    assert bad == {"e4m3": 0, "e2m1": 0}, r.stdout
    assert r.returncode == 0


def test_sweep_reports_a_planted_rounding_mistake(checker, tmp_path):
    src = open(os.path.join(os.path.dirname(oracle.__file__), "nvfp4_oracle.c")).read()
    planted = src.replace("rint(", "round(")
    assert planted != src
    (tmp_path / "nvfp4_oracle.c").write_text(planted)
    hdr = os.path.join(os.path.dirname(oracle.__file__), "nvfp4_oracle.h")
    (tmp_path / "nvfp4_oracle.h").write_text(open(hdr).read())
    lib = str(tmp_path / "libplanted.so")
    subprocess.run(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fPIC", "-shared", "-o", lib,
                    str(tmp_path / "nvfp4_oracle.c"), "-lm", "-lpthread"], check=True)
    r, bad, _ = _run(checker, lib)
    assert r.returncode == 1, r.stdout + r.stderr
    assert bad["e4m3"] > 0 and bad["e2m1"] > 0, r.stdout
