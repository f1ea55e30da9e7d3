"""Pins for the oracle's LoRA overlay (CPU only).

The overlay adds dW . input with dW = scale * B . A (page
layers/dense_ffn_overlays.rs, `apply_lora_gate_up`: gate_out += dW_gate . x
and up_out += dW_up . x before the activation; `apply_lora_down`: output +=
dW_down . act, act being silu(gate)*up).  The oracle takes the delta as two
thin products (x . A^T, then . B^T); the pins compare it with the dense
product B . A formed first (associativity, exact on small integers), and
with identity pairs whose effect on the FFN is known in closed form, which
fixes which tensor each delta reads and where it is added.
"""

import numpy as np
import pytest
import torch

import oracle
import synthetic_inputs as si


def _bf16_bits(v: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(v, dtype=np.float32)).to(
        torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _val(b: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).view(
        torch.bfloat16).double().numpy()


def _weights(hidden, inter, seed):
    _, wg, wu, wd = si.workload("tiny", seed=seed, m=1)
    # cut the tiny workload's matrices to [inter][hidden] / [hidden][inter]
    def cut(w, n, k):
        return oracle.Weight(w.codes.numpy()[:n, : k // 2].copy(),
                             w.scales.numpy()[:n, : k // 16].copy(), w.ts)
    return cut(wg, inter, hidden), cut(wu, inter, hidden), cut(wd, hidden, inter)


def test_lora_delta_equals_dense_low_rank_product():
    """Non-square shapes (r=3, k=8, n=5) so a transposed A or B fails."""
    rng = np.random.default_rng(7)
    m, k, r, n = 2, 8, 3, 5
    x = rng.integers(-3, 4, (m, k))
    a = rng.integers(-3, 4, (r, k))
    b = rng.integers(-3, 4, (n, r))
    base = rng.integers(-3, 4, (m, n))
    scale = 0.5
    got, exact = oracle.lora_delta(_bf16_bits(x), oracle.Lora(_bf16_bits(a), _bf16_bits(b), scale),
                                   _bf16_bits(base))
    want = base + scale * (x @ (b @ a).T)          # dense dW formed first, integers
    assert np.array_equal(exact, want.astype(np.float64))
    assert np.array_equal(got, _bf16_bits(want.astype(np.float64)))


def test_lora_zero_scale_and_rank_zero_leave_base_unchanged():
    rng = np.random.default_rng(8)
    x = _bf16_bits(rng.normal(size=(3, 32)))
    base = _bf16_bits(rng.normal(size=(3, 16)))
    a = _bf16_bits(rng.normal(size=(4, 32)))
    b = _bf16_bits(rng.normal(size=(16, 4)))
    got, _ = oracle.lora_delta(x, oracle.Lora(a, b, 0.0), base)
    assert np.array_equal(got, base)
    got, _ = oracle.lora_delta(x, oracle.Lora(a[:0], b[:, :0], 1.0), base)
    assert np.array_equal(got, base)


def test_ffn_without_pairs_is_the_plain_ffn():
    wg, wu, wd = _weights(64, 96, seed=3)
    x = _bf16_bits(np.random.default_rng(9).normal(size=(3, 64)))
    y0, e0 = oracle.dense_ffn(x, wg, wu, wd)
    y1, e1 = oracle.dense_ffn_lora(x, wg, wu, wd, None, None, None)
    assert np.array_equal(y0, y1) and np.array_equal(e0, e1)


def _eye(n):
    return _bf16_bits(np.eye(n))


@pytest.mark.parametrize("where", ["gate", "up", "down"])
def test_identity_pair_adds_the_right_input_at_the_right_place(where):
    """hidden == inter, dW = I: the gate/up delta adds x to that projection
    (before silu), the down delta adds act (silu(gate)*up, not x) to the
    rounded down output."""
    n = 32
    wg, wu, wd = _weights(n, n, seed=4)
    x = _bf16_bits(np.random.default_rng(10).normal(size=(2, n)))
    eye = oracle.Lora(_eye(n), _eye(n), 1.0)
    pairs = {"gate": (eye, None, None), "up": (None, eye, None), "down": (None, None, eye)}[where]
    y, _ = oracle.dense_ffn_lora(x, wg, wu, wd, *pairs)
    g, _ = oracle.gemm_w4a16(x, wg)
    u, _ = oracle.gemm_w4a16(x, wu)
    if where == "gate":
        g = _bf16_bits(_val(g) + _val(x))
    if where == "up":
        u = _bf16_bits(_val(u) + _val(x))
    act = oracle.silu_mul(g, u)
    want, _ = oracle.gemm_w4a16(act, wd)
    if where == "down":
        want = _bf16_bits(_val(want) + _val(act))
    assert np.array_equal(y, want)
