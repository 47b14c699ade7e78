"""Pins of the gated-LoRA oracle (Uno summary, section 方法: LoRA on every AR
weight matrix; a per-position mask turns the adapter off on clean rows and on
on noisy rows in one concatenated forward)."""

import itertools
import math

import numpy as np
import pytest

import oracle
import workloads

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _brute(x, w, a, b, g, s):
    """Pure-Python loops, math.fsum accumulation."""
    m, k = x.shape
    n, r = b.shape
    y = np.zeros((m, n))
    for i in range(m):
        t = [math.fsum(float(x[i, kk]) * float(a[j, kk]) for kk in range(k)) for j in range(r)]
        for o in range(n):
            base = math.fsum(float(x[i, kk]) * float(w[o, kk]) for kk in range(k))
            lora = math.fsum(t[j] * float(b[o, j]) for j in range(r))
            y[i, o] = base + s * float(g[i]) * lora
    return y


@pytest.mark.parametrize("gate", list(itertools.product([0, 1], repeat=3)))
def test_bruteforce_every_gate_pattern(gate):
    rng = np.random.default_rng(7)
    m, n, k, r = 3, 5, 4, 2          # non-square everywhere: transposes would fail
    x = rng.normal(size=(m, k))
    w = rng.normal(size=(n, k))
    a = rng.normal(size=(r, k))
    b = rng.normal(size=(n, r))
    g = np.array(gate, dtype=np.uint8)
    got = oracle.gated_lora_linear(x, w, a, b, g, lora_scale=0.75)
    np.testing.assert_allclose(got, _brute(x, w, a, b, g, 0.75), rtol=1e-13, atol=1e-13)


def test_gate_off_or_b_zero_is_base_matmul():
    c = workloads.gated_lora_case(16, 48, 40, 8, dtype="bf16", seed=3)
    x, w, a, b = c["x_f32"], c["w_f32"], c["a_f32"], c["b_f32"]
    y0 = oracle.gated_lora_linear(x, w, a, b, np.zeros(16, np.uint8))
    ynone = oracle.gated_lora_linear(x, w, a, b, None)
    ybz = oracle.gated_lora_linear(x, w, a, np.zeros_like(b), np.ones(16, np.uint8))
    base = _brute(x, w, a, np.zeros_like(b), np.zeros(16), 0.0)
    np.testing.assert_allclose(y0, base, rtol=1e-12, atol=1e-12)
    np.testing.assert_array_equal(y0, ynone)
    np.testing.assert_allclose(ybz, base, rtol=1e-12, atol=1e-12)


def test_gate_on_is_merged_weight():
    """g = 1: X W^T + X A^T B^T == X (W + B A)^T (LoRA merge identity)."""
    c = workloads.gated_lora_case(12, 36, 28, 6, dtype="f32", seed=5)
    x, w, a, b = (c[k].astype(np.float64) for k in ("x_f32", "w_f32", "a_f32", "b_f32"))
    y1 = oracle.gated_lora_linear(x, w, a, b, np.ones(12, np.uint8))
    merged = w + b @ a
    ref = np.array([[math.fsum(x[i] * merged[o]) for o in range(36)] for i in range(12)])
    np.testing.assert_allclose(y1, ref, rtol=1e-11, atol=1e-12)


def test_merged_weight_bruteforce_and_gate_on_rows():
    """merged_weight against an element-by-element fsum of W + s sum_j B A, and
    a gated row of gated_lora_linear equals that row times the merged weight."""
    c = workloads.gated_lora_case(5, 9, 11, 4, dtype="f32", seed=8)
    x, w, a, b = (c[k].astype(np.float64) for k in ("x_f32", "w_f32", "a_f32", "b_f32"))
    s = 0.75
    m = oracle.merged_weight(w, a, b, s)
    brute = np.array([[math.fsum([w[n, k]] + [s * b[n, j] * a[j, k] for j in range(4)]) for k in range(11)]
                      for n in range(9)])
    np.testing.assert_allclose(m, brute, rtol=1e-13, atol=1e-14)
    g = np.array([1, 0, 1, 1, 0], np.uint8)
    y = oracle.gated_lora_linear(x, w, a, b, g, lora_scale=s)
    on = np.array([[math.fsum(x[i] * m[o]) for o in range(9)] for i in range(5)])
    off = np.array([[math.fsum(x[i] * w[o]) for o in range(9)] for i in range(5)])
    np.testing.assert_allclose(y[g == 1], on[g == 1], rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(y[g == 0], off[g == 0], rtol=1e-11, atol=1e-12)


def test_rows_gated_independently_and_low_rank():
    c = workloads.gated_lora_case(32, 64, 48, 4, dtype="f32", seed=9)
    x, w, a, b = c["x_f32"], c["w_f32"], c["a_f32"], c["b_f32"]
    g = workloads.default_gate(32)
    y = oracle.gated_lora_linear(x, w, a, b, g)
    y0 = oracle.gated_lora_linear(x, w, a, b, np.zeros(32, np.uint8))
    y1 = oracle.gated_lora_linear(x, w, a, b, np.ones(32, np.uint8))
    on = g.astype(bool)
    np.testing.assert_array_equal(y[~on], y0[~on])
    np.testing.assert_allclose(y[on], y1[on], rtol=1e-13, atol=1e-15)
    sv = np.linalg.svd(y1 - y0, compute_uv=False)
    assert np.sum(sv > 1e-9 * sv[0]) <= 4        # rank(delta) <= r


def test_lora_scale_is_linear():
    c = workloads.gated_lora_case(8, 16, 24, 4, dtype="f32", seed=1)
    args = (c["x_f32"], c["w_f32"], c["a_f32"], c["b_f32"], np.ones(8, np.uint8))
    y0 = oracle.gated_lora_linear(*args, lora_scale=0.0)
    y1 = oracle.gated_lora_linear(*args, lora_scale=1.0)
    y3 = oracle.gated_lora_linear(*args, lora_scale=3.0)
    np.testing.assert_allclose(y3 - y0, 3.0 * (y1 - y0), rtol=1e-11, atol=1e-14)
