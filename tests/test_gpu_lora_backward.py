"""GPU parity of the gated-LoRA backward (uno_gated_lora_backward) against
oracle.gated_lora_backward.

Source: Uno summary (hyper.ai, arXiv 2609.04010), section 方法 (adapters on
every AR weight matrix, trained by distillation with the AR weights frozen;
the adapter masked off on clean rows of the concatenated forward).

Bar: every row of dx, dA and dB within 2e-2 of its own max-norm
(max_row ||got - ref||_inf / ||ref||_inf), the library's bf16 bar.  The
inputs are exact bf16 values; the error is the bf16 rounding of U and dT
between the products and of dx on output (2^-9 relative each), summed over
random-signed terms: an fp64 emulation of exactly that rounding stays below
6e-3 on these cases.  The adapter terms are scaled (A, B ~ N(0, 0.05^2)) so
that leaving the adapter out of dx, or inverting the gate, moves the result
by well over the bar (asserted on the CPU side for every case)."""

import numpy as np
import pytest

import oracle
import workloads
from _parity import row_relerr, say, to_dev, to_host

pytestmark = pytest.mark.gpu

BAR = 2e-2


def _run(dad, c, gate, scale, want_dx=True, with_wt=False):
    import torch
    g = to_dev(gate) if gate is not None else None
    w = to_dev(c["w"])
    wt = dad.transpose_bf16(w) if with_wt else None
    out = dad.gated_lora_backward(to_dev(c["x"]), w, to_dev(c["a"]), to_dev(c["b"]), g, to_dev(c["dy"]),
                                  scale, want_dx=want_dx, w_t=wt)
    torch.cuda.synchronize()
    return {k: to_host(v) for k, v in out.items()}


def _check(c, gate, scale, got):
    ref = oracle.gated_lora_backward(c["x_f32"], c["w_f32"], c["a_f32"], c["b_f32"], c["dy_f32"], gate, scale)
    errs = {k: row_relerr(got[k], ref[k]) for k in got}
    say("  rel err " + ", ".join(f"{k} {v:.2e}" for k, v in errs.items()))
    for k, v in errs.items():
        assert v <= BAR, f"{k}: {v:.3g}"
    if gate is not None and np.any(gate):
        # power: the adapter's share of dx and one gated row's share of dB
        no_adapter = c["dy_f32"].astype(np.float64) @ c["w_f32"].astype(np.float64)
        if "dx" in got:
            assert row_relerr(no_adapter, ref["dx"]) > 3 * BAR
        inv = (gate == 0).astype(np.uint8)
        ref2 = oracle.gated_lora_backward(c["x_f32"], c["w_f32"], c["a_f32"], c["b_f32"], c["dy_f32"], inv, scale)
        assert min(row_relerr(ref2["db"], ref["db"]), row_relerr(ref2["da"], ref["da"])) > 3 * BAR
    return ref


@pytest.mark.parametrize("with_wt", [False, True])
@pytest.mark.parametrize("m,n,k,r,gate_kind,scale", [
    (40, 64, 72, 8, "alt", 1.0),          # one partial tile everywhere
    (300, 256, 136, 24, "blocks", 0.5),   # ragged M and K tiles, structured gate
    (512, 384, 520, 40, "random", 2.0),
    (130, 96, 264, 16, "blocks", 1.0),
])
def test_backward_matches_oracle(gpu_lib, m, n, k, r, gate_kind, scale, with_wt):
    say(f"lora backward M={m} N={n} K={k} r={r} gate={gate_kind} w_t={with_wt}")
    rng = np.random.default_rng(m + n)
    gate = {"alt": (np.arange(m) % 2).astype(np.uint8),
            "blocks": workloads.default_gate(m),
            "random": rng.integers(0, 2, m).astype(np.uint8)}[gate_kind]
    c = workloads.lora_backward_case(m, n, k, r, seed=m + k, gate=gate)
    got = _run(gpu_lib, c, gate, scale, with_wt=with_wt)
    _check(c, gate, scale, got)


@pytest.mark.parametrize("with_wt", [False, True])
def test_backward_layer_shape(gpu_lib, with_wt):
    """The q projection of the 1024-row layer workload: M = 1024 (64
    sequences x 8 clean + 8 noisy rows), N = K = 4096, r = 128."""
    say("lora backward M=1024 N=K=4096 r=128")
    c = workloads.lora_backward_case(1024, 4096, 4096, 128, seed=3)
    got = _run(gpu_lib, c, c["gate"], 1.0, with_wt=with_wt)
    _check(c, c["gate"], 1.0, got)


def test_backward_without_gate_and_without_dx(gpu_lib):
    """No gate: every row clean, no adapter gradient, dx = dY W.  No dx:
    the adapter gradients alone."""
    c = workloads.lora_backward_case(96, 128, 64, 16, seed=5)
    got = _run(gpu_lib, c, None, 1.0)
    assert not np.any(got["da"]) and not np.any(got["db"])
    _check(c, None, 1.0, got)
    got = _run(gpu_lib, c, c["gate"], 1.0, want_dx=False)
    assert "dx" not in got
    _check(c, c["gate"], 1.0, got)


def test_backward_is_deterministic(gpu_lib):
    c = workloads.lora_backward_case(256, 512, 384, 32, seed=6)
    for with_wt in (False, True):
        a = _run(gpu_lib, c, c["gate"], 1.0, with_wt=with_wt)
        b = _run(gpu_lib, c, c["gate"], 1.0, with_wt=with_wt)
        for key in a:
            assert np.array_equal(a[key], b[key])


@pytest.mark.parametrize("rows,cols", [(1, 1), (64, 64), (100, 37), (4096, 130), (129, 4100)])
def test_transpose_is_exact(gpu_lib, rows, cols):
    import torch
    x = np.random.default_rng(rows + cols).normal(size=(rows, cols)).astype(np.float32)
    bits = workloads.bf16_bits(x)
    out = gpu_lib.transpose_bf16(to_dev(bits))
    torch.cuda.synchronize()
    got = out.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got, bits.T)
