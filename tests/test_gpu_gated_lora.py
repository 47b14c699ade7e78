"""GPU parity: uno_gated_lora_linear against the oracle.

Bar: max over rows of ||y - y_ref||_inf / ||y_ref||_inf <= 2e-2 (bf16) and
<= 1e-5 (fp32); rows with gate 0 bit-identical to the same call without the
adapter.
"""

import numpy as np
import pytest

import oracle
import workloads
from _parity import row_relerr, say, to_dev, to_host

pytestmark = pytest.mark.gpu

LAYER = {   # (N, K) of the per-layer projections of a Qwen3-8B-shaped layer
    "q": (4096, 4096), "k": (1024, 4096), "v": (1024, 4096), "o": (4096, 4096),
    "gate": (12288, 4096), "up": (12288, 4096), "down": (4096, 12288),
}


def _run(dad, c, gate="case", r_off=False, b_zero=False):
    import torch
    dt = None
    x, w, a, b = (to_dev(c[n]) for n in ("x", "w", "a", "b"))
    if b_zero:
        b = torch.zeros_like(b)
    g = to_dev(c["gate"]) if gate == "case" else gate
    if r_off:
        y = dad.gated_lora_linear(x, w, None, None, None)
    else:
        y = dad.gated_lora_linear(x, w, a, b, g)
    torch.cuda.synchronize()
    return y


def _ref(c, rows=None):
    sel = slice(None) if rows is None else rows
    return oracle.gated_lora_linear(c["x_f32"][sel], c["w_f32"], c["a_f32"], c["b_f32"], c["gate"][sel])


def test_tiny_fp32_step(gpu_lib):
    say("gated_lora tiny fp32 8x256x256 r=8")
    c = workloads.tiny_step(0)["lora"]
    y = to_host(_run(gpu_lib, c))
    assert row_relerr(y, _ref(c)) <= 1e-5


@pytest.mark.parametrize("m,n,k,r,dtype", [
    (200, 300, 264, 16, "bf16"),       # ragged M, N and K + r across tiles
    (1, 1, 8, 8, "bf16"),
    (129, 257, 1024, 128, "bf16"),
    (64, 96, 4096, 128, "bf16"),
    (37, 70, 100, 5, "f32"),
    (3, 1000, 2000, 64, "f32"),
])
def test_parity_shapes(gpu_lib, m, n, k, r, dtype):
    say(f"gated_lora {m}x{n}x{k} r={r} {dtype}")
    c = workloads.gated_lora_case(m, n, k, r, dtype=dtype, seed=m + n)
    y = to_host(_run(gpu_lib, c))
    tol = 2e-2 if dtype == "bf16" else 1e-5
    err = row_relerr(y, _ref(c))
    say(f"  row rel err {err:.3g}")
    assert err <= tol


def test_gate_zero_rows_bit_identical_to_no_adapter(gpu_lib):
    say("gated_lora gate-0 rows bit identity")
    import torch
    c = workloads.gated_lora_case(256, 384, 512, 64, dtype="bf16", seed=4)
    y = _run(gpu_lib, c)
    y0 = _run(gpu_lib, c, r_off=True)
    off = torch.from_numpy(c["gate"] == 0).cuda()
    assert torch.equal(y[off].view(torch.int16), y0[off].view(torch.int16))
    assert not torch.equal(y[~off], y0[~off])
    ynone = _run(gpu_lib, c, gate=None)
    assert torch.equal(ynone.view(torch.int16), y0.view(torch.int16))
    yb0 = _run(gpu_lib, c, b_zero=True)
    assert torch.equal(yb0.view(torch.int16), y0.view(torch.int16))


def test_strided_operands(gpu_lib):
    say("gated_lora strided leading dimensions")
    import torch
    c = workloads.gated_lora_case(96, 160, 256, 32, dtype="bf16", seed=8)
    xs = torch.zeros((96, 264), dtype=torch.bfloat16, device="cuda")
    xs[:, :256] = to_dev(c["x"])
    ws = torch.zeros((160, 272), dtype=torch.bfloat16, device="cuda")
    ws[:, :256] = to_dev(c["w"])
    out = torch.zeros((96, 168), dtype=torch.bfloat16, device="cuda")
    gpu_lib.gated_lora_linear(xs[:, :256], ws[:, :256], to_dev(c["a"]), to_dev(c["b"]), to_dev(c["gate"]),
                              out=out[:, :160])
    torch.cuda.synchronize()
    assert row_relerr(to_host(out[:, :160]), _ref(c)) <= 2e-2
    assert torch.all(out[:, 160:] == 0)


@pytest.mark.parametrize("proj", list(LAYER))
def test_layer_projection_full_size_sampled_rows(gpu_lib, proj):
    """1024 rows = 64 sequences x (8 clean + 8 noisy), rank 128, bf16; the
    oracle recomputes 48 sampled rows (both gate values)."""
    n, k = LAYER[proj]
    say(f"gated_lora layer projection {proj}: 1024 x {n} x {k}")
    c = workloads.gated_lora_case(1024, n, k, 128, dtype="bf16", seed=0, tag=list(LAYER).index(proj))
    y = to_host(_run(gpu_lib, c))
    rows = np.sort(np.random.default_rng(2).choice(1024, 48, replace=False))
    assert set(c["gate"][rows].tolist()) == {0, 1}
    err = row_relerr(y[rows], _ref(c, rows))
    say(f"  row rel err {err:.3g}")
    assert err <= 2e-2
    assert np.all(np.isfinite(y))


@pytest.mark.parametrize("m,k,r", [(4096, 4096, 256), (4096, 4096, 384), (2072, 1032, 384)])
def test_grouped_adapter_ranks_at_decode_rows(gpu_lib, m, k, r):
    """4096 rows (128 sequences x (16 clean + 16 noisy)) with the adapter ranks
    of the grouped LoRA-down launches (gate|up: 2 x 128, q|k|v: 3 x 128), which
    take the one-tile-wide LoRA-down kernels, plus a ragged case (a partial
    last row tile and a partial last K-tile); 48 sampled rows against the
    oracle."""
    say(f"gated_lora grouped rank {r}: {m} x 1024 x {k}")
    c = workloads.gated_lora_case(m, 1024, k, r, dtype="bf16", seed=3, tag=r + k,
                                  gate=workloads.default_gate(m, 4 if m % 32 else 16))
    y = to_host(_run(gpu_lib, c))
    rows = np.sort(np.concatenate([np.random.default_rng(5).choice(m - 8, 40, replace=False),
                                   np.arange(m - 8, m)]))
    assert set(c["gate"][rows].tolist()) == {0, 1}
    err = row_relerr(y[rows], _ref(c, rows))
    say(f"  row rel err {err:.3g}")
    assert err <= 2e-2
    assert np.all(np.isfinite(y))


@pytest.mark.parametrize("n,k,r,scale", [
    (300, 1001, 8, 0.5),      # odd K: the element-wise path
    (256, 4096, 128, 1.0),    # a projection's shape class: 16-byte path
    (64, 12288, 128, 1.0),    # the down projection's K
])
def test_lora_merge_matches_oracle(gpu_lib, n, k, r, scale):
    """uno_lora_merge against oracle.merged_weight (W + s B A in float64) on the
    same bf16 operands: the bf16 result equals the round-to-nearest-even of the
    exact value except where the fp32 sum lands on the other side of a rounding
    tie, and is within one bf16 step of it everywhere."""
    import torch
    say(f"lora merge N={n} K={k} r={r} s={scale}")
    c = workloads.gated_lora_case(4, n, k, r, dtype="bf16", seed=n + k, weight_std=0.05)
    out = gpu_lib.lora_merge(to_dev(c["w"]), to_dev(c["a"]), to_dev(c["b"]), scale)
    torch.cuda.synchronize()
    got = to_host(out).astype(np.float64)          # bf16 values, widened exactly
    ref = oracle.merged_weight(c["w_f32"], c["a_f32"], c["b_f32"], scale)
    exact = workloads.bf16_to_f32(workloads.bf16_bits(ref)).astype(np.float64)
    # one bf16 step of the result, plus the fp32 rounding of the r products,
    # their sum and the final add (bounded through the operand magnitudes; it
    # dominates only where W and s B A nearly cancel)
    mag = np.abs(c["w_f32"]).astype(np.float64) + abs(scale) * (np.abs(c["b_f32"]) @ np.abs(c["a_f32"]))
    bound = np.abs(exact) * 2.0 ** -7 + mag * (r + 2) * 2.0 ** -24
    excess = np.abs(got - exact) - bound
    say(f"  worst excess over the bound {excess.max():.3g}")
    assert np.all(excess <= 0)
    frac = np.mean(got == exact)
    say(f"  equal to the rounded exact value: {frac:.6f}")
    assert frac >= 0.999
