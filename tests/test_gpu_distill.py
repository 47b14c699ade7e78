"""GPU parity of the distillation losses (uno_distill_loss) against
oracle.distill_losses.

Source: Uno summary (hyper.ai, arXiv 2609.04010), section 方法, paragraphs
on diffusion distillation (alpha * L_DCD + beta * L_TV over the teacher
(clean) and student (noisy) rows of the gated forward).

Bar (fp32 arithmetic over up to 2^20 terms, relative rounding ~1e-6 per
term, 10x margin): KL within 1e-5 * (sum_v q_v |ln q_v - ln p_v| + |KL|) +
1e-7; TV within 1e-5; every gradient entry within
  grad_scale / T * q_v * 2e-5 * (alpha (|ln q_v - ln p_v| + |KL| + 1) + beta)
plus, for tokens whose |q_v - p_v| is within 1e-5 of q_v (where the sign of
q - p may go either way in fp32), beta / 2 * their q mass (the TV
subgradient), plus the bf16 rounding of the stored gradient (2^-8 of it)."""

import numpy as np
import pytest

import oracle
import workloads
from _parity import say, to_dev, to_host

pytestmark = pytest.mark.gpu

FULL_V = 151936


def _logits(batch, rows, vocab, dtype, seed, sigma):
    """Teacher rows ~ N(0, 2^2); student rows = teacher + N(0, sigma^2)
    (a draft head near its AR model), stored in dtype."""
    rng = np.random.default_rng(seed)
    t = rng.normal(0, 2.0, (batch, rows, vocab)).astype(np.float32)
    s = (t + rng.normal(0, sigma, (batch, rows, vocab))).astype(np.float32)
    if dtype == "bf16":
        return workloads.bf16_bits(t), workloads.bf16_bits(s), workloads.round_bf16(t), workloads.round_bf16(s)
    return t, s, t, s


def _check(t32, s32, gpu, T, alpha, beta, gs, bf16_grad):
    t64 = np.asarray(t32, np.float64).reshape(-1, t32.shape[-1])
    s64 = np.asarray(s32, np.float64).reshape(-1, s32.shape[-1])
    o = oracle.distill_losses(t64, s64, T, alpha, beta, gs)
    lq, lp = oracle.log_softmax_rows(s64, T), oracle.log_softmax_rows(t64, T)
    q, p = np.exp(lq), np.exp(lp)
    dln = np.abs(lq - lp)
    kl_g = gpu["kl"].reshape(-1)
    tv_g = gpu["tv"].reshape(-1)
    scale = np.sum(q * dln, axis=-1) + np.abs(o["kl"])
    assert np.all(np.abs(kl_g - o["kl"]) <= 1e-5 * scale + 1e-7), np.max(np.abs(kl_g - o["kl"]) / (scale + 1e-7))
    assert np.max(np.abs(tv_g - o["tv"])) <= 1e-5
    if "grad" not in gpu:
        return
    g = gpu["grad"].reshape(t64.shape).astype(np.float64)
    ref = o["grad"]
    c = gs / T
    tol = c * q * 2e-5 * (alpha * (dln + np.abs(o["kl"])[:, None] + 1.0) + beta)
    near = np.abs(q - p) <= 1e-5 * q
    tol += c * beta * q * near + c * beta * q * np.sum(q * near, axis=-1, keepdims=True)
    if bf16_grad:
        tol += 2.0 ** -8 * np.abs(ref) + 1e-38
    bad = np.abs(g - ref) > tol
    assert not np.any(bad), f"{int(bad.sum())} gradient entries off; worst {np.max((np.abs(g - ref) - tol))}"


@pytest.mark.parametrize("batch,rows,vocab,dtype,T,alpha,beta,gs,sigma", [
    (2, 3, 1000, "f32", 1.0, 1.0, 1.0, 1.0, 0.5),
    (3, 4, 8193, "bf16", 0.7, 0.5, 2.0, 0.25, 1.0),     # ragged tail
    (1, 2, 7, "f32", 1.3, 1.0, 0.0, 1.0, 2.0),           # fewer tokens than one thread's group
    (2, 5, 40000, "f32", 1.0, 0.0, 1.0, 1.0, 0.3),       # TV only
    (4, 16, FULL_V, "bf16", 1.0, 1.0, 1.0, 1.0 / 64, 0.5),
    (1, 3, FULL_V, "f32", 0.8, 1.0, 0.5, 1.0, 2.0),
])
def test_distill_matches_oracle(gpu_lib, batch, rows, vocab, dtype, T, alpha, beta, gs, sigma):
    import torch
    say(f"distill {batch}x{rows} V={vocab} {dtype} T={T} a={alpha} b={beta}")
    t, s, t32, s32 = _logits(batch, rows, vocab, dtype, seed=vocab + rows, sigma=sigma)
    out = gpu_lib.distill_loss(to_dev(t), to_dev(s), T, alpha, beta, gs)
    torch.cuda.synchronize()
    gpu = {k: to_host(v) for k, v in out.items()}
    _check(t32, s32, gpu, T, alpha, beta, gs, dtype == "bf16")


def test_distill_losses_only_and_degenerate_rows(gpu_lib):
    """No gradient buffer: losses only.  One-token rows and equal rows: no
    loss and (equal rows) no gradient."""
    import torch
    t, s, t32, s32 = _logits(2, 2, 3000, "f32", seed=1, sigma=1.0)
    out = gpu_lib.distill_loss(to_dev(t), to_dev(s), want_grad=False)
    torch.cuda.synchronize()
    assert "grad" not in out
    _check(t32, s32, {k: to_host(v) for k, v in out.items()}, 1.0, 1.0, 1.0, 1.0, False)
    one = np.array([[[3.0]], [[-2.0]]], np.float32)
    out = gpu_lib.distill_loss(to_dev(one), to_dev(one[::-1].copy()))
    torch.cuda.synchronize()
    assert np.all(to_host(out["kl"]) == 0) and np.all(to_host(out["tv"]) == 0) and np.all(to_host(out["grad"]) == 0)
    out = gpu_lib.distill_loss(to_dev(t), to_dev(t))
    torch.cuda.synchronize()
    assert np.all(to_host(out["kl"]) == 0) and np.all(to_host(out["tv"]) == 0)
    assert np.all(to_host(out["grad"]) == 0)


def test_distill_on_a_step_logits_buffer(gpu_lib):
    """The teacher and student rows passed in place as the clean and noisy
    halves of a step's logits [B, 2*block, V] (bf16), the gradient written
    into the noisy half of a same-shaped buffer."""
    import torch
    B, block, V = 3, 8, 20000
    t, s, t32, s32 = _logits(B, block, V, "bf16", seed=5, sigma=0.7)
    full = np.concatenate([t, s], axis=1)
    dev = to_dev(full)
    gbuf = torch.zeros((B, 2 * block, V), dtype=torch.bfloat16, device="cuda")
    outputs = {"kl": torch.empty((B, block), dtype=torch.float32, device="cuda"),
               "tv": torch.empty((B, block), dtype=torch.float32, device="cuda"),
               "grad": gbuf[:, block:]}
    gpu_lib.distill_loss(dev[:, :block], dev[:, block:], outputs=outputs)
    torch.cuda.synchronize()
    assert not torch.any(gbuf[:, :block] != 0)          # the clean half is not touched
    gpu = {"kl": to_host(outputs["kl"]), "tv": to_host(outputs["tv"]), "grad": to_host(gbuf[:, block:])}
    _check(t32, s32, gpu, 1.0, 1.0, 1.0, 1.0, True)


def test_distill_is_deterministic(gpu_lib):
    import torch
    t, s, _, _ = _logits(4, 4, FULL_V, "bf16", seed=8, sigma=0.5)
    td, sd = to_dev(t), to_dev(s)
    a = gpu_lib.distill_loss(td, sd)
    b = gpu_lib.distill_loss(td, sd)
    torch.cuda.synchronize()
    for k in a:
        assert torch.equal(a[k].view(torch.int16) if a[k].dtype == torch.bfloat16 else a[k],
                           b[k].view(torch.int16) if b[k].dtype == torch.bfloat16 else b[k])
