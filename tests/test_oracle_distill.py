"""Pins of oracle/distill.py: the distillation and TV losses of row pairs,
their gradient with respect to the student logits, and the gated-LoRA
backward.

Source: Uno summary (hyper.ai, arXiv 2609.04010), section 方法, paragraphs
on diffusion distillation (objective alpha * L_DCD + beta * L_TV; teacher
logits from the clean rows with the adapter off, student logits from the
noisy rows with it on; the TV loss lengthens the accepted draft prefix)."""

import numpy as np
import pytest

import oracle


def _rows(rng, r, v, scale=2.0):
    return rng.normal(0, scale, (r, v)), rng.normal(0, scale, (r, v))


def test_two_token_closed_form():
    """q = (1 - a, a), p = (1 - b, b): KL(q || p) is the binary relative
    entropy and TV = |a - b|."""
    for a, b in ((0.3, 0.6), (0.05, 0.9), (0.5, 0.5), (0.999, 0.001)):
        teacher = np.array([[0.0, np.log(b / (1 - b))]])
        student = np.array([[0.0, np.log(a / (1 - a))]])
        o = oracle.distill_losses(teacher, student)
        kl = a * np.log(a / b) + (1 - a) * np.log((1 - a) / (1 - b))
        assert abs(o["kl"][0] - kl) < 1e-12
        assert abs(o["tv"][0] - abs(a - b)) < 1e-12


def test_identical_rows_have_no_loss_and_no_gradient():
    """Equal rows: no loss, no gradient.  A shifted copy is the same
    distribution up to rounding: no loss and no KL gradient (the TV term's
    subgradient there follows the rounding of q - p and is left out)."""
    rng = np.random.default_rng(0)
    t, _ = _rows(rng, 3, 50)
    o = oracle.distill_losses(t, t, temperature=0.8)
    assert not np.any(o["kl"]) and not np.any(o["tv"]) and not np.any(o["grad"])
    o = oracle.distill_losses(t, t + 7.0, temperature=0.8, beta=0.0)
    assert np.max(np.abs(o["kl"])) < 1e-13 and np.max(np.abs(o["tv"])) < 1e-13
    assert np.max(np.abs(o["grad"])) < 1e-13


def test_gradient_by_central_differences():
    """The analytic gradient against central differences of the oracle's own
    loss values (alpha * KL + beta * TV is smooth away from q_v = p_v; the
    rows are drawn so that no |q_v - p_v| is within 1e-4)."""
    rng = np.random.default_rng(1)
    for trial in range(6):
        t, s = _rows(rng, 2, 7)
        T = [1.0, 0.7, 1.6][trial % 3]
        alpha, beta, gs = rng.uniform(0.2, 2.0), rng.uniform(0.0, 2.0), rng.uniform(0.5, 3.0)
        o = oracle.distill_losses(t, s, T, alpha, beta, gs)
        p, q = oracle.softmax_rows(t, T), oracle.softmax_rows(s, T)
        assert np.min(np.abs(q - p)) > 1e-4

        def loss(z):
            r = oracle.distill_losses(t, z, T, alpha, beta)
            return gs * float(np.sum(alpha * r["kl"] + beta * r["tv"]))
        h = 1e-6
        fd = np.zeros_like(s)
        for i in range(s.shape[0]):
            for j in range(s.shape[1]):
                zp, zm = s.copy(), s.copy()
                zp[i, j] += h
                zm[i, j] -= h
                fd[i, j] = (loss(zp) - loss(zm)) / (2 * h)
        np.testing.assert_allclose(o["grad"], fd, rtol=0, atol=2e-7)


def test_against_torch_autograd():
    """torch's own KL divergence and autograd (float64, CPU) as an independent
    implementation of the losses and the gradient."""
    import torch
    import torch.nn.functional as F
    rng = np.random.default_rng(2)
    t, s = _rows(rng, 4, 300)
    T, alpha, beta, gs = 0.9, 0.7, 1.3, 0.25
    o = oracle.distill_losses(t, s, T, alpha, beta, gs)
    tt = torch.tensor(t, dtype=torch.float64)
    st = torch.tensor(s, dtype=torch.float64, requires_grad=True)
    lp = F.log_softmax(tt / T, dim=-1)
    lq = F.log_softmax(st / T, dim=-1)
    kl = F.kl_div(lp, lq, reduction="none", log_target=True).sum(-1)     # KL(q || p)
    tv = 0.5 * (lq.exp() - lp.exp()).abs().sum(-1)
    (gs * (alpha * kl + beta * tv).sum()).backward()
    np.testing.assert_allclose(o["kl"], kl.detach().numpy(), rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(o["tv"], tv.detach().numpy(), rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(o["grad"], st.grad.numpy(), rtol=1e-10, atol=1e-15)


def test_invariants():
    """Shift invariance (the gradient sums to 0 over the vocabulary), Pinsker
    (TV <= sqrt(KL / 2)), and a temperature acting as a logit scale."""
    rng = np.random.default_rng(3)
    t, s = _rows(rng, 8, 40, scale=3.0)
    o = oracle.distill_losses(t, s, 1.0, 1.0, 1.0)
    assert np.max(np.abs(o["grad"].sum(-1))) < 1e-14
    assert np.all(o["tv"] <= np.sqrt(o["kl"] / 2) + 1e-15)
    o2 = oracle.distill_losses(2 * t, 2 * s, 2.0, 1.0, 1.0)
    np.testing.assert_allclose(o2["kl"], o["kl"], rtol=1e-12)
    np.testing.assert_allclose(2 * o2["grad"], o["grad"], rtol=1e-9, atol=1e-15)


def test_tv_is_the_rejection_probability_of_the_verify():
    """1 - TV(q, p) is the probability that the linear verify (k = 1) accepts
    a draft drawn from q: integrated over the draft token and a midpoint grid
    of the accept uniform, through oracle.verify_linear."""
    rng = np.random.default_rng(4)
    V, G = 5, 2000
    t, s = _rows(rng, 1, V, scale=1.2)
    q = oracle.softmax_rows(s[0])
    u = (np.arange(G) + 0.5) / G
    B = V * G
    p_l = np.broadcast_to(np.stack([t[0], t[0]]), (B, 2, V))
    q_l = np.broadcast_to(s[0][None, None], (B, 1, V))
    drafts = np.repeat(np.arange(V), G)[:, None]
    ua = np.tile(u, V)[:, None]
    r = oracle.verify_linear(p_l, q_l, drafts, ua, np.full(B, 0.5))
    acc = (r["accept_len"] == 1).reshape(V, G).mean(axis=1)
    p_acc = float(np.sum(q * acc))
    tv = oracle.distill_losses(t, s)["tv"][0]
    assert abs(p_acc - (1 - tv)) < 1.0 / G


def test_gated_lora_backward_by_differences():
    """Gradients against central differences of the pinned forward
    (oracle.gated_lora_linear) of L = sum(dY * y): y is linear in x, A and B
    separately, so the differences are exact up to rounding."""
    rng = np.random.default_rng(5)
    M, N, K, r = 6, 5, 7, 3
    x, w = rng.normal(size=(M, K)), rng.normal(size=(N, K))
    a, b = rng.normal(size=(r, K)), rng.normal(size=(N, r))
    dy = rng.normal(size=(M, N))
    gate = np.array([0, 1, 1, 0, 1, 0])
    s = 0.75
    o = oracle.gated_lora_backward(x, w, a, b, dy, gate, s)

    def loss(x_, a_, b_):
        return float(np.sum(dy * oracle.gated_lora_linear(x_, w, a_, b_, gate, s)))
    h = 1e-3
    for name, arr in (("dx", x), ("da", a), ("db", b)):
        fd = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            ap, am = arr.copy(), arr.copy()
            ap[idx] += h
            am[idx] -= h
            args_p = {"dx": (ap, a, b), "da": (x, ap, b), "db": (x, a, ap)}[name]
            args_m = {"dx": (am, a, b), "da": (x, am, b), "db": (x, a, am)}[name]
            fd[idx] = (loss(*args_p) - loss(*args_m)) / (2 * h)
        np.testing.assert_allclose(o[name], fd, rtol=0, atol=1e-9, err_msg=name)


def test_gated_lora_backward_against_torch_autograd():
    import torch
    rng = np.random.default_rng(6)
    M, N, K, r = 9, 11, 13, 4
    x, w = rng.normal(size=(M, K)), rng.normal(size=(N, K))
    a, b = rng.normal(size=(r, K)), rng.normal(size=(N, r))
    dy = rng.normal(size=(M, N))
    gate = rng.integers(0, 2, M)
    o = oracle.gated_lora_backward(x, w, a, b, dy, gate, 0.5)
    xt, at, bt = (torch.tensor(v, requires_grad=True) for v in (x, a, b))
    wt = torch.tensor(w)
    g = torch.tensor(gate, dtype=torch.float64)[:, None]
    y = torch.nn.functional.linear(xt, wt) + 0.5 * torch.nn.functional.linear(g * torch.nn.functional.linear(xt, at), bt)
    y.backward(torch.tensor(dy))
    for name, t in (("dx", xt), ("da", at), ("db", bt)):
        np.testing.assert_allclose(o[name], t.grad.numpy(), rtol=1e-12, atol=1e-12, err_msg=name)


def test_gated_lora_backward_special_cases():
    """Every gate 0: no adapter gradient and dx = dY W; B = 0: no gradient
    reaches A."""
    rng = np.random.default_rng(7)
    M, N, K, r = 4, 6, 5, 2
    x, w = rng.normal(size=(M, K)), rng.normal(size=(N, K))
    a, b = rng.normal(size=(r, K)), rng.normal(size=(N, r))
    dy = rng.normal(size=(M, N))
    o = oracle.gated_lora_backward(x, w, a, b, dy, np.zeros(M), 1.0)
    assert not np.any(o["da"]) and not np.any(o["db"])
    np.testing.assert_allclose(o["dx"], dy @ w, rtol=1e-14)
    o = oracle.gated_lora_backward(x, w, a, np.zeros_like(b), dy, np.ones(M), 1.0)
    assert not np.any(o["da"])
