"""Helpers for GPU-vs-oracle parity tests (host side only)."""

import sys

import numpy as np

import oracle

# Accept decisions and inverse-CDF draws are compared bit-exactly except where
# the uniform lies within this distance of the decision boundary (|u - p/q| for
# an accept, the CDF boundary for a draw).  The GPU evaluates probabilities in
# fp32 over up to 2^20 terms (relative error ~1e-6); the band is 10x that.
TIE = 1e-5


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(arr, torch_dtype=None):
    import torch
    arr = np.ascontiguousarray(arr)
    if arr.dtype == np.uint16:
        t = torch.from_numpy(arr.view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(arr)
    if torch_dtype is not None:
        t = t.to(torch_dtype)
    return t.to("cuda")


def to_host(t):
    import torch
    t = t.detach()
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy()
    return t.cpu().numpy()


def row_relerr(got, ref):
    """max over rows of ||got - ref||_inf / ||ref||_inf (rows = all but last axis)."""
    got = np.asarray(got, dtype=np.float64).reshape(-1, np.shape(ref)[-1])
    ref = np.asarray(ref, dtype=np.float64).reshape(-1, np.shape(ref)[-1])
    num = np.max(np.abs(got - ref), axis=1)
    den = np.maximum(np.max(np.abs(ref), axis=1), 1e-300)
    return float(np.max(num / den))


def draw_is_valid(w, u, y, tie=TIE):
    """True if token y is a draw of inverse-CDF(w) at u up to `tie` on the CDF."""
    w = np.asarray(w, dtype=np.float64)
    if y < 0 or y >= len(w) or w[y] <= 0.0:
        return False
    c = np.cumsum(w) / np.sum(w)
    lo = c[y - 1] if y > 0 else 0.0
    return lo - tie <= u <= c[y] + tie


def check_linear(case_rows, gpu, seqs, k, temperature=1.0, tie=TIE, prob_rtol=1e-5, mass_atol=1e-5):
    """Compare GPU linear-verify outputs with the oracle for the listed sequences.

    case_rows(b) -> (p_f32 [k+1, V], q_f32 [k, V], drafts [k], u_acc [k], u_s)
    gpu: dict of host arrays over the whole batch.
    Returns the number of near-tie sequences (accepted, counted).
    """
    ties = 0
    for b in seqs:
        p, q, d, ua, us = case_rows(b)
        o = oracle.verify_linear(p[None], q[None], d[None], ua[None], np.array([us]), temperature)
        Lo, yo = int(o["accept_len"][0]), int(o["token"][0])
        Lg, yg = int(gpu["accept_len"][b]), int(gpu["token"][b])
        if k > 0 and "p_draft" in gpu:
            for name in ("p_draft", "q_draft"):
                ref = o[name][0]
                got = gpu[name][b]
                err = np.max(np.abs(got - ref) / np.maximum(ref, 1e-300))
                assert err <= prob_rtol, f"seq {b} {name} rel err {err:.3g}"
        if Lo != Lg:
            i = min(Lo, Lg)
            ratio = o["p_draft"][0, i] / o["q_draft"][0, i]
            assert abs(float(ua[i]) - ratio) < tie, f"seq {b}: L gpu {Lg} oracle {Lo}, |u - p/q| = {abs(ua[i] - ratio):.3g}"
            ties += 1
            continue
        if "residual_mass" in gpu:
            err = abs(gpu["residual_mass"][b] - o["residual_mass"][0])
            assert err <= mass_atol, f"seq {b} residual mass err {err:.3g}"
        if yg != yo:
            pr = oracle.softmax_rows(p[Lo], temperature)
            if Lo < k:
                w, s = oracle.residual_weights(pr, oracle.softmax_rows(q[Lo], temperature))
                if s == 0.0:
                    w = pr
            else:
                w = pr
            assert draw_is_valid(w, us, yg, tie), f"seq {b}: token gpu {yg} oracle {yo} (L={Lo})"
            ties += 1
    return ties


def tree_outcome_near(parent, tokens, p, q, ua, us, temperature, gpu_out, tie=TIE):
    """True if perturbing one visited uniform (or u_s) by at most `tie` makes
    the oracle produce the GPU's (L, path, y): the GPU differs only on a
    near-tie decision."""
    base = oracle.verify_tree(parent[None], tokens[None], p[None], q[None], ua[None], np.array([us]),
                              temperature, return_visited=True)
    L, path, y = gpu_out

    def same(r):
        Lr = int(r["accept_len"][0])
        return Lr == L and list(r["path"][0, :Lr]) == list(path[:L]) and int(r["token"][0]) == y

    for node, _acc in base["visited"][0]:
        for delta in (-tie, tie):
            u2 = ua.copy()
            u2[node] = min(max(u2[node] + delta, 0.0), 1.0 - 1e-12)
            r = oracle.verify_tree(parent[None], tokens[None], p[None], q[None], u2[None], np.array([us]),
                                   temperature)
            if same(r):
                return True
    for delta in (-tie, tie):
        r = oracle.verify_tree(parent[None], tokens[None], p[None], q[None], ua[None],
                               np.array([min(max(us + delta, 0.0), 1.0 - 1e-12)]), temperature)
        if same(r):
            return True
    return False
