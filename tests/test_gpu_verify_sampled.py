"""GPU parity: uno_psi_spec_verify_linear_sampled (the linear verify under
top-k, top-p and greedy) against oracle.verify_linear with the same
transform.

Bar: accepted lengths and tokens bit-exact except near-ties (|u - p~/q~| <
1e-5, a draw within 1e-5 of a CDF boundary, or a row whose top-p boundary
lies within 1e-6 of deciding the other way), which are counted; transformed
draft probabilities within 1e-5 relative (so the kept sets match exactly:
a token the oracle drops must be 0 on the GPU); residual mass within 1e-5.
"""

import numpy as np
import pytest

import oracle
import workloads
from _parity import check_linear_sampled, say, to_dev, to_host

pytestmark = pytest.mark.gpu


def _case(batch, k, vocab, sigma, dtype, seed, T, top_k, top_p, greedy, integer_logits=False, eighths=False):
    """Logits of the linear-verify workload (or small integers, for many ties;
    or the workload's logits rounded to multiples of 1/8, for a few ties at
    the top); drafts drawn from the transformed draft rows."""
    c = workloads.verify_linear_case(batch, k, vocab, sigma, dtype=dtype, seed=seed, workers=4)
    if eighths:
        pv = (np.round(c["p_f32"] * 8.0) / 8.0).astype(np.float32)     # exact in bf16 below 32
        qv = (np.round(c["q_f32"] * 8.0) / 8.0).astype(np.float32)
        if dtype == "bf16":
            c["p"], c["q"] = workloads.bf16_bits(pv), workloads.bf16_bits(qv)
        else:
            c["p"], c["q"] = pv, qv
        c["p_f32"], c["q_f32"] = pv, qv
    if integer_logits:
        rng = workloads.rng_for(seed, 77)
        pv = rng.integers(-6, 4, (batch, k + 1, vocab)).astype(np.float32)
        qv = (pv[:, :k] + rng.integers(-1, 2, (batch, k, vocab))).astype(np.float32)
        if dtype == "bf16":
            c["p"], c["q"] = workloads.bf16_bits(pv), workloads.bf16_bits(qv)
        else:
            c["p"], c["q"] = pv, qv
        c["p_f32"], c["q_f32"] = pv, qv
    rng = workloads.rng_for(seed, 78)
    drafts = np.zeros((batch, k), np.int32)
    for b in range(batch):
        for i in range(k):
            qt = oracle.transform_probs(c["q_f32"][b, i], T, top_k, top_p, greedy)
            drafts[b, i] = oracle.inverse_cdf(qt, rng.random())
    c["drafts"] = drafts
    return c


CASES = [
    # batch, k, vocab, sigma, dtype, T, top_k, top_p, greedy
    (4, 5, 1000, 0.5, "f32", 1.0, 10, 1.0, False),
    (4, 5, 1000, 0.5, "bf16", 0.8, 50, 1.0, False),
    (3, 4, 20000, 0.5, "bf16", 1.0, 0, 0.9, False),
    (3, 4, 20000, 0.3, "f32", 1.3, 0, 0.5, False),
    (3, 6, 5000, 0.5, "bf16", 1.0, 100, 0.8, False),
    (4, 6, 3000, 0.5, "bf16", 1.0, 0, 1.0, True),
    (3, 3, 4099, 1.0, "f32", 1.0, 1, 1.0, False),     # top-1 without ties: greedy by another road
    (2, 3, 151936, 0.5, "bf16", 1.0, 50, 0.95, False),
]


@pytest.mark.parametrize("batch,k,vocab,sigma,dtype,T,top_k,top_p,greedy", CASES)
def test_sampled_verify_parity(gpu_lib, batch, k, vocab, sigma, dtype, T, top_k, top_p, greedy):
    import torch
    say(f"sampled verify B={batch} k={k} V={vocab} {dtype} T={T} top_k={top_k} top_p={top_p} greedy={greedy}")
    c = _case(batch, k, vocab, sigma, dtype, batch * 13 + k + vocab % 97, T, top_k, top_p, greedy)
    out = gpu_lib.psi_spec_verify_linear_sampled(to_dev(c["p"]), to_dev(c["q"]), to_dev(c["drafts"]),
                                                 to_dev(c["u_acc"]), to_dev(c["u_s"]), T, top_k, top_p, greedy)
    torch.cuda.synchronize()
    g = {kk: to_host(v) for kk, v in out.items()}

    def rows(b):
        return c["p_f32"][b], c["q_f32"][b], c["drafts"][b], c["u_acc"][b], float(c["u_s"][b])

    ties = check_linear_sampled(rows, g, range(batch), k, T, top_k, top_p, greedy)
    say(f"  L {g['accept_len'].tolist()}, ties {ties}")
    assert ties <= 1


@pytest.mark.parametrize("dtype,top_k,top_p", [("bf16", 7, 1.0), ("f32", 0, 0.6), ("bf16", 20, 0.7)])
def test_sampled_verify_tie_groups(gpu_lib, dtype, top_k, top_p):
    """Small integer logits: most values repeat, so every boundary cuts through
    a tie group, which the transform keeps whole."""
    import torch
    say(f"sampled verify, integer logits {dtype} top_k={top_k} top_p={top_p}")
    c = _case(4, 4, 3001, 0.5, dtype, 5, 1.0, top_k, top_p, False, integer_logits=True)
    out = gpu_lib.psi_spec_verify_linear_sampled(to_dev(c["p"]), to_dev(c["q"]), to_dev(c["drafts"]),
                                                 to_dev(c["u_acc"]), to_dev(c["u_s"]), 1.0, top_k, top_p, False)
    torch.cuda.synchronize()
    g = {kk: to_host(v) for kk, v in out.items()}

    def rows(b):
        return c["p_f32"][b], c["q_f32"][b], c["drafts"][b], c["u_acc"][b], float(c["u_s"][b])

    assert check_linear_sampled(rows, g, range(4), 4, 1.0, top_k, top_p, False) <= 1


@pytest.mark.parametrize("dtype,top_k,top_p,eighths", [("bf16", 50, 1.0, True), ("bf16", 50, 0.9, True),
                                                       ("f32", 64, 0.8, True), ("f32", 1024, 1.0, False),
                                                       ("bf16", 1025, 0.95, False)])
def test_sampled_verify_topk_candidate_edges(gpu_lib, dtype, top_k, top_p, eighths):
    """Top-k's two roads: the candidate keys gathered above the k-th largest of
    the threads' maxima (with a few ties at the boundary when the logits are
    multiples of 1/8; top-p then resolved among the candidates), k = 1024
    (the largest k that road takes) and k = 1025 (the radix descent)."""
    import torch
    say(f"sampled verify, candidate edges {dtype} top_k={top_k} top_p={top_p} eighths={eighths}")
    c = _case(3, 4, 20000, 0.5, dtype, 31 + top_k, 1.0, top_k, top_p, False, eighths=eighths)
    out = gpu_lib.psi_spec_verify_linear_sampled(to_dev(c["p"]), to_dev(c["q"]), to_dev(c["drafts"]),
                                                 to_dev(c["u_acc"]), to_dev(c["u_s"]), 1.0, top_k, top_p, False)
    torch.cuda.synchronize()
    g = {kk: to_host(v) for kk, v in out.items()}

    def rows(b):
        return c["p_f32"][b], c["q_f32"][b], c["drafts"][b], c["u_acc"][b], float(c["u_s"][b])

    assert check_linear_sampled(rows, g, range(3), 4, 1.0, top_k, top_p, False) <= 1
    if eighths:   # the boundary of some row falls inside a tie group: the cut keeps it whole
        tied = 0
        for b in range(3):
            for r in c["p_f32"][b]:
                kth = np.sort(r)[::-1][top_k - 1]
                tied += int(np.sum(r == kth) > 1)
        assert tied > 0


def test_sampled_verify_off_matches_plain_verify(gpu_lib):
    """top_k = 0, top_p = 1, greedy off: the same decisions as the plain verify."""
    import torch
    c = workloads.verify_linear_case(6, 5, 5000, 0.5, dtype="bf16", seed=9, workers=4)
    args = [to_dev(c[n]) for n in ("p", "q", "drafts", "u_acc", "u_s")]
    a = gpu_lib.psi_spec_verify_linear_sampled(*args, 1.0, 0, 1.0, False)
    b = gpu_lib.psi_spec_verify_linear(*args, 1.0)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_host(a["accept_len"]), to_host(b["accept_len"]))
    np.testing.assert_array_equal(to_host(a["token"]), to_host(b["token"]))
    np.testing.assert_allclose(to_host(a["p_draft"]), to_host(b["p_draft"]), rtol=1e-5)
