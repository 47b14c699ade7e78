"""GPU parity: uno_psi_spec_verify_linear against the oracle.

Bar: accepted lengths and tokens bit-exact except near-ties (|u - p/q| < 1e-5,
or a draw within 1e-5 of a CDF boundary), which are counted; probabilities of
the drafts within 1e-5 relative (fp32 outputs); residual mass within 1e-5
absolute (a sum of at most 2^20 fp32 probability differences).
"""

import json
import os

import numpy as np
import pytest

import oracle
import workloads
from _parity import TIE, check_linear, draw_is_valid, say, to_dev, to_host

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "verify_linear_handworked.json")

pytestmark = pytest.mark.gpu


def _run(dad, c, temperature=None, q_override=None):
    import torch
    t = c["temperature"] if temperature is None else temperature
    p = to_dev(c["p"])
    q = to_dev(c["q"]) if q_override is None else q_override
    out = dad.psi_spec_verify_linear(p, q, to_dev(c["drafts"]), to_dev(c["u_acc"]), to_dev(c["u_s"]), t)
    torch.cuda.synchronize()
    return {kk: to_host(v) for kk, v in out.items()}, p


def _rows(c):
    def f(b):
        return c["p_f32"][b], c["q_f32"][b], c["drafts"][b], c["u_acc"][b], float(c["u_s"][b])
    return f


@pytest.mark.parametrize("batch,k,vocab,sigma,dtype", [
    (2, 3, 1024, 0.5, "f32"),          # the tiny fp32 step
    (8, 5, 20000, 0.5, "bf16"),        # several 8192-element tiles + ragged tail
    (4, 7, 20000, 0.1, "f32"),
    (3, 64, 3000, 0.05, "bf16"),       # maximum k
    (5, 0, 4099, 1.0, "bf16"),         # k = 0: bonus draw only
    (6, 4, 1001, 1.0, "bf16"),         # odd vocab: rows not 16-byte aligned
    (4, 2, 7, 1.0, "f32"),             # vocab smaller than one vector
    (3, 2, 1, 1.0, "bf16"),            # vocab 1
    (1, 15, 151936, 2.0, "bf16"),      # one sequence at the full vocabulary
])
def test_parity_small(gpu_lib, batch, k, vocab, sigma, dtype):
    say(f"verify_linear small batch={batch} k={k} V={vocab} sigma={sigma} {dtype}")
    c = workloads.verify_linear_case(batch, k, vocab, sigma, dtype=dtype, seed=batch * 7 + k, workers=4)
    g, _ = _run(gpu_lib, c)
    ties = check_linear(_rows(c), g, range(batch), k)
    assert ties <= max(1, batch // 50)


@pytest.mark.parametrize("temperature", [0.7, 1.6])
def test_parity_temperature(gpu_lib, temperature):
    say(f"verify_linear temperature={temperature}")
    c = workloads.verify_linear_case(6, 6, 5000, 0.5, dtype="bf16", seed=31, temperature=temperature, workers=4)
    g, _ = _run(gpu_lib, c)
    assert check_linear(_rows(c), g, range(6), 6, temperature=temperature) <= 1


def test_identical_draft_accepts_all_and_determinism(gpu_lib):
    say("verify_linear q = p, determinism")
    import torch
    c = workloads.verify_linear_case(16, 7, 9000, 0.5, dtype="bf16", seed=5, workers=4)
    p = to_dev(c["p"])
    qsame = p[:, :7]                      # strided view: q rows are the p rows themselves
    out = gpu_lib.psi_spec_verify_linear(p, qsame, to_dev(c["drafts"]), to_dev(c["u_acc"]),
                                         to_dev(c["u_s"]))
    torch.cuda.synchronize()
    assert np.all(to_host(out["accept_len"]) == 7)
    g1, _ = _run(gpu_lib, c)
    g2, _ = _run(gpu_lib, c)
    for kk in g1:
        np.testing.assert_array_equal(g1[kk], g2[kk])


@pytest.mark.parametrize("sigma", [0.1, 0.5, 2.0])
def test_parity_full_vocab_batch(gpu_lib, sigma):
    """The sampler workload at batch 256 x block 16 (k = 15), vocab 151,936,
    bf16, checked on sampled sequences (the oracle recomputes each one)."""
    batch = 256
    say(f"verify_linear full V sigma={sigma} batch={batch}: generating")
    c = workloads.verify_linear_case(batch, 15, 151936, sigma, dtype="bf16", seed=0, keep_f32=False)
    say("  running on GPU")
    g, _ = _run(gpu_lib, c)
    assert np.all((g["accept_len"] >= 0) & (g["accept_len"] <= 15))
    assert np.all((g["token"] >= 0) & (g["token"] < 151936))
    rng = np.random.default_rng(1)
    seqs = sorted(set(rng.choice(batch, size=min(batch, 12), replace=False).tolist()) | {0, batch - 1})

    def rows(b):
        ps, qs, pf, qf, d = workloads.verify_linear_seq(0, b, 15, 151936, sigma, "bf16")
        assert np.array_equal(d, c["drafts"][b])
        return pf, qf, d, c["u_acc"][b], float(c["u_s"][b])

    say(f"  oracle on {len(seqs)} sequences")
    ties = check_linear(rows, g, seqs, 15)
    say(f"  ties: {ties}; mean accepted length {g['accept_len'].mean():.3f}")
    assert ties <= 1


def _logits(prob):
    """ln(prob), with probability 0 as the logit -1e4 (exp(-1e4) is 0 in fp32
    and in float64 alike; the data contract bounds |logit / T| by 1e4)."""
    with np.errstate(divide="ignore"):
        return np.maximum(np.log(np.asarray(prob, np.float64)), -1e4)


def _f32_case(p, q, drafts, u_acc, u_s):
    """Device tensors of one sequence given as probabilities (fp32 logits ln p)."""
    pl = _logits(p).astype(np.float32)[None]
    ql = _logits(q).astype(np.float32).reshape(1, -1, pl.shape[2])
    return [to_dev(pl), to_dev(ql), to_dev(np.asarray([drafts], np.int32)),
            to_dev(np.asarray([u_acc], np.float32).reshape(1, -1)), to_dev(np.asarray([u_s], np.float32))]


def test_handworked_golden_cases(gpu_lib):
    """The hand-worked cases of tests/golden/verify_linear_handworked.json
    (residual point mass, accept then bonus, p/q = 1, all accepted, a bonus
    draw exactly on a CDF boundary) through the HIP kernels with fp32 logits
    ln(p): accepted length and token exactly as worked by hand, the draft
    probabilities within 1e-5 relative, the residual mass within 1e-5."""
    import torch
    with open(GOLDEN) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        say(f"golden {c['name']}")
        out = gpu_lib.psi_spec_verify_linear(*_f32_case(c["p"], c["q"], c["drafts"], c["u_accept"], c["u_sample"]))
        torch.cuda.synchronize()
        g = {kk: to_host(v) for kk, v in out.items()}
        e = c["expect"]
        assert int(g["accept_len"][0]) == e["accept_len"], c["name"]
        assert int(g["token"][0]) == e["token"], c["name"]
        np.testing.assert_allclose(g["p_draft"][0], e["p_draft"], rtol=1e-5)
        np.testing.assert_allclose(g["q_draft"][0], e["q_draft"], rtol=1e-5)
        assert abs(float(g["residual_mass"][0]) - e["residual_mass"]) <= 1e-5, c["name"]


def test_edge_one_hot_and_zero_residual(gpu_lib):
    """Edge cases of the accept rule and the residual draw, each against the
    oracle and its closed form:
    * p one-hot at v != d: every draft rejected, y = v;
    * q one-hot at d: the draft is accepted iff u < p(d), and a rejection draws
      from p without d;
    * a rejected draft of probability 0 under p = q: the residual
      max(0, p - q) has no mass, so y is drawn from p instead (S = 0 fallback,
      residual mass reported as 1)."""
    import torch
    V = 300
    rng = np.random.default_rng(3)
    base = rng.dirichlet(np.ones(V))
    # p one-hot at 17 (every other token probability exactly 0), drafts elsewhere
    p = np.zeros((3, V))
    p[:, 17] = 1.0
    q = np.tile(base, (2, 1))
    out = gpu_lib.psi_spec_verify_linear(*_f32_case(p, q, [3, 4], [0.0, 0.0], 0.9))
    torch.cuda.synchronize()
    assert int(to_host(out["accept_len"])[0]) == 0 and int(to_host(out["token"])[0]) == 17
    # q one-hot at the draft d = 5: accept iff u < p(5)
    p = np.tile(base, (2, 1))
    q = np.zeros((1, V))
    q[0, 5] = 1.0
    for u in (0.5 * base[5], 1.5 * base[5]):
        for us in (0.1, 0.6, 0.95):
            out = gpu_lib.psi_spec_verify_linear(*_f32_case(p, q, [5], [u], us))
            torch.cuda.synchronize()
            L, y = int(to_host(out["accept_len"])[0]), int(to_host(out["token"])[0])
            assert L == (1 if u < base[5] else 0)
            w = base.copy() if L == 1 else np.where(np.arange(V) == 5, 0.0, base)
            ref = oracle.inverse_cdf(w, us)
            assert y == ref or draw_is_valid(w, us, y, TIE), (u, us, y, ref)
    # S = 0: p = q, the draft has probability 0 under both, so it is rejected
    # and the residual max(0, p - q) is empty: y is drawn from p
    pz = base.copy()
    pz[9] = 0.0
    pz /= pz.sum()
    p = np.tile(pz, (2, 1))
    q = pz[None]
    for us in (0.05, 0.5, 0.97):
        out = gpu_lib.psi_spec_verify_linear(*_f32_case(p, q, [9], [0.3], us))
        torch.cuda.synchronize()
        g = {kk: to_host(v) for kk, v in out.items()}
        o = oracle.verify_linear(_logits(p)[None], _logits(q)[None], np.array([[9]]), np.array([[0.3]]),
                                 np.array([us]))
        assert int(g["accept_len"][0]) == 0 == int(o["accept_len"][0])
        assert abs(float(g["residual_mass"][0]) - 1.0) <= 1e-5          # the fallback row is p itself
        assert int(g["token"][0]) == int(o["token"][0]) or draw_is_valid(pz, us, int(g["token"][0]), TIE)
        assert int(g["token"][0]) != 9
