"""GPU parity: uno_psi_spec_verify_linear_early_exit (rows after the first
rejection mostly not read) against the oracle, and against the full verify.

Bar against the oracle: as for the full verify -- accepted lengths and tokens
bit-exact except near-ties (|u - p/q| < 1e-5, or a draw within 1e-5 of a CDF
boundary), which are counted; the draft probabilities of the evaluated
positions (0..L, the first rejection included) within 1e-5 relative and NaN
after it; residual mass within 1e-5.  Against the full verify on the same
inputs: identical bits (same row statistics, same merge order), ties
included.
"""

import numpy as np
import pytest

import oracle
import workloads
from _parity import check_linear, say, to_dev, to_host

pytestmark = pytest.mark.gpu


def _run(dad, c, early_exit=True, q=None):
    import torch
    f = dad.psi_spec_verify_linear_early_exit if early_exit else dad.psi_spec_verify_linear
    p = to_dev(c["p"])
    out = f(p, to_dev(c["q"]) if q is None else q, to_dev(c["drafts"]), to_dev(c["u_acc"]), to_dev(c["u_s"]),
            c["temperature"])
    torch.cuda.synchronize()
    return {kk: to_host(v) for kk, v in out.items()}


def _check(rows, g, seqs, k, temperature=1.0):
    """check_linear on L, y and the residual mass, then the draft probabilities
    of the evaluated positions against the oracle and NaN after them."""
    ties = check_linear(rows, {n: g[n] for n in ("accept_len", "token", "residual_mass")}, seqs, k, temperature)
    if k == 0:
        return ties
    for b in seqs:
        p, q, d, ua, us = rows(b)
        o = oracle.verify_linear(p[None], q[None], d[None], ua[None], np.array([us]), temperature)
        L = int(g["accept_len"][b])
        last = min(L, k - 1)   # the first rejection is evaluated too
        for name in ("p_draft", "q_draft"):
            got, ref = g[name][b], o[name][0]
            err = np.max(np.abs(got[:last + 1] - ref[:last + 1]) / np.maximum(ref[:last + 1], 1e-300))
            assert err <= 1e-5, f"seq {b} {name} rel err {err:.3g}"
            assert np.all(np.isnan(got[last + 1:])), f"seq {b} {name}: positions after the first rejection written"
    return ties


def _same_as_full(g, full, k):
    """Bit-identical to the full verify: L, token, residual mass, and the draft
    probabilities of the evaluated positions."""
    for name in ("accept_len", "token", "residual_mass"):
        np.testing.assert_array_equal(g[name], full[name], err_msg=name)
    for b in range(len(g["accept_len"])):
        n = min(int(g["accept_len"][b]), k - 1) + 1 if k else 0
        for name in ("p_draft", "q_draft"):
            np.testing.assert_array_equal(g[name][b][:n], full[name][b][:n], err_msg=f"seq {b} {name}")


def _rows(c):
    def f(b):
        return c["p_f32"][b], c["q_f32"][b], c["drafts"][b], c["u_acc"][b], float(c["u_s"][b])
    return f


@pytest.mark.parametrize("batch,k,vocab,sigma,dtype", [
    (2, 3, 1024, 0.5, "f32"),
    (8, 5, 20000, 0.5, "bf16"),        # several splits per row + ragged tail
    (4, 7, 20000, 0.1, "f32"),
    (3, 64, 3000, 0.05, "bf16"),       # maximum k, long accepted prefixes
    (5, 0, 4099, 1.0, "bf16"),         # k = 0: bonus draw only
    (6, 4, 1001, 1.0, "bf16"),         # odd vocab: rows not 16-byte aligned
    (4, 2, 7, 1.0, "f32"),             # vocab smaller than one vector
    (3, 2, 1, 1.0, "bf16"),            # vocab 1
    (40, 15, 9000, 2.0, "bf16"),       # mostly early rejections
    (12, 3, 5000, 0.2, "f32"),         # rounds {0, 1}, {2, 3 = bonus}
    (12, 8, 5000, 0.2, "bf16"),        # rounds {0, 1}, {2, 3}, {4..7}, {8 = bonus}
])
def test_early_exit_parity(gpu_lib, batch, k, vocab, sigma, dtype):
    say(f"verify_linear early exit batch={batch} k={k} V={vocab} sigma={sigma} {dtype}")
    c = workloads.verify_linear_case(batch, k, vocab, sigma, dtype=dtype, seed=batch * 7 + k + 1, workers=4)
    g = _run(gpu_lib, c)
    ties = _check(_rows(c), g, range(batch), k)
    assert ties <= max(1, batch // 50)
    _same_as_full(g, _run(gpu_lib, c, early_exit=False), k)


def test_early_exit_all_accepted_and_determinism(gpu_lib):
    """q = p (a strided view of the p rows): every draft accepted, the bonus
    drawn from p_k; two runs bit-identical."""
    c = workloads.verify_linear_case(16, 7, 9000, 0.5, dtype="bf16", seed=5, workers=4)
    p = to_dev(c["p"])
    g = _run(gpu_lib, c, q=p[:, :7])
    assert np.all(g["accept_len"] == 7)
    g1, g2 = _run(gpu_lib, c), _run(gpu_lib, c)
    for kk in g1:
        np.testing.assert_array_equal(g1[kk], g2[kk])


@pytest.mark.parametrize("sigma", [0.1, 0.5, 2.0])
def test_early_exit_full_vocab_batch(gpu_lib, sigma):
    """The sampler workload (batch 256, k = 15, V = 151,936, bf16): the full
    verify's outputs bit for bit, and the oracle's on sampled sequences."""
    batch = 256
    say(f"verify_linear early exit full V sigma={sigma}: generating")
    c = workloads.verify_linear_case(batch, 15, 151936, sigma, dtype="bf16", seed=0, keep_f32=False)
    g = _run(gpu_lib, c)
    full = _run(gpu_lib, c, early_exit=False)
    say(f"  mean L {g['accept_len'].mean():.3f}")
    _same_as_full(g, full, 15)
    rng = np.random.default_rng(2)
    seqs = sorted(set(rng.choice(batch, size=10, replace=False).tolist()) | {0, batch - 1})

    def rows(b):
        ps, qs, pf, qf, d = workloads.verify_linear_seq(0, b, 15, 151936, sigma, "bf16")
        assert np.array_equal(d, c["drafts"][b])
        return pf, qf, d, c["u_acc"][b], float(c["u_s"][b])

    ties = _check(rows, g, seqs, 15)
    say(f"  ties against the oracle: {ties}")
    assert ties <= 2
