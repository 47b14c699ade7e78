"""GPU parity: uno_psi_spec_verify_linear against the oracle.

Bar: accepted lengths and tokens bit-exact except near-ties (|u - p/q| < 1e-5,
or a draw within 1e-5 of a CDF boundary), which are counted; probabilities of
the drafts within 1e-5 relative (fp32 outputs); residual mass within 1e-5
absolute (a sum of at most 2^20 fp32 probability differences).
"""

import numpy as np
import pytest

import workloads
from _parity import check_linear, say, to_dev, to_host

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
    batch = 256 if sigma == 0.5 else 32
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
