"""GPU parity: uno_psi_spec_step (a whole decode step) against oracle.decode_step.

* With no decoder layers and tables chosen so that every product and sum is
  exact in fp32 (embedding rows of +-1, which normalise to +-1 in bf16, and an
  LM head of multiples of 1/64), the logits are bit-identical on both sides, so
  drafts, accepted lengths and tokens must match bit-exactly, except near-ties
  (|u - p/q| < 1e-5 for an accept, a uniform within 1e-5 of a CDF boundary for
  a draw), which are counted.
* With decoder layers, the logits are compared within the bf16 bar (row-wise
  max relative error 2e-2); the sampling decisions then sit on logits that
  differ by bf16 rounding, so their agreement with the oracle is reported,
  and checked for range and consistency, not gated bit-exactly.
"""

import numpy as np
import pytest

import oracle
import workloads
from _parity import TIE, draw_is_valid, row_relerr, say, to_dev, to_host

pytestmark = pytest.mark.gpu


def _f64(bits):
    return workloads.bf16_to_f32(bits).astype(np.float64)


def _run_step(dad, c, temperature=1.0):
    import torch
    cfg = dad.step_config(c["batch"], c["block"], c["ctx"], c["hidden"], c["inter"], c["n_heads"],
                          c["n_kv_heads"], c["r"], c["n_layers"], c["vocab"], temperature=temperature)
    keep = []
    layers = []
    for l in range(c["n_layers"]):
        wt = {k: to_dev(v) for k, v in c["layers"][l].items() if not k.endswith("_f32")}
        kc, vc = to_dev(c["k_caches"][l]), to_dev(c["v_caches"][l])
        keep += [wt, kc, vc]
        layers.append(dad.layer_weights(wt, kc, vc))
    out = dad.psi_spec_step(cfg, layers, to_dev(c["embed"]), to_dev(c["final_norm"]), to_dev(c["lm_head"]),
                            to_dev(c["tokens"]), to_dev(c["u_draft"]), to_dev(c["u_accept"]),
                            to_dev(c["u_sample"]))
    torch.cuda.synchronize()
    return {k: to_host(v) for k, v in out.items()}


def _oracle(c, seqs, temperature=1.0):
    sl = np.asarray(seqs)
    layers = [{k[:-4]: v.astype(np.float64) for k, v in lw.items() if k.endswith("_f32")} for lw in c["layers"]]
    return oracle.decode_step(c["tokens"][sl], _f64(c["embed"]), layers,
                              [_f64(kc[sl]) for kc in c["k_caches"]], [_f64(vc[sl]) for vc in c["v_caches"]],
                              _f64(c["final_norm"]), _f64(c["lm_head"]), c["u_draft"][sl], c["u_accept"][sl],
                              c["u_sample"][sl], c["block"], c["n_heads"], c["n_kv_heads"],
                              temperature=temperature)


def _rows_of(c, seqs):
    n = 2 * c["block"]
    return np.concatenate([np.arange(b * n, (b + 1) * n) for b in seqs])


def _exact_case(batch, block, vocab, hidden, seed):
    rng = workloads.rng_for(seed, 901)
    c = workloads.step_case(batch, block, 0, hidden, 8, 8, 8, 0, 0, vocab, seed=seed)
    emb = rng.choice(np.array([-1.0, 1.0], np.float32), size=(vocab, hidden))
    lm = rng.integers(-8, 9, size=(vocab, hidden)).astype(np.float32) / np.float32(64.0)
    c["embed"] = workloads.bf16_bits(emb)
    c["lm_head"] = workloads.bf16_bits(lm)
    c["final_norm"] = workloads.bf16_bits(np.ones(hidden, np.float32))
    # noisy id i equal to clean id i for i < m_b: those drafts face q_i = p_i
    # and are accepted, so the accepted lengths spread over 0..k
    for b in range(batch):
        m = b % block
        c["tokens"][b, block:block + m] = c["tokens"][b, :m]
    return c


@pytest.mark.parametrize("batch,block,vocab,hidden,temp", [
    (3, 5, 1001, 256, 1.0),
    (8, 16, 4096, 512, 1.0),
    (2, 1, 300, 64, 1.0),          # block 1: no drafts, bonus draw only
    (4, 8, 2000, 128, 0.7),
])
def test_step_zero_layers_bit_exact(gpu_lib, batch, block, vocab, hidden, temp):
    say(f"step, no layers (exact logits): B={batch} block={block} V={vocab} hidden={hidden} T={temp}")
    c = _exact_case(batch, block, vocab, hidden, seed=batch + vocab)
    g = _run_step(gpu_lib, c, temp)
    o = _oracle(c, list(range(batch)), temp)
    assert np.array_equal(g["logits"].astype(np.float64), o["logits"]), "logits not bit-identical"
    k = block - 1
    ties = 0
    lg = o["logits"].reshape(batch, 2 * block, vocab)
    for b in range(batch):
        draft_tie = False
        for i in range(k):
            if g["drafts"][b, i] != o["drafts"][b, i]:
                q = oracle.softmax_rows(lg[b, block + i], temp)
                assert draw_is_valid(q, float(c["u_draft"][b, i]), int(g["drafts"][b, i]), TIE), (b, i)
                draft_tie = True
        if draft_tie:
            ties += 1
            continue       # a draft differed at a near-tie: the rest of this sequence is not comparable
        Lo, Lg = int(o["accept_len"][b]), int(g["accept_len"][b])
        if Lo != Lg:
            i = min(Lo, Lg)
            assert abs(float(c["u_accept"][b, i]) - o["p_draft"][b, i] / o["q_draft"][b, i]) < TIE, b
            ties += 1
            continue
        if g["token"][b] != o["token"][b]:
            p = oracle.softmax_rows(lg[b, Lo], temp)
            if Lo < k:
                w, s = oracle.residual_weights(p, oracle.softmax_rows(lg[b, block + Lo], temp))
                w = p if s == 0.0 else w
            else:
                w = p
            assert draw_is_valid(w, float(c["u_sample"][b]), int(g["token"][b]), TIE), b
            ties += 1
    say(f"  L {g['accept_len'].tolist()[:8]}, near-ties {ties}")
    assert ties <= max(1, batch // 8)


@pytest.mark.parametrize("batch,block,ctx,hidden,inter,nh,nkv,r,n_layers,vocab", [
    (2, 4, 40, 256, 512, 4, 2, 16, 2, 1000),
    (3, 16, 130, 512, 1024, 8, 2, 32, 3, 4096),
])
def test_step_with_layers(gpu_lib, batch, block, ctx, hidden, inter, nh, nkv, r, n_layers, vocab):
    say(f"step: B={batch} block={block} ctx={ctx} hidden={hidden} layers={n_layers} V={vocab}")
    c = workloads.step_case(batch, block, ctx, hidden, inter, nh, nkv, r, n_layers, vocab, seed=ctx,
                            weight_std=0.05)
    g = _run_step(gpu_lib, c)
    o = _oracle(c, list(range(batch)))
    err = row_relerr(g["logits"], o["logits"])
    agree = int(np.sum((g["accept_len"] == o["accept_len"]) & (g["token"] == o["token"])))
    say(f"  logits row rel err {err:.3g}; (L, y) agree on {agree}/{batch} sequences")
    assert err <= 2e-2
    k = block - 1
    assert np.all((g["accept_len"] >= 0) & (g["accept_len"] <= k))
    assert np.all((g["token"] >= 0) & (g["token"] < vocab))
    assert np.all((g["drafts"] >= 0) & (g["drafts"] < vocab))


def test_step_full_size_two_layers(gpu_lib):
    """The decode-step shape with two Qwen3-8B-shaped layers: 128 sequences x
    (16 clean + 16 noisy) rows, 8K cache, rank-128 adapters, vocab 151,936.
    Every launch has the configuration of the 36-layer step.  The oracle
    recomputes 1 sampled sequence through both layers and the LM head."""
    say("step full size, 2 layers: B=128 block=16 ctx=8192 V=151936")
    c = workloads.step_case(128, 16, 8192, 4096, 12288, 32, 8, 128, 2, 151936, seed=11)
    g = _run_step(gpu_lib, c)
    lg = g["logits"]
    assert np.all(np.isfinite(lg))
    assert np.all((g["accept_len"] >= 0) & (g["accept_len"] <= 15))
    assert np.all((g["token"] >= 0) & (g["token"] < 151936))
    assert np.all((g["drafts"] >= 0) & (g["drafts"] < 151936))
    seqs = [77]
    o = _oracle(c, seqs)
    err = row_relerr(lg[_rows_of(c, seqs)], o["logits"])
    say(f"  logits row rel err {err:.3g}; seq 77 L gpu {g['accept_len'][77]} oracle {o['accept_len'][0]}")
    assert err <= 2e-2
