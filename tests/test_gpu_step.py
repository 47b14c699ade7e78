"""GPU parity: uno_psi_spec_step (one decode step of the decode loop) against
oracle.decode_step.

* With no decoder layers and tables chosen so that every product and sum is
  exact in fp32 (embedding rows of +-1, which normalise to +-1 in bf16, and an
  LM head of multiples of 1/64), the logits are bit-identical on both sides,
  so drafts, accepted lengths, tokens and the next step's ids must match
  bit-exactly, except near-ties (|u - p/q| < 1e-5 for an accept, a uniform
  within 1e-5 of a CDF boundary for a draw), which are counted.
* With decoder layers, the logits are compared within the bf16 bar (row-wise
  max relative error 2e-2), and every sampling decision is checked against
  the oracle run on the GPU's own bf16 logits (both sides then decide on the
  same values): bit-exact up to near-ties.
* The full-size step (two Qwen3-8B-shaped layers, 128 sequences, V =
  151,936) is run twice on the same inputs and must give bitwise identical
  results.
* "merged": the layers also carry gate-merged weights (uno_lora_merge), so
  the noisy rows read W + B A and no LoRA-down runs; the same bars hold
  against the same (unmerged) oracle.
"""

import numpy as np
import pytest

import oracle
import workloads
from _parity import TIE, check_step_decisions, row_relerr, say, to_dev, to_host

pytestmark = pytest.mark.gpu


def _f64(bits):
    return workloads.bf16_to_f32(bits).astype(np.float64)


def _layers(dad, c, merged=False):
    keep, layers = [], []
    for l in range(c["n_layers"]):
        wt = {k: to_dev(v) for k, v in c["layers"][l].items() if not k.endswith("_f32")}
        if merged:
            dad.merge_layer(wt)
        kc, vc = to_dev(c["k_caches"][l]), to_dev(c["v_caches"][l])
        keep += [wt, kc, vc]
        layers.append(dad.layer_weights(wt, kc, vc))
    return keep, layers


def _run_step(dad, c, prev_q=None, temperature=1.0, cache_len=None, merged=False):
    import torch
    cfg = dad.step_config(c["batch"], c["block"], c["ctx"], c["hidden"], c["inter"], c["n_heads"],
                          c["n_kv_heads"], c["r"], c["n_layers"], c["vocab"], temperature=temperature)
    keep, layers = _layers(dad, c, merged)
    pq = None if prev_q is None else to_dev(prev_q)
    out = dad.psi_spec_step(cfg, layers, to_dev(c["embed"]), to_dev(c["final_norm"]), to_dev(c["lm_head"]),
                            to_dev(c["tokens"]), to_dev(c["u_draft"]), to_dev(c["u_accept"]), to_dev(c["u_sample"]),
                            prev_q=pq, next_tokens=True,
                            cache_len=None if cache_len is None else to_dev(np.asarray(cache_len, np.int32)))
    torch.cuda.synchronize()
    return {k: to_host(v) for k, v in out.items()}


def _oracle(c, seqs, prev_q=None, temperature=1.0, cache_len=None, capacity=None):
    sl = np.asarray(seqs)
    layers = [{k[:-4]: v.astype(np.float64) for k, v in lw.items() if k.endswith("_f32")} for lw in c["layers"]]
    return oracle.decode_step(c["tokens"][sl], _f64(c["embed"]), layers,
                              [_f64(kc[sl]) for kc in c["k_caches"]], [_f64(vc[sl]) for vc in c["v_caches"]],
                              _f64(c["final_norm"]), _f64(c["lm_head"]),
                              None if prev_q is None else _f64(prev_q)[sl], c["u_draft"][sl], c["u_accept"][sl],
                              c["u_sample"][sl], c["block"], c["n_heads"], c["n_kv_heads"], temperature=temperature,
                              cache_len=None if cache_len is None else np.asarray(cache_len)[sl],
                              capacity=capacity)


def _rows_of(c, seqs):
    n = 2 * c["block"]
    return np.concatenate([np.arange(b * n, (b + 1) * n) for b in seqs])


def _random_prev_q(c, seed, std=2.0):
    """bf16 draft logits [B, k, V] ~ N(0, std^2) standing in for the previous step's noisy rows."""
    rng = workloads.rng_for(seed, 907)
    x = rng.standard_normal((c["batch"], c["block"] - 1, c["vocab"]), dtype=np.float32) * np.float32(std)
    return workloads.bf16_bits(x)


def _exact_case(batch, block, vocab, hidden, seed):
    """Tables with exact fp32 logits; the carried q of sequence b equals its
    clean rows' own logits on the first b % block rows (those drafts face
    q_i = p_i and are accepted, so the accepted lengths spread over 0..k) and
    is random bf16 on the rest."""
    rng = workloads.rng_for(seed, 901)
    c = workloads.step_case(batch, block, 0, hidden, 8, 8, 8, 0, 0, vocab, seed=seed)
    emb = rng.choice(np.array([-1.0, 1.0], np.float32), size=(vocab, hidden))
    lm = rng.integers(-8, 9, size=(vocab, hidden)).astype(np.float32) / np.float32(64.0)
    c["embed"] = workloads.bf16_bits(emb)
    c["lm_head"] = workloads.bf16_bits(lm)
    c["final_norm"] = workloads.bf16_bits(np.ones(hidden, np.float32))
    k = block - 1
    prev_q = _random_prev_q(c, seed)
    clean = emb[c["tokens"][:, :block]].astype(np.float64) @ lm.astype(np.float64).T   # exact
    for b in range(batch):
        m = min(b % block, k)
        prev_q[b, :m] = workloads.bf16_bits(clean[b, :m].astype(np.float32))
    return c, prev_q


@pytest.mark.parametrize("batch,block,vocab,hidden,temp,first", [
    (3, 5, 1001, 256, 1.0, False),
    (8, 16, 4096, 512, 1.0, False),
    (2, 1, 300, 64, 1.0, False),          # block 1: no drafts, bonus draw only
    (4, 8, 2000, 128, 0.7, False),
    (5, 6, 777, 64, 1.0, True),           # the loop's first step: nothing carried, nothing verified
])
def test_step_zero_layers_bit_exact(gpu_lib, batch, block, vocab, hidden, temp, first):
    say(f"step, no layers (exact logits): B={batch} block={block} V={vocab} hidden={hidden} T={temp} first={first}")
    c, prev_q = _exact_case(batch, block, vocab, hidden, seed=batch + vocab)
    pq = None if first else prev_q
    g = _run_step(gpu_lib, c, pq, temp)
    o = _oracle(c, list(range(batch)), pq, temp)
    assert np.array_equal(g["logits"].astype(np.float64), o["logits"]), "logits not bit-identical"
    if first:
        assert np.all(g["accept_len"] == 0)
    dties, ties = check_step_decisions(g["logits"], block, c["tokens"], None if first else _f64(prev_q), g,
                                       c["u_draft"], c["u_accept"], c["u_sample"], temp)
    # the next step's ids: [y, this step's drafts, the same noisy ids]
    np.testing.assert_array_equal(g["next_tokens"][:, 0], g["token"])
    np.testing.assert_array_equal(g["next_tokens"][:, 1:block], g["drafts"])
    np.testing.assert_array_equal(g["next_tokens"][:, block:], c["tokens"][:, block:])
    say(f"  L {g['accept_len'].tolist()[:8]}, near-ties: drafts {dties}, decisions {ties}")
    assert ties <= max(1, batch // 8) and dties <= max(1, batch * (block - 1) // 50)
    if not first and block > 1:
        assert len(set(g["accept_len"].tolist())) > 1


def test_step_zero_layers_capacity_flags(gpu_lib):
    """Cache lengths with a capacity: every sequence's length grows by L + 1
    when its kept rows fit; a sequence whose kept rows do not fit is flagged
    (accept_len = token = -1, next step's first id -1) and keeps its length."""
    import torch
    batch, block, vocab, hidden, cap = 6, 4, 500, 64, 40
    say(f"step, no layers, capacity {cap}: B={batch} block={block}")
    c, prev_q = _exact_case(batch, block, vocab, hidden, seed=77)
    c["ctx"] = cap
    lens = np.array([0, 10, 36, 37, 39, 40], np.int32)
    cl = to_dev(lens)
    cfg = gpu_lib.step_config(batch, block, cap, hidden, 8, 8, 8, 0, 0, vocab)
    out = gpu_lib.psi_spec_step(cfg, [], to_dev(c["embed"]), to_dev(c["final_norm"]), to_dev(c["lm_head"]),
                                to_dev(c["tokens"]), to_dev(c["u_draft"]), to_dev(c["u_accept"]),
                                to_dev(c["u_sample"]), prev_q=to_dev(prev_q), cache_len=cl, next_tokens=True)
    torch.cuda.synchronize()
    g = {k: to_host(v) for k, v in out.items()}
    o = _oracle(c, list(range(batch)), prev_q, cache_len=lens, capacity=cap)
    np.testing.assert_array_equal(g["accept_len"], o["accept_len"])
    np.testing.assert_array_equal(g["token"], o["token"])
    new = to_host(cl)
    for b in range(batch):
        if o["accept_len"][b] < 0:
            assert new[b] == lens[b] and g["next_tokens"][b, 0] == -1
        else:
            assert new[b] == lens[b] + o["accept_len"][b] + 1
    assert (o["accept_len"] < 0).any() and (o["accept_len"] >= 0).any()
    say(f"  L {g['accept_len'].tolist()}, lengths {lens.tolist()} -> {new.tolist()}")


@pytest.mark.parametrize("batch,block,ctx,hidden,inter,nh,nkv,r,n_layers,vocab,merged", [
    (2, 4, 40, 256, 512, 4, 2, 16, 2, 1000, False),
    (3, 16, 130, 512, 1024, 8, 2, 32, 3, 4096, False),
    # 512 rows: 256 clean + 256 noisy, whole tiles on both sides of the split,
    # so q, k, v, o and the fused gate/up run gate-merged (down splits K and
    # takes the LoRA-down path)
    (16, 16, 70, 512, 1024, 4, 2, 64, 2, 2048, True),
])
def test_step_with_layers(gpu_lib, batch, block, ctx, hidden, inter, nh, nkv, r, n_layers, vocab, merged):
    say(f"step: B={batch} block={block} ctx={ctx} hidden={hidden} layers={n_layers} V={vocab} merged={merged}")
    c = workloads.step_case(batch, block, ctx, hidden, inter, nh, nkv, r, n_layers, vocab, seed=ctx,
                            weight_std=0.05)
    prev_q = _random_prev_q(c, ctx)
    g = _run_step(gpu_lib, c, prev_q, merged=merged)
    o = _oracle(c, list(range(batch)), prev_q)
    err = row_relerr(g["logits"], o["logits"])
    dties, ties = check_step_decisions(g["logits"], block, c["tokens"], _f64(prev_q), g, c["u_draft"],
                                       c["u_accept"], c["u_sample"])
    say(f"  logits row rel err {err:.3g}; decisions on the GPU's logits: near-ties drafts {dties}, decisions {ties}; "
        f"L gpu {g['accept_len'].tolist()} oracle {o['accept_len'].tolist()}")
    assert err <= 2e-2
    assert ties <= 1 and dties <= 1


@pytest.mark.parametrize("merged", [False, True])
def test_step_full_size_two_layers_decisions_and_determinism(gpu_lib, merged):
    """The decode-step shape with two Qwen3-8B-shaped layers: 128 sequences x
    (16 clean + 16 noisy) rows, 8K cache, rank-128 adapters, vocab 151,936.
    Every launch has the configuration of the 36-layer step.  The oracle
    recomputes 1 sampled sequence through both layers and the LM head (logits
    within the bar); every sampling decision of all 128 sequences is checked
    on the GPU's own logits; a second run on the same inputs is bitwise
    identical (fixed-order split reductions everywhere)."""
    import torch
    say(f"step full size, 2 layers: B=128 block=16 ctx=8192 V=151936 merged={merged}")
    c = workloads.step_case(128, 16, 8192, 4096, 12288, 32, 8, 128, 2, 151936, seed=11)
    prev_q = _random_prev_q(c, 11)
    cfg = gpu_lib.step_config(128, 16, 8192, 4096, 12288, 32, 8, 128, 2, 151936)
    keep, layers = _layers(gpu_lib, c, merged)
    args = [to_dev(c[k]) for k in ("embed", "final_norm", "lm_head", "tokens", "u_draft", "u_accept", "u_sample")]
    pq = to_dev(prev_q)
    runs = []
    for rep in range(2):
        out = gpu_lib.psi_spec_step(cfg, layers, *args, prev_q=pq, next_tokens=True)
        torch.cuda.synchronize()
        runs.append({k: v.clone() for k, v in out.items()})
        say(f"  run {rep} done")
    for name in runs[0]:
        assert torch.equal(runs[0][name].view(torch.int16) if runs[0][name].dtype == torch.bfloat16 else runs[0][name],
                           runs[1][name].view(torch.int16) if runs[1][name].dtype == torch.bfloat16 else runs[1][name]), \
            f"{name} differs between two runs"
    g = {k: to_host(v) for k, v in runs[0].items()}
    lg = g["logits"]
    assert np.all(np.isfinite(lg))
    dties, ties = check_step_decisions(lg, 16, c["tokens"], _f64(prev_q), g, c["u_draft"], c["u_accept"],
                                       c["u_sample"])
    say(f"  decisions of all 128 sequences on the GPU's logits: near-ties drafts {dties} of 1920 draws, accepts/"
        f"tokens {ties} of 128; mean L {g['accept_len'].mean():.2f}")
    # near-uniform rows of 151,936 tokens give each token a mass below the
    # 1e-5 tie band, so fp32 CDF rounding puts a few percent of draws in it
    assert ties <= 4 and dties <= 1920 // 20
    seqs = [77]
    o = _oracle(c, seqs, prev_q)
    err = row_relerr(lg[_rows_of(c, seqs)], o["logits"])
    say(f"  logits row rel err {err:.3g} (seq 77)")
    assert err <= 2e-2
