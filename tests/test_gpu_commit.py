"""GPU parity of the decode loop's cache handling against the oracle:
per-sequence cache lengths in uno_block_verify_attention and
uno_decoder_layer, the clean rows' keys and values appended by the layer,
uno_kv_commit, and two chained uno_psi_spec_step calls that grow the cache.

Bar: bf16 outputs within a row-wise max relative error of 2e-2; LSE within
1e-5 * max(1, |lse|); cache rows the call must not touch and cache lengths
bit-exact.  The commit is checked given the GPU's accepted lengths (the
oracle's kv_commit takes them as input), so a near-tie accept decision cannot
make the two caches differ; agreement of the accepted lengths is reported.
"""

import numpy as np
import pytest

import oracle
import workloads
from _layer_cases import BAR as LAYER_BAR, APPEND_CASES, FULL_CASES, ids as layer_ids, make as make_layer_case
from _parity import check_step_decisions, row_relerr, say, to_dev, to_host

pytestmark = pytest.mark.gpu

SLACK = 100.0   # unused capacity is filled with this: a read of it would dominate a softmax


def _f32(bits):
    return workloads.bf16_to_f32(bits).astype(np.float64)


def _fill_slack(bits, lens):
    out = bits.copy()
    big = workloads.bf16_bits(np.array([SLACK], np.float32))[0]
    for b, n in enumerate(lens):
        out[b, n:] = big
    return out


@pytest.mark.parametrize("batch,block,cap,nh,nkv,lens", [
    (4, 4, 100, 8, 2, [0, 37, 100, 64]),       # empty, ragged tail, full, block-aligned
    (3, 16, 300, 32, 8, [1, 299, 33]),
    (2, 16, 2000, 32, 8, [2000, 517]),         # key splits; the short sequence leaves splits empty
    (1, 1, 50, 4, 4, [0]),
])
def test_block_attention_ragged_lengths(gpu_lib, batch, block, cap, nh, nkv, lens):
    say(f"block attention ragged B={batch} block={block} cap={cap} H={nh}/{nkv} lens={lens}")
    import torch
    rng = workloads.rng_for(31, batch, block, cap)
    n = 2 * block
    g = lambda s: workloads.bf16_bits(rng.standard_normal(s, dtype=np.float32))
    q, kb, vb = g((batch, n, nh, 128)), g((batch, n, nkv, 128)), g((batch, n, nkv, 128))
    kc = _fill_slack(g((batch, cap, nkv, 128)), lens)
    vc = _fill_slack(g((batch, cap, nkv, 128)), lens)
    cl = to_dev(np.asarray(lens, np.int32))
    out, lse = gpu_lib.block_verify_attention(to_dev(q), to_dev(kc), to_dev(vc), to_dev(kb), to_dev(vb), block,
                                              1.0 / np.sqrt(128), cache_len=cl)
    torch.cuda.synchronize()
    ro, rl = oracle.block_attention(_f32(q), _f32(kc), _f32(vc), _f32(kb), _f32(vb), block, 1.0 / np.sqrt(128),
                                    ctx_lens=np.asarray(lens))
    err = row_relerr(to_host(out), ro)
    lerr = np.max(np.abs(to_host(lse) - rl) / np.maximum(1.0, np.abs(rl)))
    say(f"  row rel err {err:.3g}, lse err {lerr:.3g}")
    assert err <= 2e-2
    assert lerr <= 1e-5


def test_kv_commit_lengths(gpu_lib):
    """uno_kv_commit over 300 sequences against oracle.kv_commit's lengths and
    flags: a length grows by L + 1 when the kept rows fit the capacity, else
    it stays and L becomes -1 (also for an L already -1)."""
    say("kv_commit batch=300 capacity=50")
    import torch
    rng = workloads.rng_for(8)
    lens = rng.integers(0, 51, 300).astype(np.int32)
    acc = rng.integers(-1, 16, 300).astype(np.int32)
    cl, ad = to_dev(lens), to_dev(acc)
    gpu_lib.kv_commit(ad, cl, 50)
    torch.cuda.synchronize()
    z = np.zeros((300, 50, 1, 1))
    _, _, ref_len, ref_acc = oracle.kv_commit(z, z, lens, np.zeros((300, 16, 1, 1)), np.zeros((300, 16, 1, 1)), acc)
    np.testing.assert_array_equal(to_host(cl), ref_len)
    np.testing.assert_array_equal(to_host(ad), ref_acc)
    assert (ref_acc == -1).sum() > (acc == -1).sum()      # some sequences were flagged by the capacity


@pytest.mark.parametrize("lc", APPEND_CASES, ids=layer_ids(APPEND_CASES))
def test_decoder_layer_appends_clean_rows(gpu_lib, lc):
    """A layer over caches of per-sequence lengths (tests/_layer_cases.py): the
    hidden state within the bar, the clean rows' rotated k and their v written
    after each sequence's valid rows (only the rows that fit the capacity),
    every other cache row bit-identical."""
    batch, block, cap, lens = lc["batch"], lc["block"], lc["ctx"], lc["lens"]
    nh, nkv, inter, r = lc["nh"], lc["nkv"], lc["inter"], lc["r"]
    say(f"decoder layer with cache lengths {lc['name']}: B={batch} block={block} cap={cap} lens={lens}")
    import torch
    c = make_layer_case(lc)
    kc0 = _fill_slack(c["k_cache"], lens)
    vc0 = _fill_slack(c["v_cache"], lens)
    pos = c["positions"]
    wt = {k: to_dev(v) for k, v in c["weights"].items() if not k.endswith("_f32")}
    kc, vc, h = to_dev(kc0), to_dev(vc0), to_dev(c["h"])
    lw = gpu_lib.layer_weights(wt, kc, vc)
    gpu_lib.decoder_layer(h, lw, to_dev(c["gate"]), to_dev(pos), batch, block, cap, nh, nkv, inter, r,
                          cache_len=to_dev(np.asarray(lens, np.int32)))
    torch.cuda.synchronize()
    w64 = {k[:-4]: v.astype(np.float64) for k, v in c["weights"].items() if k.endswith("_f32")}
    ref, st = oracle.decoder_layer(_f32(c["h"]), w64, c["gate"], pos, _f32(kc0), _f32(vc0), block, nh, nkv,
                                   ctx_lens=np.asarray(lens))
    err = row_relerr(to_host(h), ref)
    say(f"  hidden row rel err {err:.3g}")
    assert err <= LAYER_BAR
    kg, vg = to_host(kc), to_host(vc)
    k_ref = st["k"].reshape(batch, 2 * block, nkv, 128)
    v_ref = st["v"].reshape(batch, 2 * block, nkv, 128)
    worst = 0.0
    for b, n in enumerate(lens):
        m = min(block, cap - n)                      # clean rows that fit
        new = slice(n, n + m)
        untouched = np.ones(cap, bool)
        untouched[new] = False
        assert np.array_equal(kg[b, untouched], _f32(kc0[b, untouched])), f"seq {b}: k rows outside the append"
        assert np.array_equal(vg[b, untouched], _f32(vc0[b, untouched])), f"seq {b}: v rows outside the append"
        if m > 0:
            worst = max(worst, row_relerr(kg[b, new], k_ref[b, :m]), row_relerr(vg[b, new], v_ref[b, :m]))
    say(f"  appended k/v row rel err {worst:.3g}")
    assert worst <= 2e-2


def _step_layers(gpu_lib, c):
    keep, layers, kcs, vcs = [], [], [], []
    for l in range(c["n_layers"]):
        wt = {k: to_dev(v) for k, v in c["layers"][l].items() if not k.endswith("_f32")}
        kc, vc = to_dev(c["k_caches"][l]), to_dev(c["v_caches"][l])
        keep.append(wt)
        kcs.append(kc)
        vcs.append(vc)
        layers.append(gpu_lib.layer_weights(wt, kc, vc))
    return keep, layers, kcs, vcs


def _host_layers(c):
    return [{k[:-4]: v.astype(np.float64) for k, v in lw.items() if k.endswith("_f32")} for lw in c["layers"]]


def test_step_decode_loop_chain(gpu_lib):
    """Four chained steps on caches of per-sequence lengths, each fed only by
    the previous step's outputs on the device: its next ids (written in place
    over the token buffer), the noisy-row logits of the other logits buffer
    as the carried q, and the committed lengths.  The first step carries no
    q.  At every step the oracle, run on the same ids over its own caches,
    gives logits within the bar; every sampling decision is checked on the
    GPU's own logits (bit-exact up to near-ties); the lengths, the next ids
    and the committed cache rows (within the bar) follow the oracle's commit
    of the GPU's accepted lengths; the initial rows are never rewritten.
    Sequence 0 accepts every draft (u_accept = 0); sequence 2 does too and runs
    out of capacity at the third step, which flags it (L = y = -1, length
    unchanged)."""
    import torch
    batch, block, cap, hidden, inter, nh, nkv, r, nl, vocab = 3, 5, 48, 256, 512, 4, 2, 16, 2, 1001
    k = block - 1
    say(f"decode loop: 4 chained steps B={batch} block={block} cap={cap} layers={nl} V={vocab}")
    c = workloads.step_case(batch, block, cap, hidden, inter, nh, nkv, r, nl, vocab, seed=12, weight_std=0.05)
    lens = np.array([3, 20, 41])
    for l in range(nl):
        c["k_caches"][l] = _fill_slack(c["k_caches"][l], lens)
        c["v_caches"][l] = _fill_slack(c["v_caches"][l], lens)
    keep, layers, kcs, vcs = _step_layers(gpu_lib, c)
    cfg = gpu_lib.step_config(batch, block, cap, hidden, inter, nh, nkv, r, nl, vocab)
    dev = {name: to_dev(c[name]) for name in ("embed", "final_norm", "lm_head")}
    cl = to_dev(lens.astype(np.int32))
    toks = to_dev(c["tokens"])
    logit_bufs = [torch.empty((batch * 2 * block, vocab), dtype=torch.bfloat16, device="cuda") for _ in range(2)]
    g = workloads.rng_for(12, 5)
    w64 = _host_layers(c)
    ok_k = [_f32(x) for x in c["k_caches"]]
    ok_v = [_f32(x) for x in c["v_caches"]]
    o_len = lens.copy()
    prev_q_host = None
    for step in range(4):
        ud = g.random((batch, k), dtype=np.float32)
        ua = g.random((batch, k), dtype=np.float32)
        ua[0] = ua[2] = 0.0
        us = g.random(batch, dtype=np.float32)
        tok_before = to_host(toks)
        prev_q = None if step == 0 else gpu_lib.noisy_rows(logit_bufs[(step - 1) % 2], cfg)
        out = gpu_lib.psi_spec_step(cfg, layers, dev["embed"], dev["final_norm"], dev["lm_head"], toks, to_dev(ud),
                                    to_dev(ua), to_dev(us), prev_q=prev_q, logits=logit_bufs[step % 2],
                                    cache_len=cl, next_tokens=toks)
        torch.cuda.synchronize()
        gh = {name: to_host(v) for name, v in out.items()}
        g_len = to_host(cl)
        ref = oracle.decode_step(tok_before, _f32(c["embed"]), w64, ok_k, ok_v, _f32(c["final_norm"]),
                                 _f32(c["lm_head"]), prev_q_host, ud, ua, us, block, nh, nkv, cache_len=o_len)
        err = row_relerr(gh["logits"], ref["logits"])
        dties, ties = check_step_decisions(gh["logits"], block, tok_before, prev_q_host, gh, ud, ua, us)
        say(f"  step {step}: logits row rel err {err:.3g}; L {gh['accept_len'].tolist()} (oracle on its own "
            f"logits {ref['accept_len'].tolist()}); near-ties {dties} + {ties}; lengths {o_len.tolist()} -> "
            f"{g_len.tolist()}")
        assert err <= 2e-2
        assert ties == 0 and dties == 0
        if step == 0:
            assert np.all(gh["accept_len"] == 0)
        # the oracle commits the GPU's (checked) accepted lengths
        new_len = o_len
        for l in range(nl):
            ok_k[l], ok_v[l], new_len, acc_o = oracle.kv_commit(ok_k[l], ok_v[l], o_len, ref["k_clean"][l],
                                                                ref["v_clean"][l], gh["accept_len"])
        np.testing.assert_array_equal(g_len, new_len)
        np.testing.assert_array_equal(gh["accept_len"], acc_o)
        flagged = gh["accept_len"] < 0
        assert np.all(gh["token"][flagged] == -1)
        np.testing.assert_array_equal(gh["next_tokens"][:, 0], np.where(flagged, -1, gh["token"]))
        np.testing.assert_array_equal(gh["next_tokens"][:, 1:block], gh["drafts"])
        np.testing.assert_array_equal(gh["next_tokens"][:, block:], tok_before[:, block:])
        worst = 0.0
        for l in range(nl):
            kg, vg = to_host(kcs[l]), to_host(vcs[l])
            for b in range(batch):
                kept = slice(o_len[b], new_len[b])
                if new_len[b] > o_len[b]:
                    worst = max(worst, row_relerr(kg[b, kept], ok_k[l][b, kept]),
                                row_relerr(vg[b, kept], ok_v[l][b, kept]))
                assert np.array_equal(kg[b, :lens[b]], _f32(c["k_caches"][l][b, :lens[b]]))
                assert np.array_equal(vg[b, :lens[b]], _f32(c["v_caches"][l][b, :lens[b]]))
        say(f"  step {step}: committed k/v row rel err {worst:.3g}")
        assert worst <= 2e-2
        if step == 2:
            assert flagged[2] and not flagged[0], "sequence 2 should run out of capacity at the third step"
        o_len = new_len
        prev_q_host = gh["logits"].reshape(batch, 2 * block, vocab)[:, block:block + k].astype(np.float64)
    assert o_len[0] == lens[0] + 1 + 3 * block           # every draft of sequence 0 accepted after the first step


@pytest.mark.parametrize("lc", FULL_CASES[1:], ids=layer_ids(FULL_CASES[1:]))
def test_decoder_layer_full_size_decode_loop_sampled(gpu_lib, lc):
    """One Qwen3-8B-shaped layer in the launch configuration the bench times:
    128 sequences x (16 clean + 16 noisy) rows, caches of 8192 + 16 rows with
    8192 valid (two sequences shorter), adapters back to back; the oracle
    recomputes 3 sampled sequences, their appended rows are checked, and every
    sequence's rows outside its append are unchanged."""
    import torch
    batch, block, cap, lens = lc["batch"], lc["block"], lc["ctx"], np.asarray(lc["lens"])
    nh, nkv, inter, r = lc["nh"], lc["nkv"], lc["inter"], lc["r"]
    say(f"decoder layer {lc['name']}: B={batch} block={block} cap={cap} Qwen3-8B shapes (sampled {lc['seqs']})")
    c = make_layer_case(lc)
    for name in ("k_cache", "v_cache"):
        c[name] = _fill_slack(c[name], lens)
    pos = c["positions"]
    wt = {k: to_dev(v) for k, v in c["weights"].items() if not k.endswith("_f32")}
    for group in (("q", "k", "v"), ("g", "u")):   # adapters back to back, as the bench stores them
        cat = torch.cat([wt["a" + p] for p in group], dim=0).contiguous()
        for i, p in enumerate(group):
            wt["a" + p] = cat[i * r:(i + 1) * r]
    kc, vc, h = to_dev(c["k_cache"]), to_dev(c["v_cache"]), to_dev(c["h"])
    lw = gpu_lib.layer_weights(wt, kc, vc)
    gpu_lib.decoder_layer(h, lw, to_dev(c["gate"]), to_dev(pos), batch, block, cap, nh, nkv, inter, r,
                          cache_len=to_dev(lens.astype(np.int32)))
    torch.cuda.synchronize()
    got = to_host(h)
    assert np.all(np.isfinite(got))
    w64 = {k[:-4]: v.astype(np.float64) for k, v in c["weights"].items() if k.endswith("_f32")}
    # the caches come back as raw bf16 bits (2 GB each; no float copies of the whole cache)
    kbits = kc.view(torch.int16).cpu().numpy().view(np.uint16)
    vbits = vc.view(torch.int16).cpu().numpy().view(np.uint16)
    n = 2 * block
    for b in lc["seqs"]:
        rows = np.arange(b * n, (b + 1) * n)
        ref, st = oracle.decoder_layer(_f32(c["h"][rows]), w64, c["gate"][rows], pos[rows],
                                       _f32(c["k_cache"][b:b + 1]), _f32(c["v_cache"][b:b + 1]), block, nh, nkv,
                                       ctx_lens=lens[b:b + 1])
        err = row_relerr(got[rows], ref)
        m = min(block, cap - lens[b])
        new = slice(lens[b], lens[b] + m)
        kerr = row_relerr(_f32(kbits[b, new]), st["k"][:m])
        verr = row_relerr(_f32(vbits[b, new]), st["v"][:m])
        say(f"  seq {b} (len {lens[b]}): hidden row rel err {err:.3g}, appended k {kerr:.3g}, v {verr:.3g}")
        assert err <= LAYER_BAR and kerr <= 2e-2 and verr <= 2e-2
    # rows outside each sequence's append are untouched, for every sequence (bit for bit)
    for b in range(batch):
        m = min(block, cap - lens[b])
        keep = np.ones(cap, bool)
        keep[lens[b]:lens[b] + m] = False
        assert np.array_equal(kbits[b, keep], c["k_cache"][b, keep]), f"seq {b}: k rows outside the append"
        assert np.array_equal(vbits[b, keep], c["v_cache"][b, keep]), f"seq {b}: v rows outside the append"


@pytest.mark.parametrize("merged", [False, True])
def test_step_full_size_decode_loop_packed_adapters(gpu_lib, merged):
    """The launch configuration the bench times (merged: with gate-merged
    weights, as the bench runs it), with one layer: 128 sequences
    x (16 clean + 16 noisy) rows, caches of 8192 + 16 rows with 8192 valid
    (one sequence shorter), rank-128 adapters of q/k/v and gate/up stored back
    to back (grouped LoRA-down over the noisy rows only), V = 151,936, a
    carried q.  Every sampling decision of all 128 sequences is checked on the
    GPU's own logits; the oracle recomputes 2 sampled sequences: logits within
    the bar, committed lengths exact, committed rows within the bar."""
    import torch
    batch, block, cap, hidden, inter, nh, nkv, r, vocab = 128, 16, 8192 + 16, 4096, 12288, 32, 8, 128, 151936
    say(f"step decode loop full size, 1 layer, packed adapters: B={batch} block={block} cap={cap} V={vocab} "
        f"merged={merged}")
    c = workloads.step_case(batch, block, cap, hidden, inter, nh, nkv, r, 1, vocab, seed=17)
    lens = np.full(batch, 8192)
    lens[40] = 5000
    c["k_caches"][0] = _fill_slack(c["k_caches"][0], lens)
    c["v_caches"][0] = _fill_slack(c["v_caches"][0], lens)
    wt = {k: to_dev(v) for k, v in c["layers"][0].items() if not k.endswith("_f32")}
    for group in (("q", "k", "v"), ("g", "u")):
        cat = torch.cat([wt["a" + p] for p in group], dim=0).contiguous()
        for i, p in enumerate(group):
            wt["a" + p] = cat[i * r:(i + 1) * r]
    if merged:
        gpu_lib.merge_layer(wt)
    kc, vc = to_dev(c["k_caches"][0]), to_dev(c["v_caches"][0])
    cfg = gpu_lib.step_config(batch, block, cap, hidden, inter, nh, nkv, r, 1, vocab)
    cl = to_dev(lens.astype(np.int32))
    qx = workloads.rng_for(17, 907).standard_normal((batch, block - 1, vocab), dtype=np.float32) * np.float32(2.0)
    prev_q = workloads.bf16_bits(qx)
    out = gpu_lib.psi_spec_step(cfg, [gpu_lib.layer_weights(wt, kc, vc)], to_dev(c["embed"]), to_dev(c["final_norm"]),
                                to_dev(c["lm_head"]), to_dev(c["tokens"]), to_dev(c["u_draft"]),
                                to_dev(c["u_accept"]), to_dev(c["u_sample"]), prev_q=to_dev(prev_q), cache_len=cl,
                                next_tokens=True)
    torch.cuda.synchronize()
    gh = {name: to_host(v) for name, v in out.items()}
    lg = gh["logits"]
    acc = gh["accept_len"]
    assert np.all(np.isfinite(lg))
    np.testing.assert_array_equal(to_host(cl), lens + acc + 1)
    pq64 = _f32(prev_q)
    dties, ties = check_step_decisions(lg, block, c["tokens"], pq64, gh, c["u_draft"], c["u_accept"],
                                       c["u_sample"])
    say(f"  decisions of all {batch} sequences on the GPU's logits: near-ties drafts {dties} of "
        f"{batch * (block - 1)} draws, accepts/tokens {ties} of {batch}")
    # near-uniform rows of 151,936 tokens give each token a mass below the
    # 1e-5 tie band, so fp32 CDF rounding puts a few percent of draws in it
    assert ties <= 4 and dties <= batch * (block - 1) // 20
    w64 = _host_layers(c)
    n = 2 * block
    for b in (40, 101):
        sl = slice(b, b + 1)
        ref = oracle.decode_step(c["tokens"][sl], _f32(c["embed"]), w64, [_f32(c["k_caches"][0][sl])],
                                 [_f32(c["v_caches"][0][sl])], _f32(c["final_norm"]), _f32(c["lm_head"]), pq64[sl],
                                 c["u_draft"][sl], c["u_accept"][sl], c["u_sample"][sl], block, nh, nkv,
                                 cache_len=lens[sl])
        err = row_relerr(lg[b * n:(b + 1) * n], ref["logits"])
        kept = slice(lens[b], lens[b] + acc[b] + 1)
        kbits = kc[b, kept].view(torch.int16).cpu().numpy().view(np.uint16)
        kerr = row_relerr(_f32(kbits), ref["k_clean"][0][0, :acc[b] + 1])
        say(f"  seq {b} (len {lens[b]}): logits row rel err {err:.3g}, committed k row rel err {kerr:.3g}; "
            f"L gpu {acc[b]} oracle on its own logits {ref['accept_len'][0]}")
        assert err <= 2e-2 and kerr <= 2e-2
