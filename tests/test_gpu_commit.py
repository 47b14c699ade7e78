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
from _parity import row_relerr, say, to_dev, to_host

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
    say("kv_commit batch=300 capacity=50")
    import torch
    rng = workloads.rng_for(8)
    lens = rng.integers(0, 51, 300).astype(np.int32)
    acc = rng.integers(0, 16, 300).astype(np.int32)
    cl = to_dev(lens)
    gpu_lib.kv_commit(to_dev(acc), cl, 50)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_host(cl), np.minimum(50, lens + acc + 1))


def _positions(lens, block):
    return np.concatenate([np.concatenate([np.arange(block), np.arange(block)]) + n for n in lens]).astype(np.int32)


@pytest.mark.parametrize("batch,block,cap,lens", [
    (3, 4, 40, [0, 17, 38]),        # the last sequence has room for 2 of its 4 clean rows
    (2, 16, 300, [250, 5]),
])
def test_decoder_layer_appends_clean_rows(gpu_lib, batch, block, cap, lens):
    say(f"decoder layer with cache lengths B={batch} block={block} cap={cap} lens={lens}")
    import torch
    hidden, inter, nh, nkv, r = 256, 512, 4, 2, 16
    c = workloads.decoder_layer_case(batch, block, cap, hidden, inter, nh, nkv, r, seed=block + cap)
    kc0 = _fill_slack(c["k_cache"], lens)
    vc0 = _fill_slack(c["v_cache"], lens)
    pos = _positions(lens, block)
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
    assert err <= 2e-2
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


def test_step_decode_loop_two_steps(gpu_lib):
    """Two chained steps on caches of per-sequence lengths: each step appends
    its clean rows and commits the kept ones; the second step attends over
    what the first committed.  The oracle runs the same two steps with the
    GPU's accepted lengths."""
    import torch
    batch, block, cap, hidden, inter, nh, nkv, r, nl, vocab = 3, 5, 48, 256, 512, 4, 2, 16, 2, 1001
    say(f"decode loop: 2 steps B={batch} block={block} cap={cap} layers={nl} V={vocab}")
    c = workloads.step_case(batch, block, cap, hidden, inter, nh, nkv, r, nl, vocab, seed=12)
    c2 = workloads.step_case(batch, block, cap, hidden, inter, nh, nkv, r, 0, vocab, seed=13)   # step-2 tokens
    lens = np.array([3, 20, 41])
    for l in range(nl):
        c["k_caches"][l] = _fill_slack(c["k_caches"][l], lens)
        c["v_caches"][l] = _fill_slack(c["v_caches"][l], lens)
    keep, layers, kcs, vcs = _step_layers(gpu_lib, c)
    cfg = gpu_lib.step_config(batch, block, cap, hidden, inter, nh, nkv, r, nl, vocab)
    dev = {k: to_dev(c[k]) for k in ("embed", "final_norm", "lm_head")}
    cl = to_dev(lens.astype(np.int32))

    w64 = [{k[:-4]: v.astype(np.float64) for k, v in lw.items() if k.endswith("_f32")} for lw in c["layers"]]
    ok_k = [_f32(x) for x in c["k_caches"]]
    ok_v = [_f32(x) for x in c["v_caches"]]
    o_len = lens.copy()
    for step, src in enumerate((c, c2)):
        out = gpu_lib.psi_spec_step(cfg, layers, dev["embed"], dev["final_norm"], dev["lm_head"],
                                    to_dev(src["tokens"]), to_dev(src["u_draft"]), to_dev(src["u_accept"]),
                                    to_dev(src["u_sample"]), cache_len=cl)
        torch.cuda.synchronize()
        g_acc = to_host(out["accept_len"])
        g_len = to_host(cl)
        ref = oracle.decode_step(src["tokens"], _f32(c["embed"]), w64, ok_k, ok_v, _f32(c["final_norm"]),
                                 _f32(c["lm_head"]), src["u_draft"], src["u_accept"], src["u_sample"], block, nh,
                                 nkv, cache_len=o_len)
        err = row_relerr(to_host(out["logits"]), ref["logits"])
        say(f"  step {step}: logits row rel err {err:.3g}; accepted gpu {g_acc.tolist()} "
            f"oracle {ref['accept_len'].tolist()}; lengths {o_len.tolist()} -> {g_len.tolist()}")
        assert err <= 2e-2
        assert np.all((g_acc >= 0) & (g_acc <= block - 1))
        new_len = None
        for l in range(nl):
            ok_k[l], ok_v[l], new_len = oracle.kv_commit(ok_k[l], ok_v[l], o_len, ref["k_clean"][l],
                                                         ref["v_clean"][l], g_acc)
        np.testing.assert_array_equal(g_len, new_len)
        worst = 0.0
        for l in range(nl):
            kg, vg = to_host(kcs[l]), to_host(vcs[l])
            for b in range(batch):
                old, kept = slice(0, o_len[b]), slice(o_len[b], new_len[b])
                # rows committed by an earlier step: as the GPU left them; the oracle's own
                # copies of those rows are compared at the step that wrote them
                assert np.all(np.isfinite(kg[b, old])) and np.all(np.isfinite(vg[b, old]))
                if new_len[b] > o_len[b]:
                    worst = max(worst, row_relerr(kg[b, kept], ok_k[l][b, kept]),
                                row_relerr(vg[b, kept], ok_v[l][b, kept]))
                # the initial rows are never rewritten
                assert np.array_equal(kg[b, :lens[b]], _f32(c["k_caches"][l][b, :lens[b]]))
                assert np.array_equal(vg[b, :lens[b]], _f32(c["v_caches"][l][b, :lens[b]]))
        say(f"  step {step}: committed k/v row rel err {worst:.3g}")
        assert worst <= 2e-2
        o_len = new_len


def test_decoder_layer_full_size_decode_loop_sampled(gpu_lib):
    """One Qwen3-8B-shaped layer in the launch configuration the bench times:
    128 sequences x (16 clean + 16 noisy) rows, caches of 8192 + 16 rows with
    8192 valid (two sequences shorter), adapters back to back; the oracle
    recomputes 2 sampled sequences, their appended rows are checked, and every
    sequence's rows outside its append are unchanged."""
    import torch
    batch, block, cap = 128, 16, 8192 + 16
    hidden, inter, nh, nkv, r = 4096, 12288, 32, 8, 128
    say(f"decoder layer decode loop B={batch} block={block} cap={cap} Qwen3-8B shapes (sampled)")
    c = workloads.decoder_layer_case(batch, block, cap, hidden, inter, nh, nkv, r, seed=4)
    lens = np.full(batch, 8192)
    lens[5], lens[120] = 6001, 8191          # a ragged tail, and a sequence with room for 1 of its 16 rows
    for name in ("k_cache", "v_cache"):
        c[name] = _fill_slack(c[name], lens)
    pos = _positions(lens, block)
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
    for b in (5, 120, 77):
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
        assert err <= 2e-2 and kerr <= 2e-2 and verr <= 2e-2
    # rows outside each sequence's append are untouched, for every sequence (bit for bit)
    for b in range(batch):
        m = min(block, cap - lens[b])
        keep = np.ones(cap, bool)
        keep[lens[b]:lens[b] + m] = False
        assert np.array_equal(kbits[b, keep], c["k_cache"][b, keep]), f"seq {b}: k rows outside the append"
        assert np.array_equal(vbits[b, keep], c["v_cache"][b, keep]), f"seq {b}: v rows outside the append"


def test_step_full_size_decode_loop_packed_adapters(gpu_lib):
    """The launch configuration the bench times, with one layer: 128 sequences
    x (16 clean + 16 noisy) rows, caches of 8192 + 16 rows with 8192 valid
    (one sequence shorter), rank-128 adapters of q/k/v and gate/up stored back
    to back (grouped LoRA-down over the noisy rows only), V = 151,936.  The
    oracle recomputes 2 sampled sequences: logits within the bar, committed
    lengths exact, committed rows within the bar."""
    import torch
    batch, block, cap, hidden, inter, nh, nkv, r, vocab = 128, 16, 8192 + 16, 4096, 12288, 32, 8, 128, 151936
    say(f"step decode loop full size, 1 layer, packed adapters: B={batch} block={block} cap={cap} V={vocab}")
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
    kc, vc = to_dev(c["k_caches"][0]), to_dev(c["v_caches"][0])
    cfg = gpu_lib.step_config(batch, block, cap, hidden, inter, nh, nkv, r, 1, vocab)
    cl = to_dev(lens.astype(np.int32))
    out = gpu_lib.psi_spec_step(cfg, [gpu_lib.layer_weights(wt, kc, vc)], to_dev(c["embed"]), to_dev(c["final_norm"]),
                                to_dev(c["lm_head"]), to_dev(c["tokens"]), to_dev(c["u_draft"]),
                                to_dev(c["u_accept"]), to_dev(c["u_sample"]), cache_len=cl)
    torch.cuda.synchronize()
    lg = to_host(out["logits"])
    acc = to_host(out["accept_len"])
    assert np.all(np.isfinite(lg))
    np.testing.assert_array_equal(to_host(cl), np.minimum(cap, lens + acc + 1))
    w64 = [{k[:-4]: v.astype(np.float64) for k, v in c["layers"][0].items() if k.endswith("_f32")}]
    n = 2 * block
    for b in (40, 101):
        sl = slice(b, b + 1)
        ref = oracle.decode_step(c["tokens"][sl], _f32(c["embed"]), w64, [_f32(c["k_caches"][0][sl])],
                                 [_f32(c["v_caches"][0][sl])], _f32(c["final_norm"]), _f32(c["lm_head"]),
                                 c["u_draft"][sl], c["u_accept"][sl], c["u_sample"][sl], block, nh, nkv,
                                 cache_len=lens[sl])
        err = row_relerr(lg[b * n:(b + 1) * n], ref["logits"])
        kept = slice(lens[b], lens[b] + acc[b] + 1)
        kbits = kc[b, kept].view(torch.int16).cpu().numpy().view(np.uint16)
        kerr = row_relerr(_f32(kbits), ref["k_clean"][0][0, :acc[b] + 1])
        say(f"  seq {b} (len {lens[b]}): logits row rel err {err:.3g}, committed k row rel err {kerr:.3g}; "
            f"L gpu {acc[b]} oracle {ref['accept_len'][0]}")
        assert err <= 2e-2 and kerr <= 2e-2
