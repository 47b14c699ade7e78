"""Pins of the KV-commit oracle (oracle.kv_commit) and of per-sequence cache
lengths in the attention, layer and step oracles.

Source: Uno summary (hyper.ai, arXiv 2609.04010), section 方法 (verify the
block on the AR path and keep the longest valid prefix; the block's first
token comes from the AR weights alone) and section 实验 (one KV cache shared
by drafting and verification).  The pins tie the commit to what the shared
cache must hold afterwards: the keys and values an AR-only decoder computes
when it takes the kept tokens one at a time.  Ragged lengths are tied to a
cache cut to each sequence's length, and to the one-key closed form.
"""

import numpy as np

import oracle
import workloads

rng = np.random.default_rng(4242)


def _f64(bits):
    return workloads.bf16_to_f32(bits).astype(np.float64)


def test_commit_writes_kept_rows_only():
    """Rows are tagged 1000*b + slot; the commit must put clean rows 0..L after
    each sequence's length and leave every other row alone.  A sequence whose
    kept rows do not all fit the capacity, or that is already flagged
    (L = -1), keeps nothing and is flagged."""
    bsz, cap, block, hkv, d = 6, 10, 4, 2, 3
    kc = np.zeros((bsz, cap, hkv, d))
    for b in range(bsz):
        kc[b] = (1000 * b + np.arange(cap))[:, None, None]
    vc = -kc
    kcl = np.zeros((bsz, block, hkv, d))
    for b in range(bsz):
        kcl[b] = (-(100 * b + np.arange(block) + 1))[:, None, None]
    vcl = 7.0 * kcl
    lens = np.array([0, 3, 8, 10, 6, 2])
    acc = np.array([2, 0, 3, 1, 3, -1])
    k2, v2, l2, a2 = oracle.kv_commit(kc, vc, lens, kcl, vcl, acc)
    # 8 + 4 > 10 and 10 + 2 > 10 do not fit; 6 + 4 = 10 fits exactly; -1 stays flagged
    np.testing.assert_array_equal(l2, [3, 4, 8, 10, 10, 2])
    np.testing.assert_array_equal(a2, [2, 0, -1, -1, 3, -1])
    for b in range(bsz):
        for s in range(cap):
            j = s - lens[b]
            if a2[b] >= 0 and 0 <= j <= a2[b]:
                assert np.all(k2[b, s] == kcl[b, j]) and np.all(v2[b, s] == vcl[b, j])
            else:
                assert np.all(k2[b, s] == kc[b, s]) and np.all(v2[b, s] == vc[b, s])
    # inputs untouched
    assert kc[0, 0, 0, 0] == 0 and kc[1, 3, 0, 0] == 1003 and acc[2] == 3


def test_ragged_attention_equals_cut_cache():
    """A sequence with ctx_lens[b] valid rows attends as if its cache had
    exactly those rows; whatever sits in the unused capacity is ignored."""
    bsz, block, nh, nkv, d, cap = 3, 3, 4, 2, 128, 9
    n = 2 * block
    q = rng.standard_normal((bsz, n, nh, d))
    kc = rng.standard_normal((bsz, cap, nkv, d))
    vc = rng.standard_normal((bsz, cap, nkv, d))
    kb = rng.standard_normal((bsz, n, nkv, d))
    vb = rng.standard_normal((bsz, n, nkv, d))
    lens = np.array([9, 4, 0])
    for b in range(bsz):
        kc[b, lens[b]:] = 1.0e3       # large, finite: any leak would dominate the softmax
        vc[b, lens[b]:] = -1.0e3
    out, lse = oracle.block_attention(q, kc, vc, kb, vb, block, 0.1, ctx_lens=lens)
    for b in range(bsz):
        c = lens[b]
        o1, l1 = oracle.block_attention(q[b:b + 1], kc[b:b + 1, :c], vc[b:b + 1, :c], kb[b:b + 1], vb[b:b + 1],
                                        block, 0.1)
        np.testing.assert_allclose(out[b], o1[0], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(lse[b], l1[0], rtol=1e-12, atol=1e-12)
    # empty cache: clean row 0 sees one key, its own, so its output is that key's value row
    # and its lse is that single score
    for h in range(nh):
        g = h // (nh // nkv)
        np.testing.assert_allclose(out[2, 0, h], vb[2, 0, g], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(lse[2, 0, h], 0.1 * q[2, 0, h] @ kb[2, 0, g], rtol=1e-12, atol=1e-12)


def test_step_rows_per_sequence_positions():
    gate, pos = oracle.step_rows(2, 3, np.array([5, 9]))
    np.testing.assert_array_equal(gate, [0, 0, 0, 1, 1, 1] * 2)
    np.testing.assert_array_equal(pos, [5, 6, 7, 8, 9, 10, 9, 10, 11, 12, 13, 14])


def _tiny_model(n_layers=2, vocab=53, hidden=64, inter=64, nh=2, nkv=1, r=8, bsz=2, cap=12, seed=3):
    c = workloads.step_case(bsz, 4, cap, hidden, inter, nh, nkv, r, n_layers, vocab, seed=seed)
    layers = [{k[:-4]: v.astype(np.float64) for k, v in lw.items() if k.endswith("_f32")} for lw in c["layers"]]
    return c, layers


def _ar_one_token(c, layers, kcs, vcs, lens, tok):
    """One AR-only step per sequence on a single clean token (block 1, no
    draft verified); returns its clean-row logits and the caches with that
    token's keys and values kept."""
    bsz = len(lens)
    toks = np.stack([tok, tok], axis=1)               # block 1: the noisy row is a copy, gate 1
    z = np.zeros((bsz, 0))
    out = oracle.decode_step(toks, _f64(c["embed"]), layers, kcs, vcs, _f64(c["final_norm"]), _f64(c["lm_head"]),
                             None, z, z, np.full(bsz, 0.5), 1, c["n_heads"], c["n_kv_heads"], cache_len=lens)
    nk, nv = [], []
    for l in range(len(layers)):
        k2, v2, l2, _ = oracle.kv_commit(kcs[l], vcs[l], lens, out["k_clean"][l], out["v_clean"][l],
                                         np.zeros(bsz, dtype=int))
        nk.append(k2)
        nv.append(v2)
    return out["logits"].reshape(bsz, 2, -1)[:, 0], nk, nv, l2


def test_block_pass_then_commit_equals_ar_token_by_token():
    """Shared-cache consistency: one concatenated clean + noisy pass followed by
    kv_commit(L) leaves every layer's cache as an AR-only decoder leaves it
    after taking the kept tokens 0..L one at a time, and the clean rows'
    logits are that decoder's logits.  A noisy row leaking into a clean row,
    a wrong position or an off-by-one in the kept rows fails this."""
    c, layers = _tiny_model()
    block, bsz = c["block"], c["batch"]
    kcs = [_f64(x) for x in c["k_caches"]]
    vcs = [_f64(x) for x in c["v_caches"]]
    lens = np.array([3, 7])
    for l in range(len(layers)):
        for b in range(bsz):
            kcs[l][b, lens[b]:] = 50.0   # unused capacity: must never be read
            vcs[l][b, lens[b]:] = -50.0
    out = oracle.decode_step(c["tokens"], _f64(c["embed"]), layers, kcs, vcs, _f64(c["final_norm"]),
                             _f64(c["lm_head"]), None, c["u_draft"], c["u_accept"], c["u_sample"], block,
                             c["n_heads"], c["n_kv_heads"], cache_len=lens)
    clean_logits = out["logits"].reshape(bsz, 2 * block, -1)[:, :block]
    for acc in (np.array([3, 1]), np.array([0, 2]), out["accept_len"]):
        blk_k, blk_v = [], []
        for l in range(len(layers)):
            k2, v2, l2, _ = oracle.kv_commit(kcs[l], vcs[l], lens, out["k_clean"][l], out["v_clean"][l], acc)
            blk_k.append(k2)
            blk_v.append(v2)
        np.testing.assert_array_equal(l2, lens + acc + 1)
        # AR-only, one token at a time; a sequence stops taking tokens after its L + 1
        ar_k, ar_v, ar_len = [x.copy() for x in kcs], [x.copy() for x in vcs], lens.copy()
        for j in range(block):
            live = acc >= j
            if not live.any():
                break
            tok = c["tokens"][:, j]
            lg, nk, nv, nl = _ar_one_token(c, layers, ar_k, ar_v, ar_len, tok)
            for b in np.nonzero(live)[0]:
                np.testing.assert_allclose(lg[b], clean_logits[b, j], rtol=0, atol=2e-2 * np.abs(lg[b]).max())
                for l in range(len(layers)):
                    ar_k[l][b], ar_v[l][b] = nk[l][b], nv[l][b]
                ar_len[b] = nl[b]
        np.testing.assert_array_equal(ar_len, l2)
        _same_cache(ar_k, ar_v, blk_k, blk_v, l2)


def _same_cache(ar_k, ar_v, k, v, lens):
    """The kept prefix of each cache holds the same bf16-rounded values, up to
    the rare rounding flip of a float64 sum taken in another order."""
    for l in range(len(k)):
        for b in range(len(lens)):
            kept = slice(0, int(lens[b]))
            np.testing.assert_allclose(ar_k[l][b, kept], k[l][b, kept], rtol=2 ** -7, atol=1e-6)
            np.testing.assert_allclose(ar_v[l][b, kept], v[l][b, kept], rtol=2 ** -7, atol=1e-6)
            assert np.mean(ar_k[l][b, kept] == k[l][b, kept]) > 0.999
            assert np.mean(ar_v[l][b, kept] == v[l][b, kept]) > 0.999


def test_three_step_chain_commits_exactly_the_emitted_tokens():
    """The closed decode loop: three chained steps (the first without a
    carried q), each verifying the drafts the step before drew, against the q
    it drew them from.  After every step the shared cache must equal what an
    AR-only decoder leaves after taking the emitted token stream one token at
    a time (all of it but the newest y, which is the next block's first clean
    row), and the clean rows whose tokens were kept must carry that decoder's
    logits.  Sequence 0 accepts every draft (u_accept = 0), sequence 1 draws
    its uniforms, sequence 2 runs out of capacity at the third step and is
    flagged there."""
    c, layers = _tiny_model(bsz=3, cap=14)
    block, bsz, k = c["block"], c["batch"], c["block"] - 1
    kcs = [_f64(x) for x in c["k_caches"]]
    vcs = [_f64(x) for x in c["v_caches"]]
    lens = np.array([2, 5, 6])
    for l in range(len(layers)):
        for b in range(bsz):
            kcs[l][b, lens[b]:] = 50.0
            vcs[l][b, lens[b]:] = -50.0
    g = np.random.default_rng(11)
    uniforms = []
    for _ in range(3):
        ua = g.random((bsz, k))
        ua[0] = 0.0
        uniforms.append((g.random((bsz, k)), ua, g.random(bsz)))
    tokens0 = c["tokens"].copy()
    steps, fk, fv = oracle.decode_loop(tokens0, _f64(c["embed"]), layers, kcs, vcs, _f64(c["final_norm"]),
                                       _f64(c["lm_head"]), uniforms, block, c["n_heads"], c["n_kv_heads"], lens)
    acc = np.array([r["accept_len"] for r in steps])
    assert acc[0].tolist() == [0, 0, 0]                   # the first step verifies nothing
    assert acc[1, 0] == k and acc[2, 0] == k              # u_accept = 0 accepts every draft
    assert acc[2, 2] == -1 and steps[2]["token"][2] == -1  # 6 + 1 + 4 + 4 > 14
    stream = oracle.emitted_tokens(steps, tokens0)
    assert len(stream[0]) == 1 + 1 + (k + 1) * 2
    # AR-only decoder over each sequence's stream, one token at a time
    ar_k, ar_v, ar_len = [x.copy() for x in kcs], [x.copy() for x in vcs], lens.copy()
    ar_logits = [[] for _ in range(bsz)]
    n_max = max(len(s) for s in stream)
    for j in range(n_max - 1):
        live = np.array([j < len(stream[b]) - 1 for b in range(bsz)])
        tok = np.array([stream[b][j] if live[b] else 0 for b in range(bsz)])
        lg, nk, nv, nl = _ar_one_token(c, layers, ar_k, ar_v, ar_len, tok)
        for b in np.nonzero(live)[0]:
            ar_logits[b].append(lg[b])
            for l in range(len(layers)):
                ar_k[l][b], ar_v[l][b] = nk[l][b], nv[l][b]
            ar_len[b] = nl[b]
    final_len = steps[-1]["cache_len"]
    np.testing.assert_array_equal(ar_len, final_len)
    np.testing.assert_array_equal(final_len, [lens[b] + len(stream[b]) - 1 for b in range(bsz)])
    _same_cache(ar_k, ar_v, fk, fv, final_len)
    # each step's kept clean rows carry the AR decoder's logits at their stream position
    for t, r in enumerate(steps):
        lg = r["logits"].reshape(bsz, 2 * block, -1)
        for b in range(bsz):
            L = int(r["accept_len"][b])
            if L < 0:
                continue
            at = int((steps[t - 1]["cache_len"][b] if t else lens[b]) - lens[b])
            for j in range(L + 1):
                ref = ar_logits[b][at + j]
                np.testing.assert_allclose(lg[b, j], ref, rtol=0, atol=2e-2 * np.abs(ref).max())
    # the flagged sequence kept nothing at the step that did not fit
    assert steps[2]["cache_len"][2] == steps[1]["cache_len"][2]
