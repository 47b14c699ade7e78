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


def tree_outcome_near(parent, tokens, p, q, ua, us, temperature, gpu_out, tie=TIE, without=False):
    """True if perturbing one visited uniform (or u_s) by at most `tie` makes
    the oracle produce the GPU's (L, path, y): the GPU differs only on a
    near-tie decision."""
    kw = dict(without_replacement=without)
    base = oracle.verify_tree(parent[None], tokens[None], p[None], q[None], ua[None], np.array([us]),
                              temperature, return_visited=True, **kw)
    L, path, y = gpu_out

    def same(r):
        Lr = int(r["accept_len"][0])
        return Lr == L and list(r["path"][0, :Lr]) == list(path[:L]) and int(r["token"][0]) == y

    for node, _acc in base["visited"][0]:
        for delta in (-tie, tie):
            u2 = ua.copy()
            u2[node] = min(max(u2[node] + delta, 0.0), 1.0 - 1e-12)
            r = oracle.verify_tree(parent[None], tokens[None], p[None], q[None], u2[None], np.array([us]),
                                   temperature, **kw)
            if same(r):
                return True
    for delta in (-tie, tie):
        r = oracle.verify_tree(parent[None], tokens[None], p[None], q[None], ua[None],
                               np.array([min(max(us + delta, 0.0), 1.0 - 1e-12)]), temperature, **kw)
        if same(r):
            return True
    return False


def check_step_decisions(logits, block, tokens, prev_q, gpu, u_draft, u_accept, u_sample, temperature=1.0,
                         seqs=None, tie=TIE):
    """Every sampling decision of a decode step, checked against the oracle run
    on the GPU's own logits (so both sides decide on the same bf16 values):
    the drafts drawn from the noisy rows, the accepted length of the clean
    drafts against prev_q, and the correction/bonus token -- bit-exact except
    where a uniform lies within `tie` of its decision boundary (counted).

    logits [B * 2*block, V] (host values); tokens [B, 2*block]; prev_q
    [B, k, V] host values or None; gpu: dict of host arrays drafts [B, k],
    accept_len [B], token [B] (flagged sequences, accept_len -1, are skipped).
    Returns (draft near-ties: draft draws counted one by one, decision
    near-ties: sequences whose accepted length or token differed at a
    near-tie)."""
    bsz = np.asarray(tokens).shape[0]
    lg = np.asarray(logits).reshape(bsz, 2 * block, -1)     # converted to float64 a row at a time
    k = block - 1
    kv = k if prev_q is not None else 0
    draft_ties = ties = 0
    for b in (range(bsz) if seqs is None else seqs):
        for i in range(k):
            q = oracle.softmax_rows(lg[b, block + i], temperature)
            ref = oracle.inverse_cdf(q, u_draft[b, i])
            got = int(gpu["drafts"][b, i])
            if got != ref:
                assert draw_is_valid(q, float(u_draft[b, i]), got, tie), f"seq {b} draft {i}: gpu {got} oracle {ref}"
                draft_ties += 1
        if int(gpu["accept_len"][b]) < 0:
            continue
        pq = np.asarray(prev_q[b], dtype=np.float64)[None] if kv else np.zeros((1, 0, lg.shape[2]))
        o = oracle.verify_linear(lg[b:b + 1, :kv + 1].astype(np.float64), pq, np.asarray(tokens)[b:b + 1, 1:kv + 1],
                                 np.asarray(u_accept)[b:b + 1, :kv], np.asarray(u_sample)[b:b + 1], temperature)
        Lo, Lg = int(o["accept_len"][0]), int(gpu["accept_len"][b])
        if Lo != Lg:
            i = min(Lo, Lg)
            ratio = o["p_draft"][0, i] / o["q_draft"][0, i]
            assert abs(float(u_accept[b, i]) - ratio) < tie, f"seq {b}: L gpu {Lg} oracle {Lo}"
            ties += 1
            continue
        yo, yg = int(o["token"][0]), int(gpu["token"][b])
        if yo != yg:
            p = oracle.softmax_rows(lg[b, Lo], temperature)
            if Lo < kv:
                w, s = oracle.residual_weights(p, oracle.softmax_rows(pq[0, Lo], temperature))
                w = p if s == 0.0 else w
            else:
                w = p
            assert draw_is_valid(w, float(u_sample[b]), yg, tie), f"seq {b}: token gpu {yg} oracle {yo} (L={Lo})"
            ties += 1
    return draft_ties, ties


def top_p_margin(row, temperature, top_k, top_p):
    """Distance of a row's top-p boundary from deciding the other way: the
    smallest |mass strictly above a tie group - top_p| over the groups of the
    top-k renormalised distribution (inf when top-p is off)."""
    if top_p >= 1.0:
        return np.inf
    x = np.asarray(row, np.float64)
    p = oracle.softmax_rows(x, temperature)
    p = np.where(oracle.top_k_mask(x, top_k), p, 0.0)
    p = p / p.sum()
    vals, inv = np.unique(-x, return_inverse=True)
    gm = np.bincount(inv, weights=p, minlength=vals.size)
    above = np.concatenate(([0.0], np.cumsum(gm)[:-1]))
    live = gm > 0
    return float(np.min(np.abs(above[live] - top_p)))


def check_linear_sampled(case_rows, gpu, seqs, k, temperature, top_k, top_p, greedy, tie=TIE, prob_rtol=1e-5,
                         mass_atol=1e-5, cut_tie=1e-6):
    """check_linear under a sampling transform.  A sequence one of whose rows
    has its top-p boundary within cut_tie of flipping is counted as a tie
    (its kept set may resolve either way), as are the usual near-ties."""
    ties = 0
    kw = dict(top_k=top_k, top_p=top_p, greedy=greedy)
    for b in seqs:
        p, q, d, ua, us = case_rows(b)
        if not greedy and min(top_p_margin(r, temperature, top_k, top_p) for r in list(p) + list(q)) < cut_tie:
            ties += 1
            continue
        o = oracle.verify_linear(p[None], q[None], d[None], ua[None], np.array([us]), temperature, **kw)
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
            qd = o["q_draft"][0, i]
            ratio = o["p_draft"][0, i] / qd if qd > 0 else np.inf
            assert abs(float(ua[i]) - ratio) < tie, f"seq {b}: L gpu {Lg} oracle {Lo}, |u - p/q| = {abs(ua[i] - ratio):.3g}"
            ties += 1
            continue
        if "residual_mass" in gpu:
            err = abs(gpu["residual_mass"][b] - o["residual_mass"][0])
            assert err <= mass_atol, f"seq {b} residual mass err {err:.3g}"
        if yg != yo:
            pr = oracle.transform_probs(p[Lo], temperature, **kw)
            if Lo < k:
                w, s = oracle.residual_weights(pr, oracle.transform_probs(q[Lo], temperature, **kw))
                if s == 0.0:
                    w = pr
            else:
                w = pr
            assert draw_is_valid(w, us, yg, tie), f"seq {b}: token gpu {yg} oracle {yo} (L={Lo})"
            ties += 1
    return ties


def check_tree_build(q_logits, branching, u_draw, parent_gpu, tokens_gpu, temperature, without, tie=TIE):
    """Compare GPU-built trees with oracle.build_tree.

    q_logits [B, D, V] host values the GPU drew from; u_draw [B, n];
    parent_gpu, tokens_gpu [B, n] host arrays.  The parent arrays must equal
    the oracle's layout.  A token must equal the oracle's draw from the same
    reduced row -- q without the GPU's own earlier siblings when drawing
    without replacement -- except where u lies within `tie` of a CDF
    boundary of that row (counted and returned).  Without replacement the
    siblings must be distinct."""
    parent_ref, depth = oracle.tree_layout(branching)
    bsz, n = np.asarray(tokens_gpu).shape
    assert n == parent_ref.size
    ties = 0
    for b in range(bsz):
        assert list(parent_gpu[b]) == parent_ref.tolist(), f"tree {b}: parent array differs from the layout"
        assert int(tokens_gpu[b, 0]) == -1
        q = [oracle.softmax_rows(np.asarray(r, np.float64), temperature) for r in q_logits[b]]
        _, ref_tok = oracle.build_tree(q_logits[b], branching, u_draw[b], temperature, without)
        same = True
        kids = oracle.children_lists(parent_ref)
        for v in range(n):
            sib = kids[v]
            got_before = []
            for c in sib:
                d = int(depth[c]) - 1
                y = int(tokens_gpu[b, c])
                removed = got_before if without else []
                ref = oracle.draw_without(q[d], removed, u_draw[b, c]) if without else oracle.inverse_cdf(q[d], u_draw[b, c])
                if y != ref:
                    w = q[d].copy()
                    for t in removed:
                        w[int(t)] = 0.0
                    assert w.sum() > 0.0 and draw_is_valid(w, float(u_draw[b, c]), y, tie), \
                        f"tree {b} node {c}: gpu {y} oracle {ref} (removed {removed})"
                    ties += 1
                    same = False
                got_before.append(y)
            if without:
                toks = [int(tokens_gpu[b, c]) for c in sib]
                assert len(set(toks)) == len(toks), f"tree {b} node {v}: repeated sibling tokens {toks}"
        if same:
            assert np.array_equal(np.asarray(tokens_gpu[b]), ref_tok), f"tree {b}: tokens differ from build_tree"
    return ties
