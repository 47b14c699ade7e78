"""Exact output law of a uniform-driven sampler, by black-box bisection.

The verify samplers are deterministic functions of pre-drawn uniforms: each
visited decision compares one uniform against a threshold, and the final draw
is monotone in u_s.  Treating the sampler as a black box, the exact
probability of every outcome is recovered by

* bisection on each visited decision's uniform (holding earlier decisions at a
  representative point inside their chosen interval), which yields the
  acceptance threshold of that decision, and
* bisection on u_s for the boundaries of the final token's inverse CDF.

Nothing of the sampler's arithmetic is re-implemented here; only the call
interface is used.  Thresholds are found to ~2^-50, far below the 1e-12 the
tests ask of the resulting law.
"""

import numpy as np

BISECT_STEPS = 52


def _bisect(pred_batch, n):
    """For each of n monotone predicates (true on [0, t), false on [t, 1]),
    return t.  pred_batch(u[n]) -> bool[n]."""
    lo = np.zeros(n)
    hi = np.ones(n)
    top = pred_batch(np.ones(n))          # predicate true even at u = 1 -> t = 1
    for _ in range(BISECT_STEPS):
        mid = 0.5 * (lo + hi)
        ok = pred_batch(mid)
        lo = np.where(ok, mid, lo)
        hi = np.where(ok, hi, mid)
    t = 0.5 * (lo + hi)
    return np.where(top, 1.0, t)


def explore(cases, run, n_uacc, vocab):
    """Enumerate the outcomes of a uniform-driven sampler.

    cases: number of independent input cases (batched through `run`).
    run(case_idx[B], u_acc[B, n_uacc], u_s[B]) -> list over B of
        (visited [(slot, accepted)], emitted_prefix tuple, y)
    Returns list over cases of [(weight, emitted_prefix, y_prob[vocab])] for
    every leaf with non-zero weight; sum of weights per case is 1.
    """
    # a state: (case, fixed {slot: u}, weight)
    frontier = [(c, {}, 1.0) for c in range(cases)]
    leaves = [[] for _ in range(cases)]
    while frontier:
        idx = np.array([s[0] for s in frontier])
        base = np.full((len(frontier), n_uacc), 0.5)
        for j, (_, fixed, _) in enumerate(frontier):
            for slot, u in fixed.items():
                base[j, slot] = u
        res = run(idx, base, np.full(len(frontier), 0.5))
        open_slot = []
        for j, (_, fixed, _) in enumerate(frontier):
            nxt = None
            for slot, _acc in res[j][0]:
                if slot not in fixed:
                    nxt = slot
                    break
            open_slot.append(nxt)
        done = [j for j, s in enumerate(open_slot) if s is None]
        todo = [j for j, s in enumerate(open_slot) if s is not None]
        # leaves: law of y by bisection on u_s boundaries
        if done:
            nd = len(done)
            cidx = np.repeat(idx[done], vocab)
            ub = np.repeat(base[done], vocab, axis=0)
            vv = np.tile(np.arange(vocab), nd)

            def pred_y(us):
                r = run(cidx, ub, us)
                return np.array([r[i][2] <= vv[i] for i in range(len(r))])

            cdf = _bisect(pred_y, nd * vocab).reshape(nd, vocab)
            cdf[:, -1] = 1.0
            for t, j in enumerate(done):
                py = np.diff(np.concatenate([[0.0], cdf[t]]))
                c, _fixed, wgt = frontier[j]
                leaves[c].append((wgt, tuple(res[j][1]), py))
        if not todo:
            break
        nt = len(todo)
        slots = np.array([open_slot[j] for j in todo])
        ubase = base[todo].copy()
        tidx = idx[todo]

        def pred_acc(u):
            ua = ubase.copy()
            ua[np.arange(nt), slots] = u
            r = run(tidx, ua, np.full(nt, 0.5))
            out = []
            for i in range(nt):
                acc = [a for s, a in r[i][0] if s == slots[i]]
                out.append(bool(acc[0]))
            return np.array(out)

        theta = _bisect(pred_acc, nt)
        new_frontier = []
        for t, j in enumerate(todo):
            c, fixed, wgt = frontier[j]
            th = theta[t]
            if th > 0.0:
                f = dict(fixed)
                f[int(slots[t])] = 0.5 * th
                new_frontier.append((c, f, wgt * th))
            if th < 1.0:
                f = dict(fixed)
                f[int(slots[t])] = 0.5 * (1.0 + th)
                new_frontier.append((c, f, wgt * (1.0 - th)))
        frontier = new_frontier
    return leaves


def emitted_law(leaves_by_case, case_weight, vocab):
    """Aggregate leaves into per-prefix laws.

    Returns {prefix tuple: (reach probability, emit[vocab])}: reach = P(the
    step emits a token at position len(prefix) after emitting `prefix`),
    emit[v] = P(that token is v and the prefix was emitted).
    """
    table = {}
    for c, leaves in enumerate(leaves_by_case):
        for wgt, prefix, py in leaves:
            w = case_weight[c] * wgt
            for j in range(len(prefix) + 1):
                key = tuple(prefix[:j])
                reach, emit = table.setdefault(key, [0.0, np.zeros(vocab)])
                if j < len(prefix):
                    table[key][0] += w
                    emit[prefix[j]] += w
                else:
                    table[key][0] += w
                    emit += w * py
    return table
