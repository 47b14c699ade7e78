"""Oracle: Psi-Spec tree verify (per-node rejection).  Test infrastructure only.

Sources:
* Uno paper summary (hyper.ai, arXiv 2609.04010), section "方法", last
  paragraph: the tree sampler samples several candidates, verifies them
  concurrently as a prefix tree, and the procedure is lossless "in both
  cases" (linear and tree); the first token comes from the AR weights.
* ainews.surl.tw article on Uno: the tree sampler targets single-request
  latency; "lossless" means samples follow the AR distribution.

The pages do not spell out how a prefix tree is verified losslessly.  The
plainest lossless reading is the multi-candidate speculative sampling of
SpecInfer (Miao et al. 2023, "recursive rejection sampling"), computed here:

1. cur = root, r = softmax(p_root / T).
2. Visit the children of cur in ascending node id.  For child c with token t
   at depth delta, accept iff u_acc[c] * q_delta[t] < r[t].
   - accepted: append c to the path, cur = c, r = softmax(p_c / T), repeat 2;
   - rejected: r <- max(0, r - q_delta) / sum(...) (kept unchanged if the sum
     is 0), then try the next sibling.
3. When every child of cur was rejected, or cur has no children,
   y = inverse-CDF of r at u_s (for a leaf this is the bonus draw from p_cur).
   L = depth of cur.

Readings:
* siblings are i.i.d. draws from the per-depth marginal q_delta, with
  replacement (duplicates allowed) -- the condition for the rule above to be
  lossless;
* q is one row per depth (delta = 1..max_depth -> q row delta-1), shared by
  siblings; p is one AR row per node, scoring that node's children;
* accept comparison and inverse-CDF follow the linear sampler's conventions.

Without replacement (siblings drawn with the earlier siblings' tokens removed,
oracle/tree_build.py): sibling j is tested against q_j, the per-depth
marginal with the tokens of the siblings tried before it removed and the rest
renormalised, and a rejection subtracts q_j: r <- max(0, r - q_j) / sum
(recursive rejection sampling without replacement, Jeon et al. 2024).  A
residual with zero mass stays as it is for the node's remaining siblings.
"""

import numpy as np

from .verify_linear import softmax_rows, inverse_cdf


def node_depths(parent):
    parent = [int(x) for x in np.asarray(parent).reshape(-1)]
    depth = [0] * len(parent)
    for i in range(1, len(parent)):
        depth[i] = depth[parent[i]] + 1
    return depth


def children_lists(parent):
    parent = [int(x) for x in np.asarray(parent).reshape(-1)]
    ch = [[] for _ in parent]
    for i in range(1, len(parent)):
        ch[parent[i]].append(i)
    return ch


def _verify_one(parent, tokens, p_logits, q_logits, u_accept, u_s, temperature, without_replacement=False):
    depth = node_depths(parent)
    kids = children_lists(parent)
    max_depth = q_logits.shape[0]
    cur = 0
    r = softmax_rows(p_logits[0], temperature)
    path = []
    visited = []            # (node, accepted) in visiting order; diagnostic
    while True:
        moved = False
        removed = []             # tokens of the siblings rejected so far (without replacement)
        frozen = False
        for c in kids[cur]:
            dl = depth[c]
            assert 1 <= dl <= max_depth
            qd = softmax_rows(q_logits[dl - 1], temperature)
            if without_replacement:
                qd = qd.copy()
                for t_old in removed:
                    qd[t_old] = 0.0
                z = float(np.sum(qd))
                qd = qd / z if z > 0.0 else qd
            t = int(tokens[c])
            ok = u_accept[c] * qd[t] < r[t]
            visited.append((c, bool(ok)))
            if ok:
                path.append(c)
                cur = c
                r = softmax_rows(p_logits[c], temperature)
                moved = True
                break
            removed.append(t)
            if frozen:
                continue
            w = np.maximum(0.0, r - qd)
            s = float(np.sum(w))
            if s > 0.0:
                r = w / s
            elif without_replacement:
                frozen = True
        if not moved:
            break
    y = inverse_cdf(r, u_s)
    return len(path), path, y, visited


def verify_tree(parent, tokens, p_logits, q_logits, u_accept, u_sample, temperature=1.0,
                return_visited=False, without_replacement=False):
    """Verify a batch of candidate trees.

    parent   [B, n]  parent[b, 0] = -1, 0 <= parent[b, i] < i
    tokens   [B, n]  token of each node (root entry unused)
    p_logits [B, n, V]  AR row of each node (scores that node's children)
    q_logits [B, D, V]  draft marginal of depth 1..D
    u_accept [B, n], u_sample [B]

    Returns dict: accept_len [B], path [B, D] (node ids, -1 padded), token [B];
    with return_visited, also the per-batch list of (node, accepted) decisions.
    without_replacement: siblings were drawn without replacement (module doc).
    """
    parent = np.asarray(parent)
    tokens = np.asarray(tokens)
    p_logits = np.asarray(p_logits)
    q_logits = np.asarray(q_logits)
    u_accept = np.asarray(u_accept, dtype=np.float64)
    u_sample = np.asarray(u_sample, dtype=np.float64).reshape(-1)
    bsz, n = parent.shape
    dmax = q_logits.shape[1]
    acc = np.zeros(bsz, dtype=np.int64)
    paths = -np.ones((bsz, dmax), dtype=np.int64)
    ys = np.zeros(bsz, dtype=np.int64)
    visits = []
    for b in range(bsz):
        length, path, y, visited = _verify_one(parent[b], tokens[b], p_logits[b], q_logits[b],
                                               u_accept[b], u_sample[b], temperature, without_replacement)
        acc[b] = length
        paths[b, :length] = path
        ys[b] = y
        visits.append(visited)
    out = {"accept_len": acc, "path": paths, "token": ys}
    if return_visited:
        out["visited"] = visits
    return out
