"""Oracle: candidate-tree construction from the per-depth draft marginals.
Test infrastructure only.

Sources: Uno summary (hyper.ai, arXiv 2609.04010), section "方法", last
paragraph: the tree sampler samples several candidates from the marginal
distributions of the diffusion path and verifies them as a prefix tree,
losslessly.  The pages fix neither the tree's shape nor how the candidates
are drawn.  Readings:

* The shape is a budget per depth: every node at depth d has branching[d]
  children (depth 0 = the root, the block's AR token), laid out breadth
  first, so the node count is 1 + b0 + b0 b1 + ... .
* The children of a node at depth d draw their tokens from the draft marginal
  of depth d + 1 (q row d), each with its own uniform u[child], by the same
  inverse CDF as every other draw (smallest token id whose cumulative mass
  exceeds u times the total).
* With replacement: siblings are independent draws (duplicates possible);
  the tree verify of oracle/verify_tree.py is lossless for such siblings.
* Without replacement: sibling j draws from q with the tokens of siblings
  1..j-1 removed and the rest renormalised (no duplicates); it needs the
  verifier that removes the same tokens (verify_tree(without_replacement=True)).
  When every token of positive mass has been drawn already (the remaining
  mass is zero; the pages have no such case), the draw is the smallest token
  id not drawn yet, so siblings stay distinct.
"""

import numpy as np

from .verify_linear import inverse_cdf, softmax_rows


def tree_layout(branching):
    """Parent array of the breadth-first tree with the given branching per
    depth; also the depth of every node."""
    parent = [-1]
    depth = [0]
    level = [0]
    for d, b in enumerate(branching):
        nxt = []
        for node in level:
            for _ in range(int(b)):
                parent.append(node)
                depth.append(d + 1)
                nxt.append(len(parent) - 1)
        level = nxt
    return np.array(parent, dtype=np.int64), np.array(depth, dtype=np.int64)


def draw_without(q, removed, u):
    """Inverse-CDF draw from q with the tokens in `removed` taken out (the rest
    keeps its relative mass)."""
    w = np.asarray(q, dtype=np.float64).copy()
    for t in removed:
        w[int(t)] = 0.0
    if not np.sum(w) > 0.0:
        taken = {int(t) for t in removed}
        return next(v for v in range(w.size) if v not in taken)
    return inverse_cdf(w, u)


def build_tree(q_logits, branching, u, temperature=1.0, without_replacement=False):
    """One candidate tree.

    q_logits [D][V]  the draft marginal of depth 1..D (row d for the children
                     of depth-d nodes); branching [D]; u [n] uniforms in [0, 1)
                     (u[0], the root's, is unused).
    Returns (parent [n], tokens [n]) with tokens[0] = -1 (the root's token is
    the caller's).
    """
    parent, depth = tree_layout(branching)
    n = len(parent)
    q = [softmax_rows(r, temperature) for r in np.asarray(q_logits)]
    tokens = np.full(n, -1, dtype=np.int64)
    siblings = {}
    for v in range(1, n):
        d = int(depth[v]) - 1                      # q row of this node's draw
        got = siblings.setdefault(int(parent[v]), [])
        if without_replacement:
            tokens[v] = draw_without(q[d], got, u[v])
        else:
            tokens[v] = inverse_cdf(q[d], u[v])
        got.append(int(tokens[v]))
    return parent, tokens
