"""Oracle: sampling transforms for the verify (temperature, top-k, top-p,
greedy).  Test infrastructure only.

Sources: 4sapi.net blog on Uno, its checklist of pitfalls (re-run the
comparison with a changed temperature / top_p: the sampling settings change
the target distribution); Uno summary (hyper.ai, arXiv 2609.04010), section
"方法", last paragraph (the verify is lossless with respect to the AR
distribution).  With a sampling transform the distribution the AR model
samples from is the transformed one, so the lossless verify is speculative
sampling between the transformed AR rows p~ = T(p) and the transformed draft
rows q~ = T(q), drafts drawn from q~.

Readings (the pages name the settings but define none of them; these are the
plainest ones, each stated so that the GPU can reach the same set exactly):

* temperature t > 0: p = softmax(l / t).
* top-k (k >= 1; 0 = off): keep every token whose logit is at least the k-th
  largest logit of the row (ties at the boundary are all kept, so the kept
  set is closed under equal logits and may hold more than k tokens), then
  renormalise.
* top-p (0 < top_p <= 1; 1 = off), applied after top-k on the renormalised
  top-k distribution p': keep token v iff the mass of the tokens with a
  strictly larger logit is below top_p, sum_{u: l_u > l_v} p'_u < top_p
  (the smallest set of whole tie groups, largest logits first, whose mass
  reaches top_p), then renormalise.
* greedy: p~ = one-hot at the smallest token id with the largest logit;
  temperature, top-k and top-p do not apply.

The kept set is read off the logits (equal logits, equal fate), so a
temperature never changes which tokens top-k keeps.
"""

import numpy as np

from .verify_linear import softmax_rows


def kth_largest(logits, k):
    """The k-th largest value of a row (k >= 1, counting repeats)."""
    x = np.sort(np.asarray(logits, dtype=np.float64))[::-1]
    return float(x[min(k, x.size) - 1])


def top_k_mask(logits, k):
    """Tokens kept by top-k: logit >= the k-th largest logit (k <= 0: all)."""
    x = np.asarray(logits, dtype=np.float64)
    if k <= 0 or k >= x.size:
        return np.ones(x.shape, dtype=bool)
    return x >= kth_largest(x, k)


def top_p_mask(logits, probs, top_p):
    """Tokens kept by top-p on the distribution probs (zero outside the
    earlier filter): the mass of strictly larger logits is below top_p."""
    x = np.asarray(logits, dtype=np.float64)
    p = np.asarray(probs, dtype=np.float64)
    if top_p >= 1.0:
        return p > 0.0
    # distinct logits in decreasing order, and the mass strictly above each
    vals, inv = np.unique(-x, return_inverse=True)      # ascending in -x = descending in x
    group_mass = np.bincount(inv, weights=p, minlength=vals.size)
    above = np.concatenate(([0.0], np.cumsum(group_mass)[:-1]))
    return (above[inv] < top_p) & (p > 0.0)


def transform_probs(logits, temperature=1.0, top_k=0, top_p=1.0, greedy=False):
    """The transformed distribution of one logit row (float64, sums to 1)."""
    x = np.asarray(logits, dtype=np.float64)
    out = np.zeros(x.shape, dtype=np.float64)
    if greedy:
        out[int(np.argmax(x))] = 1.0       # numpy's argmax takes the first maximum
        return out
    p = softmax_rows(x, temperature)
    keep = top_k_mask(x, top_k)
    p = np.where(keep, p, 0.0)
    p = p / np.sum(p)
    if top_p < 1.0:
        keep = top_p_mask(x, p, top_p)
        p = np.where(keep, p, 0.0)
        p = p / np.sum(p)
    return p
