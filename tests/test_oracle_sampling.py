"""Pins of the sampling transforms (oracle/sampling.py) and of the verify
under them.

Sources: 4sapi.net blog on Uno, checklist (temperature and top_p change the
target distribution); Uno summary (hyper.ai, arXiv 2609.04010), section 方法,
last paragraph (the verify is lossless with respect to the AR distribution,
here the transformed one).
"""

import itertools
import json
import math
import os

import numpy as np
import pytest
from scipy.special import softmax as sp_softmax

import oracle
from _exact_law import explore, emitted_law

HERE = os.path.dirname(os.path.abspath(__file__))


def test_handworked_golden_cases():
    with open(os.path.join(HERE, "golden", "sampling_handworked.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        lg = np.log(np.asarray(c["logits"], np.float64)) if c["log"] else np.asarray(c["logits"], np.float64)
        got = oracle.transform_probs(lg, c.get("temperature", 1.0), c.get("top_k", 0), c.get("top_p", 1.0),
                                     c.get("greedy", False))
        np.testing.assert_allclose(got, c["expect"], rtol=0, atol=1e-12, err_msg=c["name"])


def test_identity_settings():
    x = np.random.default_rng(0).normal(0, 2, 50)
    ref = sp_softmax(x / 0.7)
    for k, p in ((0, 1.0), (50, 1.0), (80, 1.0)):
        np.testing.assert_allclose(oracle.transform_probs(x, 0.7, k, p), ref, rtol=1e-13, atol=0)


def test_top_p_against_sorted_cumsum_without_ties():
    """Tie-free rows: the kept set is the shortest prefix of the tokens sorted
    by decreasing probability whose mass reaches top_p (the usual nucleus
    statement), an independent formulation of the mass-above rule."""
    rng = np.random.default_rng(1)
    for trial in range(200):
        V = int(rng.integers(2, 40))
        x = rng.normal(0, 2.0, V)
        top_p = float(rng.uniform(0.01, 0.999))
        p = sp_softmax(x)
        order = np.argsort(-p, kind="stable")
        cum = np.cumsum(p[order])
        last = int(np.searchsorted(cum, top_p, side="left"))      # first index with cum >= top_p
        keep = np.zeros(V, bool)
        keep[order[:last + 1]] = True
        got = oracle.transform_probs(x, top_p=top_p) > 0
        # a cumulative sum landing within rounding of top_p is a tie of the two statements
        if abs(cum[min(last, V - 1)] - top_p) < 1e-12 or (last > 0 and abs(cum[last - 1] - top_p) < 1e-12):
            continue
        np.testing.assert_array_equal(got, keep, err_msg=f"trial {trial}")


def test_top_k_counts_and_temperature_invariance():
    rng = np.random.default_rng(2)
    for trial in range(100):
        V = int(rng.integers(2, 60))
        x = rng.normal(0, 1.0, V)
        k = int(rng.integers(1, V + 1))
        kept = oracle.transform_probs(x, 1.0, k) > 0
        assert kept.sum() == k                                   # continuous logits: no ties
        assert np.array_equal(kept, oracle.transform_probs(x, 3.0, k) > 0)
        # ties: integer logits; the kept set is every token at or above the k-th value
        xi = rng.integers(-3, 3, V).astype(np.float64)
        kept = oracle.transform_probs(xi, 1.0, k) > 0
        kth = np.sort(xi)[::-1][k - 1]
        np.testing.assert_array_equal(kept, xi >= kth)
        assert kept.sum() >= k


def test_greedy_is_the_first_argmax():
    rng = np.random.default_rng(3)
    for _ in range(50):
        x = rng.integers(-2, 3, 20).astype(np.float64)
        g = oracle.transform_probs(x, greedy=True)
        assert g.sum() == 1.0 and g[int(np.flatnonzero(x == x.max())[0])] == 1.0


SETTINGS = [
    dict(top_k=2), dict(top_k=3, temperature=0.6), dict(top_p=0.6), dict(top_p=0.9, temperature=1.7),
    dict(top_k=3, top_p=0.7), dict(greedy=True),
]


@pytest.mark.parametrize("vocab,k,seed", [(4, 2, 0), (5, 2, 1), (3, 3, 2)])
@pytest.mark.parametrize("setting", SETTINGS, ids=lambda s: "_".join(f"{a}{b}" for a, b in s.items()))
def test_exhaustive_emitted_law_equals_transformed_ar(vocab, k, seed, setting):
    """Lossless under the transform: drafts drawn from the transformed draft
    rows, every emitted token follows the transformed AR row given the
    emitted prefix (exact law by bisection, every draft sequence weighted by
    its probability under the transformed draft rows)."""
    T = setting.get("temperature", 1.0)
    kw = dict(top_k=setting.get("top_k", 0), top_p=setting.get("top_p", 1.0), greedy=setting.get("greedy", False))
    rng = np.random.default_rng(200 + seed)
    ar = {}
    for j in range(k + 1):
        for pre in itertools.product(range(vocab), repeat=j):
            ar[pre] = rng.normal(0.0, 1.5, vocab)
    qlog = rng.normal(0.0, 1.5, (k, vocab))
    qt = np.stack([oracle.transform_probs(r, T, **kw) for r in qlog])
    dlist = [d for d in itertools.product(range(vocab), repeat=k) if np.prod([qt[i, d[i]] for i in range(k)]) > 0]
    drafts = np.array(dlist, dtype=np.int64)
    pl = np.stack([[ar[d[:i]] for i in range(k + 1)] for d in dlist])
    ql = np.broadcast_to(qlog, (len(dlist), k, vocab)).copy()
    weight = np.array([np.prod([qt[i, d[i]] for i in range(k)]) for d in dlist])

    def run(ci, ua, us):
        r = oracle.verify_linear(pl[ci], ql[ci], drafts[ci], ua, us, temperature=T, **kw)
        out = []
        for b in range(len(ci)):
            L = int(r["accept_len"][b])
            vis = [(i, True) for i in range(L)] + ([(L, False)] if L < k else [])
            out.append((vis, tuple(drafts[ci[b], :L]), int(r["token"][b])))
        return out

    leaves = explore(len(dlist), run, k, vocab)
    table = emitted_law(leaves, weight, vocab)
    assert () in table and abs(table[()][0] - 1.0) < 1e-12
    checked = 0
    for pre, (reach, emit) in table.items():
        if reach < 1e-14:
            continue
        np.testing.assert_allclose(emit / reach, oracle.transform_probs(ar[pre], T, **kw), rtol=0, atol=1e-12,
                                   err_msg=f"prefix {pre}")
        checked += 1
    assert checked >= (1 if kw["greedy"] else 2)


def test_verify_without_transform_is_unchanged():
    rng = np.random.default_rng(4)
    pl = rng.normal(0, 2, (3, 4, 30))
    ql = rng.normal(0, 2, (3, 3, 30))
    d = rng.integers(0, 30, (3, 3))
    ua, us = rng.random((3, 3)), rng.random(3)
    a = oracle.verify_linear(pl, ql, d, ua, us, 1.3)
    b = oracle.verify_linear(pl, ql, d, ua, us, 1.3, top_k=0, top_p=1.0, greedy=False)
    for key in a:
        np.testing.assert_array_equal(a[key], b[key])
