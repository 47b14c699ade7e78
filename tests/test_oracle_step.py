"""Pins of the whole-step oracle (oracle.decode_step) and of a chain of steps
(oracle.decode_loop).

Source: Uno summary (hyper.ai, arXiv 2609.04010), section 方法 (propose a
block on the diffusion path, verify it on the AR path, keep the longest
valid prefix; the first token of a block comes from the AR weights; lossless
acceleration).  The composition is tied to closed forms that do not go
through its own code: uniform distributions, a carried q equal to the target,
a target concentrated on one token, sequence independence, and -- for the
chain -- the exact law of the emitted tokens, which must be the AR model's.
"""

import itertools

import numpy as np
from scipy.special import softmax as sp_softmax

import oracle
from _exact_law import _bisect, emitted_law, explore

rng = np.random.default_rng(99)


def _zero_layer_case(bsz=3, block=4, vocab=37, hidden=32):
    embed = rng.choice([-1.0, 1.0], size=(vocab, hidden))
    w_lm = rng.integers(-8, 9, size=(vocab, hidden)) / 64.0
    tokens = rng.integers(0, vocab, size=(bsz, 2 * block))
    k = block - 1
    # uniforms kept away from the grid i / vocab so the closed forms below are exact
    ud = (rng.integers(0, vocab, size=(bsz, k)) + rng.uniform(0.1, 0.9, size=(bsz, k))) / vocab
    ua = rng.uniform(0.0, 1.0, size=(bsz, k))
    us = (rng.integers(0, vocab, size=bsz) + rng.uniform(0.1, 0.9, size=bsz)) / vocab
    return embed, w_lm, tokens, ud, ua, us


def _run(embed, w_lm, tokens, prev_q, ud, ua, us, block):
    return oracle.decode_step(tokens, embed, [], [], [], np.ones(embed.shape[1]), w_lm, prev_q, ud, ua, us, block,
                              4, 2)


def test_rows_layout():
    """Clean row j at ctx + j, noisy row j at ctx + block + j (the next block)."""
    gate, pos = oracle.step_rows(2, 3, 100)
    np.testing.assert_array_equal(gate, [0, 0, 0, 1, 1, 1] * 2)
    np.testing.assert_array_equal(pos, [100, 101, 102, 103, 104, 105] * 2)


def test_uniform_distributions_accept_everything_and_draw_by_floor():
    """A zero LM head gives uniform p and q: every carried draft is accepted
    (u/V < 1/V), every draw is floor(u * V), and the next step's ids are
    [y, new drafts, the same noisy ids]."""
    embed, w_lm, tokens, ud, ua, us = _zero_layer_case()
    vocab = w_lm.shape[0]
    prev_q = np.zeros((3, 3, vocab))
    out = _run(embed, np.zeros_like(w_lm), tokens, prev_q, ud, ua, us, 4)
    np.testing.assert_array_equal(out["drafts"], np.floor(ud * vocab).astype(int))
    np.testing.assert_array_equal(out["accept_len"], [3, 3, 3])
    np.testing.assert_array_equal(out["token"], np.floor(us * vocab).astype(int))
    np.testing.assert_array_equal(out["next_tokens"][:, 0], out["token"])
    np.testing.assert_array_equal(out["next_tokens"][:, 1:4], out["drafts"])
    np.testing.assert_array_equal(out["next_tokens"][:, 4:], tokens[:, 4:])


def test_logits_are_lm_head_of_normed_embeddings():
    """With no layers the logits are rmsnorm(embed[t]) . W^T, here exact: the
    +-1 embedding rows normalise to +-1 in bf16 and the products are dyadic.
    The carried q of the next step is this step's noisy rows 0..k-1."""
    embed, w_lm, tokens, ud, ua, us = _zero_layer_case()
    out = _run(embed, w_lm, tokens, None, ud, ua, us, 4)
    ref = embed[tokens.reshape(-1)] @ w_lm.T
    np.testing.assert_array_equal(out["logits"], ref)
    np.testing.assert_array_equal(out["q_next"], ref.reshape(3, 8, -1)[:, 4:7])


def test_first_step_verifies_nothing_and_draws_from_clean_row_zero():
    """Without a carried q: L = 0 and y is the inverse CDF of clean row 0 (a
    numpy cumsum here), whatever the clean ids 1..k hold."""
    embed, w_lm, tokens, ud, ua, us = _zero_layer_case()
    out = _run(embed, w_lm, tokens, None, ud, np.zeros_like(ua), us, 4)
    np.testing.assert_array_equal(out["accept_len"], [0, 0, 0])
    for b in range(3):
        c = np.cumsum(sp_softmax(embed[tokens[b, 0]] @ w_lm.T))
        assert out["token"][b] == int(np.searchsorted(c, us[b], side="right"))


def test_carried_q_equal_to_target_accepts_everything():
    """A carried q equal to the clean rows' own logits gives q_i = p_i, so L = k
    and y is the bonus draw from clean row k (written out with numpy here)."""
    block = 5
    embed, w_lm, tokens, ud, ua, us = _zero_layer_case(block=block)
    prev_q = (embed[tokens[:, :block - 1]] @ w_lm.T)
    out = _run(embed, w_lm, tokens, prev_q, ud, ua, us, block)
    np.testing.assert_array_equal(out["accept_len"], [block - 1] * 3)
    for b in range(3):
        c = np.cumsum(sp_softmax(embed[tokens[b, block - 1]] @ w_lm.T))
        assert out["token"][b] == int(np.searchsorted(c, us[b], side="right"))


def test_concentrated_clean_rows_reject_other_drafts():
    """A clean row 0 whose distribution sits on token v (a huge logit) rejects
    a carried draft d != v at the first position and emits v."""
    block, vocab, hidden = 4, 29, 32
    embed, w_lm, tokens, ud, ua, us = _zero_layer_case(block=block, vocab=vocab, hidden=hidden)
    v, t_clean = 7, 3
    tokens[0, 0], tokens[0, 1] = t_clean, 11        # clean row 0 = t_clean, draft 0 = 11 != v
    w = np.zeros((vocab, hidden))
    w[v] = embed[t_clean] * 2.0                     # clean row 0 of sequence 0: logit 2 * hidden = 64 on v
    out = _run(embed, w, tokens, np.zeros((3, 3, vocab)), ud, ua, us, block)
    assert out["accept_len"][0] == 0
    assert out["token"][0] == v


def test_sequences_are_independent():
    embed, w_lm, tokens, ud, ua, us = _zero_layer_case()
    q = rng.normal(size=(3, 3, w_lm.shape[0]))
    both = _run(embed, w_lm, tokens, q, ud, ua, us, 4)
    one = _run(embed, w_lm, tokens[2:], q[2:], ud[2:], ua[2:], us[2:], 4)
    assert one["accept_len"][0] == both["accept_len"][2]
    assert one["token"][0] == both["token"][2]
    np.testing.assert_array_equal(one["drafts"][0], both["drafts"][2])


def test_kept_rows_that_do_not_fit_flag_the_sequence():
    """With a capacity, a sequence whose L + 1 kept rows do not fit after its
    valid rows is flagged (accept_len = token = -1); the others are not."""
    embed, w_lm, tokens, ud, ua, us = _zero_layer_case()
    vocab = w_lm.shape[0]
    out = oracle.decode_step(tokens, embed, [], [], [], np.ones(32), np.zeros_like(w_lm), np.zeros((3, 3, vocab)),
                             ud, ua, us, 4, 4, 2, cache_len=np.array([0, 16, 17]), capacity=20)
    np.testing.assert_array_equal(out["accept_len"], [3, 3, -1])     # 17 + 4 > 20
    np.testing.assert_array_equal(out["token"][2], -1)


# ---------------------------------------------------------------- the chain's law
def test_two_step_chain_emits_the_ar_law_exactly():
    """Lossless decode loop (the pages' claim), exactly: with no layers the AR
    model is a Markov chain, P(next = v | prefix) = softmax(E[last] W^T)_v,
    computed here with numpy/scipy.  The loop's first step (no carried q)
    emits y0; it draws k drafts from its noisy rows (the q of the mask id);
    the second step verifies those drafts against its own clean rows and the
    carried q.  Enumerating every outcome (the first step's draws by bisection
    on their uniforms, the second step's accept/residual outcomes by
    bisection with tests/_exact_law.py), the emitted law at every position and
    for every prefix must equal the Markov chain's to 1e-12."""
    vocab, hidden, block, mask = 4, 8, 3, 3
    k = block - 1
    g = np.random.default_rng(5)
    embed = g.choice([-1.0, 1.0], size=(vocab, hidden))
    w_lm = g.integers(-24, 25, size=(vocab, hidden)) / 64.0
    x0 = 1
    ar = sp_softmax(embed @ w_lm.T, axis=1)            # the AR transition table
    toks0 = np.array([[x0, 0, 0, mask, mask, mask]])

    def step0(us, ud):
        n = len(us)
        return oracle.decode_step(np.repeat(toks0, n, axis=0), embed, [], [], [], np.ones(hidden), w_lm, None,
                                  ud, np.zeros((n, k)), us, block, 2, 1)

    # law of y0 (bisection on u_s) and of each draft (bisection on u_draft)
    vv = np.arange(vocab)
    cdf_y = _bisect(lambda u: step0(u, np.full((vocab, k), 0.5))["token"] <= vv, vocab)
    cdf_d = _bisect(lambda u: step0(np.full(vocab, 0.5), np.repeat(u[:, None], k, axis=1))["drafts"][:, 0] <= vv,
                    vocab)
    cdf_y[-1] = cdf_d[-1] = 1.0
    p_y0 = np.diff(np.concatenate([[0.0], cdf_y]))
    p_d = np.diff(np.concatenate([[0.0], cdf_d]))
    np.testing.assert_allclose(p_y0, ar[x0], atol=1e-12)            # the first step is plain AR
    q_carry = step0(np.array([0.5]), np.full((1, k), 0.5))["q_next"]
    cases = [(y0,) + d for y0 in range(vocab) for d in itertools.product(range(vocab), repeat=k)]
    weight = np.array([p_y0[c[0]] * np.prod([p_d[t] for t in c[1:]]) for c in cases])

    def run(idx, ua, us):
        n = len(idx)
        toks = np.array([[cases[i][0], *cases[i][1:], mask, mask, mask] for i in idx])
        r = oracle.decode_step(toks, embed, [], [], [], np.ones(hidden), w_lm, np.repeat(q_carry, n, axis=0),
                               np.full((n, k), 0.5), ua, us, block, 2, 1)
        res = []
        for j, i in enumerate(idx):
            L = int(r["accept_len"][j])
            visited = [(s, s < L) for s in range(min(L + 1, k))]
            res.append((visited, (cases[i][0],) + tuple(cases[i][1:1 + L]), int(r["token"][j])))
        return res

    leaves = explore(len(cases), run, k, vocab)
    table = emitted_law(leaves, weight, vocab)
    assert abs(table[()][0] - 1.0) < 1e-12
    worst = 0.0
    for prefix, (reach, emit) in table.items():
        if reach < 1e-15:
            continue
        last = x0 if not prefix else prefix[-1]
        worst = max(worst, float(np.max(np.abs(emit / reach - ar[last]))))
    assert worst < 1e-12, worst
    # the law is not trivially p: the second step accepts drafts with probability strictly in (0, 1)
    assert any(len(pfx) >= 2 for pfx in table)
