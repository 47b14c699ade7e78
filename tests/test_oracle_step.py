"""Pins of the whole-step oracle (oracle.decode_step).

Source: Uno summary (hyper.ai, arXiv 2609.04010), section 方法 (propose a
block on the diffusion path, verify it on the AR path, keep the longest
valid prefix; the first token of a block comes from the AR weights).  The
composition is tied to closed forms that do not go through its own code:
uniform distributions, identical clean and noisy rows, a clean distribution
concentrated on one token, and sequence independence.
"""

import numpy as np

import oracle

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


def _run(embed, w_lm, tokens, ud, ua, us, block):
    return oracle.decode_step(tokens, embed, [], [], [], np.ones(embed.shape[1]), w_lm, ud, ua, us, block, 4, 2)


def test_rows_layout():
    gate, pos = oracle.step_rows(2, 3, 100)
    np.testing.assert_array_equal(gate, [0, 0, 0, 1, 1, 1] * 2)
    np.testing.assert_array_equal(pos, [100, 101, 102] * 4)


def test_uniform_distributions_accept_everything_and_draw_by_floor():
    """A zero LM head gives uniform p and q: every draft is accepted (u/V < 1/V)
    and every draw is floor(u * V)."""
    embed, w_lm, tokens, ud, ua, us = _zero_layer_case()
    vocab = w_lm.shape[0]
    out = _run(embed, np.zeros_like(w_lm), tokens, ud, ua, us, 4)
    np.testing.assert_array_equal(out["drafts"], np.floor(ud * vocab).astype(int))
    np.testing.assert_array_equal(out["accept_len"], [3, 3, 3])
    np.testing.assert_array_equal(out["token"], np.floor(us * vocab).astype(int))


def test_logits_are_lm_head_of_normed_embeddings():
    """With no layers the logits are rmsnorm(embed[t]) . W^T, here exact: the
    +-1 embedding rows normalise to +-1 in bf16 and the products are dyadic."""
    embed, w_lm, tokens, ud, ua, us = _zero_layer_case()
    out = _run(embed, w_lm, tokens, ud, ua, us, 4)
    ref = embed[tokens.reshape(-1)] @ w_lm.T
    np.testing.assert_array_equal(out["logits"], ref)


def test_identical_clean_and_noisy_rows_accept_everything():
    """Noisy ids equal to clean ids give q_i = p_i, so L = k and y is the bonus
    draw from the last clean row, written out with numpy here."""
    block = 5
    embed, w_lm, tokens, ud, ua, us = _zero_layer_case(block=block)
    tokens[:, block:] = tokens[:, :block]
    out = _run(embed, w_lm, tokens, ud, ua, us, block)
    np.testing.assert_array_equal(out["accept_len"], [block - 1] * 3)
    for b in range(3):
        lg = embed[tokens[b, block - 1]] @ w_lm.T
        p = np.exp(lg - lg.max())
        c = np.cumsum(p / p.sum())
        assert out["token"][b] == int(np.searchsorted(c, us[b], side="right"))


def test_concentrated_clean_rows_reject_other_drafts():
    """Clean rows whose distribution sits on token v (a huge logit) reject any
    draft d != v at the first position and emit v."""
    block, vocab, hidden = 4, 29, 32
    embed, w_lm, tokens, ud, ua, us = _zero_layer_case(block=block, vocab=vocab, hidden=hidden)
    v, t_clean, t_noisy = 7, 3, 4
    tokens[0, 0], tokens[0, block] = t_clean, t_noisy
    embed[t_noisy] = -embed[t_clean]          # noisy row 0: logit -64 on v, so the draft is not v
    w = np.zeros((vocab, hidden))
    w[v] = embed[t_clean] * 2.0               # clean row 0 of sequence 0: logit 2 * hidden = 64 on v
    out = _run(embed, w, tokens, ud, ua, us, block)
    assert out["drafts"][0, 0] != v
    assert out["accept_len"][0] == 0
    assert out["token"][0] == v


def test_sequences_are_independent():
    embed, w_lm, tokens, ud, ua, us = _zero_layer_case()
    both = _run(embed, w_lm, tokens, ud, ua, us, 4)
    one = _run(embed, w_lm, tokens[2:], ud[2:], ua[2:], us[2:], 4)
    assert one["accept_len"][0] == both["accept_len"][2]
    assert one["token"][0] == both["token"][2]
    np.testing.assert_array_equal(one["drafts"][0], both["drafts"][2])
