"""Oracle: Psi-Spec linear verify sampler.  Test infrastructure only.

Sources:
* Uno paper summary (hyper.ai, arXiv 2609.04010), section "方法", last
  paragraph: the diffusion path proposes a block of tokens; rejection sampling
  against the base AR distribution accepts the longest valid prefix; the
  linear sampler draws a single candidate sequence from the marginals; the
  first token of the block is produced with the base AR weights so the result
  matches the verification distribution exactly.
* Same summary, "方法", the causal-mask formula: the distribution of token l
  is read from the model output at position l-1 (so AR row i of a block
  scores draft i, and one extra row scores the token after the last draft).
* ainews.surl.tw article on Uno: "lossless" means the emitted samples follow
  the base AR distribution.
* 4sapi.net blog on Uno, the speculative-decoding recap: the target verifies
  the draft in one forward, keeps the run of consecutive correct tokens and
  backs off at the first error.

The pages do not write out the acceptance rule or the residual; the plainest
reading that makes the procedure lossless is standard speculative sampling
(Leviathan et al. 2023; Chen et al. 2023), which is what is computed here:

1. p_i = softmax(l^p_i / T), i = 0..k (row k is the bonus row);
   q_i = softmax(l^q_i / T), i = 0..k-1.  Max-subtracted, float64.
2. Draft d_i is accepted iff  u_acc[i] * q_i[d_i] < p_i[d_i]  (strict; this
   is "u < min(1, p/q)" without a division, for u in [0, 1)).
3. L = index of the first rejection, k if none.
4. If L < k: w = max(0, p_L - q_L), S = sum(w); if L = k: w = p_k.
   If S == 0 (exact equality p_L == q_L, reachable only by rounding) the draw
   falls back to p_L.
5. y = the smallest token id v with cumsum(w)[v] > u_s * sum(w); if rounding
   leaves no such v, y = the last v with w[v] > 0.
Emitted tokens for the step: d[0:L] followed by y.

With a sampling transform (top-k, top-p, greedy; oracle/sampling.py) every p
and q row is replaced by its transformed distribution before step 2 and the
same rules run on those (drafts are then drawn from the transformed q).
"""

import numpy as np


def softmax_rows(logits, temperature=1.0):
    """float64 softmax over the last axis of logits / temperature."""
    x = np.asarray(logits, dtype=np.float64) / float(temperature)
    m = np.max(x, axis=-1, keepdims=True)
    e = np.exp(x - m)
    return e / np.sum(e, axis=-1, keepdims=True)


def row_log_stats(logits, temperature=1.0):
    """(m, Z) with m = max(l/T) and Z = sum exp(l/T - m), per row (float64).

    log-sum-exp of the row is m + log(Z).
    """
    x = np.asarray(logits, dtype=np.float64) / float(temperature)
    m = np.max(x, axis=-1)
    z = np.sum(np.exp(x - m[..., None]), axis=-1)
    return m, z


def accept_draft(u, p_d, q_d):
    """Accept test of one draft token: u * q(d) < p(d)."""
    return u * q_d < p_d


def residual_weights(p_row, q_row):
    """Unnormalised residual w = max(0, p - q) and its mass S."""
    w = np.maximum(0.0, np.asarray(p_row, np.float64) - np.asarray(q_row, np.float64))
    return w, float(np.sum(w))


def inverse_cdf(w, u):
    """Smallest v with cumsum(w)[v] > u * sum(w) (token-id order).

    Falls back to the last v with w[v] > 0 when rounding leaves none.
    """
    w = np.asarray(w, dtype=np.float64)
    c = np.cumsum(w)
    target = float(u) * c[-1]
    hit = np.nonzero(c > target)[0]
    if hit.size:
        return int(hit[0])
    pos = np.nonzero(w > 0.0)[0]
    return int(pos[-1])


def verify_linear(p_logits, q_logits, drafts, u_accept, u_sample, temperature=1.0, top_k=0, top_p=1.0,
                  greedy=False):
    """Verify a batch of linear draft blocks.

    p_logits [B, k+1, V]  AR rows; row i scores draft i, row k is the bonus row.
    q_logits [B, k, V]    draft marginals, row i for draft i.
    drafts   [B, k]       int token ids; an id outside [0, V) has probability 0
                          under p and q and is rejected.
    u_accept [B, k], u_sample [B]: uniforms in [0, 1).
    top_k, top_p, greedy: the sampling transform of every p and q row
    (oracle.sampling.transform_probs); the defaults leave the rows unchanged.

    Returns a dict of numpy arrays:
      accept_len [B] int, token [B] int (correction or bonus y),
      p_draft [B, k], q_draft [B, k] (float64 probabilities of each draft),
      residual_mass [B] (S of the residual actually drawn from; 1 for bonus).
    """
    p_logits = np.asarray(p_logits)
    q_logits = np.asarray(q_logits)
    drafts = np.asarray(drafts)
    u_accept = np.asarray(u_accept, dtype=np.float64)
    u_sample = np.asarray(u_sample, dtype=np.float64).reshape(-1)
    bsz, k = drafts.shape
    assert p_logits.shape[:2] == (bsz, k + 1)
    assert q_logits.shape[:2] == (bsz, k)

    accept_len = np.zeros(bsz, dtype=np.int64)
    token = np.zeros(bsz, dtype=np.int64)
    p_draft = np.zeros((bsz, k), dtype=np.float64)
    q_draft = np.zeros((bsz, k), dtype=np.float64)
    res_mass = np.zeros(bsz, dtype=np.float64)

    from .sampling import transform_probs
    plain = top_k <= 0 and top_p >= 1.0 and not greedy

    def rows(lg):
        if plain:
            return softmax_rows(lg, temperature)
        return np.stack([transform_probs(r, temperature, top_k, top_p, greedy) for r in lg])

    for b in range(bsz):
        p = rows(p_logits[b])                                # [k+1, V]
        q = rows(q_logits[b]) if k else np.zeros((0, p.shape[1]))
        length = k
        for i in range(k):
            d = int(drafts[b, i])
            if 0 <= d < p.shape[1]:            # an id outside [0, V) has probability 0: rejected
                p_draft[b, i] = p[i, d]
                q_draft[b, i] = q[i, d]
        for i in range(k):
            if not accept_draft(u_accept[b, i], p_draft[b, i], q_draft[b, i]):
                length = i
                break
        if length < k:
            w, s = residual_weights(p[length], q[length])
            if s == 0.0:
                w, s = p[length], float(np.sum(p[length]))
        else:
            w, s = p[k], float(np.sum(p[k]))
        accept_len[b] = length
        token[b] = inverse_cdf(w, u_sample[b])
        res_mass[b] = s
    return {
        "accept_len": accept_len,
        "token": token,
        "p_draft": p_draft,
        "q_draft": q_draft,
        "residual_mass": res_mass,
    }
