"""Oracle: the distillation-side computations of the gated forward -- the
per-row distillation (KL) and total-variation losses between the student rows
(adapter on) and the teacher rows (adapter off), their gradient with respect
to the student logits, and the backward of the gated-LoRA linear layer.
Test infrastructure only.

Source: Uno summary (hyper.ai, arXiv 2609.04010), section "方法", the
paragraphs on diffusion distillation: the objective is alpha * L_DCD +
beta * L_TV; one forward runs over the concatenated clean and noisy rows with
the adapter masked off on clean positions (teacher logits, AR weights alone)
and on on noisy positions (student logits, AR weights plus adapters); the
block-level distillation loss minimises the KL divergence between the student
and the teacher distribution; the TV loss minimises the distance between the
diffusion and the AR distribution to lengthen the accepted draft prefix.

Readings (the pages give the objective in garbled form and no more):
* Row pairs: student row i is compared with teacher row i (both predict the
  same next token; the caller pairs the rows).  Distributions at temperature
  T: p = softmax(teacher / T), q = softmax(student / T).
* KL direction: KL(student || teacher) = sum_v q_v (log q_v - log p_v), read
  off the order the pages name the two distributions in.
* Block level: the single-step student distribution of a block is the product
  of its per-position marginals; with the teacher taken as the product of its
  per-position conditionals on the clean prefix, the KL of the block is the
  sum of the per-row KLs.  The TV loss is likewise the sum of the per-row
  TV(q, p) = 1/2 sum_v |q_v - p_v|  (= 1 - the probability that a draft drawn
  from q is accepted against p).
* The gradient is taken with respect to the student logits only (the teacher
  is the frozen AR path); at q_v = p_v the subgradient of |q_v - p_v| is 0.

Gated-LoRA backward (y = x W^T + s diag(g) (x A^T) B^T, oracle.gated_lora):
with dY = dL/dy, T = x A^T and U = diag(g) T,
    dB = s dY^T U,   dT = s diag(g) dY B,   dA = dT^T x,   dx = dY W + dT A;
W is the frozen AR weight (no gradient).
"""

import numpy as np


def log_softmax_rows(logits, temperature=1.0):
    """float64 log-softmax over the last axis of logits / T."""
    x = np.asarray(logits, dtype=np.float64) / float(temperature)
    m = np.max(x, axis=-1, keepdims=True)
    return x - m - np.log(np.sum(np.exp(x - m), axis=-1, keepdims=True))


def distill_losses(teacher, student, temperature=1.0, alpha=1.0, beta=1.0, grad_scale=1.0):
    """Per-row losses of row pairs and the gradient of
    grad_scale * sum_rows (alpha * KL + beta * TV) with respect to the student
    logits.

    teacher, student [R, V] logits (any float dtype, widened to float64).
    Returns dict kl [R], tv [R], grad [R, V] (float64)."""
    t = float(temperature)
    lp = log_softmax_rows(teacher, t)
    lq = log_softmax_rows(student, t)
    p, q = np.exp(lp), np.exp(lq)
    kl = np.sum(q * (lq - lp), axis=-1)
    diff = q - p
    tv = 0.5 * np.sum(np.abs(diff), axis=-1)
    # d/dz of sum_v f(q_v) with q = softmax(z / T): (1/T) q_v (f'(q_v) - sum_u q_u f'(q_u))
    # KL: f'(q_v) = log q_v - log p_v + 1 (the +1 cancels); TV: f'(q_v) = sign(q_v - p_v) / 2
    dkl = lq - lp
    dtv = 0.5 * np.sign(diff)
    g_row = alpha * dkl + beta * dtv
    mean = np.sum(q * g_row, axis=-1, keepdims=True)
    grad = grad_scale / t * q * (g_row - mean)
    return {"kl": kl, "tv": tv, "grad": grad}


def gated_lora_backward(x, w, a, b, dy, gate=None, lora_scale=1.0):
    """Gradients of the gated-LoRA linear layer (float64).

    x [M, K], w [N, K], a [r, K], b [N, r], dy [M, N]; gate [M] of 0/1
    (None = all 0).  Returns dict dx [M, K], da [r, K], db [N, r]."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    dy = np.asarray(dy, dtype=np.float64)
    m = x.shape[0]
    g = np.zeros(m) if gate is None else np.asarray(gate).astype(np.float64).reshape(m)
    s = float(lora_scale)
    down = x @ a.T                               # T [M, r]
    u = down * g[:, None]                        # adapter input of the gated rows
    db = s * (dy.T @ u)                          # [N, r]
    dt = s * (dy @ b) * g[:, None]               # [M, r]
    da = dt.T @ x                                # [r, K]
    dx = dy @ w + dt @ a                         # [M, K]
    return {"dx": dx, "da": da, "db": db}
