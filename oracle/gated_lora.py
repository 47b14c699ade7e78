"""Oracle: gated-LoRA linear layer.  Test infrastructure only.

Source: Uno paper summary (hyper.ai, arXiv 2609.04010), section "方法":
the diffusion weights are low-rank adapters attached to every AR weight
matrix; drafting uses the AR weights plus the adapters, verification uses the
AR weights alone; one forward pass runs over the concatenated clean and noisy
sequences and a mask switches the adapter off on clean positions and on on
noisy positions.

Computed here (float64, no intermediate rounding):

    Y = X W^T + s * diag(g) (X A^T) B^T

With a 0/1 gate, a row with g = 1 computes X (W + s B A)^T, the LoRA merge
identity; merged_weight() writes that matrix out, the weight the GPU reads
for the gated rows when it is given gate-merged weights.

Readings where the pages are silent:
* no bias term;
* the LoRA scale alpha/r is folded into B, so s = 1 by default;
* g is a binary per-row mask (0 = clean/verify row, 1 = noisy/draft row);
* the layout follows torch.nn.Linear: W [N, K], A [r, K], B [N, r].
"""

import numpy as np


def gated_lora_linear(x, w, a, b, gate=None, lora_scale=1.0):
    """Return Y[M, N] in float64.

    x [M, K], w [N, K], a [r, K], b [N, r]; gate [M] of 0/1 (None = all 0).
    Inputs may be any float dtype; they are widened to float64 exactly.
    """
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    m = x.shape[0]
    if gate is None:
        g = np.zeros(m, dtype=np.float64)
    else:
        g = np.asarray(gate).astype(np.float64).reshape(m)
    base = x @ w.T                      # theta_AR path, every row
    down = x @ a.T                      # LoRA down-projection, [M, r]
    gated = down * g[:, None]           # adapter on only where g = 1
    return base + lora_scale * (gated @ b.T)


def merged_weight(w, a, b, lora_scale=1.0):
    """W + s * B A in float64 ([N, K]): the weight a gated (g = 1) row sees."""
    w = np.asarray(w, dtype=np.float64)
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return w + lora_scale * (b @ a)
