"""Seeded synthetic inputs for the Psi-Spec hot path.

This module is the only code shared by the CPU oracle's tests and the GPU
path's tests and benchmark.  It holds no arithmetic of the method itself: it
draws random numbers, rounds them to bf16 storage, builds tree shapes, and
draws draft tokens from the draft distribution with the Gumbel-max trick
(argmax of logits/T + Gumbel noise), which samples softmax(logits/T) without
computing it.

Every stream is a PCG64 generator seeded from SeedSequence([seed, tag, ...]),
so any single row can be regenerated on its own (used to check sampled rows of
full-size runs against the oracle without regenerating everything).
"""

import os
from concurrent.futures import ProcessPoolExecutor

import numpy as np

# stream tags
_T_W, _T_A, _T_B, _T_X = 11, 12, 13, 14
_T_P, _T_Q, _T_DRAFT, _T_UACC, _T_US = 21, 22, 23, 24, 25
_T_ATT_Q, _T_ATT_KC, _T_ATT_VC, _T_ATT_KT, _T_ATT_VT = 31, 32, 33, 34, 35
_T_TREE_SHAPE, _T_TREE_BASE, _T_TREE_P, _T_TREE_Q, _T_TREE_TOK = 41, 42, 43, 44, 45
_T_TREE_UACC, _T_TREE_US = 46, 47
_T_BUILD_U = 48
_T_BWD_DY = 71


def rng_for(seed, *tags):
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(seed)] + [int(t) for t in tags])))


# ---------------------------------------------------------------- bf16 storage
def bf16_bits(x):
    """Round float32 values to bfloat16 (round to nearest, ties to even).

    Returns the uint16 bit patterns.  NaN is not expected in these inputs.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = (u + 0x7FFF + lsb) >> 16
    return r.astype(np.uint16)


def bf16_to_f32(bits):
    """Exact float32 values of bfloat16 bit patterns."""
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32)


def round_bf16(x):
    """float32 values rounded through bf16 storage."""
    return bf16_to_f32(bf16_bits(x))


def _store(x_f32, dtype):
    """Return (storage array, exact float32 values) for dtype 'f32' or 'bf16'."""
    if dtype == "bf16":
        bits = bf16_bits(x_f32)
        return bits, bf16_to_f32(bits)
    if dtype == "f32":
        x = np.ascontiguousarray(x_f32, dtype=np.float32)
        return x, x
    raise ValueError(dtype)


def gumbel_max(logits, temperature, rng):
    """One draw from softmax(logits / T) by the Gumbel-max trick (float64)."""
    u = rng.random(np.asarray(logits).shape[-1])
    u = np.clip(u, 1e-300, None)
    g = -np.log(-np.log(u))
    return int(np.argmax(np.asarray(logits, np.float64) / temperature + g))


# ---------------------------------------------------------------- gated LoRA
def gated_lora_case(m, n, k, r, dtype="bf16", seed=0, gate=None, weight_std=0.02,
                    x_std=1.0, tag=0):
    """Inputs of one gated-LoRA projection.

    W [n, k], A [r, k], B [n, r] ~ N(0, weight_std^2); X [m, k] ~ N(0, x_std^2),
    rounded to `dtype` storage.  gate: uint8 [m]; default is the sequence-major
    concatenated pattern of the 1024-row layer workload (8 clean rows, then 8
    noisy rows, per sequence) when m is a multiple of 16, else alternate
    halves per pair of rows.
    """
    w = rng_for(seed, _T_W, tag).standard_normal((n, k), dtype=np.float32) * np.float32(weight_std)
    a = rng_for(seed, _T_A, tag).standard_normal((r, k), dtype=np.float32) * np.float32(weight_std)
    b = rng_for(seed, _T_B, tag).standard_normal((n, r), dtype=np.float32) * np.float32(weight_std)
    x = rng_for(seed, _T_X, tag).standard_normal((m, k), dtype=np.float32) * np.float32(x_std)
    if gate is None:
        gate = default_gate(m)
    gate = np.asarray(gate, dtype=np.uint8).reshape(m)
    out = {"m": m, "n": n, "k": k, "r": r, "dtype": dtype, "gate": gate}
    for name, arr in (("x", x), ("w", w), ("a", a), ("b", b)):
        st, val = _store(arr, dtype)
        out[name] = st
        out[name + "_f32"] = val
    return out


def lora_backward_case(m, n, k, r, seed=0, gate=None, weight_std=0.02, adapter_std=0.05):
    """Inputs of the gated-LoRA backward, bf16: the projection of
    gated_lora_case with A, B ~ N(0, adapter_std^2) (large enough that the
    adapter's share of dx is well above bf16 rounding) and the upstream
    gradient dY [m, n] ~ N(0, 1)."""
    c = gated_lora_case(m, n, k, r, "bf16", seed=seed, gate=gate, weight_std=weight_std)
    for name, tag in (("a", _T_A), ("b", _T_B)):
        shape = (r, k) if name == "a" else (n, r)
        arr = rng_for(seed, tag, 1).standard_normal(shape, dtype=np.float32) * np.float32(adapter_std)
        c[name], c[name + "_f32"] = _store(arr, "bf16")
    dy = rng_for(seed, _T_BWD_DY).standard_normal((m, n), dtype=np.float32)
    c["dy"], c["dy_f32"] = _store(dy, "bf16")
    return c


def default_gate(m, block=8):
    """Per sequence: `block` clean rows (gate 0) then `block` noisy rows (gate 1)."""
    if m % (2 * block) == 0:
        per = np.concatenate([np.zeros(block, np.uint8), np.ones(block, np.uint8)])
        return np.tile(per, m // (2 * block))
    return (np.arange(m) % 2).astype(np.uint8)


# ------------------------------------------------------------ linear verify
def _verify_seq(args):
    seed, b, k, vocab, sigma, dtype, p_std, temperature = args
    p_st = []
    q_st = []
    p_val = []
    q_val = []
    drafts = np.zeros(k, dtype=np.int32)
    for i in range(k + 1):
        lp = rng_for(seed, _T_P, b, i).standard_normal(vocab, dtype=np.float32) * np.float32(p_std)
        st, val = _store(lp, dtype)
        p_st.append(st)
        p_val.append(val)
        if i < k:
            lq = lp + rng_for(seed, _T_Q, b, i).standard_normal(vocab, dtype=np.float32) * np.float32(sigma)
            st, val = _store(lq, dtype)
            q_st.append(st)
            q_val.append(val)
            drafts[i] = gumbel_max(val, temperature, rng_for(seed, _T_DRAFT, b, i))
    return (np.stack(p_st), np.stack(q_st) if k else None, np.stack(p_val),
            np.stack(q_val) if k else None, drafts)


def verify_linear_seq(seed, b, k, vocab, sigma, dtype="bf16", p_std=2.0, temperature=1.0):
    """Regenerate sequence b of a linear-verify workload on its own.

    Returns (p_store [k+1,V], q_store [k,V], p_f32, q_f32, drafts [k]).
    """
    return _verify_seq((seed, b, k, vocab, sigma, dtype, p_std, temperature))


def verify_linear_case(batch, k, vocab, sigma, dtype="bf16", seed=0, p_std=2.0,
                       temperature=1.0, workers=None, keep_f32=True):
    """Inputs of the linear verify sampler.

    AR logits l^p [batch, k+1, vocab] ~ N(0, p_std^2); draft logits
    l^q = l^p[:, :k] (before rounding) + N(0, sigma^2); both rounded to
    `dtype` storage.  Drafts d[b, i] ~ softmax(l^q[b, i] / T) (Gumbel-max on the
    stored values).  u_acc [batch, k], u_s [batch]: float32 uniforms in [0, 1).
    """
    if workers is None:
        workers = min(16, len(os.sched_getaffinity(0)))
    jobs = [(seed, b, k, vocab, sigma, dtype, p_std, temperature) for b in range(batch)]
    store_dt = np.uint16 if dtype == "bf16" else np.float32
    p_st = np.empty((batch, k + 1, vocab), dtype=store_dt)
    q_st = np.empty((batch, k, vocab), dtype=store_dt)
    p_f = np.empty((batch, k + 1, vocab), dtype=np.float32) if keep_f32 else None
    q_f = np.empty((batch, k, vocab), dtype=np.float32) if keep_f32 else None
    drafts = np.empty((batch, k), dtype=np.int32)

    def put(b, res):
        ps, qs, pv, qv, d = res
        p_st[b] = ps
        if k:
            q_st[b] = qs
        if keep_f32:
            p_f[b] = pv
            if k:
                q_f[b] = qv
        drafts[b] = d

    if workers > 1 and batch * (2 * k + 1) * vocab > (1 << 22):
        with ProcessPoolExecutor(max_workers=workers) as ex:
            for b, res in enumerate(ex.map(_verify_seq, jobs, chunksize=max(1, batch // (4 * workers)))):
                put(b, res)
    else:
        for b, job in enumerate(jobs):
            put(b, _verify_seq(job))
    u_acc = rng_for(seed, _T_UACC).random((batch, k), dtype=np.float32)
    u_s = rng_for(seed, _T_US).random(batch, dtype=np.float32)
    return {"batch": batch, "k": k, "vocab": vocab, "sigma": sigma, "dtype": dtype,
            "temperature": temperature, "seed": seed,
            "p": p_st, "q": q_st, "p_f32": p_f, "q_f32": q_f, "drafts": drafts,
            "u_acc": u_acc, "u_s": u_s}


# ------------------------------------------------------------ tree shapes
def tree_parent_cfg(seed, branching=4, depth=3, n_last=44):
    """Prefix tree in breadth-first order: levels 1..depth-1 full, `n_last`
    of the branching^depth slots of the last level chosen without replacement.
    Returns parent int32 [n] with parent[0] = -1."""
    parent = [-1]
    level = [0]
    for d in range(1, depth + 1):
        slots = [(p, c) for p in level for c in range(branching)]
        if d == depth and n_last is not None and n_last < len(slots):
            pick = np.sort(rng_for(seed, _T_TREE_SHAPE).choice(len(slots), n_last, replace=False))
            slots = [slots[i] for i in pick]
        nxt = []
        for (p, _c) in slots:
            parent.append(p)
            nxt.append(len(parent) - 1)
        level = nxt
    return np.asarray(parent, dtype=np.int32)


def chain_parent(n):
    return np.arange(-1, n - 1, dtype=np.int32)


def star_parent(n):
    p = np.zeros(n, dtype=np.int32)
    p[0] = -1
    return p


def random_parent(n, seed, max_children=None):
    """Random parent array with parent[i] < i (breadth-first not required)."""
    rng = rng_for(seed, _T_TREE_SHAPE, n)
    p = np.empty(n, dtype=np.int32)
    p[0] = -1
    for i in range(1, n):
        p[i] = rng.integers(0, i)
    return p


def max_children(parent):
    """Largest number of children of any node of a parent array (or batch of them)."""
    parent = np.asarray(parent).reshape(-1, np.shape(parent)[-1])
    best = 0
    for row in parent:
        counts = np.bincount(row[1:][row[1:] >= 0], minlength=1) if row.size > 1 else np.zeros(1, int)
        best = max(best, int(counts.max()) if counts.size else 0)
    return best


def _depths(parent):
    d = np.zeros(len(parent), dtype=np.int64)
    for i in range(1, len(parent)):
        d[i] = d[parent[i]] + 1
    return d


# ------------------------------------------------------------ tree attention
def tree_attention_case(batch, parent, ctx, n_heads=32, n_kv_heads=8, head_dim=128, seed=0,
                        std=1.0):
    """bf16 Q [B,n,H,D], K/V cache [B,ctx,Hkv,D], K/V tree [B,n,Hkv,D] ~ N(0, std^2).

    parent: int32 [n] (shared by the batch) or [B, n]."""
    parent = np.asarray(parent, dtype=np.int32)
    if parent.ndim == 1:
        parent = np.tile(parent, (batch, 1))
    n = parent.shape[1]
    shapes = {
        "q": (_T_ATT_Q, (batch, n, n_heads, head_dim)),
        "k_cache": (_T_ATT_KC, (batch, ctx, n_kv_heads, head_dim)),
        "v_cache": (_T_ATT_VC, (batch, ctx, n_kv_heads, head_dim)),
        "k_tree": (_T_ATT_KT, (batch, n, n_kv_heads, head_dim)),
        "v_tree": (_T_ATT_VT, (batch, n, n_kv_heads, head_dim)),
    }
    out = {"batch": batch, "n": n, "ctx": ctx, "n_heads": n_heads, "n_kv_heads": n_kv_heads,
           "head_dim": head_dim, "parent": parent, "scale": 1.0 / np.sqrt(head_dim)}
    for name, (tag, shp) in shapes.items():
        x = rng_for(seed, tag).standard_normal(shp, dtype=np.float32) * np.float32(std)
        st, val = _store(x, "bf16")
        out[name] = st
        out[name + "_f32"] = val
    return out


# ------------------------------------------------------------ tree verify
def tree_verify_case(parent, vocab, dtype="bf16", seed=0, base_std=2.0, node_std=0.5,
                     q_std=0.5, temperature=1.0, batch=1):
    """Logits and tokens of a candidate tree.

    base_d ~ N(0, base_std^2) for depth d = 1..D+1; the AR row of a node at
    depth d is base_{d+1} + N(0, node_std^2); the draft marginal of depth d is
    base_d + N(0, q_std^2).  Node tokens ~ softmax(q_depth / T) (Gumbel-max),
    i.i.d. per node.  u_acc [B, n], u_s [B] float32 in [0, 1).
    """
    parent = np.asarray(parent, dtype=np.int32)
    n = parent.shape[0]
    depth = _depths(parent)
    dmax = int(depth.max()) if n > 1 else 1
    dmax = max(dmax, 1)
    store_dt = np.uint16 if dtype == "bf16" else np.float32
    p_st = np.empty((batch, n, vocab), dtype=store_dt)
    q_st = np.empty((batch, dmax, vocab), dtype=store_dt)
    p_f = np.empty((batch, n, vocab), dtype=np.float32)
    q_f = np.empty((batch, dmax, vocab), dtype=np.float32)
    tokens = np.zeros((batch, n), dtype=np.int32)
    for b in range(batch):
        base = [rng_for(seed, _T_TREE_BASE, b, d).standard_normal(vocab, dtype=np.float32)
                * np.float32(base_std) for d in range(dmax + 2)]
        for d in range(1, dmax + 1):
            lq = base[d] + rng_for(seed, _T_TREE_Q, b, d).standard_normal(vocab, dtype=np.float32) * np.float32(q_std)
            q_st[b, d - 1], q_f[b, d - 1] = _store(lq, dtype)
        for i in range(n):
            lp = base[depth[i] + 1] + rng_for(seed, _T_TREE_P, b, i).standard_normal(vocab, dtype=np.float32) * np.float32(node_std)
            p_st[b, i], p_f[b, i] = _store(lp, dtype)
            if i > 0:
                tokens[b, i] = gumbel_max(q_f[b, depth[i] - 1], temperature,
                                          rng_for(seed, _T_TREE_TOK, b, i))
    u_acc = rng_for(seed, _T_TREE_UACC).random((batch, n), dtype=np.float32)
    u_s = rng_for(seed, _T_TREE_US).random(batch, dtype=np.float32)
    return {"batch": batch, "n": n, "max_depth": dmax, "vocab": vocab, "dtype": dtype,
            "temperature": temperature, "parent": np.tile(parent, (batch, 1)),
            "tokens": tokens, "p": p_st, "q": q_st, "p_f32": p_f, "q_f32": q_f,
            "u_acc": u_acc, "u_s": u_s}


def level_depths(branching):
    """Depth of every node of the breadth-first tree with `branching[d]`
    children per depth-d node (root depth 0), in node-id order."""
    depth = [0]
    width = 1
    for d, b in enumerate(branching):
        width *= int(b)
        depth += [d + 1] * width
    return np.asarray(depth, dtype=np.int64)


def tree_build_case(batch, branching, vocab, dtype="bf16", seed=0, base_std=2.0, node_std=0.5, q_std=0.5):
    """Inputs of the candidate-tree construction and of the verify of the
    built tree, with the distributions of tree_verify_case: base_d ~
    N(0, base_std^2); the draft marginal of depth d (q row d - 1) is base_d +
    N(0, q_std^2); the AR row of a node at depth d is base_{d+1} +
    N(0, node_std^2).  u_draw [B, n] (entry 0 unused), u_acc [B, n], u_s [B]
    float32 in [0, 1)."""
    depth = level_depths(branching)
    n = depth.size
    dmax = len(branching)
    store_dt = np.uint16 if dtype == "bf16" else np.float32
    q_st = np.empty((batch, dmax, vocab), dtype=store_dt)
    q_f = np.empty((batch, dmax, vocab), dtype=np.float32)
    p_st = np.empty((batch, n, vocab), dtype=store_dt)
    p_f = np.empty((batch, n, vocab), dtype=np.float32)
    for b in range(batch):
        base = [rng_for(seed, _T_TREE_BASE, b, d).standard_normal(vocab, dtype=np.float32)
                * np.float32(base_std) for d in range(dmax + 2)]
        for d in range(1, dmax + 1):
            lq = base[d] + rng_for(seed, _T_TREE_Q, b, d).standard_normal(vocab, dtype=np.float32) * np.float32(q_std)
            q_st[b, d - 1], q_f[b, d - 1] = _store(lq, dtype)
        for i in range(n):
            lp = base[depth[i] + 1] + rng_for(seed, _T_TREE_P, b, i).standard_normal(vocab, dtype=np.float32) * np.float32(node_std)
            p_st[b, i], p_f[b, i] = _store(lp, dtype)
    return {"batch": batch, "n": n, "max_depth": dmax, "vocab": vocab, "dtype": dtype, "branching": list(branching),
            "q": q_st, "q_f32": q_f, "p": p_st, "p_f32": p_f,
            "u_draw": rng_for(seed, _T_BUILD_U).random((batch, n), dtype=np.float32),
            "u_acc": rng_for(seed, _T_TREE_UACC).random((batch, n), dtype=np.float32),
            "u_s": rng_for(seed, _T_TREE_US).random(batch, dtype=np.float32)}


# ------------------------------------------------------------ named workloads
def tiny_step(seed=0):
    """The tiny fp32 step: gated LoRA 8 x 256 -> 256, rank 8 (2 sequences of
    2 clean + 2 noisy rows), and a linear verify of batch 2 x block 4 (k = 3)
    over vocab 1024 with AR logits ~ N(0, 2^2) and draft logits = AR + N(0, 0.5^2)."""
    gate = np.array([0, 0, 1, 1, 0, 0, 1, 1], dtype=np.uint8)
    lora = gated_lora_case(8, 256, 256, 8, dtype="f32", seed=seed, gate=gate)
    ver = verify_linear_case(2, 3, 1024, 0.5, dtype="f32", seed=seed, workers=1)
    return {"lora": lora, "verify": ver}


# ------------------------------------------------------------ decoder layer
_T_LAYER_H, _T_LAYER_W, _T_LAYER_A, _T_LAYER_B, _T_LAYER_NORM = 51, 52, 53, 54, 55
_T_LAYER_KC, _T_LAYER_VC = 56, 57
_T_ROWS_L, _T_ROWS_U = 61, 62

LAYER_PROJ = ("q", "k", "v", "o", "g", "u", "d")     # q, k, v, o, gate, up, down


def layer_shapes(hidden, inter, n_heads, n_kv_heads, head_dim=128):
    """(out, in) of the seven projections of a Qwen3-style layer."""
    qd, kvd = n_heads * head_dim, n_kv_heads * head_dim
    return {"q": (qd, hidden), "k": (kvd, hidden), "v": (kvd, hidden), "o": (hidden, qd),
            "g": (inter, hidden), "u": (inter, hidden), "d": (hidden, inter)}


def layer_weights_case(hidden, inter, n_heads, n_kv_heads, r, seed=0, layer=0, weight_std=0.02,
                       norm_std=0.1, lora_std=None, qk_norm=True):
    """bf16 weights of one layer: w{p} [out, in] ~ N(0, weight_std^2), a{p}
    [r, in] and b{p} [out, r] ~ N(0, lora_std^2) (default weight_std);
    attn_norm, mlp_norm = 1 + N(0, norm_std^2); with qk_norm also the
    per-head q_norm, k_norm [128] = 1 + N(0, norm_std^2).

    Returns {name: uint16 bits} and {name + "_f32": exact values}."""
    out = {}
    lora_std = weight_std if lora_std is None else lora_std
    for i, (p, (n_out, n_in)) in enumerate(layer_shapes(hidden, inter, n_heads, n_kv_heads).items()):
        for name, tag, shp in (("w", _T_LAYER_W, (n_out, n_in)), ("a", _T_LAYER_A, (r, n_in)),
                               ("b", _T_LAYER_B, (n_out, r))):
            std = weight_std if name == "w" else lora_std
            x = rng_for(seed, tag, layer, i).standard_normal(shp, dtype=np.float32) * np.float32(std)
            out[name + p], out[name + p + "_f32"] = _store(x, "bf16")
    for j, name in enumerate(("attn_norm", "mlp_norm")):
        x = 1.0 + rng_for(seed, _T_LAYER_NORM, layer, j).standard_normal(hidden, dtype=np.float32) * np.float32(norm_std)
        out[name], out[name + "_f32"] = _store(x, "bf16")
    if qk_norm:
        for j, name in ((2, "q_norm"), (3, "k_norm")):
            x = 1.0 + rng_for(seed, _T_LAYER_NORM, layer, j).standard_normal(128, dtype=np.float32) * np.float32(norm_std)
            out[name], out[name + "_f32"] = _store(x, "bf16")
    return out


def layer_seq_rows(seed, b, block, hidden, x_std=1.0):
    """Residual-stream rows of sequence b: 2*block rows of N(0, x_std^2), bf16
    bits (clean rows then noisy rows)."""
    x = rng_for(seed, _T_LAYER_H, b).standard_normal((2 * block, hidden), dtype=np.float32) * np.float32(x_std)
    return bf16_bits(x)


def _kv_seq(args):
    seed, layer, b, ctx, nkv, head_dim, std = args
    k = rng_for(seed, _T_LAYER_KC, layer, b).standard_normal((ctx, nkv, head_dim), dtype=np.float32)
    v = rng_for(seed, _T_LAYER_VC, layer, b).standard_normal((ctx, nkv, head_dim), dtype=np.float32)
    return bf16_bits(k * np.float32(std)), bf16_bits(v * np.float32(std))


def kv_cache_seq(seed, layer, b, ctx, n_kv_heads, head_dim=128, std=1.0):
    """KV cache of sequence b in one layer: (k, v) bf16 bits [ctx, Hkv, D] ~ N(0, std^2)."""
    return _kv_seq((seed, layer, b, ctx, n_kv_heads, head_dim, std))


def kv_cache_case(batch, ctx, n_kv_heads, seed=0, layer=0, std=1.0, workers=None):
    """KV cache of a batch, (k, v) bf16 bits [batch, ctx, Hkv, 128]; sequence b
    equals kv_cache_seq(seed, layer, b, ...)."""
    kc = np.empty((batch, ctx, n_kv_heads, 128), dtype=np.uint16)
    vc = np.empty((batch, ctx, n_kv_heads, 128), dtype=np.uint16)
    jobs = [(seed, layer, b, ctx, n_kv_heads, 128, std) for b in range(batch)]
    if workers is None:
        workers = min(16, len(os.sched_getaffinity(0)))
    if workers > 1 and batch * ctx * n_kv_heads * 128 > (1 << 24):
        with ProcessPoolExecutor(max_workers=workers) as ex:
            for b, (k, v) in enumerate(ex.map(_kv_seq, jobs, chunksize=max(1, batch // (4 * workers)))):
                kc[b], vc[b] = k, v
    else:
        for b, job in enumerate(jobs):
            kc[b], vc[b] = _kv_seq(job)
    return kc, vc


def block_positions(batch, block, ctx):
    """Clean row i of every sequence sits at position ctx + i and noisy row i
    at ctx + block + i (the noisy rows stand for the next block)."""
    per = np.arange(2 * block) + ctx
    return np.tile(per, batch).astype(np.int32)


def decoder_layer_case(batch, block, ctx, hidden, inter, n_heads, n_kv_heads, r, seed=0, layer=0,
                       weight_std=0.02, norm_std=0.1, kv_std=1.0, workers=None, x_std=1.0, lora_std=None,
                       qk_norm=True):
    """Inputs of one decoder layer over `batch` sequences of `block` clean +
    `block` noisy rows: residual stream h [rows, hidden] ~ N(0, x_std^2), gate
    (0 clean, 1 noisy), positions, KV cache [batch, ctx, Hkv, 128] ~
    N(0, kv_std^2) and the weights (all bf16 bits).  Sequence b's rows and
    cache can be regenerated alone with layer_seq_rows / kv_cache_seq."""
    rows = batch * 2 * block
    h = np.concatenate([layer_seq_rows(seed, b, block, hidden, x_std) for b in range(batch)], axis=0)
    kc, vc = kv_cache_case(batch, ctx, n_kv_heads, seed, layer, kv_std, workers)
    return {"batch": batch, "block": block, "ctx": ctx, "hidden": hidden, "inter": inter,
            "n_heads": n_heads, "n_kv_heads": n_kv_heads, "r": r, "seed": seed, "layer": layer,
            "h": h, "gate": default_gate(rows, block), "positions": block_positions(batch, block, ctx),
            "k_cache": kc, "v_cache": vc,
            "weights": layer_weights_case(hidden, inter, n_heads, n_kv_heads, r, seed, layer, weight_std,
                                          norm_std, lora_std, qk_norm)}


def rows_case(rows, vocab, dtype="bf16", seed=0, std=2.0):
    """Logits [rows, vocab] ~ N(0, std^2) in `dtype` storage and uniforms [rows]."""
    x = rng_for(seed, _T_ROWS_L).standard_normal((rows, vocab), dtype=np.float32) * np.float32(std)
    st, val = _store(x, dtype)
    u = rng_for(seed, _T_ROWS_U).random(rows, dtype=np.float32)
    return {"logits": st, "logits_f32": val, "u": u}


# ------------------------------------------------------------ decode step
_T_EMBED, _T_LMHEAD, _T_FNORM, _T_TOK, _T_UDRAFT, _T_UACC2, _T_US2 = 71, 72, 73, 74, 75, 76, 77


def step_case(batch, block, ctx, hidden, inter, n_heads, n_kv_heads, r, n_layers, vocab, seed=0,
              weight_std=0.02, embed_std=1.0, norm_std=0.1):
    """Inputs of one decode step: embedding and LM-head tables [vocab, hidden]
    (embedding ~ N(0, embed_std^2), LM head ~ N(0, weight_std^2)), final norm
    weights, n_layers layers (layer_weights_case) with their KV caches
    (kv_cache_case), token ids [batch, 2*block] uniform over the vocabulary,
    and the uniforms u_draft, u_accept [batch, block-1], u_sample [batch].
    All tables are bf16 bits; the values are the bf16 values."""
    k = block - 1
    emb = rng_for(seed, _T_EMBED).standard_normal((vocab, hidden), dtype=np.float32) * np.float32(embed_std)
    lm = rng_for(seed, _T_LMHEAD).standard_normal((vocab, hidden), dtype=np.float32) * np.float32(weight_std)
    fn = 1.0 + rng_for(seed, _T_FNORM).standard_normal(hidden, dtype=np.float32) * np.float32(norm_std)
    layers, kcs, vcs = [], [], []
    for l in range(n_layers):
        layers.append(layer_weights_case(hidden, inter, n_heads, n_kv_heads, r, seed, l, weight_std, norm_std))
        kc, vc = kv_cache_case(batch, ctx, n_kv_heads, seed, l)
        kcs.append(kc)
        vcs.append(vc)
    return {"batch": batch, "block": block, "ctx": ctx, "hidden": hidden, "inter": inter, "n_heads": n_heads,
            "n_kv_heads": n_kv_heads, "r": r, "n_layers": n_layers, "vocab": vocab,
            "embed": bf16_bits(emb), "lm_head": bf16_bits(lm), "final_norm": bf16_bits(fn),
            "layers": layers, "k_caches": kcs, "v_caches": vcs,
            "tokens": rng_for(seed, _T_TOK).integers(0, vocab, size=(batch, 2 * block)).astype(np.int32),
            "u_draft": rng_for(seed, _T_UDRAFT).random((batch, k), dtype=np.float32),
            "u_accept": rng_for(seed, _T_UACC2).random((batch, k), dtype=np.float32),
            "u_sample": rng_for(seed, _T_US2).random(batch, dtype=np.float32)}
