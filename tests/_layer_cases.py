"""The decoder-layer cases the GPU parity tests run, in one list.

tests/test_gpu_layer.py and tests/test_gpu_commit.py run these cases on the
GPU; tests/test_layer_mutations.py checks on the CPU, for every case, that
each planted wiring mistake moves the oracle's output by at least three times
the bf16 bar, so a GPU path with that mistake would fail the GPU test.

Scales: weights ~ N(0, 0.05^2) and a residual stream ~ N(0, 0.1^2), so the
layer's own update is of the size of its input and attention is far from
uniform; at the scale of a trained model's residual stream (N(0, 1)) with
weights ~ N(0, 0.02^2) the update is a few percent of the output and most
planted mistakes stay under the bar.

Positions: clean row j of a sequence sits at position ctx + j and noisy row j
at ctx + block + j (the noisy rows are the next block), with ctx the
sequence's count of valid cache rows.

Test infrastructure only.
"""

import numpy as np

import workloads

WEIGHT_STD = 0.05
X_STD = 0.1
# Bar for the layer's output hidden state (row-wise max relative error).  The
# single-operation bf16 bar is 2e-2 (each stage of the layer is held to it on
# its own in tests/test_gpu_layer.py).  The hidden state chains ten bf16
# storage points (the norm, q/k/v, the rotated q/k, the attention output, o and
# its residual add, the MLP norm, gate/up, the SwiGLU product, down and its
# residual add); at each, a value that fp32 and float64 accumulation place on
# opposite sides of a bf16 rounding boundary rounds one ulp apart (2^-8 to
# 2^-7 of the element) between two correct implementations, and later stages
# carry the difference on.  Allowing ~4 such ulps at a row's largest element
# gives 3e-2.
BAR = 3e-2
POWER = 3.0          # each planted mistake must move the output by POWER * BAR


def case(name, batch, block, ctx, hidden, inter, nh, nkv, r, packed=False, lens=None, seqs=None, gate=True,
         seed=None, qk_norm=True):
    """One GPU layer case.  lens: per-sequence valid cache rows (ctx is then
    the capacity, the decode loop's form); seqs: the sequences the oracle
    recomputes (None: all); gate False: no adapter anywhere; qk_norm False:
    a layer without the per-head q/k RMSNorm."""
    return {"name": name, "batch": batch, "block": block, "ctx": ctx, "hidden": hidden, "inter": inter,
            "nh": nh, "nkv": nkv, "r": r, "packed": packed, "lens": lens, "seqs": seqs, "gate": gate,
            "seed": batch + ctx if seed is None else seed, "qk_norm": qk_norm}


LAYER_CASES = [
    case("small", 2, 4, 40, 256, 512, 4, 2, 16),
    case("small_packed", 2, 4, 40, 256, 512, 4, 2, 16, packed=True),
    case("block16", 3, 16, 300, 512, 1024, 8, 2, 32),
    case("block16_packed", 3, 16, 300, 512, 1024, 8, 2, 32, packed=True),
    # no cache: a shift of every position is an exact symmetry here (RoPE
    # scores depend on relative positions only), so that mistake is exempt
    case("no_cache", 1, 3, 0, 128, 384, 2, 1, 8),
    # rank a multiple of 64 with adapters back to back: gate, up and SwiGLU
    # run as one GEMM (ragged feature tile: 1088 = 8.5 x 128)
    case("swiglu_fused_packed", 2, 8, 136, 512, 1088, 8, 2, 64, packed=True),
    case("swiglu_fused", 2, 8, 136, 512, 1088, 8, 2, 64),
    # 2048 rows: k and v as one two-segment GEMM, gate/up/SwiGLU as one GEMM
    case("rows2048_sampled", 64, 16, 40, 512, 1024, 8, 2, 64, packed=True, seqs=[3, 60], seed=21),
    case("no_adapters", 2, 8, 136, 512, 1088, 8, 2, 64, gate=False, seed=11),
    case("no_qk_norm", 2, 4, 40, 256, 512, 4, 2, 16, qk_norm=False, seed=12),
]

# decode-loop form: per-sequence cache lengths, the clean rows appended
APPEND_CASES = [
    # the last sequence has room for 2 of its 4 clean rows; the first has no cache
    case("append_small", 3, 4, 40, 256, 512, 4, 2, 16, lens=[0, 17, 38], seed=44),
    case("append_block16", 2, 16, 300, 256, 512, 4, 2, 16, lens=[250, 5], seed=316),
]


# the decode step's launch configuration (Qwen3-8B shapes, 128 x (16 + 16)
# rows, 8K cache, rank-128 adapters stored as the bench stores them); the
# oracle recomputes the sampled sequences
QWEN = dict(hidden=4096, inter=12288, nh=32, nkv=8, r=128)
FULL_CASES = [
    case("full_size", 128, 16, 8192, packed=True, seqs=[5, 120], seed=3, **QWEN),
    # decode-loop form: 8192 + 16 rows of capacity, a ragged sequence and one
    # with room for 1 of its 16 clean rows
    case("full_size_append", 128, 16, 8192 + 16, packed=True, seqs=[5, 120, 77], seed=4,
         lens=[6001 if b == 5 else 8191 if b == 120 else 8192 for b in range(128)], **QWEN),
]


def positions(lens, block):
    """Per sequence: clean row j at len + j, noisy row j at len + block + j."""
    return np.concatenate([np.arange(2 * block) + int(n) for n in lens]).astype(np.int32)


def make(c):
    """Seeded inputs of a case (workloads.decoder_layer_case at the scales above)."""
    d = workloads.decoder_layer_case(c["batch"], c["block"], c["ctx"], c["hidden"], c["inter"], c["nh"], c["nkv"],
                                     c["r"], seed=c["seed"], weight_std=WEIGHT_STD, x_std=X_STD,
                                     qk_norm=c["qk_norm"])
    if not c["gate"]:
        d["gate"] = np.zeros_like(d["gate"])
    if c["lens"] is not None:
        d["positions"] = positions(c["lens"], c["block"])
    return d


def make_seqs(c):
    """The inputs of the sampled sequences only (rows, caches) plus the
    weights, regenerated from their own seeded streams: equal to the
    corresponding parts of make(c) without generating the whole batch."""
    seqs, rows = seq_rows(c)
    h = np.concatenate([workloads.layer_seq_rows(c["seed"], b, c["block"], c["hidden"], X_STD) for b in seqs])
    kv = [workloads.kv_cache_seq(c["seed"], 0, b, c["ctx"], c["nkv"]) for b in seqs]
    gate = np.tile(np.concatenate([np.zeros(c["block"]), np.ones(c["block"])]).astype(np.uint8), len(seqs))
    if not c["gate"]:
        gate[:] = 0
    lens = [c["ctx"]] * c["batch"] if c["lens"] is None else c["lens"]
    return {"h": h, "gate": gate, "positions": positions([lens[b] for b in seqs], c["block"]),
            "k_cache": np.stack([k for k, _ in kv]), "v_cache": np.stack([v for _, v in kv]),
            "lens": None if c["lens"] is None else np.asarray(c["lens"])[seqs],
            "weights": workloads.layer_weights_case(c["hidden"], c["inter"], c["nh"], c["nkv"], c["r"], c["seed"],
                                                    0, WEIGHT_STD, qk_norm=c["qk_norm"])}


def seq_rows(c):
    """(sequence indices, row indices) the oracle recomputes."""
    seqs = list(range(c["batch"])) if c["seqs"] is None else list(c["seqs"])
    n = 2 * c["block"]
    return np.asarray(seqs), np.concatenate([np.arange(b * n, (b + 1) * n) for b in seqs])


def ids(cases):
    return [c["name"] for c in cases]
