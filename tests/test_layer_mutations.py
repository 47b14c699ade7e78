"""Power of the GPU decoder-layer parity tests.

For every case the GPU layer tests run (tests/_layer_cases.py), each planted
wiring mistake of tests/_layer_mutations.py must move the oracle's output by
at least 3x the layer bar (row-wise max relative error 3e-2, the composite of
ten bf16 storage points; 9e-2, above 3x the single-operation bar of 2e-2 as
well), so that a GPU path making that mistake fails its parity test instead
of passing inside the tolerance.  The mistakes: a clean row seeing the noisy rows, wrong rotary
positions, SwiGLU operands swapped, each adapter group dropped, attention
dropped, the MLP norm reading the wrong residual, the per-head q/k norm
dropped.

Source of what the layer computes: Uno summary (hyper.ai, arXiv 2609.04010),
section 方法 (one forward over concatenated clean and noisy rows, the adapter
gated per row) and section 实验 (Qwen3-8B base).
"""

import numpy as np
import pytest

import oracle
import workloads
from _layer_cases import APPEND_CASES, BAR, FULL_CASES, LAYER_CASES, POWER, ids, make, make_seqs, seq_rows
from _layer_mutations import ADAPTER_MUTATIONS, MUTATIONS, mutated_layer, row_relerr


def _f64(bits):
    return workloads.bf16_to_f32(bits).astype(np.float64)


ALL = LAYER_CASES + APPEND_CASES + FULL_CASES


def test_sampled_sequences_regenerate_alone():
    """make_seqs (used below for the full-size cases) gives exactly the sampled
    sequences' part of the whole-batch inputs the GPU tests generate."""
    for c in (LAYER_CASES[7], APPEND_CASES[0]):
        d, s = make(c), make_seqs(c)
        seqs, rows = seq_rows(c)
        for name in ("h", "gate", "positions"):
            np.testing.assert_array_equal(s[name], d[name][rows])
        for name in ("k_cache", "v_cache"):
            np.testing.assert_array_equal(s[name], d[name][seqs])
        for name, v in d["weights"].items():
            np.testing.assert_array_equal(s["weights"][name], v)


@pytest.mark.parametrize("c", ALL, ids=ids(ALL))
def test_every_planted_mistake_exceeds_the_bar(c):
    d = make_seqs(c)
    w = {k[:-4]: v.astype(np.float64) for k, v in d["weights"].items() if k.endswith("_f32")}
    lens = d["lens"]
    args = (_f64(d["h"]), w, d["gate"], d["positions"], _f64(d["k_cache"]), _f64(d["v_cache"]), c["block"],
            c["nh"], c["nkv"])
    ref, _ = oracle.decoder_layer(*args, ctx_lens=lens)
    # the harness without a mistake is the oracle, bit for bit
    np.testing.assert_array_equal(mutated_layer(*args, mutation=None, ctx_lens=lens), ref)
    weak = {}
    for m in MUTATIONS:
        if m in ADAPTER_MUTATIONS and not c["gate"]:
            continue          # no adapter anywhere: nothing to drop
        if m == "positions_shift" and c["ctx"] == 0:
            continue          # no cache: a global shift is an exact symmetry of RoPE attention
        if m == "drop_qk_norm" and not c["qk_norm"]:
            continue          # the layer has no per-head norm to drop
        err = row_relerr(mutated_layer(*args, mutation=m, ctx_lens=lens), ref)
        if err < POWER * BAR:
            weak[m] = err
    assert not weak, f"planted mistakes within {POWER} x the bar: {weak}"
