"""GPU parity of the candidate-tree construction (uno_psi_spec_build_tree)
against oracle.build_tree, with and without replacement.

Source: Uno summary (hyper.ai, arXiv 2609.04010), section 方法, last
paragraph (the tree sampler draws candidates from the diffusion path's
marginals); the shape and draw readings are the oracle's (a budget per depth,
breadth-first ids, inverse-CDF draws, siblings without replacement drawn from
q with the earlier siblings' tokens removed)."""

import numpy as np
import pytest

import oracle
import workloads
from _parity import say, to_dev, to_host, check_tree_build

pytestmark = pytest.mark.gpu

FULL_V = 151936


@pytest.fixture(scope="module")
def dad():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import diffusion_augmented_decoding_amd as m
    m.load()
    return m


def _run(dad, case, temperature, without, q_dev=None):
    import torch
    q = q_dev if q_dev is not None else to_dev(case["q"])
    u = to_dev(case["u_draw"])
    out = dad.psi_spec_build_tree(q, case["branching"], u, temperature, without)
    torch.cuda.synchronize()
    return to_host(out["parent"]), to_host(out["tokens"])


CASES = [  # (batch, branching, vocab, dtype, temperature)
    (3, [4, 2, 2], 1000, "f32", 1.0),
    (3, [4, 2, 2], 1000, "bf16", 0.7),
    (2, [3, 3], 8193, "bf16", 1.0),           # ragged chunk tail
    (2, [64], 100, "f32", 1.0),               # 64 siblings out of 100 tokens
    (64, [2, 2], 257, "f32", 1.3),            # many trees
    (1, [31, 32], 300, "bf16", 1.0),          # 1024 nodes, the maximum
    (1, [2] * 9, 50, "f32", 1.0),             # 1023 nodes over 9 levels
    (2, [1, 1, 1, 1], 64, "bf16", 1.0),       # a chain
]


@pytest.mark.parametrize("without", [False, True])
@pytest.mark.parametrize("batch,branching,vocab,dtype,temperature", CASES)
def test_build_matches_oracle(dad, batch, branching, vocab, dtype, temperature, without):
    say(f"build {batch} {branching} V={vocab} {dtype} T={temperature} without={without}")
    case = workloads.tree_build_case(batch, branching, vocab, dtype, seed=7 + vocab + len(branching))
    par, tok = _run(dad, case, temperature, without)
    ties = check_tree_build(case["q_f32"], branching, case["u_draw"], par, tok, temperature, without)
    assert ties <= max(1, tok.size // 100), f"{ties} near-ties"


@pytest.mark.parametrize("without", [False, True])
def test_build_full_vocabulary(dad, without):
    """V = 151,936, bf16, a 69-node tree per sequence (4, 4, 3 children per
    level), 4 sequences."""
    branching = [4, 4, 3]
    case = workloads.tree_build_case(4, branching, FULL_V, "bf16", seed=11)
    say(f"build full V, without={without}")
    par, tok = _run(dad, case, 1.0, without)
    ties = check_tree_build(case["q_f32"], branching, case["u_draw"], par, tok, 1.0, without)
    assert ties <= 2


def test_build_from_strided_noisy_rows(dad):
    """q given in place as the noisy rows of a step's logits [B, 2*block, V]:
    depth d draws from noisy row d of its sequence."""
    import torch
    block, V = 8, 3000
    branching = [3, 2, 2]
    case = workloads.tree_build_case(3, branching, V, "bf16", seed=5)
    full = np.zeros((3, 2 * block, V), dtype=np.uint16)
    full[:, block:block + 3] = case["q"]
    full[:, :block] = workloads.bf16_bits(np.full((3, block, V), 9.0, np.float32))   # must not be read
    dev = to_dev(full)
    par, tok = _run(dad, case, 1.0, True, q_dev=dev[:, block:block + 3])
    check_tree_build(case["q_f32"], branching, case["u_draw"], par, tok, 1.0, True)


def test_without_replacement_past_the_support(dad):
    """All of q's mass on two tokens: without replacement the later siblings
    take the smallest ids not drawn yet; with replacement every sibling stays
    in the support (the oracle pin's case)."""
    import torch
    V = 6
    ql = np.full((1, 1, V), -1.0e4, np.float32)
    ql[0, 0, 3] = ql[0, 0, 5] = 0.0
    u = np.array([[0.0, 0.7, 0.9, 0.1, 0.5, 0.2]], np.float32)
    for without, want in ((True, [-1, 5, 3, 0, 1, 2]), (False, [-1, 5, 5, 3, 5, 3])):
        out = dad.psi_spec_build_tree(to_dev(ql), [5], to_dev(u), 1.0, without)
        torch.cuda.synchronize()
        assert to_host(out["tokens"])[0].tolist() == want
        assert to_host(out["parent"])[0].tolist() == [-1, 0, 0, 0, 0, 0]


def test_build_is_deterministic(dad):
    import torch
    branching = [4, 4, 3]
    case = workloads.tree_build_case(2, branching, 20000, "bf16", seed=3)
    q, u = to_dev(case["q"]), to_dev(case["u_draw"])
    a = dad.psi_spec_build_tree(q, branching, u, 1.0, True)
    b = dad.psi_spec_build_tree(q, branching, u, 1.0, True)
    torch.cuda.synchronize()
    assert torch.equal(a["tokens"], b["tokens"]) and torch.equal(a["parent"], b["parent"])
