"""GPU: the data-contract checks (UNO_DEBUG / uno_debug_checks) report token
ids and uniforms outside the contract as UNO_ERR_INVALID_ARGUMENT, and let
valid calls through unchanged."""

import numpy as np
import pytest

import workloads
from _parity import say, to_dev, to_host

pytestmark = pytest.mark.gpu


def _expect_invalid(fn):
    import diffusion_augmented_decoding_amd as dad
    with pytest.raises(dad.UnoError) as e:
        fn()
    assert e.value.status == 1, str(e.value)


def test_debug_checks_catch_contract_violations(gpu_lib):
    import torch
    say("debug checks on: verify, tree verify, sampler, step")
    was = gpu_lib.debug_checks()
    try:
        gpu_lib.debug_checks(True)
        c = workloads.verify_linear_case(3, 4, 500, 0.5, dtype="bf16", seed=2, workers=1)
        p, q, d, ua, us = (to_dev(c[n]) for n in ("p", "q", "drafts", "u_acc", "u_s"))
        ok = gpu_lib.psi_spec_verify_linear(p, q, d, ua, us)
        torch.cuda.synchronize()
        gpu_lib.debug_checks(False)
        ref = gpu_lib.psi_spec_verify_linear(p, q, d, ua, us)
        torch.cuda.synchronize()
        gpu_lib.debug_checks(True)
        np.testing.assert_array_equal(to_host(ok["token"]), to_host(ref["token"]))
        bad = d.clone()
        bad[1, 2] = 500                                   # vocab 500: out of range
        _expect_invalid(lambda: gpu_lib.psi_spec_verify_linear(p, q, bad, ua, us))
        bad[1, 2] = -1
        _expect_invalid(lambda: gpu_lib.psi_spec_verify_linear_sampled(p, q, bad, ua, us, 1.0, 5))
        ua2 = ua.clone()
        ua2[0, 0] = 1.0                                   # uniforms live in [0, 1)
        _expect_invalid(lambda: gpu_lib.psi_spec_verify_linear(p, q, d, ua2, us))
        us2 = us.clone()
        us2[2] = float("nan")
        _expect_invalid(lambda: gpu_lib.psi_spec_verify_linear_noalloc(p, q, d, ua, us2))
        # tree verify: a node token out of range (the root's is not checked)
        parent = workloads.tree_parent_cfg(0, branching=2, depth=2, n_last=2)
        cv = workloads.tree_verify_case(parent, 300, dtype="bf16", seed=1)
        tv = {kk: to_dev(cv[kk]) for kk in ("parent", "tokens", "p", "q", "u_acc", "u_s")}
        mc = workloads.max_children(parent)
        gpu_lib.psi_spec_verify_tree(tv["parent"], tv["tokens"], tv["p"], tv["q"], tv["u_acc"], tv["u_s"],
                                     max_children=mc)
        torch.cuda.synchronize()
        tb = tv["tokens"].clone()
        tb[0, 0] = 10 ** 6                                # root: unused, allowed
        gpu_lib.psi_spec_verify_tree(tv["parent"], tb, tv["p"], tv["q"], tv["u_acc"], tv["u_s"], max_children=mc)
        tb[0, 3] = 300
        _expect_invalid(lambda: gpu_lib.psi_spec_verify_tree(tv["parent"], tb, tv["p"], tv["q"], tv["u_acc"],
                                                             tv["u_s"], max_children=mc))
        # the row sampler's uniforms
        lg = to_dev(workloads.bf16_bits(np.zeros((2, 64), np.float32)))
        u = torch.tensor([0.5, 1.5], device="cuda")
        _expect_invalid(lambda: gpu_lib.sample_rows(lg, u))
    finally:
        gpu_lib.debug_checks(was)
