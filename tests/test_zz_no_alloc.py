"""GPU check of uno_psi_spec_verify_linear_noalloc, the allocation-free
linear verify (its scratch is the library's own per-GPU device array): two
calls in a row through the C ABI, the second on a smaller input, each
against uno_psi_spec_verify_linear (the same kernels with a caller
workspace) on the same inputs.  The outputs must be identical: accepted
lengths and tokens bit-exact, the probabilities and residual masses too
(same kernels, same fixed-order reductions), which is inside the oracle
comparison's bar of the linear verify tests.  The oracle itself checks two
sequences of each call."""

import numpy as np
import pytest

import oracle
import workloads
from _parity import check_linear, say, to_dev, to_host

pytestmark = pytest.mark.gpu


def test_noalloc_verify_matches_workspace_entry_point(gpu_lib):
    import torch
    for batch, k, vocab, sigma, dtype in ((64, 15, 151936, 0.5, "bf16"), (3, 7, 1001, 2.0, "f32")):
        say(f"verify_linear_noalloc batch={batch} k={k} V={vocab} {dtype}")
        c = workloads.verify_linear_case(batch, k, vocab, sigma, dtype=dtype, seed=batch + k)
        args = [to_dev(c[n]) for n in ("p", "q", "drafts", "u_acc", "u_s")]
        ref = gpu_lib.psi_spec_verify_linear(*args)
        outs = {"accept_len": torch.full((batch,), -7, dtype=torch.int32, device="cuda"),
                "token": torch.full((batch,), -7, dtype=torch.int32, device="cuda"),
                "p_draft": torch.zeros((batch, k), dtype=torch.float32, device="cuda"),
                "q_draft": torch.zeros((batch, k), dtype=torch.float32, device="cuda"),
                "residual_mass": torch.zeros(batch, dtype=torch.float32, device="cuda")}
        got = gpu_lib.psi_spec_verify_linear_noalloc(*args, outputs=outs)
        torch.cuda.synchronize()
        for name in ref:
            assert torch.equal(ref[name], got[name]), f"{name} differs from the workspace entry point"
        g = {name: to_host(v) for name, v in got.items()}
        assert np.all((g["accept_len"] >= 0) & (g["accept_len"] <= k))

        def rows(b):
            return c["p_f32"][b], c["q_f32"][b], c["drafts"][b], c["u_acc"][b], c["u_s"][b]

        ties = check_linear(rows, g, [0, batch - 1], k)
        say(f"  identical to the workspace entry point; L {g['accept_len'][:6].tolist()}, oracle near-ties {ties}")
