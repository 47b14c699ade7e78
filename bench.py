#!/usr/bin/env python3
"""Benchmark of the Psi-Spec decode-step hot path on one MI355X.

One step = one pass of every hot-path kernel over one batch of synthetic,
seeded inputs already resident in HBM:
  * gated-LoRA linear on the seven projections of a Qwen3-8B-shaped layer,
    1024 rows = 64 sequences x (8 clean + 8 noisy), rank 128, bf16;
  * linear Psi-Spec verify, batch 256 x block 16 (k = 15), vocab 151,936,
    bf16 logits, draft = AR + N(0, sigma^2);
  * tree verify at batch 1: tree-masked attention (65 nodes, 1K cache, GQA
    32/8) and per-node rejection over vocab 151,936.
value = verified tokens per second: the tokens the step's samplers emit
(sum over sequences of accepted length + 1, linear batch plus the tree)
divided by the step time.

    python bench.py [--steps K] [--warmup W] [--sigma S]

Prints one JSON line.
"""

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0

LAYER = [("q", 4096, 4096), ("k", 1024, 4096), ("v", 1024, 4096), ("o", 4096, 4096),
         ("gate", 12288, 4096), ("up", 12288, 4096), ("down", 4096, 12288)]
M_ROWS, RANK = 1024, 128
LIN_BATCH, LIN_K, VOCAB = 256, 15, 151936


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--sigma", type=float, default=0.5)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this build measures one GPU only; run with --gpus 1 "
                                   "(the hot path shards by sequence with no exchange; see the design notes)"}))
        sys.exit(2)

    import numpy as np
    import torch

    import diffusion_augmented_decoding_amd as dad
    import workloads

    dad.load()
    dev = torch.device("cuda:0")

    def up(a):
        a = np.ascontiguousarray(a)
        t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16) if a.dtype == np.uint16 else torch.from_numpy(a)
        return t.to(dev)

    # ------------------------------------------------------------ inputs
    t0 = time.time()
    lora = []
    for i, (name, n, k) in enumerate(LAYER):
        c = workloads.gated_lora_case(M_ROWS, n, k, RANK, dtype="bf16", seed=args.seed, tag=i)
        ws = torch.empty(dad.gated_lora_linear_workspace(dad.UNO_BF16, M_ROWS, n, k, RANK), dtype=torch.uint8,
                         device=dev)
        lora.append({"name": name, "n": n, "k": k, "x": up(c["x"]), "w": up(c["w"]), "a": up(c["a"]),
                     "b": up(c["b"]), "gate": up(c["gate"]), "ws": ws,
                     "y": torch.empty((M_ROWS, n), dtype=torch.bfloat16, device=dev),
                     "m_on": int(c["gate"].sum()), "host": c if name == "gate" else None})
    log(f"gated-LoRA inputs ready ({time.time() - t0:.1f}s)")
    lin = workloads.verify_linear_case(LIN_BATCH, LIN_K, VOCAB, args.sigma, dtype="bf16", seed=args.seed,
                                       keep_f32=False)
    lin_dev = {"p": up(lin["p"]), "q": up(lin["q"]), "d": up(lin["drafts"]), "ua": up(lin["u_acc"]),
               "us": up(lin["u_s"])}
    del lin["p"], lin["q"]
    lin_out = {"accept_len": torch.empty(LIN_BATCH, dtype=torch.int32, device=dev),
               "token": torch.empty(LIN_BATCH, dtype=torch.int32, device=dev)}
    lin_ws = torch.empty(dad.psi_spec_verify_linear_workspace(LIN_BATCH, LIN_K, VOCAB), dtype=torch.uint8,
                         device=dev)
    log(f"sampler inputs ready ({time.time() - t0:.1f}s)")
    parent = workloads.tree_parent_cfg(args.seed)
    ta = workloads.tree_attention_case(1, parent, 1024, 32, 8, 128, seed=args.seed)
    ta_dev = {k: up(ta[k]) for k in ("q", "k_cache", "v_cache", "k_tree", "v_tree")}
    ta_dev["parent"] = up(ta["parent"].astype(np.int32))
    ta_out = torch.empty_like(ta_dev["q"])
    ta_lse = torch.empty((1, ta["n"], 32), dtype=torch.float32, device=dev)
    tv = workloads.tree_verify_case(parent, VOCAB, dtype="bf16", seed=args.seed)
    tv_dev = {k: up(tv[k]) for k in ("parent", "tokens", "p", "q", "u_acc", "u_s")}
    tv_out = {"accept_len": torch.empty(1, dtype=torch.int32, device=dev),
              "path": torch.empty((1, tv["max_depth"]), dtype=torch.int32, device=dev),
              "token": torch.empty(1, dtype=torch.int32, device=dev)}
    tv_maxc = workloads.max_children(parent)
    tv_ws = torch.empty(dad.psi_spec_verify_tree_workspace(1, tv["n"], tv["max_depth"], tv_maxc, VOCAB),
                        dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    log(f"all inputs resident ({time.time() - t0:.1f}s)")

    def step():
        for e in lora:
            dad.gated_lora_linear(e["x"], e["w"], e["a"], e["b"], e["gate"], out=e["y"], workspace=e["ws"])
        dad.psi_spec_verify_linear(lin_dev["p"], lin_dev["q"], lin_dev["d"], lin_dev["ua"], lin_dev["us"],
                                   outputs=lin_out, workspace=lin_ws)
        dad.tree_verify_attention(ta_dev["q"], ta_dev["k_cache"], ta_dev["v_cache"], ta_dev["k_tree"],
                                  ta_dev["v_tree"], ta_dev["parent"], ta["scale"], out=ta_out, lse=ta_lse)
        dad.psi_spec_verify_tree(tv_dev["parent"], tv_dev["tokens"], tv_dev["p"], tv_dev["q"], tv_dev["u_acc"],
                                 tv_dev["u_s"], max_children=tv_maxc, outputs=tv_out, workspace=tv_ws)

    # ------------------------------------------------------------ warmup + per-kernel breakdown
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # per-kernel breakdown on two further untimed steps (after code loading)
    n_prof = 2
    dad.profile_reset()
    dad.profile_enable(True)
    for _ in range(n_prof):
        step()
    torch.cuda.synchronize()
    kernels = ["uno_gemm_bf16", "uno_gemm_reduce", "uno_lora_down_bf16", "uno_lora_gate", "uno_row_stats",
               "uno_accept", "uno_draw_seg", "uno_draw_resolve", "uno_tree_attention", "uno_tree_setup",
               "uno_tree_stats", "uno_tree_round", "uno_tree_walk", "uno_tree_draw"]
    breakdown = {}
    for kname in kernels:
        ms, cnt = dad.profile_query(kname)
        breakdown[kname] = ms / n_prof
    # per-projection GEMM times (one launch each, events around the main GEMM)
    per_proj = {}
    for e in lora:
        dad.profile_reset()
        dad.gated_lora_linear(e["x"], e["w"], e["a"], e["b"], e["gate"], out=e["y"], workspace=e["ws"])
        ms = sum(dad.profile_query(kn)[0] for kn in ("uno_gemm_bf16", "uno_gemm_reduce", "uno_lora_down_bf16",
                                                      "uno_lora_gate"))
        flops = 2.0 * M_ROWS * e["n"] * e["k"] + 2.0 * e["m_on"] * RANK * (e["k"] + e["n"])
        per_proj[e["name"]] = {"us": ms * 1e3, "tflops": flops / (ms * 1e-3) / 1e12}
    dad.profile_enable(False)
    dad.profile_reset()
    dominant = max(breakdown, key=breakdown.get)

    # ------------------------------------------------------------ timed region
    dad.profile_enable(True, dominant)
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    t_end = time.perf_counter()
    dom_ms, dom_cnt = dad.profile_query(dominant)
    dad.profile_enable(False)
    dad.profile_reset()
    ms_per_step = (t_end - t_start) * 1e3 / args.steps

    L = lin_out["accept_len"].cpu().numpy()
    tl = int(tv_out["accept_len"].cpu().numpy()[0])
    tokens_per_step = int(np.sum(L + 1)) + (tl + 1)
    value = tokens_per_step / (ms_per_step * 1e-3)

    # ------------------------------------------------------------ roofline of the dominant kernel
    gemm_flops_step = sum(2.0 * M_ROWS * e["n"] * e["k"] + 2.0 * e["m_on"] * RANK * (e["k"] + e["n"]) for e in lora)
    sampler_bytes = float(LIN_BATCH) * (2 * LIN_K + 1) * VOCAB * 2
    tree_stat_bytes = float(tv["n"] + tv["max_depth"]) * VOCAB * 2
    attn_bytes = float(2 * 1024 * 8 * 128 * 2 + ta["n"] * (32 + 2 * 8 + 32) * 128 * 2)
    per_launch_avg_ms = dom_ms / max(1, dom_cnt)
    launches_per_step = dom_cnt / args.steps
    if dominant == "uno_gemm_bf16":
        algo = gemm_flops_step / launches_per_step
        achieved = algo / (per_launch_avg_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": achieved, "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s"}
    else:
        algo = {"uno_row_stats": sampler_bytes, "uno_tree_stats": tree_stat_bytes,
                "uno_tree_attention": attn_bytes}.get(dominant, sampler_bytes)
        achieved = algo / (per_launch_avg_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = None
    roof["kernel"] = dominant
    roof["avg_launch_us"] = per_launch_avg_ms * 1e3

    gemm_ms = (breakdown["uno_gemm_bf16"] + breakdown["uno_gemm_reduce"] + breakdown["uno_lora_down_bf16"]
               + breakdown["uno_lora_gate"])
    sampler_ms = (breakdown["uno_row_stats"] + breakdown["uno_accept"] + breakdown["uno_draw_seg"]
                  + breakdown["uno_draw_resolve"])
    components = {
        "gated_lora_layer": {"us": gemm_ms * 1e3, "tflops": gemm_flops_step / (gemm_ms * 1e-3) / 1e12,
                             "mfma_frac": gemm_flops_step / (gemm_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
                             "per_projection": per_proj},
        "linear_verify": {"us": sampler_ms * 1e3,
                          "row_stats_gbs": sampler_bytes / (breakdown["uno_row_stats"] * 1e-3) / 1e9,
                          "row_stats_hbm_frac": sampler_bytes / (breakdown["uno_row_stats"] * 1e-3) / 1e9 / HBM_PEAK_GBS,
                          "mean_accept_len": float(np.mean(L)), "tokens": int(np.sum(L + 1))},
        "tree": {"attention_us": breakdown["uno_tree_attention"] * 1e3,
                 "verify_us": (breakdown["uno_tree_setup"] + breakdown["uno_tree_stats"] + breakdown["uno_tree_round"]
                               + breakdown["uno_tree_walk"] + breakdown["uno_tree_draw"]) * 1e3, "accept_len": tl},
        "kernel_ms_per_step": breakdown,
    }

    # ------------------------------------------------------------ CPU oracle baseline (bounded sample)
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(args, lin, lora, ta, tv, tokens_per_step)

    out = {
        "metric": "verified tokens/s per Psi-Spec step",
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; random-init Qwen3-8B-shaped weights, N(0, sigma^2) logits)",
        "config": {"workload": "psi_spec_hot_path_step",
                   "gated_lora": "7 projections of a Qwen3-8B-shaped layer, 1024 rows (64 seq x 8 clean + 8 noisy), r=128",
                   "linear_verify": f"batch {LIN_BATCH} x block 16 (k={LIN_K}), vocab {VOCAB}, sigma {args.sigma}",
                   "tree_verify": "batch 1, 65-node tree (branching 4, depth 3), ctx 1024, GQA 32/8, vocab 151936",
                   "tokens_per_step": tokens_per_step, "parallelism": "single GPU"},
        "roofline": roof,
        "cpu_baseline": cpu,
        "components": components,
    }
    print(json.dumps(out), flush=True)


def cpu_baseline(args, lin, lora, ta, tv, tokens_per_step):
    """The float64 CPU oracle, timed on a bounded sample of the same step."""
    import numpy as np

    import oracle
    import workloads
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        blas_threads = 1
    t_lora = 0.0
    rows = 16
    for i, (name, n, k) in enumerate(LAYER):
        c = workloads.gated_lora_case(rows, n, k, RANK, dtype="bf16", seed=args.seed + 1000, tag=i)
        t0 = time.perf_counter()
        oracle.gated_lora_linear(c["x_f32"], c["w_f32"], c["a_f32"], c["b_f32"], c["gate"])
        t_lora += time.perf_counter() - t0
    n_seq = 16
    t_lin = 0.0
    for b in range(n_seq):
        _, _, pf, qf, d = workloads.verify_linear_seq(args.seed, b, LIN_K, VOCAB, args.sigma, "bf16")
        t0 = time.perf_counter()
        oracle.verify_linear(pf[None], qf[None], d[None], lin["u_acc"][b:b + 1], lin["u_s"][b:b + 1])
        t_lin += time.perf_counter() - t0
    t0 = time.perf_counter()
    oracle.tree_attention(ta["q_f32"], ta["k_cache_f32"], ta["v_cache_f32"], ta["k_tree_f32"], ta["v_tree_f32"],
                          ta["parent"], ta["scale"])
    t_att = time.perf_counter() - t0
    t0 = time.perf_counter()
    oracle.verify_tree(tv["parent"], tv["tokens"], tv["p_f32"], tv["q_f32"], tv["u_acc"], tv["u_s"])
    t_tree = time.perf_counter() - t0
    step_s = t_lora * (M_ROWS / rows) + t_lin * (LIN_BATCH / n_seq) + t_att + t_tree
    return {"value": tokens_per_step / step_s, "unit": "tokens/s", "cores": blas_threads, "kind": "oracle",
            "sample": (f"gated LoRA on {rows} of {M_ROWS} rows per projection (x{M_ROWS // rows}), linear verify on "
                       f"{n_seq} of {LIN_BATCH} sequences (x{LIN_BATCH // n_seq}), tree attention and tree verify "
                       f"whole; float64 NumPy, BLAS threads = cores, sampler loops single-threaded"),
            "step_seconds_extrapolated": step_s}


if __name__ == "__main__":
    main()
