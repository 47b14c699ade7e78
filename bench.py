#!/usr/bin/env python3
"""Benchmark of the Psi-Spec decode step on one MI355X.

Default workload ("psi_spec_full_step"): one whole decode step of a 36-layer
Qwen3-8B-shaped random-init stack (hidden 4096, MLP 12288, GQA 32/8,
head_dim 128, rank-128 gated LoRA on all seven projections, bf16), batch 128
x block 16 (16 clean + 16 noisy rows per sequence, 4096 rows), an 8K-token KV
cache per sequence and layer, vocab 151,936: token embeddings, 36 decoder
layers, final norm + LM head, the draft draw from the noisy rows and the
linear verify, all through uno_psi_spec_step on inputs already resident in
HBM.  value = verified tokens per second = sum over sequences of
(accepted length + 1) / step time.  The acceptance rate is an artefact of the
random weights; the step's work does not depend on it.

The same run also measures, as components, the other hot-path workloads:
the seven gated-LoRA projections of one layer at 1024 rows (MFMA
utilisation), the linear verify sampler at batch 256 x block 16 over the full
vocabulary (HBM bandwidth) and the tree path at batch 1 (tree attention +
tree verify).  `--workload hot_path` times those three together as the step
instead.

    python bench.py [--steps K] [--warmup W] [--sigma S] [--workload step|hot_path]

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

# the whole-step workload
FULL = dict(batch=128, block=16, ctx=8192, hidden=4096, inter=12288, n_heads=32, n_kv=8, r=128, n_layers=36,
            vocab=151936)
# the per-layer / sampler / tree workloads
LAYER = [("q", 4096, 4096), ("k", 1024, 4096), ("v", 1024, 4096), ("o", 4096, 4096),
         ("gate", 12288, 4096), ("up", 12288, 4096), ("down", 4096, 12288)]
M_ROWS, RANK = 1024, 128
LIN_BATCH, LIN_K, VOCAB = 256, 15, 151936


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def measured_traffic(summary, source):
    """HBM bytes per launch from a committed rocprofv3 counter summary, or None
    when the kernel source has changed since the counters were taken."""
    import hashlib
    try:
        text = open(os.path.join(ROOT, "profiles", summary)).read()
        src = open(os.path.join(ROOT, "diffusion_augmented_decoding_amd", "csrc", source), "rb").read()
    except OSError:
        return None
    fields = dict(line.split(None, 1) for line in text.splitlines()
                  if line.startswith(("traffic_bytes_per_launch", "source_sha256")))
    if fields.get("source_sha256", "").strip() != hashlib.sha256(src).hexdigest():
        return None
    return float(fields["traffic_bytes_per_launch"])


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        return 1


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--sigma", type=float, default=0.5)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--workload", choices=("step", "hot_path"), default="step")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-components", action="store_true", help="skip the per-layer/sampler/tree workloads")
    ap.add_argument("--copy-probe", action="store_true",
                    help="end with a plain 1 GiB device copy (calibrates HBM byte counters)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this build measures one GPU only; run with --gpus 1 "
                                   "(the path shards by sequence with no exchange; see the design notes)"}))
        sys.exit(2)

    import torch

    import diffusion_augmented_decoding_amd as dad

    dad.load()
    if args.workload == "step":
        out = bench_full_step(args, dad, torch)
        if not args.no_components:
            comp = bench_hot_path(args, dad, torch, steps=max(3, args.steps), warmup=2, with_cpu=False)
            out["components"]["layer_1024_rows"] = comp["components"]["gated_lora_layer"]
            out["components"]["linear_verify_256x16"] = comp["components"]["linear_verify"]
            out["components"]["tree_batch1"] = comp["components"]["tree"]
    else:
        out = bench_hot_path(args, dad, torch, steps=args.steps, warmup=args.warmup,
                             with_cpu=not args.no_cpu_baseline)
    if args.copy_probe:
        # a plain copy of known size: FETCH_SIZE / WRITE_SIZE of this kernel
        # give the scale between the counters and bytes moved
        src = torch.empty(1 << 29, dtype=torch.bfloat16, device="cuda")
        dst = torch.empty_like(src)
        src.fill_(1.0)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        out["copy_probe_bytes"] = {"read": 1 << 30, "write": 1 << 30}
    print(json.dumps(out), flush=True)


# ====================================================================== full step
def full_step_flops(m_on):
    """Algorithmic GEMM work of one step: base projections + on-row LoRA-up (main
    GEMM kernel), on-row LoRA-down (its own kernel), LM head."""
    f = FULL
    rows = f["batch"] * 2 * f["block"]
    qd, kvd = f["n_heads"] * 128, f["n_kv"] * 128
    shapes = [(qd, f["hidden"]), (kvd, f["hidden"]), (kvd, f["hidden"]), (f["hidden"], qd),
              (f["inter"], f["hidden"]), (f["inter"], f["hidden"]), (f["hidden"], f["inter"])]
    main = sum(2.0 * rows * n * k + 2.0 * m_on * f["r"] * n for n, k in shapes) * f["n_layers"]
    down = sum(2.0 * m_on * f["r"] * k for n, k in shapes) * f["n_layers"]
    head = 2.0 * rows * f["vocab"] * f["hidden"]
    return main + head, down


def full_step_attention_bytes():
    """Algorithmic HBM bytes of one block-attention launch: the KV cache of every
    sequence, the block's q, k, v and the output (bf16)."""
    f = FULL
    n = 2 * f["block"]
    kv = 2.0 * f["batch"] * f["ctx"] * f["n_kv"] * 128 * 2
    blk = f["batch"] * n * (2 * f["n_heads"] + 2 * f["n_kv"]) * 128 * 2
    return kv + blk


def bench_full_step(args, dad, torch):
    import numpy as np
    f = FULL
    dev = torch.device("cuda:0")
    B, blk, ctx, H, Hkv, V = f["batch"], f["block"], f["ctx"], f["n_heads"], f["n_kv"], f["vocab"]
    hid, inter, r, nl = f["hidden"], f["inter"], f["r"], f["n_layers"]
    rows, k = B * 2 * blk, blk - 1
    t0 = time.time()
    gen = torch.Generator(device=dev)
    gen.manual_seed(args.seed)

    def randn(shape, std):
        t = torch.empty(shape, dtype=torch.bfloat16, device=dev)
        t.normal_(0.0, std, generator=gen)
        return t

    qd, kvd = H * 128, Hkv * 128
    shapes = {"q": (qd, hid), "k": (kvd, hid), "v": (kvd, hid), "o": (hid, qd), "g": (inter, hid),
              "u": (inter, hid), "d": (hid, inter)}
    layers, keep = [], []
    for li in range(nl):
        w = {"attn_norm": 1.0 + randn((hid,), 0.1), "mlp_norm": 1.0 + randn((hid,), 0.1)}
        # the adapters of q/k/v and of gate/up are stored back to back, so each
        # group's LoRA-down runs as one launch
        a_qkv = randn((3 * r, hid), 0.02)
        a_gu = randn((2 * r, hid), 0.02)
        packed_a = {"q": a_qkv[:r], "k": a_qkv[r:2 * r], "v": a_qkv[2 * r:], "g": a_gu[:r], "u": a_gu[r:]}
        for p, (n_out, n_in) in shapes.items():
            w["w" + p] = randn((n_out, n_in), 0.02)
            w["a" + p] = packed_a[p] if p in packed_a else randn((r, n_in), 0.02)
            w["b" + p] = randn((n_out, r), 0.02)
        # ctx valid rows per sequence plus one block of free slots for the append
        kc = randn((B, ctx + blk, Hkv, 128), 1.0)
        vc = randn((B, ctx + blk, Hkv, 128), 1.0)
        keep.append((w, kc, vc))
        layers.append(dad.layer_weights(w, kc, vc))
    arr = dad.layer_array(layers)
    embed = randn((V, hid), 1.0)
    lm_head = randn((V, hid), 0.02)
    final_norm = 1.0 + randn((hid,), 0.1)
    tokens = torch.randint(0, V, (B, 2 * blk), dtype=torch.int32, device=dev, generator=gen)
    u_draft = torch.rand((B, k), dtype=torch.float32, device=dev, generator=gen)
    u_accept = torch.rand((B, k), dtype=torch.float32, device=dev, generator=gen)
    u_sample = torch.rand((B,), dtype=torch.float32, device=dev, generator=gen)
    cfg = dad.step_config(B, blk, ctx + blk, hid, inter, H, Hkv, r, nl, V)
    # the decode loop's form: every layer appends the block's clean keys and
    # values after the ctx valid rows and the step commits the kept ones; the
    # lengths go back to ctx before each step so every step does the same work
    cache_len0 = torch.full((B,), ctx, dtype=torch.int32, device=dev)
    cache_len = cache_len0.clone()
    logits = torch.empty((rows, V), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(dad.psi_spec_step_workspace(cfg), dtype=torch.uint8, device=dev)
    outs = {"drafts": torch.empty((B, k), dtype=torch.int32, device=dev),
            "accept_len": torch.empty(B, dtype=torch.int32, device=dev),
            "token": torch.empty(B, dtype=torch.int32, device=dev)}
    torch.cuda.synchronize()
    log(f"full step: inputs resident ({time.time() - t0:.1f}s, "
        f"{torch.cuda.memory_allocated() / 2**30:.1f} GiB allocated)")

    def step():
        cache_len.copy_(cache_len0)
        dad.psi_spec_step(cfg, arr, embed, final_norm, lm_head, tokens, u_draft, u_accept, u_sample,
                          logits=logits, outputs=outs, workspace=ws, cache_len=cache_len)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log("full step: warm")

    # per-kernel breakdown over two untimed steps
    n_prof = 2
    dad.profile_reset()
    dad.profile_enable(True)
    for _ in range(n_prof):
        step()
    torch.cuda.synchronize()
    names = ["uno_step_setup", "uno_rms_norm", "uno_add_rms_norm", "uno_rope", "uno_silu_mul", "uno_lora_down_bf16",
             "uno_lora_gate", "uno_gemm_bf16", "uno_gemm_reduce", "uno_block_attention", "uno_sample_stats",
             "uno_sample_desc", "uno_sample_seg", "uno_sample_resolve", "uno_row_stats", "uno_accept",
             "uno_draw_seg", "uno_draw_resolve", "uno_kv_commit"]
    breakdown = {}
    for kn in names:
        ms, cnt = dad.profile_query(kn)
        breakdown[kn] = ms / n_prof
    # the attention entry counts its combine launches too (substring match)
    dad.profile_enable(False)
    dad.profile_reset()
    dominant = max(("uno_gemm_bf16", "uno_block_attention"), key=breakdown.get)
    log(f"full step: breakdown {json.dumps({k: round(v, 3) for k, v in breakdown.items()})}")

    # timed region; events around the dominant kernel's launches only
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

    L = outs["accept_len"].cpu().numpy()
    tokens_per_step = int(np.sum(L + 1))
    value = tokens_per_step / (ms_per_step * 1e-3)

    m_on = B * blk
    gemm_flops, down_flops = full_step_flops(m_on)
    attn_bytes = full_step_attention_bytes()
    launches_per_step = dom_cnt / args.steps
    per_launch_ms = dom_ms / max(1, dom_cnt)
    if dominant == "uno_gemm_bf16":
        algo = gemm_flops / launches_per_step
        roof = {"bound": "mfma", "achieved": algo / (per_launch_ms * 1e-3) / 1e12, "peak": MFMA_BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s"}
    else:
        algo = attn_bytes
        roof = {"bound": "hbm", "achieved": algo / (per_launch_ms * 1e-3) / 1e9, "peak": HBM_PEAK_GBS,
                "unit": "GB/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = (measured_traffic("uno_gemm_bf16_full_step_traffic.txt", "gated_lora.hip")
                       if dominant == "uno_gemm_bf16" else None)
    roof["kernel"] = dominant
    roof["avg_launch_us"] = per_launch_ms * 1e3
    roof["launches_per_step"] = launches_per_step

    gemm_ms = breakdown["uno_gemm_bf16"] + breakdown["uno_gemm_reduce"]
    attn_ms = breakdown["uno_block_attention"]
    kv_bytes_step = attn_bytes * nl
    sampler_ms = sum(breakdown[n] for n in ("uno_sample_stats", "uno_sample_desc", "uno_sample_seg",
                                            "uno_sample_resolve", "uno_row_stats", "uno_accept", "uno_draw_seg",
                                            "uno_draw_resolve"))
    sampler_bytes = float(B) * (3 * k + 1) * V * 2          # draft rows once, verify rows once
    gemm_s, attn_s = gemm_flops / (MFMA_BF16_PEAK_TFLOPS * 1e12), kv_bytes_step / (HBM_PEAK_GBS * 1e9)
    lower_bound_ms = (gemm_s + attn_s) * 1e3
    components = {
        "step_lower_bound_ms": lower_bound_ms,
        "step_frac_of_lower_bound": lower_bound_ms / ms_per_step,
        "gemm": {"ms": gemm_ms, "tflop": gemm_flops / 1e12, "tflops": gemm_flops / (gemm_ms * 1e-3) / 1e12,
                 "mfma_frac": gemm_flops / (gemm_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS},
        "lora_down": {"ms": breakdown["uno_lora_down_bf16"] + breakdown["uno_lora_gate"],
                      "tflop": down_flops / 1e12},
        "block_attention": {"ms": attn_ms, "gb": kv_bytes_step / 1e9,
                            "gbs": kv_bytes_step / (attn_ms * 1e-3) / 1e9,
                            "hbm_frac": kv_bytes_step / (attn_ms * 1e-3) / 1e9 / HBM_PEAK_GBS},
        "norm_rope_silu_ms": sum(breakdown[n] for n in ("uno_rms_norm", "uno_add_rms_norm", "uno_rope",
                                                        "uno_silu_mul", "uno_step_setup")),
        "sampler": {"ms": sampler_ms, "gb": sampler_bytes / 1e9, "gbs": sampler_bytes / (sampler_ms * 1e-3) / 1e9},
        "mean_accept_len": float(np.mean(L)),
        "kernel_ms_per_step": breakdown,
    }
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline_step(args, tokens_per_step)
    del keep, layers, arr, embed, lm_head, logits, ws
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return {
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
        "data": "synthetic (seeded on the device; random-init Qwen3-8B-shaped weights, N(0,1) KV cache, "
                "uniform token ids)",
        "config": {"workload": "psi_spec_full_step",
                   "model": "36-layer Qwen3-8B-shaped stack, hidden 4096, MLP 12288, GQA 32/8, head_dim 128, "
                            "rank-128 gated LoRA on q/k/v/o/gate/up/down, vocab 151936",
                   "batch": B, "block": blk, "rows": rows, "ctx_len": ctx, "drafts_per_seq": k,
                   "kv_cache": "decode loop: ctx_len valid rows per sequence; each layer appends the block's "
                               "clean k/v and the step commits the kept rows (lengths reset before each step)",
                   "tokens_per_step": tokens_per_step, "parallelism": "single GPU"},
        "roofline": roof,
        "cpu_baseline": cpu,
        "components": components,
    }


def cpu_baseline_step(args, tokens_per_step):
    """The float64 oracle on a bounded sample of the whole step: 2 of the 128
    sequences (32 rows each) through 36 applications of one full-size layer
    over that sequence's 8K cache (the layer's values do not change its cost),
    the LM head over a 1/16 slice of the vocabulary, and the draft draw +
    verify of one sequence at the full vocabulary; scaled to 128 sequences,
    36 layers and the whole vocabulary."""
    import numpy as np

    import oracle
    import workloads
    f = FULL
    blk, ctx, V, hid = f["block"], f["ctx"], f["vocab"], f["hidden"]
    n_seq, n_apply = 2, 36
    gate, pos = oracle.step_rows(1, blk, ctx)
    w = workloads.layer_weights_case(hid, f["inter"], f["n_heads"], f["n_kv"], f["r"], args.seed, 0)
    w64 = {kk[:-4]: v.astype(np.float64) for kk, v in w.items() if kk.endswith("_f32")}
    t_layers = 0.0
    hs = []
    for b in range(n_seq):
        h = workloads.bf16_to_f32(workloads.layer_seq_rows(args.seed, b, blk, hid)).astype(np.float64)
        kc, vc = workloads.kv_cache_seq(args.seed, 0, b, ctx, f["n_kv"])
        kc = workloads.bf16_to_f32(kc).astype(np.float64)[None]
        vc = workloads.bf16_to_f32(vc).astype(np.float64)[None]
        t0 = time.perf_counter()
        for _ in range(n_apply):
            h, _ = oracle.decoder_layer(h, w64, gate, pos, kc, vc, blk, f["n_heads"], f["n_kv"])
        t_layers += time.perf_counter() - t0
        hs.append(h)
    vs = V // 16
    rng = workloads.rng_for(args.seed, 999)
    w_lm = workloads.round_bf16(rng.standard_normal((vs, hid), dtype=np.float32) * np.float32(0.02)).astype(np.float64)
    t0 = time.perf_counter()
    oracle.lm_head(hs[0], np.ones(hid), w_lm)
    t_head = (time.perf_counter() - t0) * 16
    lg = workloads.round_bf16(rng.standard_normal((2 * blk, V), dtype=np.float32) * np.float32(2.0)).astype(np.float64)
    ud = rng.random((1, blk - 1))
    ua = rng.random((1, blk - 1))
    us = rng.random(1)
    t0 = time.perf_counter()
    d = np.array([[oracle.inverse_cdf(oracle.softmax_rows(lg[blk + i]), ud[0, i]) for i in range(blk - 1)]])
    oracle.verify_linear(lg[None, :blk], lg[None, blk:2 * blk - 1], d, ua, us)
    t_samp = time.perf_counter() - t0
    per_seq = t_layers / (n_seq * n_apply) * f["n_layers"] + t_head + t_samp
    step_s = per_seq * f["batch"]
    return {"value": tokens_per_step / step_s, "unit": "tokens/s", "cores": blas_threads(), "kind": "oracle",
            "sample": (f"{n_seq} of {f['batch']} sequences through {n_apply} applications of one full-size layer "
                       f"(x{f['n_layers'] / n_apply:g} layers), LM head on 1/16 of the vocabulary (x16), draft "
                       f"draw + verify of one sequence; scaled x{f['batch']} sequences; float64 NumPy, BLAS threads "
                       f"= cores, sampler loops single-threaded"),
            "step_seconds_extrapolated": step_s,
            "sample_seconds": t_layers + t_head / 16 + t_samp}


# ====================================================================== hot-path workloads
def bench_hot_path(args, dad, torch, steps, warmup, with_cpu):
    """The seven gated-LoRA projections of one layer at 1024 rows, the linear
    verify at batch 256 x block 16, and tree attention + tree verify at batch
    1, run back to back as one step."""
    import numpy as np

    import workloads
    dev = torch.device("cuda:0")

    def up(a):
        a = np.ascontiguousarray(a)
        t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16) if a.dtype == np.uint16 else torch.from_numpy(a)
        return t.to(dev)

    t0 = time.time()
    lora = []
    for i, (name, n, k) in enumerate(LAYER):
        c = workloads.gated_lora_case(M_ROWS, n, k, RANK, dtype="bf16", seed=args.seed, tag=i)
        ws = torch.empty(dad.gated_lora_linear_workspace(dad.UNO_BF16, M_ROWS, n, k, RANK), dtype=torch.uint8,
                         device=dev)
        lora.append({"name": name, "n": n, "k": k, "x": up(c["x"]), "w": up(c["w"]), "a": up(c["a"]),
                     "b": up(c["b"]), "gate": up(c["gate"]), "ws": ws,
                     "y": torch.empty((M_ROWS, n), dtype=torch.bfloat16, device=dev),
                     "m_on": int(c["gate"].sum())})
    log(f"hot path: gated-LoRA inputs ready ({time.time() - t0:.1f}s)")
    lin = workloads.verify_linear_case(LIN_BATCH, LIN_K, VOCAB, args.sigma, dtype="bf16", seed=args.seed,
                                       keep_f32=False)
    lin_dev = {"p": up(lin["p"]), "q": up(lin["q"]), "d": up(lin["drafts"]), "ua": up(lin["u_acc"]),
               "us": up(lin["u_s"])}
    del lin["p"], lin["q"]
    lin_out = {"accept_len": torch.empty(LIN_BATCH, dtype=torch.int32, device=dev),
               "token": torch.empty(LIN_BATCH, dtype=torch.int32, device=dev)}
    lin_ws = torch.empty(dad.psi_spec_verify_linear_workspace(LIN_BATCH, LIN_K, VOCAB), dtype=torch.uint8,
                         device=dev)
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
    log(f"hot path: all inputs resident ({time.time() - t0:.1f}s)")

    def step():
        for e in lora:
            dad.gated_lora_linear(e["x"], e["w"], e["a"], e["b"], e["gate"], out=e["y"], workspace=e["ws"])
        dad.psi_spec_verify_linear(lin_dev["p"], lin_dev["q"], lin_dev["d"], lin_dev["ua"], lin_dev["us"],
                                   outputs=lin_out, workspace=lin_ws)
        dad.tree_verify_attention(ta_dev["q"], ta_dev["k_cache"], ta_dev["v_cache"], ta_dev["k_tree"],
                                  ta_dev["v_tree"], ta_dev["parent"], ta["scale"], out=ta_out, lse=ta_lse)
        dad.psi_spec_verify_tree(tv_dev["parent"], tv_dev["tokens"], tv_dev["p"], tv_dev["q"], tv_dev["u_acc"],
                                 tv_dev["u_s"], max_children=tv_maxc, outputs=tv_out, workspace=tv_ws)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
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

    dad.profile_enable(True, dominant)
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    t_end = time.perf_counter()
    dom_ms, dom_cnt = dad.profile_query(dominant)
    dad.profile_enable(False)
    dad.profile_reset()
    ms_per_step = (t_end - t_start) * 1e3 / steps

    L = lin_out["accept_len"].cpu().numpy()
    tl = int(tv_out["accept_len"].cpu().numpy()[0])
    tokens_per_step = int(np.sum(L + 1)) + (tl + 1)
    value = tokens_per_step / (ms_per_step * 1e-3)

    gemm_flops_step = sum(2.0 * M_ROWS * e["n"] * e["k"] + 2.0 * e["m_on"] * RANK * (e["k"] + e["n"]) for e in lora)
    sampler_bytes = float(LIN_BATCH) * (2 * LIN_K + 1) * VOCAB * 2
    tree_stat_bytes = float(tv["n"] + tv["max_depth"]) * VOCAB * 2
    attn_bytes = float(2 * 1024 * 8 * 128 * 2 + ta["n"] * (32 + 2 * 8 + 32) * 128 * 2)
    per_launch_avg_ms = dom_ms / max(1, dom_cnt)
    launches_per_step = dom_cnt / steps
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
        "linear_verify": {"us": sampler_ms * 1e3, "sigma": args.sigma,
                          "row_stats_gbs": sampler_bytes / (breakdown["uno_row_stats"] * 1e-3) / 1e9,
                          "row_stats_hbm_frac": sampler_bytes / (breakdown["uno_row_stats"] * 1e-3) / 1e9 / HBM_PEAK_GBS,
                          "mean_accept_len": float(np.mean(L)), "tokens": int(np.sum(L + 1)),
                          "verified_tokens_per_s": int(np.sum(L + 1)) / (sampler_ms * 1e-3)},
        "tree": {"attention_us": breakdown["uno_tree_attention"] * 1e3,
                 "verify_us": (breakdown["uno_tree_setup"] + breakdown["uno_tree_stats"] + breakdown["uno_tree_round"]
                               + breakdown["uno_tree_walk"] + breakdown["uno_tree_draw"]) * 1e3, "accept_len": tl},
        "kernel_ms_per_step": breakdown,
    }
    cpu = cpu_baseline_hot_path(args, lin, ta, tv, tokens_per_step) if with_cpu else None
    del lora, lin_dev, ta_dev, tv_dev
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return {
        "metric": "verified tokens/s per Psi-Spec step",
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
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


def cpu_baseline_hot_path(args, lin, ta, tv, tokens_per_step):
    """The float64 CPU oracle, timed on a bounded sample of the hot-path step."""
    import oracle
    import workloads
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
    return {"value": tokens_per_step / step_s, "unit": "tokens/s", "cores": blas_threads(), "kind": "oracle",
            "sample": (f"gated LoRA on {rows} of {M_ROWS} rows per projection (x{M_ROWS // rows}), linear verify on "
                       f"{n_seq} of {LIN_BATCH} sequences (x{LIN_BATCH // n_seq}), tree attention and tree verify "
                       f"whole; float64 NumPy, BLAS threads = cores, sampler loops single-threaded"),
            "step_seconds_extrapolated": step_s}


if __name__ == "__main__":
    main()
