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
    ap.add_argument("--unmerged", action="store_true",
                    help="full step without gate-merged weights: every projection runs the LoRA-down path")
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
            out["components"]["linear_verify_sigma_sweep"] = bench_linear_sigma_sweep(args, dad, torch)
            out["components"]["tree_batch1_graph"] = bench_tree_graph(args, dad, torch)
            out["components"]["tree_batch16_built"] = bench_tree_batch(args, dad, torch)
            out["components"]["distill_loss_128x16"] = bench_distill(args, dad, torch)
            out["components"]["gated_lora_backward_1024_rows"] = bench_lora_backward(args, dad, torch)
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
def full_step_flops(m_on, merged=False):
    """GEMM work of one step: base projections + on-row LoRA-up (main GEMM
    kernel), on-row LoRA-down (its own kernel), LM head.  merged: the gated
    rows read W + B A, so the main GEMM does 2 M N K per projection and there
    is no LoRA-down (the work executed; the adapter's own flops are not
    credited)."""
    f = FULL
    rows = f["batch"] * 2 * f["block"]
    qd, kvd = f["n_heads"] * 128, f["n_kv"] * 128
    shapes = [(qd, f["hidden"]), (kvd, f["hidden"]), (kvd, f["hidden"]), (f["hidden"], qd),
              (f["inter"], f["hidden"]), (f["inter"], f["hidden"]), (f["hidden"], f["inter"])]
    up = 0.0 if merged else 1.0
    main = sum(2.0 * rows * n * k + up * 2.0 * m_on * f["r"] * n for n, k in shapes) * f["n_layers"]
    down = up * sum(2.0 * m_on * f["r"] * k for n, k in shapes) * f["n_layers"]
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
    # the decode loop: every step may keep up to a block of rows, so the
    # caches hold ctx valid rows plus a block of room for every step run
    n_prof = 2
    n_total = args.warmup + n_prof + args.steps
    if n_total > 512:
        raise SystemExit("at most 512 warmup + timed steps (the KV capacity grows with the step count)")
    cap = ctx + blk * (n_total + 1)
    layers, keep = [], []
    for li in range(nl):
        w = {"attn_norm": 1.0 + randn((hid,), 0.1), "mlp_norm": 1.0 + randn((hid,), 0.1),
             "q_norm": 1.0 + randn((128,), 0.1), "k_norm": 1.0 + randn((128,), 0.1)}
        # the adapters of q/k/v and of gate/up are stored back to back, so each
        # group's LoRA-down runs as one launch
        a_qkv = randn((3 * r, hid), 0.02)
        a_gu = randn((2 * r, hid), 0.02)
        packed_a = {"q": a_qkv[:r], "k": a_qkv[r:2 * r], "v": a_qkv[2 * r:], "g": a_gu[:r], "u": a_gu[r:]}
        for p, (n_out, n_in) in shapes.items():
            w["w" + p] = randn((n_out, n_in), 0.02)
            w["a" + p] = packed_a[p] if p in packed_a else randn((r, n_in), 0.02)
            w["b" + p] = randn((n_out, r), 0.02)
        if not args.unmerged:
            # load-time set-up: the gated (noisy) rows read W + B A
            dad.merge_layer(w)
        kc = randn((B, cap, Hkv, 128), 1.0)
        vc = randn((B, cap, Hkv, 128), 1.0)
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
    cfg = dad.step_config(B, blk, cap, hid, inter, H, Hkv, r, nl, V)
    # the decode loop's form: each step takes the previous step's next ids
    # (written in place over `tokens`), verifies their drafts against the
    # previous step's noisy-row logits (two logits buffers used in turn),
    # appends its clean keys and values in every layer and commits the kept
    # rows, so the caches grow from ctx rows by the emitted tokens
    cache_len = torch.full((B,), ctx, dtype=torch.int32, device=dev)
    bufs = [torch.empty((rows, V), dtype=torch.bfloat16, device=dev) for _ in range(2)]
    ws = torch.empty(dad.psi_spec_step_workspace(cfg), dtype=torch.uint8, device=dev)
    outs = {"drafts": torch.empty((B, k), dtype=torch.int32, device=dev),
            "accept_len": torch.empty(B, dtype=torch.int32, device=dev),
            "token": torch.empty(B, dtype=torch.int32, device=dev)}
    torch.cuda.synchronize()
    log(f"full step: inputs resident ({time.time() - t0:.1f}s, "
        f"{torch.cuda.memory_allocated() / 2**30:.1f} GiB allocated, capacity {cap} rows per sequence)")
    state = {"t": 0}

    def step():
        t = state["t"]
        prev = None if t == 0 else dad.noisy_rows(bufs[(t - 1) % 2], cfg)
        dad.psi_spec_step(cfg, arr, embed, final_norm, lm_head, tokens, u_draft, u_accept, u_sample,
                          prev_q=prev, logits=bufs[t % 2], outputs=outs, workspace=ws, cache_len=cache_len,
                          next_tokens=tokens)
        state["t"] = t + 1

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
             "uno_draw_seg", "uno_draw_resolve", "uno_step_finish"]
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
    len_start = cache_len.cpu().numpy().astype(np.int64)
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

    # every step keeps L + 1 rows per sequence and emits L + 1 tokens (L
    # accepted drafts and y), so the growth of the cache lengths over the
    # timed steps counts the verified tokens
    len_end = cache_len.cpu().numpy().astype(np.int64)
    L = outs["accept_len"].cpu().numpy()
    assert np.all(L >= 0), "a sequence ran out of KV capacity"
    tokens_timed = int(np.sum(len_end - len_start))
    tokens_per_step = tokens_timed / args.steps
    value = tokens_timed / (args.steps * ms_per_step * 1e-3)

    m_on = B * blk
    gemm_flops, down_flops = full_step_flops(m_on, merged=not args.unmerged)
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
    sampler_bytes = float(B) * (3 * k + 1) * V * 2          # draft rows, verify's p rows and carried q rows
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
        "mean_accept_len": tokens_per_step / B - 1.0,
        "kernel_ms_per_step": breakdown,
    }
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline_step(args, tokens_per_step)
    del keep, layers, arr, embed, lm_head, bufs, ws
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
                            "per-head q/k RMSNorm, rank-128 gated LoRA on q/k/v/o/gate/up/down, vocab 151936",
                   "batch": B, "block": blk, "rows": rows, "ctx_len": ctx, "drafts_per_seq": k,
                   "kv_cache": "decode loop: ctx_len valid rows per sequence at the first step; each layer "
                               "appends the block's clean k/v and the step commits the kept rows, so the cache "
                               "grows by the emitted tokens",
                   "decode_loop": "chained: each step takes the previous step's ids [y, drafts, noisy ids] and "
                                  "verifies the drafts against the previous step's noisy-row logits",
                   "ctx_len_timed_mean": float((len_start.mean() + len_end.mean()) / 2),
                   "lora": ("LoRA-down over the noisy rows + [x|T][W|B]^T" if args.unmerged else
                            "gate-merged weights set up at load (uno_lora_merge): clean rows x W^T, noisy rows "
                            "x (W + B A)^T, no LoRA-down in the step"),
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
               "uno_accept", "uno_draw_seg", "uno_draw_resolve", "uno_tree_attention", "uno_tree_stats",
               "uno_tree_flow"]
    breakdown = {}
    for kname in kernels:
        ms, cnt = dad.profile_query(kname)
        breakdown[kname] = ms / n_prof
    # each projection timed over 20 passes of the whole layer: the layer's
    # weights (386 MB) exceed the memory-side cache, so no projection finds
    # its weights cached from its previous call
    n_rep = 20
    names = ("uno_gemm_bf16", "uno_gemm_reduce", "uno_lora_down_bf16", "uno_lora_gate")
    proj_ms = {e["name"]: 0.0 for e in lora}
    dad.profile_enable(False)
    for _ in range(n_rep):
        for e in lora:
            dad.profile_reset()
            dad.profile_enable(True)
            dad.gated_lora_linear(e["x"], e["w"], e["a"], e["b"], e["gate"], out=e["y"], workspace=e["ws"])
            dad.profile_enable(False)
            torch.cuda.synchronize()
            proj_ms[e["name"]] += sum(dad.profile_query(kn)[0] for kn in names) / n_rep
    per_proj = {}
    for e in lora:
        ms = proj_ms[e["name"]]
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
                 "verify_us": (breakdown["uno_tree_stats"] + breakdown["uno_tree_flow"]) * 1e3, "accept_len": tl},
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


def bench_linear_sigma_sweep(args, dad, torch, sigmas=(0.1, 0.5, 2.0), reps=20):
    """The linear verify at batch 256 x block 16 (k = 15), V = 151,936, bf16, for
    several draft/target distances sigma: AR logits ~ N(0, 2^2), draft logits =
    AR logits + N(0, sigma^2), drafts by Gumbel-max from the draft rows (the
    distribution of workloads.verify_linear_case, generated on the device).
    Reports the verify's time (HIP events around its launches), its HBM rate
    over the rows it reads, the mean accepted length, and two lower bounds at
    the 8 TB/s peak: reading every row once (what this design reads), and
    reading only the rows an early exit at the first rejection would need
    (p and q rows 0..L, plus the residual or bonus rows of the draw); then the
    early-exit verify itself on the same inputs, its rate over those rows."""
    import numpy as np
    dev = torch.device("cuda:0")
    B, k, V = LIN_BATCH, LIN_K, VOCAB
    gen = torch.Generator(device=dev)
    gen.manual_seed(args.seed + 1)
    ws = torch.empty(dad.psi_spec_verify_linear_workspace(B, k, V), dtype=torch.uint8, device=dev)
    out = {"accept_len": torch.empty(B, dtype=torch.int32, device=dev),
           "token": torch.empty(B, dtype=torch.int32, device=dev)}
    names = ("uno_row_stats", "uno_accept", "uno_draw_seg", "uno_draw_resolve")
    res = []
    for sigma in sigmas:
        lp = torch.randn((B, k + 1, V), device=dev, generator=gen) * 2.0
        lq = lp[:, :k] + torch.randn((B, k, V), device=dev, generator=gen) * sigma
        p = lp.to(torch.bfloat16)
        q = lq.to(torch.bfloat16)
        del lp, lq
        g = -torch.log(-torch.log(torch.rand((B, k, V), device=dev, generator=gen).clamp_(1e-30, 1.0)))
        drafts = torch.argmax(q.float() + g, dim=-1).to(torch.int32)
        del g
        ua = torch.rand((B, k), device=dev, generator=gen)
        us = torch.rand((B,), device=dev, generator=gen)
        for _ in range(3):
            dad.psi_spec_verify_linear(p, q, drafts, ua, us, outputs=out, workspace=ws)
        torch.cuda.synchronize()
        dad.profile_reset()
        dad.profile_enable(True)
        for _ in range(reps):
            dad.psi_spec_verify_linear(p, q, drafts, ua, us, outputs=out, workspace=ws)
        torch.cuda.synchronize()
        ms = sum(dad.profile_query(n)[0] for n in names) / reps
        stats_ms = dad.profile_query("uno_row_stats")[0] / reps
        dad.profile_enable(False)
        dad.profile_reset()
        L = out["accept_len"].cpu().numpy().astype(np.int64)
        row = V * 2.0
        full_bytes = B * (2 * k + 1) * row
        draw_rows = np.where(L < k, 2, 1)               # residual: p_L and q_L; bonus: p_k
        needed = (L + 1) + np.minimum(L + 1, k) + draw_rows
        early_bytes = float(needed.sum()) * row
        res.append({"sigma": sigma, "us": ms * 1e3, "row_stats_us": stats_ms * 1e3,
                    "row_stats_gbs": full_bytes / (stats_ms * 1e-3) / 1e9,
                    "row_stats_hbm_frac": full_bytes / (stats_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                    "mean_accept_len": float(L.mean()),
                    "full_read_lower_bound_us": full_bytes / (HBM_PEAK_GBS * 1e9) * 1e6,
                    "early_exit_lower_bound_us": early_bytes / (HBM_PEAK_GBS * 1e9) * 1e6})
        log(f"linear verify sigma {sigma}: {ms * 1e3:.1f} us, mean L {L.mean():.2f}")
        # the early-exit variant on the same inputs: rows after each sequence's
        # first rejection are not read (uno_psi_spec_verify_linear_early_exit)
        ws_e = torch.empty(dad.psi_spec_verify_linear_early_exit_workspace(B, k, V), dtype=torch.uint8, device=dev)
        out_e = {"accept_len": torch.empty(B, dtype=torch.int32, device=dev),
                 "token": torch.empty(B, dtype=torch.int32, device=dev)}
        for _ in range(3):
            dad.psi_spec_verify_linear_early_exit(p, q, drafts, ua, us, outputs=out_e, workspace=ws_e)
        torch.cuda.synchronize()
        dad.profile_reset()
        dad.profile_enable(True)
        for _ in range(reps):
            dad.psi_spec_verify_linear_early_exit(p, q, drafts, ua, us, outputs=out_e, workspace=ws_e)
        torch.cuda.synchronize()
        ee_ms = sum(dad.profile_query(n)[0] for n in ("uno_ee_init", "uno_ee_stats", "uno_ee_accept",
                                                     "uno_draw_seg", "uno_draw_resolve")) / reps
        ee_stats_ms = dad.profile_query("uno_ee_stats")[0] / reps
        dad.profile_enable(False)
        dad.profile_reset()
        Le = out_e["accept_len"].cpu().numpy().astype(np.int64)
        # rows actually read: every round up to the one holding L (rounds of
        # 2, 2, 4, then 8 positions), then the draw rows again
        ends, i0 = [], 0
        while i0 <= k:
            i0 = min(i0 + (2 if len(ends) < 2 else 4 if len(ends) == 2 else 8), k + 1)
            ends.append(i0)
        upto = np.array([next(e for e in ends if e > x) for x in Le])
        read_bytes = float((upto + np.minimum(upto, k) + draw_rows).sum()) * row
        res[-1]["early_exit"] = {"us": ee_ms * 1e3, "stats_us": ee_stats_ms * 1e3,
                                 "gbs": read_bytes / (ee_ms * 1e-3) / 1e9,
                                 "hbm_frac": read_bytes / (ee_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                                 "bytes_read": read_bytes, "bytes_needed": early_bytes,
                                 "same_as_full": int(((Le == L) & (out_e["token"].cpu().numpy() ==
                                                                   out["token"].cpu().numpy())).sum())}
        log(f"  early exit: {ee_ms * 1e3:.1f} us ({read_bytes / 1e9:.2f} GB read, {early_bytes / 1e9:.2f} needed)")
        if sigma == 0.5:
            # the same rows under sampling transforms (uno_psi_spec_verify_linear_sampled;
            # the drafts here come from the untransformed rows, which changes no work)
            ws_s = torch.empty(dad.psi_spec_verify_linear_sampled_workspace(B, k, V), dtype=torch.uint8, device=dev)
            sampled = {}
            for name, kw in (("top_k_50", dict(top_k=50)), ("top_p_0.9", dict(top_p=0.9)),
                             ("top_k_50_top_p_0.9", dict(top_k=50, top_p=0.9)), ("greedy", dict(greedy=True))):
                for _ in range(2):
                    dad.psi_spec_verify_linear_sampled(p, q, drafts, ua, us, outputs=out, workspace=ws_s, **kw)
                torch.cuda.synchronize()
                dad.profile_reset()
                dad.profile_enable(True)
                for _ in range(reps // 2):
                    dad.psi_spec_verify_linear_sampled(p, q, drafts, ua, us, outputs=out, workspace=ws_s, **kw)
                torch.cuda.synchronize()
                sm = sum(dad.profile_query(n)[0] for n in ("uno_row_cut", "uno_accept", "uno_draw_seg",
                                                          "uno_draw_resolve")) / (reps // 2)
                cut_ms = dad.profile_query("uno_row_cut")[0] / (reps // 2)
                dad.profile_enable(False)
                dad.profile_reset()
                sampled[name] = {"us": sm * 1e3, "row_cut_us": cut_ms * 1e3,
                                 "mean_accept_len": float(out["accept_len"].float().mean())}
                log(f"  sampled verify {name}: {sm * 1e3:.1f} us")
            res[-1]["sampled"] = sampled
            del ws_s
        del p, q, drafts
        torch.cuda.empty_cache()
    return res


def bench_tree_graph(args, dad, torch, copies=64, distinct=4, replays=5):
    """The batch-1 tree path (tree attention over a 1024-row cache + tree
    verify of a 65-node tree, V = 151,936), `copies` trees per replay, each on
    its own copy of the inputs (so no replay finds a tree's rows in cache),
    captured once as a HIP graph and replayed: per-tree time without host
    launch gaps.  `distinct` seeded trees fill the copies in turn.  Bytes per
    tree: the cache's K and V, the tree's q, k, v and output, and every logit
    row of the verify read once."""
    import numpy as np
    import workloads
    dev = torch.device("cuda:0")

    def up(a):
        a = np.ascontiguousarray(a)
        t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16) if a.dtype == np.uint16 else torch.from_numpy(a)
        return t.to(dev)

    parent = workloads.tree_parent_cfg(args.seed)
    maxc = workloads.max_children(parent)
    cases = []
    for s in range(distinct):
        ta = workloads.tree_attention_case(1, parent, 1024, 32, 8, 128, seed=args.seed + 100 + s)
        tv = workloads.tree_verify_case(parent, VOCAB, dtype="bf16", seed=args.seed + 100 + s)
        cases.append((ta, tv))
    n, dmax = cases[0][1]["n"], cases[0][1]["max_depth"]
    ws_a = torch.empty(max(1, dad.tree_verify_attention_workspace(1, n, 1024, 32, 8, 128)), dtype=torch.uint8,
                       device=dev)
    ws_v = torch.empty(dad.psi_spec_verify_tree_workspace(1, n, dmax, maxc, VOCAB), dtype=torch.uint8, device=dev)
    inst = []
    for i in range(copies):
        ta, tv = cases[i % distinct]
        e = {k: up(ta[k]) for k in ("q", "k_cache", "v_cache", "k_tree", "v_tree")}
        e["parent"] = up(ta["parent"].astype(np.int32))
        e.update({"v_" + k: up(tv[k]) for k in ("parent", "tokens", "p", "q", "u_acc", "u_s")})
        e["scale"] = ta["scale"]
        e["out"] = torch.empty_like(e["q"])
        e["lse"] = torch.empty((1, n, 32), dtype=torch.float32, device=dev)
        e["res"] = {"accept_len": torch.empty(1, dtype=torch.int32, device=dev),
                    "path": torch.empty((1, dmax), dtype=torch.int32, device=dev),
                    "token": torch.empty(1, dtype=torch.int32, device=dev)}
        inst.append(e)

    def run_all():
        for e in inst:
            dad.tree_verify_attention(e["q"], e["k_cache"], e["v_cache"], e["k_tree"], e["v_tree"], e["parent"],
                                      e["scale"], out=e["out"], lse=e["lse"], workspace=ws_a)
            dad.psi_spec_verify_tree(e["v_parent"], e["v_tokens"], e["v_p"], e["v_q"], e["v_u_acc"], e["v_u_s"],
                                     max_children=maxc, outputs=e["res"], workspace=ws_v)

    run_all()
    torch.cuda.synchronize()
    # launches of one tree (every library launch is bracketed when profiling is on)
    dad.profile_reset()
    dad.profile_enable(True)
    e0 = inst[0]
    dad.tree_verify_attention(e0["q"], e0["k_cache"], e0["v_cache"], e0["k_tree"], e0["v_tree"], e0["parent"],
                              e0["scale"], out=e0["out"], lse=e0["lse"], workspace=ws_a)
    dad.psi_spec_verify_tree(e0["v_parent"], e0["v_tokens"], e0["v_p"], e0["v_q"], e0["v_u_acc"], e0["v_u_s"],
                             max_children=maxc, outputs=e0["res"], workspace=ws_v)
    torch.cuda.synchronize()
    launches = int(dad.profile_query("uno_")[1])
    dad.profile_enable(False)
    dad.profile_reset()
    eager = [(int(e["res"]["accept_len"][0]), int(e["res"]["token"][0])) for e in inst[:distinct]]
    eager_out = inst[0]["out"].clone()
    timing = "hip_graph"
    g = None
    try:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            run_all()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            run_all()
        torch.cuda.synchronize()
    except Exception as exc:   # the runtime cannot capture one of the launches
        log(f"tree path: graph capture unavailable ({exc}); timing stream launches")
        g = None
        timing = "stream"
        torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    checks_ok = True
    times = []
    for r in range(replays):
        for e in inst[:distinct]:
            e["res"]["accept_len"].fill_(-7)
        torch.cuda.synchronize()
        start.record()
        if g is not None:
            g.replay()
        else:
            run_all()
        stop.record()
        torch.cuda.synchronize()
        times.append(start.elapsed_time(stop))
        got = [(int(e["res"]["accept_len"][0]), int(e["res"]["token"][0])) for e in inst[:distinct]]
        checks_ok &= got == eager and bool(torch.equal(inst[0]["out"].view(torch.int16), eager_out.view(torch.int16)))
    per_tree_us = float(np.median(times)) * 1e3 / copies
    attn_bytes = 2.0 * 1024 * 8 * 128 * 2 + n * (32 + 2 * 8 + 32) * 128 * 2
    verify_bytes = float(n + dmax) * VOCAB * 2
    return {"timing": timing, "copies": copies, "replays": replays, "us_per_tree": per_tree_us,
            "gbs": (attn_bytes + verify_bytes) / (per_tree_us * 1e-6) / 1e9, "bytes_per_tree": attn_bytes + verify_bytes,
            "replays_match_eager": bool(checks_ok), "launches_per_tree": launches}


def bench_tree_batch(args, dad, torch, batch=16, branching=(4, 4, 3), sigma=0.5, reps=20):
    """The tree sampler at batch 16 with the trees built on the device: 69-node
    trees (4, 4, 3 children per level), V = 151,936, bf16, drawn from the
    per-depth draft rows with and without replacement, then verified by the
    matching rule.  Rows as in workloads.tree_build_case, generated on the
    device: base_d ~ N(0, 2^2); the draft row of depth d is base_d +
    N(0, sigma^2); the AR row of a node at depth d is base_{d+1} + N(0, 0.5^2).
    Times are HIP events around each call's launches, averaged over `reps`
    calls; the byte rates count every row the call reads once (build: the
    draft rows; verify: every AR row and the draft rows)."""
    import numpy as np
    import workloads
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev)
    gen.manual_seed(args.seed + 3)
    br = list(branching)
    D = len(br)
    depth = workloads.level_depths(br)
    n = int(depth.size)
    base = torch.randn((batch, D + 2, VOCAB), device=dev, generator=gen) * 2.0
    q = (base[:, 1:D + 1] + torch.randn((batch, D, VOCAB), device=dev, generator=gen) * sigma).to(torch.bfloat16)
    idx = torch.from_numpy(depth + 1).to(dev)
    p = (base[:, idx] + torch.randn((batch, n, VOCAB), device=dev, generator=gen) * 0.5).to(torch.bfloat16)
    del base
    u_draw = torch.rand((batch, n), device=dev, generator=gen)
    ua = torch.rand((batch, n), device=dev, generator=gen)
    us = torch.rand((batch,), device=dev, generator=gen)
    maxc = max(br)
    ws_b = torch.empty(dad.psi_spec_build_tree_workspace(batch, D, VOCAB), dtype=torch.uint8, device=dev)
    row = VOCAB * 2.0
    build_bytes = batch * D * row
    verify_bytes = batch * (n + D) * row
    res = {"batch": batch, "branching": br, "n_tree": n, "vocab": VOCAB, "sigma": sigma}

    def timed(fn, names):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        dad.profile_reset()
        dad.profile_enable(True)
        for _ in range(reps):
            fn()
        torch.cuda.synchronize()
        ms = sum(dad.profile_query(nm)[0] for nm in names) / reps
        dad.profile_enable(False)
        dad.profile_reset()
        return ms

    for wor in (False, True):
        key = "without_replacement" if wor else "with_replacement"
        built = dad.psi_spec_build_tree(q, br, u_draw, 1.0, wor)
        b_ms = timed(lambda: dad.psi_spec_build_tree(q, br, u_draw, 1.0, wor, outputs=built, workspace=ws_b),
                     ("uno_build_stats", "uno_build_desc", "uno_build_seg", "uno_build_draw"))
        tokens = built["tokens"].clone()
        tokens[:, 0] = 0
        ws_v = torch.empty(dad.psi_spec_verify_tree_workspace(batch, n, D, maxc, VOCAB, wor), dtype=torch.uint8,
                           device=dev)
        res_v = dad.psi_spec_verify_tree(built["parent"], tokens, p, q, ua, us, max_children=maxc, workspace=ws_v,
                                         without_replacement=wor)
        v_ms = timed(lambda: dad.psi_spec_verify_tree(built["parent"], tokens, p, q, ua, us, max_children=maxc,
                                                      outputs=res_v, workspace=ws_v, without_replacement=wor),
                     ("uno_tree_stats", "uno_tree_flow"))
        L = res_v["accept_len"].float()
        res[key] = {"build_us": b_ms * 1e3, "build_gbs": build_bytes / (b_ms * 1e-3) / 1e9,
                    "verify_us": v_ms * 1e3, "verify_gbs": verify_bytes / (v_ms * 1e-3) / 1e9,
                    "verify_hbm_frac": verify_bytes / (v_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                    "mean_accept_len": float(L.mean()),
                    "distinct_siblings": bool(wor)}
        log(f"tree batch {batch} {key}: build {b_ms * 1e3:.1f} us, verify {v_ms * 1e3:.1f} us, "
            f"mean L {float(L.mean()):.2f}")
        del ws_v
    del p, q
    torch.cuda.empty_cache()
    return res


def bench_distill(args, dad, torch, batch=128, block=16, sigma=0.5, reps=10):
    """The distillation losses over the logits of one concatenated forward at
    the step's shape: 128 sequences x (16 clean + 16 noisy) rows, V = 151,936,
    bf16; teacher rows ~ N(0, 2^2), student rows = teacher + N(0, sigma^2),
    generated on the device.  The teacher and student halves are passed in
    place; the gradient goes into the noisy half of a same-shaped buffer.
    Algorithmic bytes per pair: both rows read once and the gradient row
    written once (3 V x 2 bytes); losses only: the two reads."""
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev)
    gen.manual_seed(args.seed + 4)
    t = torch.randn((batch, block, VOCAB), device=dev, generator=gen) * 2.0
    s = t + torch.randn((batch, block, VOCAB), device=dev, generator=gen) * sigma
    logits = torch.cat([t, s], dim=1).to(torch.bfloat16)
    del t, s
    gbuf = torch.empty_like(logits)
    kl = torch.empty((batch, block), dtype=torch.float32, device=dev)
    tv = torch.empty_like(kl)
    res = {"batch": batch, "block": block, "vocab": VOCAB, "sigma": sigma}
    pairs = batch * block
    for name, want in (("with_grad", True), ("losses_only", False)):
        outs = {"kl": kl, "tv": tv}
        if want:
            outs["grad"] = gbuf[:, block:]
        for _ in range(2):
            dad.distill_loss(logits[:, :block], logits[:, block:], grad_scale=1.0 / pairs, outputs=outs)
        torch.cuda.synchronize()
        dad.profile_reset()
        dad.profile_enable(True)
        for _ in range(reps):
            dad.distill_loss(logits[:, :block], logits[:, block:], grad_scale=1.0 / pairs, outputs=outs)
        torch.cuda.synchronize()
        ms = dad.profile_query("uno_distill")[0] / reps
        dad.profile_enable(False)
        dad.profile_reset()
        nbytes = pairs * VOCAB * 2.0 * (3 if want else 2)
        res[name] = {"us": ms * 1e3, "bytes": nbytes, "gbs": nbytes / (ms * 1e-3) / 1e9,
                     "hbm_frac": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS}
        log(f"distill {name}: {ms * 1e3:.1f} us, {nbytes / (ms * 1e-3) / 1e9:.0f} GB/s")
    res["mean_kl"] = float(kl.mean())
    res["mean_tv"] = float(tv.mean())
    del logits, gbuf
    torch.cuda.empty_cache()
    return res


def bench_lora_backward(args, dad, torch, reps=10):
    """The gated-LoRA backward of the 1024-row layer workload's projections
    (64 sequences x 8 clean + 8 noisy rows, Qwen3-8B shapes, rank 128, bf16):
    q (N = K = 4096), gate/up (N = 12288, K = 4096) and down (N = 4096,
    K = 12288).  Per launch: HIP-event time and MFMA rate against the dense
    bf16 peak; FLOPs of the five products 2 M r K (U), 2 M r N (dT),
    2 N r M (dB), 2 r K M (dA) and 2 M K (N + r) (dx)."""
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev)
    gen.manual_seed(args.seed + 5)
    M, r = 1024, 128
    gate = torch.tensor(([0] * 8 + [1] * 8) * (M // 16), dtype=torch.uint8, device=dev)
    # phases of the call with W^T given: per-call transposes of A and B, the LoRA-down
    # for U and dT, the adapter gradients, the main GEMM for dx
    phases = {"transpose": ("uno_transpose",), "u_dt": ("uno_lora_down", "uno_lora_gate"),
              "da_db": ("uno_lora_bwd_dadb",), "dx": ("uno_gemm",)}
    res = {"rows": M, "rank": r}
    for proj, N, K in (("q", 4096, 4096), ("gate_up", 12288, 4096), ("down", 4096, 12288)):
        x = (torch.randn((M, K), device=dev, generator=gen)).to(torch.bfloat16)
        w = (torch.randn((N, K), device=dev, generator=gen) * 0.02).to(torch.bfloat16)
        a = (torch.randn((r, K), device=dev, generator=gen) * 0.05).to(torch.bfloat16)
        b = (torch.randn((N, r), device=dev, generator=gen) * 0.05).to(torch.bfloat16)
        dy = torch.randn((M, N), device=dev, generator=gen).to(torch.bfloat16)
        wt = dad.transpose_bf16(w)   # the frozen weight, transposed once
        ws = torch.empty(dad.gated_lora_backward_workspace(M, N, K, r, True), dtype=torch.uint8, device=dev)
        outs = dad.gated_lora_backward(x, w, a, b, gate, dy, workspace=ws, w_t=wt)
        for _ in range(2):
            dad.gated_lora_backward(x, w, a, b, gate, dy, outputs=outs, workspace=ws, w_t=wt)
        torch.cuda.synchronize()
        dad.profile_reset()
        dad.profile_enable(True)
        for _ in range(reps):
            dad.gated_lora_backward(x, w, a, b, gate, dy, outputs=outs, workspace=ws, w_t=wt)
        torch.cuda.synchronize()
        flops = {"transpose": 0.0, "u_dt": 2.0 * M * r * (K + N), "da_db": 2.0 * r * M * (N + K),
                 "dx": 2.0 * M * K * (N + r)}
        per = {}
        total_ms = 0.0
        for ph, nms in phases.items():
            ms = sum(dad.profile_query(nm)[0] for nm in nms) / reps
            total_ms += ms
            per[ph] = {"us": ms * 1e3, "tflops": flops[ph] / (ms * 1e-3) / 1e12,
                       "mfma_frac": flops[ph] / (ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS}
        dad.profile_enable(False)
        dad.profile_reset()
        tf = sum(flops.values())
        res[proj] = {"N": N, "K": K, "w_t": True, "us": total_ms * 1e3, "tflops": tf / (total_ms * 1e-3) / 1e12,
                     "mfma_frac": tf / (total_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, "launches": per}
        log(f"lora backward {proj}: {total_ms * 1e3:.1f} us, {tf / (total_ms * 1e-3) / 1e12:.0f} TFLOP/s")
        del x, w, a, b, dy, ws, outs, wt
    torch.cuda.empty_cache()
    return res


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
