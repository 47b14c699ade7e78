"""GPU parity: the decoder-layer entry points of the composed decode step
(uno_rms_norm, uno_rope, uno_silu_mul, uno_block_verify_attention,
uno_sample_rows, uno_decoder_layer) against the oracle.

Bar: bf16 outputs within a row-wise max relative error of 2e-2
(max_row ||y - y_ref||_inf / ||y_ref||_inf); the residual add of uno_rms_norm
bit-exact (one fp32 add of two bf16 values, one rounding to bf16, on both
sides); LSE within 1e-5 * max(1, |lse|); sampled tokens bit-exact unless the
uniform lies within 1e-5 of a CDF boundary (near-tie, counted).
"""

import numpy as np
import pytest

import oracle
import workloads
from _layer_cases import BAR as LAYER_BAR, FULL_CASES, LAYER_CASES, ids as layer_ids, make as make_layer_case, seq_rows as layer_seq_rows
from _parity import TIE, draw_is_valid, row_relerr, say, to_dev, to_host

pytestmark = pytest.mark.gpu

def _bits_dev(bits):
    return to_dev(bits)


def _f32(bits):
    return workloads.bf16_to_f32(bits).astype(np.float64)


# ---------------------------------------------------------------- rms norm
@pytest.mark.parametrize("rows,dim,with_res", [
    (5, 256, False), (3, 4096, True), (2, 16384, True), (7, 8, False), (300, 1032, True),
])
def test_rms_norm(gpu_lib, rows, dim, with_res):
    say(f"rms_norm rows={rows} dim={dim} res={with_res}")
    import torch
    rng = workloads.rng_for(rows, dim, 1)
    x = workloads.bf16_bits(rng.standard_normal((rows, dim), dtype=np.float32) * 3)
    res = workloads.bf16_bits(rng.standard_normal((rows, dim), dtype=np.float32))
    w = workloads.bf16_bits(1.0 + 0.2 * rng.standard_normal(dim, dtype=np.float32))
    xd, rd, wd = _bits_dev(x), _bits_dev(res), _bits_dev(w)
    if with_res:
        out = gpu_lib.rms_norm(xd, wd, 1e-6, res=rd)
        torch.cuda.synchronize()
        s_ref = oracle.round_bf16(_f32(x) + _f32(res))
        assert np.array_equal(to_host(xd).astype(np.float64), s_ref), "residual sum not bit-exact"
        ref = oracle.rms_norm(s_ref, _f32(w), 1e-6)
    else:
        out = gpu_lib.rms_norm(xd, wd, 1e-6)
        torch.cuda.synchronize()
        ref = oracle.rms_norm(_f32(x), _f32(w), 1e-6)
    err = row_relerr(to_host(out), ref)
    say(f"  row rel err {err:.3g}")
    assert err <= 2e-2


def test_rms_norm_residual_only(gpu_lib):
    say("rms_norm residual add only, strided sum_out")
    import torch
    rng = workloads.rng_for(9, 9)
    x = workloads.bf16_bits(rng.standard_normal((6, 64), dtype=np.float32))
    res = workloads.bf16_bits(rng.standard_normal((6, 64), dtype=np.float32))
    dst = torch.zeros((6, 72), dtype=torch.bfloat16, device="cuda")
    r = gpu_lib.rms_norm(_bits_dev(x), _bits_dev(np.ones(64, np.uint16) * 0x3F80), res=_bits_dev(res),
                         sum_out=dst[:, :64], want_out=False)
    torch.cuda.synchronize()
    assert r is None
    assert np.array_equal(to_host(dst[:, :64]).astype(np.float64), oracle.round_bf16(_f32(x) + _f32(res)))
    assert torch.all(dst[:, 64:] == 0)


# ---------------------------------------------------------------- rope
@pytest.mark.parametrize("rows,heads", [(4, 1), (37, 8), (64, 32)])
def test_rope(gpu_lib, rows, heads):
    say(f"rope rows={rows} heads={heads}")
    import torch
    rng = workloads.rng_for(rows, heads, 2)
    x = workloads.bf16_bits(rng.standard_normal((rows, heads * 128), dtype=np.float32))
    pos = rng.integers(0, 9000, rows).astype(np.int32)
    pos[0] = 0
    pos[-1] = 131071
    xd = _bits_dev(x)
    gpu_lib.rope(xd, to_dev(pos), 1.0e6)
    torch.cuda.synchronize()
    ref = oracle.rope(_f32(x).reshape(rows, heads, 128), pos, 1.0e6)
    got = to_host(xd).reshape(rows, heads, 128)
    err = row_relerr(got, ref)
    say(f"  row rel err {err:.3g}")
    assert err <= 2e-2
    # position 0 is the identity
    assert np.array_equal(got[0], _f32(x)[0].reshape(heads, 128))


def test_rope_unaligned_rows(gpu_lib):
    """Rows 130 elements apart (not a multiple of 4): the element-wise kernel
    instead of the 8-byte one; the bytes between rows stay untouched."""
    say("rope rows=9 heads=1 ldx=130")
    import torch
    rng = workloads.rng_for(9, 1, 3)
    x = workloads.bf16_bits(rng.standard_normal((9, 128), dtype=np.float32))
    pos = rng.integers(0, 131072, 9).astype(np.int32)
    buf = torch.zeros((9, 130), dtype=torch.bfloat16, device="cuda")
    buf[:, :128] = _bits_dev(x)
    buf[:, 128:] = 7.0
    gpu_lib.rope(buf[:, :128], to_dev(pos), 1.0e6)
    torch.cuda.synchronize()
    ref = oracle.rope(_f32(x).reshape(9, 1, 128), pos, 1.0e6)
    got = to_host(buf[:, :128]).reshape(9, 1, 128)
    assert row_relerr(got, ref) <= 2e-2
    assert torch.all(buf[:, 128:] == 7.0)


# ---------------------------------------------------------------- silu * mul
@pytest.mark.parametrize("rows,dim", [(3, 8), (100, 12288), (17, 1000)])
def test_silu_mul(gpu_lib, rows, dim):
    say(f"silu_mul rows={rows} dim={dim}")
    import torch
    rng = workloads.rng_for(rows, dim, 3)
    g = workloads.bf16_bits(rng.standard_normal((rows, dim), dtype=np.float32) * 4)
    u = workloads.bf16_bits(rng.standard_normal((rows, dim), dtype=np.float32))
    out = gpu_lib.silu_mul(_bits_dev(g), _bits_dev(u))
    torch.cuda.synchronize()
    err = row_relerr(to_host(out), oracle.silu_mul(_f32(g), _f32(u)))
    say(f"  row rel err {err:.3g}")
    assert err <= 2e-2


# ---------------------------------------------------------------- block attention
def _block_attn_case(batch, block, ctx, nh, nkv, seed):
    rng = workloads.rng_for(seed, batch, block, ctx)
    n = 2 * block
    shp = {"q": (batch, n, nh, 128), "k_cache": (batch, ctx, nkv, 128), "v_cache": (batch, ctx, nkv, 128),
           "k_block": (batch, n, nkv, 128), "v_block": (batch, n, nkv, 128)}
    return {name: workloads.bf16_bits(rng.standard_normal(s, dtype=np.float32)) for name, s in shp.items()}


@pytest.mark.parametrize("batch,block,ctx,nh,nkv", [
    (2, 4, 37, 8, 2),
    (1, 1, 0, 4, 4),          # no cache, one clean + one noisy row
    (3, 16, 300, 32, 8),      # ragged cache over key blocks
    (1, 128, 64, 8, 1),       # largest block, G = 8
    (2, 16, 2000, 32, 8),     # long cache, key splits
])
def test_block_attention(gpu_lib, batch, block, ctx, nh, nkv):
    say(f"block attention B={batch} block={block} ctx={ctx} H={nh}/{nkv}")
    import torch
    c = _block_attn_case(batch, block, ctx, nh, nkv, seed=5)
    dev = {k: _bits_dev(v) for k, v in c.items()}
    out, lse = gpu_lib.block_verify_attention(dev["q"], dev["k_cache"], dev["v_cache"], dev["k_block"],
                                              dev["v_block"], block, 1.0 / np.sqrt(128))
    torch.cuda.synchronize()
    ro, rl = oracle.block_attention(_f32(c["q"]), _f32(c["k_cache"]), _f32(c["v_cache"]), _f32(c["k_block"]),
                                    _f32(c["v_block"]), block, 1.0 / np.sqrt(128))
    err = row_relerr(to_host(out), ro)
    lerr = np.max(np.abs(to_host(lse) - rl) / np.maximum(1.0, np.abs(rl)))
    say(f"  row rel err {err:.3g}, lse err {lerr:.3g}")
    assert err <= 2e-2
    assert lerr <= 1e-5


def test_block_attention_full_size_sampled_sequences(gpu_lib):
    """The decode-step shape: 128 sequences x (16 clean + 16 noisy) rows, 8K
    cache, GQA 32/8; the oracle recomputes 2 sampled sequences."""
    say("block attention B=128 block=16 ctx=8192 H=32/8 (sampled)")
    import torch
    batch, block, ctx, nh, nkv = 128, 16, 8192, 32, 8
    rng = workloads.rng_for(77)
    q = workloads.bf16_bits(rng.standard_normal((batch, 2 * block, nh, 128), dtype=np.float32))
    kb = workloads.bf16_bits(rng.standard_normal((batch, 2 * block, nkv, 128), dtype=np.float32))
    vb = workloads.bf16_bits(rng.standard_normal((batch, 2 * block, nkv, 128), dtype=np.float32))
    kc, vc = workloads.kv_cache_case(batch, ctx, nkv, seed=77)
    out, lse = gpu_lib.block_verify_attention(_bits_dev(q), _bits_dev(kc), _bits_dev(vc), _bits_dev(kb),
                                              _bits_dev(vb), block, 1.0 / np.sqrt(128))
    torch.cuda.synchronize()
    o, l = to_host(out), to_host(lse)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(l))
    for b in (0, 97):
        ro, rl = oracle.block_attention(_f32(q[b:b + 1]), _f32(kc[b:b + 1]), _f32(vc[b:b + 1]),
                                        _f32(kb[b:b + 1]), _f32(vb[b:b + 1]), block, 1.0 / np.sqrt(128))
        err = row_relerr(o[b:b + 1], ro)
        lerr = np.max(np.abs(l[b:b + 1] - rl) / np.maximum(1.0, np.abs(rl)))
        say(f"  seq {b}: row rel err {err:.3g}, lse err {lerr:.3g}")
        assert err <= 2e-2
        assert lerr <= 1e-5


# ---------------------------------------------------------------- row sampler
@pytest.mark.parametrize("rows,vocab,dtype,temp", [
    (8, 1, "f32", 1.0), (33, 7, "bf16", 1.0), (16, 1001, "f32", 0.7), (64, 20000, "bf16", 1.0),
    (1920, 151936, "bf16", 1.0),      # the 15 draft rows of 128 sequences at the full vocabulary
])
def test_sample_rows(gpu_lib, rows, vocab, dtype, temp):
    say(f"sample_rows rows={rows} V={vocab} {dtype} T={temp}")
    import torch
    c = workloads.rows_case(rows, vocab, dtype, seed=rows + vocab)
    tok = gpu_lib.sample_rows(to_dev(c["logits"]), to_dev(c["u"]), temp)
    torch.cuda.synchronize()
    got = tok.cpu().numpy()
    check = range(rows) if rows <= 64 else np.random.default_rng(0).choice(rows, 48, replace=False)
    ties = 0
    for i in check:
        p = oracle.softmax_rows(c["logits_f32"][i], temp)
        ref = oracle.inverse_cdf(p, c["u"][i])
        if got[i] != ref:
            assert draw_is_valid(p, float(c["u"][i]), int(got[i]), TIE), f"row {i}: gpu {got[i]} oracle {ref}"
            ties += 1
    assert np.all((got >= 0) & (got < vocab))
    say(f"  near-ties {ties}")
    assert ties <= 1


# ---------------------------------------------------------------- decoder layer
def _layer_oracle_weights(wt):
    return {k[:-4]: v.astype(np.float64) for k, v in wt.items() if k.endswith("_f32")}


def _run_layer(dad, c, gate=True, packed=False):
    import torch
    wt = {k: _bits_dev(v) for k, v in c["weights"].items() if not k.endswith("_f32")}
    if packed:
        # adapters of q/k/v and of gate/up back to back: the grouped LoRA-down path
        for group in (("q", "k", "v"), ("g", "u")):
            cat = torch.cat([wt["a" + p] for p in group], dim=0).contiguous()
            r = wt["a" + group[0]].shape[0]
            for i, p in enumerate(group):
                wt["a" + p] = cat[i * r:(i + 1) * r]
    kc, vc = _bits_dev(c["k_cache"]), _bits_dev(c["v_cache"])
    h = _bits_dev(c["h"])
    lw = dad.layer_weights(wt, kc, vc)
    dad.decoder_layer(h, lw, to_dev(c["gate"]) if gate else None, to_dev(c["positions"]), c["batch"],
                      c["block"], c["ctx"], c["n_heads"], c["n_kv_heads"], c["inter"], c["r"])
    torch.cuda.synchronize()
    return to_host(h)


def _layer_ref(c, seqs):
    n = 2 * c["block"]
    rows = np.concatenate([np.arange(b * n, (b + 1) * n) for b in seqs])
    sl = np.asarray(seqs)
    out, _ = oracle.decoder_layer(_f32(c["h"][rows]), _layer_oracle_weights(c["weights"]), c["gate"][rows],
                                  c["positions"][rows], _f32(c["k_cache"][sl]), _f32(c["v_cache"][sl]),
                                  c["block"], c["n_heads"], c["n_kv_heads"])
    return rows, out


@pytest.mark.parametrize("lc", LAYER_CASES, ids=layer_ids(LAYER_CASES))
def test_decoder_layer(gpu_lib, lc):
    """The layer cases of tests/_layer_cases.py: small shapes with the adapters
    stored apart and back to back, no cache, the fused gate/up/SwiGLU GEMM
    (rank 64 back to back, ragged 1088-feature tail), 2048 rows (k and v as one
    two-segment GEMM) on 2 sampled sequences, and no adapters at all.  Each
    planted wiring mistake moves these outputs by >= 3x the bar
    (tests/test_layer_mutations.py)."""
    say(f"decoder layer {lc['name']}: B={lc['batch']} block={lc['block']} ctx={lc['ctx']} hidden={lc['hidden']} "
        f"inter={lc['inter']} H={lc['nh']}/{lc['nkv']} r={lc['r']} packed={lc['packed']} gate={lc['gate']}")
    c = make_layer_case(lc)
    got = _run_layer(gpu_lib, c, gate=lc["gate"], packed=lc["packed"])
    assert np.all(np.isfinite(got))
    seqs, _ = layer_seq_rows(lc)
    rows, ref = _layer_ref(c, list(seqs))
    err = row_relerr(got[rows], ref)
    say(f"  row rel err {err:.3g}")
    assert err <= LAYER_BAR


@pytest.mark.parametrize("lc", FULL_CASES[:1], ids=layer_ids(FULL_CASES[:1]))
def test_decoder_layer_full_size_sampled_sequences(gpu_lib, lc):
    """One Qwen3-8B-shaped layer at the decode-step shape: 128 sequences x
    (16 clean + 16 noisy) rows, 8K cache, rank-128 adapters stored as the
    bench stores them (q/k/v and gate/up adapters back to back); the oracle
    recomputes 2 sampled sequences (64 rows, both gate values)."""
    say(f"decoder layer {lc['name']}: B=128 block=16 ctx=8192 Qwen3-8B shapes (sampled {lc['seqs']})")
    c = make_layer_case(lc)
    got = _run_layer(gpu_lib, c, packed=True)
    assert np.all(np.isfinite(got))
    rows, ref = _layer_ref(c, lc["seqs"])
    err = row_relerr(got[rows], ref)
    say(f"  row rel err {err:.3g}")
    assert err <= LAYER_BAR


@pytest.mark.parametrize("name", ["small", "block16", "no_cache", "no_qk_norm"])
def test_decoder_layer_stages_within_single_op_bar(gpu_lib, name):
    """Each stage of the layer, run through its own entry point on the GPU's
    output of the stage before, against the oracle's stage on the same input:
    every stage within the single-operation bf16 bar (2e-2), and the whole
    layer (uno_decoder_layer, adapters stored apart so it takes the same
    kernels) bit-identical to the chain of stages.  The layer's hidden state
    is held to the composite bar (3e-2) because these per-stage differences,
    one bf16 rounding each, add up along the chain."""
    import torch
    lc = [c for c in LAYER_CASES if c["name"] == name][0]
    say(f"decoder layer stages {name}")
    c = make_layer_case(lc)
    nh, nkv, block, B = lc["nh"], lc["nkv"], lc["block"], lc["batch"]
    n = 2 * block
    w64 = _layer_oracle_weights(c["weights"])
    Wd = {k: _bits_dev(v) for k, v in c["weights"].items() if not k.endswith("_f32")}
    h = _f32(c["h"])
    gate, pos = c["gate"], c["positions"]
    rows = h.shape[0]
    gt = to_dev(gate)
    bf = oracle.round_bf16

    def dev(x):
        return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).cuda()

    def back(t):
        torch.cuda.synchronize()
        return to_host(t).astype(np.float64)

    def proj(x, p):
        got = back(gpu_lib.gated_lora_linear(dev(x), Wd["w" + p], Wd["a" + p], Wd["b" + p], gt))
        return got, bf(oracle.gated_lora_linear(x, w64["w" + p], w64["a" + p], w64["b" + p], gate))

    err = {}
    a = back(gpu_lib.rms_norm(dev(h), Wd["attn_norm"], 1e-6))
    err["attn_norm"] = row_relerr(a, bf(oracle.rms_norm(h, w64["attn_norm"])))
    qkv = {}
    for p in "qkv":
        qkv[p], ref = proj(a, p)
        err[p] = row_relerr(qkv[p], ref)
    qd, kd = dev(qkv["q"]), dev(qkv["k"])
    gpu_lib.rope(qd, to_dev(pos), 1e6, norm_weight=Wd.get("q_norm"))
    gpu_lib.rope(kd, to_dev(pos), 1e6, norm_weight=Wd.get("k_norm"))
    qr, kr = back(qd), back(kd)

    def headnorm(x, name):
        return oracle.rms_norm(x, w64[name], 1e-6) if name in w64 else x

    err["rope_q"] = row_relerr(qr, bf(oracle.rope(headnorm(qkv["q"].reshape(rows, nh, 128), "q_norm"),
                                                  pos)).reshape(rows, -1))
    err["rope_k"] = row_relerr(kr, bf(oracle.rope(headnorm(qkv["k"].reshape(rows, nkv, 128), "k_norm"),
                                                  pos)).reshape(rows, -1))
    att_d, _ = gpu_lib.block_verify_attention(dev(qr).view(B, n, nh, 128), _bits_dev(c["k_cache"]),
                                              _bits_dev(c["v_cache"]), dev(kr).view(B, n, nkv, 128),
                                              dev(qkv["v"]).view(B, n, nkv, 128), block, 1 / np.sqrt(128))
    att = back(att_d).reshape(rows, -1)
    ra, _ = oracle.block_attention(qr.reshape(B, n, nh, 128), _f32(c["k_cache"]), _f32(c["v_cache"]),
                                   kr.reshape(B, n, nkv, 128), qkv["v"].reshape(B, n, nkv, 128), block,
                                   1 / np.sqrt(128))
    err["attention"] = row_relerr(att, bf(ra.reshape(rows, -1)))
    o, ref = proj(att, "o")
    err["o"] = row_relerr(o, ref)
    h1 = bf(h + o)
    a2 = back(gpu_lib.rms_norm(dev(h1), Wd["mlp_norm"], 1e-6))
    err["mlp_norm"] = row_relerr(a2, bf(oracle.rms_norm(h1, w64["mlp_norm"])))
    g, ref = proj(a2, "g")
    err["gate"] = row_relerr(g, ref)
    u, ref = proj(a2, "u")
    err["up"] = row_relerr(u, ref)
    m = back(gpu_lib.silu_mul(dev(g), dev(u)))
    err["swiglu"] = row_relerr(m, bf(oracle.silu_mul(g, u)))
    d, ref = proj(m, "d")
    err["down"] = row_relerr(d, ref)
    chain = bf(h1 + d)
    say("  " + ", ".join(f"{k} {v:.3g}" for k, v in err.items()))
    assert max(err.values()) <= 2e-2
    whole = _run_layer(gpu_lib, c, gate=lc["gate"], packed=False)
    assert np.array_equal(whole, chain), "the fused layer differs from the chain of its stages"
    ref_layer, _ = oracle.decoder_layer(h, w64, gate, pos, _f32(c["k_cache"]), _f32(c["v_cache"]), block, nh, nkv)
    say(f"  layer row rel err {row_relerr(whole, ref_layer):.3g} (composite bar {LAYER_BAR})")
