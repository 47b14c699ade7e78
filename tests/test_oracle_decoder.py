"""Pins of the decoder-layer oracle (composed decode step).

Source: Uno summary (hyper.ai, arXiv 2609.04010), sections 方法 (concatenated
clean + noisy rows, gated adapters) and 实验 (Qwen3-8B base, rank-128
adapters, shared KV cache, full attention).  Each function is tied to a
library routine or to a closed-form property rather than to its own formula.
"""

import numpy as np
import pytest
import torch

import oracle

rng = np.random.default_rng(1234)


def test_round_bf16_matches_torch_conversion():
    x = np.concatenate([rng.standard_normal(5000) * 10.0 ** rng.integers(-6, 6, 5000),
                        [0.0, -0.0, 1.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -9, 65504.0, 3.0e38, -1e-40]])
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(oracle.round_bf16(x), ref)
    # ties go to even: 1 + 2^-8 is halfway between 1 and 1 + 2^-7
    assert oracle.round_bf16(np.array([1.0 + 2.0 ** -8]))[0] == 1.0


def test_rms_norm_matches_torch_and_is_scale_free():
    x = rng.standard_normal((7, 64))
    w = rng.standard_normal(64)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(x), (64,), torch.from_numpy(w), eps=1e-6).numpy()
    np.testing.assert_allclose(oracle.rms_norm(x, w, 1e-6), ref, rtol=1e-12, atol=1e-12)
    # without eps the output does not depend on the row's scale, and has unit RMS with w = 1
    one = np.ones(64)
    np.testing.assert_allclose(oracle.rms_norm(3.7 * x, one, 0.0), oracle.rms_norm(x, one, 0.0), rtol=1e-12)
    np.testing.assert_allclose(np.sqrt(np.mean(oracle.rms_norm(x, one, 0.0) ** 2, axis=1)), 1.0, rtol=1e-12)


def test_rope_is_complex_rotation():
    """Pair (x_i, x_{i+D/2}) as the complex number x_i + j x_{i+D/2}, multiplied by e^{j pos f_i}."""
    d, theta = 128, 1.0e6
    x = rng.standard_normal((5, 3, d))
    pos = np.array([0, 1, 17, 1000, 8191])
    f = theta ** (-np.arange(d // 2) * 2.0 / d)
    z = (x[..., : d // 2] + 1j * x[..., d // 2:]) * np.exp(1j * pos[:, None, None] * f[None, None, :])
    ref = np.concatenate([z.real, z.imag], axis=-1)
    np.testing.assert_allclose(oracle.rope(x, pos, theta), ref, rtol=1e-12, atol=1e-12)


def test_rope_scores_depend_on_relative_position_only():
    d = 128
    q = rng.standard_normal((1, 1, d))
    k = rng.standard_normal((1, 1, d))
    s1 = np.sum(oracle.rope(q, [40]) * oracle.rope(k, [12]))
    s2 = np.sum(oracle.rope(q, [540]) * oracle.rope(k, [512]))
    assert abs(s1 - s2) < 1e-9 * max(1.0, abs(s1))
    # position 0 is the identity, and the rotation keeps norms
    np.testing.assert_array_equal(oracle.rope(q, [0]), q)
    np.testing.assert_allclose(np.linalg.norm(oracle.rope(q, [777])), np.linalg.norm(q), rtol=1e-12)


def _sdpa(q, k, v, mask=None):
    """torch CPU float64 attention: q [H, n, D], k/v [H, L, D]."""
    out = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
        attn_mask=None if mask is None else torch.from_numpy(mask))
    return out.numpy()


def _attn_case(bsz=2, block=4, ctx=6, nh=4, nkv=2, hd=16):
    n = 2 * block
    return (rng.standard_normal((bsz, n, nh, hd)), rng.standard_normal((bsz, ctx, nkv, hd)),
            rng.standard_normal((bsz, ctx, nkv, hd)), rng.standard_normal((bsz, n, nkv, hd)),
            rng.standard_normal((bsz, n, nkv, hd)))


def test_block_attention_noisy_rows_are_full_attention_and_clean_rows_causal():
    block, ctx, nh, nkv, hd = 4, 6, 4, 2, 16
    q, kc, vc, kb, vb = _attn_case(2, block, ctx, nh, nkv, hd)
    out, lse = oracle.block_attention(q, kc, vc, kb, vb, block, 1.0 / np.sqrt(hd))
    group = nh // nkv
    for b in range(2):
        keys = np.concatenate([kc[b], kb[b]], axis=0)          # [ctx + n, Hkv, D]
        vals = np.concatenate([vc[b], vb[b]], axis=0)
        kh = np.repeat(keys.transpose(1, 0, 2), group, axis=0)
        vh = np.repeat(vals.transpose(1, 0, 2), group, axis=0)
        # noisy rows: plain attention over cache + the whole block (no mask at all)
        ref_noisy = _sdpa(q[b, block:].transpose(1, 0, 2), kh, vh)
        np.testing.assert_allclose(out[b, block:], ref_noisy.transpose(1, 0, 2), rtol=1e-10, atol=1e-12)
        # clean rows: attention over cache + clean rows only, causal among them
        kcl, vcl = kh[:, : ctx + block], vh[:, : ctx + block]
        causal = torch.ones(block, block, dtype=torch.bool).tril().numpy()
        mask = np.concatenate([np.ones((block, ctx), dtype=bool), causal], axis=1)
        ref_clean = _sdpa(q[b, :block].transpose(1, 0, 2), kcl, vcl, mask)
        np.testing.assert_allclose(out[b, :block], ref_clean.transpose(1, 0, 2), rtol=1e-10, atol=1e-12)
        # LSE of the noisy rows against torch.logsumexp of the full score rows
        s = torch.from_numpy(np.einsum("nhd,hld->hnl", q[b, block:], kh) / np.sqrt(hd))
        np.testing.assert_allclose(lse[b, block:], torch.logsumexp(s, dim=-1).numpy().T, rtol=1e-12)


def test_block_attention_invariant_to_cache_order():
    q, kc, vc, kb, vb = _attn_case()
    perm = rng.permutation(kc.shape[1])
    o1, _ = oracle.block_attention(q, kc, vc, kb, vb, 4, 0.25)
    o2, _ = oracle.block_attention(q, kc[:, perm], vc[:, perm], kb, vb, 4, 0.25)
    np.testing.assert_allclose(o1, o2, rtol=1e-12, atol=1e-12)


def test_silu_mul_matches_torch():
    g = rng.standard_normal(1000) * 5
    u = rng.standard_normal(1000)
    ref = (torch.nn.functional.silu(torch.from_numpy(g)) * torch.from_numpy(u)).numpy()
    np.testing.assert_allclose(oracle.silu_mul(g, u), ref, rtol=1e-12, atol=1e-15)


def _layer_weights(hidden, inter, nh, nkv, r, scale=0.05, seed=0, qk_norm=False):
    g = np.random.default_rng(seed)
    shapes = {"q": (nh * 128, hidden), "k": (nkv * 128, hidden), "v": (nkv * 128, hidden),
              "o": (hidden, nh * 128), "g": (inter, hidden), "u": (inter, hidden), "d": (hidden, inter)}
    w = {"attn_norm": oracle.round_bf16(1.0 + 0.1 * g.standard_normal(hidden)),
         "mlp_norm": oracle.round_bf16(1.0 + 0.1 * g.standard_normal(hidden))}
    for p, (n_out, n_in) in shapes.items():
        w["w" + p] = oracle.round_bf16(g.standard_normal((n_out, n_in)) * scale)
        w["a" + p] = oracle.round_bf16(g.standard_normal((r, n_in)) * scale)
        w["b" + p] = oracle.round_bf16(g.standard_normal((n_out, r)) * scale)
    if qk_norm:
        w["q_norm"] = oracle.round_bf16(1.0 + 0.3 * g.standard_normal(128))
        w["k_norm"] = oracle.round_bf16(1.0 + 0.3 * g.standard_normal(128))
    return w


def _layer_inputs(bsz, block, ctx, hidden, nkv, seed=1):
    g = np.random.default_rng(seed)
    rows = bsz * 2 * block
    h = oracle.round_bf16(g.standard_normal((rows, hidden)))
    gate = np.tile(np.concatenate([np.zeros(block), np.ones(block)]).astype(np.uint8), bsz)
    pos = np.tile(np.concatenate([np.arange(block), np.arange(block)]) + ctx, bsz)
    kc = oracle.round_bf16(g.standard_normal((bsz, ctx, nkv, 128)))
    vc = oracle.round_bf16(g.standard_normal((bsz, ctx, nkv, 128)))
    return h, gate, pos, kc, vc


def test_layer_with_zero_output_projections_is_identity():
    hidden, inter, nh, nkv, r, block, ctx = 256, 384, 2, 1, 8, 3, 5
    w = _layer_weights(hidden, inter, nh, nkv, r)
    for p in ("o", "d"):
        w["w" + p] = np.zeros_like(w["w" + p])
        w["b" + p] = np.zeros_like(w["b" + p])
    h, gate, pos, kc, vc = _layer_inputs(2, block, ctx, hidden, nkv)
    out, _ = oracle.decoder_layer(h, w, gate, pos, kc, vc, block, nh, nkv)
    np.testing.assert_array_equal(out, h)


def test_layer_gate_off_rows_ignore_adapter_and_sequences_are_independent():
    hidden, inter, nh, nkv, r, block, ctx = 256, 384, 2, 1, 8, 3, 5
    w = _layer_weights(hidden, inter, nh, nkv, r)
    h, gate, pos, kc, vc = _layer_inputs(2, block, ctx, hidden, nkv)
    off = np.zeros_like(gate)
    out_off, _ = oracle.decoder_layer(h, w, off, pos, kc, vc, block, nh, nkv)
    w0 = dict(w)
    for p in "qkvogud":
        w0["b" + p] = np.zeros_like(w["b" + p])
    out_b0, _ = oracle.decoder_layer(h, w0, gate, pos, kc, vc, block, nh, nkv)
    np.testing.assert_array_equal(out_off, out_b0)
    # the adapter changes the noisy rows only through the on gates
    out_on, _ = oracle.decoder_layer(h, w, gate, pos, kc, vc, block, nh, nkv)
    assert not np.allclose(out_on, out_off)
    # sequence 1 alone gives the same rows as inside the batch of two
    rows = 2 * block
    one, _ = oracle.decoder_layer(h[rows:], w, gate[rows:], pos[rows:], kc[1:], vc[1:], block, nh, nkv)
    np.testing.assert_array_equal(one, out_on[rows:])


def test_lm_head_matches_torch_pipeline():
    h = oracle.round_bf16(rng.standard_normal((6, 64)))
    nw = 1.0 + 0.1 * rng.standard_normal(64)
    wl = rng.standard_normal((50, 64)) * 0.1
    a = torch.nn.functional.rms_norm(torch.from_numpy(h), (64,), torch.from_numpy(nw), eps=1e-6)
    a = a.to(torch.float32).to(torch.bfloat16).to(torch.float64)
    ref = (a @ torch.from_numpy(wl).T).numpy()
    np.testing.assert_allclose(oracle.lm_head(h, nw, wl), ref, rtol=1e-12, atol=1e-12)


def _torch_layer(h, w, gate, pos, kc, vc, block, nh, nkv, ctx_lens=None, eps=1e-6, theta=1.0e6):
    """The layer written independently of the oracle, from torch CPU float64
    primitives: F.rms_norm, F.linear for W x and the gated B(A x), F.rms_norm
    over each 128-wide q and k head when the layer has q_norm / k_norm, RoPE
    as a complex rotation (torch.polar), F.scaled_dot_product_attention under
    an explicit boolean block mask, F.silu(gate) * up, residual adds; storage
    rounding fp32 -> bf16 at the same points as the GPU kernels."""
    F = torch.nn.functional
    T = torch.float64

    def t(a):
        return torch.as_tensor(np.asarray(a, dtype=np.float64))

    def bf(x):
        return x.to(torch.float32).to(torch.bfloat16).to(T)

    H = t(h)
    rows, hidden = H.shape
    n = 2 * block
    bsz = rows // n
    g = torch.as_tensor(np.asarray(gate, dtype=np.float64))[:, None]

    def lin(x, p):
        return bf(F.linear(x, t(w["w" + p])) + g * F.linear(F.linear(x, t(w["a" + p])), t(w["b" + p])))

    def rot(x):
        z = torch.complex(x[..., :64], x[..., 64:])
        freq = theta ** (-torch.arange(64, dtype=T) / 64.0)
        ang = torch.as_tensor(np.asarray(pos, dtype=np.float64))[:, None] * freq[None, :]
        z = z * torch.polar(torch.ones_like(ang), ang)[:, None, :]
        return torch.cat([z.real, z.imag], dim=-1)

    def head_norm(x, name):
        return F.rms_norm(x, (128,), t(w[name]), eps) if name in w else x

    a = bf(F.rms_norm(H, (hidden,), t(w["attn_norm"]), eps))
    q = bf(rot(head_norm(lin(a, "q").view(rows, nh, 128), "q_norm")))
    k = bf(rot(head_norm(lin(a, "k").view(rows, nkv, 128), "k_norm")))
    v = lin(a, "v").view(rows, nkv, 128)
    blk = torch.zeros(n, n, dtype=torch.bool)
    blk[:block, :block] = torch.ones(block, block, dtype=torch.bool).tril()   # clean: causal over clean rows
    blk[block:, :] = True                                                     # noisy: the whole block
    att = torch.empty(rows, nh, 128, dtype=T)
    cap = np.asarray(kc).shape[1]
    for b in range(bsz):
        c = cap if ctx_lens is None else int(ctx_lens[b])
        sl = slice(b * n, (b + 1) * n)
        keys = torch.cat([t(kc[b, :c]), k[sl]], dim=0).transpose(0, 1).repeat_interleave(nh // nkv, dim=0)
        vals = torch.cat([t(vc[b, :c]), v[sl]], dim=0).transpose(0, 1).repeat_interleave(nh // nkv, dim=0)
        mask = torch.cat([torch.ones(n, c, dtype=torch.bool), blk], dim=1)
        att[sl] = F.scaled_dot_product_attention(q[sl].transpose(0, 1), keys, vals, attn_mask=mask).transpose(0, 1)
    att = bf(att.reshape(rows, nh * 128))
    h1 = bf(H + lin(att, "o"))
    a2 = bf(F.rms_norm(h1, (hidden,), t(w["mlp_norm"]), eps))
    m = bf(F.silu(lin(a2, "g")) * lin(a2, "u"))
    return bf(h1 + lin(m, "d")).numpy()


@pytest.mark.parametrize("qk_norm", [False, True])
@pytest.mark.parametrize("lens", [None, [9, 0, 4]])
def test_decoder_layer_matches_torch_composition(lens, qk_norm):
    """oracle.decoder_layer against the torch composition above, with the
    whole cache valid and with per-sequence lengths (one empty), without and
    with the per-head q/k norm.  Both sides
    compute in float64 and round to bf16 at the same points; summation order
    differs, so a value sitting on a bf16 rounding boundary may land one bf16
    ulp apart, which can then move later values by a few ulps."""
    hidden, inter, nh, nkv, r, block, ctx, bsz = 256, 384, 4, 2, 16, 3, 9, 3
    w = _layer_weights(hidden, inter, nh, nkv, r, scale=0.05, seed=7, qk_norm=qk_norm)
    g = np.random.default_rng(8)
    h = oracle.round_bf16(0.1 * g.standard_normal((bsz * 2 * block, hidden)))
    gate = np.tile(np.concatenate([np.zeros(block), np.ones(block)]).astype(np.uint8), bsz)
    starts = [ctx] * bsz if lens is None else lens
    pos = np.concatenate([np.arange(2 * block) + s for s in starts])
    kc = oracle.round_bf16(g.standard_normal((bsz, ctx, nkv, 128)))
    vc = oracle.round_bf16(g.standard_normal((bsz, ctx, nkv, 128)))
    if lens is not None:
        for b, n in enumerate(lens):      # unused capacity: large values a wrong mask would pick up
            kc[b, n:] = 30.0
            vc[b, n:] = -30.0
    got, _ = oracle.decoder_layer(h, w, gate, pos, kc, vc, block, nh, nkv, ctx_lens=lens)
    ref = _torch_layer(h, w, gate, pos, kc, vc, block, nh, nkv, ctx_lens=lens)
    assert np.mean(got == ref) > 0.999
    np.testing.assert_allclose(got, ref, rtol=4 * 2.0 ** -8, atol=1e-3)
    # the layer moved the stream: the comparison is not of the identity
    assert np.max(np.abs(got - h)) > 0.1 * np.max(np.abs(h))
    if qk_norm:
        # and the per-head norm matters at this scale: without it the result moves
        w0 = {k: v for k, v in w.items() if k not in ("q_norm", "k_norm")}
        plain, _ = oracle.decoder_layer(h, w0, gate, pos, kc, vc, block, nh, nkv, ctx_lens=lens)
        assert np.max(np.abs(plain - got)) > 10 * 4 * 2.0 ** -8 * np.max(np.abs(got))
