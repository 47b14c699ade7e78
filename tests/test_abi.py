"""C-ABI checks that need no GPU: the library loads, exports every function
include/uno.h declares, and rejects invalid calls on the host (before any HIP
call) with the documented status codes."""

import ctypes
import os
import re

import pytest

import diffusion_augmented_decoding_amd as dad

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "uno.h")

OK, INVALID, UNSUPPORTED, WORKSPACE = 0, 1, 2, 3
F32, BF16 = 0, 1
P = ctypes.c_void_p
FAKE = ctypes.c_void_p(0x1000)          # never dereferenced: validation fails first
FAKE16 = ctypes.c_void_p(0x10000)


@pytest.fixture(scope="module")
def lib():
    return dad.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(uno_[a-z0-9_]+)\s*\(", text)))


def test_header_and_binding_agree():
    assert set(declared_functions()) == set(dad.EXPORTS)


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert len(names) >= 14
    for name in names:
        assert hasattr(lib, name), name


def test_version_and_strings(lib):
    assert lib.uno_abi_version() == 8
    for s in range(6):
        assert lib.uno_status_string(s)
    assert lib.uno_status_string(99) == b"unknown status"


def _ws_gl(lib, dtype, m, n, k, r):
    out = ctypes.c_size_t(0)
    st = lib.uno_gated_lora_linear_workspace(dtype, m, n, k, r, ctypes.byref(out))
    return st, out.value


def test_gated_lora_workspace_queries(lib):
    assert _ws_gl(lib, BF16, 1024, 12288, 4096, 128)[0] == OK
    assert _ws_gl(lib, BF16, 1024, 12288, 4096, 0) == (OK, 0)
    assert _ws_gl(lib, F32, 8, 256, 256, 8)[1] >= 8 * 8 * 4
    assert _ws_gl(lib, BF16, 0, 1, 8, 8)[0] == INVALID
    assert _ws_gl(lib, BF16, 4, 4, 12, 8)[0] == UNSUPPORTED      # K not multiple of 8
    assert _ws_gl(lib, BF16, 4, 4, 16, 4)[0] == UNSUPPORTED      # r not multiple of 8
    assert _ws_gl(lib, 7, 4, 4, 16, 8)[0] == INVALID             # dtype
    assert lib.uno_gated_lora_linear_workspace(BF16, 4, 4, 16, 8, None) == INVALID


def _gl(lib, **kw):
    a = dict(stream=None, dtype=BF16, M=16, N=16, K=16, r=8, x=FAKE16, ldx=16, W=FAKE16, ldw=16,
             A=FAKE16, lda=16, B=FAKE16, ldb=8, gate=FAKE16, scale=1.0, y=FAKE16, ldy=16, ws=FAKE16,
             wsb=1 << 20)
    a.update(kw)
    return lib.uno_gated_lora_linear(a["stream"], a["dtype"], a["M"], a["N"], a["K"], a["r"], a["x"], a["ldx"],
                                     a["W"], a["ldw"], a["A"], a["lda"], a["B"], a["ldb"], a["gate"], a["scale"],
                                     a["y"], a["ldy"], a["ws"], a["wsb"])


def test_gated_lora_rejects_bad_calls(lib):
    assert _gl(lib, x=None) == INVALID
    assert _gl(lib, y=None) == INVALID
    assert _gl(lib, A=None) == INVALID                           # r > 0 with a gate needs A, B
    assert _gl(lib, M=0) == INVALID
    assert _gl(lib, ldx=8) == INVALID                            # ldx < K
    assert _gl(lib, ldy=12) == INVALID
    assert _gl(lib, ldx=20) == UNSUPPORTED                       # bf16 ld not multiple of 8
    assert _gl(lib, y=ctypes.c_void_p(0x10001)) == INVALID         # y must be 2-byte aligned
    assert _gl(lib, x=FAKE16.value + 2) == UNSUPPORTED            # misaligned
    assert _gl(lib, wsb=0) == WORKSPACE
    assert _gl(lib, ws=None) == WORKSPACE
    assert _gl(lib, scale=float("nan")) == INVALID
    assert b"workspace" in lib.uno_last_error() or b"lora_scale" in lib.uno_last_error()


def _vl(lib, early_exit=False, **kw):
    a = dict(dtype=BF16, batch=2, k=3, vocab=64, p=FAKE16, ps=256, pr=64, q=FAKE16, qs=192, qr=64,
             d=FAKE16, ua=FAKE16, us=FAKE16, T=1.0, L=FAKE16, y=FAKE16, ws=FAKE16, wsb=1 << 20)
    a.update(kw)
    f = lib.uno_psi_spec_verify_linear_early_exit if early_exit else lib.uno_psi_spec_verify_linear
    return f(None, a["dtype"], a["batch"], a["k"], a["vocab"], a["p"], a["ps"], a["pr"], a["q"], a["qs"], a["qr"],
             a["d"], a["ua"], a["us"], a["T"], a["L"], a["y"], None, None, None, a["ws"], a["wsb"])


@pytest.mark.parametrize("early_exit", [False, True])
def test_verify_linear_rejects_bad_calls(lib, early_exit):
    def call(lib, **kw):   # the same checks for both entry points
        return _vl(lib, early_exit=early_exit, **kw)

    assert call(lib, k=65) == INVALID
    assert call(lib, k=-1) == INVALID
    assert call(lib, batch=0) == INVALID
    assert call(lib, vocab=0) == INVALID
    assert call(lib, vocab=(1 << 20) + 1, pr=(1 << 20) + 1, ps=4 * ((1 << 20) + 1),
               qr=(1 << 20) + 1, qs=3 * ((1 << 20) + 1)) == UNSUPPORTED
    assert call(lib, p=None) == INVALID
    assert call(lib, q=None) == INVALID
    assert call(lib, T=0.0) == INVALID
    assert call(lib, T=float("inf")) == INVALID
    assert call(lib, pr=63) == INVALID
    assert call(lib, ps=100) == INVALID
    assert call(lib, qs=100) == INVALID
    assert call(lib, wsb=8) == WORKSPACE
    assert call(lib, dtype=5) == INVALID
    ws = ctypes.c_size_t(0)
    wsq = lib.uno_psi_spec_verify_linear_early_exit_workspace if early_exit else lib.uno_psi_spec_verify_linear_workspace
    assert wsq(256, 15, 151936, ctypes.byref(ws)) == OK
    assert ws.value >= 256 * 31 * 16
    assert wsq(256, 65, 151936, ctypes.byref(ws)) == INVALID
    assert wsq(1 << 24, 64, 1 << 20, ctypes.byref(ws)) == UNSUPPORTED   # rows beyond 2^31


def _ta(lib, **kw):
    a = dict(batch=1, n=65, ctx=1024, H=32, Hkv=8, D=128, q=FAKE16, kc=FAKE16, vc=FAKE16, kt=FAKE16, vt=FAKE16,
             par=FAKE16, scale=0.088, out=FAKE16, lse=None, ws=None, wsb=0)
    a.update(kw)
    return lib.uno_tree_verify_attention(None, a["batch"], a["n"], a["ctx"], a["H"], a["Hkv"], a["D"], a["q"],
                                         a["kc"], a["vc"], a["kt"], a["vt"], a["par"], a["scale"], a["out"],
                                         a["lse"], a["ws"], a["wsb"])


def test_tree_attention_rejects_bad_calls(lib):
    assert _ta(lib, D=64) == UNSUPPORTED
    assert _ta(lib, H=30) == INVALID
    assert _ta(lib, H=80, Hkv=8) == UNSUPPORTED     # 10 heads per KV head
    assert _ta(lib, n=257) == UNSUPPORTED
    assert _ta(lib, n=0) == INVALID
    assert _ta(lib, q=None) == INVALID
    assert _ta(lib, kc=None) == INVALID
    assert _ta(lib, par=None) == INVALID
    assert _ta(lib, out=ctypes.c_void_p(0x10008)) == UNSUPPORTED
    assert _ta(lib, scale=-1.0) == INVALID
    assert _ta(lib) == WORKSPACE                     # decode size: key splits need partials


def test_tree_attention_workspace_queries(lib):
    ws = ctypes.c_size_t(1)
    # 65 nodes x 4 heads per KV head = 9 query tiles x 8 KV heads: split keys, fp32 partials
    assert lib.uno_tree_verify_attention_workspace(1, 65, 1024, 32, 8, 128, ctypes.byref(ws)) == OK
    assert ws.value >= 72 * 2 * 32 * 128 * 4
    # 64 tiles x 4 KV heads x batch 3 fill the device without splitting
    assert lib.uno_tree_verify_attention_workspace(3, 256, 40, 32, 4, 128, ctypes.byref(ws)) == OK
    assert ws.value == 0
    assert lib.uno_tree_verify_attention_workspace(1, 65, 1024, 32, 8, 128, None) == INVALID


def _tv(lib, **kw):
    a = dict(dtype=BF16, batch=1, n=65, D=3, C=4, V=1000, par=FAKE16, tok=FAKE16, p=FAKE16, q=FAKE16, ua=FAKE16,
             us=FAKE16, T=1.0, L=FAKE16, path=FAKE16, y=FAKE16, ws=FAKE16, wsb=1 << 20)
    a.update(kw)
    return lib.uno_psi_spec_verify_tree(None, a["dtype"], a["batch"], a["n"], a["D"], a["C"], a["V"], a["par"],
                                        a["tok"], a["p"], a["q"], a["ua"], a["us"], a["T"], a["L"], a["path"],
                                        a["y"], a["ws"], a["wsb"])


def test_tree_verify_rejects_bad_calls(lib):
    assert _tv(lib, n=1025) == UNSUPPORTED
    assert _tv(lib, D=65) == UNSUPPORTED
    assert _tv(lib, D=0) == INVALID
    assert _tv(lib, C=-1) == INVALID
    assert _tv(lib, C=1024) == INVALID
    assert _tv(lib, batch=65536) == UNSUPPORTED
    ws = ctypes.c_size_t(0)
    assert lib.uno_psi_spec_verify_tree_workspace(1, 65, 3, 4, 151936, ctypes.byref(ws)) == OK
    assert ws.value > 0
    assert _tv(lib, par=None) == INVALID
    assert _tv(lib, path=None) == INVALID
    assert _tv(lib, T=-1.0) == INVALID
    assert _tv(lib, wsb=16) == WORKSPACE
    assert _tv(lib, dtype=3) == INVALID


def test_profile_query_without_records(lib):
    ms = ctypes.c_double(1.0)
    cnt = ctypes.c_int64(5)
    assert lib.uno_profile_query(b"uno_", ctypes.byref(ms), ctypes.byref(cnt)) == OK
    assert cnt.value == 0 and ms.value == 0.0
    assert lib.uno_profile_query(None, ctypes.byref(ms), ctypes.byref(cnt)) == INVALID


def test_binding_fails_loudly_without_library(tmp_path):
    import importlib
    mod = importlib.reload(dad)
    mod._lib = None
    with pytest.raises(RuntimeError):
        mod.load(str(tmp_path / "missing.so"))
    importlib.reload(dad)


def test_layer_ops_reject_bad_calls(lib):
    # uno_rms_norm(stream, rows, dim, x, ldx, res, ldr, sum_out, ld_sum, weight, eps, out, ldo)
    assert lib.uno_rms_norm(None, 0, 64, FAKE16, 64, None, 64, None, 64, FAKE16, 1e-6, FAKE16, 64) == INVALID
    assert lib.uno_rms_norm(None, 4, 12, FAKE16, 12, None, 12, None, 12, FAKE16, 1e-6, FAKE16, 12) == UNSUPPORTED
    assert lib.uno_rms_norm(None, 4, 16392, FAKE16, 16392, None, 0, None, 0, FAKE16, 1e-6, FAKE16,
                            16392) == UNSUPPORTED
    assert lib.uno_rms_norm(None, 4, 64, FAKE16, 64, None, 64, None, 64, FAKE16, 1e-6, None, 64) == INVALID
    assert lib.uno_rms_norm(None, 4, 64, FAKE16, 64, FAKE16, 64, None, 64, FAKE16, 1e-6, FAKE16, 64) == INVALID
    assert lib.uno_rms_norm(None, 4, 64, FAKE16, 60, None, 64, None, 64, FAKE16, 1e-6, FAKE16, 64) == UNSUPPORTED
    assert lib.uno_rms_norm(None, 4, 64, ctypes.c_void_p(0x10002), 64, None, 64, None, 64, FAKE16, 1e-6,
                            FAKE16, 64) == UNSUPPORTED
    assert lib.uno_rms_norm(None, 4, 64, FAKE16, 64, None, 64, None, 64, FAKE16, -1.0, FAKE16, 64) == INVALID
    # uno_rope(stream, rows, n_heads, x, ldx, positions, theta, norm_weight, norm_eps)
    assert lib.uno_rope(None, 0, 8, FAKE16, 1024, FAKE16, 1e6, None, 1e-6) == INVALID
    assert lib.uno_rope(None, 4, 8, FAKE16, 1000, FAKE16, 1e6, None, 1e-6) == INVALID
    assert lib.uno_rope(None, 4, 8, FAKE16, 1024, None, 1e6, None, 1e-6) == INVALID
    assert lib.uno_rope(None, 4, 8, FAKE16, 1024, FAKE16, 1.0, None, 1e-6) == INVALID
    assert lib.uno_rope(None, 4, 8, FAKE16, 1024, FAKE16, 1e6, FAKE16, -1.0) == INVALID       # norm eps
    assert lib.uno_rope(None, 4, 8, FAKE16, 1024, FAKE16, 1e6, ctypes.c_void_p(0x10001), 1e-6) == UNSUPPORTED
    # uno_silu_mul(stream, rows, dim, g, ldg, u, ldu, out, ldo)
    assert lib.uno_silu_mul(None, 4, 12, FAKE16, 12, FAKE16, 12, FAKE16, 12) == INVALID
    assert lib.uno_silu_mul(None, 4, 16, FAKE16, 16, None, 16, FAKE16, 16) == INVALID
    assert lib.uno_silu_mul(None, 4, 16, FAKE16, 20, FAKE16, 16, FAKE16, 16) == UNSUPPORTED


def test_block_attention_rejects_bad_calls(lib):
    ws = ctypes.c_size_t(0)
    assert lib.uno_block_verify_attention_workspace(128, 16, 8192, 32, 8, 128, ctypes.byref(ws)) == OK
    assert ws.value == 0                          # 16 tiles x 8 KV heads x 128 sequences: no key splits
    assert lib.uno_block_verify_attention_workspace(1, 16, 8192, 32, 8, 128, ctypes.byref(ws)) == OK
    assert ws.value > 0
    assert lib.uno_block_verify_attention_workspace(1, 129, 64, 32, 8, 128, ctypes.byref(ws)) == UNSUPPORTED
    assert lib.uno_block_verify_attention_workspace(1, 16, 64, 32, 8, 64, ctypes.byref(ws)) == UNSUPPORTED
    assert lib.uno_block_verify_attention_workspace(1, 16, 64, 30, 8, 128, ctypes.byref(ws)) == INVALID

    def call(**kw):
        a = dict(batch=2, block=4, ctx=2000, H=8, Hkv=2, D=128, q=FAKE16, kc=FAKE16, vc=FAKE16, cl=None,
                 kb=FAKE16, vb=FAKE16, scale=0.088, out=FAKE16, lse=None, ws=FAKE16, wsb=1 << 24)
        a.update(kw)
        return lib.uno_block_verify_attention(None, a["batch"], a["block"], a["ctx"], a["H"], a["Hkv"], a["D"],
                                              a["q"], a["kc"], a["vc"], a["cl"], a["kb"], a["vb"], a["scale"],
                                              a["out"], a["lse"], a["ws"], a["wsb"])
    assert call(block=0) == INVALID
    assert call(q=None) == INVALID
    assert call(kc=None) == INVALID
    assert call(kb=ctypes.c_void_p(0x10008)) == UNSUPPORTED
    assert call(scale=0.0) == INVALID
    assert call(ws=None, wsb=0) == WORKSPACE


def test_sample_rows_rejects_bad_calls(lib):
    ws = ctypes.c_size_t(0)
    assert lib.uno_sample_rows_workspace(1920, 151936, ctypes.byref(ws)) == OK
    assert ws.value > 0
    assert lib.uno_sample_rows_workspace(0, 10, ctypes.byref(ws)) == INVALID

    def call(**kw):
        a = dict(dtype=BF16, rows=4, V=100, l=FAKE16, rs=100, u=FAKE16, T=1.0, y=FAKE16, ws=FAKE16, wsb=1 << 20)
        a.update(kw)
        return lib.uno_sample_rows(None, a["dtype"], a["rows"], a["V"], a["l"], a["rs"], a["u"], a["T"], a["y"],
                                   a["ws"], a["wsb"])
    assert call(dtype=4) == INVALID
    assert call(rows=0) == INVALID
    assert call(rows=65536) == UNSUPPORTED
    assert call(rs=99) == INVALID
    assert call(u=None) == INVALID
    assert call(T=0.0) == INVALID
    assert call(wsb=4) == WORKSPACE


def test_tree_verify_wor_rejects_bad_calls(lib):
    ws = ctypes.c_size_t(0)
    assert lib.uno_psi_spec_verify_tree_wor_workspace(1, 65, 3, 4, 1000, ctypes.byref(ws)) == OK
    wor = ws.value
    assert lib.uno_psi_spec_verify_tree_workspace(1, 65, 3, 4, 1000, ctypes.byref(ws)) == OK
    assert wor > ws.value                                  # the children lists and C_k
    assert lib.uno_psi_spec_verify_tree_wor_workspace(1, 65, 3, 65, 1000, ctypes.byref(ws)) == UNSUPPORTED

    def call(**kw):
        a = dict(dtype=BF16, batch=1, n=65, D=3, C=4, V=1000, par=FAKE16, tok=FAKE16, p=FAKE16, q=FAKE16, ua=FAKE16,
                 us=FAKE16, T=1.0, L=FAKE16, path=FAKE16, y=FAKE16, ws=FAKE16, wsb=1 << 20)
        a.update(kw)
        return lib.uno_psi_spec_verify_tree_wor(None, a["dtype"], a["batch"], a["n"], a["D"], a["C"], a["V"],
                                                a["par"], a["tok"], a["p"], a["q"], a["ua"], a["us"], a["T"],
                                                a["L"], a["path"], a["y"], a["ws"], a["wsb"])
    assert call(C=65) == UNSUPPORTED
    assert call(n=1025) == UNSUPPORTED
    assert call(tok=None) == INVALID
    assert call(T=-1.0) == INVALID
    assert call(wsb=wor - 1) == WORKSPACE


def test_gated_lora_backward_rejects_bad_calls(lib):
    ws = ctypes.c_size_t(0)
    assert lib.uno_gated_lora_backward_workspace(1024, 4096, 4096, 128, 0, ctypes.byref(ws)) == OK
    assert ws.value >= 2 * 1024 * 128 * 2
    plain = ws.value
    assert lib.uno_gated_lora_backward_workspace(1024, 4096, 4096, 128, 1, ctypes.byref(ws)) == OK
    assert ws.value > plain                               # the transposes of A and B
    assert lib.uno_gated_lora_backward_workspace(1024, 4008, 4096, 128, 0, ctypes.byref(ws)) == UNSUPPORTED

    def call(**kw):
        a = dict(M=64, N=256, K=128, r=16, x=FAKE16, ldx=128, w=FAKE16, ldw=128, a=FAKE16, lda=128, b=FAKE16, ldb=16,
                 g=FAKE16, s=1.0, dy=FAKE16, lddy=256, dx=FAKE16, lddx=128, da=FAKE16, ldda=128, db=FAKE16, lddb=16,
                 wt=None, ldwt=0, ws=FAKE16, wsb=16)
        a.update(kw)
        return lib.uno_gated_lora_backward(None, a["M"], a["N"], a["K"], a["r"], a["x"], a["ldx"], a["w"], a["ldw"],
                                           a["a"], a["lda"], a["b"], a["ldb"], a["g"], a["s"], a["dy"], a["lddy"],
                                           a["dx"], a["lddx"], a["da"], a["ldda"], a["db"], a["lddb"], a["wt"],
                                           a["ldwt"], a["ws"], a["wsb"])
    assert call(M=0) == INVALID
    assert call(N=250, lddy=256) == UNSUPPORTED
    assert call(K=100, ldx=104, lda=104, ldw=104, lddx=104, ldda=104) == UNSUPPORTED
    assert call(x=None) == INVALID
    assert call(w=None) == INVALID                     # W is read for dx
    assert call(ldb=8) == INVALID
    assert call(lddy=260) == UNSUPPORTED
    assert call(dy=ctypes.c_void_p(0x10008)) == UNSUPPORTED
    assert call(s=float("nan")) == INVALID
    assert call(wsb=8) == WORKSPACE
    assert call(wt=FAKE16, ldwt=128) == INVALID           # ldwt below N
    assert call(wt=FAKE16, ldwt=260) == INVALID           # not a multiple of 8
    assert lib.uno_transpose_bf16(None, 0, 8, FAKE16, 8, FAKE16, 8) == INVALID
    assert lib.uno_transpose_bf16(None, 8, 8, FAKE16, 7, FAKE16, 8) == INVALID
    assert lib.uno_transpose_bf16(None, 8, 8, ctypes.c_void_p(0x10001), 8, FAKE16, 8) == INVALID


def test_distill_loss_rejects_bad_calls(lib):
    def call(**kw):
        a = dict(dtype=BF16, batch=2, rows=3, V=100, t=FAKE16, ts=300, tr=100, s=FAKE16, ss=300, sr=100, T=1.0,
                 alpha=1.0, beta=1.0, gs=1.0, kl=FAKE16, tv=FAKE16, g=FAKE16, gsq=300, gr=100)
        a.update(kw)
        return lib.uno_distill_loss(None, a["dtype"], a["batch"], a["rows"], a["V"], a["t"], a["ts"], a["tr"],
                                    a["s"], a["ss"], a["sr"], a["T"], a["alpha"], a["beta"], a["gs"], a["kl"],
                                    a["tv"], a["g"], a["gsq"], a["gr"])
    assert call(dtype=9) == INVALID
    assert call(batch=0) == INVALID
    assert call(rows=0) == INVALID
    assert call(V=(1 << 20) + 1, tr=1 << 21, sr=1 << 21, gr=1 << 21) == UNSUPPORTED
    assert call(t=None) == INVALID
    assert call(tv=None) == INVALID
    assert call(sr=99) == INVALID
    assert call(gr=99) == INVALID
    assert call(ts=-1) == INVALID
    assert call(T=0.0) == INVALID
    assert call(alpha=float("inf")) == INVALID
    assert call(gs=float("nan")) == INVALID
    assert call(batch=1 << 16, rows=1 << 15) == UNSUPPORTED


def test_build_tree_rejects_bad_calls(lib):
    ws = ctypes.c_size_t(0)
    assert lib.uno_psi_spec_build_tree_workspace(256, 15, 151936, ctypes.byref(ws)) == OK
    assert ws.value > 0
    assert lib.uno_psi_spec_build_tree_workspace(0, 3, 100, ctypes.byref(ws)) == INVALID
    assert lib.uno_psi_spec_build_tree_workspace(1, 65, 100, ctypes.byref(ws)) == INVALID

    def call(br=(4, 2, 2), **kw):
        a = dict(dtype=BF16, batch=2, D=len(br), V=100, q=FAKE16, qs=300, qr=100, u=FAKE16, n=29, T=1.0, wor=0,
                 par=FAKE16, tok=FAKE16, ws=FAKE16, wsb=1 << 20)
        a.update(kw)
        arr = (ctypes.c_int32 * max(len(br), 1))(*br)
        return lib.uno_psi_spec_build_tree(None, a["dtype"], a["batch"], a["D"], arr if br is not None else None,
                                           a["V"], a["q"], a["qs"], a["qr"], a["u"], a["n"], a["T"], a["wor"],
                                           a["par"], a["tok"], a["ws"], a["wsb"])
    assert call(dtype=7) == INVALID
    assert call(batch=0) == INVALID
    assert call(batch=65536) == INVALID
    assert call(n=28) == INVALID                         # 1 + 4 + 8 + 16 = 29
    assert call(br=(4, 0, 2)) == INVALID
    assert call(br=(65,), n=66) == INVALID               # at most 64 children per node
    assert call(br=(8, 8, 8, 8), n=1 + 8 + 64 + 512 + 4096) == UNSUPPORTED
    assert call(br=(5,), n=6, V=4, qr=4, wor=1) == INVALID   # distinct siblings need vocab >= branching
    assert call(wor=2) == INVALID
    assert call(qr=99) == INVALID
    assert call(qs=-1) == INVALID
    assert call(u=None) == INVALID
    assert call(T=float("nan")) == INVALID
    assert call(wsb=16) == WORKSPACE


def test_decoder_layer_rejects_bad_calls(lib):
    ws = ctypes.c_size_t(0)
    assert lib.uno_decoder_layer_workspace(128, 16, 8192, 4096, 12288, 32, 8, 128, ctypes.byref(ws)) == OK
    assert ws.value >= 4096 * 12288 * 2 * 2          # gate and up activations
    assert lib.uno_decoder_layer_workspace(128, 16, 8192, 4100, 12288, 32, 8, 128,
                                           ctypes.byref(ws)) == UNSUPPORTED
    assert lib.uno_decoder_layer_workspace(128, 16, 8192, 4096, 12288, 32, 8, 12, ctypes.byref(ws)) == UNSUPPORTED
    lw = lib.uno_decoder_layer.argtypes[9]._type_()      # the struct type the loaded library was declared with
    assert lib.uno_decoder_layer(None, 2, 4, 8, 256, 512, 4, 2, 8, ctypes.byref(lw), FAKE16, FAKE16, None, 1e-6, 1e6,
                                 1.0, FAKE16, FAKE16, 1 << 30) == INVALID      # null weights
    lw.attn_norm = lw.mlp_norm = FAKE16.value
    for i in range(dad.NUM_PROJ):
        lw.w[i] = lw.a[i] = lw.b[i] = FAKE16.value
    lw.k_cache = lw.v_cache = FAKE16.value
    assert lib.uno_decoder_layer(None, 2, 4, 8, 256, 512, 4, 2, 8, ctypes.byref(lw), FAKE16, FAKE16, None, 1e-6, 1e6,
                                 1.0, FAKE16, FAKE16, 16) == WORKSPACE
    assert lib.uno_decoder_layer(None, 2, 4, 8, 256, 512, 4, 2, 8, ctypes.byref(lw), FAKE16, FAKE16, None, 1e-6, 0.5,
                                 1.0, FAKE16, FAKE16, 1 << 30) == INVALID      # rope theta
    lw.q_norm = FAKE16.value                                                   # q_norm without k_norm
    assert lib.uno_decoder_layer(None, 2, 4, 8, 256, 512, 4, 2, 8, ctypes.byref(lw), FAKE16, FAKE16, None, 1e-6, 1e6,
                                 1.0, FAKE16, FAKE16, 1 << 30) == INVALID
    lw.k_norm = 0x10008                                                        # unaligned
    assert lib.uno_decoder_layer(None, 2, 4, 8, 256, 512, 4, 2, 8, ctypes.byref(lw), FAKE16, FAKE16, None, 1e-6, 1e6,
                                 1.0, FAKE16, FAKE16, 1 << 30) == UNSUPPORTED
    lw.q_norm = lw.k_norm = None
    lw.w[3] = None
    assert lib.uno_decoder_layer(None, 2, 4, 8, 256, 512, 4, 2, 8, ctypes.byref(lw), FAKE16, FAKE16, None, 1e-6, 1e6,
                                 1.0, FAKE16, FAKE16, 1 << 30) == INVALID


def test_step_rejects_bad_calls(lib):
    cfg_t = lib.uno_psi_spec_step.argtypes[1]._type_
    lw_t = lib.uno_psi_spec_step.argtypes[2]._type_

    def cfg(**kw):
        a = dict(batch=128, block=16, ctx_len=8192, hidden=4096, inter=12288, n_heads=32, n_kv_heads=8, r=128,
                 n_layers=36, vocab=151936, rms_eps=1e-6, rope_theta=1e6, lora_scale=1.0, temperature=1.0)
        a.update(kw)
        return cfg_t(*a.values())
    ws = ctypes.c_size_t(0)
    assert lib.uno_psi_spec_step_workspace(ctypes.byref(cfg()), ctypes.byref(ws)) == OK
    assert ws.value >= 2 * 4096 * 4096 * 2
    for bad, code in ((dict(block=66), UNSUPPORTED), (dict(batch=0), INVALID), (dict(n_heads=30), INVALID),
                      (dict(vocab=(1 << 20) + 1), UNSUPPORTED), (dict(r=4), UNSUPPORTED),
                      (dict(temperature=0.0), INVALID), (dict(hidden=4100), UNSUPPORTED),
                      (dict(batch=8192, block=9), UNSUPPORTED)):
        assert lib.uno_psi_spec_step_workspace(ctypes.byref(cfg(**bad)), ctypes.byref(ws)) == code, bad
    assert lib.uno_psi_spec_step_workspace(None, ctypes.byref(ws)) == INVALID
    layers = (lw_t * 2)()

    def call(c, lay=layers, ws_bytes=1 << 40, **kw):
        a = dict(embed=FAKE16, fnorm=FAKE16, lm=FAKE16, tok=FAKE16, pq=FAKE16, pq_seq=3 * 1000, pq_row=1000,
                 ud=FAKE16, ua=FAKE16, us=FAKE16, logits=FAKE16, drafts=FAKE16, L=FAKE16, y=FAKE16, nxt=None)
        a.update(kw)
        return lib.uno_psi_spec_step(None, ctypes.byref(c), lay, a["embed"], a["fnorm"], a["lm"], a["tok"],
                                     a.get("cl"), a["pq"], a["pq_seq"], a["pq_row"], a["ud"], a["ua"], a["us"],
                                     a["logits"], a["drafts"], a["L"], a["y"], a["nxt"], FAKE16, ws_bytes)
    small = cfg(batch=2, block=4, ctx_len=8, hidden=256, inter=512, n_heads=4, n_kv_heads=2, r=8, n_layers=2,
                vocab=1000)
    assert call(small) == INVALID                          # layer weights are NULL
    for l in range(2):
        layers[l].attn_norm = layers[l].mlp_norm = layers[l].k_cache = layers[l].v_cache = FAKE16.value
        for i in range(7):
            layers[l].w[i] = layers[l].a[i] = layers[l].b[i] = FAKE16.value
    assert call(small, embed=None) == INVALID
    layers[1].k_norm = FAKE16.value                        # k_norm without q_norm
    assert call(small) == INVALID
    layers[1].k_norm = None
    assert call(small, ud=None) == INVALID
    assert call(small, ua=None) == INVALID                 # a carried q needs the accept uniforms
    assert call(small, pq_row=999) == INVALID              # row stride below the vocabulary
    assert call(small, pq_seq=2 * 1000) == INVALID         # sequence stride below k rows
    assert call(small, pq=ctypes.c_void_p(0x10001)) == UNSUPPORTED
    assert call(small, pq=None, ua=None, ws_bytes=64) == WORKSPACE   # the first step needs no accept uniforms
    assert call(small, lm=ctypes.c_void_p(0x10008)) == UNSUPPORTED
    assert call(small, ws_bytes=64) == WORKSPACE
    layers[1].b[6] = None
    assert call(small) == INVALID


def test_kv_commit_rejects_bad_calls(lib):
    assert lib.uno_kv_commit(None, 0, 16, FAKE16, FAKE16) == INVALID
    assert lib.uno_kv_commit(None, 4, -1, FAKE16, FAKE16) == INVALID
    assert lib.uno_kv_commit(None, 4, 16, None, FAKE16) == INVALID
    assert lib.uno_kv_commit(None, 4, 16, FAKE16, None) == INVALID


def test_verify_linear_noalloc_rejects_bad_calls(lib):
    """Host validation of the allocation-free verify: the linear verify's
    argument checks, and a call whose scratch would exceed the library's
    16 MiB per-GPU array is refused before anything is enqueued."""
    def call(**kw):
        a = dict(dtype=BF16, batch=4, k=3, vocab=1000, p=FAKE16, ps=4000, pr=1000, q=FAKE16, qs=3000, qr=1000,
                 d=FAKE16, ua=FAKE16, us=FAKE16, t=1.0, L=FAKE16, y=FAKE16)
        a.update(kw)
        return lib.uno_psi_spec_verify_linear_noalloc(None, a["dtype"], a["batch"], a["k"], a["vocab"], a["p"],
                                                      a["ps"], a["pr"], a["q"], a["qs"], a["qr"], a["d"], a["ua"],
                                                      a["us"], a["t"], a["L"], a["y"], None, None, None)
    assert call(p=None) == INVALID
    assert call(k=65) == INVALID
    assert call(t=0.0) == INVALID
    assert call(pr=999) == INVALID
    big = dict(batch=8192, k=64, vocab=151936, ps=65 * 151936, pr=151936, qs=64 * 151936, qr=151936)
    assert call(**big) == UNSUPPORTED
    assert b"16777216" in lib.uno_last_error()


def _merge(lib, **kw):
    a = dict(stream=None, N=16, K=16, r=8, W=FAKE16, ldw=16, A=FAKE16, lda=16, B=FAKE16, ldb=8, scale=1.0,
             out=FAKE16, ldo=16)
    a.update(kw)
    return lib.uno_lora_merge(a["stream"], a["N"], a["K"], a["r"], a["W"], a["ldw"], a["A"], a["lda"], a["B"],
                              a["ldb"], a["scale"], a["out"], a["ldo"])


def test_lora_merge_rejects_bad_calls(lib):
    assert _merge(lib, N=0) == INVALID
    assert _merge(lib, r=0) == INVALID
    assert _merge(lib, W=None) == INVALID
    assert _merge(lib, out=None) == INVALID
    assert _merge(lib, ldw=8) == INVALID                 # leading dimension below K
    assert _merge(lib, ldb=4) == INVALID                 # below r
    assert _merge(lib, scale=float("inf")) == INVALID
    assert _merge(lib, N=70000) == UNSUPPORTED
    assert _merge(lib, out=ctypes.c_void_p(0x10001)) == INVALID   # not 2-byte aligned


def _vls(lib, **kw):
    a = dict(stream=None, dtype=BF16, batch=2, k=3, vocab=100, p=FAKE16, ps=400, pr=100, q=FAKE16, qs=300, qr=100,
             d=FAKE16, ua=FAKE16, us=FAKE16, t=1.0, top_k=5, top_p=0.9, greedy=0, L=FAKE16, y=FAKE16, pd=None,
             qd=None, mass=None, ws=FAKE16, wsb=1 << 30)
    a.update(kw)
    return lib.uno_psi_spec_verify_linear_sampled(a["stream"], a["dtype"], a["batch"], a["k"], a["vocab"], a["p"],
                                                  a["ps"], a["pr"], a["q"], a["qs"], a["qr"], a["d"], a["ua"],
                                                  a["us"], a["t"], a["top_k"], a["top_p"], a["greedy"], a["L"],
                                                  a["y"], a["pd"], a["qd"], a["mass"], a["ws"], a["wsb"])


def test_verify_linear_sampled_rejects_bad_calls(lib):
    assert _vls(lib, top_k=-1) == INVALID
    assert _vls(lib, top_p=0.0) == INVALID
    assert _vls(lib, top_p=1.5) == INVALID
    assert _vls(lib, top_p=float("nan")) == INVALID
    assert _vls(lib, greedy=2) == INVALID
    assert _vls(lib, t=0.0) == INVALID
    assert _vls(lib, p=None) == INVALID
    assert _vls(lib, ws=None) == WORKSPACE
    assert _vls(lib, wsb=16) == WORKSPACE
    out = ctypes.c_size_t(0)
    assert lib.uno_psi_spec_verify_linear_sampled_workspace(256, 15, 151936, ctypes.byref(out)) == OK
    assert out.value > 0


def test_debug_checks_switch(lib):
    was = lib.uno_debug_checks_enabled()
    lib.uno_debug_checks(1)
    assert lib.uno_debug_checks_enabled() == 1
    lib.uno_debug_checks(0)
    assert lib.uno_debug_checks_enabled() == 0
    lib.uno_debug_checks(was)
