"""Python binding of libunospec (the Psi-Spec decode-step hot path on MI355X).

Argument marshalling only: every computation runs in the HIP kernels of
libunospec.so, reached through its C ABI (include/uno.h) with ctypes.
PyTorch supplies device memory and the current HIP stream.  There is no CPU
fallback: if the library is missing, `load()` raises.
"""

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libunospec.so")

UNO_F32, UNO_BF16 = 0, 1
_STATUS = {0: "ok", 1: "invalid argument", 2: "unsupported", 3: "workspace too small", 4: "HIP error",
           5: "internal error"}

EXPORTS = (
    "uno_abi_version", "uno_status_string", "uno_last_error",
    "uno_gated_lora_linear_workspace", "uno_gated_lora_linear", "uno_lora_merge",
    "uno_psi_spec_verify_linear_workspace", "uno_psi_spec_verify_linear", "uno_psi_spec_verify_linear_noalloc",
    "uno_psi_spec_verify_linear_early_exit_workspace", "uno_psi_spec_verify_linear_early_exit",
    "uno_psi_spec_verify_linear_sampled_workspace", "uno_psi_spec_verify_linear_sampled",
    "uno_tree_verify_attention_workspace", "uno_tree_verify_attention",
    "uno_psi_spec_verify_tree_workspace", "uno_psi_spec_verify_tree",
    "uno_psi_spec_verify_tree_wor_workspace", "uno_psi_spec_verify_tree_wor",
    "uno_psi_spec_build_tree_workspace", "uno_psi_spec_build_tree",
    "uno_distill_loss",
    "uno_gated_lora_backward_workspace", "uno_gated_lora_backward", "uno_transpose_bf16",
    "uno_rms_norm", "uno_rope", "uno_silu_mul",
    "uno_block_verify_attention_workspace", "uno_block_verify_attention",
    "uno_sample_rows_workspace", "uno_sample_rows",
    "uno_decoder_layer_workspace", "uno_decoder_layer",
    "uno_psi_spec_step_workspace", "uno_psi_spec_step",
    "uno_kv_commit",
    "uno_profile_enable", "uno_profile_reset", "uno_profile_query",
    "uno_debug_checks", "uno_debug_checks_enabled",
)


NUM_PROJ = 7
PROJ = ("q", "k", "v", "o", "g", "u", "d")    # q, k, v, o, gate, up, down (UNO_PROJ_* order)


class LayerWeights(ctypes.Structure):
    """uno_layer_weights: device pointers of one decoder layer."""
    _fields_ = [("attn_norm", ctypes.c_void_p), ("mlp_norm", ctypes.c_void_p),
                ("w", ctypes.c_void_p * NUM_PROJ), ("a", ctypes.c_void_p * NUM_PROJ),
                ("b", ctypes.c_void_p * NUM_PROJ), ("k_cache", ctypes.c_void_p), ("v_cache", ctypes.c_void_p),
                ("w_merged", ctypes.c_void_p * NUM_PROJ), ("q_norm", ctypes.c_void_p), ("k_norm", ctypes.c_void_p)]


class StepConfig(ctypes.Structure):
    """uno_step_config: shapes and scalars of one decode step."""
    _fields_ = [(n, ctypes.c_int32) for n in ("batch", "block", "ctx_len", "hidden", "inter", "n_heads",
                                              "n_kv_heads", "r", "n_layers", "vocab")] + \
               [(n, ctypes.c_float) for n in ("rms_eps", "rope_theta", "lora_scale", "temperature")]


class UnoError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"{_STATUS.get(status, status)}: {message}")
        self.status = status


_lib = None

_p = ctypes.c_void_p
_i32 = ctypes.c_int32
_i64 = ctypes.c_int64
_f32 = ctypes.c_float
_sz = ctypes.c_size_t


def _declare(lib):
    sig = {
        "uno_abi_version": (ctypes.c_int, []),
        "uno_status_string": (ctypes.c_char_p, [ctypes.c_int]),
        "uno_last_error": (ctypes.c_char_p, []),
        "uno_gated_lora_linear_workspace": (ctypes.c_int, [ctypes.c_int, _i64, _i64, _i64, _i64, ctypes.POINTER(_sz)]),
        "uno_gated_lora_linear": (ctypes.c_int, [_p, ctypes.c_int, _i64, _i64, _i64, _i64,
                                                 _p, _i64, _p, _i64, _p, _i64, _p, _i64,
                                                 _p, _f32, _p, _i64, _p, _sz]),
        "uno_psi_spec_verify_linear_workspace": (ctypes.c_int, [_i32, _i32, _i32, ctypes.POINTER(_sz)]),
        "uno_psi_spec_verify_linear": (ctypes.c_int, [_p, ctypes.c_int, _i32, _i32, _i32,
                                                      _p, _i64, _i64, _p, _i64, _i64,
                                                      _p, _p, _p, _f32, _p, _p, _p, _p, _p, _p, _sz]),
        "uno_psi_spec_verify_linear_early_exit_workspace": (ctypes.c_int, [_i32, _i32, _i32, ctypes.POINTER(_sz)]),
        "uno_psi_spec_verify_linear_early_exit": (ctypes.c_int, [_p, ctypes.c_int, _i32, _i32, _i32,
                                                                 _p, _i64, _i64, _p, _i64, _i64,
                                                                 _p, _p, _p, _f32, _p, _p, _p, _p, _p, _p, _sz]),
        "uno_psi_spec_verify_linear_sampled_workspace": (ctypes.c_int, [_i32, _i32, _i32, ctypes.POINTER(_sz)]),
        "uno_psi_spec_verify_linear_sampled": (ctypes.c_int, [_p, ctypes.c_int, _i32, _i32, _i32,
                                                              _p, _i64, _i64, _p, _i64, _i64,
                                                              _p, _p, _p, _f32, _i32, _f32, _i32,
                                                              _p, _p, _p, _p, _p, _p, _sz]),
        "uno_psi_spec_verify_linear_noalloc": (ctypes.c_int, [_p, ctypes.c_int, _i32, _i32, _i32,
                                                              _p, _i64, _i64, _p, _i64, _i64,
                                                              _p, _p, _p, _f32, _p, _p, _p, _p, _p]),
        "uno_tree_verify_attention_workspace": (ctypes.c_int, [_i32, _i32, _i32, _i32, _i32, _i32,
                                                               ctypes.POINTER(_sz)]),
        "uno_tree_verify_attention": (ctypes.c_int, [_p, _i32, _i32, _i32, _i32, _i32, _i32,
                                                     _p, _p, _p, _p, _p, _p, _f32, _p, _p, _p, _sz]),
        "uno_psi_spec_verify_tree_workspace": (ctypes.c_int, [_i32, _i32, _i32, _i32, _i32, ctypes.POINTER(_sz)]),
        "uno_psi_spec_verify_tree": (ctypes.c_int, [_p, ctypes.c_int, _i32, _i32, _i32, _i32, _i32,
                                                    _p, _p, _p, _p, _p, _p, _f32, _p, _p, _p, _p, _sz]),
        "uno_psi_spec_verify_tree_wor_workspace": (ctypes.c_int, [_i32, _i32, _i32, _i32, _i32,
                                                                  ctypes.POINTER(_sz)]),
        "uno_psi_spec_verify_tree_wor": (ctypes.c_int, [_p, ctypes.c_int, _i32, _i32, _i32, _i32, _i32,
                                                        _p, _p, _p, _p, _p, _p, _f32, _p, _p, _p, _p, _sz]),
        "uno_psi_spec_build_tree_workspace": (ctypes.c_int, [_i32, _i32, _i32, ctypes.POINTER(_sz)]),
        "uno_gated_lora_backward_workspace": (ctypes.c_int, [_i64, _i64, _i64, _i64, _i32, ctypes.POINTER(_sz)]),
        "uno_gated_lora_backward": (ctypes.c_int, [_p, _i64, _i64, _i64, _i64, _p, _i64, _p, _i64, _p, _i64, _p, _i64,
                                                   _p, _f32, _p, _i64, _p, _i64, _p, _i64, _p, _i64, _p, _i64, _p,
                                                   _sz]),
        "uno_transpose_bf16": (ctypes.c_int, [_p, _i64, _i64, _p, _i64, _p, _i64]),
        "uno_distill_loss": (ctypes.c_int, [_p, ctypes.c_int, _i32, _i32, _i32, _p, _i64, _i64, _p, _i64, _i64,
                                            _f32, _f32, _f32, _f32, _p, _p, _p, _i64, _i64]),
        "uno_psi_spec_build_tree": (ctypes.c_int, [_p, ctypes.c_int, _i32, _i32, _p, _i32, _p, _i64, _i64, _p, _i32,
                                                   _f32, _i32, _p, _p, _p, _sz]),
        "uno_rms_norm": (ctypes.c_int, [_p, _i64, _i32, _p, _i64, _p, _i64, _p, _i64, _p, _f32, _p, _i64]),
        "uno_rope": (ctypes.c_int, [_p, _i64, _i32, _p, _i64, _p, _f32, _p, _f32]),
        "uno_silu_mul": (ctypes.c_int, [_p, _i64, _i32, _p, _i64, _p, _i64, _p, _i64]),
        "uno_block_verify_attention_workspace": (ctypes.c_int, [_i32, _i32, _i32, _i32, _i32, _i32,
                                                                ctypes.POINTER(_sz)]),
        "uno_block_verify_attention": (ctypes.c_int, [_p, _i32, _i32, _i32, _i32, _i32, _i32,
                                                      _p, _p, _p, _p, _p, _p, _f32, _p, _p, _p, _sz]),
        "uno_sample_rows_workspace": (ctypes.c_int, [_i32, _i32, ctypes.POINTER(_sz)]),
        "uno_sample_rows": (ctypes.c_int, [_p, ctypes.c_int, _i32, _i32, _p, _i64, _p, _f32, _p, _p, _sz]),
        "uno_decoder_layer_workspace": (ctypes.c_int, [_i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                                                       ctypes.POINTER(_sz)]),
        "uno_decoder_layer": (ctypes.c_int, [_p, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                                             ctypes.POINTER(LayerWeights), _p, _p, _p, _f32, _f32, _f32,
                                             _p, _p, _sz]),
        "uno_psi_spec_step_workspace": (ctypes.c_int, [ctypes.POINTER(StepConfig), ctypes.POINTER(_sz)]),
        "uno_psi_spec_step": (ctypes.c_int, [_p, ctypes.POINTER(StepConfig), ctypes.POINTER(LayerWeights),
                                             _p, _p, _p, _p, _p, _p, _i64, _i64, _p, _p, _p, _p, _p, _p, _p, _p,
                                             _p, _sz]),
        "uno_kv_commit": (ctypes.c_int, [_p, _i32, _i32, _p, _p]),
        "uno_debug_checks": (None, [_i32]),
        "uno_debug_checks_enabled": (ctypes.c_int32, []),
        "uno_lora_merge": (ctypes.c_int, [_p, _i64, _i64, _i64, _p, _i64, _p, _i64, _p, _i64, _f32, _p, _i64]),
        "uno_profile_enable": (None, [ctypes.c_int, ctypes.c_char_p]),
        "uno_profile_reset": (None, []),
        "uno_profile_query": (ctypes.c_int, [ctypes.c_char_p, ctypes.POINTER(ctypes.c_double),
                                             ctypes.POINTER(_i64)]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args


def load(path=None):
    """Load libunospec.so (built in-tree by build.py).  Raises if missing."""
    global _lib
    if _lib is not None:
        return _lib
    path = path or LIB_PATH
    if not os.path.exists(path):
        raise RuntimeError(f"libunospec.so not built at {path}; run "
                           "`python -m diffusion_augmented_decoding_amd.build`")
    lib = ctypes.CDLL(path)
    _declare(lib)
    _lib = lib
    return lib


def _check(status):
    if status != 0:
        raise UnoError(status, _lib.uno_last_error().decode(errors="replace"))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _dtype_code(t):
    import torch
    if t.dtype == torch.bfloat16:
        return UNO_BF16
    if t.dtype == torch.float32:
        return UNO_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _workspace(nbytes, device, workspace):
    import torch
    if nbytes == 0:
        return None
    if workspace is not None and workspace.numel() * workspace.element_size() >= nbytes:
        return workspace
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def _nbytes(t):
    return 0 if t is None else t.numel() * t.element_size()


# ------------------------------------------------------------------ gated LoRA
def gated_lora_linear_workspace(dtype_code, m, n, k, r):
    load()
    out = _sz(0)
    _check(_lib.uno_gated_lora_linear_workspace(dtype_code, m, n, k, r, ctypes.byref(out)))
    return out.value


def gated_lora_linear(x, w, a, b, gate, lora_scale=1.0, out=None, workspace=None, stream=None):
    """y = x W^T + lora_scale * diag(gate) (x A^T) B^T  (uno_gated_lora_linear).

    x [M, K], w [N, K], a [r, K], b [N, r] (bf16 or fp32, same dtype, row
    strides taken from the tensors), gate uint8 [M] or None.
    """
    import torch
    load()
    m, k = x.shape
    n = w.shape[0]
    r = a.shape[0] if a is not None else 0
    code = _dtype_code(x)
    if out is None:
        out = torch.empty((m, n), dtype=x.dtype, device=x.device)
    nb = gated_lora_linear_workspace(code, m, n, k, r if gate is not None else 0)
    ws = _workspace(nb, x.device, workspace)
    _check(_lib.uno_gated_lora_linear(
        _stream(stream), code, m, n, k, r,
        _ptr(x), x.stride(0), _ptr(w), w.stride(0),
        _ptr(a), a.stride(0) if a is not None else k, _ptr(b), b.stride(0) if b is not None else r,
        _ptr(gate), float(lora_scale), _ptr(out), out.stride(0), _ptr(ws), _nbytes(ws)))
    return out


# ------------------------------------------------------------------ linear verify
def psi_spec_verify_linear_workspace(batch, k, vocab):
    load()
    out = _sz(0)
    _check(_lib.uno_psi_spec_verify_linear_workspace(batch, k, vocab, ctypes.byref(out)))
    return out.value


def psi_spec_verify_linear(p_logits, q_logits, drafts, u_accept, u_sample, temperature=1.0,
                           outputs=None, want_probs=True, workspace=None, stream=None):
    """Linear Psi-Spec verify (uno_psi_spec_verify_linear).

    p_logits [B, k+1, V], q_logits [B, k, V] (bf16/fp32, last dim contiguous),
    drafts int32 [B, k], u_accept f32 [B, k], u_sample f32 [B].
    Returns dict of device tensors: accept_len, token, and (want_probs)
    p_draft, q_draft, residual_mass.
    """
    import torch
    load()
    bsz, k1, vocab = p_logits.shape
    k = k1 - 1
    dev = p_logits.device
    if outputs is None:
        outputs = {
            "accept_len": torch.empty(bsz, dtype=torch.int32, device=dev),
            "token": torch.empty(bsz, dtype=torch.int32, device=dev),
        }
        if want_probs:
            outputs["p_draft"] = torch.empty((bsz, k), dtype=torch.float32, device=dev)
            outputs["q_draft"] = torch.empty((bsz, k), dtype=torch.float32, device=dev)
            outputs["residual_mass"] = torch.empty(bsz, dtype=torch.float32, device=dev)
    ws = _workspace(psi_spec_verify_linear_workspace(bsz, k, vocab), dev, workspace)
    qs = q_logits.stride() if q_logits is not None else (0, 0, 1)
    _check(_lib.uno_psi_spec_verify_linear(
        _stream(stream), _dtype_code(p_logits), bsz, k, vocab,
        _ptr(p_logits), p_logits.stride(0), p_logits.stride(1),
        _ptr(q_logits), qs[0], qs[1],
        _ptr(drafts), _ptr(u_accept), _ptr(u_sample), float(temperature),
        _ptr(outputs["accept_len"]), _ptr(outputs["token"]),
        _ptr(outputs.get("p_draft")), _ptr(outputs.get("q_draft")), _ptr(outputs.get("residual_mass")),
        _ptr(ws), _nbytes(ws)))
    return outputs


def psi_spec_verify_linear_early_exit_workspace(batch, k, vocab):
    load()
    out = _sz(0)
    _check(_lib.uno_psi_spec_verify_linear_early_exit_workspace(batch, k, vocab, ctypes.byref(out)))
    return out.value


def psi_spec_verify_linear_early_exit(p_logits, q_logits, drafts, u_accept, u_sample, temperature=1.0,
                                      outputs=None, want_probs=True, workspace=None, stream=None):
    """Early-exit linear verify (uno_psi_spec_verify_linear_early_exit): the
    arguments and outputs of psi_spec_verify_linear; p_draft / q_draft are NaN
    after the first rejection."""
    import torch
    load()
    bsz, k1, vocab = p_logits.shape
    k = k1 - 1
    dev = p_logits.device
    if outputs is None:
        outputs = {
            "accept_len": torch.empty(bsz, dtype=torch.int32, device=dev),
            "token": torch.empty(bsz, dtype=torch.int32, device=dev),
        }
        if want_probs:
            outputs["p_draft"] = torch.empty((bsz, k), dtype=torch.float32, device=dev)
            outputs["q_draft"] = torch.empty((bsz, k), dtype=torch.float32, device=dev)
            outputs["residual_mass"] = torch.empty(bsz, dtype=torch.float32, device=dev)
    ws = _workspace(psi_spec_verify_linear_early_exit_workspace(bsz, k, vocab), dev, workspace)
    qs = q_logits.stride() if q_logits is not None else (0, 0, 1)
    _check(_lib.uno_psi_spec_verify_linear_early_exit(
        _stream(stream), _dtype_code(p_logits), bsz, k, vocab,
        _ptr(p_logits), p_logits.stride(0), p_logits.stride(1),
        _ptr(q_logits), qs[0], qs[1],
        _ptr(drafts), _ptr(u_accept), _ptr(u_sample), float(temperature),
        _ptr(outputs["accept_len"]), _ptr(outputs["token"]),
        _ptr(outputs.get("p_draft")), _ptr(outputs.get("q_draft")), _ptr(outputs.get("residual_mass")),
        _ptr(ws), _nbytes(ws)))
    return outputs


def psi_spec_verify_linear_sampled_workspace(batch, k, vocab):
    load()
    out = _sz(0)
    _check(_lib.uno_psi_spec_verify_linear_sampled_workspace(batch, k, vocab, ctypes.byref(out)))
    return out.value


def psi_spec_verify_linear_sampled(p_logits, q_logits, drafts, u_accept, u_sample, temperature=1.0, top_k=0,
                                   top_p=1.0, greedy=False, outputs=None, want_probs=True, workspace=None,
                                   stream=None):
    """Linear verify under a sampling transform (uno_psi_spec_verify_linear_sampled):
    top_k (0 off), top_p (1 off), greedy.  Arguments and outputs as
    psi_spec_verify_linear; p_draft / q_draft are transformed probabilities."""
    import torch
    load()
    bsz, k1, vocab = p_logits.shape
    k = k1 - 1
    dev = p_logits.device
    if outputs is None:
        outputs = {
            "accept_len": torch.empty(bsz, dtype=torch.int32, device=dev),
            "token": torch.empty(bsz, dtype=torch.int32, device=dev),
        }
        if want_probs:
            outputs["p_draft"] = torch.empty((bsz, k), dtype=torch.float32, device=dev)
            outputs["q_draft"] = torch.empty((bsz, k), dtype=torch.float32, device=dev)
            outputs["residual_mass"] = torch.empty(bsz, dtype=torch.float32, device=dev)
    ws = _workspace(psi_spec_verify_linear_sampled_workspace(bsz, k, vocab), dev, workspace)
    qs = q_logits.stride() if q_logits is not None else (0, 0, 1)
    _check(_lib.uno_psi_spec_verify_linear_sampled(
        _stream(stream), _dtype_code(p_logits), bsz, k, vocab,
        _ptr(p_logits), p_logits.stride(0), p_logits.stride(1),
        _ptr(q_logits), qs[0], qs[1],
        _ptr(drafts), _ptr(u_accept), _ptr(u_sample), float(temperature), int(top_k), float(top_p),
        1 if greedy else 0,
        _ptr(outputs["accept_len"]), _ptr(outputs["token"]),
        _ptr(outputs.get("p_draft")), _ptr(outputs.get("q_draft")), _ptr(outputs.get("residual_mass")),
        _ptr(ws), _nbytes(ws)))
    return outputs


def psi_spec_verify_linear_noalloc(p_logits, q_logits, drafts, u_accept, u_sample, temperature=1.0,
                                   outputs=None, want_probs=True, stream=None):
    """uno_psi_spec_verify_linear_noalloc: the linear verify with no workspace
    (the library's own per-GPU scratch; see include/uno.h).  Arguments and the
    returned dict as psi_spec_verify_linear; `outputs` may be passed so that
    nothing at all is allocated here."""
    import torch
    load()
    bsz, k1, vocab = p_logits.shape
    k = k1 - 1
    dev = p_logits.device
    if outputs is None:
        outputs = {
            "accept_len": torch.empty(bsz, dtype=torch.int32, device=dev),
            "token": torch.empty(bsz, dtype=torch.int32, device=dev),
        }
        if want_probs:
            outputs["p_draft"] = torch.empty((bsz, k), dtype=torch.float32, device=dev)
            outputs["q_draft"] = torch.empty((bsz, k), dtype=torch.float32, device=dev)
            outputs["residual_mass"] = torch.empty(bsz, dtype=torch.float32, device=dev)
    qs = q_logits.stride() if q_logits is not None else (0, 0, 1)
    _check(_lib.uno_psi_spec_verify_linear_noalloc(
        _stream(stream), _dtype_code(p_logits), bsz, k, vocab,
        _ptr(p_logits), p_logits.stride(0), p_logits.stride(1),
        _ptr(q_logits), qs[0], qs[1],
        _ptr(drafts), _ptr(u_accept), _ptr(u_sample), float(temperature),
        _ptr(outputs["accept_len"]), _ptr(outputs["token"]),
        _ptr(outputs.get("p_draft")), _ptr(outputs.get("q_draft")), _ptr(outputs.get("residual_mass"))))
    return outputs


# ------------------------------------------------------------------ tree attention
def tree_verify_attention_workspace(batch, n_tree, ctx, n_heads, n_kv, head_dim):
    load()
    out = _sz(0)
    _check(_lib.uno_tree_verify_attention_workspace(batch, n_tree, ctx, n_heads, n_kv, head_dim,
                                                    ctypes.byref(out)))
    return out.value


def tree_verify_attention(q, k_cache, v_cache, k_tree, v_tree, parent, softmax_scale,
                          out=None, lse=None, want_lse=True, workspace=None, stream=None):
    """Tree-masked GQA attention (uno_tree_verify_attention).

    q [B, n, H, 128], k_cache/v_cache [B, ctx, Hkv, 128], k_tree/v_tree
    [B, n, Hkv, 128] (bf16, contiguous), parent int32 [B, n].
    Returns (out bf16 [B, n, H, 128], lse f32 [B, n, H] or None).
    """
    import torch
    load()
    bsz, n, nh, hd = q.shape
    ctx = k_cache.shape[1]
    nkv = k_tree.shape[2]
    if out is None:
        out = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty((bsz, n, nh), dtype=torch.float32, device=q.device)
    ws = _workspace(tree_verify_attention_workspace(bsz, n, ctx, nh, nkv, hd), q.device, workspace)
    _check(_lib.uno_tree_verify_attention(
        _stream(stream), bsz, n, ctx, nh, nkv, hd,
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_tree), _ptr(v_tree), _ptr(parent),
        float(softmax_scale), _ptr(out), _ptr(lse), _ptr(ws), _nbytes(ws)))
    return out, lse


# ------------------------------------------------------------------ tree verify
def psi_spec_verify_tree_workspace(batch, n_tree, max_depth, max_children, vocab, without_replacement=False):
    load()
    out = _sz(0)
    fn = _lib.uno_psi_spec_verify_tree_wor_workspace if without_replacement else _lib.uno_psi_spec_verify_tree_workspace
    _check(fn(batch, n_tree, max_depth, max_children, vocab, ctypes.byref(out)))
    return out.value


def psi_spec_verify_tree(parent, tokens, p_logits, q_logits, u_accept, u_sample, temperature=1.0,
                         max_children=None, outputs=None, workspace=None, stream=None, without_replacement=False):
    """Tree Psi-Spec verify (uno_psi_spec_verify_tree, or
    uno_psi_spec_verify_tree_wor for siblings drawn without replacement).

    parent, tokens int32 [B, n]; p_logits [B, n, V]; q_logits [B, D, V]
    (contiguous); u_accept f32 [B, n]; u_sample f32 [B].  max_children: bound
    on the children of any node (None: n - 1, at most 64 without replacement).
    Returns dict: accept_len [B], path [B, D], token [B] (int32 device tensors).
    """
    import torch
    load()
    bsz, n, vocab = p_logits.shape
    dmax = q_logits.shape[1]
    dev = p_logits.device
    if max_children is None:
        max_children = max(n - 1, 0)
        if without_replacement:
            max_children = min(max_children, 64)
    if outputs is None:
        outputs = {
            "accept_len": torch.empty(bsz, dtype=torch.int32, device=dev),
            "path": torch.empty((bsz, dmax), dtype=torch.int32, device=dev),
            "token": torch.empty(bsz, dtype=torch.int32, device=dev),
        }
    ws = _workspace(psi_spec_verify_tree_workspace(bsz, n, dmax, max_children, vocab, without_replacement), dev,
                    workspace)
    fn = _lib.uno_psi_spec_verify_tree_wor if without_replacement else _lib.uno_psi_spec_verify_tree
    _check(fn(
        _stream(stream), _dtype_code(p_logits), bsz, n, dmax, max_children, vocab,
        _ptr(parent), _ptr(tokens), _ptr(p_logits), _ptr(q_logits), _ptr(u_accept), _ptr(u_sample),
        float(temperature), _ptr(outputs["accept_len"]), _ptr(outputs["path"]), _ptr(outputs["token"]),
        _ptr(ws), _nbytes(ws)))
    return outputs


def tree_size(branching):
    """Node count of the breadth-first tree with the given branching per depth."""
    n, width = 1, 1
    for b in branching:
        width *= int(b)
        n += width
    return n


def psi_spec_build_tree_workspace(batch, max_depth, vocab):
    load()
    out = _sz(0)
    _check(_lib.uno_psi_spec_build_tree_workspace(batch, max_depth, vocab, ctypes.byref(out)))
    return out.value


def psi_spec_build_tree(q_logits, branching, u_draw, temperature=1.0, without_replacement=False, outputs=None,
                        workspace=None, stream=None):
    """Candidate trees from the per-depth draft marginals (uno_psi_spec_build_tree).

    q_logits [B, D, V] (last dim contiguous; any batch and depth strides, e.g.
    the noisy rows of a step's logits); branching: D ints; u_draw f32 [B, n]
    with n = tree_size(branching).  Returns dict parent, tokens (int32 [B, n]
    device tensors; parent[:, 0] = tokens[:, 0] = -1).
    """
    import torch
    load()
    bsz, dmax, vocab = q_logits.shape
    if q_logits.stride(2) != 1:
        raise ValueError("q_logits: the vocabulary dimension must be contiguous")
    n = tree_size(branching)
    dev = q_logits.device
    if outputs is None:
        outputs = {"parent": torch.empty((bsz, n), dtype=torch.int32, device=dev),
                   "tokens": torch.empty((bsz, n), dtype=torch.int32, device=dev)}
    br = (ctypes.c_int32 * max(len(branching), 1))(*[int(b) for b in branching])
    ws = _workspace(psi_spec_build_tree_workspace(bsz, dmax, vocab), dev, workspace)
    _check(_lib.uno_psi_spec_build_tree(
        _stream(stream), _dtype_code(q_logits), bsz, dmax, br, vocab, _ptr(q_logits), q_logits.stride(0),
        q_logits.stride(1), _ptr(u_draw), n, float(temperature), int(bool(without_replacement)),
        _ptr(outputs["parent"]), _ptr(outputs["tokens"]), _ptr(ws), _nbytes(ws)))
    return outputs


def gated_lora_backward_workspace(M, N, K, r, with_w_t=False):
    load()
    out = _sz(0)
    _check(_lib.uno_gated_lora_backward_workspace(M, N, K, r, int(bool(with_w_t)), ctypes.byref(out)))
    return out.value


def transpose_bf16(src, out=None, stream=None):
    """out = src^T for a bf16 [rows, cols] matrix (uno_transpose_bf16)."""
    import torch
    load()
    rows, cols = src.shape
    if out is None:
        out = torch.empty((cols, rows), dtype=src.dtype, device=src.device)
    _check(_lib.uno_transpose_bf16(_stream(stream), rows, cols, _ptr(src), src.stride(0), _ptr(out), out.stride(0)))
    return out


def gated_lora_backward(x, w, a, b, gate, dy, lora_scale=1.0, want_dx=True, outputs=None, workspace=None,
                        stream=None, w_t=None):
    """Gradients of the gated-LoRA linear layer (uno_gated_lora_backward).

    bf16 x [M, K], w [N, K], a [r, K], b [N, r], dy [M, N] (rows with a
    contiguous last dim); gate uint8 [M] or None; w_t: optional W^T [K, N]
    (transpose_bf16(w), made once for a frozen weight).  Returns dict da (f32
    [r, K]), db (f32 [N, r]) and dx (bf16 [M, K]) when want_dx."""
    import torch
    load()
    M, K = x.shape
    N = w.shape[0]
    r = a.shape[0]
    dev = x.device
    if outputs is None:
        outputs = {"da": torch.empty((r, K), dtype=torch.float32, device=dev),
                   "db": torch.empty((N, r), dtype=torch.float32, device=dev)}
        if want_dx:
            outputs["dx"] = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
    dx = outputs.get("dx")
    ws = _workspace(gated_lora_backward_workspace(M, N, K, r, w_t is not None), dev, workspace)
    _check(_lib.uno_gated_lora_backward(
        _stream(stream), M, N, K, r, _ptr(x), x.stride(0), _ptr(w), w.stride(0), _ptr(a), a.stride(0), _ptr(b),
        b.stride(0), _ptr(gate), float(lora_scale), _ptr(dy), dy.stride(0), _ptr(dx),
        dx.stride(0) if dx is not None else K, _ptr(outputs["da"]), outputs["da"].stride(0), _ptr(outputs["db"]),
        outputs["db"].stride(0), _ptr(w_t), w_t.stride(0) if w_t is not None else 0, _ptr(ws), _nbytes(ws)))
    return outputs


def distill_loss(teacher, student, temperature=1.0, alpha=1.0, beta=1.0, grad_scale=1.0, want_grad=True,
                 outputs=None, stream=None):
    """Distillation losses of row pairs (uno_distill_loss).

    teacher, student [B, R, V] (last dim contiguous; any batch and row strides,
    e.g. the clean and noisy halves of a step's logits).  Returns dict kl, tv
    (f32 [B, R]) and grad ([B, R, V], the logits' dtype) when want_grad."""
    import torch
    load()
    bsz, rows, vocab = student.shape
    if teacher.shape != student.shape or teacher.dtype != student.dtype:
        raise ValueError("teacher and student must have the same shape and dtype")
    if teacher.stride(2) != 1 or student.stride(2) != 1:
        raise ValueError("the vocabulary dimension must be contiguous")
    dev = student.device
    if outputs is None:
        outputs = {"kl": torch.empty((bsz, rows), dtype=torch.float32, device=dev),
                   "tv": torch.empty((bsz, rows), dtype=torch.float32, device=dev)}
        if want_grad:
            outputs["grad"] = torch.empty((bsz, rows, vocab), dtype=student.dtype, device=dev)
    g = outputs.get("grad")
    _check(_lib.uno_distill_loss(
        _stream(stream), _dtype_code(student), bsz, rows, vocab, _ptr(teacher), teacher.stride(0), teacher.stride(1),
        _ptr(student), student.stride(0), student.stride(1), float(temperature), float(alpha), float(beta),
        float(grad_scale), _ptr(outputs["kl"]), _ptr(outputs["tv"]), _ptr(g),
        g.stride(0) if g is not None else 0, g.stride(1) if g is not None else vocab))
    return outputs


# ------------------------------------------------------------------ layer ops
def rms_norm(x, weight, eps=1e-6, res=None, sum_out=None, out=None, want_out=True, stream=None):
    """RMSNorm of x [rows, dim] (uno_rms_norm); with res, x + res is formed
    first and written to sum_out (default: x itself).  Returns out (or None)."""
    import torch
    load()
    rows, dim = x.shape
    if res is not None and sum_out is None:
        sum_out = x
    if out is None and want_out:
        out = torch.empty((rows, dim), dtype=x.dtype, device=x.device)
    _check(_lib.uno_rms_norm(
        _stream(stream), rows, dim, _ptr(x), x.stride(0), _ptr(res), res.stride(0) if res is not None else dim,
        _ptr(sum_out), sum_out.stride(0) if sum_out is not None else dim, _ptr(weight), float(eps),
        _ptr(out), out.stride(0) if out is not None else dim))
    return out


def rope(x, positions, theta=1.0e6, norm_weight=None, norm_eps=1e-6, stream=None):
    """Rotary embedding in place on x [rows, n_heads * 128] (uno_rope), each
    head first normed with norm_weight [128] when given."""
    load()
    rows, width = x.shape
    _check(_lib.uno_rope(_stream(stream), rows, width // 128, _ptr(x), x.stride(0), _ptr(positions), float(theta),
                         _ptr(norm_weight) if norm_weight is not None else None, float(norm_eps)))
    return x


def silu_mul(g, u, out=None, stream=None):
    """out = silu(g) * u on [rows, dim] bf16 (uno_silu_mul)."""
    import torch
    load()
    rows, dim = g.shape
    if out is None:
        out = torch.empty_like(g)
    _check(_lib.uno_silu_mul(_stream(stream), rows, dim, _ptr(g), g.stride(0), _ptr(u), u.stride(0),
                             _ptr(out), out.stride(0)))
    return out


def block_verify_attention_workspace(batch, block, ctx, n_heads, n_kv, head_dim):
    load()
    out = _sz(0)
    _check(_lib.uno_block_verify_attention_workspace(batch, block, ctx, n_heads, n_kv, head_dim,
                                                     ctypes.byref(out)))
    return out.value


def block_verify_attention(q, k_cache, v_cache, k_block, v_block, block, softmax_scale,
                           out=None, lse=None, want_lse=True, workspace=None, stream=None, cache_len=None):
    """Block-masked GQA attention (uno_block_verify_attention).

    q [B, 2*block, H, 128], k_cache/v_cache [B, ctx, Hkv, 128], k_block/v_block
    [B, 2*block, Hkv, 128] (bf16, contiguous); cache_len int32 [B] (optional):
    valid cache rows per sequence.  Returns (out, lse or None).
    """
    import torch
    load()
    bsz, n, nh, hd = q.shape
    ctx = k_cache.shape[1]
    nkv = k_block.shape[2]
    if out is None:
        out = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty((bsz, n, nh), dtype=torch.float32, device=q.device)
    ws = _workspace(block_verify_attention_workspace(bsz, block, ctx, nh, nkv, hd), q.device, workspace)
    _check(_lib.uno_block_verify_attention(
        _stream(stream), bsz, block, ctx, nh, nkv, hd, _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(cache_len),
        _ptr(k_block), _ptr(v_block), float(softmax_scale), _ptr(out), _ptr(lse), _ptr(ws), _nbytes(ws)))
    return out, lse


def sample_rows_workspace(rows, vocab):
    load()
    out = _sz(0)
    _check(_lib.uno_sample_rows_workspace(rows, vocab, ctypes.byref(out)))
    return out.value


def sample_rows(logits, u, temperature=1.0, out=None, workspace=None, stream=None):
    """Inverse-CDF draw per row of softmax(logits / T) (uno_sample_rows).
    logits [rows, V] (last dim contiguous), u f32 [rows].  Returns int32 [rows]."""
    import torch
    load()
    rows, vocab = logits.shape
    if out is None:
        out = torch.empty(rows, dtype=torch.int32, device=logits.device)
    ws = _workspace(sample_rows_workspace(rows, vocab), logits.device, workspace)
    _check(_lib.uno_sample_rows(_stream(stream), _dtype_code(logits), rows, vocab, _ptr(logits), logits.stride(0),
                                _ptr(u), float(temperature), _ptr(out), _ptr(ws), _nbytes(ws)))
    return out


def decoder_layer_workspace(batch, block, ctx, hidden, inter, n_heads, n_kv, r):
    load()
    out = _sz(0)
    _check(_lib.uno_decoder_layer_workspace(batch, block, ctx, hidden, inter, n_heads, n_kv, r,
                                            ctypes.byref(out)))
    return out.value


def lora_merge(w, a, b, lora_scale=1.0, out=None, stream=None):
    """uno_lora_merge: bf16(w + lora_scale * b @ a) for bf16 w [N][K], a [r][K],
    b [N][r] (rows may be strided; the last dimension contiguous)."""
    import torch
    N, K = w.shape
    r = a.shape[0]
    if out is None:
        out = torch.empty((N, K), dtype=torch.bfloat16, device=w.device)
    for t in (w, a, b, out):
        if t.dtype != torch.bfloat16 or t.stride(1) != 1:
            raise ValueError("bf16 matrices with contiguous rows expected")
    _check(_lib.uno_lora_merge(_stream(stream), N, K, r, _ptr(w), w.stride(0), _ptr(a), a.stride(0), _ptr(b),
                               b.stride(0), float(lora_scale), _ptr(out), out.stride(0)))
    return out


def merge_layer(w, lora_scale=1.0, stream=None):
    """The gate-merged weights of one layer's dict (see layer_weights): adds
    "m" + p = bf16(w_p + lora_scale * b_p a_p) for every projection p."""
    for p in PROJ:
        w["m" + p] = lora_merge(w["w" + p], w["a" + p], w["b" + p], lora_scale, stream=stream)
    return w


def layer_weights(w, k_cache=None, v_cache=None):
    """uno_layer_weights from a dict of device tensors: attn_norm, mlp_norm and
    w/a/b + one of q k v o g u d (gate, up, down), e.g. "wq", "aq", "bq",
    optionally the per-head "q_norm", "k_norm" (both or neither) and the
    gate-merged "mq", ... (all seven; see merge_layer)."""
    lw = LayerWeights()
    lw.attn_norm = w["attn_norm"].data_ptr()
    lw.mlp_norm = w["mlp_norm"].data_ptr()
    lw.q_norm = w["q_norm"].data_ptr() if "q_norm" in w else None
    lw.k_norm = w["k_norm"].data_ptr() if "k_norm" in w else None
    for i, p in enumerate(PROJ):
        lw.w[i] = w["w" + p].data_ptr()
        lw.a[i] = w["a" + p].data_ptr() if ("a" + p) in w else None
        lw.b[i] = w["b" + p].data_ptr() if ("b" + p) in w else None
    lw.k_cache = k_cache.data_ptr() if k_cache is not None else None
    lw.v_cache = v_cache.data_ptr() if v_cache is not None else None
    if all(("m" + p) in w for p in PROJ):
        for i, p in enumerate(PROJ):
            lw.w_merged[i] = w["m" + p].data_ptr()
    return lw


def decoder_layer(hidden_state, weights, gate, positions, batch, block, ctx, n_heads, n_kv, inter, r,
                  rms_eps=1e-6, rope_theta=1.0e6, lora_scale=1.0, workspace=None, stream=None, cache_len=None):
    """One decoder layer in place on hidden_state [rows, hidden] (uno_decoder_layer).
    weights: a LayerWeights (see layer_weights); cache_len int32 [batch]
    (optional): valid cache rows per sequence, ctx then being the capacity;
    the clean rows' k and v are written after them."""
    load()
    hidden = hidden_state.shape[1]
    ws = _workspace(decoder_layer_workspace(batch, block, ctx, hidden, inter, n_heads, n_kv, r),
                    hidden_state.device, workspace)
    _check(_lib.uno_decoder_layer(_stream(stream), batch, block, ctx, hidden, inter, n_heads, n_kv, r,
                                  ctypes.byref(weights), _ptr(gate), _ptr(positions), _ptr(cache_len), float(rms_eps),
                                  float(rope_theta), float(lora_scale), _ptr(hidden_state), _ptr(ws), _nbytes(ws)))
    return hidden_state


# ------------------------------------------------------------------ decode step
def step_config(batch, block, ctx_len, hidden, inter, n_heads, n_kv_heads, r, n_layers, vocab,
                rms_eps=1e-6, rope_theta=1.0e6, lora_scale=1.0, temperature=1.0):
    return StepConfig(batch, block, ctx_len, hidden, inter, n_heads, n_kv_heads, r, n_layers, vocab,
                      rms_eps, rope_theta, lora_scale, temperature)


def psi_spec_step_workspace(cfg):
    load()
    out = _sz(0)
    _check(_lib.uno_psi_spec_step_workspace(ctypes.byref(cfg), ctypes.byref(out)))
    return out.value


def psi_spec_step(cfg, layers, embed, final_norm, lm_head, tokens, u_draft, u_accept, u_sample,
                  prev_q=None, logits=None, outputs=None, workspace=None, stream=None, cache_len=None,
                  next_tokens=None):
    """One decode step of the decode loop (uno_psi_spec_step).

    cfg: StepConfig; layers: sequence (or ctypes array) of LayerWeights, one per layer;
    embed, lm_head bf16 [vocab, hidden]; final_norm bf16 [hidden];
    tokens int32 [batch, 2*block] (clean ids [y, drafts], then noisy ids);
    u_draft, u_accept f32 [batch, block-1]; u_sample f32 [batch].
    prev_q: bf16 [batch, block-1, vocab] view (any strides, last dim
    contiguous) of the previous step's noisy-row logits the clean drafts were
    drawn from (e.g. noisy_rows(previous logits, cfg)); None on the loop's
    first step (no draft verified).
    Returns a dict of device tensors: logits [batch*2*block, vocab] bf16,
    drafts [batch, block-1], accept_len and token [batch] (`outputs`, if
    given, is such a dict to write into), and next_tokens when asked for
    (next_tokens: an int32 [batch, 2*block] tensor, or True for a new one;
    it may be `tokens` itself).
    cache_len int32 [batch] (optional, updated in place): valid cache rows per
    sequence out of cfg.ctx_len; the step appends the clean rows' k and v and
    commits the kept ones (a sequence whose kept rows do not fit gets
    accept_len = token = -1).
    """
    import torch
    load()
    dev = tokens.device
    rows = cfg.batch * 2 * cfg.block
    k = cfg.block - 1
    if logits is None:
        logits = torch.empty((rows, cfg.vocab), dtype=torch.bfloat16, device=dev)
    if outputs is None:
        outputs = {"drafts": torch.empty((cfg.batch, max(k, 0)), dtype=torch.int32, device=dev),
                   "accept_len": torch.empty(cfg.batch, dtype=torch.int32, device=dev),
                   "token": torch.empty(cfg.batch, dtype=torch.int32, device=dev)}
    if next_tokens is True:
        next_tokens = torch.empty_like(tokens)
    drafts, acc, tok = outputs["drafts"], outputs["accept_len"], outputs["token"]
    arr = layers if isinstance(layers, ctypes.Array) else (LayerWeights * max(len(layers), 1))(*layers)
    ws = _workspace(psi_spec_step_workspace(cfg), dev, workspace)
    qs = prev_q.stride() if prev_q is not None else (0, 0, 1)
    _check(_lib.uno_psi_spec_step(_stream(stream), ctypes.byref(cfg), arr, _ptr(embed), _ptr(final_norm),
                                  _ptr(lm_head), _ptr(tokens), _ptr(cache_len), _ptr(prev_q), qs[0], qs[1],
                                  _ptr(u_draft), _ptr(u_accept), _ptr(u_sample), _ptr(logits),
                                  _ptr(drafts) if k > 0 else None, _ptr(acc), _ptr(tok), _ptr(next_tokens),
                                  _ptr(ws), _nbytes(ws)))
    out = {"logits": logits, "drafts": drafts, "accept_len": acc, "token": tok}
    if next_tokens is not None:
        out["next_tokens"] = next_tokens
    return out


def noisy_rows(logits, cfg):
    """The [batch, block-1, vocab] view of a step's logits holding its noisy
    rows 0..k-1: the q the next step verifies its drafts against."""
    lg = logits.view(cfg.batch, 2 * cfg.block, cfg.vocab)
    return lg[:, cfg.block:2 * cfg.block - 1]


def kv_commit(accept_len, cache_len, capacity, stream=None):
    """cache_len[b] += accept_len[b] + 1 in place when the kept rows fit the
    capacity, else accept_len[b] = -1 (uno_kv_commit)."""
    load()
    _check(_lib.uno_kv_commit(_stream(stream), int(cache_len.shape[0]), int(capacity), _ptr(accept_len),
                              _ptr(cache_len)))
    return cache_len


def layer_array(layers):
    """A ctypes array of LayerWeights (reusable across psi_spec_step calls)."""
    return (LayerWeights * max(len(layers), 1))(*layers)


# ------------------------------------------------------------------ kernel timing
def debug_checks(on=None):
    """Data-contract checks of token ids and uniforms (uno_debug_checks): set
    them on or off, or (on=None) return whether they are on."""
    load()
    if on is not None:
        _lib.uno_debug_checks(1 if on else 0)
    return bool(_lib.uno_debug_checks_enabled())


def profile_enable(on=True, name_filter=None):
    """Record HIP events around kernels whose name contains name_filter (None = all)."""
    load()
    _lib.uno_profile_enable(1 if on else 0, name_filter.encode() if name_filter else None)


def profile_reset():
    load()
    _lib.uno_profile_reset()


def profile_query(name):
    """(total milliseconds, launch count) of kernels whose name contains `name`."""
    load()
    ms = ctypes.c_double(0.0)
    cnt = _i64(0)
    _check(_lib.uno_profile_query(name.encode(), ctypes.byref(ms), ctypes.byref(cnt)))
    return ms.value, cnt.value
