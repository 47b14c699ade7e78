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
    "uno_gated_lora_linear_workspace", "uno_gated_lora_linear",
    "uno_psi_spec_verify_linear_workspace", "uno_psi_spec_verify_linear",
    "uno_tree_verify_attention_workspace", "uno_tree_verify_attention",
    "uno_psi_spec_verify_tree_workspace", "uno_psi_spec_verify_tree",
    "uno_profile_enable", "uno_profile_reset", "uno_profile_query",
)


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
        "uno_tree_verify_attention_workspace": (ctypes.c_int, [_i32, _i32, _i32, _i32, _i32, _i32,
                                                               ctypes.POINTER(_sz)]),
        "uno_tree_verify_attention": (ctypes.c_int, [_p, _i32, _i32, _i32, _i32, _i32, _i32,
                                                     _p, _p, _p, _p, _p, _p, _f32, _p, _p, _p, _sz]),
        "uno_psi_spec_verify_tree_workspace": (ctypes.c_int, [_i32, _i32, _i32, _i32, _i32, ctypes.POINTER(_sz)]),
        "uno_psi_spec_verify_tree": (ctypes.c_int, [_p, ctypes.c_int, _i32, _i32, _i32, _i32, _i32,
                                                    _p, _p, _p, _p, _p, _p, _f32, _p, _p, _p, _p, _sz]),
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
def psi_spec_verify_tree_workspace(batch, n_tree, max_depth, max_children, vocab):
    load()
    out = _sz(0)
    _check(_lib.uno_psi_spec_verify_tree_workspace(batch, n_tree, max_depth, max_children, vocab,
                                                   ctypes.byref(out)))
    return out.value


def psi_spec_verify_tree(parent, tokens, p_logits, q_logits, u_accept, u_sample, temperature=1.0,
                         max_children=None, outputs=None, workspace=None, stream=None):
    """Tree Psi-Spec verify (uno_psi_spec_verify_tree).

    parent, tokens int32 [B, n]; p_logits [B, n, V]; q_logits [B, D, V]
    (contiguous); u_accept f32 [B, n]; u_sample f32 [B].  max_children: bound
    on the children of any node (None: n - 1).
    Returns dict: accept_len [B], path [B, D], token [B] (int32 device tensors).
    """
    import torch
    load()
    bsz, n, vocab = p_logits.shape
    dmax = q_logits.shape[1]
    dev = p_logits.device
    if max_children is None:
        max_children = max(n - 1, 0)
    if outputs is None:
        outputs = {
            "accept_len": torch.empty(bsz, dtype=torch.int32, device=dev),
            "path": torch.empty((bsz, dmax), dtype=torch.int32, device=dev),
            "token": torch.empty(bsz, dtype=torch.int32, device=dev),
        }
    ws = _workspace(psi_spec_verify_tree_workspace(bsz, n, dmax, max_children, vocab), dev, workspace)
    _check(_lib.uno_psi_spec_verify_tree(
        _stream(stream), _dtype_code(p_logits), bsz, n, dmax, max_children, vocab,
        _ptr(parent), _ptr(tokens), _ptr(p_logits), _ptr(q_logits), _ptr(u_accept), _ptr(u_sample),
        float(temperature), _ptr(outputs["accept_len"]), _ptr(outputs["path"]), _ptr(outputs["token"]),
        _ptr(ws), _nbytes(ws)))
    return outputs


# ------------------------------------------------------------------ kernel timing
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
