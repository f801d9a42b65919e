"""ctypes binding of libgdn (include/gdn.h).

The raw entry points keep the C names and take integer device addresses:
``gdn_chunk_fwd``, ``gdn_chunk_fwd_prologue``, ``gdn_chunk_bwd``,
``gdn_fwd_channel_decay``, ``gdn_recurrent_step``, ``gdn_chunk_fwd_noalloc``,
``gdn_chunk_fwd_workspace_bytes``, ``gdn_chunk_fwd_prologue_workspace_bytes``,
``gdn_chunk_bwd_workspace_bytes``, ``gdn_status_str``.  ``chunk_fwd``,
``chunk_fwd_prologue``, ``chunk_bwd``, ``fwd_channel_decay`` and ``recurrent_step`` are conveniences for
torch tensors: they check dtypes and shapes, allocate outputs with torch, pass
``data_ptr()`` and the current HIP stream, and raise on a non-OK status.  Every
step of the computation runs in the HIP kernels; there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgdn.so")

GDN_OK, GDN_ERR_NULL, GDN_ERR_SHAPE, GDN_ERR_DTYPE = 0, 1, 2, 3
GDN_ERR_UNSUPPORTED, GDN_ERR_ALIGN, GDN_ERR_WORKSPACE, GDN_ERR_HIP = 4, 5, 6, 7
GDN_F32, GDN_BF16, GDN_C64 = 0, 1, 2
GDN_NOALLOC_MAX_WORKSPACE = 128 << 20  # include/gdn.h

EXPORTS = ("gdn_chunk_fwd_workspace_bytes", "gdn_chunk_fwd", "gdn_chunk_fwd_prologue_workspace_bytes",
           "gdn_chunk_fwd_prologue", "gdn_chunk_bwd_workspace_bytes",
           "gdn_chunk_bwd", "gdn_fwd_channel_decay", "gdn_recurrent_step", "gdn_status_str", "gdn_chunk_fwd_noalloc")

_lib = None


class GdnError(RuntimeError):
    def __init__(self, status: int):
        self.status = status
        super().__init__(gdn_status_str(status))


def load(path: str | None = None) -> ctypes.CDLL:
    """Load libgdn.so (built by ``python -m linear_attention_sequence_gated_amd.build``)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise ImportError(f"{p} is missing: build it with `python -m linear_attention_sequence_gated_amd.build`")
    lib = ctypes.CDLL(p)
    vp, ci, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    lib.gdn_chunk_fwd_workspace_bytes.argtypes = [ci] * 7
    lib.gdn_chunk_fwd_workspace_bytes.restype = sz
    lib.gdn_chunk_fwd.argtypes = [vp, vp, vp, vp, vp, vp, ci, vp, vp, ci, ci, ci, ci, ci, ci, vp, sz, vp]
    lib.gdn_chunk_fwd.restype = ci
    lib.gdn_chunk_fwd_prologue_workspace_bytes.argtypes = [ci] * 7
    lib.gdn_chunk_fwd_prologue_workspace_bytes.restype = sz
    lib.gdn_chunk_fwd_prologue.argtypes = [vp, vp, vp, vp, vp, ctypes.c_float, vp, ci, vp, vp, ci, ci, ci, ci, ci,
                                           ci, vp, sz, vp]
    lib.gdn_chunk_fwd_prologue.restype = ci
    lib.gdn_chunk_bwd_workspace_bytes.argtypes = [ci] * 6
    lib.gdn_chunk_bwd_workspace_bytes.restype = sz
    lib.gdn_chunk_bwd.argtypes = [vp] * 14 + [ci] * 6 + [vp, sz, vp]
    lib.gdn_chunk_bwd.restype = ci
    lib.gdn_fwd_channel_decay.argtypes = [vp] * 8 + [ci] * 6 + [vp]
    lib.gdn_fwd_channel_decay.restype = ci
    lib.gdn_recurrent_step.argtypes = [vp, vp, vp, vp, vp, vp, vp, ci, ci, ci, ci, vp]
    lib.gdn_recurrent_step.restype = ci
    lib.gdn_chunk_fwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, ci, vp, vp, ci, ci, ci, ci, ci, ci, vp]
    lib.gdn_chunk_fwd_noalloc.restype = ci
    lib.gdn_status_str.argtypes = [ci]
    lib.gdn_status_str.restype = ctypes.c_char_p
    if path is None:
        _lib = lib
    return lib


# ------------------------------------------------------------------ raw C ABI
def gdn_status_str(status: int) -> str:
    return load().gdn_status_str(int(status)).decode()


def gdn_chunk_fwd_workspace_bytes(B, T, H, dk, dv, chunk, dtype) -> int:
    return int(load().gdn_chunk_fwd_workspace_bytes(B, T, H, dk, dv, chunk, dtype))


def gdn_chunk_fwd(q, k, v, alpha, beta, S0, chunk, out, S_final, B, T, H, dk, dv, dtype,
                  workspace, workspace_bytes, stream) -> int:
    return int(load().gdn_chunk_fwd(q, k, v, alpha, beta, S0, chunk, out, S_final, B, T, H, dk, dv, dtype,
                                    workspace, workspace_bytes, stream))


def gdn_chunk_fwd_noalloc(q, k, v, alpha, beta, S0, chunk, out, S_final, B, T, H, dk, dv, dtype, stream) -> int:
    return int(load().gdn_chunk_fwd_noalloc(q, k, v, alpha, beta, S0, chunk, out, S_final, B, T, H, dk, dv, dtype,
                                            stream))


def gdn_chunk_fwd_prologue_workspace_bytes(B, T, H, dk, dv, chunk, dtype) -> int:
    return int(load().gdn_chunk_fwd_prologue_workspace_bytes(B, T, H, dk, dv, chunk, dtype))


def gdn_chunk_fwd_prologue(q, k, v, a_logit, b_logit, beta_scale, S0, chunk, out, S_final, B, T, H, dk, dv,
                           dtype, workspace, workspace_bytes, stream) -> int:
    return int(load().gdn_chunk_fwd_prologue(q, k, v, a_logit, b_logit, float(beta_scale), S0, chunk, out, S_final,
                                             B, T, H, dk, dv, dtype, workspace, workspace_bytes, stream))


def gdn_chunk_bwd_workspace_bytes(B, T, H, dk, dv, dtype) -> int:
    return int(load().gdn_chunk_bwd_workspace_bytes(B, T, H, dk, dv, dtype))


def gdn_chunk_bwd(q, k, v, alpha, beta, S0, grad_out, grad_S_final, grad_q, grad_k, grad_v, grad_alpha, grad_beta,
                  grad_S0, B, T, H, dk, dv, dtype, workspace, workspace_bytes, stream) -> int:
    return int(load().gdn_chunk_bwd(q, k, v, alpha, beta, S0, grad_out, grad_S_final, grad_q, grad_k, grad_v,
                                    grad_alpha, grad_beta, grad_S0, B, T, H, dk, dv, dtype, workspace,
                                    workspace_bytes, stream))


def gdn_fwd_channel_decay(q, k, v, r, beta, S0, out, S_final, B, T, H, dk, dv, dtype, stream) -> int:
    return int(load().gdn_fwd_channel_decay(q, k, v, r, beta, S0, out, S_final, B, T, H, dk, dv, dtype, stream))


def gdn_recurrent_step(q, k, v, alpha, beta, S, out, N, dk, dv, dtype, stream) -> int:
    return int(load().gdn_recurrent_step(q, k, v, alpha, beta, S, out, N, dk, dv, dtype, stream))


# ------------------------------------------------------------- torch helpers
def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return GDN_BF16
    if t.dtype == torch.float32:
        return GDN_F32
    if t.dtype == torch.complex64:
        return GDN_C64
    raise TypeError(f"unsupported dtype {t.dtype}; use bfloat16, float32 or complex64")


def _state_dtype(code: int):
    import torch
    return torch.complex64 if code == GDN_C64 else torch.float32


def _ptr(t):
    return None if t is None else t.data_ptr()


def _check(t, name, shape, dtype, device):
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if t.device != device:
        raise ValueError(f"{name}: expected device {device}, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")


def chunk_fwd(q, k, v, alpha, beta, S0=None, chunk: int = 64, out=None, S_final=None, stream=None):
    """Chunked forward on device tensors.  q, k [B,T,H,dk]; v [B,T,H,dv]; alpha, beta [B,T,H] fp32.

    Returns (out [B,T,H,dv], S_final [B,H,dk,dv]).
    """
    import torch
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    code = _dtype_code(q)
    dev = q.device
    _check(q, "q", (B, T, H, dk), q.dtype, dev)
    if dev.type != "cuda":
        raise ValueError("chunk_fwd: tensors must live on a HIP device")
    _check(k, "k", (B, T, H, dk), q.dtype, dev)
    _check(v, "v", (B, T, H, dv), q.dtype, dev)
    _check(alpha, "alpha", (B, T, H), torch.float32, dev)
    _check(beta, "beta", (B, T, H), torch.float32, dev)
    sdt = _state_dtype(code)
    if S0 is not None:
        _check(S0, "S0", (B, H, dk, dv), sdt, dev)
    if out is None:
        out = torch.empty((B, T, H, dv), dtype=q.dtype, device=dev)
    _check(out, "out", (B, T, H, dv), q.dtype, dev)
    if S_final is None:
        S_final = torch.empty((B, H, dk, dv), dtype=sdt, device=dev)
    _check(S_final, "S_final", (B, H, dk, dv), sdt, dev)
    ws_bytes = gdn_chunk_fwd_workspace_bytes(B, T, H, dk, dv, chunk, code)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev) if ws_bytes else None
    st = stream if stream is not None else torch.cuda.current_stream(dev).cuda_stream
    s = gdn_chunk_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(S0), chunk, _ptr(out),
                      _ptr(S_final), B, T, H, dk, dv, code, _ptr(ws), ws_bytes, st)
    if s != GDN_OK:
        raise GdnError(s)
    return out, S_final


def chunk_fwd_prologue(q, k, v, a_logit, b_logit, beta_scale: float = 1.0, S0=None, chunk: int = 64, out=None,
                       S_final=None, stream=None):
    """Chunked forward from raw projections: q and k are L2-normalised per row, alpha = exp(-softplus(a_logit))
    and beta = beta_scale * sigmoid(b_logit), all on the device.  q, k, v [B,T,H,d] in any supported dtype
    (bfloat16 d 64 or 128, float32 d 64, complex64 d 32); a_logit, b_logit [B,T,H] float32.  The workspace is
    allocated here with torch.  Returns (out [B,T,H,d], S_final [B,H,d,d], float32 or complex64).
    """
    import torch
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    code = _dtype_code(q)
    dev = q.device
    _check(q, "q", (B, T, H, dk), q.dtype, dev)
    if dev.type != "cuda":
        raise ValueError("chunk_fwd_prologue: tensors must live on a HIP device")
    _check(k, "k", (B, T, H, dk), q.dtype, dev)
    _check(v, "v", (B, T, H, dv), q.dtype, dev)
    _check(a_logit, "a_logit", (B, T, H), torch.float32, dev)
    _check(b_logit, "b_logit", (B, T, H), torch.float32, dev)
    sdt = _state_dtype(code)
    if S0 is not None:
        _check(S0, "S0", (B, H, dk, dv), sdt, dev)
    if out is None:
        out = torch.empty((B, T, H, dv), dtype=q.dtype, device=dev)
    _check(out, "out", (B, T, H, dv), q.dtype, dev)
    if S_final is None:
        S_final = torch.empty((B, H, dk, dv), dtype=sdt, device=dev)
    _check(S_final, "S_final", (B, H, dk, dv), sdt, dev)
    ws_bytes = gdn_chunk_fwd_prologue_workspace_bytes(B, T, H, dk, dv, chunk, code)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev) if ws_bytes else None
    st = stream if stream is not None else torch.cuda.current_stream(dev).cuda_stream
    s = gdn_chunk_fwd_prologue(_ptr(q), _ptr(k), _ptr(v), _ptr(a_logit), _ptr(b_logit), beta_scale, _ptr(S0), chunk,
                               _ptr(out), _ptr(S_final), B, T, H, dk, dv, code, _ptr(ws), ws_bytes, st)
    if s != GDN_OK:
        raise GdnError(s)
    return out, S_final


def chunk_bwd(q, k, v, alpha, beta, grad_out, S0=None, grad_S_final=None, stream=None):
    """Gradients of sum(out * grad_out) + sum(S_final * grad_S_final) for chunk_fwd's forward (for complex data
    Re sum(conj(grad_out) out) + Re sum(conj(grad_S_final) S_final), gradients dL/dRe + i dL/dIm).

    q, k, v, grad_out [B,T,H,d]: float32 (d 64), bfloat16 (d 64 or 128) or complex64 (d 32), one dtype;
    alpha, beta [B,T,H] float32; S0 and grad_S_final [B,H,d,d] float32 (complex64 for complex data) or None.
    Returns (grad_q, grad_k, grad_v, grad_alpha, grad_beta, grad_S0): float32, complex64 for the complex
    ones of complex data.  The workspace is allocated here with torch.
    """
    import torch
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    code = _dtype_code(q)
    dev = q.device
    _check(q, "q", (B, T, H, dk), q.dtype, dev)
    if dev.type != "cuda":
        raise ValueError("chunk_bwd: tensors must live on a HIP device")
    for t, name, shp in ((k, "k", (B, T, H, dk)), (v, "v", (B, T, H, dv)),
                         (grad_out, "grad_out", (B, T, H, dv))):
        _check(t, name, shp, q.dtype, dev)
    _check(alpha, "alpha", (B, T, H), torch.float32, dev)
    _check(beta, "beta", (B, T, H), torch.float32, dev)
    gdt = _state_dtype(code)
    if S0 is not None:
        _check(S0, "S0", (B, H, dk, dv), gdt, dev)
    if grad_S_final is not None:
        _check(grad_S_final, "grad_S_final", (B, H, dk, dv), gdt, dev)
    g = dict(dtype=gdt, device=dev)
    gq, gk, gv = torch.empty((B, T, H, dk), **g), torch.empty((B, T, H, dk), **g), torch.empty((B, T, H, dv), **g)
    f32 = dict(dtype=torch.float32, device=dev)
    ga, gb = torch.empty((B, T, H), **f32), torch.empty((B, T, H), **f32)
    gS0 = torch.empty((B, H, dk, dv), **g)
    ws_bytes = gdn_chunk_bwd_workspace_bytes(B, T, H, dk, dv, code)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    st = stream if stream is not None else torch.cuda.current_stream(dev).cuda_stream
    s = gdn_chunk_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(S0), _ptr(grad_out),
                      _ptr(grad_S_final), _ptr(gq), _ptr(gk), _ptr(gv), _ptr(ga), _ptr(gb), _ptr(gS0), B, T, H, dk, dv,
                      code, ws.data_ptr() if ws_bytes else None, ws_bytes, st)
    if s != GDN_OK:
        raise GdnError(s)
    return gq, gk, gv, ga, gb, gS0


def fwd_channel_decay(q, k, v, r, beta, S0=None, out=None, S_final=None, stream=None):
    """Forward with a per-output-channel decay r [B,T,H,d] fp32 (one factor per token and value channel).
    q, k, v [B,T,H,d]: float32 or bfloat16 with d = 64, or complex64 with d = 32; beta [B,T,H] fp32;
    S0 [B,H,d,d] (fp32, complex64 for complex data) or None.
    Returns (out [B,T,H,d] in q's dtype, S_final [B,H,d,d] in the state's dtype)."""
    import torch
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    code = _dtype_code(q)
    dev = q.device
    _check(q, "q", (B, T, H, dk), q.dtype, dev)
    if dev.type != "cuda":
        raise ValueError("fwd_channel_decay: tensors must live on a HIP device")
    _check(k, "k", (B, T, H, dk), q.dtype, dev)
    _check(v, "v", (B, T, H, dv), q.dtype, dev)
    _check(r, "r", (B, T, H, dv), torch.float32, dev)
    _check(beta, "beta", (B, T, H), torch.float32, dev)
    sdt = _state_dtype(code)
    if S0 is not None:
        _check(S0, "S0", (B, H, dk, dv), sdt, dev)
    if out is None:
        out = torch.empty((B, T, H, dv), dtype=q.dtype, device=dev)
    _check(out, "out", (B, T, H, dv), q.dtype, dev)
    if S_final is None:
        S_final = torch.empty((B, H, dk, dv), dtype=sdt, device=dev)
    _check(S_final, "S_final", (B, H, dk, dv), sdt, dev)
    st = stream if stream is not None else torch.cuda.current_stream(dev).cuda_stream
    s = gdn_fwd_channel_decay(_ptr(q), _ptr(k), _ptr(v), _ptr(r), _ptr(beta), _ptr(S0), _ptr(out), _ptr(S_final),
                              B, T, H, dk, dv, code, st)
    if s != GDN_OK:
        raise GdnError(s)
    return out, S_final


def recurrent_step(q, k, v, alpha, beta, S, out=None, stream=None):
    """One decode step, in place on S [N,dk,dv].  q, k [N,dk]; v [N,dv]; alpha, beta [N].  Returns out [N,dv]."""
    import torch
    N, dk = q.shape
    dv = v.shape[-1]
    code = _dtype_code(q)
    dev = q.device
    _check(q, "q", (N, dk), q.dtype, dev)
    if dev.type != "cuda":
        raise ValueError("recurrent_step: tensors must live on a HIP device")
    _check(k, "k", (N, dk), q.dtype, dev)
    _check(v, "v", (N, dv), q.dtype, dev)
    _check(alpha, "alpha", (N,), torch.float32, dev)
    _check(beta, "beta", (N,), torch.float32, dev)
    _check(S, "S", (N, dk, dv), _state_dtype(code), dev)
    if out is None:
        out = torch.empty((N, dv), dtype=q.dtype, device=dev)
    _check(out, "out", (N, dv), q.dtype, dev)
    st = stream if stream is not None else torch.cuda.current_stream(dev).cuda_stream
    s = gdn_recurrent_step(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(S), _ptr(out), N, dk, dv,
                           code, st)
    if s != GDN_OK:
        raise GdnError(s)
    return out
