"""Gated DeltaNet token mixer for AMD MI355X (gfx950): Python binding of libgdn.so.

The library (``libgdn.so``, built from ``csrc/`` by ``build.py``) exports the C ABI
declared in ``include/gdn.h``.  This module only marshals arguments: it takes
torch tensors that already live on the GPU, checks their dtype / shape /
contiguity, allocates outputs and workspace with torch, and passes raw device
pointers and the current HIP stream to the library.  Every step of the
computation runs in the library's HIP kernels; there is no fallback.

    q, k, v = conv_qk_prep(x, conv_w, Hk, Hv, dk, dv, cu_seqlens, conv_state_in, conv_state_out)
    o, final_state = chunk_prefill(q, k, v, g, beta, cu_seqlens, initial_state)
    o, final_state = prefill(x, conv_w, g, beta, Hk, Hv, dk, dv, cu_seqlens, ...)   # both in one call
    o = decode_step(x, conv_w, conv_state, g, beta, state, Hk, Hv, dk, dv)
    out, final_state = layer_prefill(hidden, w_in, conv_w, gamma, w_out, Hk, Hv, dk, dv, ...)
    out = layer_decode(hidden, w_in, conv_w, gamma, w_out, conv_state, state, Hk, Hv, dk, dv)
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = ["conv_qk_prep", "chunk_prefill", "prefill", "prefill_local", "gated_rmsnorm", "decode_step_gated", "chunk_prefill_local", "chunk_prefill_state", "decode_step", "workspace_size", "lib", "GdnError",
           "GDN_F32", "GDN_BF16", "GDN_MATH_F32", "GDN_MATH_MFMA", "GDN_MATH_F32_CHUNKED", "GDN_ORDER_DECAY_FIRST", "GDN_ORDER_RETRIEVE_FIRST",
           "LIB_PATH", "abi_version", "mfma_supported", "linear", "in_proj", "layer_prefill", "layer_decode",
           "layer_prefill_workspace_size", "layer_decode_workspace_size", "prefill_workspace_status",
           "GDN_OK", "GDN_ERR_TIMEOUT", "GDN_ERR_NONFINITE", "set_wait_bound", "layer_decode_noalloc"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libgdn.so")
GDN_F32, GDN_BF16 = 0, 1
GDN_MATH_F32, GDN_MATH_MFMA, GDN_MATH_F32_CHUNKED = 0, 1, 2
GDN_ORDER_DECAY_FIRST, GDN_ORDER_RETRIEVE_FIRST = 0, 1
GDN_OK, GDN_ERR_TIMEOUT, GDN_ERR_NONFINITE = 0, 8, 9
_SPIN_TAG = 0x7370696E   # high half of the workspace header word that bounds the state pass's waits
_lib = None


class GdnError(RuntimeError):
    def __init__(self, fn: str, status: int):
        msg = lib().gdn_status_string(status).decode()
        super().__init__(f"{fn} failed with status {status}: {msg}")
        self.status = status


def lib() -> ctypes.CDLL:
    """Load libgdn.so; raises ImportError when it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m hybrid_linear_attention_gated_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P, I, F, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
        L.gdn_conv_qk_prep.argtypes = [P, P, P, I, P, P, P, P, P, I, I, I, I, I, I, F, P]
        L.gdn_conv_qk_prep.restype = I
        L.gdn_chunk_prefill_workspace_size.argtypes = [I, I, I, I, I, I, I]
        L.gdn_chunk_prefill_workspace_size.restype = Z
        L.gdn_chunk_prefill.argtypes = [P, P, P, P, P, P, I, P, P, P, F, I, I, I, I, I, I, I, P, Z, P]
        L.gdn_chunk_prefill.restype = I
        L.gdn_chunk_prefill_local.argtypes = [P, P, P, P, P, P, I, F, I, I, I, I, I, I, P, Z, P]
        L.gdn_chunk_prefill_local.restype = I
        L.gdn_chunk_prefill_state.argtypes = [P, I, P, P, P, I, I, I, I, I, P, Z, P]
        L.gdn_chunk_prefill_state.restype = I
        L.gdn_prefill.argtypes = [P, P, P, I, P, P, P, P, P, P, P, F, F, I, I, I, I, I, I, I, P, Z, P]
        L.gdn_prefill.restype = I
        L.gdn_prefill_local.argtypes = [P, P, P, I, P, P, P, P, F, F, I, I, I, I, I, I, I, P, Z, P]
        L.gdn_prefill_local.restype = I
        L.gdn_decode_step_gated.argtypes = [P, P, P, P, P, P, P, P, P, F, F, F, I, I, I, I, I, I, I, P]
        L.gdn_decode_step_gated.restype = I
        L.gdn_gated_rmsnorm.argtypes = [P, P, P, P, ctypes.c_long, I, F, I, P]
        L.gdn_gated_rmsnorm.restype = I
        L.gdn_decode_step.argtypes = [P, P, P, P, P, P, P, F, F, I, I, I, I, I, I, I, P]
        L.gdn_decode_step.restype = I
        L.gdn_linear.argtypes = [P, P, P, I, I, I, P]
        L.gdn_linear.restype = I
        L.gdn_in_proj.argtypes = [P, P, P, P, P, P, I, I, I, I, I, I, P]
        L.gdn_in_proj.restype = I
        L.gdn_layer_prefill_workspace_size.argtypes = [I, I, I, I, I, I]
        L.gdn_layer_prefill_workspace_size.restype = Z
        L.gdn_layer_prefill.argtypes = [P, P, P, P, P, P, I, P, P, P, P, P, F, F, F, I, I, I, I, I, I, I, P, Z, P]
        L.gdn_layer_prefill.restype = I
        L.gdn_layer_decode_workspace_size.argtypes = [I, I, I, I, I, I]
        L.gdn_layer_decode_workspace_size.restype = Z
        L.gdn_layer_decode.argtypes = [P, P, P, P, P, P, P, P, F, F, F, I, I, I, I, I, I, I, P, Z, P]
        L.gdn_layer_decode.restype = I
        L.gdn_layer_decode_noalloc.argtypes = [P, P, P, P, P, P, P, P, F, F, F, I, I, I, I, I, I, I, P]
        L.gdn_layer_decode_noalloc.restype = I
        L.gdn_prefill_workspace_status.argtypes = [P, Z, P]
        L.gdn_prefill_workspace_status.restype = I
        L.gdn_status_string.argtypes = [I]
        L.gdn_status_string.restype = ctypes.c_char_p
        L.gdn_abi_version.argtypes = []
        L.gdn_abi_version.restype = I
        _lib = L
    return _lib


def abi_version() -> int:
    return lib().gdn_abi_version()


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return GDN_BF16
    if t.dtype == torch.float32:
        return GDN_F32
    raise TypeError(f"unsupported element dtype {t.dtype}")


def _check(t, name, dtype=None, shape=None, optional=False):
    if t is None:
        if optional:
            return None
        raise ValueError(f"{name} is required")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return t


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _seqs(cu_seqlens, T):
    if cu_seqlens is None:
        return None, 1
    _check(cu_seqlens, "cu_seqlens", torch.int32)
    return cu_seqlens, cu_seqlens.numel() - 1


def conv_qk_prep(x, conv_w, Hk, Hv, dk, dv, cu_seqlens=None, conv_state_in=None, conv_state_out=None,
                 l2_eps=1e-6, q=None, k=None, v=None):
    """Depthwise causal conv (kernel 4) + SiLU + split + L2(q, k).

    x [T, conv_dim], conv_w [conv_dim, 4]; conv states [N, 3, conv_dim].
    Returns fp32 q, k [T, Hk, dk] and v [T, Hv, dv].
    """
    dt = x.dtype
    C = 2 * Hk * dk + Hv * dv
    _check(x, "x", dt)
    if x.dim() != 2 or x.shape[1] != C:
        raise ValueError(f"x must be [T, {C}], got {tuple(x.shape)}")
    T = x.shape[0]
    cu, N = _seqs(cu_seqlens, T)
    _check(conv_w, "conv_w", dt, (C, 4))
    _check(conv_state_in, "conv_state_in", dt, (N, 3, C), optional=True)
    _check(conv_state_out, "conv_state_out", dt, (N, 3, C), optional=True)
    f32 = torch.float32
    q = torch.empty((T, Hk, dk), dtype=f32, device=x.device) if q is None else _check(q, "q", f32, (T, Hk, dk))
    k = torch.empty((T, Hk, dk), dtype=f32, device=x.device) if k is None else _check(k, "k", f32, (T, Hk, dk))
    v = torch.empty((T, Hv, dv), dtype=f32, device=x.device) if v is None else _check(v, "v", f32, (T, Hv, dv))
    st = lib().gdn_conv_qk_prep(_p(x), _p(conv_w), _p(cu), N, _p(conv_state_in), _p(conv_state_out),
                                _p(q), _p(k), _p(v), T, Hk, Hv, dk, dv, _dt(x), float(l2_eps), _stream())
    if st != 0:
        raise GdnError("gdn_conv_qk_prep", st)
    return q, k, v


def prefill(x, conv_w, g, beta, Hk, Hv, dk, dv, cu_seqlens=None, conv_state_in=None, conv_state_out=None,
            initial_state=None, final_state=None, scale=1.0, l2_eps=1e-6, output_final_state=True, o=None,
            workspace=None, order=0):
    """conv_qk_prep + chunk_prefill (MFMA path) in one call, q / k / v never written out.

    x [T, conv_dim] (bf16 or fp32), conv_w [conv_dim, 4]; g, beta [T, Hv] fp32; states
    [N, Hv, dk, dv] fp32; conv states [N, 3, conv_dim].  Returns o [T, Hv, dv] fp32 and
    the final state (None when output_final_state is False and none is given).
    """
    dt = x.dtype
    C = 2 * Hk * dk + Hv * dv
    _check(x, "x", dt)
    if x.dim() != 2 or x.shape[1] != C:
        raise ValueError(f"x must be [T, {C}], got {tuple(x.shape)}")
    T = x.shape[0]
    cu, N = _seqs(cu_seqlens, T)
    f32 = torch.float32
    _check(conv_w, "conv_w", dt, (C, 4))
    _check(conv_state_in, "conv_state_in", dt, (N, 3, C), optional=True)
    _check(conv_state_out, "conv_state_out", dt, (N, 3, C), optional=True)
    _check(g, "g", f32, (T, Hv))
    _check(beta, "beta", f32, (T, Hv))
    _check(initial_state, "initial_state", f32, (N, Hv, dk, dv), optional=True)
    if final_state is None and output_final_state:
        final_state = torch.empty((N, Hv, dk, dv), dtype=f32, device=x.device)
    _check(final_state, "final_state", f32, (N, Hv, dk, dv), optional=True)
    o = torch.empty((T, Hv, dv), dtype=f32, device=x.device) if o is None else _check(o, "o", f32, (T, Hv, dv))
    need = workspace_size(T, N, Hk, Hv, dk, dv, "mfma")
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    _check(workspace, "workspace")
    st = lib().gdn_prefill(_p(x), _p(conv_w), _p(cu), N, _p(conv_state_in), _p(conv_state_out), _p(g), _p(beta),
                           _p(initial_state), _p(final_state), _p(o), float(scale), float(l2_eps), T, Hk, Hv, dk, dv,
                           _dt(x), int(order), _p(workspace), workspace.numel() * workspace.element_size(), _stream())
    if st != 0:
        raise GdnError("gdn_prefill", st)
    return o, final_state


def prefill_local(x, conv_w, g, beta, workspace, Hk, Hv, dk, dv, cu_seqlens=None, conv_state_in=None,
                  conv_state_out=None, scale=1.0, l2_eps=1e-6, order=0):
    """First phase of `prefill` (conv prep + chunk-local records into `workspace`);
    `chunk_prefill_state` finishes it."""
    dt = x.dtype
    C = 2 * Hk * dk + Hv * dv
    _check(x, "x", dt)
    if x.dim() != 2 or x.shape[1] != C:
        raise ValueError(f"x must be [T, {C}], got {tuple(x.shape)}")
    T = x.shape[0]
    cu, N = _seqs(cu_seqlens, T)
    _check(conv_w, "conv_w", dt, (C, 4))
    _check(conv_state_in, "conv_state_in", dt, (N, 3, C), optional=True)
    _check(conv_state_out, "conv_state_out", dt, (N, 3, C), optional=True)
    _check(g, "g", torch.float32, (T, Hv))
    _check(beta, "beta", torch.float32, (T, Hv))
    _check(workspace, "workspace")
    st = lib().gdn_prefill_local(_p(x), _p(conv_w), _p(cu), N, _p(conv_state_in), _p(conv_state_out), _p(g),
                                 _p(beta), float(scale), float(l2_eps), T, Hk, Hv, dk, dv, _dt(x), int(order),
                                 _p(workspace),
                                 workspace.numel() * workspace.element_size(), _stream())
    if st != 0:
        raise GdnError("gdn_prefill_local", st)


def prefill_workspace_status(workspace) -> int:
    """Status of the chunked prefills that used `workspace` since the last query (GDN_OK,
    GDN_ERR_TIMEOUT or GDN_ERR_NONFINITE); waits for their completion and clears it."""
    _check(workspace, "workspace")
    st = lib().gdn_prefill_workspace_status(_p(workspace), workspace.numel() * workspace.element_size(), _stream())
    if st not in (GDN_OK, GDN_ERR_TIMEOUT, GDN_ERR_NONFINITE):
        raise GdnError("gdn_prefill_workspace_status", st)
    return st


def set_wait_bound(workspace, iterations=None):
    """Write the workspace header word that bounds the concurrent state pass's waits for a
    record or a row sum (`iterations` of a ~128-cycle sleep), or restore the default (None).
    A prefill workspace or a layer prefill workspace (which starts with its prefill's).  For
    tests of the timeout path."""
    _check(workspace, "workspace", torch.uint8)
    word = 0 if iterations is None else (_SPIN_TAG << 32) | int(iterations)
    workspace[8:16].copy_(torch.tensor([word], dtype=torch.int64).view(torch.uint8))


def mfma_supported(dk, dv) -> bool:
    return dk == dv and dk in (64, 128)


def _math(math, dk, dv) -> int:
    if math == "auto":
        return GDN_MATH_MFMA if mfma_supported(dk, dv) else GDN_MATH_F32
    return {"f32": GDN_MATH_F32, "mfma": GDN_MATH_MFMA, "f32_chunked": GDN_MATH_F32_CHUNKED}[math]


def workspace_size(T, N, Hk, Hv, dk, dv, math="auto") -> int:
    return int(lib().gdn_chunk_prefill_workspace_size(T, N, Hk, Hv, dk, dv, _math(math, dk, dv)))


def chunk_prefill(q, k, v, g, beta, cu_seqlens=None, initial_state=None, final_state=None, scale=1.0,
                  output_final_state=True, o=None, workspace=None, math="auto", order=0):
    """Gated delta rule over packed sequences.

    q, k [T, Hk, dk]; v [T, Hv, dv]; g, beta [T, Hv]; states [N, Hv, dk, dv]; all fp32.
    math: "mfma" (chunked MFMA path), "f32" (fp32 token recurrence), "f32_chunked" (the
    chunked form in fp32, head dims 16..64) or "auto" (mfma where the head dims allow it,
    else f32).  order: 0 decays the state before the
    retrieval, 1 retrieves from the undecayed state (GDN_ORDER_*).
    Returns (o [T, Hv, dv] fp32, final_state or None).  final_state may be initial_state
    (updated in place).
    """
    dt = torch.float32
    _check(q, "q", dt)
    T, Hk, dk = q.shape
    _check(k, "k", dt, (T, Hk, dk))
    _check(v, "v", dt)
    if v.dim() != 3 or v.shape[0] != T:
        raise ValueError("v must be [T, Hv, dv]")
    Hv, dv = v.shape[1], v.shape[2]
    _check(g, "g", torch.float32, (T, Hv))
    _check(beta, "beta", torch.float32, (T, Hv))
    cu, N = _seqs(cu_seqlens, T)
    _check(initial_state, "initial_state", torch.float32, (N, Hv, dk, dv), optional=True)
    if final_state is None and output_final_state:
        final_state = torch.empty((N, Hv, dk, dv), dtype=torch.float32, device=q.device)
    _check(final_state, "final_state", torch.float32, (N, Hv, dk, dv), optional=True)
    o = torch.empty((T, Hv, dv), dtype=torch.float32, device=q.device) if o is None else \
        _check(o, "o", torch.float32, (T, Hv, dv))
    m = _math(math, dk, dv)
    need = workspace_size(T, N, Hk, Hv, dk, dv, math)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().gdn_chunk_prefill(_p(q), _p(k), _p(v), _p(g), _p(beta), _p(cu), N, _p(initial_state),
                                 _p(final_state), _p(o), float(scale), T, Hk, Hv, dk, dv, m, int(order),
                                 _p(workspace), ws_bytes, _stream())
    if st != 0:
        raise GdnError("gdn_chunk_prefill", st)
    return o, final_state


def chunk_prefill_local(q, k, v, g, beta, workspace, cu_seqlens=None, scale=1.0, order=0):
    """First phase of the MFMA chunked prefill: per-chunk quantities into `workspace`."""
    T, Hk, dk = q.shape
    Hv, dv = v.shape[1], v.shape[2]
    cu, N = _seqs(cu_seqlens, T)
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (g, "g"), (beta, "beta")):
        _check(t, n, torch.float32)
    _check(workspace, "workspace")
    st = lib().gdn_chunk_prefill_local(_p(q), _p(k), _p(v), _p(g), _p(beta), _p(cu), N, float(scale), T, Hk, Hv,
                                       dk, dv, int(order), _p(workspace), workspace.numel() * workspace.element_size(),
                                       _stream())
    if st != 0:
        raise GdnError("gdn_chunk_prefill_local", st)


def chunk_prefill_state(workspace, o, T, Hk, Hv, dk, dv, cu_seqlens=None, initial_state=None, final_state=None):
    """Second phase of the MFMA chunked prefill: the state pass over chunks."""
    cu, N = _seqs(cu_seqlens, T)
    _check(o, "o", torch.float32, (T, Hv, dv))
    _check(workspace, "workspace")
    _check(initial_state, "initial_state", torch.float32, (N, Hv, dk, dv), optional=True)
    _check(final_state, "final_state", torch.float32, (N, Hv, dk, dv), optional=True)
    st = lib().gdn_chunk_prefill_state(_p(cu), N, _p(initial_state), _p(final_state), _p(o), T, Hk, Hv, dk, dv,
                                       _p(workspace), workspace.numel() * workspace.element_size(), _stream())
    if st != 0:
        raise GdnError("gdn_chunk_prefill_state", st)


def decode_step(x, conv_w, conv_state, g, beta, state, Hk, Hv, dk, dv, scale=1.0, l2_eps=1e-6, o=None, order=0):
    """One decode token per row; conv_state [B, 3, conv_dim] and state [B, Hv, dk, dv]
    are updated in place.  Returns o [B, Hv, dv] fp32."""
    dt = x.dtype
    C = 2 * Hk * dk + Hv * dv
    _check(x, "x", dt)
    if x.dim() != 2 or x.shape[1] != C:
        raise ValueError(f"x must be [B, {C}]")
    B = x.shape[0]
    _check(conv_w, "conv_w", dt, (C, 4))
    _check(conv_state, "conv_state", dt, (B, 3, C))
    _check(g, "g", torch.float32, (B, Hv))
    _check(beta, "beta", torch.float32, (B, Hv))
    _check(state, "state", torch.float32, (B, Hv, dk, dv))
    o = torch.empty((B, Hv, dv), dtype=torch.float32, device=x.device) if o is None else \
        _check(o, "o", torch.float32, (B, Hv, dv))
    st = lib().gdn_decode_step(_p(x), _p(conv_w), _p(conv_state), _p(g), _p(beta), _p(state), _p(o),
                               float(scale), float(l2_eps), B, Hk, Hv, dk, dv, _dt(x), int(order), _stream())
    if st != 0:
        raise GdnError("gdn_decode_step", st)
    return o


def decode_step_gated(x, conv_w, conv_state, g, beta, state, z, gamma, Hk, Hv, dk, dv, scale=1.0, l2_eps=1e-6,
                      norm_eps=1e-6, out=None, order=0):
    """decode_step with the gated RMSNorm fused: returns out [B, Hv, dv] in x's dtype,
    RMSNorm(o) * gamma * SiLU(z) per head (z [B, Hv, dv] and gamma [dv] in x's dtype)."""
    dt = x.dtype
    C = 2 * Hk * dk + Hv * dv
    _check(x, "x", dt)
    if x.dim() != 2 or x.shape[1] != C:
        raise ValueError(f"x must be [B, {C}]")
    B = x.shape[0]
    _check(conv_w, "conv_w", dt, (C, 4))
    _check(conv_state, "conv_state", dt, (B, 3, C))
    _check(g, "g", torch.float32, (B, Hv))
    _check(beta, "beta", torch.float32, (B, Hv))
    _check(state, "state", torch.float32, (B, Hv, dk, dv))
    _check(z, "z", dt, (B, Hv, dv))
    _check(gamma, "gamma", dt, (dv,))
    out = torch.empty((B, Hv, dv), dtype=dt, device=x.device) if out is None else _check(out, "out", dt, (B, Hv, dv))
    st = lib().gdn_decode_step_gated(_p(x), _p(conv_w), _p(conv_state), _p(g), _p(beta), _p(state), _p(z),
                                     _p(gamma), _p(out), float(scale), float(l2_eps), float(norm_eps), B, Hk, Hv,
                                     dk, dv, _dt(x), int(order), _stream())
    if st != 0:
        raise GdnError("gdn_decode_step_gated", st)
    return out


def gated_rmsnorm(y, z, gamma, eps=1e-6, out=None):
    """Gated RMSNorm over the last axis of y (fp32, [..., dv]): y / sqrt(mean y^2 + eps) *
    gamma * SiLU(z), returned in z's dtype (z same shape as y, gamma [dv])."""
    _check(y, "y", torch.float32)
    dt = z.dtype
    dv = y.shape[-1]
    _check(z, "z", dt, tuple(y.shape))
    _check(gamma, "gamma", dt, (dv,))
    out = torch.empty(y.shape, dtype=dt, device=y.device) if out is None else _check(out, "out", dt, tuple(y.shape))
    rows = y.numel() // dv if dv else 0
    st = lib().gdn_gated_rmsnorm(_p(y), _p(z), _p(gamma), _p(out), rows, dv, float(eps), _dt(z), _stream())
    if st != 0:
        raise GdnError("gdn_gated_rmsnorm", st)
    return out


# ------------------------------------------------------------------ layer forward

def linear(a, w, y=None):
    """y = a w^T on bf16 MFMA: a [M, K], w [N, K] bf16 (K % 64 == 0, N % 4 == 0);
    returns y [M, N] bf16."""
    bf = torch.bfloat16
    _check(a, "a", bf)
    _check(w, "w", bf)
    if a.dim() != 2 or w.dim() != 2 or a.shape[1] != w.shape[1]:
        raise ValueError(f"a [M, K] and w [N, K] expected, got {tuple(a.shape)} and {tuple(w.shape)}")
    M, K = a.shape
    N = w.shape[0]
    y = torch.empty((M, N), dtype=bf, device=a.device) if y is None else _check(y, "y", bf, (M, N))
    st = lib().gdn_linear(_p(a), _p(w), _p(y), M, N, K, _stream())
    if st != 0:
        raise GdnError("gdn_linear", st)
    return y


def _layer_weights(w_in, conv_w, gamma, w_out, E, Hk, Hv, dk, dv):
    bf = torch.bfloat16
    C = 2 * Hk * dk + Hv * dv
    _check(w_in, "w_in", bf, (C + Hv * dv + 2 * Hv, E))
    if conv_w is not None:
        _check(conv_w, "conv_w", bf, (C, 4))
    if gamma is not None:
        _check(gamma, "gamma", bf, (dv,))
    if w_out is not None:
        _check(w_out, "w_out", bf, (E, Hv * dv))
    return C


def in_proj(hidden, w_in, Hk, Hv, dk, dv, x=None, z=None, g=None, beta=None):
    """The layer's input projection: hidden [T, E] bf16, w_in [conv_dim + Hv dv + 2 Hv, E]
    bf16 (rows q|k|v, z, a, b).  Returns x [T, conv_dim] bf16, z [T, Hv dv] bf16,
    g = -softplus(a) and beta = sigmoid(b) [T, Hv] fp32 (written into the given tensors
    when passed)."""
    _check(hidden, "hidden", torch.bfloat16)
    T, E = hidden.shape
    C = _layer_weights(w_in, None, None, None, E, Hk, Hv, dk, dv)
    dev = hidden.device
    bf, f32 = torch.bfloat16, torch.float32
    x = torch.empty((T, C), dtype=bf, device=dev) if x is None else _check(x, "x", bf, (T, C))
    z = torch.empty((T, Hv * dv), dtype=bf, device=dev) if z is None else _check(z, "z", bf, (T, Hv * dv))
    g = torch.empty((T, Hv), dtype=f32, device=dev) if g is None else _check(g, "g", f32, (T, Hv))
    beta = torch.empty((T, Hv), dtype=f32, device=dev) if beta is None else _check(beta, "beta", f32, (T, Hv))
    st = lib().gdn_in_proj(_p(hidden), _p(w_in), _p(x), _p(z), _p(g), _p(beta), T, E, Hk, Hv, dk, dv, _stream())
    if st != 0:
        raise GdnError("gdn_in_proj", st)
    return x, z, g, beta


def layer_prefill_workspace_size(T, N, Hk, Hv, dk, dv) -> int:
    return int(lib().gdn_layer_prefill_workspace_size(T, N, Hk, Hv, dk, dv))


def layer_decode_workspace_size(B, E, Hk, Hv, dk, dv) -> int:
    return int(lib().gdn_layer_decode_workspace_size(B, E, Hk, Hv, dk, dv))


def layer_prefill(hidden, w_in, conv_w, gamma, w_out, Hk, Hv, dk, dv, cu_seqlens=None, conv_state_in=None,
                  conv_state_out=None, initial_state=None, final_state=None, scale=1.0, l2_eps=1e-6,
                  norm_eps=1e-6, output_final_state=True, out=None, workspace=None, order=0):
    """The linear-attention layer over packed sequences: hidden [T, E] bf16 -> out [T, E]
    bf16 (input projection, conv + SiLU + L2, gated delta rule, gated RMSNorm, output
    projection).  Weights bf16: w_in [conv_dim + Hv dv + 2 Hv, E], conv_w [conv_dim, 4],
    gamma [dv], w_out [E, Hv dv].  Conv caches [N, 3, conv_dim] fp32 (the layer keeps its
    pre-conv inputs in fp32), states as in `prefill`.  Returns (out, final_state)."""
    bf, f32 = torch.bfloat16, torch.float32
    _check(hidden, "hidden", bf)
    if hidden.dim() != 2:
        raise ValueError("hidden must be [T, E]")
    T, E = hidden.shape
    C = _layer_weights(w_in, conv_w, gamma, w_out, E, Hk, Hv, dk, dv)
    cu, N = _seqs(cu_seqlens, T)
    _check(conv_state_in, "conv_state_in", f32, (N, 3, C), optional=True)
    _check(conv_state_out, "conv_state_out", f32, (N, 3, C), optional=True)
    _check(initial_state, "initial_state", f32, (N, Hv, dk, dv), optional=True)
    if final_state is None and output_final_state:
        final_state = torch.empty((N, Hv, dk, dv), dtype=f32, device=hidden.device)
    _check(final_state, "final_state", f32, (N, Hv, dk, dv), optional=True)
    out = torch.empty((T, E), dtype=bf, device=hidden.device) if out is None else _check(out, "out", bf, (T, E))
    need = layer_prefill_workspace_size(T, N, Hk, Hv, dk, dv)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=hidden.device)
    _check(workspace, "workspace")
    st = lib().gdn_layer_prefill(_p(hidden), _p(w_in), _p(conv_w), _p(gamma), _p(w_out), _p(cu), N,
                                 _p(conv_state_in), _p(conv_state_out), _p(initial_state), _p(final_state), _p(out),
                                 float(scale), float(l2_eps), float(norm_eps), T, E, Hk, Hv, dk, dv, int(order),
                                 _p(workspace), workspace.numel() * workspace.element_size(), _stream())
    if st != 0:
        raise GdnError("gdn_layer_prefill", st)
    return out, final_state


def layer_decode(hidden, w_in, conv_w, gamma, w_out, conv_state, state, Hk, Hv, dk, dv, scale=1.0, l2_eps=1e-6,
                 norm_eps=1e-6, out=None, workspace=None, order=0):
    """One token per sequence through the layer: hidden [B, E] bf16 -> out [B, E] bf16;
    conv_state [B, 3, conv_dim] fp32 and state [B, Hv, dk, dv] fp32 are updated in place."""
    bf = torch.bfloat16
    _check(hidden, "hidden", bf)
    if hidden.dim() != 2:
        raise ValueError("hidden must be [B, E]")
    B, E = hidden.shape
    C = _layer_weights(w_in, conv_w, gamma, w_out, E, Hk, Hv, dk, dv)
    _check(conv_state, "conv_state", torch.float32, (B, 3, C))
    _check(state, "state", torch.float32, (B, Hv, dk, dv))
    out = torch.empty((B, E), dtype=bf, device=hidden.device) if out is None else _check(out, "out", bf, (B, E))
    need = layer_decode_workspace_size(B, E, Hk, Hv, dk, dv)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=hidden.device)
    _check(workspace, "workspace")
    st = lib().gdn_layer_decode(_p(hidden), _p(w_in), _p(conv_w), _p(gamma), _p(w_out), _p(conv_state), _p(state),
                                _p(out), float(scale), float(l2_eps), float(norm_eps), B, E, Hk, Hv, dk, dv,
                                int(order), _p(workspace), workspace.numel() * workspace.element_size(), _stream())
    if st != 0:
        raise GdnError("gdn_layer_decode", st)
    return out


def layer_decode_noalloc(hidden, w_in, conv_w, gamma, w_out, conv_state, state, Hk, Hv, dk, dv, out, scale=1.0,
                         l2_eps=1e-6, norm_eps=1e-6, order=0):
    """`layer_decode` through the allocation-free entry point: the intermediates live in the
    library's scratch array on the device, and `out` [B, E] bf16 must be given (nothing is
    allocated)."""
    bf = torch.bfloat16
    _check(hidden, "hidden", bf)
    B, E = hidden.shape
    C = _layer_weights(w_in, conv_w, gamma, w_out, E, Hk, Hv, dk, dv)
    _check(conv_state, "conv_state", torch.float32, (B, 3, C))
    _check(state, "state", torch.float32, (B, Hv, dk, dv))
    _check(out, "out", bf, (B, E))
    st = lib().gdn_layer_decode_noalloc(_p(hidden), _p(w_in), _p(conv_w), _p(gamma), _p(w_out), _p(conv_state),
                                        _p(state), _p(out), float(scale), float(l2_eps), float(norm_eps), B, E, Hk,
                                        Hv, dk, dv, int(order), _stream())
    if st != 0:
        raise GdnError("gdn_layer_decode_noalloc", st)
    return out
