"""fp64 CPU oracle for the Gated DeltaNet token mixer.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  The product path
(``hybrid_linear_attention_gated_amd``) never imports it, and it never imports
the product path.

``gdn_oracle.c`` (built into ``liboracle.so`` with gcc) is the token-by-token
fp64 recurrence used for parity at full sizes; ``gdn_ref.py`` is an
independent numpy fp64 reference used to cross-check it on small cases.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = False) -> str:
    """Compile gdn_oracle.c with gcc (-O2, OpenMP, strict IEEE fp64)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared",
                               "-fno-fast-math", "-ffp-contract=off", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def lib():
    global _lib
    if _lib is None:
        build()
        L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i = ctypes.c_int
        d = ctypes.c_double
        L.oracle_threads.argtypes = [i]
        L.oracle_threads.restype = i
        L.oracle_prep.argtypes = [P, P, P, i, P, P, P, P, P, i, i, i, i, i, d]
        L.oracle_prep.restype = None
        L.oracle_recurrence.argtypes = [P, P, P, P, P, P, i, P, P, P, d, i, i, i, i, i, P, i, i]
        L.oracle_recurrence.restype = None
        L.oracle_decode.argtypes = [P, P, P, P, P, P, P, P, P, d, d, i, i, i, i, i, i]
        L.oracle_decode.restype = None
        L.oracle_gated_rmsnorm.argtypes = [P, P, P, P, ctypes.c_long, i, d]
        L.oracle_gated_rmsnorm.restype = None
        _lib = L
    return _lib


def _f32(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.float32))


def _f64(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _i32(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def threads(units: int) -> int:
    return lib().oracle_threads(int(units))


def prep(x, w, cu, Hk, Hv, dk, dv, cs_in=None, eps=1e-6, want_cs_out=True):
    """fp64 conv+SiLU+L2.  x [T,C], w [C,4], cu [N+1], cs_in [N,3,C] or None (any float
    dtype; used as fp64)."""
    x = _f64(x); w = _f64(w); cu = _i32(cu)
    T, C = x.shape
    assert C == 2 * Hk * dk + Hv * dv and w.shape == (C, 4)
    N = len(cu) - 1
    csi = None if cs_in is None else _f64(cs_in)
    q = np.zeros((T, Hk, dk)); k = np.zeros((T, Hk, dk)); v = np.zeros((T, Hv, dv))
    cso = np.zeros((N, 3, C)) if want_cs_out else None
    lib().oracle_prep(_p(x), _p(w), _p(cu), N, _p(csi), _p(cso), _p(q), _p(k), _p(v),
                      T, Hk, Hv, dk, dv, float(eps))
    return q, k, v, cso


def recurrence(q, k, v, g, beta, cu, s0=None, scale=1.0, heads=None, order=0):
    """fp64 token recurrence.  q,k [T,Hk,dk], v [T,Hv,dv] (any float dtype;
    used as fp64), g, beta [T,Hv] fp32, s0 [N,Hv,dk,dv] fp32 or None.
    heads: optional list of v-heads to compute (others left zero).
    order: 0 = decay before retrieval, 1 = retrieval from the undecayed state."""
    q = _f64(q); k = _f64(k); v = _f64(v)
    g = _f32(g); beta = _f32(beta); cu = _i32(cu)
    T, Hk, dk = k.shape
    Hv, dv = v.shape[1], v.shape[2]
    N = len(cu) - 1
    s0a = None if s0 is None else _f32(s0)
    o = np.zeros((T, Hv, dv)); fin = np.zeros((N, Hv, dk, dv))
    hs = None if heads is None else _i32(heads)
    lib().oracle_recurrence(_p(q), _p(k), _p(v), _p(g), _p(beta), _p(cu), N, _p(s0a), _p(fin), _p(o),
                            float(scale), T, Hk, Hv, dk, dv, _p(hs), 0 if hs is None else len(hs), int(order))
    return o, fin


def decode(x, w, cs, g, beta, state, Hk, Hv, dk, dv, scale=1.0, eps=1e-6, order=0):
    """fp64 decode step (x, w, cs of any float dtype, used as fp64; g, beta and the state
    as float32, the library's types).  Returns o [B,Hv,dv], new state, new conv cache."""
    x = _f64(x); w = _f64(w); cs = _f64(cs); g = _f32(g); beta = _f32(beta); st = _f32(state)
    B = x.shape[0]
    o = np.zeros((B, Hv, dv)); st_out = np.zeros((B, Hv, dk, dv)); cs_out = np.zeros(cs.shape)
    lib().oracle_decode(_p(x), _p(w), _p(cs), _p(cs_out), _p(g), _p(beta), _p(st), _p(st_out), _p(o),
                        float(scale), float(eps), B, Hk, Hv, dk, dv, int(order))
    return o, st_out, cs_out


def gated_rmsnorm(y, z, gamma, eps=1e-6):
    """fp64 gated RMSNorm over the last axis: y / sqrt(mean y^2 + eps) * gamma * SiLU(z).
    y [..., dv], z same shape and gamma [dv] (any float dtype, used as fp64)."""
    y = _f64(y)
    dv = y.shape[-1]
    z = _f64(z)
    gamma = _f64(gamma)
    assert z.shape == y.shape and gamma.shape == (dv,)
    out = np.zeros(y.shape)
    rows = y.size // dv if dv else 0
    lib().oracle_gated_rmsnorm(_p(y), _p(z), _p(gamma), _p(out), rows, dv, float(eps))
    return out


def layer_prefill(hidden, w_in, conv_w, gamma, w_out, cu, Hk, Hv, dk, dv, cs_in=None, s0=None, scale=1.0,
                  l2_eps=1e-6, norm_eps=1e-6, order=0, heads=None):
    """Layer forward of ``gdn_ref.layer_prefill`` with the conv prep, the recurrence and
    the gated RMSNorm taken from the C library (fast enough for the 0.8B layer shape).
    heads: optional list of value heads whose recurrence is computed (the others'
    outputs and states are zero, and so is ``out``'s dependence on them); ``None`` =
    all heads.  Returns out [T, E], final states, conv caches, and the intermediate
    tensors {x, z, g, beta, y} (y = the normalised output entering the output
    projection).  Nothing between the input projection and the output is rounded."""
    from . import gdn_ref
    hidden = _f64(hidden)
    T = hidden.shape[0]
    x, z, ap, bp = gdn_ref.layer_split(hidden @ _f64(w_in).T, Hk, Hv, dk, dv)
    g, beta = gdn_ref.layer_gates(ap, bp)
    q, k, v, cs_out = prep(x, conv_w, cu, Hk, Hv, dk, dv, cs_in, l2_eps)
    o, fin = recurrence(q, k, v, g, beta, cu, s0, scale, heads=heads, order=order)
    y = gated_rmsnorm(o, z.reshape(T, Hv, dv), gamma, norm_eps).reshape(T, Hv * dv)
    if heads is not None:
        keep = np.zeros((Hv, dv))
        keep[list(heads)] = 1.0
        y = y * keep.reshape(1, Hv * dv)
    out = y @ _f64(w_out).T
    return out, fin, cs_out, {"x": x, "z": z, "g": g, "beta": beta, "y": y}


def layer_decode(hidden, w_in, conv_w, gamma, w_out, cs, state, Hk, Hv, dk, dv, scale=1.0, l2_eps=1e-6,
                 norm_eps=1e-6, order=0):
    """``gdn_ref.layer_decode`` with the decode step and the gated RMSNorm taken from
    the C library.  Returns out [B, E], new state, new conv cache, and {x, z, g, beta, y}."""
    from . import gdn_ref
    hidden = _f64(hidden)
    B = hidden.shape[0]
    x, z, ap, bp = gdn_ref.layer_split(hidden @ _f64(w_in).T, Hk, Hv, dk, dv)
    g, beta = gdn_ref.layer_gates(ap, bp)
    o, st, cso = decode(x, conv_w, cs, g, beta, state, Hk, Hv, dk, dv, scale, l2_eps, order)
    y = gated_rmsnorm(o, z.reshape(B, Hv, dv), gamma, norm_eps).reshape(B, Hv * dv)
    return y @ _f64(w_out).T, st, cso, {"x": x, "z": z, "g": g, "beta": beta, "y": y}
