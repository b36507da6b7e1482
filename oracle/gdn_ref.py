"""Independent numpy fp64 reference for the Gated DeltaNet token mixer.

TEST INFRASTRUCTURE ONLY: imported by the test suite, the smoke check and the
benchmark's CPU-baseline leg, never by the product path.

This module is written independently of ``gdn_oracle.c`` so the two can check
each other.  It uses the *product* form of the gated delta rule,

    S_t = a_t * S_{t-1} (I - b_t k_t k_t^T) + b_t v_t k_t^T,    o_t = S_t q_t,

with a value-major state S in R^{dv x dk}, whereas the C oracle follows the
step-by-step recurrent form of "Hugging Face Transformers: Qwen3.5-MoE series
explained" (section 4.3: decay, retrieve, correct, write, read) on a key-major
state.  Expanding the product form gives exactly the step form transposed, so
agreement between the two pins the orientation and the order of decay and
retrieval.

It also holds the chunked (WY / UT) form of the same recurrence, derived from
the recurrence alone, in fp64.  It is exact in exact arithmetic, so its
agreement with the token recurrence pins the algebra that any chunked kernel
relies on.

Conv / SiLU / L2 follow "7.6 Qwen3.5: the linear-attention hybrid" (LLM
full-stack book), section 7.6.2: depthwise causal conv1d, kernel 4, no bias,
then L2 normalisation of q and k per head; SiLU on every conv channel.
"""
from __future__ import annotations

import numpy as np

CONV_K = 4
L2_EPS = 1e-6


def silu(y: np.ndarray) -> np.ndarray:
    return y / (1.0 + np.exp(-y))


def l2norm(x: np.ndarray, eps: float = L2_EPS) -> np.ndarray:
    """x / sqrt(sum x^2 + eps) over the last axis."""
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)


def causal_conv_silu(x_seq: np.ndarray, w: np.ndarray, hist: np.ndarray | None) -> np.ndarray:
    """Depthwise causal conv (kernel 4) over one sequence, then SiLU.

    x_seq [L, C], w [C, 4], hist [3, C] (oldest first) or None (zeros).
    Output y[p] = sum_j w[:, j] * xe[p - 3 + j] with xe = concat(hist, x_seq).
    """
    L, C = x_seq.shape
    h = np.zeros((CONV_K - 1, C)) if hist is None else np.asarray(hist, dtype=np.float64)
    xe = np.concatenate([h, np.asarray(x_seq, dtype=np.float64)], axis=0)
    y = np.zeros((L, C))
    for j in range(CONV_K):
        y += w[:, j][None, :] * xe[j:j + L]
    return silu(y)


def prep(x, w, cu, Hk, Hv, dk, dv, cs_in=None, eps=L2_EPS):
    """Conv + SiLU + split + L2 over packed varlen sequences.

    Returns q [T,Hk,dk], k [T,Hk,dk], v [T,Hv,dv], cs_out [N,3,C] (fp64).
    """
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    T, C = x.shape
    N = len(cu) - 1
    qk = Hk * dk
    q = np.zeros((T, Hk, dk)); k = np.zeros((T, Hk, dk)); v = np.zeros((T, Hv, dv))
    cs_out = np.zeros((N, CONV_K - 1, C))
    for s in range(N):
        t0, t1 = int(cu[s]), int(cu[s + 1])
        hist = None if cs_in is None else cs_in[s]
        y = causal_conv_silu(x[t0:t1], w, hist)
        q[t0:t1] = l2norm(y[:, :qk].reshape(-1, Hk, dk), eps)
        k[t0:t1] = l2norm(y[:, qk:2 * qk].reshape(-1, Hk, dk), eps)
        v[t0:t1] = y[:, 2 * qk:].reshape(-1, Hv, dv)
        h = np.zeros((CONV_K - 1, C)) if cs_in is None else np.asarray(cs_in[s], dtype=np.float64)
        xe = np.concatenate([h, x[t0:t1]], axis=0)
        cs_out[s] = xe[-(CONV_K - 1):]
    return q, k, v, cs_out


def recurrence(q, k, v, g, beta, cu, s0=None, scale=1.0, order=0):
    """Product-form gated delta rule, token by token, vectorised over v-heads.

    q, k [T,Hk,dk]; v [T,Hv,dv]; g, beta [T,Hv]; s0 [N,Hv,dk,dv] (key-major,
    the library's layout) or None.  Returns o [T,Hv,dv] and the final state
    [N,Hv,dk,dv] (key-major).  order 0: S_t = a S (I - b k k^T) + b v k^T;
    order 1 (retrieval from the undecayed state, "7.6 Qwen3.5" 7.6.2):
    S_t = S (a I - b k k^T) + b v k^T.
    """
    q = np.asarray(q, np.float64); k = np.asarray(k, np.float64); v = np.asarray(v, np.float64)
    g = np.asarray(g, np.float64); beta = np.asarray(beta, np.float64)
    T, Hk, dk = k.shape
    Hv, dv = v.shape[1], v.shape[2]
    rep = Hv // Hk
    N = len(cu) - 1
    o = np.zeros((T, Hv, dv))
    fin = np.zeros((N, Hv, dk, dv))
    eye = np.eye(dk)
    for s in range(N):
        # value-major state: Sv[h] in R^{dv x dk}
        Sv = np.zeros((Hv, dv, dk)) if s0 is None else np.transpose(np.asarray(s0[s], np.float64), (0, 2, 1)).copy()
        for t in range(int(cu[s]), int(cu[s + 1])):
            kt = np.repeat(k[t], rep, axis=0)              # [Hv, dk]
            qt = scale * np.repeat(q[t], rep, axis=0)      # [Hv, dk]
            a = np.exp(g[t])                               # [Hv]
            b = beta[t]
            kk = b[:, None, None] * kt[:, :, None] * kt[:, None, :]                  # b k k^T
            if order == 0:
                Sv = a[:, None, None] * (Sv @ (eye[None] - kk))
            else:
                Sv = Sv @ (a[:, None, None] * eye[None] - kk)
            Sv = Sv + b[:, None, None] * v[t][:, :, None] * kt[:, None, :]
            o[t] = np.einsum('hjd,hd->hj', Sv, qt)
        fin[s] = np.transpose(Sv, (0, 2, 1))
    return o, fin


def decode_step(x, w, cs, g, beta, state, Hk, Hv, dk, dv, scale=1.0, eps=L2_EPS, order=0):
    """One decode step for every row b: conv window [cs[b], x[b]], then one
    product-form step.  Returns o [B,Hv,dv], new state, new conv cache."""
    x = np.asarray(x, np.float64); cs = np.asarray(cs, np.float64)
    B = x.shape[0]
    o = np.zeros((B, Hv, dv))
    new_state = np.zeros((B, Hv, dk, dv))
    new_cs = np.zeros_like(cs)
    cu = np.array([0, 1])
    for b in range(B):
        qb, kb, vb, cso = prep(x[b:b + 1], w, cu, Hk, Hv, dk, dv, cs_in=cs[b:b + 1], eps=eps)
        ob, fb = recurrence(qb, kb, vb, np.asarray(g)[b:b + 1], np.asarray(beta)[b:b + 1], cu,
                            s0=np.asarray(state)[b:b + 1], scale=scale, order=order)
        o[b] = ob[0]; new_state[b] = fb[0]; new_cs[b] = cso[0]
    return o, new_state, new_cs


def chunked(q, k, v, g, beta, cu, s0=None, scale=1.0, C=64, order=0):
    """Chunked (WY / UT) form in fp64, per sequence and v-head.

    Within a chunk with local cumulative log-decay G_t = sum_{s<=t} g_s:
      A[t,i] = b_t e^{G_t-G_i} (k_t . k_i)  (i < t),   Tm = (I + A)^{-1}
      W = Tm diag(b e^G) K,   U = Tm diag(b) V,   Delta = U - W S0
      O = diag(e^G) Q S0 + P Delta,   P[t,i] = e^{G_t-G_i} (q_t . k_i)  (i <= t)
      S_end = e^{G_c} S0 + (diag(e^{G_c - G}) K)^T Delta
    Key-major state S [dk, dv].  Chunks restart at every sequence start.
    order 1 (retrieval from the undecayed state) replaces e^{G_t} by e^{G_{t-1}}
    = e^{G_t - g_t} in A (first factor) and in W; U, P, O and S_end are unchanged.
    """
    q = np.asarray(q, np.float64); k = np.asarray(k, np.float64); v = np.asarray(v, np.float64)
    g = np.asarray(g, np.float64); beta = np.asarray(beta, np.float64)
    T, Hk, dk = k.shape
    Hv, dv = v.shape[1], v.shape[2]
    rep = Hv // Hk
    N = len(cu) - 1
    o = np.zeros((T, Hv, dv))
    fin = np.zeros((N, Hv, dk, dv))
    for s in range(N):
        for h in range(Hv):
            kh = h // rep
            S = np.zeros((dk, dv)) if s0 is None else np.asarray(s0[s, h], np.float64).copy()
            for c0 in range(int(cu[s]), int(cu[s + 1]), C):
                c1 = min(c0 + C, int(cu[s + 1]))
                K = k[c0:c1, kh]; Q = scale * q[c0:c1, kh]; V = v[c0:c1, h]
                b = beta[c0:c1, h]
                G = np.cumsum(g[c0:c1, h])
                Gr = G - g[c0:c1, h] if order else G    # decay applied before the retrieval or not
                D = G[:, None] - G[None, :]
                Dr = Gr[:, None] - G[None, :]
                lower = np.tril(np.ones((c1 - c0, c1 - c0)), -1)
                A = lower * b[:, None] * np.exp(np.where(lower > 0, Dr, 0.0)) * (K @ K.T)
                Tm = np.linalg.inv(np.eye(c1 - c0) + A)
                W = Tm @ ((b * np.exp(Gr))[:, None] * K)
                U = Tm @ (b[:, None] * V)
                Delta = U - W @ S
                causal = np.tril(np.ones((c1 - c0, c1 - c0)))
                P = causal * np.exp(np.where(causal > 0, D, 0.0)) * (Q @ K.T)
                o[c0:c1, h] = np.exp(G)[:, None] * (Q @ S) + P @ Delta
                S = np.exp(G[-1]) * S + (np.exp(G[-1] - G)[:, None] * K).T @ Delta
            fin[s, h] = S
    return o, fin


def gated_rmsnorm(y, z, gamma, eps=1e-6):
    """Gated RMSNorm ("7.6 Qwen3.5: the linear-attention hybrid", 7.6.2 output gate,
    7.6.3 RMSNorm), per row of the last axis: RMSNorm(y) * gamma * SiLU(z)."""
    y = np.asarray(y, dtype=np.float64)
    rms = np.sqrt(np.mean(y * y, axis=-1, keepdims=True) + eps)
    return (y / rms) * np.asarray(gamma, dtype=np.float64) * silu(np.asarray(z, dtype=np.float64))


# ---------------------------------------------------------------- layer forward
#
# The whole linear-attention token mixer around the core ("7.6 Qwen3.5: the
# linear-attention hybrid", section 7.6.2, with the layer widths of the 7.6.1 table;
# "Hugging Face Transformers: Qwen3.5-MoE series explained", sections 4.3 and 8.2):
# a bias-free input projection gives the pre-conv q|k|v, the output gate z and one
# decay and one update pre-activation per value head; conv + SiLU + L2 and the gated
# delta rule follow; the output passes the gated RMSNorm with SiLU(z) and a bias-free
# output projection.  The pages do not say how the two gate pre-activations become
# gates; the reading taken here is g = -softplus(a) (so a = exp(g) lies in (0, 1)) and
# beta = sigmoid(b), the maps under which N(0, 1) pre-activations give the layer
# shape's gate distributions.  Nothing between the input projection and the output
# is rounded: the pre-conv q|k|v, z and the normalised output entering the output
# projection are the exact fp64 values; g and beta are taken as fp32 (the library's
# gate type, as for the core's inputs).


def softplus(x):
    """log(1 + e^x), without overflow."""
    return np.logaddexp(0.0, np.asarray(x, dtype=np.float64))


def sigmoid(x):
    """1 / (1 + e^-x), without overflow."""
    return 0.5 * (1.0 + np.tanh(0.5 * np.asarray(x, dtype=np.float64)))


def layer_gates(a, b):
    """Decay log g = -softplus(a) and update gate beta = sigmoid(b), rounded to fp32."""
    return (-softplus(a)).astype(np.float32), sigmoid(b).astype(np.float32)


def layer_split(proj, Hk, Hv, dk, dv):
    """Split input-projection outputs [rows, conv_dim + Hv dv + 2 Hv] into the
    pre-conv q|k|v, z, a and b column blocks (in that order)."""
    C = 2 * Hk * dk + Hv * dv
    Z = Hv * dv
    assert proj.shape[1] == C + Z + 2 * Hv
    return proj[:, :C], proj[:, C:C + Z], proj[:, C + Z:C + Z + Hv], proj[:, C + Z + Hv:]


def layer_prefill(hidden, w_in, conv_w, gamma, w_out, cu, Hk, Hv, dk, dv, cs_in=None, s0=None, scale=1.0,
                  l2_eps=L2_EPS, norm_eps=1e-6, order=0):
    """Layer forward over packed sequences.  hidden [T, E], w_in [conv_dim + Hv dv +
    2 Hv, E] and w_out [E, Hv dv] stored as a linear layer stores them (out = in W^T);
    conv_w [conv_dim, 4]; gamma [dv] the gain as applied.  Returns out [T, E], the
    final states [N, Hv, dk, dv] and the conv caches [N, 3, conv_dim]."""
    hidden = np.asarray(hidden, np.float64)
    T = hidden.shape[0]
    x, z, ap, bp = layer_split(hidden @ np.asarray(w_in, np.float64).T, Hk, Hv, dk, dv)
    g, beta = layer_gates(ap, bp)
    q, k, v, cs_out = prep(x, conv_w, cu, Hk, Hv, dk, dv, cs_in, l2_eps)
    o, fin = recurrence(q, k, v, g, beta, cu, s0, scale, order)
    y = gated_rmsnorm(o, z.reshape(T, Hv, dv), gamma, norm_eps).reshape(T, Hv * dv)
    return y @ np.asarray(w_out, np.float64).T, fin, cs_out


def layer_decode(hidden, w_in, conv_w, gamma, w_out, cs, state, Hk, Hv, dk, dv, scale=1.0, l2_eps=L2_EPS,
                 norm_eps=1e-6, order=0):
    """One token of B sequences through the layer: hidden [B, E]; cs [B, 3, conv_dim]
    and state [B, Hv, dk, dv] are the caches.  Returns out [B, E], the new state and
    the new conv cache."""
    hidden = np.asarray(hidden, np.float64)
    B = hidden.shape[0]
    x, z, ap, bp = layer_split(hidden @ np.asarray(w_in, np.float64).T, Hk, Hv, dk, dv)
    g, beta = layer_gates(ap, bp)
    o, new_state, new_cs = decode_step(x, conv_w, cs, g, beta, state, Hk, Hv, dk, dv, scale, l2_eps, order)
    y = gated_rmsnorm(o, z.reshape(B, Hv, dv), gamma, norm_eps).reshape(B, Hv * dv)
    return y @ np.asarray(w_out, np.float64).T, new_state, new_cs
