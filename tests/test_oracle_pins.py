"""Pins of the fp64 CPU oracle to facts outside itself (CPU only).

Each test checks the oracle (the C library and the independent numpy reference)
against something the pages or the mathematics fix: hand-worked examples
stored under tests/golden/, exact rational brute force of the product form of
the recurrence, closed forms and invariants of the gated delta rule, and
library routines for the conv / SiLU / L2 prep.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle import gdn_ref

RNG = np.random.default_rng(7)


def _unit(shape, rng=RNG):
    z = rng.standard_normal(shape)
    return z / np.linalg.norm(z, axis=-1, keepdims=True)


def _f32(a):
    return np.asarray(a, dtype=np.float32)


def _rand_core(T, Hk, Hv, dk, dv, rng, N=1, lengths=None, s0=True, decay=(0.8, 1.0)):
    lengths = lengths or [T]
    T = sum(lengths)
    q = _unit((T, Hk, dk), rng)
    k = _unit((T, Hk, dk), rng)
    v = rng.standard_normal((T, Hv, dv))
    g = _f32(np.log(rng.uniform(*decay, (T, Hv))))
    b = _f32(rng.uniform(0.05, 0.95, (T, Hv)))
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    st = _f32(rng.standard_normal((len(lengths), Hv, dk, dv)) * 0.3) if s0 else None
    return q, k, v, g, b, cu, st


# ---------------------------------------------------------------- golden

def test_worked_delta_rule_golden(golden_dir):
    fx = json.load(open(os.path.join(golden_dir, "worked_delta_rule.json")))
    T = len(fx["a"])
    q = np.array(fx["q"])[:, None, :]
    k = np.array(fx["k"])[:, None, :]
    v = np.array(fx["v"])[:, None, :]
    g = _f32(np.log(fx["a"]))[:, None]
    b = _f32(fx["b"])[:, None]
    cu = np.array([0, T], np.int32)
    for impl in (oracle.recurrence, gdn_ref.recurrence):
        o, fin = impl(q, k, v, g, b, cu)
        np.testing.assert_allclose(o[:, 0], fx["o"], atol=1e-6)
        np.testing.assert_allclose(fin[0, 0], fx["final_state"], atol=1e-6)


def test_worked_conv_golden(golden_dir):
    fx = json.load(open(os.path.join(golden_dir, "worked_conv.json")))
    Hk, Hv, dk, dv = fx["Hk"], fx["Hv"], fx["dk"], fx["dv"]
    x = np.array(fx["x"], np.float64)
    w = np.array(fx["w"], np.float64)
    hist = np.array(fx["history"], np.float64)[None]
    y = torch.tensor(fx["y_pre_silu"], dtype=torch.float64)
    act = F.silu(y)                               # library SiLU
    eq = F.normalize(act[:, 0:2], dim=-1).numpy()   # library L2 (eps differs by < 1e-6 rel.)
    ek = F.normalize(act[:, 2:4], dim=-1).numpy()
    ev = act[:, 4:6].numpy()
    cu = np.array([0, 4], np.int32)
    for impl in (oracle.prep, gdn_ref.prep):
        q, k, v, cso = impl(x, w, cu, Hk, Hv, dk, dv, cs_in=hist)
        np.testing.assert_allclose(q[:, 0], eq, rtol=1e-5, atol=1e-7)
        np.testing.assert_allclose(k[:, 0], ek, rtol=1e-5, atol=1e-7)
        np.testing.assert_allclose(v[:, 0], ev, rtol=1e-12)
        np.testing.assert_array_equal(cso[0], np.array(fx["conv_state_out"], np.float64))


def test_shape_table_golden(golden_dir):
    from hybrid_linear_attention_gated_amd import inputs
    fx = json.load(open(os.path.join(golden_dir, "shape_0p8b.json")))
    # workloads are built on the printed layer shape
    assert (16, 16, 128, 128) == (fx["linear_num_key_heads"], fx["linear_num_value_heads"],
                                   fx["linear_key_head_dim"], fx["linear_value_head_dim"])
    wl = inputs.prefill_workload("probe", 99, [8], 16, 16)
    assert (wl.Hk, wl.Hv, wl.dk, wl.dv) == (16, 16, 128, 128)
    assert wl.conv_w.shape[1] == fx["linear_conv_kernel_dim"]
    assert wl.conv_dim == 2 * 16 * 128 + 16 * 128
    # the state the oracle returns per layer is Hv x dk x dv and does not grow with T
    q, k, v, g, b, cu, _ = _rand_core(3, 2, 2, 4, 4, RNG, s0=False)
    _, fin = oracle.recurrence(q, k, v, g, b, cu)
    assert fin.shape[1:] == (2, 4, 4)
    total = fx["linear_layers"] * 16 * 128 * 128 * fx["state_bytes_per_elem_bf16"]
    assert abs(total / 1e6 - fx["printed_state_total_MB"]) < 0.05


# ---------------------------------------------------------------- exact brute force

def _rational_product_form(q, k, v, a, b):
    """S_t = a S (I - b k k^T) + b v k^T, o = S q, value-major, exact rationals."""
    T, dk = len(k), len(k[0])
    dv = len(v[0])
    S = [[Fraction(0)] * dk for _ in range(dv)]
    outs = []
    for t in range(T):
        kt = [Fraction(x) for x in k[t]]
        P = [[(Fraction(1) if i == j else Fraction(0)) - b[t] * kt[i] * kt[j] for j in range(dk)]
             for i in range(dk)]
        SP = [[sum(S[r][m] * P[m][c] for m in range(dk)) for c in range(dk)] for r in range(dv)]
        S = [[a[t] * SP[r][c] + b[t] * Fraction(v[t][r]) * kt[c] for c in range(dk)] for r in range(dv)]
        outs.append([sum(S[r][c] * Fraction(q[t][c]) for c in range(dk)) for r in range(dv)])
    return outs, S


@pytest.mark.parametrize("seed", [0, 1])
def test_exact_rational_bruteforce(seed):
    rng = np.random.default_rng(100 + seed)
    T, dk, dv = 5, 3, 2
    # dyadic rationals are exact in float32 and float64
    q = rng.integers(-8, 9, (T, dk)) / 8.0
    k = rng.integers(-8, 9, (T, dk)) / 8.0
    v = rng.integers(-8, 9, (T, dv)) / 4.0
    g32 = _f32(np.log(rng.uniform(0.5, 1.0, T)))
    b32 = _f32(rng.integers(1, 8, T) / 8.0)
    a_exact = [Fraction(math.exp(float(x))) for x in g32]    # same double as the oracle's exp
    b_exact = [Fraction(float(x)) for x in b32]
    outs, S = _rational_product_form(q.tolist(), k.tolist(), v.tolist(), a_exact, b_exact)
    o_ex = np.array([[float(x) for x in r] for r in outs])
    S_ex = np.array([[float(x) for x in r] for r in S]).T         # key-major
    cu = np.array([0, T], np.int32)
    for impl in (oracle.recurrence, gdn_ref.recurrence):
        o, fin = impl(q[:, None], k[:, None], v[:, None], g32[:, None], b32[:, None], cu)
        np.testing.assert_allclose(o[:, 0], o_ex, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(fin[0, 0], S_ex, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- closed forms / invariants

def test_I1_identity_gates():
    q, k, v, g, b, cu, s0 = _rand_core(20, 2, 2, 8, 6, RNG)
    g[:] = 0.0; b[:] = 0.0
    o, fin = oracle.recurrence(q, k, v, g, b, cu, s0=s0)
    np.testing.assert_allclose(fin[0], s0[0], rtol=0, atol=0)
    np.testing.assert_allclose(o, np.einsum('hij,thi->thj', s0[0].astype(np.float64), q), rtol=1e-12, atol=1e-12)


def test_I2_pure_decay():
    q, k, v, g, b, cu, s0 = _rand_core(30, 2, 2, 8, 6, RNG)
    b[:] = 0.0
    o, fin = oracle.recurrence(q, k, v, g, b, cu, s0=s0)
    cum = np.exp(np.cumsum(g.astype(np.float64), axis=0))      # [T, H]
    np.testing.assert_allclose(fin[0], cum[-1][:, None, None] * s0[0], rtol=1e-12)
    exp_o = cum[:, :, None] * np.einsum('hij,thi->thj', s0[0].astype(np.float64), q)
    np.testing.assert_allclose(o, exp_o, rtol=1e-11, atol=1e-13)


def test_I3_delta_write_is_exact_for_unit_keys():
    q, k, v, g, b, cu, s0 = _rand_core(25, 2, 2, 8, 6, RNG)
    b[:] = 1.0
    q = k.copy()
    for impl in (oracle.recurrence, gdn_ref.recurrence):
        o, _ = impl(q, k, v, g, b, cu, s0=s0)
        np.testing.assert_allclose(o, v, rtol=1e-11, atol=1e-11)


def test_I4_orthonormal_keys_reduce_to_linear_attention():
    d, T = 8, 8
    Qm, _ = np.linalg.qr(RNG.standard_normal((d, d)))
    k = Qm.T[:, None, :]                     # rows are orthonormal keys
    v = RNG.standard_normal((T, 1, 5))
    g = np.zeros((T, 1), np.float32); b = np.ones((T, 1), np.float32)
    q = RNG.standard_normal((T, 1, d))
    cu = np.array([0, T], np.int32)
    o, fin = oracle.recurrence(q, k, v, g, b, cu)
    lin = np.einsum('ti,tj->ij', k[:, 0], v[:, 0])           # sum_i k_i v_i^T
    np.testing.assert_allclose(fin[0, 0], lin, atol=1e-12)
    np.testing.assert_allclose(fin[0, 0].T @ k[:, 0].T, v[:, 0].T, atol=1e-12)   # exact retrieval
    # outputs equal causal linear attention sum_{i<=t} (q_t . k_i) v_i
    causal = np.tril(q[:, 0] @ k[:, 0].T) @ v[:, 0]
    np.testing.assert_allclose(o[:, 0], causal, atol=1e-12)


def test_I5_single_token():
    q, k, v, g, b, cu, _ = _rand_core(1, 3, 3, 8, 5, RNG, s0=False)
    o, fin = oracle.recurrence(q, k, v, g, b, cu)
    bb = b[0].astype(np.float64)
    kq = np.sum(k[0] * q[0], axis=-1)
    np.testing.assert_allclose(o[0], (bb * kq)[:, None] * v[0], rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(fin[0], bb[:, None, None] * k[0][:, :, None] * v[0][:, None, :], rtol=1e-13)


def test_I6_linearity():
    q, k, v, g, b, cu, s0 = _rand_core(40, 2, 2, 8, 6, RNG)
    v2 = RNG.standard_normal(v.shape)
    s2 = _f32(RNG.standard_normal(s0.shape))
    o1, f1 = oracle.recurrence(q, k, v, g, b, cu, s0=s0)
    o2, f2 = oracle.recurrence(q, k, v2, g, b, cu, s0=s2)
    # 0.5*(v, s0) + 0.25*(v2, s2) -- the float32 sums below are exact for these values
    s3 = _f32(0.5 * s0.astype(np.float64) + 0.25 * s2.astype(np.float64))
    exact = np.array_equal(s3.astype(np.float64), 0.5 * s0.astype(np.float64) + 0.25 * s2.astype(np.float64))
    o3, f3 = oracle.recurrence(q, k, 0.5 * v + 0.25 * v2, g, b, cu, s0=s3)
    tol = 1e-12 if exact else 1e-6
    np.testing.assert_allclose(o3, 0.5 * o1 + 0.25 * o2, rtol=tol, atol=tol)
    np.testing.assert_allclose(f3, 0.5 * f1 + 0.25 * f2, rtol=tol, atol=tol)
    o4, f4 = oracle.recurrence(q, k, v, g, b, cu, s0=s0, scale=2.5)
    np.testing.assert_allclose(o4, 2.5 * o1, rtol=1e-13, atol=1e-14)
    np.testing.assert_array_equal(f4, f1)


@pytest.mark.parametrize("L", [1, 63, 64, 65, 200])
def test_I7_chunked_equals_recurrent(L):
    q, k, v, g, b, cu, s0 = _rand_core(L, 2, 4, 16, 8, RNG)
    o_r, f_r = oracle.recurrence(q, k, v, g, b, cu, s0=s0, scale=0.7)
    o_c, f_c = gdn_ref.chunked(q, k, v, g, b, cu, s0=s0, scale=0.7, C=64)
    np.testing.assert_allclose(o_c, o_r, rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(f_c, f_r, rtol=1e-10, atol=1e-11)


@pytest.mark.parametrize("t1", [1, 64, 100])
def test_I8_split_carry(t1):
    T, Hk, Hv, dk, dv = 160, 2, 2, 8, 8
    C = 2 * Hk * dk + Hv * dv
    x = _f32(RNG.standard_normal((T, C)))
    w = _f32(RNG.standard_normal((C, 4)) * 0.5)
    g = _f32(np.log(RNG.uniform(0.8, 1.0, (T, Hv))))
    b = _f32(RNG.uniform(0.1, 0.9, (T, Hv)))
    s0 = _f32(RNG.standard_normal((1, Hv, dk, dv)) * 0.1)
    cs0 = _f32(RNG.standard_normal((1, 3, C)))
    full = np.array([0, T], np.int32)
    q, k, v, cso = oracle.prep(x, w, full, Hk, Hv, dk, dv, cs_in=cs0)
    o, fin = oracle.recurrence(q, k, v, g, b, full, s0=s0)
    q1, k1, v1, cs1 = oracle.prep(x[:t1], w, np.array([0, t1], np.int32), Hk, Hv, dk, dv, cs_in=cs0)
    o1, f1 = oracle.recurrence(q1, k1, v1, g[:t1], b[:t1], np.array([0, t1], np.int32), s0=s0)
    q2, k2, v2, cs2 = oracle.prep(x[t1:], w, np.array([0, T - t1], np.int32), Hk, Hv, dk, dv, cs_in=_f32(cs1))
    o2, f2 = oracle.recurrence(q2, k2, v2, g[t1:], b[t1:], np.array([0, T - t1], np.int32), s0=_f32(f1))
    # carried state passes through float32 here, so compare with a float32-level tolerance
    np.testing.assert_allclose(np.concatenate([o1, o2]), o, rtol=1e-5, atol=1e-6)
    np.testing.assert_allclose(f2, fin, rtol=1e-5, atol=1e-6)
    np.testing.assert_array_equal(cs2, cso)


def test_I9_varlen_packing_equals_separate_runs():
    lengths = [5, 1, 70, 0, 33]
    Hk, Hv, dk, dv = 1, 2, 8, 8
    C = 2 * Hk * dk + Hv * dv
    T = sum(lengths)
    x = _f32(RNG.standard_normal((T, C)))
    w = _f32(RNG.standard_normal((C, 4)) * 0.5)
    g = _f32(np.log(RNG.uniform(0.8, 1.0, (T, Hv))))
    b = _f32(RNG.uniform(0.1, 0.9, (T, Hv)))
    s0 = _f32(RNG.standard_normal((len(lengths), Hv, dk, dv)) * 0.1)
    cs = _f32(RNG.standard_normal((len(lengths), 3, C)))
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    q, k, v, cso = oracle.prep(x, w, cu, Hk, Hv, dk, dv, cs_in=cs)
    o, fin = oracle.recurrence(q, k, v, g, b, cu, s0=s0)
    for s, L in enumerate(lengths):
        t0, t1 = cu[s], cu[s + 1]
        one = np.array([0, L], np.int32)
        qs, ks, vs, css = oracle.prep(x[t0:t1], w, one, Hk, Hv, dk, dv, cs_in=cs[s:s + 1])
        os_, fs = oracle.recurrence(qs, ks, vs, g[t0:t1], b[t0:t1], one, s0=s0[s:s + 1])
        np.testing.assert_array_equal(o[t0:t1], os_)
        np.testing.assert_array_equal(fin[s], fs[0])
        np.testing.assert_array_equal(cso[s], css[0])
    # zero-length sequence: state and conv cache pass through unchanged
    np.testing.assert_array_equal(fin[3], s0[3].astype(np.float64))
    np.testing.assert_array_equal(cso[3], cs[3].astype(np.float64))


def test_I10_gqa_equals_repeat_interleave():
    q, k, v, g, b, cu, s0 = _rand_core(50, 2, 6, 8, 8, RNG)
    o, fin = oracle.recurrence(q, k, v, g, b, cu, s0=s0)
    qr = np.repeat(q, 3, axis=1); kr = np.repeat(k, 3, axis=1)
    o2, f2 = oracle.recurrence(qr, kr, v, g, b, cu, s0=s0)
    np.testing.assert_array_equal(o, o2)
    np.testing.assert_array_equal(fin, f2)


def test_I11_contraction_bound_long_run():
    T, H, d = 3000, 2, 16
    q, k, v, g, b, cu, s0 = _rand_core(T, H, H, d, d, RNG, decay=(0.99, 1.0))
    b = _f32(RNG.uniform(0.0, 2.0, (T, H)))
    prev = s0.astype(np.float64)
    step = 200
    # check the bound on the state every `step` tokens, carrying the state exactly in fp64 via numpy
    o_all, fin = gdn_ref.recurrence(q, k, v, g, b, cu, s0=s0)
    St = prev[0]
    for t0 in range(0, T, step):
        one = np.array([0, min(step, T - t0)], np.int32)
        _, f = gdn_ref.recurrence(q[t0:t0 + step], k[t0:t0 + step], v[t0:t0 + step],
                                  g[t0:t0 + step], b[t0:t0 + step], one, s0=St[None])
        a = np.exp(g[t0:t0 + step].astype(np.float64))
        bound = np.linalg.norm(St, axis=(1, 2))
        for t in range(one[1]):
            bound = a[t] * bound + b[t].astype(np.float64) * np.linalg.norm(v[t0 + t], axis=-1)
        assert np.all(np.linalg.norm(f[0], axis=(1, 2)) <= bound * (1 + 1e-12))
        St = f[0]
    np.testing.assert_allclose(St, fin[0], rtol=1e-9, atol=1e-12)


def test_I12_prep_matches_library_conv():
    lengths = [7, 1, 40]
    Hk, Hv, dk, dv = 2, 4, 8, 4
    C = 2 * Hk * dk + Hv * dv
    T = sum(lengths)
    x = _f32(RNG.standard_normal((T, C)))
    w = _f32(RNG.standard_normal((C, 4)) * 0.5)
    cs = _f32(RNG.standard_normal((3, 3, C)))
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    for impl in (oracle.prep, gdn_ref.prep):
        q, k, v, cso = impl(x, w, cu, Hk, Hv, dk, dv, cs_in=cs)
        for s in range(3):
            t0, t1 = cu[s], cu[s + 1]
            xe = torch.tensor(np.concatenate([cs[s], x[t0:t1]]), dtype=torch.float64).T[None]  # [1,C,3+L]
            y = F.conv1d(xe, torch.tensor(w, dtype=torch.float64)[:, None, :], groups=C)[0].T  # valid conv
            y = F.silu(y)
            eq = F.normalize(y[:, :Hk * dk].reshape(-1, Hk, dk), dim=-1).numpy()
            ek = F.normalize(y[:, Hk * dk:2 * Hk * dk].reshape(-1, Hk, dk), dim=-1).numpy()
            np.testing.assert_allclose(q[t0:t1], eq, rtol=2e-5, atol=1e-8)   # eps 1e-6 inside the sqrt
            np.testing.assert_allclose(k[t0:t1], ek, rtol=2e-5, atol=1e-8)
            np.testing.assert_allclose(v[t0:t1], y[:, 2 * Hk * dk:].reshape(-1, Hv, dv).numpy(), rtol=1e-12, atol=1e-14)
    # zero history equals the padded-convolution definition (padding 3, keep the first T outputs)
    q, k, v, _ = oracle.prep(x[:7], w, np.array([0, 7], np.int32), Hk, Hv, dk, dv)
    xt = torch.tensor(x[:7], dtype=torch.float64).T[None]
    y = F.silu(F.conv1d(xt, torch.tensor(w, dtype=torch.float64)[:, None, :], groups=C, padding=3)[0, :, :7].T)
    np.testing.assert_allclose(v, y[:, 2 * Hk * dk:].reshape(-1, Hv, dv).numpy(), rtol=1e-12, atol=1e-14)


def test_silu_and_l2_identities():
    # silu(y) - silu(-y) = y, silu(0) = 0; L2 output has unit norm (up to eps) and keeps direction
    Hk, Hv, dk, dv = 1, 1, 4, 4
    C = 2 * dk + dv
    x = _f32(np.random.default_rng(11).standard_normal((5, C)) * 4.0)
    w = np.zeros((C, 4), np.float32); w[:, 3] = 1.0
    _, _, vp, _ = oracle.prep(x, w, np.array([0, 5], np.int32), Hk, Hv, dk, dv)
    _, _, vn, _ = oracle.prep(-x, w, np.array([0, 5], np.int32), Hk, Hv, dk, dv)
    np.testing.assert_allclose(vp - vn, x[:, 2 * dk:].reshape(5, 1, dv), rtol=1e-12, atol=1e-14)
    q, k, _, _ = oracle.prep(x, w, np.array([0, 5], np.int32), Hk, Hv, dk, dv)
    nrm = np.linalg.norm(q, axis=-1)
    assert np.all(nrm <= 1.0) and np.all(1.0 - nrm < 1e-5)
    zero = np.zeros((1, C), np.float32)
    qz, kz, vz, _ = oracle.prep(zero, w, np.array([0, 1], np.int32), Hk, Hv, dk, dv)
    assert np.all(qz == 0) and np.all(kz == 0) and np.all(vz == 0)


def test_I13_decode_steps_equal_prefill():
    T, Hk, Hv, dk, dv = 12, 2, 4, 8, 8
    C = 2 * Hk * dk + Hv * dv
    x = _f32(RNG.standard_normal((T, C)))
    w = _f32(RNG.standard_normal((C, 4)) * 0.5)
    g = _f32(np.log(RNG.uniform(0.8, 1.0, (T, Hv))))
    b = _f32(RNG.uniform(0.1, 0.9, (T, Hv)))
    cu = np.array([0, T], np.int32)
    q, k, v, cso = oracle.prep(x, w, cu, Hk, Hv, dk, dv)
    o, fin = oracle.recurrence(q, k, v, g, b, cu, scale=0.5)
    st = np.zeros((1, Hv, dk, dv)); cs = np.zeros((1, 3, C))
    outs = []
    for t in range(T):
        ot, st, cs = oracle.decode(x[t:t + 1], w, _f32(cs), g[t:t + 1], b[t:t + 1], _f32(st), Hk, Hv, dk, dv, scale=0.5)
        outs.append(ot[0])
    # the decode state passes through float32 between steps
    np.testing.assert_allclose(np.stack(outs), o, rtol=1e-5, atol=1e-6)
    np.testing.assert_allclose(st[0], fin[0], rtol=1e-5, atol=1e-6)
    np.testing.assert_array_equal(cs, cso)


# ---------------------------------------------------------------- C oracle vs numpy reference

def test_c_oracle_matches_numpy_reference():
    lengths = [3, 70, 0, 129]
    Hk, Hv, dk, dv = 2, 4, 16, 8
    C = 2 * Hk * dk + Hv * dv
    T = sum(lengths)
    x = _f32(RNG.standard_normal((T, C)))
    w = _f32(RNG.standard_normal((C, 4)) * 0.5)
    g = _f32(-np.logaddexp(0, RNG.standard_normal((T, Hv))))
    b = _f32(1 / (1 + np.exp(-RNG.standard_normal((T, Hv)))))
    s0 = _f32(RNG.standard_normal((4, Hv, dk, dv)) * 0.1)
    cs = _f32(RNG.standard_normal((4, 3, C)))
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    qc, kc, vc, csc = oracle.prep(x, w, cu, Hk, Hv, dk, dv, cs_in=cs)
    qn, kn, vn, csn = gdn_ref.prep(x, w, cu, Hk, Hv, dk, dv, cs_in=cs)
    np.testing.assert_allclose(qc, qn, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(kc, kn, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(vc, vn, rtol=1e-12, atol=1e-14)
    np.testing.assert_array_equal(csc, csn)
    oc, fc = oracle.recurrence(qc, kc, vc, g, b, cu, s0=s0, scale=0.3)
    on, fn = gdn_ref.recurrence(qn, kn, vn, g, b, cu, s0=s0, scale=0.3)
    np.testing.assert_allclose(oc, on, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(fc, fn, rtol=1e-10, atol=1e-12)
    # head subset leaves other heads untouched and matches the full run
    oh, fh = oracle.recurrence(qc, kc, vc, g, b, cu, s0=s0, scale=0.3, heads=[1, 3])
    np.testing.assert_array_equal(oh[:, [1, 3]], oc[:, [1, 3]])
    assert np.all(oh[:, [0, 2]] == 0)


def test_decode_c_matches_numpy():
    B, Hk, Hv, dk, dv = 5, 2, 4, 8, 8
    C = 2 * Hk * dk + Hv * dv
    x = _f32(RNG.standard_normal((B, C)))
    w = _f32(RNG.standard_normal((C, 4)) * 0.5)
    cs = _f32(RNG.standard_normal((B, 3, C)))
    g = _f32(np.log(RNG.uniform(0.9, 1.0, (B, Hv))))
    b = _f32(RNG.uniform(0.1, 0.9, (B, Hv)))
    st = _f32(RNG.standard_normal((B, Hv, dk, dv)) * 0.1)
    oc, sc, csc = oracle.decode(x, w, cs, g, b, st, Hk, Hv, dk, dv, scale=0.7)
    on, sn, csn = gdn_ref.decode_step(x, w, cs, g, b, st, Hk, Hv, dk, dv, scale=0.7)
    np.testing.assert_allclose(oc, on, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(sc, sn, rtol=1e-10, atol=1e-12)
    np.testing.assert_array_equal(csc, csn)
    # the conv cache shifts by one slot and appends the new input
    np.testing.assert_array_equal(csc[:, :2], cs[:, 1:].astype(np.float64))
    np.testing.assert_array_equal(csc[:, 2], x.astype(np.float64))


def test_planted_mistakes_are_caught():
    """Mutations of the numpy reference (in-test, on the CPU) fail the exact pins."""
    T, dk, dv = 4, 3, 2
    rng = np.random.default_rng(5)
    q = rng.integers(-4, 5, (T, dk)) / 4.0
    k = rng.integers(-4, 5, (T, dk)) / 4.0
    v = rng.integers(-4, 5, (T, dv)) / 2.0
    a = [Fraction(1, 2), Fraction(3, 4), Fraction(1), Fraction(7, 8)]
    b = [Fraction(1, 2), Fraction(1), Fraction(1, 4), Fraction(3, 4)]
    outs, _ = _rational_product_form(q.tolist(), k.tolist(), v.tolist(), a, b)
    ref = np.array([[float(x) for x in r] for r in outs])

    def stepform(retrieve_before_decay=False, sign=1.0):
        S = np.zeros((dk, dv)); out = []
        for t in range(T):
            aa, bb = float(a[t]), float(b[t])
            m = S.T @ k[t] if retrieve_before_decay else (aa * S).T @ k[t]
            S = aa * S
            d = bb * (v[t] - sign * m)
            S = S + np.outer(k[t], d)
            out.append(S.T @ q[t])
        return np.array(out)

    np.testing.assert_allclose(stepform(), ref, atol=1e-12)
    assert not np.allclose(stepform(retrieve_before_decay=True), ref, atol=1e-6)
    assert not np.allclose(stepform(sign=-1.0), ref, atol=1e-6)


# ------------------------------------------------------------------ gated RMSNorm epilogue
# "7.6 Qwen3.5: the linear-attention hybrid", 7.6.2 (output gate o = RMSNorm(y) * SiLU(z))
# and 7.6.3 (RMSNorm: x * rsqrt(mean x^2 + eps) times a per-channel gain).

SIGMOID_1 = 0.7310585786300049    # logistic(1), tabulated
SIGMOID_3 = 0.9525741268224334    # logistic(3), tabulated


def _both_norms(y, z, gamma, eps):
    return oracle.gated_rmsnorm(y, z, gamma, eps), gdn_ref.gated_rmsnorm(y, z, gamma, eps)


def test_gated_rmsnorm_constant_gate_closed_forms():
    rng = np.random.default_rng(21)
    dv = 16
    y = _f32(rng.standard_normal((4, dv)) * 3.0)
    ones = np.ones(dv, np.float32)
    for c, silu_c in [(0.0, 0.0), (1.0, SIGMOID_1), (-1.0, -(1.0 - SIGMOID_1)), (3.0, 3.0 * SIGMOID_3)]:
        z = np.full(y.shape, c, np.float32)
        for out in _both_norms(y, z, ones, 0.0):
            rms = np.sqrt(np.mean(out * out, axis=-1))
            np.testing.assert_allclose(rms, abs(silu_c), rtol=1e-12, atol=1e-15)
            if c != 0.0:   # direction of y, sign of SiLU(c)
                yn = y / np.linalg.norm(y, axis=-1, keepdims=True)
                on = out / np.linalg.norm(out, axis=-1, keepdims=True)
                np.testing.assert_allclose(on, np.sign(silu_c) * yn, atol=1e-12)


def test_gated_rmsnorm_invariants():
    rng = np.random.default_rng(22)
    rows, dv = 6, 32
    y = _f32(rng.standard_normal((rows, dv)))
    z = _f32(rng.standard_normal((rows, dv)))
    gamma = _f32(rng.uniform(0.5, 2.0, dv))
    base, _ = _both_norms(y, z, gamma, 0.0)
    # scale invariance (eps = 0): powers of two keep the float32 inputs exact
    for lam in (2.0 ** -10, 2.0 ** 12):
        np.testing.assert_allclose(oracle.gated_rmsnorm(y * lam, z, gamma, 0.0), base, rtol=1e-12)
    # the gain multiplies channel by channel
    ones = np.ones(dv, np.float32)
    unit, _ = _both_norms(y, z, ones, 0.0)
    np.testing.assert_allclose(base, unit * gamma, rtol=1e-12)
    # rows are independent (the norm axis is the last one): heads of very different size
    y2 = y.copy(); y2[0] *= 1024.0; y2[3] *= 2.0 ** -10
    out2 = oracle.gated_rmsnorm(y2, z, gamma, 0.0)
    np.testing.assert_allclose(out2, base, rtol=1e-9)
    # odd in y
    np.testing.assert_allclose(oracle.gated_rmsnorm(-y, z, gamma, 0.0), -base, rtol=1e-12)
    # eps: a constant row y = 2^-10 with eps = 2^-20 has mean y^2 = eps, so y / rms = 1/sqrt(2)
    yc = np.full((1, dv), 2.0 ** -10, np.float32)
    zc = np.full((1, dv), 1.0, np.float32)
    for out in _both_norms(yc, zc, ones, 2.0 ** -20):
        np.testing.assert_allclose(out, math.sqrt(0.5) * SIGMOID_1, rtol=1e-12)
    # a zero row stays zero with eps > 0
    out0 = oracle.gated_rmsnorm(np.zeros((2, dv), np.float32), z[:2], gamma, 1e-6)
    assert np.all(out0 == 0.0)


def test_gated_rmsnorm_matches_library_rms_norm():
    rng = np.random.default_rng(23)
    y = _f32(rng.standard_normal((3, 5, 64)) * np.array([1e-2, 1.0, 30.0])[:, None, None])
    z = _f32(rng.standard_normal((3, 5, 64)) * 2.0)
    gamma = _f32(rng.uniform(-1.0, 2.0, 64))
    ref = F.rms_norm(torch.from_numpy(y).double(), (64,), torch.from_numpy(gamma).double(), eps=1e-6) \
        * F.silu(torch.from_numpy(z).double())
    for out in _both_norms(y, z, gamma, 1e-6):
        np.testing.assert_allclose(out, ref.numpy(), rtol=1e-12, atol=1e-15)


def test_gated_rmsnorm_planted_mistakes_are_caught():
    """Mutations of the norm (on the CPU) fail the closed-form pins above."""
    dv = 8
    y = np.arange(1, 2 * dv + 1, dtype=np.float64).reshape(2, dv)
    z = np.full(y.shape, 3.0)
    ones = np.ones(dv)
    silu3 = 3.0 * SIGMOID_3

    def rms_of(out):
        return np.sqrt(np.mean(out * out, axis=-1))

    good = gdn_ref.gated_rmsnorm(y, z, ones, 0.0)
    np.testing.assert_allclose(rms_of(good), silu3, rtol=1e-12)
    sum_not_mean = y / np.sqrt(np.sum(y * y, axis=-1, keepdims=True)) * gdn_ref.silu(z)
    sigmoid_gate = y / np.sqrt(np.mean(y * y, axis=-1, keepdims=True)) / (1.0 + np.exp(-z))
    wrong_axis = y / np.sqrt(np.mean(y * y, axis=0, keepdims=True)) * gdn_ref.silu(z)
    for bad in (sum_not_mean, sigmoid_gate, wrong_axis):
        assert not np.allclose(rms_of(bad), silu3, rtol=1e-6)


# ------------------------------------------------------------------ retrieval order (NEXT-3)
# "7.6 Qwen3.5: the linear-attention hybrid", 7.6.2 writes S_t = a S_{t-1} + k [b (v - S_{t-1}^T k)]^T:
# the retrieval reads the state before the decay (order 1), where "Hugging Face Transformers:
# Qwen3.5-MoE series explained", 4.3 decays first (order 0).

def _rational_order1(q, k, v, a, b):
    """S_t = S (a I - b k k^T) + b v k^T, o = S q, value-major, exact rationals."""
    T, dk = len(k), len(k[0])
    dv = len(v[0])
    S = [[Fraction(0)] * dk for _ in range(dv)]
    outs = []
    for t in range(T):
        kt = [Fraction(x) for x in k[t]]
        P = [[(a[t] if i == j else Fraction(0)) - b[t] * kt[i] * kt[j] for j in range(dk)] for i in range(dk)]
        SP = [[sum(S[r][m] * P[m][c] for m in range(dk)) for c in range(dk)] for r in range(dv)]
        S = [[SP[r][c] + b[t] * Fraction(v[t][r]) * kt[c] for c in range(dk)] for r in range(dv)]
        outs.append([sum(S[r][c] * Fraction(q[t][c]) for c in range(dk)) for r in range(dv)])
    return outs, S


@pytest.mark.parametrize("seed", [0, 1])
def test_order1_exact_rational_bruteforce(seed):
    rng = np.random.default_rng(200 + seed)
    T, dk, dv = 5, 3, 2
    q = rng.integers(-8, 9, (T, dk)) / 8.0
    k = rng.integers(-8, 9, (T, dk)) / 8.0
    v = rng.integers(-8, 9, (T, dv)) / 4.0
    g32 = _f32(np.log(rng.uniform(0.5, 1.0, T)))
    b32 = _f32(rng.integers(1, 8, T) / 8.0)
    a_exact = [Fraction(math.exp(float(x))) for x in g32]
    b_exact = [Fraction(float(x)) for x in b32]
    outs, S = _rational_order1(q.tolist(), k.tolist(), v.tolist(), a_exact, b_exact)
    o_ex = np.array([[float(x) for x in r] for r in outs])
    S_ex = np.array([[float(x) for x in r] for r in S]).T
    cu = np.array([0, T], np.int32)
    for impl in (oracle.recurrence, gdn_ref.recurrence):
        o, fin = impl(q[:, None], k[:, None], v[:, None], g32[:, None], b32[:, None], cu, order=1)
        np.testing.assert_allclose(o[:, 0], o_ex, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(fin[0, 0], S_ex, rtol=1e-12, atol=1e-12)
    # with a < 1 the two orders differ; with a = 1 they coincide
    o0, _ = oracle.recurrence(q[:, None], k[:, None], v[:, None], g32[:, None], b32[:, None], cu, order=0)
    assert not np.allclose(o0[:, 0], o_ex, atol=1e-6)
    z = np.zeros_like(g32)
    oa, fa = oracle.recurrence(q[:, None], k[:, None], v[:, None], z[:, None], b32[:, None], cu, order=0)
    ob, fb = oracle.recurrence(q[:, None], k[:, None], v[:, None], z[:, None], b32[:, None], cu, order=1)
    np.testing.assert_array_equal(oa, ob)
    np.testing.assert_array_equal(fa, fb)


@pytest.mark.parametrize("L", [1, 63, 64, 65, 200])
def test_order1_chunked_equals_recurrent(L):
    q, k, v, g, b, cu, s0 = _rand_core(L, 2, 4, 16, 8, RNG)
    o_r, f_r = oracle.recurrence(q, k, v, g, b, cu, s0=s0, scale=0.7, order=1)
    o_c, f_c = gdn_ref.chunked(q, k, v, g, b, cu, s0=s0, scale=0.7, C=64, order=1)
    np.testing.assert_allclose(o_c, o_r, rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(f_c, f_r, rtol=1e-10, atol=1e-11)


def test_order1_c_matches_numpy_and_decode_equals_prefill():
    lengths = [3, 70, 0, 29]
    Hk, Hv, dk, dv = 2, 4, 8, 8
    C = 2 * Hk * dk + Hv * dv
    T = sum(lengths)
    x = _f32(RNG.standard_normal((T, C)))
    w = _f32(RNG.standard_normal((C, 4)) * 0.5)
    g = _f32(-np.logaddexp(0, RNG.standard_normal((T, Hv))))
    b = _f32(1 / (1 + np.exp(-RNG.standard_normal((T, Hv)))))
    s0 = _f32(RNG.standard_normal((4, Hv, dk, dv)) * 0.1)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    q, k, v, _ = oracle.prep(x, w, cu, Hk, Hv, dk, dv)
    oc, fc = oracle.recurrence(q, k, v, g, b, cu, s0=s0, scale=0.3, order=1)
    on, fn = gdn_ref.recurrence(q, k, v, g, b, cu, s0=s0, scale=0.3, order=1)
    np.testing.assert_allclose(oc, on, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(fc, fn, rtol=1e-10, atol=1e-12)
    # decode steps of the first sequence (3 tokens, zero conv history) equal its prefill
    st = s0[:1].astype(np.float64); cs = np.zeros((1, 3, C))
    outs = []
    for t in range(3):
        csf, stf = _f32(cs), _f32(st)
        ot, st, cs = oracle.decode(x[t:t + 1], w, csf, g[t:t + 1], b[t:t + 1], stf, Hk, Hv, dk, dv, scale=0.3,
                                   order=1)
        ot2, st2, _ = gdn_ref.decode_step(x[t:t + 1], w, csf, g[t:t + 1], b[t:t + 1], stf, Hk, Hv, dk, dv,
                                          scale=0.3, order=1)
        np.testing.assert_allclose(ot, ot2, rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(st, st2, rtol=1e-10, atol=1e-12)
        outs.append(ot[0])
    np.testing.assert_allclose(np.stack(outs), oc[:3], rtol=1e-5, atol=1e-6)
    np.testing.assert_allclose(st[0], fc[0], rtol=1e-5, atol=1e-6)


# ------------------------------------------------------------------ layer forward (NEXT-4)
# "7.6 Qwen3.5: the linear-attention hybrid", 7.6.1 (layer widths) and 7.6.2 (input
# projection -> causal conv -> L2 -> gated delta rule -> RMSNorm(y) * SiLU(z) -> output
# projection); the gate maps g = -softplus(a), beta = sigmoid(b) are the reading stated in
# the oracle.

def _bf16_vals(a):
    """fp64 array of bf16-representable values (torch's fp32 -> bf16 rounding)."""
    return torch.from_numpy(np.asarray(a, np.float32)).to(torch.bfloat16).to(torch.float64).numpy()


def test_layer_gates_closed_forms():
    a = np.array([0.0, math.log(math.e - 1.0), -40.0, 40.0])
    b = np.array([0.0, math.log(3.0), -math.log(3.0), 0.0])
    g, beta = gdn_ref.layer_gates(a, b)
    assert g.dtype == np.float32 and beta.dtype == np.float32
    np.testing.assert_allclose(g[:2], [-math.log(2.0), -1.0], rtol=1e-7)
    np.testing.assert_allclose(g[2], -math.exp(-40.0), rtol=1e-6)     # softplus(x) ~ e^x far left
    np.testing.assert_allclose(g[3], -40.0, rtol=1e-7)                  # softplus(x) ~ x far right
    np.testing.assert_allclose(beta[:3], [0.5, 0.75, 0.25], rtol=1e-7)
    x = np.random.default_rng(301).standard_normal(64) * 5
    gl, bl = gdn_ref.layer_gates(x, x)
    np.testing.assert_allclose(gl, -F.softplus(torch.from_numpy(x)).numpy(), rtol=1e-6)
    np.testing.assert_allclose(bl, torch.sigmoid(torch.from_numpy(x)).numpy(), rtol=1e-6)


def _layer_params(rng, E, Hk, Hv, dk, dv, scale_in=None):
    C = 2 * Hk * dk + Hv * dv
    rows = C + Hv * dv + 2 * Hv
    w_in = _bf16_vals(rng.standard_normal((rows, E)) * (scale_in or 1.0 / math.sqrt(E)))
    conv_w = _bf16_vals(rng.standard_normal((C, 4)) * 0.5)
    gamma = _bf16_vals(rng.uniform(0.5, 1.5, dv))
    w_out = _bf16_vals(rng.standard_normal((E, Hv * dv)) / math.sqrt(Hv * dv))
    return w_in, conv_w, gamma, w_out


def _both_layers(*args, **kw):
    out_c, fin_c, cs_c, _ = oracle.layer_prefill(*args, **kw)
    out_n, fin_n, cs_n = gdn_ref.layer_prefill(*args, **kw)
    return (out_c, fin_c, cs_c), (out_n, fin_n, cs_n)


def test_layer_single_token_closed_form():
    """One token from a zero state and zero conv history, eps = 0: the state after the
    token is beta v k^T, so o = scale beta (k.q) v, and the gated RMSNorm removes the
    scalar up to its sign: y_h = sign(scale beta k.q) v_h / rms(v_h) * gamma * SiLU(z_h)."""
    rng = np.random.default_rng(302)
    E, Hk, Hv, dk, dv = 24, 1, 2, 4, 4
    C = 2 * Hk * dk + Hv * dv
    w_in, conv_w, gamma, w_out = _layer_params(rng, E, Hk, Hv, dk, dv, scale_in=0.4)
    h = _bf16_vals(rng.standard_normal((1, E)))
    cu = np.array([0, 1], np.int32)
    proj = h @ w_in.T
    x = proj[0, :C]
    z = proj[0, C:C + Hv * dv].reshape(Hv, dv)
    beta = 1.0 / (1.0 + np.exp(-proj[0, C + Hv * dv + Hv:]))
    u = x * conv_w[:, 3]                      # only the newest tap sees a nonzero input
    act = u / (1.0 + np.exp(-u))
    qv, kv, vv = act[:dk], act[dk:2 * dk], act[2 * dk:].reshape(Hv, dv)
    scale = -0.75
    kq = np.dot(kv, qv)                       # the key head is shared by both value heads
    y = np.zeros((Hv, dv))
    for hh in range(Hv):
        s = np.sign(scale * beta[hh] * kq)
        y[hh] = s * vv[hh] / np.sqrt(np.mean(vv[hh] ** 2)) * gamma * (z[hh] / (1.0 + np.exp(-z[hh])))
    ref = y.reshape(1, Hv * dv) @ w_out.T
    for out, fin, cs in _both_layers(h, w_in, conv_w, gamma, w_out, cu, Hk, Hv, dk, dv, scale=scale, l2_eps=0.0,
                                     norm_eps=0.0):
        np.testing.assert_allclose(out, ref, rtol=1e-9, atol=1e-12)
        # final state beta v k^T / |k| (key-major), conv cache [0, 0, x]
        kn = kv / np.linalg.norm(kv)
        for hh in range(Hv):
            np.testing.assert_allclose(fin[0, hh], beta[hh].astype(np.float32) * np.outer(kn, vv[hh]),
                                       rtol=1e-6, atol=1e-12)
        np.testing.assert_allclose(cs[0], np.stack([np.zeros(C), np.zeros(C), x]), atol=0)


def _identity_layer_case(seed):
    """Identity input projection, selecting output projection: the layer reduces to the
    pinned conv prep, recurrence and gated RMSNorm on columns of the input, with the gates
    from the library's softplus and logistic functions."""
    rng = np.random.default_rng(seed)
    Hk, Hv, dk, dv = 1, 2, 8, 8
    C = 2 * Hk * dk + Hv * dv
    E = C + Hv * dv + 2 * Hv
    lengths = [5, 0, 9]
    T = sum(lengths)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    h = _bf16_vals(rng.standard_normal((T, E)))
    w_in = np.eye(E)
    _, conv_w, gamma, _ = _layer_params(rng, E, Hk, Hv, dk, dv)
    w_out = np.zeros((Hv * dv + 3, Hv * dv))
    w_out[:Hv * dv] = np.eye(Hv * dv)
    cs_in = _bf16_vals(rng.standard_normal((3, 3, C)))
    s0 = _f32(rng.standard_normal((3, Hv, dk, dv)) * 0.2)
    a_cols = torch.from_numpy(h[:, C + Hv * dv:C + Hv * dv + Hv])
    b_cols = torch.from_numpy(h[:, C + Hv * dv + Hv:])
    g = _f32(-F.softplus(a_cols).numpy())
    beta = _f32(torch.sigmoid(b_cols).numpy())
    q, k, v, cs_ref = oracle.prep(h[:, :C], conv_w, cu, Hk, Hv, dk, dv, cs_in=cs_in)
    o, fin_ref = oracle.recurrence(q, k, v, g, beta, cu, s0=s0, scale=0.5)
    y = oracle.gated_rmsnorm(o, h[:, C:C + Hv * dv].reshape(T, Hv, dv), gamma).reshape(T, Hv * dv)
    args = (h, w_in, conv_w, gamma, w_out, cu, Hk, Hv, dk, dv)
    kw = dict(cs_in=cs_in, s0=s0, scale=0.5)
    return args, kw, y, fin_ref, cs_ref


def test_layer_identity_projections_reduce_to_the_core():
    args, kw, y_ref, fin_ref, cs_ref = _identity_layer_case(303)
    n = y_ref.shape[1]
    for out, fin, cs in _both_layers(*args, **kw):
        np.testing.assert_allclose(out[:, :n], y_ref, rtol=1e-12, atol=1e-12)
        assert np.all(out[:, n:] == 0.0)
        np.testing.assert_allclose(fin, fin_ref, rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(cs, cs_ref, atol=0)


@pytest.mark.parametrize("order", [0, 1])
def test_layer_decode_continues_prefill(order):
    """Prefill of L + 1 tokens = prefill of L tokens, then one decode step of the layer."""
    rng = np.random.default_rng(304 + order)
    E, Hk, Hv, dk, dv = 40, 1, 2, 8, 8
    L = 6
    w_in, conv_w, gamma, w_out = _layer_params(rng, E, Hk, Hv, dk, dv)
    h = _bf16_vals(rng.standard_normal((L + 1, E)))
    s0 = _f32(rng.standard_normal((1, Hv, dk, dv)) * 0.2)
    kw = dict(scale=0.3, order=order)
    full, fin_full, cs_full, _ = oracle.layer_prefill(h, w_in, conv_w, gamma, w_out, np.array([0, L + 1], np.int32),
                                                      Hk, Hv, dk, dv, s0=s0, **kw)
    part, fin_part, cs_part, _ = oracle.layer_prefill(h[:L], w_in, conv_w, gamma, w_out, np.array([0, L], np.int32),
                                                      Hk, Hv, dk, dv, s0=s0, **kw)
    for impl in (oracle.layer_decode, gdn_ref.layer_decode):
        # the decode step takes the carried state as fp32 (the library's state type), so
        # agreement is to fp32 rounding of that state
        res = impl(h[L:], w_in, conv_w, gamma, w_out, cs_part, _f32(fin_part), Hk, Hv, dk, dv, **kw)
        np.testing.assert_allclose(res[0], full[L:], rtol=2e-6, atol=1e-8)
        np.testing.assert_allclose(res[1], fin_full, rtol=2e-6, atol=1e-8)
        np.testing.assert_allclose(res[2], cs_full, atol=0)
    np.testing.assert_allclose(part, full[:L], rtol=1e-12, atol=1e-14)


def test_layer_c_matches_numpy_reference():
    rng = np.random.default_rng(305)
    E, Hk, Hv, dk, dv = 48, 2, 4, 8, 8
    lengths = [7, 1, 12]
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    w_in, conv_w, gamma, w_out = _layer_params(rng, E, Hk, Hv, dk, dv)
    h = _bf16_vals(rng.standard_normal((sum(lengths), E)))
    (oc, fc, cc), (on, fn, cn) = _both_layers(h, w_in, conv_w, gamma, w_out, cu, Hk, Hv, dk, dv, scale=0.7)
    np.testing.assert_allclose(oc, on, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(fc, fn, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(cc, cn, atol=0)


def test_layer_planted_mistakes_are_caught():
    """Mutations of the layer's wiring (on the CPU) fail the pins above: v and z swapped
    fails the single-token closed form; the gate columns swapped or the decay sign
    flipped fails the identity-projection reduction (one token from a zero state never
    sees the decay, and beta cancels in the norm, so those need several tokens)."""
    rng = np.random.default_rng(306)
    E, Hk, Hv, dk, dv = 24, 1, 2, 4, 4
    w_in, conv_w, gamma, w_out = _layer_params(rng, E, Hk, Hv, dk, dv, scale_in=0.4)
    h = _bf16_vals(rng.standard_normal((1, E)))
    cu = np.array([0, 1], np.int32)
    kw1 = dict(scale=1.0, l2_eps=0.0, norm_eps=0.0)
    good1 = gdn_ref.layer_prefill(h, w_in, conv_w, gamma, w_out, cu, Hk, Hv, dk, dv, **kw1)[0]
    args, kw, y_ref, _, _ = _identity_layer_case(307)
    n = y_ref.shape[1]
    np.testing.assert_allclose(gdn_ref.layer_prefill(*args, **kw)[0][:, :n], y_ref, rtol=1e-12, atol=1e-12)
    split = gdn_ref.layer_split

    def swapped_zv(proj, *a):
        x, z, ga, gb = split(proj, *a)
        C = x.shape[1]
        x2 = np.concatenate([x[:, :C - z.shape[1]], z], axis=1)
        return x2, x[:, C - z.shape[1]:], ga, gb

    def swapped_gates(proj, *a):
        x, z, ga, gb = split(proj, *a)
        return x, z, gb, ga

    def flipped_decay(a, b):
        return (+gdn_ref.softplus(a)).astype(np.float32) * 0.1, gdn_ref.sigmoid(b).astype(np.float32)

    for name, fn, single in [("layer_split", swapped_zv, True), ("layer_split", swapped_gates, False),
                             ("layer_gates", flipped_decay, False)]:
        saved = getattr(gdn_ref, name)
        setattr(gdn_ref, name, fn)
        try:
            if single:
                bad = gdn_ref.layer_prefill(h, w_in, conv_w, gamma, w_out, cu, Hk, Hv, dk, dv, **kw1)[0]
                assert not np.allclose(bad, good1, rtol=1e-6), fn.__name__
            else:
                bad = gdn_ref.layer_prefill(*args, **kw)[0][:, :n]
                assert not np.allclose(bad, y_ref, rtol=1e-6), fn.__name__
        finally:
            setattr(gdn_ref, name, saved)
    # a transposed output projection does not even fit
    with pytest.raises(ValueError):
        gdn_ref.layer_prefill(h, w_in, conv_w, gamma, w_out.T.copy(), cu, Hk, Hv, dk, dv, **kw1)
