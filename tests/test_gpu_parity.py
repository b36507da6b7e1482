"""GPU parity: the HIP library (through its C ABI) against the fp64 CPU oracle.

Every case feeds the same seeded inputs to both sides and checks
max|gpu - oracle| <= tol * RMS(oracle) per output tensor (tol 1e-4 for the
fp32 element type, 2e-2 for bf16 inputs with an fp32 state); copies of input
values (conv caches) must match bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
from helpers import (TOL_BF16, TOL_F32, announce, assert_bf16_rounded, assert_parity, assert_parity_bf16_out,
                     err_ratio, f32np)
from hybrid_linear_attention_gated_amd import inputs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def gdn():
    import hybrid_linear_attention_gated_amd as m
    m.lib()
    return m


def _cuda(t):
    return None if t is None else t.to(DEV).contiguous()


def _rand(rng, shape, std=1.0):
    return rng.standard_normal(shape).astype(np.float32) * np.float32(std)


# ------------------------------------------------------------------ decode

@pytest.mark.parametrize("B,Hk,Hv,d,dtype", [(3, 2, 2, 16, "f32"), (5, 2, 4, 32, "bf16"), (4, 1, 2, 64, "f32"),
                                            (7, 2, 2, 128, "bf16"), (2, 2, 4, 128, "f32")])
def test_decode_small(gdn, B, Hk, Hv, d, dtype):
    announce(f"decode B={B} Hk={Hk} Hv={Hv} d={d} {dtype}")
    rng = np.random.default_rng(1000 + B + d)
    C = 2 * Hk * d + Hv * d
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    x = torch.from_numpy(_rand(rng, (B, C))).to(tdt)
    w = torch.from_numpy(_rand(rng, (C, 4), 0.5)).to(tdt)
    cs = torch.from_numpy(_rand(rng, (B, 3, C))).to(tdt)
    g = torch.from_numpy(np.log(rng.uniform(0.9, 1.0, (B, Hv))).astype(np.float32))
    b = torch.from_numpy((1 / (1 + np.exp(-rng.standard_normal((B, Hv))))).astype(np.float32))
    st = torch.from_numpy(_rand(rng, (B, Hv, d, d), 0.1))
    o_ref, st_ref, cs_ref = oracle.decode(f32np(x), f32np(w), f32np(cs), f32np(g), f32np(b), f32np(st),
                                          Hk, Hv, d, d, scale=0.5)
    csd, std = _cuda(cs), _cuda(st)
    o = gdn.decode_step(_cuda(x), _cuda(w), csd, _cuda(g), _cuda(b), std, Hk, Hv, d, d, scale=0.5)
    torch.cuda.synchronize()
    # decode computes in fp32 from the stored inputs whatever their element type
    assert_parity("o", f32np(o), o_ref, TOL_F32)
    assert_parity("state", f32np(std), st_ref, TOL_F32)
    np.testing.assert_array_equal(f32np(csd), cs_ref)


def test_decode256_full(gdn):
    announce("decode256 full config")
    wl = inputs.decode256()
    o_ref, st_ref, cs_ref = oracle.decode(f32np(wl.x), f32np(wl.conv_w), f32np(wl.conv_state), f32np(wl.g),
                                          f32np(wl.beta), f32np(wl.state), wl.Hk, wl.Hv, wl.dk, wl.dv)
    csd, std = _cuda(wl.conv_state), _cuda(wl.state)
    o = gdn.decode_step(_cuda(wl.x), _cuda(wl.conv_w), csd, _cuda(wl.g), _cuda(wl.beta), std,
                        wl.Hk, wl.Hv, wl.dk, wl.dv)
    torch.cuda.synchronize()
    assert_parity("o", f32np(o), o_ref, TOL_F32)
    assert_parity("state", f32np(std), st_ref, TOL_F32)
    np.testing.assert_array_equal(f32np(csd), cs_ref)


# ------------------------------------------------------------------ prep

@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f32", 16), ("bf16", 64)])
def test_prep_varlen(gdn, dtype, d):
    announce(f"prep varlen {dtype} d={d}")
    rng = np.random.default_rng(77 + d)
    lengths = [1, 2, 0, 37, 16, 100, 3]
    Hk, Hv = 2, 4
    C = 2 * Hk * d + Hv * d
    T = sum(lengths)
    N = len(lengths)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    x = torch.from_numpy(_rand(rng, (T, C))).to(tdt)
    w = torch.from_numpy(_rand(rng, (C, 4), 0.5)).to(tdt)
    cs = torch.from_numpy(_rand(rng, (N, 3, C))).to(tdt)
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lengths)]), dtype=torch.int32)
    q_ref, k_ref, v_ref, cs_ref = oracle.prep(f32np(x), f32np(w), cu.numpy(), Hk, Hv, d, d, cs_in=f32np(cs))
    cso = torch.empty((N, 3, C), dtype=tdt, device=DEV)
    q, k, v = gdn.conv_qk_prep(_cuda(x), _cuda(w), Hk, Hv, d, d, cu_seqlens=_cuda(cu), conv_state_in=_cuda(cs),
                               conv_state_out=cso)
    torch.cuda.synchronize()
    def check(name, gpu, ref):   # fp32 outputs computed in fp32 from the stored inputs
        assert_parity(name, f32np(gpu), ref, TOL_F32)
    check("q", q, q_ref)
    check("k", k, k_ref)
    check("v", v, v_ref)
    np.testing.assert_array_equal(f32np(cso), cs_ref)
    # conv_state_out may alias conv_state_in
    csd = _cuda(cs)
    gdn.conv_qk_prep(_cuda(x), _cuda(w), Hk, Hv, d, d, cu_seqlens=_cuda(cu), conv_state_in=csd, conv_state_out=csd)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(f32np(csd), cs_ref)
    # zero history when no conv_state_in is given
    q0, _, v0 = gdn.conv_qk_prep(_cuda(x), _cuda(w), Hk, Hv, d, d, cu_seqlens=_cuda(cu))
    q0_ref, _, v0_ref, _ = oracle.prep(f32np(x), f32np(w), cu.numpy(), Hk, Hv, d, d)
    torch.cuda.synchronize()
    check("q (zero history)", q0, q0_ref)
    check("v (zero history)", v0, v0_ref)


# ------------------------------------------------------------------ core (chunk prefill)

def _core_case(gdn, wl, math, heads=None, inplace=False):
    tol = TOL_F32 if math in ("f32", "f32_chunked") else TOL_BF16
    cu = wl.cu_seqlens
    o_ref, f_ref = oracle.recurrence(f32np(wl.q), f32np(wl.k), f32np(wl.v), f32np(wl.g), f32np(wl.beta),
                                     cu.numpy(), s0=None if wl.state is None else f32np(wl.state),
                                     scale=wl.scale, heads=heads)
    s0 = _cuda(wl.state)
    fin = s0 if (inplace and s0 is not None) else None
    o, f = gdn.chunk_prefill(_cuda(wl.q), _cuda(wl.k), _cuda(wl.v), _cuda(wl.g), _cuda(wl.beta),
                             cu_seqlens=_cuda(cu), initial_state=s0, final_state=fin, scale=wl.scale,
                             math=math)
    torch.cuda.synchronize()
    o, f = f32np(o), f32np(f)
    if heads is not None:
        o, o_ref = o[:, heads], o_ref[:, heads]
        f, f_ref = f[:, heads], f_ref[:, heads]
    assert_parity("o", o, o_ref, tol)
    assert_parity("final_state", f, f_ref, tol)


def test_tiny_f32_config(gdn):
    announce("tiny_f32 config (fp32 recurrent path)")
    _core_case(gdn, inputs.tiny_f32(), "f32")


def test_tiny_f32_config_chunked(gdn):
    """The tiny fp32 configuration through the chunked WY / UT form computed in fp32."""
    announce("tiny_f32 config (chunked form in fp32)")
    _core_case(gdn, inputs.tiny_f32(), "f32_chunked")


@pytest.mark.parametrize("dk,dv,lengths", [(16, 16, [70, 0, 5, 130]), (32, 32, [1, 63, 64, 65, 200]),
                                           (64, 32, [129, 0, 3]), (32, 64, [300]), (64, 64, [64, 191, 2])])
def test_core_f32_chunked_path(gdn, dk, dv, lengths):
    """Chunked fp32 path: ragged sequences (empty, single token, chunk edges, several chunks),
    two value heads per key head, random initial states, scale 0.5."""
    announce(f"core chunked fp32 path dk={dk} dv={dv} lengths={lengths}")
    wl = inputs.core_workload("chf32", 560 + dk + dv + len(lengths), lengths, 2, 4, dk, dv, random_states=True,
                              scale=0.5)
    _core_case(gdn, wl, "f32_chunked")


def test_core_f32_chunked_slow_decay_inplace(gdn):
    announce("core chunked fp32 path, slow decay, final state aliasing the initial state")
    wl = inputs.core_workload("chf32slow", 590, [500, 77], 1, 2, 32, 32, random_states=True, decay="slow")
    _core_case(gdn, wl, "f32_chunked", inplace=True)


@pytest.mark.parametrize("dk,dv", [(16, 16), (32, 32), (64, 32), (128, 128)])
def test_core_f32_path(gdn, dk, dv):
    announce(f"core fp32 recurrent path dk={dk} dv={dv}")
    wl = inputs.core_workload("rec", 500 + dk + dv, [70, 0, 5, 130], 2, 4, dk, dv, random_states=True, scale=0.5)
    _core_case(gdn, wl, "f32")


@pytest.mark.parametrize("lengths", [[1], [63], [64], [65], [127, 128, 129], [1, 0, 200, 64, 3, 0, 191]])
def test_core_chunked_lengths(gdn, lengths):
    announce(f"core chunked d=128 lengths={lengths}")
    wl = inputs.core_workload("chunk", 600 + len(lengths) + sum(lengths), lengths, 2, 2, 128, 128,
                              random_states=True)
    _core_case(gdn, wl, "mfma")


@pytest.mark.parametrize("d", [64, 128])
def test_core_chunked_gqa_scale_slow_decay(gdn, d):
    announce(f"core chunked GQA d={d} slow decay")
    wl = inputs.core_workload("gqa", 700 + d, [300, 129], 2, 4, d, d, random_states=True,
                              decay="slow", scale=d ** -0.5)
    _core_case(gdn, wl, "mfma")


@pytest.mark.parametrize("Hk,Hv,lengths", [(2, 8, [300, 129, 64, 1]), (1, 8, [190, 0, 65, 7, 128, 64, 33, 250])])
def test_core_chunked_key_groups(gdn, Hk, Hv, lengths):
    """Four and eight value heads per key head at d = 128 in the sequential schedule: only a
    key group's first value head stores K^T in its records and the state passes of the
    others copy it from there; the (sequence, head) units fill whole runs of 8 groups, so a
    group's units also share an XCD.  Every head against the oracle."""
    announce(f"core chunked d=128, {Hv // Hk} value heads per key head, lengths={lengths}")
    wl = inputs.core_workload("kgrp", 720 + Hv // Hk + len(lengths), lengths, Hk, Hv, 128, 128, random_states=True)
    _core_case(gdn, wl, "mfma")


def test_core_chunked_inplace_state(gdn):
    announce("core chunked in-place state (final_state aliases initial_state)")
    wl = inputs.core_workload("inplace", 801, [150, 64], 2, 2, 128, 128, random_states=True)
    _core_case(gdn, wl, "mfma", inplace=True)


def test_core_f32_inplace_state(gdn):
    announce("core fp32 in-place state")
    wl = inputs.core_workload("inplace32", 802, [40, 9], 2, 2, 32, 32, random_states=True)
    _core_case(gdn, wl, "f32", inplace=True)


# 275 packed chunks (T / 64 + N) over 7 sequences x 4 value heads (128 state-pass
# workgroups, half of MI355X's 256 compute units): the one-call prefill cuts them into four
# pipeline segments, so sequences start and end inside segments and span several of them;
# the batch also holds an empty and a one-token sequence.
SEGMENTED_LENGTHS = [9000, 1, 0, 5000, 65, 129, 3000]


def test_core_chunked_segmented_varlen(gdn):
    announce(f"core chunked, segmented pipeline, lengths={SEGMENTED_LENGTHS}")
    wl = inputs.core_workload("seg", 901, SEGMENTED_LENGTHS, 2, 4, 128, 128, random_states=True)
    _core_case(gdn, wl, "mfma")


def test_segmented_equals_split_phases(gdn):
    """The one-call prefill (segment pipeline over two streams) and the two split-phase
    calls (one launch each) run the same per-chunk arithmetic: results are bit-identical."""
    announce("one-call segmented prefill == chunk_prefill_local + chunk_prefill_state (bitwise)")
    wl = inputs.core_workload("seg2", 902, SEGMENTED_LENGTHS, 2, 4, 128, 128, random_states=True)
    q, k, v, g, b = (_cuda(t) for t in (wl.q, wl.k, wl.v, wl.g, wl.beta))
    cu, s0 = _cuda(wl.cu_seqlens), _cuda(wl.state)
    o1, f1 = gdn.chunk_prefill(q, k, v, g, b, cu_seqlens=cu, initial_state=s0, math="mfma")
    ws = torch.empty(gdn.workspace_size(wl.T, wl.N, wl.Hk, wl.Hv, wl.dk, wl.dv, "mfma"), dtype=torch.uint8,
                     device=DEV)
    o2 = torch.empty_like(o1)
    f2 = torch.empty_like(f1)
    gdn.chunk_prefill_local(q, k, v, g, b, ws, cu_seqlens=cu)
    gdn.chunk_prefill_state(ws, o2, wl.T, wl.Hk, wl.Hv, wl.dk, wl.dv, cu_seqlens=cu, initial_state=s0,
                            final_state=f2)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    assert torch.equal(f1, f2)


# more sequences than the state pass ranks by length (64), with ties, empties and ragged tails
MANY_LENGTHS = [int(x) for x in np.random.default_rng(4242).integers(0, 200, size=80)] + [0, 64, 64, 130]


def test_core_chunked_many_sequences(gdn):
    announce(f"core chunked d=128, {len(MANY_LENGTHS)} sequences (0..199 tokens)")
    wl = inputs.core_workload("many", 4300, MANY_LENGTHS, 2, 4, 128, 128, random_states=True)
    _core_case(gdn, wl, "mfma")


def test_core_chunked_many_sequences_d64(gdn):
    """The many-sequence case at d = 64: 336 (sequence, head) units, so the state pass's 672
    workgroups take several rounds of the compute units."""
    announce(f"core chunked d=64, {len(MANY_LENGTHS)} sequences, several rounds of state-pass workgroups")
    wl = inputs.core_workload("many64", 4302, MANY_LENGTHS, 2, 4, 64, 64, random_states=True)
    _core_case(gdn, wl, "mfma")


def test_core_chunked_ranked_sequences(gdn):
    """60 sequences (the state pass takes them longest first) with repeated chunk counts."""
    lengths = MANY_LENGTHS[:60]
    announce(f"core chunked d=64, {len(lengths)} sequences, longest-first state pass")
    wl = inputs.core_workload("ranked", 4301, lengths, 2, 2, 64, 64, random_states=True)
    _core_case(gdn, wl, "mfma")


def test_core_empty_sequences(gdn):
    announce("core: all sequences empty (T = 0)")
    H, d = 2, 128
    cu = torch.zeros(4, dtype=torch.int32, device=DEV)
    s0 = torch.randn((3, H, d, d), device=DEV)
    e = torch.empty((0, H, d), dtype=torch.float32, device=DEV)
    z = torch.empty((0, H), dtype=torch.float32, device=DEV)
    o, f = gdn.chunk_prefill(e, e, e, z, z, cu_seqlens=cu, initial_state=s0, math="mfma")
    torch.cuda.synchronize()
    assert o.shape == (0, H, d)
    assert torch.equal(f, s0)


# ------------------------------------------------------------------ end to end: prep + chunk prefill

def _e2e_reference(wl):
    """The oracle's prep and recurrence for a workload, over every value head."""
    cu = wl.cu_seqlens
    x32 = f32np(wl.x)
    q_r, k_r, v_r, cs_r = oracle.prep(x32, f32np(wl.conv_w), cu.numpy(), wl.Hk, wl.Hv, wl.dk, wl.dv,
                                      cs_in=None if wl.conv_state is None else f32np(wl.conv_state))
    del x32
    o_ref, f_ref = oracle.recurrence(q_r, k_r, v_r, f32np(wl.g), f32np(wl.beta), cu.numpy(),
                                     s0=None if wl.state is None else f32np(wl.state))
    return o_ref, f_ref, cs_r


# The long_64k reference (65536 tokens x 32 value heads, every head) takes the oracle about
# ten seconds on the machine's cores; the two long_64k tests share it.
_LONG_REF = {}


def _long_64k_reference(wl):
    if "ref" not in _LONG_REF:
        _LONG_REF["ref"] = _e2e_reference(wl)
    return _LONG_REF["ref"]


def _e2e(gdn, wl, fused=False, ref=None):
    cu = wl.cu_seqlens
    N = wl.N
    o_ref, f_ref, cs_r = _e2e_reference(wl) if ref is None else ref
    cso = torch.empty((N, 3, wl.conv_dim), dtype=torch.bfloat16, device=DEV)
    if fused:
        o, f = gdn.prefill(_cuda(wl.x), _cuda(wl.conv_w), _cuda(wl.g), _cuda(wl.beta), wl.Hk, wl.Hv, wl.dk, wl.dv,
                           cu_seqlens=_cuda(cu), conv_state_in=_cuda(wl.conv_state), conv_state_out=cso,
                           initial_state=_cuda(wl.state))
    else:
        q, k, v = gdn.conv_qk_prep(_cuda(wl.x), _cuda(wl.conv_w), wl.Hk, wl.Hv, wl.dk, wl.dv,
                                   cu_seqlens=_cuda(cu), conv_state_in=_cuda(wl.conv_state), conv_state_out=cso)
        o, f = gdn.chunk_prefill(q, k, v, _cuda(wl.g), _cuda(wl.beta), cu_seqlens=_cuda(cu),
                                 initial_state=_cuda(wl.state), math="mfma")
    torch.cuda.synchronize()
    assert_parity("o", f32np(o), o_ref, TOL_BF16)
    assert_parity("final_state", f32np(f), f_ref, TOL_BF16)
    np.testing.assert_array_equal(f32np(cso), cs_r)


def test_layer_4k_config(gdn):
    announce("layer_4k config end to end")
    _e2e(gdn, inputs.layer_4k())


def test_varlen8_config(gdn):
    announce("varlen8 config end to end")
    _e2e(gdn, inputs.varlen8())


def test_long_64k_config(gdn):
    announce("long_64k config end to end (all 32 value heads)")
    wl = inputs.long_64k()
    _e2e(gdn, wl, ref=_long_64k_reference(wl))


# ------------------------------------------------------------------ fused prep + chunk prefill (one call)

def test_fused_layer_4k_config(gdn):
    announce("layer_4k config, fused prefill")
    _e2e(gdn, inputs.layer_4k(), fused=True)


def test_fused_varlen8_config(gdn):
    announce("varlen8 config, fused prefill")
    _e2e(gdn, inputs.varlen8(), fused=True)


def test_fused_long_64k_config(gdn):
    announce("long_64k config, fused prefill (all 32 value heads)")
    wl = inputs.long_64k()
    _e2e(gdn, wl, fused=True, ref=_long_64k_reference(wl))
    _LONG_REF.clear()


# short and empty sequences, sequences shorter than the conv window, ragged tails
FUSED_LENGTHS = [1, 2, 0, 37, 64, 65, 3, 200, 129]


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f32", 128), ("bf16", 64), ("f32", 64)])
def test_fused_small_varlen(gdn, dtype, d):
    announce(f"fused prefill {dtype} d={d} lengths={FUSED_LENGTHS}")
    wl = inputs.prefill_workload("fused_small", 910 + d, FUSED_LENGTHS, 2, 4, d, random_states=True)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    x, w, cs = wl.x.to(tdt), wl.conv_w.to(tdt), wl.conv_state.to(tdt)
    cu = wl.cu_seqlens
    q_r, k_r, v_r, cs_r = oracle.prep(f32np(x), f32np(w), cu.numpy(), 2, 4, d, d, cs_in=f32np(cs))
    o_ref, f_ref = oracle.recurrence(q_r, k_r, v_r, f32np(wl.g), f32np(wl.beta), cu.numpy(), s0=f32np(wl.state),
                                     scale=0.3)
    cso = torch.empty(cs.shape, dtype=tdt, device=DEV)
    o, f = gdn.prefill(_cuda(x), _cuda(w), _cuda(wl.g), _cuda(wl.beta), 2, 4, d, d, cu_seqlens=_cuda(cu),
                       conv_state_in=_cuda(cs), conv_state_out=cso, initial_state=_cuda(wl.state), scale=0.3)
    torch.cuda.synchronize()
    assert_parity("o", f32np(o), o_ref, TOL_BF16)
    assert_parity("final_state", f32np(f), f_ref, TOL_BF16)
    np.testing.assert_array_equal(f32np(cso), cs_r)
    # conv_state_out aliasing conv_state_in, final_state aliasing initial_state
    csd, sd = _cuda(cs), _cuda(wl.state)
    o2, f2 = gdn.prefill(_cuda(x), _cuda(w), _cuda(wl.g), _cuda(wl.beta), 2, 4, d, d, cu_seqlens=_cuda(cu),
                         conv_state_in=csd, conv_state_out=csd, initial_state=sd, final_state=sd, scale=0.3)
    torch.cuda.synchronize()
    assert f2 is sd
    assert torch.equal(o2, o)
    assert torch.equal(sd, f)
    np.testing.assert_array_equal(f32np(csd), cs_r)
    # zero conv history and zero initial state
    q0, k0, v0, _ = oracle.prep(f32np(x), f32np(w), cu.numpy(), 2, 4, d, d)
    o0_ref, f0_ref = oracle.recurrence(q0, k0, v0, f32np(wl.g), f32np(wl.beta), cu.numpy())
    o0, f0 = gdn.prefill(_cuda(x), _cuda(w), _cuda(wl.g), _cuda(wl.beta), 2, 4, d, d, cu_seqlens=_cuda(cu))
    torch.cuda.synchronize()
    assert_parity("o (zero history)", f32np(o0), o0_ref, TOL_BF16)
    assert_parity("final_state (zero history)", f32np(f0), f0_ref, TOL_BF16)


def test_fused_segmented_varlen(gdn):
    """Enough chunks that the one call runs the segment pipeline (local and state
    passes on two streams)."""
    announce(f"fused prefill, segmented pipeline, lengths={SEGMENTED_LENGTHS}")
    _e2e(gdn, inputs.prefill_workload("fused_seg", 913, SEGMENTED_LENGTHS, 2, 4, 128, random_states=True),
         fused=True)


def test_fused_equals_split_phases(gdn):
    """gdn_prefill_local + gdn_chunk_prefill_state run the same kernels as one gdn_prefill
    call (which overlaps them segment by segment): results are bit-identical."""
    announce("one-call fused prefill == prefill_local + chunk_prefill_state (bitwise)")
    wl = inputs.prefill_workload("fused_split", 914, SEGMENTED_LENGTHS, 2, 4, 128, random_states=True)
    x, w, g, b, cu, s0, cs = (_cuda(t) for t in (wl.x, wl.conv_w, wl.g, wl.beta, wl.cu_seqlens, wl.state,
                                                 wl.conv_state))
    cso1, cso2 = torch.empty_like(cs), torch.empty_like(cs)
    o1, f1 = gdn.prefill(x, w, g, b, 2, 4, 128, 128, cu_seqlens=cu, conv_state_in=cs, conv_state_out=cso1,
                         initial_state=s0)
    ws = torch.empty(gdn.workspace_size(wl.T, wl.N, 2, 4, 128, 128, "mfma"), dtype=torch.uint8, device=DEV)
    o2, f2 = torch.empty_like(o1), torch.empty_like(f1)
    gdn.prefill_local(x, w, g, b, ws, 2, 4, 128, 128, cu_seqlens=cu, conv_state_in=cs, conv_state_out=cso2)
    gdn.chunk_prefill_state(ws, o2, wl.T, 2, 4, 128, 128, cu_seqlens=cu, initial_state=s0, final_state=f2)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    assert torch.equal(f1, f2)
    assert torch.equal(cso1, cso2)


def test_fused_all_empty(gdn):
    announce("fused prefill: all sequences empty (T = 0)")
    Hk, Hv, d = 2, 4, 128
    C = 2 * Hk * d + Hv * d
    cu = torch.zeros(4, dtype=torch.int32, device=DEV)
    x = torch.empty((0, C), dtype=torch.bfloat16, device=DEV)
    w = torch.randn((C, 4), device=DEV).to(torch.bfloat16)
    z = torch.empty((0, Hv), dtype=torch.float32, device=DEV)
    s0 = torch.randn((3, Hv, d, d), device=DEV)
    cs = torch.randn((3, 3, C), device=DEV).to(torch.bfloat16)
    cso = torch.empty_like(cs)
    o, f = gdn.prefill(x, w, z, z, Hk, Hv, d, d, cu_seqlens=cu, conv_state_in=cs, conv_state_out=cso,
                       initial_state=s0)
    torch.cuda.synchronize()
    assert o.shape == (0, Hv, d)
    assert torch.equal(f, s0)
    assert torch.equal(cso, cs)


# ------------------------------------------------------------------ decode steps == prefill

def test_decode_steps_equal_prefill(gdn):
    announce("16 decode steps vs one prefill of 16 tokens (both against the oracle)")
    wl = inputs.prefill_workload("dec_vs_pre", 900, [16], 2, 4, 64)
    C = wl.conv_dim
    q_r, k_r, v_r, _ = oracle.prep(f32np(wl.x), f32np(wl.conv_w), wl.cu_seqlens.numpy(), 2, 4, 64, 64)
    o_ref, f_ref = oracle.recurrence(q_r, k_r, v_r, f32np(wl.g), f32np(wl.beta), wl.cu_seqlens.numpy())
    cs = torch.zeros((1, 3, C), dtype=torch.bfloat16, device=DEV)
    st = torch.zeros((1, 4, 64, 64), dtype=torch.float32, device=DEV)
    xs, gs, bs, ws = _cuda(wl.x), _cuda(wl.g), _cuda(wl.beta), _cuda(wl.conv_w)
    outs = []
    for t in range(16):
        outs.append(gdn.decode_step(xs[t:t + 1].contiguous(), ws, cs, gs[t:t + 1].contiguous(),
                                    bs[t:t + 1].contiguous(), st, 2, 4, 64, 64))
    torch.cuda.synchronize()
    assert_parity("o (decode)", f32np(torch.cat(outs)), o_ref, TOL_BF16)
    assert_parity("state (decode)", f32np(st), f_ref, TOL_BF16)
    np.testing.assert_array_equal(f32np(cs)[0], f32np(wl.x)[-3:])


# ------------------------------------------------------------------ gated RMSNorm epilogue

def _check_norm_out(name, gpu, ref, dtype):
    if dtype == "bf16":
        assert_bf16_rounded(name, f32np(gpu), ref)
    else:
        assert_parity(name, f32np(gpu), ref, TOL_F32)


@pytest.mark.parametrize("dtype,dv,rows", [("bf16", 128, 1003), ("f32", 128, 1003), ("bf16", 16, 77),
                                           ("f32", 64, 130), ("bf16", 256, 65), ("f32", 32, 1)])
def test_gated_rmsnorm(gdn, dtype, dv, rows):
    announce(f"gated rmsnorm {dtype} dv={dv} rows={rows}")
    y = inputs.norm_rows(920 + dv, rows, dv)
    z, gamma = inputs.gate_inputs(921 + dv, (rows, dv), dv, dtype)
    ref = oracle.gated_rmsnorm(f32np(y), f32np(z), f32np(gamma), 1e-6)
    out = gdn.gated_rmsnorm(_cuda(y), _cuda(z), _cuda(gamma), eps=1e-6)
    torch.cuda.synchronize()
    _check_norm_out("out", out, ref, dtype)
    # in place over z, and (fp32) over y
    zd = _cuda(z)
    gdn.gated_rmsnorm(_cuda(y), zd, _cuda(gamma), eps=1e-6, out=zd)
    torch.cuda.synchronize()
    assert torch.equal(zd, out)
    if dtype == "f32":
        yd = _cuda(y)
        gdn.gated_rmsnorm(yd, _cuda(z), _cuda(gamma), eps=1e-6, out=yd)
        torch.cuda.synchronize()
        assert torch.equal(yd, out)


def test_gated_rmsnorm_empty(gdn):
    announce("gated rmsnorm, no rows")
    y = torch.empty((0, 4, 128), dtype=torch.float32, device=DEV)
    z = torch.empty((0, 4, 128), dtype=torch.bfloat16, device=DEV)
    out = gdn.gated_rmsnorm(y, z, torch.ones(128, dtype=torch.bfloat16, device=DEV))
    torch.cuda.synchronize()
    assert out.shape == (0, 4, 128)


@pytest.mark.parametrize("B,Hk,Hv,d,dtype", [(5, 2, 4, 32, "bf16"), (3, 2, 2, 128, "f32"), (256, 16, 16, 128, "bf16")])
def test_decode_gated(gdn, B, Hk, Hv, d, dtype):
    announce(f"gated decode B={B} Hk={Hk} Hv={Hv} d={d} {dtype}")
    dw = inputs.decode_workload("dec_gated", 930 + d, B, Hk, Hv, d)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    x, w, cs = dw.x.to(tdt), dw.conv_w.to(tdt), dw.conv_state.to(tdt)
    z, gamma = inputs.gate_inputs(931 + d, (B, Hv, d), d, dtype)
    o_ref, s_ref, cs_ref = oracle.decode(f32np(x), f32np(w), f32np(cs), f32np(dw.g), f32np(dw.beta),
                                         f32np(dw.state), Hk, Hv, d, d)
    ref = oracle.gated_rmsnorm(o_ref, f32np(z), f32np(gamma), 1e-6)
    st, csd = _cuda(dw.state), _cuda(cs)
    out = gdn.decode_step_gated(_cuda(x), _cuda(w), csd, _cuda(dw.g), _cuda(dw.beta), st, _cuda(z), _cuda(gamma),
                                Hk, Hv, d, d)
    torch.cuda.synchronize()
    _check_norm_out("out", out, ref, dtype)
    assert_parity("state", f32np(st), s_ref, TOL_F32)
    np.testing.assert_array_equal(f32np(csd), cs_ref)


def test_fused_prefill_then_gated_rmsnorm_layer_4k(gdn):
    """The layer_4k prefill (one gdn_prefill call) followed by the gated RMSNorm on its
    output, element by element against the oracle's prep, recurrence and norm."""
    announce("layer_4k: gdn_prefill + gated rmsnorm (bf16 gate / output)")
    wl = inputs.layer_4k()
    z, gamma = inputs.gate_inputs(940, (wl.T, wl.Hv, wl.dv), wl.dv, "bf16")
    q_r, k_r, v_r, _ = oracle.prep(f32np(wl.x), f32np(wl.conv_w), wl.cu_seqlens.numpy(), wl.Hk, wl.Hv, wl.dk,
                                   wl.dv)
    o_ref, _ = oracle.recurrence(q_r, k_r, v_r, f32np(wl.g), f32np(wl.beta), wl.cu_seqlens.numpy())
    ref = oracle.gated_rmsnorm(o_ref, f32np(z), f32np(gamma), 1e-6)
    o, _ = gdn.prefill(_cuda(wl.x), _cuda(wl.conv_w), _cuda(wl.g), _cuda(wl.beta), wl.Hk, wl.Hv, wl.dk, wl.dv,
                       cu_seqlens=_cuda(wl.cu_seqlens))
    out = gdn.gated_rmsnorm(o, _cuda(z), _cuda(gamma))
    torch.cuda.synchronize()
    # the norm's bf16 output is heavy tailed (elements of ~30 RMS): 2e-2 RMS plus its own
    # rounding, one bf16 ulp of each element
    assert_parity_bf16_out("out", f32np(out), ref, TOL_BF16)


# ------------------------------------------------------------------ retrieval order 1 (undecayed retrieval)

def _differs(name, gpu, other_ref, tol):
    """The order flag reaches the kernel: the result is far from the other order's reference."""
    r = err_ratio(gpu, other_ref)
    print(f"    {name} vs the other order: {r:.3e}", flush=True)
    assert r > 50 * tol


@pytest.mark.parametrize("math,d", [("mfma", 128), ("mfma", 64), ("f32", 128), ("f32", 32), ("f32_chunked", 32),
                                    ("f32_chunked", 64)])
def test_core_order1(gdn, math, d):
    lengths = [1, 63, 0, 200, 65, 129]
    announce(f"core order 1 ({math}, d={d}) lengths={lengths}")
    wl = inputs.core_workload("ord1", 950 + d, lengths, 2, 4, d, d, random_states=True, scale=0.5)
    tol = TOL_F32 if math in ("f32", "f32_chunked") else TOL_BF16
    args = (f32np(wl.q), f32np(wl.k), f32np(wl.v), f32np(wl.g), f32np(wl.beta), wl.cu_seqlens.numpy())
    o1, f1 = oracle.recurrence(*args, s0=f32np(wl.state), scale=0.5, order=1)
    o0, _ = oracle.recurrence(*args, s0=f32np(wl.state), scale=0.5, order=0)
    o, f = gdn.chunk_prefill(_cuda(wl.q), _cuda(wl.k), _cuda(wl.v), _cuda(wl.g), _cuda(wl.beta),
                             cu_seqlens=_cuda(wl.cu_seqlens), initial_state=_cuda(wl.state), scale=0.5, math=math,
                             order=1)
    torch.cuda.synchronize()
    assert_parity("o", f32np(o), o1, tol)
    assert_parity("final_state", f32np(f), f1, tol)
    _differs("o", f32np(o), o0, tol)


def test_fused_prefill_order1(gdn):
    announce(f"fused prefill order 1, lengths={FUSED_LENGTHS}")
    wl = inputs.prefill_workload("fused_ord1", 960, FUSED_LENGTHS, 2, 4, 128, random_states=True)
    cu = wl.cu_seqlens
    q_r, k_r, v_r, cs_r = oracle.prep(f32np(wl.x), f32np(wl.conv_w), cu.numpy(), 2, 4, 128, 128,
                                      cs_in=f32np(wl.conv_state))
    o1, f1 = oracle.recurrence(q_r, k_r, v_r, f32np(wl.g), f32np(wl.beta), cu.numpy(), s0=f32np(wl.state), order=1)
    cso = torch.empty(wl.conv_state.shape, dtype=torch.bfloat16, device=DEV)
    o, f = gdn.prefill(_cuda(wl.x), _cuda(wl.conv_w), _cuda(wl.g), _cuda(wl.beta), 2, 4, 128, 128,
                       cu_seqlens=_cuda(cu), conv_state_in=_cuda(wl.conv_state), conv_state_out=cso,
                       initial_state=_cuda(wl.state), order=1)
    torch.cuda.synchronize()
    assert_parity("o", f32np(o), o1, TOL_BF16)
    assert_parity("final_state", f32np(f), f1, TOL_BF16)
    np.testing.assert_array_equal(f32np(cso), cs_r)


@pytest.mark.parametrize("gated", [False, True])
def test_decode_order1(gdn, gated):
    announce(f"decode order 1 (gated={gated})")
    B, Hk, Hv, d = 6, 2, 4, 64
    dw = inputs.decode_workload("dec_ord1", 970, B, Hk, Hv, d)
    args = (f32np(dw.x), f32np(dw.conv_w), f32np(dw.conv_state), f32np(dw.g), f32np(dw.beta), f32np(dw.state),
            Hk, Hv, d, d)
    o1, s1, cs1 = oracle.decode(*args, order=1)
    o0, _, _ = oracle.decode(*args, order=0)
    st, cs = _cuda(dw.state), _cuda(dw.conv_state)
    if gated:
        z, gamma = inputs.gate_inputs(971, (B, Hv, d), d, "bf16")
        out = gdn.decode_step_gated(_cuda(dw.x), _cuda(dw.conv_w), cs, _cuda(dw.g), _cuda(dw.beta), st, _cuda(z),
                                    _cuda(gamma), Hk, Hv, d, d, order=1)
        torch.cuda.synchronize()
        assert_bf16_rounded("out", f32np(out), oracle.gated_rmsnorm(o1, f32np(z), f32np(gamma), 1e-6))
    else:
        o = gdn.decode_step(_cuda(dw.x), _cuda(dw.conv_w), cs, _cuda(dw.g), _cuda(dw.beta), st, Hk, Hv, d, d, order=1)
        torch.cuda.synchronize()
        assert_parity("o", f32np(o), o1, TOL_F32)
        _differs("o", f32np(o), o0, TOL_F32)
    assert_parity("state", f32np(st), s1, TOL_F32)
    np.testing.assert_array_equal(f32np(cs), cs1)


# ------------------------------------------------------------------ concurrent schedule

def test_concurrent_schedule_equals_split_phases(gdn):
    """One sequence of 8000 tokens x 4 value heads takes the concurrent schedule (the
    state pass waits for records the chunk-local kernel publishes while it runs).  Three
    different batches in a row on one workspace, each bit-identical to the split-phase
    calls and the first against the oracle, so a record read before it was written (or a
    stale one from the previous batch) shows.  The workspace starts with every byte 0xff
    and then holds the previous batch's ready flags: a flag counts only with the call's own
    value."""
    announce("concurrent schedule: T=8000, Hk=2, Hv=4, three batches on one workspace")
    T, Hk, Hv, d = 8000, 2, 4, 128
    ws = torch.full((gdn.workspace_size(T, 1, Hk, Hv, d, d, "mfma"),), 255, dtype=torch.uint8, device=DEV)
    for it in range(3):
        wl = inputs.prefill_workload("conc", 980 + it, [T], Hk, Hv, d, random_states=True)
        x, w, g, b, s0, cs = (_cuda(t) for t in (wl.x, wl.conv_w, wl.g, wl.beta, wl.state, wl.conv_state))
        o1, f1 = gdn.prefill(x, w, g, b, Hk, Hv, d, d, conv_state_in=cs, initial_state=s0, workspace=ws)
        ws2 = torch.empty_like(ws)
        o2, f2 = torch.empty_like(o1), torch.empty_like(f1)
        gdn.prefill_local(x, w, g, b, ws2, Hk, Hv, d, d, conv_state_in=cs)
        gdn.chunk_prefill_state(ws2, o2, T, Hk, Hv, d, d, initial_state=s0, final_state=f2)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2), f"batch {it}: o differs from the split phases"
        assert torch.equal(f1, f2), f"batch {it}: final state differs from the split phases"
        if it == 0:
            cu = wl.cu_seqlens.numpy()
            q_r, k_r, v_r, _ = oracle.prep(f32np(wl.x), f32np(wl.conv_w), cu, Hk, Hv, d, d,
                                           cs_in=f32np(wl.conv_state))
            o_ref, f_ref = oracle.recurrence(q_r, k_r, v_r, f32np(wl.g), f32np(wl.beta), cu, s0=f32np(wl.state))
            assert_parity("o", f32np(o1), o_ref, TOL_BF16)
            assert_parity("final_state", f32np(f1), f_ref, TOL_BF16)


@pytest.mark.parametrize("alias,dtype", [(False, "bf16"), (True, "bf16"), (True, "f32")])
def test_concurrent_schedule_conv_cache(gdn, alias, dtype):
    """Concurrent schedule with a conv cache to write (the state pass writes it): 4
    sequences of 2, 0, 7998 and 1 tokens, 2 key / 4 value heads (16 state units, 129
    chunks x 4 heads: the state pass holds a quarter of the compute units), the output
    cache separate from or aliasing the input cache.  o and the final state bit-identical
    to the split-phase calls; the cache equal to the oracle's bit for bit (the short and
    empty sequences take rows from the input cache).  x, conv_w and the caches in bf16
    or fp32 (the same values)."""
    announce(f"concurrent schedule conv cache: lengths [2, 0, 7998, 1], Hk=2, Hv=4, alias={alias} {dtype}")
    Hk, Hv, d = 2, 4, 128
    wl = inputs.prefill_workload("conc_cache", 1010 + int(alias), [2, 0, 7998, 1], Hk, Hv, d, random_states=True)
    T, cu = wl.T, _cuda(wl.cu_seqlens)
    x, w, g, b, s0 = (_cuda(t) for t in (wl.x, wl.conv_w, wl.g, wl.beta, wl.state))
    cs_in = _cuda(wl.conv_state)
    if dtype == "f32":
        x, w, cs_in = x.float(), w.float(), cs_in.float()
    cs_out = cs_in if alias else torch.empty_like(cs_in)
    ws = torch.empty(gdn.workspace_size(T, 4, Hk, Hv, d, d, "mfma"), dtype=torch.uint8, device=DEV)
    ws2 = torch.empty_like(ws)
    o2 = torch.empty((T, Hv, d), dtype=torch.float32, device=DEV)
    f2 = torch.empty_like(s0)
    # split phases first (they read the input cache before the concurrent call may overwrite it)
    gdn.prefill_local(x, w, g, b, ws2, Hk, Hv, d, d, cu_seqlens=cu, conv_state_in=cs_in)
    gdn.chunk_prefill_state(ws2, o2, T, Hk, Hv, d, d, cu_seqlens=cu, initial_state=s0, final_state=f2)
    o1, f1 = gdn.prefill(x, w, g, b, Hk, Hv, d, d, cu_seqlens=cu, conv_state_in=cs_in, conv_state_out=cs_out,
                         initial_state=s0, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2), "o differs from the split phases"
    assert torch.equal(f1, f2), "final state differs from the split phases"
    _, _, _, cs_ref = oracle.prep(f32np(wl.x), f32np(wl.conv_w), wl.cu_seqlens.numpy(), Hk, Hv, d, d,
                                  cs_in=f32np(wl.conv_state))
    np.testing.assert_array_equal(f32np(cs_out), cs_ref)


@pytest.mark.gpu
def test_concurrent_schedule_from_several_streams(gdn):
    """Four caller streams each start a concurrent-schedule prefill (own workspace, inputs
    and outputs) before any of them has finished; every result is bit-identical to the
    split-phase calls on the default stream.  Covers the ordering of the one-launch
    concurrent schedule across caller streams (the first change of stream, then the
    event that a call from another stream waits for)."""
    announce("concurrent schedule: T=8000, Hk=2, Hv=4, four caller streams")
    T, Hk, Hv, d, n = 8000, 2, 4, 128, 4
    wsz = gdn.workspace_size(T, 1, Hk, Hv, d, d, "mfma")
    cases = []
    for j in range(n):
        wl = inputs.prefill_workload("conc_streams", 990 + j, [T], Hk, Hv, d, random_states=True)
        x, w, g, b, s0, cs = (_cuda(t) for t in (wl.x, wl.conv_w, wl.g, wl.beta, wl.state, wl.conv_state))
        ws = torch.empty(wsz, dtype=torch.uint8, device=DEV)
        o_ref = torch.empty((T, Hv, d), dtype=torch.float32, device=DEV)
        f_ref = torch.empty((1, Hv, d, d), dtype=torch.float32, device=DEV)
        gdn.prefill_local(x, w, g, b, ws, Hk, Hv, d, d, conv_state_in=cs)
        gdn.chunk_prefill_state(ws, o_ref, T, Hk, Hv, d, d, initial_state=s0, final_state=f_ref)
        cases.append(dict(x=x, w=w, g=g, b=b, s0=s0, cs=cs, ws=torch.empty(wsz, dtype=torch.uint8, device=DEV),
                          o=torch.empty_like(o_ref), f=torch.empty_like(f_ref), o_ref=o_ref, f_ref=f_ref))
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(device=DEV) for _ in range(n)]
    for s, c in zip(streams, cases):
        with torch.cuda.stream(s):
            gdn.prefill(c["x"], c["w"], c["g"], c["b"], Hk, Hv, d, d, conv_state_in=c["cs"], initial_state=c["s0"],
                        o=c["o"], final_state=c["f"], workspace=c["ws"])
    torch.cuda.synchronize()
    for j, c in enumerate(cases):
        assert torch.equal(c["o"], c["o_ref"]), f"stream {j}: o differs from the split phases"
        assert torch.equal(c["f"], c["f_ref"]), f"stream {j}: final state differs from the split phases"


# ------------------------------------------------------------------ failure reporting and graph capture

def test_concurrent_wait_bound_reports_timeout(gdn):
    """The concurrent schedule's state pass with its record waits bounded to one sleep
    (set in the workspace header from the host): the first record is not published that
    fast, so the state pass stops waiting, writes NaN outputs and final states and sets
    the workspace status to GDN_ERR_TIMEOUT; the chunk-local kernel runs to its end.  With
    the default bound restored, the same workspace gives the split phases' result and the
    status reads GDN_OK."""
    announce("concurrent schedule with a one-sleep wait bound: T=8000, Hk=2, Hv=4")
    T, Hk, Hv, d = 8000, 2, 4, 128
    wl = inputs.prefill_workload("timeout", 1020, [T], Hk, Hv, d, random_states=True)
    x, w, g, b, s0 = (_cuda(t) for t in (wl.x, wl.conv_w, wl.g, wl.beta, wl.state))
    ws = torch.zeros(gdn.workspace_size(T, 1, Hk, Hv, d, d, "mfma"), dtype=torch.uint8, device=DEV)
    assert gdn.prefill_workspace_status(ws) == gdn.GDN_OK
    gdn.set_wait_bound(ws, 1)
    o1, f1 = gdn.prefill(x, w, g, b, Hk, Hv, d, d, initial_state=s0, workspace=ws)
    torch.cuda.synchronize()
    assert gdn.prefill_workspace_status(ws) == gdn.GDN_ERR_TIMEOUT
    assert torch.isnan(f1).any(), "the final state of a failed call is NaN"
    assert torch.isnan(o1).any(), "the outputs of a failed call are NaN"
    assert gdn.prefill_workspace_status(ws) == gdn.GDN_OK   # the query cleared it
    gdn.set_wait_bound(ws, None)
    o2, f2 = gdn.prefill(x, w, g, b, Hk, Hv, d, d, initial_state=s0, workspace=ws)
    ws_ref = torch.empty_like(ws)
    o_ref, f_ref = torch.empty_like(o2), torch.empty_like(f2)
    gdn.prefill_local(x, w, g, b, ws_ref, Hk, Hv, d, d)
    gdn.chunk_prefill_state(ws_ref, o_ref, T, Hk, Hv, d, d, initial_state=s0, final_state=f_ref)
    torch.cuda.synchronize()
    assert gdn.prefill_workspace_status(ws) == gdn.GDN_OK
    assert torch.equal(o2, o_ref) and torch.equal(f2, f_ref)


@pytest.mark.parametrize("T", [200, 8000])
def test_state_overflow_reports_nonfinite(gdn, T):
    """An initial state beyond the fp16 range of the state pass's operands (+-65504) makes
    the outputs non-finite; the status word says so (sequential schedule at T = 200, the
    concurrent one at T = 8000)."""
    announce(f"state beyond the fp16 range, T={T}: status GDN_ERR_NONFINITE")
    Hk, Hv, d = 2, 4, 128
    wl = inputs.prefill_workload("overflow", 1030, [T], Hk, Hv, d, random_states=True)
    s0 = wl.state.clone()
    s0[0, 1, 5, 7] = 1.0e6
    ws = torch.zeros(gdn.workspace_size(T, 1, Hk, Hv, d, d, "mfma"), dtype=torch.uint8, device=DEV)
    o, f = gdn.prefill(_cuda(wl.x), _cuda(wl.conv_w), _cuda(wl.g), _cuda(wl.beta), Hk, Hv, d, d,
                       initial_state=_cuda(s0), workspace=ws)
    torch.cuda.synchronize()
    assert not bool(torch.isfinite(o).all()) or not bool(torch.isfinite(f).all())
    assert gdn.prefill_workspace_status(ws) == gdn.GDN_ERR_NONFINITE
    # a finite call on the same workspace reports nothing
    gdn.prefill(_cuda(wl.x), _cuda(wl.conv_w), _cuda(wl.g), _cuda(wl.beta), Hk, Hv, d, d,
                initial_state=_cuda(wl.state), workspace=ws)
    assert gdn.prefill_workspace_status(ws) == gdn.GDN_OK


_DEBUG_CHILD = r"""
import sys, torch
sys.path.insert(0, sys.argv[1])
import hybrid_linear_attention_gated_amd as gdn
from hybrid_linear_attention_gated_amd import inputs
dev = "cuda:0"
wl = inputs.prefill_workload("dbg", 1040, [70, 0, 130], 2, 4, 128, random_states=True)
x, w, g, b, s0 = (t.to(dev) for t in (wl.x, wl.conv_w, wl.g, wl.beta, wl.state))
cu = wl.cu_seqlens.to(dev)
o, f = gdn.prefill(x, w, g, b, 2, 4, 128, 128, cu_seqlens=cu, initial_state=s0)
torch.cuda.synchronize()
bad = torch.tensor([0, 70, 60, 200], dtype=torch.int32, device=dev)   # decreasing
codes = []
for cus, st in ((bad, s0), (cu, None)):
    if st is None:
        st = s0.clone()
        st[2, 2, 3, 4] = 1.0e6   # sequence 2 (130 tokens; sequence 1 is empty)
    try:
        gdn.prefill(x, w, g, b, 2, 4, 128, 128, cu_seqlens=cus, initial_state=st)
        codes.append(0)
    except gdn.GdnError as e:
        codes.append(e.status)
print("codes", codes[0], codes[1], flush=True)
"""


def test_debug_check_environment(gdn, tmp_path):
    """With GDN_DEBUG_CHECK=1 (a child process: the library reads it once), a prefill call
    returns GDN_ERR_BAD_SHAPE for a decreasing cu_seqlens before launching anything, and
    GDN_ERR_NONFINITE itself for a state beyond the fp16 range."""
    import os
    import subprocess
    import sys
    announce("GDN_DEBUG_CHECK=1 in a child process: bad cu_seqlens, non-finite output")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    env = dict(os.environ, GDN_DEBUG_CHECK="1")
    r = subprocess.run([sys.executable, "-c", _DEBUG_CHILD, root], env=env, capture_output=True, text=True,
                       timeout=100)
    print(r.stdout[-2000:], r.stderr[-2000:], flush=True)
    assert r.returncode == 0
    assert "codes 2 9" in r.stdout


def test_graph_capture_of_layer_4k_prefill(gdn):
    """gdn_prefill at the layer_4k shape captured into a HIP graph (torch.cuda.graph): under
    capture the concurrent schedule's one launch follows a kernel that clears its ready flags,
    and every replay uses the graph's own flag value.  The graph is replayed three times with
    other eager work and synchronisations in between; every replay is bit-identical to the
    eager call, and so is an eager call on the same workspace after the replays (the flags
    the replays left do not pass for its own)."""
    announce("graph capture of gdn_prefill at layer_4k, three replays")
    wl = inputs.layer_4k()
    x, w, g, b = (_cuda(t) for t in (wl.x, wl.conv_w, wl.g, wl.beta))
    T, Hk, Hv, d = wl.T, wl.Hk, wl.Hv, wl.dk
    ws = torch.empty(gdn.workspace_size(T, 1, Hk, Hv, d, d, "mfma"), dtype=torch.uint8, device=DEV)
    o = torch.empty((T, Hv, d), dtype=torch.float32, device=DEV)
    f = torch.empty((1, Hv, d, d), dtype=torch.float32, device=DEV)
    cso = torch.empty((1, 3, wl.conv_dim), dtype=torch.bfloat16, device=DEV)
    o_ref, f_ref = gdn.prefill(x, w, g, b, Hk, Hv, d, d, conv_state_out=cso)
    cso_ref = cso.clone()
    torch.cuda.synchronize()
    side = torch.cuda.Stream(device=DEV)
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            gdn.prefill(x, w, g, b, Hk, Hv, d, d, conv_state_out=cso, o=o, final_state=f, workspace=ws)
    torch.cuda.synchronize()
    for rep in range(3):
        o.zero_()
        f.zero_()
        cso.zero_()
        junk = torch.randn(1 << 20, device=DEV).sum()   # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref), f"replay {rep}: o differs from the eager call"
        assert torch.equal(f, f_ref), f"replay {rep}: final state differs from the eager call"
        assert torch.equal(cso, cso_ref), f"replay {rep}: conv cache differs"
        del junk
    o.zero_()
    f.zero_()
    gdn.prefill(x, w, g, b, Hk, Hv, d, d, conv_state_out=cso, o=o, final_state=f, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(f, f_ref), "eager call after the replays differs"
    assert gdn.prefill_workspace_status(ws) == gdn.GDN_OK
