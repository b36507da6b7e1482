"""GPU parity of the linear-attention layer forward (projections, gates, core, gated
RMSNorm) through the C ABI against the fp64 CPU oracle.

Projection outputs the GPU stores in bf16 are checked element by element against the
fp64 products (within one bf16 rounding, see helpers.assert_bf16_rounded); the gates to
fp32 accuracy.  The layer cases draw their inputs and weights from N(0, 1)-scaled
distributions with no constraint (the bench's own layer inputs among them) and hold the
final states to 2e-2 RMS (bf16 weights and layer input, fp32 state) and the bf16 layer
output to 2e-2 RMS plus its own rounding (one bf16 ulp of each element).
The oracle rounds nothing between the input projection and the output: inside the
layer the pre-conv q|k|v and the conv caches are fp32 on the GPU (the recurrent state
amplifies one-ulp changes of its inputs), and the gate and the normalised output that
enter the output projection are bf16, whose roundings the 2e-2 bar covers.  One case
draws the input and the input projection on grids on which every projected value is
exact in fp32, as an extra check of the same path.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import gdn_ref
from helpers import TOL_BF16, TOL_F32, announce, assert_bf16_rounded, assert_parity, assert_parity_bf16_out, f32np
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


def _bf16_tensor(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)


def _sample_rows(M, n, seed):
    rng = np.random.default_rng(seed)
    rows = set(rng.choice(M, size=min(n, M), replace=False).tolist())
    rows.update({0, M - 1, min(M - 1, 255), min(M - 1, 256)})
    return np.array(sorted(rows))


# ------------------------------------------------------------------ projections

# the 256 x 256 tile runs when its tiles alone fill the chip (M, N >= 4096 here) and takes k
# 64 deep per stage, two stages per loop pass: K = 64, 128, 192 give one, two and three stages
# (a lone stage, one pass, a pass and a tail); the 128 x 128 tile takes k 128 deep when K allows
# (K = 128, 1024, 2048) and 64 deep otherwise (K = 64, 192)
@pytest.mark.parametrize("M,N,K", [(1, 16, 64), (77, 100, 128), (300, 260, 192), (513, 1028, 1024),
                                   (0, 64, 64), (4100, 4100, 128), (4096, 1024, 2048), (4096, 4096, 64),
                                   (4100, 4108, 192)])
def test_linear(gdn, M, N, K):
    announce(f"linear M={M} N={N} K={K}")
    rng = np.random.default_rng(7000 + M + N + K)
    a = _bf16_tensor(rng.standard_normal((M, K)))
    w = _bf16_tensor(rng.standard_normal((N, K)) / np.sqrt(K))
    y = gdn.linear(_cuda(a), _cuda(w))
    torch.cuda.synchronize()
    assert y.shape == (M, N)
    if M == 0:
        return
    rows = _sample_rows(M, 96, M) if M * N > 1 << 22 else np.arange(M)
    ref = f32np(a)[rows].astype(np.float64) @ f32np(w).astype(np.float64).T
    assert_bf16_rounded("y", f32np(y)[rows], ref)


@pytest.mark.parametrize("T,E,Hk,Hv,d", [(300, 128, 1, 2, 64), (257, 256, 2, 4, 64), (100, 1024, 16, 32, 128),
                                         (4096, 1024, 16, 16, 128)])
def test_in_proj(gdn, T, E, Hk, Hv, d):
    announce(f"in_proj T={T} E={E} Hk={Hk} Hv={Hv} d={d}")
    wts = inputs.layer_weights(600 + Hv, E, Hk, Hv, d, d)
    h = inputs.layer_hidden(610 + T, T, E)
    x, z, g, beta = gdn.in_proj(_cuda(h), _cuda(wts.w_in), Hk, Hv, d, d)
    torch.cuda.synchronize()
    rows = _sample_rows(T, 128, T) if T > 512 else np.arange(T)
    proj = f32np(h)[rows].astype(np.float64) @ f32np(wts.w_in).astype(np.float64).T
    xp, zp, ap, bp = gdn_ref.layer_split(proj, Hk, Hv, d, d)
    g_ref, b_ref = gdn_ref.layer_gates(ap, bp)
    assert_bf16_rounded("x", f32np(x)[rows], xp)
    assert_bf16_rounded("z", f32np(z)[rows], zp)
    np.testing.assert_allclose(f32np(g)[rows], g_ref, rtol=2e-5, atol=2e-6)
    np.testing.assert_allclose(f32np(beta)[rows], b_ref, rtol=2e-5, atol=2e-6)


# ------------------------------------------------------------------ layer prefill

def _layer_case(gdn, lengths, E, Hk, Hv, d, seed, caches, scale, order=0, exact=False, hidden_seed=None):
    T = int(sum(lengths))
    N = len(lengths)
    cu = torch.from_numpy(np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32))
    wts = inputs.layer_weights(seed, E, Hk, Hv, d, d, exact=exact)
    h = inputs.layer_hidden(seed + 1 if hidden_seed is None else hidden_seed, T, E, exact=exact)
    cs_in, s0 = inputs.layer_caches(seed + 2, N, Hk, Hv, d, d) if caches else (None, None)
    out_ref, fin_ref, cs_ref, _ = oracle.layer_prefill(
        f32np(h), f32np(wts.w_in), f32np(wts.conv_w), f32np(wts.gamma), f32np(wts.w_out), cu.numpy(), Hk, Hv, d, d,
        cs_in=None if cs_in is None else f32np(cs_in), s0=None if s0 is None else f32np(s0), scale=scale,
        order=order)
    C = 2 * Hk * d + Hv * d
    cs_out = torch.empty((N, 3, C), dtype=torch.float32, device=DEV)
    out, fin = gdn.layer_prefill(_cuda(h), _cuda(wts.w_in), _cuda(wts.conv_w), _cuda(wts.gamma), _cuda(wts.w_out),
                                 Hk, Hv, d, d, cu_seqlens=_cuda(cu) if N > 1 else None,
                                 conv_state_in=_cuda(cs_in), conv_state_out=cs_out, initial_state=_cuda(s0),
                                 scale=scale, order=order)
    torch.cuda.synchronize()
    return (out, fin, cs_out), (out_ref, fin_ref, cs_ref)


def _check_layer(out, fin, cs, out_ref, fin_ref, cs_ref):
    # the layer output is stored in bf16: its own rounding (one bf16 ulp at most) on top of
    # the 2e-2 RMS bar
    assert_parity_bf16_out("out", f32np(out), out_ref, TOL_BF16)
    assert_parity("final state", f32np(fin), fin_ref, TOL_BF16)
    # the conv cache holds fp32 projections (or copies of the incoming cache)
    assert_parity("conv cache", f32np(cs), cs_ref, TOL_F32)


@pytest.mark.parametrize("order", [0, 1])
def test_layer_prefill_small_varlen(gdn, order):
    announce(f"layer prefill varlen small order={order}")
    gpu, ref = _layer_case(gdn, [70, 0, 150, 1], 128, 1, 2, 64, 620, True, 0.125, order)
    _check_layer(*gpu, *ref)


def test_layer_prefill_gqa_128(gdn):
    announce("layer prefill Hk=2 Hv=4 d=128 two sequences")
    gpu, ref = _layer_case(gdn, [129, 200], 256, 2, 4, 128, 630, True, 1.0)
    _check_layer(*gpu, *ref)


def test_layer_prefill_wide_gates_gqa4(gdn):
    """32 value heads over 8 key heads (the widest gate block the input projection takes: 64
    gate columns) at head dim 64, two sequences with caches in."""
    announce("layer prefill Hk=8 Hv=32 d=64 two sequences")
    gpu, ref = _layer_case(gdn, [120, 77], 256, 8, 32, 64, 635, True, 0.5)
    _check_layer(*gpu, *ref)


def test_layer_prefill_0p8b_shape_bench_inputs(gdn):
    """The 0.8B layer shape with the bench's own layer inputs: T = 4096, hidden 1024, 16 / 16
    heads of 128, zero caches, weights from seed 7 and the hidden rows from seed 8."""
    announce("layer prefill T=4096 E=1024 16/16 heads d=128 (bench inputs)")
    gpu, ref = _layer_case(gdn, [4096], 1024, 16, 16, 128, 7, False, 1.0, hidden_seed=8)
    _check_layer(*gpu, *ref)


def test_layer_prefill_grid_inputs(gdn):
    """The layer on grid-drawn input and input projection (every projected value exact in
    fp32), two sequences with caches in."""
    announce("layer prefill on grid inputs, Hk=2 Hv=4 d=128")
    gpu, ref = _layer_case(gdn, [300, 65], 512, 2, 4, 128, 640, True, 1.0, exact=True)
    _check_layer(*gpu, *ref)


def test_layer_prefill_norm_in_prefill_ragged(gdn):
    """Four sequences (3000, 3, 2900 and 64 tokens) over 2 key / 4 value heads of 128, caches
    in: 16 (sequence, head) units and 97 chunks put the prefill in its concurrent schedule,
    where the state pass forms the gated RMSNorm itself (ragged last chunks, a sequence
    shorter than the conv window, one of exactly one chunk)."""
    announce("layer prefill, norm formed in the prefill, 4 ragged sequences, Hk=2 Hv=4 d=128")
    gpu, ref = _layer_case(gdn, [3000, 3, 2900, 64], 256, 2, 4, 128, 655, True, 0.5)
    _check_layer(*gpu, *ref)


def test_layer_prefill_norm_in_prefill_degenerate_sequences(gdn):
    """Seven sequences over 1 key / 2 value heads of 128, among them an empty one, a single
    token and three tokens, caches in: 14 units and 192 chunks keep the prefill in its
    concurrent schedule, so the norm waves run their prologue and tail on sequences of 0, 1
    and a few chunks beside long ones."""
    announce("layer prefill, norm formed in the prefill, 7 sequences incl. empty / 1 / 3 tokens, Hv=2 d=128")
    gpu, ref = _layer_case(gdn, [5200, 0, 3, 4100, 64, 2500, 1], 256, 1, 2, 128, 660, True, 1.0)
    _check_layer(*gpu, *ref)


def test_layer_prefill_norm_in_prefill_order1(gdn):
    """The retrieval-order variant (order 1) through the layer with the norm formed in the
    prefill: four sequences over 2 key / 4 value heads of 128 in the concurrent schedule."""
    announce("layer prefill, norm formed in the prefill, order 1, Hk=2 Hv=4 d=128")
    gpu, ref = _layer_case(gdn, [2500, 700, 2900, 17], 256, 2, 4, 128, 665, True, 0.5, order=1)
    _check_layer(*gpu, *ref)


def _layer_4k_bench_run(gdn, separate, monkeypatch, **kw):
    wts = inputs.layer_weights(7, 1024, 16, 16, 128, 128)
    h = _cuda(inputs.layer_hidden(8, 4096, 1024))
    w = [_cuda(t) for t in (wts.w_in, wts.conv_w, wts.gamma, wts.w_out)]
    if separate:
        monkeypatch.setenv("GDN_LAYER_NORM_SEPARATE", "1")
    else:
        monkeypatch.delenv("GDN_LAYER_NORM_SEPARATE", raising=False)
    out, fin = gdn.layer_prefill(h, *w, 16, 16, 128, 128, **kw)
    torch.cuda.synchronize()
    monkeypatch.delenv("GDN_LAYER_NORM_SEPARATE", raising=False)
    return (h, w), out, fin


def test_layer_prefill_norm_in_prefill_vs_separate_pass(gdn, monkeypatch):
    """The bench's layer (T = 4096, hidden 1024, 16 / 16 heads of 128) with the gated RMSNorm
    formed inside the prefill against the same call with the norm as a pass of its own over
    the fp32 core output (GDN_LAYER_NORM_SEPARATE).  The two take each row's mean square in
    different orders, so a few normalised values (a few dozen of 8.4 M) round to the
    neighbouring bf16 value, and the output projection spreads each such one-ulp change over
    a row of the output.  So: the final states are bit-identical, fewer than 0.1 % of the
    outputs differ, by at most 2^-5 of the output RMS (one bf16 ulp of an output near 1 is
    about 1.3 % of it), and the outputs are not all equal (the two paths really ran)."""
    announce("layer prefill T=4096: norm in the prefill vs a separate norm pass")
    _, out_f, fin_f = _layer_4k_bench_run(gdn, False, monkeypatch)
    _, out_s, fin_s = _layer_4k_bench_run(gdn, True, monkeypatch)
    assert torch.equal(fin_f, fin_s), "the final states differ"
    a, b = out_f.float(), out_s.float()
    diff = (a - b).abs()
    rms = float(b.pow(2).mean().sqrt())
    assert float(diff.max()) <= 2.0 ** -5 * rms, f"max |diff| {float(diff.max()):.3g}, rms {rms:.3g}"
    assert int((diff > 0).sum()) <= a.numel() // 1000, f"{int((diff > 0).sum())} outputs differ"
    assert not torch.equal(out_f, out_s), "identical outputs: the norm was not formed in the prefill"


def test_graph_capture_of_layer_prefill_4k(gdn, monkeypatch):
    """gdn_layer_prefill at the bench's layer shape captured into a HIP graph: under capture
    the prefill's ready flags and the norm's strip flags are cleared by kernels before the
    combined launch.  Three replays with eager work in between, each bit-identical to the
    eager call, then an eager call on the same workspace."""
    announce("graph capture of gdn_layer_prefill at T=4096, three replays")
    (h, w), out_ref, fin_ref = _layer_4k_bench_run(gdn, False, monkeypatch)
    ws = torch.empty(gdn.layer_prefill_workspace_size(4096, 1, 16, 16, 128, 128), dtype=torch.uint8, device=DEV)
    out = torch.empty_like(out_ref)
    fin = torch.empty_like(fin_ref)
    side = torch.cuda.Stream(device=DEV)
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            gdn.layer_prefill(h, *w, 16, 16, 128, 128, out=out, final_state=fin, workspace=ws)
    torch.cuda.synchronize()
    for rep in range(3):
        out.zero_()
        fin.zero_()
        junk = torch.randn(1 << 20, device=DEV).sum()   # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, out_ref), f"replay {rep}: output differs from the eager call"
        assert torch.equal(fin, fin_ref), f"replay {rep}: final state differs from the eager call"
        del junk
    out.zero_()
    gdn.layer_prefill(h, *w, 16, 16, 128, 128, out=out, final_state=fin, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(out, out_ref) and torch.equal(fin, fin_ref), "eager call after the replays differs"


def test_layer_prefill_wait_bound_reports_timeout(gdn, monkeypatch):
    """The bench's layer with the concurrent state pass's waits (for records and for the
    norm's row sums) bounded to one sleep through the layer workspace's header: the call
    ends (every kernel exits), its output and final state are NaN and the workspace status
    reads GDN_ERR_TIMEOUT.  With the default bound restored the same workspace gives the
    unbounded call's result and the status reads GDN_OK."""
    announce("layer prefill T=4096 with a one-sleep wait bound: status GDN_ERR_TIMEOUT")
    (h, w), out_ref, fin_ref = _layer_4k_bench_run(gdn, False, monkeypatch)
    ws = torch.zeros(gdn.layer_prefill_workspace_size(4096, 1, 16, 16, 128, 128), dtype=torch.uint8, device=DEV)
    assert gdn.prefill_workspace_status(ws) == gdn.GDN_OK
    gdn.set_wait_bound(ws, 1)
    out1, fin1 = gdn.layer_prefill(h, *w, 16, 16, 128, 128, workspace=ws)
    torch.cuda.synchronize()
    assert gdn.prefill_workspace_status(ws) == gdn.GDN_ERR_TIMEOUT
    assert torch.isnan(fin1.float()).any(), "the final state of a failed call is NaN"
    assert torch.isnan(out1.float()).any(), "the output of a failed call is NaN"
    gdn.set_wait_bound(ws, None)
    out2, fin2 = gdn.layer_prefill(h, *w, 16, 16, 128, 128, workspace=ws)
    torch.cuda.synchronize()
    assert gdn.prefill_workspace_status(ws) == gdn.GDN_OK
    assert torch.equal(out2, out_ref) and torch.equal(fin2, fin_ref)


def test_layer_prefill_state_in_place(gdn):
    """final_state aliasing initial_state and conv_state_out aliasing conv_state_in (the
    exact aliases the ABI allows): the same results as separate output buffers."""
    announce("layer prefill with the state and the conv cache updated in place")
    lengths, E, Hk, Hv, d = [90, 0, 40], 128, 1, 2, 64
    T, N = sum(lengths), len(lengths)
    cu = _cuda(torch.from_numpy(np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)))
    wts = inputs.layer_weights(645, E, Hk, Hv, d, d)
    h = _cuda(inputs.layer_hidden(646, T, E))
    cs_in, s0 = inputs.layer_caches(647, N, Hk, Hv, d, d)
    w = [_cuda(t) for t in (wts.w_in, wts.conv_w, wts.gamma, wts.w_out)]
    cso = torch.empty(cs_in.shape, dtype=torch.float32, device=DEV)
    out1, fin1 = gdn.layer_prefill(h, *w, Hk, Hv, d, d, cu_seqlens=cu, conv_state_in=_cuda(cs_in),
                                   conv_state_out=cso, initial_state=_cuda(s0))
    cs2, st2 = _cuda(cs_in), _cuda(s0)
    out2, fin2 = gdn.layer_prefill(h, *w, Hk, Hv, d, d, cu_seqlens=cu, conv_state_in=cs2, conv_state_out=cs2,
                                   initial_state=st2, final_state=st2)
    torch.cuda.synchronize()
    assert fin2 is st2
    assert torch.equal(out1, out2) and torch.equal(fin1, st2) and torch.equal(cso, cs2)


def test_layer_prefill_empty(gdn):
    announce("layer prefill T=0 with caches")
    (out, fin, cs), (out_ref, fin_ref, cs_ref) = _layer_case(gdn, [0, 0], 128, 1, 2, 64, 650, True, 1.0)
    assert out.shape == (0, 128)
    np.testing.assert_array_equal(f32np(fin), fin_ref)
    np.testing.assert_array_equal(f32np(cs), cs_ref)


# ------------------------------------------------------------------ layer decode

def _decode_case(gdn, B, E, Hk, Hv, d, seed, order=0, exact=False):
    wts = inputs.layer_weights(seed, E, Hk, Hv, d, d, exact=exact)
    h = inputs.layer_hidden(seed + 1, B, E, exact=exact)
    cs, st = inputs.layer_caches(seed + 2, B, Hk, Hv, d, d)
    return _decode_run(gdn, wts, h, cs, st, Hk, Hv, d, 0.5, order)


def _decode_run(gdn, wts, h, cs, st, Hk, Hv, d, scale, order=0):
    out_ref, st_ref, cs_ref, _ = oracle.layer_decode(f32np(h), f32np(wts.w_in), f32np(wts.conv_w), f32np(wts.gamma),
                                                     f32np(wts.w_out), f32np(cs), f32np(st), Hk, Hv, d, d,
                                                     scale=scale, order=order)
    csd, std = _cuda(cs), _cuda(st)
    out = gdn.layer_decode(_cuda(h), _cuda(wts.w_in), _cuda(wts.conv_w), _cuda(wts.gamma), _cuda(wts.w_out), csd, std,
                           Hk, Hv, d, d, scale=scale, order=order)
    torch.cuda.synchronize()
    return (out, std, csd), (out_ref, st_ref, cs_ref)


def _check_decode(out, st, cs, out_ref, st_ref, cs_ref):
    assert_parity_bf16_out("out", f32np(out), out_ref, TOL_BF16)
    assert_parity("state", f32np(st), st_ref, TOL_BF16)
    assert_parity("conv cache", f32np(cs), cs_ref, TOL_F32)


# (33, 192, ...) and (256, 1024, ...) split the output projection's k extent (4 and 16 slices
# summed in a second pass; 33 x 192 also leaves a partial column tile)
@pytest.mark.parametrize("B,E,Hk,Hv,d,order", [(5, 128, 2, 4, 32, 0), (3, 64, 1, 2, 64, 1), (33, 192, 2, 4, 128, 0),
                                               (256, 1024, 16, 16, 128, 0)])
def test_layer_decode(gdn, B, E, Hk, Hv, d, order):
    announce(f"layer decode B={B} E={E} Hk={Hk} Hv={Hv} d={d} order={order}")
    gpu, ref = _decode_case(gdn, B, E, Hk, Hv, d, 660 + B, order)
    _check_decode(*gpu, *ref)


def test_layer_decode_bench_inputs(gdn):
    """The bench's layer decode step: 256 rows of hidden 1024 (seed 11) through the layer
    weights of seed 7, with the decode256 workload's state and conv cache (as fp32)."""
    announce("layer decode B=256 E=1024 16/16 heads d=128 (bench inputs)")
    dw = inputs.decode256()
    wts = inputs.layer_weights(7, 1024, 16, 16, 128, 128)
    h = inputs.layer_hidden(11, 256, 1024)
    gpu, ref = _decode_run(gdn, wts, h, dw.conv_state.float(), dw.state, 16, 16, 128, 1.0)
    _check_decode(*gpu, *ref)


def test_layer_decode_grid_inputs(gdn):
    announce("layer decode on grid inputs, B=40 Hk=2 Hv=4 d=64")
    gpu, ref = _decode_case(gdn, 40, 256, 2, 4, 64, 690, exact=True)
    _check_decode(*gpu, *ref)


def test_layer_decode_continues_layer_prefill(gdn):
    """GPU prefill of L tokens, then one GPU decode step, against the oracle's prefill of
    L + 1 tokens."""
    announce("layer prefill + decode vs oracle prefill of one more token")
    E, Hk, Hv, d, L = 256, 2, 4, 64, 131
    wts = inputs.layer_weights(670, E, Hk, Hv, d, d)
    h = inputs.layer_hidden(671, L + 1, E)
    cu = np.array([0, L + 1], np.int32)
    out_ref, fin_ref, cs_ref, _ = oracle.layer_prefill(f32np(h), f32np(wts.w_in), f32np(wts.conv_w),
                                                       f32np(wts.gamma), f32np(wts.w_out), cu, Hk, Hv, d, d)
    C = 2 * Hk * d + Hv * d
    cs = torch.zeros((1, 3, C), dtype=torch.float32, device=DEV)
    out_p, fin = gdn.layer_prefill(_cuda(h[:L]), _cuda(wts.w_in), _cuda(wts.conv_w), _cuda(wts.gamma),
                                   _cuda(wts.w_out), Hk, Hv, d, d, conv_state_out=cs)
    out_d = gdn.layer_decode(_cuda(h[L:]), _cuda(wts.w_in), _cuda(wts.conv_w), _cuda(wts.gamma), _cuda(wts.w_out),
                             cs, fin, Hk, Hv, d, d)
    torch.cuda.synchronize()
    gpu = np.concatenate([f32np(out_p), f32np(out_d)])
    assert_parity_bf16_out("out", gpu, out_ref, TOL_BF16)
    assert_parity("final state", f32np(fin), fin_ref, TOL_BF16)
    assert_parity("conv cache", f32np(cs), cs_ref, TOL_F32)
