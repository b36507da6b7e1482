#!/usr/bin/env python3
"""Benchmark of the Gated DeltaNet hot path on one MI355X.

One step = one pass of the whole hot path over one batch of seeded synthetic
input:
  prefill of one linear-attention layer of the 0.8B hybrid shape
  (T = 4096 tokens, 16 key / 16 value heads, head dims 128, bf16 pre-conv x):
      gdn_prefill (one call, one launch: conv + SiLU + L2 inside the chunk-local
      workgroups, while the same launch's state-pass workgroups consume each
      chunk's record as soon as it is published; q, k, v never reach HBM)
  followed by one decode step of 256 sequences (gdn_decode_step, fp32 state in place).

Reported beside it (not part of `value`): the whole linear-attention layer at the
same shape with hidden size 1024 and random weights, gdn_layer_prefill (input
projection, the prefill above with the gated RMSNorm formed in its state pass, output
projection) and
gdn_layer_decode for the 256 decode rows, under "layer", with torch's library GEMM
(torch.mm) on the two projection shapes timed in the same region for context.

`value` is prefill tokens/s: 4096 tokens over the event time of the gdn_prefill
call, averaged over the timed steps; the decode part is reported under "decode"
as tokens/s and state GB/s.  A second timed region runs the same prefill as
gdn_conv_qk_prep + gdn_chunk_prefill (reported under "prefill_two_call"), and a
third through the split-phase entry points so that every kernel sits alone
between two HIP events on the stream it is launched on; those per-kernel
durations give "kernels" (the split region also times the gated RMSNorm epilogue,
gdn_gated_rmsnorm, on the prefill output, and the layer's input and output
projections, gdn_in_proj and gdn_linear).  At this shape gdn_prefill is one launch
(prefill_concurrent_kernel: the chunk-local workgroups and the state pass's in one
grid), so the first region's events time that kernel: it is "roofline" (the whole
prefill's algorithmic flops over its duration) and kernels["prefill_concurrent"].  x, g and beta
rotate over 3 copies at different addresses and the decode state over 2 sets
(512 MiB), so no input is served from the 256 MB Infinity Cache; the prefill
workspace is one buffer reused every step, as a caller reuses it, and its lines
stay cached from one step to the next (the decode step reads its state with
non-temporal loads).  "prefill_cold_ms" times the same gdn_prefill call with the
caches flushed before every call (a 1 GiB buffer read and written in between).
"kernels" and "roofline" also carry, while the library sources match those of the
committed counter summary (profiles/counters_layer_4k.txt), each kernel's HBM
bytes from the L2's memory-fabric request counters ("traffic") and, for the MFMA
kernels, the MFMA work it executes (split-operand repeats included) over this
run's time and its MFMA busy fraction under the profiler ("counter_mfma";
"counter_mfma_frac" / "counter_mfma_busy" in "roofline").  After the timed regions, "achievable" records two measured
ceilings (a plain streaming kernel's GB/s, the library's bf16 GEMM on 8192^3), and the
decode and projection figures are also given as fractions of them.

Usage: python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--no-cpu-baseline]
Profiler runs: --split-only (the metric's region and the split-phase region),
--metric-only (the gdn_prefill + decode region alone),
--copy-calibration (a 512 MiB streaming copy after the timed steps, a check of the
request-counter bytes against a known stream).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, GB/s
PEAK_MFMA_TFLOPS = 2500.0      # MI355X dense bf16 / fp16 MFMA, TFLOP/s
PEAK_F32_TFLOPS = 157.3        # MI355X fp32 vector, TFLOP/s

METRIC = "GDN prefill tokens/s + decode state GB/s (fraction of MI355X roofline)"
LAYER_HIDDEN = 1024            # hidden size of the 0.8B model's layers
# bench kernel name -> the profile's name for the kernel that call launches
PROFILE_NAME = {"in_proj": "proj_256", "out_proj": "proj_128"}


def algorithmic_counts(T, Hk, Hv, d, C, N, B):
    """Algorithmic work per launch of each kernel.

    Prefill flops are the chunk method's own (lower triangles only) per token
    and value head: (3C-1) dk + 2C dv + C^2/3 for the chunk-local products and
    the triangular solve (K K^T, Q K^T, T K, T V, P Delta) and 6 dk dv for the
    state contractions (W S, Q S, K^T Delta); extra products that a kernel
    issues for its own reasons (split operands, P W) are not counted.  Bytes
    are those the kernel's interface must move once."""
    conv_dim = 2 * Hk * d + Hv * d
    prep_bytes = T * conv_dim * 2 + T * (2 * Hk * d + Hv * d) * 4 + conv_dim * 4 * 2 + N * 3 * conv_dim * 2
    local_flops = T * Hv * ((3 * C - 1) * d + 2 * C * d + C * C // 3)
    state_flops = T * Hv * 6 * d * d
    dec_state = 2 * B * Hv * d * d * 4
    dec_bytes = dec_state + B * conv_dim * 2 + 2 * B * 3 * conv_dim * 2 + B * Hv * d * 4 + 2 * B * Hv * 4 \
        + conv_dim * 4 * 2
    return prep_bytes, local_flops, state_flops, dec_bytes


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(wl, dw, dec_bytes, min_seconds=10.0):
    """The fp64 oracle on the same batches, on this host's cores: whole layer_4k prefill
    passes (prep, then the token recurrence) repeated until at least `min_seconds` have run
    (three passes at least), then decode256 steps for a few seconds; medians are reported."""
    import numpy as np
    import oracle
    x = wl.x.float().numpy()
    w = wl.conv_w.float().numpy()
    cu = wl.cu_seqlens.numpy()
    g = wl.g.numpy()
    b = wl.beta.numpy()
    oracle.lib()
    times = []
    start = time.perf_counter()
    while len(times) < 3 or time.perf_counter() - start < min_seconds:
        t0 = time.perf_counter()
        q, k, v, _ = oracle.prep(x, w, cu, wl.Hk, wl.Hv, wl.dk, wl.dv)
        oracle.recurrence(q, k, v, g, b, cu)
        times.append(time.perf_counter() - t0)
    t = float(np.median(times))
    dargs = [t.float().numpy() for t in (dw.x, dw.conv_w, dw.conv_state, dw.g, dw.beta, dw.state)]
    dtimes = []
    start = time.perf_counter()
    while len(dtimes) < 3 or time.perf_counter() - start < 3.0:
        t0 = time.perf_counter()
        oracle.decode(*dargs, dw.Hk, dw.Hv, dw.dk, dw.dv)
        dtimes.append(time.perf_counter() - t0)
    td = float(np.median(dtimes))
    threads = oracle.threads(1 << 30)
    return {"value": wl.T / t, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "nproc": os.cpu_count(), "cpu_model": cpu_model(),
            "sample": f"whole layer_4k prefill (conv+SiLU+L2 over T={wl.T}, then the fp64 token recurrence over all "
                      f"{wl.Hv} heads) repeated {len(times)} times ({sum(times):.1f} s); median pass {t:.2f} s. "
                      f"OpenMP: {threads} threads over tokens in prep, min({threads}, {wl.Hv}) over heads in the "
                      f"recurrence",
            "decode": {"steps_per_s": 1.0 / td, "tokens_per_s": dw.N / td, "gb_per_s": dec_bytes / td / 1e9,
                       "sample": f"decode256 step (B={dw.N}, {dw.Hv} heads, fp64 state) repeated {len(dtimes)} "
                                 f"times; median {td * 1e3:.1f} ms; OpenMP over rows; GB/s counts the GPU's "
                                 f"algorithmic bytes per step"}}


def prefill_flops_per_token_head(d, C=64):
    """The chunk method's algorithmic flops per token and value head at head dim d:
    (3C - 1) d + 2C d + C^2/3 (chunk-local products and solve) + 6 d^2 (state contractions)."""
    return (3 * C - 1) * d + 2 * C * d + C * C // 3 + 6 * d * d


def ratio(gpu, ref):
    import numpy as np
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.max(np.abs(gpu - ref)) / np.sqrt(np.mean(ref * ref)))


def config_records(torch, gdn, inputs, dev, reps=10):
    """One record per prefill configuration not in the metric (tiny_f32, varlen8, long_64k):
    the prefill call timed with HIP events (inputs resident, `reps` calls after 2 warm-ups,
    mean), tokens/s, algorithmic flop rate and its fraction of the peak the arithmetic
    runs on, and parity against the fp64 oracle (max|err|/RMS of o and of the final state)."""
    import oracle
    recs = {}

    def time_calls(fn, n):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    # tiny_f32: the core alone in fp32, chunked WY / UT form in fp32 and the token recurrence
    wl = inputs.tiny_f32()
    args = [t.to(dev) for t in (wl.q, wl.k, wl.v, wl.g, wl.beta)]
    cu = wl.cu_seqlens.to(dev)
    o_ref, f_ref = oracle.recurrence(*(t.numpy() for t in (wl.q, wl.k, wl.v, wl.g, wl.beta)), wl.cu_seqlens.numpy())
    rec = {"workload": "tiny_f32 (T=64, H=2, dk=dv=16, fp32, core only)", "tolerance": 1e-4}
    flops = wl.T * wl.Hv * prefill_flops_per_token_head(wl.dk)
    for math in ("f32_chunked", "f32"):
        fn = lambda: gdn.chunk_prefill(*args, cu_seqlens=cu, math=math)
        ms = time_calls(fn, reps)
        o, f = fn()
        torch.cuda.synchronize()
        rec[math] = {"ms": ms, "tokens_per_s": wl.T / (ms / 1e3), "achieved_tflops": flops / ms / 1e9,
                     "frac_fp32_vector_peak": flops / ms / 1e9 / PEAK_F32_TFLOPS,
                     "parity": {"o": ratio(o.cpu(), o_ref), "final_state": ratio(f.cpu(), f_ref)}}
    recs["tiny_f32"] = rec

    # varlen8 and long_64k: gdn_prefill (fused prep) with bf16 x, fp32 state
    for name, n_rep in (("varlen8", reps), ("long_64k", max(2, reps // 2))):
        wl = inputs.get(name)
        x, w, g, b = (t.to(dev) for t in (wl.x, wl.conv_w, wl.g, wl.beta))
        cu = wl.cu_seqlens.to(dev)
        s0 = None if wl.state is None else wl.state.to(dev)
        csi = None if wl.conv_state is None else wl.conv_state.to(dev)
        ws = torch.empty(gdn.workspace_size(wl.T, wl.N, wl.Hk, wl.Hv, wl.dk, wl.dv, "mfma"), dtype=torch.uint8,
                         device=dev)
        o = torch.empty((wl.T, wl.Hv, wl.dv), dtype=torch.float32, device=dev)
        fin = torch.empty((wl.N, wl.Hv, wl.dk, wl.dv), dtype=torch.float32, device=dev)
        fn = lambda: gdn.prefill(x, w, g, b, wl.Hk, wl.Hv, wl.dk, wl.dv, cu_seqlens=cu, conv_state_in=csi,
                                 initial_state=s0, final_state=fin, o=o, workspace=ws)
        ms = time_calls(fn, n_rep)
        fn()
        torch.cuda.synchronize()
        o_gpu, f_gpu = o.cpu(), fin.cpu()
        del x, w, g, b, ws, o, fin
        torch.cuda.empty_cache()
        q_r, k_r, v_r, _ = oracle.prep(wl.x.float().numpy(), wl.conv_w.float().numpy(), wl.cu_seqlens.numpy(),
                                       wl.Hk, wl.Hv, wl.dk, wl.dv,
                                       cs_in=None if wl.conv_state is None else wl.conv_state.float().numpy())
        o_ref, f_ref = oracle.recurrence(q_r, k_r, v_r, wl.g.numpy(), wl.beta.numpy(), wl.cu_seqlens.numpy(),
                                         s0=None if wl.state is None else wl.state.numpy())
        del q_r, k_r, v_r
        flops = wl.T * wl.Hv * prefill_flops_per_token_head(wl.dk)
        recs[name] = {"workload": f"{name} (T={wl.T}, N={wl.N}, Hk={wl.Hk}, Hv={wl.Hv}, dk=dv={wl.dk}, bf16 x, "
                                  f"fp32 state)", "entry_point": "gdn_prefill", "ms": ms,
                      "tokens_per_s": wl.T / (ms / 1e3), "achieved_tflops": flops / ms / 1e9,
                      "frac_mfma": flops / ms / 1e9 / PEAK_MFMA_TFLOPS, "tolerance": 2e-2,
                      "parity": {"o": ratio(o_gpu, o_ref), "final_state": ratio(f_gpu, f_ref)}}
        del o_ref, f_ref, o_gpu, f_gpu
    return recs


COUNTERS_FILE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles", "counters_layer_4k.txt")


def measured_counters():
    """Per-kernel figures of the committed counter summary (HBM bytes, MFMA flops executed,
    MFMA busy fraction per launch): {kernel: {figure: value}}, empty when the library sources
    changed since the counters were taken."""
    from hybrid_linear_attention_gated_amd import profiling
    rec = profiling.read_traffic(COUNTERS_FILE)
    if not rec or rec.get("source_sha256") != profiling.source_sha256():
        return {}
    out = {}
    for key, val in rec.items():
        if "." in key and key != "source_sha256":
            kern, fig = key.split(".", 1)
            out.setdefault(kern, {})[fig] = float(val)
    return out


def copy_calibration(torch, dev):
    """A plain streaming copy of known size (torch.neg over 512 MiB): a check of the
    request-counter bytes of the counter runs against a known stream."""
    from hybrid_linear_attention_gated_amd import profiling
    n = profiling.COPY_BYTES // 4
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    del src, dst


def achievable_peaks(torch, dev):
    """Measured ceilings on this GPU, for context beside the datasheet peaks: a plain
    elementwise stream (torch.neg, 512 MiB read + 512 MiB written) and the library's bf16
    GEMM (torch.mm, hipBLASLt) on an 8192^3 product; HIP events, best of several runs."""
    n = (512 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    a = torch.randn(8192, 8192, device=dev).to(torch.bfloat16)
    b = torch.randn(8192, 8192, device=dev).to(torch.bfloat16)
    c = torch.empty(8192, 8192, dtype=torch.bfloat16, device=dev)

    def best_ms(fn, reps):
        fn()
        torch.cuda.synchronize()
        times = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1))
        return min(times)

    stream_ms = best_ms(lambda: torch.neg(src, out=dst), 10)
    gemm_ms = best_ms(lambda: torch.mm(a, b.t(), out=c), 5)
    del src, dst, a, b, c
    return {"stream_gb_per_s": 2 * n * 4 / stream_ms / 1e6, "library_gemm_tflops": 2 * 8192 ** 3 / gemm_ms / 1e9,
            "what": "torch.neg over 512 MiB fp32 (read + write); torch.mm bf16 8192^3; best of 10 / 5 runs"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--sets", type=int, default=3, help="input copies rotated across steps")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the per-configuration records (tiny_f32, varlen8, long_64k) and the parity checks")
    ap.add_argument("--split-only", action="store_true",
                    help="time only the metric's region and the split-phase region (one launch per kernel per "
                         "step), for profiler runs")
    ap.add_argument("--metric-only", action="store_true",
                    help="time only the metric's region (gdn_prefill + decode step) and print its two times, "
                         "for kernel-trace runs of the concurrent prefill schedule")
    ap.add_argument("--layer-only", action="store_true",
                    help="time only the layer region (gdn_layer_prefill + gdn_layer_decode) and print its times, "
                         "for kernel traces of the layer path")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after the timed steps, stream 512 MiB through one elementwise kernel (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the hot path is data-parallel per sequence and per head, and the "
              "library runs on a single MI355X; --gpus must be 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import hybrid_linear_attention_gated_amd as gdn
    from hybrid_linear_attention_gated_amd import inputs

    gdn.lib()   # fails loudly when the HIP library is missing
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    wl = inputs.layer_4k()
    dw = inputs.decode256()
    T, Hk, Hv, d, N = wl.T, wl.Hk, wl.Hv, wl.dk, wl.N
    B = dw.N
    R = max(2, args.sets)

    # prefill buffers (inputs rotated over R copies)
    xs = [wl.x.to(dev) for _ in range(R)]
    gs = [wl.g.to(dev) for _ in range(R)]
    bs = [wl.beta.to(dev) for _ in range(R)]
    cw = wl.conv_w.to(dev)
    cu = wl.cu_seqlens.to(dev)
    q = torch.empty((T, Hk, d), dtype=torch.float32, device=dev)
    k = torch.empty_like(q)
    v = torch.empty((T, Hv, d), dtype=torch.float32, device=dev)
    o = torch.empty((T, Hv, d), dtype=torch.float32, device=dev)
    cso = torch.empty((N, 3, wl.conv_dim), dtype=torch.bfloat16, device=dev)
    fin = torch.empty((N, Hv, d, d), dtype=torch.float32, device=dev)
    ws = torch.empty(gdn.workspace_size(T, N, Hk, Hv, d, d, "mfma"), dtype=torch.uint8, device=dev)

    # gated RMSNorm epilogue on the prefill output (bf16 gate, gain and output)
    zg_cpu, gam_cpu = inputs.gate_inputs(5, (T, Hv, d), d, "bf16")
    zg, gam = zg_cpu.to(dev), gam_cpu.to(dev)
    nout = torch.empty((T, Hv, d), dtype=torch.bfloat16, device=dev)

    # decode buffers: >= 2 state sets (>= 512 MiB) so no step finds its state in the Infinity Cache
    Rd = 2
    dstate = [dw.state.to(dev) for _ in range(Rd)]
    dcs = [dw.conv_state.to(dev) for _ in range(Rd)]
    dx = dw.x.to(dev)
    dcw = dw.conv_w.to(dev)
    dg = dw.g.to(dev)
    db = dw.beta.to(dev)
    do = torch.empty((B, Hv, d), dtype=torch.float32, device=dev)
    dz_cpu, dgam_cpu = inputs.gate_inputs(6, (B, Hv, d), d, "bf16")
    dz, dgam = dz_cpu.to(dev), dgam_cpu.to(dev)
    dout = torch.empty((B, Hv, d), dtype=torch.bfloat16, device=dev)

    # layer forward (hidden size 1024 of the 0.8B model): inputs rotated like x
    E = LAYER_HIDDEN
    Z = Hv * d
    lw = inputs.layer_weights(7, E, Hk, Hv, d, d)
    w_in, lcw, lgam, w_out = lw.w_in.to(dev), lw.conv_w.to(dev), lw.gamma.to(dev), lw.w_out.to(dev)
    hs = [inputs.layer_hidden(8 + i, T, E).to(dev) for i in range(R)]
    lout = torch.empty((T, E), dtype=torch.bfloat16, device=dev)
    lcso = torch.empty((N, 3, wl.conv_dim), dtype=torch.float32, device=dev)
    lfin = torch.empty((N, Hv, d, d), dtype=torch.float32, device=dev)
    lws = torch.empty(gdn.layer_prefill_workspace_size(T, N, Hk, Hv, d, d), dtype=torch.uint8, device=dev)
    dh = inputs.layer_hidden(11, B, E).to(dev)
    lcs_dec = [dw.conv_state.float().to(dev) for _ in range(Rd)]   # the layer keeps fp32 conv caches
    dlout = torch.empty((B, E), dtype=torch.bfloat16, device=dev)
    dlws = torch.empty(gdn.layer_decode_workspace_size(B, E, Hk, Hv, d, d), dtype=torch.uint8, device=dev)
    px = torch.empty((T, wl.conv_dim), dtype=torch.bfloat16, device=dev)
    pz = torch.empty((T, Z), dtype=torch.bfloat16, device=dev)
    pg = torch.empty((T, Hv), dtype=torch.float32, device=dev)
    pb = torch.empty((T, Hv), dtype=torch.float32, device=dev)
    nout.copy_(zg)            # defined values until the split region's gated RMSNorm writes it
    ynorm = nout.view(T, Z)   # the gated RMSNorm's bf16 output feeds the output projection
    pout = torch.empty((T, E), dtype=torch.bfloat16, device=dev)
    lib_in = torch.empty((T, w_in.shape[0]), dtype=torch.bfloat16, device=dev)

    # Timed region 1 (the metric): one step = gdn_prefill (prep fused into the chunked
    # prefill, one call) + one decode step.
    def step(i, ev):
        r = i % R
        ev[0].record()
        gdn.prefill(xs[r], cw, gs[r], bs[r], Hk, Hv, d, d, cu_seqlens=cu, conv_state_out=cso, final_state=fin,
                    o=o, workspace=ws)
        ev[1].record()
        gdn.decode_step(dx, dcw, dcs[i % Rd], dg, db, dstate[i % Rd], Hk, Hv, d, d, o=do)
        ev[2].record()

    # Timed region 1b: the same prefill as gdn_conv_qk_prep + gdn_chunk_prefill (q, k, v
    # written to HBM and read back).
    def step_two(i, ev):
        r = i % R
        ev[0].record()
        gdn.conv_qk_prep(xs[r], cw, Hk, Hv, d, d, cu_seqlens=cu, conv_state_out=cso, q=q, k=k, v=v)
        ev[1].record()
        gdn.chunk_prefill(q, k, v, gs[r], bs[r], cu_seqlens=cu, final_state=fin, o=o, workspace=ws, math="mfma")
        ev[2].record()

    # Timed region 2 (per-kernel durations for the roofline): the same prefill through the
    # split-phase entry points, one kernel between each pair of events: the fused chunk-local
    # kernel (gdn_prefill_local without a conv cache to write, so the interval holds that
    # kernel alone), the state pass, the decode step; then the two-call path's prep and
    # chunk-local kernels, the gated RMSNorm epilogue on the prefill output and the decode
    # step with the gated RMSNorm fused.
    def step_split(i, ev):
        r = i % R
        ev[0].record()
        gdn.prefill_local(xs[r], cw, gs[r], bs[r], ws, Hk, Hv, d, d, cu_seqlens=cu)
        ev[1].record()
        gdn.chunk_prefill_state(ws, o, T, Hk, Hv, d, d, cu_seqlens=cu, final_state=fin)
        ev[2].record()
        gdn.decode_step(dx, dcw, dcs[i % Rd], dg, db, dstate[i % Rd], Hk, Hv, d, d, o=do)
        ev[3].record()
        gdn.conv_qk_prep(xs[r], cw, Hk, Hv, d, d, cu_seqlens=cu, conv_state_out=cso, q=q, k=k, v=v)
        ev[4].record()
        gdn.chunk_prefill_local(q, k, v, gs[r], bs[r], ws, cu_seqlens=cu)
        ev[5].record()
        gdn.gated_rmsnorm(o, zg, gam, out=nout)
        ev[6].record()
        gdn.decode_step_gated(dx, dcw, dcs[(i + 1) % Rd], dg, db, dstate[(i + 1) % Rd], dz, dgam, Hk, Hv, d, d,
                              out=dout)
        ev[7].record()
        gdn.in_proj(hs[r], w_in, Hk, Hv, d, d, x=px, z=pz, g=pg, beta=pb)
        ev[8].record()
        gdn.linear(ynorm, w_out, y=pout)
        ev[9].record()

    # Timed region 3: the whole layer (prefill of the 4096 tokens, then one decode step
    # of the 256 rows), and the library GEMM on the two projection shapes.
    def step_layer(i, ev):
        r = i % R
        ev[0].record()
        gdn.layer_prefill(hs[r], w_in, lcw, lgam, w_out, Hk, Hv, d, d, cu_seqlens=cu, conv_state_out=lcso,
                          final_state=lfin, out=lout, workspace=lws)
        ev[1].record()
        gdn.layer_decode(dh, w_in, lcw, lgam, w_out, lcs_dec[i % Rd], dstate[i % Rd], Hk, Hv, d, d, out=dlout,
                         workspace=dlws)
        ev[2].record()
        torch.mm(hs[r], w_in.t(), out=lib_in)
        ev[3].record()
        torch.mm(ynorm, w_out.t(), out=pout)
        ev[4].record()

    def events(n):
        return [torch.cuda.Event(enable_timing=True) for _ in range(n)]

    def mean_ms(ev_list, j):
        return sum(ev[j].elapsed_time(ev[j + 1]) for ev in ev_list) / len(ev_list)

    def timed(fn, n_ev):
        for i in range(args.warmup):
            fn(i, events(n_ev))
        torch.cuda.synchronize()
        evs = [events(n_ev) for _ in range(args.steps)]
        t0 = time.perf_counter()
        for i in range(args.steps):
            fn(args.warmup + i, evs[i])
        torch.cuda.synchronize()
        return evs, time.perf_counter() - t0

    names = ["chunk_local_fused", "state_pass", "decode", "prep", "chunk_local", "gated_rmsnorm", "decode_gated",
             "in_proj", "out_proj"]
    two_call = None
    layer = None
    prefill_cold_ms = None
    if args.layer_only:
        evs_l, _ = timed(step_layer, 5)
        print(json.dumps({"layer_prefill_ms": mean_ms(evs_l, 0), "layer_decode_ms": mean_ms(evs_l, 1),
                          "steps": args.steps, "warmup": args.warmup}))
        return
    evs, wall = timed(step, 3)
    prefill_ms, decode_ms = mean_ms(evs, 0), mean_ms(evs, 1)
    if args.metric_only:
        print(json.dumps({"prefill_ms": prefill_ms, "decode_ms": decode_ms, "entry_point": "gdn_prefill",
                          "steps": args.steps, "warmup": args.warmup}))
        return
    if not args.split_only:
        # Timed region 1c: the same gdn_prefill with every cache cold.  Before each call a
        # 1 GiB buffer (four times the Infinity Cache) is read and written, so the call finds
        # neither its workspace nor its inputs in the Infinity Cache or the L2, as in a model
        # whose other layers run between two calls of this one.
        flush = torch.empty(1 << 28, dtype=torch.float32, device=dev)

        def step_cold(i, ev):
            r = i % R
            flush.neg_()
            ev[0].record()
            gdn.prefill(xs[r], cw, gs[r], bs[r], Hk, Hv, d, d, cu_seqlens=cu, conv_state_out=cso, final_state=fin,
                        o=o, workspace=ws)
            ev[1].record()
        evs_cold, _ = timed(step_cold, 2)
        prefill_cold_ms = mean_ms(evs_cold, 0)
        del flush
        evs_two, _ = timed(step_two, 3)
        two_prep, two_call_ms = mean_ms(evs_two, 0), mean_ms(evs_two, 1)
        two_call = {"ms": two_prep + two_call_ms, "prep_ms": two_prep, "chunk_prefill_ms": two_call_ms,
                    "tokens_per_s": T / ((two_prep + two_call_ms) / 1e3)}
        evs_l, _ = timed(step_layer, 5)
        lp, ld, gi, go = (mean_ms(evs_l, j) for j in range(4))
        layer = {"workload": f"linear-attention layer, hidden {E}, T={T} prefill + B={B} decode, random bf16 "
                             "weights",
                 "prefill_ms": lp, "prefill_tokens_per_s": T / (lp / 1e3),
                 "decode_ms": ld, "decode_tokens_per_s": B / (ld / 1e3),
                 "library_gemm_ms": {"in_proj": gi, "out_proj": go}}
    evs2, _ = timed(step_split, 10)
    per = {n: mean_ms(evs2, j) for j, n in enumerate(names)}   # ms per launch (split phases)
    # gdn_prefill at this shape is one launch (prefill_concurrent_kernel: the chunk-local
    # workgroups and the state pass's), so the metric region's events time that kernel
    per["prefill_concurrent"] = prefill_ms

    prep_b, local_f, state_f, dec_b = algorithmic_counts(T, Hk, Hv, d, 64, N, B)
    norm_b = T * Hv * d * (4 + 2 + 2) + d * 2   # y fp32 in, z bf16 in, out bf16, gain
    decg_b = dec_b - B * Hv * d * 4 + B * Hv * d * (2 + 2) + d * 2   # o fp32 replaced by z in, out bf16
    in_f = 2 * T * E * w_in.shape[0]    # input projection: T x E times E x (conv_dim + Hv dv + 2 Hv)
    out_f = 2 * T * Z * E               # output projection: T x Hv dv times Hv dv x E
    kern = {
        "prefill_concurrent": {"bound": "mfma", "achieved": (local_f + state_f) / per["prefill_concurrent"] / 1e9,
                               "peak": PEAK_MFMA_TFLOPS, "unit": "TFLOP/s"},
        "chunk_local_fused": {"bound": "mfma", "achieved": local_f / per["chunk_local_fused"] / 1e9,
                              "peak": PEAK_MFMA_TFLOPS, "unit": "TFLOP/s"},
        "prep": {"bound": "hbm", "achieved": prep_b / per["prep"] / 1e6, "peak": PEAK_HBM_GBS, "unit": "GB/s"},
        "chunk_local": {"bound": "mfma", "achieved": local_f / per["chunk_local"] / 1e9, "peak": PEAK_MFMA_TFLOPS,
                        "unit": "TFLOP/s"},
        "state_pass": {"bound": "mfma", "achieved": state_f / per["state_pass"] / 1e9, "peak": PEAK_MFMA_TFLOPS,
                       "unit": "TFLOP/s"},
        "decode": {"bound": "hbm", "achieved": dec_b / per["decode"] / 1e6, "peak": PEAK_HBM_GBS, "unit": "GB/s"},
        "gated_rmsnorm": {"bound": "hbm", "achieved": norm_b / per["gated_rmsnorm"] / 1e6, "peak": PEAK_HBM_GBS,
                          "unit": "GB/s"},
        "decode_gated": {"bound": "hbm", "achieved": decg_b / per["decode_gated"] / 1e6, "peak": PEAK_HBM_GBS,
                         "unit": "GB/s"},
        "in_proj": {"bound": "mfma", "achieved": in_f / per["in_proj"] / 1e9, "peak": PEAK_MFMA_TFLOPS,
                    "unit": "TFLOP/s"},
        "out_proj": {"bound": "mfma", "achieved": out_f / per["out_proj"] / 1e9, "peak": PEAK_MFMA_TFLOPS,
                     "unit": "TFLOP/s"},
    }
    counters = measured_counters()   # per-launch counter figures of the committed summary, or {}
    for n in ["prefill_concurrent"] + names:
        kern[n]["ms"] = per[n]
        kern[n]["frac"] = kern[n]["achieved"] / kern[n]["peak"]
        c = counters.get(PROFILE_NAME.get(n, n), {})
        kern[n]["traffic"] = c.get("traffic_bytes")
        if kern[n]["bound"] == "mfma" and "mfma_flops" in c:
            # MFMA work the kernel executes (split-operand repeats and zero padding included)
            # over this run's time, and the MFMA busy fraction under the profiler
            kern[n]["counter_mfma"] = {"executed_tflops": c["mfma_flops"] / per[n] / 1e9,
                                       "frac": c["mfma_flops"] / per[n] / 1e9 / PEAK_MFMA_TFLOPS,
                                       "busy_frac": c.get("mfma_busy_frac")}
    dominant = "prefill_concurrent"   # the metric path's prefill: one launch
    roof = {key: kern[dominant][key] for key in ("bound", "achieved", "peak", "unit", "frac", "traffic")}
    roof["kernel"] = dominant
    if "counter_mfma" in kern[dominant]:
        roof["counter_mfma_frac"] = kern[dominant]["counter_mfma"]["frac"]
        roof["counter_mfma_busy"] = kern[dominant]["counter_mfma"]["busy_frac"]

    out = {
        "metric": METRIC,
        "value": T / (prefill_ms / 1e3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall * 1e3 / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 x; fp16/bf16 MFMA with fp32 accumulation; fp32 state",
        "data": "synthetic",
        "config": {"workload": "layer_4k prefill (T=4096, Hk=Hv=16, dk=dv=128, chunk 64, bf16 x, fp32 q/k/v/o) "
                               "+ decode256 step (B=256, fp32 state 256 MiB, 2 rotating state sets)",
                   "T": T, "heads_k": Hk, "heads_v": Hv, "head_dim": d, "chunk": 64, "decode_batch": B},
        "prefill": {"ms": prefill_ms, "entry_point": "gdn_prefill",
                    "tokens_per_s": T / (prefill_ms / 1e3),
                    "algorithmic_tflops": (local_f + state_f) / prefill_ms / 1e9,
                    "frac_mfma": (local_f + state_f) / prefill_ms / 1e9 / PEAK_MFMA_TFLOPS},
        "prefill_cold_ms": prefill_cold_ms,
        "prefill_two_call": two_call,
        "layer": layer,
        "decode": {"ms": decode_ms, "tokens_per_s": B / (decode_ms / 1e3),
                   "state_gb_per_s": dec_b / decode_ms / 1e6, "frac_hbm": dec_b / decode_ms / 1e6 / PEAK_HBM_GBS,
                   "bytes_per_step": dec_b},
        "roofline": roof,
        "kernels": kern,
    }
    if not (args.split_only or args.metric_only):
        cal = achievable_peaks(torch, dev)
        out["achievable"] = cal
        out["decode"]["frac_of_stream"] = out["decode"]["state_gb_per_s"] / cal["stream_gb_per_s"]
        for n in ("in_proj", "out_proj"):
            kern[n]["frac_of_library_gemm"] = kern[n]["achieved"] / cal["library_gemm_tflops"]
    if args.copy_calibration:
        copy_calibration(torch, dev)
    if not (args.split_only or args.no_configs):
        # parity of the metric's own configurations (layer_4k prefill, decode256 step) on the
        # outputs of the last timed calls, then the other configurations' records
        import oracle
        gdn.prefill(xs[0], cw, gs[0], bs[0], Hk, Hv, d, d, cu_seqlens=cu, conv_state_out=cso, final_state=fin,
                    o=o, workspace=ws)
        torch.cuda.synchronize()
        o_last, f_last = o.cpu(), fin.cpu()
        q_r, k_r, v_r, _ = oracle.prep(wl.x.float().numpy(), wl.conv_w.float().numpy(), wl.cu_seqlens.numpy(),
                                       Hk, Hv, d, d)
        o_ref, f_ref = oracle.recurrence(q_r, k_r, v_r, wl.g.numpy(), wl.beta.numpy(), wl.cu_seqlens.numpy())
        out["prefill"]["parity"] = {"o": ratio(o_last, o_ref), "final_state": ratio(f_last, f_ref), "tolerance": 2e-2}
        ds, dc = dw.state.to(dev), dw.conv_state.to(dev)
        do_ = gdn.decode_step(dx, dcw, dc, dg, db, ds, Hk, Hv, d, d)
        torch.cuda.synchronize()
        do_ref, ds_ref, _ = oracle.decode(*(t.float().numpy() for t in (dw.x, dw.conv_w, dw.conv_state, dw.g,
                                                                          dw.beta, dw.state)), Hk, Hv, d, d)
        out["decode"]["parity"] = {"o": ratio(do_.cpu(), do_ref), "state": ratio(ds.cpu(), ds_ref),
                                   "tolerance": 1e-4}
        del ds, dc, q_r, k_r, v_r, o_ref, f_ref
        out["configs"] = config_records(torch, gdn, inputs, dev)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl, dw, dec_b)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
