"""Summaries of rocprofv3 output for the library's kernels.

  python -m hybrid_linear_attention_gated_amd.profiling stats DIR
      per-kernel launch count and average / min / max duration from a
      `rocprofv3 --kernel-trace --stats --output-format csv -d DIR` run.
  python -m hybrid_linear_attention_gated_amd.profiling traffic FETCH_DIR WRITE_DIR
      HBM bytes per launch from two `rocprofv3 --pmc FETCH_SIZE` and
      `--pmc WRITE_SIZE` runs of `bench.py --copy-calibration`: each counter is
      scaled by what it reads for the plain streaming copy of known size that
      the calibration launches, and the lines end with the SHA-256 of the kernel
      sources and the build script, so a reader can tell when the figures went stale.
  python -m hybrid_linear_attention_gated_amd.profiling timeline DIR [FIRST [SKIP]]
      kernel start / end offsets inside one step, averaged over the steps of a
      `rocprofv3 --kernel-trace` run: a step begins at each launch of the kernel
      FIRST (short name, default prefill_concurrent: the one launch of the concurrent
      prefill schedule) and the first SKIP steps (warm-up) are dropped.  Shows how
      the kernels of a step follow one another (or, on two streams, overlap).

  python -m hybrid_linear_attention_gated_amd.profiling counters DIR [DIR ...]
      per-kernel mean per dispatch of every counter of `rocprofv3 --pmc` runs (CSV).
  python -m hybrid_linear_attention_gated_amd.profiling bytes DIR [DIR ...]
      HBM-side read and write bytes per dispatch from the L2's memory-fabric request
      counters (TCC_EA0_RDREQ_32B/_64B/_128B_sum, TCC_EA0_WRREQ_sum and _64B_sum), and the
      `<kernel>.traffic_bytes` lines bench.py reads.
  python -m hybrid_linear_attention_gated_amd.profiling summary DIR [DIR ...]
      per-kernel counter summary of `rocprofv3 --pmc` passes over the same workload: MFMA
      work executed (SQ_INSTS_VALU_MFMA_MOPS_F16 / _BF16, 512 flops each), MFMA busy
      fraction (SQ_VALU_MFMA_BUSY_CYCLES over every SIMD's share of GRBM_GUI_ACTIVE), VALU
      instructions, LDS instructions and bank-conflict cycles, HBM-side bytes as above; then
      the `<kernel>.<figure> = value` lines bench.py reads and the sources' SHA-256.

Only text is produced; nothing here touches the GPU.
"""
from __future__ import annotations

import csv
import glob
import hashlib
import os
import sys
from collections import defaultdict

_CSRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc")

# kernel symbol fragment -> short name used by bench.py
KERNELS = [
    ("prep_kernel", "prep"),
    ("conv_state_out_kernel", "conv_state_out"),
    ("chunk_local_kernel", "chunk_local"),   # "chunk_local_fused" for the FUSED = true instances
    ("chunk_local_fused", "chunk_local_fused"),
    ("decode_gated", "decode_gated"),
    ("state_pass_kernel", "state_pass"),
    ("prefill_concurrent_kernel", "prefill_concurrent"),   # "_x32" for the fp32-x instances
    ("prefill_recurrent_kernel", "prefill_recurrent"),
    ("decode_kernel", "decode"),
    ("gated_rmsnorm_kernel", "gated_rmsnorm"),
]
# the projection kernel's two tile shapes (named by short_name from its template arguments)
PROJ_NAMES = ("proj_256", "proj_128", "proj_256_layer", "proj_128_layer")
# bench.py --copy-calibration streams a buffer through torch.neg (one elementwise
# kernel that reads and writes COPY_BYTES); host-to-device uploads use blit
# kernels of other names and are not counted as the calibration copy.
COPY_NAMES = ("elementwise_kernel",)


def short_name(symbol: str) -> str:
    if "chunk_local_kernel" in symbol and ("ELb1E" in symbol or ", true," in symbol):
        # FUSED = true; fp32 x (the layer's prefill) or 16-bit x
        return "chunk_local_fused_x32" if ("ELb1Ef" in symbol or ", true, float" in symbol) else "chunk_local_fused"
    if "prefill_concurrent_kernel" in symbol:
        # chunk-local and state pass in one launch; fp32 x (the layer's prefill) or 16-bit x;
        # last template argument NORM = true: the layer's gated RMSNorm formed in the state pass
        if "Lb1EEEv" in symbol or ", true>(" in symbol or symbol.endswith(", true>"):
            return "prefill_concurrent_norm"
        fp32x = "ELb1Ef" in symbol or ", true, float" in symbol
        return "prefill_concurrent_x32" if fp32x else "prefill_concurrent"
    if "decode_kernel" in symbol and ("Lb1E" in symbol or ", true>" in symbol):
        return "decode_gated"        # template argument GATED = true
    if "proj_kernel" in symbol:      # projection GEMM, named by its output tile and mode
        base = "proj_256" if ("ILi128ELi128E" in symbol or "proj_kernel<128, 128" in symbol) else "proj_128"
        head = symbol.rstrip(")").split("(")[0]
        if "ELi1EE" in symbol or "ELi2EE" in symbol or head.endswith(", 1>") or head.endswith(", 2>"):
            return base + "_layer"   # the layer's input projections (fp32 x; the prefill's also fp32 z)
        return base
    for frag, short in KERNELS:
        if frag in symbol:
            return short
    for frag in COPY_NAMES:
        if frag in symbol:
            return "copy"
    return symbol[:48]


def source_sha256() -> str:
    """SHA-256 over the HIP sources and headers the library is built from and the build
    script (its compiler options shape the kernels too)."""
    h = hashlib.sha256()
    paths = [p for p in glob.glob(os.path.join(_CSRC, "*")) if p.endswith((".hip", ".hpp", ".cpp", ".h"))]
    paths.append(os.path.join(os.path.dirname(_CSRC), "build.py"))
    for path in sorted(paths):
        h.update(os.path.basename(path).encode())
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def _csv_rows(directory: str, suffix: str):
    rows = []
    for path in sorted(glob.glob(os.path.join(directory, "**", "*" + suffix), recursive=True)):
        with open(path, newline="") as f:
            rows += list(csv.DictReader(f))
    if not rows:
        raise FileNotFoundError(f"no *{suffix} under {directory}")
    return rows


def kernel_stats(directory: str) -> dict:
    """short name -> {calls, avg_us, min_us, max_us} from the kernel trace."""
    per = defaultdict(list)
    for r in _csv_rows(directory, "kernel_trace.csv"):
        per[short_name(r["Kernel_Name"])].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    return {k: {"calls": len(v), "avg_us": sum(v) / len(v), "min_us": min(v), "max_us": max(v)}
            for k, v in per.items()}


def counter_means(directory: str, counter: str) -> dict:
    """short name -> (dispatches, mean counter value per dispatch)."""
    per = defaultdict(list)
    for r in _csv_rows(directory, "counter_collection.csv"):
        if r["Counter_Name"] == counter:
            per[short_name(r["Kernel_Name"])].append(float(r["Counter_Value"]))
    return {k: (len(v), sum(v) / len(v)) for k, v in per.items()}


# The calibration copy moves this many bytes each way (bench.py --copy-calibration).
COPY_BYTES = 512 << 20

# Counters whose per-dispatch value is the maximum over their dimensions (a clock that every
# XCD counts) rather than the sum (events counted per instance).
_MAX_COUNTERS = ("GRBM_GUI_ACTIVE", "GRBM_COUNT")


def counter_table(*directories: str) -> dict:
    """short name -> {counter: mean value per dispatch} over the `counter_collection.csv`
    files under the directories (one rocprofv3 --pmc pass each).  Rows of one dispatch and
    counter (one per hardware instance, when the file lists them separately) are summed,
    or for a clock counter the largest is taken."""
    per = defaultdict(lambda: defaultdict(dict))   # kernel -> counter -> dispatch -> value
    for d in directories:
        for r in _csv_rows(d, "counter_collection.csv"):
            name, ctr = short_name(r["Kernel_Name"]), r["Counter_Name"]
            disp = (d, r.get("Dispatch_Id") or r.get("Correlation_Id") or len(per[name][ctr]))
            v = float(r["Counter_Value"])
            old = per[name][ctr].get(disp)
            if old is None:
                per[name][ctr][disp] = v
            else:
                per[name][ctr][disp] = max(old, v) if ctr in _MAX_COUNTERS else old + v
    return {k: {c: sum(vals.values()) / len(vals) for c, vals in ctrs.items()} for k, ctrs in per.items()}


def request_bytes(row: dict) -> tuple:
    """HBM-side bytes per dispatch from the L2's memory-fabric request counters: reads of
    32, 64 and 128 bytes (TCC_EA0_RDREQ_32B / _64B / _128B), writes of 32 or 64 bytes
    (TCC_EA0_WRREQ, of which TCC_EA0_WRREQ_64B are 64 bytes).  Returns (read, write) or
    None for a side whose counters are missing."""
    rd = wr = None
    if all(f"TCC_EA0_RDREQ_{w}B_sum" in row for w in (32, 64, 128)):
        rd = 32 * row["TCC_EA0_RDREQ_32B_sum"] + 64 * row["TCC_EA0_RDREQ_64B_sum"] + 128 * row["TCC_EA0_RDREQ_128B_sum"]
    if "TCC_EA0_WRREQ_sum" in row and "TCC_EA0_WRREQ_64B_sum" in row:
        w64 = row["TCC_EA0_WRREQ_64B_sum"]
        wr = 32 * (row["TCC_EA0_WRREQ_sum"] - w64) + 64 * w64
    return rd, wr


def traffic(fetch_dir: str, write_dir: str) -> dict:
    fetch = counter_means(fetch_dir, "FETCH_SIZE")
    write = counter_means(write_dir, "WRITE_SIZE")
    if "copy" not in fetch or "copy" not in write:
        raise RuntimeError("calibration copy not found in the counter runs")
    # counters are in KiB; the factor maps the counter to the copy's known bytes
    f_fac = COPY_BYTES / (fetch["copy"][1] * 1024.0)
    w_fac = COPY_BYTES / (write["copy"][1] * 1024.0)
    out = {"fetch_factor": f_fac, "write_factor": w_fac, "kernels": {}}
    known = {short for _, short in KERNELS} | set(PROJ_NAMES)
    for k in fetch:
        if k not in known or k not in write:
            continue
        fb = fetch[k][1] * 1024.0 * f_fac
        wb = write[k][1] * 1024.0 * w_fac
        out["kernels"][k] = {"dispatches": fetch[k][0], "fetch_bytes": fb, "write_bytes": wb,
                             "traffic_bytes": fb + wb}
    return out


def timeline(directory: str, first: str = "prefill_concurrent", skip: int = 0, lead_us: float = 20.0) -> dict:
    """Mean (start, end) offsets in us of each kernel of a step from the step's first start.

    A step begins at each launch of the kernel `first`; a kernel that starts up to
    `lead_us` before such a launch belongs to that step too (kernels on two streams do not
    always start in issue order).  Kernels are keyed by short name and occurrence inside
    the step ("decode", "decode#2").  Returns {"steps": n, "kernels": [(key, start, end),
    ...] in order of mean start, "span": mean first-start-to-last-end}."""
    rows = sorted(_csv_rows(directory, "kernel_trace.csv"), key=lambda r: int(r["Start_Timestamp"]))
    recs = [(short_name(r["Kernel_Name"]), int(r["Start_Timestamp"]), int(r["End_Timestamp"])) for r in rows]
    marks = [a for n, a, _ in recs if n == first]
    if not marks:
        raise RuntimeError(f"no step starting with {first} under {directory}")
    steps = [[] for _ in marks]
    lead = int(lead_us * 1e3)
    j = -1
    for rec in recs:
        while j + 1 < len(marks) and marks[j + 1] <= rec[1] + lead:
            j += 1
        if j >= 0:
            steps[j].append(rec)
    steps = steps[skip:]
    if not steps:
        raise RuntimeError(f"no step starting with {first} under {directory}")
    acc, spans = defaultdict(list), []
    for st in steps:
        t0 = min(a for _, a, _ in st)
        seen = defaultdict(int)
        for name, a, b in sorted(st, key=lambda t: t[1]):
            seen[name] += 1
            key = name if seen[name] == 1 else f"{name}#{seen[name]}"
            acc[key].append(((a - t0) / 1e3, (b - t0) / 1e3))
        spans.append((max(b for _, _, b in st) - t0) / 1e3)
    kern = [(k, sum(x for x, _ in v) / len(v), sum(y for _, y in v) / len(v)) for k, v in acc.items()
            if len(v) == len(steps)]
    kern.sort(key=lambda t: t[1])
    return {"steps": len(steps), "kernels": kern, "span": sum(spans) / len(spans)}


def main(argv):
    if len(argv) >= 2 and argv[0] == "stats":
        st = kernel_stats(argv[1])
        print(f"{'kernel':20s} {'calls':>6s} {'avg_us':>10s} {'min_us':>10s} {'max_us':>10s}")
        for k, v in sorted(st.items(), key=lambda kv: -kv[1]["avg_us"] * kv[1]["calls"]):
            print(f"{k:20s} {v['calls']:6d} {v['avg_us']:10.2f} {v['min_us']:10.2f} {v['max_us']:10.2f}")
        return 0
    if len(argv) >= 3 and argv[0] == "traffic":
        t = traffic(argv[1], argv[2])
        print(f"fetch_factor = {t['fetch_factor']:.6f}")
        print(f"write_factor = {t['write_factor']:.6f}")
        for k, v in sorted(t["kernels"].items()):
            print(f"{k}.fetch_bytes = {v['fetch_bytes']:.0f}")
            print(f"{k}.write_bytes = {v['write_bytes']:.0f}")
            print(f"{k}.traffic_bytes = {v['traffic_bytes']:.0f}")
        print(f"source_sha256 = {source_sha256()}")
        return 0
    if len(argv) >= 2 and argv[0] == "timeline":
        tl = timeline(argv[1], argv[2] if len(argv) > 2 else "prefill_concurrent", int(argv[3]) if len(argv) > 3 else 0)
        print(f"{tl['steps']} steps; offsets from the start of each step's first kernel, us (mean)")
        print(f"{'kernel':20s} {'start':>8s} {'end':>8s} {'dur':>8s}")
        for k, a, b in tl["kernels"]:
            print(f"{k:20s} {a:8.1f} {b:8.1f} {b - a:8.1f}")
        print(f"{'step span':20s} {'':8s} {tl['span']:8.1f}")
        return 0
    if len(argv) >= 2 and argv[0] == "counters":
        tab = counter_table(*argv[1:])
        ctrs = sorted({c for row in tab.values() for c in row})
        print("kernel," + ",".join(ctrs))
        for k in sorted(tab):
            print(k + "," + ",".join(f"{tab[k][c]:.6g}" if c in tab[k] else "" for c in ctrs))
        return 0
    if len(argv) >= 2 and argv[0] == "bytes":
        tab = counter_table(*argv[1:])
        print(f"{'kernel':20s} {'read_MB':>10s} {'write_MB':>10s}")
        for k in sorted(tab):
            rd, wr = request_bytes(tab[k])
            if rd is None and wr is None:
                continue
            print(f"{k:20s} {'' if rd is None else f'{rd / 1e6:10.2f}':>10s} "
                  f"{'' if wr is None else f'{wr / 1e6:10.2f}':>10s}")
        for k in sorted(tab):
            rd, wr = request_bytes(tab[k])
            if rd is not None and wr is not None and k in {s for _, s in KERNELS} | set(PROJ_NAMES):
                print(f"{k}.traffic_bytes = {rd + wr:.0f}")
        print(f"source_sha256 = {source_sha256()}")
        return 0
    if len(argv) >= 2 and argv[0] == "summary":
        print(summary(*argv[1:]), end="")
        return 0
    print(__doc__, file=sys.stderr)
    return 2


# MI355X: 256 compute units of 4 SIMDs in 8 XCDs.  GRBM_GUI_ACTIVE is counted by every XCD
# and the per-dispatch value sums them; the MFMA busy counter sums every SIMD.
N_SIMD, N_XCD = 1024, 8
MFMA_FLOPS_PER_MOP = 512   # SQ_INSTS_VALU_MFMA_MOPS_* count 512-flop units


def summary(*directories: str) -> str:
    """Counter summary of the library's kernels (text, see the module docstring)."""
    tab = counter_table(*directories)
    known = {short for _, short in KERNELS} | set(PROJ_NAMES)
    rows = []
    keys = []
    for k in sorted(tab):
        if k not in known:
            continue
        r = tab[k]
        rd, wr = request_bytes(r)
        gui = r.get("GRBM_GUI_ACTIVE")
        gui_x = gui / N_XCD if gui else None
        mops = None
        if "SQ_INSTS_VALU_MFMA_MOPS_F16" in r or "SQ_INSTS_VALU_MFMA_MOPS_BF16" in r:
            mops = r.get("SQ_INSTS_VALU_MFMA_MOPS_F16", 0.0) + r.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0)
        flops = None if mops is None else mops * MFMA_FLOPS_PER_MOP
        busy = None
        if "SQ_VALU_MFMA_BUSY_CYCLES" in r and gui_x:
            busy = r["SQ_VALU_MFMA_BUSY_CYCLES"] / (N_SIMD * gui_x)
        valu = r.get("SQ_INSTS_VALU")
        lds = r.get("SQ_INSTS_LDS")
        conf = r.get("SQ_LDS_BANK_CONFLICT")
        rows.append((k, gui_x, flops, busy, valu, lds, conf, rd, wr))
        for name, val in (("gui_cycles_per_xcd", gui_x), ("mfma_flops", flops), ("mfma_busy_frac", busy),
                          ("valu_insts", valu), ("lds_insts", lds), ("lds_bank_conflict_cycles", conf),
                          ("read_bytes", rd), ("write_bytes", wr),
                          ("traffic_bytes", None if rd is None or wr is None else rd + wr)):
            if val is not None:
                keys.append(f"{k}.{name} = {val:.6g}" if name.endswith("frac") else f"{k}.{name} = {val:.0f}")

    def f(v, scale=1.0, fmt="{:10.2f}"):
        return f"{'-':>10s}" if v is None else fmt.format(v / scale)
    out = [f"{'kernel':22s} {'cycles/XCD':>10s} {'MFMA GF':>10s} {'MFMA busy':>10s} {'VALU k':>10s} "
           f"{'LDS k':>10s} {'conflict k':>10s} {'read MB':>10s} {'write MB':>10s}"]
    for k, gui_x, flops, busy, valu, lds, conf, rd, wr in rows:
        out.append(f"{k:22s} {f(gui_x, 1, '{:10.0f}')} {f(flops, 1e9)} {f(busy, 1, '{:10.4f}')} {f(valu, 1e3, '{:10.1f}')} "
                   f"{f(lds, 1e3, '{:10.1f}')} {f(conf, 1e3, '{:10.1f}')} {f(rd, 1e6)} {f(wr, 1e6)}")
    out.append("")
    out += keys
    out.append(f"source_sha256 = {source_sha256()}")
    return "\n".join(out) + "\n"


def read_traffic(path: str) -> dict:
    """Parse the `key = value` lines written by `traffic`; {} when the file is absent."""
    if not os.path.exists(path):
        return {}
    out = {}
    with open(path) as f:
        for line in f:
            if " = " in line and not line.startswith(("#", " ", "|")):
                key, val = line.split(" = ", 1)
                out[key.strip()] = val.strip()
    return out


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
