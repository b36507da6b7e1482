"""Host-side summaries of rocprofv3 output (hybrid_linear_attention_gated_amd.profiling),
checked on small synthetic CSV files with known answers."""
import csv
import os

import pytest

from hybrid_linear_attention_gated_amd import profiling

LOCAL = "void gdn::chunk_local_kernel<128, true, __hip_bfloat16>(float const*, ...)"
STATE = "void gdn::state_pass_kernel<128, true>(char const*, ...)"
DECODE = "void gdn::decode_kernel<float, 128, 128, false>(...)"
COPY = "void at::native::elementwise_kernel<128, 4, ...>(int, ...)"


def _write(path, fields, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=fields)
        w.writeheader()
        w.writerows(rows)


def _trace(tmp_path, launches):
    rows = [{"Kernel_Name": n, "Start_Timestamp": a, "End_Timestamp": b} for n, a, b in launches]
    _write(str(tmp_path / "t" / "run_kernel_trace.csv"), ["Kernel_Name", "Start_Timestamp", "End_Timestamp"], rows)
    return str(tmp_path / "t")


def test_short_names():
    assert profiling.short_name(LOCAL) == "chunk_local_fused"
    assert profiling.short_name(LOCAL.replace("true", "false")) == "chunk_local"
    assert profiling.short_name(STATE) == "state_pass"
    assert profiling.short_name(
        "void gdn::prefill_concurrent_kernel<128, true, __hip_bfloat16, __hip_bfloat16>(...)") == "prefill_concurrent"
    assert profiling.short_name(
        "void gdn::prefill_concurrent_kernel<128, true, float, __hip_bfloat16>(...)") == "prefill_concurrent_x32"
    assert profiling.short_name(
        "_ZN3gdn25prefill_concurrent_kernelILi128ELb1EfDF16bEEvNS_9LocalArgsIT1_T2_EENS_9StateArgsEi") == \
        "prefill_concurrent_x32"
    assert profiling.short_name(
        "_ZN3gdn25prefill_concurrent_kernelILi128ELb1EfDF16bLb0EEEvNS_9LocalArgsIT1_T2_EENS_9StateArgsEi") == \
        "prefill_concurrent_x32"
    assert profiling.short_name(
        "_ZN3gdn25prefill_concurrent_kernelILi128ELb1EfDF16bLb1EEEvNS_9LocalArgsIT1_T2_EENS_9StateArgsEi") == \
        "prefill_concurrent_norm"
    assert profiling.short_name(
        "void gdn::prefill_concurrent_kernel<128, true, float, __hip_bfloat16, true>(...)") == "prefill_concurrent_norm"
    assert profiling.short_name(
        "void gdn::prefill_concurrent_kernel<128, true, float, __hip_bfloat16, false>(...)") == "prefill_concurrent_x32"
    assert profiling.short_name(DECODE) == "decode"
    assert profiling.short_name(DECODE.replace("false>", "true>")) == "decode_gated"
    assert profiling.short_name(COPY) == "copy"
    assert profiling.short_name("void gdn::proj_kernel<128, 128, 64>(gdn::ProjArgs)") == "proj_256"
    assert profiling.short_name("_ZN3gdn11proj_kernelILi128ELi128ELi64EEEvNS_8ProjArgsE") == "proj_256"
    assert profiling.short_name("void gdn::proj_kernel<64, 64, 128>(gdn::ProjArgs)") == "proj_128"
    assert profiling.short_name("_ZN3gdn11proj_kernelILi128ELi128ELi64ELi0EEEvNS_8ProjArgsE") == "proj_256"
    assert profiling.short_name("_ZN3gdn11proj_kernelILi128ELi128ELi64ELi1EEEvNS_8ProjArgsE") == "proj_256_layer"
    assert profiling.short_name("void gdn::proj_kernel<64, 64, 128, 1>(gdn::ProjArgs)") == "proj_128_layer"
    assert profiling.short_name("_ZN3gdn11proj_kernelILi128ELi128ELi64ELi2EEEvNS_8ProjArgsE") == "proj_256_layer"
    assert profiling.short_name("void gdn::proj_kernel<128, 128, 64, 2>(gdn::ProjArgs)") == "proj_256_layer"
    assert profiling.short_name("_ZN3gdn18chunk_local_kernelILi128ELb1EfDF16bEEvPKf") == "chunk_local_fused_x32"
    assert profiling.short_name("_ZN3gdn18chunk_local_kernelILi128ELb1EDF16bS1_EEvPKf") == "chunk_local_fused"


def test_kernel_stats(tmp_path):
    d = _trace(tmp_path, [(STATE, 0, 10_000), (STATE, 20_000, 50_000), (DECODE, 60_000, 61_000)])
    st = profiling.kernel_stats(d)
    assert st["state_pass"] == {"calls": 2, "avg_us": 20.0, "min_us": 10.0, "max_us": 30.0}
    assert st["decode"]["calls"] == 1 and st["decode"]["avg_us"] == 1.0


def test_timeline_offsets_and_skip(tmp_path):
    # four steps: the state pass, the chunk-local kernel overlapping it, then decode (twice,
    # to check occurrence keys); the first step is dropped as warm-up; in the last step the
    # chunk-local kernel starts 2 us before the state pass and still belongs to that step
    launches = []
    for base, local0, extra in ((0, 10_000, 999_000), (1_000_000, 10_000, 0), (2_000_000, 10_000, 2_000),
                                (3_000_000, -2_000, 0)):
        launches += [(STATE, base, base + 130_000), (LOCAL, base + local0, base + 110_000 + extra),
                     (DECODE, base + 131_000, base + 231_000), (DECODE, base + 232_000, base + 330_000)]
    tl = profiling.timeline(_trace(tmp_path, launches), "state_pass", 1)
    assert tl["steps"] == 3
    got = {k: (a, b) for k, a, b in tl["kernels"]}
    assert [k for k, _, _ in tl["kernels"]] == ["state_pass", "chunk_local_fused", "decode", "decode#2"]
    # offsets count from each step's first start: the last step starts with the chunk-local kernel
    assert got["chunk_local_fused"] == pytest.approx(((10 + 10 + 0) / 3, (110 + 112 + 112) / 3))
    assert got["state_pass"] == pytest.approx(((0 + 0 + 2) / 3, (130 + 130 + 132) / 3))
    assert got["decode#2"] == pytest.approx(((232 + 232 + 234) / 3, (330 + 330 + 332) / 3))
    assert tl["span"] == pytest.approx((330 + 330 + 332) / 3)
    with pytest.raises(RuntimeError):
        profiling.timeline(_trace(tmp_path, launches), "state_pass", 4)


def test_traffic_scaled_by_copy(tmp_path):
    kib = profiling.COPY_BYTES / 1024.0

    def counters(sub, counter, copy_kib, state_kib):
        rows = [{"Kernel_Name": COPY, "Counter_Name": counter, "Counter_Value": copy_kib},
                {"Kernel_Name": STATE, "Counter_Name": counter, "Counter_Value": state_kib},
                {"Kernel_Name": STATE, "Counter_Name": counter, "Counter_Value": 3 * state_kib}]
        _write(str(tmp_path / sub / "run_counter_collection.csv"), ["Kernel_Name", "Counter_Name", "Counter_Value"],
               rows)
        return str(tmp_path / sub)

    # the counters read half (fetch) and twice (write) the copy's true bytes
    f = counters("f", "FETCH_SIZE", kib / 2, 100.0)
    w = counters("w", "WRITE_SIZE", kib * 2, 100.0)
    t = profiling.traffic(f, w)
    assert t["fetch_factor"] == pytest.approx(2.0) and t["write_factor"] == pytest.approx(0.5)
    k = t["kernels"]["state_pass"]
    assert k["dispatches"] == 2
    assert k["fetch_bytes"] == pytest.approx(200.0 * 1024 * 2.0)
    assert k["write_bytes"] == pytest.approx(200.0 * 1024 * 0.5)
    assert "copy" not in t["kernels"]


def test_counter_table_and_request_bytes(tmp_path):
    """Rows of one dispatch are summed (clock counters: the largest), dispatches averaged;
    request counts become bytes by their widths."""
    fields = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
    rows = []
    for disp, scale in ((1, 1), (2, 3)):
        for inst in range(2):   # two hardware instances listed separately
            rows += [{"Dispatch_Id": disp, "Kernel_Name": STATE, "Counter_Name": c, "Counter_Value": v * scale}
                     for c, v in (("TCC_EA0_RDREQ_32B_sum", 1), ("TCC_EA0_RDREQ_64B_sum", 2),
                                  ("TCC_EA0_RDREQ_128B_sum", 3), ("TCC_EA0_WRREQ_sum", 10),
                                  ("TCC_EA0_WRREQ_64B_sum", 4), ("GRBM_GUI_ACTIVE", 100 + inst))]
    _write(str(tmp_path / "c" / "run_counter_collection.csv"), fields, rows)
    tab = profiling.counter_table(str(tmp_path / "c"))
    row = tab["state_pass"]
    assert row["TCC_EA0_RDREQ_32B_sum"] == 4.0          # (2 + 6) / 2 dispatches
    assert row["GRBM_GUI_ACTIVE"] == (101 + 303) / 2    # the larger instance of each dispatch
    rd, wr = profiling.request_bytes(row)
    assert rd == 32 * 4 + 64 * 8 + 128 * 12
    assert wr == 32 * (40 - 16) + 64 * 16


def test_summary_figures_and_bench_reader(tmp_path, monkeypatch):
    """The counter summary turns MFMA op counts into flops (512 each), the busy counter into
    a fraction of every SIMD's share of the clock, and the request counts into bytes; the
    key = value lines it ends with are what bench.py reads back."""
    fields = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
    gui = 8 * 1000.0                     # 1000 cycles on each of the 8 XCDs
    rows = [{"Dispatch_Id": 1, "Kernel_Name": STATE, "Counter_Name": c, "Counter_Value": v}
            for c, v in (("SQ_INSTS_VALU_MFMA_MOPS_F16", 300.0), ("SQ_INSTS_VALU_MFMA_MOPS_BF16", 100.0),
                         ("SQ_VALU_MFMA_BUSY_CYCLES", 0.25 * 1024 * 1000), ("GRBM_GUI_ACTIVE", gui),
                         ("SQ_INSTS_VALU", 5000.0), ("TCC_EA0_RDREQ_32B_sum", 0.0),
                         ("TCC_EA0_RDREQ_64B_sum", 10.0), ("TCC_EA0_RDREQ_128B_sum", 20.0),
                         ("TCC_EA0_WRREQ_sum", 7.0), ("TCC_EA0_WRREQ_64B_sum", 7.0))]
    _write(str(tmp_path / "s" / "run_counter_collection.csv"), fields, rows)
    text = profiling.summary(str(tmp_path / "s"))
    path = tmp_path / "counters.txt"
    path.write_text("# header\n" + text)
    rec = profiling.read_traffic(str(path))
    assert float(rec["state_pass.mfma_flops"]) == 400 * 512
    assert float(rec["state_pass.mfma_busy_frac"]) == pytest.approx(0.25)
    assert float(rec["state_pass.gui_cycles_per_xcd"]) == 1000
    assert float(rec["state_pass.read_bytes"]) == 64 * 10 + 128 * 20
    assert float(rec["state_pass.write_bytes"]) == 64 * 7
    assert float(rec["state_pass.traffic_bytes"]) == 64 * 10 + 128 * 20 + 64 * 7
    assert rec["source_sha256"] == profiling.source_sha256()

    import importlib.util
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    spec = importlib.util.spec_from_file_location("bench_mod", os.path.join(root, "bench.py"))
    bench = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(bench)
    monkeypatch.setattr(bench, "COUNTERS_FILE", str(path))
    got = bench.measured_counters()
    assert got["state_pass"]["mfma_flops"] == 400 * 512
    assert got["state_pass"]["traffic_bytes"] == 64 * 10 + 128 * 20 + 64 * 7
    # a summary of other sources is ignored
    path.write_text(text.replace(profiling.source_sha256(), "0" * 64))
    assert bench.measured_counters() == {}
