"""Host logic of the rocprofv3 harness (gated_gqa_causal_amd/rocprof_harness.py):
CSV parsing, the per-kernel figures and the traffic records bench.py reads.
The CSV headers are those rocprofv3 (ROCm 7.2) writes."""

import importlib.util
import json
import os

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _load(path, name):
    spec = importlib.util.spec_from_file_location(name, path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


H = _load(os.path.join(ROOT, "gated_gqa_causal_amd", "rocprof_harness.py"), "rocprof_harness_under_test")
BENCH = _load(os.path.join(ROOT, "bench.py"), "bench_under_test")

STATS_HDR = '"Name","Calls","TotalDurationNs","AverageNs","Percentage","MinNs","MaxNs","StdDev"\n'
CTR_HDR = ('"Correlation_Id","Dispatch_Id","Agent_Id","Queue_Id","Process_Id","Thread_Id","Grid_Size",'
           '"Kernel_Id","Kernel_Name","Workgroup_Size","LDS_Block_Size","Scratch_Size","VGPR_Count",'
           '"Accum_VGPR_Count","SGPR_Count","Counter_Name","Counter_Value","Start_Timestamp","End_Timestamp"\n')
TRACE_HDR = ('"Kind","Agent_Id","Queue_Id","Stream_Id","Thread_Id","Dispatch_Id","Kernel_Id","Kernel_Name",'
             '"Correlation_Id","Start_Timestamp","End_Timestamp","LDS_Block_Size","Scratch_Size","VGPR_Count",'
             '"Accum_VGPR_Count","SGPR_Count","Workgroup_Size_X","Workgroup_Size_Y","Workgroup_Size_Z",'
             '"Grid_Size_X","Grid_Size_Y","Grid_Size_Z"\n')
ATT = "void ga::attn_fwd8<false, false>(ga::AttnParams)"
PRO = "void ga::kv_prologue<false>(ga::KvPrologueParams)"


def _ctr_row(disp, name, ctr, val, t0, t1):
    return f'{disp},{disp},"Agent 1",1,9,9,512,3,"{name}",512,0,0,8,0,32,"{ctr}",{val},{t0},{t1}\n'


def _trace_row(disp, name, t0, t1):
    return f'"KERNEL_DISPATCH","Agent 1",1,0,9,{disp},3,"{name}",{disp},{t0},{t1},0,0,8,0,32,512,1,1,512,1,1\n'


def _write(d, fname, text):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, fname), "w") as f:
        f.write(text)


def test_kernel_stats_and_counters(tmp_path):
    _write(str(tmp_path / "trace" / "host"), "12_kernel_stats.csv",
           STATS_HDR + f'"{ATT}",4,2000000,500000.0,97.0,450000,550000,10.0\n'
           + f'"{PRO}",4,60000,15000.0,3.0,14000,16000,1.0\n')
    st = H.read_kernel_stats(str(tmp_path / "trace"))
    assert st[ATT] == {"calls": 4, "avg_ns": 500000.0, "min_ns": 450000.0, "max_ns": 550000.0}
    # Two dispatches; dispatch 2's FETCH_SIZE comes in two rows (summed), and
    # the mean over dispatches is taken after that.
    _write(str(tmp_path / "fetch" / "host"), "12_counter_collection.csv",
           CTR_HDR + _ctr_row(1, ATT, "FETCH_SIZE", 100.0, 1000, 401000)
           + _ctr_row(2, ATT, "FETCH_SIZE", 60.0, 2000, 602000)
           + _ctr_row(2, ATT, "FETCH_SIZE", 40.0, 2000, 602000))
    c = H.read_counters(str(tmp_path / "fetch"))
    assert c[ATT]["FETCH_SIZE"] == pytest.approx(100.0)
    assert c[ATT]["dispatch_ns"] == pytest.approx(500000.0)
    c1 = H.read_counters(str(tmp_path / "fetch"), last=1)       # the last dispatch only
    assert c1[ATT]["FETCH_SIZE"] == pytest.approx(100.0) and c1[ATT]["dispatch_ns"] == 600000.0
    # Per-dispatch durations in dispatch order (rows out of order in the file).
    _write(str(tmp_path / "trace" / "host"), "12_kernel_trace.csv",
           TRACE_HDR + _trace_row(3, ATT, 100, 400) + _trace_row(1, ATT, 0, 50) + _trace_row(2, PRO, 60, 90))
    assert H.read_dispatches(str(tmp_path / "trace")) == {ATT: [50.0, 300.0], PRO: [30.0]}


def _fake_run(tmp_path):
    d = str(tmp_path)
    _write(os.path.join(d, "trace", "h"), "1_kernel_stats.csv",
           STATS_HDR + f'"{ATT}",2,1000000,500000.0,97.0,490000,510000,1.0\n'
           + f'"{PRO}",2,30000,15000.0,3.0,14000,16000,1.0\n'
           + '"__amd_rocclr_copyBuffer",1,3000,3000.0,0.1,3000,3000,0.0\n')
    # A one-time set-up launch (60 us), then the two timed steps at 0.5 ms.
    _write(os.path.join(d, "trace", "h"), "1_kernel_trace.csv",
           TRACE_HDR + _trace_row(1, ATT, 0, 60000) + _trace_row(2, PRO, 0, 15000)
           + _trace_row(3, ATT, 100000, 600000) + _trace_row(4, PRO, 0, 15000)
           + _trace_row(5, ATT, 700000, 1200000))
    # 0.5 ms per attention launch; 1000 KiB fetched (x2 after calibration),
    # 500 KiB written; 1e9 MOPS = 512 GFLOP; 8 XCDs x 850,000 cycles over a
    # 0.5 ms counter dispatch = 1.7 GHz; busy = half the SIMD-cycles.
    rows = {"fetch": [("FETCH_SIZE", 1000.0)], "write": [("WRITE_SIZE", 500.0)],
            "mfma": [("SQ_INSTS_VALU_MFMA_MOPS_BF16", 1e9), ("GRBM_GUI_ACTIVE", 8 * 850000.0),
                     ("SQ_VALU_MFMA_BUSY_CYCLES", 0.5 * 850000.0 * 1024)],
            "lds": [("SQ_LDS_BANK_CONFLICT", 10.0), ("SQ_LDS_IDX_ACTIVE", 1000.0)]}
    counters = {}
    for p, ctrs in rows.items():
        _write(os.path.join(d, p, "h"), "1_counter_collection.csv",
               CTR_HDR + "".join(_ctr_row(5, ATT, n, v, 0, 500000) for n, v in ctrs)
               + _ctr_row(6, PRO, "GRBM_GUI_ACTIVE", 1e6, 0, 15000))
        counters[p] = H.read_counters(os.path.join(d, p))
    alg = {"attention": {"flop": 500e9, "read_bytes": 1 << 20, "write_bytes": 1 << 19},
           "kv_prologue": {"read_bytes": 1 << 20, "write_bytes": 1 << 20}}
    trace = {"dir": os.path.join(d, "trace"),
             "bench": {"kernels_algorithmic": alg, "kernels_ms": {}, "ms_per_step": 0.6, "steps": 2}}
    cal = {"FETCH_SIZE": {"factor": 2.0}, "WRITE_SIZE": {"factor": 1.0}}
    return H.summarise("wl_test", [], trace, counters, cal, [["rocprofv3", "--", "python3", "bench.py"]], 256, 8)


def test_summary_figures(tmp_path):
    s = _fake_run(tmp_path)
    att = next(k for k in s["kernels"] if k["key"] == "attention")
    assert att["timed"] == 2 and att["avg_ns"] == 500000.0 and att["stats_avg_ns"] == 500000.0
    assert att["alg_tflops"] == pytest.approx(1000.0)
    assert att["alg_frac"] == pytest.approx(0.4)
    assert att["mfma_tflops"] == pytest.approx(1024.0)
    assert att["clock_ghz"] == pytest.approx(1.7)
    assert att["mfma_busy"] == pytest.approx(0.5)
    assert att["read_bytes"] == 2000 * 1024 and att["write_bytes"] == 500 * 1024
    assert att["gbs"] == pytest.approx(2500 * 1024 / 0.5e-3 / 1e9)
    assert att["lds_conflict"] == pytest.approx(0.01)
    pro = next(k for k in s["kernels"] if k["key"] == "kv_prologue")
    assert "clock_ghz" not in pro and "mfma_busy" not in pro        # no MFMAs: no clock figure
    md = H.markdown(s)
    assert "`ga::attn_fwd8<false, false>`" in md and "0.500" in md
    assert "__amd_rocclr_copyBuffer" in md.split("Other kernels")[1]


def test_merge_feeds_bench(tmp_path, monkeypatch):
    s = _fake_run(tmp_path)
    path = tmp_path / "summary.json"
    path.write_text(json.dumps(s))
    traffic = {"attention": str(tmp_path / "ta.json"), "weights": str(tmp_path / "tw.json")}
    monkeypatch.setattr(H, "TRAFFIC", traffic)

    class A:
        summaries = [str(path)]
    assert H.cmd_merge(A) == 0
    rec = json.loads(open(traffic["attention"]).read())["workloads"]["wl_test"]
    assert rec["bytes_per_launch"] == 2500 * 1024 and rec["kernel"] == "ga::attn_fwd8<false, false>"
    assert not os.path.exists(traffic["weights"])
    # bench.py reads the record while the kernel source is unchanged.
    assert BENCH.measured_traffic("wl_test", traffic["attention"]) == 2500 * 1024
    assert BENCH.measured_traffic("other", traffic["attention"]) is None
    monkeypatch.setattr(BENCH, "kernel_source_hash", lambda: "0" * 16)
    assert BENCH.measured_traffic("wl_test", traffic["attention"]) is None


def test_committed_traffic_records_name_their_workload():
    for key in ("attention", "weights"):
        rec = json.loads(open(H.TRAFFIC[key]).read())
        assert rec["workloads"], key
        for w, r in rec["workloads"].items():
            assert {"kernel", "kernel_source_sha256_16", "bytes_per_launch"} <= set(r), (key, w)


def test_kernel_algorithmic_bytes():
    import synth
    p = synth.make_problem(T=100, n_q_heads=4, n_kv_heads=2, seed=1)
    a = BENCH.kernel_algorithmic(p, p.rows, p.T, p.T, p.flops(), False)
    # q|gate (rows x Hq x 2D bf16) + K and V^T (2 x Hkv x T x D bf16) + cos/sin (2 x rows x 32 fp32).
    assert a["attention"]["read_bytes"] == 100 * 4 * 512 * 2 + 2 * 2 * 100 * 256 * 2 + 2 * 100 * 32 * 4
    assert a["attention"]["write_bytes"] == 100 * 4 * 256 * 2
    assert "mask_pack" not in a and "weights" not in a
    pm = synth.make_problem(T=100, n_q_heads=4, n_kv_heads=2, seed=1, mask_budget=10)
    am = BENCH.kernel_algorithmic(pm, pm.rows, pm.T, pm.T, pm.flops(), True)
    words = sum(i // 32 + 1 for i in range(100))
    assert am["mask_pack"]["read_bytes"] == 32 * words
    assert am["attention"]["read_bytes"] == a["attention"]["read_bytes"] + 4 * words
    assert am["weights"]["write_bytes"] == 100 * 4 * 100 * 2
