"""Host logic of bench.py (no GPU): the one-GPU refusal, the workload table,
and the guard that reports stored HBM-traffic counters only for the kernel
sources they were taken on."""
import json
import os
import subprocess
import sys

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    out = r.stdout + r.stderr
    assert "one GPU" in out
    assert '"metric"' not in out          # no JSON line for a configuration it does not run


def test_code_only_ignores_comments_and_blank_lines():
    a = 'int f(int x) {\n  return x + 1;  // one more\n}\n'
    b = '/* a block\n   comment */\nint f(int x) {\n\n  return x + 1;\n}\n'
    assert bench.code_only(a) == bench.code_only(b)
    assert bench.code_only('const char* s = "// not a comment";') == 'const char* s = "// not a comment";'
    assert bench.code_only("int y = 2;") != bench.code_only("int y = 3;")


def test_source_hash_is_stable_and_hex():
    h = bench.kernel_source_hash()
    assert h == bench.kernel_source_hash()
    assert len(h) == 16 and int(h, 16) >= 0


def test_stored_traffic_only_for_matching_sources(tmp_path, monkeypatch):
    key = "some_kernel"
    rec = {key: {"source_hash": bench.kernel_source_hash(), "bytes_per_launch": 1234}}
    (tmp_path / "traffic.json").write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    assert bench.stored_traffic(key) == 1234
    assert bench.stored_traffic("another_kernel") is None
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "0" * 16)
    assert bench.stored_traffic(key) is None          # the kernels changed since the counters
    (tmp_path / "traffic.json").write_text("not json")
    assert bench.stored_traffic(key) is None


@pytest.mark.parametrize("name,n,batch,dirs,passes", [
    ("w1", 1024, 8, 1, 1), ("w2", 4096, 16384, 2, 1), ("w3", 1 << 22, 32, 1, 2),
    ("w4", 2048, 1024, 2, 1), ("w5", 8192 * 8192, 1, 1, 2), ("w6", 1000, 65536, 2, 1)])
def test_workload_table(name, n, batch, dirs, passes):
    s = bench.workload_spec(name)
    assert (s["n"], s["batch"], len(s["dirs"]), s["passes"]) == (n, batch, dirs, passes)
    assert s["label"]


def test_any_length_spec_keeps_about_the_same_bytes():
    for n in (1009, 1019, 10001, 4194301):
        s = bench.any_length_spec(n)
        assert s["n"] == n and s["batch"] >= 1
        assert abs(s["n"] * s["batch"] - 1000 * 65536) <= n


def test_work_per_exec_counts():
    """Algorithmic bytes and flops per exec of the five configurations."""
    f, b = bench.work_per_exec(bench.workload_spec("w2"))
    assert b == 2 * 16384 * 4096 * 8 and f == 5.0 * 4096 * 12 * 16384
    f, b = bench.work_per_exec(bench.workload_spec("w3"))
    assert b == 2 * 2 * 32 * (1 << 22) * 8 and f == 5.0 * (1 << 22) * 22 * 32    # two HBM passes
    f, b = bench.work_per_exec(bench.workload_spec("w5"))
    assert b == 2 * 2 * 8192 * 8192 * 8 and f == 5.0 * 8192 * 8192 * 26
    f, b = bench.work_per_exec(bench.workload_spec("w4"))
    assert b == 1024 * 2048 * 4 + 683 * 1024 * 8 and f == 2.5 * 2048 * 11 * 1024


def test_configs_table_covers_c1_to_c5():
    assert [c for c, _ in bench.CONFIGS] == ["c1", "c2", "c3", "c4", "c5"]
    assert set(bench.BAR_CONFIGS) == {"c2", "c3", "c5"}
    for _, w in bench.CONFIGS:
        assert w in bench.TRAFFIC_KEY


def test_cpu_model_is_a_name():
    m = bench.cpu_model()
    assert isinstance(m, str) and m


def test_summarize_trace(tmp_path):
    """Per-kernel median/mean/min/max of a kernel trace in rocprofv3's CSV layout."""
    cols = ["Kind", "Kernel_Name", "Start_Timestamp", "End_Timestamp", "LDS_Block_Size", "Scratch_Size",
            "VGPR_Count", "Accum_VGPR_Count"]
    rows = [["KERNEL_DISPATCH", "k_a", 1000, 3000, 512, 0, 52, 0],
            ["KERNEL_DISPATCH", "k_a", 5000, 9000, 512, 0, 52, 0],
            ["KERNEL_DISPATCH", "k_a", 10000, 13000, 512, 0, 52, 0],
            ["KERNEL_DISPATCH", "k_b", 20000, 30000, 0, 0, 128, 4]]
    p = tmp_path / "t.csv"
    p.write_text("\n".join(",".join(f'"{v}"' for v in r) for r in [cols] + rows) + "\n")
    import io
    buf = io.StringIO()
    bench.summarize_trace(str(p), out=buf)
    lines = buf.getvalue().splitlines()
    a = next(l for l in lines if "`k_a`" in l).split("|")
    assert [x.strip() for x in a[2:7]] == ["3", "3.0", "3.0", "2.0", "4.0"]
    b = next(l for l in lines if "`k_b`" in l).split("|")
    assert [x.strip() for x in b[2:9]] == ["1", "10.0", "10.0", "10.0", "10.0", "128", "4"]


def test_summarize_counters(tmp_path, monkeypatch):
    """Counter summary: calibration on the copy kernel, per-record sums."""
    cols = ["Kernel_Name", "Counter_Name", "Counter_Value"]

    def write(path, counter, vals):
        rows = [cols] + [[k, counter, v] for k, v in vals]
        path.write_text("\n".join(",".join(f'"{x}"' for x in r) for r in rows) + "\n")
    f = tmp_path / "f.csv"
    w = tmp_path / "w.csv"
    half = (1 << 29) // 2048        # the copy reads half its bytes in FETCH_SIZE KiB
    write(f, "FETCH_SIZE", [("__amd_rocclr_copyBuffer", half),
                            ("void fftamd::k_c2c_rows<4096, -1, 1>(fftamd::RowsArgs)", 262144),
                            ("void fftamd::k_c2c_rows<4096, 1, 1>(fftamd::RowsArgs)", 262144)])
    write(w, "WRITE_SIZE", [("__amd_rocclr_copyBuffer", (1 << 29) // 1024),
                            ("void fftamd::k_c2c_rows<4096, -1, 1>(fftamd::RowsArgs)", 524288),
                            ("void fftamd::k_c2c_rows<4096, 1, 1>(fftamd::RowsArgs)", 524288)])
    import io
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    rec = bench.summarize_counters(str(f), str(w), out=io.StringIO(), write_traffic=True)
    assert rec["c2c_rows_4096"] == 2 * 512 * 1024 * 1024       # 512 MiB read + 512 MiB written
    stored = json.load(open(tmp_path / "traffic.json"))
    assert stored["c2c_rows_4096"]["source_hash"] == bench.kernel_source_hash()
    assert "fourstep_2^22" not in rec                            # no counters for its kernels


def test_summarize_trace_keeps_the_timed_windows(tmp_path):
    cols = ["Kernel_Name", "Start_Timestamp", "End_Timestamp"]
    rows = [["k_a", 100, 200], ["k_a", 1000, 1100], ["k_a", 1200, 1500], ["k_a", 5000, 9000]]
    p = tmp_path / "t.csv"
    p.write_text("\n".join(",".join(f'"{v}"' for v in r) for r in [cols] + rows) + "\n")
    w = tmp_path / "w.jsonl"
    w.write_text(json.dumps({"label": "w2", "t0_ns": 900, "t1_ns": 2000}) + "\n")
    import io
    buf = io.StringIO()
    bench.summarize_trace(str(p), str(w), out=buf)
    a = next(l for l in buf.getvalue().splitlines() if "`k_a`" in l).split("|")
    assert [x.strip() for x in a[2:7]] == ["2", "0.3", "0.2", "0.1", "0.3"]


def test_summarize_pmc_merges_groups_and_derives_ratios(tmp_path):
    """LDS/VALU summary: two counter groups merged by kernel, mean per
    dispatch, conflict share, VALUBusy over per-XCD clocks, VALUUtilization."""
    cols = ["Kernel_Name", "Counter_Name", "Counter_Value"]
    k = "void fftamd::k_fs_cols<2048, -1, 16, false>(fftamd::FourStepArgs)"

    def write(path, rows):
        path.write_text("\n".join(",".join(f'"{x}"' for x in r) for r in [cols] + rows) + "\n")
    lds, valu = tmp_path / "lds.csv", tmp_path / "valu.csv"
    write(lds, [[k, "SQ_LDS_IDX_ACTIVE", 1000], [k, "SQ_LDS_BANK_CONFLICT", 250], [k, "SQ_INSTS_LDS", 10],
                [k, "SQ_LDS_IDX_ACTIVE", 3000], [k, "SQ_LDS_BANK_CONFLICT", 750], [k, "SQ_INSTS_LDS", 30],
                ["__amd_rocclr_copyBuffer", "SQ_INSTS_LDS", 5]])
    # 256 CUs busy half of the per-XCD clocks; 48 of 64 lanes active
    write(valu, [[k, "SQ_ACTIVE_INST_VALU", 256 * 500], [k, "GRBM_GUI_ACTIVE", 8 * 1000],
                 [k, "SQ_THREAD_CYCLES_VALU", 48 * 256 * 500], [k, "SQ_INSTS_VALU", 77]])
    import io
    buf = io.StringIO()
    bench.summarize_pmc([str(lds), str(valu)], out=buf)
    lines = [l for l in buf.getvalue().splitlines() if l.startswith("| `")]
    assert len(lines) == 1                                       # torch's and the copy's kernels left out
    c = [x.strip() for x in lines[0].split("|")[1:-1]]
    assert c[0] == "`fftamd::k_fs_cols<2048, -1, 16, false>`"
    assert c[1] == "2"                                           # dispatches
    assert c[2:6] == ["20", "2000", "500", "0.250"]              # means per dispatch and the share
    assert c[6:9] == ["77", "50.0", "75.0"]
