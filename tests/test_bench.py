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
