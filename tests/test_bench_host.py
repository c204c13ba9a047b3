"""Host logic of bench.py that runs without a GPU: the one-GPU guard, the algorithmic
byte counts the roofline divides by, and the rule that counter traffic is reported only
for the kernel sources it was measured on."""

import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

B_ROW = 7168 * 2


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_algorithmic_bytes():
    # consumer at TP=8, M=4096 with residual: TP slot reads + residual + gamma + out and
    # residual_out + TP re-arm writes
    assert bench.reduce_bytes(8, 4096, True) == (8 + 1 + 2 + 8) * 4096 * B_ROW + B_ROW == 1_115_699_200
    assert bench.reduce_bytes(8, 4, False) == (8 + 2 + 8) * 4 * B_ROW + B_ROW
    # push: every slot row read once and written once
    assert bench.push_bytes(8, 4096) == 2 * 8 * 4096 * B_ROW == 939_524_096
    # Gather TP=8, M=32, S=896: push reads and writes every word; the poll reads them,
    # copies them out and re-arms them (or only reads them, without copy)
    assert bench.gather_bytes(8, 32, 896) == (1_835_008, 2_752_512)
    assert bench.gather_bytes(8, 32, 896, copy=False)[1] == 917_504
    # two-shot at TP=8, M=4096: owner reads and re-arms the TP slots and writes the row
    assert bench.twoshot_bytes(8, 4096) == (998_244_352, 3 * 4096 * B_ROW)


def test_sources_hash_is_stable():
    h = bench.kernel_sources_hash()
    assert h == bench.kernel_sources_hash()
    assert len(h) == 16 and int(h, 16) >= 0


def test_traffic_only_for_the_measured_sources(tmp_path, monkeypatch):
    key = "reduce_norm_tp8_m4096_res"
    prof = tmp_path / "profiles"
    prof.mkdir()
    sha = bench.kernel_sources_hash()
    rec = {key: {"bytes_per_launch": 123, "sources_sha": sha}}
    (prof / "hbm_traffic.json").write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_sources_hash", lambda: sha)
    assert bench.committed_traffic(key) == 123
    rec[key]["sources_sha"] = "0" * 16
    (prof / "hbm_traffic.json").write_text(json.dumps(rec))
    assert bench.committed_traffic(key) is None
    assert bench.committed_traffic("no_such_kernel") is None


def test_committed_profiles_name_their_command():
    """Every committed kernel summary gives the command that made it and the sources it
    measured."""
    names = ["arnorm_tp8_m4_kernel_stats.md", "arnorm_tp8_m4096_kernel_stats.md",
             "gather_tp8_m32_s896_kernel_stats.md", "twoshot_tp8_kernel_stats.md",
             "arnorm_tp8_m4096_hbm_traffic.md"]
    for n in names:
        with open(os.path.join(ROOT, "profiles", n)) as f:
            text = f.read()
        assert "rocprofv3" in text and "python bench.py" in text and "sha256" in text, n


def test_profile_table_median_from_trace(tmp_path):
    """The profile summary's median column comes from the per-dispatch kernel trace."""
    stats = tmp_path / "k_kernel_stats.csv"
    stats.write_text('"Name","Calls","TotalDurationNs","AverageNs","Percentage","MinNs","MaxNs","StdDev"\n'
                     '"void arn::k(int)","3","9000","3000","100.0","1000","5000","0"\n')
    trace = tmp_path / "k_kernel_trace.csv"
    trace.write_text('"Kernel_Name","Start_Timestamp","End_Timestamp"\n'
                     '"void arn::k(int)","100","1100"\n"void arn::k(int)","2000","7000"\n'
                     '"void arn::k(int)","9000","12000"\n')
    _, table = bench._stats_table(str(stats), str(trace))
    assert "median µs" in table
    assert "| `arn::k` | 3 | 3.00 | 3.00 | 1.00 | 5.00 | 100.0 % |" in table
    _, plain = bench._stats_table(str(stats), str(tmp_path / "absent.csv"))
    assert "median" not in plain and "| `arn::k` | 3 | 3.00 | 1.00 | 5.00 | 100.0 % |" in plain


def test_profile_shape_table(tmp_path):
    """Launch shapes of the library's kernels are told apart by grid size."""
    trace = tmp_path / "lat_kernel_trace.csv"
    trace.write_text('"Kernel_Name","Start_Timestamp","End_Timestamp","Grid_Size_X","Workgroup_Size_X"\n'
                     '"void arn::k(int)","0","1000","128","128"\n"void arn::k(int)","0","3000","128","128"\n'
                     '"void arn::k(int)","0","5000","896","128"\n"void at::native::other()","0","9","1","1"\n')
    table = bench._shape_table(str(trace))
    assert "| `arn::k` | 128 | 128 | 2 | 2.00 | 2.00 |" in table
    assert "| `arn::k` | 896 | 128 | 1 | 5.00 | 5.00 |" in table
    assert "other" not in table
    assert bench._shape_table(str(tmp_path / "absent.csv")) is None
