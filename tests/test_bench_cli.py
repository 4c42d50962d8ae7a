"""Host-side checks of bench.py's command line (no GPU needed)."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    # one process drives one GPU; N > 1 must stop before touching a device
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True, timeout=120)
    assert p.returncode == 2
    assert "one GPU" in p.stderr
    assert p.stdout == ""


def test_profiled_traffic_is_read_only_for_the_profiled_kernel_source(tmp_path, monkeypatch):
    sys.path.insert(0, ROOT)
    import bench
    # the committed summaries carry a stamp of the attention sources they were taken with
    for name in ("video-dit-L", "video-dit-S"):
        t = bench.profiled_traffic(name)
        if t is not None:
            assert t["total"] == t["read"] + t["write"] > 0
    # a summary whose stamp does not match the sources yields no traffic figure
    prof = tmp_path / "profiles"
    prof.mkdir()
    (prof / "kernels_x.md").write_text(
        "attn_bf16_kernel traffic_bytes_per_launch=3 read=2 write=1 avg_ns=5 source=0000000000000000\n")
    csrc = tmp_path / "piecewise_block_sparse_amd" / "csrc"
    csrc.mkdir(parents=True)
    for f in ("attn_bf16.hip", "lds_stream.hpp", "common.hpp", "topk.hpp"):
        (csrc / f).write_text("x")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.profiled_traffic("x") is None
    assert bench.profiled_traffic("missing") is None


def test_phase_counters_follow_each_lines_own_source_stamp(tmp_path, monkeypatch):
    sys.path.insert(0, ROOT)
    import bench
    csrc = tmp_path / "piecewise_block_sparse_amd" / "csrc"
    csrc.mkdir(parents=True)
    for f in ("attn_bf16.hip", "lds_stream.hpp", "common.hpp", "topk.hpp", "stats.hip"):
        (csrc / f).write_text(f)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    attn = bench._source_stamp(bench._ATTN_SOURCES)
    stats = bench._source_stamp(bench._STATS_SOURCES)
    prof = tmp_path / "profiles"
    prof.mkdir()
    (prof / "kernels_x.md").write_text(
        "text before\n"
        f"exact_phase mfma_gflop=2500.0 mfma_busy=0.5 coexec=0.25 clock_ghz=2.0 avg_ns=2000000 source={attn}\n"
        f"approx_phase mfma_gflop=10.0 read_bytes=5 write_bytes=0 avg_ns=0 operand_stream_bytes=7 source={attn}\n"
        f"statistics avg_ns=1000 algorithmic_bytes=4000000 read_bytes=1 write_bytes=2 pass1_write_bytes=2 "
        f"source={stats}\n")
    c = bench.phase_counters("x")
    assert c["exact_phase"]["profiled_tflops"] == 2500.0 / 2e-3 / 1e3           # 1250 TFLOP/s
    assert abs(c["exact_phase"]["frac"] - 0.5) < 1e-12
    assert c["approx_phase"]["operand_stream_gbs"] is None                     # no time, no rate
    assert abs(c["statistics"]["algorithmic_gbs"] - 4000.0) < 1e-9
    assert abs(c["statistics"]["frac"] - 0.5) < 1e-12
    # a change to stats.hip drops the statistics line only
    (csrc / "stats.hip").write_text("changed")
    c = bench.phase_counters("x")
    assert "statistics" not in c and "exact_phase" in c
    # a change to the attention kernel drops its lines
    (csrc / "attn_bf16.hip").write_text("changed")
    assert bench.phase_counters("x") is None


def test_flops_model_matches_the_stated_algorithmic_work():
    sys.path.insert(0, ROOT)
    import bench
    from piecewise_block_sparse_amd import workloads as wl
    w = wl.WORKLOADS[4]                       # video-DiT-L: 40 heads, 32K, d 128, B 128, k 32
    f = bench.flops(w, w.k)
    assert f["exact"] == 40 * 256 * 4 * 128 * (32 * 128) * 128          # 2748.8 GFLOP
    assert round(f["exact"] / 1e9, 1) == 2748.8
    assert f["step"] == f["exact"] + f["approx"] + f["stats"] + f["route"]
    json.dumps(f)
