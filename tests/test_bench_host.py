"""Host-side logic of bench.py, on the CPU: the refusals that need no GPU,
the traffic figure from two rocprofv3 counter files, and the check that
keeps a traffic figure from being reported for a changed kernel."""
import csv
import io
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def run_bench(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=120)


def test_more_than_one_gpu_is_refused():
    r = run_bench("--gpus", "2")
    assert r.returncode == 2 and "one GPU only" in r.stderr


def test_rank_environment_is_refused():
    env = dict(os.environ, WORLD_SIZE="2")
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")], capture_output=True,
                       text=True, timeout=120, env=env)
    assert r.returncode == 2 and "one GPU only" in r.stderr


@pytest.mark.parametrize("args,msg", [(["--vocab-shard", "0"], "at least 1"),
                                      (["--mode", "tree", "--workload", "5"], "does not run"),
                                      (["--mode", "sample", "--workload", "4"], "does not run")])
def test_bad_arguments_are_refused(args, msg):
    r = run_bench(*args)
    assert r.returncode == 2 and msg in r.stderr


def write_counters(path, counter, rows):
    """A counter_collection.csv as rocprofv3 writes it: one row per dispatch."""
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for i, (name, kib) in enumerate(rows):
            w.writerow({"Dispatch_Id": i + 1, "Kernel_Name": name, "Counter_Name": counter,
                        "Counter_Value": kib})


STATS = "void sv::k_softmax_stats<2, true>(sv::StatsArgs)"
COPY = "void at::native::elementwise_kernel<...copy...>"


def test_traffic_scales_each_counter_by_the_calibration_copy(tmp_path):
    """A copy of 2^30 bytes reads 1.25x and writes 0.5x its size on these
    counters: the kernel's figures are divided by the same factors."""
    gib = 1 << 30
    fetch = tmp_path / "fetch.csv"
    write = tmp_path / "write.csv"
    write_counters(fetch, "FETCH_SIZE", [(STATS, 1000.0), ("other", 5.0), (STATS, 1200.0),
                                         (COPY, 1.25 * gib / 1024)])
    write_counters(write, "WRITE_SIZE", [(STATS, 10.0), (STATS, 30.0), (COPY, 0.5 * gib / 1024)])
    out = tmp_path / "traffic.json"
    bench.traffic_from_pmc(str(fetch), str(write), out_path=str(out), copy_bytes=gib)
    t = json.loads(out.read_text())
    assert t["fetch_scale"] == pytest.approx(1.25) and t["write_scale"] == pytest.approx(0.5)
    assert t["bytes_per_launch"] == pytest.approx(1100.0 * 1024 / 1.25 + 20.0 * 1024 / 0.5)
    assert t["kernel"] == STATS and t["kernel_digest"] == bench.stats_kernel_digest()


def test_traffic_needs_the_copy_last(tmp_path):
    fetch = tmp_path / "fetch.csv"
    write = tmp_path / "write.csv"
    write_counters(fetch, "FETCH_SIZE", [(COPY, 1.0), (STATS, 2.0)])
    write_counters(write, "WRITE_SIZE", [(COPY, 1.0), (STATS, 2.0)])
    with pytest.raises(SystemExit):
        bench.traffic_from_pmc(str(fetch), str(write), out_path=str(tmp_path / "t.json"))


def test_traffic_is_reported_only_for_the_kernel_it_was_taken_on(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "traffic_file", lambda kernel, cid: str(tmp_path / f"{kernel}_{cid}.json"))
    f = tmp_path / "k_argmax_stats_4.json"
    f.write_text(json.dumps({"kernel_digest": bench.stats_kernel_digest(), "bytes_per_launch": 123.0}))
    assert bench.measured_traffic("k_argmax_stats", 4) == 123.0
    assert bench.measured_traffic("k_argmax_stats", 5) is None          # another workload: no file
    assert bench.measured_traffic("k_softmax_stats", 4) is None         # another kernel: no file
    f.write_text(json.dumps({"kernel_digest": "0" * 16, "bytes_per_launch": 123.0}))
    assert bench.measured_traffic("k_argmax_stats", 4) is None


def test_digest_follows_the_build_flags(monkeypatch):
    """The streaming kernels' build flags are part of the digest; other
    build.py changes are not."""
    d0 = bench.stats_kernel_digest()
    monkeypatch.setattr(bench, "_build_flags", lambda: b"other flags")
    assert bench.stats_kernel_digest() != d0


def test_digest_follows_the_kernel_source(monkeypatch):
    """Any change to a source the statistics kernel's counters depend on
    changes the digest."""
    d0 = bench.stats_kernel_digest()
    src = os.path.join(ROOT, "draft_verification_verify_amd", "csrc", "sv_stats.hip")
    real_open = open

    def fake_open(path, mode="r", *a, **k):
        fh = real_open(path, mode, *a, **k)
        if os.path.abspath(path) == src and "b" in mode:
            data = fh.read() + b"\n// changed\n"
            fh.close()
            return io.BytesIO(data)
        return fh
    monkeypatch.setattr("builtins.open", fake_open)
    assert bench.stats_kernel_digest() != d0


@pytest.mark.parametrize("k,bounds", [(16, [0, 1, 2, 4, 8, 17]), (8, [0, 1, 2, 4, 9]), (4, [0, 1, 2, 5]),
                                      (1, [0, 2]), (5, [0, 1, 2, 4, 6]), (63, [0, 1, 2, 4, 8, 16, 32, 64])])
def test_lazy_window_schedule(k, bounds):
    """The early-exit windows 0, 1, 2, 4, 8, ... clipped to k+1, where a last
    window holding only the bonus row joins the window before it."""
    assert bench.lazy_bounds(k) == bounds


def test_lazy_streamed_rows():
    """Rows an early-exit call streams, worked by hand for k = 4 (windows
    [0,1), [1,2), [2,5)): a sequence rejecting at 0 streams window 0's target
    and draft row and the draw re-reads the pair; one accepting everything
    streams 1+1, 1+1 and 3+2 rows and re-reads the bonus row."""
    assert bench.lazy_streamed_rows([0], 4, True) == (2, 2)
    assert bench.lazy_streamed_rows([1], 4, True) == (4, 2)
    assert bench.lazy_streamed_rows([2], 4, True) == (9, 2)
    assert bench.lazy_streamed_rows([3], 4, True) == (9, 2)
    assert bench.lazy_streamed_rows([4], 4, True) == (9, 1)
    assert bench.lazy_streamed_rows([0, 4, 1], 4, True) == (15, 5)
    assert bench.lazy_streamed_rows([0, 2, 4], 4, False) == (1 + 5 + 5, 0)


def test_one_pass_top_k_limit_matches_the_library():
    """bench.py names the truncation kernel from the library's dispatch rule:
    its top-k limit for the candidate-list pass must be the library's."""
    import re
    csrc = os.path.join(ROOT, "draft_verification_verify_amd", "csrc")
    src = open(os.path.join(csrc, "sv_trunc.hip")).read()
    hdr = open(os.path.join(csrc, "sv_launch.h")).read()
    m = re.search(r"constexpr int kTopkMax = (\d+);", hdr)
    assert m and int(m.group(1)) == bench.TOPK_ONE_PASS_MAX
    for name, val in (("kListRowsPerCU", bench.LIST_ROWS_PER_CU), ("kSplitTarget", bench.SPLIT_TARGET),
                      ("kSplitFewRows", bench.SPLIT_FEW_ROWS), ("kSplitMinVecFew", bench.SPLIT_MIN_VEC_FEW),
                      ("kSplitMinVecMany", bench.SPLIT_MIN_VEC_MANY), ("kSplitMax", bench.SPLIT_MAX),
                      ("kVec", 8)):
        m = re.search(r"constexpr int %s = (\d+);" % name, hdr)
        assert m and int(m.group(1)) == val, name
    m = re.search(r"constexpr int kLdsRowMax = (\d+);", src)
    assert m and int(m.group(1)) == bench.LDS_ROW_MAX


def test_truncation_kernel_names():
    """The launch bench.py times for truncated sampling, by element size,
    vocabulary and top-k, as the library dispatches it."""
    tk = lambda es, V, top_k, n: bench.truncation_kernel(es, V, top_k, n, 256)
    n = 512 * 33                                   # workload 5's rows
    assert tk(2, 128256, 50, n) == "k_topk16"
    assert tk(2, 128256, 256, n) == "k_topk16"
    assert tk(2, 128256, 257, n) == "k_trunc16"
    assert tk(2, 128256, 0, n) == "k_trunc16"
    assert tk(2, 100, 100, n) == "k_trunc16"       # top-k >= V is off
    assert tk(2, 7, 3, n) == "k_trunc_rows"       # no whole vector
    assert tk(2, 128256, 50, 768) == "k_trunc16"  # 3 rows per compute unit: the histogram pass
    assert tk(2, 128256, 50, 769) == "k_topk16"
    assert tk(4, 32000, 50, n) == "k_topk32"
    assert tk(4, 32000, 0, n) == "k_trunc_rows_lds"
    assert tk(4, 32768, 300, n) == "k_trunc_rows_lds"
    assert tk(4, 32769, 0, n) == "k_trunc_rows"
    assert tk(4, 7, 3, n) == "k_trunc_rows_lds"
    # few fp32 rows: slices of at least 16 KB (at most 64 rows) or 64 KB,
    # about 1024 workgroups in all
    assert tk(4, 32000, 50, 9) == "k_topk32_sliced"       # 7 slices of 512+ vectors
    assert tk(4, 32000, 50, 72) == "k_topk32"             # 4000 vectors: one 64 KB slice
    assert tk(4, 128256, 50, 288) == "k_topk32_sliced"    # 3 slices
    assert tk(4, 128256, 50, 513) == "k_topk32"           # 1024 // 513 = 1
    assert tk(4, 8191, 50, 9) == "k_topk32"               # 1023 vectors: one slice
    assert tk(4, 128256, 0, 9) == "k_trunc_rows"          # no top-k: the radix passes
    assert bench.split_slices(9, 32000) == 7
    assert bench.split_slices(9, 128256) == 31
    assert bench.split_slices(1, 1 << 24) == 32
    assert bench.split_slices(144, 128256) == 7
    assert bench.split_slices(512, 1 << 24) == 2
