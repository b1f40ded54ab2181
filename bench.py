#!/usr/bin/env python3
"""Throughput of the verification step on one MI355X.

A step is one spec_verify_sample call over workload 5: B = 512 sequences,
k = 16 drafts, V = 128256, bf16 logits, T = 1.0 (the largest workload; all
inputs already resident in HBM).  --workload / --mode measure the other
workloads and entry points; workloads smaller than 1 GiB rotate over several
input sets, call by call, so that no call reads its rows from the MALL.  One
call runs the whole hot path: the vocabulary-streaming statistics pass over
every target and draft row, the per-sequence decisions, and the residual or
bonus draw.  The metric counts verified positions: B * (k+1) rows per call.

Prints one JSON line.  Also reports, for the dominant kernel (the statistics
pass), its average duration from HIP events recorded on the launch stream
during the timed region and its achieved HBM bandwidth against the 8 TB/s
peak, and the CPU oracle timed on a bounded sample of the same workload.
After the timed region it replays the same calls captured in one HIP graph
(config.graph_replay_ms_per_call: the per-call time without host and launch
overhead, which bounds the small, launch-bound workloads).
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
METRIC = "verified positions/sec (B·(k+1) rows/s) and achieved HBM GB/s vs peak"
STATS_SOURCES = ["sv_stats.hip", "sv_device.h", "sv_launch.h"]
STREAM_KERNELS = ("k_softmax_stats", "k_argmax_stats")
# Rows under a top-k of at most this take a candidate-list pass: k_topk32 for
# fp32 rows, k_topk16 for 16-bit rows that outnumber the compute units more
# than LIST_ROWS_PER_CU times.  Other 16-bit rows take the 65536-bin
# histogram pass (k_trunc16), other fp32 rows the radix passes
TOPK_ONE_PASS_MAX = 256
LIST_ROWS_PER_CU = 3
LDS_ROW_MAX = 32768                    # fp32 rows up to this run the radix passes from LDS
# Few fp32 rows under such a top-k are cut into slices: about SPLIT_TARGET
# workgroups in all, at most SPLIT_MAX per row, each of at least
# SPLIT_MIN_VEC_FEW 8-logit vectors for at most SPLIT_FEW_ROWS rows, else
# SPLIT_MIN_VEC_MANY; each slice's candidates go to k_trunc_merge
SPLIT_TARGET, SPLIT_FEW_ROWS, SPLIT_MIN_VEC_FEW, SPLIT_MIN_VEC_MANY, SPLIT_MAX = 1024, 64, 512, 2048, 32
TRUNC_NOTES = {
    "k_topk16": "k_topk16 (one pass per 16-bit row: per-wave lists of the candidates above a "
                "rising floor) followed by k_trunc_rows over the rows it marked",
    "k_topk32": "k_topk32 (one pass per fp32 row: per-wave lists of the candidates above a "
                "rising floor) followed by k_trunc_rows over the rows it marked",
    "k_topk32_sliced": "k_topk32 on row slices (each slice's candidates above its own rising "
                       "floor) followed by k_trunc_merge (one workgroup per row merges them; "
                       "the radix passes for rows the slices could not summarise)",
    "k_trunc16": "k_trunc16 (one pass per 16-bit row: an exact LDS histogram of all 65536 bit "
                 "patterns) followed by k_trunc_rows over the rows it marked",
    "k_trunc_rows_lds": "k_trunc_rows_lds (on an LDS copy of each fp32 row, read from HBM once: "
                        "value bins, then radix levels among the boundary bin's keys)",
    "k_trunc_rows": "k_trunc_rows (one workgroup per row, each pass streaming the row, the first "
                    "from HBM and later ones mostly from cache: value bins, then radix levels "
                    "among the boundary bin's keys for fp32 rows, radix selection otherwise)",
}


def split_slices(n_rows: int, V: int) -> int:
    """Slices per fp32 row for the candidate-list pass (1: rows whole)."""
    min_vec = SPLIT_MIN_VEC_FEW if n_rows <= SPLIT_FEW_ROWS else SPLIT_MIN_VEC_MANY
    s = min(SPLIT_TARGET // max(n_rows, 1), (V // 8) // min_vec, SPLIT_MAX)
    return s if s >= 2 else 1


def truncation_kernel(es: int, V: int, top_k: int, n_rows: int, cus: int) -> str:
    """The launch that summarises every row for truncated sampling, for
    n_rows rows of V logits of es bytes on a GPU of `cus` compute units."""
    small_topk = 1 <= top_k <= TOPK_ONE_PASS_MAX and top_k < V
    if es == 2:
        if V < 8:
            return "k_trunc_rows"
        return "k_topk16" if small_topk and n_rows > LIST_ROWS_PER_CU * cus else "k_trunc16"
    if small_topk and V >= 8 and split_slices(n_rows, V) > 1:
        return "k_topk32_sliced"
    if small_topk and V >= 8:
        return "k_topk32"
    return "k_trunc_rows_lds" if V <= LDS_ROW_MAX else "k_trunc_rows"


def traffic_file(kernel: str, cid: int) -> str:
    """Where the committed counter figures of a streaming kernel on a workload live."""
    return os.path.join(ROOT, "profiles", f"{kernel}_workload{cid}_traffic.json")


def _plan_source() -> bytes:
    """The launch plan of the statistics kernel (plan_stats in sv_api.hip),
    from its signature to its closing brace."""
    with open(os.path.join(ROOT, "draft_verification_verify_amd", "csrc", "sv_api.hip"), "rb") as fh:
        src = fh.read()
    a = src.index(b"StatsPlan plan_stats(")
    return src[a:src.index(b"\n}\n", a) + 3]


def _build_flags() -> bytes:
    """The compiler flags the streaming kernels are built with (build.py's
    common flags and those of sv_stats.hip)."""
    import importlib.util
    spec = importlib.util.spec_from_file_location(
        "_sv_build_flags", os.path.join(ROOT, "draft_verification_verify_amd", "build.py"))
    b = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(b)
    common = [f for f in b.COMMON if not f.startswith("-I")]
    return repr((b.HIPCC.split("/")[-1], common, b.SOURCES["sv_stats.hip"])).encode()


def stats_kernel_digest() -> str:
    """What the streaming kernels' counters depend on: their source, the
    headers it includes, their launch plan and the build flags."""
    h = hashlib.sha256()
    for f in STATS_SOURCES:
        with open(os.path.join(ROOT, "draft_verification_verify_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    h.update(_plan_source())
    h.update(_build_flags())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str, cid: int):
    """HBM bytes per launch of a streaming kernel on a workload from the
    committed rocprofv3 counter runs, if they were taken on the current
    kernel source."""
    path = traffic_file(kernel, cid)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_digest") != stats_kernel_digest():
        return None
    return t.get("bytes_per_launch")


CHAIN_MODES = ("sample", "greedy", "greedy_ext", "lenient", "sample_lazy", "greedy_lazy", "truncated")
CAND_MODES = ("candidates", "candidates_ext", "tree")
MALL_DEFEAT_BYTES = 1 << 30            # inputs rotated over at least this many bytes (MALL: 256 MB)
CPU_SHARE = 16                         # host CPUs per GPU when one host serves several GPUs
CEILING_VECS = (1024, 2048, 4096, 8192)  # workgroup sizes (16-byte vectors) of the plain streaming read


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--mode", default="sample", choices=list(CHAIN_MODES + CAND_MODES),
                    help="sample (default, the benchmark line), greedy / greedy_ext (with the "
                         "#Match by-products), lenient (--lenience), sample_lazy / greedy_lazy "
                         "(early exit), truncated (--top-k, --top-p): chain workloads; "
                         "candidates / candidates_ext / tree (shared rows stored once): workload 4")
    ap.add_argument("--workload", type=int, default=None, choices=[1, 2, 3, 4, 5],
                    help="default: 5 for chain modes, 4 for candidate modes")
    ap.add_argument("--sets", type=int, default=0,
                    help="input sets rotated over, call by call (0: enough to span 1 GiB, so "
                         "that no call finds its rows in the 256 MB MALL)")
    ap.add_argument("--vocab-shard", type=int, default=1, metavar="G",
                    help="one GPU's share of a vocabulary-parallel LM head over G GPUs: every "
                         "row holds ceil(V/G) logits (the exchange of row partials between "
                         "the GPUs is not part of the measurement)")
    ap.add_argument("--lenience", type=float, default=2.0)
    ap.add_argument("--top-k", type=int, default=50)
    ap.add_argument("--top-p", type=float, default=0.8)
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="CPU oracle baseline budget (sample mode; 0 disables it)")
    ap.add_argument("--graph-calls", type=int, default=100,
                    help="calls captured in one HIP graph and replayed after the timed region "
                         "(0: skip); reported as config.graph_replay_ms_per_call")
    ap.add_argument("--profile-every", type=int, default=5,
                    help="time the streaming kernel on every N-th timed call (a pair of events "
                         "the library records around it)")
    ap.add_argument("--drafts", default="auto", choices=["auto", "sampled", "argmax"],
                    help="draft tokens of chain workloads: sampled from the draft rows, or the "
                         "draft's argmax (greedy drafting); auto: argmax for greedy modes on "
                         "workload 3, sampled otherwise")
    ap.add_argument("--ceiling-vec", type=int, default=-1,
                    help="16-byte vectors per workgroup of the plain streaming read that gives "
                         "the device's achievable read rate (roofline.ceiling): -1 takes the best "
                         "of 1024, 2048, 4096 and 8192, 0 skips it")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a 1 GiB device copy (scale for the rocprofv3 byte counters)")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write a streaming kernel's measured HBM traffic on --workload from two "
                         "rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) and exit")
    ap.add_argument("--traffic-kernel", default="k_softmax_stats", choices=list(STREAM_KERNELS))
    args = ap.parse_args()
    if args.traffic_from:
        traffic_from_pmc(*args.traffic_from, kernel=args.traffic_kernel,
                         out_path=traffic_file(args.traffic_kernel, args.workload or 5))
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (sequences "
              "shard over GPUs with no exchange, so one GPU's rate is its share); run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)
    if args.vocab_shard < 1:
        print("--vocab-shard must be at least 1", file=sys.stderr)
        sys.exit(2)
    cand = args.mode in CAND_MODES
    cid = args.workload or (4 if cand else 5)
    if cand != (cid == 4):
        print(f"mode {args.mode} does not run on workload {cid}", file=sys.stderr)
        sys.exit(2)

    import torch

    import draft_verification_verify_amd as sv
    import synthetic

    dev = "cuda:0"
    torch.cuda.set_device(0)
    cfg0 = synthetic.WORKLOADS[cid]
    v_full = cfg0.V
    if args.vocab_shard > 1:
        cfg0 = dataclasses.replace(cfg0, V=-(-v_full // args.vocab_shard))
    es = {"fp32": 4, "fp16": 2, "bf16": 2}[cfg0.dtype]
    if cand:
        stream_rows = cfg0.C * cfg0.R
    else:
        stream_rows = 2 * cfg0.k + 1 if args.mode in ("sample", "lenient", "sample_lazy", "truncated") \
            else cfg0.k + 1
    set_bytes = cfg0.B * stream_rows * cfg0.V * es
    sets = args.sets or max(1, min(1000, -(-MALL_DEFEAT_BYTES // set_bytes)))
    if sets > 1 and set_bytes * sets > (6 << 30):
        sets = max(1, (6 << 30) // set_bytes)
    t0 = time.perf_counter()
    wall = synthetic.generate(cid, device=dev, B=cfg0.B * sets, V=cfg0.V)
    torch.cuda.synchronize()
    gen_s = time.perf_counter() - t0
    B = cfg0.B

    def part(t, s):
        return None if t is None else t[s * B:(s + 1) * B]

    greedy_mode = args.mode in ("greedy", "greedy_ext", "greedy_lazy")
    drafts = args.drafts
    if drafts == "auto":
        drafts = "argmax" if (greedy_mode and cid == 3) else "sampled"
    if drafts == "argmax" and not cand:
        wall.tokens = synthetic.greedy_drafts(wall.draft)
    slices = [synthetic.Workload(cfg0, part(wall.target, s), part(wall.draft, s), part(wall.tokens, s),
                                 part(wall.uniforms, s), wall.T) for s in range(sets)]
    w = slices[0]

    if args.mode == "tree":
        trees = [synthetic.as_tree(x) for x in slices]
        _, C, R, V = w.target.shape
        L = w.tokens.shape[2]
        N = trees[0][0].shape[1]
        rows = B * C * R
        ws = torch.empty(sv.workspace_bytes(B, N, V, trees[0][0].dtype), dtype=torch.uint8, device=dev)

        def call(i, ev=None):
            nodes, cand_rows = trees[i % sets]
            sv.greedy_tree(nodes, slices[i % sets].tokens, cand_rows, workspace=ws, events=ev)
        stats_rows = B * N
        workload = f"workload {cid}: spec_verify_greedy_tree B={B} C={C} L={L} R={R} N={N} V={V} {cfg0.dtype}"
    elif cand:
        _, C, R, V = w.target.shape
        L = w.tokens.shape[2]
        rows = B * C * R
        out = (torch.empty((B, L + 1), dtype=torch.int32, device=dev),
               torch.empty(B, dtype=torch.int32, device=dev), torch.empty(B, dtype=torch.int32, device=dev))
        ws = torch.empty(sv.workspace_bytes(B, C * R, V, w.target.dtype), dtype=torch.uint8, device=dev)

        if args.mode == "candidates":
            def call(i, ev=None):
                x = slices[i % sets]
                sv.greedy_candidates(x.target, x.tokens, out_tokens=out[0], out_num_accepted=out[1],
                                     out_best=out[2], workspace=ws, events=ev)
        else:
            def call(i, ev=None):
                x = slices[i % sets]
                sv.greedy_candidates_ext(x.target, x.tokens, workspace=ws, events=ev)
        stats_rows = rows
        workload = f"workload {cid}: spec_verify_greedy_{args.mode} B={B} C={C} L={L} R={R} V={V} {cfg0.dtype}"
    else:
        _, k1, V = w.target.shape
        k = k1 - 1
        rows = B * k1
        out_t = torch.empty((B, k1), dtype=torch.int32, device=dev)
        out_n = torch.empty(B, dtype=torch.int32, device=dev)
        sampling = stream_rows == 2 * k + 1
        ws = torch.empty(sv.workspace_bytes(B, 2 * k + 1 if sampling else k + 1, V, w.target.dtype),
                         dtype=torch.uint8, device=dev)
        name = {"sample": "spec_verify_sample", "lenient": "spec_verify_sample_lenient",
                "sample_lazy": "spec_verify_sample_lazy", "truncated": "spec_verify_sample_truncated",
                "greedy": "spec_verify_greedy", "greedy_ext": "spec_verify_greedy_ext",
                "greedy_lazy": "spec_verify_greedy_lazy"}[args.mode]
        extra = {"lenient": f" l={args.lenience}",
                 "truncated": f" top_k={args.top_k} top_p={args.top_p}"}.get(args.mode, "")
        workload = (f"workload {cid}: {name} B={B} k={k} V={V} {cfg0.dtype}"
                    f"{' T=' + str(w.T) if sampling else ''}{extra}")
        stats_rows = B * stream_rows

        def call(i, ev=None):
            # the early-exit modes have no single streaming kernel to time: `ev` is unused there
            x = slices[i % sets]
            if args.mode == "sample":
                sv.sample(x.target, x.draft, x.tokens, x.uniforms, x.T, out_tokens=out_t,
                          out_num_accepted=out_n, workspace=ws, events=ev)
            elif args.mode == "lenient":
                sv.sample_lenient(x.target, x.draft, x.tokens, x.uniforms, x.T, args.lenience,
                                  workspace=ws, events=ev)
            elif args.mode == "sample_lazy":
                sv.sample_lazy(x.target, x.draft, x.tokens, x.uniforms, x.T, out_tokens=out_t,
                               out_num_accepted=out_n, workspace=ws)
            elif args.mode == "truncated":
                sv.sample_truncated(x.target, x.draft, x.tokens, x.uniforms, x.T, args.top_k,
                                    args.top_p, workspace=ws, events=ev)
            elif args.mode == "greedy_lazy":
                sv.greedy_lazy(x.target, x.tokens, out_tokens=out_t, out_num_accepted=out_n,
                               workspace=ws)
            elif args.mode == "greedy_ext":
                sv.greedy_ext(x.target, x.tokens, workspace=ws, events=ev)
            else:
                sv.greedy(x.target, x.tokens, out_tokens=out_t, out_num_accepted=out_n, workspace=ws,
                          events=ev)

    if args.vocab_shard > 1:
        workload += f" (one of {args.vocab_shard} vocabulary shards of V={v_full})"

    # algorithmic bytes of the streaming kernel: every logit row read once
    # (V * element size) plus its 8-byte partial written
    bytes_per_row = V * es + 8
    stats_bytes = stats_rows * bytes_per_row

    for i in range(args.warmup):
        call(i)
    torch.cuda.synchronize()

    # the streaming kernel is timed by a pair of events the library records
    # around it, on every `profile_every`-th call of the timed region (each
    # pair adds a few microseconds of queue time to the call it brackets)
    lazy = args.mode.endswith("_lazy")
    timed_ids = [] if lazy else list(range(0, args.steps, max(1, args.profile_every)))
    kev = {i: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for i in timed_ids}
    for e0, e1 in kev.values():                    # creates the events' handles before the timed region
        e0.record()
        e1.record()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    start.record()
    for i in range(args.steps):
        call(args.warmup + i, kev.get(i))
    end.record()
    torch.cuda.synchronize()
    wall_s = time.perf_counter() - w0
    kernel_ms = [e0.elapsed_time(e1) for e0, e1 in kev.values()]
    total_ms = start.elapsed_time(end)
    ms_per_step = total_ms / args.steps
    value = rows * args.steps / (total_ms / 1e3)

    # after the timed region: each call on its own between two events, for
    # the spread of single-call times
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    for i, (e0, e1) in enumerate(evs):
        e0.record()
        call(i)
        e1.record()
    torch.cuda.synchronize()
    per_call = sorted(e0.elapsed_time(e1) for e0, e1 in evs)

    def pct(q):
        return per_call[min(len(per_call) - 1, int(q * (len(per_call) - 1) + 0.5))]

    # the same calls captured in one HIP graph and replayed: the per-call time
    # without host and launch overhead (a call enqueues no allocation, memset
    # or synchronisation, so it can be captured); each captured call reads the
    # input set it would read in the timed region
    graph_ms, graph_n = None, 0
    if args.graph_calls > 0:
        graph_n = args.graph_calls
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(graph_n):
                call(i)
        g.replay()
        torch.cuda.synchronize()
        g0 = torch.cuda.Event(enable_timing=True)
        g1 = torch.cuda.Event(enable_timing=True)
        reps = 3
        g0.record()
        for _ in range(reps):
            g.replay()
        g1.record()
        torch.cuda.synchronize()
        graph_ms = g0.elapsed_time(g1) / (reps * graph_n)
        del g

    k_avg_ms = statistics.fmean(kernel_ms) if kernel_ms else None
    achieved = stats_bytes / (k_avg_ms / 1e3) / 1e9 if kernel_ms else None

    # early exit: the bytes a call actually streams follow from each
    # sequence's accepted count (the windows it stayed undecided through, and
    # the draw's re-read), worked out per input set
    lazy_bytes = None
    if lazy:
        per_set = []
        for si in range(sets):
            call(si)
            torch.cuda.synchronize()
            r_stats, r_draw = lazy_streamed_rows(out_n.cpu().tolist(), k, args.mode == "sample_lazy")
            per_set.append(r_stats * bytes_per_row + r_draw * V * es)
        lazy_bytes = statistics.fmean(per_set[(args.warmup + i) % sets] for i in range(args.steps))
        achieved = lazy_bytes / (ms_per_step / 1e3) / 1e9

    # the device's achievable read rate: a plain 16-byte streaming read of the
    # same buffers (the same input sets, rotated the same way), one launch
    # over each call's logits
    ceiling = None
    if args.ceiling_vec != 0:
        if args.mode == "tree":
            bufs = [(nodes, None) for nodes, _ in trees]
        elif cand or stream_rows != 2 * cfg0.k + 1:
            bufs = [(x.target, None) for x in slices]
        else:
            bufs = [(x.target, x.draft) for x in slices]
        vecs = CEILING_VECS if args.ceiling_vec < 0 else (args.ceiling_vec,)
        ceiling = stream_ceiling(bufs, max(args.steps, 20), vecs)
    kernel_name = {"sample": "k_softmax_stats", "lenient": "k_softmax_stats",
                   "truncated": truncation_kernel(es, V, args.top_k, cfg0.B * stream_rows,
                                                 torch.cuda.get_device_properties(0).multi_processor_count)}.get(args.mode, "k_argmax_stats")
    traffic = measured_traffic(kernel_name, cid) \
        if (kernel_name in STREAM_KERNELS and args.vocab_shard == 1 and args.mode != "tree"
            and not lazy) else None

    line = {
        "metric": METRIC,
        "value": value,
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": workload,
            "input_dtype": cfg0.dtype,
            "rows_per_call": rows,
            "logit_bytes_per_call": stats_rows * V * es,
            "call_effective_GBps": stats_rows * V * es / (ms_per_step / 1e3) / 1e9,
            "input_sets_rotated": sets,
            "draft_tokens": "argmax of the draft rows (greedy drafting)" if (drafts == "argmax" and not cand)
            else None if cand else "sampled from softmax(draft / T)",
            "single_call_ms_p10_p50_p90": [pct(0.1), pct(0.5), pct(0.9)],
            "graph_replay_ms_per_call": graph_ms,
            "graph_calls": graph_n,
            "wall_s_timed_region": wall_s,
            "input_generation_s": gen_s,
            "device": torch.cuda.get_device_name(0),
        },
        "roofline": {
            "kernel": "the whole call (windows of k_lazy_stats, their decisions, the draw)",
            "note": ("early exit has no single streaming kernel: achieved = the bytes the call "
                     "streams (every row of each window a sequence is still undecided at, plus "
                     "the draw's re-read; from the calls' accepted counts) / ms_per_step"),
            "bound": "hbm",
            "achieved": achieved,
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": achieved / PEAK_HBM_GBS,
            "ceiling": ceiling["GBps"] if ceiling else None,
            "frac_of_ceiling": achieved / ceiling["GBps"] if ceiling else None,
            "ceiling_run": ceiling,
            "traffic": None,
            "streamed_bytes_per_call": lazy_bytes,
            "full_pass_bytes_per_call": stats_bytes,
        } if lazy else {
            "kernel": kernel_name,
            "note": ("the timed launch is " + TRUNC_NOTES[kernel_name]
                     + "; algorithmic bytes: every row read once")
            if args.mode == "truncated" else (
                "rows counts every scored candidate position (B*C*R); the kernel reads "
                "B*N unique node rows") if args.mode == "tree" else None,
            "bound": "hbm",
            "achieved": achieved,
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": achieved / PEAK_HBM_GBS if achieved else None,
            "ceiling": ceiling["GBps"] if ceiling else None,
            "frac_of_ceiling": achieved / ceiling["GBps"] if (ceiling and achieved) else None,
            "ceiling_run": ceiling,
            "traffic": traffic,
            "kernel_ms_avg": k_avg_ms,
            "kernel_ms_min": min(kernel_ms) if kernel_ms else None,
            "kernel_ms_max": max(kernel_ms) if kernel_ms else None,
            "kernel_launches_timed": len(kernel_ms),
            "algorithmic_bytes_per_launch": stats_bytes,
        },
    }

    if args.cpu_seconds > 0 and args.mode == "sample":
        call(0)                        # slice 0 again, for the parity comparison
        torch.cuda.synchronize()
        line["cpu_baseline"] = cpu_baseline(w, out_t, out_n, args.cpu_seconds)
    if args.calibrate_copy:
        calibrate_copy()
    print(json.dumps(line), flush=True)


def lazy_bounds(k):
    """Window bounds of the early-exit entry points: 0, 1, 2, 4, 8, ...
    clipped to k+1, a last window that would hold only the bonus row joining
    the window before it (the schedule the library launches)."""
    b = [0]
    nxt = 1
    while b[-1] < k + 1:
        b.append(min(nxt, k + 1))
        nxt = nxt + 1 if nxt < 2 else nxt * 2
    if len(b) >= 3 and b[-2] == k:
        b[-2] = k + 1
        b.pop()
    return b


def lazy_streamed_rows(num_accepted, k, sampling):
    """(rows streamed by the statistics windows, rows re-read by the draw) of
    one early-exit call: a sequence with j accepted drafts is undecided at
    every window that starts at or before position j and is streamed there
    (the window's target rows, and when sampling its draft rows below k);
    the draw re-reads the rejected row pair, or the bonus row."""
    b = lazy_bounds(k)
    stats = draw = 0
    for j in num_accepted:
        for w0, w1 in zip(b[:-1], b[1:]):
            if j < w0:
                break
            stats += w1 - w0
            if sampling:
                stats += max(0, min(w1, k) - w0)
        if sampling:
            draw += 2 if j < k else 1
    return stats, draw


def stream_ceiling(bufs, calls, vecs):
    """GB/s of a plain 16-byte non-temporal streaming read (libsvceiling.so)
    over `bufs` [(a, b or None), ...] device tensors, one launch per entry,
    rotated like the calls: for each workgroup size in `vecs` (16-byte
    vectors per workgroup), `calls` launches between two events after a few
    untimed ones; the best size gives the ceiling."""
    import ctypes

    import torch
    path = os.path.join(ROOT, "draft_verification_verify_amd", "libsvceiling.so")
    if not os.path.exists(path):
        raise SystemExit(f"{path} is not built (run __graft_entry__.build())")
    L = ctypes.CDLL(path)
    P, LL, I = ctypes.c_void_p, ctypes.c_longlong, ctypes.c_int
    L.sv_stream_read_blocks.argtypes = [LL, LL, I]
    L.sv_stream_read_blocks.restype = LL
    L.sv_stream_read.argtypes = [P, LL, P, LL, I, P, LL, P]
    L.sv_stream_read.restype = I

    def nbytes(t):
        return 0 if t is None else t.numel() * t.element_size()

    blocks = max(L.sv_stream_read_blocks(nbytes(a), nbytes(b), v) for a, b in bufs for v in vecs)
    sink = torch.zeros(blocks, dtype=torch.int32, device="cuda:0")
    st = torch.cuda.current_stream().cuda_stream
    per = statistics.fmean(nbytes(a) + nbytes(b) for a, b in bufs)

    def launch(i, vec):
        a, b = bufs[i % len(bufs)]
        rc = L.sv_stream_read(a.data_ptr(), nbytes(a), None if b is None else b.data_ptr(), nbytes(b),
                              vec, sink.data_ptr(), blocks, st)
        if rc != 0:
            raise RuntimeError(f"sv_stream_read failed: {rc}")

    runs = {}
    for vec in vecs:
        for i in range(5):
            launch(i, vec)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for i in range(calls):
            launch(5 + i, vec)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / calls
        runs[vec] = {"GBps": per / (ms / 1e3) / 1e9, "ms_per_launch": ms}
    best = max(runs, key=lambda v: runs[v]["GBps"])
    return {"GBps": runs[best]["GBps"], "ms_per_launch": runs[best]["ms_per_launch"], "bytes_per_launch": per,
            "launches": calls, "vec_per_block": best, "kernel": "k_stream_read",
            "GBps_by_vec_per_block": {str(v): runs[v]["GBps"] for v in vecs}}


def cpu_baseline(w, out_t, out_n, budget_s):
    """The CPU oracle, as written (double precision, one sequence after
    another), timed on a bounded sample of the same workload: the first
    sequences of the batch, copied to host memory outside the timed part, run
    repeatedly until the budget is spent.  First on one thread (a quarter of
    the budget), then on every host core the process may use (the oracle is
    a C library; ctypes releases the interpreter lock around each call, so
    the threads run in parallel).  The oracle's results on the sample are also
    compared with the GPU's call on the same sequences."""
    import threading

    import numpy as np

    import oracle
    from oracle import parity
    if not os.path.exists(oracle.LIB_PATH):
        oracle.build()
    B, k1, V = w.target.shape
    nseq = min(B, 64)
    z = w.target[:nseq].float().cpu().numpy()
    y = w.draft[:nseq].float().cpu().numpy()
    x = w.tokens[:nseq].cpu().numpy()
    u = w.uniforms[:nseq].cpu().numpy()
    rep = parity.check_sample(z, y, x, u, w.T, out_t[:nseq].cpu().numpy(), out_n[:nseq].cpu().numpy(),
                              seq_ids=np.arange(nseq))
    chunk = 4
    starts = list(range(0, nseq, chunk))

    def run(threads, seconds):
        lock = threading.Lock()
        state = {"next": 0, "seqs": 0}
        stop = time.perf_counter() + seconds

        def worker():
            while time.perf_counter() < stop:
                with lock:
                    i = state["next"]
                    state["next"] += 1
                b0 = starts[i % len(starts)]
                b1 = min(nseq, b0 + chunk)
                oracle.sample(z[b0:b1], y[b0:b1], x[b0:b1], u[b0:b1], w.T)
                with lock:
                    state["seqs"] += b1 - b0
        t0 = time.perf_counter()
        ts = [threading.Thread(target=worker) for _ in range(threads)]
        for t in ts:
            t.start()
        for t in ts:
            t.join()
        return state["seqs"], time.perf_counter() - t0

    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:
        affinity = os.cpu_count() or 1
    # a job that drives one GPU of a shared host gets a share of 16 of the
    # host's CPUs (worker pools are sized to that share, whatever the host
    # has in all)
    cores = max(1, min(CPU_SHARE, affinity))
    s1, t1 = run(1, budget_s / 4)
    sn, tn = run(cores, budget_s * 3 / 4)
    return {
        "value": sn * k1 / tn,
        "unit": "rows/s",
        "cores": cores,
        "kind": "oracle",
        "value_1_core": s1 * k1 / t1,
        "host_nproc": os.cpu_count(),
        "host_affinity_cpus": affinity,
        "cpu_share": CPU_SHARE,
        "cpu_model": _cpu_model(),
        "sample": (f"the first {nseq} sequences of the same workload ({nseq * k1} rows), run "
                   f"repeatedly in chunks of {chunk}: {s1} sequences on 1 thread in {t1:.1f} s, "
                   f"then {sn} sequences on {cores} threads in {tn:.1f} s; C oracle in double "
                   f"precision, unchanged; it stops at each sequence's first rejection, so it "
                   f"reads fewer rows than it counts"),
        "parity_vs_gpu": rep.summary(),
    }


def _cpu_model() -> str:
    """The host CPU's model name, as lscpu reports it, else /proc/cpuinfo (or
    "unknown")."""
    import subprocess
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in out.splitlines():
            if line.strip().startswith("Model name:"):
                return line.split(":", 1)[1].strip()
    except (OSError, subprocess.SubprocessError):
        pass
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def calibrate_copy(nbytes=1 << 30):
    """A plain device-to-device copy of known size, for scaling the rocprofv3
    FETCH_SIZE / WRITE_SIZE counters (run under --pmc)."""
    import torch
    a = torch.empty(nbytes, dtype=torch.uint8, device="cuda:0")
    b = torch.empty_like(a)
    a.fill_(1)
    torch.cuda.synchronize()
    b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"calibration_copy_bytes": nbytes}), flush=True)


def traffic_from_pmc(fetch_csv, write_csv, kernel="k_softmax_stats", out_path=None, copy_bytes=1 << 30):
    """Turn two rocprofv3 --pmc counter_collection.csv files (FETCH_SIZE, then
    WRITE_SIZE, in KiB per dispatch) into HBM bytes per launch of a
    streaming kernel, each counter scaled by what it reads for the
    calibration copy of `copy_bytes`."""
    out_path = out_path or traffic_file(kernel, 5)
    import csv

    def dispatches(path, counter):
        rows = [r for r in csv.DictReader(open(path)) if r.get("Counter_Name") == counter]
        return sorted(rows, key=lambda r: int(r["Dispatch_Id"]))

    def stats_mean(rows):
        v = [float(r["Counter_Value"]) for r in rows if kernel in r["Kernel_Name"]]
        if not v:
            raise SystemExit(f"no {kernel} dispatch in the counter file")
        return statistics.fmean(v), next(r["Kernel_Name"] for r in rows if kernel in r["Kernel_Name"])

    def last_copy(rows):
        # the calibration copy is the process's last dispatch
        r = rows[-1]
        if "copy" not in r["Kernel_Name"].lower():
            raise SystemExit(f"last dispatch is not the calibration copy: {r['Kernel_Name']}")
        return float(r["Counter_Value"]), r["Kernel_Name"]

    f = dispatches(fetch_csv, "FETCH_SIZE")
    wr = dispatches(write_csv, "WRITE_SIZE")
    fk, fname = stats_mean(f)
    wk, _ = stats_mean(wr)
    fc, cname = last_copy(f)
    wc, _ = last_copy(wr)
    f_scale = fc * 1024 / copy_bytes
    w_scale = wc * 1024 / copy_bytes
    out = {
        "kernel": fname,
        "kernel_digest": stats_kernel_digest(),
        "fetch_kib_per_dispatch": fk,
        "write_kib_per_dispatch": wk,
        "copy_kernel": cname,
        "copy_bytes": copy_bytes,
        "copy_fetch_kib": fc,
        "copy_write_kib": wc,
        "fetch_scale": f_scale,
        "write_scale": w_scale,
        "bytes_per_launch": fk * 1024 / f_scale + wk * 1024 / w_scale,
    }
    with open(out_path, "w") as fh:
        json.dump(out, fh, indent=1)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
