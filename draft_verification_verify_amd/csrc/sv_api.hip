// sv_api.hip -- the C ABI of libspecverify.so: argument validation, workspace
// layout and kernel launches on the caller's stream.  Declared and documented
// in include/spec_verify.h.

#include <math.h>
#include <stdint.h>
#include <stdlib.h>

#include <atomic>
#include <mutex>

#include "spec_verify.h"
#include "sv_launch.h"

using namespace sv;

// The scratch of spec_verify_sample_noalloc: one copy per device, held until
// the process ends.  Host code never passes this name to a kernel (on the host
// it is a stand-in, not a device address): it uses the address that
// hipGetSymbolAddress gives for the current device (scratch_address below).
static __device__ __align__(256) unsigned char scratch[SV_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxV = 1 << 28;
constexpr int kMaxTruncV = 1 << 23;    // truncated rows: fixed-point masses of 2^-40 fit 63 bits
constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool dtype_ok(int dt) { return dt == SV_F32 || dt == SV_F16 || dt == SV_BF16; }

// How a set of rows is split along the vocabulary for the streaming pass
// (512-thread workgroups): slices of about 4096 logical vectors (8 per
// thread, 64 KiB of bf16), more slices when there are too few rows for 512
// workgroups, and never slices under 512 vectors (one per thread).  Measured
// on the 512 x 33 x 128256 bf16 shape: 4 slices of 512 threads per row beat
// 1-8 slices of 256 and 1024-thread workgroups; on 704 rows of 32000 (45 MB)
// one slice per row (12.0 us) beat 3 (14.0 us) and more.
struct StatsPlan {
    int nvec;
    int splits;
    int vec_per_split;
};

StatsPlan plan_stats(long long rows, int V)
{
    StatsPlan p;
    p.nvec = (V + kVec - 1) / kVec;
    long long s = (p.nvec + 2048) / 4096;
    const long long fill = (512 + rows - 1) / rows;
    if (s < fill) s = fill;
    long long smax = p.nvec / 512;
    if (smax < 1) smax = 1;
    if (s > smax) s = smax;
    if (s > 64) s = 64;
    if (s < 1) s = 1;
    p.splits = (int)s;
    p.vec_per_split = (p.nvec + p.splits - 1) / p.splits;
    // drop splits that would be empty
    p.splits = (p.nvec + p.vec_per_split - 1) / p.vec_per_split;
    return p;
}

// The sampled row (pair) is cut into chunks of whole rounds (kBlock logical
// vectors each), at most kMaxChunks of them, one chunk per workgroup of the
// chunk pass; chunks are lengthened until the pass has at most
// kSampleBlocks workgroups (a sweep on 512 row pairs of 128256 bf16 logits:
// 63 one-round chunks per row, 32256 workgroups, 49.5 us; 32 two-round
// chunks, 16384 workgroups, 42.6 us; four rounds per workgroup as four
// one-round chunks, 51.9 us).  Fewer rounds per chunk keep the draw's
// rescan of one chunk short.
constexpr long long kSampleBlocks = 16384;

// Chunk passes of at most this many workgroups also decide the round (the
// fused pass); measured: workload 1 (16 workgroups) 18.0 -> 15.9 us and
// workload 2 (1024) 25.3 -> 22.6 us per call, while at 2048 workgroups (B =
// 128, k = 5, V = 32000 fp16) the fused pass lost 0.7 us (graph replays),
// at 4096 2-3 us, and workload 3 (8192) went from 200 to 210 us and
// workload 5 (16384) from 666 to 691 us.
constexpr long long kFuseDecideBlocks = 1024;

// Fused passes of at most this many workgroups also make the draw, in each
// sequence's last workgroup (one dependent launch fewer), found with
// per-sequence counters that the call's first kernel zeroes.  Measured from
// graph replays: at 128 workgroups the fused draw saves 0.3-0.6 us a call
// (B = 8 fp16 V = 32000 14.9 -> 14.3 us), at 256 it loses 0.7 us; with the
// draw in every pass, workload 5 went from 673 to 728 us per call, workload
// 3 from 201 to 223 us and workload 2 from 22.7 to 25.8 us.
constexpr long long kFusePickBlocks = 128;

struct SamplePlan {
    int nchunks;
    int vec_per_chunk;
    int chunks_per_block;
    int blocks_per_seq;
};

SamplePlan plan_sample(int B, int nvec)
{
    SamplePlan p;
    const int rounds = (nvec + kBlock - 1) / kBlock;
    int rpc = (rounds + kMaxChunks - 1) / kMaxChunks;
    // two-round chunks whenever one-round chunks would give more than half
    // the cap (512 x 63 rounds: 16384 two-round workgroups; 256 x 63 rounds:
    // 8192 two-round workgroups, 23.7 us against 27.5 us for 16128 one-round
    // ones, and a shorter chunk-total walk in the draw)
    if (rounds >= 2 && (long long)B * rounds > kSampleBlocks / 2 && rpc < 2) rpc = 2;
    while (rpc < rounds && (long long)B * ((rounds + rpc - 1) / rpc) > kSampleBlocks) ++rpc;
    // chunks of up to four rounds when that brings the pass within the fused
    // decision's limit (graph replays, bf16 V = 128256, k = 4: B = 24 28.9 ->
    // 25.4 us a call, B = 32 32.4 -> 28.9 us, B = 64 46.6 -> 44.1 us; B = 96
    // and 128 unchanged)
    for (int r = rpc; r <= 4 && r <= rounds; ++r)
        if ((long long)B * ((rounds + r - 1) / r) <= kFuseDecideBlocks) {
            rpc = r;
            break;
        }
    p.vec_per_chunk = rpc * kBlock;
    p.nchunks = (nvec + p.vec_per_chunk - 1) / p.vec_per_chunk;
    p.chunks_per_block = 1;
    p.blocks_per_seq = p.nchunks;
    return p;
}

struct Workspace {
    void* partials;
    TruncRow* trunc;                   // truncated sampling: one per row
    SampleDesc* desc;
    float* chunk_sums;
    int* lists;                        // early exit: two lists of B sequence ids
    int* counts;                       // early exit: their two counters
    int* done;                         // the draw in the chunk pass: B counters
    uint32_t* cand;                    // truncation of few rows: candidate keys per row slice
    uint32_t* cand_hdr;                // and each slice's floor, largest key, count, overflow
    size_t bytes;
};

// Layout: [split partials][truncated rows][sample descriptors][chunk totals]
// [work lists][counters][draw counters][slice candidates][slice headers],
// each region 256-byte aligned; the last two only for a call that cuts its
// rows into `slices` > 1 (a truncated call with a small top-k, few rows).
Workspace layout(char* base, int B, long long rows, int V, int slices)
{
    Workspace w;
    const StatsPlan sp = plan_stats(rows, V);
    const SamplePlan pp = plan_sample(B, sp.nvec);
    size_t off = 0;
    w.partials = base ? base + off : nullptr;
    off += align_up((size_t)rows * sp.splits * 8);
    w.trunc = base ? reinterpret_cast<TruncRow*>(base + off) : nullptr;
    off += align_up((size_t)rows * sizeof(TruncRow));
    w.desc = base ? reinterpret_cast<SampleDesc*>(base + off) : nullptr;
    off += align_up((size_t)B * sizeof(SampleDesc));
    w.chunk_sums = base ? reinterpret_cast<float*>(base + off) : nullptr;
    off += align_up((size_t)B * pp.nchunks * sizeof(float));
    w.lists = base ? reinterpret_cast<int*>(base + off) : nullptr;
    off += align_up((size_t)2 * B * sizeof(int));
    w.counts = base ? reinterpret_cast<int*>(base + off) : nullptr;
    off += align_up(2 * sizeof(int));
    w.done = base ? reinterpret_cast<int*>(base + off) : nullptr;
    off += align_up((size_t)B * sizeof(int));
    const int sl = slices;
    w.cand = nullptr;
    w.cand_hdr = nullptr;
    if (sl > 1) {
        w.cand = base ? reinterpret_cast<uint32_t*>(base + off) : nullptr;
        off += align_up((size_t)rows * sl * kCandMax * sizeof(uint32_t));
        w.cand_hdr = base ? reinterpret_cast<uint32_t*>(base + off) : nullptr;
        off += align_up((size_t)rows * sl * 4 * sizeof(uint32_t));
    }
    w.bytes = off;
    return w;
}

bool fits_grid(long long rows, int V)
{
    const StatsPlan sp = plan_stats(rows, V);
    return rows * sp.splits < (1LL << 31);
}

bool vec_ok(const void* p, long long stride, int dt)
{
    const long long es = elem_size(dt);
    return ((uintptr_t)p % 16 == 0) && ((stride * es) % 16 == 0);
}

// ---- measurement variants: the caller's two events (hipEvent_t, or null for
// none) recorded on the call's stream right before and right after the
// vocabulary-streaming kernel.  The library keeps no state of its own.
struct Timing {
    hipEvent_t begin = nullptr;
    hipEvent_t end = nullptr;
};

hipError_t mark(hipEvent_t ev, hipStream_t st)
{
    return ev ? hipEventRecord(ev, st) : hipSuccess;
}

// What every greedy entry point checks and derives before its first launch.
struct GreedyCall {
    Workspace w;
    StatsPlan sp;
    long long rows;
    bool vec;
    hipStream_t st;
};

int prepare_greedy(const void* target_logits, long long target_row_stride, const int* draft_tokens,
                   int B, int k, int V, int dtype, const int* out_tokens, const int* out_num_accepted,
                   void* workspace, size_t workspace_bytes, void* hip_stream, GreedyCall& gc)
{
    if (!dtype_ok(dtype)) return SV_EDTYPE;
    if (!target_logits || !draft_tokens || !out_tokens || !out_num_accepted) return SV_EINVAL;
    if (B < 1 || k < 1 || k > SV_MAX_K || V < 1 || V > kMaxV || target_row_stride < V) return SV_EINVAL;
    gc.rows = (long long)B * (k + 1);
    if (!fits_grid(gc.rows, V)) return SV_EINVAL;
    gc.w = layout(static_cast<char*>(workspace), B, gc.rows, V, 1);
    if (!workspace || workspace_bytes < gc.w.bytes) return SV_EWORKSPACE;
    gc.st = static_cast<hipStream_t>(hip_stream);
    gc.vec = vec_ok(target_logits, target_row_stride, dtype);
    gc.sp = plan_stats(gc.rows, V);
    return SV_OK;
}

DecideGreedyArgs decide_greedy_args(const int* draft_tokens, int B, int k, const GreedyCall& gc,
                                    int* out_tokens, int* out_num_accepted, int* out_argmax,
                                    unsigned long long* out_match_mask, int* out_num_match)
{
    DecideGreedyArgs da;
    da.tokens = draft_tokens;
    da.B = B;
    da.k = k;
    da.splits = gc.sp.splits;
    da.partials = static_cast<const ArgPartial*>(gc.w.partials);
    da.out_tokens = out_tokens;
    da.out_num_accepted = out_num_accepted;
    da.out_argmax = out_argmax;
    da.out_match_mask = out_match_mask;
    da.out_num_match = out_num_match;
    return da;
}

int greedy_impl(const void* target_logits, long long target_row_stride,
                const int* draft_tokens, int B, int k, int V, int dtype,
                int* out_tokens, int* out_num_accepted, int* out_argmax,
                unsigned long long* out_match_mask, int* out_num_match,
                void* workspace, size_t workspace_bytes, void* hip_stream, const Timing& tm = Timing())
{
    GreedyCall gc;
    const int status = prepare_greedy(target_logits, target_row_stride, draft_tokens, B, k, V, dtype,
                                      out_tokens, out_num_accepted, workspace, workspace_bytes, hip_stream, gc);
    if (status != SV_OK) return status;

    StatsArgs sa{};
    sa.target = target_logits;
    sa.t_stride = target_row_stride;
    sa.draft = nullptr;
    sa.d_stride = 0;
    sa.n_target_rows = (int)gc.rows;
    sa.n_rows = (int)gc.rows;
    sa.V = V;
    sa.nvec = gc.sp.nvec;
    sa.splits = gc.sp.splits;
    sa.vec_per_split = gc.sp.vec_per_split;
    sa.c = 0.f;
    sa.partials = gc.w.partials;
    if (mark(tm.begin, gc.st) != hipSuccess) return SV_EHIP;
    if (launch_argmax_stats(dtype, gc.vec, sa, gc.st) != hipSuccess) return SV_EHIP;
    if (mark(tm.end, gc.st) != hipSuccess) return SV_EHIP;

    const DecideGreedyArgs da = decide_greedy_args(draft_tokens, B, k, gc, out_tokens, out_num_accepted,
                                                   out_argmax, out_match_mask, out_num_match);
    if (launch_decide_greedy(da, gc.st) != hipSuccess) return SV_EHIP;
    return SV_OK;
}

// What every sampling entry point checks and derives before its first
// launch, in this order: arguments, the workspace, the statistics plan, the
// stream and c = log2(e) / T.
struct SampleCall {
    Workspace w;
    StatsPlan sp;
    long long rows;
    float c;
    bool vec;
    bool trunc;                        // top-k or top-p is on
    int slices;                        // truncation: slices per row (1: none)
    hipStream_t st;
};

int prepare_sample(const void* target_logits, long long target_row_stride,
                   const void* draft_logits, long long draft_row_stride,
                   const int* draft_tokens, const float* uniforms, float temperature,
                   float lenience, int top_k, float top_p, int B, int k, int V, int dtype,
                   const int* out_tokens, const int* out_num_accepted,
                   void* workspace, size_t workspace_bytes, void* hip_stream, SampleCall& sc)
{
    if (!dtype_ok(dtype)) return SV_EDTYPE;
    if (!target_logits || !draft_logits || !draft_tokens || !uniforms || !out_tokens ||
        !out_num_accepted)
        return SV_EINVAL;
    if (B < 1 || k < 1 || k > SV_MAX_K || V < 1 || V > kMaxV) return SV_EINVAL;
    if (target_row_stride < V || draft_row_stride < V) return SV_EINVAL;
    if (!(temperature > 0.f) || !isfinite(temperature)) return SV_EINVAL;
    if (!(lenience >= 1.f) || !isfinite(lenience)) return SV_EINVAL;
    if (top_k < 0 || !(top_p > 0.f) || isnan(top_p)) return SV_EINVAL;
    sc.trunc = (top_k >= 1 && top_k < V) || top_p < 1.f;
    if (sc.trunc && V > kMaxTruncV) return SV_EINVAL;
    const double cd = 1.4426950408889634 / (double)temperature;
    if (!isfinite(cd) || cd > 3.0e38) return SV_EINVAL;
    sc.rows = (long long)B * (2 * k + 1);
    if (!fits_grid(sc.rows, V)) return SV_EINVAL;
    sc.slices = sc.trunc ? trunc_slices(sc.rows, V, elem_size(dtype), top_k) : 1;
    sc.w = layout(static_cast<char*>(workspace), B, sc.rows, V, sc.slices);
    if (!workspace || workspace_bytes < sc.w.bytes) return SV_EWORKSPACE;
    sc.st = static_cast<hipStream_t>(hip_stream);
    sc.c = (float)cd;
    sc.vec = vec_ok(target_logits, target_row_stride, dtype) && vec_ok(draft_logits, draft_row_stride, dtype);
    sc.sp = plan_stats(sc.rows, V);
    return SV_OK;
}

// The decision kernel's arguments: the rows' slice partials, or with
// truncation the truncated rows' summaries.
DecideSampleArgs decide_sample_args(const void* target_logits, long long target_row_stride,
                                    const void* draft_logits, long long draft_row_stride,
                                    const int* draft_tokens, const float* uniforms, float lenience,
                                    int B, int k, int V, const SampleCall& sc,
                                    int* out_tokens, int* out_num_accepted,
                                    float* out_p_x, float* out_q_x)
{
    DecideSampleArgs da;
    da.target = target_logits;
    da.t_stride = target_row_stride;
    da.draft = draft_logits;
    da.d_stride = draft_row_stride;
    da.tokens = draft_tokens;
    da.uniforms = uniforms;
    da.B = B;
    da.k = k;
    da.V = V;
    da.splits = sc.sp.splits;
    da.c = sc.c;
    da.log2_lenience = (float)log2((double)lenience);
    da.partials = static_cast<const SoftPartial*>(sc.w.partials);
    da.trunc = sc.trunc ? sc.w.trunc : nullptr;
    da.out_tokens = out_tokens;
    da.out_num_accepted = out_num_accepted;
    da.out_p_x = out_p_x;
    da.out_q_x = out_q_x;
    da.desc = sc.w.desc;
    return da;
}

// The sampler's arguments: the round's one draw per sequence (in the chunk
// pass when `pick_in_pass`).
SampleArgs sampler_args(const void* target_logits, long long target_row_stride,
                        const void* draft_logits, long long draft_row_stride,
                        int B, int k, int V, const SampleCall& sc, int* out_tokens, bool pick_in_pass = false)
{
    const SamplePlan pp = plan_sample(B, sc.sp.nvec);
    SampleArgs ma{};
    ma.target = target_logits;
    ma.t_stride = target_row_stride;
    ma.draft = draft_logits;
    ma.d_stride = draft_row_stride;
    ma.V = V;
    ma.nvec = sc.sp.nvec;
    ma.nchunks = pp.nchunks;
    ma.vec_per_chunk = pp.vec_per_chunk;
    ma.chunks_per_block = pp.chunks_per_block;
    ma.blocks_per_seq = pp.blocks_per_seq;
    ma.c = sc.c;
    ma.desc = sc.w.desc;
    ma.chunk_sums = sc.w.chunk_sums;
    ma.out_tokens = out_tokens;
    ma.out_row = k + 1;
    ma.n_target_rows = B * (k + 1);
    ma.n_draft_rows = B * k;
    ma.done = pick_in_pass ? sc.w.done : nullptr;
    return ma;
}

int sample_impl(const void* target_logits, long long target_row_stride,
                const void* draft_logits, long long draft_row_stride,
                const int* draft_tokens, const float* uniforms, float temperature,
                float lenience, int top_k, float top_p, int B, int k, int V, int dtype,
                int* out_tokens, int* out_num_accepted,
                float* out_p_x, float* out_q_x,
                void* workspace, size_t workspace_bytes, void* hip_stream, const Timing& tm = Timing())
{
    SampleCall sc;
    const int status = prepare_sample(target_logits, target_row_stride, draft_logits, draft_row_stride,
                                      draft_tokens, uniforms, temperature, lenience, top_k, top_p, B, k, V,
                                      dtype, out_tokens, out_num_accepted, workspace, workspace_bytes,
                                      hip_stream, sc);
    if (status != SV_OK) return status;
    // small passes decide the round and make the draw in the chunk pass's
    // launch, its counters zeroed by the first kernel
    const SamplePlan pp = plan_sample(B, sc.sp.nvec);
    const bool pick_in_pass = (long long)B * pp.blocks_per_seq <= kFusePickBlocks;

    if (mark(tm.begin, sc.st) != hipSuccess) return SV_EHIP;
    if (sc.trunc) {
        TruncArgs ta{};
        ta.target = target_logits;
        ta.t_stride = target_row_stride;
        ta.draft = draft_logits;
        ta.d_stride = draft_row_stride;
        ta.n_target_rows = B * (k + 1);
        ta.n_rows = (int)sc.rows;
        ta.V = V;
        ta.c = sc.c;
        ta.top_k = top_k;
        ta.top_p = top_p;
        ta.rows = sc.w.trunc;
        ta.zero = pick_in_pass ? sc.w.done : nullptr;
        ta.n_zero = pick_in_pass ? B : 0;
        ta.slices = sc.slices;
        ta.cand = sc.w.cand;
        ta.cand_hdr = sc.w.cand_hdr;
        if (launch_trunc_rows(dtype, sc.vec, ta, sc.st) != hipSuccess) return SV_EHIP;
    } else {
        StatsArgs sa{};
        sa.target = target_logits;
        sa.t_stride = target_row_stride;
        sa.draft = draft_logits;
        sa.d_stride = draft_row_stride;
        sa.n_target_rows = B * (k + 1);
        sa.n_rows = (int)sc.rows;
        sa.V = V;
        sa.nvec = sc.sp.nvec;
        sa.splits = sc.sp.splits;
        sa.vec_per_split = sc.sp.vec_per_split;
        sa.c = sc.c;
        sa.partials = sc.w.partials;
        sa.zero = pick_in_pass ? sc.w.done : nullptr;
        sa.n_zero = pick_in_pass ? B : 0;
        if (launch_softmax_stats(dtype, sc.vec, sa, sc.st) != hipSuccess) return SV_EHIP;
    }
    if (mark(tm.end, sc.st) != hipSuccess) return SV_EHIP;

    const DecideSampleArgs da =
        decide_sample_args(target_logits, target_row_stride, draft_logits, draft_row_stride, draft_tokens,
                           uniforms, lenience, B, k, V, sc, out_tokens, out_num_accepted, out_p_x, out_q_x);
    const SampleArgs ma = sampler_args(target_logits, target_row_stride, draft_logits, draft_row_stride, B, k, V,
                                       sc, out_tokens, pick_in_pass);
    // Small passes decide in the chunk pass's own launch (one dependent
    // launch fewer); large ones decide in a kernel of their own, since every
    // chunk workgroup would repeat its sequence's decision and scattered
    // gathers (workload 5: 71 us for the fused pass against 5 + 42 us).
    if ((long long)B * ma.blocks_per_seq > kFuseDecideBlocks) {
        if (launch_decide_sample(dtype, da, sc.st) != hipSuccess) return SV_EHIP;
        if (launch_sample(dtype, sc.vec, sc.trunc, B, nullptr, ma, sc.st) != hipSuccess) return SV_EHIP;
    } else {
        if (launch_sample(dtype, sc.vec, sc.trunc, B, &da, ma, sc.st) != hipSuccess) return SV_EHIP;
    }
    return SV_OK;
}

int candidates_impl(const void* target_logits, long long row_stride,
                    const int* cand_tokens, const int* cand_rows, int N, int B, int C, int L, int R,
                    int V, int dtype, int* out_tokens, int* out_num_accepted,
                    int* out_best_candidate, int* out_argmax,
                    void* workspace, size_t workspace_bytes, void* hip_stream, const Timing& tm = Timing())
{
    if (!dtype_ok(dtype)) return SV_EDTYPE;
    if (!target_logits || !cand_tokens || !out_tokens || !out_num_accepted || !out_best_candidate)
        return SV_EINVAL;
    if (B < 1 || C < 1 || L < 1 || L > SV_MAX_K || (long long)C * L > SV_MAX_CANDIDATE_TOKENS)
        return SV_EINVAL;
    if ((R != L && R != L + 1) || V < 1 || V > kMaxV || row_stride < V) return SV_EINVAL;
    if (cand_rows && N < 1) return SV_EINVAL;
    const long long rows = (long long)B * (cand_rows ? (long long)N : (long long)C * R);
    if (!fits_grid(rows, V)) return SV_EINVAL;
    Workspace w = layout(static_cast<char*>(workspace), B, rows, V, 1);
    if (!workspace || workspace_bytes < w.bytes) return SV_EWORKSPACE;
    hipStream_t st = static_cast<hipStream_t>(hip_stream);

    const StatsPlan sp = plan_stats(rows, V);
    StatsArgs sa{};
    sa.target = target_logits;
    sa.t_stride = row_stride;
    sa.draft = nullptr;
    sa.d_stride = 0;
    sa.n_target_rows = (int)rows;
    sa.n_rows = (int)rows;
    sa.V = V;
    sa.nvec = sp.nvec;
    sa.splits = sp.splits;
    sa.vec_per_split = sp.vec_per_split;
    sa.c = 0.f;
    sa.partials = w.partials;
    if (mark(tm.begin, st) != hipSuccess) return SV_EHIP;
    if (launch_argmax_stats(dtype, vec_ok(target_logits, row_stride, dtype), sa, st) != hipSuccess)
        return SV_EHIP;
    if (mark(tm.end, st) != hipSuccess) return SV_EHIP;

    DecideCandArgs da;
    da.cand = cand_tokens;
    da.cand_rows = cand_rows;
    da.N = N;
    da.B = B;
    da.C = C;
    da.L = L;
    da.R = R;
    da.splits = sp.splits;
    da.partials = static_cast<const ArgPartial*>(w.partials);
    da.out_tokens = out_tokens;
    da.out_num_accepted = out_num_accepted;
    da.out_best = out_best_candidate;
    da.out_argmax = out_argmax;
    if (launch_decide_candidates(da, st) != hipSuccess) return SV_EHIP;
    return SV_OK;
}

// ---- early exit -------------------------------------------------------------
// Window bounds 0, 1, 2, 4, 8, ... clipped to k+1: one position at a time while
// most sequences are still deciding, then doubling.
int lazy_bounds(int k, int* bounds)
{
    int n = 0;
    bounds[n++] = 0;
    int next = 1;
    while (bounds[n - 1] < k + 1) {
        bounds[n++] = next < k + 1 ? next : k + 1;
        next = next < 2 ? next + 1 : next * 2;
    }
    // a last window [k, k+1) would hold only the bonus row and cost two
    // launches that are nearly always empty: the window before takes it
    if (n >= 3 && bounds[n - 2] == k) {
        bounds[n - 2] = k + 1;
        --n;
    }
    return n;
}

// Workgroups of an early-exit statistics launch, which loop over the window's
// (row, slice) units.  A late window is often nearly empty, and every one of
// its workgroups is still dispatched to find no work: 2048 (8 per CU) kept
// the full first window's rate and made greedy early exit about 4% faster
// than 4096 on a 512-sequence batch; 1024 slowed the sampling form.
constexpr int kLazyGrid = 2048;

LazyArgs lazy_args(const void* target, long long ts, const void* draft, long long ds, int B, int k,
                   int V, const StatsPlan& sp, float c, const Workspace& w)
{
    LazyArgs l;
    l.target = target;
    l.t_stride = ts;
    l.draft = draft;
    l.d_stride = ds;
    l.B = B;
    l.k = k;
    l.V = V;
    l.nvec = sp.nvec;
    l.splits = sp.splits;
    l.vec_per_split = sp.vec_per_split;
    l.n_target_rows = B * (k + 1);
    l.c = c;
    l.partials = w.partials;
    return l;
}

// Point window `p` of the schedule at its input and output work lists.
void lazy_window(LazyArgs& l, const Workspace& w, const int* bounds, int p, int B)
{
    l.w0 = bounds[p];
    l.w1 = bounds[p + 1];
    l.list_in = p == 0 ? nullptr : w.lists + (size_t)(p % 2) * B;
    l.count_in = p == 0 ? nullptr : w.counts + (p % 2);
    l.list_out = w.lists + (size_t)((p + 1) % 2) * B;
    l.count_out = w.counts + ((p + 1) % 2);
    l.count_clear = l.count_out;
}

int lazy_grid(const LazyArgs& l, bool with_draft)
{
    const int nt = l.w1 - l.w0;
    const int nd = with_draft ? (l.w0 < l.k ? (l.w1 < l.k ? l.w1 : l.k) - l.w0 : 0) : 0;
    const long long units = (long long)l.B * (nt + nd) * l.splits;
    return (int)(units < kLazyGrid ? units : kLazyGrid);
}

// The device address of the current device's copy of `scratch`, looked up
// with hipGetSymbolAddress on the first call on that device (with that device
// current) and kept per device; null if the lookup fails.
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

void* scratch_address(int dev)
{
    if (dev < 0 || dev >= kMaxDevices) return nullptr;
    void* p = g_scratch[dev].load(std::memory_order_acquire);
    if (p) return p;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (!p) {
        void* q = nullptr;
        if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || !q) return nullptr;
        g_scratch[dev].store(q, std::memory_order_release);
        p = q;
    }
    return p;
}

}  // namespace

extern "C" {

int spec_verify_version(void) { return 200; }

const char* spec_verify_status_string(int s)
{
    switch (s) {
    case SV_OK: return "SV_OK";
    case SV_EINVAL: return "SV_EINVAL: invalid argument";
    case SV_EDTYPE: return "SV_EDTYPE: unknown dtype";
    case SV_EWORKSPACE: return "SV_EWORKSPACE: workspace missing or too small";
    case SV_EHIP: return "SV_EHIP: HIP launch error";
    case SV_ESCRATCH: return "SV_ESCRATCH: the call needs more scratch than SV_NOALLOC_SCRATCH_BYTES";
    default: return "unknown status";
    }
}

size_t spec_verify_workspace_bytes(int B, int rows_per_seq, int V, int dtype)
{
    if (B < 1 || rows_per_seq < 1 || V < 1 || V > kMaxV || !dtype_ok(dtype)) return 0;
    const long long rows = (long long)B * rows_per_seq;
    if (!fits_grid(rows, V)) return 0;
    // enough for any call: fp32 rows may be cut into slices
    return layout(nullptr, B, rows, V, elem_size(dtype) == 4 ? split_slices(rows, V) : 1).bytes;
}

int spec_verify_greedy(const void* target_logits, long long target_row_stride,
                       const int* draft_tokens, int B, int k, int V, int dtype,
                       int* out_tokens, int* out_num_accepted,
                       void* workspace, size_t workspace_bytes, void* hip_stream)
{
    return greedy_impl(target_logits, target_row_stride, draft_tokens, B, k, V, dtype, out_tokens,
                       out_num_accepted, nullptr, nullptr, nullptr, workspace, workspace_bytes,
                       hip_stream);
}

int spec_verify_greedy_ext(const void* target_logits, long long target_row_stride,
                           const int* draft_tokens, int B, int k, int V, int dtype,
                           int* out_tokens, int* out_num_accepted, int* out_target_argmax,
                           unsigned long long* out_match_mask, int* out_num_match,
                           void* workspace, size_t workspace_bytes, void* hip_stream)
{
    return greedy_impl(target_logits, target_row_stride, draft_tokens, B, k, V, dtype, out_tokens,
                       out_num_accepted, out_target_argmax, out_match_mask, out_num_match,
                       workspace, workspace_bytes, hip_stream);
}

int spec_verify_sample(const void* target_logits, long long target_row_stride,
                       const void* draft_logits, long long draft_row_stride,
                       const int* draft_tokens, const float* uniforms, float temperature,
                       int B, int k, int V, int dtype,
                       int* out_tokens, int* out_num_accepted,
                       float* out_p_x, float* out_q_x,
                       void* workspace, size_t workspace_bytes, void* hip_stream)
{
    return sample_impl(target_logits, target_row_stride, draft_logits, draft_row_stride,
                       draft_tokens, uniforms, temperature, 1.f, 0, 1.f, B, k, V, dtype, out_tokens,
                       out_num_accepted, out_p_x, out_q_x, workspace, workspace_bytes, hip_stream);
}

int spec_verify_sample_lenient(const void* target_logits, long long target_row_stride,
                               const void* draft_logits, long long draft_row_stride,
                               const int* draft_tokens, const float* uniforms, float temperature,
                               float lenience, int B, int k, int V, int dtype,
                               int* out_tokens, int* out_num_accepted,
                               float* out_p_x, float* out_q_x,
                               void* workspace, size_t workspace_bytes, void* hip_stream)
{
    return sample_impl(target_logits, target_row_stride, draft_logits, draft_row_stride,
                       draft_tokens, uniforms, temperature, lenience, 0, 1.f, B, k, V, dtype, out_tokens,
                       out_num_accepted, out_p_x, out_q_x, workspace, workspace_bytes, hip_stream);
}

int spec_verify_sample_truncated(const void* target_logits, long long target_row_stride,
                                 const void* draft_logits, long long draft_row_stride,
                                 const int* draft_tokens, const float* uniforms, float temperature,
                                 int top_k, float top_p, int B, int k, int V, int dtype,
                                 int* out_tokens, int* out_num_accepted,
                                 float* out_p_x, float* out_q_x,
                                 void* workspace, size_t workspace_bytes, void* hip_stream)
{
    return sample_impl(target_logits, target_row_stride, draft_logits, draft_row_stride,
                       draft_tokens, uniforms, temperature, 1.f, top_k, top_p, B, k, V, dtype,
                       out_tokens, out_num_accepted, out_p_x, out_q_x, workspace, workspace_bytes,
                       hip_stream);
}

int spec_verify_greedy_candidates(const void* target_logits, long long row_stride,
                                  const int* cand_tokens, int B, int C, int L, int R, int V,
                                  int dtype, int* out_tokens, int* out_num_accepted,
                                  int* out_best_candidate,
                                  void* workspace, size_t workspace_bytes, void* hip_stream)
{
    return candidates_impl(target_logits, row_stride, cand_tokens, nullptr, 0, B, C, L, R, V, dtype,
                           out_tokens, out_num_accepted, out_best_candidate, nullptr, workspace,
                           workspace_bytes, hip_stream);
}

int spec_verify_greedy_tree(const void* node_logits, long long row_stride, int N,
                            const int* cand_tokens, const int* cand_rows, int B, int C, int L, int R,
                            int V, int dtype, int* out_tokens, int* out_num_accepted,
                            int* out_best_candidate,
                            void* workspace, size_t workspace_bytes, void* hip_stream)
{
    if (!cand_rows) return SV_EINVAL;
    return candidates_impl(node_logits, row_stride, cand_tokens, cand_rows, N, B, C, L, R, V, dtype,
                           out_tokens, out_num_accepted, out_best_candidate, nullptr, workspace,
                           workspace_bytes, hip_stream);
}

int spec_verify_greedy_candidates_ext(const void* target_logits, long long row_stride,
                                      const int* cand_tokens, int B, int C, int L, int R, int V,
                                      int dtype, int* out_tokens, int* out_num_accepted,
                                      int* out_best_candidate, int* out_target_argmax,
                                      void* workspace, size_t workspace_bytes, void* hip_stream)
{
    return candidates_impl(target_logits, row_stride, cand_tokens, nullptr, 0, B, C, L, R, V, dtype,
                           out_tokens, out_num_accepted, out_best_candidate, out_target_argmax,
                           workspace, workspace_bytes, hip_stream);
}

int spec_verify_sample_lazy(const void* target_logits, long long target_row_stride,
                            const void* draft_logits, long long draft_row_stride,
                            const int* draft_tokens, const float* uniforms, float temperature,
                            int B, int k, int V, int dtype, int* out_tokens, int* out_num_accepted,
                            void* workspace, size_t workspace_bytes, void* hip_stream)
{
    SampleCall sc;
    const int status = prepare_sample(target_logits, target_row_stride, draft_logits, draft_row_stride,
                                      draft_tokens, uniforms, temperature, 1.f, 0, 1.f, B, k, V, dtype,
                                      out_tokens, out_num_accepted, workspace, workspace_bytes, hip_stream,
                                      sc);
    if (status != SV_OK) return status;

    const DecideSampleArgs da =
        decide_sample_args(target_logits, target_row_stride, draft_logits, draft_row_stride, draft_tokens,
                           uniforms, 1.f, B, k, V, sc, out_tokens, out_num_accepted, nullptr, nullptr);
    LazyArgs l = lazy_args(target_logits, target_row_stride, draft_logits, draft_row_stride, B, k, V,
                           sc.sp, sc.c, sc.w);
    int bounds[16];
    const int nb = lazy_bounds(k, bounds);
    for (int p = 0; p + 1 < nb; ++p) {
        lazy_window(l, sc.w, bounds, p, B);
        if (launch_lazy_stats(dtype, sc.vec, true, lazy_grid(l, true), l, sc.st) != hipSuccess) return SV_EHIP;
        if (launch_lazy_decide_sample(dtype, l, da, sc.st) != hipSuccess) return SV_EHIP;
    }
    const SampleArgs ma =
        sampler_args(target_logits, target_row_stride, draft_logits, draft_row_stride, B, k, V, sc, out_tokens);
    if (launch_sample(dtype, sc.vec, false, B, nullptr, ma, sc.st) != hipSuccess) return SV_EHIP;
    return SV_OK;
}

int spec_verify_greedy_lazy(const void* target_logits, long long target_row_stride,
                            const int* draft_tokens, int B, int k, int V, int dtype,
                            int* out_tokens, int* out_num_accepted,
                            void* workspace, size_t workspace_bytes, void* hip_stream)
{
    GreedyCall gc;
    const int status = prepare_greedy(target_logits, target_row_stride, draft_tokens, B, k, V, dtype,
                                      out_tokens, out_num_accepted, workspace, workspace_bytes, hip_stream, gc);
    if (status != SV_OK) return status;

    const DecideGreedyArgs da =
        decide_greedy_args(draft_tokens, B, k, gc, out_tokens, out_num_accepted, nullptr, nullptr, nullptr);
    LazyArgs l = lazy_args(target_logits, target_row_stride, nullptr, 0, B, k, V, gc.sp, 0.f, gc.w);
    int bounds[16];
    const int nb = lazy_bounds(k, bounds);
    for (int p = 0; p + 1 < nb; ++p) {
        lazy_window(l, gc.w, bounds, p, B);
        if (launch_lazy_stats(dtype, gc.vec, false, lazy_grid(l, false), l, gc.st) != hipSuccess) return SV_EHIP;
        if (launch_lazy_decide_greedy(l, da, gc.st) != hipSuccess) return SV_EHIP;
    }
    return SV_OK;
}

int spec_verify_sample_noalloc(const void* target_logits, long long target_row_stride,
                               const void* draft_logits, long long draft_row_stride,
                               const int* draft_tokens, const float* uniforms, float temperature,
                               int B, int k, int V, int dtype,
                               int* out_tokens, int* out_num_accepted,
                               float* out_p_x, float* out_q_x, void* hip_stream)
{
    // a call whose shape needs more scratch than the static buffer is refused
    // before anything else (shapes any call rejects are left to the checks of
    // spec_verify_sample, which follow)
    if (B >= 1 && k >= 1 && k <= SV_MAX_K && V >= 1 && V <= kMaxV && dtype_ok(dtype)) {
        const long long rows = (long long)B * (2 * k + 1);
        if (fits_grid(rows, V) && layout(nullptr, B, rows, V, 1).bytes > SV_NOALLOC_SCRATCH_BYTES)
            return SV_ESCRATCH;
    }
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return SV_EHIP;
    if (hip_stream) {
        hipDevice_t sdev = -1;
        if (hipStreamGetDevice(static_cast<hipStream_t>(hip_stream), &sdev) != hipSuccess) return SV_EHIP;
        if (sdev != dev) return SV_EINVAL;
    }
    void* ws = scratch_address(dev);
    if (!ws) return SV_EHIP;
    return sample_impl(target_logits, target_row_stride, draft_logits, draft_row_stride,
                       draft_tokens, uniforms, temperature, 1.f, 0, 1.f, B, k, V, dtype, out_tokens,
                       out_num_accepted, out_p_x, out_q_x, ws, SV_NOALLOC_SCRATCH_BYTES, hip_stream);
}

int spec_verify_sample_timed(const void* target_logits, long long target_row_stride,
                             const void* draft_logits, long long draft_row_stride,
                             const int* draft_tokens, const float* uniforms, float temperature,
                             float lenience, int top_k, float top_p, int B, int k, int V, int dtype,
                             int* out_tokens, int* out_num_accepted, float* out_p_x, float* out_q_x,
                             void* workspace, size_t workspace_bytes, void* hip_stream,
                             void* event_begin, void* event_end)
{
    if (!event_begin || !event_end) return SV_EINVAL;
    Timing tm;
    tm.begin = static_cast<hipEvent_t>(event_begin);
    tm.end = static_cast<hipEvent_t>(event_end);
    return sample_impl(target_logits, target_row_stride, draft_logits, draft_row_stride,
                       draft_tokens, uniforms, temperature, lenience, top_k, top_p, B, k, V, dtype,
                       out_tokens, out_num_accepted, out_p_x, out_q_x, workspace, workspace_bytes,
                       hip_stream, tm);
}

int spec_verify_greedy_timed(const void* target_logits, long long target_row_stride,
                             const int* draft_tokens, int B, int k, int V, int dtype,
                             int* out_tokens, int* out_num_accepted, int* out_target_argmax,
                             unsigned long long* out_match_mask, int* out_num_match,
                             void* workspace, size_t workspace_bytes, void* hip_stream,
                             void* event_begin, void* event_end)
{
    if (!event_begin || !event_end) return SV_EINVAL;
    Timing tm;
    tm.begin = static_cast<hipEvent_t>(event_begin);
    tm.end = static_cast<hipEvent_t>(event_end);
    return greedy_impl(target_logits, target_row_stride, draft_tokens, B, k, V, dtype, out_tokens,
                       out_num_accepted, out_target_argmax, out_match_mask, out_num_match,
                       workspace, workspace_bytes, hip_stream, tm);
}

int spec_verify_candidates_timed(const void* target_logits, long long row_stride,
                                 const int* cand_tokens, const int* cand_rows, int N,
                                 int B, int C, int L, int R, int V, int dtype,
                                 int* out_tokens, int* out_num_accepted, int* out_best_candidate,
                                 int* out_target_argmax,
                                 void* workspace, size_t workspace_bytes, void* hip_stream,
                                 void* event_begin, void* event_end)
{
    if (!event_begin || !event_end) return SV_EINVAL;
    Timing tm;
    tm.begin = static_cast<hipEvent_t>(event_begin);
    tm.end = static_cast<hipEvent_t>(event_end);
    return candidates_impl(target_logits, row_stride, cand_tokens, cand_rows, N, B, C, L, R, V, dtype,
                           out_tokens, out_num_accepted, out_best_candidate, out_target_argmax,
                           workspace, workspace_bytes, hip_stream, tm);
}

}  // extern "C"
