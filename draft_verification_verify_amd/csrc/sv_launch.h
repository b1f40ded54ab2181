// sv_launch.h -- argument blocks and launchers shared by the host layer
// (sv_api.hip) and the kernel files.  Internal to libspecverify.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sv {

constexpr int kBlock = 256;            // threads per workgroup (4 wave64s)
constexpr int kWaves = kBlock / 64;
constexpr int kStatsBlock = 512;       // the vocabulary-streaming pass: 8 wave64s
constexpr int kVec = 8;                // elements per logical vector (16 B of bf16/fp16)

enum : int { DT_F32 = 0, DT_F16 = 1, DT_BF16 = 2 };

inline int elem_size(int dt) { return dt == DT_F32 ? 4 : 2; }

// Per-(row, split) partial of the softmax statistics: running max m (raw
// logit units) and s = sum exp2(z c - stab_of(m, c)), c = log2(e) / T.
struct SoftPartial { float m; float s; };
// Per-(row, split) partial of the argmax: value and lowest index (INT32_MAX
// when the split holds nothing above -inf).
struct ArgPartial { float v; int i; };

// Vocabulary-streaming statistics over a set of rows.  Rows [0, n_target_rows)
// are target rows r at target + r * t_stride; the rest are draft rows
// (r - n_target_rows) at draft + (r - n_target_rows) * d_stride (strides in
// elements).  Row r, split s covers logical vectors
// [s * vec_per_split, min((s + 1) * vec_per_split, nvec)).
struct StatsArgs {
    const void* target;
    long long t_stride;
    const void* draft;
    long long d_stride;
    int n_target_rows;
    int n_rows;
    int V;
    int nvec;                          // ceil(V / 8)
    int splits;
    int vec_per_split;
    float c;                           // log2(e) / T (softmax statistics only)
    void* partials;                    // [n_rows][splits] SoftPartial or ArgPartial
    int* zero;                         // softmax statistics: n_zero counters that a later
    int n_zero;                        // kernel of the call needs at 0 (null, 0: none)
};

// One sampling step per sequence, prepared by the decision kernel: draw from
// target row t_row or, for kind 0, from the residual max(0, p - q) against
// draft row d_row; write the token at out_pos of the sequence's output row.
// The sampler weighs each token by s_t times its normalised weight (the draw
// divides by the total, so a common factor does not change it):
// p~ = exp2(z c - h_t) and the residual max(0, p~ - kq q~) with
// q~ = exp2(y c - h_d), h = stab_of(m, c); on truncated rows exp2((z - m) c),
// masked by the key threshold.
struct SampleDesc {
    int t_row;
    int d_row;
    int out_pos;
    int kind;                          // 0 residual, 1 target row (bonus)
    float m_t;                         // target row max
    float m_d;                         // draft row max (kind 0)
    float kq;                          // s_t / s_d, the rows' (kept) masses (kind 0)
    float u;
    uint32_t tau_t;                    // truncation: keep z with key >= tau_t (0: keep all)
    uint32_t tau_d;
};

// A truncated row (top-k, then top-p): its max m, log2 of the kept mass
// relative to exp2(m * c), and the smallest kept ordering key (key_of in
// sv_device.h): token t keeps p'(t) = exp2((z_t - m) * c - l2s) iff
// key(z_t) >= tau, else 0.  pad = 1 marks a row the one-pass 16-bit kernel
// left to the radix kernel.
struct TruncRow {
    float m;
    float l2s;
    uint32_t tau;
    uint32_t pad;
};

// Few fp32 rows under a small top-k are cut into slices, each summarised by
// its own workgroup as the candidates a row's top_k can come from (at most
// kCandMax keys per slice), and merged per row by a second launch.  Slices
// per row: as many as give about kSplitTarget workgroups, at most kSplitMax,
// each of at least kSplitMinVecFew whole 8-logit vectors (16 KB) when the
// rows number at most kSplitFewRows, else kSplitMinVecMany (64 KB); 1 (no
// split) when that leaves fewer than two.  More rows keep the chip busy
// whole, and smaller slices give the merge more candidates to gather.
constexpr int kCandMax = 512;
constexpr int kSplitTarget = 1024;
constexpr int kSplitFewRows = 64;
constexpr int kSplitMinVecFew = 512;
constexpr int kSplitMinVecMany = 2048;
constexpr int kSplitMax = 32;

inline int split_slices(long long n_rows, int V)
{
    const long long nfull = V / kVec;
    const long long min_vec = n_rows <= kSplitFewRows ? kSplitMinVecFew : kSplitMinVecMany;
    long long s = n_rows > 0 ? kSplitTarget / n_rows : 1;
    if (s > nfull / min_vec) s = nfull / min_vec;
    if (s > kSplitMax) s = kSplitMax;
    return s < 2 ? 1 : (int)s;
}

// Top-k values of at most kTopkMax take the candidate lists (one pass per
// row): fp32 rows always, 16-bit rows when they outnumber the compute units
// more than kListRowsPerCU times (fewer take the histogram pass).  Only fp32
// rows are cut into slices; trunc_slices gives a truncated call's slices per
// row (1: none).
constexpr int kTopkMax = 256;
constexpr int kListRowsPerCU = 3;

inline int trunc_slices(long long n_rows, int V, int elem_bytes, int top_k)
{
    return elem_bytes == 4 && top_k >= 1 && top_k <= kTopkMax && top_k < V && V >= 8
               ? split_slices(n_rows, V) : 1;
}

// Truncation of every row of a batch (sv_trunc.hip), rows numbered as in
// StatsArgs.  top_k in [1, V) or 0 (off); top_p in (0, 1), or >= 1 (off).
struct TruncArgs {
    const void* target;
    long long t_stride;
    const void* draft;
    long long d_stride;
    int n_target_rows;
    int n_rows;
    int V;
    float c;
    int top_k;
    float top_p;
    TruncRow* rows;
    int only_marked;                   // radix kernel: only rows whose pad the exact kernel set to 1
    int* zero;                         // n_zero counters zeroed by the first launch, as in
    int n_zero;                        // StatsArgs (null, 0: none)
    int slices;                        // trunc_slices: fp32 rows, a top-k of at most 256
    uint32_t* cand;                    // [n_rows][slices][kCandMax] candidate keys (slices > 1)
    uint32_t* cand_hdr;                // [n_rows][slices][4]: floor, largest key, count, overflow
};

struct DecideSampleArgs {
    const void* target;
    long long t_stride;
    const void* draft;
    long long d_stride;
    const int* tokens;                 // [B][k]
    const float* uniforms;             // [B][k+1]
    int B, k, V, splits;
    float c;
    float log2_lenience;               // log2 l, 0 for the exact rule (l = 1)
    const SoftPartial* partials;       // target rows then draft rows
    const TruncRow* trunc;             // truncated rows (same numbering) or null
    int* out_tokens;                   // [B][k+1]
    int* out_num_accepted;             // [B]
    float* out_p_x;                    // [B][k] or null
    float* out_q_x;                    // [B][k] or null
    SampleDesc* desc;                  // [B]
};

struct DecideGreedyArgs {
    const int* tokens;                 // [B][k]
    int B, k, splits;
    const ArgPartial* partials;        // [B*(k+1)][splits]
    int* out_tokens;
    int* out_num_accepted;
    int* out_argmax;                   // [B][k+1] or null: v_i, the target argmax per position
    unsigned long long* out_match_mask;  // [B] or null: bit i = [x_i == v_i], i < k
    int* out_num_match;                // [B] or null: #Match
};

struct DecideCandArgs {
    const int* cand;                   // [B][C][L]
    const int* cand_rows;              // [B][C][R] node row per position (tree layout) or null (flat)
    int N;                             // node rows per sequence (tree layout)
    int B, C, L, R, splits;
    const ArgPartial* partials;        // [B*C*R][splits]
    int* out_tokens;                   // [B][L+1]
    int* out_num_accepted;
    int* out_best;
    int* out_argmax;                   // [B][C][R] or null: argmax of every scored row
};

// The draw of each sequence (sv_sample.hip).  The sampled row (pair) is cut
// into `nchunks` chunks of `vec_per_chunk` logical vectors (a multiple of
// kBlock); k_sample_chunks writes every chunk's total weight, `chunks_per_block`
// chunks per workgroup; k_sample_pick (one workgroup per sequence) locates
// u * total among the chunk totals and resolves the token inside one chunk.
struct SampleArgs {
    const void* target;
    long long t_stride;
    const void* draft;
    long long d_stride;
    int V, nvec;
    int nchunks;
    int vec_per_chunk;
    int chunks_per_block;
    int blocks_per_seq;
    float c;
    const SampleDesc* desc;
    float* chunk_sums;                 // [B][nchunks]
    int* out_tokens;                   // [B][out_row]
    int out_row;
    int n_target_rows, n_draft_rows;   // bounds every descriptor is checked against
    int* done;                         // [B] the draw in the chunk pass: workgroups finished per
                                       // sequence, zeroed by the call's first kernel (else null)
};

constexpr int kMaxChunks = 128;

// Early-exit verification (sv_stats.hip k_lazy_stats, sv_decide.hip
// k_lazy_decide_*): positions are taken in windows [w0, w1); a window's rows
// are streamed only for the sequences still undecided after the previous
// windows (list_in / count_in; null list_in: every sequence, in order).  The
// decision kernel finishes every sequence that rejects inside the window (or
// reaches position k) and appends the others to list_out / count_out.  The
// statistics kernel zeroes count_clear (the next decision's output counter).
struct LazyArgs {
    const void* target;
    long long t_stride;
    const void* draft;                 // null for greedy
    long long d_stride;
    int B, k, V, nvec, splits, vec_per_split;
    int n_target_rows;                 // B*(k+1); draft rows follow in the partials
    float c;
    void* partials;
    int w0, w1;
    const int* list_in;
    const int* count_in;
    int* list_out;
    int* count_out;
    int* count_clear;
};

hipError_t launch_softmax_stats(int dt, bool vec, const StatsArgs& a, hipStream_t st);
hipError_t launch_argmax_stats(int dt, bool vec, const StatsArgs& a, hipStream_t st);
hipError_t launch_decide_greedy(const DecideGreedyArgs& a, hipStream_t st);
hipError_t launch_decide_candidates(const DecideCandArgs& a, hipStream_t st);
hipError_t launch_decide_sample(int dt, const DecideSampleArgs& a, hipStream_t st);
// The round's draw, after a decision kernel (da null) or deciding the round
// in the same launch as the chunk pass (da given).
hipError_t launch_sample(int dt, bool vec, bool mask, int B, const DecideSampleArgs* da, const SampleArgs& a,
                         hipStream_t st);
hipError_t launch_trunc_rows(int dt, bool vec, const TruncArgs& a, hipStream_t st);
hipError_t launch_lazy_stats(int dt, bool vec, bool soft, int grid, const LazyArgs& a, hipStream_t st);
hipError_t launch_lazy_decide_sample(int dt, const LazyArgs& l, const DecideSampleArgs& a, hipStream_t st);
hipError_t launch_lazy_decide_greedy(const LazyArgs& l, const DecideGreedyArgs& a, hipStream_t st);

}  // namespace sv
