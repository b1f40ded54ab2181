// sv_decide.hip -- per-sequence decisions, one wave64 per sequence.
//
// Lane i handles draft position i (k <= 63, so the k+1 positions fit one
// wave).  The lanes merge their rows' split partials in a fixed order, take
// their own accept/reject decision independently, and a 64-bit ballot plus a
// find-first-set gives the first rejection: the left-to-right scan of the
// rule (production blog, "The acceptance rule") without a serial loop.

#include "sv_device.h"

namespace sv {

constexpr int kSeqPerBlock = kBlock / 64;

// Larger value wins; equal values keep the smaller index.  An all -inf row
// has index INT32_MAX in every split and maps to 0.  The partials are read
// eight at a time (none past `splits`), so each batch's loads overlap.
__device__ __forceinline__ int merge_arg(const ArgPartial* p, int splits)
{
    const unsigned long long* p8 = reinterpret_cast<const unsigned long long*>(p);
    float v = -INFINITY;
    int idx = INT32_MAX;
    for (int i0 = 0; i0 < splits; i0 += 8) {
        ArgPartial q[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {                  // one 8-byte load per partial
            q[u] = ArgPartial{-INFINITY, INT32_MAX};
            if (i0 + u < splits) {
                const unsigned long long w = p8[i0 + u];
                q[u] = ArgPartial{__uint_as_float((uint32_t)w), (int)(uint32_t)(w >> 32)};
            }
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            if (i0 + u < splits && (q[u].v > v || (q[u].v == v && q[u].i < idx))) {
                v = q[u].v;
                idx = q[u].i;
            }
        }
    }
    return idx == INT32_MAX ? 0 : idx;
}

__device__ __forceinline__ unsigned long long ballot64(bool pred)
{
    return __ballot(pred);
}

// ---- sampling --------------------------------------------------------------
// log2 p_i(x) = (z_x - m) * c - log2 s with c = log2(e)/T (log2_prob).  The
// ratio test is taken in the log domain so that no probability underflows: accept iff
// log q <= log p + log l (ratio >= 1, and q = 0) or u < exp2(log p + log l -
// log q).  Lenience l (Cascade Speculative Drafting, review function) is 1
// for the exact rule, where log l = 0 leaves the test unchanged.  With
// truncation, s is the kept mass and a token below the row's key threshold
// has p = 0 (log p = -inf).

// A row's normaliser: max m, l2s = log2 of the (kept) mass relative to the
// max's weight (exp2(stab_of(m, c)) on softmax rows, exp2(m c) on truncated
// rows, as log2_prob reads it), and the key threshold (0 keeps every token).
struct RowNorm {
    float m, l2s;
    uint32_t tau;
};

// The normalisers of target row rt and, when has_d, draft row rd, with the
// two rows' loads issued together: their truncation summaries (TRUNC), or
// each batch of their slice partials.  Without has_d, d is left as no row.
// TRUNC is a template parameter so that neither form's loads share a branch
// join with the other's (which would make the compiler wait for both).
template <bool TRUNC>
__device__ __forceinline__ void row_norms(const DecideSampleArgs& a, long long rt, long long rd, bool has_d,
                                          RowNorm& t, RowNorm& d)
{
    const long long rd_ = has_d ? rd : rt;         // a valid row either way
    d = RowNorm{-INFINITY, -INFINITY, 0u};
    if constexpr (TRUNC) {
        const TruncRow tt = a.trunc[rt];
        const TruncRow td = a.trunc[rd_];
        t = RowNorm{tt.m, tt.l2s, tt.tau};
        if (has_d) d = RowNorm{td.m, td.l2s, td.tau};
        return;
    }
    const SoftPartial* pt = a.partials + rt * a.splits;
    const SoftPartial* pd = a.partials + rd_ * a.splits;
    float mt = -INFINITY, st = 0.f, md = -INFINITY, sd = 0.f;
    for (int i0 = 0; i0 < a.splits; i0 += kSoftBatch) {
        SoftPartial qt[kSoftBatch], qd[kSoftBatch];
        load_soft_batch(pt, i0, a.splits, qt);
        load_soft_batch(pd, i0, a.splits, qd);
        const int n = min(kSoftBatch, a.splits - i0);
        merge_soft_batch(qt, n, a.c, mt, st);
        merge_soft_batch(qd, n, a.c, md, sd);
    }
    t = RowNorm{mt, log2f(st), 0u};
    if (has_d) d = RowNorm{md, log2f(sd), 0u};
}

// log2 of a token's probability, in the form its row's mass was summed in:
// exp2((z - m) c) on truncated rows (the truncation kernel's weights),
// exp2(z c - h) with h = stab_of(m, c) on softmax rows (the statistics
// kernel's terms), so that the rounding of h cancels against the mass's.
__device__ __forceinline__ float log2_prob(float z, const RowNorm& r, float c, bool trunc)
{
    return (trunc ? (z - r.m) * c : __builtin_fmaf(z, c, -stab_of(r.m, c))) - r.l2s;
}

// The statistics of target row (b, pos) and, for pos < k, the decision at pos.
struct PosSample {
    RowNorm t, d;
    float px, qx;
    int x;
    bool reject;
};

template <int DT, bool TRUNC>
__device__ __forceinline__ PosSample sample_position(const DecideSampleArgs& a, int b, int pos)
{
    constexpr int ES = DT == DT_F32 ? 4 : 2;
    const int k = a.k;
    const float c = a.c;
    PosSample r;
    r.d = RowNorm{-INFINITY, -INFINITY, 0u};
    r.px = 0.f;
    r.qx = 0.f;
    r.x = -1;
    r.reject = false;
    const int tr = b * (k + 1) + pos;
    const int dr = b * k + pos;
    const bool has_d = pos < k;
    // the loads that depend on nothing go first: the draft token and its
    // uniform, then both rows' statistics; only the gathers wait for them
    const int pc = has_d ? pos : k - 1;            // unconditional loads (no branch to join)
    const int xl = a.tokens[(long long)b * k + pc];
    const float u = a.uniforms[(long long)b * (k + 1) + pc];
    const int x = has_d ? xl : -1;
    row_norms<TRUNC>(a, tr, (long long)a.B * (k + 1) + dr, has_d, r.t, r.d);
    if (has_d) {
        r.x = x;
        const bool valid = r.x >= 0 && r.x < a.V;
        if (valid) {
            const float zx = load_elem<DT>(row_ptr(a.target, tr, a.t_stride, ES), r.x);
            const float yx = load_elem<DT>(row_ptr(a.draft, dr, a.d_stride, ES), r.x);
            const float lp = key_of<DT>(zx) >= r.t.tau ? log2_prob(zx, r.t, c, TRUNC) : -INFINITY;
            const float lq = key_of<DT>(yx) >= r.d.tau ? log2_prob(yx, r.d, c, TRUNC) : -INFINITY;
            const float lpl = lp + a.log2_lenience;
            const bool accept = (lq <= lpl) || (u < exp2f(lpl - lq));
            r.reject = !accept;
            r.px = exp2f(lp);
            r.qx = exp2f(lq);
        } else {
            r.reject = true;
        }
    }
    return r;
}

// The round's one draw: the residual against draft row j, or the bonus row k.
__device__ __forceinline__ void write_desc(const DecideSampleArgs& a, int b, int j, const PosSample& r)
{
    const int k = a.k;
    SampleDesc d;
    d.t_row = b * (k + 1) + j;
    d.d_row = j < k ? b * k + j : -1;
    d.out_pos = j;
    d.kind = j < k ? 0 : 1;
    d.m_t = r.t.m;
    d.m_d = j < k ? r.d.m : 0.f;
    d.kq = j < k ? exp2f(r.t.l2s - r.d.l2s) : 0.f;
    d.u = a.uniforms[(long long)b * (k + 1) + k];
    d.tau_t = r.t.tau;
    d.tau_d = j < k ? r.d.tau : 0u;
    a.desc[b] = d;
    a.out_num_accepted[b] = j;
}

template <int DT, bool TRUNC>
__global__ __launch_bounds__(kBlock) void k_decide_sample(DecideSampleArgs a)
{
    const int b = blockIdx.x * kSeqPerBlock + (threadIdx.x >> 6);
    if (b >= a.B) return;
    const int lane = threadIdx.x & 63;
    const int k = a.k;
    PosSample r{};
    if (lane <= k) r = sample_position<DT, TRUNC>(a, b, lane);
    const unsigned long long rej = ballot64(lane < k && r.reject);
    const int j = rej ? (__ffsll((long long)rej) - 1) : k;

    int* out = a.out_tokens + (long long)b * (k + 1);
    if (lane < j) out[lane] = r.x;
    else if (lane > j && lane <= k) out[lane] = -1;
    if (lane < k) {
        if (a.out_p_x) a.out_p_x[(long long)b * k + lane] = r.px;
        if (a.out_q_x) a.out_q_x[(long long)b * k + lane] = r.qx;
    }
    if (lane == j) write_desc(a, b, j, r);
}

// Early exit: lane i takes position w0 + i of window [w0, w1).  A rejection
// inside the window (or reaching position k) finishes the sequence exactly as
// k_decide_sample would; otherwise its accepted drafts are written and it
// moves on to the next window.
template <int DT>
__global__ __launch_bounds__(kBlock) void k_lazy_decide_sample(LazyArgs l, DecideSampleArgs a)
{
    const int li = blockIdx.x * kSeqPerBlock + (threadIdx.x >> 6);
    const int count = l.list_in ? min(*l.count_in, a.B) : a.B;
    if (li >= count) return;
    const int b = l.list_in ? l.list_in[li] : li;
    if (b < 0 || b >= a.B) return;
    const int lane = threadIdx.x & 63;
    const int k = a.k;
    const int pos = l.w0 + lane;
    const bool in = pos < l.w1;
    PosSample r{};
    if (in) r = sample_position<DT, false>(a, b, pos);      // early exit runs without truncation
    const unsigned long long rej = ballot64(in && pos < k && r.reject);
    int j = -1;
    if (rej) j = l.w0 + __ffsll((long long)rej) - 1;
    else if (l.w1 == k + 1) j = k;
    int* out = a.out_tokens + (long long)b * (k + 1);
    if (in && pos < k && (j < 0 || pos < j)) out[pos] = r.x;
    if (j >= 0) {
        if (pos == j) write_desc(a, b, j, r);
        if (lane > j && lane <= k) out[lane] = -1;
    } else if (lane == 0) {
        const int slot = atomicAdd(l.count_out, 1);
        l.list_out[slot] = b;
    }
}

// ---- greedy ----------------------------------------------------------------
__global__ __launch_bounds__(kBlock) void k_decide_greedy(DecideGreedyArgs a)
{
    const int b = blockIdx.x * kSeqPerBlock + (threadIdx.x >> 6);
    if (b >= a.B) return;
    const int lane = threadIdx.x & 63;
    const int k = a.k;
    // the token's load first (clamped, unconditional), so it overlaps the partials'
    const int xl = a.tokens[(long long)b * k + min(lane, k - 1)];
    int amax = 0, x = -1;
    bool miss = false;
    if (lane <= k) amax = merge_arg(a.partials + (long long)(b * (k + 1) + lane) * a.splits, a.splits);
    if (lane < k) {
        x = xl;
        miss = x != amax;
    }
    const unsigned long long mm = ballot64(miss);
    const int j = mm ? (__ffsll((long long)mm) - 1) : k;
    if (lane <= k) {
        int* out = a.out_tokens + (long long)b * (k + 1);
        out[lane] = lane < j ? x : (lane == j ? amax : -1);
        if (a.out_argmax) a.out_argmax[(long long)b * (k + 1) + lane] = amax;
    }
    // by-products for phrase harvesting (Ouroboros 3.4.4, Eq. 10): matches
    // anywhere among the k drafts, not only in the accepted prefix
    const unsigned long long match = ballot64(lane < k && !miss);
    if (lane == 0) {
        a.out_num_accepted[b] = j;
        if (a.out_match_mask) a.out_match_mask[b] = match;
        if (a.out_num_match) a.out_num_match[b] = __popcll(match);
    }
}

__global__ __launch_bounds__(kBlock) void k_lazy_decide_greedy(LazyArgs l, DecideGreedyArgs a)
{
    const int li = blockIdx.x * kSeqPerBlock + (threadIdx.x >> 6);
    const int count = l.list_in ? min(*l.count_in, a.B) : a.B;
    if (li >= count) return;
    const int b = l.list_in ? l.list_in[li] : li;
    if (b < 0 || b >= a.B) return;
    const int lane = threadIdx.x & 63;
    const int k = a.k;
    const int pos = l.w0 + lane;
    const bool in = pos < l.w1;
    const int xl = a.tokens[(long long)b * k + min(pos, k - 1)];   // overlaps the partials' loads
    int amax = 0, x = -1;
    bool miss = false;
    if (in) {
        amax = merge_arg(a.partials + (long long)(b * (k + 1) + pos) * a.splits, a.splits);
        if (pos < k) {
            x = xl;
            miss = x != amax;
        }
    }
    const unsigned long long mm = ballot64(in && pos < k && miss);
    int j = -1;
    if (mm) j = l.w0 + __ffsll((long long)mm) - 1;
    else if (l.w1 == k + 1) j = k;
    int* out = a.out_tokens + (long long)b * (k + 1);
    if (in && pos < k && (j < 0 || pos < j)) out[pos] = x;
    if (j >= 0) {
        if (pos == j) {
            out[pos] = amax;
            a.out_num_accepted[b] = j;
        }
        if (lane > j && lane <= k) out[lane] = -1;
    } else if (lane == 0) {
        const int slot = atomicAdd(l.count_out, 1);
        l.list_out[slot] = b;
    }
}

// ---- multi-candidate greedy ------------------------------------------------
// Lane c*L + i holds candidate c's position i (C*L <= 64).  Candidate c's
// accepted length is the index of its first mismatch bit; the longest wins,
// ties to the lowest c (Ouroboros 3.4.3, "Selecting the accepted tokens").
// Flat layout: row (c, i) of sequence b is row (b*C + c)*R + i.  Tree layout
// (Ouroboros Figure 3, each node scored once): the row is b*N + cand_rows[b][c][i];
// an index outside [0, N) is never read: cand_argmax gives -1 for it, which the
// decision counts as a mismatch whatever the token (a -1 padding token included),
// and -1 is also its correction.
__device__ __forceinline__ int cand_argmax(const DecideCandArgs& a, int b, int c, int i)
{
    long long row;
    if (a.cand_rows) {
        const int r = a.cand_rows[((long long)b * a.C + c) * a.R + i];
        if (r < 0 || r >= a.N) return -1;
        row = (long long)b * a.N + r;
    } else {
        row = ((long long)b * a.C + c) * a.R + i;
    }
    return merge_arg(a.partials + row * a.splits, a.splits);
}

__global__ __launch_bounds__(kBlock) void k_decide_candidates(DecideCandArgs a)
{
    const int b = blockIdx.x * kSeqPerBlock + (threadIdx.x >> 6);
    if (b >= a.B) return;
    const int lane = threadIdx.x & 63;
    const int C = a.C, L = a.L, R = a.R;
    const bool active = lane < C * L;
    const int c = active ? lane / L : 0;
    const int i = active ? lane - c * L : 0;
    int amax = 0, tok = -1;
    bool miss = false;
    if (active) {
        amax = cand_argmax(a, b, c, i);
        tok = a.cand[((long long)b * C + c) * L + i];
        miss = amax < 0 || tok != amax;
    }
    const unsigned long long mm = ballot64(miss);
    int acc = 0;
    if (active) {
        const unsigned long long lo_mask = (L == 64) ? ~0ull : ((1ull << L) - 1ull);
        const unsigned long long bits = (mm >> (c * L)) & lo_mask;
        acc = bits ? (__ffsll((long long)bits) - 1) : L;
    }
    int A = wave_max_int(active ? acc : -1);
    const int cs = wave_min_int(active && acc == A ? c : 1 << 30);
    // committed tokens: cand(c*, 0..A-1), then the correction or the bonus row
    const int src = cs * L + (lane < L ? lane : 0);
    const int ctok = __shfl(tok, src, 64);
    const int camx = __shfl(amax, src, 64);
    int bonus = -1;
    if (A == L && R == L + 1 && lane == L) bonus = cand_argmax(a, b, cs, L);
    if (a.out_argmax) {
        if (active) a.out_argmax[((long long)b * C + c) * R + i] = amax;
        if (R == L + 1 && lane < C) a.out_argmax[((long long)b * C + lane) * R + L] = cand_argmax(a, b, lane, L);
    }
    if (lane <= L) {
        int v;
        if (lane < A) v = ctok;
        else if (lane == A && A < L) v = camx;
        else if (lane == L && A == L && R == L + 1) v = bonus;
        else v = -1;
        a.out_tokens[(long long)b * (L + 1) + lane] = v;
    }
    if (lane == 0) {
        a.out_num_accepted[b] = A;
        a.out_best[b] = cs;
    }
}

hipError_t launch_decide_sample(int dt, const DecideSampleArgs& a, hipStream_t st)
{
    void* args[] = {const_cast<DecideSampleArgs*>(&a)};
    const unsigned grid = (unsigned)((a.B + kSeqPerBlock - 1) / kSeqPerBlock);
    const bool t = a.trunc != nullptr;
    const void* f = dt == DT_F32 ? (t ? reinterpret_cast<const void*>(k_decide_sample<DT_F32, true>)
                                      : reinterpret_cast<const void*>(k_decide_sample<DT_F32, false>))
                  : dt == DT_F16 ? (t ? reinterpret_cast<const void*>(k_decide_sample<DT_F16, true>)
                                      : reinterpret_cast<const void*>(k_decide_sample<DT_F16, false>))
                                 : (t ? reinterpret_cast<const void*>(k_decide_sample<DT_BF16, true>)
                                      : reinterpret_cast<const void*>(k_decide_sample<DT_BF16, false>));
    return hipLaunchKernel(f, dim3(grid), dim3(kBlock), args, 0, st);
}

hipError_t launch_lazy_decide_sample(int dt, const LazyArgs& l, const DecideSampleArgs& a, hipStream_t st)
{
    if (a.trunc) return hipErrorInvalidValue;     // early exit has no truncated form
    void* args[] = {const_cast<LazyArgs*>(&l), const_cast<DecideSampleArgs*>(&a)};
    const unsigned grid = (unsigned)((a.B + kSeqPerBlock - 1) / kSeqPerBlock);
    const void* f = dt == DT_F32 ? reinterpret_cast<const void*>(k_lazy_decide_sample<DT_F32>)
                  : dt == DT_F16 ? reinterpret_cast<const void*>(k_lazy_decide_sample<DT_F16>)
                                 : reinterpret_cast<const void*>(k_lazy_decide_sample<DT_BF16>);
    return hipLaunchKernel(f, dim3(grid), dim3(kBlock), args, 0, st);
}

hipError_t launch_lazy_decide_greedy(const LazyArgs& l, const DecideGreedyArgs& a, hipStream_t st)
{
    void* args[] = {const_cast<LazyArgs*>(&l), const_cast<DecideGreedyArgs*>(&a)};
    const unsigned grid = (unsigned)((a.B + kSeqPerBlock - 1) / kSeqPerBlock);
    return hipLaunchKernel(reinterpret_cast<const void*>(k_lazy_decide_greedy), dim3(grid), dim3(kBlock),
                           args, 0, st);
}

hipError_t launch_decide_greedy(const DecideGreedyArgs& a, hipStream_t st)
{
    void* args[] = {const_cast<DecideGreedyArgs*>(&a)};
    const unsigned grid = (unsigned)((a.B + kSeqPerBlock - 1) / kSeqPerBlock);
    return hipLaunchKernel(reinterpret_cast<const void*>(k_decide_greedy), dim3(grid), dim3(kBlock),
                           args, 0, st);
}

hipError_t launch_decide_candidates(const DecideCandArgs& a, hipStream_t st)
{
    void* args[] = {const_cast<DecideCandArgs*>(&a)};
    const unsigned grid = (unsigned)((a.B + kSeqPerBlock - 1) / kSeqPerBlock);
    return hipLaunchKernel(reinterpret_cast<const void*>(k_decide_candidates), dim3(grid), dim3(kBlock),
                           args, 0, st);
}

}  // namespace sv
