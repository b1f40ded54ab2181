// sv_rule.h -- the acceptance rule for one sequence, decided by one wave64:
// lane i takes draft position i (k <= 63, so the k+1 positions fit one wave),
// merges its rows' statistics in a fixed order and takes its own
// accept/reject decision; a 64-bit ballot plus find-first-set gives the first
// rejection, the left-to-right scan of the rule (production blog, "The
// acceptance rule") without a serial loop.  Shared by the early-exit decision
// kernel (sv_decide.hip) and the pass that decides and streams the draw's
// row in one launch (sv_sample.hip).
#pragma once

#include "sv_device.h"

namespace sv {

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
__device__ __forceinline__ SampleDesc make_desc(const DecideSampleArgs& a, int b, int j, const PosSample& r)
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
    return d;
}

__device__ __forceinline__ void write_desc(const DecideSampleArgs& a, int b, int j, const PosSample& r)
{
    a.desc[b] = make_desc(a, b, j, r);
    a.out_num_accepted[b] = j;
}

// The decision of sequence b by one wave64, lane i taking position i: every
// lane decides its own position, and a ballot plus find-first-set gives the
// first rejection j (k if none).  With `write`, the round's outputs: the
// accepted drafts, -1 after position j, p_i(x_i) and q_i(x_i) if requested,
// the accepted count and the draw's descriptor.  Returns j, and in *desc, on
// lane j, the draw's descriptor.
template <int DT, bool TRUNC>
__device__ __forceinline__ int decide_sequence(const DecideSampleArgs& a, int b, bool write, SampleDesc* desc)
{
    const int lane = threadIdx.x & 63;
    const int k = a.k;
    PosSample r{};
    if (lane <= k) r = sample_position<DT, TRUNC>(a, b, lane);
    const unsigned long long rej = ballot64(lane < k && r.reject);
    const int j = rej ? (__ffsll((long long)rej) - 1) : k;
    if (write) {
        int* out = a.out_tokens + (long long)b * (k + 1);
        if (lane < j) out[lane] = r.x;
        else if (lane > j && lane <= k) out[lane] = -1;
        if (lane < k) {
            if (a.out_p_x) a.out_p_x[(long long)b * k + lane] = r.px;
            if (a.out_q_x) a.out_q_x[(long long)b * k + lane] = r.qx;
        }
        if (lane == j) write_desc(a, b, j, r);
    }
    if (lane == j) *desc = make_desc(a, b, j, r);
    return j;
}

}  // namespace sv
