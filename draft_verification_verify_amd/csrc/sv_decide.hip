// sv_decide.hip -- per-sequence decisions, one wave64 per sequence: the
// greedy rule (lane i compares draft i with its row's argmax), the
// multi-candidate selection, and the early-exit windows of both rules (the
// sampling rule itself is in sv_rule.h).  A 64-bit ballot plus a
// find-first-set gives the first rejection: the left-to-right scan of the
// rule (production blog, "The acceptance rule") without a serial loop.

#include "sv_rule.h"

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

// The decision of every sequence, one wave each, before a separate chunk pass.
template <int DT, bool TRUNC>
__global__ __launch_bounds__(kBlock) void k_decide_sample(DecideSampleArgs a)
{
    const int b = blockIdx.x * kSeqPerBlock + (threadIdx.x >> 6);
    if (b >= a.B) return;
    SampleDesc d;
    decide_sequence<DT, TRUNC>(a, b, true, &d);
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
