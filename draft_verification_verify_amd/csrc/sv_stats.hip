// sv_stats.hip -- the vocabulary-streaming pass: one read of every logit row.
//
// Sampling needs, per row, the softmax normaliser of z / T (production blog,
// "The acceptance rule": p and q at every position); greedy needs the argmax
// (same section, greedy collapse).  Both are row reductions over V with no
// contraction, bound by HBM bandwidth: each 512-thread workgroup streams a
// contiguous slice of one row with 16-byte non-temporal loads (four per
// thread in flight), reduces it in registers and writes one 8-byte partial.  The
// partials of a row's slices are merged in a fixed order by the decision
// kernels.
//
// Built with -fno-honor-nans: NaN logits are outside the library's contract,
// which lets max() map to bare v_max3_f32.

#include "sv_device.h"

namespace sv {

// Online softmax statistics in base 2, relative to the stabiliser h = m c
// with m the running max and the product rounded once (stab_of):
// s = sum exp2(z c - h).  Each term is exp2(fma(z, c, -h)); a new max
// rescales s by exp2(h_old - h_new), both rounded as the terms saw them.  So
// every term of s carries the one rounding error of h, as does a
// probability formed later as exp2(fma(z, c, -h) - log2 s), and the two
// cancel: no error grows with |m c| (large logits, low temperatures), and
// each element costs one fma.  The rescale's own rounding is exact for
// nearby maxima and otherwise applies to terms scaled down by 2^-|h_old - h_new|.
// Rescales s once per group of N elements (one exp2), not per element.
template <int N>
__device__ __forceinline__ void soft_update(const float* e, float& m, float& s, float c)
{
    float cm0 = e[0], cm1 = e[1];
#pragma unroll
    for (int j = 2; j < N; j += 2) {
        cm0 = fmaxf(cm0, e[j]);
        cm1 = fmaxf(cm1, e[j + 1]);
    }
    const float mn = fmaxf(m, fmaxf(cm0, cm1));
    const float hn = stab_of(mn, c);
    const float scale = (m == mn) ? 1.f : __builtin_amdgcn_exp2f(stab_of(m, c) - hn);
    const float off = (mn == -INFINITY) ? 0.f : -hn;   // an all -inf group adds exp2(-inf) = 0
    float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
#pragma unroll
    for (int j = 0; j < N; j += 4) {
        a0 += __builtin_amdgcn_exp2f(__builtin_fmaf(e[j + 0], c, off));
        a1 += __builtin_amdgcn_exp2f(__builtin_fmaf(e[j + 1], c, off));
        a2 += __builtin_amdgcn_exp2f(__builtin_fmaf(e[j + 2], c, off));
        a3 += __builtin_amdgcn_exp2f(__builtin_fmaf(e[j + 3], c, off));
    }
    s = s * scale + ((a0 + a1) + (a2 + a3));
    m = mn;
}

__device__ __forceinline__ const char* stats_row(const StatsArgs& a, int row, int es)
{
    return row < a.n_target_rows
               ? row_ptr(a.target, row, a.t_stride, es)
               : row_ptr(a.draft, row - a.n_target_rows, a.d_stride, es);
}

constexpr int kSB = kStatsBlock;
constexpr int kSW = kStatsBlock / 64;

// A thread's last round of a slice: its vectors v + j kSB (j < 4) below
// vend, loaded together like a full round, so that no wave trails the
// others by a chain of single loads.  The loads past vend are clamped to
// vend - 1 (v < vend) and their elements read as -inf.  Returns the number
// of vectors below vend (a prefix of the four).
template <int DT, bool VEC>
__device__ __forceinline__ int last_round(const char* rp, int v, int vend, float* e)
{
    const int last = vend - 1;
    const Raw<DT> r0 = load_raw<DT, VEC>(rp, v);
    const Raw<DT> r1 = load_raw<DT, VEC>(rp, min(v + kSB, last));
    const Raw<DT> r2 = load_raw<DT, VEC>(rp, min(v + 2 * kSB, last));
    const Raw<DT> r3 = load_raw<DT, VEC>(rp, min(v + 3 * kSB, last));
    decode<DT>(r0, e);
    decode<DT>(r1, e + 8);
    decode<DT>(r2, e + 16);
    decode<DT>(r3, e + 24);
    int n = 1;
#pragma unroll
    for (int j = 1; j < 4; ++j) {
        const bool ok = v + j * kSB < vend;
        n += ok ? 1 : 0;
#pragma unroll
        for (int t = 0; t < kVec; ++t) e[kVec * j + t] = ok ? e[kVec * j + t] : -INFINITY;
    }
    return n;
}

// A thread's last (at most eight) vectors of a slice, v + j kSB (j < 8) below
// vend, all loaded before any is reduced, so that a slice of two rounds per
// thread costs one memory round trip rather than two.  They are reduced in
// two groups of four, as two rounds would be (the same groups, so the same
// result bit for bit); loads past vend are clamped to vend - 1 and read as
// -inf.  A group with nothing below vend leaves (m, s) exactly as they were
// (s * 1 + 0), so the second group is reduced without a branch, which would
// let the compiler issue its loads only after the first group's arithmetic.
template <int DT, bool VEC>
__device__ __forceinline__ void last_rounds_soft(const char* rp, int v, int vend, float c, float& m, float& s)
{
    const int last = vend - 1;
    Raw<DT> r[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) r[j] = load_raw<DT, VEC>(rp, min(v + j * kSB, last));
    __builtin_amdgcn_sched_barrier(0);             // all eight loads issue before the arithmetic
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        float e[4 * kVec];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            decode<DT>(r[4 * h + q], e + kVec * q);
            const bool ok = v + (4 * h + q) * kSB < vend;
#pragma unroll
            for (int t = 0; t < kVec; ++t) e[kVec * q + t] = ok ? e[kVec * q + t] : -INFINITY;
        }
        soft_update<4 * kVec>(e, m, s, c);
    }
}

// The thread that takes a row's partial last vector (V not a multiple of 8)
// when it falls in slice [v0, v1): the one whose vectors v0 + tid + n kSB reach it.
__device__ __forceinline__ bool takes_partial(int v0, int v1, int nfull)
{
    return nfull < v1 && (nfull - v0) % kSB == (int)threadIdx.x;
}

// (max, sum of exp2) of logical vectors [v0, v1) of one row, reduced over the
// 512-thread workgroup in a fixed order; thread 0 holds the result.  Called
// by every thread of the workgroup.
template <int DT, bool VEC>
__device__ __forceinline__ SoftPartial slice_softmax(const char* rp, int v0, int v1, int V, float c,
                                                     float* lds_m, float* lds_s)
{
    const int nfull = V >> 3;
    const int vend = min(v1, nfull);
    float m = -INFINITY, s = 0.f;
    int v = v0 + (int)threadIdx.x;
    for (; v + 8 * kSB < vend; v += 4 * kSB) {   // while more than eight vectors remain per thread
        Raw<DT> r0 = load_raw<DT, VEC>(rp, v);
        Raw<DT> r1 = load_raw<DT, VEC>(rp, v + kSB);
        Raw<DT> r2 = load_raw<DT, VEC>(rp, v + 2 * kSB);
        Raw<DT> r3 = load_raw<DT, VEC>(rp, v + 3 * kSB);
        float e[4 * kVec];
        decode<DT>(r0, e);
        decode<DT>(r1, e + 8);
        decode<DT>(r2, e + 16);
        decode<DT>(r3, e + 24);
        soft_update<4 * kVec>(e, m, s, c);
    }
    // at most eight vectors left per thread: more than four (for thread 0,
    // which has the most) are loaded together; four or fewer as one round
    if (vend - (v - (int)threadIdx.x) > 4 * kSB) {
        last_rounds_soft<DT, VEC>(rp, v, vend, c, m, s);
    } else if (v < vend) {
        float e[4 * kVec];
        last_round<DT, VEC>(rp, v, vend, e);
        soft_update<4 * kVec>(e, m, s, c);
    }
    if (takes_partial(v0, v1, nfull)) {    // the row's partial last vector
        float e[kVec];
        load_partial<DT>(rp, nfull, V - 8 * nfull, -INFINITY, e);
        soft_update<kVec>(e, m, s, c);
    }

    // Merging: the wave's max first (exact in any order), then every lane's
    // sum rescaled to it, exp2(stab(m) - stab(max)) with the same rounded
    // stabilisers as the terms, and summed in a fixed order; the workgroup's
    // eight wave results the same way.  One exp2 per lane instead of one per
    // pairwise merge.  A lane or wave without a finite element holds s = 0.
    const float wm = wave_max(m);
    const float ws = wave_sum_f(wm == -INFINITY ? 0.f : s * __builtin_amdgcn_exp2f(stab_of(m, c) - stab_of(wm, c)));
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    if (lane == 0) {
        lds_m[w] = wm;
        lds_s[w] = ws;
    }
    __syncthreads();
    float M = -INFINITY, S = 0.f;
    if (threadIdx.x == 0) {
#pragma unroll
        for (int i = 0; i < kSW; ++i) M = fmaxf(M, lds_m[i]);
        if (M != -INFINITY) {
            const float hM = stab_of(M, c);
#pragma unroll
            for (int i = 0; i < kSW; ++i) S += lds_s[i] * __builtin_amdgcn_exp2f(stab_of(lds_m[i], c) - hM);
        }
    }
    __syncthreads();                   // the LDS slots may be reused by the caller
    return SoftPartial{M, S};
}

// Argmax with the lowest index among equal maxima over logical vectors
// [v0, v1) of one row.  Each thread keeps the largest value it has seen and
// the first group of vectors where it appeared (strictly-greater updates keep
// the first occurrence, in ascending index order within the thread).  After
// the block maximum M is known, only the threads holding M reload that one
// group to locate their first index of M; the block takes the smallest.
// -0.0 and +0.0 compare equal throughout.  Called by every thread.
template <int DT, bool VEC>
__device__ __forceinline__ ArgPartial slice_argmax(const char* rp, int v0, int v1, int V,
                                                   float* lds_f, int* lds_i)
{
    const int nfull = V >> 3;
    const int vend = min(v1, nfull);
    float bv = -INFINITY;
    int bvec = -1, bcnt = 0;
    int v = v0 + (int)threadIdx.x;
    for (; v + 3 * kSB < vend; v += 4 * kSB) {
        Raw<DT> r0 = load_raw<DT, VEC>(rp, v);
        Raw<DT> r1 = load_raw<DT, VEC>(rp, v + kSB);
        Raw<DT> r2 = load_raw<DT, VEC>(rp, v + 2 * kSB);
        Raw<DT> r3 = load_raw<DT, VEC>(rp, v + 3 * kSB);
        float e[4 * kVec];
        decode<DT>(r0, e);
        decode<DT>(r1, e + 8);
        decode<DT>(r2, e + 16);
        decode<DT>(r3, e + 24);
        float cm0 = e[0], cm1 = e[1];
#pragma unroll
        for (int j = 2; j < 4 * kVec; j += 2) {
            cm0 = fmaxf(cm0, e[j]);
            cm1 = fmaxf(cm1, e[j + 1]);
        }
        const float cm = fmaxf(cm0, cm1);
        const bool up = cm > bv;
        bv = up ? cm : bv;
        bvec = up ? v : bvec;
        bcnt = up ? 4 : bcnt;
    }
    if (v < vend) {
        float e[4 * kVec];
        const int n = last_round<DT, VEC>(rp, v, vend, e);
        float cm0 = e[0], cm1 = e[1];
#pragma unroll
        for (int j = 2; j < 4 * kVec; j += 2) {
            cm0 = fmaxf(cm0, e[j]);
            cm1 = fmaxf(cm1, e[j + 1]);
        }
        const float cm = fmaxf(cm0, cm1);
        const bool up = cm > bv;
        bv = up ? cm : bv;
        bvec = up ? v : bvec;
        bcnt = up ? n : bcnt;
    }
    if (takes_partial(v0, v1, nfull)) {
        float e[kVec];
        load_partial<DT>(rp, nfull, V - 8 * nfull, -INFINITY, e);
        float cm = e[0];
#pragma unroll
        for (int j = 1; j < kVec; ++j) cm = fmaxf(cm, e[j]);
        if (cm > bv) {
            bv = cm;
            bvec = nfull;
            bcnt = 1;
        }
    }

    const float M = block_max<kSW>(bv, lds_f);
    int idx = INT32_MAX;
    if (bv == M && M > -INFINITY) {
        for (int j = 0; j < bcnt && idx == INT32_MAX; ++j) {
            const int vv = bvec + j * kSB;
            float e[kVec];
            load8<DT, VEC>(rp, vv, nfull, V, -INFINITY, e);
#pragma unroll
            for (int t = kVec - 1; t >= 0; --t)
                if (e[t] == M) idx = 8 * vv + t;
        }
    }
    idx = block_min_int<kSW>(idx, lds_i);
    return ArgPartial{M, idx};
}

template <int DT, bool VEC>
__global__ __launch_bounds__(kStatsBlock) void k_softmax_stats(StatsArgs a)
{
    __shared__ float lds_m[kSW], lds_s[kSW];
    constexpr int ES = DT == DT_F32 ? 4 : 2;
    const int unit = blockIdx.x;
    const int row = unit / a.splits;
    const int split = unit - row * a.splits;
    const int v0 = split * a.vec_per_split;
    const int v1 = min(v0 + a.vec_per_split, a.nvec);
    if (unit == 0)
        for (int i = (int)threadIdx.x; i < a.n_zero; i += kStatsBlock) a.zero[i] = 0;
    const SoftPartial r = slice_softmax<DT, VEC>(stats_row(a, row, ES), v0, v1, a.V, a.c, lds_m, lds_s);
    if (threadIdx.x == 0) reinterpret_cast<SoftPartial*>(a.partials)[unit] = r;
}

template <int DT, bool VEC>
__global__ __launch_bounds__(kStatsBlock) void k_argmax_stats(StatsArgs a)
{
    __shared__ float lds_f[kSW];
    __shared__ int lds_i[kSW];
    constexpr int ES = DT == DT_F32 ? 4 : 2;
    const int unit = blockIdx.x;
    const int row = unit / a.splits;
    const int split = unit - row * a.splits;
    const int v0 = split * a.vec_per_split;
    const int v1 = min(v0 + a.vec_per_split, a.nvec);
    const ArgPartial r = slice_argmax<DT, VEC>(stats_row(a, row, ES), v0, v1, a.V, lds_f, lds_i);
    if (threadIdx.x == 0) reinterpret_cast<ArgPartial*>(a.partials)[unit] = r;
}

// Early-exit statistics: the rows of window [w0, w1) of every listed
// sequence, one (row, slice) unit at a time in a workgroup-strided loop (the
// grid is sized for the worst case and workgroups past the live units exit).
// Row and slice numbering is the full pass's, so partials match it bit for bit.
template <int DT, bool VEC, bool SOFT>
__global__ __launch_bounds__(kStatsBlock) void k_lazy_stats(LazyArgs a)
{
    __shared__ float lds_f[kSW], lds_s[kSW];
    __shared__ int lds_i[kSW];
    constexpr int ES = DT == DT_F32 ? 4 : 2;
    if (blockIdx.x == 0 && threadIdx.x == 0 && a.count_clear) *a.count_clear = 0;
    const int count = a.list_in ? min(*a.count_in, a.B) : a.B;
    const int nt = a.w1 - a.w0;
    const int nd = a.draft ? max(0, min(a.w1, a.k) - a.w0) : 0;
    const int per_seq = (nt + nd) * a.splits;
    const long long n_units = (long long)count * per_seq;
    for (long long u = blockIdx.x; u < n_units; u += gridDim.x) {
        const int li = (int)(u / per_seq);
        const int rem = (int)(u - (long long)li * per_seq);
        const int r = rem / a.splits;
        const int split = rem - r * a.splits;
        const int b = a.list_in ? a.list_in[li] : li;
        if (b < 0 || b >= a.B) continue;         // uniform across the workgroup
        long long row;
        const char* rp;
        if (r < nt) {
            row = (long long)b * (a.k + 1) + a.w0 + r;
            rp = row_ptr(a.target, row, a.t_stride, ES);
        } else {
            const long long drow = (long long)b * a.k + a.w0 + (r - nt);
            row = a.n_target_rows + drow;
            rp = row_ptr(a.draft, drow, a.d_stride, ES);
        }
        const int v0 = split * a.vec_per_split;
        const int v1 = min(v0 + a.vec_per_split, a.nvec);
        if constexpr (SOFT) {
            const SoftPartial p = slice_softmax<DT, VEC>(rp, v0, v1, a.V, a.c, lds_f, lds_s);
            if (threadIdx.x == 0) reinterpret_cast<SoftPartial*>(a.partials)[row * a.splits + split] = p;
        } else {
            const ArgPartial p = slice_argmax<DT, VEC>(rp, v0, v1, a.V, lds_f, lds_i);
            if (threadIdx.x == 0) reinterpret_cast<ArgPartial*>(a.partials)[row * a.splits + split] = p;
        }
    }
}

template <int DT, bool VEC>
static hipError_t launch_lazy_dt(bool soft, int grid, const LazyArgs& a, hipStream_t st)
{
    void* args[] = {const_cast<LazyArgs*>(&a)};
    const void* f = soft ? reinterpret_cast<const void*>(k_lazy_stats<DT, VEC, true>)
                         : reinterpret_cast<const void*>(k_lazy_stats<DT, VEC, false>);
    return hipLaunchKernel(f, dim3((unsigned)grid), dim3(kStatsBlock), args, 0, st);
}

hipError_t launch_lazy_stats(int dt, bool vec, bool soft, int grid, const LazyArgs& a, hipStream_t st)
{
    switch (dt) {
    case DT_F32: return vec ? launch_lazy_dt<DT_F32, true>(soft, grid, a, st) : launch_lazy_dt<DT_F32, false>(soft, grid, a, st);
    case DT_F16: return vec ? launch_lazy_dt<DT_F16, true>(soft, grid, a, st) : launch_lazy_dt<DT_F16, false>(soft, grid, a, st);
    default:     return vec ? launch_lazy_dt<DT_BF16, true>(soft, grid, a, st) : launch_lazy_dt<DT_BF16, false>(soft, grid, a, st);
    }
}

template <typename K>
static hipError_t launch_rows(K kernel, const StatsArgs& a, hipStream_t st)
{
    void* args[] = {const_cast<StatsArgs*>(&a)};
    const unsigned grid = (unsigned)((long long)a.n_rows * a.splits);
    return hipLaunchKernel(reinterpret_cast<const void*>(kernel), dim3(grid), dim3(kStatsBlock), args, 0, st);
}

hipError_t launch_softmax_stats(int dt, bool vec, const StatsArgs& a, hipStream_t st)
{
    switch (dt) {
    case DT_F32: return vec ? launch_rows(k_softmax_stats<DT_F32, true>, a, st)
                            : launch_rows(k_softmax_stats<DT_F32, false>, a, st);
    case DT_F16: return vec ? launch_rows(k_softmax_stats<DT_F16, true>, a, st)
                            : launch_rows(k_softmax_stats<DT_F16, false>, a, st);
    default:     return vec ? launch_rows(k_softmax_stats<DT_BF16, true>, a, st)
                            : launch_rows(k_softmax_stats<DT_BF16, false>, a, st);
    }
}

hipError_t launch_argmax_stats(int dt, bool vec, const StatsArgs& a, hipStream_t st)
{
    switch (dt) {
    case DT_F32: return vec ? launch_rows(k_argmax_stats<DT_F32, true>, a, st)
                            : launch_rows(k_argmax_stats<DT_F32, false>, a, st);
    case DT_F16: return vec ? launch_rows(k_argmax_stats<DT_F16, true>, a, st)
                            : launch_rows(k_argmax_stats<DT_F16, false>, a, st);
    default:     return vec ? launch_rows(k_argmax_stats<DT_BF16, true>, a, st)
                            : launch_rows(k_argmax_stats<DT_BF16, false>, a, st);
    }
}

}  // namespace sv
