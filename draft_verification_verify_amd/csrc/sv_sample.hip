// sv_sample.hip -- the round's single draw, on the one selected row per sequence.
//
// After a rejection at position j the replacement is drawn from the residual
// max(0, p_j - q_j) normalised; after a full acceptance the bonus is drawn
// from p_k (production blog, "The acceptance rule"; Cascade Speculative
// Drafting, review function).  The draw is an inverse CDF over the vocabulary
// in ascending index order: the smallest token whose cumulative weight
// exceeds u times the total.
//
// Two launches, so that no workgroup waits on another inside a launch:
//  - k_decide_chunks decides the round (every workgroup of a sequence decides
//    it alike) and streams the sampled row (pair) of every sequence once,
//    writing the total weight of each chunk (a whole number of rounds of
//    kBlock logical vectors), several rounds' loads in flight per thread;
//    after a separate decision (large batches, early exit), k_sample_chunks
//    does the same from its descriptors;
//  - k_sample_pick, one workgroup per sequence, accumulates the chunk totals
//    in chunk order, finds the chunk where u * total is crossed, rescans only
//    that chunk and resolves the token with a workgroup prefix scan.
// A chunk pass of at most 128 workgroups makes the draw itself instead, in
// the last workgroup of each sequence to finish (k_decide_chunks, PICK).
// A round's total is the same block scan in both kernels and a chunk's total
// is the sequential sum of its rounds' totals, so the two kernels agree bit
// for bit; every reduction runs in a fixed order, so draws are deterministic.

#include "sv_rule.h"

namespace sv {

// The weight arithmetic, shared by every pass, in units of the target row's
// mass s_t (the draw divides by the total): p~ = s_t p, and for kind 0 the
// residual max(0, p~ - kq q~) = s_t max(0, p - q), with each exponent in the
// form its row's mass was summed in (h = stab_of(m, c) on softmax rows,
// z - m on truncated rows).  MASK: the rows are truncated, and a logit whose
// key is below its row's threshold has probability 0.
template <int DT, bool MASK>
__device__ __forceinline__ float weight_of(float ez, float ey, int kind, float c, float h_t, float h_d,
                                           const SampleDesc& d)
{
    float p = __builtin_amdgcn_exp2f(MASK ? (ez - d.m_t) * c : __builtin_fmaf(ez, c, -h_t));
    if (MASK && key_of<DT>(ez) < d.tau_t) p = 0.f;
    if (kind != 0) return p;
    float q = __builtin_amdgcn_exp2f(MASK ? (ey - d.m_d) * c : __builtin_fmaf(ey, c, -h_d));
    if (MASK && key_of<DT>(ey) < d.tau_d) q = 0.f;
    return fmaxf(__builtin_fmaf(-d.kq, q, p), 0.f);
}

// Weights of logical vector v (0 past the row's end).
template <int DT, bool VEC, bool MASK>
__device__ __forceinline__ void weights8(const char* zr, const char* yr, int v, int nfull, int V,
                                         int kind, float c, const SampleDesc& d, float* w)
{
    float ez[kVec], ey[kVec];
    load8<DT, VEC>(zr, v, nfull, V, -INFINITY, ez);
    if (kind == 0) load8<DT, VEC>(yr, v, nfull, V, -INFINITY, ey);
#pragma unroll
    for (int j = 0; j < kVec; ++j)
        w[j] = weight_of<DT, MASK>(ez[j], kind == 0 ? ey[j] : 0.f, kind, c, stab_of(d.m_t, c),
                                   stab_of(d.m_d, c), d);
}

__device__ __forceinline__ float sum8(const float* w)
{
    float ts = 0.f;
#pragma unroll
    for (int j = 0; j < kVec; ++j) ts += w[j];
    return ts;
}

// Total weight of chunk [c0, c1), one round (kBlock vectors) at a time.
template <int DT, bool VEC, bool MASK>
__device__ float chunk_total(const SampleArgs& a, const char* zr, const char* yr, int kind,
                             const SampleDesc& d, int c0, int c1, float* lds)
{
    const int nfull = a.V >> 3;
    float total = 0.f;
    for (int r0 = c0; r0 < c1; r0 += kBlock) {
        const int v = r0 + (int)threadIdx.x;
        float ts = 0.f;
        if (v < c1) {
            float w[kVec];
            weights8<DT, VEC, MASK>(zr, yr, v, nfull, a.V, kind, a.c, d, w);
            ts = sum8(w);
        }
        float ex, rt;
        block_scan(ts, &ex, &rt, lds);
        total += rt;
    }
    return total;
}

// Inverse CDF inside chunk [c0, c1) at threshold rem (relative to the chunk
// start).  Rounds of kBlock vectors are scanned in order; in the round where
// the running total first exceeds rem, the first thread whose inclusive prefix
// exceeds it walks its 8 weights.  Always returns a token of positive weight
// when the chunk has one: if rounding leaves no crossing, the chunk's last
// positive token; if the crossing thread holds no positive weight, the
// nearest positive token of the round before it, else after it.  Returns -1
// only for a chunk without positive weight.
template <int DT, bool VEC, bool MASK>
__device__ int chunk_pick(const SampleArgs& a, const char* zr, const char* yr, int kind,
                          const SampleDesc& d, int c0, int c1, float rem,
                          float* lds, int* ilds)
{
    const int nfull = a.V >> 3;
    const int vfull = min(c1, nfull);
    float R = 0.f;
    int last_tok = -1;
    // a round's full vectors are loaded while the round before it is scanned
    Raw<DT> nz, ny;
    auto issue = [&](int r0) {
        const int v = r0 + (int)threadIdx.x;
        if (v < vfull) {
            nz = load_raw<DT, VEC>(zr, v);
            if (kind == 0) ny = load_raw<DT, VEC>(yr, v);
        }
    };
    issue(c0);
    for (int r0 = c0; r0 < c1; r0 += kBlock) {
        const int v = r0 + (int)threadIdx.x;
        const Raw<DT> cz = nz, cy = ny;
        if (r0 + kBlock < c1) issue(r0 + kBlock);
        float w[kVec];
        float ts = 0.f;
        int firstpos = -1, lastpos = -1;
        if (v < c1) {
            float ez[kVec], ey[kVec];
            if (v < nfull) {
                decode<DT>(cz, ez);
                if (kind == 0) decode<DT>(cy, ey);
            } else {
                load_partial<DT>(zr, v, a.V - 8 * v, -INFINITY, ez);
                if (kind == 0) load_partial<DT>(yr, v, a.V - 8 * v, -INFINITY, ey);
            }
#pragma unroll
            for (int j = 0; j < kVec; ++j)
                w[j] = weight_of<DT, MASK>(ez[j], kind == 0 ? ey[j] : 0.f, kind, a.c, stab_of(d.m_t, a.c),
                                           stab_of(d.m_d, a.c), d);
#pragma unroll
            for (int j = 0; j < kVec; ++j) {
                ts += w[j];
                if (w[j] > 0.f) {
                    lastpos = j;
                    if (firstpos < 0) firstpos = j;
                }
            }
        } else {
#pragma unroll
            for (int j = 0; j < kVec; ++j) w[j] = 0.f;
        }
        float ex, rt;
        const float in = block_scan(ts, &ex, &rt, lds);
        const int round_last = block_max_int(lastpos >= 0 ? 8 * v + lastpos : -1, ilds);
        const float Rn = R + rt;
        if (Rn > rem) {
            const float rr = rem - R;
            const int tfirst = block_min_int(in > rr ? (int)threadIdx.x : INT32_MAX, ilds);
            int pick = -1;
            if ((int)threadIdx.x == tfirst) {
                float acc = ex;
                for (int j = 0; j < kVec; ++j) {
                    acc += w[j];
                    if (acc > rr && w[j] > 0.f) {
                        pick = j;
                        break;
                    }
                }
                if (pick < 0) pick = lastpos;
                if (pick >= 0) pick += 8 * v;
            }
            int tok = block_max_int(pick, ilds);
            if (tok < 0) {
                const int t0 = tfirst == INT32_MAX ? kBlock : tfirst;
                const int before = ((int)threadIdx.x < t0 && lastpos >= 0) ? 8 * v + lastpos : -1;
                tok = block_max_int(before, ilds);
                if (tok < 0) {
                    const int after =
                        ((int)threadIdx.x > t0 && firstpos >= 0) ? 8 * v + firstpos : INT32_MAX;
                    const int t2 = block_min_int(after, ilds);
                    tok = t2 == INT32_MAX ? -1 : t2;
                }
            }
            if (tok >= 0) return tok;
        }
        if (round_last >= 0) last_tok = round_last;
        R = Rn;
    }
    return last_tok;
}

constexpr int kRoundsInFlight = 4;

// Chunk totals: workgroup (b, g) covers chunks [g * chunks_per_block, ...) of
// sequence b's sampled row, kRoundsInFlight rounds per step with every load of
// the step issued before any arithmetic.
// A descriptor names rows inside the batch and a position inside the output
// row; anything else (never produced by the decision kernels) is skipped.
__device__ __forceinline__ bool desc_ok(const SampleArgs& a, const SampleDesc& d)
{
    if (d.t_row < 0 || d.t_row >= a.n_target_rows) return false;
    if (d.out_pos < 0 || d.out_pos >= a.out_row) return false;
    if (d.kind == 0 && (d.d_row < 0 || d.d_row >= a.n_draft_rows)) return false;
    return true;
}

// Chunk totals of workgroup (b, g), which covers chunks [g * chunks_per_block,
// ...) of sequence b's sampled row (pair) as descriptor d names it.  Called by
// every thread of the workgroup.
template <int DT, bool VEC, bool MASK>
__device__ __forceinline__ void chunk_totals(const SampleArgs& a, int b, int g, const SampleDesc d,
                                             float* lds)
{
    constexpr int ES = DT == DT_F32 ? 4 : 2;
    const int ch0 = g * a.chunks_per_block;
    const int ch1 = min(ch0 + a.chunks_per_block, a.nchunks);
    if (ch0 >= ch1 || !desc_ok(a, d)) return;     // uniform across the workgroup
    const char* zr = row_ptr(a.target, d.t_row, a.t_stride, ES);
    const char* yr = d.kind == 0 ? row_ptr(a.draft, d.d_row, a.d_stride, ES) : zr;
    const int v0 = ch0 * a.vec_per_chunk;
    const int v1 = min(ch1 * a.vec_per_chunk, a.nvec);
    const int nfull = a.V >> 3;
    const int vfull = min(v1, nfull);
    const int kind = d.kind;
    const float h_t = stab_of(d.m_t, a.c), h_d = stab_of(d.m_d, a.c);

    float acc = 0.f;
    for (int r0 = v0; r0 < v1; r0 += kRoundsInFlight * kBlock) {
        Raw<DT> rz[kRoundsInFlight], ry[kRoundsInFlight];
#pragma unroll
        for (int u = 0; u < kRoundsInFlight; ++u) {
            const int v = r0 + u * kBlock + (int)threadIdx.x;
            if (v < vfull) {
                rz[u] = load_raw<DT, VEC>(zr, v);
                if (kind == 0) ry[u] = load_raw<DT, VEC>(yr, v);
            }
        }
#pragma unroll
        for (int u = 0; u < kRoundsInFlight; ++u) {
            const int rr = r0 + u * kBlock;
            if (rr >= v1) break;                  // uniform
            const int v = rr + (int)threadIdx.x;
            float ts = 0.f;
            if (v < v1) {
                float ez[kVec], ey[kVec], w[kVec];
                if (v < nfull) {
                    decode<DT>(rz[u], ez);
                    if (kind == 0) decode<DT>(ry[u], ey);
                } else {
                    load_partial<DT>(zr, v, a.V - 8 * v, -INFINITY, ez);
                    if (kind == 0) load_partial<DT>(yr, v, a.V - 8 * v, -INFINITY, ey);
                }
#pragma unroll
                for (int j = 0; j < kVec; ++j)
                    w[j] = weight_of<DT, MASK>(ez[j], kind == 0 ? ey[j] : 0.f, kind, a.c, h_t, h_d, d);
                ts = sum8(w);
            }
            float ex, rt;
            block_scan(ts, &ex, &rt, lds);
            acc += rt;
            const int ch = rr / a.vec_per_chunk;
            const int cend = min((ch + 1) * a.vec_per_chunk, a.nvec);
            if (rr + kBlock >= cend) {            // the chunk's last round
                // written through to the device's coherence point (a relaxed
                // agent-scope store), for a draw in this launch to read
                if (threadIdx.x == 0)
                    __hip_atomic_store(a.chunk_sums + (long long)b * a.nchunks + ch, acc, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
                acc = 0.f;
            }
        }
    }
}

// The draw of sequence b from its chunk totals and descriptor d: accumulate
// the totals in chunk order, find the chunk where u * total is crossed,
// rescan only that chunk.  Called by every thread of one workgroup.
struct PickShared {
    float lds[kWaves];
    int ilds[kWaves];
    float sums[kMaxChunks];
    int chunk;
    float rem;
};

template <int DT, bool VEC, bool MASK>
__device__ __forceinline__ void pick_sequence(const SampleArgs& a, int b, const SampleDesc& d, float my_sum,
                                              PickShared& ps)
{
    constexpr int ES = DT == DT_F32 ? 4 : 2;
    if (!desc_ok(a, d)) return;                   // uniform across the workgroup
    const char* zr = row_ptr(a.target, d.t_row, a.t_stride, ES);
    const char* yr = d.kind == 0 ? row_ptr(a.draft, d.d_row, a.d_stride, ES) : zr;

    if ((int)threadIdx.x < a.nchunks) ps.sums[threadIdx.x] = my_sum;
    __syncthreads();
    int kind = d.kind;
    double S = 0.0;
    for (int i = 0; i < a.nchunks; ++i) S += (double)ps.sums[i];
    if (!(S > 0.0) && kind == 0) {
        // no residual mass (p = q after rounding): draw from p instead
        kind = 1;
        for (int i = 0; i < a.nchunks; ++i) {
            const int e0 = i * a.vec_per_chunk;
            const int e1 = min(e0 + a.vec_per_chunk, a.nvec);
            const float t = chunk_total<DT, VEC, MASK>(a, zr, yr, kind, d, e0, e1, ps.lds);
            if (threadIdx.x == 0) ps.sums[i] = t;
        }
        __syncthreads();
        S = 0.0;
        for (int i = 0; i < a.nchunks; ++i) S += (double)ps.sums[i];
    }
    if (threadIdx.x == 0) {
        const double thr = (double)d.u * S;
        double pre = 0.0;
        int cs = -1, lastpos = -1;
        float rem = 0.f;
        for (int i = 0; i < a.nchunks; ++i) {
            const double nx = pre + (double)ps.sums[i];
            if (ps.sums[i] > 0.f) lastpos = i;
            if (cs < 0 && nx > thr) {
                cs = i;
                rem = (float)(thr - pre);
            }
            pre = nx;
        }
        if (cs < 0) {                  // rounding left no crossing: the last positive chunk, its end
            cs = lastpos < 0 ? 0 : lastpos;
            rem = ps.sums[cs];
        }
        ps.chunk = cs;
        ps.rem = fmaxf(rem, 0.f);
    }
    __syncthreads();
    const int cs = ps.chunk;
    const int e0 = cs * a.vec_per_chunk;
    const int e1 = min(e0 + a.vec_per_chunk, a.nvec);
    int tok = chunk_pick<DT, VEC, MASK>(a, zr, yr, kind, d, e0, e1, ps.rem, ps.lds, ps.ilds);
    if (threadIdx.x == 0) {
        if (tok < 0 || tok >= a.V) tok = 0;    // only for inputs outside the contract
        a.out_tokens[(long long)b * a.out_row + d.out_pos] = tok;
    }
}

// After the chunk totals of sequence b in a fused pass: true (uniform over
// the workgroup) in the last of the sequence's workgroups to finish, which
// then makes the draw.  The count is a per-sequence counter (a.done, zeroed
// by the call's first kernel).  Thread 0 wrote this workgroup's totals with
// relaxed agent-scope stores, which write through to the device's coherence
// point; it waits for them to be acknowledged (vmcnt counts stores on this
// architecture) before adding 1 to the counter, so a workgroup that sees
// every other count finds every total there too and reads them with
// agent-scope loads.  Neither side writes back or invalidates its XCD's L2,
// as an acquire-release increment would.
__device__ __forceinline__ bool last_of_sequence(const SampleArgs& a, int b, int* s_last)
{
    if (threadIdx.x == 0) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        const int before = __hip_atomic_fetch_add(a.done + b, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        *s_last = before == a.blocks_per_seq - 1;
    }
    __syncthreads();
    return *s_last != 0;
}

// This thread's chunk total for the draw (threads past the chunks repeat the last).
__device__ __forceinline__ float draw_total(const SampleArgs& a, int b)
{
    const int ct = min((int)threadIdx.x, a.nchunks - 1);
    return __hip_atomic_load(a.chunk_sums + (long long)b * a.nchunks + ct, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
}

// The chunk pass after a separate decision (large batches, early exit): the
// descriptor comes from the decision kernels.
template <int DT, bool VEC, bool MASK>
__global__ __launch_bounds__(kBlock) void k_sample_chunks(SampleArgs a)
{
    __shared__ float lds[kWaves];
    const int b = blockIdx.x / a.blocks_per_seq;
    const int g = blockIdx.x - b * a.blocks_per_seq;
    const SampleDesc d = a.desc[b];               // once, into registers
    chunk_totals<DT, VEC, MASK>(a, b, g, d, lds);
}

// The decision and the chunk pass in one launch: wave 0 of every workgroup
// of sequence b decides the whole round (decide_sequence), the same
// computation on the same inputs in each, so all agree bit for bit on the
// draw's row and weights; workgroup 0 also writes the round's outputs and
// the descriptor the draw reads.  Removes a dependent launch, for the price
// of reading the sequence's row statistics (a few hundred bytes) once per
// workgroup.  MASK: truncated rows.
//
// PICK: the sequence's last workgroup to finish also makes the draw
// (last_of_sequence).
template <int DT, bool VEC, bool MASK, bool PICK>
__global__ __launch_bounds__(kBlock) void k_decide_chunks(DecideSampleArgs da, SampleArgs a)
{
    __shared__ float lds[kWaves];
    __shared__ SampleDesc s_desc;
    __shared__ int s_last;
    const int b = blockIdx.x / a.blocks_per_seq;
    const int g = blockIdx.x - b * a.blocks_per_seq;
    if (threadIdx.x < 64) {
        SampleDesc d;
        const int j = decide_sequence<DT, MASK>(da, b, g == 0, &d);
        if ((int)threadIdx.x == j) s_desc = d;
    }
    __syncthreads();
    const SampleDesc d = s_desc;
    chunk_totals<DT, VEC, MASK>(a, b, g, d, lds);
    if constexpr (PICK) {
        if (!last_of_sequence(a, b, &s_last)) return;
        __shared__ PickShared ps;
        pick_sequence<DT, VEC, MASK>(a, b, d, draw_total(a, b), ps);
    }
}

// The draw: one workgroup per sequence.
template <int DT, bool VEC, bool MASK>
__global__ __launch_bounds__(kBlock) void k_sample_pick(SampleArgs a)
{
    __shared__ PickShared ps;
    const int b = blockIdx.x;
    // the chunk totals do not depend on the descriptor: both loads go out together
    const int ct = min((int)threadIdx.x, a.nchunks - 1);
    const float my_sum = a.chunk_sums[(long long)b * a.nchunks + ct];
    const SampleDesc d = a.desc[b];
    pick_sequence<DT, VEC, MASK>(a, b, d, my_sum, ps);
}

// The chunk pass, by k_decide_chunks when `da` is given (and then deciding
// the round too) or by k_sample_chunks after a separate decision, then the
// draw.
template <int DT, bool VEC, bool MASK>
static hipError_t launch_pair(int B, const DecideSampleArgs* da, const SampleArgs& a, hipStream_t st)
{
    const dim3 grid((unsigned)((long long)B * a.blocks_per_seq));
    hipError_t e;
    if (da && a.done) {                           // the draw in the same launch
        void* args[] = {const_cast<DecideSampleArgs*>(da), const_cast<SampleArgs*>(&a)};
        return hipLaunchKernel(reinterpret_cast<const void*>(k_decide_chunks<DT, VEC, MASK, true>), grid,
                               dim3(kBlock), args, 0, st);
    }
    if (da) {
        void* args[] = {const_cast<DecideSampleArgs*>(da), const_cast<SampleArgs*>(&a)};
        e = hipLaunchKernel(reinterpret_cast<const void*>(k_decide_chunks<DT, VEC, MASK, false>), grid,
                            dim3(kBlock), args, 0, st);
    } else {
        void* args[] = {const_cast<SampleArgs*>(&a)};
        e = hipLaunchKernel(reinterpret_cast<const void*>(k_sample_chunks<DT, VEC, MASK>), grid, dim3(kBlock),
                            args, 0, st);
    }
    if (e != hipSuccess) return e;
    void* args[] = {const_cast<SampleArgs*>(&a)};
    return hipLaunchKernel(reinterpret_cast<const void*>(k_sample_pick<DT, VEC, MASK>), dim3((unsigned)B),
                           dim3(kBlock), args, 0, st);
}

template <int DT>
static hipError_t launch_dt(bool vec, bool mask, int B, const DecideSampleArgs* da, const SampleArgs& a,
                            hipStream_t st)
{
    if (mask) return vec ? launch_pair<DT, true, true>(B, da, a, st) : launch_pair<DT, false, true>(B, da, a, st);
    return vec ? launch_pair<DT, true, false>(B, da, a, st) : launch_pair<DT, false, false>(B, da, a, st);
}

hipError_t launch_sample(int dt, bool vec, bool mask, int B, const DecideSampleArgs* da, const SampleArgs& a,
                         hipStream_t st)
{
    switch (dt) {
    case DT_F32: return launch_dt<DT_F32>(vec, mask, B, da, a, st);
    case DT_F16: return launch_dt<DT_F16>(vec, mask, B, da, a, st);
    default:     return launch_dt<DT_BF16>(vec, mask, B, da, a, st);
    }
}

}  // namespace sv
