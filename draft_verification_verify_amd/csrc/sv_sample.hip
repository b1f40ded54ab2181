// sv_sample.hip -- the round's single draw, on the one selected row per sequence.
//
// After a rejection at position j the replacement is drawn from the residual
// max(0, p_j - q_j) normalised; after a full acceptance the bonus is drawn
// from p_k (production blog, "The acceptance rule"; Cascade Speculative
// Drafting, review function).  The draw is an inverse CDF over the vocabulary
// in ascending index order: the smallest token whose cumulative weight
// exceeds u times the total.
//
// Work split: the sampled row (pair) of each sequence is cut into `nchunks`
// chunks, one workgroup each.  A workgroup streams its chunk once and writes
// the chunk's total weight.  The last workgroup of a sequence to finish
// (elected by an atomic counter) reads the chunk totals in chunk order, finds
// the chunk where u * total is crossed, rescans only that chunk and resolves
// the token with a workgroup prefix scan.  Chunk totals are recomputed by the
// same code in the rescan, so the two passes agree bit for bit; every
// reduction runs in a fixed order, so the result is deterministic.

#include "sv_device.h"

namespace sv {

// Weights of logical vector v: kind 0 the residual, otherwise p (unnormalised
// by a common factor that cancels).  Padding elements get weight 0.
template <int DT, bool VEC>
__device__ __forceinline__ void weights8(const char* zr, const char* yr, int v, int nfull, int V,
                                         int kind, float c, float off_t, float off_d, float* w)
{
    float ez[kVec];
    load8<DT, VEC>(zr, v, nfull, V, -INFINITY, ez);
    if (kind == 0) {
        float ey[kVec];
        load8<DT, VEC>(yr, v, nfull, V, -INFINITY, ey);
#pragma unroll
        for (int j = 0; j < kVec; ++j) {
            const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(ez[j], c, -off_t));
            const float q = __builtin_amdgcn_exp2f(__builtin_fmaf(ey[j], c, -off_d));
            w[j] = fmaxf(p - q, 0.f);
        }
    } else {
#pragma unroll
        for (int j = 0; j < kVec; ++j) w[j] = __builtin_amdgcn_exp2f(__builtin_fmaf(ez[j], c, -off_t));
    }
}

template <int DT, bool VEC>
__device__ float chunk_total(const SampleArgs& a, const char* zr, const char* yr, int kind,
                             float off_t, float off_d, int c0, int c1, float* lds)
{
    const int nfull = a.V >> 3;
    float total = 0.f;
    for (int r0 = c0; r0 < c1; r0 += kBlock) {
        const int v = r0 + (int)threadIdx.x;
        float ts = 0.f;
        if (v < c1) {
            float w[kVec];
            weights8<DT, VEC>(zr, yr, v, nfull, a.V, kind, a.c, off_t, off_d, w);
#pragma unroll
            for (int j = 0; j < kVec; ++j) ts += w[j];
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
template <int DT, bool VEC>
__device__ int chunk_pick(const SampleArgs& a, const char* zr, const char* yr, int kind,
                          float off_t, float off_d, int c0, int c1, float rem,
                          float* lds, int* ilds)
{
    const int nfull = a.V >> 3;
    float R = 0.f;
    int last_tok = -1;
    for (int r0 = c0; r0 < c1; r0 += kBlock) {
        const int v = r0 + (int)threadIdx.x;
        float w[kVec];
        float ts = 0.f;
        int firstpos = -1, lastpos = -1;
        if (v < c1) {
            weights8<DT, VEC>(zr, yr, v, nfull, a.V, kind, a.c, off_t, off_d, w);
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

template <int DT, bool VEC>
__global__ __launch_bounds__(kBlock) void k_sample(SampleArgs a)
{
    __shared__ float lds[kWaves];
    __shared__ int ilds[kWaves];
    __shared__ float s_sums[kMaxChunks];
    __shared__ int s_last, s_chunk, s_kind;
    __shared__ float s_rem;
    constexpr int ES = DT == DT_F32 ? 4 : 2;

    const int b = blockIdx.x / a.nchunks;
    const int ch = blockIdx.x - b * a.nchunks;
    const SampleDesc d = a.desc[b];
    const char* zr = row_ptr(a.target, d.t_row, a.t_stride, ES);
    const char* yr = d.kind == 0 ? row_ptr(a.draft, d.d_row, a.d_stride, ES) : zr;
    const int c0 = ch * a.vec_per_chunk;
    const int c1 = min(c0 + a.vec_per_chunk, a.nvec);

    const float tot = chunk_total<DT, VEC>(a, zr, yr, d.kind, d.off_t, d.off_d, c0, c1, lds);
    if (threadIdx.x == 0) {
        __hip_atomic_store(&a.chunk_sums[(long long)b * a.nchunks + ch], tot, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
        const unsigned old = __hip_atomic_fetch_add(&a.counters[b], 1u, __ATOMIC_ACQ_REL,
                                                    __HIP_MEMORY_SCOPE_AGENT);
        s_last = old == (unsigned)(a.nchunks - 1);
    }
    __syncthreads();
    if (!s_last) return;

    // the last workgroup of sequence b: locate the chunk holding u * total
    if (threadIdx.x < a.nchunks)
        s_sums[threadIdx.x] = __hip_atomic_load(&a.chunk_sums[(long long)b * a.nchunks + threadIdx.x],
                                                __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    int kind = d.kind;
    double S = 0.0;
    for (int i = 0; i < a.nchunks; ++i) S += (double)s_sums[i];
    if (!(S > 0.0) && kind == 0) {
        // no residual mass (p = q after rounding): draw from p instead
        kind = 1;
        for (int i = 0; i < a.nchunks; ++i) {
            const int e0 = i * a.vec_per_chunk;
            const int e1 = min(e0 + a.vec_per_chunk, a.nvec);
            const float t = chunk_total<DT, VEC>(a, zr, yr, kind, d.off_t, d.off_d, e0, e1, lds);
            if (threadIdx.x == 0) s_sums[i] = t;
        }
        __syncthreads();
        S = 0.0;
        for (int i = 0; i < a.nchunks; ++i) S += (double)s_sums[i];
    }
    if (threadIdx.x == 0) {
        const double thr = (double)d.u * S;
        double pre = 0.0;
        int cs = -1, lastpos = -1;
        float rem = 0.f;
        for (int i = 0; i < a.nchunks; ++i) {
            const double nx = pre + (double)s_sums[i];
            if (s_sums[i] > 0.f) lastpos = i;
            if (cs < 0 && nx > thr) {
                cs = i;
                rem = (float)(thr - pre);
            }
            pre = nx;
        }
        if (cs < 0) {                  // rounding left no crossing: last positive chunk, its end
            cs = lastpos < 0 ? 0 : lastpos;
            rem = s_sums[cs];
        }
        s_chunk = cs;
        s_rem = fmaxf(rem, 0.f);
        s_kind = kind;
    }
    __syncthreads();
    const int cs = s_chunk;
    const int e0 = cs * a.vec_per_chunk;
    const int e1 = min(e0 + a.vec_per_chunk, a.nvec);
    int tok = chunk_pick<DT, VEC>(a, zr, yr, s_kind, d.off_t, d.off_d, e0, e1, s_rem, lds, ilds);
    if (threadIdx.x == 0) {
        if (tok < 0 || tok >= a.V) tok = 0;    // only for inputs outside the contract
        a.out_tokens[(long long)b * a.out_row + d.out_pos] = tok;
    }
}

hipError_t launch_sample(int dt, bool vec, int B, const SampleArgs& a, hipStream_t st)
{
    void* args[] = {const_cast<SampleArgs*>(&a)};
    const unsigned grid = (unsigned)((long long)B * a.nchunks);
    const void* f;
    switch (dt) {
    case DT_F32: f = vec ? reinterpret_cast<const void*>(k_sample<DT_F32, true>)
                         : reinterpret_cast<const void*>(k_sample<DT_F32, false>); break;
    case DT_F16: f = vec ? reinterpret_cast<const void*>(k_sample<DT_F16, true>)
                         : reinterpret_cast<const void*>(k_sample<DT_F16, false>); break;
    default:     f = vec ? reinterpret_cast<const void*>(k_sample<DT_BF16, true>)
                         : reinterpret_cast<const void*>(k_sample<DT_BF16, false>); break;
    }
    return hipLaunchKernel(f, dim3(grid), dim3(kBlock), args, 0, st);
}

}  // namespace sv
