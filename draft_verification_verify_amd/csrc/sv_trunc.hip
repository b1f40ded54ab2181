// sv_trunc.hip -- top-k / top-p truncation of every row of a batch, applied
// to the target's and the draft's rows alike so that the acceptance rule runs
// on the two distributions actually sampled from (production blog,
// "Integration with the serving engine" and "Failure modes"; Ouroboros
// samples with top-p 0.8).
//
// Per row, with w_t = exp2((z_t - m) * c):
//   top-k keeps t iff fewer than top_k tokens have a strictly larger logit;
//   top-p then keeps t iff the kept tokens with strictly larger logits hold
//   less than top_p of the kept mass; equal logits are kept or dropped
//   together.  Both keep a set {t : key(z_t) >= tau} for an ordering key
//   (key_of), so a row is summarised by (m, tau, kept mass).
//
// One 512-thread workgroup per row finds tau by radix selection on the key,
// most significant digit first (11 bits, then 5 for 16-bit keys; 11, 11 and
// 10 bits for fp32 keys).  Each pass streams the row once (the first from
// HBM, the rest mostly from cache) and histograms the next digit of the keys
// that share the prefix chosen so far: counts for top-k, masses for top-p.
// Masses are fixed-point integers (w * 2^40, truncated), summed with integer
// atomics and integer reductions, so every result is independent of
// scheduling and bitwise reproducible.

#include "sv_device.h"

namespace sv {

namespace {

constexpr int kTB = kStatsBlock;       // 512 threads
constexpr int kTW = kTB / 64;
constexpr int kBins = 2048;            // the widest digit (11 bits)
constexpr int kFixBits = 40;           // masses in units of 2^-40 of the row max

typedef unsigned long long u64;

// floor(w * 2^40) for w in [0, 1], from the bits of w (0 below 2^-40).
__device__ __forceinline__ u64 fixed40(float w)
{
    const uint32_t b = __float_as_uint(w);
    const int e = (int)(b >> 23) - 127;
    if (e < -kFixBits) return 0;
    const u64 mant = (b & 0x7fffffu) | 0x800000u;
    const int s = e + kFixBits - 23;
    return s >= 0 ? mant << s : mant >> (-s);
}

__device__ __forceinline__ float weight(float z, float m, float c)
{
    return __builtin_amdgcn_exp2f((z - m) * c);
}

// The digits of the key, most significant first.
template <int DT>
struct Digits {
    static constexpr int levels = DT == DT_F32 ? 3 : 2;
    __device__ static int bits(int L)
    {
        if constexpr (DT == DT_F32) return L < 2 ? 11 : 10;
        else return L == 0 ? 11 : 5;
    }
    // key >> shift(L) & (2^bits - 1) is digit L
    __device__ static int shift(int L)
    {
        if constexpr (DT == DT_F32) return L == 0 ? 21 : (L == 1 ? 10 : 0);
        else return L == 0 ? 5 : 0;
    }
};

// Every element of a row, in any order: f(z).  Four vectors in flight per
// thread; cached loads, since the row is streamed again by the next pass.
template <int DT, bool VEC, typename F>
__device__ __forceinline__ void for_each_elem(const char* rp, int V, F&& f)
{
    const int nfull = V >> 3;
    int v = (int)threadIdx.x;
    for (; v + 3 * kTB < nfull; v += 4 * kTB) {
        Raw<DT> r[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) r[u] = load_raw_cached<DT, VEC>(rp, v + u * kTB);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            float e[kVec];
            decode<DT>(r[u], e);
#pragma unroll
            for (int j = 0; j < kVec; ++j) f(e[j]);
        }
    }
    for (; v < nfull; v += kTB) {
        Raw<DT> r = load_raw_cached<DT, VEC>(rp, v);
        float e[kVec];
        decode<DT>(r, e);
#pragma unroll
        for (int j = 0; j < kVec; ++j) f(e[j]);
    }
    if (v == nfull) {
        const int n = V - 8 * nfull;   // the partial last vector, if any
        for (int j = 0; j < n; ++j) f(load_elem<DT>(rp, 8LL * nfull + j));
    }
}

__device__ __forceinline__ u64 wave_sum_u64(u64 x)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
    return x;
}

// Sum over the workgroup; every thread gets it (integer: order-free).
__device__ __forceinline__ u64 block_sum_u64(u64 x, u64* lds)
{
    x = wave_sum_u64(x);
    if ((threadIdx.x & 63) == 0) lds[threadIdx.x >> 6] = x;
    __syncthreads();
    u64 r = 0;
#pragma unroll
    for (int w = 0; w < kTW; ++w) r += lds[w];
    __syncthreads();
    return r;
}

// Inclusive scan over the workgroup in thread order; *excl gets the exclusive value.
__device__ __forceinline__ u64 block_scan_u64(u64 x, u64* excl, u64* lds)
{
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    u64 incl = x;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const u64 y = __shfl_up(incl, o, 64);
        if (lane >= o) incl += y;
    }
    if (lane == 63) lds[w] = incl;
    __syncthreads();
    u64 pre = 0;
    for (int i = 0; i < w; ++i) pre += lds[i];
    __syncthreads();
    *excl = pre + incl - x;
    return pre + incl;
}

struct Shared {
    uint32_t cnt[kBins];
    u64 mass[kBins];
    u64 red[kTW];
    float redf[kTW];
    int sel;
    u64 incl;
};

// Digit selection, highest digit first: the first digit d (of nb) with
// base + sum_{d' >= d} val[d'] >= thr.  Sets sh.sel (-1 if none) and sh.incl
// (the inclusive sum at d, base included).  Called by every thread.
template <typename T>
__device__ void select_desc(const T* val, int nb, u64 base, double thr, Shared& sh)
{
    const int per = (nb + kTB - 1) / kTB;
    const int t = (int)threadIdx.x;
    u64 mine = 0;
    for (int j = 0; j < per; ++j) {
        const int pos = t * per + j;
        if (pos < nb) mine += (u64)val[nb - 1 - pos];
    }
    u64 excl;
    const u64 incl = block_scan_u64(mine, &excl, sh.red);
    if (t == 0) sh.sel = -1;
    __syncthreads();
    // the reaching thread is unique: the one whose range holds the crossing
    const bool before = (double)(base + excl) >= thr;
    const bool after = (double)(base + incl) >= thr;
    if (after && !before) {
        u64 acc = base + excl;
        for (int j = 0; j < per; ++j) {
            const int pos = t * per + j;
            if (pos >= nb) break;
            acc += (u64)val[nb - 1 - pos];
            if ((double)acc >= thr) {
                sh.sel = nb - 1 - pos;
                sh.incl = acc;
                break;
            }
        }
    }
    if (t == 0 && before) {            // thread 0 with base alone reaching thr
        sh.sel = nb - 1;
        sh.incl = base + (u64)val[nb - 1];
    }
    __syncthreads();
}

// One histogram pass at digit level L: among the keys >= lo, those whose
// digits above L equal `prefix` are binned by digit L (counts if CNT, masses
// if MASS); those with a larger prefix are summed into *above_cnt /
// *above_mass.  Level 0 has no prefix: every key >= lo is binned.
template <int DT, bool VEC, bool CNT, bool MASS>
__device__ void hist_pass(const char* rp, int V, int L, uint32_t prefix, uint32_t lo, float m,
                          float c, Shared& sh, u64* above_cnt, u64* above_mass)
{
    using D = Digits<DT>;
    for (int i = (int)threadIdx.x; i < kBins; i += kTB) {
        if (CNT) sh.cnt[i] = 0;
        if (MASS) sh.mass[i] = 0;
    }
    __syncthreads();
    const int sh_lo = D::shift(L);
    const uint32_t mask = (1u << D::bits(L)) - 1u;
    const int sh_hi = L == 0 ? 0 : D::shift(L - 1);
    uint32_t ac = 0;
    u64 am = 0;
    for_each_elem<DT, VEC>(rp, V, [&](float z) {
        const uint32_t key = key_of<DT>(z);
        if (key < lo) return;
        if (L > 0) {
            const uint32_t hp = key >> sh_hi;
            if (hp != prefix) {
                if (hp > prefix) {
                    ++ac;
                    if (MASS) am += fixed40(weight(z, m, c));
                }
                return;
            }
        }
        const uint32_t d = (key >> sh_lo) & mask;
        if (CNT) atomicAdd(&sh.cnt[d], 1u);
        if (MASS) {
            const u64 f = fixed40(weight(z, m, c));
            if (f) atomicAdd(&sh.mass[d], f);
        }
    });
    __syncthreads();
    *above_cnt = block_sum_u64(ac, sh.red);
    *above_mass = MASS ? block_sum_u64(am, sh.red) : 0;
}

template <int DT, bool VEC>
__global__ __launch_bounds__(kTB) void k_trunc_rows(TruncArgs a)
{
    using D = Digits<DT>;
    constexpr int ES = DT == DT_F32 ? 4 : 2;
    __shared__ Shared sh;
    const int row = blockIdx.x;
    if (row >= a.n_rows) return;
    const char* rp = row < a.n_target_rows ? row_ptr(a.target, row, a.t_stride, ES)
                                           : row_ptr(a.draft, row - a.n_target_rows, a.d_stride, ES);
    const int V = a.V;
    const float c = a.c;
    const bool topk = a.top_k >= 1 && a.top_k < V;
    const bool topp = a.top_p < 1.f;

    // pass 1: the row max, and the top digit's counts when top-k is on
    float mx = -INFINITY;
    if (topk) {
        for (int i = (int)threadIdx.x; i < kBins; i += kTB) sh.cnt[i] = 0;
        __syncthreads();
        const int s0 = D::shift(0);
        for_each_elem<DT, VEC>(rp, V, [&](float z) {
            mx = fmaxf(mx, z);
            atomicAdd(&sh.cnt[key_of<DT>(z) >> s0], 1u);
        });
    } else {
        for_each_elem<DT, VEC>(rp, V, [&](float z) { mx = fmaxf(mx, z); });
    }
    const float m = block_max<kTW>(mx, sh.redf);
    if (m == -INFINITY) {              // nothing to keep; the rule never reads such a row
        if (threadIdx.x == 0) a.rows[row] = TruncRow{m, -INFINITY, 0u, 0u};
        return;
    }

    uint32_t tau = 0;
    u64 kept = 0;
    if (topk) {
        uint32_t prefix = 0;
        u64 above_c = 0, above_m = 0;
        for (int L = 0; L < D::levels; ++L) {
            const bool last = L == D::levels - 1;
            if (L > 0) {
                if (last && !topp)
                    hist_pass<DT, VEC, true, true>(rp, V, L, prefix, 0u, m, c, sh, &above_c, &above_m);
                else
                    hist_pass<DT, VEC, true, false>(rp, V, L, prefix, 0u, m, c, sh, &above_c, &above_m);
            }
            select_desc(sh.cnt, 1 << D::bits(L), above_c, (double)a.top_k, sh);
            const int d = sh.sel < 0 ? 0 : sh.sel;
            prefix = (prefix << D::bits(L)) | (uint32_t)d;
            if (last && !topp) {
                // kept mass: everything above the final digit plus digits >= d
                u64 mine = 0;
                for (int i = (int)threadIdx.x; i < (1 << D::bits(L)); i += kTB)
                    if (i >= d) mine += sh.mass[i];
                kept = above_m + block_sum_u64(mine, sh.red);
            }
        }
        tau = prefix;
    }
    if (topp) {
        const uint32_t lo = tau;
        uint32_t prefix = 0;
        double budget = 0.0;
        for (int L = 0; L < D::levels; ++L) {
            u64 above_c = 0, above_m = 0;
            hist_pass<DT, VEC, false, true>(rp, V, L, prefix, lo, m, c, sh, &above_c, &above_m);
            if (L == 0) {
                u64 mine = 0;
                for (int i = (int)threadIdx.x; i < kBins; i += kTB) mine += sh.mass[i];
                const u64 M = block_sum_u64(mine, sh.red);
                budget = (double)a.top_p * (double)M;
            }
            select_desc(sh.mass, 1 << D::bits(L), above_m, budget, sh);
            const int d = sh.sel < 0 ? 0 : sh.sel;
            prefix = (prefix << D::bits(L)) | (uint32_t)d;
            kept = sh.incl;
        }
        tau = prefix;
    }
    if (threadIdx.x == 0) {
        const float l2s = (float)(log2((double)kept) - (double)kFixBits);
        a.rows[row] = TruncRow{m, l2s, tau, 0u};
    }
}

template <int DT>
hipError_t launch_dt(bool vec, const TruncArgs& a, hipStream_t st)
{
    void* args[] = {const_cast<TruncArgs*>(&a)};
    const void* f = vec ? reinterpret_cast<const void*>(k_trunc_rows<DT, true>)
                        : reinterpret_cast<const void*>(k_trunc_rows<DT, false>);
    return hipLaunchKernel(f, dim3((unsigned)a.n_rows), dim3(kTB), args, 0, st);
}

}  // namespace

hipError_t launch_trunc_rows(int dt, bool vec, const TruncArgs& a, hipStream_t st)
{
    switch (dt) {
    case DT_F32: return launch_dt<DT_F32>(vec, a, st);
    case DT_F16: return launch_dt<DT_F16>(vec, a, st);
    default:     return launch_dt<DT_BF16>(vec, a, st);
    }
}

}  // namespace sv
