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
// Five kernels find tau and the kept mass:
//  - k_topk16 and k_topk32 (16-bit rows under a top-k of at most 256 that
//    outnumber the compute units more than three times; fp32 rows under such
//    a top-k): one pass per row keeping only the logits that can still be
//    among the top_k largest, the thresholds found among those;
//  - k_trunc_merge: few fp32 rows are cut into slices, each k_topk32's, whose
//    candidates one workgroup per row merges;
//  - k_trunc16 (other fp16 / bf16 rows): one pass per row, an exact count of
//    all 65536 bit patterns in LDS, the thresholds read off the histogram;
//  - k_trunc_rows (other fp32 rows, and the rare row the one-pass kernels
//    cannot summarise): one 512-thread workgroup per row streaming the row
//    once per pass (the first from HBM, the rest mostly from cache).  fp32
//    rows are first binned by value and the threshold found among the keys
//    of the boundary bin (trunc_row_binned); otherwise radix selection on
//    the key, most significant digit first (11, 11 and 10 bits for fp32
//    keys; 11 then 5 for 16-bit keys), histogramming the next digit of the
//    keys that share the prefix chosen so far: counts for top-k, masses for
//    top-p.  k_trunc_rows_lds runs the same passes on fp32 rows of at most
//    32768 logits held in LDS, read from memory once.
// Masses are fixed-point integers (w * 2^40, truncated), summed with integer
// atomics and integer reductions, so every result is independent of
// scheduling and bitwise reproducible, and every kernel gives the same
// integers for the same row.  The kernels agree bit for bit on every row
// summary.

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

// Where a radix pass finds the row: streamed from memory on every pass
// (StreamRow), or held in LDS (LdsRow).  Both visit every element exactly
// once per pass, in any order; every pass's result (counts, integer masses,
// the max) is independent of that order.
template <int DT, bool VEC>
struct StreamRow {
    const char* rp;
    int V;
    template <typename F>
    __device__ __forceinline__ void each(F&& f) const { for_each_elem<DT, VEC>(rp, V, f); }
};

// An fp32 row of at most kLdsRowMax logits held in LDS: loaded from memory
// once (four vectors per thread in flight), then every pass reads LDS.
constexpr int kLdsRowMax = 32768;

struct LdsRow {
    const float* buf;                  // LDS, V floats
    int V;
    template <typename F>
    __device__ __forceinline__ void each(F&& f) const
    {
        const int nfull = V >> 3;
        for (int v = (int)threadIdx.x; v < nfull; v += kTB) {
            const float4 x = *reinterpret_cast<const float4*>(buf + 8 * v);
            const float4 y = *reinterpret_cast<const float4*>(buf + 8 * v + 4);
            f(x.x);
            f(x.y);
            f(x.z);
            f(x.w);
            f(y.x);
            f(y.y);
            f(y.z);
            f(y.w);
        }
        if ((int)threadIdx.x == nfull % kTB) {   // the partial last vector, if any
            for (int j = 8 * nfull; j < V; ++j) f(buf[j]);
        }
    }
};

template <bool VEC>
__device__ __forceinline__ void load_row_lds(float* buf, const char* rp, int V)
{
    const int nfull = V >> 3;
    for (int v0 = 0; v0 < nfull; v0 += 4 * kTB) {
        Raw<DT_F32> r[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int v = v0 + u * kTB + (int)threadIdx.x;
            if (v < nfull) r[u] = load_raw<DT_F32, VEC>(rp, v);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int v = v0 + u * kTB + (int)threadIdx.x;
            if (v < nfull) {
                float e[kVec];
                decode<DT_F32>(r[u], e);
                *reinterpret_cast<float4*>(buf + 8 * v) = float4{e[0], e[1], e[2], e[3]};
                *reinterpret_cast<float4*>(buf + 8 * v + 4) = float4{e[4], e[5], e[6], e[7]};
            }
        }
    }
    const int n = V - 8 * nfull;
    if ((int)threadIdx.x < n) buf[8 * nfull + threadIdx.x] = load_elem<DT_F32>(rp, 8LL * nfull + threadIdx.x);
    __syncthreads();
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
template <int DT, bool CNT, bool MASS, typename Src>
__device__ __forceinline__ void hist_pass(const Src& src, int L, uint32_t prefix, uint32_t lo, float m,
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
    src.each([&](float z) {
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

// The counters a later kernel of the call needs at zero, by the first
// launch's workgroup 0.
__device__ __forceinline__ void zero_counters(const TruncArgs& a)
{
    if (blockIdx.x == 0)
        for (int i = (int)threadIdx.x; i < a.n_zero; i += (int)blockDim.x) a.zero[i] = 0;
}

template <int DT>
__device__ __forceinline__ const char* trunc_row_ptr(const TruncArgs& a, int row)
{
    constexpr int ES = DT == DT_F32 ? 4 : 2;
    return row < a.n_target_rows ? row_ptr(a.target, row, a.t_stride, ES)
                                 : row_ptr(a.draft, row - a.n_target_rows, a.d_stride, ES);
}

// Radix digits of a key's offset o from a base, for keys spanning [base,
// base + range]: the first level takes the top (up to) 8 of the bits the
// range needs, each later one the next 8; level l's digit is o's bits
// [ls, hs) (level 0: every bit from ls up), ls = shift(l), hs = shift(l - 1).
struct OffDigits {
    int top;                           // bits the range needs (0: a single key)
    __device__ explicit OffDigits(uint32_t range) : top(range ? 32 - __clz((int)range) : 0) {}
    __device__ int shift(int l) const
    {
        const int s = top - 8 * (l + 1);
        return s > 0 ? s : 0;
    }
    __device__ static uint32_t digit(uint32_t o, int level, int hs, int ls)
    {
        return level == 0 ? o >> ls : (o >> ls) & ((1u << (hs - ls)) - 1u);
    }
};

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v)
{
    return (uint32_t)wave_max_int((int)(v ^ 0x80000000u)) ^ 0x80000000u;
}

template <int DT, typename Src>
__device__ __forceinline__ void trunc_row_radix(const TruncArgs& a, int row, Shared& sh, const Src& src)
{
    using D = Digits<DT>;
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
        src.each([&](float z) {
            mx = fmaxf(mx, z);
            atomicAdd(&sh.cnt[key_of<DT>(z) >> s0], 1u);
        });
    } else {
        src.each([&](float z) { mx = fmaxf(mx, z); });
    }
    const float m = block_max<kTW>(mx, sh.redf);
    if (m == -INFINITY) {              // nothing to keep; the rule never reads such a row
        if (threadIdx.x == 0) a.rows[row] = TruncRow{m, -INFINITY, 0u, 0u};
        __syncthreads();
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
                    hist_pass<DT, true, true>(src, L, prefix, 0u, m, c, sh, &above_c, &above_m);
                else
                    hist_pass<DT, true, false>(src, L, prefix, 0u, m, c, sh, &above_c, &above_m);
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
            hist_pass<DT, false, true>(src, L, prefix, lo, m, c, sh, &above_c, &above_m);
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
    __syncthreads();                   // the shared state is reused by the next row
}

// key_of's fp32 key back to the value (+0.0 for the merged zero)
__device__ __forceinline__ float value_of_key32(uint32_t k)
{
    return __uint_as_float(k >= 0x80000000u ? (k & 0x7FFFFFFFu) : ~k);
}

// ---- fp32 rows: value bins first ---------------------------------------------
// The radix passes' first digit of an fp32 key is its sign and top exponent
// bits, so a row's logits fall into a handful of bins and the passes' LDS
// atomics serialise on them.  For fp32 rows the first level instead bins the
// finite logits by value, kBins equal intervals from the smallest finite
// logit to the max: bin(z) = floor((z/2 - zlo/2) s), clamped (halving keeps
// the difference finite; each step is monotone in z, so a bin never holds a
// key above one of a higher bin, and equal keys share a bin).  One pass
// counts (top-k) and sums the fixed-point masses (top-p, the kept mass) of
// every bin; -inf logits are counted apart (they carry no mass).  The bin
// where a selection crosses its threshold is then gathered, at most kBins
// keys, and the threshold key found among them by radix levels on the
// offset from their smallest key, with the radix passes' integer sums and
// their >= rule, so tau and the kept mass are the radix passes' own.  A
// boundary bin too full to gather (long runs of equal or nearly equal
// logits) sends the row to the radix passes.

struct BinShared {
    uint32_t hc[256];
    u64 hm[256];
    uint32_t n;
};

__device__ __forceinline__ int value_bin(float z, float hz, float s)
{
    const float t = (0.5f * z - hz) * s;           // >= 0, finite
    return (int)fminf(t, (float)(kBins - 1));
}

__device__ __forceinline__ uint32_t block_max_u32(uint32_t v, u64* lds)
{
    v = wave_max_u32(v);
    if ((threadIdx.x & 63) == 0) lds[threadIdx.x >> 6] = v;
    __syncthreads();
    uint32_t r = 0;
#pragma unroll
    for (int w = 0; w < kTW; ++w) r = (uint32_t)lds[w] > r ? (uint32_t)lds[w] : r;
    __syncthreads();
    return r;
}

// The keys of the finite logits in value bin b into sh.cnt (any order);
// their number, which exceeds kBins when they do not fit.
template <typename Src>
__device__ __forceinline__ uint32_t gather_bin(const Src& src, int b, float hz, float s, Shared& sh, BinShared& bs)
{
    if (threadIdx.x == 0) bs.n = 0;
    __syncthreads();
    src.each([&](float z) {
        if (z != -INFINITY && value_bin(z, hz, s) == b) {
            const uint32_t pos = atomicAdd(&bs.n, 1u);
            if (pos < (uint32_t)kBins) sh.cnt[pos] = key_of<DT_F32>(z);
        }
    });
    __syncthreads();
    return bs.n;
}

// Among the n gathered keys (sh.cnt) at or above lo: the largest key tau
// with base + (sum over the keys >= tau of 1, or of their masses if MASS) >=
// thr, one 8-bit digit of the offset from the smallest key per level; the
// caller guarantees that all of them reach thr.  *incl gets that sum.
template <bool MASS>
__device__ __forceinline__ void list_select(Shared& sh, BinShared& bs, uint32_t n, uint32_t lo, u64 base, double thr,
                            float m, float c, uint32_t* tau, u64* incl)
{
    constexpr int P = kBins / kTB;
    const int t = (int)threadIdx.x;
    uint32_t k[P];
    u64 v[P];
    uint32_t kmx = 0u, nmn = 0u;       // the largest key, and the complement of the smallest
#pragma unroll
    for (int p = 0; p < P; ++p) {
        const uint32_t i = (uint32_t)(t + p * kTB);
        const uint32_t key = i < n ? sh.cnt[i] : 0u;
        k[p] = key >= lo ? key : 0u;   // 0: none (no finite logit has key 0)
        v[p] = k[p] ? (MASS ? fixed40(weight(value_of_key32(k[p]), m, c)) : 1u) : 0u;
        if (k[p]) {
            kmx = k[p] > kmx ? k[p] : kmx;
            nmn = ~k[p] > nmn ? ~k[p] : nmn;
        }
    }
    kmx = block_max_u32(kmx, sh.red);
    const uint32_t kmn = ~block_max_u32(nmn, sh.red);
    const OffDigits od(kmx - kmn);
    uint32_t prefix = 0u;
    u64 b = base;
    int hs = od.top, ls = od.shift(0);
    for (int level = 0;; ++level) {
        if (t < 256) {
            if (MASS) bs.hm[t] = 0;
            else bs.hc[t] = 0u;
        }
        __syncthreads();
#pragma unroll
        for (int p = 0; p < P; ++p) {
            const uint32_t o = k[p] - kmn;
            if (k[p] && (level == 0 || (o >> hs) == prefix)) {
                if (MASS) atomicAdd(&bs.hm[OffDigits::digit(o, level, hs, ls)], v[p]);
                else atomicAdd(&bs.hc[OffDigits::digit(o, level, hs, ls)], 1u);
            }
        }
        __syncthreads();
        if (MASS) select_desc(bs.hm, 1 << (hs - ls), b, thr, sh);
        else select_desc(bs.hc, 1 << (hs - ls), b, thr, sh);
        const int d = sh.sel < 0 ? 0 : sh.sel;
        const u64 own = MASS ? bs.hm[d] : (u64)bs.hc[d];
        prefix = (prefix << (hs - ls)) | (uint32_t)d;
        *incl = sh.incl;
        b = sh.incl - own;             // everything above the chosen digit
        __syncthreads();               // the histogram is cleared next
        if (ls == 0) break;
        hs = ls;
        ls = od.shift(level + 1);
    }
    *tau = kmn + prefix;
}

// One fp32 row by value bins; false (uniform) when a boundary bin holds more
// than kBins logits: the row is then left to the radix passes.
template <typename Src>
__device__ __forceinline__ bool trunc_row_binned(const TruncArgs& a, int row, Shared& sh, BinShared& bs, const Src& src)
{
    const int V = a.V;
    const float c = a.c;
    const bool topk = a.top_k >= 1 && a.top_k < V;
    const bool topp = a.top_p < 1.f;
    const int t = (int)threadIdx.x;

    // pass 1: the max and the smallest finite logit
    float mx = -INFINITY, mn = INFINITY;
    src.each([&](float z) {
        mx = fmaxf(mx, z);
        if (z != -INFINITY) mn = fminf(mn, z);
    });
    const float m = block_max<kTW>(mx, sh.redf);
    if (m == -INFINITY) {              // nothing to keep; the rule never reads such a row
        if (t == 0) a.rows[row] = TruncRow{m, -INFINITY, 0u, 0u};
        __syncthreads();
        return true;
    }
    const float zlo = -block_max<kTW>(-mn, sh.redf);
    const float hz = 0.5f * zlo;
    const float s = m > zlo ? fminf((float)(kBins - 1) / (0.5f * m - hz), 1e30f) : 0.f;

    // pass 2: each bin's count (top-k) and mass
    for (int i = t; i < kBins; i += kTB) {
        if (topk) sh.cnt[i] = 0u;
        sh.mass[i] = 0;
    }
    __syncthreads();
    src.each([&](float z) {
        if (z == -INFINITY) return;
        const int b = value_bin(z, hz, s);
        if (topk) atomicAdd(&sh.cnt[b], 1u);
        // a zero mass is added too: a branch around the atomic costs more
        atomicAdd(&sh.mass[b], fixed40(weight(z, m, c)));
    });
    __syncthreads();

    // top-k: the top_k-th largest key lo (keys >= lo survive); its bin bk
    // (-1: every finite logit survives) and the survivors' mass M
    uint32_t lo = 0u, nk = 0u;
    int bk = -1;
    u64 M = 0, mk = 0;                 // mk: the survivors' mass inside bin bk
    if (topk) {
        select_desc(sh.cnt, kBins, 0, (double)a.top_k, sh);
        bk = sh.sel;
        if (bk >= 0) {
            const uint32_t above = (uint32_t)(sh.incl - sh.cnt[bk]);
            __syncthreads();           // sh.cnt is overwritten by the gather
            nk = gather_bin(src, bk, hz, s, sh, bs);
            if (nk > (uint32_t)kBins) return false;
            u64 incl;
            list_select<false>(sh, bs, nk, 0u, above, (double)a.top_k, m, c, &lo, &incl);
            u64 mine = 0;
            for (int i = t; i < (int)nk; i += kTB) {
                const uint32_t key = sh.cnt[i];
                if (key >= lo) mine += fixed40(weight(value_of_key32(key), m, c));
            }
            mk = block_sum_u64(mine, sh.red);
        } else {
            lo = key_of<DT_F32>(-INFINITY);   // the top_k-th largest is -inf: every key survives
        }
    }
    {
        u64 mine = 0;
        for (int i = t; i < kBins; i += kTB)
            if (i > bk) mine += sh.mass[i];
        M = block_sum_u64(mine, sh.red) + mk;
    }

    uint32_t tau = lo;
    u64 kept = M;
    if (topp) {
        const double budget = (double)a.top_p * (double)M;
        // the bins wholly above bk first, highest first
        select_desc(sh.mass + (bk + 1), kBins - 1 - bk, 0, budget, sh);
        const int sel = sh.sel;
        if (sel >= 0) {
            const int bp = bk + 1 + sel;
            const u64 above = sh.incl - sh.mass[bp];
            __syncthreads();
            const uint32_t np = gather_bin(src, bp, hz, s, sh, bs);
            if (np > (uint32_t)kBins) return false;
            list_select<true>(sh, bs, np, 0u, above, budget, m, c, &tau, &kept);
        } else {                       // inside bin bk, among the survivors
            list_select<true>(sh, bs, nk, lo, M - mk, budget, m, c, &tau, &kept);
        }
    }
    if (t == 0) {
        const float l2s = (float)(log2((double)kept) - (double)kFixBits);
        a.rows[row] = TruncRow{m, l2s, tau, 0u};
    }
    __syncthreads();                   // the shared state is reused by the next row
    return true;
}

// fp32 rows of at most kLdsRowMax logits: each workgroup loads its row into
// LDS once and runs the radix passes on the LDS copy, instead of streaming
// the row again for every digit.  The copy and the radix state fill most of
// a CU's LDS, so one workgroup per CU.
template <bool VEC>
__global__ __launch_bounds__(kTB) void k_trunc_rows_lds(TruncArgs a)
{
    __shared__ Shared sh;
    __shared__ BinShared bs;
    __shared__ __attribute__((aligned(16))) float buf[kLdsRowMax];
    zero_counters(a);
    for (int row = blockIdx.x; row < a.n_rows; row += gridDim.x) {
        load_row_lds<VEC>(buf, trunc_row_ptr<DT_F32>(a, row), a.V);
        if (!trunc_row_binned(a, row, sh, bs, LdsRow{buf, a.V}))
            trunc_row_radix<DT_F32>(a, row, sh, LdsRow{buf, a.V});
    }
}

// Rows blockIdx.x, blockIdx.x + gridDim.x, ...; with only_marked, just the
// rows the one-pass kernel marked (pad = 1): the workgroup reads the marks of
// kTB rows at once (rows blockIdx.x * kTB + i, then gridDim.x * kTB further)
// and runs the marked ones.
template <int DT, bool VEC>
__global__ __launch_bounds__(kTB) void k_trunc_rows(TruncArgs a)
{
    __shared__ Shared sh;
    __shared__ BinShared bs;
    __shared__ int marked[kTB];
    __shared__ int n_marked;
    if (!a.only_marked) {
        zero_counters(a);
        for (int row = blockIdx.x; row < a.n_rows; row += gridDim.x) {
            const StreamRow<DT, VEC> src{trunc_row_ptr<DT>(a, row), a.V};
            if constexpr (DT == DT_F32) {
                if (trunc_row_binned(a, row, sh, bs, src)) continue;
            }
            trunc_row_radix<DT>(a, row, sh, src);
        }
        return;
    }
    for (int base = blockIdx.x * kTB; base < a.n_rows; base += gridDim.x * kTB) {
        if (threadIdx.x == 0) n_marked = 0;
        __syncthreads();
        const int row = base + (int)threadIdx.x;
        if (row < a.n_rows && a.rows[row].pad == 1u) marked[atomicAdd(&n_marked, 1)] = row;
        __syncthreads();
        const int n = n_marked;
        // each row's result depends on that row alone, so the order is free
        for (int i = 0; i < n; ++i)
            trunc_row_radix<DT>(a, marked[i], sh, StreamRow<DT, VEC>{trunc_row_ptr<DT>(a, marked[i]), a.V});
        __syncthreads();
    }
}

// ---- one pass for 16-bit logits ---------------------------------------------
// A 16-bit logit has one of 65536 bit patterns, so one streaming pass can
// count every value exactly: 32768 LDS words, each holding the counts of two
// adjacent patterns in its 16-bit halves (four integer ops and one ds_add
// per element, no exp in the stream).  The max, the top-k threshold, the
// top-p threshold and the kept mass are then read off the histogram: a
// value's mass is its count times the fixed-point weight of that one value,
// the same integer the radix passes sum element by element.
//
// Special patterns: +-inf are even and their odd neighbours are NaNs, so
// their words count them as plain 32-bit integers (a masked row can hold any
// number of -inf); -0.0 is merged into +0.0.  A half that reached 65536 (that
// many equal finite logits) would carry into its neighbour: the total no
// longer matches the row length, and the row is marked for the radix kernel.
//
// Analysis runs in position order: position d = 65535 - key is 0 for the
// largest value, and the patterns map to it as d < 32768: 32767 - d
// (positive values, descending), d >= 32768: d (negative values).  The 1024
// chunks of 64 positions are summed by thread (16 * lane + wave) so that the
// dense middle of the range is shared by every wave; a thread reads its 32
// words rotated by its lane, which puts the wave's reads in 32 different LDS
// banks.  The chunk where a threshold is crossed is resolved by one wave, a
// lane per position.

constexpr int kT16 = 1024;
constexpr int kW16 = kT16 / 64;
constexpr int kWords = 32768;          // 65536 patterns, two per word
constexpr int kChunks = 1024;

template <int DT>
__device__ __forceinline__ uint32_t ninf_bits()
{
    return DT == DT_BF16 ? 0xFF80u : 0xFC00u;
}

template <int DT>
__device__ __forceinline__ uint32_t pinf_bits()
{
    return DT == DT_BF16 ? 0x7F80u : 0x7C00u;
}

__device__ __forceinline__ uint32_t bits_at(uint32_t d)
{
    return d < 32768u ? 32767u - d : d;
}

template <int DT>
__device__ __forceinline__ float value_of_bits(uint32_t bits)
{
    if constexpr (DT == DT_BF16) return __uint_as_float(bits << 16);
    else return (float)__builtin_bit_cast(_Float16, (unsigned short)bits);
}

// Count the two 16-bit logits packed in w.
__device__ __forceinline__ void count_word(uint32_t* hist, uint32_t w)
{
    char* base = reinterpret_cast<char*>(hist);
    const uint32_t a0 = (w << 1) & 0x1FFFCu;               // byte offset of word (w & 0xFFFF) >> 1
    const uint32_t i0 = (w & 1u) * 0xFFFFu + 1u;           // 1 (low half) or 0x10000 (high half)
    const uint32_t a1 = (w >> 15) & 0x1FFFCu;
    const uint32_t i1 = ((w >> 16) & 1u) * 0xFFFFu + 1u;
    atomicAdd(reinterpret_cast<uint32_t*>(base + a0), i0);
    atomicAdd(reinterpret_cast<uint32_t*>(base + a1), i1);
}

// The count of pattern `bits` (-0.0 merged into +0.0; +-inf whole words).
template <int DT>
__device__ __forceinline__ uint32_t count_bits(const uint32_t* hist, uint32_t bits, uint32_t negzero)
{
    const uint32_t w = hist[bits >> 1];
    const uint32_t even = bits & ~1u;
    if (even == ninf_bits<DT>() || even == pinf_bits<DT>()) return (bits & 1u) ? 0u : w;
    if (bits == 0x8000u) return 0u;
    const uint32_t c = (w >> ((bits & 1u) * 16u)) & 0xFFFFu;
    return bits == 0u ? c + negzero : c;
}

// Per-chunk counts and masses are stored owner-major: chunk position
// p = 16 * lane + wave sits at slot(p) = 68 * (p % 16) + p / 16, so a wave's
// own 64 chunks are 64 consecutive slots, and 64 consecutive positions
// (p = 64 g + lane) fall in 64 different banks (68 = 4 mod 64).
constexpr int kSlotStride = 68;
__device__ __forceinline__ int slot_of(int p)
{
    return kSlotStride * (p & 15) + (p >> 4);
}

struct Scratch16 {
    uint32_t cnt[kSlotStride * 16];    // chunk counts, by slot
    u64 mass[kSlotStride * 16];        // chunk masses, by slot
    uint32_t wcnt[kW16];
    int wmin[kW16];
    int state;                         // 0: analyse; 1: overflowed half; 2: every logit -inf
    uint32_t d;
    uint32_t dk;
};

// ---- wave scans in DPP (row shifts, then row broadcasts), no LDS ----------
template <int CTRL, int ROWS, bool BC>
__device__ __forceinline__ uint32_t dpp32(uint32_t x)
{
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, ROWS, 0xf, BC);
}

template <int CTRL, int ROWS, bool BC>
__device__ __forceinline__ u64 dpp64(u64 x)
{
    const uint32_t lo = dpp32<CTRL, ROWS, BC>((uint32_t)x);
    const uint32_t hi = dpp32<CTRL, ROWS, BC>((uint32_t)(x >> 32));
    return ((u64)hi << 32) | lo;
}

// Inclusive scan over the wave in lane order.
__device__ __forceinline__ uint32_t wave_scan_u32(uint32_t x)
{
    x += dpp32<0x111, 0xf, true>(x);   // row_shr:1
    x += dpp32<0x112, 0xf, true>(x);   // row_shr:2
    x += dpp32<0x114, 0xf, true>(x);   // row_shr:4
    x += dpp32<0x118, 0xf, true>(x);   // row_shr:8
    x += dpp32<0x142, 0xa, false>(x);  // row_bcast:15 into rows 1 and 3
    x += dpp32<0x143, 0xc, false>(x);  // row_bcast:31 into rows 2 and 3
    return x;
}

__device__ __forceinline__ u64 wave_scan_u64(u64 x)
{
    x += dpp64<0x111, 0xf, true>(x);
    x += dpp64<0x112, 0xf, true>(x);
    x += dpp64<0x114, 0xf, true>(x);
    x += dpp64<0x118, 0xf, true>(x);
    x += dpp64<0x142, 0xa, false>(x);
    x += dpp64<0x143, 0xc, false>(x);
    return x;
}

__device__ __forceinline__ uint32_t lane63_u32(uint32_t x)
{
    return (uint32_t)__builtin_amdgcn_readlane((int)x, 63);
}

// x of lane `l` (uniform), to every lane
__device__ __forceinline__ u64 readlane_u64(u64 x, int l)
{
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)x, l);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(x >> 32), l);
    return ((u64)hi << 32) | lo;
}

__device__ __forceinline__ u64 lane63_u64(u64 x)
{
    return readlane_u64(x, 63);
}

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

// lo half + hi half + acc, in one instruction
__device__ __forceinline__ uint32_t add_halves(uint32_t w, uint32_t acc)
{
    return __builtin_amdgcn_udot2(__builtin_bit_cast(u16x2, w), u16x2{1, 1}, acc, false);
}

// floor(w * 2^40) for w in [0, 1] without branches, equal to fixed40(w):
// f = w * 2^40 is exact, and so are its high part floor(f / 2^32) and the
// remainder f - high * 2^32 (a multiple of f's last place, below 2^32).
__device__ __forceinline__ u64 fixed40_nb(float w)
{
    const float f = w * 1099511627776.0f;                     // 2^40
    const float hf = truncf(f * 2.3283064365386963e-10f);     // 2^-32
    const uint32_t hi = (uint32_t)hf;
    const uint32_t lo = (uint32_t)(f - hf * 4294967296.0f);
    return ((u64)hi << 32) | lo;
}

// The sum over each row of 16 lanes, in every lane of the row.
__device__ __forceinline__ u64 row_sum_u64(u64 x)
{
    x += dpp64<0x121, 0xf, false>(x);  // row_ror:1
    x += dpp64<0x122, 0xf, false>(x);  // row_ror:2
    x += dpp64<0x124, 0xf, false>(x);  // row_ror:4
    x += dpp64<0x128, 0xf, false>(x);  // row_ror:8
    return x;
}

// Persistent: workgroup g takes rows g, g + gridDim.x, ...  Its rows form
// one stream of rounds (four vectors per thread each, a row padded to an even
// number of rounds); two round buffers in registers alternate, and a buffer
// reloads the round two ahead as soon as it has been counted, so loads stay
// in flight across row ends: the next row's first two rounds arrive while the
// current row is analysed.  Every load is issued unconditionally (indices past
// a row's end, and rounds past the last row, read the row's first vector
// again, and only counting is predicated), which keeps the loads countable:
// each count waits for its own round's loads only.  Needs V >= 8.
template <int DT, bool VEC>
__global__ __launch_bounds__(kT16) void k_trunc16(TruncArgs a)
{
    constexpr int ES = 2;
    constexpr int kRound = 4 * kT16;   // vectors per round
    __shared__ __attribute__((aligned(16))) uint32_t hist[kWords];
    __shared__ __attribute__((aligned(16))) Scratch16 sc;
    const int V = a.V;
    const int t = (int)threadIdx.x;
    const int lane = t & 63, wv = t >> 6;
    const int nfull = V >> 3;
    const int R2 = 2 * ((nfull + 2 * kRound - 1) / (2 * kRound));   // rounds per row, even
    u32x4* h4 = reinterpret_cast<u32x4*>(hist);
    zero_counters(a);
    auto row_of = [&](int r) -> const char* {
        return r < a.n_target_rows ? row_ptr(a.target, r, a.t_stride, ES)
                                   : row_ptr(a.draft, r - a.n_target_rows, a.d_stride, ES);
    };

    // issue cursor: round ir of row irow
    int irow = blockIdx.x, ir = 0;
    auto issue = [&](Raw<DT> (&buf)[4]) {
        const bool live = irow < a.n_rows;
        const char* p = row_of(live ? irow : (int)blockIdx.x);
        const int v0 = ir * kRound + t;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int v = v0 + u * kT16;
            buf[u] = load_raw<DT, VEC>(p, live && v < nfull ? v : 0);
        }
        if (++ir == R2) {
            ir = 0;
            irow += (int)gridDim.x;
        }
    };
    auto count = [&](const Raw<DT> (&buf)[4], int ri) {
        const int v0 = ri * kRound + t;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            if (v0 + u * kT16 < nfull) {
                count_word(hist, buf[u].a.x);
                count_word(hist, buf[u].a.y);
                count_word(hist, buf[u].a.z);
                count_word(hist, buf[u].a.w);
            }
        }
    };

    Raw<DT> bufA[4], bufB[4];
    issue(bufA);
    issue(bufB);
    // The histogram is zeroed once here; after each row, only the chunks that
    // row touched are zeroed again, each by the thread that summed it.
    for (int i = t; i < kWords / 4; i += kT16) h4[i] = u32x4{0u, 0u, 0u, 0u};
    // thread 0's finished row, whose summary (with its fp64 log) is written
    // while the next row streams rather than inside the analysis
    int pend_row = -1;
    float pend_m = 0.f;
    u64 pend_kept = 0;
    uint32_t pend_tau = 0;
    auto flush = [&]() {
        if (t == 0 && pend_row >= 0) {
            const float l2s = (float)(log2((double)pend_kept) - (double)kFixBits);
            a.rows[pend_row] = TruncRow{pend_m, l2s, pend_tau, 0u};
            pend_row = -1;
        }
    };
    for (int row = blockIdx.x; row < a.n_rows; row += gridDim.x) {
    const char* rp = row_of(row);
    __syncthreads();
    flush();

    // the pass: count every pattern
    for (int ri = 0; ri < R2; ri += 2) {
        count(bufA, ri);
        issue(bufA);
        count(bufB, ri + 1);
        issue(bufB);
    }
    if (t == nfull % kT16 && 8 * nfull < V) {   // the partial last vector: one thread
        const unsigned short* e = reinterpret_cast<const unsigned short*>(rp) + 8LL * nfull;
        for (int j = 0; j < V - 8 * nfull; ++j) {
            const uint32_t b = e[j];
            atomicAdd(&hist[b >> 1], (b & 1u) * 0xFFFFu + 1u);
        }
    }
    __syncthreads();
    const uint32_t negzero = hist[0x8000u >> 1] & 0xFFFFu;     // -0.0
    const uint32_t ninf = hist[ninf_bits<DT>() >> 1];

    // chunk sums: thread (lane, wave) sums chunk position 16 * lane + wave,
    // reading its 8 groups of 4 words rotated by lane
    const int cp = 16 * lane + wv;
    const int bc = cp < 512 ? 511 - cp : cp;                  // its pattern chunk
    uint32_t my_cnt = 0;
    u32x4* const cw = h4 + 8 * bc;
    bool dirty;
    {
#pragma unroll
        for (int g = 0; g < 8; ++g) {
            const u32x4 q = cw[(g + lane) & 7];
            my_cnt = add_halves(q.x, my_cnt);
            my_cnt = add_halves(q.y, my_cnt);
            my_cnt = add_halves(q.z, my_cnt);
            my_cnt = add_halves(q.w, my_cnt);
        }
        dirty = my_cnt != 0u;          // a nonzero word has a nonzero half
        // whole-word counters and the -0.0 / +0.0 merge
        if (bc == (int)(ninf_bits<DT>() >> 6)) my_cnt += ninf - add_halves(ninf, 0u);
        if (bc == (int)(pinf_bits<DT>() >> 6)) {
            const uint32_t w = hist[pinf_bits<DT>() >> 1];
            my_cnt += w - add_halves(w, 0u);
        }
        if (bc == 512) my_cnt -= negzero;
        if (bc == 0) my_cnt += negzero;
    }
    const int own = kSlotStride * wv + lane;                  // slot_of(cp)
    sc.cnt[own] = my_cnt;
    const uint32_t fin_cnt = bc == (int)(ninf_bits<DT>() >> 6) ? my_cnt - ninf : my_cnt;
    {
        const uint32_t wt = lane63_u32(wave_scan_u32(my_cnt));
        const unsigned long long ne = __ballot(fin_cnt != 0u);
        if (lane == 0) {
            sc.wcnt[wv] = wt;
            sc.wmin[wv] = ne ? 16 * (__ffsll((long long)ne) - 1) + wv : INT32_MAX;
        }
    }
    // after every reader of the row's histogram is done: zero this thread's chunk
    auto clear_chunk = [&]() {
        __syncthreads();
        if (dirty) {
#pragma unroll
            for (int g = 0; g < 8; ++g) cw[(g + lane) & 7] = u32x4{0u, 0u, 0u, 0u};
        }
    };
    __syncthreads();

    // wave 0: the row's count, the max (first nonempty position of the first
    // nonempty chunk), then top-k
    if (wv == 0) {
        const uint32_t total = lane63_u32(wave_scan_u32(lane < kW16 ? sc.wcnt[lane] : 0u));
        const int cmax = wave_min_int(lane < kW16 ? sc.wmin[lane] : INT32_MAX);
        const uint32_t finite = total - ninf;
        // a half overflowed: the row goes to the radix kernel
        const int state = total != (uint32_t)V ? 1 : finite == 0 ? 2 : 0;
        uint32_t d = 0, dk = 65535u;   // positions <= dk survive top-k
        if (state == 0) {
            {
                const uint32_t dd = 64u * cmax + lane;
                const uint32_t bb = bits_at(dd);
                const bool nz = bb != ninf_bits<DT>() && count_bits<DT>(hist, bb, negzero) != 0u;
                const unsigned long long hit = __ballot(nz);
                d = 64u * cmax + (uint32_t)(__ffsll((long long)hit) - 1);
            }
            if (a.top_k >= 1 && (uint32_t)a.top_k < finite) {
                const uint32_t need = (uint32_t)a.top_k;
                uint32_t base = 0;
                int ch = -1;
                for (int g = cmax >> 6; g < kChunks / 64 && ch < 0; ++g) {   // uniform; earlier chunks are empty
                    const uint32_t x = sc.cnt[slot_of(64 * g + lane)];
                    const uint32_t incl = base + wave_scan_u32(x);
                    const unsigned long long hit = __ballot(incl >= need);
                    if (hit) {
                        const int f = __ffsll((long long)hit) - 1;
                        ch = 64 * g + f;
                        base = (uint32_t)__builtin_amdgcn_readlane((int)(incl - x), f);
                    } else {
                        base = lane63_u32(incl);
                    }
                }
                if (ch < 0) ch = kChunks - 1;             // unreachable: top_k < finite
                const uint32_t dd = 64u * ch + lane;
                const uint32_t incl = base + wave_scan_u32(count_bits<DT>(hist, bits_at(dd), negzero));
                const unsigned long long hit = __ballot(incl >= need);
                dk = 64u * ch + (uint32_t)(__ffsll((long long)hit) - 1);
            }
        }
        if (lane == 0) {
            sc.state = state;
            sc.d = d;
            sc.dk = dk;
        }
    }
    __syncthreads();
    {
        const int state = sc.state;
        if (state != 0) {
            if (t == 0) a.rows[row] = state == 1 ? TruncRow{0.f, 0.f, 0u, 1u}
                                                 : TruncRow{-INFINITY, -INFINITY, 0u, 0u};
            clear_chunk();
            continue;
        }
    }
    const float m = value_of_bits<DT>(bits_at(sc.d));
    const float c = a.c;
    const uint32_t dk = sc.dk;

    // masses of the chunks (positions <= dk): each wave takes the nonempty
    // chunks its own threads summed, four at a time, a row of 16 lanes per
    // chunk and four adjacent patterns (one 8-byte read) per lane; no
    // branches, so the four weights of a lane overlap
    {
        sc.mass[own] = 0;
        unsigned long long todo = __ballot(fin_cnt != 0 && (uint32_t)cp <= (dk >> 6));
        const int r = lane >> 4;
        const uint32_t q = (uint32_t)(lane & 15);
        while (todo) {
            int pick[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                pick[i] = todo ? __ffsll((long long)todo) - 1 : -1;
                todo &= todo - 1;
            }
            const int bit = r == 0 ? pick[0] : r == 1 ? pick[1] : r == 2 ? pick[2] : pick[3];
            const bool live = bit >= 0;                    // rows without a chunk add zero
            const uint32_t d0 = 64u * (uint32_t)(16 * (live ? bit : 0) + wv) + 4u * q;
            const bool pos = d0 < 32768u;
            const uint32_t pb = pos ? 32764u - d0 : d0;    // the lowest of the four patterns
            const uint2 hw = *reinterpret_cast<const uint2*>(hist + (pb >> 1));
            uint32_t n[4] = {hw.x & 0xFFFFu, hw.x >> 16, hw.y & 0xFFFFu, hw.y >> 16};
            n[0] = pb == 0u ? n[0] + negzero : n[0];       // +0.0 takes -0.0's count
            n[0] = pb == 0x8000u ? 0u : n[0];
            const bool ni = pb == ninf_bits<DT>();          // -inf and its 32-bit counter
            n[0] = ni ? 0u : n[0];
            n[1] = ni ? 0u : n[1];
            u64 mk = 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t d = pos ? d0 + 3u - (uint32_t)i : d0 + (uint32_t)i;
                const uint32_t ni_ = live && d <= dk ? n[i] : 0u;
                mk += (u64)ni_ * fixed40_nb(weight(value_of_bits<DT>(pb + (uint32_t)i), m, c));
            }
            mk = row_sum_u64(mk);
            if (q == 0 && live) sc.mass[kSlotStride * wv + bit] = mk;
        }
    }
    __syncthreads();

    // wave 0: the kept mass M, then the top-p boundary: the lane, the chunk
    // and the position where the running mass first reaches top_p * M
    if (wv == 0) {
        u64 lsum = 0;                  // lane l: chunk positions 16 l .. 16 l + 15
#pragma unroll
        for (int j = 0; j < 16; ++j) lsum += sc.mass[kSlotStride * j + lane];
        const u64 incl = wave_scan_u64(lsum);
        const u64 M = lane63_u64(incl);
        u64 kept = M;
        uint32_t dtau = dk;
        if (a.top_p < 1.f) {
            const double budget = (double)a.top_p * (double)M;
            const unsigned long long hit = __ballot((double)incl >= budget);
            const int L = hit ? __ffsll((long long)hit) - 1 : 63;
            const u64 base = readlane_u64(incl - lsum, L);
            // lane j < 16: chunk position 16 L + j
            const u64 x = lane < 16 ? sc.mass[kSlotStride * lane + L] : 0;
            const u64 incl1 = base + wave_scan_u64(x);
            const unsigned long long hit1 = __ballot(lane < 16 && (double)incl1 >= budget);
            const int f = hit1 ? __ffsll((long long)hit1) - 1 : 15;
            const int ch = 16 * L + f;
            const u64 excl_f = readlane_u64(incl1 - x, f);
            const uint32_t d = 64u * ch + lane;
            u64 mk = 0;
            if (d <= dk) {
                const uint32_t b = bits_at(d);
                const uint32_t n = count_bits<DT>(hist, b, negzero);
                mk = (u64)n * fixed40_nb(weight(value_of_bits<DT>(b), m, c));
            }
            const u64 incl2 = excl_f + wave_scan_u64(mk);
            const unsigned long long hit2 = __ballot((double)incl2 >= budget);
            const int f2 = hit2 ? __ffsll((long long)hit2) - 1 : 63;
            dtau = 64u * ch + (uint32_t)f2;
            kept = readlane_u64(incl2, f2);
        }
        if (lane == 0) {               // thread 0: written during the next row's pass
            pend_row = row;
            pend_m = m;
            pend_kept = kept;
            pend_tau = 65535u - dtau;
        }
    }
    clear_chunk();
    }
    flush();
}

// ---- one pass for 16-bit logits under a small top-k -------------------------
// With top-k on, only the top_k largest logits (with the ties at the
// boundary) can be kept, so for top_k <= kTopkMax a row needs no histogram of
// every pattern.  One 256-thread workgroup takes one row, eight to a CU (the
// analysis of one row overlaps the streaming of the others).  It runs when
// the rows outnumber the compute units more than three times: fewer rows
// take k_trunc16, whose stream has no compaction for a load to wait on, and
// with so few rows the histograms' LDS atomics do not bound it.  Each wave
// keeps, in LDS, a list of the 32-bit words (two logits each) it has streamed that
// may still hold a kept logit, and a floor F: the list holds every word with
// a logit whose key is at least F.  When a lane's part of the list fills up,
// the wave raises F to the (top_k + 1)-th largest key at or above F in its
// list (that many logits of the row are at least as large, so F never passes
// the row's top_k-th largest key, and the row has more than top_k finite
// logits) and drops the words with nothing left above it.  F starts just
// above -inf, so an -inf logit never counts, or, for top_k < 64, at the
// (top_k + 1)-th largest of the wave's 64 lane maxima over its first vectors
// if positive (that many different logits are at least that large; found bit
// by bit with ballots).
//
// After the stream the workgroup merges its waves' lists above the largest
// floor Fg: the top_k-th largest key among them is the row's; if no wave
// raised its floor the lists hold every finite logit and top-k is off when
// they number at most top_k (as in k_trunc16).  The row max is the largest
// key.  The kept keys (at most kKeptMax, else the row goes to the radix
// kernel) are gathered, and top-p runs on their fixed-point masses.  Both
// searches are radix selections on the 16-bit key, high byte then low byte,
// over a 256-bin histogram, and every count, mass and threshold equals
// k_trunc16's.  A wave whose list still overflows after raising F (more than
// 64 * (kSlots - 4) words tied at the floor) marks the row for the radix
// kernel too.
//
// Keys here are key_of's with -0.0 merged into +0.0 and every negative value
// one higher (word_keys: both halves of a word in four operations); tau is
// converted back when written.  The stream tests raw bits, two operations a
// word: above a positive floor F only positive logits can count, and their
// 16-bit patterns, read as signed integers, are their keys minus 0x8000, so
// a word may hold one iff the larger of its halves is at least F - 0x8000;
// at or below +0.0, every positive logit counts and a negative pattern's key
// falls as the pattern, read unsigned, grows, so a word may hold one iff the
// smaller of its halves, read unsigned, is at most 0x10000 - F.

constexpr int kKeptMax = 512;          // kept keys gathered after top-k

constexpr int kTK = 256;               // threads per row
constexpr int kTKW = kTK / 64;
constexpr int kSlots = 12;             // list words per lane (eight workgroups to a CU)

struct TopkShared {
    static constexpr int NW = kTKW;
    uint32_t list[NW * kSlots * 64];    // wave w, lane l, word j: [w][j * 64 + l]
    uint32_t whist[NW * 256];           // each wave's radix histogram; after the stream, the kept keys
    u64 hist[256];                      // the workgroup's: counts (low 1 KB) or masses
    u64 red[NW];
    uint32_t mx[NW];
    uint32_t F[NW];
    uint32_t over[NW];
    uint32_t nk;
    uint32_t sel;
    uint32_t total;
    u64 above;
    u64 incl;
};

typedef short s16x2 __attribute__((ext_vector_type(2)));

// The keys of the two logits of a word, low half in the low 16 bits: key_of,
// -0.0 merged into +0.0 and negative values one up (an order-preserving map).
__device__ __forceinline__ uint32_t word_keys(uint32_t x)
{
    const uint32_t m = __builtin_bit_cast(uint32_t, __builtin_bit_cast(s16x2, x) >> (short)15);
    const uint32_t v = x ^ (m | 0x80008000u);
    return __builtin_bit_cast(uint32_t, __builtin_bit_cast(u16x2, v) + __builtin_bit_cast(u16x2, m & 0x00010001u));
}

// word_keys' key back to key_of's, and to the value
__device__ __forceinline__ uint32_t std_key(uint32_t k)
{
    return k >= 0x8000u ? k : k - 1u;
}

template <int DT>
__device__ __forceinline__ float value_of_key(uint32_t k)
{
    return value_of_bits<DT>(k >= 0x8000u ? (k & 0x7FFFu) : (~(k - 1u) & 0xFFFFu));
}

// Orders this wave's LDS accesses: the hardware runs a wave's LDS
// instructions in order; this keeps the compiler from moving them.
__device__ __forceinline__ void wave_lds_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ uint32_t lane_prefix(unsigned long long bal)
{
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
}

// A 256-bin count histogram read from the top: its total, the bin at which
// the count first reaches `need` (if the total does) and the count in the
// bins above it, in every lane.  Lane l holds bins 255 - 4l down to 252 - 4l.
__device__ __forceinline__ uint32_t find_desc_count(const uint32_t* h, uint32_t need, uint32_t& bin,
                                                    uint32_t& above)
{
    const int lane = (int)threadIdx.x & 63;
    const u32x4 q = reinterpret_cast<const u32x4*>(h)[63 - lane];
    const uint32_t s = q.x + q.y + q.z + q.w;
    const uint32_t incl = wave_scan_u32(s);
    const unsigned long long hit = __ballot(incl >= need);
    const int L = hit ? __ffsll((long long)hit) - 1 : 63;
    const uint32_t acc = incl - s;
    uint32_t b = 3u, a = acc + q.w + q.z + q.y;
    if (acc + q.w >= need) { b = 0u; a = acc; }
    else if (acc + q.w + q.z >= need) { b = 1u; a = acc + q.w; }
    else if (acc + q.w + q.z + q.y >= need) { b = 2u; a = acc + q.w + q.z; }
    bin = 255u - 4u * (uint32_t)L - (uint32_t)__builtin_amdgcn_readlane((int)b, L);
    above = (uint32_t)__builtin_amdgcn_readlane((int)a, L);
    return lane63_u32(incl);
}

// The same for a 256-bin mass histogram: the bin at which base plus the mass
// from the top, as a double, first reaches `budget` (the total reaches it).
__device__ __forceinline__ void find_desc_mass(const u64* h, u64 base, double budget, uint32_t& bin, u64& above)
{
    const int lane = (int)threadIdx.x & 63;
    const u64 m0 = h[255 - 4 * lane], m1 = h[254 - 4 * lane], m2 = h[253 - 4 * lane], m3 = h[252 - 4 * lane];
    const u64 s = m0 + m1 + m2 + m3;
    const u64 incl = base + wave_scan_u64(s);
    const unsigned long long hit = __ballot((double)incl >= budget);
    const int L = hit ? __ffsll((long long)hit) - 1 : 63;
    const u64 acc = incl - s;
    uint32_t b = 3u;
    u64 a = acc + m0 + m1 + m2;
    if ((double)(acc + m0) >= budget) { b = 0u; a = acc; }
    else if ((double)(acc + m0 + m1) >= budget) { b = 1u; a = acc + m0; }
    else if ((double)(acc + m0 + m1 + m2) >= budget) { b = 2u; a = acc + m0 + m1; }
    bin = 255u - 4u * (uint32_t)L - (uint32_t)__builtin_amdgcn_readlane((int)b, L);
    above = readlane_u64(a, L);
}

constexpr int kMergeMax = 4096;        // candidates the merge of a row's slices gathers

// A slice's candidates, when fp32 rows are cut into S slices: the keys at or
// above the slice's floor Fs.  Fs is the largest floor Fg of its waves when
// the n keys at or above Fg are few (at most K1, or S * n at most half of
// what the merge gathers), else the K1-th largest of those n keys.  Either
// way K1 different logits of the row are at least Fs (a wave raises its
// floor only under K1 of its own keys), so Fs never passes the row's
// top_k-th largest key, and every key at or above the largest floor of a
// row's slices is among the row's candidates.  kr: this lane's keys (0 for
// none; keys below the wave's floor are skipped), F: its wave's floor.
// Wave 0 writes the keys and a header (Fs, the largest key, their number,
// and an overflow flag, set when a wave's list overflowed or when the keys
// at or above Fs outnumber kCandMax).  The list area holds the J keys of
// each of the NT lanes.  Called by every thread of the workgroup.
template <int NT, int J>
__device__ __forceinline__ void slice_candidates(const uint32_t (&kr)[J], uint32_t F, uint32_t K1, int S, uint32_t* list, uint32_t* wh0, uint32_t* sF, uint32_t* smx,
                                                 const uint32_t* sover, uint32_t* snk, uint32_t* cand, uint32_t* hdr)
{
    constexpr int NW = NT / 64;
    const int t = (int)threadIdx.x, lane = t & 63, wv = t >> 6;
    {
        uint32_t mx_t = 0;
#pragma unroll
        for (int j = 0; j < J; ++j) mx_t = kr[j] > mx_t ? kr[j] : mx_t;
        const uint32_t mx = wave_max_u32(mx_t);
        if (lane == 0) {
            sF[wv] = F;
            smx[wv] = mx;
        }
    }
    __syncthreads();
    uint32_t Fg = sF[0], mxk = smx[0], over = sover[0];
#pragma unroll
    for (int w = 1; w < NW; ++w) {
        Fg = sF[w] > Fg ? sF[w] : Fg;
        mxk = smx[w] > mxk ? smx[w] : mxk;
        over |= sover[w];
    }
    if (over) {
        if (t == 0) {
            hdr[0] = 0u;
            hdr[1] = 0u;
            hdr[2] = 0u;
            hdr[3] = 1u;
        }
        return;
    }
    // the keys at or above Fg, gathered into the list area (every key is in registers)
#pragma unroll
    for (int j = 0; j < J; ++j) {
        const bool keep = kr[j] >= Fg;     // Fg >= f0 > 0: empty slots never kept
        const unsigned long long bal = __ballot(keep);
        if (bal) {
            const int first = __ffsll((long long)bal) - 1;
            uint32_t base = 0;
            if (lane == first) base = atomicAdd(snk, (uint32_t)__popcll(bal));
            base = (uint32_t)__builtin_amdgcn_readlane((int)base, first);
            if (keep) list[base + lane_prefix(bal)] = kr[j];
        }
    }
    __syncthreads();
    if (wv != 0) return;
    const uint32_t n = *snk;
    uint32_t Fs = Fg;
    if (n >= K1 && (n > (uint32_t)kCandMax || (long long)S * n > kMergeMax / 2)) {
        // uniform: the K1-th largest, one offset digit per level
        const OffDigits od(mxk - Fg);
        uint32_t prefix = 0, need = K1;
        int hs = od.top, ls = od.shift(0);   // level 0 has no prefix
        for (int level = 0;; ++level) {
            reinterpret_cast<u32x4*>(wh0)[lane] = u32x4{0u, 0u, 0u, 0u};
            wave_lds_sync();
            for (uint32_t i = (uint32_t)lane; i < n; i += 64) {
                const uint32_t o = list[i] - Fg;
                if (level == 0 || (o >> hs) == prefix) atomicAdd(&wh0[od.digit(o, level, hs, ls)], 1u);
            }
            wave_lds_sync();
            uint32_t bin, above;
            find_desc_count(wh0, need, bin, above);
            wave_lds_sync();
            prefix = (prefix << (hs - ls)) | bin;
            need -= above;
            if (ls == 0) break;
            hs = ls;
            ls = od.shift(level + 1);
        }
        Fs = Fg + prefix;
    }
    uint32_t cnt = 0;
    for (uint32_t i0 = 0; i0 < n; i0 += 64) {
        const uint32_t i = i0 + (uint32_t)lane;
        const uint32_t k = i < n ? list[i] : 0u;
        const bool keep = k >= Fs;
        const unsigned long long bal = __ballot(keep);
        const uint32_t pos = cnt + lane_prefix(bal);
        if (keep && pos < (uint32_t)kCandMax) cand[pos] = k;
        cnt += (uint32_t)__popcll(bal);
    }
    if (lane == 0) {
        hdr[0] = Fs;
        hdr[1] = mxk;
        hdr[2] = cnt < (uint32_t)kCandMax ? cnt : (uint32_t)kCandMax;
        hdr[3] = cnt > (uint32_t)kCandMax ? 1u : 0u;
    }
}

template <int DT, bool VEC>
__global__ __launch_bounds__(kTK) __attribute__((amdgpu_waves_per_eu(8))) void k_topk16(TruncArgs a)
{
    constexpr int KS = kSlots;
    static_assert(kTKW * 256 >= kKeptMax, "the kept keys reuse the wave histograms");
    __shared__ __attribute__((aligned(16))) TopkShared sh;
    const int row = (int)blockIdx.x;
    const int t = (int)threadIdx.x;
    const int lane = t & 63, wv = t >> 6;
    const char* const rp = trunc_row_ptr<DT>(a, row);
    const int V = a.V;
    const int nfull = V >> 3;                                  // >= 1
    const uint32_t K1 = (uint32_t)a.top_k + 1u;
    const uint32_t f0 = (~ninf_bits<DT>() & 0xFFFFu) + 2u;      // just above -inf
    uint32_t* const lst = sh.list + wv * (KS * 64);
    uint32_t* const wh = sh.whist + wv * 256;
    uint32_t* const hc = reinterpret_cast<uint32_t*>(sh.hist);
    uint32_t F = f0;                   // the wave's floor (uniform)
    uint32_t* const lane_list = lst + lane;
    uint32_t* wp = lane_list;          // this lane's next word
    uint32_t* const room = lane_list + 64 * (KS - 4);   // beyond: no room for a vector
    int c = 0;                         // this lane's words (while compacting)

    // raise the floor and drop the words with nothing above it; all lanes, uniform
    auto compact = [&]() {
        c = (int)((wp - lane_list) >> 6);
        const int cmax = wave_max_int(c);
        uint32_t total = 0, b1 = 0, above = 0;
#pragma unroll
        for (int level = 0; level < 2; ++level) {
            reinterpret_cast<u32x4*>(wh)[lane] = u32x4{0u, 0u, 0u, 0u};
            wave_lds_sync();
            for (int j = 0; j < c; ++j) {
                const uint32_t u = word_keys(lst[j * 64 + lane]);
                const uint32_t k0 = u & 0xFFFFu, k1 = u >> 16;
                if (level == 0) {
                    if (k0 >= F) atomicAdd(&wh[k0 >> 8], 1u);
                    if (k1 >= F) atomicAdd(&wh[k1 >> 8], 1u);
                } else {
                    if (k0 >= F && (k0 >> 8) == b1) atomicAdd(&wh[k0 & 255u], 1u);
                    if (k1 >= F && (k1 >> 8) == b1) atomicAdd(&wh[k1 & 255u], 1u);
                }
            }
            wave_lds_sync();
            uint32_t bin, ab;
            const uint32_t tot = find_desc_count(wh, level == 0 ? K1 : K1 - above, bin, ab);
            wave_lds_sync();
            if (level == 0) {
                total = tot;
                if (total < K1) break; // uniform: too few keys to raise the floor
                b1 = bin;
                above = ab;
            } else {
                const uint32_t B = (b1 << 8) | bin;
                F = B > F ? B : F;
            }
        }
        uint32_t base = 0;
        for (int j = 0; j < cmax; ++j) {
            const uint32_t x = j < c ? lst[j * 64 + lane] : 0u;
            const uint32_t u = word_keys(x);
            const bool keep = j < c && ((u & 0xFFFFu) >= F || (u >> 16) >= F);
            const unsigned long long bal = __ballot(keep);
            if (keep) lst[base + lane_prefix(bal)] = x;   // at or below every unread word
            base += (uint32_t)__popcll(bal);
        }
        wave_lds_sync();
        if (base > 64u * (KS - 4)) {                  // tied at the floor: the radix kernel
            if (lane == 0) sh.over[wv] = 1u;
            F = 0xFFFFu + 0x8000u;                         // no pattern reaches it
            c = 0;
        } else {
            c = base > (uint32_t)lane ? (int)((base - (uint32_t)lane + 63u) >> 6) : 0;
        }
        wp = lane_list + 64 * c;
    };
    // a word (two 16-bit logits) that may hold a key >= F: above +0.0 ...
    auto take_pos = [&](uint32_t x, bool ok, int tp) {
        const s16x2 h = __builtin_bit_cast(s16x2, x);
        const int mx = h.x > h.y ? h.x : h.y;
        if (ok && mx >= tp) {
            *wp = x;
            wp += 64;
        }
    };
    // ... and at or below it
    auto take_neg = [&](uint32_t x, bool ok, uint32_t un) {
        const uint32_t lo = x & 0xFFFFu, hi = x >> 16;
        const uint32_t mn = lo < hi ? lo : hi;
        if (ok && mn <= un) {
            *wp = x;
            wp += 64;
        }
    };
    if (lane == 0) sh.over[wv] = 0u;
    zero_counters(a);
    if (t < 256) hc[t] = 0u;           // the merge's first histogram
    if (t == 0) sh.nk = 0u;

    // the stream: vector t + i * kTK at step i, in groups of four steps; two
    // register buffers alternate, each reloading the group two ahead as soon
    // as it is taken, so a group's loads are in flight while the one before
    // it is taken.  Loads past the row (the last two groups' reloads among
    // them) read its last full vector again and are not taken.
    const int ngroups = 2 * ((nfull + 8 * kTK - 1) / (8 * kTK));   // even
    auto issue = [&](Raw<DT> (&buf)[4], int g) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int v = t + (4 * g + u) * kTK;
            buf[u] = load_raw<DT, VEC>(rp, v < nfull ? v : nfull - 1);
        }
    };
    auto take_group = [&](const Raw<DT> (&buf)[4], int g) {
        if (g == 0 && K1 <= 64u) {     // uniform: a first floor from the first group
            // each lane's largest logit among its first four vectors; if
            // positive, the (top_k + 1)-th largest of the 64 may start the
            // floor (for top_k < 64)
            int lm = -32768;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                if (t + u * kTK < nfull) {
                    const u32x4 q = buf[u].a;
                    const s16x2 h0 = __builtin_bit_cast(s16x2, q.x), h1 = __builtin_bit_cast(s16x2, q.y);
                    const s16x2 h2 = __builtin_bit_cast(s16x2, q.z), h3 = __builtin_bit_cast(s16x2, q.w);
                    lm = max(lm, max(max((int)h0.x, (int)h0.y), max((int)h1.x, (int)h1.y)));
                    lm = max(lm, max(max((int)h2.x, (int)h2.y), max((int)h3.x, (int)h3.y)));
                }
            }
            // the K1-th largest of the 64 lane maxima, bit by bit: K1 different
            // logits are at least that large
            const uint32_t lu = (uint32_t)(lm + 32768);
            uint32_t sel = 0u;
            for (int b = 15; b >= 0; --b) {
                const uint32_t cand = sel | (1u << b);
                if ((uint32_t)__popcll(__ballot(lu >= cand)) >= K1) sel = cand;
            }
            const int mn = (int)sel - 32768;
            if (mn > 0) F = 0x8000u + (uint32_t)mn;
        }
#pragma unroll
        for (int u0 = 0; u0 < 4; u0 += 1) {
            if (__ballot(wp > room)) compact();           // room for a vector
            if (F > 0x8000u) {                            // uniform
                const int tp = (int)F - 0x8000;
#pragma unroll
                for (int u = u0; u < u0 + 1; ++u) {
                    const bool ok = t + (4 * g + u) * kTK < nfull;
                    take_pos(buf[u].a.x, ok, tp);
                    take_pos(buf[u].a.y, ok, tp);
                    take_pos(buf[u].a.z, ok, tp);
                    take_pos(buf[u].a.w, ok, tp);
                }
            } else {
                const uint32_t un = 0x10000u - F;
#pragma unroll
                for (int u = u0; u < u0 + 1; ++u) {
                    const bool ok = t + (4 * g + u) * kTK < nfull;
                    take_neg(buf[u].a.x, ok, un);
                    take_neg(buf[u].a.y, ok, un);
                    take_neg(buf[u].a.z, ok, un);
                    take_neg(buf[u].a.w, ok, un);
                }
            }
        }
    };
    Raw<DT> bufA[4], bufB[4];
    issue(bufA, 0);
    issue(bufB, 1);
    for (int g = 0; g < ngroups; g += 2) {
        take_group(bufA, g);
        issue(bufA, g + 2);            // unconditional: each group waits for its own loads only
        take_group(bufB, g + 1);
        issue(bufB, g + 3);
    }
    if (__ballot(wp > room)) compact();
    if (t == 0) {                      // the partial last vector: at most four words, like a vector,
        const unsigned short* e = reinterpret_cast<const unsigned short*>(rp) + 8LL * nfull;
        const int n = V - 8 * nfull;   // -inf past its end
        for (int j = 0; j < n; j += 2) {
            const uint32_t hi = j + 1 < n ? (uint32_t)e[j + 1] : ninf_bits<DT>();
            const uint32_t x = (uint32_t)e[j] | (hi << 16);
            if (F > 0x8000u) take_pos(x, true, (int)F - 0x8000);
            else take_neg(x, true, 0x10000u - F);
        }
    }
    c = (int)((wp - lane_list) >> 6);
    if (lane == 0) sh.F[wv] = F;
    __syncthreads();

    uint32_t Fg = sh.F[0];
    uint32_t over = sh.over[0];
#pragma unroll
    for (int w = 1; w < kTKW; ++w) {
        Fg = sh.F[w] > Fg ? sh.F[w] : Fg;
        over |= sh.over[w];
    }
    if (over) {
        if (t == 0) a.rows[row] = TruncRow{0.f, 0.f, 0u, 1u};
        return;
    }

    // the keys at or above Fg: a histogram of their high bytes (its total is
    // their number) and the largest
    {
        uint32_t mx_t = 0;
        const int cmax = wave_max_int(c);
        for (int j = 0; j < cmax; ++j) {
            const uint32_t u = j < c ? word_keys(lst[j * 64 + lane]) : 0u;
            const uint32_t k0 = u & 0xFFFFu, k1 = u >> 16;
            if (k0 >= Fg) atomicAdd(&hc[k0 >> 8], 1u);
            if (k1 >= Fg) atomicAdd(&hc[k1 >> 8], 1u);
            mx_t = k0 >= Fg && k0 > mx_t ? k0 : mx_t;
            mx_t = k1 >= Fg && k1 > mx_t ? k1 : mx_t;
        }
        const uint32_t mx = (uint32_t)wave_max_int((int)mx_t);
        if (lane == 0) sh.mx[wv] = mx;
    }
    __syncthreads();
    if (wv == 0) {
        uint32_t bin, above;
        const uint32_t total = find_desc_count(hc, (uint32_t)a.top_k, bin, above);
        if (lane == 0) {
            sh.total = total;
            sh.sel = bin;
            sh.above = above;
        }
    }
    __syncthreads();
    const uint32_t nU = sh.total;
    if (nU == 0u) {                    // every logit -inf
        if (t == 0) a.rows[row] = TruncRow{-INFINITY, -INFINITY, 0u, 0u};
        return;
    }
    uint32_t mxk = sh.mx[0];
#pragma unroll
    for (int w = 1; w < kTKW; ++w) mxk = sh.mx[w] > mxk ? sh.mx[w] : mxk;

    // top-k: the top_k-th largest key at or above Fg, its low byte from a
    // second histogram over the keys with its high byte
    uint32_t lo = Fg;                  // keys >= lo survive top-k
    bool topk_on = Fg > f0 || (uint32_t)a.top_k < nU;
    if (topk_on) {
        const uint32_t b1 = sh.sel;
        const uint32_t need = (uint32_t)a.top_k - (uint32_t)sh.above;
        if (t < 256) hc[t] = 0u;
        __syncthreads();
        for (int j = 0; j < c; ++j) {
            const uint32_t u = word_keys(lst[j * 64 + lane]);
            const uint32_t k0 = u & 0xFFFFu, k1 = u >> 16;
            if (k0 >= Fg && (k0 >> 8) == b1) atomicAdd(&hc[k0 & 255u], 1u);
            if (k1 >= Fg && (k1 >> 8) == b1) atomicAdd(&hc[k1 & 255u], 1u);
        }
        __syncthreads();
        if (wv == 0) {
            uint32_t bin, above;
            find_desc_count(hc, need, bin, above);
            if (lane == 0) sh.sel = bin;
        }
        __syncthreads();
        lo = (b1 << 8) | sh.sel;
    }

    // gather the kept keys
    uint32_t* const kk = sh.whist;
    {
        const int cmax = wave_max_int(c);
        for (int j = 0; j < cmax; ++j) {
            const uint32_t u = j < c ? word_keys(lst[j * 64 + lane]) : 0u;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const uint32_t k = h == 0 ? (u & 0xFFFFu) : (u >> 16);
                const bool keep = k >= lo;     // lo >= f0 > 0: empty slots never kept
                const unsigned long long bal = __ballot(keep);
                if (bal) {
                    const int first = __ffsll((long long)bal) - 1;
                    uint32_t base = 0;
                    if (lane == first) base = atomicAdd(&sh.nk, (uint32_t)__popcll(bal));
                    base = (uint32_t)__builtin_amdgcn_readlane((int)base, first);
                    const uint32_t i = base + lane_prefix(bal);
                    if (keep && i < (uint32_t)kKeptMax) kk[i] = k;
                }
            }
        }
    }
    __syncthreads();
    const uint32_t nk = sh.nk;
    if (nk > (uint32_t)kKeptMax) {     // a tie group too large to gather: the radix kernel
        if (t == 0) a.rows[row] = TruncRow{0.f, 0.f, 0u, 1u};
        return;
    }

    // the kept logits' masses, two keys per thread at most (one with 1024 threads)
    const float m = value_of_key<DT>(mxk);
    const float cc = a.c;
    u64 f[2] = {0, 0};
    uint32_t kt[2] = {0u, 0u};
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int i = t + h * kTK;
        if (i < (int)nk) {
            kt[h] = kk[i];
            f[h] = fixed40_nb(weight(value_of_key<DT>(kt[h]), m, cc));
        }
    }
    {
        const u64 s = lane63_u64(wave_scan_u64(f[0] + f[1]));
        if (lane == 0) sh.red[wv] = s;
    }
    __syncthreads();
    u64 M = 0;
#pragma unroll
    for (int w = 0; w < kTKW; ++w) M += sh.red[w];
    u64 kept = M;
    uint32_t tau = topk_on ? std_key(lo) : 0u;    // top-k off: every key

    // top-p: the key at which the mass from the top first reaches top_p * M
    if (a.top_p < 1.f) {
        const double budget = (double)a.top_p * (double)M;
        uint32_t hi = 0u;
        u64 base = 0;
#pragma unroll
        for (int level = 0; level < 2; ++level) {
            if (t < 256) sh.hist[t] = 0;
            __syncthreads();
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                if (f[h] && (level == 0 || (kt[h] >> 8) == hi))
                    atomicAdd(&sh.hist[level == 0 ? kt[h] >> 8 : kt[h] & 255u], f[h]);
            }
            __syncthreads();
            if (wv == 0) {
                uint32_t bin;
                u64 above;
                find_desc_mass(sh.hist, base, budget, bin, above);
                if (lane == 0) {
                    sh.sel = bin;
                    sh.above = above;                  // the mass of every larger key
                    sh.incl = above + sh.hist[bin];    // and the bin's own
                }
            }
            __syncthreads();
            if (level == 0) {
                hi = sh.sel;
                base = sh.above;
            } else {
                hi = (hi << 8) | sh.sel;
                kept = sh.incl;
            }
            __syncthreads();
        }
        tau = std_key(hi);
    }
    if (t == 0) {
        const float l2s = (float)(log2((double)kept) - (double)kFixBits);
        a.rows[row] = TruncRow{m, l2s, tau, 0u};
    }
}

// ---- one pass for fp32 logits under a small top-k ---------------------------
// k_topk16's design on 32-bit keys, with these differences:
//  - a list entry is one logit (its bits) and the stream test one float
//    comparison against the floor's value;
//  - radix digits are taken from a key's offset above a base (the floor),
//    starting at the top bit of the range the keys span (OffDigits): the high
//    bits of an fp32 key are mostly its exponent, and digits of the key itself
//    would put nearly every candidate in one or two bins, whose LDS atomics
//    then serialise;
//  - a wave raises its floor to the 16-bit offset prefix of the (top_k + 1)-th
//    largest key in its list (the keys with that prefix or a larger one stay:
//    at least top_k + 1 of them), also once more after the stream, so that few
//    keys are above the largest floor;
//  - for top_k < 64 the first floor is the (top_k + 1)-th largest of the
//    wave's 64 lane maxima over its first vectors (that many different
//    logits are at least as large), found one bit at a time with ballots;
//  - after the stream the keys at or above the largest floor are gathered,
//    and one wave finds the top_k-th largest of them and then top-p on the
//    kept masses, with no workgroup barrier.
// Every count, mass and threshold equals the radix passes'.  NT threads take
// one row: 256 (eight workgroups to a CU) when the rows outnumber the compute
// units, else 1024, so that few rows still keep many loads in flight (a
// 32000-logit row is one load per 16 bytes of the workgroup's first round).
// With SPLIT, a 256-thread workgroup takes one slice of a row (split_slices)
// and ends with the slice's candidates (slice_candidates) for k_trunc_merge.

// list entries per lane: 16 with 1024 threads (one workgroup to a CU), 12
// with 256 (eight to a CU)
template <int NT>
constexpr int kS32 = NT == 1024 ? 16 : 12;

template <int NT>
struct Topk32Shared {
    static constexpr int NW = NT / 64;
    uint32_t list[NW * kS32<NT> * 64]; // wave w, lane l, entry j: [w][j * 64 + l]; then the keys >= the floor
    uint32_t whist[NW * 256];           // each wave's histogram while compacting; then wave 0's and the kept keys
    u64 mh[256];                        // wave 0's mass histogram
    uint32_t mx[NW];
    uint32_t F[NW];
    uint32_t over[NW];
    uint32_t nk;
};

__device__ __forceinline__ uint32_t key32(uint32_t x)
{
    return key_of<DT_F32>(__uint_as_float(x));
}

template <bool VEC, int NT, bool SPLIT>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(NT == 256 ? 8 : 4)))
void k_topk32(TruncArgs a)
{
    constexpr int NW = NT / 64;
    constexpr int KS = kS32<NT>;
    static_assert(NW >= 3, "wave 0's histogram and the kept keys fit in the wave histograms");
    __shared__ __attribute__((aligned(16))) Topk32Shared<NT> sh;
    // SPLIT: workgroup (row, slice) streams the slice's whole vectors only
    const int S = SPLIT ? a.slices : 1;
    const int row = SPLIT ? (int)blockIdx.x / S : (int)blockIdx.x;
    const int slice = (int)blockIdx.x - row * S;
    const int t = (int)threadIdx.x;
    const int lane = t & 63, wv = t >> 6;
    const char* const rrow = trunc_row_ptr<DT_F32>(a, row);
    const int V = a.V;
    const int nall = V >> 3;                                   // >= 1
    const int vps = (nall + S - 1) / S;
    const int vb = slice * vps;
    const char* rp = rrow + 32LL * vb;                         // 32 bytes per logical vector
    const int nfull = (vb + vps < nall ? vb + vps : nall) - vb; // >= 1
    const bool last_slice = slice == S - 1;
    const uint32_t K1 = (uint32_t)a.top_k + 1u;
    const uint32_t f0 = key32(0xFF800000u) + 1u;               // just above -inf
    uint32_t* const lst = sh.list + wv * (KS * 64);
    uint32_t* const wh = sh.whist + wv * 256;
    uint32_t F = f0;                   // the wave's floor (uniform) and its value
    float fF = value_of_key32(F);
    uint32_t* const lane_list = lst + lane;
    uint32_t* wp = lane_list;          // this lane's next entry
    uint32_t* const room = lane_list + 64 * (KS - 4);   // beyond: no room for four more
    int c = 0;

    // Raise the floor F to the 16-bit offset prefix of the K1-th largest of
    // the wave's keys at or above it (at least K1 of them stay at or above
    // it), or leave it when they are fewer; key(j) is this lane's j-th key
    // (j < n).  All lanes, uniform.
    auto raise_floor = [&](auto&& key, int n) {
        uint32_t mk = F;
        for (int j = 0; j < n; ++j) {
            const uint32_t k = key(j);
            mk = k > mk ? k : mk;
        }
        const OffDigits od(wave_max_u32(mk) - F);
        uint32_t prefix = 0, need = K1;
        int hs = od.top, ls = od.shift(0);   // level 0 has no prefix
#pragma unroll
        for (int level = 0; level < 2; ++level) {
            reinterpret_cast<u32x4*>(wh)[lane] = u32x4{0u, 0u, 0u, 0u};
            wave_lds_sync();
            for (int j = 0; j < n; ++j) {
                const uint32_t k = key(j), o = k - F;
                if (k >= F && (level == 0 || (o >> hs) == prefix)) atomicAdd(&wh[od.digit(o, level, hs, ls)], 1u);
            }
            wave_lds_sync();
            uint32_t bin, ab;
            const uint32_t tot = find_desc_count(wh, need, bin, ab);
            wave_lds_sync();
            if (level == 0 && tot < K1) break;   // uniform: too few keys to raise the floor
            prefix = (prefix << (hs - ls)) | bin;
            need -= ab;
            if (level == 1 || ls == 0) {
                F += prefix << ls;
                break;
            }
            hs = ls;
            ls = od.shift(1);
        }
    };
    // raise the floor and drop the entries below it; all lanes, uniform
    auto compact = [&]() {
        c = (int)((wp - lane_list) >> 6);
        const int cmax = wave_max_int(c);
        raise_floor([&](int j) { return key32(lst[j * 64 + lane]); }, c);
        uint32_t base = 0;
        for (int j = 0; j < cmax; ++j) {
            const uint32_t x = j < c ? lst[j * 64 + lane] : 0u;
            const bool keep = j < c && key32(x) >= F;
            const unsigned long long bal = __ballot(keep);
            if (keep) lst[base + lane_prefix(bal)] = x;   // at or below every unread entry
            base += (uint32_t)__popcll(bal);
        }
        wave_lds_sync();
        if (base > 64u * (KS - 4)) {                    // tied at the floor: the radix kernel
            if (lane == 0) sh.over[wv] = 1u;
            F = 0xFFFFFFFFu;                               // its value is a NaN: nothing passes
            c = 0;
        } else {
            c = base > (uint32_t)lane ? (int)((base - (uint32_t)lane + 63u) >> 6) : 0;
        }
        wp = lane_list + 64 * c;
        fF = value_of_key32(F);
    };
    // a logit whose key may be >= F: its value is >= F's (-0.0 and +0.0 alike)
    auto take = [&](uint32_t x, bool ok) {
        if (ok && __uint_as_float(x) >= fF) {
            *wp = x;
            wp += 64;
        }
    };
    auto take4 = [&](const u32x4& q, bool ok) {
        if (__ballot(wp > room)) compact();
        take(q.x, ok);
        take(q.y, ok);
        take(q.z, ok);
        take(q.w, ok);
    };
    if (lane == 0) sh.over[wv] = 0u;
    zero_counters(a);
    if (t == 0) sh.nk = 0u;

    // the stream: vector t + i * NT at step i, in groups of two steps; two
    // register buffers alternate as in k_topk16.  With 1024 threads the last
    // two groups are taken after the loop, so that no load is issued past them
    // (the registers they would fill are reused, so the merge would wait for
    // them); with 256 the loop reloads past the row.  A lane's vectors past
    // the row read its last full vector again and are not taken.
    const int ngroups = 2 * ((nfull + 4 * NT - 1) / (4 * NT));   // even
    auto issue = [&](Raw<DT_F32> (&buf)[2], int g) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int v = t + (2 * g + u) * NT;
            buf[u] = load_raw<DT_F32, VEC>(rp, v < nfull ? v : nfull - 1);
        }
    };
    auto take_group = [&](const Raw<DT_F32> (&buf)[2], int g) {
        if (g == 0 && K1 <= 64u) {     // uniform: a first floor from the first group
            // each lane's largest logit among its first two vectors: K1
            // different logits of the row are at least as large as the K1-th
            // largest of the 64, found one bit at a time
            float lm = -INFINITY;
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                if (t + u * NT < nfull) {
                    const u32x4 p = buf[u].a, q = buf[u].b;
                    lm = fmaxf(lm, fmaxf(fmaxf(__uint_as_float(p.x), __uint_as_float(p.y)),
                                         fmaxf(__uint_as_float(p.z), __uint_as_float(p.w))));
                    lm = fmaxf(lm, fmaxf(fmaxf(__uint_as_float(q.x), __uint_as_float(q.y)),
                                         fmaxf(__uint_as_float(q.z), __uint_as_float(q.w))));
                }
            }
            const uint32_t lk = lm > -INFINITY ? key_of<DT_F32>(lm) : 0u;   // 0: below every key
            uint32_t s = 0u;
            for (int b = 31; b >= 0; --b) {
                const uint32_t cand = s | (1u << b);
                if ((uint32_t)__popcll(__ballot(lk >= cand)) >= K1) s = cand;
            }
            if (s > F) {
                F = s;
                fF = value_of_key32(F);
            }
        }
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const bool ok = t + (2 * g + u) * NT < nfull;
            take4(buf[u].a, ok);
            take4(buf[u].b, ok);
        }
    };
    Raw<DT_F32> bufA[2], bufB[2];
    issue(bufA, 0);
    issue(bufB, 1);
    if constexpr (NT == 1024) {
        for (int g = 0; g + 2 < ngroups; g += 2) {
            take_group(bufA, g);
            issue(bufA, g + 2);        // unconditional: each group waits for its own loads only
            take_group(bufB, g + 1);
            issue(bufB, g + 3);
        }
        take_group(bufA, ngroups - 2);
        take_group(bufB, ngroups - 1);
    } else {                           // in 64 registers: one copy of the groups, reloads past the row
        for (int g = 0; g < ngroups; g += 2) {
            take_group(bufA, g);
            issue(bufA, g + 2);
            take_group(bufB, g + 1);
            issue(bufB, g + 3);
        }
    }
    if (__ballot(wp > room)) compact();
    if (last_slice && t < 2) {         // the partial last vector: up to four logits on each of two lanes
        const float* e = reinterpret_cast<const float*>(rrow) + 8LL * nall;
        const int n = V - 8 * nall;
        for (int j = 4 * t; j < n && j < 4 * t + 4; ++j) take(__float_as_uint(e[j]), true);
    }
    c = (int)((wp - lane_list) >> 6);
    uint32_t kr[KS];                 // this lane's keys (0 past its list: below every floor)
#pragma unroll
    for (int j = 0; j < KS; ++j) kr[j] = j < c ? key32(lst[j * 64 + lane]) : 0u;
    // the wave's last floor, raised on its final list: few keys above the
    // largest floor are left for the merge
    if (F != 0xFFFFFFFFu) raise_floor([&](int j) { return kr[j]; }, KS);
    if constexpr (SPLIT) {
        const long long sl = (long long)row * S + slice;
        slice_candidates<NT, KS>(kr, F, K1, S, sh.list, sh.whist, sh.F, sh.mx, sh.over, &sh.nk,
                                 a.cand + sl * kCandMax, a.cand_hdr + sl * 4);
        return;
    }
    {
        uint32_t mx_t = 0;             // the largest key in the lists is the row's
#pragma unroll
        for (int j = 0; j < KS; ++j) mx_t = kr[j] > mx_t ? kr[j] : mx_t;
        const uint32_t mx = wave_max_u32(mx_t);
        if (lane == 0) {
            sh.F[wv] = F;
            sh.mx[wv] = mx;
        }
    }
    __syncthreads();

    uint32_t Fg = sh.F[0], mxk = sh.mx[0];
    uint32_t over = sh.over[0];
#pragma unroll
    for (int w = 1; w < NW; ++w) {
        Fg = sh.F[w] > Fg ? sh.F[w] : Fg;
        mxk = sh.mx[w] > mxk ? sh.mx[w] : mxk;
        over |= sh.over[w];
    }
    if (over) {
        if (t == 0) a.rows[row] = TruncRow{0.f, 0.f, 0u, 1u};
        return;
    }
    if (mxk < Fg) {                    // no key at or above the floor: every logit -inf
        if (t == 0) a.rows[row] = TruncRow{-INFINITY, -INFINITY, 0u, 0u};
        return;
    }

    // gather the keys at or above Fg into the list area (free: every key is
    // in registers); wave 0 then finds both thresholds alone
    uint32_t* const gk = sh.list;
#pragma unroll
    for (int j = 0; j < KS; ++j) {
        const bool keep = kr[j] >= Fg;     // Fg >= f0 > 0: empty slots never kept
        const unsigned long long bal = __ballot(keep);
        if (bal) {
            const int first = __ffsll((long long)bal) - 1;
            uint32_t base = 0;
            if (lane == first) base = atomicAdd(&sh.nk, (uint32_t)__popcll(bal));
            base = (uint32_t)__builtin_amdgcn_readlane((int)base, first);
            if (keep) gk[base + lane_prefix(bal)] = kr[j];
        }
    }
    __syncthreads();
    if (wv != 0) return;
    const uint32_t n = sh.nk;          // >= 1: the row max is among them

    // top-k: the top_k-th largest of the n keys, one digit of its offset from
    // Fg per level; with every finite logit among them (no floor raised) top-k
    // is off for at most top_k of them
    const bool topk_on = Fg > f0 || (uint32_t)a.top_k < n;
    uint32_t lo = Fg;                  // keys >= lo survive top-k
    if (topk_on) {
        const OffDigits od(mxk - Fg);
        uint32_t prefix = 0, need = (uint32_t)a.top_k;
        int hs = od.top, ls = od.shift(0);   // level 0 has no prefix
        for (int level = 0;; ++level) {
            reinterpret_cast<u32x4*>(wh)[lane] = u32x4{0u, 0u, 0u, 0u};
            wave_lds_sync();
            for (uint32_t i0 = 0; i0 < n; i0 += 256) {   // four reads in flight per lane
                uint32_t q[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const uint32_t i = i0 + (uint32_t)(lane + 64 * u);
                    q[u] = i < n ? gk[i] : 0u;
                }
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const uint32_t o = q[u] - Fg;
                    if (q[u] >= Fg && (level == 0 || (o >> hs) == prefix))
                        atomicAdd(&wh[od.digit(o, level, hs, ls)], 1u);
                }
            }
            wave_lds_sync();
            uint32_t bin, above;
            find_desc_count(wh, need, bin, above);
            wave_lds_sync();
            prefix = (prefix << (hs - ls)) | bin;
            need -= above;
            if (ls == 0) break;
            hs = ls;
            ls = od.shift(level + 1);
        }
        lo = Fg + prefix;
    }

    // the kept keys (at most kKeptMax, else the row goes to the radix kernel)
    uint32_t* const kk = sh.whist + 256;
    uint32_t nk = 0;
    for (uint32_t i0 = 0; i0 < n; i0 += 64) {
        const uint32_t i = i0 + (uint32_t)lane;
        const uint32_t k = i < n ? gk[i] : 0u;
        const bool keep = k >= lo;     // lo >= f0 > 0
        const unsigned long long bal = __ballot(keep);
        const uint32_t pos = nk + lane_prefix(bal);
        if (keep && pos < (uint32_t)kKeptMax) kk[pos] = k;
        nk += (uint32_t)__popcll(bal);
    }
    if (nk > (uint32_t)kKeptMax) {     // a tie group too large to gather
        if (t == 0) a.rows[row] = TruncRow{0.f, 0.f, 0u, 1u};
        return;
    }
    wave_lds_sync();

    // the kept logits' masses, eight keys per lane at most, and the kept
    // mass; top-p: the key at which the mass from the top first reaches top_p
    // of it, one digit of its offset from lo per level
    constexpr int H = kKeptMax / 64;
    const float m = value_of_key32(mxk);
    const float cc = a.c;
    u64 f[H];
    uint32_t kt[H];
    u64 fs = 0;
#pragma unroll
    for (int h = 0; h < H; ++h) {
        const uint32_t i = (uint32_t)(lane + 64 * h);
        kt[h] = i < nk ? kk[i] : 0u;
        f[h] = i < nk ? fixed40_nb(weight(value_of_key32(kt[h]), m, cc)) : 0;
        fs += f[h];
    }
    u64 kept = lane63_u64(wave_scan_u64(fs));
    uint32_t tau = topk_on ? lo : 0u;  // top-k off: every key
    if (a.top_p < 1.f) {
        const double budget = (double)a.top_p * (double)kept;
        u64* const hm = sh.mh;
        const OffDigits od(mxk - lo);  // the kept keys: lo .. mxk
        uint32_t prefix = 0u;
        u64 base = 0;
        int hs = od.top, ls = od.shift(0);   // level 0 has no prefix
        for (int level = 0;; ++level) {
            reinterpret_cast<u32x4*>(hm)[2 * lane] = u32x4{0u, 0u, 0u, 0u};
            reinterpret_cast<u32x4*>(hm)[2 * lane + 1] = u32x4{0u, 0u, 0u, 0u};
            wave_lds_sync();
#pragma unroll
            for (int h = 0; h < H; ++h) {
                const uint32_t o = kt[h] - lo;
                if (f[h] && (level == 0 || (o >> hs) == prefix))
                    atomicAdd(&hm[od.digit(o, level, hs, ls)], f[h]);
            }
            wave_lds_sync();
            uint32_t bin;
            u64 above;
            find_desc_mass(hm, base, budget, bin, above);
            kept = above + hm[bin];    // the mass of every larger key and the bin's own
            base = above;
            prefix = (prefix << (hs - ls)) | bin;
            wave_lds_sync();
            if (ls == 0) break;
            hs = ls;
            ls = od.shift(level + 1);
        }
        tau = lo + prefix;
    }
    if (t == 0) {
        const float l2s = (float)(log2((double)kept) - (double)kFixBits);
        a.rows[row] = TruncRow{m, l2s, tau, 0u};
    }
}

// ---- the merge of a row's slices ---------------------------------------------
// fp32 rows cut into slices (split_slices > 1, top-k of at most 256): every
// key of a row at or above the largest floor Fr of its slices is among the
// slices' candidates, and Fr never passes the row's top_k-th largest key.
// One 512-thread workgroup per row gathers them and finds the top_k-th
// largest, the kept keys' fixed-point masses and the top-p boundary as the
// one-pass kernels do (the same integers, so the same summary); a row whose
// slices overflowed, or with more candidates or kept keys than it can
// gather, takes the radix passes in the same workgroup.

struct MergeShared {
    uint32_t hdr[kSplitMax][4];
    uint32_t pre[kSplitMax];           // the slices' candidate counts, exclusive prefix
    uint32_t total;
    uint32_t keys[kMergeMax];
    uint32_t kk[kKeptMax];
    uint32_t hc[256];
    u64 hm[256];
    u64 red[kTW];
    uint32_t nk;
    uint32_t nkept;
    uint32_t sel;
    uint32_t above;
    u64 mabove;
    u64 incl;
};

// One row's summary from its slices' candidates at or above Fr; false (uniform
// over the workgroup) when there are more candidates or kept keys than it
// gathers.
__device__ __forceinline__ bool merge_row(const TruncArgs& a, int row, uint32_t Fr, uint32_t mxk,
                                          const uint32_t* cand, MergeShared& ms)
{
    const int t = (int)threadIdx.x;
    const int lane = t & 63, wv = t >> 6;
    const int S = a.slices;
    const uint32_t f0 = key32(0xFF800000u) + 1u;               // just above -inf
    if (mxk < Fr) {                    // no finite logit
        if (t == 0) a.rows[row] = TruncRow{-INFINITY, -INFINITY, 0u, 0u};
        return true;
    }

    // the candidates at or above Fr: candidate i of the row is entry i - pre[s]
    // of slice s, the last slice with pre[s] <= i; every load of a round is
    // issued before the first is used
    if (wv == 0) {
        const uint32_t c = lane < S ? ms.hdr[lane][2] : 0u;
        const uint32_t inc = (uint32_t)wave_scan_u64(c);
        if (lane < S) ms.pre[lane] = inc - c;
        if (lane == 63) ms.total = inc;
    }
    __syncthreads();
    const uint32_t total = ms.total;   // at most kSplitMax * kCandMax
    constexpr int R = 8;
    for (uint32_t i0 = 0; i0 < total; i0 += R * kTB) {
        uint32_t q[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const uint32_t i = i0 + (uint32_t)(t + r * kTB);
            int s0 = 0, s1 = S - 1;    // pre[0] = 0 <= i
            while (s0 < s1) {
                const int mid = (s0 + s1 + 1) >> 1;
                if (ms.pre[mid] <= i) s0 = mid;
                else s1 = mid - 1;
            }
            q[r] = i < total ? cand[(long long)s0 * kCandMax + (i - ms.pre[s0])] : 0u;
        }
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const bool keep = q[r] >= Fr;   // Fr >= f0 > 0: past the end never kept
            const unsigned long long bal = __ballot(keep);
            if (bal) {
                const int first = __ffsll((long long)bal) - 1;
                uint32_t base = 0;
                if (lane == first) base = atomicAdd(&ms.nk, (uint32_t)__popcll(bal));
                base = (uint32_t)__builtin_amdgcn_readlane((int)base, first);
                const uint32_t pos = base + lane_prefix(bal);
                if (keep && pos < (uint32_t)kMergeMax) ms.keys[pos] = q[r];
            }
        }
    }
    __syncthreads();
    const uint32_t n = ms.nk;
    if (n > (uint32_t)kMergeMax) return false;

    // top-k: the top_k-th largest of the n keys, one offset digit per level;
    // with every finite logit among them (no floor raised) top-k is off for
    // at most top_k of them
    const bool topk_on = Fr > f0 || (uint32_t)a.top_k < n;
    uint32_t lo = Fr;                  // keys >= lo survive top-k
    if (topk_on) {
        const OffDigits od(mxk - Fr);
        uint32_t prefix = 0, need = (uint32_t)a.top_k;
        int hs = od.top, ls = od.shift(0);   // level 0 has no prefix
        for (int level = 0;; ++level) {
            if (t < 256) ms.hc[t] = 0u;      // read by the last find, before the last barrier
            __syncthreads();
            for (uint32_t i = (uint32_t)t; i < n; i += kTB) {
                const uint32_t o = ms.keys[i] - Fr;
                if (level == 0 || (o >> hs) == prefix) atomicAdd(&ms.hc[od.digit(o, level, hs, ls)], 1u);
            }
            __syncthreads();
            if (wv == 0) {
                uint32_t bin, above;
                find_desc_count(ms.hc, need, bin, above);
                if (lane == 0) {
                    ms.sel = bin;
                    ms.above = above;
                }
            }
            __syncthreads();
            prefix = (prefix << (hs - ls)) | ms.sel;   // rewritten two barriers later
            need -= ms.above;
            if (ls == 0) break;
            hs = ls;
            ls = od.shift(level + 1);
        }
        lo = Fr + prefix;
    }

    // the kept keys
    for (uint32_t i0 = 0; i0 < n; i0 += kTB) {
        const uint32_t i = i0 + (uint32_t)t;
        const uint32_t k = i < n ? ms.keys[i] : 0u;
        const bool keep = k >= lo;     // lo >= f0 > 0
        const unsigned long long bal = __ballot(keep);
        if (bal) {
            const int first = __ffsll((long long)bal) - 1;
            uint32_t base = 0;
            if (lane == first) base = atomicAdd(&ms.nkept, (uint32_t)__popcll(bal));
            base = (uint32_t)__builtin_amdgcn_readlane((int)base, first);
            const uint32_t pos = base + lane_prefix(bal);
            if (keep && pos < (uint32_t)kKeptMax) ms.kk[pos] = k;
        }
    }
    __syncthreads();
    const uint32_t nk = ms.nkept;
    if (nk > (uint32_t)kKeptMax) return false;

    // the kept logits' masses, one per thread
    const float m = value_of_key32(mxk);
    const uint32_t kt = t < (int)nk ? ms.kk[t] : 0u;
    const u64 f = t < (int)nk ? fixed40_nb(weight(value_of_key32(kt), m, a.c)) : 0;
    u64 kept = block_sum_u64(f, ms.red);
    const u64 M = kept;
    uint32_t tau = topk_on ? lo : 0u;  // top-k off: every key

    // top-p: the key at which the mass from the top first reaches top_p * M
    if (a.top_p < 1.f) {
        const double budget = (double)a.top_p * (double)M;
        const OffDigits od(mxk - lo);  // the kept keys: lo .. mxk
        uint32_t prefix = 0u;
        u64 base = 0;
        int hs = od.top, ls = od.shift(0);   // level 0 has no prefix
        for (int level = 0;; ++level) {
            if (t < 256) ms.hm[t] = 0;
            __syncthreads();
            const uint32_t o = kt - lo;
            if (f && (level == 0 || (o >> hs) == prefix)) atomicAdd(&ms.hm[od.digit(o, level, hs, ls)], f);
            __syncthreads();
            if (wv == 0) {
                uint32_t bin;
                u64 above;
                find_desc_mass(ms.hm, base, budget, bin, above);
                if (lane == 0) {
                    ms.sel = bin;
                    ms.mabove = above;                 // the mass of every larger key
                    ms.incl = above + ms.hm[bin];      // and the bin's own
                }
            }
            __syncthreads();
            prefix = (prefix << (hs - ls)) | ms.sel;   // rewritten two barriers later
            base = ms.mabove;
            kept = ms.incl;
            if (ls == 0) break;
            hs = ls;
            ls = od.shift(level + 1);
        }
        tau = lo + prefix;
    }
    if (t == 0) {
        const float l2s = (float)(log2((double)kept) - (double)kFixBits);
        a.rows[row] = TruncRow{m, l2s, tau, 0u};
    }
    return true;
}

template <bool VEC>
__global__ __launch_bounds__(kTB) void k_trunc_merge(TruncArgs a)
{
    static_assert(kKeptMax == kTB, "one kept key per thread");
    static_assert(4 * kSplitMax <= kTB, "one header word per thread");
    __shared__ Shared sh;              // the radix passes
    __shared__ __attribute__((aligned(16))) MergeShared ms;
    const int row = (int)blockIdx.x;
    const int t = (int)threadIdx.x;
    const int S = a.slices;
    const uint32_t* const hdr = a.cand_hdr + (long long)row * S * 4;
    const uint32_t* const cand = a.cand + (long long)row * S * kCandMax;
    if (t < 4 * S) ms.hdr[t >> 2][t & 3] = hdr[t];
    if (t == 0) {
        ms.nk = 0u;
        ms.nkept = 0u;
    }
    __syncthreads();
    uint32_t Fr = 0u, mxk = 0u, over = 0u;
    for (int sl = 0; sl < S; ++sl) {
        Fr = ms.hdr[sl][0] > Fr ? ms.hdr[sl][0] : Fr;
        mxk = ms.hdr[sl][1] > mxk ? ms.hdr[sl][1] : mxk;
        over |= ms.hdr[sl][3];
    }
    if (!over && merge_row(a, row, Fr, mxk, cand, ms)) return;
    // the slices overflowed, or too many candidates or kept keys: the radix passes
    trunc_row_radix<DT_F32>(a, row, sh, StreamRow<DT_F32, VEC>{trunc_row_ptr<DT_F32>(a, row), a.V});
}

// The current device's compute units (queried once per device).
int compute_units()
{
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (!cached[dev]) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1) n = 256;
        cached[dev] = n;
    }
    return cached[dev];
}

template <int DT>
hipError_t launch_dt(bool vec, const TruncArgs& a, hipStream_t st)
{
    TruncArgs b = a;
    b.only_marked = 0;
    void* args[] = {&b};
    const void* marked = vec ? reinterpret_cast<const void*>(k_trunc_rows<DT, true>)
                             : reinterpret_cast<const void*>(k_trunc_rows<DT, false>);
    // rows the one-pass kernels could not summarise (pad = 1): 65536 or more
    // equal finite 16-bit logits (k_trunc16), or too many tied at a list's
    // floor (k_topk16, k_topk32)
    auto run_marked = [&]() {
        b.only_marked = 1;
        const int blocks = (a.n_rows + kTB - 1) / kTB;
        const unsigned grid = (unsigned)(blocks < 1024 ? blocks : 1024);
        return hipLaunchKernel(marked, dim3(grid), dim3(kTB), args, 0, st);
    };
    const bool small_topk = a.top_k >= 1 && a.top_k <= kTopkMax && a.top_k < a.V;
    if constexpr (DT == DT_F32) {
        // few rows under a small top-k: cut into slices, each summarised by its
        // own workgroup, merged per row (the merge also runs the radix passes
        // for rows a slice could not summarise)
        if (small_topk && a.V >= 8 && a.slices > 1 && a.cand && a.cand_hdr) {
            const void* f = vec ? reinterpret_cast<const void*>(k_topk32<true, 256, true>)
                                : reinterpret_cast<const void*>(k_topk32<false, 256, true>);
            const hipError_t e = hipLaunchKernel(f, dim3((unsigned)(a.n_rows * a.slices)), dim3(256), args, 0, st);
            if (e != hipSuccess) return e;
            const void* g = vec ? reinterpret_cast<const void*>(k_trunc_merge<true>)
                                : reinterpret_cast<const void*>(k_trunc_merge<false>);
            return hipLaunchKernel(g, dim3((unsigned)a.n_rows), dim3(kTB), args, 0, st);
        }
        if (small_topk && a.V >= 8) {
            const bool wide = a.n_rows <= compute_units();   // few rows: 1024 threads each
            const void* f = wide ? (vec ? reinterpret_cast<const void*>(k_topk32<true, 1024, false>)
                                        : reinterpret_cast<const void*>(k_topk32<false, 1024, false>))
                                 : (vec ? reinterpret_cast<const void*>(k_topk32<true, 256, false>)
                                        : reinterpret_cast<const void*>(k_topk32<false, 256, false>));
            const hipError_t e = hipLaunchKernel(f, dim3((unsigned)a.n_rows), dim3(wide ? 1024 : 256), args, 0, st);
            return e != hipSuccess ? e : run_marked();
        }
        const bool in_lds = a.V <= kLdsRowMax;
        const void* f = in_lds ? (vec ? reinterpret_cast<const void*>(k_trunc_rows_lds<true>)
                                      : reinterpret_cast<const void*>(k_trunc_rows_lds<false>))
                               : (vec ? reinterpret_cast<const void*>(k_trunc_rows<DT, true>)
                                      : reinterpret_cast<const void*>(k_trunc_rows<DT, false>));
        return hipLaunchKernel(f, dim3((unsigned)a.n_rows), dim3(kTB), args, 0, st);
    } else {
        if (a.V < 8)                   // no whole vector: the radix kernel takes every row
            return hipLaunchKernel(marked, dim3((unsigned)a.n_rows), dim3(kTB), args, 0, st);
        hipError_t e;
        const int cus = compute_units();
        // a small top-k on many rows: the candidate lists; on fewer, the
        // histogram pass (no compaction in its stream) is the faster
        if (small_topk && (long long)a.n_rows > (long long)kListRowsPerCU * cus) {
            const void* f = vec ? reinterpret_cast<const void*>(k_topk16<DT, true>)
                                : reinterpret_cast<const void*>(k_topk16<DT, false>);
            e = hipLaunchKernel(f, dim3((unsigned)a.n_rows), dim3(kTK), args, 0, st);
        } else {
            const void* f = vec ? reinterpret_cast<const void*>(k_trunc16<DT, true>)
                                : reinterpret_cast<const void*>(k_trunc16<DT, false>);
            const unsigned g16 = (unsigned)(a.n_rows < cus ? a.n_rows : cus);   // one workgroup fills a CU's LDS
            e = hipLaunchKernel(f, dim3(g16), dim3(kT16), args, 0, st);
        }
        return e != hipSuccess ? e : run_marked();
    }
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
