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
// Two kernels find tau and the kept mass:
//  - k_trunc16 (fp16 / bf16 rows): one pass per row, an exact count of all
//    65536 bit patterns in LDS, the thresholds read off the histogram;
//  - k_trunc_rows (fp32 rows, and the rare 16-bit row the histogram cannot
//    hold): radix selection on the key, most significant digit first (11, 11
//    and 10 bits for fp32 keys; 11 then 5 for 16-bit keys), one 512-thread
//    workgroup per row streaming the row once per digit (the first pass from
//    HBM, the rest mostly from cache) and histogramming the next digit of the
//    keys that share the prefix chosen so far: counts for top-k, masses for
//    top-p.
// Masses are fixed-point integers (w * 2^40, truncated), summed with integer
// atomics and integer reductions, so every result is independent of
// scheduling and bitwise reproducible, and both kernels give the same
// integers for the same row.

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
__device__ void trunc_row_radix(const TruncArgs& a, int row, Shared& sh)
{
    using D = Digits<DT>;
    constexpr int ES = DT == DT_F32 ? 4 : 2;
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
    __syncthreads();                   // the shared state is reused by the next row
}

// Rows blockIdx.x, blockIdx.x + gridDim.x, ...; with only_marked, just the
// rows the one-pass kernel marked (pad = 1): the workgroup reads the marks of
// kTB rows at once (rows blockIdx.x * kTB + i, then gridDim.x * kTB further)
// and runs the marked ones.
template <int DT, bool VEC>
__global__ __launch_bounds__(kTB) void k_trunc_rows(TruncArgs a)
{
    __shared__ Shared sh;
    __shared__ int marked[kTB];
    __shared__ int n_marked;
    if (!a.only_marked) {
        for (int row = blockIdx.x; row < a.n_rows; row += gridDim.x) trunc_row_radix<DT, VEC>(a, row, sh);
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
        for (int i = 0; i < n; ++i) trunc_row_radix<DT, VEC>(a, marked[i], sh);
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

struct Scratch16 {
    uint32_t cnt[kChunks];             // chunk counts, by chunk position
    u64 mass[kChunks];                 // chunk masses, by chunk position
    u64 gmass[kW16];                   // masses of 64-chunk groups
    uint32_t wcnt[kW16];
    int wmin[kW16];
    uint32_t d;
    uint32_t dk;
    u64 incl;
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

// Persistent: workgroup g takes rows g, g + gridDim.x, ...  While it
// analyses one row, the first round of its next row is already loading.
template <int DT, bool VEC>
__global__ __launch_bounds__(kT16) void k_trunc16(TruncArgs a)
{
    constexpr int ES = 2;
    constexpr int kAhead = 4;          // vectors per thread loaded ahead
    __shared__ __attribute__((aligned(16))) uint32_t hist[kWords];
    __shared__ __attribute__((aligned(16))) Scratch16 sc;
    const int V = a.V;
    const int t = (int)threadIdx.x;
    const int lane = t & 63, wv = t >> 6;
    const int nfull = V >> 3;
    u32x4* h4 = reinterpret_cast<u32x4*>(hist);
    auto row_of = [&](int r) -> const char* {
        return r < a.n_target_rows ? row_ptr(a.target, r, a.t_stride, ES)
                                   : row_ptr(a.draft, r - a.n_target_rows, a.d_stride, ES);
    };

    Raw<DT> ahead[kAhead];
    int row = blockIdx.x;
    if (row < a.n_rows) {
        const char* rp = row_of(row);
#pragma unroll
        for (int u = 0; u < kAhead; ++u)
            if (t + u * kT16 < nfull) ahead[u] = load_raw<DT, VEC>(rp, t + u * kT16);
    }
    // The histogram is zeroed once here; after each row, only the chunks that
    // row touched are zeroed again, each by the thread that summed it.
    for (int i = t; i < kWords / 4; i += kT16) h4[i] = u32x4{0u, 0u, 0u, 0u};
    for (; row < a.n_rows; row += gridDim.x) {
    const char* rp = row_of(row);
    __syncthreads();

    // the pass: count every pattern (the first kAhead vectors are already here)
#pragma unroll
    for (int u = 0; u < kAhead; ++u) {
        if (t + u * kT16 < nfull) {
            count_word(hist, ahead[u].a.x);
            count_word(hist, ahead[u].a.y);
            count_word(hist, ahead[u].a.z);
            count_word(hist, ahead[u].a.w);
        }
    }
    int v = t + kAhead * kT16;
    for (; v + 3 * kT16 < nfull; v += 4 * kT16) {
        Raw<DT> r[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) r[u] = load_raw<DT, VEC>(rp, v + u * kT16);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            count_word(hist, r[u].a.x);
            count_word(hist, r[u].a.y);
            count_word(hist, r[u].a.z);
            count_word(hist, r[u].a.w);
        }
    }
    for (; v < nfull; v += kT16) {
        const Raw<DT> r = load_raw<DT, VEC>(rp, v);
        count_word(hist, r.a.x);
        count_word(hist, r.a.y);
        count_word(hist, r.a.z);
        count_word(hist, r.a.w);
    }
    if (t == nfull % kT16 && 8 * nfull < V) {   // the partial last vector: one thread
        const unsigned short* e = reinterpret_cast<const unsigned short*>(rp) + 8LL * nfull;
        for (int j = 0; j < V - 8 * nfull; ++j) {
            const uint32_t b = e[j];
            atomicAdd(&hist[b >> 1], (b & 1u) * 0xFFFFu + 1u);
        }
    }
    // the next row's first vectors load during the analysis
    {
        const int nrow = row + (int)gridDim.x;
        if (nrow < a.n_rows) {
            const char* np = row_of(nrow);
#pragma unroll
            for (int u = 0; u < kAhead; ++u)
                if (t + u * kT16 < nfull) ahead[u] = load_raw<DT, VEC>(np, t + u * kT16);
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
    sc.cnt[cp] = my_cnt;
    const uint32_t fin_cnt = bc == (int)(ninf_bits<DT>() >> 6) ? my_cnt - ninf : my_cnt;
    {
        const uint32_t wt = lane63_u32(wave_scan_u32(my_cnt));
        const unsigned long long ne = __ballot(fin_cnt != 0u);
        if (lane == 0) {
            sc.wcnt[wv] = wt;
            sc.wmin[wv] = ne ? 16 * (__ffsll((long long)ne) - 1) + wv : INT32_MAX;
        }
    }
    __syncthreads();
    uint32_t total = 0;
    int cmax = INT32_MAX;
#pragma unroll
    for (int i = 0; i < kW16; ++i) {
        total += sc.wcnt[i];
        cmax = min(cmax, sc.wmin[i]);
    }
    // after every reader of the row's histogram is done: zero this thread's chunk
    auto clear_chunk = [&]() {
        __syncthreads();
        if (dirty) {
#pragma unroll
            for (int g = 0; g < 8; ++g) cw[(g + lane) & 7] = u32x4{0u, 0u, 0u, 0u};
        }
    };
    if (total != (uint32_t)V) {        // a half overflowed: leave the row to the radix kernel
        if (t == 0) a.rows[row] = TruncRow{0.f, 0.f, 0u, 1u};
        clear_chunk();
        continue;
    }
    const uint32_t finite = total - ninf;
    if (finite == 0) {                 // every logit is -inf
        if (t == 0) a.rows[row] = TruncRow{-INFINITY, -INFINITY, 0u, 0u};
        clear_chunk();
        continue;
    }

    // wave 0: the max (first nonempty position of chunk cmax), then top-k
    if (wv == 0) {
        {
            const uint32_t d = 64u * cmax + lane;
            const uint32_t b = bits_at(d);
            const bool nz = b != ninf_bits<DT>() && count_bits<DT>(hist, b, negzero) != 0u;
            const unsigned long long hit = __ballot(nz);
            if (lane == 0) sc.d = 64u * cmax + (uint32_t)(__ffsll((long long)hit) - 1);
        }
        uint32_t dk = 65535u;          // positions <= dk survive top-k
        if (a.top_k >= 1 && (uint32_t)a.top_k < finite) {
            const uint32_t need = (uint32_t)a.top_k;
            uint32_t base = 0;
            int ch = -1;
            for (int g = 0; g < kChunks / 64 && ch < 0; ++g) {   // uniform across the wave
                const uint32_t x = sc.cnt[64 * g + lane];
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
            if (ch < 0) ch = kChunks - 1;                 // unreachable: top_k < finite
            const uint32_t d = 64u * ch + lane;
            const uint32_t incl = base + wave_scan_u32(count_bits<DT>(hist, bits_at(d), negzero));
            const unsigned long long hit = __ballot(incl >= need);
            dk = 64u * ch + (uint32_t)(__ffsll((long long)hit) - 1);
        }
        if (lane == 0) sc.dk = dk;
    }
    __syncthreads();
    const float m = value_of_bits<DT>(bits_at(sc.d));
    const float c = a.c;
    const uint32_t dk = sc.dk;

    // masses of the chunks (positions <= dk), one wave per chunk, each wave
    // taking the nonempty chunks its own threads summed
    auto mass_at = [=](uint32_t d) -> u64 {
        if (d > dk) return 0;
        const uint32_t b = bits_at(d);
        const uint32_t n = count_bits<DT>(hist, b, negzero);
        return n ? (u64)n * fixed40(weight(value_of_bits<DT>(b), m, c)) : 0;
    };
    {
        sc.mass[cp] = 0;
        unsigned long long todo = __ballot(fin_cnt != 0 && (uint32_t)cp <= (dk >> 6));
        while (todo) {
            const int bit = __ffsll((long long)todo) - 1;
            todo &= todo - 1;
            const int ch = 16 * bit + wv;
            const u64 mk = lane63_u64(wave_scan_u64(mass_at(64u * ch + lane)));
            if (lane == 0) sc.mass[ch] = mk;
        }
    }
    __syncthreads();
    // group totals: wave w sums chunk positions 64w .. 64w + 63
    {
        const u64 gt = lane63_u64(wave_scan_u64(sc.mass[64 * wv + lane]));
        if (lane == 0) sc.gmass[wv] = gt;
    }
    __syncthreads();
    // every wave: the group totals as a scan over lanes 0..15
    const u64 gm = lane < kW16 ? sc.gmass[lane] : 0;
    const u64 ginc = wave_scan_u64(gm);
    const u64 M = lane63_u64(ginc);
    u64 kept = M;
    uint32_t dtau = dk;
    if (a.top_p < 1.f) {
        const double budget = (double)a.top_p * (double)M;
        // the group, then the chunk, then the position where budget is reached
        const unsigned long long ghit = __ballot(lane < kW16 && (double)ginc >= budget);
        const int G = ghit ? __ffsll((long long)ghit) - 1 : kW16 - 1;
        const u64 gbase = readlane_u64(ginc - gm, G);
        if (wv == G) {
            const u64 x = sc.mass[64 * G + lane];
            const u64 incl = gbase + wave_scan_u64(x);
            const unsigned long long hit = __ballot((double)incl >= budget);
            const int f = hit ? __ffsll((long long)hit) - 1 : 63;
            const int ch = 64 * G + f;
            const u64 excl_f = readlane_u64(incl - x, f);
            const uint32_t d = 64u * ch + lane;
            const u64 mk = mass_at(d);
            const u64 incl2 = excl_f + wave_scan_u64(mk);
            const unsigned long long hit2 = __ballot((double)incl2 >= budget);
            const int f2 = hit2 ? __ffsll((long long)hit2) - 1 : 63;
            if (lane == f2) {
                sc.d = d;
                sc.incl = incl2;
            }
        }
        __syncthreads();
        dtau = sc.d;
        kept = sc.incl;
    }
    if (t == 0) {
        const float l2s = (float)(log2((double)kept) - (double)kFixBits);
        a.rows[row] = TruncRow{m, l2s, 65535u - dtau, 0u};
    }
    clear_chunk();
    }
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
    if constexpr (DT == DT_F32) {
        const void* f = vec ? reinterpret_cast<const void*>(k_trunc_rows<DT, true>)
                            : reinterpret_cast<const void*>(k_trunc_rows<DT, false>);
        return hipLaunchKernel(f, dim3((unsigned)a.n_rows), dim3(kTB), args, 0, st);
    } else {
        const void* f = vec ? reinterpret_cast<const void*>(k_trunc16<DT, true>)
                            : reinterpret_cast<const void*>(k_trunc16<DT, false>);
        const int cus = compute_units();
        const unsigned g16 = (unsigned)(a.n_rows < cus ? a.n_rows : cus);   // one workgroup fills a CU's LDS
        hipError_t e = hipLaunchKernel(f, dim3(g16), dim3(kT16), args, 0, st);
        if (e != hipSuccess) return e;
        // rows with 65536 or more equal finite logits
        b.only_marked = 1;
        const void* g = vec ? reinterpret_cast<const void*>(k_trunc_rows<DT, true>)
                            : reinterpret_cast<const void*>(k_trunc_rows<DT, false>);
        const int blocks = (a.n_rows + kTB - 1) / kTB;
        const unsigned grid = (unsigned)(blocks < 1024 ? blocks : 1024);
        return hipLaunchKernel(g, dim3(grid), dim3(kTB), args, 0, st);
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
