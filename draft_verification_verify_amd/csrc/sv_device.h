// sv_device.h -- device-side building blocks of libspecverify.so: loading
// logical 8-element vectors of a logit row, and workgroup reductions/scans in
// a fixed order (so every result is reproducible bit for bit).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "sv_launch.h"

namespace sv {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// ---- element decoding ------------------------------------------------------
// bf16 -> f32 is exact: the bf16 bits are the high half of the f32.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float f16_bits(uint32_t h)
{
    return (float)__builtin_bit_cast(_Float16, (unsigned short)(h & 0xffffu));
}

template <int DT>
__device__ __forceinline__ float load_elem(const char* row, long long i)
{
    if constexpr (DT == DT_F32) {
        return reinterpret_cast<const float*>(row)[i];
    } else if constexpr (DT == DT_BF16) {
        return bf16_lo(reinterpret_cast<const unsigned short*>(row)[i]);
    } else {
        return f16_bits(reinterpret_cast<const unsigned short*>(row)[i]);
    }
}

// The raw bits of one logical vector (8 elements).
template <int DT>
struct Raw {
    u32x4 a;
    u32x4 b;                           // used by fp32 only
};

// Load logical vector v (elements 8v .. 8v+7, all inside the row).  VEC: the
// row is 16-byte aligned and the vector is one (two for fp32) 16-byte
// non-temporal loads; otherwise element loads.
template <int DT, bool VEC>
__device__ __forceinline__ Raw<DT> load_raw(const char* row, int v)
{
    Raw<DT> r;
    if constexpr (VEC) {
        if constexpr (DT == DT_F32) {
            const u32x4* p = reinterpret_cast<const u32x4*>(row) + 2 * v;
            r.a = __builtin_nontemporal_load(p);
            r.b = __builtin_nontemporal_load(p + 1);
        } else {
            const u32x4* p = reinterpret_cast<const u32x4*>(row) + v;
            r.a = __builtin_nontemporal_load(p);
        }
    } else {
        if constexpr (DT == DT_F32) {
            const uint32_t* p = reinterpret_cast<const uint32_t*>(row) + 8 * (long long)v;
            r.a = u32x4{p[0], p[1], p[2], p[3]};
            r.b = u32x4{p[4], p[5], p[6], p[7]};
        } else {
            const unsigned short* p = reinterpret_cast<const unsigned short*>(row) + 8 * (long long)v;
            r.a = u32x4{p[0] | ((uint32_t)p[1] << 16), p[2] | ((uint32_t)p[3] << 16),
                        p[4] | ((uint32_t)p[5] << 16), p[6] | ((uint32_t)p[7] << 16)};
        }
    }
    return r;
}

// The same with ordinary (cached) loads, for rows that are read again soon.
template <int DT, bool VEC>
__device__ __forceinline__ Raw<DT> load_raw_cached(const char* row, int v)
{
    if constexpr (VEC) {
        Raw<DT> r;
        if constexpr (DT == DT_F32) {
            const u32x4* p = reinterpret_cast<const u32x4*>(row) + 2 * v;
            r.a = p[0];
            r.b = p[1];
        } else {
            r.a = reinterpret_cast<const u32x4*>(row)[v];
        }
        return r;
    } else {
        return load_raw<DT, false>(row, v);
    }
}

template <int DT>
__device__ __forceinline__ void decode(const Raw<DT>& r, float* e)
{
    if constexpr (DT == DT_F32) {
        e[0] = __uint_as_float(r.a.x); e[1] = __uint_as_float(r.a.y);
        e[2] = __uint_as_float(r.a.z); e[3] = __uint_as_float(r.a.w);
        e[4] = __uint_as_float(r.b.x); e[5] = __uint_as_float(r.b.y);
        e[6] = __uint_as_float(r.b.z); e[7] = __uint_as_float(r.b.w);
    } else if constexpr (DT == DT_BF16) {
        e[0] = bf16_lo(r.a.x); e[1] = bf16_hi(r.a.x);
        e[2] = bf16_lo(r.a.y); e[3] = bf16_hi(r.a.y);
        e[4] = bf16_lo(r.a.z); e[5] = bf16_hi(r.a.z);
        e[6] = bf16_lo(r.a.w); e[7] = bf16_hi(r.a.w);
    } else {
        e[0] = f16_bits(r.a.x); e[1] = f16_bits(r.a.x >> 16);
        e[2] = f16_bits(r.a.y); e[3] = f16_bits(r.a.y >> 16);
        e[4] = f16_bits(r.a.z); e[5] = f16_bits(r.a.z >> 16);
        e[6] = f16_bits(r.a.w); e[7] = f16_bits(r.a.w >> 16);
    }
}

// The row's last, partial vector (n < 8 valid elements); the rest is `fill`.
template <int DT>
__device__ __forceinline__ void load_partial(const char* row, int v, int n, float fill, float* e)
{
#pragma unroll
    for (int j = 0; j < kVec; ++j) e[j] = j < n ? load_elem<DT>(row, 8LL * v + j) : fill;
}

// Any logical vector: full ones through load_raw, the partial tail element-wise.
template <int DT, bool VEC>
__device__ __forceinline__ void load8(const char* row, int v, int nfull, int V, float fill, float* e)
{
    if (v < nfull) {
        Raw<DT> r = load_raw<DT, VEC>(row, v);
        decode<DT>(r, e);
    } else {
        load_partial<DT>(row, v, V - 8 * v, fill, e);
    }
}

__device__ __forceinline__ const char* row_ptr(const void* base, long long row, long long stride, int es)
{
    return reinterpret_cast<const char*>(base) + row * stride * es;
}

// ---- ordering keys -----------------------------------------------------------
// An unsigned key that orders like the logit: equal logits share a key
// (-0.0 is mapped to +0.0), larger logits get larger keys.  16-bit formats
// use their own 16 bits, fp32 its 32.  NaN is outside the contract.
template <int DT>
__device__ __forceinline__ uint32_t key_of(float v)
{
    if constexpr (DT == DT_F32) {
        uint32_t u = __float_as_uint(v);
        u = (u == 0x80000000u) ? 0u : u;
        return (u >> 31) ? ~u : (u | 0x80000000u);
    } else {
        uint32_t u;
        if constexpr (DT == DT_BF16) {
            u = __float_as_uint(v) >> 16;
        } else {
            u = __builtin_bit_cast(unsigned short, (_Float16)v);
        }
        u = (u == 0x8000u) ? 0u : u;
        return (u >> 15) ? (~u & 0xffffu) : (u | 0x8000u);
    }
}

// The stabiliser of softmax statistics with max m: h = m * c, rounded once
// and never contracted into a neighbouring operation, so that every kernel
// forms the same h from the same m.  A softmax row's mass is
// s = sum_t exp2(z_t c - h) and its probabilities are exp2(fma(z, c, -h) - log2 s).
__device__ __forceinline__ float stab_of(float m, float c)
{
    return __fmul_rn(m, c);
}

// Slice partials are read kSoftBatch at a time, the batch's loads issued
// together (one round trip per batch).  Partials past `splits` are not read
// (the condition is uniform, so it costs a scalar branch, not a wait).
constexpr int kSoftBatch = 8;

__device__ __forceinline__ void load_soft_batch(const SoftPartial* p, int i0, int splits, SoftPartial* q)
{
    // one 8-byte load per partial, so (m, s) arrive together
    const unsigned long long* p8 = reinterpret_cast<const unsigned long long*>(p);
#pragma unroll
    for (int u = 0; u < kSoftBatch; ++u) {
        q[u] = SoftPartial{-INFINITY, 0.f};
        if (i0 + u < splits) {
            const unsigned long long w = p8[i0 + u];
            q[u] = SoftPartial{__uint_as_float((uint32_t)w), __uint_as_float((uint32_t)(w >> 32))};
        }
    }
}

// Adds partials q[0..N) to (m, s): the new max first, then every sum
// rescaled to it, exp2(stab(m_i) - stab(max)), and added in slice order.
// s stays 0 while every max is -inf.
template <int N>
__device__ __forceinline__ void merge_soft_n(const SoftPartial* q, float c, float& m, float& s)
{
    float mn = m;
#pragma unroll
    for (int u = 0; u < N; ++u) mn = fmaxf(mn, q[u].m);
    if (mn == -INFINITY) return;
    const float hn = stab_of(mn, c);
    float sn = m == -INFINITY ? 0.f : s * exp2f(stab_of(m, c) - hn);
#pragma unroll
    for (int u = 0; u < N; ++u) sn += q[u].s * exp2f(stab_of(q[u].m, c) - hn);
    m = mn;
    s = sn;
}

// The same for a uniform count n in [1, kSoftBatch]: one straight-line body
// per count, so no merge is computed and then discarded.
__device__ __forceinline__ void merge_soft_batch(const SoftPartial* q, int n, float c, float& m, float& s)
{
    switch (n) {
    case 1: merge_soft_n<1>(q, c, m, s); break;
    case 2: merge_soft_n<2>(q, c, m, s); break;
    case 3: merge_soft_n<3>(q, c, m, s); break;
    case 4: merge_soft_n<4>(q, c, m, s); break;
    case 5: merge_soft_n<5>(q, c, m, s); break;
    case 6: merge_soft_n<6>(q, c, m, s); break;
    case 7: merge_soft_n<7>(q, c, m, s); break;
    default: merge_soft_n<kSoftBatch>(q, c, m, s); break;
    }
}

// The merged (max, sum of exp2(z c - h)) of a row from its slice partials;
// each partial's sum is relative to its own stabiliser.
__device__ __forceinline__ void merge_soft(const SoftPartial* p, int splits, float c, float& m, float& s)
{
    m = -INFINITY;
    s = 0.f;
    for (int i0 = 0; i0 < splits; i0 += kSoftBatch) {
        SoftPartial q[kSoftBatch];
        load_soft_batch(p, i0, splits, q);
        merge_soft_batch(q, min(kSoftBatch, splits - i0), c, m, s);
    }
}

// ---- fixed-order workgroup collectives -------------------------------------
// Wave reductions in DPP: rotations by 1, 2, 4 and 8 lanes inside each row of
// 16 leave every lane holding its row's result; the four rows' results are
// then read as scalars and combined in row order, the same on every lane.
// No LDS round trip.
template <int N>
__device__ __forceinline__ uint32_t row_ror(uint32_t x)
{
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x120 + N, 0xf, 0xf, false);
}

__device__ __forceinline__ float row_ror_f(float x, int n)
{
    switch (n) {
    case 1: return __uint_as_float(row_ror<1>(__float_as_uint(x)));
    case 2: return __uint_as_float(row_ror<2>(__float_as_uint(x)));
    case 4: return __uint_as_float(row_ror<4>(__float_as_uint(x)));
    default: return __uint_as_float(row_ror<8>(__float_as_uint(x)));
    }
}

__device__ __forceinline__ int row_ror_i(int x, int n)
{
    switch (n) {
    case 1: return (int)row_ror<1>((uint32_t)x);
    case 2: return (int)row_ror<2>((uint32_t)x);
    case 4: return (int)row_ror<4>((uint32_t)x);
    default: return (int)row_ror<8>((uint32_t)x);
    }
}

__device__ __forceinline__ float lane_f(float x, int l)
{
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), l));
}

__device__ __forceinline__ float wave_max(float v)
{
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) v = fmaxf(v, row_ror_f(v, o));
    return fmaxf(fmaxf(lane_f(v, 0), lane_f(v, 16)), fmaxf(lane_f(v, 32), lane_f(v, 48)));
}

// The wave's sum in a fixed order: each row of 16 by DPP rotations, then the
// four row sums in row order (the same result on every lane).
__device__ __forceinline__ float wave_sum_f(float v)
{
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) v += row_ror_f(v, o);
    return ((lane_f(v, 0) + lane_f(v, 16)) + lane_f(v, 32)) + lane_f(v, 48);
}

__device__ __forceinline__ int wave_min_int(int v)
{
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) v = min(v, row_ror_i(v, o));
    return min(min(__builtin_amdgcn_readlane(v, 0), __builtin_amdgcn_readlane(v, 16)),
               min(__builtin_amdgcn_readlane(v, 32), __builtin_amdgcn_readlane(v, 48)));
}

__device__ __forceinline__ int wave_max_int(int v)
{
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) v = max(v, row_ror_i(v, o));
    return max(max(__builtin_amdgcn_readlane(v, 0), __builtin_amdgcn_readlane(v, 16)),
               max(__builtin_amdgcn_readlane(v, 32), __builtin_amdgcn_readlane(v, 48)));
}

// Block-wide reductions over a workgroup of NW wave64s; `lds` holds at least
// NW entries.  Every thread gets the result.
template <int NW = kWaves>
__device__ __forceinline__ float block_max(float v, float* lds)
{
    v = wave_max(v);
    if ((threadIdx.x & 63) == 0) lds[threadIdx.x >> 6] = v;
    __syncthreads();
    float r = lds[0];
#pragma unroll
    for (int w = 1; w < NW; ++w) r = fmaxf(r, lds[w]);
    __syncthreads();
    return r;
}

template <int NW = kWaves>
__device__ __forceinline__ int block_min_int(int v, int* lds)
{
    v = wave_min_int(v);
    if ((threadIdx.x & 63) == 0) lds[threadIdx.x >> 6] = v;
    __syncthreads();
    int r = lds[0];
#pragma unroll
    for (int w = 1; w < NW; ++w) r = min(r, lds[w]);
    __syncthreads();
    return r;
}

template <int NW = kWaves>
__device__ __forceinline__ int block_max_int(int v, int* lds)
{
    v = wave_max_int(v);
    if ((threadIdx.x & 63) == 0) lds[threadIdx.x >> 6] = v;
    __syncthreads();
    int r = lds[0];
#pragma unroll
    for (int w = 1; w < NW; ++w) r = max(r, lds[w]);
    __syncthreads();
    return r;
}

// Inclusive scan of x over the workgroup in thread order.  Returns the
// inclusive value; *excl gets the exclusive value, bitwise equal to the
// inclusive value of the previous thread (0 for thread 0); *total gets the
// block total, bitwise equal to the last thread's inclusive value.
__device__ __forceinline__ float block_scan(float x, float* excl, float* total, float* lds)
{
    const int w = threadIdx.x >> 6;
    // inclusive scan of the wave in DPP: row shifts, then row broadcasts
    // (disabled lanes and rows add +0.0)
    auto dpp = [](float v, auto ctrl, auto rows, auto bc) {
        return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), decltype(ctrl)::value,
                                                          decltype(rows)::value, 0xf, decltype(bc)::value));
    };
    using B1 = std::integral_constant<bool, true>;
    using B0 = std::integral_constant<bool, false>;
    using RA = std::integral_constant<int, 0xf>;
    float incl = x;
    incl += dpp(incl, std::integral_constant<int, 0x111>{}, RA{}, B1{});   // row_shr:1
    incl += dpp(incl, std::integral_constant<int, 0x112>{}, RA{}, B1{});   // row_shr:2
    incl += dpp(incl, std::integral_constant<int, 0x114>{}, RA{}, B1{});   // row_shr:4
    incl += dpp(incl, std::integral_constant<int, 0x118>{}, RA{}, B1{});   // row_shr:8
    incl += dpp(incl, std::integral_constant<int, 0x142>{}, std::integral_constant<int, 0xa>{}, B0{});  // row_bcast:15
    incl += dpp(incl, std::integral_constant<int, 0x143>{}, std::integral_constant<int, 0xc>{}, B0{});  // row_bcast:31
    // the previous lane's inclusive value (0 for lane 0): wave_shr:1
    const float wex = dpp(incl, std::integral_constant<int, 0x138>{}, RA{}, B1{});
    if ((threadIdx.x & 63) == 63) lds[w] = incl;
    __syncthreads();
    float pre = 0.f;
    for (int i = 0; i < w; ++i) pre += lds[i];
    float tot = 0.f;
#pragma unroll
    for (int i = 0; i < kWaves - 1; ++i) tot += lds[i];
    tot += lds[kWaves - 1];
    __syncthreads();
    *excl = pre + wex;
    *total = tot;
    return pre + incl;
}

}  // namespace sv
