// sv_ceiling.hip -- libsvceiling.so: the achievable HBM read rate on the
// device, for comparison with the verification kernels.  A measurement tool
// for bench.py, not part of the verification library's ABI.
//
// k_stream_read reads two buffers once, end to end, with 16-byte non-temporal
// loads (four per thread in flight, the loads of the streaming statistics
// pass), in 512-thread workgroups of `vec_per_block` 16-byte vectors, and
// does nothing with the data but fold it with XOR.  One launch covers both
// buffers, as one statistics launch covers the target and the draft rows.
// A workgroup stores its fold only if it equals a fixed constant (a store the
// compiler must keep, so the loads stay; it writes at most one word per
// workgroup, inside `sink`).

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 512;
constexpr unsigned kMagic = 0x9e3779b9u;

__global__ __launch_bounds__(kThreads) void k_stream_read(const u32x4* a, long long a_vec, const u32x4* b,
                                                          long long b_vec, int vec_per_block, int a_blocks,
                                                          unsigned* sink)
{
    const bool first = (int)blockIdx.x < a_blocks;
    const u32x4* p = first ? a : b;
    const long long n = first ? a_vec : b_vec;
    const long long blk = first ? blockIdx.x : blockIdx.x - a_blocks;
    const long long v0 = blk * vec_per_block;
    const long long v1 = v0 + vec_per_block < n ? v0 + vec_per_block : n;
    u32x4 acc = {0u, 0u, 0u, 0u};
    long long v = v0 + threadIdx.x;
    for (; v + 3 * kThreads < v1; v += 4 * kThreads) {
        const u32x4 r0 = __builtin_nontemporal_load(p + v);
        const u32x4 r1 = __builtin_nontemporal_load(p + v + kThreads);
        const u32x4 r2 = __builtin_nontemporal_load(p + v + 2 * kThreads);
        const u32x4 r3 = __builtin_nontemporal_load(p + v + 3 * kThreads);
        acc ^= (r0 ^ r1) ^ (r2 ^ r3);
    }
    for (; v < v1; v += kThreads) acc ^= __builtin_nontemporal_load(p + v);
    const unsigned x = acc.x ^ acc.y ^ acc.z ^ acc.w;
    if (x == kMagic) sink[blockIdx.x] = x;
}

}  // namespace

extern "C" {

// Workgroups one sv_stream_read call launches (the sink needs this many words).
long long sv_stream_read_blocks(long long a_bytes, long long b_bytes, int vec_per_block)
{
    if (a_bytes < 0 || b_bytes < 0 || vec_per_block < 1) return -1;
    const long long av = a_bytes / 16, bv = b_bytes / 16;
    return (av + vec_per_block - 1) / vec_per_block + (bv + vec_per_block - 1) / vec_per_block;
}

// Reads floor(a_bytes / 16) and floor(b_bytes / 16) 16-byte vectors of the
// DEVICE buffers a and b (16-byte aligned; b may be NULL with b_bytes 0) on
// `stream`.  sink: DEVICE, at least sv_stream_read_blocks(...) words.
// Returns 0, or a HIP error code (1 for invalid arguments, nothing launched).
int sv_stream_read(const void* a, long long a_bytes, const void* b, long long b_bytes, int vec_per_block,
                   unsigned* sink, long long sink_words, void* stream)
{
    const long long blocks = sv_stream_read_blocks(a_bytes, b_bytes, vec_per_block);
    if (blocks < 1 || blocks > sink_words || blocks >= (1LL << 31) || !a || !sink) return 1;
    if ((uintptr_t)a % 16 || (b && (uintptr_t)b % 16) || (!b && b_bytes)) return 1;
    const long long av = a_bytes / 16, bv = b_bytes / 16;
    const int a_blocks = (int)((av + vec_per_block - 1) / vec_per_block);
    hipLaunchKernelGGL(k_stream_read, dim3((unsigned)blocks), dim3(kThreads), 0,
                       static_cast<hipStream_t>(stream), static_cast<const u32x4*>(a), av,
                       static_cast<const u32x4*>(b), bv, vec_per_block, a_blocks, sink);
    return (int)hipGetLastError();
}

}  // extern "C"
