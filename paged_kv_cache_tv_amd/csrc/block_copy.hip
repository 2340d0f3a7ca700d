// Block copy for copy-on-write ("vLLM" page, section "가상 메모리 방식의 해결":
// requests sharing a prompt share its blocks, and a block is copied only when a
// branch writes into it).  Copies every K/V head of block src to block dst in
// both pools: a bit copy of two contiguous runs of
// num_kv_heads * block_size * head_dim values.
//
// One workgroup per (pair, pool), copying the run in passes of THREADS x
// UNROLL 16-byte chunks: UNROLL loads, then UNROLL stores.  Both are
// non-temporal: the source is read once and the destination is next read by
// a later launch.  A 16 KiB run of the decode shape is one pass in either
// shape.  Up to 512 pairs (the copy-on-write copies of a decode step), 256
// threads of 4 chunks: more wavefronts per run finish a small launch sooner
// (64 pairs 3.8-4.1 against 6.2-6.6 us, 512 pairs 7.1 against 8.2 us).  From
// about 1024 pairs on the two shapes tie, and past that 128 threads of 8
// chunks keep a large launch closer to the bandwidth (2048 pairs 23.1
// against 25.6 us).
#include "tv_internal.h"

namespace tv {
namespace {

constexpr int64_t kWideUpTo = 512;    // pairs up to which the 256-thread shape is used

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <int kThreads, int kUnroll>
__global__ __launch_bounds__(kThreads) void block_copy_kernel(BlockCopyArgs a)
{
    const int64_t pair = blockIdx.x >> 1;
    const int pool = blockIdx.x & 1;
    const int64_t src = a.pairs[2 * pair];
    const int64_t dst = a.pairs[2 * pair + 1];
    if (src < 0 || src >= a.num_blocks || dst < 0 || dst >= a.num_blocks || src == dst)
        return;
    uint16_t *base = pool ? a.v_cache : a.k_cache;
    const u32x4 *from = reinterpret_cast<const u32x4 *>(base + src * a.block_elems);
    u32x4 *to = reinterpret_cast<u32x4 *>(base + dst * a.block_elems);
    const int64_t chunks = a.block_elems / 8;
    for (int64_t c0 = 0; c0 < chunks; c0 += kThreads * kUnroll) {
        u32x4 x[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int64_t c = c0 + u * kThreads + threadIdx.x;
            if (c < chunks)
                x[u] = __builtin_nontemporal_load(from + c);
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int64_t c = c0 + u * kThreads + threadIdx.x;
            if (c < chunks)
                __builtin_nontemporal_store(x[u], to + c);
        }
    }
}

}  // namespace

hipError_t launch_block_copy(const BlockCopyArgs &a, hipStream_t stream)
{
    const dim3 grid((unsigned)(2 * a.num_pairs));
    if (a.num_pairs <= kWideUpTo)
        hipLaunchKernelGGL((block_copy_kernel<256, 4>), grid, dim3(256), 0, stream, a);
    else
        hipLaunchKernelGGL((block_copy_kernel<128, 8>), grid, dim3(128), 0, stream, a);
    return hipGetLastError();
}

}  // namespace tv
