// Streaming read: the yardstick for the HBM-bound kernels.  It reads a
// buffer once with coalesced 16-byte non-temporal loads and does nothing
// else but fold each 8 KiB chunk to one 32-bit XOR (so every byte is used
// and the result can be checked on the host).  Its rate is the read
// bandwidth the device sustains for one kernel of a given size, which is
// what the attention kernels' bytes per second are set against next to
// the 8 TB/s specification.
//
// One 256-thread workgroup per 8 KiB chunk: thread t loads 16-byte pieces t
// and t + 256 of its chunk (each wavefront load 1 KiB contiguous), XORs
// their words, and the workgroup combines its 256 values through shuffles
// and LDS.  Of the shapes measured on 304 MB and 1 GiB reads -- 2, 4, 6, 8
// or 16 loads per thread, 128 to 512 threads, non-temporal or ordinary
// loads -- this one read fastest (6.75 and 6.93 TB/s cold; 8 loads per
// thread 6.59 and 6.83, ordinary loads 6.04 and 6.23).
#include "tv_internal.h"

namespace tv {
namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 2;
static_assert(kThreads * kUnroll * 16 == kStreamChunkBytes, "chunk size");

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kThreads) void stream_read_kernel(StreamReadArgs a)
{
    const u32x4 *p = reinterpret_cast<const u32x4 *>(a.buf);
    const int64_t base = (int64_t)blockIdx.x * (kThreads * kUnroll) + threadIdx.x;
    u32x4 x[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
        const int64_t i = base + (int64_t)u * kThreads;
        x[u] = i < a.pieces ? __builtin_nontemporal_load(p + i) : u32x4{0u, 0u, 0u, 0u};
    }
    uint32_t h = 0;
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
        h ^= (x[u].x ^ x[u].y) ^ (x[u].z ^ x[u].w);
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1)
        h ^= (uint32_t)__shfl_xor((int)h, m);
    __shared__ uint32_t part[kThreads / 64];
    if ((threadIdx.x & 63) == 0)
        part[threadIdx.x >> 6] = h;
    __syncthreads();
    if (threadIdx.x == 0)
        a.chunk_xor[blockIdx.x] = (part[0] ^ part[1]) ^ (part[2] ^ part[3]);
}

}  // namespace

hipError_t launch_stream_read(const StreamReadArgs &a, hipStream_t stream)
{
    const int64_t chunks = (a.pieces * 16 + kStreamChunkBytes - 1) / kStreamChunkBytes;
    hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)chunks), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace tv
