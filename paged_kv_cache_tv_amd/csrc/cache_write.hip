// Cache write: scatter each new token's K and V rows into the slot the engine
// chose for it ("Tiny-vLLM" page, slot_mapping; "vLLM" page, fixed 16-token
// blocks).  A pure bit copy.
//
// One wavefront per token.  A token's K (or V) is num_kv_heads * head_dim bf16
// values, contiguous in the input; lanes take 16-byte chunks (8 values of one
// head, since head_dim % 8 == 0).  The K tile of a (block, head) is stored as
// head_dim / 8 chunks of [block_size tokens][8 dims], so each K chunk is one
// 16-byte store at (chunk, token offset); V values go to 8 consecutive rows of
// the dimension-major V tile, one 2-byte store each.
#include "tv_internal.h"

namespace tv {
namespace {

constexpr int kWavesPerGroup = 4;

__global__ __launch_bounds__(64 * kWavesPerGroup) void cache_write_kernel(CacheWriteArgs a)
{
    const int64_t tok = (int64_t)blockIdx.x * kWavesPerGroup + (threadIdx.x >> 6);
    if (tok >= a.num_tokens)
        return;
    const int lane = threadIdx.x & 63;
    const int row = a.num_kv_heads * a.head_dim;
    const int chunks = row >> 3;
    const uint4 *ksrc = reinterpret_cast<const uint4 *>(a.k + tok * row);
    const uint4 *vsrc = reinterpret_cast<const uint4 *>(a.v + tok * row);
    // The first chunk of each lane is loaded together with the slot number, so
    // the common case (num_kv_heads * head_dim <= 512) waits on memory once.
    const bool have0 = lane < chunks;
    const uint4 k0 = have0 ? ksrc[lane] : make_uint4(0, 0, 0, 0);
    const uint4 v0 = have0 ? vsrc[lane] : make_uint4(0, 0, 0, 0);
    const int64_t slot = a.slot_mapping[tok];
    if (slot < 0 || slot >= a.num_slots)
        return;
    const int64_t blk = slot / a.block_size;
    const int off = (int)(slot - blk * a.block_size);
    for (int c = lane; c < chunks; c += 64) {
        const uint4 kk = c == lane ? k0 : ksrc[c];
        const uint4 vv = c == lane ? v0 : vsrc[c];
        const int h = (c << 3) / a.head_dim;
        const int d = (c << 3) - h * a.head_dim;
        const int64_t tile = blk * a.num_kv_heads + h;
        *reinterpret_cast<uint4 *>(a.k_cache + tile * a.head_dim * a.block_size +
                                   ((int64_t)(d >> 3) * a.block_size + off) * 8) = kk;
        uint16_t *vdst = a.v_cache + (tile * a.head_dim + d) * a.block_size + off;
        const uint32_t w[4] = {vv.x, vv.y, vv.z, vv.w};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t word = w[i >> 1];
            vdst[(int64_t)i * a.block_size] = (uint16_t)((i & 1) ? (word >> 16) : (word & 0xFFFFu));
        }
    }
}

}  // namespace

hipError_t launch_cache_write(const CacheWriteArgs &a, hipStream_t stream)
{
    const int64_t groups = (a.num_tokens + kWavesPerGroup - 1) / kWavesPerGroup;
    hipLaunchKernelGGL(cache_write_kernel, dim3((unsigned)groups), dim3(64 * kWavesPerGroup), 0,
                       stream, a);
    return hipGetLastError();
}

}  // namespace tv
