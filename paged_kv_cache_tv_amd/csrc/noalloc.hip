// The decode step for callers that cannot allocate device memory (code under
// HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
// tv_paged_attention_decode_step with its partition workspace placed in a
// fixed device array instead of caller-owned buffers.
//
// `scratch` is a file-scope device array.  In host code its name is only a
// host-side stand-in, never a device address: the array's device address is
// looked up once per device with hipGetSymbolAddress (with that device
// current) and kept per device, and only that address is handed to the
// kernels.  Each GPU the library runs on holds its own copy of the array until
// the process ends.  Every call on one GPU shares that GPU's copy, so calls
// that overlap on one GPU (on different streams, or from different host
// threads without ordering) race on it.  Nothing in it has to start at zero:
// the partition pass writes every partial the merge reads, and the merge
// selects the partitions past a sequence's end away, so whatever an earlier
// call left behind is never used.
#include "../../include/tv.h"
#include "tv_internal.h"

#include <mutex>

namespace {

constexpr int64_t kScratchBytes = TV_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes % 256 == 0, "scratch size");

__device__ __align__(256) char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
void *g_scratch[kMaxDevices];        // device address of `scratch`, per device (nullptr: not yet)
std::mutex g_scratch_mu;

// The current device's address of `scratch`, looked up on the first call on
// that device.  No allocation: the array is part of the loaded code object.
hipError_t scratch_address(void **out)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    if (dev < 0 || dev >= kMaxDevices)
        return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess)
            return e;
        if (!p)
            return hipErrorInvalidSymbol;
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return hipSuccess;
}

}  // namespace

extern "C" tv_status tv_paged_attention_decode_step_noalloc(
    float *out, const uint16_t *q, const uint16_t *k_new, const uint16_t *v_new,
    const int64_t *slot_mapping, uint16_t *k_cache, uint16_t *v_cache,
    const int32_t *block_tables, const int32_t *context_lens, int32_t num_seqs,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
    int32_t max_blocks_per_seq, int64_t num_blocks, int32_t max_context_len,
    int32_t partition_size, float scale, void *stream)
{
    const bool sizes_ok = num_seqs > 0 && num_q_heads > 0 && head_dim > 0 && partition_size > 0 &&
                          max_context_len > 0;
    const int64_t parts = sizes_ok ? ((int64_t)max_context_len + partition_size - 1) / partition_size : 0;
    float *acc = nullptr, *mx = nullptr, *sum = nullptr;
    if (parts > 1) {
        // Workspace rows (s, h, p), each head_dim + 2 floats; every factor is
        // checked against the limit before the next multiply, so nothing overflows.
        const int64_t limit = kScratchBytes / (((int64_t)head_dim + 2) * 4);
        if (num_seqs > limit || num_q_heads > limit || (int64_t)num_seqs * num_q_heads > limit ||
            parts > limit || (int64_t)num_seqs * num_q_heads * parts > limit)
            return TV_ERR_SCRATCH;
        const int64_t rows = (int64_t)num_seqs * num_q_heads * parts;
        // The workspace: part_acc [S][Hq][P][D] at the array's start (256-byte
        // aligned), then part_max and part_sum [S][Hq][P].
        void *base = nullptr;
        if (scratch_address(&base) != hipSuccess)
            return TV_ERR_HIP;
        acc = static_cast<float *>(base);
        mx = acc + rows * head_dim;
        sum = mx + rows;
    }
    // With one partition (or none) the step needs no workspace; invalid sizes
    // are reported by the step's own checks before anything is launched.
    return tv_paged_attention_decode_step(out, acc, mx, sum, q, k_new, v_new, slot_mapping, k_cache,
                                          v_cache, block_tables, context_lens, num_seqs,
                                          num_q_heads, num_kv_heads, head_dim, block_size,
                                          max_blocks_per_seq, num_blocks, max_context_len,
                                          partition_size, scale, stream);
}
