// Internal launch interface between the C entry points (tv_api.cpp) and the
// kernels.  Argument checking happens in tv_api.cpp; the launchers assume
// valid, checked arguments.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tv {

// Shapes served by the decode kernels.
constexpr int kHeadDim = 64;
constexpr int kBlockSize = 16;
constexpr int kMaxGroup = 16;   // query heads per K/V head (MFMA N dimension)

struct CacheWriteArgs {
    const uint16_t *k;
    const uint16_t *v;
    uint16_t *k_cache;
    uint16_t *v_cache;
    const int64_t *slot_mapping;
    int64_t num_tokens;
    int32_t num_kv_heads;
    int32_t head_dim;
    int32_t block_size;
    int64_t num_slots;          // num_blocks * block_size
    // Rotary embedding of K on the way in; positions == nullptr: plain copy.
    const int32_t *positions;   // [num_tokens]
    const float *inv_freq;      // [head_dim / 2]
    int32_t rope_style;         // 0: pairs (2k, 2k+1); 1: pairs (k, k + head_dim/2)
};

struct RopeArgs {
    uint16_t *x;                // [num_tokens][num_heads][head_dim], rotated in place
    const int32_t *positions;
    const float *inv_freq;
    int64_t num_tokens;
    int32_t num_heads;
    int32_t head_dim;
    int32_t style;
};

struct DecodeArgs {
    float *part_acc;
    float *part_max;
    float *part_sum;
    const uint16_t *q;
    const uint16_t *k_cache;
    const uint16_t *v_cache;
    const int32_t *block_tables;
    const int32_t *context_lens;
    int32_t num_seqs;
    int32_t num_kv_heads;
    int32_t group;              // query heads per K/V head
    int32_t max_blocks;         // row stride of block_tables
    int32_t num_parts;          // P: partitions per (sequence, head) in the workspace
    int32_t part_tiles;         // partition_size / block_size
    int32_t max_context_len;
    int64_t num_blocks;
    float scale_log2;           // scale * log2(e)
    // Append (tv_paged_attention_decode_append): one new token per sequence,
    // written into the pools before it is attended to.  k_new == nullptr: none.
    const uint16_t *k_new;      // [num_seqs][num_kv_heads][head_dim]
    const uint16_t *v_new;
    const int64_t *slot_mapping;   // [num_seqs]
    uint16_t *k_cache_w;        // the pools again, writable
    uint16_t *v_cache_w;
    // Shared prefixes (tv_paged_attention_decode_shared): shared_len == nullptr: none.
    const int32_t *shared_len;  // [num_groups]: leading tokens shared by group g's sequences
    const int32_t *group_order; // [num_seqs] or nullptr: position p holds sequence group_order[p]
    int32_t group_size;         // sequences per group (consecutive), 1 .. 16 / group
    int32_t num_groups;         // ceil(num_seqs / group_size)
    // Set by the launcher: > 0 selects the balanced workgroup order and gives
    // how many compute units consecutive workgroups of one K/V head are dealt
    // over; 0 keeps the plain (partition, sequence, head) order.
    int32_t plan_width;
    // 1: a single partition per (sequence, head) (num_parts == 1, no shared
    // prefix), whose log-sum-exp merge is just acc / l: the pass writes that
    // (0 where nothing was attended) into part_acc, which is then the output
    // [num_seqs][num_q_heads][head_dim], and writes no max or sum.
    int32_t normalize;
};

struct ReduceArgs {
    float *out;
    const float *part_acc;
    const float *part_max;
    const float *part_sum;
    const int32_t *context_lens;
    int32_t num_seqs;
    int32_t num_q_heads;
    int32_t num_parts;
    int32_t partition_size;
    int32_t max_context_len;
};

struct PrefillArgs {
    float *out;                 // [rows][num_q_heads][head_dim]
    const uint16_t *q;          // [rows][num_q_heads][head_dim]
    const int32_t *query_start; // [num_seqs + 1]
    const uint16_t *k_cache;
    const uint16_t *v_cache;
    const int32_t *block_tables;
    const int32_t *context_lens;
    int32_t num_seqs;
    int32_t num_kv_heads;
    int32_t group;              // query heads per K/V head: 1, 2, 4, 8 or 16
    int32_t max_blocks;         // row stride of block_tables
    int32_t max_query_len;
    int32_t max_context_len;
    int64_t num_blocks;
    float scale_log2;           // scale * log2(e)
};

struct BlockCopyArgs {
    uint16_t *k_cache;
    uint16_t *v_cache;
    const int64_t *pairs;       // [num_pairs][2]: source block, destination block
    int64_t num_pairs;
    int64_t num_blocks;
    int64_t block_elems;        // num_kv_heads * block_size * head_dim (a multiple of 8)
};

constexpr int64_t kStreamChunkBytes = 8192;    // bytes folded into one XOR by tv_stream_read

struct StreamReadArgs {
    const void *buf;            // 16-byte aligned
    int64_t pieces;             // bytes / 16
    uint32_t *chunk_xor;        // [ceil(bytes / kStreamChunkBytes)]
};

hipError_t launch_cache_write(const CacheWriteArgs &a, hipStream_t stream);
hipError_t launch_rope(const RopeArgs &a, hipStream_t stream);
hipError_t launch_block_copy(const BlockCopyArgs &a, hipStream_t stream);
hipError_t launch_paged_prefill(const PrefillArgs &a, hipStream_t stream);
hipError_t launch_paged_decode(const DecodeArgs &a, hipStream_t stream);
hipError_t launch_paged_decode_vector(const DecodeArgs &a, hipStream_t stream);
bool paged_decode_seq_fits(const DecodeArgs &a);
hipError_t launch_paged_decode_seq(const DecodeArgs &a, hipStream_t stream);
bool paged_decode_group_fits(const DecodeArgs &a);
hipError_t launch_paged_decode_group(const DecodeArgs &a, hipStream_t stream);
hipError_t launch_paged_reduce(const ReduceArgs &a, hipStream_t stream);
hipError_t launch_stream_read(const StreamReadArgs &a, hipStream_t stream);

}  // namespace tv
