// C entry points of libtv: host-side argument checks, then one launch each on
// the caller's stream.  Nothing is allocated and no state is kept.
#include "../../include/tv.h"
#include "tv_internal.h"

#include <cmath>
#include <cstdint>

namespace {

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

tv_status from_hip(hipError_t e) { return e == hipSuccess ? TV_OK : TV_ERR_HIP; }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace

extern "C" {

const char *tv_status_string(tv_status status)
{
    switch (status) {
    case TV_OK: return "TV_OK";
    case TV_ERR_NULL: return "TV_ERR_NULL: a required pointer is NULL";
    case TV_ERR_SHAPE: return "TV_ERR_SHAPE: invalid or inconsistent sizes";
    case TV_ERR_UNSUPPORTED: return "TV_ERR_UNSUPPORTED: shape not implemented";
    case TV_ERR_HIP: return "TV_ERR_HIP: HIP runtime error";
    case TV_ERR_ALIGNMENT: return "TV_ERR_ALIGNMENT: misaligned pointer";
    case TV_ERR_NO_BLOCKS: return "TV_ERR_NO_BLOCKS: no free block (or no host memory)";
    case TV_ERR_SCRATCH: return "TV_ERR_SCRATCH: workspace larger than the fixed scratch array";
    }
    return "unknown tv_status";
}

int32_t tv_num_partitions(int32_t max_context_len, int32_t partition_size)
{
    if (partition_size <= 0)
        return -1;
    if (max_context_len <= 0)
        return 0;
    return (int32_t)ceil_div(max_context_len, partition_size);
}

tv_status tv_cache_write(const uint16_t *k, const uint16_t *v, uint16_t *k_cache,
                         uint16_t *v_cache, const int64_t *slot_mapping, int64_t num_tokens,
                         int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                         int64_t num_blocks, void *stream)
{
    if (num_tokens < 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 || num_blocks <= 0)
        return TV_ERR_SHAPE;
    if (num_tokens == 0)
        return TV_OK;
    if (!k || !v || !k_cache || !v_cache || !slot_mapping)
        return TV_ERR_NULL;
    if (head_dim % 8 != 0)
        return TV_ERR_UNSUPPORTED;
    if (num_blocks > INT64_MAX / block_size)
        return TV_ERR_SHAPE;
    if ((int64_t)num_kv_heads * head_dim > (1 << 24))
        return TV_ERR_UNSUPPORTED;
    if (ceil_div(num_tokens, 4) > 0xffffff)            // 256-thread workgroups of 4 tokens
        return TV_ERR_UNSUPPORTED;
    if (!aligned(k, 16) || !aligned(v, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 2) ||
        !aligned(slot_mapping, 8))
        return TV_ERR_ALIGNMENT;
    tv::CacheWriteArgs a{k, v, k_cache, v_cache, slot_mapping, num_tokens, num_kv_heads,
                         head_dim, block_size, num_blocks * block_size};
    return from_hip(tv::launch_cache_write(a, static_cast<hipStream_t>(stream)));
}

tv_status tv_cache_write_rope(const uint16_t *k, const uint16_t *v, uint16_t *k_cache,
                              uint16_t *v_cache, const int64_t *slot_mapping,
                              const int32_t *positions, const float *inv_freq,
                              int64_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                              int32_t block_size, int64_t num_blocks, int32_t rope_style,
                              void *stream)
{
    if (num_tokens < 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 ||
        num_blocks <= 0 || (rope_style != 0 && rope_style != 1))
        return TV_ERR_SHAPE;
    if (num_tokens == 0)
        return TV_OK;
    if (!k || !v || !k_cache || !v_cache || !slot_mapping || !positions || !inv_freq)
        return TV_ERR_NULL;
    if (head_dim % 8 != 0 || head_dim > 128)
        return TV_ERR_UNSUPPORTED;
    if (num_blocks > INT64_MAX / block_size)
        return TV_ERR_SHAPE;
    if ((int64_t)num_kv_heads * head_dim > (1 << 24))
        return TV_ERR_UNSUPPORTED;
    if (ceil_div(num_tokens, 4) > 0xffffff)            // 256-thread workgroups of 4 tokens
        return TV_ERR_UNSUPPORTED;
    if (!aligned(k, 16) || !aligned(v, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 2) ||
        !aligned(slot_mapping, 8) || !aligned(positions, 4) || !aligned(inv_freq, 4))
        return TV_ERR_ALIGNMENT;
    tv::CacheWriteArgs a{k, v, k_cache, v_cache, slot_mapping, num_tokens, num_kv_heads,
                         head_dim, block_size, num_blocks * block_size};
    a.positions = positions;
    a.inv_freq = inv_freq;
    a.rope_style = rope_style;
    return from_hip(tv::launch_cache_write(a, static_cast<hipStream_t>(stream)));
}

tv_status tv_rope(uint16_t *x, const int32_t *positions, const float *inv_freq,
                  int64_t num_tokens, int32_t num_heads, int32_t head_dim, int32_t rope_style,
                  void *stream)
{
    if (num_tokens < 0 || num_heads <= 0 || head_dim <= 0 || (rope_style != 0 && rope_style != 1))
        return TV_ERR_SHAPE;
    if (num_tokens == 0)
        return TV_OK;
    if (!x || !positions || !inv_freq)
        return TV_ERR_NULL;
    if (head_dim % 8 != 0 || head_dim > 128 || (int64_t)num_heads * head_dim > (1 << 24))
        return TV_ERR_UNSUPPORTED;
    if (ceil_div(num_tokens, 4) > 0xffffff)            // 256-thread workgroups of 4 tokens
        return TV_ERR_UNSUPPORTED;
    if (!aligned(x, 16) || !aligned(positions, 4) || !aligned(inv_freq, 4))
        return TV_ERR_ALIGNMENT;
    tv::RopeArgs a{x, positions, inv_freq, num_tokens, num_heads, head_dim, rope_style};
    return from_hip(tv::launch_rope(a, static_cast<hipStream_t>(stream)));
}

namespace {

// Checks shared by both decode entry points; fills `a` on success.  Returns
// TV_OK with a.num_parts == 0 when there is nothing to launch.
static tv_status check_decode(tv::DecodeArgs &a, float *part_acc, float *part_max, float *part_sum,
                              const uint16_t *q, const uint16_t *k_cache, const uint16_t *v_cache,
                              const int32_t *block_tables, const int32_t *context_lens,
                              int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                              int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                              int64_t num_blocks, int32_t max_context_len, int32_t partition_size,
                              float scale)
{
    if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
        block_size <= 0 || max_blocks_per_seq <= 0 || num_blocks <= 0 || max_context_len < 0 ||
        partition_size <= 0)
        return TV_ERR_SHAPE;
    if (num_q_heads % num_kv_heads != 0 || partition_size % block_size != 0)
        return TV_ERR_SHAPE;
    if ((int64_t)max_context_len > (int64_t)max_blocks_per_seq * block_size)
        return TV_ERR_SHAPE;
    if (!(scale > 0.f) || !std::isfinite(scale))
        return TV_ERR_SHAPE;
    if (head_dim != tv::kHeadDim || block_size != tv::kBlockSize ||
        num_q_heads / num_kv_heads > tv::kMaxGroup)
        return TV_ERR_UNSUPPORTED;
    a = tv::DecodeArgs{};
    if (num_seqs == 0 || max_context_len == 0)
        return TV_OK;
    if (!part_acc || !part_max || !part_sum || !q || !k_cache || !v_cache || !block_tables ||
        !context_lens)
        return TV_ERR_NULL;
    const int64_t parts = ceil_div(max_context_len, partition_size);
    // Workgroups of up to 256 work-items: the grid must stay below 2^32 of them.
    if ((int64_t)num_kv_heads * num_seqs * parts > 0xffffff)
        return TV_ERR_UNSUPPORTED;
    if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) ||
        !aligned(block_tables, 4) || !aligned(context_lens, 4) || !aligned(part_acc, 16) ||
        !aligned(part_max, 4) || !aligned(part_sum, 4))
        return TV_ERR_ALIGNMENT;
    a.part_acc = part_acc;
    a.part_max = part_max;
    a.part_sum = part_sum;
    a.q = q;
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    a.block_tables = block_tables;
    a.context_lens = context_lens;
    a.num_seqs = num_seqs;
    a.num_kv_heads = num_kv_heads;
    a.group = num_q_heads / num_kv_heads;
    a.max_blocks = max_blocks_per_seq;
    a.num_parts = (int32_t)parts;
    a.part_tiles = partition_size / block_size;
    a.max_context_len = max_context_len;
    a.num_blocks = num_blocks;
    a.scale_log2 = (float)((double)scale * 1.4426950408889634);   // log2(e)
    return TV_OK;
}

}  // namespace

tv_status tv_paged_attention_decode(float *part_acc, float *part_max, float *part_sum,
                                    const uint16_t *q, const uint16_t *k_cache,
                                    const uint16_t *v_cache, const int32_t *block_tables,
                                    const int32_t *context_lens, int32_t num_seqs,
                                    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                    int32_t block_size, int32_t max_blocks_per_seq,
                                    int64_t num_blocks, int32_t max_context_len,
                                    int32_t partition_size, float scale, void *stream)
{
    tv::DecodeArgs a;
    const tv_status st = check_decode(a, part_acc, part_max, part_sum, q, k_cache, v_cache,
                                      block_tables, context_lens, num_seqs, num_q_heads,
                                      num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                                      num_blocks, max_context_len, partition_size, scale);
    if (st != TV_OK || a.num_parts == 0)
        return st;
    return from_hip(tv::launch_paged_decode(a, static_cast<hipStream_t>(stream)));
}

tv_status tv_paged_attention_decode_vector(float *part_acc, float *part_max, float *part_sum,
                                           const uint16_t *q, const uint16_t *k_cache,
                                           const uint16_t *v_cache, const int32_t *block_tables,
                                           const int32_t *context_lens, int32_t num_seqs,
                                           int32_t num_q_heads, int32_t num_kv_heads,
                                           int32_t head_dim, int32_t block_size,
                                           int32_t max_blocks_per_seq, int64_t num_blocks,
                                           int32_t max_context_len, int32_t partition_size,
                                           float scale, void *stream)
{
    tv::DecodeArgs a;
    const tv_status st = check_decode(a, part_acc, part_max, part_sum, q, k_cache, v_cache,
                                      block_tables, context_lens, num_seqs, num_q_heads,
                                      num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                                      num_blocks, max_context_len, partition_size, scale);
    if (st != TV_OK)
        return st;
    if (num_q_heads != 4 * num_kv_heads)
        return TV_ERR_UNSUPPORTED;
    if (a.num_parts == 0)
        return TV_OK;
    return from_hip(tv::launch_paged_decode_vector(a, static_cast<hipStream_t>(stream)));
}

tv_status tv_paged_attention_decode_append(float *part_acc, float *part_max, float *part_sum,
                                           const uint16_t *q, const uint16_t *k_new,
                                           const uint16_t *v_new, const int64_t *slot_mapping,
                                           uint16_t *k_cache, uint16_t *v_cache,
                                           const int32_t *block_tables,
                                           const int32_t *context_lens, int32_t num_seqs,
                                           int32_t num_q_heads, int32_t num_kv_heads,
                                           int32_t head_dim, int32_t block_size,
                                           int32_t max_blocks_per_seq, int64_t num_blocks,
                                           int32_t max_context_len, int32_t partition_size,
                                           float scale, void *stream)
{
    tv::DecodeArgs a;
    const tv_status st = check_decode(a, part_acc, part_max, part_sum, q, k_cache, v_cache,
                                      block_tables, context_lens, num_seqs, num_q_heads,
                                      num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                                      num_blocks, max_context_len, partition_size, scale);
    if (st != TV_OK || a.num_parts == 0)
        return st;
    if (!k_new || !v_new || !slot_mapping)
        return TV_ERR_NULL;
    if (!aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(slot_mapping, 8))
        return TV_ERR_ALIGNMENT;
    if (num_blocks > INT64_MAX / block_size)
        return TV_ERR_SHAPE;
    a.k_new = k_new;
    a.v_new = v_new;
    a.slot_mapping = slot_mapping;
    a.k_cache_w = k_cache;
    a.v_cache_w = v_cache;
    return from_hip(tv::launch_paged_decode(a, static_cast<hipStream_t>(stream)));
}

tv_status tv_paged_attention_prefill(float *out, const uint16_t *q, const int32_t *query_start,
                                     const uint16_t *k_cache, const uint16_t *v_cache,
                                     const int32_t *block_tables, const int32_t *context_lens,
                                     int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                     int32_t head_dim, int32_t block_size,
                                     int32_t max_blocks_per_seq, int64_t num_blocks,
                                     int32_t max_query_len, int32_t max_context_len, float scale,
                                     void *stream)
{
    if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
        block_size <= 0 || max_blocks_per_seq <= 0 || num_blocks <= 0 || max_query_len < 0 ||
        max_context_len < 0)
        return TV_ERR_SHAPE;
    if (num_q_heads % num_kv_heads != 0)
        return TV_ERR_SHAPE;
    if ((int64_t)max_context_len > (int64_t)max_blocks_per_seq * block_size)
        return TV_ERR_SHAPE;
    if (!(scale > 0.f) || !std::isfinite(scale))
        return TV_ERR_SHAPE;
    const int32_t group = num_q_heads / num_kv_heads;
    if (head_dim != tv::kHeadDim || block_size != tv::kBlockSize ||
        (group != 1 && group != 2 && group != 4 && group != 8 && group != 16))
        return TV_ERR_UNSUPPORTED;
    if (num_seqs == 0 || max_query_len == 0)
        return TV_OK;
    if (!out || !q || !query_start || !k_cache || !v_cache || !block_tables || !context_lens)
        return TV_ERR_NULL;
    const int64_t rows_per_wg = 256 / group;
    if ((int64_t)num_kv_heads * num_seqs * ceil_div(max_query_len, rows_per_wg) > 0x7fffff)
        return TV_ERR_UNSUPPORTED;
    if (!aligned(out, 16) || !aligned(q, 16) || !aligned(query_start, 4) ||
        !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(block_tables, 4) ||
        !aligned(context_lens, 4))
        return TV_ERR_ALIGNMENT;
    tv::PrefillArgs a{};
    a.out = out;
    a.q = q;
    a.query_start = query_start;
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    a.block_tables = block_tables;
    a.context_lens = context_lens;
    a.num_seqs = num_seqs;
    a.num_kv_heads = num_kv_heads;
    a.group = group;
    a.max_blocks = max_blocks_per_seq;
    a.max_query_len = max_query_len;
    a.max_context_len = max_context_len;
    a.num_blocks = num_blocks;
    a.scale_log2 = (float)((double)scale * 1.4426950408889634);   // log2(e)
    return from_hip(tv::launch_paged_prefill(a, static_cast<hipStream_t>(stream)));
}

tv_status tv_paged_attention_decode_shared(float *part_acc, float *part_max, float *part_sum,
                                           const uint16_t *q, const uint16_t *k_cache,
                                           const uint16_t *v_cache, const int32_t *block_tables,
                                           const int32_t *context_lens, const int32_t *shared_len,
                                           const int32_t *group_order, int32_t group_size,
                                           int32_t num_seqs,
                                           int32_t num_q_heads, int32_t num_kv_heads,
                                           int32_t head_dim, int32_t block_size,
                                           int32_t max_blocks_per_seq, int64_t num_blocks,
                                           int32_t max_context_len, int32_t partition_size,
                                           float scale, void *stream)
{
    if (group_size < 1)
        return TV_ERR_SHAPE;
    if (num_kv_heads > 0 && num_q_heads > 0 && num_q_heads % num_kv_heads == 0 &&
        (int64_t)group_size * (num_q_heads / num_kv_heads) > tv::kMaxGroup)
        return TV_ERR_UNSUPPORTED;
    tv::DecodeArgs a;
    const tv_status st = check_decode(a, part_acc, part_max, part_sum, q, k_cache, v_cache,
                                      block_tables, context_lens, num_seqs, num_q_heads,
                                      num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                                      num_blocks, max_context_len, partition_size, scale);
    if (st != TV_OK)
        return st;
    if (a.num_parts == 0)
        return TV_OK;
    if (!shared_len)
        return TV_ERR_NULL;
    if (!aligned(shared_len, 4) || !aligned(group_order, 4))
        return TV_ERR_ALIGNMENT;
    a.shared_len = shared_len;
    a.group_order = group_order;
    a.group_size = group_size;
    a.num_groups = (int32_t)ceil_div(num_seqs, group_size);
    return from_hip(tv::launch_paged_decode(a, static_cast<hipStream_t>(stream)));
}

tv_status tv_paged_attention_decode_shared_append(
    float *part_acc, float *part_max, float *part_sum, const uint16_t *q, const uint16_t *k_new,
    const uint16_t *v_new, const int64_t *slot_mapping, uint16_t *k_cache, uint16_t *v_cache,
    const int32_t *block_tables, const int32_t *context_lens, const int32_t *shared_len,
    const int32_t *group_order, int32_t group_size, int32_t num_seqs, int32_t num_q_heads,
    int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
    int64_t num_blocks, int32_t max_context_len, int32_t partition_size, float scale, void *stream)
{
    if (group_size < 1)
        return TV_ERR_SHAPE;
    if (num_kv_heads > 0 && num_q_heads > 0 && num_q_heads % num_kv_heads == 0 &&
        (int64_t)group_size * (num_q_heads / num_kv_heads) > tv::kMaxGroup)
        return TV_ERR_UNSUPPORTED;
    tv::DecodeArgs a;
    const tv_status st = check_decode(a, part_acc, part_max, part_sum, q, k_cache, v_cache,
                                      block_tables, context_lens, num_seqs, num_q_heads,
                                      num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                                      num_blocks, max_context_len, partition_size, scale);
    if (st != TV_OK || a.num_parts == 0)
        return st;
    if (!shared_len || !k_new || !v_new || !slot_mapping)
        return TV_ERR_NULL;
    if (!aligned(shared_len, 4) || !aligned(group_order, 4) || !aligned(k_new, 16) ||
        !aligned(v_new, 16) || !aligned(slot_mapping, 8))
        return TV_ERR_ALIGNMENT;
    if (num_blocks > INT64_MAX / block_size)
        return TV_ERR_SHAPE;
    a.shared_len = shared_len;
    a.group_order = group_order;
    a.group_size = group_size;
    a.num_groups = (int32_t)ceil_div(num_seqs, group_size);
    a.k_new = k_new;
    a.v_new = v_new;
    a.slot_mapping = slot_mapping;
    a.k_cache_w = k_cache;
    a.v_cache_w = v_cache;
    return from_hip(tv::launch_paged_decode(a, static_cast<hipStream_t>(stream)));
}

tv_status tv_paged_attention_decode_shared_step(
    float *out, float *part_acc, float *part_max, float *part_sum, const uint16_t *q,
    const uint16_t *k_new, const uint16_t *v_new, const int64_t *slot_mapping, uint16_t *k_cache,
    uint16_t *v_cache, const int32_t *block_tables, const int32_t *context_lens,
    const int32_t *shared_len, const int32_t *group_order, int32_t group_size, int32_t num_seqs,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
    int32_t max_blocks_per_seq, int64_t num_blocks, int32_t max_context_len,
    int32_t partition_size, float scale, void *stream)
{
    if (group_size < 1)
        return TV_ERR_SHAPE;
    if (num_kv_heads > 0 && num_q_heads > 0 && num_q_heads % num_kv_heads == 0 &&
        (int64_t)group_size * (num_q_heads / num_kv_heads) > tv::kMaxGroup)
        return TV_ERR_UNSUPPORTED;
    tv::DecodeArgs a;
    const tv_status st = check_decode(a, part_acc, part_max, part_sum, q, k_cache, v_cache,
                                      block_tables, context_lens, num_seqs, num_q_heads,
                                      num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                                      num_blocks, max_context_len, partition_size, scale);
    if (st != TV_OK || num_seqs == 0)
        return st;
    if (a.num_parts == 0)                         // max_context_len == 0: out rows are 0
        return tv_paged_attention_reduce(out, part_acc, part_max, part_sum, context_lens,
                                         num_seqs, num_q_heads, head_dim, max_context_len,
                                         partition_size, stream);
    if (!out || !shared_len || !k_new || !v_new || !slot_mapping)
        return TV_ERR_NULL;
    if ((int64_t)num_seqs * num_q_heads > 0xffffff)
        return TV_ERR_UNSUPPORTED;
    if (!aligned(out, 16) || !aligned(shared_len, 4) || !aligned(group_order, 4) ||
        !aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(slot_mapping, 8))
        return TV_ERR_ALIGNMENT;
    if (num_blocks > INT64_MAX / block_size)
        return TV_ERR_SHAPE;
    a.shared_len = shared_len;
    a.group_order = group_order;
    a.group_size = group_size;
    a.num_groups = (int32_t)ceil_div(num_seqs, group_size);
    a.k_new = k_new;
    a.v_new = v_new;
    a.slot_mapping = slot_mapping;
    a.k_cache_w = k_cache;
    a.v_cache_w = v_cache;
    const hipStream_t hs = static_cast<hipStream_t>(stream);
    if (tv::paged_decode_group_fits(a)) {
        // One workgroup per (group, K/V head): the group's shared tiles once,
        // every member's own tiles, the appends and the merge, in one launch.
        a.part_acc = out;
        a.part_max = nullptr;
        a.part_sum = nullptr;
        return from_hip(tv::launch_paged_decode_group(a, hs));
    }
    const tv_status sd = from_hip(tv::launch_paged_decode(a, hs));
    if (sd != TV_OK)
        return sd;
    tv::ReduceArgs r{out, part_acc, part_max, part_sum, context_lens, num_seqs, num_q_heads,
                     a.num_parts, partition_size, max_context_len};
    return from_hip(tv::launch_paged_reduce(r, hs));
}

int32_t tv_paged_attention_decode_shared_step_form(int32_t num_seqs, int32_t num_q_heads,
                                                   int32_t num_kv_heads, int32_t head_dim,
                                                   int32_t block_size, int32_t max_context_len,
                                                   int32_t partition_size, int32_t group_size,
                                                   int32_t has_group_order)
{
    if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
        block_size <= 0 || max_context_len < 0 || partition_size <= 0 || group_size < 1 ||
        num_q_heads % num_kv_heads != 0 || partition_size % block_size != 0)
        return -1;
    if (head_dim != tv::kHeadDim || block_size != tv::kBlockSize ||
        (int64_t)group_size * (num_q_heads / num_kv_heads) > tv::kMaxGroup)
        return -1;
    if (num_seqs == 0 || max_context_len == 0)
        return 0;
    tv::DecodeArgs a{};
    static const int32_t one = 0;
    static const uint16_t dummy = 0;
    a.shared_len = &one;                       // only the pointers' presence is consulted
    a.group_order = has_group_order ? &one : nullptr;
    a.k_new = &dummy;
    a.group_size = group_size;
    a.num_groups = (int32_t)ceil_div(num_seqs, group_size);
    a.num_seqs = num_seqs;
    a.num_kv_heads = num_kv_heads;
    a.group = num_q_heads / num_kv_heads;
    a.num_parts = (int32_t)ceil_div(max_context_len, partition_size);
    a.part_tiles = partition_size / block_size;
    a.max_context_len = max_context_len;
    return tv::paged_decode_group_fits(a) ? 1 : 2;
}

tv_status tv_paged_attention_decode_step(float *out, float *part_acc, float *part_max,
                                         float *part_sum, const uint16_t *q,
                                         const uint16_t *k_new, const uint16_t *v_new,
                                         const int64_t *slot_mapping, uint16_t *k_cache,
                                         uint16_t *v_cache, const int32_t *block_tables,
                                         const int32_t *context_lens, int32_t num_seqs,
                                         int32_t num_q_heads, int32_t num_kv_heads,
                                         int32_t head_dim, int32_t block_size,
                                         int32_t max_blocks_per_seq, int64_t num_blocks,
                                         int32_t max_context_len, int32_t partition_size,
                                         float scale, void *stream)
{
    // One partition per (sequence, head): the merge is acc / l, written by the
    // partition pass itself into out (the workspace is not used).
    const bool one = partition_size > 0 && max_context_len > 0 && max_context_len <= partition_size;
    tv::DecodeArgs a;
    const tv_status st = check_decode(a, one ? out : part_acc, one ? out : part_max,
                                      one ? out : part_sum, q, k_cache, v_cache, block_tables,
                                      context_lens, num_seqs, num_q_heads, num_kv_heads, head_dim,
                                      block_size, max_blocks_per_seq, num_blocks,
                                      max_context_len, partition_size, scale);
    if (st != TV_OK || num_seqs == 0)
        return st;
    if (a.num_parts == 0)                         // max_context_len == 0: out rows are 0
        return tv_paged_attention_reduce(out, part_acc, part_max, part_sum, context_lens,
                                         num_seqs, num_q_heads, head_dim, max_context_len,
                                         partition_size, stream);
    if (!out || !k_new || !v_new || !slot_mapping)
        return TV_ERR_NULL;
    if ((int64_t)num_seqs * num_q_heads > 0xffffff)
        return TV_ERR_UNSUPPORTED;
    if (!aligned(out, 16) || (!one && !aligned(part_acc, 16)) || !aligned(k_new, 16) ||
        !aligned(v_new, 16) || !aligned(slot_mapping, 8))
        return TV_ERR_ALIGNMENT;
    if (num_blocks > INT64_MAX / block_size)
        return TV_ERR_SHAPE;
    a.k_new = k_new;
    a.v_new = v_new;
    a.slot_mapping = slot_mapping;
    a.k_cache_w = k_cache;
    a.v_cache_w = v_cache;
    const hipStream_t hs = static_cast<hipStream_t>(stream);
    if (one) {
        a.part_max = nullptr;
        a.part_sum = nullptr;
        a.normalize = 1;
        return from_hip(tv::launch_paged_decode(a, hs));
    }
    if (tv::paged_decode_seq_fits(a)) {
        // Every (sequence, K/V head) in one resident workgroup whose
        // wavefronts take one equal range of the context each and merge in
        // LDS: one launch, the workspace unused.
        a.part_acc = out;
        a.part_max = nullptr;
        a.part_sum = nullptr;
        return from_hip(tv::launch_paged_decode_seq(a, hs));
    }
    const tv_status sd = from_hip(tv::launch_paged_decode(a, hs));
    if (sd != TV_OK)
        return sd;
    tv::ReduceArgs r{out, part_acc, part_max, part_sum, context_lens, num_seqs, num_q_heads,
                     a.num_parts, partition_size, max_context_len};
    return from_hip(tv::launch_paged_reduce(r, hs));
}

int32_t tv_paged_attention_decode_step_form(int32_t num_seqs, int32_t num_q_heads,
                                            int32_t num_kv_heads, int32_t head_dim,
                                            int32_t block_size, int32_t max_context_len,
                                            int32_t partition_size)
{
    if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
        block_size <= 0 || max_context_len < 0 || partition_size <= 0 ||
        num_q_heads % num_kv_heads != 0 || partition_size % block_size != 0)
        return -1;
    if (head_dim != tv::kHeadDim || block_size != tv::kBlockSize ||
        num_q_heads / num_kv_heads > tv::kMaxGroup)
        return -1;
    if (num_seqs == 0 || max_context_len == 0)
        return 0;
    if (max_context_len <= partition_size)
        return 1;
    tv::DecodeArgs a{};
    a.num_seqs = num_seqs;
    a.num_kv_heads = num_kv_heads;
    a.group = num_q_heads / num_kv_heads;
    a.num_parts = (int32_t)ceil_div(max_context_len, partition_size);
    a.part_tiles = partition_size / block_size;
    a.max_context_len = max_context_len;
    return tv::paged_decode_seq_fits(a) ? 2 : 3;
}

tv_status tv_paged_attention_reduce(float *out, const float *part_acc, const float *part_max,
                                    const float *part_sum, const int32_t *context_lens,
                                    int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                                    int32_t max_context_len, int32_t partition_size, void *stream)
{
    if (num_seqs < 0 || num_q_heads <= 0 || head_dim <= 0 || max_context_len < 0 ||
        partition_size <= 0)
        return TV_ERR_SHAPE;
    if (head_dim != tv::kHeadDim)
        return TV_ERR_UNSUPPORTED;
    if (num_seqs == 0)
        return TV_OK;
    const int64_t parts = ceil_div(max_context_len, partition_size);
    if (!out || !context_lens || (parts > 0 && (!part_acc || !part_max || !part_sum)))
        return TV_ERR_NULL;
    if ((int64_t)num_seqs * num_q_heads > 0xffffff)
        return TV_ERR_UNSUPPORTED;
    if (!aligned(out, 16) || !aligned(part_acc, 16) || !aligned(part_max, 4) ||
        !aligned(part_sum, 4) || !aligned(context_lens, 4))
        return TV_ERR_ALIGNMENT;
    tv::ReduceArgs a{out, part_acc, part_max, part_sum, context_lens, num_seqs, num_q_heads,
                     (int32_t)parts, partition_size, max_context_len};
    return from_hip(tv::launch_paged_reduce(a, static_cast<hipStream_t>(stream)));
}

}  // extern "C"

tv_status tv_copy_blocks(uint16_t *k_cache, uint16_t *v_cache, const int64_t *block_pairs,
                         int64_t num_pairs, int32_t num_kv_heads, int32_t head_dim,
                         int32_t block_size, int64_t num_blocks, void *stream)
{
    if (num_pairs < 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 ||
        num_blocks <= 0)
        return TV_ERR_SHAPE;
    const int64_t block_elems = (int64_t)num_kv_heads * head_dim * block_size;
    if (block_elems % 8 != 0)
        return TV_ERR_UNSUPPORTED;
    if (num_pairs == 0)
        return TV_OK;
    if (!k_cache || !v_cache || !block_pairs)
        return TV_ERR_NULL;
    if (2 * num_pairs > 0x1ffffff)                   // 128-thread workgroups
        return TV_ERR_UNSUPPORTED;
    if (num_blocks > INT64_MAX / block_elems)
        return TV_ERR_SHAPE;
    if (!aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(block_pairs, 8))
        return TV_ERR_ALIGNMENT;
    tv::BlockCopyArgs a{k_cache, v_cache, block_pairs, num_pairs, num_blocks, block_elems};
    return from_hip(tv::launch_block_copy(a, static_cast<hipStream_t>(stream)));
}

tv_status tv_stream_read(const void *buf, int64_t bytes, uint32_t *chunk_xor, void *stream)
{
    if (bytes < 0)
        return TV_ERR_SHAPE;
    if (bytes % 16 != 0)
        return TV_ERR_UNSUPPORTED;
    if (bytes == 0)
        return TV_OK;
    if (!buf || !chunk_xor)
        return TV_ERR_NULL;
    if (ceil_div(bytes, tv::kStreamChunkBytes) > 0xffffff)   // 256-thread workgroups
        return TV_ERR_UNSUPPORTED;
    if (!aligned(buf, 16) || !aligned(chunk_xor, 4))
        return TV_ERR_ALIGNMENT;
    tv::StreamReadArgs a{buf, bytes / 16, chunk_xor};
    return from_hip(tv::launch_stream_read(a, static_cast<hipStream_t>(stream)));
}
