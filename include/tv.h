/*
 * tv.h -- C interface of libtv: the decode step of a paged KV cache on
 * AMD Instinct MI355X (gfx950).
 *
 * Three calls make one decode step for one attention layer:
 *   1. tv_cache_write            -- store each new token's K and V in the slot
 *                                   the engine chose for it;
 *   2. tv_paged_attention_decode -- grouped-query attention of each sequence's
 *                                   newest query over its whole cached context,
 *                                   one partial result per context partition;
 *   3. tv_paged_attention_reduce -- merge the partial results into the output.
 * tv_paged_attention_decode_append does steps 1 and 2 in one launch when each
 * sequence brings one new token.
 *
 * Sources (the pages this library is built from):
 *   - "vLLM" (blog.rlaisqls.com), section "가상 메모리 방식의 해결": the KV
 *     cache is split into fixed-size blocks (16 tokens by default) and each
 *     sequence keeps a table from logical positions to physical blocks, which
 *     need not be contiguous; blocks may be shared between sequences.
 *   - "Tiny-vLLM: 거대 LLM 추론, 작은 엔진이..." (trendpick100.com), second
 *     Q&A: before the model runs, the engine supplies a slot_mapping telling
 *     the KV store where each token's key/value vectors are written.
 *   - "vLLM", section "Flash Attention": attention is S = Q K^T,
 *     P = softmax(S), O = P V, and can be accumulated block by block with a
 *     running maximum and a running sum (online softmax).
 *   - "tiny-vllm 씹뜯맛즐 - (1)" (geonuchoi.com), section "2. Multi-Head
 *     Attention 대신 GQA": consecutive query heads share one K/V head
 *     (query heads 0-3 -> K/V head 0, 4-7 -> K/V head 1, ...).
 *
 * Conventions for every call:
 *   - Pointers are DEVICE pointers on the current HIP device, except where
 *     stated.  bf16 values travel as raw 16-bit patterns (uint16_t).
 *   - The caller allocates and owns every buffer, including the partition
 *     workspace.  The library allocates nothing, frees nothing and keeps no
 *     state between calls; it is safe to call from several host threads.
 *   - Work is queued on `stream` (a hipStream_t; NULL = the default stream)
 *     and the call returns without waiting for it.  Buffers must stay alive
 *     until the stream has passed the call.
 *   - Arguments are checked on the host before anything is launched; on any
 *     error nothing is launched and nothing is written.
 *   - Device data cannot raise errors; the kernels' behaviour on odd data is
 *     defined per call below and never reads or writes outside the buffers.
 *
 * Cache layout (a pool of num_blocks physical blocks; K and V pools separate):
 *   K pool: [num_blocks][num_kv_heads][head_dim / 8][block_size][8]
 *   V pool: [num_blocks][num_kv_heads][head_dim][block_size]
 * i.e. one (block, K/V head) tile of K is head_dim / 8 chunks, chunk c holding
 * dimensions 8c..8c+7 of every token of the block (16 bytes per token), and
 * the matching V tile holds its values dimension-major.  Both tiles are
 * contiguous (block_size * head_dim values each).  Token position t of a
 * sequence lives in physical block block_table[t / block_size] at offset
 * t % block_size; its slot number is block * block_size + offset.
 */
#ifndef TV_H
#define TV_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum tv_status {
    TV_OK = 0,
    TV_ERR_NULL = 1,         /* a required pointer is NULL */
    TV_ERR_SHAPE = 2,        /* sizes are negative, zero where they must not be, or inconsistent */
    TV_ERR_UNSUPPORTED = 3,  /* valid shape that this build does not implement */
    TV_ERR_HIP = 4,          /* the HIP runtime reported an error when launching */
    TV_ERR_ALIGNMENT = 5,    /* a pointer is not aligned as required */
    TV_ERR_NO_BLOCKS = 6,    /* block manager: no free block left (or host memory exhausted) */
    TV_ERR_SCRATCH = 7       /* the call's workspace exceeds the fixed scratch array
                                (tv_paged_attention_decode_step_noalloc) */
} tv_status;

/* Human-readable name of a status code (static storage; never NULL). */
const char *tv_status_string(tv_status status);

/*
 * Number of context partitions the decode call uses for contexts of up to
 * max_context_len tokens: ceil(max_context_len / partition_size).  Returns 0
 * for max_context_len <= 0 and -1 if partition_size <= 0.  (Host-only.)
 */
int32_t tv_num_partitions(int32_t max_context_len, int32_t partition_size);

/*
 * Cache write ("Tiny-vLLM" page, slot_mapping; "vLLM" page, blocks).
 *
 * For every token i < num_tokens with 0 <= slot_mapping[i] < num_blocks *
 * block_size, with b = slot_mapping[i] / block_size, o = slot_mapping[i] %
 * block_size, for every K/V head h and dimension d:
 *     k_cache[b][h][d / 8][o][d % 8] = k[i][h][d]
 *     v_cache[b][h][d][o]            = v[i][h][d]
 * Other tokens (negative slots mark padding; slots past the pool) are
 * skipped.  Every other element of the pools keeps its bits.  The copy is
 * bit-exact.
 *
 *   k, v          [num_tokens][num_kv_heads][head_dim] bf16, 16-byte aligned
 *   k_cache       K pool (layout above), 16-byte aligned
 *   v_cache       V pool (layout above), 2-byte aligned
 *   slot_mapping  int64 [num_tokens], 8-byte aligned
 *   head_dim      multiple of 8
 *
 * Two tokens naming the same slot is a caller error: which one lands is not
 * specified.  num_tokens == 0 is a no-op (pointers may then be NULL).
 * Errors: TV_ERR_NULL, TV_ERR_SHAPE (negative count, non-positive sizes),
 * TV_ERR_UNSUPPORTED (head_dim not a multiple of 8, or num_tokens above
 * 4 * (2^24 - 1): the launch grid), TV_ERR_ALIGNMENT, TV_ERR_HIP.
 */
tv_status tv_cache_write(const uint16_t *k, const uint16_t *v,
                         uint16_t *k_cache, uint16_t *v_cache,
                         const int64_t *slot_mapping, int64_t num_tokens,
                         int32_t num_kv_heads, int32_t head_dim,
                         int32_t block_size, int64_t num_blocks, void *stream);

/*
 * Rotary position embedding ("tiny-vllm 씹뜯맛즐 - (1)" page, section "5. 절대
 * 위치 임베딩 대신 RoPE": q and k of position p are turned by a rotation R_p,
 * so that (R_i q)^T (R_j k) = q^T R_{j-i} k; "tiny-vLLM으로 처음부터 고성능 LLM
 * 추론 엔진 구축하기" page: complex-number math with sine and cosine, done
 * inline in the kernels).
 *
 * R_p turns each pair of dimensions (a, b) = pair k, k < head_dim / 2, by the
 * angle positions[i] * inv_freq[k]:  a' = a cos - b sin,  b' = a sin + b cos.
 *   rope_style 0: pair k = dims (2k, 2k+1) (the pair as a complex number);
 *   rope_style 1: pair k = dims (k, k + head_dim/2).
 * The angle is formed exactly and reduced modulo 2 pi in the kernel; the
 * rotated values are computed in fp32 and rounded to bf16 (ties to even).
 * inv_freq (float [head_dim / 2], device) is the caller's: base^(-2k/D) for
 * plain RoPE, or any scaled table (context-extension schemes only change it).
 *
 * tv_cache_write_rope: tv_cache_write with every written token's K turned by
 * R_{positions[i]} (V is copied unchanged).
 *   positions  int32 [num_tokens] (device), 4-byte aligned; the position of
 *              each token in its sequence (not its slot)
 *   other arguments as for tv_cache_write
 * tv_rope: x [num_tokens][num_heads][head_dim] bf16 (16-byte aligned) turned
 * in place by R_{positions[i]} (q before attention, or a new token's K before
 * tv_paged_attention_decode_append).
 * Supported: head_dim a multiple of 8, at most 128; num_tokens at most
 * 4 * (2^24 - 1) (the launch grid).  Errors: TV_ERR_NULL,
 * TV_ERR_SHAPE (negative counts, non-positive sizes, a style other than 0/1),
 * TV_ERR_UNSUPPORTED, TV_ERR_ALIGNMENT, TV_ERR_HIP.  num_tokens == 0 is a no-op.
 */
tv_status tv_cache_write_rope(const uint16_t *k, const uint16_t *v, uint16_t *k_cache,
                              uint16_t *v_cache, const int64_t *slot_mapping,
                              const int32_t *positions, const float *inv_freq,
                              int64_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                              int32_t block_size, int64_t num_blocks, int32_t rope_style,
                              void *stream);
tv_status tv_rope(uint16_t *x, const int32_t *positions, const float *inv_freq,
                  int64_t num_tokens, int32_t num_heads, int32_t head_dim, int32_t rope_style,
                  void *stream);

/*
 * Paged decode attention, partition pass ("vLLM" page: PagedAttention and
 * Flash Attention's online softmax; "tiny-vllm" page: GQA grouping).
 *
 * For every sequence s with n = context_lens[s] cached tokens (the token just
 * written included), every query head h (K/V head g = h / (num_q_heads /
 * num_kv_heads)) and every partition p < ceil(n / partition_size) covering
 * token positions [p * partition_size, min((p+1) * partition_size, n)):
 *     part_max[s][h][p]    = max over the partition of scale * q[s][h] . K_t,
 *                            in base-2 units (multiplied by log2(e))
 *     part_sum[s][h][p]    = sum over the partition of 2^(score_t - part_max)
 *     part_acc[s][h][p][:] = sum over the partition of 2^(score_t - part_max) * V_t
 * (score_t in the same base-2 units).  Entries for p >= ceil(n /
 * partition_size) are not written.  tv_paged_attention_reduce turns these
 * into softmax(scale * q K^T) V.
 *
 *   part_acc      float [num_seqs][num_q_heads][P][head_dim], P = tv_num_partitions(max_context_len, partition_size),
 *                 16-byte aligned (written with 16-byte stores)
 *   part_max      float [num_seqs][num_q_heads][P], 4-byte aligned
 *   part_sum      float [num_seqs][num_q_heads][P], 4-byte aligned
 *   q             bf16  [num_seqs][num_q_heads][head_dim], 16-byte aligned
 *   k_cache, v_cache  pools as above, 16-byte aligned
 *   block_tables  int32 [num_seqs][max_blocks_per_seq].  Only the first
 *                 ceil(n / block_size) entries of a row are used.  Entries
 *                 up to min(max_blocks_per_seq, P * partition_size /
 *                 block_size) of a row may be read (a partition's entries
 *                 are loaded before its length is known), so the whole row
 *                 must be readable memory; what unused entries hold does not
 *                 matter
 *   context_lens  int32 [num_seqs]
 *   max_context_len  host-side upper bound of context_lens (sizes the launch);
 *                 must be <= max_blocks_per_seq * block_size
 *   partition_size   tokens per partition, a positive multiple of block_size
 *   scale         score factor (1/sqrt(head_dim) for standard attention), > 0
 *
 * Supported shapes: head_dim == 64, block_size == 16, 1 <= num_q_heads /
 * num_kv_heads <= 16 (num_q_heads a multiple of num_kv_heads), and
 * num_kv_heads * num_seqs * P < 2^24 (the launch grid).
 * Odd device data: a context length below 0 counts as 0 and one above
 * max_context_len is cut to max_context_len; a table entry outside
 * [0, num_blocks) drops that block's tokens from the softmax (a partition with
 * no usable token gets part_max = -inf, part_sum = 0, part_acc = 0).
 * Tokens at positions >= n are never read, so stale or NaN data there and in
 * unused table entries cannot reach the result.
 * Errors: TV_ERR_NULL, TV_ERR_SHAPE, TV_ERR_UNSUPPORTED, TV_ERR_ALIGNMENT,
 * TV_ERR_HIP.  num_seqs == 0 or max_context_len == 0 is a no-op.
 */
tv_status tv_paged_attention_decode(float *part_acc, float *part_max, float *part_sum,
                                    const uint16_t *q,
                                    const uint16_t *k_cache, const uint16_t *v_cache,
                                    const int32_t *block_tables, const int32_t *context_lens,
                                    int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                    int32_t head_dim, int32_t block_size,
                                    int32_t max_blocks_per_seq, int64_t num_blocks,
                                    int32_t max_context_len, int32_t partition_size,
                                    float scale, void *stream);

/*
 * The same partition pass with the QK and PV contractions on the vector ALUs
 * (v_dot2_f32_bf16 scores, lane-swap and DPP reductions, the weights read out
 * to scalar registers for the PV multiply-adds) instead of MFMA: the same
 * partials as tv_paged_attention_decode, from the same softmax definition,
 * up to fp32 rounding order.  It exists as the measured alternative to the
 * matrix form ("vLLM" page, section "Flash Attention": the score and
 * weighted-sum products of each partition); on MI355X it is the slower of the
 * two on every workload measured, so no other call takes it.
 * Arguments, layouts, alignment and defined behaviour on odd data are those of
 * tv_paged_attention_decode.  Supported shapes: as there, with exactly 4 query
 * heads per K/V head (num_q_heads == 4 * num_kv_heads); other groupings give
 * TV_ERR_UNSUPPORTED.
 */
tv_status tv_paged_attention_decode_vector(float *part_acc, float *part_max, float *part_sum,
                                           const uint16_t *q, const uint16_t *k_cache,
                                           const uint16_t *v_cache, const int32_t *block_tables,
                                           const int32_t *context_lens, int32_t num_seqs,
                                           int32_t num_q_heads, int32_t num_kv_heads,
                                           int32_t head_dim, int32_t block_size,
                                           int32_t max_blocks_per_seq, int64_t num_blocks,
                                           int32_t max_context_len, int32_t partition_size,
                                           float scale, void *stream);

/*
 * Partition pass for sequences that share a prompt prefix ("vLLM" page,
 * section "가상 메모리 방식의 해결": the samples of one prompt share its
 * blocks).  The same partials as tv_paged_attention_decode; the shared
 * prefix's tiles are read once per group instead of once per sequence.
 *
 * The sequences at positions g*group_size .. min((g+1)*group_size, num_seqs)
 * - 1 form group g, where position p holds sequence group_order[p] (a
 * permutation of 0 .. num_seqs-1), or sequence p when group_order is NULL.
 * With sh = min(shared_len[g], context length of every member of g), the
 * partitions p < floor(sh / partition_size) of the group's members are
 * computed together from the block table of the group's first member.
 * Precondition: for those positions every member's table holds the same
 * blocks as the first member's (as after tv_bm_fork).  Then the partials are
 * those of tv_paged_attention_decode bit for bit.  shared_len[g] = 0 (or
 * group_size 1) leaves a group to the per-sequence pass.
 *
 *   shared_len   int32 [ceil(num_seqs / group_size)] (device), 4-byte aligned
 *   group_order  int32 [num_seqs] (device) or NULL, 4-byte aligned.  An entry
 *                outside [0, num_seqs) leaves its position out (its group
 *                shares nothing); a sequence listed twice, or not at all, is
 *                the caller's error (its partials are computed twice, or not
 *                written).
 *   group_size   1 .. 16 / (num_q_heads / num_kv_heads)  (4 for groups of 4 heads)
 *   other arguments as for tv_paged_attention_decode.
 * Errors: as for tv_paged_attention_decode, plus TV_ERR_SHAPE for
 * group_size < 1, TV_ERR_UNSUPPORTED for a group too large for one MFMA's 16
 * columns, TV_ERR_NULL for a NULL shared_len.
 */
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
                                           float scale, void *stream);

/*
 * Partition pass with the cache write folded in (the same two steps as
 * tv_cache_write of one new token per sequence followed by
 * tv_paged_attention_decode, in one launch).
 *
 * For every sequence s with n = context_lens[s] >= 1 (n counts the new token)
 * and 0 <= slot_mapping[s] < num_blocks * block_size, the new token's K and V
 * (k_new[s], v_new[s]: [num_kv_heads][head_dim] bf16) are written into that
 * slot exactly as tv_cache_write writes token s; slot_mapping[s] < 0 (or
 * n == 0) appends nothing for s.  The partials are then those of
 * tv_paged_attention_decode over the pools after the writes.
 *
 * Precondition (the usual one for a decode step, where the block a sequence
 * appends to is its own): slot_mapping[s] is negative or is the slot the
 * block table gives for position n - 1 of sequence s, no other sequence of
 * the call reads that slot, and no other sequence of the call appends into
 * the same block.  Then the result equals the two-call sequence bit for bit.
 * The token is written by storing back the whole 16-token tile of its block
 * and head as this call read it, with the new token in place; another
 * sequence appending into the same block in the same call may therefore
 * lose its token.  A slot elsewhere is still written (its row alone), but
 * position n - 1 is read from the pool, and a slot that another sequence of
 * the same call reads gives unspecified values for that sequence.
 *
 *   k_new         bf16 [num_seqs][num_kv_heads][head_dim], 16-byte aligned
 *   v_new         bf16 [num_seqs][num_kv_heads][head_dim], 16-byte aligned
 *   slot_mapping  int64 [num_seqs], 8-byte aligned
 *   other arguments as for tv_paged_attention_decode (the pools writable).
 * Supported shapes and errors: as for tv_paged_attention_decode, plus
 * TV_ERR_NULL for a NULL k_new, v_new or slot_mapping.
 */
tv_status tv_paged_attention_decode_append(float *part_acc, float *part_max, float *part_sum,
                                           const uint16_t *q, const uint16_t *k_new,
                                           const uint16_t *v_new, const int64_t *slot_mapping,
                                           uint16_t *k_cache, uint16_t *v_cache,
                                           const int32_t *block_tables,
                                           const int32_t *context_lens,
                                           int32_t num_seqs, int32_t num_q_heads,
                                           int32_t num_kv_heads, int32_t head_dim,
                                           int32_t block_size, int32_t max_blocks_per_seq,
                                           int64_t num_blocks, int32_t max_context_len,
                                           int32_t partition_size, float scale, void *stream);

/*
 * Shared-prefix partition pass with the cache write folded in: the same
 * results as tv_cache_write of one new token per sequence (as in
 * tv_paged_attention_decode_append) followed by
 * tv_paged_attention_decode_shared, in one launch on `stream` (the group
 * pass's workgroups first, then the per-sequence ones, which also write the
 * tokens).  The
 * parallel-sampling decode step ("vLLM" page, section "가상 메모리 방식의
 * 해결": samples share their prompt's blocks; each sample's new token goes
 * to a block of its own).
 *
 * Preconditions: those of both calls -- slot_mapping[s] is negative or the
 * slot the block table gives for position n - 1 of sequence s, and for the
 * shared positions every member's table holds the first member's blocks --
 * and position n - 1 of every member lies past its group's shared
 * partitions (n - 1 >= floor(sh / partition_size) * partition_size, sh as
 * for tv_paged_attention_decode_shared), which holds whenever the new token's
 * block is the member's own.  Then the partials equal the two-call sequence
 * bit for bit.  If a member's position n - 1 lies in a shared partition, its
 * token is still written, but the group pass has attended that slot's
 * previous contents.
 *
 *   arguments as for tv_paged_attention_decode_append, plus shared_len,
 *   group_order and group_size as for tv_paged_attention_decode_shared.
 * Supported shapes and errors: the union of both calls'.
 */
tv_status tv_paged_attention_decode_shared_append(
    float *part_acc, float *part_max, float *part_sum, const uint16_t *q, const uint16_t *k_new,
    const uint16_t *v_new, const int64_t *slot_mapping, uint16_t *k_cache, uint16_t *v_cache,
    const int32_t *block_tables, const int32_t *context_lens, const int32_t *shared_len,
    const int32_t *group_order, int32_t group_size, int32_t num_seqs, int32_t num_q_heads,
    int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
    int64_t num_blocks, int32_t max_context_len, int32_t partition_size, float scale,
    void *stream);

/*
 * The parallel-sampling decode step in one call ("vLLM" page, section "가상
 * 메모리 방식의 해결": the samples of one prompt share its blocks, and each
 * sample's new token goes to a block of its own; section "Flash Attention":
 * the running maximum / running sum rule): the cache write of one new token
 * per sequence, shared-prefix attention and the log-sum-exp merge, writing
 * out = softmax(q K^T * scale) V per (sequence, query head) as
 * tv_paged_attention_decode_shared_append followed by
 * tv_paged_attention_reduce would.
 *
 * Forms (from the shapes alone, never the data; a call is deterministic):
 *   group_size <= 4 (with or without group_order) and every (group, K/V
 *   head) workgroup resident at once on the device (num_groups *
 *   num_kv_heads <= 2 * 256 on MI355X): one launch with one 8-wavefront
 *   workgroup per (group, K/V head).  The group's shared tiles (its shared length cut as for
 *   tv_paged_attention_decode_shared) are read once with every member's
 *   query heads, each member's other tiles with its own; the group's tiles
 *   (the shared ones, then each member's) are cut into 8 equal consecutive
 *   parts, one per wavefront, and the parts merge in on-chip memory.  The
 *   workspace is neither read nor written (it must still be non-NULL and
 *   aligned), and out equals the two-call result up to rounding, within
 *   2^-16 * max|V| as for tv_paged_attention_decode_step's one-launch forms
 *   (the parts are not its 512-token partitions).
 *   otherwise: tv_paged_attention_decode_shared_append, then
 *   tv_paged_attention_reduce, on `stream`; out bitwise the two calls'.
 * With max_context_len == 0 every row of out is set to zero.
 *
 *   out   float [num_seqs][num_q_heads][head_dim], 16-byte aligned
 *   other arguments, preconditions and odd-data behaviour as for
 *   tv_paged_attention_decode_shared_append (the workspace sized for
 *   ceil(max_context_len / partition_size) partitions).
 * Supported shapes: those of tv_paged_attention_decode_shared_append, and
 * num_seqs * num_q_heads < 2^24.  Errors: TV_ERR_NULL, TV_ERR_SHAPE,
 * TV_ERR_UNSUPPORTED, TV_ERR_ALIGNMENT, TV_ERR_HIP; all argument errors are
 * found before anything is launched.  num_seqs == 0 is a no-op.
 */
tv_status tv_paged_attention_decode_shared_step(
    float *out, float *part_acc, float *part_max, float *part_sum, const uint16_t *q,
    const uint16_t *k_new, const uint16_t *v_new, const int64_t *slot_mapping, uint16_t *k_cache,
    uint16_t *v_cache, const int32_t *block_tables, const int32_t *context_lens,
    const int32_t *shared_len, const int32_t *group_order, int32_t group_size, int32_t num_seqs,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
    int32_t max_blocks_per_seq, int64_t num_blocks, int32_t max_context_len,
    int32_t partition_size, float scale, void *stream);

/*
 * Which form tv_paged_attention_decode_shared_step takes for these shapes on
 * the current device: 0 nothing is launched (num_seqs == 0 or
 * max_context_len == 0), 1 one launch (one workgroup per (group, K/V head)),
 * 2 two launches through the workspace, -1 the step would reject these
 * shapes.  has_group_order: nonzero if a group_order array is passed (it
 * does not change the form).
 * Host-only; reads the current device's compute-unit count and occupancy.
 */
int32_t tv_paged_attention_decode_shared_step_form(int32_t num_seqs, int32_t num_q_heads,
                                                   int32_t num_kv_heads, int32_t head_dim,
                                                   int32_t block_size, int32_t max_context_len,
                                                   int32_t partition_size, int32_t group_size,
                                                   int32_t has_group_order);

/*
 * Log-sum-exp merge of the partitions ("vLLM" page, Flash Attention: the
 * running maximum / running sum rule applied across partitions).
 *
 * For every sequence s and query head h, with P_s = ceil(n / partition_size)
 * partitions (n = context_lens[s], cut to [0, max_context_len]):
 *     M = max_p part_max[s][h][p],  w_p = 2^(part_max[s][h][p] - M)
 *     out[s][h][:] = (sum_p w_p * part_acc[s][h][p][:]) / (sum_p w_p * part_sum[s][h][p])
 * over p < P_s.  A sequence with n == 0 (or whose partitions hold no usable
 * token) gets a zero row.
 *
 *   out           float [num_seqs][num_q_heads][head_dim], 16-byte aligned
 *   part_*        as written by tv_paged_attention_decode with the same
 *                 num_seqs, num_q_heads, head_dim, max_context_len and
 *                 partition_size; part_acc 16-byte aligned
 *   context_lens  int32 [num_seqs]
 *
 * Supported shapes: head_dim == 64, num_seqs * num_q_heads < 2^24 (one
 * workgroup per row in the launch grid).
 * Errors: TV_ERR_NULL, TV_ERR_SHAPE, TV_ERR_UNSUPPORTED, TV_ERR_ALIGNMENT,
 * TV_ERR_HIP.  num_seqs == 0 is a no-op.  With max_context_len == 0 every row
 * of out is set to zero.
 */
tv_status tv_paged_attention_reduce(float *out, const float *part_acc,
                                    const float *part_max, const float *part_sum,
                                    const int32_t *context_lens,
                                    int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                                    int32_t max_context_len, int32_t partition_size,
                                    void *stream);

/*
 * A whole decode step in one call: the new tokens' cache write, the partition
 * pass and the log-sum-exp merge ("vLLM" page, Flash Attention: the running
 * maximum / running sum rule; a single partition merges to acc / l).
 *
 * With P = ceil(max_context_len / partition_size) the call takes one of
 * three forms; all compute the same softmax(q K^T * scale) V per row, and the
 * form depends only on the shapes, never on the data, so a call is
 * deterministic:
 *   P == 1: the partition pass divides by the sum itself and writes out; one
 *     launch; out is bitwise what tv_paged_attention_decode_append followed
 *     by tv_paged_attention_reduce gives.
 *   2 <= P <= 8, num_seqs <= 256 and num_seqs * num_kv_heads within one
 *     resident wave of workgroups on the device: one launch with one
 *     workgroup per (sequence, K/V head); each sequence's context is cut
 *     into 8 equal consecutive ranges (each at most partition_size tokens),
 *     one per wavefront, and the 8 partial results are merged in on-chip
 *     memory by the same log-sum-exp rule.  The ranges differ from the
 *     partition_size partitions of the two-call form, so out equals that
 *     form's result up to rounding, not bitwise: both fold the softmax
 *     weights into V with at least 16 significant bits against an exact
 *     fp32 sum, so the two are within 2^-16 * max|V| (plus fp32 summation
 *     order) of each other.
 *   otherwise: tv_paged_attention_decode_append followed by
 *     tv_paged_attention_reduce on the same stream, two launches through the
 *     workspace; out is bitwise what those two calls give.
 * With max_context_len == 0 every row of out is set to zero.
 *
 *   out        float [num_seqs][num_q_heads][head_dim], 16-byte aligned
 *   part_*     the workspace as for tv_paged_attention_decode (part_acc
 *              16-byte aligned), sized for P partitions; unused (may be NULL)
 *              with one partition; in the one-launch form for 2 <= P <= 8 it
 *              is neither read nor written, but must still be non-NULL and
 *              aligned as stated
 *   other arguments, the append precondition and the odd-data behaviour as
 *   for tv_paged_attention_decode_append
 *
 * Supported shapes: those of tv_paged_attention_decode_append, and
 * num_seqs * num_q_heads < 2^24.  Errors: TV_ERR_NULL, TV_ERR_SHAPE,
 * TV_ERR_UNSUPPORTED, TV_ERR_ALIGNMENT, TV_ERR_HIP; all argument errors are
 * found before anything is launched.  num_seqs == 0 is a no-op.
 */
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
                                         float scale, void *stream);

/*
 * Which form tv_paged_attention_decode_step (and its _noalloc variant) takes
 * for these shapes on the current device, with
 * P = ceil(max_context_len / partition_size):
 *   0  nothing is launched (num_seqs == 0 or max_context_len == 0)
 *   1  one launch, one partition (P == 1)
 *   2  one launch, one workgroup per (sequence, K/V head) (2 <= P <= 8 and
 *      the grid fits one resident wave of workgroups)
 *   3  two launches through the workspace
 *  -1  the step would reject these shapes (TV_ERR_SHAPE or
 *      TV_ERR_UNSUPPORTED)
 * Host-only; reads the current device's compute-unit count and occupancy
 * (the first call on a device queries the runtime).  Launches nothing.
 */
int32_t tv_paged_attention_decode_step_form(int32_t num_seqs, int32_t num_q_heads,
                                            int32_t num_kv_heads, int32_t head_dim,
                                            int32_t block_size, int32_t max_context_len,
                                            int32_t partition_size);

/*
 * The decode step for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Computes exactly what tv_paged_attention_decode_step computes (out is
 * bitwise the same: the same form is taken for the same shapes) and takes the same arguments minus the workspace: the
 * partition workspace lives in a fixed device array of
 * TV_NOALLOC_SCRATCH_BYTES inside the library, one per GPU, held from the
 * first such call on that GPU until the process ends.  The call allocates
 * nothing and frees nothing.
 *
 * Limit: with P = ceil(max_context_len / partition_size) > 1 the workspace is
 * num_seqs * num_q_heads * P * (head_dim + 2) * 4 bytes and must not exceed
 * TV_NOALLOC_SCRATCH_BYTES (16 MiB: e.g. 64 sequences x 32 heads x 8
 * partitions of 512 tokens takes 4.3 MB, 4 x 32 x 256 partitions 8.7 MB);
 * beyond it the call returns TV_ERR_SCRATCH before anything is launched.
 * With P <= 1 no workspace is used and there is no limit.
 *
 * Every call on one GPU shares that GPU's array and may leave anything in
 * it; nothing in it needs clearing between calls.  Calls that overlap on one
 * GPU (two streams, or two host threads without ordering) race on the array
 * and give unspecified results: order them on one stream.
 *
 * Errors: those of tv_paged_attention_decode_step, plus TV_ERR_SCRATCH.
 */
#define TV_NOALLOC_SCRATCH_BYTES (16 * 1024 * 1024)
tv_status tv_paged_attention_decode_step_noalloc(
    float *out, const uint16_t *q, const uint16_t *k_new, const uint16_t *v_new,
    const int64_t *slot_mapping, uint16_t *k_cache, uint16_t *v_cache,
    const int32_t *block_tables, const int32_t *context_lens, int32_t num_seqs,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
    int32_t max_blocks_per_seq, int64_t num_blocks, int32_t max_context_len,
    int32_t partition_size, float scale, void *stream);

/*
 * Prefill and chunked prefill ("tiny-vLLM으로 처음부터 고성능 LLM 추론 엔진
 * 구축하기" page, section "고급 추론 개념": prefill runs the whole prompt,
 * decode only the newest token; "tiny-vllm 씹뜯맛즐 - (1)" page, section 1:
 * causal decoder; "vLLM" page: paged K/V and Flash Attention's online softmax).
 *
 * Sequence s brings m = query_start[s+1] - query_start[s] query rows, q rows
 * query_start[s] .. query_start[s+1]-1, which are the last m positions of its
 * n = context_lens[s] cached positions (the chunk's own K/V already written,
 * e.g. by tv_cache_write).  Row query_start[s] + i sits at position
 * p = n - m + i and, for every query head h (K/V head h / (num_q_heads /
 * num_kv_heads)):
 *     out[row][h][:] = softmax over t <= p of (scale * q[row][h] . K_t) applied to V_t.
 * A full prefill is m = n; m = 1 is a decode step.  Rows with p < 0 (a chunk
 * longer than the context) are 0.
 *
 *   out           float [rows][num_q_heads][head_dim], 16-byte aligned
 *   q             bf16  [rows][num_q_heads][head_dim], 16-byte aligned
 *   query_start   int32 [num_seqs + 1], non-decreasing (device)
 *   k_cache, v_cache, block_tables, context_lens   as for the decode call
 *   max_query_len    host-side upper bound of the m; rows i >= max_query_len
 *                    of a sequence are not written
 *   max_context_len  host-side upper bound of context_lens, <= max_blocks_per_seq * block_size
 *
 * Supported shapes: head_dim == 64, block_size == 16, num_q_heads /
 * num_kv_heads in {1, 2, 4, 8, 16}; num_kv_heads * num_seqs *
 * ceil(max_query_len / (256 / (num_q_heads / num_kv_heads))) < 2^23 (the
 * launch grid).  Arithmetic: bf16 products accumulated
 * in fp32, softmax weights rounded to bf16 for the product with V.  The
 * summation order, and so the last bits of the result, follows from the
 * host bounds and the device: a launch of fewer workgroups than two per
 * compute unit splits each row's keys into two interleaved shares merged at
 * the end.  The same call on the same device gives the same bits.
 * Odd device data as for the decode call: context lengths are clamped to
 * [0, max_context_len], table entries outside [0, num_blocks) drop their
 * tokens (a row left with no token is 0), positions >= n are never read.
 * Errors: TV_ERR_NULL, TV_ERR_SHAPE, TV_ERR_UNSUPPORTED, TV_ERR_ALIGNMENT,
 * TV_ERR_HIP.  num_seqs == 0 or max_query_len == 0 is a no-op.
 */
tv_status tv_paged_attention_prefill(float *out, const uint16_t *q, const int32_t *query_start,
                                     const uint16_t *k_cache, const uint16_t *v_cache,
                                     const int32_t *block_tables, const int32_t *context_lens,
                                     int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                     int32_t head_dim, int32_t block_size,
                                     int32_t max_blocks_per_seq, int64_t num_blocks,
                                     int32_t max_query_len, int32_t max_context_len, float scale,
                                     void *stream);

/*
 * Copy-on-write support ("vLLM" page, section "가상 메모리 방식의 해결":
 * requests sharing a prompt share its blocks; a block is copied when a branch
 * writes into it).
 *
 * For every pair i < num_pairs, with src = block_pairs[2i] and dst =
 * block_pairs[2i + 1]: every element of block dst (all K/V heads, both pools)
 * becomes a copy of the same element of block src.  Pairs with src or dst
 * outside [0, num_blocks), or src == dst, are skipped.  The copy is bit-exact.
 *
 *   k_cache, v_cache  pools (layout above), 16-byte aligned
 *   block_pairs   int64 [num_pairs][2] (device), 8-byte aligned
 *   num_kv_heads * head_dim * block_size must be a multiple of 8
 *
 * The destinations must be distinct and no destination may also be a source
 * of the same call; otherwise the result is unspecified.  num_pairs < 2^24
 * (the launch grid); num_pairs == 0 is a
 * no-op.  Errors: TV_ERR_NULL, TV_ERR_SHAPE, TV_ERR_UNSUPPORTED,
 * TV_ERR_ALIGNMENT, TV_ERR_HIP.
 */
tv_status tv_copy_blocks(uint16_t *k_cache, uint16_t *v_cache, const int64_t *block_pairs,
                         int64_t num_pairs, int32_t num_kv_heads, int32_t head_dim,
                         int32_t block_size, int64_t num_blocks, void *stream);

/*
 * Block manager: host-side bookkeeping of the physical blocks ("vLLM" page,
 * section "가상 메모리 방식의 해결": blocks handed out one at a time as tokens
 * arrive -- 300 tokens take 19 blocks of 16 --, a per-sequence table from
 * logical to physical blocks that need not be contiguous, and blocks shared
 * between requests of one prompt with copy-on-write at the branch).
 *
 * A manager owns num_blocks physical block numbers and up to max_seqs
 * sequences, identified by the caller's numbers 0 .. max_seqs-1.  It keeps a
 * reference count per block: a block returns to the free list when no
 * sequence refers to it.  The first blocks handed out are 0, 1, 2, ...; freed
 * blocks are reused first.  All calls are host-only, do no GPU work and are
 * not thread-safe for one manager (different managers are independent).
 * The caller moves K/V data: tv_cache_write (or
 * tv_paged_attention_decode_append) for the slots the manager returns, and
 * tv_copy_blocks for the copy-on-write pairs it returns.
 */
typedef struct tv_block_manager tv_block_manager;

/* New manager in *out (NULL on failure).  TV_ERR_SHAPE for non-positive sizes,
 * TV_ERR_NO_BLOCKS if host memory runs out. */
tv_status tv_bm_create(int32_t num_blocks, int32_t block_size, int32_t max_seqs,
                       int32_t max_blocks_per_seq, tv_block_manager **out);
void tv_bm_destroy(tv_block_manager *bm);              /* NULL is a no-op */

/* Free blocks; reference count of a block; token count of a sequence (-1 for
 * an unused sequence number or a bad argument). */
int32_t tv_bm_num_free(const tv_block_manager *bm);
int32_t tv_bm_refcount(const tv_block_manager *bm, int32_t block);
int32_t tv_bm_length(const tv_block_manager *bm, int32_t seq);

/* Start sequence `seq` (unused) with num_tokens positions and ceil(num_tokens /
 * block_size) fresh blocks.  TV_ERR_NO_BLOCKS (nothing changed) if too few
 * blocks are free; TV_ERR_SHAPE for a sequence in use or more than
 * max_blocks_per_seq blocks. */
tv_status tv_bm_add_sequence(tv_block_manager *bm, int32_t seq, int32_t num_tokens);

/* Sequence `child` (unused) starts as a copy of `parent`: same length, same
 * blocks, each block's reference count + 1.  No data moves. */
tv_status tv_bm_fork(tv_block_manager *bm, int32_t parent, int32_t child);

/* Reserve the next position n (= the current length) of `seq` and return its
 * slot (block * block_size + offset); the length becomes n + 1.
 *   - n % block_size == 0: a fresh block is appended to the table;
 *   - otherwise, if the block holding n is shared (reference count > 1), it is
 *     replaced in this table by a fresh block and *copy_src / *copy_dst name
 *     the pair the caller must copy (tv_copy_blocks) before writing the slot;
 *     else *copy_src = *copy_dst = -1.
 * TV_ERR_NO_BLOCKS (nothing changed) if a block is needed and none is free. */
tv_status tv_bm_append_slot(tv_block_manager *bm, int32_t seq, int64_t *slot,
                            int64_t *copy_src, int64_t *copy_dst);

/* One decode step's host-side inputs for the sequences seqs[0 .. num_seqs):
 * for r = 0, 1, ... in order, the next position of seqs[r] is reserved as by
 * tv_bm_append_slot, and then
 *   slot_mapping[r]             its slot,
 *   context_lens[r]             the new length (the new token included),
 *   block_tables[r*width + j]   block j of its table, 0 past its last block,
 *   copy_pairs[2c], [2c + 1]    the c-th copy-on-write pair (src, dst), in
 *                               order of r, c < *num_copies <= num_seqs.
 * All outputs are host memory: block_tables int32 [num_seqs][width],
 * context_lens int32 [num_seqs], slot_mapping int64 [num_seqs], copy_pairs
 * int64 [num_seqs][2].  These are the inputs of tv_copy_blocks (run first),
 * then tv_paged_attention_decode_append: every slot lies in a block that only
 * its own sequence's table holds, so the append precondition holds; the copy
 * destinations are fresh blocks, distinct and never a source of the call.
 * The seqs must be distinct live sequences whose new block count fits width
 * and max_blocks_per_seq, else TV_ERR_SHAPE before anything changes.
 * All-or-nothing: on TV_ERR_NO_BLOCKS (a block is needed and none is free)
 * every reservation already made is taken back, leaving the manager, its free
 * list order included, as before the call; the outputs are then unspecified.
 * num_seqs == 0 sets *num_copies = 0. */
tv_status tv_bm_prepare_decode(tv_block_manager *bm, const int32_t *seqs, int32_t num_seqs,
                               int32_t width, int32_t *block_tables, int32_t *context_lens,
                               int64_t *slot_mapping, int64_t *copy_pairs, int32_t *num_copies);

/* Drop sequence `seq`: every block's reference count - 1, blocks reaching 0
 * return to the free list. */
tv_status tv_bm_free_sequence(tv_block_manager *bm, int32_t seq);

/* The block table of `seq` into row[0 .. *num_blocks) (host memory);
 * TV_ERR_SHAPE if it has more than `width` blocks. */
tv_status tv_bm_block_table(const tv_block_manager *bm, int32_t seq, int32_t *row,
                            int32_t width, int32_t *num_blocks);

/* Slots of positions start .. start+count-1 of `seq` (host memory). */
tv_status tv_bm_slots(const tv_block_manager *bm, int32_t seq, int32_t start, int32_t count,
                      int64_t *slots);

/* ------------------------------------------------------------------------
 * Streaming-read yardstick.  The decode path is bound by HBM reads (the K/V
 * of every context token once per step), and its bytes per second are
 * reported as a fraction of the 8 TB/s specification and, for context, of
 * what a plain read of the same size achieves on the device.  This call is
 * that plain read: buf[0 .. bytes) read once, coalesced, non-temporal.
 *
 *   buf        device memory, 16-byte aligned; bytes a multiple of 16
 *   chunk_xor  uint32 [ceil(bytes / 8192)] (device), 4-byte aligned:
 *              entry c = XOR of the 32-bit words of bytes
 *              [8192 c, min(8192 (c + 1), bytes)), little-endian
 *
 * bytes == 0 is a no-op.  Errors: TV_ERR_SHAPE (bytes < 0), TV_ERR_NULL,
 * TV_ERR_UNSUPPORTED (bytes not a multiple of 16, or 2^24 chunks or more:
 * the launch grid), TV_ERR_ALIGNMENT, TV_ERR_HIP.
 * ---------------------------------------------------------------------- */
tv_status tv_stream_read(const void *buf, int64_t bytes, uint32_t *chunk_xor, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* TV_H */
