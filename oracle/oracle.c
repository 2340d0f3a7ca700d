/*
 * oracle.c -- plain, slow CPU reference for paged GQA attention (decode step,
 * prefill / chunked prefill, block copy, rotary position embedding).
 *
 * TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg load this library.  The GPU library never
 * calls it and shares no code, header or table with it.
 *
 * What it computes, and where the pages define it:
 *
 *   Cache write.  "Tiny-vLLM: 거대 LLM 추론, 작은 엔진이..." page, second Q&A
 *   ("'Tiny-vLLM'은 이 거대한 복잡성을..."): before the model runs, a
 *   slot_mapping tells the KV store where each new token's key/value vectors go.
 *   Slot encoding (our reading, the pages are silent): slot = block * BS + offset;
 *   a slot < 0 or >= NB * BS is padding and is skipped.
 *
 *   Paging.  "vLLM" page, section "가상 메모리 방식의 해결": the cache is cut
 *   into fixed blocks of 16 tokens and a table per sequence maps logical
 *   positions to physical blocks, like an OS page table.  Position t of
 *   sequence s lives in block block_tables[s][t / BS] at offset t % BS.
 *
 *   Attention.  "vLLM" page, section "Flash Attention": standard attention is
 *   S = Q K^T, P = softmax(S), O = P V.  The query is the newest token's; it
 *   attends to every cached position 0..n-1 of its sequence (decoder-only,
 *   causal: "tiny-vllm 씹뜯맛즐 - (1)" page, section 1).  Scores carry the
 *   factor 1/sqrt(head_dim) (0.125 for head_dim 64 = 2048 / 32, same page,
 *   dimension list after section 6).
 *
 *   GQA.  "tiny-vllm 씹뜯맛즐 - (1)" page, section "2. Multi-Head Attention
 *   대신 GQA", figure: query heads 0-3 share K/V head 0, heads 4-7 share K/V
 *   head 1, ...; so query head h reads K/V head h / (Hq / Hkv).
 *
 * Cache layout (part of the library's interface, indexed here on its own):
 *   K pool: [NB][Hkv][D/8][BS][8]  (one block and head = D/8 chunks; chunk c
 *                                   holds dimensions 8c..8c+7 of the BS tokens,
 *                                   8 consecutive values per token)
 *   V pool: [NB][Hkv][D][BS]       (one block and head stored dimension-major)
 *   bf16 values are raw uint16 bit patterns; head_dim is a multiple of 8.
 *
 * Arithmetic: double precision from the exact bf16 values; the two-pass
 * softmax of the definition (max, then exponentials, then their sum); no
 * blocking, no online update, no partitions.  The parallel loop runs over
 * (sequence, query head) pairs only, so results do not depend on the thread
 * count.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

#define KCHUNK 8    /* K pool: dimensions stored together per token (16 bytes) */

/* Element (block blk, K/V head h, token offset off, dimension d) of the K pool. */
static long k_index(long blk, int h, long off, int d, int num_kv_heads, int head_dim, int block_size)
{
    long tile = (blk * num_kv_heads + h) * (long)head_dim * block_size;
    return tile + ((long)(d / KCHUNK) * block_size + off) * KCHUNK + d % KCHUNK;
}

static double bf16_value(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/*
 * Copy token i's K and V rows (k, v: [T][Hkv][D]) into the slot
 * slot_mapping[i] of the pools.  Returns the number of tokens written,
 * -1 on a bad argument, -2 if two tokens name the same slot (no pool is
 * touched in either error case).
 */
long oracle_cache_write(const uint16_t *k, const uint16_t *v,
                        uint16_t *k_cache, uint16_t *v_cache,
                        const int64_t *slot_mapping, long num_tokens,
                        int num_kv_heads, int head_dim, int block_size,
                        long num_blocks)
{
    if (num_tokens < 0 || num_kv_heads < 1 || head_dim < 1 || head_dim % KCHUNK != 0 ||
        block_size < 1 || num_blocks < 1)
        return -1;
    long num_slots = num_blocks * (long)block_size;
    unsigned char *taken = calloc((size_t)num_slots, 1);
    if (!taken)
        return -1;
    for (long i = 0; i < num_tokens; ++i) {
        int64_t slot = slot_mapping[i];
        if (slot < 0 || slot >= num_slots)
            continue;
        if (taken[slot]) {
            free(taken);
            return -2;
        }
        taken[slot] = 1;
    }
    free(taken);

    long written = 0;
    for (long i = 0; i < num_tokens; ++i) {
        int64_t slot = slot_mapping[i];
        if (slot < 0 || slot >= num_slots)
            continue;
        long blk = (long)(slot / block_size);
        long off = (long)(slot % block_size);
        for (int h = 0; h < num_kv_heads; ++h) {
            for (int d = 0; d < head_dim; ++d) {
                long src = ((long)i * num_kv_heads + h) * head_dim + d;
                long kdst = k_index(blk, h, off, d, num_kv_heads, head_dim, block_size);
                long vdst = ((blk * num_kv_heads + h) * head_dim + d) * block_size + off;
                k_cache[kdst] = k[src];
                v_cache[vdst] = v[src];
            }
        }
        ++written;
    }
    return written;
}

/*
 * Copy-on-write of whole blocks ("vLLM" page, "가상 메모리 방식의 해결":
 * requests of one prompt share its blocks; a branch writing into a shared
 * block gets its own copy).  For each pair (src, dst) = (pairs[2i],
 * pairs[2i+1]), every element of block dst in both pools becomes a copy of
 * block src.  Pairs with a block outside the pool or src == dst are skipped.
 * Returns the number of blocks copied, -1 on a bad argument, -2 if a
 * destination repeats or is also a source (no pool is touched then).
 */
long oracle_copy_blocks(uint16_t *k_cache, uint16_t *v_cache, const int64_t *pairs,
                        long num_pairs, int num_kv_heads, int head_dim, int block_size,
                        long num_blocks)
{
    if (num_pairs < 0 || num_kv_heads < 1 || head_dim < 1 || block_size < 1 || num_blocks < 1)
        return -1;
    for (long i = 0; i < num_pairs; ++i) {
        int64_t src = pairs[2 * i], dst = pairs[2 * i + 1];
        if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks || src == dst)
            continue;
        for (long j = 0; j < num_pairs; ++j) {
            int64_t s2 = pairs[2 * j], d2 = pairs[2 * j + 1];
            int valid2 = s2 >= 0 && s2 < num_blocks && d2 >= 0 && d2 < num_blocks && s2 != d2;
            if (valid2 && j != i && (d2 == dst || s2 == dst))
                return -2;
        }
    }
    long block_elems = (long)num_kv_heads * head_dim * block_size;
    long copied = 0;
    for (long i = 0; i < num_pairs; ++i) {
        int64_t src = pairs[2 * i], dst = pairs[2 * i + 1];
        if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks || src == dst)
            continue;
        for (long e = 0; e < block_elems; ++e) {
            k_cache[dst * block_elems + e] = k_cache[src * block_elems + e];
            v_cache[dst * block_elems + e] = v_cache[src * block_elems + e];
        }
        ++copied;
    }
    return copied;
}

/*
 * o[d] = softmax over t < count of scale * qv . K_t, applied to V_t, for K/V
 * head g of sequence s, with K_t and V_t read from the pools through the
 * sequence's table row.  count = 0 gives a zero row.  Returns 0, or 1 if host
 * memory ran out.
 */
static int attend(double *o, const double *qv, const uint16_t *k_cache, const uint16_t *v_cache,
                  const int32_t *table_row, int g, int count, int num_kv_heads, int head_dim,
                  int block_size, double scale)
{
    for (int d = 0; d < head_dim; ++d)
        o[d] = 0.0;
    if (count == 0)
        return 0;
    double *score = malloc(sizeof(double) * (size_t)count);
    if (!score)
        return 1;

    /* S = scale * q K^T over the positions, gathered through the table. */
    for (int t = 0; t < count; ++t) {
        long blk = table_row[t / block_size];
        long off = t % block_size;
        double dot = 0.0;
        for (int d = 0; d < head_dim; ++d)
            dot += qv[d] * bf16_value(k_cache[k_index(blk, g, off, d, num_kv_heads, head_dim,
                                                      block_size)]);
        score[t] = scale * dot;
    }

    /* P = softmax(S): subtract the maximum, exponentiate, normalise. */
    double m = score[0];
    for (int t = 1; t < count; ++t)
        if (score[t] > m)
            m = score[t];
    double l = 0.0;
    for (int t = 0; t < count; ++t) {
        score[t] = exp(score[t] - m);
        l += score[t];
    }

    /* O = P V. */
    for (int t = 0; t < count; ++t) {
        long blk = table_row[t / block_size];
        long off = t % block_size;
        const uint16_t *vtile = v_cache + (blk * num_kv_heads + g) * (long)head_dim * block_size;
        double p = score[t] / l;
        for (int d = 0; d < head_dim; ++d)
            o[d] += p * bf16_value(vtile[(long)d * block_size + off]);
    }
    free(score);
    return 0;
}

/* Every table entry a context of n tokens uses lies in the pool. */
static int table_ok(const int32_t *table_row, int n, int block_size, long num_blocks)
{
    for (int b = 0; b < (n + block_size - 1) / block_size; ++b)
        if (table_row[b] < 0 || table_row[b] >= num_blocks)
            return 0;
    return 1;
}

/*
 * out[s][h][d] (double, [S][Hq][D]) = softmax over t < n of
 * scale * q[s][h] . K_t, applied to V_t, with K_t, V_t read from the pools
 * through block_tables (int32 [S][max_blocks]) and n = context_lens[s].
 * n = 0 gives a zero row.  Returns 0, or -1 on a bad argument (including a
 * context longer than the table or a table entry outside the pool).
 */
int oracle_paged_attention(double *out, const uint16_t *q,
                           const uint16_t *k_cache, const uint16_t *v_cache,
                           const int32_t *block_tables, const int32_t *context_lens,
                           int num_seqs, int num_q_heads, int num_kv_heads,
                           int head_dim, int block_size, int max_blocks,
                           long num_blocks, double scale, int num_threads)
{
    if (num_seqs < 0 || num_kv_heads < 1 || num_q_heads % num_kv_heads != 0 ||
        head_dim < 1 || head_dim % KCHUNK != 0 || block_size < 1 || max_blocks < 1 ||
        num_blocks < 1)
        return -1;
    for (int s = 0; s < num_seqs; ++s) {
        int n = context_lens[s];
        if (n < 0 || n > max_blocks * block_size ||
            !table_ok(block_tables + (long)s * max_blocks, n, block_size, num_blocks))
            return -1;
    }
    const int group = num_q_heads / num_kv_heads;
    const long pairs = (long)num_seqs * num_q_heads;
    int bad = 0;

#ifdef _OPENMP
    if (num_threads < 1)
        num_threads = 1;
#pragma omp parallel for schedule(dynamic, 1) num_threads(num_threads) reduction(| : bad)
#endif
    for (long pair = 0; pair < pairs; ++pair) {
        const int s = (int)(pair / num_q_heads);
        const int h = (int)(pair % num_q_heads);
        const int g = h / group;                      /* the K/V head this query head reads */
        double *qv = malloc(sizeof(double) * (size_t)head_dim);
        if (!qv) {
            bad = 1;
            continue;
        }
        for (int d = 0; d < head_dim; ++d)
            qv[d] = bf16_value(q[pair * head_dim + d]);
        bad |= attend(out + pair * head_dim, qv, k_cache, v_cache,
                      block_tables + (long)s * max_blocks, g, context_lens[s], num_kv_heads,
                      head_dim, block_size, scale);
        free(qv);
    }
    return bad ? -1 : 0;
}

/*
 * Prefill and chunked prefill ("tiny-vLLM으로 처음부터 고성능 LLM 추론 엔진
 * 구축하기" page, section "고급 추론 개념": prefill runs the whole prompt,
 * decode only the newest token; "tiny-vllm 씹뜯맛즐 - (1)" page, section 1:
 * each position attends to itself and the positions before it).
 *
 * Sequence s owns query rows query_start[s] .. query_start[s+1]-1 (m rows of
 * q, [rows][Hq][D]).  Its context holds n = context_lens[s] positions, the
 * chunk's own tokens being the last m of them (already in the pools).  Row
 * query_start[s] + i sits at position p = n - m + i and attends to positions
 * 0..p:
 *     out[row][h][:] = softmax over t <= p of scale * q[row][h] . K_t, applied to V_t.
 * A row with p < 0 (a chunk longer than the context) is zero.  A full prefill
 * is m = n; a decode step is m = 1.
 * Returns 0, or -1 on a bad argument (query_start decreasing or negative, a
 * context longer than the table, a table entry outside the pool).
 */
int oracle_paged_prefill(double *out, const uint16_t *q, const int32_t *query_start,
                         const uint16_t *k_cache, const uint16_t *v_cache,
                         const int32_t *block_tables, const int32_t *context_lens,
                         int num_seqs, int num_q_heads, int num_kv_heads,
                         int head_dim, int block_size, int max_blocks,
                         long num_blocks, double scale, int num_threads)
{
    if (num_seqs < 0 || num_kv_heads < 1 || num_q_heads % num_kv_heads != 0 ||
        head_dim < 1 || head_dim % KCHUNK != 0 || block_size < 1 || max_blocks < 1 ||
        num_blocks < 1 || query_start[0] < 0)
        return -1;
    for (int s = 0; s < num_seqs; ++s) {
        int n = context_lens[s];
        if (query_start[s + 1] < query_start[s] || n < 0 || n > max_blocks * block_size ||
            !table_ok(block_tables + (long)s * max_blocks, n, block_size, num_blocks))
            return -1;
    }
    const long rows = query_start[num_seqs];
    int *seq_of_row = malloc(sizeof(int) * (size_t)(rows > 0 ? rows : 1));
    if (!seq_of_row)
        return -1;
    for (int s = 0; s < num_seqs; ++s)
        for (long r = query_start[s]; r < query_start[s + 1]; ++r)
            seq_of_row[r] = s;
    const int group = num_q_heads / num_kv_heads;
    int bad = 0;

#ifdef _OPENMP
    if (num_threads < 1)
        num_threads = 1;
#pragma omp parallel for schedule(dynamic, 16) num_threads(num_threads) reduction(| : bad)
#endif
    for (long pair = (long)query_start[0] * num_q_heads; pair < rows * num_q_heads; ++pair) {
        const long row = pair / num_q_heads;
        const int h = (int)(pair % num_q_heads);
        const int s = seq_of_row[row];
        const int m = query_start[s + 1] - query_start[s];
        const int p = context_lens[s] - m + (int)(row - query_start[s]);
        double *qv = malloc(sizeof(double) * (size_t)head_dim);
        if (!qv) {
            bad = 1;
            continue;
        }
        for (int d = 0; d < head_dim; ++d)
            qv[d] = bf16_value(q[pair * head_dim + d]);
        bad |= attend(out + pair * head_dim, qv, k_cache, v_cache,
                      block_tables + (long)s * max_blocks, h / group, p >= 0 ? p + 1 : 0,
                      num_kv_heads, head_dim, block_size, scale);
        free(qv);
    }
    free(seq_of_row);
    return bad ? -1 : 0;
}

/*
 * Nearest bf16 to v, ties to even, taken directly from the double (no
 * intermediate float rounding): v = m * 2^e with 0.5 <= |m| < 1, so the 8
 * significant bits of bf16 are rint(m * 2^8).  Finite, normal-range inputs
 * only (the rotated values of bf16 data); 0 maps to +0 or -0.
 */
static uint16_t bf16_round(double v)
{
    if (v == 0.0)
        return signbit(v) ? 0x8000u : 0u;
    int e;
    double m = frexp(v, &e);
    double r = rint(m * 256.0);                      /* default rounding mode: ties to even */
    float f = (float)ldexp(r, e - 8);                /* 8 significant bits: exact in float */
    uint32_t bits;
    memcpy(&bits, &f, sizeof bits);
    return (uint16_t)(bits >> 16);
}

/* out[i] = bf16_round(v[i]) for i < n (exported so the rounding can be pinned). */
void oracle_bf16_round(const double *v, long n, uint16_t *out)
{
    for (long i = 0; i < n; ++i)
        out[i] = bf16_round(v[i]);
}

/*
 * Rotary position embedding ("tiny-vllm 씹뜯맛즐 - (1)" page, section "5. 절대
 * 위치 임베딩 대신 RoPE": q and k at position p are multiplied by a rotation
 * R_p, so that (R_i q)^T (R_j k) = q^T R_{j-i} k; "tiny-vLLM으로 처음부터 고성능
 * LLM 추론 엔진 구축하기" page: complex-number math with sine and cosine).
 *
 * R_p turns each pair of dimensions (a, b) = pair k by the angle
 * p * inv_freq[k]:  a' = a cos - b sin,  b' = a sin + b cos.
 *   style 0: pair k is dims (2k, 2k+1), the complex number a + i b times e^{i angle};
 *   style 1: pair k is dims (k, k + D/2).
 * x: [T][H][D] bf16 bits; positions: int32 [T]; inv_freq: float [D/2].
 * out_f64 ([T][H][D], may be NULL) gets the rotated values in double
 * precision, out_bits (may be NULL) the same rounded to bf16 (ties to even).
 * Returns 0, or -1 on a bad argument.
 */
int oracle_rope(const uint16_t *x, const int32_t *positions, const float *inv_freq,
                long num_tokens, int num_heads, int head_dim, int style, double *out_f64,
                uint16_t *out_bits)
{
    if (num_tokens < 0 || num_heads < 1 || head_dim < 2 || head_dim % 2 != 0 ||
        (style != 0 && style != 1))
        return -1;
    const int half = head_dim / 2;
    for (long t = 0; t < num_tokens; ++t) {
        for (int k = 0; k < half; ++k) {
            const double angle = (double)positions[t] * (double)inv_freq[k];
            const double c = cos(angle), sn = sin(angle);
            const int ia = style == 0 ? 2 * k : k;
            const int ib = style == 0 ? 2 * k + 1 : k + half;
            for (int h = 0; h < num_heads; ++h) {
                const long row = (t * num_heads + h) * (long)head_dim;
                const double a = bf16_value(x[row + ia]);
                const double b = bf16_value(x[row + ib]);
                const double ra = a * c - b * sn;
                const double rb = a * sn + b * c;
                if (out_f64) {
                    out_f64[row + ia] = ra;
                    out_f64[row + ib] = rb;
                }
                if (out_bits) {
                    out_bits[row + ia] = bf16_round(ra);
                    out_bits[row + ib] = bf16_round(rb);
                }
            }
        }
    }
    return 0;
}

/* Number of OpenMP threads the library would use by default (1 without OpenMP). */
int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
