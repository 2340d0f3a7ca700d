// Paged GQA prefill / chunked-prefill attention for gfx950.
//
// What is computed ("tiny-vLLM으로 처음부터 고성능 LLM 추론 엔진 구축하기"
// page, section "고급 추론 개념": prefill runs every token of the prompt;
// "tiny-vllm 씹뜯맛즐 - (1)" page, section 1: each position attends to itself
// and the positions before it; "vLLM" page, sections "가상 메모리 방식의
// 해결" and "Flash Attention": K/V gathered block by block through the block
// table, softmax accumulated online with a running maximum and sum): sequence
// s brings a chunk of m query rows, the last m positions of its n-token
// context, and row i (position n - m + i) attends to positions 0 .. n - m + i.
//
// Mapping to CDNA4:
//   * One 512-thread workgroup (8 wavefronts) per (sequence, K/V head, tile of
//     256 / G chunk rows), G = query heads per K/V head.  The G query heads of
//     a token are stacked as MFMA columns, so each K/V element loaded feeds
//     every head of the group.  Launch index: K/V head fastest (one XCD per
//     head, so the tiles of one (sequence, head) share an L2), and the last,
//     heaviest tiles of every sequence first.
//   * Keys go in chunks of 128 (8 blocks).  All 512 threads load a chunk's K
//     and V tiles (32 KiB) into registers one chunk ahead and store them to
//     LDS, double-buffered, with one barrier per chunk; each wavefront then
//     works through the chunk in 32-key halves and stops at the first half
//     past its last row.  K tiles are stored
//     verbatim (every 1 KiB operand read contiguous).  V is stored in PV
//     operand order: one 16-byte slot per (dimension, token group) holding 4
//     tokens of the dimension from each of two blocks, the slots of one
//     operand read in lane order.  Each thread loads its slot's two 8-byte
//     halves from the two blocks and stores the slot with one 16-byte write,
//     so every LDS store and every operand read covers 1 KiB contiguous, which
//     gfx950 serves without bank conflicts.
//   * Each wavefront owns 32 rows (2 tiles of 16 MFMA columns); the register
//     budget is cut to 128 so that four wavefronts share each SIMD, which
//     hides the latency of the LDS reads and the MFMA results.  Scores
//     S^T[16 keys][16 rows] = K . Q^T take two v_mfma_f32_16x16x32_bf16 per
//     tile (dims 0-31, 32-63).  Lane (q = lane/16, c = lane%16) then holds
//     keys 4q..4q+3 of every 16-key tile for row c, and two such tiles form
//     the lane's 8 k-slots of the B operand of O^T += V^T . P^T
//     (v_mfma_f32_16x16x32_bf16 over 32 keys), with V^T read from LDS in the
//     same key order.
//   * Softmax in base-2 units (v_exp_f32), scale * log2(e) folded into one
//     multiply-add per score.  The weights are rounded to bf16 for the PV
//     product, and the running sum adds those same rounded weights
//     (v_dot2c_f32_bf16 against (1, 1)), so each row's output is exactly a
//     weighted mean of V rows.  The row maximum uses v_maximum3_f32 and the
//     gfx950 lane-swap instructions across the 4 lane groups (no LDS).
//   * The running maximum is a reference value that only moves when needed.
//     The weights of each 32 keys are first taken against the reference as
//     it stands; only if a row has no reference yet, or a lane's 8 weights
//     sum to more than 2^8 (kLaneSumLimit; an overflow to inf also fails the
//     test), is the row maximum of those keys computed, the reference
//     moved up to it, the row's output and sum rescaled, and the weights taken
//     again.  Weights therefore never exceed 2^8, well inside bf16 and fp32
//     range, and the result is the same softmax (the reference cancels in the
//     final division).  With well-scaled scores the reference is set by a
//     row's first keys, and later keys skip both the row maximum and the
//     rescale of 16 accumulators per row tile.
//   * Masked scores (future positions, keys past the context, blocks outside
//     the pool) become -inf, and V of keys past the context or in dropped
//     blocks is zeroed in LDS, because stale slots may hold NaN.
#include "tv_internal.h"

#include <math.h>

namespace tv {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

constexpr int D = kHeadDim;
constexpr int BS = kBlockSize;
constexpr int kWaves = 8;                        // wavefronts per workgroup
constexpr int kRowTiles = 2;                     // 16-column MFMA tiles per wavefront
constexpr int kThreads = 64 * kWaves;
constexpr int kWavesPerSimd = 4;                 // occupancy the register budget is cut for
constexpr int kChunkBlocks = 8;                  // blocks per key chunk
constexpr int kChunkKeys = kChunkBlocks * BS;    // 128
constexpr int kPairs = kChunkBlocks / 2;         // 32-key halves of a chunk, one block pair each
constexpr int kLoads = kChunkBlocks * 128 / kThreads;   // 16-byte K pieces (and V slots) per thread
constexpr int kTileBytes = BS * D * 2;           // one (block, K/V head) tile: 2 KiB
constexpr int kBufBytes = 2 * kChunkBlocks * kTileBytes;   // K then V of one chunk: 16 KiB
constexpr float kLaneSumLimit = 256.0f;          // a lane's weights of 32 keys may sum to this
static_assert(kLoads * kThreads == kChunkBlocks * 128, "whole 16-byte K pieces per thread");
static_assert(kLoads * kThreads == kPairs * D * 4, "whole 16-byte V slots per thread");
static_assert(kThreads % 256 == 0, "a V slot's block pair is the same for a whole wavefront");
constexpr int kKStep = kThreads / 128;           // blocks whose K pieces one load round covers
constexpr int kVStep = kThreads / 256;           // block pairs whose V slots one round covers

__device__ __forceinline__ unsigned zero_from(unsigned w, int lim, int e)
{
    // Clear the 16-bit halves of word w holding elements e, e+1 that are >= lim.
    const unsigned lo = e >= lim ? 0u : (w & 0xFFFFu);
    const unsigned hi = e + 1 >= lim ? 0u : (w & 0xFFFF0000u);
    return lo | hi;
}

__device__ __forceinline__ float max2(float a, float b) { return __builtin_elementwise_maximum(a, b); }

// The pair (x[l], x[l ^ 32]) (swap32) or (x[l], x[l ^ 16]) (swap16), in some
// order, from v_permlane32_swap / v_permlane16_swap.  The results are copied
// out of the returned vector before the bit casts: a bit cast of a vector
// element reads the vector's first element here.
__device__ __forceinline__ void swap32(float x, float &a, float &b)
{
    const unsigned u = __builtin_bit_cast(unsigned, x);
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    const unsigned r0 = r[0], r1 = r[1];
    a = __builtin_bit_cast(float, r0);
    b = __builtin_bit_cast(float, r1);
}
__device__ __forceinline__ void swap16(float x, float &a, float &b)
{
    const unsigned u = __builtin_bit_cast(unsigned, x);
    const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    const unsigned r0 = r[0], r1 = r[1];
    a = __builtin_bit_cast(float, r0);
    b = __builtin_bit_cast(float, r1);
}

// Maximum and sum over the lanes l, l^16, l^32, l^48 (the 4 lane groups
// holding one row's keys), without LDS.
__device__ __forceinline__ float group_max(float x)
{
    float a, b;
    swap32(x, a, b);
    swap16(max2(a, b), a, b);
    return max2(a, b);
}

__device__ __forceinline__ float group_sum(float x)
{
    float a, b;
    swap32(x, a, b);
    swap16(a + b, a, b);
    return a + b;
}

template <int G>
__global__ __launch_bounds__(kThreads, kWavesPerSimd) void paged_prefill_kernel(PrefillArgs a)
{
    constexpr int kTokPerWave = 16 * kRowTiles / G;
    constexpr int kTokPerWg = kWaves * kTokPerWave;
    __shared__ __attribute__((aligned(16))) char lds[2 * kBufBytes];

    const int kvh = (int)(blockIdx.x % (unsigned)a.num_kv_heads);
    const int rest = (int)(blockIdx.x / (unsigned)a.num_kv_heads);
    const int s = rest % a.num_seqs;
    const int tile_from_end = rest / a.num_seqs;

    const int q0 = a.query_start[s];
    const int m = a.query_start[s + 1] - q0;                  // chunk rows (device data)
    const int mq = min(max(m, 0), a.max_query_len);           // rows this launch covers
    const int tiles = (mq + kTokPerWg - 1) / kTokPerWg;
    const int t = tiles - 1 - tile_from_end;
    if (t < 0)
        return;
    int n = a.context_lens[s];
    n = n < 0 ? 0 : (n > a.max_context_len ? a.max_context_len : n);

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: scalar row ranges
    const int lane = tid & 63;
    const int col = lane & 15;
    const int lq = lane >> 4;
    const int Hq = a.num_kv_heads * G;

    const int i0 = t * kTokPerWg;                             // first chunk row of the tile
    const int i1 = min(mq, i0 + kTokPerWg);
    const int base_pos = n - m;                               // position of chunk row 0
    const int wg_last_pos = base_pos + i1 - 1;
    const int nchunks = wg_last_pos >= 0 ? wg_last_pos / kChunkKeys + 1 : 0;

    // This wavefront's rows.
    const int iw0 = i0 + wave * kTokPerWave;
    const int iw1 = min(i1, iw0 + kTokPerWave);
    const int wave_first_pos = base_pos + iw0;
    const int wave_last_pos = iw1 > iw0 ? base_pos + iw1 - 1 : -1;   // -1: no rows

    // Queries: column col of row tile rt is wave row r = 16 rt + col, i.e.
    // chunk row iw0 + r / G and query head kvh * G + r % G.
    bf16x8 qop[kRowTiles][2];
    int pos[kRowTiles];
    bool row_ok[kRowTiles];
#pragma unroll
    for (int rt = 0; rt < kRowTiles; ++rt) {
        const int r = 16 * rt + col;
        const int i = iw0 + r / G;
        row_ok[rt] = i < iw1;
        pos[rt] = base_pos + i;
        const u32x4 zero = {0u, 0u, 0u, 0u};
        u32x4 x0 = zero, x1 = zero;
        if (row_ok[rt]) {
            const u32x4 *qp = reinterpret_cast<const u32x4 *>(
                a.q + ((int64_t)(q0 + i) * Hq + kvh * G + r % G) * D + 8 * lq);
            x0 = qp[0];
            x1 = qp[4];                                       // dims 32 + 8 lq ..
        }
        qop[rt][0] = __builtin_bit_cast(bf16x8, x0);
        qop[rt][1] = __builtin_bit_cast(bf16x8, x1);
    }

    // Chunk loading.  K: thread tid moves the 16-byte pieces tid & 127 of the
    // tiles of blocks kb + kKStep u (kb = tid >> 7, u < kLoads).  V: thread
    // tid takes slot tid & 255 = (dt, g, c) of block pairs vp + kVStep u
    // (vp = tid >> 8):
    // tokens 4g .. 4g + 3 of dimension d = 16 dt + c from each block of the
    // pair (8 bytes each), stored as one 16-byte slot.  That is exactly the
    // operand lane (c + 16 g) of the PV product for dimension tile dt reads,
    // so both the stores and the operand reads cover 1 KiB contiguous per
    // instruction (conflict-free on gfx950; strided 16-byte reads are not).
    // kb and vp are the same for the whole wavefront, so the table entries,
    // validity and tile addresses are scalar values.
    const int kb = __builtin_amdgcn_readfirstlane(tid >> 7);
    const int vp = __builtin_amdgcn_readfirstlane(tid >> 8);
    const int vg = (tid >> 4) & 3;
    const int vd = ((tid >> 6) & 3) * 16 + (tid & 15);
    const uint32_t k_off = 16u * (uint32_t)(tid & 127);                 // bytes in a K tile
    const uint32_t v_off = (uint32_t)(vd * (2 * BS) + 8 * vg);          // bytes in a V tile
    const int k_st = kb * kTileBytes + 16 * (tid & 127);
    const int v_st = kChunkBlocks * kTileBytes + vp * 4096 + 16 * (tid & 255);
    const int32_t *table = a.block_tables + (int64_t)s * a.max_blocks;
    // Entries outside [0, num_blocks) drop their block: one unsigned compare
    // against the pool size (capped where it exceeds every int32 entry).
    const uint32_t nb_cap = a.num_blocks > 0x7fffffff ? 0x80000000u : (uint32_t)a.num_blocks;
    const char *kheads = reinterpret_cast<const char *>(a.k_cache) + (int64_t)kvh * kTileBytes;
    const char *vheads = reinterpret_cast<const char *>(a.v_cache) + (int64_t)kvh * kTileBytes;
    const int64_t block_stride = (int64_t)a.num_kv_heads * kTileBytes;

    u32x4 kpre[kLoads];
    u32x2 vpre0[kLoads], vpre1[kLoads];
    unsigned valid_next = 0;
    auto entry = [&](int b) -> int32_t { return b * BS < n ? table[b] : -1; };
    auto load_chunk = [&](int c) {
        const int b0 = c * kChunkBlocks;
        valid_next = 0;
#pragma unroll
        for (int j = 0; j < kChunkBlocks; ++j)
            valid_next |= ((uint32_t)entry(b0 + j) < nb_cap ? 1u : 0u) << j;
        const u32x4 z4 = {0u, 0u, 0u, 0u};
        const u32x2 z2 = {0u, 0u};
#pragma unroll
        for (int u = 0; u < kLoads; ++u) {
            const int32_t pk = entry(b0 + kb + kKStep * u);
            const int32_t pa = entry(b0 + 2 * (vp + kVStep * u));
            const int32_t pb = entry(b0 + 2 * (vp + kVStep * u) + 1);
            kpre[u] = (uint32_t)pk < nb_cap
                          ? *reinterpret_cast<const u32x4 *>(kheads + pk * block_stride + k_off)
                          : z4;
            vpre0[u] = (uint32_t)pa < nb_cap
                           ? *reinterpret_cast<const u32x2 *>(vheads + pa * block_stride + v_off)
                           : z2;
            vpre1[u] = (uint32_t)pb < nb_cap
                           ? *reinterpret_cast<const u32x2 *>(vheads + pb * block_stride + v_off)
                           : z2;
        }
    };
    auto store_chunk = [&](int c, char *buf) {
#pragma unroll
        for (int u = 0; u < kLoads; ++u) {
            *reinterpret_cast<u32x4 *>(buf + k_st + kKStep * u * kTileBytes) = kpre[u];
            u32x2 x0 = vpre0[u], x1 = vpre1[u];
            if (c * kChunkKeys + kChunkKeys > n) {
                // The chunk holding the context end: V of keys at or past it
                // is 0 (the slot may hold NaN).
                const int lim0 = n - ((c * kChunkBlocks + 2 * (vp + kVStep * u)) * BS + 4 * vg);
                const int lim1 = lim0 - BS;
                x0[0] = zero_from(x0[0], lim0, 0);
                x0[1] = zero_from(x0[1], lim0, 2);
                x1[0] = zero_from(x1[0], lim1, 0);
                x1[1] = zero_from(x1[1], lim1, 2);
            }
            const u32x4 slot = {x0[0], x0[1], x1[0], x1[1]};
            *reinterpret_cast<u32x4 *>(buf + v_st + kVStep * u * 4096) = slot;
        }
    };

    f32x4 o[kRowTiles][4];
    float m_ref[kRowTiles], m_use[kRowTiles], l_run[kRowTiles];   // base-2 units
#pragma unroll
    for (int rt = 0; rt < kRowTiles; ++rt) {
        m_ref[rt] = -INFINITY;                               // reference maximum (base-2 units)
        m_use[rt] = 0.f;                                     // the same, 0 while no key is seen
        l_run[rt] = 0.f;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
            o[rt][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    const float cs = a.scale_log2;
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};

    if (nchunks > 0)
        load_chunk(0);
    for (int c = 0; c < nchunks; ++c) {
        char *buf = lds + (c & 1) * kBufBytes;
        const unsigned valid = valid_next;
        store_chunk(c, buf);
        __syncthreads();
        if (c + 1 < nchunks)
            load_chunk(c + 1);
        if (c * kChunkKeys > wave_last_pos)
            continue;                                        // this wave's rows are done

        // The chunk in halves of 32 keys (block pair kp = blocks 2 kp and
        // 2 kp + 1): scores, softmax weights, then their PV product, so only
        // 32 keys of scores and weights are live at a time.
        const int key0 = c * kChunkKeys + 4 * lq;           // this lane's key of slot (kt 0, j 0)
        const char *vb = buf + kChunkBlocks * kTileBytes + 16 * lane;
#pragma unroll
        for (int kp = 0; kp < kPairs; ++kp) {
            if (c * kChunkKeys + 32 * kp > wave_last_pos)
                break;                                       // keys past this wave's rows
            const bool mask = c * kChunkKeys + 32 * kp + 31 > wave_first_pos ||
                              ((valid >> (2 * kp)) & 3u) != 3u;
            // Scores of key tiles 2 kp + h.
            f32x4 sc[kRowTiles][2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const char *kbuf = buf + (2 * kp + h) * kTileBytes + 16 * lane;
                const bf16x8 k0 = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(kbuf));
                const bf16x8 k1 = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(kbuf + 1024));
#pragma unroll
                for (int rt = 0; rt < kRowTiles; ++rt) {
                    f32x4 z = {0.f, 0.f, 0.f, 0.f};
                    z = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k0, qop[rt][0], z, 0, 0, 0);
                    sc[rt][h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k1, qop[rt][1], z, 0, 0, 0);
                }
            }

            // Mask keys after a row's position and keys of dropped blocks.
            if (mask) {
#pragma unroll
                for (int rt = 0; rt < kRowTiles; ++rt) {
                    const int thr = pos[rt] - key0;
#pragma unroll
                    for (int h = 0; h < 2; ++h)
#pragma unroll
                        for (int j = 0; j < 4; ++j)
                            if (16 * (2 * kp + h) + j > thr || !((valid >> (2 * kp + h)) & 1u))
                                sc[rt][h][j] = -INFINITY;
                }
            }

            // Softmax weights.  They are first taken against the row's
            // reference maximum as it stands.  Only when some row of the
            // wavefront has no reference yet, or some lane's 8 weights sum
            // to more than 2^8 (also true for an overflow to inf), is the
            // row maximum of these keys computed, the reference moved up to
            // it (rescaling the output and sum), and the weights taken again
            // -- then each is at most 1.
            u32x4 pw[kRowTiles];                              // bf16 pairs of P
#pragma unroll
            for (int rt = 0; rt < kRowTiles; ++rt) {
                auto weights = [&](float mu) {
                    float csum = 0.f;
#pragma unroll
                    for (int h = 0; h < 2; ++h)
#pragma unroll
                        for (int j = 0; j < 4; j += 2) {
                            const float p0 = __builtin_amdgcn_exp2f(fmaf(sc[rt][h][j], cs, -mu));
                            const float p1 = __builtin_amdgcn_exp2f(fmaf(sc[rt][h][j + 1], cs, -mu));
                            const bf16x2 pp = {(__bf16)p0, (__bf16)p1};
                            csum = __builtin_amdgcn_fdot2_f32_bf16(pp, ones, csum, false);
                            pw[rt][2 * h + j / 2] = __builtin_bit_cast(unsigned, pp);
                        }
                    return csum;
                };
                float csum = 0.f;
                bool fresh = __builtin_amdgcn_ballot_w64(m_ref[rt] == -INFINITY) != 0;
                if (!fresh) {
                    csum = weights(m_use[rt]);
                    fresh = __builtin_amdgcn_ballot_w64(!(csum <= kLaneSumLimit)) != 0;
                }
                if (fresh) {
                    float mx = max2(max2(sc[rt][0][0], sc[rt][0][1]), sc[rt][0][2]);
                    mx = max2(max2(mx, sc[rt][0][3]), sc[rt][1][0]);
                    mx = max2(max2(mx, sc[rt][1][1]), sc[rt][1][2]);
                    mx = max2(mx, sc[rt][1][3]);
                    const float mc = group_max(mx) * cs;    // the row maximum of these keys
                    const float m_new = max2(m_ref[rt], mc);
                    const float alpha = m_new > m_ref[rt] ? __builtin_amdgcn_exp2f(m_ref[rt] - m_new) : 1.f;
                    m_ref[rt] = m_new;
                    m_use[rt] = m_new == -INFINITY ? 0.f : m_new;
                    l_run[rt] *= alpha;
#pragma unroll
                    for (int dt = 0; dt < 4; ++dt)
                        o[rt][dt] *= alpha;
                    csum = weights(m_use[rt]);
                }
                l_run[rt] += csum;
            }

            // O^T[dims][rows] += V^T . P^T: V^T lane (dim 16 dt + col, keys of
            // k-slots 8 lq .. 8 lq + 7) = V[2 kp][dim][4 lq .. 4 lq + 3],
            // V[2 kp + 1][dim][4 lq ..], which is slot lane of the pair's
            // dimension tile dt.
#pragma unroll
            for (int dt = 0; dt < 4; ++dt) {
                const bf16x8 vop = __builtin_bit_cast(
                    bf16x8, *reinterpret_cast<const u32x4 *>(vb + kp * 4096 + dt * 1024));
#pragma unroll
                for (int rt = 0; rt < kRowTiles; ++rt)
                    o[rt][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        vop, __builtin_bit_cast(bf16x8, pw[rt]), o[rt][dt], 0, 0, 0);
            }
        }
    }

    // Normalise and store: lane holds dims 16 dt + 4 lq .. + 3 of its row.
#pragma unroll
    for (int rt = 0; rt < kRowTiles; ++rt) {
        const float l = group_sum(l_run[rt]);
        if (!row_ok[rt])
            continue;
        const float inv = l > 0.f ? 1.f / l : 0.f;
        const int r = 16 * rt + col;
        float *op = a.out + ((int64_t)(q0 + iw0 + r / G) * Hq + kvh * G + r % G) * D + 4 * lq;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
            *reinterpret_cast<f32x4 *>(op + 16 * dt) = o[rt][dt] * inv;
    }
}

template <int G>
hipError_t launch_g(const PrefillArgs &a, hipStream_t stream)
{
    constexpr int kTokPerWg = kWaves * 16 * kRowTiles / G;
    const int64_t tiles = (a.max_query_len + kTokPerWg - 1) / kTokPerWg;
    const int64_t grid = tiles * a.num_seqs * a.num_kv_heads;
    if (grid == 0)
        return hipSuccess;
    if (grid > 0x7FFFFFFF)
        return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(paged_prefill_kernel<G>, dim3((unsigned)grid), dim3(kThreads), 0, stream,
                       a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_paged_prefill(const PrefillArgs &a, hipStream_t stream)
{
    switch (a.group) {
    case 1: return launch_g<1>(a, stream);
    case 2: return launch_g<2>(a, stream);
    case 4: return launch_g<4>(a, stream);
    case 8: return launch_g<8>(a, stream);
    case 16: return launch_g<16>(a, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace tv
