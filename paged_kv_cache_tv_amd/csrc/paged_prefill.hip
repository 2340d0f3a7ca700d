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
//   * Keys go in chunks of 64 (4 blocks).  All 512 threads load a chunk's K
//     and V tiles (16 KiB) into registers one chunk ahead and store them to
//     LDS, double-buffered, with one barrier per chunk.  Each wavefront then
//     reads MFMA operands from LDS: K tiles verbatim (every 1 KiB operand
//     read contiguous), V rearranged so that one 16-byte read is a whole PV
//     operand and 16 consecutive dims fall on distinct banks.
//   * Each wavefront owns 32 rows (2 tiles of 16 MFMA columns); the register
//     budget is cut to 128 so that four wavefronts share each SIMD, which
//     hides the latency of the LDS reads, the cross-lane maximum and the
//     MFMA results.  Scores
//     S^T[16 keys][16 rows] = K . Q^T take two v_mfma_f32_16x16x32_bf16 per
//     tile (dims 0-31, 32-63).  Lane (q = lane/16, c = lane%16) then holds
//     keys 4q..4q+3 of every 16-key tile for row c, and two such tiles form
//     the lane's 8 k-slots of the B operand of O^T += V^T . P^T
//     (v_mfma_f32_16x16x32_bf16 over 32 keys), with V^T read from LDS in the
//     same key order.  P is rounded to bf16 for that product; the running
//     sum uses the fp32 values.
//   * exp is 2^x (v_exp_f32) with scale * log2(e) folded into one multiply-add
//     per score.  Masked scores (future positions, keys past the context,
//     blocks outside the pool) become -inf, and V of keys past the context or
//     in dropped blocks is zeroed in LDS, because stale slots may hold NaN.
#include "tv_internal.h"

#include <math.h>

namespace tv {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

constexpr int D = kHeadDim;
constexpr int BS = kBlockSize;
constexpr int kWaves = 8;                        // wavefronts per workgroup
constexpr int kRowTiles = 2;                     // 16-column MFMA tiles per wavefront
constexpr int kThreads = 64 * kWaves;
constexpr int kWavesPerSimd = 4;                 // occupancy the register budget is cut for
constexpr int kChunkBlocks = 4;                  // blocks per key chunk
constexpr int kChunkKeys = kChunkBlocks * BS;    // 64
constexpr int kTileBytes = BS * D * 2;           // one (block, K/V head) tile: 2 KiB
constexpr int kBufBytes = 2 * kChunkBlocks * kTileBytes;   // K then V of one chunk: 16 KiB

__device__ __forceinline__ unsigned zero_from(unsigned w, int lim, int e)
{
    // Clear the 16-bit halves of word w holding elements e, e+1 that are >= lim.
    const unsigned lo = e >= lim ? 0u : (w & 0xFFFFu);
    const unsigned hi = e + 1 >= lim ? 0u : (w & 0xFFFF0000u);
    return lo | hi;
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
    const int wave = tid >> 6;
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

    // Chunk loading: a chunk is 4 blocks x (K tile, V tile) x 128 pieces of
    // 16 bytes.  Piece p = tid + kThreads * u (u < kLoads) is byte 16 (p & 127)
    // of the K (bit 7 of p clear) or V tile of block p / 256.
    constexpr int kLoads = kChunkBlocks * 256 / kThreads;
    static_assert(kLoads * kThreads == kChunkBlocks * 256, "pieces per thread");
    const bool is_v = (tid >> 7) & 1;
    const int piece = tid & 127;
    const char *pool = reinterpret_cast<const char *>(is_v ? a.v_cache : a.k_cache);
    const int32_t *table = a.block_tables + (int64_t)s * a.max_blocks;
    // V piece = dimension piece / 2, tokens 8 (piece & 1) .. + 8 of its block.
    const int v_tok0 = 8 * (piece & 1);

    u32x4 pre[kLoads];
    unsigned valid_next = 0;
    auto load_chunk = [&](int c) {
        valid_next = 0;
#pragma unroll
        for (int j = 0; j < kChunkBlocks; ++j) {
            const int b = c * kChunkBlocks + j;
            const int32_t phys = b * BS < n ? table[b] : -1;
            valid_next |= (phys >= 0 && (int64_t)phys < a.num_blocks ? 1u : 0u) << j;
        }
#pragma unroll
        for (int u = 0; u < kLoads; ++u) {
            const int j = (tid + kThreads * u) >> 8;
            const int b = c * kChunkBlocks + j;
            const u32x4 zero = {0u, 0u, 0u, 0u};
            pre[u] = zero;
            if ((valid_next >> j) & 1u)
                pre[u] = *reinterpret_cast<const u32x4 *>(
                    pool + ((int64_t)table[b] * a.num_kv_heads + kvh) * kTileBytes + 16 * piece);
        }
    };
    auto store_chunk = [&](int c, char *buf) {
#pragma unroll
        for (int u = 0; u < kLoads; ++u) {
            const int j = (tid + kThreads * u) >> 8;
            u32x4 x = pre[u];
            if (is_v) {
                // Keys at or past the context end: V = 0 (the slot may hold NaN).
                const int lim = n - ((c * kChunkBlocks + j) * BS + v_tok0);
                if (lim < 8) {
#pragma unroll
                    for (int w = 0; w < 4; ++w)
                        x[w] = zero_from(x[w], lim, 2 * w);
                }
            }
            if (is_v) {
                // V of a chunk in LDS: [block pair kp][dim d][slot][block of the
                // pair], 8 bytes (4 tokens) each, so that one 16-byte read gives
                // the PV operand of 4 tokens of both blocks.  Token group g of
                // dim d sits in slot g ^ f(d % 16), f(c) = (c ^ (c >> 2)) & 3,
                // which keeps the operand reads of 16 consecutive dims on
                // distinct banks.
                const int d = piece >> 1, g0 = 2 * (piece & 1);
                const int f = (d ^ (d >> 2)) & 3;
                char *row = buf + kChunkBlocks * kTileBytes + (j >> 1) * 4096 + d * 64 + 8 * (j & 1);
                const u32x2 lo = {x[0], x[1]}, hi = {x[2], x[3]};
                *reinterpret_cast<u32x2 *>(row + 16 * (g0 ^ f)) = lo;
                *reinterpret_cast<u32x2 *>(row + 16 * ((g0 + 1) ^ f)) = hi;
            } else {
                *reinterpret_cast<u32x4 *>(buf + j * kTileBytes + 16 * piece) = x;
            }
        }
    };

    f32x4 o[kRowTiles][4];
    float m_run[kRowTiles], l_run[kRowTiles];
#pragma unroll
    for (int rt = 0; rt < kRowTiles; ++rt) {
        m_run[rt] = -INFINITY;
        l_run[rt] = 0.f;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
            o[rt][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    const float cs = a.scale_log2;

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

        // Scores.
        f32x4 sc[kRowTiles][4];
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
            const char *kb = buf + kt * kTileBytes + 16 * lane;
            const bf16x8 k0 = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(kb));
            const bf16x8 k1 = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(kb + 1024));
#pragma unroll
            for (int rt = 0; rt < kRowTiles; ++rt) {
                f32x4 z = {0.f, 0.f, 0.f, 0.f};
                z = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k0, qop[rt][0], z, 0, 0, 0);
                sc[rt][kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k1, qop[rt][1], z, 0, 0, 0);
            }
        }

        // Mask keys after a row's position and keys of dropped blocks.
        const int key0 = c * kChunkKeys + 4 * lq;           // this lane's key of slot (kt 0, j 0)
        if (c * kChunkKeys + kChunkKeys - 1 > wave_first_pos || valid != 0xFu) {
#pragma unroll
            for (int rt = 0; rt < kRowTiles; ++rt) {
                const int thr = pos[rt] - key0;
#pragma unroll
                for (int kt = 0; kt < 4; ++kt)
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        if (16 * kt + j > thr || !((valid >> kt) & 1u))
                            sc[rt][kt][j] = -INFINITY;
            }
        }

        // Online softmax per row tile, then P (bf16) into the PV product.
        bf16x8 pb[kRowTiles][2];
#pragma unroll
        for (int rt = 0; rt < kRowTiles; ++rt) {
            float mx = sc[rt][0][0];
#pragma unroll
            for (int kt = 0; kt < 4; ++kt)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    mx = fmaxf(mx, sc[rt][kt][j]);
            mx = fmaxf(mx, __shfl_xor(mx, 16));
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            const float m_new = fmaxf(m_run[rt], mx * cs);
            const float m_use = m_new == -INFINITY ? 0.f : m_new;   // rows with no key yet
            const float alpha = __builtin_amdgcn_exp2f(m_run[rt] - m_use);
            m_run[rt] = m_new;
            float lsum = 0.f;
#pragma unroll
            for (int kp = 0; kp < 2; ++kp) {
#pragma unroll
                for (int h = 0; h < 2; ++h)
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const float p = __builtin_amdgcn_exp2f(fmaf(sc[rt][2 * kp + h][j], cs, -m_use));
                        lsum += p;
                        pb[rt][kp][4 * h + j] = (__bf16)p;
                    }
            }
            l_run[rt] = fmaf(l_run[rt], alpha, lsum);
#pragma unroll
            for (int dt = 0; dt < 4; ++dt)
                o[rt][dt] *= alpha;
        }

        // O^T[dims][rows] += V^T . P^T: V^T lane (dim 16 dt + col, keys of k-slots
        // 8 lq .. 8 lq + 7) = V[2 kp][dim][4 lq .. 4 lq + 3], V[2 kp + 1][dim][4 lq ..].
        const char *vb = buf + kChunkBlocks * kTileBytes + col * 64 +
                         16 * (lq ^ ((col ^ (col >> 2)) & 3));
#pragma unroll
        for (int kp = 0; kp < 2; ++kp)
#pragma unroll
            for (int dt = 0; dt < 4; ++dt) {
                const bf16x8 vop = __builtin_bit_cast(
                    bf16x8, *reinterpret_cast<const u32x4 *>(vb + kp * 4096 + dt * 16 * 64));
#pragma unroll
                for (int rt = 0; rt < kRowTiles; ++rt)
                    o[rt][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, pb[rt][kp], o[rt][dt],
                                                                        0, 0, 0);
            }
    }

    // Normalise and store: lane holds dims 16 dt + 4 lq .. + 3 of its row.
#pragma unroll
    for (int rt = 0; rt < kRowTiles; ++rt) {
        float l = l_run[rt];
        l += __shfl_xor(l, 16);
        l += __shfl_xor(l, 32);
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
