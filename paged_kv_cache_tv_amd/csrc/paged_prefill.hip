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
//   * Small grids (fewer workgroups than two per compute unit: chunked
//     prefill of a few sequences) take two key shares: the workgroup's 8
//     wavefronts are 4 row wavefronts (128 / G chunk rows) times 2 shares,
//     share h taking the 32-key steps kp with kp % 2 == h of every chunk, so
//     a long context's chain of steps per wavefront halves and the grid
//     doubles.  At the end share 1 leaves its (reference, sum, output) in the
//     chunk buffers and share 0 folds it in by the running-maximum rule.
//   * Keys go in chunks of 128 (8 blocks), double-buffered in LDS with one
//     barrier per chunk.  Wavefront w copies block w of the next chunk
//     straight from memory into LDS (global_load_lds, 16 bytes per lane, no
//     registers): the K tile verbatim, the V tile with its 16-byte pieces
//     swizzled so that the PV operand reads hit every bank once.  The block
//     table entries of a chunk are loaded one chunk before its copy, so no
//     wait on them falls behind copies in flight; the barrier's wait is the
//     only one in the loop.
//   * Each wavefront owns 32 rows (one 32-column tile of
//     v_mfma_f32_32x32x16_bf16); the register budget is cut to 128 so that
//     four wavefronts share each SIMD.  Scores S^T[32 keys][32 rows] =
//     K . Q^T over 32 keys (one block pair) take four MFMAs (16 dims each).
//     The K rows are fed in a permuted order chosen so that result lane
//     (row c, half h) holds keys 8h .. 8h + 7 and 16 + 8h .. 16 + 8h + 7 of
//     the pair: exactly the k-slots the PV product O^T += V^T . P^T
//     (v_mfma_f32_32x32x16_bf16 over 16 keys) takes from lane (c, h), so the
//     weights need no lane exchange, and V^T's operand is one 16-byte piece
//     of a V tile (8 tokens of one dimension).  The larger MFMA also leaves
//     more room for vector work between matrix instructions than
//     16x16x32 did.
//   * Softmax in base-2 units (v_exp_f32), scale * log2(e) folded into one
//     multiply-add per score.  The weights are rounded to bf16 for the PV
//     product, and the running sum adds those same rounded weights
//     (v_dot2c_f32_bf16 against (1, 1)), so each row's output is exactly a
//     weighted mean of V rows.  A row's keys are split over lanes l and
//     l ^ 32; their maximum and sum are combined with v_permlane32_swap.
//   * The running maximum is a reference value that only moves when needed.
//     The weights of each 32 keys are first taken against the reference as
//     it stands; only if a row has no reference yet, or a lane's 16 weights
//     sum to more than 2^8 (kLaneSumLimit; an overflow to inf also fails the
//     test), is the row maximum of those keys computed, the reference
//     moved up to it, the row's output and sum rescaled, and the weights taken
//     again.  Weights therefore never exceed 2^8, well inside bf16 and fp32
//     range, and the result is the same softmax (the reference cancels in the
//     final division).  With well-scaled scores the reference is set by a
//     row's first keys, and later keys skip both the row maximum and the
//     rescale of 32 accumulators.
//   * Masked scores (future positions, keys past the context, blocks outside
//     the pool) become -inf.  V of keys past the context or in dropped blocks
//     is zeroed in registers after its LDS read (only in chunks that hold the
//     context end or a dropped block), because LDS may hold stale data there,
//     NaN included.
#include "tv_internal.h"

#include <math.h>

#include <atomic>

namespace tv {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

#define TV_GLOBAL __attribute__((address_space(1)))
#define TV_LDS __attribute__((address_space(3)))

constexpr int D = kHeadDim;
constexpr int BS = kBlockSize;
constexpr int kWaves = 8;                        // wavefronts per workgroup
constexpr int kRows = 32;                        // MFMA columns (query rows) per wavefront
constexpr int kThreads = 64 * kWaves;
constexpr int kWavesPerSimd = 4;                 // occupancy the register budget is cut for
constexpr int kChunkBlocks = kWaves;             // blocks per key chunk: one per wavefront
constexpr int kChunkKeys = kChunkBlocks * BS;    // 128
constexpr int kPairs = kChunkBlocks / 2;         // 32-key steps of a chunk, one block pair each
constexpr int kTileBytes = BS * D * 2;           // one (block, K/V head) tile: 2 KiB
constexpr int kHalfBytes = kChunkBlocks * kTileBytes;   // K (or V) of one chunk: 16 KiB
constexpr int kBufBytes = 2 * kHalfBytes;        // K then V of one chunk
constexpr float kLaneSumLimit = 256.0f;          // a lane's 16 weights of a 32-key step may sum to this
static_assert(D == 64 && BS == 16, "tile layout assumes 64 dims and 16-token blocks");

__device__ __forceinline__ unsigned zero_from(unsigned w, int lim, int e)
{
    // Clear the 16-bit halves of word w holding elements e, e+1 that are >= lim.
    const unsigned lo = e >= lim ? 0u : (w & 0xFFFFu);
    const unsigned hi = e + 1 >= lim ? 0u : (w & 0xFFFF0000u);
    return lo | hi;
}

__device__ __forceinline__ float max2(float a, float b) { return __builtin_elementwise_maximum(a, b); }

// The pair (x[l], x[l ^ 32]) in some order, from v_permlane32_swap.  The
// results are copied out of the returned vector before the bit casts: a bit
// cast of a vector element reads the vector's first element here.
__device__ __forceinline__ void swap32(float x, float &a, float &b)
{
    const unsigned u = __builtin_bit_cast(unsigned, x);
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    const unsigned r0 = r[0], r1 = r[1];
    a = __builtin_bit_cast(float, r0);
    b = __builtin_bit_cast(float, r1);
}

// Maximum and sum over the lanes l and l ^ 32, which hold one row's keys.
__device__ __forceinline__ float pair_max(float x)
{
    float a, b;
    swap32(x, a, b);
    return max2(a, b);
}

__device__ __forceinline__ float pair_sum(float x)
{
    float a, b;
    swap32(x, a, b);
    return a + b;
}

// Copy 1 KiB with one wavefront: lane l moves the 16 bytes at its own src
// to lds + 16 l (lds is the wavefront's base, the same in every lane),
// straight from memory to LDS without passing through registers.
__device__ __forceinline__ void copy_to_lds(const char *src, char *lds)
{
    __builtin_amdgcn_global_load_lds((const TV_GLOBAL void *)src, (TV_LDS void *)lds, 16, 0, 0);
}

template <int G, int KS>
__global__ __launch_bounds__(kThreads, kWavesPerSimd) void paged_prefill_kernel(PrefillArgs a)
{
    constexpr int kRowWaves = kWaves / KS;             // wavefronts per key share
    constexpr int kTokPerWave = kRows / G;
    constexpr int kTokPerWg = kRowWaves * kTokPerWave;
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
    const int rw = wave % kRowWaves;                          // row wavefront
    const int kh = wave / kRowWaves;                          // key share: steps kp with kp % KS == kh
    const int lane = tid & 63;
    const int col = lane & 31;                                // this lane's row (MFMA column)
    const int hh = lane >> 5;                                 // which half of the k-slots
    const int Hq = a.num_kv_heads * G;

    const int i0 = t * kTokPerWg;                             // first chunk row of the tile
    const int i1 = min(mq, i0 + kTokPerWg);
    const int base_pos = n - m;                               // position of chunk row 0
    const int wg_last_pos = base_pos + i1 - 1;
    const int nchunks = wg_last_pos >= 0 ? wg_last_pos / kChunkKeys + 1 : 0;

    // This wavefront's rows.
    const int iw0 = i0 + rw * kTokPerWave;
    const int iw1 = min(i1, iw0 + kTokPerWave);
    const int wave_first_pos = base_pos + iw0;
    const int wave_last_pos = iw1 > iw0 ? base_pos + iw1 - 1 : -1;   // -1: no rows

    // Query operand: column col is wave row col = chunk row iw0 + col / G,
    // query head kvh * G + col % G; k-slots 8 hh .. 8 hh + 7 of dimension
    // slab d16 are dims 16 d16 + 8 hh ...
    bf16x8 qop[4];
    const int qi = iw0 + col / G;
    const bool row_ok = qi < iw1;
    const int pos = base_pos + qi;
    {
        const u32x4 zero = {0u, 0u, 0u, 0u};
        const int qa = row_ok ? qi : 0;                       // an existing row for the address
        const u32x4 *qp = reinterpret_cast<const u32x4 *>(
            a.q + ((int64_t)(q0 + qa) * Hq + kvh * G + col % G) * D + 8 * hh);
#pragma unroll
        for (int d16 = 0; d16 < 4; ++d16)
            qop[d16] = __builtin_bit_cast(bf16x8, row_ok ? qp[2 * d16] : zero);
    }

    // Chunk loading: wavefront w copies block w of the chunk, K tile
    // verbatim (2 x 1 KiB) and V tile with its 16-byte pieces swizzled:
    // piece (dim d, token half h) goes to LDS offset 32 d + 16 (h ^ ((d >> 3) & 1)),
    // so that 32 lanes reading one half of 32 consecutive dims hit all 64
    // banks once.  Lane l of copy i takes LDS slot l, i.e. dim 32 i + l / 2,
    // half (l & 1) ^ (dim >> 3 & 1).
    const int32_t *table = a.block_tables + (int64_t)s * a.max_blocks;
    const uint32_t nb_cap = a.num_blocks > 0x7fffffff ? 0x80000000u : (uint32_t)a.num_blocks;
    const char *kheads = reinterpret_cast<const char *>(a.k_cache) + (int64_t)kvh * kTileBytes;
    const char *vheads = reinterpret_cast<const char *>(a.v_cache) + (int64_t)kvh * kTileBytes;
    const int64_t block_stride = (int64_t)a.num_kv_heads * kTileBytes;
    const int vd_lane = lane >> 1;
    const int v_src_off = vd_lane * 32 + 16 * ((lane & 1) ^ ((vd_lane >> 3) & 1));   // copy 0; copy 1 adds 1 KiB
    // Table entries of a chunk: lane j < 8 holds block j's entry (-1 past
    // the context), loaded one chunk before the copy that needs it, so that
    // no wait on the entry falls behind copies still in flight.
    auto entries = [&](int c) -> int32_t {
        const int b = c * kChunkBlocks + lane;
        return lane < kChunkBlocks && b * BS < n ? table[b] : -1;
    };
    auto load_chunk = [&](int32_t e, char *buf) {
        if ((uint32_t)e < nb_cap) {
            const char *kt = kheads + (int64_t)e * block_stride;
            const char *vt = vheads + (int64_t)e * block_stride;
            char *kl = buf + wave * kTileBytes;
            char *vl = buf + kHalfBytes + wave * kTileBytes;
            copy_to_lds(kt + 16 * lane, kl);
            copy_to_lds(kt + 1024 + 16 * lane, kl + 1024);
            copy_to_lds(vt + v_src_off, vl);
            copy_to_lds(vt + 1024 + v_src_off, vl + 1024);
        }
    };
    auto valid_of = [&](int32_t e) {
        return (unsigned)__builtin_amdgcn_ballot_w64((uint32_t)e < nb_cap) & ((1u << kChunkBlocks) - 1);
    };

    // Operand addresses within a chunk buffer.  Scores S^T = K . Q^T over
    // 32 keys of block pair kp: A-operand row r (lane r + 32 h reads dims
    // 16 d16 + 8 h ..) is the key 16 (r / 16) + 8 ((r / 4) & 1) + 4 ((r / 8) & 1) + r % 4,
    // so that result lane (col, hh) holds keys 8 hh .. 8 hh + 7 (elements
    // 0..7) and 16 + 8 hh .. (elements 8..15) of the pair for row col: the
    // B operand of the PV product for keys 0-15 and 16-31 as it stands.
    const int kr = col;
    const int ktok = 8 * ((kr >> 2) & 1) + 4 * ((kr >> 3) & 1) + (kr & 3);
    const int k_rd = (kr >> 4) * kTileBytes + hh * 256 + ktok * 16;     // + kp tiles, + 512 d16
    // PV: A operand lane (col, hh) of dim tile dt = V^T[dim 32 dt + col][tokens 8 hh ..]
    // of the block, from its swizzled slot.
    const int v_rd0 = col * 32 + 16 * (hh ^ ((col >> 3) & 1));          // dim tile 0
    const int v_rd1 = (32 + col) * 32 + 16 * (hh ^ (((32 + col) >> 3) & 1));

    f32x16 o[2];
#pragma unroll
    for (int dt = 0; dt < 2; ++dt)
#pragma unroll
        for (int j = 0; j < 16; ++j)
            o[dt][j] = 0.f;
    float m_ref = -INFINITY;                                  // reference maximum (base-2 units)
    float m_use = 0.f;                                        // the same, 0 while no key is seen
    float l_run = 0.f;
    const float cs = a.scale_log2;
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
    // Whether every row of the wavefront has a reference maximum.  Uniform;
    // set only where the reference moves, so the common step tests a scalar.
    bool all_ref = false;

    unsigned valid_next = 0;
    int32_t e_next = -1;                                      // entries of chunk c + 1 (lanes 0..7)
    if (nchunks > 0) {
        const int32_t e0 = entries(0);
        valid_next = valid_of(e0);
        load_chunk(__builtin_amdgcn_readlane(e0, wave), lds);
        if (nchunks > 1)
            e_next = entries(1);
    }
    for (int c = 0; c < nchunks; ++c) {
        char *buf = lds + (c & 1) * kBufBytes;
        const unsigned valid = valid_next;
        __syncthreads();                                     // chunk c in LDS; buffer c + 1 free
        if (c + 1 < nchunks) {
            valid_next = valid_of(e_next);
            load_chunk(__builtin_amdgcn_readlane(e_next, wave), lds + ((c + 1) & 1) * kBufBytes);
            if (c + 2 < nchunks)
                e_next = entries(c + 2);
        }
        if (c * kChunkKeys > wave_last_pos)
            continue;                                        // this wave's rows are done
        // V of keys past the context end or in dropped blocks is zeroed in
        // registers (LDS may hold stale data there, NaN included).
        // (Kept as a uniform integer: as a bool the compiler carried it
        // through a vector register and back on every step.)
        const int vfix = __builtin_amdgcn_readfirstlane(
            (c * kChunkKeys + kChunkKeys > n || valid != (1u << kChunkBlocks) - 1) ? 1 : 0);

#pragma unroll
        for (int kp = 0; kp < kPairs; ++kp) {
            const int key_base = c * kChunkKeys + 32 * kp;
            if (key_base > wave_last_pos)
                break;                                       // keys past this wave's rows
            if (KS > 1 && kp % KS != kh)
                continue;                                    // the other key share's step
            const bool mask = key_base + 31 > wave_first_pos || ((valid >> (2 * kp)) & 3u) != 3u;
            const char *kb = buf + 2 * kp * kTileBytes + k_rd;
            f32x16 sc = {};
#pragma unroll
            for (int d16 = 0; d16 < 4; ++d16) {
                const bf16x8 kop = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(kb + 512 * d16));
                sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, qop[d16], sc, 0, 0, 0);
            }
            // Element j of this lane is key key_base + 16 (j / 8) + 8 hh + j % 8.
            if (mask) {
                const int thr = pos - key_base - 8 * hh;
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    const int kk = 16 * (j / 8) + (j % 8);
                    if (kk > thr || !((valid >> (2 * kp + j / 8)) & 1u))
                        sc[j] = -INFINITY;
                }
            }

            // Softmax weights against the reference maximum; the row maximum,
            // the move of the reference and the rescale only when some row has
            // no reference yet or some lane's 16 weights sum past 2^8.
            u32x4 pw[2];                                      // bf16 pairs of P: keys 0-15, 16-31
            auto weights = [&](float mu) {
                float csum = 0.f;
#pragma unroll
                for (int j = 0; j < 16; j += 2) {
                    const float p0 = __builtin_amdgcn_exp2f(fmaf(sc[j], cs, -mu));
                    const float p1 = __builtin_amdgcn_exp2f(fmaf(sc[j + 1], cs, -mu));
                    const bf16x2 pp = {(__bf16)p0, (__bf16)p1};
                    csum = __builtin_amdgcn_fdot2_f32_bf16(pp, ones, csum, false);
                    pw[j / 8][(j % 8) / 2] = __builtin_bit_cast(unsigned, pp);
                }
                return csum;
            };
            float csum = 0.f;
            bool fresh = !all_ref;
            if (!fresh) {
                csum = weights(m_use);
                fresh = __builtin_amdgcn_ballot_w64(!(csum <= kLaneSumLimit)) != 0;
            }
            if (fresh) {
                float mx = max2(max2(sc[0], sc[1]), sc[2]);
#pragma unroll
                for (int j = 3; j < 16; j += 2)
                    mx = max2(max2(mx, sc[j]), sc[j + 1 < 16 ? j + 1 : j]);
                const float mc = pair_max(mx) * cs;   // the row maximum of these keys
                const float m_new = max2(m_ref, mc);
                const float alpha = m_new > m_ref ? __builtin_amdgcn_exp2f(m_ref - m_new) : 1.f;
                m_ref = m_new;
                m_use = m_new == -INFINITY ? 0.f : m_new;
                l_run *= alpha;
#pragma unroll
                for (int dt = 0; dt < 2; ++dt)
                    o[dt] *= alpha;
                csum = weights(m_use);
                all_ref = __builtin_amdgcn_ballot_w64(m_ref == -INFINITY) == 0;
            }
            l_run += csum;

            // O^T[dims][rows] += V^T . P^T over keys 0-15 (block 2 kp) and
            // 16-31 (block 2 kp + 1).
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int blk = 2 * kp + h;
                const char *vb = buf + kHalfBytes + blk * kTileBytes;
                u32x4 v0 = *reinterpret_cast<const u32x4 *>(vb + v_rd0);
                u32x4 v1 = *reinterpret_cast<const u32x4 *>(vb + v_rd1);
                if (vfix) {
                    const int lim = ((valid >> blk) & 1u) ? n - (c * kChunkKeys + blk * BS + 8 * hh) : 0;
#pragma unroll
                    for (int w = 0; w < 4; ++w) {
                        v0[w] = zero_from(v0[w], lim, 2 * w);
                        v1[w] = zero_from(v1[w], lim, 2 * w);
                    }
                }
                const bf16x8 pop = __builtin_bit_cast(bf16x8, pw[h]);
                o[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, v0), pop, o[0], 0, 0, 0);
                o[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, v1), pop, o[1], 0, 0, 0);
            }
        }
    }

    if (KS > 1) {
        // Fold the other key shares' states into share 0's, through the chunk
        // buffers (free once every wavefront is past its last chunk).
        constexpr int kF = 2 + 32;                           // m, l, o: floats per lane
        float *st = reinterpret_cast<float *>(lds);
        auto at = [&](int share, int f) -> float & {
            return st[((share - 1) * kF + f) * (kRowWaves * 64) + rw * 64 + lane];
        };
        __syncthreads();
        if (kh > 0) {
            at(kh, 0) = m_ref;
            at(kh, 1) = l_run;
#pragma unroll
            for (int dt = 0; dt < 2; ++dt)
#pragma unroll
                for (int j = 0; j < 16; ++j)
                    at(kh, 2 + 16 * dt + j) = o[dt][j];
        }
        __syncthreads();
        if (kh > 0)
            return;
#pragma unroll
        for (int sh = 1; sh < KS; ++sh) {
            const float mb = at(sh, 0);
            const float mm = max2(m_ref, mb);
            if (mm != -INFINITY) {
                // A state with no reference yet holds l = 0 and o = 0 (its
                // values are relative to 0), so it weighs 0.
                const float wa = m_ref == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_ref - mm);
                const float wb = mb == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mb - mm);
                l_run = l_run * wa + at(sh, 1) * wb;
#pragma unroll
                for (int dt = 0; dt < 2; ++dt)
#pragma unroll
                    for (int j = 0; j < 16; ++j)
                        o[dt][j] = o[dt][j] * wa + at(sh, 2 + 16 * dt + j) * wb;
                m_ref = mm;
            }
        }
    }

    // Normalise and store: element j of dim tile dt is dim 32 dt + 8 (j / 4) + 4 hh + j % 4.
    const float l = pair_sum(l_run);
    if (!row_ok)
        return;
    const float inv = l > 0.f ? 1.f / l : 0.f;
    float *op = a.out + ((int64_t)(q0 + qi) * Hq + kvh * G + col % G) * D + 4 * hh;
#pragma unroll
    for (int dt = 0; dt < 2; ++dt)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const f32x4 v = {o[dt][4 * g] * inv, o[dt][4 * g + 1] * inv, o[dt][4 * g + 2] * inv,
                             o[dt][4 * g + 3] * inv};
            *reinterpret_cast<f32x4 *>(op + 32 * dt + 8 * g) = v;
        }
}

// Compute units of the current device (cached; 0 if unknown).
int prefill_cus()
{
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0)
        return 0;
    if (dev < 64) {
        const int c = cache[dev].load(std::memory_order_relaxed);
        if (c > 0)
            return c;
    }
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return 0;
    if (dev < 64)
        cache[dev].store(cus, std::memory_order_relaxed);
    return cus;
}

template <int G, int KS>
hipError_t launch_gk(const PrefillArgs &a, hipStream_t stream)
{
    constexpr int kTokPerWg = (kWaves / KS) * kRows / G;
    const int64_t tiles = (a.max_query_len + kTokPerWg - 1) / kTokPerWg;
    const int64_t grid = tiles * a.num_seqs * a.num_kv_heads;
    if (grid == 0)
        return hipSuccess;
    if (grid > 0x7FFFFFFF)
        return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((paged_prefill_kernel<G, KS>), dim3((unsigned)grid), dim3(kThreads), 0,
                       stream, a);
    return hipGetLastError();
}

// Grids smaller than the device's two workgroup slots per compute unit
// (chunked prefill of a few sequences) take two key shares per row tile.
template <int G>
hipError_t launch_g(const PrefillArgs &a, hipStream_t stream)
{
    constexpr int kTokPerWg = kWaves * kRows / G;
    const int64_t grid1 = (int64_t)((a.max_query_len + kTokPerWg - 1) / kTokPerWg) * a.num_seqs *
                          a.num_kv_heads;
    const int cus = prefill_cus();
    if (cus > 0 && grid1 < 2 * (int64_t)cus)
        return launch_gk<G, 2>(a, stream);
    return launch_gk<G, 1>(a, stream);
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
