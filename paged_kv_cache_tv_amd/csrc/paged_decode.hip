// Paged GQA decode attention, partition pass, for gfx950.
//
// What is computed ("vLLM" page, sections "가상 메모리 방식의 해결" and "Flash
// Attention"; "tiny-vllm 씹뜯맛즐 - (1)" page, section 2 on GQA): for one
// sequence, one K/V head g and one context partition, the query heads of g's
// group attend to the partition's cached tokens, gathered block by block
// through the sequence's block table.  The softmax is accumulated online: a
// running maximum and running sum per query head, rescaling the partial
// output whenever the maximum grows.  The partition's (max, sum, output)
// triple is written for the merge kernel.
//
// Mapping to CDNA4:
//   * One workgroup of 4 wavefronts per (sequence, K/V head, partition).  The
//     launch index runs K/V head fastest, so the workgroups reading one
//     physical block land on the same XCD (dispatch is round-robin over the
//     8 XCDs) when several sequences share it.
//   * Each wavefront takes every 4th 16-token block of the partition.  One
//     block of one K/V head is a 2 KiB K tile [16 tokens][64] plus a 2 KiB V
//     tile [64][16 tokens]; each lane loads 32 B of K and 4 x 8 B of V
//     straight from HBM into registers, already in MFMA operand layout.
//   * Scores S^T[16 tokens][16 heads] = K . Q^T come from two
//     v_mfma_f32_16x16x32_bf16 (K is the A operand, the group's queries the B
//     operand; columns past the group size are zero).  Lane (g = lane/16,
//     r = lane%16) then holds the scores of tokens 4g..4g+3 for query head r,
//     which is exactly the B-operand layout of a 16x16x16 MFMA contracting over
//     those 4 tokens -- so the probabilities never leave the lane.
//   * O^T[64 dims][16 heads] += V^T . P^T uses v_mfma_f32_16x16x16_bf16 four
//     times (16 dims each).  P is split into bf16 hi + lo parts (two MFMAs)
//     so the products keep ~16 bits of P's mantissa instead of 8.
//   * exp is computed as 2^x (v_exp_f32) with scale*log2(e) folded into the
//     scores; the running maximum is kept in those base-2 units.
//   * The wavefronts' (max, sum, output) are merged through LDS at the end.
#include "tv_internal.h"

#include <math.h>

namespace tv {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int D = kHeadDim;
constexpr int BS = kBlockSize;
constexpr int kTileElems = BS * D;   // one (block, K/V head) tile: 1024 bf16
constexpr int kWaves = 4;

struct Tile {
    bf16x8 k0, k1;       // K[token r][16g .. 16g+8), K[token r][16g+8 .. 16g+16)
    i16x4 v[4];          // V^T[16j + r][4g .. 4g+4), j = 0..3
};

__device__ __forceinline__ void load_tile(Tile &t, const uint16_t *kt, const uint16_t *vt,
                                          int r, int g)
{
    const uint4 *kp = reinterpret_cast<const uint4 *>(kt + r * D + g * 16);
    t.k0 = __builtin_bit_cast(bf16x8, kp[0]);
    t.k1 = __builtin_bit_cast(bf16x8, kp[1]);
#pragma unroll
    for (int j = 0; j < 4; ++j)
        t.v[j] = __builtin_bit_cast(i16x4, *reinterpret_cast<const uint2 *>(vt + (16 * j + r) * BS + 4 * g));
}

// Fold one 16-token tile into the running (m, l, o) of this lane's query head.
// `valid` = how many of this lane's 4 tokens (4g..4g+3) lie inside the context;
// only consulted when MASK is set (the partition's last, partial tile).
template <bool MASK>
__device__ __forceinline__ void attend_tile(const Tile &t, bf16x8 qb0, bf16x8 qb1, int valid,
                                            float c, float &m_run, float &l_run, f32x4 (&o)[4])
{
    // No multiply-add contraction here: the base-2 scores must be rounded once
    // and reused unchanged by the max and by every exponent.
#pragma clang fp contract(off)
    f32x4 sc = {0.f, 0.f, 0.f, 0.f};
    sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(t.k0, qb0, sc, 0, 0, 0);
    sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(t.k1, qb1, sc, 0, 0, 0);

    i16x4 v0 = t.v[0], v1 = t.v[1], v2 = t.v[2], v3 = t.v[3];
    if (MASK) {
        // Tokens past the context: score -inf (weight exactly 0) and V forced
        // to 0, since stale slots may hold NaN and 0 * NaN is NaN.
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (i >= valid) {
                sc[i] = -INFINITY;
                v0[i] = 0;
                v1[i] = 0;
                v2[i] = 0;
                v3[i] = 0;
            }
        }
    }

    // Scores in base-2 units, rounded once, so the maximum token's weight is
    // exactly 2^0 = 1 (a one-token context returns its V bit for bit).
    float s2[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
        s2[i] = sc[i] * c;
    float mx = fmaxf(fmaxf(s2[0], s2[1]), fmaxf(s2[2], s2[3]));
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    float p[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
        p[i] = __builtin_amdgcn_exp2f(s2[i] - m_new);
    l_run = fmaf(l_run, alpha, (p[0] + p[1]) + (p[2] + p[3]));
    m_run = m_new;
#pragma unroll
    for (int j = 0; j < 4; ++j)
        o[j] *= alpha;

    bf16x4 hi, lo;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        hi[i] = (__bf16)p[i];
        lo[i] = (__bf16)(p[i] - (float)hi[i]);
    }
    const i16x4 phi = __builtin_bit_cast(i16x4, hi);
    const i16x4 plo = __builtin_bit_cast(i16x4, lo);
    o[0] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(v0, phi, o[0], 0, 0, 0);
    o[1] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(v1, phi, o[1], 0, 0, 0);
    o[2] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(v2, phi, o[2], 0, 0, 0);
    o[3] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(v3, phi, o[3], 0, 0, 0);
    o[0] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(v0, plo, o[0], 0, 0, 0);
    o[1] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(v1, plo, o[1], 0, 0, 0);
    o[2] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(v2, plo, o[2], 0, 0, 0);
    o[3] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(v3, plo, o[3], 0, 0, 0);
}

__global__ __launch_bounds__(64 * kWaves) void paged_decode_kernel(DecodeArgs a)
{
    const int kvh = (int)(blockIdx.x % (unsigned)a.num_kv_heads);
    const int rest = (int)(blockIdx.x / (unsigned)a.num_kv_heads);
    const int s = rest % a.num_seqs;
    const int part = rest / a.num_seqs;

    int n = a.context_lens[s];
    n = n < 0 ? 0 : (n > a.max_context_len ? a.max_context_len : n);
    const int first_tok = part * a.part_tiles * BS;
    if (first_tok >= n)
        return;
    const int ptok = min(n - first_tok, a.part_tiles * BS);    // tokens in this partition
    const int ntiles = (ptok + BS - 1) / BS;

    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int r = lane & 15;
    const int g = lane >> 4;
    const float c = a.scale_log2;
    const int G = a.group;

    // B operand of the score MFMA: column r = query head kvh*G + r.
    bf16x8 qb0 = {}, qb1 = {};
    if (r < G) {
        const uint4 *qp = reinterpret_cast<const uint4 *>(
            a.q + ((int64_t)s * a.num_kv_heads * G + (int64_t)kvh * G + r) * D + g * 16);
        qb0 = __builtin_bit_cast(bf16x8, qp[0]);
        qb1 = __builtin_bit_cast(bf16x8, qp[1]);
    }

    float m_run = -INFINITY, l_run = 0.f;
    f32x4 o[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
        o[j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int32_t *bt = a.block_tables + (int64_t)s * a.max_blocks + (int64_t)part * a.part_tiles;
    const int64_t tile_stride = (int64_t)a.num_kv_heads * kTileElems;
    const uint16_t *kbase = a.k_cache + (int64_t)kvh * kTileElems;
    const uint16_t *vbase = a.v_cache + (int64_t)kvh * kTileElems;
    const int ntw = w < ntiles ? (ntiles - w + kWaves - 1) / kWaves : 0;   // tiles of this wave

    for (int c0 = 0; c0 < ntw; c0 += 64) {
        const int cn = min(64, ntw - c0);
        // This wave's table entries for the chunk, one per lane.
        const int32_t phys_lane = lane < cn ? bt[w + kWaves * (c0 + lane)] : 0;

        auto tile_block = [&](int k) -> int64_t {
            const int32_t b = __builtin_amdgcn_readlane(phys_lane, k);
            return (b >= 0 && b < a.num_blocks) ? (int64_t)b : -1;
        };
        auto issue = [&](Tile &t, int64_t b) {
            const int64_t bb = b < 0 ? 0 : b;
            load_tile(t, kbase + bb * tile_stride, vbase + bb * tile_stride, r, g);
        };
        auto consume = [&](const Tile &t, int k, int64_t b) {
            if (b < 0)
                return;                                     // entry outside the pool: skipped
            const int it = w + kWaves * (c0 + k);           // tile index inside the partition
            if ((it + 1) * BS <= ptok)
                attend_tile<false>(t, qb0, qb1, 4, c, m_run, l_run, o);
            else
                attend_tile<true>(t, qb0, qb1, ptok - it * BS - 4 * g, c, m_run, l_run, o);
        };

        Tile ta, tb;
        int64_t ba = tile_block(0), bb2 = -1;
        issue(ta, ba);
        for (int k = 0; k < cn; k += 2) {
            if (k + 1 < cn) {
                bb2 = tile_block(k + 1);
                issue(tb, bb2);
            }
            consume(ta, k, ba);
            if (k + 1 >= cn)
                break;
            if (k + 2 < cn) {
                ba = tile_block(k + 2);
                issue(ta, ba);
            }
            consume(tb, k + 1, bb2);
        }
    }

    // Sum the lane groups' partial l (same query head, different tokens).
    l_run += __shfl_xor(l_run, 16);
    l_run += __shfl_xor(l_run, 32);

    __shared__ float sm_m[kWaves][16];
    __shared__ float sm_l[kWaves][16];
    __shared__ float sm_o[kWaves][16][D];
    if (g == 0) {
        sm_m[w][r] = m_run;
        sm_l[w][r] = l_run;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            sm_o[w][r][16 * j + 4 * g + i] = o[j][i];
    __syncthreads();

    const int hq = a.num_kv_heads * G;
    for (int e = threadIdx.x; e < G * D; e += 64 * kWaves) {
        const int hr = e / D;
        const int d = e % D;
        float M = -INFINITY;
#pragma unroll
        for (int x = 0; x < kWaves; ++x)
            M = fmaxf(M, sm_m[x][hr]);
        float num = 0.f, den = 0.f;
#pragma unroll
        for (int x = 0; x < kWaves; ++x) {
            const float mx = sm_m[x][hr];
            const float f = mx == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mx - M);
            num = fmaf(f, sm_o[x][hr][d], num);
            den = fmaf(f, sm_l[x][hr], den);
        }
        const int64_t row = ((int64_t)s * hq + (int64_t)kvh * G + hr) * a.num_parts + part;
        a.part_acc[row * D + d] = num;
        if (d == 0) {
            a.part_max[row] = M;
            a.part_sum[row] = den;
        }
    }
}

}  // namespace

hipError_t launch_paged_decode(const DecodeArgs &a, hipStream_t stream)
{
    const int64_t groups = (int64_t)a.num_kv_heads * a.num_seqs * a.num_parts;
    hipLaunchKernelGGL(paged_decode_kernel, dim3((unsigned)groups), dim3(64 * kWaves), 0, stream, a);
    return hipGetLastError();
}

}  // namespace tv
