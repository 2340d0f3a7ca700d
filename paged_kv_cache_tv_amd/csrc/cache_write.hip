// Cache write: scatter each new token's K and V rows into the slot the engine
// chose for it ("Tiny-vLLM" page, slot_mapping; "vLLM" page, fixed 16-token
// blocks).  A pure bit copy, or with K turned by the rotary position
// embedding on the way in (and the same rotation in place for q).
//
// A token's K (or V) is num_kv_heads * head_dim bf16 values, contiguous in
// the input; lanes take 16-byte chunks (8 values of one head, since head_dim %
// 8 == 0).  The K tile of a (block, head) is stored as head_dim / 8 chunks of
// [block_size tokens][8 dims], so each K chunk is one 16-byte store at
// (chunk, token offset); the V tile is dimension-major [head_dim][block_size].
#include "rope_math.h"
#include "tv_internal.h"

namespace tv {
namespace {

// Streaming (non-temporal) 16-byte loads and stores for the bulk form and
// the in-place rotation: a prompt's K/V rows (or q) are read once and what is
// written is not read back by the same kernel, so neither should displace
// other data in the caches.
// Measured on 16,384 prompt tokens: the plain write 17.1 -> 12.7 us and the
// RoPE write 20.9 -> 17.0 us (launch loops, same process).
typedef uint32_t nt_u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void nt_store(const uint4 &x, uint4 *p)
{
    const nt_u32x4 v = {x.x, x.y, x.z, x.w};
    __builtin_nontemporal_store(v, reinterpret_cast<nt_u32x4 *>(p));
}
__device__ __forceinline__ uint4 nt_load(const uint4 *p)
{
    const nt_u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const nt_u32x4 *>(p));
    return make_uint4(v[0], v[1], v[2], v[3]);
}

constexpr int kWavesPerGroup = 4;      // wavefronts per workgroup (one token each, unstaged forms)
constexpr int kTokensPerGroup = 16;    // tokens per workgroup, staged form (4 per wavefront)
constexpr int64_t kStagedFrom = 512;   // launches of at least this many tokens use the staged form

// One wavefront per token.
// STAGED (launches of many tokens, e.g. a prompt): 16 consecutive tokens per
// workgroup.  When they fill one whole block in order (slots 16b .. 16b + 15)
// their K rows (turned, with ROPE) and V rows are staged in LDS, and the
// block goes out as whole 16-byte runs in address order: the block's K for
// all heads is one contiguous [head][chunk][16 tokens][8 dims] region, each
// thread storing one (chunk, token) piece; V's thread writes 8 tokens of one
// dim of the dimension-major V tile.  Otherwise (and in the unstaged form, 4
// tokens per workgroup with no LDS and no barrier, for the few tokens of a
// decode step) each token's K goes out as 16-byte chunk stores and its V as
// 2-byte stores down its column.
//
// ROPE: K is turned by the rotary embedding of positions[tok] before the
// store (see rope_math.h).  Lanes 0 .. head_dim/2 - 1 compute the token's
// (cos, sin) per pair once; a lane handling pairs 4q .. 4q+3 of a head (q =
// its group within the head) fetches them with shuffles, in a loop whose trip
// count is the same for every lane.  Style 0 pairs dims (2k, 2k+1), so group
// q is the 16-byte chunk q of the head; style 1 pairs (k, k + head_dim/2), so
// group q is dims 4q .. 4q+3 and their partners, two 8-byte pieces.
template <bool ROPE, bool STAGED>
__global__ __launch_bounds__(64 * kWavesPerGroup)
void cache_write_kernel(CacheWriteArgs a)
{
    constexpr int kPerWave = STAGED ? kTokensPerGroup / kWavesPerGroup : 1;   // tokens per wavefront
    constexpr int kTok = kWavesPerGroup * kPerWave;                          // tokens per workgroup
    __shared__ int64_t s_slot[STAGED ? kTokensPerGroup : 1];
    __shared__ uint4 s_v[STAGED ? kTokensPerGroup * 64 : 1];   // V rows of a full block (<= 512 values each)
    // K rows of a full block, one row per token padded to 65 chunks so that
    // the 16 tokens of one chunk sit on distinct banks.
    constexpr int kKStride = 65;
    __shared__ uint4 s_k[STAGED ? kTokensPerGroup * kKStride : 1];
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform: scalar token loads
    const int lane = threadIdx.x & 63;
    const int row = a.num_kv_heads * a.head_dim;
    const int chunks = row >> 3;
    // Wavefront w takes tokens kPerWave*w .. kPerWave*w + kPerWave - 1 of the
    // workgroup.  Every load the common case (num_kv_heads * head_dim <= 512)
    // needs is issued before any is used, so the wavefront waits on memory
    // once: first each token's slot and, with ROPE, its position (wave-uniform
    // addresses: scalar loads), then its first K and V chunk per lane.  The
    // row loads are unconditional (a token past the end reads the last token's
    // row, a lane past the row its last chunk; neither value is used), so no
    // wait is tied to a branch around them.
    int64_t toks[kPerWave], tcs[kPerWave], slots[kPerWave];
    uint4 k0s[kPerWave], v0s[kPerWave];
    int poss[kPerWave];
#pragma unroll
    for (int i = 0; i < kPerWave; ++i) {
        toks[i] = (int64_t)blockIdx.x * kTok + w * kPerWave + i;
        tcs[i] = toks[i] < a.num_tokens ? toks[i] : a.num_tokens - 1;
        slots[i] = a.slot_mapping[tcs[i]];
        poss[i] = ROPE ? a.positions[tcs[i]] : 0;
    }
    const float f_lane = ROPE ? a.inv_freq[lane % (a.head_dim >> 1)] : 0.f;
    const int cl = lane < chunks ? lane : chunks - 1;
#pragma unroll
    for (int i = 0; i < kPerWave; ++i) {
        const uint4 *krow = reinterpret_cast<const uint4 *>(a.k + tcs[i] * row) + cl;
        const uint4 *vrow = reinterpret_cast<const uint4 *>(a.v + tcs[i] * row) + cl;
        // RoPE reads K with cached loads: style 1 re-reads the row as 8-byte
        // pieces, which a streaming load would have pushed out.
        k0s[i] = STAGED && !ROPE ? nt_load(krow) : *krow;
        v0s[i] = STAGED ? nt_load(vrow) : *vrow;
    }
#pragma unroll
    for (int i = 0; i < kPerWave; ++i)
        if (toks[i] >= a.num_tokens)
            slots[i] = -1;
    bool full = false;
    int64_t s0 = 0;
    if (STAGED) {
        if (lane == 0) {
#pragma unroll
            for (int i = 0; i < kPerWave; ++i)
                s_slot[w * kPerWave + i] = slots[i];
        }
        // A full block: 16 tokens, slots 16b .. 16b + 15 in order, V rows that
        // fit in LDS, and a V pool aligned for 16-byte stores.
        full = row <= 512 && a.block_size == kTokensPerGroup &&
               (reinterpret_cast<uintptr_t>(a.v_cache) & 15) == 0;
        __syncthreads();
        s0 = s_slot[0];
        full = full && s0 >= 0 && s0 % kTokensPerGroup == 0 && s0 + kTokensPerGroup <= a.num_slots;
#pragma unroll
        for (int i = 1; i < kTokensPerGroup; ++i)
            full = full && s_slot[i] == s0 + i;
        if (full && lane < chunks) {
#pragma unroll
            for (int i = 0; i < kPerWave; ++i)
                s_v[(w * kPerWave + i) * 64 + lane] = v0s[i];
        }
    } else if (toks[0] >= a.num_tokens) {
        return;
    }

#pragma unroll
    for (int ti = 0; ti < kPerWave; ++ti) {
        const int64_t tok = toks[ti];
        const bool live_tok = tok < a.num_tokens;
        const int64_t slot = slots[ti];
        const uint4 k0 = k0s[ti];
        const uint4 v0 = v0s[ti];
        const uint4 *ksrc = reinterpret_cast<const uint4 *>(a.k + tok * row);
        const uint4 *vsrc = reinterpret_cast<const uint4 *>(a.v + tok * row);
        uint16_t *const sk_row =
            reinterpret_cast<uint16_t *>(s_k + (STAGED ? (w * kPerWave + ti) * kKStride : 0));
        const bool write = slot >= 0 && slot < a.num_slots;
        const int64_t blk = write ? slot / a.block_size : 0;
        const int off = write ? (int)(slot - blk * a.block_size) : 0;
        float pc = 1.f, ps = 0.f;
        if (ROPE && live_tok)
            rope_cos_sin(poss[ti], f_lane, pc, ps);
        for (int base = 0; base < chunks; base += 64) {
            const int c = base + lane;
            float cs[4], sn[4];
            if (ROPE) {
                const int q = c % (a.head_dim >> 3);
    #pragma unroll
                for (int i = 0; i < 4; ++i) {
                    cs[i] = __shfl(pc, 4 * q + i);
                    sn[i] = __shfl(ps, 4 * q + i);
                }
            }
            if (!write || c >= chunks)
                continue;
            const int h = (c << 3) / a.head_dim;
            const int d = (c << 3) - h * a.head_dim;
            const int64_t tile = blk * a.num_kv_heads + h;
            uint16_t *ktile = a.k_cache + tile * a.head_dim * a.block_size;
            if (!ROPE) {
                const uint4 kk = c == lane ? k0 : ksrc[c];
                if (STAGED && full)
                    reinterpret_cast<uint4 *>(sk_row)[c] = kk;
                else
                    *reinterpret_cast<uint4 *>(ktile + ((int64_t)(d >> 3) * a.block_size + off) * 8) = kk;
            } else if (a.rope_style == 0) {
                // Pairs (d + 2i, d + 2i + 1), i < 4: one 16-byte chunk in and out.
                const uint4 kk = c == lane ? k0 : ksrc[c];
                const uint32_t wd[4] = {kk.x, kk.y, kk.z, kk.w};
                uint32_t o[4];
    #pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float ra, rb;
                    rope_turn(__uint_as_float(wd[i] << 16), __uint_as_float(wd[i] & 0xFFFF0000u),
                              cs[i], sn[i], ra, rb);
                    o[i] = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)ra) |
                           ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)rb) << 16);
                }
                if (STAGED && full)
                    reinterpret_cast<uint4 *>(sk_row)[c] = make_uint4(o[0], o[1], o[2], o[3]);
                else
                    *reinterpret_cast<uint4 *>(ktile + ((int64_t)(d >> 3) * a.block_size + off) * 8) =
                        make_uint4(o[0], o[1], o[2], o[3]);
            } else {
                // Pairs (4q + i, 4q + i + head_dim/2), i < 4, q = d / 8 within the head.
                const int half = a.head_dim >> 1;
                const int da = d >> 1;                           // 4q
                const uint16_t *src = a.k + tok * row + h * a.head_dim;
                const uint2 pa = *reinterpret_cast<const uint2 *>(src + da);
                const uint2 pb = *reinterpret_cast<const uint2 *>(src + da + half);
                const uint32_t wa[2] = {pa.x, pa.y}, wb[2] = {pb.x, pb.y};
                uint32_t oa[2] = {0u, 0u}, ob[2] = {0u, 0u};
    #pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const uint32_t xa = (wa[i >> 1] >> (16 * (i & 1))) & 0xFFFFu;
                    const uint32_t xb = (wb[i >> 1] >> (16 * (i & 1))) & 0xFFFFu;
                    float ra, rb;
                    rope_turn(__uint_as_float(xa << 16), __uint_as_float(xb << 16), cs[i], sn[i], ra,
                              rb);
                    oa[i >> 1] |= (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)ra) << (16 * (i & 1));
                    ob[i >> 1] |= (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)rb) << (16 * (i & 1));
                }
                const int db = da + half;
                if (STAGED && full) {
                    *reinterpret_cast<uint2 *>(sk_row + h * a.head_dim + da) = make_uint2(oa[0], oa[1]);
                    *reinterpret_cast<uint2 *>(sk_row + h * a.head_dim + db) = make_uint2(ob[0], ob[1]);
                } else {
                    *reinterpret_cast<uint2 *>(ktile + ((int64_t)(da >> 3) * a.block_size + off) * 8 +
                                               (da & 7)) = make_uint2(oa[0], oa[1]);
                    *reinterpret_cast<uint2 *>(ktile + ((int64_t)(db >> 3) * a.block_size + off) * 8 +
                                               (db & 7)) = make_uint2(ob[0], ob[1]);
                }
            }
            if (full)
                continue;
            const uint4 vv = c == lane ? v0 : vsrc[c];
            uint16_t *vdst = a.v_cache + (tile * a.head_dim + d) * a.block_size + off;
            const uint32_t wd[4] = {vv.x, vv.y, vv.z, vv.w};
    #pragma unroll
            for (int i = 0; i < 8; ++i) {
                const uint32_t word = wd[i >> 1];
                vdst[(int64_t)i * a.block_size] = (uint16_t)((i & 1) ? (word >> 16) : (word & 0xFFFFu));
            }
        }
    }
    if (!STAGED || !full)
        return;
    // Full block: thread t writes tokens 8 (t & 1) .. + 7 of dim d = (t / 2) %
    // head_dim of head t / (2 head_dim), 16 bytes of the V tile.
    __syncthreads();
    const uint16_t *sv = reinterpret_cast<const uint16_t *>(s_v);
    const int64_t vblk = s0 / kTokensPerGroup;
    // K: piece u = chunk * 16 + token of the block's contiguous K region.
    for (int u = threadIdx.x; u < chunks * kTokensPerGroup; u += 64 * kWavesPerGroup)
        nt_store(s_k[(u & (kTokensPerGroup - 1)) * kKStride + (u >> 4)],
                 reinterpret_cast<uint4 *>(a.k_cache + vblk * (int64_t)row * kTokensPerGroup) + u);
    for (int t = threadIdx.x; t < 2 * row; t += 64 * kWavesPerGroup) {
        const int e = t >> 1;                                  // h * head_dim + d
        const int t0 = 8 * (t & 1);
        uint32_t o[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            o[i] = (uint32_t)sv[(t0 + 2 * i) * 512 + e] |
                   ((uint32_t)sv[(t0 + 2 * i + 1) * 512 + e] << 16);
        const int h = e / a.head_dim;
        const int d = e - h * a.head_dim;
        nt_store(make_uint4(o[0], o[1], o[2], o[3]),
                 reinterpret_cast<uint4 *>(a.v_cache + ((vblk * a.num_kv_heads + h) * a.head_dim + d) *
                                           a.block_size + t0));
    }
}

// In-place rotary embedding of x [tokens][heads][head_dim], one wavefront per
// token, with the same lane layout as the cache write above.  A lane's
// chunks (up to kRopeChunks rounds of 64) are all loaded before the first is
// turned, so a token waits on memory once.  Style 0 reads and writes its
// 16-byte chunks with streaming accesses (each is read once and written
// once: 27.4 -> 24.1 us on 16,384 x 32 heads); style 1's two 8-byte pieces
// of one line stay cached (streaming them was slower).
constexpr int kRopeChunks = 8;

__global__ __launch_bounds__(64 * kWavesPerGroup) void rope_kernel(RopeArgs a)
{
    const int64_t tok = (int64_t)blockIdx.x * kWavesPerGroup + (threadIdx.x >> 6);
    if (tok >= a.num_tokens)
        return;
    const int lane = threadIdx.x & 63;
    const int half = a.head_dim >> 1;
    const int groups = (a.num_heads * a.head_dim) >> 3;
    uint16_t *xt = a.x + tok * a.num_heads * a.head_dim;
    // Lane's pieces: style 0 one 16-byte chunk c; style 1 dims 4q..4q+3 of
    // head h and their partners half further on (two 8-byte pieces).
    auto piece_a = [&](int c) -> uint16_t * {
        if (a.style == 0)
            return xt + 8 * c;
        const int h = (c << 3) / a.head_dim;
        const int q = c % (a.head_dim >> 3);
        return xt + h * a.head_dim + 4 * q;
    };
    uint4 in[kRopeChunks];
#pragma unroll
    for (int it = 0; it < kRopeChunks; ++it) {
        const int c = it * 64 + lane;
        in[it] = make_uint4(0, 0, 0, 0);
        if (it * 64 < groups && c < groups) {
            uint16_t *pa = piece_a(c);
            if (a.style == 0) {
                in[it] = nt_load(reinterpret_cast<const uint4 *>(pa));
            } else {
                const uint2 lo = *reinterpret_cast<const uint2 *>(pa);
                const uint2 hi = *reinterpret_cast<const uint2 *>(pa + half);
                in[it] = make_uint4(lo.x, lo.y, hi.x, hi.y);
            }
        }
    }
    float pc, ps;
    rope_cos_sin(a.positions[tok], a.inv_freq[lane % half], pc, ps);
    for (int base = 0; base < groups; base += 64) {
        const int it = base >> 6;
        const int c = base + lane;
        const int q = c % (a.head_dim >> 3);
        float cs[4], sn[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            cs[i] = __shfl(pc, 4 * q + i);
            sn[i] = __shfl(ps, 4 * q + i);
        }
        if (c >= groups)
            continue;
        uint4 kk = make_uint4(0, 0, 0, 0);
        if (it < kRopeChunks) {
#pragma unroll
            for (int j = 0; j < kRopeChunks; ++j)
                if (j == it)
                    kk = in[j];
        } else if (a.style == 0) {
            kk = *reinterpret_cast<const uint4 *>(piece_a(c));
        } else {
            const uint2 lo = *reinterpret_cast<const uint2 *>(piece_a(c));
            const uint2 hi = *reinterpret_cast<const uint2 *>(piece_a(c) + half);
            kk = make_uint4(lo.x, lo.y, hi.x, hi.y);
        }
        if (a.style == 0) {
            const uint32_t w[4] = {kk.x, kk.y, kk.z, kk.w};
            uint32_t o[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float ra, rb;
                rope_turn(__uint_as_float(w[i] << 16), __uint_as_float(w[i] & 0xFFFF0000u),
                          cs[i], sn[i], ra, rb);
                o[i] = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)ra) |
                       ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)rb) << 16);
            }
            nt_store(make_uint4(o[0], o[1], o[2], o[3]), reinterpret_cast<uint4 *>(piece_a(c)));
        } else {
            const uint32_t wa[2] = {kk.x, kk.y}, wb[2] = {kk.z, kk.w};
            uint32_t oa[2] = {0u, 0u}, ob[2] = {0u, 0u};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t xa = (wa[i >> 1] >> (16 * (i & 1))) & 0xFFFFu;
                const uint32_t xb = (wb[i >> 1] >> (16 * (i & 1))) & 0xFFFFu;
                float ra, rb;
                rope_turn(__uint_as_float(xa << 16), __uint_as_float(xb << 16), cs[i], sn[i], ra,
                          rb);
                oa[i >> 1] |= (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)ra) << (16 * (i & 1));
                ob[i >> 1] |= (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)rb) << (16 * (i & 1));
            }
            uint16_t *pa = piece_a(c);
            *reinterpret_cast<uint2 *>(pa) = make_uint2(oa[0], oa[1]);
            *reinterpret_cast<uint2 *>(pa + half) = make_uint2(ob[0], ob[1]);
        }
    }
}

}  // namespace

template <bool ROPE>
void launch_cw(const CacheWriteArgs &a, hipStream_t stream)
{
    if (a.num_tokens >= kStagedFrom) {
        const int64_t groups = (a.num_tokens + kTokensPerGroup - 1) / kTokensPerGroup;
        hipLaunchKernelGGL((cache_write_kernel<ROPE, true>), dim3((unsigned)groups),
                           dim3(64 * kWavesPerGroup), 0, stream, a);
    } else {
        const int64_t groups = (a.num_tokens + kWavesPerGroup - 1) / kWavesPerGroup;
        hipLaunchKernelGGL((cache_write_kernel<ROPE, false>), dim3((unsigned)groups),
                           dim3(64 * kWavesPerGroup), 0, stream, a);
    }
}

hipError_t launch_cache_write(const CacheWriteArgs &a, hipStream_t stream)
{
    if (a.positions)
        launch_cw<true>(a, stream);
    else
        launch_cw<false>(a, stream);
    return hipGetLastError();
}

hipError_t launch_rope(const RopeArgs &a, hipStream_t stream)
{
    const int64_t groups = (a.num_tokens + kWavesPerGroup - 1) / kWavesPerGroup;
    hipLaunchKernelGGL(rope_kernel, dim3((unsigned)groups), dim3(64 * kWavesPerGroup), 0, stream,
                       a);
    return hipGetLastError();
}

}  // namespace tv
