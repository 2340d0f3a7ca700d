// Paged GQA decode attention for gfx950: the partition pass, and the whole
// decode step in one launch (whole-sequence and whole-group forms).
//
// What is computed ("vLLM" page, sections "가상 메모리 방식의 해결" and "Flash
// Attention"; "tiny-vllm 씹뜯맛즐 - (1)" page, section 2 on GQA): for one
// sequence, one K/V head g and one context partition, the query heads of g's
// group attend to the partition's cached tokens, gathered block by block
// through the sequence's block table.  The softmax is accumulated online: a
// running maximum and running sum per query head, rescaling the partial
// output whenever the maximum grows.  The partition's (max, sum, output)
// triple is written for the merge kernel.  In the one-launch forms a
// workgroup takes a whole (sequence, K/V head) -- or a whole (group of
// sequences sharing a prefix, K/V head) -- cuts its tiles into equal ranges,
// one per wavefront, merges the ranges' triples in LDS by the same rule and
// writes the normalised output rows (paged_decode_seq_kernel,
// paged_decode_group_kernel).  With the cache write folded in, the
// wavefront holding a sequence's last tile substitutes the new token in
// registers and stores that tile back whole.
//
// Mapping to CDNA4:
//   * One workgroup per (sequence, K/V head, partition), of 4 wavefronts or
//     of 1 (the launch policy is at launch_paged_decode).  The launch index
//     runs K/V head fastest, so with 8 K/V heads each head's workgroups run
//     on one XCD (dispatch is round-robin over the 8 XCDs) and workgroups
//     reading one shared physical block share that XCD's L2.  Within an XCD
//     the dispatcher deals consecutive workgroups round-robin over its
//     compute units, each wavefront to the next SIMD; a SIMD's finishing time
//     follows the tiles it was dealt.  With 4 wavefronts the partition's
//     tiles are split evenly over the CU's 4 SIMDs.  Grids larger than what
//     the device holds at once take a balanced order derived from the
//     context lengths (plan_unit).
//   * One block of one K/V head is a 2 KiB K tile, stored as 8 chunks of
//     [16 tokens][8 dims], plus a 2 KiB V tile [64 dims][16 tokens].  Each
//     K load instruction reads 1 KiB contiguous (lane l: bytes 16l..16l+15 of
//     chunks 0-3, then of chunks 4-7) and each V load instruction 512 B
//     contiguous, so every 128-byte line is fetched by exactly one
//     instruction; the data arrives already in MFMA operand layout.  The
//     loads are non-temporal: K/V lines are used once and should not push the
//     partition results out of L2.  A ring of tile buffers keeps the next
//     tiles in flight while one is consumed: four buffers with one wavefront
//     per partition, two with four (which then fit in 128 registers, 4
//     wavefronts per SIMD).
//   * Scores S^T[16 tokens][16 heads] = K . Q^T come from two
//     v_mfma_f32_16x16x32_bf16 over dims 0-31 and 32-63 (K is the A operand,
//     the group's queries the B operand; columns past the group size are
//     zero), so the K tile is read once for all query heads of the group.
//     Lane (g = lane/16, r = lane%16) then holds the scores of tokens
//     4g..4g+3 for query head r, which is exactly the B-operand layout of a
//     16x16x16 MFMA contracting over those 4 tokens -- so the probabilities
//     never leave the lane.
//   * O^T[64 dims][16 heads] += V^T . P^T uses v_mfma_f32_16x16x16_bf16 four
//     times (16 dims each).  P is split into bf16 hi + lo parts (two MFMAs)
//     so the products keep ~16 bits of P's mantissa instead of 8.
//   * exp is computed as 2^x (v_exp_f32) with scale*log2(e) folded into the
//     scores; the running maximum is kept in those base-2 units.  The only
//     cross-lane traffic is the max over the 4 lane groups (2 shuffles per
//     tile) and one final sum; no barrier inside the tile loop.  LDS holds
//     the appended token's row in the append variant and, with 4 wavefronts,
//     the wavefronts' (max, sum, output) for the one barrier at the end.
#include "tv_internal.h"

#include <math.h>

#include <atomic>
#include <numeric>

namespace tv {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

constexpr int D = kHeadDim;
constexpr int BS = kBlockSize;
constexpr int kTileBytes = BS * D * 2;   // one (block, K/V head) tile: 1024 bf16
// Tile buffers per wavefront: one wavefront per partition streams up to 32
// tiles and keeps 3 in flight; with 4 per partition each streams a quarter,
// and a 2-deep ring lets 4 wavefronts share each SIMD (batch 64 x 512-4096
// tokens: 52.7 against 54.6 us).
template <int SPLIT>
constexpr int kRingFor = SPLIT > 1 ? 2 : 4;
// The whole-sequence form: one workgroup per (sequence, K/V head), wavefront
// p streaming partition p (so at most kSeqWaves partitions), two workgroups
// per compute unit (4 wavefronts per SIMD, registers capped at 128).
constexpr int kSeqWaves = 8;
constexpr int kSeqRing = 2;

struct Tile {
    bf16x8 k0, k1;       // K[token r][8g .. 8g+8), K[token r][32+8g .. 32+8g+8)
    i16x4 v[4];          // V^T[16j + r][4g .. 4g+4), j = 0..3
};

// kt, vt: tile bases (uniform); koff = 16*lane and voff = (r*16 + 4g)*2 bytes
// are this lane's offsets, the same for every tile.
__device__ __forceinline__ void load_tile(Tile &t, const char *kt, const char *vt, uint32_t koff,
                                          uint32_t voff)
{
    t.k0 = __builtin_bit_cast(bf16x8, __builtin_nontemporal_load(
                                          reinterpret_cast<const u32x4 *>(kt + koff)));
    t.k1 = __builtin_bit_cast(bf16x8, __builtin_nontemporal_load(
                                          reinterpret_cast<const u32x4 *>(kt + 1024 + koff)));
#pragma unroll
    for (int j = 0; j < 4; ++j)
        t.v[j] = __builtin_bit_cast(i16x4, __builtin_nontemporal_load(
                                               reinterpret_cast<const u32x2 *>(vt + voff + 512 * j)));
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

constexpr int kPlanChunks = 4;            // the balanced order serves up to 4 x 64 sequences

__device__ __forceinline__ int wave_scan_incl(int x, int lane)
{
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int y = __shfl_up(x, d);
        if (lane >= d)
            x += y;
    }
    return x;
}

struct Unit {
    int s;       // sequence (-1: this workgroup has no partition)
    int part;
};

// The partition that workgroup j of a K/V head takes in the balanced order.
// The work is every partition of every sequence; a partition's cost is its
// tile count.  Consecutive workgroups of a head are dealt round-robin over
// a.plan_width compute units, so the order is:
//   1. every partition that is not its sequence's last one (all full-sized),
//      sequence by sequence;
//   2. the sequences' last partitions from the largest to the smallest (ties:
//      lower sequence first), placed along a path that runs forward over the
//      CUs in one round and backward in the next, so a CU that got a large
//      one gets a small one next;
//   3. workgroups past the work (none).
// Every workgroup computes the same order from the same lengths, so each
// partition is taken exactly once.  num_seqs <= 64 * kPlanChunks.
__device__ Unit plan_unit(const DecodeArgs &a, int j, int lane)
{
    const int PT = a.part_tiles;
    int len[kPlanChunks];
#pragma unroll
    for (int k = 0; k < kPlanChunks; ++k) {
        // Unconditional loads (a lane past the batch reads the last length),
        // so all of them are in flight before the first is waited for.
        const int s = k * 64 + lane;
        len[k] = a.context_lens[s < a.num_seqs ? s : a.num_seqs - 1];
    }
#pragma unroll
    for (int k = 0; k < kPlanChunks; ++k)
        if (k * 64 + lane >= a.num_seqs)
            len[k] = 0;
    int last[kPlanChunks], nparts[kPlanChunks];
    int F = 0, L = 0;                            // partitions in step 1; sequences in step 2
    Unit u = {-1, 0};
#pragma unroll
    for (int k = 0; k < kPlanChunks; ++k) {
        int n = len[k];
        n = n < 0 ? 0 : (n > a.max_context_len ? a.max_context_len : n);
        const int tiles = (n + BS - 1) / BS;
        const int P = (tiles + PT - 1) / PT;
        const int nonlast = P > 0 ? P - 1 : 0;
        nparts[k] = P;
        last[k] = P > 0 ? tiles - nonlast * PT : 0;
        if (k * 64 >= a.num_seqs)
            continue;                            // no sequence in this chunk
        const int incl = wave_scan_incl(nonlast, lane);
        const int excl = incl - nonlast;
        const uint64_t m = __ballot(j >= F + excl && j < F + incl);
        if (u.s < 0 && m) {
            const int l = (int)__builtin_ctzll(m);
            u.s = k * 64 + l;
            u.part = j - F - __builtin_amdgcn_readlane(excl, l);
        }
        F += __builtin_amdgcn_readlane(incl, 63);
        L += (int)__popcll(__ballot(P > 0));
    }
    if (u.s >= 0 || j >= F + L)
        return u;

    // Position t of j along the path over positions F .. F+L-1: rounds of C
    // positions, forward in the first round (which starts at F) and
    // alternating after it; the last round may be partial.
    const int C = a.plan_width;
    const int E = F + L;
    const int r = j / C, c = j - r * C;
    const int lo = max(F, r * C) - r * C;
    const int hi = min(E, (r + 1) * C) - r * C - 1;
    const int t = (max(r * C, F) - F) + (((r - F / C) & 1) ? hi - c : c - lo);

    // The t-th largest last partition: the largest size b with more than t
    // last partitions of size >= b, then the right one among those of size b.
    auto count_ge = [&](int b) {
        int cnt = 0;
#pragma unroll
        for (int k = 0; k < kPlanChunks; ++k)
            cnt += (int)__popcll(__ballot(last[k] >= b));
        return cnt;
    };
    int blo = 1, bhi = PT;
    while (blo < bhi) {
        const int mid = (blo + bhi + 1) >> 1;
        if (count_ge(mid) > t)
            blo = mid;
        else
            bhi = mid - 1;
    }
    int rank = t - count_ge(blo + 1);
#pragma unroll
    for (int k = 0; k < kPlanChunks; ++k) {
        uint64_t m = __ballot(last[k] == blo);
        const int cnt = (int)__popcll(m);
        if (u.s < 0 && rank < cnt) {
            for (int i = 0; i < rank; ++i)
                m &= m - 1;                      // drop the lowest set lanes
            const int l = (int)__builtin_ctzll(m);
            u.s = k * 64 + l;
            u.part = __builtin_amdgcn_readlane(nparts[k], l) - 1;
        }
        rank -= cnt;
    }
    return u;
}

// The sequence that workgroup k of a K/V head takes in the whole-sequence
// form: the sequences ordered by tile count (largest first; ties: lower
// sequence first) and laid along a path that runs forward over the
// a.plan_width compute units one workgroup of the head is dealt to in turn,
// then backward in the next round, so that the compute unit that gets a long
// sequence's workgroup gets a short one's next.  num_seqs <= 64 * kPlanChunks.
// Workgroup k's unit in the pairing order: units (lanes' entries of `cost`,
// unit u = kk * 64 + lane, -1 past the count) ranked by cost, largest first,
// and dealt over C compute units forward in one round and backward in the
// next, so that a CU that got a large unit in one round gets a small one in
// the next.  `bound` is at least every cost.
__device__ int ranked_unit(const int (&cost)[kPlanChunks], int count, int bound, int C, int k)
{
    const int r = k / C, c = k - r * C;
    const int round_end = min(count, (r + 1) * C) - r * C;     // workgroups in this round
    const int t = r * C + ((r & 1) ? round_end - 1 - c : c);
    auto count_ge = [&](int b) {
        int cnt = 0;
#pragma unroll
        for (int kk = 0; kk < kPlanChunks; ++kk)
            if (kk * 64 < count)                 // only the chunks that hold units
                cnt += (int)__popcll(__ballot(cost[kk] >= b));
        return cnt;
    };
    // The t-th largest cost b, then the right unit among those of cost b.
    int blo = 0, bhi = bound;
    while (blo < bhi) {
        const int mid = (blo + bhi + 1) >> 1;
        if (count_ge(mid) > t)
            blo = mid;
        else
            bhi = mid - 1;
    }
    int rank = t - count_ge(blo + 1);
    int u = 0;
#pragma unroll
    for (int kk = 0; kk < kPlanChunks; ++kk) {
        if (kk * 64 >= count)
            break;
        uint64_t m = __ballot(cost[kk] == blo);
        const int cnt = (int)__popcll(m);
        if (rank >= 0 && rank < cnt) {
            for (int i = 0; i < rank; ++i)
                m &= m - 1;                      // drop the lowest set lanes
            u = kk * 64 + (int)__builtin_ctzll(m);
        }
        rank -= cnt;
    }
    return u;
}

// The sequence of whole-sequence workgroup k of a head: sequences ranked by
// tile count in the pairing order when they outnumber the head's compute
// units, else in their own order (one workgroup of the head per CU).
__device__ int seq_unit(const DecodeArgs &a, int k, int lane)
{
    const int S = a.num_seqs;
    const int C = a.plan_width;
    if (S <= C)
        return k;
    int tiles[kPlanChunks];
#pragma unroll
    for (int kk = 0; kk < kPlanChunks; ++kk) {
        const int s = kk * 64 + lane;
        tiles[kk] = a.context_lens[s < S ? s : S - 1];   // all loads issued before any is used
    }
#pragma unroll
    for (int kk = 0; kk < kPlanChunks; ++kk) {
        const int s = kk * 64 + lane;
        int n = tiles[kk];
        n = n < 0 ? 0 : (n > a.max_context_len ? a.max_context_len : n);
        tiles[kk] = s < S ? (n + BS - 1) / BS : -1;   // -1: no sequence
    }
    return ranked_unit(tiles, S, (a.max_context_len + BS - 1) / BS, C, k);
}

// APPEND: sequence s also brings a new token (k_new, v_new) for slot
// slot_mapping[s].  The workgroup holding the sequence's last partition writes
// the token's K/V of its head into the pools, and -- when that slot is the one
// the block table gives for position n-1 -- attends to the new values straight
// from registers, so no other workgroup and no earlier kernel is involved.
//
// Shared prefixes (a.shared_len != nullptr): the sequences at positions
// g*group_size .. g*group_size + group_size - 1 form group g (position p
// holds sequence group_order[p], or p without an order; an entry outside
// [0, num_seqs) leaves its position out), and the partitions lying wholly
// inside its first shared_len[g] tokens (clamped to every member's context)
// hold the same blocks for all members.  SHARED: one workgroup per (group,
// K/V head, such partition) attends for every member at once -- column r of
// the MFMAs is query head r % G of member r / G -- reading each tile once.
// The per-sequence pass skips those partitions (with APPEND it still writes a
// new token whose position lies in one, and attends nothing there).
//
// SPLIT wavefronts per workgroup (1 or 4): the partition's tiles are divided
// into SPLIT equal consecutive ranges, wavefront w attends to range w with
// its own running (max, sum, output), and the ranges' triples are merged in
// LDS, in range order, by the same log-sum-exp rule the merge kernel uses
// across partitions.  With 4 wavefronts one workgroup occupies one slot on
// each SIMD of its CU, so the CU's SIMDs share every partition's bytes
// equally.
//
// decode_unit is the work of one workgroup; `bid` is its index in its pass.
//
// SEQ (the whole-sequence form, SPLIT == kSeqWaves): the workgroup holds all
// of one (sequence, K/V head) and wavefront w attends to partition w, a whole
// 512-token partition of its own; the partitions' triples are merged in LDS
// exactly as the split ranges above are, and wavefront 0 writes out = acc / l
// (part_acc then holds the output, with one partition in its layout).
template <bool APPEND, bool SHARED, bool PLAN, int SPLIT, bool SEQ = false>
__device__ __forceinline__ void decode_unit(const DecodeArgs &a, unsigned bid)
{
    constexpr int kRing = SEQ ? kSeqRing : kRingFor<SPLIT>;
    const int lane = (int)(threadIdx.x & 63);
    const int wv = (int)(threadIdx.x >> 6);       // wavefront in the workgroup
    const int kvh = (int)(bid % (unsigned)a.num_kv_heads);
    const int rest = (int)(bid / (unsigned)a.num_kv_heads);
    const int units = SHARED ? a.num_groups : a.num_seqs;
    int part = rest / units;
    int s = rest % units;                      // SHARED: the group; the sequence below
    int ptiles = a.part_tiles;                 // tiles per unit
    if (SEQ) {
        // The sequence's tiles in kSeqWaves equal consecutive ranges, one per
        // wavefront (at most part_tiles each, as the launch requires
        // max_context_len <= kSeqWaves * partition_size).
        s = seq_unit(a, rest, lane);
        part = wv;
        int ns = a.context_lens[s];
        ns = ns < 0 ? 0 : (ns > a.max_context_len ? a.max_context_len : ns);
        ptiles = max(1, ((ns + BS - 1) / BS + kSeqWaves - 1) / kSeqWaves);
    }
    if (PLAN) {
        const Unit u = plan_unit(a, rest, lane);
        if (u.s < 0)
            return;
        s = u.s;
        part = u.part;
    }
    int members = 1;
    int n = 0;
    bool write_only = false;
    int first = 0;                             // SHARED: position of the group's first member
    auto seq_at = [&](int p) -> int { return a.group_order ? a.group_order[p] : p; };
    if (a.shared_len) {
        const int grp = SHARED ? s : s / a.group_size;   // s: the group, or a position
        first = grp * a.group_size;
        const int cnt = min(a.group_size, a.num_seqs - first);
        int sh = a.shared_len[grp];
        for (int m = 0; m < cnt; ++m) {
            const int sm = seq_at(first + m);
            int nm = sm >= 0 && sm < a.num_seqs ? a.context_lens[sm] : 0;   // left out: no sharing
            nm = nm < 0 ? 0 : (nm > a.max_context_len ? a.max_context_len : nm);
            sh = min(sh, nm);
        }
        const int shared_parts = sh > 0 ? sh / (a.part_tiles * BS) : 0;
        if (!SHARED) {
            s = seq_at(s);                     // the position's sequence
            if (s < 0 || s >= a.num_seqs)
                return;
        }
        if (SHARED) {
            if (part >= shared_parts)
                return;
            s = seq_at(first);
            members = cnt;
            n = shared_parts * a.part_tiles * BS;
        } else if (part < shared_parts) {
            if (!APPEND)
                return;                        // computed by the shared pass
            // The shared pass attends this partition; the unit is left only
            // the cache write of a new token at position n-1, if that lies
            // here (it does not when the precondition holds).
            int ns = a.context_lens[s];
            ns = ns < 0 ? 0 : (ns > a.max_context_len ? a.max_context_len : ns);
            const int p0 = part * a.part_tiles * BS;
            if (ns - 1 < p0 || ns - 1 >= p0 + a.part_tiles * BS)
                return;
            write_only = true;
        }
    }
    // The partition's table entries (partitions of up to 64 blocks) are
    // loaded together with the context length, before the length says how
    // many of them are used: entry l of the partition in lane l.  The row
    // holds them: part * part_tiles < max_blocks since max_context_len <=
    // max_blocks * block_size.
    const bool table_ahead = ptiles <= 64;
    const int64_t row0 = (int64_t)s * a.max_blocks + (int64_t)part * ptiles;
    const int32_t ahead_lane =
        table_ahead && lane < min(ptiles, a.max_blocks - part * ptiles)
            ? a.block_tables[row0 + lane]
            : 0;
    if (!SHARED) {
        n = a.context_lens[s];
        n = n < 0 ? 0 : (n > a.max_context_len ? a.max_context_len : n);
    }
    const int first_tok = part * ptiles * BS;
    if (!SEQ && first_tok >= n) {
        if (a.normalize && threadIdx.x < 64) {
            // An empty context with the only partition: its rows of the
            // output are 0 (the merge of no partition).  The plain order is
            // used here, so the unit knows its sequence.
            float4 *o0 = reinterpret_cast<float4 *>(
                a.part_acc + ((int64_t)s * a.num_kv_heads * a.group + (int64_t)kvh * a.group) * D);
            for (int e = lane; e < a.group * (D / 4); e += 64)
                o0[e] = make_float4(0.f, 0.f, 0.f, 0.f);
        }
        return;
    }
    // Tokens in this partition (SEQ: 0 for a wavefront past the sequence's end).
    const int ptok = max(0, min(n - first_tok, ptiles * BS));
    const int ntiles = (ptok + BS - 1) / BS;

    const int r = lane & 15;
    const int g = lane >> 4;
    const float c = a.scale_log2;
    const int G = a.group;

    // B operands of the score MFMAs: column r = query head kvh*G + r % G of
    // the group's member r / G in the shared pass (r < members * G), of
    // sequence s otherwise (r < G); rows = dims 8g..8g+7 (first MFMA) and
    // 32+8g..32+8g+7 (second).
    const bool col_ok = SHARED ? r < members * G : r < G;
    const int col_seq = SHARED ? (col_ok ? seq_at(first + r / G) : 0) : s;
    bf16x8 qb0 = {}, qb1 = {};
    if (col_ok) {
        const uint16_t *qp = a.q + ((int64_t)col_seq * a.num_kv_heads * G + (int64_t)kvh * G + r % G) * D + g * 8;
        qb0 = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(qp));
        qb1 = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(qp + 32));
    }

    // This wavefront's tiles of the partition: [t_lo, t_hi).
    int t_lo = 0, t_hi = ntiles;
    if (SPLIT > 1 && !SEQ) {
        const int per = (ntiles + SPLIT - 1) / SPLIT;
        t_lo = min(ntiles, wv * per);
        t_hi = min(ntiles, t_lo + per);
    }

    // Append: the wavefront holding position n-1 loads the new token's K/V row
    // of this head with its first loads, stages it in LDS once its first tile
    // loads are out, replaces position n-1 with the staged row when the slot
    // is that position's (the pool copy of that slot is never read back in
    // this launch), and writes the row into the pools after its loop.
    __shared__ uint16_t s_new_all[SPLIT][2 * D];   // per wavefront: K row then V row
    uint16_t *const s_new = s_new_all[wv];
    const bool append_here = APPEND && first_tok + ptok == n && t_lo < t_hi && t_hi == ntiles;
    int64_t wslot = -1;                   // slot to write (-1: none)
    int32_t tblk = -1;                    // table entry of position n-1
    uint32_t new_pair = 0;                // lane l: K dims 2l, 2l+1 (l < 32) or V dims 2(l-32), +1
    if (append_here) {
        wslot = a.slot_mapping[s];
        tblk = a.block_tables[(int64_t)s * a.max_blocks + (n - 1) / BS];
        new_pair = *reinterpret_cast<const uint32_t *>((lane < 32 ? a.k_new : a.v_new) +
                                                       ((int64_t)s * a.num_kv_heads + kvh) * D +
                                                       2 * (lane & 31));
    }
    int sub_off = -1;                     // token of the last tile replaced (-1: none)
    bool row_done = false;                // the new row went out with its whole tile

    // The cache write of the new token, this head, from the row staged in LDS.
    auto store_new_row = [&]() {
        const int64_t wblk = wslot / BS;
        const int woff = (int)(wslot - wblk * BS);
        uint16_t *kt = a.k_cache_w + (wblk * a.num_kv_heads + kvh) * (int64_t)(BS * D);
        uint16_t *vt = a.v_cache_w + (wblk * a.num_kv_heads + kvh) * (int64_t)(BS * D);
        if (lane < D / 8)                 // K: chunk `lane` (16 bytes)
            *reinterpret_cast<uint4 *>(kt + (lane * BS + woff) * 8) =
                *reinterpret_cast<const uint4 *>(s_new + 8 * lane);
        vt[lane * BS + woff] = s_new[D + lane];   // V: dimension `lane`
    };
    if (APPEND && write_only) {
        // The sequence's last partition lies in its group's shared prefix (a
        // broken precondition of the shared call): the shared pass has
        // attended it already; the new token is still written.
        if (append_here && wslot >= 0 && wslot < a.num_blocks * BS) {
            reinterpret_cast<uint32_t *>(s_new)[lane] = new_pair;
            __builtin_amdgcn_s_waitcnt(0xC07F);           // LDS stores done (lgkmcnt 0)
            __builtin_amdgcn_wave_barrier();
            store_new_row();
        }
        return;
    }

    float m_run = -INFINITY, l_run = 0.f;
    f32x4 o[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
        o[j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int32_t *bt = a.block_tables + (int64_t)s * a.max_blocks + (int64_t)part * ptiles + t_lo;
    const char *kpool = reinterpret_cast<const char *>(a.k_cache) + (int64_t)kvh * kTileBytes;
    const char *vpool = reinterpret_cast<const char *>(a.v_cache) + (int64_t)kvh * kTileBytes;
    const int64_t tile_stride = (int64_t)a.num_kv_heads * kTileBytes;
    const uint32_t koff = (uint32_t)lane * 16u;                   // this lane's K bytes in a tile
    const uint32_t voff = (uint32_t)(r * BS + g * 4) * 2u;        // this lane's V^T bytes (j = 0)

    auto issue = [&](Tile &t, int32_t b) {
        const int64_t bb = (b >= 0 && b < a.num_blocks) ? (int64_t)b : 0;
        load_tile(t, kpool + bb * tile_stride, vpool + bb * tile_stride, koff, voff);
    };
    auto consume = [&](const Tile &t, int tile, int32_t b) {
        if (b < 0 || b >= a.num_blocks)
            return;                                     // entry outside the pool: skipped
        if (APPEND && sub_off >= 0 && tile == ntiles - 1) {
            Tile u = t;                                 // position n-1 takes the new token
            if (r == sub_off) {
                u.k0 = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(s_new + 8 * g));
                u.k1 = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(s_new + 32 + 8 * g));
            }
            if (g == (sub_off >> 2)) {
#pragma unroll
                for (int j = 0; j < 4; ++j)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        if (i == (sub_off & 3))
                            u.v[j][i] = (short)s_new[D + 16 * j + r];
            }
            attend_tile<true>(u, qb0, qb1, ptok - tile * BS - 4 * g, c, m_run, l_run, o);
            // The cache write: the whole tile goes back with the new token in
            // place (every other position rewritten with the bits just read),
            // as coalesced 16- and 8-byte stores instead of the row's 8 chunk
            // and 64 column stores, none of which fills a 32-byte sector.
            char *kw = reinterpret_cast<char *>(a.k_cache_w) + (int64_t)b * tile_stride +
                       (int64_t)kvh * kTileBytes;
            char *vw = reinterpret_cast<char *>(a.v_cache_w) + (int64_t)b * tile_stride +
                       (int64_t)kvh * kTileBytes;
            *reinterpret_cast<u32x4 *>(kw + koff) = __builtin_bit_cast(u32x4, u.k0);
            *reinterpret_cast<u32x4 *>(kw + 1024 + koff) = __builtin_bit_cast(u32x4, u.k1);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                *reinterpret_cast<u32x2 *>(vw + voff + 512 * j) = __builtin_bit_cast(u32x2, u.v[j]);
            row_done = true;
            return;
        }
        if ((tile + 1) * BS <= ptok)
            attend_tile<false>(t, qb0, qb1, 4, c, m_run, l_run, o);
        else
            attend_tile<true>(t, qb0, qb1, ptok - tile * BS - 4 * g, c, m_run, l_run, o);
    };

    // Tiles are streamed through a ring of kRing register buffers: while tile k
    // is consumed, tiles k+1 .. k+kRing-1 are in flight.  Every steady-state
    // iteration issues the same loads, so each wait leaves exactly
    // (kRing-1) tiles outstanding.  Past the last tile the ring re-loads the
    // last tile (an L2 hit) instead of branching around the loads.
    const int nt = t_hi - t_lo;
    for (int c0 = 0; c0 < nt; c0 += 64) {
        const int cn = min(64, nt - c0);
        // One table entry per lane: the entries loaded ahead (then nt <= 64,
        // so c0 == 0 and the wavefront's tiles start at entry t_lo), or the
        // chunk's own.
        const int32_t phys_lane = table_ahead ? ahead_lane : (lane < cn ? bt[c0 + lane] : 0);
        const int first = table_ahead ? t_lo : 0;
        auto block_of = [&](int k) -> int32_t {
            return __builtin_amdgcn_readlane(phys_lane, first + min(k, cn - 1));
        };
        Tile ring[kRing];
#pragma unroll
        for (int u = 0; u < kRing; ++u)
            issue(ring[u], block_of(u));
        if (APPEND && c0 == 0 && append_here) {
            if (wslot >= 0 && wslot < a.num_blocks * BS) {
                reinterpret_cast<uint32_t *>(s_new)[lane] = new_pair;   // stage the row in LDS
                if ((int64_t)tblk * BS + (n - 1) % BS == wslot)
                    sub_off = (n - 1) % BS;
            } else {
                wslot = -1;
            }
            __builtin_amdgcn_s_waitcnt(0xC07F);           // LDS stores done (lgkmcnt 0)
            __builtin_amdgcn_wave_barrier();
        }
        const int nit = (cn + kRing - 1) / kRing;
        for (int it = 0; it + 1 < nit; ++it) {
#pragma unroll
            for (int u = 0; u < kRing; ++u) {
                const int k = it * kRing + u;
                consume(ring[u], t_lo + c0 + k, block_of(k));
                issue(ring[u], block_of(k + kRing));
            }
        }
#pragma unroll
        for (int u = 0; u < kRing; ++u) {
            const int k = (nit - 1) * kRing + u;
            if (k < cn)
                consume(ring[u], t_lo + c0 + k, block_of(k));
        }
    }

    if (APPEND && wslot >= 0 && !row_done)
        store_new_row();

    if (SPLIT > 1) {
        // Merge the wavefronts' (max, sum, output) per lane, in range order.
        // A wavefront with no usable token holds (-inf, 0, 0) and weighs 0.
        __shared__ float s_m[SPLIT][64], s_l[SPLIT][64];
        __shared__ f32x4 s_o[SPLIT][4][64];
        if (wv > 0) {
            s_m[wv][lane] = m_run;
            s_l[wv][lane] = l_run;
#pragma unroll
            for (int j = 0; j < 4; ++j)
                s_o[wv][j][lane] = o[j];
        }
        __syncthreads();
        if (wv > 0)
            return;
        float mm = m_run;
#pragma unroll
        for (int w = 1; w < SPLIT; ++w)
            mm = fmaxf(mm, s_m[w][lane]);
        if (mm != -INFINITY) {
            const float a0 = __builtin_amdgcn_exp2f(m_run - mm);
            l_run *= a0;
#pragma unroll
            for (int j = 0; j < 4; ++j)
                o[j] *= a0;
#pragma unroll
            for (int w = 1; w < SPLIT; ++w) {
                const float aw = __builtin_amdgcn_exp2f(s_m[w][lane] - mm);
                l_run = fmaf(s_l[w][lane], aw, l_run);
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    o[j] += s_o[w][j][lane] * aw;
            }
            m_run = mm;
        }
    }

    // Sum the lane groups' partial l (same query head, different tokens).
    l_run += __shfl_xor(l_run, 16);
    l_run += __shfl_xor(l_run, 32);

    if (col_ok) {
        const int hq = a.num_kv_heads * G;
        const int64_t row = ((int64_t)col_seq * hq + (int64_t)kvh * G + r % G) * a.num_parts + part;
        float *acc = a.part_acc + row * D + 4 * g;
        if (a.normalize) {
            // The only partition: merging it is dividing by its sum.
            const bool none = m_run == -INFINITY;
#pragma unroll
            for (int j = 0; j < 4; ++j)
                *reinterpret_cast<float4 *>(acc + 16 * j) =
                    none ? make_float4(0.f, 0.f, 0.f, 0.f)
                         : make_float4(o[j][0] / l_run, o[j][1] / l_run, o[j][2] / l_run,
                                       o[j][3] / l_run);
        } else {
            if (g == 0) {
                a.part_max[row] = m_run;
                a.part_sum[row] = l_run;
            }
#pragma unroll
            for (int j = 0; j < 4; ++j)
                *reinterpret_cast<float4 *>(acc + 16 * j) =
                    make_float4(o[j][0], o[j][1], o[j][2], o[j][3]);
        }
    }
}

template <bool APPEND, bool SHARED, bool PLAN, int SPLIT>
__global__ __launch_bounds__(64 * SPLIT)
__attribute__((amdgpu_waves_per_eu(SPLIT > 1 ? 4 : 3, SPLIT > 1 ? 4 : 8)))
void paged_decode_kernel(DecodeArgs a)
{
    decode_unit<APPEND, SHARED, PLAN, SPLIT>(a, blockIdx.x);
}

// The whole-sequence form: one workgroup of kSeqWaves wavefronts per
// (sequence, K/V head), two per compute unit.
template <bool APPEND>
__global__ __launch_bounds__(64 * kSeqWaves) __attribute__((amdgpu_waves_per_eu(4, 4)))
void paged_decode_seq_kernel(DecodeArgs a)
{
    decode_unit<APPEND, false, false, kSeqWaves, true>(a, blockIdx.x);
}

// The whole-group form of the shared-prefix decode step: one workgroup of
// kGroupWaves wavefronts per (group, K/V head), the cache write of every
// member's new token folded in and the log-sum-exp merge done in LDS, so
// the step is one launch with no workspace ("vLLM" page, section "가상 메모리
// 방식의 해결": the samples of one prompt share its blocks; section "Flash
// Attention": pieces of a softmax merge by the running maximum / sum rule).
//   * The group's shared tiles (its shared length cut to whole partitions, as
//     in the group pass) are read once, with every member's query heads as
//     MFMA columns (column r: member r / G, head r % G), and each member's
//     private tiles with the same columns, of which only the member's own are
//     kept.  The group's tiles -- the shared ones, then each member's own --
//     form one sequence, cut into kGroupWaves equal consecutive parts, one
//     per wavefront; a part may span several ranges, streamed back to back
//     through one ring.  Groups are dealt to compute units in the pairing
//     order (group_unit), so a CU's two workgroups carry a large and a
//     small group.
//   * A wavefront folds each range's tiles into one running state in
//     registers; at the end of a range that state is merged into the
//     wavefront's accumulated state, kept in LDS: for every column after the
//     shared range, for the member's own columns only after a member's range
//     (the other columns, the member's K/V against other members' queries,
//     are dropped).
//   * The wavefront holding a member's last tile writes that member's new
//     token, substituting it in registers and storing the whole tile back,
//     as the append pass does; a slot elsewhere gets its row alone at the end.
//   * The kGroupWaves states merge in LDS in wavefront order and the rows are
//     written to `out` (part_acc), divided by their sums.
//   * Member m of group g is the sequence at position g * group_size + m, or
//     group_order's entry for it; an entry outside the batch leaves that
//     member out (no length, so the group shares nothing; no row written),
//     as the group pass does.
constexpr int kGroupWaves = 8;
constexpr int kGroupRing = 2;
constexpr int kGroupMaxMembers = 4;

struct RunState {
    float m, l;
    f32x4 o[4];
};

__device__ __forceinline__ void state_init(RunState &st)
{
    st.m = -INFINITY;
    st.l = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j)
        st.o[j] = f32x4{0.f, 0.f, 0.f, 0.f};
}

// dst <- dst (+) src by the running maximum / sum rule; a state with
// m = -inf holds nothing and weighs 0.
__device__ __forceinline__ void state_merge(RunState &dst, const RunState &src)
{
    if (src.m == -INFINITY)
        return;
    const float mm = fmaxf(dst.m, src.m);
    const float ad = dst.m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(dst.m - mm);
    const float as = __builtin_amdgcn_exp2f(src.m - mm);
    dst.l = fmaf(src.l, as, dst.l * ad);
#pragma unroll
    for (int j = 0; j < 4; ++j)
        dst.o[j] = dst.o[j] * ad + src.o[j] * as;
    dst.m = mm;
}

// The group of whole-group workgroup k of a head: groups ranked by their
// tile count (shared tiles once plus every member's own) in the pairing
// order when they outnumber the head's compute units, else in their own
// order.
__device__ int group_unit(const DecodeArgs &a, int k, int lane)
{
    const int NG = a.num_groups;
    const int C = a.plan_width;
    if (NG <= C || NG > 64 * kPlanChunks)
        return k;
    int tiles[kPlanChunks];
#pragma unroll
    for (int kk = 0; kk < kPlanChunks; ++kk) {
        const int gi = kk * 64 + lane;
        tiles[kk] = -1;                          // -1: no group
        if (kk * 64 < NG) {
            // Every length and the shared length are loaded (clamped to the
            // batch) before any is used, so the lane waits on memory once.
            const int gc = gi < NG ? gi : NG - 1;
            const int f = gc * a.group_size;
            const int cnt = min(a.group_size, a.num_seqs - f);
            int sh = a.shared_len[gc];
            int nm[kGroupMaxMembers];
            if (a.group_order) {
                // Member m is sequence group_order[f + m]; an entry outside
                // the batch counts as an empty member.
                int sq[kGroupMaxMembers];
#pragma unroll
                for (int m = 0; m < kGroupMaxMembers; ++m)
                    sq[m] = a.group_order[min(f + m, a.num_seqs - 1)];
#pragma unroll
                for (int m = 0; m < kGroupMaxMembers; ++m) {
                    const bool ok = sq[m] >= 0 && sq[m] < a.num_seqs;
                    nm[m] = a.context_lens[ok ? sq[m] : 0];
                    nm[m] = ok ? nm[m] : 0;
                }
            } else {
#pragma unroll
                for (int m = 0; m < kGroupMaxMembers; ++m)
                    nm[m] = a.context_lens[min(f + m, a.num_seqs - 1)];
            }
            int sum = 0;
#pragma unroll
            for (int m = 0; m < kGroupMaxMembers; ++m) {
                // Selects, not a branch on m < cnt: a branch would let the
                // compiler sink each load into it and wait for each in turn.
                int n = nm[m];
                n = n < 0 ? 0 : (n > a.max_context_len ? a.max_context_len : n);
                sh = m < cnt ? min(sh, n) : sh;
                sum += m < cnt ? (n + BS - 1) / BS : 0;
            }
            const int st = sh > 0 ? (sh / (a.part_tiles * BS)) * a.part_tiles : 0;
            if (gi < NG)
                tiles[kk] = sum - (cnt - 1) * st;    // the shared tiles counted once
        }
    }
    const int bound = kGroupMaxMembers * ((a.max_context_len + BS - 1) / BS);
    return ranked_unit(tiles, NG, bound, C, k);
}

template <bool APPEND>
__global__ __launch_bounds__(64 * kGroupWaves) __attribute__((amdgpu_waves_per_eu(4, 4)))
void paged_decode_group_kernel(DecodeArgs a)
{
    const int lane = (int)(threadIdx.x & 63);
    const int wv = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int kvh = (int)(blockIdx.x % (unsigned)a.num_kv_heads);
    const int grp = group_unit(a, (int)(blockIdx.x / (unsigned)a.num_kv_heads), lane);
    const int first = grp * a.group_size;
    const int cnt = min(a.group_size, a.num_seqs - first);
    const int G = a.group;
    const int r = lane & 15;
    const int g = lane >> 4;
    const float c = a.scale_log2;

    // Lane m < cnt: member m's sequence (position first + m, through
    // group_order when given; -1 for an entry outside the batch, a member
    // left out: no length, no tiles, no row) and its context length
    // (clamped).  The shared length is cut to every member's context and to
    // whole partitions, so a left-out member leaves its group nothing shared.
    int seq_lane = -1;
    int n_lane = 0;
    if (lane < cnt) {
        const int sq = a.group_order ? a.group_order[first + lane] : first + lane;
        seq_lane = sq >= 0 && sq < a.num_seqs ? sq : -1;
        n_lane = seq_lane >= 0 ? a.context_lens[seq_lane] : 0;
        n_lane = n_lane < 0 ? 0 : (n_lane > a.max_context_len ? a.max_context_len : n_lane);
    }
    // The members' sequences as uniform values (scalar registers), picked per
    // lane by member index where a lane needs one.
    static_assert(kGroupMaxMembers == 4, "one scalar per member below");
    const int sq0 = __builtin_amdgcn_readlane(seq_lane, 0);
    const int sq1 = __builtin_amdgcn_readlane(seq_lane, 1);
    const int sq2 = __builtin_amdgcn_readlane(seq_lane, 2);
    const int sq3 = __builtin_amdgcn_readlane(seq_lane, 3);
    auto seq_of_member = [&](int m) {
        return m == 0 ? sq0 : (m == 1 ? sq1 : (m == 2 ? sq2 : sq3));
    };
    int sh = a.shared_len[grp];
    for (int m = 0; m < cnt; ++m)
        sh = min(sh, __builtin_amdgcn_readlane(n_lane, m));
    const int ST = sh > 0 ? (sh / (a.part_tiles * BS)) * a.part_tiles : 0;   // shared tiles

    // The group's tiles in one sequence: the shared tiles [0, ST), then member
    // 0's own tiles, member 1's, ...; g_end (lane m) is one past member m's
    // last place in it.  Wavefront wv takes places [v_lo, v_hi), an eighth.
    const int t_all = (n_lane + BS - 1) / BS;
    const int pt = lane < cnt ? max(0, t_all - ST) : 0;
    int g_end = pt;
#pragma unroll
    for (int d = 1; d < kGroupMaxMembers; d <<= 1) {
        const int y = __shfl_up(g_end, d);
        if (lane >= d)
            g_end += y;
    }
    g_end += ST;
    const int total = __builtin_amdgcn_readlane(g_end, cnt - 1);   // cnt >= 1
    const int v_lo = (int)((int64_t)wv * total / kGroupWaves);
    const int v_hi = (int)((int64_t)(wv + 1) * total / kGroupWaves);
    const int nv = v_hi - v_lo;

    // Columns: member r / G (r < cnt * G, the member not left out), query
    // head kvh * G + r % G.
    const int col_mem = r < cnt * G ? r / G : 0;
    const int col_seq = seq_of_member(col_mem);
    const bool col_ok = r < cnt * G && col_seq >= 0;
    bf16x8 qb0 = {}, qb1 = {};
    if (col_ok) {
        const uint16_t *qp =
            a.q + ((int64_t)col_seq * a.num_kv_heads * G + (int64_t)kvh * G + r % G) * D +
            g * 8;
        qb0 = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(qp));
        qb1 = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(qp + 32));
    }

    // Append: lane m < cnt -- does this wavefront hold member m's last tile
    // (position n_m - 1 past the shared tiles), its slot, and the table entry
    // of position n_m - 1.  The new rows of the members it holds are staged
    // in LDS after the first tile loads are out.
    __shared__ uint16_t s_new[kGroupWaves][kGroupMaxMembers][2 * D];
    const int last_t = (n_lane - 1) / BS;
    const bool hold_lane = APPEND && lane < cnt && n_lane > 0 && last_t >= ST &&
                           g_end - 1 >= v_lo && g_end - 1 < v_hi;   // its last place
    const uint64_t held = __ballot(hold_lane);
    int64_t wslot_lane = -1;
    int32_t tblk_lane = -1;
    if (hold_lane) {                      // n_lane > 0: a member in the batch
        wslot_lane = a.slot_mapping[seq_lane];
        tblk_lane = a.block_tables[(int64_t)seq_lane * a.max_blocks + last_t];
    }
    uint32_t new_pair[kGroupMaxMembers];
#pragma unroll
    for (int m = 0; m < kGroupMaxMembers; ++m) {
        new_pair[m] = 0;
        if (APPEND && ((held >> m) & 1ull))
            new_pair[m] = *reinterpret_cast<const uint32_t *>(
                (lane < 32 ? a.k_new : a.v_new) +
                ((int64_t)seq_of_member(m) * a.num_kv_heads + kvh) * D +
                2 * (lane & 31));
    }
    int sub_lane = -1;        // lane m: token of member m's last tile replaced (-1: none)
    bool done_lane = false;   // lane m: member m's row went out with its tile

    const char *kpool = reinterpret_cast<const char *>(a.k_cache) + (int64_t)kvh * kTileBytes;
    const char *vpool = reinterpret_cast<const char *>(a.v_cache) + (int64_t)kvh * kTileBytes;
    const int64_t tile_stride = (int64_t)a.num_kv_heads * kTileBytes;
    const uint32_t koff = (uint32_t)lane * 16u;
    const uint32_t voff = (uint32_t)(r * BS + g * 4) * 2u;
    auto issue = [&](Tile &t, int32_t b) {
        const int64_t bb = (b >= 0 && b < a.num_blocks) ? (int64_t)b : 0;
        load_tile(t, kpool + bb * tile_stride, vpool + bb * tile_stride, koff, voff);
    };

    // The wavefront's accumulated state, in LDS (also the final merge's input).
    __shared__ float s_m[kGroupWaves][64], s_l[kGroupWaves][64];
    __shared__ f32x4 s_o[kGroupWaves][4][64];
    s_m[wv][lane] = -INFINITY;
    s_l[wv][lane] = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j)
        s_o[wv][j][lane] = f32x4{0.f, 0.f, 0.f, 0.f};
    auto fold_into_lds = [&](const RunState &R) {
        RunState A;
        A.m = s_m[wv][lane];
        A.l = s_l[wv][lane];
#pragma unroll
        for (int j = 0; j < 4; ++j)
            A.o[j] = s_o[wv][j][lane];
        state_merge(A, R);
        s_m[wv][lane] = A.m;
        s_l[wv][lane] = A.l;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            s_o[wv][j][lane] = A.o[j];
    };

    RunState R;               // the range being folded
    state_init(R);
    int cur = -1;             // the range being folded: -1 shared, m >= 0 member m
    int cur_end = min(max(ST - v_lo, 0), nv);   // its end, local place
    int cur_tile0 = v_lo;     // tile index of local place 0 in this range
    int cur_n = ST * BS;      // tokens of the range's sequence (masking)
    // Close the ranges that end at or before virtual index k: fold R into the
    // accumulated state (every column after the shared range, the member's
    // own after a member's) and step to the next range.
    auto advance_to = [&](int k) {
        while (k >= cur_end && cur + 1 < cnt) {
            if (cur < 0 || (col_ok && col_mem == cur))
                fold_into_lds(R);
            state_init(R);
            ++cur;
            const int ge = __builtin_amdgcn_readlane(g_end, cur);
            const int gb = ge - __builtin_amdgcn_readlane(pt, cur);
            cur_end = min(max(ge - v_lo, 0), nv);
            cur_tile0 = v_lo - gb + ST;
            cur_n = __builtin_amdgcn_readlane(n_lane, cur);
        }
    };

    auto consume = [&](const Tile &t, int k, int32_t b) {
        advance_to(k);
        if (b < 0 || b >= a.num_blocks)
            return;                                     // entry outside the pool: skipped
        const int tile = cur_tile0 + k;
        const int valid = cur_n - tile * BS - 4 * g;
        const bool partial = (tile + 1) * BS > cur_n;
        const int so = APPEND && cur >= 0 ? __builtin_amdgcn_readlane(sub_lane, cur) : -1;
        const bool sub = APPEND && so >= 0 && tile == (cur_n - 1) / BS;
        if (!sub && !partial) {
            attend_tile<false>(t, qb0, qb1, 4, c, R.m, R.l, R.o);
            return;
        }
        Tile u = t;
        if (sub) {                                      // position n-1 takes the new token
            const uint16_t *sn = s_new[wv][cur];
            if (r == so) {
                u.k0 = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(sn + 8 * g));
                u.k1 = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(sn + 32 + 8 * g));
            }
            if (g == (so >> 2)) {
#pragma unroll
                for (int j = 0; j < 4; ++j)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        if (i == (so & 3))
                            u.v[j][i] = (short)sn[D + 16 * j + r];
            }
        }
        attend_tile<true>(u, qb0, qb1, valid, c, R.m, R.l, R.o);
        if (sub) {
            char *kw = reinterpret_cast<char *>(a.k_cache_w) + (int64_t)b * tile_stride +
                       (int64_t)kvh * kTileBytes;
            char *vw = reinterpret_cast<char *>(a.v_cache_w) + (int64_t)b * tile_stride +
                       (int64_t)kvh * kTileBytes;
            *reinterpret_cast<u32x4 *>(kw + koff) = __builtin_bit_cast(u32x4, u.k0);
            *reinterpret_cast<u32x4 *>(kw + 1024 + koff) = __builtin_bit_cast(u32x4, u.k1);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                *reinterpret_cast<u32x2 *>(vw + voff + 512 * j) = __builtin_bit_cast(u32x2, u.v[j]);
            done_lane = done_lane || lane == cur;
        }
    };

    for (int c0 = 0; c0 < nv; c0 += 64) {
        const int cn = min(64, nv - c0);
        // Lane l: the table entry of virtual tile c0 + l.
        int32_t phys_lane = 0;
        {
            const int gp = v_lo + c0 + lane;           // this lane's place in the sequence
            int mem = 0;                               // member m: places [g_end(m-1), g_end(m))
            for (int m = 0; m + 1 < cnt; ++m)
                if (gp >= __builtin_amdgcn_readlane(g_end, m))
                    mem = m + 1;
            // Shuffles with every lane active: a lane outside exec would not
            // deliver its value.
            const int ge = __shfl(g_end, mem);
            const int gb = ge - __shfl(pt, mem);
            const bool in_shared = gp < ST;
            const int seq = seq_of_member(in_shared ? 0 : mem);   // >= 0 wherever a tile lies
            const int tix = in_shared ? gp : ST + (gp - gb);
            if (lane < cn)
                phys_lane = a.block_tables[(int64_t)seq * a.max_blocks + tix];
        }
        auto block_of = [&](int k) -> int32_t {
            return __builtin_amdgcn_readlane(phys_lane, min(k, cn - 1));
        };
        Tile ring[kGroupRing];
#pragma unroll
        for (int u = 0; u < kGroupRing; ++u)
            issue(ring[u], block_of(u));
        if (APPEND && c0 == 0 && held) {
            // Stage the held members' rows; note which last tiles take them.
#pragma unroll
            for (int m = 0; m < kGroupMaxMembers; ++m)
                if ((held >> m) & 1ull)
                    reinterpret_cast<uint32_t *>(s_new[wv][m])[lane] = new_pair[m];
            if (hold_lane) {
                if (wslot_lane >= 0 && wslot_lane < a.num_blocks * BS) {
                    if ((int64_t)tblk_lane * BS + (n_lane - 1) % BS == wslot_lane)
                        sub_lane = (n_lane - 1) % BS;
                } else {
                    wslot_lane = -1;
                }
            }
            __builtin_amdgcn_s_waitcnt(0xC07F);           // LDS stores done (lgkmcnt 0)
            __builtin_amdgcn_wave_barrier();
        }
        const int nit = (cn + kGroupRing - 1) / kGroupRing;
        for (int it = 0; it + 1 < nit; ++it) {
#pragma unroll
            for (int u = 0; u < kGroupRing; ++u) {
                const int k = it * kGroupRing + u;
                consume(ring[u], c0 + k, block_of(k));
                issue(ring[u], block_of(k + kGroupRing));
            }
        }
#pragma unroll
        for (int u = 0; u < kGroupRing; ++u) {
            const int k = (nit - 1) * kGroupRing + u;
            if (k < cn)
                consume(ring[u], c0 + k, block_of(k));
        }
    }
    // Close the ranges that remain (the last member's, and empty ones).
    advance_to(INT32_MAX);
    if (cur < 0 || (col_ok && col_mem == cur))
        fold_into_lds(R);

    // Rows whose slot is not position n-1's: the row alone.
    if (APPEND && held) {
#pragma unroll
        for (int m = 0; m < kGroupMaxMembers; ++m) {
            if (!((held >> m) & 1ull))
                continue;
            const int64_t ws =
                (int64_t)(((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(wslot_lane >> 32), m)
                           << 32) |
                          (uint32_t)__builtin_amdgcn_readlane((int)wslot_lane, m));
            const bool dn = __builtin_amdgcn_readlane((int)done_lane, m) != 0;
            if (ws < 0 || dn)
                continue;
            const int64_t wblk = ws / BS;
            const int woff = (int)(ws - wblk * BS);
            uint16_t *kt = a.k_cache_w + (wblk * a.num_kv_heads + kvh) * (int64_t)(BS * D);
            uint16_t *vt = a.v_cache_w + (wblk * a.num_kv_heads + kvh) * (int64_t)(BS * D);
            const uint16_t *sn = s_new[wv][m];
            if (lane < D / 8)
                *reinterpret_cast<uint4 *>(kt + (lane * BS + woff) * 8) =
                    *reinterpret_cast<const uint4 *>(sn + 8 * lane);
            vt[lane * BS + woff] = sn[D + lane];
        }
    }

    // Merge the wavefronts' states in wavefront order and write the rows.
    __syncthreads();
    if (APPEND && wv == 0) {
        // A member whose position n-1 lies in the shared tiles (a broken
        // precondition): its token is still written, after every wavefront
        // has read the shared tiles.
        for (int m = 0; m < cnt; ++m) {
            const int nm = __builtin_amdgcn_readlane(n_lane, m);
            if (nm <= 0 || (nm - 1) / BS >= ST)
                continue;
            const int sm = seq_of_member(m);                         // nm > 0: in the batch
            const int64_t ws = a.slot_mapping[sm];
            if (ws < 0 || ws >= a.num_blocks * BS)
                continue;
            const int64_t wblk = ws / BS;
            const int woff = (int)(ws - wblk * BS);
            uint16_t *kt = a.k_cache_w + (wblk * a.num_kv_heads + kvh) * (int64_t)(BS * D);
            uint16_t *vt = a.v_cache_w + (wblk * a.num_kv_heads + kvh) * (int64_t)(BS * D);
            const uint16_t *kn = a.k_new + ((int64_t)sm * a.num_kv_heads + kvh) * D;
            const uint16_t *vn = a.v_new + ((int64_t)sm * a.num_kv_heads + kvh) * D;
            if (lane < D / 8)
                *reinterpret_cast<uint4 *>(kt + (lane * BS + woff) * 8) =
                    *reinterpret_cast<const uint4 *>(kn + 8 * lane);
            vt[lane * BS + woff] = vn[lane];
        }
    }
    if (wv > 0)
        return;
    RunState S;
    state_init(S);
#pragma unroll
    for (int w = 0; w < kGroupWaves; ++w) {
        RunState o;
        o.m = s_m[w][lane];
        o.l = s_l[w][lane];
#pragma unroll
        for (int j = 0; j < 4; ++j)
            o.o[j] = s_o[w][j][lane];
        state_merge(S, o);
    }
    float l = S.l;
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    if (col_ok) {
        const int hq = a.num_kv_heads * G;
        const int64_t row = (int64_t)seq_of_member(col_mem) * hq + (int64_t)kvh * G + r % G;
        float *acc = a.part_acc + row * D + 4 * g;
        const bool none = S.m == -INFINITY;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            *reinterpret_cast<float4 *>(acc + 16 * j) =
                none ? make_float4(0.f, 0.f, 0.f, 0.f)
                     : make_float4(S.o[j][0] / l, S.o[j][1] / l, S.o[j][2] / l, S.o[j][3] / l);
    }
}

// A shared-prefix launch in one grid: workgroups [0, shared_groups) take the
// group pass, the rest the per-sequence pass.  The two passes read disjoint
// partitions and write disjoint partials, so one grid lets each fill the
// other's tail.  shared_groups is a multiple of the K/V head count, so every
// workgroup keeps its head's XCD.
template <bool APPEND, int SPLIT, bool PLAN>
__global__ __launch_bounds__(64 * SPLIT)
__attribute__((amdgpu_waves_per_eu(SPLIT > 1 ? 4 : 3, SPLIT > 1 ? 4 : 8)))
void paged_decode_shared_kernel(DecodeArgs a, unsigned shared_groups)
{
    if (blockIdx.x < shared_groups)
        decode_unit<false, true, false, SPLIT>(a, blockIdx.x);
    else
        decode_unit<APPEND, false, PLAN, SPLIT>(a, blockIdx.x - shared_groups);
}

// What the launcher needs to know of the device: its compute units and how
// many one-wavefront decode workgroups each holds at once (cached per device;
// zeros if unknown).
struct DeviceShape {
    int cus;
    int waves_per_cu;
};

DeviceShape device_shape()
{
    static std::atomic<int> cus_cache[64], waves_cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0)
        return {0, 0};
    if (dev < 64) {
        const int c = cus_cache[dev].load(std::memory_order_relaxed);
        const int w = waves_cache[dev].load(std::memory_order_relaxed);
        if (c > 0 && w > 0)
            return {c, w};
    }
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &per_cu, reinterpret_cast<const void *>(paged_decode_kernel<false, false, false, 1>), 64,
            0) != hipSuccess)
        return {0, 0};
    if (dev < 64) {
        cus_cache[dev].store(cus, std::memory_order_relaxed);
        waves_cache[dev].store(per_cu, std::memory_order_relaxed);
    }
    return {cus, per_cu};
}

// Workgroups of the whole-sequence kernel one compute unit holds at once
// (cached per device; 0 if unknown).
int seq_wgs_per_cu()
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
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &per_cu, reinterpret_cast<const void *>(paged_decode_seq_kernel<true>), 64 * kSeqWaves,
            0) != hipSuccess)
        return 0;
    if (dev < 64)
        cache[dev].store(per_cu, std::memory_order_relaxed);
    return per_cu;
}

// Workgroups of the whole-group kernel one compute unit holds at once
// (cached per device; 0 if unknown).
int group_wgs_per_cu()
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
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &per_cu, reinterpret_cast<const void *>(paged_decode_group_kernel<true>),
            64 * kGroupWaves, 0) != hipSuccess)
        return 0;
    if (dev < 64)
        cache[dev].store(per_cu, std::memory_order_relaxed);
    return per_cu;
}

// The vector-ALU form of the partition pass (tv_paged_attention_decode_vector):
// the same grid, partition split, table handling, tile ring, merge of the 4
// wavefronts and epilogue as paged_decode_kernel<false, false, PLAN, 4>, with
// the QK and PV contractions done by the vector ALUs instead of MFMA, for a
// group of 4 query heads per K/V head.  It is the measured alternative to the
// matrix form: on MI355X it is slower on every workload measured (per
// 16-token tile the MFMA form's compiled step is 10 matrix and about 75
// vector instructions, this one's about 300 vector instructions).
//   * K arrives as in the matrix form: lane (r = lane % 16, g = lane / 16)
//     holds token r's dims 8g..8g+7 and 32+8g..32+8g+7.  Each lane takes its
//     16-dim part of token r's score for each of the 4 heads (8
//     v_dot2_f32_bf16 per head), and the 4 lane rows' parts are summed with
//     v_permlane16_swap / v_permlane32_swap, in the same order in every row,
//     so all 4 lanes of column r hold token r's 4 scores.
//   * The tile maximum per head is a DPP butterfly within a 16-lane row.
//   * V arrives as one 32-byte row per lane: lane d holds V[dim d][tokens
//     0..15], so the output O[h][d] of all 4 heads stays in lane d; the 64
//     weights go to scalar registers (v_readlane) and PV is 64 FMAs per lane.
//   * At the end of its range a wavefront passes its (max, sum, output)
//     through LDS into the matrix form's lane layout (lane (r, g), r < 4:
//     head r, dims 16j + 4g + i), and the matrix form's merge and stores
//     follow unchanged.
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
constexpr int kVecGroup = 4;

struct VecTile {
    bf16x8 k0, k1;
    u32x4 va, vb;        // V[dim lane][tokens 0..7], [tokens 8..15]
};

__device__ __forceinline__ void load_vec_tile(VecTile &t, const char *kt, const char *vt,
                                              uint32_t koff, uint32_t vdoff)
{
    t.k0 = __builtin_bit_cast(bf16x8, __builtin_nontemporal_load(
                                          reinterpret_cast<const u32x4 *>(kt + koff)));
    t.k1 = __builtin_bit_cast(bf16x8, __builtin_nontemporal_load(
                                          reinterpret_cast<const u32x4 *>(kt + 1024 + koff)));
    t.va = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(vt + vdoff));
    t.vb = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(vt + vdoff + 16));
}

template <int CTRL>
__device__ __forceinline__ float dpp_move(float x)
{
    return __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

// Maximum / sum over the 16 lanes of each row, in every lane of the row:
// quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_half_mirror, row_mirror.
__device__ __forceinline__ float row_max16(float x)
{
    x = fmaxf(x, dpp_move<0xB1>(x));
    x = fmaxf(x, dpp_move<0x4E>(x));
    x = fmaxf(x, dpp_move<0x141>(x));
    return fmaxf(x, dpp_move<0x140>(x));
}
__device__ __forceinline__ float row_sum16(float x)
{
    x = x + dpp_move<0xB1>(x);
    x = x + dpp_move<0x4E>(x);
    x = x + dpp_move<0x141>(x);
    return x + dpp_move<0x140>(x);
}

// Sum over lanes l, l ^ 16, l ^ 32, l ^ 48 as (x[row 0] + x[row 1]) +
// (x[row 2] + x[row 3]) for the lane's column, in every row.
__device__ __forceinline__ float sum_over_rows(float x)
{
    const unsigned u = __builtin_bit_cast(unsigned, x);
    const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    const unsigned a0 = a[0], a1 = a[1];
    const float y = __builtin_bit_cast(float, a0) + __builtin_bit_cast(float, a1);
    const unsigned w = __builtin_bit_cast(unsigned, y);
    const auto b = __builtin_amdgcn_permlane32_swap(w, w, false, false);
    const unsigned b0 = b[0], b1 = b[1];
    return __builtin_bit_cast(float, b0) + __builtin_bit_cast(float, b1);
}

// Fold one tile into the running state: m[h] (base-2 units, the same in every
// lane), l[h] (this lane's column's weights; every row holds the same), o[h]
// = O[h][dim lane].  `valid`: tokens of the tile inside the context (MASK only).
template <bool MASK>
__device__ __forceinline__ void attend_vec_tile(const VecTile &t, const bf16x8 (&qa)[kVecGroup],
                                                const bf16x8 (&qb)[kVecGroup], int valid, float c,
                                                int r, float (&m)[kVecGroup],
                                                float (&l)[kVecGroup], float (&o)[kVecGroup])
{
#pragma clang fp contract(off)
    float s2[kVecGroup];
#pragma unroll
    for (int h = 0; h < kVecGroup; ++h) {
        float acc = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const bf16x2 kk = {t.k0[2 * i], t.k0[2 * i + 1]};
            const bf16x2 qq = {qa[h][2 * i], qa[h][2 * i + 1]};
            acc = __builtin_amdgcn_fdot2_f32_bf16(kk, qq, acc, false);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const bf16x2 kk = {t.k1[2 * i], t.k1[2 * i + 1]};
            const bf16x2 qq = {qb[h][2 * i], qb[h][2 * i + 1]};
            acc = __builtin_amdgcn_fdot2_f32_bf16(kk, qq, acc, false);
        }
        s2[h] = sum_over_rows(acc) * c;           // base-2 units, rounded once
        if (MASK && r >= valid)
            s2[h] = -INFINITY;
    }
    float p[kVecGroup];
#pragma unroll
    for (int h = 0; h < kVecGroup; ++h) {
        const float m_new = fmaxf(m[h], row_max16(s2[h]));
        const float alpha = __builtin_amdgcn_exp2f(m[h] - m_new);
        p[h] = __builtin_amdgcn_exp2f(s2[h] - m_new);
        m[h] = m_new;
        l[h] = fmaf(l[h], alpha, p[h]);
        o[h] *= alpha;
    }
    // V[dim lane][t] as fp32; tokens past the context forced to 0, since stale
    // slots may hold NaN and 0 * NaN is NaN.
    float v[16];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        v[2 * w] = __builtin_bit_cast(float, t.va[w] << 16);
        v[2 * w + 1] = __builtin_bit_cast(float, t.va[w] & 0xFFFF0000u);
        v[8 + 2 * w] = __builtin_bit_cast(float, t.vb[w] << 16);
        v[9 + 2 * w] = __builtin_bit_cast(float, t.vb[w] & 0xFFFF0000u);
    }
    if (MASK) {
#pragma unroll
        for (int i = 0; i < 16; ++i)
            if (i >= valid)
                v[i] = 0.f;
    }
#pragma unroll
    for (int h = 0; h < kVecGroup; ++h) {
        const int pb = __builtin_bit_cast(int, p[h]);
#pragma unroll
        for (int i = 0; i < 16; ++i)
            o[h] = fmaf(__builtin_bit_cast(float, __builtin_amdgcn_readlane(pb, i)), v[i], o[h]);
    }
}

template <bool PLAN>
__device__ __forceinline__ void decode_unit_vec(const DecodeArgs &a, unsigned bid)
{
    constexpr int SPLIT = 4;
    constexpr int kRing = kRingFor<SPLIT>;
    const int lane = (int)(threadIdx.x & 63);
    const int wv = (int)(threadIdx.x >> 6);
    const int kvh = (int)(bid % (unsigned)a.num_kv_heads);
    const int rest = (int)(bid / (unsigned)a.num_kv_heads);
    int part = rest / a.num_seqs;
    int s = rest % a.num_seqs;
    const int ptiles = a.part_tiles;
    if (PLAN) {
        const Unit u = plan_unit(a, rest, lane);
        if (u.s < 0)
            return;
        s = u.s;
        part = u.part;
    }
    // Table entries loaded with the context length, as in the matrix form.
    const int64_t row0 = (int64_t)s * a.max_blocks + (int64_t)part * ptiles;
    const bool table_ahead = ptiles <= 64;
    const int32_t ahead_lane = table_ahead && lane < min(ptiles, a.max_blocks - part * ptiles)
                                   ? a.block_tables[row0 + lane]
                                   : 0;
    int n = a.context_lens[s];
    n = n < 0 ? 0 : (n > a.max_context_len ? a.max_context_len : n);
    const int first_tok = part * ptiles * BS;
    if (first_tok >= n)
        return;
    const int ptok = min(n - first_tok, ptiles * BS);
    const int ntiles = (ptok + BS - 1) / BS;
    const int r = lane & 15;
    const int g = lane >> 4;
    const float c = a.scale_log2;

    // q of the group's 4 heads: lane (r, g) holds dims 8g..8g+7 (qa) and
    // 32+8g..32+8g+7 (qb).
    bf16x8 qa[kVecGroup], qb[kVecGroup];
#pragma unroll
    for (int h = 0; h < kVecGroup; ++h) {
        const uint16_t *qp =
            a.q + ((int64_t)s * a.num_kv_heads * kVecGroup + (int64_t)kvh * kVecGroup + h) * D + g * 8;
        qa[h] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(qp));
        qb[h] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(qp + 32));
    }
    const int per = (ntiles + SPLIT - 1) / SPLIT;
    const int t_lo = min(ntiles, wv * per);
    const int t_hi = min(ntiles, t_lo + per);

    float m[kVecGroup], l[kVecGroup], o[kVecGroup];
#pragma unroll
    for (int h = 0; h < kVecGroup; ++h) {
        m[h] = -INFINITY;
        l[h] = 0.f;
        o[h] = 0.f;
    }
    const int32_t *bt = a.block_tables + row0 + t_lo;
    const char *kpool = reinterpret_cast<const char *>(a.k_cache) + (int64_t)kvh * kTileBytes;
    const char *vpool = reinterpret_cast<const char *>(a.v_cache) + (int64_t)kvh * kTileBytes;
    const int64_t tile_stride = (int64_t)a.num_kv_heads * kTileBytes;
    const uint32_t koff = (uint32_t)lane * 16u;
    const uint32_t vdoff = (uint32_t)lane * 32u;
    auto issue = [&](VecTile &t, int32_t b) {
        const int64_t bb = (b >= 0 && b < a.num_blocks) ? (int64_t)b : 0;
        load_vec_tile(t, kpool + bb * tile_stride, vpool + bb * tile_stride, koff, vdoff);
    };
    auto consume = [&](const VecTile &t, int tile, int32_t b) {
        if (b < 0 || b >= a.num_blocks)
            return;                                   // entry outside the pool: skipped
        if ((tile + 1) * BS <= ptok)
            attend_vec_tile<false>(t, qa, qb, BS, c, r, m, l, o);
        else
            attend_vec_tile<true>(t, qa, qb, ptok - tile * BS, c, r, m, l, o);
    };
    // The ring as in the matrix form.
    const int nt = t_hi - t_lo;
    for (int c0 = 0; c0 < nt; c0 += 64) {
        const int cn = min(64, nt - c0);
        const int32_t phys_lane = table_ahead ? ahead_lane : (lane < cn ? bt[c0 + lane] : 0);
        const int first = table_ahead ? t_lo : 0;
        auto block_of = [&](int k) -> int32_t {
            return __builtin_amdgcn_readlane(phys_lane, first + min(k, cn - 1));
        };
        VecTile ring[kRing];
#pragma unroll
        for (int u = 0; u < kRing; ++u)
            issue(ring[u], block_of(u));
        const int nit = (cn + kRing - 1) / kRing;
        for (int it = 0; it + 1 < nit; ++it) {
#pragma unroll
            for (int u = 0; u < kRing; ++u) {
                const int k = it * kRing + u;
                consume(ring[u], t_lo + c0 + k, block_of(k));
                issue(ring[u], block_of(k + kRing));
            }
        }
#pragma unroll
        for (int u = 0; u < kRing; ++u) {
            const int k = (nit - 1) * kRing + u;
            if (k < cn)
                consume(ring[u], t_lo + c0 + k, block_of(k));
        }
    }

    // Into the matrix form's layout: lane (r, g), r < 4, holds head r's max,
    // dims 16j + 4g .. 16j + 4g + 3, and (in its g = 0 lane) its sum.
    __shared__ __attribute__((aligned(16))) float s_vo[SPLIT][kVecGroup][64];
#pragma unroll
    for (int h = 0; h < kVecGroup; ++h)
        s_vo[wv][h][lane] = o[h];
    float lt[kVecGroup];
#pragma unroll
    for (int h = 0; h < kVecGroup; ++h)
        lt[h] = row_sum16(l[h]);
    __builtin_amdgcn_s_waitcnt(0xC07F);               // LDS stores done (lgkmcnt 0)
    __builtin_amdgcn_wave_barrier();
    const bool head_lane = r < kVecGroup;
    const int hr = head_lane ? r : 0;
    const float m_h = hr == 0 ? m[0] : (hr == 1 ? m[1] : (hr == 2 ? m[2] : m[3]));
    const float l_h = hr == 0 ? lt[0] : (hr == 1 ? lt[1] : (hr == 2 ? lt[2] : lt[3]));
    float m_run = head_lane ? m_h : -INFINITY;
    float l_run = head_lane && g == 0 && m_run != -INFINITY ? l_h : 0.f;
    f32x4 oo[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const f32x4 x = *reinterpret_cast<const f32x4 *>(&s_vo[wv][hr][16 * j + 4 * g]);
        oo[j] = head_lane ? x : f32x4{0.f, 0.f, 0.f, 0.f};
    }

    // Merge the 4 wavefronts in range order and store, as the matrix form does.
    __shared__ float s_m[SPLIT][64], s_l[SPLIT][64];
    __shared__ f32x4 s_o[SPLIT][4][64];
    if (wv > 0) {
        s_m[wv][lane] = m_run;
        s_l[wv][lane] = l_run;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            s_o[wv][j][lane] = oo[j];
    }
    __syncthreads();
    if (wv > 0)
        return;
    float mm = m_run;
#pragma unroll
    for (int w = 1; w < SPLIT; ++w)
        mm = fmaxf(mm, s_m[w][lane]);
    if (mm != -INFINITY) {
        const float a0 = __builtin_amdgcn_exp2f(m_run - mm);
        l_run *= a0;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            oo[j] *= a0;
#pragma unroll
        for (int w = 1; w < SPLIT; ++w) {
            const float aw = __builtin_amdgcn_exp2f(s_m[w][lane] - mm);
            l_run = fmaf(s_l[w][lane], aw, l_run);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                oo[j] += s_o[w][j][lane] * aw;
        }
        m_run = mm;
    }
    l_run += __shfl_xor(l_run, 16);
    l_run += __shfl_xor(l_run, 32);
    if (head_lane) {
        const int64_t row =
            ((int64_t)s * a.num_kv_heads * kVecGroup + (int64_t)kvh * kVecGroup + r) * a.num_parts + part;
        float *acc = a.part_acc + row * D + 4 * g;
        if (g == 0) {
            a.part_max[row] = m_run;
            a.part_sum[row] = l_run;
        }
#pragma unroll
        for (int j = 0; j < 4; ++j)
            *reinterpret_cast<float4 *>(acc + 16 * j) =
                make_float4(oo[j][0], oo[j][1], oo[j][2], oo[j][3]);
    }
}

template <bool PLAN>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4, 4)))
void paged_decode_vec_kernel(DecodeArgs a)
{
    decode_unit_vec<PLAN>(a, blockIdx.x);
}

template <bool APPEND, bool SHARED, bool PLAN, int SPLIT>
void launch(const DecodeArgs &a, int64_t groups, hipStream_t stream)
{
    hipLaunchKernelGGL((paged_decode_kernel<APPEND, SHARED, PLAN, SPLIT>), dim3((unsigned)groups),
                       dim3(64 * SPLIT), 0, stream, a);
}

}  // namespace

// Launch policy, from the grid G of one-wavefront workgroups per (sequence,
// head, partition) that the host bounds give and the number R of them the
// device holds at once:
//   * G <= 2R: 4 wavefronts per partition.  The launch then has many small
//     workgroups, the hardware hands them out as slots free up, and each
//     CU's 4 SIMDs share every partition's bytes, so no SIMD is left with
//     more tiles than the others at the end (measured on batch 64 x
//     512-4096 tokens: 53.6 against 56.6 us), and small batches get 4x the
//     wavefronts;
//   * G > 2R (few very long sequences, or many sequences with room for long
//     ones): one wavefront per partition;
//   * G > R and at most 256 sequences (no shared prefixes): the balanced
//     order of plan_unit, which moves the grid's empty partitions behind the
//     work (batch 4 x 32k-128k tokens: 110.8 against 121.9 us; batch 64 x
//     512-4096 with 4 wavefronts: 53.6 against 54.8 us).  Below R the order's
//     prologue is not hidden behind other workgroups' loads (batch 8: 9.3
//     against 8.2 us), so small grids keep the plain order.
// The shared-prefix launch takes the split its per-sequence grid would get,
// so its partitions round exactly as the per-sequence pass's do.
// The whole-sequence form serves a step whose contexts span 2 .. kSeqWaves
// partitions of at most 64 blocks, with every (sequence, K/V head) workgroup
// resident at once (at most wgs_per_cu * CUs of them: one round, so that the
// order of seq_unit pairs long and short sequences on each compute unit) and
// at most 64 * kPlanChunks sequences.
bool paged_decode_seq_fits(const DecodeArgs &a)
{
    if (a.shared_len || a.num_parts < 2 || a.num_parts > kSeqWaves || a.part_tiles > 64 ||
        a.num_seqs > 64 * kPlanChunks)
        return false;
    const DeviceShape dev = device_shape();
    const int per_cu = seq_wgs_per_cu();
    return dev.cus > 0 && per_cu > 0 &&
           (int64_t)a.num_seqs * a.num_kv_heads <= (int64_t)per_cu * dev.cus;
}

// The whole decode step in one launch (a.part_acc = out); requires
// paged_decode_seq_fits(a).
hipError_t launch_paged_decode_seq(const DecodeArgs &args, hipStream_t stream)
{
    DecodeArgs a = args;
    const DeviceShape dev = device_shape();
    a.plan_width = dev.cus / std::gcd(a.num_kv_heads, dev.cus);
    a.num_parts = 1;                         // out's layout: one "partition" per (sequence, head)
    a.normalize = 1;
    const dim3 grid((unsigned)((int64_t)a.num_seqs * a.num_kv_heads));
    if (a.k_new)
        hipLaunchKernelGGL(paged_decode_seq_kernel<true>, grid, dim3(64 * kSeqWaves), 0, stream, a);
    else
        hipLaunchKernelGGL(paged_decode_seq_kernel<false>, grid, dim3(64 * kSeqWaves), 0, stream, a);
    return hipGetLastError();
}

// The whole-group form serves a shared-prefix step (with its appends) with
// groups of at most kGroupMaxMembers sequences (in their own order or through
// group_order) and every (group, K/V head) workgroup resident at once.
bool paged_decode_group_fits(const DecodeArgs &a)
{
    if (!a.shared_len || !a.k_new || a.group_size > kGroupMaxMembers || a.num_parts < 1)
        return false;
    const DeviceShape dev = device_shape();
    const int per_cu = group_wgs_per_cu();
    return dev.cus > 0 && per_cu > 0 &&
           (int64_t)a.num_groups * a.num_kv_heads <= (int64_t)per_cu * dev.cus;
}

// The whole shared-prefix step in one launch (a.part_acc = out); requires
// paged_decode_group_fits(a).
hipError_t launch_paged_decode_group(const DecodeArgs &args, hipStream_t stream)
{
    DecodeArgs a = args;
    const DeviceShape dev = device_shape();
    a.plan_width = dev.cus / std::gcd(a.num_kv_heads, dev.cus);
    const dim3 grid((unsigned)((int64_t)a.num_groups * a.num_kv_heads));
    hipLaunchKernelGGL(paged_decode_group_kernel<true>, grid, dim3(64 * kGroupWaves), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_paged_decode(const DecodeArgs &args, hipStream_t stream)
{
    DecodeArgs a = args;
    const DeviceShape dev = device_shape();
    const int64_t groups = (int64_t)a.num_kv_heads * a.num_seqs * a.num_parts;
    const int64_t resident = (int64_t)dev.cus * dev.waves_per_cu;
    const bool split = resident > 0 && groups <= 2 * resident;
    if (a.shared_len) {
        // One workgroup per (group, head, partition) for the group pass, then
        // one per (sequence, head, partition) for the rest, in one grid; the
        // rest in the balanced order when the sequences are in their own
        // order (no group_order) and the grid is larger than the device holds.
        const int64_t shared_groups = (int64_t)a.num_kv_heads * a.num_groups * a.num_parts;
        const dim3 grid((unsigned)(shared_groups + groups));
        a.plan_width = 0;
        if (groups > resident && !a.group_order && a.num_seqs <= 64 * kPlanChunks && dev.cus > 0)
            a.plan_width = dev.cus / std::gcd(a.num_kv_heads, dev.cus);
        const unsigned sg = (unsigned)shared_groups;
        if (split && a.k_new)
            hipLaunchKernelGGL((paged_decode_shared_kernel<true, 4, false>), grid, dim3(256), 0,
                               stream, a, sg);
        else if (split)
            hipLaunchKernelGGL((paged_decode_shared_kernel<false, 4, false>), grid, dim3(256), 0,
                               stream, a, sg);
        else if (a.k_new && a.plan_width > 0)
            hipLaunchKernelGGL((paged_decode_shared_kernel<true, 1, true>), grid, dim3(64), 0,
                               stream, a, sg);
        else if (a.plan_width > 0)
            hipLaunchKernelGGL((paged_decode_shared_kernel<false, 1, true>), grid, dim3(64), 0,
                               stream, a, sg);
        else if (a.k_new)
            hipLaunchKernelGGL((paged_decode_shared_kernel<true, 1, false>), grid, dim3(64), 0,
                               stream, a, sg);
        else
            hipLaunchKernelGGL((paged_decode_shared_kernel<false, 1, false>), grid, dim3(64), 0,
                               stream, a, sg);
        return hipGetLastError();
    }
    // Balanced order: consecutive workgroups of one head cycle over
    // cus / gcd(heads, cus) compute units (32 on one XCD for 8 heads).  Not
    // with a single, self-normalised partition: there an empty context's
    // unit must know its sequence to write its zero rows.
    a.plan_width = 0;
    if (groups > resident && !a.shared_len && !a.normalize && a.num_seqs <= 64 * kPlanChunks &&
        dev.cus > 0)
        a.plan_width = dev.cus / std::gcd(a.num_kv_heads, dev.cus);
    if (split && a.plan_width > 0) {
        if (a.k_new)
            launch<true, false, true, 4>(a, groups, stream);
        else
            launch<false, false, true, 4>(a, groups, stream);
    } else if (split) {
        if (a.k_new)
            launch<true, false, false, 4>(a, groups, stream);
        else
            launch<false, false, false, 4>(a, groups, stream);
    } else if (a.plan_width > 0) {
        if (a.k_new)
            launch<true, false, true, 1>(a, groups, stream);
        else
            launch<false, false, true, 1>(a, groups, stream);
    } else {
        if (a.k_new)
            launch<true, false, false, 1>(a, groups, stream);
        else
            launch<false, false, false, 1>(a, groups, stream);
    }
    return hipGetLastError();
}

// The vector-ALU form of the plain partition pass: 4 wavefronts per
// partition always, in the balanced order when the grid is larger than the
// device holds (as the matrix form's policy), for 4 query heads per K/V head.
hipError_t launch_paged_decode_vector(const DecodeArgs &args, hipStream_t stream)
{
    DecodeArgs a = args;
    if (a.group != kVecGroup || a.k_new || a.shared_len || a.normalize)
        return hipErrorInvalidValue;
    const DeviceShape dev = device_shape();
    const int64_t groups = (int64_t)a.num_kv_heads * a.num_seqs * a.num_parts;
    const int64_t resident = (int64_t)dev.cus * dev.waves_per_cu;
    a.plan_width = 0;
    if (groups > resident && a.num_seqs <= 64 * kPlanChunks && dev.cus > 0)
        a.plan_width = dev.cus / std::gcd(a.num_kv_heads, dev.cus);
    if (a.plan_width > 0)
        hipLaunchKernelGGL(paged_decode_vec_kernel<true>, dim3((unsigned)groups), dim3(256), 0,
                           stream, a);
    else
        hipLaunchKernelGGL(paged_decode_vec_kernel<false>, dim3((unsigned)groups), dim3(256), 0,
                           stream, a);
    return hipGetLastError();
}

}  // namespace tv
