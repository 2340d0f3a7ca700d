// Log-sum-exp merge of the decode partitions ("vLLM" page, section "Flash
// Attention": the running maximum / running sum rule, applied across the
// context partitions of one sequence and query head).
//
// Short contexts (at most kMerge partitions in the workspace): one wavefront
// per (sequence, query head), four per workgroup.  Such a merge is
// latency-bound (a few hundred bytes per wavefront), so it waits on memory
// once: the context length, the partition maxima and sums (lane p holds
// partition p) and the rows of every workspace partition (lane d holds
// dimension d) are loaded together, and the partitions past the sequence's
// end -- never written, so any bits -- are selected away afterwards.
//
// 9 to 256 partitions and few rows (s, h) -- very long contexts at a small
// batch, where one workgroup per row would leave most of the device idle:
// each row is split over four workgroups of four float4 columns each, and a
// workgroup waits on memory once (every partition's column, maximum and sum
// loaded together with the context length).
//
// Otherwise: one 256-thread workgroup per (sequence, query head); thread
// (group q = tid/16, column c = tid%16) accumulates the float4 column c of
// partitions q, q+16, q+32, ..., eight rows in flight at a time, and the 16
// groups are summed through shuffles and LDS.
//
// Summation orders are fixed, so results are bitwise reproducible run to run.
#include "tv_internal.h"

#include <math.h>

namespace tv {
namespace {

constexpr int D = kHeadDim;
constexpr int kWavesPerGroup = 4;
constexpr int kMerge = 8;          // partitions whose rows are loaded up front

__device__ __forceinline__ float wave_max(float x)
{
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1)
        x = fmaxf(x, __shfl_xor(x, m));
    return x;
}

__device__ __forceinline__ float wave_sum(float x)
{
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1)
        x += __shfl_xor(x, m);
    return x;
}

// Lane j's float, broadcast (the lane-read builtin moves 32-bit integers).
__device__ __forceinline__ float lane_value(float x, int j)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), j));
}

__global__ __launch_bounds__(64 * kWavesPerGroup) void paged_reduce_kernel(ReduceArgs a)
{
    const int64_t sh = (int64_t)blockIdx.x * kWavesPerGroup + (threadIdx.x >> 6);   // s * Hq + h
    if (sh >= (int64_t)a.num_seqs * a.num_q_heads)
        return;
    const int lane = threadIdx.x & 63;
    const int s = (int)(sh / a.num_q_heads);

    // Issue every load before using any of them.
    const int P = a.num_parts;                     // <= kMerge here, so np <= kMerge
    const float *pm = a.part_max + sh * P;
    const float *pl = a.part_sum + sh * P;
    const float *pa = a.part_acc + sh * P * D;
    int n = a.context_lens[s];
    float rows[kMerge];
#pragma unroll
    for (int j = 0; j < kMerge; ++j)
        rows[j] = j < P ? pa[(int64_t)j * D + lane] : 0.f;
    const float m_raw = lane < P ? pm[lane] : -INFINITY;
    const float l_raw = lane < P ? pl[lane] : 0.f;
    n = n < 0 ? 0 : (n > a.max_context_len ? a.max_context_len : n);
    const int np = (n + a.partition_size - 1) / a.partition_size;
    float *out = a.out + sh * D;
    const float m_lane = lane < np ? m_raw : -INFINITY;
    const float l_lane = lane < np ? l_raw : 0.f;

    const float M = wave_max(m_lane);
    if (M == -INFINITY) {                          // no partition / no usable token
        out[lane] = 0.f;
        return;
    }

    const float w_lane = m_lane == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_lane - M);
    const float den_part = w_lane * l_lane;
    float acc = 0.f;
#pragma unroll
    for (int j = 0; j < kMerge; ++j)
        if (j < np)
            acc = fmaf(lane_value(w_lane, j), rows[j], acc);
    const float den = wave_sum(den_part);
    out[lane] = acc / den;
}

// 9 .. kMid workspace partitions: every load issued at once.  The 16 float4
// columns of a (s, h) row are split over SPLIT workgroups (blockIdx.y), so
// that short batches still spread over the device; each workgroup holds
// C = 16 / SPLIT columns.  Thread (group q = tid / C, column c = tid % C)
// holds its column of partitions q, q + G, q + 2G, ... (G = 256 / C groups)
// together with their maxima and sums, loaded alongside the context length;
// partitions past the sequence's end are selected away.  The maximum, the
// sum and the groups' partial rows are then combined through shuffles and
// LDS in a fixed order.
constexpr int kMid = 256;
constexpr int kMidSplit = 4;
// Rows (s, h) up to which the split form runs.  Past it the grid fills the
// device anyway, and the wide kernel's whole-row loads (a wavefront reads
// four contiguous 256-byte rows) and single read of the maxima and sums
// win: at 2048 rows it is 1.9x (64 partitions) to 3x (256) faster.
constexpr int64_t kMidRows = 256;

template <int SPLIT>
__global__ __launch_bounds__(256) void paged_reduce_mid_kernel(ReduceArgs a)
{
    constexpr int C = 16 / SPLIT;                  // float4 columns per workgroup
    constexpr int G = 256 / C;                     // partition groups
    constexpr int U = kMid / G;                    // partitions per thread
    const int64_t sh = blockIdx.x;                 // s * Hq + h
    const int s = (int)(sh / a.num_q_heads);
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wv = tid >> 6;
    const int q = tid / C;
    const int c = tid % C;
    const int col = (int)blockIdx.y * C + c;
    const int P = a.num_parts;                     // kMerge < P <= kMid
    const float *pm = a.part_max + sh * P;
    const float *pl = a.part_sum + sh * P;
    const float4 *pa = reinterpret_cast<const float4 *>(a.part_acc + sh * P * D);
    float4 *out = reinterpret_cast<float4 *>(a.out + sh * D);

    int n = a.context_lens[s];
    float4 x[U];
    float mp[U], lp[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int p = q + G * u;
        const bool in = p < P;
        x[u] = in ? pa[(int64_t)p * 16 + col] : make_float4(0.f, 0.f, 0.f, 0.f);
        mp[u] = in ? pm[p] : -INFINITY;
        lp[u] = in ? pl[p] : 0.f;
    }
    n = n < 0 ? 0 : (n > a.max_context_len ? a.max_context_len : n);
    const int np = (n + a.partition_size - 1) / a.partition_size;

    __shared__ float red[4];
    __shared__ float4 part4[4][C];

    float m = -INFINITY;
#pragma unroll
    for (int u = 0; u < U; ++u)
        if (q + G * u < np)
            m = fmaxf(m, mp[u]);
    m = wave_max(m);
    if (lane == 0)
        red[wv] = m;
    __syncthreads();
    const float M = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    __syncthreads();
    if (M == -INFINITY) {                          // no partition / no usable token
        if (tid < C)
            out[col] = make_float4(0.f, 0.f, 0.f, 0.f);
        return;
    }

    float den = 0.f;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const bool live = q + G * u < np && mp[u] != -INFINITY;
        const float w = live ? __builtin_amdgcn_exp2f(mp[u] - M) : 0.f;
        if (live) {
            den = fmaf(w, lp[u], den);
            acc.x = fmaf(w, x[u].x, acc.x);
            acc.y = fmaf(w, x[u].y, acc.y);
            acc.z = fmaf(w, x[u].z, acc.z);
            acc.w = fmaf(w, x[u].w, acc.w);
        }
    }
    // Sum the wavefront's partition groups (lanes c, c + C, c + 2C, ...).
#pragma unroll
    for (int mk = C; mk <= 32; mk <<= 1) {
        den += __shfl_xor(den, mk);
        acc.x += __shfl_xor(acc.x, mk);
        acc.y += __shfl_xor(acc.y, mk);
        acc.z += __shfl_xor(acc.z, mk);
        acc.w += __shfl_xor(acc.w, mk);
    }
    if (lane < C)
        part4[wv][lane] = acc;
    if (lane == 0)
        red[wv] = den;                             // every column's groups hold the same sums
    __syncthreads();
    if (tid < C) {
        const float DEN = (red[0] + red[1]) + (red[2] + red[3]);
        float4 t = part4[0][tid];
#pragma unroll
        for (int w4 = 1; w4 < 4; ++w4) {
            t.x += part4[w4][tid].x;
            t.y += part4[w4][tid].y;
            t.z += part4[w4][tid].z;
            t.w += part4[w4][tid].w;
        }
        out[col] = make_float4(t.x / DEN, t.y / DEN, t.z / DEN, t.w / DEN);
    }
}

__global__ __launch_bounds__(256) void paged_reduce_wide_kernel(ReduceArgs a)
{
    const int64_t sh = blockIdx.x;                 // s * Hq + h
    const int s = (int)(sh / a.num_q_heads);
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wv = tid >> 6;

    int n = a.context_lens[s];
    n = n < 0 ? 0 : (n > a.max_context_len ? a.max_context_len : n);
    const int np = (n + a.partition_size - 1) / a.partition_size;
    float *out = a.out + sh * D;
    const float *pm = a.part_max + sh * a.num_parts;
    const float *pl = a.part_sum + sh * a.num_parts;
    const float4 *pa = reinterpret_cast<const float4 *>(a.part_acc + sh * a.num_parts * D);

    __shared__ float red[4];
    __shared__ float4 part4[4][16];

    float m = -INFINITY;
    for (int p = tid; p < np; p += 256)
        m = fmaxf(m, pm[p]);
    m = wave_max(m);
    if (lane == 0)
        red[wv] = m;
    __syncthreads();
    const float M = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    __syncthreads();
    if (M == -INFINITY) {
        if (tid < D)
            out[tid] = 0.f;
        return;
    }

    float den = 0.f;
    for (int p = tid; p < np; p += 256) {
        const float mp = pm[p];
        if (mp != -INFINITY)
            den = fmaf(__builtin_amdgcn_exp2f(mp - M), pl[p], den);
    }
    den = wave_sum(den);
    if (lane == 0)
        red[wv] = den;

    const int q = tid >> 4;
    const int c = tid & 15;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int p0 = q; p0 < np; p0 += 16 * 8) {
        float4 x[8];
        float w[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int p = p0 + 16 * u;
            const bool live = p < np;
            x[u] = live ? pa[(int64_t)p * 16 + c] : make_float4(0.f, 0.f, 0.f, 0.f);
            const float mp = live ? pm[p] : -INFINITY;
            w[u] = mp == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mp - M);
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            acc.x = fmaf(w[u], x[u].x, acc.x);
            acc.y = fmaf(w[u], x[u].y, acc.y);
            acc.z = fmaf(w[u], x[u].z, acc.z);
            acc.w = fmaf(w[u], x[u].w, acc.w);
        }
    }
    // Sum the four partition groups of this wavefront (lanes c, c+16, c+32, c+48).
#pragma unroll
    for (int mk = 16; mk <= 32; mk <<= 1) {
        acc.x += __shfl_xor(acc.x, mk);
        acc.y += __shfl_xor(acc.y, mk);
        acc.z += __shfl_xor(acc.z, mk);
        acc.w += __shfl_xor(acc.w, mk);
    }
    if (lane < 16)
        part4[wv][lane] = acc;
    __syncthreads();
    if (tid < 16) {
        const float DEN = (red[0] + red[1]) + (red[2] + red[3]);
        float4 t = part4[0][tid];
#pragma unroll
        for (int x = 1; x < 4; ++x) {
            t.x += part4[x][tid].x;
            t.y += part4[x][tid].y;
            t.z += part4[x][tid].z;
            t.w += part4[x][tid].w;
        }
        reinterpret_cast<float4 *>(out)[tid] = make_float4(t.x / DEN, t.y / DEN, t.z / DEN, t.w / DEN);
    }
}

}  // namespace

hipError_t launch_paged_reduce(const ReduceArgs &a, hipStream_t stream)
{
    if (a.num_parts > kMerge) {
        const int64_t groups = (int64_t)a.num_seqs * a.num_q_heads;
        if (a.num_parts <= kMid && groups <= kMidRows)
            hipLaunchKernelGGL(paged_reduce_mid_kernel<kMidSplit>,
                               dim3((unsigned)groups, kMidSplit), dim3(256), 0, stream, a);
        else
            hipLaunchKernelGGL(paged_reduce_wide_kernel, dim3((unsigned)groups), dim3(256), 0,
                               stream, a);
        return hipGetLastError();
    }
    const int64_t waves = (int64_t)a.num_seqs * a.num_q_heads;
    const int64_t groups = (waves + kWavesPerGroup - 1) / kWavesPerGroup;
    hipLaunchKernelGGL(paged_reduce_kernel, dim3((unsigned)groups), dim3(64 * kWavesPerGroup), 0,
                       stream, a);
    return hipGetLastError();
}

}  // namespace tv
