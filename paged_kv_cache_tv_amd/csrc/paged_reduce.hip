// Log-sum-exp merge of the decode partitions ("vLLM" page, section "Flash
// Attention": the running maximum / running sum rule, applied across the
// context partitions of one sequence and query head).
//
// One 256-thread workgroup per (sequence, query head).  Pass 1 finds the
// largest partition maximum M; pass 2 sums the weights 2^(m_p - M) * l_p;
// pass 3 has 16 partition lanes x 16 four-wide column lanes accumulate the
// weighted partial outputs, merged through LDS in a fixed order (so the result
// is bitwise reproducible run to run).
#include "tv_internal.h"

#include <math.h>

namespace tv {
namespace {

constexpr int D = kHeadDim;
constexpr int kThreads = 256;

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

__global__ __launch_bounds__(kThreads) void paged_reduce_kernel(ReduceArgs a)
{
    const int sh = blockIdx.x;                     // s * num_q_heads + h
    const int s = sh / a.num_q_heads;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wv = tid >> 6;

    int n = a.context_lens[s];
    n = n < 0 ? 0 : (n > a.max_context_len ? a.max_context_len : n);
    const int np = (n + a.partition_size - 1) / a.partition_size;
    float *out = a.out + (int64_t)sh * D;

    const float *pm = a.part_max + (int64_t)sh * a.num_parts;
    const float *pl = a.part_sum + (int64_t)sh * a.num_parts;
    const float *pa = a.part_acc + (int64_t)sh * a.num_parts * D;

    __shared__ float red[kThreads / 64];
    __shared__ float4 acc_sm[16][16];

    // Pass 1: M = max_p m_p.
    float m = -INFINITY;
    for (int p = tid; p < np; p += kThreads)
        m = fmaxf(m, pm[p]);
    m = wave_max(m);
    if (lane == 0)
        red[wv] = m;
    __syncthreads();
    const float M = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    __syncthreads();

    if (M == -INFINITY) {                          // no partition / no usable token
        if (tid < D)
            out[tid] = 0.f;
        return;
    }

    // Pass 2: denominator.
    float den = 0.f;
    for (int p = tid; p < np; p += kThreads)
        den = fmaf(__builtin_amdgcn_exp2f(pm[p] - M), pl[p], den);
    den = wave_sum(den);
    if (lane == 0)
        red[wv] = den;
    __syncthreads();
    const float DEN = (red[0] + red[1]) + (red[2] + red[3]);

    // Pass 3: numerator, dims 4c..4c+3 for partitions pg, pg+16, ...
    const int pg = tid >> 4;
    const int cidx = tid & 15;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int p = pg; p < np; p += 16) {
        const float wgt = __builtin_amdgcn_exp2f(pm[p] - M);
        const float4 x = reinterpret_cast<const float4 *>(pa + (int64_t)p * D)[cidx];
        acc.x = fmaf(wgt, x.x, acc.x);
        acc.y = fmaf(wgt, x.y, acc.y);
        acc.z = fmaf(wgt, x.z, acc.z);
        acc.w = fmaf(wgt, x.w, acc.w);
    }
    acc_sm[pg][cidx] = acc;
    __syncthreads();
    if (tid < 16) {
        float4 t = acc_sm[0][tid];
#pragma unroll
        for (int q = 1; q < 16; ++q) {
            const float4 y = acc_sm[q][tid];
            t.x += y.x;
            t.y += y.y;
            t.z += y.z;
            t.w += y.w;
        }
        const float inv = 1.f / DEN;
        reinterpret_cast<float4 *>(out)[tid] = make_float4(t.x * inv, t.y * inv, t.z * inv, t.w * inv);
    }
}

}  // namespace

hipError_t launch_paged_reduce(const ReduceArgs &a, hipStream_t stream)
{
    const int64_t groups = (int64_t)a.num_seqs * a.num_q_heads;
    hipLaunchKernelGGL(paged_reduce_kernel, dim3((unsigned)groups), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace tv
