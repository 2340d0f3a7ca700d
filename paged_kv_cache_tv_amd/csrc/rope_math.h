// Rotation angles of the rotary position embedding ("tiny-vllm 씹뜯맛즐 - (1)"
// page, section "5. 절대 위치 임베딩 대신 RoPE": q and k at position p are
// turned by R_p; each pair of dimensions by the angle p * inv_freq[pair]).
//
// The angle p * f is formed exactly as hi + lo (a float product and its fma
// residual; p is exact in float for |p| < 2^24) and reduced modulo 2 pi with a
// three-part split of 2 pi (Cody and Waite's additive range reduction), so
// that cos and sin see an argument in [-pi, pi] accurate to a few ulp even
// at positions near 2^17, where the plain float product would be off by
// ~1e-2 rad.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>

namespace tv {

__device__ __forceinline__ void rope_cos_sin(int p, float f, float &c, float &s)
{
    constexpr float kTwoPiA = 6.2831854820251465f;        // 2 pi = A + B + C (+ 4e-23)
    constexpr float kTwoPiB = -1.7484555314695172e-07f;
    constexpr float kTwoPiC = -6.8604980400235275e-15f;
    constexpr float kInvTwoPi = 0.15915493667125702f;
    const float pf = (float)p;
    const float hi = pf * f;
    const float lo = fmaf(pf, f, -hi);
    const float n = rintf(hi * kInvTwoPi);
    float r = fmaf(-n, kTwoPiA, hi);
    r = fmaf(-n, kTwoPiB, r);
    r = fmaf(-n, kTwoPiC, r);
    r += lo;
    sincosf(r, &s, &c);
}

// Rotate the pair (a, b) by (c, s): (a c - b s, a s + b c).
__device__ __forceinline__ void rope_turn(float a, float b, float c, float s, float &ra, float &rb)
{
    ra = fmaf(a, c, -(b * s));
    rb = fmaf(a, s, b * c);
}

}  // namespace tv
