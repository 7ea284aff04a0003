// QK-norm and RoPE of one (row, head) of the merged q/k/v projection, on 16
// lanes ("Tensor parallelism from scratch", "Implementation",
// TPAttention.forward: RMSNorm of each q and k head over d, then RoPE at the
// token's absolute position).  Norm: v / sqrt(mean(v^2) + eps) * w; RoPE:
// rotate-half, the pair (v[i], v[i+64]) turns by pos * theta^(-2i/128)
// (Qwen3 conventions, which the pages import without printing).
//
// Lane j of the 16 holds d = 4j .. 4j+3 in x[0..3] and their RoPE partners
// d + 64 in x[4..7], so the rotation stays inside the lane and the norm is a
// 16-lane reduction.  rope_coef() gives theta^(-2i/128) / (2 pi) for the
// lane's four indices i = 4j + e as a float head plus tail; rope_sincos()
// forms the angle in revolutions, pos * coef, without losing the fraction
// (the head product's rounding error by FMA, the integer part dropped before
// the small terms are added; positions are exact in fp32 below 2^24), and
// the hardware sine and cosine take revolutions.
#pragma once

#include "common.h"

namespace tps {

struct RopeCoef {
  float hi[4], lo[4];
};
__device__ __forceinline__ RopeCoef rope_coef(float theta, int j) {
  RopeCoef c;
  const double l2t = log2((double)theta);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const double cr = exp2(-(double)(2 * (4 * j + e)) / 128.0 * l2t) * 0.159154943091895335768883;
    c.hi[e] = (float)cr;
    c.lo[e] = (float)(cr - (double)c.hi[e]);
  }
  return c;
}
__device__ __forceinline__ void rope_sincos(int pos, float hi, float lo, float& sn, float& cs) {
  const float p = (float)pos;
  const float q = p * hi;
  const float err = __builtin_fmaf(p, hi, -q);   // q + err == p * hi exactly
  const float rev = (q - __builtin_rintf(q)) + __builtin_fmaf(p, lo, err);
  sn = __builtin_amdgcn_sinf(rev);
  cs = __builtin_amdgcn_cosf(rev);
}
// the lane's norm weights, d = 4j .. 4j+3 and d + 64, as floats
struct NormW {
  float v[8];
};
__device__ __forceinline__ NormW norm_w(const bf16* w, int j) {
  const bf16x4 w0 = *reinterpret_cast<const bf16x4*>(w + 4 * j), w1 = *reinterpret_cast<const bf16x4*>(w + 64 + 4 * j);
  NormW r;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    r.v[e] = bf2f(w0[e]);
    r.v[4 + e] = bf2f(w1[e]);
  }
  return r;
}
// x *= rsqrt(mean(x^2) + eps) * w over the head's 128 values (16 lanes),
// then the rotation at position pos.  The reciprocal square root is the
// hardware one (about 1 ulp of fp32, far below the bf16 rounding of the
// result).
__device__ __forceinline__ void qk_norm_rope(float (&x)[8], const NormW& w, int pos, const RopeCoef& rc, float eps) {
  float ss = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) ss += x[e] * x[e];
  ss = row_sum16(ss);
  const float inv = __builtin_amdgcn_rsqf(ss * (1.0f / 128.0f) + eps);
#pragma unroll
  for (int e = 0; e < 8; ++e) x[e] *= inv * w.v[e];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    float sn, cs;
    rope_sincos(pos, rc.hi[e], rc.lo[e], sn, cs);
    const float x1 = x[e], x2 = x[4 + e];
    x[e] = x1 * cs - x2 * sn;
    x[4 + e] = x2 * cs + x1 * sn;
  }
}
__device__ __forceinline__ void qk_norm_rope(float (&x)[8], const bf16* w, int pos, int j, const RopeCoef& rc,
                                             float eps) {
  qk_norm_rope(x, norm_w(w, j), pos, rc, eps);
}
// the lane's eight values of a 128-wide head row at dst, as bf16
__device__ __forceinline__ void store_head_lanes(bf16* dst, const float (&x)[8], int j) {
  const bf16x4 o0 = {f2bf(x[0]), f2bf(x[1]), f2bf(x[2]), f2bf(x[3])};
  const bf16x4 o1 = {f2bf(x[4]), f2bf(x[5]), f2bf(x[6]), f2bf(x[7])};
  *reinterpret_cast<bf16x4*>(dst + 4 * j) = o0;
  *reinterpret_cast<bf16x4*>(dst + 64 + 4 * j) = o1;
}

}  // namespace tps
