// QKV post-processing of the attention shard ("Tensor parallelism from
// scratch", "Implementation", TPAttention.forward): split the merged
// projection into the rank's lq q heads and lkv k/v heads, apply the per-head
// QK-norm (weights of length head_dim, a full copy on every rank), rotate q
// and k by RoPE at the token's absolute position, and append k and v to the
// rank's cache at positions past .. past+T-1 (the cache holds only the rank's
// kv heads).
//
// Norm: v / sqrt(mean(v^2) + eps) * w.  RoPE: rotate-half, the pair
// (v[i], v[i+64]) turns by pos * theta^(-2i/128).  (Qwen3 conventions; the
// pages import both without printing them.)
//
// One wave per (row, head): lane i holds elements i and i+64, which is the
// rotate-half pair, so RoPE is lane-local and the norm is one wave reduction.
#include "common.h"

namespace tps {

namespace {

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__global__ __launch_bounds__(256) void qkv_norm_rope_kernel(QkvArgs a, int heads) {
  const int lane = threadIdx.x & 63;
  const int h = blockIdx.y * 4 + (threadIdx.x >> 6);
  if (h >= heads) return;
  const int64_t m = blockIdx.x;                  // row = b*T + t
  const int b = (int)(m / a.T), t = (int)(m - (int64_t)b * a.T);
  const int pos = a.past + t;
  const int64_t n_qkv = (int64_t)heads * 128;
  const float* src = a.qkv + m * n_qkv + (int64_t)h * 128;
  float x1 = src[lane], x2 = src[lane + 64];

  if (h < a.lq + a.lkv) {
    const bf16* w = h < a.lq ? a.q_norm_w : a.k_norm_w;
    const float ss = wave_sum(x1 * x1 + x2 * x2);
    const float inv = 1.0f / sqrtf(ss * (1.0f / 128.0f) + a.eps);
    x1 *= inv * bf2f(w[lane]);
    x2 *= inv * bf2f(w[lane + 64]);
    // angle in double (pos up to ~1e6 would lose fp32 bits), reduced to
    // [-pi, pi] before the fp32 sin/cos
    const double inv_freq = exp2(-(double)(2 * lane) / 128.0 * log2((double)a.theta));
    double ang = (double)pos * inv_freq;
    ang -= 6.283185307179586476925 * rint(ang * 0.159154943091895335768883);
    float sn, cs;
    sincosf((float)ang, &sn, &cs);
    const float y1 = x1 * cs - x2 * sn;
    const float y2 = x2 * cs + x1 * sn;
    x1 = y1;
    x2 = y2;
  }
  bf16* dst;
  if (h < a.lq) {
    dst = a.q_out + m * ((int64_t)a.lq * 128) + (int64_t)h * 128;
  } else if (h < a.lq + a.lkv) {
    dst = a.k_cache + (((int64_t)b * a.lkv + (h - a.lq)) * a.S_max + pos) * 128;
  } else {
    dst = a.v_cache + (((int64_t)b * a.lkv + (h - a.lq - a.lkv)) * a.S_max + pos) * 128;
  }
  dst[lane] = f2bf(x1);
  dst[lane + 64] = f2bf(x2);
}

}  // namespace

hipError_t qkv_norm_rope_store(const QkvArgs& a, hipStream_t s) {
  const int64_t M = (int64_t)a.B * a.T;
  if (M <= 0) return hipSuccess;
  const int heads = a.lq + 2 * a.lkv;
  dim3 grid((unsigned)M, (heads + 3) / 4);
  qkv_norm_rope_kernel<<<grid, 256, 0, s>>>(a, heads);
  return hipGetLastError();
}

}  // namespace tps
