// The replicated step around a row-parallel layer ("Tensor parallelism from
// scratch", "Implementation", TPTransformer.forward: the block adds the
// attention output to the residual stream and normalises the sum before the
// MLP; the row-parallel outputs are the sums over ranks of the ranks'
// partials; "The cost of communication": engines fuse that all-reduce with
// the following RMSNorm):
//
//   h = bf16(residual + sum_r partial_r)      the new residual stream
//   y = bf16(h / sqrt(mean(h^2) + eps) * w)   the next layer's normed input
//
// On one GPU the ranks' partials arrive stacked [n, M, H] and are summed
// here in rank order (fp32, residual first), in the same pass as the add and
// the norm.  The threads of a row keep it in registers between the sum and
// the scaling: every input byte is read once and each output written once.
#include "common.h"

namespace tps {

namespace {

constexpr int kNormThreads = 256;
constexpr int kNormGroup = 4;   // partials whose loads are in flight together

// TPR threads (one to four waves) per row, NC 16-byte chunks per thread:
// H <= TPR * NC * 8.  Wide rows spread over more waves so that a launch has
// enough loads in flight; the partials are read kNormGroup at a time.
template <int TPR, int NC>
__global__ __launch_bounds__(kNormThreads) void residual_rmsnorm_kernel(const bf16* __restrict__ partials, int n,
                                                                        int64_t M, int H, const bf16* residual,
                                                                        const bf16* __restrict__ w, float eps,
                                                                        bf16* h_out, bf16* __restrict__ y_out) {
  constexpr int ROWS = kNormThreads / TPR;
  const int t = threadIdx.x % TPR;
  const int64_t m = (int64_t)blockIdx.x * ROWS + threadIdx.x / TPR;
  const bool live = m < M;
  const int nc = H / 8;
  const int64_t row = (live ? m : 0) * H;
  const int64_t plane = M * H;
  bool on[NC];
#pragma unroll
  for (int k = 0; k < NC; ++k) on[k] = live && t + k * TPR < nc;
  // residual, norm weight and the first group of partials are all
  // requested before the first use of any of them
  bf16x8 rv[NC], wv[NC], v[kNormGroup][NC];
#pragma unroll
  for (int k = 0; k < NC; ++k)
    if (on[k]) {
      rv[k] = *reinterpret_cast<const bf16x8*>(residual + row + (int64_t)(t + k * TPR) * 8);
      wv[k] = *reinterpret_cast<const bf16x8*>(w + (int64_t)(t + k * TPR) * 8);
    }
  float acc[NC][8];
  for (int r0 = 0; r0 < n; r0 += kNormGroup) {
#pragma unroll
    for (int g = 0; g < kNormGroup; ++g)
#pragma unroll
      for (int k = 0; k < NC; ++k)
        if (r0 + g < n && on[k])
          v[g][k] = *reinterpret_cast<const bf16x8*>(partials + (int64_t)(r0 + g) * plane + row +
                                                     (int64_t)(t + k * TPR) * 8);
    if (r0 == 0)
#pragma unroll
      for (int k = 0; k < NC; ++k)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[k][e] = on[k] ? bf2f(rv[k][e]) : 0.f;
#pragma unroll
    for (int g = 0; g < kNormGroup; ++g)   // rank order
      if (r0 + g < n)
#pragma unroll
        for (int k = 0; k < NC; ++k)
          if (on[k])
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[k][e] += bf2f(v[g][k][e]);
  }
  float ss = 0.f;
#pragma unroll
  for (int k = 0; k < NC; ++k) {
    if (on[k]) {
      bf16x8 hb;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        hb[e] = f2bf(acc[k][e]);
        acc[k][e] = bf2f(hb[e]);   // the norm sees the stored (rounded) residual
        ss += acc[k][e] * acc[k][e];
      }
      __builtin_nontemporal_store(hb, reinterpret_cast<bf16x8*>(h_out + row + (int64_t)(t + k * TPR) * 8));
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) ss += __shfl_xor(ss, o, 64);
  if constexpr (TPR > 64) {
    __shared__ float s_ss[kNormThreads / 64];
    if ((threadIdx.x & 63) == 0) s_ss[threadIdx.x >> 6] = ss;
    __syncthreads();
    const int w0 = (threadIdx.x / TPR) * (TPR / 64);
    ss = 0.f;
#pragma unroll
    for (int i = 0; i < TPR / 64; ++i) ss += s_ss[w0 + i];
  }
  const float inv = 1.0f / sqrtf(ss / (float)H + eps);
#pragma unroll
  for (int k = 0; k < NC; ++k) {
    if (on[k]) {
      bf16x8 yb;
#pragma unroll
      for (int e = 0; e < 8; ++e) yb[e] = f2bf(acc[k][e] * inv * bf2f(wv[k][e]));
      __builtin_nontemporal_store(yb, reinterpret_cast<bf16x8*>(y_out + row + (int64_t)(t + k * TPR) * 8));
    }
  }
}

template <int TPR, int NC>
void launch_norm(const bf16* partials, int n, int64_t M, int H, const bf16* residual, const bf16* w, float eps,
                 bf16* h_out, bf16* y_out, hipStream_t s) {
  constexpr int ROWS = kNormThreads / TPR;
  const unsigned grid = (unsigned)((M + ROWS - 1) / ROWS);
  residual_rmsnorm_kernel<TPR, NC><<<grid, kNormThreads, 0, s>>>(partials, n, M, H, residual, w, eps, h_out, y_out);
}

template <int TPR>
void launch_norm_tpr(int nc_per, const bf16* partials, int n, int64_t M, int H, const bf16* residual, const bf16* w,
                     float eps, bf16* h_out, bf16* y_out, hipStream_t s) {
  switch (nc_per) {
    case 1: launch_norm<TPR, 1>(partials, n, M, H, residual, w, eps, h_out, y_out, s); break;
    case 2: launch_norm<TPR, 2>(partials, n, M, H, residual, w, eps, h_out, y_out, s); break;
    case 3: launch_norm<TPR, 3>(partials, n, M, H, residual, w, eps, h_out, y_out, s); break;
    default: launch_norm<TPR, 4>(partials, n, M, H, residual, w, eps, h_out, y_out, s); break;
  }
}

}  // namespace

hipError_t residual_rmsnorm(const bf16* partials, int n, int64_t M, int H, const bf16* residual, const bf16* w,
                            float eps, bf16* h_out, bf16* y_out, hipStream_t s) {
  if (M <= 0) return hipSuccess;
  if (H <= 0 || H % 8 || H > 8192 || n < 1) return hipErrorInvalidValue;
  // rows of up to 64 (128) chunks take one (two) waves; wider rows all four
  // waves of the workgroup, up to four chunks per thread
  const int nc = H / 8;   // 1..1024
  if (nc <= 64)
    launch_norm<64, 1>(partials, n, M, H, residual, w, eps, h_out, y_out, s);
  else if (nc <= 128)
    launch_norm<128, 1>(partials, n, M, H, residual, w, eps, h_out, y_out, s);
  else
    launch_norm_tpr<256>((nc + 255) / 256, partials, n, M, H, residual, w, eps, h_out, y_out, s);
  return hipGetLastError();
}

}  // namespace tps
