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
// On one GPU the ranks' partials arrive stacked (partial r of row m at
// partials + r * plane + m * H) and are summed here in rank order (fp32,
// residual first), in the same pass as the add and the norm.  The
// sequence-parallel form ("Exercises", sequence parallelism) is the same pass
// over the rank's token slice: plane stays the full M * H, the row pointers
// start at the slice.  The threads of a row keep it in registers between the sum and
// the scaling: every input byte is read once and each output written once.
//
// With no partials it is the plain RMSNorm, and with a row list it reads
// input row in_rows[m] for output row m: the final norm on each sequence's
// last position before the head ("Implementation", TPTransformer.forward
// norms x[:, -1:]).
#include "common.h"

namespace tps {

namespace {

// TPR threads per row (one wave up to a 1024-thread workgroup), NC 16-byte
// chunks per thread: H <= TPR * NC * 8.  A workgroup holds max(TPR, 256)
// threads, so up to four rows.  The partials are read G at a time, all G
// loads in flight together; G shrinks as the chunks per thread grow so that
// the loads fit in registers.
template <int NC>
constexpr int norm_group() { return NC == 1 ? 16 : NC == 2 ? 8 : 4; }

template <int TPR, int NC>
__global__ __launch_bounds__(TPR > 256 ? TPR : 256) void residual_rmsnorm_kernel(NormArgs a) {
  constexpr int BLOCK = TPR > 256 ? TPR : 256, ROWS = BLOCK / TPR, G = norm_group<NC>();
  const bf16* __restrict__ partials = a.partials;
  const bf16* residual = a.residual;
  const bf16* __restrict__ w = a.w;
  bf16* h_out = a.h_out;
  bf16* __restrict__ y_out = a.y_out;
  const int n = a.n, H = a.H;
  const int64_t plane = a.plane, M = a.M;
  const int t = threadIdx.x % TPR;
  const int64_t m = (int64_t)blockIdx.x * ROWS + threadIdx.x / TPR;
  const bool live = m < M;
  const int nc = H / 8;
  const int64_t row = (live ? m : 0) * H;
  // input row: m, or in_rows[m] (outside [0, in_nrows): a zero row)
  int64_t src = live ? m : 0;
  bool in_ok = live;
  if (a.in_rows && live) {
    src = a.in_rows[m];
    in_ok = src >= 0 && src < a.in_nrows;
    if (!in_ok) src = 0;
  }
  const int64_t irow = src * H;
  bool on[NC], ld[NC];
#pragma unroll
  for (int k = 0; k < NC; ++k) {
    on[k] = live && t + k * TPR < nc;
    ld[k] = on[k] && in_ok;
  }
  // residual, norm weight and the first group of partials are all
  // requested before the first use of any of them
  bf16x8 rv[NC], wv[NC], v[G][NC];
#pragma unroll
  for (int k = 0; k < NC; ++k) {
    rv[k] = bf16x8{};
    if (ld[k]) rv[k] = *reinterpret_cast<const bf16x8*>(residual + irow + (int64_t)(t + k * TPR) * 8);
    if (on[k]) wv[k] = *reinterpret_cast<const bf16x8*>(w + (int64_t)(t + k * TPR) * 8);
  }
  float acc[NC][8];
#pragma unroll
  for (int k = 0; k < NC; ++k)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[k][e] = ld[k] ? bf2f(rv[k][e]) : 0.f;
  for (int r0 = 0; r0 < n; r0 += G) {
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int k = 0; k < NC; ++k)
        if (r0 + g < n && ld[k])
          v[g][k] = *reinterpret_cast<const bf16x8*>(partials + (int64_t)(r0 + g) * plane + irow +
                                                     (int64_t)(t + k * TPR) * 8);
#pragma unroll
    for (int g = 0; g < G; ++g)   // rank order
      if (r0 + g < n)
#pragma unroll
        for (int k = 0; k < NC; ++k)
          if (ld[k])
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
      if (h_out) __builtin_nontemporal_store(hb, reinterpret_cast<bf16x8*>(h_out + row + (int64_t)(t + k * TPR) * 8));
    }
  }
  ss = wave_sum64(ss);
  if constexpr (TPR > 64) {
    __shared__ float s_ss[BLOCK / 64];
    if ((threadIdx.x & 63) == 0) s_ss[threadIdx.x >> 6] = ss;
    __syncthreads();
    const int w0 = (threadIdx.x / TPR) * (TPR / 64);
    ss = 0.f;
#pragma unroll
    for (int i = 0; i < TPR / 64; ++i) ss += s_ss[w0 + i];
  }
  const float inv = 1.0f / sqrtf(ss / (float)H + a.eps);
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
void launch_norm(const NormArgs& a, hipStream_t s) {
  constexpr int BLOCK = TPR > 256 ? TPR : 256, ROWS = BLOCK / TPR;
  const unsigned grid = (unsigned)((a.M + ROWS - 1) / ROWS);
  residual_rmsnorm_kernel<TPR, NC><<<grid, BLOCK, 0, s>>>(a);
}

template <int TPR>
void launch_norm_tpr(int nc_per, const NormArgs& a, hipStream_t s) {
  switch (nc_per) {
    case 1: launch_norm<TPR, 1>(a, s); break;
    case 2: launch_norm<TPR, 2>(a, s); break;
    case 3: launch_norm<TPR, 3>(a, s); break;
    default: launch_norm<TPR, 4>(a, s); break;
  }
}

}  // namespace

int norm_threads_per_row(int64_t M, int H) {
  const int nc = H / 8;
  int tpr = 64;
  while (tpr * 4 < nc) tpr *= 2;   // at most four chunks per thread
  // few rows: spread each over more waves until the launch has ~8 waves per
  // CU or a thread per chunk
  while (tpr < 1024 && tpr < nc && M * (tpr / 64) < 8 * kCUs) tpr *= 2;
  return tpr;
}

hipError_t residual_rmsnorm(const NormArgs& a, hipStream_t s) {
  if (a.M <= 0) return hipSuccess;
  if (a.H <= 0 || a.H % 8 || a.H > 8192 || a.n < 0 || (a.n > 0 && !a.partials) || (a.n > 0 && !a.h_out))
    return hipErrorInvalidValue;
  const int nc = a.H / 8;   // 1..1024
  const int tpr = norm_threads_per_row(a.M, a.H);
  const int per = (nc + tpr - 1) / tpr;   // 1..4
  switch (tpr) {
    case 64: launch_norm_tpr<64>(per, a, s); break;
    case 128: launch_norm_tpr<128>(per, a, s); break;
    case 256: launch_norm_tpr<256>(per, a, s); break;
    case 512: launch_norm_tpr<512>(per, a, s); break;
    default: launch_norm_tpr<1024>(per, a, s); break;
  }
  kmark(s, a.in_rows ? "rmsnorm_rows" : a.n ? "residual_rmsnorm" : "rmsnorm");
  return hipGetLastError();
}

}  // namespace tps
