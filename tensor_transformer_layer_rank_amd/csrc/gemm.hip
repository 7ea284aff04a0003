// Linear layers of the shard: C = A * B^T with B in the [out, in] layout.
//
// "Tensor parallelism from scratch", "Two ways to split": a column-parallel
// layer (q/k/v, gate/up, the vocab-split lm_head) is a GEMM over the rank's
// rows of W; a row-parallel layer (o_proj, down_proj) is a GEMM over the
// rank's columns of W, giving a partial sum.  Both are the same NT GEMM on
// the rank's local weight.  "Implementation", TPMLP: silu(gate) * up is
// elementwise on the column shard, so it is fused into the gate_up epilogue.
//
// gfx950 design: v_mfma_f32_32x32x16_bf16; A and B tiles staged through LDS
// (double-buffered, 16-byte chunks XOR-swizzled so that the 32 rows an MFMA
// operand read touches hit distinct banks); workgroup ids remapped so that
// each of the 8 XCDs (fed round-robin by the dispatcher) works on a
// contiguous, M-grouped range of tiles and shares A/B panels in its own L2.
#include "common.h"

namespace tps {

namespace {

constexpr int kXcds = 8;
constexpr int kCUs = 256;

__device__ __forceinline__ int xcd_remap(int bid, int nb) {
  const int xcd = bid % kXcds, idx = bid / kXcds;
  const int per = nb / kXcds, rem = nb % kXcds;
  return (xcd < rem ? xcd * (per + 1) : rem * (per + 1) + (xcd - rem) * per) + idx;
}

// 16-byte chunk position inside a 128-byte tile row: 16 consecutive rows
// land on 16 distinct 16-byte slots of the 256-byte bank space.
__device__ __forceinline__ int swz(int row, int chunk) { return chunk ^ ((row >> 1) & 7); }

template <int BM, int BN, int WGM, int WGN, int EPI, bool SPLIT, int GROUP_M>
__global__ __launch_bounds__(WGM * WGN * 64) void gemm_kernel(GemmProblem p, int tiles_m, int tiles_n,
                                                              int64_t k_per_split) {
  constexpr int BK = 64;
  constexpr int NT = WGM * WGN * 64;
  constexpr int WM = BM / WGM, WN = BN / WGN;
  constexpr int TM = WM / 32, TN = WN / 32;
  constexpr int KC = BK / 8;
  constexpr int A_LD = BM * KC / NT, B_LD = BN * KC / NT;
  static_assert(BM * KC % NT == 0 && BN * KC % NT == 0, "tile/threads mismatch");
  static_assert(TM >= 1 && TN >= 1, "wave tile must hold a 32x32 block");
  static_assert(EPI != EPI_SILU_BF16 || (TN % 2 == 0), "silu pairs need an even number of n-blocks");
  constexpr int STAGE = (BM + BN) * BK;
  __shared__ __attribute__((aligned(16))) bf16 smem[2 * STAGE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WGN, wn = wave % WGN;

  // tile coordinates: XCD-contiguous, then GROUP_M m-tiles per n-column sweep
  int tm, tn;
  {
    const int t = xcd_remap(blockIdx.x, gridDim.x);
    const int per_group = GROUP_M * tiles_n;
    const int g = t / per_group;
    const int first_m = g * GROUP_M;
    const int gm = min(tiles_m - first_m, GROUP_M);
    const int r = t - g * per_group;
    tm = first_m + r % gm;
    tn = r / gm;
  }
  const int64_t M = p.M, K = p.K;
  const int64_t m0 = (int64_t)tm * BM;
  int64_t kbeg = 0, kend = K;
  if (SPLIT) {
    kbeg = (int64_t)blockIdx.y * k_per_split;
    kend = min(K, kbeg + k_per_split);
  }
  const int nk = kend > kbeg ? (int)((kend - kbeg + BK - 1) / BK) : 0;

  // global row of B for tile row n (-1 = outside the matrix)
  auto b_row = [&](int n) -> int64_t {
    if (EPI == EPI_SILU_BF16) {
      const int half = n / (BN / 2);
      const int64_t hcol = (int64_t)tn * (BN / 2) + (n - half * (BN / 2));
      return hcol < p.li ? half * p.li + hcol : -1;
    }
    const int64_t r = (int64_t)tn * BN + n;
    return r < p.N ? r : -1;
  };

  // per-thread global source pointers (fixed over k); nullptr = zero fill
  const bf16* a_src[A_LD];
  const bf16* b_src[B_LD];
#pragma unroll
  for (int i = 0; i < A_LD; ++i) {
    const int q = tid + i * NT, row = q / KC, ch = q % KC;
    const int64_t gm = m0 + row;
    a_src[i] = gm < M ? p.A + gm * p.lda + ch * 8 : nullptr;
  }
#pragma unroll
  for (int i = 0; i < B_LD; ++i) {
    const int q = tid + i * NT, row = q / KC, ch = q % KC;
    const int64_t gr = b_row(row);
    b_src[i] = gr >= 0 ? p.B + gr * p.ldb + ch * 8 : nullptr;
  }

  u32x4 ra[A_LD], rb[B_LD];
  auto gload = [&](int64_t k0) {
#pragma unroll
    for (int i = 0; i < A_LD; ++i) {
      const int ch = (tid + i * NT) % KC;
      const bool ok = a_src[i] && (k0 + ch * 8 < kend);
      ra[i] = ok ? *reinterpret_cast<const u32x4*>(a_src[i] + k0) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int i = 0; i < B_LD; ++i) {
      const int ch = (tid + i * NT) % KC;
      const bool ok = b_src[i] && (k0 + ch * 8 < kend);
      rb[i] = ok ? *reinterpret_cast<const u32x4*>(b_src[i] + k0) : u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto sstore = [&](int buf) {
    bf16* sA = smem + buf * STAGE;
    bf16* sB = sA + BM * BK;
#pragma unroll
    for (int i = 0; i < A_LD; ++i) {
      const int q = tid + i * NT, row = q / KC, ch = q % KC;
      *reinterpret_cast<u32x4*>(sA + row * BK + swz(row, ch) * 8) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < B_LD; ++i) {
      const int q = tid + i * NT, row = q / KC, ch = q % KC;
      *reinterpret_cast<u32x4*>(sB + row * BK + swz(row, ch) * 8) = rb[i];
    }
  };
  // tile-local column of the j-th 32-wide n-block of this wave
  auto ncol = [&](int j) -> int {
    if (EPI == EPI_SILU_BF16)
      return j < TN / 2 ? wn * (WN / 2) + j * 32 : BN / 2 + wn * (WN / 2) + (j - TN / 2) * 32;
    return wn * WN + j * 32;
  };

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  if (nk > 0) {
    gload(kbeg);
    sstore(0);
    __syncthreads();
  }
  const int lr = lane & 31, lh = lane >> 5;
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) gload(kbeg + (int64_t)(kt + 1) * BK);
    const bf16* sA = smem + cur * STAGE;
    const bf16* sB = sA + BM * BK;
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      const int c = ks * 2 + lh;
      bf16x8 af[TM], bfr[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int row = wm * WM + i * 32 + lr;
        af[i] = *reinterpret_cast<const bf16x8*>(sA + row * BK + swz(row, c) * 8);
      }
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int row = ncol(j) + lr;
        bfr[j] = *reinterpret_cast<const bf16x8*>(sB + row * BK + swz(row, c) * 8);
      }
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) sstore(cur ^ 1);
    __syncthreads();
  }

  // epilogue: lane holds column (lane & 31) and rows 8*(e/4) + 4*(lane/32) + e%4
  if (EPI == EPI_SILU_BF16) {
    bf16* C = static_cast<bf16*>(p.C);
#pragma unroll
    for (int j = 0; j < TN / 2; ++j) {
      const int64_t hcol = (int64_t)tn * (BN / 2) + wn * (WN / 2) + j * 32 + lr;
      if (hcol >= p.li) continue;
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int64_t gm = m0 + wm * WM + i * 32 + 8 * (e >> 2) + 4 * lh + (e & 3);
          if (gm < M) {
            const float g = acc[i][j][e], u = acc[i][j + TN / 2][e];
            C[gm * p.ldc + hcol] = f2bf(g / (1.f + __expf(-g)) * u);
          }
        }
    }
  } else {
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int64_t gn = (int64_t)tn * BN + ncol(j) + lr;
      if (gn >= p.N) continue;
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int64_t gm = m0 + wm * WM + i * 32 + 8 * (e >> 2) + 4 * lh + (e & 3);
          if (gm >= M) continue;
          if (EPI == EPI_BF16) {
            static_cast<bf16*>(p.C)[gm * p.ldc + gn] = f2bf(acc[i][j][e]);
          } else {
            float* C = static_cast<float*>(p.C) + (SPLIT ? (int64_t)blockIdx.y * M * p.ldc : 0);
            C[gm * p.ldc + gn] = acc[i][j][e];
          }
        }
    }
  }
}

// Sums split-K partials [splits, M, N] in a fixed order and applies the
// final epilogue.
template <int EPI>
__global__ __launch_bounds__(256) void splitk_reduce(const float* __restrict__ part, int splits, int64_t M,
                                                     int64_t N, void* out, int64_t ldc, int64_t li) {
  const int64_t cols = EPI == EPI_SILU_BF16 ? li : N;
  const int64_t total = M * cols;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256) {
    const int64_t m = i / cols, n = i - m * cols;
    if (EPI == EPI_SILU_BF16) {
      float g = 0.f, u = 0.f;
      for (int z = 0; z < splits; ++z) {
        g += part[((int64_t)z * M + m) * N + n];
        u += part[((int64_t)z * M + m) * N + li + n];
      }
      static_cast<bf16*>(out)[m * ldc + n] = f2bf(g / (1.f + __expf(-g)) * u);
    } else {
      float s = 0.f;
      for (int z = 0; z < splits; ++z) s += part[((int64_t)z * M + m) * N + n];
      if (EPI == EPI_BF16)
        static_cast<bf16*>(out)[m * ldc + n] = f2bf(s);
      else
        static_cast<float*>(out)[m * ldc + n] = s;
    }
  }
}

// ---- tile-shape choice -----------------------------------------------------

enum TileCfg { TILE_256x256 = 0, TILE_128x128 = 1, TILE_64x128 = 2, TILE_128x64 = 3, TILE_COUNT };
struct TileShape { int bm, bn; float eff; };
constexpr TileShape kShapes[TILE_COUNT] = {{256, 256, 1.0f}, {128, 128, 0.75f}, {64, 128, 0.5f}, {128, 64, 0.5f}};

struct Plan { int tile; int splits; int64_t kps; int tiles_m, tiles_n; };

Plan make_plan(int64_t M, int64_t N, int64_t K, int epi, bool allow_split) {
  const int64_t ncols = epi == EPI_SILU_BF16 ? N / 2 : N;   // output columns
  Plan best{TILE_256x256, 1, K, 0, 0};
  double best_cost = 1e300;
  for (int t = 0; t < TILE_COUNT; ++t) {
    const TileShape s = kShapes[t];
    const int64_t bn_out = epi == EPI_SILU_BF16 ? s.bn / 2 : s.bn;
    const int64_t tm = (M + s.bm - 1) / s.bm, tn = (ncols + bn_out - 1) / bn_out;
    const int64_t tiles = tm * tn;
    const int64_t waves = (tiles + kCUs - 1) / kCUs;
    const double cost = (double)waves * s.bm * s.bn / s.eff;
    if (cost < best_cost * 0.999) {
      best_cost = cost;
      best = Plan{t, 1, K, (int)tm, (int)tn};
    }
  }
  // Split K when the grid cannot fill the GPU and K is long enough to share.
  const int64_t tiles = (int64_t)best.tiles_m * best.tiles_n;
  // fp32 partials cost splits*M*N*8 bytes of traffic against the N*K*2
  // bytes of B, so the split count is capped at K / (8 M) (<= half of it).
  if (allow_split && tiles < kCUs && K >= 512) {
    int64_t splits = (2 * kCUs + tiles - 1) / tiles;
    const int64_t kblocks = K / 64;
    const int64_t cap = K / (8 * M);
    if (splits > cap) splits = cap;
    if (splits > kblocks) splits = kblocks;
    if (splits > 1) {
      // split-K re-reads nothing but writes fp32 partials; the tile is
      // computed with the plain [gate; up] column order in that case
      const int64_t kps = ((K / 64 + splits - 1) / splits) * 64;
      splits = (K + kps - 1) / kps;
      if (splits > 1) {
        const TileShape s = kShapes[best.tile];
        best.tiles_n = (int)((N + s.bn - 1) / s.bn);
        best.splits = (int)splits;
        best.kps = kps;
      }
    }
  }
  return best;
}

template <int BM, int BN, int WGM, int WGN>
hipError_t launch_tile(const GemmProblem& p, int epi, const Plan& pl, void* scratch, hipStream_t s) {
  constexpr int NT = WGM * WGN * 64;
  constexpr int GM = 8;
  if (pl.splits > 1) {
    GemmProblem q = p;
    q.C = scratch;
    q.ldc = p.N;
    dim3 grid(pl.tiles_m * pl.tiles_n, pl.splits);
    gemm_kernel<BM, BN, WGM, WGN, EPI_F32, true, GM><<<grid, NT, 0, s>>>(q, pl.tiles_m, pl.tiles_n, pl.kps);
    const int64_t cols = epi == EPI_SILU_BF16 ? p.li : p.N;
    int64_t g = (p.M * cols + 255) / 256;
    if (g > 4096) g = 4096;
    if (epi == EPI_SILU_BF16)
      splitk_reduce<EPI_SILU_BF16><<<(int)g, 256, 0, s>>>((const float*)scratch, pl.splits, p.M, p.N, p.C, p.ldc, p.li);
    else if (epi == EPI_BF16)
      splitk_reduce<EPI_BF16><<<(int)g, 256, 0, s>>>((const float*)scratch, pl.splits, p.M, p.N, p.C, p.ldc, 0);
    else
      splitk_reduce<EPI_F32><<<(int)g, 256, 0, s>>>((const float*)scratch, pl.splits, p.M, p.N, p.C, p.ldc, 0);
    return hipGetLastError();
  }
  dim3 grid(pl.tiles_m * pl.tiles_n);
  if (epi == EPI_SILU_BF16)
    gemm_kernel<BM, BN, WGM, WGN, EPI_SILU_BF16, false, GM><<<grid, NT, 0, s>>>(p, pl.tiles_m, pl.tiles_n, p.K);
  else if (epi == EPI_BF16)
    gemm_kernel<BM, BN, WGM, WGN, EPI_BF16, false, GM><<<grid, NT, 0, s>>>(p, pl.tiles_m, pl.tiles_n, p.K);
  else
    gemm_kernel<BM, BN, WGM, WGN, EPI_F32, false, GM><<<grid, NT, 0, s>>>(p, pl.tiles_m, pl.tiles_n, p.K);
  return hipGetLastError();
}

// fp32: one thread per output element; silu_li > 0 selects silu(gate)*up
// with gate rows [0, li) and up rows [li, 2 li) of B.
__global__ __launch_bounds__(256) void gemm_f32_kernel(const float* __restrict__ A, const float* __restrict__ B,
                                                       float* __restrict__ C, int64_t M, int64_t N, int64_t K,
                                                       int64_t silu_li) {
  const int64_t cols = silu_li > 0 ? silu_li : N;
  const int64_t total = M * cols;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256) {
    const int64_t m = i / cols, n = i - m * cols;
    const float* a = A + m * K;
    if (silu_li > 0) {
      const float* g = B + n * K;
      const float* u = B + (silu_li + n) * K;
      float sg = 0.f, su = 0.f;
      for (int64_t k = 0; k < K; ++k) {
        sg = fmaf(a[k], g[k], sg);
        su = fmaf(a[k], u[k], su);
      }
      C[m * cols + n] = sg / (1.f + expf(-sg)) * su;
    } else {
      const float* b = B + n * K;
      float s = 0.f;
      for (int64_t k = 0; k < K; ++k) s = fmaf(a[k], b[k], s);
      C[m * cols + n] = s;
    }
  }
}

}  // namespace

size_t gemm_scratch_bytes(int64_t M, int64_t N, int64_t K, int epi) {
  if (M <= 0 || N <= 0) return 0;
  const Plan pl = make_plan(M, N, K, epi, true);
  return pl.splits > 1 ? (size_t)pl.splits * M * N * sizeof(float) : 0;
}

hipError_t gemm_bf16(const GemmProblem& p, int epi, void* scratch, size_t scratch_bytes, hipStream_t s) {
  if (p.M <= 0 || p.N <= 0) return hipSuccess;
  const bool can_split = scratch != nullptr && scratch_bytes >= gemm_scratch_bytes(p.M, p.N, p.K, epi);
  const Plan pl = make_plan(p.M, p.N, p.K, epi, can_split);
  switch (pl.tile) {
    case TILE_256x256: return launch_tile<256, 256, 2, 2>(p, epi, pl, scratch, s);
    case TILE_128x128: return launch_tile<128, 128, 2, 2>(p, epi, pl, scratch, s);
    case TILE_64x128: return launch_tile<64, 128, 2, 2>(p, epi, pl, scratch, s);
    default: return launch_tile<128, 64, 4, 1>(p, epi, pl, scratch, s);
  }
}

hipError_t gemm_f32(const float* A, const float* B, float* C, int64_t M, int64_t N, int64_t K, int silu_li,
                    hipStream_t s) {
  const int64_t cols = silu_li > 0 ? silu_li : N;
  if (M <= 0 || cols <= 0) return hipSuccess;
  int64_t g = (M * cols + 255) / 256;
  if (g > 8192) g = 8192;
  gemm_f32_kernel<<<(int)g, 256, 0, s>>>(A, B, C, M, N, K, silu_li);
  return hipGetLastError();
}

}  // namespace tps
