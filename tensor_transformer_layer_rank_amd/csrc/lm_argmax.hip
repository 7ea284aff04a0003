// Greedy next token over vocab-parallel logits ("Tensor parallelism from
// scratch", "Implementation": the decode loop takes the argmax of the last
// position's logits, which the vocab-split output layer produces a slice of
// per rank before the all-gather).  Instead of gathering V logits per row,
// each rank reduces its slice to one candidate (max, first global index of
// it), and the candidates of all ranks combine to the max, ties to the
// smaller global index -- the first maximum of the concatenated logits.
//
// The logits never reach memory.  Up to 64 rows with a hidden size of at
// most 1024 go to argmax_resident_kernel (below: rows resident in LDS, the
// vocab slice streamed once); other shapes to the logits GEMM, which reduces
// each tile row to a candidate in its epilogue (EPI_ARGMAX in gemm.hip).
// argmax_pairs: one workgroup per row reduces the row's candidates (a
// per-thread best, then wave shuffles and LDS).  combine_candidates: one
// thread per row over the ranks.
#include "common.h"

namespace tps {

namespace {

// better candidate: larger value, or equal value and smaller index; an
// index < 0 marks "none"
__device__ __forceinline__ bool better(float v, int i, float bv, int bi) { return cand_better(v, i, bv, bi); }

// best of 256 threads' (value, column) pairs -> thread 0
__device__ __forceinline__ void block_best(float& bv, int& bi) {
  cand_best64(bv, bi);
  __shared__ float s_v[4];
  __shared__ int s_i[4];
  const int tid = threadIdx.x;
  if ((tid & 63) == 0) {
    s_v[tid >> 6] = bv;
    s_i[tid >> 6] = bi;
  }
  __syncthreads();
  if (tid == 0) {
    for (int w = 1; w < 4; ++w)
      if (better(s_v[w], s_i[w], bv, bi)) {
        bv = s_v[w];
        bi = s_i[w];
      }
  }
}

__global__ __launch_bounds__(256) void argmax_pairs(const u32x2* __restrict__ cand, int64_t n, int64_t idx0,
                                                    float* __restrict__ out_val, int32_t* __restrict__ out_idx) {
  const int64_t m = blockIdx.x;
  float bv = -INFINITY;
  int bi = -1;
  for (int64_t t = threadIdx.x; t < n; t += 256) {
    const u32x2 c = cand[m * n + t];
    const float v = __uint_as_float(c[0]);
    const int i = (int)c[1];
    if (better(v, i, bv, bi)) {
      bv = v;
      bi = i;
    }
  }
  block_best(bv, bi);
  if (threadIdx.x == 0) {
    out_val[m] = bi < 0 ? -INFINITY : bv;
    out_idx[m] = bi < 0 ? -1 : (int32_t)(idx0 + bi);
  }
}

__global__ __launch_bounds__(256) void combine_candidates(const float* __restrict__ vals,
                                                          const int32_t* __restrict__ idx, int n_shards,
                                                          int64_t M, int32_t* __restrict__ out_idx,
                                                          float* __restrict__ out_val) {
  for (int64_t m = (int64_t)blockIdx.x * 256 + threadIdx.x; m < M; m += (int64_t)gridDim.x * 256) {
    float bv = -INFINITY;
    int bi = -1;
    for (int r = 0; r < n_shards; ++r) {
      const float v = vals[(int64_t)r * M + m];
      const int i = idx[(int64_t)r * M + m];
      if (better(v, i, bv, bi)) {
        bv = v;
        bi = i;
      }
    }
    out_idx[m] = bi;
    if (out_val) out_val[m] = bv;
  }
}

// ---- decode head with the rows resident in LDS ---------------------------
// For a few rows and a short hidden size (M <= 64, K <= 1024, K % 256 == 0)
// the rows fit in LDS (at most 128 KB), so every workgroup keeps them for
// the whole launch and each wave streams a contiguous run of whole 16-row
// chunks of the vocab slice straight from memory into MFMA registers: the
// slice is read once, the activations once per workgroup.  16x16x32
// products, so one load instruction reads 16 vocab rows x 64 contiguous
// bytes.  Per lane the best (value, column) of each row is kept across the
// run; lanes and waves combine at the end into one candidate per
// (row, workgroup).  Values compare as the bf16-rounded logits, as in the
// GEMM epilogue.
// NW: waves per workgroup; NB: operand buffers (NB - 1 steps of loads in
// flight while one computes); MQ: 16-row groups of the activations.  A step
// is 8 k-steps of 32 (256 of K).
constexpr int kResSegK = 256;

__device__ __forceinline__ int res_swz(int row, int chunk) { return chunk ^ (row & 15); }

template <int NW, int NB, int MQ>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(NW / 4, NW / 4)))
void argmax_resident_kernel(const bf16* __restrict__ x, int64_t M, const bf16* __restrict__ vocab, int64_t N, int K,
                            u32x2* __restrict__ cand) {
  constexpr int RW = 16 * MQ;
  __shared__ __attribute__((aligned(16))) bf16 sa[RW * 1024];  // rows x K, 16-byte chunks XOR-swizzled by row
  __shared__ float s_v[NW][RW];
  __shared__ int s_i[NW][RW];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, g = lane >> 4;
  const int kc = K / 8;                      // 16-byte chunks per row
  // 1. the rows into LDS (rows past M as zeros), eight loads in flight per
  // thread before their stores
  constexpr int NT = 64 * NW, UNR = 8;
  for (int q0 = tid; q0 < RW * kc; q0 += NT * UNR) {
    u32x4 v[UNR];
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int q = q0 + u * NT;
      const int r = q / kc, p = q - r * kc;
      v[u] = q < RW * kc && r < M ? *reinterpret_cast<const u32x4*>(x + (int64_t)r * K + res_swz(r, p) * 8)
                                  : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int q = q0 + u * NT;
      const int r = q / kc, p = q - r * kc;
      if (q < RW * kc) *reinterpret_cast<u32x4*>(sa + r * K + p * 8) = v[u];
    }
  }
  __syncthreads();

  // 2. this wave's run [r0, r0 + nrows) of whole 16-row chunks (only the last
  // run of the slice is ragged).  One descriptor spans the slice, built from
  // the arguments alone so that it stays in scalar registers; its range check
  // zero-fills the rows past N, and steps past the run take an offset beyond
  // the range, which loads zeros without a memory access.
  const int64_t gw = (int64_t)blockIdx.x * NW + wave, nw = (int64_t)gridDim.x * NW;
  const int64_t nch = (N + 15) / 16;
  const int c0 = (int)(nch * gw / nw), c1 = (int)(nch * (gw + 1) / nw);
  const int r0 = 16 * c0;
  const int nrows = (int)min(N, (int64_t)16 * c1) - r0;
  const __amdgpu_buffer_rsrc_t rb =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16*>(vocab), (short)0, (int)(N * K * 2), 0x00020000);
  const int nseg = K / kResSegK;
  const int steps = (c1 - c0) * nseg;         // (chunk of 16 rows, K segment)
  float bv[MQ][4];
  int bi[MQ][4];
  f32x4 acc[MQ];
#pragma unroll
  for (int i = 0; i < MQ; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      bv[i][e] = -INFINITY;
      bi[i][e] = -1;
      acc[i][e] = 0.f;
    }
  u32x4 bfr[NB][8];
  auto load_step = [=](int t, u32x4 (&b)[8]) __attribute__((always_inline)) {
    const int ch = t / nseg, seg = t - ch * nseg;
    const uint32_t off = t < steps ? (uint32_t)((r0 + ch * 16 + l16) * K + seg * kResSegK + g * 8) * 2u : 0x80000000u;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
      b[ks] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rb, off + ks * 64u, 0, 0));
    // steps issue in order: a later step's load moved ahead of an earlier
    // one makes the wait for the earlier one drain the queue
    __builtin_amdgcn_sched_barrier(0);
  };
  auto compute_step = [&](int t, const u32x4 (&b)[8]) __attribute__((always_inline)) {
    const int ch = t / nseg, seg = t - ch * nseg;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const int c = seg * (kResSegK / 8) + ks * 4 + g;
      const bf16x8 bb = __builtin_bit_cast(bf16x8, b[ks]);
#pragma unroll
      for (int i = 0; i < MQ; ++i) {
        const int row = i * 16 + l16;
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(sa + row * K + res_swz(row, c) * 8);
        acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bb, acc[i], 0, 0, 0);
      }
    }
    if (seg == nseg - 1) {                   // the chunk's logits are complete
      const int col = ch * 16 + l16;         // row of the wave's run
      const int gcol = r0 + col;
#pragma unroll
      for (int i = 0; i < MQ; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float v = bf2f(f2bf(acc[i][e]));
          const bool take = col < nrows && cand_better(v, gcol, bv[i][e], bi[i][e]);
          bv[i][e] = take ? v : bv[i][e];
          bi[i][e] = take ? gcol : bi[i][e];
          acc[i][e] = 0.f;
        }
    }
  };
  // The loads are unconditional (past the run they load zeros without a
  // memory access): with no branch around them the compiler's wait counts
  // stay exact, where a conditional load makes later waits drain the queue.
#pragma unroll
  for (int p = 0; p < NB - 1; ++p) load_step(p, bfr[p]);
  for (int t = 0; t < steps; t += NB) {
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      load_step(t + u + NB - 1, bfr[(u + NB - 1) % NB]);
      if (t + u < steps) compute_step(t + u, bfr[u]);
    }
  }

  // 3. lanes (the 16 of a row group), then waves, to one candidate per row
#pragma unroll
  for (int i = 0; i < MQ; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float v = bv[i][e];
      int id = bi[i][e];
      cand_best16(v, id);
      if (l16 == 0) {
        s_v[wave][i * 16 + 4 * g + e] = v;
        s_i[wave][i * 16 + 4 * g + e] = id;
      }
    }
  __syncthreads();
  if (tid < RW && tid < M) {
    float v = s_v[0][tid];
    int id = s_i[0][tid];
    for (int w = 1; w < NW; ++w)
      if (cand_better(s_v[w][tid], s_i[w][tid], v, id)) {
        v = s_v[w][tid];
        id = s_i[w][tid];
      }
    cand[(int64_t)tid * gridDim.x + blockIdx.x] = u32x2{__float_as_uint(v), (uint32_t)id};
  }
}

}  // namespace

bool argmax_resident_ok(int64_t M, int64_t N, int64_t K) {
  // offsets into the slice are 32-bit with the top bit free for the
  // out-of-range marker
  return M >= 1 && M <= 64 && N >= 1 && K >= kResSegK && K <= 1024 && K % kResSegK == 0 &&
         N * K * 2 < ((int64_t)1 << 31);
}

int argmax_resident_groups() { return kCUs; }

hipError_t argmax_resident(const void* x, int64_t M, const void* vocab, int64_t N, int64_t K, void* cand,
                           hipStream_t s) {
  if (!argmax_resident_ok(M, N, K)) return hipErrorInvalidValue;
  const bf16* xb = static_cast<const bf16*>(x);
  const bf16* vb = static_cast<const bf16*>(vocab);
  u32x2* cb = static_cast<u32x2*>(cand);
  // wave count and pipeline depth from a sweep on the 75968 x 1024 slice
  if (M <= 16)
    argmax_resident_kernel<4, 3, 1><<<kCUs, 256, 0, s>>>(xb, M, vb, N, (int)K, cb);
  else if (M <= 32)
    argmax_resident_kernel<8, 2, 2><<<kCUs, 512, 0, s>>>(xb, M, vb, N, (int)K, cb);
  else
    argmax_resident_kernel<8, 2, 4><<<kCUs, 512, 0, s>>>(xb, M, vb, N, (int)K, cb);
  return hipGetLastError();
}

hipError_t argmax_candidates(const void* cand, int64_t M, int64_t n, int64_t idx0, float* out_val, int32_t* out_idx,
                             hipStream_t s) {
  if (M <= 0) return hipSuccess;
  argmax_pairs<<<(unsigned)M, 256, 0, s>>>(static_cast<const u32x2*>(cand), n, idx0, out_val, out_idx);
  return hipGetLastError();
}

hipError_t argmax_combine(const float* vals, const int32_t* idx, int n_shards, int64_t M, int32_t* out_idx,
                          float* out_val, hipStream_t s) {
  if (M <= 0) return hipSuccess;
  int64_t g = (M + 255) / 256;
  if (g > 1024) g = 1024;
  combine_candidates<<<(unsigned)g, 256, 0, s>>>(vals, idx, n_shards, M, out_idx, out_val);
  return hipGetLastError();
}

}  // namespace tps
