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
#include <mutex>
#include <type_traits>

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

// ---- decode head with the rows resident on chip ---------------------------
// For a few rows and a short hidden size (M <= 64, K = 256, 512, 768 or
// 1024) the activations stay on chip for the whole launch and the vocab slice
// is streamed once, straight into MFMA registers (16x16x32 products: one load
// instruction reads 16 vocab rows x 64 contiguous bytes); no logits tile is
// staged.  A workgroup (one per CU) runs a contiguous run of whole 16-row
// vocab chunks; its four waves split K into quarters, so each wave keeps its
// quarter of the rows (MQ 16-row groups x KS k-steps of 32) in VGPRs, and all
// four work on the same chunk.  Their partial products meet in LDS
// (double-buffered, one barrier per chunk); wave w then sums the four
// partials of row group w in K order -- the MFMA output layout, so lane
// (l16, g) owns rows 16w + 4g + e at chunk column l16 -- and keeps the
// running best (value, column) of the bf16-rounded logits, as the GEMM
// epilogue compares them.  At the end each row's 16 column slots reduce to
// one candidate per (row, workgroup).
// The loads are unconditional: past the run (and past N) their offsets fall
// outside the descriptors' ranges and load zeros without a memory access,
// so no branch disturbs the compiler's wait counts; a scheduling barrier
// after each chunk's loads keeps chunks in issue order.
constexpr int kResSegK = 256;                // K granularity of the head

template <int MQ, int KS, int NB>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void argmax_resident_kernel(const bf16* __restrict__ x, int64_t M, const int32_t* __restrict__ rows,
                            int64_t x_rows, const bf16* __restrict__ vocab, int64_t N, u32x2* __restrict__ cand) {
  constexpr int K = KS * 128;                 // 4 waves x KS steps x 32
  // rows padded to 20 floats: the four 16-lane groups of a wave write rows 4
  // apart, which then start 16 banks apart instead of on the same banks
  __shared__ float red[2][4][16 * MQ][20];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, g = lane >> 4;
  const int kw0 = wave * (K / 4);             // this wave's K quarter
  // the rows' fragments of this quarter: row r, or x row rows[r] with a row
  // list; rows past M and indices outside x read as zeros (past the range)
  const __amdgpu_buffer_rsrc_t rx =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16*>(x), (short)0, (int)((rows ? x_rows : M) * K * 2), 0x00020000);
  uint32_t xoff[MQ];
#pragma unroll
  for (int i = 0; i < MQ; ++i) {
    const int r = i * 16 + l16;
    int64_t src = r < M ? r : -1;
    if (rows && r < M) src = rows[r] >= 0 && rows[r] < x_rows ? rows[r] : -1;
    xoff[i] = src >= 0 ? (uint32_t)(src * K + kw0 + g * 8) * 2u : 0x80000000u;
  }
  bf16x8 af[KS][MQ];
#pragma unroll
  for (int s = 0; s < KS; ++s)
#pragma unroll
    for (int i = 0; i < MQ; ++i)
      af[s][i] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rx, xoff[i] + s * 64u, 0, 0));
  // this workgroup's run of whole 16-row chunks
  const int64_t nch = (N + 15) / 16;
  const int c0 = (int)(nch * blockIdx.x / gridDim.x), c1 = (int)(nch * (blockIdx.x + 1) / gridDim.x);
  const int n = c1 - c0;
  const __amdgpu_buffer_rsrc_t rb =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16*>(vocab), (short)0, (int)(N * K * 2), 0x00020000);
  u32x4 bfr[NB][KS];
  auto load_chunk = [&](int j, u32x4 (&b)[KS]) __attribute__((always_inline)) {
    const uint32_t off = j < n ? (uint32_t)(((c0 + j) * 16 + l16) * K + kw0 + g * 8) * 2u : 0x80000000u;
#pragma unroll
    for (int s = 0; s < KS; ++s)
      b[s] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rb, off + s * 64u, 0, 0));
    __builtin_amdgcn_sched_barrier(0);
  };
  float bv[4];
  int bi[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    bv[e] = -INFINITY;
    bi[e] = -1;
  }
  auto chunk = [&](int j, const u32x4 (&b)[KS]) __attribute__((always_inline)) {
    f32x4 acc[MQ];
#pragma unroll
    for (int i = 0; i < MQ; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const bf16x8 bb = __builtin_bit_cast(bf16x8, b[s]);
#pragma unroll
      for (int i = 0; i < MQ; ++i) acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[s][i], bb, acc[i], 0, 0, 0);
    }
    float (*rr)[16 * MQ][20] = red[j & 1];
#pragma unroll
    for (int i = 0; i < MQ; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) rr[wave][i * 16 + 4 * g + e][l16] = acc[i][e];
    __syncthreads();
    if (wave < MQ) {
      const int col = (c0 + j) * 16 + l16;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = wave * 16 + 4 * g + e;
        const float sum = ((rr[0][r][l16] + rr[1][r][l16]) + rr[2][r][l16]) + rr[3][r][l16];   // K order
        const float v = bf2f(f2bf(sum));
        const bool take = col < N && cand_better(v, col, bv[e], bi[e]);
        bv[e] = take ? v : bv[e];
        bi[e] = take ? col : bi[e];
      }
    }
  };
#pragma unroll
  for (int p = 0; p < NB - 1; ++p) load_chunk(p, bfr[p]);
  for (int j = 0; j < n; j += NB) {
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      load_chunk(j + u + NB - 1, bfr[(u + NB - 1) % NB]);
      if (j + u < n) chunk(j + u, bfr[u]);
    }
  }
  if (wave < MQ) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float v = bv[e];
      int id = bi[e];
      cand_best16(v, id);
      const int r = wave * 16 + 4 * g + e;
      if (l16 == 0 && r < M) cand[(int64_t)r * gridDim.x + blockIdx.x] = u32x2{__float_as_uint(v), (uint32_t)id};
    }
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

hipError_t argmax_resident(const void* x, int64_t M, const int32_t* rows, int64_t x_rows, const void* vocab,
                           int64_t N, int64_t K, void* cand, hipStream_t s) {
  if (!argmax_resident_ok(M, N, K)) return hipErrorInvalidValue;
  const bf16* xb = static_cast<const bf16*>(x);
  const bf16* vb = static_cast<const bf16*>(vocab);
  u32x2* cb = static_cast<u32x2*>(cand);
  // chunks in flight per wave from a sweep on the 75968 x 1024 slice
  auto go = [&](auto ks) {
    constexpr int KS = decltype(ks)::value;
    if (M <= 16)
      argmax_resident_kernel<1, KS, 3><<<kCUs, 256, 0, s>>>(xb, M, rows, x_rows, vb, N, cb);
    else if (M <= 32)
      argmax_resident_kernel<2, KS, 3><<<kCUs, 256, 0, s>>>(xb, M, rows, x_rows, vb, N, cb);
    else
      argmax_resident_kernel<4, KS, 2><<<kCUs, 256, 0, s>>>(xb, M, rows, x_rows, vb, N, cb);
  };
  switch (K) {
    case 256: go(std::integral_constant<int, 2>{}); break;
    case 512: go(std::integral_constant<int, 4>{}); break;
    case 768: go(std::integral_constant<int, 6>{}); break;
    default: go(std::integral_constant<int, 8>{}); break;
  }
  kmark(s, "argmax_resident");
  return hipGetLastError();
}

hipError_t argmax_candidates(const void* cand, int64_t M, int64_t n, int64_t idx0, float* out_val, int32_t* out_idx,
                             hipStream_t s) {
  if (M <= 0) return hipSuccess;
  argmax_pairs<<<(unsigned)M, 256, 0, s>>>(static_cast<const u32x2*>(cand), n, idx0, out_val, out_idx);
  kmark(s, "argmax_pairs");
  return hipGetLastError();
}

// ---- the decode head's candidates without an allocation --------------------
// A file-scope device array holds the candidates for callers that cannot
// allocate (graph capture, tight serving loops).  In host code `scratch`
// names a host-side stand-in, not the device copy: its device address is
// looked up once per device with that device current, and only that address
// is handed to kernels.  Every call on a device shares the device's array.
namespace {
__device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t noalloc_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

hipError_t argmax_combine(const float* vals, const int32_t* idx, int n_shards, int64_t M, int32_t* out_idx,
                          float* out_val, hipStream_t s) {
  if (M <= 0) return hipSuccess;
  int64_t g = (M + 255) / 256;
  if (g > 1024) g = 1024;
  combine_candidates<<<(unsigned)g, 256, 0, s>>>(vals, idx, n_shards, M, out_idx, out_val);
  kmark(s, "combine_candidates");
  return hipGetLastError();
}

}  // namespace tps
