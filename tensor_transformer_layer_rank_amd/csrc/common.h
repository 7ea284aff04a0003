// Internal declarations shared by the HIP translation units of libtpshard.
// gfx950 (CDNA4) only: wave64, MFMA bf16 32x32x16, 160 KB LDS per CU.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

namespace tps {

constexpr int kCUs = 256;   // compute units (8 XCDs x 32)

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf2f(bf16 v) { return (float)v; }

// Cross-lane sums without LDS round trips: DPP lane permutations inside each
// 16-lane row (xor 1 and xor 2 as quad permutes, then the 8- and 16-lane
// mirrors, each pairing a lane with one of the other half), then the gfx950
// row-pair and half-wave swaps.  Every lane receives the sum.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float row_sum16(float v) {
  v += dpp_f<0xB1>(v);    // quad_perm [1,0,3,2]
  v += dpp_f<0x4E>(v);    // quad_perm [2,3,0,1]
  v += dpp_f<0x141>(v);   // row_half_mirror
  v += dpp_f<0x140>(v);   // row_mirror
  return v;
}
// Greedy candidates (value, index): better = larger value, or equal value
// and smaller index; index < 0 is "none".  A total order, so any pairing of
// lanes reduces to the same winner.
__device__ __forceinline__ bool cand_better(float v, int i, float bv, int bi) {
  return i >= 0 && (bi < 0 || v > bv || (v == bv && i < bi));
}
template <int CTRL>
__device__ __forceinline__ void cand_step_dpp(float& v, int& i) {
  const float ov = dpp_f<CTRL>(v);
  const int oi = __builtin_amdgcn_update_dpp(i, i, CTRL, 0xF, 0xF, false);
  if (cand_better(ov, oi, v, i)) {
    v = ov;
    i = oi;
  }
}
// best candidate of each 16-lane row of the wave, in all its lanes
__device__ __forceinline__ void cand_best16(float& v, int& i) {
  cand_step_dpp<0xB1>(v, i);    // quad_perm [1,0,3,2]
  cand_step_dpp<0x4E>(v, i);    // quad_perm [2,3,0,1]
  cand_step_dpp<0x141>(v, i);   // row_half_mirror
  cand_step_dpp<0x140>(v, i);   // row_mirror
}
// best candidate of each 32-lane half of the wave, in all its lanes
__device__ __forceinline__ void cand_best32(float& v, int& i) {
  cand_best16(v, i);
  const auto pv = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  const auto pi = __builtin_amdgcn_permlane16_swap((unsigned)i, (unsigned)i, false, false);
  // each lane sees its own row's value in one output and the paired row's in
  // the other; take the better of the two
  const float v0 = __uint_as_float(pv[0]), v1 = __uint_as_float(pv[1]);
  const int i0 = (int)pi[0], i1 = (int)pi[1];
  if (cand_better(v1, i1, v0, i0)) {
    v = v1;
    i = i1;
  } else {
    v = v0;
    i = i0;
  }
}
// best candidate of the whole wave, in all lanes
__device__ __forceinline__ void cand_best64(float& v, int& i) {
  cand_best32(v, i);
  const auto pv = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  const auto pi = __builtin_amdgcn_permlane32_swap((unsigned)i, (unsigned)i, false, false);
  const float v0 = __uint_as_float(pv[0]), v1 = __uint_as_float(pv[1]);
  const int i0 = (int)pi[0], i1 = (int)pi[1];
  if (cand_better(v1, i1, v0, i0)) {
    v = v1;
    i = i1;
  } else {
    v = v0;
    i = i0;
  }
}

// max / sum of a value and its partner 32 lanes away (one lane-swap move)
__device__ __forceinline__ float pair_max(float v) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ __forceinline__ float pair_sum(float v) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}
__device__ __forceinline__ float wave_sum64(float v) {
  v = row_sum16(v);
  const auto p16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(p16[0]) + __uint_as_float(p16[1]);
  const auto p32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(p32[0]) + __uint_as_float(p32[1]);
}
__device__ __forceinline__ bf16 f2bf(float v) { return (bf16)v; }   // RNE (v_cvt_pk_bf16_f32)
// two floats to packed bf16 (lo in bits 0..15), one v_cvt_pk_bf16_f32, RNE
// silu(g) * u ("Implementation", TPMLP: silu(gate) times up), with the
// hardware reciprocal (about 1 ulp of fp32) in place of an IEEE division,
// whose expansion dominated the SiLU epilogues
__device__ __forceinline__ float silu_mul(float g, float u) {
  return g * __builtin_amdgcn_rcpf(1.f + __expf(-g)) * u;
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t{lo, hi}), bf16x2_t));
}

// --- GEMM -----------------------------------------------------------------
// C[M, N] = A[M, K] * B[N, K]^T, A and B bf16 with K contiguous, fp32
// accumulation.  Epilogues:
enum GemmEpi {
  EPI_BF16 = 0,       // C bf16 [M, N] (row stride ldc)
  EPI_F32 = 1,        // C fp32 [M, N]; with split-K: partials [splits, M, N]
  EPI_SILU_BF16 = 2,  // B = [gate; up] with `li` rows each; C = silu(gate)*up, bf16 [M, li]
  EPI_QKV = 3,        // merged q/k/v projection finished per head (QkvArgs); C unused
  EPI_ARGMAX = 4      // per row and N tile: (max of the bf16-rounded values, first column);
                      // C = 8-byte candidates [M, tiles_n] (float value, int32 column), ldc = tiles_n
};

// Per-head finish of the merged QKV projection (row m = b*T + t, N = (lq +
// 2 lkv) * 128 columns, head h = column / 128): q and k heads get the QK-norm
// v / sqrt(mean(v^2) + eps) * w and the rotate-half RoPE at position past + t;
// q heads go to q_out [M, lq*128], k and v heads to the caches
// [B, lkv, S_max, 128] at position past + t.
struct QkvArgs {
  const bf16* q_norm_w;  // [128]
  const bf16* k_norm_w;  // [128]
  bf16* q_out;
  bf16* k_cache;
  bf16* v_cache;
  int B, T, past, S_max, lq, lkv;
  float eps, theta;
  int head0;             // head of column 0 (a problem restricted to later columns)
};

struct GemmProblem {
  const bf16* A;
  const bf16* B;
  void* C;
  int64_t M, N, K;      // N = rows of B (for EPI_SILU_BF16: 2*li)
  int64_t lda, ldb, ldc;
  int64_t li;           // EPI_SILU_BF16 only
  QkvArgs qkv;          // EPI_QKV only
  // optional row gather of A: row m of the product reads A row a_rows[m]
  // (an index outside [0, a_total) reads as a zero row); a_total * lda * 2
  // must be below 2^31.  Never used with EPI_QKV or a split plan.
  const int32_t* a_rows;
  int64_t a_total;
  // EPI_SILU_BF16: rows from a gate row to its up row (0: li)
  int64_t up_off;
  // m-tiles per group of the tile order (0: the kernel's default)
  int group_m;
  // EPI_ARGMAX: id of this problem's column 0 (a column slice of a wider
  // problem reports ids of the whole one)
  int64_t col0;
};

// Chooses a tile shape and launches.  When the grid would not fill the GPU
// and `scratch` holds at least gemm_scratch_bytes() for the same problem,
// K is split and fp32 partials in scratch are summed by a second kernel;
// otherwise (scratch NULL or too small) no split is made.
size_t gemm_scratch_bytes(int64_t M, int64_t N, int64_t K, int epi);
// N tiles of the plan gemm_bf16 uses for an EPI_ARGMAX problem (never split)
int64_t gemm_argmax_tiles_n(int64_t M, int64_t N, int64_t K);
hipError_t gemm_bf16(const GemmProblem& p, int epi, void* scratch, size_t scratch_bytes, hipStream_t s);

// fp32 GEMM (small problems): C = A B^T, or silu-mul of the gate/up halves.
hipError_t gemm_f32(const float* A, const float* B, float* C, int64_t M, int64_t N, int64_t K,
                    int silu_li, hipStream_t s);

// --- copies ---------------------------------------------------------------
// dst[r, c] = src[(row0 + r) * src_ld + col0 + c] for r < rows, c < cols
// (elements of `esize` bytes); dst row stride dst_ld.
hipError_t copy2d(const void* src, int64_t src_ld, int64_t row0, int64_t col0, void* dst,
                  int64_t dst_ld, int64_t rows, int64_t cols, int esize, hipStream_t s);

hipError_t embed_masked(const int32_t* ids, int64_t n, const void* table, int64_t vstart,
                        int64_t vend, int64_t H, int esize, void* out, hipStream_t s);

// --- attention block ------------------------------------------------------

struct AttnArgs {
  const bf16* q;         // [B*T, lq*128]
  const bf16* k_cache;   // [B, lkv, S_max, 128]
  const bf16* v_cache;
  bf16* out;             // [B*T, lq*128]
  int B, T, past, S_max, lq, lkv;
  // Decode only, optional: the QKV projection as split-K fp32 partials
  // [qkv_splits, B, (lq + 2 lkv) * 128] still to be summed and finished
  // (QK-norm, RoPE, k / v appended at position past; q kept on chip and,
  // when q_store is set, also written there).  q is then not read.
  const float* qkv_part;
  int qkv_splits;
  const bf16* q_norm_w;
  const bf16* k_norm_w;
  float eps, theta;
  bf16* q_store;
};
// Prefill kernel whose workgroups each cover a (kv head, row block) with all
// its q heads; used when those workgroups alone fill the GPU.
bool attn_prefill_fills(int B, int T, int lq, int lkv);
hipError_t attn_prefill(const AttnArgs& a, hipStream_t s);
// One-pass flash attention for decode (rows = the q heads of a kv head) and
// for the prefills that attn_prefill would leave the GPU short of work.
hipError_t attn_flash(const AttnArgs& a, hipStream_t s);
// The merged QKV projection (EPI_QKV).  With defer set and a split-K plan,
// only the fp32 partials [splits, M, N] are written to scratch and
// *splits_out > 0: the decode attention finishes them (AttnArgs.qkv_part).
// Otherwise the projection is finished here and *splits_out = 0.
hipError_t gemm_qkv(const GemmProblem& p, void* scratch, size_t scratch_bytes, bool defer, int* splits_out,
                    hipStream_t s);

// --- greedy argmax over vocab-parallel logits ------------------------------
// out_val[m], out_idx[m] = the best of the n candidates cand[m, 0:n] (8 bytes
// each: float value, int32 column, column < 0 = none), column + idx0.
hipError_t argmax_candidates(const void* cand, int64_t M, int64_t n, int64_t idx0, float* out_val, int32_t* out_idx,
                             hipStream_t s);
// Decode head with the rows resident in LDS (M <= 64, K <= 1024, K % 256
// == 0, N >= 1, N * K * 2 < 2^31): one candidate per (row, workgroup) into
// cand [M, groups] (groups = argmax_resident_groups()), columns local to
// the vocab slice.
bool argmax_resident_ok(int64_t M, int64_t N, int64_t K);
int argmax_resident_groups();
// rows: optional row list (row m reads x row rows[m]; outside [0, x_rows):
// zeros), with x_rows * K * 2 < 2^31
hipError_t argmax_resident(const void* x, int64_t M, const int32_t* rows, int64_t x_rows, const void* vocab,
                           int64_t N, int64_t K, void* cand, hipStream_t s);
// Device address, on the current device, of the library's static candidate
// array of kNoAllocScratchBytes (looked up once per device; no allocation).
constexpr size_t kNoAllocScratchBytes = size_t(4) << 20;
hipError_t noalloc_scratch(void** ptr);
// out_idx[m] = the candidate (vals, idx [n_shards, M]) with the largest
// value, ties to the smallest index, idx < 0 skipped; out_val optional.
hipError_t argmax_combine(const float* vals, const int32_t* idx, int n_shards, int64_t M, int32_t* out_idx,
                          float* out_val, hipStream_t s);

// --- residual + RMSNorm over summed row-parallel partials -----------------
// For output row m < M, with input row i = in_rows ? in_rows[m] : m (an i
// outside [0, in_nrows) reads as a zero row):
//   h[m] = bf16(residual[i] + sum_{r < n} partials[r * plane + i])
//   y[m] = bf16(rms_norm(h[m]) * w)
// H % 8 == 0 and H <= 8192; h_out may alias residual, and may be NULL when
// n == 0 (plain RMSNorm).
struct NormArgs {
  const bf16* partials;
  int n;
  int64_t plane, M;
  int H;
  const bf16* residual;
  const bf16* w;
  float eps;
  bf16* h_out;
  bf16* y_out;
  const int32_t* in_rows;
  int64_t in_nrows;
};
hipError_t residual_rmsnorm(const NormArgs& a, hipStream_t s);
// threads that residual_rmsnorm gives one row of M x H (64 .. 1024)
int norm_threads_per_row(int64_t M, int H);

// --- per-kernel timing marks (tp_kernel_marks, host thread-local) ---------
// After each kernel launch the launching code calls kmark: when the calling
// host thread has armed marks, the next event is recorded on `s` and the
// kernel's name kept beside it; otherwise nothing happens.
bool kmarks_armed();
void kmark(hipStream_t s, const char* name);

}  // namespace tps
