// Greedy next token over vocab-parallel logits ("Tensor parallelism from
// scratch", "Implementation": the decode loop takes the argmax of the last
// position's logits, which the vocab-split output layer produces a slice of
// per rank before the all-gather).  Instead of gathering V logits per row,
// each rank reduces its slice to one candidate (max, first global index of
// it), and the candidates of all ranks combine to the max, ties to the
// smaller global index -- the first maximum of the concatenated logits.
//
// The logits GEMM reduces each tile row to a candidate in its epilogue
// (EPI_ARGMAX in gemm.hip), so the logits never reach memory.
// argmax_pairs: one workgroup per row reduces the row's tile candidates
// (a per-thread best, then wave shuffles and LDS).  combine_candidates: one
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

}  // namespace

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
