// Bit-exact copies: shard gather and the masked vocab embedding.
//
// Shard gather ("8. How several ranks share one ledger", "Weights are cut by
// name"): a rank's shard is a block of rows (column-parallel weights, vocab
// rows) or of columns (row-parallel weights) of the full [out, in] matrix.
// Both are a 2-D strided copy.  HBM-bound: each thread moves 16 bytes, rows
// are read and written in contiguous 16-byte runs.
//
// Masked embedding ("Tensor parallelism from scratch", "Implementation",
// VocabParallelEmbedding): ids outside the rank's vocab range give +0.0 rows.
#include "common.h"

namespace tps {

namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void copy2d_v16(const uint8_t* __restrict__ src, int64_t src_ld_b,
                                                       uint8_t* __restrict__ dst, int64_t dst_ld_b,
                                                       int64_t rows, int64_t chunks_per_row) {
  const int64_t total = rows * chunks_per_row;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * kThreads) {
    const int64_t r = i / chunks_per_row, c = i - r * chunks_per_row;
    const u32x4 v = *reinterpret_cast<const u32x4*>(src + r * src_ld_b + c * 16);
    *reinterpret_cast<u32x4*>(dst + r * dst_ld_b + c * 16) = v;
  }
}

template <typename T>
__global__ __launch_bounds__(kThreads) void copy2d_scalar(const T* __restrict__ src, int64_t src_ld,
                                                          T* __restrict__ dst, int64_t dst_ld,
                                                          int64_t rows, int64_t cols) {
  const int64_t total = rows * cols;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * kThreads) {
    const int64_t r = i / cols, c = i - r * cols;
    dst[r * dst_ld + c] = src[r * src_ld + c];
  }
}

// One 16-byte chunk of one output row per thread; the id decides between a
// copy of the table row and zeros.
__global__ __launch_bounds__(kThreads) void embed_masked_v16(const int32_t* __restrict__ ids, int64_t n,
                                                             const uint8_t* __restrict__ table,
                                                             int64_t vstart, int64_t vend,
                                                             int64_t row_b, uint8_t* __restrict__ out) {
  const int64_t cpr = row_b / 16;
  const int64_t total = n * cpr;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * kThreads) {
    const int64_t t = i / cpr, c = i - t * cpr;
    const int64_t id = ids[t];
    u32x4 v = {0u, 0u, 0u, 0u};
    if (id >= vstart && id < vend) v = *reinterpret_cast<const u32x4*>(table + (id - vstart) * row_b + c * 16);
    *reinterpret_cast<u32x4*>(out + t * row_b + c * 16) = v;
  }
}

int grid_for(int64_t work) {
  int64_t g = (work + kThreads - 1) / kThreads;
  if (g > 8192) g = 8192;      // grid-stride beyond 32 waves per CU
  return g < 1 ? 1 : (int)g;
}

}  // namespace

hipError_t copy2d(const void* src, int64_t src_ld, int64_t row0, int64_t col0, void* dst, int64_t dst_ld,
                  int64_t rows, int64_t cols, int esize, hipStream_t s) {
  if (rows <= 0 || cols <= 0) return hipSuccess;
  const uint8_t* sp = static_cast<const uint8_t*>(src) + (row0 * src_ld + col0) * esize;
  uint8_t* dp = static_cast<uint8_t*>(dst);
  const int64_t row_b = cols * esize, sld_b = src_ld * esize, dld_b = dst_ld * esize;
  const bool v16 = (row_b % 16 == 0) && (sld_b % 16 == 0) && (dld_b % 16 == 0) &&
                   ((uintptr_t)sp % 16 == 0) && ((uintptr_t)dp % 16 == 0);
  if (v16) {
    const int64_t cpr = row_b / 16;
    copy2d_v16<<<grid_for(rows * cpr), kThreads, 0, s>>>(sp, sld_b, dp, dld_b, rows, cpr);
  } else if (esize == 4) {
    copy2d_scalar<uint32_t><<<grid_for(rows * cols), kThreads, 0, s>>>(
        reinterpret_cast<const uint32_t*>(sp), src_ld, reinterpret_cast<uint32_t*>(dp), dst_ld, rows, cols);
  } else {
    copy2d_scalar<uint16_t><<<grid_for(rows * cols), kThreads, 0, s>>>(
        reinterpret_cast<const uint16_t*>(sp), src_ld, reinterpret_cast<uint16_t*>(dp), dst_ld, rows, cols);
  }
  kmark(s, v16 ? "copy2d_v16" : "copy2d_scalar");
  return hipGetLastError();
}

hipError_t embed_masked(const int32_t* ids, int64_t n, const void* table, int64_t vstart, int64_t vend,
                        int64_t H, int esize, void* out, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int64_t row_b = H * esize;   // the caller guarantees row_b % 16 == 0
  embed_masked_v16<<<grid_for(n * (row_b / 16)), kThreads, 0, s>>>(
      ids, n, static_cast<const uint8_t*>(table), vstart, vend, row_b, static_cast<uint8_t*>(out));
  kmark(s, "embed_masked_v16");
  return hipGetLastError();
}

}  // namespace tps
