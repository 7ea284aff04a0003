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
#include <type_traits>

#include <algorithm>
#include <cstdio>

#include "common.h"
#include "qkv_finish.h"

namespace tps {

namespace {

constexpr int kXcds = 8;

__device__ __forceinline__ int xcd_remap(int bid, int nb) {
  const int xcd = bid % kXcds, idx = bid / kXcds;
  const int per = nb / kXcds, rem = nb % kXcds;
  return (xcd < rem ? xcd * (per + 1) : rem * (per + 1) + (xcd - rem) * per) + idx;
}

// 16-byte chunk position inside a tile row of BK bf16 (128 or 64 bytes):
// 16 consecutive rows land on 16 distinct 16-byte slots of the 256-byte
// bank space.
template <int BK>
__device__ __forceinline__ int swz(int row, int chunk) {
  static_assert(BK == 64 || BK == 32, "tile rows of 128 or 64 bytes");
  return BK == 64 ? chunk ^ ((row >> 1) & 7) : chunk ^ ((row >> 2) & 3);
}

typedef __attribute__((address_space(3))) void lds_void_t;

// Buffer descriptor over [base, base + bytes): loads past the end return
// zero instead of touching memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const int64_t n = bytes < 0 ? 0 : (bytes > 0xFFFFFFFFll ? 0xFFFFFFFFll : bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)(uint32_t)n, 0x00020000);
}
// buffer_load_dwordx4 ... lds: each lane's 16 bytes go straight to LDS at
// lds_base + 16 * lane (lds_base is wave-uniform), no VGPR staging.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint32_t voff, void* lds_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)lds_base, 16, voff, 0, 0, 0);
}
__device__ __forceinline__ u32x4 load16(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, 0));
}
__device__ __forceinline__ void wait_vm0() { __builtin_amdgcn_s_waitcnt(0x0F70); }   // vmcnt(0)
// s_waitcnt vmcnt(N) (expcnt and lgkmcnt left at their maximum)
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}
// ---- merged QKV finish: QK-norm and RoPE per (row, head) in qkv_finish.h;
// here the store of q, or the append of k / v to the caches.
// x[0..3] hold d = 4j .. 4j+3 of (row m = b T + t, head h), x[4..7] hold d + 64;
// nw: the lane's weights of that head's norm (q or k)
__device__ __forceinline__ const bf16* norm_of(const QkvArgs& a, int h) {
  return h + a.head0 < a.lq ? a.q_norm_w : a.k_norm_w;
}
__device__ __forceinline__ void qkv_finish_at(const QkvArgs& a, float (&x)[8], int64_t m, int b, int t, int h, int j,
                                              const RopeCoef& rc, const NormW& nw) {
  h += a.head0;
  const int pos = a.past + t;
  if (h < a.lq + a.lkv) qk_norm_rope(x, nw, pos, rc, a.eps);
  bf16* dst;
  if (h < a.lq)
    dst = a.q_out + m * ((int64_t)a.lq * 128) + (int64_t)h * 128;
  else if (h < a.lq + a.lkv)
    dst = a.k_cache + (((int64_t)b * a.lkv + (h - a.lq)) * a.S_max + pos) * 128;
  else
    dst = a.v_cache + (((int64_t)b * a.lkv + (h - a.lq - a.lkv)) * a.S_max + pos) * 128;
  store_head_lanes(dst, x, j);
}
__device__ __forceinline__ void qkv_finish(const QkvArgs& a, float (&x)[8], int64_t m, int h, int j,
                                           const RopeCoef& rc) {
  // (a 32-bit division where the row index allows: the 64-bit one is a
  // long expansion)
  const int b = m < 0x7fffffff ? (int)((uint32_t)m / (uint32_t)a.T) : (int)(m / a.T);
  qkv_finish_at(a, x, m, b, (int)(m - (int64_t)b * a.T), h, j, rc, norm_w(norm_of(a, h), j));
}
// problems of at most this many rows run the small tiles in the 16x16 form
constexpr int64_t kMf16RowsPlan = 256;
// the 320-wide tile: no QKV or argmax epilogue, no row gather; beyond one
// round only unsplit and at K >= 2048
constexpr bool wide_tile(int bn) { return bn == 320; }
// the fp32 tile of a QKV epilogue fits the LDS ring and covers whole heads
// (the epilogue stages the tile 128 columns -- one head -- at a time)
constexpr bool qkv_tile_ok(int bm, int bn, int stages, int bk = 64) {
  return bn % 128 == 0 && bm * 128 * 4 <= stages * (bm + bn) * bk * 2;
}

// Default LDS stages per tile shape: as many as let two workgroups share a
// CU's 160 KB (at least 2, at most 6).  Weight-streaming shapes (few rows)
// pick deeper rings explicitly.
constexpr int gemm_stages(int bm, int bn) {
  return (81920 / ((bm + bn) * 64 * 2)) > 6 ? 6 : ((81920 / ((bm + bn) * 64 * 2)) < 2 ? 2 : 81920 / ((bm + bn) * 64 * 2));
}
// waves per SIMD that one CU holds for a tile shape and ring depth (LDS-limited)
constexpr int gemm_waves_per_simd(int bm, int bn, int nw, int stages, int bk = 64) {
  return (nw / 4 < 1 ? 1 : nw / 4) * (163840 / (stages * (bm + bn) * bk * 2));
}

// MF16: v_mfma_f32_16x16x32_bf16 on 16x16 output blocks instead of
// v_mfma_f32_32x32x16_bf16 on 32x32 ones (the launch picks it for the
// weight-streaming GEMMs of few rows, where it measured 2-7% faster; on the
// 256-row prefill tiles its larger operand sets ran out of registers).
template <int BM, int BN, int WGM, int WGN, int EPI, bool SPLIT, int GROUP_M, int S, int BK = 64, bool MF16 = false>
__global__ __launch_bounds__(WGM * WGN * 64)
__attribute__((amdgpu_waves_per_eu(gemm_waves_per_simd(BM, BN, WGM * WGN, S, BK),
                                   gemm_waves_per_simd(BM, BN, WGM * WGN, S, BK))))
void gemm_kernel(GemmProblem p, int tiles_m, int tiles_n, int64_t k_per_split) {
  constexpr int NT = WGM * WGN * 64;
  constexpr int WM = BM / WGM, WN = BN / WGN;
  constexpr int BW = MF16 ? 16 : 32;         // output block edge of one MFMA
  constexpr int NE = BW * BW / 64;           // accumulator values per lane and block
  constexpr int TM = WM / BW, TN = WN / BW;
  constexpr int KC = BK / 8;                 // 16-byte chunks per tile row
  static_assert(WM % 32 == 0 && WN % 32 == 0, "wave tile in whole 32-row / 32-column units");
  // SiLU tiles hold gate and up rows in one of two layouts: with an even
  // number of 32-column blocks per wave, gate rows in the tile's first half
  // and up rows in its second (block j pairs with block j + TN / 2); with an
  // odd number (256 x 320 tiles: 5 per wave), each 32-row block holds 16
  // gate rows and the 16 matching up rows (SI), so that in the C^T
  // accumulator layout a lane's values e < 8 are gate sums and e + 8 the
  // up sums of the same output
  constexpr bool SI = EPI == EPI_SILU_BF16 && TN % 2 == 1;
  static_assert(!SI || !MF16, "the interleaved silu layout needs 32x32 blocks");
  // bf16 outputs accumulate C^T (B fragment as the first MFMA operand): a
  // lane then holds four consecutive output columns of one row, staged by
  // one 8-byte LDS write
  constexpr bool TR = EPI == EPI_BF16 || EPI == EPI_SILU_BF16;
  constexpr int STAGE = (BM + BN) * BK;
  // LDS ring of S stages: S - 1 blocks in flight
  static_assert(S >= 2 && S * STAGE * 2 <= 163840, "ring must be double-buffered and fit the CU's LDS");
  __shared__ __attribute__((aligned(16))) bf16 smem[S * STAGE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = __builtin_amdgcn_readfirstlane(wave) / WGN, wn = __builtin_amdgcn_readfirstlane(wave) % WGN;

  // tile coordinates: XCD-contiguous, then GROUP_M m-tiles per n-column sweep
  int tm, tn;
  {
    const int t = xcd_remap(blockIdx.x, gridDim.x);
    const int group_m = p.group_m > 0 ? p.group_m : GROUP_M;
    const int per_group = group_m * tiles_n;
    const int g = t / per_group;
    const int first_m = g * group_m;
    const int gm = min(tiles_m - first_m, group_m);
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

  // Tile loads.  One load instruction fills RPI rows (1 KB): wave w fills
  // row groups g = w, w + NW, ... of each stage; lane l of a group writes
  // LDS row RPI*g + l/KC, physical chunk l%KC, and so fetches the logical
  // chunk that the swizzle puts there.  One
  // buffer descriptor per operand covers the tile's rows from column 0 to
  // the end of the matrix; a block at column k0 adds 2*k0 to the lane
  // offsets, so the range check drops exactly what lies past the matrix
  // (rows past M or N, and columns past the last row's end).  Those zeros
  // only feed outputs that are never stored, or are cleared by zero_tail.
  constexpr int NW = WGM * WGN;
  constexpr int RPI = 512 / BK;             // rows per 1 KB load instruction
  static_assert(BM % (RPI * NW) == 0 && BN % (RPI * NW) == 0, "row groups must split evenly");
  static_assert(EPI != EPI_SILU_BF16 || (BN / 2) % RPI == 0, "gate/up halves must hold whole groups");
  constexpr int A_G = BM / (RPI * NW), B_G = BN / (RPI * NW);
  constexpr int NV = A_G + B_G;             // direct-to-LDS loads per block per wave
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int grow = lane / KC, gpc = lane % KC;
  const int64_t lda_b = p.lda * 2, ldb_b = p.ldb * 2;
  // B rows of this tile: [b_row0, +BN) or, for silu, [gate0, +BN/2) and [up0, +BN/2)
  const int64_t nrow0 = EPI == EPI_SILU_BF16 ? (int64_t)tn * (BN / 2) : (int64_t)tn * BN;
  const int64_t nrows = EPI == EPI_SILU_BF16 ? p.li - nrow0 : p.N - nrow0;
  // A rows: the tile's own rows from m0, or (row gather, bf16 and argmax
  // outputs on tiles up to 256 wide) rows a_rows[m0 + r] of the whole A, a
  // row past M or an index outside A at an offset past the descriptor's
  // range (2^31 + a K offset below 2^23: zeros)
  constexpr bool GATHER_OK = !SPLIT && (EPI == EPI_BF16 || EPI == EPI_ARGMAX) && !wide_tile(BN);
  const bool gather = GATHER_OK && p.a_rows != nullptr;
  const __amdgpu_buffer_rsrc_t ra =
      gather ? make_rsrc(p.A, p.a_total * lda_b) : make_rsrc(p.A + m0 * p.lda, (M - m0) * lda_b);
  const __amdgpu_buffer_rsrc_t rg = make_rsrc(p.B + nrow0 * p.ldb, nrows * ldb_b);
  const __amdgpu_buffer_rsrc_t ru = make_rsrc(p.B + ((p.up_off ? p.up_off : p.li) + nrow0) * p.ldb, nrows * ldb_b);
  // Slice offsets.  A slice's rows are its first source row R (wave-uniform)
  // plus the lane's row grow; R % 16 is the same for every slice of a wave
  // (slices lie NW * RPI rows apart, gate/up halves and blocks are whole
  // multiples of 16 rows) and the chunk swizzle has a period of 16 rows, so
  // a lane's offset is a per-lane part per operand plus R times the row
  // pitch, which the scalar unit computes.
  // SI: LDS row 32 b + r (r < 16) holds gate row 16 b + r, 32 b + 16 + r the
  // up row 16 b + r.
  auto b_up = [&](int g) { return EPI == EPI_SILU_BF16 && (SI ? ((g * RPI) & 16) != 0 : g * RPI >= BN / 2); };
  auto src_row0 = [&](bool isA, int g) -> int {
    if (isA) return g * RPI;
    if (SI) return (g * RPI) / 32 * 16 + (g * RPI) % 16;
    return g * RPI - (b_up(g) ? BN / 2 : 0);
  };
  static_assert(EPI != EPI_SILU_BF16 || (BN / 2) % 16 == 0, "gate/up halves in whole 16-row units");
  const uint32_t lsw = (uint32_t)(swz<BK>(((wave_u * RPI) & 15) + grow, gpc) << 4);
  const uint32_t lane_a = (uint32_t)(grow * lda_b) + lsw, lane_b = (uint32_t)(grow * ldb_b) + lsw;
  // gathered A rows: one offset per slice and lane
  uint32_t ga[GATHER_OK ? A_G : 1];
  if constexpr (GATHER_OK) {
#pragma unroll
    for (int v = 0; v < A_G; ++v) {
      const int row = (wave_u + v * NW) * RPI + grow;
      const int64_t src = gather && m0 + row < M ? (int64_t)p.a_rows[m0 + row] : -1;
      ga[v] = (src >= 0 && src < p.a_total ? (uint32_t)(src * lda_b) : 0x80000000u) + lsw;
    }
  }
  auto dma_slice = [&](int v, int64_t k0, int buf) {
    bf16* st = smem + buf * STAGE;
    const uint32_t ko = (uint32_t)(k0 * 2);
    if (v < A_G) {
      const int g = wave_u + v * NW;
      uint32_t off = lane_a + (uint32_t)(src_row0(true, g) * lda_b);
      if constexpr (GATHER_OK) off = gather ? ga[v] : off;
      dma16(ra, off + ko, st + g * RPI * BK);
    } else {
      const int g = wave_u + (v - A_G) * NW;
      dma16(b_up(g) ? ru : rg, lane_b + (uint32_t)(src_row0(false, g) * ldb_b) + ko, st + BM * BK + g * RPI * BK);
    }
  };
  // The last block may end inside the 64-wide K window: its columns at or
  // past kend were loaded from the next row (or read as zero past the
  // matrix) and are cleared here, after the block has landed.
  auto zero_tail = [&](int buf, int64_t k0) {
    bf16* st = smem + buf * STAGE;
    for (int q = tid; q < (BM + BN) * KC; q += NT) {
      const int row = q / KC, lc = q % KC;
      if (k0 + lc * 8 >= kend) *reinterpret_cast<u32x4*>(st + row * BK + swz<BK>(row, lc) * 8) = u32x4{0u, 0u, 0u, 0u};
    }
  };
  // tile-local column of the j-th BW-wide n-block of this wave
  auto ncol = [&](int j) -> int {
    if (EPI == EPI_SILU_BF16 && !SI)
      return j < TN / 2 ? wn * (WN / 2) + j * BW : BN / 2 + wn * (WN / 2) + (j - TN / 2) * BW;
    return wn * WN + j * BW;
  };

  using AccT = std::conditional_t<MF16, f32x4, f32x16>;
  AccT acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int e = 0; e < NE; ++e) acc[i][j][e] = 0.f;

  // lane lr of a block edge; lh: the lane's group (k values 8 lh .. 8 lh + 7
  // of an operand, rows 4 lh .. of an output block)
  const int lr = lane & (BW - 1), lh = lane / BW;
  // An operand row a lane reads is lr plus a multiple of 16 (wave tiles,
  // blocks and gate/up halves start on such rows), and the chunk swizzle has
  // a period of 16 rows: a fragment's LDS offset is a per-lane part per k
  // chunk c plus a wave-uniform row offset.
  auto lfo = [&](int c) { return lr * BK + swz<BK>(lr, c) * 8; };
  if constexpr (MF16) {
    // v_mfma_f32_16x16x32_bf16: lane l supplies row (or column) l & 15 of a
    // 16-row operand block and its k values 8 (l >> 4) .. + 7 of the k-step's
    // 32.  One K block is KS k-steps of 32.  A fragments come in two sets
    // (set ks & 1 holds k-step ks; the next k-step's are read while this
    // one's MFMAs run), B fragments in one: the MFMAs go out column by
    // column (B fragment j with every A fragment), and each B fragment is
    // refilled for the next k-step right after its last MFMA.  The stream is
    // fenced (sched_barrier) per column; the first k-step also carries
    // slices of a later block's direct-to-LDS loads.  In the last k-step the
    // wave waits for the next block (vmcnt, then a barrier) after half of its
    // columns, then reads the next block's A fragments and the B fragments
    // already used, and the rest as their columns finish, so a block boundary
    // leaves no gap in the matrix pipe.
    bf16x8 fa[2][TM], fb[TN];
    constexpr int KS = BK / 32;
    static_assert(KS % 2 == 0, "A fragment sets alternate per k-step");
    static_assert(TN >= TM, "the next k-step's A reads follow the first TM columns");
    constexpr int JW = TN / 2;                 // columns of the last k-step before the wait
    auto rdA = [&](const bf16* sA, int ks, int set, int i) {
      fa[set][i] = *reinterpret_cast<const bf16x8*>(sA + (wm * WM + i * 16) * BK + lfo(ks * 4 + lh));
    };
    auto rdB = [&](const bf16* sB, int ks, int j) {
      fb[j] = *reinterpret_cast<const bf16x8*>(sB + ncol(j) * BK + lfo(ks * 4 + lh));
    };
    auto mfma_col = [&](int set, int j) {
  #pragma unroll
      for (int i = 0; i < TM; ++i) {
        if constexpr (TR)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb[j], fa[set][i], acc[i][j], 0, 0, 0);
        else
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[set][i], fb[j], acc[i][j], 0, 0, 0);
      }
    };
    const bool tail = (kend - kbeg) % BK != 0;
    auto kblk = [&](int blk) { return kbeg + (int64_t)blk * BK; };
    // A bare s_barrier, not __syncthreads(): the latter's workgroup release
    // fence waits for every outstanding direct-to-LDS load (vmcnt(0)), which
    // would collapse the ring to one block in flight.  Before it each wave
    // has waited (vmcnt) for its own loads of the block about to be read and
    // (lhkmcnt) for its reads of the block just finished; the barrier makes
    // both true for all waves, so the block can be read and the stage it
    // frees can be refilled.  The asm memory clobber keeps the compiler from
    // moving LDS accesses across it.
    auto settle = [&](int blk) {
      __builtin_amdgcn_s_waitcnt(0xC07F);   // lhkmcnt(0)
      asm volatile("s_barrier" ::: "memory");
      if (tail && blk == nk - 1) {
        zero_tail(blk % S, kblk(blk));
        __builtin_amdgcn_s_waitcnt(0xC07F);   // the zero stores are done
        asm volatile("s_barrier" ::: "memory");
      }
    };
    // One block from stage kt % S.  DMA: this block issues block kt + S - 1
    // (steady state); NEXT: a block kt + 1 follows.
    auto block = [&](auto dma_tag, auto next_tag, int kt) {
      constexpr bool DMA = decltype(dma_tag)::value;
      constexpr bool NEXT = decltype(next_tag)::value;
      const int cur = kt % S;
      const bf16* sA = smem + cur * STAGE;
      const bf16* sB = sA + BM * BK;
      const int nxt = (kt + 1) % S;
      const bf16* nA = smem + nxt * STAGE;
      const bf16* nB = nA + BM * BK;
      const int64_t dk0 = kblk(kt + S - 1);
      const int dbuf = (kt + S - 1) % S;
      __builtin_amdgcn_sched_barrier(0);
      int v = 0;
  #pragma unroll
      for (int ks = 0; ks < KS - 1; ++ks) {
  #pragma unroll
        for (int j = 0; j < TN; ++j) {
          mfma_col(ks & 1, j);
          rdB(sB, ks + 1, j);
          if (j < TM) rdA(sA, ks + 1, (ks + 1) & 1, j);
          if constexpr (DMA) {
            if (ks == 0) {
              while (v < NV && (j + 1) * NV >= (v + 1) * TN) dma_slice(v++, dk0, dbuf);
            }
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
  #pragma unroll
      for (int j = 0; j < TN; ++j) {
        mfma_col((KS - 1) & 1, j);
        if constexpr (NEXT) {
          if (j == JW - 1) {
            if constexpr (DMA)
              wait_vm<(S - 2) * NV>();
            else
              wait_vm0();
            settle(kt + 1);
            __builtin_amdgcn_sched_barrier(0);
  #pragma unroll
            for (int i = 0; i < TM; ++i) rdA(nA, 0, 0, i);
  #pragma unroll
            for (int jj = 0; jj < JW; ++jj) rdB(nB, 0, jj);
          } else if (j >= JW) {
            rdB(nB, 0, j);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    };

    // Pipeline: blocks 0 .. S-2 are issued up front; block kt issues block
    // kt + S - 1 in its first k-step and waits for block kt + 1 in its last
    // (vmcnt counts this wave's outstanding loads, which complete in issue
    // order).
    if (nk > 0) {
      const int pro = nk < S - 1 ? nk : S - 1;
      for (int blk = 0; blk < pro; ++blk)
  #pragma unroll
        for (int v = 0; v < NV; ++v) dma_slice(v, kblk(blk), blk);
      if (pro - 1 == S - 2)
        wait_vm<(S - 2) * NV>();
      else
        wait_vm0();
      settle(0);
  #pragma unroll
      for (int i = 0; i < TM; ++i) rdA(smem, 0, 0, i);
  #pragma unroll
      for (int j = 0; j < TN; ++j) rdB(smem + BM * BK, 0, j);
    }
    int kt = 0;
    for (; kt + S - 1 < nk; ++kt) block(std::true_type{}, std::true_type{}, kt);      // steady state
    for (; kt + 1 < nk; ++kt) block(std::false_type{}, std::true_type{}, kt);         // drain
    if (kt < nk) block(std::false_type{}, std::false_type{}, kt);                     // last block
  } else {
    bf16x8 af[2][TM], bfr[2][TN];
    // One K block is KS k-steps of 16.  Each k-step's MFMAs go out two at a
    // time in a fenced, hand-ordered stream (sched_barrier keeps it): after
    // each pair come the operand reads of the following k-step and, in the
    // first k-step, slices of a later block's direct-to-LDS loads.  In the
    // last k-step the wave waits for the next block (vmcnt, then a barrier)
    // after half of its MFMAs, and reads the next block's first operands
    // under the other half, so a block boundary leaves no gap in the matrix
    // pipe.  Fragment set ks & 1 holds k-step ks (KS is even).
    constexpr int KS = BK / 16;
    static_assert(KS % 2 == 0, "fragment sets alternate per k-step");
    constexpr int NF = TM + TN, NMF = TM * TN;
    constexpr int NPAIR = (NMF + 1) / 2;
    constexpr int RDP = (NF + NPAIR - 1) / NPAIR;   // operand reads after each MFMA pair
    constexpr int H1 = NPAIR / 2;                    // pairs of the last k-step before the wait
    constexpr int RDP2 = (NF + (NPAIR - H1) - 1) / (NPAIR - H1);
    auto read_frag = [&](const bf16* sA, const bf16* sB, int ks, int fs, int x) {
      // order A0, B0..B(TN-1), A1..A(TM-1): the next k-step's first MFMAs
      // need A0 with every B
      const int c = ks * 2 + lh;
      if (x == 0 || x > TN) {
        const int i = x == 0 ? 0 : x - TN;
        af[fs][i] = *reinterpret_cast<const bf16x8*>(sA + (wm * WM + i * 32) * BK + lfo(c));
      } else {
        bfr[fs][x - 1] = *reinterpret_cast<const bf16x8*>(sB + ncol(x - 1) * BK + lfo(c));
      }
    };
    auto mfma_pair = [&](int fs, int pr) {
  #pragma unroll
      for (int m = 2 * pr; m < 2 * pr + 2 && m < NMF; ++m) {
        if constexpr (TR)
          acc[m / TN][m % TN] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[fs][m % TN], af[fs][m / TN],
                                                                      acc[m / TN][m % TN], 0, 0, 0);
        else
          acc[m / TN][m % TN] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[fs][m / TN], bfr[fs][m % TN],
                                                                      acc[m / TN][m % TN], 0, 0, 0);
      }
    };
    const bool tail = (kend - kbeg) % BK != 0;
    auto kblk = [&](int blk) { return kbeg + (int64_t)blk * BK; };
    // A bare s_barrier, not __syncthreads(): the latter's workgroup release
    // fence waits for every outstanding direct-to-LDS load (vmcnt(0)), which
    // would collapse the ring to one block in flight.  Before it each wave
    // has waited (vmcnt) for its own loads of the block about to be read and
    // (lgkmcnt) for its reads of the block just finished; the barrier makes
    // both true for all waves, so the block can be read and the stage it
    // frees can be refilled.  The asm memory clobber keeps the compiler from
    // moving LDS accesses across it.
    auto settle = [&](int blk) {
      __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
      asm volatile("s_barrier" ::: "memory");
      if (tail && blk == nk - 1) {
        zero_tail(blk % S, kblk(blk));
        __builtin_amdgcn_s_waitcnt(0xC07F);   // the zero stores are done
        asm volatile("s_barrier" ::: "memory");
      }
    };
    // One block from stage kt % S.  DMA: this block issues block kt + S - 1
    // (steady state); NEXT: a block kt + 1 follows; SD: the steady-state
    // wait (S - 2 blocks may stay in flight) rather than vmcnt(0).
    auto block = [&](auto dma_tag, auto next_tag, int kt) {
      constexpr bool DMA = decltype(dma_tag)::value;
      constexpr bool NEXT = decltype(next_tag)::value;
      const int cur = kt % S;
      const bf16* sA = smem + cur * STAGE;
      const bf16* sB = sA + BM * BK;
      const int nxt = (kt + 1) % S;
      const bf16* nA = smem + nxt * STAGE;
      const bf16* nB = nA + BM * BK;
      const int64_t dk0 = kblk(kt + S - 1);
      const int dbuf = (kt + S - 1) % S;
      __builtin_amdgcn_sched_barrier(0);
      int v = 0;
  #pragma unroll
      for (int ks = 0; ks < KS - 1; ++ks) {
  #pragma unroll
        for (int pr = 0; pr < NPAIR; ++pr) {
          mfma_pair(ks & 1, pr);
  #pragma unroll
          for (int x = pr * RDP; x < pr * RDP + RDP && x < NF; ++x) read_frag(sA, sB, ks + 1, (ks + 1) & 1, x);
          if constexpr (DMA) {
            if (ks == 0) {
              while (v < NV && (pr + 1) * NV >= (v + 1) * NPAIR) dma_slice(v++, dk0, dbuf);
            }
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
  #pragma unroll
      for (int pr = 0; pr < H1; ++pr) {
        mfma_pair(1, pr);
        __builtin_amdgcn_sched_barrier(0);
      }
      if constexpr (NEXT) {
        if constexpr (DMA)
          wait_vm<(S - 2) * NV>();
        else
          wait_vm0();
        settle(kt + 1);
        __builtin_amdgcn_sched_barrier(0);
      }
  #pragma unroll
      for (int pr = H1; pr < NPAIR; ++pr) {
        mfma_pair(1, pr);
        if constexpr (NEXT) {
  #pragma unroll
          for (int x = (pr - H1) * RDP2; x < (pr - H1) * RDP2 + RDP2 && x < NF; ++x) read_frag(nA, nB, 0, 0, x);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    };

    // Pipeline: blocks 0 .. S-2 are issued up front; block kt issues block
    // kt + S - 1 in its first k-step and waits for block kt + 1 in its last
    // (vmcnt counts this wave's outstanding loads, which complete in issue
    // order).
    if (nk > 0) {
      const int pro = nk < S - 1 ? nk : S - 1;
      for (int blk = 0; blk < pro; ++blk)
  #pragma unroll
        for (int v = 0; v < NV; ++v) dma_slice(v, kblk(blk), blk);
      if (pro - 1 == S - 2)
        wait_vm<(S - 2) * NV>();
      else
        wait_vm0();
      settle(0);
  #pragma unroll
      for (int x = 0; x < NF; ++x) read_frag(smem, smem + BM * BK, 0, 0, x);
    }
    int kt = 0;
    for (; kt + S - 1 < nk; ++kt) block(std::true_type{}, std::true_type{}, kt);      // steady state
    for (; kt + 1 < nk; ++kt) block(std::false_type{}, std::true_type{}, kt);         // drain
    if (kt < nk) block(std::false_type{}, std::false_type{}, kt);                     // last block
  }

  // ---- epilogue.  MFMA layout: lane holds column lr = lane % BW and rows
  // 8*(e/4) + 4*lh + e%4 of each BW x BW block, lh = lane / BW (for BW = 16
  // that is rows 4*lh + e, e < 4; transposed for TR).
  if constexpr (EPI == EPI_ARGMAX) {
    // Greedy-decode candidates: per tile row, the largest bf16-rounded
    // value over the tile's columns and the first column holding it (ties
    // to the smaller column, as argmax takes the first maximum); the BW
    // lanes of a lane group hold BW columns of a row, then the WGN waves of
    // the tile combine through LDS.
    static_assert(!SPLIT, "argmax candidates come from whole K");
    __syncthreads();   // the ring is no longer read
    float* cv = reinterpret_cast<float*>(smem);
    int* ci = reinterpret_cast<int*>(cv + WGN * BM);
    auto better = [](float v, int i, float bv, int bi) { return i >= 0 && (bi < 0 || v > bv || (v == bv && i < bi)); };
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int e = 0; e < NE; ++e) {
        float bv = -INFINITY;
        int bi = -1;
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const int64_t col = (int64_t)tn * BN + ncol(j) + lr;
          const float v = bf2f(f2bf(acc[i][j][e]));
          if (col < p.N && better(v, (int)(p.col0 + col), bv, bi)) {
            bv = v;
            bi = (int)(p.col0 + col);
          }
        }
        if constexpr (MF16)
          cand_best16(bv, bi);
        else
          cand_best32(bv, bi);
        if (lr == 0) {
          const int r = wm * WM + i * BW + 8 * (e >> 2) + 4 * lh + (e & 3);
          cv[wn * BM + r] = bv;
          ci[wn * BM + r] = bi;
        }
      }
    __syncthreads();
    u32x2* cand = static_cast<u32x2*>(p.C);
    for (int r = tid; r < BM; r += NT) {
      if (m0 + r >= M) continue;
      float bv = cv[r];
      int bi = ci[r];
      for (int w = 1; w < WGN; ++w)
        if (better(cv[w * BM + r], ci[w * BM + r], bv, bi)) {
          bv = cv[w * BM + r];
          bi = ci[w * BM + r];
        }
      cand[(m0 + r) * p.ldc + tn] = u32x2{__float_as_uint(bv), (uint32_t)bi};
    }
    return;
  }
  if constexpr (EPI == EPI_QKV) {
    static_assert(qkv_tile_ok(BM, BN, S, BK), "QKV tile must cover whole heads and fit the ring");
    // one head (128 columns) at a time: stage its fp32 columns [BM][128] in
    // LDS (column c of row r at c ^ BW * ((r / 4) % (64 / BW)): the 64 / BW
    // lane groups of a block write rows 4 apart, and land on different
    // banks), then finish it 16 lanes per row
    float* st = reinterpret_cast<float*>(smem);
    auto st_off = [&](int r, int c) -> int { return r * 128 + (c ^ (BW * ((r >> 2) & (64 / BW - 1)))); };
    const int j16 = tid & 15;
    const RopeCoef rc = rope_coef(p.qkv.theta, j16);
    constexpr int HPT = BN / 128;                      // heads per tile
    const int heads = (int)(p.N / 128);
    // sequence and position of this thread's first row (one 64-bit
    // division); the rows after it step by NT / 16 and wrap at T
    const int64_t mf = m0 + (tid >> 4);
    const int bf0 = (int)(mf / p.qkv.T), tf0 = (int)(mf - (int64_t)bf0 * p.qkv.T);
#pragma unroll
    for (int hh = 0; hh < HPT; ++hh) {
      __syncthreads();   // the ring (first head) or the previous head's staging is no longer read
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int c0 = ncol(j);
        if (c0 / 128 != hh) continue;
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int e = 0; e < NE; ++e)
            st[st_off(wm * WM + i * BW + 8 * (e >> 2) + 4 * lh + (e & 3), c0 - hh * 128 + lr)] = acc[i][j][e];
      }
      __syncthreads();
      const int h = tn * HPT + hh;
      const NormW nw = norm_w(norm_of(p.qkv, h), j16);
      int b = bf0, t = tf0;
      for (int r = tid >> 4; r < BM; r += NT / 16) {
        const int64_t m = m0 + r;
        if (m < M && h < heads) {
          // four consecutive columns are one 16-byte group of the staged tile
          const f32x4 v0 = *reinterpret_cast<const f32x4*>(st + st_off(r, 4 * j16));
          const f32x4 v1 = *reinterpret_cast<const f32x4*>(st + st_off(r, 64 + 4 * j16));
          float x[8] = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
          qkv_finish_at(p.qkv, x, m, b, t, h, j16, rc, nw);
        }
        t += NT / 16;
        if (t >= p.qkv.T) {
          const int q = t / p.qkv.T;
          b += q;
          t -= q * p.qkv.T;
        }
      }
    }
    return;
  }
  if (EPI == EPI_F32) {
    float* C = static_cast<float*>(p.C) + (SPLIT ? (int64_t)blockIdx.y * M * p.ldc : 0);
    const bool full = m0 + BM <= M && (int64_t)(tn + 1) * BN <= p.N;
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int64_t gn = (int64_t)tn * BN + ncol(j) + lr;
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int e = 0; e < NE; ++e) {
          const int64_t gm = m0 + wm * WM + i * BW + 8 * (e >> 2) + 4 * lh + (e & 3);
          if (full || (gm < M && gn < p.N)) C[gm * p.ldc + gn] = acc[i][j][e];
        }
    }
    return;
  }
  // bf16 outputs: each wave stages its tile in LDS (row-major, 16-byte
  // chunks XOR-swizzled by row), then writes whole 16-byte row chunks.
  constexpr int OC = EPI == EPI_SILU_BF16 ? WN / 2 : WN;     // output columns per wave
  constexpr int OCH = OC / 8;                                // 16-byte chunks per staged row
  // rows staged per pass: the whole wave tile, or 32 rows at a time where
  // that does not fit the ring (256 x 320 tiles)
  constexpr int PR = WM * OC * 2 * WGM * WGN <= S * STAGE * 2 ? WM : 32;
  static_assert(PR * OC * 2 * WGM * WGN <= S * STAGE * 2, "staging does not fit");
  bf16* so = smem + wave * (PR * OC);
  // the staging area overlaps ring stages that slower waves may still be
  // reading for the last K block
  __syncthreads();
  // chunk c of staged row r sits at chunk och(r, c): XOR-swizzled by the
  // row, or rotated by it where a row's chunk count is not a power of two
  auto och = [&](int r, int c) { return (OCH & (OCH - 1)) == 0 ? c ^ (r & (OCH - 1)) : (c + r) % OCH; };
  auto so_idx = [&](int r, int c) { return r * OC + (och(r, c >> 3) << 3) + (c & 7); };
  const int64_t ncols = EPI == EPI_SILU_BF16 ? p.li : p.N;
  const int64_t col0 = EPI == EPI_SILU_BF16 ? (int64_t)tn * (BN / 2) + wn * (WN / 2) : (int64_t)tn * BN + wn * WN;
  bf16* C = static_cast<bf16*>(p.C);
  const bool vec = (p.ldc % 8) == 0;
  // A pass rewrites staging rows the previous pass read; one wave's LDS
  // accesses run in order, so it needs no wait.
#pragma unroll
  for (int ps = 0; ps < WM / PR; ++ps) {
  // (C^T layout: row i * BW + lr, columns j * BW + 8 * g4 + 4 * lh .. + 3)
  // (SI: block j gives output columns j * 16 + 8 * g4 + 4 * lh .. + 3 from
  // its values e = 4 * g4 + q, e < 8, and e + 8)
#pragma unroll
  for (int j = 0; j < (EPI == EPI_SILU_BF16 && !SI ? TN / 2 : TN); ++j)
#pragma unroll
    for (int i = ps * (PR / BW); i < (ps + 1) * (PR / BW); ++i)
#pragma unroll
      for (int g4 = 0; g4 < (SI ? NE / 8 : NE / 4); ++g4) {
        float v[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int e = 4 * g4 + q;
          if (EPI == EPI_SILU_BF16) {
            const float g = acc[i][j][e], u = SI ? acc[i][j][e + 8] : acc[i][j + TN / 2][e];
            v[q] = silu_mul(g, u);
          } else {
            v[q] = acc[i][j][e];
          }
        }
        const int c = SI ? j * 16 + 8 * g4 + 4 * lh : j * BW + 8 * g4 + 4 * lh;
        *reinterpret_cast<u32x2*>(so + so_idx(i * BW - ps * PR + lr, c)) =
            u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
      }
  __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): this wave's staging writes are done
  __builtin_amdgcn_wave_barrier();
  const int64_t row0 = m0 + wm * WM + ps * PR;
  // a pass wholly inside the output (the common case): no per-chunk bounds,
  // 32-bit offsets from the pass's first element (rows below 2^22 elements)
  if (vec && row0 + PR <= M && col0 + OC <= ncols && p.ldc < (int64_t(1) << 22)) {
    bf16* cb = C + row0 * p.ldc + col0;
    const uint32_t ldc = (uint32_t)p.ldc;
#pragma unroll 4
    for (int q = lane; q < PR * OCH; q += 64) {
      const int r = q / OCH, c = q % OCH;
      const u32x4 v = *reinterpret_cast<const u32x4*>(so + r * OC + (och(r, c) << 3));
      // streaming store: the output is not read again by this kernel, and
      // allocating it in L2 would evict the A/B panels that other tiles
      // still read (the lm_head writes four times the bytes it reads)
      __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(cb + ((uint32_t)r * ldc + (uint32_t)(c * 8))));
    }
    continue;
  }
#pragma unroll 4
  for (int q = lane; q < PR * OCH; q += 64) {
    const int r = q / OCH, c = q % OCH;
    const int64_t gm = row0 + r, gc = col0 + c * 8;
    if (gm >= M || gc >= ncols) continue;
    const u32x4 v = *reinterpret_cast<const u32x4*>(so + r * OC + (och(r, c) << 3));
    if (vec && gc + 8 <= ncols) {
      // streaming store (as above)
      __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(C + gm * p.ldc + gc));
    } else {
#pragma unroll
      for (int t = 0; t < 8; ++t)
        if (gc + t < ncols) C[gm * p.ldc + gc + t] = __builtin_bit_cast(bf16, (uint16_t)(v[t >> 1] >> (16 * (t & 1))));
    }
  }
  }
}

// 16-byte chunk swizzle of the persistent epilogue's 32 x 64 staging tile:
// the 8-byte writes of one instruction cover 32 rows x one chunk, and rows
// of equal parity start on the same bank, so the chunk is permuted by
// (row / 2) % 8 to spread each parity's 16 rows over all 8 chunk slots.
__device__ __forceinline__ int stage_swz(int r) { return (r >> 1) & 7; }

// Persistent variant for grids of many tiles (bf16 and silu epilogues): one
// workgroup per CU walks a share of the tiles of its XCD, and the LDS ring
// runs on across tile boundaries, so the next tile's first block is already
// in LDS (and its first operands in VGPRs) when a tile ends, and no
// workgroup launch, pipeline fill or ring drain separates two tiles.  The
// epilogue stages each wave's outputs, 32 rows x 64 columns at a time,
// through a 4 KB LDS region of its own next to the ring, so it needs no
// workgroup barrier and never touches a ring stage.  The MFMAs take the B
// (weight) fragment as their first operand and so accumulate C^T: each lane
// then holds four consecutive output columns of one row, staged by one
// 8-byte LDS write instead of four 2-byte ones.
//
// Tile order: the tiles (GROUP_M-grouped as in gemm_kernel) are cut into 8
// contiguous ranges, one per XCD; workgroup b runs on XCD b % 8 (the
// dispatcher deals workgroups round-robin) and takes every G-th tile of its
// XCD's range, G = the XCD's workgroup count, so the CUs of one XCD work on
// neighbouring tiles at any time and share A and B panels in its L2.
template <int BM, int BN, int WGM, int WGN, int EPI, int GROUP_M, int S, int BK = 64>
__global__ __launch_bounds__(WGM * WGN * 64)
__attribute__((amdgpu_waves_per_eu(WGM * WGN / 4, WGM * WGN / 4)))
void gemm_persist_kernel(GemmProblem p, int tiles_m, int tiles_n) {
  static_assert(EPI == EPI_BF16 || EPI == EPI_SILU_BF16, "bf16 outputs only");
  constexpr int NW = WGM * WGN, NT = NW * 64;
  constexpr int WM = BM / WGM, WN = BN / WGN;
  constexpr int TM = WM / 32, TN = WN / 32;
  constexpr int KC = BK / 8;
  constexpr int STAGE = (BM + BN) * BK;
  constexpr int RING = S * STAGE * 2;               // bytes
  constexpr int OCW = EPI == EPI_SILU_BF16 ? WN / 2 : WN;   // output columns per wave
  static_assert(OCW % 64 == 0 && TN % 2 == 0, "epilogue passes are 32 x 64");
  static_assert(RING + NW * 4096 <= 163840, "ring and staging must fit the CU's LDS");
  __shared__ __attribute__((aligned(16))) bf16 smem[(RING + NW * 4096) / 2];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int wm = wave_u / WGN, wn = wave_u % WGN;
  const int lr = lane & 31, lh = lane >> 5;
  const int64_t M = p.M, K = p.K;
  const int nk = (int)((K + BK - 1) / BK);
  const bool tail = K % BK != 0;

  // this workgroup's tiles: first + j * step, j < n_my
  int first, step, n_my;
  {
    const int ntiles = tiles_m * tiles_n;
    const int xcd = blockIdx.x % kXcds, slot = blockIdx.x / kXcds;
    const int per = ntiles / kXcds, rem = ntiles % kXcds;
    const int cs = xcd * per + min(xcd, rem), len = per + (xcd < rem);
    const int g = ((int)gridDim.x - xcd + kXcds - 1) / kXcds;
    first = cs + slot;
    step = g;
    n_my = slot < len ? (len - slot + g - 1) / g : 0;
  }
  auto coords = [&](int j, int64_t& m0, int64_t& nrow0) __attribute__((always_inline)) {
    const int t = first + j * step;
    const int group_m = p.group_m > 0 ? p.group_m : GROUP_M;
    const int per_group = group_m * tiles_n;
    const int gi = t / per_group;
    const int first_m = gi * group_m;
    const int gm = min(tiles_m - first_m, group_m);
    const int r = t - gi * per_group;
    m0 = (int64_t)(first_m + r % gm) * BM;
    nrow0 = (int64_t)(r / gm) * (EPI == EPI_SILU_BF16 ? BN / 2 : BN);
  };

  constexpr int RPI = 512 / BK;             // rows per 1 KB load instruction
  static_assert(BM % (RPI * NW) == 0 && BN % (RPI * NW) == 0, "row groups must split evenly");
  constexpr int A_G = BM / (RPI * NW), B_G = BN / (RPI * NW), NV = A_G + B_G;
  const int grow = lane / KC, gpc = lane % KC;
  const int64_t lda_b = p.lda * 2, ldb_b = p.ldb * 2;
  // slice offsets: a per-lane part per operand plus the slice's first row
  // times the row pitch (wave-uniform; every slice of a wave starts on the
  // same row modulo the swizzle's 16-row period)
  static_assert(EPI != EPI_SILU_BF16 || (BN / 2) % 16 == 0, "gate/up halves in whole 16-row units");
  auto b_up = [&](int g) { return EPI == EPI_SILU_BF16 && g * RPI >= BN / 2; };
  auto src_row0 = [&](bool isA, int g) -> int { return g * RPI - (!isA && b_up(g) ? BN / 2 : 0); };
  const uint32_t lsw = (uint32_t)(swz<BK>(((wave_u * RPI) & 15) + grow, gpc) << 4);
  const uint32_t lane_a = (uint32_t)(grow * lda_b) + lsw, lane_b = (uint32_t)(grow * ldb_b) + lsw;
  // descriptors of the tile that the loads are filling (they run ahead of
  // the MFMAs by S - 1 blocks, so into the next tile near a tile's end)
  __amdgpu_buffer_rsrc_t ra, rg, ru;
  auto set_dma_tile = [&](int j) __attribute__((always_inline)) {
    int64_t m0, nrow0;
    coords(j, m0, nrow0);
    const int64_t nrows = EPI == EPI_SILU_BF16 ? p.li - nrow0 : p.N - nrow0;
    ra = make_rsrc(p.A + m0 * p.lda, (M - m0) * lda_b);
    rg = make_rsrc(p.B + nrow0 * p.ldb, nrows * ldb_b);
    ru = make_rsrc(p.B + ((p.up_off ? p.up_off : p.li) + nrow0) * p.ldb, nrows * ldb_b);
  };
  auto slice = [&](int v, bf16* st, uint32_t ko) __attribute__((always_inline)) {
    if (v < A_G) {
      const int g = wave_u + v * NW;
      dma16(ra, lane_a + (uint32_t)(src_row0(true, g) * lda_b) + ko, st + g * RPI * BK);
    } else {
      const int g = wave_u + (v - A_G) * NW;
      dma16(b_up(g) ? ru : rg, lane_b + (uint32_t)(src_row0(false, g) * ldb_b) + ko, st + BM * BK + g * RPI * BK);
    }
  };
  int dj = 0, dkb = 0;                    // tile and K block of the next load
  auto dma_next = [&](int buf) __attribute__((always_inline)) {
    if (dkb == 0) set_dma_tile(dj);
    bf16* st = smem + buf * STAGE;
    const uint32_t ko = (uint32_t)dkb * (BK * 2);
#pragma unroll
    for (int v = 0; v < NV; ++v) slice(v, st, ko);
    if (++dkb == nk) {
      dkb = 0;
      ++dj;
    }
  };
  // one slice of the next load (issued inside the fenced MFMA stream)
  auto dma_slice = [&](int v, int buf) __attribute__((always_inline)) {
    slice(v, smem + buf * STAGE, (uint32_t)dkb * (BK * 2));
  };
  auto zero_tail = [&](int buf) __attribute__((always_inline)) {
    bf16* st = smem + buf * STAGE;
    const int64_t k0 = (int64_t)(nk - 1) * BK;
    for (int q = tid; q < (BM + BN) * KC; q += NT) {
      const int row = q / KC, lc = q % KC;
      if (k0 + lc * 8 >= K) *reinterpret_cast<u32x4*>(st + row * BK + swz<BK>(row, lc) * 8) = u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto ncol = [&](int j) __attribute__((always_inline)) -> int {
    if (EPI == EPI_SILU_BF16)
      return j < TN / 2 ? wn * (WN / 2) + j * 32 : BN / 2 + wn * (WN / 2) + (j - TN / 2) * 32;
    return wn * WN + j * 32;
  };

  f32x16 acc[TM][TN];
  auto zero_acc = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
  };
  zero_acc();
  bf16x8 af[2][TM], bfr[2][TN];
  constexpr int KS = BK / 16;
  constexpr int NF = TM + TN, NMF = TM * TN;
  constexpr int NPAIR = (NMF + 1) / 2;
  constexpr int RDP = (NF + NPAIR - 1) / NPAIR;
  constexpr int H1 = NPAIR / 2;
  constexpr int RDP2 = (NF + (NPAIR - H1) - 1) / (NPAIR - H1);
  auto read_frag = [&](const bf16* sA, const bf16* sB, int ks, int fs, int x) __attribute__((always_inline)) {
    // lane row lr plus a multiple of 16: a per-lane part per k chunk and a
    // wave-uniform row offset
    const int c = ks * 2 + lh, lo = lr * BK + swz<BK>(lr, c) * 8;
    if (x == 0 || x > TN) {
      const int i = x == 0 ? 0 : x - TN;
      af[fs][i] = *reinterpret_cast<const bf16x8*>(sA + (wm * WM + i * 32) * BK + lo);
    } else {
      bfr[fs][x - 1] = *reinterpret_cast<const bf16x8*>(sB + ncol(x - 1) * BK + lo);
    }
  };
  auto mfma_pair = [&](int fs, int pr) __attribute__((always_inline)) {
#pragma unroll
    for (int m = 2 * pr; m < 2 * pr + 2 && m < NMF; ++m)
      acc[m / TN][m % TN] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[fs][m % TN], af[fs][m / TN],
                                                                  acc[m / TN][m % TN], 0, 0, 0);
  };
  // the block just landed in `buf` is read next: all waves have their
  // loads of it (vmcnt, before the call) and are done reading the stage it
  // frees (lgkmcnt); a tile's last block also has its K tail cleared
  auto settle = [&](int buf, bool last_of_tile) __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(0xC07F);
    asm volatile("s_barrier" ::: "memory");
    if (tail && last_of_tile) {
      zero_tail(buf);
      __builtin_amdgcn_s_waitcnt(0xC07F);
      asm volatile("s_barrier" ::: "memory");
    }
  };

  // epilogue of tile j through this wave's staging region
  bf16* so = smem + RING / 2 + wave_u * 2048;
  auto epilogue = [&](int j) __attribute__((always_inline)) {
    int64_t m0, nrow0;
    coords(j, m0, nrow0);
    const int64_t ncols = EPI == EPI_SILU_BF16 ? p.li : p.N;
    const int64_t col0 = nrow0 + wn * OCW;       // output column of this wave's first column
    bf16* C = static_cast<bf16*>(p.C);
    const bool vec = (p.ldc % 8) == 0;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int ps = 0; ps < OCW / 64; ++ps) {
#pragma unroll
        for (int jj = 0; jj < 2; ++jj)
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            float v[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int e = 4 * g4 + q;
              if (EPI == EPI_SILU_BF16) {
                const float g = acc[i][ps * 2 + jj][e], u = acc[i][ps * 2 + jj + TN / 2][e];
                v[q] = silu_mul(g, u);
              } else {
                v[q] = acc[i][ps * 2 + jj][e];
              }
            }
            // row lr, columns jj * 32 + 8 * g4 + 4 * lh .. + 3: one 8-byte write
            const u32x2 w{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
            *reinterpret_cast<u32x2*>(so + lr * 64 + (((jj * 4 + g4) ^ stage_swz(lr)) << 3) + 4 * lh) = w;
          }
        __builtin_amdgcn_s_waitcnt(0xC07F);
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int q = lane + 64 * u, r = q >> 3, cc = q & 7;
          const u32x4 v = *reinterpret_cast<const u32x4*>(so + r * 64 + ((cc ^ stage_swz(r)) << 3));
          const int64_t gm = m0 + wm * WM + i * 32 + r, gc = col0 + ps * 64 + cc * 8;
          if (gm < M && gc < ncols) {
            if (vec && gc + 8 <= ncols) {
              __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(C + gm * p.ldc + gc));
            } else {
#pragma unroll
              for (int t = 0; t < 8; ++t)
                if (gc + t < ncols)
                  C[gm * p.ldc + gc + t] = __builtin_bit_cast(bf16, (uint16_t)(v[t >> 1] >> (16 * (t & 1))));
            }
          }
        }
        __builtin_amdgcn_s_waitcnt(0xC07F);   // reads done before the next pass overwrites
        __builtin_amdgcn_wave_barrier();
      }
  };

  const int total = n_my * nk;
  int ckb = 0, cj = 0;                    // K block and tile of the block being computed
  // block gb: stage gb % S; it issues block gb + S - 1 (DMA) and, unless it
  // is the last one, waits for block gb + 1 and reads its first operands
  auto block = [&](auto dma_tag, auto next_tag, int gb) __attribute__((always_inline)) {
    constexpr bool DMA = decltype(dma_tag)::value;
    constexpr bool NEXT = decltype(next_tag)::value;
    const int cur = gb % S;
    const bf16* sA = smem + cur * STAGE;
    const bf16* sB = sA + BM * BK;
    const int nxt = (gb + 1) % S;
    const bf16* nA = smem + nxt * STAGE;
    const bf16* nB = nA + BM * BK;
    const int dbuf = (gb + S - 1) % S;
    if constexpr (DMA) {
      if (dkb == 0) set_dma_tile(dj);
    }
    __builtin_amdgcn_sched_barrier(0);
    int v = 0;
#pragma unroll
    for (int ks = 0; ks < KS - 1; ++ks) {
#pragma unroll
      for (int pr = 0; pr < NPAIR; ++pr) {
        mfma_pair(ks & 1, pr);
#pragma unroll
        for (int x = pr * RDP; x < pr * RDP + RDP && x < NF; ++x) read_frag(sA, sB, ks + 1, (ks + 1) & 1, x);
        if constexpr (DMA) {
          if (ks == 0) {
            while (v < NV && (pr + 1) * NV >= (v + 1) * NPAIR) dma_slice(v++, dbuf);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if constexpr (DMA) {
      if (++dkb == nk) {
        dkb = 0;
        ++dj;
      }
    }
#pragma unroll
    for (int pr = 0; pr < H1; ++pr) {
      mfma_pair(1, pr);
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (NEXT) {
      if constexpr (DMA)
        wait_vm<(S - 2) * NV>();
      else
        wait_vm0();
      settle(nxt, nk == 1 || ckb + 1 == nk - 1);
      __builtin_amdgcn_sched_barrier(0);
    }
    // at a tile's end the next operands are read after the epilogue, which
    // then has the registers of the fragment set to itself
    const bool tile_end = ckb == nk - 1;
#pragma unroll
    for (int pr = H1; pr < NPAIR; ++pr) {
      mfma_pair(1, pr);
      if constexpr (NEXT) {
        if (!tile_end) {
#pragma unroll
          for (int x = (pr - H1) * RDP2; x < (pr - H1) * RDP2 + RDP2 && x < NF; ++x) read_frag(nA, nB, 0, 0, x);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if (tile_end) {
      epilogue(cj);
      zero_acc();
      if constexpr (NEXT) {
#pragma unroll
        for (int x = 0; x < NF; ++x) read_frag(nA, nB, 0, 0, x);
      }
    }
    // both counters stored on every path (increments of one or the other
    // became a select of their addresses, which kept them in scratch)
    cj += tile_end ? 1 : 0;
    ckb = tile_end ? 0 : ckb + 1;
  };

  if (total > 0) {
    const int pro = total < S - 1 ? total : S - 1;
    for (int blk = 0; blk < pro; ++blk) dma_next(blk);
    if (pro - 1 == S - 2)
      wait_vm<(S - 2) * NV>();
    else
      wait_vm0();
    settle(0, nk == 1);
#pragma unroll
    for (int x = 0; x < NF; ++x) read_frag(smem, smem + BM * BK, 0, 0, x);
  }
  int gb = 0;
  for (; gb + S - 1 < total; ++gb) block(std::true_type{}, std::true_type{}, gb);
  for (; gb + 1 < total; ++gb) block(std::false_type{}, std::true_type{}, gb);
  if (gb < total) block(std::false_type{}, std::false_type{}, gb);
}

// Sums split-K partials [splits, M, N] in a fixed order and applies the
// final epilogue.  Four consecutive columns per thread; the loads of all
// splits (at most kMaxSplits) are issued before the first add, so a thread
// waits for memory once, not once per split.
constexpr int kMaxSplits = 8;

template <int EPI>
__global__ __launch_bounds__(256) void splitk_reduce(const float* __restrict__ part, int splits, int64_t M,
                                                     int64_t N, void* out, int64_t ldc, int64_t li) {
  const int64_t cols = EPI == EPI_SILU_BF16 ? li : N;
  const int64_t quads = M * (cols / 4);
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < quads; i += (int64_t)gridDim.x * 256) {
    const int64_t m = i / (cols / 4), n = (i - m * (cols / 4)) * 4;
    f32x4 g[kMaxSplits], u[kMaxSplits];
#pragma unroll
    for (int z = 0; z < kMaxSplits; ++z)
      if (z < splits) {
        const float* src = part + ((int64_t)z * M + m) * N + n;
        g[z] = *reinterpret_cast<const f32x4*>(src);
        if (EPI == EPI_SILU_BF16) u[z] = *reinterpret_cast<const f32x4*>(src + li);
      }
    f32x4 sg = {0.f, 0.f, 0.f, 0.f}, su = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int z = 0; z < kMaxSplits; ++z)
      if (z < splits) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          sg[e] += g[z][e];
          if (EPI == EPI_SILU_BF16) su[e] += u[z][e];
        }
      }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (EPI == EPI_SILU_BF16)
        static_cast<bf16*>(out)[m * ldc + n + e] = f2bf(silu_mul(sg[e], su[e]));
      else if (EPI == EPI_BF16)
        static_cast<bf16*>(out)[m * ldc + n + e] = f2bf(sg[e]);
      else
        static_cast<float*>(out)[m * ldc + n + e] = sg[e];
    }
  }
}

// Sums the split-K partials of a merged QKV projection in split order and
// finishes each (row, head), 16 lanes per unit.
__global__ __launch_bounds__(256) void splitk_reduce_qkv(const float* __restrict__ part, int splits, int64_t M,
                                                         int64_t N, QkvArgs a) {
  const int heads = (int)(N / 128);
  const int j = threadIdx.x & 15;
  const RopeCoef rc = rope_coef(a.theta, j);
  const bool narrow = M * heads < 0x7fffffff;   // 32-bit unit indices
  for (int64_t u = ((int64_t)blockIdx.x * 256 + threadIdx.x) >> 4; u < M * heads; u += (int64_t)gridDim.x * 16) {
    const int64_t m = narrow ? (int64_t)((uint32_t)u / (uint32_t)heads) : u / heads;
    const int h = (int)(u - m * heads);
    f32x4 v0[kMaxSplits], v1[kMaxSplits];
#pragma unroll
    for (int z = 0; z < kMaxSplits; ++z)
      if (z < splits) {
        const float* src = part + ((int64_t)z * M + m) * N + (int64_t)h * 128 + 4 * j;
        v0[z] = *reinterpret_cast<const f32x4*>(src);
        v1[z] = *reinterpret_cast<const f32x4*>(src + 64);
      }
    float x[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int z = 0; z < kMaxSplits; ++z)
      if (z < splits) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          x[e] += v0[z][e];
          x[4 + e] += v1[z][e];
        }
      }
    qkv_finish(a, x, m, h, j, rc);
  }
}

// ---- tile-shape choice -----------------------------------------------------
//
// Each variant is a tile shape, a wave layout and an LDS ring depth.  The
// planner prices every (variant, split) pair with a two-sided model and keeps
// the cheapest:
//   compute: rounds of resident workgroups x (K blocks x time per K block +
//            output tile write), with the per-block times measured on this
//            GPU at full load;
//   memory:  weight bytes (+ fp32 split partials, written and read back) at
//            the streaming rate, or at the per-workgroup rate when too few
//            workgroups are resident to fill HBM;
// plus a fixed cost per launch (a split adds the reduction launch).
struct Variant {
  int bm, bn, stages;
  int resident;        // workgroups one CU holds (LDS-limited)
  float t_kb_us;       // time per 64-wide K block per resident round at full load
  bool silu;           // the tile can hold gate/up pairs
};
// V256x320: 256 x 320 tiles (waves of 64 x 160).  The row-parallel
// projections' N = 5120 is 16 such tiles: at 4096 rows that is one round of
// 256 tiles, where 256-wide tiles need 1.25 rounds (or a second launch for
// the last 1024 columns); the 32B gate_up (12800 SiLU outputs, 160 per
// tile) is five whole rounds at 4096 rows, where 256-wide tiles need 6.25.
// On long grids at K = 5120 it also beats 256-wide tiles per flop (the
// 32B lm_head 8-10%, at 2048 and 4096 rows); its time per K block is the
// measured one, below the 1.25 x 256 x 256 one its area would give.  Bf16,
// fp32 and SiLU outputs (a 320-wide tile does not hold whole 128-column
// heads); grids beyond one round only unsplit and at K >= 2048.
enum VariantId {
  V256x256, V256x128, V128x128_4, V128x128_2, V128x64_3, V128x64_6, V64x128_3, V64x64_8, V256x320, V128x192,
  V_COUNT
};
constexpr Variant kVariants[V_COUNT] = {
    {256, 256, 2, 1, 1.96f, true}, {256, 128, 3, 1, 0.98f, true}, {128, 128, 4, 1, 0.59f, true},
    {128, 128, 2, 2, 1.08f, true}, {128, 64, 3, 2, 0.73f, true},  {128, 64, 6, 1, 0.45f, true},
    {64, 128, 3, 2, 0.75f, true},  {64, 64, 8, 1, 0.30f, false},  {256, 320, 2, 1, 2.29f, true},
    {128, 192, 4, 1, 0.885f, true},
};
// Constants fitted to a sweep of every (variant, split) plan over the
// decode, prefill, lm_head and decode-argmax shapes of the Qwen3-0.6B / 32B
// shards on MI355X (27 shapes; the chosen plans are within 1% of the
// measured best on average, 26 us of regret summed over all of them).
constexpr double kHbmBytesPerUs = 5.5e6;       // sustained weight streaming, bytes per microsecond
constexpr double kWgBytesPerUs = 3.0e4;        // one workgroup's streaming rate
constexpr double kLaunchUs = 2.0;
constexpr double kReduceUs = 5.0;              // the split-K reduction kernel: launch and ramp
constexpr double kEpiUsPerKB = 0.03;           // tile write-out per resident round

struct Plan { int v; int splits; int64_t kps; int tiles_m, tiles_n; };

// consumer_sums: the split partials are summed by the next kernel, so a
// split costs their traffic but no reduction launch
double plan_cost(const Variant& v, int64_t M, int64_t N, int64_t K, int epi, int64_t splits, int64_t* tm_out,
                 int64_t* tn_out, bool consumer_sums = false) {
  const int64_t ncols = epi == EPI_SILU_BF16 ? N / 2 : N;
  const int64_t bn_out = epi == EPI_SILU_BF16 && splits == 1 ? v.bn / 2 : v.bn;
  const int64_t cols = splits == 1 ? ncols : N;   // split partials use the plain column order
  const int64_t tm = (M + v.bm - 1) / v.bm, tn = (cols + bn_out - 1) / bn_out;
  *tm_out = tm;
  *tn_out = tn;
  const int64_t wgs = tm * tn * splits;
  const int64_t resident = (int64_t)kCUs * v.resident;
  const int64_t rounds = (wgs + resident - 1) / resident;
  const int64_t kb = (K / 64 + splits - 1) / splits + (K % 64 != 0);
  const double out_kb = (double)v.bm * v.bn * (splits > 1 || epi == EPI_F32 ? 4 : 2) / 1024.0;
  const double t_comp = rounds * (kb * v.t_kb_us + out_kb * kEpiUsPerKB);
  const double partial = splits > 1 ? (double)splits * M * N * 4 : 0.0;
  const double bytes = (double)N * K * 2 + (double)M * K * 2 + partial;
  // Idle CUs are charged through the rate: a round with fewer workgroups
  // than it takes to saturate HBM streams its share of the bytes at their
  // summed per-workgroup rate.  That is a grid below one round, and for a
  // tile that fits once per CU also the ragged last round of a longer grid;
  // with two per CU the leftover workgroups start beside running ones or
  // alone on a CU, and measured no such loss.  (Sweeps of every plan on the
  // decode shapes of the 0.6B and 32B shards put the chosen plan within
  // about 1 us of the measured best.)
  auto round_us = [&](int64_t active) {
    const double rate = active * kWgBytesPerUs < kHbmBytesPerUs ? active * kWgBytesPerUs : kHbmBytesPerUs;
    return (double)active * (bytes / (double)wgs) / rate;
  };
  const int64_t full_rounds = v.resident == 1 ? wgs / resident : 0;
  const int64_t last = v.resident == 1 ? wgs % resident : (wgs < resident ? wgs : resident);
  const double t_mem = v.resident == 1 ? (double)full_rounds * round_us(resident) + (last ? round_us(last) : 0.0)
                                       : (double)wgs / (double)last * round_us(last);
  // the reduction runs after the GEMM: it reads every partial and writes C
  const double t_red = splits <= 1 ? 0.0
                      : consumer_sums ? partial / kHbmBytesPerUs
                                      : (partial + (double)M * ncols * (epi == EPI_F32 ? 4 : 2)) / kHbmBytesPerUs + kReduceUs;
  return (t_comp > t_mem ? t_comp : t_mem) + kLaunchUs + t_red;
}

Plan make_plan(int64_t M, int64_t N, int64_t K, int epi, bool allow_split, bool consumer_sums = false,
               double* cost_out = nullptr, bool gathered = false) {
  Plan best{V256x256, 1, K, 0, 0};
  double best_cost = 1e300;
  const int64_t kblocks = (K + 63) / 64;
  // the reductions read the partials four columns at a time
  const bool quad_cols = N % 4 == 0 && (epi != EPI_SILU_BF16 || (N / 2) % 4 == 0);
  for (int vi = 0; vi < V_COUNT; ++vi) {
    const Variant& v = kVariants[vi];
    for (int64_t sp = 1; sp <= kMaxSplits; ++sp) {
      if (sp > 1 && (!allow_split || !quad_cols || kblocks < 4 * sp)) break;
      if (epi == EPI_SILU_BF16 && !v.silu) continue;
      if (wide_tile(v.bn) && (epi == EPI_QKV || epi == EPI_ARGMAX || gathered)) continue;
      if (v.bn == 192 && (epi != EPI_SILU_BF16 || M <= kMf16RowsPlan || sp > 1)) continue;
      if (epi == EPI_QKV && sp == 1 && !qkv_tile_ok(v.bm, v.bn, v.stages)) continue;
      int64_t tm, tn;
      // a split must win clearly: its partials also cost workspace
      const double c = plan_cost(v, M, N, K, epi, sp, &tm, &tn, consumer_sums) * (sp > 1 ? 1.05 : 1.0);
      // beyond one round only unsplit and with at least 32 K blocks: on the
      // 0.6B lm_head (K = 1024) the persistent kernel measured 2-3% faster
      if (wide_tile(v.bn) && tm * tn * sp > kCUs && (sp > 1 || K < 32 * 64)) continue;
      if (c < best_cost * 0.999) {
        best_cost = c;
        const int64_t kps = sp == 1 ? K : ((kblocks + sp - 1) / sp) * 64;
        best = Plan{vi, sp == 1 ? 1 : (int)((K + kps - 1) / kps), kps, (int)tm, (int)tn};
      }
    }
  }
  if (cost_out) *cost_out = best_cost;
  return best;
}

// timing mark after a GEMM-family launch: kernel, tile, epilogue and the
// launched product M x N x K (N = rows of B, so the launch does 2 M N K flops)
const char* const kEpiNames[] = {"bf16", "f32", "silu", "qkv", "argmax"};
void mark_gemm(hipStream_t s, const char* kern, int bm, int bn, int stages, int epi, const GemmProblem& p) {
  if (!kmarks_armed()) return;
  char buf[128];
  snprintf(buf, sizeof buf, "%s<%d,%d,%d>/%s[%lldx%lldx%lld]", kern, bm, bn, stages, kEpiNames[epi],
           (long long)p.M, (long long)p.N, (long long)p.K);
  kmark(s, buf);
}

// finish = false: a split plan stops after the partials (the consumer sums
// them itself)
template <int BM, int BN, int WGM, int WGN, int S, bool MF16 = false>
hipError_t launch_tile(const GemmProblem& p, int epi, const Plan& pl, void* scratch, hipStream_t s,
                       bool finish = true) {
  constexpr int NT = WGM * WGN * 64;
  constexpr int GM = 8;
  if (pl.splits > 1) {
    GemmProblem q = p;
    q.C = scratch;
    q.ldc = p.N;
    dim3 grid(pl.tiles_m * pl.tiles_n, pl.splits);
    gemm_kernel<BM, BN, WGM, WGN, EPI_F32, true, GM, S, 64, MF16><<<grid, NT, 0, s>>>(q, pl.tiles_m, pl.tiles_n, pl.kps);
    mark_gemm(s, "gemm_splitk", BM, BN, S, epi, p);
    if (!finish) return hipGetLastError();
    const int64_t cols = epi == EPI_SILU_BF16 ? p.li : p.N;
    int64_t g = (p.M * (cols / 4) + 255) / 256;
    if (g > 4096) g = 4096;
    if (epi == EPI_QKV) {
      int64_t gq = (p.M * (p.N / 128) * 16 + 255) / 256;
      if (gq > 4096) gq = 4096;
      splitk_reduce_qkv<<<(int)gq, 256, 0, s>>>((const float*)scratch, pl.splits, p.M, p.N, p.qkv);
    } else if (epi == EPI_SILU_BF16)
      splitk_reduce<EPI_SILU_BF16><<<(int)g, 256, 0, s>>>((const float*)scratch, pl.splits, p.M, p.N, p.C, p.ldc, p.li);
    else if (epi == EPI_BF16)
      splitk_reduce<EPI_BF16><<<(int)g, 256, 0, s>>>((const float*)scratch, pl.splits, p.M, p.N, p.C, p.ldc, 0);
    else
      splitk_reduce<EPI_F32><<<(int)g, 256, 0, s>>>((const float*)scratch, pl.splits, p.M, p.N, p.C, p.ldc, 0);
    kmark(s, epi == EPI_QKV ? "splitk_reduce/qkv" : "splitk_reduce");
    return hipGetLastError();
  }
  dim3 grid(pl.tiles_m * pl.tiles_n);
  if constexpr ((BN / WGN / 32) % 2 == 0 || !MF16) {
    if (epi == EPI_SILU_BF16) {
      gemm_kernel<BM, BN, WGM, WGN, EPI_SILU_BF16, false, GM, S, 64, MF16><<<grid, NT, 0, s>>>(p, pl.tiles_m, pl.tiles_n, p.K);
      mark_gemm(s, "gemm_tile", BM, BN, S, EPI_SILU_BF16, p);
      return hipGetLastError();
    }
  }
  if constexpr (qkv_tile_ok(BM, BN, S)) {
    if (epi == EPI_QKV) {
      gemm_kernel<BM, BN, WGM, WGN, EPI_QKV, false, GM, S, 64, MF16><<<grid, NT, 0, s>>>(p, pl.tiles_m, pl.tiles_n, p.K);
      mark_gemm(s, "gemm_tile", BM, BN, S, EPI_QKV, p);
      return hipGetLastError();
    }
  }
  // the planner never picks a variant that cannot run the epilogue
  if (epi == EPI_SILU_BF16 || epi == EPI_QKV) return hipErrorInvalidValue;
  if (epi == EPI_ARGMAX) {
    if constexpr (!wide_tile(BN)) {
      gemm_kernel<BM, BN, WGM, WGN, EPI_ARGMAX, false, GM, S, 64, MF16><<<grid, NT, 0, s>>>(p, pl.tiles_m, pl.tiles_n, p.K);
      mark_gemm(s, "gemm_tile", BM, BN, S, EPI_ARGMAX, p);
      return hipGetLastError();
    }
    return hipErrorInvalidValue;
  }
  if (epi == EPI_BF16)
    gemm_kernel<BM, BN, WGM, WGN, EPI_BF16, false, GM, S, 64, MF16><<<grid, NT, 0, s>>>(p, pl.tiles_m, pl.tiles_n, p.K);
  else
    gemm_kernel<BM, BN, WGM, WGN, EPI_F32, false, GM, S, 64, MF16><<<grid, NT, 0, s>>>(p, pl.tiles_m, pl.tiles_n, p.K);
  mark_gemm(s, "gemm_tile", BM, BN, S, epi, p);
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

// ---- last-round tail ---------------------------------------------------------
// When a plan's tiles fill whole rounds of resident workgroups plus at most
// half a round more, that last round would leave most CUs idle.  The
// columns of the whole rounds then run as one launch and the remaining
// columns as a problem of their own, with a plan chosen for that shape
// (smaller tiles, or split K).
struct Schedule {
  Plan main;
  int64_t c_split;   // first output column of the tail (0: no tail)
  Plan tail;
};

// eight or more rounds of 256 x 256 tiles with a bf16 output: one persistent
// workgroup per CU (measured: faster from about that many rounds on, when the
// per-tile fill and relaunch it saves are a visible part of a tile's time)
bool persistent_plan(const Plan& pl, int epi, bool gathered) {
  return pl.v == V256x256 && pl.splits == 1 && epi == EPI_BF16 && !gathered &&
         (int64_t)pl.tiles_m * pl.tiles_n >= 8 * kCUs;
}

Schedule make_schedule(int64_t M, int64_t N, int64_t K, int epi, bool allow_split, bool gathered) {
  double best_cost = 0;
  Schedule best{make_plan(M, N, K, epi, allow_split, false, &best_cost, gathered), 0, Plan{}};
  if (!(epi == EPI_BF16 || epi == EPI_SILU_BF16 || epi == EPI_QKV || epi == EPI_ARGMAX)) return best;
  // a row gather reads A the same way in every column slice; the schedule of
  // a gathered problem is the plain one for the argmax epilogue (whose
  // candidate count the host sizes from the plain schedule) and has no tail
  // otherwise
  if (gathered && epi != EPI_ARGMAX) return best;
  // the persistent kernel spreads a ragged last round over its walk; on the
  // lm_head shapes it measured faster than every tail schedule, which the
  // per-tile cost model does not see
  if (persistent_plan(best.main, epi, false)) return best;
  const int64_t ncols = epi == EPI_SILU_BF16 ? N / 2 : N;
  // each unsplit variant whose tiles leave a last round at most half full:
  // its whole rounds, then the tail with the best plan for its own shape
  for (int vi = 0; vi < V_COUNT; ++vi) {
    const Variant& v = kVariants[vi];
    if (epi == EPI_SILU_BF16 && !v.silu) continue;
    if (wide_tile(v.bn) || v.bn == 192) continue;   // single-plan tiles: nothing to split off
    if (epi == EPI_QKV && !qkv_tile_ok(v.bm, v.bn, v.stages)) continue;
    int64_t tm, tn;
    plan_cost(v, M, N, K, epi, 1, &tm, &tn);
    const int64_t R = (int64_t)kCUs * v.resident, T = tm * tn;
    if (vi == V256x256 && epi == EPI_BF16 && T >= 8 * kCUs) continue;   // the persistent kernel's case
    const int64_t full = T / R * R;
    if (full == 0 || full == T || full % tm || (T - full) * 2 > R) continue;
    const int64_t bn_out = epi == EPI_SILU_BF16 ? v.bn / 2 : v.bn;
    const int64_t c_split = full / tm * bn_out;
    if (c_split >= ncols) continue;
    const int64_t n1 = epi == EPI_SILU_BF16 ? 2 * c_split : c_split;
    const int64_t n2 = epi == EPI_SILU_BF16 ? 2 * (ncols - c_split) : ncols - c_split;
    int64_t tm1, tn1;
    const double c1 = plan_cost(v, M, n1, K, epi, 1, &tm1, &tn1);
    double c2 = 0;
    // a SiLU tail has its gate and up rows apart: it never splits K
    const Plan tail = make_plan(M, n2, K, epi, allow_split && epi != EPI_SILU_BF16, false, &c2);
    if (c1 + c2 < best_cost * 0.999) {
      best_cost = c1 + c2;
      best = Schedule{Plan{vi, 1, K, (int)tm1, (int)tn1}, c_split, tail};
    }
  }
  return best;
}

// output columns [c0, c1) of p as a problem of its own
GemmProblem col_slice(const GemmProblem& p, int epi, int64_t c0, int64_t c1) {
  GemmProblem q = p;
  q.B = p.B + c0 * p.ldb;
  if (epi == EPI_SILU_BF16) {
    q.up_off = p.up_off ? p.up_off : p.li;
    q.li = c1 - c0;
    q.N = 2 * (c1 - c0);
    q.C = static_cast<bf16*>(p.C) + c0;
  } else if (epi == EPI_QKV) {
    q.N = c1 - c0;
    q.qkv.head0 = p.qkv.head0 + (int)(c0 / 128);
  } else if (epi == EPI_ARGMAX) {
    q.N = c1 - c0;       // the caller moves C to the slice's first candidate
    q.col0 = p.col0 + c0;
  } else {
    q.N = c1 - c0;
    q.C = static_cast<bf16*>(p.C) + c0;
  }
  return q;
}

size_t split_bytes(const Plan& pl, int64_t M, int64_t N) {
  return pl.splits > 1 ? (size_t)pl.splits * M * N * sizeof(float) : 0;
}

}  // namespace

size_t gemm_scratch_bytes(int64_t M, int64_t N, int64_t K, int epi) {
  if (M <= 0 || N <= 0 || epi == EPI_ARGMAX) return 0;
  const Schedule sc = make_schedule(M, N, K, epi, true, false);
  size_t b = split_bytes(sc.main, M, N);
  if (sc.c_split) {
    const int64_t ncols = epi == EPI_SILU_BF16 ? N / 2 : N;
    const int64_t n2 = epi == EPI_SILU_BF16 ? 2 * (ncols - sc.c_split) : ncols - sc.c_split;
    b = std::max(b, split_bytes(sc.tail, M, n2));
  }
  // the QKV projection may also run with its partials summed by the decode
  // attention, which can prefer more splits
  if (epi == EPI_QKV) b = std::max(b, split_bytes(make_plan(M, N, K, epi, true, true), M, N));
  return b;
}

int64_t gemm_argmax_tiles_n(int64_t M, int64_t N, int64_t K) {
  if (M <= 0 || N <= 0) return 0;
  const Schedule sc = make_schedule(M, N, K, EPI_ARGMAX, false, false);
  return sc.main.tiles_n + (sc.c_split ? sc.tail.tiles_n : 0);
}

namespace {

// Problems of at most this many rows (decode batches: the weight stream)
// run the small tiles in the 16x16x32 form.
constexpr int64_t kMf16Rows = kMf16RowsPlan;
template <int BM, int BN, int WGM, int WGN, int S>
hipError_t launch_rows(const GemmProblem& p, int epi, const Plan& pl, void* scratch, hipStream_t s, bool finish) {
  if (p.M <= kMf16Rows) return launch_tile<BM, BN, WGM, WGN, S, true>(p, epi, pl, scratch, s, finish);
  return launch_tile<BM, BN, WGM, WGN, S, false>(p, epi, pl, scratch, s, finish);
}

hipError_t launch_plan(const GemmProblem& p, int epi, const Plan& pl, void* scratch, hipStream_t s,
                       bool finish = true) {
  switch (pl.v) {
    case V256x256: return launch_tile<256, 256, 4, 2, 2>(p, epi, pl, scratch, s, finish);
    case V256x128: return launch_tile<256, 128, 4, 2, 3>(p, epi, pl, scratch, s, finish);
    case V128x128_4: return launch_rows<128, 128, 4, 2, 4>(p, epi, pl, scratch, s, finish);
    case V128x128_2: return launch_rows<128, 128, 4, 2, 2>(p, epi, pl, scratch, s, finish);
    case V128x64_3: return launch_rows<128, 64, 4, 1, 3>(p, epi, pl, scratch, s, finish);
    case V128x64_6: return launch_rows<128, 64, 4, 1, 6>(p, epi, pl, scratch, s, finish);
    case V64x128_3: return launch_rows<64, 128, 2, 2, 3>(p, epi, pl, scratch, s, finish);
    case V256x320: return launch_tile<256, 320, 4, 2, 2>(p, epi, pl, scratch, s, finish);
    case V128x192: return launch_tile<128, 192, 4, 2, 4>(p, epi, pl, scratch, s, finish);
    default: return launch_rows<64, 64, 2, 2, 8>(p, epi, pl, scratch, s, finish);
  }
}

}  // namespace

hipError_t gemm_bf16(const GemmProblem& p, int epi, void* scratch, size_t scratch_bytes, hipStream_t s) {
  if (p.M <= 0 || p.N <= 0) return hipSuccess;
  const bool can_split = epi != EPI_ARGMAX && !p.a_rows && scratch != nullptr &&
                         scratch_bytes >= gemm_scratch_bytes(p.M, p.N, p.K, epi);
  const Schedule sc = make_schedule(p.M, p.N, p.K, epi, can_split, p.a_rows != nullptr);
  const Plan& pl = sc.main;
  if (persistent_plan(pl, epi, p.a_rows != nullptr)) {
    gemm_persist_kernel<256, 256, 4, 2, EPI_BF16, 8, 2><<<kCUs, 512, 0, s>>>(p, pl.tiles_m, pl.tiles_n);
    mark_gemm(s, "gemm_persist", 256, 256, 2, EPI_BF16, p);
    return hipGetLastError();
  }
  if (!sc.c_split) return launch_plan(p, epi, pl, scratch, s);
  const int64_t ncols = epi == EPI_SILU_BF16 ? p.li : p.N;
  const hipError_t e = launch_plan(col_slice(p, epi, 0, sc.c_split), epi, pl, scratch, s);
  if (e != hipSuccess) return e;
  GemmProblem tail = col_slice(p, epi, sc.c_split, ncols);
  // argmax: the tail's candidates follow the main launch's N tiles in each
  // row (ldc counts both)
  if (epi == EPI_ARGMAX) tail.C = static_cast<uint64_t*>(p.C) + pl.tiles_n;
  return launch_plan(tail, epi, sc.tail, scratch, s);
}

hipError_t gemm_qkv(const GemmProblem& p, void* scratch, size_t scratch_bytes, bool defer, int* splits_out,
                    hipStream_t s) {
  *splits_out = 0;
  if (p.M <= 0 || p.N <= 0) return hipSuccess;
  if (!defer) return gemm_bf16(p, EPI_QKV, scratch, scratch_bytes, s);
  Plan pl = make_plan(p.M, p.N, p.K, EPI_QKV, scratch != nullptr, true);
  if (pl.splits > 1 && scratch_bytes < (size_t)pl.splits * p.M * p.N * sizeof(float))
    pl = make_plan(p.M, p.N, p.K, EPI_QKV, false, true);   // no room for the partials
  const bool split = pl.splits > 1;
  if (split) *splits_out = pl.splits;
  // unsplit: the tile finishes its heads in the epilogue as usual
  switch (pl.v) {
    case V256x256: return launch_tile<256, 256, 4, 2, 2>(p, EPI_QKV, pl, scratch, s, !split);
    case V256x128: return launch_tile<256, 128, 4, 2, 3>(p, EPI_QKV, pl, scratch, s, !split);
    case V128x128_4: return launch_rows<128, 128, 4, 2, 4>(p, EPI_QKV, pl, scratch, s, !split);
    case V128x128_2: return launch_rows<128, 128, 4, 2, 2>(p, EPI_QKV, pl, scratch, s, !split);
    case V128x64_3: return launch_rows<128, 64, 4, 1, 3>(p, EPI_QKV, pl, scratch, s, !split);
    case V128x64_6: return launch_rows<128, 64, 4, 1, 6>(p, EPI_QKV, pl, scratch, s, !split);
    case V64x128_3: return launch_rows<64, 128, 2, 2, 3>(p, EPI_QKV, pl, scratch, s, !split);
    case V256x320:   // never planned for QKV
    case V128x192: return hipErrorInvalidValue;
    default: return launch_rows<64, 64, 2, 2, 8>(p, EPI_QKV, pl, scratch, s, !split);
  }
}

hipError_t gemm_f32(const float* A, const float* B, float* C, int64_t M, int64_t N, int64_t K, int silu_li,
                    hipStream_t s) {
  const int64_t cols = silu_li > 0 ? silu_li : N;
  if (M <= 0 || cols <= 0) return hipSuccess;
  int64_t g = (M * cols + 255) / 256;
  if (g > 8192) g = 8192;
  gemm_f32_kernel<<<(int)g, 256, 0, s>>>(A, B, C, M, N, K, silu_li);
  kmark(s, silu_li > 0 ? "gemm_f32/silu" : "gemm_f32");
  return hipGetLastError();
}

}  // namespace tps
