// Attention over the rank's local heads, prefill and decode ("Tensor
// parallelism from scratch", "Implementation", TPAttention.forward; "Two ways
// to split": heads are independent, so a rank attends with its own q heads
// over its own kv-cache heads; q head i reads kv head i / rep):
//
//   out[t, h, :] = sum_s softmax_s(q[t,h] . k[h/rep, s] / sqrt(128)) v[h/rep, s]
//   over the keys s = 0 .. past + t (query t sits at position past + t).
//
// Flash attention on MFMA (v_mfma_f32_32x32x16_bf16).  A workgroup owns 32
// query rows that share one kv head:
//  * prefill: 32 consecutive tokens of one q head;
//  * decode (T = 1): the rep q heads of one (sequence, kv head), one row
//    each (rows past rep are padding and never stored).
// Its four waves split the block's key range into four contiguous parts.
// Each wave streams its part through a private ring of two LDS stages
// (32-key K and V tiles, direct global->LDS buffer loads, 16-byte chunks of
// a key row XOR-swizzled by a rotation of the key so that operand reads avoid bank
// conflicts) and keeps an online softmax in the exp2 domain:
//  * S^T[32 keys, 32 q] = K . Q^T with Q^T in VGPRs: each lane column is one
//    query row, so its max and sum are lane-local plus one exchange with the
//    other half-wave;
//  * O^T[128 d, 32 q] += V^T . P^T, V^T read with the transposing LDS load
//    ds_read_b64_tr_b16.
// The four partial (max, sum, O) are merged through LDS at the end, so a
// block needs no second pass; prefill blocks run heaviest (latest) first.
// Prefill, where the block's matrix and vector work is the larger cost,
// pipelines the tiles: a stage holds K of tile j and V of tile j - 1, so the
// MFMAs of S for tile i + 1 are in flight while the VALU runs the softmax
// of tile i.  Decode, bound by the stream of K and V, keeps K and V of one
// tile per stage (one more tile of loads in flight).
#include <type_traits>

#include "common.h"
#include "qkv_finish.h"

namespace tps {

namespace {

typedef __bf16 lds_bf16x4 __attribute__((__vector_size__(4 * sizeof(__bf16))));
typedef int i32x4 __attribute__((ext_vector_type(4)));

constexpr int kKeys = 32;                    // keys per tile
constexpr int kTileB = kKeys * 256;          // bytes of one K or V tile
constexpr int kStageB = 2 * kTileB;          // K tile, then V tile
constexpr int kLoads = kTileB / 1024;        // 1 KB direct-to-LDS loads per tile (K or V)
constexpr int kMergeStride = 129;            // floats per merged row (odd: no bank conflicts)
constexpr float kQScale = 0.08838834764831845f * 1.4426950408889634f;   // log2(e) / sqrt(128)
constexpr float kSlack = 8.f;                 // lazy-rescale margin, log2 units

__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }
// byte offset of 16-byte chunk c (d = 8c .. 8c+7) of key row `key` in a tile
// Key row swizzle: a rotation of the key's low four bits.  The transposing
// V reads take 4 consecutive keys x 4 chunks per 32 lanes and the K reads 16
// consecutive keys x 1 chunk; both land on distinct banks (plain key & 15
// maps keys k and k ^ 1 onto the same pair of chunks: 2-way conflicts).
__device__ __forceinline__ int kswz(int key) { return ((key << 2) | ((key >> 2) & 3)) & 15; }
__device__ __forceinline__ uint32_t toff(int key, int c) { return (uint32_t)(key * 256 + ((c ^ kswz(key)) << 4)); }
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}
// raw buffer descriptor: base, stride 0, num_records bytes (reads at or past
// the end return zero)
__device__ __forceinline__ i32x4 buffer_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)base;
  return i32x4{__builtin_amdgcn_readfirstlane((int)(uint32_t)a), __builtin_amdgcn_readfirstlane((int)((a >> 32) & 0xFFFF)),
               __builtin_amdgcn_readfirstlane((int)bytes), 0x00020000};
}
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const unsigned char*)p;
}
// buffer_load_dwordx4 ... lds: lane l's 16 bytes land at LDS byte lds + 16 l.
// Issued from asm so that the compiler, which would otherwise order every
// later LDS read behind all outstanding loads (vmcnt(0)), leaves the
// ordering to the explicit waits of the ring; M0 is set right here and
// nothing else in this kernel reads it.
__device__ __forceinline__ void dma16(const i32x4& rsrc, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff), "s"(rsrc),
               "s"(__builtin_amdgcn_readfirstlane(lds))
               : "memory");
}

// NWV waves per workgroup, NST ring stages per wave (NST - 1 tiles in
// flight while one is computed).
template <int NWV, int NST, bool PIPE>
__global__ __launch_bounds__(NWV * 64) __attribute__((amdgpu_waves_per_eu(1, 1)))
void attn_flash_kernel(AttnArgs a, int n_rb) {
  constexpr int NT = NWV * 64;
  constexpr int kWaveRingB = NST * kStageB;
  static_assert(NWV * kWaveRingB <= 163840, "rings fit the CU's LDS");
  static_assert(NWV * 32 * (kMergeStride + 2) * 4 <= NWV * kWaveRingB, "merge area fits the rings");
  __shared__ __attribute__((aligned(16))) unsigned char smem[NWV * kWaveRingB];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 31, lh = lane >> 5;
  const int rep = a.lq / a.lkv;
  const bool decode = a.T == 1;
  const int64_t ldq = (int64_t)a.lq * 128;

  // the block: sequence b, kv head kvh, first q head head0, first token t0
  int b, kvh, head0, t0;
  if (decode) {
    // Consecutive blocks to one XCD (the dispatcher deals blocks to the 8
    // XCDs in turn), so each XCD streams a contiguous run of sequences.  In
    // plain order XCD x took sequences x, x + 8, ..., whose cache slabs share
    // address bits, and the XCDs' key loops differed by up to 22%; this
    // order measured 3% faster on the 32B decode shapes.
    const int nb = (int)gridDim.x, xcd = (int)blockIdx.x % 8, idx = (int)blockIdx.x / 8;
    const int per = nb / 8, rem = nb % 8;
    const int blk = (xcd < rem ? xcd * (per + 1) : rem * (per + 1) + (xcd - rem) * per) + idx;
    b = blk / a.lkv;
    kvh = blk % a.lkv;
    head0 = kvh * rep;
    t0 = 0;
  } else {
    const int per_rb = a.B * a.lq;
    const int rb = n_rb - 1 - (int)(blockIdx.x / per_rb);
    const int rest = (int)(blockIdx.x % per_rb);
    b = rest / a.lq;
    head0 = rest % a.lq;
    kvh = head0 / rep;
    t0 = rb * 32;
  }
  const bool row_ok = decode ? lr < rep : t0 + lr < a.T;
  const int qpos = a.past + (decode ? 0 : t0 + lr);       // this lane column's query position
  const int min_pos = a.past + t0;                        // the block's first query position
  const int n_keys = decode ? a.past + 1 : a.past + min(a.T, t0 + 32);
  const int nt = (n_keys + kKeys - 1) / kKeys;
  const int w0 = wave * nt / NWV, w1 = (wave + 1) * nt / NWV;   // this wave's tiles

  // K/V tile loads: load i (0..7) of a tile holds keys 4i .. 4i+3; lane l
  // writes physical chunk l % 16 of key 4i + l / 16.  Keys at or past
  // past + T read as zero (descriptor bound) and are masked.
  const int64_t slab = ((int64_t)b * a.lkv + kvh) * a.S_max * 128;
  const uint32_t valid_bytes = (uint32_t)(a.past + a.T) * 256u;
  const i32x4 rk = buffer_rsrc(a.k_cache + slab, valid_bytes);
  const i32x4 rv = buffer_rsrc(a.v_cache + slab, valid_bytes);
  unsigned char* ring = smem + wave * kWaveRingB;
  // a stage: K of tile kt and V of tile kt (PIPE: of tile kt - 1).  A tile
  // outside the wave's range may be loaded and is never read; below key 0
  // the offset wraps past the descriptor bound and reads zero.
  auto dma_tile = [&](int kt, int st) {
    const uint32_t base = lds_addr(ring + st * kStageB);
    const int vt = PIPE ? kt - 1 : kt;
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int key = 4 * i + (lane >> 4);
      const uint32_t sw = (uint32_t)(((lane & 15) ^ kswz(key)) << 4);
      dma16(rk, (uint32_t)(kt * kKeys + key) * 256u + sw, base + i * 1024);
      dma16(rv, (uint32_t)(vt * kKeys + key) * 256u + sw, base + kTileB + i * 1024);
    }
  };

  // Decode issues each wave's first K/V tile before Q is ready, so that its
  // load latency overlaps the Q prologue.  With the projection deferred, the
  // tile that holds position past is written by the prologue below: a wave
  // whose first tile is that one waits for it instead.
  const bool early = decode && w1 > w0 && (a.qkv_splits == 0 || w0 < nt - 1);
  if (early) dma_tile(w0, 0);

  // Q^T operands: lane supplies q[row lr, ks*16 + lh*8 .. +8]
  bf16x8 qf[8];
  if (decode && a.qkv_splits > 0) {
    // The projection arrives as split-K partials: sum them (split order) for
    // this block's rep q heads and its kv head, apply QK-norm and RoPE at
    // position past, append k and v to the caches there, and keep q on chip
    // (staged in LDS, which the rings reuse afterwards).
    const int n_qkv = (a.lq + 2 * a.lkv) * 128;
    const int64_t plane = (int64_t)a.B * n_qkv;
    const float* prow = a.qkv_part + (int64_t)b * n_qkv;
    // [rep][128] in wave 0's second ring stage (the first may hold an early tile)
    bf16* qs = reinterpret_cast<bf16*>(smem + kStageB);
    const int j16 = tid & 15;
    const RopeCoef rc = rope_coef(a.theta, j16);
    for (int u = tid >> 4; u < rep + 2; u += NT / 16) {   // a unit: 16 lanes, one head row
      const int col = u < rep ? (head0 + u) * 128 : (u == rep ? a.lq + kvh : a.lq + a.lkv + kvh) * 128;
      f32x4 v0 = {0.f, 0.f, 0.f, 0.f}, v1 = {0.f, 0.f, 0.f, 0.f};
      for (int z = 0; z < a.qkv_splits; ++z) {
        const float* src = prow + z * plane + col + 4 * j16;
        const f32x4 p0 = *reinterpret_cast<const f32x4*>(src), p1 = *reinterpret_cast<const f32x4*>(src + 64);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          v0[e] += p0[e];
          v1[e] += p1[e];
        }
      }
      float x[8] = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
      if (u <= rep) qk_norm_rope(x, u < rep ? a.q_norm_w : a.k_norm_w, a.past, j16, rc, a.eps);
      if (u < rep) {
        store_head_lanes(qs + u * 128, x, j16);
        if (a.q_store) store_head_lanes(a.q_store + (int64_t)b * ldq + (int64_t)(head0 + u) * 128, x, j16);
      } else {
        bf16* cache = const_cast<bf16*>(u == rep ? a.k_cache : a.v_cache);
        store_head_lanes(cache + (((int64_t)b * a.lkv + kvh) * a.S_max + a.past) * 128, x, j16);
      }
    }
    // the cache rows are complete in L2 before any wave loads its tiles
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
      qf[ks] = row_ok ? *reinterpret_cast<const bf16x8*>(qs + lr * 128 + ks * 16 + lh * 8) : bf16x8{};
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): the staging is read before the rings refill it
    __syncthreads();
  } else {
    const bf16* qp = decode ? a.q + (int64_t)b * ldq + (int64_t)(head0 + (row_ok ? lr : 0)) * 128
                            : a.q + ((int64_t)b * a.T + (row_ok ? t0 + lr : 0)) * ldq + (int64_t)head0 * 128;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const u32x4 v = row_ok ? *reinterpret_cast<const u32x4*>(qp + ks * 16 + lh * 8) : u32x4{0u, 0u, 0u, 0u};
      qf[ks] = __builtin_bit_cast(bf16x8, v);
    }
    // land Q before the ring starts: a first use inside the loop would make
    // the compiler wait for every load in flight there
    wait_vm<0>();
  }

  f32x16 o[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[db][e] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  // transposing-read source address of this lane for V^T rows db*32 ..,
  // keys kbase .. kbase+3 of its half-wave (lanes 16g .. 16g+15, g = lane/16)
  const int trg = lane >> 4, tri = lane & 15;
  const int tr_key = 4 * (trg >> 1) + (tri >> 2);          // + sub*16 + rd*8
  const int tr_d = (trg & 1) * 16 + 4 * (tri & 3);         // + db*32
  // S^T of the K tile in stage st
  auto s_tile = [&](int st) -> f32x16 {
    const unsigned char* K = ring + st * kStageB;
    f32x16 s;
#pragma unroll
    for (int e = 0; e < 16; ++e) s[e] = 0.f;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const bf16x8 kf = *reinterpret_cast<const bf16x8*>(K + toff(lr, ks * 2 + lh));
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ks], s, 0, 0, 0);
    }
    return s;
  };
  // online softmax of tile kt's scores s, then O^T += V^T P^T with the V
  // tile in stage st
  // (s is the caller's tile, masked in place: it is dead afterwards)
  auto soft_pv = [&](f32x16& s, int kt, int st) {
    const unsigned char* V = ring + st * kStageB + kTileB;
    const int key0 = kt * kKeys;
    // V^T operands do not depend on P: their transposing reads go out first
    // and land while the VALU does the softmax
    bf16x8 vf[4][2];
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int sub = 0; sub < 2; ++sub) {
        const int key = sub * 16 + tr_key;
        const int d = db * 32 + tr_d;
        const uint32_t a0 = toff(key, d >> 3) + ((d >> 2) & 1) * 8;
        const uint32_t a1 = toff(key + 8, d >> 3) + ((d >> 2) & 1) * 8;
        const lds_bf16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((__attribute__((address_space(3))) lds_bf16x4*)(V + a0));
        const lds_bf16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((__attribute__((address_space(3))) lds_bf16x4*)(V + a1));
        vf[db][sub] = bf16x8{v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
      }
    __builtin_amdgcn_sched_barrier(0);
    // raw max over this tile's visible scores (the scale is positive)
    float mx = -INFINITY;
    if (key0 + kKeys - 1 > min_pos) {                      // some key may follow some row
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        if (key0 + 8 * (e >> 2) + 4 * lh + (e & 3) > qpos) s[e] = -INFINITY;
        mx = fmaxf(mx, s[e]);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[e]);
    }
    mx = pair_max(mx) * kQScale;
    // Lazy rescale: the exponent base m_run only moves when some row's max
    // passes it by more than kSlack, so P stays below 2^kSlack and O and l,
    // which share the base, stay exact; most tiles skip the O update.
    if (__any(mx > m_run + kSlack)) {
      const float mn = fmaxf(m_run, mx);
      const float corr = m_run == -INFINITY ? 0.f : ex2(m_run - mn);
      m_run = mn;
      l_run *= corr;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[db][e] *= corr;
    }
    const float base = m_run == -INFINITY ? 0.f : m_run;
    bf16x8 pf[2];
    float ps[4] = {0.f, 0.f, 0.f, 0.f};    // four short chains instead of one of 16
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const float pv = ex2(__builtin_fmaf(s[e], kQScale, -base));   // masked: 2^-inf = 0
      ps[e & 3] += pv;
      pf[e >> 3][e & 7] = f2bf(pv);
    }
    l_run += (ps[0] + ps[1]) + (ps[2] + ps[3]);
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int sub = 0; sub < 2; ++sub) o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[db][sub], pf[sub], o[db], 0, 0, 0);
  };

  const int n = w1 - w0;
  if constexpr (!PIPE) {
    // tile w0 + i lives in stage i % NST; tiles up to i + NST - 1 are in
    // flight while tile i is computed.  The stage a load refills was read
    // by the previous tile: lgkmcnt(0) first.
    for (int j = early ? 1 : 0; j < NST - 1 && j < n; ++j) dma_tile(w0 + j, j);
    for (int i = 0; i < n; ++i) {
      if (i + NST - 1 < n) {
        __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
        dma_tile(w0 + i + NST - 1, (i + NST - 1) % NST);
        wait_vm<(NST - 1) * 2 * kLoads>();
      } else {
        wait_vm<0>();
      }
      f32x16 sc = s_tile(i % NST);
      soft_pv(sc, w0 + i, i % NST);
    }
  } else if (n > 0) {
    // stage j = {K of tile w0 + j, V of tile w0 + j - 1}, j = 0 .. n, in
    // buffer j % 2.  Iteration i reads stage i + 1 (K for S of tile i + 1,
    // V for tile i), then refills its buffer with stage i + 3.
    static_assert(NST == 2, "the pipelined loop uses two stages");
    constexpr int SL = 2 * kLoads;         // loads per stage
    dma_tile(w0, 0);
    dma_tile(w0 + 1, 1);
    wait_vm<SL>();
    f32x16 s_a = s_tile(0), s_b = s_a;
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): stage 0 read
    if (2 <= n) dma_tile(w0 + 2, 0);
    // iteration i: S of tile i is in `cur`, S of tile i + 1 goes to `nxt`;
    // unrolled by two so that the stage (i + 1) % 2 is a constant (LDS
    // offsets fold into the instructions) and S alternates between s_a and
    // s_b without copies
    auto step = [&](int i, auto st_tag, f32x16& cur, f32x16& nxt) __attribute__((always_inline)) {
      constexpr int st = decltype(st_tag)::value;
      if (i + 2 <= n)
        wait_vm<SL>();
      else
        wait_vm<0>();
      nxt = s_tile(st);   // on the last tile: a settled stage, result unused
      soft_pv(cur, w0 + i, st);
      if (i + 3 <= n) {
        __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): stage i + 1 read
        dma_tile(w0 + i + 3, st);
      }
    };
    for (int i = 0; i < n; i += 2) {
      step(i, std::integral_constant<int, 1>{}, s_a, s_b);
      if (i + 1 < n) step(i + 1, std::integral_constant<int, 0>{}, s_b, s_a);
    }
  }

  // merge the four waves' partials through LDS (the area overlaps the rings)
  __syncthreads();
  float* mo = reinterpret_cast<float*>(smem);                       // [wave][q][kMergeStride]
  float* mml = mo + NWV * 32 * kMergeStride;                         // [wave][q][2]
  {
    float* row = mo + (wave * 32 + lr) * kMergeStride;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int e = 0; e < 16; ++e) row[db * 32 + 8 * (e >> 2) + 4 * lh + (e & 3)] = o[db][e];
    const float l = pair_sum(l_run);
    if (lh == 0) {
      mml[(wave * 32 + lr) * 2] = m_run;
      mml[(wave * 32 + lr) * 2 + 1] = l;
    }
  }
  __syncthreads();
  {
    constexpr int TPR = NT / 32, DPT = 128 / TPR;           // threads per row, d per thread
    const int q = tid / TPR, dc = (tid % TPR) * DPT;
    const bool ok = decode ? q < rep : t0 + q < a.T;
    if (!ok) return;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NWV; ++w) M = fmaxf(M, mml[(w * 32 + q) * 2]);
    float wt[NWV], L = 0.f;
#pragma unroll
    for (int w = 0; w < NWV; ++w) {
      const float mw = mml[(w * 32 + q) * 2];
      wt[w] = mw == -INFINITY ? 0.f : ex2(mw - M);
      L += wt[w] * mml[(w * 32 + q) * 2 + 1];
    }
    const float inv = L > 0.f ? 1.f / L : 0.f;
    bf16* dst = decode ? a.out + (int64_t)b * ldq + (int64_t)(head0 + q) * 128 + dc
                       : a.out + ((int64_t)b * a.T + t0 + q) * ldq + (int64_t)head0 * 128 + dc;
#pragma unroll
    for (int c = 0; c < DPT / 8; ++c) {
      bf16x8 ob;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        float acc = 0.f;
#pragma unroll
        for (int w = 0; w < NWV; ++w) acc += wt[w] * mo[(w * 32 + q) * kMergeStride + dc + 8 * c + j];
        ob[j] = f2bf(acc * inv);
      }
      *reinterpret_cast<bf16x8*>(dst + 8 * c) = ob;
    }
  }
}

}  // namespace

hipError_t attn_flash(const AttnArgs& a, hipStream_t s) {
  if (a.B <= 0 || a.T <= 0) return hipSuccess;
  const int rep = a.lq / a.lkv;
  if (a.lkv <= 0 || a.lq % a.lkv != 0 || rep > 32) return hipErrorInvalidValue;
  const int n_rb = (a.T + 31) / 32;
  const int64_t blocks = a.T == 1 ? (int64_t)a.B * a.lkv : (int64_t)a.B * a.lq * n_rb;
  if (a.T == 1)
    attn_flash_kernel<4, 2, false><<<(unsigned)blocks, 256, 0, s>>>(a, n_rb);
  else
    attn_flash_kernel<4, 2, true><<<(unsigned)blocks, 256, 0, s>>>(a, n_rb);
  kmark(s, a.T == 1 ? "attn_flash/decode" : "attn_flash/prefill");
  return hipGetLastError();
}

}  // namespace tps
