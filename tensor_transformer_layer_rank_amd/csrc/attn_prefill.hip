// Prefill attention over the rank's local heads ("Tensor parallelism from
// scratch", "Implementation", TPAttention.forward): causal GQA attention of
// T new tokens after `past` cached ones; query t (position past + t) sees
// keys 0 .. past + t, q head i reads kv head i / rep, scale 1/sqrt(128).
//
// Flash attention on MFMA (v_mfma_f32_32x32x16_bf16).  A workgroup is eight
// waves, two per SIMD, working on one kv head:
//  * each wave owns 32 query rows of HW q heads of that kv head (HW = 1: with
//    two waves per SIMD the registers allow one head, and the other wave's
//    MFMAs run while a wave does its softmax on the VALU);
//  * K and V tiles of 64 keys go from HBM straight into LDS (buffer loads
//    with the lds flag) through a ring of NS stages; 16-byte chunks of a key
//    row are XOR-swizzled by a rotation of the key so that operand reads avoid bank
//    conflicts;
//  * S^T[64 keys, 32 q] = K . Q^T with Q^T held in VGPRs: each lane column
//    is one query, so its row max and sum are lane-local plus one exchange
//    with the other half-wave;
//  * O^T[128 d, 32 q] += V^T . P^T, V^T read with the transposing LDS load
//    ds_read_b64_tr_b16: in each 16-lane group, source lane s reads 4 d of
//    key base + s/4 and lane i receives d = dbase + i of keys base .. base+3;
//  * the softmax runs in the exp2 domain with a running max per query.
// Early query blocks need few keys; heavy (late) blocks are launched first.
// This kernel serves prefills whose blocks alone fill the GPU; smaller ones
// (and GQA ratios it has no wave shape for) go to the one-pass kernel of
// attn_flash.hip, which splits each block's keys among its waves instead.
#include <type_traits>

#include "common.h"

namespace tps {

namespace {

typedef __bf16 lds_bf16x4 __attribute__((__vector_size__(4 * sizeof(__bf16))));

constexpr int kKeys = 64;                    // keys per tile
constexpr int kTile = kKeys * 256;           // bytes of one K or V tile (64 rows x 128 bf16)
constexpr int kStage = 2 * kTile;            // K tile, then V tile
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
// Workgroup barrier without the release fence of __syncthreads(), which
// would wait for every outstanding direct-to-LDS load; each wave waits for
// its own loads of the next tile (vmcnt) before arriving.
__device__ __forceinline__ void barrier() { asm volatile("s_barrier" ::: "memory"); }

typedef int i32x4 __attribute__((ext_vector_type(4)));
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
// later LDS read of the ring behind all outstanding loads (vmcnt(0)), leaves
// the ordering to the explicit waits of the ring; M0 is set right here and
// nothing else in these kernels reads it.
__device__ __forceinline__ void dma16(const i32x4& rsrc, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff), "s"(rsrc),
               "s"(__builtin_amdgcn_readfirstlane(lds))
               : "memory");
}

struct PrefillPlan {
  int rows;       // query rows per workgroup (32 per wave row block)
  int n_rb;       // query row blocks
  int hgroups;    // workgroups per kv head along the q heads
};

__host__ __device__ inline int rb_tiles(int T, int past, int rows, int r) {
  const int end = (r + 1) * rows < T ? (r + 1) * rows : T;
  return (past + end + kKeys - 1) / kKeys;
}
// NWV waves (NWV / 4 per SIMD), HG of them along the heads; NS ring stages
template <int HW, int HG, int NS, int NWV>
__global__ __launch_bounds__(NWV * 64) __attribute__((amdgpu_waves_per_eu(NWV / 4, NWV / 4)))
void attn_prefill_kernel(AttnArgs a, PrefillPlan p) {
  static_assert(NWV % HG == 0 && (kStage / 1024) % (2 * NWV) == 0, "waves split the rows and the tile loads");
  constexpr int kLoadsPerWave = kStage / 1024 / NWV;
  constexpr int RB = NWV / HG;         // 32-row blocks per workgroup
  constexpr int WGH = HW * HG;         // q heads per workgroup
  // one array per ring stage: reads of one stage then carry alias scopes
  // that tell them apart from direct-to-LDS loads still landing in another,
  // so the compiler adds no wait for those loads before them
  __shared__ __attribute__((aligned(16))) unsigned char smem0[kStage];
  __shared__ __attribute__((aligned(16))) unsigned char smem1[kStage];
  __shared__ __attribute__((aligned(16))) unsigned char smem2[NS > 2 ? kStage : 16];
  static_assert(NS == 2 || NS == 3, "ring of two or three stages");
  auto stage = [&](auto st) -> unsigned char* {
    constexpr int v = decltype(st)::value;
    return v == 0 ? smem0 : (v == 1 ? smem1 : smem2);
  };

  const int groups = a.B * a.lkv * p.hgroups;
  const int w = blockIdx.x / groups, grp = blockIdx.x % groups;
  const int hgrp = grp % p.hgroups;
  const int kvh = (grp / p.hgroups) % a.lkv;
  const int b = grp / (p.hgroups * a.lkv);
  const int r = p.n_rb - 1 - w;                           // heaviest blocks first
  const int kt0 = 0, kt1 = rb_tiles(a.T, a.past, p.rows, r);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 31, lh = lane >> 5;
  const int hg = wave / RB, rr = wave % RB;
  const int rep = a.lq / a.lkv;
  const int head0 = kvh * rep + hgrp * WGH + hg * HW;
  const int t0w = r * p.rows + rr * 32;                  // first query row of this wave
  const bool active = t0w < a.T;
  const int nt_w = active ? (a.past + min(a.T, t0w + 32) + kKeys - 1) / kKeys : 0;
  const int qpos = a.past + t0w + lr;                    // this lane's query position
  const int64_t ldq = (int64_t)a.lq * 128;

  // Q^T operands: lane supplies q[t0w + lr, head, ks*16 + lh*8 .. +8]
  bf16x8 qf[HW][8];
  {
    const int tq = t0w + lr;
    const bool ok = tq < a.T;
#pragma unroll
    for (int hw = 0; hw < HW; ++hw) {
      const bf16* qp = a.q + ((int64_t)b * a.T + (ok ? tq : 0)) * ldq + (int64_t)(head0 + hw) * 128 + lh * 8;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const u32x4 v = ok ? *reinterpret_cast<const u32x4*>(qp + ks * 16) : u32x4{0u, 0u, 0u, 0u};
        qf[hw][ks] = __builtin_bit_cast(bf16x8, v);
      }
    }
    // land Q before the ring starts: a first use inside the loop would make
    // the compiler wait for every load in flight on each iteration
    wait_vm<0>();
  }

  // K/V loads: load i (0..15) of a tile holds keys 4i .. 4i+3; lane l writes
  // physical chunk l % 16 of key 4i + l / 16.  Keys at or past past + T read
  // as zero (descriptor bound) and are masked as lying after every query.
  const int64_t slab = ((int64_t)b * a.lkv + kvh) * a.S_max * 128;
  const uint32_t valid_bytes = (uint32_t)(a.past + a.T) * 256u;
  const i32x4 rk = buffer_rsrc(a.k_cache + slab, valid_bytes);
  const i32x4 rv = buffer_rsrc(a.v_cache + slab, valid_bytes);
  auto dma_tile = [&](int kt, auto st) {
    const uint32_t base = lds_addr(stage(st));
#pragma unroll
    for (int j = 0; j < kLoadsPerWave / 2; ++j) {
      const int i = wave * (kLoadsPerWave / 2) + j;
      const int key = 4 * i + (lane >> 4);
      const uint32_t off = (uint32_t)(kt * kKeys + key) * 256u + (uint32_t)(((lane & 15) ^ kswz(key)) << 4);
      dma16(rk, off, base + i * 1024);
      dma16(rv, off, base + kTile + i * 1024);
    }
  };

  f32x16 o[HW][4];
#pragma unroll
  for (int hw = 0; hw < HW; ++hw)
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int e = 0; e < 16; ++e) o[hw][db][e] = 0.f;
  float m_run[HW], l_run[HW];
#pragma unroll
  for (int hw = 0; hw < HW; ++hw) {
    m_run[hw] = -INFINITY;
    l_run[hw] = 0.f;
  }

  // transposing-read source address of this lane for V^T rows db*32 ..,
  // keys kbase .. kbase+3 of its half-wave (lanes 16g .. 16g+15, g = lane/16)
  const int trg = lane >> 4, tri = lane & 15;
  const int tr_key = 4 * (trg >> 1) + (tri >> 2);          // + kb*32 + sub*16 + rd*8
  const int tr_d = (trg & 1) * 16 + 4 * (tri & 3);         // + db*32
  // The key swizzle depends only on a key's low four bits, so the read
  // offsets of keys 16 apart differ by a constant: the per-lane offsets are
  // computed once (V^T: keys tr_key and tr_key + 8 of each 32-wide d block;
  // K: row lr of each 16-wide k-step) and the tile loop adds immediates.
  uint32_t vbo[4][2], kbo[8];
#pragma unroll
  for (int db = 0; db < 4; ++db) {
    const int d = db * 32 + tr_d;
    vbo[db][0] = toff(tr_key, d >> 3) + ((d >> 2) & 1) * 8;
    vbo[db][1] = toff(tr_key + 8, d >> 3) + ((d >> 2) & 1) * 8;
  }
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) kbo[ks] = toff(lr, ks * 2 + lh);
  auto compute = [&](int kt, auto st) {
    const unsigned char* K = stage(st);
    const unsigned char* V = K + kTile;
    f32x16 s[HW][2];
#pragma unroll
    for (int hw = 0; hw < HW; ++hw)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) s[hw][kb][e] = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(K + kbo[ks] + kb * 8192);
#pragma unroll
        for (int hw = 0; hw < HW; ++hw)
          s[hw][kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[hw][ks], s[hw][kb], 0, 0, 0);
      }
    const int key0 = kt * kKeys;
    const bool diag = key0 + kKeys - 1 > a.past + t0w;     // some key may follow some row
    bf16x8 pf[HW][4];
#pragma unroll
    for (int hw = 0; hw < HW; ++hw) {
      // raw max over this tile's visible scores (the scale is positive)
      float mx = -INFINITY;
      if (diag) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            if (key0 + kb * 32 + 8 * (e >> 2) + 4 * lh + (e & 3) > qpos) s[hw][kb][e] = -INFINITY;
            mx = fmaxf(mx, s[hw][kb][e]);
          }
      } else {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[hw][kb][e]);
      }
      mx = pair_max(mx) * kQScale;
      // Lazy rescale: the exponent base m_run only moves when some row's max
      // passes it by more than kSlack, so P stays below 2^kSlack and O and
      // l, which share the base, stay exact; most tiles skip the O update.
      if (__any(mx > m_run[hw] + kSlack)) {
        const float mn = fmaxf(m_run[hw], mx);
        const float corr = m_run[hw] == -INFINITY ? 0.f : ex2(m_run[hw] - mn);
        m_run[hw] = mn;
        l_run[hw] *= corr;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
          for (int e = 0; e < 16; ++e) o[hw][db][e] *= corr;
      }
      const float base = m_run[hw] == -INFINITY ? 0.f : m_run[hw];
      float ps = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const float pv = ex2(__builtin_fmaf(s[hw][kb][e], kQScale, -base));   // masked: 2^-inf = 0
          ps += pv;
          pf[hw][kb * 2 + (e >> 3)][e & 7] = f2bf(pv);
        }
      l_run[hw] += ps;
    }
    // V^T operands (another wave's work covers their latency)
    bf16x8 vf[4][2][2];
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int sub = 0; sub < 2; ++sub) {
          const uint32_t a0 = vbo[db][0] + (uint32_t)((kb * 32 + sub * 16) * 256);
          const uint32_t a1 = vbo[db][1] + (uint32_t)((kb * 32 + sub * 16) * 256);
          const lds_bf16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((__attribute__((address_space(3))) lds_bf16x4*)(V + a0));
          const lds_bf16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((__attribute__((address_space(3))) lds_bf16x4*)(V + a1));
          vf[db][kb][sub] = bf16x8{v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
        }
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int sub = 0; sub < 2; ++sub)
#pragma unroll
          for (int hw = 0; hw < HW; ++hw)
            o[hw][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[db][kb][sub], pf[hw][kb * 2 + sub], o[hw][db], 0,
                                                                0, 0);
  };

  // ring: tiles kt0 + i live in stage i % NS; NS - 1 tiles in flight.  The
  // loop is unrolled by NS so that every stage index is a constant.
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  using S2 = std::integral_constant<int, (NS > 2 ? 2 : 0)>;
  const int ntiles = kt1 - kt0;
  dma_tile(kt0, S0{});
  if (NS > 2 && ntiles > 1) dma_tile(kt0 + 1, S1{});
  if (NS > 2 && ntiles > 1)
    wait_vm<(NS - 2) * kLoadsPerWave>();
  else
    wait_vm<0>();
  barrier();
  // one ring step: tile i in stage `cur`, tile i + NS - 1 goes to `nxt`
  auto step = [&](int i, auto cur, auto nxt) {
    const bool issue = i + NS - 1 < ntiles;
    if (issue) dma_tile(kt0 + i + NS - 1, nxt);
    const int kt = kt0 + i;
    if (kt < nt_w) compute(kt, cur);
    if (i + 1 < ntiles) {
      if (issue)
        wait_vm<(NS - 2) * kLoadsPerWave>();
      else
        wait_vm<0>();
      barrier();
    }
  };
  for (int i = 0; i < ntiles; i += NS) {
    if constexpr (NS == 3) {
      step(i, S0{}, S2{});
      if (i + 1 < ntiles) step(i + 1, S1{}, S0{});
      if (i + 2 < ntiles) step(i + 2, S2{}, S1{});
    } else {
      step(i, S0{}, S1{});
      if (i + 1 < ntiles) step(i + 1, S1{}, S0{});
    }
  }

  // 8 KB staging region ri of the (wave, head) outputs: stage ri / 4
  auto stage_region = [&](int ri) -> bf16* {
    unsigned char* base = ri < 4 ? smem0 : smem1;
    return reinterpret_cast<bf16*>(base + (ri & 3) * (32 * 128 * 2));
  };
  // normalise; stage [32 q][128 d] per (wave, head) through LDS, then
  // write whole 16-byte chunks of each row
  __syncthreads();   // the staging area overlaps the ring
#pragma unroll
  for (int hw = 0; hw < HW; ++hw) {
    const float l = pair_sum(l_run[hw]);
    const float inv = l > 0.f ? 1.f / l : 0.f;
    bf16* so = stage_region(wave * HW + hw);
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int d = db * 32 + 8 * (e >> 2) + 4 * lh + (e & 3);
        so[lr * 128 + (((d >> 3) ^ (lr & 15)) << 3) + (d & 7)] = f2bf(o[hw][db][e] * inv);
      }
  }
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): this wave's staging writes are done
  __builtin_amdgcn_wave_barrier();
  if (!active) return;
#pragma unroll
  for (int hw = 0; hw < HW; ++hw) {
    const bf16* so = stage_region(wave * HW + hw);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int q = lane + i * 64, row = q >> 4, cc = q & 15;
      const int t = t0w + row;
      if (t < a.T) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(so + row * 128 + ((cc ^ (row & 15)) << 3));
        *reinterpret_cast<u32x4*>(a.out + ((int64_t)b * a.T + t) * ldq + (int64_t)(head0 + hw) * 128 + cc * 8) = v;
      }
    }
  }
}

// Two ring stages: with two waves per SIMD a third measured no faster, and
// it costs registers.
constexpr int kStages = 2;
constexpr int kWaves = 8;
// q heads per wave and waves along the heads for a GQA ratio; false when no
// kernel instance has that shape
bool prefill_shape(int rep, int* hw, int* hg) {
  *hw = 1;
  *hg = rep < kWaves ? rep : kWaves;
  return rep >= 1 && (*hg == 1 || *hg == 2 || *hg == 4 || *hg == 8) && rep % *hg == 0;
}

PrefillPlan prefill_plan(int B, int T, int lq, int lkv) {
  int hw, hg;
  (void)prefill_shape(lq / lkv, &hw, &hg);
  PrefillPlan p{};
  p.rows = 32 * (kWaves / hg);
  p.n_rb = (T + p.rows - 1) / p.rows;
  p.hgroups = lq / lkv / (hw * hg);
  return p;
}

template <int HW, int HG>
hipError_t launch(const AttnArgs& a, const PrefillPlan& p, hipStream_t s) {
  const int64_t groups = (int64_t)a.B * a.lkv * p.hgroups;
  attn_prefill_kernel<HW, HG, kStages, kWaves><<<(unsigned)(groups * p.n_rb), kWaves * 64, 0, s>>>(a, p);
  kmark(s, "attn_prefill");
  return hipGetLastError();
}

}  // namespace

bool attn_prefill_fills(int B, int T, int lq, int lkv) {
  if (B <= 0 || T <= 0 || lkv <= 0 || lq % lkv) return false;
  int hw, hg;
  if (!prefill_shape(lq / lkv, &hw, &hg)) return false;
  const PrefillPlan p = prefill_plan(B, T, lq, lkv);
  return (int64_t)B * lkv * p.hgroups * p.n_rb >= 256;
}

hipError_t attn_prefill(const AttnArgs& a, hipStream_t s) {
  if (a.B <= 0 || a.T <= 0) return hipSuccess;
  // the kernel's wave shape comes from the same choice as the plan, and
  // together they must cover the GQA group exactly
  int hw, hg;
  if (a.lkv <= 0 || a.lq % a.lkv || !prefill_shape(a.lq / a.lkv, &hw, &hg)) return hipErrorInvalidValue;
  const PrefillPlan p = prefill_plan(a.B, a.T, a.lq, a.lkv);
  if (hw * hg * p.hgroups != a.lq / a.lkv) return hipErrorInvalidValue;
  if (hw == 1 && hg == 1) return launch<1, 1>(a, p, s);
  if (hw == 1 && hg == 2) return launch<1, 2>(a, p, s);
  if (hw == 1 && hg == 4) return launch<1, 4>(a, p, s);
  if (hw == 1 && hg == 8) return launch<1, 8>(a, p, s);
  return hipErrorInvalidValue;
}

}  // namespace tps
