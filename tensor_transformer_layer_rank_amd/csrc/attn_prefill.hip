// Prefill attention over the rank's local heads ("Tensor parallelism from
// scratch", "Implementation", TPAttention.forward): causal GQA attention of
// T new tokens after `past` cached ones, query t (position past + t) sees
// keys 0 .. past + t; q head i reads kv head i / rep; scale 1/sqrt(128).
//
// Flash-style on MFMA (v_mfma_f32_32x32x16_bf16).  A workgroup is 4 waves;
// each wave owns 32 query rows of one q head, and the waves of a workgroup
// share one kv head (up to 4 heads of the GQA group x the same rows, or
// fewer heads x more rows), so every K/V tile staged in LDS serves 128
// query rows.  Per 64-key tile:
//   S^T[64 keys, 32 q] = K_tile . Q^T   (A = K rows from LDS, B = Q in VGPRs)
// puts one query per lane column, so row max / row sum are lane-local plus
// one exchange with lane ^ 32; then
//   O^T[128 d, 32 q] += V^T . P^T       (A = V^T from LDS, B = P in VGPRs)
// V is transposed while being written to LDS (4 keys x 8 d per thread).
// The softmax runs in the exp2 domain with the running max per query.
#include "common.h"

namespace tps {

namespace {

constexpr int kTileKeys = 64;
constexpr int kStage = kTileKeys * 128 * 2;   // bf16 elements: K tile + V^T tile

__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

// K tile: [64 keys][16 chunks of 8 d]; chunk slot XOR (key & 15)
__device__ __forceinline__ int k_off(int key, int chunk) { return key * 128 + ((chunk ^ (key & 15)) << 3); }
// V^T tile: [128 d][16 granules of 4 keys]; granule slot XOR ((d >> 1) & 15)
__device__ __forceinline__ int vt_off(int d, int granule) { return d * 64 + ((granule ^ ((d >> 1) & 15)) << 2); }

template <int REP>
__global__ __launch_bounds__(256) void attn_prefill_kernel(AttnArgs a, int n_tb, float qscale) {
  constexpr int HPW = REP < 4 ? REP : 4;   // q heads per workgroup
  constexpr int RB = 4 / HPW;              // 32-row blocks per workgroup
  constexpr int ROWS = 32 * RB;
  __shared__ __attribute__((aligned(16))) bf16 smem[2 * kStage];

  // grid: [(b, kvh, head group) x row blocks]; heavy (late) row blocks first
  const int tb = n_tb - 1 - (int)(blockIdx.x % n_tb);
  int rest = blockIdx.x / n_tb;
  const int hgroups = REP / HPW;
  const int hg = rest % hgroups;
  rest /= hgroups;
  const int kvh = rest % a.lkv, b = rest / a.lkv;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 31, lh = lane >> 5;
  const int hh = wave / RB, rr = wave % RB;
  const int head = kvh * REP + hg * HPW + hh;
  const int t0 = tb * ROWS;
  const int tq = t0 + rr * 32 + lr;            // this lane's query row
  const int qpos = a.past + tq;
  const int64_t ldq = (int64_t)a.lq * 128;

  // Q^T fragments: lane supplies q[tq, head, ks*16 + lh*8 .. +8]
  bf16x8 qf[8];
  {
    const bool ok = tq < a.T;
    const bf16* qp = a.q + ((int64_t)b * a.T + (ok ? tq : 0)) * ldq + (int64_t)head * 128 + lh * 8;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      u32x4 r = ok ? *reinterpret_cast<const u32x4*>(qp + ks * 16) : u32x4{0u, 0u, 0u, 0u};
      qf[ks] = *reinterpret_cast<bf16x8*>(&r);
    }
  }

  const int t_end = min(a.T, t0 + ROWS);                 // rows of this block
  const int n_keys = a.past + t_end;                     // keys any row needs
  const int n_tiles = (n_keys + kTileKeys - 1) / kTileKeys;
  const int64_t slab = ((int64_t)b * a.lkv + kvh) * a.S_max * 128;
  const bf16* kg = a.k_cache + slab;
  const bf16* vg = a.v_cache + slab;

  // tile loaders: K 4 chunks per thread; V 4 keys x 8 d per thread
  u32x4 kr[4], vr[4];
  const int vq = tid >> 4, vdc = tid & 15;              // key quad, d chunk
  auto gload = [&](int tile) {
    const int key0 = tile * kTileKeys;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int q = tid + i * 256, key = q >> 4, c = q & 15;
      kr[i] = key0 + key < n_keys ? *reinterpret_cast<const u32x4*>(kg + (int64_t)(key0 + key) * 128 + c * 8)
                                  : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int key = key0 + vq * 4 + i;
      vr[i] = key < n_keys ? *reinterpret_cast<const u32x4*>(vg + (int64_t)key * 128 + vdc * 8)
                           : u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto sstore = [&](int buf) {
    bf16* sk = smem + buf * kStage;
    bf16* sv = sk + kTileKeys * 128;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int q = tid + i * 256, key = q >> 4, c = q & 15;
      *reinterpret_cast<u32x4*>(sk + k_off(key, c)) = kr[i];
    }
    // transpose: for d = vdc*8 + j, the 4 keys vq*4 .. +3 form one granule
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int w = j >> 1;
      uint32_t lo, hi;
      if (j & 1) {
        lo = (vr[0][w] >> 16) | (vr[1][w] & 0xFFFF0000u);
        hi = (vr[2][w] >> 16) | (vr[3][w] & 0xFFFF0000u);
      } else {
        lo = (vr[0][w] & 0xFFFFu) | (vr[1][w] << 16);
        hi = (vr[2][w] & 0xFFFFu) | (vr[3][w] << 16);
      }
      *reinterpret_cast<u32x2*>(sv + vt_off(vdc * 8 + j, vq)) = u32x2{lo, hi};
    }
  };

  f32x16 o[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[db][e] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  gload(0);
  sstore(0);
  __syncthreads();
  for (int tile = 0; tile < n_tiles; ++tile) {
    const int cur = tile & 1;
    if (tile + 1 < n_tiles) gload(tile + 1);
    const bf16* sk = smem + cur * kStage;
    const bf16* sv = sk + kTileKeys * 128;

    // S^T for keys kb*32 .. +32
    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int e = 0; e < 16; ++e) s[kb][e] = 0.f;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const int key = kb * 32 + lr;
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(sk + k_off(key, ks * 2 + lh));
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ks], s[kb], 0, 0, 0);
      }
    }
    // scale, causal mask, running max
    const int key0 = tile * kTileKeys;
    float mt = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int key = key0 + kb * 32 + 8 * (e >> 2) + 4 * lh + (e & 3);
        const float v = key <= qpos ? s[kb][e] * qscale : -INFINITY;
        s[kb][e] = v;
        mt = fmaxf(mt, v);
      }
    mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
    const float mn = fmaxf(m_run, mt);
    const float corr = m_run == -INFINITY ? 0.f : ex2(m_run - mn);
    m_run = mn;
    float ps = 0.f;
    bf16x8 pf[4];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float p = s[kb][e] == -INFINITY ? 0.f : ex2(s[kb][e] - mn);
        ps += p;
        pf[kb * 2 + (e >> 3)][e & 7] = f2bf(p);
      }
    l_run = l_run * corr + ps;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int e = 0; e < 16; ++e) o[db][e] *= corr;
    // O^T += V^T P^T; k-step ks covers keys (ks/2)*32 + (ks%2)*16 .. +16
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int g0 = ((ks >> 1) * 32 + (ks & 1) * 16) / 4 + lh;
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const int d = db * 32 + lr;
        const u32x2 x = *reinterpret_cast<const u32x2*>(sv + vt_off(d, g0));
        const u32x2 y = *reinterpret_cast<const u32x2*>(sv + vt_off(d, g0 + 2));
        u32x4 r = {x[0], x[1], y[0], y[1]};
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<bf16x8*>(&r), pf[ks], o[db], 0, 0, 0);
      }
    }
    if (tile + 1 < n_tiles) sstore(cur ^ 1);
    __syncthreads();
  }

  // normalise; stage [32 q][128 d] per wave through LDS for 16-byte stores
  const float l = l_run + __shfl_xor(l_run, 32, 64);
  const float inv = l > 0.f ? 1.f / l : 0.f;
  bf16* so = smem + wave * (32 * 128);
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int d = db * 32 + 8 * (e >> 2) + 4 * lh + (e & 3);
      so[lr * 128 + (((d >> 3) ^ (lr & 15)) << 3) + (d & 7)] = f2bf(o[db][e] * inv);
    }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int q = lane + i * 64, row = q >> 4, c = q & 15;
    const int t = t0 + rr * 32 + row;
    if (t < a.T) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(so + row * 128 + ((c ^ (row & 15)) << 3));
      *reinterpret_cast<u32x4*>(a.out + ((int64_t)b * a.T + t) * ldq + (int64_t)head * 128 + c * 8) = v;
    }
  }
}

template <int REP>
hipError_t launch(const AttnArgs& a, hipStream_t s) {
  constexpr int HPW = REP < 4 ? REP : 4;
  constexpr int ROWS = 32 * (4 / HPW);
  const int n_tb = (a.T + ROWS - 1) / ROWS;
  const int64_t blocks = (int64_t)n_tb * (REP / HPW) * a.lkv * a.B;
  const float qscale = 0.08838834764831845f * 1.4426950408889634f;   // log2(e)/sqrt(128)
  attn_prefill_kernel<REP><<<(unsigned)blocks, 256, 0, s>>>(a, n_tb, qscale);
  return hipGetLastError();
}

}  // namespace

hipError_t attn_prefill(const AttnArgs& a, hipStream_t s) {
  if (a.B <= 0 || a.T <= 0) return hipSuccess;
  switch (a.lq / a.lkv) {
    case 1: return launch<1>(a, s);
    case 2: return launch<2>(a, s);
    case 4: return launch<4>(a, s);
    case 8: return launch<8>(a, s);
    case 16: return launch<16>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace tps
