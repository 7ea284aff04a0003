// Decode attention over the rank's local heads ("Tensor parallelism from
// scratch", "Implementation", TPAttention.forward with one new token; "Two
// ways to split": heads are independent, so a rank attends with its own q
// heads over its own kv-cache heads; q head i reads kv head i / rep).
//
//   out[b, h, :] = sum_s softmax_s(q[b,h] . k[b,h/rep,s] / sqrt(128)) v[b,h/rep,s]
//   over s = 0 .. past (the new token was appended at position past).
//
// HBM-bound: every K and V row of the (b, kv head) slab is read once and
// serves all rep q heads of the group.  A workgroup takes one (b, kv head,
// key split); its 16 workers of 16 lanes stream key rows (16 lanes x 16 bytes
// = one 256-byte row, 4 rows per wave instruction), keep an online softmax
// per head (exp2 domain), and merge by log-sum-exp; splits are merged by a
// second kernel when more than one is used.
#include "common.h"

namespace tps {

namespace {

constexpr int kMinKeysPerSplit = 512;
constexpr int kTargetBlocks = 256;

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
}
// all 16 lanes of a DPP row get the row's sum
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp<0xB1>(v);    // quad_perm [1,0,3,2]
  v += dpp<0x4E>(v);    // quad_perm [2,3,0,1]
  v += dpp<0x141>(v);   // row_half_mirror
  v += dpp<0x140>(v);   // row_mirror
  return v;
}

__device__ __forceinline__ void unpack8(const u32x4& r, float* f) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(r[i] << 16);
    f[2 * i + 1] = __uint_as_float(r[i] & 0xFFFF0000u);
  }
}

__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

// reinterpret one 32-bit word as a bf16 pair (the word arrives by value:
// bit_cast applied directly to an element of a vector type is not reliable)
__device__ __forceinline__ bf16x2 as_bf16x2(uint32_t w) { return __builtin_bit_cast(bf16x2, w); }

// weight of a state with max m inside a merge whose max is M (0 for empty)
__device__ __forceinline__ float lse_w(float m, float M) { return m == -INFINITY ? 0.f : ex2(m - M); }

// REP q heads share a kv head; HS blocks split them (RH = REP / HS heads
// each) and read the same K/V rows -- the HS blocks of one item are placed
// on one XCD back to back, so all but the first read hit that XCD's L2.
template <int REP, int HS>
__global__ __launch_bounds__(256) void attn_decode_kernel(AttnArgs a, int nsplit, int keys_per_split,
                                                          float qscale) {
  constexpr int RH = REP / HS;
  __shared__ float s_o[4][RH][128];
  __shared__ float s_ml[4][RH][2];
  int item, hs;
  {
    const int bid = blockIdx.x, xcd = bid % 8, j = bid / 8;
    const int nitems = gridDim.x / HS;          // gridDim.x = items * HS, items % 8 == 0 when HS > 1
    item = HS == 1 ? bid : (j / HS) * 8 + xcd;
    hs = HS == 1 ? 0 : j % HS;
    (void)nitems;
  }
  const int split = item % nsplit;
  const int bk = item / nsplit;
  const int kvh = bk % a.lkv, b = bk / a.lkv;
  const int h0 = kvh * REP + hs * RH;            // first q head of this block
  const int S = a.past + 1;
  const int s0 = split * keys_per_split;
  const int s1 = min(S, s0 + keys_per_split);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15;
  const int worker = wave * 4 + (lane >> 4);

  // q stays packed (bf16 pairs); q.k uses v_dot2_f32_bf16 on the packed K row
  bf16x2 q2[RH][4];
#pragma unroll
  for (int h = 0; h < RH; ++h) {
    const bf16* qp = a.q + (int64_t)b * a.lq * 128 + (int64_t)(h0 + h) * 128 + l16 * 8;
    const u32x4 r = *reinterpret_cast<const u32x4*>(qp);
#pragma unroll
    for (int i = 0; i < 4; ++i) q2[h][i] = as_bf16x2(r[i]);
  }
  float m[RH], l[RH], o[RH][8];
#pragma unroll
  for (int h = 0; h < RH; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) o[h][i] = 0.f;
  }
  const int64_t slab = ((int64_t)b * a.lkv + kvh) * a.S_max * 128 + l16 * 8;
  const bf16* kb = a.k_cache + slab;
  const bf16* vb = a.v_cache + slab;

  // Branch-free streaming, one stage of U rows per worker ahead: while a
  // stage is scored, the next stage's K/V rows are already in flight.  Rows
  // past the split are clamped to its last row and their scores masked.
  constexpr int U = 4;
  const int n_it = (s1 - s0 + 16 * U - 1) / (16 * U);
  u32x4 kc[U], vc[U], kn[U], vn[U];
  auto load_rows = [&](u32x4* kk, u32x4* vv, int s) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int ss = min(s + 16 * u, s1 - 1);
      kk[u] = *reinterpret_cast<const u32x4*>(kb + (int64_t)ss * 128);
      vv[u] = *reinterpret_cast<const u32x4*>(vb + (int64_t)ss * 128);
    }
  };
  load_rows(kn, vn, s0 + worker);
  for (int it = 0; it < n_it; ++it) {
    const int s = s0 + worker + it * 16 * U;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      kc[u] = kn[u];
      vc[u] = vn[u];
    }
    if (it + 1 < n_it) load_rows(kn, vn, s + 16 * U);
    float sc[U][RH];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool valid = s + 16 * u < s1;
#pragma unroll
      for (int h = 0; h < RH; ++h) {
        float d = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) d = __builtin_amdgcn_fdot2_f32_bf16(q2[h][i], as_bf16x2(kc[u][i]), d, false);
        d = row16_sum(d) * qscale;
        sc[u][h] = valid ? d : -INFINITY;
      }
    }
#pragma unroll
    for (int h = 0; h < RH; ++h) {
      float mx = sc[0][h];
#pragma unroll
      for (int u = 1; u < U; ++u) mx = fmaxf(mx, sc[u][h]);
      const float mn = fmaxf(m[h], mx);
      const float corr = lse_w(m[h], mn);
      l[h] *= corr;
#pragma unroll
      for (int i = 0; i < 8; ++i) o[h][i] *= corr;
      m[h] = mn;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float vf[8];
      unpack8(vc[u], vf);
#pragma unroll
      for (int h = 0; h < RH; ++h) {
        const float p = lse_w(sc[u][h], m[h]);
        l[h] += p;
#pragma unroll
        for (int i = 0; i < 8; ++i) o[h][i] = fmaf(p, vf[i], o[h][i]);
      }
    }
  }

  // merge the 4 workers of each wave (rows of 16 lanes) by log-sum-exp
#pragma unroll
  for (int off = 16; off <= 32; off <<= 1) {
#pragma unroll
    for (int h = 0; h < RH; ++h) {
      const float m2 = __shfl_xor(m[h], off, 64);
      const float l2 = __shfl_xor(l[h], off, 64);
      const float mn = fmaxf(m[h], m2);
      const float w1 = lse_w(m[h], mn), w2 = lse_w(m2, mn);
      l[h] = l[h] * w1 + l2 * w2;
#pragma unroll
      for (int i = 0; i < 8; ++i) o[h][i] = o[h][i] * w1 + __shfl_xor(o[h][i], off, 64) * w2;
      m[h] = mn;
    }
  }
  if (lane < 16) {
#pragma unroll
    for (int h = 0; h < RH; ++h) {
#pragma unroll
      for (int i = 0; i < 8; ++i) s_o[wave][h][l16 * 8 + i] = o[h][i];
      if (l16 == 0) {
        s_ml[wave][h][0] = m[h];
        s_ml[wave][h][1] = l[h];
      }
    }
  }
  __syncthreads();
  for (int e = tid; e < RH * 128; e += 256) {
    const int h = e / 128, d = e % 128;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, s_ml[w][h][0]);
    float L = 0.f, O = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float wt = lse_w(s_ml[w][h][0], M);
      L += s_ml[w][h][1] * wt;
      O += s_o[w][h][d] * wt;
    }
    if (nsplit == 1) {
      a.out[(int64_t)b * a.lq * 128 + (int64_t)(h0 + h) * 128 + d] = f2bf(L > 0.f ? O / L : 0.f);
    } else {
      const int64_t base = (int64_t)item * REP + hs * RH + h;
      a.scratch[base * 128 + d] = O;
      if (d == 0) {
        float* ml = a.scratch + (int64_t)(gridDim.x / HS) * REP * 128;
        ml[base * 2] = M;
        ml[base * 2 + 1] = L;
      }
    }
  }
}

// merge the splits of each (b, q head): one thread per output element
__global__ __launch_bounds__(256) void attn_decode_combine(AttnArgs a, int nsplit, int rep, int items) {
  const int64_t total = (int64_t)a.B * a.lq * 128;
  const float* ml = a.scratch + (int64_t)items * rep * 128;
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < total; e += (int64_t)gridDim.x * 256) {
    const int d = (int)(e % 128);
    const int64_t bh = e / 128;
    const int hq = (int)(bh % a.lq);
    const int b = (int)(bh / a.lq);
    const int kvh = hq / rep, h = hq % rep;
    const int64_t item0 = ((int64_t)b * a.lkv + kvh) * nsplit;
    float M = -INFINITY;
    for (int sp = 0; sp < nsplit; ++sp) M = fmaxf(M, ml[((item0 + sp) * rep + h) * 2]);
    float L = 0.f, O = 0.f;
    for (int sp = 0; sp < nsplit; ++sp) {
      const int64_t base = (item0 + sp) * rep + h;
      const float wt = lse_w(ml[base * 2], M);
      L += ml[base * 2 + 1] * wt;
      O += a.scratch[base * 128 + d] * wt;
    }
    a.out[(int64_t)b * a.lq * 128 + (int64_t)hq * 128 + d] = f2bf(L > 0.f ? O / L : 0.f);
  }
}

// One split per (b, kv head) while that already gives about one block per
// CU: a block then streams its whole slab and no merge pass is needed.
// Smaller grids split the keys (at least kMinKeysPerSplit per split).
void split_plan(int B, int lkv, int S, int& nsplit, int& kps) {
  const int items = B * lkv;
  int ns = (kTargetBlocks + items - 1) / items;
  const int maxs = (S + kMinKeysPerSplit - 1) / kMinKeysPerSplit;
  if (ns > maxs) ns = maxs;
  if (ns < 1) ns = 1;
  kps = (S + ns - 1) / ns;
  nsplit = (S + kps - 1) / kps;    // every split holds at least one key
}

template <int REP, int HS>
hipError_t launch(const AttnArgs& a, hipStream_t s) {
  const int S = a.past + 1;
  int nsplit, kps;
  split_plan(a.B, a.lkv, S, nsplit, kps);
  const int items = a.B * a.lkv * nsplit;
  // 1/sqrt(128) with log2(e) folded in: scores are in the exp2 domain
  const float qscale = 0.08838834764831845f * 1.4426950408889634f;
  if (HS > 1 && items % 8 != 0) return launch<REP, 1>(a, s);
  attn_decode_kernel<REP, HS><<<items * HS, 256, 0, s>>>(a, nsplit, kps, qscale);
  if (nsplit > 1) {
    const int64_t total = (int64_t)a.B * a.lq * 128;
    int64_t g = (total + 255) / 256;
    if (g > 4096) g = 4096;
    attn_decode_combine<<<(int)g, 256, 0, s>>>(a, nsplit, REP, items);
  }
  return hipGetLastError();
}

}  // namespace

size_t attn_decode_scratch_bytes(int B, int lq, int lkv, int ctx) {
  if (B <= 0 || lkv <= 0 || ctx <= 0) return 0;
  int nsplit, kps;
  split_plan(B, lkv, ctx, nsplit, kps);
  if (nsplit == 1) return 0;
  return (size_t)B * lq * nsplit * (128 + 2) * sizeof(float);
}

hipError_t attn_decode(const AttnArgs& a, hipStream_t s) {
  if (a.B <= 0) return hipSuccess;
  switch (a.lq / a.lkv) {
    case 1: return launch<1, 1>(a, s);
    case 2: return launch<2, 1>(a, s);
    case 4: return launch<4, 1>(a, s);
    case 8: return launch<8, 2>(a, s);
    case 16: return launch<16, 4>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace tps
