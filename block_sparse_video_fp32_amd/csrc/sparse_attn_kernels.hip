// gfx950 kernels of routed block-sparse attention.
//
//   pool_kernel    per-64-row-block means of Q, K, V in FP32 (HBM-bound
//                  stream), plus bf16 copies of the K and V centroids for the
//                  MFMA centroid pass (Star7 README, 工作原理 > Sol: Q64/K64
//                  blocks; Spark-H3 news, Spark-Reweight: mean-pooled K/V).
//   select_kernel  fp32 block scores Qbar_a . Kbar_c for a group of query
//                  blocks against every key block, then per query block
//                  (one wave each) the threshold mean + tau * std (two-pass,
//                  population) or an exact radix top-K, the prefix sink, and
//                  ballot compaction into an ascending index list
//                  (thakicloud accel-stack post, 이 기술은 무엇인가; Spark-H3
//                  news, 워크플로: topk_ratio).
//   attend_kernel  one workgroup per (b, h, query block): exact bf16
//                  attention on MFMA over the listed key blocks, then one
//                  centroid logit per unselected block with the log-mass bias,
//                  all merged into the same FP32 online softmax (Star7 README,
//                  Sol: missed blocks contribute through a K/V centroid in the
//                  same FP32 online softmax).
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "sa_internal.h"
#include "sparse_attn.h"

namespace sa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// float -> bf16 bits, round to nearest even (NaN kept quiet).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ float lane_bf16(const uint4& w, int e) {
  const uint32_t word = (e < 2) ? w.x : (e < 4) ? w.y : (e < 6) ? w.z : w.w;
  return bf16_bits_to_f32((e & 1) ? (word >> 16) : (word & 0xffffu));
}

__device__ __forceinline__ uint32_t half16(const uint4& w, int e) {
  const uint32_t word = (e < 2) ? w.x : (e < 4) ? w.y : (e < 6) ? w.z : w.w;
  return (e & 1) ? (word >> 16) : (word & 0xffffu);
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

// ---------------------------------------------------------------------------
// pool: grid (n_bp, 3 tensors, B * head groups), 256 threads.  A thread owns
// one 16-byte column chunk (8 values of one head) and sums half of the
// block's rows; the two halves are added in a fixed order.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void pool_kernel(Shape s, const uint16_t* __restrict__ q,
                                                   const uint16_t* __restrict__ k,
                                                   const uint16_t* __restrict__ v, Workspace ws) {
  constexpr int CPH = D / 8;          // chunks per head row
  constexpr int HG = 128 / CPH;       // heads per workgroup
  constexpr int CHUNKS = HG * CPH;    // 128 chunks
  constexpr int RPS = 32;             // rows per half
  static_assert(CHUNKS * 2 == 256, "two row halves of 128 chunks");
  __shared__ float part[CHUNKS * 8];

  const int j = blockIdx.x;
  const int t = blockIdx.y;
  const int hgroups = (s.H + HG - 1) / HG;
  const int b = blockIdx.z / hgroups;
  const int hg = blockIdx.z - b * hgroups;
  const int tid = threadIdx.x;
  const int chunk = tid % CHUNKS;
  const int half = tid / CHUNKS;
  const int h = hg * HG + chunk / CPH;
  const int d0 = (chunk % CPH) * 8;
  const bool active = h < s.H;
  const long long bh = (long long)b * s.H + h;

  if (j >= s.nb) {  // zero padding rows of the bf16 centroid arrays
    if (t > 0 && active && half == 0) {
      uint16_t* dst = (t == 1 ? ws.kbar16 : ws.vbar16) + (bh * s.nbp + j) * D + d0;
      *reinterpret_cast<uint4*>(dst) = make_uint4(0, 0, 0, 0);
    }
    return;
  }

  const uint16_t* src = (t == 0) ? q : (t == 1) ? k : v;
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.0f;
  const int r0 = j * kBlock + half * RPS;
  const int rend = min(s.N, r0 + RPS);
  if (active && r0 < rend) {
    const uint16_t* p = src + (long long)b * s.isb + (long long)h * s.ish + d0 + (long long)r0 * s.ist;
    const int n = rend - r0;
    int r = 0;
    for (; r + 8 <= n; r += 8) {
      uint4 x[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) x[u] = *reinterpret_cast<const uint4*>(p + (long long)(r + u) * s.ist);
#pragma unroll
      for (int u = 0; u < 8; ++u)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] += lane_bf16(x[u], e);
    }
    for (; r < n; ++r) {
      const uint4 x = *reinterpret_cast<const uint4*>(p + (long long)r * s.ist);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += lane_bf16(x, e);
    }
  }
  if (half == 1) {
#pragma unroll
    for (int e = 0; e < 8; ++e) part[chunk * 8 + e] = acc[e];
  }
  __syncthreads();
  if (half == 0 && active) {
    const float n = (float)min(kBlock, s.N - j * kBlock);
    float m[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) m[e] = (acc[e] + part[chunk * 8 + e]) / n;
    float* dst = (t == 0 ? ws.qbar : t == 1 ? ws.kbar : ws.vbar) + (bh * s.nb + j) * D + d0;
    reinterpret_cast<float4*>(dst)[0] = make_float4(m[0], m[1], m[2], m[3]);
    reinterpret_cast<float4*>(dst)[1] = make_float4(m[4], m[5], m[6], m[7]);
    if (t > 0) {
      uint4 w;
      w.x = f32_to_bf16_bits(m[0]) | (f32_to_bf16_bits(m[1]) << 16);
      w.y = f32_to_bf16_bits(m[2]) | (f32_to_bf16_bits(m[3]) << 16);
      w.z = f32_to_bf16_bits(m[4]) | (f32_to_bf16_bits(m[5]) << 16);
      w.w = f32_to_bf16_bits(m[6]) | (f32_to_bf16_bits(m[7]) << 16);
      uint16_t* d16 = (t == 1 ? ws.kbar16 : ws.vbar16) + (bh * s.nbp + j) * D + d0;
      *reinterpret_cast<uint4*>(d16) = w;
    }
  }
}

// ---------------------------------------------------------------------------
// select: grid (ceil(n_b / R), H, B), 256 threads, dynamic LDS.
// Phase 1: S[r][c] for R query blocks and every key block, fp32, the dot
// product summed in d order.  Phase 2: wave w routes rows w*R/4 .. +R/4-1.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t order_key(float f) {
  if (f == 0.0f) f = 0.0f;  // -0 and +0 rank together
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

template <int D, int R>
__global__ __launch_bounds__(256) void select_kernel(Shape s, Workspace ws) {
  constexpr int KSTR = D + 4;  // fp32 row stride of the key tile
  constexpr int RPW = R / 4;   // rows per wave
  extern __shared__ __attribute__((aligned(16))) float sm[];
  float* qs = sm;                 // [R][D]
  float* ks = qs + R * D;         // [64][KSTR]
  float* S = ks + 64 * KSTR;      // [R][nb]
  int* hist = reinterpret_cast<int*>(S + R * s.nb);  // [4][256]

  const int nb = s.nb;
  const int a0 = blockIdx.x * R;
  const int h = blockIdx.y, b = blockIdx.z;
  const long long bh = (long long)b * s.H + h;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const float* qbar = ws.qbar + bh * nb * D;
  const float* kbar = ws.kbar + bh * nb * D;

  for (int i = tid; i < R * D / 4; i += 256) {
    const int r = i / (D / 4), c4 = i % (D / 4);
    float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
    if (a0 + r < nb) x = reinterpret_cast<const float4*>(qbar + (long long)(a0 + r) * D)[c4];
    reinterpret_cast<float4*>(qs + r * D)[c4] = x;
  }
  for (int c0 = 0; c0 < nb; c0 += 64) {
    __syncthreads();
    for (int i = tid; i < 64 * D / 4; i += 256) {
      const int r = i / (D / 4), c4 = i % (D / 4);
      float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
      if (c0 + r < nb) x = reinterpret_cast<const float4*>(kbar + (long long)(c0 + r) * D)[c4];
      reinterpret_cast<float4*>(ks + r * KSTR)[c4] = x;
    }
    __syncthreads();
    float acc[RPW];
#pragma unroll
    for (int i = 0; i < RPW; ++i) acc[i] = 0.0f;
    const float* kr = ks + lane * KSTR;
#pragma unroll 4
    for (int d = 0; d < D; d += 4) {
      const float4 kv = *reinterpret_cast<const float4*>(kr + d);
#pragma unroll
      for (int i = 0; i < RPW; ++i) {
        const float4 qv = *reinterpret_cast<const float4*>(qs + (w * RPW + i) * D + d);
        acc[i] = fmaf(qv.x, kv.x, acc[i]);
        acc[i] = fmaf(qv.y, kv.y, acc[i]);
        acc[i] = fmaf(qv.z, kv.z, acc[i]);
        acc[i] = fmaf(qv.w, kv.w, acc[i]);
      }
    }
    const int c = c0 + lane;
    if (c < nb) {
#pragma unroll
      for (int i = 0; i < RPW; ++i) S[(w * RPW + i) * nb + c] = acc[i];
    }
  }
  __syncthreads();

  int* my_hist = hist + w * 256;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int i = 0; i < RPW; ++i) {
    const int r = w * RPW + i;
    const int a = a0 + r;
    if (a >= nb) break;
    const float* Srow = S + r * nb;
    int* list = ws.lists + (bh * nb + a) * (long long)nb;
    if (s.dense || a < s.pb) {  // dense row: every block
      for (int c = lane; c < nb; c += 64) list[c] = c;
      if (lane == 0) ws.counts[bh * nb + a] = nb;
      continue;
    }
    int base = 0;
    if (s.route == SA_ROUTE_TAU) {
      float thr;
      if (isinf(s.tau) && s.tau > 0.0f) {
        thr = INFINITY;
      } else {
        float sum = 0.0f;
        for (int c = lane; c < nb; c += 64) sum += Srow[c];
        const float mu = wave_sum(sum) / (float)nb;
        float ss = 0.0f;
        for (int c = lane; c < nb; c += 64) {
          const float dlt = Srow[c] - mu;
          ss = fmaf(dlt, dlt, ss);
        }
        const float sigma = sqrtf(wave_sum(ss) / (float)nb);
        thr = fmaf(s.tau, sigma, mu);
      }
      for (int c0 = 0; c0 < nb; c0 += 64) {
        const int c = c0 + lane;
        const bool pred = c < nb && (Srow[c] >= thr || c < s.pb);
        const uint64_t m = __ballot(pred);
        if (pred) list[base + __popcll(m & lt_mask)] = c;
        base += __popcll(m);
      }
    } else {
      // Exact k-th largest key by four 8-bit radix passes (MSB first).
      uint32_t prefix = 0, pmask = 0;
      int kk = s.topk;
      for (int shift = 24; shift >= 0; shift -= 8) {
        for (int x = lane; x < 256; x += 64) my_hist[x] = 0;
        wave_lds_sync();
        for (int c = lane; c < nb; c += 64) {
          const uint32_t u = order_key(Srow[c]);
          if ((u & pmask) == prefix) atomicAdd(&my_hist[(u >> shift) & 255u], 1);
        }
        wave_lds_sync();
        // lane owns digits 255-4l .. 252-4l (descending)
        const int h0 = my_hist[255 - 4 * lane], h1 = my_hist[254 - 4 * lane];
        const int h2 = my_hist[253 - 4 * lane], h3 = my_hist[252 - 4 * lane];
        const int tot = h0 + h1 + h2 + h3;
        int incl = tot;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
          const int y = __shfl_up(incl, o);
          if (lane >= o) incl += y;
        }
        const int excl = incl - tot;
        const bool mine = excl < kk && kk <= incl;
        int digit = 0, above = 0;
        if (mine) {
          if (kk <= excl + h0) { digit = 255 - 4 * lane; above = excl; }
          else if (kk <= excl + h0 + h1) { digit = 254 - 4 * lane; above = excl + h0; }
          else if (kk <= excl + h0 + h1 + h2) { digit = 253 - 4 * lane; above = excl + h0 + h1; }
          else { digit = 252 - 4 * lane; above = excl + h0 + h1 + h2; }
        }
        const uint64_t mb = __ballot(mine);
        const int src = __ffsll((long long)mb) - 1;
        digit = __shfl(digit, src);
        above = __shfl(above, src);
        kk -= above;
        prefix |= (uint32_t)digit << shift;
        pmask |= 0xffu << shift;
        wave_lds_sync();
      }
      const uint32_t T = prefix;
      int eqbase = 0;
      for (int c0 = 0; c0 < nb; c0 += 64) {
        const int c = c0 + lane;
        const uint32_t u = c < nb ? order_key(Srow[c]) : 0u;
        const bool eq = c < nb && u == T;
        const uint64_t em = __ballot(eq);
        const int eqpos = eqbase + __popcll(em & lt_mask);
        eqbase += __popcll(em);
        const bool pred = c < nb && (u > T || (eq && eqpos < kk) || c < s.pb);
        const uint64_t m = __ballot(pred);
        if (pred) list[base + __popcll(m & lt_mask)] = c;
        base += __popcll(m);
      }
    }
    if (lane == 0) ws.counts[bh * nb + a] = base;
  }
}

// ---------------------------------------------------------------------------
// attend: grid B*H*n_b (XCD-aware order), 256 threads = 4 waves of 16 query
// rows.  Per tile of 64 keys (an exact block, or 64 centroids) K is staged
// row-major and V transposed in LDS, double-buffered.  Each wave computes
// S^T = K Q^T with v_mfma_f32_16x16x32_bf16 (lane l holds keys 4(l/16)+i of
// each 16-key tile for query l%16), so the softmax reductions are in-lane
// plus two cross-lane steps, and P^T feeds O^T = V^T P^T straight from
// registers: the MFMA's k index is a free permutation as long as both
// operands agree, and the V^T reads follow the register order of P^T.
// ---------------------------------------------------------------------------
template <int D>
struct AttendCfg {
  static constexpr int KS = D + 8;        // K tile row stride (bf16)
  static constexpr int VS = 64 + 8;       // V^T tile row stride (bf16)
  static constexpr int KT = 64 * KS;
  static constexpr int VT = D * VS;
  static constexpr int BUF = KT + VT;     // one stage, bf16 elements
  static constexpr int NS = D / 32;       // k-steps of Q K^T
  static constexpr int NDT = D / 16;      // 16-row tiles of O^T
  static constexpr int CPR = D / 8;       // 16-byte chunks per row
  static constexpr int NCH = CPR / 4;     // chunks per thread per tensor
  static constexpr int KPT = CPR / 4;     // consecutive keys per thread (V)
};

struct TileInfo {
  const uint16_t* ksrc;  // row 0 of the K (or Kbar) tile
  const uint16_t* vsrc;
  long long rstride;     // element stride between rows
  int nvalid;            // rows that exist
  int kind;              // 0 exact block, 1 centroid tile
  int c;                 // block index or centroid tile index
};

template <int D>
__global__ __launch_bounds__(256) void attend_kernel(Shape s, const uint16_t* __restrict__ q,
                                                     const uint16_t* __restrict__ k,
                                                     const uint16_t* __restrict__ v,
                                                     uint16_t* __restrict__ out, Workspace ws) {
  using C = AttendCfg<D>;
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * C::BUF];
  __shared__ uint32_t selbits[SA_MAX_BLOCKS / 32];

  // Consecutive logical ids go to one XCD (workgroups are dealt to the 8 XCDs
  // round-robin), so one head's query blocks share that XCD's L2.
  const int G = gridDim.x, bid = blockIdx.x;
  const int xcd = bid & 7, kx = bid >> 3, qq = G >> 3, rr = G & 7;
  const int lid = (xcd < rr) ? xcd * (qq + 1) + kx : rr * (qq + 1) + (xcd - rr) * qq + kx;
  const int nb = s.nb;
  const int a = lid % nb;
  const int bhi = lid / nb;
  const int h = bhi % s.H, b = bhi / s.H;
  const long long bh = bhi;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int l16 = lane & 15, g = lane >> 4;

  // Q^T fragments (B operand): query a*64 + wave*16 + l16, d = 32 s + 8 g + e.
  const long long in_base = (long long)b * s.isb + (long long)h * s.ish;
  const int qrow = a * kBlock + wave * 16 + l16;
  bf16x8 qf[C::NS];
#pragma unroll
  for (int st = 0; st < C::NS; ++st) {
    uint4 x = make_uint4(0, 0, 0, 0);
    if (qrow < s.N) x = *reinterpret_cast<const uint4*>(q + in_base + (long long)qrow * s.ist + 32 * st + 8 * g);
    qf[st] = __builtin_bit_cast(bf16x8, x);
  }

  int count = nb;
  if (!s.dense) count = min(max(ws.counts[bh * nb + a], 0), nb);
  const int* list = ws.lists + (bh * nb + a) * (long long)nb;
  const bool cpass = !s.dense && s.centroid && count < nb;
  const int ctiles = cpass ? s.nbp / 64 : 0;
  if (cpass) {
    for (int i = tid; i < s.nbp / 32; i += 256) selbits[i] = 0u;
    __syncthreads();
    for (int i = tid; i < count; i += 256) {
      const int c = list[i];
      if (c >= 0 && c < nb) atomicOr(&selbits[c >> 5], 1u << (c & 31));
    }
  }
  const int T = count + ctiles;

  auto tile_info = [&](int t) {
    TileInfo ti;
    if (t < count) {
      const int c = s.dense ? t : list[t];
      const bool ok = c >= 0 && c < nb;
      const int cc = ok ? c : 0;
      ti.ksrc = k + in_base + (long long)cc * kBlock * s.ist;
      ti.vsrc = v + in_base + (long long)cc * kBlock * s.ist;
      ti.rstride = s.ist;
      ti.nvalid = ok ? min(kBlock, s.N - cc * kBlock) : 0;
      ti.kind = 0;
      ti.c = cc;
    } else {
      const int j = t - count;
      const long long off = (bh * s.nbp + (long long)j * 64) * D;
      ti.ksrc = ws.kbar16 + off;
      ti.vsrc = ws.vbar16 + off;
      ti.rstride = D;
      ti.nvalid = 64;
      ti.kind = 1;
      ti.c = j;
    }
    return ti;
  };

  uint4 kreg[C::NCH], vreg[C::KPT];
  const int kcol = tid % C::CPR;
  const int krow0 = tid / C::CPR;             // K rows krow0 + (256/CPR) i
  const int vgrp = tid / C::CPR;              // V rows vgrp*KPT + i
  auto load_tile = [&](const TileInfo& ti) {
#pragma unroll
    for (int i = 0; i < C::NCH; ++i) {
      const int r = krow0 + (256 / C::CPR) * i;
      kreg[i] = (r < ti.nvalid) ? *reinterpret_cast<const uint4*>(ti.ksrc + (long long)r * ti.rstride + kcol * 8)
                                : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < C::KPT; ++i) {
      const int r = vgrp * C::KPT + i;
      vreg[i] = (r < ti.nvalid) ? *reinterpret_cast<const uint4*>(ti.vsrc + (long long)r * ti.rstride + kcol * 8)
                                : make_uint4(0, 0, 0, 0);
    }
  };
  auto store_tile = [&](int buf) {
    uint16_t* Kl = smem + buf * C::BUF;
    uint16_t* Vl = Kl + C::KT;
#pragma unroll
    for (int i = 0; i < C::NCH; ++i) {
      const int r = krow0 + (256 / C::CPR) * i;
      *reinterpret_cast<uint4*>(Kl + r * C::KS + kcol * 8) = kreg[i];
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      uint16_t* dst = Vl + (kcol * 8 + e) * C::VS + vgrp * C::KPT;
      if constexpr (C::KPT == 4) {
        uint2 w2;
        w2.x = half16(vreg[0], e) | (half16(vreg[1], e) << 16);
        w2.y = half16(vreg[2], e) | (half16(vreg[3], e) << 16);
        *reinterpret_cast<uint2*>(dst) = w2;
      } else {
        *reinterpret_cast<uint32_t*>(dst) = half16(vreg[0], e) | (half16(vreg[1], e) << 16);
      }
    }
  };

  float m_run = -INFINITY, l_run = 0.0f;
  f32x4 acc[C::NDT];
#pragma unroll
  for (int dt = 0; dt < C::NDT; ++dt) acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  TileInfo cur;
  if (T > 0) {
    cur = tile_info(0);
    load_tile(cur);
    store_tile(0);
  }
  __syncthreads();

  for (int t = 0; t < T; ++t) {
    const int buf = t & 1;
    TileInfo nxt;
    const bool more = t + 1 < T;
    if (more) {
      nxt = tile_info(t + 1);
      load_tile(nxt);
    }
    const uint16_t* Kl = smem + buf * C::BUF;
    const uint16_t* Vl = Kl + C::KT;

    // S^T tiles: st[kt][i] = K[16 kt + 4 g + i] . Q[l16]
    f32x4 st[4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      st[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ss = 0; ss < C::NS; ++ss) {
        const uint4 x = *reinterpret_cast<const uint4*>(Kl + (16 * kt + l16) * C::KS + 32 * ss + 8 * g);
        st[kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, x), qf[ss], st[kt], 0, 0, 0);
      }
    }

    // logits in the log2 domain, masked
    float x[4][4];
    if (cur.kind == 0) {
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = 16 * kt + 4 * g + i;
          x[kt][i] = (key < cur.nvalid) ? st[kt][i] * s.c1 : -INFINITY;
        }
    } else {
      const int cbase = cur.c * 64;
      const uint64_t bits = (uint64_t)selbits[cbase >> 5] | ((uint64_t)selbits[(cbase >> 5) + 1] << 32);
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = 16 * kt + 4 * g + i;
          const int cc = cbase + key;
          const bool ok = cc < nb && !((bits >> key) & 1ull);
          const float bias = (cc == nb - 1) ? s.bias_tail : s.bias_full;
          x[kt][i] = ok ? fmaf(st[kt][i], s.c1, bias) : -INFINITY;
        }
    }

    float mx = x[0][0];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int i = 0; i < 4; ++i) mx = fmaxf(mx, x[kt][i]);
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));

    // Lazy rescale: keep the running max until a row grows by more than 2^8.
    if (__ballot(mx > m_run + 8.0f)) {
      const float mnew = fmaxf(m_run, mx);
      const float alpha = (m_run == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(m_run - mnew);
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < C::NDT; ++dt) acc[dt] *= alpha;
      m_run = mnew;
    }
    const float msub = (m_run == -INFINITY) ? 0.0f : m_run;

    bf16x8 pb[2];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = __builtin_amdgcn_exp2f(x[kt][i] - msub);
        l_run += p;
        pb[kt >> 1][(kt & 1) * 4 + i] = (__bf16)p;
      }

    // O^T += V^T P^T; lane reads V^T[d][32 s + 4 g + 0..3] and [.. + 16 + 0..3]
#pragma unroll
    for (int dt = 0; dt < C::NDT; ++dt) {
#pragma unroll
      for (int ss = 0; ss < 2; ++ss) {
        const uint16_t* vp = Vl + (16 * dt + l16) * C::VS + 32 * ss + 4 * g;
        const uint2 lo = *reinterpret_cast<const uint2*>(vp);
        const uint2 hi = *reinterpret_cast<const uint2*>(vp + 16);
        const uint4 x4 = make_uint4(lo.x, lo.y, hi.x, hi.y);
        acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, x4), pb[ss], acc[dt], 0, 0, 0);
      }
    }

    if (more) {
      store_tile(buf ^ 1);
      cur = nxt;
    }
    __syncthreads();
  }

  float l = l_run;
  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);
  const float inv = (l > 0.0f) ? 1.0f / l : 0.0f;
  if (qrow < s.N) {
    uint16_t* o = out + (long long)b * s.osb + (long long)h * s.osh + (long long)qrow * s.ost;
#pragma unroll
    for (int dt = 0; dt < C::NDT; ++dt) {
      uint2 w2;
      w2.x = f32_to_bf16_bits(acc[dt][0] * inv) | (f32_to_bf16_bits(acc[dt][1] * inv) << 16);
      w2.y = f32_to_bf16_bits(acc[dt][2] * inv) | (f32_to_bf16_bits(acc[dt][3] * inv) << 16);
      *reinterpret_cast<uint2*>(o + 16 * dt + 4 * g) = w2;
    }
  }
}

template <int D, int R>
hipError_t launch_select_t(const Shape& s, const Workspace& ws, hipStream_t stream) {
  const size_t lds = (size_t)(R * D + 64 * (D + 4) + R * s.nb) * sizeof(float) + 4 * 256 * sizeof(int);
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&select_kernel<D, R>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  dim3 grid((s.nb + R - 1) / R, s.H, s.B);
  hipLaunchKernelGGL((select_kernel<D, R>), grid, dim3(256), lds, stream, s, ws);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_pool(const Shape& s, const void* q, const void* k, const void* v, const Workspace& ws,
                       hipStream_t stream) {
  const int hg = 128 / (s.D / 8);
  dim3 grid(s.nbp, 3, s.B * ((s.H + hg - 1) / hg));
  const auto* qq = static_cast<const uint16_t*>(q);
  const auto* kk = static_cast<const uint16_t*>(k);
  const auto* vv = static_cast<const uint16_t*>(v);
  if (s.D == 128)
    hipLaunchKernelGGL(pool_kernel<128>, grid, dim3(256), 0, stream, s, qq, kk, vv, ws);
  else
    hipLaunchKernelGGL(pool_kernel<64>, grid, dim3(256), 0, stream, s, qq, kk, vv, ws);
  return hipGetLastError();
}

hipError_t launch_select(const Shape& s, const Workspace& ws, hipStream_t stream) {
  const bool big = s.nb > 1536;
  if (s.D == 128) return big ? launch_select_t<128, 8>(s, ws, stream) : launch_select_t<128, 16>(s, ws, stream);
  return big ? launch_select_t<64, 8>(s, ws, stream) : launch_select_t<64, 16>(s, ws, stream);
}

hipError_t launch_attend(const Shape& s, const void* q, const void* k, const void* v, void* out,
                         const Workspace& ws, hipStream_t stream) {
  dim3 grid((unsigned)((long long)s.B * s.H * s.nb));
  const auto* qq = static_cast<const uint16_t*>(q);
  const auto* kk = static_cast<const uint16_t*>(k);
  const auto* vv = static_cast<const uint16_t*>(v);
  auto* oo = static_cast<uint16_t*>(out);
  if (s.D == 128)
    hipLaunchKernelGGL(attend_kernel<128>, grid, dim3(256), 0, stream, s, qq, kk, vv, oo, ws);
  else
    hipLaunchKernelGGL(attend_kernel<64>, grid, dim3(256), 0, stream, s, qq, kk, vv, oo, ws);
  return hipGetLastError();
}

}  // namespace sa
