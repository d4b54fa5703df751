// gfx950 kernels of routed block-sparse attention.
//
//   pool_q_kernel  per-64-row-block means of Q in FP32 (HBM-bound stream;
//                  Star7 README, 工作原理 > Sol: Q64/K64 blocks).
//   pack_kv_kernel per block of one head: the FP32 means of K and V (the
//                  centroids; Spark-H3 news, Spark-Reweight: mean-pooled K/V
//                  summaries), plus K, V^T and the centroids rewritten in the
//                  register order of the attend kernel's MFMA operands, so
//                  that every operand load there is one coalesced 1 KB read.
//   select_kernel  fp32 block scores Qbar_a . Kbar_c for a group of query
//                  blocks against every key block, then per query block
//                  (one wave each) the threshold mean + tau * std (two-pass,
//                  population) or an exact radix top-K, the prefix sink, and
//                  ballot compaction into an ascending index list
//                  (thakicloud accel-stack post, 이 기술은 무엇인가; Spark-H3
//                  news, 워크플로: topk_ratio).
//   attend_kernel  one wave per (b, h, query block): exact bf16 attention on
//                  MFMA over the listed key blocks, then one centroid logit
//                  per unselected block with the log-mass bias, all merged
//                  into the same FP32 online softmax (Star7 README, Sol:
//                  missed blocks contribute through a K/V centroid in the
//                  same FP32 online softmax).
//
// Packed operand layouts (bf16).  A "half tile" is 32 keys x D.
//   K half tile:   element ((kt*NS + ss)*64 + lane)*8 + e holds
//                  K[16 kt + lane%16][32 ss + 8 (lane/16) + e]   (NS = D/32)
//   V^T half tile: element d*32 + 8 g + e holds V[keyslot(g, e)][d] with
//                  keyslot(g, e) = 4 g + e for e < 4, 16 + 4 g + e - 4 else.
// These are the A-operand registers of v_mfma_f32_16x16x32_bf16 for
// S^T = K Q^T and O^T = V^T P^T; keyslot() is the order in which the S^T
// accumulator holds the keys, so P^T goes from accumulator to B operand
// without any lane movement.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <type_traits>

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
// pool_q: grid (n_b, 1, B * head groups), 256 threads.  A thread owns one
// 16-byte column chunk (8 values of one head) and sums half of the block's
// rows; the two halves are added in a fixed order.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void pool_q_kernel(Shape s, const uint16_t* __restrict__ q, Workspace ws) {
  constexpr int CPH = D / 8;          // chunks per head row
  constexpr int HG = 128 / CPH;       // heads per workgroup
  constexpr int CHUNKS = HG * CPH;    // 128 chunks
  constexpr int RPS = 32;             // rows per half
  static_assert(CHUNKS * 2 == 256, "two row halves of 128 chunks");
  __shared__ float part[CHUNKS * 8];

  const int j = blockIdx.x;
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

  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.0f;
  const int r0 = j * kBlock + half * RPS;
  const int rend = min(s.N, r0 + RPS);
  if (active && r0 < rend) {
    const uint16_t* p = q + (long long)b * s.isb + (long long)h * s.ish + d0 + (long long)r0 * s.ist;
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
    float* dst = ws.qbar + (bh * s.nb + j) * D + d0;
    reinterpret_cast<float4*>(dst)[0] = make_float4(m[0], m[1], m[2], m[3]);
    reinterpret_cast<float4*>(dst)[1] = make_float4(m[4], m[5], m[6], m[7]);
  }
}

// Position of key r (0..31 within a half tile) in the packed V^T order.
__device__ __forceinline__ int v_slot(int r) {
  return (r & 16) ? 8 * ((r - 16) >> 2) + 4 + (r & 3) : 8 * (r >> 2) + (r & 3);
}
// Key held in packed V^T position 8 g + e.
__device__ __forceinline__ int v_key(int g, int e) { return (e < 4) ? 4 * g + e : 16 + 4 * g + (e - 4); }

// ---------------------------------------------------------------------------
// pack_kv: grid (n_bp, H, B), 256 threads.  Stages the block's K and V rows
// (zero past N) in LDS, writes the fp32 means Kbar, Vbar (sequential row
// sums), the packed half tiles of K and V^T, and the bf16 centroids into
// their packed centroid half tile (block j is centroid row j % 32 of centroid
// half tile j / 32).  Blocks j >= n_b only zero their centroid rows.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void pack_kv_kernel(Shape s, const uint16_t* __restrict__ k,
                                                      const uint16_t* __restrict__ v, Workspace ws) {
  constexpr int NS = D / 32;
  constexpr int CPR = D / 8;
  constexpr int LS = D + 8;  // LDS row stride (bf16)
  constexpr int HT = 32 * D; // elements of one packed half tile
  __shared__ __attribute__((aligned(16))) uint16_t Kl[64 * LS];
  __shared__ __attribute__((aligned(16))) uint16_t Vl[64 * LS];

  const int j = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const long long bh = (long long)b * s.H + h;
  const int tid = threadIdx.x;
  const int J = j >> 5, r = j & 31;  // centroid half tile and row
  uint16_t* kc = ws.kbp + (bh * (s.nbp / 32) + J) * HT;
  uint16_t* vc = ws.vbp + (bh * (s.nbp / 32) + J) * HT;
  const int ckt = r >> 4, cl16 = r & 15;
  auto kc_index = [&](int d) {
    const int ss = d >> 5, g = (d & 31) >> 3, e = d & 7;
    return ((ckt * NS + ss) * 64 + 16 * g + cl16) * 8 + e;
  };

  if (j >= s.nb) {
    if (tid < D) {
      kc[kc_index(tid)] = 0;
      vc[tid * 32 + v_slot(r)] = 0;
    }
    return;
  }

  const int n = min(kBlock, s.N - j * kBlock);
  const long long base = (long long)b * s.isb + (long long)h * s.ish + (long long)j * kBlock * s.ist;
#pragma unroll
  for (int i = 0; i < CPR / 4; ++i) {
    const int id = tid + 256 * i;
    const int row = id / CPR, col = id % CPR;
    uint4 xk = make_uint4(0, 0, 0, 0), xv = make_uint4(0, 0, 0, 0);
    if (row < n) {
      xk = *reinterpret_cast<const uint4*>(k + base + (long long)row * s.ist + col * 8);
      xv = *reinterpret_cast<const uint4*>(v + base + (long long)row * s.ist + col * 8);
    }
    *reinterpret_cast<uint4*>(Kl + row * LS + col * 8) = xk;
    *reinterpret_cast<uint4*>(Vl + row * LS + col * 8) = xv;
  }
  __syncthreads();

  if (tid < 2 * D) {
    const uint16_t* src = (tid < D) ? Kl : Vl;
    const int d = tid % D;
    float sum = 0.0f;
    for (int row = 0; row < n; ++row) sum += bf16_bits_to_f32(src[row * LS + d]);
    const float mean = sum / (float)n;
    if (tid < D) {
      ws.kbar[(bh * s.nb + j) * D + d] = mean;
      kc[kc_index(d)] = (uint16_t)f32_to_bf16_bits(mean);
    } else {
      ws.vbar[(bh * s.nb + j) * D + d] = mean;
      vc[d * 32 + v_slot(r)] = (uint16_t)f32_to_bf16_bits(mean);
    }
  }

  uint16_t* kp = ws.kp + (bh * s.nb + j) * (2LL * HT);
  uint16_t* vp = ws.vp + (bh * s.nb + j) * (2LL * HT);
#pragma unroll
  for (int i = 0; i < CPR / 4; ++i) {
    const int o = tid + 256 * i;  // output 16-byte chunk, 64 * CPR of them
    {
      const int ht = o / (128 * NS), rem = o % (128 * NS);
      const int kt = rem / (64 * NS), rem2 = rem % (64 * NS);
      const int ss = rem2 / 64, lane = rem2 % 64;
      const int row = 32 * ht + 16 * kt + (lane & 15);
      const int d0 = 32 * ss + 8 * (lane >> 4);
      *reinterpret_cast<uint4*>(kp + (long long)o * 8) = *reinterpret_cast<const uint4*>(Kl + row * LS + d0);
    }
    {
      const int ht = o / (4 * D), rem = o % (4 * D);
      const int d = rem >> 2, g = rem & 3;
      uint32_t w[4];
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) {
        const uint32_t lo = Vl[(32 * ht + v_key(g, 2 * e2)) * LS + d];
        const uint32_t hi = Vl[(32 * ht + v_key(g, 2 * e2 + 1)) * LS + d];
        w[e2] = lo | (hi << 16);
      }
      *reinterpret_cast<uint4*>(vp + (long long)o * 8) = make_uint4(w[0], w[1], w[2], w[3]);
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
// attend: one wave per (b, h, query block); grid B*H*n_b in an XCD-aware
// order.  The wave keeps its 64 query rows as MFMA B operands (Q^T) in
// registers and walks half tiles of 32 keys: first the two halves of every
// listed key block, then the centroid half tiles that hold at least one
// unselected block.  Per half tile:
//   S^T[key][q] = K Q^T            8 v_mfma_f32_16x16x32_bf16 per 16 queries
//   online softmax per query       in-lane over 8 keys + 2 cross-lane steps
//   O^T[d][q] += V^T P^T           8 MFMAs per 16 queries
// Operands come from the packed buffers in a double-buffered register
// pipeline (the next half tile is loaded while the current one computes).
// ---------------------------------------------------------------------------
template <int D>
__device__ __forceinline__ void load_k(uint4 (&kf)[2][D / 32], const uint16_t* __restrict__ base, int lane) {
  constexpr int NS = D / 32;
#pragma unroll
  for (int kt = 0; kt < 2; ++kt)
#pragma unroll
    for (int ss = 0; ss < NS; ++ss)
      kf[kt][ss] = *reinterpret_cast<const uint4*>(base + ((kt * NS + ss) * 64 + lane) * 8);
}

template <int D>
__device__ __forceinline__ void load_v(uint4 (&vf)[D / 16], const uint16_t* __restrict__ base, int lane) {
  const int l16 = lane & 15, g = lane >> 4;
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) vf[dt] = *reinterpret_cast<const uint4*>(base + (16 * dt + l16) * 32 + 8 * g);
}

template <int D>
__global__ __launch_bounds__(64) void attend_kernel(Shape s, const uint16_t* __restrict__ q,
                                                    uint16_t* __restrict__ out, Workspace ws) {
  constexpr int NS = D / 32, NDT = D / 16, HT = 32 * D;
  __shared__ uint32_t selbits[SA_MAX_BLOCKS / 32];
  __shared__ int ctile[SA_MAX_BLOCKS / 32];

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
  const int lane = threadIdx.x, l16 = lane & 15, g = lane >> 4;

  // Q^T fragments: query a*64 + 16 qt + l16, d = 32 ss + 8 g + e.
  const long long in_base = (long long)b * s.isb + (long long)h * s.ish;
  bf16x8 qf[4][NS];
#pragma unroll
  for (int qt = 0; qt < 4; ++qt) {
    const int row = a * kBlock + 16 * qt + l16;
#pragma unroll
    for (int ss = 0; ss < NS; ++ss) {
      uint4 x = make_uint4(0, 0, 0, 0);
      if (row < s.N) x = *reinterpret_cast<const uint4*>(q + in_base + (long long)row * s.ist + 32 * ss + 8 * g);
      qf[qt][ss] = __builtin_bit_cast(bf16x8, x);
    }
  }

  int count = nb;
  if (!s.dense) count = min(max(ws.counts[bh * nb + a], 0), nb);
  const int* list = ws.lists + (bh * nb + a) * (long long)nb;
  const int nct = s.nbp / 32;  // centroid half tiles
  int nc = 0;                  // centroid half tiles to visit
  if (!s.dense && s.centroid && count < nb) {
    for (int i = lane; i < nct; i += 64) selbits[i] = 0u;
    __syncthreads();
    for (int i = lane; i < count; i += 64) {
      const int c = list[i];
      if (c >= 0 && c < nb) atomicOr(&selbits[c >> 5], 1u << (c & 31));
    }
    __syncthreads();
    // keep the centroid half tiles with at least one unselected, existing block
    int base = 0;
    for (int i0 = 0; i0 < nct; i0 += 64) {
      const int i = i0 + lane;
      bool keep = false;
      if (i < nct) {
        const int valid = min(32, nb - 32 * i);
        const uint32_t vmask = valid >= 32 ? 0xffffffffu : ((1u << max(valid, 0)) - 1u);
        keep = (~selbits[i] & vmask) != 0u;
      }
      const uint64_t m = __ballot(keep);
      if (keep) ctile[base + __popcll(m & ((lane == 0) ? 0ull : (~0ull >> (64 - lane))))] = i;
      base += __popcll(m);
    }
    nc = base;
    __syncthreads();
  }
  const int T = 2 * count + nc;

  // Half tile t: pointers into the packed buffers and the additive per-key
  // term in the log2 domain (0 for a valid key of an exact block, log2(n_c)
  // or 0 for an unselected centroid, -inf for keys past N, selected
  // centroids and centroid rows past n_b), the same for every query.  Both
  // are computed without branches so that the loop body stays one block.
  const uint16_t* kp_bh = ws.kp + bh * nb * 2LL * HT;
  const uint16_t* vp_bh = ws.vp + bh * nb * 2LL * HT;
  const uint16_t* kc_bh = ws.kbp + bh * nct * (long long)HT;
  const uint16_t* vc_bh = ws.vbp + bh * nct * (long long)HT;
  const int nexact = 2 * count;
  auto tile_off = [&](int t, bool& centroid, int& c) {
    centroid = t >= nexact;
    const int ce = s.dense ? (t >> 1) : list[min(t, nexact - 1) >> 1];
    const int ci = ctile[max(t - nexact, 0)];
    c = centroid ? ci : ((ce >= 0 && ce < nb) ? ce : -1);
    const long long e_off = ((long long)max(c, 0) * 2 + (t & 1)) * HT;
    const long long c_off = (long long)ci * HT;
    return centroid ? c_off : e_off;
  };
  auto tile_ptrs = [&](int t, const uint16_t*& kb, const uint16_t*& vb) {
    bool centroid;
    int c;
    const long long off = tile_off(t, centroid, c);
    kb = (centroid ? kc_bh : kp_bh) + off;
    vb = (centroid ? vc_bh : vp_bh) + off;
  };
  auto key_bias = [&](int t, float (&kb)[2][4]) {
    bool centroid;
    int c;
    tile_off(t, centroid, c);
    // exact: valid keys 32*(t&1) + r < nvalid; centroid: r unselected and 32c + r < nb
    const int nvalid = (c >= 0) ? min(kBlock, s.N - c * kBlock) : 0;
    const uint32_t sel = centroid ? selbits[c] : 0u;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * kt + 4 * g + i;
        const int cc = 32 * c + r;
        const bool ok_e = 32 * (t & 1) + r < nvalid;
        const bool ok_c = cc < nb && !((sel >> r) & 1u);
        const float bc = (cc == nb - 1) ? s.bias_tail : s.bias_full;
        kb[kt][i] = centroid ? (ok_c ? bc : -INFINITY) : (ok_e ? 0.0f : -INFINITY);
      }
  };
  // Q K^T of one half tile: the d steps are the outer loop so that eight
  // independent accumulators separate two MFMAs into the same one.
  auto qk = [&](const uint4 (&kf)[2][NS], f32x4 (&st)[4][2]) {
#pragma unroll
    for (int qt = 0; qt < 4; ++qt)
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) st[qt][kt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ss = 0; ss < NS; ++ss)
#pragma unroll
      for (int qt = 0; qt < 4; ++qt)
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
          st[qt][kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kf[kt][ss]),
                                                              qf[qt][ss], st[qt][kt], 0, 0, 0);
  };

  // Softmax reference.  Every logit x of query row q is scored as
  // p = exp2(x - mref[q]) with a fixed mref[q]: the exact maximum over the
  // row's first half tile plus 32 (log2 units).  Terms of that tile then lie
  // below 2^-32 and the row's largest term is at least 2^-32, far inside the
  // fp32 / bf16 exponent range, and no running maximum or rescaling of the
  // accumulators is needed.  The ratio acc / l is independent of mref, so
  // this is the same softmax up to rounding.  Should a later term exceed
  // mref by so much that the row sum leaves [0, 2^100] (or is not finite),
  // the query block is recomputed with the exact row maxima from a
  // Q K^T-only pass.
  const bf16x8 ones = __builtin_bit_cast(bf16x8, make_uint4(0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u));
  f32x4 acc[4][NDT], lacc[4];
  auto zero_acc = [&]() {
#pragma unroll
    for (int qt = 0; qt < 4; ++qt) {
      lacc[qt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) acc[qt][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  };
  // Row maxima of one half tile's logits (used for the reference only).
  auto row_max = [&](const f32x4 (&st)[4][2], int tt, float (&mx)[4]) {
    float kb[2][4];
    key_bias(tt, kb);
#pragma unroll
    for (int qt = 0; qt < 4; ++qt) {
      float m = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) m = fmaxf(m, fmaf(st[qt][kt][i], s.c1, kb[kt][i]));
      const auto p16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(m), __float_as_uint(m), false, false);
      m = fmaxf(__uint_as_float(p16[0]), __uint_as_float(p16[1]));
      const auto p32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m), false, false);
      mx[qt] = fmaxf(__uint_as_float(p32[0]), __uint_as_float(p32[1]));
    }
  };

  // Pipeline state entering step t: S^T of t in the current st buffer, K of
  // t+1 in kf, V of t in vf.  Step t issues Q K^T of t+1 (MFMA) and the
  // exponentials of t (VALU) in one basic block, so that the scheduler can
  // interleave them and the MFMA pipe of this single wave works while the
  // VALU does; P V of t and the row sums (an MFMA against ones) follow.  K of
  // t+2 and V of t+1 are requested as soon as their registers are free.
  // Indices past the end are clamped (a redundant last Q K^T).
  uint4 kf[2][NS], vf[NDT];
  f32x4 stA[4][2], stB[4][2];
  auto prologue = [&]() {
    const uint16_t *kb0, *vb0;
    tile_ptrs(0, kb0, vb0);
    load_k<D>(kf, kb0, lane);
    load_v<D>(vf, vb0, lane);
    qk(kf, stA);
    tile_ptrs(min(1, T - 1), kb0, vb0);
    load_k<D>(kf, kb0, lane);
  };
  auto step = [&](auto plain_c, int t, const f32x4 (&st)[4][2], f32x4 (&st_next)[4][2],
                  const float (&mref)[4]) {
    constexpr bool plain = decltype(plain_c)::value;
    const uint16_t *kb2, *vb2, *kb1, *vb1;
    tile_ptrs(min(t + 2, T - 1), kb2, vb2);
    tile_ptrs(min(t + 1, T - 1), kb1, vb1);
    float kb[2][4];
    if constexpr (!plain) key_bias(t, kb);
    qk(kf, st_next);
    load_k<D>(kf, kb2, lane);
    bf16x8 pb[4];
#pragma unroll
    for (int qt = 0; qt < 4; ++qt)
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float bias = plain ? -mref[qt] : kb[kt][i] - mref[qt];
          pb[qt][kt * 4 + i] = (__bf16)__builtin_amdgcn_exp2f(fmaf(st[qt][kt][i], s.c1, bias));
        }
#pragma unroll
    for (int qt = 0; qt < 4; ++qt) {
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
        acc[qt][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, vf[dt]), pb[qt],
                                                             acc[qt][dt], 0, 0, 0);
      lacc[qt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pb[qt], lacc[qt], 0, 0, 0);
    }
    load_v<D>(vf, vb1, lane);
  };
  // Exact half tiles come first (lists are ascending) and only a ragged
  // last block and the centroid tiles need per-key terms, so the plain tiles
  // are a prefix of the sequence and each of the two loops below runs one
  // step variant.
  int nplain = nexact;
  if (nexact > 0 && s.tail < kBlock) {
    const int clast = s.dense ? nb - 1 : list[count - 1];
    if (clast == nb - 1) nplain = nexact - 2;
  }
  auto run = [&](const float (&mref)[4]) {
    int t = 0;
    for (; t + 1 < nplain; t += 2) {
      step(std::true_type{}, t, stA, stB, mref);
      step(std::true_type{}, t + 1, stB, stA, mref);
    }
    if (t < nplain) {
      step(std::true_type{}, t, stA, stB, mref);
      ++t;
#pragma unroll
      for (int qt = 0; qt < 4; ++qt)
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) stA[qt][kt] = stB[qt][kt];
    }
    for (; t + 1 < T; t += 2) {
      step(std::false_type{}, t, stA, stB, mref);
      step(std::false_type{}, t + 1, stB, stA, mref);
    }
    if (t < T) step(std::false_type{}, t, stA, stB, mref);
  };

  float mref[4] = {0.f, 0.f, 0.f, 0.f};
  zero_acc();
  if (T > 0) {
    prologue();
    float mx[4];
    row_max(stA, 0, mx);
#pragma unroll
    for (int qt = 0; qt < 4; ++qt) mref[qt] = (mx[qt] == -INFINITY) ? 0.0f : mx[qt] + 32.0f;
    run(mref);
    bool bad = false;
#pragma unroll
    for (int qt = 0; qt < 4; ++qt) bad |= !(lacc[qt][0] <= 0x1p100f);
    if (__ballot(bad)) {
      // Exact row maxima over every half tile, then the same computation.
      float mtrue[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
      for (int t = 0; t < T; ++t) {
        const uint16_t *kb0, *vb0;
        tile_ptrs(t, kb0, vb0);
        load_k<D>(kf, kb0, lane);
        qk(kf, stA);
        float mx2[4];
        row_max(stA, t, mx2);
#pragma unroll
        for (int qt = 0; qt < 4; ++qt) mtrue[qt] = fmaxf(mtrue[qt], mx2[qt]);
      }
#pragma unroll
      for (int qt = 0; qt < 4; ++qt) mref[qt] = (mtrue[qt] == -INFINITY) ? 0.0f : mtrue[qt];
      zero_acc();
      prologue();
      run(mref);
    }
  }

  const long long out_base = (long long)b * s.osb + (long long)h * s.osh;
#pragma unroll
  for (int qt = 0; qt < 4; ++qt) {
    const float l = lacc[qt][0];  // every row of the ones product holds the column sum
    const float inv = (l > 0.0f) ? 1.0f / l : 0.0f;
    const int row = a * kBlock + 16 * qt + l16;
    if (row < s.N) {
      uint16_t* o = out + out_base + (long long)row * s.ost;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        uint2 w2;
        w2.x = f32_to_bf16_bits(acc[qt][dt][0] * inv) | (f32_to_bf16_bits(acc[qt][dt][1] * inv) << 16);
        w2.y = f32_to_bf16_bits(acc[qt][dt][2] * inv) | (f32_to_bf16_bits(acc[qt][dt][3] * inv) << 16);
        *reinterpret_cast<uint2*>(o + 16 * dt + 4 * g) = w2;
      }
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

hipError_t launch_pool_q(const Shape& s, const void* q, const Workspace& ws, hipStream_t stream) {
  const int hg = 128 / (s.D / 8);
  dim3 grid(s.nb, 1, s.B * ((s.H + hg - 1) / hg));
  const auto* qq = static_cast<const uint16_t*>(q);
  if (s.D == 128)
    hipLaunchKernelGGL(pool_q_kernel<128>, grid, dim3(256), 0, stream, s, qq, ws);
  else
    hipLaunchKernelGGL(pool_q_kernel<64>, grid, dim3(256), 0, stream, s, qq, ws);
  return hipGetLastError();
}

hipError_t launch_pack_kv(const Shape& s, const void* k, const void* v, const Workspace& ws,
                          hipStream_t stream) {
  dim3 grid(s.nbp, s.H, s.B);
  const auto* kk = static_cast<const uint16_t*>(k);
  const auto* vv = static_cast<const uint16_t*>(v);
  if (s.D == 128)
    hipLaunchKernelGGL(pack_kv_kernel<128>, grid, dim3(256), 0, stream, s, kk, vv, ws);
  else
    hipLaunchKernelGGL(pack_kv_kernel<64>, grid, dim3(256), 0, stream, s, kk, vv, ws);
  return hipGetLastError();
}

hipError_t launch_select(const Shape& s, const Workspace& ws, hipStream_t stream) {
  const bool big = s.nb > 1536;
  if (s.D == 128) return big ? launch_select_t<128, 8>(s, ws, stream) : launch_select_t<128, 16>(s, ws, stream);
  return big ? launch_select_t<64, 8>(s, ws, stream) : launch_select_t<64, 16>(s, ws, stream);
}

hipError_t launch_attend(const Shape& s, const void* q, void* out, const Workspace& ws, hipStream_t stream) {
  dim3 grid((unsigned)((long long)s.B * s.H * s.nb));
  const auto* qq = static_cast<const uint16_t*>(q);
  auto* oo = static_cast<uint16_t*>(out);
  if (s.D == 128)
    hipLaunchKernelGGL(attend_kernel<128>, grid, dim3(64), 0, stream, s, qq, oo, ws);
  else
    hipLaunchKernelGGL(attend_kernel<64>, grid, dim3(64), 0, stream, s, qq, oo, ws);
  return hipGetLastError();
}

}  // namespace sa
