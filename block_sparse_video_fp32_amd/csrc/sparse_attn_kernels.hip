// gfx950 kernels of routed block-sparse attention.
//
//   pool_q_kernel  per-64-row-block means of Q in FP32 (HBM-bound stream;
//                  Star7 README, 工作原理 > Sol: Q64/K64 blocks).
//   anchor_kernel  Spark-Reweight only: the mean of a head's video query
//                  rows, from the block means (Spark-H3 news, Spark-Reweight).
//   pack_kv_kernel per block of one head: the FP32 means of K and V (the
//                  centroids; Spark-H3 news, Spark-Reweight: mean-pooled K/V
//                  summaries), plus K, V^T and the centroids rewritten in the
//                  register order of the attend kernel's MFMA operands, so
//                  that every operand load there is one coalesced 1 KB read;
//                  optionally the anchor-weighted centroids and their bias
//                  (Spark-Reweight) or the INT8 residual codes of K
//                  (thakicloud accel-stack post, measured results).
//   select_kernel  fp32 block scores Qbar_a . Kbar_c for a group of query
//                  blocks against every key block, then per query block
//                  (one wave each) the threshold mean + tau * std (two-pass,
//                  population) or an exact radix top-K, the prefix sink, and
//                  ballot compaction into an ascending index list
//                  (thakicloud accel-stack post, 이 기술은 무엇인가; Spark-H3
//                  news, 워크플로: topk_ratio).
//   attend_kernel  one workgroup per pair of neighbouring query blocks of
//                  one (b, h): exact bf16 attention on MFMA over the key
//                  blocks either block listed, K and V^T staged in LDS by
//                  direct global->LDS copies, then one centroid logit per
//                  unselected block with the log-mass bias, all merged into
//                  the same FP32 softmax (Star7 README, Sol: missed blocks
//                  contribute through a K/V centroid in the same FP32 online
//                  softmax).  Template instances add the reweight bias and
//                  INT8 QK^T without touching the default instance.
//   pair_order_kernel  the order in which the attend workgroups of one
//                  (b, h) take its pairs: longest lists first, so that the
//                  shortest run last and the launch drains sooner.
//   head_order_kernel  which heads each XCD's run of attend workgroups
//                  serves: dealt in snake order of decreasing total list
//                  length, so that the XCDs finish together.
//
// Packed operand layouts (bf16).  A "half tile" is 32 keys x D, stored as
// D/16 blocks of 64 lanes x 8 elements (1 KB at D = 128); kappa(r) is r with
// bits 3 and 4 swapped.
//   K half tile:   element ((m*64 + l)*8 + e) holds
//                  K[kappa(l % 32)][16 m + 8 (l / 32) + e]
//   V^T half tile: element ((m*64 + l)*8 + e), m = 2 dt + j, holds
//                  V[16 (e / 4) + 8 j + 4 (l / 32) + e % 4][32 dt + l % 32]
// Block m of K is lane l's A operand of the m-th v_mfma_f32_32x32x16_bf16 of
// S^T = K Q^T; block m of V^T is the A operand of k-step j of O^T = V^T P^T
// for d tile dt.  The key order is the one in which the S^T accumulator
// holds the keys, so P^T goes from accumulator to B operand without any lane
// movement, and each block is one linear 1 KB copy into LDS.
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
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// 16-byte store that bypasses cache retention: the packed tiles are written
// once here and read back by later launches from HBM either way.
__device__ __forceinline__ void store_stream(void* dst, uint32_t x, uint32_t y, uint32_t z, uint32_t w) {
  __builtin_nontemporal_store(u32x4{x, y, z, w}, reinterpret_cast<u32x4*>(dst));
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// Row of the caller's Q (side 0) or K and V (side 1) behind row r of (b, h)
// on the path: with Spark-Reblock orders in use, row rb_r0 + i is the
// caller's row rb_r0 + order[i] of the partition's final order (the prefix
// blocks stay; in the shared layout both sides use the query partition);
// otherwise r itself.
__device__ __forceinline__ int src_row(const Shape& s, const Workspace& ws, int side, long long bh, int r) {
  if (!s.permuted || r < s.rb_r0) return r;
  const long long p = (long long)(s.rb_kv_own ? side : 0) * s.B * s.H + bh;
  return s.rb_r0 + ws.rb_ord[((long long)(s.rb_levels & 1) * s.rb_P + p) * s.rb_n + (r - s.rb_r0)];
}

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
    const uint16_t* p = q + (long long)b * s.isb + (long long)h * s.ish + d0;
    const int n = rend - r0;
    int r = 0;
    for (; r + 8 <= n; r += 8) {
      uint4 x[8];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        x[u] = *reinterpret_cast<const uint4*>(p + (long long)src_row(s, ws, 0, bh, r0 + r + u) * s.ist);
#pragma unroll
      for (int u = 0; u < 8; ++u)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] += lane_bf16(x[u], e);
    }
    for (; r < n; ++r) {
      const uint4 x = *reinterpret_cast<const uint4*>(p + (long long)src_row(s, ws, 0, bh, r0 + r) * s.ist);
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

// ---------------------------------------------------------------------------
// anchor: grid (H, B), 256 threads.  The reweight anchor of one head, the
// mean of the query rows first .. N - 1, first = prefix_len (0 when no video
// rows would remain): every block that starts at or after first adds
// n_a * Qbar_a, and the rows of a block that straddles first are read from Q.
// (Spark-H3 news, Spark-Reweight: one anchor per head from the video query
// rows.)
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void anchor_kernel(Shape s, const uint16_t* __restrict__ q, Workspace ws) {
  constexpr int G = 256 / D;  // row groups
  constexpr int U = 4;        // independent partial sums per thread
  __shared__ float part[256];
  const int h = blockIdx.x, b = blockIdx.y;
  const long long bh = (long long)b * s.H + h;
  const int tid = threadIdx.x, d = tid % D, g = tid / D;
  const int first = (s.prefix_len > 0 && s.prefix_len < s.N) ? s.prefix_len : 0;
  const int af = (first + kBlock - 1) / kBlock;  // first block wholly at or after first
  float acc[U];
#pragma unroll
  for (int u = 0; u < U; ++u) acc[u] = 0.0f;
  const float* qb = ws.qbar + bh * s.nb * D + d;
  int a = af + g;
  for (; a + (U - 1) * G < s.nb; a += U * G) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = a + u * G;
      acc[u] += (float)min(kBlock, s.N - c * kBlock) * qb[(long long)c * D];
    }
  }
  for (; a < s.nb; a += G) acc[0] += (float)min(kBlock, s.N - a * kBlock) * qb[(long long)a * D];
  const uint16_t* qp = q + (long long)b * s.isb + (long long)h * s.ish + d;
  const int rend = min(af * kBlock, s.N);
  for (int r = first + g; r < rend; r += G) acc[1] += bf16_bits_to_f32(qp[(long long)r * s.ist]);
  part[tid] = (acc[0] + acc[1]) + (acc[2] + acc[3]);
  __syncthreads();
  if (tid < D) {
    float t = 0.0f;
#pragma unroll
    for (int k = 0; k < G; ++k) t += part[k * D + tid];
    ws.anchor[bh * D + tid] = t / (float)(s.N - first);
  }
}

// Packed half-tile orders (see the file header): kappa(r) swaps bits 3 and 4
// of a key index r (an involution).
__device__ __forceinline__ int kappa(int r) { return (r & 7) | ((r & 8) << 1) | ((r & 16) >> 1); }
// Key held in element e of lane l's chunk of a V^T block of k-step j.
__device__ __forceinline__ int vt_key(int j, int l, int e) {
  return 16 * (e >> 2) + 8 * j + 4 * (l >> 5) + (e & 3);
}

// ---------------------------------------------------------------------------
// pack_kv: grid (n_bp, H, B), 256 threads.  Stages the block's K and V rows
// (zero past N) in LDS, writes the fp32 means Kbar, Vbar (sequential row
// sums), the packed half tiles of K and V^T, and the bf16 centroids into
// their packed centroid half tile (block j is centroid row j % 32 of centroid
// half tile j / 32).  In reweight mode the packed centroids are the
// anchor-weighted summaries and the block's bias goes to cbias; the fp32
// means are still written (routing uses them).  Blocks j >= n_b only zero
// their centroid rows (and bias).
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void pack_kv_kernel(Shape s, const uint16_t* __restrict__ k,
                                                      const uint16_t* __restrict__ v, Workspace ws) {
  constexpr int CPR = D / 8;
  constexpr int LS = D + 8;  // LDS row stride (bf16)
  constexpr int HT = 32 * D; // elements of one packed half tile
  __shared__ __attribute__((aligned(16))) uint16_t Kl[64 * LS];
  __shared__ __attribute__((aligned(16))) uint16_t Vl[64 * LS];
  __shared__ float al[D];   // reweight anchor
  __shared__ float wl[64];  // reweight row weights
  __shared__ float red[8];
  __shared__ float kbl[D];  // INT8 QK^T base row (bf16 values)

  const int j = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const long long bh = (long long)b * s.H + h;
  const int tid = threadIdx.x;
  const int J = j >> 5, r = j & 31;  // centroid half tile and row
  uint16_t* kc = ws.kbp + (bh * (s.nbp / 32) + J) * HT;
  uint16_t* vc = ws.vbp + (bh * (s.nbp / 32) + J) * HT;
  // element of centroid row r, dimension d, in the packed K and V^T orders
  auto kc_index = [&](int d) { return (((d >> 4) * 64 + kappa(r) + 32 * ((d >> 3) & 1)) * 8) + (d & 7); };
  auto vc_index = [&](int d) {
    const int m = 2 * (d >> 5) + ((r >> 3) & 1), l = (d & 31) + 32 * ((r >> 2) & 1);
    return (m * 64 + l) * 8 + 4 * (r >> 4) + (r & 3);
  };

  if (j >= s.nb) {
    if (tid < D) {
      kc[kc_index(tid)] = 0;
      vc[vc_index(tid)] = 0;
    }
    if (s.reweight && tid == 0) ws.cbias[bh * s.nbp + j] = 0.0f;
    return;
  }
  if (s.reweight && tid < D) al[tid] = ws.anchor[bh * D + tid];

  const int n = min(kBlock, s.N - j * kBlock);
  const long long base = (long long)b * s.isb + (long long)h * s.ish;
#pragma unroll
  for (int i = 0; i < CPR / 4; ++i) {
    const int id = tid + 256 * i;
    const int row = id / CPR, col = id % CPR;
    uint4 xk = make_uint4(0, 0, 0, 0), xv = make_uint4(0, 0, 0, 0);
    if (row < n) {
      const long long off = base + (long long)src_row(s, ws, 1, bh, j * kBlock + row) * s.ist + col * 8;
      xk = *reinterpret_cast<const uint4*>(k + off);
      xv = *reinterpret_cast<const uint4*>(v + off);
    }
    *reinterpret_cast<uint4*>(Kl + row * LS + col * 8) = xk;
    *reinterpret_cast<uint4*>(Vl + row * LS + col * 8) = xv;
  }
  __syncthreads();

  // Spark-Reweight (Spark-H3 news): row weights w = softmax(x) with
  // x_r = scale * anchor . k_r over the block's rows, in log2 units.
  // Four threads per row, each over every fourth pair of dimensions.
  if (s.reweight) {
    const int row = tid >> 2, p4 = tid & 3;
    const uint32_t* kr = reinterpret_cast<const uint32_t*>(Kl + row * LS);
    float xr = 0.0f;
#pragma unroll
    for (int i = 0; i < D / 8; ++i) {
      const int pr = p4 + 4 * i;
      const uint32_t two = kr[pr];
      xr += al[2 * pr] * bf16_bits_to_f32(two & 0xffffu) + al[2 * pr + 1] * bf16_bits_to_f32(two >> 16);
    }
    xr += __shfl_xor(xr, 1);
    xr += __shfl_xor(xr, 2);
    if (p4 == 0) wl[row] = xr * s.c1;
    __syncthreads();
    if (tid < 64) {
      const float xv = tid < n ? wl[tid] : -INFINITY;
      float m = xv;
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
      const float e = tid < n ? exp2f(xv - m) : 0.0f;
      float z = e;
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) z += __shfl_xor(z, o);
      wl[tid] = e / z;
      if (tid == 0) {
        red[0] = m;
        red[1] = z;
      }
    }
    __syncthreads();
  }

  // Block means (fp32, sequential over rows); with reweight the packed
  // centroids hold the weighted sums Ktilde, Vtilde instead.
  float kdot = 0.0f;  // anchor . Ktilde, this thread's dimension
  if (tid < 2 * D) {
    const uint16_t* src = (tid < D) ? Kl : Vl;
    const int d = tid % D;
    float sum = 0.0f, wsum = 0.0f;
    if (s.reweight) {
      for (int row = 0; row < n; ++row) {
        const float x = bf16_bits_to_f32(src[row * LS + d]);
        sum += x;
        wsum += wl[row] * x;
      }
    } else {
      for (int row = 0; row < n; ++row) sum += bf16_bits_to_f32(src[row * LS + d]);
    }
    const float mean = sum / (float)n;
    const float cval = s.reweight ? wsum : mean;
    if (tid < D) {
      ws.kbar[(bh * s.nb + j) * D + d] = mean;
      kc[kc_index(d)] = (uint16_t)f32_to_bf16_bits(cval);
      kdot = al[d] * wsum;
      if (s.int8) {
        const uint32_t bb = f32_to_bf16_bits(mean);
        ws.kbase[(bh * s.nb + j) * (D + 8) + d] = (uint16_t)bb;
        kbl[d] = bf16_bits_to_f32(bb);
      }
    } else {
      ws.vbar[(bh * s.nb + j) * D + d] = mean;
      vc[vc_index(d)] = (uint16_t)f32_to_bf16_bits(cval);
    }
  }
  // bias = logsumexp(x) - scale * anchor . Ktilde, in log2 units.
  if (s.reweight) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) kdot += __shfl_xor(kdot, o);
    if ((tid & 63) == 0 && tid < D) red[2 + (tid >> 6)] = kdot;
    __syncthreads();
    if (tid == 0) {
      float ak = 0.0f;
#pragma unroll
      for (int k = 0; k < D / 64; ++k) ak += red[2 + k];
      ws.cbias[bh * s.nbp + j] = red[0] + log2f(red[1]) - s.c1 * ak;
    }
  }

  // INT8 QK^T (thakicloud accel-stack post, measured results): residual
  // codes of the keys about the bf16 base row, one scale per block, in the
  // A-operand order of v_mfma_i32_32x32x32_i8; the bf16 K tiles are not
  // needed then.
  if (s.int8) {
    __syncthreads();
    float mx = 0.0f;
    for (int e = tid; e < n * D; e += 256) {
      const int row = e / D, d = e % D;
      mx = fmaxf(mx, fabsf(bf16_bits_to_f32(Kl[row * LS + d]) - kbl[d]));
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
    if ((tid & 63) == 0) red[4 + (tid >> 6)] = mx;
    __syncthreads();
    const float sc = fmaxf(fmaxf(red[4], red[5]), fmaxf(red[6], red[7])) / 127.0f;
    uint16_t* rec = ws.kbase + (bh * s.nb + j) * (D + 8);
    if (tid == 0) *reinterpret_cast<uint4*>(rec + D) = make_uint4(__float_as_uint(sc), 0u, 0u, 0u);
    uint8_t* k8 = ws.k8 + (bh * s.nb + j) * (64LL * D);
    for (int o = tid; o < 4 * D; o += 256) {  // 16-byte chunks, 2 * (D/32) * 64 of them
      const int ht = o / (2 * D), t = (o / 64) % (D / 32), l = o % 64;
      const int row = 32 * ht + kappa(l & 31);
      uint32_t wd[4] = {0u, 0u, 0u, 0u};
      if (row < n && sc > 0.0f) {
#pragma unroll
        for (int jj = 0; jj < 16; ++jj) {
          const int d = 32 * t + 16 * (jj >> 3) + 8 * (l >> 5) + (jj & 7);
          const float x = bf16_bits_to_f32(Kl[row * LS + d]) - kbl[d];
          const int code = (int)fminf(fmaxf(rintf(x / sc), -127.0f), 127.0f);
          wd[jj >> 2] |= ((uint32_t)code & 0xffu) << (8 * (jj & 3));
        }
      }
      store_stream(k8 + (long long)o * 16, wd[0], wd[1], wd[2], wd[3]);
    }
  }

  uint16_t* kp = ws.kp + (bh * s.nb + j) * (2LL * HT);
  uint16_t* vp = ws.vp + (bh * s.nb + j) * (2LL * HT);
#pragma unroll
  for (int i = 0; i < CPR / 4; ++i) {
    const int o = tid + 256 * i;  // output 16-byte chunk, 64 * CPR of them
    const int ht = o / (64 * (D / 16)), m = (o / 64) % (D / 16), l = o % 64;
    if (!s.int8) {
      // K: chunk (m, l) = K[kappa(l % 32)][16 m + 8 (l / 32) .. +8]
      const int row = 32 * ht + kappa(l & 31);
      const int d0 = 16 * m + 8 * (l >> 5);
      const uint4 t4 = *reinterpret_cast<const uint4*>(Kl + row * LS + d0);
      store_stream(kp + (long long)o * 8, t4.x, t4.y, t4.z, t4.w);
    }
    {
      // V^T: chunk (m = 2 dt + jj, l) = V[vt_key(jj, l, e)][32 dt + l % 32], e = 0..7
      const int d = 32 * (m >> 1) + (l & 31), jj = m & 1;
      uint32_t w[4];
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) {
        const uint32_t lo = Vl[(32 * ht + vt_key(jj, l, 2 * e2)) * LS + d];
        const uint32_t hi = Vl[(32 * ht + vt_key(jj, l, 2 * e2 + 1)) * LS + d];
        w[e2] = lo | (hi << 16);
      }
      store_stream(vp + (long long)o * 8, w[0], w[1], w[2], w[3]);
    }
  }
}

// ---------------------------------------------------------------------------
// select: grid ceil(n_b / 16) * H * B (XCD-grouped by head), 256 threads,
// dynamic LDS.
// Phase 1: S[r][c] = Qbar_(a0+r) . Kbar_c for 16 query blocks and every key
// block, an fp32 GEMM on v_mfma_f32_16x16x4_f32.  Phase 2: wave w routes rows
// 4w .. 4w + 3.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t order_key(float f) {
  if (f == 0.0f) f = 0.0f;  // -0 and +0 rank together
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

template <int D>
__global__ __launch_bounds__(256) void select_kernel(Shape s, Workspace ws) {
  constexpr int R = 16;       // query blocks per workgroup = MFMA rows
  constexpr int RPW = R / 4;  // rows routed per wave
  constexpr int KS = D / 4;   // k-steps of the score GEMM
  extern __shared__ __attribute__((aligned(16))) float sm[];
  float* S = sm;                                     // [R][nb]
  int* hist = reinterpret_cast<int*>(S + R * s.nb);  // [4][256]

  const int nb = s.nb;
  // One-dimensional grid, remapped so that the workgroups of one head run on
  // one XCD (workgroups go to the 8 XCDs round-robin), which then fetches
  // that head's Kbar into its L2 once.
  const int G = gridDim.x, bid = blockIdx.x;
  const int xcd = bid & 7, kx = bid >> 3, qq = G >> 3, rr = G & 7;
  const int lid = (xcd < rr) ? xcd * (qq + 1) + kx : rr * (qq + 1) + (xcd - rr) * qq + kx;
  const int ngroups = (s.nb + R - 1) / R;
  const int a0 = (lid % ngroups) * R;
  const int h = (lid / ngroups) % s.H, b = lid / (ngroups * s.H);
  const long long bh = (long long)b * s.H + h;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int l16 = lane & 15, g = lane >> 4;
  const float* qbar = ws.qbar + bh * nb * D;
  const float* kbar = ws.kbar + bh * nb * D;

  // MFMA operands: lane l holds A = Qbar[a0 + l%16][KS (l/16) + j] and
  // B = Kbar[c + l%16][KS (l/16) + j] for k-step j, so every k-step sums
  // four d values and the steps together cover d once (the summation order
  // differs from a sequential one only by fp32 rounding).
  float qa[KS];
  {
    const int r = a0 + l16;
#pragma unroll
    for (int j = 0; j < KS; j += 4) {
      float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
      if (r < nb) x = *reinterpret_cast<const float4*>(qbar + (long long)r * D + KS * g + j);
      qa[j] = x.x;
      qa[j + 1] = x.y;
      qa[j + 2] = x.z;
      qa[j + 3] = x.w;
    }
  }
  // Kbar fragments in chunks of 8 k-steps, software-pipelined: the next
  // chunk (after the last one, the first chunk of the next pair of key
  // tiles) is requested before the current chunk's MFMAs, so the loads of
  // a wave overlap its own MFMAs.  The k-step order of each accumulator is
  // unchanged.
  constexpr int CH = 8, NCH = KS / CH;
  auto load_chunk = [&](int c, int ch, float (&kb)[CH]) {
#pragma unroll
    for (int j = 0; j < CH; j += 4) {
      float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
      if (c < nb) x = *reinterpret_cast<const float4*>(kbar + (long long)c * D + KS * g + CH * ch + j);
      kb[j] = x.x;
      kb[j + 1] = x.y;
      kb[j + 2] = x.z;
      kb[j + 3] = x.w;
    }
  };
  // Wave w takes the key tiles of 16 blocks at 32 w + 128 t and 32 w + 128 t + 16
  // (two independent accumulator chains).
  if (32 * w < nb) {
    float b0[2][CH], b1[2][CH];
    load_chunk(32 * w + l16, 0, b0[0]);
    load_chunk(32 * w + 16 + l16, 0, b1[0]);
    for (int c0 = 32 * w; c0 < nb; c0 += 128) {
      f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ch = 0; ch < NCH; ++ch) {
        const int cur = ch & 1;
        if (ch + 1 < NCH) {
          load_chunk(c0 + l16, ch + 1, b0[cur ^ 1]);
          load_chunk(c0 + 16 + l16, ch + 1, b1[cur ^ 1]);
        } else if (c0 + 128 < nb) {
          load_chunk(c0 + 128 + l16, 0, b0[cur ^ 1]);
          load_chunk(c0 + 144 + l16, 0, b1[cur ^ 1]);
        }
#pragma unroll
        for (int j = 0; j < CH; ++j) {
          acc0 = __builtin_amdgcn_mfma_f32_16x16x4f32(qa[CH * ch + j], b0[cur][j], acc0, 0, 0, 0);
          acc1 = __builtin_amdgcn_mfma_f32_16x16x4f32(qa[CH * ch + j], b1[cur][j], acc1, 0, 0, 0);
        }
      }
      // accumulator lane l, register i: row 4 (l/16) + i, key c + l%16
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (c0 + l16 < nb) S[(4 * g + i) * nb + c0 + l16] = acc0[i];
        if (c0 + 16 + l16 < nb) S[(4 * g + i) * nb + c0 + 16 + l16] = acc1[i];
      }
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
    if (s.dense || (a < s.pb && s.prefix_rows)) {  // dense row: every block
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
// attend: one workgroup of four waves per pair of neighbouring query blocks
// (a0 = 2p, a1 = 2p + 1) of one (b, h); wave w owns the 32 query rows
// 32 (w & 1) .. + 31 of block a0 + (w >> 1).  The pair walks the union of
// its two key-block lists, in half tiles of 32 keys: first both halves of
// every key block either block selected (ascending), then every centroid
// half tile that either block needs.  Each half tile (K and V^T, 16 KB at
// D = 128) is copied once from global memory straight into an LDS ring of S
// stages and read from there by the waves whose block needs it; the other
// waves skip it.  Per half tile and wave (32 keys x 32 queries):
//   S^T = K Q^T     D/16 v_mfma_f32_32x32x16_bf16
//   P = exp2(S^T c1 + bias - mref), row sums in-lane (VALU)
//   O^T += V^T P^T  D/16 MFMAs
// Three waves run per SIMD (at most 168 VGPRs each, a two-stage ring so that
// three workgroups fit a CU's LDS), so that the waves of one workgroup that
// skip a half tile or wait at its barrier leave the SIMD to the others.
//
// LDS order of a half tile: 1 KB blocks of 64 lanes x 16 bytes, each the
// A operand of one MFMA for lane = position:
//   K block s (s < D/16):      lane l holds K[key(l % 32)][16 s + 8 (l/32) .. +8]
//   V^T block 2 dt + j:        lane l holds V^T[32 dt + l % 32][keys of
//                              k-step j, 8 (l/32) .. +8]
// with key(r) = r with bits 3 and 4 swapped: exactly the packed K and V^T
// half tiles one after the other.  That key order makes the S^T accumulator
// registers 8 j .. 8 j + 7 of a lane exactly the P^T B operand of k-step j,
// so P^T goes from accumulator to operand with no lane movement, and every
// LDS read is a linear, conflict-free ds_read_b128.
// ---------------------------------------------------------------------------
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x16 __attribute__((ext_vector_type(16)));

// s_waitcnt immediate: vmcnt(n) and lgkmcnt(0), expcnt untouched.
constexpr int wait_vm_lgkm0(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4); }

// Workgroup barrier that orders LDS accesses around it in the compiler but,
// unlike __syncthreads, does not wait for outstanding global->LDS copies.
__device__ __forceinline__ void ring_barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Entry of union half tile u of a workgroup: index (key block, or centroid
// half tile when u >= te) in bits 0..11, flags (which of the two query
// blocks needs it) above.
__device__ __forceinline__ int union_entry(const uint16_t* ulist, const uint16_t* uct, int te, int u) {
  const int e = (u >= te) ? (int)uct[min(max(u - te, 0), SA_MAX_BLOCKS / 32 - 1)]
                          : (int)ulist[min(u >> 1, SA_MAX_BLOCKS - 1)];
  return __builtin_amdgcn_readfirstlane(e);
}

// This wave's PER 1 KB blocks of one half tile, global -> LDS: lane l's 16
// bytes land at dst + 1024 i + 16 l (global_load_lds_dwordx4, LDS address in
// M0).  Written as asm so that the compiler does not track these copies: it
// would otherwise wait for all of them before every LDS read.  Completion is
// established by the explicit vmcnt waits and barriers of the ring.  The
// instruction has no result register.  M0 is saved and restored around each
// copy (it is reserved to the compiler), with one wait state between the M0
// write and the copy that reads it.
template <int PER>
__device__ __forceinline__ void copy_blocks(const uint16_t* src, const int (&doff)[PER], uint32_t dst) {
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %2\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, off\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(src + doff[i]), "s"(dst + i * 1024)
        : "memory");
  }
}

__device__ __forceinline__ bf16x8 lds_frag(const uint8_t* stage, int blk, int lane) {
  return *reinterpret_cast<const bf16x8*>(stage + blk * 1024 + lane * 16);
}

// One global -> LDS copy of this lane's 16 bytes at src to dst + 16 * lane
// (same instruction and M0 handling as copy_blocks).
__device__ __forceinline__ void copy_one(const void* src, uint32_t dst) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(src), "s"(dst)
      : "memory");
}

// INT8 QK^T of one half tile: S^T = R8 Q8^T on v_mfma_i32_32x32x32_i8 (exact
// int32 sums), returned as fp32.  Step t pairs byte j of lane l of the code
// block with byte j of lane l of q8[t]: both hold dimension
// 32 t + 16 (j/8) + 8 (l/32) + j % 8.
template <int NT>
__device__ __forceinline__ f32x16 tile_qk_i8(const uint8_t* stage, int lane, const i32x4 (&q8)[NT]) {
  i32x4 kf[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) kf[t] = *reinterpret_cast<const i32x4*>(stage + t * 1024 + lane * 16);
  i32x16 iacc = {};
#pragma unroll
  for (int t = 0; t < NT; ++t) iacc = __builtin_amdgcn_mfma_i32_32x32x32_i8(kf[t], q8[t], iacc, 0, 0, 0);
  __builtin_amdgcn_sched_group_barrier(0x100, NT, 0);
  __builtin_amdgcn_sched_group_barrier(0x008, NT, 0);
  f32x16 sacc;
#pragma unroll
  for (int i = 0; i < 16; ++i) sacc[i] = (float)iacc[i];
  return sacc;
}

// q . base_c of this lane's query row against the bf16 base row at rec: each
// half of the wave holds the dimensions of its own Q fragments, the two
// partial sums are added across the halves.
template <int NK>
__device__ __forceinline__ float mean_dot(const uint8_t* rec, int hh, const bf16x8 (&qf)[NK]) {
  float a0 = 0.0f, a1 = 0.0f;
#pragma unroll
  for (int k = 0; k < NK; ++k) {
    const uint4 bw = *reinterpret_cast<const uint4*>(rec + (16 * k + 8 * hh) * 2);
    const uint4 qw = __builtin_bit_cast(uint4, qf[k]);
    a0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, bw.x), __builtin_bit_cast(bf16x2, qw.x), a0, false);
    a1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, bw.y), __builtin_bit_cast(bf16x2, qw.y), a1, false);
    a0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, bw.z), __builtin_bit_cast(bf16x2, qw.z), a0, false);
    a1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, bw.w), __builtin_bit_cast(bf16x2, qw.w), a1, false);
  }
  const float part = a0 + a1;
  const auto ps = __builtin_amdgcn_permlane32_swap(__float_as_uint(part), __float_as_uint(part), false, false);
  return __uint_as_float(ps[0]) + __uint_as_float(ps[1]);
}

// S^T (32 keys x this wave's 32 queries) of the half tile in `stage`, added
// to init.
template <int NK>
__device__ __forceinline__ f32x16 tile_qk(const uint8_t* stage, int lane, const bf16x8 (&qf)[NK],
                                          const f32x16& init) {
  bf16x8 kf[NK];
#pragma unroll
  for (int k = 0; k < NK; ++k) kf[k] = lds_frag(stage, k, lane);
  f32x16 sacc = init;
#pragma unroll
  for (int k = 0; k < NK; ++k) sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[k], qf[k], sacc, 0, 0, 0);
  // all LDS reads first, then the MFMA chain
  __builtin_amdgcn_sched_group_barrier(0x100, NK, 0);
  __builtin_amdgcn_sched_group_barrier(0x008, NK, 0);
  return sacc;
}

// Additive per-key term (log2 domain) of a half tile for one query block:
// 0 for a valid key of an exact block and -inf past N; for a centroid,
// log2(n_c) (0 without the log-mass bias) if that block exists and the query
// block did not select it, else -inf.  Register i of the lane holds key
// key(8 (i/4) + 4 hh + i % 4).
__device__ __forceinline__ void tile_key_bias(float (&kb)[16], bool cen, int c, int half, int N, int nb,
                                              uint32_t sbits, int hh, float bias_full, float bias_tail) {
  // One bit per key of the half tile: set = no term (selected centroid,
  // block past n_b, or key past N).
  const int nv = cen ? nb - 32 * c : min(kBlock, N - c * kBlock) - 32 * half;  // valid keys
  uint32_t m = (nv >= 32) ? 0u : ~((1u << max(nv, 0)) - 1u);
  if (cen) m |= sbits;
  const float bval = cen ? bias_full : 0.0f;
  const uint32_t sb = m >> (4 * hh);
#pragma unroll
  for (int i = 0; i < 16; ++i) kb[i] = ((sb >> (16 * ((i >> 2) & 1) + 8 * (i >> 3) + (i & 3))) & 1u) ? -INFINITY : bval;
  // the centroid of a ragged last block carries log2 of its own row count
  const int rt = nb - 1 - 32 * c;
  if (cen && rt >= 0 && rt < 32 && !((m >> rt) & 1u) && bias_tail != bias_full) {
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (16 * ((i >> 2) & 1) + 8 * (i >> 3) + 4 * hh + (i & 3) == rt) kb[i] = bias_tail;
  }
}

// Maximum logit of this lane's query over one half tile.
__device__ __forceinline__ float tile_row_max(const f32x16& sacc, const float (&kb)[16], float a) {
  float m = -INFINITY;
#pragma unroll
  for (int i = 0; i < 16; ++i) m = fmaxf(m, fmaf(sacc[i], a, kb[i]));
  const auto p32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m), false, false);
  return fmaxf(__uint_as_float(p32[0]), __uint_as_float(p32[1]));
}

// P = exp2(S^T a + kb - mref) in bf16 (kb replaced by the lane constant boff
// on plain tiles), row sums, O^T += V^T P^T.  V^T starts at block vblk of the
// stage.
template <int NK, bool PLAIN>
__device__ __forceinline__ void tile_pv(const uint8_t* stage, int vblk, int lane, const f32x16& sacc,
                                        const float (&kb)[16], float a, float boff, float mref,
                                        f32x16 (&acc)[NK / 2], float (&lsum)[2]) {
  bf16x8 vf[NK];
#pragma unroll
  for (int k = 0; k < NK; ++k) vf[k] = lds_frag(stage, vblk + k, lane);
  float pe[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) pe[i] = __builtin_amdgcn_exp2f(fmaf(sacc[i], a, (PLAIN ? boff : kb[i]) - mref));
  bf16x8 pb[2];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int e = 0; e < 8; ++e) pb[j][e] = (__bf16)pe[8 * j + e];
  // Row sums of the bf16-rounded P that the MFMAs use (so that the final
  // division is consistent with the accumulated P V), two bf16 per
  // v_dot2_f32_bf16 against (1, 1), in two independent chains.
  const bf16x2 one2 = __builtin_bit_cast(bf16x2, 0x3f803f80u);
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const uint4 wd = __builtin_bit_cast(uint4, pb[j]);
    lsum[0] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, wd.x), one2, lsum[0], false);
    lsum[1] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, wd.y), one2, lsum[1], false);
    lsum[0] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, wd.z), one2, lsum[0], false);
    lsum[1] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, wd.w), one2, lsum[1], false);
  }
#pragma unroll
  for (int dt = 0; dt < NK / 2; ++dt)
#pragma unroll
    for (int j = 0; j < 2; ++j)
      acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[2 * dt + j], pb[j], acc[dt], 0, 0, 0);
  // V^T reads are in flight while the exponentials run
  __builtin_amdgcn_sched_group_barrier(0x100, NK, 0);
  __builtin_amdgcn_sched_group_barrier(0x002, 64, 0);
  __builtin_amdgcn_sched_group_barrier(0x008, NK, 0);
}

// Heads ordered across the XCDs only up to this many (the ordering takes
// O((B H)^2) comparisons in one workgroup).
constexpr int kMaxOrderedHeads = 4096;

template <int D, int S, bool RW, bool Q8>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(Q8 ? 2 : 3, Q8 ? 2 : 3))) void attend_kernel(
    Shape s, const uint16_t* __restrict__ q, uint16_t* __restrict__ out, Workspace ws) {
  constexpr int NK = D / 16;          // QK k-steps = K blocks = PV MFMAs per tile
  constexpr int NDT = D / 32;         // 32-row d tiles of O^T
  constexpr int NBLK = 2 * NK;        // 1 KB LDS blocks per half tile
  constexpr int PER = NBLK / 4;       // copies per wave per half tile
  constexpr int HT = 32 * D;          // elements of a half tile
  constexpr int STAGE = NBLK * 1024;  // bytes of one ring stage
  constexpr int NW = SA_MAX_BLOCKS / 32;
  constexpr int NT = D / 32;          // INT8 QK k-steps
  static_assert(!Q8 || S == 2, "INT8 copies are not balanced across waves: every ring step waits for all");
  extern __shared__ __attribute__((aligned(16))) uint8_t ring[];  // S * STAGE bytes
  __shared__ uint32_t sel[2][NW];            // selected key blocks of a0, a1
  __shared__ uint16_t ulist[SA_MAX_BLOCKS];  // union of the two lists
  __shared__ uint16_t uct[NW];               // centroid half tiles either needs
  __shared__ int info[8];
  __shared__ __attribute__((aligned(16))) float cbs[RW ? SA_MAX_BLOCKS : 4];  // reweight biases / c1

  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, hh = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int G = gridDim.x, bid = blockIdx.x;
  const int xcd = bid & 7, kx = bid >> 3, qq = G >> 3, rr = G & 7;
  const int lid = (xcd < rr) ? xcd * (qq + 1) + kx : rr * (qq + 1) + (xcd - rr) * qq + kx;
  const int nb = s.nb, N = s.N;
  const float c1 = s.c1;
  const int np = (nb + 1) >> 1;
  const int nbh = s.B * s.H;
  const int bhi = (s.dense || (nbh & 7) || nbh > kMaxOrderedHeads) ? lid / np
                                                           : min(max(ws.head_order[lid / np], 0), nbh - 1);
  const int p = s.dense ? lid % np : min(max(ws.pair_order[(long long)bhi * np + lid % np], 0), np - 1);
  const int h = bhi % s.H, b = bhi / s.H;
  const long long bh = bhi;
  const int a0 = 2 * p;
  const bool has1 = a0 + 1 < nb;
  const int x = w >> 1;  // this wave's block is a0 + x
  const bool exists = x == 0 || has1;
  const int myflag = 1 << x;

  // Q^T B-operand fragments: lane l holds Q[row l % 32][16 k + 8 (l/32) .. +8].
  const int qrow = (a0 + x) * kBlock + 32 * (w & 1) + l32;
  const int qorig = (exists && qrow < N) ? src_row(s, ws, 0, bh, qrow) : 0;  // the caller's row
  bf16x8 qf[NK];
  {
    const uint16_t* qp = q + (long long)b * s.isb + (long long)h * s.ish + (long long)qorig * s.ist + 8 * hh;
#pragma unroll
    for (int k = 0; k < NK; ++k) {
      uint4 v4 = make_uint4(0, 0, 0, 0);
      if (exists && qrow < N) v4 = *reinterpret_cast<const uint4*>(qp + 16 * k);
      qf[k] = __builtin_bit_cast(bf16x8, v4);
    }
  }
  // INT8 QK^T: the row's scale s_q = max |q| / 127 and its codes, in the
  // B-operand order of the int8 MFMA (bytes 0..7 of step t from qf[2t],
  // bytes 8..15 from qf[2t + 1]).
  i32x4 q8[Q8 ? NT : 1];
  float sq = 0.0f;
  if constexpr (Q8) {
    float amax = 0.0f;
#pragma unroll
    for (int k = 0; k < NK; ++k)
#pragma unroll
      for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf((float)qf[k][e]));
    const auto pm = __builtin_amdgcn_permlane32_swap(__float_as_uint(amax), __float_as_uint(amax), false, false);
    amax = fmaxf(__uint_as_float(pm[0]), __uint_as_float(pm[1]));
    sq = amax / 127.0f;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      uint32_t wd[4] = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int jj = 0; jj < 16; ++jj) {
        const float xq = (float)qf[2 * t + (jj >> 3)][jj & 7];
        const int code = sq > 0.0f ? (int)fminf(fmaxf(rintf(xq / sq), -127.0f), 127.0f) : 0;
        wd[jj >> 2] |= ((uint32_t)code & 0xffu) << (8 * (jj & 3));
      }
      q8[t] = i32x4{(int)wd[0], (int)wd[1], (int)wd[2], (int)wd[3]};
    }
  }

  // Union of the two lists and the centroid half tiles either block needs,
  // as a table in LDS, and the first half tile each block needs.
  const int nct = s.nbp / 32;
  if (s.dense) {
    const int fl = (1 | ((int)has1 << 1)) << 12;
    for (int i = tid; i < nb; i += 256) ulist[i] = (uint16_t)(i | fl);
    if (tid == 0) {
      info[0] = nb;
      info[1] = 0;
      info[3] = 0;
      info[4] = has1 ? 0 : 2 * nb;
    }
  } else {
    if (RW) {
      const float inv_c1 = 1.0f / s.c1;
      for (int i = tid; i < s.nbp; i += 256) cbs[i] = ws.cbias[bh * s.nbp + i] * inv_c1;
    }
    const int cnt0 = min(max(ws.counts[bh * nb + a0], 0), nb);
    const int cnt1 = has1 ? min(max(ws.counts[bh * nb + a0 + 1], 0), nb) : 0;
    for (int i = tid; i < 2 * NW; i += 256) sel[i / NW][i % NW] = 0u;
    __syncthreads();
    const int* L0 = ws.lists + (bh * nb + a0) * (long long)nb;
    for (int i = tid; i < cnt0; i += 256) {
      const int c = L0[i];
      if (c >= 0 && c < nb) atomicOr(&sel[0][c >> 5], 1u << (c & 31));
    }
    for (int i = tid; i < cnt1; i += 256) {
      const int c = L0[nb + i];
      if (c >= 0 && c < nb) atomicOr(&sel[1][c >> 5], 1u << (c & 31));
    }
    __syncthreads();
    if (w == 0) {
      const int nwords = (nb + 31) >> 5;
      const uint32_t m0 = lane < nwords ? sel[0][lane] : 0u, m1 = lane < nwords ? sel[1][lane] : 0u;
      uint32_t um = m0 | m1;
      const int cw = __popc(um);
      int incl = cw;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int t = __shfl_up(incl, o);
        if (lane >= o) incl += t;
      }
      const int excl = incl - cw;
      // union position of the first block of each list
      int first[2];
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const uint32_t mk = k ? m1 : m0;
        const uint64_t any = __ballot(mk != 0u);
        const int fl = any ? __ffsll((long long)any) - 1 : 0;
        const int pos = excl + __popc(um & ((mk & (0u - mk)) - 1u));
        first[k] = any ? 2 * __shfl(pos, fl) : -1;
      }
      int pos = excl;
      while (um) {
        const int bit = __ffs(um) - 1;
        um &= um - 1u;
        ulist[pos++] = (uint16_t)((lane * 32 + bit) | (((m0 >> bit) & 1u) << 12) | (((m1 >> bit) & 1u) << 13));
      }
      const int nu = __shfl(incl, 63);
      int ncu = 0;
      if (s.centroid) {
        bool n0 = false, n1 = false;
        if (lane < nct) {
          const int valid = min(32, nb - 32 * lane);
          const uint32_t vmask = valid >= 32 ? 0xffffffffu : ((1u << max(valid, 0)) - 1u);
          n0 = cnt0 < nb && (~m0 & vmask) != 0u;
          n1 = has1 && cnt1 < nb && (~m1 & vmask) != 0u;
        }
        const bool keep = n0 || n1;
        const uint64_t bm = __ballot(keep);
        const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
        const int slot = __popcll(bm & lt);
        if (keep) uct[slot] = (uint16_t)(lane | ((int)n0 << 12) | ((int)n1 << 13));
        ncu = __popcll(bm);
        const uint64_t b0 = __ballot(n0), b1 = __ballot(n1);
        if (first[0] < 0 && b0) first[0] = 2 * nu + __popcll(bm & ((b0 & (0ull - b0)) - 1ull));
        if (first[1] < 0 && b1) first[1] = 2 * nu + __popcll(bm & ((b1 & (0ull - b1)) - 1ull));
      }
      if (lane == 0) {
        info[0] = nu;
        info[1] = ncu;
        info[3] = first[0] < 0 ? 2 * nu + ncu : first[0];
        info[4] = first[1] < 0 ? 2 * nu + ncu : first[1];
      }
    }
  }
  if (tid == 0) info[2] = 0;
  __syncthreads();
  const int nu = __builtin_amdgcn_readfirstlane(info[0]), ncu = __builtin_amdgcn_readfirstlane(info[1]);
  const int TE = 2 * nu, TU = TE + ncu;
  const int fme = __builtin_amdgcn_readfirstlane(info[3 + x]);  // first half tile this wave needs

  // Per-lane element offsets of this wave's copies inside a packed half tile:
  // waves 0, 1 copy the K blocks, waves 2, 3 the V^T blocks.
  const bool kwave = w < 2;
  // (the packed tiles are stored in LDS order: each block is a linear copy)
  int doff[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) doff[i] = (((w & 1) * PER + i) * 64 + lane) * 8;
  const uint16_t* ex_bh = (kwave ? ws.kp : ws.vp) + bh * nb * 2LL * HT;
  const uint16_t* ce_bh = (kwave ? ws.kbp : ws.vbp) + bh * nct * (long long)HT;
  const uint32_t my_dst =
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)ring + w * PER * 1024;
  const uint8_t* const rd = ring;
  // (reweight mode: no log-mass term; its bias enters through the centroid
  // tile's accumulator, see qk)
  const float bias_full = RW ? 0.0f : s.bias_full, bias_tail = RW ? 0.0f : s.bias_tail;

  // Exact half tiles come first (the union is ascending) and only a ragged
  // last block and the centroid tiles need per-key terms, so the plain tiles
  // are a prefix of the sequence.
  int nplain = TE;
  if (nu > 0 && s.tail < kBlock && (union_entry(ulist, uct, TE, TE - 1) & 0xfff) == nb - 1) nplain = TE - 2;

  // Softmax reference: every logit x of a query is scored as
  // p = exp2(x - mref) with a fixed mref, the exact maximum over the first
  // half tile the query sees plus 32 (log2 units).  Terms of that tile lie
  // below 2^-32 and the row's largest term is at least 2^-32, well inside
  // the fp32 / bf16 range, so no running maximum or rescaling is needed; the
  // ratio acc / l does not depend on mref.  If a later term exceeds mref by
  // so much that a row sum leaves [0, 2^100] (or is not finite), the pair is
  // recomputed with the exact row maxima from a Q K^T-only pass.
  f32x16 acc[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) acc[dt] = f32x16{};
  float lsum[2] = {0.0f, 0.0f}, mref = 0.0f, mmax = -INFINITY;
  bool safe = false;

  // One pass over the union through the ring: at step u every wave waits for
  // its own copies of half tile u, the barrier makes all of them visible and
  // frees the stage read at step u - 1, and half tile u + S - 1 (clamped to
  // the last one, so that every step waits on the same count) is requested
  // into that stage.  Half tile v always lands in stage v % S.  eq[] holds
  // the table entries of the half tiles in flight (u .. u + S - 2).
  int eq[S - 1];
  int st = 0;
  // Table entries of 64 consecutive half tiles, one per lane, so that a
  // lookup is a v_readlane instead of an LDS round trip on every step.
  int tab_base = 0, tabv = 0;
  auto tab_load = [&](int base) {
    tab_base = base;
    const int v = min(base + lane, max(TU - 1, 0));
    tabv = (v >= TE) ? (int)uct[min(max(v - TE, 0), NW - 1)] : (int)ulist[min(v >> 1, SA_MAX_BLOCKS - 1)];
  };
  auto lookup = [&](int v) {
    if (v >= tab_base + 64) tab_load(v & ~63);
    return __builtin_amdgcn_readlane(tabv, v - tab_base);
  };
  // INT8 exact half tile: 1 KB blocks [codes 0 .. NT-1 | V^T 0 .. NK-1 |
  // base record], block i copied by wave i % 4.  Per copy slot of this wave:
  // the lane's source for key block 0 and the byte strides per half tile
  // (codes, V^T) or per key block (the record, D/8 + 1 lanes).
  constexpr int NQ = NT + NK + 1, PQ = (NQ + 3) / 4;
  const uint8_t* qsrc[PQ];
  int qht[PQ], qblk[PQ];
  bool qlane[PQ];
#pragma unroll
  for (int i = 0; i < PQ; ++i) {
    const int bi = w + 4 * i;
    if (bi < NT) {
      qsrc[i] = ws.k8 + bh * nb * 64LL * D + bi * 1024 + lane * 16;
      qht[i] = 32 * D;
      qblk[i] = 0;
    } else if (bi < NT + NK) {
      qsrc[i] = reinterpret_cast<const uint8_t*>(ws.vp + bh * nb * 2LL * HT + (bi - NT) * 512 + lane * 8);
      qht[i] = 2 * HT;
      qblk[i] = 0;
    } else {
      qsrc[i] = reinterpret_cast<const uint8_t*>(ws.kbase + bh * nb * (long long)(D + 8) + lane * 8);
      qht[i] = 0;
      qblk[i] = 2 * (D + 8);
    }
    qlane[i] = bi < NT + NK || (bi == NT + NK && lane <= D / 8);
  }
  const uint32_t ring_lds = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)ring;
  auto copy_q8 = [&](int c, int ht, int stg) {
    const uint32_t base = ring_lds + stg * STAGE;
#pragma unroll
    for (int i = 0; i < PQ; ++i) {
      if (w + 4 * i < NQ && qlane[i])
        copy_one(qsrc[i] + (long long)(2 * c + ht) * qht[i] + (long long)c * qblk[i], base + (w + 4 * i) * 1024);
    }
  };
  auto copy_tile = [&](int v, int e, int stg) {
    const int c = e & 0xfff;
    if constexpr (Q8) {
      if (v < TE) {
        copy_q8(c, v & 1, stg);
        return;
      }
    }
    const long long off = (v >= TE) ? (long long)c * HT : ((long long)c * 2 + (v & 1)) * HT;
    copy_blocks<PER>(((v >= TE) ? ce_bh : ex_bh) + off, doff, my_dst + stg * STAGE);
  };
  auto ring_start = [&]() {
    st = 0;
    tab_load(0);
#pragma unroll
    for (int k = 0; k < S - 1; ++k) {
      const int v = min(k, TU - 1);
      eq[k] = lookup(v);
      copy_tile(v, eq[k], k);
    }
  };
  // Returns the entry of half tile u; afterwards the stage of u is rd + st*STAGE.
  auto ring_step = [&](int u) {
    __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0((S - 2) * PER));
    ring_barrier();
    const int v = min(u + S - 1, TU - 1);
    const int ev = lookup(v);
    copy_tile(v, ev, st == 0 ? S - 1 : st - 1);
    const int eu = eq[0];
#pragma unroll
    for (int k = 0; k < S - 2; ++k) eq[k] = eq[k + 1];
    eq[S - 2] = ev;
    return eu;
  };
  auto ring_next = [&]() { st = (st == S - 1) ? 0 : st + 1; };
  auto bias_of = [&](int u, int eu, float (&kb)[16]) {
    const bool cen = u >= TE;
    tile_key_bias(kb, cen, eu & 0xfff, u & 1, N, nb, sel[x][cen ? (eu & (NW - 1)) : 0], hh, bias_full, bias_tail);
  };

  // Scores of a half tile.  The logit (log2 units) is sacc * ta + tb plus the
  // per-key term; bf16 QK^T gives ta = c1, tb = 0.  INT8 exact tiles give
  // ta = c1 s_q s_c and tb = c1 q . base_c, taken at the block's first half
  // tile from the base record that follows V^T in the stage.
  float ta = c1, tb = 0.0f;
  int vblk = NK;  // first V^T block of the stage
  auto qk_exact = [&](int u, const uint8_t* stage) -> f32x16 {  // u < TE
    if constexpr (Q8) {
      const uint8_t* rec = stage + (NT + NK) * 1024;
      if (!(u & 1)) {
        ta = c1 * (sq * *reinterpret_cast<const float*>(rec + 2 * D));
        tb = c1 * mean_dot<NK>(rec, hh, qf);
      }
      vblk = NT;
      return tile_qk_i8<NT>(stage, lane, q8);
    }
    return tile_qk<NK>(stage, lane, qf, f32x16{});
  };
  // Any half tile.  Reweight mode: the accumulator of a centroid tile starts
  // at each block's bias / c1 (four consecutive registers hold four
  // consecutive keys), so the logit carries the bias without a per-key term.
  auto qk = [&](int u, int eu, const uint8_t* stage) -> f32x16 {
    if constexpr (Q8) {
      if (u < TE) return qk_exact(u, stage);
      ta = c1;
      tb = 0.0f;
      vblk = NK;
    }
    f32x16 init = {};
    if constexpr (RW) {
      if (u >= TE) {
        const float* cb = cbs + 32 * (eu & 0xfff) + 4 * hh;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const float4 t = *reinterpret_cast<const float4*>(cb + 16 * (g & 1) + 8 * (g >> 1));
          init[4 * g] = t.x;
          init[4 * g + 1] = t.y;
          init[4 * g + 2] = t.z;
          init[4 * g + 3] = t.w;
        }
      }
    }
    return tile_qk<NK>(stage, lane, qf, init);
  };
  auto bias_t = [&](int u, int eu, float (&kb)[16]) {
    bias_of(u, eu, kb);
    if constexpr (Q8) {
      if (u < TE)
#pragma unroll
        for (int i = 0; i < 16; ++i) kb[i] += tb;
    }
  };

  // Q and the lists are in registers / LDS before the first copy is issued.
  __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(0));
  for (int attempt = 0; attempt < 2 && TU > 0; ++attempt) {
    if (attempt == 1) {
      // Safe mode: exact row maxima over every half tile first.
      ring_start();
      for (int u = 0; u < TU; ++u) {
        const int eu = ring_step(u);
        if ((eu >> 12) & myflag) {
          const f32x16 sacc = qk(u, eu, rd + st * STAGE);
          float kb[16];
          bias_t(u, eu, kb);
          mmax = fmaxf(mmax, tile_row_max(sacc, kb, ta));
        }
        ring_next();
      }
      __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(0));
      mref = (mmax == -INFINITY) ? 0.0f : mmax;
      lsum[0] = lsum[1] = 0.0f;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) acc[dt] = f32x16{};
      __syncthreads();
    }
    ring_start();
    int u = 0;
    // half tiles before the first one this wave needs: ring only
    for (; u < fme; ++u) {
      ring_step(u);
      ring_next();
    }
    if (u < TU) {
      const int eu = ring_step(u);
      const uint8_t* stage = rd + st * STAGE;
      const f32x16 sacc = qk(u, eu, stage);
      float kb[16];
      bias_t(u, eu, kb);
      if (!safe) {
        const float m = tile_row_max(sacc, kb, ta);
        mref = (m == -INFINITY) ? 0.0f : m + 32.0f;
      }
      tile_pv<NK, false>(stage, vblk, lane, sacc, kb, ta, 0.0f, mref, acc, lsum);
      ring_next();
      ++u;
    }
    for (; u < nplain; ++u) {
      const int eu = ring_step(u);
      if ((eu >> 12) & myflag) {
        const uint8_t* stage = rd + st * STAGE;
        const f32x16 sacc = qk_exact(u, stage);
        float kb[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) kb[i] = 0.0f;
        tile_pv<NK, true>(stage, vblk, lane, sacc, kb, ta, tb, mref, acc, lsum);
      }
      ring_next();
    }
    for (; u < TU; ++u) {
      const int eu = ring_step(u);
      if ((eu >> 12) & myflag) {
        const uint8_t* stage = rd + st * STAGE;
        const f32x16 sacc = qk(u, eu, stage);
        float kb[16];
        bias_t(u, eu, kb);
        tile_pv<NK, false>(stage, vblk, lane, sacc, kb, ta, 0.0f, mref, acc, lsum);
      }
      ring_next();
    }
    __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(0));
    if (attempt == 1) break;
    const float lpart = lsum[0] + lsum[1];
    const auto ps = __builtin_amdgcn_permlane32_swap(__float_as_uint(lpart), __float_as_uint(lpart), false, false);
    const float ltot = __uint_as_float(ps[0]) + __uint_as_float(ps[1]);
    if (__ballot(!(ltot <= 0x1p100f)) && lane == 0) info[2] = 1;
    __syncthreads();
    if (!__builtin_amdgcn_readfirstlane(info[2])) break;
    safe = true;
  }

  const float lpart = lsum[0] + lsum[1];
  const auto ps = __builtin_amdgcn_permlane32_swap(__float_as_uint(lpart), __float_as_uint(lpart), false, false);
  const float l = __uint_as_float(ps[0]) + __uint_as_float(ps[1]);
  const float inv = (l > 0.0f) ? 1.0f / l : 0.0f;
  if (exists && qrow < N) {
    uint16_t* o = out + (long long)b * s.osb + (long long)h * s.osh + (long long)qorig * s.ost + 4 * hh;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        uint2 w2;
        w2.x = f32_to_bf16_bits(acc[dt][4 * j] * inv) | (f32_to_bf16_bits(acc[dt][4 * j + 1] * inv) << 16);
        w2.y = f32_to_bf16_bits(acc[dt][4 * j + 2] * inv) | (f32_to_bf16_bits(acc[dt][4 * j + 3] * inv) << 16);
        *reinterpret_cast<uint2*>(o + 32 * dt + 8 * j) = w2;
      }
  }
}


// ---------------------------------------------------------------------------
// pair_order: grid B H, 256 threads.  The attend workgroups of one (b, h)
// take its pairs of query blocks longest first (by the two list lengths,
// ties by position), so that the shortest ones run last and the end of the
// launch drains sooner.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void pair_order_kernel(Shape s, Workspace ws) {
  __shared__ int len[SA_MAX_BLOCKS / 2];
  const long long bh = blockIdx.x;
  const int nb = s.nb, np = (nb + 1) >> 1;
  for (int p = threadIdx.x; p < np; p += 256) {
    const int a = 2 * p;
    int l = min(max(ws.counts[bh * nb + a], 0), nb);
    if (a + 1 < nb) l += min(max(ws.counts[bh * nb + a + 1], 0), nb);
    len[p] = l;
  }
  __syncthreads();
  int tot = 0;
  for (int p = threadIdx.x; p < np; p += 256) {
    const int l = len[p];
    tot += l;
    int rank = 0;
    for (int r = 0; r < np; ++r) {
      const int lr = len[r];
      rank += (lr > l || (lr == l && r < p)) ? 1 : 0;
    }
    ws.pair_order[bh * np + rank] = p;
  }
  // the head's total list length (its work), for head_order_kernel
  __shared__ int part[4];
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) tot += __shfl_xor(tot, o);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = tot;
  __syncthreads();
  if (threadIdx.x == 0) ws.head_work[bh] = part[0] + part[1] + part[2] + part[3];
}

// ---------------------------------------------------------------------------
// head_order: one workgroup, 256 threads.  The attend launch gives each XCD
// a contiguous run of B H / 8 heads; the heads are dealt to the eight runs
// in snake order of decreasing work (0..7, 7..0, ...), so that every XCD
// gets about the same total.  Used when B H is a multiple of 8.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void head_order_kernel(int nbh, Workspace ws) {
  const int per = nbh / 8;
  for (int h = threadIdx.x; h < nbh; h += 256) {
    const int wk = ws.head_work[h];
    int rank = 0;
    for (int r = 0; r < nbh; ++r) {
      const int wr = ws.head_work[r];
      rank += (wr > wk || (wr == wk && r < h)) ? 1 : 0;
    }
    const int round = rank / 8, pos = rank % 8;
    const int xcd = (round & 1) ? 7 - pos : pos;
    ws.head_order[xcd * per + round] = h;
  }
}

// Ring depth: half tile u + 1 is requested while u is computed.  At
// N = 16384 and 32768, 2, 3 and 4 stages ran within 1% of each other at the
// same occupancy; two stages (32 KB at D = 128) let three workgroups share a
// CU, which is 6-9% faster than two.
constexpr int kAttendStages = 2;

template <int D, int S, bool RW, bool Q8>
hipError_t launch_attend_t(const Shape& s, const uint16_t* q, uint16_t* out, const Workspace& ws,
                           hipStream_t stream) {
  constexpr int bytes = S * (D / 8) * 1024;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&attend_kernel<D, S, RW, Q8>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e != hipSuccess) return e;
  if (!s.dense) {
    hipLaunchKernelGGL(pair_order_kernel, dim3((unsigned)(s.B * s.H)), dim3(256), 0, stream, s, ws);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int nbh = s.B * s.H;
    if (!(nbh & 7) && nbh <= kMaxOrderedHeads) {
      hipLaunchKernelGGL(head_order_kernel, dim3(1), dim3(256), 0, stream, nbh, ws);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  dim3 grid((unsigned)((long long)s.B * s.H * ((s.nb + 1) / 2)));
  hipLaunchKernelGGL((attend_kernel<D, S, RW, Q8>), grid, dim3(256), bytes, stream, s, q, out, ws);
  return hipGetLastError();
}

template <int D, bool RW>
hipError_t launch_attend_d(const Shape& s, const uint16_t* q, uint16_t* out, const Workspace& ws,
                           hipStream_t stream) {
  if (s.int8) return launch_attend_t<D, kAttendStages, RW, true>(s, q, out, ws, stream);
  return launch_attend_t<D, kAttendStages, RW, false>(s, q, out, ws, stream);
}

template <int D>
hipError_t launch_select_t(const Shape& s, const Workspace& ws, hipStream_t stream) {
  const size_t lds = (size_t)16 * s.nb * sizeof(float) + 4 * 256 * sizeof(int);
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&select_kernel<D>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  dim3 grid((unsigned)(((s.nb + 15) / 16) * s.H * s.B));
  hipLaunchKernelGGL((select_kernel<D>), grid, dim3(256), lds, stream, s, ws);
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

hipError_t launch_anchor(const Shape& s, const void* q, const Workspace& ws, hipStream_t stream) {
  dim3 grid(s.H, s.B);
  const auto* qq = static_cast<const uint16_t*>(q);
  if (s.D == 128)
    hipLaunchKernelGGL(anchor_kernel<128>, grid, dim3(256), 0, stream, s, qq, ws);
  else
    hipLaunchKernelGGL(anchor_kernel<64>, grid, dim3(256), 0, stream, s, qq, ws);
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
  if (s.D == 128) return launch_select_t<128>(s, ws, stream);
  return launch_select_t<64>(s, ws, stream);
}


hipError_t launch_attend(const Shape& s, const void* q, void* out, const Workspace& ws, hipStream_t stream) {
  const auto* qq = static_cast<const uint16_t*>(q);
  auto* oo = static_cast<uint16_t*>(out);
  // Reweight and INT8 QK^T are instantiations of their own, so that the
  // default kernel carries none of their registers or LDS.
  if (s.reweight) {
    if (s.D == 128) return launch_attend_d<128, true>(s, qq, oo, ws, stream);
    return launch_attend_d<64, true>(s, qq, oo, ws, stream);
  }
  if (s.D == 128) return launch_attend_d<128, false>(s, qq, oo, ws, stream);
  return launch_attend_d<64, false>(s, qq, oo, ws, stream);
}

}  // namespace sa
