// gfx950 kernels of the Spark-Reblock partition (Spark-H3 news, Spark-Reblock
// bullet): the fixed 64-row tiles are replaced by an input-dependent
// partition per (b, h) and side, in which rows are alike when their score
// patterns over the other side are alike (the cosine in the metric of the
// other side's second moment), split top-down until every leaf holds one
// block.
//
// A "problem" p < 2 B H is one (side, b, h): side 0 partitions the query rows
// in the metric M = K^T K, side 1 the key rows (and with them the values) in
// M = Q^T Q.  Only the rows after the prefix blocks move (n_v of them).
//
//   gram_kernel        partial M over 2048-row chunks of the other side, on
//                      v_mfma_f32_32x32x16_bf16 (bf16 rows, exact products,
//                      fp32 sums; the chunk is staged transposed in LDS so
//                      that both operands are 16-byte LDS reads)
//   gram_reduce_kernel M = sum of the partials, in chunk order
//   embed_kernel       u_i = x_i / sqrt(x_i^T M x_i) and M u_i in bf16 (X M
//                      on MFMA with M rounded to bf16, M being symmetric so
//                      that its rows are the B operand; x^T M x from the
//                      bf16 X M) and the identity order
//   split_kernel       one level of the partition, one workgroup per group:
//                      the mean direction, the two pivots (least similar to
//                      the mean, then least similar to the first pivot), the
//                      rank values (M u_j) . (u_b - u_a), an exact radix
//                      select of the left child's size (ties by position)
//                      and a stable two-way partition of the group's order
// The path then reads Q, K, V rows through the final orders and writes each
// output row at its own position (no reordered copies).
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "sa_internal.h"
#include "sparse_attn.h"

namespace sa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kRbBlock = 64;

__device__ __forceinline__ float bf(uint32_t b) { return __uint_as_float(b << 16); }

__device__ __forceinline__ uint32_t to_bf16(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

struct Prob {
  int b, h, side;
};

__device__ __forceinline__ Prob prob_of(const Shape& s, int p) {
  const int bh = p % (s.B * s.H);
  return {bh / s.H, bh % s.H, p / (s.B * s.H)};
}

// Rows of the problem's own side (other = false) or of the other side.
__device__ __forceinline__ const uint16_t* rows_of(const Shape& s, const Prob& pr, const uint16_t* q,
                                                   const uint16_t* k, bool other) {
  const uint16_t* base = ((pr.side == 0) != other) ? q : k;
  return base + (long long)pr.b * s.isb + (long long)pr.h * s.ish;
}

// ---------------------------------------------------------------------------
// gram: grid (chunks, problems), 256 threads.  Wave w accumulates output
// tiles (t / (D/32), t % (D/32)) for t = w, w + 4, ...; each 64-row
// sub-chunk is staged as T[d][r] (bf16), so that the A operand
// (A[i][k] = Y[k][32 ti + i]) and the B operand (B[k][j] = Y[k][32 tj + j])
// are both 8 consecutive rows of one dimension.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void gram_kernel(Shape s, const uint16_t* __restrict__ q,
                                                   const uint16_t* __restrict__ k, Workspace ws) {
  constexpr int TP = kRbBlock + 8;  // LDS pitch of T (elements)
  constexpr int NTD = D / 32;
  constexpr int TPW = NTD * NTD / 4;
  __shared__ __attribute__((aligned(16))) uint16_t T[D * TP];
  const int c = blockIdx.x, p = blockIdx.y;
  const Prob pr = prob_of(s, p);
  const uint16_t* y = rows_of(s, pr, q, k, true);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, hh = lane >> 5, l32 = lane & 31;
  f32x16 acc[TPW];
  int ti[TPW], tj[TPW];
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    acc[t] = f32x16{};
    ti[t] = (w + 4 * t) / NTD;
    tj[t] = (w + 4 * t) % NTD;
  }
  const int r_begin = c * kGramChunk, r_end = min(s.N, r_begin + kGramChunk);
  // each thread stages LPT 16-byte chunks of a sub-chunk; the next
  // sub-chunk is loaded into registers while the current one is multiplied
  constexpr int LPT = kRbBlock * (D / 8) / 256;
  uint4 nxt[LPT];
  auto fetch = [&](int r0) {
#pragma unroll
    for (int u = 0; u < LPT; ++u) {
      const int i = tid + 256 * u, r = i / (D / 8), c8 = i % (D / 8);
      nxt[u] = (r0 + r < r_end) ? *reinterpret_cast<const uint4*>(y + (long long)(r0 + r) * s.ist + c8 * 8)
                                : make_uint4(0u, 0u, 0u, 0u);
    }
  };
  if (r_begin < r_end) fetch(r_begin);
  for (int r0 = r_begin; r0 < r_end; r0 += kRbBlock) {
    __syncthreads();
#pragma unroll
    for (int u = 0; u < LPT; ++u) {
      const int i = tid + 256 * u, r = i / (D / 8), c8 = i % (D / 8);
      const uint32_t wv[4] = {nxt[u].x, nxt[u].y, nxt[u].z, nxt[u].w};
#pragma unroll
      for (int e = 0; e < 8; ++e) T[(c8 * 8 + e) * TP + r] = (uint16_t)((wv[e >> 1] >> (16 * (e & 1))) & 0xffffu);
    }
    __syncthreads();
    if (r0 + kRbBlock < r_end) fetch(r0 + kRbBlock);
#pragma unroll
    for (int kk = 0; kk < kRbBlock / 16; ++kk) {
      const int k0 = 16 * kk + 8 * hh;
#pragma unroll
      for (int t = 0; t < TPW; ++t) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(T + (32 * ti[t] + l32) * TP + k0);
        const bf16x8 b = *reinterpret_cast<const bf16x8*>(T + (32 * tj[t] + l32) * TP + k0);
        acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[t], 0, 0, 0);
      }
    }
  }
  float* out = ws.rb_part + ((long long)p * s.rb_chunks + c) * D * D;
#pragma unroll
  for (int t = 0; t < TPW; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int row = 32 * ti[t] + 8 * (i >> 2) + 4 * hh + (i & 3);
      out[row * D + 32 * tj[t] + l32] = acc[t][i];
    }
}

// gram_reduce: grid (D*D/256, problems).  M = sum over chunks, in order.
template <int D>
__global__ __launch_bounds__(256) void gram_reduce_kernel(Shape s, Workspace ws) {
  const int p = blockIdx.y, e = blockIdx.x * 256 + threadIdx.x;
  if (e >= D * D) return;
  const float* part = ws.rb_part + (long long)p * s.rb_chunks * D * D + e;
  float m = 0.0f;
  for (int c = 0; c < s.rb_chunks; ++c) m += part[(long long)c * D * D];
  ws.rb_M[(long long)p * D * D + e] = m;
}

// ---------------------------------------------------------------------------
// embed: grid (ceil(n_v / kEmbedRows), problems), 256 threads, 64 rows at a
// time.  Y = X M on MFMA (M rounded to bf16; M is symmetric, so its rows are
// the B operand), stored as bf16 in LDS; four threads per row then take
// x^T M x = x . y over their quarters of the row (two shuffles) and write the
// unit row u = x / sqrt(x^T M x) and M u = y / sqrt(x^T M x), both bf16,
// and the identity order.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void embed_kernel(Shape s, const uint16_t* __restrict__ q,
                                                    const uint16_t* __restrict__ k, Workspace ws) {
  constexpr int LP = D + 8, TW = D / 64, NK = D / 16, QD = D / 4;
  __shared__ __attribute__((aligned(16))) uint16_t Mb[D * LP];
  __shared__ __attribute__((aligned(16))) uint16_t Xs[kRbBlock * LP];
  __shared__ __attribute__((aligned(16))) uint16_t Ys[kRbBlock * LP];
  const int p = blockIdx.y;
  const Prob pr = prob_of(s, p);
  const uint16_t* x = rows_of(s, pr, q, k, false);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, hh = lane >> 5, l32 = lane & 31;
  const float* M = ws.rb_M + (long long)p * D * D;
  for (int i = tid; i < D * D; i += 256) Mb[(i / D) * LP + i % D] = (uint16_t)to_bf16(M[i]);
  const int nv = s.rb_n;
  uint16_t* U = ws.rb_U + (long long)p * nv * D;
  uint16_t* MU = ws.rb_MU + (long long)p * nv * D;
  int* ord0 = ws.rb_ord + (long long)p * nv;
  const int rt = w & 1;
  const int jend = min(nv, (int)(blockIdx.x + 1) * kEmbedRows);
  constexpr int LPT = kRbBlock * (D / 8) / 256;
  uint4 nxt[LPT];
  auto fetch = [&](int j0) {
#pragma unroll
    for (int u = 0; u < LPT; ++u) {
      const int i = tid + 256 * u, r = i / (D / 8), c8 = i % (D / 8);
      nxt[u] = (j0 + r < nv) ? *reinterpret_cast<const uint4*>(x + (long long)(s.rb_r0 + j0 + r) * s.ist + c8 * 8)
                             : make_uint4(0u, 0u, 0u, 0u);
    }
  };
  if ((int)blockIdx.x * kEmbedRows < jend) fetch(blockIdx.x * kEmbedRows);
  const int r = tid >> 2, qd = tid & 3;  // the row and quarter this thread finishes
  for (int j0 = blockIdx.x * kEmbedRows; j0 < jend; j0 += kRbBlock) {
    __syncthreads();
#pragma unroll
    for (int u = 0; u < LPT; ++u) {
      const int i = tid + 256 * u, rr = i / (D / 8), c8 = i % (D / 8);
      *reinterpret_cast<uint4*>(Xs + rr * LP + c8 * 8) = nxt[u];
    }
    __syncthreads();
    if (j0 + kRbBlock < jend) fetch(j0 + kRbBlock);
#pragma unroll
    for (int t = 0; t < TW; ++t) {
      const int ct = (w >> 1) * TW + t;
      f32x16 acc = {};
#pragma unroll
      for (int kk = 0; kk < NK; ++kk) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(Xs + (32 * rt + l32) * LP + 16 * kk + 8 * hh);
        const bf16x8 b = *reinterpret_cast<const bf16x8*>(Mb + (32 * ct + l32) * LP + 16 * kk + 8 * hh);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < 16; ++i)
        Ys[(32 * rt + 8 * (i >> 2) + 4 * hh + (i & 3)) * LP + 32 * ct + l32] = (uint16_t)to_bf16(acc[i]);
    }
    __syncthreads();
    float xs[QD], ys[QD];
#pragma unroll
    for (int d = 0; d < QD; d += 8) {
      const uint4 xv = *reinterpret_cast<const uint4*>(Xs + r * LP + qd * QD + d);
      const uint4 yv = *reinterpret_cast<const uint4*>(Ys + r * LP + qd * QD + d);
      const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w}, yw[4] = {yv.x, yv.y, yv.z, yv.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        xs[d + e] = bf((xw[e >> 1] >> (16 * (e & 1))) & 0xffffu);
        ys[d + e] = bf((yw[e >> 1] >> (16 * (e & 1))) & 0xffffu);
      }
    }
    float n2 = 0.0f;
#pragma unroll
    for (int d = 0; d < QD; ++d) n2 += xs[d] * ys[d];
    n2 += __shfl_xor(n2, 1);
    n2 += __shfl_xor(n2, 2);
    const float inv = n2 > 0.0f ? 1.0f / sqrtf(n2) : 0.0f;
    if (j0 + r < nv) {
#pragma unroll
      for (int d = 0; d < QD; d += 8) {
        uint32_t wu[4], wm[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          wu[e] = to_bf16(xs[d + 2 * e] * inv) | (to_bf16(xs[d + 2 * e + 1] * inv) << 16);
          wm[e] = to_bf16(ys[d + 2 * e] * inv) | (to_bf16(ys[d + 2 * e + 1] * inv) << 16);
        }
        *reinterpret_cast<uint4*>(U + (long long)(j0 + r) * D + qd * QD + d) = make_uint4(wu[0], wu[1], wu[2], wu[3]);
        *reinterpret_cast<uint4*>(MU + (long long)(j0 + r) * D + qd * QD + d) = make_uint4(wm[0], wm[1], wm[2], wm[3]);
      }
      if (qd == 0) ord0[j0 + r] = j0 + r;
    }
  }
}

// Start and size of node g at depth `level` of the split tree of n rows
// (children: left 64 ceil(m/2) rows, right the rest; a node of <= 64 rows is
// a leaf and is carried by its all-left descendants, the others are empty).
__host__ __device__ __forceinline__ void group_range(int n, int level, int g, int& start, int& size) {
  start = 0;
  size = n;
  for (int t = 0; t < level; ++t) {
    const int bit = (g >> (level - 1 - t)) & 1;
    if (size <= kRbBlock) {
      if (bit) {
        size = 0;
        return;
      }
      continue;
    }
    const int m = (size + kRbBlock - 1) / kRbBlock, nl = kRbBlock * ((m + 1) / 2);
    if (bit) {
      start += nl;
      size -= nl;
    } else {
      size = nl;
    }
  }
}

__device__ __forceinline__ uint32_t order_bits(float f) {
  if (f == 0.0f) f = 0.0f;  // -0 and +0 rank together
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// ---------------------------------------------------------------------------
// split: grid (2^level, problems), NT threads.  Node g of the level reads
// its rows' order from buffer level & 1 and writes its children's order to
// buffer (level + 1) & 1.  Rows are read D/8 lanes per row (one 16-byte
// chunk each), so a wave covers 64 / (D/8) rows per step and a lane keeps
// the 8 matching entries of the current vector in registers.
// ---------------------------------------------------------------------------
template <int D, int NT>
__global__ __launch_bounds__(NT) void split_kernel(Shape s, int level, Workspace ws) {
  constexpr int CPR = D / 8;      // lanes per row
  constexpr int RPW = 64 / CPR;   // rows per wave step
  constexpr int NWV = NT / 64;    // waves
  constexpr int STEP = NWV * RPW;
  __shared__ float vec[D];
  __shared__ float wsum[NWV][D];
  __shared__ float rv[NWV];
  __shared__ int ri[NWV];
  __shared__ uint32_t hist[256];
  __shared__ int sel[2];
  __shared__ int wc[2][NWV];
  const int g = blockIdx.x, p = blockIdx.y, nv = s.rb_n, tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6, sub = lane / CPR, c8 = lane % CPR;
  int start, n;
  group_range(nv, level, g, start, n);
  if (n == 0) return;
  const int* oin = ws.rb_ord + ((long long)(level & 1) * s.rb_P + p) * nv + start;
  int* oout = ws.rb_ord + ((long long)((level + 1) & 1) * s.rb_P + p) * nv + start;
  if (n <= kRbBlock) {
    for (int i = tid; i < n; i += NT) oout[i] = oin[i];
    return;
  }
  const int m = (n + kRbBlock - 1) / kRbBlock, nl = kRbBlock * ((m + 1) / 2);
  const uint16_t* U = ws.rb_U + (long long)p * nv * D;
  const uint16_t* MU = ws.rb_MU + (long long)p * nv * D;
  uint32_t* keys = ws.rb_key + (long long)p * nv + start;

  // Row loops take UN steps at a time: the order entries first, then the
  // rows, so that the loads of a step do not wait on the previous step.
  constexpr int UN = 4;
  // mean direction ubar (fp32)
  {
    float a[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int j0 = wv * RPW + sub; j0 < n; j0 += STEP * UN) {
      int idx[UN];
#pragma unroll
      for (int u = 0; u < UN; ++u) idx[u] = (j0 + u * STEP < n) ? oin[j0 + u * STEP] : -1;
      uint4 v[UN];
#pragma unroll
      for (int u = 0; u < UN; ++u)
        v[u] = idx[u] >= 0 ? *reinterpret_cast<const uint4*>(U + (long long)idx[u] * D + c8 * 8)
                           : make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
      for (int u = 0; u < UN; ++u) {
        const uint32_t wd[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
        for (int e = 0; e < 8; ++e) a[e] += bf((wd[e >> 1] >> (16 * (e & 1))) & 0xffffu);
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e)
#pragma unroll
      for (int o = CPR; o < 64; o <<= 1) a[e] += __shfl_xor(a[e], o);
    if (sub == 0)
#pragma unroll
      for (int e = 0; e < 8; ++e) wsum[wv][c8 * 8 + e] = a[e];
    __syncthreads();
    if (tid < D) {
      float t = 0.0f;
      for (int i = 0; i < NWV; ++i) t += wsum[i][tid];
      vec[tid] = t / (float)n;
    }
    __syncthreads();
  }
  // (M u_j) . vec for group position j, in every lane of the row's lanes
  float gvec[8];
  auto take_vec = [&]() {
#pragma unroll
    for (int e = 0; e < 8; ++e) gvec[e] = vec[c8 * 8 + e];
  };
  // UN steps of rows: dots (M u_j) . vec for group positions
  // j0 + u STEP + sub, in every lane of each row's lanes
  auto row_dots = [&](int j0, float (&t)[UN]) {
    int idx[UN];
#pragma unroll
    for (int u = 0; u < UN; ++u) idx[u] = (j0 + u * STEP + sub < n) ? oin[j0 + u * STEP + sub] : -1;
    uint4 v[UN];
#pragma unroll
    for (int u = 0; u < UN; ++u)
      v[u] = idx[u] >= 0 ? *reinterpret_cast<const uint4*>(MU + (long long)idx[u] * D + c8 * 8)
                         : make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
    for (int u = 0; u < UN; ++u) {
      const uint32_t wd[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
      float x = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) x += bf((wd[e >> 1] >> (16 * (e & 1))) & 0xffffu) * gvec[e];
#pragma unroll
      for (int o = 1; o < CPR; o <<= 1) x += __shfl_xor(x, o);
      t[u] = x;
    }
  };
  // smallest (value, position) over the group; ties to the lower position
  auto argmin_pass = [&]() {
    take_vec();
    float best = INFINITY;
    int bj = 0x7fffffff;
    for (int j0 = wv * RPW; j0 < n; j0 += STEP * UN) {
      float t[UN];
      row_dots(j0, t);
#pragma unroll
      for (int u = 0; u < UN; ++u) {
        const int j = j0 + u * STEP + sub;
        if (j < n && t[u] < best) {
          best = t[u];
          bj = j;
        }
      }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float v2 = __shfl_xor(best, o);
      const int j2 = __shfl_xor(bj, o);
      if (v2 < best || (v2 == best && j2 < bj)) {
        best = v2;
        bj = j2;
      }
    }
    __syncthreads();
    if (lane == 0) {
      rv[wv] = best;
      ri[wv] = bj;
    }
    __syncthreads();
    float bv = rv[0];
    int bb = ri[0];
    for (int i = 1; i < NWV; ++i)
      if (rv[i] < bv || (rv[i] == bv && ri[i] < bb)) {
        bv = rv[i];
        bb = ri[i];
      }
    return bb;
  };
  auto set_vec = [&](int ja, int jb) {  // vec = u_jb - u_ja (jb < 0: u_ja)
    __syncthreads();
    if (tid < D) {
      const float xa = bf(U[(long long)oin[ja] * D + tid]);
      vec[tid] = (jb < 0) ? xa : bf(U[(long long)oin[jb] * D + tid]) - xa;
    }
    __syncthreads();
  };

  const int a = argmin_pass();  // least similar to the mean direction
  set_vec(a, -1);
  const int b = argmin_pass();  // least similar to a
  set_vec(a, b);                // u_b - u_a
  take_vec();
  for (int j0 = wv * RPW; j0 < n; j0 += STEP * UN) {
    float t[UN];
    row_dots(j0, t);
#pragma unroll
    for (int u = 0; u < UN; ++u) {
      const int j = j0 + u * STEP + sub;
      if (j < n && c8 == 0) keys[j] = order_bits(t[u]);
    }
  }
  __syncthreads();

  // Groups of at most NT rows: each row's rank (keys, then positions) by
  // comparison with every other row; the left child is the ranks < nl.
  if (n <= NT) {
    uint32_t* kl = hist;  // reused as the group's keys (n <= 256 here)
    const bool in = tid < n;
    const uint32_t key = in ? keys[tid] : 0u;
    if (NT == 256 && in) kl[tid] = key;
    __syncthreads();
    int rank = 0;
    if (in)
      for (int i = 0; i < n; ++i) {
        const uint32_t ki = (NT == 256) ? kl[i] : keys[i];
        rank += (ki < key || (ki == key && i < tid)) ? 1 : 0;
      }
    const bool left = in && rank < nl;
    const unsigned long long bl = __ballot(left);
    const unsigned long long lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    if (lane == 0) wc[1][wv] = __popcll(bl);
    __syncthreads();
    int loff = 0;
    for (int i = 0; i < wv; ++i) loff += wc[1][i];
    if (in) {
      const int lrank = loff + __popcll(bl & lt_mask);
      oout[left ? lrank : nl + (tid - lrank)] = oin[tid];
    }
    return;
  }

  // T = the nl-th smallest key (radix select, 8 bits at a time from the
  // top); `want` ends as its rank among the keys equal to T.
  uint32_t prefix = 0u;
  int want = nl - 1;
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int i = tid; i < 256; i += NT) hist[i] = 0u;
    __syncthreads();
    const uint32_t mask = (shift == 24) ? 0u : (~0u << (shift + 8));
    for (int j = tid; j < n; j += NT) {
      const uint32_t key = keys[j];
      if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (wv == 0) {
      const uint32_t h0 = hist[4 * lane], h1 = hist[4 * lane + 1], h2 = hist[4 * lane + 2], h3 = hist[4 * lane + 3];
      const int cnt = (int)(h0 + h1 + h2 + h3);
      int incl = cnt;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int t = __shfl_up(incl, o);
        if (lane >= o) incl += t;
      }
      const int excl = incl - cnt;
      if (excl <= want && want < incl) {
        int r = want - excl, d = 4 * lane;
        const uint32_t hs[4] = {h0, h1, h2, h3};
        for (int i = 0; i < 3 && r >= (int)hs[i]; ++i) {
          r -= (int)hs[i];
          ++d;
        }
        sel[0] = d;
        sel[1] = r;
      }
    }
    __syncthreads();
    prefix |= (uint32_t)sel[0] << shift;
    want = sel[1];
    __syncthreads();
  }
  const uint32_t T = prefix;

  // stable partition: keys < T, then the first want + 1 keys equal to T, go
  // left (nl rows); the rest go right
  int base_l = 0, base_e = 0;
  for (int j0 = 0; j0 < n; j0 += NT) {
    const int j = j0 + tid;
    const bool in = j < n;
    const uint32_t key = in ? keys[j] : 0xffffffffu;
    const bool eq = in && key == T;
    const unsigned long long be = __ballot(eq);
    const unsigned long long lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    const int erank_w = __popcll(be & lt_mask);
    if (lane == 0) wc[0][wv] = __popcll(be);
    __syncthreads();
    int eoff = 0, etot = 0;
    for (int i = 0; i < NWV; ++i) {
      if (i < wv) eoff += wc[0][i];
      etot += wc[0][i];
    }
    const bool left = in && (key < T || (eq && base_e + eoff + erank_w <= want));
    const unsigned long long bl = __ballot(left);
    const int lrank_w = __popcll(bl & lt_mask);
    if (lane == 0) wc[1][wv] = __popcll(bl);
    __syncthreads();
    int loff = 0, ltot = 0;
    for (int i = 0; i < NWV; ++i) {
      if (i < wv) loff += wc[1][i];
      ltot += wc[1][i];
    }
    if (in) {
      const int lrank = base_l + loff + lrank_w;  // left rows before j
      oout[left ? lrank : nl + (j - lrank)] = oin[j];
    }
    base_l += ltot;
    base_e += etot;
    __syncthreads();
  }
}

template <int D>
hipError_t partition_t(const Shape& s, const uint16_t* q, const uint16_t* k, const Workspace& ws,
                       hipStream_t stream) {
  hipLaunchKernelGGL(gram_kernel<D>, dim3(s.rb_chunks, s.rb_P), dim3(256), 0, stream, s, q, k, ws);
  hipLaunchKernelGGL(gram_reduce_kernel<D>, dim3((D * D + 255) / 256, s.rb_P), dim3(256), 0, stream, s, ws);
  if (s.rb_n > 0) {
    hipLaunchKernelGGL(embed_kernel<D>, dim3((s.rb_n + kEmbedRows - 1) / kEmbedRows, s.rb_P), dim3(256), 0, stream,
                       s, q, k, ws);
    int biggest = s.rb_n;  // largest group of the level (the all-left node)
    for (int level = 0; level < s.rb_levels; ++level) {
      if (biggest > 1024)
        hipLaunchKernelGGL((split_kernel<D, 1024>), dim3(1u << level, s.rb_P), dim3(1024), 0, stream, s, level, ws);
      else
        hipLaunchKernelGGL((split_kernel<D, 256>), dim3(1u << level, s.rb_P), dim3(256), 0, stream, s, level, ws);
      if (biggest > kRbBlock) biggest = kRbBlock * (((biggest + kRbBlock - 1) / kRbBlock + 1) / 2);
    }
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_reblock_partition(const Shape& s, const void* q, const void* k, const Workspace& ws,
                                    hipStream_t stream) {
  const auto* qq = static_cast<const uint16_t*>(q);
  const auto* kk = static_cast<const uint16_t*>(k);
  if (s.D == 128) return partition_t<128>(s, qq, kk, ws, stream);
  return partition_t<64>(s, qq, kk, ws, stream);
}


}  // namespace sa
