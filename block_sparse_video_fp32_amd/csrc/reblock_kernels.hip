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
//   embed_kernel       u_i = x_i / sqrt(x_i^T M x_i) in bf16 (the row norms
//                      from X M on MFMA with M rounded to bf16; M is
//                      symmetric, so its rows are the B operand) and the
//                      identity order
//   split_kernel       one level of the partition, one workgroup per group:
//                      the mean direction, the two pivots (least similar to
//                      the mean, then least similar to the first pivot), the
//                      rank keys (projection on M (u_b - u_a), position), an
//                      exact radix select of the left child's size and a
//                      stable two-way partition of the group's order
//   gather / scatter   Q, K, V rows into the new orders (contiguous copies
//                      in the workspace) and the output rows back
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
  for (int r0 = r_begin; r0 < r_end; r0 += kRbBlock) {
    __syncthreads();
    for (int i = tid; i < kRbBlock * (D / 8); i += 256) {
      const int r = i / (D / 8), c8 = i % (D / 8);
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (r0 + r < r_end) v = *reinterpret_cast<const uint4*>(y + (long long)(r0 + r) * s.ist + c8 * 8);
      const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) T[(c8 * 8 + e) * TP + r] = (uint16_t)((wv[e >> 1] >> (16 * (e & 1))) & 0xffffu);
    }
    __syncthreads();
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
// embed: grid (ceil(n_v / 256), problems), 256 threads, 64 rows at a time.
// (X M) on MFMA, times X, summed over each tile's columns by shuffles and
// over the column tiles in order: x^T M x per row; then the unit rows.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void embed_kernel(Shape s, const uint16_t* __restrict__ q,
                                                    const uint16_t* __restrict__ k, Workspace ws) {
  constexpr int LP = D + 8, TW = D / 64, NK = D / 16;
  __shared__ __attribute__((aligned(16))) uint16_t Mb[D * LP];
  __shared__ __attribute__((aligned(16))) uint16_t Xs[kRbBlock * LP];
  __shared__ float part[D / 32][kRbBlock];
  const int p = blockIdx.y;
  const Prob pr = prob_of(s, p);
  const uint16_t* x = rows_of(s, pr, q, k, false);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, hh = lane >> 5, l32 = lane & 31;
  const float* M = ws.rb_M + (long long)p * D * D;
  for (int i = tid; i < D * D; i += 256) Mb[(i / D) * LP + i % D] = (uint16_t)to_bf16(M[i]);
  const int nv = s.rb_n;
  uint16_t* U = ws.rb_U + (long long)p * nv * D;
  int* ord0 = ws.rb_ord + (long long)p * nv;
  const int rt = w & 1;
  const int jend = min(nv, (int)(blockIdx.x + 1) * kEmbedRows);
  for (int j0 = blockIdx.x * kEmbedRows; j0 < jend; j0 += kRbBlock) {
    __syncthreads();
    for (int i = tid; i < kRbBlock * (D / 8); i += 256) {
      const int r = i / (D / 8), c8 = i % (D / 8);
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (j0 + r < nv) v = *reinterpret_cast<const uint4*>(x + (long long)(s.rb_r0 + j0 + r) * s.ist + c8 * 8);
      *reinterpret_cast<uint4*>(Xs + r * LP + c8 * 8) = v;
    }
    __syncthreads();
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
      for (int i = 0; i < 16; ++i) {
        const int row = 32 * rt + 8 * (i >> 2) + 4 * hh + (i & 3);
        float v = acc[i] * bf(Xs[row * LP + 32 * ct + l32]);
#pragma unroll
        for (int o = 1; o < 32; o <<= 1) v += __shfl_xor(v, o);
        if (l32 == 0) part[ct][row] = v;
      }
    }
    __syncthreads();
    const int r = tid >> 2, qd = tid & 3;
    float n2 = 0.0f;
#pragma unroll
    for (int ct = 0; ct < D / 32; ++ct) n2 += part[ct][r];
    const float inv = n2 > 0.0f ? 1.0f / sqrtf(n2) : 0.0f;
    if (j0 + r < nv) {
#pragma unroll
      for (int d = qd * (D / 4); d < (qd + 1) * (D / 4); d += 8) {
        uint32_t wd[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          wd[e] = to_bf16(bf(Xs[r * LP + d + 2 * e]) * inv) | (to_bf16(bf(Xs[r * LP + d + 2 * e + 1]) * inv) << 16);
        *reinterpret_cast<uint4*>(U + (long long)(j0 + r) * D + d) = make_uint4(wd[0], wd[1], wd[2], wd[3]);
      }
      if (qd == 0) ord0[j0 + r] = j0 + r;
    }
  }
}

// Start and size of node g at depth `level` of the split tree of n rows
// (children: left 64 ceil(m/2) rows, right the rest; a node of <= 64 rows is
// a leaf and is carried by its all-left descendants, the others are empty).
__device__ __forceinline__ void group_range(int n, int level, int g, int& start, int& size) {
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

// Smallest (value, index) of the workgroup; index ties go to the lower one.
__device__ __forceinline__ int block_argmin(float v, int j, float* rv, int* ri) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float v2 = __shfl_xor(v, o);
    const int j2 = __shfl_xor(j, o);
    if (v2 < v || (v2 == v && j2 < j)) {
      v = v2;
      j = j2;
    }
  }
  __syncthreads();
  if ((tid & 63) == 0) {
    rv[tid >> 6] = v;
    ri[tid >> 6] = j;
  }
  __syncthreads();
  float bv = rv[0];
  int bj = ri[0];
  for (int i = 1; i < 4; ++i)
    if (rv[i] < bv || (rv[i] == bv && ri[i] < bj)) {
      bv = rv[i];
      bj = ri[i];
    }
  return bj;
}

// ---------------------------------------------------------------------------
// split: grid (2^level, problems), 256 threads.  Node g of the level reads
// its rows' order from buffer level & 1 and writes its children's order to
// buffer (level + 1) & 1.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void split_kernel(Shape s, int level, Workspace ws) {
  constexpr int CPR = D / 8;        // 16-byte chunks per row
  constexpr int RPP = 256 / CPR;    // rows per pass of the mean
  __shared__ float vec[D];
  __shared__ float gv[D];
  __shared__ float msum[RPP][D];
  __shared__ float rv[4];
  __shared__ int ri[4];
  __shared__ uint32_t hist[256];
  __shared__ int sel[2];
  __shared__ int wcount[4];
  const int g = blockIdx.x, p = blockIdx.y, nv = s.rb_n, tid = threadIdx.x;
  int start, n;
  group_range(nv, level, g, start, n);
  if (n == 0) return;
  const int* oin = ws.rb_ord + ((long long)(level & 1) * s.rb_P + p) * nv + start;
  int* oout = ws.rb_ord + ((long long)((level + 1) & 1) * s.rb_P + p) * nv + start;
  if (n <= kRbBlock) {
    for (int i = tid; i < n; i += 256) oout[i] = oin[i];
    return;
  }
  const int m = (n + kRbBlock - 1) / kRbBlock, nl = kRbBlock * ((m + 1) / 2);
  const uint16_t* U = ws.rb_U + (long long)p * nv * D;
  const float* M = ws.rb_M + (long long)p * D * D;
  unsigned long long* keys = ws.rb_key + (long long)p * nv + start;

  // mean direction
  {
    const int c8 = tid % CPR, rl = tid / CPR;
    float a[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int j = rl; j < n; j += RPP) {
      const uint4 v = *reinterpret_cast<const uint4*>(U + (long long)oin[j] * D + c8 * 8);
      const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) a[e] += bf((wv[e >> 1] >> (16 * (e & 1))) & 0xffffu);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) msum[rl][c8 * 8 + e] = a[e];
    __syncthreads();
    if (tid < D) {
      float t = 0.0f;
      for (int i = 0; i < RPP; ++i) t += msum[i][tid];
      vec[tid] = t / (float)n;
    }
    __syncthreads();
  }
  // gv = M vec
  auto matvec = [&]() {
    if (tid < D) {
      const float* mr = M + (long long)tid * D;
      float t = 0.0f;
      for (int e = 0; e < D; e += 4) {
        const float4 m4 = *reinterpret_cast<const float4*>(mr + e);
        t += m4.x * vec[e] + m4.y * vec[e + 1] + m4.z * vec[e + 2] + m4.w * vec[e + 3];
      }
      gv[tid] = t;
    }
    __syncthreads();
  };
  // dot of row j (group position) with gv
  auto row_dot = [&](int j) {
    const uint16_t* ur = U + (long long)oin[j] * D;
    float t = 0.0f;
#pragma unroll
    for (int c8 = 0; c8 < CPR; ++c8) {
      const uint4 v = *reinterpret_cast<const uint4*>(ur + c8 * 8);
      const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) t += bf((wv[e >> 1] >> (16 * (e & 1))) & 0xffffu) * gv[c8 * 8 + e];
    }
    return t;
  };
  auto load_row = [&](int j, float sign, bool add) {  // vec (+)= sign * u_j
    if (tid < D) {
      const float x = sign * bf(U[(long long)oin[j] * D + tid]);
      vec[tid] = add ? vec[tid] + x : x;
    }
    __syncthreads();
  };
  auto argmin_pass = [&]() {
    float best = INFINITY;
    int bj = 0x7fffffff;
    for (int j = tid; j < n; j += 256) {
      const float t = row_dot(j);
      if (t < best) {
        best = t;
        bj = j;
      }
    }
    return block_argmin(best, bj, rv, ri);
  };

  matvec();
  const int a = argmin_pass();  // least similar to the mean direction
  __syncthreads();
  load_row(a, 1.0f, false);
  matvec();
  const int b = argmin_pass();  // least similar to a
  __syncthreads();
  load_row(b, 1.0f, false);
  load_row(a, -1.0f, true);     // vec = u_b - u_a
  matvec();
  for (int j = tid; j < n; j += 256)
    keys[j] = ((unsigned long long)order_bits(row_dot(j)) << 32) | (unsigned long long)j;
  __syncthreads();

  // the nl-th smallest key: radix select, 8 bits at a time from the top
  unsigned long long prefix = 0ull;
  int want = nl - 1;
  for (int shift = 56; shift >= 0; shift -= 8) {
    hist[tid] = 0u;
    __syncthreads();
    const unsigned long long mask = (shift == 56) ? 0ull : (~0ull << (shift + 8));
    for (int j = tid; j < n; j += 256) {
      const unsigned long long key = keys[j];
      if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (tid == 0) {
      int cum = 0, d = 0;
      for (; d < 255; ++d) {
        if (cum + (int)hist[d] > want) break;
        cum += (int)hist[d];
      }
      sel[0] = d;
      sel[1] = want - cum;
    }
    __syncthreads();
    prefix |= (unsigned long long)sel[0] << shift;
    want = sel[1];
    __syncthreads();
  }
  const unsigned long long kstar = prefix;

  // stable partition: keys <= kstar (exactly nl of them) to the left
  int base_l = 0;
  const int lane = tid & 63, wv_ = tid >> 6;
  for (int j0 = 0; j0 < n; j0 += 256) {
    const int j = j0 + tid;
    const bool in = j < n;
    const bool left = in && keys[j] <= kstar;
    const unsigned long long bl = __ballot(left);
    const int rank_w = __popcll(bl & ((lane == 0) ? 0ull : (~0ull >> (64 - lane))));
    if (lane == 0) wcount[wv_] = __popcll(bl);
    __syncthreads();
    int off = 0;
    for (int i = 0; i < wv_; ++i) off += wcount[i];
    int tot = 0;
    for (int i = 0; i < 4; ++i) tot += wcount[i];
    if (in) {
      const int lrank = base_l + off + rank_w;  // left rows before j
      const int dst = left ? lrank : nl + (j - lrank);
      oout[dst] = oin[j];
    }
    base_l += tot;
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// gather: grid (N, B), 256 threads.  Row i of the reordered Q (K, V) is row
// perm(i) of the input: i itself in the prefix blocks, else the final order.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int perm_row(const Shape& s, const int* ord, int p, int i) {
  return (i < s.rb_r0) ? i : s.rb_r0 + ord[(long long)p * s.rb_n + (i - s.rb_r0)];
}

template <int D>
__global__ __launch_bounds__(256) void gather_kernel(Shape s, const uint16_t* __restrict__ q,
                                                     const uint16_t* __restrict__ k,
                                                     const uint16_t* __restrict__ v, Workspace ws) {
  constexpr int CPR = D / 8;
  const int i = blockIdx.x, b = blockIdx.y, BH = s.B * s.H;
  const int* ord = ws.rb_ord + (long long)(s.rb_levels & 1) * s.rb_P * s.rb_n;
  const int per = s.H * CPR;
  for (int c = threadIdx.x; c < 3 * per; c += 256) {
    const int tsel = c / per, rem = c % per, h = rem / CPR, c8 = rem % CPR;
    const int side = tsel == 0 ? 0 : 1;
    const int src = perm_row(s, ord, side * BH + b * s.H + h, i);
    const uint16_t* base = tsel == 0 ? q : (tsel == 1 ? k : v);
    uint16_t* dst = tsel == 0 ? ws.rb_q : (tsel == 1 ? ws.rb_k : ws.rb_v);
    const uint4 x = *reinterpret_cast<const uint4*>(base + (long long)b * s.isb + (long long)src * s.ist +
                                                    (long long)h * s.ish + c8 * 8);
    *reinterpret_cast<uint4*>(dst + (((long long)b * s.N + i) * s.H + h) * D + c8 * 8) = x;
  }
}

// scatter: grid (N, B).  Output row perm_q(i) <- row i of the reordered output.
template <int D>
__global__ __launch_bounds__(256) void scatter_kernel(Shape s, uint16_t* __restrict__ out, Workspace ws) {
  constexpr int CPR = D / 8;
  const int i = blockIdx.x, b = blockIdx.y;
  const int* ord = ws.rb_ord + (long long)(s.rb_levels & 1) * s.rb_P * s.rb_n;
  for (int c = threadIdx.x; c < s.H * CPR; c += 256) {
    const int h = c / CPR, c8 = c % CPR;
    const int dst = perm_row(s, ord, b * s.H + h, i);
    const uint4 x = *reinterpret_cast<const uint4*>(ws.rb_out + (((long long)b * s.N + i) * s.H + h) * D + c8 * 8);
    *reinterpret_cast<uint4*>(out + (long long)b * s.osb + (long long)dst * s.ost + (long long)h * s.osh + c8 * 8) = x;
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
    for (int level = 0; level < s.rb_levels; ++level)
      hipLaunchKernelGGL(split_kernel<D>, dim3(1u << level, s.rb_P), dim3(256), 0, stream, s, level, ws);
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

hipError_t launch_reblock_gather(const Shape& s, const void* q, const void* k, const void* v, const Workspace& ws,
                                 hipStream_t stream) {
  const auto* qq = static_cast<const uint16_t*>(q);
  const auto* kk = static_cast<const uint16_t*>(k);
  const auto* vv = static_cast<const uint16_t*>(v);
  if (s.D == 128)
    hipLaunchKernelGGL(gather_kernel<128>, dim3(s.N, s.B), dim3(256), 0, stream, s, qq, kk, vv, ws);
  else
    hipLaunchKernelGGL(gather_kernel<64>, dim3(s.N, s.B), dim3(256), 0, stream, s, qq, kk, vv, ws);
  return hipGetLastError();
}

hipError_t launch_reblock_scatter(const Shape& s, void* out, const Workspace& ws, hipStream_t stream) {
  auto* oo = static_cast<uint16_t*>(out);
  if (s.D == 128)
    hipLaunchKernelGGL(scatter_kernel<128>, dim3(s.N, s.B), dim3(256), 0, stream, s, oo, ws);
  else
    hipLaunchKernelGGL(scatter_kernel<64>, dim3(s.N, s.B), dim3(256), 0, stream, s, oo, ws);
  return hipGetLastError();
}

}  // namespace sa
