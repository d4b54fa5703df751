// gfx950 kernels of the Spark-Reblock partition (Spark-H3 news, Spark-Reblock
// bullet): the fixed 64-row tiles are replaced by an input-dependent
// partition per (b, h) and side, in which rows are alike when their score
// patterns over the other side are alike (the cosine in the metric of the
// other side's second moment), split top-down until every leaf holds one
// block.
//
// A "problem" p is one (side, b, h): side 0 partitions the query rows in the
// metric M = K^T K.  In the shared layout (reblock_layout=q_reuse_k, the one
// the Spark-H3 news's workflows pin) the keys and values reuse that
// partition and there are B H problems; with SA_FLAG_REBLOCK_KV_OWN side 1
// partitions the key rows (and with them the values) in M = Q^T Q, 2 B H
// problems.  Only the rows after the prefix blocks move (n_v of them).
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
//                      and a stable two-way partition of the group's order;
//                      groups of at most 8 or 16 row steps keep their M u
//                      rows in registers, so each row is read once a level
//   wide_pass_kernel,  the same level for levels with too few groups to fill
//   wide_select_kernel the chip: each pass spread over 1024-row chunks (the
//                      first level's mean comes from the embed's chunk
//                      sums), then one workgroup per group selects and
//                      partitions
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
constexpr int kWideRows = 1024;      // rows per chunk workgroup of a wide split level
constexpr int kWideMaxGroups = 128;  // a level is wide when groups x problems is below this

__device__ __forceinline__ float bf(uint32_t b) { return __uint_as_float(b << 16); }

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Two floats rounded to nearest-even bf16 by one v_cvt_pk_bf16_f32, packed
// as (lo | hi << 16).
__device__ __forceinline__ uint32_t bf16_pair(float lo, float hi) {
  const bf16x2 t = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, t);
}

__device__ __forceinline__ uint16_t to_bf16(float x) { return (uint16_t)(bf16_pair(x, 0.0f) & 0xffffu); }

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
// tiles (t / (D/32), t % (D/32)) for t = w, w + 4, ...  Each 64-row
// sub-chunk is staged row-major in LDS with 16-byte stores, and the MFMA
// operands A[i][k] = Y[k][32 ti + i] and B[k][j] = Y[k][32 tj + j] come out
// of it transposed by ds_read_b64_tr_b16: in each 16-lane group, lane 4a+e
// receives element e of the 8-byte pieces addressed by lanes a, a+4, a+8 and
// a+12 of the group.  So lane L = 16g + 4m + a addresses row k0 + 8(g/2) + m
// (k0 + 4 more for the upper half of the operand) at column
// 32 t + 16(g%2) + 4a, and every lane receives its operand's 8 rows of one
// column in k order.
// ---------------------------------------------------------------------------
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef short v8i16 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ bf16x8 lds_tr_frag(const uint16_t* p0, const uint16_t* p1) {
  const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)(p0));
  const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)(p1));
  const v8i16 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, v);
}

template <int D>
__global__ __launch_bounds__(256) void gram_kernel(Shape s, const uint16_t* __restrict__ q,
                                                   const uint16_t* __restrict__ k, Workspace ws) {
  constexpr int YP = D + 32;  // LDS pitch (elements): four consecutive rows cover all banks
  constexpr int NTD = D / 32;
  constexpr int TPW = NTD * NTD / 4;
  __shared__ __attribute__((aligned(16))) uint16_t Ys[kRbBlock * YP];
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
  // this lane's transposed-read address within a 16-row k step and a
  // 32-column tile
  const int g = lane >> 4, trow = 8 * (g >> 1) + ((lane >> 2) & 3), tcol = 16 * (g & 1) + 4 * (lane & 3);
  const int r_begin = c * kGramChunk, r_end = min(s.N, r_begin + kGramChunk);
  // each thread stages LPT 16-byte chunks of a sub-chunk; the sub-chunks
  // two ahead are loaded into registers (two register sets in turn) while
  // the current one is multiplied
  constexpr int LPT = kRbBlock * (D / 8) / 256;
  uint4 na[LPT], nb[LPT];
  auto fetch = [&](uint4(&dst)[LPT], int r0) {
#pragma unroll
    for (int u = 0; u < LPT; ++u) {
      const int i = tid + 256 * u, r = i / (D / 8), c8 = i % (D / 8);
      dst[u] = (r0 + r < r_end) ? *reinterpret_cast<const uint4*>(y + (long long)(r0 + r) * s.ist + c8 * 8)
                                : make_uint4(0u, 0u, 0u, 0u);
    }
  };
  auto step = [&](uint4(&cur)[LPT], int r0) {
    __syncthreads();
#pragma unroll
    for (int u = 0; u < LPT; ++u) {
      const int i = tid + 256 * u, r = i / (D / 8), c8 = i % (D / 8);
      *reinterpret_cast<uint4*>(Ys + r * YP + c8 * 8) = cur[u];
    }
    __syncthreads();
    if (r0 + 2 * kRbBlock < r_end) fetch(cur, r0 + 2 * kRbBlock);
#pragma unroll
    for (int kk = 0; kk < kRbBlock / 16; ++kk) {
      const uint16_t* base = Ys + (16 * kk + trow) * YP + tcol;
#pragma unroll
      for (int t = 0; t < TPW; ++t) {
        const bf16x8 a = lds_tr_frag(base + 32 * ti[t], base + 4 * YP + 32 * ti[t]);
        const bf16x8 b = lds_tr_frag(base + 32 * tj[t], base + 4 * YP + 32 * tj[t]);
        acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[t], 0, 0, 0);
      }
    }
  };
  if (r_begin < r_end) fetch(na, r_begin);
  if (r_begin + kRbBlock < r_end) fetch(nb, r_begin + kRbBlock);
  for (int r0 = r_begin; r0 < r_end; r0 += 2 * kRbBlock) {
    step(na, r0);
    if (r0 + kRbBlock < r_end) step(nb, r0 + kRbBlock);
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
#pragma unroll 8
  for (int c = 0; c < s.rb_chunks; ++c) m += part[(long long)c * D * D];  // loads batched, sums in order
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
                                                    const uint16_t* __restrict__ k, Workspace ws,
                                                    float* __restrict__ usum) {
  constexpr int LP = D + 8, TW = D / 64, NK = D / 16, QD = D / 4;
  __shared__ __attribute__((aligned(16))) uint16_t Mb[D * LP];
  __shared__ __attribute__((aligned(16))) uint16_t Xs[kRbBlock * LP];
  __shared__ __attribute__((aligned(16))) uint16_t Ys[kRbBlock * LP];
  const int p = blockIdx.y;
  const Prob pr = prob_of(s, p);
  const uint16_t* x = rows_of(s, pr, q, k, false);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, hh = lane >> 5, l32 = lane & 31;
  const float* M = ws.rb_M + (long long)p * D * D;
  {
    // M rounded to bf16 into LDS: every thread's 16-byte loads in flight at
    // once (one load at a time took tens of microseconds per workgroup)
    constexpr int MV = D * D / 4 / 256;
    float4 mv[MV];
#pragma unroll
    for (int u = 0; u < MV; ++u) mv[u] = reinterpret_cast<const float4*>(M)[tid + 256 * u];
#pragma unroll
    for (int u = 0; u < MV; ++u) {
      const int i = 4 * (tid + 256 * u), row = i / D, col = i % D;
      *reinterpret_cast<uint2*>(Mb + row * LP + col) = make_uint2(bf16_pair(mv[u].x, mv[u].y), bf16_pair(mv[u].z, mv[u].w));
    }
  }
  const int nv = s.rb_n;
  uint16_t* U = ws.rb_U + (long long)p * nv * D;
  uint16_t* MU = ws.rb_MU + (long long)p * nv * D;
  int* ord0 = ws.rb_ord + (long long)p * nv;
  const int rt = w & 1;
  const int jend = min(nv, (int)(blockIdx.x + 1) * kEmbedRows);
  // the sub-chunks two ahead are loaded into registers (two register sets
  // in turn) while the current one is processed
  constexpr int LPT = kRbBlock * (D / 8) / 256;
  uint4 na[LPT], nb[LPT];
  auto fetch = [&](uint4(&dst)[LPT], int j0) {
#pragma unroll
    for (int u = 0; u < LPT; ++u) {
      const int i = tid + 256 * u, r = i / (D / 8), c8 = i % (D / 8);
      dst[u] = (j0 + r < nv) ? *reinterpret_cast<const uint4*>(x + (long long)(s.rb_r0 + j0 + r) * s.ist + c8 * 8)
                             : make_uint4(0u, 0u, 0u, 0u);
    }
  };
  const int jbeg = blockIdx.x * kEmbedRows;
  if (jbeg < jend) fetch(na, jbeg);
  if (jbeg + kRbBlock < jend) fetch(nb, jbeg + kRbBlock);
  const int r = tid >> 2, qd = tid & 3;  // the row and quarter this thread finishes
  float us[QD];  // sum of this thread's bf16 u quarters (for usum)
#pragma unroll
  for (int d = 0; d < QD; ++d) us[d] = 0.0f;
  auto step = [&](uint4(&cur)[LPT], int j0) {
    __syncthreads();
#pragma unroll
    for (int u = 0; u < LPT; ++u) {
      const int i = tid + 256 * u, rr = i / (D / 8), c8 = i % (D / 8);
      *reinterpret_cast<uint4*>(Xs + rr * LP + c8 * 8) = cur[u];
    }
    __syncthreads();
    if (j0 + 2 * kRbBlock < jend) fetch(cur, j0 + 2 * kRbBlock);
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
          wu[e] = bf16_pair(xs[d + 2 * e] * inv, xs[d + 2 * e + 1] * inv);
          wm[e] = bf16_pair(ys[d + 2 * e] * inv, ys[d + 2 * e + 1] * inv);
          us[d + 2 * e] += bf(wu[e] & 0xffffu);
          us[d + 2 * e + 1] += bf(wu[e] >> 16);
        }
        *reinterpret_cast<uint4*>(U + (long long)(j0 + r) * D + qd * QD + d) = make_uint4(wu[0], wu[1], wu[2], wu[3]);
        *reinterpret_cast<uint4*>(MU + (long long)(j0 + r) * D + qd * QD + d) = make_uint4(wm[0], wm[1], wm[2], wm[3]);
      }
      if (qd == 0) ord0[j0 + r] = j0 + r;
    }
  };
  for (int j0 = jbeg; j0 < jend; j0 += 2 * kRbBlock) {
    step(na, j0);
    if (j0 + kRbBlock < jend) step(nb, j0 + kRbBlock);
  }
  // the chunk's sum of u (the bf16 values stored), for the mean direction
  // of a wide first split level: over the 16 rows of a wave, then the waves
  // in order
  if (usum != nullptr) {
#pragma unroll
    for (int d = 0; d < QD; ++d)
#pragma unroll
      for (int o = 4; o < 64; o <<= 1) us[d] += __shfl_xor(us[d], o);
    __syncthreads();
    float* red = reinterpret_cast<float*>(Xs);  // [4 waves][D]
    if (lane < 4)
#pragma unroll
      for (int d = 0; d < QD; ++d) red[w * D + qd * QD + d] = us[d];
    __syncthreads();
    if (tid < D)
      usum[((long long)p * gridDim.x + blockIdx.x) * D + tid] = red[tid] + red[D + tid] + red[2 * D + tid] + red[3 * D + tid];
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

// Stable two-way partition of a group's order (oin -> oout) by its rank
// keys: the nl rows of smallest (key, position) go left in position order,
// the others right.  T = the nl-th smallest key, by an exact radix select (8
// bits at a time from the top); `want` ends as the rank, among the keys equal
// to T, of the last one that goes left.  Each wave then walks a contiguous
// segment of positions twice: once to count its left rows and its keys equal
// to T, and, after one barrier, to place its rows.
template <int NT>
__device__ void select_partition(const uint32_t* __restrict__ keys, int n, int nl, const int* __restrict__ oin,
                                 int* __restrict__ oout, uint32_t* hist, int* sel, int (*wc)[NT / 64]) {
  constexpr int NWV = NT / 64;
  constexpr int UN = 4;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  uint32_t prefix = 0u;
  int want = nl - 1;
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int i = tid; i < 256; i += NT) hist[i] = 0u;
    __syncthreads();
    const uint32_t mask = (shift == 24) ? 0u : (~0u << (shift + 8));
    for (int j0 = tid; j0 < n; j0 += NT * UN) {
      uint32_t kk[UN];
#pragma unroll
      for (int u = 0; u < UN; ++u) kk[u] = (j0 + u * NT < n) ? keys[j0 + u * NT] : 0u;
#pragma unroll
      for (int u = 0; u < UN; ++u)
        if (j0 + u * NT < n && (kk[u] & mask) == prefix) atomicAdd(&hist[(kk[u] >> shift) & 255u], 1u);
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

  const int seg = (((n + NWV - 1) / NWV) + 63) & ~63;
  const int j0 = min(n, wv * seg), j1 = min(n, j0 + seg);
  const unsigned long long lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int cl = 0, ce = 0;
  for (int b0 = j0; b0 < j1; b0 += 64 * UN) {
    uint32_t kk[UN];
#pragma unroll
    for (int u = 0; u < UN; ++u) {
      const int j = b0 + 64 * u + lane;
      kk[u] = (j < j1) ? keys[j] : 0xffffffffu;
    }
#pragma unroll
    for (int u = 0; u < UN; ++u) {
      const bool in = b0 + 64 * u + lane < j1;
      cl += __popcll(__ballot(in && kk[u] < T));
      ce += __popcll(__ballot(in && kk[u] == T));
    }
  }
  if (lane == 0) {
    wc[0][wv] = cl;
    wc[1][wv] = ce;
  }
  __syncthreads();
  int L = 0, E = 0;
  for (int i = 0; i < wv; ++i) {
    L += wc[0][i];
    E += wc[1][i];
  }
  // L counts the rows below T before the segment; add the equal keys that
  // go left before it
  L += min(E, want + 1);
  for (int b0 = j0; b0 < j1; b0 += 64 * UN) {
    uint32_t kk[UN];
    int oi[UN];
#pragma unroll
    for (int u = 0; u < UN; ++u) {
      const int j = b0 + 64 * u + lane;
      kk[u] = (j < j1) ? keys[j] : 0xffffffffu;
      oi[u] = (j < j1) ? oin[j] : 0;
    }
#pragma unroll
    for (int u = 0; u < UN; ++u) {
      const int j = b0 + 64 * u + lane;
      const bool in = j < j1;
      const bool eq = in && kk[u] == T;
      const unsigned long long be = __ballot(eq);
      const bool left = in && (kk[u] < T || (eq && E + __popcll(be & lt_mask) <= want));
      const unsigned long long bl = __ballot(left);
      const int lrank = L + __popcll(bl & lt_mask);  // left rows before position j
      if (in) oout[left ? lrank : nl + (j - lrank)] = oi[u];
      L += __popcll(bl);
      E += __popcll(be);
    }
  }
}

// ---------------------------------------------------------------------------
// split: grid (2^level, problems), NT threads.  Node g of the level reads
// its rows' order from buffer level & 1 and writes its children's order to
// buffer (level + 1) & 1.  Rows are read D/8 lanes per row (one 16-byte
// chunk each), so a wave covers 64 / (D/8) rows per step and a lane keeps
// the 8 matching entries of the current vector in registers.  With KR > 0
// (groups of at most KR steps of rows) the mean pass also loads every row's
// M u chunk into registers, the two argmin passes and the key pass run from
// there, and the keys stay in LDS: each row is read from memory once per
// level.
// ---------------------------------------------------------------------------
template <int D, int NT, int KR>
__global__ __launch_bounds__(NT) void split_kernel(Shape s, int level, Workspace ws) {
  constexpr int CPR = D / 8;      // lanes per row
  constexpr int RPW = 64 / CPR;   // rows per wave step
  constexpr int NWV = NT / 64;    // waves
  constexpr int STEP = NWV * RPW;
  constexpr bool STASH = KR > 0;  // row steps held per lane
  constexpr int NK = STASH ? KR * STEP : 1;
  // Row loops take UN steps at a time: the order entries first, then the
  // rows, so that the loads of a step do not wait on the previous step.
  constexpr int UN = 4;
  __shared__ float vec[D];
  __shared__ float wsum[NWV][D];
  __shared__ float rv[NWV];
  __shared__ int ri[NWV];
  __shared__ uint32_t hist[256];
  __shared__ uint32_t kst[NK];
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

  uint4 mst[STASH ? KR : 1];  // M u chunks of rows wv RPW + sub + i STEP
  // mean direction ubar (fp32)
  {
    float a[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    auto add = [&](const uint4& v) {
      const uint32_t wd[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) a[e] += bf((wd[e >> 1] >> (16 * (e & 1))) & 0xffffu);
    };
    if constexpr (STASH) {
#pragma unroll
      for (int i0 = 0; i0 < KR; i0 += UN) {
        // positions past the group load its first row (in bounds) and are
        // left out of the sums and of every later pass
        int idx[UN];
#pragma unroll
        for (int u = 0; u < UN; ++u) {
          const int j = wv * RPW + sub + (i0 + u) * STEP;
          idx[u] = oin[j < n ? j : 0];
        }
        uint4 v[UN];
#pragma unroll
        for (int u = 0; u < UN; ++u) {
          v[u] = *reinterpret_cast<const uint4*>(U + (long long)idx[u] * D + c8 * 8);
          mst[i0 + u] = *reinterpret_cast<const uint4*>(MU + (long long)idx[u] * D + c8 * 8);
        }
#pragma unroll
        for (int u = 0; u < UN; ++u)
          if (wv * RPW + sub + (i0 + u) * STEP < n) add(v[u]);
        // keep the next steps' loads after these sums: only UN u chunks
        // are live at a time beside the stash
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
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
        for (int u = 0; u < UN; ++u) add(v[u]);
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
    // each pass converts the stashed bf16 afresh: without this the compiler
    // keeps the converted fp32 rows of all passes live (8 registers a row)
    if constexpr (STASH)
#pragma unroll
      for (int i = 0; i < KR; ++i) asm volatile("" : "+v"(mst[i].x), "+v"(mst[i].y), "+v"(mst[i].z), "+v"(mst[i].w));
  };
  auto dot = [&](const uint4& v) {
    const uint32_t wd[4] = {v.x, v.y, v.z, v.w};
    float x = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) x += bf((wd[e >> 1] >> (16 * (e & 1))) & 0xffffu) * gvec[e];
#pragma unroll
    for (int o = 1; o < CPR; o <<= 1) x += __shfl_xor(x, o);
    return x;
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
    for (int u = 0; u < UN; ++u) t[u] = dot(v[u]);
  };
  // smallest (value, position) over the group; ties to the lower position
  auto argmin_pass = [&]() {
    take_vec();
    float best = INFINITY;
    int bj = 0x7fffffff;
    if constexpr (STASH) {
#pragma unroll
      for (int i = 0; i < KR; ++i) {
        const float t = dot(mst[i]);
        const int j = wv * RPW + sub + i * STEP;
        if (j < n && t < best) {
          best = t;
          bj = j;
        }
        if ((i & 3) == 3) __builtin_amdgcn_sched_barrier(0);  // 4 rows' conversions live at a time
      }
    } else {
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
  // rank keys: in LDS with STASH, else in the workspace
  uint32_t* kout = STASH ? kst : keys;
  if constexpr (STASH) {
#pragma unroll
    for (int i = 0; i < KR; ++i) {
      const float t = dot(mst[i]);
      const int j = wv * RPW + sub + i * STEP;
      if (j < n && c8 == 0) kst[j] = order_bits(t);
      if ((i & 3) == 3) __builtin_amdgcn_sched_barrier(0);
    }
  } else {
    for (int j0 = wv * RPW; j0 < n; j0 += STEP * UN) {
      float t[UN];
      row_dots(j0, t);
#pragma unroll
      for (int u = 0; u < UN; ++u) {
        const int j = j0 + u * STEP + sub;
        if (j < n && c8 == 0) keys[j] = order_bits(t[u]);
      }
    }
  }
  __syncthreads();

  // Groups of at most 256 rows: each row's rank (keys, then positions) by
  // comparison with every other row; the left child is the ranks < nl.
  if (n <= 256) {
    uint32_t* kl = STASH ? kst : hist;
    const bool in = tid < n;
    const uint32_t key = in ? kout[tid] : 0u;
    if (!STASH) {
      if (in) kl[tid] = key;
      __syncthreads();
    }
    int rank = 0;
    if (in)
      for (int i = 0; i < n; ++i) {
        const uint32_t ki = kl[i];
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
  select_partition<NT>(kout, n, nl, oin, oout, hist, sel, wc);
}

// ---------------------------------------------------------------------------
// Wide split levels.  When a level has too few groups to fill the chip, each
// group's row passes are spread over chunk workgroups of kWideRows rows:
// grid (nch, 2^level, problems), 256 threads, one launch per pass.
//   phase 0  partial sums of u over the chunk
//   phase 1  the mean direction (the partials summed in chunk order), then
//            the chunk's smallest (M u_j) . ubar and its position
//   phase 2  a = the group's smallest of phase 1 (ties to the lower
//            position), then the chunk's smallest (M u_j) . u_a
//   phase 3  b likewise; the chunk's rank keys (M u_j) . (u_b - u_a)
// wide_select_kernel then selects and partitions each group.  The row dots
// are those of split_kernel, so only the mean's summation order differs
// from a level run by one workgroup per group.  The partials live in the
// rb_part section, which is free once M is reduced: sums [P][G][nch][D]
// fp32, then two minima arrays [P][G][nch] of (value bits, position).
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void wide_pass_kernel(Shape s, int level, int phase, int nch, Workspace ws) {
  constexpr int NT = 256, CPR = D / 8, RPW = 64 / CPR, NWV = NT / 64, STEP = NWV * RPW, UN = 4;
  __shared__ float vec[D];
  __shared__ float wsum[NWV][D];
  __shared__ float rv[NWV];
  __shared__ int ri[NWV];
  __shared__ int piv[2];
  const int c = blockIdx.x, g = blockIdx.y, p = blockIdx.z, G = gridDim.y, nv = s.rb_n, tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6, sub = lane / CPR, c8 = lane % CPR;
  int start, n;
  group_range(nv, level, g, start, n);
  if (n <= kRbBlock) return;  // leaves and empty nodes: the select kernel copies them
  const int nc = (n + kWideRows - 1) / kWideRows;
  if (c >= nc) return;
  const int r0 = c * kWideRows, r1 = min(n, r0 + kWideRows);
  const int* oin = ws.rb_ord + ((long long)(level & 1) * s.rb_P + p) * nv + start;
  const uint16_t* U = ws.rb_U + (long long)p * nv * D;
  const uint16_t* MU = ws.rb_MU + (long long)p * nv * D;
  const long long pg = (long long)p * G + g;
  float* sums = ws.rb_part + pg * nch * D;
  int2* mins = reinterpret_cast<int2*>(ws.rb_part + (long long)s.rb_P * G * nch * D);
  const long long mstride = (long long)s.rb_P * G * nch;

  if (phase == 0) {
    float a[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int j0 = r0 + wv * RPW + sub; j0 < r1; j0 += STEP * UN) {
      int idx[UN];
#pragma unroll
      for (int u = 0; u < UN; ++u) idx[u] = (j0 + u * STEP < r1) ? oin[j0 + u * STEP] : -1;
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
      sums[(long long)c * D + tid] = t;
    }
    return;
  }

  // the group's smallest (value, position) over the chunk minima of an
  // earlier phase; (value, position) pairs are distinct, so the result does
  // not depend on the order of the comparisons
  if (wv == 0) {
    for (int which = 0; which < phase - 1; ++which) {
      float best = INFINITY;
      int bj = 0x7fffffff;
      for (int i = lane; i < nc; i += 64) {
        const int2 e = mins[which * mstride + pg * nch + i];
        const float v = __int_as_float(e.x);
        if (v < best || (v == best && e.y < bj)) {
          best = v;
          bj = e.y;
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
      if (lane == 0) piv[which] = bj;
    }
  }
  __syncthreads();
  if (tid < D) {
    if (phase == 1) {
      float t = 0.0f;
#pragma unroll 8
      for (int i = 0; i < nc; ++i) t += sums[(long long)i * D + tid];  // loads batched, sums in order
      vec[tid] = t / (float)n;
    } else {
      const float xa = bf(U[(long long)oin[piv[0]] * D + tid]);
      vec[tid] = (phase == 2) ? xa : bf(U[(long long)oin[piv[1]] * D + tid]) - xa;
    }
  }
  __syncthreads();
  float gvec[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) gvec[e] = vec[c8 * 8 + e];
  float best = INFINITY;
  int bj = 0x7fffffff;
  uint32_t* keys = ws.rb_key + (long long)p * nv + start;
  for (int j0 = r0 + wv * RPW; j0 < r1; j0 += STEP * UN) {
    int idx[UN];
#pragma unroll
    for (int u = 0; u < UN; ++u) idx[u] = (j0 + u * STEP + sub < r1) ? oin[j0 + u * STEP + sub] : -1;
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
      const int j = j0 + u * STEP + sub;
      if (j < r1) {
        if (phase == 3) {
          if (c8 == 0) keys[j] = order_bits(x);
        } else if (x < best) {
          best = x;
          bj = j;
        }
      }
    }
  }
  if (phase == 3) return;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float v2 = __shfl_xor(best, o);
    const int j2 = __shfl_xor(bj, o);
    if (v2 < best || (v2 == best && j2 < bj)) {
      best = v2;
      bj = j2;
    }
  }
  if (lane == 0) {
    rv[wv] = best;
    ri[wv] = bj;
  }
  __syncthreads();
  if (tid == 0) {
    float bv = rv[0];
    int bb = ri[0];
    for (int i = 1; i < NWV; ++i)
      if (rv[i] < bv || (rv[i] == bv && ri[i] < bb)) {
        bv = rv[i];
        bb = ri[i];
      }
    mins[(phase - 1) * mstride + pg * nch + c] = make_int2(__float_as_int(bv), bb);
  }
}

// wide_select: grid (2^level, problems), NT threads: copies the leaves and
// partitions every other group of a wide level by the keys of phase 3.
template <int NT>
__global__ __launch_bounds__(NT) void wide_select_kernel(Shape s, int level, Workspace ws) {
  __shared__ uint32_t hist[256];
  __shared__ int sel[2];
  __shared__ int wc[2][NT / 64];
  const int g = blockIdx.x, p = blockIdx.y, nv = s.rb_n, tid = threadIdx.x;
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
  select_partition<NT>(ws.rb_key + (long long)p * nv + start, n, nl, oin, oout, hist, sel, wc);
}

template <int D>
hipError_t partition_t(const Shape& s, const uint16_t* q, const uint16_t* k, const Workspace& ws,
                       hipStream_t stream) {
  hipLaunchKernelGGL(gram_kernel<D>, dim3(s.rb_chunks, s.rb_P), dim3(256), 0, stream, s, q, k, ws);
  hipLaunchKernelGGL(gram_reduce_kernel<D>, dim3((D * D + 255) / 256, s.rb_P), dim3(256), 0, stream, s, ws);
  if (s.rb_n > 0) {
    const long long part_floats = (long long)s.rb_P * s.rb_chunks * D * D;
    // a level is wide when its groups leave most of the chip idle; its
    // partials then go to rb_part (free once M is reduced), which must hold
    // them
    auto is_wide = [&](int groups, int nch) {
      return groups * s.rb_P < kWideMaxGroups && nch >= 2 && (long long)s.rb_P * groups * nch * (D + 4) <= part_floats;
    };
    static_assert(kEmbedRows == kWideRows, "an embed workgroup sums one chunk of the first wide level");
    const int nch0 = (s.rb_n + kWideRows - 1) / kWideRows;
    const bool wide0 = s.rb_levels > 0 && is_wide(1, nch0);
    // with a wide first level the embed also writes its chunk sums of u (phase 0 of that level)
    hipLaunchKernelGGL(embed_kernel<D>, dim3(nch0, s.rb_P), dim3(256), 0, stream, s, q, k, ws,
                       wide0 ? ws.rb_part : nullptr);
    int biggest = s.rb_n;  // largest group of the level (the all-left node)
    // rows per step of a 256-thread split workgroup; groups of up to 8 or 16
    // steps keep their M u rows in registers
    constexpr int kStep256 = 4 * (64 / (D / 8));
    for (int level = 0; level < s.rb_levels; ++level) {
      const int groups = 1 << level, nch = (biggest + kWideRows - 1) / kWideRows;
      if (is_wide(groups, nch)) {
        for (int phase = level == 0 ? 1 : 0; phase < 4; ++phase)
          hipLaunchKernelGGL(wide_pass_kernel<D>, dim3(nch, groups, s.rb_P), dim3(256), 0, stream, s, level, phase,
                             nch, ws);
        hipLaunchKernelGGL(wide_select_kernel<1024>, dim3(groups, s.rb_P), dim3(1024), 0, stream, s, level, ws);
      } else if (biggest > 1024) {
        hipLaunchKernelGGL((split_kernel<D, 1024, 0>), dim3(1u << level, s.rb_P), dim3(1024), 0, stream, s, level, ws);
      } else if (biggest > 16 * kStep256) {
        hipLaunchKernelGGL((split_kernel<D, 256, 0>), dim3(1u << level, s.rb_P), dim3(256), 0, stream, s, level, ws);
      } else if (biggest > 8 * kStep256) {
        hipLaunchKernelGGL((split_kernel<D, 256, 16>), dim3(1u << level, s.rb_P), dim3(256), 0, stream, s, level, ws);
      } else {
        hipLaunchKernelGGL((split_kernel<D, 256, 8>), dim3(1u << level, s.rb_P), dim3(256), 0, stream, s, level, ws);
      }
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
