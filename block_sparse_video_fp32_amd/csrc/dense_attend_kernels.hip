// gfx950 kernel of the dense path of routed block-sparse attention
// (tau = -inf: every key block attended exactly, no routing, no centroids;
// Star7 README, 工作原理 > Sol, the exact-block attention with its FP32
// softmax, applied to every block).  It reads the packed K and V^T half
// tiles that pack_kv_kernel writes (layout in sparse_attn_kernels.hip) and
// computes, row for row, what attend_kernel computes when every key block
// is selected: the same MFMA sequences per accumulator, the same fixed
// softmax reference and the same recompute rule, so the two agree bit for
// bit; this kernel only arranges the work for the dense case, four query
// blocks per workgroup and 64 rows per wave.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "sa_internal.h"
#include "sparse_attn.h"

namespace sa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// float -> bf16 bits, round to nearest even (NaN kept quiet).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// s_waitcnt immediate: vmcnt(n) and lgkmcnt(0), expcnt untouched.
constexpr int wait_vm_lgkm0(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4); }

// Workgroup barrier that orders LDS accesses around it in the compiler but
// does not wait for outstanding global->LDS copies.
__device__ __forceinline__ void ring_barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Lane l's 16 bytes of 1 KB block blk of an LDS area: an MFMA operand.
__device__ __forceinline__ bf16x8 lds_frag(const uint8_t* area, int blk, int lane) {
  return *reinterpret_cast<const bf16x8*>(area + blk * 1024 + lane * 16);
}

// ---------------------------------------------------------------------------
// dense_attend: tau = -inf (every key block exact, no lists, no centroids),
// bf16 QK^T.  grid B * H * ceil(n_b / 4) (XCD-grouped like attend), 256
// threads: the workgroup takes four neighbouring query blocks of one (b, h)
// and wave w owns block 4 quad + w, all 64 rows, as two 32-row halves that
// share every K and V^T fragment read from LDS.  Every half tile of the
// sequence is needed by all four blocks, so one copy serves 256 query rows
// (twice the rows of the pair kernel) and one K or V^T fragment read serves
// 64.  Two waves run per SIMD: the accumulators of both halves (128 VGPRs)
// and the first half's Q fragments (32) stay in registers, the second
// half's Q fragments are read from LDS at every step (8 KB per wave).  Same
// ring, same packed tiles, same fixed softmax reference and recompute rule
// as attend, so each half does the same arithmetic in the same order as
// attend does for its rows.
// ---------------------------------------------------------------------------

// S^T of both halves against one half tile: each K fragment is read once
// and feeds two MFMAs; the second half's Q fragments come from LDS (qlds,
// 1 KB per k step, lane l at 16 l).
template <int NK>
__device__ __forceinline__ void tile_qk2(const uint8_t* stage, const uint8_t* qlds, int lane,
                                         const bf16x8 (&qa)[NK], f32x16& sa, f32x16& sb) {
  sa = f32x16{};
  sb = f32x16{};
  // fragments of step k + 1 are requested before the MFMAs of step k
  bf16x8 kf = lds_frag(stage, 0, lane), qf = lds_frag(qlds, 0, lane);
#pragma unroll
  for (int k = 0; k < NK; ++k) {
    bf16x8 kn = kf, qn = qf;
    if (k + 1 < NK) {
      kn = lds_frag(stage, k + 1, lane);
      qn = lds_frag(qlds, k + 1, lane);
    }
    sa = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qa[k], sa, 0, 0, 0);
    sb = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf, sb, 0, 0, 0);
    kf = kn;
    qf = qn;
  }
  // keep that order: two reads ahead of every pair of MFMAs
  __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
  for (int k = 0; k + 1 < NK; ++k) {
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
}

// P of one half: exp2(S^T a - mref) in bf16, 0 for the keys whose bit of
// kmask is set (keys past N: register i of a lane holds key
// key(8 (i/4) + 4 hh + i % 4) with bits 3 and 4 of the key swapped), and
// the row sums of the rounded P that the MFMAs use, two bf16 per
// v_dot2_f32_bf16 against (1, 1) in two chains.  Each pair of exponentials
// is rounded as soon as it exists, so that few fp32 values are live at
// once.
template <bool PLAIN>
__device__ __forceinline__ void tile_p(const f32x16& sacc, uint32_t kmask, float a, float mref, bf16x8 (&pb)[2],
                                       float (&lsum)[2]) {
  uint32_t wd[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float x = __builtin_amdgcn_exp2f(fmaf(sacc[2 * i], a, -mref));
    float y = __builtin_amdgcn_exp2f(fmaf(sacc[2 * i + 1], a, -mref));
    if (!PLAIN && ((kmask >> (2 * i)) & 1u)) x = 0.0f;
    if (!PLAIN && ((kmask >> (2 * i + 1)) & 1u)) y = 0.0f;
    const bf16x2 t = {(__bf16)x, (__bf16)y};
    wd[i] = __builtin_bit_cast(uint32_t, t);
  }
  const bf16x2 one2 = __builtin_bit_cast(bf16x2, 0x3f803f80u);
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    lsum[0] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, wd[4 * j]), one2, lsum[0], false);
    lsum[1] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, wd[4 * j + 1]), one2, lsum[1], false);
    lsum[0] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, wd[4 * j + 2]), one2, lsum[0], false);
    lsum[1] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, wd[4 * j + 3]), one2, lsum[1], false);
    pb[j] = __builtin_bit_cast(bf16x8, uint4{wd[4 * j], wd[4 * j + 1], wd[4 * j + 2], wd[4 * j + 3]});
  }
}

// Maximum logit of this lane's query over one half tile, keys in kmask left
// out.
__device__ __forceinline__ float tile_row_max_m(const f32x16& sacc, uint32_t kmask, float a) {
  float m = -INFINITY;
#pragma unroll
  for (int i = 0; i < 16; ++i)
    if (!((kmask >> i) & 1u)) m = fmaxf(m, sacc[i] * a);
  const auto p32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m), false, false);
  return fmaxf(__uint_as_float(p32[0]), __uint_as_float(p32[1]));
}

// O^T += V^T P^T for both halves: each V^T fragment is read once and feeds
// two MFMAs.
template <int NK>
__device__ __forceinline__ void tile_v2(const uint8_t* stage, int lane, const bf16x8 (&pa)[2],
                                        const bf16x8 (&pb)[2], f32x16 (&acca)[NK / 2], f32x16 (&accb)[NK / 2]) {
#pragma unroll
  for (int dt = 0; dt < NK / 2; ++dt)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const bf16x8 vf = lds_frag(stage, NK + 2 * dt + j, lane);
      acca[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pa[j], acca[dt], 0, 0, 0);
      accb[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pb[j], accb[dt], 0, 0, 0);
    }
}

// O^T += V^T P^T of half a while P of half b is formed: the MFMAs of one
// half and the exponentials of the other are independent, so they are
// written interleaved (one MFMA of half a, then one pair of half b's
// probabilities) and the VALU work can run in the shadow of the MFMAs.
// Half b's product follows, with its V^T fragments read again.  Per
// accumulator the order of the MFMAs, and of the row-sum terms, is that of
// tile_p and tile_v2.
template <int NK>
__device__ __forceinline__ void tile_pv_overlap(const uint8_t* stage, int lane, const bf16x8 (&pa)[2],
                                                const f32x16& sb, float a, float mref, bf16x8 (&pb)[2],
                                                float (&lb)[2], f32x16 (&acca)[NK / 2], f32x16 (&accb)[NK / 2]) {
  static_assert(NK == 8, "one MFMA of half a per probability pair of half b");
  uint32_t wd[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int dt = i >> 1, j = i & 1;
    const bf16x8 vf = lds_frag(stage, NK + 2 * dt + j, lane);
    acca[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pa[j], acca[dt], 0, 0, 0);
    const float x = __builtin_amdgcn_exp2f(fmaf(sb[2 * i], a, -mref));
    const float y = __builtin_amdgcn_exp2f(fmaf(sb[2 * i + 1], a, -mref));
    const bf16x2 t = {(__bf16)x, (__bf16)y};
    wd[i] = __builtin_bit_cast(uint32_t, t);
  }
  const bf16x2 one2 = __builtin_bit_cast(bf16x2, 0x3f803f80u);
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    lb[0] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, wd[4 * j]), one2, lb[0], false);
    lb[1] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, wd[4 * j + 1]), one2, lb[1], false);
    lb[0] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, wd[4 * j + 2]), one2, lb[0], false);
    lb[1] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, wd[4 * j + 3]), one2, lb[1], false);
    pb[j] = __builtin_bit_cast(bf16x8, uint4{wd[4 * j], wd[4 * j + 1], wd[4 * j + 2], wd[4 * j + 3]});
  }
  // half b: each V^T read one MFMA ahead
  bf16x8 vf = lds_frag(stage, NK, lane);
#pragma unroll
  for (int i = 0; i < NK; ++i) {
    bf16x8 vn = vf;
    if (i + 1 < NK) vn = lds_frag(stage, NK + i + 1, lane);
    accb[i >> 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pb[i & 1], accb[i >> 1], 0, 0, 0);
    vf = vn;
  }
  __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
  for (int i = 0; i + 1 < NK; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
}

// This wave's PER consecutive 1 KB blocks of one half tile, global -> LDS:
// lane l's 16 bytes of block i come from src + 1024 i + 16 l (bytes) and
// land at dst + 1024 i + 16 l (global_load_lds_dwordx4, LDS address in M0).
// Each copy's address is formed from the one pointer right before it, and
// no instruction offset is used, so that the LDS address is M0 + 16 l
// alone.  Written as asm so that the compiler does not wait for these
// copies before every LDS read; completion is established by the ring's
// explicit vmcnt waits and barriers.  M0 is saved and restored around each
// copy, with one wait state between its write and the copy.
template <int PER>
__device__ __forceinline__ void copy_blocks_seq(const uint16_t* src, uint32_t dst) {
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
        : "v"(src + 512 * i), "s"(dst + i * 1024)
        : "memory");
  }
}

template <int D, int S>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void dense_attend_kernel(
    Shape s, const uint16_t* __restrict__ q, uint16_t* __restrict__ out, Workspace ws) {
  constexpr int NK = D / 16, NDT = D / 32, NBLK = 2 * NK, PER = NBLK / 4, HT = 32 * D, STAGE = NBLK * 1024;
  extern __shared__ __attribute__((aligned(16))) uint8_t ring[];  // S * STAGE + 4 * NK * 1024 bytes
  __shared__ int flag;

  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, hh = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int G = gridDim.x, bid = blockIdx.x;
  const int xcd = bid & 7, kx = bid >> 3, qq = G >> 3, rr = G & 7;
  const int lid = (xcd < rr) ? xcd * (qq + 1) + kx : rr * (qq + 1) + (xcd - rr) * qq + kx;
  const int nb = s.nb, N = s.N;
  const float c1 = s.c1;
  const int nquad = (nb + 3) >> 2;
  const int bhi = lid / nquad;
  const int a = 4 * (lid % nquad) + w;  // this wave's query block
  const int h = bhi % s.H, b = bhi / s.H;
  const long long bh = bhi;
  const bool exists = a < nb;

  // Q^T B-operand fragments of both halves: lane l of half t holds
  // Q[64 a + 32 t + l % 32][16 k + 8 (l/32) .. +8]; half 1's go to this
  // wave's 8 KB of LDS after the ring.
  bf16x8 qa[NK];
  uint8_t* const qlds = ring + S * STAGE + w * NK * 1024;
  {
    const int r0 = a * kBlock + l32, r1 = r0 + 32;
    const uint16_t* qp = q + (long long)b * s.isb + (long long)h * s.ish + 8 * hh;
#pragma unroll
    for (int k = 0; k < NK; ++k) {
      uint4 v0 = make_uint4(0, 0, 0, 0), v1 = make_uint4(0, 0, 0, 0);
      if (exists && r0 < N) v0 = *reinterpret_cast<const uint4*>(qp + (long long)r0 * s.ist + 16 * k);
      if (exists && r1 < N) v1 = *reinterpret_cast<const uint4*>(qp + (long long)r1 * s.ist + 16 * k);
      qa[k] = __builtin_bit_cast(bf16x8, v0);
      *reinterpret_cast<uint4*>(qlds + k * 1024 + lane * 16) = v1;
    }
  }

  // Copies: waves 0, 1 the K blocks of a half tile, waves 2, 3 the V^T
  // blocks (as attend).
  const bool kwave = w < 2;
  const uint16_t* ex_bh =
      (kwave ? ws.kp : ws.vp) + bh * nb * 2LL * HT + ((w & 1) * PER * 64 + lane) * 8;
  const uint32_t my_dst =
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)ring + w * PER * 1024;
  const int TU = 2 * nb;
  // the last key block takes per-key terms (keys past N) when it is ragged
  const int nplain = (s.tail < kBlock) ? TU - 2 : TU;

  f32x16 acca[NDT], accb[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) acca[dt] = accb[dt] = f32x16{};
  float la[2] = {0.0f, 0.0f}, lb[2] = {0.0f, 0.0f};
  float mrefa = 0.0f, mrefb = 0.0f, mmaxa = -INFINITY, mmaxb = -INFINITY;
  bool safe = false;
  if (tid == 0) flag = 0;
  __syncthreads();

  int st = 0;
  auto copy_tile = [&](int v, int stg) { copy_blocks_seq<PER>(ex_bh + (long long)v * HT, my_dst + stg * STAGE); };
  auto ring_start = [&]() {
    st = 0;
#pragma unroll
    for (int k = 0; k < S - 1; ++k) copy_tile(min(k, TU - 1), k);
  };
  // half tile u + S - 1 (clamped, so that every step waits on the same
  // count) is requested into the stage that step u - 1 read
  auto ring_step = [&](int u) {
    __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0((S - 2) * PER));
    ring_barrier();
    copy_tile(min(u + S - 1, TU - 1), st == 0 ? S - 1 : st - 1);
  };
  auto ring_next = [&]() { st = (st == S - 1) ? 0 : st + 1; };
  // keys of half tile u past N, one bit per accumulator register (register
  // i of the lane holds key 16 ((i/4) % 2) + 8 (i/8) + 4 hh + i % 4: the
  // packed key order of the K half tiles)
  auto key_mask = [&](int u) -> uint32_t {
    const int nv = min(kBlock, N - (u >> 1) * kBlock) - 32 * (u & 1);  // valid keys
    uint32_t m = 0u;
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (16 * ((i >> 2) & 1) + 8 * (i >> 3) + 4 * hh + (i & 3) >= nv) m |= 1u << i;
    return m;
  };

  for (int attempt = 0; attempt < 2; ++attempt) {
    if (attempt == 1) {
      // exact row maxima over every half tile first
      ring_start();
      for (int u = 0; u < TU; ++u) {
        ring_step(u);
        if (exists) {
          f32x16 sa, sb;
          tile_qk2<NK>(ring + st * STAGE, qlds, lane, qa, sa, sb);
          const uint32_t km = key_mask(u);
          mmaxa = fmaxf(mmaxa, tile_row_max_m(sa, km, c1));
          mmaxb = fmaxf(mmaxb, tile_row_max_m(sb, km, c1));
        }
        ring_next();
      }
      __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(0));
      mrefa = (mmaxa == -INFINITY) ? 0.0f : mmaxa;
      mrefb = (mmaxb == -INFINITY) ? 0.0f : mmaxb;
      la[0] = la[1] = lb[0] = lb[1] = 0.0f;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) acca[dt] = accb[dt] = f32x16{};
      __syncthreads();
    }
    // The first half tile (it sets the reference) and the ragged last key
    // block take the key mask; the half tiles in between are plain.  The
    // three runs are written one after the other, not as a branch inside
    // one loop, which keeps the register allocation of the plain run tight.
    auto edge_step = [&](int u) {
      ring_step(u);
      if (exists) {
        const uint8_t* stage = ring + st * STAGE;
        f32x16 sa, sb;
        tile_qk2<NK>(stage, qlds, lane, qa, sa, sb);
        const uint32_t km = key_mask(u);
        if (u == 0 && !safe) {
          const float ma = tile_row_max_m(sa, km, c1), mb = tile_row_max_m(sb, km, c1);
          mrefa = (ma == -INFINITY) ? 0.0f : ma + 32.0f;
          mrefb = (mb == -INFINITY) ? 0.0f : mb + 32.0f;
        }
        bf16x8 pa[2], pb[2];
        tile_p<false>(sa, km, c1, mrefa, pa, la);
        tile_p<false>(sb, km, c1, mrefb, pb, lb);
        tile_v2<NK>(stage, lane, pa, pb, acca, accb);
      }
      ring_next();
    };
    ring_start();
    edge_step(0);
    int u = 1;
    for (; u < nplain; ++u) {
      ring_step(u);
      if (exists) {
        const uint8_t* stage = ring + st * STAGE;
        f32x16 sa, sb;
        tile_qk2<NK>(stage, qlds, lane, qa, sa, sb);
        bf16x8 pa[2], pb[2];
        tile_p<true>(sa, 0u, c1, mrefa, pa, la);
        if constexpr (NK == 8) {
          tile_pv_overlap<NK>(stage, lane, pa, sb, c1, mrefb, pb, lb, acca, accb);
        } else {
          tile_p<true>(sb, 0u, c1, mrefb, pb, lb);
          tile_v2<NK>(stage, lane, pa, pb, acca, accb);
        }
      }
      ring_next();
    }
    for (; u < TU; ++u) edge_step(u);
    __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(0));
    if (attempt == 1) break;
    bool bad = false;
    {
      const float pa_ = la[0] + la[1], pb_ = lb[0] + lb[1];
      const auto xa = __builtin_amdgcn_permlane32_swap(__float_as_uint(pa_), __float_as_uint(pa_), false, false);
      const auto xb = __builtin_amdgcn_permlane32_swap(__float_as_uint(pb_), __float_as_uint(pb_), false, false);
      const float ta = __uint_as_float(xa[0]) + __uint_as_float(xa[1]);
      const float tb = __uint_as_float(xb[0]) + __uint_as_float(xb[1]);
      bad = !(ta <= 0x1p100f) || !(tb <= 0x1p100f);
    }
    if (__ballot(bad) && lane == 0) flag = 1;
    __syncthreads();
    if (!__builtin_amdgcn_readfirstlane(flag)) break;
    safe = true;
  }

  // O = acc / l in bf16 (round to nearest even), rows below N only.
  auto store_half = [&](const f32x16 (&acc)[NDT], const float (&ls)[2], int r) {
    const float part = ls[0] + ls[1];
    const auto ps = __builtin_amdgcn_permlane32_swap(__float_as_uint(part), __float_as_uint(part), false, false);
    const float l = __uint_as_float(ps[0]) + __uint_as_float(ps[1]);
    const float inv = (l > 0.0f) ? 1.0f / l : 0.0f;
    if (!exists || r >= N) return;
    uint16_t* o = out + (long long)b * s.osb + (long long)h * s.osh + (long long)r * s.ost + 4 * hh;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        uint2 w2;
        w2.x = f32_to_bf16_bits(acc[dt][4 * j] * inv) | (f32_to_bf16_bits(acc[dt][4 * j + 1] * inv) << 16);
        w2.y = f32_to_bf16_bits(acc[dt][4 * j + 2] * inv) | (f32_to_bf16_bits(acc[dt][4 * j + 3] * inv) << 16);
        *reinterpret_cast<uint2*>(o + 32 * dt + 8 * j) = w2;
      }
  };
  store_half(acca, la, a * kBlock + l32);
  store_half(accb, lb, a * kBlock + 32 + l32);
}


template <int D, int S>
hipError_t launch_dense_t(const Shape& s, const uint16_t* q, uint16_t* out, const Workspace& ws,
                          hipStream_t stream) {
  constexpr int bytes = S * (D / 8) * 1024 + 4 * (D / 16) * 1024;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&dense_attend_kernel<D, S>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e != hipSuccess) return e;
  dim3 grid((unsigned)((long long)s.B * s.H * ((s.nb + 3) / 4)));
  hipLaunchKernelGGL((dense_attend_kernel<D, S>), grid, dim3(256), bytes, stream, s, q, out, ws);
  return hipGetLastError();
}


// Two ring stages, as attend: the next half tile is requested while the
// current one is computed.
constexpr int kDenseStages = 2;

}  // namespace

hipError_t launch_dense_attend(const Shape& s, const void* q, void* out, const Workspace& ws,
                               hipStream_t stream) {
  const auto* qq = static_cast<const uint16_t*>(q);
  auto* oo = static_cast<uint16_t*>(out);
  if (s.D == 128) return launch_dense_t<128, kDenseStages>(s, qq, oo, ws, stream);
  return launch_dense_t<64, kDenseStages>(s, qq, oo, ws, stream);
}

}  // namespace sa
