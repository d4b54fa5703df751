// Internal interface between the C-ABI host layer (sparse_attn_api.cpp) and
// the gfx950 kernels (sparse_attn_kernels.hip).  Not installed.
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

namespace sa {

constexpr int kBlock = 64;
constexpr int kGramChunk = 2048;  // rows per partial second moment (reblock)
constexpr int kEmbedRows = 1024;  // rows per embed workgroup (reblock)

// Everything a launch needs, derived once by the plan.
struct Shape {
  int B, N, H, D;
  long long isb, ist, ish;  // q/k/v element strides (d-stride 1)
  long long osb, ost, osh;  // out element strides
  int nb;                   // n_b = ceil(N / 64)
  int nbp;                  // n_b rounded up to 64
  int tail;                 // rows of block nb - 1
  int pb;                   // prefix blocks, <= nb
  int route;                // SA_ROUTE_TAU / SA_ROUTE_TOPK
  int topk;                 // k for top-K routing
  int dense;                // tau = -inf
  float tau;
  float c1;                 // softmax scale * log2(e)
  float bias_full;          // log2(64) when the log-mass bias is on, else 0
  float bias_tail;          // log2(tail) when on, else 0
  int centroid;             // centroid terms on
  int prefix_rows;          // query blocks holding prefix rows are dense
  int reweight;             // Spark-Reweight centroids (never on the dense path)
  float scale;              // softmax scale
  int prefix_len;
  int int8;                 // INT8 QK^T on the exact blocks
  int reblock;              // Spark-Reblock orders (never on the dense path)
  int rb_r0;                // first reordered row (prefix blocks stay)
  int rb_n;                 // reordered rows per (b, h), N - rb_r0
  int rb_levels;            // levels of the split tree
  int rb_chunks;            // partial second moments per problem
  int rb_P;                 // problems: B x H (shared layout) or 2 sides x B x H
  int rb_kv_own;            // keys and values take a partition of their own
  int permuted;             // the path reads Q, K, V rows (and writes output
                            // rows) through the final reblock orders
};

// Device workspace sections (see the layout notes in sparse_attn.h).
struct Workspace {
  float* qbar;    // [B,H,nb,D] fp32 block means
  float* kbar;
  float* vbar;
  uint16_t* kp;   // K of every block in MFMA fragment order, bf16
  uint16_t* vp;   // V^T of every block in MFMA fragment order, bf16
  uint16_t* kbp;  // centroids Kbar in the same packed order, bf16
  uint16_t* vbp;  // centroids Vbar^T in the same packed order, bf16
  int* counts;
  int* lists;
  float* anchor;  // [B,H,D] reweight anchor
  float* cbias;   // [B,H,nbp] reweight centroid bias, log2 units
  uint8_t* k8;     // [B,H,nb,2 half tiles] int8 residual codes, MFMA order
  uint16_t* kbase; // [B,H,nb] records: bf16 base row (D), fp32 scale, zero (D + 8 slots)
  float* rb_part;  // [P, chunks, D, D] partial second moments
  float* rb_M;     // [P, D, D] second moment of the other side
  uint16_t* rb_U;  // [P, rb_n, D] bf16 unit rows in the metric
  uint16_t* rb_MU; // [P, rb_n, D] bf16 M u of the unit rows
  int* rb_ord;     // [2, P, rb_n] orders (ping-pong by level)
  uint32_t* rb_key;  // [P, rb_n] rank keys
  int* pair_order;  // [B,H,ceil(nb/2)] pairs of each (b, h), longest lists first
  int* head_work;   // [B,H] total list length of each (b, h)
  int* head_order;  // [B,H] (b, h) of each head slot, balanced over the XCDs
};

hipError_t launch_pool_q(const Shape& s, const void* q, const Workspace& ws, hipStream_t stream);
hipError_t launch_anchor(const Shape& s, const void* q, const Workspace& ws, hipStream_t stream);
hipError_t launch_pack_kv(const Shape& s, const void* k, const void* v, const Workspace& ws,
                          hipStream_t stream);
hipError_t launch_select(const Shape& s, const Workspace& ws, hipStream_t stream);
hipError_t launch_reblock_partition(const Shape& s, const void* q, const void* k, const Workspace& ws,
                                    hipStream_t stream);
hipError_t launch_attend(const Shape& s, const void* q, void* out, const Workspace& ws,
                         hipStream_t stream);
// tau = -inf with bf16 QK^T (dense_attend_kernels.hip): four query blocks per
// workgroup, the same result as launch_attend bit for bit.
hipError_t launch_dense_attend(const Shape& s, const void* q, void* out, const Workspace& ws,
                               hipStream_t stream);

}  // namespace sa
