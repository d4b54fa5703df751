/*
 * sparse_attn.h -- C ABI of routed block-sparse attention for AMD MI355X.
 *
 * The method (Sol-style routing, as the Star7 "MiniMax H3 Activation Chunk &
 * Attention Acceleration" README describes it in section 工作原理 > Sol, and
 * the thakicloud "MiniMax-H3 ComfyUI accel stack" post in section
 * 이 기술은 무엇인가):
 *   1. Q, K and V are mean-pooled per 64-row block in FP32;
 *   2. every query block a is scored against every key block c with
 *      S[a][c] = Qbar_a . Kbar_c;
 *   3. key blocks are selected per query block either by a threshold
 *      S >= mean_a + tau * std_a (population std over all key blocks) or by
 *      a top-K ratio (comfyui-wiki "Spark-H3" news, 워크플로 section); key
 *      blocks holding rows of the packed prefix are always selected (exact KV
 *      sink) and query blocks holding prefix rows attend densely (Star7
 *      README, Sol; aikraft.ru Sol-Attn news, exact_kv_and_rows), or, with
 *      SA_FLAG_EXACT_KV_ONLY, are routed like the others (exact_kv);
 *   4. selected blocks are attended exactly (bf16 QK^T and PV on MFMA);
 *      every unselected block contributes once through its centroid,
 *      logit q_i . Kbar_c * scale + log(n_c), value Vbar_c, where n_c is the
 *      block's valid row count (log-mass bias, "Spark-H3" news,
 *      Spark-Reweight bullet); both kinds of term share one FP32 online
 *      softmax.
 * Optional modes (flags, each documented at its definition): Spark-Reweight
 * centroids (SA_FLAG_REWEIGHT), INT8 QK^T on the exact blocks
 * (SA_FLAG_INT8_QK) and the Spark-Reblock partition (SA_FLAG_REBLOCK).
 *
 * Tensors are bf16 in the BTHD layout [B, N, H, D] with D contiguous (the
 * layout of the aikraft.ru RTX 5090 table), D in {64, 128}.  A ragged last
 * block (N not a multiple of 64) holds N - 64 (n_b - 1) rows.
 *
 * Ownership: the caller owns every device buffer (q, k, v, out, workspace).
 * The library never allocates or frees device memory and never synchronises:
 * each call only enqueues kernels on the given HIP stream and returns.  A
 * plan is host memory owned by the library from sparse_attn_plan_create to
 * sparse_attn_plan_destroy; it may be reused for any number of calls with
 * the same shape and parameters, from any thread.
 *
 * Errors: every entry point returns 0 on success or a negative SA_E* code.
 * Host-detectable errors (bad arguments, wrong device, small workspace) are
 * reported before anything is launched.  sparse_attn_last_error() returns a
 * thread-local message for the last failing call on the calling thread.
 * There is no fallback: an unsupported device or shape is an error.  NaN or
 * Inf inputs are not checked; they propagate to the output.
 */
#ifndef SPARSE_ATTN_H
#define SPARSE_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SA_BLOCK 64          /* rows per query / key block */
#define SA_MAX_BLOCKS 2048   /* largest supported n_b = ceil(N / 64) */
#define SA_ABI_VERSION 6

/* Routing modes (sparse_attn_params.route). */
#define SA_ROUTE_TAU 0   /* S >= mean + tau * std; tau = -inf is the dense path */
#define SA_ROUTE_TOPK 1  /* keep k = clamp(ceil(r * n_b - 1e-6), 1, n_b) blocks */

/* Flags (sparse_attn_params.flags). */
#define SA_FLAG_CENTROID 1u /* unselected blocks contribute through centroids */
#define SA_FLAG_LOGMASS 2u  /* add log(n_c) to every centroid logit */
/* Prefix mode exact_kv (aikraft.ru Sol-Attn news, section
 * "Нововведения версии 2.0"): the prefix key blocks stay an exact sink for
 * every query block, but query blocks holding prefix rows are routed like
 * the others.  Without it (exact_kv_and_rows, the default) those query
 * blocks attend to every key block. */
#define SA_FLAG_EXACT_KV_ONLY 4u
/* Spark-Reweight (comfyui-wiki "Spark-H3" news, Spark-Reweight bullet and
 * the compression-branch figure caption): every centroid is the
 * anchor-weighted summary of its block instead of its mean, with a bias that
 * restores the block's mass, scored against one anchor per head, the mean of
 * the video query rows (rows >= prefix_len, all rows if there are none).
 * With x_j = anchor . k_j * scale over the block's rows and
 * w = softmax(x): Ktilde = sum w_j k_j, Vtilde = sum w_j v_j,
 * bias = logsumexp(x) - anchor . Ktilde * scale, used in place of log(n_c).
 * Requires SA_FLAG_CENTROID; routing still uses the block means. */
#define SA_FLAG_REWEIGHT 8u
/* INT8 QK^T on the exact blocks (thakicloud "MiniMax-H3 ComfyUI accel
 * stack" post, section on measured results: only each key block's residual
 * about its mean is quantised, the mean term stays bf16).  Reading:
 * base_c = bf16(fp32 mean of the block's keys); one scale per key block
 * s_c = max |k - base_c| / 127 over its valid rows; one scale per query row
 * s_q = max_d |q| / 127; codes rint(x / s) clipped to +-127, decided in fp32;
 * exact logit = scale * (q . base_c + s_q s_c (q8 . r8)).  Centroid logits
 * and P V are unchanged.  Without it (the default) QK^T is bf16. */
#define SA_FLAG_INT8_QK 16u
/* Spark-Reblock (comfyui-wiki "Spark-H3" news, Spark-Reblock bullet): an
 * input-dependent block partition per (b, h).  Reading: the query rows after
 * the prefix blocks are partitioned in the metric M = K^T K (the cosine of
 * their score patterns over the keys), and the keys and values reuse that
 * partition (the layout reblock_layout=q_reuse_k that the news's 워크플로
 * section says every shipped workflow pins; SA_FLAG_REBLOCK_KV_OWN gives the
 * keys a partition of their own instead).  Unit rows u = x / sqrt(x^T M x);
 * a group of n > 64 rows splits into a left child of 64 ceil(ceil(n/64) / 2)
 * rows and the rest: pivot a = the row least similar (u^T M ubar) to the
 * group's mean direction, pivot b = the row least similar to a, and the left
 * child takes the rows ranked first by u^T M (u_b - u_a), ties by position;
 * children keep their parent's order.  The path then runs on Q, K, V in the
 * new orders, reading their rows through the orders, and writes every
 * output row at its own position.  sparse_attn_forward only (the stage
 * calls reject it); off on the dense path, whose result does not depend on
 * the order. */
#define SA_FLAG_REBLOCK 32u
/* With SA_FLAG_REBLOCK: the separate layout, in which the key rows (with
 * their values) are partitioned on their own, in M = Q^T Q, by the same
 * rule.  Without it the keys and values reuse the query partition. */
#define SA_FLAG_REBLOCK_KV_OWN 64u
#define SA_FLAGS_DEFAULT (SA_FLAG_CENTROID | SA_FLAG_LOGMASS)

/* Error codes. */
#define SA_OK 0
#define SA_EINVAL (-1)              /* null pointer, bad parameter value */
#define SA_EUNSUPPORTED_SHAPE (-2)  /* D not 64/128, n_b > SA_MAX_BLOCKS, B*H*n_b > 2^30,
                                       H > 65535, B*ceil(H/8) > 65535,
                                       B*H (2*B*H with SA_FLAG_REBLOCK_KV_OWN)
                                       > 65535 with SA_FLAG_REBLOCK */
#define SA_EUNSUPPORTED_DEVICE (-3) /* current device is not gfx950 */
#define SA_EWORKSPACE (-4)          /* workspace smaller than required */
#define SA_EALIGN (-5)              /* pointer or stride not 16-byte aligned */
#define SA_ELAUNCH (-6)             /* a HIP launch or runtime call failed */

typedef struct sparse_attn_params {
  int32_t B, N, H, D;
  /* Element strides of q, k and v (which share them) and of out.  The
   * d-stride is 1.  All three zero means contiguous BTHD:
   * (N*H*D, H*D, D).  Otherwise each stride must be positive and a multiple
   * of 8 elements (16 bytes). */
  int64_t in_stride_b, in_stride_t, in_stride_h;
  int64_t out_stride_b, out_stride_t, out_stride_h;
  int32_t route;      /* SA_ROUTE_TAU or SA_ROUTE_TOPK */
  float tau;          /* SA_ROUTE_TAU: any value but NaN; +inf keeps only the sink */
  float topk_ratio;   /* SA_ROUTE_TOPK: in (0, 1] */
  int32_t prefix_len; /* 0..N: rows of the packed prefix (sink + dense rows) */
  float sm_scale;     /* softmax scale; <= 0 means 1/sqrt(D) */
  uint32_t flags;     /* SA_FLAG_* bits; SA_FLAGS_DEFAULT is the method */
} sparse_attn_params;

typedef struct sparse_attn_plan sparse_attn_plan; /* opaque, host memory */

/* Byte offsets of the workspace sections (all 256-byte aligned; a section
 * a plan does not use has size 0).  total_bytes also covers a last,
 * unlisted scratch section that sparse_attn_attend rewrites on every routed
 * call (the order in which the heads and each (b, h)'s pairs of query blocks
 * run).
 *
 * After sparse_attn_pool:
 *   qbar, kbar, vbar  fp32 [B, H, n_b, D]: the block means of Q, K, V.
 *   k_packed          bf16, one 64*D-element tile per (b, h, block): the
 *                     block's K rows (zero past N) in MFMA operand order,
 *                     as two 32-row half tiles; in a half tile, element
 *                     ((m*64 + l)*8 + e) holds
 *                     K[kappa(l % 32)][16 m + 8 (l / 32) + e], m < D/16,
 *                     where kappa(r) is r with bits 3 and 4 swapped.
 *   v_packed          bf16, same tiling for V^T: in a half tile, element
 *                     ((m*64 + l)*8 + e) with m = 2 dt + j holds
 *                     V[16 (e/4) + 8 j + 4 (l/32) + e % 4][32 dt + l % 32].
 *   kbar_packed,      bf16 centroids (the means rounded to nearest even;
 *   vbar_packed       with SA_FLAG_REWEIGHT the weighted summaries Ktilde,
 *                     Vtilde), [B, H, n_bp/32] half tiles in the same two
 *                     orders; block c is row c % 32 of half tile c / 32;
 *                     rows of blocks >= n_b are zero (n_bp = n_b rounded up
 *                     to 64).
 *   anchor            fp32 [B, H, D]: the reweight anchor (written only with
 *                     SA_FLAG_REWEIGHT, off the dense path).
 *   cbias             fp32 [B, H, n_bp]: the reweight centroid bias of each
 *                     block in log2 units (bias / ln 2); same condition.
 *   k_int8            int8, with SA_FLAG_INT8_QK only: per (b, h, block) two
 *                     half tiles of residual codes (zero past N); in a half
 *                     tile, byte ((t*64 + l)*16 + j) holds the code of
 *                     K[kappa(l % 32)][32 t + 16 (j/8) + 8 (l/32) + j % 8],
 *                     t < D/32 (the A operand of v_mfma_i32_32x32x32_i8).
 *   kbase             with SA_FLAG_INT8_QK only: per (b, h, block) a record
 *                     of D + 8 16-bit slots: the bf16 base row base_c, then
 *                     the fp32 block scale s_c in slots D, D + 1, then zero.
 * With SA_FLAG_REBLOCK only (problem p = side * B * H + b * H + h, side 0 =
 * query rows; side 1 = key rows exists with SA_FLAG_REBLOCK_KV_OWN only, so
 * P = B H problems, or 2 B H with it; n_v = N - 64 * prefix_blocks rows move):
 *   rb_gram           fp32 scratch: partial second moments, then (once M
 *                     is reduced) the partial sums and minima of the split
 *                     levels run over 1024-row chunks.
 *   rb_metric         fp32 [P, D, D]: M = Y^T Y of the other side.
 *   rb_units          bf16 [P, n_v, D]: the unit rows u of the moving rows.
 *   rb_munits         bf16 [P, n_v, D]: M u of the same rows (the split
 *                     compares rows through these).
 *   rb_order          int32 [2, P, n_v]: after sparse_attn_forward, buffer
 *                     reblock_levels % 2 holds the final order: new
 *                     position 64 * prefix_blocks + i holds row
 *                     64 * prefix_blocks + order[p][i].
 *   rb_keys           scratch.
 *   rb_qkv, rb_out    empty (no reordered copies are made).  After
 *                     sparse_attn_forward the sections above describe the
 *                     path in the new orders: block j of (b, h) holds the
 *                     rows at new positions 64 j .. 64 j + 63.
 * After sparse_attn_select:
 *   counts            int32 [B, H, n_b]: selected key blocks per query block.
 *   lists             int32 [B, H, n_b, n_b]: the selected key blocks in
 *                     ascending order in the first `count` entries of each
 *                     row (the rest of the row is unspecified). */
typedef struct sparse_attn_ws_layout {
  uint64_t total_bytes;
  uint64_t qbar, kbar, vbar;
  uint64_t k_packed, v_packed;
  uint64_t kbar_packed, vbar_packed;
  uint64_t counts, lists;
  uint64_t anchor, cbias;
  uint64_t k_int8, kbase;
  uint64_t rb_gram, rb_metric, rb_units, rb_munits, rb_order, rb_keys, rb_qkv, rb_out;
  int32_t n_blocks;        /* n_b */
  int32_t n_blocks_padded; /* n_bp */
  int32_t tail_rows;       /* valid rows of block n_b - 1 */
  int32_t prefix_blocks;   /* ceil(prefix_len / 64), capped at n_b */
  int32_t topk;            /* k of SA_ROUTE_TOPK, else 0 */
  int32_t dense;           /* 1 if tau = -inf: every block exact, no routing */
  int32_t reblock_levels;  /* levels of the Spark-Reblock split tree, else 0 */
} sparse_attn_ws_layout;

/* Validates *params (host only, touches no device) and creates a plan.
 * The Star7 README, section 环境与分发, describes the native library
 * boundary this follows: the library is handed tensor addresses, shapes and
 * the current stream only and links no PyTorch ABI; the plan is the host
 * record of shape, strides and routing those calls share.  (The call is
 * named sparse_attn_plan_create because sparse_attn_plan is the name of the
 * opaque plan type in C.)
 * params: read only, copied into the plan.  *plan: receives a plan owned by
 * the caller until sparse_attn_plan_destroy.
 * Returns SA_EINVAL / SA_EUNSUPPORTED_SHAPE / SA_EALIGN on bad input, in
 * which case *plan is set to NULL.  With the environment variable
 * SPARSE_ATTN_LOG=1 each plan prints one summary line on stderr (shape,
 * routing, prefix mode, flags, workspace size), in the spirit of the compact
 * verbose summary of the Star7 README, section 错误处理与日志. */
int sparse_attn_plan_create(const sparse_attn_params* params, sparse_attn_plan** plan);

/* Frees a plan (NULL is ignored).  Host only; no device memory is involved
 * (Star7 README, 环境与分发: the caller owns the tensors). */
void sparse_attn_plan_destroy(sparse_attn_plan* plan);

/* Fills *layout for the plan's shape (host only): the byte offsets of the
 * workspace sections described above.  Returns SA_EINVAL on NULL
 * arguments. */
int sparse_attn_workspace_layout(const sparse_attn_plan* plan, sparse_attn_ws_layout* layout);

/* *bytes = the device workspace a call with this plan needs
 * (layout.total_bytes; host only).  The caller allocates it (the library
 * never allocates device memory: Star7 README, 环境与分发, addresses only).
 * Returns SA_EINVAL on NULL arguments. */
int sparse_attn_workspace_bytes(const sparse_attn_plan* plan, size_t* bytes);

/* Full forward, the method of the Star7 README, section 工作原理 > Sol
 * (blockwise routing, exact selected blocks, centroids of the missed ones in
 * one FP32 softmax), across the boundary of its section 环境与分发
 * (addresses, shapes and the current stream; strict architecture check, no
 * fallback): pool, select and attend (pool and attend alone on the dense
 * path) enqueued on `stream` (a hipStream_t; NULL is the null stream); with
 * SA_FLAG_REBLOCK, first the partition, then the same steps reading the
 * rows of q, k, v through the new orders and writing each output row at its
 * own position.
 * q, k, v are read-only bf16 device pointers and may alias one another; out
 * is a bf16 device pointer that must not overlap them or ws.  ws points to at
 * least layout.total_bytes of device memory (256-byte aligned), ws_bytes is
 * its size; its contents on entry do not matter. */
int sparse_attn_forward(const sparse_attn_plan* plan, const void* q, const void* k, const void* v,
                        void* out, void* ws, size_t ws_bytes, void* stream);

/* Step 1 alone: block means of Q, K, V (Star7 README, 工作原理 > Sol: 64-row
 * Q and K blocks; Spark-H3 news, Spark-Reweight bullet: mean-pooled K/V
 * summaries) and the packed K, V^T and centroid tiles (every section listed
 * under "After sparse_attn_pool").  Arguments and errors as
 * sparse_attn_forward without out.  The stage
 * calls (pool, select, route, attend) refuse a SA_FLAG_REBLOCK plan with
 * SA_EINVAL: its steps run through sparse_attn_forward only. */
int sparse_attn_pool(const sparse_attn_plan* plan, const void* q, const void* k, const void* v,
                     void* ws, size_t ws_bytes, void* stream);

/* Steps 2-3 alone: scores every block pair from the pooled means already
 * in ws and writes counts and lists: threshold mean + tau * std of the
 * row's block scores (thakicloud accel-stack post, 이 기술은 무엇인가) or
 * top-K ratio (Spark-H3 news, 워크플로), the prefix key sink and dense prefix
 * query rows (Star7 README, Sol; aikraft.ru news, Нововведения версии 2.0).
 * Returns SA_EINVAL (NULL plan or ws), SA_EWORKSPACE, SA_EALIGN,
 * SA_EUNSUPPORTED_DEVICE or SA_ELAUNCH. */
int sparse_attn_select(const sparse_attn_plan* plan, void* ws, size_t ws_bytes, void* stream);

/* Steps 1-3: the routing of every query block (sparse_attn_pool followed
 * by sparse_attn_select; passages as cited there), leaving counts and lists
 * in ws for inspection or for sparse_attn_attend.  Same arguments and errors as sparse_attn_pool;
 * on the dense path it only pools (there is nothing to route). */
int sparse_attn_route(const sparse_attn_plan* plan, const void* q, const void* k, const void* v, void* ws,
                      size_t ws_bytes, void* stream);

/* Step 4 alone (Star7 README, 工作原理 > Sol: selected blocks exact, every
 * missed block through its centroid in the same FP32 softmax; Spark-H3 news,
 * Spark-Reweight bullet: the log-mass bias): exact attention over each query
 * block's list and centroid
 * terms for every other block, reading q and, from ws, the packed tiles,
 * counts and lists.  A caller may write its own lists: entries should be
 * distinct block indices in [0, n_b) (out-of-range entries are ignored and
 * a repeated entry counts once), counts in [0, n_b]; a query block whose
 * count is n_b gets no centroid term.  On the dense path lists are not
 * read. */
int sparse_attn_attend(const sparse_attn_plan* plan, const void* q, void* out, void* ws, size_t ws_bytes,
                       void* stream);

/* Largest workspace the allocation-free entry point can serve (bytes of
 * its per-device scratch array). */
#define SA_NOALLOC_SCRATCH_BYTES (128ull << 20)

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * computation as sparse_attn_forward, with the same arguments except the
 * workspace, which is a library-owned scratch array of
 * SA_NOALLOC_SCRATCH_BYTES bytes per device (held until the process ends).
 * The call allocates and frees nothing.  Plans whose workspace_bytes exceed
 * the array are refused with SA_EWORKSPACE before anything is launched.
 * Every call on a device shares that device's array: calls that overlap on
 * one device race, so serialise them (one stream, or events between
 * streams).  The array's contents on entry do not matter. */
int sparse_attn_forward_noalloc(const sparse_attn_plan* plan, const void* q, const void* k, const void* v,
                                void* out, void* stream);

/* Static message for an error code.  Errors are reported, never repaired:
 * the Star7 README, section 环境与分发, stops the job on an architecture
 * mismatch with an error naming the required and detected capability and
 * no fallback backend, and its section 错误处理与日志 runs strict modes with
 * no fallback. */
const char* sparse_attn_strerror(int code);

/* Thread-local detail of the last failing call on this thread ("" if none),
 * e.g. "requires gfx950, found gfx942": the required and the detected
 * architecture, as the Star7 README, section 环境与分发, asks of a mismatch.
 * Test hook: with SPARSE_ATTN_ARCH_OVERRIDE set to an architecture name
 * other than gfx950, every call that checks the device fails with
 * SA_EUNSUPPORTED_DEVICE naming that architecture, without touching any
 * device (the variable can only refuse, never admit a device). */
const char* sparse_attn_last_error(void);

/* SA_ABI_VERSION of the built library (compare with the header's). */
int sparse_attn_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SPARSE_ATTN_H */
