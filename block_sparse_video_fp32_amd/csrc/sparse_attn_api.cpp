// C-ABI host layer: parameter validation, plans, workspace layout, device
// check and the launch sequence.  The declarations and their contracts are
// in include/sparse_attn.h.
#include "sparse_attn.h"

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "sa_internal.h"

struct sparse_attn_plan {
  sparse_attn_params params;
  sa::Shape shape;
  sparse_attn_ws_layout layout;
  uint64_t order_off;  // attend dispatch order (after the public sections)
};

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int ok() {
  g_last_error.clear();
  return SA_OK;
}

uint64_t align256(uint64_t x) { return (x + 255) & ~uint64_t(255); }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Per-device result of the architecture check, filled on first use.
std::mutex g_dev_mu;
std::vector<int> g_dev_ok;            // 0 unknown, 1 gfx950, -1 other
std::vector<std::string> g_dev_arch;  // arch name as reported

// Test hook for the mismatch error: SPARSE_ATTN_ARCH_OVERRIDE=<name> makes
// the check report <name> as the detected architecture without querying any
// device.  It can only refuse: a value naming gfx950 is ignored and the real
// device is checked as usual.
const char* arch_override() {
  const char* o = std::getenv("SPARSE_ATTN_ARCH_OVERRIDE");
  if (!o || !*o || std::strncmp(o, "gfx950", 6) == 0) return nullptr;
  return o;
}

int check_device() {
  if (const char* o = arch_override())
    return fail(SA_EUNSUPPORTED_DEVICE, "requires gfx950, found %s (SPARSE_ATTN_ARCH_OVERRIDE)", o);
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0)
    return fail(SA_EUNSUPPORTED_DEVICE, "requires gfx950, found no HIP device (%s)",
                hipGetErrorString(e));
  std::lock_guard<std::mutex> lock(g_dev_mu);
  if ((int)g_dev_ok.size() <= dev) {
    g_dev_ok.resize(dev + 1, 0);
    g_dev_arch.resize(dev + 1);
  }
  if (g_dev_ok[dev] == 0) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess)
      return fail(SA_EUNSUPPORTED_DEVICE, "requires gfx950, device %d not queryable (%s)", dev,
                  hipGetErrorString(e));
    const char* name = prop.gcnArchName;
    g_dev_arch[dev] = name;
    g_dev_ok[dev] = (std::strncmp(name, "gfx950", 6) == 0 && (name[6] == 0 || name[6] == ':')) ? 1 : -1;
  }
  if (g_dev_ok[dev] != 1)
    return fail(SA_EUNSUPPORTED_DEVICE, "requires gfx950, found %s (device %d)",
                g_dev_arch[dev].c_str(), dev);
  return SA_OK;
}

int check_strides(const char* what, int64_t sb, int64_t st, int64_t sh) {
  if (sb <= 0 || st <= 0 || sh <= 0)
    return fail(SA_EINVAL, "%s strides must all be positive (or all zero for contiguous BTHD)", what);
  if ((sb % 8) || (st % 8) || (sh % 8))
    return fail(SA_EALIGN, "%s strides must be multiples of 8 elements (16 bytes)", what);
  return SA_OK;
}

int validate_params(const sparse_attn_params& p) {
  if (p.B < 1 || p.N < 1 || p.H < 1)
    return fail(SA_EINVAL, "B, N and H must be >= 1 (got B=%d N=%d H=%d)", p.B, p.N, p.H);
  if (p.D != 64 && p.D != 128)
    return fail(SA_EUNSUPPORTED_SHAPE, "head dim D must be 64 or 128 (got %d)", p.D);
  const int64_t nb = (int64_t(p.N) + sa::kBlock - 1) / sa::kBlock;
  if (nb > SA_MAX_BLOCKS)
    return fail(SA_EUNSUPPORTED_SHAPE, "N=%d gives %lld blocks, more than %d", p.N, (long long)nb,
                SA_MAX_BLOCKS);
  if ((int64_t)p.B * p.H * nb > (int64_t)1 << 30)
    return fail(SA_EUNSUPPORTED_SHAPE, "B*H*n_b too large");
  // grid y and z extents of the launches (at most 65535 each)
  if (p.H > 65535 || (int64_t)p.B * ((p.H + 7) / 8) > 65535)
    return fail(SA_EUNSUPPORTED_SHAPE, "B=%d, H=%d exceed the launch grid (H <= 65535, B*ceil(H/8) <= 65535)", p.B,
                p.H);
  if ((p.flags & SA_FLAG_REBLOCK_KV_OWN) && !(p.flags & SA_FLAG_REBLOCK))
    return fail(SA_EINVAL, "SA_FLAG_REBLOCK_KV_OWN needs SA_FLAG_REBLOCK");
  if ((p.flags & SA_FLAG_REBLOCK) &&
      ((p.flags & SA_FLAG_REBLOCK_KV_OWN) ? 2 : 1) * (int64_t)p.B * p.H > 65535)
    return fail(SA_EUNSUPPORTED_SHAPE, "SA_FLAG_REBLOCK needs %s <= 65535 (got B=%d, H=%d)",
                (p.flags & SA_FLAG_REBLOCK_KV_OWN) ? "2*B*H" : "B*H", p.B, p.H);
  const bool in0 = p.in_stride_b == 0 && p.in_stride_t == 0 && p.in_stride_h == 0;
  const bool out0 = p.out_stride_b == 0 && p.out_stride_t == 0 && p.out_stride_h == 0;
  int rc;
  if (!in0 && (rc = check_strides("input", p.in_stride_b, p.in_stride_t, p.in_stride_h))) return rc;
  if (!out0 && (rc = check_strides("output", p.out_stride_b, p.out_stride_t, p.out_stride_h))) return rc;
  if (p.route == SA_ROUTE_TAU) {
    if (std::isnan(p.tau)) return fail(SA_EINVAL, "tau must not be NaN");
  } else if (p.route == SA_ROUTE_TOPK) {
    if (!(p.topk_ratio > 0.0f && p.topk_ratio <= 1.0f))
      return fail(SA_EINVAL, "topk_ratio must be in (0, 1] (got %g)", (double)p.topk_ratio);
  } else {
    return fail(SA_EINVAL, "route must be SA_ROUTE_TAU or SA_ROUTE_TOPK (got %d)", p.route);
  }
  if (p.prefix_len < 0 || p.prefix_len > p.N)
    return fail(SA_EINVAL, "prefix_len must be in [0, N] (got %d, N=%d)", p.prefix_len, p.N);
  if (!std::isfinite(p.sm_scale)) return fail(SA_EINVAL, "sm_scale must be finite");
  if ((p.flags & SA_FLAG_REWEIGHT) && !(p.flags & SA_FLAG_CENTROID))
    return fail(SA_EINVAL, "SA_FLAG_REWEIGHT needs SA_FLAG_CENTROID");
  if (p.flags &
      ~(SA_FLAG_CENTROID | SA_FLAG_LOGMASS | SA_FLAG_EXACT_KV_ONLY | SA_FLAG_REWEIGHT | SA_FLAG_INT8_QK |
        SA_FLAG_REBLOCK | SA_FLAG_REBLOCK_KV_OWN))
    return fail(SA_EINVAL, "unknown flag bits 0x%x", p.flags);
  return SA_OK;
}

void build_plan(sparse_attn_plan* pl) {
  const sparse_attn_params& p = pl->params;
  sa::Shape& s = pl->shape;
  s.B = p.B;
  s.N = p.N;
  s.H = p.H;
  s.D = p.D;
  const bool in0 = p.in_stride_b == 0 && p.in_stride_t == 0 && p.in_stride_h == 0;
  const bool out0 = p.out_stride_b == 0 && p.out_stride_t == 0 && p.out_stride_h == 0;
  const long long hd = (long long)p.H * p.D;
  s.isb = in0 ? hd * p.N : p.in_stride_b;
  s.ist = in0 ? hd : p.in_stride_t;
  s.ish = in0 ? p.D : p.in_stride_h;
  s.osb = out0 ? hd * p.N : p.out_stride_b;
  s.ost = out0 ? hd : p.out_stride_t;
  s.osh = out0 ? p.D : p.out_stride_h;
  s.nb = (p.N + sa::kBlock - 1) / sa::kBlock;
  s.nbp = (s.nb + 63) / 64 * 64;
  s.tail = p.N - sa::kBlock * (s.nb - 1);
  s.pb = (p.prefix_len + sa::kBlock - 1) / sa::kBlock;
  if (s.pb > s.nb) s.pb = s.nb;
  s.route = p.route;
  s.tau = p.tau;
  s.dense = (p.route == SA_ROUTE_TAU && std::isinf(p.tau) && p.tau < 0) ? 1 : 0;
  s.topk = 0;
  if (p.route == SA_ROUTE_TOPK) {
    // k = clamp(ceil(r * n_b - 1e-6), 1, n_b) with r the float32 ratio.
    double k = std::ceil((double)p.topk_ratio * s.nb - 1e-6);
    if (k < 1) k = 1;
    if (k > s.nb) k = s.nb;
    s.topk = (int)k;
  }
  const double scale = p.sm_scale > 0.0f ? (double)p.sm_scale : 1.0 / std::sqrt((double)p.D);
  s.c1 = (float)(scale * 1.4426950408889634);  // log2(e)
  const bool logmass = (p.flags & SA_FLAG_LOGMASS) != 0;
  s.bias_full = logmass ? 6.0f : 0.0f;  // log2(64)
  s.bias_tail = logmass ? (float)std::log2((double)s.tail) : 0.0f;
  s.centroid = (p.flags & SA_FLAG_CENTROID) ? 1 : 0;
  s.prefix_rows = (p.flags & SA_FLAG_EXACT_KV_ONLY) ? 0 : 1;
  s.reweight = ((p.flags & SA_FLAG_REWEIGHT) && !s.dense) ? 1 : 0;
  s.scale = (float)scale;
  s.prefix_len = p.prefix_len;
  s.int8 = (p.flags & SA_FLAG_INT8_QK) ? 1 : 0;
  // Spark-Reblock: the rows after the prefix blocks are reordered; the split
  // tree of n rows has ceil(log2(ceil(n / 64))) levels.
  s.reblock = ((p.flags & SA_FLAG_REBLOCK) && !s.dense) ? 1 : 0;
  s.rb_r0 = s.pb * sa::kBlock < p.N ? s.pb * sa::kBlock : p.N;
  s.rb_n = p.N - s.rb_r0;
  s.rb_levels = 0;
  for (int m = (s.rb_n + sa::kBlock - 1) / sa::kBlock; (1 << s.rb_levels) < m;) ++s.rb_levels;
  s.rb_chunks = (p.N + sa::kGramChunk - 1) / sa::kGramChunk;
  s.rb_kv_own = (p.flags & SA_FLAG_REBLOCK_KV_OWN) ? 1 : 0;
  s.rb_P = (s.rb_kv_own ? 2 : 1) * p.B * p.H;
  s.permuted = 0;

  sparse_attn_ws_layout& L = pl->layout;
  std::memset(&L, 0, sizeof(L));
  const uint64_t bh = (uint64_t)p.B * p.H;
  const uint64_t pooled = bh * s.nb * p.D * sizeof(float);
  const uint64_t packed = bh * s.nb * 64ull * p.D * sizeof(uint16_t);
  const uint64_t cpacked = bh * s.nbp * (uint64_t)p.D * sizeof(uint16_t);
  uint64_t off = 0;
  L.qbar = off; off = align256(off + pooled);
  L.kbar = off; off = align256(off + pooled);
  L.vbar = off; off = align256(off + pooled);
  L.k_packed = off; off = align256(off + packed);
  L.v_packed = off; off = align256(off + packed);
  L.kbar_packed = off; off = align256(off + cpacked);
  L.vbar_packed = off; off = align256(off + cpacked);
  L.counts = off; off = align256(off + bh * s.nb * sizeof(int32_t));
  L.lists = off; off = align256(off + bh * s.nb * (uint64_t)s.nb * sizeof(int32_t));
  L.anchor = off; off = align256(off + bh * p.D * sizeof(float));
  L.cbias = off; off = align256(off + bh * s.nbp * sizeof(float));
  L.k_int8 = off; off = align256(off + (s.int8 ? bh * s.nb * 64ull * p.D : 0));
  L.kbase = off; off = align256(off + (s.int8 ? bh * s.nb * (uint64_t)(p.D + 8) * sizeof(uint16_t) : 0));
  const uint64_t rb = s.reblock ? 1 : 0;
  const uint64_t P = (uint64_t)s.rb_P, dd = (uint64_t)p.D * p.D;
  L.rb_gram = off; off = align256(off + rb * P * s.rb_chunks * dd * sizeof(float));
  L.rb_metric = off; off = align256(off + rb * P * dd * sizeof(float));
  L.rb_units = off; off = align256(off + rb * P * s.rb_n * (uint64_t)p.D * sizeof(uint16_t));
  L.rb_munits = off; off = align256(off + rb * P * s.rb_n * (uint64_t)p.D * sizeof(uint16_t));
  L.rb_order = off; off = align256(off + rb * 2 * P * s.rb_n * sizeof(int32_t));
  L.rb_keys = off; off = align256(off + rb * P * s.rb_n * sizeof(uint32_t));
  // rb_qkv, rb_out: no reordered copies (the path reads through the orders)
  L.rb_qkv = off;
  L.rb_out = off;
  pl->order_off = off; off = align256(off + (bh * (uint64_t)((s.nb + 1) / 2) + 2 * bh) * sizeof(int32_t));
  L.total_bytes = off;
  L.n_blocks = s.nb;
  L.n_blocks_padded = s.nbp;
  L.tail_rows = s.tail;
  L.prefix_blocks = s.pb;
  L.topk = s.topk;
  L.dense = s.dense;
  L.reblock_levels = s.reblock ? s.rb_levels : 0;
}

sa::Workspace carve(const sparse_attn_plan* pl, void* ws) {
  char* base = static_cast<char*>(ws);
  const sparse_attn_ws_layout& L = pl->layout;
  sa::Workspace w;
  w.qbar = reinterpret_cast<float*>(base + L.qbar);
  w.kbar = reinterpret_cast<float*>(base + L.kbar);
  w.vbar = reinterpret_cast<float*>(base + L.vbar);
  w.kp = reinterpret_cast<uint16_t*>(base + L.k_packed);
  w.vp = reinterpret_cast<uint16_t*>(base + L.v_packed);
  w.kbp = reinterpret_cast<uint16_t*>(base + L.kbar_packed);
  w.vbp = reinterpret_cast<uint16_t*>(base + L.vbar_packed);
  w.counts = reinterpret_cast<int*>(base + L.counts);
  w.lists = reinterpret_cast<int*>(base + L.lists);
  w.anchor = reinterpret_cast<float*>(base + L.anchor);
  w.cbias = reinterpret_cast<float*>(base + L.cbias);
  w.k8 = reinterpret_cast<uint8_t*>(base + L.k_int8);
  w.kbase = reinterpret_cast<uint16_t*>(base + L.kbase);
  w.rb_part = reinterpret_cast<float*>(base + L.rb_gram);
  w.rb_M = reinterpret_cast<float*>(base + L.rb_metric);
  w.rb_U = reinterpret_cast<uint16_t*>(base + L.rb_units);
  w.rb_MU = reinterpret_cast<uint16_t*>(base + L.rb_munits);
  w.rb_ord = reinterpret_cast<int*>(base + L.rb_order);
  w.rb_key = reinterpret_cast<uint32_t*>(base + L.rb_keys);
  w.pair_order = reinterpret_cast<int*>(base + pl->order_off);
  const uint64_t nbh = (uint64_t)pl->params.B * pl->params.H;
  w.head_work = w.pair_order + nbh * (uint64_t)((pl->shape.nb + 1) / 2);
  w.head_order = w.head_work + nbh;
  return w;
}

int check_ws(const sparse_attn_plan* pl, void* ws, size_t ws_bytes) {
  if (!ws) return fail(SA_EINVAL, "workspace pointer is NULL");
  if (reinterpret_cast<uintptr_t>(ws) & 255u)
    return fail(SA_EALIGN, "workspace must be 256-byte aligned");
  if (ws_bytes < pl->layout.total_bytes)
    return fail(SA_EWORKSPACE, "workspace has %zu bytes, plan needs %llu", ws_bytes,
                (unsigned long long)pl->layout.total_bytes);
  return SA_OK;
}

int check_tensors(const void* q, const void* k, const void* v, const void* out, bool need_out) {
  if (!q || !k || !v || (need_out && !out)) return fail(SA_EINVAL, "q, k, v and out must be non-NULL");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || (need_out && !aligned16(out)))
    return fail(SA_EALIGN, "q, k, v and out must be 16-byte aligned");
  return SA_OK;
}

// SPARSE_ATTN_LOG=1: one compact line per plan on stderr (shape, routing,
// flags, blocks, workspace), so that a run shows what each call does without
// per-call output.
bool log_on() {
  static const bool on = [] {
    const char* v = std::getenv("SPARSE_ATTN_LOG");
    return v && *v && std::strcmp(v, "0") != 0;
  }();
  return on;
}

void log_plan(const sparse_attn_plan* pl) {
  if (!log_on()) return;
  const sparse_attn_params& p = pl->params;
  const sa::Shape& s = pl->shape;
  char route[64];
  if (s.dense)
    std::snprintf(route, sizeof(route), "dense (tau=-inf)");
  else if (p.route == SA_ROUTE_TOPK)
    std::snprintf(route, sizeof(route), "topk %.4g (k=%d)", (double)p.topk_ratio, s.topk);
  else
    std::snprintf(route, sizeof(route), "tau %.4g", (double)p.tau);
  std::fprintf(stderr,
               "sparse_attn: plan B=%d N=%d H=%d D=%d n_b=%d tail=%d | %s | prefix %d rows (%d blocks, %s) | "
               "centroid %d logmass %d reweight %d int8_qk %d reblock %d (%s, %d levels) | scale %.6g | "
               "workspace %.1f MiB\n",
               p.B, p.N, p.H, p.D, s.nb, s.tail, route, p.prefix_len, s.pb,
               s.prefix_rows ? "exact_kv_and_rows" : "exact_kv", s.centroid, (p.flags & SA_FLAG_LOGMASS) ? 1 : 0,
               s.reweight, s.int8, s.reblock, s.rb_kv_own ? "separate" : "q_reuse_k", s.reblock ? s.rb_levels : 0,
               (double)s.scale,
               (double)pl->layout.total_bytes / (1024.0 * 1024.0));
  std::fflush(stderr);
}

int launched(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(SA_ELAUNCH, "%s launch failed: %s", what, hipGetErrorString(e));
  return SA_OK;
}

}  // namespace

extern "C" {

int sparse_attn_abi_version(void) { return SA_ABI_VERSION; }

const char* sparse_attn_strerror(int code) {
  switch (code) {
    case SA_OK: return "success";
    case SA_EINVAL: return "invalid argument";
    case SA_EUNSUPPORTED_SHAPE: return "unsupported shape";
    case SA_EUNSUPPORTED_DEVICE: return "unsupported device (requires gfx950)";
    case SA_EWORKSPACE: return "workspace too small";
    case SA_EALIGN: return "misaligned pointer or stride";
    case SA_ELAUNCH: return "kernel launch failed";
    default: return "unknown error";
  }
}

const char* sparse_attn_last_error(void) { return g_last_error.c_str(); }

int sparse_attn_plan_create(const sparse_attn_params* params, sparse_attn_plan** plan) {
  if (!plan) return fail(SA_EINVAL, "plan output pointer is NULL");
  *plan = nullptr;
  if (!params) return fail(SA_EINVAL, "params is NULL");
  int rc = validate_params(*params);
  if (rc) return rc;
  sparse_attn_plan* pl = new (std::nothrow) sparse_attn_plan;
  if (!pl) return fail(SA_EINVAL, "out of host memory");
  pl->params = *params;
  build_plan(pl);
  *plan = pl;
  log_plan(pl);
  return ok();
}

void sparse_attn_plan_destroy(sparse_attn_plan* plan) { delete plan; }

int sparse_attn_workspace_layout(const sparse_attn_plan* plan, sparse_attn_ws_layout* layout) {
  if (!plan || !layout) return fail(SA_EINVAL, "plan and layout must be non-NULL");
  *layout = plan->layout;
  return ok();
}

int sparse_attn_pool(const sparse_attn_plan* plan, const void* q, const void* k, const void* v,
                     void* ws, size_t ws_bytes, void* stream) {
  if (!plan) return fail(SA_EINVAL, "plan is NULL");
  if (plan->shape.reblock) return fail(SA_EINVAL, "SA_FLAG_REBLOCK runs through sparse_attn_forward only");
  int rc;
  if ((rc = check_tensors(q, k, v, nullptr, false))) return rc;
  if ((rc = check_ws(plan, ws, ws_bytes))) return rc;
  if ((rc = check_device())) return rc;
  const sa::Workspace w = carve(plan, ws);
  hipStream_t st = (hipStream_t)stream;
  if ((rc = launched(sa::launch_pool_q(plan->shape, q, w, st), "pool_q"))) return rc;
  if (plan->shape.reweight) {
    if ((rc = launched(sa::launch_anchor(plan->shape, q, w, st), "anchor"))) return rc;
  }
  if ((rc = launched(sa::launch_pack_kv(plan->shape, k, v, w, st), "pack_kv"))) return rc;
  return ok();
}

int sparse_attn_workspace_bytes(const sparse_attn_plan* plan, size_t* bytes) {
  if (!plan || !bytes) return fail(SA_EINVAL, "plan and bytes must be non-NULL");
  *bytes = (size_t)plan->layout.total_bytes;
  return ok();
}

int sparse_attn_route(const sparse_attn_plan* plan, const void* q, const void* k, const void* v, void* ws,
                      size_t ws_bytes, void* stream) {
  int rc = sparse_attn_pool(plan, q, k, v, ws, ws_bytes, stream);
  if (rc || plan->shape.dense) return rc;
  return sparse_attn_select(plan, ws, ws_bytes, stream);
}

int sparse_attn_select(const sparse_attn_plan* plan, void* ws, size_t ws_bytes, void* stream) {
  if (!plan) return fail(SA_EINVAL, "plan is NULL");
  if (plan->shape.reblock) return fail(SA_EINVAL, "SA_FLAG_REBLOCK runs through sparse_attn_forward only");
  int rc;
  if ((rc = check_ws(plan, ws, ws_bytes))) return rc;
  if ((rc = check_device())) return rc;
  if ((rc = launched(sa::launch_select(plan->shape, carve(plan, ws), (hipStream_t)stream), "select")))
    return rc;
  return ok();
}

// The attend step: the dense path (tau = -inf, bf16 QK^T, rows in place)
// has a kernel of its own; everything else runs the routed kernel.
static hipError_t attend(const sa::Shape& s, const void* q, void* out, const sa::Workspace& w,
                         hipStream_t st) {
  if (s.dense && !s.int8 && !s.permuted) return sa::launch_dense_attend(s, q, out, w, st);
  return sa::launch_attend(s, q, out, w, st);
}

int sparse_attn_attend(const sparse_attn_plan* plan, const void* q, void* out, void* ws, size_t ws_bytes,
                       void* stream) {
  if (!plan) return fail(SA_EINVAL, "plan is NULL");
  if (plan->shape.reblock) return fail(SA_EINVAL, "SA_FLAG_REBLOCK runs through sparse_attn_forward only");
  int rc;
  if ((rc = check_tensors(q, q, q, out, true))) return rc;
  if ((rc = check_ws(plan, ws, ws_bytes))) return rc;
  if ((rc = check_device())) return rc;
  if ((rc = launched(attend(plan->shape, q, out, carve(plan, ws), (hipStream_t)stream), "attend")))
    return rc;
  return ok();
}

int sparse_attn_forward(const sparse_attn_plan* plan, const void* q, const void* k, const void* v,
                        void* out, void* ws, size_t ws_bytes, void* stream) {
  if (!plan) return fail(SA_EINVAL, "plan is NULL");
  int rc;
  if ((rc = check_tensors(q, k, v, out, true))) return rc;
  if ((rc = check_ws(plan, ws, ws_bytes))) return rc;
  if ((rc = check_device())) return rc;
  const sa::Workspace w = carve(plan, ws);
  hipStream_t st = (hipStream_t)stream;
  sa::Shape s = plan->shape;
  if (s.reblock) {
    // the partition; the path then reads its rows through the final orders
    // and writes every output row at its own position
    if ((rc = launched(sa::launch_reblock_partition(s, q, k, w, st), "reblock partition"))) return rc;
    s.permuted = 1;
  }
  if (!s.dense) {
    if ((rc = launched(sa::launch_pool_q(s, q, w, st), "pool_q"))) return rc;
  }
  if (s.reweight) {
    if ((rc = launched(sa::launch_anchor(s, q, w, st), "anchor"))) return rc;
  }
  if ((rc = launched(sa::launch_pack_kv(s, k, v, w, st), "pack_kv"))) return rc;
  if (!s.dense) {
    if ((rc = launched(sa::launch_select(s, w, st), "select"))) return rc;
  }
  if ((rc = launched(attend(s, q, out, w, st), "attend"))) return rc;
  return ok();
}

// The per-device scratch array lives in sparse_attn_noalloc.hip (a device
// variable must be defined in device code); this returns its device address
// for the current device, looked up once per device.
__attribute__((visibility("hidden"))) int sparse_attn_noalloc_scratch(void** ptr);

int sparse_attn_forward_noalloc(const sparse_attn_plan* plan, const void* q, const void* k, const void* v,
                                void* out, void* stream) {
  if (!plan) return fail(SA_EINVAL, "plan is NULL");
  if (plan->layout.total_bytes > SA_NOALLOC_SCRATCH_BYTES)
    return fail(SA_EWORKSPACE, "plan needs a %llu-byte workspace, the allocation-free scratch holds %llu",
                (unsigned long long)plan->layout.total_bytes, (unsigned long long)SA_NOALLOC_SCRATCH_BYTES);
  int rc;
  if ((rc = check_tensors(q, k, v, out, true))) return rc;
  if ((rc = check_device())) return rc;
  void* ws = nullptr;
  if ((rc = sparse_attn_noalloc_scratch(&ws)))
    return fail(rc, "could not look up the device scratch array");
  return sparse_attn_forward(plan, q, k, v, out, ws, (size_t)SA_NOALLOC_SCRATCH_BYTES, stream);
}

}  // extern "C"
