// C ABI of libfasa: argument checks, context tables, workspace layout and the
// launch order of each call.  Declarations and semantics: include/fasa.h.

#include <hip/hip_runtime.h>

#include <dlfcn.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "device_common.hpp"
#include "fasa_internal.hpp"

using namespace fasa;

namespace {

thread_local std::string g_last_error;

// Host-side call log and trace ranges (no GPU work, off by default):
//   FASA_LOG=1    one line per C-ABI call on stderr (the call and the
//                 arguments that shape its launches), and one per error it
//                 returns;
//   FASA_ROCTX=1  a roctx range around each call (rocprofv3 --marker-trace
//                 shows them next to the kernels), through the ROCm marker
//                 library, loaded on first use.
bool env_on(const char* name) {
  const char* v = std::getenv(name);
  return v != nullptr && v[0] != '\0' && std::strcmp(v, "0") != 0;
}

bool log_on() {
  static const bool on = env_on("FASA_LOG");
  return on;
}

struct Roctx {
  int (*push)(const char*) = nullptr;
  int (*pop)() = nullptr;
};

const Roctx& roctx() {
  static const Roctx r = [] {
    Roctx x;
    if (!env_on("FASA_ROCTX")) return x;
    void* h = dlopen("librocprofiler-sdk-roctx.so.1", RTLD_NOW | RTLD_LOCAL);
    if (h == nullptr) {
      std::fprintf(stderr, "fasa: FASA_ROCTX set but the roctx library did not load: %s\n",
                   dlerror());
      return x;
    }
    x.push = reinterpret_cast<int (*)(const char*)>(dlsym(h, "roctxRangePushA"));
    x.pop = reinterpret_cast<int (*)()>(dlsym(h, "roctxRangePop"));
    if (x.push == nullptr || x.pop == nullptr) x = Roctx{};
    return x;
  }();
  return r;
}

thread_local const char* g_call = nullptr;  // the C-ABI call in progress (for the log)

// One per C-ABI call: logs the call, opens and closes its roctx range.
class ApiScope {
 public:
  ApiScope(const char* name, const char* fmt, ...) : outer_(g_call) {
    g_call = name;
    if (log_on()) {
      char buf[384];
      va_list ap;
      va_start(ap, fmt);
      std::vsnprintf(buf, sizeof buf, fmt, ap);
      va_end(ap);
      std::fprintf(stderr, "fasa: %s(%s)\n", name, buf);
    }
    if (roctx().push) roctx().push(name);
  }
  ~ApiScope() {
    if (roctx().pop) roctx().pop();
    g_call = outer_;
  }
  ApiScope(const ApiScope&) = delete;
  ApiScope& operator=(const ApiScope&) = delete;

 private:
  const char* outer_;
};

#define FASA_API(...) ApiScope api_scope_(__func__, __VA_ARGS__)

fasa_status fail(fasa_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  if (log_on()) std::fprintf(stderr, "fasa: %s: error %d: %s\n", g_call ? g_call : "?", (int)st, buf);
  return st;
}

fasa_status ok() {
  g_last_error.clear();
  return FASA_OK;
}

fasa_status hip_fail(hipError_t e, const char* what) {
  return fail(FASA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

size_t dtype_size(fasa_dtype t) { return t == FASA_BF16 ? 2 : 4; }

void build_layout(fasa_ctx* c) {
  WsLayout& w = c->ws;
  const size_t rows = (size_t)c->batch * c->hq;
  w.fac_splits = (c->max_budget + kFacSplitRows - 1) / kFacSplitRows;
  w.dense_splits = (c->cap + kDenseSplitTokens - 1) / kDenseSplitTokens;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t at = off;
    off = align256(off + bytes);
    return at;
  };
  w.err = take(16);
  w.nb = take(sizeof(int32_t) * c->batch);
  w.qrot = take(sizeof(float) * rows * c->d);
  w.scores = take(sizeof(float) * rows * c->cap);
  w.idx = take(sizeof(int32_t) * rows * c->max_budget);
  {
    // Chunk candidates of the longest row (chunks of 4096 positions or more;
    // the select never takes more than kTwoStageMaxCand).
    const long long nch = (c->cap + 4095) / 4096;
    const long long all = nch * c->max_budget;
    const int need = all < kTwoStageMaxCand ? (int)all : kTwoStageMaxCand;
    w.cand_stride = (need + 3) & ~3;  // rows start 32-byte aligned
    w.cand = take(sizeof(uint64_t) * rows * w.cand_stride);
  }
  w.gstride = (c->cap + kGroupTokens - 1) / kGroupTokens;
  w.gmax = take(sizeof(uint32_t) * rows * w.gstride);
  w.fac = take(sizeof(float) * rows * w.fac_splits * (c->d + 2));
  w.dense = take(sizeof(float) * rows * w.dense_splits * (c->d + 2));
  w.total = off;
}

fasa_status check_ctx(const fasa_ctx* c) {
  if (!c) return fail(FASA_ERR_INVALID_ARG, "null context");
  return FASA_OK;
}

fasa_status check_len(const fasa_ctx* c, int max_seq_len) {
  if (max_seq_len < 1) return fail(FASA_ERR_INVALID_ARG, "max_seq_len %d < 1", max_seq_len);
  if (max_seq_len > c->cap)
    return fail(FASA_ERR_CAPACITY, "max_seq_len %d exceeds capacity %d", max_seq_len, c->cap);
  return FASA_OK;
}

fasa_status check_budget(const fasa_ctx* c, int budget) {
  if (budget < 1) return fail(FASA_ERR_INVALID_ARG, "budget %d < 1", budget);
  if (budget > c->max_budget)
    return fail(FASA_ERR_CAPACITY, "budget %d exceeds max_budget %d", budget, c->max_budget);
  return FASA_OK;
}

constexpr int kTimingPairs = 4096;

// Brackets one launch with a pair of events when timing is enabled.
class Timed {
 public:
  Timed(fasa_ctx* c, int family, hipStream_t s) : c_(c), s_(s), pair_(-1) {
    if (!c->timing || c->ev_used >= kTimingPairs) return;
    pair_ = c->ev_used++;
    c->ev_family[pair_] = family;
    (void)hipEventRecord(c->ev[2 * pair_], s_);
  }
  ~Timed() {
    if (pair_ >= 0) (void)hipEventRecord(c_->ev[2 * pair_ + 1], s_);
  }

 private:
  fasa_ctx* c_;
  hipStream_t s_;
  int pair_;
};

#define FASA_NONNULL(p)                                                  \
  do {                                                                   \
    if ((p) == nullptr) return fail(FASA_ERR_INVALID_ARG, "%s is null", #p); \
  } while (0)

#define FASA_TRY(expr)                      \
  do {                                      \
    fasa_status _st = (expr);               \
    if (_st != FASA_OK) return _st;         \
  } while (0)

#define FASA_HIP(expr, what)                \
  do {                                      \
    hipError_t _e = (expr);                 \
    if (_e != hipSuccess) return hip_fail(_e, what); \
  } while (0)

}  // namespace

extern "C" {

fasa_status fasa_create(fasa_ctx** out, int batch, int n_q_heads, int n_kv_heads, int head_dim,
                        int capacity, double rope_theta, fasa_dtype dtype,
                        const int32_t* dom_fc, int n_dom, int max_budget) {
  return fasa_create_partial_rope(out, batch, n_q_heads, n_kv_heads, head_dim, head_dim,
                                  capacity, rope_theta, dtype, dom_fc, n_dom, max_budget);
}

fasa_status fasa_create_partial_rope(fasa_ctx** out, int batch, int n_q_heads, int n_kv_heads,
                                     int head_dim, int rotary_dim, int capacity,
                                     double rope_theta, fasa_dtype dtype, const int32_t* dom_fc,
                                     int n_dom, int max_budget) {
  FASA_API("batch=%d hq=%d hkv=%d d=%d r=%d cap=%d theta=%g dtype=%d n_dom=%d max_budget=%d", batch, n_q_heads, n_kv_heads, head_dim, rotary_dim, capacity, rope_theta, (int)dtype, n_dom, max_budget);
  if (out == nullptr) return fail(FASA_ERR_INVALID_ARG, "out is null");
  *out = nullptr;
  if (batch < 1) return fail(FASA_ERR_INVALID_ARG, "batch %d < 1", batch);
  if (n_q_heads < 1 || n_kv_heads < 1)
    return fail(FASA_ERR_INVALID_ARG, "head counts must be >= 1 (%d, %d)", n_q_heads, n_kv_heads);
  if (n_q_heads % n_kv_heads)
    return fail(FASA_ERR_INVALID_ARG, "n_q_heads %d not a multiple of n_kv_heads %d", n_q_heads,
                n_kv_heads);
  const int G = n_q_heads / n_kv_heads;
  if (n_kv_heads > kArgKvHeads)
    return fail(FASA_ERR_UNSUPPORTED, "n_kv_heads %d above %d", n_kv_heads, kArgKvHeads);
  if (G != 1 && G != 2 && G != 4 && G != 8)
    return fail(FASA_ERR_UNSUPPORTED, "query heads per KV head %d not in {1,2,4,8}", G);
  if (head_dim != 64 && head_dim != 128)
    return fail(FASA_ERR_UNSUPPORTED, "head_dim %d not in {64,128}", head_dim);
  if (rotary_dim < 2 || rotary_dim > head_dim || rotary_dim % 2)
    return fail(FASA_ERR_INVALID_ARG, "rotary_dim %d must be even and in [2, %d]", rotary_dim,
                head_dim);
  if (capacity < 64 || capacity % 64)
    return fail(FASA_ERR_INVALID_ARG, "capacity %d must be a positive multiple of 64", capacity);
  if (capacity > kMaxCapacity)
    return fail(FASA_ERR_CAPACITY, "capacity %d above %d", capacity, kMaxCapacity);
  if (!(rope_theta > 1.0) || !std::isfinite(rope_theta))
    return fail(FASA_ERR_INVALID_ARG, "rope_theta must be finite and > 1");
  if (dtype != FASA_F32 && dtype != FASA_BF16)
    return fail(FASA_ERR_UNSUPPORTED, "dtype %d", (int)dtype);
  if (dom_fc == nullptr) return fail(FASA_ERR_INVALID_ARG, "dom_fc is null");
  const int C = head_dim / 2;
  if (n_dom < 1 || n_dom > C)
    return fail(FASA_ERR_INVALID_ARG, "n_dom %d not in [1, %d]", n_dom, C);
  if (max_budget < 1 || max_budget > capacity)
    return fail(FASA_ERR_INVALID_ARG, "max_budget %d not in [1, capacity]", max_budget);
  for (int h = 0; h < n_q_heads; ++h) {
    uint64_t seen = 0;
    for (int f = 0; f < n_dom; ++f) {
      const int v = dom_fc[(size_t)h * n_dom + f];
      if (v < 0 || v >= C)
        return fail(FASA_ERR_INVALID_ARG, "dom_fc[%d][%d] = %d outside [0, %d)", h, f, v, C);
      if (seen >> v & 1ull)
        return fail(FASA_ERR_INVALID_ARG, "dom_fc[%d] repeats FC %d", h, v);
      seen |= 1ull << v;
    }
  }

  // FAC runs one workgroup per (sequence, query head, split of the budget) in a
  // 1-D grid, padded to whole rounds of 8 (b, KV head, split) tuples; a 1-D
  // launch holds at most 2^32 - 1 work items.
  const long long fac_tuples =
      (long long)((max_budget + kFacSplitRows - 1) / kFacSplitRows) * n_kv_heads * batch;
  if ((fac_tuples + 7) / 8 * 8 * G * kFacThreads > 0xffffffffLL)
    return fail(FASA_ERR_UNSUPPORTED, "batch %d x heads %d x budget %d exceeds one FAC launch",
                batch, n_q_heads, max_budget);

  fasa_ctx* c = new (std::nothrow) fasa_ctx();
  if (!c) return fail(FASA_ERR_INVALID_ARG, "out of host memory");
  c->batch = batch;
  c->hq = n_q_heads;
  c->hkv = n_kv_heads;
  c->d = head_dim;
  c->C = C;
  c->R = rotary_dim / 2;
  c->cap = capacity;
  c->G = G;
  c->F = n_dom;
  c->max_budget = max_budget;
  c->theta = rope_theta;
  c->dtype = dtype;
  c->dom.assign(dom_fc, dom_fc + (size_t)n_q_heads * n_dom);
  c->dev_alloc = nullptr;
  c->cus = 0;

  // Sidecar planes: per KV head, the union of its query heads' dominant FCs.
  std::vector<int32_t> fc_slot((size_t)n_kv_heads * C, -1);
  std::vector<uint64_t> mask(n_q_heads, 0);
  for (int h = 0; h < n_q_heads; ++h)
    for (int f = 0; f < n_dom; ++f) mask[h] |= 1ull << c->dom[(size_t)h * n_dom + f];
  c->plane_off.assign(n_kv_heads + 1, 0);
  for (int g = 0; g < n_kv_heads; ++g) {
    uint64_t uni = 0;
    for (int k = 0; k < G; ++k) uni |= mask[(size_t)g * G + k];
    int slot = 0;
    for (int fc = 0; fc < C; ++fc)
      if (uni >> fc & 1ull) {
        fc_slot[(size_t)g * C + fc] = slot++;
        c->plane_fc.push_back(fc);
      }
    c->plane_off[g + 1] = c->plane_off[g] + slot;
  }
  c->P = c->plane_off[n_kv_heads];
  c->max_union = 0;
  for (int g = 0; g < n_kv_heads; ++g)
    c->max_union = std::max(c->max_union, c->plane_off[g + 1] - c->plane_off[g]);
  // Rotated FCs at theta^(-2c/rotary_dim); pass-through FCs at frequency 0.
  std::vector<double> omega(C, 0.0);
  for (int i = 0; i < c->R; ++i) omega[i] = std::pow(rope_theta, -2.0 * i / rotary_dim);

  build_layout(c);

  // One device allocation for the constant tables.
  const size_t b_off = align256(sizeof(int32_t) * (n_kv_heads + 1));
  const size_t b_slot = align256(sizeof(int32_t) * fc_slot.size());
  const size_t b_mask = align256(sizeof(uint64_t) * mask.size());
  const size_t b_omega = align256(sizeof(double) * C);
  // Per query head, its dominant FCs ascending with their planes (the first
  // 16; TIP's per-head layout is used only when a head has at most 16).
  constexpr int kHeadFcSlots = 16;
  std::vector<int2> head_fc((size_t)n_q_heads * kHeadFcSlots, make_int2(-1, -1));
  for (int h = 0; h < n_q_heads; ++h) {
    int k = 0;
    for (int fc = 0; fc < C && k < kHeadFcSlots; ++fc)
      if (mask[h] >> fc & 1ull)
        head_fc[(size_t)h * kHeadFcSlots + k++] = make_int2(fc, fc_slot[(size_t)(h / G) * C + fc]);
  }
  const size_t b_head = align256(sizeof(int2) * head_fc.size());
  const size_t bytes = b_off + b_slot + b_mask + b_omega + b_head;
  hipError_t e = hipGetDevice(&c->device);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&c->cus, hipDeviceAttributeMultiprocessorCount, c->device);
  if (e == hipSuccess) e = hipMalloc(&c->dev_alloc, bytes);
  if (e != hipSuccess) {
    c->dev_alloc = nullptr;
    fasa_destroy(c);
    return hip_fail(e, "fasa_create: device tables");
  }
  uint8_t* base = static_cast<uint8_t*>(c->dev_alloc);
  c->tab.plane_off = reinterpret_cast<int32_t*>(base);
  c->tab.fc_slot = reinterpret_cast<int32_t*>(base + b_off);
  c->tab.dom_mask = reinterpret_cast<uint64_t*>(base + b_off + b_slot);
  c->tab.omega = reinterpret_cast<double*>(base + b_off + b_slot + b_mask);
  c->tab.head_fc = reinterpret_cast<int2*>(base + b_off + b_slot + b_mask + b_omega);
  e = hipMemcpy(c->tab.plane_off, c->plane_off.data(), sizeof(int32_t) * c->plane_off.size(),
                hipMemcpyHostToDevice);
  if (e == hipSuccess)
    e = hipMemcpy(c->tab.fc_slot, fc_slot.data(), sizeof(int32_t) * fc_slot.size(),
                  hipMemcpyHostToDevice);
  if (e == hipSuccess)
    e = hipMemcpy(c->tab.dom_mask, mask.data(), sizeof(uint64_t) * mask.size(),
                  hipMemcpyHostToDevice);
  if (e == hipSuccess)
    e = hipMemcpy(c->tab.omega, omega.data(), sizeof(double) * C, hipMemcpyHostToDevice);
  if (e == hipSuccess)
    e = hipMemcpy(c->tab.head_fc, head_fc.data(), sizeof(int2) * head_fc.size(),
                  hipMemcpyHostToDevice);
  if (e != hipSuccess) {
    fasa_destroy(c);
    return hip_fail(e, "fasa_create: uploading tables");
  }
  *out = c;
  return ok();
}

void fasa_destroy(fasa_ctx* ctx) {
  FASA_API("ctx=%p", (void*)ctx);
  if (!ctx) return;
  for (hipEvent_t e : ctx->ev) (void)hipEventDestroy(e);
  if (ctx->dev_alloc) (void)hipFree(ctx->dev_alloc);
  delete ctx;
}

size_t fasa_kv_cache_bytes(const fasa_ctx* c) {
  if (!c) return 0;
  return (size_t)c->batch * c->hkv * c->cap * c->d * dtype_size(c->dtype);
}

size_t fasa_sidecar_bytes(const fasa_ctx* c) {
  if (!c) return 0;
  return (size_t)c->batch * c->P * c->cap * 2 * dtype_size(c->dtype);
}

size_t fasa_workspace_bytes(const fasa_ctx* c) { return c ? c->ws.total : 0; }

int fasa_sidecar_layout(const fasa_ctx* c, int32_t* plane_offset, int32_t* plane_fc) {
  if (!c) return (int)fail(FASA_ERR_INVALID_ARG, "null context");
  if (plane_offset) std::memcpy(plane_offset, c->plane_off.data(), sizeof(int32_t) * (c->hkv + 1));
  if (plane_fc && c->P) std::memcpy(plane_fc, c->plane_fc.data(), sizeof(int32_t) * c->P);
  return c->P;
}

fasa_status fasa_workspace_init(fasa_ctx* c, void* workspace, hipStream_t stream) {
  FASA_API("ctx=%p ws=%p", (void*)c, workspace);
  FASA_TRY(check_ctx(c));
  FASA_NONNULL(workspace);
  FASA_HIP(launch_fill_zero(workspace, c->ws.total, stream), "fasa_workspace_init");
  return ok();
}

fasa_status fasa_append_kv(fasa_ctx* c, void* k_cache, void* v_cache, void* sidecar,
                           const void* k_new, const void* v_new, const int32_t* start_pos,
                           int n_new, void* workspace, hipStream_t stream) {
  FASA_API("ctx=%p n_new=%d ws=%p stream=%p", (void*)c, n_new, workspace, (void*)stream);
  FASA_TRY(check_ctx(c));
  if (n_new < 0) return fail(FASA_ERR_INVALID_ARG, "n_new %d < 0", n_new);
  if (n_new > c->cap) return fail(FASA_ERR_CAPACITY, "n_new %d exceeds capacity", n_new);
  if (n_new == 0) return ok();
  FASA_NONNULL(k_cache);
  FASA_NONNULL(v_cache);
  FASA_NONNULL(sidecar);
  FASA_NONNULL(k_new);
  FASA_NONNULL(v_new);
  FASA_NONNULL(start_pos);
  FASA_NONNULL(workspace);
  {
    Timed t(c, FASA_K_APPEND, stream);
    FASA_HIP(launch_append(c, k_cache, v_cache, sidecar, k_new, v_new, start_pos, n_new,
                           static_cast<uint8_t*>(workspace), stream),
             "fasa_append_kv");
  }
  return ok();
}

fasa_status fasa_tip_scores(fasa_ctx* c, const void* sidecar, const void* q,
                            const int32_t* seq_lens, int max_seq_len, float* scores,
                            void* workspace, hipStream_t stream) {
  FASA_API("ctx=%p max_seq_len=%d ws=%p stream=%p", (void*)c, max_seq_len, workspace, (void*)stream);
  FASA_TRY(check_ctx(c));
  FASA_TRY(check_len(c, max_seq_len));
  FASA_NONNULL(sidecar);
  FASA_NONNULL(q);
  FASA_NONNULL(seq_lens);
  FASA_NONNULL(scores);
  FASA_NONNULL(workspace);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  TipArgs a{const_cast<void*>(sidecar), q, nullptr, nullptr, nullptr, nullptr, seq_lens,
            max_seq_len};
  {
    Timed t(c, FASA_K_TIP, stream);
    FASA_HIP(launch_tip(c, kPrologueQueryOnly, a, scores, ws, stream), "fasa_tip_scores");
  }
  return ok();
}

static fasa_status topk_impl(fasa_ctx* c, const float* scores, const int32_t* seq_lens,
                             int max_seq_len, const int32_t* head_budget, int budget,
                             int32_t* idx, void* workspace, hipStream_t stream) {
  FASA_TRY(check_ctx(c));
  FASA_TRY(check_len(c, max_seq_len));
  FASA_TRY(check_budget(c, budget));
  FASA_NONNULL(scores);
  FASA_NONNULL(seq_lens);
  FASA_NONNULL(idx);
  FASA_NONNULL(workspace);
  {
    Timed t(c, FASA_K_TOPK, stream);
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    if (select_path_applies(max_seq_len, budget))
      FASA_HIP(launch_select(c, scores, seq_lens, max_seq_len, budget, idx, nullptr, nullptr,
                             nullptr, nullptr, ws, stream, head_budget),
               "fasa_topk: row select");
    else
      FASA_HIP(launch_topk(c, scores, seq_lens, max_seq_len, budget, idx, nullptr, ws, stream,
                           head_budget),
               "fasa_topk");
  }
  return ok();
}

fasa_status fasa_topk(fasa_ctx* c, const float* scores, const int32_t* seq_lens,
                      int max_seq_len, int budget, int32_t* idx, void* workspace,
                      hipStream_t stream) {
  FASA_API("ctx=%p max_seq_len=%d budget=%d ws=%p stream=%p", (void*)c, max_seq_len, budget, workspace, (void*)stream);
  return topk_impl(c, scores, seq_lens, max_seq_len, nullptr, budget, idx, workspace, stream);
}

fasa_status fasa_topk_per_head(fasa_ctx* c, const float* scores, const int32_t* seq_lens,
                               int max_seq_len, const int32_t* head_budget, int budget,
                               int32_t* idx, void* workspace, hipStream_t stream) {
  FASA_API("ctx=%p max_seq_len=%d budget=%d head_budget=%p ws=%p stream=%p", (void*)c, max_seq_len, budget, (const void*)head_budget, workspace, (void*)stream);
  FASA_NONNULL(head_budget);
  return topk_impl(c, scores, seq_lens, max_seq_len, head_budget, budget, idx, workspace,
                   stream);
}

fasa_status fasa_sparse_attn(fasa_ctx* c, const void* k_cache, const void* v_cache,
                             const void* q, const int32_t* seq_lens, const int32_t* idx,
                             int budget, float* out, void* workspace, hipStream_t stream) {
  FASA_API("ctx=%p budget=%d ws=%p stream=%p", (void*)c, budget, workspace, (void*)stream);
  FASA_TRY(check_ctx(c));
  FASA_TRY(check_budget(c, budget));
  FASA_NONNULL(k_cache);
  FASA_NONNULL(v_cache);
  FASA_NONNULL(q);
  FASA_NONNULL(seq_lens);
  FASA_NONNULL(idx);
  FASA_NONNULL(out);
  FASA_NONNULL(workspace);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  {
    Timed t(c, FASA_K_PROLOGUE, stream);
    FASA_HIP(launch_prologue(c, q, seq_lens, c->cap, ws, stream), "fasa_sparse_attn: prologue");
  }
  {
    Timed t(c, FASA_K_FAC, stream);
    FASA_HIP(launch_fac(c, k_cache, v_cache, reinterpret_cast<const int32_t*>(ws + c->ws.nb),
                        c->cap, idx, budget, out, ws, stream),
             "fasa_sparse_attn");
  }
  return ok();
}

static fasa_status decode_impl(fasa_ctx* c, void* k_cache, void* v_cache, void* sidecar,
                               const void* q, const void* k_new, const void* v_new,
                               int32_t* seq_lens, int max_seq_len, const int32_t* head_budget,
                               int budget, float* out, int32_t* idx_out, void* workspace,
                               unsigned flags, hipStream_t stream) {
  FASA_TRY(check_ctx(c));
  FASA_TRY(check_len(c, max_seq_len));
  FASA_TRY(check_budget(c, budget));
  FASA_NONNULL(k_cache);
  FASA_NONNULL(v_cache);
  FASA_NONNULL(sidecar);
  FASA_NONNULL(q);
  FASA_NONNULL(k_new);
  FASA_NONNULL(v_new);
  FASA_NONNULL(seq_lens);
  FASA_NONNULL(out);
  FASA_NONNULL(workspace);
  if (flags & ~FASA_ADVANCE_SEQ_LENS) return fail(FASA_ERR_INVALID_ARG, "unknown flags 0x%x", flags);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  const int32_t* nb = reinterpret_cast<const int32_t*>(ws + c->ws.nb);
  float* scores = reinterpret_cast<float*>(ws + c->ws.scores);
  int32_t* idx = idx_out ? idx_out : reinterpret_cast<int32_t*>(ws + c->ws.idx);
  int32_t* advance = (flags & FASA_ADVANCE_SEQ_LENS) ? seq_lens : nullptr;
  TipArgs a{sidecar, q, k_new, v_new, k_cache, v_cache, seq_lens, max_seq_len};
  // Long rows with a fused budget: TIP also writes each token group's largest
  // score, and one launch selects from those and attends.
  const bool filtered = filter_path_applies(max_seq_len, budget);
  {
    // Append, query rotation and TIP in one launch.
    Timed t(c, FASA_K_TIP, stream);
    FASA_HIP(launch_tip(c, kPrologueDecode, a, scores, ws, stream,
                        filtered ? reinterpret_cast<uint32_t*>(ws + c->ws.gmax) : nullptr),
             "fasa_decode_step: tip");
  }
  if (filtered) {
    Timed t(c, FASA_K_SELECT_FAC, stream);
    // K and V in host memory: one workgroup per row, so each selected row
    // crosses the host link once (column parts would each fetch its K row).
    if (c->kv_kind.ptr.load(std::memory_order_relaxed) != k_cache) {
      c->kv_kind.host.store(fasa_pointer_kind(k_cache) == FASA_PTR_HOST_MAPPED,
                            std::memory_order_relaxed);
      c->kv_kind.ptr.store(k_cache, std::memory_order_relaxed);
    }
    FASA_HIP(launch_filter_select(c, scores, nb, max_seq_len, budget, idx_out, k_cache, v_cache,
                                  out, advance, ws, stream, head_budget,
                                  c->kv_kind.host.load(std::memory_order_relaxed)),
             "fasa_decode_step: filtered select+fac");
    return ok();
  }
  if (select_path_applies(max_seq_len, budget)) {
    if (budget <= kFusedMaxBudget) {
      // Selection and FAC in one workgroup per row: the selected rows never
      // leave LDS.
      Timed t(c, FASA_K_SELECT_FAC, stream);
      FASA_HIP(launch_select(c, scores, nb, max_seq_len, budget, idx_out, k_cache, v_cache, out,
                             advance, ws, stream, head_budget),
               "fasa_decode_step: select+fac");
      return ok();
    }
    {
      Timed t(c, FASA_K_TOPK, stream);
      FASA_HIP(launch_select(c, scores, nb, max_seq_len, budget, idx, nullptr, nullptr, nullptr,
                             advance, ws, stream, head_budget),
               "fasa_decode_step: select");
    }
    {
      Timed t(c, FASA_K_FAC, stream);
      FASA_HIP(launch_fac(c, k_cache, v_cache, nb, max_seq_len, idx, budget, out, ws, stream),
               "fasa_decode_step: fac");
    }
    return ok();
  }
  if (budget <= kFusedMaxBudget) {
    // Selection and FAC in one kernel: the selected rows never leave LDS.
    Timed t(c, FASA_K_SELECT_FAC, stream);
    FASA_HIP(launch_select_attend(c, scores, nb, max_seq_len, budget, idx_out, k_cache, v_cache,
                                  out, advance, ws, stream, head_budget),
             "fasa_decode_step: select+fac");
    return ok();
  }
  {
    Timed t(c, FASA_K_TOPK, stream);
    FASA_HIP(launch_topk(c, scores, nb, max_seq_len, budget, idx, advance, ws, stream,
                         head_budget),
             "fasa_decode_step: topk");
  }
  {
    Timed t(c, FASA_K_FAC, stream);
    FASA_HIP(launch_fac(c, k_cache, v_cache, nb, max_seq_len, idx, budget, out, ws, stream),
             "fasa_decode_step: fac");
  }
  return ok();
}

fasa_status fasa_decode_step(fasa_ctx* c, void* k_cache, void* v_cache, void* sidecar,
                             const void* q, const void* k_new, const void* v_new,
                             int32_t* seq_lens, int max_seq_len, int budget, float* out,
                             int32_t* idx_out, void* workspace, unsigned flags,
                             hipStream_t stream) {
  FASA_API("ctx=%p max_seq_len=%d budget=%d idx=%p flags=%u ws=%p stream=%p", (void*)c, max_seq_len, budget, (void*)idx_out, flags, workspace, (void*)stream);
  return decode_impl(c, k_cache, v_cache, sidecar, q, k_new, v_new, seq_lens, max_seq_len,
                     nullptr, budget, out, idx_out, workspace, flags, stream);
}

fasa_status fasa_decode_step_per_head(fasa_ctx* c, void* k_cache, void* v_cache, void* sidecar,
                                      const void* q, const void* k_new, const void* v_new,
                                      int32_t* seq_lens, int max_seq_len,
                                      const int32_t* head_budget, int budget, float* out,
                                      int32_t* idx_out, void* workspace, unsigned flags,
                                      hipStream_t stream) {
  FASA_API("ctx=%p max_seq_len=%d budget=%d head_budget=%p idx=%p flags=%u ws=%p stream=%p", (void*)c, max_seq_len, budget, (const void*)head_budget, (void*)idx_out, flags, workspace, (void*)stream);
  FASA_NONNULL(head_budget);
  return decode_impl(c, k_cache, v_cache, sidecar, q, k_new, v_new, seq_lens, max_seq_len,
                     head_budget, budget, out, idx_out, workspace, flags, stream);
}

}  // extern "C"

// The workspace of fasa_decode_step_static: one array per GPU the library
// runs on, zero at load, held until the process ends.  Host code never uses
// its name as an address: the device address comes from hipGetSymbolAddress,
// once per device.
static __device__ __align__(256) uint8_t scratch[FASA_STATIC_SCRATCH_BYTES];

namespace {

constexpr int kScratchDevices = 64;
std::mutex g_scratch_mu;
uint8_t* g_scratch_ptr[kScratchDevices] = {};

// The device address of `scratch` on `device`, looked up on first use with
// that device current.
fasa_status scratch_on(int device, uint8_t** out) {
  if (device < 0 || device >= kScratchDevices)
    return fail(FASA_ERR_UNSUPPORTED, "device %d outside [0, %d)", device, kScratchDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[device] == nullptr) {
    int cur = -1;
    FASA_HIP(hipGetDevice(&cur), "fasa_decode_step_static: current device");
    if (cur != device) FASA_HIP(hipSetDevice(device), "fasa_decode_step_static: set device");
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != device) (void)hipSetDevice(cur);
    if (e != hipSuccess) return hip_fail(e, "fasa_decode_step_static: scratch address");
    if (p == nullptr) return fail(FASA_ERR_HIP, "fasa_decode_step_static: null scratch address");
    g_scratch_ptr[device] = static_cast<uint8_t*>(p);
  }
  *out = g_scratch_ptr[device];
  return FASA_OK;
}

}  // namespace

extern "C" {

fasa_status fasa_decode_step_static(fasa_ctx* c, void* k_cache, void* v_cache, void* sidecar,
                                    const void* q, const void* k_new, const void* v_new,
                                    int32_t* seq_lens, int max_seq_len, int budget, float* out,
                                    int32_t* idx_out, uint32_t* dev_flags, unsigned flags,
                                    hipStream_t stream) {
  FASA_API("ctx=%p max_seq_len=%d budget=%d idx=%p flags=%u stream=%p", (void*)c, max_seq_len, budget, (void*)idx_out, flags, (void*)stream);
  FASA_TRY(check_ctx(c));
  if (c->ws.total > FASA_STATIC_SCRATCH_BYTES)
    return fail(FASA_ERR_CAPACITY,
                "fasa_decode_step_static: the context needs a %zu-byte workspace, above the "
                "%zu-byte static scratch", c->ws.total, (size_t)FASA_STATIC_SCRATCH_BYTES);
  uint8_t* ws = nullptr;
  FASA_TRY(scratch_on(c->device, &ws));
  // Only the flag word must start at zero: every other region is written
  // before it is read within one step.
  FASA_HIP(launch_fill_zero(ws + c->ws.err, 16, stream), "fasa_decode_step_static: flags");
  FASA_TRY(decode_impl(c, k_cache, v_cache, sidecar, q, k_new, v_new, seq_lens, max_seq_len,
                       nullptr, budget, out, idx_out, ws, flags, stream));
  if (dev_flags != nullptr)
    FASA_HIP(launch_copy_u32(reinterpret_cast<const uint32_t*>(ws + c->ws.err), dev_flags, stream),
             "fasa_decode_step_static: flags out");
  return ok();
}

fasa_status fasa_dense_attn(fasa_ctx* c, const void* k_cache, const void* v_cache,
                            const void* q, const int32_t* seq_lens, int max_seq_len,
                            float* out, void* workspace, hipStream_t stream) {
  FASA_API("ctx=%p max_seq_len=%d ws=%p stream=%p", (void*)c, max_seq_len, workspace, (void*)stream);
  FASA_TRY(check_ctx(c));
  FASA_TRY(check_len(c, max_seq_len));
  FASA_NONNULL(k_cache);
  FASA_NONNULL(v_cache);
  FASA_NONNULL(q);
  FASA_NONNULL(seq_lens);
  FASA_NONNULL(out);
  FASA_NONNULL(workspace);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  if (c->dtype == FASA_BF16 && c->d == 128) {
    Timed t(c, FASA_K_DENSE, stream);
    FASA_HIP(launch_dense_fused(c, k_cache, v_cache, q, seq_lens, max_seq_len, out, ws, stream),
             "fasa_dense_attn");
    return ok();
  }
  {
    Timed t(c, FASA_K_PROLOGUE, stream);
    FASA_HIP(launch_prologue(c, q, seq_lens, max_seq_len, ws, stream), "fasa_dense_attn: prologue");
  }
  {
    Timed t(c, FASA_K_DENSE, stream);
    FASA_HIP(launch_dense(c, k_cache, v_cache, reinterpret_cast<const int32_t*>(ws + c->ws.nb),
                          max_seq_len, out, ws, stream),
             "fasa_dense_attn");
  }
  return ok();
}

size_t fasa_calibrate_workspace_bytes(const fasa_ctx* c, int topk) {
  if (!c || topk < 1) return 0;
  return calib_layout(c, topk).ws.total;
}

fasa_status fasa_calibrate(fasa_ctx* c, const void* k_cache, const void* q,
                           const int32_t* seq_lens, int max_seq_len, int topk, float* ca,
                           void* workspace, hipStream_t stream) {
  FASA_API("ctx=%p max_seq_len=%d topk=%d ws=%p stream=%p", (void*)c, max_seq_len, topk, workspace, (void*)stream);
  FASA_TRY(check_ctx(c));
  FASA_TRY(check_len(c, max_seq_len));
  if (topk < 1 || topk > c->cap || topk > kCalibMaxTopk)
    return fail(FASA_ERR_INVALID_ARG, "topk %d not in [1, min(%d, capacity)]", topk,
                kCalibMaxTopk);
  FASA_NONNULL(k_cache);
  FASA_NONNULL(q);
  FASA_NONNULL(seq_lens);
  FASA_NONNULL(ca);
  FASA_NONNULL(workspace);
  {
    Timed t(c, FASA_K_CALIBRATE, stream);
    FASA_HIP(launch_calibrate(c, k_cache, q, seq_lens, max_seq_len, topk, ca,
                              static_cast<uint8_t*>(workspace), stream),
             "fasa_calibrate");
  }
  return ok();
}

fasa_status fasa_select_dominant(const float* ca, int samples, int n_q_heads, int n_fc,
                                 int n_dom, int32_t* dom_out) {
  FASA_API("samples=%d hq=%d n_fc=%d n_dom=%d", samples, n_q_heads, n_fc, n_dom);
  if (!ca || !dom_out) return fail(FASA_ERR_INVALID_ARG, "null pointer");
  if (samples < 1 || n_q_heads < 1 || n_fc < 1 || n_dom < 1 || n_dom > n_fc)
    return fail(FASA_ERR_INVALID_ARG, "sizes out of range (samples %d, heads %d, fc %d, dom %d)",
                samples, n_q_heads, n_fc, n_dom);
  std::vector<double> mean(n_fc);
  std::vector<int> order(n_fc);
  for (int h = 0; h < n_q_heads; ++h) {
    for (int f = 0; f < n_fc; ++f) {
      double s = 0.0;
      for (int b = 0; b < samples; ++b) s += ca[((size_t)b * n_q_heads + h) * n_fc + f];
      mean[f] = s / samples;
      order[f] = f;
    }
    // Highest mean first, equal means to the lower FC.
    std::stable_sort(order.begin(), order.end(),
                     [&](int x, int y) { return mean[x] > mean[y]; });
    std::vector<int> pick(order.begin(), order.begin() + n_dom);
    std::sort(pick.begin(), pick.end());
    for (int f = 0; f < n_dom; ++f) dom_out[(size_t)h * n_dom + f] = pick[f];
  }
  return ok();
}

fasa_ptr_kind fasa_pointer_kind(const void* ptr) {
  if (!ptr) return FASA_PTR_UNUSABLE;
  hipPointerAttribute_t attr;
  if (hipPointerGetAttributes(&attr, ptr) != hipSuccess) {
    (void)hipGetLastError();  // pageable memory reports an error: clear it
    return FASA_PTR_UNUSABLE;
  }
  if (attr.type == hipMemoryTypeDevice) return FASA_PTR_DEVICE;
  if (attr.type == hipMemoryTypeHost && attr.devicePointer == ptr) return FASA_PTR_HOST_MAPPED;
  return FASA_PTR_UNUSABLE;
}

fasa_status fasa_read_probe(const void* buf, size_t bytes, float* sink, hipStream_t stream) {
  FASA_API("bytes=%zu stream=%p", bytes, (void*)stream);
  if (buf == nullptr || sink == nullptr) return fail(FASA_ERR_INVALID_ARG, "null pointer");
  if (bytes == 0 || bytes % 16 || reinterpret_cast<uintptr_t>(buf) % 16)
    return fail(FASA_ERR_INVALID_ARG, "bytes (%zu) and buf must be non-zero multiples of 16",
                bytes);
  if (bytes / 16 > kReadProbeMax16) return fail(FASA_ERR_INVALID_ARG, "buffer too large");
  FASA_HIP(launch_read_probe(buf, bytes / 16, sink, stream), "fasa_read_probe");
  return ok();
}

fasa_select_layout_kind fasa_select_layout(int max_seq_len, int budget, int* threads,
                                           int* per_thread, int* chunk) {
  if (max_seq_len < 1 || budget < 1) return FASA_LAYOUT_NONE;
  const SelectLayout l = select_layout(max_seq_len, budget);
  if (threads) *threads = l.threads;
  if (per_thread) *per_thread = l.per_thread;
  if (chunk) *chunk = l.chunk;
  return static_cast<fasa_select_layout_kind>(l.kind);
}

fasa_select_layout_kind fasa_decode_layout(int max_seq_len, int budget, int* threads,
                                           int* per_thread, int* chunk) {
  if (max_seq_len < 1 || budget < 1) return FASA_LAYOUT_NONE;
  if (!filter_path_applies(max_seq_len, budget))
    return fasa_select_layout(max_seq_len, budget, threads, per_thread, chunk);
  if (threads) *threads = kFilterSelectThreads;
  if (per_thread) *per_thread = filter_group_slots(max_seq_len);
  if (chunk) *chunk = kGroupTokens;
  return FASA_LAYOUT_GROUP_FILTER;
}

fasa_status fasa_check(fasa_ctx* c, void* workspace, hipStream_t stream, uint32_t* flags) {
  FASA_API("ctx=%p ws=%p stream=%p", (void*)c, workspace, (void*)stream);
  FASA_TRY(check_ctx(c));
  FASA_NONNULL(workspace);
  if (flags) *flags = 0;
  FASA_HIP(hipStreamSynchronize(stream), "fasa_check: synchronize");
  uint32_t v = 0;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  FASA_HIP(hipMemcpy(&v, ws + c->ws.err, sizeof v, hipMemcpyDeviceToHost), "fasa_check: read");
  if (v) {
    const uint32_t zero = 0;
    FASA_HIP(hipMemcpy(ws + c->ws.err, &zero, sizeof zero, hipMemcpyHostToDevice),
             "fasa_check: clear");
  }
  if (flags) *flags = v;
  if (v) return fail(FASA_ERR_DEVICE_FLAG, "device error flag 0x%x", v);
  return ok();
}

fasa_status fasa_timing_enable(fasa_ctx* c, int enable) {
  FASA_API("ctx=%p enable=%d", (void*)c, enable);
  FASA_TRY(check_ctx(c));
  if (enable && c->ev.empty()) {
    c->ev.assign(2 * kTimingPairs, nullptr);
    c->ev_family.assign(kTimingPairs, 0);
    for (auto& e : c->ev) FASA_HIP(hipEventCreate(&e), "fasa_timing_enable");
  }
  c->timing = enable != 0;
  return ok();
}

fasa_status fasa_timing_collect(fasa_ctx* c, double* total_ms, int32_t* launches) {
  FASA_API("ctx=%p", (void*)c);
  FASA_TRY(check_ctx(c));
  if (total_ms)
    for (int k = 0; k < FASA_K_COUNT; ++k) total_ms[k] = 0.0;
  if (launches)
    for (int k = 0; k < FASA_K_COUNT; ++k) launches[k] = 0;
  for (int i = 0; i < c->ev_used; ++i) {
    FASA_HIP(hipEventSynchronize(c->ev[2 * i + 1]), "fasa_timing_collect: wait");
    float ms = 0.0f;
    FASA_HIP(hipEventElapsedTime(&ms, c->ev[2 * i], c->ev[2 * i + 1]), "fasa_timing_collect");
    const int f = c->ev_family[i];
    if (total_ms) total_ms[f] += ms;
    if (launches) launches[f] += 1;
  }
  c->ev_used = 0;
  return ok();
}

const char* fasa_status_string(fasa_status s) {
  switch (s) {
    case FASA_OK: return "ok";
    case FASA_ERR_INVALID_ARG: return "invalid argument";
    case FASA_ERR_CAPACITY: return "capacity exceeded";
    case FASA_ERR_UNSUPPORTED: return "unsupported configuration";
    case FASA_ERR_HIP: return "HIP runtime error";
    case FASA_ERR_DEVICE_FLAG: return "device error flag set";
  }
  return "unknown status";
}

const char* fasa_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
