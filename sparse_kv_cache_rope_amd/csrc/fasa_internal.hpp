// Host-side context, workspace layout and kernel launchers of libfasa.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <atomic>
#include <vector>

#include "../../include/fasa.h"

namespace fasa {

// A pointer and whether it is host memory mapped into the device, read and
// written from any thread (copyable, so a context can be copied).
struct KvKindHint {
  std::atomic<const void*> ptr{nullptr};
  std::atomic<bool> host{false};
  KvKindHint() = default;
  KvKindHint(const KvKindHint& o)
      : ptr(o.ptr.load(std::memory_order_relaxed)), host(o.host.load(std::memory_order_relaxed)) {}
  KvKindHint& operator=(const KvKindHint& o) {
    ptr.store(o.ptr.load(std::memory_order_relaxed), std::memory_order_relaxed);
    host.store(o.host.load(std::memory_order_relaxed), std::memory_order_relaxed);
    return *this;
  }
};

// Device-resident constant tables, one allocation.
struct DeviceTables {
  int32_t* plane_off;  // [Hkv + 1]
  int32_t* fc_slot;    // [Hkv][C]: plane index within the KV head, or -1
  uint64_t* dom_mask;  // [Hq]: bit c set when FC c is dominant for head h
  double* omega;       // [C]: theta^(-2c/d), fp64
  int2* head_fc;       // [Hq][16]: head h's dominant FCs ascending, (FC, plane); (-1, -1) past them
};

// Byte offsets of the workspace regions (each 256-byte aligned).
struct WsLayout {
  size_t err = 0;       // uint32 [4]: device error flag
  size_t nb = 0;        // int32 [b]: tokens attended by the current call
  size_t qrot = 0;      // float [b][Hq][d]: rotated queries
  size_t scores = 0;    // float [b][Hq][cap]
  size_t idx = 0;       // int32 [b][Hq][max_budget]
  size_t cand = 0;      // uint64 [b*Hq][cand_stride]: two-stage top-B candidates
  size_t gmax = 0;      // uint32 [b*Hq][gstride]: TIP's largest score key per token group
  size_t fac = 0;       // float [b*Hq][fac_splits][d + 2]
  size_t dense = 0;     // float [b*Hq][dense_splits][d + 2]
  size_t total = 0;
  int fac_splits = 0;
  int dense_splits = 0;
  int cand_stride = 0;
  int gstride = 0;  // token groups per row of gmax: ceil(cap / kGroupTokens)
};

}  // namespace fasa

struct fasa_ctx {
  int batch, hq, hkv, d, C, cap, G, F, max_budget;
  int R;  // rotated FCs: rotary_dim / 2 (C for full RoPE)
  int max_union;  // largest |U_g| over the KV heads (sidecar planes of one head)
  int cus;        // compute units of the context's device
  double theta;
  fasa_dtype dtype;
  int device;
  std::vector<int32_t> dom;         // [Hq][F]
  std::vector<int32_t> plane_off;   // [Hkv + 1]
  std::vector<int32_t> plane_fc;    // [P]
  int P;
  void* dev_alloc;
  fasa::DeviceTables tab;
  fasa::WsLayout ws;
  // Event timing (fasa_timing_enable / fasa_timing_collect).
  bool timing = false;
  std::vector<hipEvent_t> ev;     // pairs: ev[2i] start, ev[2i+1] stop
  std::vector<int> ev_family;     // family of each recorded pair
  int ev_used = 0;
  // The last K cache pointer a decode step saw and whether it is host memory
  // mapped into the device (a launch-shape hint only: both shapes give the
  // same results).
  fasa::KvKindHint kv_kind;
};

namespace fasa {

// Rows of a FAC split and tokens of a dense split (one workgroup each).
constexpr int kFacSplitRows = 256;
// Threads of a FAC workgroup: 8 waves with 8 rows in flight per row slot
// (80 VGPRs, 3 workgroups per CU) hid the gather's latency chain better than
// 16 waves with 4 (2 per CU) or 4 waves with 16.
constexpr int kFacThreads = 512;
constexpr int kDenseSplitTokens = 256;
// Largest budget the fused select + FAC kernels keep in LDS.
constexpr int kFusedMaxBudget = 1024;
// Row select (select2.hip): positions per chunk of a long row (at most), and
// the most chunk candidates the final selection takes.
constexpr int kSelectChunk = 16384;
constexpr int kTwoStageMaxCand = 16384;

// Token groups: in a decode step whose selection is filtered
// (filter_path_applies) the TIP launch also writes, per query head, the
// largest score key (select_common.hpp order) of every kGroupTokens
// consecutive tokens; 0 for a group past the row.
constexpr int kGroupTokens = 16;

// How a launch reads seq_lens.
enum PrologueMode : int {
  kPrologueQueryOnly = 0,  // seq_lens = n_b; rotate q at n_b - 1
  kPrologueDecode = 1      // seq_lens = cached tokens; append at that position first
};

// Most KV heads whose sidecar plane offsets travel as a kernel argument.
constexpr int kArgKvHeads = 128;
struct PlaneOffsets {
  int32_t off[kArgKvHeads + 1];
};

struct TipArgs {
  void* sidecar;
  const void* q;
  const void* k_new;  // decode mode only
  const void* v_new;
  void* k_cache;
  void* v_cache;
  const int32_t* seq_lens;
  int max_seq_len;
};

// Every launcher reads n_b (tokens attended) from `nb`, a device int32 [b];
// a value outside [0, min(max_seq_len, cap)] raises FASA_DEVFLAG_SEQ_LEN and
// the row is treated as empty.
hipError_t launch_append(const fasa_ctx* c, void* k_cache, void* v_cache, void* sidecar,
                         const void* k_new, const void* v_new, const int32_t* start_pos,
                         int n_new, uint8_t* ws, hipStream_t s);
// Query-only mode: writes ws.nb and ws.qrot (queries rotated to n_b - 1).
hipError_t launch_prologue(const fasa_ctx* c, const void* q, const int32_t* seq_lens,
                           int max_seq_len, uint8_t* ws, hipStream_t s);
// TIP scores with the step's prologue fused in: writes ws.nb, ws.qrot and
// scores; in decode mode also appends the step's token.  Never writes
// seq_lens (see `advance` below).
// With group_max (decode mode only), also writes every group's largest score
// key there (ws.gmax layout).
hipError_t launch_tip(const fasa_ctx* c, PrologueMode mode, const TipArgs& a, float* scores,
                      uint8_t* ws, hipStream_t s, uint32_t* group_max = nullptr);
// The launchers below that take `advance` (may be null) store n_b into
// advance[b] from a kernel that reads only ws.nb, so it can be seq_lens.
// Those that take `head_budget` (device int32 [Hq], may be null) give query
// head h the budget head_budget[h] (in [0, budget]) instead of `budget`; idx
// rows stay `budget` wide.
hipError_t launch_topk(const fasa_ctx* c, const float* scores, const int32_t* nb,
                       int max_seq_len, int budget, int32_t* idx, int32_t* advance, uint8_t* ws,
                       hipStream_t s, const int32_t* head_budget = nullptr);
// Streams n16 16-byte words from buf with reads only (fasa_read_probe).
hipError_t launch_read_probe(const void* buf, size_t n16, float* sink, hipStream_t stream);
// Largest n16 one probe launch takes.
constexpr size_t kReadProbeMax16 = (size_t)0x7fffffff * 2048;

hipError_t launch_fac(const fasa_ctx* c, const void* k_cache, const void* v_cache,
                      const int32_t* nb, int max_seq_len, const int32_t* idx, int budget,
                      float* out, uint8_t* ws, hipStream_t s);
hipError_t launch_dense(const fasa_ctx* c, const void* k_cache, const void* v_cache,
                        const int32_t* nb, int max_seq_len, float* out, uint8_t* ws,
                        hipStream_t s);
// bf16 caches at d = 128: validation, query rotation and dense decode in one
// launch (matrix cores for q . K), then the merge (attention.hip).
hipError_t launch_dense_fused(const fasa_ctx* c, const void* k_cache, const void* v_cache,
                              const void* q, const int32_t* seq_lens, int max_seq_len,
                              float* out, uint8_t* ws, hipStream_t s);
// Top-B selection fused with FAC (budget <= kFusedMaxBudget): one workgroup
// per (h, b) selects and attends; idx may be null.
hipError_t launch_select_attend(const fasa_ctx* c, const float* scores, const int32_t* nb,
                                int max_seq_len, int budget, int32_t* idx, const void* k_cache,
                                const void* v_cache, float* out, int32_t* advance, uint8_t* ws,
                                hipStream_t s, const int32_t* head_budget = nullptr);
// Register-resident top-B (when select_path_applies(max_seq_len, budget)):
// rows up to kSelectChunk positions in one workgroup each, longer rows in
// chunks of at most kSelectChunk then their candidates, and, for budgets past
// kFusedMaxBudget, rows up to 40960 positions whole in one 1024-thread
// workgroup when chunks would not cut them much.  Fused with FAC when `out` is
// given (then budget <= kFusedMaxBudget and k_cache / v_cache too); idx may be
// null then.
bool select_path_applies(int max_seq_len, int budget);
// The launch plan above as fasa_select_layout reports it (kind 1 whole row,
// 2 chunked, 3 whole row in 1024 threads, 4 one workgroup per row).
struct SelectLayout {
  int kind = 4, threads = 0, per_thread = 0, chunk = 0;
};
SelectLayout select_layout(int max_seq_len, int budget);
hipError_t launch_select(const fasa_ctx* c, const float* scores, const int32_t* nb,
                         int max_seq_len, int budget, int32_t* idx, const void* k_cache,
                         const void* v_cache, float* out, int32_t* advance, uint8_t* ws,
                         hipStream_t s, const int32_t* head_budget = nullptr);
hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t s);
// *dst = *src (one device word, a one-thread kernel).
hipError_t launch_copy_u32(const uint32_t* src, uint32_t* dst, hipStream_t s);

// Filtered top-B + FAC of a decode step (filter.hip): one histogram pass over
// TIP's group maxima bounds the row's threshold from below; only the groups
// whose maximum clears that bound are read from the scores and selected
// exactly (streaming passes over the row where that would not fit).  Applies
// to fused budgets on rows longer than one whole-row select holds, up to
// kFilterMaxGroups groups.
constexpr int kFilterSelectThreads = 512;
constexpr int kFilterMaxGroups = kFilterSelectThreads * 20;
bool filter_path_applies(int max_seq_len, int budget);
// Group-maximum keys per thread of the filter select's first pass (4 or 20),
// and survivor slots per thread of its second (12 or 40).
int filter_group_slots(int max_seq_len);
int filter_survivor_slots(int budget);
// whole_rows: one workgroup per row even when the rows are few (K and V in
// host memory: each row crosses the host link once instead of once per
// column part).
hipError_t launch_filter_select(const fasa_ctx* c, const float* scores, const int32_t* nb,
                                int max_seq_len, int budget, int32_t* idx, const void* k_cache,
                                const void* v_cache, float* out, int32_t* advance, uint8_t* ws,
                                hipStream_t s, const int32_t* head_budget = nullptr,
                                bool whole_rows = false);

// Calibration (calibrate.hip): its workspace regions (err, nb, qrot, scores
// [b][Hq (C + 1)][cap], idx [b][Hq (C + 1)][topk], cand), and the launcher.
struct CalLayout {
  WsLayout ws;
};
CalLayout calib_layout(const fasa_ctx* c, int topk);
// Largest k the agreement kernel keeps in LDS.
constexpr int kCalibMaxTopk = 8192;
hipError_t launch_calibrate(const fasa_ctx* c, const void* k_cache, const void* q,
                            const int32_t* seq_lens, int max_seq_len, int topk, float* ca,
                            uint8_t* ws, hipStream_t s);

}  // namespace fasa
