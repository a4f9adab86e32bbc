// Host-side context, workspace layout and kernel launchers of libfasa.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <vector>

#include "../../include/fasa.h"

namespace fasa {

// Device-resident constant tables, one allocation.
struct DeviceTables {
  int32_t* plane_off;  // [Hkv + 1]
  int32_t* fc_slot;    // [Hkv][C]: plane index within the KV head, or -1
  uint64_t* dom_mask;  // [Hq]: bit c set when FC c is dominant for head h
  double* omega;       // [C]: theta^(-2c/d), fp64
};

// Byte offsets of the workspace regions (each 256-byte aligned).
struct WsLayout {
  size_t err = 0;       // uint32 [4]
  size_t nb = 0;        // int32 [b]: tokens attended by the current call
  size_t qrot = 0;      // float [b][Hq][d]: rotated queries
  size_t tipw = 0;      // float [b][P][G][2]: TIP weights per sidecar plane
  size_t scores = 0;    // float [b][Hq][cap]
  size_t hist = 0;      // uint32 [b*Hq][kHistBins]
  size_t ticket = 0;    // uint32 [b*Hq][kTicketsPerRow]
  size_t rowst = 0;     // RowState [b*Hq]
  size_t cand = 0;      // uint64 [b*Hq][cap]
  size_t chunk_gt = 0;  // uint32 [b*Hq][max_chunks]
  size_t chunk_off = 0; // uint32 [b*Hq][max_chunks]
  size_t idx = 0;       // int32 [b][Hq][max_budget]
  size_t fac = 0;       // float [b*Hq][fac_splits][d + 2]
  size_t dense = 0;     // float [b*Hq][dense_splits][d + 2]
  size_t total = 0;
  int max_chunks = 0;
  int fac_splits = 0;
  int dense_splits = 0;
};

}  // namespace fasa

struct fasa_ctx {
  int batch, hq, hkv, d, C, cap, G, F, max_budget;
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
};

namespace fasa {

// Rows of a FAC split and tokens of a dense split (one workgroup each).
constexpr int kFacSplitRows = 64;
constexpr int kDenseSplitTokens = 256;

// Modes of the query-rotation prologue.
enum PrologueMode : int {
  kPrologueQueryOnly = 0,  // seq_lens = n_b; rotate q at n_b - 1
  kPrologueDecode = 1      // seq_lens = cached tokens; append at that position first
};

struct PrologueArgs {
  const void* q;
  const void* k_new;  // decode mode only
  const void* v_new;
  void* k_cache;
  void* v_cache;
  void* sidecar;
  const int32_t* seq_lens;
  int max_seq_len;
};

// Every launcher reads n_b (tokens attended) from `nb`, a device int32 [b];
// a value outside [0, min(max_seq_len, cap)] raises FASA_DEVFLAG_SEQ_LEN and
// the row is treated as empty.
hipError_t launch_append(const fasa_ctx* c, void* k_cache, void* v_cache, void* sidecar,
                         const void* k_new, const void* v_new, const int32_t* start_pos,
                         int n_new, uint8_t* ws, hipStream_t s);
// Writes ws.nb, ws.qrot and ws.tipw (and, in decode mode, appends the token).
hipError_t launch_prologue(const fasa_ctx* c, PrologueMode mode, const PrologueArgs& a,
                           uint8_t* ws, hipStream_t s);
hipError_t launch_tip(const fasa_ctx* c, const void* sidecar, const int32_t* nb,
                      int max_seq_len, float* scores, int32_t* advance_seq_lens,
                      uint8_t* ws, hipStream_t s);
hipError_t launch_topk(const fasa_ctx* c, const float* scores, const int32_t* nb,
                       int max_seq_len, int budget, int32_t* idx, uint8_t* ws, hipStream_t s);
hipError_t launch_fac(const fasa_ctx* c, const void* k_cache, const void* v_cache,
                      const int32_t* nb, int max_seq_len, const int32_t* idx, int budget,
                      float* out, uint8_t* ws, hipStream_t s);
hipError_t launch_dense(const fasa_ctx* c, const void* k_cache, const void* v_cache,
                        const int32_t* nb, int max_seq_len, float* out, uint8_t* ws,
                        hipStream_t s);
hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t s);

}  // namespace fasa
