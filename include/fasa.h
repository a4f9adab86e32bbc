/*
 * fasa.h -- C ABI of the FASA decode hot path on MI355X (gfx950).
 *
 * FASA ("FASA: Frequency-aware Sparse Attention") scores every cached token
 * with only the dominant RoPE frequency chunks (FCs) of each query head (TIP),
 * keeps the top-B tokens per head (the critical set T_t) and runs full
 * attention over those tokens only (FAC).  Passages: gist.science/pt,
 * "Resumo Tecnico" section 2 ("A Descoberta"; TIP "Calibracao Offline" and
 * "Previsao Online"; FAC bullets) and "Variantes de Implementacao" (FASA-C keeps
 * the cache on the GPU and reads a sparse subset of it).
 *
 * Conventions shared by every call
 * --------------------------------
 * - Shapes are row-major.  b = batch, Hq = query heads, Hkv = KV heads,
 *   G = Hq / Hkv, d = head_dim (64 or 128), C = d / 2 FCs, cap = capacity.
 *   Query head h reads KV head h / G.
 * - FC c is the dimension pair (c, c + C) (rotate-half); its frequency is
 *   theta^(-2c/d); the angle at absolute position m is m * theta^(-2c/d),
 *   formed in fp64.  Under partial RoPE (fasa_create_partial_rope) only the
 *   first r = rotary_dim dims rotate: with R = r / 2, FC c < R is the pair
 *   (c, c + R) at theta^(-2c/r), and FC c >= R is the pass-through pair
 *   (c + R, c + C) at frequency 0 (stored and used as given).
 * - Element type ("dtype") of q, k_new, v_new, the K/V caches and the sidecar:
 *   FASA_F32 = float, FASA_BF16 = bfloat16 (raw 16-bit patterns).
 *   Accumulation is fp32; outputs and scores are float.
 * - K cache, V cache: [b][Hkv][cap][d] dtype.  Slot j holds absolute position
 *   j.  K holds RoPE(k, j) rounded once (nearest-even) to dtype; V holds v.
 *   Both may live in device memory or (FASA-M, same page, "Variantes de
 *   Implementacao") in pinned host memory the device maps at the same address
 *   (fasa_pointer_kind() says which); every other buffer is device memory.
 * - Sidecar: the K columns of each KV head's union U_g of its query heads'
 *   dominant FCs, packed FC-major so TIP reads them with coalesced loads:
 *   [b][P][cap] pairs, P = sum_g |U_g|, plane fasa_sidecar_layout() gives the
 *   FC of each plane; a pair is the K columns of the FC's two dims, lower dim
 *   first (bf16: low half; f32: two floats).  It is bit-identical to them.
 * - seq_lens: device int32 [b].  Its meaning is stated per call.
 * - max_seq_len: host-side upper bound on every sequence length the call
 *   will see on the device (sizes the launch grid); must be <= cap.
 * - Every device pointer is caller-owned (allocate with hipMalloc or a
 *   framework); the library owns only the context and its small constant
 *   tables.  All calls are asynchronous on `stream`, never synchronise, never
 *   allocate (except fasa_create / fasa_check).
 * - Workspace: fasa_workspace_bytes() bytes of device memory, zero-filled
 *   before its first use (fasa_workspace_init does it); every call leaves it in
 *   that state again.  Calls that share one workspace must be ordered on one
 *   stream; calls on different workspaces may overlap.
 * - Errors: a call that finds a bad argument on the host returns a negative
 *   status and enqueues nothing; fasa_last_error() describes it.  Bad values
 *   only the device can see (a sequence length beyond max_seq_len or cap, an
 *   index >= its sequence length) set a sticky flag in the workspace; the
 *   affected rows produce zeros / -1 and fasa_check() reports the flag.
 * - Tracing (host side, off by default, read once per process): with
 *   FASA_LOG=1 every call below (getters aside) writes one line to stderr,
 *   "fasa: <call>(<arguments that shape its launches>)", and one more,
 *   "fasa: <call>: error <status>: <message>", when it refuses its
 *   arguments; with FASA_ROCTX=1 every such call is a roctx range (loaded from
 *   the ROCm marker library on first use; rocprofv3 --marker-trace records
 *   them around the call's kernels).
 */
#ifndef FASA_H
#define FASA_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct fasa_ctx fasa_ctx;

typedef enum {
  FASA_OK = 0,
  FASA_ERR_INVALID_ARG = -1,  /* bad shape, null pointer, out-of-range value */
  FASA_ERR_CAPACITY = -2,     /* max_seq_len / budget / rows beyond the ctx limits */
  FASA_ERR_UNSUPPORTED = -3,  /* valid but not built: d, G or dtype */
  FASA_ERR_HIP = -4,          /* a HIP runtime call failed */
  FASA_ERR_DEVICE_FLAG = -5   /* fasa_check found the device error flag set */
} fasa_status;

typedef enum { FASA_F32 = 0, FASA_BF16 = 1 } fasa_dtype;

/* fasa_decode_step flag: add 1 to every seq_lens[b] after the step. */
#define FASA_ADVANCE_SEQ_LENS 1u

/* Device error-flag bits (fasa_check's *flags). */
#define FASA_DEVFLAG_SEQ_LEN 1u   /* a sequence length outside [1, max_seq_len] or > cap */
#define FASA_DEVFLAG_INDEX 2u     /* an index >= its sequence length */
#define FASA_DEVFLAG_APPEND 4u    /* an append beyond cap */
#define FASA_DEVFLAG_BUDGET 8u    /* a per-head budget outside [0, budget] (clamped) */
#define FASA_DEVFLAG_SELECT 16u   /* a filtered selection found its tile lists inconsistent and
                                     fell back to reading the row (never expected) */

/*
 * Create a context for one attention layer's shapes.
 * dom_fc: host int32 [n_q_heads][n_dom], the offline-calibrated dominant FC
 *   indices I_dom of each query head (gist.science/pt, "Resumo Tecnico"
 *   section 2, TIP "Calibracao Offline"), each in [0, C), distinct per head.
 *   Copied; the caller keeps ownership.
 * Limits: head_dim 64 or 128; G in {1, 2, 4, 8}; n_kv_heads <= 128
 *   (FASA_ERR_UNSUPPORTED above); capacity a positive multiple of 64, at most
 *   2^24; 1 <= n_dom <= C; 1 <= max_budget <= capacity; batch * n_q_heads *
 *   ceil(max_budget / 256) at most about 8 million (one FAC launch; the
 *   exact bound rounds batch * n_kv_heads * ceil(max_budget / 256) up to a
 *   multiple of 8, times G, times 512 threads, below 2^32;
 *   FASA_ERR_UNSUPPORTED above).
 * Allocates the constant tables on the current HIP device (the device every
 * later call must run on).  *out is NULL on failure.
 */
fasa_status fasa_create(fasa_ctx** out, int batch, int n_q_heads, int n_kv_heads,
                        int head_dim, int capacity, double rope_theta,
                        fasa_dtype dtype, const int32_t* dom_fc, int n_dom,
                        int max_budget);

/*
 * fasa_create for heads with partial RoPE (gist.science/pt, "Resumo
 * Tecnico", "Contribuicoes": the functional sparsity also holds under
 * Partial-RoPE): only the first rotary_dim dims of each q and k row are
 * rotated (rotate-half within them, frequencies theta^(-2c/rotary_dim)); the
 * other dims pass through and are paired into zero-frequency FCs (see the
 * conventions above), which calibration and I_dom treat like any other FC.
 * rotary_dim: even, in [2, head_dim]; head_dim gives fasa_create.  Every other
 * argument and limit as fasa_create.
 */
fasa_status fasa_create_partial_rope(fasa_ctx** out, int batch, int n_q_heads, int n_kv_heads,
                                     int head_dim, int rotary_dim, int capacity,
                                     double rope_theta, fasa_dtype dtype, const int32_t* dom_fc,
                                     int n_dom, int max_budget);
void fasa_destroy(fasa_ctx* ctx);

/* Sizes in bytes of one K (or V) cache, the sidecar and the workspace. */
size_t fasa_kv_cache_bytes(const fasa_ctx* ctx);
size_t fasa_sidecar_bytes(const fasa_ctx* ctx);
size_t fasa_workspace_bytes(const fasa_ctx* ctx);

/*
 * Sidecar layout.  plane_offset: host int32 [Hkv + 1] (planes of KV head g
 * are plane_offset[g] .. plane_offset[g+1]-1); plane_fc: host int32 [P], the
 * FC held by each plane (ascending within a KV head).  Either may be NULL.
 * Returns P (>= 0) or a negative status.
 */
int fasa_sidecar_layout(const fasa_ctx* ctx, int32_t* plane_offset, int32_t* plane_fc);

/* Zero-fill a workspace (a fill kernel on `stream`, no memset node). */
fasa_status fasa_workspace_init(fasa_ctx* ctx, void* workspace, hipStream_t stream);

/*
 * Append n_new tokens per sequence (prefill, or a decode step's new token).
 * Rotates each key at its absolute position (start_pos[b] + t) with RoPE in
 * fp64, rounds once to dtype, writes the K row, the V row (copied) and the
 * sidecar pairs.  Source: gist.science/pt, "Resumo Tecnico" section 2, FAC
 * third bullet (absolute positions are kept) and "A Descoberta" (FCs);
 * section 1 (the cache grows per generated token).
 * k_new, v_new: device [b][Hkv][n_new][d] dtype, pre-RoPE.
 * start_pos: device int32 [b], first position written; rows past cap are
 *   skipped and raise FASA_DEVFLAG_APPEND.
 * n_new: >= 0 (0 is a no-op).  workspace: only its error flag is used.
 */
fasa_status fasa_append_kv(fasa_ctx* ctx, void* k_cache, void* v_cache, void* sidecar,
                           const void* k_new, const void* v_new,
                           const int32_t* start_pos, int n_new, void* workspace,
                           hipStream_t stream);

/*
 * TIP scores (gist.science/pt, "Resumo Tecnico" section 2, TIP "Previsao
 * Online"): for every query head h and cached token j < n_b,
 *   scores[b][h][j] = sum_{c in I_dom(h)} q~_c K[j][c] + q~_{c+C} K[j][c+C],
 * with q~ = RoPE(q, n_b - 1) kept in fp32.  Read from the sidecar only.
 * q: device [b][Hq][d] dtype, pre-RoPE.  seq_lens[b] = n_b, tokens scored
 * (the query's position is n_b - 1).  scores: device float [b][Hq][cap];
 * entries j >= n_b are not written.
 */
fasa_status fasa_tip_scores(fasa_ctx* ctx, const void* sidecar, const void* q,
                            const int32_t* seq_lens, int max_seq_len, float* scores,
                            void* workspace, hipStream_t stream);

/*
 * Top-B selection of the critical set T_t (gist.science/pt, "Resumo Tecnico"
 * section 2, FAC first bullet): per (b, h), the min(budget, n_b) positions
 * with the highest scores[b][h][0 .. n_b), equal scores going to the lower
 * position, written ascending to idx[b][h][0 ..] and padded with -1 up to
 * budget.  Exact (radix select on order-preserving keys of the fp32 scores).
 * scores: device float [b][Hq][cap]; seq_lens[b] = n_b; 1 <= budget <=
 * max_budget; idx: device int32 [b][Hq][budget].
 */
fasa_status fasa_topk(fasa_ctx* ctx, const float* scores, const int32_t* seq_lens,
                      int max_seq_len, int budget, int32_t* idx, void* workspace,
                      hipStream_t stream);

/*
 * Top-B with a budget per query head (the pages' "Variantes de Implementacao"
 * note that FASA composes with budget allocation across layers; a per-layer
 * budget is the `budget` of each layer's call, and this call lets the heads
 * of one layer differ too).  As fasa_topk with B = head_budget[h] for query
 * head h: idx[b][h][0 .. min(B, n_b)) holds the set, ascending, and -1 fills
 * the row up to `budget`.  head_budget: device int32 [Hq], each in
 * [0, budget] (0: the head selects nothing); a value outside is clamped into
 * that range and raises FASA_DEVFLAG_BUDGET.  budget: as for fasa_topk, the
 * idx row width and an upper bound on every head_budget[h].
 */
fasa_status fasa_topk_per_head(fasa_ctx* ctx, const float* scores, const int32_t* seq_lens,
                               int max_seq_len, const int32_t* head_budget, int budget,
                               int32_t* idx, void* workspace, hipStream_t stream);

/*
 * FAC (gist.science/pt, "Resumo Tecnico" section 2, FAC second and third
 * bullets): per (b, h), attention of q~ = RoPE(q, n_b - 1) over the rows
 * idx[b][h][0 .. min(budget, n_b)) of the caches only:
 *   out = sum_j softmax_j(q~ . K[j] / sqrt(d)) V[j], softmax over those rows.
 * Entries < 0 are skipped; an entry >= n_b is skipped and raises
 * FASA_DEVFLAG_INDEX.  A head with no row gets zeros.
 * q: device [b][Hq][d] dtype, pre-RoPE; seq_lens[b] = n_b; idx: device int32
 * [b][Hq][budget]; out: device float [b][Hq][d].
 */
fasa_status fasa_sparse_attn(fasa_ctx* ctx, const void* k_cache, const void* v_cache,
                             const void* q, const int32_t* seq_lens, const int32_t* idx,
                             int budget, float* out, void* workspace, hipStream_t stream);

/*
 * One whole decode step (gist.science/pt, "Resumo Tecnico" sections 1-2):
 * append the new token at position seq_lens[b] (as fasa_append_kv), then
 * with n_b = seq_lens[b] + 1 run TIP, top-B and FAC as the three calls
 * above, the query at position n_b - 1.
 * seq_lens: device int32 [b], tokens cached BEFORE this step; incremented on
 *   the device after the step when flags has FASA_ADVANCE_SEQ_LENS.
 * max_seq_len >= every n_b of this step.  q: [b][Hq][d]; k_new, v_new:
 * [b][Hkv][d] (pre-RoPE, dtype).  out: float [b][Hq][d].  idx_out: int32
 * [b][Hq][budget] or NULL.
 */
fasa_status fasa_decode_step(fasa_ctx* ctx, void* k_cache, void* v_cache, void* sidecar,
                             const void* q, const void* k_new, const void* v_new,
                             int32_t* seq_lens, int max_seq_len, int budget, float* out,
                             int32_t* idx_out, void* workspace, unsigned flags,
                             hipStream_t stream);

/*
 * fasa_decode_step with a budget per query head: the top-B stage is
 * fasa_topk_per_head's, so query head h attends over its min(head_budget[h],
 * n_b) selected rows (a head with budget 0 outputs zeros).  head_budget:
 * device int32 [Hq] in [0, budget]; budget: idx_out row width and upper bound.
 */
fasa_status fasa_decode_step_per_head(fasa_ctx* ctx, void* k_cache, void* v_cache,
                                      void* sidecar, const void* q, const void* k_new,
                                      const void* v_new, int32_t* seq_lens, int max_seq_len,
                                      const int32_t* head_budget, int budget, float* out,
                                      int32_t* idx_out, void* workspace, unsigned flags,
                                      hipStream_t stream);

/*
 * fasa_decode_step for callers that cannot allocate: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  Same
 * arguments and results as fasa_decode_step (no head budgets), except that
 * the workspace is a file-scope device array of the library, 64 MiB per GPU
 * (FASA_STATIC_SCRATCH_BYTES), held until the process ends: a context whose
 * fasa_workspace_bytes exceeds it is refused with FASA_ERR_CAPACITY before
 * anything is enqueued.  The call allocates nothing (no hipMalloc, hipFree or
 * allocating library routine); its first call on a device looks the array's
 * device address up once, with the context's device current.  Every call on
 * a GPU shares that GPU's array, which keeps the last call's contents: the
 * call clears the device error flag word first, so calls that overlap on one
 * GPU (other streams, other host threads) race and must be ordered by the
 * caller.  dev_flags: device uint32 (may be NULL) that receives the call's
 * FASA_DEVFLAG_* bits (fasa_check cannot reach the array).
 */
#define FASA_STATIC_SCRATCH_BYTES ((size_t)64 << 20)
fasa_status fasa_decode_step_static(fasa_ctx* ctx, void* k_cache, void* v_cache, void* sidecar,
                                    const void* q, const void* k_new, const void* v_new,
                                    int32_t* seq_lens, int max_seq_len, int budget, float* out,
                                    int32_t* idx_out, uint32_t* dev_flags, unsigned flags,
                                    hipStream_t stream);

/*
 * Dense full-KV decode attention over all n_b cached tokens (the comparator
 * the pages measure FASA against: full KV, gist.science/pt, "Resumo Tecnico"
 * section 4).  seq_lens[b] = n_b; out: float [b][Hq][d].
 */
fasa_status fasa_dense_attn(fasa_ctx* ctx, const void* k_cache, const void* v_cache,
                            const void* q, const int32_t* seq_lens, int max_seq_len,
                            float* out, void* workspace, hipStream_t stream);

/*
 * Offline calibration of the dominant FCs (gist.science/pt, "Resumo Tecnico"
 * section 2, TIP "Calibracao Offline": I_dom of each head comes from a
 * contextual agreement between one FC's attention scores and the full
 * head's on a small calibration set).  The pages give no formula; here the
 * agreement of FC c for one calibration query of head h is
 *   CA = |top_k(s_c) intersect top_k(s)| / min(k, n_b),
 * with s_c[j] = q~_c K[j][c] + q~_{c+C} K[j][c+C] FC c's score, s = sum_c s_c
 * the full head's, and top_k the selection rule of fasa_topk (ties to the
 * lower position).  Each sequence b of the context is one calibration
 * sample: q is its query (pre-RoPE, rotated to position n_b - 1),
 * seq_lens[b] = n_b its cached tokens in k_cache (filled by fasa_append_kv).
 * The context's own dominant FCs are not used (any valid set will do).
 * k_cache: device [b][Hkv][cap][d] dtype; q: device [b][Hq][d] dtype;
 * seq_lens: device int32 [b]; topk in [1, min(8192, capacity)]; ca: device
 * float [b][Hq][C], written.  workspace: device, at least
 * fasa_calibrate_workspace_bytes(ctx, topk) bytes, zero-filled once with
 * fasa_workspace_init-style zeros (any earlier fasa_calibrate leaves it
 * valid); holds the full score matrix, b * Hq * (C + 1) * cap floats.
 * Errors: host-checkable arguments as the other calls; lengths outside
 * [0, min(max_seq_len, capacity)] raise FASA_DEVFLAG_SEQ_LEN (zeros written).
 */
size_t fasa_calibrate_workspace_bytes(const fasa_ctx* ctx, int topk);
fasa_status fasa_calibrate(fasa_ctx* ctx, const void* k_cache, const void* q,
                           const int32_t* seq_lens, int max_seq_len, int topk, float* ca,
                           void* workspace, hipStream_t stream);

/*
 * Host-only: I_dom from agreement values (no GPU call).  ca: host float
 * [samples][n_q_heads][n_fc]; per head the n_dom FCs of highest mean
 * agreement over the samples, equal means to the lower FC, written ascending
 * to dom_out: host int32 [n_q_heads][n_dom].  FASA_ERR_INVALID_ARG for a null
 * pointer or sizes out of range (1 <= n_dom <= n_fc, samples >= 1).
 */
fasa_status fasa_select_dominant(const float* ca, int samples, int n_q_heads, int n_fc,
                                 int n_dom, int32_t* dom_out);

/*
 * Where a buffer lives, for callers that place the K and V caches in host
 * memory (FASA-M, gist.science/pt, "Resumo Tecnico" section 2, "Variantes de
 * Implementacao": the value cache and the non-dominant key parts go to CPU
 * memory, the GPU keeps what TIP needs, here the sidecar).  Every call takes
 * such caches unchanged: kernels read and write them through the host link.
 * Returns FASA_PTR_DEVICE for device memory, FASA_PTR_HOST_MAPPED for pinned
 * host memory the current device reaches at the same address (hipHostMalloc,
 * torch pin_memory), FASA_PTR_UNUSABLE otherwise (pageable host memory, or a
 * pinned buffer whose device alias differs).  No GPU work is enqueued.
 */
typedef enum { FASA_PTR_UNUSABLE = 0, FASA_PTR_DEVICE = 1, FASA_PTR_HOST_MAPPED = 2 } fasa_ptr_kind;
fasa_ptr_kind fasa_pointer_kind(const void* ptr);

/*
 * A plain streaming read (a measurement aid, not part of the decode path):
 * one pass over `bytes` bytes of device memory at `buf` with 16-byte loads
 * and no stores (`sink`, one device float, is never written for real data).
 * Timed next to the TIP kernel, it shows what a kernel that only streams the
 * same number of bytes gets from HBM.  buf and bytes: non-zero multiples of
 * 16.  Asynchronous on `stream`.
 */
fasa_status fasa_read_probe(const void* buf, size_t bytes, float* sink, hipStream_t stream);

/*
 * The top-B layout that fasa_topk, fasa_decode_step and their per-head
 * variants use for rows of up to max_seq_len positions and a budget of
 * `budget` (the selection of gist.science/pt "Resumo Tecnico" section 2, FAC
 * first bullet).  A host-side query: no GPU work, no context needed.
 *   FASA_LAYOUT_WHOLE       each row held whole in one workgroup's registers;
 *   FASA_LAYOUT_CHUNKED     chunks of *chunk positions keep their own top B,
 *                           then one workgroup per row selects among those
 *                           candidates;
 *   FASA_LAYOUT_WHOLE_WIDE  each row whole in one 1024-thread workgroup
 *                           (budgets past 1024 on rows that chunks would not
 *                           cut much);
 *   FASA_LAYOUT_PER_ROW     one 512-thread workgroup per row reading its
 *                           scores in passes (rows no layout above fits).
 * *threads and *per_thread (workgroup size, elements held per thread)
 * describe the register-resident layouts (for FASA_LAYOUT_CHUNKED, its
 * candidate stage; 0 for FASA_LAYOUT_PER_ROW) and *chunk the chunk length (0
 * when the row is not chunked); each may be NULL.  Returns FASA_LAYOUT_NONE (outputs
 * untouched) for max_seq_len < 1 or budget < 1.
 */
typedef enum {
  FASA_LAYOUT_NONE = 0,
  FASA_LAYOUT_WHOLE = 1,
  FASA_LAYOUT_CHUNKED = 2,
  FASA_LAYOUT_WHOLE_WIDE = 3,
  FASA_LAYOUT_PER_ROW = 4
} fasa_select_layout_kind;
fasa_select_layout_kind fasa_select_layout(int max_seq_len, int budget, int* threads,
                                           int* per_thread, int* chunk);

/*
 * The top-B layout of a decode step (fasa_decode_step and its per-head
 * variant) for rows of up to max_seq_len positions at `budget`: the same as
 * fasa_select_layout, except FASA_LAYOUT_GROUP_FILTER where the step filters.
 * There the TIP launch also writes, per query head, the largest score of
 * every 16 consecutive tokens, and one launch selects and runs FAC: the B-th
 * largest group maximum bounds the B-th largest score from below (group
 * maxima are scores of distinct tokens), so only groups whose maximum
 * reaches that bound's histogram bin are read again and selected exactly;
 * rows where those would not fit are selected by streaming passes over their
 * scores.  The result is the exact T_t either way (gist.science/pt "Resumo
 * Tecnico" section 2, FAC first bullet).  The step filters when
 * budget <= 1024 and 8192 < max_seq_len <= 163840.  *threads = 512 there,
 * *per_thread = group maxima held per thread (4 or 20), *chunk = 16 (the
 * group); each may be NULL.  Host-side, no context needed.  Returns
 * FASA_LAYOUT_NONE for max_seq_len < 1 or budget < 1.
 */
#define FASA_LAYOUT_GROUP_FILTER ((fasa_select_layout_kind)5)
fasa_select_layout_kind fasa_decode_layout(int max_seq_len, int budget, int* threads,
                                           int* per_thread, int* chunk);

/*
 * Synchronise `stream`, read and clear the workspace's device error flag.
 * *flags (may be NULL) receives the FASA_DEVFLAG_* bits.  Returns
 * FASA_ERR_DEVICE_FLAG when any bit was set.
 */
fasa_status fasa_check(fasa_ctx* ctx, void* workspace, hipStream_t stream, uint32_t* flags);

/*
 * Kernel timing with HIP events (a measurement aid, off by default).  While
 * enabled, every launch made by the calls above is bracketed by a pair of
 * hipEvents recorded on the call's stream, grouped by kernel family.
 * fasa_timing_collect waits for the recorded events, adds each family's
 * elapsed milliseconds and launch count into total_ms[FASA_K_COUNT] and
 * launches[FASA_K_COUNT] (host arrays, may be NULL) and forgets them.  At
 * most 4096 launches are kept between collects; later ones are not timed.
 * Not for use under stream capture.
 */
typedef enum {
  FASA_K_APPEND = 0,    /* bulk append kernel */
  FASA_K_PROLOGUE = 1,  /* query rotation of fasa_sparse_attn / fasa_dense_attn */
  FASA_K_TIP = 2,       /* TIP scoring over the sidecar, with the step's query
                           rotation and (fasa_decode_step) token append fused in */
  FASA_K_TOPK = 3,      /* the three top-B kernels together */
  FASA_K_FAC = 4,       /* sparse attention */
  FASA_K_DENSE = 5,     /* dense comparator */
  FASA_K_SELECT_FAC = 6, /* top-B fused with FAC (budgets up to 1024) */
  FASA_K_CALIBRATE = 7, /* fasa_calibrate, all its kernels together */
  FASA_K_COUNT = 8
} fasa_kernel_family;
fasa_status fasa_timing_enable(fasa_ctx* ctx, int enable);
fasa_status fasa_timing_collect(fasa_ctx* ctx, double* total_ms, int32_t* launches);

const char* fasa_status_string(fasa_status status);
/* Detail of the last host-side error on the calling thread ("" if none). */
const char* fasa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* FASA_H */
