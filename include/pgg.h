/*
 * pgg.h — C ABI of the MI355X (gfx950) fused MoE backward that produces d_x.
 *
 * The operation (MoeInitRoutingGroupedMatmulGrad design page, §数学定义和公式):
 *
 *     d_x[b,k] = sum over expanded rows i with p(i) / topK == b
 *                of  sum_n d_y[i,n] * W[g(i),k,n]
 *
 * i.e. the grouped-matmul gradient d_y · Wᵀ (Step 1) fused with the routing
 * scatter-add back to the tokens (Step 2).  fp32 tiles go through a
 * workspace ring of at most 1 GiB, whatever M, and a consumer stage adds
 * them into d_x in a fixed order with no floating-point atomics, so repeated
 * calls give bit-identical results.  The ring holds min(M*K*4 bytes, the
 * bound): when the whole fp32 [M,K] intermediate fits under the bound (small
 * M), a one-chunk plan's ring is exactly that intermediate; above it the ring
 * holds one chunk of rows of one column panel.
 *
 * Two-phase use, as in the page's aclnn interface (§2.2.2): ask for the
 * workspace size from the shapes alone, allocate it, then call the execute
 * entry point.  The library never allocates, frees or synchronises inside
 * pgg_moe_dx; it only enqueues kernels on the caller's stream.
 *
 * Thread safety: every entry point except pgg_timing_begin / pgg_timing_end
 * is reentrant.
 * Calls that share a workspace must be ordered by the caller (same stream or
 * explicit events).
 */
#ifndef PGG_H
#define PGG_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of grad_y and weight (§1.2 I/O table: FLOAT / FLOAT16 / BF16). */
typedef enum { PGG_F32 = 0, PGG_F16 = 1, PGG_BF16 = 2 } pgg_dtype;

/* Host-side status of every entry point. */
typedef enum {
  PGG_OK = 0,
  PGG_ERR_INVALID_ARG = 1,          /* a constraint of §1.2 / §2.3 is violated, or a NULL pointer */
  PGG_ERR_UNSUPPORTED = 2,          /* valid per the page but beyond this library (e.g. M >= 2^31) */
  PGG_ERR_WORKSPACE_TOO_SMALL = 3,  /* workspace_bytes below pgg_moe_dx_workspace_size */
  PGG_ERR_HIP = 4,                  /* a HIP runtime call failed */
  PGG_ERR_MISALIGNED = 5            /* workspace not 256-byte aligned, or an input / output pointer
                                       not aligned to its element size */
} pgg_status;

/* Data-dependent errors found on the device (read with
 * pgg_moe_dx_read_device_error).  When one is set, d_x is unspecified. */
typedef enum {
  PGG_DEV_OK = 0,
  PGG_DEV_GROUP_NEGATIVE = 1,       /* group_list[g] < 0; detail = g */
  PGG_DEV_GROUP_SUM = 2,            /* sum(group_list) != M; detail = the sum (clamped to >= 0) */
  PGG_DEV_INDEX_RANGE = 3,          /* expanded_row_idx[t] outside [0, M); detail = t */
  PGG_DEV_INDEX_DUP = 4,            /* expanded_row_idx is not a permutation; detail = a repeated value */
  PGG_DEV_EXPERT_RANGE = 5          /* pgg_moe_routing: an expert id outside [0, experts);
                                       detail = the smallest such position */
} pgg_device_error;

/*
 * Problem descriptor.  All sizes are element counts; every tensor is dense
 * and row-major (last index fastest).
 *
 *   grad_y            [grad_y_rows = M, grad_y_cols = N]          dtype
 *   weight            [weight_groups = G, weight_rows = K, weight_cols = N]  dtype
 *   expanded_row_idx  [idx_len = L]                                int64
 *   group_list        [group_list_len = G]                         int64
 *   grad_x (output)   [batch, K]                                   float32, always
 *
 * Constraints checked on the host (§1.2 constraints table, §2.3.3 checks):
 * grad_y_cols == weight_cols; group_list_len == weight_groups; topk > 0;
 * batch > 0; row_idx_type in {0, 1}; grad_y_dtype == weight_dtype; and
 * L == M == batch * topk (the page bounds L by batch <= L <= batch*topK and
 * L >= M, which with M = batch*topK leaves only L == M).
 *
 * row_idx_type (§1.2 notes): 0 = gather, expanded_row_idx[i] is the original
 * position p = b*topK + j of expanded row i; 1 = scatter,
 * expanded_row_idx[p] is the expanded row of original position p.
 * group_list holds per-expert row counts (not a cumulative sum); expert g
 * owns the expanded rows [sum_{h<g} group_list[h], sum_{h<=g} group_list[h]).
 */
typedef struct {
  int64_t grad_y_rows, grad_y_cols;
  int64_t weight_groups, weight_rows, weight_cols;
  int64_t idx_len;
  int64_t group_list_len;
  int64_t batch, topk;
  int32_t row_idx_type;
  int32_t grad_y_dtype;   /* pgg_dtype */
  int32_t weight_dtype;   /* pgg_dtype */
  int32_t reserved;       /* must be 0 */
} pgg_moe_dx_desc;

/*
 * Workspace size in bytes for a descriptor (host only; shapes only; no HIP
 * call).  Returns PGG_ERR_INVALID_ARG / PGG_ERR_UNSUPPORTED for descriptors
 * pgg_moe_dx would reject (PGG_ERR_UNSUPPORTED: M >= 2^31, G >= 2^30,
 * N >= 2^31 or K >= 2^29).  The size is O(M + G) integer index tables plus
 * an fp32 tile ring of min(M*K*4 bytes, 1 GiB).
 * Three environment variables, read when a plan is made, tune the schedule
 * (the size and every call planned under the same setting follow them; a
 * fixed setting gives fixed results): PGG_RING_MB sets the ring bound in MiB
 * (at most 1024), PGG_PANEL_COLS the width of the column panels (ignored by
 * the weight sweep, which keeps one panel), and PGG_REGIME the producer
 * family: "large" (the 256- or 128-row tiles), "few" (the weight sweep, or
 * for fp32 the 64- or 128-row tiles) or "sweep" (the weight sweep).
 */
pgg_status pgg_moe_dx_workspace_size(const pgg_moe_dx_desc* desc, size_t* bytes);

/*
 * Enqueue the fused backward on `stream` (asynchronous; no host sync).
 *
 * grad_y, weight, expanded_row_idx, group_list: device pointers, read only.
 * grad_x: device pointer to batch*K floats; fully overwritten (no pre-zeroing
 *   needed).  It must not alias any input or the workspace.
 * workspace: device pointer, 256-byte aligned, at least the queried size;
 *   owned by the caller; its contents on entry are ignored.
 *
 * Host-checkable violations return a status before anything is enqueued.
 * Data-dependent violations (negative count, sum != M, index out of range,
 * index not a permutation) are recorded in the workspace; read them with
 * pgg_moe_dx_read_device_error.  Empty experts' weight slices are never read.
 */
pgg_status pgg_moe_dx(const pgg_moe_dx_desc* desc, const void* grad_y, const void* weight,
                      const int64_t* expanded_row_idx, const int64_t* group_list,
                      float* grad_x, void* workspace, size_t workspace_bytes,
                      hipStream_t stream);

/*
 * Allocation-free variant of pgg_moe_dx, for callers that cannot allocate
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same computation, arguments and results, without the
 * workspace argument.  The workspace is a fixed device array of 64 MiB inside
 * the library, one per GPU, held until the process ends; the ring is planned
 * to fit it (more chunks than pgg_moe_dx may use, so results equal
 * pgg_moe_dx's bit for bit when both plans coincide and otherwise within the
 * same fp32 rounding bounds).  It calls no hipMalloc, hipFree or allocating
 * routine; the first call on a device looks up that device's array.
 *
 * device_error: NULL, or a device pointer to 2 int64 (8-byte aligned) that
 *   receive, after the call's kernels, the device error of this call as
 *   [pgg_device_error code, detail] ([0, 0] when there is none).
 * Errors: those of pgg_moe_dx, and PGG_ERR_WORKSPACE_TOO_SMALL when the
 * index tables plus the ring rows of one m-tile do not fit the 64 MiB (about
 * M > 8 million expanded rows, or a very wide K).
 * Every call on a GPU shares that GPU's array, which keeps the last call's
 * contents (every call rewrites all it reads): calls that overlap on one GPU
 * (different streams without ordering) race and give unspecified results.
 */
pgg_status pgg_moe_dx_noalloc(const pgg_moe_dx_desc* desc, const void* grad_y, const void* weight,
                              const int64_t* expanded_row_idx, const int64_t* group_list,
                              float* grad_x, int64_t* device_error, hipStream_t stream);

/*
 * Read the device error word of the last pgg_moe_dx (or pgg_moe_fwd,
 * pgg_moe_dw, pgg_moe_routing, pgg_moe_unpermute[_grad]) that used `workspace`.
 * Synchronises `stream`.  Reads the workspace's first 64 bytes (the error
 * word's region), which every workspace of those calls holds.  *code
 * receives a pgg_device_error; *detail its detail value (may be NULL).  When several violations exist, the one with
 * the smallest (code, detail) is reported, so the report is deterministic.
 */
pgg_status pgg_moe_dx_read_device_error(const void* workspace, hipStream_t stream,
                                        int32_t* code, int64_t* detail);

/*
 * Copy the index tables the last call built into host arrays (tests only;
 * synchronises `stream`).  `workspace` is that call's, of the size queried
 * for `desc`: the tables sit in its first table_bytes (pgg_moe_dx_plan).
 * inv_host[p] (length M) = expanded row of original position p; ori_host[i]
 * (length M) = original position of expanded row i.  Either pointer may be
 * NULL.
 */
pgg_status pgg_moe_dx_debug_tables(const pgg_moe_dx_desc* desc, const void* workspace,
                                   hipStream_t stream, int32_t* inv_host, int32_t* ori_host);

/*
 * The m-tile table the last call built (tests only; synchronises `stream`;
 * `workspace` as for pgg_moe_dx_debug_tables): tiles_host receives up to max_tiles entries of 3 int32 (expert, first
 * expanded row, row count), in expert order, empty experts contributing none;
 * *n_tiles the number of tiles.
 */
pgg_status pgg_moe_dx_debug_tiles(const pgg_moe_dx_desc* desc, const void* workspace,
                                  hipStream_t stream, int32_t* tiles_host, int32_t max_tiles,
                                  int32_t* n_tiles);

/* Execution plan the library picks for a descriptor (host only, for reports). */
typedef struct {
  int32_t regime;          /* 0 = large-M MFMA tiles, 1 = weight-streaming (small M), 2 = fp32 */
  int32_t block_m, block_n;/* output tile: expanded rows x output columns */
  int32_t tiles_per_chunk; /* m-tiles whose rows share one ring buffer */
  int32_t max_tiles;       /* upper bound on m-tiles: ceil(M/block_m) + G */
  int32_t max_chunks;      /* chunks enqueued per panel */
  int32_t ring_rows;       /* rows of one ring buffer: min(tiles_per_chunk * block_m, M) */
  int32_t fused_prep;      /* 1 when index preparation runs in one workgroup: a kernel of its
                              own, or -- one-chunk weight-streaming plans with G <= 256, when
                              the rows are 16-byte aligned -- a spare workgroup of the
                              producer launch; 0: three preparation kernels */
  int32_t n_panels;        /* column panels: the output columns are cut into panels of
                              panel_cols and each panel runs every chunk (tiled regimes;
                              the weight-streaming regime keeps one panel) */
  int32_t reserved0;
  int64_t panel_cols;      /* columns per panel and fp32 values per ring row */
  size_t ring_bytes;       /* fp32 ring: ring_rows x panel_cols */
  size_t table_bytes;      /* index / tile tables and header */
  size_t workspace_bytes;  /* total, as returned by pgg_moe_dx_workspace_size */
} pgg_plan;

pgg_status pgg_moe_dx_plan(const pgg_moe_dx_desc* desc, pgg_plan* plan);

/*
 * Kernel timing hook (benchmarks).  Between pgg_timing_begin and
 * pgg_timing_end, pgg_moe_dx records a HIP event on its stream before and
 * after every kernel it launches.  pgg_timing_begin creates `capacity` event
 * pairs (it allocates; never use it where allocation is forbidden) and
 * pgg_timing_end waits for them and reports, per kernel name, the number of
 * launches and their summed duration.  Not thread safe; one session at a
 * time per process.
 */
typedef struct {
  char name[32];
  int32_t launches;
  double total_ms;
} pgg_kernel_time;

pgg_status pgg_timing_begin(int32_t capacity);
pgg_status pgg_timing_end(pgg_kernel_time* out, int32_t max_out, int32_t* n_out);

/*
 * Kernel benchmark hook.  Runs one full pgg_moe_dx call (same arguments and
 * contract), which fills the workspace tables, then launches one kernel of
 * the path back to back, `repeats` times per (panel, chunk) launch of the call (which = 0:
 * the producer, the grouped-matmul stage; which = 1: the consumer, the
 * routing scatter-add), between two HIP events on `stream`, waits, and
 * returns the average duration of one launch in *avg_ms and the number of
 * such launches one pgg_moe_dx call makes in *launches_per_call (may be
 * NULL).  Back-to-back launches hide the dispatch latency a per-launch event
 * pair would add to a kernel of ~100 us.  Repeated producers rewrite the
 * ring with the values a call leaves there; repeated consumers work on a ring
 * that holds only the last chunk, so after them one more full call is
 * enqueued: grad_x and the workspace end as after pgg_moe_dx.  Creates two
 * events (it allocates).  Errors: those of pgg_moe_dx; PGG_ERR_INVALID_ARG
 * for `which` outside {0, 1}, repeats <= 0 or avg_ms NULL.
 */
pgg_status pgg_moe_dx_kernel_time(const pgg_moe_dx_desc* desc, const void* grad_y,
                                  const void* weight, const int64_t* expanded_row_idx,
                                  const int64_t* group_list, float* grad_x, void* workspace,
                                  size_t workspace_bytes, hipStream_t stream, int32_t which,
                                  int32_t repeats, double* avg_ms, int32_t* launches_per_call);

/*
 * Forward of the same layer: MoeInitRouting (Permute) followed by
 * GroupedMatmul (MoeInitRoutingGroupedMatmulGrad design page, §数学定义和公式,
 * forward formulas; §1.1 steps 1 and 2):
 *
 *     expanded_x[i,:] = x[p(i) / topK, :]
 *     y[i,n]          = sum_k expanded_x[i,k] * W[g(i),k,n]
 *
 * with p(i) the original position of expanded row i and g(i) its expert, as
 * for pgg_moe_dx.  expanded_x is never stored: every output tile gathers its
 * rows of x directly.  fp32 accumulation; y is float32, always.
 *
 *   x                 [x_rows = batch, x_cols = K]                  dtype
 *   weight            [weight_groups = G, weight_rows = K, weight_cols = N]  dtype
 *   expanded_row_idx  [idx_len = M = batch * topk]                  int64
 *   group_list        [group_list_len = G]                          int64
 *   y (output)        [M, N]                                        float32
 *
 * y rows are in expanded (expert-grouped) order: row i belongs to expert g(i).
 * Constraints checked on the host: x_rows == batch; x_cols == weight_rows;
 * group_list_len == weight_groups; topk > 0; batch > 0; idx_len ==
 * batch * topk; row_idx_type in {0, 1}; x_dtype == weight_dtype.
 */
typedef struct {
  int64_t x_rows, x_cols;
  int64_t weight_groups, weight_rows, weight_cols;
  int64_t idx_len;
  int64_t group_list_len;
  int64_t batch, topk;
  int32_t row_idx_type;
  int32_t x_dtype;        /* pgg_dtype */
  int32_t weight_dtype;   /* pgg_dtype */
  int32_t reserved;       /* must be 0 */
} pgg_moe_fwd_desc;

/* Workspace size of the forward (host only; shapes only): O(M + G) integer
 * index and tile tables, plus -- for few rows per expert (M <= 64 G, 16-bit
 * types), when the reduction is split over workgroups -- fp32 partials of y,
 * ksplit x M x N floats with ksplit <= 8. */
pgg_status pgg_moe_fwd_workspace_size(const pgg_moe_fwd_desc* desc, size_t* bytes);

/*
 * Enqueue the forward on `stream` (asynchronous; no host sync, no allocation).
 * x, weight, expanded_row_idx, group_list: device pointers, read only.
 * y: device pointer to M*N floats; every row of a non-empty expert is fully
 *   written (with group_list summing to M, that is all of y).  It must not
 *   alias an input or the workspace.
 * workspace: device pointer, 256-byte aligned, at least the queried size;
 *   owned by the caller; contents on entry ignored.
 * Errors: host-checkable violations return a status before anything is
 * enqueued (PGG_ERR_MISALIGNED for a workspace not 256-byte aligned or an
 * input / output pointer not aligned to its element size).  Data-dependent
 * violations set the workspace's error word, as for pgg_moe_dx (then y is
 * unspecified); pgg_moe_dx_read_device_error reads it from this workspace
 * too.  Empty experts' weight slices are never read.
 */
pgg_status pgg_moe_fwd(const pgg_moe_fwd_desc* desc, const void* x, const void* weight,
                       const int64_t* expanded_row_idx, const int64_t* group_list, float* y,
                       void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Plan of the forward (host only): regime 0 = 256x256 tiles, 1 = 32-row
 * m-tiles for few rows per expert, 2 = fp32; tiles_per_chunk = max_tiles,
 * max_chunks = 1; ring_rows / ring_bytes describe the split partials
 * (ksplit x M rows of N floats; 0 when the reduction is not split). */
pgg_status pgg_moe_fwd_plan(const pgg_moe_fwd_desc* desc, pgg_plan* plan);

/*
 * Kernel benchmark hook of the forward: one full pgg_moe_fwd call (same
 * contract), then its grouped-matmul kernel `repeats` times back to back
 * between two HIP events on `stream`; waits and returns the average duration
 * of one launch in *avg_ms.  Repeats rewrite y with the same values.  Creates
 * two events (it allocates).  Errors: those of pgg_moe_fwd;
 * PGG_ERR_INVALID_ARG for repeats <= 0 or avg_ms NULL.
 */
pgg_status pgg_moe_fwd_kernel_time(const pgg_moe_fwd_desc* desc, const void* x, const void* weight,
                                   const int64_t* expanded_row_idx, const int64_t* group_list,
                                   float* y, void* workspace, size_t workspace_bytes,
                                   hipStream_t stream, int32_t repeats, double* avg_ms);

/*
 * Weight gradient of the same layer: the operator the design page leaves
 * d_weight to (MoeInitRoutingGroupedMatmulGrad design page, §1.2, expanded_x^T
 * @ d_y per expert), with the permute fused into the operand load:
 *
 *     grad_w[g,k,n] = sum over expert g's expanded rows i of x[p(i)/topK, k] * grad_y[i, n]
 *
 * fp32 accumulation; grad_w is float32 [G, K, N], fully overwritten (an expert
 * without rows gets zeros).  Each output element is reduced by one
 * workgroup in a fixed order, so repeated calls give bit-identical results.
 * It takes the forward's descriptor: x [x_rows = batch, x_cols = K],
 * weight_groups / weight_rows / weight_cols = G, K, N (the shape of grad_w),
 * expanded_row_idx and group_list as for pgg_moe_dx; grad_y is [batch*topk, N]
 * in the same dtype (x_dtype == weight_dtype names it).
 * Errors and workspace rules as for pgg_moe_fwd; the workspace holds only
 * the O(M + G) index tables.
 */
pgg_status pgg_moe_dw_workspace_size(const pgg_moe_fwd_desc* desc, size_t* bytes);
pgg_status pgg_moe_dw(const pgg_moe_fwd_desc* desc, const void* x, const void* grad_y,
                      const int64_t* expanded_row_idx, const int64_t* group_list, float* grad_w,
                      void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Kernel benchmark hook of the weight gradient, as pgg_moe_fwd_kernel_time. */
pgg_status pgg_moe_dw_kernel_time(const pgg_moe_fwd_desc* desc, const void* x, const void* grad_y,
                                  const int64_t* expanded_row_idx, const int64_t* group_list,
                                  float* grad_w, void* workspace, size_t workspace_bytes,
                                  hipStream_t stream, int32_t repeats, double* avg_ms);

/*
 * MoeInitRouting on the device (MoeInitRoutingGroupedMatmulGrad design page,
 * §1.1 step 1: tokens grouped by expert, semantically a permute; original
 * position p = b*topK + j as in §数学定义和公式): from the router's choices
 * it builds the tables the operators above take.
 *
 *   expert_ids   [batch, topk] int64, each in [0, experts)       input
 *   x            [batch, x_cols] x_dtype (only when x_cols > 0)  input
 *   group_list   [experts] int64: rows per expert                output
 *   eri_gather   [M] int64: original position of expanded row i (row_idx_type 0)   output, may be NULL
 *   eri_scatter  [M] int64: expanded row of position p (row_idx_type 1)            output, may be NULL
 *   expanded_x   [M, x_cols] x_dtype: row i = x[eri_gather[i] / topk]              output, may be NULL
 *
 * Expanded rows are grouped by expert in expert order and keep ascending p
 * inside an expert (the page fixes no order there; this stable order makes
 * the tables unique), so repeated calls give identical tables.  An id outside
 * [0, experts) sets the workspace error word (PGG_DEV_EXPERT_RANGE, read with
 * pgg_moe_dx_read_device_error); the outputs are then unspecified.  Limits:
 * experts <= 8192, M < 2^31 and x_cols < 2^25 (PGG_ERR_UNSUPPORTED beyond).  Pointers:
 * expert_ids and the int64 outputs 8-byte aligned, x / expanded_x aligned to
 * their element size; workspace 256-byte aligned.
 */
typedef struct {
  int64_t batch, topk;
  int64_t experts;
  int64_t x_cols;         /* 0: no expanded_x */
  int32_t x_dtype;        /* pgg_dtype of x and expanded_x when x_cols > 0 */
  int32_t reserved;       /* must be 0 */
} pgg_moe_routing_desc;

pgg_status pgg_moe_routing_workspace_size(const pgg_moe_routing_desc* desc, size_t* bytes);
pgg_status pgg_moe_routing(const pgg_moe_routing_desc* desc, const int64_t* expert_ids,
                           const void* x, int64_t* group_list, int64_t* eri_gather,
                           int64_t* eri_scatter, void* expanded_x, void* workspace,
                           size_t workspace_bytes, hipStream_t stream);

/*
 * Unpermute and its gradient (TileLang-Ascend operator page, sections 4 and 5:
 * MoeTokenUnpermute, MoeTokenUnpermuteGrad), on this library's routing index
 * (expanded_row_idx and row_idx_type as for pgg_moe_dx); row(t, j) is the
 * expanded row of original position t*topk + j.  Values are widened to fp32,
 * multiplied and summed in fp32, and rounded once (round to nearest even) to
 * `dtype`, the type of every value tensor (probs included).
 *
 * With probs (non-NULL, [batch, topk]):
 *   pgg_moe_unpermute:       out [batch, H] = sum_j probs[t, j] * permuted[row(t, j)]   (slot order)
 *   pgg_moe_unpermute_grad:  perm_grad [M, H]: perm_grad[row(t, j)] = grad[t] * probs[t, j]
 *                            probs_grad [batch, topk] = sum_h grad[t, h] * permuted[row(t, j), h]
 *                            (grad is [batch, H]; a fixed summation order)
 * Without probs (NULL): the forward is the gather out [M, H], out[p] =
 * permuted[row(p)], and its gradient the scatter perm_grad[row(p)] = grad[p]
 * (grad [M, H]; permuted and probs_grad unused).
 *
 * Every output element is written.  The routing index is checked on the
 * device (out of range / not a permutation: the workspace error word, read
 * with pgg_moe_dx_read_device_error; outputs unspecified).  Value pointers
 * aligned to the element size, workspace 256-byte aligned.
 */
typedef struct {
  int64_t batch, topk;
  int64_t hidden;          /* H */
  int32_t row_idx_type;
  int32_t dtype;           /* pgg_dtype of permuted, probs, grad and the outputs */
  int32_t reserved;        /* must be 0 */
  int32_t pad;
} pgg_moe_unpermute_desc;

pgg_status pgg_moe_unpermute_workspace_size(const pgg_moe_unpermute_desc* desc, size_t* bytes);
pgg_status pgg_moe_unpermute(const pgg_moe_unpermute_desc* desc, const void* permuted,
                             const int64_t* expanded_row_idx, const void* probs, void* out,
                             void* workspace, size_t workspace_bytes, hipStream_t stream);
pgg_status pgg_moe_unpermute_grad(const pgg_moe_unpermute_desc* desc, const void* permuted,
                                  const void* grad, const int64_t* expanded_row_idx,
                                  const void* probs, void* perm_grad, void* probs_grad,
                                  void* workspace, size_t workspace_bytes, hipStream_t stream);

const char* pgg_status_string(pgg_status status);
const char* pgg_device_error_string(int32_t code);

#ifdef __cplusplus
}
#endif

#endif /* PGG_H */
