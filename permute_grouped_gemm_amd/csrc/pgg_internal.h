// Internal definitions shared by the host planner, the C ABI and the HIP
// kernels of the fused MoE d_x backward.  Not part of the public ABI.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime.h>

#include "pgg.h"

namespace pgg {

// ---------------------------------------------------------------------------
// Workspace header (offset 0).  `err` packs a device error as
// (code << 48) | detail and is lowered with atomicMin, so the smallest
// (code, detail) wins and the report does not depend on thread timing.
// kNoError means no error.
// ---------------------------------------------------------------------------
constexpr unsigned long long kNoError = ~0ull;
constexpr int kErrShift = 48;
constexpr unsigned long long kDetailMask = (1ull << kErrShift) - 1;

struct alignas(16) WsHeader {
  unsigned long long err;
  int32_t n_tiles;      // m-tiles actually produced by the group pass
  int32_t reserved0;
  int64_t reserved[6];
};

// One m-tile: up to block_m consecutive expanded rows of one expert.
struct alignas(16) MTile {
  int32_t g;
  int32_t row0;   // first expanded row
  int32_t rows;   // 1..block_m; 0 marks an unused slot
  int32_t pad;
};

enum Regime : int32_t { kLarge = 0, kStream = 1, kF32 = 2 };

// Workspace regions are aligned to 512 bytes, as the page's tiling aligns its
// workspace regions (MoeInitRoutingGroupedMatmulGrad design, §2.4.3).
constexpr size_t kRegionAlign = 512;
constexpr size_t kWorkspaceAlign = 256;

struct Plan {
  // problem: N is the reduction length and K the number of output columns
  // (the backward's N and K; a forward plan stores the forward's K in N and
  // its N in K)
  int64_t M, N, G, K, batch, topk;
  int32_t row_idx_type;
  int32_t dtype;
  // schedule
  int32_t regime;
  int32_t bm, bn;
  int32_t tc;          // m-tiles per chunk
  int32_t max_tiles;   // ceil(M/bm) + G
  int32_t max_chunks;  // ceil(max_tiles / tc)
  int32_t ring_rows;   // min(tc * bm, M)
  int32_t n_col_tiles; // column tiles of one panel: ceil(panel_cols / bn)
  int32_t n_panels;    // column panels: ceil(K / panel_cols)
  int64_t panel_cols;  // columns per panel (a multiple of bn, or K); the ring row length
  int32_t ksplit;      // forward, few rows per expert: reduction splits (partials in the ring region)
  int32_t kspan;       // reduction elements per split
  bool fused_prep;
  // large tiles with about one m-tile per expert: each weight slab is read
  // once, so its loads carry the non-temporal hint
  bool stream_weights;
  // layout (byte offsets into the workspace)
  size_t off_header, off_offsets, off_tiles, off_chunks, off_inv, off_ori, off_ring, total;
  size_t ring_bytes, table_bytes;
};

// Fills *plan from a descriptor; returns PGG_OK or the rejection status.
pgg_status make_plan(const pgg_moe_dx_desc* desc, Plan* plan);
// The same plan with its ring cut so the whole workspace fits max_total bytes
// (more chunks); PGG_ERR_WORKSPACE_TOO_SMALL when even one m-tile's ring rows
// and the tables do not fit.
pgg_status make_plan_within(const pgg_moe_dx_desc* desc, size_t max_total, Plan* plan);
// The forward's plan: one chunk holding every m-tile, no ring.
pgg_status make_fwd_plan(const pgg_moe_fwd_desc* desc, Plan* plan);
// The weight gradient's plan: the forward's validation and tables, no partials.
pgg_status make_dw_plan(const pgg_moe_fwd_desc* desc, Plan* plan);

// The allocation-free entry point's workspace: a fixed device array of this
// size per GPU (noalloc.hip).  noalloc_scratch returns the array's device
// address on the stream's device (looked up once per device);
// launch_export_error copies a workspace's error word, decoded into
// [code, detail], to a caller's device buffer.
constexpr size_t kNoAllocScratchBytes = size_t(64) << 20;
hipError_t noalloc_scratch(hipStream_t stream, void** ptr);
hipError_t launch_export_error(const WsHeader* hdr, int64_t* out, hipStream_t s);

// Views of the workspace regions.
struct WsView {
  WsHeader* hdr;
  int64_t* offsets;     // [G+1]
  MTile* tiles;         // [max_tiles]
  int32_t* chunk_row0;  // [max_chunks+1]
  int32_t* inv;         // [M]  original position -> expanded row
  int32_t* ori;         // [M]  expanded row -> original position
  float* ring;          // [ring_rows, panel_cols]
};

inline WsView ws_view(const Plan& p, void* ws) {
  char* b = static_cast<char*>(ws);
  WsView v;
  v.hdr = reinterpret_cast<WsHeader*>(b + p.off_header);
  v.offsets = reinterpret_cast<int64_t*>(b + p.off_offsets);
  v.tiles = reinterpret_cast<MTile*>(b + p.off_tiles);
  v.chunk_row0 = reinterpret_cast<int32_t*>(b + p.off_chunks);
  v.inv = reinterpret_cast<int32_t*>(b + p.off_inv);
  v.ori = reinterpret_cast<int32_t*>(b + p.off_ori);
  v.ring = reinterpret_cast<float*>(b + p.off_ring);
  return v;
}

// ---------------------------------------------------------------------------
// Kernel launchers (each enqueues exactly one kernel).
// ---------------------------------------------------------------------------
hipError_t launch_prep_fused(const Plan& p, const int64_t* eri, const int64_t* group_list,
                             const WsView& w, hipStream_t s);
hipError_t launch_prep_groups(const Plan& p, const int64_t* group_list, const WsView& w,
                              hipStream_t s);
hipError_t launch_prep_index(const Plan& p, const int64_t* eri, const WsView& w, hipStream_t s);
hipError_t launch_prep_verify(const Plan& p, const int64_t* eri, const WsView& w, hipStream_t s);

// Columns [lo, hi) of panel `panel`.
inline void panel_range(const Plan& p, int panel, int64_t* lo, int64_t* hi) {
  *lo = int64_t(panel) * p.panel_cols;
  *hi = *lo + p.panel_cols < p.K ? *lo + p.panel_cols : p.K;
}

// Producer: chunk c's m-tiles x the column tiles of one panel -> ring rows.
bool produce_uses_dma(const Plan& p, bool aligned);
hipError_t launch_produce_sweep(const Plan& p, int chunk, const void* grad_y, const void* weight,
                                bool aligned, const WsView& w, hipStream_t s);
// One-chunk weight-sweep plans with aligned rows and few groups: the producer
// launch also runs the index preparation (in a spare workgroup), replacing
// the preparation kernel.
constexpr int64_t kSweepPrepMaxGroups = 256;
bool sweep_can_prepare(const Plan& p, bool aligned);
hipError_t launch_produce_sweep_prepared(const Plan& p, const void* grad_y, const void* weight,
                                         const int64_t* eri, const int64_t* gl, const WsView& w,
                                         hipStream_t s);
hipError_t launch_produce_dma(const Plan& p, int chunk, int panel, const void* grad_y,
                              const void* weight, const WsView& w, hipStream_t s);
hipError_t launch_produce(const Plan& p, int chunk, int panel, const void* grad_y,
                          const void* weight, bool aligned, const WsView& w, hipStream_t s);

// Consumer: ordered scatter-add of chunk c's ring rows (one panel's columns)
// into d_x.  One chunk and up to kFewChunks chunks per panel are consumed by
// token; more chunks by ring row.
constexpr int kFewChunks = 4;
hipError_t launch_consume(const Plan& p, int chunk, int panel, const WsView& w, float* grad_x,
                          hipStream_t s);

const char* produce_kernel_name(const Plan& p);

// Unpermute and its gradient: workspace layout and launches.
struct UnpermutePlan {
  int64_t M, batch, topk, H;
  int32_t dtype, row_idx_type;
  size_t off_header, off_inv, off_ori, total;
};
pgg_status make_unpermute_plan(const pgg_moe_unpermute_desc* desc, UnpermutePlan* plan);
hipError_t launch_unpermute(const UnpermutePlan& p, void* ws, const int64_t* eri, const void* permuted,
                            const void* grad, const void* probs, void* out, void* probs_grad,
                            bool is_grad, hipStream_t s);

// MoeInitRouting on the device: workspace layout and launches.
struct RoutePlan {
  int64_t M, G, topk, K;
  int32_t dtype, nblocks;
  size_t off_header, off_table, off_bad, off_offsets, off_rows, total;
};
pgg_status make_routing_plan(const pgg_moe_routing_desc* desc, RoutePlan* plan);
hipError_t launch_routing(const RoutePlan& p, const int64_t* ids, const void* x, int64_t* group_list,
                          int64_t* eri_gather, int64_t* eri_scatter, void* expanded_x, void* ws,
                          bool vec, hipStream_t s);

// Forward grouped matmul with the permute gathered into the A operand:
// y[i, :] = x[ori[i] / topK, :] · W[g(i)] for every m-tile of the plan.
hipError_t launch_forward(const Plan& p, const void* x, const void* weight, float* y, bool aligned,
                          const WsView& w, hipStream_t s);
const char* forward_kernel_name(const Plan& p);
// 256x256 direct-to-LDS forward tile (16-bit types, 16-byte aligned rows).
// Weight gradient dW[g] = (rows of x gathered for expert g)^T · d_y[rows of g].
hipError_t launch_dw(const Plan& p, const void* x, const void* grad_y, float* dw, bool aligned,
                     const WsView& w, hipStream_t s);
const char* dw_kernel_name(const Plan& p);
// Direct-to-LDS weight-gradient tile (16-bit types, 16-byte aligned rows).
hipError_t launch_dw_large(const Plan& p, const void* x, const void* grad_y, float* dw,
                           const WsView& w, hipStream_t s);

// Sum of the forward's reduction splits, in split order, into y.
hipError_t launch_forward_reduce(const Plan& p, const WsView& w, float* y, hipStream_t s);
hipError_t launch_forward_large(const Plan& p, const void* x, const void* weight, float* y,
                                const WsView& w, hipStream_t s);

}  // namespace pgg
