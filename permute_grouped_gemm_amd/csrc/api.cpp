// C ABI of the fused MoE d_x backward, of the layer's forward, of its weight
// gradient, of on-device routing and of unpermute and its gradient (declared
// in include/pgg.h).
//
// The execute call validates the descriptor on the host, lays out the
// workspace, and enqueues on the caller's stream:
//   1. index preparation (one workgroup for small M, three grid-wide passes
//      otherwise): group offsets, the m-tile table, inv/ori tables, checks;
//   2. for every column panel, and within it every chunk of m-tiles: the
//      MFMA producer, which writes the chunk's fp32 rows (the panel's
//      columns) into the ring, then the ordered consumer, which adds them
//      into those columns of d_x.
// One-chunk weight-streaming calls with aligned rows and few groups take two
// launches: the producer runs the preparation in a spare workgroup.  Stream
// order carries every dependency; there is no host synchronisation and no
// allocation on this path.
#include <stdio.h>
#include <string.h>

#include <vector>

#include "pgg_internal.h"

using namespace pgg;

namespace {

// ---------------------------------------------------------------------------
// timing hook
// ---------------------------------------------------------------------------
struct TimingSession {
  bool active = false;
  std::vector<hipEvent_t> start, stop;
  std::vector<const char*> names;
  int used = 0;
  bool overflow = false;
};

TimingSession g_timing;

struct TimedLaunch {
  const char* name;
  hipStream_t stream;
  int idx = -1;
  TimedLaunch(const char* n, hipStream_t s) : name(n), stream(s) {
    if (!g_timing.active) return;
    if (g_timing.used >= static_cast<int>(g_timing.start.size())) {
      g_timing.overflow = true;
      return;
    }
    idx = g_timing.used++;
    g_timing.names[idx] = name;
    (void)hipEventRecord(g_timing.start[idx], stream);
  }
  ~TimedLaunch() {
    if (idx >= 0) (void)hipEventRecord(g_timing.stop[idx], stream);
  }
};

bool is_aligned(const void* ptr, size_t a) { return reinterpret_cast<uintptr_t>(ptr) % a == 0; }

size_t elem_size(int32_t dtype) { return dtype == PGG_F32 ? 4 : 2; }

struct Call {
  Plan plan;
  WsView w;
  bool aligned;
};

// plan: a plan already made for desc (the allocation-free entry point's), or
// NULL to make the default one
pgg_status check_call(const pgg_moe_dx_desc* desc, const void* grad_y, const void* weight,
                      const int64_t* expanded_row_idx, const int64_t* group_list,
                      const float* grad_x, void* workspace, size_t workspace_bytes, Call* c,
                      const Plan* plan = nullptr) {
  Plan& p = c->plan;
  if (plan) {
    p = *plan;
  } else {
    const pgg_status st = make_plan(desc, &p);
    if (st != PGG_OK) return st;
  }
  if (!grad_y || !weight || !expanded_row_idx || !group_list || !grad_x || !workspace)
    return PGG_ERR_INVALID_ARG;
  if (workspace_bytes < p.total) return PGG_ERR_WORKSPACE_TOO_SMALL;
  if (!is_aligned(workspace, kWorkspaceAlign)) return PGG_ERR_MISALIGNED;
  if (!is_aligned(expanded_row_idx, 8) || !is_aligned(group_list, 8) || !is_aligned(grad_x, 4) ||
      !is_aligned(grad_y, elem_size(p.dtype)) || !is_aligned(weight, elem_size(p.dtype)))
    return PGG_ERR_MISALIGNED;

  const bool aligned = is_aligned(grad_y, 16) && is_aligned(weight, 16) &&
                       (size_t(p.N) * elem_size(p.dtype)) % 16 == 0;
  c->aligned = aligned;
  c->w = ws_view(p, workspace);
  return PGG_OK;
}

// Index preparation: group offsets, m-tile table, inv/ori, checks.
hipError_t enqueue_prep(const Plan& p, const int64_t* expanded_row_idx, const int64_t* group_list,
                        const WsView& w, hipStream_t stream) {
  hipError_t e = hipSuccess;
  if (p.fused_prep) {
    TimedLaunch t("prep_fused", stream);
    e = launch_prep_fused(p, expanded_row_idx, group_list, w, stream);
  } else {
    {
      TimedLaunch t("prep_groups", stream);
      e = launch_prep_groups(p, group_list, w, stream);
    }
    if (e == hipSuccess) {
      TimedLaunch t("prep_index", stream);
      e = launch_prep_index(p, expanded_row_idx, w, stream);
    }
    if (e == hipSuccess) {
      TimedLaunch t("prep_verify", stream);
      e = launch_prep_verify(p, expanded_row_idx, w, stream);
    }
  }
  return e;
}

pgg_status enqueue(const Call& c, const void* grad_y, const void* weight,
                   const int64_t* expanded_row_idx, const int64_t* group_list, float* grad_x,
                   hipStream_t stream) {
  const Plan& p = c.plan;
  const WsView& w = c.w;
  const bool aligned = c.aligned;
  hipError_t e = hipSuccess;
  if (sweep_can_prepare(p, aligned)) {
    // one chunk of few rows per expert: the producer launch prepares too
    {
      TimedLaunch t(produce_kernel_name(p), stream);
      e = launch_produce_sweep_prepared(p, grad_y, weight, expanded_row_idx, group_list, w, stream);
    }
    if (e == hipSuccess) {
      TimedLaunch t("consume", stream);
      e = launch_consume(p, 0, 0, w, grad_x, stream);
    }
    return e == hipSuccess ? PGG_OK : PGG_ERR_HIP;
  }
  e = enqueue_prep(p, expanded_row_idx, group_list, w, stream);
  const char* pname = produce_kernel_name(p);
  // column panels one after another; within a panel, chunks in row order
  for (int pn = 0; pn < p.n_panels && e == hipSuccess; ++pn) {
    for (int ch = 0; ch < p.max_chunks && e == hipSuccess; ++ch) {
      {
        TimedLaunch t(pname, stream);
        e = launch_produce(p, ch, pn, grad_y, weight, aligned, w, stream);
      }
      if (e != hipSuccess) break;
      TimedLaunch t("consume", stream);
      e = launch_consume(p, ch, pn, w, grad_x, stream);
    }
  }
  return e == hipSuccess ? PGG_OK : PGG_ERR_HIP;
}

pgg_status check_fwd(const pgg_moe_fwd_desc* desc, const void* x, const void* weight,
                     const int64_t* expanded_row_idx, const int64_t* group_list, const float* y,
                     void* workspace, size_t workspace_bytes, Call* c, bool dw = false) {
  Plan& p = c->plan;
  const pgg_status st = dw ? make_dw_plan(desc, &p) : make_fwd_plan(desc, &p);
  if (st != PGG_OK) return st;
  if (!x || !weight || !expanded_row_idx || !group_list || !y || !workspace)
    return PGG_ERR_INVALID_ARG;
  if (workspace_bytes < p.total) return PGG_ERR_WORKSPACE_TOO_SMALL;
  if (!is_aligned(workspace, kWorkspaceAlign)) return PGG_ERR_MISALIGNED;
  const size_t es = elem_size(p.dtype);
  if (!is_aligned(expanded_row_idx, 8) || !is_aligned(group_list, 8) || !is_aligned(y, 4) ||
      !is_aligned(x, es) || !is_aligned(weight, es))
    return PGG_ERR_MISALIGNED;
  // x rows hold the reduction (plan N), weight rows the output columns (plan K)
  c->aligned = is_aligned(x, 16) && is_aligned(weight, 16) && (size_t(p.N) * es) % 16 == 0 &&
               (size_t(p.K) * es) % 16 == 0;
  c->w = ws_view(p, workspace);
  return PGG_OK;
}

pgg_status enqueue_fwd(const Call& c, const void* x, const void* weight,
                       const int64_t* expanded_row_idx, const int64_t* group_list, float* y,
                       hipStream_t stream) {
  const Plan& p = c.plan;
  hipError_t e = enqueue_prep(p, expanded_row_idx, group_list, c.w, stream);
  if (e == hipSuccess) {
    TimedLaunch t(forward_kernel_name(p), stream);
    e = launch_forward(p, x, weight, y, c.aligned, c.w, stream);
  }
  if (e == hipSuccess && p.ksplit > 1) {
    TimedLaunch t("forward_reduce", stream);
    e = launch_forward_reduce(p, c.w, y, stream);
  }
  return e == hipSuccess ? PGG_OK : PGG_ERR_HIP;
}

// The weight gradient: same checks as the forward, with grad_y in the
// weight's place (its rows hold N elements, as the weight's rows do).
pgg_status check_dw(const pgg_moe_fwd_desc* desc, const void* x, const void* grad_y,
                    const int64_t* expanded_row_idx, const int64_t* group_list, const float* dw,
                    void* workspace, size_t workspace_bytes, Call* c) {
  return check_fwd(desc, x, grad_y, expanded_row_idx, group_list, dw, workspace, workspace_bytes, c,
                   true);
}

pgg_status enqueue_dw(const Call& c, const void* x, const void* grad_y,
                      const int64_t* expanded_row_idx, const int64_t* group_list, float* dw,
                      hipStream_t stream) {
  const Plan& p = c.plan;
  hipError_t e = enqueue_prep(p, expanded_row_idx, group_list, c.w, stream);
  if (e == hipSuccess) {
    TimedLaunch t(dw_kernel_name(p), stream);
    e = launch_dw(p, x, grad_y, dw, c.aligned, c.w, stream);
  }
  return e == hipSuccess ? PGG_OK : PGG_ERR_HIP;
}

void fill_plan(const Plan& p, pgg_plan* out) {
  out->regime = p.regime;
  out->block_m = p.bm;
  out->block_n = p.bn;
  out->tiles_per_chunk = p.tc;
  out->max_tiles = p.max_tiles;
  out->max_chunks = p.max_chunks;
  out->ring_rows = p.ring_rows;
  out->n_panels = p.n_panels;
  out->panel_cols = p.panel_cols;
  out->fused_prep = p.fused_prep ? 1 : 0;
  out->ring_bytes = p.ring_bytes;
  out->table_bytes = p.table_bytes;
  out->workspace_bytes = p.total;
}

}  // namespace

extern "C" {

pgg_status pgg_moe_dx_workspace_size(const pgg_moe_dx_desc* desc, size_t* bytes) {
  if (!bytes) return PGG_ERR_INVALID_ARG;
  Plan p;
  const pgg_status st = make_plan(desc, &p);
  if (st != PGG_OK) return st;
  *bytes = p.total;
  return PGG_OK;
}

pgg_status pgg_moe_dx_plan(const pgg_moe_dx_desc* desc, pgg_plan* out) {
  if (!out) return PGG_ERR_INVALID_ARG;
  Plan p;
  const pgg_status st = make_plan(desc, &p);
  if (st != PGG_OK) return st;
  fill_plan(p, out);
  return PGG_OK;
}

pgg_status pgg_moe_dx(const pgg_moe_dx_desc* desc, const void* grad_y, const void* weight,
                      const int64_t* expanded_row_idx, const int64_t* group_list, float* grad_x,
                      void* workspace, size_t workspace_bytes, hipStream_t stream) {
  Call c;
  const pgg_status st = check_call(desc, grad_y, weight, expanded_row_idx, group_list, grad_x,
                                   workspace, workspace_bytes, &c);
  if (st != PGG_OK) return st;
  return enqueue(c, grad_y, weight, expanded_row_idx, group_list, grad_x, stream);
}

pgg_status pgg_moe_dx_noalloc(const pgg_moe_dx_desc* desc, const void* grad_y, const void* weight,
                              const int64_t* expanded_row_idx, const int64_t* group_list,
                              float* grad_x, int64_t* device_error, hipStream_t stream) {
  Plan plan;
  pgg_status st = make_plan_within(desc, kNoAllocScratchBytes, &plan);
  if (st != PGG_OK) return st;
  if (device_error && !is_aligned(device_error, 8)) return PGG_ERR_MISALIGNED;
  void* scratch = nullptr;
  if (!grad_y || !weight || !expanded_row_idx || !group_list || !grad_x) return PGG_ERR_INVALID_ARG;
  if (noalloc_scratch(stream, &scratch) != hipSuccess) return PGG_ERR_HIP;
  Call c;
  st = check_call(desc, grad_y, weight, expanded_row_idx, group_list, grad_x, scratch,
                  kNoAllocScratchBytes, &c, &plan);
  if (st != PGG_OK) return st;
  st = enqueue(c, grad_y, weight, expanded_row_idx, group_list, grad_x, stream);
  if (st != PGG_OK || !device_error) return st;
  return launch_export_error(c.w.hdr, device_error, stream) == hipSuccess ? PGG_OK : PGG_ERR_HIP;
}

pgg_status pgg_moe_dx_kernel_time(const pgg_moe_dx_desc* desc, const void* grad_y,
                                  const void* weight, const int64_t* expanded_row_idx,
                                  const int64_t* group_list, float* grad_x, void* workspace,
                                  size_t workspace_bytes, hipStream_t stream, int32_t which,
                                  int32_t repeats, double* avg_ms, int32_t* launches_per_call) {
  if ((which != 0 && which != 1) || repeats <= 0 || !avg_ms) return PGG_ERR_INVALID_ARG;
  Call c;
  pgg_status st = check_call(desc, grad_y, weight, expanded_row_idx, group_list, grad_x, workspace,
                             workspace_bytes, &c);
  if (st != PGG_OK) return st;
  // one full call fills the workspace tables the kernels read
  st = enqueue(c, grad_y, weight, expanded_row_idx, group_list, grad_x, stream);
  if (st != PGG_OK) return st;
  const Plan& p = c.plan;
  const bool prepared = sweep_can_prepare(p, c.aligned);
  hipEvent_t ev[2] = {nullptr, nullptr};
  for (auto& e : ev)
    if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) st = PGG_ERR_HIP;
  hipError_t e = st == PGG_OK ? hipEventRecord(ev[0], stream) : hipErrorUnknown;
  for (int32_t r = 0; r < repeats && e == hipSuccess; ++r) {
    for (int pn = 0; pn < p.n_panels && e == hipSuccess; ++pn) {
      for (int ch = 0; ch < p.max_chunks && e == hipSuccess; ++ch) {
        if (which == 1)
          e = launch_consume(p, ch, pn, c.w, grad_x, stream);
        else if (prepared)
          e = launch_produce_sweep_prepared(p, grad_y, weight, expanded_row_idx, group_list, c.w,
                                            stream);
        else
          e = launch_produce(p, ch, pn, grad_y, weight, c.aligned, c.w, stream);
      }
    }
  }
  if (e == hipSuccess) e = hipEventRecord(ev[1], stream);
  if (e == hipSuccess) e = hipEventSynchronize(ev[1]);
  float ms = 0.0f;
  if (e == hipSuccess) e = hipEventElapsedTime(&ms, ev[0], ev[1]);
  for (auto& x : ev)
    if (x) (void)hipEventDestroy(x);
  if (st != PGG_OK) return st;
  if (e != hipSuccess) return PGG_ERR_HIP;
  // Repeated consumers read a ring that holds only the last chunk and add
  // into d_x again: one more full call restores the results.
  if (which == 1) {
    st = enqueue(c, grad_y, weight, expanded_row_idx, group_list, grad_x, stream);
    if (st != PGG_OK) return st;
  }
  const int32_t launches = p.max_chunks * p.n_panels;
  *avg_ms = double(ms) / (double(repeats) * double(launches));
  if (launches_per_call) *launches_per_call = launches;
  return PGG_OK;
}

pgg_status pgg_moe_fwd_workspace_size(const pgg_moe_fwd_desc* desc, size_t* bytes) {
  if (!bytes) return PGG_ERR_INVALID_ARG;
  Plan p;
  const pgg_status st = make_fwd_plan(desc, &p);
  if (st != PGG_OK) return st;
  *bytes = p.total;
  return PGG_OK;
}

pgg_status pgg_moe_fwd_plan(const pgg_moe_fwd_desc* desc, pgg_plan* out) {
  if (!out) return PGG_ERR_INVALID_ARG;
  Plan p;
  const pgg_status st = make_fwd_plan(desc, &p);
  if (st != PGG_OK) return st;
  fill_plan(p, out);
  return PGG_OK;
}

pgg_status pgg_moe_fwd(const pgg_moe_fwd_desc* desc, const void* x, const void* weight,
                       const int64_t* expanded_row_idx, const int64_t* group_list, float* y,
                       void* workspace, size_t workspace_bytes, hipStream_t stream) {
  Call c;
  const pgg_status st = check_fwd(desc, x, weight, expanded_row_idx, group_list, y, workspace,
                                  workspace_bytes, &c);
  if (st != PGG_OK) return st;
  return enqueue_fwd(c, x, weight, expanded_row_idx, group_list, y, stream);
}

pgg_status pgg_moe_fwd_kernel_time(const pgg_moe_fwd_desc* desc, const void* x, const void* weight,
                                   const int64_t* expanded_row_idx, const int64_t* group_list,
                                   float* y, void* workspace, size_t workspace_bytes,
                                   hipStream_t stream, int32_t repeats, double* avg_ms) {
  if (repeats <= 0 || !avg_ms) return PGG_ERR_INVALID_ARG;
  Call c;
  pgg_status st = check_fwd(desc, x, weight, expanded_row_idx, group_list, y, workspace,
                            workspace_bytes, &c);
  if (st != PGG_OK) return st;
  st = enqueue_fwd(c, x, weight, expanded_row_idx, group_list, y, stream);
  if (st != PGG_OK) return st;
  hipEvent_t ev[2] = {nullptr, nullptr};
  for (auto& e : ev)
    if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) st = PGG_ERR_HIP;
  hipError_t e = st == PGG_OK ? hipEventRecord(ev[0], stream) : hipErrorUnknown;
  for (int32_t r = 0; r < repeats && e == hipSuccess; ++r)
    e = launch_forward(c.plan, x, weight, y, c.aligned, c.w, stream);
  if (e == hipSuccess) e = hipEventRecord(ev[1], stream);
  if (e == hipSuccess) e = hipEventSynchronize(ev[1]);
  float ms = 0.0f;
  if (e == hipSuccess) e = hipEventElapsedTime(&ms, ev[0], ev[1]);
  for (auto& x_ev : ev)
    if (x_ev) (void)hipEventDestroy(x_ev);
  if (st != PGG_OK) return st;
  if (e != hipSuccess) return PGG_ERR_HIP;
  *avg_ms = double(ms) / double(repeats);
  return PGG_OK;
}

pgg_status pgg_moe_dw_workspace_size(const pgg_moe_fwd_desc* desc, size_t* bytes) {
  if (!bytes) return PGG_ERR_INVALID_ARG;
  Plan p;
  const pgg_status st = make_dw_plan(desc, &p);
  if (st != PGG_OK) return st;
  *bytes = p.total;
  return PGG_OK;
}

pgg_status pgg_moe_dw(const pgg_moe_fwd_desc* desc, const void* x, const void* grad_y,
                      const int64_t* expanded_row_idx, const int64_t* group_list, float* grad_w,
                      void* workspace, size_t workspace_bytes, hipStream_t stream) {
  Call c;
  const pgg_status st = check_dw(desc, x, grad_y, expanded_row_idx, group_list, grad_w, workspace,
                                 workspace_bytes, &c);
  if (st != PGG_OK) return st;
  return enqueue_dw(c, x, grad_y, expanded_row_idx, group_list, grad_w, stream);
}

pgg_status pgg_moe_dw_kernel_time(const pgg_moe_fwd_desc* desc, const void* x, const void* grad_y,
                                  const int64_t* expanded_row_idx, const int64_t* group_list,
                                  float* grad_w, void* workspace, size_t workspace_bytes,
                                  hipStream_t stream, int32_t repeats, double* avg_ms) {
  if (repeats <= 0 || !avg_ms) return PGG_ERR_INVALID_ARG;
  Call c;
  pgg_status st = check_dw(desc, x, grad_y, expanded_row_idx, group_list, grad_w, workspace,
                           workspace_bytes, &c);
  if (st != PGG_OK) return st;
  st = enqueue_dw(c, x, grad_y, expanded_row_idx, group_list, grad_w, stream);
  if (st != PGG_OK) return st;
  hipEvent_t ev[2] = {nullptr, nullptr};
  for (auto& e : ev)
    if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) st = PGG_ERR_HIP;
  hipError_t e = st == PGG_OK ? hipEventRecord(ev[0], stream) : hipErrorUnknown;
  for (int32_t r = 0; r < repeats && e == hipSuccess; ++r)
    e = launch_dw(c.plan, x, grad_y, grad_w, c.aligned, c.w, stream);
  if (e == hipSuccess) e = hipEventRecord(ev[1], stream);
  if (e == hipSuccess) e = hipEventSynchronize(ev[1]);
  float ms = 0.0f;
  if (e == hipSuccess) e = hipEventElapsedTime(&ms, ev[0], ev[1]);
  for (auto& x_ev : ev)
    if (x_ev) (void)hipEventDestroy(x_ev);
  if (st != PGG_OK) return st;
  if (e != hipSuccess) return PGG_ERR_HIP;
  *avg_ms = double(ms) / double(repeats);
  return PGG_OK;
}

pgg_status pgg_moe_routing_workspace_size(const pgg_moe_routing_desc* desc, size_t* bytes) {
  if (!bytes) return PGG_ERR_INVALID_ARG;
  RoutePlan p;
  const pgg_status st = make_routing_plan(desc, &p);
  if (st != PGG_OK) return st;
  *bytes = p.total;
  return PGG_OK;
}

pgg_status pgg_moe_routing(const pgg_moe_routing_desc* desc, const int64_t* expert_ids,
                           const void* x, int64_t* group_list, int64_t* eri_gather,
                           int64_t* eri_scatter, void* expanded_x, void* workspace,
                           size_t workspace_bytes, hipStream_t stream) {
  RoutePlan p;
  const pgg_status st = make_routing_plan(desc, &p);
  if (st != PGG_OK) return st;
  if (!expert_ids || !group_list || !workspace) return PGG_ERR_INVALID_ARG;
  if (expanded_x && (p.K == 0 || !x)) return PGG_ERR_INVALID_ARG;
  if (workspace_bytes < p.total) return PGG_ERR_WORKSPACE_TOO_SMALL;
  if (!is_aligned(workspace, kWorkspaceAlign) || !is_aligned(expert_ids, 8) ||
      !is_aligned(group_list, 8) || (eri_gather && !is_aligned(eri_gather, 8)) ||
      (eri_scatter && !is_aligned(eri_scatter, 8)))
    return PGG_ERR_MISALIGNED;
  const size_t es = elem_size(p.dtype);
  if (expanded_x && (!is_aligned(x, es) || !is_aligned(expanded_x, es))) return PGG_ERR_MISALIGNED;
  const bool vec = expanded_x && is_aligned(x, 16) && is_aligned(expanded_x, 16) &&
                   (size_t(p.K) * es) % 16 == 0;
  hipError_t e;
  {
    TimedLaunch t("routing", stream);
    e = launch_routing(p, expert_ids, x, group_list, eri_gather, eri_scatter, expanded_x, workspace,
                       vec, stream);
  }
  return e == hipSuccess ? PGG_OK : PGG_ERR_HIP;
}

pgg_status pgg_moe_unpermute_workspace_size(const pgg_moe_unpermute_desc* desc, size_t* bytes) {
  if (!bytes) return PGG_ERR_INVALID_ARG;
  UnpermutePlan p;
  const pgg_status st = make_unpermute_plan(desc, &p);
  if (st != PGG_OK) return st;
  *bytes = p.total;
  return PGG_OK;
}

static pgg_status check_unpermute(const pgg_moe_unpermute_desc* desc, const void* const* values,
                                  int n_values, const int64_t* eri, void* workspace,
                                  size_t workspace_bytes, UnpermutePlan* p) {
  const pgg_status st = make_unpermute_plan(desc, p);
  if (st != PGG_OK) return st;
  if (!eri || !workspace) return PGG_ERR_INVALID_ARG;
  if (workspace_bytes < p->total) return PGG_ERR_WORKSPACE_TOO_SMALL;
  if (!is_aligned(workspace, kWorkspaceAlign) || !is_aligned(eri, 8)) return PGG_ERR_MISALIGNED;
  for (int i = 0; i < n_values; ++i) {
    if (!values[i]) return PGG_ERR_INVALID_ARG;
    if (!is_aligned(values[i], elem_size(p->dtype))) return PGG_ERR_MISALIGNED;
  }
  return PGG_OK;
}

pgg_status pgg_moe_unpermute(const pgg_moe_unpermute_desc* desc, const void* permuted,
                             const int64_t* expanded_row_idx, const void* probs, void* out,
                             void* workspace, size_t workspace_bytes, hipStream_t stream) {
  UnpermutePlan p;
  const void* vals[3] = {permuted, out, probs};
  const pgg_status st = check_unpermute(desc, vals, probs ? 3 : 2, expanded_row_idx, workspace,
                                        workspace_bytes, &p);
  if (st != PGG_OK) return st;
  hipError_t e;
  {
    TimedLaunch t("unpermute", stream);
    e = launch_unpermute(p, workspace, expanded_row_idx, permuted, nullptr, probs, out, nullptr, false,
                         stream);
  }
  return e == hipSuccess ? PGG_OK : PGG_ERR_HIP;
}

pgg_status pgg_moe_unpermute_grad(const pgg_moe_unpermute_desc* desc, const void* permuted,
                                  const void* grad, const int64_t* expanded_row_idx,
                                  const void* probs, void* perm_grad, void* probs_grad,
                                  void* workspace, size_t workspace_bytes, hipStream_t stream) {
  UnpermutePlan p;
  const void* with[5] = {grad, perm_grad, probs, permuted, probs_grad};
  const pgg_status st = check_unpermute(desc, with, probs ? 5 : 2, expanded_row_idx, workspace,
                                        workspace_bytes, &p);
  if (st != PGG_OK) return st;
  hipError_t e;
  {
    TimedLaunch t("unpermute_grad", stream);
    e = launch_unpermute(p, workspace, expanded_row_idx, permuted, grad, probs, perm_grad, probs_grad,
                         true, stream);
  }
  return e == hipSuccess ? PGG_OK : PGG_ERR_HIP;
}

pgg_status pgg_moe_dx_read_device_error(const void* workspace, hipStream_t stream, int32_t* code,
                                        int64_t* detail) {
  if (!workspace || !code) return PGG_ERR_INVALID_ARG;
  WsHeader h;
  if (hipMemcpyAsync(&h, workspace, sizeof(h), hipMemcpyDeviceToHost, stream) != hipSuccess)
    return PGG_ERR_HIP;
  if (hipStreamSynchronize(stream) != hipSuccess) return PGG_ERR_HIP;
  if (h.err == kNoError) {
    *code = PGG_DEV_OK;
    if (detail) *detail = 0;
  } else {
    *code = static_cast<int32_t>(h.err >> kErrShift);
    if (detail) *detail = static_cast<int64_t>(h.err & kDetailMask);
  }
  return PGG_OK;
}

pgg_status pgg_moe_dx_debug_tables(const pgg_moe_dx_desc* desc, const void* workspace,
                                   hipStream_t stream, int32_t* inv_host, int32_t* ori_host) {
  Plan p;
  const pgg_status st = make_plan(desc, &p);
  if (st != PGG_OK) return st;
  if (!workspace) return PGG_ERR_INVALID_ARG;
  const WsView w = ws_view(p, const_cast<void*>(workspace));
  const size_t bytes = sizeof(int32_t) * size_t(p.M);
  if (inv_host && hipMemcpyAsync(inv_host, w.inv, bytes, hipMemcpyDeviceToHost, stream) != hipSuccess)
    return PGG_ERR_HIP;
  if (ori_host && hipMemcpyAsync(ori_host, w.ori, bytes, hipMemcpyDeviceToHost, stream) != hipSuccess)
    return PGG_ERR_HIP;
  return hipStreamSynchronize(stream) == hipSuccess ? PGG_OK : PGG_ERR_HIP;
}

pgg_status pgg_moe_dx_debug_tiles(const pgg_moe_dx_desc* desc, const void* workspace,
                                  hipStream_t stream, int32_t* tiles_host, int32_t max_tiles,
                                  int32_t* n_tiles) {
  Plan p;
  const pgg_status st = make_plan(desc, &p);
  if (st != PGG_OK) return st;
  if (!workspace || !n_tiles || (max_tiles > 0 && !tiles_host)) return PGG_ERR_INVALID_ARG;
  const WsView w = ws_view(p, const_cast<void*>(workspace));
  WsHeader h;
  if (hipMemcpyAsync(&h, w.hdr, sizeof(h), hipMemcpyDeviceToHost, stream) != hipSuccess)
    return PGG_ERR_HIP;
  if (hipStreamSynchronize(stream) != hipSuccess) return PGG_ERR_HIP;
  *n_tiles = h.n_tiles;
  const int32_t n = h.n_tiles < max_tiles ? h.n_tiles : max_tiles;
  if (n > 0) {
    std::vector<MTile> t(static_cast<size_t>(n));
    if (hipMemcpyAsync(t.data(), w.tiles, sizeof(MTile) * t.size(), hipMemcpyDeviceToHost, stream) !=
        hipSuccess)
      return PGG_ERR_HIP;
    if (hipStreamSynchronize(stream) != hipSuccess) return PGG_ERR_HIP;
    for (int32_t i = 0; i < n; ++i) {
      tiles_host[3 * i + 0] = t[i].g;
      tiles_host[3 * i + 1] = t[i].row0;
      tiles_host[3 * i + 2] = t[i].rows;
    }
  }
  return PGG_OK;
}

pgg_status pgg_timing_begin(int32_t capacity) {
  if (capacity <= 0 || g_timing.active) return PGG_ERR_INVALID_ARG;
  g_timing.start.assign(static_cast<size_t>(capacity), nullptr);
  g_timing.stop.assign(static_cast<size_t>(capacity), nullptr);
  g_timing.names.assign(static_cast<size_t>(capacity), nullptr);
  // timing-only events: no system-scope fence on record (it would write back
  // and invalidate the caches between the kernels being timed)
  for (int32_t i = 0; i < capacity; ++i) {
    if (hipEventCreateWithFlags(&g_timing.start[i], hipEventDisableSystemFence) != hipSuccess ||
        hipEventCreateWithFlags(&g_timing.stop[i], hipEventDisableSystemFence) != hipSuccess)
      return PGG_ERR_HIP;
  }
  g_timing.used = 0;
  g_timing.overflow = false;
  g_timing.active = true;
  return PGG_OK;
}

pgg_status pgg_timing_end(pgg_kernel_time* out, int32_t max_out, int32_t* n_out) {
  if (!g_timing.active) return PGG_ERR_INVALID_ARG;
  g_timing.active = false;
  std::vector<pgg_kernel_time> acc;
  pgg_status st = PGG_OK;
  for (int i = 0; i < g_timing.used; ++i) {
    if (hipEventSynchronize(g_timing.stop[i]) != hipSuccess) { st = PGG_ERR_HIP; break; }
    float ms = 0.0f;
    if (hipEventElapsedTime(&ms, g_timing.start[i], g_timing.stop[i]) != hipSuccess) {
      st = PGG_ERR_HIP;
      break;
    }
    size_t k = 0;
    for (; k < acc.size(); ++k)
      if (strncmp(acc[k].name, g_timing.names[i], sizeof(acc[k].name)) == 0) break;
    if (k == acc.size()) {
      pgg_kernel_time t{};
      snprintf(t.name, sizeof(t.name), "%s", g_timing.names[i]);
      acc.push_back(t);
    }
    acc[k].launches += 1;
    acc[k].total_ms += ms;
  }
  for (size_t i = 0; i < g_timing.start.size(); ++i) {
    if (g_timing.start[i]) (void)hipEventDestroy(g_timing.start[i]);
    if (g_timing.stop[i]) (void)hipEventDestroy(g_timing.stop[i]);
  }
  g_timing.start.clear();
  g_timing.stop.clear();
  g_timing.names.clear();
  const int32_t n = static_cast<int32_t>(acc.size());
  if (n_out) *n_out = n;
  for (int32_t i = 0; i < n && i < max_out && out; ++i) out[i] = acc[static_cast<size_t>(i)];
  if (st == PGG_OK && g_timing.overflow) st = PGG_ERR_INVALID_ARG;
  return st;
}

const char* pgg_status_string(pgg_status s) {
  switch (s) {
    case PGG_OK: return "ok";
    case PGG_ERR_INVALID_ARG: return "invalid argument";
    case PGG_ERR_UNSUPPORTED: return "unsupported problem size";
    case PGG_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case PGG_ERR_HIP: return "HIP runtime error";
    case PGG_ERR_MISALIGNED: return "misaligned pointer";
  }
  return "unknown status";
}

const char* pgg_device_error_string(int32_t code) {
  switch (code) {
    case PGG_DEV_OK: return "ok";
    case PGG_DEV_GROUP_NEGATIVE: return "group_list has a negative count";
    case PGG_DEV_GROUP_SUM: return "sum(group_list) != M";
    case PGG_DEV_INDEX_RANGE: return "expanded_row_idx value outside [0, M)";
    case PGG_DEV_INDEX_DUP: return "expanded_row_idx is not a permutation";
    case PGG_DEV_EXPERT_RANGE: return "expert id outside [0, experts)";
  }
  return "unknown device error";
}

}  // extern "C"
