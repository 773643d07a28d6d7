// Index preparation on the device: group prefix sums and the m-tile table
// from group_list, and normalisation of expanded_row_idx into both
// directions of the routing permutation.  Nothing here needs a host sync:
// the tile count is data dependent, so the table is padded to the host-side
// bound and later stages skip unused slots.
//
// Semantics (MoeInitRoutingGroupedMatmulGrad design page):
//  * group_list holds per-expert counts, not a cumulative sum (§1.2 I/O
//    table); the page keeps per-expert prefix tables of counts, work ids and
//    m-block ids for its vector cores (§2.5.3) — here they become `offsets`
//    and the flat m-tile list.  Empty experts get no tile, so their weights
//    are never read (§1.2 constraints: empty groups are skipped).
//  * row_idx_type 0: eri[i] is the original position of expanded row i;
//    row_idx_type 1: eri[p] is the expanded row of original position p
//    (§1.2 I/O notes; the page inverts the scatter form on its vector cores,
//    §2.4.4 / §2.5.1).  Both are turned into inv (position -> row) and ori
//    (row -> position); the token of row i is ori[i] / topK (§数学定义和公式,
//    Step 2).
//  * Data-dependent violations (negative count, sum != M, index out of range,
//    index not a permutation) are recorded in the workspace error word.
#pragma once

#include "pgg_internal.h"

namespace pgg {

namespace {

constexpr int kPrepThreads = 1024;

__device__ __forceinline__ void set_error(WsHeader* h, int code, long long detail) {
  if (detail < 0) detail = 0;
  unsigned long long key = (static_cast<unsigned long long>(code) << kErrShift) |
                           (static_cast<unsigned long long>(detail) & kDetailMask);
  atomicMin(&h->err, key);
}

struct PrepArgs {
  int64_t M, G, topk;
  int32_t bm, tc, max_tiles, max_chunks;
  int32_t row_idx_type;
};

// Block-wide: header reset (thread 0; caller syncs before errors may be set).
__device__ void reset_header(WsHeader* h) {
  if (threadIdx.x == 0) {
    h->err = kNoError;
    h->n_tiles = 0;
  }
}

// One workgroup: offsets, tile table, chunk table.  s_rows and s_tiles are
// LDS scratch of blockDim.x entries each.
__device__ void groups_phase(const PrepArgs& a, const int64_t* __restrict__ gl, const WsView& w,
                             long long* s_rows, long long* s_tiles) {
  const int tid = threadIdx.x;
  const int nt = blockDim.x;
  const int64_t seg = (a.G + nt - 1) / nt;
  const int64_t g0 = min<int64_t>(a.G, tid * seg);
  const int64_t g1 = min<int64_t>(a.G, g0 + seg);

  // Each thread's scanned tile count is its own count capped at 2^32 (a valid
  // total is below 2^31, so the cap never binds then) plus kNegFlag if it saw
  // a negative count: the scanned total then also says whether any count was
  // negative (at most 1024 threads: capped parts stay below 2^42, flags below
  // 2^62).
  constexpr long long kTileCap = 1ll << 32;
  constexpr long long kNegFlag = 1ll << 52;
  long long rows = 0, tiles = 0;
  bool neg = false;
  for (int64_t g = g0; g < g1; ++g) {
    long long c = gl[g];
    if (c < 0) {
      set_error(w.hdr, PGG_DEV_GROUP_NEGATIVE, g);
      neg = true;
      continue;
    }
    if (c > a.M) c = a.M + 1;  // keeps the sums far from overflow; the total check fails anyway
    rows += c;
    tiles = min(kTileCap, tiles + (c + a.bm - 1) / a.bm);
  }
  const long long mine = tiles + (neg ? kNegFlag : 0);
  s_rows[tid] = rows;
  s_tiles[tid] = mine;
  __syncthreads();
  for (int d = 1; d < nt; d <<= 1) {   // inclusive Hillis-Steele scan
    long long r = 0, t = 0;
    if (tid >= d) { r = s_rows[tid - d]; t = s_tiles[tid - d]; }
    __syncthreads();
    s_rows[tid] += r;
    s_tiles[tid] += t;
    __syncthreads();
  }
  const long long total_rows = s_rows[nt - 1];
  const long long total_tiles = s_tiles[nt - 1];
  const bool any_neg = total_tiles >= kNegFlag;
  const bool valid = !any_neg && total_rows == a.M && total_tiles <= a.max_tiles;
  if (!any_neg && total_rows != a.M && tid == 0)
    set_error(w.hdr, PGG_DEV_GROUP_SUM, total_rows);
  const int32_t n_tiles = valid ? static_cast<int32_t>(total_tiles) : 0;

  long long r = s_rows[tid] - rows;
  long long t = s_tiles[tid] - mine;
  for (int64_t g = g0; g < g1; ++g) {
    long long c = gl[g];
    if (c < 0) c = 0;
    if (c > a.M) c = a.M + 1;
    w.offsets[g] = r;
    if (valid) {
      const long long mt = (c + a.bm - 1) / a.bm;
      for (long long q = 0; q < mt; ++q) {
        MTile e;
        e.g = static_cast<int32_t>(g);
        e.row0 = static_cast<int32_t>(r + q * a.bm);
        e.rows = static_cast<int32_t>(min<long long>(a.bm, c - q * a.bm));
        e.pad = 0;
        w.tiles[t + q] = e;
      }
    }
    r += c;
    t += (c + a.bm - 1) / a.bm;
  }
  if (tid == 0) {
    w.offsets[a.G] = total_rows;
    w.hdr->n_tiles = n_tiles;
  }
  for (int s = n_tiles + tid; s < a.max_tiles; s += nt) {
    MTile e = {0, 0, 0, 0};
    w.tiles[s] = e;
  }
  __syncthreads();
  for (int c = tid; c <= a.max_chunks; c += nt) {
    const int64_t first = static_cast<int64_t>(c) * a.tc;
    w.chunk_row0[c] = first < n_tiles ? w.tiles[first].row0 : static_cast<int32_t>(a.M);
  }
}

__device__ __forceinline__ void index_one(const PrepArgs& a, const int64_t* __restrict__ eri,
                                          const WsView& w, int64_t t) {
  const int64_t v = eri[t];
  if (v < 0 || v >= a.M) {
    set_error(w.hdr, PGG_DEV_INDEX_RANGE, t);
    return;
  }
  if (a.row_idx_type == 0) {   // t: expanded row, v: original position
    w.ori[t] = static_cast<int32_t>(v);
    w.inv[v] = static_cast<int32_t>(t);
  } else {                     // t: original position, v: expanded row
    w.inv[t] = static_cast<int32_t>(v);
    w.ori[v] = static_cast<int32_t>(t);
  }
}

// After index_one has run for every t: a repeated value leaves one writer
// in the inverse slot, so the other fails this round trip.
__device__ __forceinline__ void verify_one(const PrepArgs& a, const int64_t* __restrict__ eri,
                                           const WsView& w, int64_t t) {
  const int64_t v = eri[t];
  if (v < 0 || v >= a.M) return;
  const int32_t back = a.row_idx_type == 0 ? w.inv[v] : w.ori[v];
  if (back != t) set_error(w.hdr, PGG_DEV_INDEX_DUP, v);
}

// The whole preparation in one workgroup (any block size; LDS scratch of
// 2 * blockDim.x entries).
__device__ void prep_block(const PrepArgs& a, const int64_t* __restrict__ eri,
                           const int64_t* __restrict__ gl, const WsView& w, long long* scratch) {
  reset_header(w.hdr);
  __syncthreads();
  groups_phase(a, gl, w, scratch, scratch + blockDim.x);
  for (int64_t t = threadIdx.x; t < a.M; t += blockDim.x) index_one(a, eri, w, t);
  __syncthreads();
  for (int64_t t = threadIdx.x; t < a.M; t += blockDim.x) verify_one(a, eri, w, t);
}

inline PrepArgs prep_args(const Plan& p) {
  PrepArgs a;
  a.M = p.M;
  a.G = p.G;
  a.topk = p.topk;
  a.bm = p.bm;
  a.tc = p.tc;
  a.max_tiles = p.max_tiles;
  a.max_chunks = p.max_chunks;
  a.row_idx_type = p.row_idx_type;
  return a;
}

}  // namespace

}  // namespace pgg
