// MoeInitRouting on the device (MoeInitRoutingGroupedMatmulGrad design page,
// §1.1 step 1: tokens are grouped by expert, semantically a permute; positions
// p = b * topK + j as in §数学定义和公式).  From the router's choices
// expert_ids [batch, topK] it builds:
//   group_list[g]  rows of expert g (counts);
//   eri_gather[i]  original position of expanded row i (row_idx_type 0);
//   eri_scatter[p] expanded row of position p (row_idx_type 1);
//   expanded_x[i]  = x[eri_gather[i] / topK] (optional).
// Expanded rows are grouped by expert in expert order and keep ascending p
// inside an expert, so the tables are unique and reproducible.
//
// Four launches: per-block histograms (LDS integer counters; the counts do
// not depend on the order the adds land in), one workgroup turning them into
// per-block bases and expert offsets, a placement pass in which one wave per
// block walks its positions in order (a lane's rank among the earlier lanes
// of the same expert comes from comparing lane by lane, and the last lane of
// each expert advances that expert's running count; it also keeps the
// expanded row of every position in the workspace), and the optional row
// gather, by token: each token's row is read once and stored to its topK
// expanded rows.  An id outside [0, G) sets the workspace error word (the smallest
// offending position wins) and leaves the outputs unspecified.
#include "pgg_device.h"

namespace pgg {

namespace {

constexpr int kBlockPos = 1024;     // positions per block
constexpr int kCountThreads = 256;
constexpr int kScanThreads = 1024;
constexpr int64_t kNoBad = INT64_MAX;
constexpr int kMaxExperts = 8192;   // the planner's limit; per-expert LDS arrays are static

__global__ __launch_bounds__(kCountThreads) void route_count_kernel(const int64_t* ids, int64_t M,
                                                                    int32_t G, int32_t* table,
                                                                    int64_t* bad) {
  __shared__ int32_t hist[kMaxExperts];
  __shared__ unsigned long long s_bad;
  for (int g = threadIdx.x; g < G; g += blockDim.x) hist[g] = 0;
  if (threadIdx.x == 0) s_bad = static_cast<unsigned long long>(kNoBad);
  __syncthreads();
  const int64_t p0 = static_cast<int64_t>(blockIdx.x) * kBlockPos;
  for (int t = threadIdx.x; t < kBlockPos; t += blockDim.x) {
    const int64_t p = p0 + t;
    if (p >= M) break;
    const int64_t e = ids[p];
    if (e >= 0 && e < G)
      atomicAdd(&hist[e], 1);
    else
      atomicMin(&s_bad, static_cast<unsigned long long>(p));
  }
  __syncthreads();
  for (int g = threadIdx.x; g < G; g += blockDim.x)
    table[static_cast<int64_t>(blockIdx.x) * G + g] = hist[g];
  if (threadIdx.x == 0) bad[blockIdx.x] = static_cast<int64_t>(s_bad);
}

// One workgroup: header reset, per-block exclusive bases (in place), counts,
// expert offsets, and the range error.
__global__ __launch_bounds__(kScanThreads) void route_scan_kernel(WsHeader* hdr, int32_t* table,
                                                                  const int64_t* bad, int32_t nblocks,
                                                                  int32_t G, int64_t* offsets,
                                                                  int64_t* group_list) {
  __shared__ long long s_part[kScanThreads];
  __shared__ long long s_bad[kScanThreads];
  const int tid = threadIdx.x;
  if (tid == 0) {
    hdr->err = kNoError;
    hdr->n_tiles = 0;
  }
  // per expert: exclusive prefix over blocks; thread t owns a contiguous run of experts
  const int per = (G + kScanThreads - 1) / kScanThreads;
  const int g0 = min(G, tid * per), g1 = min(G, g0 + per);
  long long mine = 0;
  for (int g = g0; g < g1; ++g) {
    int64_t run = 0;
    int32_t b = 0;
    // eight blocks at a time: the loads are independent, so they overlap
    for (; b + 8 <= nblocks; b += 8) {
      int32_t v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = table[static_cast<int64_t>(b + u) * G + g];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        table[static_cast<int64_t>(b + u) * G + g] = static_cast<int32_t>(run);
        run += v[u];
      }
    }
    for (; b < nblocks; ++b) {
      int32_t* c = &table[static_cast<int64_t>(b) * G + g];
      const int32_t v = *c;
      *c = static_cast<int32_t>(run);
      run += v;
    }
    group_list[g] = run;
    mine += run;
  }
  long long mbad = kNoBad;
  for (int32_t b = tid; b < nblocks; b += kScanThreads) mbad = bad[b] < mbad ? bad[b] : mbad;
  s_part[tid] = mine;
  s_bad[tid] = mbad;
  __syncthreads();
  // exclusive scan of the threads' expert totals (threads own ascending experts)
  for (int d = 1; d < kScanThreads; d <<= 1) {
    const long long v = tid >= d ? s_part[tid - d] : 0;
    const long long w = tid + d < kScanThreads ? s_bad[tid + d] : kNoBad;
    __syncthreads();
    s_part[tid] += v;
    s_bad[tid] = w < s_bad[tid] ? w : s_bad[tid];
    __syncthreads();
  }
  int64_t base = s_part[tid] - mine;
  for (int g = g0; g < g1; ++g) {
    offsets[g] = base;
    base += group_list[g];
  }
  if (tid == kScanThreads - 1) offsets[G] = s_part[tid];
  // the word was reset above by this thread: a plain store of (code << 48) | detail
  if (tid == 0 && s_bad[0] != kNoBad)
    hdr->err = (static_cast<unsigned long long>(PGG_DEV_EXPERT_RANGE) << kErrShift) |
               (static_cast<unsigned long long>(s_bad[0]) & kDetailMask);
}

// One wave per block: positions in order, 64 at a time.
__global__ __launch_bounds__(64) void route_place_kernel(const WsHeader* hdr, const int64_t* ids,
                                                         int64_t M, int32_t G, const int32_t* table,
                                                         const int64_t* offsets, int32_t* row_of,
                                                         int64_t* eri_gather, int64_t* eri_scatter) {
  __shared__ int32_t run[kMaxExperts];
  if (hdr->err != kNoError) return;
  const int lane = threadIdx.x;
  for (int g = lane; g < G; g += 64)
    run[g] = static_cast<int32_t>(offsets[g]) + table[static_cast<int64_t>(blockIdx.x) * G + g];
  __syncthreads();
  const int64_t p0 = static_cast<int64_t>(blockIdx.x) * kBlockPos;
  // chunks of 64 positions up to the last one that holds a position (uniform bound)
  const int n_chunks = static_cast<int>(min<int64_t>(kBlockPos / 64, (M - p0 + 63) / 64));
  for (int c = 0; c < n_chunks; ++c) {
    const int64_t p = p0 + c * 64 + lane;
    const int32_t e = p < M ? static_cast<int32_t>(ids[p]) : -1;
    int rank = 0, cnt = 0;
    for (int j = 0; j < 64; ++j) {
      const int32_t ej = __builtin_amdgcn_readlane(e, j);
      if (ej == e) {
        cnt += 1;
        if (j < lane) rank += 1;
      }
    }
    int32_t row = 0;
    if (e >= 0) {
      row = run[e] + rank;
      row_of[p] = row;
      if (eri_gather) eri_gather[row] = p;
      if (eri_scatter) eri_scatter[p] = row;
    }
    __syncthreads();                       // every lane has read run[] for this chunk
    if (e >= 0 && rank == cnt - 1) run[e] += cnt;
    __syncthreads();
  }
}

// expanded_x[row_of[b * topK + j]] = x[b] for every slot j: workgroup
// (b, y) reads piece y of token b's row once, kGatherLoads 16-byte chunks per
// thread at a time (rows 16-byte aligned; bytes otherwise), and stores them to
// the token's topK expanded rows.  Large batches take 16 KiB pieces (one per
// row at the usual widths: reading a token's row once is what saves the
// traffic); small ones 4 KiB pieces, so a few tokens still spread over many
// compute units.  The loads are unconditional, on an in-bounds piece (the
// thread's first of the group stands in past the row end), so that none waits
// inside a branch of its own; only the stores are guarded.
constexpr int kGatherLoads = 4;
constexpr int64_t kGatherGroup = 256 * 16 * kGatherLoads;   // bytes the workgroup loads at a time
constexpr int64_t kGatherBigBatch = 2048;

__global__ __launch_bounds__(256) void route_gather_kernel(const WsHeader* hdr, const int32_t* row_of,
                                                           int64_t topk, const char* x, char* ex,
                                                           int64_t row_bytes, int64_t piece,
                                                           int32_t vec) {
  if (hdr->err != kNoError) return;
  const int64_t b = blockIdx.x;
  const char* src = x + b * row_bytes;
  const int32_t* rows = row_of + b * topk;
  const int64_t p0 = static_cast<int64_t>(blockIdx.y) * piece;
  const int64_t p1 = row_bytes < p0 + piece ? row_bytes : p0 + piece;
  if (vec) {
    for (int64_t b0 = p0 + threadIdx.x * 16; b0 < p1; b0 += kGatherGroup) {
      u32x4_t v[kGatherLoads];
#pragma unroll
      for (int u = 0; u < kGatherLoads; ++u) {
        const int64_t bb = b0 + u * 256 * 16;
        v[u] = *reinterpret_cast<const u32x4_t*>(src + (bb < p1 ? bb : b0));
      }
      for (int64_t j = 0; j < topk; ++j) {
        char* dst = ex + static_cast<int64_t>(rows[j]) * row_bytes;
#pragma unroll
        for (int u = 0; u < kGatherLoads; ++u) {
          const int64_t bb = b0 + u * 256 * 16;
          if (bb < p1) *reinterpret_cast<u32x4_t*>(dst + bb) = v[u];
        }
      }
    }
  } else {
    for (int64_t c = p0 + threadIdx.x; c < p1; c += 256) {
      const char v = src[c];
      for (int64_t j = 0; j < topk; ++j) ex[static_cast<int64_t>(rows[j]) * row_bytes + c] = v;
    }
  }
}

}  // namespace

hipError_t launch_routing(const RoutePlan& p, const int64_t* ids, const void* x, int64_t* group_list,
                          int64_t* eri_gather, int64_t* eri_scatter, void* expanded_x, void* ws,
                          bool vec, hipStream_t s) {
  char* b = static_cast<char*>(ws);
  WsHeader* hdr = reinterpret_cast<WsHeader*>(b + p.off_header);
  int32_t* table = reinterpret_cast<int32_t*>(b + p.off_table);
  int64_t* bad = reinterpret_cast<int64_t*>(b + p.off_bad);
  int64_t* offsets = reinterpret_cast<int64_t*>(b + p.off_offsets);
  int32_t* row_of = reinterpret_cast<int32_t*>(b + p.off_rows);
  hipLaunchKernelGGL(route_count_kernel, dim3(p.nblocks), dim3(kCountThreads), 0, s, ids,
                     p.M, static_cast<int32_t>(p.G), table, bad);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(route_scan_kernel, dim3(1), dim3(kScanThreads), 0, s, hdr, table, bad,
                     p.nblocks, static_cast<int32_t>(p.G), offsets, group_list);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(route_place_kernel, dim3(p.nblocks), dim3(64), 0, s, hdr, ids, p.M,
                     static_cast<int32_t>(p.G), table, offsets, row_of, eri_gather, eri_scatter);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (expanded_x && p.K > 0) {
    const int64_t row_bytes = p.K * (p.dtype == PGG_F32 ? 4 : 2);
    const int64_t batch = p.M / p.topk;
    const int64_t piece = batch >= kGatherBigBatch ? kGatherGroup : kGatherGroup / 4;
    const dim3 grid(static_cast<unsigned>(batch), static_cast<unsigned>((row_bytes + piece - 1) / piece));
    hipLaunchKernelGGL(route_gather_kernel, grid, dim3(256), 0, s, hdr, row_of, p.topk,
                       static_cast<const char*>(x), static_cast<char*>(expanded_x), row_bytes, piece,
                       vec ? 1 : 0);
    e = hipGetLastError();
  }
  return e;
}

}  // namespace pgg
