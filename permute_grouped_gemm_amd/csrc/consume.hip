// Consumer: the routing scatter-add of the fused op,
//
//   d_x[b, k] = sum of C[i, k] over the expanded rows i of token b
//
// (MoeInitRoutingGroupedMatmulGrad design page, §数学定义和公式 Step 2; the
// output is fp32 and the additions are fp32, §2.6.2), applied to the ring
// rows of one chunk and the columns of one panel.
//
// Order, with no atomics: chunks run one after another on the stream, and
// within a chunk every token with rows there is handled by exactly one
// workgroup per column block, which adds the token's rows that lie in the
// chunk in ascending topK slot j — the order the TileLang token-permute-grad
// kernel uses for its fp32 gather-reduce — onto either +0 (the token's first
// chunk) or the d_x value left by earlier chunks.  So each element's
// additions happen in an order fixed by the inputs and the tile schedule
// alone, and repeated calls are bit-identical.  When the whole problem is
// one chunk the order is exactly j = 0..topK-1.
//
// Three kernels: by token for one chunk per panel (consume_tokens_kernel) and
// for a few (consume_chunk_kernel), by ring row for many
// (consume_rows_kernel).  The token-indexed ones take slots kBatch at a
// time: their row indices, and then their ring rows and the token's earlier
// d_x value, are all requested before the first addition, so a token costs
// two memory latencies per batch instead of two per slot.
#include "pgg_internal.h"

namespace pgg {

namespace {

constexpr int kBatch = 8;

struct ConsumeArgs {
  const WsHeader* hdr;
  const int32_t* chunk_row0;
  const int32_t* inv;
  const int32_t* ori;
  const float* ring;        // [ring_rows, ldc]: columns [k_lo, k_hi) of the panel
  float* dx;
  int64_t M, K, topk;
  int64_t k_lo, k_hi, ldc;
  int32_t chunk;
  int32_t col_blocks;       // column blocks of the panel
};

// A few chunks: one workgroup of kChunkThreads per (token, block of
// kChunkThreads * VEC columns); most tokens have several rows in each chunk.
// Ring rows and the earlier d_x value are read with range-checked buffer
// loads: a slot outside the chunk, or the d_x value of a token's first chunk,
// gets an offset past the buffer's end, which the hardware answers with zeros
// without touching memory, so every load is issued unconditionally and the
// additions keep their order.  Tokens with no row in the chunk leave at once.
constexpr uint32_t kOutside = 0x80000000u;   // byte offset past every buffer here

// AUX: the load's cache policy (2: non-temporal, for ring rows, each read
// once).
template <int VEC, int AUX = 0>
__device__ __forceinline__ void buffer_load(__amdgpu_buffer_rsrc_t r, uint32_t off, float (&v)[VEC]) {
  if constexpr (VEC == 4) {
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 x = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, AUX));
    const unsigned x0 = x[0], x1 = x[1], x2 = x[2], x3 = x[3];   // scalar copies (no element bit-casts)
    v[0] = __builtin_bit_cast(float, x0);
    v[1] = __builtin_bit_cast(float, x1);
    v[2] = __builtin_bit_cast(float, x2);
    v[3] = __builtin_bit_cast(float, x3);
  } else {
    v[0] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, AUX));
  }
}

// One wave (256 columns with 16-byte accesses): panels are whole tiles of
// 256 (or 128) columns wide, so no block is left mostly idle (1024-column
// blocks left a 256-wide remainder block of a 1280-wide panel).
constexpr int kChunkThreads = 64;

template <int VEC>
__global__ __launch_bounds__(kChunkThreads) void consume_chunk_kernel(ConsumeArgs a) {
  if (a.hdr->err != kNoError) return;
  const int64_t r0 = a.chunk_row0[a.chunk];
  const int64_t r1 = a.chunk_row0[a.chunk + 1];
  const int64_t b = blockIdx.x / a.col_blocks;
  const int cb = static_cast<int>(blockIdx.x - b * a.col_blocks);
  const int32_t* __restrict__ slots = a.inv + b * a.topk;
  bool fresh = true, any = false;
  for (int64_t j = 0; j < a.topk; ++j) {
    const int64_t ij = slots[j];
    fresh = fresh && ij >= r0;
    any = any || (ij >= r0 && ij < r1);
  }
  if (!any) return;
  const int64_t kk = (static_cast<int64_t>(cb) * kChunkThreads + threadIdx.x) * VEC;   // panel column
  if (a.k_lo + kk >= a.k_hi) return;
  // ring rows of the chunk (at most 256 MiB) and this token's d_x row
  const int32_t ring_bytes = static_cast<int32_t>((r1 - r0) * a.ldc * 4);
  const __amdgpu_buffer_rsrc_t ring = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(a.ring), 0, ring_bytes, 0x00020000);
  float* __restrict__ out = a.dx + b * a.K + a.k_lo;
  const __amdgpu_buffer_rsrc_t dxr = __builtin_amdgcn_make_buffer_rsrc(
      out, 0, static_cast<int32_t>((a.k_hi - a.k_lo) * 4), 0x00020000);
  float acc[VEC];
  buffer_load<VEC>(dxr, fresh ? kOutside : static_cast<uint32_t>(kk * 4), acc);
  for (int64_t j0 = 0; j0 < a.topk; j0 += kBatch) {
    bool in[kBatch];
    float v[kBatch][VEC];
#pragma unroll
    for (int q = 0; q < kBatch; ++q) {
      const int64_t ij = j0 + q < a.topk ? slots[j0 + q] : -1;
      in[q] = ij >= r0 && ij < r1;
      const uint32_t off = in[q] ? static_cast<uint32_t>(((ij - r0) * a.ldc + kk) * 4) : kOutside;
      buffer_load<VEC, 2>(ring, off, v[q]);
    }
#pragma unroll
    for (int q = 0; q < kBatch; ++q)
      if (in[q]) {
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc[e] += v[q][e];
      }
  }
  if constexpr (VEC == 4) {
    *reinterpret_cast<float4*>(out + kk) = make_float4(acc[0], acc[1], acc[2], acc[3]);
  } else {
    out[kk] = acc[0];
  }
}

// Many chunks: one workgroup of kRowThreads per (ring row, block of
// kRowThreads * VEC columns).  Every token with rows in the chunk is handled
// by the workgroups of its smallest row there, the others leave at once.
// With many chunks most tokens have one row in a chunk, and this form moves
// the d_x read-modify-write traffic faster than the token-indexed one.
constexpr int kRowThreads = 256;

template <int VEC>
__global__ __launch_bounds__(kRowThreads) void consume_rows_kernel(ConsumeArgs a) {
  if (a.hdr->err != kNoError) return;
  const int64_t r0 = a.chunk_row0[a.chunk];
  const int64_t r1 = a.chunk_row0[a.chunk + 1];
  const int64_t local = blockIdx.x / a.col_blocks;
  const int cb = static_cast<int>(blockIdx.x - local * a.col_blocks);
  const int64_t i = r0 + local;
  if (i >= r1) return;
  const int32_t p = a.ori[i];
  if (p < 0 || p >= a.M) return;
  const int64_t b = p / a.topk;
  const int32_t* __restrict__ slots = a.inv + b * a.topk;

  bool fresh = true;
  for (int64_t j = 0; j < a.topk; ++j) {
    const int64_t ij = slots[j];
    if (ij < r0) fresh = false;
    else if (ij < i) return;   // a smaller row of this token in the chunk owns it
  }

  const int64_t kk = (static_cast<int64_t>(cb) * kRowThreads + threadIdx.x) * VEC;   // panel column
  if (a.k_lo + kk >= a.k_hi) return;
  float* __restrict__ out = a.dx + b * a.K + a.k_lo + kk;
  float acc[VEC];
  if (fresh) {
#pragma unroll
    for (int v = 0; v < VEC; ++v) acc[v] = 0.0f;
  } else if constexpr (VEC == 4) {
    const float4 o = *reinterpret_cast<const float4*>(out);
    acc[0] = o.x; acc[1] = o.y; acc[2] = o.z; acc[3] = o.w;
  } else {
    acc[0] = out[0];
  }
  for (int64_t j = 0; j < a.topk; ++j) {
    const int64_t ij = slots[j];
    if (ij < r0 || ij >= r1) continue;
    const float* __restrict__ src = a.ring + (ij - r0) * a.ldc + kk;
    if constexpr (VEC == 4) {
      const float4 v = *reinterpret_cast<const float4*>(src);
      acc[0] += v.x; acc[1] += v.y; acc[2] += v.z; acc[3] += v.w;
    } else {
      acc[0] += src[0];
    }
  }
  if constexpr (VEC == 4) {
    *reinterpret_cast<float4*>(out) = make_float4(acc[0], acc[1], acc[2], acc[3]);
  } else {
    out[0] = acc[0];
  }
}

// The whole problem is one chunk: every token's rows are all in the ring, so
// token b simply adds its topK rows in slot order onto +0.  One one-wave
// workgroup per (token, column block), so a small batch still spreads over
// many compute units.  The error word is read beside the row indices and
// decides only whether d_x is written: every ring read is bounds checked, so
// nothing read under a bad index leaves the ring.
constexpr int kTokenThreads = 64;

template <int VEC>
__global__ __launch_bounds__(kTokenThreads) void consume_tokens_kernel(ConsumeArgs a) {
  typedef float vec_t __attribute__((ext_vector_type(VEC)));
  const uint64_t err = a.hdr->err;
  const int64_t b = blockIdx.x / a.col_blocks;
  const int cb = static_cast<int>(blockIdx.x - b * a.col_blocks);
  const int64_t k = a.k_lo + (static_cast<int64_t>(cb) * kTokenThreads + threadIdx.x) * VEC;
  if (k >= a.k_hi) return;
  const int32_t* __restrict__ slots = a.inv + b * a.topk;
  vec_t acc = vec_t(0.0f);
  for (int64_t j0 = 0; j0 < a.topk; j0 += kBatch) {
    int64_t row[kBatch];
#pragma unroll
    for (int q = 0; q < kBatch; ++q) row[q] = j0 + q < a.topk ? slots[j0 + q] : -1;
    vec_t v[kBatch];
#pragma unroll
    for (int q = 0; q < kBatch; ++q) {
      const bool ok = row[q] >= 0 && row[q] < a.M;
      // each ring row is read once: non-temporal
      v[q] = ok ? __builtin_nontemporal_load(
                      reinterpret_cast<const vec_t*>(a.ring + row[q] * a.ldc + (k - a.k_lo)))
                : vec_t(0.0f);
    }
#pragma unroll
    for (int q = 0; q < kBatch; ++q)
      if (row[q] >= 0 && row[q] < a.M) acc += v[q];
  }
  if (err != kNoError) return;
  *reinterpret_cast<vec_t*>(a.dx + b * a.K + k) = acc;
}

}  // namespace

hipError_t launch_consume(const Plan& p, int chunk, int panel, const WsView& w, float* grad_x,
                          hipStream_t s) {
  ConsumeArgs a;
  a.hdr = w.hdr;
  a.chunk_row0 = w.chunk_row0;
  a.inv = w.inv;
  a.ori = w.ori;
  a.ring = w.ring;
  a.dx = grad_x;
  a.M = p.M;
  a.K = p.K;
  a.topk = p.topk;
  a.chunk = chunk;
  panel_range(p, panel, &a.k_lo, &a.k_hi);
  a.ldc = p.panel_cols;
  const int64_t width = a.k_hi - a.k_lo;
  // 16-byte accesses need K, the panel's first column and the ring row
  // length to be multiples of 4 floats
  const bool vec4 = (p.K % 4 == 0) && (a.k_lo % 4 == 0) && (a.ldc % 4 == 0) &&
                    (reinterpret_cast<uintptr_t>(grad_x) % 16 == 0);
  const int vec = vec4 ? 4 : 1;
  if (p.max_chunks == 1) {
    // one chunk holds every row: chunk_row0[0] == 0 then
    a.col_blocks = static_cast<int32_t>((width + int64_t(kTokenThreads) * vec - 1) /
                                        (int64_t(kTokenThreads) * vec));
    const dim3 grid(static_cast<unsigned>(p.batch * a.col_blocks));
    if (vec4)
      hipLaunchKernelGGL(consume_tokens_kernel<4>, grid, dim3(kTokenThreads), 0, s, a);
    else
      hipLaunchKernelGGL(consume_tokens_kernel<1>, grid, dim3(kTokenThreads), 0, s, a);
    return hipGetLastError();
  }
  if (p.max_chunks > kFewChunks) {
    a.col_blocks = static_cast<int32_t>((width + int64_t(kRowThreads) * vec - 1) /
                                        (int64_t(kRowThreads) * vec));
    const dim3 grid(static_cast<unsigned>(int64_t(p.ring_rows) * a.col_blocks));
    if (vec4)
      hipLaunchKernelGGL(consume_rows_kernel<4>, grid, dim3(kRowThreads), 0, s, a);
    else
      hipLaunchKernelGGL(consume_rows_kernel<1>, grid, dim3(kRowThreads), 0, s, a);
    return hipGetLastError();
  }
  a.col_blocks = static_cast<int32_t>((width + int64_t(kChunkThreads) * vec - 1) /
                                      (int64_t(kChunkThreads) * vec));
  const dim3 grid(static_cast<unsigned>(p.batch * a.col_blocks));
  if (vec4)
    hipLaunchKernelGGL(consume_chunk_kernel<4>, grid, dim3(kChunkThreads), 0, s, a);
  else
    hipLaunchKernelGGL(consume_chunk_kernel<1>, grid, dim3(kChunkThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace pgg
