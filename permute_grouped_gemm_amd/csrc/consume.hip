// Consumer: the routing scatter-add of the fused op,
//
//   d_x[b, k] = sum of C[i, k] over the expanded rows i of token b
//
// (MoeInitRoutingGroupedMatmulGrad design page, §数学定义和公式 Step 2; the
// output is fp32 and the additions are fp32, §2.6.2), applied to the ring
// rows of one chunk.
//
// Order, with no atomics: chunks run one after another on the stream, and
// within a chunk every token that has rows in it is handled by exactly one
// workgroup (the one launched for its smallest row in the chunk), which adds
// that token's rows of the chunk in ascending topK slot j — the order the
// TileLang token-permute-grad kernel uses for its fp32 gather-reduce — onto
// either +0 (the token's first chunk) or the d_x row left by earlier chunks.
// So each element's additions happen in an order fixed by the inputs and the
// tile schedule alone, and repeated calls are bit-identical.  When the whole
// problem is one chunk the order is exactly j = 0..topK-1, and the consumer is
// indexed by token directly.
#include "pgg_internal.h"

namespace pgg {

namespace {

constexpr int kConsumeThreads = 256;

struct ConsumeArgs {
  const WsHeader* hdr;
  const int32_t* chunk_row0;
  const int32_t* inv;
  const int32_t* ori;
  const float* ring;
  float* dx;
  int64_t M, K, topk;
  int32_t chunk;
  int32_t col_blocks;
};

template <int VEC>
__global__ __launch_bounds__(kConsumeThreads) void consume_kernel(ConsumeArgs a) {
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

  const int64_t k = (static_cast<int64_t>(cb) * kConsumeThreads + threadIdx.x) * VEC;
  if (k >= a.K) return;
  float* __restrict__ out = a.dx + b * a.K + k;
  float acc[VEC];
  if (fresh) {
#pragma unroll
    for (int v = 0; v < VEC; ++v) acc[v] = 0.0f;
  } else if constexpr (VEC == 4) {
    const float4 o = *reinterpret_cast<const float4*>(out);
    acc[0] = o.x; acc[1] = o.y; acc[2] = o.z; acc[3] = o.w;
  } else {
#pragma unroll
    for (int v = 0; v < VEC; ++v) acc[v] = out[v];
  }
  for (int64_t j = 0; j < a.topk; ++j) {
    const int64_t ij = slots[j];
    if (ij < r0 || ij >= r1) continue;
    const float* __restrict__ src = a.ring + (ij - r0) * a.K + k;
    if constexpr (VEC == 4) {
      const float4 s = *reinterpret_cast<const float4*>(src);
      acc[0] += s.x; acc[1] += s.y; acc[2] += s.z; acc[3] += s.w;
    } else {
#pragma unroll
      for (int v = 0; v < VEC; ++v) acc[v] += src[v];
    }
  }
  if constexpr (VEC == 4) {
    *reinterpret_cast<float4*>(out) = make_float4(acc[0], acc[1], acc[2], acc[3]);
  } else {
#pragma unroll
    for (int v = 0; v < VEC; ++v) out[v] = acc[v];
  }
}

// The whole problem is one chunk: every token's rows are all in the ring, so
// token b simply adds its topK rows in slot order onto +0.  One one-wave
// workgroup per (token, column block), so a small batch still spreads over
// many compute units.  Slots are taken kBatch at a time: their row indices
// and then their rows are all requested before the first addition, so a
// token costs two memory latencies per batch instead of two per slot; the
// additions still run in slot order.  The error word is read beside the row
// indices and decides only whether d_x is written: every ring read is bounds
// checked, so nothing read under a bad index leaves the ring.
constexpr int kBatch = 8;
constexpr int kTokenThreads = 64;

template <int VEC>
__global__ __launch_bounds__(kTokenThreads) void consume_tokens_kernel(ConsumeArgs a) {
  typedef float vec_t __attribute__((ext_vector_type(VEC)));
  const uint64_t err = a.hdr->err;
  const int64_t b = blockIdx.x / a.col_blocks;
  const int cb = static_cast<int>(blockIdx.x - b * a.col_blocks);
  const int64_t k = (static_cast<int64_t>(cb) * kTokenThreads + threadIdx.x) * VEC;
  if (k >= a.K) return;
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
      v[q] = ok ? *reinterpret_cast<const vec_t*>(a.ring + row[q] * a.K + k) : vec_t(0.0f);
    }
#pragma unroll
    for (int q = 0; q < kBatch; ++q)
      if (row[q] >= 0 && row[q] < a.M) acc += v[q];
  }
  if (err != kNoError) return;
  *reinterpret_cast<vec_t*>(a.dx + b * a.K + k) = acc;
}

}  // namespace

hipError_t launch_consume(const Plan& p, int chunk, const WsView& w, float* grad_x, hipStream_t s) {
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
  const bool vec4 = (p.K % 4 == 0) && (reinterpret_cast<uintptr_t>(grad_x) % 16 == 0);
  const int vec = vec4 ? 4 : 1;
  a.col_blocks = static_cast<int32_t>((p.K + int64_t(kConsumeThreads) * vec - 1) /
                                      (int64_t(kConsumeThreads) * vec));
  if (p.max_chunks == 1) {
    // one chunk holds every row: consume by token (chunk_row0[0] == 0 then)
    a.col_blocks = static_cast<int32_t>((p.K + int64_t(kTokenThreads) * vec - 1) /
                                        (int64_t(kTokenThreads) * vec));
    const dim3 grid(static_cast<unsigned>(p.batch * a.col_blocks));
    if (vec4)
      hipLaunchKernelGGL(consume_tokens_kernel<4>, grid, dim3(kTokenThreads), 0, s, a);
    else
      hipLaunchKernelGGL(consume_tokens_kernel<1>, grid, dim3(kTokenThreads), 0, s, a);
    return hipGetLastError();
  }
  const dim3 grid(static_cast<unsigned>(int64_t(p.ring_rows) * a.col_blocks));
  if (vec4)
    hipLaunchKernelGGL(consume_kernel<4>, grid, dim3(kConsumeThreads), 0, s, a);
  else
    hipLaunchKernelGGL(consume_kernel<1>, grid, dim3(kConsumeThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace pgg
