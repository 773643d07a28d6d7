// Unpermute and its gradient (TileLang-Ascend operator page, sections 4 and 5:
// MoeTokenUnpermute, MoeTokenUnpermuteGrad), on the routing tables of the
// other operators:
//
//   with probabilities:  out[t]            = sum_j probs[t, j] * permuted[row(t, j)]      [batch, H]
//                        perm_grad[row(t,j)] = grad[t] * probs[t, j]                      [M, H]
//                        probs_grad[t, j]  = sum_h grad[t, h] * permuted[row(t, j), h]   [batch, topK]
//   without:             out[p] = permuted[row(p)],  perm_grad[row(p)] = grad[p]           [M, H]
//
// row(t, j) is the expanded row of original position t*topK + j.  Values are
// widened to fp32, multiplied and summed in fp32 (slot order for out; a fixed
// tree over h for probs_grad) and rounded once to the tensors' type, so every
// result is independent of timing.  The routing index is inverted and checked
// first by the shared index-preparation kernels.
#include <algorithm>

#include "pgg_device.h"

namespace pgg {

namespace {

template <class T> __device__ __forceinline__ float ld(const void* p, int64_t i);
template <> __device__ __forceinline__ float ld<TF32>(const void* p, int64_t i) {
  return static_cast<const float*>(p)[i];
}
template <> __device__ __forceinline__ float ld<TF16>(const void* p, int64_t i) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<const uint16_t*>(p)[i]));
}
template <> __device__ __forceinline__ float ld<TBf16>(const void* p, int64_t i) {
  return __builtin_bit_cast(float, static_cast<uint32_t>(static_cast<const uint16_t*>(p)[i]) << 16);
}

template <class T> __device__ __forceinline__ void st(void* p, int64_t i, float v);
template <> __device__ __forceinline__ void st<TF32>(void* p, int64_t i, float v) {
  static_cast<float*>(p)[i] = v;
}
template <> __device__ __forceinline__ void st<TF16>(void* p, int64_t i, float v) {
  static_cast<uint16_t*>(p)[i] = __builtin_bit_cast(uint16_t, static_cast<_Float16>(v));   // RNE
}
template <> __device__ __forceinline__ void st<TBf16>(void* p, int64_t i, float v) {
  const uint32_t u = __builtin_bit_cast(uint32_t, v);
  uint16_t r;
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu))
    r = 0x7FC0;                                               // NaN stays NaN
  else
    r = static_cast<uint16_t>((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);   // round to nearest even
  static_cast<uint16_t*>(p)[i] = r;
}

// 16-byte chunks: 16 / sizeof(elem) values widened to fp32 / rounded back.
template <class T> struct Chunk { static constexpr int N = 16 / int(sizeof(typename T::elem)); };

template <class T>
__device__ __forceinline__ void widen(const u32x4_t& raw, float (&v)[Chunk<T>::N]) {
  if constexpr (Chunk<T>::N == 4) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t w = raw[k];   // a scalar copy: bit-casting the vector element lvalue read element 0
      v[k] = __builtin_bit_cast(float, w);
    }
  } else {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint16_t lo = static_cast<uint16_t>(raw[k] & 0xFFFFu), hi = static_cast<uint16_t>(raw[k] >> 16);
      v[2 * k] = ld<T>(&lo, 0);
      v[2 * k + 1] = ld<T>(&hi, 0);
    }
  }
}

// Loads that must all be in flight together are issued raw and
// unconditionally (on an in-bounds address) and only their use is guarded, so
// that no load waits inside a branch of its own.  Every row is read and
// written once: the 16-byte loads and stores are non-temporal.
template <class T>
__device__ __forceinline__ u32x4_t ldraw(const void* base, int64_t i) {
  return __builtin_nontemporal_load(
      reinterpret_cast<const u32x4_t*>(static_cast<const typename T::elem*>(base) + i));
}

template <class T>
__device__ __forceinline__ void ldv(const void* base, int64_t i, float (&v)[Chunk<T>::N]) {
  widen<T>(ldraw<T>(base, i), v);
}

template <class T>
__device__ __forceinline__ void stv(void* base, int64_t i, const float (&v)[Chunk<T>::N]) {
  u32x4_t raw;
  if constexpr (Chunk<T>::N == 4) {
#pragma unroll
    for (int k = 0; k < 4; ++k) raw[k] = __builtin_bit_cast(uint32_t, v[k]);
  } else {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      uint16_t lo, hi;
      st<T>(&lo, 0, v[2 * k]);
      st<T>(&hi, 0, v[2 * k + 1]);
      raw[k] = static_cast<uint32_t>(lo) | (static_cast<uint32_t>(hi) << 16);
    }
  }
  __builtin_nontemporal_store(raw, reinterpret_cast<u32x4_t*>(static_cast<typename T::elem*>(base) + i));
}

__global__ void unpermute_reset_kernel(WsHeader* hdr) {
  hdr->err = kNoError;
  hdr->n_tiles = 0;
}

constexpr int kThreads = 256;
constexpr int kPerThread = 4;
constexpr int kCols = kThreads * kPerThread;    // columns per workgroup

// out[t, h] = sum_j probs[t, j] * permuted[inv[t*topK + j], h]; grid (batch, column blocks)
template <class T>
__global__ __launch_bounds__(kThreads) void unpermute_kernel(const WsHeader* hdr, const int32_t* inv,
                                                             const void* permuted, const void* probs,
                                                             void* out, int64_t H, int64_t topk) {
  if (hdr->err != kNoError) return;
  const int64_t t = blockIdx.x;
  const int64_t h0 = static_cast<int64_t>(blockIdx.y) * kCols + threadIdx.x;
  float acc[kPerThread];
#pragma unroll
  for (int k = 0; k < kPerThread; ++k) acc[k] = 0.0f;
  for (int64_t j = 0; j < topk; ++j) {
    const int64_t r = inv[t * topk + j];
    const float pj = ld<T>(probs, t * topk + j);
#pragma unroll
    for (int k = 0; k < kPerThread; ++k) {
      const int64_t h = h0 + k * kThreads;
      if (h < H) acc[k] += pj * ld<T>(permuted, r * H + h);
    }
  }
#pragma unroll
  for (int k = 0; k < kPerThread; ++k) {
    const int64_t h = h0 + k * kThreads;
    if (h < H) st<T>(out, t * H + h, acc[k]);
  }
}

// The same with 16-byte chunks (rows 16-byte aligned): thread = one chunk of
// the token's row; grid (batch, chunk blocks of kThreads).  Slots are taken
// kSlotLoads at a time: all their chunks are requested before the first
// addition, which still runs in slot order.
constexpr int kSlotLoads = 8;

template <class T>
__global__ __launch_bounds__(kThreads) void unpermute_vec_kernel(const WsHeader* hdr,
                                                                 const int32_t* inv,
                                                                 const void* permuted,
                                                                 const void* probs, void* out,
                                                                 int64_t H, int64_t topk) {
  constexpr int N = Chunk<T>::N;
  if (hdr->err != kNoError) return;
  const int64_t t = blockIdx.x;
  const int64_t h = (static_cast<int64_t>(blockIdx.y) * kThreads + threadIdx.x) * N;
  if (h >= H) return;
  float acc[N];
#pragma unroll
  for (int k = 0; k < N; ++k) acc[k] = 0.0f;
  for (int64_t j0 = 0; j0 < topk; j0 += kSlotLoads) {
    const int nq = static_cast<int>(topk - j0 < kSlotLoads ? topk - j0 : kSlotLoads);
    u32x4_t raw[kSlotLoads];
    float pj[kSlotLoads];
#pragma unroll
    for (int q = 0; q < kSlotLoads; ++q) {
      const int64_t j = j0 + (q < nq ? q : 0);   // past the last slot: slot j0 again, unused
      pj[q] = ld<T>(probs, t * topk + j);
      raw[q] = ldraw<T>(permuted, static_cast<int64_t>(inv[t * topk + j]) * H + h);
    }
#pragma unroll
    for (int q = 0; q < kSlotLoads; ++q)
      if (q < nq) {
        float v[N];
        widen<T>(raw[q], v);
#pragma unroll
        for (int k = 0; k < N; ++k) acc[k] += pj[q] * v[k];
      }
  }
  stv<T>(out, t * H + h, acc);
}

// Row copies: dst[drow(p)] = src[srow(p)] for every position p; grid (M, column blocks).
// gather: drow = p, srow = inv[p]; scatter: drow = inv[p], srow = p.
__global__ __launch_bounds__(kThreads) void permute_rows_kernel(const WsHeader* hdr,
                                                                const int32_t* inv,
                                                                const uint16_t* src, uint16_t* dst,
                                                                int64_t row_halves, int32_t scatter) {
  if (hdr->err != kNoError) return;
  const int64_t p = blockIdx.x;
  const int64_t r = inv[p];
  const uint16_t* s = src + (scatter ? p : r) * row_halves;
  uint16_t* d = dst + (scatter ? r : p) * row_halves;
  for (int64_t b = static_cast<int64_t>(blockIdx.y) * kThreads + threadIdx.x; b < row_halves;
       b += static_cast<int64_t>(gridDim.y) * kThreads)
    d[b] = s[b];
}

// One workgroup per token: for every slot j, perm_grad[row] = grad[t] * p and
// probs_grad[t, j] = sum_h grad[t, h] * permuted[row, h] (per-thread sums over
// a fixed set of h, a fixed butterfly within each wave, then the waves in order).
template <class T>
__global__ __launch_bounds__(kThreads) void unpermute_grad_kernel(
    const WsHeader* hdr, const int32_t* inv, const void* permuted, const void* grad,
    const void* probs, void* perm_grad, void* probs_grad, int64_t H, int64_t topk) {
  __shared__ float s_wave[kThreads / 64];
  if (hdr->err != kNoError) return;
  const int64_t t = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int64_t j = 0; j < topk; ++j) {
    const int64_t r = inv[t * topk + j];
    const float pj = ld<T>(probs, t * topk + j);
    float part = 0.0f;
    for (int64_t h = threadIdx.x; h < H; h += kThreads) {
      const float g = ld<T>(grad, t * H + h);
      st<T>(perm_grad, r * H + h, g * pj);
      part += g * ld<T>(permuted, r * H + h);
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) part += __shfl_xor(part, m);
    if (lane == 0) s_wave[wave] = part;
    __syncthreads();
    if (threadIdx.x == 0) {
      float sum = s_wave[0];
#pragma unroll
      for (int w = 1; w < kThreads / 64; ++w) sum += s_wave[w];
      st<T>(probs_grad, t * topk + j, sum);
    }
    __syncthreads();
  }
}

// The gradient with 16-byte chunks for rows too long for the register kernel
// (rows 16-byte aligned).
template <class T>
__global__ __launch_bounds__(kThreads) void unpermute_grad_vec_kernel(
    const WsHeader* hdr, const int32_t* inv, const void* permuted, const void* grad,
    const void* probs, void* perm_grad, void* probs_grad, int64_t H, int64_t topk) {
  constexpr int N = Chunk<T>::N;
  __shared__ float s_wave[kThreads / 64];
  if (hdr->err != kNoError) return;
  const int64_t t = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int64_t j = 0; j < topk; ++j) {
    const int64_t r = inv[t * topk + j];
    const float pj = ld<T>(probs, t * topk + j);
    float part = 0.0f;
    for (int64_t h = static_cast<int64_t>(threadIdx.x) * N; h < H; h += kThreads * N) {
      float g[N], x[N], o[N];
      ldv<T>(grad, t * H + h, g);
      ldv<T>(permuted, r * H + h, x);
#pragma unroll
      for (int k = 0; k < N; ++k) {
        o[k] = g[k] * pj;
        part += g[k] * x[k];
      }
      stv<T>(perm_grad, r * H + h, o);
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) part += __shfl_xor(part, m);
    if (lane == 0) s_wave[wave] = part;
    __syncthreads();
    if (threadIdx.x == 0) {
      float sum = s_wave[0];
#pragma unroll
      for (int w = 1; w < kThreads / 64; ++w) sum += s_wave[w];
      st<T>(probs_grad, t * topk + j, sum);
    }
    __syncthreads();
  }
}

// The gradient with the token's grad row held in registers (rows 16-byte
// aligned, H <= kGradChunks * kThreads chunks): grad[t] is read once, not once
// per slot.  Each slot's per-thread sum and butterfly run as in the kernel
// above (same order, so the same bits); the slots' rows and probabilities,
// kSlotBatch at a time, are staged in LDS, and the waves' sums of those slots
// wait in LDS for one barrier and are then added in wave order.
constexpr int kGradChunks = 4;
constexpr int kSlotBatch = 16;

template <class T>
__global__ __launch_bounds__(kThreads) void unpermute_grad_reg_kernel(
    const WsHeader* hdr, const int32_t* inv, const void* permuted, const void* grad,
    const void* probs, void* perm_grad, void* probs_grad, int64_t H, int64_t topk) {
  constexpr int N = Chunk<T>::N;
  __shared__ float s_part[kSlotBatch][kThreads / 64];
  __shared__ int32_t s_row[kSlotBatch];
  __shared__ float s_prob[kSlotBatch];
  if (hdr->err != kNoError) return;
  const int64_t t = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // this thread's chunks: h = (threadIdx.x + c * kThreads) * N; a chunk past
  // the row loads chunk 0 instead and is not used
  int64_t hc[kGradChunks];
  bool has[kGradChunks];
  u32x4_t g[kGradChunks];
#pragma unroll
  for (int c = 0; c < kGradChunks; ++c) {
    const int64_t h = static_cast<int64_t>(threadIdx.x + c * kThreads) * N;
    has[c] = h < H;
    hc[c] = has[c] ? h : 0;
    g[c] = ldraw<T>(grad, t * H + hc[c]);
  }
  for (int64_t j0 = 0; j0 < topk; j0 += kSlotBatch) {
    const int nj = static_cast<int>(topk - j0 < kSlotBatch ? topk - j0 : kSlotBatch);
    // the previous batch's readers of s_row, s_prob and s_part are past the
    // barrier below it
    if (static_cast<int>(threadIdx.x) < nj) {
      s_row[threadIdx.x] = inv[t * topk + j0 + threadIdx.x];
      s_prob[threadIdx.x] = ld<T>(probs, t * topk + j0 + threadIdx.x);
    }
    __syncthreads();
    for (int q = 0; q < nj; ++q) {
      const int64_t r = s_row[q];
      const float pj = s_prob[q];
      u32x4_t x[kGradChunks];
#pragma unroll
      for (int c = 0; c < kGradChunks; ++c) x[c] = ldraw<T>(permuted, r * H + hc[c]);
      // the dot product adds +0 for an unused chunk (exact: part is never -0),
      // so every load is consumed outside a branch and none waits inside one
      float part = 0.0f;
#pragma unroll
      for (int c = 0; c < kGradChunks; ++c) {
        float gv[N], xv[N];
        widen<T>(g[c], gv);
        widen<T>(x[c], xv);
#pragma unroll
        for (int k = 0; k < N; ++k) part += has[c] ? gv[k] * xv[k] : 0.0f;
      }
#pragma unroll
      for (int c = 0; c < kGradChunks; ++c)
        if (has[c]) {
          float gv[N], o[N];
          widen<T>(g[c], gv);
#pragma unroll
          for (int k = 0; k < N; ++k) o[k] = gv[k] * pj;
          stv<T>(perm_grad, r * H + hc[c], o);
        }
#pragma unroll
      for (int m = 32; m >= 1; m >>= 1) part += __shfl_xor(part, m);
      if (lane == 0) s_part[q][wave] = part;
    }
    __syncthreads();
    if (static_cast<int>(threadIdx.x) < nj) {
      float sum = s_part[threadIdx.x][0];
#pragma unroll
      for (int w = 1; w < kThreads / 64; ++w) sum += s_part[threadIdx.x][w];
      st<T>(probs_grad, t * topk + j0 + threadIdx.x, sum);
    }
    __syncthreads();
  }
}

template <class T>
hipError_t launch_typed(const UnpermutePlan& p, const int32_t* inv, const void* a, const void* b,
                        const void* probs, void* o1, void* o2, bool grad, bool vec, hipStream_t s,
                        const WsHeader* hdr) {
  constexpr int N = Chunk<T>::N;
  if (!grad) {
    if (vec) {
      const dim3 grid(static_cast<unsigned>(p.batch),
                      static_cast<unsigned>((p.H / N + kThreads - 1) / kThreads));
      hipLaunchKernelGGL(unpermute_vec_kernel<T>, grid, dim3(kThreads), 0, s, hdr, inv, a, probs, o1,
                         p.H, p.topk);
    } else {
      const dim3 grid(static_cast<unsigned>(p.batch), static_cast<unsigned>((p.H + kCols - 1) / kCols));
      hipLaunchKernelGGL(unpermute_kernel<T>, grid, dim3(kThreads), 0, s, hdr, inv, a, probs, o1, p.H,
                         p.topk);
    }
  } else if (vec && p.H <= int64_t(kGradChunks) * kThreads * N) {
    hipLaunchKernelGGL(unpermute_grad_reg_kernel<T>, dim3(static_cast<unsigned>(p.batch)),
                       dim3(kThreads), 0, s, hdr, inv, a, b, probs, o1, o2, p.H, p.topk);
  } else if (vec) {
    hipLaunchKernelGGL(unpermute_grad_vec_kernel<T>, dim3(static_cast<unsigned>(p.batch)),
                       dim3(kThreads), 0, s, hdr, inv, a, b, probs, o1, o2, p.H, p.topk);
  } else {
    hipLaunchKernelGGL(unpermute_grad_kernel<T>, dim3(static_cast<unsigned>(p.batch)), dim3(kThreads),
                       0, s, hdr, inv, a, b, probs, o1, o2, p.H, p.topk);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_unpermute(const UnpermutePlan& p, void* ws, const int64_t* eri, const void* permuted,
                            const void* grad, const void* probs, void* out, void* probs_grad,
                            bool is_grad, hipStream_t s) {
  char* base = static_cast<char*>(ws);
  WsHeader* hdr = reinterpret_cast<WsHeader*>(base + p.off_header);
  Plan q{};
  q.M = p.M;
  q.topk = p.topk;
  q.row_idx_type = p.row_idx_type;
  WsView w{};
  w.hdr = hdr;
  w.inv = reinterpret_cast<int32_t*>(base + p.off_inv);
  w.ori = reinterpret_cast<int32_t*>(base + p.off_ori);
  hipLaunchKernelGGL(unpermute_reset_kernel, dim3(1), dim3(1), 0, s, hdr);
  hipError_t e = hipGetLastError();
  if (e == hipSuccess) e = launch_prep_index(q, eri, w, s);
  if (e == hipSuccess) e = launch_prep_verify(q, eri, w, s);
  if (e != hipSuccess) return e;
  if (!probs) {
    // gather (forward) or scatter (gradient) of whole rows
    // rows copied in 2-byte units (every element type is a whole number of them)
    const int64_t row_halves = p.H * (p.dtype == PGG_F32 ? 2 : 1);
    const unsigned yblocks =
        static_cast<unsigned>(std::min<int64_t>((row_halves + kThreads - 1) / kThreads, 16));
    const uint16_t* src = static_cast<const uint16_t*>(is_grad ? grad : permuted);
    hipLaunchKernelGGL(permute_rows_kernel, dim3(static_cast<unsigned>(p.M), yblocks), dim3(kThreads), 0,
                       s, hdr, w.inv, src, static_cast<uint16_t*>(out), row_halves, is_grad ? 1 : 0);
    return hipGetLastError();
  }
  // 16-byte chunks when every row and pointer is 16-byte aligned
  const size_t es = p.dtype == PGG_F32 ? 4 : 2;
  auto a16 = [](const void* q) { return q == nullptr || reinterpret_cast<uintptr_t>(q) % 16 == 0; };
  const bool vec = (size_t(p.H) * es) % 16 == 0 && a16(permuted) && a16(grad) && a16(out);
  if (p.dtype == PGG_F32)
    return launch_typed<TF32>(p, w.inv, permuted, grad, probs, out, probs_grad, is_grad, vec, s, hdr);
  if (p.dtype == PGG_BF16)
    return launch_typed<TBf16>(p, w.inv, permuted, grad, probs, out, probs_grad, is_grad, vec, s, hdr);
  return launch_typed<TF16>(p, w.inv, permuted, grad, probs, out, probs_grad, is_grad, vec, s, hdr);
}

}  // namespace pgg
