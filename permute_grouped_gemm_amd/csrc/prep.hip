// Kernels of the index preparation; the device code is in pgg_prep.h (the
// weight-sweep producer runs the same preparation in a spare workgroup).
#include "pgg_prep.h"

namespace pgg {

namespace {

__global__ __launch_bounds__(kPrepThreads) void prep_fused_kernel(PrepArgs a, const int64_t* eri,
                                                                  const int64_t* gl, WsView w) {
  __shared__ long long scratch[2 * kPrepThreads];
  prep_block(a, eri, gl, w, scratch);
}

__global__ __launch_bounds__(kPrepThreads) void prep_groups_kernel(PrepArgs a, const int64_t* gl,
                                                                   WsView w) {
  __shared__ long long scratch[2 * kPrepThreads];
  reset_header(w.hdr);
  __syncthreads();
  groups_phase(a, gl, w, scratch, scratch + kPrepThreads);
}

__global__ __launch_bounds__(256) void prep_index_kernel(PrepArgs a, const int64_t* eri, WsView w) {
  const int64_t t = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (t < a.M) index_one(a, eri, w, t);
}

__global__ __launch_bounds__(256) void prep_verify_kernel(PrepArgs a, const int64_t* eri, WsView w) {
  const int64_t t = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (t < a.M) verify_one(a, eri, w, t);
}

}  // namespace

hipError_t launch_prep_fused(const Plan& p, const int64_t* eri, const int64_t* gl,
                             const WsView& w, hipStream_t s) {
  // one wave for small problems: its scan barriers cost next to nothing
  const unsigned threads = (p.M <= 4096 && p.G <= 4096) ? 64u : unsigned(kPrepThreads);
  hipLaunchKernelGGL(prep_fused_kernel, dim3(1), dim3(threads), 0, s, prep_args(p), eri, gl, w);
  return hipGetLastError();
}

hipError_t launch_prep_groups(const Plan& p, const int64_t* gl, const WsView& w, hipStream_t s) {
  hipLaunchKernelGGL(prep_groups_kernel, dim3(1), dim3(kPrepThreads), 0, s, prep_args(p), gl, w);
  return hipGetLastError();
}

hipError_t launch_prep_index(const Plan& p, const int64_t* eri, const WsView& w, hipStream_t s) {
  const unsigned blocks = static_cast<unsigned>((p.M + 255) / 256);
  hipLaunchKernelGGL(prep_index_kernel, dim3(blocks), dim3(256), 0, s, prep_args(p), eri, w);
  return hipGetLastError();
}

hipError_t launch_prep_verify(const Plan& p, const int64_t* eri, const WsView& w, hipStream_t s) {
  const unsigned blocks = static_cast<unsigned>((p.M + 255) / 256);
  hipLaunchKernelGGL(prep_verify_kernel, dim3(blocks), dim3(256), 0, s, prep_args(p), eri, w);
  return hipGetLastError();
}

}  // namespace pgg
