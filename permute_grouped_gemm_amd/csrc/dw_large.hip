// Weight gradient for fp16 / bf16 rows that are 16-byte aligned:
//
//   dW[g, k, n] = sum over expert g's expanded rows i of x[p(i) / topK, k] * d_y[i, n]
//
// (MoeInitRoutingGroupedMatmulGrad design page, §1.2: expanded_x^T · d_y per
// expert), on 256 x 256 tiles of (k, n), each reduced over all of the expert's
// rows by one workgroup in a fixed order.
//
// The pipeline is the forward's large tile (8 waves of 128 x 64 fp32
// accumulators, two LDS stages of 64 reduction rows filled by direct
// global -> LDS loads, explicit waits, staggered refill, XCD raster).  Both
// operands are stages of reduction rows i, 512 bytes each (64-byte segments
// XOR-swizzled by row): the tile's 256 columns of x (row i gathered: token
// ori[i] / topK) and of d_y (row i).  A load instruction fills two stage rows,
// lanes 0-31 the first and 32-63 the second, so the two rows' positions are
// one scalar load of ori (its own counter, so waiting for it never drains
// the direct-to-LDS loads in flight).  Both MFMA operands are transposed LDS
// reads (ds_read_b64_tr_b16: in each 16-lane group, lane i receives element
// i % 4 of the 8-byte chunks addressed by lanes 4j + i / 4, so lanes
// addressing rows r0 + s / 4, columns c0 + 4 (s % 4) give lane i column c0 + i
// at rows r0 .. r0+3; two reads give the 8 reduction rows of an operand).
//
// Rows past the expert's last, and columns past K or N, load 16 zero bytes
// from a constant in global memory; an expert without rows writes zeros.
#include "pgg_device.h"

namespace pgg {

namespace {

typedef __fp16 h16x4_t __attribute__((__vector_size__(4 * sizeof(__fp16))));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kBM = 256, kBN = 256;           // k x n per tile
constexpr int kThreads = 512, kWaves = 8;
constexpr int kWM = 2;
constexpr int kWTM = 128, kWTN = 64;
constexpr int kFM = kWTM / 32, kFN = kWTN / 32;
constexpr int kBK = 64;                       // reduction rows per stage
constexpr int kPairs = 4;                     // 16-row MFMA steps per stage, in pairs
constexpr int kStages = 2;
constexpr int kRowChunks = 512 / 16;          // chunks per stage row
constexpr int kSlots = kBK * kRowChunks;      // per operand and stage
constexpr int kStageSlots = 2 * kSlots;
constexpr int kRowsPerLoad = 64 / kRowChunks; // stage rows one wave instruction covers
constexpr int kLoads = kSlots / kThreads;     // per operand, thread and stage
constexpr int kLoadsPerStage = 2 * kLoads;
constexpr int kSuperM = 8, kSuperN = 4;
constexpr int kSuper = kSuperM * kSuperN;
constexpr int kXcds = 8;
static_assert(kLoadsPerStage * kStages <= 63, "vmcnt range");
static_assert(kRowsPerLoad * kWaves * kLoads == kBK, "loads cover the stage rows");

struct DwLargeArgs {
  const void* X;            // x [batch, K]
  const void* DY;           // d_y [M, N]
  const WsHeader* hdr;
  const int64_t* offsets;   // [G + 1]
  const int32_t* ori;       // [M]
  float* dw;                // [G, K, N]
  int64_t K, N, topk;
  int32_t n_kb, n_slots, n_col_tiles;
};

__device__ __forceinline__ uint32_t st_off(int r, int b) {
  return static_cast<uint32_t>(r * 512 + ((((b >> 6) ^ (r & 3))) << 6) + (b & 63));
}

// ori[i] and, when `pair`, ori[i + 1]: wave-uniform scalar loads (reads only).
__device__ __forceinline__ void scalar_ori(const int32_t* p, bool pair, int32_t& a, int32_t& b) {
  if (pair) {
    i32x2_t v;
    asm volatile("s_load_dwordx2 %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(p) : "memory");
    a = v[0];
    b = v[1];
  } else {
    int32_t v;
    asm volatile("s_load_dword %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(p) : "memory");
    a = v;
    b = v;
  }
}

template <class T>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void dw_large_kernel(DwLargeArgs a) {
  using E = typename T::elem;
  __shared__ u32x4_t lds[kStages * kStageSlots];

  if (a.hdr->err != kNoError) return;
  int slot, ct;
  if (!raster<kSuperM, kSuperN>(blockIdx.x, a.n_slots, a.n_col_tiles, slot, ct)) return;
  const int g = slot / a.n_kb;
  const int64_t k0 = static_cast<int64_t>(slot % a.n_kb) * kBM;
  const int64_t n0 = static_cast<int64_t>(ct) * kBN;
  const int kvalid = static_cast<int>(min<int64_t>(kBM, a.K - k0));
  const int nvalid = static_cast<int>(min<int64_t>(kBN, a.N - n0));
  const int64_t r_begin = a.offsets[g], r_end = a.offsets[g + 1];
  const int64_t K = a.K, N = a.N;
  const uint32_t topk32 = static_cast<uint32_t>(a.topk);   // below 2^31

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave % kWM, wn = wave / kWM;
  const int lr = lane & 31;
  // Load j of this lane fills stage row (j*kWaves + wave)*2 + lane/32 at
  // physical chunk lane % 32, which holds logical chunk lc (the same for all j).
  const int half = lane >> 5;
  const int pc = lane & 31;
  const int lc = (((pc >> 2) ^ ((2 * wave + half) & 3)) << 2) | (pc & 3);
  const bool a_col = k0 + lc * 8 < K;
  const bool b_col = n0 + lc * 8 < N;
  const E* xcol = static_cast<const E*>(a.X) + k0 + lc * 8;
  const E* dycol = static_cast<const E*>(a.DY) + n0 + lc * 8;
  const void* zero = &kZero16;
  const uint32_t lds0 = __builtin_amdgcn_readfirstlane(lds_offset(lds));

  auto issue = [&](int kt) {
    const uint32_t base = lds0 + static_cast<uint32_t>((kt % kStages) * kStageSlots * 16);
    const int64_t i0 = r_begin + static_cast<int64_t>(kt) * kBK;
#pragma unroll
    for (int j = 0; j < kLoads; ++j) {
      const int64_t pair0 = i0 + (j * kWaves + wave) * kRowsPerLoad;   // wave-uniform
      int32_t p0 = 0, p1 = 0;
      if (pair0 < r_end) scalar_ori(a.ori + pair0, pair0 + 1 < r_end, p0, p1);
      const int64_t i = pair0 + half;
      const bool row_ok = i < r_end;
      const int64_t tok = static_cast<uint32_t>(half ? p1 : p0) / topk32;
      dma16(row_ok && a_col ? static_cast<const void*>(xcol + tok * K) : zero,
            base + static_cast<uint32_t>((j * kWaves + wave) * 64 * 16));
      dma16(row_ok && b_col ? static_cast<const void*>(dycol + i * N) : zero,
            base + static_cast<uint32_t>((kSlots + (j * kWaves + wave) * 64) * 16));
    }
  };

  // Operand of columns colbase .. colbase+31, chunk pair q: the 8 reduction
  // rows starting at 8*(2q + lane/32).
  auto load_tr = [&](__attribute__((address_space(3))) char* region, int colbase, int q) -> u32x4_t {
    const int grp = lane >> 4, s = lane & 15;
    const int cb = 2 * (colbase + 16 * (grp & 1) + 4 * (s & 3));
    const int r0 = 8 * (2 * q + (grp >> 1)) + (s >> 2);
    const u32x2_t lo = __builtin_bit_cast(
        u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4f16(
                     (__attribute__((address_space(3))) h16x4_t*)(region + st_off(r0, cb))));
    const u32x2_t hi = __builtin_bit_cast(
        u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4f16(
                     (__attribute__((address_space(3))) h16x4_t*)(region + st_off(r0 + 4, cb))));
    return u32x4_t{lo[0], lo[1], hi[0], hi[1]};
  };
  auto load_frags = [&](int kt, int q, u32x4_t (&fa)[kFM], u32x4_t (&fb)[kFN]) {
    const u32x4_t* st = lds + (kt % kStages) * kStageSlots;
    auto ra = (__attribute__((address_space(3))) char*)(reinterpret_cast<const char*>(st));
    auto rb = (__attribute__((address_space(3))) char*)(reinterpret_cast<const char*>(st + kSlots));
#pragma unroll
    for (int i = 0; i < kFM; ++i) fa[i] = load_tr(ra, wm * kWTM + i * 32, q);
#pragma unroll
    for (int j = 0; j < kFN; ++j) fb[j] = load_tr(rb, wn * kWTN + j * 32, q);
  };
  f32x16_t acc[kFM][kFN];
#pragma unroll
  for (int i = 0; i < kFM; ++i)
#pragma unroll
    for (int j = 0; j < kFN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;
  auto mfmas = [&](const u32x4_t (&fa)[kFM], const u32x4_t (&fb)[kFN]) {
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < kFM; ++i)
#pragma unroll
      for (int j = 0; j < kFN; ++j) mma<T>(acc[i][j], fa[i], fb[j]);
    __builtin_amdgcn_sched_barrier(0);
  };

  const int nk = static_cast<int>((r_end - r_begin + kBK - 1) / kBK);
  if (nk > 0) {
#pragma unroll
    for (int s = 0; s < kStages; ++s)
      if (s < nk) issue(s);
    u32x4_t fa0[kFM], fb0[kFN], fa1[kFM], fb1[kFN];
    if (nk > 1) wait_then_barrier<kLoadsPerStage>(); else wait_then_barrier<0>();
    load_frags(0, 0, fa0, fb0);
    int kt = 0;
    for (; kt + kStages < nk; ++kt) {
#pragma unroll
      for (int q = 0; q < kPairs; ++q) {
        if (q + 1 < kPairs) {
          if (q & 1) load_frags(kt, q + 1, fa0, fb0); else load_frags(kt, q + 1, fa1, fb1);
        } else {
          wait_then_barrier<0>();
          if (wave < kWaves / 2) issue(kt + kStages);
          load_frags(kt + 1, 0, fa0, fb0);
        }
        if (q & 1) mfmas(fa1, fb1); else mfmas(fa0, fb0);
        if (q + 1 == kPairs && wave >= kWaves / 2) issue(kt + kStages);
      }
    }
    for (; kt < nk; ++kt) {
#pragma unroll
      for (int q = 0; q < kPairs; ++q) {
        if (q + 1 < kPairs) {
          if (q & 1) load_frags(kt, q + 1, fa0, fb0); else load_frags(kt, q + 1, fa1, fb1);
        } else if (kt + 1 < nk) {
          wait_then_barrier<0>();
          load_frags(kt + 1, 0, fa0, fb0);
        }
        if (q & 1) mfmas(fa1, fb1); else mfmas(fa0, fb0);
      }
    }
  }

  // Epilogue: accumulator v of lane (lr, half) is row 8*(v/4) + 4*half + v%4
  // (a k), column lr (an n) of its 32x32 block.
  float* __restrict__ out = a.dw + (static_cast<int64_t>(g) * K + k0) * N + n0;
  const bool full = kvalid == kBM && nvalid == kBN;
#pragma unroll
  for (int i = 0; i < kFM; ++i)
#pragma unroll
    for (int j = 0; j < kFN; ++j) {
      const int n = wn * kWTN + j * 32 + lr;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int m = wm * kWTM + i * 32 + 8 * (v >> 2) + 4 * half + (v & 3);
        if (full || (m < kvalid && n < nvalid))
          __builtin_nontemporal_store(acc[i][j][v], out + static_cast<int64_t>(m) * N + n);
      }
    }
}

}  // namespace

hipError_t launch_dw_large(const Plan& p, const void* x, const void* grad_y, float* dw,
                           const WsView& w, hipStream_t s) {
  DwLargeArgs a;
  a.X = x;
  a.DY = grad_y;
  a.hdr = w.hdr;
  a.offsets = w.offsets;
  a.ori = w.ori;
  a.dw = dw;
  a.K = p.N;
  a.N = p.K;
  a.topk = p.topk;
  a.n_kb = static_cast<int32_t>((a.K + kBM - 1) / kBM);
  a.n_slots = static_cast<int32_t>(p.G) * a.n_kb;
  a.n_col_tiles = static_cast<int32_t>((a.N + kBN - 1) / kBN);
  unsigned tiles = static_cast<unsigned>(a.n_slots) * static_cast<unsigned>(a.n_col_tiles);
  tiles = (tiles + kXcds * kSuper - 1) / (kXcds * kSuper) * (kXcds * kSuper);
  if (p.dtype == PGG_BF16)
    hipLaunchKernelGGL(dw_large_kernel<TBf16>, dim3(tiles), dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL(dw_large_kernel<TF16>, dim3(tiles), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace pgg
