// Forward grouped matmul for many rows per expert (fp16 / bf16), rows 16-byte
// aligned: y[i, n] = sum_k x[p(i) / topK, k] * W[g(i), k, n] with fp32
// accumulation (MoeInitRoutingGroupedMatmulGrad design page, §数学定义和公式,
// forward formulas), on 256x256 output tiles.
//
// The pipeline is the backward's large-tile producer: 8 waves (two per SIMD)
// of 128 x 64 fp32 accumulators, two LDS stages of 64 reduction elements
// filled by direct global -> LDS loads (global_load_lds_dwordx4: lane i's 16
// bytes land at M0 + 16 i), explicit waits on the vector-memory counter, the
// refill of a stage issued by the first wave of each SIMD right after the
// stage barrier and by the second after its last MFMAs of the stage, and the
// XCD super-block raster.  What differs is where the operands come from:
//
// * A (64 KiB of a stage's 128): the tile's rows are gathered.  Row r is token
//   ori[row0 + r] / topK of x; every lane keeps the addresses of its 4 rows.
//   LDS rows are 128 bytes (8 chunks), chunk c of row r at slot
//   c ^ ((r >> 1) & 7), read as in the backward.
// * B: W[g] is [K, N] with n contiguous, so the stage holds 64 rows of k, each
//   the tile's 256 columns (512 bytes, 8 segments of 64 bytes; segment s of
//   row k at s ^ (k & 3)).  A load instruction fills 1 KiB = two rows, each
//   lane a fixed 16-byte slot, so each lane fetches the global chunk that
//   belongs in its slot.  MFMA operands are read with ds_read_b64_tr_b16:
//   in each 16-lane group, lane i receives element i % 4 of the 8-byte chunks
//   addressed by lanes 4j + i / 4 (j = 0..3); lanes addressing rows k0 + s / 4,
//   columns n0 + 4 (s % 4) give lane i column n0 + i at rows k0 .. k0+3, and
//   two reads give the 8 consecutive k of a 32x32x16 operand.  The 4 rows one
//   half-wave reads sit in 4 different 64-byte bank groups.
//
// Masked-off lanes (rows past the tile, columns past N, reduction past K)
// load 16 zero bytes from a constant in global memory.  y is stored with
// non-temporal stores.
#include "pgg_device.h"

namespace pgg {

namespace {

typedef __fp16 h16x4_t __attribute__((__vector_size__(4 * sizeof(__fp16))));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kBM = 256, kBN = 256;
constexpr int kThreads = 512, kWaves = 8;    // two waves per SIMD
constexpr int kWM = 2;                        // waves along rows
constexpr int kWTM = 128, kWTN = 64;          // wave tile
constexpr int kFM = kWTM / 32, kFN = kWTN / 32;
constexpr int kRowChunks = 8;                 // A: 16-byte chunks per LDS row per stage
constexpr int kBK = kRowChunks * 8;           // reduction elements per stage
constexpr int kPairs = kRowChunks / 2;
constexpr int kStages = 2;
constexpr int kSlotsA = kBM * kRowChunks;
constexpr int kBRowChunks = kBN * 2 / 16;     // B: chunks per row (512 bytes)
constexpr int kSlotsB = kBK * kBRowChunks;
constexpr int kStageSlots = kSlotsA + kSlotsB;
constexpr int kRowsPerLoad = 64 / kRowChunks;          // A rows one wave instruction covers
constexpr int kLoadRows = kRowsPerLoad * kWaves;       // A rows one load index covers
constexpr int kBRowsPerLoad = 64 / kBRowChunks;        // B rows one wave instruction covers
constexpr int kLoadsA = kSlotsA / kThreads;
constexpr int kLoadsB = kSlotsB / kThreads;
constexpr int kLoadsPerStage = kLoadsA + kLoadsB;
constexpr int kSuperM = 8, kSuperN = 4;
constexpr int kSuper = kSuperM * kSuperN;
constexpr int kXcds = 8;
static_assert(kLoadsPerStage * kStages <= 63, "vmcnt range");
static_assert(kPairs % 2 == 0, "a stage must end on the second fragment set");
static_assert(kRowsPerLoad * kWaves * kLoadsA == kBM, "A loads cover the tile rows");
static_assert(kBRowsPerLoad * kWaves * kLoadsB == kBK, "B loads cover the stage rows");

struct FwdLargeArgs {
  const void* X;            // x [batch, R]
  const void* W;            // weight [G, R, C]
  const WsHeader* hdr;
  const MTile* tiles;
  const int32_t* ori;
  float* y;                 // [M, C]
  int64_t R, C, topk;
  int32_t n_slots, n_col_tiles;
};

__device__ __forceinline__ int slot_of(int r, int c) { return c ^ ((r >> 1) & 7); }

// byte offset of byte b of B row k inside the B region
__device__ __forceinline__ uint32_t b_off(int k, int b) {
  return static_cast<uint32_t>(k * 512 + ((((b >> 6) ^ (k & 3))) << 6) + (b & 63));
}

template <class T>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fwd_large_kernel(FwdLargeArgs a) {
  using E = typename T::elem;
  __shared__ u32x4_t lds[kStages * kStageSlots];

  if (a.hdr->err != kNoError) return;
  int slot, ct;
  if (!raster<kSuperM, kSuperN>(blockIdx.x, a.n_slots, a.n_col_tiles, slot, ct)) return;
  if (slot >= a.hdr->n_tiles) return;
  const MTile tile = a.tiles[slot];
  if (tile.rows <= 0) return;
  const int rows = tile.rows;
  const int64_t col0 = static_cast<int64_t>(ct) * kBN;
  const int cols = static_cast<int>(min<int64_t>(kBN, a.C - col0));
  const int64_t R = a.R, C = a.C;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave % kWM, wn = wave / kWM;
  const int lr = lane & 31, lh = lane >> 5;

  // A: load j of this lane fills row r0 + kLoadRows j, physical slot lane % 8,
  // which holds chunk dma_c (the same for every j).
  const int r0 = wave * kRowsPerLoad + (lane >> 3);
  const int dma_c = slot_of(r0, lane & 7);
  // topK and positions are below M < 2^31: 32-bit unsigned division
  const uint32_t topk32 = static_cast<uint32_t>(a.topk);
  const E* pa[kLoadsA];
  uint32_t va = 0;
#pragma unroll
  for (int j = 0; j < kLoadsA; ++j) {
    const int r = r0 + kLoadRows * j;
    const bool ok = r < rows;
    const int64_t tok = ok ? static_cast<uint32_t>(a.ori[tile.row0 + r]) / topk32 : 0;
    pa[j] = static_cast<const E*>(a.X) + tok * R + dma_c * 8;
    va |= (ok ? 1u : 0u) << j;
  }
  // B: load j of this lane fills stage row kb_j, physical chunk lane % 32,
  // which holds logical chunk lc_j.
  const E* Wg = static_cast<const E*>(a.W) + static_cast<int64_t>(tile.g) * R * C;
  int kb[kLoadsB];
  int64_t boff[kLoadsB];
  uint32_t vb = 0;
#pragma unroll
  for (int j = 0; j < kLoadsB; ++j) {
    kb[j] = (j * kWaves + wave) * kBRowsPerLoad + lane / kBRowChunks;
    const int pc = lane % kBRowChunks;
    const int lc = (((pc >> 2) ^ (kb[j] & 3)) << 2) | (pc & 3);
    const int64_t col = col0 + lc * 8;
    boff[j] = kb[j] * C + col;
    vb |= (col < C ? 1u : 0u) << j;
  }
  const void* zero = &kZero16;
  const uint32_t lds0 = __builtin_amdgcn_readfirstlane(lds_offset(lds));

  auto issue = [&](int kt) {
    const uint32_t base = lds0 + static_cast<uint32_t>((kt % kStages) * kStageSlots * 16);
    const int64_t k0 = static_cast<int64_t>(kt) * kBK;
    const bool in_k = k0 + dma_c * 8 < R;
#pragma unroll
    for (int j = 0; j < kLoadsA; ++j)
      dma16(in_k && ((va >> j) & 1) ? static_cast<const void*>(pa[j] + k0) : zero,
            base + static_cast<uint32_t>((j * kWaves + wave) * 64 * 16));
    const E* wk = Wg + k0 * C;
#pragma unroll
    for (int j = 0; j < kLoadsB; ++j)
      dma16(k0 + kb[j] < R && ((vb >> j) & 1) ? static_cast<const void*>(wk + boff[j]) : zero,
            base + static_cast<uint32_t>((kSlotsA + (j * kWaves + wave) * 64) * 16));
  };

  auto load_frags = [&](int kt, int q, u32x4_t (&fa)[kFM], u32x4_t (&fb)[kFN]) {
    const u32x4_t* st = lds + (kt % kStages) * kStageSlots;
    const int sl = slot_of(lr, 2 * q + lh);
#pragma unroll
    for (int i = 0; i < kFM; ++i) fa[i] = st[(wm * kWTM + i * 32 + lr) * kRowChunks + sl];
    auto breg = (__attribute__((address_space(3))) char*)(reinterpret_cast<const char*>(st + kSlotsA));
    const int grp = lane >> 4, s = lane & 15;
    const int k0 = 8 * (2 * q + (grp >> 1)) + (s >> 2);
#pragma unroll
    for (int j = 0; j < kFN; ++j) {
      const int nb = 2 * (wn * kWTN + j * 32 + 16 * (grp & 1) + 4 * (s & 3));
      const u32x2_t lo = __builtin_bit_cast(
          u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4f16(
                       (__attribute__((address_space(3))) h16x4_t*)(breg + b_off(k0, nb))));
      const u32x2_t hi = __builtin_bit_cast(
          u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4f16(
                       (__attribute__((address_space(3))) h16x4_t*)(breg + b_off(k0 + 4, nb))));
      fb[j] = u32x4_t{lo[0], lo[1], hi[0], hi[1]};
    }
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

  const int nk = static_cast<int>((R + kBK - 1) / kBK);
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

  // Epilogue: accumulator v of lane (lr, lh) is row 8*(v/4) + 4*lh + v%4,
  // column lr of its 32x32 block.
  float* __restrict__ out = a.y + static_cast<int64_t>(tile.row0) * C + col0;
  const bool full = rows == kBM && cols == kBN;
#pragma unroll
  for (int i = 0; i < kFM; ++i)
#pragma unroll
    for (int j = 0; j < kFN; ++j) {
      const int n = wn * kWTN + j * 32 + lr;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int m = wm * kWTM + i * 32 + 8 * (v >> 2) + 4 * lh + (v & 3);
        if (full || (m < rows && n < cols))
          __builtin_nontemporal_store(acc[i][j][v], out + static_cast<int64_t>(m) * C + n);
      }
    }
}

}  // namespace

hipError_t launch_forward_large(const Plan& p, const void* x, const void* weight, float* y,
                                const WsView& w, hipStream_t s) {
  FwdLargeArgs a;
  a.X = x;
  a.W = weight;
  a.hdr = w.hdr;
  a.tiles = w.tiles;
  a.ori = w.ori;
  a.y = y;
  a.R = p.N;
  a.C = p.K;
  a.topk = p.topk;
  a.n_slots = p.max_tiles;
  a.n_col_tiles = p.n_col_tiles;
  unsigned tiles = static_cast<unsigned>(p.max_tiles) * static_cast<unsigned>(p.n_col_tiles);
  tiles = (tiles + kXcds * kSuper - 1) / (kXcds * kSuper) * (kXcds * kSuper);   // whole raster rounds
  if (p.dtype == PGG_BF16)
    hipLaunchKernelGGL(fwd_large_kernel<TBf16>, dim3(tiles), dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL(fwd_large_kernel<TF16>, dim3(tiles), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace pgg
