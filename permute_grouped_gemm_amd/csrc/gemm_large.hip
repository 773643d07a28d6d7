// Producer for many rows per expert (fp16 / bf16): the grouped-matmul
// gradient C[i, k] = sum_n d_y[i, n] * W[g(i), k, n] with fp32 accumulation
// (MoeInitRoutingGroupedMatmulGrad design page, §数学定义和公式 Step 1; fp32
// cube output, §2.6.2) on 256x256 output tiles, written into the chunk's ring
// rows.
//
// One workgroup per tile, mapped by the XCD super-block raster (raster<8,4>):
// the 32 workgroups an XCD runs together share 8 d_y slabs and 4 weight slabs
// in its L2.
//
// Operand staging is direct global -> LDS (global_load_lds_dwordx4: lane i's
// 16 bytes land at M0 + 16 i), two stages of 64 reduction elements (64 KiB
// each: 256 d_y rows + 256 weight rows of 128 bytes, whole cache lines).  The
// loads are issued by inline assembly so the compiler does not serialise them
// with a blanket wait before every LDS read; the waits on their counter are
// explicit (vector memory operations complete in issue order, and these loads
// write no register).
//
// Per stage and wave (2 x 4 waves, two per SIMD, 128 x 64 fp32 accumulators
// each): four chunk pairs of 8 MFMA 32x32x16; the fragments of the next pair
// are read while the current pair multiplies, across stage boundaries too.
// The second wave on each SIMD keeps the matrix unit fed while the other
// issues its loads or waits on LDS.
//
// LDS rows are 128 bytes (8 chunks).  128-bit LDS reads are served 16 lanes
// at a time over 64 banks (256 bytes = 2 rows); a fragment read puts 16
// consecutive rows, same chunk, in those lanes, so chunk c of row r sits at
// slot c ^ ((r >> 1) & 7): the 8 rows of each parity get 8 different slots.
//
// Masked-off lanes (rows past the tile's rows, columns past K, reduction past
// N) load 16 zero bytes from a constant in global memory instead.  Ring stores are
// ordinary (temporal) stores: the consumer, which reads each ring row once
// with non-temporal loads right after this launch, then finds part of the
// ring in the last-level cache.
#include "pgg_device.h"

namespace pgg {

namespace {

constexpr int kBM = 256, kBN = 256;
constexpr int kThreads = 512, kWaves = 8;    // two waves per SIMD
constexpr int kWM = 2;                        // waves along rows
constexpr int kWTM = 128, kWTN = 64;          // wave tile
constexpr int kFM = kWTM / 32, kFN = kWTN / 32;
constexpr int kRowChunks = 8;                 // 16-byte chunks per LDS row per stage
constexpr int kBK = kRowChunks * 8;           // reduction elements per stage
constexpr int kPairs = kRowChunks / 2;
constexpr int kStages = 2;
constexpr int kSlotsA = kBM * kRowChunks;
constexpr int kSlotsB = kBN * kRowChunks;
constexpr int kStageSlots = kSlotsA + kSlotsB;
constexpr int kRowsPerLoad = 64 / kRowChunks;          // rows one wave instruction covers
constexpr int kLoadRows = kRowsPerLoad * kWaves;       // rows one load index covers across the waves
constexpr int kLoadsA = kSlotsA / kThreads;            // direct-to-LDS loads per thread per stage
constexpr int kLoadsB = kSlotsB / kThreads;
constexpr int kLoadsPerStage = kLoadsA + kLoadsB;
constexpr int kSuperM = 8, kSuperN = 4;                // super-block of tiles per XCD round
constexpr int kSuper = kSuperM * kSuperN;
constexpr int kXcds = 8;
static_assert(kLoadsPerStage * kStages <= 63, "vmcnt range");
static_assert(kPairs % 2 == 0, "a stage must end on the second fragment set");
static_assert(kRowsPerLoad * kWaves * kLoadsA == kBM && kRowsPerLoad * kWaves * kLoadsB == kBN,
              "loads cover the tile rows");

struct LargeArgs {
  const void* A;            // grad_y [M, N]
  const void* B;            // weight [G, K, N]
  const WsHeader* hdr;
  const MTile* tiles;
  const int32_t* chunk_row0;
  float* ring;              // [ring_rows, ldc]: columns [k_lo, k_hi) of the panel
  int64_t N, K;
  int64_t k_lo, k_hi, ldc;
  int32_t chunk, tc, n_col_tiles;
};

__device__ __forceinline__ int slot_of(int r, int c) { return c ^ ((r >> 1) & 7); }

template <class T>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void produce_large_kernel(LargeArgs a) {
  using E = typename T::elem;
  __shared__ u32x4_t lds[kStages * kStageSlots];

  if (a.hdr->err != kNoError) return;
  int slot, ct;
  if (!raster<kSuperM, kSuperN>(blockIdx.x, a.tc, a.n_col_tiles, slot, ct)) return;
  const int64_t tile_idx = static_cast<int64_t>(a.chunk) * a.tc + slot;
  if (tile_idx >= a.hdr->n_tiles) return;
  const MTile tile = a.tiles[tile_idx];
  if (tile.rows <= 0) return;
  const int rows = tile.rows;
  const int64_t col0 = a.k_lo + static_cast<int64_t>(ct) * kBN;
  const int cols = static_cast<int>(min<int64_t>(kBN, a.k_hi - col0));
  if (cols <= 0) return;
  const int64_t N = a.N;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave % kWM, wn = wave / kWM;
  const int lr = lane & 31, lh = lane >> 5;
  // Direct-to-LDS load j of this wave fills slots (j*kWaves + wave)*64 + lane of a
  // region: row r0 + kLoadRows j (r0 = wave*8 + lane/8), slot lane%8, which
  // holds chunk (lane%8) ^ ((r0/2)%8) -- the same for every j.
  const int r0 = wave * kRowsPerLoad + (lane >> 3);
  const int dma_c = slot_of(r0, lane & 7);
  const E* pa = static_cast<const E*>(a.A) + (static_cast<int64_t>(tile.row0) + r0) * N + dma_c * 8;
  const E* pb =
      static_cast<const E*>(a.B) + (static_cast<int64_t>(tile.g) * a.K + col0 + r0) * N + dma_c * 8;
  uint32_t va = 0, vb = 0;   // bit j: load j's row lies inside the tile
#pragma unroll
  for (int j = 0; j < kLoadsA; ++j) va |= (r0 + kLoadRows * j < rows ? 1u : 0u) << j;
#pragma unroll
  for (int j = 0; j < kLoadsB; ++j) vb |= (r0 + kLoadRows * j < cols ? 1u : 0u) << j;
  const void* zero = &kZero16;
  const uint32_t lds0 = __builtin_amdgcn_readfirstlane(lds_offset(lds));
  const int64_t row_step = kLoadRows * N;

  auto issue = [&](int kt) {
    const uint32_t base = lds0 + static_cast<uint32_t>((kt % kStages) * kStageSlots * 16);
    const int64_t n0 = static_cast<int64_t>(kt) * kBK;
    const bool in_n = n0 + dma_c * 8 < N;
#pragma unroll
    for (int j = 0; j < kLoadsA; ++j)
      dma16(in_n && ((va >> j) & 1) ? static_cast<const void*>(pa + j * row_step + n0) : zero,
            base + static_cast<uint32_t>((j * kWaves + wave) * 64 * 16));
#pragma unroll
    for (int j = 0; j < kLoadsB; ++j)
      dma16(in_n && ((vb >> j) & 1) ? static_cast<const void*>(pb + j * row_step + n0) : zero,
            base + static_cast<uint32_t>((kSlotsA + (j * kWaves + wave) * 64) * 16));
  };

  // fragment rows start at multiples of 32, so (row >> 1) & 7 == (lr >> 1) & 7
  auto load_frags = [&](int kt, int q, u32x4_t (&fa)[kFM], u32x4_t (&fb)[kFN]) {
    const u32x4_t* st = lds + (kt % kStages) * kStageSlots;
    const int sl = slot_of(lr, 2 * q + lh);
#pragma unroll
    for (int i = 0; i < kFM; ++i) fa[i] = st[(wm * kWTM + i * 32 + lr) * kRowChunks + sl];
#pragma unroll
    for (int j = 0; j < kFN; ++j) fb[j] = st[kSlotsA + (wn * kWTN + j * 32 + lr) * kRowChunks + sl];
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

  const int nk = static_cast<int>((N + kBK - 1) / kBK);
#pragma unroll
  for (int s = 0; s < kStages; ++s)
    if (s < nk) issue(s);
  u32x4_t fa0[kFM], fb0[kFN], fa1[kFM], fb1[kFN];
  // stage 0 landed (stage 1, if any, may still be in flight)
  if (nk > 1) wait_then_barrier<kLoadsPerStage>(); else wait_then_barrier<0>();
  load_frags(0, 0, fa0, fb0);
  int kt = 0;
  // steady state, free of branches so the compiler's LDS wait counts stay exact
  for (; kt + kStages < nk; ++kt) {
#pragma unroll
    for (int q = 0; q < kPairs; ++q) {
      if (q + 1 < kPairs) {
        if (q & 1) load_frags(kt, q + 1, fa0, fb0); else load_frags(kt, q + 1, fa1, fb1);
      } else {
        // stage kt+1 landed everywhere and every wave is done with stage kt;
        // the refill of stage kt's buffer is issued by the first wave of each
        // SIMD before its last MFMAs of the stage and by the second after
        // them, so one of the two is always feeding the matrix unit
        wait_then_barrier<0>();
        if (wave < kWaves / 2) issue(kt + kStages);
        load_frags(kt + 1, 0, fa0, fb0);
      }
      if (q & 1) mfmas(fa1, fb1); else mfmas(fa0, fb0);
      if (q + 1 == kPairs && wave >= kWaves / 2) issue(kt + kStages);
    }
  }
  // last stages: nothing more to issue
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
  const int64_t ring_row0 = static_cast<int64_t>(tile.row0) - a.chunk_row0[a.chunk];
  float* __restrict__ out = a.ring + ring_row0 * a.ldc + (col0 - a.k_lo);
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
          out[static_cast<int64_t>(m) * a.ldc + n] = acc[i][j][v];
      }
    }
}

}  // namespace

bool produce_uses_dma(const Plan& p, bool aligned) {
  return aligned && p.regime == kLarge && p.dtype != PGG_F32;
}

hipError_t launch_produce_dma(const Plan& p, int chunk, int panel, const void* grad_y,
                              const void* weight, const WsView& w, hipStream_t s) {
  LargeArgs a;
  a.A = grad_y;
  a.B = weight;
  a.hdr = w.hdr;
  a.tiles = w.tiles;
  a.chunk_row0 = w.chunk_row0;
  a.ring = w.ring;
  a.N = p.N;
  a.K = p.K;
  panel_range(p, panel, &a.k_lo, &a.k_hi);
  a.ldc = p.panel_cols;
  a.chunk = chunk;
  a.tc = p.tc;
  a.n_col_tiles = p.n_col_tiles;
  unsigned tiles = static_cast<unsigned>(p.tc) * static_cast<unsigned>(p.n_col_tiles);
  tiles = (tiles + kXcds * kSuper - 1) / (kXcds * kSuper) * (kXcds * kSuper);   // whole raster rounds
  if (p.dtype == PGG_BF16)
    hipLaunchKernelGGL(produce_large_kernel<TBf16>, dim3(tiles), dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL(produce_large_kernel<TF16>, dim3(tiles), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace pgg
