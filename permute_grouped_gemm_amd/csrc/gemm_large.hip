// Producer for many rows per expert (fp16 / bf16): the grouped-matmul
// gradient C[i, k] = sum_n d_y[i, n] * W[g(i), k, n] with fp32 accumulation
// (MoeInitRoutingGroupedMatmulGrad design page, §数学定义和公式 Step 1; fp32
// cube output, §2.6.2) on 256x256 output tiles, written into the chunk's ring
// rows.
//
// Operand staging is direct global -> LDS (global_load_lds_dwordx4: each
// lane's 16 bytes land at M0 + 16 * lane), so no registers or ds_write
// instructions carry the tiles.  Four LDS stages of 32 reduction elements
// (32 KiB each: 256 d_y rows + 256 weight rows of 64 bytes) are in flight; a
// stage is consumed three stages after its loads were issued.  The loads are
// issued by inline assembly so that the compiler does not serialise them with
// a blanket wait before every LDS read; the waits on their counter are
// explicit (vmcnt counts loads in issue order).
//
// Per stage, per wave (2 x 2 waves, 128 x 128 accumulators each): two chunk
// pairs of 16 MFMA 32x32x16.  The fragments of pair q+1 are read while pair q
// multiplies, and the first pair of the next stage is read while the last
// pair of this stage multiplies; one barrier per stage makes the next stage
// visible and frees the buffer that is refilled.
//
// LDS rows are 64 bytes (4 chunks).  A wave's 128-bit reads are served 16
// lanes at a time over 64 banks (256 bytes = 4 rows); fragment reads put 16
// consecutive rows in those lanes, so chunk c of row r sits at slot
// c ^ ((r >> 2) & 3): the 4 rows sharing a bank quarter get 4 different slots.
//
// Masked-off lanes (rows past the tile's rows, columns past K, reduction
// past N) load 16 zero bytes from the workspace header instead.
#include "pgg_device.h"

namespace pgg {

namespace {

constexpr int kBM = 256, kBN = 256;
constexpr int kThreads = 256, kWaves = 4;
constexpr int kWM = 2;                        // waves along rows
constexpr int kWTM = 128, kWTN = 128;         // wave tile
constexpr int kFM = kWTM / 32, kFN = kWTN / 32;
constexpr int kRowChunks = 4;                 // 16-byte chunks per LDS row per stage
constexpr int kBK = kRowChunks * 8;           // reduction elements per stage
constexpr int kStages = 4;
constexpr int kSlotsA = kBM * kRowChunks;
constexpr int kSlotsB = kBN * kRowChunks;
constexpr int kStageSlots = kSlotsA + kSlotsB;
constexpr int kLoadsA = kSlotsA / kThreads;   // direct-to-LDS loads per thread per stage
constexpr int kLoadsB = kSlotsB / kThreads;
constexpr int kLoadsPerStage = kLoadsA + kLoadsB;
static_assert(kLoadsPerStage * (kStages - 1) <= 63, "vmcnt range");

struct LargeArgs {
  const void* A;            // grad_y [M, N]
  const void* B;            // weight [G, K, N]
  const WsHeader* hdr;
  const MTile* tiles;
  const int32_t* chunk_row0;
  float* ring;
  int64_t N, K;
  int32_t chunk, tc, n_col_tiles;
};

__device__ __forceinline__ int slot_of(int r, int c) { return c ^ ((r >> 2) & 3); }

__device__ __forceinline__ void dma16(const void* src, uint32_t m0) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off"
               :: "s"(m0), "v"(src) : "memory", "m0");
}

// Wait until at most `n` of this wave's direct-to-LDS loads are outstanding and
// its LDS reads are done, then barrier the workgroup.  The wait is the
// builtin (the compiler's wait insertion then knows the LDS reads are done);
// the empty asm statements keep memory accesses from moving across.
template <int N>
__device__ __forceinline__ void wait_then_barrier() {
  // s_waitcnt immediate: vmcnt[3:0] in bits 3:0, expcnt 6:4 (7 = no wait),
  // lgkmcnt 11:8 (0), vmcnt[5:4] in bits 15:14
  constexpr int kImm = (N & 15) | (7 << 4) | ((N >> 4) << 14);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(kImm);
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ void wait_stages_then_barrier(int stages_outstanding) {
  switch (stages_outstanding) {
    case 0: wait_then_barrier<0>(); break;
    case 1: wait_then_barrier<kLoadsPerStage>(); break;
    case 2: wait_then_barrier<2 * kLoadsPerStage>(); break;
    default: wait_then_barrier<3 * kLoadsPerStage>(); break;
  }
}

template <class T>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void produce_large_kernel(LargeArgs a) {
  using E = typename T::elem;
  __shared__ u32x4_t lds[kStages * kStageSlots];

  if (a.hdr->err != kNoError) return;
  int slot, ct;
  if (!raster<8, 4>(blockIdx.x, a.tc, a.n_col_tiles, slot, ct)) return;
  const int64_t tile_idx = static_cast<int64_t>(a.chunk) * a.tc + slot;
  if (tile_idx >= a.hdr->n_tiles) return;
  const MTile tile = a.tiles[tile_idx];
  if (tile.rows <= 0) return;
  const int rows = tile.rows;
  const int64_t col0 = static_cast<int64_t>(ct) * kBN;
  const int cols = static_cast<int>(min<int64_t>(kBN, a.K - col0));
  const int64_t ring_row0 = static_cast<int64_t>(tile.row0) - a.chunk_row0[a.chunk];
  const int64_t N = a.N;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave % kWM, wn = wave / kWM;
  const int lr = lane & 31, lh = lane >> 5;

  // Direct-to-LDS load j of this wave covers slots (j*4 + wave)*64 + lane of a
  // region: row (j*4 + wave)*16 + lane/4, slot lane%4, whose logical chunk
  // (lane%4) ^ ((lane/16)%4) is the same for every j.
  const int dma_c = (lane & 3) ^ ((lane >> 4) & 3);
  const E* pa[kLoadsA];
  const E* pb[kLoadsB];
  bool va[kLoadsA], vb[kLoadsB];
  const E* Ab = static_cast<const E*>(a.A) + static_cast<int64_t>(tile.row0) * N + dma_c * 8;
  const E* Bb = static_cast<const E*>(a.B) + (static_cast<int64_t>(tile.g) * a.K + col0) * N + dma_c * 8;
#pragma unroll
  for (int j = 0; j < kLoadsA; ++j) {
    const int r = (j * kWaves + wave) * 16 + (lane >> 2);
    va[j] = r < rows;
    pa[j] = Ab + static_cast<int64_t>(va[j] ? r : 0) * N;
  }
#pragma unroll
  for (int j = 0; j < kLoadsB; ++j) {
    const int r = (j * kWaves + wave) * 16 + (lane >> 2);
    vb[j] = r < cols;
    pb[j] = Bb + static_cast<int64_t>(vb[j] ? r : 0) * N;
  }
  const void* zero = a.hdr->zero;
  const uint32_t lds0 = __builtin_amdgcn_readfirstlane(lds_offset(lds));

  auto issue = [&](int kt) {
    const uint32_t base = lds0 + static_cast<uint32_t>((kt % kStages) * kStageSlots * 16);
    const int64_t n0 = static_cast<int64_t>(kt) * kBK;
    const bool in_n = n0 + dma_c * 8 < N;
#pragma unroll
    for (int j = 0; j < kLoadsA; ++j)
      dma16(va[j] && in_n ? static_cast<const void*>(pa[j] + n0) : zero,
            base + static_cast<uint32_t>((j * kWaves + wave) * 64 * 16));
#pragma unroll
    for (int j = 0; j < kLoadsB; ++j)
      dma16(vb[j] && in_n ? static_cast<const void*>(pb[j] + n0) : zero,
            base + static_cast<uint32_t>((kSlotsA + (j * kWaves + wave) * 64) * 16));
  };

  f32x16_t acc[kFM][kFN];
#pragma unroll
  for (int i = 0; i < kFM; ++i)
#pragma unroll
    for (int j = 0; j < kFN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  // fragment rows start at multiples of 32, so (row >> 2) & 3 == (lr >> 2) & 3
  auto load_frags = [&](int kt, int q, u32x4_t (&fa)[kFM], u32x4_t (&fb)[kFN]) {
    const u32x4_t* st = lds + (kt % kStages) * kStageSlots;
    const int sl = slot_of(lr, 2 * q + lh);
#pragma unroll
    for (int i = 0; i < kFM; ++i) fa[i] = st[(wm * kWTM + i * 32 + lr) * kRowChunks + sl];
#pragma unroll
    for (int j = 0; j < kFN; ++j) fb[j] = st[kSlotsA + (wn * kWTN + j * 32 + lr) * kRowChunks + sl];
  };
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
  wait_stages_then_barrier(min(kStages, nk) - 1);
  u32x4_t fa0[kFM], fb0[kFN], fa1[kFM], fb1[kFN];
  load_frags(0, 0, fa0, fb0);
  int kt = 0;
  // Steady state, free of branches so the compiler's LDS wait counts stay
  // exact across iterations: stage kt+1 is complete after the barrier, and
  // stages kt+2, kt+3 may still be landing.
  for (; kt + kStages < nk; ++kt) {
    load_frags(kt, 1, fa1, fb1);
    mfmas(fa0, fb0);
    wait_then_barrier<(kStages - 2) * kLoadsPerStage>();
    issue(kt + kStages);            // refills stage kt's buffer
    load_frags(kt + 1, 0, fa0, fb0);
    mfmas(fa1, fb1);
  }
  // Drain: the last kStages stages, nothing left to issue.
  for (; kt < nk; ++kt) {
    load_frags(kt, 1, fa1, fb1);
    mfmas(fa0, fb0);
    if (kt + 1 < nk) {
      wait_stages_then_barrier(nk - 2 - kt);
      load_frags(kt + 1, 0, fa0, fb0);
    }
    mfmas(fa1, fb1);
  }

  // Epilogue: accumulator v of lane (lr, lh) is row 8*(v/4) + 4*lh + v%4,
  // column lr of its 32x32 block.
  float* __restrict__ out = a.ring + ring_row0 * a.K + col0;
#pragma unroll
  for (int i = 0; i < kFM; ++i) {
#pragma unroll
    for (int j = 0; j < kFN; ++j) {
      const int n = wn * kWTN + j * 32 + lr;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int m = wm * kWTM + i * 32 + 8 * (v >> 2) + 4 * lh + (v & 3);
        if (m < rows && n < cols) out[static_cast<int64_t>(m) * a.K + n] = acc[i][j][v];
      }
    }
  }
}

}  // namespace

bool produce_uses_dma(const Plan& p, bool aligned) {
  return aligned && p.regime == kLarge && p.dtype != PGG_F32;
}

hipError_t launch_produce_dma(const Plan& p, int chunk, const void* grad_y, const void* weight,
                              const WsView& w, hipStream_t s) {
  LargeArgs a;
  a.A = grad_y;
  a.B = weight;
  a.hdr = w.hdr;
  a.tiles = w.tiles;
  a.chunk_row0 = w.chunk_row0;
  a.ring = w.ring;
  a.N = p.N;
  a.K = p.K;
  a.chunk = chunk;
  a.tc = p.tc;
  a.n_col_tiles = p.n_col_tiles;
  unsigned tiles = static_cast<unsigned>(p.tc) * static_cast<unsigned>(p.n_col_tiles);
  tiles = (tiles + 255u) / 256u * 256u;   // whole rounds of 8 super-blocks of 32 tiles
  if (p.dtype == PGG_BF16)
    hipLaunchKernelGGL(produce_large_kernel<TBf16>, dim3(tiles), dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL(produce_large_kernel<TF16>, dim3(tiles), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace pgg
