// Producer: the grouped-matmul gradient of the fused op,
//
//   C[i, k] = sum_n d_y[i, n] * W[g(i), k, n]        (fp32 accumulate)
//
// (MoeInitRoutingGroupedMatmulGrad design page, §数学定义和公式 Step 1; the
// page's cube output type is fp32 whatever the input type, §2.6.2), for the
// m-tiles of one chunk, written into that chunk's fp32 ring rows.  This file
// holds the general register-staged tile: 64x128 or 128x128 for fp32 inputs
// with a middling number of rows per expert, 256x256 for rows that are not
// 16-byte aligned.  Aligned
// rows with many rows per expert take the direct-to-LDS 256x256 tile (every
// input type), and 16-bit inputs with few rows per expert the weight sweep.
//
// Both operands are contiguous along the reduction index n: a d_y row and a
// W[g] row (one output column) are each a run of N elements.  That is the
// layout MFMA operands want: every lane of a 32x32 MFMA takes a 16-byte run
// of one row, so tiles are staged in LDS with rows of 16-byte chunks and no
// transpose.
//
// Workgroup = one output tile (BM expanded rows of one expert x BN output
// columns).  Waves are laid out WM x WN over the tile; each wave owns a
// (BM/WM) x (BN/WN) block of 32x32 MFMA accumulators.  The reduction runs in
// stages of 8 chunks per row (64 elements for 16-bit types, 32 for fp32),
// double-buffered in LDS with a register prefetch of the next stage.  LDS
// rows are 128 bytes, with chunks XOR-swizzled (lds_slot) so fragment reads
// are free of bank conflicts.
//
// Row tails (experts whose last tile is partial), column tails (K not a
// multiple of BN) and reduction tails (N not a multiple of the stage) are
// zero-filled on load and masked on store.  ALIGNED=false handles rows that
// are not 16-byte aligned (N*elem_size % 16 != 0 or unaligned base pointers)
// with element loads.
#include "pgg_device.h"

namespace pgg {

namespace {

struct GemmArgs {
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

// Physical 16-byte slot of chunk c of LDS row r (rows of 8 chunks).  A
// wave's 128-bit LDS reads are served 16 lanes at a time over 64 four-byte
// banks (256 bytes), and a fragment read puts 16 consecutive rows, same
// logical chunk, in those 16 lanes.  Row parity picks the bank half, and
// XOR-ing the chunk with (r >> 1) & 7 gives the 8 rows of each parity 8
// different slots.
__device__ __forceinline__ int lds_slot(int r, int c) { return c ^ ((r >> 1) & 7); }

// Waves per SIMD each tile is built for: the 256x256 tile holds 256
// accumulator registers per lane (one wave per SIMD); the fp32 tile two.
template <int BM, int BN>
constexpr int waves_per_eu() { return BM * BN >= 256 * 256 ? 1 : 2; }

template <class T, int BM, int BN, int WM, int WN, bool ALIGNED>
__global__ __launch_bounds__(WM * WN * 64)
__attribute__((amdgpu_waves_per_eu(waves_per_eu<BM, BN>(), waves_per_eu<BM, BN>())))
void produce_kernel(GemmArgs a) {
  using E = typename T::elem;
  constexpr int NT = WM * WN * 64;
  constexpr int EPC = T::kPerChunk;
  constexpr int kChunks = 8;    // 16-byte chunks per LDS row (one stage of the reduction)
  constexpr int BK = kChunks * EPC;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int FM = WTM / 32, FN = WTN / 32;
  constexpr int A_CHUNKS = BM * kChunks, B_CHUNKS = BN * kChunks;
  constexpr int A_PER_T = A_CHUNKS / NT, B_PER_T = B_CHUNKS / NT;
  static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile must hold whole 32x32 blocks");
  static_assert(A_CHUNKS % NT == 0 && B_CHUNKS % NT == 0, "stage must split evenly");

  __shared__ u32x4_t lds[2][A_CHUNKS + B_CHUNKS];

  if (a.hdr->err != kNoError) return;
  int slot, ct;
  if (!raster<8, 4>(blockIdx.x, a.tc, a.n_col_tiles, slot, ct)) return;
  const int64_t tile_idx = static_cast<int64_t>(a.chunk) * a.tc + slot;
  if (tile_idx >= a.hdr->n_tiles) return;
  const MTile tile = a.tiles[tile_idx];
  if (tile.rows <= 0) return;
  const int rows = tile.rows;
  const int64_t col0 = a.k_lo + static_cast<int64_t>(ct) * BN;
  const int cols = static_cast<int>(min<int64_t>(BN, a.k_hi - col0));
  if (cols <= 0) return;
  const int64_t ring_row0 = static_cast<int64_t>(tile.row0) - a.chunk_row0[a.chunk];
  const int64_t N = a.N;

  const E* __restrict__ Ab = static_cast<const E*>(a.A) + static_cast<int64_t>(tile.row0) * N;
  const E* __restrict__ Bb =
      static_cast<const E*>(a.B) + (static_cast<int64_t>(tile.g) * a.K + col0) * N;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave % WM;
  const int wn = wave / WM;
  const int lr = lane & 31;
  const int lh = lane >> 5;

  // Per-thread staging slots: chunk id q -> (row q / 8, chunk q % 8).
  u32x4_t ra0[A_PER_T], rb0[B_PER_T];
  auto load_stage = [&](int kt, auto& ra, auto& rb) {
    const int64_t n0 = static_cast<int64_t>(kt) * BK;
#pragma unroll
    for (int s = 0; s < A_PER_T; ++s) {
      const int q = tid + s * NT;
      const int r = q / kChunks, c = q % kChunks;
      ra[s] = load_chunk<T, ALIGNED>(Ab + static_cast<int64_t>(r) * N, r < rows, n0 + c * EPC, N);
    }
#pragma unroll
    for (int s = 0; s < B_PER_T; ++s) {
      const int q = tid + s * NT;
      const int r = q / kChunks, c = q % kChunks;
      rb[s] = load_chunk<T, ALIGNED>(Bb + static_cast<int64_t>(r) * N, r < cols, n0 + c * EPC, N);
    }
  };
  auto store_stage = [&](int buf, const auto& ra, const auto& rb) {
#pragma unroll
    for (int s = 0; s < A_PER_T; ++s) {
      const int q = tid + s * NT;
      const int r = q / kChunks, c = q % kChunks;
      lds[buf][r * kChunks + lds_slot(r, c)] = ra[s];
    }
#pragma unroll
    for (int s = 0; s < B_PER_T; ++s) {
      const int q = tid + s * NT;
      const int r = q / kChunks, c = q % kChunks;
      lds[buf][A_CHUNKS + r * kChunks + lds_slot(r, c)] = rb[s];
    }
  };

  f32x16_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  // One stage: kChunks/2 chunk pairs.  Fragments are double-buffered in
  // registers so the LDS reads of pair q+1 are in flight while the MFMAs of
  // pair q run.
  auto compute = [&](int buf) {
    const u32x4_t* As = lds[buf];
    const u32x4_t* Bs = lds[buf] + A_CHUNKS;
    u32x4_t fa[2][FM], fb[2][FN];
    auto load_frags = [&](int q, u32x4_t (&xa)[FM], u32x4_t (&xb)[FN]) {
      const int sw = lds_slot(lr, 2 * q + lh);   // fragment rows start at multiples of 32
#pragma unroll
      for (int i = 0; i < FM; ++i) xa[i] = As[(wm * WTM + i * 32 + lr) * kChunks + sw];
#pragma unroll
      for (int j = 0; j < FN; ++j) xb[j] = Bs[(wn * WTN + j * 32 + lr) * kChunks + sw];
    };
    load_frags(0, fa[0], fb[0]);
#pragma unroll
    for (int q = 0; q < kChunks / 2; ++q) {
      // Issue the next pair's LDS reads, then this pair's MFMAs; the
      // scheduling fences keep the compiler from sinking each read down to
      // its first use, which would stall the MFMA pipe on LDS latency.
      if (q + 1 < kChunks / 2) load_frags(q + 1, fa[(q + 1) & 1], fb[(q + 1) & 1]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) mma<T>(acc[i][j], fa[q & 1][i], fb[q & 1][j]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // LDS buffer b holds stage kt when kt % 2 == b.
  const int nk = static_cast<int>((N + BK - 1) / BK);
  load_stage(0, ra0, rb0);
  store_stage(0, ra0, rb0);
  // stage kt+1 is loaded into registers while stage kt is multiplied
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) load_stage(kt + 1, ra0, rb0);
    compute(buf);
    if (kt + 1 < nk) store_stage(buf ^ 1, ra0, rb0);
    __syncthreads();
  }

  // Epilogue: accumulator v of lane (lr, lh) is row 8*(v/4) + 4*lh + v%4,
  // column lr of its 32x32 block.
  float* __restrict__ out = a.ring + ring_row0 * a.ldc + (col0 - a.k_lo);
#pragma unroll
  for (int i = 0; i < FM; ++i) {
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int n = wn * WTN + j * 32 + lr;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int m = wm * WTM + i * 32 + 8 * (v >> 2) + 4 * lh + (v & 3);
        if (m < rows && n < cols) out[static_cast<int64_t>(m) * a.ldc + n] = acc[i][j][v];
      }
    }
  }
}

template <class T, int BM, int BN, int WM, int WN>
hipError_t launch_cfg(const Plan& p, const GemmArgs& args, bool aligned, hipStream_t s) {
  unsigned tiles = static_cast<unsigned>(p.tc) * static_cast<unsigned>(p.n_col_tiles);
  tiles = (tiles + 255u) / 256u * 256u;   // whole rounds of 8 super-blocks
  const dim3 grid(tiles);
  const dim3 block(WM * WN * 64);
  if (aligned)
    hipLaunchKernelGGL((produce_kernel<T, BM, BN, WM, WN, true>), grid, block, 0, s, args);
  else
    hipLaunchKernelGGL((produce_kernel<T, BM, BN, WM, WN, false>), grid, block, 0, s, args);
  return hipGetLastError();
}

template <class T>
hipError_t launch_typed(const Plan& p, const GemmArgs& args, bool aligned, hipStream_t s) {
  switch (p.regime) {
    case kLarge:   // rows that are not 16-byte aligned, or too short a reduction
      return p.bm == 128 ? launch_cfg<T, 128, 256, 2, 2>(p, args, aligned, s)
                         : launch_cfg<T, 256, 256, 2, 2>(p, args, aligned, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

const char* produce_kernel_name(const Plan& p) {
  if (p.regime == kStream) return "produce_stream";
  if (p.dtype == PGG_F32) return "produce_f32";
  switch (p.regime) {
    case kLarge: return "produce_large";
    case kStream: return "produce_stream";
    default: return "produce_f32";
  }
}

hipError_t launch_produce(const Plan& p, int chunk, int panel, const void* grad_y,
                          const void* weight, bool aligned, const WsView& w, hipStream_t s) {
  if (p.regime == kStream) {
    if (panel != 0 || p.n_panels != 1) return hipErrorInvalidValue;
    return launch_produce_sweep(p, chunk, grad_y, weight, aligned, w, s);
  }
  if (produce_uses_dma(p, aligned))
    return launch_produce_dma(p, chunk, panel, grad_y, weight, w, s);
  GemmArgs args;
  args.A = grad_y;
  args.B = weight;
  args.hdr = w.hdr;
  args.tiles = w.tiles;
  args.chunk_row0 = w.chunk_row0;
  args.ring = w.ring;
  args.N = p.N;
  args.K = p.K;
  panel_range(p, panel, &args.k_lo, &args.k_hi);
  args.ldc = p.panel_cols;
  args.chunk = chunk;
  args.tc = p.tc;
  args.n_col_tiles = p.n_col_tiles;
  switch (p.dtype) {
    case PGG_BF16: return launch_typed<TBf16>(p, args, aligned, s);
    case PGG_F16: return launch_typed<TF16>(p, args, aligned, s);
    default:
      if (p.regime == kLarge) return launch_cfg<TF32, 256, 256, 2, 2>(p, args, aligned, s);
      return p.bm == 64 ? launch_cfg<TF32, 64, 128, 2, 2>(p, args, aligned, s)
                        : launch_cfg<TF32, 128, 128, 2, 2>(p, args, aligned, s);
  }
}

}  // namespace pgg
