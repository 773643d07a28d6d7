// Producer: the grouped-matmul gradient of the fused op,
//
//   C[i, k] = sum_n d_y[i, n] * W[g(i), k, n]        (fp32 accumulate)
//
// (MoeInitRoutingGroupedMatmulGrad design page, §数学定义和公式 Step 1; the
// page's cube output type is fp32 whatever the input type, §2.6.2), for the
// m-tiles of one chunk, written into that chunk's fp32 ring rows.
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
// rows are 128 bytes; chunk c of row r is stored at slot c ^ (r & 7) so the
// 16-byte fragment reads of a wave spread over all banks.
//
// Row tails (experts whose last tile is partial), column tails (K not a
// multiple of BN) and reduction tails (N not a multiple of the stage) are
// zero-filled on load and masked on store.  ALIGNED=false handles rows that
// are not 16-byte aligned (N*elem_size % 16 != 0 or unaligned base pointers)
// with element loads.
#include "pgg_internal.h"

namespace pgg {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

struct TBf16 { using elem = uint16_t; static constexpr int kPerChunk = 8; };
struct TF16 { using elem = uint16_t; static constexpr int kPerChunk = 8; };
struct TF32 { using elem = float; static constexpr int kPerChunk = 4; };

constexpr int kChunks = 8;  // 16-byte chunks per LDS row (one stage of the reduction)

struct GemmArgs {
  const void* A;            // grad_y [M, N]
  const void* B;            // weight [G, K, N]
  const WsHeader* hdr;
  const MTile* tiles;
  const int32_t* chunk_row0;
  float* ring;              // [ring_rows, K]
  int64_t N, K;
  int32_t chunk, tc, n_col_tiles;
};

// Accumulate one chunk pair: lane half h holds chunk 2q+h of its row for both
// operands, so the MFMA's reduction slots pair equal reduction indices.
template <class T>
__device__ __forceinline__ void mma(f32x16_t& acc, u32x4_t a, u32x4_t b);

template <>
__device__ __forceinline__ void mma<TBf16>(f32x16_t& acc, u32x4_t a, u32x4_t b) {
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                __builtin_bit_cast(bf16x8_t, b), acc, 0, 0, 0);
}

template <>
__device__ __forceinline__ void mma<TF16>(f32x16_t& acc, u32x4_t a, u32x4_t b) {
  acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a),
                                               __builtin_bit_cast(f16x8_t, b), acc, 0, 0, 0);
}

template <>
__device__ __forceinline__ void mma<TF32>(f32x16_t& acc, u32x4_t a, u32x4_t b) {
  const f32x4_t fa = __builtin_bit_cast(f32x4_t, a);
  const f32x4_t fb = __builtin_bit_cast(f32x4_t, b);
  acc = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[0], fb[0], acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[1], fb[1], acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[2], fb[2], acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[3], fb[3], acc, 0, 0, 0);
}

// Load one 16-byte chunk of a row (elements [n, n + kPerChunk)), zero outside
// the row or past N.
template <class T, bool ALIGNED>
__device__ __forceinline__ u32x4_t load_chunk(const typename T::elem* __restrict__ row, bool row_ok,
                                              int64_t n, int64_t N) {
  using E = typename T::elem;
  constexpr int EPC = T::kPerChunk;
  u32x4_t v = {0u, 0u, 0u, 0u};
  if (!row_ok || n >= N) return v;
  if constexpr (ALIGNED) {
    v = *reinterpret_cast<const u32x4_t*>(row + n);
  } else {
    E e[EPC];
#pragma unroll
    for (int t = 0; t < EPC; ++t) e[t] = (n + t < N) ? row[n + t] : E(0);
    __builtin_memcpy(&v, e, sizeof(v));
  }
  return v;
}

template <class T, int BM, int BN, int WM, int WN, bool ALIGNED>
__global__ __launch_bounds__(WM * WN * 64) void produce_kernel(GemmArgs a) {
  using E = typename T::elem;
  constexpr int NT = WM * WN * 64;
  constexpr int EPC = T::kPerChunk;
  constexpr int BK = kChunks * EPC;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int FM = WTM / 32, FN = WTN / 32;
  constexpr int A_CHUNKS = BM * kChunks, B_CHUNKS = BN * kChunks;
  constexpr int A_PER_T = A_CHUNKS / NT, B_PER_T = B_CHUNKS / NT;
  static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile must hold whole 32x32 blocks");
  static_assert(A_CHUNKS % NT == 0 && B_CHUNKS % NT == 0, "stage must split evenly");

  __shared__ u32x4_t lds[2][A_CHUNKS + B_CHUNKS];

  if (a.hdr->err != kNoError) return;
  const int slot = blockIdx.x / a.n_col_tiles;
  const int ct = blockIdx.x - slot * a.n_col_tiles;
  const int64_t tile_idx = static_cast<int64_t>(a.chunk) * a.tc + slot;
  if (tile_idx >= a.hdr->n_tiles) return;
  const MTile tile = a.tiles[tile_idx];
  if (tile.rows <= 0) return;
  const int rows = tile.rows;
  const int64_t col0 = static_cast<int64_t>(ct) * BN;
  const int cols = static_cast<int>(min<int64_t>(BN, a.K - col0));
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
  u32x4_t ra[A_PER_T], rb[B_PER_T];
  auto load_stage = [&](int kt) {
    const int64_t n0 = static_cast<int64_t>(kt) * BK;
#pragma unroll
    for (int s = 0; s < A_PER_T; ++s) {
      const int q = tid + s * NT;
      const int r = q >> 3, c = q & 7;
      ra[s] = load_chunk<T, ALIGNED>(Ab + static_cast<int64_t>(r) * N, r < rows, n0 + c * EPC, N);
    }
#pragma unroll
    for (int s = 0; s < B_PER_T; ++s) {
      const int q = tid + s * NT;
      const int r = q >> 3, c = q & 7;
      rb[s] = load_chunk<T, ALIGNED>(Bb + static_cast<int64_t>(r) * N, r < cols, n0 + c * EPC, N);
    }
  };
  auto store_stage = [&](int buf) {
#pragma unroll
    for (int s = 0; s < A_PER_T; ++s) {
      const int q = tid + s * NT;
      const int r = q >> 3, c = q & 7;
      lds[buf][r * kChunks + (c ^ (r & 7))] = ra[s];
    }
#pragma unroll
    for (int s = 0; s < B_PER_T; ++s) {
      const int q = tid + s * NT;
      const int r = q >> 3, c = q & 7;
      lds[buf][A_CHUNKS + r * kChunks + (c ^ (r & 7))] = rb[s];
    }
  };

  f32x16_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  const int nk = static_cast<int>((N + BK - 1) / BK);
  load_stage(0);
  store_stage(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) load_stage(kt + 1);
    const u32x4_t* As = lds[buf];
    const u32x4_t* Bs = lds[buf] + A_CHUNKS;
#pragma unroll
    for (int q = 0; q < kChunks / 2; ++q) {
      const int c = 2 * q + lh;
      const int sw = c ^ (lr & 7);   // rows of a fragment start at multiples of 32
      u32x4_t fa[FM], fb[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) fa[i] = As[(wm * WTM + i * 32 + lr) * kChunks + sw];
#pragma unroll
      for (int j = 0; j < FN; ++j) fb[j] = Bs[(wn * WTN + j * 32 + lr) * kChunks + sw];
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) mma<T>(acc[i][j], fa[i], fb[j]);
    }
    if (kt + 1 < nk) store_stage(buf ^ 1);
    __syncthreads();
  }

  // Epilogue: accumulator v of lane (lr, lh) is row 8*(v/4) + 4*lh + v%4,
  // column lr of its 32x32 block.
  float* __restrict__ out = a.ring + ring_row0 * a.K + col0;
#pragma unroll
  for (int i = 0; i < FM; ++i) {
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int n = wn * WTN + j * 32 + lr;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int m = wm * WTM + i * 32 + 8 * (v >> 2) + 4 * lh + (v & 3);
        if (m < rows && n < cols) out[static_cast<int64_t>(m) * a.K + n] = acc[i][j][v];
      }
    }
  }
}

template <class T, int BM, int BN, int WM, int WN>
hipError_t launch_cfg(const Plan& p, const GemmArgs& args, bool aligned, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(p.tc) * static_cast<unsigned>(p.n_col_tiles));
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
    case kLarge: return launch_cfg<T, 256, 256, 2, 2>(p, args, aligned, s);
    case kStream: return launch_cfg<T, 32, 128, 1, 4>(p, args, aligned, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

const char* produce_kernel_name(const Plan& p) {
  switch (p.regime) {
    case kLarge: return "produce_large";
    case kStream: return "produce_stream";
    default: return "produce_f32";
  }
}

hipError_t launch_produce(const Plan& p, int chunk, const void* grad_y, const void* weight,
                          bool aligned, const WsView& w, hipStream_t s) {
  GemmArgs args;
  args.A = grad_y;
  args.B = weight;
  args.hdr = w.hdr;
  args.tiles = w.tiles;
  args.chunk_row0 = w.chunk_row0;
  args.ring = w.ring;
  args.N = p.N;
  args.K = p.K;
  args.chunk = chunk;
  args.tc = p.tc;
  args.n_col_tiles = p.n_col_tiles;
  switch (p.dtype) {
    case PGG_BF16: return launch_typed<TBf16>(p, args, aligned, s);
    case PGG_F16: return launch_typed<TF16>(p, args, aligned, s);
    default: return launch_cfg<TF32, 128, 128, 2, 2>(p, args, aligned, s);
  }
}

}  // namespace pgg
