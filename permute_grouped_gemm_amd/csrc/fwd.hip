// Forward of the layer: MoeInitRouting (Permute) followed by GroupedMatmul
// (MoeInitRoutingGroupedMatmulGrad design page, §数学定义和公式, forward
// formulas, and §1.1 steps 1-2):
//
//   y[i, n] = sum_k x[p(i) / topK, k] * W[g(i), k, n]        (fp32 accumulate)
//
// The permuted copy expanded_x is never stored: each tile gathers its rows of
// x straight from the token rows, through the expanded-row -> original-position
// table the index preparation builds (ori[i] = p(i)).
//
// Workgroup = one output tile (BM expanded rows of one expert x BN output
// columns), waves laid out WM x WN, each owning (BM/WM) x (BN/WN) of 32x32
// MFMA accumulators.  The reduction over k runs in stages of BK elements,
// double-buffered in LDS with a register prefetch of the next stage.  With
// few rows per expert the reduction may be split (blockIdx.y = split, kspan
// elements each, a multiple of BK): each split writes an fp32 partial tile
// to the workspace and fwd_reduce_kernel adds the splits in split order, so
// the result does not depend on timing.
//
// Operand layouts.  A gathered x row is contiguous along k, the reduction,
// which is what an MFMA operand wants (every lane takes a run of consecutive
// k of one row): the A region holds BM rows of 8 16-byte chunks, XOR-swizzled
// (lds_slot) as in the backward producer.  W[g] is [K, N] with n contiguous,
// so a k-run of one output column is strided.  The B region keeps the stage
// as loaded, BK rows of k with BN columns each (512 bytes), and the operand is
// read transposed:
// * 16-bit types: ds_read_b64_tr_b16.  In each group of 16 lanes, lane i
//   receives element i % 4 of the 8-byte chunks addressed by lanes 4j + i / 4,
//   j = 0..3.  When lane s of the group addresses row k0 + s / 4, columns
//   n0 + 4 (s % 4) .. + 3, lane i receives column n0 + i at rows k0 .. k0+3;
//   two such reads give a lane the 8 consecutive k of its column.
// * fp32: the MFMA takes one k per lane and step, so four 4-byte reads.
// Rows of the B region are 8 segments of 64 bytes; segment s of row k sits at
// s ^ swz(k), so the rows one read instruction touches land on different
// banks (4 consecutive rows for the transposed read; rows k and k+4 for fp32).
//
// Aligned 16-bit rows with many rows per expert take the direct-to-LDS tile
// of fwd_large.hip instead.
//
// Row tails (an expert's last tile), column tails (N not a multiple of BN)
// and reduction tails (K not a multiple of BK) are zero-filled on load and
// masked on store.  ALIGNED=false handles rows that are not 16-byte aligned
// with element loads.
#include <algorithm>

#include "pgg_device.h"

namespace pgg {

namespace {

typedef __fp16 h16x4_t __attribute__((__vector_size__(4 * sizeof(__fp16))));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));

struct FwdArgs {
  const void* X;            // x [batch, R]
  const void* W;            // weight [G, R, C]
  const WsHeader* hdr;
  const MTile* tiles;
  const int32_t* ori;       // expanded row -> original position
  float* y;                 // [M, C], or the split partials [ksplit, M, C]
  int64_t R, C, topk;       // reduction length (K), output columns (N), topK
  int64_t M, kspan;         // expanded rows; reduction elements per split (blockIdx.y)
  int32_t n_slots, n_col_tiles;
};

// A region: chunk c of row r at slot c ^ ((r >> 1) & 7) (16 consecutive rows,
// same chunk, over 64 banks).
__device__ __forceinline__ int lds_slot(int r, int c) { return c ^ ((r >> 1) & 7); }

// B region: byte offset of element column n of row k (rows of 512 bytes).
template <class T>
__device__ __forceinline__ uint32_t b_offset(int k, int byte_in_row) {
  const int swz = T::kPerChunk == 8 ? (k & 3) : (((k >> 2) & 1) << 1);
  return static_cast<uint32_t>(k * 512 + ((((byte_in_row >> 6) ^ swz)) << 6) + (byte_in_row & 63));
}

template <int BM, int BN>
constexpr int waves_per_eu() { return BM * BN >= 256 * 256 ? 1 : 2; }

template <class T, int BM, int BN, int WM, int WN, bool ALIGNED>
__global__ __launch_bounds__(WM * WN * 64)
__attribute__((amdgpu_waves_per_eu(waves_per_eu<BM, BN>(), waves_per_eu<BM, BN>())))
void fwd_kernel(FwdArgs a) {
  using E = typename T::elem;
  constexpr int NT = WM * WN * 64;
  constexpr int EPC = T::kPerChunk;
  constexpr int kChunks = 8;                     // A chunks per row and stage
  constexpr int BK = kChunks * EPC;              // reduction elements per stage
  constexpr int kRowChunksB = BN * int(sizeof(E)) / 16;   // chunks per B row
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int FM = WTM / 32, FN = WTN / 32;
  constexpr int A_CHUNKS = BM * kChunks, B_CHUNKS = BK * kRowChunksB;
  constexpr int A_PER_T = A_CHUNKS / NT, B_PER_T = B_CHUNKS / NT;
  static_assert(BN * sizeof(E) == 512, "B rows are 512 bytes");
  static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile must hold whole 32x32 blocks");
  static_assert(A_CHUNKS % NT == 0 && B_CHUNKS % NT == 0, "stage must split evenly");

  __shared__ u32x4_t lds[2][A_CHUNKS + B_CHUNKS];

  if (a.hdr->err != kNoError) return;
  int slot, ct;
  if (!raster<8, 4>(blockIdx.x, a.n_slots, a.n_col_tiles, slot, ct)) return;
  if (slot >= a.hdr->n_tiles) return;
  const MTile tile = a.tiles[slot];
  if (tile.rows <= 0) return;
  const int rows = tile.rows;
  const int64_t col0 = static_cast<int64_t>(ct) * BN;
  const int cols = static_cast<int>(min<int64_t>(BN, a.C - col0));
  const int64_t C = a.C;
  // reduction range of this workgroup's split: [kbeg, R)
  const int64_t kbeg = static_cast<int64_t>(blockIdx.y) * a.kspan;
  const int64_t R = min<int64_t>(a.R, kbeg + a.kspan);
  const int64_t RX = a.R;     // x row length

  const E* __restrict__ X = static_cast<const E*>(a.X);
  const E* __restrict__ Wg = static_cast<const E*>(a.W) + static_cast<int64_t>(tile.g) * RX * C;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave % WM;
  const int wn = wave / WM;
  const int lr = lane & 31;
  const int lh = lane >> 5;

  // Gathered A rows of this thread's staging slots: chunk id q -> (row q / 8,
  // chunk q % 8); row r of the tile is token ori[row0 + r] / topK of x.
  // topK and positions are below M < 2^31: 32-bit unsigned division
  const uint32_t topk32 = static_cast<uint32_t>(a.topk);
  const E* arow[A_PER_T];
#pragma unroll
  for (int s = 0; s < A_PER_T; ++s) {
    const int r = (tid + s * NT) / kChunks;
    const int64_t tok = r < rows ? static_cast<uint32_t>(a.ori[tile.row0 + r]) / topk32 : 0;
    arow[s] = X + tok * RX;
  }

  u32x4_t ra[A_PER_T], rb[B_PER_T];
  auto load_stage = [&](int kt) {
    const int64_t k0 = kbeg + static_cast<int64_t>(kt) * BK;
#pragma unroll
    for (int s = 0; s < A_PER_T; ++s) {
      const int q = tid + s * NT;
      const int r = q / kChunks, c = q % kChunks;
      ra[s] = load_chunk<T, ALIGNED>(arow[s], r < rows, k0 + c * EPC, R);
    }
#pragma unroll
    for (int s = 0; s < B_PER_T; ++s) {
      const int q = tid + s * NT;
      const int k = q / kRowChunksB, c = q % kRowChunksB;
      const bool k_ok = k0 + k < R;
      // the weights: non-temporal for few-row tiles (an expert's one m-tile
      // streams its strip of W[g] once); larger tiles share W[g] through L2
      rb[s] = load_chunk<T, ALIGNED, (BM <= 32)>(Wg + (k_ok ? (k0 + k) * C : 0), k_ok,
                                                 col0 + c * EPC, C);
    }
  };
  auto store_stage = [&](int buf) {
#pragma unroll
    for (int s = 0; s < A_PER_T; ++s) {
      const int q = tid + s * NT;
      const int r = q / kChunks, c = q % kChunks;
      lds[buf][r * kChunks + lds_slot(r, c)] = ra[s];
    }
    char* bbase = reinterpret_cast<char*>(&lds[buf][A_CHUNKS]);
#pragma unroll
    for (int s = 0; s < B_PER_T; ++s) {
      const int q = tid + s * NT;
      const int k = q / kRowChunksB, c = q % kRowChunksB;
      *reinterpret_cast<u32x4_t*>(bbase + b_offset<T>(k, c * 16)) = rb[s];
    }
  };

  f32x16_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  // B fragment of column block j, chunk pair q: the 8 (16-bit) or 4 (fp32)
  // consecutive k of column wn*WTN + j*32 + lr starting at k = EPC*(2q + lh).
  auto load_b = [&](int buf, int q, int j) -> u32x4_t {
    const char* bgen = reinterpret_cast<const char*>(&lds[buf][A_CHUNKS]);
    if constexpr (EPC == 8) {
      const int grp = lane >> 4, s = lane & 15;
      const int n = wn * WTN + j * 32 + 16 * (grp & 1) + 4 * (s & 3);
      const int kb = 8 * (2 * q + (grp >> 1)) + (s >> 2);
      u32x2_t part[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const char* p = bgen + b_offset<T>(kb + 4 * u, n * 2);
        auto lp = (__attribute__((address_space(3))) h16x4_t*)(
            (__attribute__((address_space(3))) char*)(p));
        part[u] = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4f16(lp));
      }
      return u32x4_t{part[0][0], part[0][1], part[1][0], part[1][1]};
    } else {
      const int n = wn * WTN + j * 32 + lr;
      const int kb = 4 * (2 * q + lh);
      u32x4_t v;
#pragma unroll
      for (int t = 0; t < 4; ++t)
        v[t] = *reinterpret_cast<const uint32_t*>(bgen + b_offset<T>(kb + t, n * 4));
      return v;
    }
  };

  auto compute = [&](int buf) {
    const u32x4_t* As = lds[buf];
    u32x4_t fa[2][FM], fb[2][FN];
    auto load_frags = [&](int q, u32x4_t (&xa)[FM], u32x4_t (&xb)[FN]) {
      const int sw = lds_slot(lr, 2 * q + lh);   // fragment rows start at multiples of 32
#pragma unroll
      for (int i = 0; i < FM; ++i) xa[i] = As[(wm * WTM + i * 32 + lr) * kChunks + sw];
#pragma unroll
      for (int j = 0; j < FN; ++j) xb[j] = load_b(buf, q, j);
    };
    load_frags(0, fa[0], fb[0]);
#pragma unroll
    for (int q = 0; q < kChunks / 2; ++q) {
      if (q + 1 < kChunks / 2) load_frags(q + 1, fa[(q + 1) & 1], fb[(q + 1) & 1]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) mma<T>(acc[i][j], fa[q & 1][i], fb[q & 1][j]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  const int nk = static_cast<int>((R - kbeg + BK - 1) / BK);
  load_stage(0);
  store_stage(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) load_stage(kt + 1);
    compute(buf);
    if (kt + 1 < nk) store_stage(buf ^ 1);
    __syncthreads();
  }

  // Epilogue: accumulator v of lane (lr, lh) is row 8*(v/4) + 4*lh + v%4,
  // column lr of its 32x32 block.
  float* __restrict__ out =
      a.y + (static_cast<int64_t>(blockIdx.y) * a.M + tile.row0) * C + col0;
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int n = wn * WTN + j * 32 + lr;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int m = wm * WTM + i * 32 + 8 * (v >> 2) + 4 * lh + (v & 3);
        if (m < rows && n < cols) out[static_cast<int64_t>(m) * C + n] = acc[i][j][v];
      }
    }
}

template <class T, int BM, int BN, int WM, int WN>
hipError_t launch_typed(const Plan& p, const FwdArgs& a, bool aligned, hipStream_t s) {
  unsigned tiles = static_cast<unsigned>(a.n_slots) * static_cast<unsigned>(a.n_col_tiles);
  tiles = (tiles + 8 * 32 - 1) / (8 * 32) * (8 * 32);   // whole raster rounds
  if (tiles == 0) return hipSuccess;
  const dim3 grid(tiles, static_cast<unsigned>(p.ksplit));
  if (aligned)
    hipLaunchKernelGGL((fwd_kernel<T, BM, BN, WM, WN, true>), grid, dim3(WM * WN * 64), 0, s, a);
  else
    hipLaunchKernelGGL((fwd_kernel<T, BM, BN, WM, WN, false>), grid, dim3(WM * WN * 64), 0, s, a);
  return hipGetLastError();
}

// y[e] = part[0][e] + part[1][e] + ... in split order (e over all M x C).
__global__ __launch_bounds__(256) void fwd_reduce_kernel(const WsHeader* hdr, const float* part,
                                                         float* y, int64_t n, int32_t ksplit) {
  if (hdr->err != kNoError) return;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t e = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; e < n; e += stride) {
    float acc = part[e];
    for (int32_t s = 1; s < ksplit; ++s) acc += part[static_cast<int64_t>(s) * n + e];
    y[e] = acc;
  }
}

}  // namespace

hipError_t launch_forward(const Plan& p, const void* x, const void* weight, float* y, bool aligned,
                          const WsView& w, hipStream_t s) {
  FwdArgs a;
  a.X = x;
  a.W = weight;
  a.hdr = w.hdr;
  a.tiles = w.tiles;
  a.ori = w.ori;
  a.y = p.ksplit > 1 ? w.ring : y;   // split partials go to the workspace
  a.R = p.N;            // the plan keeps the reduction length in N
  a.C = p.K;            // and the output columns in K
  a.topk = p.topk;
  a.M = p.M;
  a.kspan = p.kspan;
  a.n_slots = p.max_tiles;
  a.n_col_tiles = p.n_col_tiles;
  if (p.dtype == PGG_F32) return launch_typed<TF32, 128, 128, 2, 2>(p, a, aligned, s);
  if (p.regime == kStream) {
    if (p.dtype == PGG_BF16) return launch_typed<TBf16, 32, 256, 1, 4>(p, a, aligned, s);
    return launch_typed<TF16, 32, 256, 1, 4>(p, a, aligned, s);
  }
  if (aligned) return launch_forward_large(p, x, weight, y, w, s);
  if (p.dtype == PGG_BF16) return launch_typed<TBf16, 256, 256, 2, 2>(p, a, aligned, s);
  return launch_typed<TF16, 256, 256, 2, 2>(p, a, aligned, s);
}

hipError_t launch_forward_reduce(const Plan& p, const WsView& w, float* y, hipStream_t s) {
  const int64_t n = p.M * p.K;
  const int64_t blocks = std::min<int64_t>((n + 255) / 256, 2048);
  hipLaunchKernelGGL(fwd_reduce_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, w.hdr,
                     w.ring, y, n, p.ksplit);
  return hipGetLastError();
}

const char* forward_kernel_name(const Plan& p) {
  if (p.dtype == PGG_F32) return "forward_f32";
  return p.regime == kStream ? "forward_stream" : "forward_large";
}

}  // namespace pgg
