// Weight gradient of the layer (MoeInitRoutingGroupedMatmulGrad design page,
// §1.2: the operator d_weight is left to computes expanded_x^T · d_y per
// expert), with the permute fused into the operand load:
//
//   dW[g, k, n] = sum over expert g's expanded rows i of x[p(i) / topK, k] * d_y[i, n]
//
// fp32 accumulation, dW written as fp32 [G, K, N]; an expert without rows
// gets zeros.  Each workgroup owns one output tile (expert g, BM values of k,
// BN values of n) and reduces over all of g's rows in a fixed order, so the
// result does not depend on timing.
//
// The reduction index i is the row index of both sources, so both operand
// stages hold rows of i: BK rows of the tile's k columns of x (gathered: row
// i is token ori[i] / topK) and BK rows of its n columns of d_y, 512 bytes
// per row, 64-byte segments XOR-swizzled by row.  MFMA operands want 8 (16-bit)
// or 4 (fp32) consecutive reduction indices of one column per lane, which is
// a transposed read of these stages: ds_read_b64_tr_b16 (in each 16-lane
// group, lane i receives element i % 4 of the 8-byte chunks addressed by
// lanes 4j + i / 4, so lanes addressing rows r0 + s / 4, columns c0 + 4 (s % 4)
// give lane i column c0 + i at rows r0 .. r0+3), or four 4-byte reads for
// fp32.  Stages are double-buffered in LDS with a register prefetch of the
// next stage.  Row tails (the expert's last stage), k and n tails are
// zero-filled on load and masked on store; ALIGNED=false handles rows that
// are not 16-byte aligned with element loads.  Aligned 16-bit rows with many
// rows per expert take the direct-to-LDS tile of dw_large.hip instead.
#include "pgg_device.h"

namespace pgg {

namespace {

typedef __fp16 h16x4_t __attribute__((__vector_size__(4 * sizeof(__fp16))));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));

struct DwArgs {
  const void* X;            // x [batch, K]
  const void* DY;           // d_y [M, N]
  const WsHeader* hdr;
  const int64_t* offsets;   // [G + 1] expert row ranges
  const int32_t* ori;       // expanded row -> original position
  float* dw;                // [G, K, N]
  int64_t K, N, topk;
  int32_t n_kb, n_slots, n_col_tiles;   // k blocks per expert, G * n_kb, n blocks
  int32_t write_order;      // 1: few rows per expert, the call is its grad_w writes
};

// byte offset of byte b of stage row r (rows of 512 bytes)
template <class T>
__device__ __forceinline__ uint32_t st_off(int r, int b) {
  const int swz = T::kPerChunk == 8 ? (r & 3) : (((r >> 2) & 1) << 1);
  return static_cast<uint32_t>(r * 512 + ((((b >> 6) ^ swz)) << 6) + (b & 63));
}

template <int BM, int BN>
constexpr int dw_waves_per_eu() { return BM * BN >= 256 * 256 ? 1 : 2; }

template <class T, int BM, int BN, int WM, int WN, bool ALIGNED>
__global__ __launch_bounds__(WM * WN * 64)
__attribute__((amdgpu_waves_per_eu(dw_waves_per_eu<BM, BN>(), dw_waves_per_eu<BM, BN>())))
void dw_kernel(DwArgs a) {
  using E = typename T::elem;
  constexpr int NT = WM * WN * 64;
  constexpr int EPC = T::kPerChunk;
  constexpr int BK = 8 * EPC;                    // reduction rows per stage
  constexpr int kRowChunks = 512 / 16;           // chunks per stage row
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int FM = WTM / 32, FN = WTN / 32;
  constexpr int CHUNKS = BK * kRowChunks;        // per operand and stage
  constexpr int PER_T = CHUNKS / NT;
  static_assert(BM * sizeof(E) == 512 && BN * sizeof(E) == 512, "stage rows are 512 bytes");
  static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile must hold whole 32x32 blocks");
  static_assert(CHUNKS % NT == 0, "stage must split evenly");

  __shared__ u32x4_t lds[2][2 * CHUNKS];

  if (a.hdr->err != kNoError) return;
  int slot, ct;
  // Tile order.  With many rows per expert, 8 k-blocks x 4 n-blocks per XCD
  // round share their operand rows in L2.  With few, the kernel is its grad_w
  // stores, and 2 k-blocks x 16 n-blocks per round write 16 n-blocks of each
  // row together (whole 16 KB rows at N = 4096): 5.0 -> 5.8 TB/s measured.
  const bool placed = a.write_order ? raster<2, 16>(blockIdx.x, a.n_slots, a.n_col_tiles, slot, ct)
                                    : raster<8, 4>(blockIdx.x, a.n_slots, a.n_col_tiles, slot, ct);
  if (!placed) return;
  const int g = slot / a.n_kb;
  const int64_t k0 = static_cast<int64_t>(slot % a.n_kb) * BM;
  const int64_t n0 = static_cast<int64_t>(ct) * BN;
  const int kvalid = static_cast<int>(min<int64_t>(BM, a.K - k0));
  const int nvalid = static_cast<int>(min<int64_t>(BN, a.N - n0));
  const int64_t r_begin = a.offsets[g], r_end = a.offsets[g + 1];
  const int64_t K = a.K, N = a.N;
  const E* __restrict__ X = static_cast<const E*>(a.X);
  const E* __restrict__ DY = static_cast<const E*>(a.DY);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave % WM;
  const int wn = wave / WM;
  const int lr = lane & 31;
  const int lh = lane >> 5;

  // topK and positions are below M < 2^31: 32-bit unsigned division
  const uint32_t topk32 = static_cast<uint32_t>(a.topk);
  u32x4_t ra[PER_T], rb[PER_T];
  auto load_stage = [&](int kt) {
    const int64_t i0 = r_begin + static_cast<int64_t>(kt) * BK;
#pragma unroll
    for (int s = 0; s < PER_T; ++s) {
      const int q = tid + s * NT;
      const int r = q / kRowChunks, c = q % kRowChunks;
      const int64_t i = i0 + r;
      const bool ok = i < r_end;
      const int64_t tok = ok ? static_cast<uint32_t>(a.ori[i]) / topk32 : 0;
      ra[s] = load_chunk<T, ALIGNED>(X + tok * K, ok, k0 + c * EPC, K);
      rb[s] = load_chunk<T, ALIGNED>(DY + (ok ? i : 0) * N, ok, n0 + c * EPC, N);
    }
  };
  auto store_stage = [&](int buf) {
    char* abase = reinterpret_cast<char*>(&lds[buf][0]);
    char* bbase = reinterpret_cast<char*>(&lds[buf][CHUNKS]);
#pragma unroll
    for (int s = 0; s < PER_T; ++s) {
      const int q = tid + s * NT;
      const int r = q / kRowChunks, c = q % kRowChunks;
      *reinterpret_cast<u32x4_t*>(abase + st_off<T>(r, c * 16)) = ra[s];
      *reinterpret_cast<u32x4_t*>(bbase + st_off<T>(r, c * 16)) = rb[s];
    }
  };

  // Operand fragment of column `col` of a stage region, chunk pair q: the
  // EPC consecutive reduction rows starting at EPC*(2q + lh).
  auto load_tr = [&](const char* region, int colbase, int q) -> u32x4_t {
    if constexpr (EPC == 8) {
      const int grp = lane >> 4, s = lane & 15;
      const int col = colbase + 16 * (grp & 1) + 4 * (s & 3);
      const int r0 = 8 * (2 * q + (grp >> 1)) + (s >> 2);
      u32x2_t part[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const char* p = region + st_off<T>(r0 + 4 * u, col * 2);
        auto lp = (__attribute__((address_space(3))) h16x4_t*)(
            (__attribute__((address_space(3))) char*)(p));
        part[u] = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4f16(lp));
      }
      return u32x4_t{part[0][0], part[0][1], part[1][0], part[1][1]};
    } else {
      const int col = colbase + lr;
      const int r0 = 4 * (2 * q + lh);
      u32x4_t v;
#pragma unroll
      for (int t = 0; t < 4; ++t)
        v[t] = *reinterpret_cast<const uint32_t*>(region + st_off<T>(r0 + t, col * 4));
      return v;
    }
  };

  f32x16_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  auto compute = [&](int buf) {
    const char* abase = reinterpret_cast<const char*>(&lds[buf][0]);
    const char* bbase = reinterpret_cast<const char*>(&lds[buf][CHUNKS]);
    u32x4_t fa[2][FM], fb[2][FN];
    auto load_frags = [&](int q, u32x4_t (&xa)[FM], u32x4_t (&xb)[FN]) {
#pragma unroll
      for (int i = 0; i < FM; ++i) xa[i] = load_tr(abase, wm * WTM + i * 32, q);
#pragma unroll
      for (int j = 0; j < FN; ++j) xb[j] = load_tr(bbase, wn * WTN + j * 32, q);
    };
    load_frags(0, fa[0], fb[0]);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (q + 1 < 4) load_frags(q + 1, fa[(q + 1) & 1], fb[(q + 1) & 1]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) mma<T>(acc[i][j], fa[q & 1][i], fb[q & 1][j]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  const int nk = static_cast<int>((r_end - r_begin + BK - 1) / BK);
  if (nk > 0) {
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
  }

  // Epilogue: accumulator v of lane (lr, lh) is row 8*(v/4) + 4*lh + v%4
  // (a k), column lr (an n) of its 32x32 block.
  float* __restrict__ out = a.dw + (static_cast<int64_t>(g) * K + k0) * N + n0;
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int n = wn * WTN + j * 32 + lr;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int m = wm * WTM + i * 32 + 8 * (v >> 2) + 4 * lh + (v & 3);
        if (m < kvalid && n < nvalid)
          __builtin_nontemporal_store(acc[i][j][v], out + static_cast<int64_t>(m) * N + n);
      }
    }
}

template <class T, int BM, int BN, int WM, int WN>
hipError_t launch_typed(const Plan& p, DwArgs a, bool aligned, hipStream_t s) {
  a.n_kb = static_cast<int32_t>((a.K + BM - 1) / BM);
  a.n_slots = static_cast<int32_t>(p.G) * a.n_kb;
  a.n_col_tiles = static_cast<int32_t>((a.N + BN - 1) / BN);
  unsigned tiles = static_cast<unsigned>(a.n_slots) * static_cast<unsigned>(a.n_col_tiles);
  tiles = (tiles + 8 * 32 - 1) / (8 * 32) * (8 * 32);   // whole raster rounds
  if (aligned)
    hipLaunchKernelGGL((dw_kernel<T, BM, BN, WM, WN, true>), dim3(tiles), dim3(WM * WN * 64), 0, s, a);
  else
    hipLaunchKernelGGL((dw_kernel<T, BM, BN, WM, WN, false>), dim3(tiles), dim3(WM * WN * 64), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_dw(const Plan& p, const void* x, const void* grad_y, float* dw, bool aligned,
                     const WsView& w, hipStream_t s) {
  DwArgs a{};
  a.X = x;
  a.DY = grad_y;
  a.hdr = w.hdr;
  a.offsets = w.offsets;
  a.ori = w.ori;
  a.dw = dw;
  a.K = p.N;            // the forward plan keeps x's row length (K) in N
  a.N = p.K;            // and the weight's last dimension (N) in K
  a.topk = p.topk;
  a.write_order = p.M <= 64 * p.G ? 1 : 0;   // at most 64 rows per expert on average
  if (p.dtype == PGG_F32) return launch_typed<TF32, 128, 128, 2, 2>(p, a, aligned, s);
  // many rows per expert: the direct-to-LDS tile; with few, every tile is
  // one or two stages and the register-staged tile is as fast
  if (aligned && p.regime == kLarge) return launch_dw_large(p, x, grad_y, dw, w, s);
  if (p.dtype == PGG_BF16) return launch_typed<TBf16, 256, 256, 2, 2>(p, a, aligned, s);
  return launch_typed<TF16, 256, 256, 2, 2>(p, a, aligned, s);
}

const char* dw_kernel_name(const Plan& p) { return p.dtype == PGG_F32 ? "dweight_f32" : "dweight"; }

}  // namespace pgg
