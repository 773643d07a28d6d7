// Producer for many rows per expert (fp16 / bf16 / fp32, 16-byte aligned
// rows): the grouped-matmul gradient C[i, k] = sum_n d_y[i, n] * W[g(i), k, n]
// with fp32 accumulation (MoeInitRoutingGroupedMatmulGrad design page,
// §数学定义和公式 Step 1; fp32 cube output, §2.6.2) on output tiles of 256
// columns and 256 rows (or 128 rows, for 16-bit inputs with about one such
// m-tile per expert), written into the chunk's ring rows.  fp32 inputs run the same tile: a
// 16-byte chunk then holds 4 reduction elements instead of 8, so a stage
// covers 32 of them, and each fragment pair feeds four 32x32x2 fp32 MFMAs
// (sixteen times the MFMA time per stage against the same loads).
//
// Persistent: one workgroup per compute unit walks the launch's tiles
// t = blockIdx.x + j * gridDim.x in the XCD super-block raster (raster<8,4>;
// gridDim.x is a multiple of 8, so all of a workgroup's tiles sit on one XCD,
// and in round j the 32 workgroups of an XCD share 8 d_y slabs and 4 weight
// slabs in its L2).  A workgroup first reads its tiles' table entries into LDS.
// The operand loads then run as one stream of stages across its tiles: the
// next tile's first two stages load during the current tile's last two, so a
// tile starts without waiting for loads, and its predecessor's ring stores
// drain while it multiplies.
//
// Operand staging is direct buffer -> LDS (buffer_load_dwordx4 ... lds: lane
// i's 16 bytes land at M0 + 16 i), stages of 128 bytes per row (whole cache
// lines): two of 64 KiB (256 d_y rows + 256 weight rows) for the 256-row
// tile, three of 48 KiB for the 128-row one, whose barriers then leave the
// stage after next in flight.  The
// loads are issued by inline assembly so the compiler does not serialise them
// with a blanket wait before every LDS read; the waits on their counter are
// explicit (vector memory operations complete in issue order, and these loads
// write no register).
//
// Per stage and wave (2 x 4 waves, two per SIMD, 128 x 64 fp32 accumulators
// each): four chunk pairs of 8 MFMA 32x32x16; the 6 fragments of the next
// pair are read one beside each of the current pair's first 6 MFMAs (a burst
// of reads ahead of the MFMAs measured ~2 % slower), and the next stage's
// first fragments right after the stage barrier, across tile boundaries too.
// The second wave on each SIMD keeps the matrix unit fed while the other
// issues its loads or waits on LDS.
//
// LDS rows are 128 bytes (8 chunks).  128-bit LDS reads are served 16 lanes
// at a time over 64 banks (256 bytes = 2 rows); a fragment read puts 16
// consecutive rows, same chunk, in those lanes, so chunk c of row r sits at
// slot c ^ ((r >> 1) & 7): the 8 rows of each parity get 8 different slots.
//
// Operands are loaded through buffer resources that end at the tile's last
// row, so rows past the tile's rows or past K read zeros; chunks past N get an
// offset outside every buffer and read zeros too.  Weight slabs carry the
// non-temporal hint (NT_B) when the plan expects about one m-tile per expert,
// so that no other tile reads them again.  Ring stores
// are ordinary (temporal) stores: the consumer, which reads each ring row once
// with non-temporal loads right after this launch, then finds part of the
// ring in the last-level cache.
#include <algorithm>

#include "pgg_device.h"

namespace pgg {

namespace {

constexpr int kBN = 256;
constexpr int kThreads = 512, kWaves = 8;    // two waves per SIMD
constexpr int kWM = 2;                        // waves along rows
constexpr int kWTN = 64;                      // wave tile columns
constexpr int kFN = kWTN / 32;
constexpr int kRowChunks = 8;                 // 16-byte chunks per LDS row per stage
// reduction elements per stage: 128 bytes of each row
template <class T>
constexpr int stage_elems() { return kRowChunks * T::kPerChunk; }
constexpr int kPairs = kRowChunks / 2;
constexpr int kSlotsB = kBN * kRowChunks;
constexpr int kRowsPerLoad = 64 / kRowChunks;          // rows one wave instruction covers
constexpr int kLoadRows = kRowsPerLoad * kWaves;       // rows one load index covers across the waves
constexpr int kLoadsB = kSlotsB / kThreads;            // direct-to-LDS loads per thread per stage
constexpr int kSuperM = 8, kSuperN = 4;                // super-block of tiles per XCD round
constexpr int kSuper = kSuperM * kSuperN;
constexpr int kXcds = 8;
constexpr int kRound = kXcds * kSuper;                 // tiles of one raster round (256)
constexpr int kMaxTilesPerWg = 64;                     // LDS tile-table entries per workgroup
static_assert(kPairs % 2 == 0, "a stage must end on the second fragment set");
static_assert(kRowsPerLoad * kWaves * kLoadsB == kBN, "loads cover the tile columns");

// Tile heights.  256 rows with two LDS stages for many rows per expert; 128
// rows with three stages (two in flight at each barrier) when each expert has
// about one 128-row m-tile, where the weight stream, not the multiply, is the
// bound and the extra stage in flight streams it faster.
template <int BM>
struct Shape {
  static constexpr int kStages = BM == 256 ? 2 : 3;
  static constexpr int kWTM = BM / kWM;                // wave tile rows
  static constexpr int kFM = kWTM / 32;
  static constexpr int kSlotsA = BM * kRowChunks;
  static constexpr int kStageSlots = kSlotsA + kSlotsB;
  static constexpr int kLoadsA = kSlotsA / kThreads;
  static constexpr int kLoadsPerStage = kLoadsA + kLoadsB;
  static constexpr int kLoadsMax = kLoadsA > kLoadsB ? kLoadsA : kLoadsB;
  static_assert(BM == 256 || BM == 128, "tile heights");
  static_assert(kLoadsPerStage * kStages <= 63, "vmcnt range");
  static_assert(kRowsPerLoad * kWaves * kLoadsA == BM, "loads cover the tile rows");
  static_assert(kFM * kFN >= kFM + kFN, "a pair's MFMAs read every fragment of the next pair");
};

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
  int32_t span;             // raster positions of the launch (a multiple of kRound)
};

// A tile's operands as buffer resources: its d_y rows and its weight rows
// (the tile's output columns), each exactly as long as the tile holds rows,
// so loads of rows past the tile read zeros from the range check.
struct Operands {
  __amdgpu_buffer_rsrc_t a, b;
};

__device__ __forceinline__ int slot_of(int r, int c) { return c ^ ((r >> 1) & 7); }

template <class T, bool NT_B, int BM>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void produce_large_kernel(LargeArgs a) {
  using E = typename T::elem;
  using Sh = Shape<BM>;
  constexpr int kStages = Sh::kStages, kWTM = Sh::kWTM, kFM = Sh::kFM;
  constexpr int kSlotsA = Sh::kSlotsA, kStageSlots = Sh::kStageSlots;
  constexpr int kLoadsA = Sh::kLoadsA, kLoadsPerStage = Sh::kLoadsPerStage, kLoadsMax = Sh::kLoadsMax;
  constexpr int kBK = stage_elems<T>();
  __shared__ u32x4_t lds[kStages * kStageSlots];
  // this workgroup's tiles: {g, row0, rows, column tile}; rows 0 = no tile
  __shared__ int4 tab[kMaxTilesPerWg];

  if (a.hdr->err != kNoError) return;
  const int tid = threadIdx.x;
  const int grid = static_cast<int>(gridDim.x);
  const int n_mine = (a.span - static_cast<int>(blockIdx.x) + grid - 1) / grid;
  {
    const int n_tiles = a.hdr->n_tiles;
    for (int j = tid; j < n_mine; j += kThreads) {
      int slot, ct;
      int4 e = make_int4(0, 0, 0, 0);
      if (raster<kSuperM, kSuperN>(static_cast<int>(blockIdx.x) + j * grid, a.tc, a.n_col_tiles,
                                   slot, ct)) {
        const int64_t idx = static_cast<int64_t>(a.chunk) * a.tc + slot;
        const int64_t col0 = a.k_lo + static_cast<int64_t>(ct) * kBN;
        if (idx < n_tiles && col0 < a.k_hi) {
          const MTile m = a.tiles[idx];
          if (m.rows > 0) e = make_int4(m.g, m.row0, m.rows, ct);
        }
      }
      tab[j] = e;
    }
  }
  __syncthreads();
  // table entry j, the same in every lane (kept in scalar registers)
  auto entry = [&](int j) {
    const int4 e = tab[j];
    return make_int4(__builtin_amdgcn_readfirstlane(e.x), __builtin_amdgcn_readfirstlane(e.y),
                     __builtin_amdgcn_readfirstlane(e.z), __builtin_amdgcn_readfirstlane(e.w));
  };
  auto next_tile = [&](int j) {   // first entry at or after j with rows
    while (j < n_mine && entry(j).z <= 0) ++j;
    return j;
  };
  int cur = next_tile(0);
  if (cur >= n_mine) return;
  int nxt = next_tile(cur + 1);

  const int64_t N = a.N;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave % kWM, wn = wave / kWM;
  const int lr = lane & 31, lh = lane >> 5;
  // Direct-to-LDS load j of this wave fills slots (j*kWaves + wave)*64 + lane of a
  // region: row r0 + kLoadRows j (r0 = wave*8 + lane/8), slot lane%8, which
  // holds chunk (lane%8) ^ ((r0/2)%8) -- the same for every j.
  const int r0 = wave * kRowsPerLoad + (lane >> 3);
  const int dma_c = slot_of(r0, lane & 7);
  const uint32_t lds0 = __builtin_amdgcn_readfirstlane(lds_offset(lds));
  const int64_t chunk_row0 = a.chunk_row0[a.chunk];
  const uint32_t row_bytes = static_cast<uint32_t>(N * sizeof(E));
  // byte offset of load j's row chunk within a tile's operand buffer (the
  // same for d_y and weight rows)
  uint32_t voff[kLoadsMax];
#pragma unroll
  for (int j = 0; j < kLoadsMax; ++j)
    voff[j] = static_cast<uint32_t>(r0 + kLoadRows * j) * row_bytes + static_cast<uint32_t>(dma_c * 16);

  auto operands = [&](int j) {
    const int4 e = entry(j);
    const int64_t col0 = a.k_lo + static_cast<int64_t>(e.w) * kBN;
    const int cols = static_cast<int>(min<int64_t>(kBN, a.k_hi - col0));
    Operands o;
    o.a = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<E*>(static_cast<const E*>(a.A) + static_cast<int64_t>(e.y) * N), 0,
        static_cast<int>(static_cast<uint32_t>(e.z) * row_bytes), 0x00020000);
    o.b = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<E*>(static_cast<const E*>(a.B) + (static_cast<int64_t>(e.x) * a.K + col0) * N), 0,
        static_cast<int>(static_cast<uint32_t>(cols) * row_bytes), 0x00020000);
    return o;
  };
  // stage kt of a tile into LDS slot s; chunks past N read zeros
  // (offsets stay below 2^31 in range, and below 2^32 from kOutside)
  auto issue = [&](const Operands& o, int kt, int s) {
    const uint32_t base = lds0 + static_cast<uint32_t>(s * kStageSlots * 16);
    const uint32_t koff = static_cast<uint32_t>(kt) * kRowChunks * 16u;
    const bool in_n = static_cast<int64_t>(kt) * kBK + dma_c * T::kPerChunk < N;
#pragma unroll
    for (int j = 0; j < kLoadsA; ++j)
      dma16_buf(o.a, (in_n ? voff[j] : kOutside) + koff,
                base + static_cast<uint32_t>((j * kWaves + wave) * 64 * 16));
#pragma unroll
    for (int j = 0; j < kLoadsB; ++j) {
      const uint32_t vo = (in_n ? voff[j] : kOutside) + koff;
      const uint32_t m0 = base + static_cast<uint32_t>((kSlotsA + (j * kWaves + wave) * 64) * 16);
      if constexpr (NT_B) dma16_buf_nt(o.b, vo, m0);
      else dma16_buf(o.b, vo, m0);
    }
  };
  // fragment rows start at multiples of 32, so (row >> 1) & 7 == (lr >> 1) & 7
  auto load_frags = [&](int s, int q, u32x4_t (&fa)[kFM], u32x4_t (&fb)[kFN]) {
    const u32x4_t* st = lds + s * kStageSlots;
    const int sl = slot_of(lr, 2 * q + lh);
#pragma unroll
    for (int i = 0; i < kFM; ++i) fa[i] = st[(wm * kWTM + i * 32 + lr) * kRowChunks + sl];
#pragma unroll
    for (int j = 0; j < kFN; ++j) fb[j] = st[kSlotsA + (wn * kWTN + j * 32 + lr) * kRowChunks + sl];
  };
  // fragment idx (0..5: a0, b0, b1, a1, a2, a3, the order the MFMAs below
  // use them) of pair q of the stage in slot s
  auto load_frag = [&](int s, int q, int idx, u32x4_t (&fa)[kFM], u32x4_t (&fb)[kFN]) {
    const u32x4_t* st = lds + s * kStageSlots;
    const int sl = slot_of(lr, 2 * q + lh);
    if (idx == 0) fa[0] = st[(wm * kWTM + lr) * kRowChunks + sl];
    else if (idx <= kFN) fb[idx - 1] = st[kSlotsA + (wn * kWTN + (idx - 1) * 32 + lr) * kRowChunks + sl];
    else fa[idx - kFN] = st[(wm * kWTM + (idx - kFN) * 32 + lr) * kRowChunks + sl];
  };
  f32x16_t acc[kFM][kFN];
  // MFMA t of a pair multiplies block (t / kFN, t % kFN); the next pair's
  // fragment t is read beside it
  auto mfmas_reading = [&](const u32x4_t (&fa)[kFM], const u32x4_t (&fb)[kFN], int s, int q,
                           u32x4_t (&na)[kFM], u32x4_t (&nb)[kFN]) {
#pragma unroll
    for (int t = 0; t < kFM * kFN; ++t) {
      __builtin_amdgcn_sched_barrier(0);
      if (t < kFM + kFN) load_frag(s, q, t, na, nb);
      mma<T>(acc[t / kFN][t % kFN], fa[t / kFN], fb[t % kFN]);
    }
    __builtin_amdgcn_sched_barrier(0);
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
  Operands oc = operands(cur);
  Operands on = nxt < n_mine ? operands(nxt) : oc;
  // stage d of the stream counted from the current tile's first stage: the
  // current tile's, or -- past its last -- the next tile's, into LDS slot
  // (d + par) mod kStages.  d <= nk + kStages - 1 < 2 nk, since the host runs
  // this kernel only for nk >= kStages, so the stream never reaches past the
  // next tile.  With three stages, each barrier waits for all but the last
  // stage's loads, so past the stream's end a stage of zeros (every offset
  // past its buffer: no memory access) keeps that count; it lands in a slot
  // nobody reads again.
  auto issue_stream = [&](int d, int par) {
    if constexpr (kStages == 2) {
      if (d < nk) issue(oc, d, (d + par) & 1);
      else if (nxt < n_mine) issue(on, d - nk, (d + par) & 1);
    } else {
      if (d < nk) issue(oc, d, (d + par) % kStages);
      else if (nxt < n_mine) issue(on, d - nk, (d + par) % kStages);
      else issue(oc, nk, (d + par) % kStages);
    }
  };
  int par = 0;   // LDS slot of the current tile's stage 0
  issue_stream(0, par);
  issue_stream(1, par);
  if constexpr (kStages > 2) issue_stream(2, par);
  u32x4_t fa0[kFM], fb0[kFN], fa1[kFM], fb1[kFN];
  // stage 0 landed (the later ones may still be in flight)
  wait_then_barrier<(kStages - 1) * kLoadsPerStage>();
  load_frags(par, 0, fa0, fb0);
  for (;;) {
#pragma unroll
    for (int i = 0; i < kFM; ++i)
#pragma unroll
      for (int j = 0; j < kFN; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;
    const bool more = nxt < n_mine;
    for (int kt = 0; kt < nk; ++kt) {
      const int s = kStages == 2 ? (kt + par) & 1 : (kt + par) % kStages;
#pragma unroll
      for (int q = 0; q + 1 < kPairs; ++q) {
        if (q & 1) mfmas_reading(fa1, fb1, s, q + 1, fa0, fb0);
        else mfmas_reading(fa0, fb0, s, q + 1, fa1, fb1);
      }
      // Last pair: the stream's next stage landed everywhere and every wave
      // is done with this one; its slot is refilled with the stage kStages
      // ahead by the first wave of each SIMD before its last MFMAs of the stage and
      // by the second after them, so one of the two is always feeding the
      // matrix unit.  This runs unconditionally: issue_stream skips stages
      // past the stream's end, and after the last stage the barrier and the
      // fragment reads are merely idle.  A branch here would join ahead of
      // these MFMAs with the next stage's reads in flight, and the compiler
      // then waits for those reads before the MFMAs.
      wait_then_barrier<(kStages - 2) * kLoadsPerStage>();
      if (wave < kWaves / 2) issue_stream(kt + kStages, par);
      load_frags(kStages == 2 ? s ^ 1 : (kt + 1 + par) % kStages, 0, fa0, fb0);
      mfmas(fa1, fb1);
      if (wave >= kWaves / 2) issue_stream(kt + kStages, par);
    }

    // Epilogue: accumulator v of lane (lr, lh) is row 8*(v/4) + 4*lh + v%4,
    // column lr of its 32x32 block.  The stores go through a buffer resource
    // that ends at the tile's last element, so rows past the tile's rows are
    // dropped by the range check; lanes of columns past the tile's columns
    // get an offset outside it.
    {
      const int4 e = entry(cur);
      const int rows = e.z;
      const int64_t cofs = static_cast<int64_t>(e.w) * kBN;
      const int cols = static_cast<int>(min<int64_t>(kBN, a.k_hi - a.k_lo - cofs));
      const uint32_t ld4 = static_cast<uint32_t>(a.ldc) * 4u;   // ring row bytes
      const __amdgpu_buffer_rsrc_t out = __builtin_amdgcn_make_buffer_rsrc(
          a.ring + (static_cast<int64_t>(e.y) - chunk_row0) * a.ldc + cofs, 0,
          static_cast<int>(static_cast<uint32_t>(rows - 1) * ld4 + static_cast<uint32_t>(cols) * 4u),
          0x00020000);
      const uint32_t lane_off = static_cast<uint32_t>(wm * kWTM + 4 * lh) * ld4;
#pragma unroll
      for (int j = 0; j < kFN; ++j) {
        const int n = wn * kWTN + j * 32 + lr;
        // r * ld4 < 2^31 (256 rows of fewer than 2^21 floats): no wrap from kOutside
        const uint32_t voff = n < cols ? lane_off + static_cast<uint32_t>(n) * 4u : kOutside;
#pragma unroll
        for (int i = 0; i < kFM; ++i)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const uint32_t r = static_cast<uint32_t>(i * 32 + 8 * (v >> 2) + (v & 3));
            // a scalar copy first: a bit-cast of the vector element itself
            // compiles to element 0 whatever v is
            const float x = acc[i][j][v];
            __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, x), out, voff + r * ld4,
                                                  0, 0);
          }
      }
    }
    if (!more) break;
    // the next tile becomes current; its first stage sits in slot (par + nk) mod kStages
    par = kStages == 2 ? (par + nk) & 1 : (par + nk) % kStages;
    cur = nxt;
    oc = on;
    nxt = next_tile(cur + 1);
    if (nxt < n_mine) on = operands(nxt);
  }
  // the stages of zeros issued past the stream's end land before the
  // workgroup's LDS is released
  if constexpr (kStages > 2) wait_then_barrier<0>();
}

}  // namespace

// The tile stream needs at least two stages per tile, and a tile's
// operand rows and ring rows must each span less than 2^31 bytes (256 N
// elements, 256 ring rows of panel_cols floats); other shapes take the
// register-staged tile.
bool produce_uses_dma(const Plan& p, bool aligned) {
  const int64_t bk = p.dtype == PGG_F32 ? stage_elems<TF32>() : stage_elems<TBf16>();
  // at least kStages stages of the reduction
  const bool shape = p.bm == 256 ? p.N > bk : p.bm == 128 && p.dtype != PGG_F32 && p.N > 2 * bk;
  return aligned && p.regime == kLarge && shape &&
         p.N < (int64_t(1) << 22) && p.panel_cols < (int64_t(1) << 21);
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
  if (!produce_uses_dma(p, true)) return hipErrorInvalidValue;
  // raster positions in whole rounds; one workgroup per compute unit, more
  // (whole rounds) only when a workgroup's tile table would overflow
  const int64_t span = (int64_t(p.tc) * p.n_col_tiles + kRound - 1) / kRound * kRound;
  if (span >= (int64_t(1) << 30)) return hipErrorInvalidValue;
  a.span = static_cast<int32_t>(span);
  int64_t grid = std::min<int64_t>(span, kRound);
  const int64_t need = (span + kMaxTilesPerWg - 1) / kMaxTilesPerWg;
  if (grid < need) grid = (need + kRound - 1) / kRound * kRound;
  const dim3 g(static_cast<unsigned>(grid)), b(kThreads);
  const bool nt = p.stream_weights;
  if (p.bm == 128) {   // 16-bit, about one m-tile per expert: weight stream, non-temporal
    if (p.dtype == PGG_BF16) hipLaunchKernelGGL((produce_large_kernel<TBf16, true, 128>), g, b, 0, s, a);
    else hipLaunchKernelGGL((produce_large_kernel<TF16, true, 128>), g, b, 0, s, a);
  } else if (p.dtype == PGG_BF16) {
    if (nt) hipLaunchKernelGGL((produce_large_kernel<TBf16, true, 256>), g, b, 0, s, a);
    else hipLaunchKernelGGL((produce_large_kernel<TBf16, false, 256>), g, b, 0, s, a);
  } else if (p.dtype == PGG_F32) {
    if (nt) hipLaunchKernelGGL((produce_large_kernel<TF32, true, 256>), g, b, 0, s, a);
    else hipLaunchKernelGGL((produce_large_kernel<TF32, false, 256>), g, b, 0, s, a);
  } else {
    if (nt) hipLaunchKernelGGL((produce_large_kernel<TF16, true, 256>), g, b, 0, s, a);
    else hipLaunchKernelGGL((produce_large_kernel<TF16, false, 256>), g, b, 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace pgg
