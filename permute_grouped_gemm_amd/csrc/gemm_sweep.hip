// Producer for few rows per expert (bf16, fp16 and fp32 inputs): the same
// grouped-matmul gradient as the tiled producers,
//
//   C[i, k] = sum_n d_y[i, n] * W[g(i), k, n]        (fp32 accumulate)
//
// (MoeInitRoutingGroupedMatmulGrad design page, §数学定义和公式 Step 1;
// fp32 cube output, §2.6.2), organised around the weight stream, which is
// nearly all of the traffic when experts hold a few dozen rows or fewer.
//
// Work unit = one m-tile (at most 32 rows of one expert) x 16 weight rows
// (16 output columns) with the whole reduction over n.  A persistent grid
// takes units round-robin (unit u goes to workgroup u mod grid), and units
// are numbered in weight-address order (tile-major, weight rows within the
// expert fastest), so at any moment the grid reads a narrow moving window of
// the weight tensor, the pattern under which HBM delivers its best read rate.
// Workgroups that each own a long block of weight rows for the whole launch
// spread their concurrent reads over the full tensor and read measurably
// slower.
//
// A unit runs in stages of a fixed number of bytes per row.  Wave w
// multiplies the w-th quarter of every row of a stage with 16x16x32 MFMAs
// (16-bit) or 16x16x4 fp32 MFMAs; at the end of a unit the four waves'
// partial sums are added in wave order (fixed, so the result is
// bit-reproducible) and written to the ring.
//
// Rows that are 16-byte aligned take sweep_dma_kernel: stages of 512 bytes
// per row; the weight slab (16 rows) and the tile's d_y rows (16 or 32) of a
// stage are loaded straight into LDS through buffer resources that end at
// the unit's last weight row and the tile's last d_y row (so rows past them
// read zeros with no memory access), two rows per wave instruction (512-byte
// contiguous runs), three stages deep, so a stage's loads are issued two
// stages before it is multiplied and never drained at a stage boundary; two
// workgroups per CU overlap one's multiply with the other's waits.  Other
// rows take sweep_reg_kernel: stages of 1 KB per row through registers, one
// stage ahead.
//
// Chunk c (16 bytes) of LDS row r sits at slot c ^ (r & 15).  A fragment read
// puts 16 rows, same logical chunk, in 16 lanes, which then hit 16 different
// 16-byte bank groups; a row load or store (16 consecutive chunks per 16
// lanes) does too.
#include "pgg_device.h"
#include "pgg_prep.h"

namespace pgg {

namespace {

constexpr int kSwRows = 16;                 // weight rows per unit (output columns)
constexpr int kSwMS = 2;                    // 16-row MFMA blocks per m-tile (32 rows)
constexpr int kSwThreads = 256;             // 4 waves
constexpr int kSwWaves = 4;

// direct-to-LDS kernel
constexpr int kDmaChunks = 32;              // 16-byte chunks per row per stage (512 bytes)
constexpr int kDmaRPI = 64 / kDmaChunks;    // rows per wave instruction
constexpr int kDmaLoads = 16 / (kSwWaves * kDmaRPI);   // instructions per wave per 16-row block
constexpr int kDmaSteps = kDmaChunks / 16;  // 32-element MFMA steps per wave per stage
constexpr int kDmaStages = 3;
constexpr unsigned kDmaGrid = 512;          // two workgroups per CU
constexpr int kDmaSlotsW = kSwRows * kDmaChunks;
constexpr int kDmaSlotsA = kSwMS * 16 * kDmaChunks;
constexpr int kDmaStageSlots = kDmaSlotsW + kDmaSlotsA;
// loads one wave issues per stage for a tile of at most 16 rows
constexpr int kDmaMin = 2 * kDmaLoads;
static_assert(2 * (kDmaLoads * (1 + kSwMS)) + 2 <= 63, "vmcnt range");

// register-staged kernel
constexpr int kRegChunks = 64;              // 1 KB per row per stage, one row per wave instruction
constexpr int kRegLoads = kSwRows / kSwWaves;
constexpr int kRegSteps = kRegChunks / 16;
constexpr int kRegSlotsW = kSwRows * kRegChunks;
constexpr unsigned kRegGrid = 512;

struct SweepArgs {
  const void* A;            // grad_y [M, N]
  const void* B;            // weight [G, K, N]
  const WsHeader* hdr;
  const MTile* tiles;
  const int32_t* chunk_row0;
  float* ring;              // [ring_rows, K]
  int64_t N, K;
  int32_t chunk, tc, nkb;   // nkb: 16-column blocks of K
  // preparation inside the producer launch (one-chunk plans)
  const int64_t* eri;
  const int64_t* gl;
  PrepArgs prep;
  WsView ws;
};

template <class T>
__device__ __forceinline__ void mma16(f32x4_t& acc, u32x4_t a, u32x4_t b);

template <>
__device__ __forceinline__ void mma16<TBf16>(f32x4_t& acc, u32x4_t a, u32x4_t b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                __builtin_bit_cast(bf16x8_t, b), acc, 0, 0, 0);
}

template <>
__device__ __forceinline__ void mma16<TF16>(f32x4_t& acc, u32x4_t a, u32x4_t b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                               __builtin_bit_cast(f16x8_t, b), acc, 0, 0, 0);
}

// fp32: a chunk holds 4 reduction elements.  MFMA i takes element i of every
// lane's chunk; lane group g supplies reduction slot g of both operands, and
// both hold the same chunk there, so the four MFMAs cover the 16 elements of
// the four chunks once each.
template <>
__device__ __forceinline__ void mma16<TF32>(f32x4_t& acc, u32x4_t a, u32x4_t b) {
  const f32x4_t fa = __builtin_bit_cast(f32x4_t, a);
  const f32x4_t fb = __builtin_bit_cast(f32x4_t, b);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(fa[0], fb[0], acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(fa[1], fb[1], acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(fa[2], fb[2], acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(fa[3], fb[3], acc, 0, 0, 0);
}

// One unit's operands and output window.
template <class E>
struct Unit {
  const E* A;         // first d_y row of the m-tile
  __amdgpu_buffer_rsrc_t a_buf;   // the m-tile's d_y rows, exactly: rows past them read zeros
  const E* B;         // first weight row of the unit
  __amdgpu_buffer_rsrc_t b_buf;   // the unit's weight rows, exactly
  int rows, cols;     // valid d_y rows (<= 32) and weight rows (<= 16)
  int64_t ring_row;   // ring row of the tile's first row
  int64_t k0;         // first output column
};

template <class E>
__device__ __forceinline__ Unit<E> make_unit(const SweepArgs& a, const MTile& tile, int kb,
                                             int64_t chunk_base) {
  Unit<E> x;
  x.rows = tile.rows;
  x.k0 = static_cast<int64_t>(kb) * kSwRows;
  x.cols = static_cast<int>(min<int64_t>(kSwRows, a.K - x.k0));
  x.A = static_cast<const E*>(a.A) + static_cast<int64_t>(tile.row0) * a.N;
  x.a_buf = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<E*>(x.A), 0, static_cast<int>(static_cast<uint32_t>(tile.rows) * uint32_t(a.N * sizeof(E))),
      0x00020000);
  x.B = static_cast<const E*>(a.B) + (static_cast<int64_t>(tile.g) * a.K + x.k0) * a.N;
  x.b_buf = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<E*>(x.B), 0, static_cast<int>(static_cast<uint32_t>(x.cols) * uint32_t(a.N * sizeof(E))),
      0x00020000);
  x.ring_row = static_cast<int64_t>(tile.row0) - chunk_base;
  return x;
}

// End of a unit: every wave holds a partial 16x16 block per d_y block over
// its slice of the reduction (D layout: lane (lr, lg) -> row 4 lg + v,
// column lr).  The partials are summed in wave order and written to the ring.
template <class E, class Barrier>
__device__ __forceinline__ void finish_unit(const SweepArgs& a, const Unit<E>& x, f32x4_t (&acc)[kSwMS],
                                            float (*red)[kSwMS][256], Barrier barrier) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, lg = lane >> 4;
#pragma unroll
  for (int ms = 0; ms < kSwMS; ++ms) {
#pragma unroll
    for (int v = 0; v < 4; ++v) red[wave][ms][(4 * lg + v) * 16 + lr] = acc[ms][v];
    acc[ms] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  }
  barrier();
  float* __restrict__ out = a.ring + x.ring_row * a.K + x.k0;
  const int e = tid;   // element (e / 16, e % 16) of a 16x16 block
  const int k = e & 15;
#pragma unroll
  for (int ms = 0; ms < kSwMS; ++ms) {
    const int i = ms * 16 + (e >> 4);
    if (i < x.rows && k < x.cols) {
      const float s = ((red[0][ms][e] + red[1][ms][e]) + red[2][ms][e]) + red[3][ms][e];
      out[static_cast<int64_t>(i) * a.K + k] = s;
    }
  }
}

// ---------------------------------------------------------------- direct-to-LDS

// FUSED (one-chunk plans): block 0 runs the index preparation (tables, tile
// table, error word) for the consumer, and the other blocks take their tiles
// straight from group_list, so no preparation kernel has to finish first.
// They read neither the error word nor the tile table of this call; they check
// the group counts themselves (a failing check leaves the reporting to block
// 0) and the d_y rows they touch are then within [0, M).
template <class T, bool FUSED>
__global__ __launch_bounds__(kSwThreads) void sweep_dma_kernel(SweepArgs a) {
  using E = typename T::elem;
  constexpr int EPC = T::kPerChunk;
  __shared__ u32x4_t lds[kDmaStages * kDmaStageSlots];   // per stage: weight slab, then d_y rows
  __shared__ float red[kSwWaves][kSwMS][256];
  static_assert(sizeof(red) >= 2 * kSwThreads * sizeof(long long), "preparation scratch");

  int bid = static_cast<int>(blockIdx.x), nwg = static_cast<int>(gridDim.x);
  int tiles_here;
  int64_t chunk_base;
  if constexpr (FUSED) {
    if (bid == 0) {
      prep_block(a.prep, a.eri, a.gl, a.ws, reinterpret_cast<long long*>(&red[0][0][0]));
      return;
    }
    --bid;
    --nwg;
    // lane l of every wave reads groups l, l + 64, ... and the wave reduces:
    // total rows, total tiles, any count outside [0, M] (at most
    // kSweepPrepMaxGroups groups of at most M rows: no overflow)
    const int l = static_cast<int>(threadIdx.x & 63);
    int64_t rows = 0;
    int tiles = 0;
    bool out_of_range = false;
    for (int g = l; g < a.prep.G; g += 64) {
      const int64_t c = a.gl[g];
      out_of_range |= c < 0 || c > a.prep.M;
      rows += c;
      tiles += static_cast<int>((max<int64_t>(c, 0) + 16 * kSwMS - 1) / (16 * kSwMS));
    }
    const bool bad = __any(out_of_range);
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) {
      rows += __shfl_xor(rows, d);
      tiles += __shfl_xor(tiles, d);
    }
    if (bad || rows != a.prep.M) return;
    tiles_here = __builtin_amdgcn_readfirstlane(tiles);
    chunk_base = 0;
  } else {
    if (a.hdr->err != kNoError) return;
    tiles_here = min(a.tc, a.hdr->n_tiles - a.chunk * a.tc);
    chunk_base = a.chunk_row0[a.chunk];
  }
  const int nkb = a.nkb;
  // Every active workgroup takes the same number of units: with
  // q = ceil(units / grid) units each, only ceil(units / q) workgroups are
  // needed, and the rest leave, so no half of the grid idles through the
  // last round while the other half streams.
  {
    const int64_t units = static_cast<int64_t>(tiles_here) * nkb;
    const int64_t per = (units + nwg - 1) / nwg;
    if (per > 0) nwg = static_cast<int>((units + per - 1) / per);
  }
  if (bid >= nwg) return;
  // unit u = t * nkb + kb; this workgroup takes u = bid + j * nwg
  const int t0 = bid / nkb;
  if (t0 >= tiles_here) return;
  const int dq = nwg / nkb;
  const int dr = nwg - dq * nkb;

  const int64_t N = a.N;
  const int ns = static_cast<int>((N + kDmaChunks * EPC - 1) / (kDmaChunks * EPC));
  if (ns <= 0) return;   // the plan rejects N <= 0; the stage loop needs a stage
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 15;
  const int lg = lane >> 4;
  const int sub = lane / kDmaChunks;   // row of a wave instruction this lane loads
  const int ci = lane % kDmaChunks;    // LDS slot it fills
  const uint32_t lds_base = lds_offset(lds);

  // step cursor: (tile t, column block kb, stage st)
  struct Cursor {
    Unit<E> x;
    int t, kb, st;
    bool ok;
  };
  // FUSED: group gc's tiles start at tile tb and its rows at row rb; tiles are
  // opened in increasing order, so this cursor only moves forward
  int gc = 0, tb = 0;
  int64_t rb = 0;
  auto locate = [&](int t) {
    MTile tile;
    for (;;) {
      const int64_t c = scalar_load_i64(a.gl + gc);
      const int nt = static_cast<int>((c + 16 * kSwMS - 1) / (16 * kSwMS));
      if (t < tb + nt) {
        const int q = t - tb;
        tile.g = gc;
        tile.row0 = static_cast<int32_t>(rb + int64_t(q) * 16 * kSwMS);
        tile.rows = static_cast<int32_t>(min<int64_t>(16 * kSwMS, c - int64_t(q) * 16 * kSwMS));
        tile.pad = 0;
        return tile;
      }
      tb += nt;
      rb += c;
      ++gc;
    }
  };
  auto open = [&](Cursor& c) {
    c.ok = c.t < tiles_here;
    if (!c.ok) return;
    const int t = __builtin_amdgcn_readfirstlane(c.t);
    const int kb = __builtin_amdgcn_readfirstlane(c.kb);
    MTile tile;
    if constexpr (FUSED)
      tile = locate(t);
    else
      tile = scalar_load_tile(a.tiles + (static_cast<int64_t>(a.chunk) * a.tc + t));
    c.x = make_unit<E>(a, tile, kb, chunk_base);
  };
  auto advance = [&](const Cursor& c) {
    Cursor n = c;
    if (!c.ok) return n;
    if (++n.st == ns) {
      n.st = 0;
      n.t += dq;
      n.kb += dr;
      if (n.kb >= nkb) {
        n.kb -= nkb;
        ++n.t;
      }
      open(n);
    }
    return n;
  };

  // Issue one stage's loads into LDS stage `buf`.  Wave instruction l loads
  // rows r0, r0 + 1 (r0 = 2 (4 l + wave) within a 16-row block): lane i takes
  // row r0 + i / 32 and fetches its logical chunk (i % 32) ^ (r & 15), which
  // lands in slot i % 32.  The second d_y block is loaded only when the tile
  // has rows there, and first, so a wait that assumes the shorter count only
  // ever over-waits on it.
  // weight slabs are read once per call: non-temporal loads; d_y rows are
  // read by every unit of their tile, through the tile's buffer resource, so
  // rows past the tile cost no memory access
  const uint32_t row_bytes = static_cast<uint32_t>(N * sizeof(E));
  auto load_block_w = [&](const Unit<E>& x, uint32_t dst, int64_t nc) {
#pragma unroll
    for (int l = 0; l < kDmaLoads; ++l) {
      const int r0 = (4 * l + wave) * kDmaRPI;
      const int r = r0 + sub;
      const int64_t n = (nc + (ci ^ (r & 15))) * EPC;
      const uint32_t voff = n < N ? static_cast<uint32_t>(r) * row_bytes + static_cast<uint32_t>(n * sizeof(E))
                                  : kOutside;
      dma16_buf_nt(x.b_buf, voff, dst + static_cast<uint32_t>(r0 * kDmaChunks) * 16u);
    }
  };
  // r * row_bytes < 2^31 (the host runs this kernel only when 32 rows span
  // less than 2^31 bytes): no wrap from kOutside
  auto load_block_a = [&](const Unit<E>& x, int row0, uint32_t dst, int64_t nc) {
#pragma unroll
    for (int l = 0; l < kDmaLoads; ++l) {
      const int r0 = row0 + (4 * l + wave) * kDmaRPI;
      const int r = r0 + sub;
      const int64_t n = (nc + (ci ^ (r & 15))) * EPC;
      const uint32_t voff = n < N ? static_cast<uint32_t>(r) * row_bytes + static_cast<uint32_t>(n * sizeof(E))
                                  : kOutside;
      dma16_buf(x.a_buf, voff, dst + static_cast<uint32_t>(r0 * kDmaChunks) * 16u);
    }
  };
  auto issue = [&](const Cursor& c, int buf) {
    const uint32_t stage = lds_base + static_cast<uint32_t>(buf * kDmaStageSlots) * 16u;
    const int64_t nc = static_cast<int64_t>(c.st) * kDmaChunks;
    if (c.x.rows > 16) load_block_a(c.x, 16, stage + kDmaSlotsW * 16u, nc);
    load_block_w(c.x, stage, nc);
    load_block_a(c.x, 0, stage + kDmaSlotsW * 16u, nc);
  };

  f32x4_t acc[kSwMS];
#pragma unroll
  for (int ms = 0; ms < kSwMS; ++ms) acc[ms] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

  // wave w multiplies chunks [8 w, 8 w + 8) of the stage; MFMA step j, lane
  // group lg takes chunk 8 w + 4 j + lg
  auto compute = [&](const Cursor& c, int buf) {
    const u32x4_t* Ws = lds + buf * kDmaStageSlots;
    const u32x4_t* As = Ws + kDmaSlotsW;
    u32x4_t bf[kDmaSteps], af[kDmaSteps];
#pragma unroll
    for (int j = 0; j < kDmaSteps; ++j) {
      const int s = lr * kDmaChunks + ((wave * (kDmaChunks / 4) + j * 4 + lg) ^ lr);
      bf[j] = Ws[s];
      af[j] = As[s];
    }
#pragma unroll
    for (int j = 0; j < kDmaSteps; ++j) mma16<T>(acc[0], af[j], bf[j]);
    if (c.x.rows > 16) {
#pragma unroll
      for (int j = 0; j < kDmaSteps; ++j)
        af[j] = As[(16 + lr) * kDmaChunks + ((wave * (kDmaChunks / 4) + j * 4 + lg) ^ lr)];
#pragma unroll
      for (int j = 0; j < kDmaSteps; ++j) mma16<T>(acc[1], af[j], bf[j]);
    }
  };

  Cursor c0;
  c0.t = t0;
  c0.kb = bid - t0 * nkb;
  c0.st = 0;
  open(c0);
  Cursor c1 = advance(c0);
  Cursor c2 = advance(c1);
  issue(c0, 0);
  if (c1.ok) issue(c1, 1);
  int buf = 0;
  for (;;) {
    // stage `buf` (step c0) has landed once only step c1's loads (and ring
    // stores of a finished unit, which only make this wait longer) remain
    if (c1.ok)
      wait_then_barrier<kDmaMin>();
    else
      wait_then_barrier<0>();
    if (c2.ok) issue(c2, buf == 0 ? kDmaStages - 1 : buf - 1);   // the stage read one step ago
    compute(c0, buf);
    if (c0.st == ns - 1) finish_unit<E>(a, c0.x, acc, red, lds_barrier);
    if (!c1.ok) break;
    c0 = c1;
    c1 = c2;
    c2 = advance(c2);
    buf = buf == kDmaStages - 1 ? 0 : buf + 1;
  }
}

// ---------------------------------------------------------------- register staged

template <class T>
__global__ __launch_bounds__(kSwThreads) void sweep_reg_kernel(SweepArgs a) {
  using E = typename T::elem;
  constexpr int EPC = T::kPerChunk;
  __shared__ u32x4_t wst[2][kRegSlotsW];
  __shared__ float red[kSwWaves][kSwMS][256];

  if (a.hdr->err != kNoError) return;
  const int tiles_here = min(a.tc, a.hdr->n_tiles - a.chunk * a.tc);
  if (tiles_here <= 0) return;
  const int64_t units = static_cast<int64_t>(tiles_here) * a.nkb;
  int64_t u = blockIdx.x;
  if (u >= units) return;

  const int64_t N = a.N;
  const int ns = static_cast<int>((N + kRegChunks * EPC - 1) / (kRegChunks * EPC));
  if (ns <= 0) return;
  const int64_t chunk_base = a.chunk_row0[a.chunk];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int lr = lane & 15;
  const int lg = lane >> 4;

  auto unit_of = [&](int64_t uu) {
    const int tt = static_cast<int>(uu / a.nkb);
    const MTile tile = a.tiles[static_cast<int64_t>(a.chunk) * a.tc + tt];
    return make_unit<E>(a, tile, static_cast<int>(uu - static_cast<int64_t>(tt) * a.nkb), chunk_base);
  };
  auto load_w = [&](const Unit<E>& x, int st, u32x4_t (&wr)[kRegLoads]) {
    const int64_t n = static_cast<int64_t>(st) * kRegChunks * EPC + lane * EPC;
#pragma unroll
    for (int l = 0; l < kRegLoads; ++l) {
      const int r = 4 * l + wave;
      wr[l] = load_chunk<T, false>(x.B + static_cast<int64_t>(r) * N, r < x.cols, n, N);
    }
  };
  auto store_w = [&](int buf, const u32x4_t (&wr)[kRegLoads]) {
#pragma unroll
    for (int l = 0; l < kRegLoads; ++l) {
      const int r = 4 * l + wave;
      wst[buf][r * kRegChunks + (lane ^ r)] = wr[l];
    }
  };
  // d_y fragments of a stage for this wave's slice: MFMA step j, lane group
  // lg takes chunk 16 wave + 4 j + lg
  auto load_a = [&](const Unit<E>& x, int st, u32x4_t (&ar)[kSwMS][kRegSteps]) {
#pragma unroll
    for (int ms = 0; ms < kSwMS; ++ms) {
      const int i = ms * 16 + lr;
      const E* row = x.A + static_cast<int64_t>(i) * N;
#pragma unroll
      for (int j = 0; j < kRegSteps; ++j) {
        const int64_t n = (static_cast<int64_t>(st) * kRegChunks + wave * 16 + j * 4 + lg) * EPC;
        ar[ms][j] = load_chunk<T, false>(row, i < x.rows, n, N);
      }
    }
  };

  f32x4_t acc[kSwMS];
#pragma unroll
  for (int ms = 0; ms < kSwMS; ++ms) acc[ms] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

  auto compute = [&](int buf, const Unit<E>& x, const u32x4_t (&ar)[kSwMS][kRegSteps]) {
    u32x4_t bf[kRegSteps];
#pragma unroll
    for (int j = 0; j < kRegSteps; ++j) bf[j] = wst[buf][lr * kRegChunks + ((wave * 16 + j * 4 + lg) ^ lr)];
#pragma unroll
    for (int j = 0; j < kRegSteps; ++j) mma16<T>(acc[0], ar[0][j], bf[j]);
    if (x.rows > 16) {
#pragma unroll
      for (int j = 0; j < kRegSteps; ++j) mma16<T>(acc[1], ar[1][j], bf[j]);
    }
  };

  // step t+1's weight slab and d_y fragments are in flight while step t is
  // multiplied
  Unit<E> cur = unit_of(u);
  int st = 0;
  u32x4_t wr[kRegLoads];
  u32x4_t ar[kSwMS][kRegSteps], an[kSwMS][kRegSteps];
  load_w(cur, 0, wr);
  load_a(cur, 0, ar);
  store_w(0, wr);
  __syncthreads();
  int buf = 0;
  for (;;) {
    int st_n = st + 1;
    int64_t u_n = u;
    if (st_n == ns) {
      st_n = 0;
      u_n = u + gridDim.x;
    }
    const bool more = u_n < units;
    Unit<E> nxt = cur;
    if (more) {
      if (u_n != u) nxt = unit_of(u_n);
      load_w(nxt, st_n, wr);
      load_a(nxt, st_n, an);
    }
    compute(buf, cur, ar);
    if (st == ns - 1) finish_unit<E>(a, cur, acc, red, [] { __syncthreads(); });
    if (!more) break;
    store_w(buf ^ 1, wr);
    __syncthreads();
    buf ^= 1;
#pragma unroll
    for (int ms = 0; ms < kSwMS; ++ms)
#pragma unroll
      for (int j = 0; j < kRegSteps; ++j) ar[ms][j] = an[ms][j];
    cur = nxt;
    u = u_n;
    st = st_n;
  }
}

// The direct-to-LDS sweep addresses an m-tile's d_y rows through a buffer
// resource: 32 rows must span less than 2^31 bytes.
bool sweep_dma_fits(const Plan& p) {
  const int64_t elem = p.dtype == PGG_F32 ? 4 : 2;
  return int64_t(16 * kSwMS) * p.N * elem < (int64_t(1) << 31);
}

template <class T>
hipError_t launch_typed(const Plan& p, const SweepArgs& args, bool aligned, bool fused, hipStream_t s) {
  const int64_t units = static_cast<int64_t>(p.tc) * p.n_col_tiles;
  if (fused) {
    // block 0 prepares; the others sweep (one slot of the two-per-CU grid
    // is lent to the preparation for its few microseconds)
    const dim3 grid(static_cast<unsigned>(std::min<int64_t>(units, kDmaGrid - 1) + 1));
    hipLaunchKernelGGL((sweep_dma_kernel<T, true>), grid, dim3(kSwThreads), 0, s, args);
  } else if (aligned && sweep_dma_fits(p)) {
    const dim3 grid(static_cast<unsigned>(std::min<int64_t>(units, kDmaGrid)));
    hipLaunchKernelGGL((sweep_dma_kernel<T, false>), grid, dim3(kSwThreads), 0, s, args);
  } else {
    const dim3 grid(static_cast<unsigned>(std::min<int64_t>(units, kRegGrid)));
    hipLaunchKernelGGL((sweep_reg_kernel<T>), grid, dim3(kSwThreads), 0, s, args);
  }
  return hipGetLastError();
}

SweepArgs sweep_args(const Plan& p, int chunk, const void* grad_y, const void* weight, const WsView& w) {
  SweepArgs a{};
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
  a.nkb = p.n_col_tiles;
  a.prep = prep_args(p);
  a.ws = w;
  return a;
}

hipError_t launch(const Plan& p, const SweepArgs& a, bool aligned, bool fused, hipStream_t s) {
  if (p.bm != 16 * kSwMS || p.bn != kSwRows) return hipErrorInvalidValue;
  switch (p.dtype) {
    case PGG_BF16: return launch_typed<TBf16>(p, a, aligned, fused, s);
    case PGG_F16: return launch_typed<TF16>(p, a, aligned, fused, s);
    case PGG_F32: return launch_typed<TF32>(p, a, aligned, fused, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

bool sweep_can_prepare(const Plan& p, bool aligned) {
  return aligned && sweep_dma_fits(p) && p.regime == kStream && p.n_panels == 1 && p.max_chunks == 1 &&
         p.G <= kSweepPrepMaxGroups;
}

hipError_t launch_produce_sweep(const Plan& p, int chunk, const void* grad_y, const void* weight,
                                bool aligned, const WsView& w, hipStream_t s) {
  return launch(p, sweep_args(p, chunk, grad_y, weight, w), aligned, false, s);
}

hipError_t launch_produce_sweep_prepared(const Plan& p, const void* grad_y, const void* weight,
                                         const int64_t* eri, const int64_t* gl, const WsView& w,
                                         hipStream_t s) {
  if (!sweep_can_prepare(p, true)) return hipErrorInvalidValue;
  SweepArgs a = sweep_args(p, 0, grad_y, weight, w);
  a.eri = eri;
  a.gl = gl;
  return launch(p, a, true, true, s);
}

}  // namespace pgg
