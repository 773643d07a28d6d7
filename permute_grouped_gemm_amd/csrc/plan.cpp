// Host-side validation and workspace planning (shapes only; no HIP calls).
//
// Validation follows the constraints table of the MoeInitRoutingGroupedMatmulGrad
// design page (§1.2) and its infershape checks (§2.3.3).  The schedule splits
// the expert-ordered list of m-tiles into chunks whose fp32 output rows fit a
// ring of bounded size, so the workspace does not grow with M·K.
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <cmath>

#include "pgg_internal.h"

namespace pgg {

namespace {

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Bound on the fp32 ring (bytes): 1 GiB, a fixed amount whatever M (0.35 %
// of an MI355X's 288 GB).  Measured against 256 and 512 MiB with the panel
// choice below: the large fp16 call (M 110592, K 7168, N 2048) took 3.92
// against 4.34 and 4.07 ms, fewer chunks per panel meaning fewer
// read-modify-writes of d_x.  PGG_RING_MB lowers it for tuning; a fixed
// setting gives fixed results.  At most 1 GiB: ring offsets stay below 2^30
// bytes.
size_t ring_budget() {
  constexpr long kMaxMb = 1024;
  const char* e = getenv("PGG_RING_MB");
  if (e) {
    long mb = strtol(e, nullptr, 10);
    if (mb > 0) return static_cast<size_t>(std::min<long>(mb, kMaxMb)) << 20;
  }
  return static_cast<size_t>(kMaxMb) << 20;
}

struct TileShape { int bm, bn; };

// Columns per panel when K is cut into n panels: whole tiles of bn columns.
int64_t panel_width(int64_t K, int n, int bn) {
  const int64_t w = (K + n - 1) / n;
  return std::min<int64_t>(K, (w + bn - 1) / bn * bn);
}

// m-tiles per chunk when a ring row holds `cols` fp32 columns.
int64_t tiles_per_chunk(int bm, int64_t cols, size_t budget, int64_t max_tiles) {
  const size_t per_tile = size_t(bm) * size_t(cols) * sizeof(float);
  const int64_t tc = static_cast<int64_t>(budget / per_tile);
  return std::max<int64_t>(1, std::min<int64_t>(tc, max_tiles));
}

// Panel count.  PGG_PANEL_COLS fixes the panel width (tuning; a fixed
// setting gives fixed results).  Otherwise a time estimate picks it, with
// rates measured on MI355X at the large fp16, large fp32 and mid bf16 shapes:
//  - the consumer reads every ring row once.  With C chunks per panel, each
//    of a token's topK rows in any chunk alike, the token's rows fall in
//    E = C (1 - (1 - 1/C)^topK) distinct chunks and its d_x row is read and
//    written 2E - 1 times (once when C = 1); it moves these bytes at about
//    6.4-6.8 TB/s with up to 3 chunks per panel, about 5 TB/s with 4 (the
//    chunk consumer) and about 5 TB/s by ring row (more chunks);
//  - every panel past the first reads d_y again: about 15 TB/s of extra
//    reads for the 16-bit producers, which hide most of it behind the
//    multiply, and 4.7 TB/s for the fp32 producer;
//  - the large-tile producer runs one 256 x 256 tile per compute unit at a
//    time, so a launch of T tiles takes ceil(T / 256) rounds of about
//    21 us + 0.022 us x N each for 16-bit inputs (measured at N = 2048 and
//    4096), and about 16 times that per N for fp32 (the MFMA rate).  The
//    true m-tile count is known only on the device; rounds are counted at
//    its expectation under routing that is uniform over the experts
//    (expected_tiles), cut into chunks of the plan's size (which the bound
//    sets).  The bound (M / 256 plus one partial tile per expert)
//    overstates a launch by up to G / 2 m-tiles, which at 64 experts of
//    about 512 rows (K 7168, N 2048) made 7 panels of one chunk look as fast
//    as 2 panels of three, against 1.52 and 1.38 ms measured.
// The weight-streaming producer keeps one panel.
// Rounds of the large-tile producer over all panels of width w with chunks
// of tc m-tiles, for `tiles` m-tiles.
int64_t producer_rounds(const Plan& q, int64_t w, int64_t tc, int64_t tiles) {
  constexpr int64_t kCUs = 256;
  int64_t rounds = 0;
  for (int64_t k0 = 0; k0 < q.K; k0 += w) {
    const int64_t ct = (std::min<int64_t>(w, q.K - k0) + q.bn - 1) / q.bn;
    for (int64_t left = tiles; left > 0; left -= tc)
      rounds += (std::min<int64_t>(left, tc) * ct + kCUs - 1) / kCUs;
  }
  return rounds;
}

// Expected m-tiles of bm rows per expert when each token's topK experts are
// distinct and uniform: an expert's row count is then Binomial(batch, topK /
// G), and E[ceil(c / bm)] = sum_j P(c > j bm), taken from the normal
// approximation with continuity correction.  Terms more than 8 standard
// deviations below the mean are 1 and are counted without the loop, so the
// loop runs over at most 16 sd / bm + 2 terms.
double expected_tiles_per_expert(const Plan& q, int bm) {
  const double p = std::min(1.0, double(q.topk) / double(q.G));
  const double mu = double(q.batch) * p;
  const double sd = std::sqrt(double(q.batch) * p * (1.0 - p));
  const int64_t j0 = static_cast<int64_t>(std::max(0.0, mu - 8.0 * sd - 1.0) / bm);
  double per_expert = double(j0);
  for (int64_t j = j0; double(j) * bm < mu + 8.0 * sd + 1.0; ++j) {
    const double x = double(j) * bm;
    per_expert += sd > 0.0 ? 0.5 * std::erfc((x + 0.5 - mu) / (sd * std::sqrt(2.0))) : (mu > x ? 1.0 : 0.0);
  }
  return per_expert;
}

// The same over all experts, clamped to [ceil(M / bm), max_tiles].
int64_t expected_tiles(const Plan& q, int64_t max_tiles) {
  const int64_t lo = (q.M + q.bm - 1) / q.bm;
  const int64_t est = static_cast<int64_t>(std::ceil(expected_tiles_per_expert(q, q.bm) * double(q.G)));
  return std::max<int64_t>(lo, std::min<int64_t>(est, max_tiles));
}

// Producer family, and for the fp32 tiles their height.  Measured on MI355X
// with uniform routing (K x N of 7168 x 4096, 7168 x 2048 and 2048 x 1408;
// 16, 60 and 64 experts):
//  - 16-bit: the weight sweep reads every expert's weights once per 32-row
//    m-tile, the 256 x 256 tiles once per 256 rows.  The sweep is faster up
//    to 24 rows per expert (197 against 236 us, 405 against 456 us) and the
//    tiles from 32 (240 against 253 us, 473 against 534 us, 112 against 140
//    us), so the sweep takes M <= 28 G.
//  - fp32 up to 32 rows per expert: the weight sweep (fp32 MFMAs on the same
//    staged chunks), 359 against 1057 us for the 128 x 128 tile at 8 rows
//    per expert (16 experts, 7168 x 4096); at 32 it ties with the 64 x 128
//    tile (606 against about 600 us) and at 48 it loses (921 against 598).
//  - fp32 above that: the tiles are bound by the fp32 MFMAs, which also
//    multiply the padding rows of each expert's last m-tile.  The tile with
//    the least expected padded rows at its relative rate is taken: 0.73 for
//    64 x 128, 0.78 for 128 x 128 and 0.85 for the direct-to-LDS 256 x 256,
//    fitted to the measured choices: 64 rows at 48-64, 128-256 rows per
//    expert (598 against 1081 us at 48, 1469 against 1631 at 128), 128 rows
//    at 96 (1100 against 1175 us), 256 rows at 192 and 1024 and at the large
//    fp32 shape (1.95 against 2.04 ms, 16.05 against 16.51 ms, 25.4 against
//    27.4 ms).
struct Family {
  int32_t regime;
  int32_t bm;   // fp32 tile rows (kF32 only)
};

Family choose_family(const Plan& q) {
  if (q.dtype != PGG_F32) return {q.M <= 28 * q.G ? kStream : kLarge, 0};
  const double c64 = expected_tiles_per_expert(q, 64) * 64.0 / 0.73;
  const double c128 = expected_tiles_per_expert(q, 128) * 128.0 / 0.78;
  const double c256 = expected_tiles_per_expert(q, 256) * 256.0 / 0.85;
  const int32_t bm = c64 <= c128 ? 64 : 128;
  if (q.M <= 32 * q.G) return {kStream, bm};
  if (c256 < std::min(c64, c128)) return {kLarge, bm};
  return {kF32, bm};
}

int choose_panels(const Plan& q, size_t budget, int64_t max_tiles) {
  // the weight sweep stores whole K-column ring rows: one panel, whatever the override
  if (q.regime == kStream) return 1;
  const int64_t max_panels = (q.K + q.bn - 1) / q.bn;
  if (const char* e = getenv("PGG_PANEL_COLS")) {
    const long c = strtol(e, nullptr, 10);
    if (c > 0) {
      const int64_t w = std::min<int64_t>(q.K, (c + q.bn - 1) / q.bn * q.bn);
      return static_cast<int>((q.K + w - 1) / w);
    }
  }
  constexpr double kConsumeRate = 6.7, kManyChunkRate = 5.0;
  constexpr int64_t kFastChunks = 3;
  const double reread_rate = q.dtype == PGG_F32 ? 4.7 : 15.0;
  const double elem = q.dtype == PGG_F32 ? 4.0 : 2.0;
  const double dy_bytes = double(q.M) * double(q.N) * elem;
  const double ring_bytes = double(q.M) * double(q.K) * 4.0;
  const double dx_bytes = double(q.batch) * double(q.K) * 4.0;
  // one round of 256 x 256 tiles, in ps (fp32: the MFMA rate is 16 times lower)
  const double round_ps = 21.0e6 + (q.dtype == PGG_F32 ? 230.0e3 : 22.0e3) * double(q.N);
  const int64_t est_tiles = expected_tiles(q, max_tiles);
  int best = 1;
  double best_time = 0.0;
  int64_t last_width = -1;
  for (int64_t n = 1; n <= std::min<int64_t>(max_panels, 64); ++n) {
    const int64_t w = panel_width(q.K, static_cast<int>(n), q.bn);
    if (w == last_width) continue;   // same width as a smaller count
    last_width = w;
    const int64_t panels = (q.K + w - 1) / w;
    const int64_t tc = tiles_per_chunk(q.bm, w, budget, max_tiles);
    const int64_t chunks = (max_tiles + tc - 1) / tc;
    const double c = double(chunks);
    const double e = c * (1.0 - std::pow(1.0 - 1.0 / c, double(q.topk)));
    double t = (ring_bytes + dx_bytes * (2.0 * e - 1.0)) /
               (chunks <= kFastChunks ? kConsumeRate : kManyChunkRate);
    t += double(panels - 1) * dy_bytes / reread_rate;
    if (q.regime == kLarge) t += double(producer_rounds(q, w, tc, est_tiles)) * round_ps;
    if (n == 1 || t < best_time) {
      best = static_cast<int>(panels);
      best_time = t;
    }
  }
  return best;
}

// Output tile per regime: large-M MFMA tiles (every input type); for few rows
// per expert, m-tiles of 32 rows crossed with units of 16 weight rows that a
// persistent grid streams in address order; for fp32 in between, tiles 128
// wide and 64 or 128 rows high (the height chosen with the family).
TileShape tile_shape(int32_t regime) {
  switch (regime) {
    case kLarge: return {256, 256};
    case kStream: return {32, 16};
    default: return {128, 128};
  }
}

}  // namespace

namespace {

pgg_status plan_with_budget(const pgg_moe_dx_desc* d, size_t budget, Plan* p) {
  if (!d || !p) return PGG_ERR_INVALID_ARG;
  const int64_t M = d->grad_y_rows, N = d->grad_y_cols;
  const int64_t G = d->weight_groups, K = d->weight_rows;
  if (d->reserved != 0) return PGG_ERR_INVALID_ARG;
  if (d->topk <= 0 || d->batch <= 0) return PGG_ERR_INVALID_ARG;
  if (d->row_idx_type != 0 && d->row_idx_type != 1) return PGG_ERR_INVALID_ARG;
  if (d->grad_y_dtype != d->weight_dtype) return PGG_ERR_INVALID_ARG;
  if (d->grad_y_dtype < PGG_F32 || d->grad_y_dtype > PGG_BF16) return PGG_ERR_INVALID_ARG;
  if (N != d->weight_cols) return PGG_ERR_INVALID_ARG;
  if (d->group_list_len != G) return PGG_ERR_INVALID_ARG;
  if (G <= 0 || K <= 0 || N <= 0 || M <= 0) return PGG_ERR_INVALID_ARG;
  if (d->topk > INT64_MAX / d->batch) return PGG_ERR_INVALID_ARG;
  if (M != d->batch * d->topk) return PGG_ERR_INVALID_ARG;
  const int64_t L = d->idx_len;
  if (L < d->batch || L > d->batch * d->topk || L < M) return PGG_ERR_INVALID_ARG;
  // Row indices are kept as int32 on the device; the page limits M to 2^31.
  if (M >= (int64_t(1) << 31) - 1) return PGG_ERR_UNSUPPORTED;
  if (G >= (int64_t(1) << 30) || K >= (int64_t(1) << 31) || N >= (int64_t(1) << 31))
    return PGG_ERR_UNSUPPORTED;
  // the consumer addresses a d_x row (4K bytes) through a 32-bit range
  if (K >= (int64_t(1) << 29)) return PGG_ERR_UNSUPPORTED;

  Plan q{};
  q.n_panels = 1;
  q.M = M; q.N = N; q.G = G; q.K = K; q.batch = d->batch; q.topk = d->topk;
  q.row_idx_type = d->row_idx_type;
  q.panel_cols = q.K;
  q.dtype = d->grad_y_dtype;
  // few rows per expert: the weight sweep, or for fp32 between the sweep and
  // the large tile the 64 x 128 or 128 x 128 tile
  const Family fam = choose_family(q);
  q.regime = fam.regime;
  // Non-temporal weight loads in the large tiles pay when each expert has
  // about one 256-row m-tile, so no other tile reads its slabs (measured:
  // 6-9 % faster at 64-128 rows per expert, 4-7 % slower at the large and mid
  // shapes, where every slab serves several m-tiles through L2).
  q.stream_weights = expected_tiles_per_expert(q, 256) <= 1.25;
  // PGG_REGIME=large, =few or =sweep fixes the producer family (tuning)
  if (const char* e = getenv("PGG_REGIME")) {
    if (!strcmp(e, "large")) q.regime = kLarge;
    else if (!strcmp(e, "few")) q.regime = q.dtype == PGG_F32 ? kF32 : kStream;
    else if (!strcmp(e, "sweep")) q.regime = kStream;
  }
  const TileShape ts = tile_shape(q.regime);
  q.bm = q.regime == kF32 ? fam.bm : ts.bm;
  q.bn = ts.bn;
  // 16-bit tiles 128 rows high (three LDS stages) when each expert has about
  // one such m-tile: measured 6-16 % faster than the 256-row tiles at 32-96
  // rows per expert, slower from 128 (two m-tiles for half the experts).
  if (q.regime == kLarge && q.dtype != PGG_F32 && q.stream_weights &&
      expected_tiles_per_expert(q, 128) <= 1.2)
    q.bm = 128;
  const int64_t max_tiles = (M + q.bm - 1) / q.bm + G;
  if (max_tiles >= (int64_t(1) << 31)) return PGG_ERR_UNSUPPORTED;
  q.max_tiles = static_cast<int32_t>(max_tiles);
  // Column panels: the output columns are cut into panels of panel_cols
  // (a multiple of the tile width), and every panel runs the whole chunk
  // sequence over the rows.  A ring row then holds one panel's columns, so a
  // chunk holds K / panel_cols times more rows: fewer chunks touch each token,
  // and the consumer re-reads and re-writes fewer d_x rows, at the price of
  // reading d_y once per panel.
  const int n_panels = choose_panels(q, budget, max_tiles);
  q.n_panels = n_panels;
  q.panel_cols = panel_width(K, n_panels, q.bn);
  int64_t tc = tiles_per_chunk(q.bm, q.panel_cols, budget, max_tiles);
  // keep the consumer grid (ring rows x column blocks of 256) well inside 2^31 work-items
  const int64_t col_blocks_worst = (int64_t(q.panel_cols) + 255) / 256;
  while (tc > 1 && tc * q.bm * col_blocks_worst >= (int64_t(1) << 23)) tc /= 2;
  if (int64_t(q.bm) * col_blocks_worst >= (int64_t(1) << 23)) return PGG_ERR_UNSUPPORTED;
  q.tc = static_cast<int32_t>(tc);
  q.max_chunks = static_cast<int32_t>((max_tiles + tc - 1) / tc);
  // a chunk's rows are at most its tiles' capacity and at most M; producers store
  // only the rows their tiles hold, at (row - first row of the chunk)
  q.ring_rows = static_cast<int32_t>(std::min<int64_t>(int64_t(q.tc) * q.bm, M));
  // column tiles of one panel (the last panel may use fewer)
  q.n_col_tiles = static_cast<int32_t>((q.panel_cols + q.bn - 1) / q.bn);
  q.fused_prep = M <= 16384;
  q.ksplit = 1;
  q.kspan = static_cast<int32_t>(N);

  size_t off = 0;
  q.off_header = off;   off = align_up(off + sizeof(WsHeader), kRegionAlign);
  q.off_offsets = off;  off = align_up(off + sizeof(int64_t) * size_t(G + 1), kRegionAlign);
  q.off_tiles = off;    off = align_up(off + sizeof(MTile) * size_t(q.max_tiles), kRegionAlign);
  q.off_chunks = off;   off = align_up(off + sizeof(int32_t) * size_t(q.max_chunks + 1), kRegionAlign);
  q.off_inv = off;      off = align_up(off + sizeof(int32_t) * size_t(M), kRegionAlign);
  q.off_ori = off;      off = align_up(off + sizeof(int32_t) * size_t(M), kRegionAlign);
  q.table_bytes = off;
  q.off_ring = off;
  q.ring_bytes = size_t(q.ring_rows) * size_t(q.panel_cols) * sizeof(float);
  off = align_up(off + q.ring_bytes, kRegionAlign);
  q.total = off;
  *p = q;
  return PGG_OK;
}

}  // namespace

pgg_status make_plan(const pgg_moe_dx_desc* d, Plan* p) {
  return plan_with_budget(d, ring_budget(), p);
}

pgg_status make_plan_within(const pgg_moe_dx_desc* d, size_t max_total, Plan* p) {
  Plan q;
  pgg_status st = plan_with_budget(d, ring_budget(), &q);
  if (st != PGG_OK) return st;
  // the tables' size with the largest possible chunk table (one chunk per m-tile)
  const size_t tables = q.table_bytes +
                        align_up(sizeof(int32_t) * size_t(q.max_tiles + 1), kRegionAlign) + kRegionAlign;
  if (max_total <= tables) return PGG_ERR_WORKSPACE_TOO_SMALL;
  st = plan_with_budget(d, std::min(ring_budget(), max_total - tables), &q);
  if (st != PGG_OK) return st;
  if (q.total > max_total) return PGG_ERR_WORKSPACE_TOO_SMALL;
  *p = q;
  return PGG_OK;
}

pgg_status make_fwd_plan(const pgg_moe_fwd_desc* d, Plan* p) {
  if (!d || !p) return PGG_ERR_INVALID_ARG;
  const int64_t batch = d->x_rows, K = d->x_cols;
  const int64_t G = d->weight_groups, N = d->weight_cols;
  if (d->reserved != 0) return PGG_ERR_INVALID_ARG;
  if (d->topk <= 0 || d->batch <= 0 || batch != d->batch) return PGG_ERR_INVALID_ARG;
  if (d->row_idx_type != 0 && d->row_idx_type != 1) return PGG_ERR_INVALID_ARG;
  if (d->x_dtype != d->weight_dtype) return PGG_ERR_INVALID_ARG;
  if (d->x_dtype < PGG_F32 || d->x_dtype > PGG_BF16) return PGG_ERR_INVALID_ARG;
  if (K != d->weight_rows) return PGG_ERR_INVALID_ARG;
  if (d->group_list_len != G) return PGG_ERR_INVALID_ARG;
  if (G <= 0 || K <= 0 || N <= 0) return PGG_ERR_INVALID_ARG;
  if (d->topk > INT64_MAX / d->batch) return PGG_ERR_INVALID_ARG;
  const int64_t M = d->batch * d->topk;
  if (d->idx_len != M) return PGG_ERR_INVALID_ARG;
  if (M >= (int64_t(1) << 31) - 1) return PGG_ERR_UNSUPPORTED;
  if (G >= (int64_t(1) << 30) || K >= (int64_t(1) << 31) || N >= (int64_t(1) << 31))
    return PGG_ERR_UNSUPPORTED;

  Plan q{};
  q.n_panels = 1;
  q.M = M; q.N = K; q.G = G; q.K = N; q.batch = d->batch; q.topk = d->topk;
  q.row_idx_type = d->row_idx_type;
  q.panel_cols = q.K;
  q.dtype = d->x_dtype;
  if (q.dtype == PGG_F32) {
    q.regime = kF32;
    q.bm = 128; q.bn = 128;
  } else if (M <= 64 * G) {
    q.regime = kStream;   // few rows per expert: 32-row m-tiles
    q.bm = 32; q.bn = 256;
  } else {
    q.regime = kLarge;
    q.bm = 256; q.bn = 256;
  }
  const int64_t max_tiles = (M + q.bm - 1) / q.bm + G;
  const int64_t col_tiles = (N + q.bn - 1) / q.bn;
  // the launch grid covers max_tiles x col_tiles workgroups
  if (max_tiles * col_tiles >= (int64_t(1) << 31) - 8 * 32) return PGG_ERR_UNSUPPORTED;
  q.max_tiles = static_cast<int32_t>(max_tiles);
  q.tc = q.max_tiles;
  q.max_chunks = 1;
  q.ring_rows = 0;
  q.n_col_tiles = static_cast<int32_t>(col_tiles);
  q.fused_prep = M <= 16384;
  // Few rows per expert: each tile streams its expert's weight columns over
  // the whole reduction.  When the tiles alone would leave the GPU short of
  // workgroups (at most max_tiles x col_tiles have work), the reduction is
  // split so that up to about 512 workgroups stream at once: one per resident
  // slot (two per compute unit).  More would run as a second, partly empty
  // wave (at the decode shape 2 splits took 133 us, 3 took 146 us, 4 took
  // 139 us).  Each split writes an fp32 partial of y and a reduction kernel
  // adds them in split order.
  q.ksplit = 1;
  q.kspan = static_cast<int32_t>(K);
  if (q.regime == kStream) {
    constexpr int64_t kStage = 64, kMinSpan = 512, kTarget = 512;
    const int64_t units = max_tiles * col_tiles;
    int64_t split = (kTarget + units - 1) / units;
    split = std::min<int64_t>(split, std::max<int64_t>(1, K / kMinSpan));
    split = std::max<int64_t>(1, std::min<int64_t>(split, 8));
    int64_t span = (K + split - 1) / split;
    span = (span + kStage - 1) / kStage * kStage;
    split = (K + span - 1) / span;
    q.ksplit = static_cast<int32_t>(split);
    q.kspan = static_cast<int32_t>(span);
  }

  size_t off = 0;
  q.off_header = off;   off = align_up(off + sizeof(WsHeader), kRegionAlign);
  q.off_offsets = off;  off = align_up(off + sizeof(int64_t) * size_t(G + 1), kRegionAlign);
  q.off_tiles = off;    off = align_up(off + sizeof(MTile) * size_t(q.max_tiles), kRegionAlign);
  q.off_chunks = off;   off = align_up(off + sizeof(int32_t) * size_t(q.max_chunks + 1), kRegionAlign);
  q.off_inv = off;      off = align_up(off + sizeof(int32_t) * size_t(M), kRegionAlign);
  q.off_ori = off;      off = align_up(off + sizeof(int32_t) * size_t(M), kRegionAlign);
  q.table_bytes = off;
  q.off_ring = off;
  q.ring_bytes = q.ksplit > 1 ? size_t(q.ksplit) * size_t(M) * size_t(N) * sizeof(float) : 0;
  q.ring_rows = q.ksplit > 1 ? static_cast<int32_t>(q.ksplit * M) : 0;
  off = align_up(off + q.ring_bytes, kRegionAlign);
  q.total = off;
  *p = q;
  return PGG_OK;
}

pgg_status make_routing_plan(const pgg_moe_routing_desc* d, RoutePlan* p) {
  if (!d || !p) return PGG_ERR_INVALID_ARG;
  if (d->reserved != 0 || d->batch <= 0 || d->topk <= 0 || d->experts <= 0 || d->x_cols < 0)
    return PGG_ERR_INVALID_ARG;
  if (d->x_cols > 0 && (d->x_dtype < PGG_F32 || d->x_dtype > PGG_BF16)) return PGG_ERR_INVALID_ARG;
  if (d->topk > INT64_MAX / d->batch) return PGG_ERR_INVALID_ARG;
  const int64_t M = d->batch * d->topk;
  constexpr int64_t kBlockPos = 1024;
  if (M >= (int64_t(1) << 31) - 1 || d->experts > 8192) return PGG_ERR_UNSUPPORTED;
  // the gather splits a row into pieces of at least 4 KiB along a grid
  // dimension of at most 65535
  if (d->x_cols >= (int64_t(1) << 25)) return PGG_ERR_UNSUPPORTED;
  const int64_t nblocks = (M + kBlockPos - 1) / kBlockPos;
  if (nblocks * d->experts >= (int64_t(1) << 28)) return PGG_ERR_UNSUPPORTED;
  RoutePlan q{};
  q.M = M;
  q.G = d->experts;
  q.topk = d->topk;
  q.K = d->x_cols;
  q.dtype = d->x_dtype;
  q.nblocks = static_cast<int32_t>(nblocks);
  size_t off = 0;
  q.off_header = off;  off = align_up(off + sizeof(WsHeader), kRegionAlign);
  q.off_table = off;   off = align_up(off + sizeof(int32_t) * size_t(nblocks * q.G), kRegionAlign);
  q.off_bad = off;     off = align_up(off + sizeof(int64_t) * size_t(nblocks), kRegionAlign);
  q.off_offsets = off; off = align_up(off + sizeof(int64_t) * size_t(q.G + 1), kRegionAlign);
  q.off_rows = off;    off = align_up(off + sizeof(int32_t) * size_t(M), kRegionAlign);
  q.total = off;
  *p = q;
  return PGG_OK;
}

pgg_status make_unpermute_plan(const pgg_moe_unpermute_desc* d, UnpermutePlan* p) {
  if (!d || !p) return PGG_ERR_INVALID_ARG;
  if (d->reserved != 0 || d->batch <= 0 || d->topk <= 0 || d->hidden <= 0) return PGG_ERR_INVALID_ARG;
  if (d->row_idx_type != 0 && d->row_idx_type != 1) return PGG_ERR_INVALID_ARG;
  if (d->dtype < PGG_F32 || d->dtype > PGG_BF16) return PGG_ERR_INVALID_ARG;
  if (d->topk > INT64_MAX / d->batch) return PGG_ERR_INVALID_ARG;
  const int64_t M = d->batch * d->topk;
  if (M >= (int64_t(1) << 31) - 1 || d->batch >= (int64_t(1) << 31) ||
      d->hidden >= (int64_t(1) << 40) / M)
    return PGG_ERR_UNSUPPORTED;
  UnpermutePlan q{};
  q.M = M;
  q.batch = d->batch;
  q.topk = d->topk;
  q.H = d->hidden;
  q.dtype = d->dtype;
  q.row_idx_type = d->row_idx_type;
  size_t off = 0;
  q.off_header = off; off = align_up(off + sizeof(WsHeader), kRegionAlign);
  q.off_inv = off;    off = align_up(off + sizeof(int32_t) * size_t(M), kRegionAlign);
  q.off_ori = off;    off = align_up(off + sizeof(int32_t) * size_t(M), kRegionAlign);
  q.total = off;
  *p = q;
  return PGG_OK;
}

pgg_status make_dw_plan(const pgg_moe_fwd_desc* d, Plan* p) {
  Plan q;
  const pgg_status st = make_fwd_plan(d, &q);
  if (st != PGG_OK) return st;
  q.ksplit = 1;
  q.kspan = static_cast<int32_t>(q.N);
  q.ring_rows = 0;
  q.ring_bytes = 0;
  q.total = q.table_bytes;
  *p = q;
  return PGG_OK;
}

}  // namespace pgg
