/*
 * CPU oracle for the fused MoE backward that produces only d_x.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or
 * load this file or the library built from it; only the tests, the smoke
 * check and the CPU-baseline leg of the benchmark use it.  It shares no code
 * with the HIP implementation.
 *
 * What it computes (MoeInitRoutingGroupedMatmulGrad design page, §数学定义和公式):
 *
 *   Step 1  d_expanded_x[i,k] = sum_n d_y[i,n] * W[g(i),k,n]
 *   Step 2  d_x[b,k]          = sum over expanded rows i whose original
 *                               position p(i) satisfies p(i)/topK == b
 *                               of d_expanded_x[i,k]
 *
 * written out directly with explicit loops.  Inputs are decoded to double
 * (fp32 exactly; fp16 and bf16 by the decoders below), products and sums of
 * Step 1 are taken in double in ascending n, and the row is rounded once to
 * float (the page's cube output type is fp32, §2.6.2).  Step 2 is offered in
 * three orders:
 *   ORC_SLOT   float adds, d_x[b] starts at +0 and adds its rows for
 *              j = 0..topK-1 (the order the token-permute-grad kernel of the
 *              TileLang page uses: accumulate the topK gathered rows in fp32);
 *   ORC_ASCEND float adds in ascending expanded row i (the order of a plain
 *              scatter_add over i, the naive baseline of §4.1);
 *   ORC_EXACT  everything in double, no intermediate rounding; the reference
 *              for tolerance checks.
 * Every order is a correct result of the formula; they differ only by fp32
 * rounding.
 *
 * Index conventions (§1.2 I/O table and its notes): original position
 * p = b*topK + j; row_idx_type 0 means eri[i] is the original position of
 * expanded row i; row_idx_type 1 means eri[p] is the expanded row of original
 * position p.  group_list holds per-expert row counts (not a cumulative sum);
 * expert g owns expanded rows [off[g], off[g+1]).
 *
 * Build: gcc -O2 -ffp-contract=off -shared -fPIC -pthread (see build.py).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum {
  ORC_OK = 0,
  ORC_ERR_SHAPE = 1,        /* a shape / attribute constraint of §1.2 is violated */
  ORC_ERR_GROUP_NEG = 2,    /* a group_list entry is negative */
  ORC_ERR_GROUP_SUM = 3,    /* sum(group_list) != M */
  ORC_ERR_INDEX_RANGE = 4,  /* an eri entry is outside [0, M) */
  ORC_ERR_INDEX_DUP = 5,    /* eri is not a permutation of [0, M) */
  ORC_ERR_ALLOC = 6
};

enum { ORC_F32 = 0, ORC_F16 = 1, ORC_BF16 = 2 };
enum { ORC_SLOT = 0, ORC_ASCEND = 1, ORC_EXACT = 2 };

typedef struct {
  int64_t M, N, G, K, batch, topk;
  int32_t row_idx_type, dtype;
  const void* grad_y;         /* [M, N] row-major, dtype */
  const void* weight;         /* [G, K, N] row-major, dtype */
  const int64_t* eri;         /* [M] */
  const int64_t* group_list;  /* [G] */
} orc_problem;

/* ------------------------------------------------------------------------ */
/* decoders                                                                  */
/* ------------------------------------------------------------------------ */

/* IEEE-754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
double orc_half_to_double(uint16_t h) {
  int sign = (h >> 15) & 1;
  int e = (h >> 10) & 0x1f;
  int f = h & 0x3ff;
  double v;
  if (e == 0) {
    v = ldexp((double)f, -24);                 /* zero or subnormal: f * 2^-24 */
  } else if (e == 31) {
    v = f ? NAN : INFINITY;
  } else {
    v = ldexp((double)(f + 1024), e - 25);     /* (1 + f/1024) * 2^(e-15) */
  }
  return sign ? -v : v;
}

/* bfloat16 is the top half of a binary32. */
double orc_bf16_to_double(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float x;
  memcpy(&x, &u, sizeof x);
  return (double)x;
}

static inline double load_elem(int32_t dtype, const void* base, int64_t idx) {
  switch (dtype) {
    case ORC_F32: return (double)((const float*)base)[idx];
    case ORC_F16: return orc_half_to_double(((const uint16_t*)base)[idx]);
    default:      return orc_bf16_to_double(((const uint16_t*)base)[idx]);
  }
}

void orc_decode(int32_t dtype, const void* src, int64_t n, double* dst) {
  for (int64_t t = 0; t < n; ++t) dst[t] = load_elem(dtype, src, t);
}

/* ------------------------------------------------------------------------ */
/* constraints (§1.2 constraints table, §2.3 infershape checks)              */
/* ------------------------------------------------------------------------ */

/* Shapes: grad_y [M, Ny], weight [G, K, Nw], eri [L], group_list [Gl].
 * The page bounds L by batch <= L <= batch*topK and L >= M with M = batch*topK,
 * which leaves L == M.  Dtypes of grad_y and weight must match and be one of
 * the three float types. */
int orc_check(int64_t M, int64_t Ny, int64_t G, int64_t K, int64_t Nw, int64_t L,
              int64_t Gl, int64_t batch, int64_t topk, int32_t row_idx_type,
              int32_t dtype_y, int32_t dtype_w) {
  if (topk <= 0 || batch <= 0) return ORC_ERR_SHAPE;
  if (row_idx_type != 0 && row_idx_type != 1) return ORC_ERR_SHAPE;
  if (dtype_y != dtype_w || dtype_y < 0 || dtype_y > 2) return ORC_ERR_SHAPE;
  if (Ny != Nw) return ORC_ERR_SHAPE;
  if (Gl != G || G <= 0) return ORC_ERR_SHAPE;
  if (M != batch * topk) return ORC_ERR_SHAPE;
  if (L < batch || L > batch * topk || L < M) return ORC_ERR_SHAPE;
  if (M <= 0 || Ny <= 0 || K <= 0) return ORC_ERR_SHAPE;
  return ORC_OK;
}

/* off[g] = first expanded row of expert g; off[G] = M. */
int orc_offsets(int64_t G, const int64_t* group_list, int64_t M, int64_t* off) {
  off[0] = 0;
  for (int64_t g = 0; g < G; ++g) {
    if (group_list[g] < 0) return ORC_ERR_GROUP_NEG;
    off[g + 1] = off[g] + group_list[g];
  }
  return off[G] == M ? ORC_OK : ORC_ERR_GROUP_SUM;
}

/* The expert that owns expanded row i: the g with off[g] <= i < off[g+1]
 * (empty experts own no row). */
static int64_t expert_of_row(int64_t G, const int64_t* off, int64_t i) {
  int64_t g = 0;
  while (g + 1 < G && off[g + 1] <= i) ++g;
  return g;
}

/* ori[i] = original position of expanded row i; inv[p] = expanded row of
 * original position p.  Either encoding must be a permutation of [0, M). */
int orc_index(int64_t M, int32_t row_idx_type, const int64_t* eri, int64_t* ori, int64_t* inv) {
  for (int64_t t = 0; t < M; ++t) { ori[t] = -1; inv[t] = -1; }
  for (int64_t t = 0; t < M; ++t) {
    int64_t v = eri[t];
    if (v < 0 || v >= M) return ORC_ERR_INDEX_RANGE;
    if (row_idx_type == 0) {            /* t is an expanded row, v its original position */
      if (inv[v] != -1) return ORC_ERR_INDEX_DUP;
      ori[t] = v;
      inv[v] = t;
    } else {                            /* t is an original position, v its expanded row */
      if (ori[v] != -1) return ORC_ERR_INDEX_DUP;
      inv[t] = v;
      ori[v] = t;
    }
  }
  return ORC_OK;
}

/* Full validation: shapes are checked by the caller with orc_check. */
static int prepare(const orc_problem* pr, int64_t* off, int64_t* ori, int64_t* inv) {
  int rc = orc_offsets(pr->G, pr->group_list, pr->M, off);
  if (rc) return rc;
  return orc_index(pr->M, pr->row_idx_type, pr->eri, ori, inv);
}

/* ------------------------------------------------------------------------ */
/* Step 1 for one expanded row                                               */
/* ------------------------------------------------------------------------ */

/* dex64[k] = sum_n d_y[i,n] * W[g,k,n] in double (ascending n);
 * abs64[k] = sum_n |d_y[i,n]| * |W[g,k,n]| (for error bounds). */
static void dex_row(const orc_problem* pr, int64_t i, int64_t g, double* dyrow,
                    double* dex64, double* abs64) {
  const int64_t N = pr->N, K = pr->K;
  for (int64_t n = 0; n < N; ++n) dyrow[n] = load_elem(pr->dtype, pr->grad_y, i * N + n);
  for (int64_t k = 0; k < K; ++k) {
    const int64_t wbase = (g * K + k) * N;
    double s = 0.0, a = 0.0;
    for (int64_t n = 0; n < N; ++n) {
      double w = load_elem(pr->dtype, pr->weight, wbase + n);
      s += dyrow[n] * w;
      if (abs64) a += fabs(dyrow[n]) * fabs(w);
    }
    dex64[k] = s;
    if (abs64) abs64[k] = a;
  }
}

/* ------------------------------------------------------------------------ */
/* threading helper                                                          */
/* ------------------------------------------------------------------------ */

typedef struct {
  const orc_problem* pr;
  const int64_t* off;
  const int64_t* ori;
  const int64_t* inv;
  const int64_t* tokens;  /* token subset (orc_dx_tokens) */
  int64_t ntok;
  float* dex32;
  double* dex64;
  double* abs64;
  float* dx32;
  double* dx64;
  double* absdot;
  int64_t begin, end;
  int failed;
} work_t;

static int run_threads(void* (*fn)(void*), work_t* proto, int64_t total, int nthreads) {
  if (nthreads < 1) nthreads = 1;
  if (nthreads > total) nthreads = (int)(total > 0 ? total : 1);
  pthread_t* th = (pthread_t*)calloc((size_t)nthreads, sizeof(pthread_t));
  work_t* w = (work_t*)calloc((size_t)nthreads, sizeof(work_t));
  if (!th || !w) { free(th); free(w); return ORC_ERR_ALLOC; }
  for (int t = 0; t < nthreads; ++t) {
    w[t] = *proto;
    w[t].begin = total * t / nthreads;
    w[t].end = total * (t + 1) / nthreads;
    pthread_create(&th[t], NULL, fn, &w[t]);
  }
  int failed = 0;
  for (int t = 0; t < nthreads; ++t) {
    pthread_join(th[t], NULL);
    failed |= w[t].failed;
  }
  free(th);
  free(w);
  return failed ? ORC_ERR_ALLOC : ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Step 1 over all rows                                                      */
/* ------------------------------------------------------------------------ */

static void* dex_worker(void* arg) {
  work_t* w = (work_t*)arg;
  const orc_problem* pr = w->pr;
  double* dyrow = (double*)malloc(sizeof(double) * (size_t)pr->N);
  double* row64 = (double*)malloc(sizeof(double) * (size_t)pr->K);
  double* rowabs = w->abs64 ? (double*)malloc(sizeof(double) * (size_t)pr->K) : NULL;
  if (!dyrow || !row64 || (w->abs64 && !rowabs)) { w->failed = 1; goto out; }
  for (int64_t i = w->begin; i < w->end; ++i) {
    int64_t g = expert_of_row(pr->G, w->off, i);
    dex_row(pr, i, g, dyrow, row64, rowabs);
    for (int64_t k = 0; k < pr->K; ++k) {
      w->dex32[i * pr->K + k] = (float)row64[k];
      if (w->dex64) w->dex64[i * pr->K + k] = row64[k];
      if (w->abs64) w->abs64[i * pr->K + k] = rowabs[k];
    }
  }
out:
  free(dyrow); free(row64); free(rowabs);
  return NULL;
}

/* d_expanded_x (Step 1) for every expanded row.  dex64 / abs64 may be NULL. */
int orc_dex(const orc_problem* pr, float* dex32, double* dex64, double* abs64, int nthreads) {
  int64_t* off = (int64_t*)malloc(sizeof(int64_t) * (size_t)(pr->G + 1));
  int64_t* ori = (int64_t*)malloc(sizeof(int64_t) * (size_t)pr->M);
  int64_t* inv = (int64_t*)malloc(sizeof(int64_t) * (size_t)pr->M);
  int rc = ORC_ERR_ALLOC;
  if (off && ori && inv) {
    rc = prepare(pr, off, ori, inv);
    if (rc == ORC_OK) {
      work_t proto = {0};
      proto.pr = pr; proto.off = off; proto.dex32 = dex32; proto.dex64 = dex64; proto.abs64 = abs64;
      rc = run_threads(dex_worker, &proto, pr->M, nthreads);
    }
  }
  free(off); free(ori); free(inv);
  return rc;
}

/* ------------------------------------------------------------------------ */
/* Step 2 over all tokens, from a materialised d_expanded_x                  */
/* ------------------------------------------------------------------------ */

/* mode ORC_SLOT: dx32[b,k] = (((+0 + dex[i_0,k]) + dex[i_1,k]) + ...) with
 *                i_j = inv[b*topK + j], float adds.
 * mode ORC_ASCEND: float adds into dx32[ori[i]/topK] for i = 0..M-1.
 * mode ORC_EXACT: dx64[b,k] = sum_j dex64[i_j,k] in double (slot order).
 * absdot (optional, with abs64): sum_j abs64[i_j,k]. */
int orc_scatter(const orc_problem* pr, const float* dex32, const double* dex64,
                const double* abs64, int32_t mode, float* dx32, double* dx64, double* absdot) {
  int64_t* off = (int64_t*)malloc(sizeof(int64_t) * (size_t)(pr->G + 1));
  int64_t* ori = (int64_t*)malloc(sizeof(int64_t) * (size_t)pr->M);
  int64_t* inv = (int64_t*)malloc(sizeof(int64_t) * (size_t)pr->M);
  int rc = ORC_ERR_ALLOC;
  if (!(off && ori && inv)) goto out;
  rc = prepare(pr, off, ori, inv);
  if (rc) goto out;
  const int64_t K = pr->K, topk = pr->topk, batch = pr->batch;
  if (mode == ORC_ASCEND) {
    for (int64_t t = 0; t < batch * K; ++t) dx32[t] = 0.0f;
    for (int64_t i = 0; i < pr->M; ++i) {
      int64_t b = ori[i] / topk;
      for (int64_t k = 0; k < K; ++k) dx32[b * K + k] = dx32[b * K + k] + dex32[i * K + k];
    }
  } else {
    for (int64_t b = 0; b < batch; ++b) {
      for (int64_t k = 0; k < K; ++k) {
        float a32 = 0.0f;
        double a64 = 0.0, aa = 0.0;
        for (int64_t j = 0; j < topk; ++j) {
          int64_t i = inv[b * topk + j];
          if (mode == ORC_SLOT) a32 = a32 + dex32[i * K + k];
          else a64 += dex64[i * K + k];
          if (absdot && abs64) aa += abs64[i * K + k];
        }
        if (mode == ORC_SLOT) dx32[b * K + k] = a32;
        else dx64[b * K + k] = a64;
        if (absdot && abs64) absdot[b * K + k] = aa;
      }
    }
  }
  rc = ORC_OK;
out:
  free(off); free(ori); free(inv);
  return rc;
}

/* ------------------------------------------------------------------------ */
/* Both steps for a subset of tokens, one dex row at a time                  */
/* ------------------------------------------------------------------------ */

static void* tokens_worker(void* arg) {
  work_t* w = (work_t*)arg;
  const orc_problem* pr = w->pr;
  const int64_t K = pr->K;
  double* dyrow = (double*)malloc(sizeof(double) * (size_t)pr->N);
  double* row64 = (double*)malloc(sizeof(double) * (size_t)K);
  double* rowabs = (double*)malloc(sizeof(double) * (size_t)K);
  if (!dyrow || !row64 || !rowabs) { w->failed = 1; goto out; }
  for (int64_t t = w->begin; t < w->end; ++t) {
    int64_t b = w->tokens[t];
    float* o32 = w->dx32 ? w->dx32 + t * K : NULL;
    double* o64 = w->dx64 ? w->dx64 + t * K : NULL;
    double* oab = w->absdot ? w->absdot + t * K : NULL;
    for (int64_t k = 0; k < K; ++k) {
      if (o32) o32[k] = 0.0f;
      if (o64) o64[k] = 0.0;
      if (oab) oab[k] = 0.0;
    }
    for (int64_t j = 0; j < pr->topk; ++j) {
      int64_t i = w->inv[b * pr->topk + j];
      int64_t g = expert_of_row(pr->G, w->off, i);
      dex_row(pr, i, g, dyrow, row64, oab ? rowabs : NULL);
      for (int64_t k = 0; k < K; ++k) {
        if (o32) o32[k] = o32[k] + (float)row64[k];
        if (o64) o64[k] += row64[k];
        if (oab) oab[k] += rowabs[k];
      }
    }
  }
out:
  free(dyrow); free(row64); free(rowabs);
  return NULL;
}

/* d_x rows for the listed tokens: dx32 in slot order (Step 1 rounded to
 * float, float adds), dx64 exact, absdot the matching sum of |terms|.
 * Outputs are [ntok, K]; any of them may be NULL. */
int orc_dx_tokens(const orc_problem* pr, const int64_t* tokens, int64_t ntok,
                  float* dx32, double* dx64, double* absdot, int nthreads) {
  int64_t* off = (int64_t*)malloc(sizeof(int64_t) * (size_t)(pr->G + 1));
  int64_t* ori = (int64_t*)malloc(sizeof(int64_t) * (size_t)pr->M);
  int64_t* inv = (int64_t*)malloc(sizeof(int64_t) * (size_t)pr->M);
  int rc = ORC_ERR_ALLOC;
  if (off && ori && inv) {
    rc = prepare(pr, off, ori, inv);
    if (rc == ORC_OK) {
      for (int64_t t = 0; t < ntok; ++t)
        if (tokens[t] < 0 || tokens[t] >= pr->batch) { rc = ORC_ERR_SHAPE; break; }
    }
    if (rc == ORC_OK) {
      work_t proto = {0};
      proto.pr = pr; proto.off = off; proto.ori = ori; proto.inv = inv;
      proto.tokens = tokens; proto.ntok = ntok;
      proto.dx32 = dx32; proto.dx64 = dx64; proto.absdot = absdot;
      rc = run_threads(tokens_worker, &proto, ntok, nthreads);
    }
  }
  free(off); free(ori); free(inv);
  return rc;
}

/* ------------------------------------------------------------------------ */
/* Column sums over every expanded row, for selected output columns          */
/* ------------------------------------------------------------------------ */

/* For each listed column k: colsum[t] = sum_i sum_n d_y[i,n] * W[g(i),k,n]
 * and colabs[t] = the same sum of |terms|, both in double.  Step 2 only
 * regroups the rows by token, so the sum over all tokens of d_x[:, k] equals
 * this sum over all expanded rows of d_expanded_x[:, k] (the column-sum
 * invariant); it holds at any size and touches every row. */
typedef struct {
  const orc_problem* pr;
  const int64_t* off;
  const int64_t* cols;
  int64_t ncols;
  double* sum;   /* [nthreads][ncols] partials */
  double* asum;
  int64_t begin, end;
} colsum_work_t;

static void* colsum_worker(void* arg) {
  colsum_work_t* w = (colsum_work_t*)arg;
  const orc_problem* pr = w->pr;
  for (int64_t i = w->begin; i < w->end; ++i) {
    int64_t g = expert_of_row(pr->G, w->off, i);
    for (int64_t t = 0; t < w->ncols; ++t) {
      const int64_t k = w->cols[t];
      double s = 0.0, a = 0.0;
      for (int64_t n = 0; n < pr->N; ++n) {
        double y = load_elem(pr->dtype, pr->grad_y, i * pr->N + n);
        double x = load_elem(pr->dtype, pr->weight, (g * pr->K + k) * pr->N + n);
        s += y * x;
        a += fabs(y) * fabs(x);
      }
      w->sum[t] += s;
      w->asum[t] += a;
    }
  }
  return NULL;
}

int orc_colsum(const orc_problem* pr, const int64_t* cols, int64_t ncols, double* colsum,
               double* colabs, int nthreads) {
  int64_t* off = (int64_t*)malloc(sizeof(int64_t) * (size_t)(pr->G + 1));
  if (!off) return ORC_ERR_ALLOC;
  int rc = orc_offsets(pr->G, pr->group_list, pr->M, off);
  if (rc) { free(off); return rc; }
  for (int64_t t = 0; t < ncols; ++t)
    if (cols[t] < 0 || cols[t] >= pr->K) { free(off); return ORC_ERR_SHAPE; }
  if (nthreads < 1) nthreads = 1;
  if (nthreads > pr->M) nthreads = (int)pr->M;
  pthread_t* th = (pthread_t*)calloc((size_t)nthreads, sizeof(pthread_t));
  colsum_work_t* w = (colsum_work_t*)calloc((size_t)nthreads, sizeof(colsum_work_t));
  double* part = (double*)calloc((size_t)nthreads * (size_t)ncols * 2, sizeof(double));
  if (!th || !w || !part) { free(off); free(th); free(w); free(part); return ORC_ERR_ALLOC; }
  for (int t = 0; t < nthreads; ++t) {
    w[t].pr = pr; w[t].off = off; w[t].cols = cols; w[t].ncols = ncols;
    w[t].sum = part + (size_t)t * (size_t)ncols * 2;
    w[t].asum = w[t].sum + ncols;
    w[t].begin = pr->M * t / nthreads;
    w[t].end = pr->M * (t + 1) / nthreads;
    pthread_create(&th[t], NULL, colsum_worker, &w[t]);
  }
  for (int t = 0; t < nthreads; ++t) pthread_join(th[t], NULL);
  for (int64_t c = 0; c < ncols; ++c) {
    double s = 0.0, a = 0.0;
    for (int t = 0; t < nthreads; ++t) { s += w[t].sum[c]; a += w[t].asum[c]; }
    colsum[c] = s;
    if (colabs) colabs[c] = a;
  }
  free(off); free(th); free(w); free(part);
  return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Both steps for every token, on a subset of output columns                 */
/* ------------------------------------------------------------------------ */

/* For every token b and each listed column cols[t]: Step 1 for the token's
 * expanded rows at that column only (a double dot product over n, ascending,
 * rounded once to float), then Step 2 in slot order j = 0..topK-1:
 *   dx32[b,t] = (((+0 + (float)e_0) + (float)e_1) + ...),  e_j the Step 1
 *               value of row inv[b*topK + j] at column cols[t];
 *   dx64[b,t] = sum_j e_j in double;  absdot[b,t] = the matching sum of
 *               |d_y|·|W| over every term.
 * The same values as orc_dx_tokens at those columns, for all tokens, at a
 * cost of M * ncols * N multiply-adds. */
typedef struct {
  const orc_problem* pr;
  const int64_t* off;
  const int64_t* inv;
  const int64_t* cols;
  int64_t ncols;
  float* dx32;
  double* dx64;
  double* absdot;
  int64_t begin, end;
  int failed;
} cols_work_t;

static void* cols_worker(void* arg) {
  cols_work_t* w = (cols_work_t*)arg;
  const orc_problem* pr = w->pr;
  const int64_t N = pr->N, K = pr->K, nc = w->ncols;
  double* dyrow = (double*)malloc(sizeof(double) * (size_t)N);
  if (!dyrow) { w->failed = 1; return NULL; }
  for (int64_t b = w->begin; b < w->end; ++b) {
    for (int64_t t = 0; t < nc; ++t) {
      w->dx32[b * nc + t] = 0.0f;
      w->dx64[b * nc + t] = 0.0;
      w->absdot[b * nc + t] = 0.0;
    }
    for (int64_t j = 0; j < pr->topk; ++j) {
      const int64_t i = w->inv[b * pr->topk + j];
      const int64_t g = expert_of_row(pr->G, w->off, i);
      for (int64_t n = 0; n < N; ++n) dyrow[n] = load_elem(pr->dtype, pr->grad_y, i * N + n);
      for (int64_t t = 0; t < nc; ++t) {
        const int64_t wbase = (g * K + w->cols[t]) * N;
        double s = 0.0, a = 0.0;
        for (int64_t n = 0; n < N; ++n) {
          const double x = load_elem(pr->dtype, pr->weight, wbase + n);
          s += dyrow[n] * x;
          a += fabs(dyrow[n]) * fabs(x);
        }
        w->dx32[b * nc + t] = w->dx32[b * nc + t] + (float)s;
        w->dx64[b * nc + t] += s;
        w->absdot[b * nc + t] += a;
      }
    }
  }
  free(dyrow);
  return NULL;
}

/* Outputs are [batch, ncols]. */
int orc_dx_cols(const orc_problem* pr, const int64_t* cols, int64_t ncols, float* dx32,
                double* dx64, double* absdot, int nthreads) {
  for (int64_t t = 0; t < ncols; ++t)
    if (cols[t] < 0 || cols[t] >= pr->K) return ORC_ERR_SHAPE;
  int64_t* off = (int64_t*)malloc(sizeof(int64_t) * (size_t)(pr->G + 1));
  int64_t* ori = (int64_t*)malloc(sizeof(int64_t) * (size_t)pr->M);
  int64_t* inv = (int64_t*)malloc(sizeof(int64_t) * (size_t)pr->M);
  int rc = ORC_ERR_ALLOC;
  if (off && ori && inv) rc = prepare(pr, off, ori, inv);
  if (rc == ORC_OK) {
    if (nthreads < 1) nthreads = 1;
    if (nthreads > pr->batch) nthreads = (int)pr->batch;
    pthread_t* th = (pthread_t*)calloc((size_t)nthreads, sizeof(pthread_t));
    cols_work_t* w = (cols_work_t*)calloc((size_t)nthreads, sizeof(cols_work_t));
    if (!th || !w) {
      rc = ORC_ERR_ALLOC;
    } else {
      for (int t = 0; t < nthreads; ++t) {
        w[t].pr = pr; w[t].off = off; w[t].inv = inv; w[t].cols = cols; w[t].ncols = ncols;
        w[t].dx32 = dx32; w[t].dx64 = dx64; w[t].absdot = absdot;
        w[t].begin = pr->batch * t / nthreads;
        w[t].end = pr->batch * (t + 1) / nthreads;
        pthread_create(&th[t], NULL, cols_worker, &w[t]);
      }
      for (int t = 0; t < nthreads; ++t) {
        pthread_join(th[t], NULL);
        if (w[t].failed) rc = ORC_ERR_ALLOC;
      }
    }
    free(th); free(w);
  }
  free(off); free(ori); free(inv);
  return rc;
}
