/*
 * sgqa_oracle.c -- plain, slow CPU definition of the blockwise Sparse GQA path.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may call this code: only the tests, the
 * smoke check and the CPU-baseline leg of the benchmark load it. It shares no code, header, table
 * or helper with the HIP library; it is written straight from the method's description:
 *
 *   "Inside Step 5 Preview" (StepFun blog), section "Sparse GQA":
 *     paragraph "Reducing indexer's cost"        -> block compression of the index keys (orc_compress)
 *                                                    and block-level indexer + top-k (orc_index_topk)
 *     paragraph "Efficient implementation ..."   -> union of adjacent prefill queries (orc_union)
 *     paragraph "Trade-off between top-k and
 *                block size"                      -> k tokens = k/B blocks; token coverage (orc_coverage)
 *     Figure 3 caption                            -> shared index keys, per-KV-group selection, own
 *                                                    block read causally (orc_attend, orc_decode)
 *     the pages' FP8 KV cache (deployment notes)  -> orc_fp8_e4m3_to_f64, orc_decode_f8
 *     training use of Sparse GQA (the pages train
 *     with it; the gradient is that of the same
 *     attention)                                  -> orc_attend_bwd, orc_attend_bwd_part (the
 *                                                    same gradient on sampled rows / keys)
 *     "Efficient implementation ..." read as
 *     scheduling only (each query keeps its own
 *     selection)                                  -> orc_attend_sel
 *
 * The pages do not fix the indexer's form. The reading used here (and by the library) is:
 *   block key   kbar[b] = bf16_rne(mean of the B index keys of block b)       (complete blocks only)
 *   score       s(i,g,b) = sum_h w[g][h] * max(0, <qi[i][g][h], kbar[b]>)      for b < c(i) = floor(i/B)
 *   selection   first min(K_B, c(i)) candidates in the order (s descending, b ascending)
 *   attended    Sel(i,g) plus the own block c(i); token-level causal mask j <= i
 *   union       every query of tile t = floor(i/Tq) attends over the union of the tile's sets
 *
 * Arithmetic: fp64 everywhere except where the method fixes a storage type (block keys are bf16).
 * Loops are the definitions written out; OpenMP only splits independent rows across threads, the
 * arithmetic inside a row is sequential, so results do not depend on the thread count.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ---------------------------------------------------------------- bf16 <-> fp64 ---------------- */

/* bf16 is the upper half of an IEEE binary32; widening is exact. */
double orc_bf16_to_f64(uint16_t h) {
  uint32_t u = ((uint32_t)h) << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* Round a double to the nearest bf16 (8 significant bits, exponent range of binary32),
 * ties to even, by the definition: scale so that one unit in the last place is 1, round with
 * rint() (default rounding mode = nearest-even), scale back. Overflow gives +-inf; NaN stays NaN. */
uint16_t orc_f64_to_bf16(double x) {
  if (isnan(x)) return 0x7FC0;
  double r;
  if (x == 0.0 || isinf(x)) {
    r = x;
  } else {
    int e;
    frexp(x, &e);                  /* |x| = m * 2^e with 0.5 <= m < 1, leading bit 2^(e-1) */
    int ulp_exp = (e - 1) - 7;     /* 7 stored fraction bits */
    if (ulp_exp < -133) ulp_exp = -133;  /* subnormal spacing of binary32/bf16: 2^-126 * 2^-7 */
    r = ldexp(rint(ldexp(x, -ulp_exp)), ulp_exp);
    if (fabs(r) > 3.3895313892515355e38) r = copysign(INFINITY, x);  /* largest bf16 = 0x7F7F */
  }
  float f = (float)r;             /* exact: r is representable in bf16, hence in binary32 */
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  return (uint16_t)(u >> 16);
}

/* ---------------------------------------------------------------- compress --------------------- */

/* kbar[s][b][d] = bf16_rne( (sum_{j<B} ki[s][b*B+j][d]) / B ) for b < floor(N/B).
 * "Reducing indexer's cost": B adjacent historical positions share one block representation.
 * The sum of B bf16 values is formed in fp64 and rounded once to bf16. */
void orc_compress(int S, int N, int dI, int B, const uint16_t* ki, uint16_t* kbar) {
  int NB = N / B;
#pragma omp parallel for collapse(2) schedule(static)
  for (int s = 0; s < S; ++s) {
    for (int b = 0; b < NB; ++b) {
      for (int d = 0; d < dI; ++d) {
        double sum = 0.0;
        for (int j = 0; j < B; ++j) sum += orc_bf16_to_f64(ki[((size_t)s * N + (size_t)b * B + j) * dI + d]);
        kbar[((size_t)s * NB + b) * dI + d] = orc_f64_to_bf16(sum / (double)B);
      }
    }
  }
}

/* ---------------------------------------------------------------- scores and top-k ------------- */

/* Scores of one (query, group) row against candidate blocks 0..nc-1.
 *   qi_row [HI][dI] bf16, w_row [HI] fp32, kbar [>= nc][dI] bf16, out s[nc].
 * A score of -0 is replaced by +0 so that zero scores compare equal. */
void orc_block_scores(int HI, int dI, const uint16_t* qi_row, const float* w_row, const uint16_t* kbar,
                      int nc, double* s) {
  for (int b = 0; b < nc; ++b) {
    double total = 0.0;
    for (int h = 0; h < HI; ++h) {
      double dot = 0.0;
      for (int d = 0; d < dI; ++d)
        dot += orc_bf16_to_f64(qi_row[h * dI + d]) * orc_bf16_to_f64(kbar[(size_t)b * dI + d]);
      double relu = dot > 0.0 ? dot : 0.0;
      total += (double)w_row[h] * relu;
    }
    if (total == 0.0) total = 0.0;  /* -0 -> +0 */
    s[b] = total;
  }
}

typedef struct {
  double s;
  int32_t b;
} orc_cand;

/* Candidate order of the selection: higher score first, lower block id on equal scores. */
static int orc_cand_cmp(const void* pa, const void* pb) {
  const orc_cand* a = (const orc_cand*)pa;
  const orc_cand* b = (const orc_cand*)pb;
  if (a->s > b->s) return -1;
  if (a->s < b->s) return 1;
  return (a->b < b->b) ? -1 : (a->b > b->b);
}

static int orc_int_cmp(const void* pa, const void* pb) {
  int32_t a = *(const int32_t*)pa, b = *(const int32_t*)pb;
  return (a > b) - (a < b);
}

/* Keep the first min(KB, nc) candidates of the order above; write them ascending by block id,
 * then -1 up to KB entries. */
void orc_select(int nc, const double* s, int KB, int32_t* out) {
  orc_cand* c = (orc_cand*)malloc(sizeof(orc_cand) * (size_t)(nc > 0 ? nc : 1));
  for (int b = 0; b < nc; ++b) {
    c[b].s = s[b];
    c[b].b = b;
  }
  qsort(c, (size_t)nc, sizeof(orc_cand), orc_cand_cmp);
  int m = nc < KB ? nc : KB;
  for (int x = 0; x < m; ++x) out[x] = c[x].b;
  qsort(out, (size_t)m, sizeof(int32_t), orc_int_cmp);
  for (int x = m; x < KB; ++x) out[x] = -1;
  free(c);
}

/* Sel(i,g) for the queries rows[0..nrows) (rows == NULL: all queries 0..N-1, nrows = N).
 *   qi [N][G][HI][dI] bf16, w [G][HI] fp32, kbar [floor(N/B)][dI] bf16
 *   topk out [G][nrows][KB] int32 (ascending block ids, -1 padding). */
void orc_index_topk(int N, int G, int HI, int dI, int B, int KB, const uint16_t* qi, const float* w,
                    const uint16_t* kbar, int nrows, const int32_t* rows, int32_t* topk) {
#pragma omp parallel for collapse(2) schedule(dynamic, 4)
  for (int g = 0; g < G; ++g) {
    for (int x = 0; x < nrows; ++x) {
      int i = rows ? rows[x] : x;
      int nc = i / B; /* c(i): the complete blocks before the query's own block */
      double* s = (double*)malloc(sizeof(double) * (size_t)(nc > 0 ? nc : 1));
      orc_block_scores(HI, dI, qi + ((size_t)i * G + g) * HI * dI, w + (size_t)g * HI, kbar, nc, s);
      orc_select(nc, s, KB, topk + ((size_t)g * nrows + x) * KB);
      free(s);
    }
  }
  (void)N;
}

/* Number of (query, candidate block) pairs the indexer scores for one group: sum_i floor(i/B). */
long long orc_scored_pairs(int N, int B) {
  long long total = 0;
  for (int i = 0; i < N; ++i) total += i / B;
  return total;
}

/* ---------------------------------------------------------------- union ------------------------ */

/* U(t,g) = union over i in [t*Tq, min((t+1)*Tq, N)) of Sel(i,g) and the own block floor(i/B).
 *   topk [G][N][KB] -> umask [G][T][W] (bit b%32 of word b/32), ucount [G][T] = |U(t,g)|. */
void orc_union(int N, int G, int B, int KB, int Tq, const int32_t* topk, uint32_t* umask, int32_t* ucount) {
  int T = (N + Tq - 1) / Tq;
  int NBc = (N + B - 1) / B;
  int W = (NBc + 31) / 32;
#pragma omp parallel for collapse(2) schedule(static)
  for (int g = 0; g < G; ++g) {
    for (int t = 0; t < T; ++t) {
      uint32_t* m = umask + ((size_t)g * T + t) * W;
      for (int w = 0; w < W; ++w) m[w] = 0;
      int i_end = (t + 1) * Tq < N ? (t + 1) * Tq : N;
      for (int i = t * Tq; i < i_end; ++i) {
        const int32_t* sel = topk + ((size_t)g * N + i) * KB;
        for (int x = 0; x < KB; ++x)
          if (sel[x] >= 0) m[sel[x] / 32] |= 1u << (sel[x] % 32);
        int own = i / B;
        m[own / 32] |= 1u << (own % 32);
      }
      int count = 0;
      for (int b = 0; b < NBc; ++b) count += (m[b / 32] >> (b % 32)) & 1u;
      ucount[(size_t)g * T + t] = count;
    }
  }
}

/* ---------------------------------------------------------------- attention -------------------- */

/* Softmax attention of one query vector over an explicit token list, fp64.
 *   qv [D] bf16, k/v rows kv_base + j*D for j in toks[0..nt), out [D] fp64. */
static void orc_attend_list(int D, double scale, const uint16_t* qv, const uint16_t* kbase,
                            const uint16_t* vbase, const int32_t* toks, int nt, double* logit, double* out) {
  double mx = -INFINITY;
  for (int x = 0; x < nt; ++x) {
    const uint16_t* kr = kbase + (size_t)toks[x] * D;
    double dot = 0.0;
    for (int d = 0; d < D; ++d) dot += orc_bf16_to_f64(qv[d]) * orc_bf16_to_f64(kr[d]);
    logit[x] = scale * dot;
    if (logit[x] > mx) mx = logit[x];
  }
  double den = 0.0;
  for (int x = 0; x < nt; ++x) {
    logit[x] = exp(logit[x] - mx);
    den += logit[x];
  }
  for (int d = 0; d < D; ++d) out[d] = 0.0;
  for (int x = 0; x < nt; ++x) {
    const uint16_t* vr = vbase + (size_t)toks[x] * D;
    double p = logit[x] / den;
    for (int d = 0; d < D; ++d) out[d] += p * orc_bf16_to_f64(vr[d]);
  }
}

/* Prefill attention for the queries rows[0..nrows) (NULL: all).
 *   q [N][Hq][D], k/v [G][N][D] bf16, umask [G][T][W] -> out [nrows][Hq][D] fp64.
 * For head h of group g = h / (Hq/G) the token set is J = { j <= i : block floor(j/B) in U(t,g) }.
 * scale <= 0 means 1/sqrt(D). */
void orc_attend(int N, int Hq, int G, int D, int B, int Tq, double scale, const uint16_t* q,
                const uint16_t* k, const uint16_t* v, const uint32_t* umask, int nrows, const int32_t* rows,
                double* out) {
  int T = (N + Tq - 1) / Tq;
  int NBc = (N + B - 1) / B;
  int W = (NBc + 31) / 32;
  int r = Hq / G;
  if (scale <= 0.0) scale = 1.0 / sqrt((double)D);
#pragma omp parallel for schedule(dynamic, 1)
  for (int x = 0; x < nrows; ++x) {
    int i = rows ? rows[x] : x;
    int t = i / Tq;
    int32_t* toks = (int32_t*)malloc(sizeof(int32_t) * (size_t)(i + 1));
    double* logit = (double*)malloc(sizeof(double) * (size_t)(i + 1));
    for (int g = 0; g < G; ++g) {
      const uint32_t* m = umask + ((size_t)g * T + t) * W;
      int nt = 0;
      for (int j = 0; j <= i; ++j)
        if ((m[(j / B) / 32] >> ((j / B) % 32)) & 1u) toks[nt++] = j;
      for (int hh = 0; hh < r; ++hh) {
        int h = g * r + hh;
        orc_attend_list(D, scale, q + ((size_t)i * Hq + h) * D, k + (size_t)g * N * D, v + (size_t)g * N * D,
                        toks, nt, logit, out + ((size_t)x * Hq + h) * D);
      }
    }
    free(toks);
    free(logit);
  }
}

/* Prefill attention where every query keeps its own selection: the second reading of "Efficient
 * implementation of sparse attention", in which grouping adjacent queries only organises the work
 * and changes no query's attended set. For head h of group g = h / (Hq/G) the token set is
 *   J = { j <= i : floor(j/B) in Sel(i,g) or floor(j/B) = floor(i/B) }      (Figure 3 caption)
 * topk [G][N][KB] (ascending ids, -1 padded) -> out [nrows][Hq][D] fp64 for rows[0..nrows) (NULL:
 * all). scale <= 0 means 1/sqrt(D). */
void orc_attend_sel(int N, int Hq, int G, int D, int B, int KB, double scale, const uint16_t* q,
                    const uint16_t* k, const uint16_t* v, const int32_t* topk, int nrows, const int32_t* rows,
                    double* out) {
  int r = Hq / G;
  if (scale <= 0.0) scale = 1.0 / sqrt((double)D);
#pragma omp parallel for schedule(dynamic, 1)
  for (int x = 0; x < nrows; ++x) {
    int i = rows ? rows[x] : x;
    int32_t* toks = (int32_t*)malloc(sizeof(int32_t) * (size_t)(i + 1));
    double* logit = (double*)malloc(sizeof(double) * (size_t)(i + 1));
    for (int g = 0; g < G; ++g) {
      const int32_t* sel = topk + ((size_t)g * N + i) * KB;
      int nt = 0;
      for (int j = 0; j <= i; ++j) {
        int b = j / B, in = b == i / B;
        for (int e = 0; e < KB && !in; ++e) in = sel[e] == b;
        if (in) toks[nt++] = j;
      }
      for (int hh = 0; hh < r; ++hh) {
        int h = g * r + hh;
        orc_attend_list(D, scale, q + ((size_t)i * Hq + h) * D, k + (size_t)g * N * D, v + (size_t)g * N * D,
                        toks, nt, logit, out + ((size_t)x * Hq + h) * D);
      }
    }
    free(toks);
    free(logit);
  }
}

/* Gradient of the prefill attention (union reading, token sets as in orc_attend) for an upstream
 * gradient dout [N][Hq][D] bf16: with p the row's softmax over J, o = sum_j p_j v_j,
 *   dv_j += p_j * dout_i,   dp_j = <dout_i, v_j>,   ds_j = p_j * (dp_j - <dout_i, o_i>),
 *   dq_i += scale * sum_j ds_j k_j,   dk_j += scale * ds_j q_i
 * (the gradient of softmax attention, with the heads of a group summed into its K/V gradients).
 * Two kinds of independent outputs: per row (softmax max, denominator, delta = <dout_i, o_i>, and
 * dq_i), then per key (dk_j, dv_j summed over the rows whose set holds j, in ascending row order). */

/* Row i's token set J(i,g) (tokens j <= i whose block is in U(tile(i), g)) into toks; returns its
 * size. */
static int orc_row_tokens(int i, int B, const uint32_t* mrow, int32_t* toks) {
  int nt = 0;
  for (int j = 0; j <= i; ++j)
    if ((mrow[(j / B) / 32] >> ((j / B) % 32)) & 1u) toks[nt++] = j;
  return nt;
}

/* One (row, head): qi, di = the row's q and dout (fp64), kg, vg = the group's keys and values [N][D]
 * (fp64), toks[0..nt) its token set; lg, o: scratch of nt and D doubles. Returns the softmax
 * maximum, denominator and delta; writes dq_i to dqi unless it is NULL. */
static void orc_bwd_row(int D, double scale, const double* qi, const double* di, const double* kg, const double* vg,
                        const int32_t* toks, int nt, double* lg, double* o, double* mx_out, double* den_out,
                        double* del_out, double* dqi) {
  double mx = -INFINITY;
  for (int x = 0; x < nt; ++x) {
    const double* kr = kg + (size_t)toks[x] * D;
    double dot = 0.0;
    for (int d = 0; d < D; ++d) dot += qi[d] * kr[d];
    lg[x] = scale * dot;
    if (lg[x] > mx) mx = lg[x];
  }
  double den = 0.0;
  for (int x = 0; x < nt; ++x) den += exp(lg[x] - mx);
  for (int d = 0; d < D; ++d) o[d] = 0.0;
  for (int x = 0; x < nt; ++x) {
    const double p = exp(lg[x] - mx) / den;
    const double* vr = vg + (size_t)toks[x] * D;
    for (int d = 0; d < D; ++d) o[d] += p * vr[d];
  }
  double delta = 0.0;
  for (int d = 0; d < D; ++d) delta += di[d] * o[d];
  if (dqi) {
    for (int d = 0; d < D; ++d) dqi[d] = 0.0;
    for (int x = 0; x < nt; ++x) {
      const double p = exp(lg[x] - mx) / den;
      const double* kr = kg + (size_t)toks[x] * D;
      const double* vr = vg + (size_t)toks[x] * D;
      double dp = 0.0;
      for (int d = 0; d < D; ++d) dp += di[d] * vr[d];
      const double ds = p * (dp - delta);
      for (int d = 0; d < D; ++d) dqi[d] += scale * ds * kr[d];
    }
  }
  *mx_out = mx;
  *den_out = den;
  *del_out = delta;
}

/* Row i's (head's) term in key j's gradients, from the row's statistics. */
static void orc_bwd_key_term(int D, double scale, const double* qi, const double* di, const double* kr,
                             const double* vr, double mx, double den, double delta, double* dkj, double* dvj) {
  double dot = 0.0, dp = 0.0;
  for (int d = 0; d < D; ++d) {
    dot += qi[d] * kr[d];
    dp += di[d] * vr[d];
  }
  const double p = exp(scale * dot - mx) / den;
  const double ds = p * (dp - delta);
  for (int d = 0; d < D; ++d) {
    dvj[d] += p * di[d];
    dkj[d] += scale * ds * qi[d];
  }
}

static double* orc_to_f64(const uint16_t* a, size_t n) {
  double* f = (double*)malloc(sizeof(double) * n);
  for (size_t x = 0; x < n; ++x) f[x] = orc_bf16_to_f64(a[x]);
  return f;
}

/* Outputs fp64: dq [N][Hq][D], dk, dv [G][N][D]. */
void orc_attend_bwd(int N, int Hq, int G, int D, int B, int Tq, double scale, const uint16_t* q, const uint16_t* k,
                    const uint16_t* v, const uint32_t* umask, const uint16_t* dout, double* dq, double* dk,
                    double* dv) {
  int T = (N + Tq - 1) / Tq;
  int NBc = (N + B - 1) / B;
  int W = (NBc + 31) / 32;
  int r = Hq / G;
  if (scale <= 0.0) scale = 1.0 / sqrt((double)D);
  size_t nq = (size_t)N * Hq * D, nk = (size_t)G * N * D;
  double* qf = orc_to_f64(q, nq);
  double* of = orc_to_f64(dout, nq);
  double* kf = orc_to_f64(k, nk);
  double* vf = orc_to_f64(v, nk);
  double* rmax = (double*)malloc(sizeof(double) * (size_t)N * Hq);
  double* rden = (double*)malloc(sizeof(double) * (size_t)N * Hq);
  double* rdel = (double*)malloc(sizeof(double) * (size_t)N * Hq);
  /* rows */
#pragma omp parallel for schedule(dynamic, 1)
  for (int i = 0; i < N; ++i) {
    int t = i / Tq;
    double* lg = (double*)malloc(sizeof(double) * (size_t)(i + 1));
    int32_t* toks = (int32_t*)malloc(sizeof(int32_t) * (size_t)(i + 1));
    double* o = (double*)malloc(sizeof(double) * (size_t)D);
    for (int g = 0; g < G; ++g) {
      const int nt = orc_row_tokens(i, B, umask + ((size_t)g * T + t) * W, toks);
      for (int hh = 0; hh < r; ++hh) {
        const size_t ih = (size_t)i * Hq + g * r + hh;
        orc_bwd_row(D, scale, qf + ih * D, of + ih * D, kf + (size_t)g * N * D, vf + (size_t)g * N * D, toks, nt, lg,
                    o, &rmax[ih], &rden[ih], &rdel[ih], dq + ih * D);
      }
    }
    free(lg);
    free(toks);
    free(o);
  }
  /* keys */
#pragma omp parallel for collapse(2) schedule(dynamic, 16)
  for (int g = 0; g < G; ++g) {
    for (int j = 0; j < N; ++j) {
      const double* kr = kf + ((size_t)g * N + j) * D;
      const double* vr = vf + ((size_t)g * N + j) * D;
      double* dkj = dk + ((size_t)g * N + j) * D;
      double* dvj = dv + ((size_t)g * N + j) * D;
      for (int d = 0; d < D; ++d) {
        dkj[d] = 0.0;
        dvj[d] = 0.0;
      }
      const int b = j / B;
      for (int i = j; i < N; ++i) {
        const uint32_t* m = umask + ((size_t)g * T + i / Tq) * W;
        if (!((m[b / 32] >> (b % 32)) & 1u)) continue;
        for (int hh = 0; hh < r; ++hh) {
          const size_t ih = (size_t)i * Hq + g * r + hh;
          orc_bwd_key_term(D, scale, qf + ih * D, of + ih * D, kr, vr, rmax[ih], rden[ih], rdel[ih], dkj, dvj);
        }
      }
    }
  }
  free(qf);
  free(of);
  free(kf);
  free(vf);
  free(rmax);
  free(rden);
  free(rdel);
}

/* The same gradient on a subset, where the whole one is out of reach: dq of the rows rows[0..nr)
 * (dq_rows [nr][Hq][D]), and dk, dv of group g0's keys key_lo .. key_hi - 1 (dk_keys, dv_keys
 * [key_hi - key_lo][D]) summed over every row that attends them, in ascending row order. Each
 * output is computed term for term as in orc_attend_bwd, with the statistics of only the rows it
 * needs. */
void orc_attend_bwd_part(int N, int Hq, int G, int D, int B, int Tq, double scale, const uint16_t* q,
                         const uint16_t* k, const uint16_t* v, const uint32_t* umask, const uint16_t* dout, int nr,
                         const int32_t* rows, double* dq_rows, int g0, int key_lo, int key_hi, double* dk_keys,
                         double* dv_keys) {
  int T = (N + Tq - 1) / Tq;
  int NBc = (N + B - 1) / B;
  int W = (NBc + 31) / 32;
  int r = Hq / G;
  if (scale <= 0.0) scale = 1.0 / sqrt((double)D);
  size_t nk = (size_t)G * N * D;
  double* kf = orc_to_f64(k, nk);
  double* vf = orc_to_f64(v, nk);
  /* dq rows */
#pragma omp parallel for schedule(dynamic, 1)
  for (int x = 0; x < nr; ++x) {
    const int i = rows[x], t = i / Tq;
    double* lg = (double*)malloc(sizeof(double) * (size_t)(i + 1));
    int32_t* toks = (int32_t*)malloc(sizeof(int32_t) * (size_t)(i + 1));
    double* buf = (double*)malloc(sizeof(double) * (size_t)3 * D);
    for (int g = 0; g < G; ++g) {
      const int nt = orc_row_tokens(i, B, umask + ((size_t)g * T + t) * W, toks);
      for (int hh = 0; hh < r; ++hh) {
        const size_t ih = (size_t)i * Hq + g * r + hh;
        for (int d = 0; d < D; ++d) {
          buf[d] = orc_bf16_to_f64(q[ih * D + d]);
          buf[D + d] = orc_bf16_to_f64(dout[ih * D + d]);
        }
        double mx, den, del;
        orc_bwd_row(D, scale, buf, buf + D, kf + (size_t)g * N * D, vf + (size_t)g * N * D, toks, nt, lg, buf + 2 * D,
                    &mx, &den, &del, dq_rows + ((size_t)x * Hq + g * r + hh) * D);
      }
    }
    free(lg);
    free(toks);
    free(buf);
  }
  if (key_hi <= key_lo) {
    free(kf);
    free(vf);
    return;
  }
  /* statistics of group g0's rows i >= key_lo whose tile union holds a block of the key range */
  const int nrow = N - key_lo, b_lo = key_lo / B, b_hi = (key_hi - 1) / B;
  double* rmax = (double*)malloc(sizeof(double) * (size_t)nrow * r);
  double* rden = (double*)malloc(sizeof(double) * (size_t)nrow * r);
  double* rdel = (double*)malloc(sizeof(double) * (size_t)nrow * r);
#pragma omp parallel for schedule(dynamic, 1)
  for (int i = key_lo; i < N; ++i) {
    const uint32_t* m = umask + ((size_t)g0 * T + i / Tq) * W;
    int hit = 0;
    for (int b = b_lo; b <= b_hi; ++b) hit |= (int)((m[b / 32] >> (b % 32)) & 1u);
    if (!hit) continue;
    double* lg = (double*)malloc(sizeof(double) * (size_t)(i + 1));
    int32_t* toks = (int32_t*)malloc(sizeof(int32_t) * (size_t)(i + 1));
    double* buf = (double*)malloc(sizeof(double) * (size_t)3 * D);
    const int nt = orc_row_tokens(i, B, m, toks);
    for (int hh = 0; hh < r; ++hh) {
      const size_t ih = (size_t)i * Hq + g0 * r + hh;
      const size_t sx = (size_t)(i - key_lo) * r + hh;
      for (int d = 0; d < D; ++d) {
        buf[d] = orc_bf16_to_f64(q[ih * D + d]);
        buf[D + d] = orc_bf16_to_f64(dout[ih * D + d]);
      }
      orc_bwd_row(D, scale, buf, buf + D, kf + (size_t)g0 * N * D, vf + (size_t)g0 * N * D, toks, nt, lg, buf + 2 * D,
                  &rmax[sx], &rden[sx], &rdel[sx], NULL);
    }
    free(lg);
    free(toks);
    free(buf);
  }
  /* the keys */
#pragma omp parallel for schedule(dynamic, 1)
  for (int j = key_lo; j < key_hi; ++j) {
    const double* kr = kf + ((size_t)g0 * N + j) * D;
    const double* vr = vf + ((size_t)g0 * N + j) * D;
    double* dkj = dk_keys + (size_t)(j - key_lo) * D;
    double* dvj = dv_keys + (size_t)(j - key_lo) * D;
    double* buf = (double*)malloc(sizeof(double) * (size_t)2 * D);
    for (int d = 0; d < D; ++d) {
      dkj[d] = 0.0;
      dvj[d] = 0.0;
    }
    const int b = j / B;
    for (int i = j; i < N; ++i) {
      const uint32_t* m = umask + ((size_t)g0 * T + i / Tq) * W;
      if (!((m[b / 32] >> (b % 32)) & 1u)) continue;
      for (int hh = 0; hh < r; ++hh) {
        const size_t ih = (size_t)i * Hq + g0 * r + hh;
        const size_t sx = (size_t)(i - key_lo) * r + hh;
        for (int d = 0; d < D; ++d) {
          buf[d] = orc_bf16_to_f64(q[ih * D + d]);
          buf[D + d] = orc_bf16_to_f64(dout[ih * D + d]);
        }
        orc_bwd_key_term(D, scale, buf, buf + D, kr, vr, rmax[sx], rden[sx], rdel[sx], dkj, dvj);
      }
    }
    free(buf);
  }
  free(kf);
  free(vf);
  free(rmax);
  free(rden);
  free(rdel);
}

/* ---------------------------------------------------------------- decode ----------------------- */

/* Single-token decode for the sequences seqs[0..nseq) (NULL: all S). For sequence s the query is
 * position L-1; candidates are blocks b < c = floor((L-1)/B); Sel is the selection above; the
 * attended tokens are those of Sel plus the own-block tokens c*B .. L-1 (no union).
 *   q [S][Hq][D], kc/vc [S][G][L][D], kbar [S][floor(L/B)][dI], qi [S][G][HI][dI] bf16, w [G][HI]
 *   topk_out [nseq][G][KB] int32 (may be NULL), out [nseq][Hq][D] fp64. */
void orc_decode(int S, int L, int Hq, int G, int D, int HI, int dI, int B, int KB, double scale,
                const uint16_t* q, const uint16_t* kc, const uint16_t* vc, const uint16_t* kbar,
                const uint16_t* qi, const float* w, int nseq, const int32_t* seqs, int32_t* topk_out,
                double* out) {
  int r = Hq / G;
  int NB = L / B;
  int i = L - 1;
  (void)S;
  int c = i / B;
  if (scale <= 0.0) scale = 1.0 / sqrt((double)D);
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
  for (int x = 0; x < nseq; ++x) {
    for (int g = 0; g < G; ++g) {
      int s = seqs ? seqs[x] : x;
      double* sc = (double*)malloc(sizeof(double) * (size_t)(c > 0 ? c : 1));
      int32_t* sel = (int32_t*)malloc(sizeof(int32_t) * (size_t)KB);
      orc_block_scores(HI, dI, qi + ((size_t)s * G + g) * HI * dI, w + (size_t)g * HI,
                       kbar + (size_t)s * NB * dI, c, sc);
      orc_select(c, sc, KB, sel);
      if (topk_out) memcpy(topk_out + ((size_t)x * G + g) * KB, sel, sizeof(int32_t) * (size_t)KB);
      int32_t* toks = (int32_t*)malloc(sizeof(int32_t) * (size_t)(KB * B + B));
      double* logit = (double*)malloc(sizeof(double) * (size_t)(KB * B + B));
      int nt = 0;
      for (int e = 0; e < KB && sel[e] >= 0; ++e)
        for (int j = 0; j < B; ++j) toks[nt++] = sel[e] * B + j;
      for (int j = c * B; j <= i; ++j) toks[nt++] = j;
      const uint16_t* kb = kc + ((size_t)s * G + g) * (size_t)L * D;
      const uint16_t* vb = vc + ((size_t)s * G + g) * (size_t)L * D;
      for (int hh = 0; hh < r; ++hh) {
        int h = g * r + hh;
        orc_attend_list(D, scale, q + ((size_t)s * Hq + h) * D, kb, vb, toks, nt, logit,
                        out + ((size_t)x * Hq + h) * D);
      }
      free(toks);
      free(logit);
      free(sc);
      free(sel);
    }
  }
}

/* ---------------------------------------------------------------- FP8 K/V decode -------------- */

/* OCP FP8 E4M3 ("e4m3fn"), the storage format of the FP8 K/V cache: 1 sign bit, 4 exponent bits
 * (bias 7), 3 mantissa bits; exponent field 0 encodes subnormals m * 2^-9; there are no infinities
 * and S.1111.111 is NaN. Written from the format's definition. */
double orc_fp8_e4m3_to_f64(uint8_t b) {
  int sgn = (b >> 7) & 1, e = (b >> 3) & 15, m = b & 7;
  double v;
  if (e == 15 && m == 7) return NAN;
  if (e == 0)
    v = ldexp((double)m, -9);
  else
    v = ldexp(1.0 + (double)m / 8.0, e - 7);
  return sgn ? -v : v;
}

/* orc_attend_list for a cache row in FP8: element d of key row t is k8[t][d] * ks (and of the value
 * row v8[t][d] * vs). Same definition, same order of operations. */
static void orc_attend_list_f8(int D, double scale, const uint16_t* qv, const uint8_t* kbase, double ks,
                               const uint8_t* vbase, double vs, const int32_t* toks, int nt, double* logit,
                               double* out) {
  double mx = -INFINITY;
  for (int x = 0; x < nt; ++x) {
    const uint8_t* kr = kbase + (size_t)toks[x] * D;
    double dot = 0.0;
    for (int d = 0; d < D; ++d) dot += orc_bf16_to_f64(qv[d]) * (orc_fp8_e4m3_to_f64(kr[d]) * ks);
    logit[x] = scale * dot;
    if (logit[x] > mx) mx = logit[x];
  }
  double den = 0.0;
  for (int x = 0; x < nt; ++x) {
    logit[x] = exp(logit[x] - mx);
    den += logit[x];
  }
  for (int d = 0; d < D; ++d) out[d] = 0.0;
  for (int x = 0; x < nt; ++x) {
    const uint8_t* vr = vbase + (size_t)toks[x] * D;
    double p = logit[x] / den;
    for (int d = 0; d < D; ++d) out[d] += p * (orc_fp8_e4m3_to_f64(vr[d]) * vs);
  }
}

/* orc_decode with FP8 K/V caches k8, v8 [S][G][L][D] and one scale per (sequence, group) for each:
 * kv_scale [S][G][2] = (key scale, value scale). Selection is unchanged (it reads only the bf16
 * index keys); the attended rows are the dequantized K/V. */
void orc_decode_f8(int S, int L, int Hq, int G, int D, int HI, int dI, int B, int KB, double scale,
                   const uint16_t* q, const uint8_t* kc, const uint8_t* vc, const float* kv_scale,
                   const uint16_t* kbar, const uint16_t* qi, const float* w, int nseq, const int32_t* seqs,
                   int32_t* topk_out, double* out) {
  int r = Hq / G;
  int NB = L / B;
  int i = L - 1;
  (void)S;
  int c = i / B;
  if (scale <= 0.0) scale = 1.0 / sqrt((double)D);
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
  for (int x = 0; x < nseq; ++x) {
    for (int g = 0; g < G; ++g) {
      int s = seqs ? seqs[x] : x;
      double* sc = (double*)malloc(sizeof(double) * (size_t)(c > 0 ? c : 1));
      int32_t* sel = (int32_t*)malloc(sizeof(int32_t) * (size_t)KB);
      orc_block_scores(HI, dI, qi + ((size_t)s * G + g) * HI * dI, w + (size_t)g * HI,
                       kbar + (size_t)s * NB * dI, c, sc);
      orc_select(c, sc, KB, sel);
      if (topk_out) memcpy(topk_out + ((size_t)x * G + g) * KB, sel, sizeof(int32_t) * (size_t)KB);
      int32_t* toks = (int32_t*)malloc(sizeof(int32_t) * (size_t)(KB * B + B));
      double* logit = (double*)malloc(sizeof(double) * (size_t)(KB * B + B));
      int nt = 0;
      for (int e = 0; e < KB && sel[e] >= 0; ++e)
        for (int j = 0; j < B; ++j) toks[nt++] = sel[e] * B + j;
      for (int j = c * B; j <= i; ++j) toks[nt++] = j;
      const uint8_t* kb = kc + ((size_t)s * G + g) * (size_t)L * D;
      const uint8_t* vb = vc + ((size_t)s * G + g) * (size_t)L * D;
      double ks = kv_scale[((size_t)s * G + g) * 2 + 0];
      double vs = kv_scale[((size_t)s * G + g) * 2 + 1];
      for (int hh = 0; hh < r; ++hh) {
        int h = g * r + hh;
        orc_attend_list_f8(D, scale, q + ((size_t)s * Hq + h) * D, kb, ks, vb, vs, toks, nt, logit,
                           out + ((size_t)x * Hq + h) * D);
      }
      free(toks);
      free(logit);
      free(sc);
      free(sel);
    }
  }
}

/* ---------------------------------------------------------------- coverage --------------------- */

/* Token coverage of a block-level selection against a token-level one ("Trade-off between top-k
 * and block size" compares the two by token coverage; the pages do not define the measure, this is
 * the reading used here). For query i and group g:
 *   T1 = Sel1(i,g) + {i}                        (token-level selection, B = 1)
 *   TB = tokens of the blocks Sel_B(i,g), plus the own-block tokens floor(i/B)*B .. i
 *   cov(i,g) = |T1 intersect TB| / |T1|
 * Returned: the mean of cov over g < G and i in [i_min, N).
 *   sel1 [G][N][KB1] (block ids = token ids), selB [G][N][KBB]. */
double orc_coverage(int N, int G, int B, int KB1, int KBB, const int32_t* sel1, const int32_t* selB, int i_min) {
  double total = 0.0;
  long long rows = 0;
  int NBc = (N + B - 1) / B;
#pragma omp parallel for collapse(2) reduction(+ : total, rows) schedule(dynamic, 16)
  for (int g = 0; g < G; ++g) {
    for (int i = i_min; i < N; ++i) {
      unsigned char* inB = (unsigned char*)calloc((size_t)NBc, 1);
      const int32_t* sb = selB + ((size_t)g * N + i) * KBB;
      for (int x = 0; x < KBB; ++x)
        if (sb[x] >= 0) inB[sb[x]] = 1;
      inB[i / B] = 1; /* own block: its tokens up to i are visible, and every token of T1 is <= i */
      const int32_t* s1 = sel1 + ((size_t)g * N + i) * KB1;
      int n1 = 1, hit = 1; /* token i itself: always in its own block */
      for (int x = 0; x < KB1; ++x) {
        if (s1[x] < 0) continue;
        n1 += 1;
        hit += inB[s1[x] / B];
      }
      total += (double)hit / (double)n1;
      rows += 1;
      free(inB);
    }
  }
  return rows ? total / (double)rows : 0.0;
}
