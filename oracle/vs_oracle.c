/*
 * vs_oracle.c -- plain, slow, fp64 CPU oracle for vertical-slash sparse prefill.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or constant with the HIP path and must never be used to
 * produce a product result.
 *
 * What it follows (VSPrefill summary pages on gist.science, paper 2603.04460):
 *  - the pattern: "Technical Summary, 2. Methodology, Core Concept:
 *    Vertical-Slash Pattern" (English page) and "2. Methodik, A. Das
 *    Vertical-Slash-Muster" (German page, which writes the slash as a
 *    relative shift i-j): a query attends to selected key columns and to
 *    keys at selected relative offsets;
 *  - the indexer: "Key Components, 1. VSIndexer": a shared-weight two-layer
 *    linear net over concat(K with RoPE, V) with separate vertical and slash
 *    output heads;
 *  - selection: "3. Adaptive Inference Pipeline, Dynamic Budgeting": the
 *    fewest top-scored indices whose cumulative predicted mass reaches a
 *    threshold;
 *  - attention: "Fused Kernel Execution": attention restricted to the merged
 *    index set.  Here that is written out as its plain definition (two-pass
 *    softmax per row), not as a tiled kernel.
 *
 * Readings where the pages are silent (all documented with the build):
 *  scale is a caller argument (1/sqrt(d) by default); index sets belong to a KV
 *  head and are shared by its query heads (h -> g = h / (hq/hkv)); the slash
 *  offset is o = i - j >= 0 and applies to row i only when o <= i; a key in
 *  both sets counts once; a vertical column c is visible to row i only if
 *  c <= i; a row with no visible key gets out = 0 and lse = -inf.
 *
 * Selection arithmetic is fixed exactly so that an integer decision (the
 * budget K) has one answer: m = max score in fp32; x = score - m in fp32;
 * u = 0 if x < -32 else rint(exp_spec(x) * 2^32) as an unsigned 64-bit
 * integer; U = sum u; T = ceil(mass * U) in IEEE double; order by (score
 * descending, candidate index ascending); K = length of the shortest prefix
 * with cumulative u >= T, then min(K, cap).  exp_spec is Cody and Waite's
 * range reduction (W. J. Cody, W. Waite, "Software Manual for the Elementary
 * Functions", 1980) with a two-piece ln 2, followed by the degree-7 Taylor
 * polynomial of e^r evaluated by Horner's rule with fused multiply-adds, all
 * in fp32.  Build with -ffp-contract=off so no other fusion happens.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { VSO_BF16 = 0, VSO_F32 = 1, VSO_F64 = 2 };
enum { VSO_VERTICAL = 0, VSO_SLASH = 1 };

/* ---------------------------------------------------------------- input decode */

static double load_elem(const void* base, int dtype, int64_t i) {
  if (dtype == VSO_BF16) {
    uint32_t w = (uint32_t)((const uint16_t*)base)[i] << 16;
    float f;
    memcpy(&f, &w, sizeof f);
    return (double)f;
  }
  if (dtype == VSO_F32) return (double)((const float*)base)[i];
  return ((const double*)base)[i];
}

static void load_row(const void* base, int dtype, int64_t off, int len, double* dst) {
  for (int t = 0; t < len; ++t) dst[t] = load_elem(base, dtype, off + t);
}

/* ---------------------------------------------------------------- the pattern */

/* Index set of row i for one KV head: every j with 0 <= j <= i such that j is
 * a selected column or i - j is a selected offset, each j once, ascending.
 * Built by walking the two sorted lists together: columns <= i ascending, and
 * keys i - o for offsets o <= i taken from the largest offset down.
 * Returns |S_i|. */
static int row_set(const int32_t* cols, int ncols, const int32_t* offs, int noffs, int i,
                   int32_t* out) {
  int nc = 0;
  while (nc < ncols && cols[nc] <= i) ++nc;
  int no = 0;
  while (no < noffs && offs[no] <= i) ++no;
  int a = 0, b = no - 1, m = 0;
  while (a < nc || b >= 0) {
    int ja = a < nc ? cols[a] : INT32_MAX;
    int jb = b >= 0 ? i - offs[b] : INT32_MAX;
    int j = ja < jb ? ja : jb;
    if (ja == j) ++a;
    if (jb == j) --b;
    out[m++] = j;
  }
  return m;
}

int vso_row_set(const int32_t* vidx, const int32_t* vcnt, int cap_v, const int32_t* soff,
                const int32_t* scnt, int cap_s, int g, int i, int32_t* out) {
  return row_set(vidx + (int64_t)g * cap_v, vcnt[g], soff + (int64_t)g * cap_s, scnt[g], i, out);
}

/* sum over rows of |S_i| for one KV head, by building every row's set */
int64_t vso_pair_count(const int32_t* vidx, const int32_t* vcnt, int cap_v, const int32_t* soff,
                       const int32_t* scnt, int cap_s, int g, int n) {
  int32_t* buf = (int32_t*)malloc(sizeof(int32_t) * (size_t)(n > 0 ? n : 1));
  int64_t total = 0;
  for (int i = 0; i < n; ++i) total += vso_row_set(vidx, vcnt, cap_v, soff, scnt, cap_s, g, i, buf);
  free(buf);
  return total;
}

/* ---------------------------------------------------------------- attention */

/* For every requested (head, row): out_r = sum_{j in S_i} softmax_j(scale*q_i.k_j) v_j
 * and lse_r = log sum_{j in S_i} exp(scale*q_i.k_j), in fp64, two passes. */
int vso_attn_rows(const void* q, const void* k, const void* v, int dtype, int hq, int hkv, int n,
                  int d, double scale, const int32_t* vidx, const int32_t* vcnt, int cap_v,
                  const int32_t* soff, const int32_t* scnt, int cap_s, const int32_t* row_h,
                  const int32_t* row_i, int64_t nrows, double* out, double* lse, int nthreads) {
  if (hq <= 0 || hkv <= 0 || hq % hkv != 0 || n <= 0 || d <= 0) return 1;
  const int group = hq / hkv;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#else
  (void)nthreads;
#endif
  int err = 0;
#pragma omp parallel
  {
    int32_t* set = (int32_t*)malloc(sizeof(int32_t) * (size_t)n);
    double* s = (double*)malloc(sizeof(double) * (size_t)n);
    double* qi = (double*)malloc(sizeof(double) * (size_t)d);
    double* kj = (double*)malloc(sizeof(double) * (size_t)d);
    double* acc = (double*)malloc(sizeof(double) * (size_t)d);
#pragma omp for schedule(dynamic, 16)
    for (int64_t r = 0; r < nrows; ++r) {
      int h = row_h[r], i = row_i[r];
      if (h < 0 || h >= hq || i < 0 || i >= n) {
        err = 1;
        continue;
      }
      int g = h / group;
      int m = vso_row_set(vidx, vcnt, cap_v, soff, scnt, cap_s, g, i, set);
      double* o = out + r * d;
      if (m == 0) {
        for (int t = 0; t < d; ++t) o[t] = 0.0;
        lse[r] = -INFINITY;
        continue;
      }
      load_row(q, dtype, ((int64_t)h * n + i) * d, d, qi);
      double mx = -INFINITY;
      for (int a = 0; a < m; ++a) {
        load_row(k, dtype, ((int64_t)g * n + set[a]) * d, d, kj);
        double dot = 0.0;
        for (int t = 0; t < d; ++t) dot += qi[t] * kj[t];
        s[a] = scale * dot;
        if (s[a] > mx) mx = s[a];
      }
      double l = 0.0;
      for (int t = 0; t < d; ++t) acc[t] = 0.0;
      for (int a = 0; a < m; ++a) {
        double p = exp(s[a] - mx);
        l += p;
        load_row(v, dtype, ((int64_t)g * n + set[a]) * d, d, kj);
        for (int t = 0; t < d; ++t) acc[t] += p * kj[t];
      }
      for (int t = 0; t < d; ++t) o[t] = acc[t] / l;
      lse[r] = mx + log(l);
    }
    free(set);
    free(s);
    free(qi);
    free(kj);
    free(acc);
  }
  return err;
}

/* ------------------------------------------------- vertical/slash aggregation */

/* Ground truth for the indexer's distillation (VSPrefill summaries: English
 * page, section 2, "Key Components, 2. Distillation Training, Ground Truth
 * Generation"; German page, 2.B.2): full causal attention weights summed
 * along key columns and along diagonals.  For every query head h of KV head
 * g and every row i, P_ij = softmax_j(scale q_i . k_j) over j <= i (fp64, two
 * passes); a_v[g][j] += P_ij and a_s[g][i-j] += P_ij.  Sums over the group's
 * query heads and all rows, unnormalised (each of a_v[g], a_s[g] totals
 * G * n).  Rows are spread over threads, each with private sums that are
 * added at the end.  Returns 0, or 1 on invalid arguments. */
int vso_aggregate(const void* q, const void* k, int dtype, int hq, int hkv, int n, int d,
                  double scale, double* a_v, double* a_s, int nthreads) {
  if (hq <= 0 || hkv <= 0 || hq % hkv != 0 || n <= 0 || d <= 0) return 1;
  const int group = hq / hkv;
  const size_t cells = (size_t)hkv * (size_t)n;
  for (size_t t = 0; t < cells; ++t) a_v[t] = a_s[t] = 0.0;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#else
  (void)nthreads;
#endif
#pragma omp parallel
  {
    double* pv = (double*)calloc(cells, sizeof(double));
    double* ps = (double*)calloc(cells, sizeof(double));
    double* s = (double*)malloc(sizeof(double) * (size_t)n);
    double* qi = (double*)malloc(sizeof(double) * (size_t)d);
    double* kj = (double*)malloc(sizeof(double) * (size_t)d);
#pragma omp for schedule(dynamic, 16)
    for (int64_t r = 0; r < (int64_t)hq * n; ++r) {
      const int h = (int)(r / n), i = (int)(r % n), g = h / group;
      load_row(q, dtype, ((int64_t)h * n + i) * d, d, qi);
      double mx = -INFINITY;
      for (int j = 0; j <= i; ++j) {
        load_row(k, dtype, ((int64_t)g * n + j) * d, d, kj);
        double dot = 0.0;
        for (int t = 0; t < d; ++t) dot += qi[t] * kj[t];
        s[j] = scale * dot;
        if (s[j] > mx) mx = s[j];
      }
      double l = 0.0;
      for (int j = 0; j <= i; ++j) l += exp(s[j] - mx);
      for (int j = 0; j <= i; ++j) {
        const double pij = exp(s[j] - mx) / l;
        pv[(size_t)g * n + j] += pij;
        ps[(size_t)g * n + (i - j)] += pij;
      }
    }
#pragma omp critical
    {
      for (size_t t = 0; t < cells; ++t) {
        a_v[t] += pv[t];
        a_s[t] += ps[t];
      }
    }
    free(pv);
    free(ps);
    free(s);
    free(qi);
    free(kj);
  }
  return 0;
}

/* ---------------------------------------------------------------- the indexer */

/* Per KV head g and position j: x = [k_j | v_j] (2d values), h = max(0, W1 x)
 * (W1 is [hidden][2d]), then vlog = W2[0].h and slog = W2[1].h (W2 is
 * [2][hidden]); no biases; one weight set for every head; fp64 throughout. */
int vso_index(const void* k, const void* v, int dtype, int hkv, int n, int d, int hidden,
              const void* w1, const void* w2, int wdtype, double* vlog, double* slog,
              int nthreads) {
  if (hkv <= 0 || n <= 0 || d <= 0 || hidden <= 0) return 1;
  const int d2 = 2 * d;
  double* W1 = (double*)malloc(sizeof(double) * (size_t)hidden * d2);
  double* W2 = (double*)malloc(sizeof(double) * 2 * (size_t)hidden);
  load_row(w1, wdtype, 0, hidden * d2, W1);
  load_row(w2, wdtype, 0, 2 * hidden, W2);
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#else
  (void)nthreads;
#endif
  const int64_t total = (int64_t)hkv * n;
#pragma omp parallel
  {
    double* x = (double*)malloc(sizeof(double) * (size_t)d2);
    double* h = (double*)malloc(sizeof(double) * (size_t)hidden);
#pragma omp for schedule(static)
    for (int64_t r = 0; r < total; ++r) {
      load_row(k, dtype, r * d, d, x);
      load_row(v, dtype, r * d, d, x + d);
      for (int t = 0; t < hidden; ++t) {
        double a = 0.0;
        for (int c = 0; c < d2; ++c) a += W1[(int64_t)t * d2 + c] * x[c];
        h[t] = a > 0.0 ? a : 0.0;
      }
      double sv = 0.0, ss = 0.0;
      for (int t = 0; t < hidden; ++t) {
        sv += W2[t] * h[t];
        ss += W2[hidden + t] * h[t];
      }
      vlog[r] = sv;
      slog[r] = ss;
    }
    free(x);
    free(h);
  }
  free(W1);
  free(W2);
  return 0;
}

/* ---------------------------------------------------------------- selection */

/* e^x in fp32 for x in [-32, 0]: x = k ln2 + r with k = rint(x log2 e), r
 * reduced against a two-piece ln 2 (the high piece has few enough bits that
 * k * ln2_hi is exact); e^r by the degree-7 Taylor polynomial; then scale by
 * 2^k.  Constants are the fp32 values nearest to log2 e, to ln 2 cut to its
 * leading bits plus the fp32 remainder, and to 1/k!. */
float vso_exp_spec(float x) {
  const float log2e = 0x1.715476p+0f;
  const float ln2_hi = 0x1.62e4p-1f;
  const float ln2_lo = 0x1.7f7d1cp-20f;
  float kf = rintf(x * log2e);
  float r = fmaf(-kf, ln2_hi, x);
  r = fmaf(-kf, ln2_lo, r);
  float p = 0x1.a01a02p-13f;     /* 1/7! */
  p = fmaf(p, r, 0x1.6c16c2p-10f); /* 1/6! */
  p = fmaf(p, r, 0x1.111112p-7f);  /* 1/5! */
  p = fmaf(p, r, 0x1.555556p-5f);  /* 1/4! */
  p = fmaf(p, r, 0x1.555556p-3f);  /* 1/3! */
  p = fmaf(p, r, 0.5f);            /* 1/2! */
  p = fmaf(p, r, 1.0f);
  p = fmaf(p, r, 1.0f);
  return ldexpf(p, (int)kf);
}

/* quantised mass of a score that sits x below the maximum */
uint64_t vso_mass_u(float x) {
  if (x < -32.0f) return 0;
  double e = (double)vso_exp_spec(x) * 4294967296.0;
  return (uint64_t)nearbyint(e);
}

typedef struct {
  float s;
  int32_t c;
} cand_t;

static int cand_cmp(const void* pa, const void* pb) {
  const cand_t* a = (const cand_t*)pa;
  const cand_t* b = (const cand_t*)pb;
  if (a->s > b->s) return -1;
  if (a->s < b->s) return 1;
  return (a->c > b->c) - (a->c < b->c);
}

static int int_cmp(const void* pa, const void* pb) {
  int32_t a = *(const int32_t*)pa, b = *(const int32_t*)pb;
  return (a > b) - (a < b);
}

/* Per head: candidates c = 0..n-1 with score logit[c] (VERTICAL: c is a
 * column) or logit[n-1-c] (SLASH: c is an offset, scored where its diagonal
 * meets the last row).  Writes the selected candidates ascending into
 * idx[h][0..K), -1 into idx[h][K..cap), and K into count[h].  Optionally
 * returns U and T per head.  Returns 0, or 1 on invalid arguments. */
int vso_select(const float* logit, int heads, int n, int kind, double mass, int cap, int32_t* idx,
               int32_t* count, uint64_t* out_U, uint64_t* out_T) {
  if (heads <= 0 || n <= 0 || !(mass > 0.0 && mass <= 1.0) || cap < 1 || cap > n) return 1;
  if (kind != VSO_VERTICAL && kind != VSO_SLASH) return 1;
  cand_t* cs = (cand_t*)malloc(sizeof(cand_t) * (size_t)n);
  int32_t* sel = (int32_t*)malloc(sizeof(int32_t) * (size_t)n);
  for (int h = 0; h < heads; ++h) {
    const float* row = logit + (int64_t)h * n;
    float mx = -INFINITY;
    for (int c = 0; c < n; ++c) {
      float s = kind == VSO_VERTICAL ? row[c] : row[n - 1 - c];
      if (s == 0.0f) s = 0.0f; /* -0 and +0 are one score */
      cs[c].s = s;
      cs[c].c = c;
      if (s > mx) mx = s;
    }
    uint64_t U = 0;
    for (int c = 0; c < n; ++c) U += vso_mass_u(cs[c].s - mx);
    uint64_t T = (uint64_t)ceil(mass * (double)U);
    qsort(cs, (size_t)n, sizeof(cand_t), cand_cmp);
    uint64_t cum = 0;
    int K = n;
    for (int a = 0; a < n; ++a) {
      cum += vso_mass_u(cs[a].s - mx);
      if (cum >= T) {
        K = a + 1;
        break;
      }
    }
    if (K > cap) K = cap;
    for (int a = 0; a < K; ++a) sel[a] = cs[a].c;
    qsort(sel, (size_t)K, sizeof(int32_t), int_cmp);
    for (int a = 0; a < cap; ++a) idx[(int64_t)h * cap + a] = a < K ? sel[a] : -1;
    count[h] = K;
    if (out_U) out_U[h] = U;
    if (out_T) out_T[h] = T;
  }
  free(cs);
  free(sel);
  return 0;
}

/* Max-based dynamic threshold (FlashPrefill summary, arXiv 2603.06199,
 * Spanish page, "2. Metodologia, B. Umbralizacion Dinamica Basada en
 * Maximos"): keep every candidate whose score is at least alpha times the
 * largest score.  The score is the softmax probability over candidates, so
 * the test p_c >= alpha * max p is exp(s_c - m) >= alpha; it is decided on
 * the quantised masses above (the maximum has u = 2^32 exactly): keep when
 * u_c >= A = ceil(alpha * 2^32).  K = the number kept, then min(K, cap), the
 * first K in (score descending, candidate ascending) order, written
 * ascending like vso_select.  Returns 0, or 1 on invalid arguments. */
int vso_select_threshold(const float* logit, int heads, int n, int kind, double alpha, int cap,
                         int32_t* idx, int32_t* count, uint64_t* out_A) {
  if (heads <= 0 || n <= 0 || !(alpha > 0.0 && alpha <= 1.0) || cap < 1 || cap > n) return 1;
  if (kind != VSO_VERTICAL && kind != VSO_SLASH) return 1;
  const uint64_t A = (uint64_t)ceil(alpha * 4294967296.0);
  cand_t* cs = (cand_t*)malloc(sizeof(cand_t) * (size_t)n);
  int32_t* sel = (int32_t*)malloc(sizeof(int32_t) * (size_t)n);
  for (int h = 0; h < heads; ++h) {
    const float* row = logit + (int64_t)h * n;
    float mx = -INFINITY;
    for (int c = 0; c < n; ++c) {
      float s = kind == VSO_VERTICAL ? row[c] : row[n - 1 - c];
      if (s == 0.0f) s = 0.0f;
      cs[c].s = s;
      cs[c].c = c;
      if (s > mx) mx = s;
    }
    int K = 0;
    for (int c = 0; c < n; ++c) K += vso_mass_u(cs[c].s - mx) >= A ? 1 : 0;
    if (K > cap) K = cap;
    qsort(cs, (size_t)n, sizeof(cand_t), cand_cmp);
    for (int a = 0; a < K; ++a) sel[a] = cs[a].c;
    qsort(sel, (size_t)K, sizeof(int32_t), int_cmp);
    for (int a = 0; a < cap; ++a) idx[(int64_t)h * cap + a] = a < K ? sel[a] : -1;
    count[h] = K;
  }
  if (out_A) *out_A = A;
  free(cs);
  free(sel);
  return 0;
}

/* ------------------------------------------- FlashPrefill block discovery */

/* FlashPrefill (gist.science summary of arXiv 2603.06199, Spanish page,
 * "2. Metodologia", part A "Descubrimiento Instantaneo de Patrones",
 * "Estrategia de Aproximacion de Bloques", and part B "Umbralizacion Dinamica
 * Basada en Maximos"): key blocks are scored for a query block by a sparse,
 * evenly spaced set of probe ("skeleton") queries against the mean key of
 * each block, whose exponential is the geometric mean of the block's
 * exponentials (the AM-GM proxy); a query block keeps the key blocks whose
 * score is at least alpha times its largest score.
 *
 * Readings where the page is silent: query and key blocks are bs consecutive
 * positions (the last block may be short); the skeleton of query block I for
 * KV head g is, for every query head h of g, the rows bs*I + m*(bs/skel),
 * m = 0..skel-1, that are below n (row bs*I always is); the candidates of
 * query block I are the full causal blocks J < I; one probe's block
 * distribution is the softmax over the candidates of scale * q . kbar_J; a
 * block's score is that probability averaged over the probes; the diagonal
 * block J = I is always kept, and block 0 keeps only itself. */

/* kbar[g][J][t] = mean over the keys j of block J of k[g][j][t], fp64. */
int vso_block_means(const void* k, int dtype, int hkv, int n, int d, int bs, double* kbar) {
  if (hkv <= 0 || n <= 0 || d <= 0 || bs <= 0) return 1;
  const int nb = (n + bs - 1) / bs;
  double* row = (double*)malloc(sizeof(double) * (size_t)d);
  for (int g = 0; g < hkv; ++g)
    for (int J = 0; J < nb; ++J) {
      double* out = kbar + ((int64_t)g * nb + J) * d;
      const int j0 = J * bs, j1 = (j0 + bs < n ? j0 + bs : n);
      for (int t = 0; t < d; ++t) out[t] = 0.0;
      for (int j = j0; j < j1; ++j) {
        load_row(k, dtype, ((int64_t)g * n + j) * d, d, row);
        for (int t = 0; t < d; ++t) out[t] += row[t];
      }
      for (int t = 0; t < d; ++t) out[t] /= (double)(j1 - j0);
    }
  free(row);
  return 0;
}

/* score[g][I][J] for J < I (zero elsewhere), from the block means kbar
 * [hkv][nb][d]: the mean over the skeleton probes of block I of
 * exp(z_J - max z) / sum_{J' < I} exp(z_J' - max z), z_J = scale q . kbar_J.
 * With rows_g == NULL every (g, I) is computed into score [hkv][nb][nb];
 * otherwise only the nrows pairs (rows_g[r], rows_I[r]) into score [nrows][nb]. */
int vso_block_scores(const void* q, int dtype, int hq, int hkv, int n, int d, double scale, int bs,
                     int skel, const double* kbar, const int32_t* rows_g, const int32_t* rows_I,
                     int64_t nrows, double* score, int nthreads) {
  if (hq <= 0 || hkv <= 0 || hq % hkv != 0 || n <= 0 || d <= 0 || bs <= 0) return 1;
  if (skel <= 0 || skel > bs || bs % skel != 0) return 1;
  const int group = hq / hkv, nb = (n + bs - 1) / bs, step = bs / skel;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#else
  (void)nthreads;
#endif
#pragma omp parallel
  {
    double* qi = (double*)malloc(sizeof(double) * (size_t)d);
    double* z = (double*)malloc(sizeof(double) * (size_t)nb);
    const int64_t total = rows_g ? nrows : (int64_t)hkv * nb;
#pragma omp for schedule(dynamic, 4)
    for (int64_t r = 0; r < total; ++r) {
      const int g = rows_g ? rows_g[r] : (int)(r / nb), I = rows_g ? rows_I[r] : (int)(r % nb);
      if (g < 0 || g >= hkv || I < 0 || I >= nb) continue;
      double* out = score + r * nb;
      for (int J = 0; J < nb; ++J) out[J] = 0.0;
      if (I == 0) continue;
      int probes = 0;
      for (int h = g * group; h < (g + 1) * group; ++h)
        for (int m = 0; m < skel; ++m) {
          const int i = I * bs + m * step;
          if (i >= n) continue;
          load_row(q, dtype, ((int64_t)h * n + i) * d, d, qi);
          double mx = -INFINITY;
          for (int J = 0; J < I; ++J) {
            const double* kb = kbar + ((int64_t)g * nb + J) * d;
            double dot = 0.0;
            for (int t = 0; t < d; ++t) dot += qi[t] * kb[t];
            z[J] = scale * dot;
            if (z[J] > mx) mx = z[J];
          }
          double l = 0.0;
          for (int J = 0; J < I; ++J) l += exp(z[J] - mx);
          for (int J = 0; J < I; ++J) out[J] += exp(z[J] - mx) / l;
          ++probes;
        }
      for (int J = 0; J < I; ++J) out[J] /= (double)probes;
    }
    free(qi);
    free(z);
  }
  return 0;
}

/* The max-based threshold on given fp32 scores [hkv][nb][nb], decided in
 * fp32: thr = alpha * max_{J<I} score (one IEEE fp32 product); block J < I is
 * kept when score >= thr, and J = I always.  mask[g][I][w] bit b <-> block
 * 32 w + b; words_per_row >= ceil(nb / 32). */
int vso_block_select(const float* score, int hkv, int nb, float alpha, uint32_t* mask,
                     int words_per_row) {
  if (hkv <= 0 || nb <= 0 || !(alpha > 0.0f && alpha <= 1.0f) || words_per_row * 32 < nb) return 1;
  for (int g = 0; g < hkv; ++g)
    for (int I = 0; I < nb; ++I) {
      const float* row = score + ((int64_t)g * nb + I) * nb;
      uint32_t* mrow = mask + ((int64_t)g * nb + I) * words_per_row;
      for (int w = 0; w < words_per_row; ++w) mrow[w] = 0u;
      float mx = -INFINITY;
      for (int J = 0; J < I; ++J)
        if (row[J] > mx) mx = row[J];
      volatile float thr = alpha * mx;
      for (int J = 0; J < I; ++J)
        if (row[J] >= thr) mrow[J / 32] |= 1u << (J % 32);
      mrow[I / 32] |= 1u << (I % 32);
    }
  return 0;
}

/* Attention under a block mask: for each requested (head, row i) of KV head
 * g, S_i = { j <= i : bit (j / bs) of mask[g][i / bs] }, then the same fp64
 * two-pass softmax as vso_attn_rows (empty S_i: out = 0, lse = -inf). */
int vso_block_attn_rows(const void* q, const void* k, const void* v, int dtype, int hq, int hkv,
                        int n, int d, double scale, int bs, const uint32_t* mask,
                        int words_per_row, const int32_t* row_h, const int32_t* row_i,
                        int64_t nrows, double* out, double* lse, int nthreads) {
  if (hq <= 0 || hkv <= 0 || hq % hkv != 0 || n <= 0 || d <= 0 || bs <= 0) return 1;
  const int group = hq / hkv, nb = (n + bs - 1) / bs;
  if (words_per_row * 32 < nb) return 1;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#else
  (void)nthreads;
#endif
  int err = 0;
#pragma omp parallel
  {
    int32_t* set = (int32_t*)malloc(sizeof(int32_t) * (size_t)n);
    double* s = (double*)malloc(sizeof(double) * (size_t)n);
    double* qi = (double*)malloc(sizeof(double) * (size_t)d);
    double* kj = (double*)malloc(sizeof(double) * (size_t)d);
    double* acc = (double*)malloc(sizeof(double) * (size_t)d);
#pragma omp for schedule(dynamic, 16)
    for (int64_t r = 0; r < nrows; ++r) {
      const int h = row_h[r], i = row_i[r];
      if (h < 0 || h >= hq || i < 0 || i >= n) {
        err = 1;
        continue;
      }
      const int g = h / group;
      const uint32_t* mrow = mask + ((int64_t)g * nb + i / bs) * words_per_row;
      int m = 0;
      for (int j = 0; j <= i; ++j)
        if ((mrow[(j / bs) / 32] >> ((j / bs) % 32)) & 1u) set[m++] = j;
      double* o = out + r * d;
      if (m == 0) {
        for (int t = 0; t < d; ++t) o[t] = 0.0;
        lse[r] = -INFINITY;
        continue;
      }
      load_row(q, dtype, ((int64_t)h * n + i) * d, d, qi);
      double mx = -INFINITY;
      for (int a = 0; a < m; ++a) {
        load_row(k, dtype, ((int64_t)g * n + set[a]) * d, d, kj);
        double dot = 0.0;
        for (int t = 0; t < d; ++t) dot += qi[t] * kj[t];
        s[a] = scale * dot;
        if (s[a] > mx) mx = s[a];
      }
      double l = 0.0;
      for (int t = 0; t < d; ++t) acc[t] = 0.0;
      for (int a = 0; a < m; ++a) {
        const double p = exp(s[a] - mx);
        l += p;
        load_row(v, dtype, ((int64_t)g * n + set[a]) * d, d, kj);
        for (int t = 0; t < d; ++t) acc[t] += p * kj[t];
      }
      for (int t = 0; t < d; ++t) o[t] = acc[t] / l;
      lse[r] = mx + log(l);
    }
    free(set);
    free(s);
    free(qi);
    free(kj);
    free(acc);
  }
  return err;
}

int vso_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
