/*
 * CRISP sparse-prefill path: plain CPU oracle.  TEST INFRASTRUCTURE ONLY.
 *
 * Only tests, the package smoke check and the benchmark's CPU-baseline leg use
 * this file.  It shares no code with the GPU library.  Loops are written in the
 * order of the definitions on the pages; OpenMP only spreads independent heads
 * or rows over threads and never changes the arithmetic of any result.
 *
 * Sources ("CRISP" summary page, picx.dev, section "Methodology"):
 *   Eq. 2    C_struct = mean over proxy queries of the post-softmax mass at the
 *            anchor positions (first w_sink keys and the local window w_local).
 *   Eq. 3    noise floor mu = max(1 - a_first - a_last, 0) / (N_b - 2).
 *   Eq. 4    block j is important iff p_j > alpha * mu.
 *   Alg. 2   proxy map on a query subset; route to VS iff C_struct >= tau.
 *   Alg. 3   column (vertical) and diagonal (slash) scores, block-pooled,
 *            first and last blocks always kept.
 *   Alg. 4   pooled Q and K, softmax of the pooled scores, flatten, normalise,
 *            sort, keep the gamma-cumsum prefix.
 *   Motivation / Key Contributions: the Jensen-Shannon divergence router that
 *            C_struct replaces (pooled estimate against per-query estimate).
 *
 * Precision (the pages leave it open; these are the readings taken here):
 *   - proxy scores are fp32: acc = fmaf(q[k], key[k], acc) for k ascending,
 *     z = fl(acc * c) with c = fl32(1/sqrt(d)), then z = fl(z + bias);
 *   - exp_crisp below (Cody-Waite reduction, degree-7 Taylor, all fp32);
 *   - every sum that feeds a decision is an int64 fixed-point sum of
 *     rne(value * 2^40), so its value does not depend on summation order;
 *   - thresholds are compared as exact integers.
 * Build: gcc -O2 -ffp-contract=off -mfma -fopenmp (no contraction, no
 * fast-math; -mfma makes fmaf a single fused instruction rather than a call).
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define FIX_SHIFT 40

typedef __int128 i128;

/* ---------------------------------------------------------------- exp ---- */
/* e^x for x <= 0 in fp32.  Range reduction after Cody and Waite (1980):
 * x = k ln2 + r with k = rint(x log2 e) and ln2 split into a 15-bit head and a
 * tail; e^r by its Taylor series to degree 7 in Horner form (coefficients
 * 1/j! rounded to fp32); result p * 2^k.  Returns 0 below -80 so that every
 * non-zero result is a normal number. */
float oracle_exp_crisp(float x);
void oracle_exp_crisp_array(const float* x, float* y, int64_t count) {
  for (int64_t i = 0; i < count; ++i) y[i] = oracle_exp_crisp(x[i]);
}

float oracle_exp_crisp(float x) {
  if (x < -80.0f) return 0.0f;
  const float log2e = 1.44269502f;       /* 0x3FB8AA3B */
  const float ln2_hi = 0.693145751953125f; /* 0x3F317200 */
  const float ln2_lo = 1.42860677e-06f;  /* 0x35BFBE8E */
  float t = x * log2e;
  float kf = rintf(t);
  float r = fmaf(-kf, ln2_hi, x);
  r = fmaf(-kf, ln2_lo, r);
  float p = 1.0f / 5040.0f;
  p = fmaf(p, r, 1.0f / 720.0f);
  p = fmaf(p, r, 1.0f / 120.0f);
  p = fmaf(p, r, 1.0f / 24.0f);
  p = fmaf(p, r, 1.0f / 6.0f);
  p = fmaf(p, r, 0.5f);
  p = fmaf(p, r, 1.0f);
  p = fmaf(p, r, 1.0f);
  return ldexpf(p, (int)kf);
}

static inline int64_t fix_rne(float v) { /* rne(v * 2^40), v >= 0 */
  return (int64_t)rintf(ldexpf(v, FIX_SHIFT));
}

static inline float fix_to_float(int64_t L) { /* fl32(L) * 2^-40 */
  return ldexpf((float)L, -FIX_SHIFT);
}

float oracle_scale(int32_t d) { return (float)(1.0 / sqrt((double)d)); }

/* ------------------------------------------------------------- proxy ----- */
/* One proxy row: query row i against keys 0..i (causal).  z[j] for j <= i. */
static void proxy_row(const float* q, const float* K, int32_t d, int64_t i, float c,
                      int32_t nb_bias, const int32_t* boff, const float* bval, float* z) {
  for (int64_t j = 0; j <= i; ++j) {
    const float* kj = K + (size_t)j * d;
    float acc = 0.0f;
    for (int32_t k = 0; k < d; ++k) acc = fmaf(q[k], kj[k], acc);
    float s = acc * c;
    for (int32_t t = 0; t < nb_bias; ++t)
      if ((int64_t)boff[t] == i - j) s = s + bval[t];
    z[j] = s;
  }
}

/*
 * Alg. 2 + Eq. 2 + the block pooling of Alg. 3 for every query head.
 *   Qlast [bh][qrows][d] holds query rows q0..n-1 (the last query block,
 *   q0 = (N_b-1)*B, qrows = n - q0); K [bkv][n][d]; query head h reads KV
 *   head h / (bh/bkv).
 *   Outputs per head: m [qrows], L [qrows] (int64 row sums), mass_v / mass_s
 *   [N_b] (vertical block b = j/B, slash block b = (i-j)/B), total T,
 *   C_num (fixed-point anchor mass) and route (1 = VS, 0 = PE).
 *   Optional A_q [bh][qrows][n] receives rne(A*2^40) (0 where j > i).
 */
int oracle_proxy(int32_t bh, int32_t bkv, int64_t n, int32_t d, int32_t B, int32_t w_sink,
                 int32_t w_local, uint32_t tau_num, uint32_t tau_den, const float* Qlast, const float* K,
                 int32_t bias_count, const int32_t* bias_off, const float* bias_val, float* m_out,
                 int64_t* L_out, int64_t* mass_v, int64_t* mass_s, int64_t* total, int64_t* cnum,
                 uint8_t* route, int64_t* A_q_out) {
  if (bh <= 0 || bkv <= 0 || bh % bkv || n <= 0 || d <= 0 || d > 256 || B <= 0) return -1;
  const int64_t nb = (n + B - 1) / B;
  const int64_t q0 = (nb - 1) * B;
  const int64_t qrows = n - q0;
  const int32_t group = bh / bkv;
  const float c = oracle_scale(d);
  memset(mass_v, 0, sizeof(int64_t) * bh * nb);
  memset(mass_s, 0, sizeof(int64_t) * bh * nb);
  memset(cnum, 0, sizeof(int64_t) * bh);

#pragma omp parallel
  {
    float* z = (float*)malloc(sizeof(float) * n);
    float* e = (float*)malloc(sizeof(float) * n);
    int64_t* lv = (int64_t*)malloc(sizeof(int64_t) * nb);
    int64_t* ls = (int64_t*)malloc(sizeof(int64_t) * nb);
#pragma omp for collapse(2) schedule(dynamic, 1)
    for (int32_t h = 0; h < bh; ++h) {
      for (int64_t r = 0; r < qrows; ++r) {
        const int64_t i = q0 + r;
        const float* q = Qlast + ((size_t)h * qrows + r) * d;
        const float* Kh = K + (size_t)(h / group) * n * d;
        const int32_t* bo = bias_count ? bias_off + (size_t)h * bias_count : NULL;
        const float* bv = bias_count ? bias_val + (size_t)h * bias_count : NULL;
        proxy_row(q, Kh, d, i, c, bias_count, bo, bv, z);
        /* softmax statistics: exact max, fixed-point sum of exponentials */
        float m = z[0];
        for (int64_t j = 1; j <= i; ++j)
          if (z[j] > m) m = z[j];
        int64_t L = 0;
        for (int64_t j = 0; j <= i; ++j) {
          e[j] = oracle_exp_crisp(z[j] - m);
          L += fix_rne(e[j]);
        }
        const float l = fix_to_float(L);
        m_out[h * qrows + r] = m;
        L_out[h * qrows + r] = L;
        /* post-softmax map A = e / l, quantised; pooled by column and diagonal block */
        memset(lv, 0, sizeof(int64_t) * nb);
        memset(ls, 0, sizeof(int64_t) * nb);
        int64_t anchor = 0;
        for (int64_t j = 0; j <= i; ++j) {
          const float a = e[j] / l;
          const int64_t aq = fix_rne(a);
          lv[j / B] += aq;
          ls[(i - j) / B] += aq;
          if (j < w_sink || i - j < w_local) anchor += aq;
          if (A_q_out) A_q_out[((size_t)h * qrows + r) * n + j] = aq;
        }
        if (A_q_out)
          for (int64_t j = i + 1; j < n; ++j) A_q_out[((size_t)h * qrows + r) * n + j] = 0;
        for (int64_t b = 0; b < nb; ++b) {
          if (lv[b]) {
#pragma omp atomic
            mass_v[h * nb + b] += lv[b];
          }
          if (ls[b]) {
#pragma omp atomic
            mass_s[h * nb + b] += ls[b];
          }
        }
#pragma omp atomic
        cnum[h] += anchor;
      }
    }
    free(z);
    free(e);
    free(lv);
    free(ls);
  }
  for (int32_t h = 0; h < bh; ++h) {
    int64_t t = 0;
    for (int64_t b = 0; b < nb; ++b) t += mass_v[h * nb + b];
    total[h] = t;
    /* C_struct = C_num / (qrows 2^40) >= tau_num / tau_den, in integers */
    i128 lhs = (i128)tau_den * (i128)cnum[h];
    i128 rhs = (i128)tau_num * (i128)qrows * ((i128)1 << FIX_SHIFT);
    route[h] = lhs >= rhs ? 1 : 0;
  }
  return 0;
}

/* ------------------------------------------------- sink-aware selection -- */
/* Eq. 3 and Eq. 4 for one direction.  With nb <= 2 every block is kept.
 * M = max(T - p_first - p_last, 0) is the middle mass in fixed point, so
 * mu = M / (nb - 2) and p_b > alpha mu  <=>  a_den (nb-2) p_b > a_num M.
 * Output: ascending block ids; returns the count. */
int32_t oracle_vs_select(int64_t nb, const int64_t* p, int64_t T, uint32_t a_num, uint32_t a_den,
                         int32_t* out) {
  int32_t cnt = 0;
  if (nb <= 2) {
    for (int64_t b = 0; b < nb; ++b) out[cnt++] = (int32_t)b;
    return cnt;
  }
  int64_t M = T - p[0] - p[nb - 1];
  if (M < 0) M = 0;
  out[cnt++] = 0;
  for (int64_t b = 1; b <= nb - 2; ++b) {
    i128 lhs = (i128)a_den * (i128)(nb - 2) * (i128)p[b];
    i128 rhs = (i128)a_num * (i128)M;
    if (lhs > rhs) out[cnt++] = (int32_t)b;
  }
  out[cnt++] = (int32_t)(nb - 1);
  return cnt;
}

/* ---------------------------------------- cumulative-gamma baseline ------ */
typedef struct {
  int64_t v;
  int64_t idx;
} keyed;

static int by_value_desc_index_asc(const void* a, const void* b) {
  const keyed* x = (const keyed*)a;
  const keyed* y = (const keyed*)b;
  if (x->v != y->v) return x->v > y->v ? -1 : 1;
  return x->idx < y->idx ? -1 : (x->idx > y->idx);
}

static int by_int_asc(const void* a, const void* b) {
  int32_t x = *(const int32_t*)a, y = *(const int32_t*)b;
  return (x > y) - (x < y);
}

/* The coverage rule the pages argue against (summary page, Motivation):
 * order blocks by mass (ties: lower id first) and keep the shortest prefix
 * whose mass reaches gamma of the total; first and last blocks are added. */
int32_t oracle_cumulative_select(int64_t nb, const int64_t* p, int64_t T, uint32_t g_num,
                                 uint32_t g_den, int32_t* out) {
  keyed* ks = (keyed*)malloc(sizeof(keyed) * nb);
  for (int64_t b = 0; b < nb; ++b) {
    ks[b].v = p[b];
    ks[b].idx = b;
  }
  qsort(ks, nb, sizeof(keyed), by_value_desc_index_asc);
  uint8_t* keep = (uint8_t*)calloc(nb, 1);
  int64_t cum = 0;
  for (int64_t t = 0; t < nb; ++t) {
    if ((i128)g_den * cum >= (i128)g_num * T) break;
    cum += ks[t].v;
    keep[ks[t].idx] = 1;
  }
  keep[0] = 1;
  keep[nb - 1] = 1;
  int32_t cnt = 0;
  for (int64_t b = 0; b < nb; ++b)
    if (keep[b]) out[cnt++] = (int32_t)b;
  free(ks);
  free(keep);
  return cnt;
}

/* ------------------------------------------------- pooled estimation ---- */
/* Alg. 4 for one query head.  Qh [n][d], Kh [n][d].
 *   Qbar[qb][k] = fl(sum_r q[qb B + r][k], r ascending, fp32) / cnt   (K likewise)
 *   zbar[qb][kb] = fl(fma-chain(Qbar_qb, Kbar_kb) * c), kb <= qb
 *   row softmax with exp_crisp and int64 sums; Abar_q = rne(Abar * 2^40)
 *   Tbar = sum of all Abar_q; order by (Abar_q desc, flat index qb*nb+kb asc);
 *   keep the shortest prefix with g_den * cum >= g_num * Tbar; add (qb, qb).
 * Output CSR: rowptr [nb+1], cols ascending within each row.  Returns nnz.
 * Optional Abar_out [nb(nb+1)/2] receives Abar_q in row-major triangle order.
 * stats_out[0] = Tbar, stats_out[1] = length of the gamma prefix (before the
 * diagonal blocks are added). */
int64_t oracle_pe_index(int64_t n, int32_t d, int32_t B, const float* Qh, const float* Kh,
                        uint32_t g_num, uint32_t g_den, int32_t* rowptr, int32_t* cols,
                        int64_t* Abar_out, int64_t* stats_out, int32_t threads) {
  const int64_t nb = (n + B - 1) / B;
  const float c = oracle_scale(d);
  float* Qb = (float*)malloc(sizeof(float) * nb * d);
  float* Kb = (float*)malloc(sizeof(float) * nb * d);
  for (int64_t b = 0; b < nb; ++b) {
    const int64_t r0 = b * B;
    const int64_t cnt = (r0 + B <= n) ? B : n - r0;
    for (int32_t k = 0; k < d; ++k) {
      float sq = 0.0f, sk = 0.0f;
      for (int64_t r = 0; r < cnt; ++r) {
        sq = sq + Qh[(size_t)(r0 + r) * d + k];
        sk = sk + Kh[(size_t)(r0 + r) * d + k];
      }
      Qb[b * d + k] = sq / (float)cnt;
      Kb[b * d + k] = sk / (float)cnt;
    }
  }
  const int64_t ntri = nb * (nb + 1) / 2;
  keyed* all = (keyed*)malloc(sizeof(keyed) * ntri);
  int64_t Tbar = 0;
#pragma omp parallel num_threads(threads > 0 ? threads : omp_get_max_threads())
  {
    float* z = (float*)malloc(sizeof(float) * nb);
    float* e = (float*)malloc(sizeof(float) * nb);
#pragma omp for schedule(dynamic, 16) reduction(+ : Tbar)
    for (int64_t qb = 0; qb < nb; ++qb) {
      for (int64_t kb = 0; kb <= qb; ++kb) {
        float acc = 0.0f;
        for (int32_t k = 0; k < d; ++k) acc = fmaf(Qb[qb * d + k], Kb[kb * d + k], acc);
        z[kb] = acc * c;
      }
      float m = z[0];
      for (int64_t kb = 1; kb <= qb; ++kb)
        if (z[kb] > m) m = z[kb];
      int64_t L = 0;
      for (int64_t kb = 0; kb <= qb; ++kb) {
        e[kb] = oracle_exp_crisp(z[kb] - m);
        L += fix_rne(e[kb]);
      }
      const float l = fix_to_float(L);
      const int64_t base = qb * (qb + 1) / 2;
      for (int64_t kb = 0; kb <= qb; ++kb) {
        const int64_t aq = fix_rne(e[kb] / l);
        all[base + kb].v = aq;
        all[base + kb].idx = qb * nb + kb;
        if (Abar_out) Abar_out[base + kb] = aq;
        Tbar += aq;
      }
    }
    free(z);
    free(e);
  }
  qsort(all, ntri, sizeof(keyed), by_value_desc_index_asc);
  uint8_t* keep = (uint8_t*)calloc(ntri, 1);
  int64_t cum = 0, taken = 0;
  for (int64_t t = 0; t < ntri; ++t) {
    if ((i128)g_den * cum >= (i128)g_num * Tbar) break;
    cum += all[t].v;
    ++taken;
    const int64_t qb = all[t].idx / nb, kb = all[t].idx % nb;
    keep[qb * (qb + 1) / 2 + kb] = 1;
  }
  if (stats_out) {
    stats_out[0] = Tbar;
    stats_out[1] = taken;
  }
  int64_t nnz = 0;
  rowptr[0] = 0;
  for (int64_t qb = 0; qb < nb; ++qb) {
    const int64_t base = qb * (qb + 1) / 2;
    keep[base + qb] = 1;
    for (int64_t kb = 0; kb <= qb; ++kb)
      if (keep[base + kb]) cols[nnz++] = (int32_t)kb;
    rowptr[qb + 1] = (int32_t)nnz;
  }
  free(keep);
  free(all);
  free(Qb);
  free(Kb);
  return nnz;
}

/* ------------------------------------------------- divergence router ---- */
/* The router CRISP replaces (summary page, Motivation and Key Contributions):
 * a second, pooled estimate of the head's attention, compared with the
 * per-query one by the Jensen-Shannon divergence; the head goes to VS when
 * the divergence reaches a threshold.  Readings (the pages give no formula):
 *   - per-query estimate P: the proxy map of the last query block, softmax
 *     per query first, then pooled over key blocks and queries, i.e. the
 *     column block masses p^v_b / T of Alg. 3 (already exact int64 sums);
 *   - pooled estimate Q: pool first, then one softmax: the block mean of the
 *     last query block's rows against the block means of all key blocks,
 *     z_b = fl(fma-chain(Qbar, Kbar_b) c), softmax in the same fixed point as
 *     Alg. 4 (it is the last row of Alg. 4's pooled map);
 *   - JSD(P, Q) = (KL(P || M) + KL(Q || M)) / 2 with M = (P + Q) / 2, natural
 *     logarithm; route to VS iff JSD >= tau_jsd (exact rational test).
 * Arithmetic (fixed so that a GPU can reproduce every bit): P_b and Q_b in
 * fp64 by correctly rounded division of the int64 sums; per block
 * t_b = fl(fl(P log_crisp(P / M)) + fl(Q log_crisp(Q / M))) with a zero term
 * for a zero probability; J = sum_b rne(t_b 2^52) in int64, so
 * JSD = J 2^-53 and the sum is order-free. */

/* Natural logarithm in fp64 for positive normal x, after the classic
 * reduction x = 2^e m with m in (sqrt(1/2), sqrt(2)], then
 * ln m = 2 atanh(s), s = (m - 1) / (m + 1), by the odd series
 * 2 (s + s^3/3 + ... + s^23/23) in Horner form in s^2 (|s| <= 0.1716, so the
 * first omitted term is below 2^-60 relative), and
 * ln x = e ln2 + ln m with ln2 split into a 32-bit head and a tail.  Within
 * 3 ulp of the exact logarithm (tests measure it against the C library). */
double oracle_log_crisp(double x) {
  const double sqrt2 = 0x1.6a09e667f3bcdp+0;
  const double ln2_hi = 0x1.62e42ff000000p-1;
  const double ln2_lo = -0x1.718432a1b0e26p-35;
  uint64_t bits;
  memcpy(&bits, &x, sizeof bits);
  int e = (int)((bits >> 52) & 0x7ff) - 1023;
  bits = (bits & 0x000fffffffffffffULL) | 0x3ff0000000000000ULL;
  double m;
  memcpy(&m, &bits, sizeof m); /* m in [1, 2) */
  if (m > sqrt2) {
    m = m * 0.5;
    e += 1;
  }
  const double s = (m - 1.0) / (m + 1.0);
  const double s2 = s * s;
  double p = 1.0 / 23.0;
  p = fma(p, s2, 1.0 / 21.0);
  p = fma(p, s2, 1.0 / 19.0);
  p = fma(p, s2, 1.0 / 17.0);
  p = fma(p, s2, 1.0 / 15.0);
  p = fma(p, s2, 1.0 / 13.0);
  p = fma(p, s2, 1.0 / 11.0);
  p = fma(p, s2, 1.0 / 9.0);
  p = fma(p, s2, 1.0 / 7.0);
  p = fma(p, s2, 1.0 / 5.0);
  p = fma(p, s2, 1.0 / 3.0);
  p = fma(p, s2, 1.0);
  const double lm = (2.0 * s) * p;
  const double r = fma((double)e, ln2_lo, lm);
  return fma((double)e, ln2_hi, r);
}

void oracle_log_crisp_array(const double* x, double* y, int64_t count) {
  for (int64_t i = 0; i < count; ++i) y[i] = oracle_log_crisp(x[i]);
}

/* J = sum_b rne(t_b 2^52) of two fixed-point distributions p (total Tp) and
 * a (total Ta) over nb blocks.  Returns J; JSD = J 2^-53. */
int64_t oracle_jsd_fixed(int64_t nb, const int64_t* p, int64_t Tp, const int64_t* a, int64_t Ta) {
  int64_t J = 0;
  for (int64_t b = 0; b < nb; ++b) {
    const double P = (double)p[b] / (double)Tp;
    const double Q = (double)a[b] / (double)Ta;
    const double M = 0.5 * (P + Q);
    const double tp = P > 0.0 ? P * oracle_log_crisp(P / M) : 0.0;
    const double tq = Q > 0.0 ? Q * oracle_log_crisp(Q / M) : 0.0;
    const double t = tp + tq;
    J += (int64_t)llrint(ldexp(t, 52));
  }
  return J;
}

/* The pooled estimate of one query head's last query block: Qbar over the
 * last block's rows, Kbar over every key block (sequential fp32 sums, then
 * divided by the row count), z_b = fl(fma-chain(Qbar, Kbar_b) c), row max,
 * exp_crisp, int64 row sum, abar_b = rne(fl(e_b / l) 2^40).  Writes abar [nb]
 * and returns its total. */
int64_t oracle_pooled_last_row(int64_t n, int32_t d, int32_t B, const float* Qh, const float* Kh,
                               int64_t* abar) {
  const int64_t nb = (n + B - 1) / B;
  const float c = oracle_scale(d);
  float* qbar = (float*)malloc(sizeof(float) * d);
  float* kbar = (float*)malloc(sizeof(float) * d);
  float* z = (float*)malloc(sizeof(float) * nb);
  const int64_t q0 = (nb - 1) * B, qcnt = n - q0;
  for (int32_t k = 0; k < d; ++k) {
    float s = 0.0f;
    for (int64_t r = 0; r < qcnt; ++r) s = s + Qh[(size_t)(q0 + r) * d + k];
    qbar[k] = s / (float)qcnt;
  }
  for (int64_t b = 0; b < nb; ++b) {
    const int64_t r0 = b * B;
    const int64_t cnt = (r0 + B <= n) ? B : n - r0;
    for (int32_t k = 0; k < d; ++k) {
      float s = 0.0f;
      for (int64_t r = 0; r < cnt; ++r) s = s + Kh[(size_t)(r0 + r) * d + k];
      kbar[k] = s / (float)cnt;
    }
    float acc = 0.0f;
    for (int32_t k = 0; k < d; ++k) acc = fmaf(qbar[k], kbar[k], acc);
    z[b] = acc * c;
  }
  float m = z[0];
  for (int64_t b = 1; b < nb; ++b)
    if (z[b] > m) m = z[b];
  int64_t L = 0;
  for (int64_t b = 0; b < nb; ++b) L += fix_rne(oracle_exp_crisp(z[b] - m));
  const float l = fix_to_float(L);
  int64_t T = 0;
  for (int64_t b = 0; b < nb; ++b) {
    abar[b] = fix_rne(oracle_exp_crisp(z[b] - m) / l);
    T += abar[b];
  }
  free(qbar);
  free(kbar);
  free(z);
  return T;
}

/* ---------------------------------------------------- masked attention -- */
/* Reference attention for one query row in fp64 (the textbook definition:
 * scores (q.k) / sqrt(d) + bias, softmax over the allowed keys, weighted sum
 * of values).  allowed(j) is given as a byte mask over keys 0..n-1 (only
 * j <= i is ever read).  Used to pin the NumPy attention in tests. */
void oracle_attention_row(int64_t i, int32_t d, const float* q, const float* K, const float* V,
                          int32_t bias_count, const int32_t* boff, const float* bval,
                          const uint8_t* allowed, double* out) {
  const double c = 1.0 / sqrt((double)d);
  double m = -INFINITY;
  double* s = (double*)malloc(sizeof(double) * (i + 1));
  for (int64_t j = 0; j <= i; ++j) {
    if (!allowed[j]) continue;
    double dot = 0.0;
    for (int32_t k = 0; k < d; ++k) dot += (double)q[k] * (double)K[(size_t)j * d + k];
    double v = dot * c;
    for (int32_t t = 0; t < bias_count; ++t)
      if ((int64_t)boff[t] == i - j) v += (double)bval[t];
    s[j] = v;
    if (v > m) m = v;
  }
  double l = 0.0;
  for (int32_t k = 0; k < d; ++k) out[k] = 0.0;
  for (int64_t j = 0; j <= i; ++j) {
    if (!allowed[j]) continue;
    double p = exp(s[j] - m);
    l += p;
    for (int32_t k = 0; k < d; ++k) out[k] += p * (double)V[(size_t)j * d + k];
  }
  for (int32_t k = 0; k < d; ++k) out[k] /= l;
  free(s);
}
