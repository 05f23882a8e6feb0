/*
 * bsa_ref.c -- CPU oracle for block-sparse attention (fp64) and reference
 * planner. TEST INFRASTRUCTURE ONLY: the GPU library never links, loads or
 * calls this code, and this code includes nothing from the GPU library.
 *
 * The attention definition follows the Tessera abstract ("Decoupling Logical
 * Masks from GPU Execution for Dynamic Block-Sparse Attention"): attention is
 * computed only for the (query-block, key-block) pairs that the logical mask
 * selects, exactly, with the usual softmax over the allowed keys. The union
 * mode follows the CompactAttention summary (block mask as a KV-selection
 * signal; query-block union plus intra-group union into per-group KV tables).
 * Softmax scale 1/sqrt(d) and the natural-log log-sum-exp are the usual
 * scaled-dot-product-attention conventions; a row with no allowed key gives
 * output 0 and log-sum-exp -inf.
 */
#include "bsa_ref.h"

#include <math.h>
#include <omp.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* Problem bookkeeping                                                       */
/* ------------------------------------------------------------------------ */

static int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

static int is_block_size(int32_t x) {
  return x == 16 || x == 32 || x == 64 || x == 128 || x == 256 || x == 512;
}

static int mask_batches(const ref_problem *p) { return p->mask_broadcast ? 1 : p->batch; }

static int check_problem(const ref_problem *p) {
  if (!p || p->batch < 1 || p->hq < 1 || p->hkv < 1 || p->hq % p->hkv) return -1;
  if (p->sq < 0 || p->skv < 0 || p->d < 1 || !p->bq || !p->bk) return -1;
  if (p->dtype != 0 && p->dtype != 1) return -1;
  for (int h = 0; h < p->hq; ++h)
    if (p->bq[h] < 1 || p->bk[h] < 1) return -1;
  if (p->paged) {
    if (p->page_size < 1 || p->pages_per_seq < 1 || p->num_pages < 1) return -1;
    if ((int64_t)p->page_size * p->pages_per_seq < p->skv) return -1;
  }
  if (p->gqa_union) {
    int gs = p->hq / p->hkv;
    for (int h = 0; h < p->hq; ++h)
      if (p->bk[h] != p->bk[(h / gs) * gs]) return -1;
  }
  return 0;
}

/* Offset of the [nqb][nkb] mask of (mask batch bm, head h). */
static int64_t *mask_offsets(const ref_problem *p) {
  int nbm = mask_batches(p);
  int64_t *off = (int64_t *)malloc(sizeof(int64_t) * (nbm * p->hq + 1));
  int64_t o = 0;
  for (int bm = 0; bm < nbm; ++bm)
    for (int h = 0; h < p->hq; ++h) {
      off[bm * p->hq + h] = o;
      o += ceil_div(p->sq, p->bq[h]) * ceil_div(p->skv, p->bk[h]);
    }
  off[nbm * p->hq] = o;
  return off;
}

/* Union of a group's selections (CompactAttention summary): key block kb is
 * selected for group g iff some head of g selects it in some query block.
 * Returns U[bm][g][nkb_g] as bytes. */
static uint8_t *group_union(const ref_problem *p, const uint8_t *mask, const int64_t *moff,
                            int64_t *nkb_out) {
  int nbm = mask_batches(p), gs = p->hq / p->hkv;
  int64_t nkb = ceil_div(p->skv, p->bk[0]);
  for (int h = 0; h < p->hq; ++h)
    if (ceil_div(p->skv, p->bk[h]) > nkb) nkb = ceil_div(p->skv, p->bk[h]);
  uint8_t *u = (uint8_t *)calloc((size_t)nbm * p->hkv * (nkb ? nkb : 1), 1);
  for (int bm = 0; bm < nbm; ++bm)
    for (int g = 0; g < p->hkv; ++g)
      for (int hh = 0; hh < gs; ++hh) {
        int h = g * gs + hh;
        int64_t nq = ceil_div(p->sq, p->bq[h]), nk = ceil_div(p->skv, p->bk[h]);
        const uint8_t *m = mask + moff[bm * p->hq + h];
        for (int64_t qb = 0; qb < nq; ++qb)
          for (int64_t kb = 0; kb < nk; ++kb)
            if (m[qb * nk + kb]) u[((int64_t)bm * p->hkv + g) * nkb + kb] = 1;
      }
  *nkb_out = nkb;
  return u;
}

static double load_value(const void *base, int dtype, int64_t idx) {
  if (dtype == 0) {
    uint32_t bits = (uint32_t)((const uint16_t *)base)[idx] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
  }
  return (double)((const float *)base)[idx];
}

/* OCP FP8 E4M3 ("e4m3fn"): 1 sign bit, 4 exponent bits with bias 7, 3
 * mantissa bits. Exponent field 0 holds subnormals m * 2^-9; S.1111.111 is
 * NaN; there are no infinities, so the largest finite value is 1.75 * 2^8. */
double ref_e4m3(uint8_t b) {
  const int s = b >> 7, e = (b >> 3) & 15, m = b & 7;
  double v;
  if (e == 15 && m == 7) return NAN;
  if (e == 0) v = ldexp((double)m, -9);
  else v = ldexp(1.0 + m / 8.0, e - 7);
  return s ? -v : v;
}

/* Element index of K/V row j of kv-head g in batch b (dense or paged). */
static int64_t kv_index(const ref_problem *p, const int32_t *page_table, int b, int g, int64_t j) {
  if (p->paged) {
    int64_t page = page_table[(int64_t)b * p->pages_per_seq + j / p->page_size];
    return ((page * p->page_size + j % p->page_size) * p->hkv + g) * (int64_t)p->d;
  }
  return (((int64_t)b * p->hkv + g) * p->skv + j) * (int64_t)p->d;
}

/* ------------------------------------------------------------------------ */
/* Forward: exact softmax attention restricted to the allowed keys           */
/* ------------------------------------------------------------------------ */

/* K and V element idx of kv head g: the problem's dtype, or, when k_scale is
 * set, an e4m3 byte times the head's scale. */
static double kv_value(const ref_problem *p, const void *base, const float *scale, int g, int64_t idx) {
  if (scale) return (double)scale[g] * ref_e4m3(((const uint8_t *)base)[idx]);
  return load_value(base, p->dtype, idx);
}

static int forward_impl(const ref_problem *p, const uint8_t *mask, const int32_t *page_table,
                        const void *q, const void *k, const void *v, const float *k_scale,
                        const float *v_scale, int mode, const int64_t *rows, int64_t nrows,
                        double *o, double *lse, int nthreads) {
  if (check_problem(p) || (p->paged && !page_table)) return -1;
  const int d = p->d, gs = p->hq / p->hkv;
  const double scale = p->scale > 0 ? p->scale : 1.0 / sqrt((double)d);
  int64_t *moff = mask_offsets(p);
  int64_t unkb = 0;
  uint8_t *uni = p->gqa_union ? group_union(p, mask, moff, &unkb) : NULL;
  const int64_t total = rows ? nrows : (int64_t)p->batch * p->hq * p->sq;
  if (nthreads <= 0) nthreads = omp_get_max_threads();

#pragma omp parallel num_threads(nthreads)
  {
    double *s = (double *)malloc(sizeof(double) * (p->skv ? p->skv : 1));
    int64_t *js = (int64_t *)malloc(sizeof(int64_t) * (p->skv ? p->skv : 1));
    double *acc = (double *)malloc(sizeof(double) * d);
#pragma omp for schedule(dynamic, 8)
    for (int64_t r = 0; r < total; ++r) {
      int64_t b, h, i;
      if (rows) {
        b = rows[3 * r], h = rows[3 * r + 1], i = rows[3 * r + 2];
      } else {
        b = r / ((int64_t)p->hq * p->sq);
        h = (r / p->sq) % p->hq;
        i = r % p->sq;
      }
      const int g = (int)(h / gs), bm = p->mask_broadcast ? 0 : (int)b;
      const int64_t bq = p->bq[h], bk = p->bk[h];
      const int64_t nkb = ceil_div(p->skv, bk);
      /* The selection row for this query: mask row, or the group union. */
      const uint8_t *sel = p->gqa_union ? uni + ((int64_t)bm * p->hkv + g) * unkb
                                        : mask + moff[bm * p->hq + h] + (i / bq) * nkb;
      const int64_t qbase = ((b * p->hq + h) * p->sq + i) * (int64_t)d;
      int64_t n = 0;
      double m = -INFINITY;
      if (mode == 0) {
        /* Dense: the full score row, -inf where the key is not allowed. */
        for (int64_t j = 0; j < p->skv; ++j) {
          int allowed = sel[j / bk] && (!p->causal || j <= i + p->causal_offset);
          if (allowed) {
            int64_t kbase = kv_index(p, page_table, (int)b, g, j);
            double dot = 0.0;
            for (int t = 0; t < d; ++t)
              dot += load_value(q, p->dtype, qbase + t) * kv_value(p, k, k_scale, g, kbase + t);
            s[j] = scale * dot;
          } else {
            s[j] = -INFINITY;
          }
          if (s[j] > m) m = s[j];
        }
        n = p->skv;
        for (int64_t j = 0; j < n; ++j) js[j] = j;
      } else {
        /* Block skipping: only selected blocks, keys ascending. */
        for (int64_t kb = 0; kb < nkb; ++kb) {
          if (!sel[kb]) continue;
          int64_t j1 = (kb + 1) * bk < p->skv ? (kb + 1) * bk : p->skv;
          for (int64_t j = kb * bk; j < j1; ++j) {
            if (p->causal && j > i + p->causal_offset) break;
            int64_t kbase = kv_index(p, page_table, (int)b, g, j);
            double dot = 0.0;
            for (int t = 0; t < d; ++t)
              dot += load_value(q, p->dtype, qbase + t) * kv_value(p, k, k_scale, g, kbase + t);
            s[n] = scale * dot;
            js[n] = j;
            if (s[n] > m) m = s[n];
            ++n;
          }
        }
      }
      double *orow = o + r * d;
      if (m == -INFINITY) {
        for (int t = 0; t < d; ++t) orow[t] = 0.0;
        lse[r] = -INFINITY;
        continue;
      }
      double l = 0.0;
      for (int t = 0; t < d; ++t) acc[t] = 0.0;
      for (int64_t e = 0; e < n; ++e) {
        double w = exp(s[e] - m);
        l += w;
        int64_t vbase = kv_index(p, page_table, (int)b, g, js[e]);
        for (int t = 0; t < d; ++t) acc[t] += w * kv_value(p, v, v_scale, g, vbase + t);
      }
      for (int t = 0; t < d; ++t) orow[t] = acc[t] / l;
      lse[r] = m + log(l);
    }
    free(s);
    free(js);
    free(acc);
  }
  free(moff);
  free(uni);
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Backward: gradients of the restricted softmax attention                  */
/* ------------------------------------------------------------------------ */

/* Keys that query row i of head h (batch b) may see, ascending: the selected
 * blocks of its selection row, cut at the causal bound (the same set the
 * forward's mode 1 visits). Returns the count written to js. */
static int64_t allowed_keys(const ref_problem *p, const uint8_t *sel, int64_t bk, int64_t i,
                            int64_t *js) {
  const int64_t nkb = ceil_div(p->skv, bk);
  int64_t n = 0;
  for (int64_t kb = 0; kb < nkb; ++kb) {
    if (!sel[kb]) continue;
    int64_t j1 = (kb + 1) * bk < p->skv ? (kb + 1) * bk : p->skv;
    for (int64_t j = kb * bk; j < j1; ++j) {
      if (p->causal && j > i + p->causal_offset) break;
      js[n++] = j;
    }
  }
  return n;
}

typedef struct {
  const ref_problem *p;
  const uint8_t *mask, *uni;
  const int64_t *moff;
  int64_t unkb;
  const void *q, *k, *v, *dout;
  double scale;
} bwd_ctx;

/* Allowed keys js[0..n) of query row i of head h in batch b. Returns n. */
static int64_t row_keys(const bwd_ctx *c, int64_t b, int64_t h, int64_t i, int64_t *js) {
  const ref_problem *p = c->p;
  const int g = (int)(h / (p->hq / p->hkv)), bm = p->mask_broadcast ? 0 : (int)b;
  const int64_t bk = p->bk[h];
  const uint8_t *sel = p->gqa_union ? c->uni + ((int64_t)bm * p->hkv + g) * c->unkb
                                    : c->mask + c->moff[bm * p->hq + h] + (i / p->bq[h]) * ceil_div(p->skv, bk);
  return allowed_keys(p, sel, bk, i, js);
}

/* Over the n allowed keys js of row (b, h, i): S (s), P (pr), dP (dp) and dS
 * (ds) as defined below. */
static void row_gradients(const bwd_ctx *c, int64_t b, int64_t h, int64_t i, const int64_t *js,
                          int64_t n, double *s, double *pr, double *dp, double *ds) {
  const ref_problem *p = c->p;
  const int d = p->d, g = (int)(h / (p->hq / p->hkv));
  const int64_t qbase = ((b * p->hq + h) * p->sq + i) * (int64_t)d;
  double m = -INFINITY;
  for (int64_t e = 0; e < n; ++e) {
    const int64_t kbase = kv_index(p, NULL, (int)b, g, js[e]);
    double dot = 0.0;
    for (int t = 0; t < d; ++t)
      dot += load_value(c->q, p->dtype, qbase + t) * load_value(c->k, p->dtype, kbase + t);
    s[e] = c->scale * dot;
    if (s[e] > m) m = s[e];
  }
  double l = 0.0;
  for (int64_t e = 0; e < n; ++e) l += exp(s[e] - m);
  double Di = 0.0;
  for (int64_t e = 0; e < n; ++e) {
    pr[e] = exp(s[e] - m) / l;
    const int64_t vbase = kv_index(p, NULL, (int)b, g, js[e]);
    double dot = 0.0;
    for (int t = 0; t < d; ++t)
      dot += load_value(c->dout, p->dtype, qbase + t) * load_value(c->v, p->dtype, vbase + t);
    dp[e] = dot;
    Di += pr[e] * dp[e];
  }
  for (int64_t e = 0; e < n; ++e) ds[e] = pr[e] * (dp[e] - Di);
}

/* Backward of the forward above for a scalar loss L with dO = dL/dO. Over the
 * allowed keys of a row, O_i = sum_j P_ij V_j with P_ij = softmax_j(S_ij) and
 * S_ij = scale Q_i . K_j. The chain rule, with the softmax Jacobian
 * dP_ij/dS_ik = P_ij (delta_jk - P_ik), gives
 *   dV_j  = sum_i P_ij dO_i
 *   dP_ij = dO_i . V_j,   D_i = sum_j P_ij dP_ij
 *   dS_ij = P_ij (dP_ij - D_i)
 *   dQ_i  = scale sum_j dS_ij K_j,   dK_j = scale sum_i dS_ij Q_i.
 * Keys no row may see get zero gradients; a row with no allowed key gets
 * dQ_i = 0 and adds nothing to dK, dV. */
int ref_backward(const ref_problem *p, const uint8_t *mask, const void *q, const void *k,
                 const void *v, const void *dout, const int64_t *qrows, int64_t nqrows,
                 int64_t klo, int64_t khi, double *dq, double *dk, double *dv, int nthreads) {
  if (check_problem(p) || p->paged) return -1;
  if (klo < 0) klo = 0;
  if (khi > p->skv) khi = p->skv;
  const int d = p->d, gs = p->hq / p->hkv;
  const int64_t kw = khi > klo ? khi - klo : 0;
  bwd_ctx c;
  c.p = p, c.mask = mask, c.q = q, c.k = k, c.v = v, c.dout = dout;
  c.scale = p->scale > 0 ? p->scale : 1.0 / sqrt((double)d);
  int64_t *moff = mask_offsets(p);
  c.moff = moff, c.unkb = 0;
  uint8_t *uni = p->gqa_union ? group_union(p, mask, moff, &c.unkb) : NULL;
  c.uni = uni;
  if (nthreads <= 0) nthreads = omp_get_max_threads();
  const int64_t nq = qrows ? nqrows : (int64_t)p->batch * p->hq * p->sq;
  const int64_t nbg = (int64_t)p->batch * p->hkv;

#pragma omp parallel num_threads(nthreads)
  {
    const size_t cap = (size_t)(p->skv ? p->skv : 1);
    double *s = (double *)malloc(sizeof(double) * cap), *pr = (double *)malloc(sizeof(double) * cap);
    double *dp = (double *)malloc(sizeof(double) * cap), *ds = (double *)malloc(sizeof(double) * cap);
    int64_t *js = (int64_t *)malloc(sizeof(int64_t) * cap);

    /* dQ of the requested rows (rows are independent). */
    if (dq) {
#pragma omp for schedule(dynamic, 8)
      for (int64_t r = 0; r < nq; ++r) {
        int64_t b, h, i;
        if (qrows) {
          b = qrows[3 * r], h = qrows[3 * r + 1], i = qrows[3 * r + 2];
        } else {
          b = r / ((int64_t)p->hq * p->sq), h = (r / p->sq) % p->hq, i = r % p->sq;
        }
        const int64_t n = row_keys(&c, b, h, i, js);
        row_gradients(&c, b, h, i, js, n, s, pr, dp, ds);
        const int g = (int)(h / gs);
        double *out = dq + r * d;
        for (int t = 0; t < d; ++t) out[t] = 0.0;
        for (int64_t e = 0; e < n; ++e) {
          const int64_t kbase = kv_index(p, NULL, (int)b, g, js[e]);
          for (int t = 0; t < d; ++t) out[t] += ds[e] * load_value(k, p->dtype, kbase + t);
        }
        for (int t = 0; t < d; ++t) out[t] *= c.scale;
      }
    }

    /* dK, dV of keys [klo, khi): one (batch, kv head) per thread, rows of the
       group's heads in (head, query) order. Output [batch][hkv][kw][d]. */
    if (dk && dv && kw > 0) {
#pragma omp for schedule(dynamic, 1)
      for (int64_t bg = 0; bg < nbg; ++bg) {
        const int64_t b = bg / p->hkv, g = bg % p->hkv;
        double *gk = dk + bg * kw * d, *gv = dv + bg * kw * d;
        for (int64_t x = 0; x < kw * d; ++x) gk[x] = 0.0, gv[x] = 0.0;
        for (int64_t h = g * gs; h < (g + 1) * gs; ++h)
          for (int64_t i = 0; i < p->sq; ++i) {
            const int64_t n = row_keys(&c, b, h, i, js);
            int64_t hit = 0;  /* rows that see no key of the window add nothing */
            for (int64_t e = 0; e < n && !hit; ++e) hit = js[e] >= klo && js[e] < khi;
            if (!hit) continue;
            row_gradients(&c, b, h, i, js, n, s, pr, dp, ds);
            const int64_t qbase = ((b * p->hq + h) * p->sq + i) * (int64_t)d;
            for (int64_t e = 0; e < n; ++e) {
              if (js[e] < klo || js[e] >= khi) continue;
              const int64_t o = (js[e] - klo) * d;
              for (int t = 0; t < d; ++t) {
                gk[o + t] += c.scale * ds[e] * load_value(q, p->dtype, qbase + t);
                gv[o + t] += pr[e] * load_value(dout, p->dtype, qbase + t);
              }
            }
          }
      }
    }
    free(s), free(pr), free(dp), free(ds), free(js);
  }
  free(moff);
  free(uni);
  return 0;
}

int ref_forward(const ref_problem *p, const uint8_t *mask, const int32_t *page_table,
                const void *q, const void *k, const void *v, int mode, const int64_t *rows,
                int64_t nrows, double *o, double *lse, int nthreads) {
  return forward_impl(p, mask, page_table, q, k, v, NULL, NULL, mode, rows, nrows, o, lse, nthreads);
}

int ref_forward_kv8(const ref_problem *p, const uint8_t *mask, const int32_t *page_table,
                    const void *q, const uint8_t *k, const uint8_t *v, const float *k_scale,
                    const float *v_scale, int mode, const int64_t *rows, int64_t nrows, double *o,
                    double *lse, int nthreads) {
  if (!k_scale || !v_scale || p->dtype != 0) return -1;
  return forward_impl(p, mask, page_table, q, k, v, k_scale, v_scale, mode, rows, nrows, o, lse,
                      nthreads);
}

/* ------------------------------------------------------------------------ */
/* Mask features                                                             */
/* ------------------------------------------------------------------------ */

static void features(const ref_problem *p, const uint8_t *mask, const int64_t *moff,
                     const uint8_t *uni, int64_t unkb, int64_t *out) {
  int nbm = mask_batches(p), gs = p->hq / p->hkv;
  for (int bm = 0; bm < nbm; ++bm)
    for (int h = 0; h < p->hq; ++h) {
      int64_t bq = p->bq[h], bk = p->bk[h];
      int64_t nq = ceil_div(p->sq, bq), nk = ceil_div(p->skv, bk);
      const uint8_t *m = mask + moff[bm * p->hq + h];
      const uint8_t *u = uni ? uni + ((int64_t)bm * p->hkv + h / gs) * unkb : NULL;
      int64_t nnz = 0, maxrow = 0, empty = 0, eff = 0;
      for (int64_t qb = 0; qb < nq; ++qb) {
        int64_t cnt = 0;
        int64_t qlast = ((qb + 1) * bq < p->sq ? (qb + 1) * bq : p->sq) - 1;
        for (int64_t kb = 0; kb < nk; ++kb) {
          cnt += m[qb * nk + kb] != 0;
          int sel = u ? u[kb] : m[qb * nk + kb];
          if (sel && (!p->causal || kb * bk <= qlast + p->causal_offset)) ++eff;
        }
        nnz += cnt;
        if (cnt > maxrow) maxrow = cnt;
        if (cnt == 0) ++empty;
      }
      int64_t *f = out + ((int64_t)bm * p->hq + h) * 4;
      f[0] = nnz, f[1] = maxrow, f[2] = empty, f[3] = eff;
    }
}

int ref_features(const ref_problem *p, const uint8_t *mask, int64_t *out) {
  if (check_problem(p)) return -1;
  int64_t *moff = mask_offsets(p), unkb = 0;
  uint8_t *uni = p->gqa_union ? group_union(p, mask, moff, &unkb) : NULL;
  features(p, mask, moff, uni, unkb, out);
  free(moff);
  free(uni);
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Regime lookup table (Tessera, abstract: profile-guided regime selection   */
/* through a lookup table built offline). Text format, first match wins:     */
/*   bsa-lut 1                                                              */
/*   rule D dtype union paged bq_lo bq_hi bk_lo bk_hi dens_lo dens_hi        */
/*        imb_lo imb_hi -> Tq Tk sched split pack                           */
/* D, dtype, union and paged may be '*'. Ranges are inclusive.               */
/* ------------------------------------------------------------------------ */

typedef struct {
  int tq, tk, sched, split, pack;
} regime_t;

typedef struct {
  int64_t key[4];   /* D, dtype, union, paged; -1 = any */
  int64_t lo[5], hi[5]; /* min bq, min bk, density per mille, imbalance x16, Sq (version 2) */
  regime_t r;
} rule_t;

static int next_token(const char **cur, char *tok, size_t cap) {
  const char *s = *cur;
  for (;;) {
    while (*s == ' ' || *s == '\t' || *s == '\r') ++s;
    if (*s == '#') {
      while (*s && *s != '\n') ++s;
    }
    if (*s == '\n') {
      ++s;
      continue;
    }
    break;
  }
  if (!*s) {
    *cur = s;
    return 0;
  }
  size_t n = 0;
  while (*s && *s != ' ' && *s != '\t' && *s != '\r' && *s != '\n' && *s != '#') {
    if (n + 1 >= cap) return -1;
    tok[n++] = *s++;
  }
  tok[n] = 0;
  *cur = s;
  return 1;
}

static int parse_int(const char *t, int64_t *out) {
  char *end;
  long long x = strtoll(t, &end, 10);
  if (!*t || *end) return -1;
  *out = x;
  return 0;
}

static int parse_lut(const char *text, rule_t **rules_out, int *n_out) {
  const char *cur = text;
  char tok[64];
  int64_t x;
  if (next_token(&cur, tok, sizeof tok) != 1 || strcmp(tok, "bsa-lut")) return -1;
  if (next_token(&cur, tok, sizeof tok) != 1 || parse_int(tok, &x) || (x != 1 && x != 2)) return -1;
  const int nranges = x == 2 ? 5 : 4; /* version 2 adds a range on the query length */
  int cap = 16, n = 0;
  rule_t *rules = (rule_t *)malloc(sizeof(rule_t) * cap);
  for (;;) {
    int st = next_token(&cur, tok, sizeof tok);
    if (st == 0) break;
    if (st < 0 || strcmp(tok, "rule")) goto bad;
    if (n == cap) rules = (rule_t *)realloc(rules, sizeof(rule_t) * (cap *= 2));
    rule_t *r = &rules[n];
    for (int f = 0; f < 4; ++f) {
      if (next_token(&cur, tok, sizeof tok) != 1) goto bad;
      if (!strcmp(tok, "*")) r->key[f] = -1;
      else if (f == 1 && !strcmp(tok, "bf16")) r->key[f] = 0;
      else if (f == 1 && !strcmp(tok, "f32")) r->key[f] = 1;
      else if (f != 1 && !parse_int(tok, &x) && x >= 0) r->key[f] = x;
      else goto bad;
    }
    r->lo[4] = 0, r->hi[4] = INT64_MAX;
    for (int f = 0; f < nranges; ++f) {
      if (next_token(&cur, tok, sizeof tok) != 1 || parse_int(tok, &r->lo[f])) goto bad;
      if (next_token(&cur, tok, sizeof tok) != 1 || parse_int(tok, &r->hi[f])) goto bad;
    }
    if (next_token(&cur, tok, sizeof tok) != 1 || strcmp(tok, "->")) goto bad;
    int64_t v[5];
    for (int f = 0; f < 5; ++f) {
      if (next_token(&cur, tok, sizeof tok) != 1) goto bad;
      if (f == 2 && !strcmp(tok, "local")) v[f] = 0;
      else if (f == 2 && !strcmp(tok, "lpt")) v[f] = 1;
      else if (f == 2 && !strcmp(tok, "dealt")) v[f] = 2;
      else if (f != 2 && !parse_int(tok, &v[f])) {
      } else goto bad;
    }
    if ((v[0] != 128 && v[0] != 256) || (v[1] != 64 && v[1] != 128) || v[3] < 0 ||
        v[3] > (1 << 30) || v[4] < 0 || v[4] > 2)
      goto bad;
    r->r.tq = (int)v[0], r->r.tk = (int)v[1], r->r.sched = (int)v[2];
    r->r.split = (int)v[3], r->r.pack = (int)v[4];
    ++n;
  }
  *rules_out = rules;
  *n_out = n;
  return 0;
bad:
  free(rules);
  return -1;
}

/* ------------------------------------------------------------------------ */
/* Reference planner                                                         */
/* ------------------------------------------------------------------------ */

typedef struct {
  int32_t row, e0, e1, slot;
} item_t;

typedef struct {
  uint8_t *buf;
  size_t n, cap;
} out_t;

static void put(out_t *o, const void *src, size_t bytes) {
  if (o->buf && o->n + bytes <= o->cap) memcpy(o->buf + o->n, src, bytes);
  o->n += bytes;
}

static int item_cmp(const void *a, const void *b) {
  /* LPT order: longer first; equal lengths keep their original order, which
   * the caller encodes in the slot-independent 'row-major index' key. */
  const int64_t *x = (const int64_t *)a, *y = (const int64_t *)b;
  if (x[0] != y[0]) return x[0] > y[0] ? -1 : 1;
  return x[1] < y[1] ? -1 : (x[1] > y[1]);
}

/* Query-block interleave: physical query tile t of a head whose logical
 * blocks merge mq to a tile, with interleave s, gathers the blocks
 *   (t / s) * s * mq + iq * s + t % s      (iq = 0 .. mq-1)
 * while t lies in one of the floor(nq / (s * mq)) full groups of s * mq
 * blocks, and consecutive blocks after them (s = 1 is the plain merge). The
 * tiles are a partition of the head's query blocks, so the mapping keeps
 * every selected interaction (Tessera, abstract: logical blocks retained,
 * combined or subdivided while preserving the specified interactions). */
static int64_t qblock(int64_t t, int64_t iq, int64_t s, int64_t mq, int64_t nq) {
  const int64_t g = s * mq, full = nq / g;
  if (t < full * s) return (t / s) * g + iq * s + t % s;
  return full * g + (t - full * s) * mq + iq;
}

/* Key blocks listed by the tiles of one head under interleave s: for every
 * mask batch and tile, the number of key blocks that some query block of
 * the tile selects (the mask as given, before any causal bound). */
static int64_t interleave_cost(const ref_problem *p, const uint8_t *mask, const int64_t *moff,
                               int h, int64_t mq, int64_t s) {
  const int64_t nq = ceil_div(p->sq, p->bq[h]), nk = ceil_div(p->skv, p->bk[h]);
  int64_t cost = 0;
  for (int bm = 0; bm < mask_batches(p); ++bm) {
    const uint8_t *m = mask + moff[bm * p->hq + h];
    for (int64_t t = 0; t < ceil_div(nq, mq); ++t)
      for (int64_t kb = 0; kb < nk; ++kb) {
        int any = 0;
        for (int64_t iq = 0; iq < mq && !any; ++iq) {
          const int64_t qb = qblock(t, iq, s, mq, nq);
          if (qb < nq && m[qb * nk + kb]) any = 1;
        }
        cost += any;
      }
  }
  return cost;
}

/* Key tiles listed by the query tiles of one head when its query tiles
 * take interleave sq_ (mq blocks each) and its key tiles gather mk key
 * blocks with interleave s by the same rule (qblock over the key blocks):
 * for every mask batch and query tile, the number of key tiles in which
 * some query block of the tile selects one of the tile's key blocks (the
 * mask as given). */
static int64_t key_interleave_cost(const ref_problem *p, const uint8_t *mask, const int64_t *moff,
                                   int h, int64_t mq, int64_t sq_, int64_t mk, int64_t s) {
  const int64_t nq = ceil_div(p->sq, p->bq[h]), nk = ceil_div(p->skv, p->bk[h]);
  int64_t cost = 0;
  for (int bm = 0; bm < mask_batches(p); ++bm) {
    const uint8_t *m = mask + moff[bm * p->hq + h];
    for (int64_t t = 0; t < ceil_div(nq, mq); ++t)
      for (int64_t kt = 0; kt < ceil_div(nk, mk); ++kt) {
        int any = 0;
        for (int64_t ik = 0; ik < mk && !any; ++ik) {
          const int64_t kb = qblock(kt, ik, s, mk, nk);
          for (int64_t iq = 0; iq < mq && !any && kb < nk; ++iq) {
            const int64_t qb = qblock(t, iq, sq_, mq, nq);
            if (qb < nq && m[qb * nk + kb]) any = 1;
          }
        }
        cost += any;
      }
  }
  return cost;
}

int ref_plan(const ref_problem *p, const uint8_t *mask, const int32_t *page_table,
             const char *lut_text, const int32_t *force, uint8_t *image, size_t *bytes) {
  if (check_problem(p) || !bytes || (p->paged && !page_table)) return -1;
  for (int h = 0; h < p->hq; ++h)
    if (!is_block_size(p->bq[h]) || !is_block_size(p->bk[h])) return -3;
  const int gs = p->hq / p->hkv, nbm = mask_batches(p);
  int64_t *moff = mask_offsets(p), unkb = 0;
  uint8_t *uni = p->gqa_union ? group_union(p, mask, moff, &unkb) : NULL;

  /* 1. Mask features (per mask batch and head), then plan-level aggregates. */
  int64_t *feat = (int64_t *)malloc(sizeof(int64_t) * 4 * nbm * p->hq);
  features(p, mask, moff, uni, unkb, feat);
  int64_t total_nnz = 0, total_blocks = 0, imb16 = 0, min_bq = 1 << 30, min_bk = 1 << 30;
  for (int bm = 0; bm < nbm; ++bm)
    for (int h = 0; h < p->hq; ++h) {
      int64_t nq = ceil_div(p->sq, p->bq[h]), nk = ceil_div(p->skv, p->bk[h]);
      const int64_t *f = feat + ((int64_t)bm * p->hq + h) * 4;
      total_nnz += f[0];
      total_blocks += nq * nk;
      if (f[0] > 0) {
        int64_t im = 16 * f[1] * nq / f[0];
        if (im > imb16) imb16 = im;
      }
    }
  for (int h = 0; h < p->hq; ++h) {
    if (p->bq[h] < min_bq) min_bq = p->bq[h];
    if (p->bk[h] < min_bk) min_bk = p->bk[h];
  }
  int64_t density_pm = total_blocks ? 1000 * total_nnz / total_blocks : 0;

  /* 2. Regime: forced, else the first matching table rule, else the default. */
  regime_t rg = {128, 64, 0, 0, 1};
  if (force) {
    rg.tq = force[0], rg.tk = force[1], rg.sched = force[2], rg.split = force[3], rg.pack = force[4];
    if ((rg.tq != 128 && rg.tq != 256) || (rg.tk != 64 && rg.tk != 128) || rg.sched < 0 || rg.sched > 2 ||
        rg.split < 0 || rg.pack < 0 || rg.pack > 2) {
      free(moff), free(uni), free(feat);
      return -2;
    }
  } else if (lut_text) {
    rule_t *rules;
    int nr;
    if (parse_lut(lut_text, &rules, &nr)) {
      free(moff), free(uni), free(feat);
      return -2;
    }
    int64_t key[4] = {p->d, p->dtype, p->gqa_union ? 1 : 0, p->paged ? 1 : 0};
    int64_t val[5] = {min_bq, min_bk, density_pm, imb16, p->sq};
    for (int i = 0; i < nr; ++i) {
      int ok = 1;
      for (int f = 0; f < 4; ++f)
        if (rules[i].key[f] >= 0 && rules[i].key[f] != key[f]) ok = 0;
      for (int f = 0; f < 5; ++f)
        if (val[f] < rules[i].lo[f] || val[f] > rules[i].hi[f]) ok = 0;
      if (ok) {
        rg = rules[i].r;
        break;
      }
    }
    free(rules);
  }
  /* Adjustments that make the regime valid for this problem. */
  if (!(p->gqa_union && (gs == 2 || gs == 4))) rg.pack = 0;
  if (p->dtype == 1) rg.tq = 128, rg.tk = 64; /* fp32 tiles are 128 x 64 */
  if (rg.tq == 256) rg.tk = 64;                /* 256-row tiles use 64 keys */
  if (p->paged && p->page_size % rg.tk) {
    if (rg.tk == 128 && p->page_size % 64 == 0) rg.tk = 64;
    else {
      free(moff), free(uni), free(feat);
      return -3;
    }
  }
  /* At most 32 live bits per tile: shrink Tk to 64, then Tq to 128. */
  for (;;) {
    int bad = 0;
    for (int h = 0; h < p->hq; ++h) {
      int mq = (!p->gqa_union && p->bq[h] < rg.tq) ? rg.tq / p->bq[h] : 1;
      int mk = p->bk[h] < rg.tk ? rg.tk / p->bk[h] : 1;
      if (mq * mk > 32) bad = 1;
    }
    if (!bad) break;
    if (rg.tk == 128) {
      rg.tk = 64;
    } else if (rg.tq == 256) {
      rg.tq = 128;
    } else {
      free(moff), free(uni), free(feat);
      return -3;
    }
  }
  const int64_t tq = rg.tq, tk = rg.tk;
  const int64_t tr = rg.pack ? tq / gs : tq; /* query positions per physical row */
  const int64_t nkt = ceil_div(p->skv, tk);
  const int64_t nqt = ceil_div(p->sq, tr);
  const int nlb = (p->paged || !p->mask_broadcast) ? p->batch : 1;

  /* 2b. Query-block interleave per head: 128-row tiles that merge query
   * blocks of 32 rows or more (no union) take the interleave s in
   * {1, 2, 4, 8} (s * mq <= the head's query blocks) whose tiles list the
   * fewest key blocks, the smallest s on ties; every other head takes 1. */
  int32_t *qil = (int32_t *)malloc(sizeof(int32_t) * p->hq);
  for (int h = 0; h < p->hq; ++h) {
    qil[h] = 1;
    const int64_t bq = p->bq[h], nq = ceil_div(p->sq, bq);
    if (p->gqa_union || tq != 128 || bq >= tq || bq < 32) continue;
    const int64_t mq = tq / bq;
    int64_t best = interleave_cost(p, mask, moff, h, mq, 1);
    for (int64_t s = 2; s <= 8 && s * mq <= nq; s *= 2) {
      const int64_t c = interleave_cost(p, mask, moff, h, mq, s);
      if (c < best) best = c, qil[h] = (int32_t)s;
    }
  }

  /* 2c. Key-block interleave per head: when 128 x 64 tiles merge two
   * 32-key blocks per key tile and the head's query tiles merge blocks of 32
   * or 64 rows (bf16, one query head per kv head, no union, no paging, no
   * causal bound), key tile kt gathers
   * key blocks qblock(kt, ik, s, 2, nk) for the s in {1, 2, 4, 8}
   * (2 s <= the head's key blocks) whose query tiles (with the interleave of
   * 2b) list the fewest key tiles, the smallest s on ties; every other head
   * takes 1 (key tile kt holds blocks 2 kt and 2 kt + 1). */
  int32_t *kil = (int32_t *)malloc(sizeof(int32_t) * p->hq);
  for (int h = 0; h < p->hq; ++h) {
    kil[h] = 1;
    const int64_t bq = p->bq[h], bk = p->bk[h], nk = ceil_div(p->skv, bk);
    if (p->gqa_union || p->paged || p->causal || p->dtype != 0 || p->hq != p->hkv || tq != 128 ||
        tk != 64 || bk != 32 || bq >= tq || bq < 32)
      continue;
    const int64_t mq = tq / bq, mk = tk / bk;
    int64_t best = key_interleave_cost(p, mask, moff, h, mq, qil[h], mk, 1);
    for (int64_t s = 2; s <= 8 && s * mk <= nk; s *= 2) {
      const int64_t c = key_interleave_cost(p, mask, moff, h, mq, qil[h], mk, s);
      if (c < best) best = c, kil[h] = (int32_t)s;
    }
  }

  /* 3. Physical mapping: per list, ascending key tiles with live bits over the
   * merged logical sub-blocks (keep / merge / subdivide). */
  int64_t nlists = p->gqa_union ? (int64_t)nlb * p->hkv : (int64_t)nlb * p->hq * nqt;
  int64_t *list_off = (int64_t *)malloc(sizeof(int64_t) * (nlists + 1));
  int64_t ecap = 1024, nent = 0;
  int32_t *ekt = (int32_t *)malloc(sizeof(int32_t) * ecap);
  int32_t *epage = (int32_t *)malloc(sizeof(int32_t) * ecap);
  uint32_t *elive = (uint32_t *)malloc(sizeof(uint32_t) * ecap);
  for (int64_t l = 0; l < nlists; ++l) {
    list_off[l] = nent;
    int lb, h, g;
    int64_t qt = 0;
    if (p->gqa_union) {
      lb = (int)(l / p->hkv), g = (int)(l % p->hkv), h = g * gs;
    } else {
      lb = (int)(l / ((int64_t)p->hq * nqt)), h = (int)((l / nqt) % p->hq), qt = l % nqt;
      g = h / gs;
    }
    const int bm = p->mask_broadcast ? 0 : lb;
    const int64_t bq = p->bq[h], bk = p->bk[h];
    const int64_t nq = ceil_div(p->sq, bq), nk = ceil_div(p->skv, bk);
    const int64_t mq = (!p->gqa_union && bq < tq) ? tq / bq : 1;
    const int64_t mk = bk < tk ? tk / bk : 1;
    const uint8_t *m = mask + moff[bm * p->hq + h];
    const uint8_t *u = uni ? uni + ((int64_t)bm * p->hkv + g) * unkb : NULL;
    /* Sub-block extents: aq query rows by ak keys per live bit. */
    const int64_t aq = bq < tq ? bq : tq, ak = bk < tk ? bk : tk;
    for (int64_t kt = 0; kt < nkt; ++kt) {
      uint32_t live = 0;
      for (int64_t iq = 0; iq < mq; ++iq)
        for (int64_t ik = 0; ik < mk; ++ik) {
          int64_t qb = bq < tq ? qblock(qt, iq, qil[h], mq, nq) : (qt * tq) / bq;
          int64_t kb = bk < tk ? qblock(kt, ik, kil[h], mk, nk) : (kt * tk) / bk;
          if (kb >= nk || (!u && qb >= nq)) continue;
          if (!(u ? u[kb] : m[qb * nk + kb])) continue;
          if (!u && p->causal) {
            /* Drop a sub-block whose first key lies after its last query. */
            int64_t q0 = bq < tq ? qb * bq : qt * tq;
            int64_t qlast = (q0 + aq < p->sq ? q0 + aq : p->sq) - 1;
            if (kt * tk + ik * ak > qlast + p->causal_offset) continue;
          }
          live |= 1u << (iq * mk + ik);
        }
      if (!live) continue;
      if (nent == ecap) {
        ecap *= 2;
        ekt = (int32_t *)realloc(ekt, sizeof(int32_t) * ecap);
        epage = (int32_t *)realloc(epage, sizeof(int32_t) * ecap);
        elive = (uint32_t *)realloc(elive, sizeof(uint32_t) * ecap);
      }
      ekt[nent] = (int32_t)kt;
      epage[nent] = p->paged ? page_table[(int64_t)lb * p->pages_per_seq + kt * tk / p->page_size] : -1;
      elive[nent] = live;
      ++nent;
    }
  }
  list_off[nlists] = nent;
  if (nent > INT32_MAX) {
    free(moff), free(uni), free(feat), free(list_off), free(ekt), free(epage), free(elive), free(qil);
    free(kil);
    return -3;
  }

  /* 4. Rows: one per (batch, head, q-tile), or per (batch, group, q-tile)
   * when a group's heads are packed into one task. */
  const int64_t nrows = (int64_t)p->batch * (rg.pack ? p->hkv : p->hq) * nqt;
  int32_t *row_ent = (int32_t *)malloc(sizeof(int32_t) * 2 * (nrows ? nrows : 1));
  for (int64_t r = 0; r < nrows; ++r) {
    int64_t qt = r % nqt, hh = (r / nqt) % (rg.pack ? p->hkv : p->hq);
    int b = (int)(r / (nqt * (rg.pack ? p->hkv : p->hq)));
    int lb = nlb == 1 ? 0 : b;
    int64_t l = p->gqa_union ? (int64_t)lb * p->hkv + (rg.pack ? hh : hh / gs)
                             : ((int64_t)lb * p->hq + hh) * nqt + qt;
    int64_t e0 = list_off[l], e1 = list_off[l + 1];
    if (p->gqa_union && p->causal) {
      int64_t qlast = ((qt + 1) * tr < p->sq ? (qt + 1) * tr : p->sq) - 1;
      int64_t e = e0;
      while (e < e1 && (int64_t)ekt[e] * tk <= qlast + p->causal_offset) ++e;
      e1 = e;
    }
    row_ent[2 * r] = (int32_t)e0, row_ent[2 * r + 1] = (int32_t)e1;
  }

  /* 5. Work list: rows in order, heavy rows split into balanced chunks with
   * partial-result slots and one combine record each; LPT order on request. */
  int64_t icap = nrows + 16, nitems = 0, nslots = 0, ncomb = 0;
  item_t *items = (item_t *)malloc(sizeof(item_t) * icap);
  int32_t *comb = (int32_t *)malloc(sizeof(int32_t) * 3 * (nrows ? nrows : 1));
  for (int64_t r = 0; r < nrows; ++r) {
    int64_t e0 = row_ent[2 * r], n = row_ent[2 * r + 1] - e0;
    int64_t kc = (rg.split > 0 && n > rg.split) ? ceil_div(n, rg.split) : 1;
    if (nitems + kc > icap) {
      while (nitems + kc > icap) icap *= 2;
      items = (item_t *)realloc(items, sizeof(item_t) * icap);
    }
    for (int64_t j = 0; j < kc; ++j) {
      item_t *it = &items[nitems++];
      it->row = (int32_t)r;
      it->e0 = (int32_t)(e0 + j * n / kc);
      it->e1 = (int32_t)(e0 + (j + 1) * n / kc);
      it->slot = kc > 1 ? (int32_t)(nslots + j) : -1;
    }
    if (kc > 1) {
      comb[3 * ncomb] = (int32_t)r, comb[3 * ncomb + 1] = (int32_t)nslots;
      comb[3 * ncomb + 2] = (int32_t)kc;
      ++ncomb;
      nslots += kc;
    }
  }
  if (rg.sched == 1 && nitems > 1) {
    int64_t *keys = (int64_t *)malloc(sizeof(int64_t) * 2 * nitems);
    /* Key: item length capped at 1023 (longer items tie and keep row order). */
    for (int64_t i = 0; i < nitems; ++i) {
      int64_t len = items[i].e1 - items[i].e0;
      keys[2 * i] = len < 1023 ? len : 1023, keys[2 * i + 1] = i;
    }
    qsort(keys, nitems, 2 * sizeof(int64_t), item_cmp);
    item_t *sorted = (item_t *)malloc(sizeof(item_t) * nitems);
    for (int64_t i = 0; i < nitems; ++i) sorted[i] = items[keys[2 * i + 1]];
    free(items);
    free(keys);
    items = sorted;
  }

  /* 6. Canonical image. */
  out_t o = {image, 0, image ? *bytes : 0};
  put(&o, "BSAPLAN1", 8);
  int64_t hdr[40];
  memset(hdr, 0, sizeof hdr);
  int64_t hv[] = {1, p->batch, p->hq, p->hkv, p->sq, p->skv, p->d, p->dtype, p->causal,
                  p->causal_offset, p->gqa_union, p->paged, p->page_size, p->pages_per_seq,
                  p->mask_broadcast, tq, tk, rg.sched, rg.split, rg.pack, nqt, nkt, nlists,
                  nent, nrows, nitems, nslots, ncomb, total_nnz, total_blocks, density_pm,
                  imb16, min_bq, min_bk, nlb};
  memcpy(hdr, hv, sizeof hv);
  put(&o, hdr, sizeof hdr);
  put(&o, p->bq, sizeof(int32_t) * p->hq);
  put(&o, p->bk, sizeof(int32_t) * p->hq);
  put(&o, qil, sizeof(int32_t) * p->hq);
  put(&o, kil, sizeof(int32_t) * p->hq);
  put(&o, feat, sizeof(int64_t) * 4 * nbm * p->hq);
  for (int64_t l = 0; l <= nlists; ++l) {
    int32_t x = (int32_t)list_off[l];
    put(&o, &x, 4);
  }
  put(&o, ekt, sizeof(int32_t) * nent);
  if (p->paged) put(&o, epage, sizeof(int32_t) * nent);
  put(&o, elive, sizeof(uint32_t) * nent);
  put(&o, row_ent, sizeof(int32_t) * 2 * nrows);
  put(&o, items, sizeof(item_t) * nitems);
  put(&o, comb, sizeof(int32_t) * 3 * ncomb);

  int rc = (image && o.n > *bytes) ? -4 : 0;
  *bytes = o.n;
  free(moff), free(uni), free(feat), free(list_off), free(ekt), free(epage), free(elive);
  free(row_ent), free(items), free(comb), free(qil), free(kil);
  return rc;
}

/* ------------------------------------------------------------------------ */
/* Block selection from pooled scores (the mask producer)                    */
/* ------------------------------------------------------------------------ */
/*
 * The pages name the mechanism, not a formula: hierarchical sparse attention
 * picks the top-k key/value blocks by coarse attention scores (DashAttention
 * page, summary of NSA and InfLLMv2); CompactAttention (summary) treats the
 * block mask as a KV selection signal for chunked prefill; Sol-Attn (summary)
 * thresholds per query. The coarse score here is the dot product of the mean
 * of a query block's rows with the mean of a key block's rows, and each
 * query block keeps its best key blocks among the causally feasible ones.
 *
 * Floating point decides which blocks are kept, so the arithmetic is fixed
 * and done in fp32, in this order, on both sides:
 *   mean[d] = (x_first[d] + x_second[d] + ... + x_last[d]) / n   (rows in
 *             ascending order, one fp32 addition each, one fp32 division);
 *   score   = fma(qm[D-1], km[D-1], ... fma(qm[1], km[1], fma(qm[0], km[0], 0)))
 *             (d ascending, fused multiply-add, no scale: a positive scale
 *             does not change the order).
 * Key blocks are ranked by score, higher first, ties to the lower block
 * index, under the total order of fp32 bit patterns (-NaN < -inf < ... <
 * +inf < +NaN). A query block with n candidates keeps min(top_k, n) of them
 * when top_k > 0, else ceil(n * keep_tenths / 10).
 */

/* fp32 value of element idx (bf16 bit pattern or fp32). */
static float load_f32(const void *base, int dtype, int64_t idx) {
  if (dtype == 0) {
    uint32_t bits = (uint32_t)((const uint16_t *)base)[idx] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return f;
  }
  return ((const float *)base)[idx];
}

/* Order-preserving map of an fp32 bit pattern to an unsigned integer. */
static uint32_t order_key(float f) {
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

typedef struct {
  uint32_t key;
  int32_t kb;
} cand_t;

static int cand_cmp(const void *a, const void *b) {
  const cand_t *x = (const cand_t *)a, *y = (const cand_t *)b;
  if (x->key != y->key) return x->key > y->key ? -1 : 1;  /* higher score first */
  return x->kb < y->kb ? -1 : (x->kb > y->kb);             /* then lower block */
}

int ref_select(const ref_problem *p, const int32_t *page_table, const void *q, const void *k,
               int32_t keep_tenths, int32_t top_k, uint8_t *mask) {
  if (check_problem(p) || p->mask_broadcast || !mask) return -1;
  if (top_k <= 0 && (keep_tenths < 1 || keep_tenths > 10)) return -1;
  const int gs = p->hq / p->hkv;
  const int D = p->d;
  int64_t *moff = mask_offsets(p);
  float *qm = (float *)malloc(sizeof(float) * D);
  for (int b = 0; b < p->batch; ++b)
    for (int h = 0; h < p->hq; ++h) {
      const int g = h / gs;
      const int64_t bq = p->bq[h], bk = p->bk[h];
      const int64_t nqb = ceil_div(p->sq, bq), nkb = ceil_div(p->skv, bk);
      /* pooled key blocks of (b, g) at this head's key block size */
      float *km = (float *)malloc(sizeof(float) * (size_t)(nkb > 0 ? nkb : 1) * D);
      for (int64_t kb = 0; kb < nkb; ++kb) {
        const int64_t j0 = kb * bk, j1 = (kb + 1) * bk < p->skv ? (kb + 1) * bk : p->skv;
        for (int d = 0; d < D; ++d) {
          float s = 0.0f;
          for (int64_t j = j0; j < j1; ++j) s = s + load_f32(k, p->dtype, kv_index(p, page_table, b, g, j) + d);
          km[kb * D + d] = s / (float)(j1 - j0);
        }
      }
      cand_t *c = (cand_t *)malloc(sizeof(cand_t) * (size_t)(nkb > 0 ? nkb : 1));
      for (int64_t qb = 0; qb < nqb; ++qb) {
        const int64_t i0 = qb * bq, i1 = (qb + 1) * bq < p->sq ? (qb + 1) * bq : p->sq;
        for (int d = 0; d < D; ++d) {
          float s = 0.0f;
          for (int64_t i = i0; i < i1; ++i)
            s = s + load_f32(q, p->dtype, (((int64_t)b * p->hq + h) * p->sq + i) * D + d);
          qm[d] = s / (float)(i1 - i0);
        }
        uint8_t *row = mask + moff[b * p->hq + h] + qb * nkb;
        memset(row, 0, (size_t)nkb);
        int64_t n = 0;
        for (int64_t kb = 0; kb < nkb; ++kb) {
          /* causally feasible: the block's first key is not after the block's
             last query position plus the offset */
          if (p->causal && kb * bk > (i1 - 1) + p->causal_offset) continue;
          float sc = 0.0f;
          for (int d = 0; d < D; ++d) sc = fmaf(qm[d], km[kb * D + d], sc);
          c[n].key = order_key(sc);
          c[n].kb = (int32_t)kb;
          ++n;
        }
        qsort(c, (size_t)n, sizeof(cand_t), cand_cmp);
        const int64_t keep = top_k > 0 ? (top_k < n ? top_k : n) : (n * keep_tenths + 9) / 10;
        for (int64_t t = 0; t < keep; ++t) row[c[t].kb] = 1;
      }
      free(c);
      free(km);
    }
  free(qm);
  free(moff);
  return 0;
}
