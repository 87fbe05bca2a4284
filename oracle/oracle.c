/*
 * oracle.c -- plain, slow, fp64 CPU oracle for decode attention over a
 * compressed (latent) KV cache.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or helper with the GPU library; the two meet only through
 * the seeded input generators, which hold none of the method's arithmetic.
 *
 * Every function computes the plain definition of what the decode path
 * computes: softmax attention, in double precision, over values read
 * exactly from the (already bf16-rounded or fp32) inputs.  No blocking, no
 * fusion, no reordering beyond the definition: each row is an explicit
 * gather through the block table, a dot product per cache token, a max, a
 * sum of exponentials and a weighted sum.
 *
 * Sources (page title, then the part of the page):
 *   [GQLA]  "GQLA: Group-Query Latent Attention for Hardware-Adaptive Large
 *            Language Model Decoding" (gist.science explainer), technical
 *            summary section 2 "Methodology": the MQA-absorbed path (all h_q
 *            heads read the latent cache c_KV of width r_kv plus one shared
 *            RoPE key of width d^R_h), the GQA path (latent expanded into g
 *            key/value groups, 2*g*d_h per token plus the shared RoPE key),
 *            and the up-projections W_UK, W_UV indexed by group g.
 *   [X]     X post by @classiclarryd on MLA vs GQA at equal KV cache: MLA
 *            "mixes" the latent per head where GQA "copies" a KV head, and
 *            the absorb trick hides the mixing at inference.
 *   [GLA]   article on Grouped-Tied / Grouped Latent Attention (Zadouri,
 *            Strauss, Dao), section on GLA: the latent is split into a few
 *            latent heads, each shared by a group of query heads.
 *
 * Readings where the pages are silent (the tests pin each of them):
 *   - softmax scale tau is an input; scores are tau * <q, k>.
 *   - the s_q query tokens of a step already sit at cache positions
 *     L_b - s_q .. L_b - 1; with causal != 0, query token t sees cache
 *     positions [0, L_b - s_q + t]; with causal == 0 it sees [0, L_b).
 *   - LSE is the natural log of sum_j exp(score_j).
 *   - head h uses latent head / KV group / weight group h / (h_q / n).
 *   - a row with no visible cache token yields O = 0 and LSE = -inf.
 *   - W_UK and W_UV are stored [n_w][d_c][d_h]; K = c W_UK, V = c W_UV.
 *
 * Element types: dtype 0 = float32, dtype 1 = bfloat16 given as raw
 * uint16 bit patterns (a bf16 value converts to double exactly), dtype 2 =
 * float64 (used by the algebraic pins, which compare paths in double).
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_F32 0
#define ORACLE_BF16 1
#define ORACLE_F64 2

/* Read element i of a float32, bfloat16 or float64 array as a double
 * (exact in every case). */
static double elem(const void *base, int dtype, size_t i) {
  if (dtype == ORACLE_F32) return (double)((const float *)base)[i];
  if (dtype == ORACLE_F64) return ((const double *)base)[i];
  uint32_t bits = (uint32_t)((const uint16_t *)base)[i] << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

/* Cache position of logical token j of sequence b: the block table names the
 * physical page holding token j, the slot is j mod page_size. */
static size_t token_row(const int32_t *block_table, int max_pages, int page_size,
                        int b, int j) {
  int page = block_table[(size_t)b * max_pages + j / page_size];
  return (size_t)page * page_size + (size_t)(j % page_size);
}

/* Number of cache tokens query token t of sequence b may attend to. */
static int visible_len(int seqlen, int s_q, int t, int causal) {
  return causal ? seqlen - s_q + t + 1 : seqlen;
}

/* Softmax-weighted sum over n scores held in x[]: writes the weights
 * exp(x_j - m) / Z into p[] and returns LSE = m + ln Z.  n == 0 gives
 * LSE = -inf and leaves p untouched. */
static double softmax_weights(const double *x, int n, double *p) {
  if (n <= 0) return -INFINITY;
  double m = x[0];
  for (int j = 1; j < n; ++j)
    if (x[j] > m) m = x[j];
  double z = 0.0;
  for (int j = 0; j < n; ++j) {
    p[j] = exp(x[j] - m);
    z += p[j];
  }
  for (int j = 0; j < n; ++j) p[j] /= z;
  return m + log(z);
}

/* ------------------------------------------------------------------------
 * O1: MLA absorbed decode [GQLA section 2, MQA-absorbed path; GLA section
 * on latent heads for n_lat > 1].
 *
 * For row (b, t, h) with latent head l = h / (h_q / n_lat):
 *   score_j = tau * ( sum_d q_nope[b,t,h,d] * c_kv[tok_j, l, d]
 *                   + sum_e q_rope[b,t,h,e] * k_rope[tok_j, e] )
 *   O[b,t,h,:] = sum_j softmax(score)_j * c_kv[tok_j, l, :]   (latent = value)
 *   LSE[b,t,h] = ln sum_j exp(score_j)
 * over the visible tokens j, intersected with [lo_b, hi_b) when range arrays
 * are given (one split of a split-KV pass; O4).
 *
 * c_kv element (page p, slot s, latent l, d) is at
 *   (p*page_size + s) * kv_tok_stride + l*d_c + d,
 * k_rope element (p, s, e) at (p*page_size + s) * rope_tok_stride + e.
 * rows (nullable): flat row ids (b*s_q + t)*h_q + h to compute; the other
 * rows of out/lse are left untouched.  NULL computes every row.
 * ---------------------------------------------------------------------- */
typedef struct {
  int B, s_q, h_q, n_lat, d_c, d_rope, page_size, max_pages;
  double scale;
  int causal, dtype;
  const void *q_nope;   /* [B, s_q, h_q, d_c] */
  const void *q_rope;   /* [B, s_q, h_q, d_rope] */
  const void *c_kv;     /* paged, see above */
  long long kv_tok_stride;
  const void *k_rope;   /* paged, see above */
  long long rope_tok_stride;
  const int32_t *block_table; /* [B, max_pages] */
  const int32_t *seqlens;     /* [B] */
  const int32_t *range_lo;    /* [B] or NULL */
  const int32_t *range_hi;    /* [B] or NULL */
  const int32_t *rows;        /* [n_rows] or NULL */
  long long n_rows;
  double *out;                /* [B, s_q, h_q, d_c] */
  double *lse;                /* [B, s_q, h_q] */
} oracle_mla_args;

static void mla_row(const oracle_mla_args *a, long long r, double *x, double *p,
                    size_t *tok, double *o, double *lse) {
  int h = (int)(r % a->h_q);
  int t = (int)((r / a->h_q) % a->s_q);
  int b = (int)(r / ((long long)a->h_q * a->s_q));
  int l = h / (a->h_q / a->n_lat);
  int n = visible_len(a->seqlens[b], a->s_q, t, a->causal);
  int lo = a->range_lo ? a->range_lo[b] : 0;
  int hi = a->range_hi ? a->range_hi[b] : n;
  if (lo < 0) lo = 0;
  if (hi > n) hi = n;
  size_t qbase = (size_t)r * a->d_c, rbase = (size_t)r * a->d_rope;
  int cnt = 0;
  for (int j = lo; j < hi; ++j) {
    size_t row = token_row(a->block_table, a->max_pages, a->page_size, b, j);
    size_t cb = row * (size_t)a->kv_tok_stride + (size_t)l * a->d_c;
    size_t kb = row * (size_t)a->rope_tok_stride;
    double dot = 0.0;
    for (int d = 0; d < a->d_c; ++d)
      dot += elem(a->q_nope, a->dtype, qbase + d) * elem(a->c_kv, a->dtype, cb + d);
    for (int e = 0; e < a->d_rope; ++e)
      dot += elem(a->q_rope, a->dtype, rbase + e) * elem(a->k_rope, a->dtype, kb + e);
    x[cnt] = a->scale * dot;
    tok[cnt] = cb;
    ++cnt;
  }
  *lse = softmax_weights(x, cnt, p);
  for (int d = 0; d < a->d_c; ++d) o[d] = 0.0;
  for (int k = 0; k < cnt; ++k)
    for (int d = 0; d < a->d_c; ++d) o[d] += p[k] * elem(a->c_kv, a->dtype, tok[k] + d);
}

/* Largest cache length any row may see: scratch size for one row. */
static int max_seqlen(const int32_t *seqlens, int B) {
  int m = 0;
  for (int b = 0; b < B; ++b)
    if (seqlens[b] > m) m = seqlens[b];
  return m;
}

int oracle_mla_decode(const oracle_mla_args *a) {
  if (a->n_lat <= 0 || a->h_q % a->n_lat) return 1;
  long long total = (long long)a->B * a->s_q * a->h_q;
  long long count = a->rows ? a->n_rows : total;
  int L = max_seqlen(a->seqlens, a->B) + 1;
  int bad = 0;
#pragma omp parallel reduction(| : bad)
  {
    double *x = malloc(sizeof(double) * L);
    double *p = malloc(sizeof(double) * L);
    size_t *tok = malloc(sizeof(size_t) * L);
    if (!x || !p || !tok) bad = 1;
    else {
#pragma omp for schedule(dynamic, 1)
      for (long long i = 0; i < count; ++i) {
        long long r = a->rows ? a->rows[i] : i;
        mla_row(a, r, x, p, tok, a->out + (size_t)r * a->d_c, a->lse + r);
      }
    }
    free(x);
    free(p);
    free(tok);
  }
  return bad ? 2 : 0;
}

/* Softmax weights of one MLA row (b, t, h) over its visible tokens, for the
 * normalisation check (weights must sum to one).  Returns the number of
 * weights written to p_out (capacity cap). */
int oracle_mla_row_weights(const oracle_mla_args *a, int b, int t, int h, double *p_out,
                           int cap) {
  int n = visible_len(a->seqlens[b], a->s_q, t, a->causal);
  if (n > cap || n < 0) return -1;
  double *x = malloc(sizeof(double) * (n + 1));
  double *p = malloc(sizeof(double) * (n + 1));
  size_t *tok = malloc(sizeof(size_t) * (n + 1));
  double *o = malloc(sizeof(double) * a->d_c);
  double lse;
  oracle_mla_args one = *a;
  one.range_lo = one.range_hi = NULL;
  mla_row(&one, ((long long)b * a->s_q + t) * a->h_q + h, x, p, tok, o, &lse);
  memcpy(p_out, p, sizeof(double) * n);
  free(x);
  free(p);
  free(tok);
  free(o);
  return n;
}

/* ------------------------------------------------------------------------
 * O3: grouped-query decode over an expanded cache [GQLA section 2, GQA
 * path; plain GQA when d_rope == 0].
 *
 * For row (b, t, h) with KV head g = h / (h_q / n_kv):
 *   score_j = tau * ( sum_d q[b,t,h,d] * K[tok_j, g, d]
 *                   + sum_e q_rope[b,t,h,e] * k_rope[tok_j, e] )   (rope optional)
 *   O[b,t,h,:] = sum_j softmax(score)_j * V[tok_j, g, :]
 * K element (p, s, g, d) at (p*page_size + s)*k_tok_stride + g*d_h + d, V
 * likewise with v_tok_stride; shared k_rope as in O1.
 * ---------------------------------------------------------------------- */
typedef struct {
  int B, s_q, h_q, n_kv, d_h, d_rope, page_size, max_pages;
  double scale;
  int causal, dtype;
  const void *q;        /* [B, s_q, h_q, d_h] */
  const void *q_rope;   /* [B, s_q, h_q, d_rope] or NULL when d_rope == 0 */
  const void *k_cache;
  long long k_tok_stride;
  const void *v_cache;
  long long v_tok_stride;
  const void *k_rope;   /* or NULL when d_rope == 0 */
  long long rope_tok_stride;
  const int32_t *block_table;
  const int32_t *seqlens;
  const int32_t *rows;
  long long n_rows;
  double *out;          /* [B, s_q, h_q, d_h] */
  double *lse;          /* [B, s_q, h_q] */
} oracle_gqa_args;

static void gqa_row(const oracle_gqa_args *a, long long r, double *x, double *p,
                    size_t *tok) {
  int h = (int)(r % a->h_q);
  int t = (int)((r / a->h_q) % a->s_q);
  int b = (int)(r / ((long long)a->h_q * a->s_q));
  int g = h / (a->h_q / a->n_kv);
  int n = visible_len(a->seqlens[b], a->s_q, t, a->causal);
  size_t qbase = (size_t)r * a->d_h, rbase = (size_t)r * a->d_rope;
  for (int j = 0; j < n; ++j) {
    size_t row = token_row(a->block_table, a->max_pages, a->page_size, b, j);
    size_t kb = row * (size_t)a->k_tok_stride + (size_t)g * a->d_h;
    double dot = 0.0;
    for (int d = 0; d < a->d_h; ++d)
      dot += elem(a->q, a->dtype, qbase + d) * elem(a->k_cache, a->dtype, kb + d);
    for (int e = 0; e < a->d_rope; ++e)
      dot += elem(a->q_rope, a->dtype, rbase + e) *
             elem(a->k_rope, a->dtype, row * (size_t)a->rope_tok_stride + e);
    x[j] = a->scale * dot;
    tok[j] = row * (size_t)a->v_tok_stride + (size_t)g * a->d_h;
  }
  a->lse[r] = softmax_weights(x, n, p);
  double *o = a->out + (size_t)r * a->d_h;
  for (int d = 0; d < a->d_h; ++d) o[d] = 0.0;
  for (int j = 0; j < n; ++j)
    for (int d = 0; d < a->d_h; ++d) o[d] += p[j] * elem(a->v_cache, a->dtype, tok[j] + d);
}

int oracle_gqa_decode(const oracle_gqa_args *a) {
  if (a->n_kv <= 0 || a->h_q % a->n_kv) return 1;
  long long total = (long long)a->B * a->s_q * a->h_q;
  long long count = a->rows ? a->n_rows : total;
  int L = max_seqlen(a->seqlens, a->B) + 1;
  int bad = 0;
#pragma omp parallel reduction(| : bad)
  {
    double *x = malloc(sizeof(double) * L);
    double *p = malloc(sizeof(double) * L);
    size_t *tok = malloc(sizeof(size_t) * L);
    if (!x || !p || !tok) bad = 1;
    else {
#pragma omp for schedule(dynamic, 1)
      for (long long i = 0; i < count; ++i) gqa_row(a, a->rows ? a->rows[i] : i, x, p, tok);
    }
    free(x);
    free(p);
    free(tok);
  }
  return bad ? 2 : 0;
}

/* ------------------------------------------------------------------------
 * O2: explicit (non-absorbed) MLA / GQLA decode [X post: per-head "mixing"
 * of the latent; GQLA section 2: up-projections indexed by group].
 *
 * Weights W_UK, W_UV are [n_w, d_c, d_h]; head h uses w = h / (h_q / n_w)
 * (n_w = h_q: one matrix per head, MLA; n_w = g: GQLA).  The latent of every
 * visible token is expanded on the fly:
 *   k_{h,j} = [ c_j W_UK[w] ; r_j ],   v_{h,j} = c_j W_UV[w]
 * and standard attention runs with the un-absorbed query
 *   q_h = [ q_nope_h (d_h) ; q_rope_h (d_rope) ]:
 *   o[b,t,h,:] = sum_j softmax(tau <q_h, k_{h,j}>)_j v_{h,j}.
 * Single latent head (n_lat = 1).  Query and weights are double arrays.
 * ---------------------------------------------------------------------- */
typedef struct {
  int B, s_q, h_q, n_w, d_c, d_h, d_rope, page_size, max_pages;
  double scale;
  int causal, dtype;            /* dtype of the cache */
  const double *q_nope;         /* [B, s_q, h_q, d_h] (not absorbed) */
  const double *q_rope;         /* [B, s_q, h_q, d_rope] */
  const double *w_uk;           /* [n_w, d_c, d_h] */
  const double *w_uv;           /* [n_w, d_c, d_h] */
  const void *c_kv;
  long long kv_tok_stride;
  const void *k_rope;
  long long rope_tok_stride;
  const int32_t *block_table;
  const int32_t *seqlens;
  double *out;                  /* [B, s_q, h_q, d_h] */
  double *lse;                  /* [B, s_q, h_q] */
} oracle_explicit_args;

int oracle_mla_explicit(const oracle_explicit_args *a) {
  if (a->n_w <= 0 || a->h_q % a->n_w) return 1;
  long long total = (long long)a->B * a->s_q * a->h_q;
  int L = max_seqlen(a->seqlens, a->B) + 1;
  int bad = 0;
#pragma omp parallel reduction(| : bad)
  {
    double *x = malloc(sizeof(double) * L);
    double *p = malloc(sizeof(double) * L);
    double *k = malloc(sizeof(double) * a->d_h);
    double *v = malloc(sizeof(double) * (size_t)L * a->d_h);
    if (!x || !p || !k || !v) bad = 1;
    else {
#pragma omp for schedule(dynamic, 1)
      for (long long r = 0; r < total; ++r) {
        int h = (int)(r % a->h_q);
        int t = (int)((r / a->h_q) % a->s_q);
        int b = (int)(r / ((long long)a->h_q * a->s_q));
        int w = h / (a->h_q / a->n_w);
        const double *wk = a->w_uk + (size_t)w * a->d_c * a->d_h;
        const double *wv = a->w_uv + (size_t)w * a->d_c * a->d_h;
        int n = visible_len(a->seqlens[b], a->s_q, t, a->causal);
        for (int j = 0; j < n; ++j) {
          size_t row = token_row(a->block_table, a->max_pages, a->page_size, b, j);
          size_t cb = row * (size_t)a->kv_tok_stride;
          /* expand the latent of token j into this head's key and value */
          for (int e = 0; e < a->d_h; ++e) {
            k[e] = 0.0;
            v[(size_t)j * a->d_h + e] = 0.0;
          }
          for (int d = 0; d < a->d_c; ++d) {
            double c = elem(a->c_kv, a->dtype, cb + d);
            for (int e = 0; e < a->d_h; ++e) {
              k[e] += c * wk[(size_t)d * a->d_h + e];
              v[(size_t)j * a->d_h + e] += c * wv[(size_t)d * a->d_h + e];
            }
          }
          double dot = 0.0;
          for (int e = 0; e < a->d_h; ++e) dot += a->q_nope[(size_t)r * a->d_h + e] * k[e];
          for (int e = 0; e < a->d_rope; ++e)
            dot += a->q_rope[(size_t)r * a->d_rope + e] *
                   elem(a->k_rope, a->dtype, row * (size_t)a->rope_tok_stride + e);
          x[j] = a->scale * dot;
        }
        a->lse[r] = softmax_weights(x, n, p);
        double *o = a->out + (size_t)r * a->d_h;
        for (int e = 0; e < a->d_h; ++e) o[e] = 0.0;
        for (int j = 0; j < n; ++j)
          for (int e = 0; e < a->d_h; ++e) o[e] += p[j] * v[(size_t)j * a->d_h + e];
      }
    }
    free(x);
    free(p);
    free(k);
    free(v);
  }
  return bad ? 2 : 0;
}

/* ------------------------------------------------------------------------
 * Absorb trick, the two steps either side of the absorbed decode [GQLA
 * section 2, MQA-absorbed path: the up-projections fold into the query and
 * output projections; X post: absorb hides the mixing].
 *   q'_h = W_UK[w(h)] q_nope_h         (d_h -> d_c)
 *   o_h  = O'_h W_UV[w(h)]             (d_c -> d_h)
 * rows = B*s_q*h_q rows of length d_h (absorb) or d_c (up-project).
 * ---------------------------------------------------------------------- */
void oracle_absorb_query(long long rows, int h_q, int n_w, int d_c, int d_h,
                         const double *q_nope, const double *w_uk, double *q_abs) {
  for (long long r = 0; r < rows; ++r) {
    int w = (int)(r % h_q) / (h_q / n_w);
    const double *wk = w_uk + (size_t)w * d_c * d_h;
    for (int d = 0; d < d_c; ++d) {
      double s = 0.0;
      for (int e = 0; e < d_h; ++e) s += wk[(size_t)d * d_h + e] * q_nope[(size_t)r * d_h + e];
      q_abs[(size_t)r * d_c + d] = s;
    }
  }
}

void oracle_up_project(long long rows, int h_q, int n_w, int d_c, int d_h,
                       const double *o_latent, const double *w_uv, double *o) {
  for (long long r = 0; r < rows; ++r) {
    int w = (int)(r % h_q) / (h_q / n_w);
    const double *wv = w_uv + (size_t)w * d_c * d_h;
    for (int e = 0; e < d_h; ++e) {
      double s = 0.0;
      for (int d = 0; d < d_c; ++d) s += o_latent[(size_t)r * d_c + d] * wv[(size_t)d * d_h + e];
      o[(size_t)r * d_h + e] = s;
    }
  }
}

/* ------------------------------------------------------------------------
 * O5: latent expansion at cache-write time [GQLA section 2, GQA path: the
 * latent is expanded into g key/value groups once, no per-step expansion].
 * For every valid token j < L_b of every sequence b, with row = the cache
 * position of j (same page ids as the latent cache):
 *   K[row, g, :] = c_kv[row, :] W_UK[g],   V[row, g, :] = c_kv[row, :] W_UV[g]
 * Outputs are double arrays with k_tok_stride = v_tok_stride = g*d_h; rows
 * of invalid tokens are left untouched.  start_pos (nullable) skips tokens
 * j < start_pos[b] (append-only expansion).
 * ---------------------------------------------------------------------- */
typedef struct {
  int B, g, d_c, d_h, page_size, max_pages, dtype;
  const void *c_kv;
  long long kv_tok_stride;
  const double *w_uk;   /* [g, d_c, d_h] */
  const double *w_uv;   /* [g, d_c, d_h] */
  const int32_t *block_table;
  const int32_t *seqlens;
  const int32_t *start_pos;
  double *k_out;
  double *v_out;
} oracle_expand_args;

int oracle_expand_latent(const oracle_expand_args *a) {
  for (int b = 0; b < a->B; ++b) {
    int j0 = a->start_pos ? a->start_pos[b] : 0;
#pragma omp parallel for schedule(static)
    for (int j = j0; j < a->seqlens[b]; ++j) {
      size_t row = token_row(a->block_table, a->max_pages, a->page_size, b, j);
      for (int g = 0; g < a->g; ++g) {
        const double *wk = a->w_uk + (size_t)g * a->d_c * a->d_h;
        const double *wv = a->w_uv + (size_t)g * a->d_c * a->d_h;
        double *ko = a->k_out + (row * a->g + g) * (size_t)a->d_h;
        double *vo = a->v_out + (row * a->g + g) * (size_t)a->d_h;
        for (int e = 0; e < a->d_h; ++e) {
          double sk = 0.0, sv = 0.0;
          for (int d = 0; d < a->d_c; ++d) {
            double c = elem(a->c_kv, a->dtype, row * (size_t)a->kv_tok_stride + d);
            sk += c * wk[(size_t)d * a->d_h + e];
            sv += c * wv[(size_t)d * a->d_h + e];
          }
          ko[e] = sk;
          vo[e] = sv;
        }
      }
    }
  }
  return 0;
}

/* ------------------------------------------------------------------------
 * O4 combine: merge split-KV partial results.  For sequence b with works
 * w in [off[b], off[b+1]) and every (t, h):
 *   LSE = ln sum_w exp(LSE_w),   O = sum_w exp(LSE_w - LSE) O_w
 * A work with LSE_w = -inf (empty split) has weight 0.  No work at all, or
 * all empty, gives O = 0 and LSE = -inf.
 * ---------------------------------------------------------------------- */
void oracle_lse_combine(int B, int s_q, int h_q, int d_v, const double *o_part,
                        const double *lse_part, const int32_t *work_offsets, double *out,
                        double *lse) {
  size_t rows = (size_t)s_q * h_q;
  for (int b = 0; b < B; ++b) {
    for (size_t r = 0; r < rows; ++r) {
      double m = -INFINITY;
      for (int w = work_offsets[b]; w < work_offsets[b + 1]; ++w)
        if (lse_part[(size_t)w * rows + r] > m) m = lse_part[(size_t)w * rows + r];
      double *o = out + ((size_t)b * rows + r) * d_v;
      for (int d = 0; d < d_v; ++d) o[d] = 0.0;
      if (m == -INFINITY) {
        lse[(size_t)b * rows + r] = -INFINITY;
        continue;
      }
      double z = 0.0;
      for (int w = work_offsets[b]; w < work_offsets[b + 1]; ++w)
        z += exp(lse_part[(size_t)w * rows + r] - m);
      double total = m + log(z);
      for (int w = work_offsets[b]; w < work_offsets[b + 1]; ++w) {
        double wt = exp(lse_part[(size_t)w * rows + r] - total);
        const double *ow = o_part + ((size_t)w * rows + r) * d_v;
        for (int d = 0; d < d_v; ++d) o[d] += wt * ow[d];
      }
      lse[(size_t)b * rows + r] = total;
    }
  }
}

int oracle_num_threads(void) {
#ifdef _OPENMP
  extern int omp_get_max_threads(void);
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Thread count for the OpenMP loops of later calls (timing of the oracle on
 * one core or on all of them; no effect on the arithmetic). */
void oracle_set_num_threads(int n) {
#ifdef _OPENMP
  extern void omp_set_num_threads(int);
  omp_set_num_threads(n > 0 ? n : 1);
#else
  (void)n;
#endif
}
