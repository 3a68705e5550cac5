/*
 * DFlash 2 drafter, CPU oracle — TEST INFRASTRUCTURE ONLY (see dflash_oracle.h).
 *
 * Source of every definition: the docs.rs page "cortiq_engine/dflash.rs"
 * (cortiq-engine 0.8.78), cited below by the item it defines; the
 * int4 format is the one the drafter's library header declares (symmetric,
 * 32 columns per f16 scale), since the page's own four-bit format is not on
 * the pages.
 *
 * Build: gcc -O2 -ffp-contract=off -fno-fast-math -fopenmp -shared -fPIC.
 */
#include "dflash_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ---------------------------------------------------------------- f16 */

static double f16_table[65536];
static int f16_ready = 0;

/* IEEE binary16 → binary64, exact: value = (1024 + m)·2^(e−25) for normal
   numbers, m·2^−24 for subnormals. */
static double f16_decode(uint16_t h) {
  int sign = h >> 15, e = (h >> 10) & 31, m = h & 1023;
  double v;
  if (e == 0)
    v = ldexp((double)m, -24);
  else if (e == 31)
    v = m ? NAN : INFINITY;
  else
    v = ldexp((double)(m + 1024), e - 25);
  return sign ? -v : v;
}

static void init_f16(void) {
  if (f16_ready) return;
  for (int h = 0; h < 65536; ++h) f16_table[h] = f16_decode((uint16_t)h);
  f16_ready = 1;
}

double orc_f16(uint16_t h) { return f16_decode(h); }

/* ------------------------------------------------------------ matrices */

/* Element (r, c) of an int4 matrix: the nibble of column c, read as a
   two's-complement value in [−8, 7], times the f16 scale of the 32-column
   group that holds c. */
static void q4_row(const orc_q4* w, int cols, int r, double* out) {
  const uint8_t* q = w->q + (size_t)r * (cols / 2);
  const uint16_t* s = w->s + (size_t)r * (cols / 32);
  for (int c = 0; c < cols; ++c) {
    int nib = (c & 1) ? (q[c / 2] >> 4) : (q[c / 2] & 15);
    int v = nib < 8 ? nib : nib - 16;
    out[c] = (double)v * f16_table[s[c / 32]];
  }
}

static void f16_row(const uint16_t* w, int cols, int r, double* out) {
  const uint16_t* p = w + (size_t)r * cols;
  for (int c = 0; c < cols; ++c) out[c] = f16_table[p[c]];
}

void orc_dequant_q4(const orc_q4* w, int rows, int cols, double* out) {
  init_f16();
#pragma omp parallel for schedule(static)
  for (int r = 0; r < rows; ++r) q4_row(w, cols, r, out + (size_t)r * cols);
}

/* y[i][r] = Σ_c W[r][c]·x[i][c] for i < m (x is [m][cols], y is [m][rows]).
   Each output is one thread's sum over c = 0, 1, …, cols−1 in order. */
static void apply(const uint16_t* wf16, const orc_q4* wq4, int rows, int cols, const double* x,
                  int m, double* y) {
  init_f16();
  double* xt = (double*)malloc(sizeof(double) * (size_t)cols * m);
  for (int i = 0; i < m; ++i)
    for (int c = 0; c < cols; ++c) xt[(size_t)c * m + i] = x[(size_t)i * cols + c];
#pragma omp parallel
  {
    double* wr = (double*)malloc(sizeof(double) * cols);
    double* acc = (double*)malloc(sizeof(double) * m);
#pragma omp for schedule(static)
    for (int r = 0; r < rows; ++r) {
      if (wq4)
        q4_row(wq4, cols, r, wr);
      else
        f16_row(wf16, cols, r, wr);
      for (int i = 0; i < m; ++i) acc[i] = 0.0;
      for (int c = 0; c < cols; ++c) {
        const double wc = wr[c];
        const double* xc = xt + (size_t)c * m;
        for (int i = 0; i < m; ++i) acc[i] += wc * xc[i];
      }
      for (int i = 0; i < m; ++i) y[(size_t)i * rows + r] = acc[i];
    }
    free(acc);
    free(wr);
  }
  free(xt);
}

void orc_apply_f16(const uint16_t* w, int rows, int cols, const double* x, int m, double* y) {
  apply(w, NULL, rows, cols, x, m, y);
}

void orc_apply_q4(const orc_q4* w, int rows, int cols, const double* x, int m, double* y) {
  apply(NULL, w, rows, cols, x, m, y);
}

/* ------------------------------------------------------ row operations */

/* `rms`: per row of `len`, x·(1/sqrt(mean(x²) + eps))·w. */
void orc_rms(const double* x, long rows, int len, const float* w, double eps, double* y) {
  for (long r = 0; r < rows; ++r) {
    const double* xr = x + r * len;
    double* yr = y + r * len;
    double ms = 0.0;
    for (int i = 0; i < len; ++i) ms += xr[i] * xr[i];
    ms /= len;
    const double s = 1.0 / sqrt(ms + eps);
    for (int i = 0; i < len; ++i) yr[i] = xr[i] * s * (double)w[i];
  }
}

/* The rotation frequencies: θ^(−2i/hd) in binary64, kept as binary32. */
void orc_inv_freq(double theta, int hd, float* out) {
  for (int i = 0; i < hd / 2; ++i) out[i] = (float)pow(theta, -(2.0 * i) / hd);
}

/* `rotate`: row r (its `heads` heads of `hd`) turned to position pos[r]. Pair
   (x_i, x_{i+hd/2}) for i < hd/2 goes to (a·c − b·s, b·c + a·s) with c, s the
   cosine and sine of the binary32 angle (float)pos·inv_freq[i]. */
void orc_rotate(double* x, long rows, int heads, int hd, const long* pos, const float* inv_freq) {
  const int half = hd / 2;
  for (long r = 0; r < rows; ++r) {
    for (int i = 0; i < half; ++i) {
      const float angle = (float)pos[r] * inv_freq[i];
      const double c = cos((double)angle), s = sin((double)angle);
      for (int h = 0; h < heads; ++h) {
        double* v = x + (r * heads + h) * hd;
        const double a = v[i], b = v[i + half];
        v[i] = a * c - b * s;
        v[i + half] = b * c + a * s;
      }
    }
  }
}

/* `conv`: the dynamic grouped causal row convolution of one stage,
   y[r][i] = Σ_{o < min(kn, r+1)} (base[stage][o][i] + d[r][stage][o][i/gs])·x[r−o][i],
   with d laid out [row][stage][offset][group]. Rows before row 0 are zero. */
void orc_conv(int rows, int hidden, int conv_group, int conv_kernel, int stage, const float* base,
              const double* d, const double* x, double* y) {
  const int groups = hidden / conv_group;
  const int kn = conv_kernel;
  for (long i = 0; i < (long)rows * hidden; ++i) y[i] = 0.0;
  for (int r = 0; r < rows; ++r) {
    const int taps = kn < r + 1 ? kn : r + 1;
    for (int o = 0; o < taps; ++o) {
      const float* b = base + (size_t)(stage * kn + o) * hidden;
      const double* dyn = d + (size_t)r * 2 * kn * groups + (size_t)(stage * kn + o) * groups;
      const double* src = x + (size_t)(r - o) * hidden;
      double* out = y + (size_t)r * hidden;
      for (int i = 0; i < hidden; ++i) out[i] += ((double)b[i] + dyn[i / conv_group]) * src[i];
    }
  }
}

/* ----------------------------------------------------------- attention */

/* One layer's attention, as `Drafter::block` runs it. The layer holds the
   context positions [first + dropped, first + len) (`Ctx::dropped`: rows
   that fell out of its window and were let go); store row i is position
   first + dropped + i, [kv][hd] binary32 per row. The layer reads positions
   [lo, hi): hi = min(a, first+len) (never below the first held position
   base = first + dropped), lo = base, or for a window w > 0 the clamp of
   a+1−w into [base, hi]. Block row r at position a+r further hides context
   positions below a+r+1−w. Every row sees all block rows (not causal).
   Scores are scale·q·k with scale = hd^−½; a softmax over the visible keys
   weights the values, the block's rows summed first and the context's
   added. */
void orc_attention(int rows, int heads, int kv_heads, int hd, const double* q, const double* k,
                   const double* v, const float* store_k, const float* store_v, long first,
                   long len, long dropped, long a, int window, double* y) {
  const int rep = heads / kv_heads;
  const double scale = 1.0 / sqrt((double)hd);
  const long base = first + dropped;
  long hi = a < first + len ? a : first + len;
  if (hi < base) hi = base;
  long lo = base;
  if (window > 0) {
    lo = a + 1 - window;
    if (lo < 0) lo = 0;
    if (lo < base) lo = base;
    if (lo > hi) lo = hi;
  }
  const long n = hi - lo;
  const long row_stride = (long)kv_heads * hd;
#pragma omp parallel
  {
    double* s = (double*)malloc(sizeof(double) * (size_t)(n + rows));
#pragma omp for schedule(static)
    for (int qi = 0; qi < rows * heads; ++qi) {
      const int r = qi / heads, h = qi % heads, g = h / rep;
      const double* qv = q + ((size_t)r * heads + h) * hd;
      long from = 0;
      if (window > 0) {
        from = a + r + 1 - window;
        if (from < 0) from = 0;
      }
      for (long p = lo; p < hi; ++p) {
        if (window > 0 && p < from) {
          s[p - lo] = -INFINITY;
          continue;
        }
        const float* kr = store_k + (p - base) * row_stride + (long)g * hd;
        double dot = 0.0;
        for (int e = 0; e < hd; ++e) dot += qv[e] * (double)kr[e];
        s[p - lo] = scale * dot;
      }
      for (int b = 0; b < rows; ++b) {
        const double* kb = k + ((size_t)b * kv_heads + g) * hd;
        double dot = 0.0;
        for (int e = 0; e < hd; ++e) dot += qv[e] * kb[e];
        s[n + b] = scale * dot;
      }
      double mx = -INFINITY;
      for (long i = 0; i < n + rows; ++i)
        if (s[i] > mx) mx = s[i];
      double sum = 0.0;
      for (long i = 0; i < n + rows; ++i) {
        s[i] = exp(s[i] - mx);
        sum += s[i];
      }
      for (long i = 0; i < n + rows; ++i) s[i] /= sum;
      double* out = y + ((size_t)r * heads + h) * hd;
      for (int e = 0; e < hd; ++e) {
        double blk = 0.0, ctx = 0.0;
        for (int b = 0; b < rows; ++b) blk += s[n + b] * v[((size_t)b * kv_heads + g) * hd + e];
        for (long p = lo; p < hi; ++p)
          ctx += s[p - lo] * (double)store_v[(p - base) * row_stride + (long)g * hd + e];
        out[e] = blk + ctx;
      }
    }
    free(s);
  }
}

/* ---------------------------------------------------------------- settle */

/* `settle_rows`: per tap row r (position pos0 + r), t = rms(fc·taps_r,
   hidden_norm); per layer K = Wk·t with each kv head normed by k_norm and
   rotated to the row's position if the layer is rotary, V = Wv·t. Both are
   kept as binary32, [layer][n][kv][hd]. */
int orc_settle(const orc_model* m, const float* taps, int n, long pos0, float* k_out,
               float* v_out) {
  init_f16();
  if (n <= 0) return 0;
  const int hs = m->hidden, tw = m->n_taps * m->hidden, kd = m->kv_heads * m->head_dim;
  const double eps = (double)(float)m->eps;
  double* x = (double*)malloc(sizeof(double) * (size_t)n * tw);
  double* t = (double*)malloc(sizeof(double) * (size_t)n * hs);
  double* kk = (double*)malloc(sizeof(double) * (size_t)n * kd);
  double* vv = (double*)malloc(sizeof(double) * (size_t)n * kd);
  long* pos = (long*)malloc(sizeof(long) * n);
  float* inv = (float*)malloc(sizeof(float) * (m->head_dim / 2));
  orc_inv_freq(m->rope_theta, m->head_dim, inv);
  for (long i = 0; i < (long)n * tw; ++i) x[i] = (double)taps[i];
  for (int r = 0; r < n; ++r) pos[r] = pos0 + r;
  orc_apply_f16(m->fc, hs, tw, x, n, t);
  orc_rms(t, n, hs, m->hidden_norm, eps, t);
  for (int l = 0; l < m->layers; ++l) {
    const orc_layer* L = &m->layer[l];
    orc_apply_q4(&L->k, kd, hs, t, n, kk);
    orc_apply_q4(&L->v, kd, hs, t, n, vv);
    orc_rms(kk, (long)n * m->kv_heads, m->head_dim, L->k_norm, eps, kk);
    if (m->rotary[l]) orc_rotate(kk, n, m->kv_heads, m->head_dim, pos, inv);
    float* ko = k_out + (size_t)l * n * kd;
    float* vo = v_out + (size_t)l * n * kd;
    for (long i = 0; i < (long)n * kd; ++i) {
      ko[i] = (float)kk[i];
      vo[i] = (float)vv[i];
    }
  }
  free(inv);
  free(pos);
  free(vv);
  free(kk);
  free(t);
  free(x);
  return 0;
}

/* ----------------------------------------------------------------- block */

static void add_into(double* h, const double* d, long count) {
  for (long i = 0; i < count; ++i) h[i] += d[i];
}

/* `Drafter::block` from the rows [E[anchor], E[mask]…] at positions a, a+1, …,
   followed by the head over the first `width` vocabulary rows and the
   selector's projection, both of rows 1..k after the last norm:
   logits [k][width], hp [k][rank]. Layer l's store holds positions
   [first + dropped[l], first + len) (dropped NULL: none dropped). `hidden`
   (or NULL) receives every row after the last norm, `trace` (or NULL) the
   residual rows after each layer, [layers][block][hidden]. */
int orc_block(const orc_model* m, const float* const* store_k, const float* const* store_v,
              long first, long len, const long* dropped, int anchor, long a, int k, int width,
              double* logits, double* hp, double* hidden, double* trace) {
  init_f16();
  const int hs = m->hidden, B = m->block, nh = m->heads, kv = m->kv_heads, hd = m->head_dim;
  const int ffn = m->intermediate, qd = nh * hd, kd = kv * hd;
  const int gs = m->conv_group, kn = m->conv_kernel, P = 2 * kn * (hs / gs);
  if (k < 1 || k >= B || width < m->selector_top || width > m->vocab) return -1;
  if (anchor < 0 || anchor >= m->vocab || len < 0) return -1;
  const double eps = (double)(float)m->eps;
  double* h = (double*)calloc((size_t)B * hs, sizeof(double));
  double* x = (double*)malloc(sizeof(double) * (size_t)B * hs);
  double* xc = (double*)malloc(sizeof(double) * (size_t)B * hs);
  double* tmp = (double*)malloc(sizeof(double) * (size_t)B * hs);
  double* d = (double*)malloc(sizeof(double) * (size_t)B * P);
  double* q = (double*)malloc(sizeof(double) * (size_t)B * qd);
  double* kk = (double*)malloc(sizeof(double) * (size_t)B * kd);
  double* vv = (double*)malloc(sizeof(double) * (size_t)B * kd);
  double* y = (double*)malloc(sizeof(double) * (size_t)B * qd);
  double* g = (double*)malloc(sizeof(double) * (size_t)B * ffn);
  double* u = (double*)malloc(sizeof(double) * (size_t)B * ffn);
  long* pos = (long*)malloc(sizeof(long) * B);
  float* inv = (float*)malloc(sizeof(float) * (hd / 2));
  orc_inv_freq(m->rope_theta, hd, inv);
  for (int r = 0; r < B; ++r) {
    pos[r] = a + r;
    const int tok = r == 0 ? anchor : m->mask_token;
    for (int i = 0; i < hs; ++i) h[(size_t)r * hs + i] = f16_table[m->embed[(size_t)tok * hs + i]];
  }
  for (int l = 0; l < m->layers; ++l) {
    const orc_layer* L = &m->layer[l];
    /* attention, wrapped in the row convolution */
    orc_rms(h, B, hs, L->in_norm, eps, x);
    orc_apply_f16(L->attn_kproj, P, hs, x, B, d);
    orc_conv(B, hs, gs, kn, 0, L->attn_base, d, x, xc);
    orc_apply_q4(&L->q, qd, hs, xc, B, q);
    orc_apply_q4(&L->k, kd, hs, xc, B, kk);
    orc_apply_q4(&L->v, kd, hs, xc, B, vv);
    orc_rms(q, (long)B * nh, hd, L->q_norm, eps, q);
    orc_rms(kk, (long)B * kv, hd, L->k_norm, eps, kk);
    if (m->rotary[l]) {
      orc_rotate(q, B, nh, hd, pos, inv);
      orc_rotate(kk, B, kv, hd, pos, inv);
    }
    orc_attention(B, nh, kv, hd, q, kk, vv, store_k[l], store_v[l], first, len,
                  dropped ? dropped[l] : 0, a, m->windows[l], y);
    orc_apply_q4(&L->o, hs, qd, y, B, tmp);
    orc_conv(B, hs, gs, kn, 1, L->attn_base, d, tmp, xc);
    add_into(h, xc, (long)B * hs);
    /* the MLP, wrapped the same way */
    orc_rms(h, B, hs, L->post_norm, eps, x);
    orc_apply_f16(L->mlp_kproj, P, hs, x, B, d);
    orc_conv(B, hs, gs, kn, 0, L->mlp_base, d, x, xc);
    orc_apply_q4(&L->gate, ffn, hs, xc, B, g);
    orc_apply_q4(&L->up, ffn, hs, xc, B, u);
    for (long i = 0; i < (long)B * ffn; ++i) g[i] = g[i] / (1.0 + exp(-g[i])) * u[i];
    orc_apply_q4(&L->down, hs, ffn, g, B, tmp);
    orc_conv(B, hs, gs, kn, 1, L->mlp_base, d, tmp, xc);
    add_into(h, xc, (long)B * hs);
    if (trace) memcpy(trace + (size_t)l * B * hs, h, sizeof(double) * (size_t)B * hs);
  }
  orc_rms(h, B, hs, m->norm, eps, x);
  if (hidden) memcpy(hidden, x, sizeof(double) * (size_t)B * hs);
  if (logits) orc_apply_f16(m->head, width, hs, x + hs, k, logits);
  if (hp) orc_apply_f16(m->sel_proj, m->selector_rank, hs, x + hs, k, hp);
  free(inv);
  free(pos);
  free(u);
  free(g);
  free(y);
  free(vv);
  free(kk);
  free(q);
  free(d);
  free(tmp);
  free(xc);
  free(x);
  free(h);
  return 0;
}

/* ---------------------------------------------------------- selection */

typedef struct {
  double v;
  int i;
} scored;

/* larger value first; among equal values the smaller index first */
static int by_value_then_index(const void* pa, const void* pb) {
  const scored* a = (const scored*)pa;
  const scored* b = (const scored*)pb;
  if (a->v > b->v) return -1;
  if (a->v < b->v) return 1;
  return (a->i > b->i) - (a->i < b->i);
}

/* `top_k`: the k largest of x, largest first, the earlier index first among
   equal values — a sort of (value, index) pairs by that order, cut at k. */
void orc_top_k(const double* x, long n, int k, double* val, int* idx) {
  scored* all = (scored*)malloc(sizeof(scored) * (size_t)n);
  for (long i = 0; i < n; ++i) {
    all[i].v = x[i];
    all[i].i = (int)i;
  }
  qsort(all, (size_t)n, sizeof(scored), by_value_then_index);
  for (int t = 0; t < k && t < n; ++t) {
    val[t] = all[t].v;
    idx[t] = all[t].i;
  }
  free(all);
}

/* `select_with`: row j's top candidates (logit, token) re-scored as
   logit + Σ_r (P[prev][r]·hp[j][r])·C[token][r], P the predecessor and C the
   successor codebook; the first strictly largest score wins and becomes
   `prev` of row j+1, the anchor being `prev` of row 0. `forced_prev` (or
   NULL) replaces prev of every row j ≥ 1 with forced_prev[j], for comparing
   rows after a disagreement. Outputs are [k][top] (cand, unary, score) and
   [k] (chosen, plain = each row's own top candidate). */
void orc_select(const orc_model* m, const double* logits, int width, const double* hp, int k,
                int anchor, const int* forced_prev, int* cand, double* unary, double* score,
                int* chosen, int* plain) {
  init_f16();
  const int rank = m->selector_rank, top = m->selector_top;
#pragma omp parallel for schedule(static)
  for (int j = 0; j < k; ++j)
    orc_top_k(logits + (size_t)j * width, width, top, unary + (size_t)j * top,
              cand + (size_t)j * top);
  double* pc = (double*)malloc(sizeof(double) * rank);
  int prev = anchor;
  for (int j = 0; j < k; ++j) {
    if (forced_prev && j > 0) prev = forced_prev[j];
    plain[j] = cand[(size_t)j * top];
    for (int r = 0; r < rank; ++r)
      pc[r] = f16_table[m->pred_book[(size_t)prev * rank + r]] * hp[(size_t)j * rank + r];
    double best = -INFINITY;
    int best_tok = cand[(size_t)j * top];
    for (int t = 0; t < top; ++t) {
      const int tok = cand[(size_t)j * top + t];
      double dot = 0.0;
      for (int r = 0; r < rank; ++r) dot += pc[r] * f16_table[m->succ_book[(size_t)tok * rank + r]];
      const double s = unary[(size_t)j * top + t] + dot;
      score[(size_t)j * top + t] = s;
      if (s > best) {
        best = s;
        best_tok = tok;
      }
    }
    chosen[j] = best_tok;
    prev = best_tok;
  }
  free(pc);
}
