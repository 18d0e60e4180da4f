/*
 * ORACLE — test infrastructure only.
 *
 * A plain, slow, obviously correct CPU implementation of what the
 * aggregation kernels compute, in fp64.  Only the test suite, the smoke
 * check and the CPU-baseline leg of the benchmark may load it; the library
 * path never does.  It shares no code with the HIP sources.
 *
 * Source of every definition: Fomina et al., "On efficient scaling of GNNs
 * via IO-aware layer implementations" (the IO-aware GNN layers paper), and
 * for RCM the textbook Cuthill-McKee ordering named in Tang et al., "A
 * High-Throughput Solver for Marginalized Graph Kernels on GPU", section on
 * graph reordering.  Each function cites its passage.
 *
 * Conventions (shared with the kernels' contract, stated here again so the
 * oracle stands on its own):
 *   - CSR rows are destinations: row i lists the sources j of edges j -> i,
 *     col_idx[row_ptr[i] .. row_ptr[i+1]).
 *   - deg_in(i) = length of row i; deg_out(j) = number of entries equal to j;
 *     both count self loops present in the CSR.
 *   - bf16 inputs are decoded exactly (bits << 16 -> float -> double).
 *   - `rows` selects which destination rows to evaluate (NULL = all, in
 *     order); outputs are packed [n_sel x ...] in that order.
 *
 * Return codes: 0 ok, -1 invalid argument, -2 allocation failure,
 * -3 internal check failed (softmax weights not summing to 1).
 *
 * Pins: every function here is checked by the CPU test suite against a
 * dense brute force, a closed form, an invariant or a textbook special
 * case; none is "parity unpinned".
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <math.h>
#include <omp.h>

static double bf16_to_double(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

static double load_x(const void* X, int x_bf16, int64_t idx) {
  if (x_bf16) return bf16_to_double(((const uint16_t*)X)[idx]);
  return (double)((const float*)X)[idx];
}

int oracle_num_threads(void) { return omp_get_max_threads(); }

/* Threads for the following calls (n <= 0 leaves the setting unchanged). */
void oracle_set_threads(int n) {
  if (n > 0) omp_set_num_threads(n);
}

/* Degrees (paper: SpMM convolutions appendix, "normalisation as a
 * preprocessing step" — node degrees precomputed from the CSR). */
int oracle_degrees(int32_t n_rows, int32_t n_cols, const int32_t* row_ptr, const int32_t* col_idx,
                   int32_t* deg_in, int32_t* deg_out) {
  if (n_rows < 0 || n_cols < 0 || !row_ptr) return -1;
  for (int32_t i = 0; i < n_rows; ++i) {
    if (deg_in) deg_in[i] = row_ptr[i + 1] - row_ptr[i];
  }
  if (deg_out) {
    for (int32_t j = 0; j < n_cols; ++j) deg_out[j] = 0;
    for (int32_t i = 0; i < n_rows; ++i)
      for (int32_t e = row_ptr[i]; e < row_ptr[i + 1]; ++e) {
        int32_t j = col_idx[e];
        if (j < 0 || j >= n_cols) return -1;
        deg_out[j] += 1;
      }
  }
  return 0;
}

/* Edge weight of entry (i <- j) under a normalisation mode (paper: section
 * on the three operator families, GCN weight 1/sqrt(deg(i) deg(j)); and the
 * SpMM appendix naming the modes none / left / right / both):
 *   0 NONE : 1
 *   1 LEFT : 1 / deg_in(i)
 *   2 RIGHT: 1 / deg_out(j)
 *   3 BOTH : 1 / sqrt(deg_in(i) * deg_out(j))
 * multiplied by the given edge value when one is supplied. */
static double edge_weight(int norm, int32_t din_i, int32_t dout_j, const float* edge_val, int64_t e) {
  double w = 1.0;
  if (norm == 1) w = 1.0 / (double)din_i;
  else if (norm == 2) w = 1.0 / (double)dout_j;
  else if (norm == 3) w = 1.0 / sqrt((double)din_i * (double)dout_j);
  if (edge_val) w *= (double)edge_val[e];
  return w;
}

/* SpMM: Y[i, f] = sum_e w_e * X[col_e, f]  (paper: SpMM-based convolutions,
 * H' = sigma(A~ C); the appendix's Y = A X).  Yabs[i, f] = sum_e |w_e X|
 * is the magnitude used to scale errors. */
int oracle_spmm(int32_t n_rows, int32_t n_cols, const int32_t* row_ptr, const int32_t* col_idx,
                const float* edge_val, int norm, const void* X, int x_bf16, int32_t F, int64_t ldx,
                int64_t n_sel, const int32_t* rows, double* Y, double* Yabs) {
  if (!row_ptr || !col_idx || !X || !Y || F <= 0 || ldx < F || norm < 0 || norm > 3) return -1;
  int32_t* dout = NULL;
  if (norm == 2 || norm == 3) {
    dout = (int32_t*)malloc((size_t)(n_cols > 0 ? n_cols : 1) * 4);
    if (!dout) return -2;
    if (oracle_degrees(n_rows, n_cols, row_ptr, col_idx, NULL, dout)) {
      free(dout);
      return -1;
    }
  }
  if (!rows) n_sel = n_rows;
  int bad = 0;
#pragma omp parallel for schedule(dynamic, 64)
  for (int64_t s = 0; s < n_sel; ++s) {
    int32_t i = rows ? rows[s] : (int32_t)s;
    double* y = Y + s * F;
    double* ya = Yabs ? Yabs + s * F : NULL;
    for (int32_t f = 0; f < F; ++f) {
      y[f] = 0.0;
      if (ya) ya[f] = 0.0;
    }
    if (i < 0 || i >= n_rows) {
      bad = 1;
      continue;
    }
    int32_t din = row_ptr[i + 1] - row_ptr[i];
    for (int32_t e = row_ptr[i]; e < row_ptr[i + 1]; ++e) {
      int32_t j = col_idx[e];
      double w = edge_weight(norm, din, dout ? dout[j] : 0, edge_val, e);
      for (int32_t f = 0; f < F; ++f) {
        double t = w * load_x(X, x_bf16, (int64_t)j * ldx + f);
        y[f] += t;
        if (ya) ya[f] += fabs(t);
      }
    }
  }
  free(dout);
  return bad ? -1 : 0;
}

/* IEEE-754 total order on non-NaN values, with -0.0 < +0.0 (paper: reduction
 * appendix, order-preserving key — "smaller float, smaller key"; signed zero
 * is ordered as the bit patterns order it). */
static int less_total(float a, float b) {
  if (a < b) return 1;
  if (a > b) return 0;
  return signbit(a) && !signbit(b);
}

/* Segmented reductions (paper: reduction-based aggregations; reduction
 * appendix on light / heavy nodes and the packed (value, index) merge):
 *   op 0 SUM : sum_j X[j, f]
 *   op 1 MEAN: SUM / deg_in(i), 0 for an empty row
 *   op 2 MAX : largest X[j, f] under the total order; ties -> smallest j
 *   op 3 MIN : smallest X[j, f] under the total order; ties -> smallest j
 * Empty rows give 0 (and arg -1 for MAX / MIN).  MAX / MIN results are
 * inputs, returned exactly (as double). */
int oracle_reduce(int32_t n_rows, const int32_t* row_ptr, const int32_t* col_idx, const float* X,
                  int32_t F, int64_t ldx, int op, int64_t n_sel, const int32_t* rows, double* Y,
                  int32_t* arg, double* Yabs) {
  if (!row_ptr || !col_idx || !X || !Y || F <= 0 || ldx < F || op < 0 || op > 3) return -1;
  if (!rows) n_sel = n_rows;
  int bad = 0;
#pragma omp parallel for schedule(dynamic, 64)
  for (int64_t s = 0; s < n_sel; ++s) {
    int32_t i = rows ? rows[s] : (int32_t)s;
    double* y = Y + s * F;
    if (i < 0 || i >= n_rows) {
      bad = 1;
      continue;
    }
    int32_t b = row_ptr[i], en = row_ptr[i + 1];
    for (int32_t f = 0; f < F; ++f) {
      if (op <= 1) {
        double acc = 0.0, aa = 0.0;
        for (int32_t e = b; e < en; ++e) {
          double v = (double)X[(int64_t)col_idx[e] * ldx + f];
          acc += v;
          aa += fabs(v);
        }
        if (op == 1 && en > b) {
          acc /= (double)(en - b);
          aa /= (double)(en - b);
        }
        y[f] = acc;
        if (Yabs) Yabs[s * F + f] = aa;
        if (arg) arg[s * F + f] = -1;
      } else {
        int32_t best_j = -1;
        float best = 0.0f;
        for (int32_t e = b; e < en; ++e) {
          int32_t j = col_idx[e];
          float v = X[(int64_t)j * ldx + f];
          int better;
          if (best_j < 0) better = 1;
          else if (op == 2) better = less_total(best, v) || (!less_total(v, best) && j < best_j);
          else better = less_total(v, best) || (!less_total(best, v) && j < best_j);
          if (better) {
            best = v;
            best_j = j;
          }
        }
        y[f] = (best_j < 0) ? 0.0 : (double)best;
        if (arg) arg[s * F + f] = best_j;
        if (Yabs) Yabs[s * F + f] = fabs(y[f]);
      }
    }
  }
  return bad ? -1 : 0;
}

/* Element idx of a per-vertex attention input: bf16 bits (f64 = 0) or
 * float64 values (f64 = 1, the exact projections of the layer-level GATv2). */
static double load_att(const void* V, int f64, int64_t idx) {
  if (f64) return ((const double*)V)[idx];
  return bf16_to_double(((const uint16_t*)V)[idx]);
}

/* Softmax aggregation shared by both attention layers, two passes (paper:
 * attention-based layers, h_i' = sum_j alpha_ij v_j with alpha = softmax of
 * e_ij over the row; logsumexp kept per (i, h)).  logits[0..deg) for one
 * (i, h) are given; v rows come from V (bf16, or float64 if v_f64) at
 * V[j, h, :].  Returns 0, or -3 if the weights do not sum to 1 within 1e-12. */
static int softmax_aggregate(const double* logits, const int32_t* cols, int32_t deg,
                             const void* V, int v_f64, int32_t H, int32_t D, int32_t h, double* out,
                             double* lse, double* vabs) {
  for (int32_t d = 0; d < D; ++d) {
    out[d] = 0.0;
    if (vabs) vabs[d] = 0.0;
  }
  if (deg == 0) {
    *lse = -INFINITY;
    return 0;
  }
  double m = -INFINITY;
  for (int32_t k = 0; k < deg; ++k)
    if (logits[k] > m) m = logits[k];
  double ssum = 0.0;
  for (int32_t k = 0; k < deg; ++k) ssum += exp(logits[k] - m);
  double asum = 0.0;
  for (int32_t k = 0; k < deg; ++k) {
    double alpha = exp(logits[k] - m) / ssum;
    asum += alpha;
    const int64_t vj = ((int64_t)cols[k] * H + h) * D;
    for (int32_t d = 0; d < D; ++d) {
      double v = load_att(V, v_f64, vj + d);
      out[d] += alpha * v;
      if (vabs) vabs[d] += alpha * fabs(v);
    }
  }
  *lse = m + log(ssum);
  return fabs(asum - 1.0) < 1e-12 ? 0 : -3;
}

/* GATv2 (paper: section on the three families, e_ij = a^T LeakyReLU(W_l h_i
 * + W_r h_j), v_j = W_r h_j; fused GATv2 appendix, l_i and r_j precomputed
 * per vertex).  xl [n_rows, H, D] and xr [n_cols, H, D], bf16 bits or (f64)
 * float64; att [H, D] fp32; LeakyReLU(z) = z if z > 0 else slope * z.
 * out [n_sel, H, D], lse [n_sel, H], vabs [n_sel, H, D] (sum_j alpha |r_j|). */
static int gatv2_impl(int32_t n_rows, const int32_t* row_ptr, const int32_t* col_idx, const void* xl,
                      const void* xr, int f64, const float* att, int32_t H, int32_t D, float slope,
                      int64_t n_sel, const int32_t* rows, double* out, double* lse, double* vabs) {
  if (!row_ptr || !col_idx || !xl || !xr || !att || !out || !lse || H <= 0 || D <= 0) return -1;
  if (!rows) n_sel = n_rows;
  int bad = 0;
  double sl = (double)slope;
#pragma omp parallel
  {
    int32_t cap = 0;
    double* logits = NULL;
#pragma omp for schedule(dynamic, 16)
    for (int64_t s = 0; s < n_sel; ++s) {
      int32_t i = rows ? rows[s] : (int32_t)s;
      if (i < 0 || i >= n_rows) {
        bad = 1;
        continue;
      }
      int32_t b = row_ptr[i], deg = row_ptr[i + 1] - b;
      if (deg > cap) {
        free(logits);
        cap = deg;
        logits = (double*)malloc((size_t)cap * 8);
        if (!logits) {
          bad = 1;
          cap = 0;
          continue;
        }
      }
      for (int32_t h = 0; h < H; ++h) {
        const int64_t li = ((int64_t)i * H + h) * D;
        for (int32_t k = 0; k < deg; ++k) {
          const int64_t rj = ((int64_t)col_idx[b + k] * H + h) * D;
          double e = 0.0;
          for (int32_t d = 0; d < D; ++d) {
            double z = load_att(xl, f64, li + d) + load_att(xr, f64, rj + d);
            double act = z > 0.0 ? z : sl * z;
            e += (double)att[h * D + d] * act;
          }
          logits[k] = e;
        }
        int rc = softmax_aggregate(logits, col_idx + b, deg, xr, f64, H, D, h, out + (s * H + h) * D,
                                   lse + s * H + h, vabs ? vabs + (s * H + h) * D : NULL);
        if (rc) bad = 2;
      }
    }
    free(logits);
  }
  return bad == 2 ? -3 : (bad ? -1 : 0);
}

int oracle_gatv2(int32_t n_rows, const int32_t* row_ptr, const int32_t* col_idx, const uint16_t* xl,
                 const uint16_t* xr, const float* att, int32_t H, int32_t D, float slope, int64_t n_sel,
                 const int32_t* rows, double* out, double* lse, double* vabs) {
  return gatv2_impl(n_rows, row_ptr, col_idx, xl, xr, 0, att, H, D, slope, n_sel, rows, out, lse, vabs);
}

/* The same GATv2 from float64 per-vertex vectors: the layer as section 2.2
 * of the paper defines it, l_i = W_l h_i and r_j = W_r h_j taken exactly
 * (oracle_project) instead of rounded to an input format. */
int oracle_gatv2_f64(int32_t n_rows, const int32_t* row_ptr, const int32_t* col_idx, const double* xl,
                     const double* xr, const float* att, int32_t H, int32_t D, float slope, int64_t n_sel,
                     const int32_t* rows, double* out, double* lse, double* vabs) {
  return gatv2_impl(n_rows, row_ptr, col_idx, xl, xr, 1, att, H, D, slope, n_sel, rows, out, lse, vabs);
}

/* Per-vertex linear projection of the attention layers (paper: section on
 * the three families, l_i = W_l h_i, r_j = W_r h_j for GATv2, q_i = W_Q h_i,
 * k_j = W_K h_j, v_j = W_V h_j for the Graph Transformer): for every vertex i
 * and output feature o,
 *   Y[i, o] = sum_k X[i, k] W[o, k],   Yabs[i, o] = sum_k |X[i, k] W[o, k]|,
 * X [n, f_in] and W [f_out, f_in] bf16 bits (W stored output-major, one row
 * per output feature), Y and Yabs [n, f_out] float64.  Yabs may be NULL. */
int oracle_project(int64_t n, int32_t f_in, const uint16_t* X, int32_t f_out, const uint16_t* W, double* Y,
                   double* Yabs) {
  if (n < 0 || f_in <= 0 || f_out <= 0 || !X || !W || !Y) return -1;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    const uint16_t* xi = X + i * f_in;
    for (int32_t o = 0; o < f_out; ++o) {
      const uint16_t* wo = W + (int64_t)o * f_in;
      double y = 0.0, ya = 0.0;
      for (int32_t k = 0; k < f_in; ++k) {
        const double t = bf16_to_double(xi[k]) * bf16_to_double(wo[k]);
        y += t;
        ya += fabs(t);
      }
      Y[i * f_out + o] = y;
      if (Yabs) Yabs[i * f_out + o] = ya;
    }
  }
  return 0;
}

/* Graph Transformer (paper: section on the three families, q_i = W_Q h_i,
 * k_j = W_K h_j, v_j = W_V h_j, e_ij = q_i^T k_j / sqrt(D); the query belongs
 * to the destination i, keys and values to the sources j, as in the
 * block-sparse attention appendix).  q, k, v [n, H, D] bf16; scale <= 0
 * means 1 / sqrt(D).  Both the CSR and the block-sparse kernels compute this
 * same function. */
int oracle_gt(int32_t n_rows, const int32_t* row_ptr, const int32_t* col_idx, const uint16_t* q,
              const uint16_t* k, const uint16_t* v, int32_t H, int32_t D, float scale,
              int64_t n_sel, const int32_t* rows, double* out, double* lse, double* vabs) {
  if (!row_ptr || !col_idx || !q || !k || !v || !out || !lse || H <= 0 || D <= 0) return -1;
  if (!rows) n_sel = n_rows;
  double sc = scale > 0.0f ? (double)scale : 1.0 / sqrt((double)D);
  int bad = 0;
#pragma omp parallel
  {
    int32_t cap = 0;
    double* logits = NULL;
#pragma omp for schedule(dynamic, 16)
    for (int64_t s = 0; s < n_sel; ++s) {
      int32_t i = rows ? rows[s] : (int32_t)s;
      if (i < 0 || i >= n_rows) {
        bad = 1;
        continue;
      }
      int32_t b = row_ptr[i], deg = row_ptr[i + 1] - b;
      if (deg > cap) {
        free(logits);
        cap = deg;
        logits = (double*)malloc((size_t)cap * 8);
        if (!logits) {
          bad = 1;
          cap = 0;
          continue;
        }
      }
      for (int32_t h = 0; h < H; ++h) {
        const uint16_t* qi = q + ((int64_t)i * H + h) * D;
        for (int32_t t = 0; t < deg; ++t) {
          const uint16_t* kj = k + ((int64_t)col_idx[b + t] * H + h) * D;
          double dot = 0.0;
          for (int32_t d = 0; d < D; ++d) dot += bf16_to_double(qi[d]) * bf16_to_double(kj[d]);
          logits[t] = dot * sc;
        }
        int rc = softmax_aggregate(logits, col_idx + b, deg, v, 0, H, D, h, out + (s * H + h) * D,
                                   lse + s * H + h, vabs ? vabs + (s * H + h) * D : NULL);
        if (rc) bad = 2;
      }
    }
    free(logits);
  }
  return bad == 2 ? -3 : (bad ? -1 : 0);
}

/* ------------------------------------------------------------------------ */
/* Reordering                                                                */
/* ------------------------------------------------------------------------ */

/* Degree sort: perm[new] = old, ordering vertices by descending deg_in,
 * ties by ascending id (a stable sort of the ids by descending row length).
 * Implemented as a stable counting sort over the degree values. */
int oracle_degree_sort(int32_t n, const int32_t* row_ptr, int32_t* perm) {
  if (n < 0 || !row_ptr || !perm) return -1;
  int32_t maxd = 0;
  for (int32_t i = 0; i < n; ++i) {
    int32_t d = row_ptr[i + 1] - row_ptr[i];
    if (d < 0) return -1;
    if (d > maxd) maxd = d;
  }
  int64_t* start = (int64_t*)calloc((size_t)maxd + 2, 8);
  if (!start) return -2;
  for (int32_t i = 0; i < n; ++i) start[maxd - (row_ptr[i + 1] - row_ptr[i]) + 1] += 1;
  for (int32_t d = 0; d <= maxd; ++d) start[d + 1] += start[d];
  for (int32_t i = 0; i < n; ++i) {
    int32_t slot = maxd - (row_ptr[i + 1] - row_ptr[i]);
    perm[start[slot]++] = i;
  }
  free(start);
  return 0;
}

typedef struct {
  int32_t key, id;
} kv32;

static int cmp_kv(const void* a, const void* b) {
  const kv32* x = (const kv32*)a;
  const kv32* y = (const kv32*)b;
  if (x->key != y->key) return x->key < y->key ? -1 : 1;
  return (x->id > y->id) - (x->id < y->id);
}

static int cmp_i32o(const void* a, const void* b) {
  int32_t x = *(const int32_t*)a, y = *(const int32_t*)b;
  return (x > y) - (x < y);
}

/* Symmetrised pattern A u A^T without self loops, as sorted unique lists.
 * On success *adj_ptr (n+1) and *adj (entries) are malloc'd. */
static int symmetrise(int32_t n, const int32_t* row_ptr, const int32_t* col_idx, int64_t** adj_ptr,
                      int32_t** adj) {
  int64_t* cnt = (int64_t*)calloc((size_t)n + 1, 8);
  if (!cnt) return -2;
  for (int32_t i = 0; i < n; ++i)
    for (int32_t e = row_ptr[i]; e < row_ptr[i + 1]; ++e) {
      int32_t j = col_idx[e];
      if (j < 0 || j >= n) {
        free(cnt);
        return -1;
      }
      if (j == i) continue;
      cnt[i + 1]++;
      cnt[j + 1]++;
    }
  for (int32_t i = 0; i < n; ++i) cnt[i + 1] += cnt[i];
  int64_t tot = cnt[n];
  int32_t* lst = (int32_t*)malloc((size_t)(tot > 0 ? tot : 1) * 4);
  int64_t* fill = (int64_t*)malloc(((size_t)n + 1) * 8);
  if (!lst || !fill) {
    free(cnt); free(lst); free(fill);
    return -2;
  }
  memcpy(fill, cnt, ((size_t)n + 1) * 8);
  for (int32_t i = 0; i < n; ++i)
    for (int32_t e = row_ptr[i]; e < row_ptr[i + 1]; ++e) {
      int32_t j = col_idx[e];
      if (j == i) continue;
      lst[fill[i]++] = j;
      lst[fill[j]++] = i;
    }
  /* sort + unique per vertex */
  int64_t w = 0;
  int64_t* ptr = (int64_t*)malloc(((size_t)n + 1) * 8);
  if (!ptr) {
    free(cnt); free(lst); free(fill);
    return -2;
  }
  ptr[0] = 0;
  for (int32_t v = 0; v < n; ++v) {
    int64_t b = cnt[v], en = cnt[v + 1];
    if (en - b > 1) qsort(lst + b, (size_t)(en - b), 4, cmp_i32o);
    for (int64_t t = b; t < en; ++t)
      if (t == b || lst[t] != lst[t - 1]) lst[w++] = lst[t];
    ptr[v + 1] = w;
  }
  free(cnt);
  free(fill);
  *adj_ptr = ptr;
  *adj = lst;
  return 0;
}

/* Reverse Cuthill-McKee on the symmetrised pattern (textbook definition:
 * breadth-first search that visits neighbours in increasing degree, then
 * the order is reversed).  Readings fixed where the pages are silent:
 *   - delta(v) = degree of v in A u A^T without self loops;
 *   - each component starts at its unvisited vertex with the smallest
 *     (delta, id), the next component at the smallest remaining;
 *   - a FIFO queue; a popped vertex appends its unvisited neighbours
 *     sorted by (delta, id), marking them visited;
 *   - perm = reverse(visit order), perm[new] = old. */
int oracle_rcm(int32_t n, const int32_t* row_ptr, const int32_t* col_idx, int32_t* perm) {
  if (n < 0 || !row_ptr || !col_idx || !perm) return -1;
  if (n == 0) return 0;
  int64_t* ap = NULL;
  int32_t* adj = NULL;
  int rc = symmetrise(n, row_ptr, col_idx, &ap, &adj);
  if (rc) return rc;
  kv32* starts = (kv32*)malloc((size_t)n * sizeof(kv32));
  int32_t* order = (int32_t*)malloc((size_t)n * 4);
  char* seen = (char*)calloc((size_t)n, 1);
  kv32* tmp = NULL;
  int64_t tmp_cap = 0;
  if (!starts || !order || !seen) {
    rc = -2;
    goto done;
  }
  for (int32_t v = 0; v < n; ++v) {
    starts[v].key = (int32_t)(ap[v + 1] - ap[v]);
    starts[v].id = v;
  }
  qsort(starts, (size_t)n, sizeof(kv32), cmp_kv);
  int64_t head = 0, tail = 0;
  for (int32_t sidx = 0; sidx < n; ++sidx) {
    int32_t s = starts[sidx].id;
    if (seen[s]) continue;
    seen[s] = 1;
    order[tail++] = s;
    while (head < tail) {
      int32_t u = order[head++];
      int64_t cnt = 0;
      int64_t need = ap[u + 1] - ap[u];
      if (need > tmp_cap) {
        free(tmp);
        tmp_cap = need;
        tmp = (kv32*)malloc((size_t)tmp_cap * sizeof(kv32));
        if (!tmp) {
          rc = -2;
          goto done;
        }
      }
      for (int64_t t = ap[u]; t < ap[u + 1]; ++t) {
        int32_t w = adj[t];
        if (!seen[w]) {
          seen[w] = 1;
          tmp[cnt].key = (int32_t)(ap[w + 1] - ap[w]);
          tmp[cnt].id = w;
          ++cnt;
        }
      }
      if (cnt > 1) qsort(tmp, (size_t)cnt, sizeof(kv32), cmp_kv);
      for (int64_t t = 0; t < cnt; ++t) order[tail++] = tmp[t].id;
    }
  }
  for (int32_t p = 0; p < n; ++p) perm[p] = order[n - 1 - p];
done:
  free(ap);
  free(adj);
  free(starts);
  free(order);
  free(seen);
  free(tmp);
  return rc;
}

/* Apply a vertex permutation (perm[new] = old) to a square CSR: new row p is
 * old row perm[p], every column j becomes inv[j], and each row is re-sorted.
 * row_ptr_out [n+1], col_out [nnz]. */
int oracle_permute_csr(int32_t n, const int32_t* row_ptr, const int32_t* col_idx, const int32_t* perm,
                       int32_t* row_ptr_out, int32_t* col_out) {
  if (n < 0 || !row_ptr || !col_idx || !perm || !row_ptr_out || !col_out) return -1;
  int32_t* inv = (int32_t*)malloc((size_t)(n > 0 ? n : 1) * 4);
  if (!inv) return -2;
  for (int32_t i = 0; i < n; ++i) inv[i] = -1;
  for (int32_t p = 0; p < n; ++p) {
    int32_t o = perm[p];
    if (o < 0 || o >= n || inv[o] != -1) {
      free(inv);
      return -1;
    }
    inv[o] = p;
  }
  row_ptr_out[0] = 0;
  for (int32_t p = 0; p < n; ++p)
    row_ptr_out[p + 1] = row_ptr_out[p] + (row_ptr[perm[p] + 1] - row_ptr[perm[p]]);
#pragma omp parallel for schedule(dynamic, 256)
  for (int32_t p = 0; p < n; ++p) {
    int32_t o = perm[p];
    int32_t w = row_ptr_out[p];
    for (int32_t e = row_ptr[o]; e < row_ptr[o + 1]; ++e) col_out[w++] = inv[col_idx[e]];
    int32_t len = row_ptr_out[p + 1] - row_ptr_out[p];
    if (len > 1) qsort(col_out + row_ptr_out[p], (size_t)len, 4, cmp_i32o);
  }
  free(inv);
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Weighted block-sparse (WSB) layout                                        */
/* ------------------------------------------------------------------------ */

/* WSB build (paper: block-sparse appendix, "WSB format and TCB
 * construction"): destination rows are cut into windows of R = 16 rows; for
 * each window the distinct source columns of its edges are sorted and cut
 * into blocks of W = 8 columns (the last one padded with column 0); each
 * block carries a 16 x 8 occupancy bitmap as two 64-bit words, bit
 * r * 8 + c set when row 16w + r has an edge from the block's column c
 * (word = bit / 64).  Two-phase: call with tcb_col == NULL to get the block
 * count in *n_tcb and the window offsets; then again with the arrays. */
int oracle_wsb_build(int32_t n_rows, const int32_t* row_ptr, const int32_t* col_idx,
                     int32_t* win_ptr /* [n_windows + 1] */, int32_t* tcb_col /* [n_tcb * 8] */,
                     uint64_t* tcb_bits /* [n_tcb * 2] */, int64_t* n_tcb) {
  if (n_rows < 0 || !row_ptr || !col_idx || !win_ptr || !n_tcb) return -1;
  int32_t nw = (n_rows + 15) / 16;
  int rc = 0;
  win_ptr[0] = 0;
  int32_t* cols = NULL;
  int64_t cap = 0;
  for (int32_t w = 0; w < nw; ++w) {
    int32_t r0 = w * 16, r1 = r0 + 16 < n_rows ? r0 + 16 : n_rows;
    int64_t len = row_ptr[r1] - row_ptr[r0];
    if (len > cap) {
      free(cols);
      cap = len;
      cols = (int32_t*)malloc((size_t)cap * 4);
      if (!cols) return -2;
    }
    memcpy(cols, col_idx + row_ptr[r0], (size_t)len * 4);
    if (len > 1) qsort(cols, (size_t)len, 4, cmp_i32o);
    int64_t u = 0;
    for (int64_t t = 0; t < len; ++t)
      if (t == 0 || cols[t] != cols[t - 1]) cols[u++] = cols[t];
    int64_t nb = (u + 7) / 8;
    int64_t base = win_ptr[w];
    if (tcb_col) {
      for (int64_t b = 0; b < nb; ++b) {
        for (int c = 0; c < 8; ++c) {
          int64_t t = b * 8 + c;
          tcb_col[(base + b) * 8 + c] = t < u ? cols[t] : 0;
        }
        tcb_bits[(base + b) * 2] = 0;
        tcb_bits[(base + b) * 2 + 1] = 0;
      }
      for (int32_t r = r0; r < r1; ++r)
        for (int32_t e = row_ptr[r]; e < row_ptr[r + 1]; ++e) {
          /* position of the column among the window's sorted distinct columns */
          int64_t lo = 0, hi = u - 1, pos = -1;
          while (lo <= hi) {
            int64_t mid = (lo + hi) / 2;
            if (cols[mid] == col_idx[e]) { pos = mid; break; }
            if (cols[mid] < col_idx[e]) lo = mid + 1; else hi = mid - 1;
          }
          if (pos < 0) { rc = -3; continue; }
          int64_t b = pos / 8;
          int bit = (r - r0) * 8 + (int)(pos % 8);
          tcb_bits[(base + b) * 2 + bit / 64] |= (uint64_t)1 << (bit % 64);
        }
    }
    if (base + nb > 2147483647LL) { rc = -1; break; }
    win_ptr[w + 1] = (int32_t)(base + nb);
  }
  free(cols);
  *n_tcb = win_ptr[nw];
  return rc;
}

/* ------------------------------------------------------------------------ */
/* Backward passes                                                           */
/* ------------------------------------------------------------------------ */

/* SpMM backward: dX = A_norm^T dY, i.e. for every entry e = (i <- j) of row
 * i, dX[j, :] += w_e * dY[i, :] with the forward's weight w_e (paper: the
 * SpMM and reduction appendix, backward of Y = A X).  dY [n_rows, F] fp32,
 * dX and dXabs (sum of |w_e dY|) [n_cols, F] fp64.  A plain serial scatter. */
static int spmm_backward_impl(int32_t n_rows, int32_t n_cols, const int32_t* row_ptr, const int32_t* col_idx,
                              const float* edge_val, int norm, const float* dY, int32_t F,
                              const int32_t* slot, int64_t n_out, double* dX, double* dXabs) {
  int32_t* dout = (int32_t*)malloc((size_t)(n_cols > 0 ? n_cols : 1) * 4);
  if (!dout) return -2;
  if (oracle_degrees(n_rows, n_cols, row_ptr, col_idx, NULL, dout)) {
    free(dout);
    return -1;
  }
  memset(dX, 0, (size_t)n_out * F * 8);
  if (dXabs) memset(dXabs, 0, (size_t)n_out * F * 8);
  for (int32_t i = 0; i < n_rows; ++i) {
    int32_t din = row_ptr[i + 1] - row_ptr[i];
    for (int32_t e = row_ptr[i]; e < row_ptr[i + 1]; ++e) {
      int32_t j = col_idx[e];
      if (j < 0 || j >= n_cols) {
        free(dout);
        return -1;
      }
      int64_t o = slot ? slot[j] : j;  /* output row of column j, or -1: not selected */
      if (o < 0) continue;
      double w = edge_weight(norm, din, dout[j], edge_val, e);
      for (int32_t f = 0; f < F; ++f) {
        double t = w * (double)dY[(int64_t)i * F + f];
        dX[o * F + f] += t;
        if (dXabs) dXabs[o * F + f] += fabs(t);
      }
    }
  }
  free(dout);
  return 0;
}

int oracle_spmm_backward(int32_t n_rows, int32_t n_cols, const int32_t* row_ptr, const int32_t* col_idx,
                         const float* edge_val, int norm, const float* dY, int32_t F, double* dX,
                         double* dXabs) {
  if (!row_ptr || !col_idx || !dY || !dX || F <= 0 || norm < 0 || norm > 3) return -1;
  return spmm_backward_impl(n_rows, n_cols, row_ptr, col_idx, edge_val, norm, dY, F, NULL, n_cols, dX, dXabs);
}

/* The same for the selected columns cols[0 .. n_sel) only (distinct, each in
 * [0, n_cols)); output rows packed in that order.  Every entry of A is still
 * visited, so the cost is one pass over the CSR plus the selected terms. */
int oracle_spmm_backward_cols(int32_t n_rows, int32_t n_cols, const int32_t* row_ptr, const int32_t* col_idx,
                              const float* edge_val, int norm, const float* dY, int32_t F, int64_t n_sel,
                              const int32_t* cols, double* dX, double* dXabs) {
  if (!row_ptr || !col_idx || !dY || !dX || !cols || F <= 0 || norm < 0 || norm > 3 || n_sel < 0) return -1;
  int32_t* slot = (int32_t*)malloc((size_t)(n_cols > 0 ? n_cols : 1) * 4);
  if (!slot) return -2;
  for (int32_t j = 0; j < n_cols; ++j) slot[j] = -1;
  for (int64_t s = 0; s < n_sel; ++s) {
    if (cols[s] < 0 || cols[s] >= n_cols || slot[cols[s]] != -1) {
      free(slot);
      return -1;
    }
    slot[cols[s]] = (int32_t)s;
  }
  int rc = spmm_backward_impl(n_rows, n_cols, row_ptr, col_idx, edge_val, norm, dY, F, slot, n_sel, dX, dXabs);
  free(slot);
  return rc;
}

/* Reduction backward (paper: reduction appendix, backward pass).  op 0 SUM:
 * dX[j] += dY[i] for each entry (i <- j); 1 MEAN: dX[j] += dY[i] / deg_in(i);
 * 2 MAX, 3 MIN: the gradient flows only to the selected source,
 * dX[arg[i, f], f] += dY[i, f] (rows without entries have arg -1 and pass
 * nothing).  dY, arg [n_rows, F]; dX, dXabs [n_cols, F] fp64. */
int oracle_reduce_backward(int32_t n_rows, int32_t n_cols, const int32_t* row_ptr, const int32_t* col_idx,
                           int op, const float* dY, const int32_t* arg, int32_t F, double* dX,
                           double* dXabs) {
  if (!row_ptr || !col_idx || !dY || !dX || F <= 0 || op < 0 || op > 3) return -1;
  if (op <= 1) return oracle_spmm_backward(n_rows, n_cols, row_ptr, col_idx, NULL, op, dY, F, dX, dXabs);
  if (!arg) return -1;
  memset(dX, 0, (size_t)n_cols * F * 8);
  if (dXabs) memset(dXabs, 0, (size_t)n_cols * F * 8);
  for (int32_t i = 0; i < n_rows; ++i) {
    for (int32_t f = 0; f < F; ++f) {
      int32_t j = arg[(int64_t)i * F + f];
      if (j < 0) continue;
      if (j >= n_cols) return -1;
      double t = (double)dY[(int64_t)i * F + f];
      dX[(int64_t)j * F + f] += t;
      if (dXabs) dXabs[(int64_t)j * F + f] += fabs(t);
    }
  }
  return 0;
}

/* Softmax weights of one (i, h) row from its logits (two passes). */
static void softmax_weights(const double* logits, int32_t deg, double* alpha) {
  double m = -INFINITY;
  for (int32_t k = 0; k < deg; ++k)
    if (logits[k] > m) m = logits[k];
  double s = 0.0;
  for (int32_t k = 0; k < deg; ++k) s += exp(logits[k] - m);
  for (int32_t k = 0; k < deg; ++k) alpha[k] = exp(logits[k] - m) / s;
}

/* Graph Transformer backward (paper: attention appendix, backward pass with
 * the cached logsumexp and Delta[i, h] = <O[i, h, :], dO[i, h, :]>), written
 * from the definition of the forward: out_i = sum_j alpha_ij v_j,
 * alpha_ij = softmax_j(e_ij), e_ij = scale <q_i, k_j>.  With
 * g_ij = <dO_i, v_j> and Delta_i = sum_j alpha_ij g_ij (= <dO_i, out_i>),
 * de_ij = alpha_ij (g_ij - Delta_i), and
 *   dq_i += scale de_ij k_j,  dk_j += scale de_ij q_i,  dv_j += alpha_ij dO_i.
 * q [n_rows, H, D], k, v [n_cols, H, D] bf16; dO [n_rows, H, D] fp32; outputs
 * fp64.  The magnitudes (error scales) sum the absolute values of every
 * product that enters an element, those inside de_ij included:
 * |de|~ = alpha_ij (sum_d |dO_id v_jd| + sum_j' alpha_ij' sum_d |dO_id v_j'd|),
 * dq_abs_i = scale sum_j |de|~ |k_j|, dk_abs_j = scale sum_i |de|~ |q_i|,
 * dv_abs_j = sum_i alpha_ij |dO_i|. */
int oracle_gt_backward(int32_t n_rows, int32_t n_cols, const int32_t* row_ptr, const int32_t* col_idx,
                       const uint16_t* q, const uint16_t* k, const uint16_t* v, int32_t H, int32_t D,
                       float scale, const float* dO, double* dq, double* dk, double* dv, double* dq_abs,
                       double* dk_abs, double* dv_abs) {
  if (!row_ptr || !col_idx || !q || !k || !v || !dO || !dq || !dk || !dv || H <= 0 || D <= 0) return -1;
  const double sc = scale > 0.0f ? (double)scale : 1.0 / sqrt((double)D);
  const int64_t HD = (int64_t)H * D;
  memset(dq, 0, (size_t)n_rows * HD * 8);
  memset(dk, 0, (size_t)n_cols * HD * 8);
  memset(dv, 0, (size_t)n_cols * HD * 8);
  if (dq_abs) memset(dq_abs, 0, (size_t)n_rows * HD * 8);
  if (dk_abs) memset(dk_abs, 0, (size_t)n_cols * HD * 8);
  if (dv_abs) memset(dv_abs, 0, (size_t)n_cols * HD * 8);
  int32_t cap = 0;
  double *e = NULL, *a = NULL, *g = NULL, *ga = NULL;
  int rc = 0;
  for (int32_t i = 0; i < n_rows && rc == 0; ++i) {
    int32_t b = row_ptr[i], deg = row_ptr[i + 1] - b;
    if (deg > cap) {
      free(e); free(a); free(g); free(ga);
      cap = deg;
      e = (double*)malloc((size_t)cap * 8);
      a = (double*)malloc((size_t)cap * 8);
      g = (double*)malloc((size_t)cap * 8);
      ga = (double*)malloc((size_t)cap * 8);
      if (!e || !a || !g || !ga) { rc = -2; break; }
    }
    for (int32_t h = 0; h < H; ++h) {
      const uint16_t* qi = q + (int64_t)i * HD + (int64_t)h * D;
      const float* doi = dO + (int64_t)i * HD + (int64_t)h * D;
      for (int32_t t = 0; t < deg; ++t) {
        int32_t j = col_idx[b + t];
        if (j < 0 || j >= n_cols) { rc = -1; break; }
        const uint16_t* kj = k + (int64_t)j * HD + (int64_t)h * D;
        const uint16_t* vj = v + (int64_t)j * HD + (int64_t)h * D;
        double dot = 0.0, gv = 0.0, gav = 0.0;
        for (int32_t d = 0; d < D; ++d) {
          dot += bf16_to_double(qi[d]) * bf16_to_double(kj[d]);
          gv += (double)doi[d] * bf16_to_double(vj[d]);
          gav += fabs((double)doi[d] * bf16_to_double(vj[d]));
        }
        e[t] = dot * sc;
        g[t] = gv;
        ga[t] = gav;
      }
      if (rc) break;
      if (deg == 0) continue;
      softmax_weights(e, deg, a);
      double delta = 0.0, delta_abs = 0.0;
      for (int32_t t = 0; t < deg; ++t) {
        delta += a[t] * g[t];
        delta_abs += a[t] * ga[t];
      }
      for (int32_t t = 0; t < deg; ++t) {
        int32_t j = col_idx[b + t];
        const uint16_t* kj = k + (int64_t)j * HD + (int64_t)h * D;
        const double de = a[t] * (g[t] - delta);
        const double de_abs = a[t] * (ga[t] + delta_abs);
        for (int32_t d = 0; d < D; ++d) {
          const int64_t oi = (int64_t)i * HD + (int64_t)h * D + d, oj = (int64_t)j * HD + (int64_t)h * D + d;
          const double kd = bf16_to_double(kj[d]), qd = bf16_to_double(qi[d]);
          const double tv = a[t] * (double)doi[d];
          dq[oi] += sc * de * kd;
          dk[oj] += sc * de * qd;
          dv[oj] += tv;
          if (dq_abs) dq_abs[oi] += sc * de_abs * fabs(kd);
          if (dk_abs) dk_abs[oj] += sc * de_abs * fabs(qd);
          if (dv_abs) dv_abs[oj] += fabs(tv);
        }
      }
    }
  }
  free(e); free(a); free(g); free(ga);
  return rc;
}

/* GATv2 backward (paper: attention appendix, the two-kernel backward with
 * G_{i,h} = sum_j alpha_ij <dh_i, r_j> and the attention-vector gradient
 * reduced over nodes), written from the forward: e_ij = sum_d a_d s(z_ijd),
 * z_ij = l_i + r_j, s = LeakyReLU (s(z) = z if z > 0 else slope z, so its
 * derivative is 1 for z > 0 and slope otherwise, the branch the forward
 * takes at z = 0), out_i = sum_j alpha_ij r_j.  With g_ij = <dO_i, r_j>,
 * G_i = sum_j alpha_ij g_ij and de_ij = alpha_ij (g_ij - G_i):
 *   dl_i  += de_ij a (.) s'(z_ij)
 *   dr_j  += alpha_ij dO_i + de_ij a (.) s'(z_ij)
 *   da    += de_ij s(z_ij)            (summed over all entries)
 * xl [n_rows, H, D], xr [n_cols, H, D] bf16; att [H, D] fp32; dO fp32;
 * outputs fp64.  Magnitudes as for the Graph Transformer: with
 * |de|~ = alpha_ij (sum_d |dO_id r_jd| + sum_j' alpha_ij' sum_d |dO_id r_j'd|),
 * dl_abs += |de|~ |a (.) s'|, dr_abs += alpha |dO_i| + |de|~ |a (.) s'|,
 * da_abs += |de|~ |s(z)|. */
int oracle_gatv2_backward(int32_t n_rows, int32_t n_cols, const int32_t* row_ptr, const int32_t* col_idx,
                          const uint16_t* xl, const uint16_t* xr, const float* att, int32_t H, int32_t D,
                          float slope, const float* dO, double* dl, double* dr, double* da, double* dl_abs,
                          double* dr_abs, double* da_abs) {
  if (!row_ptr || !col_idx || !xl || !xr || !att || !dO || !dl || !dr || !da || H <= 0 || D <= 0) return -1;
  const int64_t HD = (int64_t)H * D;
  const double sl = (double)slope;
  memset(dl, 0, (size_t)n_rows * HD * 8);
  memset(dr, 0, (size_t)n_cols * HD * 8);
  memset(da, 0, (size_t)HD * 8);
  if (dl_abs) memset(dl_abs, 0, (size_t)n_rows * HD * 8);
  if (dr_abs) memset(dr_abs, 0, (size_t)n_cols * HD * 8);
  if (da_abs) memset(da_abs, 0, (size_t)HD * 8);
  int32_t cap = 0;
  double *e = NULL, *a = NULL, *g = NULL, *ga = NULL;
  int rc = 0;
  for (int32_t i = 0; i < n_rows && rc == 0; ++i) {
    int32_t b = row_ptr[i], deg = row_ptr[i + 1] - b;
    if (deg > cap) {
      free(e); free(a); free(g); free(ga);
      cap = deg;
      e = (double*)malloc((size_t)cap * 8);
      a = (double*)malloc((size_t)cap * 8);
      g = (double*)malloc((size_t)cap * 8);
      ga = (double*)malloc((size_t)cap * 8);
      if (!e || !a || !g || !ga) { rc = -2; break; }
    }
    for (int32_t h = 0; h < H; ++h) {
      const uint16_t* li = xl + (int64_t)i * HD + (int64_t)h * D;
      const float* doi = dO + (int64_t)i * HD + (int64_t)h * D;
      const float* ah = att + (int64_t)h * D;
      for (int32_t t = 0; t < deg; ++t) {
        int32_t j = col_idx[b + t];
        if (j < 0 || j >= n_cols) { rc = -1; break; }
        const uint16_t* rj = xr + (int64_t)j * HD + (int64_t)h * D;
        double ev = 0.0, gv = 0.0, gav = 0.0;
        for (int32_t d = 0; d < D; ++d) {
          double z = bf16_to_double(li[d]) + bf16_to_double(rj[d]);
          ev += (double)ah[d] * (z > 0.0 ? z : sl * z);
          gv += (double)doi[d] * bf16_to_double(rj[d]);
          gav += fabs((double)doi[d] * bf16_to_double(rj[d]));
        }
        e[t] = ev;
        g[t] = gv;
        ga[t] = gav;
      }
      if (rc) break;
      if (deg == 0) continue;
      softmax_weights(e, deg, a);
      double G = 0.0, G_abs = 0.0;
      for (int32_t t = 0; t < deg; ++t) {
        G += a[t] * g[t];
        G_abs += a[t] * ga[t];
      }
      for (int32_t t = 0; t < deg; ++t) {
        int32_t j = col_idx[b + t];
        const uint16_t* rj = xr + (int64_t)j * HD + (int64_t)h * D;
        const double de = a[t] * (g[t] - G);
        const double de_abs = a[t] * (ga[t] + G_abs);
        for (int32_t d = 0; d < D; ++d) {
          const int64_t oi = (int64_t)i * HD + (int64_t)h * D + d, oj = (int64_t)j * HD + (int64_t)h * D + d;
          const double z = bf16_to_double(li[d]) + bf16_to_double(rj[d]);
          const double ds = z > 0.0 ? 1.0 : sl;
          const double act = z > 0.0 ? z : sl * z;
          const double tl = de * (double)ah[d] * ds;
          const double tv = a[t] * (double)doi[d];
          dl[oi] += tl;
          dr[oj] += tv + tl;
          da[(int64_t)h * D + d] += de * act;
          if (dl_abs) dl_abs[oi] += de_abs * fabs((double)ah[d] * ds);
          if (dr_abs) dr_abs[oj] += fabs(tv) + de_abs * fabs((double)ah[d] * ds);
          if (da_abs) da_abs[(int64_t)h * D + d] += de_abs * fabs(act);
        }
      }
    }
  }
  free(e); free(a); free(g); free(ga);
  return rc;
}

/* ------------------------------------------------------------------------ */
/* dot-aggr reordering micro-benchmark                                       */
/* ------------------------------------------------------------------------ */

/* dot-aggr (paper: Experiments, the graph-reordering results with Figure 1,
 * and appendix E.1 with Figure 2).  The pages name the kernel (a dot product
 * followed by an aggregation) and fix that its feature-parallel and its
 * neighbour-parallel mapping do the same arithmetic; with one lane per
 * neighbour that arithmetic is a full dot product per edge.  So for every
 * destination i:  y_i = sum over the sources j of row i of
 * sum_d X[i, d] * X[j, d], a scalar per node; yabs_i = the same sum of
 * |X[i, d] * X[j, d]| (error scale).  The graph is square: sources index
 * rows of the same X. */
int oracle_dot_aggr(int32_t n_rows, const int32_t* row_ptr, const int32_t* col_idx, const float* X,
                    int32_t D, int64_t ldx, int64_t n_sel, const int32_t* rows, double* y,
                    double* yabs) {
  if (n_rows < 0 || !row_ptr || !y || D <= 0 || ldx < D) return -1;
  if (n_rows > 0 && !X) return -1;
  if (!rows) n_sel = n_rows;
  int bad = 0;
#pragma omp parallel for schedule(dynamic, 64)
  for (int64_t s = 0; s < n_sel; ++s) {
    int32_t i = rows ? rows[s] : (int32_t)s;
    y[s] = 0.0;
    if (yabs) yabs[s] = 0.0;
    if (i < 0 || i >= n_rows) {
      bad = 1;
      continue;
    }
    double acc = 0.0, mag = 0.0;
    for (int32_t e = row_ptr[i]; e < row_ptr[i + 1]; ++e) {
      int32_t j = col_idx[e];
      if (j < 0 || j >= n_rows) {
        bad = 1;
        break;
      }
      for (int32_t d = 0; d < D; ++d) {
        double t = (double)X[(int64_t)i * ldx + d] * (double)X[(int64_t)j * ldx + d];
        acc += t;
        mag += fabs(t);
      }
    }
    y[s] = acc;
    if (yabs) yabs[s] = mag;
  }
  return bad ? -1 : 0;
}
