/*
 * Seeded synthetic inputs for the aggregation kernels and their oracle.
 *
 * This module only draws random numbers and lays graphs out as CSR; it holds
 * none of the arithmetic the kernels or the oracle compute (no degrees used
 * as weights, no normalisation, no reductions, no attention).  Both the HIP
 * path and the CPU oracle read what it produces.
 *
 * Randomness: SplitMix64 (Steele, Lea and Flood, "Fast splittable
 * pseudorandom number generators", OOPSLA 2014) used as a counter-based
 * generator: draw(seed, i) is the i-th output of a SplitMix64 stream whose
 * state starts at `seed`, i.e. mix(seed + (i + 1) * 0x9E3779B97F4A7C15).
 * Every draw is addressed by its counter, so the output does not depend on
 * the number of threads.  Gaussians use the Box-Muller transform; bf16 is
 * the IEEE float rounded to nearest-even on its upper 16 bits.
 *
 * Graphs (CSR, rows = destinations, columns sorted ascending, no duplicate
 * entries):
 *   - R-MAT (Chakrabarti, Zhan, Faloutsos, SDM 2004) with quadrant
 *     probabilities a, b, c, d = 1 - a - b - c, drawn at scale
 *     ceil(log2 n); attempts with an endpoint >= n or a self loop are
 *     rejected, duplicates are merged, and the edge set is trimmed or topped
 *     up to exactly m distinct edges; vertices are then relabelled by a
 *     seeded uniform permutation (the Graph500 practice).
 *   - Erdos-Renyi G(n, m) over unordered pairs, stored symmetrically.
 *   - A cluster graph: contiguous clusters of `csize` nodes, each ordered
 *     intra-cluster pair present with probability p, plus
 *     round(frac * E_intra) distinct random inter-cluster ordered pairs.
 *   Optionally one self loop per node is added after loops are removed.
 *
 * Trimming rule (exactly m distinct edges): attempts are drawn in batches
 * until at least m distinct edges exist; if more exist, the m edges with the
 * smallest hash value h(key) = draw(seed ^ TRIM_SALT, key) are kept.  This
 * is deterministic and independent of the thread count.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <math.h>
#include <omp.h>

#define GOLDEN 0x9E3779B97F4A7C15ULL
#define TRIM_SALT 0xD1B54A32D192ED03ULL

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

uint64_t gen_draw(uint64_t seed, uint64_t counter) {
  return mix64(seed + (counter + 1) * GOLDEN);
}

/* uniform in [0, 1) with 53 random bits */
static inline double u01(uint64_t seed, uint64_t counter) {
  return (double)(gen_draw(seed, counter) >> 11) * (1.0 / 9007199254740992.0);
}

/* uniform integer in [0, n) (multiply-shift; bias < n / 2^64) */
static inline uint64_t uint_below(uint64_t seed, uint64_t counter, uint64_t n) {
  unsigned __int128 p = (unsigned __int128)gen_draw(seed, counter) * n;
  return (uint64_t)(p >> 64);
}

void gen_uniform_u64(uint64_t seed, int64_t n, uint64_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = gen_draw(seed, (uint64_t)i);
}

/* out[i] = stddev * z_i, z_i ~ N(0,1) by Box-Muller on the counter pair
 * (2*(i/2), 2*(i/2)+1); even i take the cosine branch, odd i the sine. */
static inline float gauss_at(uint64_t seed, int64_t i, double stddev) {
  uint64_t k = (uint64_t)(i >> 1);
  double u1 = 1.0 - u01(seed, 2 * k);      /* (0, 1] */
  double u2 = u01(seed, 2 * k + 1);
  double r = sqrt(-2.0 * log(u1));
  double t = 6.283185307179586476925286766559 * u2;
  double z = (i & 1) ? r * sin(t) : r * cos(t);
  return (float)(stddev * z);
}

void gen_gauss_f32(uint64_t seed, int64_t n, double stddev, float* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = gauss_at(seed, i, stddev);
}

static inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7F800000u) == 0x7F800000u) /* inf / nan: truncate, keep nan quiet */
    return (uint16_t)((u >> 16) | ((u & 0xFFFFu) ? 0x40u : 0u));
  uint32_t lsb = (u >> 16) & 1u;
  u += 0x7FFFu + lsb;
  return (uint16_t)(u >> 16);
}

void gen_f32_to_bf16(int64_t n, const float* in, uint16_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = f32_to_bf16_rne(in[i]);
}

void gen_gauss_bf16(uint64_t seed, int64_t n, double stddev, uint16_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = f32_to_bf16_rne(gauss_at(seed, i, stddev));
}

/* ------------------------------------------------------------------------ */
/* Edge buffers and CSR assembly                                             */
/* ------------------------------------------------------------------------ */

typedef struct {
  int32_t* src;
  int32_t* dst;
  int64_t n, cap;
} edge_buf;

static int eb_reserve(edge_buf* b, int64_t cap) {
  if (cap <= b->cap) return 0;
  int32_t* s = (int32_t*)realloc(b->src, (size_t)cap * 4);
  if (!s) return -1;
  b->src = s;
  int32_t* d = (int32_t*)realloc(b->dst, (size_t)cap * 4);
  if (!d) return -1;
  b->dst = d;
  b->cap = cap;
  return 0;
}

static void eb_free(edge_buf* b) {
  free(b->src);
  free(b->dst);
  memset(b, 0, sizeof(*b));
}

static int cmp_i32(const void* a, const void* b) {
  int32_t x = *(const int32_t*)a, y = *(const int32_t*)b;
  return (x > y) - (x < y);
}

/* Bucket the edges by destination, sort and de-duplicate each row.
 * Produces row_ptr[n+1] (int64 during assembly) and col[] (malloc'd). */
typedef struct {
  int32_t n;
  int64_t m;
  int64_t* row_ptr;
  int32_t* col;
} csr64;

static void csr64_free(csr64* c) {
  free(c->row_ptr);
  free(c->col);
  memset(c, 0, sizeof(*c));
}

static int assemble_csr(int32_t n, const edge_buf* e, csr64* out) {
  int64_t* cnt = (int64_t*)calloc((size_t)n + 1, 8);
  if (!cnt) return -1;
  int64_t ne = e->n;
#pragma omp parallel for schedule(static)
  for (int64_t k = 0; k < ne; ++k) __atomic_fetch_add(&cnt[e->dst[k] + 1], 1, __ATOMIC_RELAXED);
  for (int32_t i = 0; i < n; ++i) cnt[i + 1] += cnt[i];
  int32_t* col = (int32_t*)malloc((size_t)(ne > 0 ? ne : 1) * 4);
  int64_t* fill = (int64_t*)malloc((size_t)n * 8 + 8);
  if (!col || !fill) {
    free(cnt); free(col); free(fill);
    return -1;
  }
  memcpy(fill, cnt, (size_t)n * 8);
#pragma omp parallel for schedule(static)
  for (int64_t k = 0; k < ne; ++k) {
    int64_t p = __atomic_fetch_add(&fill[e->dst[k]], 1, __ATOMIC_RELAXED);
    col[p] = e->src[k];
  }
  /* sort and unique every row; record the unique count */
  int64_t* ucnt = fill; /* reuse */
#pragma omp parallel for schedule(dynamic, 1024)
  for (int32_t i = 0; i < n; ++i) {
    int64_t b = cnt[i], en = cnt[i + 1];
    int64_t len = en - b;
    if (len > 1) qsort(col + b, (size_t)len, 4, cmp_i32);
    int64_t u = 0;
    for (int64_t k = b; k < en; ++k)
      if (u == 0 || col[b + u - 1] != col[k]) col[b + (u++)] = col[k];
    ucnt[i] = u;
  }
  /* compact */
  int64_t* rp = (int64_t*)malloc(((size_t)n + 1) * 8);
  if (!rp) {
    free(cnt); free(col); free(fill);
    return -1;
  }
  rp[0] = 0;
  for (int32_t i = 0; i < n; ++i) rp[i + 1] = rp[i] + ucnt[i];
  int64_t m = rp[n];
  int32_t* col2 = (int32_t*)malloc((size_t)(m > 0 ? m : 1) * 4);
  if (!col2) {
    free(cnt); free(col); free(fill); free(rp);
    return -1;
  }
#pragma omp parallel for schedule(dynamic, 1024)
  for (int32_t i = 0; i < n; ++i) memcpy(col2 + rp[i], col + cnt[i], (size_t)ucnt[i] * 4);
  free(cnt);
  free(col);
  free(fill);
  out->n = n;
  out->m = m;
  out->row_ptr = rp;
  out->col = col2;
  return 0;
}

/* Keep exactly m edges of c (c->m >= m): those with the smallest trim hash. */
static int cmp_u64(const void* a, const void* b) {
  uint64_t x = *(const uint64_t*)a, y = *(const uint64_t*)b;
  return (x > y) - (x < y);
}

static inline uint64_t edge_key(int32_t dst, int32_t src) {
  return ((uint64_t)(uint32_t)dst << 32) | (uint32_t)src;
}

static int trim_csr(csr64* c, int64_t m, uint64_t seed) {
  if (c->m <= m) return 0;
  int32_t n = c->n;
  int64_t total = c->m;
  uint64_t* h = (uint64_t*)malloc((size_t)total * 8);
  if (!h) return -1;
#pragma omp parallel for schedule(dynamic, 1024)
  for (int32_t i = 0; i < n; ++i)
    for (int64_t k = c->row_ptr[i]; k < c->row_ptr[i + 1]; ++k)
      h[k] = gen_draw(seed ^ TRIM_SALT, edge_key(i, c->col[k]));
  /* threshold = m-th smallest hash, by a 16-bit radix histogram followed by
   * sorting the one bucket that holds it (hash values are distinct with
   * overwhelming probability; equal ones are kept in key order below) */
  int64_t* hist = (int64_t*)calloc(65536, 8);
  if (!hist) {
    free(h);
    return -1;
  }
#pragma omp parallel for schedule(static)
  for (int64_t k = 0; k < total; ++k) __atomic_fetch_add(&hist[h[k] >> 48], 1, __ATOMIC_RELAXED);
  int64_t acc = 0;
  int64_t bucket = 0;
  for (bucket = 0; bucket < 65536; ++bucket) {
    if (acc + hist[bucket] >= m) break;
    acc += hist[bucket];
  }
  int64_t nb = hist[bucket];
  free(hist);
  uint64_t* s = (uint64_t*)malloc((size_t)(nb > 0 ? nb : 1) * 8);
  if (!s) {
    free(h);
    return -1;
  }
  int64_t q = 0;
  for (int64_t k = 0; k < total; ++k)
    if ((int64_t)(h[k] >> 48) == bucket) s[q++] = h[k];
  qsort(s, (size_t)q, 8, cmp_u64);
  uint64_t thr = s[m - acc - 1];
  int64_t below = acc;
  for (int64_t k = 0; k < q; ++k) below += (s[k] < thr);
  int64_t take_eq = m - below; /* how many edges with hash == thr to keep (in key order) */
  free(s);
  int64_t* rp = (int64_t*)malloc(((size_t)n + 1) * 8);
  int32_t* col = (int32_t*)malloc((size_t)m * 4);
  if (!rp || !col) {
    free(h); free(rp); free(col);
    return -1;
  }
  int64_t w = 0;
  rp[0] = 0;
  for (int32_t i = 0; i < n; ++i) {
    for (int64_t k = c->row_ptr[i]; k < c->row_ptr[i + 1]; ++k) {
      if (h[k] < thr || (h[k] == thr && take_eq > 0)) {
        if (h[k] == thr) --take_eq;
        col[w++] = c->col[k];
      }
    }
    rp[i + 1] = w;
  }
  free(h);
  free(c->row_ptr);
  free(c->col);
  c->row_ptr = rp;
  c->col = col;
  c->m = w;
  return 0;
}

/* merge csr a with extra edges (keeps a's edges, adds new distinct ones) */
static int csr_to_edges(const csr64* c, edge_buf* e) {
  if (eb_reserve(e, e->n + c->m + 1)) return -1;
  for (int32_t i = 0; i < c->n; ++i)
    for (int64_t k = c->row_ptr[i]; k < c->row_ptr[i + 1]; ++k) {
      e->src[e->n] = c->col[k];
      e->dst[e->n] = i;
      e->n++;
    }
  return 0;
}

/* Public result: int32 CSR (the kernels' format). */
typedef struct {
  int32_t n;
  int64_t m;
  int32_t* row_ptr;
  int32_t* col_idx;
} gen_graph;

void gen_graph_free(gen_graph* g) {
  if (!g) return;
  free(g->row_ptr);
  free(g->col_idx);
  memset(g, 0, sizeof(*g));
}

static int finish(csr64* c, int add_loops, gen_graph* out) {
  int32_t n = c->n;
  int64_t m = c->m + (add_loops ? n : 0);
  if (m >= 2147483647LL) return -2;
  int32_t* rp = (int32_t*)malloc(((size_t)n + 1) * 4);
  int32_t* col = (int32_t*)malloc((size_t)(m > 0 ? m : 1) * 4);
  if (!rp || !col) {
    free(rp); free(col);
    return -1;
  }
  rp[0] = 0;
  for (int32_t i = 0; i < n; ++i)
    rp[i + 1] = rp[i] + (int32_t)(c->row_ptr[i + 1] - c->row_ptr[i]) + (add_loops ? 1 : 0);
#pragma omp parallel for schedule(dynamic, 1024)
  for (int32_t i = 0; i < n; ++i) {
    int64_t w = rp[i];
    int placed = !add_loops;
    for (int64_t k = c->row_ptr[i]; k < c->row_ptr[i + 1]; ++k) {
      int32_t j = c->col[k];
      if (!placed && j > i) { col[w++] = i; placed = 1; }
      col[w++] = j;
    }
    if (!placed) col[w++] = i;
  }
  out->n = n;
  out->m = m;
  out->row_ptr = rp;
  out->col_idx = col;
  return 0;
}

static int32_t ceil_log2(int64_t n) {
  int32_t s = 0;
  while (((int64_t)1 << s) < n) ++s;
  return s;
}

/* seeded uniform permutation (Fisher-Yates, draw i picks among [0, i]) */
int gen_permutation(uint64_t seed, int32_t n, int32_t* perm) {
  for (int32_t i = 0; i < n; ++i) perm[i] = i;
  for (int32_t i = n - 1; i > 0; --i) {
    int32_t j = (int32_t)uint_below(seed, (uint64_t)i, (uint64_t)i + 1);
    int32_t t = perm[i];
    perm[i] = perm[j];
    perm[j] = t;
  }
  return 0;
}

/* R-MAT.  Attempt t draws its quadrant choices from counters t*16 + l/3:
 * each 64-bit word gives three 21-bit uniforms, one per recursion level. */
int gen_rmat(uint64_t seed, int32_t n, int64_t m, double a, double b, double c, int relabel,
             int add_loops, gen_graph* out) {
  if (n <= 1 || m < 0 || m > (int64_t)n * (n - 1)) return -3;
  int32_t scale = ceil_log2(n);
  int32_t* pi = NULL;
  if (relabel) {
    pi = (int32_t*)malloc((size_t)n * 4);
    if (!pi) return -1;
    gen_permutation(seed ^ 0xA5A5A5A5A5A5A5A5ULL, n, pi);
  }
  edge_buf e = {0};
  csr64 cur = {0};
  uint64_t t0 = 0;
  int64_t have = 0;
  int rc = 0;
  double ab = a + b, abc = a + b + c;
  while (have < m) {
    int64_t need = m - have;
    int64_t batch = need + need / 8 + 4096;
    e.n = 0;
    if (cur.m > 0 && csr_to_edges(&cur, &e)) { rc = -1; break; }
    csr64_free(&cur);
    int64_t base = e.n;
    if (eb_reserve(&e, base + batch)) { rc = -1; break; }
    int32_t* ts = e.src + base;
    int32_t* td = e.dst + base;
#pragma omp parallel for schedule(static)
    for (int64_t k = 0; k < batch; ++k) {
      uint64_t t = t0 + (uint64_t)k;
      int64_t u = 0, v = 0;
      uint64_t word = 0;
      for (int32_t l = 0; l < scale; ++l) {
        /* three levels per 64-bit draw, 21 random bits (resolution 2^-21) each */
        if (l % 3 == 0) word = gen_draw(seed, t * 16 + (uint64_t)(l / 3));
        double r = (double)((word >> (21 * (l % 3))) & 0x1FFFFF) * (1.0 / 2097152.0);
        int64_t bit = (int64_t)1 << (scale - 1 - l);
        if (r < a) {
        } else if (r < ab) {
          v |= bit;
        } else if (r < abc) {
          u |= bit;
        } else {
          u |= bit;
          v |= bit;
        }
      }
      if (u >= n || v >= n || u == v) {
        ts[k] = -1;
        td[k] = -1;
      } else {
        /* edge u -> v: destination v lists source u */
        ts[k] = relabel ? pi[u] : (int32_t)u;
        td[k] = relabel ? pi[v] : (int32_t)v;
      }
    }
    /* drop rejected attempts */
    int64_t w = base;
    for (int64_t k = 0; k < batch; ++k)
      if (ts[k] >= 0) {
        e.src[w] = ts[k];
        e.dst[w] = td[k];
        ++w;
      }
    e.n = w;
    t0 += (uint64_t)batch;
    if (assemble_csr(n, &e, &cur)) { rc = -1; break; }
    have = cur.m;
  }
  eb_free(&e);
  free(pi);
  if (rc == 0) rc = trim_csr(&cur, m, seed);
  if (rc == 0) rc = finish(&cur, add_loops, out);
  csr64_free(&cur);
  return rc;
}

/* G(n, m) over unordered pairs; stored symmetrically (2m directed entries). */
int gen_er_undirected(uint64_t seed, int32_t n, int64_t m_pairs, int add_loops, gen_graph* out) {
  if (n <= 1 || m_pairs < 0 || m_pairs > (int64_t)n * (n - 1) / 2) return -3;
  edge_buf e = {0};
  csr64 cur = {0};
  uint64_t t0 = 0;
  int64_t have = 0;
  int rc = 0;
  while (have < m_pairs) {
    int64_t need = m_pairs - have;
    int64_t batch = need + need / 8 + 64;
    e.n = 0;
    if (cur.m > 0 && csr_to_edges(&cur, &e)) { rc = -1; break; }
    csr64_free(&cur);
    int64_t base = e.n;
    if (eb_reserve(&e, base + batch)) { rc = -1; break; }
    int64_t w = base;
    for (int64_t k = 0; k < batch; ++k) {
      uint64_t t = t0 + (uint64_t)k;
      int32_t u = (int32_t)uint_below(seed, 2 * t, (uint64_t)n);
      int32_t v = (int32_t)uint_below(seed, 2 * t + 1, (uint64_t)n);
      if (u == v) continue;
      /* canonical orientation: store the pair once as (min -> max) */
      e.src[w] = u < v ? u : v;
      e.dst[w] = u < v ? v : u;
      ++w;
    }
    e.n = w;
    t0 += (uint64_t)batch;
    if (assemble_csr(n, &e, &cur)) { rc = -1; break; }
    have = cur.m;
  }
  if (rc == 0) rc = trim_csr(&cur, m_pairs, seed);
  if (rc == 0) {
    /* symmetrise */
    e.n = 0;
    if (csr_to_edges(&cur, &e)) rc = -1;
    if (rc == 0 && eb_reserve(&e, 2 * e.n + 1)) rc = -1;
    if (rc == 0) {
      int64_t half = e.n;
      for (int64_t k = 0; k < half; ++k) {
        e.src[half + k] = e.dst[k];
        e.dst[half + k] = e.src[k];
      }
      e.n = 2 * half;
      csr64_free(&cur);
      if (assemble_csr(n, &e, &cur)) rc = -1;
    }
  }
  eb_free(&e);
  if (rc == 0) rc = finish(&cur, add_loops, out);
  csr64_free(&cur);
  return rc;
}

/* Cluster graph: clusters [c*csize, (c+1)*csize); ordered pair (i -> j),
 * i != j in one cluster, present with probability p (counter = global pair
 * index); then round(frac * E_intra) distinct inter-cluster ordered pairs. */
int gen_cluster(uint64_t seed, int32_t n, int32_t csize, double p, double frac, int add_loops,
                gen_graph* out) {
  if (n <= 0 || csize <= 1 || n % csize != 0) return -3;
  int64_t ncl = n / csize;
  int64_t pairs_per = (int64_t)csize * csize;
  edge_buf e = {0};
  int64_t* cnt = (int64_t*)calloc((size_t)ncl + 1, 8);
  if (!cnt) return -1;
#pragma omp parallel for schedule(static)
  for (int64_t cl = 0; cl < ncl; ++cl) {
    int64_t s = 0;
    for (int64_t q = 0; q < pairs_per; ++q) {
      int64_t i = q / csize, j = q % csize;
      if (i != j && u01(seed, (uint64_t)(cl * pairs_per + q)) < p) ++s;
    }
    cnt[cl + 1] = s;
  }
  for (int64_t cl = 0; cl < ncl; ++cl) cnt[cl + 1] += cnt[cl];
  int64_t e_intra = cnt[ncl];
  int64_t e_inter = (int64_t)llround(frac * (double)e_intra);
  if (eb_reserve(&e, e_intra + e_inter + e_inter / 4 + 64)) {
    free(cnt);
    return -1;
  }
#pragma omp parallel for schedule(static)
  for (int64_t cl = 0; cl < ncl; ++cl) {
    int64_t w = cnt[cl];
    for (int64_t q = 0; q < pairs_per; ++q) {
      int64_t i = q / csize, j = q % csize;
      if (i != j && u01(seed, (uint64_t)(cl * pairs_per + q)) < p) {
        e.src[w] = (int32_t)(cl * csize + i);
        e.dst[w] = (int32_t)(cl * csize + j);
        ++w;
      }
    }
  }
  e.n = e_intra;
  free(cnt);
  /* inter-cluster edges: separate stream, deduplicated and trimmed */
  edge_buf x = {0};
  csr64 cur = {0};
  int64_t have = 0;
  uint64_t t0 = 0;
  int rc = 0;
  uint64_t s2 = seed ^ 0x1C1C1C1C1C1C1C1CULL;
  while (have < e_inter) {
    int64_t need = e_inter - have;
    int64_t batch = need + need / 8 + 64;
    x.n = 0;
    if (cur.m > 0 && csr_to_edges(&cur, &x)) { rc = -1; break; }
    csr64_free(&cur);
    int64_t base = x.n;
    if (eb_reserve(&x, base + batch)) { rc = -1; break; }
    int64_t w = base;
    for (int64_t k = 0; k < batch; ++k) {
      uint64_t t = t0 + (uint64_t)k;
      int32_t u = (int32_t)uint_below(s2, 2 * t, (uint64_t)n);
      int32_t v = (int32_t)uint_below(s2, 2 * t + 1, (uint64_t)n);
      if (u / csize == v / csize) continue;
      x.src[w] = u;
      x.dst[w] = v;
      ++w;
    }
    x.n = w;
    t0 += (uint64_t)batch;
    if (assemble_csr(n, &x, &cur)) { rc = -1; break; }
    have = cur.m;
  }
  if (rc == 0) rc = trim_csr(&cur, e_inter, s2);
  if (rc == 0) {
    x.n = 0;
    if (csr_to_edges(&cur, &x)) rc = -1;
  }
  csr64_free(&cur);
  if (rc == 0 && eb_reserve(&e, e.n + x.n + 1)) rc = -1;
  if (rc == 0) {
    memcpy(e.src + e.n, x.src, (size_t)x.n * 4);
    memcpy(e.dst + e.n, x.dst, (size_t)x.n * 4);
    e.n += x.n;
    if (assemble_csr(n, &e, &cur)) rc = -1;
  }
  eb_free(&x);
  eb_free(&e);
  if (rc == 0) rc = finish(&cur, add_loops, out);
  csr64_free(&cur);
  return rc;
}

/* Build a CSR (rows = dst) from an explicit edge list; duplicates merged,
 * self loops kept as given.  Used by tests for hand-made graphs. */
int gen_from_edges(int32_t n, int64_t ne, const int32_t* src, const int32_t* dst, gen_graph* out) {
  edge_buf e = {0};
  if (eb_reserve(&e, ne + 1)) return -1;
  for (int64_t k = 0; k < ne; ++k) {
    if (src[k] < 0 || src[k] >= n || dst[k] < 0 || dst[k] >= n) {
      eb_free(&e);
      return -3;
    }
    e.src[k] = src[k];
    e.dst[k] = dst[k];
  }
  e.n = ne;
  csr64 cur = {0};
  int rc = assemble_csr(n, &e, &cur);
  eb_free(&e);
  if (rc == 0) rc = finish(&cur, 0, out);
  csr64_free(&cur);
  return rc;
}

int gen_num_threads(void) { return omp_get_max_threads(); }
