/*
 * CPU oracle for the wave-index build and decode. TEST INFRASTRUCTURE ONLY:
 * only the test suite, the smoke check and the benchmark's CPU-baseline leg
 * may load it. It shares no code with the HIP library.
 *
 * Sources (RetroInfer pages):
 *   [blog]  framerc.cn "KV缓存技术与RetroInfer系统在长上下文推理中的优化实践",
 *           section 2.1 (wave index: steady 4 + 64 tokens, retrieval ~1.8 %,
 *           estimation ~23 %, k-means over 8K-token segments, the
 *           segmented_kmeans sketch with per-cluster sums), section 2.2
 *           (2 KB blocks, cluster -> block mapping), section 3.1 (cluster KV
 *           stored contiguously), section 3.2 (execution buffer = steady zone
 *           + retrieved blocks, block fragments skipped), section 3.3
 *           (estimation from centroid vectors and cluster sizes, partial
 *           results merged).
 *   [news]  techwalker.com article, section 3 (three zones; estimation zone
 *           approximates the remaining tokens; segmented clustering).
 *   [gist]  gist.science summary, "Technische Samenvatting" 2A (centroids are
 *           cluster averages; segmented clustering keeps prefill cost low).
 *
 * Where the pages leave a step open the reading taken is stated at the
 * function. Every floating-point quantity that decides an integer (cluster
 * assignment, k-means++ pick) is computed in a fixed, stated order so the
 * result is a function of the inputs alone.
 */
#include "wi_oracle.h"

#include <math.h>
#include <omp.h>
#include <stdlib.h>
#include <string.h>

#define GAMMA 0x9E3779B97F4A7C15ull

/* ------------------------------------------------------------------------ */
/* Partition. Steady zone = first n_sink and last n_local tokens ([blog] 2.1;
 * [news] 3). The remaining tokens [n_sink, N - n_local) are cut into
 * consecutive seg_len-token segments, the last one possibly short; each
 * segment has min(k, n_s) clusters; cluster ids are contiguous by segment.
 * Reading: steady tokens are not clustered (they are always attended
 * exactly, so clustering them too would count them twice). */

/* Clustered tokens: the indexed range minus the pending tokens (decode-time
 * tokens whose segment has not filled yet). */
static int64_t idx_count(const wio_desc *d) {
  return d->n_ctx - d->n_sink - d->n_local - d->n_pending;
}

static int64_t seg_count(const wio_desc *d) {
  return (idx_count(d) + d->seg_len - 1) / d->seg_len;
}

static int64_t seg_len_of(const wio_desc *d, int64_t s) {
  int64_t left = idx_count(d) - s * d->seg_len;
  return left < d->seg_len ? left : d->seg_len;
}

static int tokens_per_block(const wio_desc *d) {
  int e = d->dtype == WIO_BF16 ? 2 : 4;
  return 2048 / (d->head_dim * e); /* 2 KB blocks ([blog] 2.2) */
}

int wio_sizes(const wio_desc *d, int64_t *n_segments, int64_t *n_clusters,
              int64_t *block_cap, int32_t *tpb) {
  if (d->head_dim != 128 || d->seg_len < 1 || d->clusters_per_seg < 1 ||
      d->n_sink < 0 || d->n_local < 0 || d->n_pending < 0 ||
      d->n_pending > d->seg_len ||
      d->n_ctx < (int64_t)d->n_sink + d->n_local + d->n_pending + 1)
    return -1;
  int64_t ns = seg_count(d), C = 0;
  for (int64_t s = 0; s < ns; s++) {
    int64_t n = seg_len_of(d, s);
    C += n < d->clusters_per_seg ? n : d->clusters_per_seg;
  }
  int T = tokens_per_block(d);
  int64_t n_idx = idx_count(d);
  if (n_segments) *n_segments = ns;
  if (n_clusters) *n_clusters = C;
  if (block_cap) *block_cap = (n_idx + C * (T - 1)) / T;
  if (tpb) *tpb = T;
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Counter-based generator: the SplitMix64 output finaliser (Steele, Lea and
 * Flood, "Fast splittable pseudorandom number generators", OOPSLA 2014)
 * applied to a key chained over (seed, b, l, h, s, r). The pages do not
 * state how clustering is seeded; a counter-based stream makes every
 * segment's draws independent of how segments are scheduled. */

uint64_t wio_mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

uint64_t wio_key(uint64_t seed, uint64_t b, uint64_t l, uint64_t h,
                 uint64_t s, uint64_t r) {
  uint64_t key = wio_mix64(seed + GAMMA);
  key = wio_mix64(key ^ (b + GAMMA));
  key = wio_mix64(key ^ (l + GAMMA));
  key = wio_mix64(key ^ (h + GAMMA));
  key = wio_mix64(key ^ (s + GAMMA));
  key = wio_mix64(key ^ (r + GAMMA));
  return key;
}

/* floor(r53 * m / 2^53) for the 53-bit uniform r53 = key >> 11, m < 2^63. */
static uint64_t scale53(uint64_t key, uint64_t m) {
  unsigned __int128 p = (unsigned __int128)(key >> 11) * m;
  return (uint64_t)(p >> 53);
}

/* ------------------------------------------------------------------------ */
/* Round a float32 to the nearest bfloat16, ties to even (the usual storage
 * rounding; values here are finite). */
float wio_round_bf16(float x) {
  uint32_t u;
  memcpy(&u, &x, 4);
  uint32_t lsb = (u >> 16) & 1u;
  u = (u + 0x7FFFu + lsb) & 0xFFFF0000u;
  float y;
  memcpy(&y, &u, 4);
  return y;
}

/* k-means++ distance: float32, one fused multiply-add per dimension in
 * dimension order. */
float wio_dist32(const float *x, const float *c, int d) {
  float acc = 0.0f;
  for (int t = 0; t < d; t++) {
    float delta = x[t] - c[t];
    acc = fmaf(delta, delta, acc);
  }
  return acc;
}

/* Assignment distance: float64, differences in float64, one fused
 * multiply-add per dimension in dimension order. For bf16 data every
 * difference and square is exact, so this is the squared Euclidean distance
 * up to the rounding of a 128-term sum of non-negative terms. */
double wio_dist64(const float *x, const float *c, int d) {
  double acc = 0.0;
  for (int t = 0; t < d; t++) {
    double delta = (double)x[t] - (double)c[t];
    acc = fma(delta, delta, acc);
  }
  return acc;
}

/* ------------------------------------------------------------------------ */
/* k-means++ seeding of one segment (Arthur and Vassilvitskii, "k-means++:
 * the advantages of careful seeding", SODA 2007): the first centroid is a
 * uniformly drawn point; each further centroid is a point drawn with
 * probability proportional to its squared distance to the nearest centroid
 * chosen so far. The pages name no initialisation; k-means++ is the standard
 * one for Lloyd's algorithm.
 *
 * Sampling arithmetic (reading): squared distances are float32 (wio_dist32);
 * they are turned into integer weights w_i = floor(D_i * 2^F) with F fixed
 * once per segment from the distances to the first centroid, so that the
 * total stays below 2^62; the draw is the smallest i whose inclusive prefix
 * of weights exceeds floor(U * W). This is D^2 sampling with each weight
 * rounded down to a grid of 2^-F (about 2^-49 of the largest weight) and
 * makes the pick independent of summation order. When every weight is zero
 * the smallest index not yet chosen is taken. */
void wio_kmeanspp(const float *X, int n, int d, int k, uint64_t seed,
                  uint64_t b, uint64_t l, uint64_t h, uint64_t s,
                  int32_t *picks) {
  float *D = (float *)malloc(sizeof(float) * (size_t)n);
  unsigned char *chosen = (unsigned char *)calloc((size_t)n, 1);
  uint64_t k0 = wio_key(seed, b, l, h, s, 0);
  int i0 = (int)scale53(k0, (uint64_t)n);
  picks[0] = i0;
  chosen[i0] = 1;
  float maxd = 0.0f;
  for (int i = 0; i < n; i++) {
    D[i] = wio_dist32(X + (size_t)i * d, X + (size_t)i0 * d, d);
    if (D[i] > maxd) maxd = D[i];
  }
  int L = 0;
  while ((1ll << L) < n) L++;
  int F = 0;
  if (maxd > 0.0f) {
    int e;
    frexp((double)maxd, &e); /* maxd < 2^e */
    F = 62 - L - e;
  }
  for (int r = 1; r < k; r++) {
    uint64_t W = 0;
    if (maxd > 0.0f)
      for (int i = 0; i < n; i++) W += (uint64_t)floor(ldexp((double)D[i], F));
    int pick = -1;
    if (W == 0) {
      for (int i = 0; i < n; i++)
        if (!chosen[i]) { pick = i; break; }
    } else {
      uint64_t target = scale53(wio_key(seed, b, l, h, s, (uint64_t)r), W);
      uint64_t P = 0;
      for (int i = 0; i < n; i++) {
        P += (uint64_t)floor(ldexp((double)D[i], F));
        if (P > target) { pick = i; break; }
      }
    }
    if (pick < 0) abort(); /* unreachable: target < W guarantees a pick */
    picks[r] = pick;
    chosen[pick] = 1;
    const float *c = X + (size_t)pick * d;
    for (int i = 0; i < n; i++) {
      float dn = wio_dist32(X + (size_t)i * d, c, d);
      if (dn < D[i]) D[i] = dn;
    }
  }
  free(D);
  free(chosen);
}

/* Lloyd assignment step: each point goes to the centroid at the smallest
 * squared distance (wio_dist64); ties go to the lowest centroid index. */
void wio_assign(const float *X, int n, int d, const float *C, int k,
                int32_t *a) {
  for (int i = 0; i < n; i++) {
    const float *x = X + (size_t)i * d;
    double best = wio_dist64(x, C, d);
    int bi = 0;
    for (int c = 1; c < k; c++) {
      double dc = wio_dist64(x, C + (size_t)c * d, d);
      if (dc < best) { best = dc; bi = c; }
    }
    a[i] = bi;
  }
}

/* Lloyd update step: a centroid becomes the average of its members ([gist]
 * 2A: centroids are cluster averages). Reading: the sum is taken in float64
 * over members in ascending position, divided by the count in float64,
 * rounded to float32 and then (for bf16 storage) to bf16, ties to even. An
 * empty cluster keeps its previous centroid. */
void wio_update(const float *X, int n, int d, const int32_t *a, int k,
                int dtype, float *C, int32_t *counts) {
  double *sum = (double *)calloc((size_t)k * d, sizeof(double));
  for (int c = 0; c < k; c++) counts[c] = 0;
  for (int i = 0; i < n; i++) { /* ascending position */
    int c = a[i];
    counts[c]++;
    for (int t = 0; t < d; t++) sum[(size_t)c * d + t] += (double)X[(size_t)i * d + t];
  }
  for (int c = 0; c < k; c++) {
    if (counts[c] == 0) continue;
    for (int t = 0; t < d; t++) {
      double m = sum[(size_t)c * d + t] / (double)counts[c];
      float m32 = (float)m;
      C[(size_t)c * d + t] = dtype == WIO_BF16 ? wio_round_bf16(m32) : m32;
    }
  }
  free(sum);
}

/* ------------------------------------------------------------------------ */
/* Full build ([blog] 2.1 segmented_kmeans: per segment k-means, keep the
 * centroids and per-cluster value sums; [blog] 2.2 and 3.1: cluster KV laid
 * out contiguously in 2 KB blocks). */
int wio_build(const wio_desc *d, const float *K, const float *V,
              const float *init, float *centroids, int32_t *sizes,
              float *vsum, int32_t *block_off, float *kblk, float *vblk,
              int32_t *slot_token, float *steady_k, float *steady_v,
              int32_t *assign, const unsigned char *unit_mask) {
  int64_t ns, C, cap;
  int32_t T;
  if (wio_sizes(d, &ns, &C, &cap, &T) != 0) return -1;
  if (d->n_pending != 0) return -1; /* an index is built with nothing pending */
  const int D = d->head_dim;
  const int64_t N = d->n_ctx;
  const int64_t n_idx = N - d->n_sink - d->n_local;
  const int64_t U = (int64_t)d->batch * d->n_kv_heads;
  const int kk = d->clusters_per_seg;
  int64_t *cbase = (int64_t *)malloc(sizeof(int64_t) * (size_t)(ns + 1));
  cbase[0] = 0;
  for (int64_t s = 0; s < ns; s++) {
    int64_t n = seg_len_of(d, s);
    cbase[s + 1] = cbase[s] + (n < kk ? n : kk);
  }

  /* Clustering: every (unit, segment) is independent ([blog] 2.1 runs the
   * segments in parallel). */
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t job = 0; job < U * ns; job++) {
    int64_t u = job / ns, s = job % ns;
    if (unit_mask && !unit_mask[u]) continue;
    int64_t b = u / d->n_kv_heads, h = u % d->n_kv_heads;
    int64_t start = d->n_sink + s * d->seg_len;
    int n = (int)seg_len_of(d, s);
    int k = (int)(cbase[s + 1] - cbase[s]);
    const float *X = K + ((size_t)u * N + start) * D;
    float *Cu = centroids + ((size_t)u * C + cbase[s]) * D;
    if (init) {
      memcpy(Cu, init + ((size_t)u * C + cbase[s]) * D, sizeof(float) * (size_t)k * D);
    } else {
      int32_t *picks = (int32_t *)malloc(sizeof(int32_t) * (size_t)k);
      wio_kmeanspp(X, n, D, k, d->seed, (uint64_t)b, d->layer_id, (uint64_t)h,
                   (uint64_t)s, picks);
      for (int j = 0; j < k; j++)
        memcpy(Cu + (size_t)j * D, X + (size_t)picks[j] * D, sizeof(float) * D);
      free(picks);
    }
    int32_t *a = (int32_t *)malloc(sizeof(int32_t) * (size_t)n);
    int32_t *cnt = sizes + (size_t)u * C + cbase[s];
    int iters = d->n_iters > 0 ? d->n_iters : 1;
    for (int t = 0; t < iters; t++) {
      wio_assign(X, n, D, Cu, k, a);
      if (d->n_iters > 0) wio_update(X, n, D, a, k, d->dtype, Cu, cnt);
    }
    if (d->n_iters == 0) {
      for (int c = 0; c < k; c++) cnt[c] = 0;
      for (int i = 0; i < n; i++) cnt[a[i]]++;
    }
    for (int i = 0; i < n; i++)
      assign[(size_t)u * n_idx + s * d->seg_len + i] = (int32_t)(cbase[s] + a[i]);
    free(a);
  }

  /* Layout and value sums, one unit at a time. */
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t u = 0; u < U; u++) {
    if (unit_mask && !unit_mask[u]) continue;
    const int32_t *cnt = sizes + (size_t)u * C;
    int32_t *bo = block_off + (size_t)u * (C + 1);
    bo[0] = 0;
    for (int64_t c = 0; c < C; c++) bo[c + 1] = bo[c] + (cnt[c] + T - 1) / T;
    int32_t *st = slot_token + (size_t)u * cap * T;
    float *kb = kblk + (size_t)u * cap * T * D;
    float *vb = vblk + (size_t)u * cap * T * D;
    for (int64_t j = 0; j < cap * T; j++) st[j] = -1;
    memset(kb, 0, sizeof(float) * (size_t)cap * T * D);
    memset(vb, 0, sizeof(float) * (size_t)cap * T * D);
    int32_t *fill = (int32_t *)calloc((size_t)C, sizeof(int32_t));
    double *vs = (double *)calloc((size_t)C * D, sizeof(double));
    const int32_t *au = assign + (size_t)u * n_idx;
    for (int64_t i = 0; i < n_idx; i++) { /* ascending position */
      int32_t c = au[i];
      int64_t pos = d->n_sink + i;
      int64_t slot = (int64_t)bo[c] * T + fill[c]++;
      st[slot] = (int32_t)pos;
      const float *kr = K + ((size_t)u * N + pos) * D;
      const float *vr = V + ((size_t)u * N + pos) * D;
      memcpy(kb + slot * D, kr, sizeof(float) * D);
      memcpy(vb + slot * D, vr, sizeof(float) * D);
      for (int t = 0; t < D; t++) vs[(size_t)c * D + t] += (double)vr[t];
    }
    for (int64_t c = 0; c < C; c++)
      for (int t = 0; t < D; t++)
        vsum[((size_t)u * C + c) * D + t] = (float)vs[(size_t)c * D + t];
    free(fill);
    free(vs);
    int nst = d->n_sink + d->n_local;
    for (int j = 0; j < nst; j++) {
      int64_t pos = j < d->n_sink ? j : N - d->n_local + (j - d->n_sink);
      memcpy(steady_k + ((size_t)u * nst + j) * D, K + ((size_t)u * N + pos) * D, sizeof(float) * D);
      memcpy(steady_v + ((size_t)u * nst + j) * D, V + ((size_t)u * N + pos) * D, sizeof(float) * D);
    }
  }
  free(cbase);
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Decode. */

static double dot64(const float *a, const float *b, int d) {
  double acc = 0.0;
  for (int t = 0; t < d; t++) acc += (double)a[t] * (double)b[t];
  return acc;
}

typedef struct { double g; int32_t id; } ranked;

/* Rank order: larger score first; equal scores by lower cluster id. */
static int rank_cmp(const void *pa, const void *pb) {
  const ranked *a = (const ranked *)pa, *b = (const ranked *)pb;
  if (a->g > b->g) return -1;
  if (a->g < b->g) return 1;
  return (a->id > b->id) - (a->id < b->id);
}

/* Tripartite attention for one query head ([blog] 2.1 and 3.3; [news] 3):
 *   the steady zone, the pending tokens (decode-time tokens that left the
 *   local window and wait for their segment to fill; they are no longer
 *   steady and not yet clustered, so the reading taken is that they are
 *   attended exactly) and the retrieval-zone clusters' tokens are attended
 *   exactly;
 *   each estimation-zone cluster c with n_c > 0 stands for n_c keys equal to
 *   its centroid: it adds n_c * exp(s_c) to the softmax denominator and
 *   exp(s_c) * VS_c (its value sum) to the numerator ([blog] 3.3 "centroid
 *   vectors and sizes"; the value sums are the compute_cluster_sums of the
 *   [blog] 2.1 sketch);
 *   all other clusters are dropped.
 * All arithmetic in float64; the result is one softmax over the union. */
static void attend_head(const wio_desc *d, double scale, const float *qh,
                        int64_t u, const float *centroids, const int32_t *sizes,
                        const float *vsum, const int32_t *block_off,
                        const float *kblk, const float *vblk,
                        const float *steady_k, const float *steady_v,
                        const float *pend_k, const float *pend_v,
                        int64_t C, int64_t cap, int T, const int32_t *R,
                        int n_r, const int32_t *E, int n_e, double *o) {
  const int D = d->head_dim;
  const int nst = d->n_sink + d->n_local;
  const int64_t np = d->n_pending;
  const float *sk = steady_k + (size_t)u * nst * D;
  const float *sv = steady_v + (size_t)u * nst * D;
  const float *pk = np > 0 ? pend_k + (size_t)u * d->seg_len * D : NULL;
  const float *pv = np > 0 ? pend_v + (size_t)u * d->seg_len * D : NULL;
  const float *kb = kblk + (size_t)u * cap * T * D;
  const float *vb = vblk + (size_t)u * cap * T * D;
  const int32_t *bo = block_off + (size_t)u * (C + 1);
  const int32_t *cnt = sizes + (size_t)u * C;
  /* pass 1: the maximum logit over every term */
  double m = -INFINITY;
  for (int j = 0; j < nst; j++) {
    double z = dot64(qh, sk + (size_t)j * D, D) * scale;
    if (z > m) m = z;
  }
  for (int64_t j = 0; j < np; j++) {
    double z = dot64(qh, pk + (size_t)j * D, D) * scale;
    if (z > m) m = z;
  }
  for (int r = 0; r < n_r; r++) {
    int32_t c = R[r];
    for (int32_t j = 0; j < cnt[c]; j++) {
      int64_t slot = (int64_t)bo[c] * T + j;
      double z = dot64(qh, kb + slot * D, D) * scale;
      if (z > m) m = z;
    }
  }
  for (int e = 0; e < n_e; e++) {
    int32_t c = E[e];
    if (cnt[c] == 0) continue;
    double s = dot64(qh, centroids + ((size_t)u * C + c) * D, D) * scale;
    if (s > m) m = s;
  }
  /* pass 2: numerator and denominator */
  double den = 0.0;
  for (int t = 0; t < D; t++) o[t] = 0.0;
  for (int j = 0; j < nst; j++) {
    double p = exp(dot64(qh, sk + (size_t)j * D, D) * scale - m);
    den += p;
    for (int t = 0; t < D; t++) o[t] += p * (double)sv[(size_t)j * D + t];
  }
  for (int64_t j = 0; j < np; j++) {
    double p = exp(dot64(qh, pk + (size_t)j * D, D) * scale - m);
    den += p;
    for (int t = 0; t < D; t++) o[t] += p * (double)pv[(size_t)j * D + t];
  }
  for (int r = 0; r < n_r; r++) {
    int32_t c = R[r];
    for (int32_t j = 0; j < cnt[c]; j++) {
      int64_t slot = (int64_t)bo[c] * T + j;
      double p = exp(dot64(qh, kb + slot * D, D) * scale - m);
      den += p;
      for (int t = 0; t < D; t++) o[t] += p * (double)vb[slot * D + t];
    }
  }
  for (int e = 0; e < n_e; e++) {
    int32_t c = E[e];
    if (cnt[c] == 0) continue;
    double s = dot64(qh, centroids + ((size_t)u * C + c) * D, D) * scale;
    double p = exp(s - m);
    den += (double)cnt[c] * p;
    const float *vs = vsum + ((size_t)u * C + c) * D;
    for (int t = 0; t < D; t++) o[t] += p * (double)vs[t];
  }
  for (int t = 0; t < D; t++) o[t] /= den;
}

int wio_decode(const wio_desc *d, const wio_ddesc *dd, const float *centroids,
               const int32_t *sizes, const float *vsum,
               const int32_t *block_off, const float *kblk, const float *vblk,
               const int32_t *slot_token, const float *steady_k,
               const float *steady_v, const float *pend_k,
               const float *pend_v, const float *q, double *out,
               int32_t *sel, int32_t *exec_tokens, int32_t *n_exec,
               int64_t exec_cap, double *gkey) {
  int64_t ns, C, cap;
  int32_t T;
  if (wio_sizes(d, &ns, &C, &cap, &T) != 0) return -1;
  if (dd->k_retrieve > C || dd->k_retrieve < 0 || dd->k_estimate < 0) return -1;
  if (dd->n_q_heads % d->n_kv_heads != 0) return -1;
  const int D = d->head_dim;
  const int G = dd->n_q_heads / d->n_kv_heads;
  const int K_r = dd->k_retrieve;
  const int K_e = (int)(dd->k_estimate < C - K_r ? dd->k_estimate : C - K_r);
  const double scale = dd->scale > 0 ? dd->scale : 1.0 / sqrt((double)D);
  const int64_t U = (int64_t)d->batch * d->n_kv_heads;
  const int nst = d->n_sink + d->n_local;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t u = 0; u < U; u++) {
    int64_t b = u / d->n_kv_heads, h = u % d->n_kv_heads;
    const float *qg = q + ((size_t)b * dd->n_q_heads + (size_t)h * G) * D;
    /* Score ([blog] 2.2: query the wave index for cluster ids). Reading:
     * one selection per KV head, keyed by the sum over its query heads of
     * <q_h, centroid>; this ranks like the scaled logit sum. The key is that
     * sum in float64 -- exact for bf16 data, whose products and short sums
     * are exact there -- and equal keys go to the lower cluster id. The
     * pages fix no precision for the ranking, so the oracle ranks on the
     * exact group score. */
    ranked *rk = (ranked *)malloc(sizeof(ranked) * (size_t)C);
    for (int64_t c = 0; c < C; c++) {
      double g = 0.0;
      for (int j = 0; j < G; j++)
        g += dot64(qg + (size_t)j * D, centroids + ((size_t)u * C + c) * D, D);
      rk[c].g = g;
      rk[c].id = (int32_t)c;
      if (gkey) gkey[(size_t)u * C + c] = g;
    }
    qsort(rk, (size_t)C, sizeof(ranked), rank_cmp);
    int32_t *R = (int32_t *)malloc(sizeof(int32_t) * (size_t)(K_r + 1));
    int32_t *E = (int32_t *)malloc(sizeof(int32_t) * (size_t)(K_e + 1));
    for (int r = 0; r < K_r; r++) R[r] = rk[r].id;
    for (int e = 0; e < K_e; e++) E[e] = rk[K_r + e].id;
    if (sel)
      for (int r = 0; r < K_r + K_e; r++) sel[(size_t)u * (K_r + K_e) + r] = rk[r].id;
    /* Execution buffer order ([blog] 3.2): steady tokens in position order,
     * then the pending tokens in position order, then each retrieved
     * cluster's tokens (fragments skipped), clusters in rank order, tokens in
     * ascending position. */
    if (exec_tokens || n_exec) {
      const int32_t *bo = block_off + (size_t)u * (C + 1);
      const int32_t *cnt = sizes + (size_t)u * C;
      const int32_t *st = slot_token + (size_t)u * cap * T;
      int64_t pos = 0;
      for (int j = 0; j < nst; j++, pos++) {
        int64_t tok = j < d->n_sink ? j : d->n_ctx - d->n_local + (j - d->n_sink);
        if (exec_tokens && pos < exec_cap) exec_tokens[(size_t)u * exec_cap + pos] = (int32_t)tok;
      }
      const int64_t p0 = d->n_sink + idx_count(d); /* first pending position */
      for (int64_t j = 0; j < d->n_pending; j++, pos++)
        if (exec_tokens && pos < exec_cap) exec_tokens[(size_t)u * exec_cap + pos] = (int32_t)(p0 + j);
      for (int r = 0; r < K_r; r++) {
        int32_t c = R[r];
        for (int32_t j = 0; j < cnt[c]; j++, pos++)
          if (exec_tokens && pos < exec_cap)
            exec_tokens[(size_t)u * exec_cap + pos] = st[(int64_t)bo[c] * T + j];
      }
      if (n_exec) n_exec[u] = (int32_t)pos;
    }
    for (int j = 0; j < G; j++)
      attend_head(d, scale, qg + (size_t)j * D, u, centroids, sizes, vsum,
                  block_off, kblk, vblk, steady_k, steady_v, pend_k, pend_v, C,
                  cap, T, R, K_r, E, K_e,
                  out + ((size_t)b * dd->n_q_heads + (size_t)h * G + j) * D);
    free(rk);
    free(R);
    free(E);
  }
  return 0;
}

int wio_attend_sets(const wio_desc *d, const wio_ddesc *dd,
                    const float *centroids, const int32_t *sizes,
                    const float *vsum, const int32_t *block_off,
                    const float *kblk, const float *vblk,
                    const float *steady_k, const float *steady_v,
                    const float *pend_k, const float *pend_v,
                    const float *q, const int32_t *R, int32_t n_r,
                    const int32_t *E, int32_t n_e, double *out) {
  int64_t ns, C, cap;
  int32_t T;
  if (wio_sizes(d, &ns, &C, &cap, &T) != 0) return -1;
  if (dd->n_q_heads % d->n_kv_heads != 0) return -1;
  const int D = d->head_dim;
  const int G = dd->n_q_heads / d->n_kv_heads;
  const double scale = dd->scale > 0 ? dd->scale : 1.0 / sqrt((double)D);
  const int64_t U = (int64_t)d->batch * d->n_kv_heads;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t u = 0; u < U; u++) {
    int64_t b = u / d->n_kv_heads, h = u % d->n_kv_heads;
    const float *qg = q + ((size_t)b * dd->n_q_heads + (size_t)h * G) * D;
    for (int j = 0; j < G; j++)
      attend_head(d, scale, qg + (size_t)j * D, u, centroids, sizes, vsum,
                  block_off, kblk, vblk, steady_k, steady_v, pend_k, pend_v, C,
                  cap, T, R + (size_t)u * n_r, n_r, E + (size_t)u * n_e, n_e,
                  out + ((size_t)b * dd->n_q_heads + (size_t)h * G + j) * D);
  }
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Decode steps that grow the index. Generating token t reads the history and
 * then appends the current token's key and value ([blog] 1.1, read/write
 * pattern; the cache is kept like a ring buffer). The steady zone is the
 * first n_sink and the last n_local tokens ([blog] 2.1), so appending
 * position n_ctx moves position n_ctx - n_local out of the local window.
 * Reading: that token becomes pending -- attended exactly -- until seg_len
 * such tokens form the next segment, which is then clustered like every
 * segment ([blog] 2.1: k-means per 8K-token segment, segments independent). */
int wio_append(const wio_desc *d, float *steady_k, float *steady_v,
               float *pend_k, float *pend_v, const float *k_new,
               const float *v_new) {
  int64_t ns, C, cap;
  int32_t T;
  if (wio_sizes(d, &ns, &C, &cap, &T) != 0) return -1;
  if (d->n_pending >= d->seg_len) return -1;
  const int D = d->head_dim;
  const int nst = d->n_sink + d->n_local;
  const int64_t U = (int64_t)d->batch * d->n_kv_heads;
  for (int64_t u = 0; u < U; u++) {
    float *sk = steady_k + (size_t)u * nst * D, *sv = steady_v + (size_t)u * nst * D;
    float *pk = pend_k + ((size_t)u * d->seg_len + d->n_pending) * D;
    float *pv = pend_v + ((size_t)u * d->seg_len + d->n_pending) * D;
    const float *kn = k_new + (size_t)u * D, *vn = v_new + (size_t)u * D;
    if (d->n_local > 0) {
      /* the oldest local token leaves the window */
      memcpy(pk, sk + (size_t)d->n_sink * D, sizeof(float) * D);
      memcpy(pv, sv + (size_t)d->n_sink * D, sizeof(float) * D);
      memmove(sk + (size_t)d->n_sink * D, sk + (size_t)(d->n_sink + 1) * D,
              sizeof(float) * (size_t)(d->n_local - 1) * D);
      memmove(sv + (size_t)d->n_sink * D, sv + (size_t)(d->n_sink + 1) * D,
              sizeof(float) * (size_t)(d->n_local - 1) * D);
      memcpy(sk + (size_t)(nst - 1) * D, kn, sizeof(float) * D);
      memcpy(sv + (size_t)(nst - 1) * D, vn, sizeof(float) * D);
    } else {
      memcpy(pk, kn, sizeof(float) * D);
      memcpy(pv, vn, sizeof(float) * D);
    }
  }
  return 0;
}

int wio_extend(const wio_desc *d, const float *centroids, const int32_t *sizes,
               const float *vsum, const int32_t *block_off, const float *kblk,
               const float *vblk, const int32_t *slot_token,
               const float *steady_k, const float *steady_v,
               const int32_t *assign, const float *pend_k, const float *pend_v,
               float *n_centroids, int32_t *n_sizes, float *n_vsum,
               int32_t *n_block_off, float *n_kblk, float *n_vblk,
               int32_t *n_slot_token, float *n_steady_k, float *n_steady_v,
               int32_t *n_assign) {
  int64_t ns, C, cap, ns2, C2, cap2;
  int32_t T, T2;
  if (wio_sizes(d, &ns, &C, &cap, &T) != 0) return -1;
  if (d->n_pending != d->seg_len) return -1;
  wio_desc dn = *d;
  dn.n_pending = 0;
  if (wio_sizes(&dn, &ns2, &C2, &cap2, &T2) != 0) return -1;
  const int D = d->head_dim;
  const int n = d->seg_len;
  const int k = n < d->clusters_per_seg ? n : d->clusters_per_seg;
  if (C2 != C + k) return -1;
  const int64_t n_idx = idx_count(d);
  const int64_t p0 = d->n_sink + n_idx; /* first pending position */
  const int64_t s_new = ns;             /* the new segment's ordinal */
  const int nst = d->n_sink + d->n_local;
  const int64_t U = (int64_t)d->batch * d->n_kv_heads;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t u = 0; u < U; u++) {
    const int64_t b = u / d->n_kv_heads, h = u % d->n_kv_heads;
    const float *X = pend_k + (size_t)u * n * D;
    const float *Vp = pend_v + (size_t)u * n * D;
    /* the new segment, clustered as wio_build clusters a segment */
    float *Cn = n_centroids + ((size_t)u * C2 + C) * D;
    int32_t *cnt = n_sizes + (size_t)u * C2 + C;
    int32_t *picks = (int32_t *)malloc(sizeof(int32_t) * (size_t)k);
    wio_kmeanspp(X, n, D, k, d->seed, (uint64_t)b, d->layer_id, (uint64_t)h,
                 (uint64_t)s_new, picks);
    for (int j = 0; j < k; j++)
      memcpy(Cn + (size_t)j * D, X + (size_t)picks[j] * D, sizeof(float) * D);
    free(picks);
    int32_t *a = (int32_t *)malloc(sizeof(int32_t) * (size_t)n);
    const int iters = d->n_iters > 0 ? d->n_iters : 1;
    for (int t = 0; t < iters; t++) {
      wio_assign(X, n, D, Cn, k, a);
      if (d->n_iters > 0) wio_update(X, n, D, a, k, d->dtype, Cn, cnt);
    }
    if (d->n_iters == 0) {
      for (int c = 0; c < k; c++) cnt[c] = 0;
      for (int i = 0; i < n; i++) cnt[a[i]]++;
    }
    /* the old clusters, blocks, steady rows and assignments, unchanged */
    memcpy(n_centroids + (size_t)u * C2 * D, centroids + (size_t)u * C * D,
           sizeof(float) * (size_t)C * D);
    memcpy(n_sizes + (size_t)u * C2, sizes + (size_t)u * C, sizeof(int32_t) * (size_t)C);
    memcpy(n_vsum + (size_t)u * C2 * D, vsum + (size_t)u * C * D, sizeof(float) * (size_t)C * D);
    const int32_t *bo = block_off + (size_t)u * (C + 1);
    int32_t *nbo = n_block_off + (size_t)u * (C2 + 1);
    memcpy(nbo, bo, sizeof(int32_t) * (size_t)(C + 1));
    const int64_t used = bo[C];
    int32_t *nst_tok = n_slot_token + (size_t)u * cap2 * T;
    float *nkb = n_kblk + (size_t)u * cap2 * T * D, *nvb = n_vblk + (size_t)u * cap2 * T * D;
    for (int64_t j = 0; j < cap2 * T; j++) nst_tok[j] = -1;
    memset(nkb, 0, sizeof(float) * (size_t)cap2 * T * D);
    memset(nvb, 0, sizeof(float) * (size_t)cap2 * T * D);
    memcpy(nst_tok, slot_token + (size_t)u * cap * T, sizeof(int32_t) * (size_t)used * T);
    memcpy(nkb, kblk + (size_t)u * cap * T * D, sizeof(float) * (size_t)used * T * D);
    memcpy(nvb, vblk + (size_t)u * cap * T * D, sizeof(float) * (size_t)used * T * D);
    memcpy(n_steady_k + (size_t)u * nst * D, steady_k + (size_t)u * nst * D,
           sizeof(float) * (size_t)nst * D);
    memcpy(n_steady_v + (size_t)u * nst * D, steady_v + (size_t)u * nst * D,
           sizeof(float) * (size_t)nst * D);
    memcpy(n_assign + (size_t)u * (n_idx + n), assign + (size_t)u * n_idx,
           sizeof(int32_t) * (size_t)n_idx);
    /* the new clusters take the next ids and the blocks after the used ones;
     * members in ascending position, value sums in float64 */
    for (int c = 0; c < k; c++) nbo[C + c + 1] = nbo[C + c] + (cnt[c] + T - 1) / T;
    if (nbo[C + k] > cap2) abort(); /* unreachable: cap2 bounds the used blocks */
    int32_t *fill = (int32_t *)calloc((size_t)k, sizeof(int32_t));
    double *vs = (double *)calloc((size_t)k * D, sizeof(double));
    for (int i = 0; i < n; i++) {
      const int c = a[i];
      const int64_t slot = (int64_t)nbo[C + c] * T + fill[c]++;
      nst_tok[slot] = (int32_t)(p0 + i);
      memcpy(nkb + slot * D, X + (size_t)i * D, sizeof(float) * D);
      memcpy(nvb + slot * D, Vp + (size_t)i * D, sizeof(float) * D);
      for (int t = 0; t < D; t++) vs[(size_t)c * D + t] += (double)Vp[(size_t)i * D + t];
      n_assign[(size_t)u * (n_idx + n) + n_idx + i] = (int32_t)(C + c);
    }
    for (int c = 0; c < k; c++)
      for (int t = 0; t < D; t++)
        n_vsum[((size_t)u * C2 + C + c) * D + t] = (float)vs[(size_t)c * D + t];
    free(fill);
    free(vs);
    free(a);
  }
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Per-layer zone policy pieces. [blog] 3.3 (layer-wise strategy for very
 * large models): the lower layers keep full attention for precise
 * localisation, the middle layers use the hybrid scheme, the upper layers
 * raise the estimation share (to 30 %). [blog] 4.3 problem 3: sparse
 * attention is switched off in the first two layers. [blog] 4.3 problem 1:
 * the clustering's recall@100 should exceed 0.85. */

/* Dense decode attention over all N context tokens, per query head j of KV
 * head h (standard grouped-query mapping, h = j / G):
 *   o_j = sum_i e^{z_i - m} v_i / sum_i e^{z_i - m},  z_i = scale <q_j, k_i>,
 * m = max_i z_i, all in float64. K, V: [B][H][N][d]; q: [B][Hq][d];
 * out: [B][Hq][d]. */
int wio_dense_attention(const wio_desc *d, const wio_ddesc *dd, const float *K,
                        const float *V, const float *q, double *out) {
  if (dd->n_q_heads % d->n_kv_heads != 0 || d->n_ctx < 1) return -1;
  const int D = d->head_dim;
  const int G = dd->n_q_heads / d->n_kv_heads;
  const int64_t N = d->n_ctx;
  const double scale = dd->scale > 0 ? dd->scale : 1.0 / sqrt((double)D);
  const int64_t U = (int64_t)d->batch * d->n_kv_heads;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t u = 0; u < U; u++) {
    const int64_t b = u / d->n_kv_heads, h = u % d->n_kv_heads;
    const float *Ku = K + (size_t)u * N * D;
    const float *Vu = V + (size_t)u * N * D;
    for (int j = 0; j < G; j++) {
      const float *qh = q + ((size_t)b * dd->n_q_heads + (size_t)h * G + j) * D;
      double *o = out + ((size_t)b * dd->n_q_heads + (size_t)h * G + j) * D;
      double m = -INFINITY;
      for (int64_t i = 0; i < N; i++) {
        const double z = dot64(qh, Ku + (size_t)i * D, D) * scale;
        if (z > m) m = z;
      }
      double den = 0.0;
      for (int t = 0; t < D; t++) o[t] = 0.0;
      for (int64_t i = 0; i < N; i++) {
        const double p = exp(dot64(qh, Ku + (size_t)i * D, D) * scale - m);
        den += p;
        for (int t = 0; t < D; t++) o[t] += p * (double)Vu[(size_t)i * D + t];
      }
      for (int t = 0; t < D; t++) o[t] /= den;
    }
  }
  return 0;
}

typedef struct { double s; int32_t pos; int32_t c; } scored;

/* Token order for recall: larger score first, equal scores by lower
 * position. */
static int scored_cmp(const void *pa, const void *pb) {
  const scored *a = (const scored *)pa, *b = (const scored *)pb;
  if (a->s > b->s) return -1;
  if (a->s < b->s) return 1;
  return (a->pos > b->pos) - (a->pos < b->pos);
}

/* recall@k of a retrieval zone. Reading of "recall@100" ([blog] 4.3 problem
 * 1): for query head j of unit u, take the k clustered tokens with the
 * largest exact attention scores <q_j, k_i> (the tokens attention weights
 * most; equal scores by lower position) and count the share of them that
 * belong to a cluster of the unit's retrieval zone R_u. Steady and pending
 * tokens are attended exactly anyway and are not part of the measure. The
 * keys are read from the index's blocks (each clustered token once).
 *   R: [U][n_r] cluster ids; recall: [B][Hq]; top (optional): [B][Hq][k]
 *   positions in rank order; top_score (optional): their scores <q_j, k_i>.
 * Returns -1 when k < 1 or k exceeds the clustered token count. */
int wio_recall(const wio_desc *d, const wio_ddesc *dd, const int32_t *sizes,
               const int32_t *block_off, const float *kblk,
               const int32_t *slot_token, const float *q, const int32_t *R,
               int32_t n_r, int32_t k, double *recall, int32_t *top,
               double *top_score) {
  int64_t ns, C, cap;
  int32_t T;
  if (wio_sizes(d, &ns, &C, &cap, &T) != 0) return -1;
  if (dd->n_q_heads % d->n_kv_heads != 0) return -1;
  const int64_t n_idx = idx_count(d);
  if (k < 1 || k > n_idx) return -1;
  const int D = d->head_dim;
  const int G = dd->n_q_heads / d->n_kv_heads;
  const int64_t U = (int64_t)d->batch * d->n_kv_heads;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t u = 0; u < U; u++) {
    const int64_t b = u / d->n_kv_heads, h = u % d->n_kv_heads;
    const int32_t *bo = block_off + (size_t)u * (C + 1);
    const int32_t *cnt = sizes + (size_t)u * C;
    const int32_t *st = slot_token + (size_t)u * cap * T;
    const float *kb = kblk + (size_t)u * cap * T * D;
    unsigned char *inR = (unsigned char *)calloc((size_t)C, 1);
    for (int r = 0; r < n_r; r++) inR[R[(size_t)u * n_r + r]] = 1;
    scored *all = (scored *)malloc(sizeof(scored) * (size_t)n_idx);
    for (int j = 0; j < G; j++) {
      const size_t qi = (size_t)b * dd->n_q_heads + (size_t)h * G + j;
      const float *qh = q + qi * D;
      int64_t n = 0;
      for (int64_t c = 0; c < C; c++)
        for (int32_t i = 0; i < cnt[c]; i++) {
          const int64_t slot = (int64_t)bo[c] * T + i;
          all[n].s = dot64(qh, kb + slot * D, D);
          all[n].pos = st[slot];
          all[n].c = (int32_t)c;
          n++;
        }
      qsort(all, (size_t)n, sizeof(scored), scored_cmp);
      int hit = 0;
      for (int32_t i = 0; i < k; i++) {
        hit += inR[all[i].c];
        if (top) top[qi * k + i] = all[i].pos;
        if (top_score) top_score[qi * k + i] = all[i].s;
      }
      recall[qi] = (double)hit / (double)k;
    }
    free(all);
    free(inR);
  }
  return 0;
}

int wio_num_threads(void) { return omp_get_max_threads(); }
