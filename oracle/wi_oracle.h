/*
 * CPU oracle for the wave-index build and decode.
 *
 * TEST INFRASTRUCTURE ONLY. This is a plain, slow, scalar reading of the
 * method described on the RetroInfer pages (framerc blog "KV缓存技术与
 * RetroInfer系统...", sections 2.1-3.3; techwalker article, section 3;
 * gist.science summary, "Technische Samenvatting" section 2A). Only the test
 * suite, the smoke check and the benchmark's CPU-baseline leg may load it.
 * It shares no code, header or table with the HIP library and must never be
 * used as a fallback for it.
 *
 * All tensors are passed as float32 arrays whose values are exactly the
 * stored dtype values (bf16 values are exact in float32). Floating-point
 * results that the method defines as averages or sums are produced in the
 * precision stated at each function.
 */
#ifndef WI_ORACLE_H
#define WI_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Storage dtypes. */
enum { WIO_F32 = 0, WIO_BF16 = 1 };

typedef struct {
  int32_t dtype;
  int32_t batch, n_kv_heads, head_dim;
  int64_t n_ctx;
  int32_t seg_len, clusters_per_seg, n_sink, n_local, n_iters;
  uint64_t seed;
  uint32_t layer_id;
  /* Tokens that have left the local window during decode and wait, attended
   * exactly, for their segment to fill: positions [n_sink + n_idx, n_sink +
   * n_idx + n_pending) with n_idx = n_ctx - n_sink - n_local - n_pending the
   * clustered range. 0 for an index as built. */
  int64_t n_pending;
} wio_desc;

typedef struct {
  int32_t n_q_heads;
  int32_t k_retrieve, k_estimate;
  double scale; /* 0 -> 1/sqrt(head_dim) */
} wio_ddesc;

/* ---- partition ------------------------------------------------------- */
/* Number of segments of one unit, clusters per unit, and the block
 * capacity per unit (an upper bound on sum_c ceil(n_c / T)). Returns 0 on
 * success, -1 on invalid sizes. */
int wio_sizes(const wio_desc *d, int64_t *n_segments, int64_t *n_clusters,
              int64_t *block_cap, int32_t *tokens_per_block);

/* ---- counter-based random numbers ------------------------------------ */
uint64_t wio_mix64(uint64_t z);
uint64_t wio_key(uint64_t seed, uint64_t b, uint64_t l, uint64_t h,
                 uint64_t s, uint64_t r);

/* ---- rounding and distances ------------------------------------------ */
float wio_round_bf16(float x);
float wio_dist32(const float *x, const float *c, int d);
double wio_dist64(const float *x, const float *c, int d);

/* ---- k-means pieces on one segment ------------------------------------ */
void wio_kmeanspp(const float *X, int n, int d, int k, uint64_t seed,
                  uint64_t b, uint64_t l, uint64_t h, uint64_t s,
                  int32_t *picks);
void wio_assign(const float *X, int n, int d, const float *C, int k,
                int32_t *a);
void wio_update(const float *X, int n, int d, const int32_t *a, int k,
                int dtype, float *C, int32_t *counts);

/* ---- full build ------------------------------------------------------- */
/* K, V: [B][H][N][d]. init: [B][H][C][d] or NULL (k-means++).
 * Outputs per unit u = b*H + h:
 *   centroids [U][C][d], sizes [U][C], vsum [U][C][d],
 *   block_off [U][C+1], kblk/vblk [U][cap*T][d], slot_token [U][cap*T],
 *   steady_k/steady_v [U][n_sink+n_local][d], assign [U][n_idx].
 * unit_mask: [U] or NULL; units with a zero entry are skipped (their
 * outputs are left untouched). */
int wio_build(const wio_desc *d, const float *K, const float *V,
              const float *init, float *centroids, int32_t *sizes,
              float *vsum, int32_t *block_off, float *kblk, float *vblk,
              int32_t *slot_token, float *steady_k, float *steady_v,
              int32_t *assign, const unsigned char *unit_mask);

/* ---- decode ----------------------------------------------------------- */
/* q: [B][Hq][d]. out: [B][Hq][d] (fp64). sel: [U][K_r + K_e'] cluster ids
 * in rank order (K_e' = min(K_e, C - K_r)); exec_tokens: [U][exec_cap]
 * (token positions, steady then retrieved clusters in rank order);
 * n_exec: [U]. gkey: [U][C] exact group-summed scores or NULL.
 * Returns 0, or -1 when K_r > C. */
int wio_decode(const wio_desc *d, const wio_ddesc *dd, const float *centroids,
               const int32_t *sizes, const float *vsum,
               const int32_t *block_off, const float *kblk, const float *vblk,
               const int32_t *slot_token, const float *steady_k,
               const float *steady_v, const float *pend_k,
               const float *pend_v, const float *q, double *out,
               int32_t *sel, int32_t *exec_tokens, int32_t *n_exec,
               int64_t exec_cap, double *gkey);

/* Tripartite attention for given retrieval set R [U][n_r] and estimation
 * set E [U][n_e] (cluster ids), fp64. Used to check a selection made
 * elsewhere once that selection has been validated. */
int wio_attend_sets(const wio_desc *d, const wio_ddesc *dd,
                    const float *centroids, const int32_t *sizes,
                    const float *vsum, const int32_t *block_off,
                    const float *kblk, const float *vblk,
                    const float *steady_k, const float *steady_v,
                    const float *pend_k, const float *pend_v,
                    const float *q, const int32_t *R, int32_t n_r,
                    const int32_t *E, int32_t n_e, double *out);

/* ---- decode steps that grow the index -------------------------------- */
/* One appended token per sequence: k_new, v_new [B][H][d]. The local window
 * slides by one: the token leaving it (position n_ctx - n_local; the new
 * token itself when n_local = 0) becomes pending row n_pending; the steady
 * rows keep the sinks, then the local window in position order. steady_k/v
 * [U][n_sink+n_local][d] and pend_k/v [U][seg_len][d] are updated in place;
 * afterwards the index is described by n_ctx + 1 and n_pending + 1. Returns
 * -1 when n_pending = seg_len already (the segment must be clustered first). */
int wio_append(const wio_desc *d, float *steady_k, float *steady_v,
               float *pend_k, float *pend_v, const float *k_new,
               const float *v_new);

/* Cluster a full pending segment (n_pending = seg_len) as the next segment of
 * the stream and write the grown index: its geometry is that of d with
 * n_pending = 0. The new segment is clustered exactly as the build clusters
 * a segment (k-means++ from the random stream of (seed, b, layer, h,
 * segment ordinal), then n_iters Lloyd iterations), its clusters take the
 * next ids and its blocks follow the index's used blocks. Inputs are the
 * index arrays for d (old geometry) and the pending rows; outputs the arrays
 * for the new geometry (caller-allocated). */
int wio_extend(const wio_desc *d, const float *centroids, const int32_t *sizes,
               const float *vsum, const int32_t *block_off, const float *kblk,
               const float *vblk, const int32_t *slot_token,
               const float *steady_k, const float *steady_v,
               const int32_t *assign, const float *pend_k, const float *pend_v,
               float *n_centroids, int32_t *n_sizes, float *n_vsum,
               int32_t *n_block_off, float *n_kblk, float *n_vblk,
               int32_t *n_slot_token, float *n_steady_k, float *n_steady_v,
               int32_t *n_assign);

/* ---- per-layer policy pieces --------------------------------------- */
/* Dense decode attention over all n_ctx tokens, float64 (the full-attention
 * layers of the per-layer zone policy). K, V: [B][H][N][d]; q, out:
 * [B][Hq][d]. */
int wio_dense_attention(const wio_desc *d, const wio_ddesc *dd, const float *K,
                        const float *V, const float *q, double *out);

/* recall@k of a retrieval zone R ([U][n_r] cluster ids): per query head, the
 * share of the k clustered tokens with the largest exact scores (ties to the
 * lower position) that lie in R's clusters. recall: [B][Hq]; top / top_score
 * (optional): [B][Hq][k] positions in rank order and their scores. */
int wio_recall(const wio_desc *d, const wio_ddesc *dd, const int32_t *sizes,
               const int32_t *block_off, const float *kblk,
               const int32_t *slot_token, const float *q, const int32_t *R,
               int32_t n_r, int32_t k, double *recall, int32_t *top,
               double *top_score);

int wio_num_threads(void);

#ifdef __cplusplus
}
#endif
#endif
