/*
 * wi.h -- C ABI of the wave-index library (libwi.so) for AMD Instinct MI355X
 * (gfx950).
 *
 * Two operations, as the RetroInfer pages state the problem:
 *
 *   wi_build_index      cluster each KV head's keys independently per
 *                       fixed-length segment (k-means), keep centroids,
 *                       cluster sizes and per-cluster value sums, and lay
 *                       the KV out cluster-contiguously in 2 KB blocks
 *                       (framerc blog, section 2.1 "Wave索引" and its
 *                       segmented_kmeans sketch; section 2.2, 2 KB physical
 *                       blocks; section 3.1, one cluster's KV stored
 *                       contiguously).
 *
 *   wi_decode_attention for one decode query per sequence: score every
 *                       centroid, take the top clusters as the retrieval
 *                       zone and the next tier as the estimation zone,
 *                       attend exactly over the steady zone (first n_sink and
 *                       last n_local tokens) plus the retrieved clusters'
 *                       tokens, estimate the estimation zone from centroid
 *                       score x cluster size and the cluster value sum, and
 *                       merge the partial softmaxes (framerc blog section
 *                       2.1 zones; section 2.2 sync path step 1, query the
 *                       index for cluster ids; section 3.2 execution buffer;
 *                       section 3.3 hybrid attention and merge; techwalker
 *                       article section 3, the three zones).
 *
 * Conventions (all entry points):
 *   - Every buffer is caller-owned device memory (except descriptors, which
 *     are host structs). The library never allocates or frees memory, keeps
 *     no state between calls and fully overwrites every output it is given,
 *     padding included.
 *   - All device work is enqueued on `stream` (NULL = default stream). Calls
 *     return after enqueue without synchronising. Outputs are valid, and
 *     inputs reusable, only after the caller synchronises the stream.
 *   - Validation happens on the host before any HIP call; a call that fails
 *     validation enqueues nothing.
 *   - Pointers to device buffers must be 16-byte aligned.
 *   - The same inputs and seed give bit-identical outputs on every run.
 *   - Stateless: concurrent calls on different streams with disjoint
 *     workspaces and outputs are safe.
 *   - Device faults surface at the caller's next synchronisation.
 */
#ifndef WI_H
#define WI_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  WI_OK = 0,
  WI_E_INVALID = 1,     /* null required pointer, misalignment, bad sizes  */
  WI_E_UNSUPPORTED = 2, /* head_dim != 128, unknown dtype, Hq % Hkv != 0   */
  WI_E_WORKSPACE = 3,   /* workspace smaller than the sizes call reports   */
  WI_E_HIP = 4          /* a HIP launch error; text in wi_last_error()     */
} wi_status;

enum { WI_F32 = 0, WI_BF16 = 1 };

/* Index shape. One unit = (sequence b, KV head h) of one layer.
 * Steady zone: positions [0, n_sink) and [n_ctx - n_local, n_ctx).
 * Pending tokens (decode-time only, see wi_append_token): the n_pending
 * positions just before the local window; they have left the window, wait for
 * their segment to fill and are attended exactly.
 * Clustered tokens: [n_sink, n_ctx - n_local - n_pending), n_idx of them, cut
 * into consecutive segments of seg_len tokens (as built, the last one may be
 * short; segments added by wi_extend_index are full); segment s has
 * C_s = min(clusters_per_seg, n_s) clusters; cluster ids are contiguous by
 * segment, so C = sum_s C_s clusters per unit (as if the n_idx clustered
 * tokens were cut from the start, which gives the same count).
 * Tokens per 2 KB block: T = 2048 / (head_dim * bytes(dtype)) = 8 (bf16) or
 * 4 (fp32). */
typedef struct {
  int32_t dtype;            /* WI_F32 or WI_BF16: keys, values, centroids, q */
  int32_t batch;            /* B >= 1                                        */
  int32_t n_kv_heads;       /* H >= 1                                        */
  int32_t head_dim;         /* must be 128                                   */
  int64_t n_ctx;            /* N >= n_sink + n_local + 1                     */
  int32_t seg_len;          /* tokens per segment, 1..8192 (8192 = 8K)       */
  int32_t clusters_per_seg; /* k, 1..512                                     */
  int32_t n_sink;           /* leading steady tokens (4), >= 0               */
  int32_t n_local;          /* trailing steady tokens (64), >= 0             */
  int32_t n_iters;          /* Lloyd iterations after initialisation, >= 0   */
  uint64_t seed;            /* k-means++ seed                                */
  uint32_t layer_id;        /* mixed into the k-means++ random stream        */
  int64_t kv_stride_b;      /* element strides of the K and V inputs         */
  int64_t kv_stride_h;      /*   [B, H, N, head_dim]; head_dim contiguous;   */
  int64_t kv_stride_t;      /*   all strides must be multiples of 8          */
  int64_t n_pending;        /* 0 .. seg_len; 0 for wi_build_index            */
} wi_index_desc;

/* Index buffers (device memory, caller-owned). C and cap come from
 * wi_index_sizes; U = batch * n_kv_heads; n_idx = n_ctx - n_sink - n_local -
 * n_pending; n_st = n_sink + n_local.
 *   centroids    [U][C][128] dtype   cluster means (rounded to dtype)
 *   cluster_size [U][C] int32        members per cluster
 *   value_sum    [U][C][128] float   sum of member values (fp64, rounded)
 *   block_off    [U][C+1] int32      first block of each cluster; [C] = used
 *   k_blocks     [U][cap][T][128]    keys, cluster-contiguous, 2 KB blocks
 *   v_blocks     [U][cap][T][128]    values, same layout
 *   slot_token   [U][cap*T] int32    token position of each slot, -1 = pad
 *   steady_k     [U][n_st][128]      keys of the steady zone, in order
 *   steady_v     [U][n_st][128]      values of the steady zone
 *   assign       [U][n_idx] int32    cluster id of each clustered token
 *   pend_k       [U][seg_len][128]   pending keys in position order (decode-
 *   pend_v       [U][seg_len][128]   time growth only; may be NULL while
 *                                    n_pending = 0 and no token is appended)
 * Cluster c's members occupy slots [T*block_off[c], T*block_off[c] + size[c])
 * in ascending position; remaining slots of its last block, and all blocks
 * past block_off[C], hold token -1 and zero data. */
typedef struct {
  void *centroids;
  int32_t *cluster_size;
  float *value_sum;
  int32_t *block_off;
  void *k_blocks;
  void *v_blocks;
  int32_t *slot_token;
  void *steady_k;
  void *steady_v;
  int32_t *assign;
  void *pend_k;
  void *pend_v;
} wi_index_bufs;

/* Host-only: sizes derived from the descriptor. Any output pointer may be
 * NULL. Returns WI_E_INVALID / WI_E_UNSUPPORTED for a bad descriptor. */
wi_status wi_index_sizes(const wi_index_desc *desc, int64_t *n_segments,
                         int64_t *n_clusters, int64_t *block_cap,
                         size_t *workspace_bytes);

/* Build the index of every unit (desc->n_pending must be 0).
 *   k, v          device [B][H][N][128] dtype, strides from desc
 *   init_centroids NULL: k-means++ seeding per segment (first centroid
 *                 uniform, then D^2 sampling; counter-based random stream
 *                 keyed by (seed, b, layer_id, h, segment, round)).
 *                 Non-NULL: device [U][C][128] dtype starting centroids.
 *   Then n_iters Lloyd iterations (assign to the nearest centroid, lowest id
 *   on ties; replace each non-empty cluster's centroid by the rounded mean
 *   of its members). With n_iters = 0 the centroids stay at their initial
 *   values and the membership is one assignment to them. The outputs are
 *   the last assignment's membership and the last update's centroids.
 *   ws            device workspace of >= workspace_bytes from
 *                 wi_index_sizes; contents on entry are ignored.
 *   bufs->k_blocks also serves as scratch during k-means++ seeding, before
 *   its final contents are written; no output may overlap k or v.
 */
wi_status wi_build_index(const wi_index_desc *desc, const void *k,
                         const void *v, const void *init_centroids,
                         const wi_index_bufs *bufs, void *ws, size_t ws_bytes,
                         hipStream_t stream);

/* Decode shape. Query head j maps to KV head j / (n_q_heads / n_kv_heads). */
typedef struct {
  int32_t n_q_heads;   /* multiple of n_kv_heads; G = Hq / Hkv <= 16      */
  int32_t k_retrieve;  /* K_r: retrieval-zone clusters, 0 <= K_r <= C      */
  int32_t k_estimate;  /* K_e: estimation-zone clusters, clamped to C-K_r */
  float scale;         /* softmax scale; 0 -> 1/sqrt(head_dim)            */
  int32_t wg_per_unit; /* workgroups per (sequence, KV head) of the fused
                          kernel: 0 = automatic (about one per compute
                          unit over the call); 1..64 = that many, at most
                          one per 16 clusters. Results agree to rounding
                          order across choices; each choice is itself
                          deterministic                                    */
} wi_decode_desc;

/* Host-only: workspace bytes for wi_decode_attention. Its contents on entry
 * are ignored (the call initialises what it uses). */
wi_status wi_decode_sizes(const wi_index_desc *desc,
                          const wi_decode_desc *ddesc, size_t *workspace_bytes);

/* One decode step for every sequence of the batch.
 *   q            device [B][Hq][128] dtype
 *   out          device [B][Hq][128] float32 attention output
 *   Ranking: clusters of a unit are ranked by g_c = sum over the unit's query
 *   heads of <q_j, centroid_c>, computed exactly and rounded once to float32,
 *   larger first, lower id on equal float32 keys.
 *   Ranks [0, K_r) form the retrieval zone R, the next
 *   min(K_e, C - K_r) ranks the estimation zone E. For each query head j:
 *     out_j = (sum_{i in steady + pending + members(R)} e^{z_i} v_i
 *              + sum_{c in E, n_c > 0} e^{s_c} VS_c)
 *           / (sum_{i} e^{z_i} + sum_{c in E, n_c > 0} n_c e^{s_c}),
 *   z_i = scale <q_j, k_i>, s_c = scale <q_j, centroid_c>.
 * Optional debug outputs (written only when non-NULL):
 *   sel_ids      device [U][K_r + K_e'] cluster ids in rank order
 *   exec_tokens  device [U][exec_cap] token positions of the execution
 *                buffer: steady positions in order, then the pending
 *                positions in order, then each retrieved cluster's members
 *                (rank order, ascending position);
 *                entries past exec_cap are dropped; needs slot_token
 *   n_exec       device [U] execution-buffer length (may exceed exec_cap)
 *   bufs->assign is not read; bufs->slot_token only for exec_tokens;
 *   bufs->pend_k/pend_v only when n_pending > 0. The
 *   index must be one wi_build_index wrote (cluster c's members in the
 *   first cluster_size[c] slots from block block_off[c], within block_cap).
 *   NaN in q or the centroids leaves the selection unspecified (no fault).
 *   Returns WI_E_WORKSPACE if ws_bytes is below wi_decode_sizes; a unit with
 *   no steady, retrieved or estimated token gets a zero output row.
 */
wi_status wi_decode_attention(const wi_index_desc *desc,
                              const wi_decode_desc *ddesc,
                              const wi_index_bufs *bufs, const void *q,
                              float *out, int32_t *sel_ids,
                              int32_t *exec_tokens, int32_t *n_exec,
                              int64_t exec_cap, void *ws, size_t ws_bytes,
                              hipStream_t stream);

/* Decode-time growth of the index (framerc blog section 1.1: generating a
 * token reads the cached history and then appends the token's KV, the cache
 * being kept like a ring buffer; section 2.1: the steady zone is the first
 * n_sink and last n_local tokens, and clusters are formed per seg_len-token
 * segment). One token per sequence is appended per call: the local window
 * slides by one and the token leaving it (position n_ctx - n_local; the new
 * token itself when n_local = 0) becomes pending row n_pending. Once
 * seg_len tokens are pending, wi_extend_index clusters them as the next
 * segment.
 *   k_new, v_new  device [B][H][128] dtype, the new token's key and value
 *   bufs          the index for desc; steady_k/v and pend_k/v are updated
 *                 in place (pend_k/v required)
 * Afterwards the index is described by n_ctx + 1 and n_pending + 1.
 * Returns WI_E_INVALID when n_pending = seg_len (extend first). */
wi_status wi_append_token(const wi_index_desc *desc, const wi_index_bufs *bufs,
                          const void *k_new, const void *v_new,
                          hipStream_t stream);

/* Host-only: workspace bytes of wi_append_tokens (2 x U x n_local rows). */
wi_status wi_append_sizes(const wi_index_desc *desc, size_t *workspace_bytes);

/* n_new tokens per sequence at once -- a prefill chunk, or several decode
 * steps (framerc blog section 2.1, with section 4.3 problem 3: the index is
 * built as prefill produces each segment) -- with the same effect as n_new
 * calls of wi_append_token: with the local window's rows followed by the new
 * rows, the first n_new become pending rows n_pending .. n_pending + n_new - 1
 * and the last n_local the new local window.
 *   k_new, v_new  device [B][H][n_new][128] dtype
 *   n_new         1 .. seg_len - n_pending (cluster a full segment with
 *                 wi_extend_index before appending more)
 *   ws            device workspace of wi_append_sizes bytes
 * Afterwards the index is described by n_ctx + n_new and n_pending + n_new. */
wi_status wi_append_tokens(const wi_index_desc *desc, const wi_index_bufs *bufs,
                           const void *k_new, const void *v_new, int32_t n_new,
                           void *ws, size_t ws_bytes, hipStream_t stream);

/* Host-only: workspace bytes of wi_extend_index for desc (n_pending =
 * seg_len). */
wi_status wi_extend_sizes(const wi_index_desc *desc, size_t *workspace_bytes);

/* Cluster the full pending segment (desc->n_pending = seg_len) as the
 * stream's next segment and write the grown index to new_bufs, whose
 * geometry is desc with n_pending = 0 (sizes from wi_index_sizes of that
 * descriptor). The segment is clustered exactly as wi_build_index clusters a
 * segment: k-means++ from the random stream keyed by (seed, b, layer_id, h,
 * segment ordinal = the old index's segment count), then n_iters Lloyd
 * iterations; its clusters take ids C .. C + C_s - 1 and its blocks follow
 * the old index's used blocks. Every other cluster, block, steady row and
 * assignment is copied unchanged. Old and new buffers must not overlap, except
 * new_bufs->pend_k/v, which may alias the old ones (they are not written). */
wi_status wi_extend_index(const wi_index_desc *desc, const wi_index_bufs *bufs,
                          const wi_index_bufs *new_bufs, void *ws, size_t ws_bytes,
                          hipStream_t stream);

/* ---- per-layer zone policy ------------------------------------------ */
/* framerc blog section 3.3 (layer-wise strategy, given for an 80-layer
 * model): layers 0-20 keep full attention for precise localisation, layers
 * 21-60 use the hybrid scheme, the upper layers raise the estimation share
 * to 30 %. Section 4.3, problem 3: sparse attention switched off in the
 * first two layers. Section 2.1: hybrid budgets of about 1.8 % retrieved and
 * 23 % estimated tokens. */
enum { WI_LAYER_DENSE = 0, WI_LAYER_HYBRID = 1 };
enum {
  WI_POLICY_UNIFORM = 0,      /* every layer hybrid (1.8 %, 23 %)            */
  WI_POLICY_DENSE_FIRST2 = 1, /* layers 0 and 1 dense, the rest hybrid       */
  WI_POLICY_BANDED = 2        /* dense if 80 l < 21 L; hybrid with a 30 %
                                 estimation share if 80 l >= 61 L; else
                                 hybrid (the 80-layer bands as fractions of
                                 depth L)                                    */
};

/* Host-only: the plan of layer `layer` of an n_layers-layer model at n_ctx
 * tokens: *mode (WI_LAYER_DENSE or WI_LAYER_HYBRID) and, for hybrid layers,
 * the cluster budgets round(f * n_ctx * clusters_per_seg / seg_len) for the
 * token shares f (0 and 0 for dense layers). Any output may be NULL.
 * WI_E_INVALID for an unknown policy or a layer outside [0, n_layers). */
wi_status wi_layer_plan(int32_t policy, int32_t layer, int32_t n_layers,
                        int64_t n_ctx, int32_t seg_len, int32_t clusters_per_seg,
                        int32_t *mode, int32_t *k_retrieve, int32_t *k_estimate);

/* Host-only: workspace bytes of wi_dense_attention. */
wi_status wi_dense_sizes(const wi_index_desc *desc,
                         const wi_decode_desc *ddesc, size_t *workspace_bytes);

/* Dense decode attention, for the layers a policy keeps dense: every one of
 * the n_ctx tokens is attended by each query head of its KV head,
 *   out_j = sum_i e^{z_i} v_i / sum_i e^{z_i},  z_i = scale <q_j, k_i>.
 * Only desc's dtype, batch, n_kv_heads, head_dim (128), n_ctx (>= 1) and
 * K/V strides are read; ddesc's n_q_heads and scale (0 -> 1/sqrt(128)).
 *   k, v   device [B][H][N][128] dtype, strides from desc
 *   q      device [B][Hq][128] dtype
 *   out    device [B][Hq][128] float32
 *   ws     device workspace of wi_dense_sizes bytes (chunk partials) */
wi_status wi_dense_attention(const wi_index_desc *desc,
                             const wi_decode_desc *ddesc, const void *k,
                             const void *v, const void *q, float *out,
                             void *ws, size_t ws_bytes, hipStream_t stream);

/* Host-only: workspace bytes of wi_recall_at_k (8 bytes per used slot of
 * every query head). */
wi_status wi_recall_sizes(const wi_index_desc *desc,
                          const wi_decode_desc *ddesc, size_t *workspace_bytes);

/* recall@k of a retrieval zone (framerc blog section 4.3, problem 1: the
 * clustering's recall@100 should exceed 0.85). For each query head j: the k
 * clustered tokens with the largest scores <q_j, k_i> (float32 from the
 * index's key blocks; equal scores by lower position) and the share of them
 * whose cluster is in the unit's retrieval zone.
 *   bufs        the index (block_off, k_blocks, slot_token, assign)
 *   q           device [B][Hq][128] dtype
 *   sel_ids     device, unit u's retrieval zone is sel_ids[u * sel_stride
 *               .. + n_r) (e.g. the first K_r ids of wi_decode_attention's
 *               sel_ids, sel_stride = K_r + K_e')
 *   k           1 .. min(1024, clustered tokens)
 *   recall      device [B][Hq] float32
 *   top_tokens  device [B][Hq][k] int32 positions in rank order, or NULL
 *   ws          device workspace of wi_recall_sizes bytes */
wi_status wi_recall_at_k(const wi_index_desc *desc, const wi_decode_desc *ddesc,
                         const wi_index_bufs *bufs, const void *q,
                         const int32_t *sel_ids, int32_t sel_stride,
                         int32_t n_r, int32_t k, float *recall,
                         int32_t *top_tokens, void *ws, size_t ws_bytes,
                         hipStream_t stream);

/* ---- wave buffer: a GPU block cache in front of a host-memory tier -- */
/* framerc blog section 2.2 (wave buffer): the KV blocks live in CPU
 * memory; a GPU cache holds hot 2 KB blocks with a block -> slot mapping
 * table. The synchronous access path reads a retrieved block from its cache
 * slot when cached and from CPU memory otherwise; the asynchronous update
 * path keeps an LRU replacement and the table. Per unit:
 *   block_slot  device [U][block_cap] int32   cache slot of a block, or -1
 *   slot_block  device [U][n_slots] int32     block held by a slot, or -1
 *   slot_last   device [U][n_slots] uint32    last step that used the slot
 *                                             (0: never)
 *   slot_order  device [U][n_slots] int32     the slots sorted by (slot_last,
 *                                             slot id): the eviction order
 *   cache_k/v   device [U][n_slots * T][128] dtype   the cached blocks
 * The caller owns every buffer; wi_wave_buffer_reset empties the tables. */
typedef struct {
  int32_t n_slots;          /* cache capacity per unit in blocks, 1 .. 8192 */
  int32_t *block_slot;
  int32_t *slot_block;
  uint32_t *slot_last;
  void *cache_k;
  void *cache_v;
  int32_t *slot_order;
} wi_wave_buffer;

/* Empty the cache tables (every block uncached, every slot free). */
wi_status wi_wave_buffer_reset(const wi_index_desc *desc, const wi_wave_buffer *wb,
                               hipStream_t stream);

/* Host-only: workspace bytes of wi_decode_attention_wb. */
wi_status wi_decode_wb_sizes(const wi_index_desc *desc,
                             const wi_decode_desc *ddesc, int32_t n_slots,
                             size_t *workspace_bytes);

/* wi_decode_attention with the KV blocks in host memory behind the wave
 * buffer. bufs->k_blocks and bufs->v_blocks are pinned host memory
 * (hipHostMalloc or equivalent, device-visible) holding the index's block
 * pools; every other index buffer is device memory. The output equals
 * wi_decode_attention's on the same index bit for bit: a retrieved row is
 * read from its block's cache slot when the block is cached and from host
 * memory otherwise. Then the update path runs for step `step` (> 0, larger
 * than every earlier step of this wave buffer): the blocks of the retrieved
 * clusters, ascending, are looked up; hits mark their slot used at `step`;
 * misses, ascending, take the slots not used at `step` in order of (last
 * use, slot id), evicting those slots' blocks, and are copied from host
 * memory into them (as many misses as there are such slots).
 *   stats   device [U][2] int32 (hits, misses) of this step, or NULL */
wi_status wi_decode_attention_wb(const wi_index_desc *desc,
                                 const wi_decode_desc *ddesc,
                                 const wi_index_bufs *bufs,
                                 const wi_wave_buffer *wb, uint32_t step,
                                 const void *q, float *out, int32_t *stats,
                                 void *ws, size_t ws_bytes, hipStream_t stream);

/* Largest decode workspace that wi_decode_attention_noalloc serves: 16 MiB
 * (the five model shapes of this library need at most 11.5 MiB: 8 units of
 * 65536 clusters, or 64 units of 8192). */
#define WI_NOALLOC_SCRATCH_BYTES (16ull << 20)

/* For callers that cannot allocate device memory or call an allocating
 * routine: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc. Same inputs, outputs and results as wi_decode_attention
 * (same kernels); its workspace is a fixed device array of
 * WI_NOALLOC_SCRATCH_BYTES inside the library instead of a caller buffer.
 *   - Allocates nothing: no hipMalloc, hipFree or allocating library call.
 *     On its first call on a device (that device current) it looks up that
 *     device's copy of the array once (hipGetSymbolAddress) and keeps the
 *     address; each GPU holds its copy until the process ends.
 *   - Uses the calling thread's current device; `stream` must belong to it.
 *   - Returns WI_E_WORKSPACE, before any HIP call, when wi_decode_sizes for
 *     this call exceeds WI_NOALLOC_SCRATCH_BYTES.
 *   - Every call on one GPU shares that GPU's array, which keeps the last
 *     call's contents (each call initialises what it reads): calls that may
 *     overlap in time on one GPU (different streams, or different threads)
 *     race and must be serialised by the caller. With the measurement hook
 *     (wi_timing_start) on, its event creation is the hook's, not this
 *     call's. */
wi_status wi_decode_attention_noalloc(const wi_index_desc *desc,
                                      const wi_decode_desc *ddesc,
                                      const wi_index_bufs *bufs, const void *q,
                                      float *out, int32_t *sel_ids,
                                      int32_t *exec_tokens, int32_t *n_exec,
                                      int64_t exec_cap, hipStream_t stream);

/* Measurement hook. wi_timing_start() makes every kernel launch issued by
 * this library on the calling thread be bracketed by two HIP events recorded
 * on the launch's own stream (timing-only events, recorded without a
 * system-scope memory fence), until wi_timing_stop(). wi_timing_stop()
 * synchronises those events and writes, for up to max_records launches in
 * issue order, the kernel's name id (see wi_kernel_name) and its duration in
 * milliseconds; it returns the number of launches recorded (which may exceed
 * max_records) or -1 on a HIP error. Timing adds an event pair per launch and
 * is meant for measurement runs only. */
wi_status wi_timing_start(void);
int32_t wi_timing_stop(int32_t max_records, int32_t *name_ids, float *ms);
const char *wi_kernel_name(int32_t name_id);

/* Human-readable name of a status code (static storage). */
const char *wi_status_str(wi_status s);

/* Message of the last failed call on this thread (thread-local storage;
 * empty string if none). */
const char *wi_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* WI_H */
