// Internal declarations shared by the HIP translation units of libwi.so.
// gfx950 only: wave64, MFMA, 160 KB LDS per CU.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/wi.h"

namespace wi {

constexpr int D = 128;          // head_dim
constexpr int MAX_G = 16;       // query heads per KV head
constexpr int MAX_K = 512;      // clusters per segment
constexpr int MAX_SEG = 8192;   // tokens per segment

// ---------------------------------------------------------------------------
// Geometry of one call, computed on the host from the descriptor.
struct Geom {
  int dtype;        // WI_F32 / WI_BF16
  int B, H, U;      // batch, KV heads, units
  int64_t N;        // context tokens
  int n_sink, n_local, n_st;
  int64_t n_idx;    // indexed tokens per unit
  int seg_len, kk;  // segment length, clusters per full segment
  int n_seg;        // segments per unit
  int C;            // clusters per unit
  int T;            // tokens per 2 KB block
  int64_t cap;      // block capacity per unit
  int64_t sb, sh, st;  // K/V element strides
  uint64_t seed;
  uint32_t layer;
  int n_iters;
  int cmax;         // max clusters of any segment = min(kk, seg_len, n_idx)
  int n_pend;       // pending tokens, positions [n_sink + n_idx, + n_pend)
  int seg_ord0;     // ordinal of segment 0 in the k-means++ random stream
};

// Segment s of a unit: first indexed position, length, cluster count/base.
__host__ __device__ inline int64_t seg_first(const Geom& g, int s) {
  return (int64_t)g.n_sink + (int64_t)s * g.seg_len;
}
__host__ __device__ inline int seg_n(const Geom& g, int s) {
  int64_t left = g.n_idx - (int64_t)s * g.seg_len;
  return (int)(left < g.seg_len ? left : g.seg_len);
}
__host__ __device__ inline int seg_c(const Geom& g, int s) {
  int n = seg_n(g, s);
  return n < g.kk ? n : g.kk;
}
__host__ __device__ inline int seg_cbase(const Geom& g, int s) {
  int full = g.seg_len < g.kk ? g.seg_len : g.kk;  // clusters of a full segment
  return s * full;
}

// ---------------------------------------------------------------------------
// Build workspace (device pointers carved from the caller's buffer).
struct KppPartial {
  unsigned long long sum[2];  // per parity: sum of weights of the slice
  int minun[2];               // per parity: smallest unchosen local index
  float maxd;                 // max distance after the first pick
  int pad;
};

struct BuildWs {
  float* D;                    // [U*n_idx] k-means++ distances
  unsigned long long* w[2];    // [U*n_idx] k-means++ weights, by parity
  unsigned char* chosen;       // [U*n_idx]
  KppPartial* kpp;             // [U*n_seg*kpp_slices]
  int* label;                  // [U*n_idx] local cluster index per point
  int* members;                // [U*n_idx] local token index, cluster order
  int* cl_off;                 // [U*C] first member of each cluster (segment-local)
  int* amb;                    // [1 + U*n_idx] ambiguous-point count + list
  int* seg_blocks;             // [U*n_seg] blocks used by each segment
  int* seg_bbase;              // [U*n_seg] first block of each segment
  int* unit_used;              // [U] blocks used by each unit
  void* kc;                    // [4][U*n_idx][32] dtype: the indexed keys in
                               // 32-dimension chunks, chunk-major (k-means++
                               // only; lives in the k_blocks output, which the
                               // layout step writes afterwards)
};
constexpr int KPP_SLICE = 256;  // points per k-means++ workgroup

// Decode workspace.
struct DecodeWs {
  uint32_t* key;       // [U][Cp] order-preserving ranking keys (Cp = C rounded up to 4)
  float* S;            // [U*C*GS] scaled per-head centroid logits (GS = 4, 8, 16)
  float2* mm;          // [U][score_blocks] key range (min, max) of each score workgroup
  float* part;         // [U*W*G*(2+128)] per-workgroup partials (m, l, acc)
  int* tix;            // [U] arrival counters of the fused kernel
  uint8_t* zone;       // [U*C] 1 retrieval, 2 estimation, 0 neither (debug outputs only)
  int* rank;           // [U*(K_r+K_e)] selected ids in rank order (debug outputs only)
};

// Threads per workgroup of the fused decode kernel; partials merged per unit
// by its last workgroup (at most MAX_WG workgroups per unit).
constexpr int FUSED_THREADS = 512;
constexpr int MAX_WG = 64;

// ---------------------------------------------------------------------------
// Device helpers.
__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(((uint32_t)h) << 16);
}
// Round-to-nearest-even float -> bf16 bits (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// SplitMix64 output finaliser (Steele, Lea and Flood, OOPSLA 2014).
__host__ __device__ inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}
// Counter-based draw for (seed, b, layer, h, segment, round).
__host__ __device__ inline uint64_t draw_key(uint64_t seed, uint64_t b, uint64_t l,
                                             uint64_t h, uint64_t s, uint64_t r) {
  const uint64_t G = 0x9E3779B97F4A7C15ull;
  uint64_t k = mix64(seed + G);
  k = mix64(k ^ (b + G));
  k = mix64(k ^ (l + G));
  k = mix64(k ^ (h + G));
  k = mix64(k ^ (s + G));
  return mix64(k ^ (r + G));
}
// floor((key >> 11) * m / 2^53), m < 2^63.
__device__ __forceinline__ uint64_t scale53(uint64_t key, uint64_t m) {
  uint64_t r = key >> 11;
  uint64_t lo = r * m;
  uint64_t hi = __umul64hi(r, m);
  return (hi << 11) | (lo >> 53);
}

// Order-preserving map float -> uint32 (larger float -> larger key).
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// Sum over each row of 16 lanes with DPP moves (no LDS round trip): xor-1
// and xor-2 within quads, then half-row and row mirrors. Every lane of the
// row ends with the same value (each step adds a pair in both orders, and
// addition is commutative), so results are deterministic.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
  const long long b = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_mov_dpp((int)(b & 0xFFFFFFFFll), CTRL, 0xF, 0xF, false);
  const int hi = __builtin_amdgcn_mov_dpp((int)(b >> 32), CTRL, 0xF, 0xF, false);
  return __longlong_as_double(((long long)hi << 32) | (unsigned int)lo);
}
constexpr int DPP_XOR1 = 0xB1, DPP_XOR2 = 0x4E, DPP_HALF_MIRROR = 0x141, DPP_MIRROR = 0x140;
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_f32<DPP_XOR1>(v);
  v += dpp_f32<DPP_XOR2>(v);
  v += dpp_f32<DPP_HALF_MIRROR>(v);
  v += dpp_f32<DPP_MIRROR>(v);
  return v;
}
__device__ __forceinline__ double row16_sum(double v) {
  v += dpp_f64<DPP_XOR1>(v);
  v += dpp_f64<DPP_XOR2>(v);
  v += dpp_f64<DPP_HALF_MIRROR>(v);
  v += dpp_f64<DPP_MIRROR>(v);
  return v;
}

// Wave-wide reductions (wave64).
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// ---------------------------------------------------------------------------
// Measurement hook (see wi_timing_start): no-ops unless enabled on this
// thread. Kernel name ids index a fixed table.
enum KernelId {
  K_ZERO, K_COPY, K_KPP_INIT, K_KPP_WEIGHTS, K_KPP_ROUND, K_ASSIGN, K_ASSIGN_FIX,
  K_SORT_UPDATE, K_SEG_SCAN, K_LAYOUT, K_SCORE, K_FUSED, K_RANK,
  K_EXEC, K_APPEND, K_MERGE, K_DENSE, K_DENSE_MERGE, K_RECALL, K_WB_UPDATE, K_WB_FILL, K_COUNT
};
void tmark_begin(KernelId id, hipStream_t s);
void tmark_end(hipStream_t s);

// Launch a kernel bracketed by the measurement hook.
#define WI_LAUNCH(ID, KERNEL, GRID, BLOCK, LDS, STREAM, ...)                \
  do {                                                                      \
    ::wi::tmark_begin(ID, STREAM);                                          \
    hipLaunchKernelGGL(KERNEL, GRID, BLOCK, LDS, STREAM, __VA_ARGS__);      \
    ::wi::tmark_end(STREAM);                                                \
  } while (0)

// ---------------------------------------------------------------------------
// Launchers (host functions, one per kernel family). Each returns the HIP
// status of its launches.
hipError_t launch_zero_i32(int* p, int64_t n, hipStream_t s);

hipError_t launch_kpp(const Geom& g, const void* K, void* centroids,
                      const BuildWs& ws, hipStream_t s);
hipError_t launch_copy_init(const Geom& g, const void* init, void* centroids,
                            hipStream_t s);
hipError_t launch_assign(const Geom& g, const void* K, const void* centroids,
                         const BuildWs& ws, hipStream_t s);
hipError_t launch_sort_update(const Geom& g, const void* K, void* centroids,
                              int32_t* cluster_size, const BuildWs& ws,
                              bool do_update, hipStream_t s);
hipError_t launch_layout(const Geom& g, const void* K, const void* V,
                         const wi_index_bufs& b, const BuildWs& ws,
                         hipStream_t s);

struct DecodeArgs {
  const Geom* g;
  int Hq, G, GS, K_r, K_e;  // K_e already clamped to C - K_r
  int W;                    // fused-kernel workgroups per unit (<= MAX_WG)
  float scale;
};
int score_blocks(const Geom& g);  // score-kernel workgroups per unit
hipError_t launch_score(const DecodeArgs& a, const void* centroids, const void* q,
                        const DecodeWs& ws, hipStream_t s);
// The wave buffer of one decode call: the GPU block cache and its tables,
// and the host tier's block pools as device-visible addresses.
struct WaveBufArgs {
  int n_slots;
  int32_t* block_slot;   // [U][cap]
  int32_t* slot_block;   // [U][n_slots]
  uint32_t* slot_last;   // [U][n_slots]
  int32_t* slot_order;   // [U][n_slots] slots by (last, slot id)
  void* cache_k;         // [U][n_slots * T][128]
  void* cache_v;
  const void* host_k;    // [U][cap * T][128] in host memory
  const void* host_v;
};
hipError_t launch_fused(const DecodeArgs& a, const wi_index_bufs& b, const void* q,
                        float* out, const DecodeWs& ws, bool want_lists, hipStream_t s,
                        const WaveBufArgs* wb = nullptr);
// Wave-buffer maintenance: empty tables; the per-step update from the
// retrieval zones (zone flags) and the fill of the admitted blocks.
int wb_max_slots();
hipError_t launch_wb_reset(const Geom& g, const WaveBufArgs& wb, hipStream_t s);
hipError_t launch_wb_update(const Geom& g, const WaveBufArgs& wb, const int32_t* cluster_size,
                            const int32_t* block_off, const uint8_t* zone, uint32_t step,
                            int32_t* need, int32_t* fill, int32_t* counts, int32_t* stats,
                            hipStream_t s);
hipError_t launch_append(const Geom& g, const wi_index_bufs& b, const void* k_new,
                         const void* v_new, hipStream_t s);
// n_new tokens at once ([U][n_new][128] rows); stage holds 2 x U x n_local rows.
hipError_t launch_append_many(const Geom& g, const wi_index_bufs& b, const void* k_new,
                              const void* v_new, int n_new, void* stage, hipStream_t s);
// The grown index nw (geometry gn) from the old index o (geometry go) and the
// new segment sg clustered as a one-segment index (geometry gs).
hipError_t launch_extend_merge(const Geom& go, const Geom& gn, const Geom& gs,
                               const wi_index_bufs& o, const wi_index_bufs& sg,
                               const wi_index_bufs& nw, hipStream_t s);
// Dense decode attention (full-attention layers): chunks per unit, partial
// buffer size in floats, and the two launches.
int dense_chunks(int U, int64_t N);
int64_t dense_part_floats(int U, int W, int G);
hipError_t launch_dense(int dtype, int B, int H, int Hq, int G, int64_t N, int64_t sb,
                        int64_t sh, int64_t st, float scale, const void* k, const void* v,
                        const void* q, float* out, float* part, hipStream_t s);
// recall@k: largest k served; keys is [U][G][cap*T] uint64 scratch.
int recall_max_k();
hipError_t launch_recall(const Geom& g, int Hq, int G, const wi_index_bufs& bf, const void* q,
                         const int32_t* sel, int sel_stride, int n_r, int k, float* recall,
                         int32_t* top, uint64_t* keys, hipStream_t s);
hipError_t launch_debug_outputs(const DecodeArgs& a, const wi_index_bufs& b,
                                const DecodeWs& ws, int32_t* sel_ids,
                                int32_t* exec_tokens, int32_t* n_exec,
                                int64_t exec_cap, hipStream_t s);

}  // namespace wi
