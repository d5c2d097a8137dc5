// Decode step 1: score every centroid of a unit against the unit's query
// heads (RetroInfer, framerc blog section 2.2, sync access path step 1:
// query the wave index for the key cluster ids; section 3.3: estimation from
// centroid vectors).
//
// Outputs per cluster c of unit u:
//   key[u][c]   order-preserving bits of g_c = sum_h <q_h, mu_c> rounded to
//               float32 once (the ranking key);
//   S[u][c][h]  scale * <q_h, mu_c> per query head h of the group (float32,
//               rows padded to GS = 4, 8 or 16 heads) -- the estimation-zone
//               logits.
// Both are read back by the fused select/attend kernel. The launch also
// clears the per-unit arrival counters that kernel uses.
//
// bf16 (the hot path): HBM-bound streaming of C x 256-byte rows. A wave
// walks 16-row tiles of its unit (tile w, w + stride, ...), issuing the loads
// of the next tile before computing the current one, so every wave keeps
// loads in flight. Lane i loads row (i % 16) of a tile in 16-byte pieces at
// dims 32 s + 8 (i / 16), s = 0..3: each load instruction reads 64
// contiguous bytes of 16 rows. The same registers feed
//   - the per-head logits: four v_mfma_f32_16x16x32_bf16 per tile with the
//     query heads as the 16 columns of the B operand (fp32 accumulation of
//     exact bf16 products);
//   - the ranking key: sum_t Q_t mu_t in float64 with Q = sum_h q_h formed
//     once per workgroup in float64 and kept in LDS (sums and products of
//     bf16 values are exact there, so the key is the exactly rounded group
//     score), one FMA per element in a fixed order, then a fixed two-step
//     exchange across the four lanes that share a row.
// fp32 (parity-size workloads only): 16 lanes per row, per-head float64 dot
// products reduced across the row with a fixed butterfly.
#include "wi_internal.h"

namespace wi {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int SCORE_THREADS = 256;

__device__ __forceinline__ void clear_counters(int* p, int n) {
  if (blockIdx.x == 0 && blockIdx.y == 0)
    for (int i = threadIdx.x; i < n; i += blockDim.x) p[i] = 0;
}

// The key range of the workgroup -> mm[u][block] (the select step's
// histogram bounds). Reached by every thread.
__device__ __forceinline__ void publish_range(float lo, float hi, float2* wmm, float2* out) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    lo = fminf(lo, __shfl_xor(lo, o, 64));
    hi = fmaxf(hi, __shfl_xor(hi, o, 64));
  }
  if ((threadIdx.x & 63) == 0) wmm[threadIdx.x >> 6] = make_float2(lo, hi);
  __syncthreads();
  if (threadIdx.x == 0) {
    float2 r = wmm[0];
    for (int i = 1; i < (int)(blockDim.x >> 6); i++) {
      r.x = fminf(r.x, wmm[i].x);
      r.y = fmaxf(r.y, wmm[i].y);
    }
    *out = r;
  }
}

template <int GS>
__global__ __launch_bounds__(SCORE_THREADS) void score_bf16_kernel(
    const uint16_t* __restrict__ cent, const uint16_t* __restrict__ q, int C, int Cp, int G,
    int H, int Hq, float scale, uint32_t* __restrict__ key, float* __restrict__ S,
    float2* __restrict__ mm, int* __restrict__ counters, int n_counters) {
  clear_counters(counters, n_counters);
  __shared__ __align__(16) double Qs[D];
  __shared__ float2 wmm[SCORE_THREADS / 64];
  const int u = blockIdx.y;
  const int b = u / H, h = u % H;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int r16 = lane & 15, kg = lane >> 4;
  const int ntiles = (C + 15) / 16;
  const int stride = gridDim.x * (SCORE_THREADS / 64);
  const int64_t ubase = (int64_t)u * C;
  const uint16_t* qb = q + ((int64_t)b * Hq + (int64_t)h * G) * D;

  // loads of one tile (row index clamped into the unit; rows past C are read
  // again and never written)
  auto load_tile = [&](int tile, uint4* a) {
    const int row = min(tile * 16 + r16, C - 1);
    const uint16_t* rp = cent + (ubase + row) * D + 8 * kg;
#pragma unroll
    for (int s = 0; s < 4; s++) a[s] = *reinterpret_cast<const uint4*>(rp + 32 * s);
  };
  int tile = blockIdx.x * (SCORE_THREADS / 64) + wv;
  uint4 a0[4], a1[4];
  if (tile < ntiles) load_tile(tile, a0);
  // query heads of the group: B operand (column r16 = head r16), and
  // Q_t = sum_h q_{h,t} in float64 for dim t = tid
  uint4 bq[4];
#pragma unroll
  for (int s = 0; s < 4; s++) {
    const uint4 v = *reinterpret_cast<const uint4*>(qb + (int64_t)min(r16, G - 1) * D + 8 * kg + 32 * s);
    bq[s] = r16 < G ? v : make_uint4(0u, 0u, 0u, 0u);
  }
  if (tid < D) {
    uint16_t qv[GS];
#pragma unroll
    for (int g = 0; g < GS; g++) qv[g] = qb[(int64_t)min(g, G - 1) * D + tid];
    double Q = 0.0;
#pragma unroll
    for (int g = 0; g < GS; g++) Q += g < G ? (double)bf16_to_f32(qv[g]) : 0.0;
    Qs[tid] = Q;
  }
  __syncthreads();

  float lo = INFINITY, hi = -INFINITY;  // range of this lane's keys
  auto compute_tile = [&](int tl, const uint4* a) {
    // Q is re-read from LDS per tile (a compiler fence keeps the 32 doubles
    // from being held in registers across the loop)
    asm volatile("" ::: "memory");
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    double p = 0.0;
#pragma unroll
    for (int s = 0; s < 4; s++) {
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a[s]),
                                                    __builtin_bit_cast(bf16x8_t, bq[s]), acc,
                                                    0, 0, 0);
      const double2* qp = reinterpret_cast<const double2*>(Qs + 32 * s + 8 * kg);
      const uint32_t w[4] = {a[s].x, a[s].y, a[s].z, a[s].w};
#pragma unroll
      for (int e = 0; e < 4; e++) {
        const double2 Qe = qp[e];
        p = __builtin_fma(Qe.x, (double)__uint_as_float(w[e] << 16), p);
        p = __builtin_fma(Qe.y, (double)__uint_as_float(w[e] & 0xFFFF0000u), p);
      }
    }
    // lanes r16, r16+16, r16+32, r16+48 hold the four 32-dim pieces of row r16
    p += __shfl_xor(p, 16, 64);
    p += __shfl_xor(p, 32, 64);
    const int row = tl * 16 + r16;
    const float pf = (float)p;
    if (row < C) {
      lo = fminf(lo, pf);
      hi = fmaxf(hi, pf);
    }
    if (kg == 0 && row < C) key[(int64_t)u * Cp + row] = order_key(pf);
    // D layout: lane holds rows 4 kg + j (j = 0..3) of the tile, column r16
    if (r16 < G) {
#pragma unroll
      for (int j = 0; j < 4; j++) {
        const int rj = tl * 16 + 4 * kg + j;
        if (rj < C) S[(ubase + rj) * GS + r16] = acc[j] * scale;
      }
    }
  };

  // two register buffers, alternating; the next tile's loads are issued
  // before the current tile is computed
#pragma unroll 1
  while (tile < ntiles) {
    const int t1 = tile + stride;
    if (t1 < ntiles) load_tile(t1, a1);
    compute_tile(tile, a0);
    if (t1 >= ntiles) break;
    const int t2 = t1 + stride;
    if (t2 < ntiles) load_tile(t2, a0);
    compute_tile(t1, a1);
    tile = t2;
  }
  publish_range(lo, hi, wmm, mm + (int64_t)u * gridDim.x + blockIdx.x);
}

// fp32 centroids: 16 lanes per row, per-head float64 dots.
constexpr int GROUPS = SCORE_THREADS / 16;
constexpr int ROWS = 4;

template <int GM>
__global__ __launch_bounds__(SCORE_THREADS) void score_f32_kernel(
    const float* __restrict__ cent, const float* __restrict__ q,
    int C, int Cp, int G, int H, int Hq, float scale, uint32_t* __restrict__ key,
    float* __restrict__ S, float2* __restrict__ mm, int* __restrict__ counters, int n_counters) {
  clear_counters(counters, n_counters);
  __shared__ float2 wmm[SCORE_THREADS / 64];
  const int u = blockIdx.y;
  const int b = u / H, h = u % H;
  const int tid = threadIdx.x;
  float lo = INFINITY, hi = -INFINITY;
  const int grp = tid >> 4, j = tid & 15;
  const int c0 = blockIdx.x * (GROUPS * ROWS);
  const int64_t rowbase = (int64_t)u * C;

  float4 raw[ROWS][2];
#pragma unroll
  for (int r = 0; r < ROWS; r++) {
    const int c = min(c0 + r * GROUPS + grp, C - 1);
    const float4* p = reinterpret_cast<const float4*>(cent + (rowbase + c) * D + 8 * j);
    raw[r][0] = p[0];
    raw[r][1] = p[1];
  }
  float qf[GM][8];
#pragma unroll
  for (int g = 0; g < GM; g++) {
    const float4* p = reinterpret_cast<const float4*>(
        q + ((int64_t)b * Hq + (int64_t)h * G + min(g, G - 1)) * D + 8 * j);
    const float4 x = p[0], y = p[1];
    qf[g][0] = x.x; qf[g][1] = x.y; qf[g][2] = x.z; qf[g][3] = x.w;
    qf[g][4] = y.x; qf[g][5] = y.y; qf[g][6] = y.z; qf[g][7] = y.w;
  }
#pragma unroll
  for (int r = 0; r < ROWS; r++) {
    const int c = c0 + r * GROUPS + grp;
    const double xd[8] = {raw[r][0].x, raw[r][0].y, raw[r][0].z, raw[r][0].w,
                          raw[r][1].x, raw[r][1].y, raw[r][1].z, raw[r][1].w};
    double tot = 0.0, mine = 0.0;
#pragma unroll
    for (int g = 0; g < GM; g++) {
      if (g < G) {
        double p = 0.0;
#pragma unroll
        for (int t = 0; t < 8; t++) p = __builtin_fma((double)qf[g][t], xd[t], p);
        p = row16_sum(p);
        tot += p;
        if (j == g) mine = p;
      }
    }
    if (c < C) {
      if (j < G) S[(rowbase + c) * GM + j] = (float)(mine * (double)scale);
      if (j == 0) key[(int64_t)u * Cp + c] = order_key((float)tot);
      lo = fminf(lo, (float)tot);
      hi = fmaxf(hi, (float)tot);
    }
  }
  publish_range(lo, hi, wmm, mm + (int64_t)u * gridDim.x + blockIdx.x);
}

}  // namespace

int score_blocks(const Geom& g) {
  if (g.dtype == WI_BF16) {
    // one wave per tile when the call is small; otherwise about 4096 waves
    // over the call, each walking several tiles of its unit
    const int tiles = (g.C + 15) / 16;
    int waves = (4096 + g.U - 1) / g.U;
    if (waves < 4) waves = 4;
    if (waves > tiles) waves = tiles;
    const int wpg = SCORE_THREADS / 64;
    return (waves + wpg - 1) / wpg;
  }
  return (g.C + GROUPS * ROWS - 1) / (GROUPS * ROWS);
}

hipError_t launch_score(const DecodeArgs& a, const void* cent, const void* q,
                        const DecodeWs& ws, hipStream_t s) {
  const Geom& g = *a.g;
  dim3 grid(score_blocks(g), g.U);
  if (g.dtype == WI_BF16) {
    const uint16_t* c16 = reinterpret_cast<const uint16_t*>(cent);
    const uint16_t* q16 = reinterpret_cast<const uint16_t*>(q);
#define WI_SC(GSV)                                                                          \
  WI_LAUNCH(K_SCORE, (score_bf16_kernel<GSV>), grid, dim3(SCORE_THREADS), 0, s, c16, q16,   \
            g.C, (g.C + 3) & ~3, a.G, g.H, a.Hq, a.scale, ws.key, ws.S, ws.mm, ws.tix, g.U)
    if (a.GS == 4) WI_SC(4);
    else if (a.GS == 8) WI_SC(8);
    else WI_SC(16);
#undef WI_SC
  } else {
    const float* c32 = reinterpret_cast<const float*>(cent);
    const float* q32 = reinterpret_cast<const float*>(q);
#define WI_SC(GSV)                                                                          \
  WI_LAUNCH(K_SCORE, (score_f32_kernel<GSV>), grid, dim3(SCORE_THREADS), 0, s, c32, q32,    \
            g.C, (g.C + 3) & ~3, a.G, g.H, a.Hq, a.scale, ws.key, ws.S, ws.mm, ws.tix, g.U)
    if (a.GS == 4) WI_SC(4);
    else if (a.GS == 8) WI_SC(8);
    else WI_SC(16);
#undef WI_SC
  }
  return hipGetLastError();
}

}  // namespace wi
