// Decode step 1: score every centroid of a unit against the unit's query
// heads (RetroInfer, framerc blog section 2.2, sync access path step 1:
// query the wave index for the key cluster ids; section 3.3: estimation from
// centroid vectors).
//
// Memory-bound: each centroid row (128 x dtype) is read once from HBM. A
// group of 16 lanes owns one row, each lane 8 consecutive dims loaded with a
// single 128-bit (bf16) or 2x128-bit (fp32) load, so a wave64 streams four
// 256-byte rows per load instruction. The per-head dot products are reduced
// across the 16 lanes with a fixed butterfly, so results are deterministic.
//
// Outputs per cluster c:  S[c][h] = scale * <q_h, mu_c>  (fp32, per head; rows
//                                    padded to GM = 4, 8 or 16 heads)
//                         key[c]  = order-preserving bits of sum_h <q_h, mu_c>
#include "wi_internal.h"

namespace wi {
namespace {

constexpr int SCORE_THREADS = 256;
constexpr int GROUPS = SCORE_THREADS / 16;  // rows in flight per step

template <int DT>
__device__ __forceinline__ void load_row8(const void* base, int64_t row, int j, float x[8]) {
  if constexpr (DT == WI_BF16) {
    const uint4 v = *reinterpret_cast<const uint4*>(
        reinterpret_cast<const uint16_t*>(base) + row * D + 8 * j);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int t = 0; t < 4; t++) {
      x[2 * t] = __uint_as_float(w[t] << 16);
      x[2 * t + 1] = __uint_as_float(w[t] & 0xFFFF0000u);
    }
  } else {
    const float4* p = reinterpret_cast<const float4*>(
        reinterpret_cast<const float*>(base) + row * D + 8 * j);
    const float4 a = p[0], b = p[1];
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
  }
}

// Per-head dot products are accumulated in float64: bf16 x bf16 (and fp32 x
// fp32) products are exact in float64 and on gfx950 a float64 FMA issues at
// the float32 rate, so the group score is exact up to the final rounding to
// float32 that the ranking is taken in.
//
// Latency: the whole score pass moves a few tens of MB, so every lane issues
// all of its row loads (ROWS per 16-lane group, one 16-byte load each) before
// any arithmetic; a workgroup covers GROUPS * ROWS rows.
constexpr int ROWS = 4;

template <int DT>
__device__ __forceinline__ void raw_row(const void* base, int64_t row, int j, uint4 r[2]) {
  if constexpr (DT == WI_BF16) {
    r[0] = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(base) + row * D + 8 * j);
  } else {
    const uint4* p = reinterpret_cast<const uint4*>(reinterpret_cast<const float*>(base) + row * D + 8 * j);
    r[0] = p[0];
    r[1] = p[1];
  }
}

template <int DT>
__device__ __forceinline__ void unpack8(const uint4 r[2], double xd[8]) {
  if constexpr (DT == WI_BF16) {
    const uint32_t w[4] = {r[0].x, r[0].y, r[0].z, r[0].w};
#pragma unroll
    for (int t = 0; t < 4; t++) {
      xd[2 * t] = (double)__uint_as_float(w[t] << 16);
      xd[2 * t + 1] = (double)__uint_as_float(w[t] & 0xFFFF0000u);
    }
  } else {
    const uint32_t w[8] = {r[0].x, r[0].y, r[0].z, r[0].w, r[1].x, r[1].y, r[1].z, r[1].w};
#pragma unroll
    for (int t = 0; t < 8; t++) xd[t] = (double)__uint_as_float(w[t]);
  }
}

template <int DT, int GM>
__global__ __launch_bounds__(SCORE_THREADS) void score_kernel(
    const void* __restrict__ cent, const void* __restrict__ q, int C, int G, int H,
    int Hq, float scale, uint32_t* __restrict__ key, float* __restrict__ S) {
  const int u = blockIdx.y;
  const int b = u / H, h = u % H;
  const int tid = threadIdx.x;
  const int grp = tid >> 4, j = tid & 15;
  const int c0 = blockIdx.x * (GROUPS * ROWS);
  const int64_t rowbase = (int64_t)u * C;

  // issue the row loads first
  uint4 raw[ROWS][2];
#pragma unroll
  for (int r = 0; r < ROWS; r++) {
    const int c = c0 + r * GROUPS + grp;
    if (c < C) raw_row<DT>(cent, rowbase + c, j, raw[r]);
  }
  // branch-free query loads (heads past G read head G-1 and are ignored)
  float qf[GM][8];
#pragma unroll
  for (int g = 0; g < GM; g++)
    load_row8<DT>(q, (int64_t)b * Hq + (int64_t)h * G + min(g, G - 1), j, qf[g]);
#pragma unroll
  for (int r = 0; r < ROWS; r++) {
    const int c = c0 + r * GROUPS + grp;
    if (c >= C) break;
    double xd[8];
    unpack8<DT>(raw[r], xd);
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
    if (j < G) S[(rowbase + c) * GM + j] = (float)(mine * (double)scale);
    if (j == 0) key[rowbase + c] = order_key((float)tot);
  }
}

template <int DT>
hipError_t launch_score_dt(const DecodeArgs& a, const void* cent, const void* q,
                           const DecodeWs& ws, hipStream_t s) {
  const Geom& g = *a.g;
  dim3 grid((g.C + GROUPS * ROWS - 1) / (GROUPS * ROWS), g.U);
  if (a.G <= 4)
    WI_LAUNCH(K_SCORE, (score_kernel<DT, 4>), grid, dim3(SCORE_THREADS), 0, s, cent, q,
              g.C, a.G, g.H, a.Hq, a.scale, ws.key, ws.S);
  else if (a.G <= 8)
    WI_LAUNCH(K_SCORE, (score_kernel<DT, 8>), grid, dim3(SCORE_THREADS), 0, s, cent, q,
              g.C, a.G, g.H, a.Hq, a.scale, ws.key, ws.S);
  else
    WI_LAUNCH(K_SCORE, (score_kernel<DT, 16>), grid, dim3(SCORE_THREADS), 0, s, cent, q,
              g.C, a.G, g.H, a.Hq, a.scale, ws.key, ws.S);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_score(const DecodeArgs& a, const void* cent, const void* q,
                        const DecodeWs& ws, hipStream_t s) {
  return a.g->dtype == WI_BF16 ? launch_score_dt<WI_BF16>(a, cent, q, ws, s)
                               : launch_score_dt<WI_F32>(a, cent, q, ws, s);
}

}  // namespace wi
