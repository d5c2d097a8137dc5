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
// Outputs per cluster c:  S[c][h] = scale * <q_h, mu_c>  (fp32, per head)
//                         key[c]  = order-preserving bits of sum_h <q_h, mu_c>
#include "wi_internal.h"

namespace wi {
namespace {

constexpr int SCORE_THREADS = 256;
constexpr int GROUPS = SCORE_THREADS / 16;  // rows in flight per step
constexpr int UNROLL = 4;                   // rows per group per step

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
template <int DT, int GM>
__global__ __launch_bounds__(SCORE_THREADS) void score_kernel(
    const void* __restrict__ cent, const void* __restrict__ q, int C, int G, int H,
    int Hq, int cpb, float scale, uint32_t* __restrict__ key, float* __restrict__ S) {
  const int u = blockIdx.y;
  const int b = u / H, h = u % H;
  const int tid = threadIdx.x;
  const int grp = tid >> 4, j = tid & 15;

  double qv[GM][8];
#pragma unroll
  for (int g = 0; g < GM; g++) {
    float t8[8];
    if (g < G) {
      load_row8<DT>(q, (int64_t)b * Hq + (int64_t)h * G + g, j, t8);
    } else {
#pragma unroll
      for (int t = 0; t < 8; t++) t8[t] = 0.f;
    }
#pragma unroll
    for (int t = 0; t < 8; t++) qv[g][t] = (double)t8[t];
  }

  const int c0 = blockIdx.x * cpb;
  const int c1 = min(C, c0 + cpb);
  const int64_t rowbase = (int64_t)u * C;
  for (int cb = c0 + grp; cb < c1; cb += GROUPS * UNROLL) {
    float x[UNROLL][8];
#pragma unroll
    for (int r = 0; r < UNROLL; r++) {
      const int c = cb + r * GROUPS;
      if (c < c1) load_row8<DT>(cent, rowbase + c, j, x[r]);
    }
#pragma unroll
    for (int r = 0; r < UNROLL; r++) {
      const int c = cb + r * GROUPS;
      if (c >= c1) break;
      double xd[8];
#pragma unroll
      for (int t = 0; t < 8; t++) xd[t] = (double)x[r][t];
      double tot = 0.0, mine = 0.0;
#pragma unroll
      for (int g = 0; g < GM; g++) {
        if (g < G) {
          double p = 0.0;
#pragma unroll
          for (int t = 0; t < 8; t++) p = __builtin_fma(qv[g][t], xd[t], p);
          p += __shfl_xor(p, 8, 16);
          p += __shfl_xor(p, 4, 16);
          p += __shfl_xor(p, 2, 16);
          p += __shfl_xor(p, 1, 16);
          tot += p;
          if (j == g) mine = p;
        }
      }
      if (j < G) S[(rowbase + c) * G + j] = (float)(mine * (double)scale);
      if (j == 0) key[rowbase + c] = order_key((float)tot);
    }
  }
}

template <int DT>
hipError_t launch_score_dt(const DecodeArgs& a, const void* cent, const void* q,
                           const DecodeWs& ws, hipStream_t s) {
  const Geom& g = *a.g;
  const int cpb = 256;
  dim3 grid((g.C + cpb - 1) / cpb, g.U);
  if (a.G <= 4)
    WI_LAUNCH(K_SCORE, (score_kernel<DT, 4>), grid, dim3(SCORE_THREADS), 0, s, cent, q,
                       g.C, a.G, g.H, a.Hq, cpb, a.scale, ws.key, ws.S);
  else if (a.G <= 8)
    WI_LAUNCH(K_SCORE, (score_kernel<DT, 8>), grid, dim3(SCORE_THREADS), 0, s, cent, q,
                       g.C, a.G, g.H, a.Hq, cpb, a.scale, ws.key, ws.S);
  else
    WI_LAUNCH(K_SCORE, (score_kernel<DT, 16>), grid, dim3(SCORE_THREADS), 0, s, cent, q,
                       g.C, a.G, g.H, a.Hq, cpb, a.scale, ws.key, ws.S);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_score(const DecodeArgs& a, const void* cent, const void* q,
                        const DecodeWs& ws, hipStream_t s) {
  return a.g->dtype == WI_BF16 ? launch_score_dt<WI_BF16>(a, cent, q, ws, s)
                               : launch_score_dt<WI_F32>(a, cent, q, ws, s);
}

}  // namespace wi
