// Decode steps 3-6: gather the execution buffer, exact attention over the
// steady and retrieval zones, the estimation-zone partial, and the
// log-sum-exp merge (RetroInfer, framerc blog section 3.2: execution buffer
// = steady zone + retrieved blocks with block fragments skipped; section
// 3.3: hybrid attention, estimation from centroid vectors and cluster sizes,
// partial results merged by a custom kernel; techwalker article section 3).
//
// Work split: for each unit the execution buffer (n_st steady tokens, then
// the members of every retrieval cluster) and the estimation list are cut
// into P equal chunks, one workgroup each. Inside a workgroup the chunk is
// cut again into 16 contiguous streams, one per 16-lane group; a group reads
// a 256-byte key/value row per step (8 dims per lane, 128-bit loads), so the
// gather never touches the padding slots of a block. Each stream keeps an
// online softmax (running max m, denominator l, numerator acc) per query
// head; streams are merged in a fixed order, first across the four groups
// of a wave, then across the four waves, and the chunk partial is written
// out. The combine kernel merges the P partials of each query head:
//   m = max_p m_p,  out = sum_p e^{m_p - m} acc_p / sum_p e^{m_p - m} l_p.
// An estimation cluster c enters a stream as one item with logit s_c (from
// the score step), multiplicity n_c and value sum VS_c: l += n_c e^{s_c - m},
// acc += e^{s_c - m} VS_c.
#include "wi_internal.h"

namespace wi {
namespace {

constexpr int ATT_THREADS = 256;
constexpr int STREAMS = ATT_THREADS / 16;
constexpr int PART = 2 + D;  // m, l, acc[128]

template <int DT>
__device__ __forceinline__ void load8(const void* base, int64_t row, int j, float x[8]) {
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

__device__ __forceinline__ void load8f(const float* base, int64_t row, int j, float x[8]) {
  const float4* p = reinterpret_cast<const float4*>(base + row * D + 8 * j);
  const float4 a = p[0], b = p[1];
  x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
  x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}

template <int DT>
__device__ __forceinline__ float ex(float x) {
  if constexpr (DT == WI_BF16) return __expf(x);
  else return expf(x);
}

template <int DT, int GM>
__global__ __launch_bounds__(ATT_THREADS) void attend_kernel(
    const void* __restrict__ kblk, const void* __restrict__ vblk,
    const void* __restrict__ stk, const void* __restrict__ stv,
    const int32_t* __restrict__ block_off, const int32_t* __restrict__ sizes,
    const float* __restrict__ vsum, const float* __restrict__ S,
    const int* __restrict__ Rl, const int* __restrict__ El, const int* __restrict__ Rpre,
    const void* __restrict__ q, int C, int64_t capT, int T, int n_st, int G, int H,
    int Hq, int K_r, int K_e, int P, float scale, float* __restrict__ part) {
  const int p = blockIdx.x, u = blockIdx.y;
  const int b = u / H, h = u % H;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int grp = tid >> 4, j = tid & 15;

  const int* R = Rl + (int64_t)u * K_r;
  const int* E = El + (int64_t)u * K_e;
  const int* pre = Rpre + (int64_t)u * (K_r + 1);
  const int32_t* bo = block_off + (int64_t)u * (C + 1);
  const int32_t* sz = sizes + (int64_t)u * C;

  // chunk p of the execution buffer and of the estimation list
  const int64_t NX = (int64_t)n_st + pre[K_r];
  const int64_t x0 = NX * p / P, x1 = NX * (p + 1) / P;
  const int64_t e0 = (int64_t)K_e * p / P, e1 = (int64_t)K_e * (p + 1) / P;
  const int64_t nx = x1 - x0, nitems = nx + (e1 - e0);
  const int64_t i0 = nitems * grp / STREAMS, i1 = nitems * (grp + 1) / STREAMS;

  float qv[GM][8];
#pragma unroll
  for (int g = 0; g < GM; g++) {
    if (g < G) {
      load8<DT>(q, (int64_t)b * Hq + (int64_t)h * G + g, j, qv[g]);
#pragma unroll
      for (int t = 0; t < 8; t++) qv[g][t] *= scale;
    } else {
#pragma unroll
      for (int t = 0; t < 8; t++) qv[g][t] = 0.f;
    }
  }
  float m[GM], l[GM], acc[GM][8];
#pragma unroll
  for (int g = 0; g < GM; g++) {
    m[g] = -INFINITY;
    l[g] = 0.f;
#pragma unroll
    for (int t = 0; t < 8; t++) acc[g][t] = 0.f;
  }

  // ---- exact part: execution-buffer tokens [x0 + i0, x0 + min(i1, nx)) ----
  const int64_t xa = x0 + i0, xb = x0 + (i1 < nx ? i1 : nx);
  if (xa < xb) {
    // cursor into R for flat index f >= n_st: pre[r] <= f - n_st < pre[r+1]
    int r = 0;
    if (xa >= n_st) {
      int lo = 0, hi = K_r - 1;
      const int t = (int)(xa - n_st);
      while (lo < hi) {  // last r with pre[r] <= t
        const int mid = (lo + hi + 1) >> 1;
        if (pre[mid] <= t) lo = mid; else hi = mid - 1;
      }
      r = lo;
    }
    const uint16_t* dummy = nullptr;
    (void)dummy;
    for (int64_t f = xa; f < xb; f++) {
      const void* kb;
      const void* vb;
      int64_t row;
      if (f < n_st) {
        kb = stk;
        vb = stv;
        row = (int64_t)u * n_st + f;
      } else {
        const int t = (int)(f - n_st);
        while (pre[r + 1] <= t) r++;
        const int c = R[r];
        row = (int64_t)u * capT + (int64_t)bo[c] * T + (t - pre[r]);
        kb = kblk;
        vb = vblk;
      }
      float kx[8], vx[8];
      load8<DT>(kb, row, j, kx);
      load8<DT>(vb, row, j, vx);
#pragma unroll
      for (int g = 0; g < GM; g++) {
        if (g < G) {
          float z = 0.f;
#pragma unroll
          for (int t = 0; t < 8; t++) z = fmaf(qv[g][t], kx[t], z);
          z += __shfl_xor(z, 8, 16);
          z += __shfl_xor(z, 4, 16);
          z += __shfl_xor(z, 2, 16);
          z += __shfl_xor(z, 1, 16);
          const float mn = fmaxf(m[g], z);
          const float al = ex<DT>(m[g] - mn);
          const float pz = ex<DT>(z - mn);
          m[g] = mn;
          l[g] = fmaf(l[g], al, pz);
#pragma unroll
          for (int t = 0; t < 8; t++) acc[g][t] = fmaf(acc[g][t], al, pz * vx[t]);
        }
      }
    }
  }

  // ---- estimation part: E entries [e0 + max(i0 - nx, 0), e0 + i1 - nx) ----
  const int64_t ea = e0 + (i0 > nx ? i0 - nx : 0), eb = e0 + (i1 > nx ? i1 - nx : 0);
  for (int64_t e = ea; e < eb; e++) {
    const int c = E[e];
    const int n = sz[c];
    if (n == 0) continue;
    float vx[8];
    load8f(vsum, (int64_t)u * C + c, j, vx);
    const float nf = (float)n;
    const float* sc = S + ((int64_t)u * C + c) * G;
#pragma unroll
    for (int g = 0; g < GM; g++) {
      if (g < G) {
        const float z = sc[g];
        const float mn = fmaxf(m[g], z);
        const float al = ex<DT>(m[g] - mn);
        const float pz = ex<DT>(z - mn);
        m[g] = mn;
        l[g] = fmaf(l[g], al, nf * pz);
#pragma unroll
        for (int t = 0; t < 8; t++) acc[g][t] = fmaf(acc[g][t], al, pz * vx[t]);
      }
    }
  }

  // ---- merge the four groups of each wave (fixed butterfly order) ----
#pragma unroll
  for (int g = 0; g < GM; g++) {
    if (g < G) {
      float mw = fmaxf(m[g], __shfl_xor(m[g], 16, 64));
      mw = fmaxf(mw, __shfl_xor(mw, 32, 64));
      const float f = (m[g] == -INFINITY) ? 0.f : ex<DT>(m[g] - mw);
      l[g] *= f;
#pragma unroll
      for (int t = 0; t < 8; t++) acc[g][t] *= f;
      l[g] += __shfl_xor(l[g], 16, 64);
      l[g] += __shfl_xor(l[g], 32, 64);
#pragma unroll
      for (int t = 0; t < 8; t++) {
        acc[g][t] += __shfl_xor(acc[g][t], 16, 64);
        acc[g][t] += __shfl_xor(acc[g][t], 32, 64);
      }
      m[g] = mw;
    }
  }

  // ---- merge the four waves through LDS ----
  __shared__ float sm[4][GM], sl[4][GM];
  __shared__ float sacc[4][GM][D];
  if (lane < 16) {
#pragma unroll
    for (int g = 0; g < GM; g++) {
      if (g < G) {
        if (lane == 0) {
          sm[wv][g] = m[g];
          sl[wv][g] = l[g];
        }
#pragma unroll
        for (int t = 0; t < 8; t++) sacc[wv][g][8 * j + t] = acc[g][t];
      }
    }
  }
  __syncthreads();
  float* out = part + ((int64_t)u * P + p) * G * PART;
  for (int e = tid; e < G * D; e += ATT_THREADS) {
    const int g = e / D, t = e % D;
    float mm = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; w++) mm = fmaxf(mm, sm[w][g]);
    float a = 0.f, ll = 0.f;
#pragma unroll
    for (int w = 0; w < 4; w++) {
      const float f = (sm[w][g] == -INFINITY) ? 0.f : ex<DT>(sm[w][g] - mm);
      a = fmaf(sacc[w][g][t], f, a);
      ll = fmaf(sl[w][g], f, ll);
    }
    out[g * PART + 2 + t] = a;
    if (t == 0) {
      out[g * PART] = mm;
      out[g * PART + 1] = ll;
    }
  }
}

template <int DT>
__global__ __launch_bounds__(D) void combine_kernel(const float* __restrict__ part, int G,
                                                    int H, int Hq, int P,
                                                    float* __restrict__ out) {
  const int u = blockIdx.x / G, g = blockIdx.x % G;
  const int b = u / H, h = u % H;
  const int t = threadIdx.x;
  const float* pp = part + (int64_t)u * P * G * PART + (int64_t)g * PART;
  float mm = -INFINITY;
  for (int c = 0; c < P; c++) mm = fmaxf(mm, pp[(int64_t)c * G * PART]);
  float num = 0.f, den = 0.f;
  for (int c = 0; c < P; c++) {
    const float* q = pp + (int64_t)c * G * PART;
    const float f = (q[0] == -INFINITY) ? 0.f : ex<DT>(q[0] - mm);
    num = fmaf(q[2 + t], f, num);
    den = fmaf(q[1], f, den);
  }
  out[((int64_t)b * Hq + (int64_t)h * G + g) * D + t] = num / den;
}

template <int DT>
hipError_t launch_attend_dt(const DecodeArgs& a, const wi_index_bufs& bf, const void* q,
                            float* out, const DecodeWs& ws, hipStream_t s) {
  const Geom& g = *a.g;
  dim3 grid(a.P, g.U);
  const int64_t capT = g.cap * g.T;
#define WI_ATT(GMV)                                                                        \
  WI_LAUNCH(K_ATTEND, (attend_kernel<DT, GMV>), grid, dim3(ATT_THREADS), 0, s, bf.k_blocks, \
                     bf.v_blocks, bf.steady_k, bf.steady_v, bf.block_off, bf.cluster_size, \
                     bf.value_sum, ws.S, ws.R, ws.E, ws.Rpre, q, g.C, capT, g.T, g.n_st,   \
                     a.G, g.H, a.Hq, a.K_r, a.K_e, a.P, a.scale, ws.part)
  if (a.G <= 4) WI_ATT(4);
  else if (a.G <= 8) WI_ATT(8);
  else WI_ATT(16);
#undef WI_ATT
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  WI_LAUNCH(K_COMBINE, (combine_kernel<DT>), dim3(g.U * a.G), dim3(D), 0, s, ws.part, a.G,
                     g.H, a.Hq, a.P, out);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attend(const DecodeArgs& a, const wi_index_bufs& b, const void* q,
                         float* out, const DecodeWs& ws, hipStream_t s) {
  return a.g->dtype == WI_BF16 ? launch_attend_dt<WI_BF16>(a, b, q, out, ws, s)
                               : launch_attend_dt<WI_F32>(a, b, q, out, ws, s);
}

}  // namespace wi
