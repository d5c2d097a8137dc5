// Decode steps 3-6: gather the execution buffer, exact attention over the
// steady and retrieval zones, the estimation-zone partial, and the
// log-sum-exp merge (RetroInfer, framerc blog section 3.2: execution buffer
// = steady zone + retrieved blocks with block fragments skipped; section
// 3.3: hybrid attention, estimation from centroid vectors and cluster sizes,
// partial results merged by a custom kernel; techwalker article section 3).
//
// Work split: the execution buffer of a unit (n_st steady tokens, then the
// members of every retrieval cluster, located through the row table the
// select step wrote) and its estimation list are cut into P equal chunks, one
// workgroup each; a chunk is cut again into 16 contiguous streams, one per
// 16-lane group. A group reads one 256-byte (bf16) key/value row per item,
// 8 dims per lane with 128-bit loads, so only valid slots of a block are
// read. A stream first issues the loads of up to IPS items, then computes
// their logits, takes the running maximum once per batch and accumulates
// (m, l, acc) per query head. Streams merge in a fixed order (groups of a
// wave by butterfly, waves through LDS) into the chunk partial.
//
// An estimation cluster c enters as one item with logit s_c (score step),
// multiplicity n_c and value sum VS_c: l += n_c e^{s_c - m},
// acc += e^{s_c - m} VS_c.
//
// The combine kernel merges the P partials of each query head:
//   M = max_p m_p,  out = sum_p e^{m_p - M} acc_p / sum_p e^{m_p - M} l_p.
#include "wi_internal.h"

namespace wi {
namespace {

constexpr int ATT_THREADS = 256;
constexpr int STREAMS = ATT_THREADS / 16;
constexpr int IPS = 4;        // items per stream per batch
constexpr int PART = 2 + D;   // m, l, acc[128]

template <int DT>
__device__ __forceinline__ void unpack(const uint4 r[2], float x[8]) {
  if constexpr (DT == WI_BF16) {
    const uint32_t w[4] = {r[0].x, r[0].y, r[0].z, r[0].w};
#pragma unroll
    for (int t = 0; t < 4; t++) {
      x[2 * t] = __uint_as_float(w[t] << 16);
      x[2 * t + 1] = __uint_as_float(w[t] & 0xFFFF0000u);
    }
  } else {
    const uint32_t w[8] = {r[0].x, r[0].y, r[0].z, r[0].w, r[1].x, r[1].y, r[1].z, r[1].w};
#pragma unroll
    for (int t = 0; t < 8; t++) x[t] = __uint_as_float(w[t]);
  }
}

template <int DT>
__device__ __forceinline__ void load_raw(const void* base, int64_t row, int j, uint4 r[2]) {
  if constexpr (DT == WI_BF16) {
    r[0] = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(base) + row * D + 8 * j);
  } else {
    const uint4* p = reinterpret_cast<const uint4*>(reinterpret_cast<const float*>(base) + row * D + 8 * j);
    r[0] = p[0];
    r[1] = p[1];
  }
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
    const float* __restrict__ vsum, const float* __restrict__ S,
    const int* __restrict__ Rpre, const int* __restrict__ rowtab,
    const int* __restrict__ El, const int* __restrict__ Esz, const void* __restrict__ q,
    int C, int64_t capT, int64_t n_idx, int n_st, int G, int H, int Hq, int K_r, int K_e,
    int P, float scale, float* __restrict__ part) {
  const int p = blockIdx.x, u = blockIdx.y;
  const int b = u / H, h = u % H;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int grp = tid >> 4, j = tid & 15;

  // level 1: execution-buffer length and the query
  const int64_t NX = (int64_t)n_st + Rpre[(int64_t)u * (K_r + 1) + K_r];
  float qv[GM][8];
#pragma unroll
  for (int g = 0; g < GM; g++) {
    uint4 r[2];
    load_raw<DT>(q, (int64_t)b * Hq + (int64_t)h * G + min(g, G - 1), j, r);
    unpack<DT>(r, qv[g]);
    const float sg = g < G ? scale : 0.f;
#pragma unroll
    for (int t = 0; t < 8; t++) qv[g][t] *= sg;
  }
  const int64_t x0 = NX * p / P, x1 = NX * (p + 1) / P;
  const int64_t e0 = (int64_t)K_e * p / P, e1 = (int64_t)K_e * (p + 1) / P;
  const int64_t nx = x1 - x0, nit = nx + (e1 - e0);
  const int64_t s0 = nit * grp / STREAMS, s1 = nit * (grp + 1) / STREAMS;
  const int* rt = rowtab + (int64_t)u * n_idx;
  const int* E = El + (int64_t)u * K_e;
  const int* ES = Esz + (int64_t)u * K_e;

  float m[GM], l[GM], acc[GM][8];
#pragma unroll
  for (int g = 0; g < GM; g++) {
    m[g] = -INFINITY;
    l[g] = 0.f;
#pragma unroll
    for (int t = 0; t < 8; t++) acc[g][t] = 0.f;
  }

  for (int64_t ib = s0; ib < s1; ib += IPS) {
    // level 2: item metadata, loaded unconditionally from clamped in-bounds
    // addresses so that no load waits behind a branch
    int kind[IPS];  // 0 none, 1 steady token, 2 block token, 3 estimation cluster
    int rtv[IPS], ev[IPS], esv[IPS];
#pragma unroll
    for (int k = 0; k < IPS; k++) {
      const int64_t it = ib + k;
      const int64_t f = x0 + it;
      const int64_t ri = f - n_st < 0 ? 0 : (f - n_st < n_idx ? f - n_st : n_idx - 1);
      const int64_t e = e0 + (it - nx);
      const int64_t ei = e < 0 ? 0 : (e < K_e ? e : (K_e > 0 ? K_e - 1 : 0));
      rtv[k] = rt[ri];
      ev[k] = K_e > 0 ? E[ei] : 0;
      esv[k] = K_e > 0 ? ES[ei] : 0;
      kind[k] = it >= s1 ? 0 : (it < nx ? (f < n_st ? 1 : 2) : 3);
    }
    // level 3: data (two 16-byte loads per lane and item, plus the logits of
    // an estimation cluster), again unconditional
    const uint8_t* pa[IPS];
    const uint8_t* pb[IPS];
    const float* ps[IPS];
    float mult[IPS];
#pragma unroll
    for (int k = 0; k < IPS; k++) {
      constexpr int RB = D * (DT == WI_BF16 ? 2 : 4);
      const int64_t f = x0 + ib + k;
      const uint8_t* kb8 = reinterpret_cast<const uint8_t*>(kblk);
      const uint8_t* vb8 = reinterpret_cast<const uint8_t*>(vblk);
      const uint8_t* sk8 = reinterpret_cast<const uint8_t*>(stk);
      const uint8_t* sv8 = reinterpret_cast<const uint8_t*>(stv);
      const int64_t lane_off = (int64_t)j * (RB / 16);
      if (kind[k] == 3 && esv[k] > 0) {
        const uint8_t* vr = reinterpret_cast<const uint8_t*>(vsum + ((int64_t)u * C + ev[k]) * D + 8 * j);
        pa[k] = vr;
        pb[k] = DT == WI_BF16 ? vr + 16 : vr;
        ps[k] = S + ((int64_t)u * C + ev[k]) * GM;
        mult[k] = (float)esv[k];
      } else if (kind[k] == 3) {
        kind[k] = 0;
      }
      if (kind[k] == 1) {
        const int64_t row = (int64_t)u * n_st + f;
        pa[k] = sk8 + row * RB + lane_off;
        pb[k] = sv8 + row * RB + lane_off;
      } else if (kind[k] == 2) {
        const int64_t row = (int64_t)u * capT + rtv[k];
        pa[k] = kb8 + row * RB + lane_off;
        pb[k] = vb8 + row * RB + lane_off;
      }
      if (kind[k] != 3) {
        ps[k] = S;
        mult[k] = 1.f;
      }
      if (kind[k] == 0) {
        pa[k] = sk8;
        pb[k] = sk8;
      }
    }
    constexpr int NR = DT == WI_BF16 ? 2 : 4;  // 16-byte words per lane and item
    uint4 raw[IPS][NR];
    float zs[IPS][GM];
#pragma unroll
    for (int k = 0; k < IPS; k++) {
      // token: K (then V); estimation cluster: its value sum as 8 fp32
      raw[k][0] = reinterpret_cast<const uint4*>(pa[k])[0];
      if constexpr (DT == WI_BF16) {
        raw[k][1] = *reinterpret_cast<const uint4*>(pb[k]);
      } else {
        raw[k][1] = reinterpret_cast<const uint4*>(pa[k])[1];
        raw[k][2] = reinterpret_cast<const uint4*>(pb[k])[0];
        raw[k][3] = reinterpret_cast<const uint4*>(pb[k])[1];
      }
#pragma unroll
      for (int g = 0; g < GM; g += 4) {
        const float4 z4 = *reinterpret_cast<const float4*>(ps[k] + g);
        zs[k][g] = z4.x;
        zs[k][g + 1] = z4.y;
        zs[k][g + 2] = z4.z;
        zs[k][g + 3] = z4.w;
      }
    }
    // logits
    float z[IPS][GM];
#pragma unroll
    for (int k = 0; k < IPS; k++) {
      if (kind[k] == 1 || kind[k] == 2) {
        float kx[8];
        unpack<DT>(raw[k], kx);
#pragma unroll
        for (int g = 0; g < GM; g++) {
          float zz = 0.f;
          if (g < G) {
#pragma unroll
            for (int t = 0; t < 8; t++) zz = fmaf(qv[g][t], kx[t], zz);
            zz = row16_sum(zz);
          }
          z[k][g] = zz;
        }
      } else {
#pragma unroll
        for (int g = 0; g < GM; g++) z[k][g] = zs[k][g];
      }
    }
    // accumulate
#pragma unroll
    for (int g = 0; g < GM; g++) {
      if (g >= G) continue;
      float mn = m[g];
#pragma unroll
      for (int k = 0; k < IPS; k++)
        if (kind[k] != 0) mn = fmaxf(mn, z[k][g]);
      if (mn == -INFINITY) continue;
      const float al = ex<DT>(m[g] - mn);
      l[g] *= al;
#pragma unroll
      for (int t = 0; t < 8; t++) acc[g][t] *= al;
#pragma unroll
      for (int k = 0; k < IPS; k++) {
        if (kind[k] == 0) continue;
        const float pz = ex<DT>(z[k][g] - mn);
        float vx[8];
        if (kind[k] == 3) unpack<WI_F32>(raw[k], vx);
        else unpack<DT>(&raw[k][DT == WI_BF16 ? 1 : 2], vx);
        l[g] = fmaf(mult[k], pz, l[g]);
#pragma unroll
        for (int t = 0; t < 8; t++) acc[g][t] = fmaf(pz, vx[t], acc[g][t]);
      }
      m[g] = mn;
    }
  }

  // merge the four groups of each wave (fixed butterfly order)
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

  // merge the four waves through LDS, write the chunk partial
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
  float* pout = part + ((int64_t)u * P + p) * G * PART;
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
    pout[g * PART + 2 + t] = a;
    if (t == 0) {
      pout[g * PART] = mm;
      pout[g * PART + 1] = ll;
    }
  }
}

// Merge the P chunk partials of one (unit, query head):
//   M = max_p m_p, w_p = e^{m_p - M},
//   out = sum_p w_p acc_p / sum_p w_p l_p   (sums in fixed chunk order).
// 256 threads: 32 float4 slots of the 128 dims x 8 phases over the chunks.
template <int DT>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ part, int G,
                                                      int H, int Hq, int P,
                                                      float* __restrict__ out) {
  constexpr int PHASES = 8;
  const int u = blockIdx.x / G, g = blockIdx.x % G;
  const int b = u / H, h = u % H;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  __shared__ float w[1024];
  __shared__ float red[4];
  __shared__ float4 acc4[PHASES][32];
  const float* pu = part + (int64_t)u * P * G * PART + (int64_t)g * PART;
  // M
  float mm = -INFINITY;
  for (int c = tid; c < P; c += 256) mm = fmaxf(mm, pu[(int64_t)c * G * PART]);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) mm = fmaxf(mm, __shfl_xor(mm, o, 64));
  if (lane == 0) red[wv] = mm;
  __syncthreads();
  const float M = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  __syncthreads();
  // weights and the denominator
  float dd = 0.f;
  for (int c = tid; c < P; c += 256) {
    const float* pp = pu + (int64_t)c * G * PART;
    const float mp = pp[0];
    const float wc = (mp == -INFINITY) ? 0.f : ex<DT>(mp - M);
    w[c] = wc;
    dd = fmaf(wc, pp[1], dd);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) dd += __shfl_xor(dd, o, 64);
  if (lane == 0) red[wv] = dd;
  __syncthreads();
  const float den = (red[0] + red[1]) + (red[2] + red[3]);
  // numerators
  const int f4 = tid & 31, ph = tid >> 5;
  float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll 4
  for (int c = ph; c < P; c += PHASES) {
    const float wc = w[c];
    const float4 v = *reinterpret_cast<const float4*>(pu + (int64_t)c * G * PART + 2 + 4 * f4);
    a.x = fmaf(wc, v.x, a.x);
    a.y = fmaf(wc, v.y, a.y);
    a.z = fmaf(wc, v.z, a.z);
    a.w = fmaf(wc, v.w, a.w);
  }
  acc4[ph][f4] = a;
  __syncthreads();
  if (tid < 32) {
    float4 t4 = acc4[0][tid];
#pragma unroll
    for (int q2 = 1; q2 < PHASES; q2++) {
      const float4 o = acc4[q2][tid];
      t4.x += o.x;
      t4.y += o.y;
      t4.z += o.z;
      t4.w += o.w;
    }
    const float inv = 1.f / den;
    *reinterpret_cast<float4*>(out + ((int64_t)b * Hq + (int64_t)h * G + g) * D + 4 * tid) =
        make_float4(t4.x * inv, t4.y * inv, t4.z * inv, t4.w * inv);
  }
}

template <int DT>
hipError_t launch_attend_dt(const DecodeArgs& a, const wi_index_bufs& bf, const void* q,
                            float* out, const DecodeWs& ws, hipStream_t s) {
  const Geom& g = *a.g;
  dim3 grid(a.P, g.U);
  const int64_t capT = g.cap * g.T;
#define WI_ATT(GMV)                                                                         \
  WI_LAUNCH(K_ATTEND, (attend_kernel<DT, GMV>), grid, dim3(ATT_THREADS), 0, s, bf.k_blocks, \
            bf.v_blocks, bf.steady_k, bf.steady_v, bf.value_sum, ws.S, ws.Rpre, ws.rowtab,   \
            ws.E, ws.Esz, q, g.C, capT, g.n_idx, g.n_st, a.G, g.H, a.Hq, a.K_r, a.K_e, a.P,  \
            a.scale, ws.part)
  if (a.G <= 4) WI_ATT(4);
  else if (a.G <= 8) WI_ATT(8);
  else WI_ATT(16);
#undef WI_ATT
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  WI_LAUNCH(K_COMBINE, (combine_kernel<DT>), dim3(g.U * a.G), dim3(256), 0, s, ws.part, a.G, g.H,
            a.Hq, a.P, out);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attend(const DecodeArgs& a, const wi_index_bufs& b, const void* q,
                         float* out, const DecodeWs& ws, hipStream_t s) {
  return a.g->dtype == WI_BF16 ? launch_attend_dt<WI_BF16>(a, b, q, out, ws, s)
                               : launch_attend_dt<WI_F32>(a, b, q, out, ws, s);
}

}  // namespace wi
