// Index build, Lloyd assignment step: every point of a segment goes to its
// nearest centroid (RetroInfer, framerc blog section 2.1: k-means over each
// 8K-token segment).
//
// The decision is defined exactly: nearest by the float64 squared distance
// sum_t (x_t - mu_t)^2 accumulated with one fused multiply-add per dimension
// in dimension order, lowest centroid id on ties. It is computed in two
// stages:
//
// 1. MFMA stage (dense contraction). The score s_c = 2<x, mu_c> - |mu_c|^2
//    (argmax s_c = argmin distance) of a 256-point tile against all
//    centroids of its segment: centroids are the A operand (rows), staged in
//    LDS 256 at a time, pre-doubled (exact) with 16-byte row padding; points
//    are the B operand (columns) held in registers for the whole sweep.
//    bf16 uses v_mfma_f32_32x32x16_bf16 (products exact, fp32
//    accumulation); fp32 uses v_mfma_f32_32x32x2_f32. The epilogue keeps,
//    per point, the best score, its centroid and the second-best score.
// 2. Certification. With |s~ - s| <= gamma_130 (|x|^2 + 2 max_c |mu_c|^2)
//    for either accumulation, a point whose best score leads the second by
//    more than W = 2^-12 (|x|^2 + 2 max|mu|^2) -- at least 15x that bound,
//    doubled -- has its exact nearest centroid at the MFMA winner. Other
//    points are listed and the fallback kernel evaluates the exact float64
//    distance to every centroid of their segment.
#include "wi_internal.h"

namespace wi {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int AT = 256;           // threads per workgroup (4 waves)
constexpr int CHUNK = 256;        // centroids staged in LDS per pass
constexpr int ROWB = D * 2 + 16;  // bf16 LDS row bytes (padded)
constexpr int ROWF = D * 4 + 16;  // fp32 LDS row bytes (padded)

template <int DT>
__device__ __forceinline__ const uint8_t* kptr(const void* K, const Geom& g, int u, int64_t pos) {
  const int b = u / g.H, h = u % g.H;
  const int64_t off = (int64_t)b * g.sb + (int64_t)h * g.sh + pos * g.st;
  return reinterpret_cast<const uint8_t*>(K) + off * (DT == WI_BF16 ? 2 : 4);
}

struct Best {
  float s1, s2;
  int i1;
};

__device__ __forceinline__ void upd(Best& b, float s, int i) {
  // s2 = median(s1, s2, s) keeps the second-largest of {s1, s2, s}
  b.s2 = __builtin_amdgcn_fmed3f(b.s1, b.s2, s);
  if (s > b.s1) {
    b.s1 = s;
    b.i1 = i;
  }
}

__device__ __forceinline__ Best merge(Best a, Best o) {
  Best r;
  if (o.s1 > a.s1 || (o.s1 == a.s1 && o.i1 < a.i1)) {
    r.s1 = o.s1;
    r.i1 = o.i1;
  } else {
    r.s1 = a.s1;
    r.i1 = a.i1;
  }
  r.s2 = fmaxf(fminf(a.s1, o.s1), fmaxf(a.s2, o.s2));
  return r;
}

// ---------------------------------------------------------------------------
// bf16: each wave owns 2 column tiles of 32 points (64 points per wave).
__global__ __launch_bounds__(AT, 2) void assign_bf16_kernel(Geom g, const void* __restrict__ K,
                                                            const void* __restrict__ cent,
                                                            BuildWs ws) {
  constexpr int NTL = 2;
  extern __shared__ __align__(16) uint8_t lds[];
  uint8_t* crow = lds;                                         // CHUNK rows of ROWB
  float* cnorm = reinterpret_cast<float*>(lds + CHUNK * ROWB);  // CHUNK norms
  float* red = cnorm + CHUNK;                                   // 4 floats

  const int gs = blockIdx.y, u = gs / g.n_seg, s = gs % g.n_seg;
  const int n = seg_n(g, s), Cs = seg_c(g, s), cb = seg_cbase(g, s);
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int p0 = blockIdx.x * 256;  // 4 waves x 64 points
  if (p0 >= n) return;
  const int64_t first = seg_first(g, s);

  // B fragments: point p = p0 + 64*wv + 32*t + (lane & 31), dims
  // 16*k + 8*(lane >> 5) .. +8, for k = 0..7.
  uint4 bfrag[NTL][8];
  float xn[NTL];
#pragma unroll
  for (int t = 0; t < NTL; t++) {
    const int p = p0 + 64 * wv + 32 * t + (lane & 31);
    float sq = 0.f;
    if (p < n) {
      const uint4* row = reinterpret_cast<const uint4*>(kptr<WI_BF16>(K, g, u, first + p));
#pragma unroll
      for (int k = 0; k < 8; k++) {
        bfrag[t][k] = row[2 * k + (lane >> 5)];
        const uint32_t w[4] = {bfrag[t][k].x, bfrag[t][k].y, bfrag[t][k].z, bfrag[t][k].w};
#pragma unroll
        for (int e = 0; e < 4; e++) {
          const float a = __uint_as_float(w[e] << 16), b2 = __uint_as_float(w[e] & 0xFFFF0000u);
          sq = fmaf(a, a, sq);
          sq = fmaf(b2, b2, sq);
        }
      }
    } else {
#pragma unroll
      for (int k = 0; k < 8; k++) bfrag[t][k] = make_uint4(0, 0, 0, 0);
    }
    xn[t] = sq + __shfl_xor(sq, 32, 64);
  }

  Best best[NTL];
#pragma unroll
  for (int t = 0; t < NTL; t++) best[t] = {-INFINITY, -INFINITY, 0};
  float mmax = 0.f;

  const uint16_t* C16 = reinterpret_cast<const uint16_t*>(cent) + ((int64_t)u * g.C + cb) * D;
  for (int c0 = 0; c0 < Cs; c0 += CHUNK) {
    __syncthreads();
    // stage centroids c0..c0+CHUNK: 16 lanes per row, 16 bytes each
    for (int rr = tid >> 4; rr < CHUNK; rr += AT / 16) {
      const int c = c0 + rr;
      const int j = tid & 15;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (c < Cs) v = reinterpret_cast<const uint4*>(C16 + (int64_t)c * D)[j];
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
      uint32_t o[4];
      float sq = 0.f;
#pragma unroll
      for (int e = 0; e < 4; e++) {
        const float a = __uint_as_float(w[e] << 16), b2 = __uint_as_float(w[e] & 0xFFFF0000u);
        sq = fmaf(a, a, sq);
        sq = fmaf(b2, b2, sq);
        const uint32_t a2 = __float_as_uint(2.f * a) >> 16;
        const uint32_t bb2 = __float_as_uint(2.f * b2) & 0xFFFF0000u;
        o[e] = a2 | bb2;
      }
      *reinterpret_cast<uint4*>(crow + rr * ROWB + 16 * j) = make_uint4(o[0], o[1], o[2], o[3]);
      sq += __shfl_xor(sq, 8, 16);
      sq += __shfl_xor(sq, 4, 16);
      sq += __shfl_xor(sq, 2, 16);
      sq += __shfl_xor(sq, 1, 16);
      if (j == 0) cnorm[rr] = c < Cs ? sq : INFINITY;
      if (c < Cs) mmax = fmaxf(mmax, sq);
    }
    __syncthreads();
    const int nm = min(CHUNK, Cs - c0);
    for (int m = 0; m < (nm + 31) / 32; m++) {
      f32x16_t acc[NTL];
#pragma unroll
      for (int t = 0; t < NTL; t++) acc[t] = (f32x16_t){};
      const uint8_t* arow = crow + (32 * m + (lane & 31)) * ROWB + 16 * (lane >> 5);
#pragma unroll
      for (int k = 0; k < 8; k++) {
        const uint4 av = *reinterpret_cast<const uint4*>(arow + 32 * k);
        const bf16x8_t a = __builtin_bit_cast(bf16x8_t, av);
#pragma unroll
        for (int t = 0; t < NTL; t++)
          acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              a, __builtin_bit_cast(bf16x8_t, bfrag[t][k]), acc[t], 0, 0, 0);
      }
      // epilogue: lane holds column (lane & 31), rows
      // 8*(i/4) + 4*(lane>>5) + (i%4) of this 32-row tile
#pragma unroll
      for (int q = 0; q < 4; q++) {
        const int r0 = 32 * m + 8 * q + 4 * (lane >> 5);
        const float4 nv = *reinterpret_cast<const float4*>(cnorm + r0);
        const float nn[4] = {nv.x, nv.y, nv.z, nv.w};
#pragma unroll
        for (int e = 0; e < 4; e++) {
#pragma unroll
          for (int t = 0; t < NTL; t++) upd(best[t], acc[t][4 * q + e] - nn[e], c0 + r0 + e);
        }
      }
    }
  }
  // max |mu|^2 over the segment: reduce over the block
  mmax = wave_max(mmax);
  __syncthreads();
  if (lane == 0) red[wv] = mmax;
  __syncthreads();
  mmax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));

#pragma unroll
  for (int t = 0; t < NTL; t++) {
    Best o;
    o.s1 = __shfl_xor(best[t].s1, 32, 64);
    o.s2 = __shfl_xor(best[t].s2, 32, 64);
    o.i1 = __shfl_xor(best[t].i1, 32, 64);
    const Best bb = merge(best[t], o);
    const int p = p0 + 64 * wv + 32 * t + (lane & 31);
    if (lane < 32 && p < n) {
      const float W = 0x1p-12f * (xn[t] + 2.f * mmax);
      const int64_t pid = (int64_t)u * g.n_idx + (int64_t)s * g.seg_len + p;
      if (bb.s2 >= bb.s1 - W) {
        ws.label[pid] = -1;
        const int slot = atomicAdd(ws.amb, 1);
        ws.amb[1 + slot] = (int)pid;
      } else {
        ws.label[pid] = bb.i1;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// fp32: each wave owns 1 column tile of 32 points (32 points per wave).
__global__ __launch_bounds__(AT, 2) void assign_f32_kernel(Geom g, const void* __restrict__ K,
                                                           const void* __restrict__ cent,
                                                           BuildWs ws) {
  extern __shared__ __align__(16) uint8_t lds[];
  uint8_t* crow = lds;
  float* cnorm = reinterpret_cast<float*>(lds + (CHUNK / 2) * ROWF);
  float* red = cnorm + CHUNK / 2;
  constexpr int FCH = CHUNK / 2;  // 128 fp32 centroids per pass

  const int gs = blockIdx.y, u = gs / g.n_seg, s = gs % g.n_seg;
  const int n = seg_n(g, s), Cs = seg_c(g, s), cb = seg_cbase(g, s);
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int p0 = blockIdx.x * 128;  // 128 points per block
  if (p0 >= n) return;
  const int64_t first = seg_first(g, s);

  // B operand of v_mfma_f32_32x32x2_f32: lane supplies B[k = lane>>5][col]
  const int p = p0 + 32 * wv + (lane & 31);
  float bx[64];
  float sq = 0.f;
  if (p < n) {
    const float* row = reinterpret_cast<const float*>(kptr<WI_F32>(K, g, u, first + p));
#pragma unroll
    for (int k = 0; k < 64; k++) {
      bx[k] = row[2 * k + (lane >> 5)];
      sq = fmaf(bx[k], bx[k], sq);
    }
  } else {
#pragma unroll
    for (int k = 0; k < 64; k++) bx[k] = 0.f;
  }
  const float xn = sq + __shfl_xor(sq, 32, 64);

  Best best = {-INFINITY, -INFINITY, 0};
  float mmax = 0.f;
  const float* C32 = reinterpret_cast<const float*>(cent) + ((int64_t)u * g.C + cb) * D;
  for (int c0 = 0; c0 < Cs; c0 += FCH) {
    __syncthreads();
    for (int rr = tid >> 4; rr < FCH; rr += AT / 16) {
      const int c = c0 + rr;
      const int j = tid & 15;
      float4 v0 = make_float4(0, 0, 0, 0), v1 = v0;
      if (c < Cs) {
        v0 = reinterpret_cast<const float4*>(C32 + (int64_t)c * D)[2 * j];
        v1 = reinterpret_cast<const float4*>(C32 + (int64_t)c * D)[2 * j + 1];
      }
      float q2 = 0.f;
      q2 = fmaf(v0.x, v0.x, q2); q2 = fmaf(v0.y, v0.y, q2);
      q2 = fmaf(v0.z, v0.z, q2); q2 = fmaf(v0.w, v0.w, q2);
      q2 = fmaf(v1.x, v1.x, q2); q2 = fmaf(v1.y, v1.y, q2);
      q2 = fmaf(v1.z, v1.z, q2); q2 = fmaf(v1.w, v1.w, q2);
      float4* dst = reinterpret_cast<float4*>(crow + rr * ROWF + 32 * j);
      dst[0] = make_float4(2.f * v0.x, 2.f * v0.y, 2.f * v0.z, 2.f * v0.w);
      dst[1] = make_float4(2.f * v1.x, 2.f * v1.y, 2.f * v1.z, 2.f * v1.w);
      q2 += __shfl_xor(q2, 8, 16);
      q2 += __shfl_xor(q2, 4, 16);
      q2 += __shfl_xor(q2, 2, 16);
      q2 += __shfl_xor(q2, 1, 16);
      if (j == 0) cnorm[rr] = c < Cs ? q2 : INFINITY;
      if (c < Cs) mmax = fmaxf(mmax, q2);
    }
    __syncthreads();
    const int nm = min(FCH, Cs - c0);
    for (int m = 0; m < (nm + 31) / 32; m++) {
      f32x16_t acc = (f32x16_t){};
      const float* arow = reinterpret_cast<const float*>(crow + (32 * m + (lane & 31)) * ROWF);
#pragma unroll
      for (int k = 0; k < 64; k++)
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(arow[2 * k + (lane >> 5)], bx[k], acc, 0, 0, 0);
#pragma unroll
      for (int q = 0; q < 4; q++) {
        const int r0 = 32 * m + 8 * q + 4 * (lane >> 5);
#pragma unroll
        for (int e = 0; e < 4; e++) upd(best, acc[4 * q + e] - cnorm[r0 + e], c0 + r0 + e);
      }
    }
  }
  mmax = wave_max(mmax);
  __syncthreads();
  if (lane == 0) red[wv] = mmax;
  __syncthreads();
  mmax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  Best o;
  o.s1 = __shfl_xor(best.s1, 32, 64);
  o.s2 = __shfl_xor(best.s2, 32, 64);
  o.i1 = __shfl_xor(best.i1, 32, 64);
  const Best bb = merge(best, o);
  if (lane < 32 && p < n) {
    const float W = 0x1p-12f * (xn + 2.f * mmax);
    const int64_t pid = (int64_t)u * g.n_idx + (int64_t)s * g.seg_len + p;
    if (bb.s2 >= bb.s1 - W) {
      ws.label[pid] = -1;
      const int slot = atomicAdd(ws.amb, 1);
      ws.amb[1 + slot] = (int)pid;
    } else {
      ws.label[pid] = bb.i1;
    }
  }
}

// ---------------------------------------------------------------------------
// Exact fallback: one wave per listed point, float64 distances to every
// centroid of its segment, lowest id on ties.
template <int DT>
__global__ __launch_bounds__(256) void assign_fix_kernel(Geom g, const void* __restrict__ K,
                                                          const void* __restrict__ cent,
                                                          BuildWs ws) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int cnt = ws.amb[0];
  const int nw = gridDim.x * 4;
  for (int e = blockIdx.x * 4 + wv; e < cnt; e += nw) {
    const int pid = ws.amb[1 + e];
    const int u = (int)(pid / g.n_idx);
    const int64_t loc = pid % g.n_idx;
    const int s = (int)(loc / g.seg_len);
    const int i = (int)(loc % g.seg_len);
    const int Cs = seg_c(g, s), cb = seg_cbase(g, s);
    const uint8_t* xr = kptr<DT>(K, g, u, seg_first(g, s) + i);
    // lane holds dims lane and lane + 64; broadcast with shuffles
    double xa, xb;
    if constexpr (DT == WI_BF16) {
      const uint16_t* x16 = reinterpret_cast<const uint16_t*>(xr);
      xa = (double)__uint_as_float(((uint32_t)x16[lane]) << 16);
      xb = (double)__uint_as_float(((uint32_t)x16[lane + 64]) << 16);
    } else {
      const float* x32 = reinterpret_cast<const float*>(xr);
      xa = (double)x32[lane];
      xb = (double)x32[lane + 64];
    }
    double bd = INFINITY;
    int bi = 0x7FFFFFFF;
    const int rounds = (Cs + 63) / 64;
    for (int rd = 0; rd < rounds; rd++) {
      const int c = rd * 64 + lane;
      const bool ok = c < Cs;
      const int cc = ok ? c : 0;
      double acc = 0.0;
      for (int t = 0; t < D; t++) {
        const double xt = __shfl(t < 64 ? xa : xb, t & 63, 64);
        double ct;
        if constexpr (DT == WI_BF16)
          ct = (double)__uint_as_float(((uint32_t) reinterpret_cast<const uint16_t*>(cent)
                                            [((int64_t)u * g.C + cb + cc) * D + t]) << 16);
        else
          ct = (double)reinterpret_cast<const float*>(cent)[((int64_t)u * g.C + cb + cc) * D + t];
        const double dl = xt - ct;
        acc = __builtin_fma(dl, dl, acc);
      }
      if (ok && acc < bd) {  // c grows within a lane: strict < keeps the lowest id
        bd = acc;
        bi = c;
      }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const double od = __shfl_xor(bd, o, 64);
      const int oi = __shfl_xor(bi, o, 64);
      if (od < bd || (od == bd && oi < bi)) {
        bd = od;
        bi = oi;
      }
    }
    if (lane == 0) ws.label[pid] = bi;
  }
}

}  // namespace

hipError_t launch_assign(const Geom& g, const void* K, const void* cent, const BuildWs& ws,
                         hipStream_t s) {
  hipError_t e = launch_zero_i32(ws.amb, 1, s);
  if (e != hipSuccess) return e;
  if (g.dtype == WI_BF16) {
    const size_t lds = CHUNK * ROWB + CHUNK * 4 + 16;
    dim3 grid((g.seg_len + 255) / 256, g.U * g.n_seg);
    WI_LAUNCH(K_ASSIGN, assign_bf16_kernel, grid, dim3(AT), lds, s, g, K, cent, ws);
  } else {
    const size_t lds = (CHUNK / 2) * ROWF + (CHUNK / 2) * 4 + 16;
    dim3 grid((g.seg_len + 127) / 128, g.U * g.n_seg);
    WI_LAUNCH(K_ASSIGN, assign_f32_kernel, grid, dim3(AT), lds, s, g, K, cent, ws);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (g.dtype == WI_BF16)
    WI_LAUNCH(K_ASSIGN_FIX, assign_fix_kernel<WI_BF16>, dim3(256), dim3(256), 0, s, g, K, cent, ws);
  else
    WI_LAUNCH(K_ASSIGN_FIX, assign_fix_kernel<WI_F32>, dim3(256), dim3(256), 0, s, g, K, cent, ws);
  return hipGetLastError();
}

}  // namespace wi
