// Index build, initialisation: k-means++ seeding of every segment
// (Arthur and Vassilvitskii, SODA 2007). The RetroInfer pages cluster each
// 8K-token segment independently (framerc blog section 2.1, the
// segmented_kmeans sketch; techwalker article section 3) and name no
// initialisation; k-means++ is the standard one for Lloyd's algorithm.
//
// Sampling arithmetic, fixed so the picks depend on the inputs alone:
//   - D_i: squared distance to the nearest chosen centroid, float32, one
//     fused multiply-add per dimension in dimension order (one thread per
//     point reproduces that order exactly);
//   - w_i = floor(D_i * 2^F) as 64-bit integers, F fixed per segment from
//     the distances to the first centroid so that sum_i w_i < 2^62; integer
//     sums are exact and order-free, so the parallel reduction and scan give
//     the same totals as a sequential pass;
//   - the draw for round r is the smallest i whose inclusive weight prefix
//     exceeds floor(U_r * W), with U_r the 53-bit uniform of the counter-based
//     key (seed, b, layer, h, segment, r); the first pick is
//     floor(U_0 * n_s). When every weight is zero the smallest index not yet
//     chosen is taken.
//
// Launch structure: one workgroup per (segment, 256-point slice). Round r is
// one launch over all segments of the call; every workgroup of a segment
// redundantly derives pick r from the per-slice weight sums of round r-1,
// then updates the distances and weights of its own points and writes its
// slice sum for round r. Weights and sums are double-buffered by round
// parity, so a launch only reads what the previous launch wrote.
#include "wi_internal.h"

namespace wi {
namespace {

constexpr int NT = KPP_SLICE;  // threads per workgroup = points per slice

template <int DT>
__device__ __forceinline__ const void* krow(const void* K, const Geom& g, int u, int64_t pos) {
  const int b = u / g.H, h = u % g.H;
  const int64_t off = (int64_t)b * g.sb + (int64_t)h * g.sh + pos * g.st;
  if constexpr (DT == WI_BF16) return reinterpret_cast<const uint16_t*>(K) + off;
  else return reinterpret_cast<const float*>(K) + off;
}

// Sequential float32 squared distance of a global row to an LDS centroid.
template <int DT>
__device__ __forceinline__ float dist32(const void* row, const float* mu) {
  float acc = 0.f;
  if constexpr (DT == WI_BF16) {
    const uint4* p = reinterpret_cast<const uint4*>(row);
#pragma unroll 4
    for (int c = 0; c < D / 8; c++) {
      const uint4 v = p[c];
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int t = 0; t < 4; t++) {
        const float x0 = __uint_as_float(w[t] << 16);
        const float x1 = __uint_as_float(w[t] & 0xFFFF0000u);
        const float d0 = x0 - mu[8 * c + 2 * t];
        acc = __builtin_fmaf(d0, d0, acc);
        const float d1 = x1 - mu[8 * c + 2 * t + 1];
        acc = __builtin_fmaf(d1, d1, acc);
      }
    }
  } else {
    const float4* p = reinterpret_cast<const float4*>(row);
#pragma unroll 4
    for (int c = 0; c < D / 4; c++) {
      const float4 v = p[c];
      const float x[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int t = 0; t < 4; t++) {
        const float d0 = x[t] - mu[4 * c + t];
        acc = __builtin_fmaf(d0, d0, acc);
      }
    }
  }
  return acc;
}

// The same sum, stopped early once it cannot end below `bound`. Every term
// is a square, and a round-to-nearest fused multiply-add of a non-negative
// product onto acc never lowers acc, so the running value only grows: once
// it is >= bound (or NaN, or bound is NaN) the full sum is not below bound
// either, and the caller's `dist < bound` test comes out false both ways.
// The row is read in 32-dimension chunks, so a point the new centroid cannot
// claim usually costs one chunk of its row instead of all of it. Returns the
// full sum whenever that sum is below bound.
// The first chunk is loaded by the caller (early, before the pick is
// known) and passed in; the rest is read only while the sum stays below bound.
template <int DT>
struct Chunk {
  uint4 v[DT == WI_BF16 ? 4 : 8];  // 32 dimensions
};

// Chunk ch of a point from the chunk-major key copy: `base` is the point's
// first chunk, chunks of one point lie `cstride` 16-byte vectors apart.
template <int DT>
__device__ __forceinline__ Chunk<DT> load_chunk(const uint4* base, int64_t cstride, int ch) {
  constexpr int VPC = DT == WI_BF16 ? 4 : 8;
  Chunk<DT> c;
#pragma unroll
  for (int j = 0; j < VPC; j++) c.v[j] = base[ch * cstride + j];
  return c;
}

template <int DT>
__device__ __forceinline__ float add_chunk(float acc, const Chunk<DT>& c, const float* m) {
  constexpr int VPC = DT == WI_BF16 ? 4 : 8;
#pragma unroll
  for (int j = 0; j < VPC; j++) {
    const uint32_t w[4] = {c.v[j].x, c.v[j].y, c.v[j].z, c.v[j].w};
#pragma unroll
    for (int t = 0; t < 4; t++) {
      if constexpr (DT == WI_BF16) {
        const float e0 = __uint_as_float(w[t] << 16) - m[8 * j + 2 * t];
        acc = __builtin_fmaf(e0, e0, acc);
        const float e1 = __uint_as_float(w[t] & 0xFFFF0000u) - m[8 * j + 2 * t + 1];
        acc = __builtin_fmaf(e1, e1, acc);
      } else {
        const float e0 = __uint_as_float(w[t]) - m[4 * j + t];
        acc = __builtin_fmaf(e0, e0, acc);
      }
    }
  }
  return acc;
}

template <int DT>
__device__ __forceinline__ float dist32_below(const uint4* base, int64_t cstride,
                                             const Chunk<DT>& c0, const float* mu, float bound) {
  float acc = add_chunk<DT>(0.f, c0, mu);
#pragma unroll 1
  for (int ch = 1; ch < 4 && acc < bound; ch++)
    acc = add_chunk<DT>(acc, load_chunk<DT>(base, cstride, ch), mu + 32 * ch);
  return acc;
}

template <int DT>
__device__ __forceinline__ void load_mu(const void* row, float* mu) {
  const int t = threadIdx.x;
  if (t < D) {
    if constexpr (DT == WI_BF16)
      mu[t] = __uint_as_float(((uint32_t) reinterpret_cast<const uint16_t*>(row)[t]) << 16);
    else
      mu[t] = reinterpret_cast<const float*>(row)[t];
  }
}

template <int DT>
__device__ __forceinline__ void store_centroid(void* cent, int64_t crow, const void* row) {
  const int t = threadIdx.x;
  if (t < D) {
    if constexpr (DT == WI_BF16)
      reinterpret_cast<uint16_t*>(cent)[crow * D + t] = reinterpret_cast<const uint16_t*>(row)[t];
    else
      reinterpret_cast<float*>(cent)[crow * D + t] = reinterpret_cast<const float*>(row)[t];
  }
}

__device__ __forceinline__ int ceil_log2(int n) {
  int L = 0;
  while ((1 << L) < n) L++;
  return L;
}

// Block reductions over 256 threads (4 waves).
__device__ __forceinline__ unsigned long long block_sum_u64(unsigned long long v,
                                                            unsigned long long* lds) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  const int wv = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) lds[wv] = v;
  __syncthreads();
  return lds[0] + lds[1] + lds[2] + lds[3];
}
__device__ __forceinline__ int block_min_i32(int v, int* lds) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = min(v, __shfl_xor(v, o, 64));
  const int wv = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) lds[wv] = v;
  __syncthreads();
  return min(min(lds[0], lds[1]), min(lds[2], lds[3]));
}
__device__ __forceinline__ float block_max_f32(float v, float* lds) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  const int wv = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) lds[wv] = v;
  __syncthreads();
  return fmaxf(fmaxf(lds[0], lds[1]), fmaxf(lds[2], lds[3]));
}

// F from the max distance after the first pick: max < 2^e, F = 62 - L - e.
__device__ __forceinline__ int weight_shift(float maxd, int n) {
  int e;
  frexpf(maxd, &e);
  return 62 - ceil_log2(n) - e;
}

__device__ __forceinline__ unsigned long long weight_of(float d, float maxd, int F) {
  if (!(maxd > 0.f)) return 0ull;
  return (unsigned long long)floor(ldexp((double)d, F));
}

// Round 0: first pick, distances to it, per-slice max distance.
template <int DT>
__global__ __launch_bounds__(NT) void kpp_init_kernel(Geom g, const void* __restrict__ K,
                                                       void* __restrict__ cent, BuildWs ws,
                                                       int nsl) {
  const int gs = blockIdx.y, slice = blockIdx.x;
  const int u = gs / g.n_seg, s = gs % g.n_seg;
  const int n = seg_n(g, s);
  if (slice * NT >= n) return;
  const int b = u / g.H, h = u % g.H;
  __shared__ float mu[D];
  __shared__ float red[4];
  const int i0 = (int)scale53(draw_key(g.seed, b, g.layer, h, s + g.seg_ord0, 0), (uint64_t)n);
  const int64_t first = seg_first(g, s);
  const void* r0 = krow<DT>(K, g, u, first + i0);
  load_mu<DT>(r0, mu);
  if (slice == 0) store_centroid<DT>(cent, (int64_t)u * g.C + seg_cbase(g, s), r0);
  __syncthreads();
  const int i = slice * NT + threadIdx.x;
  const int64_t pid = (int64_t)u * g.n_idx + (int64_t)s * g.seg_len + i;
  float d = 0.f;
  if (i < n) {
    // the chunk-major copy the rounds read: chunk c of point pid at vectors
    // (c * U n_idx + pid) * VPC ..
    constexpr int VPC = DT == WI_BF16 ? 4 : 8;
    const uint4* row = reinterpret_cast<const uint4*>(krow<DT>(K, g, u, first + i));
    uint4* kc = reinterpret_cast<uint4*>(ws.kc);
    const int64_t cstride = (int64_t)g.U * g.n_idx * VPC;
#pragma unroll
    for (int j = 0; j < 4 * VPC; j++) kc[(j / VPC) * cstride + pid * VPC + (j % VPC)] = row[j];
    d = dist32<DT>(row, mu);
    ws.D[pid] = d;
    ws.chosen[pid] = (i == i0);
  }
  const float mx = block_max_f32(d, red);
  if (threadIdx.x == 0) ws.kpp[(int64_t)gs * nsl + slice].maxd = mx;
}

// Weights of round 0 (parity 0) from the round-0 distances.
__global__ __launch_bounds__(NT) void kpp_weights_kernel(Geom g, BuildWs ws, int nsl) {
  const int gs = blockIdx.y, slice = blockIdx.x;
  const int s = gs % g.n_seg;
  const int n = seg_n(g, s);
  if (slice * NT >= n) return;
  const int u = gs / g.n_seg;
  __shared__ unsigned long long red64[4];
  __shared__ int redi[4];
  __shared__ float redf[4];
  const int ns = (n + NT - 1) / NT;
  float mx = threadIdx.x < ns ? ws.kpp[(int64_t)gs * nsl + threadIdx.x].maxd : 0.f;
  mx = block_max_f32(mx, redf);
  const int F = mx > 0.f ? weight_shift(mx, n) : 0;
  const int i = slice * NT + threadIdx.x;
  const int64_t pid = (int64_t)u * g.n_idx + (int64_t)s * g.seg_len + i;
  unsigned long long w = 0;
  int un = 0x7FFFFFFF;
  if (i < n) {
    w = weight_of(ws.D[pid], mx, F);
    ws.w[0][pid] = w;
    if (!ws.chosen[pid]) un = i;
  }
  const unsigned long long tot = block_sum_u64(w, red64);
  const int mun = block_min_i32(un, redi);
  if (threadIdx.x == 0) {
    ws.kpp[(int64_t)gs * nsl + slice].sum[0] = tot;
    ws.kpp[(int64_t)gs * nsl + slice].minun[0] = mun;
  }
}

// Round r >= 1: derive pick r from round r-1, update distances and weights.
// What does not depend on the pick (the point's distance, the first chunk of
// its row, the segment's slice partials) is requested first, so those reads
// overlap the pick's derivation.
template <int DT>
__global__ __launch_bounds__(NT, DT == WI_BF16 ? 8 : 5) void kpp_round_kernel(Geom g, const void* __restrict__ K,
                                                        void* __restrict__ cent, BuildWs ws,
                                                        int nsl, int r) {
  // XCD-aware placement: the dispatcher deals consecutive workgroups round
  // robin to the 8 XCDs; with a segment count that is a multiple of 8,
  // linear id L = 8 q + x runs segment (q / nsl) 8 + x, slice q % nsl, so the
  // slices of a segment share one L2 for the data every one of them reads to
  // derive the pick (slice sums, the owner slice's weights, the picked row)
  int gs, slice;
  if ((gridDim.y & 7) == 0) {
    const int L = (int)blockIdx.x + (int)blockIdx.y * (int)gridDim.x;
    const int q = L >> 3;
    gs = (q / (int)gridDim.x) * 8 + (L & 7);
    slice = q % (int)gridDim.x;
  } else {
    gs = blockIdx.y;
    slice = blockIdx.x;
  }
  const int s = gs % g.n_seg;
  const int n = seg_n(g, s);
  if (slice * NT >= n) return;
  if (r >= seg_c(g, s)) return;
  const int u = gs / g.n_seg;
  const int b = u / g.H, h = u % g.H;
  const int pin = (r - 1) & 1, pout = r & 1;
  const int ns = (n + NT - 1) / NT;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  __shared__ float mu[D];
  __shared__ unsigned long long red64[4];
  __shared__ unsigned long long wscan[4];
  __shared__ int redi[4];
  __shared__ float redf[4];
  __shared__ int pick_s;
  __shared__ unsigned long long tq_s;
  __shared__ int q_s;
  const KppPartial* kp = ws.kpp + (int64_t)gs * nsl;
  const int64_t first = seg_first(g, s);

  // pick-independent reads first
  const int i = slice * NT + tid;
  const bool in = i < n;
  const int64_t pid = (int64_t)u * g.n_idx + (int64_t)s * g.seg_len + i;
  constexpr int VPC = DT == WI_BF16 ? 4 : 8;
  const int64_t cstride = (int64_t)g.U * g.n_idx * VPC;
  const uint4* kc = reinterpret_cast<const uint4*>(ws.kc) + (in ? pid : 0) * VPC;
  const float dcur = in ? ws.D[pid] : 0.f;
  const Chunk<DT> c0 = load_chunk<DT>(kc, cstride, 0);
  const float mxl = tid < ns ? kp[tid].maxd : 0.f;
  const unsigned long long v = (wv == 0 && lane < ns) ? kp[lane].sum[pin] : 0ull;
  int mun = (wv == 0 && lane < ns) ? kp[lane].minun[pin] : 0x7FFFFFFF;

  const float mx = block_max_f32(mxl, redf);
  const int F = mx > 0.f ? weight_shift(mx, n) : 0;

  // total weight and owner slice (wave 0; ns <= 32 slices)
  if (wv == 0) {
    unsigned long long incl = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const unsigned long long y = __shfl_up(incl, o, 64);
      if (lane >= o) incl += y;
    }
    const unsigned long long W = __shfl(incl, 63, 64);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) mun = min(mun, __shfl_xor(mun, o, 64));
    if (W == 0ull) {
      if (lane == 0) {
        pick_s = mun;
        q_s = -1;
      }
    } else {
      const unsigned long long t = scale53(draw_key(g.seed, b, g.layer, h, s + g.seg_ord0, r), W);
      const bool hit = lane < ns && incl > t && (incl - v) <= t;
      if (hit) {
        q_s = lane;
        tq_s = t - (incl - v);
      }
    }
  }
  __syncthreads();
  const int q = q_s;
  if (q >= 0) {
    // smallest i in slice q whose inclusive prefix of weights exceeds tq
    const unsigned long long tq = tq_s;
    const int nq = min(NT, n - q * NT);
    const int64_t qbase = (int64_t)u * g.n_idx + (int64_t)s * g.seg_len + (int64_t)q * NT;
    const unsigned long long wq = tid < nq ? ws.w[pin][qbase + tid] : 0ull;
    unsigned long long incl = wq;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const unsigned long long y = __shfl_up(incl, o, 64);
      if (lane >= o) incl += y;
    }
    if (lane == 63) wscan[wv] = incl;
    __syncthreads();
    unsigned long long off = 0;
    for (int w2 = 0; w2 < wv; w2++) off += wscan[w2];
    incl += off;
    if (tid < nq && incl > tq && incl - wq <= tq) pick_s = q * NT + tid;
  }
  __syncthreads();
  const int pick = pick_s;
  const void* rp = krow<DT>(K, g, u, first + pick);
  load_mu<DT>(rp, mu);
  if (slice == 0) store_centroid<DT>(cent, (int64_t)u * g.C + seg_cbase(g, s) + r, rp);
  __syncthreads();

  unsigned long long w = 0;
  int un = 0x7FFFFFFF;
  if (in) {
    float d = dcur;
    // a point at distance 0 cannot get closer; skip its row
    const float dn = d > 0.f ? dist32_below<DT>(kc, cstride, c0, mu, d) : d;
    if (dn < d) {
      d = dn;
      ws.D[pid] = d;
    }
    bool ch = ws.chosen[pid];
    if (i == pick) {
      ch = true;
      ws.chosen[pid] = 1;
    }
    w = weight_of(d, mx, F);
    ws.w[pout][pid] = w;
    if (!ch) un = i;
  }
  const unsigned long long tot = block_sum_u64(w, red64);
  const int mn = block_min_i32(un, redi);
  if (tid == 0) {
    ws.kpp[(int64_t)gs * nsl + slice].sum[pout] = tot;
    ws.kpp[(int64_t)gs * nsl + slice].minun[pout] = mn;
  }
}

template <int DT>
hipError_t launch_kpp_dt(const Geom& g, const void* K, void* cent, const BuildWs& ws,
                         hipStream_t st) {
  const int nsl = (g.seg_len + NT - 1) / NT;
  dim3 grid(nsl, g.U * g.n_seg);
  WI_LAUNCH(K_KPP_INIT, (kpp_init_kernel<DT>), grid, dim3(NT), 0, st, g, K, cent, ws, nsl);
  WI_LAUNCH(K_KPP_WEIGHTS, kpp_weights_kernel, grid, dim3(NT), 0, st, g, ws, nsl);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  for (int r = 1; r < g.cmax; r++) {
    WI_LAUNCH(K_KPP_ROUND, (kpp_round_kernel<DT>), grid, dim3(NT), 0, st, g, K, cent, ws, nsl, r);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// Copy caller-given initial centroids into the centroid output.
__global__ void copy_kernel(const uint4* __restrict__ src, uint4* __restrict__ dst, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    dst[i] = src[i];
}

__global__ void zero_kernel(int* __restrict__ p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0;
}

}  // namespace

hipError_t launch_kpp(const Geom& g, const void* K, void* cent, const BuildWs& ws,
                      hipStream_t s) {
  return g.dtype == WI_BF16 ? launch_kpp_dt<WI_BF16>(g, K, cent, ws, s)
                            : launch_kpp_dt<WI_F32>(g, K, cent, ws, s);
}

hipError_t launch_copy_init(const Geom& g, const void* init, void* cent, hipStream_t s) {
  const int64_t bytes = (int64_t)g.U * g.C * D * (g.dtype == WI_BF16 ? 2 : 4);
  const int64_t n = bytes / 16;
  const int blocks = (int)std::min<int64_t>((n + 255) / 256, 4096);
  WI_LAUNCH(K_COPY, copy_kernel, dim3(blocks), dim3(256), 0, s,
                     reinterpret_cast<const uint4*>(init), reinterpret_cast<uint4*>(cent), n);
  return hipGetLastError();
}

hipError_t launch_zero_i32(int* p, int64_t n, hipStream_t s) {
  const int blocks = (int)std::min<int64_t>((n + 255) / 256, 1024);
  WI_LAUNCH(K_ZERO, zero_kernel, dim3(blocks > 0 ? blocks : 1), dim3(256), 0, s, p, n);
  return hipGetLastError();
}

}  // namespace wi
