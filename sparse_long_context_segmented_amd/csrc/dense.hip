// Dense decode attention: the full-attention layers of the per-layer zone
// policy (RetroInfer, framerc blog section 3.3: the lower layers of a large
// model keep full attention for precise localisation; section 4.3 problem 3:
// sparse attention switched off in the first two layers). Every context
// token of a KV head is attended by each of its query heads:
//   o_j = sum_i e^{z_i} v_i / sum_i e^{z_i},  z_i = scale <q_j, k_i>.
//
// HBM-bound streaming of the raw K/V rows (2 x 256 bytes per bf16 token).
// Split-K: workgroup (w, u) takes a contiguous chunk of unit u's tokens; its
// four waves walk 32-token blocks of the chunk (block wv, wv + 4, ...). Per
// block a wave computes the 32 x G logits with MFMA (tokens as rows, query
// heads as columns), updates a per-head online softmax, and adds
// sum_i p_i v_i with each lane owning two value dimensions. The waves'
// states are combined in LDS into one (m, l, acc[128]) partial per head and
// chunk; a second kernel merges the chunks of each (unit, head). Occupancy,
// not software pipelining, keeps loads in flight: every wave has a block of
// loads outstanding while others compute.
#include "wi_internal.h"

namespace wi {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int DN_THREADS = 256;
constexpr int DN_WAVES = DN_THREADS / 64;
constexpr int TB = 32;           // tokens per wave block
constexpr int PART = 2 + D;      // m, l, acc[128]

template <int DT>
__device__ __forceinline__ float ex(float x) {
  if constexpr (DT == WI_BF16) return __expf(x);
  else return expf(x);
}
__device__ __forceinline__ float rdlf(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

template <int DT, int GS>
__global__ __launch_bounds__(DN_THREADS) void dense_partial_kernel(
    const void* __restrict__ K, const void* __restrict__ V, const void* __restrict__ q,
    int64_t N, int64_t chunk, int H, int Hq, int G, int64_t sb, int64_t sh, int64_t st,
    float scale, float* __restrict__ part) {
  constexpr int EB = DT == WI_BF16 ? 2 : 4;  // bytes per element
  constexpr int NKL = DT == WI_BF16 ? 4 : 8;  // 16-byte key loads per lane per tile
  const int w = blockIdx.x, u = blockIdx.y, W = gridDim.x;
  const int b = u / H, h = u % H;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int r16 = lane & 15, kg = lane >> 4;
  __shared__ __align__(16) uint8_t qs[GS * D * EB];
  __shared__ float pb[DN_WAVES][TB * GS];
  __shared__ float wm[DN_WAVES][GS], wl[DN_WAVES][GS];
  __shared__ float wacc[DN_WAVES][GS][D];

  // the group's query rows (rows >= G are zero)
  {
    const uint8_t* qg = reinterpret_cast<const uint8_t*>(q) + ((int64_t)b * Hq + (int64_t)h * G) * D * EB;
    for (int e = tid; e < GS * D * EB / 16; e += DN_THREADS) {
      const int row = e / (D * EB / 16);
      reinterpret_cast<uint4*>(qs)[e] =
          row < G ? reinterpret_cast<const uint4*>(qg)[e] : make_uint4(0u, 0u, 0u, 0u);
    }
  }
  __syncthreads();
  uint4 bq[NKL];
#pragma unroll
  for (int s = 0; s < NKL; s++) {
    if constexpr (DT == WI_BF16)
      bq[s] = *reinterpret_cast<const uint4*>(qs + (r16 * D + 32 * s + 8 * kg) * 2);
    else
      bq[s] = *reinterpret_cast<const uint4*>(qs + (r16 * D + 32 * kg + 4 * s) * 4);
  }

  const int64_t t_lo = (int64_t)w * chunk;
  const int64_t t_hi = t_lo + chunk < N ? t_lo + chunk : N;
  const uint8_t* Kb = reinterpret_cast<const uint8_t*>(K) + ((int64_t)b * sb + (int64_t)h * sh) * EB;
  const uint8_t* Vb = reinterpret_cast<const uint8_t*>(V) + ((int64_t)b * sb + (int64_t)h * sh) * EB;
  const int64_t rs = st * EB;  // bytes between consecutive tokens

  float m_run = -INFINITY, l_run = 0.f;  // head r16 (l_run: this lane's share)
  float acc[GS][2];
#pragma unroll
  for (int g = 0; g < GS; g++) acc[g][0] = acc[g][1] = 0.f;

#pragma unroll 1
  for (int64_t t0 = t_lo + (int64_t)wv * TB; t0 < t_hi; t0 += (int64_t)DN_WAVES * TB) {
    const int nt = (int)(t_hi - t0 < TB ? t_hi - t0 : TB);
    // keys of tokens t0 + 16 j + r16 in the MFMA A layout; values: dims
    // 2 lane, 2 lane + 1 of every token (rows past the block read the first
    // token again and are masked)
    uint4 ka[2][NKL];
#pragma unroll
    for (int j = 0; j < 2; j++) {
      const int i = 16 * j + r16;
      const uint8_t* kp = Kb + (t0 + (i < nt ? i : 0)) * rs;
#pragma unroll
      for (int s = 0; s < NKL; s++) {
        if constexpr (DT == WI_BF16)
          ka[j][s] = *reinterpret_cast<const uint4*>(kp + (32 * s + 8 * kg) * 2);
        else
          ka[j][s] = *reinterpret_cast<const uint4*>(kp + (32 * kg + 4 * s) * 4);
      }
    }
    uint2 vr[TB];
#pragma unroll
    for (int t = 0; t < TB; t++) {
      const uint8_t* vp = Vb + (t0 + (t < nt ? t : 0)) * rs;
      if constexpr (DT == WI_BF16)
        vr[t].x = *reinterpret_cast<const uint32_t*>(vp + 4 * lane);
      else
        vr[t] = *reinterpret_cast<const uint2*>(vp + 8 * lane);
    }
    // logits z[token 16 j + 4 kg + jj][head r16]
    float zt[2][4];
#pragma unroll
    for (int j = 0; j < 2; j++) {
      f32x4_t za = {0.f, 0.f, 0.f, 0.f};
      if constexpr (DT == WI_BF16) {
#pragma unroll
        for (int s = 0; s < 4; s++)
          za = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, ka[j][s]),
                                                       __builtin_bit_cast(bf16x8_t, bq[s]), za,
                                                       0, 0, 0);
      } else {
#pragma unroll
        for (int s = 0; s < 8; s++) {
          const uint32_t kx[4] = {ka[j][s].x, ka[j][s].y, ka[j][s].z, ka[j][s].w};
          const uint32_t qx[4] = {bq[s].x, bq[s].y, bq[s].z, bq[s].w};
#pragma unroll
          for (int e = 0; e < 4; e++)
            za = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(kx[e]),
                                                      __uint_as_float(qx[e]), za, 0, 0, 0);
        }
      }
#pragma unroll
      for (int jj = 0; jj < 4; jj++)
        zt[j][jj] = (16 * j + 4 * kg + jj < nt && r16 < G) ? za[jj] * scale : -INFINITY;
    }
    // online softmax per head (column r16)
    float mx = m_run;
#pragma unroll
    for (int j = 0; j < 2; j++)
#pragma unroll
      for (int jj = 0; jj < 4; jj++) mx = fmaxf(mx, zt[j][jj]);
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float alpha = m_run == -INFINITY ? 0.f : ex<DT>(m_run - mx);
    m_run = mx;
    float ls = 0.f;
#pragma unroll
    for (int j = 0; j < 2; j++) {
#pragma unroll
      for (int jj = 0; jj < 4; jj++) {
        const float p = zt[j][jj] == -INFINITY ? 0.f : ex<DT>(zt[j][jj] - mx);
        ls += p;
        if (r16 < GS) pb[wv][(16 * j + 4 * kg + jj) * GS + r16] = p;
      }
    }
    l_run = fmaf(l_run, alpha, ls);
#pragma unroll
    for (int g = 0; g < GS; g++) {
      const float ag = rdlf(alpha, g);
      acc[g][0] *= ag;
      acc[g][1] *= ag;
    }
    // the weights written above are read back by every lane of the wave
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int t = 0; t < TB; t++) {
      float v0, v1;
      if constexpr (DT == WI_BF16) {
        v0 = __uint_as_float(vr[t].x << 16);
        v1 = __uint_as_float(vr[t].x & 0xFFFF0000u);
      } else {
        v0 = __uint_as_float(vr[t].x);
        v1 = __uint_as_float(vr[t].y);
      }
      const float* pt = &pb[wv][t * GS];
#pragma unroll
      for (int g = 0; g < GS; g++) {
        const float p = pt[g];
        acc[g][0] = fmaf(p, v0, acc[g][0]);
        acc[g][1] = fmaf(p, v1, acc[g][1]);
      }
    }
    // the next block rewrites the weights only after these reads
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
  // per-wave state: l summed over the four lanes of each head column
  float lt = l_run + __shfl_xor(l_run, 16, 64);
  lt += __shfl_xor(lt, 32, 64);
  if (lane < GS) {
    wm[wv][lane] = m_run;
    wl[wv][lane] = lt;
  }
#pragma unroll
  for (int g = 0; g < GS; g++) {
    wacc[wv][g][2 * lane] = acc[g][0];
    wacc[wv][g][2 * lane + 1] = acc[g][1];
  }
  __syncthreads();
  // combine the waves: one partial per head
  float* pw = part + ((int64_t)u * W + w) * G * PART;
  for (int e = tid; e < G * D; e += DN_THREADS) {
    const int g = e >> 7, t = e & (D - 1);
    float M = -INFINITY;
#pragma unroll
    for (int v = 0; v < DN_WAVES; v++) M = fmaxf(M, wm[v][g]);
    float s = 0.f, l = 0.f;
#pragma unroll
    for (int v = 0; v < DN_WAVES; v++) {
      const float f = wm[v][g] == -INFINITY ? 0.f : ex<DT>(wm[v][g] - M);
      s = fmaf(f, wacc[v][g][t], s);
      l = fmaf(f, wl[v][g], l);
    }
    pw[g * PART + 2 + t] = s;
    if (t == 0) {
      pw[g * PART] = M;
      pw[g * PART + 1] = l;
    }
  }
}

// One workgroup per (unit, head): merge the W chunk partials.
template <int DT>
__global__ __launch_bounds__(D) void dense_merge_kernel(const float* __restrict__ part, int W,
                                                        int G, int H, int Hq,
                                                        float* __restrict__ out) {
  const int u = blockIdx.x, g = blockIdx.y, t = threadIdx.x;
  const int b = u / H, h = u % H;
  const float* pu = part + (int64_t)u * W * G * PART + g * PART;
  float M = -INFINITY;
  for (int w = 0; w < W; w++) M = fmaxf(M, pu[(int64_t)w * G * PART]);
  float s = 0.f, l = 0.f;
  for (int w = 0; w < W; w++) {
    const float* p = pu + (int64_t)w * G * PART;
    const float m = p[0];
    const float f = m == -INFINITY ? 0.f : ex<DT>(m - M);
    l = fmaf(f, p[1], l);
    s = fmaf(f, p[2 + t], s);
  }
  out[((int64_t)b * Hq + (int64_t)h * G + g) * D + t] = s / l;
}

}  // namespace

int dense_chunks(int U, int64_t N) {
  int64_t W = (2048 + U - 1) / U;
  const int64_t by_len = (N + 255) / 256;  // at least 256 tokens per chunk
  if (W > by_len) W = by_len;
  if (W > 1024) W = 1024;
  if (W < 1) W = 1;
  return (int)W;
}

int64_t dense_part_floats(int U, int W, int G) { return (int64_t)U * W * G * PART; }

hipError_t launch_dense(int dtype, int B, int H, int Hq, int G, int64_t N, int64_t sb,
                        int64_t sh, int64_t st, float scale, const void* k, const void* v,
                        const void* q, float* out, float* part, hipStream_t s) {
  const int U = B * H;
  const int W = dense_chunks(U, N);
  // chunk length: a multiple of the wave block
  int64_t chunk = (N + W - 1) / W;
  chunk = (chunk + TB - 1) / TB * TB;
  const int GS = G <= 4 ? 4 : (G <= 8 ? 8 : 16);
  dim3 grid(W, U);
#define WI_DN(DTV, GSV)                                                                        \
  WI_LAUNCH(K_DENSE, (dense_partial_kernel<DTV, GSV>), grid, dim3(DN_THREADS), 0, s, k, v, q, \
            N, chunk, H, Hq, G, sb, sh, st, scale, part)
  if (dtype == WI_BF16) {
    if (GS == 4) WI_DN(WI_BF16, 4);
    else if (GS == 8) WI_DN(WI_BF16, 8);
    else WI_DN(WI_BF16, 16);
    WI_LAUNCH(K_DENSE_MERGE, dense_merge_kernel<WI_BF16>, dim3(U, G), dim3(D), 0, s, part, W,
              G, H, Hq, out);
  } else {
    if (GS == 4) WI_DN(WI_F32, 4);
    else if (GS == 8) WI_DN(WI_F32, 8);
    else WI_DN(WI_F32, 16);
    WI_LAUNCH(K_DENSE_MERGE, dense_merge_kernel<WI_F32>, dim3(U, G), dim3(D), 0, s, part, W,
              G, H, Hq, out);
  }
#undef WI_DN
  return hipGetLastError();
}

}  // namespace wi
