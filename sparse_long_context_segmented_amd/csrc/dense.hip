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
// chunk; a second kernel merges the chunks of each (unit, head). Each wave
// issues the loads of its next block before computing the current one.
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
  // B operand: column r16 = query head r16 (columns >= GS repeat the last
  // staged row and are masked with the heads >= G)
  uint4 bq[NKL];
  const int qrow = r16 < GS ? r16 : GS - 1;
#pragma unroll
  for (int s = 0; s < NKL; s++) {
    if constexpr (DT == WI_BF16)
      bq[s] = *reinterpret_cast<const uint4*>(qs + (qrow * D + 32 * s + 8 * kg) * 2);
    else
      bq[s] = *reinterpret_cast<const uint4*>(qs + (qrow * D + 32 * kg + 4 * s) * 4);
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

  // one wave block: keys of tokens t0 + 16 j + r16 in the MFMA A layout,
  // values (dims 2 lane, 2 lane + 1) of every token; rows past the block read
  // the block's first token again and are masked
  struct Blk {
    uint4 ka[TB / 16][NKL];
    uint2 vr[TB];
  };
  auto load_blk = [&](Blk& B, int64_t t0) {
    const int nt = (int)(t_hi - t0 < TB ? t_hi - t0 : TB);
#pragma unroll
    for (int j = 0; j < TB / 16; j++) {
      const int i = 16 * j + r16;
      const uint8_t* kp = Kb + (t0 + (i < nt ? i : 0)) * rs;
#pragma unroll
      for (int s = 0; s < NKL; s++) {
        if constexpr (DT == WI_BF16)
          B.ka[j][s] = *reinterpret_cast<const uint4*>(kp + (32 * s + 8 * kg) * 2);
        else
          B.ka[j][s] = *reinterpret_cast<const uint4*>(kp + (32 * kg + 4 * s) * 4);
      }
    }
#pragma unroll
    for (int t = 0; t < TB; t++) {
      const uint8_t* vp = Vb + (t0 + (t < nt ? t : 0)) * rs;
      if constexpr (DT == WI_BF16)
        B.vr[t].x = *reinterpret_cast<const uint32_t*>(vp + 4 * lane);
      else
        B.vr[t] = *reinterpret_cast<const uint2*>(vp + 8 * lane);
    }
  };
  auto compute_blk = [&](const Blk& B, int64_t t0) {
    const int nt = (int)(t_hi - t0 < TB ? t_hi - t0 : TB);
    // logits z[token 16 j + 4 kg + jj][head r16]
    float zt[TB / 16][4];
#pragma unroll
    for (int j = 0; j < TB / 16; j++) {
      f32x4_t za = {0.f, 0.f, 0.f, 0.f};
      if constexpr (DT == WI_BF16) {
#pragma unroll
        for (int s = 0; s < 4; s++)
          za = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, B.ka[j][s]),
                                                       __builtin_bit_cast(bf16x8_t, bq[s]), za,
                                                       0, 0, 0);
      } else {
#pragma unroll
        for (int s = 0; s < 8; s++) {
          const uint32_t kx[4] = {B.ka[j][s].x, B.ka[j][s].y, B.ka[j][s].z, B.ka[j][s].w};
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
    for (int j = 0; j < TB / 16; j++)
#pragma unroll
      for (int jj = 0; jj < 4; jj++) mx = fmaxf(mx, zt[j][jj]);
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float alpha = m_run == -INFINITY ? 0.f : ex<DT>(m_run - mx);
    m_run = mx;
    float ls = 0.f;
#pragma unroll
    for (int j = 0; j < TB / 16; j++) {
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
        v0 = __uint_as_float(B.vr[t].x << 16);
        v1 = __uint_as_float(B.vr[t].x & 0xFFFF0000u);
      } else {
        v0 = __uint_as_float(B.vr[t].x);
        v1 = __uint_as_float(B.vr[t].y);
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
  };

  // two register buffers, alternating: the next block's loads are issued
  // before the current block is computed
  const int64_t step = (int64_t)DN_WAVES * TB;
  Blk A, B;
  int64_t t0 = t_lo + (int64_t)wv * TB;
  if (t0 < t_hi) load_blk(A, t0);
#pragma unroll 1
  while (t0 < t_hi) {
    const int64_t t1 = t0 + step;
    if (t1 < t_hi) load_blk(B, t1);
    compute_blk(A, t0);
    if (t1 >= t_hi) break;
    const int64_t t2 = t1 + step;
    if (t2 < t_hi) load_blk(A, t2);
    compute_blk(B, t1);
    t0 = t2;
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

// One workgroup per (unit, head): merge the W chunk partials. The maxima,
// weights and denominators are formed over all chunks in parallel (weights
// kept in LDS), then each half of the workgroup sums the weighted
// accumulators of every other chunk for one output dimension per thread.
constexpr int MG_THREADS = 256;
constexpr int MAX_CHUNKS = 1024;

__device__ __forceinline__ float block_reduce(float v, float* lds, bool is_max) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float y = __shfl_xor(v, o, 64);
    v = is_max ? fmaxf(v, y) : v + y;
  }
  __syncthreads();
  if ((threadIdx.x & 63) == 0) lds[threadIdx.x >> 6] = v;
  __syncthreads();
  float r = lds[0];
  for (int i = 1; i < MG_THREADS / 64; i++) r = is_max ? fmaxf(r, lds[i]) : r + lds[i];
  return r;
}

template <int DT>
__global__ __launch_bounds__(MG_THREADS) void dense_merge_kernel(const float* __restrict__ part,
                                                                 int W, int G, int H, int Hq,
                                                                 float* __restrict__ out) {
  const int u = blockIdx.x, g = blockIdx.y, tid = threadIdx.x;
  const int b = u / H, h = u % H;
  __shared__ float fw[MAX_CHUNKS];
  __shared__ float red[MG_THREADS / 64];
  __shared__ float half_acc[D];
  const float* pu = part + (int64_t)u * W * G * PART + g * PART;
  float M = -INFINITY;
  for (int w = tid; w < W; w += MG_THREADS) M = fmaxf(M, pu[(int64_t)w * G * PART]);
  M = block_reduce(M, red, true);
  float l = 0.f;
  for (int w = tid; w < W; w += MG_THREADS) {
    const float* p = pu + (int64_t)w * G * PART;
    const float f = p[0] == -INFINITY ? 0.f : ex<DT>(p[0] - M);
    fw[w] = f;
    l = fmaf(f, p[1], l);
  }
  l = block_reduce(l, red, false);  // its barriers also publish fw
  const int t = tid & (D - 1), hf = tid >> 7;
  float s = 0.f;
#pragma unroll 8
  for (int w = hf; w < W; w += 2) s = fmaf(fw[w], pu[(int64_t)w * G * PART + 2 + t], s);
  if (hf == 1) half_acc[t] = s;
  __syncthreads();
  if (hf == 0) out[((int64_t)b * Hq + (int64_t)h * G + g) * D + t] = (s + half_acc[t]) / l;
}

}  // namespace

// About 1024 workgroups over the call (four per compute unit): enough waves
// to keep HBM busy, few enough chunk partials for a short merge.
int dense_chunks(int U, int64_t N) {
  int64_t W = (1024 + U - 1) / U;
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
    WI_LAUNCH(K_DENSE_MERGE, dense_merge_kernel<WI_BF16>, dim3(U, G), dim3(MG_THREADS), 0, s,
              part, W, G, H, Hq, out);
  } else {
    if (GS == 4) WI_DN(WI_F32, 4);
    else if (GS == 8) WI_DN(WI_F32, 8);
    else WI_DN(WI_F32, 16);
    WI_LAUNCH(K_DENSE_MERGE, dense_merge_kernel<WI_F32>, dim3(U, G), dim3(MG_THREADS), 0, s,
              part, W, G, H, Hq, out);
  }
#undef WI_DN
  return hipGetLastError();
}

}  // namespace wi
