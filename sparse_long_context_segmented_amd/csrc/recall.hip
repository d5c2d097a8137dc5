// recall@k of a retrieval zone: the index-quality check of the per-layer
// policy (RetroInfer, framerc blog section 4.3 problem 1: recall@100 of the
// clustering should exceed 0.85). For query head j of unit u: the k
// clustered tokens with the largest scores <q_j, k_i> (ties to the lower
// position), and the share of them that lie in a cluster of the unit's
// retrieval zone.
//
// 1. recall_keys_kernel: every used slot of the index's key blocks is scored
//    against the group's query heads with MFMA (slots as rows, heads as
//    columns, float32 accumulation of exact bf16 products) and written as a
//    64-bit ranking key (order-preserving score bits above the complemented
//    position; padding slots get key 0, below every token).
// 2. recall_select_kernel, one workgroup per (unit, head): radix selection
//    of the k largest keys (11/11/10-bit digits from the top, LDS
//    histograms over the keys matching the prefix so far) until at most
//    CAND keys remain undecided; those and the keys already above the
//    prefix are collected and sorted in LDS; the cluster of each of the top
//    k tokens comes from the index's assignment.
#include "wi_internal.h"

namespace wi {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int RK_THREADS = 256;
constexpr int SEL_THREADS = 1024;
constexpr int NBIN = 2048;
constexpr int CAND = 2048;        // undecided keys collected at most
constexpr int MAX_TOPK = 1024;
constexpr int SORT_N = 4096;      // >= MAX_TOPK + CAND, a power of two

template <int DT, int GS>
__global__ __launch_bounds__(RK_THREADS) void recall_keys_kernel(
    const void* __restrict__ kblk, const int32_t* __restrict__ slot_token,
    const int32_t* __restrict__ block_off, const void* __restrict__ q, int C, int64_t capT,
    int T, int H, int Hq, int G, int64_t slots_per_wg, uint64_t* __restrict__ keys) {
  constexpr int EB = DT == WI_BF16 ? 2 : 4;
  constexpr int NKL = DT == WI_BF16 ? 4 : 8;
  constexpr int RB = D * EB;
  const int u = blockIdx.y;
  const int b = u / H, h = u % H;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int r16 = lane & 15, kg = lane >> 4;
  __shared__ __align__(16) uint8_t qs[GS * D * EB];
  {
    const uint8_t* qg = reinterpret_cast<const uint8_t*>(q) + ((int64_t)b * Hq + (int64_t)h * G) * D * EB;
    for (int e = tid; e < GS * D * EB / 16; e += RK_THREADS) {
      const int row = e / (D * EB / 16);
      reinterpret_cast<uint4*>(qs)[e] =
          row < G ? reinterpret_cast<const uint4*>(qg)[e] : make_uint4(0u, 0u, 0u, 0u);
    }
  }
  __syncthreads();
  uint4 bq[NKL];
  const int qrow = r16 < GS ? r16 : GS - 1;
#pragma unroll
  for (int s = 0; s < NKL; s++) {
    if constexpr (DT == WI_BF16)
      bq[s] = *reinterpret_cast<const uint4*>(qs + (qrow * D + 32 * s + 8 * kg) * 2);
    else
      bq[s] = *reinterpret_cast<const uint4*>(qs + (qrow * D + 32 * kg + 4 * s) * 4);
  }
  const int64_t used = (int64_t)block_off[(int64_t)u * (C + 1) + C] * T;
  const int64_t s_lo = (int64_t)blockIdx.x * slots_per_wg;
  const int64_t s_hi = s_lo + slots_per_wg < used ? s_lo + slots_per_wg : used;
  const uint8_t* kb = reinterpret_cast<const uint8_t*>(kblk) + (int64_t)u * capT * RB;
  const int32_t* stu = slot_token + (int64_t)u * capT;
#pragma unroll 1
  for (int64_t t0 = s_lo + 16 * wv; t0 < s_hi; t0 += 16 * (RK_THREADS / 64)) {
    const int64_t row = t0 + r16 < s_hi ? t0 + r16 : t0;
    const uint8_t* kp = kb + row * RB;
    uint4 ka[NKL];
#pragma unroll
    for (int s = 0; s < NKL; s++) {
      if constexpr (DT == WI_BF16)
        ka[s] = *reinterpret_cast<const uint4*>(kp + (32 * s + 8 * kg) * 2);
      else
        ka[s] = *reinterpret_cast<const uint4*>(kp + (32 * kg + 4 * s) * 4);
    }
    f32x4_t za = {0.f, 0.f, 0.f, 0.f};
    if constexpr (DT == WI_BF16) {
#pragma unroll
      for (int s = 0; s < 4; s++)
        za = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, ka[s]),
                                                     __builtin_bit_cast(bf16x8_t, bq[s]), za, 0,
                                                     0, 0);
    } else {
#pragma unroll
      for (int s = 0; s < 8; s++) {
        const uint32_t kx[4] = {ka[s].x, ka[s].y, ka[s].z, ka[s].w};
        const uint32_t qx[4] = {bq[s].x, bq[s].y, bq[s].z, bq[s].w};
#pragma unroll
        for (int e = 0; e < 4; e++)
          za = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(kx[e]),
                                                    __uint_as_float(qx[e]), za, 0, 0, 0);
      }
    }
    // lane (r16, kg) holds slots t0 + 4 kg + jj for head r16
    if (r16 < G) {
#pragma unroll
      for (int jj = 0; jj < 4; jj++) {
        const int64_t sl = t0 + 4 * kg + jj;
        if (sl < s_hi) {
          const int32_t pos = stu[sl];
          const uint64_t key =
              pos < 0 ? 0ull
                      : ((uint64_t)order_key(za[jj]) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)pos);
          keys[((int64_t)u * G + r16) * capT + sl] = key;
        }
      }
    }
  }
}

__device__ __forceinline__ int block_sum_i32(int v, int* lds) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  const int wv = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) lds[wv] = v;
  __syncthreads();
  int t = 0;
  for (int i = 0; i < SEL_THREADS / 64; i++) t += lds[i];
  return t;
}

__global__ __launch_bounds__(SEL_THREADS) void recall_select_kernel(
    const uint64_t* __restrict__ keys, const int32_t* __restrict__ block_off,
    const int32_t* __restrict__ assign, const int32_t* __restrict__ sel, int sel_stride,
    int n_r, int C, int64_t capT, int T, int n_sink, int64_t n_idx, int H, int Hq, int G, int k,
    float* __restrict__ recall, int32_t* __restrict__ top) {
  const int u = blockIdx.x, g = blockIdx.y, tid = threadIdx.x;
  const int b = u / H, h = u % H;
  __shared__ int hist[NBIN];
  __shared__ int red[SEL_THREADS / 64];
  __shared__ uint64_t cand[SORT_N];
  __shared__ uint32_t inR[2048];  // bit c: cluster c is retrieved (C <= 65536)
  __shared__ int s_bin, s_need, s_cnt;
  const int64_t used = (int64_t)block_off[(int64_t)u * (C + 1) + C] * T;
  const uint64_t* ku = keys + ((int64_t)u * G + g) * capT;

  // radix selection: prefix of `plen` fixed high bits
  uint64_t prefix = 0;
  int plen = 0, need = k;
  int64_t match = used;  // keys whose top plen bits equal the prefix
  const int dig[6] = {11, 11, 10, 11, 11, 10};
  for (int lev = 0; lev < 6 && match > CAND; lev++) {
    const int db = dig[lev];
    const int shift = 64 - plen - db;
    for (int i = tid; i < NBIN; i += SEL_THREADS) hist[i] = 0;
    __syncthreads();
    for (int64_t i = tid; i < used; i += SEL_THREADS) {
      const uint64_t x = ku[i];
      if (plen == 0 || (x >> (64 - plen)) == prefix)
        atomicAdd(&hist[(int)((x >> shift) & ((1u << db) - 1))], 1);
    }
    __syncthreads();
    if (tid == 0) {
      // from the top bin down: the bin holding the need-th largest key
      int above = 0, bsel = 0;
      for (int bi = (1 << db) - 1; bi >= 0; bi--) {
        if (above + hist[bi] >= need) {
          bsel = bi;
          break;
        }
        above += hist[bi];
      }
      s_bin = bsel;
      s_need = need - above;
      s_cnt = hist[bsel];
    }
    __syncthreads();
    prefix = (prefix << db) | (uint64_t)s_bin;
    plen += db;
    need = s_need;
    match = s_cnt;
    __syncthreads();
  }
  // collect the keys above the prefix (all taken) and those matching it
  if (tid == 0) s_cnt = 0;
  for (int i = tid; i < SORT_N; i += SEL_THREADS) cand[i] = 0ull;
  __syncthreads();
  for (int64_t i = tid; i < used; i += SEL_THREADS) {
    const uint64_t x = ku[i];
    const uint64_t top_bits = plen == 0 ? 0ull : x >> (64 - plen);
    if (plen == 0 || top_bits >= prefix) {
      const int at = atomicAdd(&s_cnt, 1);
      if (at < SORT_N) cand[at] = x;
    }
  }
  // the retrieval zone's clusters
  for (int i = tid; i < 2048; i += SEL_THREADS) inR[i] = 0u;
  __syncthreads();
  for (int r = tid; r < n_r; r += SEL_THREADS) {
    const int c = sel[(int64_t)u * sel_stride + r];
    if (c >= 0 && c < C) atomicOr(&inR[c >> 5], 1u << (c & 31));
  }
  // bitonic sort, descending
  for (int len = 2; len <= SORT_N; len <<= 1) {
    for (int st = len >> 1; st > 0; st >>= 1) {
      __syncthreads();
      for (int i = tid; i < SORT_N; i += SEL_THREADS) {
        const int j = i ^ st;
        if (j > i) {
          const bool desc = (i & len) == 0;
          const uint64_t a = cand[i], c2 = cand[j];
          if (desc ? a < c2 : a > c2) {
            cand[i] = c2;
            cand[j] = a;
          }
        }
      }
    }
  }
  __syncthreads();
  int hit = 0;
  const int64_t qi = (int64_t)b * Hq + (int64_t)h * G + g;
  for (int i = tid; i < k; i += SEL_THREADS) {
    const int32_t pos = (int32_t)(0xFFFFFFFFu - (uint32_t)(cand[i] & 0xFFFFFFFFull));
    if (top) top[qi * k + i] = pos;
    const int64_t li = (int64_t)pos - n_sink;
    const int c = (li >= 0 && li < n_idx) ? assign[(int64_t)u * n_idx + li] : -1;
    if (c >= 0 && c < C && ((inR[c >> 5] >> (c & 31)) & 1u)) hit++;
  }
  hit = block_sum_i32(hit, red);
  if (tid == 0) recall[qi] = (float)hit / (float)k;
}

}  // namespace

int recall_max_k() { return MAX_TOPK; }

hipError_t launch_recall(const Geom& g, int Hq, int G, const wi_index_bufs& bf, const void* q,
                         const int32_t* sel, int sel_stride, int n_r, int k, float* recall,
                         int32_t* top, uint64_t* keys, hipStream_t s) {
  const int64_t capT = g.cap * g.T;
  // slots per workgroup: about 2048 workgroups over the call, >= 256 slots
  int64_t per = (capT * g.U + 2047) / 2048;
  if (per < 256) per = 256;
  per = (per + 63) / 64 * 64;
  const int nch = (int)((capT + per - 1) / per);
  const int GS = G <= 4 ? 4 : (G <= 8 ? 8 : 16);
  dim3 grid(nch, g.U);
#define WI_RK(DTV, GSV)                                                                       \
  WI_LAUNCH(K_RECALL, (recall_keys_kernel<DTV, GSV>), grid, dim3(RK_THREADS), 0, s, bf.k_blocks, \
            bf.slot_token, bf.block_off, q, g.C, capT, g.T, g.H, Hq, G, per, keys)
  if (g.dtype == WI_BF16) {
    if (GS == 4) WI_RK(WI_BF16, 4);
    else if (GS == 8) WI_RK(WI_BF16, 8);
    else WI_RK(WI_BF16, 16);
  } else {
    if (GS == 4) WI_RK(WI_F32, 4);
    else if (GS == 8) WI_RK(WI_F32, 8);
    else WI_RK(WI_F32, 16);
  }
#undef WI_RK
  WI_LAUNCH(K_RECALL, recall_select_kernel, dim3(g.U, G), dim3(SEL_THREADS), 0, s, keys,
            bf.block_off, bf.assign, sel, sel_stride, n_r, g.C, capT, g.T, g.n_sink, g.n_idx,
            g.H, Hq, G, k, recall, top);
  return hipGetLastError();
}

}  // namespace wi
