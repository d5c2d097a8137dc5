// Decode step 2: pick the retrieval zone R (ranks [0, K_r)) and the
// estimation zone E (ranks [K_r, K_r + K_e)) of every unit (RetroInfer,
// framerc blog section 2.1: retrieval about 1.8 % of tokens, estimation the
// next 23 %; techwalker article section 3).
//
// Rank order: larger key first, lower cluster id on equal keys. One
// workgroup per unit; every thread keeps PER consecutive keys in registers.
//   1. min / max of the key values, then a 2048-bin histogram with bins
//      linear in value (monotone, so rank ranges map to bin ranges, and it
//      spreads the keys evenly where fp32-bit digits would pile them into a
//      few bins);
//   2. a block scan over the bins (largest first) finds, for each target M
//      (K_r and K_r + K_e), the boundary bin and how many of its keys are
//      needed;
//   3. keys of a boundary bin are gathered in LDS and ranked exactly among
//      themselves by (key, id) in parallel; the chosen ones are marked in an
//      LDS bitmap (a slow out-of-line path handles boundary bins too large to
//      gather);
//   4. one block scan compacts R and E in ascending id order, with the prefix
//      sums of the R cluster sizes, the first block of each R cluster and the
//      size of each E cluster;
//   5. the workgroup fills the execution-buffer row table (the slot of every
//      retrieved token) cooperatively, one retrieved cluster per wave.
// The per-key loops are fully unrolled, so they carry only bit logic; loops
// with data-dependent trip counts stay rolled.
#include "wi_internal.h"

namespace wi {
namespace {

constexpr int SEL_THREADS = 1024;
constexpr int SEL_WAVES = SEL_THREADS / 64;
constexpr int NBINS = 2048;
constexpr int CAND_MAX = 2048;
constexpr int MAX_C = 65536;

__device__ __forceinline__ float key_value(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k ^ 0x80000000u) : ~k);
}

__device__ __forceinline__ int bin_of(uint32_t k, float lo, float inv) {
  return min(NBINS - 1, (int)((key_value(k) - lo) * inv));
}

// Exclusive block scans of two 64-bit values with one pair of barriers.
__device__ uint64_t block_scan2_u64(uint64_t v, uint64_t v2, uint64_t* lds, uint64_t* total,
                                    uint64_t* off2, uint64_t* total2) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  uint64_t x = v, x2 = v2;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint64_t y = __shfl_up(x, o, 64);
    const uint64_t y2 = __shfl_up(x2, o, 64);
    if (lane >= o) {
      x += y;
      x2 += y2;
    }
  }
  if (lane == 63) {
    lds[wv] = x;
    lds[SEL_WAVES + wv] = x2;
  }
  __syncthreads();
  uint64_t off = 0, tot = 0, o2 = 0, t2 = 0;
#pragma unroll
  for (int w = 0; w < SEL_WAVES; w++) {
    const uint64_t t = lds[w], tt = lds[SEL_WAVES + w];
    if (w < wv) {
      off += t;
      o2 += tt;
    }
    tot += t;
    t2 += tt;
  }
  __syncthreads();
  *total = tot;
  *total2 = t2;
  *off2 = o2 + x2 - v2;
  return off + x - v;
}

// Boundary bin too large to gather: every thread ranks its own keys of the
// bin against all keys of the unit read from memory (slow; only reached when
// more than CAND_MAX keys share one value bin).
__device__ __noinline__ void rank_boundary_slow(const uint32_t* key, int C, int i0, int nv,
                                                float lo, float inv, int bsel, int need,
                                                unsigned int* bits) {
#pragma unroll 1
  for (int i = 0; i < nv; i++) {
    const int id = i0 + i;
    const uint32_t k = key[id];
    if (bin_of(k, lo, inv) != bsel) continue;
    int rank = 0;
#pragma unroll 1
    for (int c2 = 0; c2 < C; c2++) {
      const uint32_t k2 = key[c2];
      rank += (bin_of(k2, lo, inv) == bsel) && ((k2 > k) || (k2 == k && c2 < id));
    }
    if (rank < need) atomicOr(&bits[id >> 5], 1u << (id & 31));
  }
}

template <int PER>
__global__ __launch_bounds__(SEL_THREADS) void select_kernel(
    const uint32_t* __restrict__ keys, const int32_t* __restrict__ sizes,
    const int32_t* __restrict__ block_off, int C, int M1, int M2, int K_e, int T,
    int64_t n_idx, int* __restrict__ Rout, int* __restrict__ Rblk, int* __restrict__ Rpre,
    int* __restrict__ Eout, int* __restrict__ Esz, int* __restrict__ rowtab) {
  const int u = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const uint32_t* key = keys + (int64_t)u * C;
  const int32_t* sz = sizes + (int64_t)u * C;
  const int32_t* bo = block_off + (int64_t)u * (C + 1);
  __shared__ int hist[NBINS];
  __shared__ float redf[2][SEL_WAVES];
  __shared__ uint64_t red64[2 * SEL_WAVES];
  __shared__ int bsel[2], bneed[2], ncand[2];
  __shared__ uint32_t candk[2][CAND_MAX];
  __shared__ int candi[2][CAND_MAX];
  __shared__ unsigned int bits[2][MAX_C / 32];

  // keys, sizes and first blocks of this thread's ids [i0, i0 + PER)
  const int i0 = tid * PER;
  uint32_t k[PER];
  int szr[PER], bor[PER];
#pragma unroll
  for (int i = 0; i < PER; i += 4) {
    if (i0 + i + 3 < C) {
      const uint4 v = *reinterpret_cast<const uint4*>(key + i0 + i);
      const int4 z = *reinterpret_cast<const int4*>(sz + i0 + i);
      k[i] = v.x; k[i + 1] = v.y; k[i + 2] = v.z; k[i + 3] = v.w;
      szr[i] = z.x; szr[i + 1] = z.y; szr[i + 2] = z.z; szr[i + 3] = z.w;
#pragma unroll
      for (int e = 0; e < 4; e++) bor[i + e] = bo[i0 + i + e];
    } else {
#pragma unroll
      for (int e = 0; e < 4; e++) {
        const bool ok = i0 + i + e < C;
        k[i + e] = ok ? key[i0 + i + e] : 0u;
        szr[i + e] = ok ? sz[i0 + i + e] : 0;
        bor[i + e] = ok ? bo[i0 + i + e] : 0;
      }
    }
  }
  const int nv = max(0, min(PER, C - i0));  // valid keys of this thread

  // 1. value range and histogram
  float lo = INFINITY, hi = -INFINITY;
#pragma unroll
  for (int i = 0; i < PER; i++) {
    if (i < nv) {
      const float f = key_value(k[i]);
      lo = fminf(lo, f);
      hi = fmaxf(hi, f);
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    lo = fminf(lo, __shfl_xor(lo, o, 64));
    hi = fmaxf(hi, __shfl_xor(hi, o, 64));
  }
  for (int i = tid; i < NBINS; i += SEL_THREADS) hist[i] = 0;
  for (int i = tid; i < 2 * ((C + 31) / 32); i += SEL_THREADS) {
    const int t = i / ((C + 31) / 32), w = i % ((C + 31) / 32);
    bits[t][w] = 0u;
  }
  if (tid < 2) ncand[tid] = 0;
  if (lane == 0) {
    redf[0][wv] = lo;
    redf[1][wv] = hi;
  }
  __syncthreads();
#pragma unroll
  for (int w = 0; w < SEL_WAVES; w++) {
    lo = fminf(lo, redf[0][w]);
    hi = fmaxf(hi, redf[1][w]);
  }
  const float inv = hi > lo ? (float)NBINS / (hi - lo) : 0.f;
  int bin[PER];
#pragma unroll
  for (int i = 0; i < PER; i++) {
    bin[i] = bin_of(k[i], lo, inv);
    if (i < nv) atomicAdd(&hist[bin[i]], 1);
  }
  __syncthreads();

  // 2. boundary bins: thread t owns bins NBINS-1-2t and NBINS-2-2t
  {
    const int ha = hist[NBINS - 1 - 2 * tid], hb = hist[NBINS - 2 - 2 * tid];
    uint64_t tot, o2, t2;
    const uint64_t above = block_scan2_u64((uint64_t)(ha + hb), 0, red64, &tot, &o2, &t2);
    const int M[2] = {M1, M2};
#pragma unroll
    for (int t = 0; t < 2; t++) {
      const int m = M[t];
      if (m > 0 && (int)above < m && m <= (int)above + ha + hb) {
        if (m <= (int)above + ha) {
          bsel[t] = NBINS - 1 - 2 * tid;
          bneed[t] = m - (int)above;
        } else {
          bsel[t] = NBINS - 2 - 2 * tid;
          bneed[t] = m - (int)above - ha;
        }
      }
    }
    if (tid == 0) {
      if (M1 == 0) { bsel[0] = NBINS; bneed[0] = 0; }
      if (M2 == 0) { bsel[1] = NBINS; bneed[1] = 0; }
    }
  }
  __syncthreads();
  const int b1 = bsel[0], b2 = bsel[1];

  // 3. boundary-bin candidates, ranked in parallel into the bitmaps
#pragma unroll
  for (int i = 0; i < PER; i++) {
    if (i < nv) {
      if (bin[i] == b1) {
        const int s = atomicAdd(&ncand[0], 1);
        if (s < CAND_MAX) { candk[0][s] = k[i]; candi[0][s] = i0 + i; }
      }
      if (bin[i] == b2) {
        const int s = atomicAdd(&ncand[1], 1);
        if (s < CAND_MAX) { candk[1][s] = k[i]; candi[1][s] = i0 + i; }
      }
    }
  }
  __syncthreads();
#pragma unroll 1
  for (int t = 0; t < 2; t++) {
    const int nc = ncand[t], need = bneed[t];
    if (nc <= CAND_MAX) {
#pragma unroll 1
      for (int s = tid; s < nc; s += SEL_THREADS) {
        const uint32_t kk = candk[t][s];
        const int id = candi[t][s];
        int rank = 0;
#pragma unroll 1
        for (int j2 = 0; j2 < nc; j2++) {
          const uint32_t k2 = candk[t][j2];
          rank += (k2 > kk) || (k2 == kk && candi[t][j2] < id);
        }
        if (rank < need) atomicOr(&bits[t][id >> 5], 1u << (id & 31));
      }
    } else {
      rank_boundary_slow(key, C, i0, nv, lo, inv, bsel[t], need, bits[t]);
    }
  }
  __syncthreads();

  // own selection flags
  uint64_t selR = 0, selS = 0;
#pragma unroll
  for (int i = 0; i < PER; i++) {
    const int id = i0 + i;
    if (i < nv) {
      const bool r1 = bin[i] > b1 || (bin[i] == b1 && ((bits[0][id >> 5] >> (id & 31)) & 1u));
      const bool r2 = bin[i] > b2 || (bin[i] == b2 && ((bits[1][id >> 5] >> (id & 31)) & 1u));
      selR |= (uint64_t)r1 << i;
      selS |= (uint64_t)r2 << i;
    }
  }
  const uint64_t selE = selS & ~selR;

  // 4. compaction in ascending id order
  int sR = 0;
#pragma unroll
  for (int i = 0; i < PER; i++) sR += ((selR >> i) & 1) ? szr[i] : 0;
  uint64_t tot, stot, soff;
  const uint64_t off = block_scan2_u64((uint64_t)__popcll(selR) | ((uint64_t)__popcll(selE) << 32),
                                       (uint64_t)sR, red64, &tot, &soff, &stot);
  int oR = (int)(off & 0xFFFFFFFFu), oE = (int)(off >> 32);
  int* R = Rout + (int64_t)u * M1;
  int* RB = Rblk + (int64_t)u * M1;
  int* RP = Rpre + (int64_t)u * (M1 + 1);
  int* E = Eout + (int64_t)u * K_e;
  int* ES = Esz + (int64_t)u * K_e;
  int run = (int)soff;
#pragma unroll
  for (int i = 0; i < PER; i++) {
    if ((selR >> i) & 1) {
      R[oR] = i0 + i;
      RB[oR] = bor[i];
      RP[oR] = run;
      run += szr[i];
      oR++;
    }
    if ((selE >> i) & 1) {
      E[oE] = i0 + i;
      ES[oE] = szr[i];
      oE++;
    }
  }
  if (tid == 0) RP[M1] = (int)stot;
  __syncthreads();

  // 5. execution-buffer row table: one retrieved cluster per wave
  int* rt = rowtab + (int64_t)u * n_idx;
#pragma unroll 1
  for (int r = wv; r < M1; r += SEL_WAVES) {
    const int b0 = RB[r], p0 = RP[r], n = RP[r + 1] - p0;
#pragma unroll 1
    for (int jj = lane; jj < n; jj += 64) rt[p0 + jj] = b0 * T + jj;
  }
}

}  // namespace

hipError_t launch_select(const DecodeArgs& a, const wi_index_bufs& b, const DecodeWs& ws,
                         hipStream_t s) {
  const Geom& g = *a.g;
  const int per = (g.C + SEL_THREADS - 1) / SEL_THREADS;
#define WI_SEL(PV)                                                                        \
  WI_LAUNCH(K_SELECT, select_kernel<PV>, dim3(g.U), dim3(SEL_THREADS), 0, s, ws.key,      \
            b.cluster_size, b.block_off, g.C, a.K_r, a.K_r + a.K_e, a.K_e, g.T, g.n_idx,   \
            ws.R, ws.Rblk, ws.Rpre, ws.E, ws.Esz, ws.rowtab)
  if (per <= 4) WI_SEL(4);
  else if (per <= 8) WI_SEL(8);
  else if (per <= 16) WI_SEL(16);
  else if (per <= 32) WI_SEL(32);
  else WI_SEL(64);
#undef WI_SEL
  return hipGetLastError();
}

}  // namespace wi
