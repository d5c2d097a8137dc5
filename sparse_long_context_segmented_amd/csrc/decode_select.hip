// Decode step 2: pick the retrieval zone R (ranks [0, K_r)) and the
// estimation zone E (ranks [K_r, K_r + K_e)) of every unit (RetroInfer,
// framerc blog section 2.1: retrieval about 1.8 % of tokens, estimation the
// next 23 %; techwalker article section 3).
//
// Rank order: larger score first, lower cluster id on equal scores. One
// workgroup per unit runs an MSB-first radix select (4 passes of 8 bits) on
// the order-preserving 32-bit keys for both targets M1 = K_r and
// M2 = K_r + K_e at once, then resolves equal keys by id with a block scan.
// The outputs are compacted in ascending id order; R also gets the prefix
// sums of its cluster sizes, which the attention step uses to split the
// execution buffer evenly across workgroups.
#include "wi_internal.h"

namespace wi {
namespace {

constexpr int SEL_THREADS = 1024;
constexpr int SEL_WAVES = SEL_THREADS / 64;

// Exclusive block scan of one int per thread; returns the exclusive prefix
// and writes the block total to *total. Uses lds[SEL_WAVES + 1].
__device__ int block_excl_scan(int v, int* lds, int* total) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) lds[wv] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    int run = 0;
    for (int w = 0; w < SEL_WAVES; w++) {
      int t = lds[w];
      lds[w] = run;
      run += t;
    }
    lds[SEL_WAVES] = run;
  }
  __syncthreads();
  int r = lds[wv] + x - v;
  *total = lds[SEL_WAVES];
  __syncthreads();
  return r;
}

__global__ __launch_bounds__(SEL_THREADS) void select_kernel(
    const uint32_t* __restrict__ keys, const int32_t* __restrict__ sizes, int C, int M1,
    int M2, int K_e, int* __restrict__ Rout, int* __restrict__ Eout,
    int* __restrict__ Rpre) {
  const int u = blockIdx.x;
  const uint32_t* key = keys + (int64_t)u * C;
  __shared__ int hist[2][256];
  __shared__ uint32_t prefix[2];
  __shared__ int rem[2];
  __shared__ int scan_lds[SEL_WAVES + 1];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int M[2] = {M1, M2};
  if (tid < 2) {
    prefix[tid] = 0;
    rem[tid] = M[tid];
  }
  __syncthreads();

  for (int pass = 0; pass < 4; pass++) {
    const int shift = 24 - 8 * pass;
    for (int i = tid; i < 512; i += SEL_THREADS) (&hist[0][0])[i] = 0;
    __syncthreads();
    const uint32_t p0 = prefix[0], p1 = prefix[1];
    const uint32_t hmask = pass == 0 ? 0u : (0xFFFFFFFFu << (shift + 8));
    for (int c = tid; c < C; c += SEL_THREADS) {
      const uint32_t k = key[c];
      const int dg = (k >> shift) & 255;
      if (M1 > 0 && ((k ^ p0) & hmask) == 0) atomicAdd(&hist[0][dg], 1);
      if (M2 > 0 && ((k ^ p1) & hmask) == 0) atomicAdd(&hist[1][dg], 1);
    }
    __syncthreads();
    // wave t finds, for target t, the digit whose bucket holds rank rem[t]
    // counting from the largest keys down.
    if (wv < 2 && M[wv] > 0) {
      const int t = wv;
      // lane owns bins 255-4*lane .. 252-4*lane (descending)
      int cnt[4];
      int local = 0;
#pragma unroll
      for (int i = 0; i < 4; i++) {
        cnt[i] = hist[t][255 - 4 * lane - i];
        local += cnt[i];
      }
      int incl = local;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        int y = __shfl_up(incl, o, 64);
        if (lane >= o) incl += y;
      }
      int above = incl - local;  // keys in strictly larger bins of earlier lanes
      const int r = rem[t];
      if (above < r && r <= incl) {
        int run = above;
        for (int i = 0; i < 4; i++) {
          if (run + cnt[i] >= r) {
            prefix[t] |= (uint32_t)(255 - 4 * lane - i) << shift;
            rem[t] = r - run;
            break;
          }
          run += cnt[i];
        }
      }
    }
    __syncthreads();
  }

  const uint32_t T1 = prefix[0], T2 = prefix[1];
  const int rem1 = rem[0], rem2 = rem[1];
  // contiguous id ranges per thread, for id-ordered tie resolution and
  // compaction
  const int per = (C + SEL_THREADS - 1) / SEL_THREADS;
  const int i0 = min(C, tid * per), i1 = min(C, i0 + per);
  int eq1 = 0, eq2 = 0;
  for (int c = i0; c < i1; c++) {
    const uint32_t k = key[c];
    eq1 += (M1 > 0 && k == T1);
    eq2 += (M2 > 0 && k == T2);
  }
  int tot;
  int e1 = block_excl_scan(eq1, scan_lds, &tot);
  int e2 = block_excl_scan(eq2, scan_lds, &tot);
  int nR = 0, nE = 0;
  for (int c = i0; c < i1; c++) {
    const uint32_t k = key[c];
    bool inR = false, inS = false;
    if (M1 > 0) {
      if (k > T1) inR = true;
      else if (k == T1) inR = (e1++ < rem1);
    }
    if (M2 > 0) {
      if (k > T2) inS = true;
      else if (k == T2) inS = (e2++ < rem2);
    }
    nR += inR;
    nE += (inS && !inR);
  }
  int oR = block_excl_scan(nR, scan_lds, &tot);
  int oE = block_excl_scan(nE, scan_lds, &tot);
  // second walk writes; the equal-key counters restart from the same bases
  e1 = block_excl_scan(eq1, scan_lds, &tot);
  e2 = block_excl_scan(eq2, scan_lds, &tot);
  int* R = Rout + (int64_t)u * M1;
  int* E = Eout + (int64_t)u * K_e;
  const int32_t* sz = sizes + (int64_t)u * C;
  const int oR0 = oR;
  int sR = 0;
  for (int c = i0; c < i1; c++) {
    const uint32_t k = key[c];
    bool inR = false, inS = false;
    if (M1 > 0) {
      if (k > T1) inR = true;
      else if (k == T1) inR = (e1++ < rem1);
    }
    if (M2 > 0) {
      if (k > T2) inS = true;
      else if (k == T2) inS = (e2++ < rem2);
    }
    if (inR) {
      R[oR++] = c;
      sR += sz[c];
    } else if (inS) {
      E[oE++] = c;
    }
  }
  // prefix sums of R cluster sizes in R order (= ascending id = thread order)
  int* pre = Rpre + (int64_t)u * (M1 + 1);
  int sTot;
  int run = block_excl_scan(sR, scan_lds, &sTot);
  for (int i = oR0; i < oR; i++) {
    pre[i] = run;
    run += sz[R[i]];
  }
  if (tid == 0) pre[M1] = sTot;
  (void)lane;
  (void)wv;
}

}  // namespace

hipError_t launch_select(const DecodeArgs& a, const DecodeWs& ws, hipStream_t s) {
  const Geom& g = *a.g;
  WI_LAUNCH(K_SELECT, select_kernel, dim3(g.U), dim3(SEL_THREADS), 0, s, ws.key,
                     a.sizes, g.C, a.K_r, a.K_r + a.K_e, a.K_e, ws.R, ws.E, ws.Rpre);
  return hipGetLastError();
}

}  // namespace wi
