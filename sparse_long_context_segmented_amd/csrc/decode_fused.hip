// Decode steps 2-6 in one launch: select the retrieval and estimation zones,
// gather the execution buffer, exact attention over the steady and
// retrieval zones, the estimation-zone partial, and the log-sum-exp merge
// (RetroInfer, framerc blog section 2.1: retrieval about 1.8 % of tokens,
// estimation the next 23 %; section 3.2: execution buffer = steady zone +
// retrieved blocks with block fragments skipped; section 3.3: estimation from
// centroid vectors and cluster sizes, partial results merged by a custom
// kernel; techwalker article section 3).
//
// Grid: W workgroups of 512 threads per unit (sequence, KV head). At batch 1
// a decode step is a few tens of MB, so the kernel is bound by dependent
// latencies, not bandwidth: every phase is written to keep the per-wave
// instruction chain short (DPP row operations and lane reads instead of LDS
// shuffles, shifts instead of divisions, matrix cores for the logits).
//
//  1. Selection, repeated by every workgroup of the unit on chip (the C
//     ranking keys are a few tens of KB; recomputing them beats a separate
//     launch). Rank order is larger key first, lower cluster id on equal
//     keys. For M in {K_r, K_r + K_e'} the M-th ranked cluster -- the pivot
//     (k*, i*) -- is found, and cluster c is among the first M iff
//     key_c > k* or (key_c = k* and c <= i*). A 2048-bin histogram linear in
//     key value (bins monotone in the key) locates the pivot's bin; its keys
//     (at most CAND_MAX) are ranked exactly by one wave. A fuller bin falls
//     back to an 8-pass radix select over the 64-bit composite (key, ~id)
//     restricted to that bin.
//  2. Compaction. One block scan in cluster-id order gives every retrieved
//     cluster with members its first token in the concatenated retrieval
//     zone and its first block (the sum of ceil(n_c / T) over lower ids,
//     which is how the index lays blocks out), and every estimation cluster
//     its position. Both lists (the estimation one only for this
//     workgroup's share) go to LDS.
//  3. Items, in rounds of up to 16 tokens and 16 estimation clusters per
//     wave. The execution buffer (n_st steady tokens, then every retrieved
//     cluster's members, fragments skipped) and the estimation list are
//     split evenly over the W workgroups. Logits: a wave computes its 16
//     tokens x 16 query-head columns with v_mfma 16x16 (bf16 keys: exact
//     products, fp32 sums), and reads the estimation clusters' logits from
//     the score step. The workgroup then takes one maximum per head over the
//     round, turns logits into weights p (estimation cluster c counts n_c
//     times in the denominator), and every lane accumulates two dims of
//     sum_i p_i v_i per head (token values, or the value sums VS_c).
//  4. Merge: waves add their accumulators in a fixed order; the workgroup's
//     (m, l, acc) per head is published with agent-coherent stores, then one
//     relaxed atomic counts arrivals; the last workgroup of the unit reads
//     the W partials and writes out = sum_w e^{m_w-M} acc_w / sum_w e^{m_w-M} l_w.
// Every sum runs in a fixed order, so results are bit-reproducible.
#include <climits>

#include "wi_internal.h"

namespace wi {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int NT = 512;        // threads per workgroup
constexpr int NW = NT / 64;    // waves
constexpr int NBINS = 2048;
constexpr int BPT = NBINS / NT;
constexpr int CAND_MAX = 64;   // pivot-bin keys ranked by one wave
constexpr int ROUND = 16 * NW; // token (and estimation) items per round
constexpr int PART = 2 + D;    // m, l, acc[128]

struct FusedArgs {
  const uint32_t* key;   // [U][Cp] ranking keys
  const float* S;        // [U][C][GS] scaled per-head logits
  const int32_t* sizes;  // [U][C]
  const void* kblk;
  const void* vblk;
  const void* stk;
  const void* stv;
  const float* vsum;
  const void* q;
  float* out;
  float* part;           // [U][W][G][PART]
  int* tix;              // [U] arrival counters, zero on entry
  int* dbgR;             // nullable: [U][K_r] retrieval ids, ascending
  int* dbgE;             // nullable: [U][K_e] estimation ids, ascending
  int C, Cp, n_st, G, H, Hq, K_r, K_e, W, lgT;
  int64_t capT;
  float scale;
};

// ---- wave primitives ------------------------------------------------------
__device__ __forceinline__ int rdl(int v, int l) { return __builtin_amdgcn_readlane(v, l); }
__device__ __forceinline__ float rdlf(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

// Inclusive prefix sum over the 64 lanes: row_shr 1, 2, 4, 8 inside rows of
// 16 lanes, then the row totals read from lanes 15, 31, 47.
__device__ __forceinline__ int wave_incl_scan(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, true);
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, true);
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, true);
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, true);
  const int row = __lane_id() >> 4;
  const int s0 = rdl(x, 15), s1 = rdl(x, 31), s2 = rdl(x, 47);
  return x + (row >= 1 ? s0 : 0) + (row >= 2 ? s1 : 0) + (row >= 3 ? s2 : 0);
}

// Row reductions (every lane of a 16-lane row gets the row's value), then the
// four rows combined in lane order: the result is wave-uniform.
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp_f32<DPP_XOR1>(v));
  v = fmaxf(v, dpp_f32<DPP_XOR2>(v));
  v = fmaxf(v, dpp_f32<DPP_HALF_MIRROR>(v));
  v = fmaxf(v, dpp_f32<DPP_MIRROR>(v));
  return v;
}
__device__ __forceinline__ float wave_max_u(float v) {
  v = row16_max(v);
  return fmaxf(fmaxf(rdlf(v, 0), rdlf(v, 16)), fmaxf(rdlf(v, 32), rdlf(v, 48)));
}
__device__ __forceinline__ float wave_min_u(float v) { return -wave_max_u(-v); }
__device__ __forceinline__ float wave_sum_u(float v) {
  v = row16_sum(v);
  return (rdlf(v, 0) + rdlf(v, 16)) + (rdlf(v, 32) + rdlf(v, 48));
}

// Exclusive block scan of four ints; offsets and totals returned.
__device__ __forceinline__ void block_scan4(const int v[4], int off[4], int tot[4], int* lds) {
  const int lane = __lane_id(), wv = threadIdx.x >> 6;
  int inc[4];
#pragma unroll
  for (int f = 0; f < 4; f++) inc[f] = wave_incl_scan(v[f]);
  if (lane == 63) {
#pragma unroll
    for (int f = 0; f < 4; f++) lds[f * NW + wv] = inc[f];
  }
  __syncthreads();
#pragma unroll
  for (int f = 0; f < 4; f++) {
    int o = 0, t = 0;
#pragma unroll
    for (int w = 0; w < NW; w++) {
      const int a = lds[f * NW + w];
      o += w < wv ? a : 0;
      t += a;
    }
    off[f] = o + inc[f] - v[f];
    tot[f] = t;
  }
  __syncthreads();
}

__device__ __forceinline__ float key_value(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k ^ 0x80000000u) : ~k);
}
__device__ __forceinline__ int bin_of(uint32_t k, float lo, float inv) {
  return max(0, min(NBINS - 1, (int)((key_value(k) - lo) * inv)));
}
// (k, id) is among the first M of the rank order with pivot (kp, ip)
__device__ __forceinline__ bool in_top(uint32_t k, int id, uint32_t kp, int ip) {
  return k > kp || (k == kp && id <= ip);
}

template <int DT>
__device__ __forceinline__ float ex(float x) {
  if constexpr (DT == WI_BF16) return __expf(x);
  else return expf(x);
}

// ---- LDS layout -----------------------------------------------------------
template <int GS>
struct Lds {
  static constexpr int HIST = 0;                              // int[NBINS]
  static constexpr int CANDK = HIST + NBINS * 4;              // uint32[2][CAND_MAX]
  static constexpr int CANDI = CANDK + 2 * CAND_MAX * 4;      // int[2][CAND_MAX]
  static constexpr int RTOK = CANDI + 2 * CAND_MAX * 4;       // int[RMAX + 4]
  static constexpr int RBLK = RTOK + (RMAX + 4) * 4;          // int[RMAX]
  static constexpr int EID = RBLK + RMAX * 4;                 // int[EMAX]
  static constexpr int ESZ = EID + EMAX * 4;                  // int[EMAX]
  static constexpr int ZBUF = ESZ + EMAX * 4;                 // float[2*ROUND][GS]
  static constexpr int MBUF = ZBUF + 2 * ROUND * GS * 4;      // float[ROUND]
  static constexpr int END = MBUF + ROUND * 4;
  static constexpr int SACC = 0;                              // float[NW][GS][D]
  static constexpr int END_MERGE = SACC + NW * GS * D * 4;
  static constexpr int BYTES = END > END_MERGE ? END : END_MERGE;
};

template <int DT, int GS, int PER>
__global__ __launch_bounds__(NT) void fused_kernel(FusedArgs a) {
  using L = Lds<GS>;
  __shared__ __align__(16) uint8_t smem[L::BYTES];
  int* hist = reinterpret_cast<int*>(smem + L::HIST);
  uint32_t* candk = reinterpret_cast<uint32_t*>(smem + L::CANDK);
  int* candi = reinterpret_cast<int*>(smem + L::CANDI);
  int* Rtok = reinterpret_cast<int*>(smem + L::RTOK);
  int* Rblk = reinterpret_cast<int*>(smem + L::RBLK);
  int* Eid = reinterpret_cast<int*>(smem + L::EID);
  int* Esz = reinterpret_cast<int*>(smem + L::ESZ);
  float* zbuf = reinterpret_cast<float*>(smem + L::ZBUF);
  float* mbuf = reinterpret_cast<float*>(smem + L::MBUF);
  __shared__ int scan_lds[4 * NW];
  __shared__ float redf[2][NW][GS];
  __shared__ int bsel[2], bneed[2], ncand[2];
  __shared__ uint32_t pk[2];
  __shared__ int pi[2];
  __shared__ int rdx[256];
  __shared__ uint64_t rpref;
  __shared__ int rneed, s_last;
  __shared__ float cden[MAX_G];

  const int w = blockIdx.x, u = blockIdx.y;
  const int b = u / a.H, h = u % a.H;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int r16 = lane & 15, kg = lane >> 4;
  const int C = a.C, G = a.G;
  const int K_r = a.K_r, K_e = a.K_e;
  const int M[2] = {K_r, K_r + K_e};
  const int NP = (C + NT * PER - 1) / (NT * PER);  // passes over the keys
  const uint32_t* key = a.key + (int64_t)u * a.Cp;
  const bool sz_vec = (C & 3) == 0;  // size rows are 16-byte aligned
  const int32_t* sz = a.sizes + (int64_t)u * C;
  const int64_t uC = (int64_t)u * C;

  // ---- the query heads as the B operand of the logit MFMA (issued first) --
  // bf16: lane supplies q[head r16][dims 32 s + 8 kg .. + 8], s = 0..3;
  // fp32: lane supplies q[head r16][dims 32 kg .. + 32].
  const int64_t qrow = (int64_t)b * a.Hq + (int64_t)h * G + min(r16, G - 1);
  uint4 bq[DT == WI_BF16 ? 4 : 8];
  if constexpr (DT == WI_BF16) {
    const uint16_t* qp = reinterpret_cast<const uint16_t*>(a.q) + qrow * D + 8 * kg;
#pragma unroll
    for (int s = 0; s < 4; s++) {
      const uint4 v = *reinterpret_cast<const uint4*>(qp + 32 * s);
      bq[s] = r16 < G ? v : make_uint4(0u, 0u, 0u, 0u);
    }
  } else {
    const uint4* qp = reinterpret_cast<const uint4*>(reinterpret_cast<const float*>(a.q) +
                                                     qrow * D + 32 * kg);
#pragma unroll
    for (int s = 0; s < 8; s++) bq[s] = r16 < G ? qp[s] : make_uint4(0u, 0u, 0u, 0u);
  }

  // ---- keys and sizes of this thread's ids [p*NT*PER + tid*PER, +PER) -----
  uint32_t kr[PER];
  int sr[PER];
  int binr[PER];
  auto load = [&](int p) {
    const int i0 = p * NT * PER + tid * PER;
#pragma unroll
    for (int i = 0; i < PER; i += 4) {
      if (i0 + i + 3 < C) {
        const uint4 v = *reinterpret_cast<const uint4*>(key + i0 + i);
        kr[i] = v.x; kr[i + 1] = v.y; kr[i + 2] = v.z; kr[i + 3] = v.w;
        if (sz_vec) {
          const int4 z = *reinterpret_cast<const int4*>(sz + i0 + i);
          sr[i] = z.x; sr[i + 1] = z.y; sr[i + 2] = z.z; sr[i + 3] = z.w;
        } else {
#pragma unroll
          for (int e = 0; e < 4; e++) sr[i + e] = sz[i0 + i + e];
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; e++) {
          const bool ok = i0 + i + e < C;
          kr[i + e] = ok ? key[i0 + i + e] : 0u;
          sr[i + e] = ok ? sz[i0 + i + e] : 0;
        }
      }
    }
  };
  auto nvalid = [&](int p) { return max(0, min(PER, C - (p * NT * PER + tid * PER))); };

  // ---- 1a. value range ------------------------------------------------------
  for (int i = tid; i < NBINS; i += NT) hist[i] = 0;
  if (tid < 2) ncand[tid] = 0;
  float lo = INFINITY, hi = -INFINITY;
  for (int p = 0; p < NP; p++) {
    load(p);
    const int nv = nvalid(p);
#pragma unroll
    for (int i = 0; i < PER; i++) {
      const float f = key_value(kr[i]);
      lo = i < nv ? fminf(lo, f) : lo;
      hi = i < nv ? fmaxf(hi, f) : hi;
    }
  }
  lo = wave_min_u(lo);
  hi = wave_max_u(hi);
  if (lane == 0) {
    redf[0][wv][0] = lo;
    redf[1][wv][0] = hi;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < NW; i++) {
    lo = fminf(lo, redf[0][i][0]);
    hi = fmaxf(hi, redf[1][i][0]);
  }
  const float inv = hi > lo ? (float)NBINS / (hi - lo) : 0.f;

  // ---- 1b. histogram --------------------------------------------------------
  for (int p = 0; p < NP; p++) {
    if (NP > 1) load(p);
    const int nv = nvalid(p);
#pragma unroll
    for (int i = 0; i < PER; i++) {
      binr[i] = bin_of(kr[i], lo, inv);
      if (i < nv) atomicAdd(&hist[binr[i]], 1);
    }
  }
  __syncthreads();

  // ---- 1c. pivot bins: thread t owns bins NBINS-1-t*BPT down ------------
  {
    int hb[BPT];
    int loc = 0;
#pragma unroll
    for (int j = 0; j < BPT; j++) {
      hb[j] = hist[NBINS - 1 - tid * BPT - j];
      loc += hb[j];
    }
    const int v4[4] = {loc, 0, 0, 0};
    int off4[4], tot4[4];
    block_scan4(v4, off4, tot4, scan_lds);
#pragma unroll
    for (int t = 0; t < 2; t++) {
      const int m = M[t];
      int run = off4[0];
#pragma unroll
      for (int j = 0; j < BPT; j++) {
        if (m > 0 && m < C && run < m && m <= run + hb[j]) {
          bsel[t] = NBINS - 1 - tid * BPT - j;
          bneed[t] = m - run;
        }
        run += hb[j];
      }
    }
    if (tid < 2) {
      // M = 0: nothing selected; M >= C: everything selected
      if (M[tid] <= 0) { pk[tid] = 0xFFFFFFFFu; pi[tid] = -1; }
      if (M[tid] >= C) { pk[tid] = 0u; pi[tid] = INT_MAX; }
    }
  }
  __syncthreads();
  const bool need_piv0 = M[0] > 0 && M[0] < C, need_piv1 = M[1] > 0 && M[1] < C;
  const int b1 = need_piv0 ? bsel[0] : -1, b2 = need_piv1 ? bsel[1] : -1;

  // ---- 1d. keys of the pivot bins ------------------------------------------
  for (int p = 0; p < NP; p++) {
    if (NP > 1) {
      load(p);
#pragma unroll
      for (int i = 0; i < PER; i++) binr[i] = bin_of(kr[i], lo, inv);
    }
    const int nv = nvalid(p);
    const int i0 = p * NT * PER + tid * PER;
#pragma unroll
    for (int i = 0; i < PER; i++) {
      if (i < nv && binr[i] == b1) {
        const int s = atomicAdd(&ncand[0], 1);
        if (s < CAND_MAX) { candk[s] = kr[i]; candi[s] = i0 + i; }
      }
      if (i < nv && binr[i] == b2) {
        const int s = atomicAdd(&ncand[1], 1);
        if (s < CAND_MAX) { candk[CAND_MAX + s] = kr[i]; candi[CAND_MAX + s] = i0 + i; }
      }
    }
  }
  __syncthreads();

  // ---- 1e. pivots: wave t ranks the keys of target t's bin -----------------
  const int nc0 = ncand[0], nc1 = ncand[1];
  if (wv < 2) {
    const int t = wv;
    const bool need = t == 0 ? need_piv0 : need_piv1;
    const int nc = t == 0 ? nc0 : nc1;
    if (need && nc <= CAND_MAX) {
      const uint32_t kk = lane < nc ? candk[t * CAND_MAX + lane] : 0u;
      const int id = lane < nc ? candi[t * CAND_MAX + lane] : INT_MAX;
      int rank = 0;
      for (int j = 0; j < nc; j++) {
        const uint32_t kj = (uint32_t)rdl((int)kk, j);
        const int idj = rdl(id, j);
        rank += (kj > kk) || (kj == kk && idj < id);
      }
      if (lane < nc && rank == bneed[t] - 1) {
        pk[t] = kk;
        pi[t] = id;
      }
    }
  }
  if ((need_piv0 && nc0 > CAND_MAX) || (need_piv1 && nc1 > CAND_MAX)) {
    // radix select over composite = key << 32 | ~id among the keys of the
    // pivot bin: the need-th largest composite is the pivot
#pragma unroll 1
    for (int t = 0; t < 2; t++) {
      const bool need = t == 0 ? need_piv0 : need_piv1;
      if (!need || (t == 0 ? nc0 : nc1) <= CAND_MAX) continue;
      const int bs = bsel[t];
      uint64_t pref = 0;
      int nd = bneed[t];
#pragma unroll 1
      for (int d = 0; d < 8; d++) {
        const int shift = 56 - 8 * d;
        for (int i = tid; i < 256; i += NT) rdx[i] = 0;
        __syncthreads();
        for (int p = 0; p < NP; p++) {
          if (NP > 1) load(p);
          const int nv = nvalid(p);
          const int i0 = p * NT * PER + tid * PER;
#pragma unroll
          for (int i = 0; i < PER; i++) {
            if (i < nv && bin_of(kr[i], lo, inv) == bs) {
              const uint64_t comp =
                  ((uint64_t)kr[i] << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)(i0 + i));
              if (d == 0 || (comp >> (shift + 8)) == (pref >> (shift + 8)))
                atomicAdd(&rdx[(comp >> shift) & 255], 1);
            }
          }
        }
        __syncthreads();
        if (tid == 0) {
          int run = 0;
          for (int dg = 255; dg >= 0; dg--) {
            if (run < nd && nd <= run + rdx[dg]) {
              rpref = pref | ((uint64_t)dg << shift);
              rneed = nd - run;
              break;
            }
            run += rdx[dg];
          }
        }
        __syncthreads();
        pref = rpref;
        nd = rneed;
        __syncthreads();
      }
      if (tid == 0) {
        pk[t] = (uint32_t)(pref >> 32);
        pi[t] = (int)(0xFFFFFFFFu - (uint32_t)(pref & 0xFFFFFFFFu));
      }
    }
  }
  __syncthreads();
  const uint32_t pkR = pk[0], pkS = pk[1];
  const int piR = pi[0], piS = pi[1];

  // ---- 2. compaction -----------------------------------------------------------
  const int e0 = (int)((int64_t)K_e * w / a.W), e1 = (int)((int64_t)K_e * (w + 1) / a.W);
  const bool dbg = (a.dbgR != nullptr) && w == 0;
  const int lgT = a.lgT, Tm1 = (1 << lgT) - 1;
  int baseRnz = 0, baseE = 0, baseTok = 0, baseB = 0, baseRall = 0;
  for (int p = 0; p < NP; p++) {
    if (NP > 1) load(p);
    const int nv = nvalid(p);
    const int i0 = p * NT * PER + tid * PER;
    uint32_t fR = 0, fE = 0, fNZ = 0;
    int sRt = 0, sB = 0;
#pragma unroll
    for (int i = 0; i < PER; i++) {
      const bool ok = i < nv;
      const bool r = ok && in_top(kr[i], i0 + i, pkR, piR);
      const bool e = ok && !r && in_top(kr[i], i0 + i, pkS, piS);
      fR |= (uint32_t)r << i;
      fE |= (uint32_t)e << i;
      fNZ |= (uint32_t)(sr[i] > 0) << i;
      sRt += r ? sr[i] : 0;
      sB += ok ? (sr[i] + Tm1) >> lgT : 0;
    }
    const int v4[4] = {(int)__popc(fR & fNZ), (int)__popc(fE), sRt, sB};
    int off4[4], tot4[4];
    block_scan4(v4, off4, tot4, scan_lds);
    int rnz = baseRnz + off4[0], e = baseE + off4[1], tok = baseTok + off4[2];
    int blk = baseB + off4[3];
    if (fR) {  // retrieved clusters are rare: most threads skip this
#pragma unroll
      for (int i = 0; i < PER; i++) {
        if ((fR >> i) & (fNZ >> i) & 1u) {
          if (rnz < RMAX) {
            Rtok[rnz] = tok;
            Rblk[rnz] = blk;
          }
          rnz++;
          tok += sr[i];
        }
        blk += (sr[i] + Tm1) >> lgT;
      }
    }
#pragma unroll
    for (int i = 0; i < PER; i++) {
      if ((fE >> i) & 1u) {
        if (e >= e0 && e < e1) {
          Eid[e - e0] = i0 + i;
          Esz[e - e0] = sr[i];
        }
        e++;
      }
    }
    if (dbg) {
      // debug lists: every retrieved and estimation id, ascending
      const int ra = wave_incl_scan((int)__popc(fR)) - (int)__popc(fR);
      const int ea = wave_incl_scan((int)__popc(fE)) - (int)__popc(fE);
      if (lane == 63) {
        scan_lds[wv] = ra + __popc(fR);
        scan_lds[NW + wv] = ea + __popc(fE);
      }
      __syncthreads();
      int rr = baseRall + ra, ee = baseE + ea;
      int tr = 0;
      for (int v = 0; v < NW; v++) {
        rr += v < wv ? scan_lds[v] : 0;
        ee += v < wv ? scan_lds[NW + v] : 0;
        tr += scan_lds[v];
      }
      for (int i = 0; i < PER; i++) {
        if ((fR >> i) & 1u) {
          if (rr < K_r) a.dbgR[(int64_t)u * K_r + rr] = i0 + i;
          rr++;
        }
        if ((fE >> i) & 1u) {
          if (ee < K_e) a.dbgE[(int64_t)u * K_e + ee] = i0 + i;
          ee++;
        }
      }
      baseRall += tr;
      __syncthreads();
    }
    baseRnz += tot4[0];
    baseE += tot4[1];
    baseTok += tot4[2];
    baseB += tot4[3];
  }
  // retrieved clusters with members (<= K_r <= RMAX; the clamp only keeps LDS
  // accesses in bounds should the counts ever disagree)
  const int NRnz = min(baseRnz, RMAX);
  const int NRtok = NRnz > 0 ? baseTok : 0;
  if (tid == 0) Rtok[NRnz] = NRtok;

  // ---- 3. items ---------------------------------------------------------------
  const int NX = a.n_st + NRtok;
  const int x0 = (int)((int64_t)NX * w / a.W), x1 = (int)((int64_t)NX * (w + 1) / a.W);
  const int nS = max(0, min(x1, a.n_st) - x0);
  const int rlo = max(x0 - a.n_st, 0), rhi = max(rlo, min(x1 - a.n_st, NRtok));
  const int nT = nS + (rhi - rlo);
  const int nEi = e1 - e0;
  const int rounds = (max(nT, nEi) + ROUND - 1) / ROUND;
  constexpr int RB = D * (DT == WI_BF16 ? 2 : 4);  // bytes per K/V row
  const uint8_t* kb8 = reinterpret_cast<const uint8_t*>(a.kblk);
  const uint8_t* vb8 = reinterpret_cast<const uint8_t*>(a.vblk);
  const uint8_t* sk8 = reinterpret_cast<const uint8_t*>(a.stk);
  const uint8_t* sv8 = reinterpret_cast<const uint8_t*>(a.stv);
  const uint8_t* dummy = reinterpret_cast<const uint8_t*>(a.vsum + uC * D);  // any valid row

  float Mrun[GS], Lrun[GS], acc[GS][2];
#pragma unroll
  for (int g = 0; g < GS; g++) {
    Mrun[g] = -INFINITY;
    Lrun[g] = 0.f;
    acc[g][0] = acc[g][1] = 0.f;
  }
  __syncthreads();  // lists complete

#pragma unroll 1
  for (int rd = 0; rd < rounds; rd++) {
    // (a) this wave's 16 tokens: row pointers (lane r16 -> token r16)
    const int tb = rd * ROUND + wv * 16;  // first token item of the wave
    const int ntw = max(0, min(16, nT - tb));
    const int tk = tb + r16;
    const uint8_t* kp = dummy;
    const uint8_t* vp = dummy;
    if (tk < nT) {
      if (tk < nS) {
        const int64_t row = (int64_t)u * a.n_st + x0 + tk;
        kp = sk8 + row * RB;
        vp = sv8 + row * RB;
      } else {
        const int t = rlo + (tk - nS);
        int j = 0;
#pragma unroll
        for (int step = RMAX / 2; step >= 1; step >>= 1)
          if (j + step < NRnz && Rtok[j + step] <= t) j += step;
        const int64_t row = (int64_t)u * a.capT + ((int64_t)Rblk[j] << lgT) + (t - Rtok[j]);
        kp = kb8 + row * RB;
        vp = vb8 + row * RB;
      }
    }
    // (b) key loads (MFMA layout) and value loads (two dims per lane)
    constexpr int NKL = DT == WI_BF16 ? 4 : 8;
    uint4 ka[NKL];
#pragma unroll
    for (int s = 0; s < NKL; s++) {
      if constexpr (DT == WI_BF16)
        ka[s] = *reinterpret_cast<const uint4*>(kp + (32 * s + 8 * kg) * 2);
      else
        ka[s] = *reinterpret_cast<const uint4*>(kp + (32 * kg + 4 * s) * 4);
    }
    uint2 vr[16];  // bf16: .x holds dims 2 lane, 2 lane + 1; fp32: both words
#pragma unroll
    for (int t = 0; t < 16; t++) {
      if (t < ntw) {
        const uint64_t pa = ((uint64_t)(uint32_t)rdl((int)(uintptr_t)vp, t)) |
                            ((uint64_t)(uint32_t)rdl((int)((uintptr_t)vp >> 32), t) << 32);
        const uint8_t* vpt = reinterpret_cast<const uint8_t*>(pa);
        if constexpr (DT == WI_BF16)
          vr[t] = make_uint2(*reinterpret_cast<const uint32_t*>(vpt + 4 * lane), 0u);
        else
          vr[t] = *reinterpret_cast<const uint2*>(vpt + 8 * lane);
      }
    }
    // (c) this wave's 16 estimation clusters: logits and value sums
    const int eb = rd * ROUND + wv * 16;
    const int new_ = max(0, min(16, nEi - eb));
    const int ei = eb + r16;
    const int eid = ei < nEi ? Eid[ei] : 0;
    const int esz = ei < nEi ? Esz[ei] : 0;
    float sl[GS];
    {
      const float* sp = a.S + (uC + eid) * GS;
#pragma unroll
      for (int g = 0; g < GS; g += 4) {
        const float4 z4 = *reinterpret_cast<const float4*>(sp + g);
        sl[g] = z4.x;
        sl[g + 1] = z4.y;
        sl[g + 2] = z4.z;
        sl[g + 3] = z4.w;
      }
    }
    float2 vs[16];
#pragma unroll
    for (int t = 0; t < 16; t++) {
      if (t < new_) {
        const int id_t = rdl(eid, t);
        vs[t] = *reinterpret_cast<const float2*>(a.vsum + (uC + id_t) * D + 2 * lane);
      }
    }
    // (d) token logits: z[token 4 kg + j][head r16]
    f32x4_t za = {0.f, 0.f, 0.f, 0.f};
    if constexpr (DT == WI_BF16) {
#pragma unroll
      for (int s = 0; s < 4; s++)
        za = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, ka[s]),
                                                     __builtin_bit_cast(bf16x8_t, bq[s]), za,
                                                     0, 0, 0);
    } else {
#pragma unroll
      for (int s = 0; s < 8; s++) {
        const float kx[4] = {__uint_as_float(ka[s].x), __uint_as_float(ka[s].y),
                             __uint_as_float(ka[s].z), __uint_as_float(ka[s].w)};
        const float qx[4] = {__uint_as_float(bq[s].x), __uint_as_float(bq[s].y),
                             __uint_as_float(bq[s].z), __uint_as_float(bq[s].w)};
#pragma unroll
        for (int e = 0; e < 4; e++)
          za = __builtin_amdgcn_mfma_f32_16x16x4f32(kx[e], qx[e], za, 0, 0, 0);
      }
    }
    if (r16 < G) {
#pragma unroll
      for (int j = 0; j < 4; j++) {
        const int it = 4 * kg + j;
        zbuf[(wv * 16 + it) * GS + r16] = it < ntw ? za[j] * a.scale : -INFINITY;
      }
    }
    if (kg == 0) {
      const bool ok = r16 < new_ && esz > 0;
#pragma unroll
      for (int g = 0; g < GS; g++) zbuf[(ROUND + wv * 16 + r16) * GS + g] = ok ? sl[g] : -INFINITY;
      mbuf[wv * 16 + r16] = (float)esz;
    }
    __syncthreads();

    // (e) maximum per head over the round, then weights and their sum
    const bool holds = tid < 2 * ROUND;  // thread tid holds item tid
    float zi[GS];
#pragma unroll
    for (int g = 0; g < GS; g++) zi[g] = holds ? zbuf[tid * GS + g] : -INFINITY;
    if (wv < 2 * ROUND / 64) {
#pragma unroll
      for (int g = 0; g < GS; g++) {
        const float mx = g < G ? wave_max_u(zi[g]) : 0.f;
        if (lane == 0) redf[0][wv][g] = mx;
      }
    }
    __syncthreads();
    float Mnew[GS], alpha[GS];
#pragma unroll
    for (int g = 0; g < GS; g++) {
      float mx = Mrun[g];
#pragma unroll
      for (int v = 0; v < 2 * ROUND / 64; v++) mx = fmaxf(mx, redf[0][v][g]);
      Mnew[g] = mx;
      alpha[g] = Mrun[g] == -INFINITY ? 0.f : ex<DT>(Mrun[g] - mx);
    }
    if (holds) {
      const float mult = tid < ROUND ? 1.f : mbuf[tid - ROUND];
#pragma unroll
      for (int g = 0; g < GS; g++) {
        const float pz = zi[g] == -INFINITY ? 0.f : ex<DT>(zi[g] - Mnew[g]);
        zbuf[tid * GS + g] = pz;
        zi[g] = mult * pz;
      }
    }
    if (wv < 2 * ROUND / 64) {
#pragma unroll
      for (int g = 0; g < GS; g++) {
        const float ls = g < G ? wave_sum_u(zi[g]) : 0.f;
        if (lane == 0) redf[1][wv][g] = ls;
      }
    }
    __syncthreads();
#pragma unroll
    for (int g = 0; g < GS; g++) {
      float ls = 0.f;
#pragma unroll
      for (int v = 0; v < 2 * ROUND / 64; v++) ls += redf[1][v][g];
      Lrun[g] = Lrun[g] * alpha[g] + ls;
      Mrun[g] = Mnew[g];
      acc[g][0] *= alpha[g];
      acc[g][1] *= alpha[g];
    }

    // (f) sum_i p_i v_i over the wave's tokens, then estimation clusters
#pragma unroll
    for (int t = 0; t < 16; t++) {
      if (t < ntw) {
        float v0, v1;
        if constexpr (DT == WI_BF16) {
          v0 = __uint_as_float(vr[t].x << 16);
          v1 = __uint_as_float(vr[t].x & 0xFFFF0000u);
        } else {
          v0 = __uint_as_float(vr[t].x);
          v1 = __uint_as_float(vr[t].y);
        }
        const float* pp = zbuf + (wv * 16 + t) * GS;
#pragma unroll
        for (int g = 0; g < GS; g += 4) {
          const float4 p4 = *reinterpret_cast<const float4*>(pp + g);
          const float pg[4] = {p4.x, p4.y, p4.z, p4.w};
#pragma unroll
          for (int e = 0; e < 4; e++) {
            acc[g + e][0] = fmaf(pg[e], v0, acc[g + e][0]);
            acc[g + e][1] = fmaf(pg[e], v1, acc[g + e][1]);
          }
        }
      }
    }
#pragma unroll
    for (int t = 0; t < 16; t++) {
      if (t < new_) {
        const float* pp = zbuf + (ROUND + wv * 16 + t) * GS;
#pragma unroll
        for (int g = 0; g < GS; g += 4) {
          const float4 p4 = *reinterpret_cast<const float4*>(pp + g);
          const float pg[4] = {p4.x, p4.y, p4.z, p4.w};
#pragma unroll
          for (int e = 0; e < 4; e++) {
            acc[g + e][0] = fmaf(pg[e], vs[t].x, acc[g + e][0]);
            acc[g + e][1] = fmaf(pg[e], vs[t].y, acc[g + e][1]);
          }
        }
      }
    }
    __syncthreads();  // zbuf is rewritten by the next round
  }

  // ---- 4. merge the waves (fixed order), publish, count arrivals --------------
  float* sacc = reinterpret_cast<float*>(smem + L::SACC);
#pragma unroll
  for (int g = 0; g < GS; g++)
    if (g < G)
      *reinterpret_cast<float2*>(sacc + (wv * GS + g) * D + 2 * lane) =
          make_float2(acc[g][0], acc[g][1]);
  __syncthreads();
  float* pw = a.part + ((int64_t)u * a.W + w) * G * PART;
  for (int e = tid; e < G * D; e += NT) {
    const int g = e >> 7, t = e & (D - 1);
    float s = 0.f;
#pragma unroll
    for (int v = 0; v < NW; v++) s += sacc[(v * GS + g) * D + t];
    __hip_atomic_store(pw + g * PART + 2 + t, s, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  if (tid < G) {
    // Mrun / Lrun are workgroup-uniform; thread g publishes head g
    float mg = 0.f, lg = 0.f;
#pragma unroll
    for (int g = 0; g < GS; g++) {
      mg = g == tid ? Mrun[g] : mg;
      lg = g == tid ? Lrun[g] : lg;
    }
    __hip_atomic_store(pw + tid * PART, mg, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(pw + tid * PART + 1, lg, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  // the agent-coherent stores above are complete before the arrival count
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (tid == 0)
    s_last = __hip_atomic_fetch_add(&a.tix[u], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
             a.W - 1;
  __syncthreads();
  if (!s_last) return;

  // ---- 5. the last workgroup of the unit merges the W partials -------------
  const float* pu = a.part + (int64_t)u * a.W * G * PART;
  const int WG = a.W * G;  // <= 64 * 16
  float* cm = reinterpret_cast<float*>(smem);  // [WG] m, then weights
  float* cl = cm + 64 * MAX_G;                 // [WG] l
  for (int i = tid; i < WG; i += NT) {
    cm[i] = __hip_atomic_load(pu + (int64_t)i * PART, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    cl[i] = __hip_atomic_load(pu + (int64_t)i * PART + 1, __ATOMIC_RELAXED,
                              __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  if (tid < G) {
    const int g = tid;
    float M2 = -INFINITY;
    for (int v = 0; v < a.W; v++) M2 = fmaxf(M2, cm[v * G + g]);
    float den = 0.f;
    for (int v = 0; v < a.W; v++) {
      const float mv = cm[v * G + g];
      const float f = (mv == -INFINITY) ? 0.f : ex<DT>(mv - M2);
      cm[v * G + g] = f;
      den = fmaf(f, cl[v * G + g], den);
    }
    cden[g] = den;
  }
  __syncthreads();
  for (int e = tid; e < G * D; e += NT) {
    const int g = e >> 7, t = e & (D - 1);
    float num = 0.f;
    for (int v0 = 0; v0 < a.W; v0 += 32) {
      float av[32];
#pragma unroll
      for (int k = 0; k < 32; k++) {
        const int v = min(v0 + k, a.W - 1);
        av[k] = __hip_atomic_load(pu + ((int64_t)v * G + g) * PART + 2 + t, __ATOMIC_RELAXED,
                                  __HIP_MEMORY_SCOPE_AGENT);
      }
#pragma unroll
      for (int k = 0; k < 32; k++)
        if (v0 + k < a.W) num = fmaf(cm[(v0 + k) * G + g], av[k], num);
    }
    const float den = cden[g];
    a.out[((int64_t)b * a.Hq + (int64_t)h * G + g) * D + t] = den > 0.f ? num / den : 0.f;
  }
}

template <int DT, int GS>
hipError_t launch_fused_gs(const DecodeArgs& da, const FusedArgs& fa, hipStream_t s) {
  dim3 grid(da.W, da.g->U);
  if (da.PER <= 4)
    WI_LAUNCH(K_FUSED, (fused_kernel<DT, GS, 4>), grid, dim3(NT), 0, s, fa);
  else if (da.PER <= 8)
    WI_LAUNCH(K_FUSED, (fused_kernel<DT, GS, 8>), grid, dim3(NT), 0, s, fa);
  else
    WI_LAUNCH(K_FUSED, (fused_kernel<DT, GS, 16>), grid, dim3(NT), 0, s, fa);
  return hipGetLastError();
}

template <int DT>
hipError_t launch_fused_dt(const DecodeArgs& da, const FusedArgs& fa, hipStream_t s) {
  if (da.GS == 4) return launch_fused_gs<DT, 4>(da, fa, s);
  if (da.GS == 8) return launch_fused_gs<DT, 8>(da, fa, s);
  return launch_fused_gs<DT, 16>(da, fa, s);
}

}  // namespace

hipError_t launch_fused(const DecodeArgs& da, const wi_index_bufs& bf, const void* q,
                        float* out, const DecodeWs& ws, bool want_lists, hipStream_t s) {
  const Geom& g = *da.g;
  FusedArgs fa;
  fa.key = ws.key;
  fa.S = ws.S;
  fa.sizes = bf.cluster_size;
  fa.kblk = bf.k_blocks;
  fa.vblk = bf.v_blocks;
  fa.stk = bf.steady_k;
  fa.stv = bf.steady_v;
  fa.vsum = bf.value_sum;
  fa.q = q;
  fa.out = out;
  fa.part = ws.part;
  fa.tix = ws.tix;
  fa.dbgR = want_lists ? ws.R : nullptr;
  fa.dbgE = want_lists ? ws.E : nullptr;
  fa.C = g.C;
  fa.Cp = (g.C + 3) & ~3;
  fa.n_st = g.n_st;
  fa.G = da.G;
  fa.H = g.H;
  fa.Hq = da.Hq;
  fa.K_r = da.K_r;
  fa.K_e = da.K_e;
  fa.W = da.W;
  fa.lgT = g.T == 8 ? 3 : 2;
  fa.capT = g.cap * g.T;
  fa.scale = da.scale;
  return g.dtype == WI_BF16 ? launch_fused_dt<WI_BF16>(da, fa, s)
                            : launch_fused_dt<WI_F32>(da, fa, s);
}

}  // namespace wi
