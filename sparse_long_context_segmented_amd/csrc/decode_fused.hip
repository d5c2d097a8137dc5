// Decode steps 2-6 in one launch: select the retrieval and estimation zones,
// gather the retrieved tokens, exact attention over the steady and retrieval
// zones, the estimation-zone partial, and the log-sum-exp merge (RetroInfer,
// framerc blog section 2.1: retrieval about 1.8 % of tokens, estimation the
// next 23 %; section 3.2: execution buffer = steady zone + retrieved blocks
// with block fragments skipped; section 3.3: estimation from centroid
// vectors and cluster sizes, partial results merged by a custom kernel;
// techwalker article section 3).
//
// Grid: W workgroups of 512 threads per unit (sequence, KV head). Cluster ids
// are cut into groups of 16 consecutive ids; workgroup w owns the groups
// w, w + W, w + 2W, ... (so every segment's clusters spread over all
// workgroups of the unit) and the exactly attended rows outside the retrieved
// clusters -- the n_st steady rows, then the n_pend pending rows (decode-time
// tokens that left the local window and wait for their segment) -- [w n_x /
// W, (w+1) n_x / W), n_x = n_st + n_pend.
// At batch 1 a decode step moves a few tens of MB, so the kernel is bound by
// latencies -- dependent memory round trips, LDS round trips, instruction
// chains -- and is laid out to keep those few:
//
//  1. Selection, repeated by every workgroup of the unit on chip (the C
//     ranking keys are a few tens of KB). Rank order is larger key first,
//     lower cluster id on equal keys. For M in {K_r, K_r + K_e'} the M-th
//     ranked cluster -- the pivot -- is found; cluster c is among the first M
//     iff comp(c) >= comp(pivot), comp = key << 32 | (2^32 - 1 - id). A
//     2048-bin histogram linear in key value over the unit's key range (the
//     score step publishes each of its workgroups' minimum and maximum), built
//     as the keys arrive, locates the pivot's bin; its keys (at most
//     CAND_MAX) are ranked exactly by four waves, one key per lane (the bin
//     at the estimation pivot of a 1M-token unit holds about 130 of its 65536
//     keys); a fuller bin falls back to an 8-pass radix select over comp
//     within that bin. The
//     sizes, block offsets and estimation logits of the workgroup's first
//     512 own clusters are loaded at kernel start, behind the selection.
//  2. Own clusters, 512 at a time: one block scan per 512 gives each
//     retrieved cluster with members its first token among the retrieved
//     tokens, and each estimation cluster with members its slot; the lists
//     of up to PASS_CHUNKS(GS) such chunks are appended before their items
//     run. Retrieved tokens are read straight from the cluster-contiguous 2 KB
//     blocks (the first n_c rows of the cluster: fragments skipped).
//  3. Items, in blocks of 32 tokens (16 for fp32) and 16 estimation clusters;
//     wave v takes blocks v, v + 8, ... and runs with no workgroup barrier.
//     A lane finds its token's row by binary search over the retrieved
//     clusters' token offsets. Token logits: one MFMA chain per 16 tokens x
//     16 query-head columns (bf16 keys: exact products, fp32 sums);
//     estimation clusters bring their logits from the score step. Each wave
//     keeps an online softmax per head (running maximum, denominator in which
//     an estimation cluster counts n_c times, and the numerator sum_i p_i v_i
//     over token values and value sums VS_c). With bf16 values and head
//     groups of up to 8 the numerator is a second MFMA chain per block: the
//     weights (split into two bf16 parts) against the tokens' values, each
//     lane reading 16 contiguous bytes per token, and against the value sums
//     (each split into two bf16 parts); otherwise two dims per lane on VALU.
//  4. Merge: the waves' states are combined in a fixed order; the
//     workgroup's (m, l, acc) per head is published with agent-coherent
//     stores and one agent-scope release atomic counts arrivals; the last
//     workgroup of the unit acquires, reads the W partials and writes
//     out = sum_w e^{m_w-M} acc_w / sum_w e^{m_w-M} l_w.
// Every sum runs in a fixed order, so results are bit-reproducible.
#include <climits>
#include <type_traits>

#include "wi_internal.h"

namespace wi {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int NT = FUSED_THREADS;  // threads per workgroup
constexpr int NW = NT / 64;        // waves
constexpr int CL = 8192;           // keys staged in LDS at a time
constexpr int KPT = CL / NT;       // staged keys per thread
constexpr int NBINS = 2048;
constexpr int BPT = NBINS / NT;    // histogram bins per thread
constexpr int CAND_MAX = 256;      // pivot-bin keys ranked on chip (4 waves per pivot)
constexpr int GRP = 16;            // consecutive cluster ids per ownership group
constexpr int EB = 16;             // estimation clusters per wave block
constexpr int PI_MAX = 32 + EB;    // items per wave block (tokens + clusters)
constexpr int PART = 2 + D;        // m, l, acc[128]
constexpr int RM_PLAIN = 0, RM_PEND = 1, RM_CACHED = 2;  // row modes of the fused kernel
static_assert(NT == 512 && BPT == 4 && KPT % 4 == 0, "thread layout");
static_assert(CAND_MAX <= 4 * 64 && NW == 8, "four waves rank each pivot's candidates");

struct FusedArgs {
  const uint32_t* key;     // [U][Cp] order-preserving ranking keys
  const float* S;          // [U][C][GS] scaled per-head logits
  const float2* mm;        // [U][NB] key ranges of the score workgroups
  const int32_t* size;     // [U][C]
  const int32_t* block_off;  // [U][C+1]
  const void* kblk;
  const void* vblk;
  const void* stk;
  const void* stv;
  const float* vsum;
  const void* q;
  float* out;
  float* part;             // [U][W][G][PART]
  int* tix;                // [U] arrival counters, zero on entry
  uint8_t* zone;           // nullable: [U][C] 1 = retrieval, 2 = estimation
  const void* pk;          // nullable while n_pend = 0: [U][seg_len] pending rows
  const void* pv;
  // wave buffer (cached kernel only): kblk/vblk are then the host tier's
  // blocks; a block with b2s[u][blk] = s >= 0 is read from cache slot s
  const int32_t* b2s;      // [U][nblk]
  const void* ck;          // [U][nslot * T] rows
  const void* cv;
  int64_t nblk;
  int nslot;
  int C, Cp, n_st, n_pend, seg_len, G, H, Hq, K_r, K_e, W, lgT, NB;
  int64_t capT;
  float scale;
};

// ---- wave primitives --------------------------------------------------------
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
__device__ __forceinline__ float wave_sum_u(float v) {
  v = row16_sum(v);
  return (rdlf(v, 0) + rdlf(v, 16)) + (rdlf(v, 32) + rdlf(v, 48));
}

// Exclusive block scan of N ints per thread (N <= 4): offsets and totals.
template <int N>
__device__ __forceinline__ void block_scan(const int* v, int* off, int* tot, int* lds) {
  const int lane = __lane_id(), wv = threadIdx.x >> 6;
  int inc[N];
#pragma unroll
  for (int f = 0; f < N; f++) inc[f] = wave_incl_scan(v[f]);
  if (lane == 63) {
#pragma unroll
    for (int f = 0; f < N; f++) lds[f * NW + wv] = inc[f];
  }
  __syncthreads();
#pragma unroll
  for (int f = 0; f < N; f++) {
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
// Monotone in the key (ties share a bin); NaN values land in bin 0.
// off = -lo * inv. fma is monotone in the value for inv >= 0, so equal keys
// share a bin and bins follow key order; the median clamps to [0, NBINS - 1]
// (a NaN value lands in bin 0).
__device__ __forceinline__ int bin_of(uint32_t k, float off, float inv) {
  return (int)__builtin_amdgcn_fmed3f(fmaf(key_value(k), inv, off), 0.f, (float)(NBINS - 1));
}
__device__ __forceinline__ uint64_t comp_of(uint32_t k, int id) {
  return ((uint64_t)k << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)id);
}

template <int DT>
__device__ __forceinline__ float ex(float x) {
  if constexpr (DT == WI_BF16) return __expf(x);
  else return expf(x);
}

// Own-cluster chunks whose item lists are gathered before their items run, as
// many as the lists' LDS allows: four (2048 clusters) for head groups of up
// to 4, two for up to 8, else one.
constexpr int PASS_CHUNKS(int GS) { return GS <= 4 ? 4 : (GS <= 8 ? 2 : 1); }

// ---- LDS layout -------------------------------------------------------------
template <int GS>
struct Lds {
  static constexpr int KEYS = 0;                              // uint32[CL]
  static constexpr int HIST = KEYS + CL * 4;                  // int[NBINS + 64] (+ spare slots)
  static constexpr int CAND = HIST + (NBINS + 64) * 4;        // uint64[2][CAND_MAX] comps
  static constexpr int BINS = CAND + 2 * CAND_MAX * 8;        // uint16[CL] histogram bin per key
  static constexpr int LN = NT * PASS_CHUNKS(GS);             // list capacity
  static constexpr int RTOK = BINS + CL * 2;                  // int[LN + 4]
  static constexpr int RBLK = RTOK + (LN + 4) * 4;            // int[LN]
  static constexpr int EID = RBLK + LN * 4;                   // int[LN]
  static constexpr int ESZ = EID + LN * 4;                    // float[LN]
  static constexpr int ELOG = ESZ + LN * 4;                   // float[LN][GS]
  static constexpr int PBUF = ELOG + LN * GS * 4;             // float[NW][PI_MAX][GS]
  static constexpr int QS = PBUF + NW * PI_MAX * GS * 4;          // query rows, GS x 128 x dtype
  static constexpr int END = QS + GS * D * 4;
  static constexpr int SACC = 0;                              // float[NW][GS][D]
  static constexpr int END_MERGE = SACC + NW * GS * D * 4;
  static constexpr int BYTES = END > END_MERGE ? END : END_MERGE;
  static_assert(CAND % 16 == 0 && RTOK % 16 == 0 && PBUF % 16 == 0 && QS % 16 == 0, "align");
};

// BIG: more than CL clusters per unit (keys staged in several LDS passes).
// Kept a separate instantiation so that the common kernel holds no
// re-staging loads, after which the compiler would place waits for
// outstanding loads.
// MODE: where the kernel reads rows. RM_PLAIN: steady rows and the HBM block
// pool only (no pending rows); RM_PEND: also pending rows; RM_CACHED: pending
// rows, and blocks from the wave buffer's cache slots or the host tier. The
// plain instantiation keeps the single two-way address select per row.
template <int DT, int GS, bool BIG, int MODE>
__global__ __launch_bounds__(NT) void fused_kernel(FusedArgs a) {
  using L = Lds<GS>;
  constexpr bool CACHED = MODE == RM_CACHED;
  constexpr bool PLAIN = MODE == RM_PLAIN;
  // token weights-by-values on MFMA (bf16 values, head groups of up to 4;
  // larger groups keep the VALU path, whose registers then fit)
  constexpr bool MPV = DT == WI_BF16 && GS <= 8;
  constexpr int NTILE = DT == WI_BF16 ? 2 : 1;  // 16-token MFMA tiles per wave block
  constexpr int TB = 16 * NTILE;                // tokens per wave block
  constexpr int PI = TB + EB;                   // items per wave block
  constexpr int NKL = DT == WI_BF16 ? 4 : 8;    // 16-byte key pieces per lane and token
  static_assert(PI <= PI_MAX, "weights buffer");
  __shared__ __align__(16) uint8_t smem[L::BYTES];
  uint32_t* keys = reinterpret_cast<uint32_t*>(smem + L::KEYS);
  int* hist = reinterpret_cast<int*>(smem + L::HIST);
  uint64_t* cand = reinterpret_cast<uint64_t*>(smem + L::CAND);  // pivot-bin comps
  uint16_t* kbin = reinterpret_cast<uint16_t*>(smem + L::BINS);
  int* Rtok = reinterpret_cast<int*>(smem + L::RTOK);
  int* Rblk = reinterpret_cast<int*>(smem + L::RBLK);
  int* Eid = reinterpret_cast<int*>(smem + L::EID);
  float* Esz = reinterpret_cast<float*>(smem + L::ESZ);
  float* Elog = reinterpret_cast<float*>(smem + L::ELOG);
  float* Pbuf = reinterpret_cast<float*>(smem + L::PBUF);
  uint8_t* qs = smem + L::QS;
  __shared__ int scan_lds[4 * NW];
  __shared__ float wm[NW][MAX_G], wl[NW][MAX_G];
  __shared__ int bsel[2], bneed[2], ncand[2];
  __shared__ uint32_t pk[2];
  __shared__ int pi[2];
  __shared__ int rdx[256];
  __shared__ uint64_t rpref;
  __shared__ int rneed, s_last;

  // XCD-aware placement: the dispatcher deals consecutive workgroups round
  // robin to the 8 XCDs, so with a unit count that is a multiple of 8 the
  // linear id L = 8 slot + x maps to unit (slot / W) 8 + x, workgroup
  // slot % W: all W workgroups of a unit run on one XCD and share its L2
  // copy of the unit's keys, scores and cluster data (a bijection on the grid)
  int w, u;
  if ((gridDim.y & 7) == 0) {
    const int L = (int)blockIdx.x + (int)blockIdx.y * (int)gridDim.x;
    const int slot = L >> 3;
    const int q = slot / (int)gridDim.x;
    u = q * 8 + (L & 7);
    w = slot - q * (int)gridDim.x;
  } else {
    w = blockIdx.x;
    u = blockIdx.y;
  }
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int C = a.C;
  const uint32_t* keyg = a.key + (int64_t)u * a.Cp;  // 16-byte aligned rows
  // The selection's first loads -- the keys of pass 0 and up to 256 of the
  // score workgroups' ranges -- are issued before the rest of the set-up
  // arithmetic, which then runs while they are in flight. (Rows are padded
  // to a multiple of 4 keys: a load at i < n stays in the row.)
  uint4 k4first[KPT / 4];
#pragma unroll
  for (int r = 0; r < KPT / 4; r++) {
    const int i = 4 * (tid + r * NT);
    k4first[r] = i < min(CL, C) ? *reinterpret_cast<const uint4*>(keyg + i)
                                : make_uint4(0u, 0u, 0u, 0u);
  }
  const float2* mmu = a.mm + (int64_t)u * a.NB;
  float2 mmr[4];
#pragma unroll
  for (int e = 0; e < 4; e++) {
    const int j = 64 * e + lane;
    mmr[e] = j < a.NB ? mmu[j] : make_float2(INFINITY, -INFINITY);
  }
  const int b = u / a.H, h = u - b * a.H;
  const int r16 = lane & 15, kg = lane >> 4;
  const int G = a.G, W = a.W;
  const int K_r = a.K_r, K_e = a.K_e;
  const int NP = BIG ? (C + CL - 1) / CL : 1;  // LDS passes over the keys
  const int64_t uC = (int64_t)u * C;
  const int n_x = a.n_st + a.n_pend;  // steady rows, then pending rows
  // (32-bit products whenever they fit: a 64-bit division is ~150 instructions)
  const int s_lo = n_x < (1 << 24) ? n_x * w / W : (int)((int64_t)n_x * w / W);
  const int s_hi = n_x < (1 << 24) ? n_x * (w + 1) / W : (int)((int64_t)n_x * (w + 1) / W);
  // own groups w, w + W, ... of the ng groups; own index k -> cluster id
  const int ng = (C + GRP - 1) / GRP;
  const int n_own = ng > w ? ((ng - 1 - w) / W + 1) * GRP : 0;
  const int n_chunks = max(1, (n_own + NT - 1) / NT);
  auto own_id = [&](int k) { return (w + (k / GRP) * W) * GRP + (k % GRP); };

  // ---- prologue: query rows to LDS; the first chunk's own-cluster data into
  // registers. All of these loads are issued before the selection starts. ----
  // (the query piece of this thread, GS rows of QB bytes in 16-byte pieces,
  // at most one per thread, goes to LDS once the histogram is built, so that
  // no wait for it precedes the selection's loads)
  constexpr int QB = D * (DT == WI_BF16 ? 2 : 4);  // bytes per query row
  static_assert(GS * QB / 16 <= NT, "one query piece per thread");
  uint4 qpiece = make_uint4(0u, 0u, 0u, 0u);
  {
    const uint8_t* qg = reinterpret_cast<const uint8_t*>(a.q) +
                        ((int64_t)b * a.Hq + (int64_t)h * G) * QB;
    if (tid < GS * QB / 16 && tid / (QB / 16) < G) qpiece = reinterpret_cast<const uint4*>(qg)[tid];
  }
  int sz0, blk0;
  f32x4_t sl0[GS / 4];
  {
    const int id0 = own_id(tid);
    const int idc = tid < n_own && id0 < C ? id0 : 0;
    sz0 = a.size[uC + idc];
    blk0 = a.block_off[(int64_t)u * (C + 1) + idc];
    const f32x4_t* sp = reinterpret_cast<const f32x4_t*>(a.S + (uC + idc) * GS);
#pragma unroll
    for (int g4 = 0; g4 < GS / 4; g4++) sl0[g4] = sp[g4];
  }

  // ---- keys of pass p (ids [p CL, p CL + n)): loads, then LDS stores -------
  auto stage_load = [&](int p, uint4* k4) {
    const int c0 = p * CL, n = min(CL, C - c0);
#pragma unroll
    for (int r = 0; r < KPT / 4; r++) {
      const int i = 4 * (tid + r * NT);
      // rows are padded to a multiple of 4 keys: a load at i < n stays in the row
      k4[r] = i < n ? *reinterpret_cast<const uint4*>(keyg + c0 + i) : make_uint4(0u, 0u, 0u, 0u);
    }
  };
  float lo = INFINITY, hi = -INFINITY, inv = 0.f, off = 0.f;
  auto stage_store = [&](int p, const uint4* k4, bool count) {
    const int n = min(CL, C - p * CL);
#pragma unroll
    for (int r = 0; r < KPT / 4; r++) {
      const int i = 4 * (tid + r * NT);
      *reinterpret_cast<uint4*>(keys + i) = k4[r];  // (i < CL: slots past the unit unused)
      if (count) {
        const uint32_t kk[4] = {k4[r].x, k4[r].y, k4[r].z, k4[r].w};
        int bn[4];
#pragma unroll
        for (int e = 0; e < 4; e++) {
          // keys past the unit count in the lane's spare slot hist[NBINS +
          // lane] (one per lane: no two lanes of an atomic share it) and carry
          // the no-bin mark (never a pivot's)
          const bool ok = i + e < n;
          const int bb = bin_of(kk[e], off, inv);
          bn[e] = ok ? bb : 0xFFFF;
          atomicAdd(&hist[ok ? bb : NBINS + lane], 1);
        }
        // (pass 0's bins are kept for the candidate scan of a one-pass unit;
        // every slot of the CL-entry array is written)
        *reinterpret_cast<uint2*>(kbin + i) =
            make_uint2((uint32_t)bn[0] | ((uint32_t)bn[1] << 16), (uint32_t)bn[2] | ((uint32_t)bn[3] << 16));
      }
    }
  };
  // C > CL: the keys of pass p straight into registers, each load issued
  // unconditionally (index clamped into the unit's key row, padded to a
  // multiple of 4; keys at i >= n are ignored), so that the next pass's
  // loads can be in flight while this pass is processed
  auto key_load = [&](int p, uint4* k4) {
    const int c0 = p * CL, n = min(CL, C - c0);
    const int last = ((n + 3) & ~3) - 4;
#pragma unroll
    for (int r = 0; r < KPT / 4; r++)
      k4[r] = *reinterpret_cast<const uint4*>(keyg + c0 + min(4 * (tid + r * NT), last));
  };
  auto count_keys = [&](int p, const uint4* k4) {
    const int n = min(CL, C - p * CL);
#pragma unroll
    for (int r = 0; r < KPT / 4; r++) {
      const int i = 4 * (tid + r * NT);
      const uint32_t kk[4] = {k4[r].x, k4[r].y, k4[r].z, k4[r].w};
#pragma unroll
      for (int e = 0; e < 4; e++)
        atomicAdd(&hist[i + e < n ? bin_of(kk[e], off, inv) : NBINS + lane], 1);
    }
  };
  // re-stage pass p for a later scan (C > CL only); leaves keys ready in LDS
  auto restage = [&](int p) {
    uint4 k4[KPT / 4];
    __syncthreads();
    stage_load(p, k4);
    stage_store(p, k4, false);
    __syncthreads();
  };

  // ---- 1a.-1b. key range (from the score step) and histogram -----------------
  for (int i = tid; i < NBINS; i += NT) hist[i] = 0;
  if (tid < 2) ncand[tid] = 0;
  // candidate lists start as comps 0, below every candidate's (whose low word
  // 2^32 - 1 - id is positive), so the ranking can read them four at a time
  // past nc
  for (int i = tid; i < 2 * CAND_MAX; i += NT) cand[i] = 0ull;
  {
    uint4 k4[KPT / 4];
#pragma unroll
    for (int r = 0; r < KPT / 4; r++) k4[r] = k4first[r];
    // every wave reduces the score workgroups' ranges the same way
#pragma unroll
    for (int e = 0; e < 4; e++) {
      lo = fminf(lo, mmr[e].x);
      hi = fmaxf(hi, mmr[e].y);
    }
#pragma unroll 1
    for (int j0 = 256; j0 < a.NB; j0 += 256) {
      float2 r[4];
#pragma unroll
      for (int e = 0; e < 4; e++) {
        const int j = j0 + 64 * e + lane;
        r[e] = j < a.NB ? mmu[j] : make_float2(INFINITY, -INFINITY);
      }
#pragma unroll
      for (int e = 0; e < 4; e++) {
        lo = fminf(lo, r[e].x);
        hi = fmaxf(hi, r[e].y);
      }
    }
    lo = -wave_max_u(-lo);
    hi = wave_max_u(hi);
    __syncthreads();  // histogram cleared
    inv = hi > lo ? (float)NBINS / (hi - lo) : 0.f;
    off = -lo * inv;
    stage_store(0, k4, true);
    if constexpr (BIG) {
      // passes 1 .. NP-1: pass p + 1 loads while pass p is counted
      uint4 kb[KPT / 4];
      key_load(1, k4);
#pragma unroll 1
      for (int p = 1; p < NP; p += 2) {
        key_load(min(p + 1, NP - 1), kb);
        count_keys(p, k4);
        key_load(min(p + 2, NP - 1), k4);
        if (p + 1 < NP) count_keys(p + 1, kb);
      }
    }
  }
  if (tid < GS * QB / 16) reinterpret_cast<uint4*>(qs)[tid] = qpiece;
  __syncthreads();

  // ---- 1c. pivot bins: thread t owns bins NBINS-1-4t down to NBINS-4-4t ----
  const int M0 = K_r, M1 = K_r + K_e;
  const bool need0 = M0 > 0 && M0 < C, need1 = M1 > 0 && M1 < C;
  {
    const int4 h4 = *reinterpret_cast<const int4*>(hist + NBINS - 4 - BPT * tid);
    const int hb[4] = {h4.w, h4.z, h4.y, h4.x};  // descending bins
    const int v1[1] = {hb[0] + hb[1] + hb[2] + hb[3]};
    int off[1], tot[1];
    block_scan<1>(v1, off, tot, scan_lds);
#pragma unroll
    for (int t = 0; t < 2; t++) {
      const int m = t == 0 ? M0 : M1;
      int run = off[0];
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
      // M <= 0: nothing selected (flagged below); M >= C: everything selected
      const int m = tid == 0 ? M0 : M1;
      if (m <= 0) { pk[tid] = 0xFFFFFFFFu; pi[tid] = -1; }
      if (m >= C) { pk[tid] = 0u; pi[tid] = INT_MAX; }
    }
  }
  __syncthreads();
  const int b1 = need0 ? bsel[0] : -1, b2 = need1 ? bsel[1] : -1;

  // ---- warm the L2 with the data the first chunk will most likely read -------
  // Once the pivot bins are known, an own cluster in a bin at or above the
  // retrieval pivot's bin may be retrieved, one at or above the estimation
  // pivot's bin may be selected. Their value sums (thread per cluster, one
  // dword per 128-byte line) and key/value rows (wave per cluster, first
  // 4 KB of each) are requested now, while the selection finishes; the
  // loaded words are only folded together at the end of the kernel, so
  // nothing waits for them.
  constexpr int RB = D * (DT == WI_BF16 ? 2 : 4);  // bytes per K/V row
  const uint8_t* kb8 = reinterpret_cast<const uint8_t*>(a.kblk) + (int64_t)u * a.capT * RB;
  const uint8_t* vb8 = reinterpret_cast<const uint8_t*>(a.vblk) + (int64_t)u * a.capT * RB;
  const uint8_t* sk8 = reinterpret_cast<const uint8_t*>(a.stk) + (int64_t)u * a.n_st * RB;
  const uint8_t* sv8 = reinterpret_cast<const uint8_t*>(a.stv) + (int64_t)u * a.n_st * RB;
  // row x of the steady-then-pending rows (x < n_st + n_pend)
  const uint8_t* pk8 = a.n_pend > 0 ? reinterpret_cast<const uint8_t*>(a.pk) +
                                          (int64_t)u * a.seg_len * RB : sk8;
  const uint8_t* pv8 = a.n_pend > 0 ? reinterpret_cast<const uint8_t*>(a.pv) +
                                          (int64_t)u * a.seg_len * RB : sv8;
  const int n_st = a.n_st;
  auto xrow = [&](const uint8_t* st8, const uint8_t* p8, int x) {
    return x < n_st ? st8 + (int64_t)x * RB : p8 + (int64_t)(x - n_st) * RB;
  };
  // row `row` of the unit's blocks: from its cache slot sl when the block is
  // cached, else from the block pool (HBM, or the host tier when CACHED)
  const uint8_t* ck8 = CACHED ? reinterpret_cast<const uint8_t*>(a.ck) +
                                    (int64_t)u * a.nslot * (RB << a.lgT) : nullptr;
  const uint8_t* cv8 = CACHED ? reinterpret_cast<const uint8_t*>(a.cv) +
                                    (int64_t)u * a.nslot * (RB << a.lgT) : nullptr;
  auto brow = [&](const uint8_t* pool8, const uint8_t* cache8, int row, int sl) {
    if constexpr (CACHED) {
      if (sl >= 0 && sl < a.nslot)
        return cache8 + (((int64_t)sl << a.lgT) + (row & ((1 << a.lgT) - 1))) * RB;
    }
    return pool8 + (int64_t)row * RB;
  };
  // a valid row of at least RB bytes, read by lanes without an item
  const uint8_t* dummy = reinterpret_cast<const uint8_t*>(a.vsum + uC * D);
  const int lgT = a.lgT;
  // kept apart until the end so that no instruction waits for them
  uint32_t w4[4] = {0u, 0u, 0u, 0u}, wk[4] = {0u, 0u, 0u, 0u}, wst = 0u;
  {
    const int id0 = own_id(tid);
    const bool ok = tid < n_own && id0 < C && sz0 > 0;
    const int bn = ok ? bin_of(NP == 1 ? keys[id0] : keyg[id0], off, inv) : -1;
    const bool maybeS = ok && (M1 >= C || (need1 && bn >= b2));
    const bool maybeR = ok && (M0 >= C || (need0 && bn >= b1));
    const bool surelyR = ok && (M0 >= C || (need0 && bn > b1));
    if (maybeS && !surelyR) {
      const uint32_t* vp = reinterpret_cast<const uint32_t*>(a.vsum + (uC + id0) * D);
#pragma unroll
      for (int j = 0; j < 4; j++) w4[j] = vp[32 * j];
    }
    // up to 4 retrieval candidates per wave; lanes 0-31 read the key rows,
    // 32-63 the value rows, one 128-byte line each
    uint64_t cand = CACHED ? 0ull : __ballot(maybeR);
#pragma unroll
    for (int c = 0; c < 4; c++) {
      if (cand) {
        const int l = __builtin_ctzll(cand);
        cand &= cand - 1;
        const int cb = rdl(blk0, l), cn = rdl(sz0, l);
        const int off = (lane & 31) * 128;
        if (off < cn * RB)
          wk[c] = *reinterpret_cast<const uint32_t*>((lane < 32 ? kb8 : vb8) +
                                                     ((int64_t)cb << lgT) * RB + off);
      }
    }
    // the steady rows of this workgroup (wave 0)
    if (wv == 0) {
      const int off = (lane & 31) * 128;
      const int s_end = min(s_hi, n_st);  // the steady rows of the share
      if (s_lo < s_end && off < (s_end - s_lo) * RB)
        wst = *reinterpret_cast<const uint32_t*>((lane < 32 ? sk8 : sv8) +
                                                   (int64_t)s_lo * RB + off);
    }
  }

  // ---- 1d. keys of the pivot bins -------------------------------------------
  // pass p's keys: from LDS (one pass) or from registers k4r (C > CL). A
  // thread's bins are read (or computed) first; each wave then takes the
  // slots of its hits with one LDS atomic per target and writes them.
  auto cand_scan = [&](int p, const uint4* k4r) {
    const int n = min(CL, C - p * CL);
    int bns[KPT];
#pragma unroll
    for (int r = 0; r < KPT / 4; r++) {
      const int i = 4 * (tid + r * NT);
      if (k4r) {
        const uint32_t kr[4] = {k4r[r].x, k4r[r].y, k4r[r].z, k4r[r].w};
#pragma unroll
        for (int e = 0; e < 4; e++) bns[4 * r + e] = i + e < n ? bin_of(kr[e], off, inv) : -2;
      } else {
        // (keys past the unit carry the no-bin mark)
        const uint2 bb = *reinterpret_cast<const uint2*>(kbin + i);
        bns[4 * r] = (int)(bb.x & 0xFFFF);
        bns[4 * r + 1] = (int)(bb.x >> 16);
        bns[4 * r + 2] = (int)(bb.y & 0xFFFF);
        bns[4 * r + 3] = (int)(bb.y >> 16);
      }
    }
    // hit masks in vector registers (bit k: key k of this thread)
    uint32_t m0 = 0u, m1 = 0u;
#pragma unroll
    for (int k = 0; k < KPT; k++) {
      m0 |= (bns[k] == b1 ? 1u : 0u) << k;
      m1 |= (bns[k] == b2 ? 1u : 0u) << k;
    }
    const int c0 = __popc(m0), c1 = __popc(m1);
    const int i0 = wave_incl_scan(c0), i1 = wave_incl_scan(c1);
    const int t0 = rdl(i0, 63), t1 = rdl(i1, 63);
    if (t0 + t1 == 0) return;  // (wave-uniform)
    int base0 = 0, base1 = 0;
    if (lane == 0) {
      if (t0) base0 = atomicAdd(&ncand[0], t0);
      if (t1) base1 = atomicAdd(&ncand[1], t1);
    }
    int s0 = rdl(base0, 0) + i0 - c0, s1 = rdl(base1, 0) + i1 - c1;
    // this thread's hits, in key order (a later pass's keys are picked out of
    // the registers, so that no load is waited for here)
    uint32_t mm = m0 | m1;
    while (mm) {
      const int k = __builtin_ctz(mm);
      mm &= mm - 1u;
      const int idx = 4 * (tid + (k >> 2) * NT) + (k & 3);
      uint32_t kk;
      if (k4r) {
        kk = 0u;
#pragma unroll
        for (int j = 0; j < KPT; j++) {
          const uint4 q4 = k4r[j >> 2];
          const uint32_t x = (j & 3) == 0 ? q4.x : (j & 3) == 1 ? q4.y : (j & 3) == 2 ? q4.z : q4.w;
          kk = k == j ? x : kk;
        }
      } else {
        kk = keys[idx];
      }
      if ((m0 >> k) & 1u) {
        if (s0 < CAND_MAX) {
          cand[s0] = comp_of(kk, p * CL + idx);
        }
        s0++;
      }
      if ((m1 >> k) & 1u) {
        if (s1 < CAND_MAX) {
          cand[CAND_MAX + s1] = comp_of(kk, p * CL + idx);
        }
        s1++;
      }
    }
  };
  // (two code paths, so that the common one issues no global load and the
  // compiler puts no wait for outstanding loads in it; with C > CL pass
  // p + 1's keys load while pass p is scanned)
  if constexpr (!BIG) {
    cand_scan(0, nullptr);
  } else {
    uint4 ka[KPT / 4], kb[KPT / 4];
    key_load(0, ka);
#pragma unroll 1
    for (int p = 0; p < NP; p += 2) {
      key_load(min(p + 1, NP - 1), kb);
      cand_scan(p, ka);
      key_load(min(p + 2, NP - 1), ka);
      if (p + 1 < NP) cand_scan(p + 1, kb);
    }
  }
  __syncthreads();

  // ---- 1e. pivots: waves 4t .. 4t + 3 rank the comps of target t's bin, one
  // candidate per lane (candidate 64 (wv % 4) + lane), comparing against
  // four candidates per pair of LDS broadcast reads, one 64-bit compare each
  // (rank = number of larger comps; distinct ids make comps distinct) -------
  const int nc0 = ncand[0], nc1 = ncand[1];
  {
    const int t = wv >> 2, qw = wv & 3;
    const bool need = t == 0 ? need0 : need1;
    const int nc = t == 0 ? nc0 : nc1;
    if (need && nc <= CAND_MAX && 64 * qw < nc) {
      const int i = 64 * qw + lane;
      const uint64_t mine = i < nc ? cand[t * CAND_MAX + i] : 0ull;
      int rank = 0;
      const uint64_t* ct = cand + t * CAND_MAX;
#pragma unroll 4
      for (int j4 = 0; j4 < (nc + 3) / 4; j4++) {
        // (entries past nc are zero and never larger)
        const ulonglong2 c01 = reinterpret_cast<const ulonglong2*>(ct)[2 * j4];
        const ulonglong2 c23 = reinterpret_cast<const ulonglong2*>(ct)[2 * j4 + 1];
        rank += (c01.x > mine) + (c01.y > mine) + (c23.x > mine) + (c23.y > mine);
      }
      if (i < nc && rank == bneed[t] - 1) {
        pk[t] = (uint32_t)(mine >> 32);
        pi[t] = (int)(0xFFFFFFFFu - (uint32_t)mine);
      }
    }
  }
  if ((need0 && nc0 > CAND_MAX) || (need1 && nc1 > CAND_MAX)) {
    // radix select over comp among the keys of the pivot bin: the need-th
    // largest comp there is the pivot
#pragma unroll 1
    for (int t = 0; t < 2; t++) {
      const bool need = t == 0 ? need0 : need1;
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
          if (NP > 1) restage(p);
          const int n = min(CL, C - p * CL);
#pragma unroll 1
          for (int i = tid; i < n; i += NT) {
            const uint32_t kk = keys[i];
            if (bin_of(kk, off, inv) == bs) {
              const uint64_t comp = comp_of(kk, p * CL + i);
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
  const uint64_t cR = comp_of(pk[0], pi[0]), cS = comp_of(pk[1], pi[1]);
  const bool noneR = M0 <= 0, noneS = M1 <= 0;

  // ---- 2.-3. own clusters, NT at a time, then their items --------------------
  float* pb = Pbuf + wv * PI_MAX * GS;  // this wave's weights p[item][head]

  // Online softmax state of this wave. Lanes of column r16 (r16, r16 + 16,
  // r16 + 32, r16 + 48) track head r16: m_run is their common running
  // maximum, l_run each lane's share of the running denominator. acc[g][.]
  // holds dims 2 lane, 2 lane + 1 of the running numerator of head g.
  float m_run = -INFINITY, l_run = 0.f;
  // VALU path: acc[g][.] holds dims 2 lane, 2 lane + 1 of the running
  // numerator of head g. MFMA path: acct[i] element jj holds
  // O[head 4 kg + jj][dim 8 r16 + i].
  float acc[MPV ? 1 : GS][2];
#pragma unroll
  for (int g = 0; g < (MPV ? 1 : GS); g++) acc[g][0] = acc[g][1] = 0.f;
  f32x4_t acct[MPV ? 8 : 1];
#pragma unroll
  for (int i = 0; i < (MPV ? 8 : 1); i++) acct[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  bool acc_live = false;  // (wave-uniform) acct holds a weighted item

  // own clusters in passes of PASS_CHUNKS(GS) chunks of NT: the item lists of
  // a pass's chunks are gathered (appended) before its items run. The first
  // pass is peeled off the loop, so that its code joins no path holding later
  // passes' loads (the compiler would otherwise place waits there that also
  // cover the warm-up loads)
  constexpr int PC = PASS_CHUNKS(GS);
  auto chunk = [&](const int c0) {
    // (i) zones of the pass's clusters and its item lists. Chunk 0's cluster
    // data was loaded at kernel start; a later chunk loads its own inside its
    // branch. Each branch consumes what it loads, so the compiler places no
    // wait for other outstanding loads after it.
    int nR = 0, nRtok = 0, nE = 0;  // running list lengths over the pass
    auto setup = [&](int ch, int n, int blk, const f32x4_t* sl) {
      const int k = ch * NT + tid;
      const int id = own_id(k);
      const bool ok = k < n_own && id < C;
      const int idc = ok ? id : 0;
      const uint32_t kk = NP == 1 ? keys[idc] : keyg[idc];
      const uint64_t comp = comp_of(kk, id);
      const bool inS = ok && !noneS && comp >= cS;
      const bool inR = inS && !noneR && comp >= cR;
      const bool inE = inS && !inR;
      if (a.zone && ok) a.zone[uC + id] = inR ? 1 : (inE ? 2 : 0);
      const bool rT = inR && n > 0, eT = inE && n > 0;  // zones with members
      // (the two flags share one scanned int: at most NT of each per chunk)
      const int v2[2] = {(int)rT | ((int)eT << 16), rT ? n : 0};
      int off2[2], tot2[2];
      block_scan<2>(v2, off2, tot2, scan_lds);
      const int oR = off2[0] & 0xFFFF, oE = off2[0] >> 16;
      if (rT) {
        Rtok[nR + oR] = nRtok + off2[1];
        Rblk[nR + oR] = blk;
      }
      if (eT) {
        Eid[nE + oE] = id;
        Esz[nE + oE] = (float)n;
        float* el = Elog + (nE + oE) * GS;
#pragma unroll
        for (int g4 = 0; g4 < GS / 4; g4++) *reinterpret_cast<f32x4_t*>(el + 4 * g4) = sl[g4];
      }
      nR += tot2[0] & 0xFFFF;
      nRtok += tot2[1];
      nE += tot2[0] >> 16;
    };
    const int c1 = min(c0 + PC, n_chunks);
#pragma unroll 1
    for (int ch = c0; ch < c1; ch++) {
      if (ch == 0) {
        setup(0, sz0, blk0, sl0);
      } else {
        const int k = ch * NT + tid;
        const int id = own_id(k);
        const int idc = k < n_own && id < C ? id : 0;
        const int n = a.size[uC + idc];
        const int blk = a.block_off[(int64_t)u * (C + 1) + idc];
        // estimation logits only for estimation clusters when the key is on
        // chip (one key pass); with several passes the key would cost one
        // more round trip, so every own cluster's logits are read
        bool wantS = true;
        if constexpr (!BIG) {
          const uint64_t comp = comp_of(keys[idc], id);
          wantS = !noneS && comp >= cS && (noneR || comp < cR);
        }
        f32x4_t sl[GS / 4];
        const f32x4_t* sp = reinterpret_cast<const f32x4_t*>(a.S + (uC + idc) * GS);
#pragma unroll
        for (int g4 = 0; g4 < GS / 4; g4++) sl[g4] = wantS ? sp[g4] : f32x4_t{0.f, 0.f, 0.f, 0.f};
        setup(ch, n, blk, sl);
      }
    }
    __syncthreads();
    const int ch = c0;  // (the first pass holds the steady tokens)
    // token items: the own steady tokens (first chunk only), then the chunk's
    // retrieved tokens; estimation items: the chunk's estimation clusters.
    // Wave wv takes token blocks (TB tokens) wv, wv + NW, ... and estimation
    // blocks (EB clusters) NW - 1 - wv, 2 NW - 1 - wv, ..., so that small
    // chunks spread both kinds of work over all waves.
    const int nS = ch == 0 ? s_hi - s_lo : 0;
    const int nT = nS + nRtok;
    const int nTB = (nT + TB - 1) / TB, nEB = (nE + EB - 1) / EB;
    const int s0 = nR > 1 ? 1 << (31 - __clz(nR - 1)) : 0;  // binary-search stride

#pragma unroll 1
    for (int it = 0; wv + it * NW < nTB || NW - 1 - wv + it * NW < nEB; it++) {
      const int t0 = (wv + it * NW) * TB, e0 = (NW - 1 - wv + it * NW) * EB;
      const int ntw = max(0, min(TB, nT - t0)), new_ = max(0, min(EB, nE - e0));
      // (a) rows: lane r16 of tile j holds token item t0 + 16 j + r16 (steady
      // row, or a slot of its retrieved cluster found by binary search)
      // (the tiles' searches advance together: one LDS round trip per step)
      int rowj[NTILE], pos[NTILE], tk[NTILE];
      bool srch[NTILE];
#pragma unroll
      for (int j = 0; j < NTILE; j++) {
        const int item = t0 + 16 * j + r16;
        tk[j] = item - nS;
        srch[j] = item < nT && tk[j] >= 0;
        pos[j] = 0;
      }
#pragma unroll 1
      for (int s = s0; s > 0; s >>= 1) {
#pragma unroll
        for (int j = 0; j < NTILE; j++)
          if (srch[j] && pos[j] + s < nR && Rtok[pos[j] + s] <= tk[j]) pos[j] += s;
      }
#pragma unroll
      for (int j = 0; j < NTILE; j++) {
        const int item = t0 + 16 * j + r16;
        rowj[j] = item < nS ? s_lo + item
                            : (item < nT ? (Rblk[pos[j]] << lgT) + (tk[j] - Rtok[pos[j]]) : 0);
      }
      // cache slot of each retrieved row's block (-1: not cached)
      int slj[NTILE];
#pragma unroll
      for (int j = 0; j < NTILE; j++) {
        slj[j] = -1;
        if constexpr (CACHED) {
          const int item = t0 + 16 * j + r16;
          if (item >= nS && item < nT) slj[j] = a.b2s[(int64_t)u * a.nblk + (rowj[j] >> lgT)];
        }
      }
      // (b) loads: keys in the MFMA layout, two value dims per lane of every
      // token, the estimation clusters' value sums. Tiles and groups of rows
      // with no item issue no loads (ntw and new_ are uniform over the wave):
      // most waves carry only one kind of item when a workgroup owns few.
      uint4 ka[NTILE][NKL];
#pragma unroll
      for (int j = 0; j < NTILE; j++) {
        if (16 * j < ntw) {
          const int item = t0 + 16 * j + r16;
          const uint8_t* kp;
          if constexpr (PLAIN)
            kp = item < nT ? (item < nS ? sk8 : kb8) + (int64_t)rowj[j] * RB : dummy;
          else
            kp = item < nT ? (item < nS ? xrow(sk8, pk8, rowj[j])
                                        : brow(kb8, ck8, rowj[j], slj[j]))
                           : dummy;
#pragma unroll
          for (int s = 0; s < NKL; s++) {
            if constexpr (DT == WI_BF16)
              ka[j][s] = *reinterpret_cast<const uint4*>(kp + (32 * s + 8 * kg) * 2);
            else
              ka[j][s] = *reinterpret_cast<const uint4*>(kp + (32 * kg + 4 * s) * 4);
          }
        } else {
#pragma unroll
          for (int s = 0; s < NKL; s++) ka[j][s] = make_uint4(0u, 0u, 0u, 0u);
        }
      }
      // values. bf16: in the B layout of the weights-by-values MFMA -- lane
      // (r16, kg) reads dims 8 r16 .. 8 r16 + 7 (16 bytes) of its eight
      // tokens tau(kg, s) = 16 (s / 4) + 4 kg + s % 4, s = 0..7, taking each
      // token's row from the lane that found it; a token past the block reads
      // nothing and is zero. fp32: two dims per lane of every token.
      uint4 vt8[MPV ? 8 : 1];
      uint2 vr[MPV ? 1 : TB];  // fp32: dims 2 lane, 2 lane + 1
      if constexpr (MPV) {
#pragma unroll
        for (int s = 0; s < 8; s++) {
          const int tok = 16 * (s >> 2) + 4 * kg + (s & 3);
          vt8[s] = make_uint4(0u, 0u, 0u, 0u);
          if (16 * (s >> 2) < ntw) {
            const int row = __shfl(rowj[s >> 2], tok & 15, 64);
            const int sl = CACHED ? __shfl(slj[s >> 2], tok & 15, 64) : -1;
            if (tok < ntw) {
              const uint8_t* vpt;
              if constexpr (PLAIN)
                vpt = (t0 + tok < nS ? sv8 : vb8) + (int64_t)row * RB;
              else
                vpt = t0 + tok < nS ? xrow(sv8, pv8, row) : brow(vb8, cv8, row, sl);
              vt8[s] = *reinterpret_cast<const uint4*>(vpt + 16 * r16);
            }
          }
        }
      }
#pragma unroll
      for (int t8 = 0; t8 < (MPV ? 0 : TB); t8 += 8) {
        if (t8 < ntw) {
#pragma unroll
          for (int t = t8; t < t8 + 8; t++) {
            const int row = rdl(rowj[t / 16], t % 16);
            const int sl = CACHED ? rdl(slj[t / 16], t % 16) : -1;
            const uint8_t* vpt;
            if constexpr (PLAIN)
              vpt = t < ntw ? (t0 + t < nS ? sv8 : vb8) + (int64_t)row * RB : dummy;
            else
              vpt = t < ntw ? (t0 + t < nS ? xrow(sv8, pv8, row) : brow(vb8, cv8, row, sl))
                            : dummy;
            if constexpr (DT == WI_BF16)
              vr[t].x = *reinterpret_cast<const uint32_t*>(vpt + 4 * lane);
            else
              vr[t] = *reinterpret_cast<const uint2*>(vpt + 8 * lane);
          }
        } else {
#pragma unroll
          for (int t = t8; t < t8 + 8; t++) vr[t] = make_uint2(0u, 0u);
        }
      }
      // estimation value sums. MFMA path: lane (r16, kg) reads dims 8 r16 ..
      // 8 r16 + 7 (32 bytes) of the value sums of clusters e0 + 4 kg + jj,
      // jj = 0..3 (the clusters whose logits it holds below); VALU path: two
      // dims per lane of every cluster of the block.
      uint4 vse[MPV ? 8 : 1];  // [2 jj + half]
      float2 vs[MPV ? 1 : EB];
      if constexpr (MPV) {
#pragma unroll
        for (int jj = 0; jj < 4; jj++) {
          const int e = 4 * kg + jj;
          vse[2 * jj] = vse[2 * jj + 1] = make_uint4(0u, 0u, 0u, 0u);
          if (e < new_) {
            const uint4* vp = reinterpret_cast<const uint4*>(a.vsum + (uC + Eid[e0 + e]) * D + 8 * r16);
            vse[2 * jj] = vp[0];
            vse[2 * jj + 1] = vp[1];
          }
        }
      }
#pragma unroll
      for (int e4 = 0; e4 < (MPV ? 0 : EB); e4 += 4) {
        if (e4 < new_) {
#pragma unroll
          for (int e = e4; e < e4 + 4; e++) {
            const int ide = e < new_ ? Eid[e0 + e] : 0;
            vs[e] = *reinterpret_cast<const float2*>(a.vsum + (uC + ide) * D + 2 * lane);
          }
        } else {
#pragma unroll
          for (int e = e4; e < e4 + 4; e++) vs[e] = make_float2(0.f, 0.f);
        }
      }
      // estimation logits in the head-per-column layout: lane (r16, kg) holds
      // clusters e0 + 4 kg + jj, head r16
      float ze[4], me[4];
#pragma unroll
      for (int jj = 0; jj < 4; jj++) {
        const int e = 4 * kg + jj;
        const bool v = e < new_ && r16 < G;
        ze[jj] = v ? Elog[(e0 + e) * GS + r16] : -INFINITY;
        me[jj] = v ? Esz[e0 + e] : 0.f;
      }
      // (c) token logits: z[token 16 j + 4 kg + jj][head r16]. B operand:
      // bf16: lane supplies q[head r16][dims 32 s + 8 kg .. + 8], s = 0..3;
      // fp32: q[head r16][dims 32 kg + 4 s .. + 4]. Query rows >= G are zero.
      uint4 bq[NKL];
#pragma unroll
      for (int s = 0; s < NKL; s++) {
        if constexpr (DT == WI_BF16)
          bq[s] = *reinterpret_cast<const uint4*>(qs + (min(r16, GS - 1) * D + 32 * s + 8 * kg) * 2);
        else
          bq[s] = *reinterpret_cast<const uint4*>(qs + (min(r16, GS - 1) * D + 32 * kg + 4 * s) * 4);
      }
      float zt[NTILE][4];
#pragma unroll
      for (int j = 0; j < NTILE; j++) {
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
          zt[j][jj] = (16 * j + 4 * kg + jj < ntw && r16 < G) ? za[jj] * a.scale : -INFINITY;
      }
      // (d) online softmax per head (column): maximum over the block, the
      // rescale of the running state, weights and this lane's denominator share
      float mx = m_run;
#pragma unroll
      for (int jj = 0; jj < 4; jj++) {
#pragma unroll
        for (int j = 0; j < NTILE; j++) mx = fmaxf(mx, zt[j][jj]);
        mx = fmaxf(mx, ze[jj]);
      }
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float alpha = m_run == -INFINITY ? 0.f : ex<DT>(m_run - mx);
      m_run = mx;
      float ls = 0.f;
      float pt[NTILE][4];  // token weights, head r16, tokens 16 j + 4 kg + jj
#pragma unroll
      for (int j = 0; j < NTILE; j++) {
#pragma unroll
        for (int jj = 0; jj < 4; jj++) {
          const float p = zt[j][jj] == -INFINITY ? 0.f : ex<DT>(zt[j][jj] - mx);
          pt[j][jj] = p;
          ls += p;
          if (!MPV && r16 < GS) pb[(16 * j + 4 * kg + jj) * GS + r16] = p;
        }
      }
      float pe[4];  // estimation weights, head r16, clusters e0 + 4 kg + jj
#pragma unroll
      for (int jj = 0; jj < 4; jj++) {
        const float p = ze[jj] == -INFINITY ? 0.f : ex<DT>(ze[jj] - mx);
        pe[jj] = p;
        ls = fmaf(me[jj], p, ls);
        if (!MPV && r16 < GS) pb[(TB + 4 * kg + jj) * GS + r16] = p;
      }
      l_run = fmaf(l_run, alpha, ls);
#pragma unroll
      for (int g = 0; g < (MPV ? 0 : GS); g++) {
        const float ag = rdlf(alpha, g);
        acc[g][0] *= ag;
        acc[g][1] *= ag;
      }
      if constexpr (MPV) {
        // the accumulator's rows are heads 4 kg + jj
        if (acc_live && __ballot(r16 < G && alpha != 1.f) != 0) {
          float ah[4];
#pragma unroll
          for (int jj = 0; jj < 4; jj++) ah[jj] = __shfl(alpha, 4 * kg + jj, 64);
#pragma unroll
          for (int i = 0; i < 8; i++) {
#pragma unroll
            for (int jj = 0; jj < 4; jj++) acct[i][jj] *= ah[jj];
          }
        }
      }
      // the weights written above are read back by every lane of the wave
      // (a wave's LDS accesses complete in issue order)
      if constexpr (!MPV) {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      }
      // (e) sum_i p_i v_i over the block's tokens, then its estimation clusters.
      // MFMA path: per 16 output dims, O[head][dim] += P[head][k] B[k][dim]
      // over 32 k-slots, the weights split into two bf16 parts (hi: p
      // truncated, lo: the exact remainder truncated; together within 2^-14
      // of p). Lane (r16, kg) holds P[head r16][k] for k-slots 8 kg .. 8 kg + 7
      // and B[k][8 r16 + i] (dim tile i), and receives O[head 4 kg + jj][8 r16
      // + i] in element jj of acct[i]. Tokens: slot 8 kg + s is token
      // tau(kg, s), B = its bf16 values. Estimation clusters: slots 8 kg + 2 jj
      // and 8 kg + 2 jj + 1 are cluster e0 + 4 kg + jj, B = the two bf16 parts
      // (truncation, truncated remainder) of its float32 value sum.
      if constexpr (MPV) {
        if (new_ > 0) {
          uint32_t ph[4], pl[4];
#pragma unroll
          for (int jj = 0; jj < 4; jj++) {
            const uint32_t h0 = __float_as_uint(pe[jj]) & 0xFFFF0000u;
            const uint32_t r0 = __float_as_uint(pe[jj] - __uint_as_float(h0)) & 0xFFFF0000u;
            ph[jj] = (h0 >> 16) | h0;
            pl[jj] = (r0 >> 16) | r0;
          }
          const bf16x8_t a_hi = __builtin_bit_cast(bf16x8_t, make_uint4(ph[0], ph[1], ph[2], ph[3]));
          const bf16x8_t a_lo = __builtin_bit_cast(bf16x8_t, make_uint4(pl[0], pl[1], pl[2], pl[3]));
#pragma unroll
          for (int i = 0; i < 8; i++) {
            uint32_t bv[4];
#pragma unroll
            for (int jj = 0; jj < 4; jj++) {
              const uint4 x = vse[2 * jj + (i >> 2)];
              const uint32_t vb = (i & 3) == 0 ? x.x : (i & 3) == 1 ? x.y : (i & 3) == 2 ? x.z : x.w;
              const uint32_t hb = vb & 0xFFFF0000u;
              const uint32_t rb = __float_as_uint(__uint_as_float(vb) - __uint_as_float(hb));
              bv[jj] = (hb >> 16) | (rb & 0xFFFF0000u);
            }
            const bf16x8_t bb = __builtin_bit_cast(bf16x8_t, make_uint4(bv[0], bv[1], bv[2], bv[3]));
            acct[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a_hi, bb, acct[i], 0, 0, 0);
            acct[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a_lo, bb, acct[i], 0, 0, 0);
          }
          acc_live = true;
        }
        if (ntw > 0) {
          uint32_t ph[4], pl[4];
#pragma unroll
          for (int q = 0; q < 4; q++) {
            const float p0 = pt[q >> 1][2 * (q & 1)], p1 = pt[q >> 1][2 * (q & 1) + 1];
            const uint32_t h0 = __float_as_uint(p0) & 0xFFFF0000u;
            const uint32_t h1 = __float_as_uint(p1) & 0xFFFF0000u;
            const uint32_t r0 = __float_as_uint(p0 - __uint_as_float(h0));
            const uint32_t r1 = __float_as_uint(p1 - __uint_as_float(h1));
            ph[q] = (h0 >> 16) | h1;
            pl[q] = (r0 >> 16) | (r1 & 0xFFFF0000u);
          }
          const bf16x8_t a_hi = __builtin_bit_cast(bf16x8_t, make_uint4(ph[0], ph[1], ph[2], ph[3]));
          const bf16x8_t a_lo = __builtin_bit_cast(bf16x8_t, make_uint4(pl[0], pl[1], pl[2], pl[3]));
#pragma unroll
          for (int i = 0; i < 8; i++) {
            uint32_t bv[4];
#pragma unroll
            for (int q = 0; q < 4; q++) {
              const uint4 x = vt8[2 * q], y = vt8[2 * q + 1];
              const uint32_t xd = (i >> 1) == 0 ? x.x : (i >> 1) == 1 ? x.y : (i >> 1) == 2 ? x.z : x.w;
              const uint32_t yd = (i >> 1) == 0 ? y.x : (i >> 1) == 1 ? y.y : (i >> 1) == 2 ? y.z : y.w;
              bv[q] = __builtin_amdgcn_perm(yd, xd, (i & 1) ? 0x07060302u : 0x05040100u);
            }
            const bf16x8_t bb = __builtin_bit_cast(bf16x8_t, make_uint4(bv[0], bv[1], bv[2], bv[3]));
            acct[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a_hi, bb, acct[i], 0, 0, 0);
            acct[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a_lo, bb, acct[i], 0, 0, 0);
          }
          acc_live = true;
        }
      }
#pragma unroll
      for (int t = 0; t < (MPV ? 0 : TB); t++) {
        if (t < ntw) {
          float v0, v1;
          if constexpr (DT == WI_BF16) {
            v0 = __uint_as_float(vr[t].x << 16);
            v1 = __uint_as_float(vr[t].x & 0xFFFF0000u);
          } else {
            v0 = __uint_as_float(vr[t].x);
            v1 = __uint_as_float(vr[t].y);
          }
          const f32x4_t* pp = reinterpret_cast<const f32x4_t*>(pb + t * GS);
#pragma unroll
          for (int g4 = 0; g4 < GS / 4; g4++) {
            const f32x4_t p4 = pp[g4];
#pragma unroll
            for (int e = 0; e < 4; e++) {
              acc[4 * g4 + e][0] = fmaf(p4[e], v0, acc[4 * g4 + e][0]);
              acc[4 * g4 + e][1] = fmaf(p4[e], v1, acc[4 * g4 + e][1]);
            }
          }
        }
      }
#pragma unroll
      for (int e = 0; e < (MPV ? 0 : EB); e++) {
        if (e < new_) {
          const f32x4_t* pp = reinterpret_cast<const f32x4_t*>(pb + (TB + e) * GS);
#pragma unroll
          for (int g4 = 0; g4 < GS / 4; g4++) {
            const f32x4_t p4 = pp[g4];
#pragma unroll
            for (int c = 0; c < 4; c++) {
              acc[4 * g4 + c][0] = fmaf(p4[c], vs[e].x, acc[4 * g4 + c][0]);
              acc[4 * g4 + c][1] = fmaf(p4[c], vs[e].y, acc[4 * g4 + c][1]);
            }
          }
        }
      }
      // the next block rewrites the weights only after these reads
      if constexpr (!MPV) {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      }
    }
  };
  chunk(0);
#pragma unroll 1
  for (int c0 = PC; c0 < n_chunks; c0 += PC) chunk(c0);

  // the warm-up values are consumed (the condition never holds: K_r >= 0)
  const uint32_t warm = w4[0] ^ w4[1] ^ w4[2] ^ w4[3] ^ wk[0] ^ wk[1] ^ wk[2] ^ wk[3] ^ wst;
  if (warm == 0x9E3779B9u && K_r < 0) a.out[0] = 0.f;

  // ---- 4. merge the waves (fixed order), publish, count arrivals --------------
  // each wave's denominator: its column's four lane shares
  l_run += __shfl_xor(l_run, 16, 64);
  l_run += __shfl_xor(l_run, 32, 64);
  __syncthreads();  // the item lists and weights are dead; sacc reuses LDS
  float* sacc = reinterpret_cast<float*>(smem + L::SACC);
  if constexpr (MPV) {
    // this wave's rows of sacc from the MFMA layout
#pragma unroll
    for (int i = 0; i < 8; i++) {
#pragma unroll
      for (int jj = 0; jj < 4; jj++) {
        const int hh = 4 * kg + jj;
        if (hh < G) sacc[(wv * GS + hh) * D + 8 * r16 + i] = acct[i][jj];
      }
    }
  } else {
#pragma unroll
    for (int g = 0; g < GS; g++)
      if (g < G)
        *reinterpret_cast<float2*>(sacc + (wv * GS + g) * D + 2 * lane) =
            make_float2(acc[g][0], acc[g][1]);
  }
  if (lane < G) {
    wm[wv][lane] = m_run;
    wl[wv][lane] = l_run;
  }
  __syncthreads();
  float* pw = a.part + ((int64_t)u * W + w) * G * PART;
#pragma unroll 1
  for (int e = tid; e < G * D; e += NT) {
    const int g = e >> 7, t = e & (D - 1);
    float M = -INFINITY;
#pragma unroll
    for (int v = 0; v < NW; v++) M = fmaxf(M, wm[v][g]);
    float s = 0.f, l = 0.f;
#pragma unroll
    for (int v = 0; v < NW; v++) {
      const float f = wm[v][g] == -INFINITY ? 0.f : ex<DT>(wm[v][g] - M);
      s = fmaf(f, sacc[(v * GS + g) * D + t], s);
      l = fmaf(f, wl[v][g], l);
    }
    __hip_atomic_store(pw + g * PART + 2 + t, s, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (t == 0) {
      __hip_atomic_store(pw + g * PART, M, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(pw + g * PART + 1, l, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  // The arrival count is a release at agent scope: the workgroup barrier
  // orders every thread's partial stores before thread 0's count, which makes
  // them visible to the workgroup that observes the final count. That last
  // workgroup then acquires at agent scope before any thread reads a partial
  // (its barrier carries the acquire to the other threads).
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (tid == 0) {
    const bool last = __hip_atomic_fetch_add(&a.tix[u], 1, __ATOMIC_RELEASE,
                                             __HIP_MEMORY_SCOPE_AGENT) == W - 1;
    if (last) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    s_last = last;
  }
  __syncthreads();
  if (!s_last) return;

  // ---- 5. the last workgroup of the unit merges the W partials -------------
  // Wave by wave, with no workgroup barrier: a wave's 64 output elements
  // belong to one head g. Its lanes load their elements' accumulators (one
  // per partial; NV = 16, 32 or 64 >= W slots, slots v >= W repeat partial
  // W - 1 and get weight 0) and, lane v, the (m, l) of partial v; the weights
  // e^{m_v - M} and the denominator are formed across the wave and read back
  // lane by lane.
  const float* pu = a.part + (int64_t)u * W * G * PART;
  auto combine = [&](auto nv) {
    constexpr int NV = decltype(nv)::value;
#pragma unroll 1
    for (int e0 = wv * 64; e0 < G * D; e0 += NT) {
      const int g = e0 >> 7, t = (e0 & (D - 1)) + lane;
      float av[NV];
#pragma unroll
      for (int v = 0; v < NV; v++)
        av[v] = __hip_atomic_load(pu + ((int64_t)min(v, W - 1) * G + g) * PART + 2 + t,
                                  __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const int64_t ml = ((int64_t)min(lane, W - 1) * G + g) * PART;
      const float m0 = __hip_atomic_load(pu + ml, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const float l0 = __hip_atomic_load(pu + ml + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const float mv = lane < W ? m0 : -INFINITY;
      const float M2 = wave_max_u(mv);
      const float f = (mv == -INFINITY) ? 0.f : ex<DT>(mv - M2);  // weight of partial lane
      const float den = wave_sum_u(f * (lane < W ? l0 : 0.f));
      float num = 0.f;
#pragma unroll
      for (int v = 0; v < NV; v++) num = fmaf(rdlf(f, v), av[v], num);
      a.out[((int64_t)b * a.Hq + (int64_t)h * G + g) * D + t] = den > 0.f ? num / den : 0.f;
    }
  };
  if (W <= 16) combine(std::integral_constant<int, 16>{});
  else if (W <= 32) combine(std::integral_constant<int, 32>{});
  else combine(std::integral_constant<int, MAX_WG>{});
}

template <int DT, bool BIG, int MODE>
hipError_t launch_fused_big(const DecodeArgs& da, const FusedArgs& fa, hipStream_t s) {
  dim3 grid(da.W, da.g->U);
  if (da.GS == 4)
    WI_LAUNCH(K_FUSED, (fused_kernel<DT, 4, BIG, MODE>), grid, dim3(NT), 0, s, fa);
  else if (da.GS == 8)
    WI_LAUNCH(K_FUSED, (fused_kernel<DT, 8, BIG, MODE>), grid, dim3(NT), 0, s, fa);
  else
    WI_LAUNCH(K_FUSED, (fused_kernel<DT, 16, BIG, MODE>), grid, dim3(NT), 0, s, fa);
  return hipGetLastError();
}

template <int DT, int MODE>
hipError_t launch_fused_dt(const DecodeArgs& da, const FusedArgs& fa, hipStream_t s) {
  return fa.C > CL ? launch_fused_big<DT, true, MODE>(da, fa, s)
                   : launch_fused_big<DT, false, MODE>(da, fa, s);
}

template <int MODE>
hipError_t launch_fused_mode(const DecodeArgs& da, const FusedArgs& fa, hipStream_t s) {
  return da.g->dtype == WI_BF16 ? launch_fused_dt<WI_BF16, MODE>(da, fa, s)
                                : launch_fused_dt<WI_F32, MODE>(da, fa, s);
}

}  // namespace

hipError_t launch_fused(const DecodeArgs& da, const wi_index_bufs& bf, const void* q,
                        float* out, const DecodeWs& ws, bool want_lists, hipStream_t s,
                        const WaveBufArgs* wb) {
  const Geom& g = *da.g;
  FusedArgs fa;
  fa.key = ws.key;
  fa.S = ws.S;
  fa.mm = ws.mm;
  fa.NB = score_blocks(g);
  fa.size = bf.cluster_size;
  fa.block_off = bf.block_off;
  fa.kblk = bf.k_blocks;
  fa.vblk = bf.v_blocks;
  fa.stk = bf.steady_k;
  fa.stv = bf.steady_v;
  fa.vsum = bf.value_sum;
  fa.q = q;
  fa.out = out;
  fa.part = ws.part;
  fa.tix = ws.tix;
  fa.zone = want_lists ? ws.zone : nullptr;
  fa.C = g.C;
  fa.Cp = (g.C + 3) & ~3;
  fa.n_st = g.n_st;
  fa.n_pend = g.n_pend;
  fa.seg_len = g.seg_len;
  fa.pk = bf.pend_k;
  fa.pv = bf.pend_v;
  fa.G = da.G;
  fa.H = g.H;
  fa.Hq = da.Hq;
  fa.K_r = da.K_r;
  fa.K_e = da.K_e;
  fa.W = da.W;
  fa.lgT = g.T == 8 ? 3 : 2;
  fa.capT = g.cap * g.T;
  fa.scale = da.scale;
  fa.b2s = wb ? wb->block_slot : nullptr;
  fa.ck = wb ? wb->cache_k : nullptr;
  fa.cv = wb ? wb->cache_v : nullptr;
  fa.nblk = g.cap;
  fa.nslot = wb ? wb->n_slots : 0;
  if (wb) {
    // the blocks are read from the host tier (device-visible addresses)
    fa.kblk = wb->host_k;
    fa.vblk = wb->host_v;
    return launch_fused_mode<RM_CACHED>(da, fa, s);
  }
  return g.n_pend > 0 ? launch_fused_mode<RM_PEND>(da, fa, s)
                      : launch_fused_mode<RM_PLAIN>(da, fa, s);
}

}  // namespace wi
