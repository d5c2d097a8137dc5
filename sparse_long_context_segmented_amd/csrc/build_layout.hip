// Index build, final layout (RetroInfer, framerc blog section 2.2: KV kept
// in 2 KB physical blocks with a cluster -> block mapping table; section
// 3.1: one cluster's KV stored as contiguously as possible; section 2.1:
// per-cluster value sums kept with the centroids; techwalker article section
// 3: a small steady-zone buffer).
//
// Cluster c of a unit owns blocks [block_off[c], block_off[c+1]) with
// block_off the exclusive scan of ceil(n_c / T) over the unit's clusters in
// id order; its members fill the first n_c slots in ascending position and
// the rest of its last block holds token -1 and zero data, as do all blocks
// past block_off[C]. Value sums are float64 sums over members in ascending
// position, rounded to float32. Four workgroups share a segment (cluster c
// goes to workgroup c % 4); the member list is staged in LDS and each wave
// keeps 16 rows in flight, so the copy is not bound by dependent round trips.
#include "wi_internal.h"

namespace wi {
namespace {

constexpr int LT = 512;
constexpr int LW = LT / 64;
constexpr int LP = 4;  // workgroups per segment: cluster c goes to workgroup c % LP

// Per unit: first block of every segment, and blocks used by the unit.
__global__ __launch_bounds__(256) void seg_scan_kernel(Geom g, BuildWs ws) {
  const int u = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  __shared__ int wsum[4];
  __shared__ int run_s;
  if (tid == 0) run_s = 0;
  __syncthreads();
  for (int base = 0; base < g.n_seg; base += 256) {
    const int s = base + tid;
    const int v = s < g.n_seg ? ws.seg_blocks[(int64_t)u * g.n_seg + s] : 0;
    int x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(x, o, 64);
      if (lane >= o) x += y;
    }
    if (lane == 63) wsum[wv] = x;
    __syncthreads();
    int off = run_s;
    for (int w = 0; w < wv; w++) off += wsum[w];
    if (s < g.n_seg) ws.seg_bbase[(int64_t)u * g.n_seg + s] = off + x - v;
    const int tot = wsum[0] + wsum[1] + wsum[2] + wsum[3];
    __syncthreads();
    if (tid == 0) run_s += tot;
    __syncthreads();
  }
  if (tid == 0) ws.unit_used[u] = run_s;
}

template <int DT>
__global__ __launch_bounds__(LT) void layout_kernel(Geom g, const void* __restrict__ K,
                                                    const void* __restrict__ V,
                                                    wi_index_bufs bf, BuildWs ws) {
  constexpr int RB = D * (DT == WI_BF16 ? 2 : 4);  // row bytes
  constexpr int LPR = RB / 16;                     // lanes per row (16 or 32)
  constexpr int RPW = 64 / LPR;                    // rows per wave step
  __shared__ int lbo[MAX_K + 1];
  __shared__ int wsum[LW + 1];
  __shared__ int smemb[MAX_SEG];  // the segment's members, cluster order
  __shared__ int scoff[MAX_K], scsz[MAX_K];
  const int gs = blockIdx.x, u = gs / g.n_seg, s = gs % g.n_seg, part = blockIdx.y;
  const int n = seg_n(g, s), Cs = seg_c(g, s), cb = seg_cbase(g, s);
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int64_t pbase = (int64_t)u * g.n_idx + (int64_t)s * g.seg_len;
  const int64_t first = seg_first(g, s);
  const int b = u / g.H, h = u % g.H;
  const int64_t kvbase = (int64_t)b * g.sb + (int64_t)h * g.sh;
  const uint8_t* Kb = reinterpret_cast<const uint8_t*>(K) + kvbase * (RB / D);
  const uint8_t* Vb = reinterpret_cast<const uint8_t*>(V) + kvbase * (RB / D);
  const int64_t strow = g.st * (RB / D);  // bytes between tokens
  const int32_t* csz = bf.cluster_size + (int64_t)u * g.C + cb;
  const int* coff = ws.cl_off + (int64_t)u * g.C + cb;
  const int* memb = ws.members + pbase;
  const int seg_b0 = ws.seg_bbase[gs];
  const int T = g.T;

  // the member list and the clusters' sizes and offsets into LDS, so that a
  // row's address is one LDS read away
  for (int i = tid; i < n; i += LT) smemb[i] = memb[i];
  if (tid < Cs) {
    scsz[tid] = csz[tid];
    scoff[tid] = coff[tid];
  }
  // block offsets of the segment's clusters (Cs <= 512 <= LT)
  {
    const int nb = tid < Cs ? (csz[tid] + T - 1) / T : 0;
    int x = nb;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(x, o, 64);
      if (lane >= o) x += y;
    }
    if (lane == 63) wsum[wv] = x;
    __syncthreads();
    if (tid == 0) {
      int run = 0;
      for (int w = 0; w < LW; w++) {
        const int t2 = wsum[w];
        wsum[w] = run;
        run += t2;
      }
      wsum[LW] = run;
    }
    __syncthreads();
    if (tid < Cs) {
      lbo[tid] = wsum[wv] + x - nb;
      if (part == 0) bf.block_off[(int64_t)u * (g.C + 1) + cb + tid] = seg_b0 + wsum[wv] + x - nb;
    }
    if (tid == 0) lbo[Cs] = wsum[LW];
    if (tid == 0 && s == g.n_seg - 1 && part == 0)
      bf.block_off[(int64_t)u * (g.C + 1) + g.C] = ws.unit_used[u];
    __syncthreads();
  }

  uint8_t* kout = reinterpret_cast<uint8_t*>(bf.k_blocks) + (int64_t)u * g.cap * T * RB;
  uint8_t* vout = reinterpret_cast<uint8_t*>(bf.v_blocks) + (int64_t)u * g.cap * T * RB;
  int32_t* stok = bf.slot_token + (int64_t)u * g.cap * T;
  const int rsub = lane / LPR, rl = lane % LPR;

  // K/V rows into slots, padding slots zero / -1; a wave moves RU row steps
  // (RU * RPW rows) per round, all loads of a round issued before its stores
  constexpr int RU = 4;
  for (int c = part + LP * wv; c < Cs; c += LP * LW) {
    const int nc = scsz[c];
    const int nsl = (lbo[c + 1] - lbo[c]) * T;
    const int64_t slot0 = (int64_t)(seg_b0 + lbo[c]) * T;
    const int* cm = smemb + scoff[c];
    for (int j0 = 0; j0 < nsl; j0 += RU * RPW) {
      uint4 kv[RU], vv[RU];
      int tok[RU];
#pragma unroll
      for (int q = 0; q < RU; q++) {
        const int j = j0 + q * RPW + rsub;
        kv[q] = vv[q] = make_uint4(0, 0, 0, 0);
        tok[q] = -1;
        if (j < nc) {
          const int64_t pos = first + cm[j];
          tok[q] = (int)pos;
          kv[q] = reinterpret_cast<const uint4*>(Kb + pos * strow)[rl];
          vv[q] = reinterpret_cast<const uint4*>(Vb + pos * strow)[rl];
        }
      }
#pragma unroll
      for (int q = 0; q < RU; q++) {
        const int j = j0 + q * RPW + rsub;
        if (j < nsl) {
          reinterpret_cast<uint4*>(kout + (slot0 + j) * RB)[rl] = kv[q];
          reinterpret_cast<uint4*>(vout + (slot0 + j) * RB)[rl] = vv[q];
          if (rl == 0) stok[slot0 + j] = tok[q];
        }
      }
    }
  }

  // value sums: one wave per cluster, lane owns dims 2*lane, 2*lane+1; the
  // rows of VU members are requested together, then added in ascending
  // position
  constexpr int VU = 16;
  for (int c = part + LP * wv; c < Cs; c += LP * LW) {
    const int nc = scsz[c];
    const int* cm = smemb + scoff[c];
    double a0 = 0.0, a1 = 0.0;
    for (int m0 = 0; m0 < nc; m0 += VU) {
      float x0[VU], x1[VU];
#pragma unroll
      for (int r = 0; r < VU; r++) {
        x0[r] = x1[r] = 0.f;
        if (m0 + r < nc) {
          const int64_t pos = first + cm[m0 + r];
          if constexpr (DT == WI_BF16) {
            const uint32_t w = reinterpret_cast<const uint32_t*>(Vb + pos * strow)[lane];
            x0[r] = __uint_as_float(w << 16);
            x1[r] = __uint_as_float(w & 0xFFFF0000u);
          } else {
            const float2 f = reinterpret_cast<const float2*>(Vb + pos * strow)[lane];
            x0[r] = f.x;
            x1[r] = f.y;
          }
        }
      }
#pragma unroll
      for (int r = 0; r < VU; r++) {
        if (m0 + r < nc) {
          a0 += (double)x0[r];
          a1 += (double)x1[r];
        }
      }
    }
    reinterpret_cast<float2*>(bf.value_sum)[((int64_t)u * g.C + cb + c) * (D / 2) + lane] =
        make_float2((float)a0, (float)a1);
  }

  // global cluster ids of the segment's points (this workgroup's quarter)
  for (int i = n * part / LP + tid; i < n * (part + 1) / LP; i += LT)
    bf.assign[pbase + i] = cb + ws.label[pbase + i];

  // this workgroup's share of the unused tail blocks
  {
    const int64_t used = ws.unit_used[u];
    const int64_t tail = g.cap - used;
    const int64_t sh = (int64_t)s * LP + part, nsh = (int64_t)g.n_seg * LP;
    const int64_t t0 = used + tail * sh / nsh, t1 = used + tail * (sh + 1) / nsh;
    for (int64_t sl = t0 * T + wv * RPW + rsub; sl < t1 * T; sl += LW * RPW) {
      reinterpret_cast<uint4*>(kout + sl * RB)[rl] = make_uint4(0, 0, 0, 0);
      reinterpret_cast<uint4*>(vout + sl * RB)[rl] = make_uint4(0, 0, 0, 0);
      if (rl == 0) stok[sl] = -1;
    }
  }

  // steady zone copies (first segment's first workgroup)
  if (s == 0 && part == 0) {
    uint8_t* sk = reinterpret_cast<uint8_t*>(bf.steady_k) + (int64_t)u * g.n_st * RB;
    uint8_t* sv = reinterpret_cast<uint8_t*>(bf.steady_v) + (int64_t)u * g.n_st * RB;
    for (int j = wv * RPW + rsub; j < g.n_st; j += LW * RPW) {
      const int64_t pos = j < g.n_sink ? j : g.N - g.n_local + (j - g.n_sink);
      reinterpret_cast<uint4*>(sk + (int64_t)j * RB)[rl] =
          reinterpret_cast<const uint4*>(Kb + pos * strow)[rl];
      reinterpret_cast<uint4*>(sv + (int64_t)j * RB)[rl] =
          reinterpret_cast<const uint4*>(Vb + pos * strow)[rl];
    }
  }
}

}  // namespace

hipError_t launch_layout(const Geom& g, const void* K, const void* V, const wi_index_bufs& b,
                         const BuildWs& ws, hipStream_t s) {
  WI_LAUNCH(K_SEG_SCAN, seg_scan_kernel, dim3(g.U), dim3(256), 0, s, g, ws);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (g.dtype == WI_BF16)
    WI_LAUNCH(K_LAYOUT, layout_kernel<WI_BF16>, dim3(g.U * g.n_seg, LP), dim3(LT), 0, s, g, K, V,
              b, ws);
  else
    WI_LAUNCH(K_LAYOUT, layout_kernel<WI_F32>, dim3(g.U * g.n_seg, LP), dim3(LT), 0, s, g, K, V,
              b, ws);
  return hipGetLastError();
}

}  // namespace wi
