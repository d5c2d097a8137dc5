// Wave buffer: a GPU cache of 2 KB KV blocks in front of a host-memory tier
// (RetroInfer, framerc blog section 2.2: the wave buffer keeps hot blocks in
// GPU memory with a cluster -> block mapping table; the synchronous access
// path reads cached blocks from GPU memory and the others from CPU memory;
// the asynchronous update path maintains an LRU replacement and the mapping
// table off the critical path; section 3.2: 2 KB blocks, execution buffer
// assembled from cached and fetched blocks).
//
// Per unit: block_slot[blk] (-1 or the block's cache slot), slot_block[s]
// (-1 or the cached block) and slot_last[s] (the step that last used the
// slot; 0 = never). After a decode step that retrieved the clusters R:
//   - the needed blocks are every block of every cluster of R, ascending;
//   - a needed block that is cached is a hit and its slot's step becomes the
//     current one;
//   - the misses, ascending, take the least recently used slots not used in
//     this step (ordered by (last step, slot id)), as many as there are;
//     each evicts the slot's previous block from the table and is copied
//     from the host tier into its slot.
// slot_order keeps the slots sorted by (last step, slot id): after a step the
// slots it used (all with the newest step) move to the end, sorted by id, and
// the others keep their order, so no step sorts more than the slots it used.
#include "wi_internal.h"

namespace wi {
namespace {

constexpr int UT = 1024;             // update threads per unit
constexpr int UW = UT / 64;
constexpr int MAX_SLOTS = 8192;      // cache slots per unit (LDS order lists)

__global__ void wb_reset_kernel(int32_t* __restrict__ b2s, int64_t nb, int32_t* __restrict__ s2b,
                                uint32_t* __restrict__ last, int32_t* __restrict__ order,
                                int64_t ns, int S) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < nb;
       i += (int64_t)gridDim.x * blockDim.x)
    b2s[i] = -1;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < ns;
       i += (int64_t)gridDim.x * blockDim.x) {
    s2b[i] = -1;
    last[i] = 0u;
    order[i] = (int32_t)(i % S);
  }
}

// Exclusive scan of one int per thread over the workgroup; returns the
// thread's offset and writes the total to *tot.
__device__ __forceinline__ int wg_scan(int v, int* lds, int* tot) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  __syncthreads();
  if (lane == 63) lds[wv] = x;
  __syncthreads();
  int off = 0, t = 0;
#pragma unroll
  for (int w = 0; w < UW; w++) {
    const int a = lds[w];
    off += w < wv ? a : 0;
    t += a;
  }
  *tot = t;
  return off + x - v;
}

__global__ __launch_bounds__(UT) void wb_update_kernel(
    int C, int64_t nblk, int T, int S, const int32_t* __restrict__ size,
    const int32_t* __restrict__ block_off, const uint8_t* __restrict__ zone, uint32_t step,
    int32_t* __restrict__ b2s, int32_t* __restrict__ s2b, uint32_t* __restrict__ last,
    int32_t* __restrict__ order, int32_t* __restrict__ need, int32_t* __restrict__ fill,
    int32_t* __restrict__ counts, int32_t* __restrict__ stats) {
  const int u = blockIdx.x, tid = threadIdx.x;
  __shared__ int scan_lds[UW];
  __shared__ int ord[MAX_SLOTS];   // the slots by (last use, slot id) before this step
  __shared__ int vic[MAX_SLOTS];   // eviction order of the slots not hit in this step
  const int32_t* sz = size + (int64_t)u * C;
  const int32_t* bo = block_off + (int64_t)u * (C + 1);
  const uint8_t* zn = zone + (int64_t)u * C;
  int32_t* b2su = b2s + (int64_t)u * nblk;
  int32_t* s2bu = s2b + (int64_t)u * S;
  uint32_t* lastu = last + (int64_t)u * S;
  int32_t* ordu = order + (int64_t)u * S;
  int32_t* needu = need + (int64_t)u * 2 * nblk;  // [needed blocks | misses]
  int32_t* missu = needu + nblk;
  int32_t* fillu = fill + (int64_t)u * 2 * S;
  for (int i = tid; i < S; i += UT) ord[i] = ordu[i];
  // thread t owns the consecutive items [t P, t P + P) of a list of n
  auto range = [&](int64_t n, int64_t& lo, int64_t& hi) {
    const int64_t P = (n + UT - 1) / UT;
    lo = (int64_t)tid * P;
    hi = lo + P < n ? lo + P : n;
    if (lo > hi) lo = hi;
  };
  int64_t lo, hi;
  int tot;

  // (a) the blocks of the retrieved clusters, ascending
  range(C, lo, hi);
  int cnt = 0;
  for (int64_t c = lo; c < hi; c++) cnt += zn[c] == 1 ? (sz[c] + T - 1) / T : 0;
  int off = wg_scan(cnt, scan_lds, &tot);
  for (int64_t c = lo; c < hi; c++) {
    if (zn[c] != 1) continue;
    const int nb = (sz[c] + T - 1) / T;
    for (int j = 0; j < nb; j++) needu[off++] = bo[c] + j;
  }
  const int n_need = tot;
  __syncthreads();
  // (b) hits refresh their slot's step; misses are compacted, ascending
  range(n_need, lo, hi);
  int hits = 0;
  cnt = 0;
  for (int64_t i = lo; i < hi; i++) {
    int sl = b2su[needu[i]];
    if (sl >= S) sl = -1;  // (tables written only by this kernel and the reset)
    if (sl >= 0) {
      lastu[sl] = step;
      hits++;
    } else {
      cnt++;
    }
  }
  off = wg_scan(cnt, scan_lds, &tot);
  for (int64_t i = lo; i < hi; i++) {
    const int sl = b2su[needu[i]];
    if (sl < 0 || sl >= S) missu[off++] = needu[i];
  }
  const int n_miss = tot;
  wg_scan(hits, scan_lds, &tot);
  const int n_hit = tot;
  __syncthreads();
  // (c) eviction order: the slots not hit in this step, in (last use, slot
  // id) order -- the order list with the hit slots taken out
  range(S, lo, hi);
  cnt = 0;
  for (int64_t i = lo; i < hi; i++) cnt += lastu[ord[i]] != step;
  off = wg_scan(cnt, scan_lds, &tot);
  for (int64_t i = lo; i < hi; i++)
    if (lastu[ord[i]] != step) vic[off++] = ord[i];
  const int n_cand = tot;
  __syncthreads();
  // (d) admit the misses in order into the eviction order's slots
  const int n_adm = n_miss < n_cand ? n_miss : n_cand;
  for (int i = tid; i < n_adm; i += UT) {
    const int sl = vic[i];
    const int blk = missu[i];
    const int old = s2bu[sl];
    if (old >= 0 && old < nblk) b2su[old] = -1;
    b2su[blk] = sl;
    s2bu[sl] = blk;
    lastu[sl] = step;
    fillu[2 * i] = blk;
    fillu[2 * i + 1] = sl;
  }
  __syncthreads();
  // (e) the new order: the slots not used in this step keep their order,
  // then the slots used in this step (hits and admissions) by slot id
  cnt = 0;
  for (int64_t i = lo; i < hi; i++) cnt += lastu[ord[i]] != step;
  off = wg_scan(cnt, scan_lds, &tot);
  for (int64_t i = lo; i < hi; i++)
    if (lastu[ord[i]] != step) ordu[off++] = ord[i];
  const int n_keep = tot;
  cnt = 0;
  for (int64_t s2 = lo; s2 < hi; s2++) cnt += lastu[s2] == step;
  off = wg_scan(cnt, scan_lds, &tot);
  for (int64_t s2 = lo; s2 < hi; s2++)
    if (lastu[s2] == step) ordu[n_keep + off++] = (int32_t)s2;
  if (tid == 0) {
    counts[u * 4 + 0] = n_need;
    counts[u * 4 + 1] = n_hit;
    counts[u * 4 + 2] = n_adm;
    counts[u * 4 + 3] = n_miss;
    if (stats) {
      stats[u * 2 + 0] = n_hit;
      stats[u * 2 + 1] = n_miss;
    }
  }
}

// Copy every admitted block (K and V, T rows each) from the host tier into
// its cache slot: 16-byte pieces, all workgroups of the unit striding over
// the admitted list. Block b of unit u is pieces [(u nblk + b) VPB, + VPB)
// of a pool, slot s pieces [(u S + s) VPB, + VPB) of a cache.
__global__ __launch_bounds__(256) void wb_fill_kernel(const uint4* __restrict__ hk,
                                                      const uint4* __restrict__ hv,
                                                      uint4* __restrict__ ck, uint4* __restrict__ cv,
                                                      const int32_t* __restrict__ fill,
                                                      const int32_t* __restrict__ counts,
                                                      int64_t nblk, int S, int VPB) {
  const int u = blockIdx.y;
  const int n_adm = counts[u * 4 + 2];
  const int32_t* fillu = fill + (int64_t)u * 2 * S;
  const int64_t per = 2 * (int64_t)VPB;  // K then V pieces of one block
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < (int64_t)n_adm * per;
       e += (int64_t)gridDim.x * blockDim.x) {
    const int i = (int)(e / per);
    const int r = (int)(e % per);
    const int64_t blk = fillu[2 * i], sl = fillu[2 * i + 1];
    const bool isv = r >= VPB;
    const int p = isv ? r - VPB : r;
    const uint4* src = isv ? hv : hk;
    uint4* dst = isv ? cv : ck;
    dst[((int64_t)u * S + sl) * VPB + p] = src[((int64_t)u * nblk + blk) * VPB + p];
  }
}

}  // namespace

int wb_max_slots() { return MAX_SLOTS; }

hipError_t launch_wb_reset(const Geom& g, const WaveBufArgs& wb, hipStream_t s) {
  WI_LAUNCH(K_ZERO, wb_reset_kernel, dim3(256), dim3(256), 0, s, wb.block_slot,
            (int64_t)g.U * g.cap, wb.slot_block, wb.slot_last, wb.slot_order,
            (int64_t)g.U * wb.n_slots, wb.n_slots);
  return hipGetLastError();
}

hipError_t launch_wb_update(const Geom& g, const WaveBufArgs& wb, const int32_t* cluster_size,
                            const int32_t* block_off, const uint8_t* zone, uint32_t step,
                            int32_t* need, int32_t* fill, int32_t* counts, int32_t* stats,
                            hipStream_t s) {
  WI_LAUNCH(K_WB_UPDATE, wb_update_kernel, dim3(g.U), dim3(UT), 0, s, g.C, g.cap, g.T,
            wb.n_slots, cluster_size, block_off, zone, step, wb.block_slot, wb.slot_block,
            wb.slot_last, wb.slot_order, need, fill, counts, stats);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int VPB = g.T * D * (g.dtype == WI_BF16 ? 2 : 4) / 16;  // 16-byte pieces per block
  WI_LAUNCH(K_WB_FILL, wb_fill_kernel, dim3(64, g.U), dim3(256), 0, s,
            reinterpret_cast<const uint4*>(wb.host_k), reinterpret_cast<const uint4*>(wb.host_v),
            reinterpret_cast<uint4*>(wb.cache_k), reinterpret_cast<uint4*>(wb.cache_v), fill,
            counts, g.cap, wb.n_slots, VPB);
  return hipGetLastError();
}

}  // namespace wi
