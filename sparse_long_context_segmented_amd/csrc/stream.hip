// Decode-time growth of the index (RetroInfer, framerc blog section 1.1:
// generating a token reads the cached history and then appends the token's
// KV, the cache being kept like a ring buffer; section 2.1: steady zone of
// the first n_sink and last n_local tokens, k-means per seg_len-token
// segment, segments clustered independently).
//
//  - append: per unit, the token leaving the local window (steady row
//    n_sink) is copied to pending row n_pend, the local rows move up by one
//    and the new token becomes the last steady row (with no local window the
//    new token goes straight to the pending rows).
//  - extend (merge step): once a segment's worth of tokens is pending, it has
//    been clustered as a one-segment index by the build kernels (the caller
//    of launch_extend_merge does that); the grown index is the old one's
//    clusters, blocks, steady rows and assignments followed by the new
//    segment's, with the new clusters' block offsets moved past the old used
//    blocks, their slot tokens moved to the pending positions and their
//    assignments moved past the old clusters.
#include "wi_internal.h"

namespace wi {
namespace {

constexpr int AT = 256;  // append threads per unit

// One unit per workgroup. Rows are moved as 16-byte vectors; every move reads
// its rows before any thread writes (barriers in between), so overlapping
// moves are safe.
__global__ __launch_bounds__(AT) void append_kernel(uint4* __restrict__ sk, uint4* __restrict__ sv,
                                                    uint4* __restrict__ pk, uint4* __restrict__ pv,
                                                    const uint4* __restrict__ kn,
                                                    const uint4* __restrict__ vn, int n_sink,
                                                    int n_local, int n_pend, int seg_len, int RV) {
  const int u = blockIdx.x, tid = threadIdx.x;
  const int n_st = n_sink + n_local;
  uint4* sku = sk + (int64_t)u * n_st * RV;
  uint4* svu = sv + (int64_t)u * n_st * RV;
  uint4* pku = pk + ((int64_t)u * seg_len + n_pend) * RV;
  uint4* pvu = pv + ((int64_t)u * seg_len + n_pend) * RV;
  const uint4* knu = kn + (int64_t)u * RV;
  const uint4* vnu = vn + (int64_t)u * RV;
  if (n_local == 0) {
    for (int i = tid; i < RV; i += AT) {
      pku[i] = knu[i];
      pvu[i] = vnu[i];
    }
    return;
  }
  // the oldest local row leaves the window
  for (int i = tid; i < RV; i += AT) {
    pku[i] = sku[(int64_t)n_sink * RV + i];
    pvu[i] = svu[(int64_t)n_sink * RV + i];
  }
  __syncthreads();
  // rows n_sink + 1 .. n_st - 1 move up by one, AT vectors at a time
  const int64_t first = (int64_t)(n_sink + 1) * RV, end = (int64_t)n_st * RV;
  for (int64_t c = first; c < end; c += AT) {
    const int64_t i = c + tid;
    uint4 k4 = make_uint4(0u, 0u, 0u, 0u), v4 = make_uint4(0u, 0u, 0u, 0u);
    if (i < end) {
      k4 = sku[i];
      v4 = svu[i];
    }
    __syncthreads();
    if (i < end) {
      sku[i - RV] = k4;
      svu[i - RV] = v4;
    }
    __syncthreads();
  }
  for (int i = tid; i < RV; i += AT) {
    sku[(int64_t)(n_st - 1) * RV + i] = knu[i];
    svu[(int64_t)(n_st - 1) * RV + i] = vnu[i];
  }
}

// Many tokens at once (a prefill chunk, or several decode steps): with the
// local window's rows L[0..n_local) followed by the n_new new rows X, the
// first n_new rows of (L, X) become pending rows n_pend .. and the last
// n_local rows of (L, X) the new local window, staged in `stage` first (the
// window's old rows are still being read).
__global__ __launch_bounds__(256) void append_many_kernel(
    const uint4* __restrict__ sk, const uint4* __restrict__ sv, uint4* __restrict__ pk,
    uint4* __restrict__ pv, const uint4* __restrict__ kn, const uint4* __restrict__ vn,
    uint4* __restrict__ stk, uint4* __restrict__ stv, int n_sink, int n_local, int n_pend,
    int seg_len, int n_new, int RV) {
  const int u = blockIdx.y;
  const int n_st = n_sink + n_local;
  const uint4* sku = sk + ((int64_t)u * n_st + n_sink) * RV;  // local rows
  const uint4* svu = sv + ((int64_t)u * n_st + n_sink) * RV;
  const uint4* knu = kn + (int64_t)u * n_new * RV;
  const uint4* vnu = vn + (int64_t)u * n_new * RV;
  const int64_t total = (int64_t)(n_new + n_local) * RV;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total;
       e += (int64_t)gridDim.x * blockDim.x) {
    const int x = (int)(e / RV), p = (int)(e % RV);  // row x of (L, X)
    const uint4 k4 = x < n_local ? sku[(int64_t)x * RV + p] : knu[(int64_t)(x - n_local) * RV + p];
    const uint4 v4 = x < n_local ? svu[(int64_t)x * RV + p] : vnu[(int64_t)(x - n_local) * RV + p];
    if (x < n_new) {
      const int64_t d = ((int64_t)u * seg_len + n_pend + x) * RV + p;
      pk[d] = k4;
      pv[d] = v4;
    } else {
      const int64_t d = ((int64_t)u * n_local + (x - n_new)) * RV + p;
      stk[d] = k4;
      stv[d] = v4;
    }
  }
}

__global__ __launch_bounds__(256) void local_from_stage_kernel(uint4* __restrict__ sk,
                                                               uint4* __restrict__ sv,
                                                               const uint4* __restrict__ stk,
                                                               const uint4* __restrict__ stv,
                                                               int n_sink, int n_local, int RV) {
  const int u = blockIdx.y;
  const int n_st = n_sink + n_local;
  const int64_t total = (int64_t)n_local * RV;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total;
       e += (int64_t)gridDim.x * blockDim.x) {
    const int64_t d = ((int64_t)u * n_st + n_sink) * RV + e;
    sk[d] = stk[(int64_t)u * n_local * RV + e];
    sv[d] = stv[(int64_t)u * n_local * RV + e];
  }
}

// A per-unit count: p ? p[u * stride + idx] * mul : c.
struct Cnt {
  const int32_t* p;
  int64_t stride;
  int64_t idx;
  int mul;
  int c;
  __device__ __forceinline__ int64_t get(int u) const {
    return p ? (int64_t)p[u * stride + idx] * mul : (int64_t)c;
  }
};
Cnt cnt_const(int c) { return Cnt{nullptr, 0, 0, 1, c}; }
Cnt cnt_dev(const int32_t* p, int64_t stride, int64_t idx, int mul) {
  return Cnt{p, stride, idx, mul, 0};
}

// dst[u][r], r < n_rows (rows of RV 16-byte vectors): a[u][r] for r < na(u),
// then b[u][r - na(u)] for the next nb(u) rows, then zero.
__global__ __launch_bounds__(256) void merge_rows_kernel(uint4* __restrict__ dst, int64_t dst_rows,
                                                         const uint4* __restrict__ a, int64_t a_rows,
                                                         Cnt na, const uint4* __restrict__ b,
                                                         int64_t b_rows, Cnt nb, int RV) {
  const int u = blockIdx.y;
  const int64_t n_a = na.get(u) * RV, n_b = nb.get(u) * RV, n = dst_rows * RV;
  uint4* d = dst + (int64_t)u * dst_rows * RV;
  const uint4* au = a + (int64_t)u * a_rows * RV;
  const uint4* bu = b + (int64_t)u * b_rows * RV;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x) {
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (i < n_a) v = au[i];
    else if (i - n_a < n_b) v = bu[i - n_a];
    d[i] = v;
  }
}

// Same for int32 elements; the b part is offset by add(u) (values < 0 are
// kept when keep_neg), the rest is fill.
__global__ __launch_bounds__(256) void merge_i32_kernel(int32_t* __restrict__ dst, int64_t dst_n,
                                                        const int32_t* __restrict__ a, int64_t a_n,
                                                        Cnt na, const int32_t* __restrict__ b,
                                                        int64_t b_n, Cnt nb, Cnt add,
                                                        bool keep_neg, int32_t fill) {
  const int u = blockIdx.y;
  const int64_t n_a = na.get(u), n_b = nb.get(u);
  const int32_t off = (int32_t)add.get(u);
  int32_t* d = dst + (int64_t)u * dst_n;
  const int32_t* au = a + (int64_t)u * a_n;
  const int32_t* bu = b + (int64_t)u * b_n;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < dst_n;
       i += (int64_t)gridDim.x * blockDim.x) {
    int32_t v = fill;
    if (i < n_a) {
      v = au[i];
    } else if (i - n_a < n_b) {
      const int32_t x = bu[i - n_a];
      v = (keep_neg && x < 0) ? x : x + off;
    }
    d[i] = v;
  }
}

dim3 merge_grid(int64_t elems, int U) {
  int64_t blocks = (elems + 255) / 256;
  if (blocks > 512) blocks = 512;
  if (blocks < 1) blocks = 1;
  return dim3((unsigned)blocks, (unsigned)U);
}

}  // namespace

hipError_t launch_append(const Geom& g, const wi_index_bufs& b, const void* k_new,
                         const void* v_new, hipStream_t s) {
  const int RV = D * (g.dtype == WI_BF16 ? 2 : 4) / 16;
  WI_LAUNCH(K_APPEND, append_kernel, dim3(g.U), dim3(AT), 0, s,
            reinterpret_cast<uint4*>(b.steady_k), reinterpret_cast<uint4*>(b.steady_v),
            reinterpret_cast<uint4*>(b.pend_k), reinterpret_cast<uint4*>(b.pend_v),
            reinterpret_cast<const uint4*>(k_new), reinterpret_cast<const uint4*>(v_new),
            g.n_sink, g.n_local, g.n_pend, g.seg_len, RV);
  return hipGetLastError();
}

hipError_t launch_append_many(const Geom& g, const wi_index_bufs& b, const void* k_new,
                              const void* v_new, int n_new, void* stage, hipStream_t s) {
  const int RV = D * (g.dtype == WI_BF16 ? 2 : 4) / 16;
  const int64_t total = (int64_t)(n_new + g.n_local) * RV;
  int gx = (int)((total + 255) / 256);
  if (gx > 256) gx = 256;
  const int64_t stage_half = (int64_t)g.U * g.n_local * RV;
  uint4* stk = reinterpret_cast<uint4*>(stage);
  uint4* stv = stk + stage_half;
  WI_LAUNCH(K_APPEND, append_many_kernel, dim3(gx, g.U), dim3(256), 0, s,
            reinterpret_cast<const uint4*>(b.steady_k), reinterpret_cast<const uint4*>(b.steady_v),
            reinterpret_cast<uint4*>(b.pend_k), reinterpret_cast<uint4*>(b.pend_v),
            reinterpret_cast<const uint4*>(k_new), reinterpret_cast<const uint4*>(v_new), stk, stv,
            g.n_sink, g.n_local, g.n_pend, g.seg_len, n_new, RV);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || g.n_local == 0) return e;
  int gl = (int)(((int64_t)g.n_local * RV + 255) / 256);
  if (gl > 64) gl = 64;
  WI_LAUNCH(K_APPEND, local_from_stage_kernel, dim3(gl, g.U), dim3(256), 0, s,
            reinterpret_cast<uint4*>(b.steady_k), reinterpret_cast<uint4*>(b.steady_v), stk, stv,
            g.n_sink, g.n_local, RV);
  return hipGetLastError();
}

hipError_t launch_extend_merge(const Geom& go, const Geom& gn, const Geom& gs,
                               const wi_index_bufs& o, const wi_index_bufs& sg,
                               const wi_index_bufs& nw, hipStream_t s) {
  const int U = go.U, T = go.T;
  const int RVc = D * (go.dtype == WI_BF16 ? 2 : 4) / 16;  // vectors per K/V/centroid row
  const int RVs = D * 4 / 16;                              // vectors per value-sum row
  const int Co = go.C, Cs = gs.C, Cn = gn.C;
  const int64_t capTo = go.cap * T, capTs = gs.cap * T, capTn = gn.cap * T;
  const int p0 = (int)(go.n_sink + go.n_idx);  // first pending position
  // used blocks of the old index and of the new segment, per unit
  const Cnt used_o_rows = cnt_dev(o.block_off, Co + 1, Co, T);
  const Cnt used_s_rows = cnt_dev(sg.block_off, Cs + 1, Cs, T);
  const Cnt used_o = cnt_dev(o.block_off, Co + 1, Co, 1);
  const Cnt zero = cnt_const(0);
  auto rows = [&](KernelId id, void* dst, int64_t dn, const void* a, int64_t an, Cnt na,
                  const void* b, int64_t bn, Cnt nb, int RV) {
    WI_LAUNCH(id, merge_rows_kernel, merge_grid(dn * RV, U), dim3(256), 0, s,
              reinterpret_cast<uint4*>(dst), dn, reinterpret_cast<const uint4*>(a), an, na,
              reinterpret_cast<const uint4*>(b), bn, nb, RV);
  };
  auto ints = [&](int32_t* dst, int64_t dn, const int32_t* a, int64_t an, Cnt na,
                  const int32_t* b, int64_t bn, Cnt nb, Cnt add, bool keep_neg, int32_t fill) {
    WI_LAUNCH(K_MERGE, merge_i32_kernel, merge_grid(dn, U), dim3(256), 0, s, dst, dn, a, an, na,
              b, bn, nb, add, keep_neg, fill);
  };
  rows(K_MERGE, nw.centroids, Cn, o.centroids, Co, cnt_const(Co), sg.centroids, Cs,
       cnt_const(Cs), RVc);
  rows(K_MERGE, nw.value_sum, Cn, o.value_sum, Co, cnt_const(Co), sg.value_sum, Cs,
       cnt_const(Cs), RVs);
  ints(nw.cluster_size, Cn, o.cluster_size, Co, cnt_const(Co), sg.cluster_size, Cs,
       cnt_const(Cs), zero, false, 0);
  // block offsets: the old ones, then the segment's moved past the old used blocks
  ints(nw.block_off, Cn + 1, o.block_off, Co + 1, cnt_const(Co), sg.block_off, Cs + 1,
       cnt_const(Cs + 1), used_o, false, 0);
  rows(K_MERGE, nw.k_blocks, capTn, o.k_blocks, capTo, used_o_rows, sg.k_blocks, capTs,
       used_s_rows, RVc);
  rows(K_MERGE, nw.v_blocks, capTn, o.v_blocks, capTo, used_o_rows, sg.v_blocks, capTs,
       used_s_rows, RVc);
  ints(nw.slot_token, capTn, o.slot_token, capTo, used_o_rows, sg.slot_token, capTs,
       used_s_rows, cnt_const(p0), true, -1);
  if (go.n_st > 0) {
    rows(K_MERGE, nw.steady_k, go.n_st, o.steady_k, go.n_st, cnt_const(go.n_st), o.steady_k,
         go.n_st, zero, RVc);
    rows(K_MERGE, nw.steady_v, go.n_st, o.steady_v, go.n_st, cnt_const(go.n_st), o.steady_v,
         go.n_st, zero, RVc);
  }
  ints(nw.assign, gn.n_idx, o.assign, go.n_idx, cnt_const((int)go.n_idx), sg.assign, gs.n_idx,
       cnt_const((int)gs.n_idx), cnt_const(Co), false, -1);
  return hipGetLastError();
}

}  // namespace wi
