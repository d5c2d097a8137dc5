// Optional decode outputs: the selected cluster ids in rank order and the
// execution-buffer token list (RetroInfer, framerc blog section 3.2: the
// execution buffer holds the steady zone followed by the retrieved blocks,
// with block fragments skipped). These are written only on request; the
// attention itself does not depend on them.
#include "wi_internal.h"

namespace wi {
namespace {

// For every selected cluster c (zone != 0):
// rank(c) = #{selected c' : key(c') > key(c), or equal keys and c' < c}.
__global__ __launch_bounds__(256) void rank_kernel(const uint32_t* __restrict__ keys,
                                                   const uint8_t* __restrict__ zones, int C,
                                                   int M, int32_t* __restrict__ ranked) {
  const int u = blockIdx.y;
  const int c = blockIdx.x * blockDim.x + threadIdx.x;
  const uint32_t* key = keys + (int64_t)u * ((C + 3) & ~3);
  const uint8_t* zone = zones + (int64_t)u * C;
  if (c >= C || zone[c] == 0) return;
  const uint32_t k = key[c];
  int rank = 0;
  for (int c2 = 0; c2 < C; c2++) {
    const uint32_t k2 = key[c2];
    rank += zone[c2] != 0 && ((k2 > k) || (k2 == k && c2 < c));
  }
  if (rank < M) ranked[(int64_t)u * M + rank] = c;
}

__global__ __launch_bounds__(256) void exec_kernel(
    const int32_t* __restrict__ ranked, const int32_t* __restrict__ sizes,
    const int32_t* __restrict__ block_off, const int32_t* __restrict__ slot_token,
    int C, int64_t capT, int T, int K_r, int M, int n_sink, int n_local, int64_t N,
    int n_pend, int32_t* __restrict__ exec, int32_t* __restrict__ n_exec, int64_t exec_cap) {
  const int u = blockIdx.x;
  const int tid = threadIdx.x;
  const int n_st = n_sink + n_local;
  const int32_t* rk = ranked + (int64_t)u * M;
  const int32_t* sz = sizes + (int64_t)u * C;
  const int32_t* bo = block_off + (int64_t)u * (C + 1);
  const int32_t* st = slot_token + (int64_t)u * capT;
  __shared__ int wsum[4];
  __shared__ int run_s;
  if (tid == 0) run_s = n_st + n_pend;
  if (exec) {
    // steady positions, then the pending ones (just before the local window)
    const int64_t p0 = N - n_local - n_pend;
    for (int j = tid; j < n_st + n_pend && j < exec_cap; j += 256)
      exec[(int64_t)u * exec_cap + j] =
          j < n_sink ? j
                     : (j < n_st ? (int32_t)(N - n_local + (j - n_sink)) : (int32_t)(p0 + j - n_st));
  }
  __syncthreads();
  for (int base = 0; base < K_r; base += 256) {
    const int r = base + tid;
    const int c0 = r < K_r ? rk[r] : -1;
    const int c = c0 >= 0 && c0 < C ? c0 : -1;
    const int n = c >= 0 ? sz[c] : 0;
    // block exclusive scan of n
    int x = n;
    const int lane = tid & 63, wv = tid >> 6;
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(x, o, 64);
      if (lane >= o) x += y;
    }
    if (lane == 63) wsum[wv] = x;
    __syncthreads();
    int off = run_s;
    for (int w = 0; w < wv; w++) off += wsum[w];
    off += x - n;
    const int tot = wsum[0] + wsum[1] + wsum[2] + wsum[3];
    if (exec && c >= 0) {
      for (int j = 0; j < n; j++)
        if (off + j < exec_cap) exec[(int64_t)u * exec_cap + off + j] = st[(int64_t)bo[c] * T + j];
    }
    __syncthreads();
    if (tid == 0) run_s += tot;
    __syncthreads();
  }
  if (tid == 0 && n_exec) n_exec[u] = run_s;
}

}  // namespace

hipError_t launch_debug_outputs(const DecodeArgs& a, const wi_index_bufs& b,
                                const DecodeWs& ws, int32_t* sel_ids,
                                int32_t* exec_tokens, int32_t* n_exec,
                                int64_t exec_cap, hipStream_t s) {
  const Geom& g = *a.g;
  const int M = a.K_r + a.K_e;
  int32_t* ranked = sel_ids ? sel_ids : ws.rank;
  if (M > 0) {
    dim3 grid((g.C + 255) / 256, g.U);
    WI_LAUNCH(K_RANK, rank_kernel, grid, dim3(256), 0, s, ws.key, ws.zone, g.C, M, ranked);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (exec_tokens || n_exec) {
    WI_LAUNCH(K_EXEC, exec_kernel, dim3(g.U), dim3(256), 0, s, ranked, b.cluster_size,
                       b.block_off, b.slot_token, g.C, g.cap * g.T, g.T, a.K_r, M,
                       g.n_sink, g.n_local, g.N, g.n_pend, exec_tokens, n_exec, exec_cap);
  }
  return hipGetLastError();
}

}  // namespace wi
