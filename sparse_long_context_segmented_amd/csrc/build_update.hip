// Index build, Lloyd update step and membership lists (RetroInfer, framerc
// blog section 2.1 segmented_kmeans sketch; gist.science summary,
// "Technische Samenvatting" 2A: centroids are cluster averages).
//
// Two workgroups (16 waves each) per segment; both sort, each computes the
// means of half the clusters (c % 2), and the first writes the lists:
//   1. stable counting sort of the segment's points by cluster: per-wave
//      histograms in LDS, a scan over (cluster, wave), then each wave places
//      its points in position order; equal labels inside a 64-point round are
//      ranked with ballots over the label bits. Members of a cluster end up
//      in ascending position, which fixes the summation order below;
//   2. cluster sizes and per-segment block counts (ceil(n_c / T));
//   3. (update) mean of each non-empty cluster: float64 sum over members in
//      ascending position, divided by n_c in float64, rounded to float32 and
//      then to the storage dtype (bf16: nearest, ties to even). An empty
//      cluster keeps its centroid.
#include "wi_internal.h"

namespace wi {
namespace {

constexpr int UT = 1024;
constexpr int UW = UT / 64;
constexpr int UP = 2;  // workgroups per segment: both sort, cluster c's mean goes to c % UP

template <int DT>
__device__ __forceinline__ const uint8_t* kp(const void* K, const Geom& g, int u, int64_t pos) {
  const int b = u / g.H, h = u % g.H;
  const int64_t off = (int64_t)b * g.sb + (int64_t)h * g.sh + pos * g.st;
  return reinterpret_cast<const uint8_t*>(K) + off * (DT == WI_BF16 ? 2 : 4);
}

template <int DT>
__global__ __launch_bounds__(UT) void sort_update_kernel(Geom g, const void* __restrict__ K,
                                                         void* __restrict__ cent,
                                                         int32_t* __restrict__ csize,
                                                         BuildWs ws, int do_update) {
  __shared__ int hist[UW][MAX_K];
  __shared__ int memb[MAX_SEG];
  __shared__ int coff[MAX_K + 1];
  __shared__ int wsum[UW + 1];
  const int gs = blockIdx.x, u = gs / g.n_seg, s = gs % g.n_seg, part = blockIdx.y;
  const int n = seg_n(g, s), Cs = seg_c(g, s), cb = seg_cbase(g, s);
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int64_t pbase = (int64_t)u * g.n_idx + (int64_t)s * g.seg_len;
  const int* lab = ws.label + pbase;
  if (part != 0 && !do_update) return;  // only the lists are wanted

  for (int i = tid; i < UW * MAX_K; i += UT) (&hist[0][0])[i] = 0;
  __syncthreads();
  // wave chunk: contiguous positions [ca, cz)
  const int cw = ((n + UW - 1) / UW + 63) & ~63;
  const int ca = min(n, wv * cw), cz = min(n, ca + cw);
  for (int i = ca + lane; i < cz; i += 64) atomicAdd(&hist[wv][lab[i]], 1);
  __syncthreads();

  // totals and exclusive offsets over clusters
  int tot = 0;
  if (tid < Cs)
    for (int w = 0; w < UW; w++) tot += hist[w][tid];
  {
    int x = tot;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(x, o, 64);
      if (lane >= o) x += y;
    }
    if (lane == 63) wsum[wv] = x;
    __syncthreads();
    if (tid == 0) {
      int run = 0;
      for (int w = 0; w < UW; w++) {
        const int t2 = wsum[w];
        wsum[w] = run;
        run += t2;
      }
      wsum[UW] = run;
    }
    __syncthreads();
    const int excl = wsum[wv] + x - tot;
    if (tid < Cs) {
      coff[tid] = excl;
      int base = excl;
      for (int w = 0; w < UW; w++) {
        const int t2 = hist[w][tid];
        hist[w][tid] = base;
        base += t2;
      }
      if (part == 0) {
        csize[(int64_t)u * g.C + cb + tid] = tot;
        ws.cl_off[(int64_t)u * g.C + cb + tid] = excl;
      }
    }
  }
  __syncthreads();
  // blocks used by the segment
  {
    int nb = tid < Cs ? (tot + g.T - 1) / g.T : 0;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) nb += __shfl_xor(nb, o, 64);
    if (lane == 0) wsum[wv] = nb;
    __syncthreads();
    if (tid == 0 && part == 0) {
      int sb = 0;
      for (int w = 0; w < UW; w++) sb += wsum[w];
      ws.seg_blocks[gs] = sb;
    }
  }

  // stable placement in position order
  int nbits = 0;
  while ((1 << nbits) < Cs) nbits++;
  for (int i0 = ca; i0 < cz; i0 += 64) {
    const int i = i0 + lane;
    const bool act = i < cz;
    const int L = act ? lab[i] : 0;
    unsigned long long peers = __ballot(act);
    for (int bt = 0; bt < nbits; bt++) {
      const bool bit = (L >> bt) & 1;
      const unsigned long long m = __ballot(act && bit);
      peers &= bit ? m : ~m;
    }
    const unsigned long long lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    const int rank = __popcll(peers & lt);
    int pos = 0;
    if (act) {
      pos = hist[wv][L] + rank;
      memb[pos] = i;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    if (act && rank == 0) hist[wv][L] += __popcll(peers);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
  }
  __syncthreads();
  if (part == 0)
    for (int i = tid; i < n; i += UT) ws.members[pbase + i] = memb[i];
  if (tid <= Cs) {
    if (tid == Cs) coff[Cs] = n;
  }
  __syncthreads();

  if (!do_update) return;
  // means: one wave per cluster, lane owns dims 2*lane, 2*lane+1
  const int64_t first = seg_first(g, s);
  for (int c = part + UP * wv; c < Cs; c += UP * UW) {
    const int m0 = coff[c], m1 = coff[c + 1];
    const int nc = m1 - m0;
    if (nc == 0) continue;
    double a0 = 0.0, a1 = 0.0;
    int m = m0;
    // the rows of 16 members are requested together, then added in order
    for (; m + 16 <= m1; m += 16) {
      float x0[16], x1[16];
#pragma unroll
      for (int r = 0; r < 16; r++) {
        const uint8_t* row = kp<DT>(K, g, u, first + memb[m + r]);
        if constexpr (DT == WI_BF16) {
          const uint32_t w = reinterpret_cast<const uint32_t*>(row)[lane];
          x0[r] = __uint_as_float(w << 16);
          x1[r] = __uint_as_float(w & 0xFFFF0000u);
        } else {
          const float2 f = reinterpret_cast<const float2*>(row)[lane];
          x0[r] = f.x;
          x1[r] = f.y;
        }
      }
#pragma unroll
      for (int r = 0; r < 16; r++) {
        a0 += (double)x0[r];
        a1 += (double)x1[r];
      }
    }
    for (; m + 4 <= m1; m += 4) {
      float x0[4], x1[4];
#pragma unroll
      for (int r = 0; r < 4; r++) {
        const uint8_t* row = kp<DT>(K, g, u, first + memb[m + r]);
        if constexpr (DT == WI_BF16) {
          const uint32_t w = reinterpret_cast<const uint32_t*>(row)[lane];
          x0[r] = __uint_as_float(w << 16);
          x1[r] = __uint_as_float(w & 0xFFFF0000u);
        } else {
          const float2 f = reinterpret_cast<const float2*>(row)[lane];
          x0[r] = f.x;
          x1[r] = f.y;
        }
      }
#pragma unroll
      for (int r = 0; r < 4; r++) {
        a0 += (double)x0[r];
        a1 += (double)x1[r];
      }
    }
    for (; m < m1; m++) {
      const uint8_t* row = kp<DT>(K, g, u, first + memb[m]);
      if constexpr (DT == WI_BF16) {
        const uint32_t w = reinterpret_cast<const uint32_t*>(row)[lane];
        a0 += (double)__uint_as_float(w << 16);
        a1 += (double)__uint_as_float(w & 0xFFFF0000u);
      } else {
        const float2 f = reinterpret_cast<const float2*>(row)[lane];
        a0 += (double)f.x;
        a1 += (double)f.y;
      }
    }
    const float m0f = (float)(a0 / (double)nc);
    const float m1f = (float)(a1 / (double)nc);
    const int64_t crow = (int64_t)u * g.C + cb + c;
    if constexpr (DT == WI_BF16) {
      const uint32_t packed = (uint32_t)f32_to_bf16_rne(m0f) | ((uint32_t)f32_to_bf16_rne(m1f) << 16);
      reinterpret_cast<uint32_t*>(cent)[crow * (D / 2) + lane] = packed;
    } else {
      reinterpret_cast<float2*>(cent)[crow * (D / 2) + lane] = make_float2(m0f, m1f);
    }
  }
}

}  // namespace

hipError_t launch_sort_update(const Geom& g, const void* K, void* cent, int32_t* csize,
                              const BuildWs& ws, bool do_update, hipStream_t s) {
  if (g.dtype == WI_BF16)
    WI_LAUNCH(K_SORT_UPDATE, sort_update_kernel<WI_BF16>, dim3(g.U * g.n_seg, UP), dim3(UT), 0,
              s, g, K, cent, csize, ws, (int)do_update);
  else
    WI_LAUNCH(K_SORT_UPDATE, sort_update_kernel<WI_F32>, dim3(g.U * g.n_seg, UP), dim3(UT), 0, s,
              g, K, cent, csize, ws, (int)do_update);
  return hipGetLastError();
}

}  // namespace wi
