// Index build, Lloyd assignment step: every point of a segment goes to its
// nearest centroid (RetroInfer, framerc blog section 2.1: k-means over each
// 8K-token segment).
//
// The decision is defined exactly: nearest by the float64 squared distance
// sum_t (x_t - mu_t)^2 accumulated with one fused multiply-add per dimension
// in dimension order, lowest centroid id on ties. It is computed in two
// stages:
//
// 1. MFMA stage (dense contraction). bf16: a workgroup of 512 points stages
//    all (<= 512) centroids of its segment in LDS once; each wave holds 64
//    points as the B operand (columns) and sweeps 32-centroid row tiles with
//    v_mfma_f32_32x32x16_bf16 (products exact, fp32 accumulation). One extra
//    k-step of 16 folds two constants into the contraction, each split
//    exactly into three bf16 parts: -|mu_c|^2 / 2 (A side, times 1 on B) and
//    off_p / 2 (B side, times 1 on A), off_p = (|x_p|^2 + 2 max_c |mu_c|^2)
//    (1 + 2^-10) + 1. The accumulator is then a_pc = (s_pc + off_p) / 2 with
//    s_pc = 2<x, mu_c> - |mu_c|^2 (argmax s = argmin distance), and a_pc > 0.
//    Its low 9 mantissa bits are replaced by 511 - c, so an unsigned max
//    keeps the best (lowest c on equal high bits) and an unsigned median
//    the second best: three integer ops per score.
//    fp32 (parity-size workloads) keeps a plain epilogue over
//    v_mfma_f32_32x32x2_f32 with the centroids staged 128 at a time.
// 2. Certification. An encoded value lies within (a - e - 2^-14 off, a + e]
//    of its exact a, with e <= gamma_144 * 1.25 off < 2^-16.3 off (fp32
//    accumulation of <= 144 terms whose magnitudes sum to <= 1.25 off) and
//    2^-14 off for the dropped bits. If another centroid held the top
//    encoded value, the lead over the second would be at most
//    2e + 2^-14 off < 2^-13 off; so a point whose best encoded value leads
//    the second by more than 2^-13 off has its exact nearest centroid at the
//    encoded winner (fp32: the previous bound, lead over 2^-12
//    (|x|^2 + 2 max|mu|^2) on s). Other points are listed and the fallback
//    kernel evaluates the exact float64 distance to every centroid of their
//    segment.
#include "wi_internal.h"

namespace wi {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int AT = 256;           // threads per workgroup (4 waves)
constexpr int CHUNK = 256;        // centroids staged in LDS per pass
constexpr int ROWB = D * 2 + 16;  // bf16 LDS row bytes (padded)
constexpr int ROWF = D * 4 + 16;  // fp32 LDS row bytes (padded)

template <int DT>
__device__ __forceinline__ const uint8_t* kptr(const void* K, const Geom& g, int u, int64_t pos) {
  const int b = u / g.H, h = u % g.H;
  const int64_t off = (int64_t)b * g.sb + (int64_t)h * g.sh + pos * g.st;
  return reinterpret_cast<const uint8_t*>(K) + off * (DT == WI_BF16 ? 2 : 4);
}

struct Best {
  float s1, s2;
  int i1;
};

__device__ __forceinline__ void upd(Best& b, float s, int i) {
  // s2 = median(s1, s2, s) keeps the second-largest of {s1, s2, s}
  b.s2 = __builtin_amdgcn_fmed3f(b.s1, b.s2, s);
  if (s > b.s1) {
    b.s1 = s;
    b.i1 = i;
  }
}

__device__ __forceinline__ Best merge(Best a, Best o) {
  Best r;
  if (o.s1 > a.s1 || (o.s1 == a.s1 && o.i1 < a.i1)) {
    r.s1 = o.s1;
    r.i1 = o.i1;
  } else {
    r.s1 = a.s1;
    r.i1 = a.i1;
  }
  r.s2 = fmaxf(fminf(a.s1, o.s1), fmaxf(a.s2, o.s2));
  return r;
}

// ---------------------------------------------------------------------------
// bf16: 8 waves x 64 points (2 column tiles of 32) per workgroup.
constexpr int BT = 512;                  // threads per workgroup
constexpr int ROWA = D * 2 + 16;         // LDS centroid row (bf16, padded)
constexpr size_t BF16_LDS = (size_t)MAX_K * ROWA + MAX_K * 16 + 64;
constexpr uint32_t BF1 = 0x3F80u;        // bf16 1.0

// x = h1 + h2 + h3 exactly up to rounding of the last part (bf16 bits)
__device__ __forceinline__ void split3(float x, uint32_t& h1, uint32_t& h2, uint32_t& h3) {
  const float a = __uint_as_float(__float_as_uint(x) & 0xFFFF0000u);
  const float r = x - a;
  const float b = __uint_as_float(__float_as_uint(r) & 0xFFFF0000u);
  const float c = r - b;
  h1 = __float_as_uint(a) >> 16;
  h2 = __float_as_uint(b) >> 16;
  h3 = f32_to_bf16_rne(c);
}

// Workgroup (blockIdx.x, segment) handles the segment's 512-point blocks
// blockIdx.x, blockIdx.x + gridDim.x, ...: the centroids are staged once.
// Its waves take 64-point units of those blocks from a counter in LDS
// (unit j = block j / 8, 64-point column j % 8), so a wave that the issue
// order favours does more units and all waves end together; the next unit's
// points are requested while the current unit's labels are written.
__global__ __launch_bounds__(BT, 1) void assign_bf16_kernel(Geom g, const void* __restrict__ K,
                                                            const void* __restrict__ cent,
                                                            BuildWs ws) {
  constexpr int NTL = 2;
  extern __shared__ __align__(16) uint8_t lds[];
  uint8_t* crow = lds;                                                  // MAX_K rows
  uint4* ctail = reinterpret_cast<uint4*>(lds + (size_t)MAX_K * ROWA);  // A tail, k 0..7
  float* red = reinterpret_cast<float*>(ctail + MAX_K);                 // 8 floats

  const int gs = blockIdx.y, u = gs / g.n_seg, s = gs % g.n_seg;
  const int n = seg_n(g, s), Cs = seg_c(g, s), cb = seg_cbase(g, s);
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  if (blockIdx.x * BT >= n) return;
  const int64_t first = seg_first(g, s);
  // rows staged: a multiple of 64 (pairs of 32-row tiles); rows past Cs are
  // zero, tail included, so their scores are 0 and never win
  const int Cp = (Cs + 63) & ~63;

  // B fragments of a block: point p = p0 + 64 wv + 32 t + (lane & 31), dims
  // 16 k + 8 (lane >> 5) .. + 8, for k = 0..7
  auto load_points = [&](int pb, uint4 (*bf)[8]) {
#pragma unroll
    for (int t = 0; t < NTL; t++) {
      const int p = min(pb + 32 * t + (lane & 31), n - 1);  // clamped; not written
      const uint4* row = reinterpret_cast<const uint4*>(kptr<WI_BF16>(K, g, u, first + p));
#pragma unroll
      for (int k = 0; k < 8; k++) bf[t][k] = row[2 * k + (lane >> 5)];
    }
  };
  // the first block's points are requested before the centroids
  uint4 bfrag[NTL][8];
  __shared__ int next_unit;
  auto unit_base = [&](int j) { return ((int)blockIdx.x + (j >> 3) * (int)gridDim.x) * BT + 64 * (j & 7); };
  int pb = unit_base(wv);  // units 0..7 go to waves 0..7
  load_points(pb, bfrag);
  // stage the segment's centroids: 16 lanes per row, 16 bytes each, 32 rows
  // per pass; |mu|^2 per row in float32 (fixed order), A tails from it
  const uint16_t* C16 = reinterpret_cast<const uint16_t*>(cent) + ((int64_t)u * g.C + cb) * D;
  float mmax = 0.f;
  {
    constexpr int PASSES = MAX_K / (BT / 16);  // 16
    uint4 cv[PASSES];
    const int j = tid & 15;
#pragma unroll
    for (int ps = 0; ps < PASSES; ps++) {
      const int c = ps * (BT / 16) + (tid >> 4);
      cv[ps] = c < Cs ? reinterpret_cast<const uint4*>(C16 + (int64_t)c * D)[j]
                      : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int ps = 0; ps < PASSES; ps++) {
      const int c = ps * (BT / 16) + (tid >> 4);
      if (c < Cp) {
        *reinterpret_cast<uint4*>(crow + c * ROWA + 16 * j) = cv[ps];
        const uint32_t w[4] = {cv[ps].x, cv[ps].y, cv[ps].z, cv[ps].w};
        float sq = 0.f;
#pragma unroll
        for (int e = 0; e < 4; e++) {
          const float a = __uint_as_float(w[e] << 16), b2 = __uint_as_float(w[e] & 0xFFFF0000u);
          sq = fmaf(a, a, sq);
          sq = fmaf(b2, b2, sq);
        }
        sq = row16_sum(sq);  // the row's 16 lanes hold its 16 pieces
        if (c < Cs) mmax = fmaxf(mmax, sq);
        if (j == 0) {
          uint32_t h1, h2, h3;
          split3(0.5f * sq, h1, h2, h3);
          // [-h1, -h2, -h3, 1, 1, 1, 0, 0] (k = 0..7); rows past Cs all zero
          ctail[c] = c < Cs ? make_uint4((h1 ^ 0x8000u) | ((h2 ^ 0x8000u) << 16),
                                         (h3 ^ 0x8000u) | (BF1 << 16), BF1 | (BF1 << 16), 0u)
                            : make_uint4(0u, 0u, 0u, 0u);
        }
      }
    }
  }
  if (tid == 0) next_unit = BT / 64;
  mmax = wave_max(mmax);
  if (lane == 0) red[wv] = mmax;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < BT / 64; i++) mmax = fmaxf(mmax, red[i]);
  const int nm = Cp / 32;

#pragma unroll 1
  while (pb < n) {

    // per point: |x|^2, the offset and the B tail [1, 1, 1, o1, o2, o3, 0, 0]
    // (lanes 0-31 supply k = 0..7 of the extra step; lanes 32-63 zeros)
    uint4 btail[NTL];
    float offs[NTL];
#pragma unroll
    for (int t = 0; t < NTL; t++) {
      float sq = 0.f;
#pragma unroll
      for (int k = 0; k < 8; k++) {
        const uint32_t w[4] = {bfrag[t][k].x, bfrag[t][k].y, bfrag[t][k].z, bfrag[t][k].w};
#pragma unroll
        for (int e = 0; e < 4; e++) {
          const float a = __uint_as_float(w[e] << 16), b2 = __uint_as_float(w[e] & 0xFFFF0000u);
          sq = fmaf(a, a, sq);
          sq = fmaf(b2, b2, sq);
        }
      }
      const float xn = sq + __shfl_xor(sq, 32, 64);
      const float off = (xn + 2.f * mmax) * (1.f + 0x1p-10f) + 1.f;
      offs[t] = off;
      uint32_t o1, o2, o3;
      split3(0.5f * off, o1, o2, o3);
      btail[t] = lane < 32 ? make_uint4(BF1 | (BF1 << 16), BF1 | (o1 << 16), o2 | (o3 << 16), 0u)
                           : make_uint4(0, 0, 0, 0);
    }

    // ~511 held in a vector register: with the code in a scalar register,
    // mask and code then fit one v_and_or_b32 (one scalar operand)
    uint32_t hi_mask;
    asm volatile("v_mov_b32 %0, 0xfffffe00" : "=v"(hi_mask));
    float s1[NTL], s2[NTL];
#pragma unroll
    for (int t = 0; t < NTL; t++) s1[t] = s2[t] = 0.f;
    // one 32-row tile: 8 k-steps of the dot products and the folded constants
    auto sweep = [&](int m, f32x16_t* acc) {
#pragma unroll
      for (int t = 0; t < NTL; t++) acc[t] = (f32x16_t){};
      const uint8_t* arow = crow + (32 * m + (lane & 31)) * ROWA + 16 * (lane >> 5);
#pragma unroll
      for (int k = 0; k < 8; k++) {
        const bf16x8_t a =
            __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(arow + 32 * k));
#pragma unroll
        for (int t = 0; t < NTL; t++)
          acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              a, __builtin_bit_cast(bf16x8_t, bfrag[t][k]), acc[t], 0, 0, 0);
      }
      // every lane loads (no branch), lanes 32-63 then supply zeros
      const uint4 tv = ctail[32 * m + (lane & 31)];
      const bool lo32 = lane < 32;
      const uint4 av = make_uint4(lo32 ? tv.x : 0u, lo32 ? tv.y : 0u, lo32 ? tv.z : 0u, 0u);
      const bf16x8_t a = __builtin_bit_cast(bf16x8_t, av);
#pragma unroll
      for (int t = 0; t < NTL; t++)
        acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            a, __builtin_bit_cast(bf16x8_t, btail[t]), acc[t], 0, 0, 0);
    };
    // epilogue: lane holds column (lane & 31), rows
    // r = 32 m + 8 (i / 4) + 4 (lane >> 5) + (i % 4); the code 511 - r goes in
    // the low 9 bits
    auto fold = [&](int m, const f32x16_t* acc) {
      // the code of row r is 511 - r = 511 ^ r. Bit 2 of r is 4 (lane >> 5)
      // and the other bits are wave-uniform, so the fold uses the uniform
      // part 511 ^ (r - 4 (lane >> 5)) (bit 2 set for every row of a lane,
      // which leaves the lane's order unchanged) and the lane's bit 2 is
      // fixed once after the sweep.
      const int cm = 511 - 32 * m;  // (the codes live in scalar registers)
      // two scores at a time: the best of {s1, e0, e1} is a three-input max,
      // the second best of {s1, s2, e0, e1} the larger of s2 and the median
      // of {s1, e0, e1} (s1 >= s2 holds throughout). The encoded values are
      // non-negative floats, whose order is the order of their bit patterns,
      // so the float three-input max and median instructions serve.
#pragma unroll
      for (int i = 0; i < 16; i += 2) {
        const uint32_t code = (uint32_t)(cm - (8 * (i >> 2) + (i & 3)));  // row i + 1: code - 1
#pragma unroll
        for (int t = 0; t < NTL; t++) {
          const float e0 = __uint_as_float((__float_as_uint(acc[t][i]) & hi_mask) | code);
          const float e1 = __uint_as_float((__float_as_uint(acc[t][i + 1]) & hi_mask) | (code - 1u));
          const float md = __builtin_amdgcn_fmed3f(e0, e1, s1[t]);
          s1[t] = fmaxf(fmaxf(s1[t], e0), e1);
          s2[t] = fmaxf(s2[t], md);
        }
      }
    };
    // two accumulator sets: tile m + 1 is swept while tile m is folded (nm
    // is even); the last two tiles are peeled so that no tile is swept
    // twice. Then the next block's points are requested, in flight while the
    // labels are written.
    f32x16_t accA[NTL], accB[NTL];

    sweep(0, accA);
#pragma unroll 1
    for (int m = 0; m < nm - 2; m += 2) {
      sweep(m + 1, accB);
      fold(m, accA);
      sweep(m + 2, accA);
      fold(m + 1, accB);
      // interleave: each MFMA followed by a few epilogue instructions
#pragma unroll
      for (int i = 0; i < 36; i++) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);
      }
    }
    sweep(nm - 1, accB);
    fold(nm - 2, accA);
#pragma unroll
    for (int i = 0; i < 18; i++) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);
    }
    fold(nm - 1, accB);
    int jn = 0;
    if (lane == 0) jn = atomicAdd(&next_unit, 1);
    const int pn = unit_base(__builtin_amdgcn_readfirstlane(jn));
    if (pn < n) load_points(pn, bfrag);

#pragma unroll
    for (int t = 0; t < NTL; t++) {
      // the lane's bit 2 of the row code (rows 4 (lane >> 5) apart)
      const uint32_t h4 = (uint32_t)(lane >> 5) << 2;
      const uint32_t c1 = __float_as_uint(s1[t]) ^ h4, c2 = __float_as_uint(s2[t]) ^ h4;
      const uint32_t o1 = __shfl_xor(c1, 32, 64), o2 = __shfl_xor(c2, 32, 64);
      const uint32_t b1 = max(c1, o1);
      const uint32_t b2 = max(min(c1, o1), max(c2, o2));
      const int p = pb + 32 * t + (lane & 31);
      if (lane < 32 && p < n) {
        const float a1 = __uint_as_float(b1 & ~511u), a2 = __uint_as_float(b2 & ~511u);
        const int64_t pid = (int64_t)u * g.n_idx + (int64_t)s * g.seg_len + p;
        if (!(a1 - a2 > 0x1p-13f * offs[t])) {
          ws.label[pid] = -1;
          const int slot = atomicAdd(ws.amb, 1);
          ws.amb[1 + slot] = (int)pid;
        } else {
          ws.label[pid] = 511 - (int)(b1 & 511u);
        }
      }
    }
    pb = pn;
  }
}

// ---------------------------------------------------------------------------
// fp32: each wave owns 1 column tile of 32 points (32 points per wave).
__global__ __launch_bounds__(AT, 2) void assign_f32_kernel(Geom g, const void* __restrict__ K,
                                                           const void* __restrict__ cent,
                                                           BuildWs ws) {
  extern __shared__ __align__(16) uint8_t lds[];
  uint8_t* crow = lds;
  float* cnorm = reinterpret_cast<float*>(lds + (CHUNK / 2) * ROWF);
  float* red = cnorm + CHUNK / 2;
  constexpr int FCH = CHUNK / 2;  // 128 fp32 centroids per pass

  const int gs = blockIdx.y, u = gs / g.n_seg, s = gs % g.n_seg;
  const int n = seg_n(g, s), Cs = seg_c(g, s), cb = seg_cbase(g, s);
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int p0 = blockIdx.x * 128;  // 128 points per block
  if (p0 >= n) return;
  const int64_t first = seg_first(g, s);

  // B operand of v_mfma_f32_32x32x2_f32: lane supplies B[k = lane>>5][col]
  const int p = p0 + 32 * wv + (lane & 31);
  float bx[64];
  float sq = 0.f;
  if (p < n) {
    const float* row = reinterpret_cast<const float*>(kptr<WI_F32>(K, g, u, first + p));
#pragma unroll
    for (int k = 0; k < 64; k++) {
      bx[k] = row[2 * k + (lane >> 5)];
      sq = fmaf(bx[k], bx[k], sq);
    }
  } else {
#pragma unroll
    for (int k = 0; k < 64; k++) bx[k] = 0.f;
  }
  const float xn = sq + __shfl_xor(sq, 32, 64);

  Best best = {-INFINITY, -INFINITY, 0};
  float mmax = 0.f;
  const float* C32 = reinterpret_cast<const float*>(cent) + ((int64_t)u * g.C + cb) * D;
  for (int c0 = 0; c0 < Cs; c0 += FCH) {
    __syncthreads();
    for (int rr = tid >> 4; rr < FCH; rr += AT / 16) {
      const int c = c0 + rr;
      const int j = tid & 15;
      float4 v0 = make_float4(0, 0, 0, 0), v1 = v0;
      if (c < Cs) {
        v0 = reinterpret_cast<const float4*>(C32 + (int64_t)c * D)[2 * j];
        v1 = reinterpret_cast<const float4*>(C32 + (int64_t)c * D)[2 * j + 1];
      }
      float q2 = 0.f;
      q2 = fmaf(v0.x, v0.x, q2); q2 = fmaf(v0.y, v0.y, q2);
      q2 = fmaf(v0.z, v0.z, q2); q2 = fmaf(v0.w, v0.w, q2);
      q2 = fmaf(v1.x, v1.x, q2); q2 = fmaf(v1.y, v1.y, q2);
      q2 = fmaf(v1.z, v1.z, q2); q2 = fmaf(v1.w, v1.w, q2);
      float4* dst = reinterpret_cast<float4*>(crow + rr * ROWF + 32 * j);
      dst[0] = make_float4(2.f * v0.x, 2.f * v0.y, 2.f * v0.z, 2.f * v0.w);
      dst[1] = make_float4(2.f * v1.x, 2.f * v1.y, 2.f * v1.z, 2.f * v1.w);
      q2 += __shfl_xor(q2, 8, 16);
      q2 += __shfl_xor(q2, 4, 16);
      q2 += __shfl_xor(q2, 2, 16);
      q2 += __shfl_xor(q2, 1, 16);
      if (j == 0) cnorm[rr] = c < Cs ? q2 : INFINITY;
      if (c < Cs) mmax = fmaxf(mmax, q2);
    }
    __syncthreads();
    const int nm = min(FCH, Cs - c0);
    for (int m = 0; m < (nm + 31) / 32; m++) {
      f32x16_t acc = (f32x16_t){};
      const float* arow = reinterpret_cast<const float*>(crow + (32 * m + (lane & 31)) * ROWF);
#pragma unroll
      for (int k = 0; k < 64; k++)
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(arow[2 * k + (lane >> 5)], bx[k], acc, 0, 0, 0);
#pragma unroll
      for (int q = 0; q < 4; q++) {
        const int r0 = 32 * m + 8 * q + 4 * (lane >> 5);
#pragma unroll
        for (int e = 0; e < 4; e++) upd(best, acc[4 * q + e] - cnorm[r0 + e], c0 + r0 + e);
      }
    }
  }
  mmax = wave_max(mmax);
  __syncthreads();
  if (lane == 0) red[wv] = mmax;
  __syncthreads();
  mmax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  Best o;
  o.s1 = __shfl_xor(best.s1, 32, 64);
  o.s2 = __shfl_xor(best.s2, 32, 64);
  o.i1 = __shfl_xor(best.i1, 32, 64);
  const Best bb = merge(best, o);
  if (lane < 32 && p < n) {
    const float W = 0x1p-12f * (xn + 2.f * mmax);
    const int64_t pid = (int64_t)u * g.n_idx + (int64_t)s * g.seg_len + p;
    if (bb.s2 >= bb.s1 - W) {
      ws.label[pid] = -1;
      const int slot = atomicAdd(ws.amb, 1);
      ws.amb[1 + slot] = (int)pid;
    } else {
      ws.label[pid] = bb.i1;
    }
  }
}

// ---------------------------------------------------------------------------
// Exact fallback: one wave per listed point, float64 distances to every
// centroid of their segment, lowest id on ties. Lane l takes centroids l,
// l + 64, ...: it reads its centroid's row with 16-byte loads, and the point
// (in LDS, float64) is read back one broadcast value per dimension; each
// distance is summed in dimension order.
template <int DT>
__global__ __launch_bounds__(256) void assign_fix_kernel(Geom g, const void* __restrict__ K,
                                                          const void* __restrict__ cent,
                                                          BuildWs ws) {
  constexpr int ES = DT == WI_BF16 ? 2 : 4;  // bytes per element
  constexpr int NV = D * ES / 16;            // 16-byte vectors per row
  constexpr int EPV = 16 / ES;               // elements per vector
  __shared__ double xs[4][D];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int cnt = ws.amb[0];
  const int nw = gridDim.x * 4;
  for (int e = blockIdx.x * 4 + wv; e < cnt; e += nw) {
    const int pid = ws.amb[1 + e];
    const int u = (int)(pid / g.n_idx);
    const int64_t loc = pid % g.n_idx;
    const int s = (int)(loc / g.seg_len);
    const int i = (int)(loc % g.seg_len);
    const int Cs = seg_c(g, s), cb = seg_cbase(g, s);
    const uint8_t* xr = kptr<DT>(K, g, u, seg_first(g, s) + i);
    // the point into LDS (lane holds dims lane and lane + 64)
    if constexpr (DT == WI_BF16) {
      const uint16_t* x16 = reinterpret_cast<const uint16_t*>(xr);
      xs[wv][lane] = (double)__uint_as_float(((uint32_t)x16[lane]) << 16);
      xs[wv][lane + 64] = (double)__uint_as_float(((uint32_t)x16[lane + 64]) << 16);
    } else {
      const float* x32 = reinterpret_cast<const float*>(xr);
      xs[wv][lane] = (double)x32[lane];
      xs[wv][lane + 64] = (double)x32[lane + 64];
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    double bd = INFINITY;
    int bi = 0x7FFFFFFF;
    const int rounds = (Cs + 63) / 64;
    for (int rd = 0; rd < rounds; rd++) {
      const int c = rd * 64 + lane;
      const bool ok = c < Cs;
      const uint4* crow = reinterpret_cast<const uint4*>(
          reinterpret_cast<const uint8_t*>(cent) + ((int64_t)u * g.C + cb + (ok ? c : 0)) * D * ES);
      uint4 cv[NV];
#pragma unroll
      for (int v = 0; v < NV; v++) cv[v] = crow[v];
      double acc = 0.0;
#pragma unroll
      for (int v = 0; v < NV; v++) {
        const uint32_t w[4] = {cv[v].x, cv[v].y, cv[v].z, cv[v].w};
#pragma unroll
        for (int k = 0; k < EPV; k++) {
          const int t = v * EPV + k;
          double ct;
          if constexpr (DT == WI_BF16)
            ct = (double)__uint_as_float((k & 1) ? (w[k >> 1] & 0xFFFF0000u) : (w[k >> 1] << 16));
          else
            ct = (double)__uint_as_float(w[k]);
          const double dl = xs[wv][t] - ct;
          acc = __builtin_fma(dl, dl, acc);
        }
      }
      if (ok && acc < bd) {  // c grows within a lane: strict < keeps the lowest id
        bd = acc;
        bi = c;
      }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const double od = __shfl_xor(bd, o, 64);
      const int oi = __shfl_xor(bi, o, 64);
      if (od < bd || (od == bd && oi < bi)) {
        bd = od;
        bi = oi;
      }
    }
    if (lane == 0) ws.label[pid] = bi;
    // the next point rewrites this wave's row of xs only after every lane read it
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
}

}  // namespace

hipError_t launch_assign(const Geom& g, const void* K, const void* cent, const BuildWs& ws,
                         hipStream_t s) {
  hipError_t e = launch_zero_i32(ws.amb, 1, s);
  if (e != hipSuccess) return e;
  if (g.dtype == WI_BF16) {
    // about one workgroup per CU: each walks several point blocks of its segment
    const int blocks = (g.seg_len + BT - 1) / BT;
    const int segs = g.U * g.n_seg;
    int per = (256 + segs - 1) / segs;
    if (per > blocks) per = blocks;
    dim3 grid(per, segs);
    WI_LAUNCH(K_ASSIGN, assign_bf16_kernel, grid, dim3(BT), BF16_LDS, s, g, K, cent, ws);
  } else {
    const size_t lds = (CHUNK / 2) * ROWF + (CHUNK / 2) * 4 + 16;
    dim3 grid((g.seg_len + 127) / 128, g.U * g.n_seg);
    WI_LAUNCH(K_ASSIGN, assign_f32_kernel, grid, dim3(AT), lds, s, g, K, cent, ws);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (g.dtype == WI_BF16)
    WI_LAUNCH(K_ASSIGN_FIX, assign_fix_kernel<WI_BF16>, dim3(256), dim3(256), 0, s, g, K, cent, ws);
  else
    WI_LAUNCH(K_ASSIGN_FIX, assign_fix_kernel<WI_F32>, dim3(256), dim3(256), 0, s, g, K, cent, ws);
  return hipGetLastError();
}

}  // namespace wi
