// C ABI of libwi.so (declared in include/wi.h): host-side validation,
// sizes, workspace carving and the stream-ordered launch sequences of the
// index build and the decode step.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <vector>

#include "wi_internal.h"

// Device scratch of wi_decode_attention_noalloc: one copy per GPU, held from
// the library's load until the process ends. In host code the name is only a
// stand-in for the symbol; the device address is obtained per device with
// hipGetSymbolAddress (see scratch_for_current_device) and only that address
// is used.
static __device__ __align__(256) unsigned char scratch[WI_NOALLOC_SCRATCH_BYTES];

namespace {

thread_local char g_err[512] = "";

wi_status fail(wi_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

wi_status hip_fail(hipError_t e, const char* where) {
  return fail(WI_E_HIP, "%s: %s", where, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int64_t align256(int64_t x) { return (x + 255) & ~int64_t(255); }

// Validate the index descriptor and derive the call geometry.
wi_status make_geom(const wi_index_desc* d, wi::Geom* g) {
  if (!d) return fail(WI_E_INVALID, "desc is NULL");
  if (d->dtype != WI_F32 && d->dtype != WI_BF16)
    return fail(WI_E_UNSUPPORTED, "unknown dtype %d", d->dtype);
  if (d->head_dim != wi::D) return fail(WI_E_UNSUPPORTED, "head_dim %d != 128", d->head_dim);
  if (d->batch < 1 || d->n_kv_heads < 1)
    return fail(WI_E_INVALID, "batch %d / n_kv_heads %d must be >= 1", d->batch, d->n_kv_heads);
  if (d->n_sink < 0 || d->n_local < 0)
    return fail(WI_E_INVALID, "n_sink %d / n_local %d must be >= 0", d->n_sink, d->n_local);
  if (d->n_ctx >= (int64_t(1) << 31)) return fail(WI_E_INVALID, "n_ctx too large");
  if (d->seg_len < 1 || d->seg_len > wi::MAX_SEG)
    return fail(WI_E_INVALID, "seg_len %d outside [1, %d]", d->seg_len, wi::MAX_SEG);
  if (d->n_pending < 0 || d->n_pending > d->seg_len)
    return fail(WI_E_INVALID, "n_pending %lld outside [0, seg_len]", (long long)d->n_pending);
  if (d->n_ctx < (int64_t)d->n_sink + d->n_local + d->n_pending + 1)
    return fail(WI_E_INVALID, "n_ctx %lld must be >= n_sink + n_local + n_pending + 1",
                (long long)d->n_ctx);
  if (d->clusters_per_seg < 1 || d->clusters_per_seg > wi::MAX_K)
    return fail(WI_E_INVALID, "clusters_per_seg %d outside [1, %d]", d->clusters_per_seg,
                wi::MAX_K);
  if (d->n_iters < 0) return fail(WI_E_INVALID, "n_iters %d < 0", d->n_iters);
  if (d->kv_stride_t <= 0 || d->kv_stride_h < 0 || d->kv_stride_b < 0 ||
      d->kv_stride_t % 8 || d->kv_stride_h % 8 || d->kv_stride_b % 8)
    return fail(WI_E_INVALID, "K/V strides must be non-negative multiples of 8 (t > 0)");
  wi::Geom& G = *g;
  G.dtype = d->dtype;
  G.B = d->batch;
  G.H = d->n_kv_heads;
  G.U = d->batch * d->n_kv_heads;
  G.N = d->n_ctx;
  G.n_sink = d->n_sink;
  G.n_local = d->n_local;
  G.n_st = d->n_sink + d->n_local;
  G.n_idx = d->n_ctx - G.n_st - d->n_pending;
  G.n_pend = (int)d->n_pending;
  G.seg_ord0 = 0;
  G.seg_len = d->seg_len;
  G.kk = d->clusters_per_seg;
  G.n_seg = (int)((G.n_idx + G.seg_len - 1) / G.seg_len);
  int64_t C = 0;
  for (int s = 0; s < G.n_seg; s++) C += wi::seg_c(G, s);
  if ((int64_t)G.U * G.n_idx >= (int64_t(1) << 31) || (int64_t)G.U * C >= (int64_t(1) << 31))
    return fail(WI_E_INVALID, "batch * heads * tokens exceeds 2^31");
  G.C = (int)C;
  G.T = 2048 / (wi::D * (d->dtype == WI_BF16 ? 2 : 4));
  G.cap = (G.n_idx + C * (G.T - 1)) / G.T;
  G.sb = d->kv_stride_b;
  G.sh = d->kv_stride_h;
  G.st = d->kv_stride_t;
  G.seed = d->seed;
  G.layer = d->layer_id;
  G.n_iters = d->n_iters;
  int cmax = G.kk < G.seg_len ? G.kk : G.seg_len;
  if ((int64_t)cmax > G.n_idx) cmax = (int)G.n_idx;
  G.cmax = cmax;
  return WI_OK;
}

// Build workspace layout; with base == nullptr only the size is computed.
int64_t carve_build(const wi::Geom& g, uint8_t* base, wi::BuildWs* w) {
  const int64_t P = (int64_t)g.U * g.n_idx;
  const int nsl = (g.seg_len + wi::KPP_SLICE - 1) / wi::KPP_SLICE;
  int64_t off = 0;
  auto take = [&](int64_t bytes) {
    uint8_t* p = base ? base + off : nullptr;
    off += align256(bytes);
    return p;
  };
  wi::BuildWs t;
  t.D = reinterpret_cast<float*>(take(P * 4));
  t.w[0] = reinterpret_cast<unsigned long long*>(take(P * 8));
  t.w[1] = reinterpret_cast<unsigned long long*>(take(P * 8));
  t.chosen = take(P);
  t.kpp = reinterpret_cast<wi::KppPartial*>(
      take((int64_t)g.U * g.n_seg * nsl * (int64_t)sizeof(wi::KppPartial)));
  t.label = reinterpret_cast<int*>(take(P * 4));
  t.members = reinterpret_cast<int*>(take(P * 4));
  t.cl_off = reinterpret_cast<int*>(take((int64_t)g.U * g.C * 4));
  t.amb = reinterpret_cast<int*>(take((P + 1) * 4));
  t.seg_blocks = reinterpret_cast<int*>(take((int64_t)g.U * g.n_seg * 4));
  t.seg_bbase = reinterpret_cast<int*>(take((int64_t)g.U * g.n_seg * 4));
  t.unit_used = reinterpret_cast<int*>(take((int64_t)g.U * 4));
  if (w) *w = t;
  return off;
}

struct DecodeShape {
  int Hq, G, GS, K_r, K_e, W;
  float scale;
};

wi_status make_decode(const wi::Geom& g, const wi_decode_desc* dd, DecodeShape* o) {
  if (!dd) return fail(WI_E_INVALID, "decode desc is NULL");
  if (dd->n_q_heads < 1 || dd->n_q_heads % g.H)
    return fail(WI_E_UNSUPPORTED, "n_q_heads %d is not a multiple of n_kv_heads %d",
                dd->n_q_heads, g.H);
  const int G = dd->n_q_heads / g.H;
  if (G > wi::MAX_G) return fail(WI_E_UNSUPPORTED, "%d query heads per KV head > %d", G, wi::MAX_G);
  if (g.C > 65536) return fail(WI_E_UNSUPPORTED, "%d clusters per unit > 65536", g.C);
  if (dd->k_retrieve < 0 || dd->k_retrieve > g.C)
    return fail(WI_E_INVALID, "k_retrieve %d outside [0, C=%d]", dd->k_retrieve, g.C);
  if (dd->k_estimate < 0) return fail(WI_E_INVALID, "k_estimate %d < 0", dd->k_estimate);
  if (!(dd->scale >= 0.f) || !std::isfinite(dd->scale))
    return fail(WI_E_INVALID, "scale must be finite and >= 0");
  if (dd->wg_per_unit < 0 || dd->wg_per_unit > wi::MAX_WG)
    return fail(WI_E_INVALID, "wg_per_unit %d outside [0, %d]", dd->wg_per_unit, wi::MAX_WG);
  o->Hq = dd->n_q_heads;
  o->G = G;
  o->GS = G <= 4 ? 4 : (G <= 8 ? 8 : 16);
  o->K_r = dd->k_retrieve;
  o->K_e = dd->k_estimate < g.C - dd->k_retrieve ? dd->k_estimate : g.C - dd->k_retrieve;
  o->scale = dd->scale > 0.f ? dd->scale : 1.0f / std::sqrt((float)wi::D);
  // fused kernel: the caller's count, or about one workgroup per CU over the
  // whole call; at most MAX_WG per unit and no more than the unit's
  // 16-cluster ownership groups
  int W = dd->wg_per_unit > 0 ? dd->wg_per_unit : (256 + g.U - 1) / g.U;
  const int groups = (g.C + 15) / 16;
  if (W > groups) W = groups;
  if (W > wi::MAX_WG) W = wi::MAX_WG;
  if (W < 1) W = 1;
  o->W = W;
  return WI_OK;
}

int64_t carve_decode(const wi::Geom& g, const DecodeShape& ds, uint8_t* base, wi::DecodeWs* w) {
  int64_t off = 0;
  auto take = [&](int64_t bytes) {
    uint8_t* p = base ? base + off : nullptr;
    off += align256(bytes);
    return p;
  };
  wi::DecodeWs t;
  const int64_t Cp = (g.C + 3) & ~3;
  t.key = reinterpret_cast<uint32_t*>(take((int64_t)g.U * Cp * 4));
  t.S = reinterpret_cast<float*>(take((int64_t)g.U * g.C * ds.GS * 4));
  t.mm = reinterpret_cast<float2*>(take((int64_t)g.U * wi::score_blocks(g) * 8));
  t.part = reinterpret_cast<float*>(take((int64_t)g.U * ds.W * ds.G * (2 + wi::D) * 4));
  t.tix = reinterpret_cast<int*>(take((int64_t)g.U * 4));
  t.zone = take((int64_t)g.U * g.C);
  t.rank = reinterpret_cast<int*>(take((int64_t)g.U * (ds.K_r + ds.K_e) * 4));
  if (w) *w = t;
  return off;
}

#define CHECK_PTR(p, name)                                              \
  do {                                                                  \
    if (!(p)) return fail(WI_E_INVALID, "%s is NULL", name);            \
    if (!aligned16(p)) return fail(WI_E_INVALID, "%s is not 16-byte aligned", name); \
  } while (0)

#define CHECK_HIP(expr, where)                 \
  do {                                         \
    hipError_t e_ = (expr);                    \
    if (e_ != hipSuccess) return hip_fail(e_, where); \
  } while (0)

// The build's launch sequence: k-means++ (or the given centroids), n_iters x
// (assign, update), layout. k_blocks holds >= U * n_idx key rows (block_cap *
// T >= n_idx) and is written only by the layout step, so k-means++ keeps its
// chunked copy of the keys there until then.
wi_status run_build(const wi::Geom& g, const void* k, const void* v, const void* init_centroids,
                    const wi_index_bufs& b, wi::BuildWs& w, hipStream_t stream) {
  w.kc = b.k_blocks;
  if (init_centroids)
    CHECK_HIP(wi::launch_copy_init(g, init_centroids, b.centroids, stream), "copy init");
  else
    CHECK_HIP(wi::launch_kpp(g, k, b.centroids, w, stream), "k-means++");
  const int iters = g.n_iters > 0 ? g.n_iters : 1;
  for (int t = 0; t < iters; t++) {
    CHECK_HIP(wi::launch_assign(g, k, b.centroids, w, stream), "assign");
    CHECK_HIP(wi::launch_sort_update(g, k, b.centroids, b.cluster_size, w, g.n_iters > 0,
                                     stream),
              "update");
  }
  CHECK_HIP(wi::launch_layout(g, k, v, b, w, stream), "layout");
  return WI_OK;
}

// Geometry of the pending segment as a one-segment index of its own (no
// steady zone; K/V rows are the pending rows [U][seg_len][128]), and the
// carve of its buffers followed by its build workspace.
wi_status segment_geom(const wi_index_desc* desc, const wi::Geom& g, wi::Geom* gs) {
  wi_index_desc d = *desc;
  d.n_ctx = g.seg_len;
  d.n_sink = 0;
  d.n_local = 0;
  d.n_pending = 0;
  d.kv_stride_b = (int64_t)g.H * g.seg_len * wi::D;
  d.kv_stride_h = (int64_t)g.seg_len * wi::D;
  d.kv_stride_t = wi::D;
  wi_status st = make_geom(&d, gs);
  if (st != WI_OK) return st;
  gs->seg_ord0 = g.n_seg;  // the new segment's ordinal in the stream
  return WI_OK;
}

int64_t carve_segment(const wi::Geom& gs, uint8_t* base, wi_index_bufs* b, wi::BuildWs* w) {
  const int64_t e = gs.dtype == WI_BF16 ? 2 : 4;
  const int64_t U = gs.U;
  int64_t off = 0;
  auto take = [&](int64_t bytes) {
    uint8_t* p = base ? base + off : nullptr;
    off += align256(bytes);
    return p;
  };
  wi_index_bufs t{};
  t.centroids = take(U * gs.C * wi::D * e);
  t.cluster_size = reinterpret_cast<int32_t*>(take(U * gs.C * 4));
  t.value_sum = reinterpret_cast<float*>(take(U * gs.C * wi::D * 4));
  t.block_off = reinterpret_cast<int32_t*>(take(U * (gs.C + 1) * 4));
  t.k_blocks = take(U * gs.cap * gs.T * wi::D * e);
  t.v_blocks = take(U * gs.cap * gs.T * wi::D * e);
  t.slot_token = reinterpret_cast<int32_t*>(take(U * gs.cap * gs.T * 4));
  t.assign = reinterpret_cast<int32_t*>(take(U * gs.n_idx * 4));
  if (b) *b = t;
  const int64_t wb = carve_build(gs, base ? base + off : nullptr, w);
  return off + wb;
}

// Measurement hook state (per host thread).
struct TimingRec {
  int id;
  hipEvent_t a, b;
};
thread_local bool t_on = false;
thread_local std::vector<TimingRec> t_recs;
thread_local std::vector<hipEvent_t> t_pool;
thread_local int t_cur = -1;

const char* const kNames[wi::K_COUNT] = {
    "zero", "copy_init", "kpp_init", "kpp_weights", "kpp_round", "assign", "assign_fix",
    "sort_update", "seg_scan", "layout", "score", "select_attend", "rank", "exec", "append",
    "merge", "dense", "dense_merge", "recall", "wb_update", "wb_fill"};

hipEvent_t take_event() {
  if (!t_pool.empty()) {
    hipEvent_t e = t_pool.back();
    t_pool.pop_back();
    return e;
  }
  // timing-only events: no system-scope fence when they are recorded, so the
  // bracket adds no cache writeback/invalidate around the launch it times
  hipEvent_t e = nullptr;
  if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) return nullptr;
  return e;
}

}  // namespace

namespace wi {
void tmark_begin(KernelId id, hipStream_t s) {
  if (!t_on) return;
  TimingRec r{(int)id, take_event(), take_event()};
  if (r.a) hipEventRecord(r.a, s);
  t_recs.push_back(r);
  t_cur = (int)t_recs.size() - 1;
}
void tmark_end(hipStream_t s) {
  if (!t_on || t_cur < 0) return;
  if (t_recs[t_cur].b) hipEventRecord(t_recs[t_cur].b, s);
  t_cur = -1;
}
}  // namespace wi

extern "C" {

wi_status wi_timing_start(void) {
  t_on = true;
  t_recs.clear();
  return WI_OK;
}

int32_t wi_timing_stop(int32_t max_records, int32_t* name_ids, float* ms) {
  t_on = false;
  int32_t n = (int32_t)t_recs.size();
  int32_t rc = n;
  for (int32_t i = 0; i < n; i++) {
    TimingRec& r = t_recs[i];
    float t = -1.f;
    if (r.a && r.b) {
      if (hipEventSynchronize(r.b) != hipSuccess || hipEventElapsedTime(&t, r.a, r.b) != hipSuccess)
        rc = -1;
    }
    if (i < max_records) {
      if (name_ids) name_ids[i] = r.id;
      if (ms) ms[i] = t;
    }
    if (r.a) t_pool.push_back(r.a);
    if (r.b) t_pool.push_back(r.b);
  }
  t_recs.clear();
  return rc;
}

const char* wi_kernel_name(int32_t id) {
  return (id >= 0 && id < wi::K_COUNT) ? kNames[id] : "unknown";
}


const char* wi_status_str(wi_status s) {
  switch (s) {
    case WI_OK: return "WI_OK";
    case WI_E_INVALID: return "WI_E_INVALID";
    case WI_E_UNSUPPORTED: return "WI_E_UNSUPPORTED";
    case WI_E_WORKSPACE: return "WI_E_WORKSPACE";
    case WI_E_HIP: return "WI_E_HIP";
  }
  return "WI_E_UNKNOWN";
}

const char* wi_last_error(void) { return g_err; }

wi_status wi_index_sizes(const wi_index_desc* desc, int64_t* n_segments, int64_t* n_clusters,
                         int64_t* block_cap, size_t* workspace_bytes) {
  wi::Geom g;
  wi_status st = make_geom(desc, &g);
  if (st != WI_OK) return st;
  if (n_segments) *n_segments = g.n_seg;
  if (n_clusters) *n_clusters = g.C;
  if (block_cap) *block_cap = g.cap;
  if (workspace_bytes) *workspace_bytes = (size_t)carve_build(g, nullptr, nullptr);
  g_err[0] = 0;
  return WI_OK;
}

wi_status wi_build_index(const wi_index_desc* desc, const void* k, const void* v,
                         const void* init_centroids, const wi_index_bufs* bufs, void* ws,
                         size_t ws_bytes, hipStream_t stream) {
  wi::Geom g;
  wi_status st = make_geom(desc, &g);
  if (st != WI_OK) return st;
  if (g.n_pend != 0) return fail(WI_E_INVALID, "an index is built with n_pending = 0");
  CHECK_PTR(k, "k");
  CHECK_PTR(v, "v");
  if (init_centroids && !aligned16(init_centroids))
    return fail(WI_E_INVALID, "init_centroids is not 16-byte aligned");
  if (!bufs) return fail(WI_E_INVALID, "bufs is NULL");
  CHECK_PTR(bufs->centroids, "bufs->centroids");
  CHECK_PTR(bufs->cluster_size, "bufs->cluster_size");
  CHECK_PTR(bufs->value_sum, "bufs->value_sum");
  CHECK_PTR(bufs->block_off, "bufs->block_off");
  CHECK_PTR(bufs->k_blocks, "bufs->k_blocks");
  CHECK_PTR(bufs->v_blocks, "bufs->v_blocks");
  CHECK_PTR(bufs->slot_token, "bufs->slot_token");
  CHECK_PTR(bufs->assign, "bufs->assign");
  if (g.n_st > 0) {
    CHECK_PTR(bufs->steady_k, "bufs->steady_k");
    CHECK_PTR(bufs->steady_v, "bufs->steady_v");
  }
  const int64_t need = carve_build(g, nullptr, nullptr);
  if (!ws || (int64_t)ws_bytes < need)
    return fail(WI_E_WORKSPACE, "workspace %zu bytes < %lld required", ws_bytes, (long long)need);
  if (!aligned16(ws)) return fail(WI_E_INVALID, "ws is not 16-byte aligned");
  wi::BuildWs w;
  carve_build(g, reinterpret_cast<uint8_t*>(ws), &w);

  st = run_build(g, k, v, init_centroids, *bufs, w, stream);
  if (st == WI_OK) g_err[0] = 0;
  return st;
}

wi_status wi_decode_sizes(const wi_index_desc* desc, const wi_decode_desc* ddesc,
                          size_t* workspace_bytes) {
  wi::Geom g;
  wi_status st = make_geom(desc, &g);
  if (st != WI_OK) return st;
  DecodeShape ds;
  st = make_decode(g, ddesc, &ds);
  if (st != WI_OK) return st;
  if (workspace_bytes) *workspace_bytes = (size_t)carve_decode(g, ds, nullptr, nullptr);
  g_err[0] = 0;
  return WI_OK;
}

}  // extern "C"

namespace {

// Host-side validation of a decode call (no HIP call); on success the
// geometry, decode shape and workspace size are returned.
wi_status validate_decode(const wi_index_desc* desc, const wi_decode_desc* ddesc,
                          const wi_index_bufs* bufs, const void* q, const float* out,
                          const int32_t* sel_ids, const int32_t* exec_tokens,
                          const int32_t* n_exec, int64_t exec_cap, wi::Geom* g,
                          DecodeShape* ds, int64_t* need) {
  wi_status st = make_geom(desc, g);
  if (st != WI_OK) return st;
  st = make_decode(*g, ddesc, ds);
  if (st != WI_OK) return st;
  if (!bufs) return fail(WI_E_INVALID, "bufs is NULL");
  CHECK_PTR(bufs->centroids, "bufs->centroids");
  CHECK_PTR(bufs->cluster_size, "bufs->cluster_size");
  CHECK_PTR(bufs->value_sum, "bufs->value_sum");
  CHECK_PTR(bufs->block_off, "bufs->block_off");
  CHECK_PTR(bufs->k_blocks, "bufs->k_blocks");
  CHECK_PTR(bufs->v_blocks, "bufs->v_blocks");
  if (g->n_st > 0) {
    CHECK_PTR(bufs->steady_k, "bufs->steady_k");
    CHECK_PTR(bufs->steady_v, "bufs->steady_v");
  }
  if (g->n_pend > 0) {
    CHECK_PTR(bufs->pend_k, "bufs->pend_k");
    CHECK_PTR(bufs->pend_v, "bufs->pend_v");
  }
  CHECK_PTR(q, "q");
  CHECK_PTR(out, "out");
  if (sel_ids && !aligned16(sel_ids)) return fail(WI_E_INVALID, "sel_ids is not 16-byte aligned");
  if (n_exec && !aligned16(n_exec)) return fail(WI_E_INVALID, "n_exec is not 16-byte aligned");
  if (exec_tokens) {
    if (!aligned16(exec_tokens)) return fail(WI_E_INVALID, "exec_tokens is not 16-byte aligned");
    if (exec_cap < 0) return fail(WI_E_INVALID, "exec_cap < 0");
    CHECK_PTR(bufs->slot_token, "bufs->slot_token");
  }
  *need = carve_decode(*g, *ds, nullptr, nullptr);
  return WI_OK;
}

// The decode launches on a validated call, with the workspace at ws.
wi_status run_decode(const wi::Geom& g, const DecodeShape& ds, const wi_index_bufs* bufs,
                     const void* q, float* out, int32_t* sel_ids, int32_t* exec_tokens,
                     int32_t* n_exec, int64_t exec_cap, void* ws, hipStream_t stream) {
  wi::DecodeWs w;
  carve_decode(g, ds, reinterpret_cast<uint8_t*>(ws), &w);
  wi::DecodeArgs a{&g, ds.Hq, ds.G, ds.GS, ds.K_r, ds.K_e, ds.W, ds.scale};
  const bool want_lists = sel_ids || exec_tokens || n_exec;
  CHECK_HIP(wi::launch_score(a, bufs->centroids, q, w, stream), "score");
  CHECK_HIP(wi::launch_fused(a, *bufs, q, out, w, want_lists, stream), "select/attend");
  if (want_lists)
    CHECK_HIP(wi::launch_debug_outputs(a, *bufs, w, sel_ids, exec_tokens, n_exec, exec_cap,
                                       stream),
              "debug outputs");
  g_err[0] = 0;
  return WI_OK;
}

// Device address of the current device's copy of `scratch`, looked up once
// per device (with that device current) and kept.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

wi_status scratch_for_current_device(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(WI_E_UNSUPPORTED, "device ordinal %d outside [0, %d)", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (!p) return fail(WI_E_HIP, "hipGetSymbolAddress(scratch) returned NULL");
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return WI_OK;
}

}  // namespace

extern "C" {

wi_status wi_decode_attention(const wi_index_desc* desc, const wi_decode_desc* ddesc,
                              const wi_index_bufs* bufs, const void* q, float* out,
                              int32_t* sel_ids, int32_t* exec_tokens, int32_t* n_exec,
                              int64_t exec_cap, void* ws, size_t ws_bytes, hipStream_t stream) {
  wi::Geom g;
  DecodeShape ds;
  int64_t need = 0;
  wi_status st = validate_decode(desc, ddesc, bufs, q, out, sel_ids, exec_tokens, n_exec,
                                 exec_cap, &g, &ds, &need);
  if (st != WI_OK) return st;
  if (!ws || (int64_t)ws_bytes < need)
    return fail(WI_E_WORKSPACE, "workspace %zu bytes < %lld required", ws_bytes, (long long)need);
  if (!aligned16(ws)) return fail(WI_E_INVALID, "ws is not 16-byte aligned");
  return run_decode(g, ds, bufs, q, out, sel_ids, exec_tokens, n_exec, exec_cap, ws, stream);
}

wi_status wi_decode_attention_noalloc(const wi_index_desc* desc, const wi_decode_desc* ddesc,
                                      const wi_index_bufs* bufs, const void* q, float* out,
                                      int32_t* sel_ids, int32_t* exec_tokens, int32_t* n_exec,
                                      int64_t exec_cap, hipStream_t stream) {
  wi::Geom g;
  DecodeShape ds;
  int64_t need = 0;
  wi_status st = validate_decode(desc, ddesc, bufs, q, out, sel_ids, exec_tokens, n_exec,
                                 exec_cap, &g, &ds, &need);
  if (st != WI_OK) return st;
  if (need > (int64_t)WI_NOALLOC_SCRATCH_BYTES)
    return fail(WI_E_WORKSPACE,
                "decode needs %lld bytes of scratch, more than the %lld-byte static array; "
                "use wi_decode_attention with a caller workspace",
                (long long)need, (long long)WI_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  st = scratch_for_current_device(&ws);
  if (st != WI_OK) return st;
  return run_decode(g, ds, bufs, q, out, sel_ids, exec_tokens, n_exec, exec_cap, ws, stream);
}

wi_status wi_append_token(const wi_index_desc* desc, const wi_index_bufs* bufs,
                          const void* k_new, const void* v_new, hipStream_t stream) {
  wi::Geom g;
  wi_status st = make_geom(desc, &g);
  if (st != WI_OK) return st;
  if (g.n_pend >= g.seg_len)
    return fail(WI_E_INVALID, "n_pending = seg_len: cluster the segment (wi_extend_index) first");
  if (!bufs) return fail(WI_E_INVALID, "bufs is NULL");
  if (g.n_st > 0) {
    CHECK_PTR(bufs->steady_k, "bufs->steady_k");
    CHECK_PTR(bufs->steady_v, "bufs->steady_v");
  }
  CHECK_PTR(bufs->pend_k, "bufs->pend_k");
  CHECK_PTR(bufs->pend_v, "bufs->pend_v");
  CHECK_PTR(k_new, "k_new");
  CHECK_PTR(v_new, "v_new");
  CHECK_HIP(wi::launch_append(g, *bufs, k_new, v_new, stream), "append");
  g_err[0] = 0;
  return WI_OK;
}

wi_status wi_append_sizes(const wi_index_desc* desc, size_t* workspace_bytes) {
  wi::Geom g;
  wi_status st = make_geom(desc, &g);
  if (st != WI_OK) return st;
  if (workspace_bytes)
    *workspace_bytes = (size_t)align256((int64_t)2 * g.U * g.n_local * wi::D *
                                        (g.dtype == WI_BF16 ? 2 : 4) + 16);
  g_err[0] = 0;
  return WI_OK;
}

wi_status wi_append_tokens(const wi_index_desc* desc, const wi_index_bufs* bufs,
                           const void* k_new, const void* v_new, int32_t n_new, void* ws,
                           size_t ws_bytes, hipStream_t stream) {
  wi::Geom g;
  wi_status st = make_geom(desc, &g);
  if (st != WI_OK) return st;
  if (n_new < 1 || (int64_t)g.n_pend + n_new > g.seg_len)
    return fail(WI_E_INVALID, "n_new %d outside [1, seg_len - n_pending = %d]", n_new,
                g.seg_len - g.n_pend);
  if (!bufs) return fail(WI_E_INVALID, "bufs is NULL");
  if (g.n_st > 0) {
    CHECK_PTR(bufs->steady_k, "bufs->steady_k");
    CHECK_PTR(bufs->steady_v, "bufs->steady_v");
  }
  CHECK_PTR(bufs->pend_k, "bufs->pend_k");
  CHECK_PTR(bufs->pend_v, "bufs->pend_v");
  CHECK_PTR(k_new, "k_new");
  CHECK_PTR(v_new, "v_new");
  size_t need = 0;
  st = wi_append_sizes(desc, &need);
  if (st != WI_OK) return st;
  if (!ws || ws_bytes < need)
    return fail(WI_E_WORKSPACE, "workspace %zu bytes < %zu required", ws_bytes, need);
  if (!aligned16(ws)) return fail(WI_E_INVALID, "ws is not 16-byte aligned");
  CHECK_HIP(wi::launch_append_many(g, *bufs, k_new, v_new, n_new, ws, stream), "append");
  g_err[0] = 0;
  return WI_OK;
}

wi_status wi_extend_sizes(const wi_index_desc* desc, size_t* workspace_bytes) {
  wi::Geom g, gs;
  wi_status st = make_geom(desc, &g);
  if (st != WI_OK) return st;
  if (g.n_pend != g.seg_len)
    return fail(WI_E_INVALID, "n_pending %d != seg_len %d", g.n_pend, g.seg_len);
  st = segment_geom(desc, g, &gs);
  if (st != WI_OK) return st;
  if (workspace_bytes) *workspace_bytes = (size_t)carve_segment(gs, nullptr, nullptr, nullptr);
  g_err[0] = 0;
  return WI_OK;
}

wi_status wi_extend_index(const wi_index_desc* desc, const wi_index_bufs* bufs,
                          const wi_index_bufs* new_bufs, void* ws, size_t ws_bytes,
                          hipStream_t stream) {
  wi::Geom g, gn, gs;
  wi_status st = make_geom(desc, &g);
  if (st != WI_OK) return st;
  if (g.n_pend != g.seg_len)
    return fail(WI_E_INVALID, "n_pending %d != seg_len %d", g.n_pend, g.seg_len);
  wi_index_desc dn = *desc;
  dn.n_pending = 0;
  st = make_geom(&dn, &gn);
  if (st != WI_OK) return st;
  st = segment_geom(desc, g, &gs);
  if (st != WI_OK) return st;
  if (gn.C != g.C + gs.C) return fail(WI_E_INVALID, "inconsistent cluster counts");
  if (!bufs || !new_bufs) return fail(WI_E_INVALID, "bufs is NULL");
  const wi_index_bufs* sides[2] = {bufs, new_bufs};
  for (const wi_index_bufs* b : sides) {
    CHECK_PTR(b->centroids, "centroids");
    CHECK_PTR(b->cluster_size, "cluster_size");
    CHECK_PTR(b->value_sum, "value_sum");
    CHECK_PTR(b->block_off, "block_off");
    CHECK_PTR(b->k_blocks, "k_blocks");
    CHECK_PTR(b->v_blocks, "v_blocks");
    CHECK_PTR(b->slot_token, "slot_token");
    CHECK_PTR(b->assign, "assign");
    if (g.n_st > 0) {
      CHECK_PTR(b->steady_k, "steady_k");
      CHECK_PTR(b->steady_v, "steady_v");
    }
  }
  CHECK_PTR(bufs->pend_k, "bufs->pend_k");
  CHECK_PTR(bufs->pend_v, "bufs->pend_v");
  const int64_t need = carve_segment(gs, nullptr, nullptr, nullptr);
  if (!ws || (int64_t)ws_bytes < need)
    return fail(WI_E_WORKSPACE, "workspace %zu bytes < %lld required", ws_bytes, (long long)need);
  if (!aligned16(ws)) return fail(WI_E_INVALID, "ws is not 16-byte aligned");
  wi_index_bufs sb;
  wi::BuildWs w;
  carve_segment(gs, reinterpret_cast<uint8_t*>(ws), &sb, &w);
  st = run_build(gs, bufs->pend_k, bufs->pend_v, nullptr, sb, w, stream);
  if (st != WI_OK) return st;
  CHECK_HIP(wi::launch_extend_merge(g, gn, gs, *bufs, sb, *new_bufs, stream), "merge");
  g_err[0] = 0;
  return WI_OK;
}

wi_status wi_layer_plan(int32_t policy, int32_t layer, int32_t n_layers, int64_t n_ctx,
                        int32_t seg_len, int32_t clusters_per_seg, int32_t* mode,
                        int32_t* k_retrieve, int32_t* k_estimate) {
  if (n_layers < 1 || layer < 0 || layer >= n_layers)
    return fail(WI_E_INVALID, "layer %d outside [0, n_layers = %d)", layer, n_layers);
  if (n_ctx < 1 || seg_len < 1 || clusters_per_seg < 1)
    return fail(WI_E_INVALID, "n_ctx, seg_len and clusters_per_seg must be >= 1");
  bool dense, upper;
  switch (policy) {
    case WI_POLICY_UNIFORM: dense = false; upper = false; break;
    case WI_POLICY_DENSE_FIRST2: dense = layer < 2; upper = false; break;
    case WI_POLICY_BANDED:
      dense = 80ll * layer < 21ll * n_layers;
      upper = 80ll * layer >= 61ll * n_layers;
      break;
    default: return fail(WI_E_INVALID, "unknown policy %d", policy);
  }
  // a token share f is f * n_ctx * clusters_per_seg / seg_len clusters, rounded half up
  auto clusters = [&](double f) {
    return (int32_t)std::floor(f * (double)n_ctx * (double)clusters_per_seg / (double)seg_len + 0.5);
  };
  if (mode) *mode = dense ? WI_LAYER_DENSE : WI_LAYER_HYBRID;
  if (k_retrieve) *k_retrieve = dense ? 0 : clusters(0.018);
  if (k_estimate) *k_estimate = dense ? 0 : clusters(upper ? 0.30 : 0.23);
  g_err[0] = 0;
  return WI_OK;
}

}  // extern "C"

namespace {

// Shapes of a dense call: the K/V layout fields of the index descriptor and
// the head mapping of the decode descriptor.
struct DenseShape {
  int dtype, B, H, U, Hq, G;
  int64_t N, sb, sh, st;
  float scale;
  int W;
};

wi_status make_dense(const wi_index_desc* d, const wi_decode_desc* dd, DenseShape* o) {
  if (!d || !dd) return fail(WI_E_INVALID, "descriptor is NULL");
  if (d->dtype != WI_F32 && d->dtype != WI_BF16)
    return fail(WI_E_UNSUPPORTED, "unknown dtype %d", d->dtype);
  if (d->head_dim != wi::D) return fail(WI_E_UNSUPPORTED, "head_dim %d != 128", d->head_dim);
  if (d->batch < 1 || d->n_kv_heads < 1)
    return fail(WI_E_INVALID, "batch %d / n_kv_heads %d must be >= 1", d->batch, d->n_kv_heads);
  if (d->n_ctx < 1 || d->n_ctx >= (int64_t(1) << 31))
    return fail(WI_E_INVALID, "n_ctx %lld outside [1, 2^31)", (long long)d->n_ctx);
  if (d->kv_stride_t <= 0 || d->kv_stride_h < 0 || d->kv_stride_b < 0 ||
      d->kv_stride_t % 8 || d->kv_stride_h % 8 || d->kv_stride_b % 8)
    return fail(WI_E_INVALID, "K/V strides must be non-negative multiples of 8 (t > 0)");
  if (dd->n_q_heads < 1 || dd->n_q_heads % d->n_kv_heads)
    return fail(WI_E_UNSUPPORTED, "n_q_heads %d is not a multiple of n_kv_heads %d",
                dd->n_q_heads, d->n_kv_heads);
  const int G = dd->n_q_heads / d->n_kv_heads;
  if (G > wi::MAX_G) return fail(WI_E_UNSUPPORTED, "%d query heads per KV head > %d", G, wi::MAX_G);
  if (!(dd->scale >= 0.f) || !std::isfinite(dd->scale))
    return fail(WI_E_INVALID, "scale must be finite and >= 0");
  o->dtype = d->dtype;
  o->B = d->batch;
  o->H = d->n_kv_heads;
  o->U = d->batch * d->n_kv_heads;
  o->Hq = dd->n_q_heads;
  o->G = G;
  o->N = d->n_ctx;
  o->sb = d->kv_stride_b;
  o->sh = d->kv_stride_h;
  o->st = d->kv_stride_t;
  o->scale = dd->scale > 0.f ? dd->scale : 1.f / std::sqrt((float)wi::D);
  o->W = wi::dense_chunks(o->U, o->N);
  return WI_OK;
}

int64_t recall_ws_bytes(const wi::Geom& g, int G) {
  return align256((int64_t)g.U * G * g.cap * g.T * 8);
}

}  // namespace

extern "C" {

wi_status wi_dense_sizes(const wi_index_desc* desc, const wi_decode_desc* ddesc,
                         size_t* workspace_bytes) {
  DenseShape ds;
  wi_status st = make_dense(desc, ddesc, &ds);
  if (st != WI_OK) return st;
  if (workspace_bytes)
    *workspace_bytes = (size_t)align256(wi::dense_part_floats(ds.U, ds.W, ds.G) * 4);
  g_err[0] = 0;
  return WI_OK;
}

wi_status wi_dense_attention(const wi_index_desc* desc, const wi_decode_desc* ddesc,
                             const void* k, const void* v, const void* q, float* out, void* ws,
                             size_t ws_bytes, hipStream_t stream) {
  DenseShape ds;
  wi_status st = make_dense(desc, ddesc, &ds);
  if (st != WI_OK) return st;
  CHECK_PTR(k, "k");
  CHECK_PTR(v, "v");
  CHECK_PTR(q, "q");
  CHECK_PTR(out, "out");
  const int64_t need = align256(wi::dense_part_floats(ds.U, ds.W, ds.G) * 4);
  if (!ws || (int64_t)ws_bytes < need)
    return fail(WI_E_WORKSPACE, "workspace %zu bytes < %lld required", ws_bytes, (long long)need);
  if (!aligned16(ws)) return fail(WI_E_INVALID, "ws is not 16-byte aligned");
  CHECK_HIP(wi::launch_dense(ds.dtype, ds.B, ds.H, ds.Hq, ds.G, ds.N, ds.sb, ds.sh, ds.st,
                             ds.scale, k, v, q, out, reinterpret_cast<float*>(ws), stream),
            "dense attention");
  g_err[0] = 0;
  return WI_OK;
}

}  // extern "C"

namespace {

// Device-visible address of a host-memory range of `bytes` bytes (pinned,
// mapped): both ends must resolve to host memory of one mapping.
wi_status host_range(const void* p, int64_t bytes, const char* name, const void** dev) {
  if (!p) return fail(WI_E_INVALID, "%s is NULL", name);
  if (!aligned16(p)) return fail(WI_E_INVALID, "%s is not 16-byte aligned", name);
  hipPointerAttribute_t a0, a1;
  if (hipPointerGetAttributes(&a0, p) != hipSuccess || a0.type != hipMemoryTypeHost ||
      !a0.devicePointer) {
    (void)hipGetLastError();
    return fail(WI_E_INVALID, "%s is not pinned host memory visible to the device", name);
  }
  const void* end = reinterpret_cast<const uint8_t*>(p) + (bytes - 1);
  if (hipPointerGetAttributes(&a1, end) != hipSuccess || a1.type != hipMemoryTypeHost ||
      reinterpret_cast<const uint8_t*>(a1.devicePointer) -
              reinterpret_cast<const uint8_t*>(a0.devicePointer) != bytes - 1) {
    (void)hipGetLastError();
    return fail(WI_E_INVALID, "%s: the pinned host allocation is smaller than the block pool",
                name);
  }
  *dev = a0.devicePointer;
  return WI_OK;
}

// Decode workspace, then the update path's lists: needed/missed blocks
// [U][2 cap], admitted (block, slot) pairs [U][2 S], counts [U][4].
int64_t wb_ws_bytes(const wi::Geom& g, const DecodeShape& ds, int S) {
  return carve_decode(g, ds, nullptr, nullptr) + align256((int64_t)g.U * 2 * g.cap * 4) +
         align256((int64_t)g.U * 2 * S * 4) + align256((int64_t)g.U * 4 * 4);
}

wi_status check_wb(const wi::Geom& g, const wi_wave_buffer* wb) {
  if (!wb) return fail(WI_E_INVALID, "wave buffer is NULL");
  if (wb->n_slots < 1 || wb->n_slots > wi::wb_max_slots())
    return fail(WI_E_INVALID, "n_slots %d outside [1, %d]", wb->n_slots, wi::wb_max_slots());
  CHECK_PTR(wb->block_slot, "wb->block_slot");
  CHECK_PTR(wb->slot_block, "wb->slot_block");
  CHECK_PTR(wb->slot_last, "wb->slot_last");
  CHECK_PTR(wb->slot_order, "wb->slot_order");
  CHECK_PTR(wb->cache_k, "wb->cache_k");
  CHECK_PTR(wb->cache_v, "wb->cache_v");
  (void)g;
  return WI_OK;
}

}  // namespace

extern "C" {

wi_status wi_wave_buffer_reset(const wi_index_desc* desc, const wi_wave_buffer* wb,
                               hipStream_t stream) {
  wi::Geom g;
  wi_status st = make_geom(desc, &g);
  if (st != WI_OK) return st;
  st = check_wb(g, wb);
  if (st != WI_OK) return st;
  wi::WaveBufArgs w{wb->n_slots, wb->block_slot, wb->slot_block, wb->slot_last,
                    wb->slot_order, wb->cache_k, wb->cache_v, nullptr, nullptr};
  CHECK_HIP(wi::launch_wb_reset(g, w, stream), "wave buffer reset");
  g_err[0] = 0;
  return WI_OK;
}

wi_status wi_decode_wb_sizes(const wi_index_desc* desc, const wi_decode_desc* ddesc,
                             int32_t n_slots, size_t* workspace_bytes) {
  wi::Geom g;
  wi_status st = make_geom(desc, &g);
  if (st != WI_OK) return st;
  DecodeShape ds;
  st = make_decode(g, ddesc, &ds);
  if (st != WI_OK) return st;
  if (n_slots < 1 || n_slots > wi::wb_max_slots())
    return fail(WI_E_INVALID, "n_slots %d outside [1, %d]", n_slots, wi::wb_max_slots());
  if (workspace_bytes) *workspace_bytes = (size_t)wb_ws_bytes(g, ds, n_slots);
  g_err[0] = 0;
  return WI_OK;
}

wi_status wi_decode_attention_wb(const wi_index_desc* desc, const wi_decode_desc* ddesc,
                                 const wi_index_bufs* bufs, const wi_wave_buffer* wb,
                                 uint32_t step, const void* q, float* out, int32_t* stats,
                                 void* ws, size_t ws_bytes, hipStream_t stream) {
  wi::Geom g;
  wi_status st = make_geom(desc, &g);
  if (st != WI_OK) return st;
  DecodeShape ds;
  st = make_decode(g, ddesc, &ds);
  if (st != WI_OK) return st;
  st = check_wb(g, wb);
  if (st != WI_OK) return st;
  if (step == 0) return fail(WI_E_INVALID, "step must be > 0");
  if (!bufs) return fail(WI_E_INVALID, "bufs is NULL");
  CHECK_PTR(bufs->centroids, "bufs->centroids");
  CHECK_PTR(bufs->cluster_size, "bufs->cluster_size");
  CHECK_PTR(bufs->value_sum, "bufs->value_sum");
  CHECK_PTR(bufs->block_off, "bufs->block_off");
  if (g.n_st > 0) {
    CHECK_PTR(bufs->steady_k, "bufs->steady_k");
    CHECK_PTR(bufs->steady_v, "bufs->steady_v");
  }
  if (g.n_pend > 0) {
    CHECK_PTR(bufs->pend_k, "bufs->pend_k");
    CHECK_PTR(bufs->pend_v, "bufs->pend_v");
  }
  CHECK_PTR(q, "q");
  CHECK_PTR(out, "out");
  if (stats && !aligned16(stats)) return fail(WI_E_INVALID, "stats is not 16-byte aligned");
  const int64_t pool = (int64_t)g.U * g.cap * g.T * wi::D * (g.dtype == WI_BF16 ? 2 : 4);
  const void *hk = nullptr, *hv = nullptr;
  st = host_range(bufs->k_blocks, pool, "bufs->k_blocks", &hk);
  if (st != WI_OK) return st;
  st = host_range(bufs->v_blocks, pool, "bufs->v_blocks", &hv);
  if (st != WI_OK) return st;
  const int64_t need = wb_ws_bytes(g, ds, wb->n_slots);
  if (!ws || (int64_t)ws_bytes < need)
    return fail(WI_E_WORKSPACE, "workspace %zu bytes < %lld required", ws_bytes, (long long)need);
  if (!aligned16(ws)) return fail(WI_E_INVALID, "ws is not 16-byte aligned");
  uint8_t* base = reinterpret_cast<uint8_t*>(ws);
  wi::DecodeWs w;
  int64_t off = carve_decode(g, ds, base, &w);
  int32_t* lists = reinterpret_cast<int32_t*>(base + off);
  off += align256((int64_t)g.U * 2 * g.cap * 4);
  int32_t* fill = reinterpret_cast<int32_t*>(base + off);
  off += align256((int64_t)g.U * 2 * wb->n_slots * 4);
  int32_t* counts = reinterpret_cast<int32_t*>(base + off);
  wi::WaveBufArgs wa{wb->n_slots, wb->block_slot, wb->slot_block, wb->slot_last,
                     wb->slot_order, wb->cache_k, wb->cache_v, hk, hv};
  wi::DecodeArgs a{&g, ds.Hq, ds.G, ds.GS, ds.K_r, ds.K_e, ds.W, ds.scale};
  CHECK_HIP(wi::launch_score(a, bufs->centroids, q, w, stream), "score");
  CHECK_HIP(wi::launch_fused(a, *bufs, q, out, w, true, stream, &wa), "select/attend");
  CHECK_HIP(wi::launch_wb_update(g, wa, bufs->cluster_size, bufs->block_off, w.zone, step,
                                 lists, fill, counts, stats, stream),
            "wave buffer update");
  g_err[0] = 0;
  return WI_OK;
}

wi_status wi_recall_sizes(const wi_index_desc* desc, const wi_decode_desc* ddesc,
                          size_t* workspace_bytes) {
  wi::Geom g;
  wi_status st = make_geom(desc, &g);
  if (st != WI_OK) return st;
  if (!ddesc) return fail(WI_E_INVALID, "decode desc is NULL");
  if (ddesc->n_q_heads < 1 || ddesc->n_q_heads % g.H)
    return fail(WI_E_UNSUPPORTED, "n_q_heads %d is not a multiple of n_kv_heads %d",
                ddesc->n_q_heads, g.H);
  const int G = ddesc->n_q_heads / g.H;
  if (G > wi::MAX_G) return fail(WI_E_UNSUPPORTED, "%d query heads per KV head > %d", G, wi::MAX_G);
  if (workspace_bytes) *workspace_bytes = (size_t)recall_ws_bytes(g, G);
  g_err[0] = 0;
  return WI_OK;
}

wi_status wi_recall_at_k(const wi_index_desc* desc, const wi_decode_desc* ddesc,
                         const wi_index_bufs* bufs, const void* q, const int32_t* sel_ids,
                         int32_t sel_stride, int32_t n_r, int32_t k, float* recall,
                         int32_t* top_tokens, void* ws, size_t ws_bytes, hipStream_t stream) {
  wi::Geom g;
  wi_status st = make_geom(desc, &g);
  if (st != WI_OK) return st;
  size_t need = 0;
  st = wi_recall_sizes(desc, ddesc, &need);
  if (st != WI_OK) return st;
  const int G = ddesc->n_q_heads / g.H;
  if (k < 1 || k > wi::recall_max_k() || (int64_t)k > g.n_idx)
    return fail(WI_E_INVALID, "k %d outside [1, min(%d, clustered tokens %lld)]", k,
                wi::recall_max_k(), (long long)g.n_idx);
  if (n_r < 0 || n_r > g.C) return fail(WI_E_INVALID, "n_r %d outside [0, C = %d]", n_r, g.C);
  if (sel_stride < n_r) return fail(WI_E_INVALID, "sel_stride %d < n_r %d", sel_stride, n_r);
  if (n_r > 0) CHECK_PTR(sel_ids, "sel_ids");
  if (!bufs) return fail(WI_E_INVALID, "bufs is NULL");
  CHECK_PTR(bufs->block_off, "bufs->block_off");
  CHECK_PTR(bufs->k_blocks, "bufs->k_blocks");
  CHECK_PTR(bufs->slot_token, "bufs->slot_token");
  CHECK_PTR(bufs->assign, "bufs->assign");
  CHECK_PTR(q, "q");
  CHECK_PTR(recall, "recall");
  if (top_tokens && !aligned16(top_tokens))
    return fail(WI_E_INVALID, "top_tokens is not 16-byte aligned");
  if (!ws || ws_bytes < need)
    return fail(WI_E_WORKSPACE, "workspace %zu bytes < %zu required", ws_bytes, need);
  if (!aligned16(ws)) return fail(WI_E_INVALID, "ws is not 16-byte aligned");
  CHECK_HIP(wi::launch_recall(g, ddesc->n_q_heads, G, *bufs, q, sel_ids, sel_stride, n_r, k,
                              recall, top_tokens, reinterpret_cast<uint64_t*>(ws), stream),
            "recall");
  g_err[0] = 0;
  return WI_OK;
}

}  // extern "C"
