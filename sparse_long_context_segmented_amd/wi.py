"""ctypes binding of libwi.so (C ABI in include/wi.h).

Argument marshalling only: every step of the build and the decode runs in the
library's HIP kernels. torch provides device memory and the stream. The
library must be built (``python -m sparse_long_context_segmented_amd._build``
or ``__graft_entry__.build()``); loading fails loudly if it is missing.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libwi.so")

WI_F32, WI_BF16 = 0, 1
WI_LAYER_DENSE, WI_LAYER_HYBRID = 0, 1
WI_POLICY_UNIFORM, WI_POLICY_DENSE_FIRST2, WI_POLICY_BANDED = 0, 1, 2
STATUS = {0: "WI_OK", 1: "WI_E_INVALID", 2: "WI_E_UNSUPPORTED", 3: "WI_E_WORKSPACE",
          4: "WI_E_HIP"}
EXPORTS = ("wi_index_sizes", "wi_build_index", "wi_decode_sizes", "wi_decode_attention",
           "wi_decode_attention_noalloc", "wi_append_token", "wi_append_sizes",
           "wi_append_tokens", "wi_extend_sizes",
           "wi_extend_index", "wi_layer_plan", "wi_dense_sizes", "wi_dense_attention",
           "wi_recall_sizes", "wi_recall_at_k", "wi_wave_buffer_reset", "wi_decode_wb_sizes",
           "wi_decode_attention_wb", "wi_status_str", "wi_last_error",
           "wi_timing_start", "wi_timing_stop", "wi_kernel_name")
NOALLOC_SCRATCH_BYTES = 16 << 20


class WIError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS.get(status, status)}: {msg}")
        self.status = status


class IndexDesc(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int32), ("batch", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("n_ctx", ctypes.c_int64), ("seg_len", ctypes.c_int32),
                ("clusters_per_seg", ctypes.c_int32), ("n_sink", ctypes.c_int32),
                ("n_local", ctypes.c_int32), ("n_iters", ctypes.c_int32),
                ("seed", ctypes.c_uint64), ("layer_id", ctypes.c_uint32),
                ("kv_stride_b", ctypes.c_int64), ("kv_stride_h", ctypes.c_int64),
                ("kv_stride_t", ctypes.c_int64), ("n_pending", ctypes.c_int64)]


class IndexBufs(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "centroids", "cluster_size", "value_sum", "block_off", "k_blocks", "v_blocks",
        "slot_token", "steady_k", "steady_v", "assign", "pend_k", "pend_v")]


class WaveBufferDesc(ctypes.Structure):
    _fields_ = [("n_slots", ctypes.c_int32), ("block_slot", ctypes.c_void_p),
                ("slot_block", ctypes.c_void_p), ("slot_last", ctypes.c_void_p),
                ("cache_k", ctypes.c_void_p), ("cache_v", ctypes.c_void_p),
                ("slot_order", ctypes.c_void_p)]


class DecodeDesc(ctypes.Structure):
    _fields_ = [("n_q_heads", ctypes.c_int32), ("k_retrieve", ctypes.c_int32),
                ("k_estimate", ctypes.c_int32), ("scale", ctypes.c_float),
                ("wg_per_unit", ctypes.c_int32)]


_lib = None


def lib():
    """Load libwi.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m sparse_long_context_segmented_amd._build`")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.c_void_p
        L.wi_index_sizes.argtypes = [P, P, P, P, P]
        L.wi_index_sizes.restype = ctypes.c_int
        L.wi_build_index.argtypes = [P, P, P, P, P, P, ctypes.c_size_t, P]
        L.wi_build_index.restype = ctypes.c_int
        L.wi_decode_sizes.argtypes = [P, P, P]
        L.wi_decode_sizes.restype = ctypes.c_int
        L.wi_decode_attention.argtypes = [P, P, P, P, P, P, P, P, ctypes.c_int64, P,
                                          ctypes.c_size_t, P]
        L.wi_decode_attention.restype = ctypes.c_int
        L.wi_decode_attention_noalloc.argtypes = [P, P, P, P, P, P, P, P, ctypes.c_int64, P]
        L.wi_decode_attention_noalloc.restype = ctypes.c_int
        L.wi_append_token.argtypes = [P, P, P, P, P]
        L.wi_append_token.restype = ctypes.c_int
        L.wi_append_sizes.argtypes = [P, P]
        L.wi_append_sizes.restype = ctypes.c_int
        L.wi_append_tokens.argtypes = [P, P, P, P, ctypes.c_int32, P, ctypes.c_size_t, P]
        L.wi_append_tokens.restype = ctypes.c_int
        L.wi_extend_sizes.argtypes = [P, P]
        L.wi_extend_sizes.restype = ctypes.c_int
        L.wi_extend_index.argtypes = [P, P, P, P, ctypes.c_size_t, P]
        L.wi_extend_index.restype = ctypes.c_int
        i32 = ctypes.c_int32
        L.wi_layer_plan.argtypes = [i32, i32, i32, ctypes.c_int64, i32, i32, P, P, P]
        L.wi_layer_plan.restype = ctypes.c_int
        L.wi_dense_sizes.argtypes = [P, P, P]
        L.wi_dense_sizes.restype = ctypes.c_int
        L.wi_dense_attention.argtypes = [P, P, P, P, P, P, P, ctypes.c_size_t, P]
        L.wi_dense_attention.restype = ctypes.c_int
        L.wi_recall_sizes.argtypes = [P, P, P]
        L.wi_recall_sizes.restype = ctypes.c_int
        L.wi_recall_at_k.argtypes = [P, P, P, P, P, i32, i32, i32, P, P, P, ctypes.c_size_t, P]
        L.wi_recall_at_k.restype = ctypes.c_int
        L.wi_wave_buffer_reset.argtypes = [P, P, P]
        L.wi_wave_buffer_reset.restype = ctypes.c_int
        L.wi_decode_wb_sizes.argtypes = [P, P, i32, P]
        L.wi_decode_wb_sizes.restype = ctypes.c_int
        L.wi_decode_attention_wb.argtypes = [P, P, P, P, ctypes.c_uint32, P, P, P, P,
                                             ctypes.c_size_t, P]
        L.wi_decode_attention_wb.restype = ctypes.c_int
        L.wi_status_str.argtypes = [ctypes.c_int]
        L.wi_status_str.restype = ctypes.c_char_p
        L.wi_last_error.argtypes = []
        L.wi_last_error.restype = ctypes.c_char_p
        L.wi_timing_start.argtypes = []
        L.wi_timing_start.restype = ctypes.c_int
        L.wi_timing_stop.argtypes = [ctypes.c_int32, P, P]
        L.wi_timing_stop.restype = ctypes.c_int32
        L.wi_kernel_name.argtypes = [ctypes.c_int32]
        L.wi_kernel_name.restype = ctypes.c_char_p
        _lib = L
    return _lib


def _check(rc: int):
    if rc != 0:
        raise WIError(rc, lib().wi_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def make_desc(dtype: str, batch: int, n_kv_heads: int, n_ctx: int, seg_len: int = 8192,
              clusters_per_seg: int = 512, n_sink: int = 4, n_local: int = 64,
              n_iters: int = 10, seed: int = 0, layer_id: int = 0,
              strides=None) -> IndexDesc:
    """Descriptor; strides default to a contiguous [B, H, N, 128] K/V."""
    if strides is None:
        strides = (n_kv_heads * n_ctx * 128, n_ctx * 128, 128)
    return IndexDesc(WI_F32 if dtype == "f32" else WI_BF16, batch, n_kv_heads, 128, n_ctx,
                     seg_len, clusters_per_seg, n_sink, n_local, n_iters, seed, layer_id,
                     *strides)


def index_sizes(desc: IndexDesc):
    ns, c, cap = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
    ws = ctypes.c_size_t()
    _check(lib().wi_index_sizes(ctypes.byref(desc), ctypes.byref(ns), ctypes.byref(c),
                                ctypes.byref(cap), ctypes.byref(ws)))
    return ns.value, c.value, cap.value, ws.value


def torch_dtype(desc: IndexDesc):
    return torch.float32 if desc.dtype == WI_F32 else torch.bfloat16


@dataclass
class Index:
    """Device tensors of a built index (all owned by torch)."""
    desc: IndexDesc
    centroids: torch.Tensor
    cluster_size: torch.Tensor
    value_sum: torch.Tensor
    block_off: torch.Tensor
    k_blocks: torch.Tensor
    v_blocks: torch.Tensor
    slot_token: torch.Tensor
    steady_k: torch.Tensor
    steady_v: torch.Tensor
    assign: torch.Tensor
    pend_k: torch.Tensor | None = None   # [U, seg_len, 128]: pending rows (decode-time growth)
    pend_v: torch.Tensor | None = None

    def bufs(self) -> IndexBufs:
        return IndexBufs(*[_ptr(getattr(self, n)) for n, _ in IndexBufs._fields_])


def alloc_index(desc: IndexDesc, device="cuda", pending=None) -> Index:
    """Buffers of an index for desc; pending: (pend_k, pend_v) to reuse, True
    to allocate new pending rows, None for none."""
    ns, C, cap, _ = index_sizes(desc)
    U = desc.batch * desc.n_kv_heads
    T = 2048 // (128 * (4 if desc.dtype == WI_F32 else 2))
    dt = torch_dtype(desc)
    n_idx = desc.n_ctx - desc.n_sink - desc.n_local - desc.n_pending
    n_st = desc.n_sink + desc.n_local
    e = lambda *s, dtype=dt: torch.empty(*s, dtype=dtype, device=device)  # noqa: E731
    pk = pv = None
    if pending is True:
        pk, pv = e(U, desc.seg_len, 128), e(U, desc.seg_len, 128)
    elif pending is not None:
        pk, pv = pending
    return Index(desc, e(U, C, 128), e(U, C, dtype=torch.int32), e(U, C, 128, dtype=torch.float32),
                 e(U, C + 1, dtype=torch.int32), e(U, cap * T, 128), e(U, cap * T, 128),
                 e(U, cap * T, dtype=torch.int32), e(U, max(n_st, 1), 128),
                 e(U, max(n_st, 1), 128), e(U, n_idx, dtype=torch.int32), pk, pv)


def index_from_host(desc: IndexDesc, arrays: dict, device="cuda") -> Index:
    """Upload an index given as host arrays (keys as in the oracle's output)."""
    dt = torch_dtype(desc)
    t = lambda a, dtype=dt: torch.as_tensor(a).to(device=device, dtype=dtype).contiguous()  # noqa: E731
    pk = t(arrays["pend_k"]) if "pend_k" in arrays else None
    pv = t(arrays["pend_v"]) if "pend_v" in arrays else None
    return Index(desc, t(arrays["centroids"]), t(arrays["sizes"], torch.int32),
                 t(arrays["vsum"], torch.float32), t(arrays["block_off"], torch.int32),
                 t(arrays["kblk"]), t(arrays["vblk"]), t(arrays["slot_token"], torch.int32),
                 t(arrays["steady_k"]), t(arrays["steady_v"]), t(arrays["assign"], torch.int32),
                 pk, pv)


def build_index(desc: IndexDesc, k: torch.Tensor, v: torch.Tensor,
                init: torch.Tensor | None = None, index: Index | None = None,
                ws: torch.Tensor | None = None, stream=None) -> Index:
    """Run wi_build_index on device tensors k, v laid out as desc's strides say."""
    _, _, _, wsb = index_sizes(desc)
    if index is None:
        index = alloc_index(desc, k.device)
    if ws is None or ws.numel() < wsb:
        ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device=k.device)
    bufs = index.bufs()
    _check(lib().wi_build_index(ctypes.byref(desc), _ptr(k), _ptr(v), _ptr(init),
                                ctypes.byref(bufs), _ptr(ws), ws.numel(), _stream(stream)))
    return index


def decode_sizes(desc: IndexDesc, ddesc: DecodeDesc) -> int:
    ws = ctypes.c_size_t()
    _check(lib().wi_decode_sizes(ctypes.byref(desc), ctypes.byref(ddesc), ctypes.byref(ws)))
    return ws.value


def decode_attention(index: Index, ddesc: DecodeDesc, q: torch.Tensor,
                     out: torch.Tensor | None = None, sel_ids: torch.Tensor | None = None,
                     exec_tokens: torch.Tensor | None = None,
                     n_exec: torch.Tensor | None = None, ws: torch.Tensor | None = None,
                     stream=None) -> torch.Tensor:
    """Run wi_decode_attention; returns out [B, Hq, 128] float32."""
    desc = index.desc
    wsb = decode_sizes(desc, ddesc)
    if out is None:
        out = torch.empty(desc.batch, ddesc.n_q_heads, 128, dtype=torch.float32, device=q.device)
    if ws is None or ws.numel() < wsb:
        ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device=q.device)
    bufs = index.bufs()
    exec_cap = 0 if exec_tokens is None else exec_tokens.shape[-1]
    _check(lib().wi_decode_attention(ctypes.byref(desc), ctypes.byref(ddesc), ctypes.byref(bufs),
                                     _ptr(q), _ptr(out), _ptr(sel_ids), _ptr(exec_tokens),
                                     _ptr(n_exec), exec_cap, _ptr(ws), ws.numel(),
                                     _stream(stream)))
    return out


def decode_attention_noalloc(index: Index, ddesc: DecodeDesc, q: torch.Tensor, out: torch.Tensor,
                             sel_ids: torch.Tensor | None = None,
                             exec_tokens: torch.Tensor | None = None,
                             n_exec: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Run wi_decode_attention_noalloc: the caller passes every output; the
    library's own static device scratch stands in for the workspace."""
    bufs = index.bufs()
    exec_cap = 0 if exec_tokens is None else exec_tokens.shape[-1]
    _check(lib().wi_decode_attention_noalloc(
        ctypes.byref(index.desc), ctypes.byref(ddesc), ctypes.byref(bufs), _ptr(q), _ptr(out),
        _ptr(sel_ids), _ptr(exec_tokens), _ptr(n_exec), exec_cap, _stream(stream)))
    return out


def _copy_desc(desc: IndexDesc) -> IndexDesc:
    return IndexDesc.from_buffer_copy(desc)


def append_token(index: Index, k_new: torch.Tensor, v_new: torch.Tensor, stream=None) -> Index:
    """Run wi_append_token (k_new, v_new [B, H, 128]): slides the local window
    of index in place and pends the departing token. Returns the same buffers
    under the grown descriptor (n_ctx + 1, n_pending + 1); pending rows are
    allocated on first use."""
    desc = index.desc
    U = desc.batch * desc.n_kv_heads
    if index.pend_k is None:
        dt = torch_dtype(desc)
        index.pend_k = torch.empty(U, desc.seg_len, 128, dtype=dt, device=k_new.device)
        index.pend_v = torch.empty(U, desc.seg_len, 128, dtype=dt, device=k_new.device)
    bufs = index.bufs()
    _check(lib().wi_append_token(ctypes.byref(desc), ctypes.byref(bufs), _ptr(k_new), _ptr(v_new),
                                 _stream(stream)))
    nd = _copy_desc(desc)
    nd.n_ctx += 1
    nd.n_pending += 1
    index.desc = nd
    return index


def append_tokens(index: Index, k_new: torch.Tensor, v_new: torch.Tensor, ws=None,
                  stream=None) -> Index:
    """Run wi_append_tokens (k_new, v_new [B, H, n, 128] contiguous, n <=
    seg_len - n_pending); returns the same buffers under the grown
    descriptor."""
    desc = index.desc
    U = desc.batch * desc.n_kv_heads
    n = k_new.shape[2]
    if index.pend_k is None:
        dt = torch_dtype(desc)
        index.pend_k = torch.empty(U, desc.seg_len, 128, dtype=dt, device=k_new.device)
        index.pend_v = torch.empty(U, desc.seg_len, 128, dtype=dt, device=k_new.device)
    need = ctypes.c_size_t()
    _check(lib().wi_append_sizes(ctypes.byref(desc), ctypes.byref(need)))
    if ws is None or ws.numel() < need.value:
        ws = torch.empty(max(need.value, 16), dtype=torch.uint8, device=k_new.device)
    bufs = index.bufs()
    _check(lib().wi_append_tokens(ctypes.byref(desc), ctypes.byref(bufs), _ptr(k_new),
                                  _ptr(v_new), n, _ptr(ws), ws.numel(), _stream(stream)))
    nd = _copy_desc(desc)
    nd.n_ctx += n
    nd.n_pending += n
    index.desc = nd
    return index


def prefill_chunk(index: Index, k_chunk: torch.Tensor, v_chunk: torch.Tensor,
                  stream=None) -> Index:
    """Feed a prefill chunk (k_chunk, v_chunk [B, H, n, 128]) into the index:
    appended in pieces that end at segment boundaries, each full pending
    segment clustered (wi_extend_index) as soon as it fills. Returns the
    (possibly new) index."""
    n = k_chunk.shape[2]
    i = 0
    while i < n:
        d = index.desc
        if d.n_pending == d.seg_len:
            index = extend_index(index, stream=stream)
            continue
        m = min(n - i, d.seg_len - d.n_pending)
        index = append_tokens(index, k_chunk[:, :, i:i + m].contiguous(),
                              v_chunk[:, :, i:i + m].contiguous(), stream=stream)
        i += m
    if index.desc.n_pending == index.desc.seg_len:
        index = extend_index(index, stream=stream)
    return index


def extend_sizes(desc: IndexDesc) -> int:
    ws = ctypes.c_size_t()
    _check(lib().wi_extend_sizes(ctypes.byref(desc), ctypes.byref(ws)))
    return ws.value


def extend_index(index: Index, ws: torch.Tensor | None = None, new: Index | None = None,
                 stream=None) -> Index:
    """Run wi_extend_index on an index whose pending segment is full: returns
    the grown index (n_pending = 0; it keeps the pending buffers)."""
    desc = index.desc
    nd = _copy_desc(desc)
    nd.n_pending = 0
    if new is None:
        new = alloc_index(nd, index.centroids.device, pending=(index.pend_k, index.pend_v))
    wsb = extend_sizes(desc)
    if ws is None or ws.numel() < wsb:
        ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device=index.centroids.device)
    ob, nb = index.bufs(), new.bufs()
    _check(lib().wi_extend_index(ctypes.byref(desc), ctypes.byref(ob), ctypes.byref(nb),
                                 _ptr(ws), ws.numel(), _stream(stream)))
    return new


def layer_plan(policy: int, layer: int, n_layers: int, n_ctx: int, seg_len: int = 8192,
               clusters_per_seg: int = 512):
    """(mode, k_retrieve, k_estimate) of one layer under a per-layer policy."""
    m, kr, ke = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
    _check(lib().wi_layer_plan(policy, layer, n_layers, n_ctx, seg_len, clusters_per_seg,
                               ctypes.byref(m), ctypes.byref(kr), ctypes.byref(ke)))
    return m.value, kr.value, ke.value


def dense_sizes(desc: IndexDesc, ddesc: DecodeDesc) -> int:
    ws = ctypes.c_size_t()
    _check(lib().wi_dense_sizes(ctypes.byref(desc), ctypes.byref(ddesc), ctypes.byref(ws)))
    return ws.value


def dense_attention(desc: IndexDesc, ddesc: DecodeDesc, k: torch.Tensor, v: torch.Tensor,
                    q: torch.Tensor, out: torch.Tensor | None = None,
                    ws: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Run wi_dense_attention (k, v laid out as desc's strides say); returns
    out [B, Hq, 128] float32."""
    wsb = dense_sizes(desc, ddesc)
    if out is None:
        out = torch.empty(desc.batch, ddesc.n_q_heads, 128, dtype=torch.float32, device=q.device)
    if ws is None or ws.numel() < wsb:
        ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device=q.device)
    _check(lib().wi_dense_attention(ctypes.byref(desc), ctypes.byref(ddesc), _ptr(k), _ptr(v),
                                    _ptr(q), _ptr(out), _ptr(ws), ws.numel(), _stream(stream)))
    return out


def recall_sizes(desc: IndexDesc, ddesc: DecodeDesc) -> int:
    ws = ctypes.c_size_t()
    _check(lib().wi_recall_sizes(ctypes.byref(desc), ctypes.byref(ddesc), ctypes.byref(ws)))
    return ws.value


def recall_at_k(index: Index, ddesc: DecodeDesc, q: torch.Tensor, sel_ids: torch.Tensor,
                n_r: int, k: int = 100, want_top: bool = False, ws: torch.Tensor | None = None,
                stream=None):
    """Run wi_recall_at_k on the retrieval zone sel_ids[:, :n_r] ([U, stride]);
    returns recall [B, Hq] float32 (and top [B, Hq, k] int32 with want_top)."""
    desc = index.desc
    wsb = recall_sizes(desc, ddesc)
    if ws is None or ws.numel() < wsb:
        ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device=q.device)
    rec = torch.empty(desc.batch, ddesc.n_q_heads, dtype=torch.float32, device=q.device)
    top = (torch.empty(desc.batch, ddesc.n_q_heads, k, dtype=torch.int32, device=q.device)
           if want_top else None)
    bufs = index.bufs()
    _check(lib().wi_recall_at_k(ctypes.byref(desc), ctypes.byref(ddesc), ctypes.byref(bufs),
                                _ptr(q), _ptr(sel_ids), sel_ids.shape[-1], n_r, k, _ptr(rec),
                                _ptr(top), _ptr(ws), ws.numel(), _stream(stream)))
    return (rec, top) if want_top else rec


@dataclass
class WaveBuffer:
    """GPU block cache and tables of the wave buffer (device tensors)."""
    n_slots: int
    block_slot: torch.Tensor   # [U, cap] int32
    slot_block: torch.Tensor   # [U, n_slots] int32
    slot_last: torch.Tensor    # [U, n_slots] int32 (uint32 values)
    cache_k: torch.Tensor      # [U, n_slots * T, 128]
    cache_v: torch.Tensor
    slot_order: torch.Tensor   # [U, n_slots] int32

    def desc(self) -> WaveBufferDesc:
        return WaveBufferDesc(self.n_slots, *[_ptr(t) for t in (
            self.block_slot, self.slot_block, self.slot_last, self.cache_k, self.cache_v,
            self.slot_order)])


def alloc_wave_buffer(desc: IndexDesc, n_slots: int, device="cuda", stream=None) -> WaveBuffer:
    """Allocate a wave buffer of n_slots blocks per unit and empty it."""
    ns, C, cap, _ = index_sizes(desc)
    U = desc.batch * desc.n_kv_heads
    T = 2048 // (128 * (4 if desc.dtype == WI_F32 else 2))
    dt = torch_dtype(desc)
    wb = WaveBuffer(n_slots, torch.empty(U, cap, dtype=torch.int32, device=device),
                    torch.empty(U, n_slots, dtype=torch.int32, device=device),
                    torch.empty(U, n_slots, dtype=torch.int32, device=device),
                    torch.empty(U, n_slots * T, 128, dtype=dt, device=device),
                    torch.empty(U, n_slots * T, 128, dtype=dt, device=device),
                    torch.empty(U, n_slots, dtype=torch.int32, device=device))
    wd = wb.desc()
    _check(lib().wi_wave_buffer_reset(ctypes.byref(desc), ctypes.byref(wd), _stream(stream)))
    return wb


def host_tier(index: Index) -> Index:
    """The same index with its K/V block pools moved to pinned host memory."""
    hk = torch.empty(index.k_blocks.shape, dtype=index.k_blocks.dtype, pin_memory=True)
    hv = torch.empty(index.v_blocks.shape, dtype=index.v_blocks.dtype, pin_memory=True)
    hk.copy_(index.k_blocks)
    hv.copy_(index.v_blocks)
    return Index(index.desc, index.centroids, index.cluster_size, index.value_sum,
                 index.block_off, hk, hv, index.slot_token, index.steady_k, index.steady_v,
                 index.assign, index.pend_k, index.pend_v)


def decode_wb_sizes(desc: IndexDesc, ddesc: DecodeDesc, n_slots: int) -> int:
    ws = ctypes.c_size_t()
    _check(lib().wi_decode_wb_sizes(ctypes.byref(desc), ctypes.byref(ddesc), n_slots,
                                    ctypes.byref(ws)))
    return ws.value


def decode_attention_wb(index: Index, ddesc: DecodeDesc, wb: WaveBuffer, step: int,
                        q: torch.Tensor, out: torch.Tensor | None = None,
                        stats: torch.Tensor | None = None, ws: torch.Tensor | None = None,
                        stream=None) -> torch.Tensor:
    """Run wi_decode_attention_wb (index from host_tier); returns out."""
    desc = index.desc
    wsb = decode_wb_sizes(desc, ddesc, wb.n_slots)
    if out is None:
        out = torch.empty(desc.batch, ddesc.n_q_heads, 128, dtype=torch.float32, device=q.device)
    if ws is None or ws.numel() < wsb:
        ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device=q.device)
    bufs = index.bufs()
    wd = wb.desc()
    _check(lib().wi_decode_attention_wb(ctypes.byref(desc), ctypes.byref(ddesc),
                                        ctypes.byref(bufs), ctypes.byref(wd), step, _ptr(q),
                                        _ptr(out), _ptr(stats), _ptr(ws), ws.numel(),
                                        _stream(stream)))
    return out


def timing_start():
    """Bracket every following kernel launch of this thread with HIP events."""
    _check(lib().wi_timing_start())


def timing_stop(max_records: int = 1 << 16):
    """Stop timing; returns a list of (kernel name, milliseconds) in issue order."""
    import numpy as np
    ids = np.zeros(max_records, np.int32)
    ms = np.zeros(max_records, np.float32)
    n = lib().wi_timing_stop(max_records, ids.ctypes.data, ms.ctypes.data)
    if n < 0:
        raise WIError(4, "timing events failed")
    n = min(n, max_records)
    return [(lib().wi_kernel_name(int(i)).decode(), float(t)) for i, t in zip(ids[:n], ms[:n])]
