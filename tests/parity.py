"""Comparison helpers shared by the GPU parity tests (no method arithmetic)."""
from __future__ import annotations

import numpy as np
import torch

import oracle
from sparse_long_context_segmented_amd import synth, wi


def to_np(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.detach().cpu().numpy()


def upload_kv(K: np.ndarray, V: np.ndarray, dtype: str, device="cuda"):
    dt = torch.float32 if dtype == "f32" else torch.bfloat16
    return (torch.from_numpy(K).to(device=device, dtype=dt).contiguous(),
            torch.from_numpy(V).to(device=device, dtype=dt).contiguous())


def upload_q(q: np.ndarray, dtype: str, device="cuda"):
    dt = torch.float32 if dtype == "f32" else torch.bfloat16
    return torch.from_numpy(q).to(device=device, dtype=dt).contiguous()


def rel_err(out: np.ndarray, ref: np.ndarray) -> float:
    """max over query heads of max_t |o - r| / max_t |r|."""
    o = out.reshape(-1, out.shape[-1]).astype(np.float64)
    r = ref.reshape(-1, ref.shape[-1]).astype(np.float64)
    num = np.abs(o - r).max(axis=1)
    den = np.abs(r).max(axis=1)
    return float((num / den).max())


def near_tie(a: float, b: float) -> bool:
    """Ranking keys within the 1e-5 relative window (logit units, floor 1)."""
    return abs(a - b) <= 1e-5 * max(abs(a), abs(b), 1.0)


def check_selection(sel_gpu: np.ndarray, gkey: np.ndarray, k_r: int) -> int:
    """Compare a selection (rank order) with the exact group scores.

    The oracle ranks on the exact (float64) group score, larger first, lower
    id on equal scores. The GPU ranks on that score rounded to float32, so two
    clusters whose scores round alike go by id there. Every position where the
    GPU order differs from the exact ranking must pair two clusters whose exact
    scores are a near-tie (within 1e-5 relative); the number of such positions
    is returned (and printed by the callers). The selected ids must be
    distinct, and the retrieval and estimation sets may differ from the exact
    ones only by near-tied swaps across their boundaries.
    """
    U, M = sel_gpu.shape
    mism = 0
    for u in range(U):
        key = gkey[u].astype(np.float64)
        order = np.lexsort((np.arange(len(key)), -key))[:M]
        assert len(set(sel_gpu[u].tolist())) == M, f"unit {u}: repeated ids"
        if np.array_equal(order, sel_gpu[u]):
            continue
        diff = np.nonzero(order != sel_gpu[u])[0]
        mism += len(diff)
        for i in diff:
            a, b = key[order[i]], key[sel_gpu[u][i]]
            assert near_tie(a, b), (u, int(i), float(a), float(b))
    return mism


def exec_reference(idx: dict, sel: np.ndarray, k_r: int, n_ctx: int, T: int, n_sink=4,
                   n_local=64, n_pending=0):
    """Execution-buffer tokens implied by a selection and an index: steady
    positions, pending positions (just before the local window), then the
    retrieved clusters' members in rank order."""
    res = []
    p0 = n_ctx - n_local - n_pending
    for u in range(sel.shape[0]):
        bo, sz, st = idx["block_off"][u], idx["sizes"][u], idx["slot_token"][u]
        toks = list(range(n_sink)) + list(range(n_ctx - n_local, n_ctx))
        toks += list(range(p0, p0 + n_pending))
        for c in sel[u][:k_r]:
            toks.extend(st[bo[c] * T: bo[c] * T + sz[c]].tolist())
        res.append(toks)
    return res


def index_to_host(ix: wi.Index, units=None) -> dict:
    """Index arrays on the host, [U, ...]; with units, only those units (in
    the order given)."""
    pick = (lambda t: t) if units is None else (lambda t: t[list(units)])  # noqa: E731
    out = dict(centroids=to_np(pick(ix.centroids)), sizes=to_np(pick(ix.cluster_size)),
               vsum=to_np(pick(ix.value_sum)), block_off=to_np(pick(ix.block_off)),
               kblk=to_np(pick(ix.k_blocks)), vblk=to_np(pick(ix.v_blocks)),
               slot_token=to_np(pick(ix.slot_token)), steady_k=to_np(pick(ix.steady_k)),
               steady_v=to_np(pick(ix.steady_v)), assign=to_np(pick(ix.assign)))
    if ix.pend_k is not None:
        out["pend_k"] = to_np(pick(ix.pend_k))
        out["pend_v"] = to_np(pick(ix.pend_v))
    return out


def assert_index_equal(got: dict, ref: dict, units=None, n_st=68):
    """Bit-exact comparison of every index array (optionally on some units)."""
    sel = slice(None) if units is None else list(units)
    for key in ("sizes", "block_off", "slot_token", "assign"):
        a, b = got[key][sel], ref[key][sel]
        assert np.array_equal(a, b), f"{key}: {int((a != b).sum())} differences"
    for key in ("centroids", "vsum", "kblk", "vblk"):
        a = np.ascontiguousarray(got[key][sel], dtype=np.float32)
        b = np.ascontiguousarray(ref[key][sel], dtype=np.float32)
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), \
            f"{key}: {int((a.view(np.uint32) != b.view(np.uint32)).sum())} differences"
    for key in ("steady_k", "steady_v"):
        a = np.ascontiguousarray(got[key][sel], dtype=np.float32)[:, :n_st]
        b = np.ascontiguousarray(ref[key][sel], dtype=np.float32)[:, :n_st]
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), key


def descs(w: synth.Workload, layer: int = 0, n_iters=None, batch=None, heads=None):
    """Matching (GPU, oracle) descriptors of a workload."""
    it = w.n_iters if n_iters is None else n_iters
    B = w.batch if batch is None else batch
    H = w.n_kv_heads if heads is None else heads
    gd = wi.make_desc(w.dtype, B, H, w.n_ctx, seg_len=w.seg_len,
                      clusters_per_seg=w.clusters_per_seg, n_iters=it, layer_id=layer)
    od = oracle.make_desc(w.dtype, B, H, w.n_ctx, seg_len=w.seg_len,
                          clusters_per_seg=w.clusters_per_seg, n_iters=it, layer_id=layer)
    return gd, od
