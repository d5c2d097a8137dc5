"""C-ABI checks that need no GPU: the library loads, exports every symbol
include/wi.h declares, derives the same sizes as the oracle, and rejects every
invalid call on the host before any HIP call."""
import ctypes
import os
import re
import subprocess

import pytest

import oracle
from sparse_long_context_segmented_amd import wi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(wi.LIB_PATH):
        from sparse_long_context_segmented_amd import _build
        _build.build()
    return wi.lib()


def _declared():
    hdr = open(os.path.join(ROOT, "include", "wi.h")).read()
    return sorted(set(re.findall(r"\b(wi_[a-z_]+)\s*\(", hdr)))


def test_exports_every_declared_symbol(L):
    names = _declared()
    assert set(names) == set(wi.EXPORTS)
    out = subprocess.run(["nm", "-D", "--defined-only", wi.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if l.strip()}
    for n in names:
        assert n in exported, n
        assert getattr(L, n) is not None


def test_status_strings(L):
    for code, name in wi.STATUS.items():
        assert L.wi_status_str(code).decode() == name


@pytest.mark.parametrize("dtype,B,H,N,seg,k", [
    ("bf16", 1, 8, 131072, 8192, 512), ("f32", 1, 1, 8192, 8192, 512),
    ("bf16", 4, 4, 262144, 8192, 512), ("bf16", 2, 3, 68 + 3 * 96 + 37, 96, 12),
    ("bf16", 1, 1, 69, 8192, 512), ("f32", 1, 2, 68 + 40, 16, 16)])
def test_sizes_match_oracle(L, dtype, B, H, N, seg, k):
    d = wi.make_desc(dtype, B, H, N, seg_len=seg, clusters_per_seg=k)
    ns, C, cap, ws = wi.index_sizes(d)
    ons, oC, ocap, T = oracle.sizes(oracle.make_desc(dtype, B, H, N, seg_len=seg,
                                                     clusters_per_seg=k))
    assert (ns, C, cap) == (ons, oC, ocap)
    assert ws > 0


def test_sizes_of_named_workloads(L):
    # segments, clusters and block capacity per unit of the five shapes
    exp = {131072: (16, 8192, 23543), 8192: (1, 512, 2415), 262144: (32, 16384, 47095),
           1048576: (128, 65536, 188407)}
    for n, (ns, c, cap) in exp.items():
        dt = "f32" if n == 8192 else "bf16"
        assert wi.index_sizes(wi.make_desc(dt, 1, 1, n))[:3] == (ns, c, cap)


def _bad_build(L, desc, ptrs=None, ws_bytes=1 << 40):
    fake = ctypes.c_void_p(0x100000)  # never dereferenced: validation fails first
    p = dict(k=fake, v=fake, init=None, ws=fake)
    if ptrs:
        p.update(ptrs)
    bufs = wi.IndexBufs(*([0x100000] * 10))
    return L.wi_build_index(ctypes.byref(desc), p["k"], p["v"], p["init"], ctypes.byref(bufs),
                            p["ws"], ws_bytes, None), bufs


def test_build_rejects_bad_descriptors(L):
    def expect(code, **kw):
        d = wi.make_desc("bf16", 1, 2, 4096, seg_len=1024, clusters_per_seg=64)
        for k_, v_ in kw.items():
            setattr(d, k_, v_)
        rc, _ = _bad_build(L, d)
        assert rc == code, (kw, rc, L.wi_last_error())
        assert L.wi_last_error().decode()
    expect(2, head_dim=64)
    expect(2, dtype=7)
    expect(1, batch=0)
    expect(1, n_kv_heads=0)
    expect(1, n_ctx=68)
    expect(1, n_sink=-1)
    expect(1, seg_len=0)
    expect(1, seg_len=8193)
    expect(1, clusters_per_seg=0)
    expect(1, clusters_per_seg=513)
    expect(1, n_iters=-1)
    expect(1, kv_stride_t=0)
    expect(1, kv_stride_t=129)
    expect(1, kv_stride_h=-8)


def test_build_rejects_bad_pointers_and_workspace(L):
    d = wi.make_desc("bf16", 1, 2, 4096, seg_len=1024, clusters_per_seg=64)
    rc, _ = _bad_build(L, d, dict(k=None))
    assert rc == 1 and b"k is NULL" in L.wi_last_error()
    rc, _ = _bad_build(L, d, dict(v=ctypes.c_void_p(0x100004)))
    assert rc == 1 and b"aligned" in L.wi_last_error()
    rc, _ = _bad_build(L, d, dict(init=ctypes.c_void_p(0x100008)))
    assert rc == 1
    need = wi.index_sizes(d)[3]
    rc, _ = _bad_build(L, d, ws_bytes=need - 1)
    assert rc == 3
    rc, _ = _bad_build(L, d, dict(ws=None), ws_bytes=need)
    assert rc == 3
    bufs = wi.IndexBufs(*([0x100000] * 10))
    bufs.centroids = None
    fake = ctypes.c_void_p(0x100000)
    rc = L.wi_build_index(ctypes.byref(d), fake, fake, None, ctypes.byref(bufs), fake, need, None)
    assert rc == 1 and b"centroids" in L.wi_last_error()
    rc = L.wi_build_index(ctypes.byref(d), fake, fake, None, None, fake, need, None)
    assert rc == 1
    rc = L.wi_build_index(None, fake, fake, None, ctypes.byref(bufs), fake, need, None)
    assert rc == 1


def _decode(L, desc, dd, **kw):
    fake = ctypes.c_void_p(0x100000)
    bufs = wi.IndexBufs(*([0x100000] * 10))
    if "bufs" in kw:
        bufs = kw.pop("bufs")
    args = dict(q=fake, out=fake, sel=None, exe=None, nexe=None, cap=0, ws=fake,
                ws_bytes=1 << 40)
    args.update(kw)
    return L.wi_decode_attention(ctypes.byref(desc), ctypes.byref(dd), ctypes.byref(bufs),
                                 args["q"], args["out"], args["sel"], args["exe"],
                                 args["nexe"], args["cap"], args["ws"], args["ws_bytes"], None)


def test_decode_rejects_invalid_calls(L):
    d = wi.make_desc("bf16", 2, 4, 4096, seg_len=1024, clusters_per_seg=64)
    C = wi.index_sizes(d)[1]
    assert _decode(L, d, wi.DecodeDesc(6, 4, 10, 0.0)) == 2       # Hq % Hkv
    assert _decode(L, d, wi.DecodeDesc(4 * 17, 4, 10, 0.0)) == 2  # G > 16
    assert _decode(L, d, wi.DecodeDesc(16, C + 1, 10, 0.0)) == 1  # K_r > C
    assert _decode(L, d, wi.DecodeDesc(16, -1, 10, 0.0)) == 1
    assert _decode(L, d, wi.DecodeDesc(16, 4, -1, 0.0)) == 1
    assert _decode(L, d, wi.DecodeDesc(16, 4, 10, -1.0)) == 1
    assert _decode(L, d, wi.DecodeDesc(16, 4, 10, float("nan"))) == 1
    assert _decode(L, d, wi.DecodeDesc(16, 4, 10, 0.0, -1)) == 1   # wg_per_unit
    assert _decode(L, d, wi.DecodeDesc(16, 4, 10, 0.0, 65)) == 1
    assert _decode(L, d, wi.DecodeDesc(16, 4, 10, 0.0), q=None) == 1
    assert _decode(L, d, wi.DecodeDesc(16, 4, 10, 0.0), out=ctypes.c_void_p(0x100002)) == 1
    need = wi.decode_sizes(d, wi.DecodeDesc(16, 4, 10, 0.0))
    assert _decode(L, d, wi.DecodeDesc(16, 4, 10, 0.0), ws_bytes=need - 1) == 3
    bufs = wi.IndexBufs(*([0x100000] * 10))
    bufs.slot_token = None
    assert _decode(L, d, wi.DecodeDesc(16, 4, 10, 0.0), bufs=bufs,
                   exe=ctypes.c_void_p(0x100000), cap=10) == 1
    d.head_dim = 96
    assert _decode(L, d, wi.DecodeDesc(16, 4, 10, 0.0)) == 2


def test_decode_sizes_grow_with_budget(L):
    d = wi.make_desc("bf16", 1, 8, 131072)
    a = wi.decode_sizes(d, wi.DecodeDesc(32, 147, 1884, 0.0))
    b = wi.decode_sizes(d, wi.DecodeDesc(32, 1000, 4000, 0.0))
    assert b > a > 8 * 8192 * 4
    # K_e is clamped to C - K_r
    assert wi.decode_sizes(d, wi.DecodeDesc(32, 4096, 5000, 0.0)) == \
        wi.decode_sizes(d, wi.DecodeDesc(32, 4096, 4096, 0.0))
    # any retrieval budget up to C is accepted
    assert wi.decode_sizes(d, wi.DecodeDesc(32, 8192, 0, 0.0)) > 0


def test_noalloc_scratch_limit_matches_header():
    hdr = open(os.path.join(ROOT, "include", "wi.h")).read()
    m = re.search(r"#define WI_NOALLOC_SCRATCH_BYTES \((\d+)ull << (\d+)\)", hdr)
    assert m and int(m.group(1)) << int(m.group(2)) == wi.NOALLOC_SCRATCH_BYTES


def test_noalloc_rejects_workspace_beyond_static_maximum(L):
    """128 units of 8192 clusters need more decode scratch than the static
    array holds: rejected on the host, before any HIP call."""
    d = wi.make_desc("bf16", 16, 8, 131072)
    dd = wi.DecodeDesc(32, 147, 1884, 0.0, 0)
    assert wi.decode_sizes(d, dd) > wi.NOALLOC_SCRATCH_BYTES
    fake = ctypes.c_void_p(0x100000)  # never dereferenced
    bufs = wi.IndexBufs(*([0x100000] * 10))
    rc = L.wi_decode_attention_noalloc(ctypes.byref(d), ctypes.byref(dd), ctypes.byref(bufs),
                                       fake, fake, None, None, None, 0, None)
    assert rc == 3
    assert "static" in L.wi_last_error().decode()


def test_noalloc_validates_like_the_workspace_entry_point(L):
    d = wi.make_desc("bf16", 1, 8, 131072)
    dd = wi.DecodeDesc(32, 147, 1884, 0.0, 0)
    fake = ctypes.c_void_p(0x100000)
    bufs = wi.IndexBufs(*([0x100000] * 10))
    for q, out, code in [(None, fake, 1), (fake, None, 1), (ctypes.c_void_p(0x100004), fake, 1)]:
        rc = L.wi_decode_attention_noalloc(ctypes.byref(d), ctypes.byref(dd), ctypes.byref(bufs),
                                           q, out, None, None, None, 0, None)
        assert rc == code
    bad = wi.DecodeDesc(30, 147, 1884, 0.0, 0)  # 30 query heads over 8 KV heads
    rc = L.wi_decode_attention_noalloc(ctypes.byref(d), ctypes.byref(bad), ctypes.byref(bufs),
                                       fake, fake, None, None, None, 0, None)
    assert rc == 2


@pytest.mark.parametrize("N,pend", [(68 + 3 * 96 + 41 + 50, 50), (68 + 2 * 96 + 96, 96),
                                    (68 + 96 + 1, 1)])
def test_sizes_with_pending_tokens_match_oracle(L, N, pend):
    d = wi.make_desc("bf16", 1, 2, N, seg_len=96, clusters_per_seg=12)
    d.n_pending = pend
    od = oracle.make_desc("bf16", 1, 2, N, seg_len=96, clusters_per_seg=12, n_pending=pend)
    assert wi.index_sizes(d)[:3] == oracle.sizes(od)[:3]


def test_growth_calls_reject_invalid_descriptors(L):
    fake = ctypes.c_void_p(0x100000)  # never dereferenced
    bufs = wi.IndexBufs(*([0x100000] * 12))
    d = wi.make_desc("bf16", 1, 2, 68 + 96 + 96, seg_len=96, clusters_per_seg=12)
    d.n_pending = 97  # beyond seg_len
    assert L.wi_append_token(ctypes.byref(d), ctypes.byref(bufs), fake, fake, None) == 1
    d.n_pending = 96  # full: cluster the segment before the next append
    assert L.wi_append_token(ctypes.byref(d), ctypes.byref(bufs), fake, fake, None) == 1
    assert b"wi_extend_index" in L.wi_last_error()
    d.n_pending = 10
    nopend = wi.IndexBufs(*([0x100000] * 10))
    assert L.wi_append_token(ctypes.byref(d), ctypes.byref(nopend), fake, fake, None) == 1
    assert b"pend_k" in L.wi_last_error()
    assert L.wi_append_token(ctypes.byref(d), ctypes.byref(bufs), None, fake, None) == 1
    ws = ctypes.c_size_t()
    assert L.wi_extend_sizes(ctypes.byref(d), ctypes.byref(ws)) == 1  # not full
    rc = L.wi_extend_index(ctypes.byref(d), ctypes.byref(bufs), ctypes.byref(bufs), fake,
                           1 << 40, None)
    assert rc == 1
    d.n_ctx = 68 + 96  # too short for 96 pending tokens plus one clustered token
    d.n_pending = 96
    assert L.wi_extend_sizes(ctypes.byref(d), ctypes.byref(ws)) == 1
    # a pending descriptor is not a build descriptor
    d2 = wi.make_desc("bf16", 1, 2, 68 + 96 + 5, seg_len=96, clusters_per_seg=12)
    d2.n_pending = 5
    need = wi.index_sizes(d2)[3]
    rc = L.wi_build_index(ctypes.byref(d2), fake, fake, None, ctypes.byref(bufs), fake, need,
                          None)
    assert rc == 1 and b"n_pending" in L.wi_last_error()


def test_extend_workspace_holds_a_one_segment_build(L):
    d = wi.make_desc("bf16", 1, 8, 131072 + 8192)
    d.n_pending = 8192
    ws = wi.extend_sizes(d)
    seg = wi.make_desc("bf16", 1, 8, 8192, n_sink=0, n_local=0)
    ns, C, cap, bws = wi.index_sizes(seg)
    index_bytes = 8 * (C * 128 * 2 + C * 4 + C * 128 * 4 + (C + 1) * 4 + 2 * cap * 8 * 128 * 2
                       + cap * 8 * 4 + 8192 * 4)
    assert ws >= bws + index_bytes
    fake = ctypes.c_void_p(0x100000)
    bufs = wi.IndexBufs(*([0x100000] * 12))
    rc = L.wi_extend_index(ctypes.byref(d), ctypes.byref(bufs), ctypes.byref(bufs), fake,
                           ws - 1, None)
    assert rc == 3


@pytest.mark.parametrize("n_layers,n_ctx", [(80, 131072), (32, 1048576), (28, 262144),
                                            (2, 8192), (1, 69)])
def test_layer_plan_matches_oracle_policy(L, n_layers, n_ctx):
    from oracle import policy
    for kind in (policy.UNIFORM, policy.DENSE_FIRST2, policy.BANDED):
        for layer in range(n_layers):
            assert wi.layer_plan(kind, layer, n_layers, n_ctx) == \
                policy.plan(kind, layer, n_layers, n_ctx), (kind, layer)


def test_layer_plan_rejects_bad_arguments(L):
    out = [ctypes.c_int32() for _ in range(3)]
    refs = [ctypes.byref(o) for o in out]
    assert L.wi_layer_plan(3, 0, 32, 131072, 8192, 512, *refs) == 1
    assert L.wi_layer_plan(0, 32, 32, 131072, 8192, 512, *refs) == 1
    assert L.wi_layer_plan(0, -1, 32, 131072, 8192, 512, *refs) == 1
    assert L.wi_layer_plan(0, 0, 32, 0, 8192, 512, *refs) == 1
    assert L.wi_layer_plan(2, 0, 32, 131072, 8192, 512, None, None, None) == 0


def test_dense_and_recall_reject_invalid_calls(L):
    fake = ctypes.c_void_p(0x100000)  # never dereferenced
    d = wi.make_desc("bf16", 1, 8, 131072)
    dd = wi.DecodeDesc(32, 0, 0, 0.0)
    need = wi.dense_sizes(d, dd)
    assert need >= 8 * 4 * 130 * 4

    def dense(desc=d, ddesc=dd, k=fake, v=fake, q=fake, out=fake, ws=fake, nb=need):
        return L.wi_dense_attention(ctypes.byref(desc), ctypes.byref(ddesc), k, v, q, out, ws,
                                    nb, None)
    assert dense(k=None) == 1
    assert dense(out=ctypes.c_void_p(0x100004)) == 1
    assert dense(nb=need - 1) == 3
    assert dense(ddesc=wi.DecodeDesc(30, 0, 0, 0.0)) == 2
    bad = wi.make_desc("bf16", 1, 8, 131072)
    bad.n_ctx = 0
    assert dense(desc=bad) == 1
    bad = wi.make_desc("bf16", 1, 8, 131072)
    bad.head_dim = 64
    assert dense(desc=bad) == 2
    # recall: k range, zone size and pointers
    bufs = wi.IndexBufs(*([0x100000] * 12))
    wsr = wi.recall_sizes(d, dd)
    assert wsr >= 8 * 4 * wi.index_sizes(d)[2] * 8 * 8

    def rec(k=100, n_r=147, stride=2031, sel=fake, nb=wsr, b=bufs):
        return L.wi_recall_at_k(ctypes.byref(d), ctypes.byref(dd), ctypes.byref(b), fake, sel,
                                stride, n_r, k, fake, None, fake, nb, None)
    assert rec(k=0) == 1
    assert rec(k=1025) == 1
    assert rec(n_r=8193) == 1
    assert rec(stride=100) == 1
    assert rec(sel=None) == 1
    assert rec(nb=wsr - 1) == 3
    nob = wi.IndexBufs(*([0x100000] * 12))
    nob.assign = None
    assert rec(b=nob) == 1


def test_timing_hook_host_side(L):
    """The measurement hook with no launch in between records nothing and
    makes no HIP call; kernel ids map to their names, others to "unknown"."""
    assert L.wi_timing_start() == 0
    assert L.wi_timing_stop(0, None, None) == 0
    assert wi.timing_stop() == []  # (stopping twice is harmless)
    assert L.wi_kernel_name(0).decode() == "zero"
    names = {L.wi_kernel_name(i).decode() for i in range(64)}
    assert {"score", "select_attend", "assign", "kpp_round"} <= names
    assert L.wi_kernel_name(-1).decode() == "unknown"
    assert L.wi_kernel_name(1 << 20).decode() == "unknown"
