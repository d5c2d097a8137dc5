"""Pins of the oracle's decode-time growth (append, pending tokens, extend)
against things other than itself: the token stream itself, the brute-force
softmax over an explicit token list, a fresh build of the same stream, and
torch's full attention."""
import math

import numpy as np
import pytest

import oracle
from oracle import brute
from sparse_long_context_segmented_amd import synth


def _stream(dtype="bf16", n_ctx=68 + 3 * 96, seg=96, k=12, n_new=96 + 40, B=1, H=2, G=2,
            iters=2, wid=95):
    """A workload whose first n_ctx tokens are built and whose next n_new
    tokens arrive one per decode step."""
    total = n_ctx + n_new
    w = synth.custom(wid, dtype, B, H * G, H, total, seg, k, n_iters=iters, n_needles=3,
                     n_components=24)
    K, V, q = synth.gen_batch(w)
    d = oracle.make_desc(dtype, B, H, n_ctx, seg_len=seg, clusters_per_seg=k, n_iters=iters)
    return w, d, K, V, q


def _advance(d, idx, K, V, steps):
    """steps appends of the stream's next tokens (extending when full)."""
    for _ in range(steps):
        if d.n_pending == d.seg_len:
            d, idx = oracle.extend(d, idx)
        p = d.n_ctx
        d = oracle.append(d, idx, K[:, :, p], V[:, :, p])
    return d, idx


def test_append_slides_window_and_pends_the_departing_token():
    w, d, K, V, q = _stream()
    idx = oracle.build(d, K[:, :, :d.n_ctx], V[:, :, :d.n_ctx])
    d1, idx = _advance(d, idx, K, V, 50)
    assert (d1.n_ctx, d1.n_pending) == (d.n_ctx + 50, 50)
    U = d.batch * d.n_kv_heads
    Ku, Vu = K.reshape(U, K.shape[2], 128), V.reshape(U, V.shape[2], 128)
    N = d1.n_ctx
    steady = list(range(4)) + list(range(N - 64, N))
    p0 = d.n_ctx - 64  # the first token that left the window
    for u in range(U):
        assert np.array_equal(idx["steady_k"][u], Ku[u][steady])
        assert np.array_equal(idx["steady_v"][u], Vu[u][steady])
        assert np.array_equal(idx["pend_k"][u][:50], Ku[u][p0:p0 + 50])
        assert np.array_equal(idx["pend_v"][u][:50], Vu[u][p0:p0 + 50])


def test_append_refuses_a_full_pending_segment():
    w, d, K, V, q = _stream()
    idx = oracle.build(d, K[:, :, :d.n_ctx], V[:, :, :d.n_ctx])
    d1, idx = _advance(d, idx, K, V, d.seg_len)
    assert d1.n_pending == d1.seg_len
    with pytest.raises(ValueError):
        oracle.append(d1, idx, K[:, :, d1.n_ctx], V[:, :, d1.n_ctx])


def _members(idx, u, T):
    bo, sz, st = idx["block_off"][u], idx["sizes"][u], idx["slot_token"][u]
    return [st[bo[c] * T: bo[c] * T + sz[c]] for c in range(len(sz))]


@pytest.mark.parametrize("steps", [1, 37, 96 + 20])
def test_decode_with_pending_equals_bruteforce(steps):
    """Decode after appends (some pending, possibly after an extension) equals
    one explicit softmax over steady + pending + retrieved tokens + estimated
    clusters, and its execution list is steady, pending, retrieved."""
    w, d, K, V, q = _stream()
    idx = oracle.build(d, K[:, :, :d.n_ctx], V[:, :, :d.n_ctx])
    d1, idx = _advance(d, idx, K, V, steps)
    ns, C, cap, T = oracle.sizes(d1)
    kr, ke = 3, 9
    res = oracle.decode(d1, 4, kr, ke, idx, q)
    N = d1.n_ctx
    U = d.batch * d.n_kv_heads
    Ku, Vu = K.reshape(U, K.shape[2], 128)[:, :N], V.reshape(U, V.shape[2], 128)[:, :N]
    p0 = N - 64 - d1.n_pending
    pend = list(range(p0, p0 + d1.n_pending))
    for u in range(U):
        b, h = divmod(u, d.n_kv_heads)
        mem = _members(idx, u, T)
        R, E = res["sel"][u][:kr], res["sel"][u][kr:]
        for j in range(2):
            ref = brute.tripartite(q[b, h * 2 + j], Ku[u], Vu[u], mem, idx["centroids"][u],
                                   R, E, 4, 64, 1 / math.sqrt(128), extra=pend)
            assert np.allclose(res["out"][b, h * 2 + j], ref, rtol=1e-9, atol=1e-12)
        exp_tok = list(range(4)) + list(range(N - 64, N)) + pend + \
            [int(t) for c in R for t in mem[c]]
        assert res["n_exec"][u] == len(exp_tok)
        assert res["exec_tokens"][u][:len(exp_tok)].tolist() == exp_tok


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_extend_equals_fresh_build_of_the_same_stream(dtype):
    """With segments aligned (the built range a whole number of segments),
    seg_len appends and one extension give exactly the index a fresh build of
    the longer stream gives: same centroids, sizes, value sums, block map,
    K/V blocks, slot map, steady rows and assignment."""
    w, d, K, V, q = _stream(dtype=dtype, n_ctx=68 + 3 * 96, n_new=96)
    idx = oracle.build(d, K[:, :, :d.n_ctx], V[:, :, :d.n_ctx])
    d1, idx = _advance(d, idx, K, V, d.seg_len)
    d2, grown = oracle.extend(d1, idx)
    assert d2.n_pending == 0 and d2.n_ctx == d.n_ctx + d.seg_len
    fresh_d = oracle.make_desc(dtype, d.batch, d.n_kv_heads, d2.n_ctx, seg_len=d.seg_len,
                               clusters_per_seg=d.clusters_per_seg, n_iters=d.n_iters)
    fresh = oracle.build(fresh_d, K[:, :, :d2.n_ctx], V[:, :, :d2.n_ctx])
    for key in ("centroids", "sizes", "vsum", "block_off", "kblk", "vblk", "slot_token",
                "steady_k", "steady_v", "assign"):
        a, b = np.asarray(grown[key]), np.asarray(fresh[key])
        assert a.shape == b.shape, key
        assert np.array_equal(a.view(np.uint32) if a.dtype == np.float32 else a,
                              b.view(np.uint32) if b.dtype == np.float32 else b), key


def test_extend_after_a_short_built_segment_keeps_every_token_once():
    """The built range ends with a short segment: the next segment starts
    right after it. Every indexed token appears in exactly one slot, the block
    map counts the sizes, the new clusters' centroids are the rounded means of
    their members and their value sums the rounded float64 sums."""
    w, d, K, V, q = _stream(n_ctx=68 + 2 * 96 + 41, n_new=2 * 96 + 5)
    idx = oracle.build(d, K[:, :, :d.n_ctx], V[:, :, :d.n_ctx])
    ns0, C0, _, T = oracle.sizes(d)
    d1, idx = _advance(d, idx, K, V, 2 * 96 + 5)  # two extensions, 5 pending
    assert d1.n_pending == 5
    ns, C, cap, T = oracle.sizes(d1)
    assert C == C0 + 2 * 12
    U = d.batch * d.n_kv_heads
    Ku, Vu = K.reshape(U, K.shape[2], 128), V.reshape(U, V.shape[2], 128)
    n_clustered = d1.n_ctx - 68 - d1.n_pending
    for u in range(U):
        st, bo, sz = idx["slot_token"][u], idx["block_off"][u], idx["sizes"][u]
        toks = st[st >= 0]
        assert sorted(toks.tolist()) == list(range(4, 4 + n_clustered))
        assert np.array_equal(np.diff(bo), (sz + T - 1) // T)
        for c in range(C0, C):
            m = st[bo[c] * T: bo[c] * T + sz[c]]
            assert np.all(np.diff(m) > 0)
            mean = (Ku[u][m].astype(np.float64).sum(0) / len(m)).astype(np.float32)
            assert np.array_equal(idx["centroids"][u][c], brute.bf16(mean))
            vs = Vu[u][m].astype(np.float64).sum(0).astype(np.float32)
            assert np.array_equal(idx["vsum"][u][c], vs)


def test_full_budget_after_growth_is_full_attention():
    """K_r = C after appends and extensions: attention over every token of
    the stream so far (torch SDPA in float64) -- no token lost or doubled."""
    import torch
    w, d, K, V, q = _stream(n_ctx=68 + 2 * 96 + 41, n_new=2 * 96 + 5)
    idx = oracle.build(d, K[:, :, :d.n_ctx], V[:, :, :d.n_ctx])
    d1, idx = _advance(d, idx, K, V, 2 * 96 + 5)
    ns, C, cap, T = oracle.sizes(d1)
    res = oracle.decode(d1, 4, C, 0, idx, q)
    N = d1.n_ctx
    for h in range(d.n_kv_heads):
        Kt = torch.from_numpy(K[0, h, :N].astype(np.float64))[None, None]
        Vt = torch.from_numpy(V[0, h, :N].astype(np.float64))[None, None]
        for j in range(2):
            Q = torch.from_numpy(q[0, h * 2 + j].astype(np.float64))[None, None, None, :]
            ref = torch.nn.functional.scaled_dot_product_attention(Q, Kt, Vt)[0, 0, 0].numpy()
            assert np.allclose(res["out"][0, h * 2 + j], ref, rtol=1e-10, atol=1e-12)
