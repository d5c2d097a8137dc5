"""Property tests of the oracle against its brute-force numpy twin over random
tiny shapes (hypothesis).

The oracle (scalar C) and brute.py (whole-matrix numpy fp64) are written in
different shapes; these tests draw shapes, budgets, dtypes and seeds at random
and require them to agree: nearest-centroid labels, mean updates, whole Lloyd
runs from the same initial centroids, the block layout's invariants, the
ranking (np.lexsort of brute-force group scores), and the tripartite output
(one explicit softmax over tokens and estimated clusters).
"""
import math

import numpy as np
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import oracle
from oracle import brute

SETTINGS = settings(max_examples=40, deadline=None,
                    suppress_health_check=[HealthCheck.too_slow])


def _rng(seed):
    return np.random.default_rng([11, seed])


def _round(x, dtype):
    return brute.bf16(x) if dtype == "bf16" else np.asarray(x, np.float32)


@SETTINGS
@given(seed=st.integers(0, 10 ** 6), n=st.integers(1, 60), k=st.integers(1, 12),
       d=st.sampled_from([1, 3, 8, 128]), dtype=st.sampled_from(["bf16", "f32"]),
       dup=st.booleans())
def test_assign_and_update_match_bruteforce(seed, n, k, d, dtype, dup):
    rng = _rng(seed)
    X = _round(rng.standard_normal((n, d)).astype(np.float32), dtype)
    if dup:  # repeated points and centroids: ties go to the lowest id
        X[n // 2:] = X[: n - n // 2]
    C = _round(rng.standard_normal((k, d)).astype(np.float32), dtype)
    if dup and k > 1:
        C[-1] = C[0]
    a = oracle.assign(X, C)
    assert np.array_equal(a, brute.assign(X, C))
    Cn, cnt = oracle.update(X, a, C, dtype)
    Cb, cntb = brute.update(X, a, C, dtype)
    assert np.array_equal(cnt, cntb)
    assert np.array_equal(Cn.view(np.uint32), Cb.view(np.uint32))


def _desc_and_data(seed, dtype, B, H, n_ctx, seg, k, iters, n_sink=4, n_local=64):
    rng = _rng(seed)
    d = oracle.make_desc(dtype, B, H, n_ctx, seg_len=seg, clusters_per_seg=k,
                         n_sink=n_sink, n_local=n_local, n_iters=iters)
    # a few well-separated modes so clusters are non-trivial
    modes = rng.standard_normal((4, 128)).astype(np.float32) * 2
    lab = rng.integers(0, 4, size=(B, H, n_ctx))
    K = _round(modes[lab] + 0.5 * rng.standard_normal((B, H, n_ctx, 128)).astype(np.float32),
               dtype)
    V = _round(rng.standard_normal((B, H, n_ctx, 128)).astype(np.float32), dtype)
    return d, K, V


shape = st.tuples(st.integers(1, 2), st.integers(1, 2), st.integers(1, 100),
                  st.sampled_from([8, 16, 33]), st.integers(1, 9))


@SETTINGS
@given(seed=st.integers(0, 10 ** 6), shp=shape, iters=st.integers(0, 3),
       dtype=st.sampled_from(["bf16", "f32"]))
def test_build_with_given_init_is_bruteforce_lloyd(seed, shp, iters, dtype):
    """From the same initial centroids, every segment's centroids and labels
    equal brute.lloyd's, and the layout holds every indexed token once."""
    B, H, n_idx, seg, k = shp
    n_ctx = n_idx + 68
    d, K, V = _desc_and_data(seed, dtype, B, H, n_ctx, seg, k, iters)
    ns, C, cap, T = oracle.sizes(d)
    parts = brute.partition(n_ctx, seg, k)
    assert len(parts) == ns and sum(p[2] for p in parts) == C
    rng = _rng(seed + 1)
    init = np.empty((B, H, C, 128), np.float32)
    for b in range(B):
        for h in range(H):
            for pos, n, c, cid in parts:
                pick = rng.choice(n, size=c, replace=False)
                init[b, h, cid:cid + c] = K[b, h, pos + pick]
    idx = oracle.build(d, K, V, init=init)
    for b in range(B):
        for h in range(H):
            u = b * H + h
            for pos, n, c, cid in parts:
                X, C0 = K[b, h, pos:pos + n], init[b, h, cid:cid + c]
                if iters:
                    Cb, ab = brute.lloyd(X, C0, iters, dtype)
                else:  # one assignment to the given centroids
                    Cb, ab = C0, brute.assign(X, C0)
                got_c = idx["centroids"][u][cid:cid + c]
                assert np.array_equal(got_c.view(np.uint32), Cb.view(np.uint32))
                off = pos - 4
                assert np.array_equal(idx["assign"][u][off:off + n], ab + cid)
            st_ = idx["slot_token"][u]
            assert sorted(st_[st_ >= 0].tolist()) == list(range(4, n_ctx - 64))
            bo, sz = idx["block_off"][u], idx["sizes"][u]
            assert np.array_equal(np.diff(bo), (sz + T - 1) // T) and bo[-1] <= cap


@SETTINGS
@given(seed=st.integers(0, 10 ** 6), shp=shape, G=st.sampled_from([1, 2, 3]),
       kr=st.integers(0, 6), ke=st.integers(0, 20), dtype=st.sampled_from(["bf16", "f32"]))
def test_decode_matches_bruteforce_softmax(seed, shp, G, kr, ke, dtype):
    B, H, n_idx, seg, k = shp
    n_ctx = n_idx + 68
    d, K, V = _desc_and_data(seed, dtype, B, H, n_ctx, seg, k, 2)
    ns, C, cap, T = oracle.sizes(d)
    kr = min(kr, C)
    idx = oracle.build(d, K, V)
    rng = _rng(seed + 2)
    q = _round(rng.standard_normal((B, H * G, 128)).astype(np.float32), dtype)
    r = oracle.decode(d, H * G, kr, ke, idx, q)
    ke_c = min(ke, C - kr)
    scale = 1 / math.sqrt(128)
    for b in range(B):
        for h in range(H):
            u = b * H + h
            cen = idx["centroids"][u].astype(np.float64)
            g = (cen @ q[b, h * G:(h + 1) * G].astype(np.float64).T).sum(axis=1)
            order = np.lexsort((np.arange(C), -g))[:kr + ke_c]
            assert np.array_equal(r["sel"][u], order)
            bo, sz, stt = idx["block_off"][u], idx["sizes"][u], idx["slot_token"][u]
            mem = [stt[bo[c] * T: bo[c] * T + sz[c]] for c in range(C)]
            for j in range(G):
                ref = brute.tripartite(q[b, h * G + j], K[b, h], V[b, h], mem,
                                       idx["centroids"][u], order[:kr], order[kr:], 4, 64,
                                       scale, vsum_f32=True)
                assert np.allclose(r["out"][b, h * G + j], ref, rtol=1e-9, atol=1e-12)


@SETTINGS
@given(seed=st.integers(0, 10 ** 6), n_built=st.integers(1, 40), steps=st.integers(1, 70),
       seg=st.sampled_from([8, 16, 24]), k=st.integers(1, 6))
def test_growth_keeps_every_token_once_and_decodes_like_bruteforce(seed, n_built, steps, seg,
                                                                   k):
    """Appends and extensions over random lengths: every token of the stream
    is in exactly one place (steady, pending or one cluster slot), and decode
    equals the brute-force softmax over steady + pending + retrieved."""
    n_ctx = n_built + 68
    d, K, V = _desc_and_data(seed, "bf16", 1, 1, n_ctx + steps, seg, k, 2)
    d = oracle.make_desc("bf16", 1, 1, n_ctx, seg_len=seg, clusters_per_seg=k, n_iters=2)
    idx = oracle.build(d, K[:, :, :n_ctx], V[:, :, :n_ctx])
    for _ in range(steps):
        if d.n_pending == d.seg_len:
            d, idx = oracle.extend(d, idx)
        d = oracle.append(d, idx, K[:, :, d.n_ctx], V[:, :, d.n_ctx])
    ns, C, cap, T = oracle.sizes(d)
    N = d.n_ctx
    p0 = N - 64 - d.n_pending
    stt = idx["slot_token"][0]
    clustered = sorted(stt[stt >= 0].tolist())
    assert clustered == list(range(4, p0))
    if d.n_pending:
        assert np.array_equal(idx["pend_k"][0][:d.n_pending], K[0, 0, p0:N - 64])
    q = brute.bf16(_rng(seed + 3).standard_normal((1, 2, 128)).astype(np.float32))
    kr, ke = min(2, C), 3
    r = oracle.decode(d, 2, kr, ke, idx, q)
    bo, sz = idx["block_off"][0], idx["sizes"][0]
    mem = [stt[bo[c] * T: bo[c] * T + sz[c]] for c in range(C)]
    sel = r["sel"][0]
    for j in range(2):
        ref = brute.tripartite(q[0, j], K[0, 0, :N], V[0, 0, :N], mem, idx["centroids"][0],
                               sel[:kr], sel[kr:], 4, 64, 1 / math.sqrt(128),
                               extra=range(p0, p0 + d.n_pending), vsum_f32=True)
        assert np.allclose(r["out"][0, j], ref, rtol=1e-9, atol=1e-12)
