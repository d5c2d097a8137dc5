"""Pins of the CPU oracle against things other than itself.

Each test ties one oracle function to a published value, a library routine,
a closed form, an invariant, or an independent brute force on tiny inputs
(oracle/brute.py), so that a dropped term, a wrong sign or index, or a
transposed operand in the oracle fails at least one of them.
"""
import math
import os

import numpy as np
import pytest

import oracle
from oracle import brute
from sparse_long_context_segmented_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _bf16(x):
    return brute.bf16(x)


# --------------------------------------------------------------------------
# Random numbers: the published SplitMix64 known-answer values.

def test_mix64_known_answers(orc):
    vals = [int(l) for l in open(os.path.join(GOLDEN, "splitmix64_seed1234567.txt"))
            if l.strip() and not l.startswith("#")]
    state = 1234567
    got = []
    for _ in range(5):
        state = (state + 0x9E3779B97F4A7C15) % (1 << 64)
        got.append(orc.mix64(state))
    assert got == vals


def test_key_chain_distinct_and_uniform(orc):
    # Different counters give different keys; the 53-bit uniforms of many
    # counters look uniform (Kolmogorov-Smirnov against U(0,1)).
    from scipy import stats
    keys = [orc.key(0, 0, 0, 0, s, r) for s in range(20) for r in range(100)]
    assert len(set(keys)) == len(keys)
    u = np.array([(k >> 11) * 2.0 ** -53 for k in keys])
    assert stats.kstest(u, "uniform").pvalue > 1e-3
    # each counter position matters
    base = orc.key(5, 1, 2, 3, 4, 6)
    for i in range(6):
        args = [5, 1, 2, 3, 4, 6]
        args[i] += 1
        assert orc.key(*args) != base


# --------------------------------------------------------------------------
# bf16 rounding: equals torch's round-to-nearest-even conversion.

def test_round_bf16_matches_torch(orc):
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.standard_normal(4000).astype(np.float32) * 10,
                        rng.standard_normal(1000).astype(np.float32) * 1e-30])
    # exact halfway cases (low 16 bits 0x8000) with odd and even kept parts
    bits = (rng.integers(0, 1 << 14, 1000, dtype=np.uint32) << 16) | np.uint32(0x8000)
    bits += np.uint32(0x3F000000)
    x = np.concatenate([x, bits.view(np.float32)]).astype(np.float32)
    ref = _bf16(x)
    got = np.array([orc.round_bf16(float(v)) for v in x], np.float32)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


# --------------------------------------------------------------------------
# Distances: exact on integer data; within the float error bound otherwise.

def test_dist_exact_on_small_integers(orc):
    rng = np.random.default_rng(2)
    x = rng.integers(-8, 8, 128).astype(np.float32)
    c = rng.integers(-8, 8, 128).astype(np.float32)
    exact = float(((x.astype(np.int64) - c.astype(np.int64)) ** 2).sum())
    X = np.stack([x, c])
    # via assign: distance ordering must follow the exact integer distances
    C = np.stack([c, x])
    assert list(orc.assign(X, C)) == [1, 0]
    lib = orc.lib()
    import ctypes
    lib.wio_dist32.restype = ctypes.c_float
    lib.wio_dist32.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int]
    lib.wio_dist64.restype = ctypes.c_double
    lib.wio_dist64.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int]
    assert lib.wio_dist32(x.ctypes.data, c.ctypes.data, 128) == exact
    assert lib.wio_dist64(x.ctypes.data, c.ctypes.data, 128) == exact
    xr = rng.standard_normal(128).astype(np.float32)
    cr = rng.standard_normal(128).astype(np.float32)
    ex = float(((xr.astype(np.float64) - cr.astype(np.float64)) ** 2).sum())
    d32 = lib.wio_dist32(xr.ctypes.data, cr.ctypes.data, 128)
    assert abs(d32 - ex) <= 130 * 2.0 ** -24 * ex
    d64 = lib.wio_dist64(xr.ctypes.data, cr.ctypes.data, 128)
    assert abs(d64 - ex) <= 130 * 2.0 ** -53 * ex


# --------------------------------------------------------------------------
# k-means++ (Arthur and Vassilvitskii 2007): sampling law and special cases.

def test_kmeanspp_full_k_is_permutation(orc):
    rng = np.random.default_rng(3)
    X = _bf16(rng.standard_normal((37, 128)).astype(np.float32))
    for s in range(5):
        p = orc.kmeanspp(X, 37, seed=s)
        assert sorted(p.tolist()) == list(range(37))


def test_kmeanspp_all_equal_points(orc):
    X = np.ones((9, 128), np.float32)
    p = orc.kmeanspp(X, 5, seed=11)
    # the first pick is drawn; every later draw sees zero weight everywhere and
    # takes the smallest index not yet chosen
    rest = [i for i in range(9) if i != p[0]][:4]
    assert p[1:].tolist() == rest


def _exact_kpp_probs(X, k):
    n = X.shape[0]
    D = ((X[:, None, :].astype(np.float64) - X[None, :, :]) ** 2).sum(-1)
    probs = {}

    def rec(seq, p):
        if len(seq) == k:
            probs[tuple(seq)] = p
            return
        dmin = D[seq].min(axis=0)
        tot = dmin.sum()
        for i in range(n):
            if dmin[i] > 0:
                rec(seq + [i], p * dmin[i] / tot)

    for i0 in range(n):
        rec([i0], 1.0 / n)
    return probs


def test_kmeanspp_sampling_law_chi2(orc):
    from scipy import stats
    rng = np.random.default_rng(4)
    X = (rng.standard_normal((6, 128)) * np.array([1, 1, 2, 2, 3, 0.5])[:, None]).astype(np.float32)
    X = _bf16(X)
    probs = _exact_kpp_probs(X, 3)
    n_draw = 30000
    counts = {}
    for s in range(n_draw):
        t = tuple(orc.kmeanspp(X, 3, seed=s).tolist())
        counts[t] = counts.get(t, 0) + 1
    assert set(counts) <= set(probs)
    keys = sorted(probs)
    obs = np.array([counts.get(t, 0) for t in keys], float)
    exp = np.array([probs[t] for t in keys]) * n_draw
    # merge cells with tiny expectation
    small = exp < 5
    if small.any():
        obs = np.append(obs[~small], obs[small].sum())
        exp = np.append(exp[~small], exp[small].sum())
    assert stats.chisquare(obs, exp).pvalue > 1e-4


def test_kmeanspp_first_pick_uniform(orc):
    from scipy import stats
    X = _bf16(np.random.default_rng(5).standard_normal((7, 128)).astype(np.float32))
    first = np.array([orc.kmeanspp(X, 1, seed=s)[0] for s in range(7000)])
    obs = np.bincount(first, minlength=7)
    assert stats.chisquare(obs).pvalue > 1e-4


# --------------------------------------------------------------------------
# Lloyd steps.

def _mixture(rng, n, d=128, comps=12, sigma=0.3):
    M = rng.standard_normal((comps, d)).astype(np.float32)
    lab = rng.integers(0, comps, n)
    return _bf16(M[lab] + sigma * rng.standard_normal((n, d)).astype(np.float32))


def test_assign_matches_bruteforce(orc):
    rng = np.random.default_rng(6)
    X = _mixture(rng, 400)
    C = X[rng.choice(400, 24, replace=False)]
    assert np.array_equal(orc.assign(X, C), brute.assign(X, C))


def test_assign_ties_go_to_lowest_index(orc):
    rng = np.random.default_rng(7)
    X = _mixture(rng, 50)
    C = X[[3, 9, 3, 20, 9]]  # duplicated centroids
    a = orc.assign(X, C)
    assert not np.any(a == 2) and not np.any(a == 4)
    assert np.array_equal(a, brute.assign(X, C))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_update_matches_numpy_mean(orc, dtype):
    rng = np.random.default_rng(8)
    X = _mixture(rng, 300)
    if dtype == "f32":
        X = X + rng.standard_normal(X.shape).astype(np.float32) * 1e-3
    C = X[:10].copy()
    a = rng.integers(0, 9, 300).astype(np.int32)  # cluster 9 stays empty
    got, cnt = orc.update(X, a, C, dtype)
    ref, rcnt = brute.update(X, a, C, dtype)
    assert np.array_equal(cnt, rcnt)
    assert cnt[9] == 0 and np.array_equal(got[9], C[9])
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


def test_lloyd_matches_sklearn(orc):
    """Textbook Lloyd (scikit-learn, float64) from the same initial centroids."""
    from sklearn.cluster import KMeans
    rng = np.random.default_rng(9)
    X = _mixture(rng, 500, comps=16, sigma=0.2)
    picks = orc.kmeanspp(X, 16, seed=1)
    C0 = X[picks]
    for it in (1, 2, 4):
        km = KMeans(16, init=C0.astype(np.float64), n_init=1, max_iter=it, tol=0.0,
                    algorithm="lloyd").fit(X.astype(np.float64))
        C = C0.copy()
        for _ in range(it):
            a = orc.assign(X, C)
            C, _ = orc.update(X, a, C, "f32")
        assert np.array_equal(C, km.cluster_centers_.astype(np.float32))


def test_objective_never_increases_beyond_rounding(orc):
    """J(a_t, mu_t) <= J(a_t, mu_{t-1}) + rho_t; J(a_{t+1}, mu_t) <= J(a_t, mu_t)."""
    rng = np.random.default_rng(10)
    X = _mixture(rng, 800, comps=40)
    C = X[orc.kmeanspp(X, 32, seed=2)]
    a = orc.assign(X, C)
    prev = brute.objective(X, a, C)
    for _ in range(8):
        Cn, cnt = orc.update(X, a, C, "bf16")
        # exact means for the rounding penalty rho
        s = np.zeros((32, 128))
        np.add.at(s, a, X.astype(np.float64))
        m = np.where(cnt[:, None] > 0, s / np.maximum(cnt, 1)[:, None], Cn)
        rho = float((cnt[:, None] * (Cn.astype(np.float64) - m) ** 2).sum())
        j_upd = brute.objective(X, a, Cn)
        assert j_upd <= prev + rho + 1e-9 * prev
        # parallel-axis identity J(a, mu) = J(a, m) + sum n_c |mu - m|^2
        assert math.isclose(j_upd, brute.objective(X, a, m) + rho, rel_tol=1e-10)
        a_new = orc.assign(X, Cn)
        j_asg = brute.objective(X, a_new, Cn)
        assert j_asg <= j_upd + 1e-9 * j_upd
        a, C, prev = a_new, Cn, j_asg


# --------------------------------------------------------------------------
# Full build: layout invariants, value sums, brute-force Lloyd per segment.

def _small(dtype="bf16", n_ctx=68 + 3 * 96 + 37, seg=96, k=12, iters=3, B=2, H=2, G=3):
    w = synth.custom(90, dtype, B, H * G, H, n_ctx, seg, k, n_iters=iters, n_needles=3,
                     n_components=24)
    K, V, q = synth.gen_batch(w)
    d = oracle.make_desc(dtype, B, H, n_ctx, seg_len=seg, clusters_per_seg=k, n_iters=iters)
    return w, d, K, V, q


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_build_layout_invariants(orc, dtype):
    w, d, K, V, q = _small(dtype)
    idx = orc.build(d, K, V)
    ns, C, cap, T = orc.sizes(d)
    assert T == (8 if dtype == "bf16" else 4)
    parts = brute.partition(d.n_ctx, d.seg_len, d.clusters_per_seg)
    assert len(parts) == ns and sum(p[2] for p in parts) == C
    U = d.batch * d.n_kv_heads
    Kf = K.reshape(U, d.n_ctx, 128)
    Vf = V.reshape(U, d.n_ctx, 128)
    for u in range(U):
        sz, bo, st = idx["sizes"][u], idx["block_off"][u], idx["slot_token"][u]
        a = idx["assign"][u]
        assert sz.sum() == d.n_ctx - 68
        assert np.array_equal(np.diff(bo), (sz + T - 1) // T)
        assert bo[-1] <= cap
        seen = []
        for c in range(C):
            toks = st[bo[c] * T: bo[c] * T + sz[c]]
            assert np.all(np.diff(toks) > 0)             # ascending position
            assert np.all(a[toks - 4] == c)              # members of c
            assert np.all(st[bo[c] * T + sz[c]: bo[c + 1] * T] == -1)  # padding
            seen.extend(toks.tolist())
        assert sorted(seen) == list(range(4, d.n_ctx - 64))  # every token once
        assert np.all(st[bo[-1] * T:] == -1)
        used = st >= 0
        assert np.array_equal(idx["kblk"][u][used], Kf[u][st[used]])
        assert np.array_equal(idx["vblk"][u][used], Vf[u][st[used]])
        assert not idx["kblk"][u][~used].any() and not idx["vblk"][u][~used].any()
        # segments: each cluster's members lie in its own segment
        for (p0, n, cs, cb) in parts:
            assert np.all((a[p0 - 4: p0 - 4 + n] >= cb) & (a[p0 - 4: p0 - 4 + n] < cb + cs))
        # value sums: float64 sum rounded to float32
        vs = np.zeros((C, 128))
        np.add.at(vs, a, Vf[u][4: d.n_ctx - 64].astype(np.float64))
        assert np.array_equal(idx["vsum"][u], vs.astype(np.float32))
        steady = list(range(4)) + list(range(d.n_ctx - 64, d.n_ctx))
        assert np.array_equal(idx["steady_k"][u], Kf[u][steady])
        assert np.array_equal(idx["steady_v"][u], Vf[u][steady])


def test_build_equals_bruteforce_lloyd(orc):
    w, d, K, V, q = _small("bf16", iters=4)
    idx = orc.build(d, K, V)
    parts = brute.partition(d.n_ctx, d.seg_len, d.clusters_per_seg)
    U = d.batch * d.n_kv_heads
    Kf = K.reshape(U, d.n_ctx, 128)
    for u in range(U):
        b, h = divmod(u, d.n_kv_heads)
        for s, (p0, n, cs, cb) in enumerate(parts):
            X = Kf[u][p0: p0 + n]
            picks = orc.kmeanspp(X, cs, seed=0, b=b, l=0, h=h, s=s)
            C, a = brute.lloyd(X, X[picks], d.n_iters, "bf16")
            assert np.array_equal(idx["centroids"][u][cb: cb + cs], C)
            assert np.array_equal(idx["assign"][u][p0 - 4: p0 - 4 + n], a + cb)


def test_build_zero_iters_and_given_init(orc):
    w, d, K, V, q = _small("bf16", iters=0)
    idx0 = orc.build(d, K, V)
    # n_iters = 0: centroids are the k-means++ picks (copies of keys)
    U = d.batch * d.n_kv_heads
    Kf = K.reshape(U, d.n_ctx, 128)
    parts = brute.partition(d.n_ctx, d.seg_len, d.clusters_per_seg)
    p0, n, cs, cb = parts[0]
    picks = orc.kmeanspp(Kf[0][p0:p0 + n], cs, seed=0)
    assert np.array_equal(idx0["centroids"][0][:cs], Kf[0][p0 + picks])
    # given init + 2 iterations == k-means++ run with 2 iterations
    d2 = oracle.make_desc("bf16", d.batch, d.n_kv_heads, d.n_ctx, seg_len=d.seg_len,
                          clusters_per_seg=d.clusters_per_seg, n_iters=2)
    full = orc.build(d2, K, V)
    again = orc.build(d2, K, V, init=idx0["centroids"])
    for key in ("centroids", "sizes", "assign", "block_off", "slot_token"):
        assert np.array_equal(full[key], again[key])


# --------------------------------------------------------------------------
# Decode.

def _members(idx, u, T):
    bo, sz, st = idx["block_off"][u], idx["sizes"][u], idx["slot_token"][u]
    return [st[bo[c] * T: bo[c] * T + sz[c]] for c in range(len(sz))]


def test_select_matches_lexsort(orc):
    w, d, K, V, q = _small("bf16")
    idx = orc.build(d, K, V)
    ns, C, cap, T = orc.sizes(d)
    G = 3
    res = orc.decode(d, 6, 5, 9, idx, q)
    for u in range(d.batch * d.n_kv_heads):
        b, h = divmod(u, d.n_kv_heads)
        g = (q[b, h * G:(h + 1) * G].astype(np.float64) @ idx["centroids"][u].astype(np.float64).T).sum(0)
        # ranking key: the exact group score (bf16 products and their short
        # sums are exact in float64), larger first, lower id on ties
        order = np.lexsort((np.arange(C), -g))
        assert np.array_equal(res["sel"][u], order[:14])
        assert np.allclose(res["gkey"][u], g, rtol=1e-12, atol=1e-12)


def test_select_exact_key_breaks_float32_ties(orc):
    """Two centroids whose group scores differ by far less than float32
    resolution: the exact score decides their order (the higher-id cluster,
    whose score is larger by |Q_t| 2^-40, ranks first), not the cluster id."""
    w, d, K, V, q = _small("bf16")
    idx = orc.build(d, K, V)
    ns, C, cap, T = orc.sizes(d)
    G = 3
    c_lo, c_hi = 2, 7
    cent = idx["centroids"]
    for u in range(d.batch * d.n_kv_heads):
        b, h = divmod(u, d.n_kv_heads)
        Q = q[b, h * G:(h + 1) * G].astype(np.float64).sum(0)
        t = int(np.argmax(np.abs(Q)))
        cent[u, c_lo, t] = 0.0
        cent[u, c_hi] = cent[u, c_lo]
        cent[u, c_hi, t] = np.float32(math.copysign(2.0 ** -40, Q[t]))  # exact in bf16
        g = (q[b, h * G:(h + 1) * G].astype(np.float64) @ cent[u].astype(np.float64).T).sum(0)
        assert g[c_hi] > g[c_lo] and np.float32(g[c_hi]) == np.float32(g[c_lo])
    res = orc.decode(d, 6, C, 0, idx, q)
    for u in range(d.batch * d.n_kv_heads):
        sel = res["sel"][u].tolist()
        assert sel.index(c_hi) == sel.index(c_lo) - 1


def test_decode_equals_bruteforce_tripartite(orc):
    w, d, K, V, q = _small("bf16")
    idx = orc.build(d, K, V)
    ns, C, cap, T = orc.sizes(d)
    G, kr, ke = 3, 4, 10
    res = orc.decode(d, 6, kr, ke, idx, q)
    U = d.batch * d.n_kv_heads
    scale = 1 / math.sqrt(128)
    Kf, Vf = K.reshape(U, d.n_ctx, 128), V.reshape(U, d.n_ctx, 128)
    for u in range(U):
        b, h = divmod(u, d.n_kv_heads)
        mem = _members(idx, u, T)
        R, E = res["sel"][u][:kr], res["sel"][u][kr:]
        for j in range(G):
            ref = brute.tripartite(q[b, h * G + j], Kf[u], Vf[u], mem, idx["centroids"][u],
                                   R, E, 4, 64, scale)
            assert np.allclose(res["out"][b, h * G + j], ref, rtol=1e-6, atol=1e-7)
        # exec buffer: steady positions then R members in rank order
        exp_tok = list(range(4)) + list(range(d.n_ctx - 64, d.n_ctx)) + \
            [int(t) for c in R for t in mem[c]]
        assert res["n_exec"][u] == len(exp_tok)
        assert res["exec_tokens"][u][:len(exp_tok)].tolist() == exp_tok


def test_full_budget_equals_full_attention(orc):
    """K_r = C: the retrieval zone is every cluster -> plain attention (torch SDPA)."""
    import torch
    for dtype in ("bf16", "f32"):
        w, d, K, V, q = _small(dtype)
        idx = orc.build(d, K, V)
        ns, C, cap, T = orc.sizes(d)
        res = orc.decode(d, 6, C, 5, idx, q)
        G = 3
        for b in range(d.batch):
            for hq in range(6):
                h = hq // G
                Q = torch.from_numpy(q[b, hq].astype(np.float64))[None, None, None, :]
                Kt = torch.from_numpy(K[b, h].astype(np.float64))[None, None]
                Vt = torch.from_numpy(V[b, h].astype(np.float64))[None, None]
                ref = torch.nn.functional.scaled_dot_product_attention(Q, Kt, Vt)[0, 0, 0].numpy()
                assert np.allclose(res["out"][b, hq], ref, rtol=1e-10, atol=1e-12)


def test_singleton_clusters_estimation_is_exact(orc):
    """k = seg_len: every cluster is one token, its centroid is the key and its
    value sum is the value, so R + E covering all clusters is exact attention."""
    import torch
    n_ctx, seg = 68 + 2 * 16 + 5, 16
    w = synth.custom(91, "bf16", 1, 2, 1, n_ctx, seg, seg, n_iters=2, n_needles=2)
    K, V, q = synth.gen_batch(w)
    d = oracle.make_desc("bf16", 1, 1, n_ctx, seg_len=seg, clusters_per_seg=seg, n_iters=2)
    idx = orc.build(d, K, V)
    ns, C, cap, T = orc.sizes(d)
    assert np.all(idx["sizes"] == 1)
    res = orc.decode(d, 2, 3, C - 3, idx, q)
    for hq in range(2):
        Q = torch.from_numpy(q[0, hq].astype(np.float64))[None, None, None, :]
        ref = torch.nn.functional.scaled_dot_product_attention(
            Q, torch.from_numpy(K[0, 0].astype(np.float64))[None, None],
            torch.from_numpy(V[0, 0].astype(np.float64))[None, None])[0, 0, 0].numpy()
        assert np.allclose(res["out"][0, hq], ref, rtol=1e-10, atol=1e-12)


def test_estimation_jensen_lower_bound(orc):
    """n_c exp(<q, mean>/sqrt d) <= sum_i exp(<q, k_i>/sqrt d) for every cluster."""
    w, d, K, V, q = _small("bf16")
    idx = orc.build(d, K, V)
    ns, C, cap, T = orc.sizes(d)
    U = d.batch * d.n_kv_heads
    Kf = K.reshape(U, d.n_ctx, 128).astype(np.float64)
    for u in range(U):
        b, h = divmod(u, d.n_kv_heads)
        for c, m in enumerate(_members(idx, u, T)):
            if len(m) == 0:
                continue
            qv = q[b, h * 3].astype(np.float64)
            z = Kf[u][m] @ qv / math.sqrt(128)
            est = len(m) * math.exp(Kf[u][m].mean(0) @ qv / math.sqrt(128))
            assert est <= np.exp(z).sum() * (1 + 1e-12)


def test_needles_land_in_retrieval_zone(orc):
    """Diagnostic on the fp32 8K workload: the clusters holding needle keys are
    ranked into the retrieval zone."""
    w = synth.WORKLOADS[0]
    K, V, q = synth.gen_batch(w)
    d = oracle.make_desc("f32", 1, 1, w.n_ctx, n_iters=2)
    idx = orc.build(d, K, V)
    kr, ke = w.budgets()
    res = orc.decode(d, 4, kr, ke, idx, q)
    pos = synth.needle_positions(w, 0, 0, 0)
    needle_clusters = set(idx["assign"][0][pos - 4].tolist())
    assert needle_clusters <= set(res["sel"][0][:kr].tolist())
