"""Pins of the oracle's per-layer policy pieces: the layer plan against the
bands the pages print, dense decode attention against torch's SDPA in
float64, and recall@k against a brute-force ranking of every clustered token
plus its closed-form special cases."""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import brute, policy
from sparse_long_context_segmented_amd import synth


def test_banded_plan_reproduces_the_80_layer_example():
    """framerc blog section 3.3: layers 0-20 full attention, 21-60 hybrid,
    61 and up hybrid with a 30 % estimation share (an 80-layer model)."""
    modes = [policy.plan(policy.BANDED, l, 80, 131072) for l in range(80)]
    assert [l for l, m in enumerate(modes) if m[0] == policy.DENSE] == list(range(21))
    mid = {m for m in modes[21:61]}
    top = {m for m in modes[61:]}
    # 128K tokens at 16 tokens per cluster: 1.8 % -> 147, 23 % -> 1884, 30 % -> 2458
    assert mid == {(policy.HYBRID, 147, 1884)}
    assert top == {(policy.HYBRID, 147, 2458)}


def test_dense_first_two_layers_and_uniform_plans():
    """framerc blog section 4.3 problem 3: sparse attention off in the first
    two layers; the uniform plan is the section 2.1 budgets everywhere."""
    p = [policy.plan(policy.DENSE_FIRST2, l, 32, 1048576) for l in range(32)]
    assert p[0] == p[1] == (policy.DENSE, 0, 0)
    assert set(p[2:]) == {(policy.HYBRID, 1180, 15073)}
    assert {policy.plan(policy.UNIFORM, l, 32, 131072) for l in range(32)} == \
        {(policy.HYBRID, 147, 1884)}
    with pytest.raises(ValueError):
        policy.plan(policy.BANDED, 32, 32, 131072)


def test_banded_plan_scales_with_depth():
    """The bands as fractions of depth: at 32 layers, 80 l < 21 * 32 gives
    layers 0-8 dense and 80 l >= 61 * 32 gives layers 25-31 upper."""
    p = [policy.plan(policy.BANDED, l, 32, 131072) for l in range(32)]
    assert [l for l in range(32) if p[l][0] == policy.DENSE] == list(range(9))
    assert [l for l in range(32) if p[l][2] == 2458] == list(range(25, 32))


def _kvq(seed, B, H, G, N, dtype="bf16"):
    rng = np.random.default_rng([21, seed])
    r = (lambda x: brute.bf16(x)) if dtype == "bf16" else (lambda x: x.astype(np.float32))
    K = r(rng.standard_normal((B, H, N, 128)).astype(np.float32))
    V = r(rng.standard_normal((B, H, N, 128)).astype(np.float32))
    q = r(rng.standard_normal((B, H * G, 128)).astype(np.float32) * 2)
    return K, V, q


@pytest.mark.parametrize("B,H,G,N", [(1, 1, 1, 1), (1, 2, 4, 37), (2, 3, 2, 300)])
def test_dense_attention_equals_sdpa(B, H, G, N):
    K, V, q = _kvq(B * 100 + N, B, H, G, N)
    d = oracle.make_desc("bf16", B, H, N, seg_len=8192, clusters_per_seg=512, n_sink=0,
                         n_local=0)
    out = oracle.dense_attention(d, H * G, K, V, q)
    Kt = torch.from_numpy(K.astype(np.float64)).repeat_interleave(G, dim=1)
    Vt = torch.from_numpy(V.astype(np.float64)).repeat_interleave(G, dim=1)
    Q = torch.from_numpy(q.astype(np.float64))[:, :, None, :]
    ref = torch.nn.functional.scaled_dot_product_attention(Q, Kt, Vt)[:, :, 0].numpy()
    assert np.allclose(out, ref, rtol=1e-11, atol=1e-13)
    if N == 1:  # one token: the output is its value
        assert np.array_equal(out[0, 0], V[0, 0, 0].astype(np.float64))


def test_dense_attention_equal_keys_give_the_mean_value():
    K, V, q = _kvq(5, 1, 1, 2, 50)
    K[:] = K[:, :, :1]
    d = oracle.make_desc("bf16", 1, 1, 50, n_sink=0, n_local=0)
    out = oracle.dense_attention(d, 2, K, V, q)
    assert np.allclose(out[0], V[0, 0].astype(np.float64).mean(0)[None], rtol=1e-12, atol=1e-14)


def _index(seed=3, n_ctx=68 + 3 * 96 + 41, B=1, H=2, G=2):
    w = synth.custom(40 + seed, "bf16", B, H * G, H, n_ctx, 96, 12, n_iters=2, n_needles=4,
                     n_components=16)
    K, V, q = synth.gen_batch(w)
    d = oracle.make_desc("bf16", B, H, n_ctx, seg_len=96, clusters_per_seg=12, n_iters=2)
    return d, K, V, q, oracle.build(d, K, V)


@pytest.mark.parametrize("k", [1, 20, 100])
def test_recall_equals_bruteforce_ranking(k):
    """Every clustered token scored by numpy in float64 and ranked by
    np.lexsort (score descending, position ascending); the oracle's top-k and
    recall must match it, for a retrieval zone taken from decode."""
    d, K, V, q, idx = _index()
    k_r = 5
    res = oracle.decode(d, 4, k_r, 10, idx, q)
    R = res["sel"][:, :k_r]
    rc = oracle.recall(d, 4, idx, q, R, k)
    N, n_idx = d.n_ctx, d.n_ctx - 68
    for u in range(2):
        h = u
        pos = np.arange(4, 4 + n_idx)
        Ku = K[0, h, 4:4 + n_idx].astype(np.float64)
        clus = idx["assign"][u]
        for j in range(2):
            s = Ku @ q[0, 2 * h + j].astype(np.float64)
            order = np.lexsort((pos, -s))[:k]
            assert rc["top"][0, 2 * h + j].tolist() == pos[order].tolist()
            assert np.allclose(rc["top_score"][0, 2 * h + j], s[order], rtol=0, atol=1e-12)
            want = np.isin(clus[order], R[u]).sum() / k
            assert rc["recall"][0, 2 * h + j] == want
    del N


def test_recall_special_cases():
    d, K, V, q, idx = _index(seed=4)
    ns, C, cap, T = oracle.sizes(d)
    U, n_idx = 2, d.n_ctx - 68
    all_c = np.tile(np.arange(C, dtype=np.int32), (U, 1))
    assert np.all(oracle.recall(d, 4, idx, q, all_c, 100)["recall"] == 1.0)
    none = np.zeros((U, 0), np.int32)
    assert np.all(oracle.recall(d, 4, idx, q, none, 100)["recall"] == 0.0)
    # k = every clustered token: the recall is R's share of the tokens
    R = np.array([[0, 3, 7], [1, 2, 11]], np.int32)
    r = oracle.recall(d, 4, idx, q, R, n_idx)["recall"]
    for u in range(U):
        share = idx["sizes"][u][R[u]].sum() / n_idx
        assert np.allclose(r[0, 2 * u:2 * u + 2], share, rtol=0, atol=1e-15)
    with pytest.raises(ValueError):
        oracle.recall(d, 4, idx, q, R, n_idx + 1)
    with pytest.raises(ValueError):
        oracle.recall(d, 4, idx, q, R, 0)


def test_recall_of_needle_queries_is_high_with_the_standard_budget():
    """The synthetic needles stand for the tokens a query must find: with the
    pages' budgets the retrieval zone holds most of each query's best tokens
    (a diagnostic on the generator, not a bound from the pages)."""
    w = synth.custom(47, "bf16", 1, 4, 1, 8192 + 68, 8192, 512, n_iters=3, n_needles=32)
    K, V, q = synth.gen_batch(w)
    d = oracle.make_desc("bf16", 1, 1, w.n_ctx, n_iters=3)
    idx = oracle.build(d, K, V)
    k_r = int(math.floor(0.018 * w.n_ctx * 512 / 8192 + 0.5))
    res = oracle.decode(d, 4, k_r, 0, idx, q)
    r = oracle.recall(d, 4, idx, q, res["sel"][:, :k_r], 32)
    assert r["recall"].min() >= 0.85, r["recall"]
