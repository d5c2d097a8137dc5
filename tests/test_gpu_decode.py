"""GPU parity of wi_decode_attention against the oracle, on an index built by
the oracle and uploaded to the device (so decode is checked independently of
the GPU build). Selection (rank order) and the execution-buffer token list are
compared exactly; the attention output to the dtype's tolerance:
2e-3 max relative error for bf16 inputs, 1e-5 for fp32."""
import numpy as np
import pytest
import torch

import oracle
from sparse_long_context_segmented_amd import synth, wi

from parity import check_selection, exec_reference, rel_err, upload_q

pytestmark = pytest.mark.gpu

TOL = {"bf16": 2e-3, "f32": 1e-5}


def _run(w, k_r, k_e, n_iters=2, batch=None, want_debug=True, scale=0.0, wg=0, mutate=None):
    print(f"[decode parity] {w.name} dtype={w.dtype} B={w.batch} H={w.n_kv_heads} "
          f"G={w.group} N={w.n_ctx} seg={w.seg_len} k={w.clusters_per_seg} "
          f"K_r={k_r} K_e={k_e} wg={wg}", flush=True)
    K, V, q = synth.gen_batch(w)
    od = oracle.make_desc(w.dtype, w.batch, w.n_kv_heads, w.n_ctx, seg_len=w.seg_len,
                          clusters_per_seg=w.clusters_per_seg, n_iters=n_iters)
    idx = oracle.build(od, K, V)
    if mutate is not None:
        mutate(idx)
    ns, C, cap, T = oracle.sizes(od)
    gd = wi.make_desc(w.dtype, w.batch, w.n_kv_heads, w.n_ctx, seg_len=w.seg_len,
                      clusters_per_seg=w.clusters_per_seg, n_iters=n_iters)
    gix = wi.index_from_host(gd, idx)
    qt = upload_q(q, w.dtype)
    U = w.batch * w.n_kv_heads
    k_e_eff = min(k_e, C - k_r)
    M = k_r + k_e_eff
    dd = wi.DecodeDesc(w.n_q_heads, k_r, k_e, scale, wg)
    sel = exe = nexe = None
    exec_cap = 68 + int(np.sort(idx["sizes"], axis=1)[:, ::-1][:, :k_r].sum(axis=1).max(initial=0))
    if want_debug:
        sel = torch.full((U, max(M, 1)), -5, dtype=torch.int32, device="cuda")
        exe = torch.full((U, exec_cap), -5, dtype=torch.int32, device="cuda")
        nexe = torch.full((U,), -5, dtype=torch.int32, device="cuda")
    out = wi.decode_attention(gix, dd, qt, sel_ids=sel, exec_tokens=exe, n_exec=nexe)
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    ref = oracle.decode(od, w.n_q_heads, k_r, k_e, idx, q, scale=scale)
    res = dict(out=out, ref=ref, idx=idx, gix=gix, qt=qt, dd=dd, od=od, q=q, C=C, T=T)
    if want_debug:
        selg = sel.cpu().numpy()[:, :M]
        res["sel"] = selg
        res["mism"] = check_selection(selg, ref["gkey"], k_r)
        # attention reference on the GPU's own zones (identical unless near-ties)
        r2 = oracle.attend_sets(od, w.n_q_heads, idx, q, selg[:, :k_r], selg[:, k_r:],
                                scale=scale)
        res["err"] = rel_err(out, r2)
        ex_ref = exec_reference(idx, selg, k_r, w.n_ctx, T)
        ne = nexe.cpu().numpy()
        ex = exe.cpu().numpy()
        for u in range(U):
            assert ne[u] == len(ex_ref[u])
            n = min(ne[u], exec_cap)
            assert ex[u][:n].tolist() == ex_ref[u][:n]
    else:
        res["err"] = rel_err(out, ref["out"])
    print(f"  rel err {res['err']:.3e}  near-tie reorders {res.get('mism', 0)}", flush=True)
    return res


SMALL = synth.custom(201, "bf16", 2, 6, 2, 68 + 5 * 1024 + 333, 1024, 64, n_needles=4)


def test_decode_small_bf16_multitile():
    r = _run(SMALL, 9, 88)
    assert r["err"] <= TOL["bf16"]
    # with no near-tie reorder the oracle's own selection gives the same answer
    if r["mism"] == 0:
        assert rel_err(r["out"], r["ref"]["out"]) <= TOL["bf16"]


def test_decode_fp32_8k():
    w = synth.WORKLOADS[0]
    k_r, k_e = w.budgets()
    r = _run(w, k_r, k_e)
    assert r["err"] <= TOL["f32"]


@pytest.mark.parametrize("k_r,k_e", [(0, 50), (9, 0), (0, 0), (30, 10_000)])
def test_decode_budget_edges(k_r, k_e):
    r = _run(SMALL, k_r, k_e)
    assert r["err"] <= TOL["bf16"]


def test_decode_full_budget_is_full_attention():
    """K_r = C: tripartite attention equals attention over every token."""
    w = synth.custom(202, "bf16", 1, 4, 1, 68 + 2 * 512 + 77, 512, 32, n_needles=2)
    od = oracle.make_desc("bf16", 1, 1, w.n_ctx, seg_len=512, clusters_per_seg=32)
    C = oracle.sizes(od)[1]
    r = _run(w, C, 0)
    K, V, q = synth.gen_batch(w)
    Kt = torch.from_numpy(K[0, 0].astype(np.float64))
    Vt = torch.from_numpy(V[0, 0].astype(np.float64))
    for hq in range(4):
        Q = torch.from_numpy(q[0, hq].astype(np.float64))[None, None, None, :]
        full = torch.nn.functional.scaled_dot_product_attention(Q, Kt[None, None], Vt[None, None])
        assert rel_err(r["out"][0, hq], full[0, 0, 0].numpy()) <= TOL["bf16"]


@pytest.mark.parametrize("G", [1, 2, 7, 8, 16])
def test_decode_group_sizes(G):
    w = synth.custom(203 + G, "bf16", 2, 2 * G, 2, 68 + 3 * 512 + 100, 512, 32, n_needles=3,
                     anisotropic=(G == 7))
    r = _run(w, 5, 40)
    assert r["err"] <= TOL["bf16"]


def test_decode_explicit_scale_and_no_debug():
    r = _run(SMALL, 9, 88, want_debug=False, scale=0.05)
    assert r["err"] <= TOL["bf16"]


def test_decode_deterministic():
    r = _run(SMALL, 9, 88)
    outs = []
    for _ in range(3):
        o = wi.decode_attention(r["gix"], r["dd"], r["qt"])
        torch.cuda.synchronize()
        outs.append(o.cpu().numpy())
    assert np.array_equal(outs[0].view(np.uint32), r["out"].view(np.uint32))
    assert all(np.array_equal(outs[0], o) for o in outs[1:])


# 562 clusters per unit (four segments of 128 and a short one of 50): with one
# workgroup per unit its own clusters come in two chunks of 512, and K_r = 400
# gives it thousands of retrieved tokens (many rounds); three workgroups give
# each an interleaved share with a partial last group of 16 ids.
MULTI = synth.custom(220, "bf16", 1, 8, 2, 68 + 4 * 1024 + 50, 1024, 128, n_needles=4)


@pytest.mark.parametrize("wg", [1, 3, 64])
def test_decode_multichunk_and_workgroup_counts(wg):
    r = _run(MULTI, 400, 150, wg=wg)
    assert r["C"] == 562
    assert r["err"] <= TOL["bf16"]


def test_decode_multichunk_fp32():
    w = synth.custom(221, "f32", 1, 4, 1, 68 + 4 * 1024 + 50, 1024, 128, n_needles=4)
    r = _run(w, 37, 300, wg=1)
    assert r["err"] <= TOL["f32"]


# A unit count that is a multiple of 8 (batch 4 x 2 KV heads, and batch 8 x 2)
# switches the fused kernel to its XCD-aware placement (unit u's workgroups
# all on XCD u mod 8). Selection, execution-buffer lists and outputs are
# compared on every unit.
XCD8 = synth.custom(250, "bf16", 4, 8, 2, 68 + 3 * 1024 + 200, 1024, 64, n_needles=4)
XCD16 = synth.custom(251, "bf16", 8, 4, 2, 68 + 2 * 1024 + 77, 1024, 64, n_needles=3)


@pytest.mark.parametrize("wg", [0, 1, 3])
def test_decode_xcd_placement_eight_units(wg):
    r = _run(XCD8, 9, 88, wg=wg)
    assert r["sel"].shape[0] == 8
    assert r["err"] <= TOL["bf16"]


def test_decode_xcd_placement_sixteen_units():
    r = _run(XCD16, 7, 60, wg=2)
    assert r["sel"].shape[0] == 16
    assert r["err"] <= TOL["bf16"]


# More clusters per unit than one LDS pass of keys holds (8192): 17 segments
# of 1024 tokens with 512 clusters each, plus a short one -> C = 8714. The
# keys are staged in two passes and, with two workgroups per unit, each owns
# about 4357 clusters (nine chunks).
LARGE_C = synth.custom(230, "bf16", 1, 8, 2, 68 + 17 * 1024 + 10, 1024, 512, n_needles=4)


@pytest.mark.parametrize("wg", [0, 2])
def test_decode_more_clusters_than_one_key_pass(wg):
    r = _run(LARGE_C, 300, 2000, n_iters=1, wg=wg)
    assert r["C"] == 8714
    assert r["err"] <= TOL["bf16"]


def _tie_centroids(idx):
    """Unit 0: every centroid equal (every ranking key ties); unit 1: the first
    200 centroids equal. Selection then goes by cluster id within the ties,
    and the pivot's histogram bin holds more keys than one wave ranks."""
    c = idx["centroids"]
    c[0, :] = c[0, 0]
    c[1, :200] = c[1, 0]


@pytest.mark.parametrize("k_r,k_e", [(9, 88), (150, 40)])
def test_decode_tied_keys(k_r, k_e):
    r = _run(SMALL, k_r, k_e, mutate=_tie_centroids)
    assert r["err"] <= TOL["bf16"]
    sel = r["sel"]
    assert sel[0].tolist() == list(range(k_r + min(k_e, r["C"] - k_r)))


@pytest.mark.parametrize("G", [7, 16])
def test_decode_gathered_lists_over_several_passes(G):
    """More than 8192 clusters per unit and two workgroups per unit: each
    workgroup owns about 4357 clusters (nine 512-cluster chunks), so the item
    lists are gathered over several passes of two chunks (groups of 5-8
    heads) or one (larger groups)."""
    w = synth.custom(240 + G, "bf16", 1, 2 * G, 2, 68 + 17 * 1024 + 10, 1024, 512, n_needles=4,
                     anisotropic=(G == 7))
    r = _run(w, 300, 2000, n_iters=1, wg=2)
    assert r["C"] == 8714
    assert r["err"] <= TOL["bf16"]


def test_decode_tied_keys_more_clusters_than_one_key_pass():
    def tie(idx):
        c = idx["centroids"]
        c[0, :] = c[0, 0]
    r = _run(LARGE_C, 300, 2000, n_iters=1, mutate=tie)
    assert r["err"] <= TOL["bf16"]
    assert r["sel"][0].tolist() == list(range(2300))


def _tie_to_pivots(w, k_r, k_e, n_tie):
    """Every unit: the n_tie clusters ranked right after each pivot (the
    K_r-th and the (K_r + K_e)-th ranked cluster of the exact group key) get
    the pivot's centroid, so each pivot's histogram bin holds more than 64
    keys (one wave's worth) but at most 256, all tied with the pivot."""
    _, _, q = synth.gen_batch(w)
    G = w.group

    def mutate(idx):
        c = idx["centroids"]
        for u in range(c.shape[0]):
            b, h = divmod(u, w.n_kv_heads)
            Q = q[b, h * G:(h + 1) * G].astype(np.float64).sum(axis=0)
            order = np.lexsort((np.arange(c.shape[1]), -(c[u].astype(np.float64) @ Q)))
            for m in (k_r, k_r + k_e):
                piv = order[m - 1]
                c[u, order[m:m + n_tie]] = c[u, piv]
    return mutate


@pytest.mark.parametrize("w,k_r,k_e", [(SMALL, 9, 88), (LARGE_C, 300, 2000)],
                         ids=["one-key-pass", "two-key-passes"])
def test_decode_pivot_bins_beyond_one_wave(w, k_r, k_e):
    r = _run(w, k_r, k_e, n_iters=1, mutate=_tie_to_pivots(w, k_r, k_e, 100))
    assert r["err"] <= TOL["bf16"]


def test_decode_graph_replay_matches_eager():
    """A decode call captured in a HIP graph and replayed several times, with
    eager decode calls of another query between the replays, gives the eager
    output bit for bit on every replay."""
    r = _run(SMALL, 9, 88, want_debug=False)
    gix, dd, qt = r["gix"], r["dd"], r["qt"]
    q2 = torch.flip(qt, dims=[1]).contiguous()
    eager = wi.decode_attention(gix, dd, qt)
    torch.cuda.synchronize()
    ref = eager.cpu().numpy().view(np.uint32).copy()
    out = torch.empty_like(eager)
    ws = torch.empty(wi.decode_sizes(gix.desc, dd), dtype=torch.uint8, device="cuda")
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        wi.decode_attention(gix, dd, qt, out=out, ws=ws)
    for _ in range(3):
        out.zero_()
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy().view(np.uint32), ref)
        other = wi.decode_attention(gix, dd, q2, ws=ws)  # eager work on the same workspace
        torch.cuda.synchronize()
        assert not np.array_equal(other.cpu().numpy().view(np.uint32), ref)


def test_timing_hook_records_decode_launches_and_keeps_outputs():
    """With the measurement hook on, a decode call records its two launches
    (score, then select_attend) with positive durations, and its output is
    bit-identical to the same call without the hook."""
    w = synth.custom(2100, "bf16", 1, 8, 2, 68 + 2 * 512 + 40, 512, 32)
    K, V, q = synth.gen_batch(w)
    gd = wi.make_desc("bf16", w.batch, w.n_kv_heads, w.n_ctx, seg_len=w.seg_len,
                      clusters_per_seg=w.clusters_per_seg, n_iters=2)
    dev = torch.device("cuda:0")
    ix = wi.build_index(gd, torch.from_numpy(K).to(dev, torch.bfloat16),
                        torch.from_numpy(V).to(dev, torch.bfloat16))
    qt = torch.from_numpy(q).to(dev, torch.bfloat16)
    dd = wi.DecodeDesc(w.n_q_heads, 3, 20, 0.0, 0)
    plain = wi.decode_attention(ix, dd, qt).clone()
    torch.cuda.synchronize()
    wi.timing_start()
    timed = wi.decode_attention(ix, dd, qt)
    recs = wi.timing_stop()
    assert [n for n, _ in recs] == ["score", "select_attend"], recs
    assert all(ms > 0.0 for _, ms in recs), recs
    assert torch.equal(timed, plain)


def _random_cases(n, seed=20261203):
    """Seeded random small shapes: dtype, batch, KV heads, group size, segment
    length (with a ragged last segment), clusters per segment, budgets and
    workgroups per unit."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        dtype = "f32" if i % 5 == 4 else "bf16"
        B, H = int(rng.integers(1, 4)), int(rng.choice([1, 2, 3, 5]))
        G = int(rng.choice([1, 2, 3, 4, 5, 7, 8, 16]))
        seg = int(rng.choice([64, 96, 128, 256, 1000]))
        k = int(rng.integers(1, min(64, seg) + 1))
        n_idx = int(rng.integers(1, 5 * seg + 1))
        full, rem = divmod(n_idx, seg)
        C = full * min(k, seg) + (min(k, rem) if rem else 0)
        k_r = int(rng.integers(0, C + 1))
        k_e = int(rng.integers(0, C + 1))
        wg = int(rng.choice([0, 1, 3]))
        cases.append((i, dtype, B, H, G, seg, k, 68 + n_idx, k_r, k_e, wg))
    return cases


@pytest.mark.parametrize("case", _random_cases(16), ids=lambda c: f"rand{c[0]}")
def test_decode_random_small_shapes(case):
    """Decode parity on seeded random small shapes (selection, execution list
    and output against the oracle, as in every decode test)."""
    i, dtype, B, H, G, seg, k, n_ctx, k_r, k_e, wg = case
    w = synth.custom(700 + i, dtype, B, H * G, H, n_ctx, seg, k, n_needles=2)
    r = _run(w, k_r, k_e, wg=wg)
    assert r["err"] <= TOL[dtype]
