"""GPU parity of decode-time growth: wi_append_token, wi_extend_index and
wi_decode_attention over pending tokens, step by step against the oracle.

Both sides start from their own build of the same seeded prefix (checked bit
for bit), then take the stream's next tokens one decode step at a time, each
on its own index: the oracle with oracle.append / oracle.extend, the GPU with
the library's calls. After every step the GPU's steady and pending rows must
equal the oracle's bit for bit, and after every extension every index array
must. Every checked step decodes a fresh query on both sides: the GPU's
selection must equal the oracle's exact ranking up to counted near-ties, its
execution list must be steady, pending, then retrieved members, and its output
must be within the decode tolerance of the oracle's tripartite attention over
the GPU's zones (2e-3 relative for bf16, 1e-5 for fp32).
"""
import numpy as np
import pytest
import torch

import oracle
from sparse_long_context_segmented_amd import synth, wi

from parity import (assert_index_equal, check_selection, exec_reference, index_to_host, rel_err,
                    upload_kv, upload_q)

pytestmark = pytest.mark.gpu

TOL = {"bf16": 2e-3, "f32": 1e-5}


def _round(x, dtype):
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).to(torch.float32).numpy()


def _query(q, step, dtype):
    """The decode step's query: the workload's query plus seeded noise."""
    rng = np.random.default_rng([7, step])
    return _round(q + 0.5 * rng.standard_normal(q.shape, dtype=np.float32), dtype)


class Stream:
    """The GPU index and the oracle's, advanced together."""

    def __init__(self, w, K, V, n_ctx, n_sink=4, n_local=64):
        self.w, self.K, self.V = w, K, V
        self.n_sink, self.n_local = n_sink, n_local
        self.n_st = n_sink + n_local
        self.T = 8 if w.dtype == "bf16" else 4
        kw = dict(seg_len=w.seg_len, clusters_per_seg=w.clusters_per_seg, n_sink=n_sink,
                  n_local=n_local, n_iters=w.n_iters)
        gd = wi.make_desc(w.dtype, w.batch, w.n_kv_heads, n_ctx, **kw)
        self.od = oracle.make_desc(w.dtype, w.batch, w.n_kv_heads, n_ctx, **kw)
        K0 = np.ascontiguousarray(K[:, :, :n_ctx])
        V0 = np.ascontiguousarray(V[:, :, :n_ctx])
        kt, vt = upload_kv(K0, V0, w.dtype)
        self.ix = wi.build_index(gd, kt, vt)
        torch.cuda.synchronize()
        del kt, vt
        self.oidx = oracle.build(self.od, K0, V0)
        self.check_index()
        self.extensions = 0
        self.reorders = 0
        self.worst = 0.0

    def check_index(self):
        assert_index_equal(index_to_host(self.ix), self.oidx, n_st=self.n_st)

    def check_rows(self):
        """Steady rows and the pending rows in use, bit for bit."""
        U = self.w.batch * self.w.n_kv_heads
        n = self.od.n_pending
        pairs = [(self.ix.steady_k, "steady_k", self.n_st), (self.ix.steady_v, "steady_v",
                                                             self.n_st)]
        if n:
            pairs += [(self.ix.pend_k, "pend_k", n), (self.ix.pend_v, "pend_v", n)]
        for t, key, rows in pairs:
            a = t[:, :rows].float().cpu().numpy().reshape(U, rows, 128)
            b = np.ascontiguousarray(self.oidx[key], dtype=np.float32)[:, :rows]
            assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), key

    def step(self):
        """One appended token per sequence (extending first when full)."""
        if self.od.n_pending == self.od.seg_len:
            self.od, self.oidx = oracle.extend(self.od, self.oidx)
            self.ix = wi.extend_index(self.ix)
            torch.cuda.synchronize()
            assert (self.ix.desc.n_ctx, self.ix.desc.n_pending) == (self.od.n_ctx, 0)
            self.check_index()
            self.extensions += 1
        p = self.od.n_ctx
        kn = np.ascontiguousarray(self.K[:, :, p])
        vn = np.ascontiguousarray(self.V[:, :, p])
        self.od = oracle.append(self.od, self.oidx, kn, vn)
        self.ix = wi.append_token(self.ix, upload_q(kn, self.w.dtype), upload_q(vn, self.w.dtype))
        assert (self.ix.desc.n_ctx, self.ix.desc.n_pending) == (self.od.n_ctx, self.od.n_pending)

    def decode(self, q, k_r, k_e, check_plain=False):
        w = self.w
        Hq = w.n_q_heads
        U = w.batch * w.n_kv_heads
        C = self.ix.cluster_size.shape[1]
        M = k_r + min(k_e, C - k_r)
        dd = wi.DecodeDesc(Hq, k_r, k_e, 0.0)
        qt = upload_q(q, w.dtype)
        exec_cap = self.n_st + self.od.n_pending + int(
            self.ix.cluster_size.topk(k_r, dim=1).values.sum(dim=1).max())
        sel = torch.full((U, M), -5, dtype=torch.int32, device="cuda")
        exe = torch.full((U, exec_cap), -5, dtype=torch.int32, device="cuda")
        nexe = torch.full((U,), -5, dtype=torch.int32, device="cuda")
        out = wi.decode_attention(self.ix, dd, qt, sel_ids=sel, exec_tokens=exe, n_exec=nexe)
        if check_plain:
            plain = wi.decode_attention(self.ix, dd, qt)
            torch.cuda.synchronize()
            assert torch.equal(out, plain), "debug outputs changed the attention output"
        torch.cuda.synchronize()
        out, sel = out.cpu().numpy(), sel.cpu().numpy()
        exe, nexe = exe.cpu().numpy(), nexe.cpu().numpy()
        r = oracle.decode(self.od, Hq, k_r, k_e, self.oidx, q)
        self.reorders += check_selection(sel, r["gkey"], k_r)
        ref = oracle.attend_sets(self.od, Hq, self.oidx, q, sel[:, :k_r], sel[:, k_r:])
        e = rel_err(out, ref)
        assert e <= TOL[w.dtype], (self.od.n_ctx, self.od.n_pending, e)
        self.worst = max(self.worst, e)
        ex_ref = exec_reference(self.oidx, sel, k_r, self.od.n_ctx, self.T, self.n_sink,
                                self.n_local, self.od.n_pending)
        for u in range(U):
            assert nexe[u] == len(ex_ref[u]), u
            assert exe[u][:nexe[u]].tolist() == ex_ref[u], u


@pytest.mark.parametrize("dtype,n_sink,n_local", [("bf16", 4, 64), ("f32", 4, 64),
                                                  ("bf16", 0, 0), ("bf16", 4, 0)])
def test_stream_small_every_step(dtype, n_sink, n_local):
    """A prefix whose last built segment is short, then 2 segments + 30 tokens
    arriving one per step (two extensions), every step checked. Without a
    local window the new token is pending at once."""
    seg, k = 96, 12
    n_ctx = 68 + 3 * seg + 41
    n_new = 2 * seg + 30
    w = synth.custom(31, dtype, 2, 4, 2, n_ctx + n_new, seg, k, n_iters=3, n_needles=3,
                     n_components=24)
    K, V, q = synth.gen_batch(w)
    s = Stream(w, K, V, n_ctx, n_sink, n_local)
    for t in range(n_new):
        s.step()
        s.check_rows()
        s.decode(_query(q, t, dtype), 3, 9, check_plain=(t % 50 == 0))
    assert s.extensions == 2
    print(f"  {dtype} sink {n_sink} local {n_local}: {n_new} steps within {s.worst:.3e}, "
          f"near-tie reorders {s.reorders}", flush=True)


def test_stream_aligned_extension_equals_fresh_gpu_build():
    """Built range a whole number of segments: seg_len appends and one
    extension give, bit for bit, the index the GPU builds from scratch for
    the longer stream."""
    seg, k = 128, 16
    n_ctx = 68 + 2 * seg
    w = synth.custom(32, "bf16", 1, 8, 4, n_ctx + seg + 1, seg, k, n_iters=4, n_needles=3,
                     n_components=24)
    K, V, q = synth.gen_batch(w)
    s = Stream(w, K, V, n_ctx)
    for _ in range(seg + 1):
        s.step()
    assert s.extensions == 1 and s.od.n_pending == 1
    n2 = n_ctx + seg
    gd = wi.make_desc("bf16", 1, 4, n2, seg_len=seg, clusters_per_seg=k, n_iters=4)
    kt, vt = upload_kv(np.ascontiguousarray(K[:, :, :n2]), np.ascontiguousarray(V[:, :, :n2]),
                       "bf16")
    fresh = index_to_host(wi.build_index(gd, kt, vt))
    # the grown index before its last append: same clusters, blocks, assignment
    grown = index_to_host(s.ix)
    for key in ("centroids", "sizes", "vsum", "block_off", "kblk", "vblk", "slot_token",
                "assign"):
        assert grown[key].shape == fresh[key].shape, key
        assert np.array_equal(grown[key], fresh[key]), key


def test_append_refuses_a_full_pending_segment():
    seg, k = 64, 8
    n_ctx = 68 + seg
    w = synth.custom(33, "bf16", 1, 2, 1, n_ctx + seg + 1, seg, k, n_iters=2, n_needles=2,
                     n_components=16)
    K, V, q = synth.gen_batch(w)
    s = Stream(w, K, V, n_ctx)
    for _ in range(seg):
        s.step()
    assert s.od.n_pending == seg
    kn = upload_q(np.ascontiguousarray(K[:, :, s.od.n_ctx]), "bf16")
    with pytest.raises(wi.WIError):
        wi.append_token(s.ix, kn, kn)
    with pytest.raises(wi.WIError):
        wi.extend_sizes(wi.make_desc("bf16", 1, 1, n_ctx, seg_len=seg, clusters_per_seg=k))


@pytest.mark.slow
@pytest.mark.timeout(900)
def test_stream_llama8b_128k_batch1():
    """The Llama3.1-8B-shaped 128K layer at batch 1 (8 KV heads, 32 query
    heads, segments of 8192 tokens with 512 clusters): 64 consecutive decode
    steps each checked, then appends up to a full pending segment (8192
    pending tokens, checked at 4096 and 8192), the extension (every index
    array bit-exact against the oracle's own extension), and 16 more checked
    steps on the grown index."""
    n_ctx = 131072
    seg = 8192
    w = synth.custom(12, "bf16", 1, 32, 8, n_ctx + seg + 16, seg, 512, n_iters=10,
                     n_needles=32)
    K, V, q = synth.gen_batch(w)
    per_tok = 512 / seg
    k_r = int(np.floor(0.018 * n_ctx * per_tok + 0.5))
    k_e = int(np.floor(0.23 * n_ctx * per_tok + 0.5))
    print(f"[stream 128K b1] build + oracle build, K_r {k_r} K_e {k_e}", flush=True)
    s = Stream(w, K, V, n_ctx)
    for t in range(64):
        s.step()
        s.check_rows()
        s.decode(_query(q, t, "bf16"), k_r, k_e, check_plain=(t % 16 == 0))
    print(f"  64 steps within {s.worst:.3e}, near-tie reorders {s.reorders}", flush=True)
    for t in range(64, seg):
        s.step()
        if s.od.n_pending in (4096, seg):
            s.check_rows()
            s.decode(_query(q, t, "bf16"), k_r, k_e, check_plain=True)
            print(f"  pending {s.od.n_pending}: within {s.worst:.3e}", flush=True)
    for t in range(seg, seg + 16):
        s.step()
        s.check_rows()
        s.decode(_query(q, t, "bf16"), k_r, k_e)
    assert s.extensions == 1
    print(f"  extension bit-exact; 16 steps after it within {s.worst:.3e}, near-tie "
          f"reorders {s.reorders}", flush=True)


@pytest.mark.parametrize("n_sink,n_local,chunks", [(4, 64, [1, 5, 63, 64, 65, 130, 7]),
                                                   (4, 0, [3, 96, 40]), (0, 64, [200, 1])])
def test_append_tokens_equals_token_by_token_oracle(n_sink, n_local, chunks):
    """Chunks of several sizes (shorter, equal and longer than the local
    window) through wi_append_tokens (via prefill_chunk, which extends at
    every segment boundary) against the oracle appending one token at a time:
    steady and pending rows after every chunk, every array after the run."""
    seg, k = 96, 12
    n_ctx = n_sink + n_local + 2 * seg + 17
    total = sum(chunks)
    w = synth.custom(34, "bf16", 2, 4, 2, n_ctx + total, seg, k, n_iters=2, n_needles=3,
                     n_components=24)
    K, V, q = synth.gen_batch(w)
    s = Stream(w, K, V, n_ctx, n_sink, n_local)
    for m in chunks:
        p = s.od.n_ctx
        kc = upload_q(np.ascontiguousarray(K[:, :, p:p + m]), "bf16")
        vc = upload_q(np.ascontiguousarray(V[:, :, p:p + m]), "bf16")
        s.ix = wi.prefill_chunk(s.ix, kc, vc)
        for t in range(m):
            if s.od.n_pending == s.od.seg_len:
                s.od, s.oidx = oracle.extend(s.od, s.oidx)
            q0 = s.od.n_ctx
            s.od = oracle.append(s.od, s.oidx, K[:, :, q0], V[:, :, q0])
        if s.od.n_pending == s.od.seg_len:
            s.od, s.oidx = oracle.extend(s.od, s.oidx)
        torch.cuda.synchronize()
        assert (s.ix.desc.n_ctx, s.ix.desc.n_pending) == (s.od.n_ctx, s.od.n_pending)
        s.check_rows()
    s.check_index()


@pytest.mark.slow
@pytest.mark.timeout(600)
def test_prefill_chunked_build_equals_one_shot_llama8b_128k():
    """Prefill-side fusion at the Llama3.1-8B 128K shape: after a one-segment
    build, 4096-token prefill chunks are fed in and every segment is
    clustered as soon as it fills; with 16 segments in all the final index
    equals the one-shot build of the same 131 140 tokens bit for bit."""
    import time
    seg = 8192
    N = 68 + 16 * seg
    w = synth.custom(13, "bf16", 1, 32, 8, N, seg, 512, n_iters=10, n_needles=32)
    K, V, q = synth.gen_batch(w)
    kt, vt = upload_kv(K, V, "bf16")
    gd = wi.make_desc("bf16", 1, 8, N)
    one = wi.build_index(gd, kt, vt)
    n0 = 68 + seg
    d0 = wi.make_desc("bf16", 1, 8, n0)
    ix = wi.build_index(d0, kt[:, :, :n0].contiguous(), vt[:, :, :n0].contiguous())
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    p, chunks = n0, 0
    while p < N:
        m = min(4096, N - p)
        ix = wi.prefill_chunk(ix, kt[:, :, p:p + m].contiguous(), vt[:, :, p:p + m].contiguous())
        p += m
        chunks += 1
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    assert (ix.desc.n_ctx, ix.desc.n_pending) == (N, 0)
    a, b = index_to_host(ix), index_to_host(one)
    for key in ("centroids", "sizes", "vsum", "block_off", "kblk", "vblk", "slot_token",
                "steady_k", "steady_v", "assign"):
        assert a[key].shape == b[key].shape, key
        assert np.array_equal(a[key], b[key]), key
    print(f"  {chunks} chunks, 15 segments clustered as they filled: {dt * 1e3:.0f} ms "
          f"(index bit-identical to the one-shot build)", flush=True)


def _random_stream_cases(n, seed=20261206):
    """Seeded random small streams: dtype, batch, KV heads, group size, sink and
    local window sizes, segment length, clusters per segment, prefix length
    (ragged), number of appended tokens (at least one extension) and budgets."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        dtype = "f32" if i % 3 == 1 else "bf16"
        B, H = int(rng.integers(1, 3)), int(rng.choice([1, 2, 3]))
        G = int(rng.choice([1, 4, 7, 16]))
        n_sink, n_local = (0, 1, 4)[i % 3], int(rng.choice([0, 5, 64]))
        seg = int(rng.choice([32, 64, 96]))
        k = int(rng.integers(1, min(24, seg) + 1))
        n_ctx = n_sink + n_local + int(rng.integers(1, 3 * seg + 1))
        n_new = int(rng.integers(seg + 1, 2 * seg + 1))  # the window is full: >= 1 extension
        n_ctx += max(0, 69 - n_ctx - n_new)  # (the generator wants streams of 69+ tokens)
        k_r, k_e = int(rng.integers(0, 6)), int(rng.integers(0, 20))
        cases.append((i, dtype, B, H, G, n_sink, n_local, seg, k, n_ctx, n_new, k_r, k_e))
    return cases


@pytest.mark.parametrize("case", _random_stream_cases(6), ids=lambda c: f"rand{c[0]}")
def test_stream_random_small_shapes(case):
    """Seeded random streams, every step checked: steady and pending rows bit
    for bit, every extension's index bit for bit, each decode like any decode."""
    i, dtype, B, H, G, n_sink, n_local, seg, k, n_ctx, n_new, k_r, k_e = case
    w = synth.custom(950 + i, dtype, B, H * G, H, n_ctx + n_new, seg, k, n_iters=2,
                     n_needles=2, n_components=24)
    K, V, q = synth.gen_batch(w)
    s = Stream(w, K, V, n_ctx, n_sink, n_local)
    for t in range(n_new):
        s.step()
        s.check_rows()
        s.decode(_query(q, t, dtype), k_r, k_e, check_plain=(t == 0))
    assert s.extensions >= 1
    print(f"  {n_new} steps, {s.extensions} extensions, within {s.worst:.3e}, "
          f"near-tie reorders {s.reorders}", flush=True)
