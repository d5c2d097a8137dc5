"""GPU parity of the wave buffer (GPU block cache over a pinned host tier).

A sequence of decode steps with drifting queries runs twice: through
wi_decode_attention on the HBM-resident index (the reference selection and
output), and through wi_decode_attention_wb on the same index with its K/V
block pools in pinned host memory behind a cache of n_slots blocks per unit.
Every step: the outputs must be equal bit for bit; the step's hits and misses
must equal the oracle's LRU simulation fed with the blocks of the same
retrieval zone; and after the step the cache tables must equal the
simulation's and every cached slot must hold its block's K and V bytes.
"""
import numpy as np
import pytest
import torch

from oracle import wavebuf
from sparse_long_context_segmented_amd import synth, wi

from parity import upload_kv, upload_q

pytestmark = pytest.mark.gpu


def _queries(q, steps, dtype, drift=0.35):
    """A slowly drifting query stream (random walk around the workload's q)."""
    rng = np.random.default_rng(99)
    out, cur = [], q.copy()
    for _ in range(steps):
        cur = cur + drift * rng.standard_normal(q.shape).astype(np.float32)
        out.append(synth._round_to_dtype(0.8 * cur + 0.2 * q, dtype))
    return out


def _run(w, n_slots_frac, steps, check_every=1, seed_slots=None):
    K, V, q = synth.gen_batch(w)
    gd = wi.make_desc(w.dtype, w.batch, w.n_kv_heads, w.n_ctx, seg_len=w.seg_len,
                      clusters_per_seg=w.clusters_per_seg, n_iters=w.n_iters)
    kt, vt = upload_kv(K, V, w.dtype)
    ix = wi.build_index(gd, kt, vt)
    del kt, vt
    hix = wi.host_tier(ix)
    U = w.batch * w.n_kv_heads
    T = 8 if w.dtype == "bf16" else 4
    cap = ix.k_blocks.shape[1] // T
    used = int(ix.block_off[:, -1].max())
    n_slots = seed_slots or max(1, int(n_slots_frac * used))
    wb = wi.alloc_wave_buffer(gd, n_slots)
    k_r, k_e = w.budgets()
    dd = wi.DecodeDesc(w.n_q_heads, k_r, k_e, 0.0)
    C = ix.cluster_size.shape[1]
    M = k_r + min(k_e, C - k_r)
    sizes = ix.cluster_size.cpu().numpy()
    bo = ix.block_off.cpu().numpy()
    kb_host = hix.k_blocks.view(torch.int16).numpy().reshape(U, cap, -1)
    vb_host = hix.v_blocks.view(torch.int16).numpy().reshape(U, cap, -1)
    sims = [wavebuf.WaveBufferSim(n_slots, cap) for _ in range(U)]
    sel = torch.empty(U, M, dtype=torch.int32, device="cuda")
    stats = torch.empty(U, 2, dtype=torch.int32, device="cuda")
    tot_h = tot_m = 0
    for t, qs in enumerate(_queries(q, steps, w.dtype), start=1):
        qt = upload_q(qs, w.dtype)
        ref = wi.decode_attention(ix, dd, qt, sel_ids=sel)
        out = wi.decode_attention_wb(hix, dd, wb, t, qt, stats=stats)
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"step {t}: output differs from the HBM decode"
        R = sel.cpu().numpy()[:, :k_r]
        st = stats.cpu().numpy()
        for u in range(U):
            need = wavebuf.needed_blocks(R[u], sizes[u], bo[u], T)
            h, m, _ = sims[u].step(t, need)
            assert (st[u, 0], st[u, 1]) == (h, m), (t, u)
            tot_h += h
            tot_m += m
        if t % check_every == 0 or t == steps:
            b2s = wb.block_slot.cpu().numpy()
            s2b = wb.slot_block.cpu().numpy()
            last = wb.slot_last.cpu().numpy().view(np.uint32)
            ck = wb.cache_k.view(torch.int16).cpu().numpy().reshape(U, n_slots, -1)
            cv = wb.cache_v.view(torch.int16).cpu().numpy().reshape(U, n_slots, -1)
            order = wb.slot_order.cpu().numpy()
            for u in range(U):
                assert order[u].tolist() == sorted(range(n_slots),
                                                   key=lambda s: (sims[u].slot_last[s], s))
                assert b2s[u].tolist() == sims[u].block_slot, (t, u)
                assert s2b[u].tolist() == sims[u].slot_block, (t, u)
                assert last[u].tolist() == sims[u].slot_last, (t, u)
                for s, b in enumerate(s2b[u]):
                    if b >= 0:
                        assert np.array_equal(ck[u, s], kb_host[u, b]), (t, u, s)
                        assert np.array_equal(cv[u, s], vb_host[u, b]), (t, u, s)
    return tot_h, tot_m, n_slots


@pytest.mark.parametrize("dtype,frac", [("bf16", 0.3), ("bf16", 0.02), ("f32", 0.25)])
def test_wave_buffer_small(dtype, frac):
    """Several steps with a cache that holds about frac of the used blocks
    (0.02: fewer slots than one step's misses, so admission is cut short)."""
    w = synth.custom(61, dtype, 2, 8, 2, 68 + 4 * 512 + 100, 512, 32, n_iters=3, n_needles=4,
                     n_components=64)
    h, m, S = _run(w, frac, 12)
    print(f"  {dtype} slots {S}: hits {h}, misses {m}", flush=True)
    assert h > 0 and m > 0


def test_wave_buffer_single_slot():
    w = synth.custom(62, "bf16", 1, 4, 1, 68 + 2 * 256, 256, 16, n_iters=2, n_components=16)
    _run(w, 0.0, 6, seed_slots=1)


@pytest.mark.slow
@pytest.mark.timeout(600)
def test_wave_buffer_llama8b_128k_batch1():
    """The 128K batch-1 layer with a cache of 10 % of the used blocks, 24
    drifting decode steps, tables checked every 8 steps."""
    h, m, S = _run(synth.WORKLOADS[1], 0.10, 24, check_every=8)
    print(f"  128K b1, {S} slots per unit: hit rate {h / (h + m):.3f}", flush=True)


def _random_wb_cases(n, seed=20261205):
    """Seeded random small shapes for the wave buffer: dtype, batch, KV heads,
    group size, segment length (ragged last segment), clusters per segment,
    retrieval budget, cache size as a share of the used blocks, steps."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        dtype = "f32" if i % 3 == 2 else "bf16"
        B, H = int(rng.integers(1, 3)), int(rng.choice([1, 2, 3]))
        G = int(rng.choice([1, 4, 7, 8, 16]))
        seg = int(rng.choice([128, 256, 512]))
        k = int(rng.integers(4, min(64, seg) + 1))
        n_idx = int(rng.integers(seg, 4 * seg + 1))
        full, rem = divmod(n_idx, seg)
        C = full * k + min(k, rem)
        k_r = int(rng.integers(1, max(2, C // 3)))
        frac = float(rng.choice([0.01, 0.1, 0.5, 1.0]))
        steps = int(rng.integers(3, 9))
        cases.append((i, dtype, B, H, G, seg, k, 68 + n_idx, k_r, frac, steps))
    return cases


@pytest.mark.parametrize("case", _random_wb_cases(8), ids=lambda c: f"rand{c[0]}")
def test_wave_buffer_random_small_shapes(case):
    """Seeded random shapes: every step's output equals the HBM decode bit for
    bit, and the cache state equals the reference model's."""
    i, dtype, B, H, G, seg, k, n_ctx, k_r, frac, steps = case
    w = synth.custom(900 + i, dtype, B, H * G, H, n_ctx, seg, k, n_iters=2, n_needles=2,
                     k_retrieve=k_r, n_components=64)
    h, m, S = _run(w, frac, steps)
    print(f"  {dtype} slots {S}: hits {h}, misses {m}", flush=True)
