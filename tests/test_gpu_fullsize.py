"""Full-size GPU parity, in the benchmark's launch configuration.

Each workload layer is built by wi_build_index and decoded by
wi_decode_attention in one call each, exactly as bench.py times them. Then:

* decode, every unit: the index the GPU built is copied to the host and the
  oracle decodes it. The GPU's selection (rank order, from a second call with
  the debug outputs, whose attention output must equal the first call's bit
  for bit) must equal the oracle's exact ranking up to counted near-ties; the
  execution-buffer token list must follow from it; and the output must be
  within 2e-3 of the oracle's tripartite attention over the GPU's zones;
* index, sampled units: the oracle rebuilds the units from the same seeded
  K/V (k-means++ from the unit's own random stream, 10 Lloyd iterations, the
  block layout), and every index array must be bit-identical.

The workloads and the units the oracle rebuilds: the Llama3.1-8B-shaped 128K
layer at batch 1 (all 8 units), at batch 8 (one unit per sequence, with KV
head = sequence, so that u mod 8 runs over 0..7: every placement residue of
the fused kernel's XCD-aware mapping), the Qwen2.5-7B-shaped 256K batch-4
layer (all 16 units), and three layers of the 1M-token Llama3-8B-1048K-shaped
model (layer 0 head 0, layer 15 head 3, layer 31 head 7; all 128 segments).
These are the slowest GPU tests (the oracle rebuilds take minutes on the
host), so this file is collected after the other parity tests.
"""
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import oracle
from sparse_long_context_segmented_amd import synth, wi

from parity import (assert_index_equal, check_selection, descs, exec_reference, index_to_host,
                    rel_err, upload_kv, upload_q)

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

N_ST = 68


def _gpu_build_and_decode(w, K, V, q, layer=0):
    """One build call and one decode call (no debug outputs: the benchmark's
    configuration), then a decode call with the debug outputs."""
    gd, _ = descs(w, layer=layer)
    kt, vt = upload_kv(K, V, w.dtype)
    ix = wi.build_index(gd, kt, vt)
    k_r, k_e = w.budgets()
    dd = wi.DecodeDesc(w.n_q_heads, k_r, k_e, 0.0)
    qt = upload_q(q, w.dtype)
    out = wi.decode_attention(ix, dd, qt)
    torch.cuda.synchronize()
    del kt, vt
    U = w.batch * w.n_kv_heads
    C = ix.cluster_size.shape[1]
    M = k_r + min(k_e, C - k_r)
    exec_cap = N_ST + int(ix.cluster_size.topk(k_r, dim=1).values.sum(dim=1).max())
    sel = torch.full((U, M), -5, dtype=torch.int32, device="cuda")
    exe = torch.full((U, exec_cap), -5, dtype=torch.int32, device="cuda")
    nexe = torch.full((U,), -5, dtype=torch.int32, device="cuda")
    out2 = wi.decode_attention(ix, dd, qt, sel_ids=sel, exec_tokens=exe, n_exec=nexe)
    torch.cuda.synchronize()
    out, out2 = out.cpu().numpy(), out2.cpu().numpy()
    assert np.array_equal(out.view(np.uint32), out2.view(np.uint32)), \
        "debug outputs changed the attention output"
    return ix, out, sel.cpu().numpy(), exe.cpu().numpy(), nexe.cpu().numpy(), (k_r, k_e)


def _check_decode_units(w, ix, q, out, sel, exe, nexe, budgets, units_per_chunk):
    """Oracle decode over the GPU-built index, every unit, in chunks of
    consecutive units (whole sequences, or single units of a sequence)."""
    k_r, k_e = budgets
    H, G = w.n_kv_heads, w.group
    U = w.batch * H
    T = 8 if w.dtype == "bf16" else 4
    worst, reorders = 0.0, 0
    for u0 in range(0, U, units_per_chunk):
        units = list(range(u0, u0 + units_per_chunk))
        b, h0 = divmod(u0, H)
        host = index_to_host(ix, units)
        od = oracle.make_desc(w.dtype, 1, len(units), w.n_ctx, seg_len=w.seg_len,
                              clusters_per_seg=w.clusters_per_seg, n_iters=w.n_iters)
        qc = q[b:b + 1, h0 * G:(h0 + len(units)) * G]
        r = oracle.decode(od, G * len(units), k_r, k_e, host, qc)
        sg = sel[units]
        reorders += check_selection(sg, r["gkey"], k_r)
        ref = oracle.attend_sets(od, G * len(units), host, qc, sg[:, :k_r], sg[:, k_r:])
        e = rel_err(out[b:b + 1, h0 * G:(h0 + len(units)) * G], ref)
        assert e <= 2e-3, (units, e)
        worst = max(worst, e)
        ex_ref = exec_reference(host, sg, k_r, w.n_ctx, T)
        for i, u in enumerate(units):
            assert nexe[u] == len(ex_ref[i]), u
            n = min(int(nexe[u]), exe.shape[1])
            assert exe[u][:n].tolist() == ex_ref[i][:n], u
        del host
    print(f"  decode: all {U} units within {worst:.3e}, near-tie reorders {reorders}",
          flush=True)


def _check_rebuilt_units(w, ix, K, V, units, layer=0):
    """The oracle rebuilds the given units (over the leading sequences that
    hold them, so each keeps its (sequence, head) random stream)."""
    H = w.n_kv_heads
    bmax = max(units) // H + 1
    od = oracle.make_desc(w.dtype, bmax, H, w.n_ctx, seg_len=w.seg_len,
                          clusters_per_seg=w.clusters_per_seg, n_iters=w.n_iters,
                          layer_id=layer)
    ref = oracle.build(od, K[:bmax], V[:bmax], units=units)
    ref = {k: v[list(units)] for k, v in ref.items()}
    got = index_to_host(ix, units)
    assert_index_equal(got, ref)
    print(f"  index: units {list(units)} bit-exact", flush=True)


def _layer(w, units_rebuilt, chunk):
    print(f"[full-size parity] {w.name}: decode all {w.batch * w.n_kv_heads} units, "
          f"rebuild units {units_rebuilt}", flush=True)
    K, V, q = synth.gen_batch(w)
    ix, out, sel, exe, nexe, budgets = _gpu_build_and_decode(w, K, V, q)
    _check_decode_units(w, ix, q, out, sel, exe, nexe, budgets, chunk)
    _check_rebuilt_units(w, ix, K, V, units_rebuilt)


@pytest.mark.timeout(600)
def test_fullsize_llama8b_128k_batch1_all_units():
    _layer(synth.WORKLOADS[1], list(range(8)), 8)


@pytest.mark.timeout(600)
def test_fullsize_llama8b_128k_batch8_every_xcd_residue():
    """64 units in one call (4 fused workgroups per unit, placed by unit mod 8)."""
    _layer(synth.WORKLOADS[2], [9 * b for b in range(8)], 8)


@pytest.mark.timeout(900)
def test_fullsize_qwen7b_256k_batch4_all_units():
    """16 384 clusters per unit (two LDS passes of keys), 7 query heads per KV
    head, anisotropic keys."""
    _layer(synth.WORKLOADS[3], list(range(16)), 4)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("layer,head", [(0, 0), (15, 3), (31, 7)])
def test_fullsize_llama8b_1m_layer(layer, head):
    """One layer of the 1M-token model: all 8 KV heads built and decoded in one
    call each (65 536 clusters per unit in 128 segments); every unit's decode
    checked on the GPU-built index; unit (0, head) rebuilt by the oracle over
    all 128 segments (the layer id enters the k-means++ random stream)."""
    w = synth.WORKLOADS[4]
    H = w.n_kv_heads
    print(f"[full-size parity] {w.name} layer {layer}: decode all {H} units, "
          f"rebuild head {head}", flush=True)
    with ThreadPoolExecutor(4) as ex:
        parts = list(ex.map(lambda h: synth.gen_unit(w, 0, layer, h), range(H)))
    K = np.stack([p[0] for p in parts])[None]
    V = np.stack([p[1] for p in parts])[None]
    q = np.concatenate([p[2] for p in parts], axis=0)[None]
    del parts
    ix, out, sel, exe, nexe, budgets = _gpu_build_and_decode(w, K, V, q, layer=layer)
    print("  GPU build + decode done", flush=True)
    _check_decode_units(w, ix, q, out, sel, exe, nexe, budgets, 1)
    _check_rebuilt_units(w, ix, K, V, [head], layer=layer)
