"""GPU parity of wi_build_index against the oracle: every output (centroids,
sizes, value sums, block map, slot tokens, K/V blocks, steady copies,
assignments) must be bit-identical."""
import numpy as np
import pytest
import torch

import oracle
from sparse_long_context_segmented_amd import synth, wi

from parity import assert_index_equal, descs, index_to_host, upload_kv

pytestmark = pytest.mark.gpu


def _build_both(w, n_iters=None, init=None, layer=0, strided=False):
    print(f"[build parity] {w.name} dtype={w.dtype} B={w.batch} H={w.n_kv_heads} "
          f"N={w.n_ctx} seg={w.seg_len} k={w.clusters_per_seg} iters={n_iters} "
          f"init={'given' if init is not None else 'kmeans++'} strided={strided}", flush=True)
    K, V, q = synth.gen_batch(w, layer=layer)
    gd, od = descs(w, layer=layer, n_iters=n_iters)
    ref = oracle.build(od, K, V, init=init)
    if strided:
        # K/V stored token-major [B, N, H, 128]; pass the [B, H, N, 128] view's strides
        dt = torch.float32 if w.dtype == "f32" else torch.bfloat16
        kt = torch.from_numpy(np.ascontiguousarray(K.transpose(0, 2, 1, 3))).to("cuda", dt)
        vt = torch.from_numpy(np.ascontiguousarray(V.transpose(0, 2, 1, 3))).to("cuda", dt)
        H = w.n_kv_heads
        gd.kv_stride_b, gd.kv_stride_h, gd.kv_stride_t = w.n_ctx * H * 128, 128, H * 128
    else:
        kt, vt = upload_kv(K, V, w.dtype)
    it = None
    if init is not None:
        it = torch.from_numpy(init).to("cuda", kt.dtype).contiguous()
    ix = wi.build_index(gd, kt, vt, init=it)
    torch.cuda.synchronize()
    got = index_to_host(ix)
    return got, ref, od


SMALL = synth.custom(301, "bf16", 2, 4, 2, 68 + 3 * 1024 + 333, 1024, 64, n_iters=4,
                     n_needles=3)


def test_build_small_bf16_exact():
    got, ref, _ = _build_both(SMALL)
    assert_index_equal(got, ref)


def test_build_fp32_8k_exact():
    got, ref, _ = _build_both(synth.WORKLOADS[0])
    assert_index_equal(got, ref)


def test_build_zero_iterations():
    got, ref, _ = _build_both(SMALL, n_iters=0)
    assert_index_equal(got, ref)


def test_build_assign_only_from_given_init():
    """n_iters = 0 from given centroids: one assignment (MFMA + exact fallback)
    and the layout, with no seeding and no update."""
    gd, od = descs(SMALL, n_iters=0)
    K, V, q = synth.gen_batch(SMALL)
    init = oracle.build(od, K, V)["centroids"]
    got, ref, _ = _build_both(SMALL, n_iters=0, init=init)
    assert_index_equal(got, ref)


def test_build_given_init():
    gd, od = descs(SMALL, n_iters=0)
    K, V, q = synth.gen_batch(SMALL)
    init = oracle.build(od, K, V)["centroids"]
    got, ref, _ = _build_both(SMALL, n_iters=3, init=init)
    assert_index_equal(got, ref)


def test_build_singleton_clusters_and_short_segments():
    # seg_len < clusters_per_seg: every point its own cluster; tiny tail segment
    w = synth.custom(302, "bf16", 1, 2, 1, 68 + 2 * 48 + 5, 48, 64, n_iters=2, n_needles=2)
    got, ref, _ = _build_both(w)
    assert_index_equal(got, ref)
    assert np.all(got["sizes"] == 1)


def test_build_strided_kv_and_layer_seed():
    got, ref, _ = _build_both(SMALL, layer=7, strided=True)
    assert_index_equal(got, ref)


def test_build_deterministic():
    w = SMALL
    K, V, q = synth.gen_batch(w)
    gd, od = descs(w)
    kt, vt = upload_kv(K, V, w.dtype)
    a = index_to_host(wi.build_index(gd, kt, vt))
    b = index_to_host(wi.build_index(gd, kt, vt))
    torch.cuda.synchronize()
    assert_index_equal(a, b)


def _full_size_sampled(w, units):
    """Build and decode a whole workload in one call each (the benchmark's
    launch configuration); the oracle rebuilds the sampled units from the
    same seeded inputs, whose index must match bit-for-bit and whose decode
    outputs must be within the bf16 tolerance."""
    from parity import rel_err, upload_q
    print(f"[full-size parity] {w.name} units {units}", flush=True)
    K, V, q = synth.gen_batch(w)
    gd, _ = descs(w)
    kt, vt = upload_kv(K, V, w.dtype)
    ix = wi.build_index(gd, kt, vt)
    k_r, k_e = w.budgets()
    dd = wi.DecodeDesc(w.n_q_heads, k_r, k_e, 0.0)
    out = wi.decode_attention(ix, dd, upload_q(q, w.dtype))
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    got = index_to_host(ix, units)  # the sampled units only, in order
    del kt, vt, ix
    H = w.n_kv_heads
    # the oracle builds only the sampled units, over the leading sequences
    # that hold them (so each keeps its (sequence, head) random stream)
    bmax = max(units) // H + 1
    od = oracle.make_desc("bf16", bmax, H, w.n_ctx, n_iters=w.n_iters)
    ref = oracle.build(od, K[:bmax], V[:bmax], units=units)
    ref = {k: v[list(units)] for k, v in ref.items()}
    assert_index_equal(got, ref)
    od1 = oracle.make_desc("bf16", 1, 1, w.n_ctx, n_iters=w.n_iters)
    for i, u in enumerate(units):
        b, h = divmod(u, H)
        sub = {k: v[i:i + 1] for k, v in ref.items()}
        qu = q[b:b + 1, h * w.group:(h + 1) * w.group]
        r = oracle.decode(od1, w.group, k_r, k_e, sub, qu)
        e = rel_err(out[b:b + 1, h * w.group:(h + 1) * w.group], r["out"])
        print(f"  unit (b={b}, h={h}): index exact, decode rel err {e:.3e}", flush=True)
        assert e <= 2e-3


@pytest.mark.slow
def test_build_and_decode_llama8b_128k_sampled_units():
    _full_size_sampled(synth.WORKLOADS[1], (0, 5))


@pytest.mark.slow
def test_build_and_decode_llama8b_128k_batch8_sampled_units():
    """64 units in one call (4 select/attend workgroups per unit)."""
    _full_size_sampled(synth.WORKLOADS[2], (2, 14))


@pytest.mark.slow
def test_build_and_decode_qwen7b_256k_batch4_sampled_units():
    """16 384 clusters per unit (two LDS passes of keys), 7 query heads per KV
    head, anisotropic keys."""
    _full_size_sampled(synth.WORKLOADS[3], (2, 5))
