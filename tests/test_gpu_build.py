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


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_build_duplicate_keys(dtype):
    """Every indexed key is one of five rows: after five picks every distance
    is 0, so k-means++ sees zero total weight and takes the smallest unchosen
    index (and never reads a row whose distance is already 0); Lloyd then
    has exact distance ties between duplicate centroids (lowest id wins) and
    many empty clusters."""
    w = synth.custom(303 if dtype == "bf16" else 304, dtype, 1, 4, 2, 68 + 2 * 1024 + 100,
                     1024, 64, n_iters=3, n_needles=2)
    print(f"[build parity] duplicate keys dtype={dtype}", flush=True)
    K, V, q = synth.gen_batch(w)
    pick = np.random.default_rng(11).integers(0, 5, size=(w.n_kv_heads, w.n_ctx - 68))
    for h in range(w.n_kv_heads):
        K[0, h, 4:w.n_ctx - 64] = K[0, h, 4:9][pick[h]]
    gd, od = descs(w)
    ref = oracle.build(od, K, V)
    kt, vt = upload_kv(K, V, w.dtype)
    got = index_to_host(wi.build_index(gd, kt, vt))
    torch.cuda.synchronize()
    assert_index_equal(got, ref)
    assert (ref["sizes"] == 0).sum() > 0


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


def _random_build_cases(n, seed=20261204):
    """Seeded random small shapes: dtype, batch, KV heads, segment length (with
    a ragged last segment), clusters per segment, Lloyd iterations, layer id
    and K/V layout."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        dtype = "f32" if i % 4 == 3 else "bf16"
        B, H = int(rng.integers(1, 3)), int(rng.choice([1, 2, 3]))
        seg = int(rng.choice([32, 96, 200, 512, 1024]))
        k = int(rng.integers(1, min(512, seg) + 1))
        n_idx = int(rng.integers(1, 4 * seg + 1))
        iters = int(rng.integers(0, 5))
        layer = int(rng.integers(0, 40))
        cases.append((i, dtype, B, H, seg, k, 68 + n_idx, iters, layer, bool(i % 3 == 1)))
    return cases


@pytest.mark.parametrize("case", _random_build_cases(10), ids=lambda c: f"rand{c[0]}")
def test_build_random_small_shapes(case):
    """Build parity on seeded random small shapes: every output bit-exact."""
    i, dtype, B, H, seg, k, n_ctx, iters, layer, strided = case
    w = synth.custom(800 + i, dtype, B, 4 * H, H, n_ctx, seg, k, n_iters=iters, n_needles=2)
    got, ref, _ = _build_both(w, n_iters=iters, layer=layer, strided=strided)
    assert_index_equal(got, ref)
