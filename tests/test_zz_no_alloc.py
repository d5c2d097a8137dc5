"""wi_decode_attention_noalloc (static device scratch, no allocation) against
wi_decode_attention (caller workspace): the same kernels, so every output --
attention output, selected ids, execution-buffer list and length -- must be
bit-identical. Two calls in a row on different inputs, the second smaller,
then the first again (the array keeps the previous call's contents), and a
HIP graph of the no-allocation call replayed with eager work in between."""
import numpy as np
import pytest
import torch

import oracle
from sparse_long_context_segmented_amd import synth, wi

from parity import upload_q

pytestmark = pytest.mark.gpu


def _case(w, k_r, k_e):
    K, V, q = synth.gen_batch(w)
    od = oracle.make_desc(w.dtype, w.batch, w.n_kv_heads, w.n_ctx, seg_len=w.seg_len,
                          clusters_per_seg=w.clusters_per_seg, n_iters=1)
    idx = oracle.build(od, K, V)
    gd = wi.make_desc(w.dtype, w.batch, w.n_kv_heads, w.n_ctx, seg_len=w.seg_len,
                      clusters_per_seg=w.clusters_per_seg, n_iters=1)
    gix = wi.index_from_host(gd, idx)
    C = idx["sizes"].shape[1]
    U = w.batch * w.n_kv_heads
    M = k_r + min(k_e, C - k_r)
    exec_cap = 68 + int(np.sort(idx["sizes"], axis=1)[:, ::-1][:, :k_r].sum(axis=1).max())
    dd = wi.DecodeDesc(w.n_q_heads, k_r, k_e, 0.0, 0)
    assert wi.decode_sizes(gd, dd) <= wi.NOALLOC_SCRATCH_BYTES
    return gix, dd, upload_q(q, w.dtype), (w.batch, w.n_q_heads, U, M, exec_cap)


def _outputs(shape):
    B, Hq, U, M, exec_cap = shape
    return (torch.full((B, Hq, 128), -7.0, dtype=torch.float32, device="cuda"),
            torch.full((U, M), -5, dtype=torch.int32, device="cuda"),
            torch.full((U, exec_cap), -5, dtype=torch.int32, device="cuda"),
            torch.full((U,), -5, dtype=torch.int32, device="cuda"))


def _compare(case):
    gix, dd, qt, shape = case
    o1, s1, e1, n1 = _outputs(shape)
    wi.decode_attention(gix, dd, qt, out=o1, sel_ids=s1, exec_tokens=e1, n_exec=n1)
    o2, s2, e2, n2 = _outputs(shape)
    wi.decode_attention_noalloc(gix, dd, qt, o2, sel_ids=s2, exec_tokens=e2, n_exec=n2)
    o3, _, _, _ = _outputs(shape)
    wi.decode_attention_noalloc(gix, dd, qt, o3)  # no debug outputs
    torch.cuda.synchronize()
    ref = o1.cpu().numpy()
    assert np.isfinite(ref).all()
    assert np.array_equal(o2.cpu().numpy().view(np.uint32), ref.view(np.uint32))
    assert np.array_equal(o3.cpu().numpy().view(np.uint32), ref.view(np.uint32))
    assert torch.equal(s1, s2) and torch.equal(e1, e2) and torch.equal(n1, n2)


# first: 8 units (batch 4 x 2 KV heads: the XCD-aware placement) of 8714
# clusters in two key passes; second: one unit of 192 clusters
LARGER = synth.custom(260, "bf16", 4, 8, 2, 68 + 17 * 1024 + 10, 1024, 512, n_needles=4)
SMALLER = synth.custom(261, "bf16", 1, 4, 1, 68 + 3 * 256 + 40, 256, 64, n_needles=2)


def test_noalloc_matches_workspace_entry_point_two_calls():
    print("[no-alloc] larger call (8 units, C=8714), then smaller (1 unit), then larger",
          flush=True)
    big = _case(LARGER, 300, 2000)
    small = _case(SMALLER, 5, 40)
    _compare(big)
    _compare(small)
    _compare(big)


def test_noalloc_graph_replay():
    print("[no-alloc] graph capture and replays", flush=True)
    gix, dd, qt, shape = _case(SMALLER, 5, 40)
    eager, _, _, _ = _outputs(shape)
    wi.decode_attention_noalloc(gix, dd, qt, eager)
    torch.cuda.synchronize()
    ref = eager.cpu().numpy().view(np.uint32).copy()
    out, _, _, _ = _outputs(shape)
    q2 = torch.flip(qt, dims=[1]).contiguous()
    other, _, _, _ = _outputs(shape)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        wi.decode_attention_noalloc(gix, dd, qt, out)
    for _ in range(3):
        out.zero_()
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy().view(np.uint32), ref)
        wi.decode_attention_noalloc(gix, dd, q2, other)  # eager call on the same scratch
        torch.cuda.synchronize()
        assert not np.array_equal(other.cpu().numpy().view(np.uint32), ref)
