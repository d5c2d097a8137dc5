"""CPU checks of the seeded input generators (no method arithmetic lives there)."""
import numpy as np
import torch

from sparse_long_context_segmented_amd import synth


def test_host_generator_is_deterministic_and_shaped():
    w = synth.custom(950, "bf16", 2, 8, 2, 68 + 1500, 512, 32, n_needles=3)
    K1, V1, q1 = synth.gen_batch(w)
    K2, V2, q2 = synth.gen_batch(w)
    assert K1.shape == (2, 2, w.n_ctx, 128) and q1.shape == (2, 8, 128)
    assert np.array_equal(K1, K2) and np.array_equal(V1, V2) and np.array_equal(q1, q2)
    # values are exactly representable in bf16
    assert np.array_equal(torch.from_numpy(K1).to(torch.bfloat16).float().numpy(), K1)
    # the needle positions lie in the indexed range and are distinct
    pos = synth.needle_positions(w, 1, 0, 1)
    assert len(set(pos.tolist())) == 3 and pos.min() >= 4 and pos.max() < w.n_ctx - 64


def test_device_generator_on_cpu():
    """The torch generator used to time the 32-layer model: same shapes and
    dtype as the host draws, deterministic per (workload, layer), different
    layers draw different values, needle keys present (rows far from every
    mixture component are rare otherwise)."""
    w = synth.custom(951, "bf16", 1, 8, 2, 68 + 3000, 1024, 64, n_needles=5)
    K, V, q = synth.gen_layer_device(w, 0, "cpu")
    K2, _, q2 = synth.gen_layer_device(w, 0, "cpu")
    K3, _, _ = synth.gen_layer_device(w, 1, "cpu")
    assert K.shape == (1, 2, w.n_ctx, 128) and V.shape == K.shape and q.shape == (1, 8, 128)
    assert K.dtype == torch.bfloat16 and q.dtype == torch.bfloat16
    assert torch.equal(K, K2) and torch.equal(q, q2)
    assert not torch.equal(K, K3)
    v = V.float()
    assert abs(float(v.mean())) < 0.05 and abs(float(v.std()) - 1.0) < 0.05
    # each head's query leans on its needle: the best-matching key scores far
    # above the typical key
    for h in range(2):
        s = K[0, h].float() @ q[0, 4 * h:4 * h + 4].float().sum(0)
        assert float(s.max()) > float(s.mean()) + 4 * float(s.std())
