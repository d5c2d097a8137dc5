"""Seeded synthetic workloads for the wave-index build and decode.

This module is shared by the tests, the benchmark and the parity checks. It
holds only workload parameters and random draws; none of the method's
arithmetic (no clustering, scoring or attention) lives here, so both the HIP
path and the CPU oracle can be fed from it without sharing any computation.

Workload shapes follow the model shapes the RetroInfer pages evaluate on
(techwalker article, section 4: Llama3.1-8B, Qwen2.5-7B and Llama3-8B-1048K).
The datasets named there (RULER, LongBench, needle-in-a-haystack) are not
available, so a seeded stand-in is drawn instead:

* keys: a mixture of 512 Gaussian components (means N(0, 1), sigma 0.3) --
  attention mass concentrated on few tokens, the sparsity premise the
  techwalker article states in section 2 (about 2 % of tokens dominate);
* "needle" keys aligned with the query direction at a few positions, as a
  stand-in for needle-in-a-haystack retrieval;
* values N(0, 1); queries N(0, I) plus 0.5x the needle direction;
* for the Qwen2.5-7B-shaped workload, per-(head, dim) log-normal scales
  (sigma 0.5) that mimic outlier channels.

Every (workload, sequence, layer, KV head) unit has its own numpy PCG64
stream seeded with [0, workload_id, b, l, h]; draws happen in a fixed order.
"""
from __future__ import annotations

import dataclasses
import numpy as np

HEAD_DIM = 128
N_SINK = 4
N_LOCAL = 64


@dataclasses.dataclass(frozen=True)
class Workload:
    """One workload shape. Sizes are the model shapes; budgets are fractions."""

    wid: int            # workload id used in the seed
    name: str
    dtype: str          # "f32" or "bf16"
    batch: int
    layers: int
    n_q_heads: int
    n_kv_heads: int
    n_ctx: int
    seg_len: int = 8192
    clusters_per_seg: int = 512
    n_iters: int = 10
    n_needles: int = 8
    anisotropic: bool = False
    retrieve_frac: float = 0.018      # share of tokens in the retrieval zone
    estimate_frac: float = 0.23       # share of tokens in the estimation zone
    k_retrieve_fixed: int | None = None  # explicit cluster count (8K fp32 case)
    n_components: int = 512

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    def budgets(self) -> tuple[int, int]:
        """(K_r, K_e) in clusters.

        The pages state both budgets as token shares (framerc blog, section
        2.1: about 1.8 % retrieved, 23 % estimated). With segments of
        seg_len tokens and clusters_per_seg clusters each, a cluster holds
        seg_len / clusters_per_seg tokens on average, so a share f of N
        tokens is round(f * N * clusters_per_seg / seg_len) clusters.
        """
        per_tok = self.clusters_per_seg / self.seg_len
        k_e = int(np.floor(self.estimate_frac * self.n_ctx * per_tok + 0.5))
        if self.k_retrieve_fixed is not None:
            k_r = self.k_retrieve_fixed
        else:
            k_r = int(np.floor(self.retrieve_frac * self.n_ctx * per_tok + 0.5))
        return k_r, k_e


# The five workload shapes. Index 0 is the small fp32 case, index 1 the
# Llama3.1-8B-shaped 128K layer the decode throughput is quoted on.
WORKLOADS = [
    Workload(1, "fp32-8k-1kv", "f32", 1, 1, 4, 1, 8192, n_needles=8,
             k_retrieve_fixed=10),
    Workload(2, "llama8b-128k-b1", "bf16", 1, 1, 32, 8, 131072, n_needles=32),
    Workload(3, "llama8b-128k-b8", "bf16", 8, 1, 32, 8, 131072, n_needles=32),
    Workload(4, "qwen7b-256k-b4", "bf16", 4, 1, 28, 4, 262144, n_needles=32,
             anisotropic=True),
    Workload(5, "llama8b-1m-32l", "bf16", 1, 32, 32, 8, 1048576, n_needles=8),
]


def custom(wid: int, dtype: str, batch: int, n_q_heads: int, n_kv_heads: int,
           n_ctx: int, seg_len: int, clusters_per_seg: int, n_iters: int = 10,
           n_needles: int = 4, anisotropic: bool = False,
           k_retrieve: int | None = None, n_components: int = 512) -> Workload:
    """A reduced workload of the same recipe, for tests that must finish fast."""
    return Workload(wid, f"custom{wid}", dtype, batch, 1, n_q_heads, n_kv_heads,
                    n_ctx, seg_len=seg_len, clusters_per_seg=clusters_per_seg,
                    n_iters=n_iters, n_needles=n_needles, anisotropic=anisotropic,
                    k_retrieve_fixed=k_retrieve, n_components=n_components)


def _round_to_dtype(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float32 values to the storage dtype and return them as float32.

    bf16 rounding is round-to-nearest-even, done by torch on the CPU.
    """
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).to(torch.float32).numpy()


def gen_unit(w: Workload, b: int, l: int, h: int, want_kv: bool = True):
    """Draw one unit (sequence b, layer l, KV head h).

    Returns (K [N, 128], V [N, 128], q [G, 128]) as float32 arrays whose
    values are exactly representable in the workload dtype.
    """
    rng = np.random.default_rng([0, w.wid, b, l, h])
    d = HEAD_DIM
    n = w.n_ctx
    means = rng.standard_normal((w.n_components, d), dtype=np.float32)
    labels = rng.integers(0, w.n_components, size=n)
    eps = rng.standard_normal((n, d), dtype=np.float32)
    k = means[labels]
    k += np.float32(0.3) * eps
    del eps
    needle = rng.standard_normal(d, dtype=np.float32)
    lo, hi = N_SINK, n - N_LOCAL
    n_needles = min(w.n_needles, max(hi - lo, 0))
    pos = np.sort(rng.choice(hi - lo, size=n_needles, replace=False)) + lo
    k[pos] = needle[None, :] + np.float32(0.3) * rng.standard_normal(
        (n_needles, d), dtype=np.float32)
    if w.anisotropic:
        sigma = np.exp(np.float32(0.5) * rng.standard_normal(d, dtype=np.float32))
        k *= sigma[None, :]
    v = rng.standard_normal((n, d), dtype=np.float32)
    z = rng.standard_normal((w.group, d), dtype=np.float32)
    q = z + np.float32(0.5) * needle[None, :]
    q = _round_to_dtype(q, w.dtype)
    if not want_kv:
        return None, None, q
    return _round_to_dtype(k, w.dtype), _round_to_dtype(v, w.dtype), q


def needle_positions(w: Workload, b: int, l: int, h: int) -> np.ndarray:
    """Positions of the needle keys of one unit (same draws as gen_unit)."""
    rng = np.random.default_rng([0, w.wid, b, l, h])
    d = HEAD_DIM
    n = w.n_ctx
    rng.standard_normal((w.n_components, d), dtype=np.float32)
    rng.integers(0, w.n_components, size=n)
    rng.standard_normal((n, d), dtype=np.float32)
    rng.standard_normal(d, dtype=np.float32)
    lo, hi = N_SINK, n - N_LOCAL
    n_needles = min(w.n_needles, max(hi - lo, 0))
    return np.sort(rng.choice(hi - lo, size=n_needles, replace=False)) + lo


def gen_batch(w: Workload, layer: int = 0, heads=None, batches=None):
    """Draw all units of one layer: K, V [B, Hkv, N, 128]; q [B, Hq, 128]."""
    heads = range(w.n_kv_heads) if heads is None else heads
    batches = range(w.batch) if batches is None else batches
    ks, vs, qs = [], [], []
    for b in batches:
        kb, vb, qb = [], [], []
        for h in heads:
            k, v, q = gen_unit(w, b, layer, h)
            kb.append(k)
            vb.append(v)
            qb.append(q)
        ks.append(np.stack(kb))
        vs.append(np.stack(vb))
        qs.append(np.concatenate(qb, axis=0))
    return np.stack(ks), np.stack(vs), np.stack(qs)


def gen_layer_device(w: Workload, layer: int, device, heads_per_draw: int = 2):
    """Draw one layer of a workload on the GPU with torch's own generator.

    Same recipe as gen_unit (mixture keys, needles, optional anisotropic
    scales, N(0, 1) values, needle-biased queries), but the draws come from a
    torch CUDA generator seeded with (workload, layer), not from numpy's
    per-unit streams, so the values differ from gen_batch. Used only to time
    workloads whose raw KV is too large to draw on the host (the 32-layer
    1M-token model, 4.3 GB of raw KV per layer); parity at that size is
    checked on host-drawn units. Returns K, V [B, Hkv, N, 128] and
    q [B, Hq, 128] in the workload dtype.
    """
    import torch
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    gen = torch.Generator(device=device)
    gen.manual_seed((w.wid << 20) ^ (layer + 1))
    B, H, N, d = w.batch, w.n_kv_heads, w.n_ctx, HEAD_DIM
    K = torch.empty(B, H, N, d, dtype=dt, device=device)
    V = torch.empty(B, H, N, d, dtype=dt, device=device)
    q = torch.empty(B, w.n_q_heads, d, dtype=dt, device=device)
    lo, hi = N_SINK, N - N_LOCAL
    n_needles = min(w.n_needles, max(hi - lo, 0))
    for b in range(B):
        for h0 in range(0, H, heads_per_draw):
            h1 = min(H, h0 + heads_per_draw)
            nh = h1 - h0
            means = torch.randn(nh, w.n_components, d, generator=gen, device=device)
            labels = torch.randint(0, w.n_components, (nh, N), generator=gen, device=device)
            k = torch.gather(means, 1, labels[..., None].expand(nh, N, d))
            k += 0.3 * torch.randn(nh, N, d, generator=gen, device=device)
            needle = torch.randn(nh, d, generator=gen, device=device)
            for j in range(nh):
                pos = torch.randperm(hi - lo, generator=gen, device=device)[:n_needles] + lo
                k[j, pos] = needle[j][None, :] + 0.3 * torch.randn(
                    n_needles, d, generator=gen, device=device)
            if w.anisotropic:
                k *= torch.exp(0.5 * torch.randn(nh, 1, d, generator=gen, device=device))
            K[b, h0:h1] = k.to(dt)
            del k, labels, means
            V[b, h0:h1] = torch.randn(nh, N, d, generator=gen, device=device).to(dt)
            z = torch.randn(nh, w.group, d, generator=gen, device=device)
            q[b, h0 * w.group:h1 * w.group] = (z + 0.5 * needle[:, None, :]).reshape(
                nh * w.group, d).to(dt)
    return K, V, q
