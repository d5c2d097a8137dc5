"""Brute-force numpy float64 twin of the oracle, for tiny inputs.

TEST INFRASTRUCTURE ONLY. Written independently of wi_oracle.c and of the HIP
library, in a deliberately different shape: whole distance matrices instead
of per-point loops, and the tripartite attention as ONE plain softmax over an
explicit list of (key, value, multiplicity) entries, where each estimation
cluster enters as n_c copies of a virtual key equal to its centroid carrying
the cluster's mean value (RetroInfer pages: framerc blog section 3.3,
estimation from centroid vectors and cluster sizes; techwalker article
section 3, the estimation zone approximates the tokens it does not load).
"""
from __future__ import annotations

import numpy as np


def partition(n_ctx, seg_len, k, n_sink=4, n_local=64):
    """List of (first token position, n_s, C_s, first cluster id)."""
    out = []
    pos, cid = n_sink, 0
    end = n_ctx - n_local
    while pos < end:
        n = min(seg_len, end - pos)
        c = min(k, n)
        out.append((pos, n, c, cid))
        pos += n
        cid += c
    return out


def bf16(x):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).to(torch.float32).numpy()


def assign(X, C):
    """Nearest centroid by full float64 distance matrix; first index on ties."""
    diff = X.astype(np.float64)[:, None, :] - C.astype(np.float64)[None, :, :]
    dist = np.einsum("ikt,ikt->ik", diff, diff)
    return np.argmin(dist, axis=1).astype(np.int32)


def update(X, a, C, dtype):
    """Mean of members (float64), rounded to float32 then to dtype; empty keep."""
    k = C.shape[0]
    s = np.zeros((k, X.shape[1]), np.float64)
    np.add.at(s, a, X.astype(np.float64))
    n = np.bincount(a, minlength=k)
    m = C.astype(np.float32).copy()
    nz = n > 0
    m[nz] = (s[nz] / n[nz, None]).astype(np.float32)
    if dtype == "bf16":
        m[nz] = bf16(m[nz])
    return m, n.astype(np.int32)


def lloyd(X, C0, iters, dtype):
    C = C0.copy()
    a = assign(X, C)
    for t in range(iters):
        if t > 0:
            a = assign(X, C)
        C, _ = update(X, a, C, dtype)
    return C, a


def objective(X, a, C):
    d = X.astype(np.float64) - C.astype(np.float64)[a]
    return float((d * d).sum())


def softmax_list(q, keys, vals, mult, scale):
    """sum_j mult_j e^{s_j} v_j / sum_j mult_j e^{s_j}, float64."""
    s = (keys.astype(np.float64) @ q.astype(np.float64)) * scale
    w = mult * np.exp(s - s.max())
    return (w[:, None] * vals.astype(np.float64)).sum(0) / w.sum()


def full_attention(q, K, V, scale):
    return softmax_list(q, K, V, np.ones(K.shape[0]), scale)


def tripartite(q, K, V, members, centroids, R, E, n_sink, n_local, scale, extra=(),
               vsum_f32=False):
    """Explicit-list tripartite attention for one query head.

    members[c]: token positions of cluster c. Steady tokens, the extra exact
    positions (pending decode-time tokens) and every token of the R clusters
    are listed as themselves; each non-empty E cluster is one entry with
    key = centroid, value = mean member value, multiplicity n_c. With
    vsum_f32 the members' value sum is first rounded to float32, the
    precision an index stores it in.
    """
    n = K.shape[0]
    steady = list(range(n_sink)) + list(range(n - n_local, n))
    toks = steady + [int(t) for t in extra] + [int(t) for c in R for t in members[c]]
    keys = [K[toks]]
    vals = [V[toks]]
    mult = [np.ones(len(toks))]
    for c in E:
        m = members[c]
        if len(m) == 0:
            continue
        keys.append(centroids[c][None, :])
        vs = V[m].astype(np.float64).sum(0)
        if vsum_f32:
            vs = vs.astype(np.float32).astype(np.float64)
        vals.append((vs / len(m))[None, :])
        mult.append(np.array([float(len(m))]))
    return softmax_list(q, np.concatenate(keys), np.concatenate(vals),
                        np.concatenate(mult), scale)
