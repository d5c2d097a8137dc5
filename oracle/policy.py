"""Per-layer zone policy, oracle side.

TEST INFRASTRUCTURE ONLY (see the package docstring). Written from the
RetroInfer pages, independently of the library's own policy function:

- [blog] framerc.cn, section 3.3 (layer-wise strategy for very large models,
  given for an 80-layer model): layers 0-20 keep full attention for precise
  localisation, layers 21-60 use the hybrid (retrieval + estimation) scheme,
  the upper layers 61 and above raise the estimation share to 30 %.
- [blog] section 4.3, problem 3: sparse attention switched off in the first
  two layers.
- [blog] section 2.1: the hybrid budgets, about 1.8 % of tokens retrieved
  and 23 % estimated.

Readings: the bands are fractions of the model's depth (the 80-layer example
scaled to n_layers: layer l is dense when 80 l < 21 n_layers and "upper" when
80 l >= 61 n_layers, which reproduces the example's bands exactly at 80
layers); token shares become cluster counts at seg_len / clusters_per_seg
tokens per cluster, rounded half up.
"""
import math

DENSE, HYBRID = 0, 1
UNIFORM, DENSE_FIRST2, BANDED = 0, 1, 2

RETRIEVE_SHARE = 0.018
ESTIMATE_SHARE = 0.23
ESTIMATE_SHARE_UPPER = 0.30


def clusters_for(share, n_ctx, seg_len, clusters_per_seg):
    return int(math.floor(share * n_ctx * clusters_per_seg / seg_len + 0.5))


def plan(kind, layer, n_layers, n_ctx, seg_len=8192, clusters_per_seg=512):
    """(mode, K_r, K_e) of one layer."""
    if not 0 <= layer < n_layers:
        raise ValueError("layer outside the model")
    if kind == UNIFORM:
        dense, upper = False, False
    elif kind == DENSE_FIRST2:
        dense, upper = layer < 2, False
    elif kind == BANDED:
        dense = 80 * layer < 21 * n_layers
        upper = 80 * layer >= 61 * n_layers
    else:
        raise ValueError("unknown policy")
    if dense:
        return DENSE, 0, 0
    e = ESTIMATE_SHARE_UPPER if upper else ESTIMATE_SHARE
    return (HYBRID, clusters_for(RETRIEVE_SHARE, n_ctx, seg_len, clusters_per_seg),
            clusters_for(e, n_ctx, seg_len, clusters_per_seg))
