"""Sampled-query head routing (oracle; test infrastructure only).

ASTA, section "Speeding up attention": Sparse VideoGen routes each head by
sampling a few queries, computing their outputs under dense, spatial and
temporal attention, and choosing the sparse mask whose output deviates least
from the dense one. Section "Support dynamic routing with fixed tensor
shapes": the result is one Boolean flag per head.

Readings taken where the page is silent (each listed in the design doc):
* The caller supplies the sampled query ids; nothing here draws randomness.
* Deviation is the squared L2 distance summed over the sampled queries:
  err_x = sum_i ||o_x(i) - o_dense(i)||^2.
* flag = 1 (temporal) iff err_temporal < err_spatial; ties choose spatial.
* Routing always uses the exact masks, never rounded ones.
"""
import numpy as np

from .geometry import KIND_SPATIAL, KIND_TEMPORAL
from .masks import keep_block
from .attention import masked_attention


def route_heads(q, k, v, F, H, W, sink_frames, spatial_band, temporal_band, sample_idx, scale):
    """q, k, v: [B, heads, N, d] frame-major. Returns flags uint8 [B, heads], err float64 [B, heads, 2].

    err[..., 0] is the spatial mask's deviation, err[..., 1] the temporal one's.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, nh, N, _ = q.shape
    idx = np.asarray(sample_idx, dtype=np.int64)
    keys = np.arange(N, dtype=np.int64)
    keep_sp = keep_block(KIND_SPATIAL, F, H, W, sink_frames, spatial_band, idx, keys)
    keep_tp = keep_block(KIND_TEMPORAL, F, H, W, sink_frames, temporal_band, idx, keys)
    keep_all = np.ones_like(keep_sp)
    flags = np.zeros((B, nh), dtype=np.uint8)
    err = np.zeros((B, nh, 2), dtype=np.float64)
    for b in range(B):
        for h in range(nh):
            qs = q[b, h, idx]
            o_d, _, _ = masked_attention(qs, k[b, h], v[b, h], keep_all, scale)
            o_s, _, _ = masked_attention(qs, k[b, h], v[b, h], keep_sp, scale)
            o_t, _, _ = masked_attention(qs, k[b, h], v[b, h], keep_tp, scale)
            e_s = float(((o_s - o_d) ** 2).sum())
            e_t = float(((o_t - o_d) ** 2).sum())
            err[b, h] = (e_s, e_t)
            flags[b, h] = 1 if e_t < e_s else 0
    return flags, err
