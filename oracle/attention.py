"""Masked softmax attention (oracle; test infrastructure only).

ASTA, section "Logical sparsity is not physical sparsity": the output is
SoftMax(Q K^T / sqrt(d)) V, and a query-key pair the mask excludes has its
score set to minus infinity before the softmax, so it gets exactly zero weight.
Section "Align the sparse mask with final execution": positions past the real
sequence length get exactly zero weight. Section "Avoid intra-tile masking when
there is nothing to mask": full and boundary tiles give the same output as the
exact mask (the retained pairs are unchanged); rounding (B3) changes the mask.

The oracle computes the whole softmax of each query row at once in float64 in
the original (frame-major) token order: no tiling, no running statistics.

Readings taken where the page is silent (each listed in the design doc):
* A row that keeps no key has output 0 and log-sum-exp minus infinity.
* The log-sum-exp is of the scaled scores, natural log.
"""
import numpy as np

from .geometry import KIND_SPATIAL
from .masks import head_keep_block
from .tilemap import MODE_DENSE, MODE_NAIVE, MODE_EXACT, MODE_ROUNDED, rounded_keep_block


def masked_attention(q, k, v, keep, scale):
    """o[i] = sum_j P[i, j] v[j] with P[i, :] = softmax over kept j of scale * q[i].k[j].

    q [n, d], k [m, d], v [m, d] (any float; computed in float64); keep bool [n, m].
    Returns o [n, d] float64, lse [n] float64 and P [n, m] float64.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    s = (q @ k.T) * scale
    s = np.where(keep, s, -np.inf)
    m = s.max(axis=1)
    m_safe = np.where(np.isfinite(m), m, 0.0)
    e = np.exp(s - m_safe[:, None])          # exp(-inf) == 0.0 exactly
    l = e.sum(axis=1)
    has = l > 0
    p = np.where(has[:, None], e / np.where(has, l, 1.0)[:, None], 0.0)
    o = p @ v
    with np.errstate(divide="ignore"):
        lse = np.where(has, m_safe + np.log(np.where(has, l, 1.0)), -np.inf)
    return o, lse, p


def mode_keep_block(mode, kind, F, H, W, sink_frames, spatial_band, temporal_band, temporal_layout,
                    bq, bkv, q_tokens, k_tokens, cls_rounded=None):
    """Keep rule that a traversal mode computes, in frame-major token ids.

    DENSE keeps every real pair; NAIVE and EXACT keep the exact head mask;
    ROUNDED keeps the pairs of the tiles that balanced rounding kept.
    """
    q_tokens = np.asarray(q_tokens, dtype=np.int64)
    k_tokens = np.asarray(k_tokens, dtype=np.int64)
    if mode == MODE_DENSE:
        return np.ones((q_tokens.size, k_tokens.size), dtype=bool)
    if mode in (MODE_NAIVE, MODE_EXACT):
        return head_keep_block(kind, F, H, W, sink_frames, spatial_band, temporal_band, q_tokens, k_tokens)
    if mode == MODE_ROUNDED:
        if cls_rounded is None:
            raise ValueError("ROUNDED needs the rounded classification")
        return rounded_keep_block(cls_rounded, F, H, W, kind, sink_frames, temporal_layout, bq, bkv,
                                  q_tokens, k_tokens)
    raise ValueError("unknown mode")


def attention_head(q, k, v, kind, F, H, W, sink_frames, spatial_band, temporal_band, temporal_layout,
                   mode, bq, bkv, scale, rows=None, cls_rounded=None, block=256):
    """Output and log-sum-exp of one head, in frame-major order.

    q, k, v: [N, d]. ``rows``: frame-major query ids to compute (default all).
    Rows are computed in blocks of ``block`` only to bound memory; each row's
    softmax is still taken over the whole key sequence at once.
    """
    N = F * H * W
    rows = np.arange(N, dtype=np.int64) if rows is None else np.asarray(rows, dtype=np.int64)
    keys = np.arange(N, dtype=np.int64)
    d = np.asarray(v).shape[1]
    o = np.empty((rows.size, d), dtype=np.float64)
    lse = np.empty(rows.size, dtype=np.float64)
    k64 = np.asarray(k, dtype=np.float64)
    v64 = np.asarray(v, dtype=np.float64)
    q64 = np.asarray(q, dtype=np.float64)
    for a in range(0, rows.size, block):
        r = rows[a:a + block]
        keep = mode_keep_block(mode, kind, F, H, W, sink_frames, spatial_band, temporal_band,
                               temporal_layout, bq, bkv, r, keys, cls_rounded)
        o[a:a + r.size], lse[a:a + r.size], _ = masked_attention(q64[r], k64, v64, keep, scale)
    return o, lse


__all__ = ["masked_attention", "mode_keep_block", "attention_head", "KIND_SPATIAL"]
