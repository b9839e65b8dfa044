"""Spatial-head and temporal-head masks (oracle; test infrastructure only).

ASTA, section "Speeding up attention", Figures 2 and 3: a spatial head attends
to the tokens of its own and nearby frames; a temporal head attends to a small
spatial region across many frames; both keep full attention to the first frame
(F00), an attention sink, next to a local band.

Readings taken where the page is silent (each listed in the design doc):
* The sink is key columns only: every query keeps every key whose frame is
  below ``sink_frames`` (Figure 6's caption places the sink as a vertical strip).
* The spatial band is frame-granular: keep |f_k - f_q| <= band.
* The temporal window is on the flattened spatial index s = h*W + w, across
  all frames in both directions: keep |s_k - s_q| <= band.
"""
import numpy as np

from .geometry import KIND_SPATIAL, KIND_TEMPORAL


def keep_block(kind, F, H, W, sink_frames, band, q_tokens, k_tokens):
    """Boolean [len(q_tokens), len(k_tokens)]: does query token q keep key token k.

    Tokens are frame-major ids. The rule is evaluated element by element from
    the tokens' (f, s) coordinates.
    """
    S = H * W
    q = np.asarray(q_tokens, dtype=np.int64)[:, None]
    k = np.asarray(k_tokens, dtype=np.int64)[None, :]
    fq, sq = q // S, q % S
    fk, sk = k // S, k % S
    sink = fk < sink_frames
    if kind == KIND_SPATIAL:
        local = np.abs(fk - fq) <= band
    elif kind == KIND_TEMPORAL:
        local = np.abs(sk - sq) <= band
    else:
        raise ValueError("unknown head kind")
    return sink | local


def head_keep_block(kind, F, H, W, sink_frames, spatial_band, temporal_band, q_tokens, k_tokens):
    """``keep_block`` with the band chosen by the head kind."""
    band = spatial_band if kind == KIND_SPATIAL else temporal_band
    return keep_block(kind, F, H, W, sink_frames, band, q_tokens, k_tokens)
