"""Token geometry and the two token orders (oracle; test infrastructure only).

ASTA, section "Arrange tokens for efficient temporal access" and Figure 9: a
video latent of F frames, each an H x W grid, is stored frame-major (F, H, W);
temporal heads run on a temporal-major order (H, W, F) in which the tokens at
one spatial position across successive frames sit next to each other.

Readings taken where the page is silent (each listed in the design doc):
* Token t in frame-major order has frame f = t // (H*W) and flattened spatial
  index s = t % (H*W) = h*W + w.
* Where the first-frame sink goes after the permutation is not stated. The
  default "sink-first" order keeps the sink frames (f < sink_frames) first, in
  their frame-major order, then every other token ordered by (s, f). The
  "literal" order orders every token by (s, f).
* Spatial heads keep the frame-major order (identity), as the section
  "Support dynamic routing with fixed tensor shapes" states.

Both orders are written as a stable sort on an explicit key, which is the plain
definition of "group by spatial position, then by frame".
"""
import numpy as np

KIND_SPATIAL = 0
KIND_TEMPORAL = 1
LAYOUT_SINK_FIRST = 0
LAYOUT_LITERAL = 1


def coords(F, H, W):
    """Frame index f and flattened spatial index s of every frame-major token."""
    S = H * W
    t = np.arange(F * S, dtype=np.int64)
    return t // S, t % S


def executed_order(F, H, W, kind, sink_frames=1, temporal_layout=LAYOUT_SINK_FIRST):
    """order[i] = frame-major token stored at position i of the executed layout.

    Spatial heads: identity. Temporal heads: a stable sort of the tokens by the
    key (group, s, f) with group 0 for sink tokens under the sink-first order
    (their own key is then just t), group 1 for the rest.
    """
    f, s = coords(F, H, W)
    t = np.arange(f.size, dtype=np.int64)
    if kind == KIND_SPATIAL:
        return t
    if temporal_layout == LAYOUT_LITERAL:
        # np.lexsort sorts by the last key first: primary s, secondary f.
        return np.lexsort((f, s)).astype(np.int64)
    if temporal_layout != LAYOUT_SINK_FIRST:
        raise ValueError("unknown temporal layout")
    is_sink = f < sink_frames
    group = np.where(is_sink, 0, 1)
    # Sink tokens: ordered by t (frame-major); others: by (s, f).
    k_s = np.where(is_sink, 0, s)
    k_f = np.where(is_sink, t, f)
    return np.lexsort((k_f, k_s, group)).astype(np.int64)


def positions(order):
    """Inverse of ``order``: p[t] = executed position of token t."""
    p = np.empty_like(order)
    p[order] = np.arange(order.size, dtype=order.dtype)
    return p


def permute(x, order):
    """Executed-layout copy of x (tokens on axis -2): out[..., i, :] = x[..., order[i], :]."""
    return np.take(x, order, axis=-2)


def unpermute(xp, order):
    """Inverse of ``permute``: out[..., order[i], :] = xp[..., i, :]."""
    out = np.empty_like(xp)
    out[..., order, :] = xp
    return out
