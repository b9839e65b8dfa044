"""Brute-force tile classification and balanced tile rounding (oracle; test infrastructure only).

ASTA, section "Logical sparsity is not physical sparsity" and Figure 5: the
attention matrix is cut into (query tile, key/value tile) blocks. A full tile
holds only retained pairs, a boundary tile holds both retained and excluded
pairs, an empty (skipped) tile holds none. Section "Avoid intra-tile masking
when there is nothing to mask": full and boundary tiles are identified before
attention runs. Section "Align the sparse mask with final execution": tiles on
the mask boundary are rounded outward or inward so the pair budget is about
kept; afterwards only tiles holding padding past the sequence end are masked.
Figure 4 names the four traversals B0 dense, B1 exact sparse, B2 classified
tiles, B3 balanced tile rounding.

Every count here comes from evaluating the keep rule on each (query, key) pair
of the tile, then summing; nothing is derived from interval formulas.

Readings taken where the page is silent (each listed in the design doc):
* Tiles live in the executed layout (temporal heads: the permuted order).
* Padded query rows (position >= N) never decide a class; padded key columns
  (position >= N) force the masking path, since they must get zero weight.
* B3's balancing rule is per tile: keep a tile iff it holds at least one
  retained pair and at least half its valid area is retained (2c >= a).
* Lists per query tile: full tiles in ascending key-tile order, then boundary
  tiles in ascending key-tile order.
"""
import numpy as np

from .geometry import executed_order
from .masks import head_keep_block

MODE_DENSE = 0    # B0: every tile visited, no mask except padding
MODE_NAIVE = 1    # B1: empty tiles skipped, exact mask evaluated on every visited tile
MODE_EXACT = 2    # B2: full tiles unmasked, exact mask on boundary tiles only
MODE_ROUNDED = 3  # B3: mask rounded to whole tiles, only padding is masked

SKIP = 0
FULL = 1
BOUNDARY = 2


def _tiles(N, bq, bkv):
    Tq = -(-N // bq)
    Tk = -(-N // bkv)
    rows_valid = np.minimum(N, (np.arange(Tq) + 1) * bq) - np.arange(Tq) * bq
    cols_valid = np.minimum(N, (np.arange(Tk) + 1) * bkv) - np.arange(Tk) * bkv
    pad_col = (np.arange(Tk) + 1) * bkv > N
    return Tq, Tk, rows_valid.astype(np.int64), cols_valid.astype(np.int64), pad_col


def tile_counts(F, H, W, kind, sink_frames, spatial_band, temporal_band, temporal_layout, bq, bkv, q_tiles=None):
    """c[I, J] = retained (query, key) pairs of tile (I, J), valid rows and columns only.

    Element scan: for every query row of tile I, the keep rule is evaluated
    against every key of the sequence (in executed order); the Booleans are
    then summed per key tile. ``q_tiles`` restricts the scan to those query
    tiles; the other rows of the result are -1.
    """
    N = F * H * W
    order = executed_order(F, H, W, kind, sink_frames, temporal_layout)
    Tq, Tk, _, _, _ = _tiles(N, bq, bkv)
    c = np.zeros((Tq, Tk), dtype=np.int64)
    tiles = range(Tq)
    if q_tiles is not None:
        c[:] = -1
        tiles = sorted(set(int(i) for i in q_tiles))
    buf = np.zeros((bq, Tk * bkv), dtype=bool)
    for I in tiles:
        rows = order[I * bq:min(N, (I + 1) * bq)]
        keep = head_keep_block(kind, F, H, W, sink_frames, spatial_band, temporal_band, rows, order)
        r = rows.size
        buf[:r, :N] = keep
        buf[:r, N:] = False
        c[I] = buf[:r].reshape(r, Tk, bkv).sum(axis=(0, 2))
    return c


def classify(F, H, W, kind, sink_frames, spatial_band, temporal_band, temporal_layout, bq, bkv, mode,
             counts=None):
    """Tile classes, per-tile counts and the canonical kv lists of one head kind.

    Returns a dict with
      cls    int8  [Tq, Tk]  SKIP / FULL / BOUNDARY
      counts int64 [Tq, Tk]  retained pairs of the exact mask (area for DENSE)
      area   int64 [Tq, Tk]  valid rows x valid columns
      n_full, n_bnd int64 [Tq]
      kv     int64 [Tq, Tk]  full tiles ascending, then boundary tiles ascending, then -1
    ``counts`` may pass in a ``tile_counts`` result of the same arguments to
    classify several modes from one element scan.
    """
    N = F * H * W
    Tq, Tk, rows_valid, cols_valid, pad_col = _tiles(N, bq, bkv)
    area = rows_valid[:, None] * cols_valid[None, :]
    if mode == MODE_DENSE:
        c = area.copy()
    elif counts is not None:
        c = np.asarray(counts, dtype=np.int64)
    else:
        c = tile_counts(F, H, W, kind, sink_frames, spatial_band, temporal_band, temporal_layout, bq, bkv)
    pad = np.broadcast_to(pad_col[None, :], (Tq, Tk))
    if mode == MODE_EXACT:
        cls = np.where(c == 0, SKIP, np.where((c == area) & ~pad, FULL, BOUNDARY))
    elif mode == MODE_NAIVE:
        cls = np.where(c == 0, SKIP, BOUNDARY)
    elif mode == MODE_DENSE:
        cls = np.where(pad, BOUNDARY, FULL)
    elif mode == MODE_ROUNDED:
        kept = (c > 0) & (2 * c >= area)
        cls = np.where(kept, np.where(pad, BOUNDARY, FULL), SKIP)
    else:
        raise ValueError("unknown mode")
    cls = cls.astype(np.int8)
    n_full = (cls == FULL).sum(axis=1).astype(np.int64)
    n_bnd = (cls == BOUNDARY).sum(axis=1).astype(np.int64)
    kv = np.full((Tq, Tk), -1, dtype=np.int64)
    for I in range(Tq):
        full = np.nonzero(cls[I] == FULL)[0]
        bnd = np.nonzero(cls[I] == BOUNDARY)[0]
        lst = np.concatenate([full, bnd])
        kv[I, :lst.size] = lst
    return {"cls": cls, "counts": c, "area": area, "n_full": n_full, "n_bnd": n_bnd, "kv": kv,
            "Tq": Tq, "Tk": Tk}


def rounded_keep_block(cls_rounded, F, H, W, kind, sink_frames, temporal_layout, bq, bkv,
                       q_tokens, k_tokens):
    """Keep rule of the B3-rounded mask, in frame-major token ids.

    A pair is kept iff the tile holding it (in the executed layout) was kept by
    rounding; positions past N do not exist, so only real tokens are asked.
    """
    order = executed_order(F, H, W, kind, sink_frames, temporal_layout)
    pos = np.empty_like(order)
    pos[order] = np.arange(order.size)
    qi = pos[np.asarray(q_tokens, dtype=np.int64)] // bq
    kj = pos[np.asarray(k_tokens, dtype=np.int64)] // bkv
    return cls_rounded[qi[:, None], kj[None, :]] != SKIP
