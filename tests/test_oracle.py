"""Pins of the oracle against facts that do not come from the oracle itself.

Each test names what pins it: a hand-derived fixture under tests/golden/, a
closed form derived from the mask definitions, an independent interval count,
a library routine (torch scaled_dot_product_attention, scipy logsumexp), or a
brute-force loop on a tiny case.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle as O
from synth import planted_qkv

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
GEOMS = [(4, 4, 8), (9, 16, 24), (5, 3, 7), (3, 2, 5), (7, 1, 1), (2, 5, 1), (6, 2, 3)]


def _read(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as fh:
        for line in fh:
            line = line.split("#")[0].strip()
            if line:
                rows.append(line.split())
    return rows


# ---------------------------------------------------------------- geometry

def test_tiny_permutation_matches_hand_table():
    """Pin: hand-derived positions (tests/golden/tiny_permutation.txt)."""
    layouts = {"sink_first": O.LAYOUT_SINK_FIRST, "literal": O.LAYOUT_LITERAL}
    cache = {}
    for layout, t, pos in _read("tiny_permutation.txt"):
        lay = layouts[layout]
        if lay not in cache:
            cache[lay] = O.positions(O.executed_order(4, 4, 8, O.KIND_TEMPORAL, 1, lay))
        assert cache[lay][int(t)] == int(pos), (layout, t)


@pytest.mark.parametrize("F,H,W", GEOMS)
@pytest.mark.parametrize("sink", [0, 1, 2])
def test_orders_are_bijections_grouping_spatial_positions(F, H, W, sink):
    """Pin: the defining property of each order, checked position by position."""
    sink = min(sink, F)
    S, N = H * W, F * H * W
    assert np.array_equal(O.executed_order(F, H, W, O.KIND_SPATIAL, sink, 0), np.arange(N))
    for lay in (O.LAYOUT_SINK_FIRST, O.LAYOUT_LITERAL):
        order = O.executed_order(F, H, W, O.KIND_TEMPORAL, sink, lay)
        assert np.array_equal(np.sort(order), np.arange(N))
        f, s = order // S, order % S
        start = 0
        if lay == O.LAYOUT_SINK_FIRST:
            start = sink * S
            assert np.array_equal(order[:start], np.arange(start))
            first_frame = sink
        else:
            first_frame = 0
        per = F - first_frame
        if per == 0:
            continue
        # after the sink block: spatial position major, frames first_frame..F-1 minor
        rest = np.arange(N - start)
        assert np.array_equal(s[start:], rest // per)
        assert np.array_equal(f[start:], first_frame + rest % per)


@pytest.mark.parametrize("F,H,W", GEOMS)
def test_permute_unpermute_roundtrip_bitwise(F, H, W):
    """Pin: unpermute(permute(x)) == x bit for bit; permute moves row t to p[t]."""
    rng = np.random.default_rng(0)
    N = F * H * W
    x = rng.standard_normal((2, N, 8))
    for lay in (0, 1):
        order = O.executed_order(F, H, W, O.KIND_TEMPORAL, 1, lay)
        p = O.positions(order)
        xp = O.permute(x, order)
        assert np.array_equal(xp[:, p], x)
        assert np.array_equal(O.unpermute(xp, order), x)


# ---------------------------------------------------------------- masks

def _closed_form_spatial(F, S, b, k):
    total = 0
    for f in range(F):
        lo, hi = max(0, f - b), min(F - 1, f + b)
        frames = (hi - lo + 1) + min(k, lo) + max(0, k - 1 - hi)
        total += frames
    return S * S * total


def _closed_form_temporal(F, S, w, k):
    if w >= S - 1:
        per_s_sum = S * S
    else:
        per_s_sum = S * (2 * w + 1) - w * (w + 1)
    # every query keeps k*S sink keys plus, in each of the F-k other frames, its window
    return F * (k * S * S + (F - k) * per_s_sum)


@pytest.mark.parametrize("F,H,W", GEOMS)
@pytest.mark.parametrize("band", [0, 1, 2, 5, 40])
@pytest.mark.parametrize("sink", [0, 1, 2])
def test_retained_pairs_closed_form(F, H, W, band, sink):
    """Pin: closed-form retained-pair counts derived from the mask definitions."""
    sink = min(sink, F)
    S, N = H * W, F * H * W
    t = np.arange(N)
    ks = O.keep_block(O.KIND_SPATIAL, F, H, W, sink, band, t, t)
    kt = O.keep_block(O.KIND_TEMPORAL, F, H, W, sink, band, t, t)
    assert ks.sum() == _closed_form_spatial(F, S, band, sink)
    assert kt.sum() == _closed_form_temporal(F, S, band, sink)


def test_tiny_and_headline_kept_fractions():
    """Pin: closed forms at the tiny and 75,600-token sizes (38.88% mix; the page quotes about 38.87%)."""
    assert _closed_form_spatial(4, 32, 1, 1) / 128 ** 2 == 0.75
    assert _closed_form_temporal(4, 32, 2, 1) == 5944
    N = 21 * 3600
    sp = _closed_form_spatial(21, 3600, 4, 1) / N ** 2
    tp = _closed_form_temporal(21, 3600, 644, 1) / N ** 2
    assert abs(sp - 0.41950) < 5e-6 and abs(tp - 0.35810) < 5e-6
    assert abs((sp + tp) / 2 - 0.3888) < 1e-4


def test_mask_examples_by_hand():
    """Pin: single pairs read off the definitions (tiny latent, S=32)."""
    # spatial band 1: query frame 2 keeps key frames 0 (sink), 1, 2, 3
    assert O.keep_block(0, 4, 4, 8, 1, 1, [64], [0, 32, 64, 96]).all()
    # spatial band 1: query frame 3 drops key frame 1
    assert not O.keep_block(0, 4, 4, 8, 1, 1, [96], [32])[0, 0]
    # temporal window 2: query s=5 keeps key s=7 in any frame, drops s=8 outside the sink
    assert O.keep_block(1, 4, 4, 8, 1, 2, [5 + 64], [7 + 96])[0, 0]
    assert not O.keep_block(1, 4, 4, 8, 1, 2, [5 + 64], [8 + 96])[0, 0]
    assert O.keep_block(1, 4, 4, 8, 1, 2, [5 + 64], [8])[0, 0]          # sink key, frame 0


# ---------------------------------------------------------------- tile classification

def _interval_counts(F, H, W, kind, k, band, layout, bq, bkv):
    """Independent count: per-row key ranges written from closed-form positions."""
    S, N = H * W, F * H * W
    Tq, Tk = -(-N // bq), -(-N // bkv)
    c = np.zeros((Tq, Tk), dtype=np.int64)
    ind = np.zeros(Tk * bkv, dtype=np.int64)
    for i in range(N):
        ind[:] = 0
        if kind == 0:
            f = i // S
            lo, hi = max(0, f - band), min(F - 1, f + band)
            ind[0:k * S] = 1
            ind[lo * S:(hi + 1) * S] = 1
        elif layout == 0:
            if i < k * S:
                s = i % S
            else:
                s = (i - k * S) // (F - k)
            lo, hi = max(0, s - band), min(S - 1, s + band)
            ind[0:k * S] = 1
            ind[k * S + lo * (F - k):k * S + (hi + 1) * (F - k)] = 1
        else:
            s = i // F
            lo, hi = max(0, s - band), min(S - 1, s + band)
            ind[lo * F:(hi + 1) * F] = 1
            j = np.arange(N)
            ind[:N][j % F < k] = 1
        c[i // bq] += ind.reshape(Tk, bkv).sum(axis=1)
    return c


@pytest.mark.parametrize("F,H,W", [(4, 4, 8), (5, 3, 7), (3, 2, 5), (6, 2, 3), (2, 5, 1)])
@pytest.mark.parametrize("kind,layout", [(0, 0), (1, 0), (1, 1)])
@pytest.mark.parametrize("tiles", [(8, 8), (16, 8), (8, 32), (7, 5)])
@pytest.mark.parametrize("sink", [0, 1, 2])
def test_tile_counts_match_interval_count(F, H, W, kind, layout, tiles, sink):
    """Pin: element-scan counts equal an independent interval count written from closed-form positions."""
    sink = min(sink, F - 1) if kind == 1 else min(sink, F)
    band = 1 if kind == 0 else 2
    bq, bkv = tiles
    c = O.tile_counts(F, H, W, kind, sink, band, band, layout, bq, bkv)
    assert np.array_equal(c, _interval_counts(F, H, W, kind, sink, band, layout, bq, bkv))


def test_tile_counts_subset_equals_full_scan():
    """Restricting the scan to some query tiles leaves those rows unchanged."""
    full = O.tile_counts(5, 3, 7, 1, 1, 1, 2, 0, 16, 8)
    part = O.tile_counts(5, 3, 7, 1, 1, 1, 2, 0, 16, 8, q_tiles=[0, 3, 3, 6])
    assert np.array_equal(part[[0, 3, 6]], full[[0, 3, 6]])
    assert (np.delete(part, [0, 3, 6], axis=0) == -1).all()


def test_tiny_spatial_classes_match_hand_grid():
    """Pin: hand-derived class grid (tests/golden/tiny_spatial_classes.txt)."""
    want = np.array([[O.FULL if x == "F" else O.SKIP for x in row] for row in _read("tiny_spatial_classes.txt")])
    got = O.classify(4, 4, 8, O.KIND_SPATIAL, 1, 1, 2, 0, 32, 32, O.MODE_EXACT)["cls"]
    assert np.array_equal(got, want)


@pytest.mark.parametrize("F,H,W,bq,bkv", [(4, 4, 8, 32, 32), (9, 16, 24, 128, 128), (5, 3, 7, 16, 8), (3, 7, 5, 32, 16)])
@pytest.mark.parametrize("kind,layout", [(0, 0), (1, 0), (1, 1)])
def test_mode_relations(F, H, W, bq, bkv, kind, layout):
    """Pin: relations the page states between the traversals.

    B1 and B2 visit the same tiles and keep the same pairs; B1 masks every
    visited tile; B2 never masks a tile whose pairs are all kept and real;
    B0 visits everything; B3's mask is a union of whole tiles that contains
    every all-kept tile and no all-excluded tile.
    """
    N = F * H * W
    args = (F, H, W, kind, 1, 1, 2, layout, bq, bkv)
    ex = O.classify(*args, O.MODE_EXACT)
    nv = O.classify(*args, O.MODE_NAIVE)
    de = O.classify(*args, O.MODE_DENSE)
    rd = O.classify(*args, O.MODE_ROUNDED)
    assert np.array_equal(ex["cls"] != O.SKIP, nv["cls"] != O.SKIP)
    assert not (nv["cls"] == O.FULL).any()
    assert (de["cls"] != O.SKIP).all()
    pad_col = (np.arange(ex["Tk"]) + 1) * bkv > N
    assert np.array_equal(de["cls"] == O.BOUNDARY, np.broadcast_to(pad_col, de["cls"].shape))
    allkept = ex["counts"] == ex["area"]
    assert (rd["cls"][allkept] != O.SKIP).all()
    assert (rd["cls"][ex["counts"] == 0] == O.SKIP).all()
    assert not ((rd["cls"] == O.BOUNDARY) & ~pad_col[None, :]).any()
    # lists: full ascending then boundary ascending, exactly the classified tiles
    for r in (ex, nv, de, rd):
        for I in range(r["Tq"]):
            nf, nb = r["n_full"][I], r["n_bnd"][I]
            lst = r["kv"][I]
            assert np.array_equal(lst[:nf], np.nonzero(r["cls"][I] == O.FULL)[0])
            assert np.array_equal(lst[nf:nf + nb], np.nonzero(r["cls"][I] == O.BOUNDARY)[0])
            assert (lst[nf + nb:] == -1).all()
    # B3 keep rule is constant on each tile
    order = O.executed_order(F, H, W, kind, 1, layout)
    keep = O.rounded_keep_block(rd["cls"], F, H, W, kind, 1, layout, bq, bkv, order, order)
    for I in range(rd["Tq"]):
        for J in range(rd["Tk"]):
            blk = keep[I * bq:(I + 1) * bq, J * bkv:(J + 1) * bkv]
            assert blk.all() or not blk.any()
            assert blk.any() == (rd["cls"][I, J] != O.SKIP)


# ---------------------------------------------------------------- attention

def test_masked_attention_equals_torch_sdpa():
    """Pin: torch.nn.functional.scaled_dot_product_attention in float64 on the CPU, without and with a mask."""
    rng = np.random.default_rng(1)
    q, k, v = (rng.standard_normal((37, 16)) for _ in range(3))
    keep = rng.random((37, 37)) < 0.4
    keep[np.arange(37), np.arange(37)] = True
    scale = 1 / math.sqrt(16)
    for m in (np.ones_like(keep), keep):
        o, _, _ = O.masked_attention(q, k, v, m, scale)
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q)[None], torch.from_numpy(k)[None], torch.from_numpy(v)[None],
            attn_mask=torch.from_numpy(m)[None], scale=scale)[0].numpy()
        assert np.abs(o - ref).max() < 1e-13


def test_log_sum_exp_matches_scipy():
    """Pin: scipy.special.logsumexp over the kept scaled scores."""
    from scipy.special import logsumexp
    rng = np.random.default_rng(2)
    q, k, v = (rng.standard_normal((20, 8)) for _ in range(3))
    keep = rng.random((20, 20)) < 0.5
    keep[:, 0] = True
    _, lse, _ = O.masked_attention(q, k, v, keep, 0.3)
    s = (q @ k.T) * 0.3
    for i in range(20):
        assert abs(lse[i] - logsumexp(s[i][keep[i]])) < 1e-12


def test_excluded_pairs_get_exactly_zero_weight_and_rows_sum_to_one():
    """Pin: the page's rule that excluded pairs contribute zero weight; softmax rows sum to 1."""
    rng = np.random.default_rng(3)
    F, H, W = 4, 4, 8
    t = np.arange(128)
    for kind in (0, 1):
        keep = O.keep_block(kind, F, H, W, 1, 1 if kind == 0 else 2, t, t)
        q, k, v = (rng.standard_normal((128, 64)) * 3 for _ in range(3))
        _, _, p = O.masked_attention(q, k, v, keep, 0.125)
        assert (p[~keep] == 0.0).all()
        assert (p[keep] > 0).all()
        assert np.abs(p.sum(axis=1) - 1).max() < 1e-12


def test_empty_row_and_single_key_row():
    """Pin: special cases. A row with no kept key gives 0 and -inf; a row with one kept key returns that value row exactly."""
    rng = np.random.default_rng(4)
    q, k, v = (rng.standard_normal((3, 5)) for _ in range(3))
    keep = np.array([[False] * 3, [False, True, False], [True] * 3])
    o, lse, _ = O.masked_attention(q, k, v, keep, 1.0)
    assert (o[0] == 0).all() and lse[0] == -np.inf
    assert np.array_equal(o[1], v[1])
    assert abs(lse[1] - q[1] @ k[1]) < 1e-15


def test_census_averages_residue_classes():
    """Pin: with Q = 0 every kept key has equal weight, so with V[k, c] = [k mod d == c]
    the output is the share of each row's kept keys in each residue class."""
    F, H, W, d = 4, 4, 8, 16
    N = 128
    t = np.arange(N)
    keep = O.keep_block(1, F, H, W, 1, 2, t, t)
    q = np.zeros((N, d))
    k = np.zeros((N, d))
    v = np.zeros((N, d))
    v[t, t % d] = 1
    o, _, _ = O.masked_attention(q, k, v, keep, 0.25)
    for i in range(N):
        kept = np.nonzero(keep[i])[0]
        want = np.bincount(kept % d, minlength=d) / kept.size
        assert np.abs(o[i] - want).max() < 1e-15


@pytest.mark.parametrize("kind,layout", [(0, 0), (1, 0), (1, 1)])
def test_attention_does_not_depend_on_token_order(kind, layout):
    """Pin: permuting tokens (rows of Q, K, V and both axes of the mask) permutes the output rows."""
    rng = np.random.default_rng(5)
    F, H, W, d = 5, 3, 4, 8
    N = F * H * W
    t = np.arange(N)
    q, k, v = (rng.standard_normal((N, d)) for _ in range(3))
    keep = O.keep_block(kind, F, H, W, 1, 1, t, t)
    o, lse, _ = O.masked_attention(q, k, v, keep, 0.4)
    order = O.executed_order(F, H, W, kind, 1, layout)
    op, lsep, _ = O.masked_attention(q[order], k[order], v[order], keep[np.ix_(order, order)], 0.4)
    assert np.abs(O.unpermute(op, order) - o).max() < 1e-13
    assert np.abs(lsep - lse[order]).max() < 1e-13


def test_attention_head_modes():
    """Pin: B1 and B2 keep the same pairs so their outputs agree; B0 equals unmasked attention."""
    rng = np.random.default_rng(6)
    F, H, W, d = 4, 4, 8, 16
    N = 128
    q, k, v = (rng.standard_normal((N, d)) for _ in range(3))
    args = (1, F, H, W, 1, 1, 2, 0)
    o_ex, _ = O.attention_head(q, k, v, *args, O.MODE_EXACT, 32, 32, 0.25)
    o_nv, _ = O.attention_head(q, k, v, *args, O.MODE_NAIVE, 32, 32, 0.25)
    o_de, _ = O.attention_head(q, k, v, *args, O.MODE_DENSE, 32, 32, 0.25)
    assert np.array_equal(o_ex, o_nv)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None], torch.from_numpy(k)[None], torch.from_numpy(v)[None], scale=0.25)[0].numpy()
    assert np.abs(o_de - ref).max() < 1e-13


# ---------------------------------------------------------------- routing

def _loop_attention(qi, k, v, kept, scale):
    scores = [sum(qi[c] * k[j][c] for c in range(len(qi))) * scale for j in kept]
    m = max(scores)
    w = [math.exp(x - m) for x in scores]
    tot = sum(w)
    return [sum(w[n] * v[j][c] for n, j in enumerate(kept)) / tot for c in range(len(v[0]))]


def test_routing_matches_python_loops_on_tiny():
    """Pin: brute force with plain Python loops, mask read directly off frame and spatial index."""
    F, H, W, d = 3, 2, 4, 6
    S, N = 8, 24
    rng = np.random.default_rng(7)
    q, k, v = (rng.standard_normal((1, 2, N, d)) * 2 for _ in range(3))
    idx = [1, 9, 14, 23]
    scale = 1 / math.sqrt(d)
    flags, err = O.route_heads(q, k, v, F, H, W, 1, 1, 1, idx, scale)
    for h in range(2):
        e = [0.0, 0.0]
        kk, vv = k[0, h].tolist(), v[0, h].tolist()
        for i in idx:
            qi = q[0, h, i].tolist()
            dense = _loop_attention(qi, kk, vv, list(range(N)), scale)
            sp = [j for j in range(N) if j // S == 0 or abs(j // S - i // S) <= 1]
            tp = [j for j in range(N) if j // S == 0 or abs(j % S - i % S) <= 1]
            for x, kept in enumerate((sp, tp)):
                o = _loop_attention(qi, kk, vv, kept, scale)
                e[x] += sum((a - b) ** 2 for a, b in zip(o, dense))
        assert abs(err[0, h, 0] - e[0]) < 1e-12 * max(1, e[0])
        assert abs(err[0, h, 1] - e[1]) < 1e-12 * max(1, e[1])
        assert flags[0, h] == (1 if e[1] < e[0] else 0)


def test_routing_degenerate_masks():
    """Pin: a band covering every frame makes the spatial mask dense (error exactly 0, flag spatial);
    a window covering every position makes the temporal mask dense (flag temporal)."""
    F, H, W, d = 4, 2, 3, 8
    N = 24
    rng = np.random.default_rng(8)
    q, k, v = (rng.standard_normal((1, 1, N, d)) for _ in range(3))
    flags, err = O.route_heads(q, k, v, F, H, W, 1, F - 1, 1, [0, 7, 20], 0.35)
    assert err[0, 0, 0] == 0.0 and flags[0, 0] == 0
    flags, err = O.route_heads(q, k, v, F, H, W, 1, 0, H * W - 1, [0, 7, 20], 0.35)
    assert err[0, 0, 1] == 0.0 and err[0, 0, 0] > 0 and flags[0, 0] == 1


def test_routing_finds_planted_head_kinds():
    """Pin: queries/keys sharing a per-frame vector route spatial; sharing a per-position vector route temporal."""
    F, H, W, d = 9, 16, 24, 128
    kinds = (0, 1, 1, 0)
    q, k, v = planted_qkv(1, F, H, W, d, kinds, seed=3)
    idx = np.sort(np.random.default_rng(0).choice(F * H * W, 64, replace=False))
    flags, err = O.route_heads(q.float().numpy(), k.float().numpy(), v.float().numpy(),
                               F, H, W, 1, 1, 24, idx, 1 / math.sqrt(d))
    assert tuple(flags[0]) == kinds


# ---------------------------------------------------------------- balanced rounding (B3)

# Tile statistics from an independent per-row interval calculation made before
# any of this code (not from the pages, whose band widths are lost): the class
# totals of the exact classification (FULL, BOUNDARY, SKIP, kept pairs) and of
# the balanced rounding (FULL, BOUNDARY, kept pairs). Keyed by
# (workload, kind, bq, bkv); geometry and masks as in synth.workloads.
INDEPENDENT_COUNTS = {
    ("tiny", 0, 32, 32): ((12, 0, 4, 12_288), (12, 0, 12_288)),
    ("tiny", 1, 32, 32): ((4, 10, 2, 5_944), (4, 0, 4_096)),
    ("small", 0, 128, 128): ((288, 0, 441, 4_718_592), (288, 0, 4_718_592)),
    ("small", 1, 128, 128): ((105, 122, 502, 2_638_656), (151, 0, 2_473_984)),
    ("headline", 0, 128, 128): ((145_514, 2_083, 201_684, 2_397_600_000), (146_358, 141, 2_398_337_280)),
    ("headline", 1, 128, 128): ((123_134, 3_608, 222_539, 2_046_668_400), (124_666, 106, 2_042_822_912)),
    ("headline", 0, 256, 128): ((72_616, 1_478, 100_842, 2_397_600_000), (73_274, 71, 2_398_697_728)),
    ("headline", 1, 256, 128): ((61_110, 2_830, 110_996, 2_046_668_400), (62_637, 53, 2_050_676_992)),
    ("headline", 0, 512, 128): ((36_013, 1_202, 50_253, 2_397_600_000), (36_705, 36, 2_403_174_656)),
    ("headline", 1, 512, 128): ((30_034, 2_438, 54_996, 2_046_668_400), (31_319, 27, 2_050_707_712)),
}
WORKLOAD_ARGS = {   # F, H, W, sink, spatial band, temporal band, layout
    "tiny": (4, 4, 8, 1, 1, 2, 0),
    "small": (9, 16, 24, 1, 1, 24, 0),
    "headline": (21, 45, 80, 1, 4, 644, 0),
}


def _b3_totals(r):
    kept = r["cls"] != O.SKIP
    return (int((r["cls"] == O.FULL).sum()), int((r["cls"] == O.BOUNDARY).sum()), int((r["area"] * kept).sum()))


@pytest.mark.parametrize("key", [k for k in INDEPENDENT_COUNTS if k[0] != "headline"],
                         ids=lambda k: f"{k[0]}-{'spatial' if k[1] == 0 else 'temporal'}-{k[2]}x{k[3]}")
def test_rounding_matches_independent_counts(key):
    """Pin: the oracle's exact and balanced-rounding (B3) classifications, run here by element scan,
    reproduce the independent interval counts above: FULL / BOUNDARY / SKIP totals and kept pairs.
    The rounding rule (keep a tile iff it holds a kept pair and kept pairs fill at least half its
    valid area) is fixed by these numbers: rounding every boundary tile outward keeps 227 tiles and
    3,719,168 pairs at the small temporal size, inward 105 tiles, against 151 and 2,473,984."""
    name, kind, bq, bkv = key
    F, H, W, sink, bs, bt, lay = WORKLOAD_ARGS[name]
    counts = O.tile_counts(F, H, W, kind, sink, bs, bt, lay, bq, bkv)
    ex = O.classify(F, H, W, kind, sink, bs, bt, lay, bq, bkv, O.MODE_EXACT, counts=counts)
    rd = O.classify(F, H, W, kind, sink, bs, bt, lay, bq, bkv, O.MODE_ROUNDED, counts=counts)
    want_ex, want_rd = INDEPENDENT_COUNTS[key]
    got_ex = (int((ex["cls"] == O.FULL).sum()), int((ex["cls"] == O.BOUNDARY).sum()),
              int((ex["cls"] == O.SKIP).sum()), int(counts.sum()))
    assert got_ex == want_ex
    assert _b3_totals(rd) == want_rd


@pytest.mark.parametrize("bq", [128, 256, 512])
def test_headline_rounding_goldens_match_independent_counts(bq):
    """Pin: the 75,600-token tile totals that tests/golden/make_tilemap_golden.py wrote with the
    oracle's element scan (about 40 s per head kind, so stored rather than rerun here) equal the
    independent interval counts, for the exact and the balanced-rounding classification."""
    g = json.load(open(os.path.join(GOLDEN, f"tilemap_headline_{bq}x128.json")))
    assert (g["F"], g["H"], g["W"], g["sink_frames"], g["spatial_band"], g["temporal_band"],
            g["temporal_layout"]) == WORKLOAD_ARGS["headline"]
    for kind, kname in ((0, "spatial"), (1, "temporal")):
        want_ex, want_rd = INDEPENDENT_COUNTS[("headline", kind, bq, 128)]
        ex, rd = g["kinds"][kname]["exact"], g["kinds"][kname]["rounded"]
        assert (ex["full"], ex["boundary"], ex["skip"], ex["retained_pairs"]) == want_ex
        assert (rd["full"], rd["boundary"], rd["retained_pairs"]) == want_rd


@pytest.mark.parametrize("tiles", [(128, 128), (64, 64), (256, 128), (96, 64)])
@pytest.mark.parametrize("kind", [0, 1])
def test_rounding_keeps_the_pair_budget(kind, tiles):
    """Pin: the page asks balanced rounding to keep the kept-pair budget approximately. At the small
    workload (3,456 tokens) the rounded mask keeps within 10% of the exact mask's pairs, and at the
    75,600-token workload (stored totals) within 1%; outward-only rounding keeps 41% more at the
    small temporal size. Every all-kept tile stays and no all-excluded tile is added."""
    F, H, W, sink, bs, bt, lay = WORKLOAD_ARGS["small"]
    bq, bkv = tiles
    args = (F, H, W, kind, sink, bs, bt, lay, bq, bkv)
    counts = O.tile_counts(*args)
    ex = O.classify(*args, O.MODE_EXACT, counts=counts)
    rd = O.classify(*args, O.MODE_ROUNDED, counts=counts)
    exact_pairs = int(counts.sum())
    rounded_pairs = _b3_totals(rd)[2]
    assert abs(rounded_pairs - exact_pairs) <= 0.10 * exact_pairs, (rounded_pairs, exact_pairs)
    assert (rd["cls"][ex["cls"] == O.FULL] == O.FULL).all()
    assert (rd["cls"][ex["cls"] == O.SKIP] == O.SKIP).all()
    for (name, k, _, _), (want_ex, want_rd) in INDEPENDENT_COUNTS.items():
        if name == "headline":
            assert abs(want_rd[2] - want_ex[3]) <= 0.01 * want_ex[3]


def test_rounding_tie_by_hand():
    """Pin: a hand-counted tie. Two frames of 4 tokens, spatial band 0, no sink, one 8 x 8 tile:
    each query keeps the 4 keys of its own frame, so 32 of the 64 pairs are kept, exactly half.
    The adopted reading keeps ties (rounds them outward), so the whole tile is kept, FULL."""
    c = O.tile_counts(2, 1, 4, O.KIND_SPATIAL, 0, 0, 0, 0, 8, 8)
    assert c.tolist() == [[32]]
    rd = O.classify(2, 1, 4, O.KIND_SPATIAL, 0, 0, 0, 0, 8, 8, O.MODE_ROUNDED)
    assert rd["cls"].tolist() == [[O.FULL]]
    # one key fewer per row (3 x 4 tokens, band 0: 3 x 16 = 48 of 144 pairs) rounds inward
    rd = O.classify(3, 1, 4, O.KIND_SPATIAL, 0, 0, 0, 0, 12, 12, O.MODE_ROUNDED)
    assert rd["cls"].tolist() == [[O.SKIP]]
