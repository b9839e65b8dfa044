"""The sparsity knob (svga_mask_for_kept_fraction) and the schedule type, on the CPU.

The bands the library picks are checked against kept-pair counts from the
oracle's element-by-element mask scan (small geometries, every band) and, at
the 75,600- and 302,400-token sizes, against the closed forms that
test_oracle.py pins to that scan. The expected band is the smallest whose
kept count reaches target * N^2, compared with exact rationals.
"""
import ctypes
import math
from fractions import Fraction

import numpy as np
import pytest

import block_sparse_spatio_amd as B
import oracle as O
from block_sparse_spatio_amd import _lib
from block_sparse_spatio_amd._lib import SvgaGeom, SvgaMask
from test_oracle import _closed_form_spatial, _closed_form_temporal


def oracle_kept_by_band(kind, F, H, W, sink):
    """Kept pairs of one head for every band from 0 to the first that keeps all pairs."""
    N, S = F * H * W, H * W
    t = np.arange(N)
    last = F - 1 if kind == O.KIND_SPATIAL else S - 1
    return [int(O.keep_block(kind, F, H, W, sink, b, t, t).sum()) for b in range(last + 1)]


def expected_band(kept, target, N):
    need = Fraction(target) * N * N
    return next(b for b, c in enumerate(kept) if c >= need)


def targets_for(kept, N, rng):
    ts = {0.0, 1.0}
    for c in kept:
        x = c / (N * N)     # the count's fraction rounded to double, and its neighbours
        ts.update({x, math.nextafter(x, 0.0), min(1.0, math.nextafter(x, 2.0))})
    ts.update(float(u) for u in rng.random(8))
    return sorted(ts)


@pytest.mark.parametrize("geom", [(4, 4, 8), (5, 3, 7), (3, 1, 1), (1, 2, 3), (7, 2, 2), (6, 1, 5)])
@pytest.mark.parametrize("sink", [0, 1, 2])
def test_knob_matches_oracle_counts(geom, sink):
    F, H, W = geom
    sink = min(sink, F)
    N = F * H * W
    rng = np.random.default_rng(F * 100 + H * 10 + W + sink)
    ks = oracle_kept_by_band(O.KIND_SPATIAL, F, H, W, sink)
    kt = oracle_kept_by_band(O.KIND_TEMPORAL, F, H, W, sink)
    for lay in (B.TL_SINK_FIRST, B.TL_LITERAL):
        for ts_ in targets_for(ks, N, rng):
            for tt in targets_for(kt, N, rng)[::3] + [ts_]:
                m, (cs, ct) = B.svga_mask_for_kept_fraction(geom, sink, ts_, tt, lay)
                bs, bt = expected_band(ks, ts_, N), expected_band(kt, tt, N)
                assert (m.sink_frames, m.spatial_band, m.temporal_band, m.temporal_layout) == (sink, bs, bt, lay), \
                    (geom, sink, ts_, tt)
                assert (cs, ct) == (ks[bs], kt[bt])


def test_knob_at_the_large_sizes():
    """75,600 and 302,400 tokens: the bands of the 38.9% mix and of the 1440p layer come back from their fractions."""
    for F, H, W in [(21, 45, 80), (21, 90, 160)]:
        S, N = H * W, F * H * W
        ks = [_closed_form_spatial(F, S, b, 1) for b in range(F)]
        kt = [_closed_form_temporal(F, S, w, 1) for w in range(S)]
        assert ks[-1] == kt[-1] == N * N
        rng = np.random.default_rng(N)
        for ts_, tt in [(0.4195, 0.3581), (ks[4] / N ** 2, kt[644] / N ** 2), (0.0, 1.0), (1.0, 0.0)] + \
                [tuple(rng.random(2)) for _ in range(20)]:
            m, kept = B.svga_mask_for_kept_fraction((F, H, W), 1, ts_, tt)
            bs, bt = expected_band(ks, ts_, N), expected_band(kt, tt, N)
            assert (m.spatial_band, m.temporal_band) == (bs, bt)
            assert kept == (ks[bs], kt[bt])
    # the headline masks: spatial band 4 (41.95% kept), temporal window 644 (35.81% kept)
    m, _ = B.svga_mask_for_kept_fraction((21, 45, 80), 1, 0.4194, 0.3580)
    assert (m.spatial_band, m.temporal_band) == (4, 644)


def test_knob_rejects_bad_arguments():
    L = _lib.lib()
    g = ctypes.byref(SvgaGeom(4, 4, 8))
    out = SvgaMask()
    for ts_, tt in [(-0.1, 0.5), (0.5, 1.5), (float("nan"), 0.5), (0.5, float("inf"))]:
        assert L.svga_mask_for_kept_fraction(g, 1, 0, ts_, tt, ctypes.byref(out), None) == B.SVGA_EINVAL
    assert L.svga_mask_for_kept_fraction(g, 5, 0, 0.5, 0.5, ctypes.byref(out), None) == B.SVGA_EINVAL   # sink > F
    assert L.svga_mask_for_kept_fraction(g, 1, 2, 0.5, 0.5, ctypes.byref(out), None) == B.SVGA_EINVAL   # layout
    assert L.svga_mask_for_kept_fraction(g, 1, 0, 0.5, 0.5, None, None) == B.SVGA_EINVAL
    assert L.svga_mask_for_kept_fraction(ctypes.byref(SvgaGeom(0, 4, 8)), 1, 0, 0.5, 0.5, ctypes.byref(out),
                                         None) == B.SVGA_EINVAL
    with pytest.raises(B.SvgaError):
        B.svga_mask_for_kept_fraction((4, 4, 8), 1, 1.01, 0.5)


def test_schedule_maps_steps_and_layers():
    geom = (9, 16, 24)
    sched = B.SparsitySchedule(geom, [(2, 0.7, 0.6), (10, 0.5, 0.4), (30, 0.35, 0.25)], sink_frames=1,
                               dense_layers=(0,))
    N = 9 * 16 * 24
    # dense before the first level and on dense layers
    for step, layer in [(0, 3), (1, 5), (12, 0)]:
        p = sched.plan(step, layer)
        assert p.mode == B.MAP_DENSE and p.kept_pairs == (N * N, N * N)
    # each level's mask is the knob's for its targets, and kept pairs fall level by level
    prev = (N * N + 1, N * N + 1)
    for step, lv in [(2, 0), (9, 0), (10, 1), (29, 1), (30, 2), (39, 2)]:
        p = sched.plan(step, 4)
        level = sched.levels[lv]
        m, kept = B.svga_mask_for_kept_fraction(geom, 1, level.spatial, level.temporal)
        assert p.mode == B.MAP_EXACT and p.kept_pairs == kept
        assert (p.mask.spatial_band, p.mask.temporal_band) == (m.spatial_band, m.temporal_band)
        assert kept[0] >= level.spatial * N * N and kept[1] >= level.temporal * N * N
    levels = [sched.plan(s, 4).kept_pairs for s in (2, 10, 30)]
    assert all(a[0] >= b[0] and a[1] >= b[1] for a, b in zip(levels, levels[1:]))
    assert levels[0] != levels[-1] and prev[0] > levels[0][0]
    with pytest.raises(ValueError):
        B.SparsitySchedule(geom, [(5, 0.5, 0.5), (5, 0.4, 0.4)])
    with pytest.raises(B.SvgaError):
        B.SparsitySchedule(geom, [(0, 0.5, 1.5)])
