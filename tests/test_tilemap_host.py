"""Host tile-map builder (C++, via the C ABI) against the oracle's element scan, bit for bit."""
import glob
import hashlib
import json
import os

import numpy as np
import pytest

import block_sparse_spatio_amd as B
import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def check_against_oracle(F, H, W, sink, bs, bt, lay, bq, bkv, mode):
    blob = B.svga_build_tilemap_host((F, H, W), (sink, bs, bt, lay), bq, bkv, mode)
    v = B.tilemap_views(blob, (F, H, W), bq, bkv)
    hdr = v["header"]
    assert hdr[0] == 0x4D475653 and list(hdr[2:5]) == [F, H, W] and list(hdr[9:14]) == [bq, bkv, v["tq"], v["tk"], mode]
    for kind in (0, 1):
        r = O.classify(F, H, W, kind, sink, bs, bt, lay, bq, bkv, mode)
        assert np.array_equal(v["cls"][kind], r["cls"]), (kind, mode)
        assert np.array_equal(v["n_full"][kind], r["n_full"])
        assert np.array_equal(v["n_bnd"][kind], r["n_bnd"])
        assert np.array_equal(v["kv"][kind], r["kv"])


@pytest.mark.parametrize("mode", [0, 1, 2, 3])
@pytest.mark.parametrize("lay", [0, 1])
def test_named_small_geometries(mode, lay):
    check_against_oracle(4, 4, 8, 1, 1, 2, lay, 32, 32, mode)
    check_against_oracle(9, 16, 24, 1, 1, 24, lay, 128, 128, mode)
    check_against_oracle(9, 16, 24, 1, 1, 24, lay, 64, 128, mode)


def test_random_geometries():
    """Random latents, bands, sink counts, layouts, tile shapes (including ragged tails and tiles larger than N)."""
    rng = np.random.default_rng(123)
    for _ in range(160):
        F, H, W = (int(x) for x in rng.integers(1, 9, 3))
        sink = int(rng.integers(0, F + 1))
        bs = int(rng.integers(0, F + 1))
        bt = int(rng.integers(0, H * W + 2))
        lay = int(rng.integers(0, 2))
        bq = int(rng.choice([1, 2, 3, 5, 8, 16, 32, 64, 100]))
        bkv = int(rng.choice([1, 2, 4, 7, 8, 16, 32, 64, 100]))
        mode = int(rng.integers(0, 4))
        check_against_oracle(F, H, W, sink, bs, bt, lay, bq, bkv, mode)


def _sha(a, dt):
    return hashlib.sha256(np.ascontiguousarray(a, dtype=dt).tobytes()).hexdigest()


GOLDEN_FILES = sorted(glob.glob(os.path.join(GOLDEN, "tilemap_*.json")))


@pytest.mark.parametrize("path", GOLDEN_FILES, ids=[os.path.basename(p) for p in GOLDEN_FILES])
def test_against_oracle_golden(path):
    """Full-size maps against digests the oracle wrote (tests/golden/make_tilemap_golden.py)."""
    g = json.load(open(path))
    geom = (g["F"], g["H"], g["W"])
    mask = (g["sink_frames"], g["spatial_band"], g["temporal_band"], g["temporal_layout"])
    for mname, mode in B.MODES.items():
        blob = B.svga_build_tilemap_host(geom, mask, g["bq"], g["bkv"], mode)
        v = B.tilemap_views(blob, geom, g["bq"], g["bkv"])
        for kind, kname in ((0, "spatial"), (1, "temporal")):
            want = g["kinds"][kname][mname]
            cls = v["cls"][kind]
            assert int((cls == 1).sum()) == want["full"]
            assert int((cls == 2).sum()) == want["boundary"]
            assert _sha(cls, "<i1") == want["sha_cls"], (mname, kname)
            assert _sha(v["n_full"][kind], "<i4") == want["sha_n_full"]
            assert _sha(v["n_bnd"][kind], "<i4") == want["sha_n_bnd"]
            assert _sha(v["kv"][kind], "<i4") == want["sha_kv"]
