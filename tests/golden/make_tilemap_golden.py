"""Write tests/golden/tilemap_*.json from the oracle's brute-force tile scan.

Calls only ``oracle``. For each workload, tile shape and head kind it stores
the class totals, the retained-pair totals and SHA-256 digests of the canonical
arrays (class matrix as int8; full/boundary counts and kv lists as little-endian
int32), so the library's tile maps can be compared bit for bit without storing
the arrays themselves.

usage: python tests/golden/make_tilemap_golden.py headline 128x128 256x128 512x128
"""
import hashlib
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle as O  # noqa: E402

# geometry and mask parameters of the named workloads (F, H, W, sink, band_s, band_t, layout)
GEOM = {
    "small": (9, 16, 24, 1, 1, 24, 0),
    "headline": (21, 45, 80, 1, 4, 644, 0),
    "1440p": (21, 90, 160, 1, 2, 2054, 0),
}
MODES = {"dense": O.MODE_DENSE, "naive": O.MODE_NAIVE, "exact": O.MODE_EXACT, "rounded": O.MODE_ROUNDED}


def digest(a, dtype):
    return hashlib.sha256(np.ascontiguousarray(a, dtype=dtype).tobytes()).hexdigest()


def summarize(F, H, W, kind, sink, bs, bt, lay, bq, bkv):
    counts = O.tile_counts(F, H, W, kind, sink, bs, bt, lay, bq, bkv)
    out = {}
    for name, mode in MODES.items():
        r = O.classify(F, H, W, kind, sink, bs, bt, lay, bq, bkv, mode, counts=counts)
        kept = (r["cls"] != O.SKIP)
        if mode == O.MODE_ROUNDED:
            retained = int((r["area"] * kept).sum())
        elif mode == O.MODE_DENSE:
            retained = int(r["area"].sum())
        else:
            retained = int(counts.sum())
        out[name] = {
            "full": int((r["cls"] == O.FULL).sum()),
            "boundary": int((r["cls"] == O.BOUNDARY).sum()),
            "skip": int((r["cls"] == O.SKIP).sum()),
            "retained_pairs": retained,
            "sha_cls": digest(r["cls"], "<i1"),
            "sha_n_full": digest(r["n_full"], "<i4"),
            "sha_n_bnd": digest(r["n_bnd"], "<i4"),
            "sha_kv": digest(r["kv"], "<i4"),
        }
    return out


def main():
    name = sys.argv[1]
    F, H, W, sink, bs, bt, lay = GEOM[name]
    for spec in sys.argv[2:]:
        bq, bkv = (int(x) for x in spec.split("x"))
        res = {"workload": name, "F": F, "H": H, "W": W, "sink_frames": sink, "spatial_band": bs,
               "temporal_band": bt, "temporal_layout": lay, "bq": bq, "bkv": bkv,
               "source": "oracle.tile_counts element scan (tests/golden/make_tilemap_golden.py)",
               "kinds": {}}
        for kind, kname in ((O.KIND_SPATIAL, "spatial"), (O.KIND_TEMPORAL, "temporal")):
            res["kinds"][kname] = summarize(F, H, W, kind, sink, bs, bt, lay, bq, bkv)
            print(name, spec, kname, res["kinds"][kname]["exact"], flush=True)
        path = os.path.join(os.path.dirname(os.path.abspath(__file__)), f"tilemap_{name}_{bq}x{bkv}.json")
        with open(path, "w") as fh:
            json.dump(res, fh, indent=1, sort_keys=True)


if __name__ == "__main__":
    main()
