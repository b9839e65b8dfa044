"""GPU parity of the HIP path (through the C ABI) against the oracle, at sizes the oracle finishes in seconds.

Bars: tile maps and permutations bit-exact; bf16 attention outputs within
max-abs 2e-2 and mean-abs 2e-3 of the fp64 oracle (plus exact-rational census
checks); routing errors within 1e-3 relative, flags equal except near-ties.
"""
import dataclasses
import math

import numpy as np
import pytest
import torch

import block_sparse_spatio_amd as B
import oracle as O
from synth import SMALL, TINY, census_qkv, normal_qkv, planted_qkv, sample_indices

pytestmark = pytest.mark.gpu

MAX_ABS, MEAN_ABS = 2e-2, 2e-3


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def say(*a):
    print(*a, flush=True)


def i16(t):
    return t.contiguous().view(torch.int16).cpu().numpy()


def run_attention(dev, geom, mask, q, k, v, kinds, bq, bkv, mode, gather=False, want_lse=False, workspace=None):
    """Frame-major in, frame-major out: permute -> attention -> unpermute (or the in-kernel gather).
    LSE rows come back in frame-major order too."""
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    Bn = q.shape[0]
    flags = torch.tensor([list(kinds)] * Bn, dtype=torch.uint8, device=dev)
    tm = B.svga_build_tilemap(geom, mask, bq, bkv, mode, device=dev)
    if gather:
        o, lse = B.svga_sparse_attn_fwd(qd, kd, vd, flags, tm, geom, mask, bq, bkv, mode, gather_temporal=True,
                                        want_lse=want_lse, workspace=workspace)
    else:
        qp, kp, vp = (B.svga_permute(x, flags, geom, mask) for x in (qd, kd, vd))
        op, lsep = B.svga_sparse_attn_fwd(qp, kp, vp, flags, tm, geom, mask, bq, bkv, mode, want_lse=want_lse,
                                          workspace=workspace)
        o = B.svga_unpermute(op, flags, geom, mask)
        lse = None
        if want_lse:
            # LSE rows follow the executed order; bring temporal heads back to frame-major
            lse = lsep.clone()
            for h, kind in enumerate(kinds):
                if kind:
                    order = torch.from_numpy(O.executed_order(geom[0], geom[1], geom[2], 1, mask[0], mask[3])).to(dev)
                    lse[:, h, order] = lsep[:, h]
    torch.cuda.synchronize()
    return o.cpu(), (lse.cpu() if lse is not None else None)


def oracle_head(geom, mask, q, k, v, kind, mode, bq, bkv, scale, rows=None):
    F, H, W = geom
    sink, bs, bt, lay = mask
    cls_r = None
    if mode == O.MODE_ROUNDED:
        cls_r = O.classify(F, H, W, kind, sink, bs, bt, lay, bq, bkv, O.MODE_ROUNDED)["cls"]
    return O.attention_head(q.double().numpy(), k.double().numpy(), v.double().numpy(), kind, F, H, W, sink, bs,
                            bt, lay, mode, bq, bkv, scale, rows=rows, cls_rounded=cls_r)


def assert_close(got, ref, what):
    err = np.abs(got.astype(np.float64) - ref)
    say(f"  {what}: max-abs {err.max():.3e} mean-abs {err.mean():.3e}")
    assert np.isfinite(got).all(), what
    assert err.max() < MAX_ABS and err.mean() < MEAN_ABS, what


# ---------------------------------------------------------------- tile maps

@pytest.mark.parametrize("w", [TINY, SMALL], ids=["tiny", "small"])
@pytest.mark.parametrize("mode", [0, 1, 2, 3])
@pytest.mark.parametrize("lay", [0, 1])
def test_device_tilemap_equals_host(dev, w, mode, lay):
    geom = (w.F, w.H, w.W)
    mask = (w.sink_frames, w.spatial_band, w.temporal_band, lay)
    say(f"tilemap {w.name} mode={mode} layout={lay}")
    for bq, bkv in ((w.bq, w.bkv), (64, 32), (32, 64)):
        d = B.svga_build_tilemap(geom, mask, bq, bkv, mode, device=dev).cpu().numpy()
        h = B.svga_build_tilemap_host(geom, mask, bq, bkv, mode)
        assert np.array_equal(d, h), (bq, bkv)


def test_device_tilemap_random_geometries(dev):
    rng = np.random.default_rng(9)
    for it in range(40):
        F, H, W = (int(x) for x in rng.integers(1, 12, 3))
        sink = int(rng.integers(0, F + 1))
        mask = (sink, int(rng.integers(0, F + 1)), int(rng.integers(0, H * W + 2)), int(rng.integers(0, 2)))
        bq, bkv = int(rng.choice([1, 3, 16, 32, 64, 128])), int(rng.choice([1, 5, 16, 32, 64, 128]))
        mode = int(rng.integers(0, 4))
        say(f"tilemap random #{it}: geom={(F, H, W)} mask={mask} tiles={bq}x{bkv} mode={mode}")
        d = B.svga_build_tilemap((F, H, W), mask, bq, bkv, mode, device=dev).cpu().numpy()
        h = B.svga_build_tilemap_host((F, H, W), mask, bq, bkv, mode)
        assert np.array_equal(d, h)


# ---------------------------------------------------------------- permutation

@pytest.mark.parametrize("geom", [(4, 4, 8), (9, 16, 24), (5, 3, 7), (3, 1, 1)])
@pytest.mark.parametrize("sink", [0, 1, 2])
@pytest.mark.parametrize("lay", [0, 1])
@pytest.mark.parametrize("d", [64, 128, 8])
def test_permute_unpermute_bitwise(dev, geom, sink, lay, d):
    F, H, W = geom
    sink = min(sink, F)
    N = F * H * W
    mask = (sink, 1, 2, lay)
    kinds = (0, 1, 1, 0, 1)
    say(f"permute geom={geom} sink={sink} layout={lay} d={d}")
    x = torch.randn(2, len(kinds), N, d).to(torch.bfloat16)
    flags = torch.tensor([kinds, kinds[::-1]], dtype=torch.uint8, device=dev)
    xd = x.to(dev)
    xp = B.svga_permute(xd, flags, geom, mask)
    back = B.svga_unpermute(xp, flags, geom, mask)
    torch.cuda.synchronize()
    order = O.executed_order(F, H, W, O.KIND_TEMPORAL, sink, lay)
    xn = i16(x)
    want = xn.copy()
    fl = flags.cpu().numpy()
    for b in range(2):
        for h in range(len(kinds)):
            if fl[b, h]:
                want[b, h] = O.permute(xn[b, h], order)
    assert np.array_equal(i16(xp), want)
    assert np.array_equal(i16(back), xn)


# ---------------------------------------------------------------- attention

@pytest.mark.parametrize("mode", [0, 1, 2, 3])
@pytest.mark.parametrize("src_dtype", ["fp32", "bf16"])
def test_attention_tiny(dev, mode, src_dtype):
    w = TINY
    geom = (w.F, w.H, w.W)
    mask = (w.sink_frames, w.spatial_band, w.temporal_band, w.temporal_layout)
    say(f"attention tiny mode={mode} inputs={src_dtype}")
    q, k, v = normal_qkv(1, w.heads, w.N, w.d, seed=0, dtype=torch.float32)
    qb, kb, vb = (x.to(torch.bfloat16) for x in (q, k, v))
    scale = 1 / math.sqrt(w.d)
    o, lse = run_attention(dev, geom, mask, qb, kb, vb, w.kinds, w.bq, w.bkv, mode, want_lse=True)
    for h, kind in enumerate(w.kinds):
        src = (q, k, v) if src_dtype == "fp32" else (qb, kb, vb)
        ref, ref_lse = oracle_head(geom, mask, src[0][0, h], src[1][0, h], src[2][0, h], kind, mode, w.bq, w.bkv,
                                   scale)
        assert_close(o[0, h].float().numpy(), ref, f"head {h}")
        if src_dtype == "bf16":
            assert np.abs(lse[0, h].numpy() - ref_lse).max() < 1e-3


@pytest.mark.parametrize("tiles", [(128, 128), (256, 128), (64, 64), (128, 64), (32, 32), (512, 128), (256, 256),
                                   (256, 96), (512, 32)])
@pytest.mark.parametrize("mode", [0, 2, 3])
def test_attention_small(dev, tiles, mode):
    w = SMALL
    bq, bkv = tiles
    geom = (w.F, w.H, w.W)
    mask = (w.sink_frames, w.spatial_band, w.temporal_band, w.temporal_layout)
    say(f"attention small tiles={tiles} mode={mode}")
    q, k, v = normal_qkv(1, w.heads, w.N, w.d, seed=1)
    scale = 1 / math.sqrt(w.d)
    o, _ = run_attention(dev, geom, mask, q, k, v, w.kinds, bq, bkv, mode)
    rows = np.sort(np.random.default_rng(0).choice(w.N, 384, replace=False))
    rows = np.unique(np.concatenate([rows, np.arange(128), np.arange(w.N - 128, w.N)]))
    for h, kind in enumerate(w.kinds):
        ref, _ = oracle_head(geom, mask, q[0, h], k[0, h], v[0, h], kind, mode, bq, bkv, scale, rows=rows)
        assert_close(o[0, h, rows].float().numpy(), ref, f"head {h}")


@pytest.mark.parametrize("level", [0, 1, 2])
def test_schedule_levels_small(dev, level):
    """Each level of a three-level sparsity schedule (masks from svga_mask_for_kept_fraction) at Small, 128x128."""
    w = SMALL
    geom = (w.F, w.H, w.W)
    sched = B.SparsitySchedule(geom, [(0, 0.7, 0.6), (10, 0.5, 0.4), (20, 0.3, 0.2)], sink_frames=w.sink_frames,
                               temporal_layout=w.temporal_layout)
    p = sched.plan(10 * level, 1)
    mask = (p.mask.sink_frames, p.mask.spatial_band, p.mask.temporal_band, p.mask.temporal_layout)
    say(f"schedule level {level}: mask {mask}, kept pairs {p.kept_pairs} of {w.N ** 2}")
    q, k, v = normal_qkv(1, w.heads, w.N, w.d, seed=11 + level)
    o, _ = run_attention(dev, geom, mask, q, k, v, w.kinds, 128, 128, p.mode)
    rows = np.sort(np.random.default_rng(level).choice(w.N, 256, replace=False))
    rows = np.unique(np.concatenate([rows, np.arange(64), np.arange(w.N - 64, w.N)]))
    for h, kind in enumerate(w.kinds):
        ref, _ = oracle_head(geom, mask, q[0, h], k[0, h], v[0, h], kind, p.mode, 128, 128, 1 / math.sqrt(w.d),
                             rows=rows)
        assert_close(o[0, h, rows].float().numpy(), ref, f"head {h}")


@pytest.mark.parametrize("tiles,mode,gather", [((256, 128), 2, False), ((256, 128), 3, True), ((512, 128), 2, False),
                                               ((128, 64), 0, False), ((32, 32), 1, False), ((256, 96), 2, True)])
def test_persistent_equals_plain_bitwise(dev, tiles, mode, gather):
    """Persistent workgroups (the workspace entry point) give the same output and LSE bits as one workgroup
    per query tile; the workspace is reused (with garbage in it) by a second, smaller call."""
    w = SMALL
    geom = (w.F, w.H, w.W)
    mask = (w.sink_frames, w.spatial_band, w.temporal_band, w.temporal_layout)
    bq, bkv = tiles
    say(f"persistent tiles={tiles} mode={mode} gather={gather}")
    q, k, v = (x.to(dev) for x in normal_qkv(2, w.heads, w.N, w.d, seed=4))
    flags = torch.tensor([list(w.kinds)] * 2, dtype=torch.uint8, device=dev)
    tm = B.svga_build_tilemap(geom, mask, bq, bkv, mode, device=dev)
    ws = torch.full((B.svga_attn_workspace_bytes(),), 0x5A, dtype=torch.uint8, device=dev)
    for batch in (2, 1):
        qb, kb, vb, fb = q[:batch], k[:batch], v[:batch], flags[:batch]
        a, la = B.svga_sparse_attn_fwd(qb, kb, vb, fb, tm, geom, mask, bq, bkv, mode, gather_temporal=gather,
                                       want_lse=True)
        b, lb = B.svga_sparse_attn_fwd(qb, kb, vb, fb, tm, geom, mask, bq, bkv, mode, gather_temporal=gather,
                                       want_lse=True, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))
        assert torch.equal(la.view(torch.int32), lb.view(torch.int32))


@pytest.mark.parametrize("wname,tiles,mode,gather", [
    ("small", (256, 128), 2, False), ("small", (256, 128), 3, True), ("small", (512, 128), 2, False),
    ("small", (128, 64), 0, False), ("small", (256, 512), 2, False), ("small", (256, 96), 1, True),
    ("tiny", (32, 32), 2, False), ("tiny", (64, 32), 1, True),
    ("small64", (256, 128), 2, False), ("small64", (512, 64), 3, True)])
def test_split_tail(dev, wname, tiles, mode, gather):
    """Persistent launch with the split-tail workspace: at bq 256 / 512 every work item here is among
    the last ones, so each runs as 4 pieces merged through their log-sum-exp (pieces with no key tile
    included at 512-key tiles); smaller bq do not split and must give the unsplit bits. Against the
    oracle on every row of two heads, and against the unsplit launch on every row (output to bf16
    rounding, LSE to fp32 rounding); the workspace starts as garbage and is reused by a second,
    smaller call."""
    w = {"small": SMALL, "tiny": TINY, "small64": dataclasses.replace(SMALL, d=64)}[wname]
    geom = (w.F, w.H, w.W)
    mask = (w.sink_frames, w.spatial_band, w.temporal_band, w.temporal_layout)
    bq, bkv = tiles
    say(f"split tail {wname} tiles={tiles} mode={mode} gather={gather}")
    qc, kc, vc = normal_qkv(2, w.heads, w.N, w.d, seed=6)
    q, k, v = qc.to(dev), kc.to(dev), vc.to(dev)
    flags = torch.tensor([list(w.kinds)] * 2, dtype=torch.uint8, device=dev)
    tm = B.svga_build_tilemap(geom, mask, bq, bkv, mode, device=dev)
    ws = torch.full((B.svga_attn_split_workspace_bytes(w.d, bq),), 0x5A, dtype=torch.uint8, device=dev)
    scale = 1 / math.sqrt(w.d)
    for batch in (2, 1):
        fb = flags[:batch]
        if gather:
            qb, kb, vb = q[:batch], k[:batch], v[:batch]
        else:
            qb, kb, vb = (B.svga_permute(x[:batch].contiguous(), fb, geom, mask) for x in (q, k, v))
        a, la = B.svga_sparse_attn_fwd(qb, kb, vb, fb, tm, geom, mask, bq, bkv, mode, gather_temporal=gather,
                                       want_lse=True)
        b, lb = B.svga_sparse_attn_fwd(qb, kb, vb, fb, tm, geom, mask, bq, bkv, mode, gather_temporal=gather,
                                       want_lse=True, workspace=ws)
        if not gather:
            b = B.svga_unpermute(b, fb, geom, mask)
            a = B.svga_unpermute(a, fb, geom, mask)
        torch.cuda.synchronize()
        d = (a.float() - b.float()).abs()
        say(f"  batch {batch}: split vs unsplit max-abs {d.max().item():.3e} mean-abs {d.mean().item():.3e}")
        if bq < 256:
            assert torch.equal(a.view(torch.int16), b.view(torch.int16)) and torch.equal(la, lb)
        assert torch.isfinite(b.float()).all()
        assert d.max().item() < 1e-2 and d.mean().item() < 5e-4
        fin = torch.isfinite(la)
        assert torch.equal(fin, torch.isfinite(lb))
        assert (la[fin] - lb[fin]).abs().max().item() < 1e-4
        bc = b.cpu()
        for h in (0, w.heads - 1):
            ref, _ = oracle_head(geom, mask, qc[batch - 1, h], kc[batch - 1, h], vc[batch - 1, h], w.kinds[h], mode,
                                 bq, bkv, scale)
            assert_close(bc[batch - 1, h].float().numpy(), ref, f"head {h}")


def test_split_tail_workspace_reuse(dev):
    """One split-tail workspace reused by a run of calls of different shapes, tile sizes and modes
    (each leaves its pieces behind for the next): every call matches the unsplit launch, and a
    repeated call reproduces its bits."""
    w = SMALL
    geom = (w.F, w.H, w.W)
    mask = (w.sink_frames, w.spatial_band, w.temporal_band, w.temporal_layout)
    qc, kc, vc = normal_qkv(2, w.heads, w.N, w.d, seed=8)
    q, k, v = qc.to(dev), kc.to(dev), vc.to(dev)
    flags = torch.tensor([list(w.kinds)] * 2, dtype=torch.uint8, device=dev)
    ws = torch.full((B.svga_attn_split_workspace_bytes(w.d, 512),), 0x3C, dtype=torch.uint8, device=dev)
    maps = {c: B.svga_build_tilemap(geom, mask, c[0], c[1], c[2], device=dev)
            for c in ((256, 128, "exact"), (512, 128, "dense"), (256, 64, "rounded"))}
    first = {}
    for rnd in range(4):
        for (bq, bkv, mode), tm in maps.items():
            batch = 2 if (rnd + bq) % 2 == 0 else 1
            args = (q[:batch], k[:batch], v[:batch], flags[:batch], tm, geom, mask, bq, bkv, mode)
            a, la = B.svga_sparse_attn_fwd(*args, want_lse=True)
            b, lb = B.svga_sparse_attn_fwd(*args, want_lse=True, workspace=ws)
            torch.cuda.synchronize()
            assert (a.float() - b.float()).abs().max().item() < 1e-2
            fin = torch.isfinite(la)
            assert torch.equal(fin, torch.isfinite(lb)) and (la[fin] - lb[fin]).abs().max().item() < 1e-4
            key = (bq, bkv, mode, batch)
            if key in first:
                assert torch.equal(first[key].view(torch.int16), b.view(torch.int16))
            else:
                first[key] = b.clone()
    say(f"split-tail workspace reuse: {len(first)} distinct calls, repeated calls bit-identical")


def test_binding_rejects_bad_buffers(dev):
    """The binding refuses host tensors, short buffers and mismatched shapes before anything is
    launched (a host pointer or a short buffer handed to a kernel would be read out of bounds)."""
    w = TINY
    geom = (w.F, w.H, w.W)
    mask = (w.sink_frames, w.spatial_band, w.temporal_band, w.temporal_layout)
    q = torch.zeros(1, 2, w.N, w.d, dtype=torch.bfloat16, device=dev)
    flags = torch.zeros(1, 2, dtype=torch.uint8, device=dev)
    tm = B.svga_build_tilemap(geom, mask, 32, 32, "exact", device=dev)
    attn = lambda **kw: B.svga_sparse_attn_fwd(kw.pop("q", q), kw.pop("k", q), q, kw.pop("flags", flags),
                                               kw.pop("tm", tm), geom, mask, 32, 32, "exact", **kw)
    bad = [dict(k=q[:, :, :96].contiguous()), dict(k=q.cpu()), dict(flags=flags.cpu()), dict(flags=flags[:, :1]),
           dict(tm=tm.cpu()), dict(tm=tm.to(torch.int32)), dict(workspace=torch.empty(256, dtype=torch.uint8)),
           dict(lse=torch.empty(1, dtype=torch.float32, device=dev)), dict(out=q[:, :1].contiguous())]
    for kw in bad:
        with pytest.raises(ValueError):
            attn(**kw)
    with pytest.raises(ValueError):
        B.svga_permute(q, flags[:, :1].contiguous(), geom, mask)
    with pytest.raises(ValueError):
        B.svga_route_heads(q, q, q, geom, mask, torch.arange(4, dtype=torch.int32))
    with pytest.raises(ValueError):
        B.svga_route_heads(q, q, q, geom, mask, torch.arange(4, dtype=torch.int64, device=dev))
    with pytest.raises(ValueError):
        B.svga_build_tilemap(geom, mask, 32, 32, "exact", out=torch.empty(tm.numel(), dtype=torch.uint8))
    o, _ = attn()   # the same call with good buffers runs
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all()


def test_gather_equals_permute_path_bitwise(dev):
    """In-kernel gather of temporal rows gives the same bits, output and LSE, as permute -> attention ->
    unpermute; also in the persistent launch with the split tail."""
    w = SMALL
    geom = (w.F, w.H, w.W)
    for lay in (0, 1):
        mask = (w.sink_frames, w.spatial_band, w.temporal_band, lay)
        q, k, v = normal_qkv(2, w.heads, w.N, w.d, seed=2)
        for bq, bkv, mode, split in ((128, 128, 2, False), (256, 128, 3, True), (64, 64, 1, False),
                                     (512, 64, 2, True), (256, 96, 2, False)):
            ws = torch.zeros(B.svga_attn_split_workspace_bytes(w.d, bq), dtype=torch.uint8, device=dev) \
                if split else None
            say(f"gather layout={lay} tiles={bq}x{bkv} mode={mode} split={split}")
            a, la = run_attention(dev, geom, mask, q, k, v, w.kinds, bq, bkv, mode, gather=False, want_lse=True,
                                  workspace=ws)
            b, lb = run_attention(dev, geom, mask, q, k, v, w.kinds, bq, bkv, mode, gather=True, want_lse=True,
                                  workspace=ws)
            assert np.array_equal(i16(a), i16(b))
            assert np.array_equal(la.numpy(), lb.numpy())


def test_naive_and_exact_agree(dev):
    """B1 and B2 keep the same pairs. B2 visits full tiles before boundary tiles, B1 in plain key
    order, so the two agree to rounding; where a head has no boundary tile the visiting order is
    the same and they agree bit for bit."""
    w = SMALL
    geom = (w.F, w.H, w.W)
    mask = (w.sink_frames, w.spatial_band, w.temporal_band, w.temporal_layout)
    q, k, v = normal_qkv(1, w.heads, w.N, w.d, seed=3)
    for bq, bkv in ((128, 128), (256, 128)):
        say(f"naive vs exact tiles={bq}x{bkv}")
        a, _ = run_attention(dev, geom, mask, q, k, v, w.kinds, bq, bkv, B.MAP_NAIVE)
        b, _ = run_attention(dev, geom, mask, q, k, v, w.kinds, bq, bkv, B.MAP_EXACT)
        ex = B.tilemap_views(B.svga_build_tilemap_host(geom, mask, bq, bkv, B.MAP_EXACT), geom, bq, bkv)
        for h, kind in enumerate(w.kinds):
            diff = np.abs(a[0, h].float().numpy() - b[0, h].float().numpy())
            assert diff.max() < 4e-3
            if ex["n_bnd"][kind].sum() == 0:
                assert np.array_equal(i16(a[0, h]), i16(b[0, h]))


def key_tile_classes(w, mask, kinds, bkv):
    """[heads, N]: the key tile of each frame-major key in its head's executed order."""
    out = np.empty((len(kinds), w.N), dtype=np.int64)
    for h, kind in enumerate(kinds):
        out[h] = O.positions(O.executed_order(w.F, w.H, w.W, kind, mask[0], mask[3])) // bkv
    return out


@pytest.mark.parametrize("tiles,split", [((128, 128), False), ((256, 128), True), ((512, 64), True)])
@pytest.mark.parametrize("form", ["tile", "residue"])
@pytest.mark.parametrize("mode", [1, 2, 3])
def test_census_counts_every_kept_key(dev, mode, form, tiles, split):
    """Q = K = 0: uniform weights over each row's kept keys, so the output is an exact rational.
    form "tile": V[k, c] = [kv_tile(k) mod d == c] with kv_tile the key's tile in the executed
    order; here every one of the 27 (or 54) key tiles has a column of its own (d = 128), so a
    dropped or doubled key tile moves its column from its share to 0 or to twice its share.
    form "residue": V[k, c] = [k mod d == c] (catches single keys misplaced inside a tile on
    temporal heads). LSE must equal ln(kept keys): one 64-key tile more or less moves it by at
    least 64/3456, against a bar of 1e-4. Every row of all four heads, in the plain launch and in
    the persistent launch with the split tail (every work item split at 3,456 tokens)."""
    w = SMALL
    bq, bkv = tiles
    geom = (w.F, w.H, w.W)
    mask = (w.sink_frames, w.spatial_band, w.temporal_band, w.temporal_layout)
    say(f"census small mode={mode} form={form} tiles={tiles} split={split}")
    cls = key_tile_classes(w, mask, w.kinds, bkv) if form == "tile" else None
    q, k, v = census_qkv(1, w.heads, w.N, w.d, key_class=cls)
    ws = torch.zeros(B.svga_attn_split_workspace_bytes(w.d, bq), dtype=torch.uint8, device=dev) if split else None
    o, lse = run_attention(dev, geom, mask, q, k, v, w.kinds, bq, bkv, mode, want_lse=True, workspace=ws)
    rows = np.arange(w.N)
    for h, kind in enumerate(w.kinds):
        ref, ref_lse = oracle_head(geom, mask, q[0, h], k[0, h], v[0, h], kind, mode, bq, bkv, 0.1, rows=rows)
        got = o[0, h].float().numpy()
        rel = np.abs(got - ref) / np.maximum(np.abs(ref), 1e-30)
        lerr = np.abs(lse[0, h].numpy() - ref_lse)
        say(f"  head {h}: max rel {rel[ref > 0].max():.3e}, LSE max err {lerr.max():.3e}")
        assert (got[ref == 0] == 0).all()
        assert rel[ref > 0].max() < 2 ** -7
        assert lerr.max() < 1e-4


@pytest.mark.parametrize("geom,mask,tiles,kinds", [
    ((3, 5, 7), (1, 1, 3, 0), (64, 64), (0, 1)),         # ragged: 105 tokens, tiles past the end
    ((3, 5, 7), (0, 0, 0, 0), (32, 32), (0, 1)),         # no sink, zero bands: each row keeps its own frame/position
    ((2, 3, 3), (1, 5, 20, 0), (128, 128), (1, 0)),      # one tile larger than the sequence
    ((6, 4, 4), (2, 1, 3, 1), (64, 32), (1, 1, 0)),      # literal order with two sink frames
    ((5, 7, 3), (5, 0, 1, 0), (32, 64), (1, 0)),         # every frame a sink frame
])
@pytest.mark.parametrize("mode", [0, 1, 2, 3])
def test_attention_edge_cases(dev, geom, mask, tiles, kinds, mode):
    F, H, W = geom
    N = F * H * W
    bq, bkv = tiles
    say(f"edge geom={geom} mask={mask} tiles={tiles} kinds={kinds} mode={mode}")
    q, k, v = normal_qkv(2, len(kinds), N, 128, seed=5)
    q = q * 3
    for gather in (False, True):
        o, lse = run_attention(dev, geom, mask, q, k, v, kinds, bq, bkv, mode, gather=gather, want_lse=not gather)
        for b in range(2):
            for h, kind in enumerate(kinds):
                ref, ref_lse = oracle_head(geom, mask, q[b, h], k[b, h], v[b, h], kind, mode, bq, bkv,
                                           1 / math.sqrt(128))
                assert_close(o[b, h].float().numpy(), ref, f"b{b} h{h} gather={gather}")
                if lse is not None:
                    fin = np.isfinite(ref_lse)
                    assert np.array_equal(np.isfinite(lse[b, h].numpy()), fin)
                    if fin.any():
                        assert np.abs(lse[b, h].numpy()[fin] - ref_lse[fin]).max() < 1e-3


# ---------------------------------------------------------------- routing

def check_routing(dev, geom, mask, q, k, v, idx, tol=1e-3):
    F, H, W = geom
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    flags, err = B.svga_route_heads(qd, kd, vd, geom, mask, torch.as_tensor(idx, dtype=torch.int32).to(dev))
    torch.cuda.synchronize()
    scale = 1 / math.sqrt(q.shape[-1])
    f_ref, e_ref = O.route_heads(q.double().numpy(), k.double().numpy(), v.double().numpy(), F, H, W, mask[0],
                                 mask[1], mask[2], np.asarray(idx), scale)
    e = err.cpu().numpy()
    f = flags.cpu().numpy()
    say(f"  err gpu {e.reshape(-1, 2)[:4].tolist()} oracle {e_ref.reshape(-1, 2)[:4].tolist()}")
    big = np.maximum(e_ref.max(axis=-1, keepdims=True), 1e-30)
    say(f"  max relative error {(np.abs(e - e_ref) / big).max():.3e} (bar {tol:g})")
    assert (np.abs(e - e_ref) <= tol * big).all()
    decided = np.abs(e_ref[..., 1] - e_ref[..., 0]) > tol * big[..., 0]
    assert np.array_equal(f[decided], f_ref[decided])
    return f, f_ref


@pytest.mark.parametrize("n", [1, 7, 32, 33, 64])
def test_routing_tiny(dev, n):
    w = TINY
    geom = (w.F, w.H, w.W)
    mask = (w.sink_frames, w.spatial_band, w.temporal_band, w.temporal_layout)
    say(f"routing tiny n_samples={n}")
    q, k, v = normal_qkv(2, 3, w.N, w.d, seed=4)
    idx = sample_indices(w.N, n, seed=n).numpy()
    check_routing(dev, geom, mask, q * 2, k, v, idx)


def test_routing_finds_planted_kinds(dev):
    w = SMALL
    geom = (w.F, w.H, w.W)
    mask = (w.sink_frames, w.spatial_band, w.temporal_band, w.temporal_layout)
    kinds = (0, 1, 1, 0, 1, 0)
    say("routing planted small")
    q, k, v = planted_qkv(1, w.F, w.H, w.W, w.d, kinds, seed=7)
    idx = sample_indices(w.N, 64, seed=0).numpy()
    f, f_ref = check_routing(dev, geom, mask, q, k, v, idx)
    assert tuple(f[0]) == kinds and tuple(f_ref[0]) == kinds


@pytest.mark.parametrize("geom,d,mask", [
    ((8, 7, 11), 64, (1, 1, 9, 0)),    # S = 77: frame boundaries inside 32-key steps; the last half ends past N
    ((8, 7, 11), 128, (2, 2, 30, 0)),
    ((6, 8, 12), 128, (1, 1, 20, 0)),  # S = 96: a frame boundary on a step's first key
    ((6, 8, 12), 64, (0, 0, 5, 0)),
])
def test_routing_frame_boundaries_inside_key_halves(dev, geom, d, mask):
    """Key halves of 64 keys that reach into a second frame: the kernel sums
    the dense output per frame and forms the spatial one from the frames a
    sample keeps, so a boundary inside a step, on a step's first key and at
    the end of the sequence must all match the oracle."""
    F, H, W = geom
    N = F * H * W
    say(f"routing frame boundaries geom={geom} d={d} mask={mask}")
    for n, seed in ((64, 11), (5, 12)):
        q, k, v = normal_qkv(1, 2, N, d, seed=seed)
        idx = sample_indices(N, n, seed=seed).numpy()
        check_routing(dev, geom, mask, q * 3, k, v, idx)


def test_routing_head_dim_128_ragged_chunks(dev):
    geom = (5, 7, 9)          # 315 tokens: chunks end mid-tile
    mask = (1, 1, 4, 0)
    say("routing d128 ragged")
    q, k, v = normal_qkv(1, 2, 315, 128, seed=6)
    idx = sample_indices(315, 40, seed=1).numpy()
    check_routing(dev, geom, mask, q * 3, k, v, idx)
