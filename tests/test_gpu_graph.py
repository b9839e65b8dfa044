"""The benchmark step (routing, tile map, permutations, attention in the split-tail launch,
unpermutation) captured as one HIP graph: every replay, with eager work and synchronisation
between replays, equals the eager step bit for bit."""
import pytest
import torch

import block_sparse_spatio_amd as B
from synth import SMALL, planted_qkv, sample_indices

pytestmark = pytest.mark.gpu


def test_step_graph_replays_equal_eager():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dev = torch.device("cuda:0")
    w = SMALL
    geom = (w.F, w.H, w.W)
    mask = (w.sink_frames, w.spatial_band, w.temporal_band, w.temporal_layout)
    q, k, v = planted_qkv(1, w.F, w.H, w.W, w.d, w.kinds, seed=2)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    idx = sample_indices(w.N, w.n_samples, seed=2).to(dev)
    ws = torch.empty(B.svga_route_workspace_bytes(1, w.heads, geom, w.d, w.n_samples), dtype=torch.uint8, device=dev)
    flags = torch.empty(1, w.heads, dtype=torch.uint8, device=dev)
    err = torch.empty(1, w.heads, 2, dtype=torch.float32, device=dev)
    tmap = torch.empty(B.svga_tilemap_layout(geom, w.bq, w.bkv).total, dtype=torch.uint8, device=dev)
    qp, kp, vp, op, o = (torch.empty_like(qd) for _ in range(5))
    aws = torch.empty(B.svga_attn_split_workspace_bytes(w.d, w.bq), dtype=torch.uint8, device=dev)

    def step():
        B.svga_route_heads(qd, kd, vd, geom, mask, idx, workspace=ws, flags_out=flags, err_out=err)
        B.svga_build_tilemap(geom, mask, w.bq, w.bkv, B.MAP_EXACT, out=tmap)
        B.svga_permute(qd, flags, geom, mask, out=qp)
        B.svga_permute(kd, flags, geom, mask, out=kp)
        B.svga_permute(vd, flags, geom, mask, out=vp)
        B.svga_sparse_attn_fwd(qp, kp, vp, flags, tmap, geom, mask, w.bq, w.bkv, B.MAP_EXACT, out=op, workspace=aws)
        B.svga_unpermute(op, flags, geom, mask, out=o)

    step()
    torch.cuda.synchronize()
    ref = (o.clone(), flags.clone(), err.clone())
    assert tuple(ref[1][0].tolist()) == w.kinds
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    other = torch.empty_like(qd)
    for r in range(4):
        # eager work on the same buffers' neighbours between replays, then the replay
        o.zero_()
        flags.fill_(7)
        B.svga_permute(kd, ref[1], geom, mask, out=other)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(o.view(torch.int16), ref[0].view(torch.int16)), f"replay {r}: output differs"
        assert torch.equal(flags, ref[1]), f"replay {r}: flags differ"
        assert torch.equal(err, ref[2]), f"replay {r}: routing errors differ"
