"""The entry point that allocates nothing (svga_sparse_attn_fwd_noalloc) against the workspace entry
point it mirrors (svga_sparse_attn_fwd_ws with a split-tail workspace): same kernels, so the same
output and LSE bits, on two calls in a row, the second with a smaller input, and once more after a
call of another shape has left its state in the library's scratch."""
import math

import numpy as np
import pytest
import torch

import block_sparse_spatio_amd as B
import oracle as O
from synth import SMALL, normal_qkv

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def say(*a):
    print(*a, flush=True)


def test_noalloc_matches_workspace_entry_point(dev):
    w = SMALL
    geom = (w.F, w.H, w.W)
    mask = (w.sink_frames, w.spatial_band, w.temporal_band, w.temporal_layout)
    qc, kc, vc = normal_qkv(2, w.heads, w.N, w.d, seed=11)
    q, k, v = qc.to(dev), kc.to(dev), vc.to(dev)
    flags = torch.tensor([list(w.kinds)] * 2, dtype=torch.uint8, device=dev)
    # (batch, bq, bkv, mode): the second call is smaller than the first; the last two change shape
    calls = [(2, 256, 128, "exact"), (1, 256, 128, "exact"), (2, 512, 64, "rounded"), (1, 128, 128, "dense")]
    for batch, bq, bkv, mode in calls:
        say(f"noalloc batch={batch} tiles={bq}x{bkv} mode={mode}")
        tm = B.svga_build_tilemap(geom, mask, bq, bkv, mode, device=dev)
        ws = torch.full((B.svga_attn_split_workspace_bytes(w.d, bq),), 0x5A, dtype=torch.uint8, device=dev)
        args = (q[:batch].contiguous(), k[:batch].contiguous(), v[:batch].contiguous(), flags[:batch].contiguous(),
                tm, geom, mask, bq, bkv, mode)
        a, la = B.svga_sparse_attn_fwd(*args, want_lse=True, workspace=ws)
        b, lb = B.svga_sparse_attn_fwd(*args, want_lse=True, noalloc=True)
        torch.cuda.synchronize()
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))
        assert torch.equal(la.view(torch.int32), lb.view(torch.int32))
        # and the oracle's bar on one head of the permuted-order input (spatial head 0: order unchanged)
        ref, _ = O.attention_head(qc[batch - 1, 0].double().numpy(), kc[batch - 1, 0].double().numpy(),
                                  vc[batch - 1, 0].double().numpy(), 0, w.F, w.H, w.W, *mask[:3], mask[3],
                                  B.MODES[mode], bq, bkv, 1 / math.sqrt(w.d),
                                  cls_rounded=(O.classify(w.F, w.H, w.W, 0, *mask[:3], mask[3], bq, bkv,
                                                          O.MODE_ROUNDED)["cls"] if mode == "rounded" else None))
        err = np.abs(b[batch - 1, 0].float().cpu().numpy() - ref)
        say(f"  bit-identical to the workspace call; head 0 vs oracle max-abs {err.max():.3e}")
        assert err.max() < 2e-2 and err.mean() < 2e-3
