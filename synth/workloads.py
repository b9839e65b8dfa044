"""Named workloads: video-latent geometry, heads, head dim, mask parameters, tiles.

Sizes follow the single-device measurement setting of "Accelerating
Spatio-Temporal Attention for Video Diffusion on TPUs" (section "Implementing
sparse attention on TPUs": 75.6K tokens, 10 heads, head dim 128, about 38.87%
of pairs kept) and its 1440p end-to-end setting (302K tokens). The page gives
no F x H x W factorisation and no band widths; the values below are chosen so
that F*H*W and the kept fraction match the page.
"""
from dataclasses import dataclass, field


@dataclass(frozen=True)
class Workload:
    name: str
    F: int
    H: int
    W: int
    kinds: tuple            # per head: 0 spatial, 1 temporal (fixed routing flags)
    d: int
    sink_frames: int
    spatial_band: int       # frames
    temporal_band: int      # flattened spatial positions
    temporal_layout: int    # 0 sink-first, 1 literal
    bq: int
    bkv: int
    batch: int = 1
    n_samples: int = 64     # sampled queries for routing

    @property
    def S(self):
        return self.H * self.W

    @property
    def N(self):
        return self.F * self.H * self.W

    @property
    def heads(self):
        return len(self.kinds)


# 4 x 4 x 8 = 128 tokens, head 0 spatial (band 1 frame), head 1 temporal (window 2), d = 64.
TINY = Workload("tiny", 4, 4, 8, (0, 1), 64, 1, 1, 2, 0, 32, 32)
# 9 x 16 x 24 = 3456 tokens, 2 spatial (band 1) + 2 temporal (window 24) heads, d = 128.
SMALL = Workload("small", 9, 16, 24, (0, 0, 1, 1), 128, 1, 1, 24, 0, 128, 128)
# 21 x 45 x 80 = 75,600 tokens, 5 spatial (band 4) + 5 temporal (window 644) heads: 38.88% kept.
HEADLINE = Workload("headline", 21, 45, 80, (0,) * 5 + (1,) * 5, 128, 1, 4, 644, 0, 256, 128)
# Same shape, run with balanced tile rounding (B3).
HEADLINE_B3 = Workload("headline_b3", 21, 45, 80, (0,) * 5 + (1,) * 5, 128, 1, 4, 644, 0, 128, 128)
# 21 x 90 x 160 = 302,400 tokens, 10 heads routed on 64 sampled queries (band 2 / window 2054).
P1440 = Workload("1440p", 21, 90, 160, (0,) * 5 + (1,) * 5, 128, 1, 2, 2054, 0, 256, 128)

WORKLOADS = {w.name: w for w in (TINY, SMALL, HEADLINE, HEADLINE_B3, P1440)}
