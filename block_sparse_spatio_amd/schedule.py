"""Sparsity schedules: a host policy from (denoising step, layer) to the mask of that attention call.

ASTA section "End-to-end results and takeaways" (Table 3) compares schedules that keep progressively
fewer attention pairs. Here a schedule is a list of levels, each in force from its first denoising step
on and giving the kept fraction wanted of spatial and of temporal heads; steps before the first level
and the layers named dense run the dense traversal. Targets become band widths only through the
library's svga_mask_for_kept_fraction; this module holds no mask arithmetic of its own.
"""
from dataclasses import dataclass

from .svga import MAP_DENSE, MAP_EXACT, TL_SINK_FIRST, _geom, svga_mask_for_kept_fraction


@dataclass(frozen=True)
class ScheduleLevel:
    first_step: int      # in force from this denoising step until the next level's
    spatial: float       # kept fraction wanted of each spatial head, in [0, 1]
    temporal: float      # kept fraction wanted of each temporal head, in [0, 1]


@dataclass(frozen=True)
class StepPlan:
    mask: object         # SvgaMask for the tile map, routing and permutation calls
    mode: int            # SVGA_MAP_* traversal for this call
    kept_pairs: tuple    # kept pairs of one (spatial, temporal) head under `mask`


class SparsitySchedule:
    """Maps (step, layer) to a StepPlan. Masks are computed once per level and reused."""

    def __init__(self, geom, levels, sink_frames=1, temporal_layout=TL_SINK_FIRST, dense_layers=(),
                 sparse_mode=MAP_EXACT):
        levels = [lv if isinstance(lv, ScheduleLevel) else ScheduleLevel(*lv) for lv in levels]
        if any(lv.first_step < 0 for lv in levels):
            raise ValueError("first_step must be >= 0")
        if any(b.first_step <= a.first_step for a, b in zip(levels, levels[1:])):
            raise ValueError("levels must have strictly increasing first_step")
        self.geom = _geom(geom)
        self.levels = levels
        self.dense_layers = frozenset(int(x) for x in dense_layers)
        self.sparse_mode = int(sparse_mode)
        # every level's mask up front, so that a bad target fails here and not mid-run
        self._plans = [self._plan(lv.spatial, lv.temporal, self.sparse_mode, sink_frames, temporal_layout)
                       for lv in levels]
        self._dense = self._plan(1.0, 1.0, MAP_DENSE, sink_frames, temporal_layout)

    def _plan(self, ts, tt, mode, sink_frames, temporal_layout):
        mask, kept = svga_mask_for_kept_fraction(self.geom, sink_frames, ts, tt, temporal_layout)
        return StepPlan(mask, mode, kept)

    def level_index(self, step):
        """Index of the level in force at `step`, or -1 before the first level."""
        idx = -1
        for i, lv in enumerate(self.levels):
            if step >= lv.first_step:
                idx = i
        return idx

    def plan(self, step, layer):
        if step < 0:
            raise ValueError("step must be >= 0")
        i = self.level_index(step)
        if i < 0 or layer in self.dense_layers:
            return self._dense
        return self._plans[i]
