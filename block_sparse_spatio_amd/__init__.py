"""Block-sparse spatio-temporal attention for AMD Instinct MI355X (gfx950).

The library is ``libsvga.so`` (C ABI in include/svga.h, HIP kernels in csrc/);
``svga`` is its thin Python binding. Build with
``python -m block_sparse_spatio_amd.build``.
"""
from .svga import (  # noqa: F401
    SvgaError, make_geom, make_mask, tilemap_views, svga_mask_for_kept_fraction,
    svga_version, svga_tilemap_layout, svga_build_tilemap_host, svga_build_tilemap,
    svga_permute, svga_unpermute, svga_route_workspace_bytes, svga_route_heads, svga_sparse_attn_fwd,
    svga_attn_workspace_bytes, svga_attn_split_workspace_bytes,
    KIND_SPATIAL, KIND_TEMPORAL, TL_SINK_FIRST, TL_LITERAL,
    MAP_DENSE, MAP_NAIVE, MAP_EXACT, MAP_ROUNDED, MODES, TILE_SKIP, TILE_FULL, TILE_BOUNDARY,
    SVGA_OK, SVGA_EINVAL, SVGA_EUNSUPPORTED, SVGA_ECAPACITY, SVGA_EHIP,
)
from .schedule import SparsitySchedule, ScheduleLevel  # noqa: F401,E402
