"""Oracle: a plain, slow CPU reference of block-sparse spatio-temporal attention.

THIS PACKAGE IS TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import it. The library in
``block_sparse_spatio_amd`` never imports it, and it never imports the library:
the two share no code. Every step here is written out from its definition,
in float64 numpy (integer work in int64), with no blocking or fusion beyond
what the definition states.

Source cited throughout as ASTA: "Accelerating Spatio-Temporal Attention for
Video Diffusion on TPUs" (Google Developers Blog). Sections are named by their
headings; figures by number.

Modules
-------
geometry  token coordinates, frame-major and temporal-major orders, permute/unpermute
masks     spatial-head and temporal-head keep rules in original coordinates
tilemap   brute-force tile classification (full / boundary / skip), balanced rounding
attention masked softmax attention and its log-sum-exp
routing   sampled-query spatial/temporal head routing

Pinning: every function is checked by ``tests/test_oracle.py`` against closed
forms, hand-derived fixtures under ``tests/golden/`` and library routines (see
each function's docstring for the pin). Nothing here is "parity unpinned".
"""
from .geometry import (coords, executed_order, positions, permute, unpermute,
                       KIND_SPATIAL, KIND_TEMPORAL, LAYOUT_SINK_FIRST, LAYOUT_LITERAL)
from .masks import keep_block, head_keep_block
from .tilemap import (classify, tile_counts, rounded_keep_block, MODE_DENSE, MODE_NAIVE,
                      MODE_EXACT, MODE_ROUNDED, SKIP, FULL, BOUNDARY)
from .attention import masked_attention, mode_keep_block, attention_head
from .routing import route_heads

__all__ = [
    "coords", "executed_order", "positions", "permute", "unpermute",
    "KIND_SPATIAL", "KIND_TEMPORAL", "LAYOUT_SINK_FIRST", "LAYOUT_LITERAL",
    "keep_block", "head_keep_block",
    "classify", "tile_counts", "rounded_keep_block", "MODE_DENSE", "MODE_NAIVE",
    "MODE_EXACT", "MODE_ROUNDED", "SKIP", "FULL", "BOUNDARY",
    "masked_attention", "mode_keep_block", "attention_head", "route_heads",
]
