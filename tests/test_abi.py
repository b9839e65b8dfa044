"""The C ABI library loads, exports every declared entry point, and rejects bad
arguments on the host with the documented status codes (no GPU needed: no
check below reaches a kernel launch)."""
import ctypes
import os
import re

import pytest

from block_sparse_spatio_amd import _lib
from block_sparse_spatio_amd._lib import SvgaGeom, SvgaMask, SvgaTilemapOffsets

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "svga.h")
FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: every call below fails validation first


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(svga_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    L = _lib.lib()
    names = declared_functions()
    assert len(names) == len(_lib.SIGNATURES) == 16
    assert set(names) == set(_lib.SIGNATURES)
    for n in names:
        assert hasattr(L, n), n


def test_version_and_status_strings():
    L = _lib.lib()
    assert L.svga_version() == 104
    assert L.svga_status_string(0) == b"ok"
    assert L.svga_status_string(-3) == b"buffer too small"


def G(F=4, H=4, W=8):
    return ctypes.byref(SvgaGeom(F, H, W))


def Mk(k=1, b=1, w=2, lay=0):
    return ctypes.byref(SvgaMask(k, b, w, lay))


def test_tilemap_layout_and_argument_errors():
    L = _lib.lib()
    off = SvgaTilemapOffsets()
    assert L.svga_tilemap_layout(G(), 32, 32, ctypes.byref(off)) == 0
    assert (off.tq, off.tk) == (4, 4)
    assert off.n_full == 64 and off.n_bnd == 64 + 32 and off.kv == 64 + 64 and off.cls == 128 + 128
    assert off.total == 512
    assert L.svga_tilemap_layout(G(), 0, 32, ctypes.byref(off)) == -1
    assert L.svga_tilemap_layout(G(0, 4, 8), 32, 32, ctypes.byref(off)) == -1
    assert L.svga_tilemap_layout(G(1 << 10, 1 << 10, 1 << 10), 32, 32, ctypes.byref(off)) == -1
    assert b"2^30" in L.svga_last_error()
    assert L.svga_tilemap_layout(None, 32, 32, ctypes.byref(off)) == -1


def test_host_builder_errors():
    L = _lib.lib()
    buf = (ctypes.c_uint8 * 512)()
    assert L.svga_build_tilemap_host(G(), Mk(), 32, 32, 2, buf, 512) == 0
    assert L.svga_build_tilemap_host(G(), Mk(), 32, 32, 2, buf, 511) == -3
    assert L.svga_build_tilemap_host(G(), Mk(), 32, 32, 7, buf, 512) == -1
    assert L.svga_build_tilemap_host(G(), Mk(k=5), 32, 32, 2, buf, 512) == -1    # sink_frames > F
    assert L.svga_build_tilemap_host(G(), Mk(b=-1), 32, 32, 2, buf, 512) == -1
    assert L.svga_build_tilemap_host(G(), Mk(lay=2), 32, 32, 2, buf, 512) == -1
    assert L.svga_build_tilemap_host(G(), Mk(), 32, 32, 2, None, 512) == -1
    assert L.svga_last_error() == b"h_map is NULL"


def test_device_entry_points_reject_bad_arguments_before_launch():
    L = _lib.lib()
    g, m = G(), Mk()
    # permute: NULL, aliasing, head_dim
    assert L.svga_permute(None, FAKE, FAKE, 1, 2, g, m, 64, None) == -1
    assert L.svga_permute(FAKE, FAKE, FAKE, 1, 2, g, m, 64, None) == -1
    assert L.svga_unpermute(FAKE, ctypes.c_void_p(0x2000), FAKE, 1, 2, g, m, 12, None) == -1
    assert L.svga_permute(FAKE, ctypes.c_void_p(0x2000), FAKE, 0, 2, g, m, 64, None) == -1
    # 2^25 tokens x 512 dims: 2^31 16-byte vectors per head, past the kernel's 31-bit indexing
    assert L.svga_permute(FAKE, ctypes.c_void_p(0x2000), FAKE, 1, 1, G(1 << 10, 1 << 10, 32), m, 512, None) == -1
    assert b"2^31" in L.svga_last_error()
    # tile map on device: capacity, too many key tiles
    assert L.svga_build_tilemap(g, m, 32, 32, 2, FAKE, 100, None) == -3
    assert L.svga_build_tilemap(G(21, 90, 160), m, 32, 32, 2, FAKE, 1 << 40, None) == -2
    # routing: head_dim, samples, workspace
    n = ctypes.c_size_t()
    assert L.svga_route_workspace_bytes(1, 2, g, 64, 64, ctypes.byref(n)) == 0 and n.value > 0
    assert L.svga_route_workspace_bytes(1, 2, g, 96, 64, ctypes.byref(n)) == -2
    assert L.svga_route_workspace_bytes(1, 2, g, 64, 65, ctypes.byref(n)) == -2
    args = (FAKE, FAKE, FAKE, 1, 2, g, m, 64, FAKE, 16, ctypes.c_float(0.125))
    assert L.svga_route_heads(*args, FAKE, n.value - 1, FAKE, None, None) == -3
    assert L.svga_route_heads(*args, FAKE, n.value, None, None, None) == -1
    # attention: unsupported head_dim / tile, capacity, aliasing, scale
    a = (FAKE, ctypes.c_void_p(0x2000), ctypes.c_void_p(0x3000))
    o = ctypes.c_void_p(0x4000)
    assert L.svga_sparse_attn_fwd(*a, o, None, 1, 2, g, m, 96, ctypes.c_float(0.1), FAKE, FAKE, 1 << 20, 32, 32, 2, 0, None) == -2
    assert L.svga_sparse_attn_fwd(*a, o, None, 1, 2, g, m, 64, ctypes.c_float(0.1), FAKE, FAKE, 1 << 20, 48, 32, 2, 0, None) == -2
    assert L.svga_sparse_attn_fwd(*a, o, None, 1, 2, g, m, 64, ctypes.c_float(0.1), FAKE, FAKE, 100, 32, 32, 2, 0, None) == -3
    assert L.svga_sparse_attn_fwd(*a, FAKE, None, 1, 2, g, m, 64, ctypes.c_float(0.1), FAKE, FAKE, 1 << 20, 32, 32, 2, 0, None) == -1
    assert L.svga_sparse_attn_fwd(*a, o, None, 1, 2, g, m, 64, ctypes.c_float(-1.0), FAKE, FAKE, 1 << 20, 32, 32, 2, 0, None) == -1
    assert L.svga_sparse_attn_fwd(*a, o, None, 1, 2, g, m, 64, ctypes.c_float(0.1), FAKE, FAKE, 1 << 20, 32, 32, 2, 2, None) == -1
    assert L.svga_sparse_attn_fwd(*a, o, None, 1, 2, g, m, 64, ctypes.c_float(0.1), None, FAKE, 1 << 20, 32, 32, 2, 0, None) == -1
    # persistent variant: workspace size query, NULL / small / misaligned workspace, then the common checks
    n = ctypes.c_size_t()
    assert L.svga_attn_workspace_bytes(ctypes.byref(n)) == 0 and n.value >= 4
    assert L.svga_attn_workspace_bytes(None) == -1
    common = (*a, o, None, 1, 2, g, m, 64, ctypes.c_float(0.1), FAKE, FAKE, 1 << 20, 32, 32, 2, 0)
    assert L.svga_sparse_attn_fwd_ws(*common, None, n.value, None) == -1
    assert L.svga_sparse_attn_fwd_ws(*common, FAKE, n.value - 1, None) == -3
    assert L.svga_sparse_attn_fwd_ws(*common, ctypes.c_void_p(0x1002), n.value, None) == -1
    assert L.svga_sparse_attn_fwd_ws(*common, ctypes.c_void_p(0x1008), n.value, None) == -1
    # split-tail workspace: only 256-row workgroups split; it grows with head_dim
    s = {}
    for d, bq in ((64, 32), (64, 256), (128, 128), (128, 256), (128, 512)):
        assert L.svga_attn_split_workspace_bytes(d, bq, ctypes.byref(n)) == 0
        s[d, bq] = n.value
    assert s[128, 256] == s[128, 512] > s[64, 256] > s[128, 128] == s[64, 32] == 256
    assert s[128, 256] == 256 + 256 * 4 * 256 * (4 + 128 * 2)
    assert L.svga_attn_split_workspace_bytes(96, 256, ctypes.byref(n)) == -2
    assert L.svga_attn_split_workspace_bytes(128, 48, ctypes.byref(n)) == -2
    assert L.svga_attn_split_workspace_bytes(128, 256, None) == -1
    bad = (*a, o, None, 1, 2, g, m, 96, ctypes.c_float(0.1), FAKE, FAKE, 1 << 20, 32, 32, 2, 0)
    assert L.svga_sparse_attn_fwd_ws(*bad, FAKE, n.value, None) == -2
    # no-alloc variant: the same host checks, before any device state is touched
    assert L.svga_sparse_attn_fwd_noalloc(*bad, None) == -2
    assert L.svga_sparse_attn_fwd_noalloc(*a, FAKE, None, 1, 2, g, m, 64, ctypes.c_float(0.1), FAKE, FAKE, 1 << 20,
                                          32, 32, 2, 0, None) == -1
    assert L.svga_sparse_attn_fwd_noalloc(*a, o, None, 1, 2, g, m, 64, ctypes.c_float(0.1), FAKE, FAKE, 100,
                                          32, 32, 2, 0, None) == -3


def test_python_binding_raises_with_message():
    import block_sparse_spatio_amd as B
    with pytest.raises(B.SvgaError) as e:
        B.svga_tilemap_layout((4, 4, 8), 0, 32)
    assert e.value.status == B.SVGA_EINVAL and "tile sizes" in str(e.value)
