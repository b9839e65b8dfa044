"""ctypes declarations of libsvga.so (include/svga.h). Loading fails loudly if the library is missing."""
import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
# SVGA_LIBRARY names another build of the same ABI (the tests' host-only sanitizer build uses it)
LIB_PATH = os.environ.get("SVGA_LIBRARY") or os.path.join(HERE, "libsvga.so")

c_i32 = ctypes.c_int32
c_size = ctypes.c_size_t
c_vp = ctypes.c_void_p
c_f32 = ctypes.c_float


class SvgaGeom(ctypes.Structure):
    _fields_ = [("F", c_i32), ("H", c_i32), ("W", c_i32)]


class SvgaMask(ctypes.Structure):
    _fields_ = [("sink_frames", c_i32), ("spatial_band", c_i32), ("temporal_band", c_i32),
                ("temporal_layout", c_i32)]


class SvgaTilemapOffsets(ctypes.Structure):
    _fields_ = [("n_full", c_size), ("n_bnd", c_size), ("kv", c_size), ("cls", c_size), ("total", c_size),
                ("tq", c_i32), ("tk", c_i32)]


G = ctypes.POINTER(SvgaGeom)
M = ctypes.POINTER(SvgaMask)

# name -> (restype, argtypes); every function declared in include/svga.h
SIGNATURES = {
    "svga_status_string": (ctypes.c_char_p, [c_i32]),
    "svga_last_error": (ctypes.c_char_p, []),
    "svga_version": (c_i32, []),
    "svga_mask_for_kept_fraction": (c_i32, [G, c_i32, c_i32, ctypes.c_double, ctypes.c_double, M,
                                            ctypes.POINTER(ctypes.c_int64)]),
    "svga_tilemap_layout": (c_i32, [G, c_i32, c_i32, ctypes.POINTER(SvgaTilemapOffsets)]),
    "svga_build_tilemap_host": (c_i32, [G, M, c_i32, c_i32, c_i32, c_vp, c_size]),
    "svga_build_tilemap": (c_i32, [G, M, c_i32, c_i32, c_i32, c_vp, c_size, c_vp]),
    "svga_permute": (c_i32, [c_vp, c_vp, c_vp, c_i32, c_i32, G, M, c_i32, c_vp]),
    "svga_unpermute": (c_i32, [c_vp, c_vp, c_vp, c_i32, c_i32, G, M, c_i32, c_vp]),
    "svga_route_workspace_bytes": (c_i32, [c_i32, c_i32, G, c_i32, c_i32, ctypes.POINTER(c_size)]),
    "svga_route_heads": (c_i32, [c_vp, c_vp, c_vp, c_i32, c_i32, G, M, c_i32, c_vp, c_i32, c_f32, c_vp, c_size,
                                 c_vp, c_vp, c_vp]),
    "svga_sparse_attn_fwd": (c_i32, [c_vp, c_vp, c_vp, c_vp, c_vp, c_i32, c_i32, G, M, c_i32, c_f32, c_vp, c_vp,
                                     c_size, c_i32, c_i32, c_i32, c_i32, c_vp]),
    "svga_attn_workspace_bytes": (c_i32, [ctypes.POINTER(c_size)]),
    "svga_attn_split_workspace_bytes": (c_i32, [c_i32, c_i32, ctypes.POINTER(c_size)]),
    "svga_sparse_attn_fwd_ws": (c_i32, [c_vp, c_vp, c_vp, c_vp, c_vp, c_i32, c_i32, G, M, c_i32, c_f32, c_vp, c_vp,
                                        c_size, c_i32, c_i32, c_i32, c_i32, c_vp, c_size, c_vp]),
    "svga_sparse_attn_fwd_noalloc": (c_i32, [c_vp, c_vp, c_vp, c_vp, c_vp, c_i32, c_i32, G, M, c_i32, c_f32, c_vp,
                                             c_vp, c_size, c_i32, c_i32, c_i32, c_i32, c_vp]),
}

_lib = None


def lib():
    """The loaded library (raises if libsvga.so has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m block_sparse_spatio_amd.build` "
                               "or __graft_entry__.build(); there is no fallback path")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib
