"""Thin Python binding of libsvga (include/svga.h): argument marshalling only.

Every function here has the name of the C entry point it calls. torch tensors
supply device memory and the current HIP stream; all computation happens in
the library's HIP kernels (there is no fallback path).
"""
import ctypes
import math

import numpy as np
import torch

from ._lib import SvgaGeom, SvgaMask, SvgaTilemapOffsets, lib

SVGA_OK = 0
SVGA_EINVAL = -1
SVGA_EUNSUPPORTED = -2
SVGA_ECAPACITY = -3
SVGA_EHIP = -4

KIND_SPATIAL, KIND_TEMPORAL = 0, 1
TL_SINK_FIRST, TL_LITERAL = 0, 1
MAP_DENSE, MAP_NAIVE, MAP_EXACT, MAP_ROUNDED = 0, 1, 2, 3
TILE_SKIP, TILE_FULL, TILE_BOUNDARY = 0, 1, 2
MODES = {"dense": MAP_DENSE, "naive": MAP_NAIVE, "exact": MAP_EXACT, "rounded": MAP_ROUNDED}


class SvgaError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(message)
        self.status = status


def _check(status):
    if status != SVGA_OK:
        L = lib()
        raise SvgaError(status, f"{L.svga_status_string(status).decode()}: {L.svga_last_error().decode()}")


def make_geom(F, H, W):
    return SvgaGeom(int(F), int(H), int(W))


def make_mask(sink_frames=1, spatial_band=0, temporal_band=0, temporal_layout=TL_SINK_FIRST):
    return SvgaMask(int(sink_frames), int(spatial_band), int(temporal_band), int(temporal_layout))


def _geom(g):
    return g if isinstance(g, SvgaGeom) else make_geom(*g)


def _mask(m):
    if isinstance(m, SvgaMask):
        return m
    if isinstance(m, dict):
        return make_mask(**m)
    return make_mask(*m)


def _mode(mode):
    return MODES[mode] if isinstance(mode, str) else int(mode)


def _vp(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _qkv_check(*ts):
    for t in ts:
        if not (isinstance(t, torch.Tensor) and t.is_cuda and t.dtype == torch.bfloat16 and t.is_contiguous()
                and t.dim() == 4):
            raise ValueError("expected contiguous bfloat16 CUDA tensors of shape [B, heads, N, head_dim]")
        if t.shape != ts[0].shape or t.device != ts[0].device:
            raise ValueError(f"tensor of shape {tuple(t.shape)} on {t.device} does not match "
                             f"{tuple(ts[0].shape)} on {ts[0].device}")


def _buf(name, t, device, dtype=None, min_numel=0):
    """A device buffer handed to the library: contiguous, on `device`, of `dtype`, large enough."""
    if t is None:
        return
    if not (isinstance(t, torch.Tensor) and t.device == device and t.is_contiguous()):
        raise ValueError(f"{name} must be a contiguous tensor on {device}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if t.numel() < min_numel:
        raise ValueError(f"{name} holds {t.numel()} elements, needs {min_numel}")


def svga_version():
    return lib().svga_version()


def svga_mask_for_kept_fraction(geom, sink_frames, spatial_target, temporal_target, temporal_layout=TL_SINK_FIRST):
    """(mask, (kept_spatial, kept_temporal)): the smallest bands whose kept pairs per head reach the targets."""
    m = SvgaMask()
    kept = (ctypes.c_int64 * 2)()
    _check(lib().svga_mask_for_kept_fraction(ctypes.byref(_geom(geom)), int(sink_frames), int(temporal_layout),
                                             float(spatial_target), float(temporal_target), ctypes.byref(m), kept))
    return m, (int(kept[0]), int(kept[1]))


def svga_tilemap_layout(geom, bq, bkv):
    off = SvgaTilemapOffsets()
    _check(lib().svga_tilemap_layout(ctypes.byref(_geom(geom)), int(bq), int(bkv), ctypes.byref(off)))
    return off


def svga_build_tilemap_host(geom, mask, bq, bkv, mode):
    """Tile map built on the CPU, as a numpy uint8 blob."""
    off = svga_tilemap_layout(geom, bq, bkv)
    blob = np.zeros(off.total, dtype=np.uint8)
    _check(lib().svga_build_tilemap_host(ctypes.byref(_geom(geom)), ctypes.byref(_mask(mask)), int(bq), int(bkv),
                                         _mode(mode), blob.ctypes.data_as(ctypes.c_void_p), blob.nbytes))
    return blob


def svga_build_tilemap(geom, mask, bq, bkv, mode, out=None, device="cuda", stream=None):
    """Tile map built by the GPU into a uint8 device tensor (enqueued, not synchronised)."""
    off = svga_tilemap_layout(geom, bq, bkv)
    if out is None:
        out = torch.empty(off.total, dtype=torch.uint8, device=device)
    if not (isinstance(out, torch.Tensor) and out.is_cuda):
        raise ValueError("out must be a CUDA tensor")
    _buf("out", out, out.device, torch.uint8)
    _check(lib().svga_build_tilemap(ctypes.byref(_geom(geom)), ctypes.byref(_mask(mask)), int(bq), int(bkv),
                                    _mode(mode), _vp(out), out.numel() * out.element_size(), _stream(stream)))
    return out


def tilemap_views(blob, geom, bq, bkv):
    """n_full, n_bnd [2, tq]; kv, cls [2, tq, tk] views of a tile-map blob (numpy or torch)."""
    off = svga_tilemap_layout(geom, bq, bkv)
    tq, tk = off.tq, off.tk
    if isinstance(blob, torch.Tensor):
        def view(o, n, dt):
            return blob[o:o + n * torch.tensor([], dtype=dt).element_size()].view(dt)
        i32, i8 = torch.int32, torch.int8
    else:
        def view(o, n, dt):
            return blob[o:o + n * np.dtype(dt).itemsize].view(dt)
        i32, i8 = np.int32, np.int8
    return {
        "header": view(0, 16, i32),
        "n_full": view(off.n_full, 2 * tq, i32).reshape(2, tq),
        "n_bnd": view(off.n_bnd, 2 * tq, i32).reshape(2, tq),
        "kv": view(off.kv, 2 * tq * tk, i32).reshape(2, tq, tk),
        "cls": view(off.cls, 2 * tq * tk, i8).reshape(2, tq, tk),
        "tq": tq, "tk": tk,
    }


def _permute(fn, x, flags, geom, mask, out, stream):
    _qkv_check(x)
    out = torch.empty_like(x) if out is None else out
    _qkv_check(x, out)
    B, H, N, d = x.shape
    _buf("flags", flags, x.device, torch.uint8, B * H)
    _check(fn(_vp(x), _vp(out), _vp(flags), B, H, ctypes.byref(_geom(geom)), ctypes.byref(_mask(mask)), d,
              _stream(stream)))
    return out


def svga_permute(x, flags, geom, mask, out=None, stream=None):
    """Frame-major -> temporal order for heads whose flag is set; copy for the others."""
    return _permute(lib().svga_permute, x, flags, geom, mask, out, stream)


def svga_unpermute(x, flags, geom, mask, out=None, stream=None):
    """Inverse of svga_permute."""
    return _permute(lib().svga_unpermute, x, flags, geom, mask, out, stream)


def svga_route_workspace_bytes(B, heads, geom, head_dim, n_samples):
    n = ctypes.c_size_t()
    _check(lib().svga_route_workspace_bytes(int(B), int(heads), ctypes.byref(_geom(geom)), int(head_dim),
                                            int(n_samples), ctypes.byref(n)))
    return n.value


def svga_route_heads(q, k, v, geom, mask, sample_idx, softmax_scale=None, workspace=None, flags_out=None,
                     err_out=None, want_err=True, stream=None):
    """Per-(batch, head) routing flags (uint8, 1 = temporal) and (err_spatial, err_temporal)."""
    _qkv_check(q, k, v)
    B, H, N, d = q.shape
    ns = sample_idx.numel()
    if workspace is None:
        workspace = torch.empty(svga_route_workspace_bytes(B, H, geom, d, ns), dtype=torch.uint8, device=q.device)
    if flags_out is None:
        flags_out = torch.empty(B, H, dtype=torch.uint8, device=q.device)
    if err_out is None and want_err:
        err_out = torch.empty(B, H, 2, dtype=torch.float32, device=q.device)
    _buf("sample_idx", sample_idx, q.device, torch.int32)
    _buf("workspace", workspace, q.device)
    _buf("flags_out", flags_out, q.device, torch.uint8, B * H)
    _buf("err_out", err_out, q.device, torch.float32, B * H * 2)
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else softmax_scale
    _check(lib().svga_route_heads(_vp(q), _vp(k), _vp(v), B, H, ctypes.byref(_geom(geom)),
                                  ctypes.byref(_mask(mask)), d, _vp(sample_idx), ns, float(scale), _vp(workspace),
                                  workspace.numel() * workspace.element_size(), _vp(flags_out), _vp(err_out),
                                  _stream(stream)))
    return flags_out, err_out


def svga_attn_workspace_bytes():
    """Device workspace bytes of svga_sparse_attn_fwd with a workspace (persistent workgroups)."""
    n = ctypes.c_size_t()
    _check(lib().svga_attn_workspace_bytes(ctypes.byref(n)))
    return n.value


def svga_attn_split_workspace_bytes(head_dim, bq):
    """Device workspace bytes with which svga_sparse_attn_fwd_ws also splits its last query tiles."""
    n = ctypes.c_size_t()
    _check(lib().svga_attn_split_workspace_bytes(int(head_dim), int(bq), ctypes.byref(n)))
    return n.value


def svga_sparse_attn_fwd(q, k, v, flags, tilemap, geom, mask, bq, bkv, mode, softmax_scale=None,
                         gather_temporal=False, out=None, lse=None, want_lse=False, workspace=None, stream=None,
                         noalloc=False):
    """Block-sparse attention forward. Returns (out, lse); lse is None unless requested.
    With `workspace` (a 16-byte aligned device tensor of at least svga_attn_workspace_bytes() bytes)
    the call runs persistent workgroups (svga_sparse_attn_fwd_ws): the same bits as without it, unless
    the workspace holds svga_attn_split_workspace_bytes(d, bq) bytes, in which case the last query
    tiles run in pieces merged through their softmax statistics (equal up to rounding).
    With `noalloc=True` (and no workspace) the call is svga_sparse_attn_fwd_noalloc: the launch of the
    split-tail workspace, on the library's own per-GPU scratch array (the library allocates nothing;
    calls on one GPU must not overlap). `out` and `lse`, when given, are then the only buffers used."""
    _qkv_check(q, k, v)
    B, H, N, d = q.shape
    out = torch.empty_like(q) if out is None else out
    _qkv_check(q, out)
    if lse is None and want_lse:
        lse = torch.empty(B, H, N, dtype=torch.float32, device=q.device)
    _buf("lse", lse, q.device, torch.float32, B * H * N)
    _buf("flags", flags, q.device, torch.uint8, B * H)
    _buf("tilemap", tilemap, q.device, torch.uint8)
    _buf("workspace", workspace, q.device)
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else softmax_scale
    args = (_vp(q), _vp(k), _vp(v), _vp(out), _vp(lse), B, H, ctypes.byref(_geom(geom)), ctypes.byref(_mask(mask)), d,
            float(scale), _vp(flags), _vp(tilemap), tilemap.numel() * tilemap.element_size(), int(bq), int(bkv),
            _mode(mode), 1 if gather_temporal else 0)
    if noalloc:
        if workspace is not None:
            raise ValueError("noalloc=True takes no workspace")
        _check(lib().svga_sparse_attn_fwd_noalloc(*args, _stream(stream)))
    elif workspace is None:
        _check(lib().svga_sparse_attn_fwd(*args, _stream(stream)))
    else:
        _check(lib().svga_sparse_attn_fwd_ws(*args, _vp(workspace), workspace.numel() * workspace.element_size(),
                                             _stream(stream)))
    return out, lse
