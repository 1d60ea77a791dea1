"""Block-sparse video attention for AMD Instinct MI355X (gfx950).

Thin Python binding over the C ABI of ``libvsa.so`` (declared in
``include/vsa.h``).  Every computation runs in the library's HIP kernels; this
module only allocates outputs and workspaces with PyTorch, passes raw device
pointers and the current HIP stream, and turns status codes into exceptions.
There is no CPU fallback: without the built library every call raises.

Functions mirror the C entry points:
    tile_permute, tile_unpermute, mask_nnz_bound, build_mask, attn_fwd,
    budget_to_radius, tile_radius_from_tokens, tile_score_from_tokens
plus ``attention``, which composes them into one block-sparse attention call.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# The in-tree build; VSA_LIBRARY names another build of the same library (the
# sanitizer-instrumented copy that build_lib --sanitize writes, for host tests).
LIB_PATH = os.environ.get("VSA_LIBRARY") or os.path.join(_HERE, "libvsa.so")

LAYOUT_TOKEN_MAJOR = 0
LAYOUT_FEATURE_MAJOR = 1

_STATUS = {0: "ok", 1: "invalid argument", 2: "unsupported", 3: "buffer too small",
           4: "index overflow", 5: "HIP runtime error"}


class VsaError(RuntimeError):
    def __init__(self, code: int, where: str, detail: str):
        super().__init__(f"{where}: {_STATUS.get(code, code)} ({detail})")
        self.code = code


class Shape(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("T", ctypes.c_int32),
                ("H", ctypes.c_int32), ("W", ctypes.c_int32)]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libvsa.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m block_sparse_attention_19_amd.build_lib`")
    L = ctypes.CDLL(LIB_PATH)
    P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    SP = ctypes.POINTER(Shape)
    sig = {
        "vsa_status_string": (ctypes.c_char_p, [ctypes.c_int]),
        "vsa_last_error": (ctypes.c_char_p, []),
        "vsa_num_tiles": (I32, [SP]),
        "vsa_tile_permute": (ctypes.c_int, [SP, P, P, I32, P]),
        "vsa_tile_unpermute": (ctypes.c_int, [SP, P, P, P]),
        "vsa_mask_nnz_bound": (I64, [SP, I32, I32]),
        "vsa_mask_workspace_bytes": (SZ, [SP]),
        "vsa_build_mask": (ctypes.c_int, [SP, P, P, I32, I32, P, P, I64, P, P, SZ, P]),
        "vsa_budget_to_radius": (ctypes.c_int, [SP, P, I32, P, P]),
        "vsa_tile_radius_from_tokens": (ctypes.c_int, [SP, P, P, P]),
        "vsa_tile_score_from_tokens": (ctypes.c_int, [SP, P, P, P]),
        "vsa_attn_workspace_bytes": (SZ, [SP, I32]),
        "vsa_attn_fwd": (ctypes.c_int, [SP, P, P, P, P, P, ctypes.c_float, P, P, I32, P, SZ, P]),
        "vsa_attn_fwd_raster": (ctypes.c_int, [SP, P, P, P, P, P, ctypes.c_float, P, P, I32, P, SZ, P]),
        "vsa_attn_noalloc_max_workspace": (SZ, []),
        "vsa_attn_fwd_raster_noalloc": (ctypes.c_int, [SP, P, P, P, P, P, ctypes.c_float, P, P, P]),
        "vsa_quantize_mxfp4": (ctypes.c_int, [SP, P, P, P, P]),
        "vsa_attn_fwd_tiered": (ctypes.c_int, [SP, P, P, P, P, P, P, P, P, P, P, ctypes.c_float,
                                               P, P, I32, P, SZ, P]),
        "vsa_attn_fwd_token_window": (ctypes.c_int, [SP, P, P, P, P, P, P, P, I32, ctypes.c_float,
                                                     P, P, I32, P, SZ, P]),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args
    _lib = L
    return L


def _check(code: int, where: str) -> None:
    if code != 0:
        raise VsaError(code, where, lib().vsa_last_error().decode())


def shape(batch: int, heads: int, head_dim: int, T: int, H: int, W: int) -> Shape:
    return Shape(batch, heads, head_dim, T, H, W)


def num_tiles(s: Shape) -> int:
    n = lib().vsa_num_tiles(ctypes.byref(s))
    if n < 0:
        raise ValueError(f"invalid shape: {lib().vsa_last_error().decode()}")
    return n


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _ptr(t: Optional[torch.Tensor]):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _require(t: torch.Tensor, dtype: torch.dtype, name: str) -> torch.Tensor:
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    return t.contiguous()


def _out(t: Optional[torch.Tensor], shp: tuple, dtype: torch.dtype, device: torch.device,
         name: str) -> Optional[torch.Tensor]:
    """A caller-supplied output buffer, checked before any launch: the kernels
    write it through a raw pointer, so its exact shape, dtype, device and
    contiguity must be those the call writes (None passes through)."""
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch tensor")
    if t.device != device:
        raise ValueError(f"{name} must be a tensor on {device}, got {t.device}")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shp):
        raise ValueError(f"{name} must have shape {tuple(shp)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _overlap(a: torch.Tensor, b: torch.Tensor) -> bool:
    """True when the byte ranges of two contiguous tensors intersect."""
    a0, b0 = a.data_ptr(), b.data_ptr()
    return a0 < b0 + b.numel() * b.element_size() and b0 < a0 + a.numel() * a.element_size()


def _same_device(device: torch.device, **tensors) -> None:
    for name, t in tensors.items():
        if t is not None and t.device != device:
            raise ValueError(f"{name} is on {t.device}, expected {device}")


def _workspace(workspace: Optional[torch.Tensor], nbytes: int, device: torch.device) -> torch.Tensor:
    """The caller's workspace if it is a contiguous uint8 buffer of at least
    `nbytes` on `device`, else a new one; a buffer of the wrong kind raises."""
    if workspace is None or workspace.numel() < nbytes:
        if workspace is not None and (workspace.dtype != torch.uint8 or workspace.device != device):
            raise ValueError(f"workspace must be a uint8 tensor on {device}")
        return torch.empty(nbytes, dtype=torch.uint8, device=device)
    if workspace.dtype != torch.uint8 or workspace.device != device or not workspace.is_contiguous():
        raise ValueError(f"workspace must be a contiguous uint8 tensor on {device}")
    return workspace


def tile_permute(x: torch.Tensor, s: Shape, layout: int = LAYOUT_TOKEN_MAJOR,
                 out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """bf16 [B, N, heads, D] raster -> tile-major (token- or feature-major tiles)."""
    x = _require(x, torch.bfloat16, "x")
    nT = num_tiles(s)
    if layout == LAYOUT_TOKEN_MAJOR:
        shp = (s.batch, s.heads, nT * 64, s.head_dim)
    else:
        shp = (s.batch, s.heads, nT, s.head_dim, 64)
    if x.shape != (s.batch, s.T * s.H * s.W, s.heads, s.head_dim):
        raise ValueError(f"x has shape {tuple(x.shape)}")
    out = _out(out, shp, torch.bfloat16, x.device, "out")
    if out is None:
        out = torch.empty(shp, dtype=torch.bfloat16, device=x.device)
    _check(lib().vsa_tile_permute(ctypes.byref(s), _ptr(x), _ptr(out), layout, _stream(x.device)),
           "vsa_tile_permute")
    return out


def tile_unpermute(o_t: torch.Tensor, s: Shape, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """bf16 [B, heads, nT*64, D] tile-major -> [B, N, heads, D] raster."""
    o_t = _require(o_t, torch.bfloat16, "o_t")
    if o_t.shape != (s.batch, s.heads, num_tiles(s) * 64, s.head_dim):
        raise ValueError(f"o_t has shape {tuple(o_t.shape)}")
    ras = (s.batch, s.T * s.H * s.W, s.heads, s.head_dim)
    out = _out(out, ras, torch.bfloat16, o_t.device, "out")
    if out is None:
        out = torch.empty(ras, dtype=torch.bfloat16, device=o_t.device)
    _check(lib().vsa_tile_unpermute(ctypes.byref(s), _ptr(o_t), _ptr(out), _stream(o_t.device)),
           "vsa_tile_unpermute")
    return out


def mask_nnz_bound(s: Shape, r_max: int, dense_count: int) -> int:
    n = lib().vsa_mask_nnz_bound(ctypes.byref(s), r_max, dense_count)
    if n < 0:
        raise ValueError("invalid shape, r_max or dense_count")
    return n


def mask_buffers(s: Shape, dense_count: int, r_max: int, device) -> Tuple[torch.Tensor, ...]:
    """Preallocated (row_ptr, col_idx, routed) for build_mask(out=...)."""
    nT = num_tiles(s)
    cap = mask_nnz_bound(s, r_max, dense_count)
    rows = s.batch * s.heads * nT
    return (torch.empty(rows + 1, dtype=torch.int32, device=device),
            torch.empty(max(cap, 1), dtype=torch.int32, device=device),
            torch.empty((s.batch, s.heads, nT), dtype=torch.uint8, device=device))


def build_mask(radii: torch.Tensor, scores: torch.Tensor, s: Shape, dense_count: int,
               r_max: Optional[int] = None, with_routed: bool = True, out=None):
    """uint8 radii / float32 scores [B, heads, nT] -> (row_ptr int32 [rows+1],
    col_idx int32 [capacity], routed uint8 [B, heads, nT] or None).

    ``r_max`` defaults to 255 (capacity for full rows).  ``out`` may pass the
    three buffers of ``mask_buffers``."""
    radii = _require(radii, torch.uint8, "radii")
    scores = _require(scores, torch.float32, "scores")
    nT = num_tiles(s)
    if radii.shape != (s.batch, s.heads, nT) or scores.shape != (s.batch, s.heads, nT):
        raise ValueError("radii / scores must be [B, heads, nT]")
    r_max = 255 if r_max is None else int(r_max)
    dev = radii.device
    _same_device(dev, scores=scores)
    if out is None:
        row_ptr, col_idx, routed = mask_buffers(s, dense_count, r_max, dev)
        if not with_routed:
            routed = None
    else:
        row_ptr, col_idx, routed = out
        rows = s.batch * s.heads * nT
        row_ptr = _out(row_ptr, (rows + 1,), torch.int32, dev, "row_ptr")
        if row_ptr is None:
            raise ValueError("out must hold a row_ptr buffer")
        if (not isinstance(col_idx, torch.Tensor) or col_idx.dim() != 1 or
                col_idx.dtype != torch.int32 or col_idx.device != dev or
                not col_idx.is_contiguous()):
            raise ValueError(f"col_idx must be a contiguous 1-d int32 tensor on {dev}")
        routed = _out(routed, (s.batch, s.heads, nT), torch.uint8, dev, "routed")
    ws_bytes = lib().vsa_mask_workspace_bytes(ctypes.byref(s))
    ws = None if routed is not None else torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    _check(lib().vsa_build_mask(ctypes.byref(s), _ptr(radii), _ptr(scores), dense_count, r_max,
                                _ptr(row_ptr), _ptr(col_idx), col_idx.numel(), _ptr(routed),
                                _ptr(ws), ws_bytes if ws is not None else 0, _stream(dev)),
           "vsa_build_mask")
    return row_ptr, col_idx, routed


def _token_array(x: torch.Tensor, s: Shape, dtype: torch.dtype, name: str) -> torch.Tensor:
    x = _require(x, dtype, name)
    if x.shape != (s.batch, s.heads, s.T * s.H * s.W):
        raise ValueError(f"{name} must be [B, heads, T*H*W], got {tuple(x.shape)}")
    return x


def budget_to_radius(budget: torch.Tensor, s: Shape, r_max: int,
                     out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """int32 key budgets per query token [B, heads, N] -> uint8 radii [B, heads, N]
    (the smallest tile radius whose window holds the budget, capped at r_max)."""
    budget = _token_array(budget, s, torch.int32, "budget")
    out = _out(out, tuple(budget.shape), torch.uint8, budget.device, "out")
    if out is None:
        out = torch.empty(budget.shape, dtype=torch.uint8, device=budget.device)
    _check(lib().vsa_budget_to_radius(ctypes.byref(s), _ptr(budget), int(r_max), _ptr(out),
                                      _stream(budget.device)), "vsa_budget_to_radius")
    return out


def tile_radius_from_tokens(token_radius: torch.Tensor, s: Shape,
                            out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """uint8 [B, heads, N] token radii -> uint8 [B, heads, nT] tile radii (max)."""
    token_radius = _token_array(token_radius, s, torch.uint8, "token_radius")
    out = _out(out, (s.batch, s.heads, num_tiles(s)), torch.uint8, token_radius.device, "out")
    if out is None:
        out = torch.empty((s.batch, s.heads, num_tiles(s)), dtype=torch.uint8,
                          device=token_radius.device)
    _check(lib().vsa_tile_radius_from_tokens(ctypes.byref(s), _ptr(token_radius), _ptr(out),
                                             _stream(token_radius.device)),
           "vsa_tile_radius_from_tokens")
    return out


def tile_score_from_tokens(token_score: torch.Tensor, s: Shape,
                           out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """float32 [B, heads, N] token scores -> float32 [B, heads, nT] tile scores
    (max in the IEEE-754 total order)."""
    token_score = _token_array(token_score, s, torch.float32, "token_score")
    out = _out(out, (s.batch, s.heads, num_tiles(s)), torch.float32, token_score.device, "out")
    if out is None:
        out = torch.empty((s.batch, s.heads, num_tiles(s)), dtype=torch.float32,
                          device=token_score.device)
    _check(lib().vsa_tile_score_from_tokens(ctypes.byref(s), _ptr(token_score), _ptr(out),
                                            _stream(token_score.device)),
           "vsa_tile_score_from_tokens")
    return out


def attn_workspace_bytes(s: Shape, kv_chunk: int = 0) -> int:
    return int(lib().vsa_attn_workspace_bytes(ctypes.byref(s), kv_chunk))


def _attn_outputs(out, lse_out, with_lse: bool, o_shape: tuple, lse_shape: tuple,
                  device: torch.device):
    """Output and LSE buffers of an attention call: the caller's, checked, or new."""
    out = _out(out, o_shape, torch.bfloat16, device, "out")
    if out is None:
        out = torch.empty(o_shape, dtype=torch.bfloat16, device=device)
    lse = _out(lse_out, lse_shape, torch.float32, device, "lse_out")
    if lse is None and with_lse:
        lse = torch.empty(lse_shape, dtype=torch.float32, device=device)
    return out, lse


def attn_fwd(q_t: torch.Tensor, k_t: torch.Tensor, v_t: torch.Tensor, row_ptr: torch.Tensor,
             col_idx: torch.Tensor, s: Shape, scale: Optional[float] = None, kv_chunk: int = 0,
             with_lse: bool = True, out: Optional[torch.Tensor] = None,
             workspace: Optional[torch.Tensor] = None,
             lse_out: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Tile-major q/k [B, heads, nT*64, D], feature-major v [B, heads, nT, D, 64]
    + CSR -> (o_t bf16 [B, heads, nT*64, D], lse float32 [B, heads, nT*64])."""
    q_t = _require(q_t, torch.bfloat16, "q_t")
    k_t = _require(k_t, torch.bfloat16, "k_t")
    v_t = _require(v_t, torch.bfloat16, "v_t")
    row_ptr = _require(row_ptr, torch.int32, "row_ptr")
    col_idx = _require(col_idx, torch.int32, "col_idx")
    nT = num_tiles(s)
    D = s.head_dim
    tok = (s.batch, s.heads, nT * 64, D)
    if q_t.shape != tok or k_t.shape != tok or v_t.shape != (s.batch, s.heads, nT, D, 64):
        raise ValueError("q_t / k_t / v_t shapes do not match the shape")
    if row_ptr.numel() != s.batch * s.heads * nT + 1:
        raise ValueError("row_ptr must have B*heads*nT + 1 entries")
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    dev = q_t.device
    _same_device(dev, k_t=k_t, v_t=v_t, row_ptr=row_ptr, col_idx=col_idx)
    out, lse = _attn_outputs(out, lse_out, with_lse, tok, tok[:3], dev)
    workspace = _workspace(workspace, attn_workspace_bytes(s, kv_chunk), dev)
    _check(lib().vsa_attn_fwd(ctypes.byref(s), _ptr(q_t), _ptr(k_t), _ptr(v_t), _ptr(row_ptr),
                              _ptr(col_idx), scale, _ptr(out), _ptr(lse), kv_chunk,
                              _ptr(workspace), workspace.numel(), _stream(dev)),
           "vsa_attn_fwd")
    return out, lse


def attn_fwd_raster(q: torch.Tensor, k_t: torch.Tensor, v_t: torch.Tensor, row_ptr: torch.Tensor,
                    col_idx: torch.Tensor, s: Shape, scale: Optional[float] = None,
                    kv_chunk: int = 0, with_lse: bool = True, out: Optional[torch.Tensor] = None,
                    workspace: Optional[torch.Tensor] = None,
                    lse_out: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Raster q [B, N, heads, D], tile-major k_t, feature-major v_t + CSR ->
    (o bf16 [B, N, heads, D], lse float32 [B, heads, N]): the Q permute and the
    O unpermute happen inside the call."""
    q = _require(q, torch.bfloat16, "q")
    k_t = _require(k_t, torch.bfloat16, "k_t")
    v_t = _require(v_t, torch.bfloat16, "v_t")
    row_ptr = _require(row_ptr, torch.int32, "row_ptr")
    col_idx = _require(col_idx, torch.int32, "col_idx")
    nT = num_tiles(s)
    D = s.head_dim
    N = s.T * s.H * s.W
    ras = (s.batch, N, s.heads, D)
    if q.shape != ras:
        raise ValueError("q must be [B, N, heads, D]")
    if k_t.shape != (s.batch, s.heads, nT * 64, D) or v_t.shape != (s.batch, s.heads, nT, D, 64):
        raise ValueError("k_t / v_t shapes do not match the shape")
    if row_ptr.numel() != s.batch * s.heads * nT + 1:
        raise ValueError("row_ptr must have B*heads*nT + 1 entries")
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    dev = q.device
    _same_device(dev, k_t=k_t, v_t=v_t, row_ptr=row_ptr, col_idx=col_idx)
    out, lse = _attn_outputs(out, lse_out, with_lse, ras, (s.batch, s.heads, N), dev)
    if _overlap(out, q):
        raise ValueError("out must not overlap q")
    workspace = _workspace(workspace, attn_workspace_bytes(s, kv_chunk), dev)
    _check(lib().vsa_attn_fwd_raster(ctypes.byref(s), _ptr(q), _ptr(k_t), _ptr(v_t),
                                     _ptr(row_ptr), _ptr(col_idx), scale, _ptr(out), _ptr(lse),
                                     kv_chunk, _ptr(workspace), workspace.numel(), _stream(dev)),
           "vsa_attn_fwd_raster")
    return out, lse


def attn_noalloc_max_workspace() -> int:
    """Bytes of the library's fixed workspace used by attn_fwd_raster_noalloc."""
    return int(lib().vsa_attn_noalloc_max_workspace())


def attn_fwd_raster_noalloc(q: torch.Tensor, k_t: torch.Tensor, v_t: torch.Tensor,
                            row_ptr: torch.Tensor, col_idx: torch.Tensor, s: Shape,
                            scale: Optional[float] = None, with_lse: bool = True,
                            out: Optional[torch.Tensor] = None,
                            lse_out: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """attn_fwd_raster (kv_chunk 0) on the library's fixed device workspace:
    the C call allocates nothing (outputs passed here are used as given; None
    allocates them on the PyTorch side).  Calls in flight at once on one GPU
    share that workspace and must be serialised."""
    q = _require(q, torch.bfloat16, "q")
    k_t = _require(k_t, torch.bfloat16, "k_t")
    v_t = _require(v_t, torch.bfloat16, "v_t")
    row_ptr = _require(row_ptr, torch.int32, "row_ptr")
    col_idx = _require(col_idx, torch.int32, "col_idx")
    nT = num_tiles(s)
    D = s.head_dim
    N = s.T * s.H * s.W
    ras = (s.batch, N, s.heads, D)
    if q.shape != ras:
        raise ValueError("q must be [B, N, heads, D]")
    if k_t.shape != (s.batch, s.heads, nT * 64, D) or v_t.shape != (s.batch, s.heads, nT, D, 64):
        raise ValueError("k_t / v_t shapes do not match the shape")
    if row_ptr.numel() != s.batch * s.heads * nT + 1:
        raise ValueError("row_ptr must have B*heads*nT + 1 entries")
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    dev = q.device
    _same_device(dev, k_t=k_t, v_t=v_t, row_ptr=row_ptr, col_idx=col_idx)
    out, lse = _attn_outputs(out, lse_out, with_lse, ras, (s.batch, s.heads, N), dev)
    if _overlap(out, q):
        raise ValueError("out must not overlap q")
    _check(lib().vsa_attn_fwd_raster_noalloc(ctypes.byref(s), _ptr(q), _ptr(k_t), _ptr(v_t),
                                             _ptr(row_ptr), _ptr(col_idx), scale, _ptr(out),
                                             _ptr(lse), _stream(dev)),
           "vsa_attn_fwd_raster_noalloc")
    return out, lse


def quantize_mxfp4(x_t: torch.Tensor, s: Shape, codes: Optional[torch.Tensor] = None,
                   scales: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Token-major tiled bf16 q or k [B, heads, nT*64, D] -> MXFP4 (codes uint8
    [B, heads, nT*64, D/2], E8M0 scales uint8 [B, heads, nT*64, D/32])."""
    x_t = _require(x_t, torch.bfloat16, "x_t")
    nT, D = num_tiles(s), s.head_dim
    tok = (s.batch, s.heads, nT * 64, D)
    if x_t.shape != tok:
        raise ValueError("x_t shape does not match the shape")
    dev = x_t.device
    codes = _out(codes, tok[:3] + (D // 2,), torch.uint8, dev, "codes")
    scales = _out(scales, tok[:3] + (D // 32,), torch.uint8, dev, "scales")
    if codes is None:
        codes = torch.empty(tok[:3] + (D // 2,), dtype=torch.uint8, device=dev)
    if scales is None:
        scales = torch.empty(tok[:3] + (D // 32,), dtype=torch.uint8, device=dev)
    _check(lib().vsa_quantize_mxfp4(ctypes.byref(s), _ptr(x_t), _ptr(codes), _ptr(scales),
                                    _stream(dev)), "vsa_quantize_mxfp4")
    return codes, scales


def attn_fwd_tiered(q_t: torch.Tensor, k_t: torch.Tensor, v_t: torch.Tensor,
                    q4: Tuple[torch.Tensor, torch.Tensor], k4: Tuple[torch.Tensor, torch.Tensor],
                    row_ptr: torch.Tensor, col_idx: torch.Tensor, tier: torch.Tensor, s: Shape,
                    scale: Optional[float] = None, kv_chunk: int = 0, with_lse: bool = True,
                    out: Optional[torch.Tensor] = None,
                    workspace: Optional[torch.Tensor] = None,
                    lse_out: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """attn_fwd with a tier byte per CSR entry (non-zero = skim: the pair's
    scores from the MXFP4 q4 / k4, each a (codes, scales) pair from
    quantize_mxfp4).  `tier` must hold at least row_ptr[-1] bytes, as col_idx
    must hold row_ptr[-1] entries: that count lives on the device, so it is
    not checked here (reading it would synchronise the stream)."""
    q_t = _require(q_t, torch.bfloat16, "q_t")
    k_t = _require(k_t, torch.bfloat16, "k_t")
    v_t = _require(v_t, torch.bfloat16, "v_t")
    row_ptr = _require(row_ptr, torch.int32, "row_ptr")
    col_idx = _require(col_idx, torch.int32, "col_idx")
    tier = _require(tier, torch.uint8, "tier")
    q4c, q4s = (_require(t, torch.uint8, "q4") for t in q4)
    k4c, k4s = (_require(t, torch.uint8, "k4") for t in k4)
    nT = num_tiles(s)
    D = s.head_dim
    tok = (s.batch, s.heads, nT * 64, D)
    if q_t.shape != tok or k_t.shape != tok or v_t.shape != (s.batch, s.heads, nT, D, 64):
        raise ValueError("q_t / k_t / v_t shapes do not match the shape")
    for c, sc in ((q4c, q4s), (k4c, k4s)):
        if c.numel() != q_t.numel() // 2 or sc.numel() != q_t.numel() // 32:
            raise ValueError("MXFP4 codes / scales do not match the shape")
    _same_device(q_t.device, q4=q4c, q4_scales=q4s, k4=k4c, k4_scales=k4s, tier=tier)
    if row_ptr.numel() != s.batch * s.heads * nT + 1:
        raise ValueError("row_ptr must have B*heads*nT + 1 entries")
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    dev = q_t.device
    _same_device(dev, k_t=k_t, v_t=v_t, row_ptr=row_ptr, col_idx=col_idx)
    out, lse = _attn_outputs(out, lse_out, with_lse, tok, tok[:3], dev)
    workspace = _workspace(workspace, attn_workspace_bytes(s, kv_chunk), dev)
    _check(lib().vsa_attn_fwd_tiered(ctypes.byref(s), _ptr(q_t), _ptr(k_t), _ptr(v_t), _ptr(q4c),
                                     _ptr(q4s), _ptr(k4c), _ptr(k4s), _ptr(row_ptr),
                                     _ptr(col_idx), _ptr(tier), scale, _ptr(out), _ptr(lse),
                                     kv_chunk, _ptr(workspace), workspace.numel(), _stream(dev)),
           "vsa_attn_fwd_tiered")
    return out, lse


def attn_fwd_token_window(q_t: torch.Tensor, k_t: torch.Tensor, v_t: torch.Tensor,
                          row_ptr: torch.Tensor, col_idx: torch.Tensor, routed: torch.Tensor,
                          token_radius: torch.Tensor, s: Shape, r_max: int,
                          scale: Optional[float] = None, kv_chunk: int = 0,
                          with_lse: bool = True, out: Optional[torch.Tensor] = None,
                          workspace: Optional[torch.Tensor] = None,
                          lse_out: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """attn_fwd with exact per-token windows: each query token attends only the
    kept key tiles inside the window of its own radius min(token_radius, r_max)
    (routed query tiles attend every kept key tile).  routed uint8 [B, heads,
    nT] and the CSR come from build_mask on tile radii that cover the token
    radii (tile_radius_from_tokens) with the same r_max; token_radius uint8
    [B, heads, T*H*W] in raster order."""
    q_t = _require(q_t, torch.bfloat16, "q_t")
    k_t = _require(k_t, torch.bfloat16, "k_t")
    v_t = _require(v_t, torch.bfloat16, "v_t")
    row_ptr = _require(row_ptr, torch.int32, "row_ptr")
    col_idx = _require(col_idx, torch.int32, "col_idx")
    routed = _require(routed, torch.uint8, "routed")
    nT = num_tiles(s)
    D = s.head_dim
    tok = (s.batch, s.heads, nT * 64, D)
    if q_t.shape != tok or k_t.shape != tok or v_t.shape != (s.batch, s.heads, nT, D, 64):
        raise ValueError("q_t / k_t / v_t shapes do not match the shape")
    if row_ptr.numel() != s.batch * s.heads * nT + 1:
        raise ValueError("row_ptr must have B*heads*nT + 1 entries")
    if routed.numel() != s.batch * s.heads * nT:
        raise ValueError("routed must be [B, heads, nT]")
    token_radius = _token_array(token_radius, s, torch.uint8, "token_radius")
    _same_device(q_t.device, routed=routed, token_radius=token_radius)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    dev = q_t.device
    _same_device(dev, k_t=k_t, v_t=v_t, row_ptr=row_ptr, col_idx=col_idx)
    out, lse = _attn_outputs(out, lse_out, with_lse, tok, tok[:3], dev)
    workspace = _workspace(workspace, attn_workspace_bytes(s, kv_chunk), dev)
    _check(lib().vsa_attn_fwd_token_window(ctypes.byref(s), _ptr(q_t), _ptr(k_t), _ptr(v_t),
                                           _ptr(row_ptr), _ptr(col_idx), _ptr(routed),
                                           _ptr(token_radius), int(r_max), scale, _ptr(out),
                                           _ptr(lse), kv_chunk, _ptr(workspace),
                                           workspace.numel(), _stream(dev)),
           "vsa_attn_fwd_token_window")
    return out, lse


def attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, grid: Tuple[int, int, int],
              radii: torch.Tensor, scores: torch.Tensor, dense_count: int,
              scale: Optional[float] = None, r_max: Optional[int] = None,
              kv_chunk: int = 0, fused: bool = True) -> torch.Tensor:
    """Block-sparse attention of bf16 q, k, v [B, N, heads, D] (token raster
    order over the T x H x W grid) -> o [B, N, heads, D].  fused: the raster
    forward call (Q gathered and O written inside it); otherwise the Q permute,
    the tile-major forward call and the O unpermute, with the same result."""
    T, H, W = grid
    B, N, heads, D = q.shape
    s = shape(B, heads, D, T, H, W)
    k_t = tile_permute(k, s, LAYOUT_TOKEN_MAJOR)
    v_t = tile_permute(v, s, LAYOUT_FEATURE_MAJOR)
    row_ptr, col_idx, _ = build_mask(radii, scores, s, dense_count, r_max, with_routed=True)
    if fused:
        o, _ = attn_fwd_raster(q, k_t, v_t, row_ptr, col_idx, s, scale, kv_chunk, with_lse=False)
        return o
    q_t = tile_permute(q, s, LAYOUT_TOKEN_MAJOR)
    o_t, _ = attn_fwd(q_t, k_t, v_t, row_ptr, col_idx, s, scale, kv_chunk, with_lse=False)
    return tile_unpermute(o_t, s)
