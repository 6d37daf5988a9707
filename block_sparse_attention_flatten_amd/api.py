"""Python binding of libnabla: the C ABI's calls under the same names, taking
torch tensors.  Argument marshalling only -- every step runs in the HIP
kernels behind include/nabla.h; PyTorch provides device memory and the stream.

Tensor layouts are those of the C header:
  THW      [B, heads, T, H, W, d]      (natural latent order, valid tokens)
  BLOCKED  [B, heads, nb, 64, d]       (fractal-flattened, padded)
  qbar float32 [B, heads, nb, d]; kbar bf16 [B, heads, nb16, 3 d]: each mean
  as three exact bf16 parts in the header's tiled order (nb16 = nb rounded up
  to 16; kbar_shape, KBAR_DTYPE, kbar_untile);
  mask words uint32 stored in int32
  tensors [B, heads, nb, ceil(nb/32)]; row counts int32 [B, heads, nb];
  row_ptr int32 [B*heads, nb+1]; col_idx int32 [B*heads, nb*nb].
"""
from __future__ import annotations

import ctypes
import math
from dataclasses import dataclass
from typing import Optional, Sequence, Tuple

import torch

from . import _lib
from ._lib import DTYPE_BF16, DTYPE_F32, LAYOUT_BLOCKED, LAYOUT_THW, nabla_geom

__all__ = [
    "NablaError", "Geometry", "nabla_num_blocks", "nabla_flatten", "nabla_unflatten",
    "nabla_pool", "nabla_mask", "nabla_compact", "nabla_mask_build", "nabla_attn_fwd",
    "nabla_transpose_v", "nabla_dense_attn_fwd", "nabla_qkv_split", "qkv_shape", "qbar_shape",
    "kbar_shape", "kbar_untile", "KBAR_DTYPE",
    "nabla_attn_fwd_vt", "nabla_forward_workspace_size", "nabla_forward", "nabla_forward_noalloc",
    "nabla_status_string",
    "nabla_attn_fwd_lse", "nabla_attn_fwd_vt_lse", "nabla_mask_transpose", "nabla_attn_bwd_dq",
    "nabla_attn_bwd_dkdv", "forward", "backward", "vt_shape", "lse_shape",
    "LAYOUT_THW", "LAYOUT_BLOCKED",
]


class NablaError(RuntimeError):
    def __init__(self, status: int, where: str):
        lib = _lib.load()
        text = lib.nabla_status_string(status).decode()
        extra = ""
        if status == -10:
            extra = f" (hipError {lib.nabla_last_hip_error()})"
        super().__init__(f"{where}: {_lib.STATUS.get(status, status)}: {text}{extra}")
        self.status = status


def _check(status: int, where: str) -> None:
    if status != _lib.NABLA_OK:
        raise NablaError(status, where)


_DT = {torch.float32: DTYPE_F32, torch.bfloat16: DTYPE_BF16}


@dataclass(frozen=True)
class Geometry:
    """Shape of one call (mirrors nabla_geom)."""

    batch: int
    heads: int
    T: int
    H: int
    W: int
    head_dim: int
    dtype: torch.dtype
    layout: int = LAYOUT_THW
    P: int = 8
    out_dtype: Optional[torch.dtype] = None   # dtype of O; None = dtype

    @property
    def odtype(self) -> torch.dtype:
        return self.dtype if self.out_dtype is None else self.out_dtype

    @property
    def gh(self) -> int:
        return -(-self.H // self.P)

    @property
    def gw(self) -> int:
        return -(-self.W // self.P)

    @property
    def nb(self) -> int:
        return self.T * self.gh * self.gw

    @property
    def nw(self) -> int:
        return -(-self.nb // 32)

    def c(self) -> nabla_geom:
        return nabla_geom(self.batch, self.heads, self.T, self.H, self.W, self.P, self.head_dim,
                          _DT.get(self.dtype, -1), self.layout, _DT.get(self.odtype, -1))

    def tensor_shape(self, layout: Optional[int] = None) -> Tuple[int, ...]:
        lay = self.layout if layout is None else layout
        if lay == LAYOUT_THW:
            return (self.batch, self.heads, self.T, self.H, self.W, self.head_dim)
        return (self.batch, self.heads, self.nb, 64, self.head_dim)

    def with_layout(self, layout: int) -> "Geometry":
        return Geometry(self.batch, self.heads, self.T, self.H, self.W, self.head_dim,
                        self.dtype, layout, self.P, self.out_dtype)


def _ptr(t: Optional[torch.Tensor], name: str, shape=None, dtype=None) -> Optional[int]:
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor (got {t.device})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must have dtype {dtype} (got {t.dtype})")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)} (got {tuple(t.shape)})")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _sta(sta: Optional[Sequence[int]]):
    if sta is None:
        return None
    arr = (ctypes.c_int32 * 3)(*[int(x) for x in sta])
    return arr


def nabla_status_string(status: int) -> str:
    return _lib.load().nabla_status_string(status).decode()


def nabla_num_blocks(g: Geometry) -> int:
    out = ctypes.c_int64(0)
    _check(_lib.load().nabla_num_blocks(ctypes.byref(g.c()), ctypes.byref(out)),
           "nabla_num_blocks")
    return out.value


def nabla_flatten(g: Geometry, x: torch.Tensor, x_blocked: torch.Tensor, stream=None) -> None:
    lib = _lib.load()
    _check(lib.nabla_flatten(ctypes.byref(g.c()),
                             _ptr(x, "x", g.tensor_shape(LAYOUT_THW), g.dtype),
                             _ptr(x_blocked, "x_blocked", g.tensor_shape(LAYOUT_BLOCKED), g.dtype),
                             _stream(stream)), "nabla_flatten")


def nabla_unflatten(g: Geometry, x_blocked: torch.Tensor, x: torch.Tensor, stream=None) -> None:
    lib = _lib.load()
    _check(lib.nabla_unflatten(ctypes.byref(g.c()),
                               _ptr(x_blocked, "x_blocked", g.tensor_shape(LAYOUT_BLOCKED),
                                    g.dtype),
                               _ptr(x, "x", g.tensor_shape(LAYOUT_THW), g.dtype),
                               _stream(stream)), "nabla_unflatten")


def qbar_shape(g: Geometry) -> Tuple[int, ...]:
    """Pooled queries [B, heads, nb, d] float32."""
    return (g.batch, g.heads, g.nb, g.head_dim)


# element type of the pooled keys (three bf16 parts per float32 mean)
KBAR_DTYPE = torch.bfloat16


def kbar_shape(g: Geometry) -> Tuple[int, ...]:
    """Pooled keys [B, heads, nb16, 3 d] of KBAR_DTYPE, nb16 = nb rounded up
    to 16: the 3 nb16 d bf16 parts of a head in the header's tiled order (the
    shape only sizes the buffer)."""
    return (g.batch, g.heads, -(-g.nb // 16) * 16, 3 * g.head_dim)


def kbar_untile(kbar: torch.Tensor, nb: int) -> torch.Tensor:
    """Pooled keys in their split, tiled encoding -> float32 [.., nb, d] rows
    (a copy for inspection: each mean is h + m + l of its three parts, summed
    in float32 as (h + m) + l, which gives the mean back exactly)."""
    *lead, nb16, d3 = kbar.shape
    d = d3 // 3
    # [tile j, k-step t, part p, channel group g, row i, channel e]
    x = kbar.reshape(*lead, nb16 // 16, d // 32, 3, 4, 16, 8).to(torch.float32)
    x = (x[..., 0, :, :, :] + x[..., 1, :, :, :]) + x[..., 2, :, :, :]   # [j, t, g, i, e]
    x = x.movedim(-2, -4)                                                 # [j, i, t, g, e]
    return x.reshape(*lead, nb16, d)[..., :nb, :]


def nabla_pool(g: Geometry, q, k, qbar, kbar, stream=None) -> None:
    shp = g.tensor_shape()
    _check(_lib.load().nabla_pool(
        ctypes.byref(g.c()), _ptr(q, "q", shp, g.dtype), _ptr(k, "k", shp, g.dtype),
        _ptr(qbar, "qbar", qbar_shape(g), torch.float32),
        _ptr(kbar, "kbar", kbar_shape(g), KBAR_DTYPE),
        _stream(stream)), "nabla_pool")


def nabla_mask(g: Geometry, qbar, kbar, thr: float, sta, mask_bits, row_count,
               adaptive_bits=None, stream=None) -> None:
    mshape = (g.batch, g.heads, g.nb, g.nw)
    _check(_lib.load().nabla_mask(
        ctypes.byref(g.c()), _ptr(qbar, "qbar", qbar_shape(g), torch.float32),
        _ptr(kbar, "kbar", kbar_shape(g), KBAR_DTYPE), float(thr), _sta(sta),
        _ptr(mask_bits, "mask_bits", mshape, torch.int32),
        _ptr(row_count, "row_count", (g.batch, g.heads, g.nb), torch.int32),
        _ptr(adaptive_bits, "adaptive_bits", mshape, torch.int32), _stream(stream)),
        "nabla_mask")


def nabla_compact(g: Geometry, mask_bits, row_count, row_ptr, col_idx, stream=None) -> None:
    bh = g.batch * g.heads
    _check(_lib.load().nabla_compact(
        ctypes.byref(g.c()),
        _ptr(mask_bits, "mask_bits", (g.batch, g.heads, g.nb, g.nw), torch.int32),
        _ptr(row_count, "row_count", (g.batch, g.heads, g.nb), torch.int32),
        _ptr(row_ptr, "row_ptr", (bh, g.nb + 1), torch.int32),
        _ptr(col_idx, "col_idx", (bh, g.nb * g.nb), torch.int32), _stream(stream)),
        "nabla_compact")


def nabla_mask_build(g: Geometry, q, k, thr: float, sta, qbar, kbar, mask_bits, row_count,
                     adaptive_bits, row_ptr, col_idx, stream=None) -> None:
    shp = g.tensor_shape()
    mshape = (g.batch, g.heads, g.nb, g.nw)
    bh = g.batch * g.heads
    _check(_lib.load().nabla_mask_build(
        ctypes.byref(g.c()), _ptr(q, "q", shp, g.dtype), _ptr(k, "k", shp, g.dtype), float(thr),
        _sta(sta), _ptr(qbar, "qbar", qbar_shape(g), torch.float32),
        _ptr(kbar, "kbar", kbar_shape(g), KBAR_DTYPE),
        _ptr(mask_bits, "mask_bits", mshape, torch.int32),
        _ptr(row_count, "row_count", (g.batch, g.heads, g.nb), torch.int32),
        _ptr(adaptive_bits, "adaptive_bits", mshape, torch.int32),
        _ptr(row_ptr, "row_ptr", (bh, g.nb + 1), torch.int32),
        _ptr(col_idx, "col_idx", (bh, g.nb * g.nb), torch.int32), _stream(stream)),
        "nabla_mask_build")


def nabla_attn_fwd(g: Geometry, q, k, v, row_ptr, col_idx, scale: float, o, stream=None) -> None:
    shp = g.tensor_shape()
    bh = g.batch * g.heads
    _check(_lib.load().nabla_attn_fwd(
        ctypes.byref(g.c()), _ptr(q, "q", shp, g.dtype), _ptr(k, "k", shp, g.dtype),
        _ptr(v, "v", shp, g.dtype), _ptr(row_ptr, "row_ptr", (bh, g.nb + 1), torch.int32),
        _ptr(col_idx, "col_idx", (bh, g.nb * g.nb), torch.int32), float(scale),
        _ptr(o, "o", shp, g.odtype), _stream(stream)), "nabla_attn_fwd")


def vt_shape(g: Geometry) -> Tuple[int, ...]:
    """Shape of the V^T operand layout [B, heads, nb, d, 64]."""
    return (g.batch, g.heads, g.nb, g.head_dim, 64)


def nabla_transpose_v(g: Geometry, v, vt, stream=None) -> None:
    _check(_lib.load().nabla_transpose_v(
        ctypes.byref(g.c()), _ptr(v, "v", g.tensor_shape(), g.dtype),
        _ptr(vt, "vt", vt_shape(g), g.dtype), _stream(stream)), "nabla_transpose_v")


def nabla_attn_fwd_vt(g: Geometry, q, k, vt, row_ptr, col_idx, scale: float, o,
                      stream=None) -> None:
    shp = g.tensor_shape()
    bh = g.batch * g.heads
    _check(_lib.load().nabla_attn_fwd_vt(
        ctypes.byref(g.c()), _ptr(q, "q", shp, g.dtype), _ptr(k, "k", shp, g.dtype),
        _ptr(vt, "vt", vt_shape(g), g.dtype),
        _ptr(row_ptr, "row_ptr", (bh, g.nb + 1), torch.int32),
        _ptr(col_idx, "col_idx", (bh, g.nb * g.nb), torch.int32), float(scale),
        _ptr(o, "o", shp, g.odtype), _stream(stream)), "nabla_attn_fwd_vt")


def qkv_shape(g: Geometry) -> Tuple[int, ...]:
    """Shape of a fused QKV projection output in the blocked token order,
    [B, nb * 64, 3, heads, d]."""
    return (g.batch, g.nb * 64, 3, g.heads, g.head_dim)


def nabla_qkv_split(g: Geometry, qkv, q, k, vt, qbar, kbar, stream=None) -> None:
    shp = g.tensor_shape(LAYOUT_BLOCKED)
    _check(_lib.load().nabla_qkv_split(
        ctypes.byref(g.c()), _ptr(qkv, "qkv", qkv_shape(g), g.dtype),
        _ptr(q, "q", shp, g.dtype), _ptr(k, "k", shp, g.dtype),
        _ptr(vt, "vt", vt_shape(g), g.dtype), _ptr(qbar, "qbar", qbar_shape(g), torch.float32),
        _ptr(kbar, "kbar", kbar_shape(g), KBAR_DTYPE), _stream(stream)), "nabla_qkv_split")


def nabla_dense_attn_fwd(g: Geometry, q, k, vt, scale: float, o, lse=None,
                         stream=None) -> None:
    shp = g.tensor_shape()
    _check(_lib.load().nabla_dense_attn_fwd(
        ctypes.byref(g.c()), _ptr(q, "q", shp, g.dtype), _ptr(k, "k", shp, g.dtype),
        _ptr(vt, "vt", vt_shape(g), g.dtype), float(scale), _ptr(o, "o", shp, g.odtype),
        _ptr(lse, "lse", lse_shape(g), torch.float32), _stream(stream)), "nabla_dense_attn_fwd")


def lse_shape(g: Geometry) -> Tuple[int, ...]:
    """Shape of the per-query float32 lse / delta arrays [B, heads, nb, 64]."""
    return (g.batch, g.heads, g.nb, 64)


def nabla_attn_fwd_lse(g: Geometry, q, k, v, row_ptr, col_idx, scale: float, o, lse,
                       stream=None) -> None:
    shp = g.tensor_shape()
    bh = g.batch * g.heads
    _check(_lib.load().nabla_attn_fwd_lse(
        ctypes.byref(g.c()), _ptr(q, "q", shp, g.dtype), _ptr(k, "k", shp, g.dtype),
        _ptr(v, "v", shp, g.dtype), _ptr(row_ptr, "row_ptr", (bh, g.nb + 1), torch.int32),
        _ptr(col_idx, "col_idx", (bh, g.nb * g.nb), torch.int32), float(scale),
        _ptr(o, "o", shp, g.odtype), _ptr(lse, "lse", lse_shape(g), torch.float32),
        _stream(stream)), "nabla_attn_fwd_lse")


def nabla_attn_fwd_vt_lse(g: Geometry, q, k, vt, row_ptr, col_idx, scale: float, o, lse,
                          stream=None) -> None:
    shp = g.tensor_shape()
    bh = g.batch * g.heads
    _check(_lib.load().nabla_attn_fwd_vt_lse(
        ctypes.byref(g.c()), _ptr(q, "q", shp, g.dtype), _ptr(k, "k", shp, g.dtype),
        _ptr(vt, "vt", vt_shape(g), g.dtype),
        _ptr(row_ptr, "row_ptr", (bh, g.nb + 1), torch.int32),
        _ptr(col_idx, "col_idx", (bh, g.nb * g.nb), torch.int32), float(scale),
        _ptr(o, "o", shp, g.odtype), _ptr(lse, "lse", lse_shape(g), torch.float32),
        _stream(stream)), "nabla_attn_fwd_vt_lse")


def nabla_mask_transpose(g: Geometry, mask_bits, mask_bits_t, row_count_t, stream=None) -> None:
    bshape = (g.batch, g.heads, g.nb, g.nw)
    _check(_lib.load().nabla_mask_transpose(
        ctypes.byref(g.c()), _ptr(mask_bits, "mask_bits", bshape, torch.int32),
        _ptr(mask_bits_t, "mask_bits_t", bshape, torch.int32),
        _ptr(row_count_t, "row_count_t", (g.batch, g.heads, g.nb), torch.int32),
        _stream(stream)), "nabla_mask_transpose")


def nabla_attn_bwd_dq(g: Geometry, q, k, v, o, dout, lse, row_ptr, col_idx, scale: float, dq,
                      delta, stream=None) -> None:
    shp = g.tensor_shape()
    bh = g.batch * g.heads
    _check(_lib.load().nabla_attn_bwd_dq(
        ctypes.byref(g.c()), _ptr(q, "q", shp, g.dtype), _ptr(k, "k", shp, g.dtype),
        _ptr(v, "v", shp, g.dtype), _ptr(o, "o", shp, g.dtype), _ptr(dout, "dout", shp, g.dtype),
        _ptr(lse, "lse", lse_shape(g), torch.float32),
        _ptr(row_ptr, "row_ptr", (bh, g.nb + 1), torch.int32),
        _ptr(col_idx, "col_idx", (bh, g.nb * g.nb), torch.int32), float(scale),
        _ptr(dq, "dq", shp, g.dtype), _ptr(delta, "delta", lse_shape(g), torch.float32),
        _stream(stream)), "nabla_attn_bwd_dq")


def nabla_attn_bwd_dkdv(g: Geometry, q, k, v, dout, lse, delta, col_ptr, row_idx, scale: float,
                        dk, dv, stream=None) -> None:
    shp = g.tensor_shape()
    bh = g.batch * g.heads
    _check(_lib.load().nabla_attn_bwd_dkdv(
        ctypes.byref(g.c()), _ptr(q, "q", shp, g.dtype), _ptr(k, "k", shp, g.dtype),
        _ptr(v, "v", shp, g.dtype), _ptr(dout, "dout", shp, g.dtype),
        _ptr(lse, "lse", lse_shape(g), torch.float32),
        _ptr(delta, "delta", lse_shape(g), torch.float32),
        _ptr(col_ptr, "col_ptr", (bh, g.nb + 1), torch.int32),
        _ptr(row_idx, "row_idx", (bh, g.nb * g.nb), torch.int32), float(scale),
        _ptr(dk, "dk", shp, g.dtype), _ptr(dv, "dv", shp, g.dtype), _stream(stream)),
        "nabla_attn_bwd_dkdv")


def nabla_forward_workspace_size(g: Geometry) -> Tuple[int, Tuple[int, ...]]:
    size = ctypes.c_size_t(0)
    offs = (ctypes.c_size_t * _lib.WORKSPACE_PARTS)()
    _check(_lib.load().nabla_forward_workspace_size(ctypes.byref(g.c()), ctypes.byref(size),
                                                    offs), "nabla_forward_workspace_size")
    return size.value, tuple(offs)


def nabla_forward(g: Geometry, q, k, v, thr: float, sta, scale: float, o, workspace,
                  stream=None) -> None:
    shp = g.tensor_shape()
    _check(_lib.load().nabla_forward(
        ctypes.byref(g.c()), _ptr(q, "q", shp, g.dtype), _ptr(k, "k", shp, g.dtype),
        _ptr(v, "v", shp, g.dtype), float(thr), _sta(sta), float(scale),
        _ptr(o, "o", shp, g.odtype), _ptr(workspace, "workspace", None, torch.uint8),
        workspace.numel(), _stream(stream)), "nabla_forward")


def nabla_forward_noalloc(g: Geometry, q, k, v, thr: float, sta, scale: float, o,
                          stream=None) -> None:
    shp = g.tensor_shape()
    _check(_lib.load().nabla_forward_noalloc(
        ctypes.byref(g.c()), _ptr(q, "q", shp, g.dtype), _ptr(k, "k", shp, g.dtype),
        _ptr(v, "v", shp, g.dtype), float(thr), _sta(sta), float(scale),
        _ptr(o, "o", shp, g.odtype), _stream(stream)), "nabla_forward_noalloc")


# ---------------------------------------------------------------------------
# convenience: allocate outputs/workspace with torch and run the whole call
# ---------------------------------------------------------------------------
@dataclass
class ForwardResult:
    o: torch.Tensor
    qbar: torch.Tensor
    kbar: torch.Tensor
    mask_bits: torch.Tensor
    row_count: torch.Tensor
    row_ptr: torch.Tensor
    col_idx: torch.Tensor


def forward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, thr: float,
            sta: Optional[Sequence[int]] = (3, 3, 3), scale: Optional[float] = None,
            layout: int = LAYOUT_THW, T: Optional[int] = None, H: Optional[int] = None,
            W: Optional[int] = None, out_dtype: Optional[torch.dtype] = None,
            stream=None) -> ForwardResult:
    """One NABLA attention call.  THW tensors carry T, H, W in their shape;
    BLOCKED tensors need T, H, W passed explicitly.  ``out_dtype`` (default:
    the input dtype) may be float32 for bf16 inputs."""
    if layout == LAYOUT_THW:
        B, h, T, H, W, d = q.shape
    else:
        B, h, _, _, d = q.shape
        if T is None or H is None or W is None:
            raise ValueError("T, H, W are required for the blocked layout")
    g = Geometry(B, h, T, H, W, d, q.dtype, layout, out_dtype=out_dtype)
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    size, offs = nabla_forward_workspace_size(g)
    ws = torch.empty(size, dtype=torch.uint8, device=q.device)
    o = torch.empty(q.shape, dtype=g.odtype, device=q.device)
    nabla_forward(g, q, k, v, thr, sta, scale, o, ws, stream)

    def part(i, dtype, shape):
        n = math.prod(shape)
        esz = torch.tensor([], dtype=dtype).element_size()
        return ws[offs[i]:offs[i] + n * esz].view(dtype).view(shape)

    bh = B * h
    return ForwardResult(
        o=o,
        qbar=part(0, torch.float32, (B, h, g.nb, d)),
        kbar=part(1, KBAR_DTYPE, kbar_shape(g)),
        mask_bits=part(2, torch.int32, (B, h, g.nb, g.nw)),
        row_count=part(3, torch.int32, (B, h, g.nb)),
        row_ptr=part(4, torch.int32, (bh, g.nb + 1)),
        col_idx=part(5, torch.int32, (bh, g.nb * g.nb)),
    )


@dataclass
class BackwardResult:
    dq: torch.Tensor
    dk: torch.Tensor
    dv: torch.Tensor
    delta: torch.Tensor
    col_ptr: torch.Tensor
    row_idx: torch.Tensor


def backward(g: Geometry, q, k, v, o, lse, dout, mask_bits, row_ptr, col_idx,
             scale: Optional[float] = None, stream=None) -> BackwardResult:
    """Gradients of one call with its mask held fixed, from the forward's o,
    lse (nabla_attn_fwd_lse / _vt_lse), mask bits and lists: transposed mask
    -> key-major lists -> dQ (and D) -> dK, dV, all on one stream."""
    scale = 1.0 / math.sqrt(g.head_dim) if scale is None else scale
    dev = q.device
    bh = g.batch * g.heads
    bits_t = torch.empty_like(mask_bits)
    cnt_t = torch.empty((g.batch, g.heads, g.nb), dtype=torch.int32, device=dev)
    col_ptr = torch.empty((bh, g.nb + 1), dtype=torch.int32, device=dev)
    row_idx = torch.empty((bh, g.nb * g.nb), dtype=torch.int32, device=dev)
    nabla_mask_transpose(g, mask_bits, bits_t, cnt_t, stream)
    nabla_compact(g, bits_t, cnt_t, col_ptr, row_idx, stream)
    dq, dk, dv = (torch.empty_like(q) for _ in range(3))
    delta = torch.empty(lse_shape(g), dtype=torch.float32, device=dev)
    nabla_attn_bwd_dq(g, q, k, v, o, dout, lse, row_ptr, col_idx, scale, dq, delta, stream)
    nabla_attn_bwd_dkdv(g, q, k, v, dout, lse, delta, col_ptr, row_idx, scale, dk, dv, stream)
    return BackwardResult(dq, dk, dv, delta, col_ptr, row_idx)


# ---------------------------------------------------------------------------
# autograd: the attention call as a differentiable torch op (mask held fixed)
# ---------------------------------------------------------------------------
class NablaAttention(torch.autograd.Function):
    """o = NABLA attention of THW tensors q, k, v [B, heads, T, H, W, d]
    (bf16 or float32, contiguous).  Forward: nabla_mask_build (pooling, mask,
    lists) and the attention with its log-sum-exp; backward: the
    gradient calls of ``backward`` with the forward's mask held fixed (the
    mask is a threshold, so thr and sta get no gradient)."""

    @staticmethod
    def forward(ctx, q, k, v, thr, sta, scale):
        B, h, T, H, W, d = q.shape
        q, k, v = q.contiguous(), k.contiguous(), v.contiguous()
        g = Geometry(B, h, T, H, W, d, q.dtype)
        scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
        dev = q.device
        nb = g.nb
        qbar = torch.empty(qbar_shape(g), dtype=torch.float32, device=dev)
        kbar = torch.empty(kbar_shape(g), dtype=KBAR_DTYPE, device=dev)
        bits = torch.empty((B, h, nb, g.nw), dtype=torch.int32, device=dev)
        cnt = torch.empty((B, h, nb), dtype=torch.int32, device=dev)
        rp = torch.empty((B * h, nb + 1), dtype=torch.int32, device=dev)
        ci = torch.empty((B * h, nb * nb), dtype=torch.int32, device=dev)
        o = torch.empty_like(q)
        lse = torch.empty(lse_shape(g), dtype=torch.float32, device=dev)
        nabla_mask_build(g, q, k, thr, sta, qbar, kbar, bits, cnt, None, rp, ci)
        if q.dtype == torch.bfloat16:
            vt = torch.empty(vt_shape(g), dtype=q.dtype, device=dev)
            nabla_transpose_v(g, v, vt)
            nabla_attn_fwd_vt_lse(g, q, k, vt, rp, ci, scale, o, lse)
        else:
            nabla_attn_fwd_lse(g, q, k, v, rp, ci, scale, o, lse)
        ctx.save_for_backward(q, k, v, o, lse, bits, rp, ci)
        ctx.geom, ctx.scale = g, scale
        return o

    @staticmethod
    def backward(ctx, dout):
        q, k, v, o, lse, bits, rp, ci = ctx.saved_tensors
        res = backward(ctx.geom, q, k, v, o, lse, dout.contiguous().to(q.dtype), bits, rp, ci,
                       ctx.scale)
        return res.dq, res.dk, res.dv, None, None, None


def nabla_attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, thr: float,
                    sta: Optional[Sequence[int]] = (3, 3, 3),
                    scale: Optional[float] = None) -> torch.Tensor:
    """Differentiable NABLA attention on THW tensors (see NablaAttention)."""
    return NablaAttention.apply(q, k, v, thr, sta, scale)


__all__ += ["NablaAttention", "nabla_attention"]
