"""Guarded W8A8 linear layer for AMD Instinct MI355X (gfx950).

Thin Python binding over ``libw8a8.so`` (C ABI in ``include/w8a8.h``).  Every
step of the path runs in the library's HIP kernels; this module only checks
tensor shapes/dtypes, allocates outputs with torch (device memory) and passes
pointers plus torch's current HIP stream.  There is no CPU fallback: if the
native library is missing, every call raises.

Method: TurboT2VA's W8A8 linear (智猩猩 article, section 01.3 "量化策略") and
padded-text compaction (same section, closing paragraph; paperlayer.ai
summary, section "C. Fused Multimodal Transformer Operations").
"""
from __future__ import annotations

import contextlib
import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libw8a8.so")

OK, EINVAL, EUNSUPPORTED, EHIP, ESCRATCH = 0, -1, -2, -3, -4
OUT_BF16, OUT_I32 = 0, 1
ACT_NONE, ACT_GELU_TANH = 0, 1
PATH_INT8, PATH_BF16 = 0, 1
NORM_LAYER, NORM_RMS = 0, 1
MAX_K = 131072
NOALLOC_SCRATCH_BYTES = 64 << 20

EXPORTS = ("w8a8_quantize_rows", "w8a8_quantize_blocks", "w8a8_gelu_quantize_rows", "w8a8_gelu_bf16", "w8a8_gemm", "w8a8_linear", "w8a8_linear_bf16",
           "compact_padded_rows", "w8a8_compact_quantize_rows", "w8a8_guard", "w8a8_linear_workspace_bytes",
           "w8a8_status_str", "w8a8_norm_mod_bf16", "w8a8_norm_mod_quantize_rows",
           "w8a8_linear_noalloc", "w8a8_gemm_splitk", "w8a8_gemm_splitk_workspace_bytes")

_lib = None


class W8A8Error(RuntimeError):
    def __init__(self, fn, status):
        super().__init__(f"{fn}: {status_str(status)} ({status})")
        self.status = status


def lib():
    """The loaded native library (ctypes.CDLL).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"native library {LIB_PATH} is missing; build it with "
                           "`python -m int8_w8a8_gemm_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    P, I64, I, SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
    L.w8a8_quantize_rows.argtypes = [P, I64, I64, P, P, P]
    L.w8a8_quantize_blocks.argtypes = [P, I64, I64, I64, I64, I64, P, P, P]
    L.w8a8_gelu_quantize_rows.argtypes = [P, I64, I64, P, P, P]
    L.w8a8_gelu_bf16.argtypes = [P, I64, P, P]
    L.w8a8_norm_mod_bf16.argtypes = [P, I64, I64, P, P, I64, I, ctypes.c_double, P, P]
    L.w8a8_norm_mod_quantize_rows.argtypes = [P, I64, I64, P, P, I64, I, ctypes.c_double, P, P, P]
    L.w8a8_gemm.argtypes = [P, P, I64, P, P, I64, I64, P, I, I, P, P]
    L.w8a8_linear.argtypes = [P, I64, I64, I64, P, P, P, P, I, P, P, SZ, P, P]
    L.w8a8_linear_bf16.argtypes = [P, I64, I64, P, I64, P, I, P, P]
    L.w8a8_linear_noalloc.argtypes = [P, I64, I64, I64, P, P, P, P, I, P, P, P]
    L.w8a8_gemm_splitk.argtypes = [P, P, I64, P, P, I64, I64, P, I, I, P, P, SZ, P]
    L.w8a8_gemm_splitk.restype = I
    L.w8a8_gemm_splitk_workspace_bytes.argtypes = [I64, I64, I64]
    L.w8a8_gemm_splitk_workspace_bytes.restype = SZ
    L.compact_padded_rows.argtypes = [P, P, I64, I64, I64, P, P, P, P]
    L.w8a8_compact_quantize_rows.argtypes = [P, P, I64, I64, I64, P, P, P, P, P]
    L.w8a8_guard.argtypes = [I64, I64]
    L.w8a8_linear_workspace_bytes.argtypes = [I64, I64]
    L.w8a8_linear_workspace_bytes.restype = SZ
    L.w8a8_status_str.argtypes = [I]
    L.w8a8_status_str.restype = ctypes.c_char_p
    for name in ("w8a8_quantize_rows", "w8a8_gelu_quantize_rows", "w8a8_gemm", "w8a8_linear", "w8a8_linear_bf16",
                 "compact_padded_rows", "w8a8_guard", "w8a8_linear_noalloc"):
        getattr(L, name).restype = I
    _lib = L
    return L


# ---------------------------------------------------------------------------
# host-only helpers
# ---------------------------------------------------------------------------

def guard(N: int, K: int) -> bool:
    """True if the INT8 GEMM serves (N, K); otherwise the linear runs in BF16."""
    return bool(lib().w8a8_guard(int(N), int(K)))


def linear_workspace_bytes(M: int, K: int) -> int:
    return int(lib().w8a8_linear_workspace_bytes(int(M), int(K)))


def status_str(status: int) -> str:
    return lib().w8a8_status_str(int(status)).decode()


# ---------------------------------------------------------------------------
# marshalling
# ---------------------------------------------------------------------------

def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _on(stream=None):
    """Context for the allocations of a call that runs on `stream`: torch's caching
    allocator ties a block to the stream that was current when it was allocated, so
    temporaries (the linear's workspace, the normed layer's codes) and default outputs
    are allocated with `stream` current.  Otherwise, once dropped, a temporary could be
    handed to work on another stream while the kernels on `stream` still read it."""
    return torch.cuda.stream(stream) if stream is not None else contextlib.nullcontext()


def _p(t: Optional[torch.Tensor]):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _need(t, name, dtype, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return t


def _check(fn, status):
    if status != OK:
        raise W8A8Error(fn, status)


# ---------------------------------------------------------------------------
# the four calls of the path (+ the BF16 fallback on its own)
# ---------------------------------------------------------------------------

def quantize_rows(x: torch.Tensor, q: Optional[torch.Tensor] = None,
                  scale: Optional[torch.Tensor] = None, stream=None):
    """Per-row symmetric INT8 quantisation: x bf16 [R, C] -> (q int8 [R, C], scale fp32 [R])."""
    _need(x, "x", torch.bfloat16)
    if x.dim() != 2:
        raise ValueError("x must be 2-D")
    R, C = x.shape
    with _on(stream):
        q = q if q is not None else torch.empty((R, C), dtype=torch.int8, device=x.device)
        scale = scale if scale is not None else torch.empty((R,), dtype=torch.float32,
                                                            device=x.device)
    _need(q, "q", torch.int8, (R, C))
    _need(scale, "scale", torch.float32, (R,))
    _check("w8a8_quantize_rows",
           lib().w8a8_quantize_rows(_p(x), R, C, _p(q), _p(scale), _stream(stream)))
    return q, scale


def quantize_blocks(x: torch.Tensor, batch: int, heads: int, block: int,
                    q: Optional[torch.Tensor] = None, scale: Optional[torch.Tensor] = None,
                    stream=None):
    """Per-block symmetric INT8 quantisation of attention Q / K: x bf16 token rows
    [batch * seq, heads * head_dim] (or [batch, seq, heads * head_dim]); one scale per
    `block` consecutive tokens of one sample and one head.  Returns (q int8 of x's shape,
    scale fp32 [batch, ceil(seq / block), heads])."""
    _need(x, "x", torch.bfloat16)
    if x.dim() not in (2, 3):
        raise ValueError("x must be 2-D or 3-D")
    rows, C = x.reshape(-1, x.shape[-1]).shape
    if batch <= 0 or heads <= 0 or block <= 0 or rows % batch or C % heads:
        raise ValueError("batch, heads and block must be positive and divide the shape")
    S, D = rows // batch, C // heads
    nblk = -(-S // block)
    with _on(stream):
        q = q if q is not None else torch.empty(x.shape, dtype=torch.int8, device=x.device)
        scale = scale if scale is not None else torch.empty((batch, nblk, heads),
                                                            dtype=torch.float32, device=x.device)
    _need(q, "q", torch.int8, tuple(x.shape))
    _need(scale, "scale", torch.float32, (batch, nblk, heads))
    _check("w8a8_quantize_blocks",
           lib().w8a8_quantize_blocks(_p(x), batch, S, heads, D, block, _p(q), _p(scale),
                                      _stream(stream)))
    return q, scale


def gelu_quantize_rows(y: torch.Tensor, q: Optional[torch.Tensor] = None,
                       scale: Optional[torch.Tensor] = None, stream=None):
    """h = GELU-tanh(y) (rounded to bf16 as the GELU epilogue), then per-row INT8 quantisation of h:
    y bf16 [R, C] -> (q int8 [R, C], scale fp32 [R]).  h is not materialised."""
    _need(y, "y", torch.bfloat16)
    if y.dim() != 2:
        raise ValueError("y must be 2-D")
    R, C = y.shape
    with _on(stream):
        q = q if q is not None else torch.empty((R, C), dtype=torch.int8, device=y.device)
        scale = scale if scale is not None else torch.empty((R,), dtype=torch.float32,
                                                            device=y.device)
    _need(q, "q", torch.int8, (R, C))
    _need(scale, "scale", torch.float32, (R,))
    _check("w8a8_gelu_quantize_rows",
           lib().w8a8_gelu_quantize_rows(_p(y), R, C, _p(q), _p(scale), _stream(stream)))
    return q, scale


def _norm_mod_args(x, shift, scale, rows_per_cond):
    _need(x, "x", torch.bfloat16)
    if x.dim() != 2:
        raise ValueError("x must be 2-D")
    R, C = x.shape
    rpc = int(rows_per_cond) if rows_per_cond else max(R, 1)
    G = -(-R // rpc) if R else 0
    for t, n in ((shift, "shift"), (scale, "scale")):
        if t is not None:
            _need(t, n, torch.bfloat16)
            if t.dim() != 2 or t.shape[1] != C or t.shape[0] < G:
                raise ValueError(f"{n} must be [>= {G}, {C}]")
    return R, C, rpc


def norm_mod_bf16(x: torch.Tensor, shift: Optional[torch.Tensor] = None,
                  scale: Optional[torch.Tensor] = None, rows_per_cond: Optional[int] = None,
                  norm: int = NORM_LAYER, eps: float = 1e-6, y: Optional[torch.Tensor] = None,
                  stream=None):
    """Normalisation (LayerNorm without affine, or RMSNorm) and modulation
    z = y * (1 + scale[g]) + shift[g], g = row // rows_per_cond, of each row of
    x bf16 [R, C]; shift, scale bf16 [G, C] or None.  Returns bf16 [R, C]."""
    R, C, rpc = _norm_mod_args(x, shift, scale, rows_per_cond)
    with _on(stream):
        y = y if y is not None else torch.empty_like(x)
    _need(y, "y", torch.bfloat16, (R, C))
    _check("w8a8_norm_mod_bf16",
           lib().w8a8_norm_mod_bf16(_p(x), R, C, _p(shift), _p(scale), rpc, int(norm), float(eps),
                                    _p(y), _stream(stream)))
    return y


def norm_mod_quantize_rows(x: torch.Tensor, shift: Optional[torch.Tensor] = None,
                           scale: Optional[torch.Tensor] = None,
                           rows_per_cond: Optional[int] = None, norm: int = NORM_LAYER,
                           eps: float = 1e-6, q: Optional[torch.Tensor] = None,
                           qscale: Optional[torch.Tensor] = None, stream=None):
    """norm_mod_bf16 fused with the per-row INT8 quantisation of its rows:
    returns (q int8 [R, C], qscale fp32 [R]); the bf16 rows are not written."""
    R, C, rpc = _norm_mod_args(x, shift, scale, rows_per_cond)
    with _on(stream):
        q = q if q is not None else torch.empty((R, C), dtype=torch.int8, device=x.device)
        qscale = qscale if qscale is not None else torch.empty((R,), dtype=torch.float32,
                                                               device=x.device)
    _need(q, "q", torch.int8, (R, C))
    _need(qscale, "qscale", torch.float32, (R,))
    _check("w8a8_norm_mod_quantize_rows",
           lib().w8a8_norm_mod_quantize_rows(_p(x), R, C, _p(shift), _p(scale), rpc, int(norm),
                                             float(eps), _p(q), _p(qscale), _stream(stream)))
    return q, qscale


def gelu_bf16(x: torch.Tensor, y: Optional[torch.Tensor] = None, stream=None):
    """Elementwise GELU-tanh on bf16: y = g(x) rounded to bf16, as the GELU epilogue."""
    _need(x, "x", torch.bfloat16)
    with _on(stream):
        y = y if y is not None else torch.empty_like(x)
    _need(y, "y", torch.bfloat16, tuple(x.shape))
    _check("w8a8_gelu_bf16", lib().w8a8_gelu_bf16(_p(x), x.numel(), _p(y), _stream(stream)))
    return y


def gemm(qa, sa, qw, sw, bias=None, act=ACT_NONE, out_kind=OUT_BF16, out=None, stream=None):
    """INT8 GEMM, INT32 accumulation, epilogue once after accumulation.
    qa int8 [M, K], sa fp32 [M], qw int8 [N, K], sw fp32 [N], bias bf16 [N] or None.
    Returns bf16 [M, N] (OUT_BF16) or int32 [M, N] (OUT_I32)."""
    _need(qa, "qa", torch.int8)
    _need(qw, "qw", torch.int8)
    M, K = qa.shape
    N = qw.shape[0]
    if qw.shape[1] != K:
        raise ValueError("qa and qw disagree on K")
    if out_kind == OUT_BF16:
        _need(sa, "sa", torch.float32, (M,))
        _need(sw, "sw", torch.float32, (N,))
    if bias is not None:
        _need(bias, "bias", torch.bfloat16, (N,))
    odt = torch.int32 if out_kind == OUT_I32 else torch.bfloat16
    with _on(stream):
        out = out if out is not None else torch.empty((M, N), dtype=odt, device=qa.device)
    _need(out, "out", odt, (M, N))
    _check("w8a8_gemm", lib().w8a8_gemm(_p(qa), _p(sa), M, _p(qw), _p(sw), N, K, _p(bias),
                                        int(act), int(out_kind), _p(out), _stream(stream)))
    return out


def gemm_splitk_workspace_bytes(M: int, N: int, K: int) -> int:
    """Workspace of gemm_splitk for (M, N, K); 0 when the shape is not split."""
    return int(lib().w8a8_gemm_splitk_workspace_bytes(int(M), int(N), int(K)))


def gemm_splitk(qa, sa, qw, sw, bias=None, act=ACT_NONE, out_kind=OUT_BF16, out=None,
                workspace=None, stream=None):
    """gemm with the K loop split across workgroups where the shape leaves most compute
    units idle (same result, bit for bit).  workspace: uint8 device tensor of at least
    gemm_splitk_workspace_bytes(M, N, K) bytes, allocated here when None."""
    _need(qa, "qa", torch.int8)
    _need(qw, "qw", torch.int8)
    M, K = qa.shape
    N = qw.shape[0]
    if qw.shape[1] != K:
        raise ValueError("qa and qw disagree on K")
    if out_kind == OUT_BF16:
        _need(sa, "sa", torch.float32, (M,))
        _need(sw, "sw", torch.float32, (N,))
    if bias is not None:
        _need(bias, "bias", torch.bfloat16, (N,))
    odt = torch.int32 if out_kind == OUT_I32 else torch.bfloat16
    need = gemm_splitk_workspace_bytes(M, N, K)
    with _on(stream):
        out = out if out is not None else torch.empty((M, N), dtype=odt, device=qa.device)
        if workspace is None and need > 0:
            workspace = torch.empty((need,), dtype=torch.uint8, device=qa.device)
    _need(out, "out", odt, (M, N))
    if workspace is not None:
        _need(workspace, "workspace", torch.uint8)
    _check("w8a8_gemm_splitk", lib().w8a8_gemm_splitk(
        _p(qa), _p(sa), M, _p(qw), _p(sw), N, K, _p(bias), int(act), int(out_kind), _p(out),
        _p(workspace), workspace.numel() if workspace is not None else 0, _stream(stream)))
    return out


def linear_bf16(x, w, bias=None, act=ACT_NONE, y=None, stream=None):
    """Native BF16 linear (the fallback path): y = bf16(x w^T + b), fp32 accumulation."""
    _need(x, "x", torch.bfloat16)
    _need(w, "w", torch.bfloat16)
    M, K = x.shape
    N = w.shape[0]
    if w.shape[1] != K:
        raise ValueError("x and w disagree on K")
    if bias is not None:
        _need(bias, "bias", torch.bfloat16, (N,))
    with _on(stream):
        y = y if y is not None else torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    _need(y, "y", torch.bfloat16, (M, N))
    _check("w8a8_linear_bf16", lib().w8a8_linear_bf16(_p(x), M, K, _p(w), N, _p(bias), int(act),
                                                      _p(y), _stream(stream)))
    return y


def linear(x, N, qw=None, sw=None, w=None, bias=None, act=ACT_NONE, y=None, workspace=None,
           stream=None):
    """The guarded W8A8 linear.  Returns (y bf16 [M, N], path) with path PATH_INT8 or PATH_BF16.
    The INT8 path needs (qw, sw) prepared with quantize_rows(W); the BF16 path needs w."""
    _need(x, "x", torch.bfloat16)
    M, K = x.shape
    if qw is not None:
        _need(qw, "qw", torch.int8, (N, K))
    if sw is not None:
        _need(sw, "sw", torch.float32, (N,))
    if w is not None:
        _need(w, "w", torch.bfloat16, (N, K))
    if bias is not None:
        _need(bias, "bias", torch.bfloat16, (N,))
    ws_bytes = linear_workspace_bytes(M, K) if guard(N, K) else 0
    with _on(stream):
        y = y if y is not None else torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
        if workspace is None and ws_bytes > 0:
            workspace = torch.empty((ws_bytes,), dtype=torch.uint8, device=x.device)
    _need(y, "y", torch.bfloat16, (M, N))
    if workspace is not None:
        _need(workspace, "workspace", torch.uint8)
    path = ctypes.c_int(-1)
    _check("w8a8_linear", lib().w8a8_linear(
        _p(x), M, K, N, _p(qw), _p(sw), _p(w), _p(bias), int(act), _p(y), _p(workspace),
        workspace.numel() if workspace is not None else 0, ctypes.byref(path), _stream(stream)))
    return y, path.value


def linear_noalloc(x, N, qw=None, sw=None, w=None, bias=None, act=ACT_NONE, y=None, stream=None):
    """The guarded W8A8 linear with the INT8 path's workspace in the library's static
    device scratch (w8a8_linear_noalloc: nothing is allocated by the call).  Returns
    (y bf16 [M, N], path).  Calls that overlap on one GPU race on the scratch."""
    _need(x, "x", torch.bfloat16)
    M, K = x.shape
    if qw is not None:
        _need(qw, "qw", torch.int8, (N, K))
    if sw is not None:
        _need(sw, "sw", torch.float32, (N,))
    if w is not None:
        _need(w, "w", torch.bfloat16, (N, K))
    if bias is not None:
        _need(bias, "bias", torch.bfloat16, (N,))
    with _on(stream):
        y = y if y is not None else torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    _need(y, "y", torch.bfloat16, (M, N))
    path = ctypes.c_int(-1)
    _check("w8a8_linear_noalloc", lib().w8a8_linear_noalloc(
        _p(x), M, K, N, _p(qw), _p(sw), _p(w), _p(bias), int(act), _p(y), ctypes.byref(path),
        _stream(stream)))
    return y, path.value


def compact_padded_rows(x, mask, out=None, src_row=None, count=None, stream=None):
    """Padded-row compaction: x bf16 [B, L, D], mask uint8 [B, L] ->
    (out bf16 [B*L, D] with the first count rows valid, src_row int32 [B*L], count int32 [1]).
    count stays on the device; read it with count.item() (a sync) when needed."""
    _need(x, "x", torch.bfloat16)
    _need(mask, "mask", torch.uint8)
    B, L, D = x.shape
    if tuple(mask.shape) != (B, L):
        raise ValueError("mask must be [B, L]")
    dev = x.device
    with _on(stream):
        out = out if out is not None else torch.empty((B * L, D), dtype=torch.bfloat16, device=dev)
        src_row = src_row if src_row is not None else torch.empty((B * L,), dtype=torch.int32,
                                                                  device=dev)
        count = count if count is not None else torch.empty((1,), dtype=torch.int32, device=dev)
    _need(out, "out", torch.bfloat16, (B * L, D))
    _need(src_row, "src_row", torch.int32, (B * L,))
    _need(count, "count", torch.int32, (1,))
    _check("compact_padded_rows", lib().compact_padded_rows(
        _p(x), _p(mask), B, L, D, _p(out), _p(src_row), _p(count), _stream(stream)))
    return out, src_row, count


def compact_quantize_rows(x, mask, q=None, scale=None, src_row=None, count=None, stream=None):
    """Compaction fused with per-row INT8 quantisation: x bf16 [B, L, D], mask uint8
    [B, L] -> (q int8 [B*L, D], scale fp32 [B*L], src_row int32 [B*L], count int32 [1]),
    the first count rows valid.  count stays on the device."""
    _need(x, "x", torch.bfloat16)
    _need(mask, "mask", torch.uint8)
    B, L, D = x.shape
    if tuple(mask.shape) != (B, L):
        raise ValueError("mask must be [B, L]")
    dev = x.device
    with _on(stream):
        q = q if q is not None else torch.empty((B * L, D), dtype=torch.int8, device=dev)
        scale = scale if scale is not None else torch.empty((B * L,), dtype=torch.float32,
                                                            device=dev)
        src_row = src_row if src_row is not None else torch.empty((B * L,), dtype=torch.int32,
                                                                  device=dev)
        count = count if count is not None else torch.empty((1,), dtype=torch.int32, device=dev)
    _need(q, "q", torch.int8, (B * L, D))
    _need(scale, "scale", torch.float32, (B * L,))
    _need(src_row, "src_row", torch.int32, (B * L,))
    _need(count, "count", torch.int32, (1,))
    _check("w8a8_compact_quantize_rows", lib().w8a8_compact_quantize_rows(
        _p(x), _p(mask), B, L, D, _p(q), _p(scale), _p(src_row), _p(count), _stream(stream)))
    return q, scale, src_row, count


@dataclass
class W8A8Linear:
    """A linear layer prepared once: the INT8 weight and its per-channel scales when
    the guard admits the shape (static weight quantisation), else the bf16 weight."""
    N: int
    K: int
    qw: Optional[torch.Tensor]
    sw: Optional[torch.Tensor]
    w: Optional[torch.Tensor]
    bias: Optional[torch.Tensor]
    act: int = ACT_NONE

    @classmethod
    def prepare(cls, w: torch.Tensor, bias: Optional[torch.Tensor] = None, act: int = ACT_NONE,
                keep_bf16: bool = False):
        N, K = w.shape
        if guard(N, K):
            qw, sw = quantize_rows(w)
            return cls(N, K, qw, sw, w if keep_bf16 else None, bias, act)
        return cls(N, K, None, None, w, bias, act)

    @property
    def path(self) -> int:
        return PATH_INT8 if self.qw is not None else PATH_BF16

    def __call__(self, x: torch.Tensor, y=None, workspace=None, stream=None):
        return linear(x, self.N, self.qw, self.sw, self.w, self.bias, self.act, y, workspace,
                      stream)[0]

    def normed(self, x: torch.Tensor, shift: Optional[torch.Tensor] = None,
               scale: Optional[torch.Tensor] = None, rows_per_cond: Optional[int] = None,
               norm: int = NORM_LAYER, eps: float = 1e-6, stream=None):
        """The layer applied to the normalised and modulated rows of x: on the INT8
        path the normalisation, modulation and activation quantisation are one
        kernel (norm_mod_quantize_rows) followed by the GEMM; on the BF16 path the
        bf16 rows of norm_mod_bf16 go through the native BF16 linear."""
        if self.qw is not None:
            q, s = norm_mod_quantize_rows(x, shift, scale, rows_per_cond, norm, eps, stream=stream)
            return gemm(q, s, self.qw, self.sw, self.bias, act=self.act, stream=stream)
        z = norm_mod_bf16(x, shift, scale, rows_per_cond, norm, eps, stream=stream)
        return linear_bf16(z, self.w, self.bias, act=self.act, stream=stream)
