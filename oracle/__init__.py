"""CPU oracle for the guarded W8A8 linear layer (TEST INFRASTRUCTURE ONLY).

The slow, plain reference implementation that the HIP library is checked
against.  Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline
leg of ``bench.py`` may import it; the product path (``int8_w8a8_gemm_amd``)
never does, and the two share no code.

All arithmetic lives in ``oracle.c`` (plain C, built with gcc); this module
only marshals numpy arrays.  bf16 tensors are passed as ``uint16`` bit
patterns.  Method source: TurboT2VA (智猩猩 article, section 01.3
"量化策略"; paperlayer.ai summary, section "C. Fused Multimodal Transformer
Operations").  Each function's docstring names the step it follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

ACT_NONE = 0
ACT_GELU_TANH = 1

_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so with gcc (no fast-math, no FP contraction)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        cmd = ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-std=c11", "-Wall",
               "-shared", "-fPIC", "-pthread", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build(force=False)
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    I = ctypes.c_int
    lib.oracle_quantize_rows.argtypes = [P, I64, I64, P, P, I]
    lib.oracle_quantize_blocks.argtypes = [P, I64, I64, I64, I64, I64, P, P, I]
    lib.oracle_gemm_i32.argtypes = [P, I64, P, I64, I64, P, I]
    lib.oracle_epilogue.argtypes = [P, P, I64, P, I64, P, I, P, I]
    lib.oracle_linear_bf16.argtypes = [P, I64, I64, P, I64, P, I, P, I]
    lib.oracle_w8a8_linear.argtypes = [P, I64, I64, P, I64, P, I, P, I]
    lib.oracle_compact_rows.argtypes = [P, P, I64, I64, I64, P, P, P]
    lib.oracle_norm_mod.argtypes = [P, I64, I64, P, P, I64, I, ctypes.c_double, P, I]
    lib.oracle_guard.argtypes = [I64, I64]
    lib.oracle_guard.restype = I
    lib.oracle_bf16_to_f32.argtypes = [ctypes.c_uint16]
    lib.oracle_bf16_to_f32.restype = ctypes.c_float
    lib.oracle_f32_to_bf16.argtypes = [ctypes.c_float]
    lib.oracle_f32_to_bf16.restype = ctypes.c_uint16
    lib.oracle_f64_to_bf16.argtypes = [ctypes.c_double]
    lib.oracle_f64_to_bf16.restype = ctypes.c_uint16
    lib.oracle_gelu_tanh_f64.argtypes = [ctypes.c_double]
    lib.oracle_gelu_tanh_f64.restype = ctypes.c_double
    lib.oracle_gelu_rows.argtypes = [P, I64, P, I]
    lib.oracle_gelu_bf16.argtypes = [ctypes.c_uint16]
    lib.oracle_gelu_bf16.restype = ctypes.c_uint16
    _lib = lib
    return lib


def usable_cores() -> int:
    """Cores this process may run on (its CPU affinity set)."""
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def default_threads() -> int:
    """Host threads the oracle uses by default: every core this process may run
    on, limited only where the host fixes the process's CPU share through
    OMP_NUM_THREADS (a host shared between GPUs does)."""
    n = usable_cores()
    try:
        share = int(os.environ.get("OMP_NUM_THREADS", "0"))
    except ValueError:
        share = 0
    if share > 0:
        n = min(n, share)
    return max(1, n)


def cpu_model() -> str:
    """The host CPU's model name (first "model name" line of /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.lower().startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:  # pragma: no cover
        pass
    return "unknown"


def _threads(nthreads):
    return int(nthreads) if nthreads else default_threads()


def _c(a, dtype):
    a = np.ascontiguousarray(a)
    if a.dtype != dtype:
        raise TypeError(f"expected {dtype}, got {a.dtype}")
    return a


def _ptr(a):
    return a.ctypes.data if a is not None else None


def _check(rc, name):
    if rc < 0:
        raise RuntimeError(f"{name} failed ({rc})")
    return rc


def quantize_rows(x_bf16: np.ndarray, nthreads=None):
    """Per-row symmetric INT8 quantisation (static per output channel for W,
    dynamic per token row for X; 智猩猩 article section 01.3).

    x_bf16: uint16 [R, C] bf16 bit patterns.  Returns (q int8 [R, C], s float32 [R]).
    """
    x = _c(x_bf16, np.uint16)
    R, C = x.shape
    q = np.empty((R, C), np.int8)
    s = np.empty((R,), np.float32)
    _check(_load().oracle_quantize_rows(_ptr(x), R, C, _ptr(q), _ptr(s), _threads(nthreads)),
           "oracle_quantize_rows")
    return q, s


def quantize_blocks(x_bf16: np.ndarray, batch: int, heads: int, block: int, nthreads=None):
    """Per-block symmetric INT8 quantisation of attention Query / Key (the
    attention paragraph of the 智猩猩 article, section 01.3, says Q and K are
    quantised to INT8; block size and layout are a reading).

    x_bf16: uint16 [batch * S, heads * D] token rows (or [batch, S, heads * D]);
    a block is `block` consecutive tokens of one sample and one head.  Returns
    (q int8 of x's shape, s float32 [batch, ceil(S / block), heads]).
    """
    x = _c(x_bf16, np.uint16)
    rows, C = x.reshape(-1, x.shape[-1]).shape
    assert rows % batch == 0 and C % heads == 0
    S, D = rows // batch, C // heads
    nblk = -(-S // block) if S else 0
    q = np.empty(x.shape, np.int8)
    s = np.empty((batch, nblk, heads), np.float32)
    _check(_load().oracle_quantize_blocks(_ptr(x), batch, S, heads, D, block, _ptr(q), _ptr(s),
                                          _threads(nthreads)), "oracle_quantize_blocks")
    return q, s


def gemm_i32(qa: np.ndarray, qw: np.ndarray, nthreads=None):
    """INT32 accumulation acc = qa . qw^T (智猩猩 article section 01.3)."""
    a = _c(qa, np.int8)
    w = _c(qw, np.int8)
    M, K = a.shape
    N, K2 = w.shape
    assert K == K2
    acc = np.empty((M, N), np.int32)
    _check(_load().oracle_gemm_i32(_ptr(a), M, _ptr(w), N, K, _ptr(acc), _threads(nthreads)),
           "oracle_gemm_i32")
    return acc


def epilogue(acc, sa, sw, bias=None, act=ACT_NONE, nthreads=None):
    """Scale and bias once after the full accumulation, bf16 output
    (智猩猩 article section 01.3); optional GELU-tanh on the bf16 result."""
    acc = _c(acc, np.int32)
    sa = _c(sa, np.float32)
    sw = _c(sw, np.float32)
    b = _c(bias, np.uint16) if bias is not None else None
    M, N = acc.shape
    y = np.empty((M, N), np.uint16)
    _check(_load().oracle_epilogue(_ptr(acc), _ptr(sa), M, _ptr(sw), N, _ptr(b), int(act),
                                   _ptr(y), _threads(nthreads)), "oracle_epilogue")
    return y


def linear_bf16(x, w, bias=None, act=ACT_NONE, nthreads=None):
    """Native BF16 linear used as the fallback (智猩猩 article section 01.3):
    float64 sum of exact products, rounded once to bf16."""
    x = _c(x, np.uint16)
    w = _c(w, np.uint16)
    b = _c(bias, np.uint16) if bias is not None else None
    M, K = x.shape
    N, K2 = w.shape
    assert K == K2
    y = np.empty((M, N), np.uint16)
    _check(_load().oracle_linear_bf16(_ptr(x), M, K, _ptr(w), N, _ptr(b), int(act), _ptr(y),
                                      _threads(nthreads)), "oracle_linear_bf16")
    return y


def w8a8_linear(x, w, bias=None, act=ACT_NONE, nthreads=None):
    """The guarded W8A8 linear: returns (y bf16 bits [M, N], path) with path 0 =
    INT8, 1 = BF16 fallback (智猩猩 article section 01.3; paperlayer.ai section C)."""
    x = _c(x, np.uint16)
    w = _c(w, np.uint16)
    b = _c(bias, np.uint16) if bias is not None else None
    M, K = x.shape
    N, K2 = w.shape
    assert K == K2
    y = np.empty((M, N), np.uint16)
    rc = _check(_load().oracle_w8a8_linear(_ptr(x), M, K, _ptr(w), N, _ptr(b), int(act), _ptr(y),
                                           _threads(nthreads)), "oracle_w8a8_linear")
    return y, rc


def gelu_rows(y, nthreads=None):
    """GELU-tanh of every bf16 element, each rounded once to bf16 (the activation
    between the FFN halves; float64 evaluation)."""
    y = _c(y, np.uint16)
    h = np.empty_like(y)
    _check(_load().oracle_gelu_rows(_ptr(y), y.size, _ptr(h), _threads(nthreads)), "oracle_gelu_rows")
    return h


def gelu_quantize_rows(y, nthreads=None):
    """Per-row INT8 quantisation of GELU-tanh(y): the down projection's input."""
    return quantize_rows(gelu_rows(y, nthreads), nthreads)


NORM_LAYER = 0
NORM_RMS = 1


def norm_mod_bf16(x, shift=None, scale=None, rows_per_cond=None, norm=NORM_LAYER, eps=1e-6,
                  nthreads=None):
    """Normalisation and modulation of each row, the fused operators ahead of a
    linear layer (paperlayer.ai summary, section C, names them; the formulas
    are readings): LayerNorm without affine (norm=0) or RMSNorm (norm=1), then
    z = y * (1 + scale[g]) + shift[g] for the row's conditioning group
    g = row // rows_per_cond; row statistics in binary64, the elementwise
    steps in binary32, z rounded to bf16.

    x: uint16 [R, D]; shift, scale: uint16 [G, D] or None.  Returns uint16 [R, D].
    """
    x = _c(x, np.uint16)
    R, D = x.shape
    rpc = int(rows_per_cond) if rows_per_cond else max(R, 1)
    G = -(-R // rpc) if R else 0
    sh = _c(shift, np.uint16) if shift is not None else None
    sc = _c(scale, np.uint16) if scale is not None else None
    for v in (sh, sc):
        assert v is None or (v.shape[0] >= G and v.shape[1] == D)
    y = np.empty_like(x)
    _check(_load().oracle_norm_mod(_ptr(x), R, D, _ptr(sh), _ptr(sc), rpc, int(norm), float(eps),
                                   _ptr(y), _threads(nthreads)), "oracle_norm_mod")
    return y


def norm_mod_quantize_rows(x, shift=None, scale=None, rows_per_cond=None, norm=NORM_LAYER,
                           eps=1e-6, nthreads=None):
    """The fused prologue of a W8A8 linear: per-row INT8 quantisation of the
    bf16 normalised and modulated rows (norm_mod_bf16 then quantize_rows)."""
    return quantize_rows(norm_mod_bf16(x, shift, scale, rows_per_cond, norm, eps, nthreads),
                         nthreads)


def guard(N: int, K: int) -> bool:
    """Shape guard of the INT8 path (reading of 智猩猩 section 01.3's fallback rule)."""
    return bool(_load().oracle_guard(int(N), int(K)))


def compact_rows(x, mask):
    """Padded-row compaction (智猩猩 section 01.3 last paragraph; paperlayer.ai
    section C).  x: uint16 [B, L, D]; mask: uint8 [B, L].
    Returns (out [count, D], src_row int32 [count], count)."""
    x = _c(x, np.uint16)
    m = _c(mask, np.uint8)
    B, L, D = x.shape
    assert m.shape == (B, L)
    out = np.empty((max(B * L, 1), D), np.uint16)
    src = np.empty((max(B * L, 1),), np.int32)
    cnt = np.zeros((1,), np.int32)
    _check(_load().oracle_compact_rows(_ptr(x), _ptr(m), B, L, D, _ptr(out), _ptr(src), _ptr(cnt)),
           "oracle_compact_rows")
    n = int(cnt[0])
    return out[:n].copy(), src[:n].copy(), n


def bf16_to_f32(h: int) -> float:
    return float(_load().oracle_bf16_to_f32(int(h)))


def f32_to_bf16(f: float) -> int:
    return int(_load().oracle_f32_to_bf16(float(f)))


def f64_to_bf16(v: float) -> int:
    return int(_load().oracle_f64_to_bf16(float(v)))


def gelu_tanh_f64(z: float) -> float:
    return float(_load().oracle_gelu_tanh_f64(float(z)))


def gelu_bf16(h: int) -> int:
    return int(_load().oracle_gelu_bf16(int(h)))
