"""C-ABI checks that need no GPU: the library loads, exports what the header
declares, and every argument check returns before anything is launched."""
from __future__ import annotations

import ctypes
import os
import re

import pytest

import int8_w8a8_gemm_amd as w8

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "w8a8.h")


def _declared():
    src = open(HEADER).read()
    return re.findall(r"W8A8_API\s+[\w\s\*]+?\b(\w+)\s*\(", src)


def test_header_declares_the_four_calls_and_helpers():
    names = set(_declared())
    for n in ("w8a8_quantize_rows", "w8a8_gemm", "w8a8_linear", "compact_padded_rows",
              "w8a8_linear_bf16", "w8a8_guard", "w8a8_linear_workspace_bytes", "w8a8_status_str"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = w8.lib()
    for n in _declared():
        assert hasattr(lib, n), n
    assert set(_declared()) == set(w8.EXPORTS)


def test_guard_truth_table():
    for N in (64, 128, 2048, 4096, 16384):
        for K in (128, 256, 2048, 4096, 16384, 131072):
            assert w8.guard(N, K), (N, K)
    for N, K in [(4100, 4096), (2048, 2050), (32, 4096), (0, 4096), (4096, 0), (4096, 64),
                 (4096, 131072 + 128), (100, 256), (128, 200), (-64, 256), (64, -128)]:
        assert not w8.guard(N, K), (N, K)


def test_workspace_bytes():
    assert w8.linear_workspace_bytes(0, 4096) == 0
    assert w8.linear_workspace_bytes(4, 0) == 0
    assert w8.linear_workspace_bytes(1, 128) == 256 + 4
    assert w8.linear_workspace_bytes(3, 100) == 512 + 12
    M, K = 24576, 4096
    assert w8.linear_workspace_bytes(M, K) == M * K + 4 * M


def test_linear_noalloc_rejects_on_the_host():
    """Inputs beyond the static scratch return ESCRATCH, bad arguments EINVAL,
    before any HIP call (the pointers are never dereferenced)."""
    L = w8.lib()
    path = ctypes.c_int(-7)

    def lin(x, M, K, N, qw, sw, w, b, act, y):
        return L.w8a8_linear_noalloc(x, M, K, N, qw, sw, w, b, act, y, ctypes.byref(path), NULL)

    K = 4096
    M_max = w8.NOALLOC_SCRATCH_BYTES // (K + 4)
    assert w8.linear_workspace_bytes(M_max, K) <= w8.NOALLOC_SCRATCH_BYTES
    assert w8.linear_workspace_bytes(M_max + 64, K) > w8.NOALLOC_SCRATCH_BYTES
    assert lin(A16, M_max + 64, K, 64, A16, A16, NULL, NULL, 0, A16) == w8.ESCRATCH
    assert lin(A16, -1, K, 64, A16, A16, NULL, NULL, 0, A16) == w8.EINVAL
    assert lin(A16, 1 << 31, K, 64, A16, A16, NULL, NULL, 0, A16) == w8.EINVAL
    assert lin(A16, 4, 130, 64, NULL, NULL, NULL, NULL, 0, A16) == w8.EINVAL  # BF16 path needs w
    assert lin(A16, 4, 128, 64, A16, A16, NULL, NULL, 3, A16) == w8.EINVAL    # bad act
    path.value = -7
    assert lin(NULL, 0, 128, 64, A16, A16, NULL, NULL, 0, NULL) == w8.OK      # empty
    assert path.value == w8.PATH_INT8
    assert "scratch" in w8.status_str(w8.ESCRATCH)


def test_gemm_splitk_workspace_and_rejections():
    """Split-K sizing is a property of the shape (host only): S * M * N * 4 bytes for
    shapes the 128 x 128 tiles leave mostly idle with long K, else 0; a missing or
    short workspace is rejected before any HIP call."""
    ws = w8.gemm_splitk_workspace_bytes
    assert ws(256, 4096, 16384) == 4 * 256 * 4096 * 4
    assert ws(100, 512, 8192) == 8 * 100 * 512 * 4
    assert ws(300, 640, 4096) == 4 * 300 * 640 * 4          # 8 slices would be < 8 stages
    for shape in [(2048, 2048, 2048), (24576, 16384, 4096), (512, 4096, 4096), (64, 64, 1024),
                  (0, 4096, 4096), (256, 4100, 16384), (256, 4096, 2050)]:
        assert ws(*shape) == 0, shape
    L = w8.lib()
    g = lambda M, N, K, wsp, wsb: L.w8a8_gemm_splitk(A16, A16, M, A16b, A16c, N, K, NULL, 0, 0,
                                                     A16, wsp, wsb, NULL)
    need = ws(256, 4096, 16384)
    assert g(256, 4096, 16384, NULL, 0) == w8.EINVAL
    assert g(256, 4096, 16384, A16, need - 1) == w8.EINVAL
    assert g(256, 4096, 16384, MIS, need) == w8.EINVAL
    assert g(256, 4100, 16384, A16, need) == w8.EUNSUPPORTED
    assert g(-1, 4096, 16384, A16, need) == w8.EINVAL
    assert g(0, 4096, 16384, NULL, 0) == w8.OK


def test_status_strings():
    assert w8.status_str(0) == "ok"
    assert "invalid" in w8.status_str(-1)
    assert "not supported" in w8.status_str(-2)
    assert "HIP" in w8.status_str(-3)
    assert w8.status_str(123) == "unknown status"


# Fake, never-dereferenced device addresses: every call below must be rejected
# (or be a no-op) on the host before any HIP call is made.
A16 = ctypes.c_void_p(0x10000)
A16b = ctypes.c_void_p(0x20000)
A16c = ctypes.c_void_p(0x30000)
MIS = ctypes.c_void_p(0x10001)
NULL = None


def test_quantize_rows_rejects_bad_arguments():
    L = w8.lib()
    assert L.w8a8_quantize_rows(A16, -1, 8, A16b, A16c, NULL) == w8.EINVAL
    assert L.w8a8_quantize_rows(A16, 4, -8, A16b, A16c, NULL) == w8.EINVAL
    assert L.w8a8_quantize_rows(NULL, 4, 8, A16b, A16c, NULL) == w8.EINVAL
    assert L.w8a8_quantize_rows(A16, 4, 8, NULL, A16c, NULL) == w8.EINVAL
    assert L.w8a8_quantize_rows(A16, 4, 8, A16b, NULL, NULL) == w8.EINVAL
    assert L.w8a8_quantize_rows(MIS, 4, 8, A16b, A16c, NULL) == w8.EINVAL
    assert L.w8a8_quantize_rows(A16, 4, 8, A16b, MIS, NULL) == w8.EINVAL
    assert L.w8a8_quantize_rows(A16, 1 << 31, 8, A16b, A16c, NULL) == w8.EINVAL
    assert L.w8a8_quantize_rows(NULL, 0, 8, NULL, NULL, NULL) == w8.OK  # empty: no-op


def test_gelu_bf16_rejects_bad_arguments():
    L = w8.lib()
    assert L.w8a8_gelu_bf16(A16, -1, A16b, NULL) == w8.EINVAL
    assert L.w8a8_gelu_bf16(NULL, 8, A16b, NULL) == w8.EINVAL
    assert L.w8a8_gelu_bf16(A16, 8, NULL, NULL) == w8.EINVAL
    assert L.w8a8_gelu_bf16(MIS, 8, A16b, NULL) == w8.EINVAL
    assert L.w8a8_gelu_bf16(A16, 8, MIS, NULL) == w8.EINVAL
    assert L.w8a8_gelu_bf16(NULL, 0, NULL, NULL) == w8.OK  # empty: no-op


def test_gemm_rejects_bad_arguments_and_unsupported_shapes():
    L = w8.lib()
    g = lambda qa, sa, M, qw, sw, N, K, b, act, kind, out: L.w8a8_gemm(
        qa, sa, M, qw, sw, N, K, b, act, kind, out, NULL)
    assert g(A16, A16, -1, A16, A16, 64, 128, NULL, 0, 0, A16) == w8.EINVAL
    assert g(A16, A16, 4, A16, A16, 64, 128, NULL, 2, 0, A16) == w8.EINVAL   # bad act
    assert g(A16, A16, 4, A16, A16, 64, 128, NULL, 0, 5, A16) == w8.EINVAL   # bad out kind
    assert g(A16, A16, 4, A16, A16, 64, 128, NULL, 1, 1, A16) == w8.EINVAL   # GELU on int32
    assert g(A16, A16, 4, A16, A16, 4100, 4096, NULL, 0, 0, A16) == w8.EUNSUPPORTED
    assert g(A16, A16, 4, A16, A16, 2048, 2050, NULL, 0, 0, A16) == w8.EUNSUPPORTED
    assert g(A16, A16, 4, A16, A16, 64, 131072 + 128, NULL, 0, 0, A16) == w8.EUNSUPPORTED
    assert g(NULL, A16, 4, A16, A16, 64, 128, NULL, 0, 0, A16) == w8.EINVAL
    assert g(A16, A16, 4, NULL, A16, 64, 128, NULL, 0, 0, A16) == w8.EINVAL
    assert g(A16, A16, 4, A16, A16, 64, 128, NULL, 0, 0, NULL) == w8.EINVAL
    assert g(A16, NULL, 4, A16, A16, 64, 128, NULL, 0, 0, A16) == w8.EINVAL  # bf16 needs scales
    assert g(MIS, A16, 4, A16, A16, 64, 128, NULL, 0, 0, A16) == w8.EINVAL
    assert g(A16, A16, 4, MIS, A16, 64, 128, NULL, 0, 0, A16) == w8.EINVAL
    assert g(A16, A16, 4, A16, A16, 64, 128, NULL, 0, 0, MIS) == w8.EINVAL
    assert g(A16, A16, 4, A16, A16, 64, 128, MIS, 0, 0, A16) == w8.EINVAL   # odd bias address
    assert g(NULL, NULL, 0, NULL, NULL, 64, 128, NULL, 0, 0, NULL) == w8.OK  # M == 0


def test_linear_rejects_bad_arguments():
    L = w8.lib()
    path = ctypes.c_int(-7)
    ws = w8.linear_workspace_bytes(4, 128)

    def lin(x, M, K, N, qw, sw, w, b, act, y, wsp, wsb):
        return L.w8a8_linear(x, M, K, N, qw, sw, w, b, act, y, wsp, wsb, ctypes.byref(path), NULL)

    assert lin(A16, -1, 128, 64, A16, A16, NULL, NULL, 0, A16, A16, ws) == w8.EINVAL
    assert lin(A16, 4, 128, 64, A16, A16, NULL, NULL, 3, A16, A16, ws) == w8.EINVAL
    # INT8 path: needs qw, sw, a big enough 256-byte-aligned workspace
    assert lin(A16, 4, 128, 64, NULL, A16, A16, NULL, 0, A16, A16, ws) == w8.EINVAL
    assert lin(A16, 4, 128, 64, A16, NULL, A16, NULL, 0, A16, A16, ws) == w8.EINVAL
    assert lin(A16, 4, 128, 64, A16, A16, NULL, NULL, 0, A16, NULL, ws) == w8.EINVAL
    assert lin(A16, 4, 128, 64, A16, A16, NULL, NULL, 0, A16, A16, ws - 1) == w8.EINVAL
    assert lin(A16, 4, 128, 64, A16, A16, NULL, NULL, 0, A16, ctypes.c_void_p(0x10010), ws) == w8.EINVAL
    assert lin(A16, 4, 128, 64, A16, A16, NULL, NULL, 0, MIS, A16, ws) == w8.EINVAL
    # BF16 path: needs w
    assert lin(A16, 4, 130, 64, NULL, NULL, NULL, NULL, 0, A16, NULL, 0) == w8.EINVAL
    assert lin(A16, 4, 128, 68, A16, A16, NULL, NULL, 0, A16, NULL, 0) == w8.EINVAL
    # empty work reports the path and launches nothing
    path.value = -7
    assert lin(NULL, 0, 128, 64, A16, A16, NULL, NULL, 0, NULL, NULL, 0) == w8.OK
    assert path.value == w8.PATH_INT8
    path.value = -7
    assert lin(NULL, 0, 130, 64, NULL, NULL, NULL, NULL, 0, NULL, NULL, 0) == w8.OK
    assert path.value == w8.PATH_BF16


def test_linear_bf16_and_compaction_reject_bad_arguments():
    L = w8.lib()
    assert L.w8a8_linear_bf16(A16, -2, 8, A16, 8, NULL, 0, A16, NULL) == w8.EINVAL
    assert L.w8a8_linear_bf16(A16, 2, 8, A16, 8, NULL, 9, A16, NULL) == w8.EINVAL
    assert L.w8a8_linear_bf16(NULL, 2, 8, A16, 8, NULL, 0, A16, NULL) == w8.EINVAL
    assert L.w8a8_linear_bf16(A16, 2, 8, A16, 8, NULL, 0, NULL, NULL) == w8.EINVAL
    assert L.w8a8_linear_bf16(MIS, 2, 8, A16, 8, NULL, 0, A16, NULL) == w8.EINVAL
    assert L.w8a8_linear_bf16(NULL, 0, 8, NULL, 8, NULL, 0, NULL, NULL) == w8.OK
    c = lambda x, m, B, Lq, D, o, s, n: L.compact_padded_rows(x, m, B, Lq, D, o, s, n, NULL)
    assert c(A16, A16, -1, 4, 8, A16, A16, A16) == w8.EINVAL
    assert c(A16, A16, 2, 4, 8, A16, A16, NULL) == w8.EINVAL          # count is required
    assert c(A16, NULL, 2, 4, 8, A16, A16, A16) == w8.EINVAL
    assert c(A16, A16, 2, 4, 8, A16, NULL, A16) == w8.EINVAL
    assert c(A16, A16, 2, 4, 8, NULL, A16, A16) == w8.EINVAL
    assert c(A16, A16, 2, 4, 8, A16, A16, MIS) == w8.EINVAL
    assert c(A16, A16, 1 << 20, 1 << 12, 8, A16, A16, A16) == w8.EINVAL  # B*L >= 2^31


def test_compact_quantize_rejects_bad_arguments():
    L = w8.lib()
    cq = lambda x, m, B, Lq, D, q, sc, s, n: L.w8a8_compact_quantize_rows(x, m, B, Lq, D, q, sc, s, n, NULL)
    assert cq(A16, A16, -1, 4, 8, A16, A16, A16, A16) == w8.EINVAL
    assert cq(A16, A16, 2, -4, 8, A16, A16, A16, A16) == w8.EINVAL
    assert cq(A16, A16, 2, 4, -8, A16, A16, A16, A16) == w8.EINVAL
    assert cq(A16, A16, 2, 4, 8, A16, A16, A16, NULL) == w8.EINVAL     # count is required
    assert cq(A16, A16, 2, 4, 8, A16, A16, A16, MIS) == w8.EINVAL      # count misaligned
    assert cq(A16, NULL, 2, 4, 8, A16, A16, A16, A16) == w8.EINVAL     # mask
    assert cq(A16, A16, 2, 4, 8, A16, NULL, A16, A16) == w8.EINVAL     # scale
    assert cq(A16, A16, 2, 4, 8, A16, MIS, A16, A16) == w8.EINVAL
    assert cq(A16, A16, 2, 4, 8, A16, A16, NULL, A16) == w8.EINVAL     # src_row
    assert cq(NULL, A16, 2, 4, 8, A16, A16, A16, A16) == w8.EINVAL     # x
    assert cq(A16, A16, 2, 4, 8, NULL, A16, A16, A16) == w8.EINVAL     # q
    assert cq(MIS, A16, 2, 4, 8, A16, A16, A16, A16) == w8.EINVAL      # x misaligned
    assert cq(A16, A16, 1 << 20, 1 << 12, 8, A16, A16, A16, A16) == w8.EINVAL  # B*L >= 2^31


def test_quantize_blocks_rejects_bad_arguments():
    L = w8.lib()
    qb = lambda x, B, S, H, D, blk, q, sc: L.w8a8_quantize_blocks(x, B, S, H, D, blk, q, sc, NULL)
    assert qb(A16, -1, 128, 2, 64, 64, A16, A16) == w8.EINVAL
    assert qb(A16, 1, -1, 2, 64, 64, A16, A16) == w8.EINVAL
    assert qb(A16, 1, 128, -2, 64, 64, A16, A16) == w8.EINVAL
    assert qb(A16, 1, 128, 2, -64, 64, A16, A16) == w8.EINVAL
    assert qb(A16, 1, 128, 2, 64, 0, A16, A16) == w8.EINVAL           # block >= 1
    assert qb(A16, 1, 128, 2, 60, 64, A16, A16) == w8.EINVAL          # head_dim % 8
    assert qb(A16, 1, 128, 2, 0, 64, A16, A16) == w8.EINVAL           # head_dim >= 8
    assert qb(A16, 1, 1024, 2, 128, 512, A16, A16) == w8.EINVAL       # block too large to hold
    assert qb(NULL, 1, 128, 2, 64, 64, A16, A16) == w8.EINVAL
    assert qb(A16, 1, 128, 2, 64, 64, NULL, A16) == w8.EINVAL
    assert qb(A16, 1, 128, 2, 64, 64, A16, NULL) == w8.EINVAL
    assert qb(MIS, 1, 128, 2, 64, 64, A16, A16) == w8.EINVAL          # x not 16-byte aligned
    assert qb(A16, 1, 1 << 40, 1 << 10, 64, 1, A16, A16) == w8.EINVAL  # 2^31 blocks or more
    assert qb(A16, 0, 128, 2, 64, 64, NULL, NULL) == w8.OK            # empty: no-op
    assert qb(A16, 1, 0, 2, 64, 64, NULL, NULL) == w8.OK


def test_norm_mod_rejects_bad_arguments():
    L = w8.lib()
    nm = lambda x, R, C, sh, sc, rpc, norm, eps, y: L.w8a8_norm_mod_bf16(x, R, C, sh, sc, rpc, norm,
                                                                         eps, y, NULL)
    nq = lambda x, R, C, rpc, norm, eps, q, s: L.w8a8_norm_mod_quantize_rows(
        x, R, C, NULL, NULL, rpc, norm, eps, q, s, NULL)
    assert nm(A16, -1, 64, NULL, NULL, 1, 0, 1e-6, A16) == w8.EINVAL
    assert nm(A16, 4, 0, NULL, NULL, 1, 0, 1e-6, A16) == w8.EINVAL     # cols >= 1
    assert nm(A16, 4, 64, NULL, NULL, 0, 0, 1e-6, A16) == w8.EINVAL    # rows_per_cond >= 1
    assert nm(A16, 4, 64, NULL, NULL, 1, 2, 1e-6, A16) == w8.EINVAL    # norm kind
    assert nm(A16, 4, 64, NULL, NULL, 1, 0, -1.0, A16) == w8.EINVAL    # eps >= 0
    assert nm(A16, 4, 64, NULL, NULL, 1, 0, float("nan"), A16) == w8.EINVAL
    assert nm(A16, 4, 64, NULL, NULL, 1, 0, float("inf"), A16) == w8.EINVAL
    assert nm(NULL, 4, 64, NULL, NULL, 1, 0, 1e-6, A16) == w8.EINVAL
    assert nm(A16, 4, 64, NULL, NULL, 1, 0, 1e-6, NULL) == w8.EINVAL
    assert nm(MIS, 4, 64, NULL, NULL, 1, 0, 1e-6, A16) == w8.EINVAL     # x 2-byte aligned
    assert nm(A16, 4, 64, MIS, NULL, 1, 0, 1e-6, A16) == w8.EINVAL     # shift 2-byte aligned
    assert nm(A16, 1 << 31, 64, NULL, NULL, 1, 0, 1e-6, A16) == w8.EINVAL  # 2^31 rows
    assert nm(NULL, 0, 64, NULL, NULL, 1, 0, 1e-6, NULL) == w8.OK      # empty: no-op
    assert nq(A16, 4, 64, 1, 1, 0.0, A16, NULL) == w8.EINVAL           # scales out needed
    assert nq(A16, 4, 64, 1, 1, 0.0, NULL, A16) == w8.EINVAL
    assert nq(A16, 4, 64, 1, 1, 0.0, A16, ctypes.c_void_p(0x10002)) == w8.EINVAL  # qscale 4-byte
    assert nq(A16, 4, 64, 0, 1, 0.0, A16, A16) == w8.EINVAL
    assert nq(NULL, 0, 64, 1, 1, 0.0, NULL, NULL) == w8.OK


def test_python_binding_refuses_cpu_tensors():
    import torch
    x = torch.zeros((4, 128), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        w8.quantize_rows(x)


ABI_CHECK = os.path.join(ROOT, "int8_w8a8_gemm_amd", "_build", "abi_check")


def test_c_program_links_only_the_library_and_hip():
    """tests/c/abi_check.cpp is built against the header and libw8a8.so alone."""
    assert os.path.exists(ABI_CHECK), "build first: __graft_entry__.build()"
    import subprocess
    out = subprocess.run(["readelf", "-d", ABI_CHECK], capture_output=True, text=True).stdout
    needed = set(re.findall(r"\(NEEDED\)\s+Shared library: \[([^\]]+)\]", out))
    assert "libw8a8.so" in needed
    assert not any("torch" in n or "python" in n for n in needed), needed


@pytest.mark.gpu
def test_c_program_through_the_abi_on_the_gpu():
    """A plain HIP program (its own hipMalloc buffers and stream, no PyTorch) runs
    the INT8 GEMM against an integer loop, a hand-worked quantisation row, and the
    guard's routing to the BF16 path; it exits 0 and prints "abi_check ok"."""
    import subprocess
    print("c abi check", flush=True)
    p = subprocess.run([ABI_CHECK], capture_output=True, text=True, timeout=60)
    assert p.returncode == 0 and "abi_check ok" in p.stdout, p.stdout + p.stderr
