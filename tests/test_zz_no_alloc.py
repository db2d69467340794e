"""w8a8_linear_noalloc (the guarded linear with its INT8 workspace in the
library's static device scratch) against w8a8_linear with a caller workspace:
bit for bit, on consecutive calls of different sizes (the second smaller, so
stale scratch contents from the first would show), near the scratch limit, on
the BF16 route, and a rejected over-size call that leaves the output untouched.
Called through the C ABI via the binding.  Runs last in collection order, and
passes alone in a fresh process as well as after the other GPU tests."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import int8_w8a8_gemm_amd as w8
import workloads as wl

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    w8.lib()
    yield
    torch.cuda.synchronize()


def _layer(M, K, N, seed, scale=1.0):
    rng = np.random.default_rng(seed)
    x = wl.to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32) * np.float32(scale))
    w = wl.to_bf16_bits(rng.standard_normal((N, K)).astype(np.float32) * np.float32(0.02))
    b = wl.to_bf16_bits(rng.standard_normal(N).astype(np.float32) * np.float32(0.01))
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(DEV).view(torch.bfloat16)
    return d(x), d(w), d(b)


def _both(x, w, b, N, act=w8.ACT_NONE):
    """(noalloc result, path), (workspace result, path), with the INT8 weight
    prepared once when the guard admits the shape."""
    if w8.guard(N, x.shape[1]):
        qw, sw = w8.quantize_rows(w)
        ya, pa = w8.linear_noalloc(x, N, qw=qw, sw=sw, bias=b, act=act)
        yb, pb = w8.linear(x, N, qw=qw, sw=sw, bias=b, act=act)
    else:
        ya, pa = w8.linear_noalloc(x, N, w=w, bias=b, act=act)
        yb, pb = w8.linear(x, N, w=w, bias=b, act=act)
    torch.cuda.synchronize()
    return (ya, pa), (yb, pb)


def test_noalloc_two_calls_second_smaller():
    print("noalloc: two calls, the second smaller", flush=True)
    x1, w1, b1 = _layer(3000, 4096, 1024, 1, scale=3.0)
    (ya, pa), (yb, pb) = _both(x1, w1, b1, 1024)
    assert pa == pb == w8.PATH_INT8
    assert torch.equal(ya.view(torch.int16), yb.view(torch.int16))
    x2, w2, b2 = _layer(700, 2048, 512, 2, scale=0.5)
    (ya, pa), (yb, pb) = _both(x2, w2, b2, 512, act=w8.ACT_GELU_TANH)
    assert pa == pb == w8.PATH_INT8
    assert torch.equal(ya.view(torch.int16), yb.view(torch.int16))


def test_noalloc_near_the_limit_then_small_and_bf16_route():
    print("noalloc: near the scratch limit, then small, then BF16", flush=True)
    K = 4096
    M = w8.NOALLOC_SCRATCH_BYTES // (K + 4) - 64
    assert w8.linear_workspace_bytes(M, K) <= w8.NOALLOC_SCRATCH_BYTES
    x, w, b = _layer(M, K, 256, 3)
    (ya, pa), (yb, pb) = _both(x, w, b, 256)
    assert pa == pb == w8.PATH_INT8
    assert torch.equal(ya.view(torch.int16), yb.view(torch.int16))
    x, w, b = _layer(5, 256, 64, 4)
    (ya, pa), (yb, pb) = _both(x, w, b, 64)
    assert torch.equal(ya.view(torch.int16), yb.view(torch.int16))
    x, w, b = _layer(300, 2050, 130, 5)           # the guard sends it to BF16
    (ya, pa), (yb, pb) = _both(x, w, b, 130)
    assert pa == pb == w8.PATH_BF16
    assert torch.equal(ya.view(torch.int16), yb.view(torch.int16))


def test_noalloc_rejects_inputs_beyond_the_scratch():
    print("noalloc: over-size input rejected", flush=True)
    K = 4096
    M = w8.NOALLOC_SCRATCH_BYTES // (K + 4) + 64
    x, w, b = _layer(M, K, 64, 6)
    qw, sw = w8.quantize_rows(w)
    y = torch.full((M, 64), 1.5, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(w8.W8A8Error) as e:
        w8.linear_noalloc(x, 64, qw=qw, sw=sw, bias=b, y=y)
    assert e.value.status == w8.ESCRATCH
    torch.cuda.synchronize()
    assert bool((y == 1.5).all())
