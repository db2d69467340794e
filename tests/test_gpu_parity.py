"""GPU parity: the HIP library, called through its C ABI, against the CPU oracle.

Bar: int8 codes, scales and INT32 accumulators bit-exact; bf16 outputs within
1 bf16 ulp (the INT8 path's epilogue follows the same binary32 sequence as the
oracle and is expected to be bit-exact); BF16 fallback within 1 ulp or the
summation bound.  Small cases are compared in full; the full-size workloads
(24576-row video shapes) on seeded sampled rows, which the oracle computes
exactly for those rows because every step is row-local.
"""
from __future__ import annotations

import math
import sys

import numpy as np
import pytest
import torch

import int8_w8a8_gemm_amd as w8
import oracle
import workloads as wl
from helpers import sweep_rows, ulp_dist_bf16

pytestmark = pytest.mark.gpu

DEV = "cuda"


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def d_bf16(a_u16: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a_u16).view(np.int16)).to(DEV).view(torch.bfloat16)


def d_i8(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def h_u16(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def h(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    w8.lib()
    yield
    torch.cuda.synchronize()


@pytest.fixture(scope="module")
def ffn():
    return wl.video_ffn()


@pytest.fixture(scope="module")
def attn():
    return wl.video_attn_proj()


# ---------------------------------------------------------------------------
# quantisation
# ---------------------------------------------------------------------------

def _check_quant(x_u16, label):
    say(f"quantize {label} {x_u16.shape}")
    q, s = w8.quantize_rows(d_bf16(x_u16))
    torch.cuda.synchronize()
    qo, so = oracle.quantize_rows(x_u16)
    assert np.array_equal(h(s).view(np.uint32), so.view(np.uint32)), label
    assert np.array_equal(h(q), qo), label


def test_quantize_tiny_and_audio():
    lin = wl.tiny()
    _check_quant(lin.x, "tiny.x")
    _check_quant(lin.w, "tiny.w")
    lin = wl.audio()
    _check_quant(lin.x, "audio.x")
    _check_quant(lin.w, "audio.w")


def test_quantize_video_and_ffn_full_size(attn, ffn):
    _check_quant(ffn.x, "ffn.x")
    _check_quant(attn.x, "attn.x")
    _check_quant(attn.w, "attn.w")
    _check_quant(ffn.w1, "ffn.w1")
    _check_quant(ffn.w2, "ffn.w2 (K=16384)")


def test_quantize_exhaustive_absmax_sweep():
    """Every bf16 absmax a >= 2^-100 (all 228 binades x 128 mantissas) against
    every bf16 x with |x| <= a that can give a nonzero code."""
    rows = sweep_rows(range(1, 255), pad_to=2312)     # vector path (cols % 8 == 0)
    _check_quant(rows, "sweep vec")
    _check_quant(np.ascontiguousarray(rows[:, :2305]), "sweep generic")  # scalar path


@pytest.mark.parametrize("cols", [1, 8, 300, 512, 520, 4096, 8192, 16384, 32768, 40000])
def test_quantize_shapes_and_degenerate_rows(cols):
    rng = np.random.default_rng(cols)
    R = 67
    x = rng.standard_normal((R, cols)).astype(np.float32)
    x *= np.float32(2.0) ** rng.integers(-30, 30, (R, 1)).astype(np.float32)
    x[3] = 0.0
    x[4] = 2.0 ** -101
    x[5] = -3.0
    if cols > 2:
        x[6, 1] = -1e4
    _check_quant(wl.to_bf16_bits(x), f"cols={cols}")


def test_quantize_empty_rows_is_noop():
    q, s = w8.quantize_rows(torch.empty((0, 64), dtype=torch.bfloat16, device=DEV))
    torch.cuda.synchronize()
    assert q.shape == (0, 64) and s.shape == (0,)


# ---------------------------------------------------------------------------
# per-block quantisation of attention Q / K
# ---------------------------------------------------------------------------

def _block_input(B, S, H, D, seed):
    rng = np.random.default_rng(seed)
    v = rng.standard_normal((B * S, H * D)).astype(np.float32)
    v *= np.float32(2.0) ** rng.integers(-40, 40, (B * S, 1)).astype(np.float32)
    x = wl.to_bf16_bits(v)
    if B * S >= 2 and H >= 2:
        x[0:2, D:2 * D] = 0                                    # zero values in block (0, 0, 1)
    return x


# Shapes: one-token blocks, ragged last blocks, several samples and heads,
# head_dim 8 .. 128, and each chunks-per-thread variant of the kernel (a block
# of block x head_dim / 8 chunks: 1 .. 16 per thread for 256 threads).
@pytest.mark.parametrize("B,S,H,D,blk", [(1, 1, 1, 8, 1), (1, 37, 1, 16, 1), (2, 37, 3, 16, 8),
                                         (3, 130, 4, 64, 64), (1, 257, 2, 128, 128),
                                         (2, 5, 2, 8, 16), (1, 96, 8, 32, 32), (2, 300, 4, 128, 256),
                                         (1, 1000, 2, 64, 64), (2, 77, 3, 256, 32)])
def test_quantize_blocks_matches_oracle(B, S, H, D, blk):
    say(f"quantize blocks B={B} S={S} H={H} D={D} block={blk}")
    x = _block_input(B, S, H, D, B * 7919 + S * 31 + H * 7 + D + blk)
    q, s = w8.quantize_blocks(d_bf16(x), B, H, blk)
    torch.cuda.synchronize()
    qo, so = oracle.quantize_blocks(x, B, H, blk)
    assert np.array_equal(h(s).view(np.uint32), so.view(np.uint32))
    assert np.array_equal(h(q), qo)


def test_quantize_blocks_degenerate_blocks():
    say("quantize blocks: zero and sub-threshold blocks")
    B, S, H, D, blk = 2, 70, 4, 16, 32
    x = _block_input(B, S, H, D, 3)
    x[:32, 16:32] = 0
    x[S:S + 32, :16] = wl.to_bf16_bits(np.full((32, 16), 2.0**-101, np.float32))
    q, s = w8.quantize_blocks(d_bf16(x), B, H, blk)
    qo, so = oracle.quantize_blocks(x, B, H, blk)
    assert np.array_equal(h(s).view(np.uint32), so.view(np.uint32)) and np.array_equal(h(q), qo)
    assert h(s)[0, 0, 1] == 0 and h(s)[1, 0, 0] == 0


@pytest.mark.parametrize("blk", [128, 64])
def test_quantize_blocks_video_attention_full_size(blk):
    """Video self-attention Q / K stand-in: 24576 tokens x 32 heads x 128, blocks
    of 128 tokens (Q) and 64 (K), compared in full."""
    say(f"quantize blocks video 24576 x 32 x 128 block={blk}")
    rng = np.random.default_rng(blk)
    x = wl.to_bf16_bits(rng.standard_normal((24576, 4096)).astype(np.float32))
    q, s = w8.quantize_blocks(d_bf16(x), 1, 32, blk)
    qo, so = oracle.quantize_blocks(x, 1, 32, blk)
    assert np.array_equal(h(s).view(np.uint32), so.view(np.uint32))
    assert np.array_equal(h(q), qo)


def _nm_input(R, D, G, seed, const_rows=True):
    """Rows ~ 3 N(0,1) + 0.5 with 1% outlier columns x30, and (when there are
    enough rows) one constant row and one zero row; modulation rows
    ~ 0.3 N(0,1)."""
    rng = np.random.default_rng(seed)
    v = rng.standard_normal((R, D)).astype(np.float32) * np.float32(3.0) + np.float32(0.5)
    cols = rng.choice(D, max(1, D // 100), replace=False)
    v[:, cols] *= np.float32(30.0)
    if const_rows and R >= 4:
        v[1] = v[1, 0]
        v[2] = 0.0
    sc = rng.standard_normal((G, D)).astype(np.float32) * np.float32(0.3)
    sh = rng.standard_normal((G, D)).astype(np.float32) * np.float32(0.3)
    return wl.to_bf16_bits(v), wl.to_bf16_bits(sh), wl.to_bf16_bits(sc)


def _f32(b):
    return (np.asarray(b).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _bf16_ulp(v):
    """Spacing of bf16 numbers at |v| (2^-133 at 0 and among subnormals)."""
    e = np.frexp(np.abs(v))[1]
    return np.ldexp(1.0, np.maximum(e - 8, -133))


def _check_norm_mod(z, x, sh, sc, rpc, norm, eps, label=""):
    """The kernel's bf16 rows against the oracle's binary64 values rounded once.
    The kernel takes the row statistics in binary64 and the elementwise steps in
    binary32: d = RN32(x - mu), y = RN32(d RN32(rstd)), z = fmaf(y, RN32(1 + scale),
    shift), so before its bf16 rounding it is off the exact value by at most
    u|z| + 4.01u|P| (u = 2^-24, P = (x - mu) rstd (1 + scale)), plus the binary64
    statistics' D 2^-53 relative terms.  Accepted: within 1 bf16 ulp of the oracle,
    or within ulp(oracle) + E with E = 2^-21 (|P| + |shift|) + D 2^-50 (mean|x| rstd
    |1 + scale| + |P|).  Returns the fraction of bit-equal values."""
    zr = oracle.norm_mod_bf16(x, sh, sc, rpc, norm, eps)
    if z.size == 0:
        return 1.0
    R, D = x.shape
    xf = _f32(x)
    mu = xf.mean(axis=1, keepdims=True) if norm == w8.NORM_LAYER else np.zeros((R, 1))
    var = ((xf - mu) ** 2).mean(axis=1, keepdims=True) + eps
    rstd = np.where(var > 0, 1.0 / np.sqrt(np.where(var > 0, var, 1.0)), 0.0)
    g = np.arange(R) // rpc
    c = 1.0 + (_f32(sc)[g] if sc is not None else 0.0)
    shf = _f32(sh)[g] if sh is not None else 0.0
    P = (xf - mu) * rstd * c
    E = 2.0 ** -21 * (np.abs(P) + np.abs(shf)) + D * 2.0 ** -50 * (
        np.abs(xf).mean(axis=1, keepdims=True) * rstd * np.abs(c) + np.abs(P))
    gf, rf = _f32(z), _f32(zr)
    ok = (ulp_dist_bf16(z, zr) <= 1) | (np.abs(gf - rf) <= _bf16_ulp(rf) + E)
    assert ok.all(), f"{label}: {int((~ok).sum())} values outside the bound"
    rate = float(np.mean(z == zr))
    say(f"{label} norm/mod exact-match rate {rate:.6f}")
    assert rate > 0.95
    return rate


def _check_norm_mod_quant(q, s, z_gpu, x, sh, sc, rpc, norm, eps, label=""):
    """Fused codes and scales: the oracle's quantiser applied to the kernel's own
    bf16 rows, bit for bit (the rows themselves are held to _check_norm_mod)."""
    qr, sr = oracle.quantize_rows(z_gpu)
    assert np.array_equal(q, qr), label
    assert np.array_equal(s.view(np.uint32), sr.view(np.uint32)), label
    qo, _ = oracle.norm_mod_quantize_rows(x, sh, sc, rpc, norm, eps)
    say(f"{label} codes equal to the all-oracle chain: {float(np.mean(q == qo)):.6f}")


NM_SHAPES = [(1, 8, 1), (7, 64, 3), (33, 1000, 5), (20, 2048, 4), (17, 1030, 4), (64, 4096, 16), (9, 8192, 3),
             (5, 16384, 2), (3, 32768, 1), (2, 40000, 1), (300, 512, 100)]


@pytest.mark.parametrize("R,D,rpc", NM_SHAPES)
@pytest.mark.parametrize("norm", [w8.NORM_LAYER, w8.NORM_RMS])
@pytest.mark.parametrize("mod", [True, False])
def test_norm_mod_matches_oracle(R, D, rpc, norm, mod):
    """bf16 rows within the norm/modulation bound of the oracle, and the fused
    quantisation's codes and scales bit-exact against the oracle's quantiser on
    those rows (vector paths of every width; 1030 and 40000 columns take the
    generic kernel)."""
    say(f"norm mod R={R} D={D} rpc={rpc} norm={norm} mod={mod}")
    G = -(-R // rpc)
    x, sh, sc = _nm_input(R, D, G, R * 7 + D + norm)
    sh, sc = (sh, sc) if mod else (None, None)
    eps = 1e-6
    dx = d_bf16(x)
    dsh, dsc = (d_bf16(sh), d_bf16(sc)) if mod else (None, None)
    z = h_u16(w8.norm_mod_bf16(dx, dsh, dsc, rpc, norm, eps))
    _check_norm_mod(z, x, sh, sc, rpc, norm, eps, f"R={R} D={D}")
    q, s = w8.norm_mod_quantize_rows(dx, dsh, dsc, rpc, norm, eps)
    _check_norm_mod_quant(h(q), h(s), z, x, sh, sc, rpc, norm, eps, f"R={R} D={D}")


def _random_nm_cases(n, seed):
    """Seeded (rows, cols, rows_per_cond, norm, eps): cols 1 .. 9000 (multiples of 8
    and not), groups of 1 .. 64 rows, both norms, eps 0 or 1e-5."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        D = int(rng.integers(1, 1126)) * 8 if i % 3 else int(rng.integers(1, 9000))
        out.append((int(rng.integers(1, 200)), D, int(rng.integers(1, 65)), i % 2,
                    0.0 if i % 4 == 0 else 1e-5))
    return out


@pytest.mark.parametrize("R,D,rpc,norm,eps", _random_nm_cases(16, 77))
def test_norm_mod_random_shapes(R, D, rpc, norm, eps):
    say(f"norm mod random R={R} D={D} rpc={rpc} norm={norm} eps={eps}")
    G = -(-R // rpc)
    x, sh, sc = _nm_input(R, D, G, R + D + rpc)
    dx, dsh, dsc = d_bf16(x), d_bf16(sh), d_bf16(sc)
    z = h_u16(w8.norm_mod_bf16(dx, dsh, dsc, rpc, norm, eps))
    _check_norm_mod(z, x, sh, sc, rpc, norm, eps, f"R={R} D={D}")
    q, s = w8.norm_mod_quantize_rows(dx, dsh, dsc, rpc, norm, eps)
    _check_norm_mod_quant(h(q), h(s), z, x, sh, sc, rpc, norm, eps, f"R={R} D={D}")


@pytest.mark.parametrize("norm", [w8.NORM_LAYER, w8.NORM_RMS])
def test_norm_mod_eps_zero_and_degenerate_rows(norm):
    """eps = 0: a constant row (LayerNorm) or a zero row normalises to 0 and
    quantises to scale 0; with modulation its z is the shift row."""
    R, D = 6, 256
    x, sh, sc = _nm_input(R, D, R, 3 + norm)
    z = h_u16(w8.norm_mod_bf16(d_bf16(x), d_bf16(sh), d_bf16(sc), 1, norm, 0.0))
    _check_norm_mod(z, x, sh, sc, 1, norm, 0.0, "eps 0")
    assert np.array_equal(z[2], sh[2])  # zero row: y = 0, z = shift
    assert np.array_equal(z[2], oracle.norm_mod_bf16(x, sh, sc, 1, norm, 0.0)[2])
    q, s = w8.norm_mod_quantize_rows(d_bf16(x), None, None, 1, norm, 0.0)
    assert h(s)[2] == 0 and not h(q)[2].any()


def test_norm_mod_video_tokens_full_size_sampled():
    """24576 video token rows of 4096 in 8 conditioning groups of 3072 rows:
    the fused quantisation compared on sampled rows (every step is row-local;
    each sampled row is checked with its group's modulation rows)."""
    R, D, rpc = 24576, 4096, 3072
    say(f"norm mod full size R={R} D={D}")
    x, sh, sc = _nm_input(R, D, R // rpc, 77)
    dx, dsh, dsc = d_bf16(x), d_bf16(sh), d_bf16(sc)
    q, s = w8.norm_mod_quantize_rows(dx, dsh, dsc, rpc)
    z = h_u16(w8.norm_mod_bf16(dx, dsh, dsc, rpc))
    rng = np.random.default_rng(78)
    rows = np.unique(np.concatenate([[0, 1, 2, rpc - 1, rpc, R - 1], rng.choice(R, 200, replace=False)]))
    g = rows // rpc
    xs, shs, scs = (np.ascontiguousarray(a) for a in (x[rows], sh[g], sc[g]))
    _check_norm_mod(z[rows], xs, shs, scs, 1, w8.NORM_LAYER, 1e-6, "video tokens")
    _check_norm_mod_quant(h(q)[rows], h(s)[rows], np.ascontiguousarray(z[rows]), xs, shs, scs, 1,
                          w8.NORM_LAYER, 1e-6, "video tokens")


def test_norm_mod_unaligned_rows_take_the_generic_kernel():
    """x, the modulation rows and the outputs 2 bytes off 16-byte alignment (cols a
    multiple of 8): the generic kernel, bit-exact as the vector one."""
    R, D = 21, 512
    x, sh, sc = _nm_input(R, D, 3, 9)
    def off(a):
        t = torch.zeros(a.size + 8, dtype=torch.int16, device=DEV)
        v = t[1:1 + a.size]
        v.copy_(torch.from_numpy(np.ascontiguousarray(a).reshape(-1).view(np.int16)).to(DEV))
        return v.view(torch.bfloat16).view(a.shape)
    dx, dsh, dsc = off(x), off(sh), off(sc)
    assert dx.data_ptr() % 16 == 2
    yb = torch.zeros(R * D + 8, dtype=torch.int16, device=DEV)
    y = yb[1:1 + R * D].view(torch.bfloat16).view(R, D)
    w8.norm_mod_bf16(dx, dsh, dsc, 7, w8.NORM_LAYER, 1e-6, y=y)
    z_ln = h_u16(y)
    _check_norm_mod(z_ln, x, sh, sc, 7, w8.NORM_LAYER, 1e-6, "unaligned LN")
    qb = torch.zeros(R * D + 16, dtype=torch.int8, device=DEV)
    q = qb[3:3 + R * D].view(R, D)
    qs = torch.empty((R,), dtype=torch.float32, device=DEV)
    w8.norm_mod_quantize_rows(dx, dsh, dsc, 7, w8.NORM_RMS, 1e-6, q=q, qscale=qs)
    w8.norm_mod_bf16(dx, dsh, dsc, 7, w8.NORM_RMS, 1e-6, y=y)
    z_rms = h_u16(y)
    _check_norm_mod(z_rms, x, sh, sc, 7, w8.NORM_RMS, 1e-6, "unaligned RMS")
    _check_norm_mod_quant(h(q), h(qs), z_rms, x, sh, sc, 7, w8.NORM_RMS, 1e-6, "unaligned RMS")


@pytest.mark.parametrize("N,act", [(512, w8.ACT_NONE), (1024, w8.ACT_GELU_TANH), (100, w8.ACT_NONE)])
def test_linear_on_normed_rows(N, act):
    """W8A8Linear.normed: norm + modulation + quantisation fused, then the INT8 GEMM
    (guarded shapes) -- bit-exact against the oracle's quantize_rows of the
    kernel's normalised rows (themselves within the norm/modulation bound),
    quantize_rows of W, INT32 product and epilogue; or, for N = 100, the bf16
    rows of norm_mod_bf16 through the BF16 fallback, within its bound."""
    M, K, rpc = 300, 1024, 100
    say(f"linear on normed rows M={M} K={K} N={N} act={act}")
    x, sh, sc = _nm_input(M, K, M // rpc, N)
    rng = np.random.default_rng(N + 1)
    w = wl.to_bf16_bits(rng.standard_normal((N, K)).astype(np.float32) * np.float32(0.03))
    b = wl.to_bf16_bits(rng.standard_normal(N).astype(np.float32) * np.float32(0.1))
    layer = w8.W8A8Linear.prepare(d_bf16(w), d_bf16(b), act)
    y = h_u16(layer.normed(d_bf16(x), d_bf16(sh), d_bf16(sc), rpc))
    z = h_u16(w8.norm_mod_bf16(d_bf16(x), d_bf16(sh), d_bf16(sc), rpc))
    _check_norm_mod(z, x, sh, sc, rpc, w8.NORM_LAYER, 1e-6, "normed linear")
    if layer.path == w8.PATH_INT8:
        qa, sa = oracle.quantize_rows(z)
        qw, sw = oracle.quantize_rows(w)
        ref = oracle.epilogue(oracle.gemm_i32(qa, qw), sa, sw, b, act=act)
        d = ulp_dist_bf16(y, ref)
        assert d.max() <= 1
        if act == w8.ACT_NONE:
            assert np.array_equal(y, ref)
    else:
        assert N == 100
        _check_fallback(y, z, w, b)


def test_norm_mod_guard_bands():
    say("norm mod guard bands")
    R, D = 37, 1024
    x, sh, sc = _nm_input(R, D, 1, 5)
    pad = 4096
    n = R * D
    big = torch.full((n + 2 * pad,), 0x5A, dtype=torch.int8, device=DEV)
    sbig = torch.full((R + 128,), -7.0, dtype=torch.float32, device=DEV)
    ybig = torch.full((n + 2 * pad,), 0x7F7F, dtype=torch.int16, device=DEV)
    q = big[pad:pad + n].view(R, D)
    s = sbig[64:64 + R]
    y = ybig[pad:pad + n].view(torch.bfloat16).view(R, D)
    w8.norm_mod_quantize_rows(d_bf16(x), d_bf16(sh), d_bf16(sc), R, q=q, qscale=s)
    w8.norm_mod_bf16(d_bf16(x), d_bf16(sh), d_bf16(sc), R, y=y)
    hb, hs, hy = h(big), h(sbig), h(ybig)
    assert np.all(hb[:pad] == 0x5A) and np.all(hb[pad + n:] == 0x5A)
    assert np.all(hs[:64] == -7.0) and np.all(hs[64 + R:] == -7.0)
    assert np.all(hy[:pad] == 0x7F7F) and np.all(hy[pad + n:] == 0x7F7F)
    z = hy[pad:pad + n].view(np.uint16).reshape(R, D)
    _check_norm_mod(z, x, sh, sc, R, w8.NORM_LAYER, 1e-6, "guard bands")
    _check_norm_mod_quant(hb[pad:pad + n].reshape(R, D), hs[64:64 + R], np.ascontiguousarray(z),
                          x, sh, sc, R, w8.NORM_LAYER, 1e-6, "guard bands")


def test_quantize_blocks_guard_bands():
    say("quantize blocks guard bands")
    B, S, H, D, blk = 2, 45, 3, 32, 16
    x = _block_input(B, S, H, D, 9)
    pad = 4096
    n = B * S * H * D
    big = torch.full((n + 2 * pad,), 0x5A, dtype=torch.int8, device=DEV)
    nblk = -(-S // blk)
    sbig = torch.full((B * nblk * H + 2 * 64,), -7.0, dtype=torch.float32, device=DEV)
    q = big[pad:pad + n].view(B * S, H * D)
    sc = sbig[64:64 + B * nblk * H].view(B, nblk, H)
    w8.quantize_blocks(d_bf16(x), B, H, blk, q=q, scale=sc)
    hb, hs = h(big), h(sbig)
    assert np.all(hb[:pad] == 0x5A) and np.all(hb[pad + n:] == 0x5A)
    assert np.all(hs[:64] == -7.0) and np.all(hs[64 + B * nblk * H:] == -7.0)
    qo, so = oracle.quantize_blocks(x, B, H, blk)
    assert np.array_equal(hb[pad:pad + n].reshape(B * S, H * D), qo)
    assert np.array_equal(hs[64:64 + B * nblk * H].view(np.uint32), so.reshape(-1).view(np.uint32))


# ---------------------------------------------------------------------------
# INT8 GEMM: int32 accumulator and bf16 epilogue
# ---------------------------------------------------------------------------

# On a 256-CU MI355X the launcher takes 256 x 256 tiles when there are at
# least 128 of them, else 128 x 128 tiles when there are at least 128 of those,
# else 64 x 64 tiles; instead of 256 x 256 it takes 192 x 256 tiles where their
# rounds of tiles per CU cost less (256 x 256 and 192 x 256 tiles run 16 x 16
# x 64 MFMAs, the smaller ones 32 x 32 x 32).  A persistent workgroup takes several tiles when there
# are more than 256.  Covered here: 64 x 64 tiles (the first seven shapes),
# 128 x 128 tiles (2048^3 and 2000 x 1984, ragged; 1000 x 2048 x 8192 with the
# 3-deep K ring of long K loops), 192 x 256 tiles with ragged
# M, with ragged N (4100 x 4096, 4096 x 4160, both with workgroups taking two
# tiles) and on a text-projection row count (2378 x 4096), 256 x 256 tiles
# with ragged M and N (3900 x 3776, 3900 x 4032).  Larger ragged shapes:
# test_gemm_mid_tiles_ragged_sampled, test_gemm_large_tiles_short_k_ragged_sampled
# and the full-size FFN tests.
GEMM_SHAPES = [(1, 64, 128), (64, 128, 256), (129, 192, 384), (300, 320, 1024), (257, 64, 4096),
               (1000, 448, 2048), (33, 256, 16384), (2048, 2048, 2048), (2000, 1984, 512),
               (1000, 2048, 8192), (4100, 4096, 256), (4096, 4160, 128), (2378, 4096, 512), (3900, 3776, 128),
               (3900, 4032, 128)]


@pytest.mark.parametrize("M,N,K", GEMM_SHAPES)
def test_gemm_int32_bit_exact(M, N, K):
    say(f"gemm i32 M={M} N={N} K={K}")
    rng = np.random.default_rng(M * 7 + N * 3 + K)
    qa = rng.integers(-127, 128, (M, K), dtype=np.int8)
    qw = rng.integers(-127, 128, (N, K), dtype=np.int8)
    acc = w8.gemm(d_i8(qa), None, d_i8(qw), None, out_kind=w8.OUT_I32)
    torch.cuda.synchronize()
    assert np.array_equal(h(acc), oracle.gemm_i32(qa, qw))


def _random_gemm_shapes(n, seed):
    """Seeded shapes the guard accepts: M any (1 .. 3000), N a multiple of 64
    (64 .. 4096), K a multiple of 128 (128 .. 8192), so that every tile
    configuration, full and ragged, is met."""
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        M = int(rng.integers(1, 3001))
        N = 64 * int(rng.integers(1, 65))
        K = 128 * int(rng.integers(1, 65))
        out.append((M, N, K))
    return out


@pytest.mark.parametrize("M,N,K", _random_gemm_shapes(24, 2024))
def test_gemm_random_shapes_int32_and_epilogue(M, N, K):
    """INT32 accumulators bit-exact and the bf16 epilogue (bias) bit-exact on
    seeded random shapes with random codes and scales."""
    say(f"gemm random M={M} N={N} K={K}")
    rng = np.random.default_rng(M * 31 + N * 7 + K)
    qa = rng.integers(-127, 128, (M, K), dtype=np.int8)
    qw = rng.integers(-127, 128, (N, K), dtype=np.int8)
    qa_d, qw_d = d_i8(qa), d_i8(qw)
    acc = oracle.gemm_i32(qa, qw)
    assert np.array_equal(h(w8.gemm(qa_d, None, qw_d, None, out_kind=w8.OUT_I32)), acc)
    sa = (rng.random(M, dtype=np.float32) * np.float32(1e-3) + np.float32(1e-6)).astype(np.float32)
    sw = (rng.random(N, dtype=np.float32) * np.float32(1e-3) + np.float32(1e-6)).astype(np.float32)
    b = wl.to_bf16_bits(rng.standard_normal(N).astype(np.float32))
    y = w8.gemm(qa_d, torch.from_numpy(sa).to(DEV), qw_d, torch.from_numpy(sw).to(DEV), d_bf16(b))
    assert np.array_equal(h_u16(y), oracle.epilogue(acc, sa, sw, b))


@pytest.mark.parametrize("M,N,K", [(2048, 2048, 2048), (512, 4096, 4096), (1000, 640, 384),
                                   (1024, 1024, 4096), (256, 512, 8192)])
def test_gemm_k_groups_exact(M, N, K):
    """The INT8 128 x 128 tiers (2-deep and 3-deep rings; 2048^3, 512 x 4096 x 4096,
    ragged 1000 x 640) split each 128-byte K stage between two groups of waves, 32
    bytes at a time (group g takes K bytes with (k // 32) % 2 == g), and add the
    groups' INT32 accumulators through LDS after the K loop.  Codes nonzero only in
    one group's bytes give that group's sum alone; then all codes, the raw INT32
    and the bf16 epilogue with and without GELU, all bit-exact."""
    say(f"gemm K groups M={M} N={N} K={K}")
    rng = np.random.default_rng(M + N + K)
    qa = rng.integers(-127, 128, (M, K), dtype=np.int8)
    qw = rng.integers(-127, 128, (N, K), dtype=np.int8)
    qw_d = d_i8(qw)
    grp = (np.arange(K) // 32) % 2
    for g in (0, 1):
        qg = np.where(grp[None, :] == g, qa, 0).astype(np.int8)
        acc = w8.gemm(d_i8(qg), None, qw_d, None, out_kind=w8.OUT_I32)
        assert np.array_equal(h(acc), oracle.gemm_i32(qg, qw)), f"group {g}"
    acc_ref = oracle.gemm_i32(qa, qw)
    qa_d = d_i8(qa)
    assert np.array_equal(h(w8.gemm(qa_d, None, qw_d, None, out_kind=w8.OUT_I32)), acc_ref)
    sa = (rng.random(M, dtype=np.float32) * np.float32(2e-4) + np.float32(1e-6)).astype(np.float32)
    sw = (rng.random(N, dtype=np.float32) * np.float32(2e-4) + np.float32(1e-6)).astype(np.float32)
    b = wl.to_bf16_bits(rng.standard_normal(N).astype(np.float32))
    sa_d, sw_d = torch.from_numpy(sa).to(DEV), torch.from_numpy(sw).to(DEV)
    for act in (w8.ACT_NONE, w8.ACT_GELU_TANH):
        y = w8.gemm(qa_d, sa_d, qw_d, sw_d, d_bf16(b), act=act)
        assert np.array_equal(h_u16(y), oracle.epilogue(acc_ref, sa, sw, b, act=act)), act


@pytest.mark.parametrize("M,N,K", [(256, 4096, 16384), (1024, 1024, 4096), (100, 512, 8192),
                                   (300, 640, 4096), (77, 192, 131072), (2048, 2048, 2048)])
def test_gemm_splitk_matches_oracle(M, N, K):
    """Split-K across workgroups (K slices of 128 x 128 tiles, INT32 partials added
    in slice order, then the epilogue): raw INT32 and bf16 with and without GELU
    bit-exact against the oracle and equal to w8a8_gemm; codes nonzero only in one
    slice give that slice's sum alone; 2048^3 is not split (workspace 0)."""
    need = w8.gemm_splitk_workspace_bytes(M, N, K)
    S = need // (M * N * 4)
    say(f"gemm split-K M={M} N={N} K={K} slices={S}")
    assert (S > 1) == ((M, N, K) != (2048, 2048, 2048))
    rng = np.random.default_rng(M * 3 + N + K)
    qa = rng.integers(-127, 128, (M, K), dtype=np.int8)
    qw = rng.integers(-127, 128, (N, K), dtype=np.int8)
    qa_d, qw_d = d_i8(qa), d_i8(qw)
    ws = torch.full((max(need, 16) + 64,), 0x5A, dtype=torch.uint8, device=DEV)
    acc_ref = oracle.gemm_i32(qa, qw)
    got = w8.gemm_splitk(qa_d, None, qw_d, None, out_kind=w8.OUT_I32, workspace=ws[:max(need, 16)])
    assert np.array_equal(h(got), acc_ref)
    assert bool((ws[max(need, 16):] == 0x5A).all())     # nothing past the workspace
    if S > 1:
        sl = np.arange(K) // (K // S)
        qs = np.where(sl[None, :] == S - 1, qa, 0).astype(np.int8)
        got = w8.gemm_splitk(d_i8(qs), None, qw_d, None, out_kind=w8.OUT_I32)
        assert np.array_equal(h(got), oracle.gemm_i32(qs, qw)), "last slice alone"
    sa = (rng.random(M, dtype=np.float32) * np.float32(2e-4) + np.float32(1e-6)).astype(np.float32)
    sw = (rng.random(N, dtype=np.float32) * np.float32(2e-4) + np.float32(1e-6)).astype(np.float32)
    b = wl.to_bf16_bits(rng.standard_normal(N).astype(np.float32))
    sa_d, sw_d = torch.from_numpy(sa).to(DEV), torch.from_numpy(sw).to(DEV)
    for act in (w8.ACT_NONE, w8.ACT_GELU_TANH):
        for bias in (b, None):
            y = h_u16(w8.gemm_splitk(qa_d, sa_d, qw_d, sw_d, d_bf16(bias) if bias is not None
                                     else None, act=act))
            assert np.array_equal(y, oracle.epilogue(acc_ref, sa, sw, bias, act=act)), (act, bias is None)
            y2 = h_u16(w8.gemm(qa_d, sa_d, qw_d, sw_d, d_bf16(bias) if bias is not None else None,
                               act=act))
            assert np.array_equal(y, y2)


def test_gemm_int32_extremes_and_max_k():
    say("gemm i32 extremes K=131072")
    M, N, K = 64, 64, 131072
    qa = np.full((M, K), 127, np.int8)
    qa[1::2] = -127
    qw = np.full((N, K), 127, np.int8)
    acc = h(w8.gemm(d_i8(qa), None, d_i8(qw), None, out_kind=w8.OUT_I32))
    assert np.all(acc[0::2] == 16129 * K) and np.all(acc[1::2] == -16129 * K)


def test_gemm_max_k_closed_form():
    """K = 131072 (the largest the guard admits: |acc| <= 127^2 K < 2^31) on the
    192 x 256 tiles with 16 x 16 x 64 MFMAs (4600 x 4096: 384 such tiles, two
    rounds, as many as 288 tiles of 256 x 256 take; ragged M).  Codes are +-127
    by row, so every accumulator is +-16129 K: a closed form, checked on all
    outputs."""
    M, N, K = 4600, 4096, 131072
    say(f"gemm max K M={M} N={N} K={K}")
    sa = torch.where(torch.arange(M, device=DEV) % 3 == 0, -1, 1).to(torch.int8)
    sw = torch.where(torch.arange(N, device=DEV) % 5 == 0, -1, 1).to(torch.int8)
    qa = (sa[:, None] * 127).expand(M, K).contiguous()
    qw = (sw[:, None] * 127).expand(N, K).contiguous()
    acc = w8.gemm(qa, None, qw, None, out_kind=w8.OUT_I32)
    torch.cuda.synchronize()
    exp = (sa.to(torch.int64)[:, None] * sw.to(torch.int64)[None, :]) * (16129 * K)
    assert torch.equal(acc.to(torch.int64), exp)
    del qa, qw, acc


@pytest.mark.parametrize("M,N,K", [(64, 128, 256), (129, 192, 384), (2048, 2048, 2048),
                                   (2000, 1984, 512), (1000, 2048, 4096), (4100, 4160, 128),
                                   (2378, 4096, 256),
                                   (3900, 3776, 128)])
@pytest.mark.parametrize("act", [w8.ACT_NONE, w8.ACT_GELU_TANH])
@pytest.mark.parametrize("with_bias", [True, False])
def test_gemm_epilogue_matches_oracle(M, N, K, act, with_bias):
    say(f"gemm bf16 M={M} N={N} K={K} act={act} bias={with_bias}")
    rng = np.random.default_rng(M + N + K + act)
    x = wl.to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    w = wl.to_bf16_bits(rng.standard_normal((N, K)).astype(np.float32) * np.float32(0.02))
    b = wl.to_bf16_bits(rng.standard_normal(N).astype(np.float32) * np.float32(0.01)) if with_bias else None
    qa, sa = oracle.quantize_rows(x)
    qw, sw = oracle.quantize_rows(w)
    y = w8.gemm(d_i8(qa), torch.from_numpy(sa).to(DEV), d_i8(qw), torch.from_numpy(sw).to(DEV),
                d_bf16(b) if b is not None else None, act=act)
    ref = oracle.epilogue(oracle.gemm_i32(qa, qw), sa, sw, b, act=act)
    got = h_u16(y)
    d = ulp_dist_bf16(got, ref)
    assert d.max() <= 1
    if act == w8.ACT_NONE:
        assert np.array_equal(got, ref)  # same binary32 sequence on both sides


def _tile_edge_rows(M, tiles, rng, extra=120):
    """Rows on both sides of every boundary of tiles of each height in `tiles`,
    the ragged last tile and a seeded random sample."""
    tiles = (tiles,) if isinstance(tiles, int) else tiles
    edges = [r for tile in tiles for b in range(tile, M, tile) for r in (b - 1, b)]
    tail = list(range(max(0, M - 70), M))
    rnd = list(rng.choice(M, extra, replace=False))
    return np.unique(np.array([0, 1] + edges + tail + rnd, dtype=np.int64))


def test_gemm_mid_tiles_ragged_sampled():
    """6100 x 4032 x 8192: 512 tiles of 192 x 256 take two rounds on a 256-CU
    MI355X, as 384 of 256 x 256 would, so the 192 x 256 path (16 x 16 x 64
    MFMAs) runs, ragged in M and in N, persistent with two tiles per
    workgroup.  INT32 accumulators and the bf16 epilogue (with bias) compared
    on sampled rows that include both sides of every 192-row tile boundary and
    the ragged last tile; all columns."""
    M, N, K = 6100, 4032, 8192
    say(f"gemm mid tiles M={M} N={N} K={K}")
    rng = np.random.default_rng(8192)
    qa = rng.integers(-127, 128, (M, K), dtype=np.int8)
    qw = rng.integers(-127, 128, (N, K), dtype=np.int8)
    rows = _tile_edge_rows(M, 192, rng)
    qa_d, qw_d = d_i8(qa), d_i8(qw)
    acc = h(w8.gemm(qa_d, None, qw_d, None, out_kind=w8.OUT_I32))
    acc_ref = oracle.gemm_i32(np.ascontiguousarray(qa[rows]), qw)
    assert np.array_equal(acc[rows], acc_ref)
    sa = (rng.random(M, dtype=np.float32) * np.float32(1e-4) + np.float32(1e-6)).astype(np.float32)
    sw = (rng.random(N, dtype=np.float32) * np.float32(1e-3) + np.float32(1e-6)).astype(np.float32)
    b = wl.to_bf16_bits(rng.standard_normal(N).astype(np.float32))
    y = w8.gemm(qa_d, torch.from_numpy(sa).to(DEV), qw_d, torch.from_numpy(sw).to(DEV), d_bf16(b))
    ref = oracle.epilogue(acc_ref, np.ascontiguousarray(sa[rows]), sw, b)
    assert np.array_equal(h_u16(y)[rows], ref)
    y = w8.gemm(qa_d, torch.from_numpy(sa).to(DEV), qw_d, torch.from_numpy(sw).to(DEV), None)
    ref = oracle.epilogue(acc_ref, np.ascontiguousarray(sa[rows]), sw, None)
    assert np.array_equal(h_u16(y)[rows], ref)


def test_gemm_large_tiles_short_k_ragged_sampled():
    """12000 x 8000 x 512: 1504 tiles of 256 x 256 (16 x 16 x 64 MFMAs, about 6
    per CU on a 256-CU MI355X) with a short K loop, ragged in M (224 rows in
    the last tile-row) and N (64 columns in the last tile-column).  INT32
    accumulators and the bf16 epilogue (with and without bias) on sampled
    rows, both sides of every 256-row boundary included."""
    M, N, K = 12000, 8000, 512
    say(f"gemm large short K M={M} N={N} K={K}")
    rng = np.random.default_rng(512)
    qa = rng.integers(-127, 128, (M, K), dtype=np.int8)
    qw = rng.integers(-127, 128, (N, K), dtype=np.int8)
    rows = _tile_edge_rows(M, 256, rng, extra=60)
    qa_d, qw_d = d_i8(qa), d_i8(qw)
    acc_ref = oracle.gemm_i32(np.ascontiguousarray(qa[rows]), qw)
    assert np.array_equal(h(w8.gemm(qa_d, None, qw_d, None, out_kind=w8.OUT_I32))[rows], acc_ref)
    sa = (rng.random(M, dtype=np.float32) * np.float32(1e-3) + np.float32(1e-5)).astype(np.float32)
    sw = (rng.random(N, dtype=np.float32) * np.float32(1e-3) + np.float32(1e-5)).astype(np.float32)
    b = wl.to_bf16_bits(rng.standard_normal(N).astype(np.float32))
    for bias in (b, None):
        y = w8.gemm(qa_d, torch.from_numpy(sa).to(DEV), qw_d, torch.from_numpy(sw).to(DEV),
                    d_bf16(bias) if bias is not None else None)
        ref = oracle.epilogue(acc_ref, np.ascontiguousarray(sa[rows]), sw, bias)
        assert np.array_equal(h_u16(y)[rows], ref)


@pytest.mark.parametrize("M,N,K", [(129, 192, 384), (2048, 2048, 2048), (6100, 4032, 8192)])
def test_gemm_without_bias_keeps_the_sign_of_zero(M, N, K):
    """Without a bias the output is the rounded product alone.  With scales whose
    product underflows to +0 that product is +0 or -0 by the sign of the
    accumulator, so the bf16 output is 0x8000 exactly where acc < 0 and 0x0000
    elsewhere (the last shape runs the 192 x 256 tiles with 16 x 16 x 64 MFMAs,
    the others smaller ones with 32 x 32 x 32).  Rows compared: every tile
    edge, the tail and a random sample."""
    say(f"gemm signed zero M={M} N={N} K={K}")
    rng = np.random.default_rng(M + 7)
    qa = rng.integers(-127, 128, (M, K), dtype=np.int8)
    qw = rng.integers(-127, 128, (N, K), dtype=np.int8)
    sa = np.full(M, 1e-30, dtype=np.float32)
    sw = np.full(N, 1e-30, dtype=np.float32)
    assert np.float32(sa[0]) * np.float32(sw[0]) == 0  # underflows in binary32
    rows = _tile_edge_rows(M, (128, 192), rng, extra=40)
    y = h_u16(w8.gemm(d_i8(qa), torch.from_numpy(sa).to(DEV), d_i8(qw), torch.from_numpy(sw).to(DEV),
                      None))[rows]
    acc = oracle.gemm_i32(np.ascontiguousarray(qa[rows]), qw)
    assert np.array_equal(y, np.where(acc < 0, 0x8000, 0).astype(np.uint16))
    assert np.array_equal(y, oracle.epilogue(acc, np.ascontiguousarray(sa[rows]), sw, None))
    assert (acc < 0).any() and (acc > 0).any()


def test_gemm_rejects_unsupported_shape_on_device():
    qa = torch.zeros((4, 2050), dtype=torch.int8, device=DEV)
    qw = torch.zeros((64, 2050), dtype=torch.int8, device=DEV)
    with pytest.raises(w8.W8A8Error) as e:
        w8.gemm(qa, torch.ones(4, device=DEV), qw, torch.ones(64, device=DEV))
    assert e.value.status == w8.EUNSUPPORTED


def test_gemm_guard_bands_untouched():
    say("gemm guard bands")
    M, N, K = 129, 192, 256
    rng = np.random.default_rng(5)
    qa = rng.integers(-127, 128, (M, K), dtype=np.int8)
    qw = rng.integers(-127, 128, (N, K), dtype=np.int8)
    pad = 4096
    big = torch.full((M * N + 2 * pad,), -12345, dtype=torch.int32, device=DEV)
    out = big[pad:pad + M * N].view(M, N)
    w8.gemm(d_i8(qa), None, d_i8(qw), None, out_kind=w8.OUT_I32, out=out)
    hb = h(big)
    assert np.all(hb[:pad] == -12345) and np.all(hb[pad + M * N:] == -12345)
    assert np.array_equal(hb[pad:pad + M * N].reshape(M, N), oracle.gemm_i32(qa, qw))
    sent = 0x7F7F
    bigb = torch.full((M * N + 2 * pad,), sent, dtype=torch.int16, device=DEV)
    y = bigb[pad:pad + M * N].view(torch.bfloat16).view(M, N)
    sa = torch.ones(M, device=DEV)
    sw = torch.ones(N, device=DEV)
    w8.gemm(d_i8(qa), sa, d_i8(qw), sw, out=y)
    hb = h(bigb)
    assert np.all(hb[:pad] == sent) and np.all(hb[pad + M * N:] == sent)


# ---------------------------------------------------------------------------
# the guarded linear on the five workloads
# ---------------------------------------------------------------------------

def _run_linear(x_u16, w_u16, b_u16, act=w8.ACT_NONE):
    xd, wd = d_bf16(x_u16), d_bf16(w_u16)
    layer = w8.W8A8Linear.prepare(wd, d_bf16(b_u16) if b_u16 is not None else None, act)
    y = layer(xd)
    torch.cuda.synchronize()
    return h_u16(y), layer.path


def test_linear_tiny_full():
    say("linear tiny")
    lin = wl.tiny()
    got, path = _run_linear(lin.x, lin.w, lin.bias)
    ref, rpath = oracle.w8a8_linear(lin.x, lin.w, lin.bias)
    assert path == rpath == w8.PATH_INT8
    assert np.array_equal(got, ref)


def test_linear_audio_full():
    say("linear audio 2048^3")
    lin = wl.audio()
    got, path = _run_linear(lin.x, lin.w, lin.bias)
    ref, _ = oracle.w8a8_linear(lin.x, lin.w, lin.bias)
    assert path == w8.PATH_INT8
    assert np.array_equal(got, ref)


def _sampled_linear(x_u16, w_u16, b_u16, rows, act=w8.ACT_NONE, label=""):
    say(f"linear {label} M={x_u16.shape[0]} N={w_u16.shape[0]} K={x_u16.shape[1]} act={act}")
    got, path = _run_linear(x_u16, w_u16, b_u16, act)
    assert path == w8.PATH_INT8
    ref, _ = oracle.w8a8_linear(np.ascontiguousarray(x_u16[rows]), w_u16, b_u16, act=act)
    return got, ref


def _video_rows(M, n=512, tiles=(256, 384), seed=1):
    """n seeded rows of [0, M): both rows at every boundary of the 256-row tiles
    the video GEMMs run on (and of 384-row tiles), the first and the last row,
    and seeded random rows to make up n (M = 24576: 256 edge rows and 256
    random ones)."""
    edges = {0, M - 1} | {r for t in tiles for b in range(t, M, t) for r in (b - 1, b)}
    rng = np.random.Generator(np.random.PCG64(seed))
    rest = [int(r) for r in rng.permutation(M) if int(r) not in edges][:max(0, n - len(edges))]
    return np.array(sorted(edges | set(rest)), dtype=np.int64)


def test_linear_video_attn_proj_sampled(attn):
    rows = _video_rows(attn.x.shape[0])
    got, ref = _sampled_linear(attn.x, attn.w, attn.bias, rows, label="attn-proj")
    assert np.array_equal(got[rows], ref)


def test_linear_video_ffn_up_gelu_sampled(ffn):
    rows = _video_rows(ffn.x.shape[0])
    got, ref = _sampled_linear(ffn.x, ffn.w1, ffn.b1, rows, act=w8.ACT_GELU_TANH, label="ffn-up")
    d = ulp_dist_bf16(got[rows], ref)
    say(f"  ffn-up: exact {np.mean(d == 0):.6f}, max ulp {d.max()}")
    assert np.array_equal(got[rows], ref)  # both sides round GELU's binary64 value once


def test_linear_video_ffn_down_on_oracle_h(ffn):
    """Down projection fed the oracle's own H rows (the GELU output), so both
    sides quantise the same bf16 input: bit-exact."""
    rows = _video_rows(ffn.x.shape[0])
    say("oracle ffn-up rows for the down projection")
    h_ref, _ = oracle.w8a8_linear(np.ascontiguousarray(ffn.x[rows]), ffn.w1, ffn.b1,
                                  act=oracle.ACT_GELU_TANH)
    got, ref = _sampled_linear(h_ref, ffn.w2, ffn.b2, np.arange(len(rows)), label="ffn-down")
    assert np.array_equal(got, ref)


def test_linear_video_ffn_chain_end_to_end(ffn):
    """Whole pair on the GPU (GPU H feeds the GPU down projection) against the
    oracle chain: both sides round GELU's binary64 value once, so bit-exact."""
    rows = _video_rows(ffn.x.shape[0])
    say("ffn chain on GPU (GELU in the up-projection epilogue)")
    up = w8.W8A8Linear.prepare(d_bf16(ffn.w1), d_bf16(ffn.b1), w8.ACT_GELU_TANH)
    down = w8.W8A8Linear.prepare(d_bf16(ffn.w2), d_bf16(ffn.b2))
    y = h_u16(down(up(d_bf16(ffn.x))))
    say("ffn chain on the oracle")
    h_ref, _ = oracle.w8a8_linear(np.ascontiguousarray(ffn.x[rows]), ffn.w1, ffn.b1,
                                  act=oracle.ACT_GELU_TANH)
    y_ref, _ = oracle.w8a8_linear(h_ref, ffn.w2, ffn.b2)
    assert np.array_equal(y[rows], y_ref)


def test_ffn_pipeline_fused_gelu_quantise(ffn):
    """The benchmark's pipeline: quantise X, up GEMM without activation, fused
    GELU + quantise of its output U, down GEMM.  X's codes and scales, and the
    codes and scales of the whole GELU output (24576 x 16384, from the GPU's own
    U), in full; U and the output on 512 sampled rows with every tile edge;
    all bit-exact against the oracle."""
    M = ffn.x.shape[0]
    rows = _video_rows(M)
    say("ffn fused pipeline on GPU")
    qw1, sw1 = w8.quantize_rows(d_bf16(ffn.w1))
    qw2, sw2 = w8.quantize_rows(d_bf16(ffn.w2))
    qx, sx = w8.quantize_rows(d_bf16(ffn.x))
    y1 = w8.gemm(qx, sx, qw1, sw1, d_bf16(ffn.b1))
    qh, sh = w8.gelu_quantize_rows(y1)
    y = h_u16(w8.gemm(qh, sh, qw2, sw2, d_bf16(ffn.b2)))
    torch.cuda.synchronize()
    say("ffn: X quantisation in full")
    qx_ref, sx_ref = oracle.quantize_rows(ffn.x)
    assert np.array_equal(h(sx).view(np.uint32), sx_ref.view(np.uint32))
    assert np.array_equal(h(qx), qx_ref)
    del qx_ref
    u = h_u16(y1)
    del y1
    say("ffn: U on sampled rows")
    y1_ref, _ = oracle.w8a8_linear(np.ascontiguousarray(ffn.x[rows]), ffn.w1, ffn.b1)
    assert np.array_equal(u[rows], y1_ref)
    say("ffn: GELU + quantisation of the whole U")
    qh_ref, sh_ref = oracle.gelu_quantize_rows(u)
    del u
    assert np.array_equal(h(sh).view(np.uint32), sh_ref.view(np.uint32))
    assert np.array_equal(h(qh), qh_ref)
    say("ffn: down projection on sampled rows")
    qw2_ref, sw2_ref = oracle.quantize_rows(ffn.w2)
    y_ref = oracle.epilogue(oracle.gemm_i32(np.ascontiguousarray(qh_ref[rows]), qw2_ref),
                            np.ascontiguousarray(sh_ref[rows]), sw2_ref, ffn.b2)
    assert np.array_equal(y[rows], y_ref)


def _small_ffn(seed, M=2048, D=1024, F=4096):
    rng = np.random.default_rng(seed)
    x = wl.to_bf16_bits(rng.standard_normal((M, D)).astype(np.float32))
    w1 = wl.to_bf16_bits(rng.standard_normal((F, D)).astype(np.float32) * np.float32(0.03))
    w2 = wl.to_bf16_bits(rng.standard_normal((D, F)).astype(np.float32) * np.float32(0.02))
    b1 = wl.to_bf16_bits(rng.standard_normal(F).astype(np.float32) * np.float32(0.01))
    b2 = wl.to_bf16_bits(rng.standard_normal(D).astype(np.float32) * np.float32(0.01))
    return x, w1, b1, w2, b2


class _FfnPipeline:
    """The benchmark's pipeline (quantise X, up GEMM, GELU + quantise, down GEMM)
    on preallocated buffers, so that it can be captured into a graph."""

    def __init__(self, w1, b1, w2, b2, M):
        self.qw1, self.sw1 = w8.quantize_rows(d_bf16(w1))
        self.qw2, self.sw2 = w8.quantize_rows(d_bf16(w2))
        self.b1, self.b2 = d_bf16(b1), d_bf16(b2)
        F, D = self.qw1.shape[0], self.qw2.shape[0]
        self.x = torch.empty((M, D), dtype=torch.bfloat16, device=DEV)
        self.qx = torch.empty((M, D), dtype=torch.int8, device=DEV)
        self.sx = torch.empty((M,), dtype=torch.float32, device=DEV)
        self.u = torch.empty((M, F), dtype=torch.bfloat16, device=DEV)
        self.qh = torch.empty((M, F), dtype=torch.int8, device=DEV)
        self.sh = torch.empty((M,), dtype=torch.float32, device=DEV)
        self.y = torch.empty((M, D), dtype=torch.bfloat16, device=DEV)

    def step(self, stream=None):
        w8.quantize_rows(self.x, self.qx, self.sx, stream=stream)
        w8.gemm(self.qx, self.sx, self.qw1, self.sw1, self.b1, out=self.u, stream=stream)
        w8.gelu_quantize_rows(self.u, self.qh, self.sh, stream=stream)
        w8.gemm(self.qh, self.sh, self.qw2, self.sw2, self.b2, out=self.y, stream=stream)


def test_ffn_pipeline_graph_capture_and_replay():
    """The four entry points of a step captured into one graph (none allocates,
    frees, synchronises or records a memset): each of three replays, on new
    inputs and with eager work between them, equals an eager run bit for bit."""
    say("ffn pipeline: graph capture and replay")
    x, w1, b1, w2, b2 = _small_ffn(21)
    M = x.shape[0]
    pipe = _FfnPipeline(w1, b1, w2, b2, M)
    eager = _FfnPipeline(w1, b1, w2, b2, M)
    pipe.x.copy_(d_bf16(x))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        pipe.step()  # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        pipe.step()
    rng = np.random.default_rng(22)
    for r in range(3):
        xr = wl.to_bf16_bits(rng.standard_normal(x.shape).astype(np.float32) * np.float32(1 + r))
        pipe.x.copy_(d_bf16(xr))
        eager.x.copy_(pipe.x)
        g.replay()
        torch.cuda.synchronize()
        eager.step()          # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(pipe.y, eager.y), f"replay {r}"
        assert torch.equal(pipe.qh, eager.qh) and torch.equal(pipe.sh, eager.sh), f"replay {r}"


def test_layer_on_a_side_stream_allocates_there():
    """W8A8Linear(x, stream=s) and .normed(..., stream=s) on a stream that is not
    the current one, kept busy so that their kernels run after the calls return:
    the workspace and the normed layer's codes they allocate and drop belong to
    s, so the current stream's allocations and writes made in between cannot
    land in them.  Every result bit-exact against the oracle."""
    say("layer calls on a side stream")
    M, K, N, rpc = 768, 2048, 1536, 256
    rng = np.random.default_rng(41)
    x = wl.to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    w = wl.to_bf16_bits(rng.standard_normal((N, K)).astype(np.float32) * np.float32(0.02))
    b = wl.to_bf16_bits(rng.standard_normal(N).astype(np.float32) * np.float32(0.01))
    _, sh, sc = _nm_input(M, K, M // rpc, 42)
    layer = w8.W8A8Linear.prepare(d_bf16(w), d_bf16(b))
    dx, dsh, dsc = d_bf16(x), d_bf16(sh), d_bf16(sc)
    z = h_u16(w8.norm_mod_bf16(dx, dsh, dsc, rpc))  # the normed rows, on the current stream
    busy_a = torch.randint(-127, 128, (8192, 8192), dtype=torch.int8, device=DEV)
    busy_s = torch.ones(8192, dtype=torch.float32, device=DEV)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    torch.cuda.synchronize()
    outs, normed = [], []
    for i in range(3):
        w8.gemm(busy_a, busy_s, busy_a, busy_s, stream=side)  # keeps `side` busy
        outs.append(layer(dx, stream=side))
        normed.append(layer.normed(dx, dsh, dsc, rpc, stream=side))
        # current-stream allocations of the sizes just dropped, written at once
        junk = [torch.full((layer_ws,), 0x55 + i, dtype=torch.uint8, device=DEV)
                for layer_ws in (w8.linear_workspace_bytes(M, K), M * K, 4 * M)]
        del junk
    torch.cuda.synchronize()
    qw, sw = oracle.quantize_rows(w)
    qa, sa = oracle.quantize_rows(x)
    ref = oracle.epilogue(oracle.gemm_i32(qa, qw), sa, sw, b)
    qz, sz = oracle.quantize_rows(z)
    ref_n = oracle.epilogue(oracle.gemm_i32(qz, qw), sz, sw, b)
    _check_norm_mod(z, x, sh, sc, rpc, w8.NORM_LAYER, 1e-6, "side stream")
    for i in range(3):
        assert np.array_equal(h_u16(outs[i]), ref), f"call {i}"
        assert np.array_equal(h_u16(normed[i]), ref_n), f"normed call {i}"


def test_two_pipelines_on_two_streams():
    """Two steps on two streams at once (different inputs and weights) give
    the results each gives alone: the library keeps no state between calls."""
    say("two pipelines on two streams")
    pa = _FfnPipeline(*_small_ffn(31)[1:], 1024)
    pb = _FfnPipeline(*_small_ffn(32)[1:], 1024)
    xa = _small_ffn(31, M=1024)[0]
    xb = _small_ffn(32, M=1024)[0]
    pa.x.copy_(d_bf16(xa))
    pb.x.copy_(d_bf16(xb))
    pa.step()
    pb.step()
    torch.cuda.synchronize()
    ya, yb = pa.y.clone(), pb.y.clone()
    pa.y.zero_()
    pb.y.zero_()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    s1.wait_stream(torch.cuda.current_stream())
    s2.wait_stream(torch.cuda.current_stream())
    for _ in range(3):
        pa.step(stream=s1)
        pb.step(stream=s2)
    torch.cuda.synchronize()
    assert torch.equal(pa.y, ya) and torch.equal(pb.y, yb)


def test_gelu_exhaustive_all_bf16_inputs():
    """GELU-tanh on every finite bf16 value, through the BF16 path with a 1x1
    identity weight (so the pre-activation is the input itself), against the
    oracle's float64 GELU rounded once: bit-exact."""
    say("gelu exhaustive")
    bits = np.arange(65536, dtype=np.uint16)
    bits = bits[(bits & 0x7F80) != 0x7F80]
    x = bits.reshape(-1, 1)
    one = wl.to_bf16_bits(np.float32([[1.0]]))
    got = h_u16(w8.linear_bf16(d_bf16(x), d_bf16(one), act=w8.ACT_GELU_TANH)).ravel()
    # the oracle of the same route: y = x * 1 (+0 for x = -0), then GELU
    ref = oracle.linear_bf16(x, one, act=oracle.ACT_GELU_TANH).ravel()
    assert np.array_equal(ref[bits != 0x8000], oracle.gelu_rows(bits)[bits != 0x8000])
    bad = np.flatnonzero(got != ref)
    assert bad.size == 0, [(hex(bits[i]), hex(got[i]), hex(ref[i])) for i in bad[:10]]


def test_gelu_bf16_elementwise_all_inputs():
    """The elementwise GELU (the lookup table every table-driven kernel reads)
    on every finite bf16 value against the oracle's GELU: bit-exact."""
    say("gelu_bf16 elementwise, all finite inputs")
    bits = np.arange(65536, dtype=np.uint16)
    bits = bits[(bits & 0x7F80) != 0x7F80]
    got = h_u16(w8.gelu_bf16(d_bf16(bits)))
    ref = oracle.gelu_rows(bits.reshape(1, -1)).ravel()
    bad = np.flatnonzero(got != ref)
    assert bad.size == 0, [(hex(bits[i]), hex(got[i]), hex(ref[i])) for i in bad[:10]]
    # odd length, offset start (2-byte alignment only)
    x = d_bf16(bits[:1001].copy())
    y = torch.empty(1001, dtype=torch.bfloat16, device=DEV)
    w8.gelu_bf16(x[1:], y[1:])
    assert np.array_equal(h_u16(y[1:]), ref[1:1001])


# The table-driven GELU + quantise kernel takes inputs of 2^24 elements and
# more; one shape per row width it is specialised for, with ragged row counts.
@pytest.mark.parametrize("rows,cols", [(4099, 4096), (2051, 8192), (1031, 16384), (517, 32768)])
def test_gelu_quantize_table_path_matches_oracle(rows, cols):
    say(f"gelu+quantise (table path) {rows}x{cols}")
    assert rows * cols >= 1 << 24
    rng = np.random.default_rng(rows)
    y = rng.standard_normal((rows, cols)).astype(np.float32) * np.float32(0.9)
    y[3] *= 30.0
    y[4] = -12.0            # GELU underflows to (-)0 / subnormals: scale 0
    y[5] = 0.0
    yb = wl.to_bf16_bits(y)
    # every finite bf16 value appears somewhere in the input
    allv = np.arange(65536, dtype=np.uint16)
    allv = allv[(allv & 0x7F80) != 0x7F80]
    yb.ravel()[7 * cols: 7 * cols + allv.size] = allv
    q, s = w8.gelu_quantize_rows(d_bf16(yb))
    qo, so = oracle.gelu_quantize_rows(yb)
    assert np.array_equal(h(s).view(np.uint32), so.view(np.uint32))
    assert np.array_equal(h(q), qo)


@pytest.mark.parametrize("cols", [4096, 16384, 300])
def test_gelu_quantize_matches_oracle(cols):
    say(f"gelu+quantise cols={cols}")
    rng = np.random.default_rng(cols + 7)
    R = 129
    y = rng.standard_normal((R, cols)).astype(np.float32) * np.float32(0.7)
    y[3] *= 20.0
    y[4] = -12.0            # GELU underflows to (-)0 / subnormals
    y[5] = 0.0
    yb = wl.to_bf16_bits(y)
    q, s = w8.gelu_quantize_rows(d_bf16(yb))
    qo, so = oracle.gelu_quantize_rows(yb)
    assert np.array_equal(h(s).view(np.uint32), so.view(np.uint32))
    assert np.array_equal(h(q), qo)


def test_guarded_mixed_batch():
    say("guarded mixed: compaction + conforming linear + two fallbacks")
    g = wl.guarded_mixed()
    B, L, D = g.x.shape
    xd = d_bf16(g.x.reshape(B * L, D)).view(B, L, D)
    out, src, cnt = w8.compact_padded_rows(xd, torch.from_numpy(g.mask).to(DEV))
    n = int(cnt.item())
    o_out, o_src, o_n = oracle.compact_rows(g.x, g.mask)
    assert n == o_n == int(g.lengths.sum())
    assert np.array_equal(h(src)[:n], o_src)
    assert np.array_equal(h_u16(out[:n]), o_out)
    xc = out[:n]
    # conforming projection on the compacted rows
    layer = w8.W8A8Linear.prepare(d_bf16(g.w), d_bf16(g.b))
    y = h_u16(layer(xc))
    ref, p = oracle.w8a8_linear(o_out, g.w, g.b)
    assert layer.path == w8.PATH_INT8 and p == 0
    assert np.array_equal(y, ref)
    # fallback A: N = 4100
    say("fallback A N=4100")
    layer = w8.W8A8Linear.prepare(d_bf16(g.w_a), d_bf16(g.b_a))
    assert layer.path == w8.PATH_BF16
    ya = h_u16(layer(xc))
    _check_fallback(ya, o_out, g.w_a, g.b_a)
    # fallback B: K = 2050 (rows only 4-byte aligned)
    say("fallback B K=2050")
    layer = w8.W8A8Linear.prepare(d_bf16(g.w_b), d_bf16(g.b_b))
    assert layer.path == w8.PATH_BF16
    yb = h_u16(layer(d_bf16(g.x_b)))
    _check_fallback(yb, g.x_b, g.w_b, g.b_b)


def _check_fallback(got, x, w, b, act=oracle.ACT_NONE):
    if act != oracle.ACT_NONE:
        return _check_fallback_gelu(got, x, w, b)
    ref = oracle.linear_bf16(x, w, b, act=act)
    d = ulp_dist_bf16(got, ref)
    ok1 = d <= 1
    frac = float(np.mean(ok1))
    say(f"  fallback within 1 ulp: {frac:.6f}, max ulp {d.max()}")
    if not np.all(ok1):
        K = x.shape[1]
        u = 2.0**-23
        gamma = K * u / (1 - K * u)
        xf = np.abs(wl.from_bf16_bits(x).astype(np.float64))
        wf = np.abs(wl.from_bf16_bits(w).astype(np.float64))
        bad = np.argwhere(~ok1)
        for i, j in bad[:20000]:
            mag = float(xf[i] @ wf[j]) + abs(float(wl.from_bf16_bits(b[j:j + 1])[0]))
            rf = float(wl.from_bf16_bits(ref[i:i + 1, j])[0])
            gf = float(wl.from_bf16_bits(got[i:i + 1, j])[0])
            ulp = math.ldexp(1.0, math.frexp(abs(rf))[1] - 8) if rf != 0 else 2.0**-133
            assert abs(gf - rf) <= ulp + gamma * mag, (i, j, gf, rf)
    assert frac > 0.999


def _gelu64(z):
    """GELU-tanh in float64 (only for tolerance intervals)."""
    return 0.5 * z * (1.0 + math.tanh(math.sqrt(2.0 / math.pi) * (z + 0.044715 * z**3)))


def _check_fallback_gelu(got, x, w, b):
    """GELU after the BF16 linear: the pre-activation may differ from the
    oracle's within the summation bound (ulp + gamma_K * sum |x||w| + |b|), and
    GELU is then applied to it.  Every output that is not bit-exact must lie in
    GELU's image of that pre-activation interval (GELU falls to its minimum at
    z = -0.7518 and rises after), widened by one output ulp for the rounding."""
    lin = oracle.linear_bf16(x, w, b)
    ref = oracle.gelu_rows(lin)
    bad = np.argwhere(got != ref)
    say(f"  fallback+GELU bit-exact: {1 - bad.shape[0] / got.size:.6f}")
    assert bad.shape[0] <= max(10, got.size // 1000)
    K = x.shape[1]
    u = 2.0**-23
    gamma = K * u / (1 - K * u)
    xf = np.abs(wl.from_bf16_bits(x).astype(np.float64))
    wf = np.abs(wl.from_bf16_bits(w).astype(np.float64))
    zmin = -0.7517916

    def ulp(v):
        return math.ldexp(1.0, math.frexp(abs(v))[1] - 8) if v != 0 else 2.0**-133

    for i, j in bad:
        zf = float(wl.from_bf16_bits(lin[i:i + 1, j])[0])
        mag = float(xf[i] @ wf[j]) + abs(float(wl.from_bf16_bits(b[j:j + 1])[0]))
        r = ulp(zf) + gamma * mag
        cand = [_gelu64(zf - r), _gelu64(zf + r)]
        if zf - r < zmin < zf + r:
            cand.append(_gelu64(zmin))
        lo, hi = min(cand), max(cand)
        gf = float(wl.from_bf16_bits(got[i:i + 1, j])[0])
        assert lo - ulp(lo) <= gf <= hi + ulp(hi), (i, j, zf, r, gf, lo, hi)


def test_fallback_on_conforming_shapes_and_gelu():
    say("fallback tiny/audio + gelu")
    lin = wl.tiny()
    y = h_u16(w8.linear_bf16(d_bf16(lin.x), d_bf16(lin.w), d_bf16(lin.bias)))
    _check_fallback(y, lin.x, lin.w, lin.bias)
    y = h_u16(w8.linear_bf16(d_bf16(lin.x), d_bf16(lin.w), d_bf16(lin.bias), act=w8.ACT_GELU_TANH))
    _check_fallback(y, lin.x, lin.w, lin.bias, act=oracle.ACT_GELU_TANH)
    rng = np.random.default_rng(3)
    for (M, N, K) in [(1, 1, 1), (5, 7, 3), (130, 67, 129), (64, 4100, 2050)]:
        x = wl.to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
        w = wl.to_bf16_bits(rng.standard_normal((N, K)).astype(np.float32) * np.float32(0.02))
        b = wl.to_bf16_bits(rng.standard_normal(N).astype(np.float32) * np.float32(0.01))
        y = h_u16(w8.linear_bf16(d_bf16(x), d_bf16(w), d_bf16(b)))
        _check_fallback(y, x, w, b)


# The tiled BF16 path (K % 64 == 0, 16-byte aligned operands) on each tile
# configuration: 64 x 64 (first four), 128 x 128, 192 x 256 (4100 x 4100 and
# 4352 x 4104, with workgroups taking two tiles; 2378 x 4098 in one round),
# 256 x 256 (3900 x 3900); with N % 8 != 0 rows are stored in 8-byte parts
# (N % 4 == 0), 4-byte parts (N = 258, 4098) or element by element (N = 255),
# K = 64 is a single stage.
@pytest.mark.parametrize("M,N,K", [(300, 100, 64), (97, 256, 1024), (300, 258, 64), (97, 255, 128),
                                   (2000, 1992, 256), (4100, 4100, 64), (4352, 4104, 192),
                                   (2378, 4098, 128), (3900, 3900, 64)])
@pytest.mark.parametrize("act", [w8.ACT_NONE, w8.ACT_GELU_TANH])
def test_fallback_tiled_path(M, N, K, act):
    say(f"fallback tiled M={M} N={N} K={K} act={act}")
    rng = np.random.default_rng(M + 3 * N + K + act)
    x = wl.to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    w = wl.to_bf16_bits(rng.standard_normal((N, K)).astype(np.float32) * np.float32(0.05))
    b = wl.to_bf16_bits(rng.standard_normal(N).astype(np.float32) * np.float32(0.01))
    y = h_u16(w8.linear_bf16(d_bf16(x), d_bf16(w), d_bf16(b), act=act))
    _check_fallback(y, x, w, b, act=act)


# The tiled BF16 path with a K tail (K even, K % 64 != 0, rows 4-byte aligned):
# the last stage's loads run on into the next row and are masked.  K = 2 is a
# single partial stage; 2048 x 2048 x 2050 is the fallback workload (128 x 128
# tiles, K split between two wave groups, 3-deep ring); 1024 x 2048 x 1026 and
# x 1042 the same tiles on the 2-deep ring with last stages of 4 and 36 bytes
# (the second reaches the other wave group's 32-byte sub-step); 4100 x 4100
# runs 192 x 256 tiles, 3900 x 4032 256 x 256 tiles.
@pytest.mark.parametrize("M,N,K", [(300, 100, 2), (97, 256, 66), (257, 192, 130),
                                   (2048, 2048, 2050), (1024, 2048, 1026), (1024, 2048, 1042),
                                   (4100, 4100, 190), (3900, 4032, 130)])
@pytest.mark.parametrize("act", [w8.ACT_NONE, w8.ACT_GELU_TANH])
def test_fallback_tiled_k_tail(M, N, K, act):
    say(f"fallback tiled K tail M={M} N={N} K={K} act={act}")
    rng = np.random.default_rng(M + 5 * N + K + act)
    x = wl.to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    w = wl.to_bf16_bits(rng.standard_normal((N, K)).astype(np.float32) * np.float32(0.05))
    b = wl.to_bf16_bits(rng.standard_normal(N).astype(np.float32) * np.float32(0.01))
    y = h_u16(w8.linear_bf16(d_bf16(x), d_bf16(w), d_bf16(b), act=act))
    _check_fallback(y, x, w, b, act=act)


@pytest.mark.parametrize("off", [1, 2, 4])
def test_fallback_tiled_store_alignment(off):
    """The 192 x 256 BF16 tiles into an output view offset by `off` elements
    from a 256-byte aligned buffer (N = 4100: rows 8-byte aligned at offset 4,
    4-byte at 2, 2-byte at 1, so each store width is taken); every element of
    the view is checked and the guard elements around it stay untouched."""
    M, N, K = 2378, 4100, 64
    say(f"fallback tiled store alignment off={off}")
    rng = np.random.default_rng(40 + off)
    x = wl.to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    w = wl.to_bf16_bits(rng.standard_normal((N, K)).astype(np.float32) * np.float32(0.05))
    b = wl.to_bf16_bits(rng.standard_normal(N).astype(np.float32) * np.float32(0.01))
    buf = torch.full((M * N + off + 8,), 1234.0, dtype=torch.bfloat16, device=DEV)
    y = buf[off:off + M * N].view(M, N)
    w8.linear_bf16(d_bf16(x), d_bf16(w), d_bf16(b), y=y)
    torch.cuda.synchronize()
    hb = h_u16(buf)
    _check_fallback(hb[off:off + M * N].reshape(M, N), x, w, b)
    guard = np.concatenate([hb[:off], hb[off + M * N:]])
    assert np.all(guard == h_u16(torch.tensor([1234.0], dtype=torch.bfloat16))[0])


def test_fallback_tiled_and_generic_agree_on_offsets():
    """The same product through the tiled kernel (aligned views) and the
    generic one (views offset by one element, 2-byte aligned): both within the
    fallback bar, output rows written exactly once."""
    say("fallback tiled vs generic")
    M, N, K = 257, 192, 128
    rng = np.random.default_rng(11)
    x = wl.to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    w = wl.to_bf16_bits(rng.standard_normal((N, K)).astype(np.float32) * np.float32(0.05))
    xg = torch.zeros(M * K + 1, dtype=torch.bfloat16, device=DEV)
    wg = torch.zeros(N * K + 1, dtype=torch.bfloat16, device=DEV)
    xg[1:] = d_bf16(x).view(-1)
    wg[1:] = d_bf16(w).view(-1)
    y_tiled = h_u16(w8.linear_bf16(d_bf16(x), d_bf16(w)))
    y_generic = h_u16(w8.linear_bf16(xg[1:].view(M, K), wg[1:].view(N, K)))
    zero_b = np.zeros(N, np.uint16)
    _check_fallback(y_tiled, x, w, zero_b)
    _check_fallback(y_generic, x, w, zero_b)


# ---------------------------------------------------------------------------
# compaction
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("B,L,D,kind", [(8, 512, 4096, "prefix"), (3, 50, 16, "random"),
                                       (2, 40, 12, "random"), (4, 33, 64, "none"),
                                       (4, 33, 64, "all"), (0, 16, 64, "none"),
                                       (1, 4096, 8, "random")])
def test_compaction_matches_oracle(B, L, D, kind):
    say(f"compact B={B} L={L} D={D} {kind}")
    rng = np.random.default_rng(B * 1000 + L + D)
    x = wl.to_bf16_bits(rng.standard_normal((B, L, D)).astype(np.float32))
    if kind == "prefix":
        lengths = rng.integers(64, L, B, endpoint=True)
        mask = (np.arange(L)[None, :] < lengths[:, None]).astype(np.uint8)
    elif kind == "random":
        mask = (rng.random((B, L)) < 0.45).astype(np.uint8) * rng.integers(1, 255, (B, L)).astype(np.uint8)
    elif kind == "none":
        mask = np.zeros((B, L), np.uint8)
    else:
        mask = np.ones((B, L), np.uint8)
    sentinel = wl.to_bf16_bits(np.float32([30000.0]))[0]
    x[mask == 0] = sentinel
    cap = max(B * L, 1)
    pad = 1024
    big = torch.full((cap * D + 2 * pad,), 0x1234, dtype=torch.int16, device=DEV)
    out = big[pad:pad + B * L * D].view(torch.bfloat16).view(B * L, D)
    xd = d_bf16(x.reshape(B * L, D)).view(B, L, D) if B * L > 0 else \
        torch.empty((B, L, D), dtype=torch.bfloat16, device=DEV)
    _, src, cnt = w8.compact_padded_rows(xd, torch.from_numpy(mask).to(DEV), out=out)
    n = int(cnt.item())
    o_out, o_src, o_n = oracle.compact_rows(x, mask)
    assert n == o_n
    assert np.array_equal(h(src)[:n], o_src)
    hb = h(big).view(np.uint16)
    got = hb[pad:pad + n * D].reshape(n, D)
    assert np.array_equal(got, o_out)
    assert not np.any(got == sentinel)
    assert np.all(hb[:pad] == 0x1234) and np.all(hb[pad + n * D:] == 0x1234)


def test_compaction_unaligned_mask_and_rows():
    """Mask not 4-byte aligned (prefix counted byte by byte) and x rows not
    16-byte aligned (copied element by element): same result as the oracle."""
    say("compact unaligned mask / rows")
    rng = np.random.default_rng(77)
    B, L, D = 5, 203, 40
    x = wl.to_bf16_bits(rng.standard_normal((B, L, D)).astype(np.float32))
    mask = (rng.random((B, L)) < 0.6).astype(np.uint8)
    mbuf = torch.zeros(B * L + 1, dtype=torch.uint8, device=DEV)
    mbuf[1:] = torch.from_numpy(mask.ravel()).to(DEV)
    xbuf = torch.zeros(B * L * D + 1, dtype=torch.bfloat16, device=DEV)
    xbuf[1:] = d_bf16(x.reshape(-1))
    out, src, cnt = w8.compact_padded_rows(xbuf[1:].view(B, L, D), mbuf[1:].view(B, L))
    n = int(cnt.item())
    o_out, o_src, o_n = oracle.compact_rows(x, mask)
    assert n == o_n
    assert np.array_equal(h(src)[:n], o_src)
    assert np.array_equal(h_u16(out[:n]), o_out)


# Compaction fused with quantisation against the oracle's compaction followed by
# its quantisation: 16-byte path with 8 and 1 chunks per lane, 16 (D = 8192),
# the element path (D % 8 != 0, D > 8192), empty / full masks, no rows at all.
@pytest.mark.parametrize("B,L,D,kind", [(8, 512, 4096, "prefix"), (3, 50, 16, "random"),
                                       (2, 33, 8192, "random"), (2, 40, 12, "random"),
                                       (1, 21, 8200, "random"), (4, 33, 64, "none"),
                                       (4, 33, 64, "all"), (0, 16, 64, "none")])
def test_compact_quantize_matches_oracle(B, L, D, kind):
    say(f"compact+quantise B={B} L={L} D={D} {kind}")
    rng = np.random.default_rng(B * 100 + L + D)
    xf = rng.standard_normal((B, L, D)).astype(np.float32)
    if B * L > 3:
        xf.reshape(-1, D)[1] = 0.0                      # a zero row: scale 0, codes 0
        xf.reshape(-1, D)[2, :: 7] *= 40.0              # outliers
    x = wl.to_bf16_bits(xf)
    if kind == "prefix":
        lengths = rng.integers(64, L, B, endpoint=True)
        mask = (np.arange(L)[None, :] < lengths[:, None]).astype(np.uint8)
    elif kind == "random":
        mask = (rng.random((B, L)) < 0.55).astype(np.uint8) * rng.integers(1, 255, (B, L)).astype(np.uint8)
        if B * L > 3:
            mask.reshape(-1)[1:3] = 1                   # keep the zero and outlier rows
    elif kind == "none":
        mask = np.zeros((B, L), np.uint8)
    else:
        mask = np.ones((B, L), np.uint8)
    xd = d_bf16(x.reshape(B * L, D)).view(B, L, D) if B * L > 0 else \
        torch.empty((B, L, D), dtype=torch.bfloat16, device=DEV)
    q, sc, src, cnt = w8.compact_quantize_rows(xd, torch.from_numpy(mask).to(DEV))
    n = int(cnt.item())
    o_out, o_src, o_n = oracle.compact_rows(x, mask)
    assert n == o_n
    assert np.array_equal(h(src)[:n], o_src)
    if n:
        qo, so = oracle.quantize_rows(o_out)
        assert np.array_equal(h(sc)[:n].view(np.uint32), so.view(np.uint32))
        assert np.array_equal(h(q)[:n], qo)


def test_compact_quantize_unaligned_and_into_gemm():
    """Unaligned mask and rows (word-free prefix, element path), then the text
    path: fused compaction + quantisation, INT8 GEMM on the count rows, equal
    to the guarded linear on the compacted bf16 rows."""
    say("compact+quantise unaligned, then GEMM")
    rng = np.random.default_rng(5)
    B, L, D, N = 3, 70, 256, 128
    x = wl.to_bf16_bits(rng.standard_normal((B, L, D)).astype(np.float32))
    mask = (rng.random((B, L)) < 0.5).astype(np.uint8)
    mbuf = torch.zeros(B * L + 1, dtype=torch.uint8, device=DEV)
    mbuf[1:] = torch.from_numpy(mask.ravel()).to(DEV)
    xbuf = torch.zeros(B * L * D + 1, dtype=torch.bfloat16, device=DEV)
    xbuf[1:] = d_bf16(x.reshape(-1))
    q, sc, src, cnt = w8.compact_quantize_rows(xbuf[1:].view(B, L, D), mbuf[1:].view(B, L))
    n = int(cnt.item())
    o_out, o_src, o_n = oracle.compact_rows(x, mask)
    qo, so = oracle.quantize_rows(o_out)
    assert n == o_n and np.array_equal(h(src)[:n], o_src)
    assert np.array_equal(h(q)[:n], qo) and np.array_equal(h(sc)[:n].view(np.uint32), so.view(np.uint32))
    # aligned input, into the INT8 GEMM
    w = wl.to_bf16_bits(rng.standard_normal((N, D)).astype(np.float32) * np.float32(0.02))
    b = wl.to_bf16_bits(rng.standard_normal(N).astype(np.float32) * np.float32(0.01))
    qw, sw = oracle.quantize_rows(w)
    q2, sc2, _, cnt2 = w8.compact_quantize_rows(d_bf16(x.reshape(B * L, D)).view(B, L, D),
                                                torch.from_numpy(mask).to(DEV))
    n2 = int(cnt2.item())
    y = w8.gemm(q2[:n2], sc2[:n2], d_i8(qw), torch.from_numpy(sw).to(DEV), d_bf16(b))
    ref, path = oracle.w8a8_linear(o_out, w, b)
    assert path == 0                                     # the INT8 path
    assert np.array_equal(h_u16(y), ref)


def test_compaction_commutes_with_linear_on_gpu():
    say("compaction commutes with the linear")
    rng = np.random.default_rng(21)
    B, L, D, N = 4, 160, 512, 192
    x = wl.to_bf16_bits(rng.standard_normal((B, L, D)).astype(np.float32))
    lengths = rng.integers(1, L + 1, B)
    mask = (np.arange(L)[None, :] < lengths[:, None]).astype(np.uint8)
    w = wl.to_bf16_bits(rng.standard_normal((N, D)).astype(np.float32) * np.float32(0.02))
    b = wl.to_bf16_bits(rng.standard_normal(N).astype(np.float32) * np.float32(0.01))
    layer = w8.W8A8Linear.prepare(d_bf16(w), d_bf16(b))
    md = torch.from_numpy(mask).to(DEV)
    xd = d_bf16(x.reshape(B * L, D)).view(B, L, D)
    xc, _, cnt = w8.compact_padded_rows(xd, md)
    n = int(cnt.item())
    y1 = h_u16(layer(xc[:n]))
    yfull = layer(xd.view(B * L, D)).view(B, L, N)
    y2, _, cnt2 = w8.compact_padded_rows(yfull, md)
    assert int(cnt2.item()) == n
    assert np.array_equal(y1, h_u16(y2[:n]))


def _general_mask(rng, R):
    """A general mask: runs of valid and padded rows of random lengths (1 .. 3000),
    nonzero values other than 1, and scattered single flips."""
    m = np.zeros(R, np.uint8)
    i, on = 0, bool(rng.integers(0, 2))
    while i < R:
        n = int(rng.integers(1, 3000))
        if on:
            m[i:i + n] = rng.integers(1, 256, min(n, R - i)).astype(np.uint8)
        i += n
        on = not on
    flips = rng.choice(R, R // 50, replace=False)
    m[flips] = np.where(m[flips] != 0, 0, 7).astype(np.uint8)
    return m


# The linear-time compaction path (more than 8192 rows: chunk counts, chunk
# scans, then the gather), against the oracle: 64 x 8192 rows with a general
# mask on the 16-byte and element paths, all / no rows valid, the first sizes
# past the single-launch path, and an unaligned mask (byte-wise chunk scans).
@pytest.mark.parametrize("B,L,D,kind,mask_off", [
    (64, 8192, 64, "general", 0), (64, 8192, 20, "general", 0), (16, 8192, 8, "all", 0),
    (16, 8192, 8, "none", 0), (1, 8193, 8, "general", 0), (2, 4100, 16, "general", 1),
    (3, 100003, 8, "general", 3), (1, 8192, 8, "general", 0)])
def test_compaction_linear_path_matches_oracle(B, L, D, kind, mask_off):
    say(f"compact linear path B={B} L={L} D={D} {kind} mask offset {mask_off}")
    rng = np.random.default_rng(B + L + D + mask_off)
    R = B * L
    x = wl.to_bf16_bits(rng.standard_normal((R, D)).astype(np.float32))
    mask = {"general": lambda: _general_mask(rng, R), "all": lambda: np.ones(R, np.uint8),
            "none": lambda: np.zeros(R, np.uint8)}[kind]().reshape(B, L)
    mbuf = torch.zeros(R + 16, dtype=torch.uint8, device=DEV)
    mbuf[mask_off:mask_off + R] = torch.from_numpy(mask.ravel()).to(DEV)
    md = mbuf[mask_off:mask_off + R].view(B, L)
    xd = d_bf16(x).view(B, L, D)
    out, src, cnt = w8.compact_padded_rows(xd, md)
    n = int(cnt.item())
    o_out, o_src, o_n = oracle.compact_rows(x.reshape(B, L, D), mask)
    assert n == o_n
    assert np.array_equal(h(src)[:n], o_src)
    assert np.array_equal(h_u16(out[:n]), o_out)
    q, sc, src2, cnt2 = w8.compact_quantize_rows(xd, md)
    assert int(cnt2.item()) == n
    assert np.array_equal(h(src2)[:n], o_src)
    if n:
        qo, so = oracle.quantize_rows(o_out)
        assert np.array_equal(h(sc)[:n].view(np.uint32), so.view(np.uint32))
        assert np.array_equal(h(q)[:n], qo)
