"""Pins of the CPU oracle against things other than itself.

Every check here runs on the CPU.  The oracle follows TurboT2VA's W8A8 recipe
(智猩猩 article, section 01.3 "量化策略") and padded-text compaction (same
section, last paragraph; paperlayer.ai summary, section "C. Fused Multimodal
Transformer Operations").  The pins are: hand-worked fixtures under
``tests/golden/``, exact rational arithmetic (``fractions``), library routines
(numpy int64 matmul, torch's bf16 conversion and GELU), closed forms,
invariants and brute force on tiny inputs.
"""
from __future__ import annotations

import math
import os
from fractions import Fraction as Fr

import numpy as np
import pytest
import torch

import oracle
import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------------------
# Exact rational models of IEEE rounding (independent of the oracle's C code)
# ---------------------------------------------------------------------------

def _round_to_grid(a: Fr, ulp: Fr) -> Fr:
    n = a / ulp
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fr(1, 2) or (rem == Fr(1, 2) and fl % 2 == 1):
        fl += 1
    return fl * ulp


def _exp2_floor(a: Fr) -> int:
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fr(2) ** e > a:
        e -= 1
    while Fr(2) ** (e + 1) <= a:
        e += 1
    return e


def rn(v: Fr, mant_bits: int, emin: int) -> Fr:
    """Round a rational to the nearest binary float with ``mant_bits``
    significant bits and minimum normal exponent ``emin`` (ties to even)."""
    if v == 0:
        return Fr(0)
    s = -1 if v < 0 else 1
    a = abs(v)
    e = max(_exp2_floor(a), emin)
    return s * _round_to_grid(a, Fr(2) ** (e - (mant_bits - 1)))


def rn32(v: Fr) -> Fr:
    return rn(v, 24, -126)


def rnbf16(v: Fr) -> Fr:
    return rn(v, 8, -126)


def rne_int(v: Fr) -> int:
    return int(_round_to_grid(v, Fr(1)))


def bf16_bits_of_value(v: float) -> int:
    """Bits of a value that is exactly a bf16 number."""
    f = np.array([v], np.float32)
    assert float(f[0]) == v
    bits = int(f.view(np.uint32)[0])
    assert bits & 0xFFFF == 0, v
    return bits >> 16


def frac_of_bf16(h: int) -> Fr:
    return Fr(float(np.array([h << 16], np.uint32).view(np.float32)[0]))


def ulp_dist_bf16(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """|ord(a) - ord(b)| for bf16 bit patterns on a monotone integer line (+-0 -> 0)."""
    def ordv(h):
        h = h.astype(np.int64)
        return np.where(h & 0x8000, -(h & 0x7FFF), h & 0x7FFF)
    return np.abs(ordv(a) - ordv(b))


# ---------------------------------------------------------------------------
# bf16 conversions
# ---------------------------------------------------------------------------

def test_bf16_widening_matches_torch_for_all_patterns():
    bits = np.arange(65536, dtype=np.uint16)
    finite = (bits & 0x7F80) != 0x7F80
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().numpy()
    got = np.array([oracle.bf16_to_f32(int(h)) for h in bits[finite]], np.float32)
    assert np.array_equal(got.view(np.uint32), ref[finite].view(np.uint32))


def test_f32_to_bf16_matches_torch_rounding():
    rng = np.random.default_rng(0)
    u = rng.integers(0, 2**32, size=20000, dtype=np.uint64).astype(np.uint32)
    f = u.view(np.float32)
    f = f[np.isfinite(f)]
    # add exact ties and near-ties
    ties = (np.arange(1, 2000, dtype=np.uint32) << 16 | 0x8000).view(np.float32)
    f = np.concatenate([f, ties, -ties, np.float32([0.0, -0.0, 3.3895314e38, 1e-40])])
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([oracle.f32_to_bf16(float(x)) for x in f], np.uint16)
    assert np.array_equal(got, ref)


def test_f64_to_bf16_rounds_once_exactly():
    rng = np.random.default_rng(1)
    vals = list(rng.standard_normal(3000) * np.exp(rng.uniform(-60, 60, 3000)))
    # halfway cases, subnormals, near overflow, and a case where rounding through
    # binary32 first would give a different answer (double rounding)
    vals += [1 + 2**-8, 1 + 2**-8 + 2**-30, -(1 + 3 * 2**-8), 2.0**-130, 3 * 2.0**-134,
             2.0**-133 * 0.5, 2.0**-133 * 0.75, 3.3895313892515355e38, 3.39e38, 1e39, 0.0]
    for v in vals:
        got = oracle.f64_to_bf16(v)
        exp = rnbf16(Fr(v))
        if abs(exp) > Fr(3.3895313892515355e38):
            assert got & 0x7FFF == 0x7F80, v
            continue
        assert frac_of_bf16(got) == exp, (v, hex(got))
    # 1 + 2^-8 + 2^-30 must round up to 1 + 2^-7 (binary32 first would give 1.0)
    assert oracle.f64_to_bf16(1 + 2**-8 + 2**-30) == bf16_bits_of_value(1 + 2**-7)


# ---------------------------------------------------------------------------
# Q: per-row quantisation
# ---------------------------------------------------------------------------

def _parse_vals(field):
    out = []
    for tok in field.split():
        if "*" in tok:
            v, n = tok.split("*")
            out += [float.fromhex(v) if v.startswith(("0x", "-0x")) else float(v)] * int(n)
        else:
            out.append(float.fromhex(tok) if tok.startswith(("0x", "-0x")) else float(tok))
    return out


def _golden_quant_cases():
    cases = []
    with open(os.path.join(GOLDEN, "quantize_rows.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            xs, qs, a = (p.strip() for p in line.split(";"))
            cases.append((_parse_vals(xs), [int(v) for v in _parse_vals(qs)], _parse_vals(a)[0]))
    return cases


@pytest.mark.parametrize("case", _golden_quant_cases(), ids=lambda c: f"n{len(c[0])}")
def test_quantize_hand_worked(case):
    xs, qs, a = case
    x = np.array([[bf16_bits_of_value(v) for v in xs]], np.uint16)
    q, s = oracle.quantize_rows(x)
    assert q[0].tolist() == qs
    exp_s = float(rn32(Fr(a) / 127)) if a >= 2.0**-100 else 0.0
    assert float(s[0]) == exp_s


def _exact_codes(xrow_bits):
    vals = [frac_of_bf16(int(h)) for h in xrow_bits]
    a = max(abs(v) for v in vals)
    if a < Fr(2) ** -100:
        return [0] * len(vals), Fr(0)
    inv = rn32(Fr(127) / a)
    return [max(-127, min(127, rne_int(rn32(v * inv)))) for v in vals], rn32(a / 127)


def test_quantize_matches_exact_rational_model_on_random_rows():
    rng = np.random.default_rng(2)
    rows = []
    for r in range(40):
        scale = np.float32(2.0 ** rng.integers(-60, 60))
        row = rng.standard_normal(24).astype(np.float32) * scale
        if r % 3 == 0:
            row[rng.integers(0, 24)] *= 50
        rows.append(row)
    x = wl.to_bf16_bits(np.stack(rows))
    q, s = oracle.quantize_rows(x)
    for r in range(x.shape[0]):
        codes, sc = _exact_codes(x[r])
        assert q[r].tolist() == codes
        assert Fr(float(s[r])) == sc


def _sweep_rows(exponent):
    """Rows [a, x...] for every bf16 mantissa of a at one binade and every bf16 x
    with |x| <= a in the 9 binades that can give a nonzero code (both signs)."""
    rows = []
    for ma in range(128):
        a_bits = (exponent << 7) | ma
        xs = []
        for e in range(exponent - 8, exponent + 1):
            if e < 1:
                continue
            for m in range(128):
                b = (e << 7) | m
                if b <= a_bits:
                    xs += [b, b | 0x8000]
        row = [a_bits] + xs
        row += [0] * (2304 + 1 - len(row))
        rows.append(row)
    return np.array(rows, np.uint16)


def test_quantize_sweep_matches_numpy_binary32_and_rational_spot_checks():
    """Every (absmax, x) pair that can give a nonzero code, for absmax in three
    binades (including the smallest kept one); numpy binary32 arithmetic as an
    independent evaluator, exact rationals on a random subset."""
    rng = np.random.default_rng(3)
    for exponent in (27, 127, 200):  # 2^-100 binade, [1,2), a large binade
        x = _sweep_rows(exponent)
        q, s = oracle.quantize_rows(x)
        xf = wl.from_bf16_bits(x)
        a = np.abs(xf).max(axis=1)
        s_np = (a / np.float32(127)).astype(np.float32)
        inv = (np.float32(127) / a).astype(np.float32)
        q_np = np.clip(np.rint((xf * inv[:, None]).astype(np.float32)), -127, 127).astype(np.int8)
        assert np.array_equal(s, s_np)
        assert np.array_equal(q, q_np)
        for _ in range(300):
            r = int(rng.integers(0, x.shape[0]))
            c = int(rng.integers(0, x.shape[1]))
            codes, sc = _exact_codes(x[r, [0, c]])
            assert q[r, c] == codes[1]


def _invariants(x_bits, q, s):
    xf = wl.from_bf16_bits(x_bits).astype(np.float64)
    a = np.abs(xf).max(axis=1)
    live = a >= 2.0**-100
    assert np.all(np.abs(q.astype(np.int32)) <= 127)
    assert np.all(q[~live] == 0) and np.all(s[~live] == 0)
    xs, qs, ss = xf[live], q[live].astype(np.float64), s[live].astype(np.float64)
    arg = np.argmax(np.abs(xs), axis=1)
    top = qs[np.arange(len(arg)), arg]
    assert np.all(top == 127 * np.sign(xs[np.arange(len(arg)), arg]))
    err = np.abs(xs - qs * ss[:, None])
    assert np.all(err <= ss[:, None] * (0.5 + 2.0**-15))
    assert np.all((np.sign(qs) == np.sign(xs)) | (qs == 0))
    order = np.argsort(xs, axis=1, kind="stable")
    qsorted = np.take_along_axis(qs, order, axis=1)
    assert np.all(np.diff(qsorted, axis=1) >= 0)


def test_quantize_invariants_on_workload_rows():
    lin = wl.tiny()
    for mat in (lin.x, lin.w):
        q, s = oracle.quantize_rows(mat)
        _invariants(mat, q, s)
    lin = wl.audio(M=128)
    q, s = oracle.quantize_rows(lin.x)
    _invariants(lin.x, q, s)
    rng = np.random.default_rng(4)
    x = wl.to_bf16_bits(rng.standard_normal((64, 300)).astype(np.float32) *
                        np.float32(2.0) ** rng.integers(-90, 90, (64, 1)).astype(np.float32))
    x[5] = 0
    x[6, :] = wl.to_bf16_bits(np.full(300, 2.0**-101, np.float32))
    x[7, :] = wl.to_bf16_bits(np.full(300, -3.0, np.float32))  # all ties for the absmax
    q, s = oracle.quantize_rows(x)
    _invariants(x, q, s)
    assert np.all(q[7] == -127)


def test_quantize_power_of_two_equivariance():
    rng = np.random.default_rng(5)
    base = rng.standard_normal((32, 200)).astype(np.float32)
    x0 = wl.to_bf16_bits(base)
    q0, s0 = oracle.quantize_rows(x0)
    for e in (-40, -7, 1, 13, 60):
        xe = wl.to_bf16_bits(wl.from_bf16_bits(x0) * np.float32(2.0**e))
        qe, se = oracle.quantize_rows(xe)
        assert np.array_equal(qe, q0)
        assert np.array_equal(se, (s0 * np.float32(2.0**e)).astype(np.float32))


def test_quantize_empty_and_single_column():
    q, s = oracle.quantize_rows(np.zeros((0, 16), np.uint16))
    assert q.shape == (0, 16) and s.shape == (0,)
    x = wl.to_bf16_bits(np.array([[3.0], [-0.25], [0.0]], np.float32))
    q, s = oracle.quantize_rows(x)
    assert q[:, 0].tolist() == [127, -127, 0]


# ---------------------------------------------------------------------------
# QB: per-block quantisation of attention Q / K
# ---------------------------------------------------------------------------

def _golden_block_cases():
    cases = []
    with open(os.path.join(GOLDEN, "quantize_blocks.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            dims, xs, qs, a = (p.strip() for p in line.split(";"))
            B, S, H, D, blk = (int(v) for v in dims.split())
            cases.append((B, S, H, D, blk, _parse_vals(xs), [int(v) for v in _parse_vals(qs)],
                          _parse_vals(a)))
    return cases


@pytest.mark.parametrize("case", _golden_block_cases(), ids=lambda c: f"B{c[0]}S{c[1]}H{c[2]}")
def test_quantize_blocks_hand_worked(case):
    B, S, H, D, blk, xs, qs, amax = case
    x = np.array([bf16_bits_of_value(v) for v in xs], np.uint16).reshape(B * S, H * D)
    q, s = oracle.quantize_blocks(x, B, H, blk)
    assert q.reshape(-1).tolist() == qs
    exp = [float(rn32(Fr(a) / 127)) if a >= 2.0**-100 else 0.0 for a in amax]
    assert s.reshape(-1).tolist() == exp


def _blocks_as_rows(x, B, H, blk):
    """Rearranges token rows [B*S, H*D] into one row per (sample, block, head),
    padding each sample with zero tokens to whole blocks.  Plain data movement:
    zeros change neither a block's absmax nor any code, so per-row quantisation
    of these rows is per-block quantisation of x."""
    rows, C = x.shape
    S, D = rows // B, C // H
    nblk = -(-S // blk)
    pad = np.zeros((B, nblk * blk, H, D), x.dtype)
    pad[:, :S] = x.reshape(B, S, H, D)
    return pad.reshape(B, nblk, blk, H, D).transpose(0, 1, 3, 2, 4).reshape(B * nblk * H, blk * D)


def _rows_as_blocks(r, B, S, H, D, blk):
    nblk = -(-S // blk)
    t = r.reshape(B, nblk, H, blk, D).transpose(0, 1, 3, 2, 4).reshape(B, nblk * blk, H, D)
    return t[:, :S].reshape(B * S, H * D)


@pytest.mark.parametrize("B,S,H,D,blk", [(1, 1, 1, 8, 1), (1, 37, 1, 16, 1), (2, 37, 3, 16, 8),
                                         (3, 130, 4, 64, 64), (1, 257, 2, 128, 128),
                                         (2, 5, 2, 8, 16), (1, 96, 8, 32, 32)])
def test_quantize_blocks_reduces_to_per_row_quantisation(B, S, H, D, blk):
    """Per-block quantisation equals the (separately pinned) per-row routine
    applied to each block laid out as one row: pins the block layout, the
    ragged last block of every sample, independence of samples and heads."""
    rng = np.random.default_rng(B * 1000 + S * 10 + H + D + blk)
    v = rng.standard_normal((B * S, H * D)).astype(np.float32)
    v *= np.float32(2.0) ** rng.integers(-60, 60, (B * S, 1)).astype(np.float32)
    x = wl.to_bf16_bits(v)
    if B * S > 3:
        x[B * S // 2, :D] = 0  # a zero token row inside a block
    q, s = oracle.quantize_blocks(x, B, H, blk)
    qr, sr = oracle.quantize_rows(_blocks_as_rows(x, B, H, blk))
    assert np.array_equal(s.reshape(-1), sr)
    assert np.array_equal(q, _rows_as_blocks(qr, B, S, H, D, blk))


def test_quantize_blocks_one_token_blocks_equal_per_row_on_one_head():
    rng = np.random.default_rng(12)
    x = wl.to_bf16_bits(rng.standard_normal((50, 96)).astype(np.float32))
    x[3] = 0
    q, s = oracle.quantize_blocks(x, 1, 1, 1)
    qr, sr = oracle.quantize_rows(x)
    assert np.array_equal(q, qr) and np.array_equal(s.reshape(-1), sr)


def test_quantize_blocks_invariants_and_degenerate_blocks():
    rng = np.random.default_rng(13)
    B, S, H, D, blk = 2, 70, 4, 16, 32
    x = wl.to_bf16_bits(rng.standard_normal((B * S, H * D)).astype(np.float32))
    x[:32, 16:32] = 0          # sample 0, block 0, head 1: all zero
    x[S:S + 32, :16] = wl.to_bf16_bits(np.full((32, 16), 2.0**-101, np.float32))  # below 2^-100
    q, s = oracle.quantize_blocks(x, B, H, blk)
    assert s[0, 0, 1] == 0 and s[1, 0, 0] == 0
    rows = _blocks_as_rows(x, B, H, blk)
    _invariants(rows, _blocks_as_rows(q, B, H, blk), s.reshape(-1))


def test_quantize_blocks_empty():
    q, s = oracle.quantize_blocks(np.zeros((0, 32), np.uint16), 1, 2, 64)
    assert q.shape == (0, 32) and s.shape == (1, 0, 2)


# ---------------------------------------------------------------------------
# I: INT32 product
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("M,N,K", [(1, 1, 1), (7, 5, 1), (13, 17, 127), (64, 128, 256),
                                   (33, 65, 257), (3, 300, 131)])
def test_gemm_matches_numpy_int64(M, N, K):
    rng = np.random.default_rng(M * 1000 + N + K)
    a = rng.integers(-127, 128, (M, K), dtype=np.int8)
    w = rng.integers(-127, 128, (N, K), dtype=np.int8)
    acc = oracle.gemm_i32(a, w)
    assert np.array_equal(acc.astype(np.int64), a.astype(np.int64) @ w.astype(np.int64).T)


def test_gemm_closed_forms():
    K = 4096
    a = np.full((4, K), 127, np.int8)
    assert np.all(oracle.gemm_i32(a, a) == 16129 * K)
    assert np.all(oracle.gemm_i32(a, -a) == -16129 * K)
    rng = np.random.default_rng(6)
    u = rng.integers(-127, 128, (9, 1), dtype=np.int8)
    v = rng.integers(-127, 128, (11, 1), dtype=np.int8)
    assert np.array_equal(oracle.gemm_i32(u, v), u.astype(np.int32) * v.astype(np.int32).T)
    K = 48
    eye = (127 * np.eye(K)).astype(np.int8)
    w = rng.integers(-127, 128, (20, K), dtype=np.int8)
    assert np.array_equal(oracle.gemm_i32(eye, w), 127 * w.astype(np.int32).T)
    # largest K the guard admits does not overflow int32
    K = 131072
    a = np.full((1, K), -127, np.int8)
    assert int(oracle.gemm_i32(a, a)[0, 0]) == 16129 * K
    assert int(oracle.gemm_i32(a, -a)[0, 0]) == -16129 * K


# ---------------------------------------------------------------------------
# E: epilogue
# ---------------------------------------------------------------------------

def _golden_epi_cases():
    cases = []
    with open(os.path.join(GOLDEN, "epilogue.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            acc, sa, sw, b, y = (p.strip() for p in line.split(";"))
            fh = lambda t: float.fromhex(t) if "0x" in t else float(t)
            cases.append((int(acc), fh(sa), fh(sw), None if b == "none" else fh(b), fh(y)))
    return cases


@pytest.mark.parametrize("case", _golden_epi_cases(), ids=lambda c: str(c[0]))
def test_epilogue_hand_worked(case):
    acc, sa, sw, b, y = case
    bias = np.array([bf16_bits_of_value(b)], np.uint16) if b is not None else None
    out = oracle.epilogue(np.array([[acc]], np.int32), np.float32([sa]), np.float32([sw]), bias)
    assert int(out[0, 0]) == bf16_bits_of_value(y)


def test_epilogue_power_of_two_scales_against_exact_rationals():
    rng = np.random.default_rng(7)
    M, N = 16, 24
    acc = rng.integers(-2**22, 2**22, (M, N)).astype(np.int32)
    sa = np.float32(2.0) ** rng.integers(-20, -5, M).astype(np.float32)
    sw = np.float32(2.0) ** rng.integers(-12, 0, N).astype(np.float32)
    b = wl.to_bf16_bits(rng.standard_normal(N).astype(np.float32))
    y = oracle.epilogue(acc, sa, sw, b)
    for i in range(M):
        for j in range(N):
            v = Fr(int(acc[i, j])) * Fr(float(sa[i])) * Fr(float(sw[j])) + frac_of_bf16(int(b[j]))
            assert frac_of_bf16(int(y[i, j])) == rnbf16(rn32(v)), (i, j)


def test_epilogue_within_binary32_error_bound_of_exact_value():
    """fp64 check: |y - exact| <= half a bf16 ulp + the binary32 sequence's bound."""
    lin = wl.tiny()
    qx, sx = oracle.quantize_rows(lin.x)
    qw, sw = oracle.quantize_rows(lin.w)
    acc = oracle.gemm_i32(qx, qw)
    y = oracle.epilogue(acc, sx, sw, lin.bias)
    t = acc.astype(np.float64)
    uexact = sx.astype(np.float64)[:, None] * sw.astype(np.float64)[None, :]
    vexact = t * uexact + wl.from_bf16_bits(lin.bias).astype(np.float64)[None, :]
    yf = wl.from_bf16_bits(y).astype(np.float64)
    ulp = np.ldexp(1.0, np.frexp(np.abs(yf))[1] - 8)
    bound = ulp / 2 + (np.abs(t * uexact) + np.abs(vexact)) * 2.0**-23 + 1e-30
    assert np.all(np.abs(yf - vexact) <= bound)


def test_integer_inputs_reduce_to_integer_matmul():
    """X with integer entries and +-127 in every row quantises to s = 1, q = X,
    so the layer is bf16(fma(X . qW^T, sW, b)) with an ordinary integer matmul."""
    rng = np.random.default_rng(8)
    M, N, K = 8, 12, 40
    x = rng.integers(-126, 127, (M, K)).astype(np.float32)
    x[np.arange(M), rng.integers(0, K, M)] = 127 * rng.choice([-1, 1], M)
    xb = wl.to_bf16_bits(x)  # integers up to 127 are exact in bf16
    qx, sx = oracle.quantize_rows(xb)
    assert np.all(sx == 1.0) and np.array_equal(qx.astype(np.float32), x)
    w = wl.to_bf16_bits(rng.standard_normal((N, K)).astype(np.float32) * np.float32(0.02))
    b = wl.to_bf16_bits(rng.standard_normal(N).astype(np.float32) * np.float32(0.01))
    qw, sw = oracle.quantize_rows(w)
    accnp = x.astype(np.int64) @ qw.astype(np.int64).T
    y2 = oracle.epilogue(oracle.gemm_i32(qx, qw), sx, sw, b)
    for i in range(M):
        for j in range(N):
            v = Fr(int(accnp[i, j])) * Fr(float(sw[j])) + frac_of_bf16(int(b[j]))
            assert frac_of_bf16(int(y2[i, j])) == rnbf16(rn32(v))


# ---------------------------------------------------------------------------
# GELU-tanh
# ---------------------------------------------------------------------------

def test_gelu_matches_tanh_form_and_identities():
    c = math.sqrt(2 / math.pi)
    for z in np.linspace(-3, 3, 601):
        z = float(z)
        ref = 0.5 * z * (1 + math.tanh(c * (z + 0.044715 * z**3)))
        assert abs(oracle.gelu_tanh_f64(z) - ref) <= 1e-15 * max(1.0, abs(z))
    for z in np.concatenate([np.linspace(-12, 12, 481), [1e-6, 0.3, 7.5]]):
        z = float(z)
        assert abs(oracle.gelu_tanh_f64(z) - oracle.gelu_tanh_f64(-z) - z) <= 4e-16 * max(1, abs(z))
    assert oracle.gelu_tanh_f64(0.0) == 0.0
    assert oracle.gelu_tanh_f64(10.0) == 10.0
    # series at 0: g(z) = z/2 + c z^2/2 + (0.044715 c/2 - c^3/6) z^4 + O(z^6)
    z = 1e-4
    series = z / 2 + c * z * z / 2 + (0.044715 * c / 2 - c**3 / 6) * z**4
    assert abs(oracle.gelu_tanh_f64(z) - series) <= 1e-20
    # deep negative tail keeps relative accuracy: g(z) ~ z * exp(2u)
    z = -9.0
    u = c * (z + 0.044715 * z**3)
    assert abs(oracle.gelu_tanh_f64(z) / (z * math.exp(2 * u)) - 1) < 1e-12


def test_gelu_bf16_matches_torch_tanh_gelu():
    bits = np.arange(65536, dtype=np.uint16)
    f = wl.from_bf16_bits(bits).astype(np.float64)
    sel = np.isfinite(f) & (np.abs(f) <= 4.0) & (np.abs(f) >= 2.0**-60)
    bits, f = bits[sel], f[sel]
    ref = torch.nn.functional.gelu(torch.from_numpy(f), approximate="tanh").numpy()
    exp = np.array([oracle.f64_to_bf16(float(v)) for v in ref], np.uint16)
    got = np.array([oracle.gelu_bf16(int(h)) for h in bits], np.uint16)
    # torch evaluates 1 + tanh(.) directly; allow the last bit where that loses accuracy
    assert np.max(ulp_dist_bf16(got, exp)) <= 1
    assert np.mean(got == exp) > 0.999


# ---------------------------------------------------------------------------
# F: BF16 fallback
# ---------------------------------------------------------------------------

def test_fallback_matches_exact_sum_on_tiny_shapes():
    rng = np.random.default_rng(9)
    for (M, N, K) in [(3, 5, 7), (4, 3, 33), (1, 1, 1)]:
        x = wl.to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
        w = wl.to_bf16_bits(rng.standard_normal((N, K)).astype(np.float32) * np.float32(0.02))
        b = wl.to_bf16_bits(rng.standard_normal(N).astype(np.float32) * np.float32(0.01))
        y = oracle.linear_bf16(x, w, b)
        for i in range(M):
            for j in range(N):
                v = sum(frac_of_bf16(int(x[i, k])) * frac_of_bf16(int(w[j, k])) for k in range(K))
                v += frac_of_bf16(int(b[j]))
                assert frac_of_bf16(int(y[i, j])) == rnbf16(v)


def test_fallback_within_summation_bound_against_torch_float64():
    lin = wl.tiny()
    y = oracle.linear_bf16(lin.x, lin.w, lin.bias)
    xf = torch.from_numpy(wl.from_bf16_bits(lin.x).astype(np.float64))
    wf = torch.from_numpy(wl.from_bf16_bits(lin.w).astype(np.float64))
    bf = torch.from_numpy(wl.from_bf16_bits(lin.bias).astype(np.float64))
    ref = (xf @ wf.T + bf).numpy()
    exp = np.array([oracle.f64_to_bf16(float(v)) for v in ref.ravel()], np.uint16).reshape(ref.shape)
    assert np.max(ulp_dist_bf16(y, exp)) <= 1
    assert np.mean(y == exp) > 0.999


# ---------------------------------------------------------------------------
# G: guard and routing
# ---------------------------------------------------------------------------

def test_guard_truth_table():
    for N in (64, 128, 2048, 4096, 16384):
        for K in (128, 256, 2048, 4096, 16384, 131072):
            assert oracle.guard(N, K), (N, K)
    for N, K in [(4100, 4096), (2048, 2050), (32, 4096), (0, 4096), (4096, 0), (4096, 64),
                 (4096, 131072 + 128), (100, 256), (128, 200)]:
        assert not oracle.guard(N, K), (N, K)


def test_linear_routes_nonconforming_shapes_to_bf16():
    rng = np.random.default_rng(10)
    for (M, N, K) in [(5, 68, 256), (6, 64, 130)]:
        x = wl.to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
        w = wl.to_bf16_bits(rng.standard_normal((N, K)).astype(np.float32) * np.float32(0.02))
        b = wl.to_bf16_bits(rng.standard_normal(N).astype(np.float32) * np.float32(0.01))
        y, path = oracle.w8a8_linear(x, w, b)
        assert path == 1
        assert np.array_equal(y, oracle.linear_bf16(x, w, b))


def test_linear_int8_path_is_quantise_gemm_epilogue():
    lin = wl.tiny()
    y, path = oracle.w8a8_linear(lin.x, lin.w, lin.bias)
    assert path == 0
    qx, sx = oracle.quantize_rows(lin.x)
    qw, sw = oracle.quantize_rows(lin.w)
    acc = qx.astype(np.int64) @ qw.astype(np.int64).T
    y2 = oracle.epilogue(acc.astype(np.int32), sx, sw, lin.bias)
    assert np.array_equal(y, y2)


def test_w8a8_close_to_bf16_linear_within_quantisation_bound():
    """|y_w8a8 - y_exact| <= sum_k(|x||dw| + |dx||w^|) + rounding, with
    |dx| <= sx (1/2 + 2^-15) and |dw| <= sw (1/2 + 2^-15)."""
    lin = wl.tiny()
    y, _ = oracle.w8a8_linear(lin.x, lin.w, lin.bias)
    x = wl.from_bf16_bits(lin.x).astype(np.float64)
    w = wl.from_bf16_bits(lin.w).astype(np.float64)
    b = wl.from_bf16_bits(lin.bias).astype(np.float64)
    _, sx = oracle.quantize_rows(lin.x)
    qw, sw = oracle.quantize_rows(lin.w)
    what = qw.astype(np.float64) * sw.astype(np.float64)[:, None]
    exact = x @ w.T + b
    c = 0.5 + 2.0**-15
    bound = (np.abs(x).sum(axis=1)[:, None] * sw.astype(np.float64)[None, :] * c
             + sx.astype(np.float64)[:, None] * c * np.abs(what).sum(axis=1)[None, :])
    yf = wl.from_bf16_bits(y).astype(np.float64)
    tol = bound + np.abs(exact) * 2.0**-7 + 1e-6
    assert np.all(np.abs(yf - exact) <= tol)


# ---------------------------------------------------------------------------
# C: compaction
# ---------------------------------------------------------------------------

def test_compaction_prefix_masks():
    g = wl.guarded_mixed(B=8, L=64, D=32)
    # lengths in the workload are drawn for L = 64 here; rebuild a prefix mask
    lengths = np.array([1, 64, 17, 0, 33, 5, 64, 2])
    mask = (np.arange(64)[None, :] < lengths[:, None]).astype(np.uint8)
    out, src, n = oracle.compact_rows(g.x, mask)
    assert n == int(lengths.sum())
    assert np.all(np.diff(src) > 0)
    flat = g.x.reshape(-1, 32)
    assert np.array_equal(out, flat[src])
    exp_src = np.concatenate([b * 64 + np.arange(l) for b, l in enumerate(lengths)])
    assert np.array_equal(src, exp_src)


def test_compaction_general_mask_sentinels_and_edges():
    rng = np.random.default_rng(11)
    B, L, D = 3, 50, 16
    x = wl.to_bf16_bits(rng.standard_normal((B, L, D)).astype(np.float32))
    mask = (rng.random((B, L)) < 0.4).astype(np.uint8)
    mask[1] *= 7  # any nonzero byte means valid
    sentinel = wl.to_bf16_bits(np.float32([30000.0]))[0]
    x[mask == 0] = sentinel
    out, src, n = oracle.compact_rows(x, mask)
    assert n == int((mask != 0).sum())
    assert not np.any(out == sentinel)
    assert sorted(src.tolist()) == src.tolist()
    out, src, n = oracle.compact_rows(x, np.zeros((B, L), np.uint8))
    assert n == 0 and out.shape == (0, D)
    out, src, n = oracle.compact_rows(x, np.ones((B, L), np.uint8))
    assert n == B * L and np.array_equal(out, x.reshape(-1, D))
    out, src, n = oracle.compact_rows(np.zeros((0, 4, D), np.uint16), np.zeros((0, 4), np.uint8))
    assert n == 0


def test_compaction_commutes_with_the_linear():
    """Quantisation and the product are row-local, so compacting before the
    linear equals compacting its output."""
    rng = np.random.default_rng(12)
    B, L, D, N = 4, 40, 256, 64
    x = wl.to_bf16_bits(rng.standard_normal((B, L, D)).astype(np.float32))
    lengths = rng.integers(1, L + 1, B)
    mask = (np.arange(L)[None, :] < lengths[:, None]).astype(np.uint8)
    w = wl.to_bf16_bits(rng.standard_normal((N, D)).astype(np.float32) * np.float32(0.02))
    b = wl.to_bf16_bits(rng.standard_normal(N).astype(np.float32) * np.float32(0.01))
    xc, src, n = oracle.compact_rows(x, mask)
    y1, p1 = oracle.w8a8_linear(xc, w, b)
    yfull, p2 = oracle.w8a8_linear(x.reshape(-1, D), w, b)
    assert p1 == p2 == 0
    y2, _, _ = oracle.compact_rows(yfull.reshape(B, L, N), mask)
    assert np.array_equal(y1, y2)


# ---------------------------------------------------------------------------
# Workloads: shapes and recipe
# ---------------------------------------------------------------------------

def test_workload_recipe_shapes_and_outliers():
    lin = wl.tiny()
    assert lin.x.shape == (64, 256) and lin.w.shape == (128, 256) and lin.bias.shape == (128,)
    assert len(lin.outlier_cols) == 4
    xf = wl.from_bf16_bits(lin.x)
    col_std = xf.std(axis=0)
    assert np.all(col_std[lin.outlier_cols] > 10) and np.median(col_std) < 1.5
    # deterministic
    assert np.array_equal(wl.tiny().x, lin.x)
    g = wl.guarded_mixed(B=8, L=512, D=8)
    assert np.all((g.lengths >= 64) & (g.lengths <= 512))
    assert np.array_equal(g.mask.sum(axis=1), g.lengths)


# ---------------------------------------------------------------------------
# NM: normalisation + modulation ahead of a linear layer (paperlayer.ai
# summary, section C names the fused operators; formulas are readings)
# ---------------------------------------------------------------------------

def _golden_nm_cases():
    cases = []
    for ln in open(os.path.join(GOLDEN, "norm_mod.txt"), encoding="utf-8"):
        ln = ln.strip()
        if not ln or ln.startswith("#"):
            continue
        head, xs, sc, sh, ys = [p.strip() for p in ln.split(";")]
        norm, eps, rpc, D = head.split()
        vals = lambda t: None if t == "-" else [float(v) for v in t.split()]
        cases.append((oracle.NORM_LAYER if norm == "LN" else oracle.NORM_RMS, float(eps), int(rpc),
                      int(D), vals(xs), vals(sc), vals(sh), vals(ys)))
    return cases


def _bits(vals, D):
    return None if vals is None else np.array([bf16_bits_of_value(v) for v in vals],
                                              np.uint16).reshape(-1, D)


@pytest.mark.parametrize("case", _golden_nm_cases(), ids=lambda c: f"n{c[0]}e{c[1]}r{c[2]}")
def test_norm_mod_hand_worked(case):
    norm, eps, rpc, D, xs, sc, sh, ys = case
    z = oracle.norm_mod_bf16(_bits(xs, D), _bits(sh, D), _bits(sc, D), rpc, norm, eps)
    assert z.reshape(-1).tolist() == [bf16_bits_of_value(v) for v in ys]


def _f64_to_bf16_value(v: np.ndarray) -> np.ndarray:
    """Nearest bf16 value (ties to even) of float64 values in bf16's normal
    range, by scaling each to its 8-bit grid and numpy's rint."""
    m, e = np.frexp(np.abs(v))
    r = np.ldexp(np.rint(np.ldexp(np.abs(v), 8 - e)), e - 8)
    return np.where(v == 0, 0.0, np.copysign(r, v))


def _tie_distance(v: np.ndarray) -> np.ndarray:
    """Distance of |v| from the nearest bf16 rounding boundary (0 on a tie)."""
    m, e = np.frexp(np.abs(v))
    f = np.ldexp(np.abs(v), 8 - e)
    return np.ldexp(np.abs(np.abs(f - np.floor(f)) - 0.5), e - 8)


@pytest.mark.parametrize("norm", [oracle.NORM_LAYER, oracle.NORM_RMS])
@pytest.mark.parametrize("R,D,rpc", [(7, 64, 7), (40, 256, 8), (9, 4096, 3)])
def test_norm_mod_matches_torch_layer_and_rms_norm(norm, R, D, rpc):
    """Reduces to library routines: torch's float64 layer_norm / rms_norm (no
    affine) give y; the modulation y * (1 + scale) + shift is then one float64
    multiply-add.  The oracle evaluates the same formula in binary64 (its sums in
    index order, torch's in its own), so the two agree after rounding to bf16
    wherever the float64 values sit more than a few binary64 ulps of |y (1 + scale)|
    and |z| away from a bf16 rounding boundary: all but a vanishing fraction."""
    rng = np.random.default_rng(R * D + norm)
    x = wl.to_bf16_bits(rng.standard_normal((R, D)).astype(np.float32) * np.float32(3.0) + 0.5)
    G = -(-R // rpc)
    sc = wl.to_bf16_bits(rng.standard_normal((G, D)).astype(np.float32) * np.float32(0.3))
    sh = wl.to_bf16_bits(rng.standard_normal((G, D)).astype(np.float32) * np.float32(0.3))
    eps = 1e-6
    z = oracle.norm_mod_bf16(x, sh, sc, rpc, norm, eps)
    xt = torch.from_numpy((x.astype(np.uint32) << 16).view(np.float32)).double()
    if norm == oracle.NORM_LAYER:
        y = torch.nn.functional.layer_norm(xt, (D,), eps=eps)
    else:
        y = torch.nn.functional.rms_norm(xt, (D,), eps=eps)
    g = np.arange(R) // rpc
    f = lambda b: (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    prod = y.numpy() * (1.0 + f(sc)[g])
    ref = prod + f(sh)[g]
    got = f(z)
    # both sides are binary64: they differ by a few 2^-53 of |y (1 + scale)| and
    # of |z| (the row sums' order and the statistics' roundings included)
    clear = _tie_distance(ref) > 2.0 ** -44 * (np.abs(prod) + np.abs(ref))
    assert clear.mean() > 0.99999
    assert np.array_equal(got[clear], _f64_to_bf16_value(ref)[clear])


@pytest.mark.parametrize("norm", [oracle.NORM_LAYER, oracle.NORM_RMS])
def test_norm_mod_power_of_two_invariance(norm):
    """With eps = 0, scaling a row by 2^k scales its mean and standard deviation
    by 2^k exactly (binary64 sums, division and square root are exact under
    power-of-two scaling), so the normalised row is bit-identical."""
    rng = np.random.default_rng(31 + norm)
    v = rng.standard_normal((12, 96)).astype(np.float32)
    sc = wl.to_bf16_bits(rng.standard_normal((1, 96)).astype(np.float32) * np.float32(0.5))
    sh = wl.to_bf16_bits(rng.standard_normal((1, 96)).astype(np.float32) * np.float32(0.5))
    z0 = oracle.norm_mod_bf16(wl.to_bf16_bits(v), sh, sc, 12, norm, 0.0)
    for k in (-40, -3, 1, 7, 60):
        zk = oracle.norm_mod_bf16(wl.to_bf16_bits(v * np.float32(2.0 ** k)), sh, sc, 12, norm, 0.0)
        assert np.array_equal(zk, z0), k


def test_norm_mod_statistics_of_the_output():
    """Without modulation a LayerNorm row has mean ~0 and variance ~1, an RMSNorm
    row mean square ~1 (to the bf16 rounding of each element)."""
    rng = np.random.default_rng(5)
    x = wl.to_bf16_bits(rng.standard_normal((16, 1024)).astype(np.float32) * np.float32(7.0) + 2.0)
    f = lambda b: (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    z = f(oracle.norm_mod_bf16(x, norm=oracle.NORM_LAYER, eps=0.0))
    assert np.all(np.abs(z.mean(axis=1)) < 2.0 ** -8)
    assert np.all(np.abs(z.var(axis=1) - 1.0) < 2.0 ** -7)
    z = f(oracle.norm_mod_bf16(x, norm=oracle.NORM_RMS, eps=0.0))
    assert np.all(np.abs((z * z).mean(axis=1) - 1.0) < 2.0 ** -7)


def test_norm_mod_quantize_is_quantisation_of_the_bf16_rows_and_degenerate_inputs():
    rng = np.random.default_rng(6)
    x = wl.to_bf16_bits(rng.standard_normal((10, 64)).astype(np.float32))
    x[4] = x[4, 0]  # constant row: normalises to 0, quantises to scale 0
    q, s = oracle.norm_mod_quantize_rows(x, eps=0.0)
    z = oracle.norm_mod_bf16(x, eps=0.0)
    qr, sr = oracle.quantize_rows(z)
    assert np.array_equal(q, qr) and np.array_equal(s, sr)
    assert s[4] == 0 and not q[4].any()
    e = oracle.norm_mod_bf16(np.zeros((0, 64), np.uint16))
    assert e.shape == (0, 64)
    with pytest.raises(RuntimeError):
        oracle.norm_mod_bf16(x, eps=-1.0)
