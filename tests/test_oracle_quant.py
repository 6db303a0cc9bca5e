"""Pins for the oracle's rounding, binary16 and quantizer arithmetic.

Each test checks the oracle against something other than itself: values the fak
MODEL-BASELINE-RESULTS page prints (ACT 4 "Correctness"), exact rational
arithmetic (Python ``fractions``), an independent formulation of the rounding
(truncate + exact fractional part, as the page's AVX-512 quantizer does it,
ACT 5 "What moved" item 3), numpy's binary16 conversion, and invariants that
the definition d = maxabs/127 implies (ACT 3 "How it was closed" item 1).
"""
import bisect
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import workloads as wl

GOLD = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- rounding

def test_rhaway_printed_pins():
    with open(os.path.join(GOLD, "rounding_pins.json")) as f:
        pins = json.load(f)["cases"]
    for c in pins:
        t = np.float32(c["t"])
        assert oracle.rhaway(float(t)) == c["rhaway"], c
        if "naive_add_half_trunc" in c:
            # the rejected form really does give 1 in fp32
            naive = int(np.float32(t + np.float32(0.5)))
            assert naive == c["naive_add_half_trunc"]


def _rhaway_trunc_frac(t: np.ndarray) -> np.ndarray:
    """Independent formulation: truncate, recover the exact fractional part in
    fp32 (t - trunc(t) is exact for floats), step one away from zero when the
    fraction is at least one half."""
    tr = np.trunc(t)
    fr = np.abs(t - tr)
    step = (fr >= np.float32(0.5)).astype(np.float32) * np.sign(t)
    return (tr + step).astype(np.int32)


def test_rhaway_exhaustive_nonnegative_code_range():
    """Every fp32 value in [0, 128] (1,124,073,473 values, denormals included)."""
    last = np.uint32(0x43000000)          # 128.0f
    chunk = 1 << 24
    start = 0
    while start <= int(last):
        stop = min(int(last) + 1, start + chunk)
        bits = np.arange(start, stop, dtype=np.uint32)
        t = bits.view(np.float32)
        got = oracle.rhaway_array(t)
        want = _rhaway_trunc_frac(t)
        bad = np.nonzero(got != want)[0]
        assert bad.size == 0, (t[bad[:5]], got[bad[:5]], want[bad[:5]])
        start = stop


def test_rhaway_sign_symmetry_sample():
    g = wl.rng(5)
    bits = g.integers(0, 0x43000001, size=1 << 20, dtype=np.uint32)
    t = bits.view(np.float32)
    assert np.array_equal(oracle.rhaway_array(-t), -oracle.rhaway_array(t))


def test_rhaway_exact_rational_sample():
    g = wl.rng(6)
    t = (g.standard_normal(4000) * 40).astype(np.float32)
    halves = (np.arange(-255, 256) * 0.5).astype(np.float32)
    nexts = np.nextafter(halves, np.float32(np.inf))
    prevs = np.nextafter(halves, np.float32(-np.inf))
    got = oracle.rhaway_array(np.concatenate([t, halves, nexts, prevs]))
    for v, r in zip(np.concatenate([t, halves, nexts, prevs]), got):
        fv = Fraction(float(v))
        want = math.floor(abs(fv) + Fraction(1, 2))
        want = -want if fv < 0 else want
        assert r == want, (float(v), r, want)


# ---------------------------------------------------------------- binary16

def test_half_to_double_matches_numpy_all_patterns():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([oracle.half_to_float(int(b)) for b in bits])
    finite = np.isfinite(ref)
    assert np.array_equal(got[finite], ref[finite])
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    assert np.array_equal(np.isinf(got), np.isinf(ref))


_POS_HALVES = None


def _pos_halves():
    global _POS_HALVES
    if _POS_HALVES is None:
        b = np.arange(0, 0x7C00, dtype=np.uint16)      # +0 .. largest finite
        _POS_HALVES = [Fraction(float(v)) for v in b.view(np.float16).astype(np.float64)]
    return _POS_HALVES


def _nearest_half_bits(v: Fraction) -> int:
    """Brute force over all non-negative finite binary16 values (sorted by
    value, so by bit pattern): nearest, ties to the even bit pattern."""
    hs = _pos_halves()
    i = bisect.bisect_left(hs, v)
    cands = [j for j in (i - 1, i) if 0 <= j < len(hs)]
    best = min(cands, key=lambda j: (abs(hs[j] - v), j & 1))
    return best


def test_half_from_double_vs_brute_force():
    g = wl.rng(7)
    vals = list(np.abs(g.standard_normal(300) * 0.02 / 127).astype(np.float32))
    vals += list(np.abs(g.standard_normal(200)).astype(np.float32) * np.float32(1000))
    vals += [np.float32(2.0 ** -24), np.float32(2.0 ** -25), np.float32(3 * 2.0 ** -26),
             np.float32(2.0 ** -14), np.float32(65504.0), np.float32(1e-9)]
    hs = _pos_halves()
    # exact midpoints between neighbouring binary16 values (ties go to even)
    for j in range(1, len(hs), 97):
        vals.append(np.float32(float((hs[j - 1] + hs[j]) / 2)))
    for v in vals:
        assert oracle.half_from_float(float(v)) == _nearest_half_bits(Fraction(float(v))), v


def test_half_from_double_matches_numpy_dense():
    g = wl.rng(8)
    bits = g.integers(0, 0x477FE000, size=1 << 18, dtype=np.uint32)   # [0, 65504]
    f = bits.view(np.float32)
    ref = f.astype(np.float16).view(np.uint16)
    got = np.array([oracle.half_from_float(float(v)) for v in f], dtype=np.uint16)
    assert np.array_equal(got, ref)


# ---------------------------------------------------------------- block scale

def test_block_scale_equals_exact_rounding_of_amax_over_127():
    g = wl.rng(9)
    amaxes = list(np.abs(g.standard_normal(400) * 0.06).astype(np.float32))
    amaxes += list(np.abs(g.standard_normal(100) * 4).astype(np.float32))
    hs = _pos_halves()
    # adversarial: amax = 127 * (binary16 midpoint), an exact tie after division
    for j in range(2000, len(hs), 331):
        mid = (hs[j - 1] + hs[j]) / 2
        a = np.float32(float(mid * 127))
        if Fraction(float(a)) == mid * 127:
            amaxes.append(a)
    for a in amaxes:
        want = _nearest_half_bits(Fraction(float(a)) / 127)
        assert oracle.block_scale(float(a)) == want, a


# ---------------------------------------------------------------- codes

def _exact_codes(block: np.ndarray, s_bits: int):
    s = Fraction(float(np.uint16(s_bits).view(np.float16)))
    out = []
    for w in block:
        if s == 0:
            out.append(0)
            continue
        t = Fraction(float(w)) / s
        r = math.floor(abs(t) + Fraction(1, 2))
        r = -r if t < 0 else r
        out.append(max(-127, min(127, r)))
    return out


def _argmin_codes(block: np.ndarray, s_bits: int):
    """Brute force: the code c in [-127, 127] minimising |w - c*s| exactly,
    ties to the larger |c|."""
    s = Fraction(float(np.uint16(s_bits).view(np.float16)))
    out = []
    for w in block:
        fw = Fraction(float(w))
        if s == 0:
            out.append(0)
            continue
        out.append(min(range(-127, 128), key=lambda c: (abs(fw - c * s), -abs(c))))
    return out


def _mixed_blocks(seed: int, nblocks: int) -> np.ndarray:
    g = wl.rng(seed)
    rows = []
    for i in range(nblocks):
        kind = i % 6
        if kind == 0:
            b = g.standard_normal(32) * 0.02
        elif kind == 1:
            b = g.standard_normal(32)
        elif kind == 2:       # wide dynamic range
            b = g.standard_normal(32) * np.exp2(g.integers(-30, 10, size=32))
        elif kind == 3:       # tiny: binary16-subnormal or zero scale
            b = g.standard_normal(32) * 10.0 ** g.integers(-9, -3)
        elif kind == 4:       # zeros and negative zeros
            b = np.where(g.integers(0, 2, size=32) == 0, -0.0, 0.0)
        else:                 # exact halves of a power-of-two scale
            e = int(g.integers(-6, 4))
            b = (g.integers(0, 127, size=32) + 0.5) * 2.0 ** e * np.where(g.integers(0, 2, size=32) == 0, -1, 1)
            b[int(g.integers(0, 32))] = 127 * 2.0 ** e
        rows.append(np.asarray(b, dtype=np.float32))
    return np.concatenate(rows).reshape(1, -1)


def test_quantize_f32_exact_rational():
    w = _mixed_blocks(10, 600)
    q, d = oracle.quantize_f32(w)
    for b in range(w.shape[1] // 32):
        blk = w[0, 32 * b:32 * b + 32]
        amax = Fraction(float(np.max(np.abs(blk))))
        assert d[0, b] == _nearest_half_bits(amax / 127), b
        assert list(q[0, 32 * b:32 * b + 32]) == _exact_codes(blk, int(d[0, b])), b


def test_quantize_f32_argmin_brute_force():
    w = _mixed_blocks(11, 36)
    q, d = oracle.quantize_f32(w)
    for b in range(w.shape[1] // 32):
        blk = w[0, 32 * b:32 * b + 32]
        assert list(q[0, 32 * b:32 * b + 32]) == _argmin_codes(blk, int(d[0, b])), b


def test_quantize_invariants_normal_weights():
    w = wl.normal_weights(12, 2048, 1536)
    q, d = oracle.quantize_f32(w)
    s = d.view(np.float16).astype(np.float64)
    nb = w.shape[1] // 32
    wb = w.astype(np.float64).reshape(-1, nb, 32)
    qb = q.astype(np.float64).reshape(-1, nb, 32)
    # scale: binary16 of fp32(amax)/127, via numpy's own conversion
    amax = np.max(np.abs(w.reshape(-1, nb, 32)), axis=2)
    ref = (amax / np.float32(127)).astype(np.float32).astype(np.float16).view(np.uint16)
    assert np.array_equal(d, ref)
    # round-trip bound |w - q s| <= s/2 (every term exact in fp64)
    err = np.abs(wb - qb * s[:, :, None])
    assert np.all(err <= s[:, :, None] / 2)
    # signs agree or the code is zero
    assert np.all((qb == 0) | (np.sign(qb) == np.sign(wb)))
    # monotone inside a block
    order = np.argsort(wb, axis=2, kind="stable")
    qs = np.take_along_axis(qb, order, axis=2)
    assert np.all(np.diff(qs, axis=2) >= 0)
    # every normal-scale block reaches the code 127 in magnitude
    assert np.all(np.max(np.abs(qb), axis=2) == 127)
    assert np.all(np.abs(q) <= 127)


def test_quantize_zero_and_negative_zero_blocks():
    w = np.zeros((2, 64), dtype=np.float32)
    w[1] = -0.0
    q, d = oracle.quantize_f32(w)
    assert np.all(q == 0) and np.all(d == 0)


def test_quantize_subnormal_scale_clamps():
    # amax so small that the binary16 scale is subnormal; codes stay in range
    blk = np.full((1, 32), 1e-4, dtype=np.float32)
    blk[0, 5] = -3e-4
    blk[0, 9] = 2.9e-4
    q, d = oracle.quantize_f32(blk)
    assert d[0, 0] != 0 and d[0, 0] < 0x0400
    assert list(q[0]) == _exact_codes(blk[0], int(d[0, 0]))
    # amax below 127 * 2^-25: the scale rounds to zero, so every code is zero
    tiny = np.full((1, 32), 1e-9, dtype=np.float32)
    q, d = oracle.quantize_f32(tiny)
    assert d[0, 0] == 0 and np.all(q == 0)


# ---------------------------------------------------------------- activations

def test_quantize_bf16_all_patterns():
    """Every finite bf16 pattern whose block scale stays finite (|x| <= 8e6).

    Values with |x| <= 3 go 31 to a block beside a fixed largest element 3.0;
    larger values are sorted by magnitude and cut into blocks of 32."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = wl.bf16_bits_to_f32(bits)
    fin = np.isfinite(vals)
    small = bits[fin & (np.abs(vals) <= np.float32(3.0))]
    nblk = -(-small.size // 31)
    xs = np.zeros((nblk, 32), dtype=np.uint16)
    flat = np.zeros(nblk * 31, dtype=np.uint16)
    flat[:small.size] = small
    xs[:, 1:] = flat.reshape(nblk, 31)
    xs[:, 0] = wl.f32_to_bf16_bits(np.array([3.0], dtype=np.float32))[0]
    big = bits[fin & (np.abs(vals) > np.float32(3.0)) & (np.abs(vals) <= np.float32(8e6))]
    big = big[np.argsort(np.abs(wl.bf16_bits_to_f32(big)), kind="stable")]
    pad = (-big.size) % 32
    big = np.concatenate([big, np.zeros(pad, dtype=np.uint16)])
    x = np.concatenate([xs.reshape(-1), big]).reshape(1, -1)
    q, d = oracle.quantize_bf16(x)
    xf = wl.bf16_bits_to_f32(x)
    for b in range(x.shape[1] // 32):
        blk = xf[0, 32 * b:32 * b + 32]
        amax = Fraction(float(np.max(np.abs(blk))))
        assert d[0, b] == _nearest_half_bits(amax / 127), b
        assert list(q[0, 32 * b:32 * b + 32]) == _exact_codes(blk, int(d[0, b])), b


def test_quantize_bf16_special_rows():
    k = 256
    sp = wl.special_rows_f32(44, k)
    x = wl.f32_to_bf16_bits(sp)
    assert np.array_equal(wl.bf16_bits_to_f32(x), sp)      # bf16-exact by construction
    q, d = oracle.quantize_bf16(x)
    assert np.all(q[:2] == 0) and np.all(d[:2] == 0)
    z = q[2].reshape(-1, 32)[::4]
    assert np.all(z == 0)
    for r in range(3, 7):                                   # exact halves: q = +-(j+1)
        s = d[r].view(np.float16).astype(np.float64)
        for b in range(k // 32):
            blk = sp[r, 32 * b:32 * b + 32].astype(np.float64) / s[b]
            want = np.sign(blk) * np.floor(np.abs(blk) + 0.5)
            assert np.array_equal(q[r, 32 * b:32 * b + 32], want.astype(np.int8))
            assert np.max(np.abs(q[r, 32 * b:32 * b + 32])) == 127
            frac = np.abs(blk) - np.floor(np.abs(blk))
            assert np.all((frac == 0.5) | (np.abs(blk) == 127))
    for r in range(7, 11):                                  # unit scale: q = rhaway(x)
        assert np.all(d[r] == 0x3C00)
        want = np.sign(sp[r]) * np.floor(np.abs(sp[r]).astype(np.float64) + 0.5)
        assert np.array_equal(q[r], want.astype(np.int8))


def test_quantize_threads_bit_identical():
    w = wl.normal_weights(13, 512, 256)
    oracle.set_threads(1)
    a = oracle.quantize_f32(w)
    oracle.set_threads(4)
    b = oracle.quantize_f32(w)
    oracle.set_threads(1)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
