"""Pins for the oracle's int4 weight format and its products.

The pages name int4 weights ("int4 core + int8 vocab" in the Frigg README's
bytes-per-token table, "int4 W / int8 vocab" in its benchmark matrix) without a
layout; the oracle reads them as the Q8_0 rule with 7 in place of 127 and two
4-bit two's-complement codes per byte (element j of a block in the low nibble
of byte j, element j + 16 in the high nibble).  These tests check that reading
against values worked out by hand, against exact rational arithmetic (Python
``fractions``), against numpy's binary16 conversion, a brute-force nearest-code
search and invariants the definition d = maxabs / 7 implies.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
import workloads as wl


def _f16(bits):
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


# ---------------------------------------------------------------- hand-worked block

# amax 7 gives the scale 7 / 7 = 1 (binary16 0x3C00), so each code is the value
# rounded half away from zero and clamped to [-7, 7].
_HAND_VALUES = [7, -7, 3.5, -3.5, 2.5, -2.5, 0.5, -0.5, 0.49999997, 6.5, -6.5, 1.5, -1.49, 0.0, -0.0, 5,
                -1, 2, -3, 4, -5, 6, -7, 0.75, -0.25, 7, 0, 1, 1, 1, 1, -6.5]
_HAND_CODES = [7, -7, 4, -4, 3, -3, 1, -1, 0, 7, -7, 2, -1, 0, 0, 5,
               -1, 2, -3, 4, -5, 6, -7, 1, 0, 7, 0, 1, 1, 1, 1, -7]
# byte j = (code j mod 16) | (code j+16 mod 16) << 4, worked out by hand
_HAND_BYTES = [0xF7, 0x29, 0xD4, 0x4C, 0xB3, 0x6D, 0x91, 0x1F,
               0x00, 0x77, 0x09, 0x12, 0x1F, 0x10, 0x10, 0x95]


def test_hand_block_codes_and_bytes():
    w = np.array([_HAND_VALUES], dtype=np.float32)
    q, d = oracle.q4_quantize_f32(w)
    assert q.shape == (1, 16) and d.shape == (1, 1)
    assert int(d[0, 0]) == 0x3C00
    assert [int(b) for b in q[0]] == _HAND_BYTES
    assert [int(c) for c in oracle.q4_unpack(q)[0]] == _HAND_CODES


def test_hand_block_scaled_and_second_block():
    # the same block times 2^-10 in the second block of a row: scale 2^-10
    # (0x1400), identical bytes; the first block is all zero
    w = np.zeros((1, 64), dtype=np.float32)
    w[0, 32:] = np.array(_HAND_VALUES, dtype=np.float32) * np.float32(2.0 ** -10)
    q, d = oracle.q4_quantize_f32(w)
    assert [int(v) for v in d[0]] == [0, 0x1400]
    assert np.all(q[0, :16] == 0)
    assert [int(b) for b in q[0, 16:]] == _HAND_BYTES


def test_unpack_hand_bytes():
    # 0x8F: low nibble 15 -> -1, high nibble 8 -> -8; 0x70: 0 and 7
    q = np.zeros((1, 16), dtype=np.uint8)
    q[0, 0] = 0x8F
    q[0, 15] = 0x70
    c = oracle.q4_unpack(q)[0]
    assert int(c[0]) == -1 and int(c[16]) == -8
    assert int(c[15]) == 0 and int(c[31]) == 7
    assert np.all(np.delete(c, [0, 16, 15, 31]) == 0)


def test_scale_hand_value():
    # 1/7 = 0.142857...; binade [2^-3, 2^-2), quantum 2^-13: 0.142857 * 2^13 =
    # 1170.29 -> 1170 = 1024 + 146, so the pattern is (12 << 10) | 146 = 0x3092
    assert oracle.q4_block_scale(1.0) == 0x3092
    assert oracle.q4_block_scale(7.0) == 0x3C00
    assert oracle.q4_block_scale(0.0) == 0


# ---------------------------------------------------------------- random blocks

def _blocks(seed: int, nblocks: int) -> np.ndarray:
    g = wl.rng(seed)
    rows = []
    for i in range(nblocks):
        kind = i % 5
        if kind == 0:
            b = g.standard_normal(32) * 0.02
        elif kind == 1:
            b = g.standard_normal(32) * np.exp2(g.integers(-20, 8, size=32))
        elif kind == 2:       # binary16-subnormal or zero scale
            b = g.standard_normal(32) * 10.0 ** g.integers(-9, -5)
        elif kind == 3:       # exact halves of a power-of-two scale
            e = int(g.integers(-8, 4))
            b = (g.integers(0, 7, size=32) + 0.5) * 2.0 ** e * np.where(g.integers(0, 2, size=32) == 0, -1, 1)
            b[int(g.integers(0, 32))] = 7 * 2.0 ** e
        else:                 # zeros and negative zeros
            b = np.where(g.integers(0, 2, size=32) == 0, -0.0, 0.0)
        rows.append(np.asarray(b, dtype=np.float32))
    return np.concatenate(rows).reshape(1, -1)


def test_scale_matches_numpy_rounding():
    w = _blocks(40, 500)
    _, d = oracle.q4_quantize_f32(w)
    amax = np.max(np.abs(w.reshape(-1, 32)), axis=1).astype(np.float64)
    # binary16 of the exact quotient: fp64 division then numpy's conversion (both
    # roundings to nearest; fp64 keeps more than 2*11+2 bits, so the double
    # rounding gives the correctly rounded quotient, as the fp32 route does)
    ref = (amax / 7.0).astype(np.float16).view(np.uint16)
    assert np.array_equal(d[0], ref)


def test_codes_argmin_brute_force():
    """Each code is the c in [-7, 7] minimising |w - c*s| exactly (ties to the
    larger |c|), s the stored scale; zero scale gives zero codes."""
    w = _blocks(41, 160)
    q, d = oracle.q4_quantize_f32(w)
    c = oracle.q4_unpack(q)[0]
    for b in range(w.shape[1] // 32):
        s = Fraction(float(_f16(d[0, b])))
        for i in range(32):
            fw = Fraction(float(w[0, 32 * b + i]))
            want = 0 if s == 0 else min(range(-7, 8), key=lambda v: (abs(fw - v * s), -abs(v)))
            assert int(c[32 * b + i]) == want, (b, i)


def test_invariants_normal_weights():
    w = wl.normal_weights(42, 512, 1536)
    q, d = oracle.q4_quantize_f32(w)
    assert q.shape == (512, 768) and d.shape == (512, 48)
    c = oracle.q4_unpack(q).astype(np.float64).reshape(512, 48, 32)
    s = _f16(d)
    wb = w.astype(np.float64).reshape(512, 48, 32)
    assert np.all(np.abs(c) <= 7)
    # round-trip bound |w - c s| <= s/2 (every term exact in fp64)
    assert np.all(np.abs(wb - c * s[:, :, None]) <= s[:, :, None] / 2)
    # signs agree or the code is zero; every block reaches magnitude 7
    assert np.all((c == 0) | (np.sign(c) == np.sign(wb)))
    assert np.all(np.max(np.abs(c), axis=2) == 7)
    # the int4 error is about (127/7)x the Q8_0 error of the same weights
    q8, d8 = oracle.quantize_f32(w)
    e8 = np.abs(wb - q8.astype(np.float64).reshape(512, 48, 32) * _f16(d8)[:, :, None]).mean()
    e4 = np.abs(wb - c * s[:, :, None]).mean()
    assert 12 < e4 / e8 < 24


def test_subnormal_scale_clamps_and_zero_scale():
    # amax 5.5e-7: 5.5e-7 / 7 = 7.86e-8 rounds to the smallest binary16
    # subnormal 2^-24 = 5.96e-8, so 5.5e-7 / 2^-24 = 9.2 clamps to 7
    blk = np.full((1, 32), 1e-7, dtype=np.float32)
    blk[0, 3] = 5.5e-7
    blk[0, 20] = -5.5e-7
    q, d = oracle.q4_quantize_f32(blk)
    assert int(d[0, 0]) == 1
    c = oracle.q4_unpack(q)[0]
    assert int(c[3]) == 7 and int(c[20]) == -7
    # 1e-7 / 2^-24 = 1.68 -> 2
    assert all(int(c[i]) == 2 for i in range(32) if i not in (3, 20))
    # amax 1e-7: 1e-7 / 7 = 1.4e-8 is below half the smallest subnormal
    tiny = np.full((1, 32), 1e-7, dtype=np.float32)
    q, d = oracle.q4_quantize_f32(tiny)
    assert int(d[0, 0]) == 0 and np.all(q == 0)


def test_threads_bit_identical():
    w = wl.normal_weights(43, 300, 512)
    oracle.set_threads(1)
    a = oracle.q4_quantize_f32(w)
    oracle.set_threads(8)
    b = oracle.q4_quantize_f32(w)
    oracle.set_threads(1)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


# ---------------------------------------------------------------- products

def _exact(c, wd, xf):
    n, k = c.shape
    m = xf.shape[0]
    s = _f16(wd)
    out = np.empty((m, n), dtype=object)
    for mi in range(m):
        for r in range(n):
            acc = Fraction(0)
            for kk in range(k):
                acc += int(c[r, kk]) * Fraction(float(s[r, kk // 32])) * Fraction(float(xf[mi, kk]))
            out[mi, r] = acc
    return out


@pytest.mark.parametrize("n,k,m", [(1, 32, 1), (5, 64, 3), (9, 96, 8), (3, 128, 2)])
def test_w4a16_exact_rational(n, k, m):
    w = wl.normal_weights(60 + n + k, n, k)
    x = wl.normal_act_bf16(61 + m, m, k)
    q, d = oracle.q4_quantize_f32(w)
    y = oracle.w4a16(q, d, x)
    xf = wl.bf16_bits_to_f32(x)
    ex = _exact(oracle.q4_unpack(q), d, xf)
    for mi in range(m):
        for r in range(n):
            assert abs(y[mi, r] - float(ex[mi, r])) <= 1e-12 * (1 + abs(float(ex[mi, r]))), (mi, r)


@pytest.mark.parametrize("n,k,m", [(4, 64, 1), (7, 96, 5)])
def test_q4q8_exact_rational(n, k, m):
    w = wl.normal_weights(70 + n + k, n, k)
    x = wl.normal_act_bf16(71 + m, m, k)
    q, d = oracle.q4_quantize_f32(w)
    xq, xd = oracle.quantize_bf16(x)
    y = oracle.q4q8(q, d, xq, xd)
    c = oracle.q4_unpack(q)
    sw, sx = _f16(d), _f16(xd)
    for mi in range(m):
        for r in range(n):
            acc = Fraction(0)
            for b in range(k // 32):
                isum = sum(int(c[r, 32 * b + i]) * int(xq[mi, 32 * b + i]) for i in range(32))
                acc += Fraction(float(sw[r, b])) * Fraction(float(sx[mi, b])) * isum
            assert abs(y[mi, r] - float(acc)) <= 1e-12 * (1 + abs(float(acc))), (mi, r)


def test_w4a16_one_hot_and_rows():
    w = wl.normal_weights(80, 6, 96)
    q, d = oracle.q4_quantize_f32(w)
    c = oracle.q4_unpack(q)
    for kk in (0, 17, 31, 32, 63, 95):
        x = np.zeros((1, 96), dtype=np.float32)
        x[0, kk] = 1.0
        y = oracle.w4a16(q, d, wl.f32_to_bf16_bits(x))
        assert np.array_equal(y[0], c[:, kk] * _f16(d[:, kk // 32]))
    x = wl.normal_act_bf16(81, 2, 96)
    full = oracle.w4a16(q, d, x)
    sub = oracle.w4a16(q, d, x, rows=[5, 0, 3])
    assert np.array_equal(sub, full[:, [5, 0, 3]])
