"""Pins for the oracle's W8A16 and Q8 x Q8 products.

The oracle is checked against exact rational arithmetic on tiny, non-square
shapes (so a transposed operand, a wrong block index or a dropped scale fails),
against closed forms (one-hot activations, power-of-two scaling, zero input),
against an independent library path (numpy fp64 matmul of the dequantized
matrix; numpy int64 products for the block sums), and against the batching rule
that identical activation rows give identical outputs (Frigg README, Finding 8).
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
import workloads as wl


def _f16(bits):
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def _tiny_case(seed, n, k, m):
    w = wl.normal_weights(seed, n, k)
    x = wl.normal_act_bf16(seed + 1, m, k)
    wq, wd = oracle.quantize_f32(w)
    return wq, wd, x


def _exact_w8a16(wq, wd, x):
    n, k = wq.shape
    m = x.shape[0]
    xf = wl.bf16_bits_to_f32(x)
    s = _f16(wd)
    out = [[Fraction(0)] * n for _ in range(m)]
    for mi in range(m):
        for r in range(n):
            acc = Fraction(0)
            for kk in range(k):
                acc += int(wq[r, kk]) * Fraction(float(s[r, kk // 32])) * Fraction(float(xf[mi, kk]))
            out[mi][r] = acc
    return out


@pytest.mark.parametrize("n,k,m", [(1, 32, 1), (5, 64, 3), (9, 96, 8), (7, 32, 2), (3, 96, 5)])
def test_w8a16_exact_rational(n, k, m):
    wq, wd, x = _tiny_case(100 + n + k + m, n, k, m)
    y = oracle.w8a16(wq, wd, x)
    ex = _exact_w8a16(wq, wd, x)
    xf = wl.bf16_bits_to_f32(x).astype(np.float64)
    absum = np.abs(xf) @ (np.abs(wq.astype(np.float64)) * np.repeat(_f16(wd), 32, axis=1)).T
    for mi in range(m):
        for r in range(n):
            bound = 2 * k * 2.0 ** -53 * absum[mi, r]
            assert abs(y[mi, r] - float(ex[mi][r])) <= bound, (mi, r)


def test_w8a16_matches_numpy_matmul():
    wq, wd, x = _tiny_case(200, 300, 512, 4)
    y = oracle.w8a16(wq, wd, x)
    deq = wq.astype(np.float64) * np.repeat(_f16(wd), 32, axis=1)
    ref = wl.bf16_bits_to_f32(x).astype(np.float64) @ deq.T
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-12)


def test_w8a16_one_hot_is_scaled_code():
    wq, wd, _ = _tiny_case(300, 17, 128, 1)
    s = _f16(wd)
    for kk in (0, 31, 32, 77, 127):
        x = np.zeros((1, 128), dtype=np.uint16)
        x[0, kk] = 0x3F80                                   # bf16 1.0
        y = oracle.w8a16(wq, wd, x)
        assert np.array_equal(y[0], wq[:, kk].astype(np.float64) * s[:, kk // 32])


def test_w8a16_power_of_two_scaling_and_zero():
    wq, wd, x = _tiny_case(301, 33, 192, 2)
    y = oracle.w8a16(wq, wd, x)
    x4 = wl.f32_to_bf16_bits(wl.bf16_bits_to_f32(x) * np.float32(4))
    assert np.array_equal(oracle.w8a16(wq, wd, x4), 4 * y)
    assert np.all(oracle.w8a16(wq, wd, np.zeros_like(x)) == 0)


def test_w8a16_identical_rows_and_row_subset():
    wq, wd, x1 = _tiny_case(302, 40, 256, 1)
    x = np.repeat(x1, 8, axis=0)
    y = oracle.w8a16(wq, wd, x)
    assert all(np.array_equal(y[0], y[i]) for i in range(8))
    rows = np.array([39, 0, 17, 17, 5])
    ys = oracle.w8a16(wq, wd, x1, rows=rows)
    assert np.array_equal(ys[0], y[0][rows])


# ------------------------------------------------------------------ Q8 x Q8

def _q8_case(seed, n, k, m):
    w = wl.normal_weights(seed, n, k)
    xb = wl.normal_act_bf16(seed + 1, m, k)
    wq, wd = oracle.quantize_f32(w)
    xq, xd = oracle.quantize_bf16(xb)
    return wq, wd, xq, xd


def test_block_dots_match_numpy_int64():
    wq, _, xq, _ = _q8_case(400, 37, 320, 6)
    isum = oracle.block_dots(wq, xq)
    ref = np.einsum("nbi,mbi->mnb",
                    wq.astype(np.int64).reshape(37, 10, 32),
                    xq.astype(np.int64).reshape(6, 10, 32))
    assert np.array_equal(isum, ref)


def test_block_dots_extremes():
    k = 64
    wq = np.full((2, k), 127, dtype=np.int8)
    wq[1] = -127
    xq = np.full((1, k), -127, dtype=np.int8)
    isum = oracle.block_dots(wq, xq)
    assert np.all(isum[0, 0] == -516128) and np.all(isum[0, 1] == 516128)


@pytest.mark.parametrize("n,k,m", [(1, 32, 1), (6, 64, 4), (9, 96, 8), (4, 160, 3)])
def test_q8q8_exact_rational(n, k, m):
    wq, wd, xq, xd = _q8_case(500 + n + k + m, n, k, m)
    y = oracle.q8q8(wq, wd, xq, xd)
    sw, sx = _f16(wd), _f16(xd)
    nb = k // 32
    for mi in range(m):
        for r in range(n):
            ex = Fraction(0)
            absum = 0.0
            for b in range(nb):
                isum = sum(int(wq[r, 32 * b + i]) * int(xq[mi, 32 * b + i]) for i in range(32))
                t = Fraction(float(sw[r, b])) * Fraction(float(sx[mi, b])) * isum
                ex += t
                absum += abs(float(t))
            assert abs(y[mi, r] - float(ex)) <= 2 * nb * 2.0 ** -53 * absum


def test_q8q8_matches_dequantized_numpy():
    wq, wd, xq, xd = _q8_case(600, 130, 384, 5)
    y = oracle.q8q8(wq, wd, xq, xd)
    dw = wq.astype(np.float64) * np.repeat(_f16(wd), 32, axis=1)
    dx = xq.astype(np.float64) * np.repeat(_f16(xd), 32, axis=1)
    assert np.allclose(y, dx @ dw.T, rtol=1e-12, atol=1e-12)


def test_q8q8_power_of_two_scales_exact():
    """Scales 2^e exactly (amax = 127 * 2^e), so every term is a dyadic rational
    and the fp64 sum is exact: y equals the integer-arithmetic result."""
    g = wl.rng(700)
    n, k, m = 12, 256, 3
    nb = k // 32
    w = g.integers(-127, 128, size=(n, k)).astype(np.float32)
    x = g.integers(-127, 128, size=(m, k)).astype(np.float32)
    ew = g.integers(-8, 3, size=(n, nb))
    ex = g.integers(-8, 3, size=(m, nb))
    w.reshape(n, nb, 32)[:, :, 0] = 127
    x.reshape(m, nb, 32)[:, :, 0] = -127
    w = (w.reshape(n, nb, 32) * np.exp2(ew)[:, :, None]).reshape(n, k).astype(np.float32)
    x = (x.reshape(m, nb, 32) * np.exp2(ex)[:, :, None]).reshape(m, k).astype(np.float32)
    wq, wd = oracle.quantize_f32(w)
    xq, xd = oracle.quantize_bf16(wl.f32_to_bf16_bits(x))
    assert np.array_equal(_f16(wd), np.exp2(ew)) and np.array_equal(_f16(xd), np.exp2(ex))
    y = oracle.q8q8(wq, wd, xq, xd)
    isum = oracle.block_dots(wq, xq).astype(np.int64)           # [m][n][nb]
    num = isum * (2 ** (ew[None, :, :] + ex[:, None, :] + 16)).astype(np.int64)
    exact = num.sum(axis=2).astype(np.float64) / 2.0 ** 16
    assert np.array_equal(y, exact)


def test_q8q8_threads_and_rows():
    wq, wd, xq, xd = _q8_case(800, 257, 128, 4)
    oracle.set_threads(1)
    a = oracle.q8q8(wq, wd, xq, xd)
    oracle.set_threads(3)
    b = oracle.q8q8(wq, wd, xq, xd)
    oracle.set_threads(1)
    assert np.array_equal(a, b)
    rows = np.array([256, 3, 100])
    assert np.array_equal(oracle.q8q8(wq, wd, xq, xd, rows=rows), a[:, rows])
