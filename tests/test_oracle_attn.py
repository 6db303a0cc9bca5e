"""Pins for the oracle's decode attention over a Q8_0 key/value cache.

The pages define the computation (one query per head against the whole cache,
no mask: Frigg README, "Masks" and "Cache"; 12 heads of 128: "The model, as
verified"), not printed values, so the oracle is pinned by closed forms and
invariants of softmax attention: a single row, zero keys (the mean of V), two
rows with exactly known scores (a logistic weight), a dominant row, shift and
permutation invariance, linearity in V, independence of heads and of the cache
rows past t.  Each is chosen so that a dropped max subtraction, a wrong
normalisation, a transposed head/row index, a misapplied scale or a read past t
fails one of them."""
import math

import numpy as np
import pytest

import oracle
import workloads as wl

D = 128
ONE_F16 = np.float16(1.0).view(np.uint16)


def kv_case(seed, heads, t_cap, d=D):
    """Random Q8_0 K and V [heads][t_cap][d] quantized from N(0,1) bf16 rows,
    and a bf16 query [heads][d]."""
    g = wl.rng(seed)
    kx = wl.f32_to_bf16_bits(g.standard_normal((heads * t_cap, d)).astype(np.float32))
    vx = wl.f32_to_bf16_bits(g.standard_normal((heads * t_cap, d)).astype(np.float32))
    kq, kd = oracle.quantize_bf16(kx)
    vq, vd = oracle.quantize_bf16(vx)
    q = wl.f32_to_bf16_bits(g.standard_normal((heads, d)).astype(np.float32))
    return (q, kq.reshape(heads, t_cap, d), kd.reshape(heads, t_cap, d // 32),
            vq.reshape(heads, t_cap, d), vd.reshape(heads, t_cap, d // 32))


def dequant(codes, scales):
    s = scales.view(np.float16).astype(np.float64)
    return codes.astype(np.float64) * np.repeat(s, 32, axis=-1)


def test_single_row_returns_that_value_row():
    q, kq, kd, vq, vd = kv_case(1, 3, 5)
    out = oracle.attn_decode(q, kq, kd, vq, vd, 1, 1.0 / math.sqrt(D))
    assert np.array_equal(out, dequant(vq[:, 0], vd[:, 0]))


@pytest.mark.parametrize("t", [1, 7, 64])
def test_zero_keys_or_zero_scale_give_the_mean_of_v(t):
    q, kq, kd, vq, vd = kv_case(2, 2, 64)
    mean = dequant(vq[:, :t], vd[:, :t]).mean(axis=1)
    out = oracle.attn_decode(q, np.zeros_like(kq), kd, vq, vd, t, 0.088)
    assert np.allclose(out, mean, rtol=0, atol=1e-13)
    out = oracle.attn_decode(q, kq, kd, vq, vd, t, 0.0)
    assert np.allclose(out, mean, rtol=0, atol=1e-13)


def _unit_query_keys(codes, heads=1, t_cap=None):
    """q = e_0 (bf16 1.0), K[j][0] = codes[j] with scale 1.0, other entries 0:
    the score of row j is exactly scale * codes[j]."""
    t = len(codes)
    t_cap = t_cap or t
    q = np.zeros((heads, D), dtype=np.uint16)
    q[:, 0] = 0x3F80
    kq = np.zeros((heads, t_cap, D), dtype=np.int8)
    kq[:, :t, 0] = np.asarray(codes, dtype=np.int8)
    kd = np.full((heads, t_cap, D // 32), ONE_F16, dtype=np.uint16)
    return q, kq, kd


@pytest.mark.parametrize("c0,c1,scale", [(3, -2, 0.5), (127, 0, 0.05), (-50, -51, 1.0), (10, 10, 0.3)])
def test_two_rows_logistic_weight(c0, c1, scale):
    q, kq, kd = _unit_query_keys([c0, c1])
    _, _, _, vq, vd = kv_case(3, 1, 2)
    w0 = 1.0 / (1.0 + math.exp(scale * (c1 - c0)))
    v = dequant(vq, vd)[0]
    expect = w0 * v[0] + (1.0 - w0) * v[1]
    out = oracle.attn_decode(q, kq, kd, vq, vd, 2, scale)[0]
    assert np.allclose(out, expect, rtol=1e-14, atol=1e-14)


def test_dominant_row():
    codes = [0, -3, 4, 100, 2, -1]
    q, kq, kd = _unit_query_keys(codes)
    _, _, _, vq, vd = kv_case(4, 1, 6)
    v = dequant(vq, vd)[0]
    out = oracle.attn_decode(q, kq, kd, vq, vd, 6, 1.0)[0]
    # every other row's weight is at most e^(4 - 100)
    assert np.max(np.abs(out - v[3])) <= 6 * math.exp(-96) * np.max(np.abs(v)) + 1e-300


def test_shift_invariance_without_overflow():
    """Adding the same amount to every score changes nothing, even when the
    scores themselves would overflow exp: the maximum is subtracted first."""
    base = [5, -7, 12, 0, 3]
    q, kq, kd = _unit_query_keys(base)
    _, _, _, vq, vd = kv_case(5, 1, 5)
    ref = oracle.attn_decode(q, kq, kd, vq, vd, 5, 0.25)
    kq2 = kq.copy()
    kq2[0, :, 0] += 100
    out = oracle.attn_decode(q, kq2, kd, vq, vd, 5, 0.25)
    assert np.allclose(out, ref, rtol=1e-13, atol=1e-15)
    big = oracle.attn_decode(q, kq2, kd, vq, vd, 5, 10.0)      # scores up to 1120: exp overflows
    assert np.all(np.isfinite(big))
    v = dequant(vq, vd)[0]
    assert np.allclose(big[0], v[2], atol=1e-12)               # row 2 (code 112) dominates


def test_row_permutation_invariance():
    q, kq, kd, vq, vd = kv_case(6, 2, 40)
    perm = wl.rng(7).permutation(40)
    ref = oracle.attn_decode(q, kq, kd, vq, vd, 40, 0.09)
    out = oracle.attn_decode(q, kq[:, perm], kd[:, perm], vq[:, perm], vd[:, perm], 40, 0.09)
    assert np.allclose(out, ref, rtol=1e-13, atol=1e-15)


def test_linear_in_v_and_convex_hull():
    q, kq, kd, vq, vd = kv_case(8, 2, 33)
    ref = oracle.attn_decode(q, kq, kd, vq, vd, 33, 0.088)
    vd2 = (vd.view(np.float16).astype(np.float32) * 2).astype(np.float16).view(np.uint16)
    assert np.array_equal(vd2.view(np.float16).astype(np.float64), 2 * vd.view(np.float16).astype(np.float64))
    out = oracle.attn_decode(q, kq, kd, vq, vd2, 33, 0.088)
    assert np.array_equal(out, 2 * ref)
    v = dequant(vq, vd)
    assert np.all(out / 2 >= v.min(axis=1) - 1e-12) and np.all(out / 2 <= v.max(axis=1) + 1e-12)


def test_heads_and_rows_past_t_are_independent():
    q, kq, kd, vq, vd = kv_case(9, 3, 50)
    ref = oracle.attn_decode(q, kq, kd, vq, vd, 20, 0.088)
    kq2, vq2, kd2 = kq.copy(), vq.copy(), kd.copy()
    kq2[:, 20:] = 127
    vq2[:, 20:] = -127
    kd2[:, 20:] = ONE_F16
    assert np.array_equal(oracle.attn_decode(q, kq2, kd2, vq2, vd, 20, 0.088), ref)
    kq3 = kq.copy()
    kq3[1] = -kq3[1]
    out = oracle.attn_decode(q, kq3, kd, vq, vd, 20, 0.088)
    assert np.array_equal(out[[0, 2]], ref[[0, 2]]) and not np.array_equal(out[1], ref[1])


def test_query_and_key_roles_are_not_swapped():
    """Score = q . K[j] with K's own block scales: scaling the key scales of one
    row by 2 doubles only that row's score."""
    codes = [10, 20]
    q, kq, kd = _unit_query_keys(codes)
    kd[0, 1, 0] = np.float16(2.0).view(np.uint16)     # row 1: scale 2 -> score 2 * 20 * s
    _, _, _, vq, vd = kv_case(10, 1, 2)
    scale = 0.05
    w0 = 1.0 / (1.0 + math.exp(scale * (40 - 10)))
    v = dequant(vq, vd)[0]
    out = oracle.attn_decode(q, kq, kd, vq, vd, 2, scale)[0]
    assert np.allclose(out, w0 * v[0] + (1 - w0) * v[1], rtol=1e-14, atol=1e-14)
