"""Pins for the oracle's decode-step glue: weightless RMSNorm (eps 1e-6), the
default rotary embedding (theta 10,000, dimension i paired with i + 64 of a
128-wide head) and SwiGLU, as the Frigg README's model table states them.

Checked against closed forms (constant and two-value vectors, the pairs whose
angle is pos or pos / 100 exactly, silu at 0 and 1), invariants (scale
invariance of the norm, norm-preserving rotation, scores that depend only on
the relative position, silu(-z) = silu(z) - z) and brute force over tiny cases.
"""
import math

import numpy as np

import oracle
import workloads as wl


def test_rmsnorm_closed_forms():
    c = np.full((1, 64), 3.0, dtype=np.float32)
    assert np.allclose(oracle.rmsnorm(c)[0], 3.0 / math.sqrt(9.0 + 1e-6), rtol=0, atol=1e-15)
    two = np.array([[3.0, 4.0]], dtype=np.float32)                  # mean square 12.5
    want = np.array([3.0, 4.0]) / math.sqrt(12.5 + 1e-6)
    assert np.allclose(oracle.rmsnorm(two)[0], want, rtol=0, atol=1e-15)
    z = np.zeros((2, 32), dtype=np.float32)
    assert np.all(oracle.rmsnorm(z) == 0.0)
    # eps matters only for tiny inputs: a vector of 1e-4 has mean square 1e-8
    t = np.full((1, 16), 1e-4, dtype=np.float32)
    assert abs(oracle.rmsnorm(t)[0, 0] - float(np.float32(1e-4)) / math.sqrt(float(np.float32(1e-4)) ** 2 + 1e-6)) < 1e-12


def test_rmsnorm_invariants():
    x = wl.rng(1).standard_normal((5, 1536)).astype(np.float32)
    y = oracle.rmsnorm(x)
    # rows are independent and each output row has mean square ms / (ms + eps)
    ms = np.mean(x.astype(np.float64) ** 2, axis=1)
    assert np.allclose(np.mean(y ** 2, axis=1), ms / (ms + 1e-6), rtol=1e-12)
    assert np.allclose(oracle.rmsnorm(x[2:3])[0], y[2], rtol=0, atol=0)
    # scaling by a power of two (exact in fp32) leaves the output almost unchanged
    y2 = oracle.rmsnorm(x * np.float32(64.0))
    assert np.allclose(y2, y, rtol=1e-6)
    # signs are kept
    assert np.all(np.sign(y) == np.sign(x))


def test_rope_closed_forms():
    d, heads = 128, 3
    v = wl.rng(2).standard_normal(heads * d)
    assert np.array_equal(oracle.rope(v, heads, d, 0), v)           # position 0: identity
    pos = 7
    r = oracle.rope(v, heads, d, pos)
    for h in range(heads):
        # pair 0 turns by exactly pos radians (theta^0 = 1)
        a, b = v[h * d], v[h * d + 64]
        assert abs(r[h * d] - (a * math.cos(pos) - b * math.sin(pos))) < 1e-12
        assert abs(r[h * d + 64] - (b * math.cos(pos) + a * math.sin(pos))) < 1e-12
        # pair 32 turns by pos * 10000^(-1/2) = pos / 100
        a, b = v[h * d + 32], v[h * d + 96]
        ang = pos / 100.0
        assert abs(r[h * d + 32] - (a * math.cos(ang) - b * math.sin(ang))) < 1e-12
        assert abs(r[h * d + 96] - (b * math.cos(ang) + a * math.sin(ang))) < 1e-12


def test_rope_invariants():
    d = 128
    g = wl.rng(3)
    q, k = g.standard_normal(d), g.standard_normal(d)
    # every pair keeps its length
    r = oracle.rope(q, 1, d, 1234)
    assert np.allclose(np.hypot(r[:64], r[64:]), np.hypot(q[:64], q[64:]), rtol=1e-12)
    # scores depend only on the relative position
    s1 = oracle.rope(q, 1, d, 100) @ oracle.rope(k, 1, d, 40)
    s2 = oracle.rope(q, 1, d, 4060) @ oracle.rope(k, 1, d, 4000)
    assert abs(s1 - s2) < 1e-9 * (1 + abs(s1))
    # turning by p then by -p is the identity
    back = oracle.rope(oracle.rope(q, 1, d, 55), 1, d, -55)
    assert np.allclose(back, q, rtol=0, atol=1e-12)


def test_swiglu_closed_forms_and_invariants():
    assert oracle.swiglu(np.array([0.0]), np.array([5.0]))[0] == 0.0
    assert abs(oracle.swiglu(np.array([1.0]), np.array([1.0]))[0] - 1.0 / (1.0 + math.exp(-1.0))) < 1e-16
    g = wl.rng(4).standard_normal(1000) * 4
    one = np.ones_like(g)
    s = oracle.swiglu(g, one)
    assert np.allclose(oracle.swiglu(-g, one), s - g, rtol=0, atol=1e-12)   # silu(-z) = silu(z) - z
    u = wl.rng(5).standard_normal(1000)
    assert np.allclose(oracle.swiglu(g, u), s * u, rtol=1e-15)
    assert abs(oracle.swiglu(np.array([40.0]), one[:1])[0] - 40.0) < 1e-12
    assert abs(oracle.swiglu(np.array([-40.0]), one[:1])[0]) < 1e-15
