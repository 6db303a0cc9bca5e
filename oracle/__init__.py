"""CPU oracle for the Q8_0 weight-streaming path (ctypes over ``q8_oracle.c``).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
benchmark's CPU-baseline leg may import this package.  It shares no code with the
HIP library and never imports it.

Every function takes and returns numpy arrays; the arithmetic lives in the C
file, which cites the passages it follows.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "q8_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

_CFLAGS = ["-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-std=c11",
           "-Wall", "-shared", "-fPIC"]


def _stale() -> bool:
    return not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC)


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (plain C, OpenMP) into ``liboracle.so``.

    Runs a compiler in a child process: call it only from a process that has
    not initialised a GPU (the build step, the test session's start, the
    benchmark's start)."""
    if force or _stale():
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", *_CFLAGS, "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def ensure_built() -> str:
    """Build the oracle only if the library is missing or older than its source."""
    return build(force=False)


_lib = None


def lib():
    """The loaded oracle library.  Never compiles: raises if ``liboracle.so`` is
    missing or older than ``q8_oracle.c`` (run ``build()`` first)."""
    global _lib
    if _lib is None:
        if _stale():
            raise ImportError(f"{_LIB} is missing or older than {_SRC}: run oracle.build() (or "
                              "__graft_entry__.build()) before using the oracle")
        L = C.CDLL(_LIB)
        P = C.c_void_p
        I64 = C.c_int64
        L.oracle_set_threads.argtypes = [C.c_int]
        L.oracle_get_threads.restype = C.c_int
        L.oracle_half_to_double.argtypes = [C.c_uint16]
        L.oracle_half_to_double.restype = C.c_double
        L.oracle_half_from_double.argtypes = [C.c_double]
        L.oracle_half_from_double.restype = C.c_uint16
        L.oracle_rhaway.argtypes = [C.c_float]
        L.oracle_rhaway.restype = C.c_double
        L.oracle_rhaway_array.argtypes = [P, I64, P]
        L.oracle_block_scale.argtypes = [C.c_float]
        L.oracle_block_scale.restype = C.c_uint16
        L.oracle_quantize_f32.argtypes = [P, I64, I64, P, P]
        L.oracle_quantize_bf16.argtypes = [P, I64, I64, P, P]
        L.oracle_w8a16.argtypes = [P, P, I64, I64, I64, P, P, I64, P]
        L.oracle_block_dots.argtypes = [P, I64, I64, P, I64, P]
        L.oracle_q8q8.argtypes = [P, P, I64, I64, I64, P, P, P, I64, P]
        L.oracle_attn_decode.argtypes = [P, P, P, P, P, I64, I64, I64, I64, C.c_double, P]
        L.oracle_q4_block_scale.argtypes = [C.c_float]
        L.oracle_q4_block_scale.restype = C.c_uint16
        L.oracle_q4_quantize_f32.argtypes = [P, I64, I64, P, P]
        L.oracle_q4_unpack.argtypes = [P, I64, I64, P]
        L.oracle_rmsnorm.argtypes = [P, I64, I64, C.c_double, P]
        L.oracle_rope.argtypes = [P, I64, I64, I64, C.c_double]
        L.oracle_swiglu.argtypes = [P, P, I64, P]
        _lib = L
    return _lib


def _p(a: np.ndarray):
    return a.ctypes.data_as(C.c_void_p)


def set_threads(n: int) -> None:
    lib().oracle_set_threads(int(n))


def get_threads() -> int:
    return lib().oracle_get_threads()


def half_to_float(h: int) -> float:
    return lib().oracle_half_to_double(int(h))


def half_from_float(v: float) -> int:
    return lib().oracle_half_from_double(float(v))


def rhaway(t: float) -> float:
    return lib().oracle_rhaway(float(t))


def rhaway_array(t: np.ndarray) -> np.ndarray:
    t = np.ascontiguousarray(t, dtype=np.float32)
    out = np.empty(t.shape, dtype=np.int32)
    lib().oracle_rhaway_array(_p(t), t.size, _p(out))
    return out


def block_scale(amax: float) -> int:
    return lib().oracle_block_scale(float(amax))


def _check_k(k: int) -> None:
    if k % 32 != 0 or k <= 0:
        raise ValueError("k must be a positive multiple of 32")


def quantize_f32(w: np.ndarray):
    """fp32 [n][k] -> (codes int8 [n][k], binary16 scale bits uint16 [n][k/32])."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    n, k = w.shape
    _check_k(k)
    q = np.empty((n, k), dtype=np.int8)
    d = np.empty((n, k // 32), dtype=np.uint16)
    lib().oracle_quantize_f32(_p(w), n, k, _p(q), _p(d))
    return q, d


def quantize_bf16(x: np.ndarray):
    """bf16 bits [m][k] -> (codes int8 [m][k], binary16 scale bits [m][k/32])."""
    x = np.ascontiguousarray(x, dtype=np.uint16)
    m, k = x.shape
    _check_k(k)
    q = np.empty((m, k), dtype=np.int8)
    d = np.empty((m, k // 32), dtype=np.uint16)
    lib().oracle_quantize_bf16(_p(x), m, k, _p(q), _p(d))
    return q, d


def _rows(rows, n):
    if rows is None:
        return None, n
    r = np.ascontiguousarray(rows, dtype=np.int64)
    if r.size and (r.min() < 0 or r.max() >= n):
        raise IndexError("row index out of range")
    return r, r.size


def w8a16(wq, wd, x, rows=None) -> np.ndarray:
    """fp64 y [m][len(rows) or n] = dequantized W (rows) times bf16 x."""
    wq = np.ascontiguousarray(wq, dtype=np.int8)
    wd = np.ascontiguousarray(wd, dtype=np.uint16)
    x = np.ascontiguousarray(x, dtype=np.uint16)
    n, k = wq.shape
    m = x.shape[0]
    assert x.shape[1] == k and wd.shape == (n, k // 32)
    r, nr = _rows(rows, n)
    y = np.empty((m, nr), dtype=np.float64)
    lib().oracle_w8a16(_p(wq), _p(wd), n, k, m, _p(x),
                       None if r is None else _p(r), nr, _p(y))
    return y


def block_dots(wq, xq) -> np.ndarray:
    """Exact int32 block sums isum [m][n][k/32]."""
    wq = np.ascontiguousarray(wq, dtype=np.int8)
    xq = np.ascontiguousarray(xq, dtype=np.int8)
    n, k = wq.shape
    m = xq.shape[0]
    assert xq.shape[1] == k
    out = np.empty((m, n, k // 32), dtype=np.int32)
    lib().oracle_block_dots(_p(wq), n, k, _p(xq), m, _p(out))
    return out


def q8q8(wq, wd, xq, xd, rows=None) -> np.ndarray:
    """fp64 y [m][len(rows) or n] = sum_b wd*xd*isum."""
    wq = np.ascontiguousarray(wq, dtype=np.int8)
    wd = np.ascontiguousarray(wd, dtype=np.uint16)
    xq = np.ascontiguousarray(xq, dtype=np.int8)
    xd = np.ascontiguousarray(xd, dtype=np.uint16)
    n, k = wq.shape
    m = xq.shape[0]
    assert xq.shape[1] == k and wd.shape == (n, k // 32) and xd.shape == (m, k // 32)
    r, nr = _rows(rows, n)
    y = np.empty((m, nr), dtype=np.float64)
    lib().oracle_q8q8(_p(wq), _p(wd), n, k, m, _p(xq), _p(xd),
                      None if r is None else _p(r), nr, _p(y))
    return y


def q4_block_scale(amax: float) -> int:
    return lib().oracle_q4_block_scale(float(amax))


def q4_quantize_f32(w: np.ndarray):
    """fp32 [n][k] -> (packed int4 codes uint8 [n][k/2], binary16 scale bits [n][k/32])."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    n, k = w.shape
    _check_k(k)
    q = np.empty((n, k // 2), dtype=np.uint8)
    d = np.empty((n, k // 32), dtype=np.uint16)
    lib().oracle_q4_quantize_f32(_p(w), n, k, _p(q), _p(d))
    return q, d


def q4_unpack(q: np.ndarray) -> np.ndarray:
    """Packed int4 codes uint8 [n][k/2] -> int8 codes [n][k] in [-8, 7]."""
    q = np.ascontiguousarray(q, dtype=np.uint8)
    n, kh = q.shape
    _check_k(2 * kh)
    out = np.empty((n, 2 * kh), dtype=np.int8)
    lib().oracle_q4_unpack(_p(q), n, 2 * kh, _p(out))
    return out


def w4a16(wq4, wd, x, rows=None) -> np.ndarray:
    """fp64 y [m][len(rows) or n] over int4 weights: the W8A16 product of the
    unpacked codes (only the selected rows are unpacked)."""
    wq4 = np.ascontiguousarray(wq4, dtype=np.uint8)
    if rows is not None:
        r = np.ascontiguousarray(rows, dtype=np.int64)
        return w8a16(q4_unpack(wq4[r]), np.ascontiguousarray(wd)[r], x)
    return w8a16(q4_unpack(wq4), wd, x)


def q4q8(wq4, wd, xq, xd, rows=None) -> np.ndarray:
    """fp64 y [m][len(rows) or n]: int4 weights times Q8 activations, the Q8 x Q8
    product of the unpacked codes."""
    wq4 = np.ascontiguousarray(wq4, dtype=np.uint8)
    if rows is not None:
        r = np.ascontiguousarray(rows, dtype=np.int64)
        return q8q8(q4_unpack(wq4[r]), np.ascontiguousarray(wd)[r], xq, xd)
    return q8q8(q4_unpack(wq4), wd, xq, xd)


# ---------------------------------------------------------------- decode-step glue

RMS_EPS = 1e-6
ROPE_THETA = 10000.0


def rmsnorm(x, eps: float = RMS_EPS) -> np.ndarray:
    """fp64 [m][k]: weightless RMSNorm of the fp32 rows of x."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    m, k = x.shape
    y = np.empty((m, k), dtype=np.float64)
    lib().oracle_rmsnorm(_p(x), m, k, float(eps), _p(y))
    return y


def rope(v, heads: int, d: int, pos: int, theta: float = ROPE_THETA) -> np.ndarray:
    """fp64 copy of v (heads x d values, natural dimension order) turned by the
    default rotary embedding at position pos."""
    out = np.ascontiguousarray(v, dtype=np.float64).copy()
    assert out.size == heads * d and d % 2 == 0
    lib().oracle_rope(_p(out), heads, d, int(pos), float(theta))
    return out


def swiglu(g, u) -> np.ndarray:
    """fp64 g / (1 + e^-g) * u, elementwise."""
    g = np.ascontiguousarray(g, dtype=np.float64)
    u = np.ascontiguousarray(u, dtype=np.float64)
    assert g.shape == u.shape
    s = np.empty(g.shape, dtype=np.float64)
    lib().oracle_swiglu(_p(g), _p(u), g.size, _p(s))
    return s


def attn_decode(q, kq, kd, vq, vd, t: int, scale: float) -> np.ndarray:
    """fp64 out [heads][d]: softmax(scale * q . K) . V over the first t cache rows.

    q: bf16 bits [heads][d]; kq, vq: int8 codes [heads][t_cap][d]; kd, vd:
    binary16 scale bits [heads][t_cap][d/32]."""
    q = np.ascontiguousarray(q, dtype=np.uint16)
    kq = np.ascontiguousarray(kq, dtype=np.int8)
    vq = np.ascontiguousarray(vq, dtype=np.int8)
    kd = np.ascontiguousarray(kd, dtype=np.uint16)
    vd = np.ascontiguousarray(vd, dtype=np.uint16)
    heads, t_cap, d = kq.shape
    _check_k(d)
    assert q.shape == (heads, d) and vq.shape == kq.shape
    assert kd.shape == (heads, t_cap, d // 32) and vd.shape == kd.shape
    if not 1 <= t <= t_cap:
        raise ValueError("need 1 <= t <= t_cap")
    out = np.empty((heads, d), dtype=np.float64)
    lib().oracle_attn_decode(_p(q), _p(kq), _p(kd), _p(vq), _p(vd), heads, int(t), t_cap, d,
                             float(scale), _p(out))
    return out

