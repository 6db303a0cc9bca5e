"""q8stream: Q8_0 int8 weight streaming on MI355X (gfx950) -- Python binding.

A thin ctypes layer over ``libq8stream.so`` (the C ABI in ``include/q8stream.h``).
It only checks tensor dtypes/devices/shapes, allocates outputs with
``torch.empty`` and passes raw pointers plus the current torch stream; every
step of the computation runs in the library's HIP kernels.  There is no
fallback: if the library is missing or the device is not a gfx950, calls raise.

Names mirror the C entry points:

    quantize_weights(w)            fp32 [n][k]            -> (wq int8 [n][k], wd uint16 [n][k/32])
    quantize_act(x)                bf16 [m][k]            -> (xq int8 [m][k], xd uint16 [m][k/32])
    gemv(wq, wd, x, xd=None)       x bf16 [k] or int8 [k] -> y fp32 [n]
    gemm_skinny(wq, wd, x, xd=None) x [m][k], m <= 8      -> y fp32 [m][n]
    gemm_prefill(wq, wd, xq, xd)   xq int8 [p][k]         -> y fp32 [p][n]
    block_dots(wq, xq)             xq int8 [m][k]         -> isum int32 [m][n][k/32]
    attn_decode(q, kq, kd, vq, vd, t, scale)              -> out fp32 [heads][128]
    q4_quantize_weights(w)         fp32 [n][k]            -> (wq uint8 [n][k/2], wd uint16 [n][k/32])
    q4_gemm_skinny(wq, wd, x, xd=None) int4 weights, m <= 8 -> y fp32 [m][n]
    gemm_fused(wq, wd, x, prologue, epilogue, out=None, rope_rows=0, pos=0)
                                   W8A16 product with decode-step glue (see q8stream.h)
    rmsnorm(x, out=None)           fp32 [m][k] -> weightless RMSNorm, fp32

Binary16 scales travel as torch.uint16 tensors holding the bit patterns
(``wd.view(torch.float16)`` gives the values).
"""
from __future__ import annotations

import ctypes as C
import os
from typing import NamedTuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libq8stream.so")

Q8_OK = 0
Q8_ACT_BF16 = 0
Q8_ACT_Q8 = 1
PRO_BF16, PRO_F32, PRO_RMSNORM = 0, 1, 2
EPI_F32, EPI_ADD, EPI_SWIGLU, EPI_ROPE = 0, 1, 2, 3
MAX_BATCH = 8

EXPORTED = (
    "q8_abi_version", "q8_status_str", "q8_last_hip_error",
    "q8_quantize_weights", "q8_quantize_act", "q8_gemv", "q8_gemm_skinny",
    "q8_gemm_prefill", "q8_block_dots", "q8_attn_decode", "q8_attn_work_words",
    "q4_quantize_weights", "q4_gemm_skinny", "q8_gemm_fused", "q8_rmsnorm", "q8_attn_decode_append",
    "q8_quantize_act_fused", "q8_attn_partial_words", "q8_attn_decode_append_partials",
    "q8_gemm_attn_residual", "q8_attn_decode_noalloc", "q8_kernel_name",
    "q8_frag_code_bytes", "q8_frag_scale_bytes", "q8_pack_frag", "q8_gemm_prefill_frag",
    "q8_quantize_act_fused_frag",
)
OP_SKINNY, OP_PREFILL, OP_Q4_SKINNY, OP_PREFILL_FRAG = 0, 1, 2, 3
ATTN_SCRATCH_WORDS = 262144


class Q8Error(RuntimeError):
    def __init__(self, fn: str, status: int, text: str, hip_error: int):
        super().__init__(f"{fn} failed: {text} (status {status}, hip error {hip_error})")
        self.status = status
        self.hip_error = hip_error


_lib = None


def load_library(path: str = LIB_PATH) -> C.CDLL:
    """Load the in-tree library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with int8_weight_streaming_amd/build.py")
    L = C.CDLL(path)
    P, I64, I = C.c_void_p, C.c_int64, C.c_int
    L.q8_abi_version.restype = I
    L.q8_status_str.argtypes = [I]
    L.q8_status_str.restype = C.c_char_p
    L.q8_last_hip_error.restype = I
    L.q8_quantize_weights.argtypes = [P, I64, I64, P, P, P]
    L.q8_quantize_act.argtypes = [P, I64, I64, P, P, P]
    L.q8_gemv.argtypes = [P, P, I64, I64, I, P, P, P, P]
    L.q8_gemm_skinny.argtypes = [P, P, I64, I64, I64, I, P, P, P, P]
    L.q8_gemm_prefill.argtypes = [P, P, I64, I64, I64, P, P, P, P]
    L.q8_block_dots.argtypes = [P, I64, I64, I64, P, P, P]
    L.q8_attn_decode.argtypes = [P, P, P, P, P, I64, I64, I64, I64, C.c_float, P, P, I64, P]
    L.q8_attn_decode.restype = I
    L.q8_attn_decode_noalloc.argtypes = [P, P, P, P, P, I64, I64, I64, I64, C.c_float, P, P]
    L.q8_attn_decode_noalloc.restype = I
    L.q8_kernel_name.argtypes = [I, I64, I64, I64, I, P, I64]
    L.q8_kernel_name.restype = I
    L.q8_attn_work_words.argtypes = [I64, I64]
    L.q8_attn_work_words.restype = I64
    L.q4_quantize_weights.argtypes = [P, I64, I64, P, P, P]
    L.q4_gemm_skinny.argtypes = [P, P, I64, I64, I64, I, P, P, P, P]
    L.q8_gemm_fused.argtypes = [P, P, I64, I64, I64, I, P, I, P, I64, I64, P]
    L.q8_rmsnorm.argtypes = [P, I64, I64, P, P]
    L.q8_quantize_act_fused.argtypes = [P, I64, I64, I, P, P, P]
    L.q8_attn_partial_words.argtypes = [I64, I64]
    L.q8_attn_partial_words.restype = I64
    L.q8_attn_decode_append_partials.argtypes = [P, P, P, P, P, I64, I64, I64, I64, C.c_float, P, P, P, I64, P]
    L.q8_attn_decode_append_partials.restype = I
    L.q8_gemm_attn_residual.argtypes = [P, P, I64, I64, P, I64, I64, P, P]
    L.q8_gemm_attn_residual.restype = I
    L.q8_attn_decode_append.argtypes = [P, P, P, P, P, I64, I64, I64, I64, C.c_float, P, P, P, P, I64, P]
    L.q8_attn_decode_append.restype = I
    L.q8_frag_code_bytes.argtypes = [I64, I64]
    L.q8_frag_code_bytes.restype = I64
    L.q8_frag_scale_bytes.argtypes = [I64, I64]
    L.q8_frag_scale_bytes.restype = I64
    L.q8_pack_frag.argtypes = [P, P, I64, I64, P, P, P]
    L.q8_gemm_prefill_frag.argtypes = [P, P, I64, I64, I64, P, P, P, P]
    L.q8_quantize_act_fused_frag.argtypes = [P, I64, I64, I, P, P, P]
    for name in ("q8_quantize_weights", "q8_quantize_act", "q8_gemv", "q8_gemm_skinny",
                 "q8_gemm_prefill", "q8_block_dots", "q4_quantize_weights", "q4_gemm_skinny",
                 "q8_gemm_fused", "q8_rmsnorm", "q8_quantize_act_fused", "q8_pack_frag",
                 "q8_gemm_prefill_frag", "q8_quantize_act_fused_frag"):
        getattr(L, name).restype = I
    _lib = L
    return L


def status_str(status: int) -> str:
    return load_library().q8_status_str(int(status)).decode()


def _check(fn: str, status: int) -> None:
    if status != Q8_OK:
        L = load_library()
        raise Q8Error(fn, status, status_str(status), L.q8_last_hip_error())


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _ptr(t: torch.Tensor | None) -> int | None:
    return None if t is None else t.data_ptr()


def _need(t: torch.Tensor, name: str, dtype: torch.dtype, ndim: int) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got shape {tuple(t.shape)}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _out(t, name: str, dtype: torch.dtype, numel: int) -> torch.Tensor:
    """A caller-provided output buffer: dtype, device and contiguity as for
    inputs, and exactly `numel` elements (any shape), so no kernel writes past
    its end."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if dtype == torch.uint16:
        t = _as_bits16(t)
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.numel() != numel:
        raise ValueError(f"{name} must hold {numel} elements, got shape {tuple(t.shape)}")
    return t


def _work(work) -> int:
    """Words of a caller-provided fp32 attention workspace (0 for None)."""
    if work is None:
        return 0
    if not isinstance(work, torch.Tensor) or work.dtype != torch.float32 or not work.is_cuda \
            or not work.is_contiguous():
        raise ValueError("work must be a contiguous fp32 device tensor")
    return work.numel()


def _as_bits16(t: torch.Tensor) -> torch.Tensor:
    if t.dtype in (torch.bfloat16, torch.float16):
        return t.view(torch.uint16)
    return t


# ------------------------------------------------------------------ quantizers

def quantize_weights(w: torch.Tensor, out=None):
    """fp32 [n][k] -> (codes int8 [n][k], binary16 scale bits uint16 [n][k/32])."""
    _need(w, "w", torch.float32, 2)
    n, k = w.shape
    if out is None:
        wq = torch.empty((n, k), dtype=torch.int8, device=w.device)
        wd = torch.empty((n, k // 32), dtype=torch.uint16, device=w.device)
    else:
        wq, wd = _out(out[0], "wq", torch.int8, n * k), _out(out[1], "wd", torch.uint16, n * (k // 32))
    _check("q8_quantize_weights", load_library().q8_quantize_weights(
        _ptr(w), n, k, _ptr(wq), _ptr(wd), _stream()))
    return wq, wd


def quantize_act(x: torch.Tensor, out=None):
    """bf16 [m][k] (torch.bfloat16 or uint16 bits) -> (int8 [m][k], uint16 [m][k/32])."""
    x = _as_bits16(x)
    _need(x, "x", torch.uint16, 2)
    m, k = x.shape
    if out is None:
        xq = torch.empty((m, k), dtype=torch.int8, device=x.device)
        xd = torch.empty((m, k // 32), dtype=torch.uint16, device=x.device)
    else:
        xq, xd = _out(out[0], "xq", torch.int8, m * k), _out(out[1], "xd", torch.uint16, m * (k // 32))
    _check("q8_quantize_act", load_library().q8_quantize_act(
        _ptr(x), m, k, _ptr(xq), _ptr(xd), _stream()))
    return xq, xd


# ------------------------------------------------------------------ products

def _weights(wq, wd):
    _need(wq, "wq", torch.int8, 2)
    wd = _as_bits16(wd)
    _need(wd, "wd", torch.uint16, 2)
    n, k = wq.shape
    if tuple(wd.shape) != (n, k // 32):
        raise ValueError(f"wd must be [{n}][{k // 32}], got {tuple(wd.shape)}")
    return wd, n, k


def gemm_skinny(wq, wd, x, xd=None, out=None):
    """y fp32 [m][n] for m = x.shape[0] <= 8; x bf16 [m][k] or int8 codes with xd."""
    wd, n, k = _weights(wq, wd)
    if xd is None:
        x = _as_bits16(x)
        _need(x, "x", torch.uint16, 2)
        act = Q8_ACT_BF16
    else:
        _need(x, "x", torch.int8, 2)
        xd = _as_bits16(xd)
        _need(xd, "xd", torch.uint16, 2)
        if tuple(xd.shape) != (x.shape[0], k // 32):
            raise ValueError("xd must be [m][k/32]")
        act = Q8_ACT_Q8
    m = x.shape[0]
    if x.shape[1] != k:
        raise ValueError(f"x must have {k} columns, got {x.shape[1]}")
    y = _out(out, "out", torch.float32, m * n) if out is not None else \
        torch.empty((m, n), dtype=torch.float32, device=wq.device)
    _check("q8_gemm_skinny", load_library().q8_gemm_skinny(
        _ptr(wq), _ptr(wd), n, k, m, act, _ptr(x), _ptr(xd), _ptr(y), _stream()))
    return y


def gemv(wq, wd, x, xd=None, out=None):
    """y fp32 [n] from one activation vector x [k] (bf16, or int8 codes with xd [k/32])."""
    wd, n, k = _weights(wq, wd)
    if xd is None:
        x = _as_bits16(x)
        _need(x, "x", torch.uint16, 1)
        act = Q8_ACT_BF16
    else:
        _need(x, "x", torch.int8, 1)
        xd = _as_bits16(xd)
        _need(xd, "xd", torch.uint16, 1)
        act = Q8_ACT_Q8
    if x.shape[0] != k:
        raise ValueError(f"x must have {k} elements, got {x.shape[0]}")
    y = _out(out, "out", torch.float32, n) if out is not None else \
        torch.empty((n,), dtype=torch.float32, device=wq.device)
    _check("q8_gemv", load_library().q8_gemv(
        _ptr(wq), _ptr(wd), n, k, act, _ptr(x), _ptr(xd), _ptr(y), _stream()))
    return y


def gemm_prefill(wq, wd, xq, xd, out=None):
    """y fp32 [p][n] = Q8 x Q8 product of p activation rows."""
    wd, n, k = _weights(wq, wd)
    _need(xq, "xq", torch.int8, 2)
    xd = _as_bits16(xd)
    _need(xd, "xd", torch.uint16, 2)
    p = xq.shape[0]
    if xq.shape[1] != k or tuple(xd.shape) != (p, k // 32):
        raise ValueError("xq must be [p][k] and xd [p][k/32]")
    y = _out(out, "out", torch.float32, p * n) if out is not None else \
        torch.empty((p, n), dtype=torch.float32, device=wq.device)
    _check("q8_gemm_prefill", load_library().q8_gemm_prefill(
        _ptr(wq), _ptr(wd), n, k, p, _ptr(xq), _ptr(xd), _ptr(y), _stream()))
    return y


class Frag(NamedTuple):
    """A Q8_0 matrix in the matrix core's fragment order (q8_pack_frag): flat
    codes (int8) and scales (uint16) buffers in the layout include/q8stream.h
    states, and the row count and K of the row-major matrix it came from."""
    q: torch.Tensor
    d: torch.Tensor
    rows: int
    k: int


def frag_bytes(rows: int, k: int) -> tuple[int, int]:
    """Bytes of the fragment-order codes and scales of a [rows][k] matrix."""
    L = load_library()
    qb, db = L.q8_frag_code_bytes(rows, k), L.q8_frag_scale_bytes(rows, k)
    if qb < 0 or db < 0:
        raise ValueError(f"invalid extents rows={rows} k={k}")
    return qb, db


def pack_frag(q, d, out=None) -> Frag:
    """Rewrite a row-major Q8_0 matrix (codes [rows][k], scales [rows][k/32])
    into fragment order; out = (codes, scales) tensors of the right sizes."""
    wd, rows, k = _weights(q, d)
    qb, db = frag_bytes(rows, k)
    if out is not None:
        qf = _out(out[0], "out[0]", torch.int8, qb)
        df = _out(out[1], "out[1]", torch.uint16, db // 2)
    else:
        qf = torch.empty((qb,), dtype=torch.int8, device=q.device)
        df = torch.empty((db // 2,), dtype=torch.uint16, device=q.device)
    _check("q8_pack_frag", load_library().q8_pack_frag(
        _ptr(q), _ptr(wd), rows, k, _ptr(qf), _ptr(df), _stream()))
    return Frag(qf, df, rows, k)


def quantize_act_fused_frag(x, prologue, out=None) -> Frag:
    """fp32 rows [m][k] -> (PRO_F32: bf16 | PRO_RMSNORM: RMSNorm, bf16) -> Q8_0
    in fragment order, one launch; out = (codes, scales) of the frag sizes."""
    _need(x, "x", torch.float32, 2)
    m, k = x.shape
    qb, db = frag_bytes(m, k)
    if out is not None:
        qf = _out(out[0], "out[0]", torch.int8, qb)
        df = _out(out[1], "out[1]", torch.uint16, db // 2)
    else:
        qf = torch.empty((qb,), dtype=torch.int8, device=x.device)
        df = torch.empty((db // 2,), dtype=torch.uint16, device=x.device)
    _check("q8_quantize_act_fused_frag", load_library().q8_quantize_act_fused_frag(
        _ptr(x), m, k, prologue, _ptr(qf), _ptr(df), _stream()))
    return Frag(qf, df, m, k)


def gemm_prefill_frag(wf: Frag, xf: Frag, out=None):
    """y fp32 [p][n] = Q8 x Q8 product of fragment-order weights (n rows) and
    activations (p rows), as gemm_prefill on the row-major operands."""
    for f, name in ((wf, "wf"), (xf, "xf")):
        if not isinstance(f, Frag):
            raise TypeError(f"{name} must be a Frag (pack_frag)")
        qb, db = frag_bytes(f.rows, f.k)
        if f.q.dtype != torch.int8 or f.q.numel() != qb or not f.q.is_contiguous() or not f.q.is_cuda:
            raise ValueError(f"{name}.q must be contiguous device int8 of {qb} bytes")
        d = _as_bits16(f.d)
        if d.dtype != torch.uint16 or d.numel() * 2 != db or not d.is_contiguous() or not d.is_cuda:
            raise ValueError(f"{name}.d must be contiguous device uint16 of {db} bytes")
    if wf.k != xf.k:
        raise ValueError("wf and xf must have the same k")
    n, p, k = wf.rows, xf.rows, wf.k
    y = _out(out, "out", torch.float32, p * n) if out is not None else \
        torch.empty((p, n), dtype=torch.float32, device=wf.q.device)
    _check("q8_gemm_prefill_frag", load_library().q8_gemm_prefill_frag(
        _ptr(wf.q), _ptr(_as_bits16(wf.d)), n, k, p, _ptr(xf.q), _ptr(_as_bits16(xf.d)), _ptr(y), _stream()))
    return y


def block_dots(wq, xq, out=None):
    """Exact int32 block sums isum [m][n][k/32] (m <= 8)."""
    _need(wq, "wq", torch.int8, 2)
    _need(xq, "xq", torch.int8, 2)
    n, k = wq.shape
    m = xq.shape[0]
    if xq.shape[1] != k:
        raise ValueError("xq must be [m][k]")
    isum = _out(out, "out", torch.int32, m * n * (k // 32)) if out is not None else \
        torch.empty((m, n, k // 32), dtype=torch.int32, device=wq.device)
    _check("q8_block_dots", load_library().q8_block_dots(
        _ptr(wq), n, k, m, _ptr(xq), _ptr(isum), _stream()))
    return isum


# ------------------------------------------------------------------ decode-step glue

def gemm_fused(wq, wd, x, prologue: int, epilogue: int, out=None, rope_rows: int = 0, pos: int = 0):
    """W8A16 product (m = x.shape[0] <= 8) with a fused prologue and epilogue.

    prologue PRO_BF16: x bf16 [m][k]; PRO_F32 / PRO_RMSNORM: x fp32 [m][k].
    epilogue EPI_F32: returns fp32 [m][n]; EPI_ADD: `out` (fp32 [m][n], required)
    += the product; EPI_SWIGLU: bf16 [m][n/2]; EPI_ROPE: bf16 [m][n] (rows below
    rope_rows rotated at position pos).  Row orders as in include/q8stream.h."""
    wd, n, k = _weights(wq, wd)
    if prologue == PRO_BF16:
        x = _as_bits16(x)
        _need(x, "x", torch.uint16, 2)
    else:
        _need(x, "x", torch.float32, 2)
    m = x.shape[0]
    if x.shape[1] != k:
        raise ValueError(f"x must have {k} columns, got {x.shape[1]}")
    fp32_out = epilogue in (EPI_F32, EPI_ADD)
    shape = (m, n // 2) if epilogue == EPI_SWIGLU else (m, n)
    if out is None:
        if epilogue == EPI_ADD:
            raise ValueError("EPI_ADD needs the residual buffer as `out`")
        out = torch.empty(shape, dtype=torch.float32 if fp32_out else torch.uint16, device=wq.device)
    else:
        out = _out(out, "out", torch.float32 if fp32_out else torch.uint16, shape[0] * shape[1])
    _check("q8_gemm_fused", load_library().q8_gemm_fused(
        _ptr(wq), _ptr(wd), n, k, m, int(prologue), _ptr(x), int(epilogue), _ptr(out),
        int(rope_rows), int(pos), _stream()))
    return out


def rmsnorm(x, out=None):
    """Weightless RMSNorm (eps 1e-6) of the fp32 rows of x; `out` may be x."""
    _need(x, "x", torch.float32, 2)
    m, k = x.shape
    y = _out(out, "out", torch.float32, m * k) if out is not None else torch.empty_like(x)
    _check("q8_rmsnorm", load_library().q8_rmsnorm(_ptr(x), m, k, _ptr(y), _stream()))
    return y


def quantize_act_fused(x, prologue, out=None):
    """fp32 [m][k] -> prologue (PRO_F32: bf16 rounding; PRO_RMSNORM: weightless
    RMSNorm, then bf16 rounding) -> Q8_0 (int8 [m][k], uint16 [m][k/32]), one launch."""
    _need(x, "x", torch.float32, 2)
    m, k = x.shape
    if out is None:
        xq = torch.empty((m, k), dtype=torch.int8, device=x.device)
        xd = torch.empty((m, k // 32), dtype=torch.uint16, device=x.device)
    else:
        xq, xd = _out(out[0], "xq", torch.int8, m * k), _out(out[1], "xd", torch.uint16, m * (k // 32))
    _check("q8_quantize_act_fused", load_library().q8_quantize_act_fused(
        _ptr(x), m, k, int(prologue), _ptr(xq), _ptr(xd), _stream()))
    return xq, xd


# ------------------------------------------------------------------ int4 weights

def q4_quantize_weights(w: torch.Tensor, out=None):
    """fp32 [n][k] -> (packed int4 codes uint8 [n][k/2], binary16 scale bits uint16 [n][k/32])."""
    _need(w, "w", torch.float32, 2)
    n, k = w.shape
    if out is None:
        wq = torch.empty((n, k // 2), dtype=torch.uint8, device=w.device)
        wd = torch.empty((n, k // 32), dtype=torch.uint16, device=w.device)
    else:
        wq, wd = _out(out[0], "wq", torch.uint8, n * (k // 2)), _out(out[1], "wd", torch.uint16, n * (k // 32))
    _check("q4_quantize_weights", load_library().q4_quantize_weights(
        _ptr(w), n, k, _ptr(wq), _ptr(wd), _stream()))
    return wq, wd


def q4_gemm_skinny(wq, wd, x, xd=None, out=None):
    """y fp32 [m][n] over int4 weights (wq uint8 [n][k/2], wd [n][k/32]) for
    m = x.shape[0] <= 8; x bf16 [m][k] or int8 codes with xd [m][k/32]."""
    _need(wq, "wq", torch.uint8, 2)
    wd = _as_bits16(wd)
    _need(wd, "wd", torch.uint16, 2)
    n, k = wq.shape[0], 2 * wq.shape[1]
    if tuple(wd.shape) != (n, k // 32):
        raise ValueError(f"wd must be [{n}][{k // 32}], got {tuple(wd.shape)}")
    if xd is None:
        x = _as_bits16(x)
        _need(x, "x", torch.uint16, 2)
        act = Q8_ACT_BF16
    else:
        _need(x, "x", torch.int8, 2)
        xd = _as_bits16(xd)
        _need(xd, "xd", torch.uint16, 2)
        if tuple(xd.shape) != (x.shape[0], k // 32):
            raise ValueError("xd must be [m][k/32]")
        act = Q8_ACT_Q8
    m = x.shape[0]
    if x.shape[1] != k:
        raise ValueError(f"x must have {k} columns, got {x.shape[1]}")
    y = _out(out, "out", torch.float32, m * n) if out is not None else \
        torch.empty((m, n), dtype=torch.float32, device=wq.device)
    _check("q4_gemm_skinny", load_library().q4_gemm_skinny(
        _ptr(wq), _ptr(wd), n, k, m, act, _ptr(x), _ptr(xd), _ptr(y), _stream()))
    return y


def attn_work_words(heads: int, t: int) -> int:
    """fp32 workspace words attn_decode needs for (heads, t)."""
    return int(load_library().q8_attn_work_words(int(heads), int(t)))


def attn_decode(q, kq, kd, vq, vd, t: int, scale: float, work=None, out=None):
    """Decode attention over a Q8_0 cache: out fp32 [heads][128] from a bf16
    query [heads][128] and the first t rows of kq, vq (int8 [heads][t_cap][128])
    with their binary16 scales kd, vd ([heads][t_cap][4])."""
    q = _as_bits16(q)
    kd = _as_bits16(kd)
    vd = _as_bits16(vd)
    _need(q, "q", torch.uint16, 2)
    _need(kq, "kq", torch.int8, 3)
    _need(vq, "vq", torch.int8, 3)
    _need(kd, "kd", torch.uint16, 3)
    _need(vd, "vd", torch.uint16, 3)
    heads, t_cap, d = kq.shape
    if tuple(vq.shape) != (heads, t_cap, d) or tuple(q.shape) != (heads, d):
        raise ValueError("q [heads][d], kq and vq [heads][t_cap][d] must agree")
    if tuple(kd.shape) != (heads, t_cap, d // 32) or tuple(vd.shape) != tuple(kd.shape):
        raise ValueError("kd and vd must be [heads][t_cap][d/32]")
    need = attn_work_words(heads, t) if 1 <= t <= t_cap else 0
    if work is None and need > 0:
        work = torch.empty((need,), dtype=torch.float32, device=kq.device)
    y = _out(out, "out", torch.float32, heads * d) if out is not None else \
        torch.empty((heads, d), dtype=torch.float32, device=kq.device)
    words = _work(work)
    _check("q8_attn_decode", load_library().q8_attn_decode(
        _ptr(q), _ptr(kq), _ptr(kd), _ptr(vq), _ptr(vd), heads, int(t), t_cap, d, float(scale),
        _ptr(y), _ptr(work), words, _stream()))
    return y


def attn_decode_noalloc(q, kq, kd, vq, vd, t: int, scale: float, out=None):
    """attn_decode without a workspace: the library keeps the chunk partials in
    its static per-GPU scratch (calls on one GPU must not overlap)."""
    q = _as_bits16(q)
    kd = _as_bits16(kd)
    vd = _as_bits16(vd)
    _need(q, "q", torch.uint16, 2)
    _need(kq, "kq", torch.int8, 3)
    _need(vq, "vq", torch.int8, 3)
    _need(kd, "kd", torch.uint16, 3)
    _need(vd, "vd", torch.uint16, 3)
    heads, t_cap, d = kq.shape
    if tuple(vq.shape) != (heads, t_cap, d) or tuple(q.shape) != (heads, d):
        raise ValueError("q [heads][d], kq and vq [heads][t_cap][d] must agree")
    if tuple(kd.shape) != (heads, t_cap, d // 32) or tuple(vd.shape) != tuple(kd.shape):
        raise ValueError("kd and vd must be [heads][t_cap][d/32]")
    y = _out(out, "out", torch.float32, heads * d) if out is not None else \
        torch.empty((heads, d), dtype=torch.float32, device=kq.device)
    _check("q8_attn_decode_noalloc", load_library().q8_attn_decode_noalloc(
        _ptr(q), _ptr(kq), _ptr(kd), _ptr(vq), _ptr(vd), heads, int(t), t_cap, d, float(scale),
        _ptr(y), _stream()))
    return y


def attn_decode_append(q, kq, kd, vq, vd, t: int, scale: float, knew, vnew, work=None, out=None):
    """attn_decode after writing the Q8_0 quantization of the bf16 rows knew,
    vnew ([heads][128]) into cache row t - 1."""
    q, kd, vd, knew, vnew = (_as_bits16(a) for a in (q, kd, vd, knew, vnew))
    _need(q, "q", torch.uint16, 2)
    _need(knew, "knew", torch.uint16, 2)
    _need(vnew, "vnew", torch.uint16, 2)
    _need(kq, "kq", torch.int8, 3)
    _need(vq, "vq", torch.int8, 3)
    _need(kd, "kd", torch.uint16, 3)
    _need(vd, "vd", torch.uint16, 3)
    heads, t_cap, d = kq.shape
    if tuple(q.shape) != (heads, d) or tuple(knew.shape) != (heads, d) or tuple(vnew.shape) != (heads, d):
        raise ValueError("q, knew and vnew must be [heads][d]")
    if tuple(vq.shape) != (heads, t_cap, d) or tuple(kd.shape) != (heads, t_cap, d // 32) or \
            tuple(vd.shape) != tuple(kd.shape):
        raise ValueError("cache shapes disagree")
    need = attn_work_words(heads, t) if 1 <= t <= t_cap else 0
    if work is None and need > 0:
        work = torch.empty((need,), dtype=torch.float32, device=kq.device)
    y = _out(out, "out", torch.float32, heads * d) if out is not None else \
        torch.empty((heads, d), dtype=torch.float32, device=kq.device)
    words = _work(work)
    _check("q8_attn_decode_append", load_library().q8_attn_decode_append(
        _ptr(q), _ptr(kq), _ptr(kd), _ptr(vq), _ptr(vd), heads, int(t), t_cap, d, float(scale),
        _ptr(knew), _ptr(vnew), _ptr(y), _ptr(work), words, _stream()))
    return y


def attn_partial_words(heads: int, t: int) -> int:
    """fp32 words of the per-chunk attention partials for (heads, t)."""
    return int(load_library().q8_attn_partial_words(int(heads), int(t)))


def attn_decode_append_partials(q, kq, kd, vq, vd, t: int, scale: float, knew, vnew, work=None):
    """attn_decode_append without the combine: the per-chunk partials are left
    in `work` (fp32, attn_partial_words(heads, t) words), which is returned."""
    q, kd, vd, knew, vnew = (_as_bits16(a) for a in (q, kd, vd, knew, vnew))
    _need(q, "q", torch.uint16, 2)
    _need(knew, "knew", torch.uint16, 2)
    _need(vnew, "vnew", torch.uint16, 2)
    _need(kq, "kq", torch.int8, 3)
    _need(vq, "vq", torch.int8, 3)
    _need(kd, "kd", torch.uint16, 3)
    _need(vd, "vd", torch.uint16, 3)
    heads, t_cap, d = kq.shape
    if tuple(q.shape) != (heads, d) or tuple(knew.shape) != (heads, d) or tuple(vnew.shape) != (heads, d):
        raise ValueError("q, knew and vnew must be [heads][d]")
    if tuple(vq.shape) != (heads, t_cap, d) or tuple(kd.shape) != (heads, t_cap, d // 32) or \
            tuple(vd.shape) != tuple(kd.shape):
        raise ValueError("cache shapes disagree")
    need = attn_partial_words(heads, t) if 1 <= t <= t_cap else 0
    if work is None:
        work = torch.empty((max(need, 1),), dtype=torch.float32, device=kq.device)
    _check("q8_attn_decode_append_partials", load_library().q8_attn_decode_append_partials(
        _ptr(q), _ptr(kq), _ptr(kd), _ptr(vq), _ptr(vd), heads, int(t), t_cap, d, float(scale),
        _ptr(knew), _ptr(vnew), _ptr(work), _work(work), _stream()))
    return work


def gemm_attn_residual(wq, wd, work, t: int, h):
    """h (fp32 [1][n] or [n]) += W * bf16(a), a the attention output combined from
    the partials in `work` (attn_decode_append_partials with heads = k / 128, t)."""
    wd, n, k = _weights(wq, wd)
    h = _out(h, "h", torch.float32, n)
    _check("q8_gemm_attn_residual", load_library().q8_gemm_attn_residual(
        _ptr(wq), _ptr(wd), n, k, _ptr(work), _work(work), int(t), _ptr(h), _stream()))
    return h


def kernel_name(op: int, n: int, k: int, rows: int, act: int = Q8_ACT_BF16) -> str:
    """The kernel a product call with these extents launches on the current
    device (op OP_SKINNY, OP_PREFILL or OP_Q4_SKINNY; rows = m or p)."""
    buf = C.create_string_buffer(96)
    _check("q8_kernel_name", load_library().q8_kernel_name(
        int(op), int(n), int(k), int(rows), int(act), C.cast(buf, C.c_void_p), len(buf)))
    return buf.value.decode()
