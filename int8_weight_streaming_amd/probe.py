"""ctypes binding of the benchmark's measurement probes (``libq8probe.so``,
``include/q8probe.h``): the HBM read probe, the grid-barrier probe, the int8
matrix-core rate probe and the exact-fold probe.  Not part of the computation; only ``bench.py`` and the
tests load it."""
from __future__ import annotations

import ctypes as C
import os

import torch

from . import Q8Error, _ptr, _stream, status_str

_HERE = os.path.dirname(os.path.abspath(__file__))
PROBE_LIB_PATH = os.path.join(_HERE, "libq8probe.so")
EXPORTED = ("q8_probe_read", "q8_probe_barrier", "q8_probe_barrier_words", "q8_probe_mfma_i8", "q8_probe_fold")
READ_LOADS_PER_THREAD = (4, 8, 12, 16)
MFMA_I8_OPS = 32 * 32 * 32 * 2           # integer operations of one v_mfma_i32_32x32x32_i8

_lib = None


def load() -> C.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(PROBE_LIB_PATH):
        raise ImportError(f"{PROBE_LIB_PATH} is missing: build it with int8_weight_streaming_amd/build.py")
    L = C.CDLL(PROBE_LIB_PATH)
    P, I64, I = C.c_void_p, C.c_int64, C.c_int
    L.q8_probe_read.argtypes = [P, I64, I, P, P]
    L.q8_probe_read.restype = I
    L.q8_probe_barrier.argtypes = [P, I, I, P]
    L.q8_probe_barrier.restype = I
    L.q8_probe_barrier_words.restype = I64
    L.q8_probe_mfma_i8.argtypes = [I, I, P, P]
    L.q8_probe_mfma_i8.restype = I
    L.q8_probe_fold.argtypes = [I, I, P, P]
    L.q8_probe_fold.restype = I
    _lib = L
    return L


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise Q8Error(fn, status, status_str(status), 0)


def sink(device) -> torch.Tensor:
    """One int32 word the probes may write into."""
    return torch.zeros((4,), dtype=torch.int32, device=device)


def read(buf: torch.Tensor, loads_per_thread: int, sink_t: torch.Tensor) -> None:
    """Stream every byte of `buf` once with the read probe."""
    if not buf.is_cuda or not buf.is_contiguous():
        raise ValueError("buf must be a contiguous device tensor")
    nbytes = buf.numel() * buf.element_size()
    _check("q8_probe_read", load().q8_probe_read(_ptr(buf), nbytes, int(loads_per_thread), _ptr(sink_t),
                                                 _stream()))


def barrier_flags(device) -> torch.Tensor:
    """A zero-filled flag buffer for barrier()."""
    return torch.zeros((load().q8_probe_barrier_words(),), dtype=torch.int32, device=device)


def barrier(flags: torch.Tensor, workgroups: int, rounds: int) -> None:
    """Enqueue `rounds` grid-wide barriers over `workgroups` single-wave
    workgroups (rounds = 0: an empty kernel).  After synchronizing, a non-zero
    last word of `flags` means a barrier timed out and the measurement is void."""
    if flags.dtype != torch.int32 or not flags.is_cuda or flags.numel() < load().q8_probe_barrier_words():
        raise ValueError("flags must come from barrier_flags()")
    _check("q8_probe_barrier", load().q8_probe_barrier(_ptr(flags), int(workgroups), int(rounds), _stream()))


def mfma_i8(workgroups: int, iters: int, sink_t: torch.Tensor) -> int:
    """Enqueue the int8 matrix-core probe; returns its integer operation count."""
    _check("q8_probe_mfma_i8", load().q8_probe_mfma_i8(int(workgroups), int(iters), _ptr(sink_t), _stream()))
    return int(workgroups) * 4 * int(iters) * 8 * MFMA_I8_OPS


def fold(workgroups: int, iters: int, sink_t: torch.Tensor) -> int:
    """Enqueue the exact-fold probe; returns the int8 operation count of the
    block-tiles it retires."""
    _check("q8_probe_fold", load().q8_probe_fold(int(workgroups), int(iters), _ptr(sink_t), _stream()))
    return int(workgroups) * 4 * int(iters) * 4 * MFMA_I8_OPS
