"""Helpers shared by the GPU parity tests: host<->device copies and the fp32
acceptance rule (max-abs 2e-3 and relative L2 1e-5 against the fp64 oracle,
per call and output tensor)."""
import os
import sys

import numpy as np
import torch

MAX_ABS = 2e-3
REL_L2 = 1e-5

DEV = "cuda:0"


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(a: np.ndarray) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(DEV).view(torch.uint16)
    return torch.from_numpy(a).to(DEV)


def to_host(t: torch.Tensor) -> np.ndarray:
    t = t.detach()
    if t.dtype == torch.uint16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def assert_close(y: np.ndarray, y64: np.ndarray, what: str = "") -> None:
    y = np.asarray(y, dtype=np.float64)
    assert y.shape == y64.shape, (what, y.shape, y64.shape)
    assert np.all(np.isfinite(y)), what
    err = np.abs(y - y64)
    max_abs = float(err.max()) if err.size else 0.0
    den = float(np.linalg.norm(y64))
    rel = float(np.linalg.norm(y - y64)) / den if den > 0 else float(np.linalg.norm(y - y64))
    assert max_abs <= MAX_ABS, f"{what}: max-abs {max_abs:.3e} > {MAX_ABS}"
    assert rel <= REL_L2, f"{what}: rel-L2 {rel:.3e} > {REL_L2}"


def oracle_threads() -> int:
    n = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    return max(1, min(16, n or 1))
