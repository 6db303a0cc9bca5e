"""The allocation-free decode attention (q8_attn_decode_noalloc), through the C
ABI: its output must be bit-identical to q8_attn_decode's with a caller
workspace (the same kernels; only where the chunk partials live differs), on
consecutive calls that share the static scratch -- a large context first, then
smaller ones, so a stale partial left by the first call would show -- and
within the fp32 tolerance of the fp64 oracle."""
import math

import numpy as np
import pytest
import torch

import int8_weight_streaming_amd as q8
import oracle
import workloads as wl
from gpu_helpers import assert_close, log, oracle_threads, to_dev, to_host

pytestmark = pytest.mark.gpu
D = 128
SCALE = float(np.float32(1.0 / math.sqrt(D)))


@pytest.fixture(scope="module", autouse=True)
def _setup():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    q8.load_library()
    oracle.set_threads(oracle_threads())
    yield
    torch.cuda.synchronize()


def cache(seed, heads, t, t_cap):
    g = wl.rng(seed)
    rows = heads * t_cap
    kq, kd = oracle.quantize_bf16(wl.f32_to_bf16_bits(g.standard_normal((rows, D)).astype(np.float32)))
    vq, vd = oracle.quantize_bf16(wl.f32_to_bf16_bits(g.standard_normal((rows, D)).astype(np.float32)))
    q = wl.f32_to_bf16_bits(g.standard_normal((heads, D)).astype(np.float32))
    return (q, kq.reshape(heads, t_cap, D), kd.reshape(heads, t_cap, D // 32),
            vq.reshape(heads, t_cap, D), vd.reshape(heads, t_cap, D // 32))


def test_noalloc_matches_workspace_call_on_consecutive_calls():
    # largest context of 12 heads whose partials fit the scratch, then smaller
    # ones (fewer heads and chunks), then a single-chunk call (no scratch)
    cases = [(12, 42240, 42240, 71), (3, 700, 1024, 72), (12, 4096, 4096, 73), (2, 130, 256, 74),
             (5, 40, 64, 75)]
    assert q8.attn_work_words(12, 42240) <= q8.ATTN_SCRATCH_WORDS
    for heads, t, t_cap, seed in cases:
        log(f"noalloc attention heads={heads} t={t} t_cap={t_cap} seed={seed}")
        host = cache(seed, heads, t, t_cap)
        dq, dkq, dkd, dvq, dvd = (to_dev(a) for a in host)
        y_na = q8.attn_decode_noalloc(dq, dkq, dkd, dvq, dvd, t, SCALE)
        torch.cuda.synchronize()
        y_ws = q8.attn_decode(dq, dkq, dkd, dvq, dvd, t, SCALE)
        torch.cuda.synchronize()
        a, b = to_host(y_na), to_host(y_ws)
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), (heads, t)
        ref = oracle.attn_decode(*host, t, SCALE)
        assert_close(a, ref, f"noalloc attention heads={heads} t={t}")
        del dq, dkq, dkd, dvq, dvd


def test_noalloc_repeat_and_out_buffer():
    heads, t, t_cap = 12, 2048, 2048
    host = cache(81, heads, t, t_cap)
    dev = [to_dev(a) for a in host]
    out = torch.empty((heads, D), dtype=torch.float32, device="cuda:0")
    first = to_host(q8.attn_decode_noalloc(*dev, t, SCALE, out=out)).copy()
    for _ in range(3):
        again = to_host(q8.attn_decode_noalloc(*dev, t, SCALE, out=out))
        assert np.array_equal(first.view(np.uint32), again.view(np.uint32))
