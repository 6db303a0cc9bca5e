"""The Python binding refuses caller-provided output and workspace buffers
that do not fit the call (wrong element count, dtype or layout) before
anything is launched, so no kernel can write past a buffer's end."""
import numpy as np
import pytest
import torch

import int8_weight_streaming_amd as q8
import workloads as wl
from gpu_helpers import DEV, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _setup():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    q8.load_library()
    yield
    torch.cuda.synchronize()


def test_bad_outputs_are_refused():
    n, k, m = 64, 96, 2
    wq, wd = q8.quantize_weights(to_dev(wl.normal_weights(1, n, k)))
    x = to_dev(wl.normal_act_bf16(2, m, k))
    h = torch.randn((m, k), device=DEV)
    f32 = lambda *s: torch.empty(s, dtype=torch.float32, device=DEV)
    u16 = lambda *s: torch.empty(s, dtype=torch.uint16, device=DEV)
    i8 = lambda *s: torch.empty(s, dtype=torch.int8, device=DEV)
    cases = [
        lambda: q8.gemm_skinny(wq, wd, x, out=f32(m, n - 1)),
        lambda: q8.gemm_skinny(wq, wd, x, out=u16(m, n)),
        lambda: q8.gemm_skinny(wq, wd, x, out=f32(n, m).t()),                  # not contiguous
        lambda: q8.gemv(wq, wd, x[0], out=f32(n + 1)),
        lambda: q8.quantize_act(x, out=(i8(m, k), u16(m, k // 32 - 1))),
        lambda: q8.quantize_weights(f32(n, k), out=(i8(n, k - 32), u16(n, k // 32))),
        lambda: q8.gemm_fused(wq, wd, h, q8.PRO_RMSNORM, q8.EPI_SWIGLU, out=u16(m, n)),
        lambda: q8.gemm_fused(wq, wd, h, q8.PRO_F32, q8.EPI_ADD, out=u16(m, n)),
        lambda: q8.rmsnorm(h, out=f32(m, k - 1)),
        lambda: q8.quantize_act_fused(h, q8.PRO_F32, out=(i8(m, k), u16(m, k))),
        lambda: q8.attn_decode(u16(2, 128), i8(2, 256, 128), u16(2, 256, 4), i8(2, 256, 128),
                               u16(2, 256, 4), 200, 0.1, work=torch.empty(4096, dtype=torch.int16, device=DEV)),
        lambda: q8.attn_decode(u16(2, 128), i8(2, 256, 128), u16(2, 256, 4), i8(2, 256, 128),
                               u16(2, 256, 4), 200, 0.1, out=f32(2, 127)),
    ]
    for i, call in enumerate(cases):
        with pytest.raises((ValueError, TypeError)):
            call()
            pytest.fail(f"case {i} was accepted")
    # the right buffers are accepted, also as other shapes of the same size
    y = f32(m * n)
    q8.gemm_skinny(wq, wd, x, out=y)
    s = torch.empty((m, n // 2), dtype=torch.bfloat16, device=DEV)
    q8.gemm_fused(wq, wd, h, q8.PRO_RMSNORM, q8.EPI_SWIGLU, out=s)
    torch.cuda.synchronize()
    assert torch.isfinite(y).all()
