"""Batch behaviour of the decode products: every output row depends on its own
activation row only.

The batched products read each weight once for all m activation rows [Frigg
README, Finding 8: one pass over the weights serves the whole batch]; no form
may mix rows.  Changing the other rows of a batch must leave a row's result
bit for bit unchanged, on every dispatch form (vector-ALU layouts at every
batch, the matrix-core forms at batch 2-8: tall, twelve-way, half-fragment
eight-way and four-way K splits; int4 weights; Q8 activations).  Bitwise
equality across different batch sizes is not promised (each batch size may
take another kernel and summation order); within a batch size it is."""
import numpy as np
import pytest
import torch

import int8_weight_streaming_amd as q8
import workloads as wl
from gpu_helpers import log, to_dev

pytestmark = pytest.mark.gpu

# (name, n as a function of the compute-unit count, k)
SHAPES = [("tall", lambda c: 128 * c + 7, 1536), ("qkv", lambda c: 18 * c, 1536),
          ("down", lambda c: 1536, 4096), ("short, K a multiple of 512 only", lambda c: 300, 2560),
          ("ragged K tile", lambda c: 77, 992)]
FORMATS = ["q8 weights, bf16 rows", "q8 weights, q8 rows", "int4 weights, bf16 rows"]


@pytest.fixture(scope="module", autouse=True)
def _setup():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    q8.load_library()
    yield
    torch.cuda.synchronize()


def product(fmt, w, x):
    if fmt == "q8 weights, bf16 rows":
        return q8.gemm_skinny(*w, x)
    if fmt == "q8 weights, q8 rows":
        xq, xd = q8.quantize_act(x)
        return q8.gemm_skinny(*w, xq, xd)
    return q8.q4_gemm_skinny(*w, x)


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("name,nf,k", SHAPES, ids=[s[0] for s in SHAPES])
@pytest.mark.parametrize("m", [2, 3, 5, 8])
def test_rows_independent_within_batch(fmt, name, nf, k, m):
    c = torch.cuda.get_device_properties(0).multi_processor_count
    n = nf(c)
    if fmt.startswith("int4") and k % 32:
        pytest.skip("int4 needs whole blocks")
    w32 = to_dev(wl.normal_weights(4100 + k % 89, n, k))
    w = q8.q4_quantize_weights(w32) if fmt.startswith("int4") else q8.quantize_weights(w32)
    del w32
    op = q8.OP_Q4_SKINNY if fmt.startswith("int4") else q8.OP_SKINNY
    act = q8.Q8_ACT_Q8 if fmt == "q8 weights, q8 rows" else q8.Q8_ACT_BF16
    log(f"rows {fmt} {name} n={n} k={k} m={m}: {q8.kernel_name(op, n, k, m, act)}")
    g = wl.rng(4200 + m)
    a = wl.f32_to_bf16_bits(g.standard_normal((m, k)).astype(np.float32))
    b = a.copy()
    # rows 1 .. m - 2 replaced (row 0 and row m - 1 kept; for m = 2 row 1 is
    # replaced and row 0 checked)
    keep = [0] if m == 2 else [0, m - 1]
    other = [i for i in range(m) if i not in keep]
    b[other] = wl.f32_to_bf16_bits(3.0 * g.standard_normal((len(other), k)).astype(np.float32))
    ya = product(fmt, w, to_dev(a))
    yb = product(fmt, w, to_dev(b))
    torch.cuda.synchronize()
    assert not torch.equal(ya[other], yb[other])
    for i in keep:
        assert torch.equal(ya[i].view(torch.int32), yb[i].view(torch.int32)), (fmt, name, m, i)
