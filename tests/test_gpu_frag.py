"""The prefill product on fragment-order operands (q8_pack_frag,
q8_gemm_prefill_frag) against the oracle.

* The packed layout, bit for bit, against a numpy re-layout of the row-major
  codes and scales written from the header's definition (padding rows and
  blocks zero).
* Parity with the fp64 oracle (max-abs 2e-3, relative L2 1e-5) on ragged
  shapes, edge-case weights and the P = 256 workload shapes.
* The int32 block sums bitwise on every compiled kernel form (the five the
  dispatch rule can reach at any compute-unit count), by the power-of-two
  construction of test_gpu_exact [fak
  MODEL-BASELINE-RESULTS, ACT 4 "Correctness": the tile kernel must equal the
  scalar reference bit for bit, remainder paths included]; each case asserts the
  form its shape selects.
* Repeat calls and HIP-graph replays give the same bits."""
import numpy as np
import pytest
import torch

import int8_weight_streaming_amd as q8
import oracle
import workloads as wl
from gpu_helpers import assert_close, log, oracle_threads, to_dev, to_host
from test_gpu_exact import abs_term_bound, assert_bitwise, assert_exact_regime, q8_pair

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _setup():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    q8.load_library()
    oracle.set_threads(oracle_threads())
    yield
    torch.cuda.synchronize()


def frag_layout(q, d):
    """Fragment order from its definition: codes [rows64/32][nbp][64][16] with
    lane l = i + 32h of (tile t, block b) holding codes 32b + 16h .. + 15 of row
    32t + i; scales [rows64/32][nbp/4][32][4] (row 32t + i, blocks 4g .. 4g+3)."""
    rows, k = q.shape
    nb = k // 32
    r64, nbp = (rows + 63) // 64 * 64, (nb + 3) // 4 * 4
    qp = np.zeros((r64, nbp * 32), dtype=np.int8)
    qp[:rows, :k] = q
    qf = qp.reshape(r64 // 32, 32, nbp, 2, 16).transpose(0, 2, 3, 1, 4)      # t, b, h, i, j
    dp = np.zeros((r64, nbp), dtype=np.uint16)
    dp[:rows, :nb] = d
    df = dp.reshape(r64 // 32, 32, nbp // 4, 4).transpose(0, 2, 1, 3)        # t, g, i, u
    return np.ascontiguousarray(qf).ravel(), np.ascontiguousarray(df).ravel()


def pack(q, d):
    return q8.pack_frag(to_dev(q), to_dev(d))


@pytest.mark.parametrize("rows,k", [(1, 32), (65, 96), (300, 1536), (33, 4128), (64, 256), (128, 128)])
def test_pack_frag_layout(rows, k):
    g = wl.rng(7100 + rows + k)
    q = g.integers(-127, 128, size=(rows, k)).astype(np.int8)
    d = g.integers(0, 1 << 16, size=(rows, k // 32)).astype(np.uint16)
    f = pack(q, d)
    torch.cuda.synchronize()
    qf, df = frag_layout(q, d)
    assert np.array_equal(to_host(f.q), qf)
    assert np.array_equal(to_host(f.d), df)
    # the caller-provided form writes the same bytes, padding included
    oq = torch.full((qf.size,), 5, dtype=torch.int8, device="cuda:0")
    od = torch.full((df.size,), 7, dtype=torch.int16, device="cuda:0").view(torch.uint16)
    q8.pack_frag(to_dev(q), to_dev(d), out=(oq, od))
    torch.cuda.synchronize()
    assert np.array_equal(to_host(oq), qf) and np.array_equal(to_host(od), df)


def _case(seed, n, k, p):
    g = wl.rng(seed)
    w = (g.standard_normal((n, k), dtype=np.float32) * np.float32(0.02)).astype(np.float32)
    if n > 3:
        w[1] = 0.0                                     # an all-zero row
        w[2, : min(k, 64)] = 0.0                       # zero blocks
        w[3] *= np.float32(16.0)                       # a row of another exponent range
    wq, wd = oracle.quantize_f32(w)
    xq, xd = oracle.quantize_bf16(wl.prefill_act_bf16(seed + 1, p, k))
    return wq, wd, xq, xd


@pytest.mark.parametrize("n,k,p", [(1, 32, 1), (3, 64, 2), (100, 96, 11), (65, 2080, 100), (300, 4096, 256),
                                   (33, 1536, 257), (257, 160, 300), (40, 16384, 40), (777, 2048, 95),
                                   (1000, 4128, 64), (4100, 512, 300), (2043, 256, 1000)])
def test_frag_prefill_parity(n, k, p):
    log(f"frag prefill n={n} k={k} p={p}: {q8.kernel_name(q8.OP_PREFILL_FRAG, n, k, p)}")
    wq, wd, xq, xd = _case(7200 + n + k + p, n, k, p)
    y = q8.gemm_prefill_frag(pack(wq, wd), pack(xq, xd))
    torch.cuda.synchronize()
    assert y.shape == (p, n)
    assert_close(to_host(y), oracle.q8q8(wq, wd, xq, xd), f"frag prefill n={n} k={k} p={p}")


def test_frag_prefill_p256_config():
    """The P = 256 workload: block-0 qkv, gate_up and down weights, both
    activation matrices with their special rows, quantized on the GPU."""
    cfg = wl.CONFIGS["prefill_p256"]
    xs = {wl.HIDDEN: wl.prefill_act_bf16(cfg["xa_seed"], 256, wl.HIDDEN),
          wl.INTER: wl.prefill_act_bf16(cfg["xb_seed"], 256, wl.INTER)}
    for proj, (name, n, k) in enumerate(wl.BLOCK_SHAPES):
        if name == "o":
            continue
        log(f"frag prefill p256 {name}: {q8.kernel_name(q8.OP_PREFILL_FRAG, n, k, 256)}")
        w = wl.normal_weights(wl.mimir_weight_seed(0, proj), n, k)
        dwq, dwd = q8.quantize_weights(to_dev(w))
        dxq, dxd = q8.quantize_act(to_dev(xs[k]))
        y = q8.gemm_prefill_frag(q8.pack_frag(dwq, dwd), q8.pack_frag(dxq, dxd))
        torch.cuda.synchronize()
        wq, wd = oracle.quantize_f32(w)
        xq, xd = oracle.quantize_bf16(xs[k])
        assert np.array_equal(to_host(dwq), wq) and np.array_equal(to_host(dxd), xd)
        assert_close(to_host(y), oracle.q8q8(wq, wd, xq, xd), f"frag prefill {name}")


def _forms():
    """(name, n, k, p) cases that reach the kernel forms of the dispatch rule
    (weight tiles per wave, waves per K split, and the 64 x 64 kernel for long
    prompts) on a 256-CU device, with ragged rows and K: K = 256 splits two
    steps over four waves (two waves get none); K = 4128 pads 129 blocks to
    132; K = 96 is one step, which a two-way split gives to one wave."""
    return [
        ("1 tile, K over 8 waves", 100, 1536, 40, (1, 8)),
        ("1 tile, K over 8 waves, K padded", 70, 4128, 20, (1, 8)),
        ("1 tile, K over 4 waves", 1536, 256, 384, (1, 4)),
        ("1 tile, K over 4 waves, ragged", 1530, 1536, 370, (1, 4)),
        ("1 tile, K over 4 waves, two steps", 2048, 256, 512, (1, 4)),
        ("1 tile, K over 4 waves, ragged, K padded", 2043, 4128, 500, (1, 4)),
        ("2 tiles, K over 2 waves, ragged", 2043, 1056, 1000, (2, 2)),
        ("2 tiles, K over 2 waves", 2048, 1536, 1024, (2, 2)),
        ("2 tiles, whole K", 2048, 512, 2048, (2, 1)),
        ("2 tiles, whole K, ragged", 2047, 160, 2040, (2, 1)),
        ("64 x 64 per wave", 2048, 160, 6144, "prefill_frag64_kernel<1>"),
        ("64 x 64 per wave, ragged", 2043, 96, 6140, "prefill_frag64_kernel<1>"),
        ("64 x 64 per wave, K over 2 waves", 1536, 160, 4096, "prefill_frag64_kernel<2>"),
        ("64 x 64 per wave, K over 2 waves, one step", 1530, 96, 4090, "prefill_frag64_kernel<2>"),
    ]


@pytest.mark.parametrize("name,n,k,p,form", _forms(), ids=[f[0] for f in _forms()])
def test_frag_block_sums_bitwise(name, n, k, p, form):
    got = q8.kernel_name(q8.OP_PREFILL_FRAG, n, k, p)
    log(f"frag {name} n={n} k={k} p={p}: {got}")
    if torch.cuda.get_device_properties(0).multi_processor_count != 256:
        pytest.skip("the shapes are chosen for 256 compute units")
    assert got == (form if isinstance(form, str) else "prefill_frag_kernel<%d,%d>" % form)
    wq, wd, xq, xd = q8_pair(7300 + k % 97 + p, n, k, p)
    assert_exact_regime(abs_term_bound(wq, wd, xq, xd), 0.25)
    y = q8.gemm_prefill_frag(pack(wq, wd), pack(xq, xd))
    torch.cuda.synchronize()
    assert_bitwise(to_host(y), oracle.q8q8(wq, wd, xq, xd), got)


@pytest.mark.parametrize("m,k,pro", [(1, 32, q8.PRO_F32), (37, 1536, q8.PRO_RMSNORM), (256, 1536, q8.PRO_RMSNORM),
                                      (256, 4096, q8.PRO_F32), (65, 2080, q8.PRO_RMSNORM), (64, 96, q8.PRO_F32),
                                      (130, 8224, q8.PRO_RMSNORM)])
def test_quantize_act_fused_frag(m, k, pro):
    """The fused activation quantizer writing fragment order: the oracle's codes
    and scales of the rows its prologue produces, in the layout of frag_layout,
    padding rows and blocks zero (k = 8224 is past the one-read row staging).
    The prologue's rows are the GPU norm's (checked against the oracle in
    test_gpu_fused) rounded to bf16, or the fp32 rows rounded to bf16."""
    g = wl.rng(7600 + m + k)
    h = (g.standard_normal((m, k), dtype=np.float32) * np.float32(3.0)).astype(np.float32)
    dh = to_dev(h)
    qf = torch.full((q8.frag_bytes(m, k)[0],), 3, dtype=torch.int8, device="cuda:0")
    df = torch.full((q8.frag_bytes(m, k)[1] // 2,), 5, dtype=torch.int16, device="cuda:0").view(torch.uint16)
    f = q8.quantize_act_fused_frag(dh, pro, out=(qf, df))
    rows = to_host(q8.rmsnorm(dh)) if pro == q8.PRO_RMSNORM else h
    torch.cuda.synchronize()
    xq, xd = oracle.quantize_bf16(wl.f32_to_bf16_bits(rows))
    eq, ed = frag_layout(xq, xd)
    assert np.array_equal(to_host(f.q), eq), "codes"
    assert np.array_equal(to_host(f.d), ed), "scales"
    # the same bytes as the row-major fused quantizer followed by the packing
    rq, rd = q8.quantize_act_fused(dh, pro)
    p2 = q8.pack_frag(rq, rd)
    torch.cuda.synchronize()
    assert torch.equal(p2.q, f.q) and torch.equal(p2.d.view(torch.int16), f.d.view(torch.int16))


def test_frag_reproducible_and_graph_replay():
    n, k, p = 1536, 4096, 256
    wq, wd, xq, xd = _case(7400, n, k, p)
    wf, xf = pack(wq, wd), pack(xq, xd)
    ref = q8.gemm_prefill_frag(wf, xf).clone()
    for _ in range(3):
        assert torch.equal(q8.gemm_prefill_frag(wf, xf), ref)
    out = torch.empty((p, n), dtype=torch.float32, device="cuda:0")
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        q8.gemm_prefill_frag(wf, xf, out=out)        # warm-up on the capture stream
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=s):
            q8.gemm_prefill_frag(wf, xf, out=out)
    for _ in range(3):
        out.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref)
        _ = torch.ones(1000, device="cuda:0").sum()   # eager work between replays
    torch.cuda.synchronize()


def test_frag_empty_calls_and_mismatch():
    wq, wd, xq, xd = _case(7500, 64, 64, 8)
    wf, xf = pack(wq, wd), pack(xq, xd)
    y0 = q8.gemm_prefill_frag(wf, q8.Frag(xf.q[:0], xf.d[:0], 0, 64))
    assert y0.shape == (0, 64)
    _, _, xq2, xd2 = _case(7501, 64, 96, 8)
    with pytest.raises(ValueError):
        q8.gemm_prefill_frag(wf, pack(xq2, xd2))      # different K
    with pytest.raises(ValueError):
        q8.gemm_prefill_frag(wf, q8.Frag(xf.q[:-16], xf.d, 8, 64))
