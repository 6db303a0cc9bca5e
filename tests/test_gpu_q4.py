"""GPU parity of the int4-weight path: the HIP quantizer and the batch 1..8
products, called through the C ABI, against the CPU oracle on identical seeded
inputs.

Packed codes and scales must match bit for bit; fp32 products must be within
max-abs 2e-3 and relative L2 1e-5 of the fp64 oracle (or within the fp32
summation bound where the weights span a wide range)."""
import numpy as np
import pytest
import torch

import int8_weight_streaming_amd as q8
import oracle
import workloads as wl
from gpu_helpers import DEV, assert_close, log, oracle_threads, to_dev, to_host
from test_gpu_parity import edge_weights, mixed_weights

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _setup():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    q8.load_library()
    oracle.set_threads(oracle_threads())
    yield
    torch.cuda.synchronize()


def _check_quant(w):
    log(f"q4 quantize {w.shape}")
    wq, wd = q8.q4_quantize_weights(to_dev(w))
    torch.cuda.synchronize()
    oq, od = oracle.q4_quantize_f32(w)
    gq, gd = to_host(wq), to_host(wd)
    assert np.array_equal(gd, od), f"scales differ at {np.argwhere(gd != od)[:5]}"
    assert np.array_equal(gq, oq), f"codes differ at {np.argwhere(gq != oq)[:5]}"
    return oq, od


@pytest.mark.parametrize("n,k", [(1, 32), (3, 64), (7, 96), (33, 160), (129, 1536), (1000, 4096)])
def test_q4_quantize_mixed(n, k):
    _check_quant(mixed_weights(9000 + n + k, n, k))


def test_q4_quantize_mimir_block():
    for proj, (_, n, k) in enumerate(wl.BLOCK_SHAPES):
        _check_quant(wl.normal_weights(wl.mimir_weight_seed(0, proj), n, k))


def _run(wq, wd, x=None, xq=None, xd=None):
    dq, dd = to_dev(wq), to_dev(wd)
    if xq is None:
        y = q8.q4_gemm_skinny(dq, dd, to_dev(x))
    else:
        y = q8.q4_gemm_skinny(dq, dd, to_dev(xq), to_dev(xd))
    torch.cuda.synchronize()
    return to_host(y)


SHAPES = [(1, 32), (5, 64), (63, 96), (65, 1536), (1000, 2048), (1536, 1536), (1536, 4096),
          (4097, 160), (300, 20480), (77, 5120)]


@pytest.mark.parametrize("n,k", SHAPES)
@pytest.mark.parametrize("m", [1, 2, 3, 8])
def test_q4_skinny_bf16(n, k, m):
    log(f"q4 skinny bf16 n={n} k={k} m={m}")
    wq, wd = oracle.q4_quantize_f32(edge_weights(9100 + n + k, n, k))
    x = wl.normal_act_bf16(9101 + m, m, k)
    assert_close(_run(wq, wd, x), oracle.w4a16(wq, wd, x), f"q4 bf16 n={n} k={k} m={m}")


@pytest.mark.parametrize("n,k", SHAPES)
@pytest.mark.parametrize("m", [1, 4, 5, 8])
def test_q4_skinny_q8(n, k, m):
    log(f"q4 skinny q8 n={n} k={k} m={m}")
    wq, wd = oracle.q4_quantize_f32(edge_weights(9200 + n + k, n, k))
    xq, xd = oracle.quantize_bf16(wl.normal_act_bf16(9201 + m, m, k))
    assert_close(_run(wq, wd, xq=xq, xd=xd), oracle.q4q8(wq, wd, xq, xd), f"q4 q8 n={n} k={k} m={m}")


@pytest.mark.parametrize("m", [1, 2, 4, 6, 8])
def test_q4_skinny_tall_ragged(m):
    """The 16-lane-group layout (enough 32-row tiles at every batch size), with a
    ragged last tile."""
    n, k = 65536 + 37, 1536
    log(f"q4 tall ragged m={m}")
    wq, wd = oracle.q4_quantize_f32(wl.normal_weights(9300 + m, n, k))
    x = wl.normal_act_bf16(9301 + m, m, k)
    assert_close(_run(wq, wd, x), oracle.w4a16(wq, wd, x), f"q4 tall bf16 m={m}")
    xq, xd = oracle.quantize_bf16(x)
    assert_close(_run(wq, wd, xq=xq, xd=xd), oracle.q4q8(wq, wd, xq, xd), f"q4 tall q8 m={m}")


@pytest.mark.parametrize("n,k,m", [(77, 1536, 1), (300, 20480, 2), (40000, 1536, 8)])
def test_q4_extreme_range_summation_bound(n, k, m):
    """Weights up to 2^8: held to the fp32 summation bound (K + 2) * 2^-24 *
    sum |c d x| instead of the fixed 2e-3."""
    log(f"q4 extreme n={n} k={k} m={m}")
    wq, wd = oracle.q4_quantize_f32(mixed_weights(9400 + n, n, k))
    x = wl.normal_act_bf16(9401 + n, m, k)
    c = oracle.q4_unpack(wq).astype(np.float64)
    s = np.repeat(wd.view(np.float16).astype(np.float64), 32, axis=1)
    absum = np.abs(wl.bf16_bits_to_f32(x).astype(np.float64)) @ (np.abs(c) * s).T
    err = np.abs(_run(wq, wd, x).astype(np.float64) - oracle.w4a16(wq, wd, x))
    assert np.all(err <= (k + 2) * 2.0 ** -24 * absum)


def test_q4_lm_head_full():
    """The lm_head shape 262144 x 1536 in int4: the quantizer bit for bit on the
    whole matrix, the batch-1 product on every row (bf16 and Q8 activations),
    batch 8 on sampled rows."""
    cfg = wl.CONFIGS["lm_head_gemv_262144x1536_b1"]
    log("q4 lm_head: generating 262144 x 1536")
    w = wl.normal_weights(cfg["w_seed"], cfg["n"], cfg["k"])
    oq, od = _check_quant(w)
    del w
    x = wl.rms_unit_act_bf16(cfg["x_seed"], cfg["k"])
    assert_close(_run(oq, od, x), oracle.w4a16(oq, od, x), "q4 lm_head b1")
    xq, xd = oracle.quantize_bf16(x)
    assert_close(_run(oq, od, xq=xq, xd=xd), oracle.q4q8(oq, od, xq, xd), "q4 lm_head b1 q8")
    x8 = wl.normal_act_bf16(9501, 8, cfg["k"])
    y8 = _run(oq, od, x8)
    rows = np.sort(wl.rng(9502).choice(cfg["n"], size=4096, replace=False))
    rows = np.concatenate([rows, [0, cfg["n"] - 1]])
    assert_close(y8[:, rows], oracle.w4a16(oq, od, x8, rows=rows), "q4 lm_head b8 sampled")


def test_q4_one_hot_gives_scaled_code():
    """x = e_k selects one weight: y = code * scale exactly (one exact product
    per row, everything else adds zeros)."""
    n, k = 200, 1536
    wq, wd = oracle.q4_quantize_f32(wl.normal_weights(9600, n, k))
    c = oracle.q4_unpack(wq)
    s = wd.view(np.float16).astype(np.float64)
    kk = [0, 15, 16, 31, 32, 777, k - 1]
    x = np.zeros((len(kk), k), dtype=np.float32)
    for i, j in enumerate(kk):
        x[i, j] = 1.0
    y = _run(wq, wd, wl.f32_to_bf16_bits(x))
    for i, j in enumerate(kk):
        assert np.array_equal(y[i].astype(np.float64), c[:, j] * s[:, j // 32]), j


def test_q4_repeat_graph_and_guard_bands():
    n, k, m = 8192, 1536, 4
    wq, wd = oracle.q4_quantize_f32(wl.normal_weights(9700, n, k))
    dq, dd = to_dev(wq), to_dev(wd)
    dx = to_dev(wl.normal_act_bf16(9701, m, k))
    ref = q8.q4_gemm_skinny(dq, dd, dx).clone()
    for _ in range(3):
        assert torch.equal(q8.q4_gemm_skinny(dq, dd, dx), ref)
    guard = 4096
    y_buf = torch.full((m * n + guard,), 7.0, dtype=torch.float32, device=DEV)
    out = y_buf[: m * n].view(m, n)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        q8.q4_gemm_skinny(dq, dd, dx, out=out)
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        q8.q4_gemm_skinny(dq, dd, dx, out=out)
    for _ in range(3):
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref)
        assert torch.all(y_buf[m * n:] == 7.0)
        q8.q4_gemm_skinny(dq, dd, dx)
        torch.cuda.synchronize()
    # the quantizer writes exactly n*k/2 code bytes and n*k/32 scales
    w = to_dev(edge_weights(9702, 100, 96))
    wq_buf = torch.full((100 * 48 + guard,), 0x5A, dtype=torch.uint8, device=DEV)
    wd_buf = torch.full((100 * 3 + guard,), 0x1234, dtype=torch.int16, device=DEV)
    q8.q4_quantize_weights(w, out=(wq_buf[: 100 * 48].view(100, 48),
                                   wd_buf[: 300].view(torch.uint16).view(100, 3)))
    torch.cuda.synchronize()
    assert torch.all(wq_buf[100 * 48:] == 0x5A) and torch.all(wd_buf[300:] == 0x1234)


def test_q4_empty_calls_are_noops():
    y = q8.q4_gemm_skinny(torch.empty((0, 32), dtype=torch.uint8, device=DEV),
                          torch.empty((0, 2), dtype=torch.uint16, device=DEV),
                          torch.zeros((2, 64), dtype=torch.uint16, device=DEV))
    assert y.shape == (2, 0)
    wq = torch.zeros((4, 32), dtype=torch.uint8, device=DEV)
    wd = torch.zeros((4, 2), dtype=torch.uint16, device=DEV)
    y = q8.q4_gemm_skinny(wq, wd, torch.zeros((0, 64), dtype=torch.uint16, device=DEV))
    assert y.shape == (0, 4)
    with pytest.raises(q8.Q8Error):
        q8.q4_gemm_skinny(wq, wd, torch.zeros((9, 64), dtype=torch.uint16, device=DEV))
