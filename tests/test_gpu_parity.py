"""GPU parity: the HIP path, called through the C ABI, against the CPU oracle on
identical seeded inputs.

Integer outputs (codes, scales, int32 block sums) must match bit for bit; fp32
outputs must be within max-abs 2e-3 and relative L2 1e-5 of the fp64 oracle, and
equal it bit for bit where the construction makes every fp32 step exact."""
import numpy as np
import pytest
import torch

import int8_weight_streaming_amd as q8
import oracle
import workloads as wl
from gpu_helpers import DEV, assert_close, log, oracle_threads, to_dev, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _setup():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    q8.load_library()
    oracle.set_threads(oracle_threads())
    yield
    torch.cuda.synchronize()


def mixed_weights(seed, n, k):
    """fp32 rows mixing N(0, 0.02) blocks with zero, negative-zero, tiny
    (binary16-subnormal or zero scale), wide-range and exact-half blocks."""
    g = wl.rng(seed)
    w = (g.standard_normal((n, k)) * 0.02).astype(np.float32)
    blocks = w.reshape(-1, 32)
    nbt = blocks.shape[0]
    kinds = g.integers(0, 8, size=nbt)
    for i in np.nonzero(kinds == 1)[0]:
        blocks[i] = 0.0
    for i in np.nonzero(kinds == 2)[0]:
        blocks[i] = -0.0
    for i in np.nonzero(kinds == 3)[0]:
        blocks[i] = (g.standard_normal(32) * 10.0 ** g.integers(-9, -3)).astype(np.float32)
    for i in np.nonzero(kinds == 4)[0]:
        blocks[i] = (g.standard_normal(32) * np.exp2(g.integers(-30, 8, size=32))).astype(np.float32)
    for i in np.nonzero(kinds == 5)[0]:
        e = int(g.integers(-8, 3))
        v = (g.integers(0, 127, size=32) + 0.5) * 2.0 ** e * np.where(g.integers(0, 2, size=32) == 0, -1, 1)
        v[int(g.integers(0, 32))] = 127 * 2.0 ** e
        blocks[i] = v.astype(np.float32)
    return w


def edge_weights(seed, n, k):
    """N(0, 0.02) rows with the quantizer's edge cases at realistic magnitude:
    zero and negative-zero blocks, tiny blocks (binary16-subnormal or zero
    scale), wide dynamic range below 2^-4, and exact halves of 2^-8..2^-6."""
    g = wl.rng(seed)
    w = (g.standard_normal((n, k)) * 0.02).astype(np.float32)
    blocks = w.reshape(-1, 32)
    kinds = g.integers(0, 8, size=blocks.shape[0])
    for i in np.nonzero(kinds == 1)[0]:
        blocks[i] = 0.0
    for i in np.nonzero(kinds == 2)[0]:
        blocks[i] = -0.0
    for i in np.nonzero(kinds == 3)[0]:
        blocks[i] = (g.standard_normal(32) * 10.0 ** g.integers(-9, -3)).astype(np.float32)
    for i in np.nonzero(kinds == 4)[0]:
        blocks[i] = (g.standard_normal(32) * np.exp2(g.integers(-30, -4, size=32))).astype(np.float32)
    for i in np.nonzero(kinds == 5)[0]:
        e = int(g.integers(-8, -5))
        v = (g.integers(0, 127, size=32) + 0.5) * 2.0 ** e * np.where(g.integers(0, 2, size=32) == 0, -1, 1)
        v[int(g.integers(0, 32))] = 127 * 2.0 ** e
        blocks[i] = v.astype(np.float32)
    return w


def assert_within_summation_bound(y, wq, wd, x, what=""):
    """Inputs of any magnitude: |y - y64| <= (K + 2) * 2^-24 * sum_k |q s x|,
    the classical bound for fp32 summation of K exact products in any order
    plus one rounding of the block scale product."""
    k = wq.shape[1]
    s = np.repeat(wd.view(np.float16).astype(np.float64), 32, axis=1)
    absum = np.abs(wl.bf16_bits_to_f32(x).astype(np.float64)) @ (np.abs(wq.astype(np.float64)) * s).T
    err = np.abs(np.asarray(y, dtype=np.float64) - oracle.w8a16(wq, wd, x))
    bound = (k + 2) * 2.0 ** -24 * absum
    assert np.all(err <= bound), f"{what}: worst err/bound {np.max(err / np.maximum(bound, 1e-300)):.3f}"


# ------------------------------------------------------------------ quantizers

def _check_quant_w(w):
    log(f"quantize_weights {w.shape}")
    wq, wd = q8.quantize_weights(to_dev(w))
    torch.cuda.synchronize()
    oq, od = oracle.quantize_f32(w)
    gq, gd = to_host(wq), to_host(wd)
    assert np.array_equal(gd, od), f"scales differ at {np.argwhere(gd != od)[:5]}"
    assert np.array_equal(gq, oq), f"codes differ at {np.argwhere(gq != oq)[:5]}"


@pytest.mark.parametrize("n,k", [(1, 32), (3, 64), (7, 96), (33, 160), (129, 1536), (1000, 4096)])
def test_quantize_weights_mixed(n, k):
    _check_quant_w(mixed_weights(1000 + n + k, n, k))


def test_quantize_weights_gemv_1536():
    cfg = wl.CONFIGS["gemv_1536x1536_b1"]
    _check_quant_w(wl.normal_weights(cfg["w_seed"], cfg["n"], cfg["k"]))


def test_quantize_weights_lm_head_full():
    cfg = wl.CONFIGS["lm_head_gemv_262144x1536_b1"]
    _check_quant_w(wl.normal_weights(cfg["w_seed"], cfg["n"], cfg["k"]))


@pytest.mark.parametrize("block", [0, 31])
def test_quantize_weights_mimir_block(block):
    for proj, (_, n, k) in enumerate(wl.BLOCK_SHAPES):
        _check_quant_w(wl.normal_weights(wl.mimir_weight_seed(block, proj), n, k))


def _check_quant_x(x_bits):
    log(f"quantize_act {x_bits.shape}")
    xq, xd = q8.quantize_act(to_dev(x_bits))
    torch.cuda.synchronize()
    oq, od = oracle.quantize_bf16(x_bits)
    assert np.array_equal(to_host(xd), od)
    assert np.array_equal(to_host(xq), oq)


def test_quantize_act_special_and_prefill_rows():
    _check_quant_x(wl.f32_to_bf16_bits(wl.special_rows_f32(3, 1536)))
    _check_quant_x(wl.prefill_act_bf16(wl.CONFIGS["prefill_p256"]["xa_seed"], 256, 1536))
    _check_quant_x(wl.prefill_act_bf16(wl.CONFIGS["prefill_p256"]["xb_seed"], 256, 4096))
    _check_quant_x(wl.normal_act_bf16(7, 8, 96))


def test_quantize_act_all_bf16_patterns():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = wl.bf16_bits_to_f32(bits)
    keep = bits[np.isfinite(vals) & (np.abs(vals) <= np.float32(8e6))]
    keep = keep[np.argsort(np.abs(wl.bf16_bits_to_f32(keep)), kind="stable")]
    pad = (-keep.size) % 1024
    x = np.concatenate([keep, np.zeros(pad, dtype=np.uint16)]).reshape(-1, 1024)
    _check_quant_x(x)
    g = wl.rng(12)
    _check_quant_x(x[:, g.permutation(1024)])


# ------------------------------------------------------------------ decode products

def _w8a16_case(n, k, m, seed, mixed=False):
    w = edge_weights(seed, n, k) if mixed else wl.normal_weights(seed, n, k)
    wq, wd = oracle.quantize_f32(w)
    x = wl.normal_act_bf16(seed + 1, m, k)
    return wq, wd, x


def _run_skinny(wq, wd, x, xq=None, xd=None):
    dq, dd = to_dev(wq), to_dev(wd)
    if xq is None:
        y = q8.gemm_skinny(dq, dd, to_dev(x))
    else:
        y = q8.gemm_skinny(dq, dd, to_dev(xq), to_dev(xd))
    torch.cuda.synchronize()
    return to_host(y)


SMALL_SHAPES = [(1, 32), (5, 64), (63, 96), (64, 1536), (65, 1536), (1000, 4096),
                (4097, 160), (1536, 4096), (300, 20480)]


@pytest.mark.parametrize("n,k", SMALL_SHAPES)
@pytest.mark.parametrize("m", [1, 2, 3, 8])
def test_skinny_bf16_small(n, k, m):
    log(f"skinny bf16 n={n} k={k} m={m}")
    wq, wd, x = _w8a16_case(n, k, m, 2000 + n + k, mixed=True)
    y = _run_skinny(wq, wd, x)
    assert_close(y, oracle.w8a16(wq, wd, x), f"bf16 n={n} k={k} m={m}")


@pytest.mark.parametrize("n,k", SMALL_SHAPES)
@pytest.mark.parametrize("m", [1, 4, 5, 8])
def test_skinny_q8_small(n, k, m):
    log(f"skinny q8 n={n} k={k} m={m}")
    wq, wd, x = _w8a16_case(n, k, m, 3000 + n + k, mixed=True)
    xq, xd = oracle.quantize_bf16(x)
    y = _run_skinny(wq, wd, x, xq, xd)
    assert_close(y, oracle.q8q8(wq, wd, xq, xd), f"q8 n={n} k={k} m={m}")


@pytest.mark.parametrize("n,k,m", [(77, 1536, 1), (300, 20480, 2), (4097, 4096, 8), (40000, 1536, 3)])
def test_skinny_extreme_range_summation_bound(n, k, m):
    """Weights up to 2^8 in magnitude: the fixed 2e-3 bound does not scale, so
    the product is held to the summation error bound instead."""
    log(f"skinny extreme n={n} k={k} m={m}")
    w = mixed_weights(2500 + n + k, n, k)
    wq, wd = oracle.quantize_f32(w)
    x = wl.normal_act_bf16(2501 + n, m, k)
    assert_within_summation_bound(_run_skinny(wq, wd, x), wq, wd, x, f"extreme n={n} k={k} m={m}")


@pytest.mark.parametrize("m", [1, 2, 4, 6, 7, 8])
def test_skinny_large_rows_ragged(m):
    """Enough rows for the 16-lane-group layout, with a ragged last tile."""
    n, k = 33000, 1536
    log(f"skinny large ragged m={m}")
    wq, wd, x = _w8a16_case(n, k, m, 4000 + m)
    assert_close(_run_skinny(wq, wd, x), oracle.w8a16(wq, wd, x), f"bf16 large m={m}")
    xq, xd = oracle.quantize_bf16(x)
    assert_close(_run_skinny(wq, wd, x, xq, xd), oracle.q8q8(wq, wd, xq, xd), f"q8 large m={m}")


@pytest.mark.parametrize("m", [3, 8])
def test_skinny_very_tall_ragged(m):
    """More than four 32-row tiles per compute unit (the tall layout at every
    batch size), with a ragged last tile."""
    n, k = 65536 + 37, 1536
    log(f"skinny very tall ragged m={m}")
    wq, wd, x = _w8a16_case(n, k, m, 4100 + m, mixed=True)
    assert_close(_run_skinny(wq, wd, x), oracle.w8a16(wq, wd, x), f"bf16 very tall m={m}")


@pytest.mark.parametrize("m", [1, 3, 8])
def test_skinny_subnormal_bf16_activations(m):
    """bf16-subnormal activations (in contract: finite) times large weights, so
    that every output lands in fp32's normal range: a flush of subnormal inputs
    or products to zero anywhere on the path would show as a wrong result."""
    n, k = 300, 1536
    g = wl.rng(4200 + m)
    w = (g.standard_normal((n, k)) * 1.0e4).astype(np.float32)
    wq, wd = oracle.quantize_f32(w)
    x = (g.integers(1, 128, size=(m, k)) | (g.integers(0, 2, size=(m, k)) << 15)).astype(np.uint16)
    assert np.all(wl.bf16_bits_to_f32(x) != 0) and np.all(np.abs(wl.bf16_bits_to_f32(x)) < 2.0 ** -126)
    y64 = oracle.w8a16(wq, wd, x)
    assert np.all(np.abs(y64) < 1e-20) and np.linalg.norm(y64) > 0
    assert_within_summation_bound(_run_skinny(wq, wd, x), wq, wd, x, f"subnormal x m={m}")
    y = _run_skinny(wq, wd, x).astype(np.float64)
    assert np.linalg.norm(y - y64) <= 1e-5 * np.linalg.norm(y64), f"subnormal x m={m}: rel-L2"


def test_gemv_1536_config():
    cfg = wl.CONFIGS["gemv_1536x1536_b1"]
    w = wl.normal_weights(cfg["w_seed"], cfg["n"], cfg["k"])
    x = wl.normal_act_bf16(cfg["x_seed"], 1, cfg["k"])
    wq, wd = q8.quantize_weights(to_dev(w))
    y = q8.gemv(wq, wd, to_dev(x[0]))
    torch.cuda.synchronize()
    oq, od = oracle.quantize_f32(w)
    assert np.array_equal(to_host(wq), oq) and np.array_equal(to_host(wd), od)
    assert_close(to_host(y)[None, :], oracle.w8a16(oq, od, x), "gemv 1536")


def test_gemv_lm_head_config_full():
    cfg = wl.CONFIGS["lm_head_gemv_262144x1536_b1"]
    log("lm_head gemv: generating 262144 x 1536")
    w = wl.normal_weights(cfg["w_seed"], cfg["n"], cfg["k"])
    x = wl.rms_unit_act_bf16(cfg["x_seed"], cfg["k"])
    wq, wd = q8.quantize_weights(to_dev(w))
    y = q8.gemv(wq, wd, to_dev(x[0]))
    torch.cuda.synchronize()
    oq, od = oracle.quantize_f32(w)
    del w
    assert np.array_equal(to_host(wq), oq) and np.array_equal(to_host(wd), od)
    assert_close(to_host(y)[None, :], oracle.w8a16(oq, od, x), "lm_head gemv")
    # the Q8-activation form on the same weights
    xq, xd = oracle.quantize_bf16(x)
    yq = q8.gemv(wq, wd, to_dev(xq[0]), to_dev(xd[0]))
    torch.cuda.synchronize()
    assert_close(to_host(yq)[None, :], oracle.q8q8(oq, od, xq, xd), "lm_head gemv q8")


@pytest.mark.parametrize("m", [2, 8])
def test_skinny_lm_head_full_batches(m):
    """The full 262144 x 1536 lm_head at batch 2 and 8 (the matrix-core form
    with bf16 activations, the vector form with Q8 activations) against the
    oracle on 4096 sampled rows."""
    cfg = wl.CONFIGS["lm_head_gemv_262144x1536_b1"]
    log(f"lm_head full m={m}: generating 262144 x 1536")
    w = wl.normal_weights(cfg["w_seed"], cfg["n"], cfg["k"])
    x = wl.normal_act_bf16(7600 + m, m, cfg["k"])
    oq, od = oracle.quantize_f32(w)                   # the oracle's codes, uploaded
    del w
    wq, wd = to_dev(oq), to_dev(od)
    rows = np.sort(wl.rng(7700 + m).choice(cfg["n"], size=4096, replace=False))
    log(f"lm_head full m={m}: {q8.kernel_name(q8.OP_SKINNY, cfg['n'], cfg['k'], m, q8.Q8_ACT_BF16)}")
    y = q8.gemm_skinny(wq, wd, to_dev(x))
    torch.cuda.synchronize()
    assert_close(to_host(y)[:, rows], oracle.w8a16(oq, od, x, rows=rows), f"lm_head bf16 m={m}")
    xq, xd = oracle.quantize_bf16(x)
    yq = q8.gemm_skinny(wq, wd, to_dev(xq), to_dev(xd))
    torch.cuda.synchronize()
    assert_close(to_host(yq)[:, rows], oracle.q8q8(oq, od, xq, xd, rows=rows), f"lm_head q8 m={m}")


def test_lm_head_row_shards_equal_rows_of_whole():
    """Splitting the lm_head's rows over G GPUs (G = 2, 4, 8) is exact: one
    GPU's share (262144 / G rows, its real shape) gives bit for bit the same
    rows as the whole product when both take the same kernel form (asserted),
    at batch 1 (bf16 and Q8 activations) and batch 8; the smallest share is
    also checked against the oracle on sampled rows."""
    cfg = wl.CONFIGS["lm_head_gemv_262144x1536_b1"]
    n, k = cfg["n"], cfg["k"]
    log("lm_head shards: generating 262144 x 1536")
    w = wl.normal_weights(cfg["w_seed"], n, k)
    oq, od = oracle.quantize_f32(w)
    del w
    wq, wd = to_dev(oq), to_dev(od)
    x1 = wl.rms_unit_act_bf16(cfg["x_seed"], k)
    x8 = wl.normal_act_bf16(7800, 8, k)
    xq, xd = oracle.quantize_bf16(x1)
    whole = {"b1 bf16": to_host(q8.gemm_skinny(wq, wd, to_dev(x1))),
             "b1 q8": to_host(q8.gemm_skinny(wq, wd, to_dev(xq), to_dev(xd))),
             "b8 bf16": to_host(q8.gemm_skinny(wq, wd, to_dev(x8)))}
    for g in (2, 4, 8):
        rows = n // g
        for s in (0, g - 1):
            sq, sd = wq[s * rows:(s + 1) * rows], wd[s * rows:(s + 1) * rows]
            part = {"b1 bf16": q8.gemm_skinny(sq, sd, to_dev(x1)),
                    "b1 q8": q8.gemm_skinny(sq, sd, to_dev(xq), to_dev(xd)),
                    "b8 bf16": q8.gemm_skinny(sq, sd, to_dev(x8))}
            torch.cuda.synchronize()
            for key, y in part.items():
                m, act = (8 if key.startswith("b8") else 1), (q8.Q8_ACT_Q8 if key.endswith("q8") else q8.Q8_ACT_BF16)
                name = q8.kernel_name(q8.OP_SKINNY, rows, k, m, act)
                log(f"shard {s} of {g} ({rows} rows) {key}: {name}")
                assert name == q8.kernel_name(q8.OP_SKINNY, n, k, m, act)
                assert np.array_equal(to_host(y).view(np.int32),
                                      whole[key][:, s * rows:(s + 1) * rows].view(np.int32)), (g, s, key)
    rows = n // 8
    pick = np.sort(wl.rng(7801).choice(rows, size=512, replace=False))
    y = to_host(q8.gemm_skinny(wq[:rows], wd[:rows], to_dev(x1)))
    assert_close(y[:, pick], oracle.w8a16(oq[:rows], od[:rows], x1, rows=pick), "lm_head shard of 8")


@pytest.mark.parametrize("m", [2, 4, 8])
def test_skinny_mimir_shapes(m):
    for proj, (name, n, k) in enumerate(wl.BLOCK_SHAPES):
        log(f"mimir {name} m={m}")
        w = wl.normal_weights(wl.mimir_weight_seed(0, proj), n, k)
        wq, wd = oracle.quantize_f32(w)
        x = wl.normal_act_bf16(7000 + proj, m, k)
        assert_close(_run_skinny(wq, wd, x), oracle.w8a16(wq, wd, x), f"{name} m={m}")


# ------------------------------------------------------------------ block dots

@pytest.mark.parametrize("n,k,m", [(1, 32, 1), (77, 1536, 8), (1536, 4096, 3)])
def test_block_dots_bit_exact(n, k, m):
    w = mixed_weights(5000 + n, n, k)
    wq, _ = oracle.quantize_f32(w)
    xq, _ = oracle.quantize_bf16(wl.normal_act_bf16(5001, m, k))
    got = to_host(q8.block_dots(to_dev(wq), to_dev(xq)))
    assert np.array_equal(got, oracle.block_dots(wq, xq))


def test_block_dots_extremes():
    k = 64
    wq = np.full((2, k), 127, dtype=np.int8)
    wq[1] = -127
    xq = np.full((1, k), -127, dtype=np.int8)
    got = to_host(q8.block_dots(to_dev(wq), to_dev(xq)))
    assert np.all(got[0, 0] == -516128) and np.all(got[0, 1] == 516128)


# ------------------------------------------------------------------ prefill

def _prefill_case(n, k, p, seed):
    w = edge_weights(seed, n, k)
    wq, wd = oracle.quantize_f32(w)
    xq, xd = oracle.quantize_bf16(wl.prefill_act_bf16(seed + 1, p, k))
    return wq, wd, xq, xd


@pytest.mark.parametrize("n,k,p", [(1, 32, 1), (64, 64, 64), (100, 96, 11), (65, 2080, 100),
                                   (300, 4096, 256), (33, 1536, 257), (40, 7168, 37), (257, 160, 300),
                                   # K a multiple of 512: the persistent streaming kernel
                                   (1, 512, 1), (31, 1024, 33), (4097, 512, 3), (40, 16384, 40),
                                   (777, 2048, 95),
                                   # enough 64 x 64 tiles (MI355X: 256 compute units) for the
                                   # 64 x 64 kernel, ragged in n and p: one group of waves
                                   # (K % 512 != 0, or >= 4 tiles per compute unit) and K split
                                   # over two groups (1.5 .. 4 tiles per compute unit)
                                   (4100, 512, 300), (4097, 256, 257), (16383, 768, 70),
                                   (16390, 512, 300), (8200, 1024, 200)])
def test_prefill_small(n, k, p):
    log(f"prefill n={n} k={k} p={p}")
    wq, wd, xq, xd = _prefill_case(n, k, p, 6000 + n + k + p)
    y = q8.gemm_prefill(to_dev(wq), to_dev(wd), to_dev(xq), to_dev(xd))
    torch.cuda.synchronize()
    assert_close(to_host(y), oracle.q8q8(wq, wd, xq, xd), f"prefill n={n} k={k} p={p}")


def test_prefill_long_k_exact_or_refused():
    """K beyond the 64 KiB-LDS bound: either computed correctly (devices with a
    larger per-workgroup LDS) or refused with Q8_ERR_SHAPE -- never wrong."""
    n, k, p = 70, 8224, 40
    wq, wd, xq, xd = _prefill_case(n, k, p, 6100)
    try:
        y = q8.gemm_prefill(to_dev(wq), to_dev(wd), to_dev(xq), to_dev(xd))
    except q8.Q8Error as e:
        assert e.status == 2
        return
    torch.cuda.synchronize()
    assert_close(to_host(y), oracle.q8q8(wq, wd, xq, xd), "prefill long K")


def test_prefill_p256_config():
    cfg = wl.CONFIGS["prefill_p256"]
    xa = wl.prefill_act_bf16(cfg["xa_seed"], 256, wl.HIDDEN)
    xb = wl.prefill_act_bf16(cfg["xb_seed"], 256, wl.INTER)
    for proj, (name, n, k) in enumerate(wl.BLOCK_SHAPES):
        if name == "o":
            continue
        log(f"prefill p256 {name}")
        w = wl.normal_weights(wl.mimir_weight_seed(0, proj), n, k)
        x = xb if k == wl.INTER else xa
        dxq, dxd = q8.quantize_act(to_dev(x))
        dwq, dwd = q8.quantize_weights(to_dev(w))
        y = q8.gemm_prefill(dwq, dwd, dxq, dxd)
        torch.cuda.synchronize()
        wq, wd = oracle.quantize_f32(w)
        xq, xd = oracle.quantize_bf16(x)
        assert np.array_equal(to_host(dxq), xq) and np.array_equal(to_host(dxd), xd)
        assert_close(to_host(y), oracle.q8q8(wq, wd, xq, xd), f"prefill {name}")


# ------------------------------------------------------------------ exact constructions

def _pow2_q8(seed, n, k, m):
    """Codes in [-127, 127] with one |127| per block and scales 2^0 or 2^-1, so
    the stored scales are exactly 2^e and every block term is a multiple of 2^-2."""
    g = wl.rng(seed)
    nb = k // 32
    def make(rows, sign):
        v = g.integers(-127, 128, size=(rows, k)).astype(np.float32)
        v.reshape(rows, nb, 32)[:, :, 3] = sign * 127
        e = g.integers(-1, 1, size=(rows, nb))
        return (v.reshape(rows, nb, 32) * np.exp2(e)[:, :, None]).reshape(rows, k).astype(np.float32)
    return make(n, 1), make(m, -1)


def _assert_exact_regime(terms_abs_sum, quantum):
    """Every partial sum of terms that are multiples of `quantum` is exact in
    fp32 when the sum of their magnitudes stays below 2^24 quanta."""
    assert np.all(terms_abs_sum < 2.0 ** 24 * quantum), "construction left the exact regime"


def test_exact_pow2_scales_bitwise():
    n, k, m = 200, 512, 8
    w, x = _pow2_q8(8000, n, k, m)
    wq, wd = oracle.quantize_f32(w)
    xb = wl.f32_to_bf16_bits(x)
    xq, xd = oracle.quantize_bf16(xb)
    sw = wd.view(np.float16).astype(np.float64)
    sx = xd.view(np.float16).astype(np.float64)
    assert set(np.unique(sw)) <= {0.5, 1.0} and set(np.unique(sx)) <= {0.5, 1.0}
    isum = oracle.block_dots(wq, xq).astype(np.float64)          # [m][n][nb]
    _assert_exact_regime((np.abs(isum) * sw[None] * sx[:, None]).sum(axis=2), 0.25)
    ref = oracle.q8q8(wq, wd, xq, xd).astype(np.float32)
    assert np.array_equal(_run_skinny(wq, wd, xb, xq, xd), ref)
    yp = to_host(q8.gemm_prefill(to_dev(wq), to_dev(wd), to_dev(xq), to_dev(xd)))
    assert np.array_equal(yp, ref)
    # W8A16 with integer activations: every product and partial sum is an
    # integer times 2^-1
    xi_f = wl.rng(8001).integers(-100, 101, size=(m, k)).astype(np.float32)
    xi = wl.f32_to_bf16_bits(xi_f)
    absum = np.abs(xi_f.astype(np.float64)) @ (np.abs(wq.astype(np.float64)) * np.repeat(sw, 32, axis=1)).T
    _assert_exact_regime(absum, 0.5)
    assert np.array_equal(_run_skinny(wq, wd, xi), oracle.w8a16(wq, wd, xi).astype(np.float32))


def test_one_hot_gives_scaled_code():
    n, k = 70, 256
    wq, wd, _ = _w8a16_case(n, k, 1, 8100)
    s = wd.view(np.float16).astype(np.float32)
    x = np.zeros((8, k), dtype=np.uint16)
    cols = [0, 31, 32, 100, 200, 255, 17, 64]
    for i, c in enumerate(cols):
        x[i, c] = 0x3F80
    y = _run_skinny(wq, wd, x)
    for i, c in enumerate(cols):
        assert np.array_equal(y[i], wq[:, c].astype(np.float32) * s[:, c // 32])
    assert np.all(_run_skinny(wq, wd, np.zeros((3, k), dtype=np.uint16)) == 0)


# ------------------------------------------------------------------ determinism, batching, guards

def test_identical_rows_identical_outputs():
    n, k = 40000, 1536
    wq, wd, x1 = _w8a16_case(n, k, 1, 8200)
    y = _run_skinny(wq, wd, np.repeat(x1, 8, axis=0))
    assert all(np.array_equal(y[0], y[i]) for i in range(1, 8))
    xq, xd = oracle.quantize_bf16(np.repeat(x1, 8, axis=0))
    yq = _run_skinny(wq, wd, None, xq, xd)
    assert all(np.array_equal(yq[0], yq[i]) for i in range(1, 8))


def test_repeat_and_graph_replay_bitwise():
    n, k = 8192, 1536
    wq, wd, x = _w8a16_case(n, k, 4, 8300)
    dq, dd, dx = to_dev(wq), to_dev(wd), to_dev(x)
    xq, xd = oracle.quantize_bf16(x)
    dxq, dxd = to_dev(xq), to_dev(xd)
    ref = q8.gemm_skinny(dq, dd, dx).clone()
    refp = q8.gemm_prefill(dq, dd, dxq, dxd).clone()
    for _ in range(3):
        assert torch.equal(q8.gemm_skinny(dq, dd, dx), ref)
        assert torch.equal(q8.gemm_prefill(dq, dd, dxq, dxd), refp)
    out = torch.empty_like(ref)
    outp = torch.empty_like(refp)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        q8.gemm_skinny(dq, dd, dx, out=out)
        q8.gemm_prefill(dq, dd, dxq, dxd, out=outp)
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        q8.gemm_skinny(dq, dd, dx, out=out)
        q8.gemm_prefill(dq, dd, dxq, dxd, out=outp)
    for _ in range(4):
        out.fill_(float("nan"))
        outp.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref) and torch.equal(outp, refp)
        # eager work between replays
        q8.gemm_skinny(dq, dd, dx)
        torch.cuda.synchronize()


def test_outputs_leave_guard_bands_untouched():
    n, k, m, p = 100, 96, 3, 5
    w = edge_weights(8400, n, k)
    guard = 4096
    wq_buf = torch.full((n * k + guard,), 0x5A, dtype=torch.int8, device=DEV)
    wd_buf = torch.full((n * k // 32 + guard,), 0x1234, dtype=torch.int16, device=DEV)
    wq = wq_buf[: n * k].view(n, k)
    wd = wd_buf[: n * k // 32].view(torch.uint16).view(n, k // 32)
    q8.quantize_weights(to_dev(w), out=(wq, wd))
    y_buf = torch.full((m * n + guard,), 7.0, dtype=torch.float32, device=DEV)
    y = y_buf[: m * n].view(m, n)
    x = to_dev(wl.normal_act_bf16(8401, m, k))
    q8.gemm_skinny(wq, wd, x, out=y)
    xq, xd = q8.quantize_act(to_dev(wl.prefill_act_bf16(8402, p, k)))
    yp_buf = torch.full((p * n + guard,), 7.0, dtype=torch.float32, device=DEV)
    q8.gemm_prefill(wq, wd, xq, xd, out=yp_buf[: p * n].view(p, n))
    torch.cuda.synchronize()
    assert torch.all(wq_buf[n * k:] == 0x5A)
    assert torch.all(wd_buf[n * k // 32:] == 0x1234)
    assert torch.all(y_buf[m * n:] == 7.0)
    assert torch.all(yp_buf[p * n:] == 7.0)
    # the streaming prefill kernel (K a multiple of 512) and the 64 x 64 kernel
    # (K a multiple of 256, enough tiles), ragged in n and p
    for n2, k2, p2 in ((45, 512, 37), (8200, 256, 130), (6200, 512, 260)):
        _guarded_prefill(n2, k2, p2, guard)


def _guarded_prefill(n2, k2, p2, guard):
    log(f"guarded prefill n={n2} k={k2} p={p2}")
    wq2, wd2 = q8.quantize_weights(to_dev(edge_weights(8403, n2, k2)))
    xq2, xd2 = q8.quantize_act(to_dev(wl.prefill_act_bf16(8404, p2, k2)))
    y2_buf = torch.full((p2 * n2 + guard,), 7.0, dtype=torch.float32, device=DEV)
    q8.gemm_prefill(wq2, wd2, xq2, xd2, out=y2_buf[: p2 * n2].view(p2, n2))
    torch.cuda.synchronize()
    assert torch.all(y2_buf[p2 * n2:] == 7.0)
    assert_close(to_host(y2_buf[: p2 * n2].view(p2, n2)),
                 oracle.q8q8(to_host(wq2), to_host(wd2), to_host(xq2), to_host(xd2)), f"guarded prefill n={n2}")


def test_empty_calls_are_noops():
    z = torch.empty((0, 64), dtype=torch.float32, device=DEV)
    wq, wd = q8.quantize_weights(z)
    assert wq.shape == (0, 64) and wd.shape == (0, 2)
    y = q8.gemm_skinny(torch.empty((0, 64), dtype=torch.int8, device=DEV),
                       torch.empty((0, 2), dtype=torch.uint16, device=DEV),
                       torch.zeros((2, 64), dtype=torch.uint16, device=DEV))
    assert y.shape == (2, 0)


def test_rejects_bad_batch_loudly():
    wq = torch.zeros((4, 64), dtype=torch.int8, device=DEV)
    wd = torch.zeros((4, 2), dtype=torch.uint16, device=DEV)
    with pytest.raises(q8.Q8Error):
        q8.gemm_skinny(wq, wd, torch.zeros((9, 64), dtype=torch.uint16, device=DEV))
