"""Bit-exact checks of the int32 block sums on every kernel form of the hot path.

The Q8 x Q8 products compute y = sum_b wd * xd * isum with isum the exact int32
sum of a block's 32 code products [fak MODEL-BASELINE-RESULTS, ACT 3 item 3;
ACT 4 "Correctness": the tile kernel must equal the scalar reference bit for
bit, remainder paths included].  With every binary16 scale an exact power of
two (a block whose largest magnitude is 127 * 2^e has scale 2^e exactly), every
block term is a multiple of a fixed quantum and every fp32 operation of any
summation order is exact while the sum of the terms' magnitudes stays below
2^24 quanta -- then the GPU's fp32 output must equal the oracle's fp64 result
rounded to fp32, bit for bit, and a wrong block sum anywhere (a lost half
block, a wrong lane, a dropped remainder) shows as a different bit pattern.
W8A16 products get the same treatment with integer bf16 activations.

Every shape is chosen to reach one dispatch arm, and the test asserts which
kernel (and lane layout) the library launches for it, so each kernel form has a
bitwise check: the decode product's tall 16-lane, short 32-lane, long-K 32- and
64-lane layouts, with activations in registers (batch 1-2) or staged in LDS
(batch 3-8); the four prefill kernels; the int4 product's layouts; the
exported block sums."""
import numpy as np
import pytest
import torch

import int8_weight_streaming_amd as q8
import oracle
import workloads as wl
from gpu_helpers import log, oracle_threads, to_dev, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _setup():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    q8.load_library()
    oracle.set_threads(oracle_threads())
    yield
    torch.cuda.synchronize()


def cus() -> int:
    return torch.cuda.get_device_properties(0).multi_processor_count


# ------------------------------------------------------------------ constructions

def pow2_rows(g, rows, k, lim, pos, sign, cmax=127):
    """fp32 rows whose blocks of 32 hold integers in [-lim, lim] with element
    `pos` set to sign * cmax, each block scaled by 2^0 or 2^-1: the quantizer
    then stores scale 2^e exactly and codes equal to the integers."""
    nb = k // 32
    v = g.integers(-lim, lim + 1, size=(rows, nb, 32)).astype(np.float32)
    v[:, :, pos] = sign * cmax
    e = g.integers(-1, 1, size=(rows, nb))
    return (v * np.exp2(e)[:, :, None].astype(np.float32)).reshape(rows, k)


def q8_pair(seed, n, k, m, lim=40):
    """Q8_0 weights [n][k] and Q8_0 activations [m][k] with power-of-two scales;
    the two sides' full-scale elements sit at different positions."""
    g = wl.rng(seed)
    w = pow2_rows(g, n, k, lim, 3, 1)
    x = pow2_rows(g, m, k, lim, 7, -1)
    wq, wd = oracle.quantize_f32(w)
    xq, xd = oracle.quantize_bf16(wl.f32_to_bf16_bits(x))
    assert set(np.unique(wd.view(np.float16).astype(np.float64))) <= {0.5, 1.0}
    assert set(np.unique(xd.view(np.float16).astype(np.float64))) <= {0.5, 1.0}
    return wq, wd, xq, xd


def abs_term_bound(wq, wd, xq, xd):
    """[m][n] upper bound of sum_b |isum_b| * wd * xd: sum_k |x_k| |w_k| scaled."""
    sw = np.repeat(wd.view(np.float16).astype(np.float64), 32, axis=1)
    sx = np.repeat(xd.view(np.float16).astype(np.float64), 32, axis=1)
    return (np.abs(xq.astype(np.float64)) * sx) @ (np.abs(wq.astype(np.float64)) * sw).T


def assert_exact_regime(bound, quantum):
    assert np.all(bound < 2.0 ** 24 * quantum), "construction left the exact regime"


def bits(a):
    return np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)


def assert_bitwise(got, ref64, what):
    ref = ref64.astype(np.float32)
    same = bits(got) == bits(ref)
    if not same.all():
        idx = np.argwhere(~same)[0]
        raise AssertionError(f"{what}: {int((~same).sum())} outputs differ, first at {tuple(idx)}: "
                             f"{got[tuple(idx)]!r} vs {ref[tuple(idx)]!r}")


# ------------------------------------------------------------------ decode products (Q8_0 weights)

# (name, n as a function of the compute-unit count, k, batches, vector-ALU layout (G, R, CPL))
SKINNY_FORMS = [
    ("tall b1-2", lambda c: 32 * c + 5, 1536, (1, 2), (16, 2, 6)),
    ("tall b2-8", lambda c: 128 * c + 7, 1536, (2, 3, 4, 8), (16, 2, 6)),
    ("tall b1-2, K in several tiles", lambda c: 32 * c + 9, 4128, (1, 2), (16, 2, 6)),
    ("tall b3-8, K in several tiles", lambda c: 128 * c + 3, 4128, (3, 8), (16, 2, 6)),
    ("short", lambda c: 200, 1536, (1, 2, 3, 5, 8), (32, 1, 3)),
    ("short, ragged K tile", lambda c: 77, 992, (1, 2, 5, 8), (32, 1, 3)),
    ("long K b1-2", lambda c: 200, 4128, (1, 2), (32, 1, 8)),
    ("long K b3-8", lambda c: 130, 4128, (3, 8), (64, 1, 2)),
    ("long K, K a multiple of 512", lambda c: 130, 4096, (3, 6, 8), (64, 1, 2)),
    ("long K, K a multiple of 512 but not 1024", lambda c: 70, 2560, (5, 8), (64, 1, 2)),
    ("down shape", lambda c: 1536, 4096, (5, 8), (64, 1, 2)),
    ("middle, ragged rows", lambda c: 64 * c + 13, 1536, (4, 7), (16, 2, 6)),
    ("qkv shape", lambda c: 18 * c, 1536, (3, 8), (32, 1, 3)),
    ("K two twelve-way steps", lambda c: 300, 3072, (5, 8), (64, 1, 2)),
]
SKINNY_CASES = [(name, nf, k, m, lay) for name, nf, k, ms, lay in SKINNY_FORMS for m in ms]


def expected_skinny(n, k, m, act, lay, c):
    """The kernel the dispatch rule picks: the matrix-core form for bf16
    activations at batch 5..8 (any shape) or 2..4 (at least 64 rows per compute
    unit), K a multiple of 512 -- two 16-row fragments per wave from 128 rows
    per compute unit on, else a twelve-way K split for K a multiple of 1536, an
    eight-way one with 8-row half fragments for K a multiple of 1024 below 32
    rows per compute unit, a four-way one otherwise; else the vector-ALU
    layout.  Named <batch, rows per fragment, fragments, K split, non-temporal>."""
    a = q8.Q8_ACT_Q8 if act == "q8" else q8.Q8_ACT_BF16
    groups = (n + 31) // 32
    mfma = act == "bf16" and k % 512 == 0 and (m >= 5 or (m >= 2 and groups >= 2 * c))
    if mfma:
        if groups >= 4 * c:
            return f"skinny_mfma_kernel<{m},16,2,4,1>"
        if k % 1536 == 0:
            return f"skinny_mfma_kernel<{m},16,1,12,0>"
        if k % 1024 == 0 and groups < c:
            return f"skinny_mfma_kernel<{m},8,1,8,0>"
        return f"skinny_mfma_kernel<{m},16,1,4,0>"
    if act == "bf16" and m >= 3 and (n + 31) // 32 < 4 * c and lay == (16, 2, 6):
        lay = (32, 1, 3) if k // 32 <= 48 else (64, 1, 2)      # a middle matrix at batch 3-8
    return f"skinny_kernel<{m},{a},{lay[0]},{lay[1]},{lay[2]}>"


@pytest.mark.parametrize("name,nf,k,m,lay", SKINNY_CASES,
                         ids=[f"{c[0]}-m{c[3]}" for c in SKINNY_CASES])
@pytest.mark.parametrize("act", ["q8", "bf16"])
def test_skinny_block_sums_bitwise(name, nf, k, m, lay, act):
    c = cus()
    n = nf(c)
    a = q8.Q8_ACT_Q8 if act == "q8" else q8.Q8_ACT_BF16
    if act == "q8" and m >= 3 and (n + 31) // 32 < 4 * c and lay == (16, 2, 6):
        lay = (32, 1, 3) if k // 32 <= 48 else (64, 1, 2)
    want = expected_skinny(n, k, m, act, lay, c)
    got_name = q8.kernel_name(q8.OP_SKINNY, n, k, m, a)
    log(f"skinny {name} act={act} n={n} k={k} m={m}: {got_name}")
    assert got_name == want
    wq, wd, xq, xd = q8_pair(9100 + m + k % 97, n, k, m)
    if act == "q8":
        assert_exact_regime(abs_term_bound(wq, wd, xq, xd), 0.25)
        y = q8.gemm_skinny(to_dev(wq), to_dev(wd), to_dev(xq), to_dev(xd))
        torch.cuda.synchronize()
        assert_bitwise(to_host(y), oracle.q8q8(wq, wd, xq, xd), f"{want} q8")
    else:
        # integer bf16 activations: every product and partial sum is a multiple of 2^-1
        xi = wl.rng(9200 + m).integers(-8, 9, size=(m, k)).astype(np.float32)
        xb = wl.f32_to_bf16_bits(xi)
        sw = np.repeat(wd.view(np.float16).astype(np.float64), 32, axis=1)
        assert_exact_regime(np.abs(xi.astype(np.float64)) @ (np.abs(wq.astype(np.float64)) * sw).T, 0.5)
        y = q8.gemm_skinny(to_dev(wq), to_dev(wd), to_dev(xb))
        torch.cuda.synchronize()
        assert_bitwise(to_host(y), oracle.w8a16(wq, wd, xb), f"{want} bf16")


def test_gemv_entry_is_the_batch1_product():
    n, k = 32 * cus() + 5, 1536
    wq, wd, xq, xd = q8_pair(9300, n, k, 1)
    y = q8.gemv(to_dev(wq), to_dev(wd), to_dev(xq[0]), to_dev(xd[0]))
    torch.cuda.synchronize()
    assert_bitwise(to_host(y)[None], oracle.q8q8(wq, wd, xq, xd), "gemv q8")


@pytest.mark.parametrize("n,k,m", [(1, 32, 1), (77, 1536, 8), (33, 4128, 3), (1536, 4096, 2)])
def test_block_dots_export_bitwise(n, k, m):
    """The exported block sums (full code range, no construction needed)."""
    g = wl.rng(9400 + n)
    wq = g.integers(-127, 128, size=(n, k)).astype(np.int8)
    xq = g.integers(-127, 128, size=(m, k)).astype(np.int8)
    wq[:, ::7] = 127
    xq[:, ::7] = 127 if m % 2 else -127
    isum = q8.block_dots(to_dev(wq), to_dev(xq))
    torch.cuda.synchronize()
    assert np.array_equal(to_host(isum), oracle.block_dots(wq, xq))


# ------------------------------------------------------------------ prefill kernels

PREFILL_FORMS = [
    # (name, n, k, p, kernel)
    ("64x64 tiles, K % 512 != 0", 1000, 768, 1000, "prefill_tile64_kernel<1>"),
    ("64x64 tiles, 4 per CU", "4cu", 512, 1000, "prefill_tile64_kernel<1>"),
    ("64x64 tiles, K split in two", 3000, 1024, 600, "prefill_tile64_kernel<2>"),
    ("gate_up shape, P = 256", 8192, 1536, 256, "prefill_tile64_kernel<2>"),
    ("qkv shape, P = 256", 4608, 1536, 256, "prefill_stream_kernel"),
    ("down shape, P = 256", 1536, 4096, 256, "prefill_stream_kernel"),
    ("streaming, ragged", 200, 1536, 40, "prefill_stream_kernel"),
    ("streaming, one row", 33, 512, 1, "prefill_stream_kernel"),
    ("one-tile kernel", 100, 800, 50, "prefill_kernel"),
    ("one-tile kernel, one block", 37, 32, 19, "prefill_kernel"),
]


@pytest.mark.parametrize("name,n,k,p,kernel", PREFILL_FORMS, ids=[f[0] for f in PREFILL_FORMS])
def test_prefill_block_sums_bitwise(name, n, k, p, kernel):
    c = cus()
    if n == "4cu":
        n = 64 * ((4 * c + 15) // 16) + 37               # >= 4 tiles of 64 x 64 per CU at p = 1000
    got_name = q8.kernel_name(q8.OP_PREFILL, n, k, p)
    log(f"prefill {name} n={n} k={k} p={p}: {got_name}")
    assert got_name == kernel
    wq, wd, xq, xd = q8_pair(9500 + k % 89 + p, n, k, p)
    assert_exact_regime(abs_term_bound(wq, wd, xq, xd), 0.25)
    y = q8.gemm_prefill(to_dev(wq), to_dev(wd), to_dev(xq), to_dev(xd))
    torch.cuda.synchronize()
    assert_bitwise(to_host(y), oracle.q8q8(wq, wd, xq, xd), kernel)


# ------------------------------------------------------------------ int4 products

def q4_weights(seed, n, k):
    """int4 weights with power-of-two scales: integers in [-7, 7], one +7 per
    block, blocks scaled by 2^0 or 2^-1 (the int4 scale is maxabs / 7)."""
    g = wl.rng(seed)
    w = pow2_rows(g, n, k, 7, 3, 1, cmax=7)
    wq4, wd = oracle.q4_quantize_f32(w)
    assert set(np.unique(wd.view(np.float16).astype(np.float64))) <= {0.5, 1.0}
    return wq4, wd


# (name, n as a function of the compute-unit count, k, batches, layout (G, R, CPL, XL) by (m, act))
def q4_layout(m, act, n_kind):
    if n_kind == "very tall":
        if m == 1:
            return (16, 2, 1, 0) if act == 0 else (16, 2, 3, 0)
        return (16, 4, 3, 1)
    if n_kind == "tall":
        return (16, 2, 3, int(m > 2))
    if n_kind == "short":
        return (32, 1, 2, int(m > 2))
    return (32, 1, 4, 0) if m <= 2 else (64, 1, 2, 1)


Q4_FORMS = [("very tall", lambda c: 256 * c + 70, 1536), ("tall", lambda c: 16 * c + 11, 1536),
            ("short", lambda c: 200, 1536), ("long K", lambda c: 150, 4128),
            ("down shape", lambda c: 1536, 4096), ("K a multiple of 512 only", lambda c: 300, 2560)]
Q4_CASES = [(kind, nf, k, m) for kind, nf, k in Q4_FORMS for m in (1, 2, 3, 8)]


def expected_q4(n, k, m, a, kind, c):
    """The int4 kernel the dispatch rule picks: the matrix-core form for bf16
    activations at batch 2..8 with K a multiple of 512 -- two 16-row fragments
    per wave from 128 rows per compute unit on, else a twelve-way K split for K
    a multiple of 1536, an eight-way one for K a multiple of 1024 below 32 rows
    per compute unit (from batch 5 only), a four-way one otherwise (the tall
    form from batch 3); else the vector-ALU layout of the shape's kind."""
    if a == q8.Q8_ACT_BF16 and 2 <= m <= 8 and k % 512 == 0:
        groups = (n + 31) // 32
        if groups >= 4 * c:
            lay = (16, 2, 4, 0)                     # (int4: cached weight loads on the tall layout)
        elif k % 1536 == 0:
            lay = (16, 1, 12, 0)
        elif k % 1024 == 0 and groups < c:
            lay = (16, 1, 8, 0)
        else:
            lay = (16, 1, 4, 0)
        if not (lay[2] == 8 and m <= 4) and not (lay[1] == 2 and m == 2):
            return f"q4_skinny_mfma_kernel<{m},{lay[0]},{lay[1]},{lay[2]},{lay[3]}>"
    lay = q4_layout(m, a, kind)
    return f"q4_skinny_kernel<{m},{a},{lay[0]},{lay[1]},{lay[2]},{lay[3]}>"


@pytest.mark.parametrize("kind,nf,k,m", Q4_CASES, ids=[f"{c[0]}-m{c[3]}" for c in Q4_CASES])
@pytest.mark.parametrize("act", ["q8", "bf16"])
def test_q4_block_sums_bitwise(kind, nf, k, m, act):
    c = cus()
    n = nf(c)
    a = q8.Q8_ACT_Q8 if act == "q8" else q8.Q8_ACT_BF16
    want = expected_q4(n, k, m, a, kind, c)
    got_name = q8.kernel_name(q8.OP_Q4_SKINNY, n, k, m, a)
    log(f"int4 {kind} act={act} n={n} k={k} m={m}: {got_name}")
    assert got_name == want
    wq4, wd = q4_weights(9600 + m + n % 13, n, k)
    codes = oracle.q4_unpack(wq4)
    if act == "q8":
        _, _, xq, xd = q8_pair(9700 + m, 1, k, m)
        assert_exact_regime(abs_term_bound(codes, wd, xq, xd), 0.25)
        y = q8.q4_gemm_skinny(to_dev(wq4), to_dev(wd), to_dev(xq), to_dev(xd))
        torch.cuda.synchronize()
        assert_bitwise(to_host(y), oracle.q4q8(wq4, wd, xq, xd), want)
    else:
        xi = wl.rng(9800 + m).integers(-100, 101, size=(m, k)).astype(np.float32)
        xb = wl.f32_to_bf16_bits(xi)
        sw = np.repeat(wd.view(np.float16).astype(np.float64), 32, axis=1)
        assert_exact_regime(np.abs(xi.astype(np.float64)) @ (np.abs(codes.astype(np.float64)) * sw).T, 0.5)
        y = q8.q4_gemm_skinny(to_dev(wq4), to_dev(wd), to_dev(xb))
        torch.cuda.synchronize()
        assert_bitwise(to_host(y), oracle.w4a16(wq4, wd, xb), want)
