"""GPU parity of the decode-step glue fused into the W8A16 products, through the
C ABI, against the oracle.

Each check runs the oracle on the same bf16 activations the product consumed:
for the RMSNorm prologue those are the GPU's normalized rows rounded to bf16
(q8_rmsnorm uses the prologue's own reduction, so they are bit-identical to
what the product read); the normalization itself is checked against the fp64
oracle separately.  fp32 outputs: max-abs 2e-3 and relative L2 1e-5.  bf16
outputs (SwiGLU, RoPE) are an fp32 result rounded once: each must lie within
one bf16 step plus the fp32 error bound of the product (the classical
summation bound, carried through the rotation or the SwiGLU) of the fp64
value, and must equal its bf16 rounding in at least 99% of places."""
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


def _bf16_to_f64(bits):
    return wl.bf16_bits_to_f32(np.asarray(bits, dtype=np.uint16)).astype(np.float64)


def assert_bf16_rounding_of(got_bits, want64, tol, what):
    """got is the bf16 rounding (nearest, ties to even) of an fp32 value within
    `tol` of the fp64 value want: so |got - want| <= one bf16 step + tol, and
    got equals the bf16 rounding of want except near midpoints (rare)."""
    got = _bf16_to_f64(got_bits)
    want_bits = wl.f32_to_bf16_bits(want64.astype(np.float32))
    differ = np.asarray(got_bits, dtype=np.uint16) != want_bits
    step = np.exp2(np.floor(np.log2(np.maximum(np.abs(want64), 1e-300))) - 7)   # bf16 spacing at |want|
    far = differ & (np.abs(got - want64) > step + tol)
    assert not np.any(far), f"{what}: {int(far.sum())} values off by more than a bf16 step + bound"
    assert np.mean(differ) < 1e-2, f"{what}: {np.mean(differ):.2e} of values differ"


def summation_bound(wq, wd, xb):
    """(K + 2) 2^-24 sum_k |q s x| per output [m][n]: the fp32 error bound of a
    product summed in any order."""
    k = wq.shape[1]
    s_ = np.repeat(wd.view(np.float16).astype(np.float64), 32, axis=1)
    absum = np.abs(_bf16_to_f64(xb)) @ (np.abs(wq.astype(np.float64)) * s_).T
    return (k + 2) * 2.0 ** -24 * absum


def _weights(seed, n, k, perm=None):
    w = wl.normal_weights(seed, n, k)
    wq, wd = oracle.quantize_f32(w)
    if perm is None:
        return wq, wd, wq, wd
    return wq, wd, np.ascontiguousarray(wq[perm]), np.ascontiguousarray(wd[perm])


def _resid(seed, m, k):
    return (wl.rng(seed).standard_normal((m, k)) * 3.0).astype(np.float32)


def _gpu_norm_bf16(h_dev):
    return wl.f32_to_bf16_bits(to_host(q8.rmsnorm(h_dev)))


@pytest.mark.parametrize("m,k", [(1, 1536), (3, 1536), (8, 4096), (2, 96)])
def test_rmsnorm_against_oracle(m, k):
    h = _resid(100 + m, m, k)
    h[0, :7] = 0.0
    dh = to_dev(h)
    y = to_host(q8.rmsnorm(dh))
    y64 = oracle.rmsnorm(h)
    assert np.max(np.abs(y - y64) / (np.abs(y64) + 1e-30)) < 2e-6
    # in place gives the same bits
    d2 = dh.clone()
    q8.rmsnorm(d2, out=d2)
    assert torch.equal(d2, torch.from_numpy(y).to(DEV))
    # the bf16 rounding of the normalized rows matches the fp64 definition
    assert_bf16_rounding_of(wl.f32_to_bf16_bits(y), y64, 2e-6 * np.abs(y64), f"rmsnorm m={m} k={k}")


@pytest.mark.parametrize("n,k,m", [(1536, 1536, 1), (262144 // 16, 1536, 2), (300, 4096, 5), (64, 96, 8)])
def test_norm_f32_and_f32_f32(n, k, m):
    log(f"fused norm/f32 n={n} k={k} m={m}")
    wq, wd, _, _ = _weights(200 + n, n, k)
    h = _resid(201 + m, m, k)
    dq, dd, dh = to_dev(wq), to_dev(wd), to_dev(h)
    y = to_host(q8.gemm_fused(dq, dd, dh, q8.PRO_RMSNORM, q8.EPI_F32))
    xb = _gpu_norm_bf16(dh)
    assert_close(y, oracle.w8a16(wq, wd, xb), f"norm+f32 n={n} m={m}")
    y2 = to_host(q8.gemm_fused(dq, dd, dh, q8.PRO_F32, q8.EPI_F32))
    assert_close(y2, oracle.w8a16(wq, wd, wl.f32_to_bf16_bits(h)), f"f32+f32 n={n} m={m}")


@pytest.mark.parametrize("n,k,m", [(1536, 1536, 1), (1536, 4096, 1), (1000, 64, 4), (8192, 1536, 8)])
def test_residual_add(n, k, m):
    log(f"fused add n={n} k={k} m={m}")
    wq, wd, _, _ = _weights(300 + n + k, n, k)
    h0 = _resid(301 + m, m, n)
    xf = _resid(302 + m, m, k)
    xb = wl.normal_act_bf16(303 + m, m, k)
    dq, dd = to_dev(wq), to_dev(wd)
    dh = to_dev(h0)
    q8.gemm_fused(dq, dd, to_dev(xf), q8.PRO_F32, q8.EPI_ADD, out=dh)
    want = h0.astype(np.float64) + oracle.w8a16(wq, wd, wl.f32_to_bf16_bits(xf))
    assert_close(to_host(dh), want, f"f32+add n={n} m={m}")
    dh = to_dev(h0)
    q8.gemm_fused(dq, dd, to_dev(xb), q8.PRO_BF16, q8.EPI_ADD, out=dh)
    assert_close(to_host(dh), h0.astype(np.float64) + oracle.w8a16(wq, wd, xb), f"bf16+add n={n} m={m}")


@pytest.mark.parametrize("n,k,m", [(8192, 1536, 1), (8192, 1536, 3), (512, 4096, 2), (256, 64, 8), (64, 1536, 1)])
def test_swiglu_epilogue(n, k, m):
    log(f"fused swiglu n={n} k={k} m={m}")
    perm = wl.swiglu_pair_rows(n)
    wq, wd, sq, sd = _weights(400 + n + k, n, k, perm)
    h = _resid(401 + m, m, k)
    dh = to_dev(h)
    s = to_host(q8.gemm_fused(to_dev(sq), to_dev(sd), dh, q8.PRO_RMSNORM, q8.EPI_SWIGLU))
    assert s.shape == (m, n // 2)
    xb = _gpu_norm_bf16(dh)
    y = oracle.w8a16(wq, wd, xb)
    b = summation_bound(wq, wd, xb)
    g, u = y[:, : n // 2], y[:, n // 2:]
    want = oracle.swiglu(g, u)
    # d/dg silu(g) u <= 1.1 |u|, d/du = silu(g) <= |g| + 0.3
    tol = 1.1 * np.abs(u) * b[:, : n // 2] + (np.abs(g) + 0.3) * b[:, n // 2:]
    assert_bf16_rounding_of(s, want, tol, f"swiglu n={n} m={m}")


@pytest.mark.parametrize("n,rope_rows,k,m,pos", [(4608, 3072, 1536, 1, 0), (4608, 3072, 1536, 1, 511),
                                                 (4608, 3072, 1536, 4, 4095), (512, 256, 4096, 2, 77),
                                                 (256, 256, 96, 8, 1), (384, 128, 64, 1, 3000)])
def test_rope_epilogue(n, rope_rows, k, m, pos):
    log(f"fused rope n={n} rope_rows={rope_rows} k={k} m={m} pos={pos}")
    perm = wl.rope_pair_rows(rope_rows, n)
    wq, wd, sq, sd = _weights(500 + n + k, n, k, perm)
    h = _resid(501 + m, m, k)
    dh = to_dev(h)
    out = to_host(q8.gemm_fused(to_dev(sq), to_dev(sd), dh, q8.PRO_RMSNORM, q8.EPI_ROPE,
                                rope_rows=rope_rows, pos=pos))
    xb = _gpu_norm_bf16(dh)
    y = oracle.w8a16(wq, wd, xb)
    b = summation_bound(wq, wd, xb)
    want = y.copy()
    tol = b.copy()
    for t in range(m):
        want[t, :rope_rows] = oracle.rope(y[t, :rope_rows], rope_rows // 128, 128, pos)
        # a rotated value mixes the two members of its pair (|cos|, |sin| <= 1),
        # plus fp32 rounding of the rotation itself
        bh = b[t, :rope_rows].reshape(-1, 2, 64)
        pair = np.concatenate([bh[:, 0] + bh[:, 1]] * 2, axis=1).reshape(-1)
        tol[t, :rope_rows] = pair + 2.0 ** -22 * np.abs(want[t, :rope_rows])
    assert_bf16_rounding_of(out, want, tol, f"rope n={n} m={m} pos={pos}")


@pytest.mark.parametrize("m,k", [(1, 1536), (256, 1536), (64, 4096), (7, 96), (3, 2048), (5, 2080), (0, 1536)])
def test_quantize_act_fused(m, k):
    """The prologue fused with the activation quantizer: codes and scales
    bit-exact against the oracle's quantizer applied to the bf16 rows the
    prologue defines (F32: the seeded prefill activations with their special
    rows; RMSNORM: q8_rmsnorm's rows rounded to bf16), and against the
    two-launch chain on the GPU."""
    log(f"quantize_act_fused m={m} k={k}")
    xb = wl.prefill_act_bf16(800 + m + k, m, k)
    x = wl.bf16_bits_to_f32(xb)
    if m > 1:
        x[m - 1] = 0.0                                   # a zero row: zero blocks, scale 0
    dx = to_dev(x)
    xq, xd = q8.quantize_act_fused(dx, q8.PRO_F32)
    oq, od = oracle.quantize_bf16(wl.f32_to_bf16_bits(x))
    assert np.array_equal(to_host(xq), oq) and np.array_equal(to_host(xd), od), "F32 prologue"
    h = _resid(801 + m, m, k)
    if m > 1:
        h[0] = 0.0
    dh = to_dev(h)
    xq, xd = q8.quantize_act_fused(dh, q8.PRO_RMSNORM)
    xb = _gpu_norm_bf16(dh)
    oq, od = oracle.quantize_bf16(xb)
    assert np.array_equal(to_host(xq), oq) and np.array_equal(to_host(xd), od), "RMSNORM prologue"
    cq, cd = q8.quantize_act_fused(q8.rmsnorm(dh), q8.PRO_F32)
    assert torch.equal(cq, xq) and torch.equal(cd, xd), "two-launch chain"


def test_fused_repeat_and_graph_replay_bitwise():
    n, k = 4608, 1536
    perm = wl.rope_pair_rows(3072, n)
    _, _, sq, sd = _weights(600, n, k, perm)
    dq, dd = to_dev(sq), to_dev(sd)
    dh = to_dev(_resid(601, 1, k))
    ref = q8.gemm_fused(dq, dd, dh, q8.PRO_RMSNORM, q8.EPI_ROPE, rope_rows=3072, pos=123).clone()
    out = torch.empty_like(ref)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        q8.gemm_fused(dq, dd, dh, q8.PRO_RMSNORM, q8.EPI_ROPE, out=out, rope_rows=3072, pos=123)
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        q8.gemm_fused(dq, dd, dh, q8.PRO_RMSNORM, q8.EPI_ROPE, out=out, rope_rows=3072, pos=123)
    for _ in range(3):
        out.fill_(0)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref)
        q8.rmsnorm(dh)
        torch.cuda.synchronize()
