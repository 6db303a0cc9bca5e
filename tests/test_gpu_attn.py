"""GPU parity of the decode attention over a Q8_0 key/value cache, through the
C ABI, against the fp64 oracle (max-abs 2e-3, relative L2 1e-5 per call).

Shapes cover one and several chunks with ragged ends (64-row chunks up to
512 rows, 128-row chunks up to 2048, 256-row chunks above, each side of both
boundaries, and more than 32 chunks, the combine's batched path), the pages' static slab (capacity 4096, 12 heads of 128) at short and
full context, and rows past t filled with NaN scales, so that any read past t
would show."""
import math

import numpy as np
import pytest
import torch

import int8_weight_streaming_amd as q8
import oracle
import workloads as wl
from gpu_helpers import DEV, assert_close, log, oracle_threads, to_dev, to_host

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


def cache(seed, heads, t, t_cap, qmul=1.0, poison=True):
    """Q8_0 K and V slabs [heads][t_cap][128] quantized from N(0,1) bf16 rows
    (rows past t get huge codes and NaN scales when `poison`), and a bf16 query."""
    g = wl.rng(seed)
    rows = heads * t_cap
    kq, kd = oracle.quantize_bf16(wl.f32_to_bf16_bits(g.standard_normal((rows, D)).astype(np.float32)))
    vq, vd = oracle.quantize_bf16(wl.f32_to_bf16_bits(g.standard_normal((rows, D)).astype(np.float32)))
    kq, vq = kq.reshape(heads, t_cap, D), vq.reshape(heads, t_cap, D)
    kd, vd = kd.reshape(heads, t_cap, D // 32), vd.reshape(heads, t_cap, D // 32)
    if poison and t < t_cap:
        kq[:, t:] = 127
        vq[:, t:] = -127
        kd[:, t:] = 0x7E00
        vd[:, t:] = 0x7E00
    q = wl.f32_to_bf16_bits((g.standard_normal((heads, D)) * qmul).astype(np.float32))
    return q, kq, kd, vq, vd


def run(q, kq, kd, vq, vd, t, scale=SCALE):
    y = q8.attn_decode(to_dev(q), to_dev(kq), to_dev(kd), to_dev(vq), to_dev(vd), t, scale)
    torch.cuda.synchronize()
    return to_host(y)


@pytest.mark.parametrize("heads,t,t_cap", [(1, 1, 1), (2, 5, 8), (12, 64, 64), (12, 65, 128), (12, 127, 128),
                                           (12, 128, 128), (12, 511, 512), (12, 513, 1024),
                                           (12, 129, 200), (3, 1000, 1024), (5, 333, 4096),
                                           (12, 512, 4096), (12, 2048, 4096), (12, 4096, 4096),
                                           (4, 2049, 4096), (3, 3001, 4096), (2, 2300, 2400),
                                           (2, 9000, 9000)])
def test_attn_matches_oracle(heads, t, t_cap):
    log(f"attn heads={heads} t={t} t_cap={t_cap}")
    q, kq, kd, vq, vd = cache(9000 + heads + t, heads, t, t_cap)
    y = run(q, kq, kd, vq, vd, t)
    assert_close(y, oracle.attn_decode(q, kq, kd, vq, vd, t, SCALE), f"attn h={heads} t={t}")


@pytest.mark.parametrize("qmul,scale", [(8.0, SCALE), (1.0, 0.0), (1.0, 2.0), (0.0, SCALE)])
def test_attn_peaked_and_flat_softmax(qmul, scale):
    """Peaked weights (large scores), exactly uniform weights (zero scale or a
    zero query: the mean of V), and scores spanning hundreds."""
    heads, t = 4, 700
    q, kq, kd, vq, vd = cache(9100, heads, t, 768, qmul=qmul)
    y = run(q, kq, kd, vq, vd, t, scale)
    assert_close(y, oracle.attn_decode(q, kq, kd, vq, vd, t, scale), f"attn qmul={qmul} scale={scale}")


def test_attn_cache_quantized_on_gpu():
    """The cache written by q8_quantize_act (K and V rows of 128 as [rows][128]
    activations) is the format the attention reads."""
    heads, t = 12, 300
    g = wl.rng(9200)
    kx = wl.f32_to_bf16_bits(g.standard_normal((heads * t, D)).astype(np.float32))
    vx = wl.f32_to_bf16_bits(g.standard_normal((heads * t, D)).astype(np.float32))
    dkq, dkd = q8.quantize_act(to_dev(kx))
    dvq, dvd = q8.quantize_act(to_dev(vx))
    q = wl.f32_to_bf16_bits(g.standard_normal((heads, D)).astype(np.float32))
    y = q8.attn_decode(to_dev(q), dkq.view(heads, t, D), dkd.view(heads, t, D // 32),
                       dvq.view(heads, t, D), dvd.view(heads, t, D // 32), t, SCALE)
    torch.cuda.synchronize()
    kq, kd = oracle.quantize_bf16(kx)
    vq, vd = oracle.quantize_bf16(vx)
    assert np.array_equal(to_host(dkq), kq) and np.array_equal(to_host(dvd), vd)
    ref = oracle.attn_decode(q, kq.reshape(heads, t, D), kd.reshape(heads, t, D // 32),
                             vq.reshape(heads, t, D), vd.reshape(heads, t, D // 32), t, SCALE)
    assert_close(to_host(y), ref, "attn gpu-quantized cache")


def test_attn_repeat_graph_replay_and_guard_band():
    heads, t, t_cap = 12, 1500, 2048
    q, kq, kd, vq, vd = cache(9300, heads, t, t_cap)
    dq, dkq, dkd, dvq, dvd = (to_dev(a) for a in (q, kq, kd, vq, vd))
    ref = q8.attn_decode(dq, dkq, dkd, dvq, dvd, t, SCALE).clone()
    guard = 1024
    out_buf = torch.full((heads * D + guard,), 7.0, dtype=torch.float32, device=DEV)
    out = out_buf[: heads * D].view(heads, D)
    work = torch.empty((q8.attn_work_words(heads, t),), dtype=torch.float32, device=DEV)
    for _ in range(3):
        q8.attn_decode(dq, dkq, dkd, dvq, dvd, t, SCALE, work=work, out=out)
        torch.cuda.synchronize()
        assert torch.equal(out, ref)
    assert torch.all(out_buf[heads * D:] == 7.0)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        q8.attn_decode(dq, dkq, dkd, dvq, dvd, t, SCALE, work=work, out=out)
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        q8.attn_decode(dq, dkq, dkd, dvq, dvd, t, SCALE, work=work, out=out)
    for _ in range(4):
        out.fill_(float("nan"))
        work.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref)
        q8.attn_decode(dq, dkq, dkd, dvq, dvd, 100, SCALE)        # eager work between replays
        torch.cuda.synchronize()
    assert_close(to_host(ref), oracle.attn_decode(q, kq, kd, vq, vd, t, SCALE), "attn replay")


def test_attn_one_workspace_across_context_lengths():
    """One workspace serves back-to-back calls on one stream with different t
    (different chunk counts, so the partials land at different places), in any
    order, with no synchronization between them."""
    heads, t_cap = 12, 4096
    q, kq, kd, vq, vd = cache(9350, heads, t_cap, t_cap)
    dq, dkq, dkd, dvq, dvd = (to_dev(a) for a in (q, kq, kd, vq, vd))
    work = torch.full((q8.attn_work_words(heads, t_cap),), float("nan"), dtype=torch.float32, device=DEV)
    ts = [4096, 129, 1000, 4000, 256, 257, 3001, 128, 2048]
    outs = [q8.attn_decode(dq, dkq, dkd, dvq, dvd, t, SCALE, work=work) for t in ts]   # no syncs between
    torch.cuda.synchronize()
    for t, y in zip(ts, outs):
        log(f"attn shared workspace t={t}")
        assert_close(to_host(y), oracle.attn_decode(q, kq, kd, vq, vd, t, SCALE), f"shared workspace t={t}")
        assert torch.equal(y, q8.attn_decode(dq, dkq, dkd, dvq, dvd, t, SCALE))


@pytest.mark.parametrize("t,t_cap", [(1, 16), (64, 64), (65, 100), (128, 256), (129, 256), (200, 200),
                                     (513, 600), (4096, 4096), (1500, 2048),
                                     (2049, 2100), (2200, 4096), (3000, 3000), (9000, 9000)])
def test_attn_append_writes_row_and_attends(t, t_cap):
    """The new key/value rows land in cache row t - 1 exactly as the activation
    quantizer writes them, nothing else in the cache changes, and the output is
    the attention over the updated cache."""
    heads = 12
    log(f"attn append t={t} t_cap={t_cap}")
    q, kq, kd, vq, vd = cache(9700 + t, heads, t_cap, t_cap)
    g = wl.rng(9701 + t)
    knew = wl.f32_to_bf16_bits(g.standard_normal((heads, D)).astype(np.float32) * 2)
    vnew = wl.f32_to_bf16_bits(g.standard_normal((heads, D)).astype(np.float32))
    knew[0, :32] = 0                                   # a zero block
    dq, dkq, dkd, dvq, dvd = (to_dev(a) for a in (q, kq, kd, vq, vd))
    y = q8.attn_decode_append(dq, dkq, dkd, dvq, dvd, t, SCALE, to_dev(knew), to_dev(vnew))
    torch.cuda.synchronize()
    ck, cks = oracle.quantize_bf16(knew)
    cv, cvs = oracle.quantize_bf16(vnew)
    kq2, kd2, vq2, vd2 = kq.copy(), kd.copy(), vq.copy(), vd.copy()
    kq2[:, t - 1], kd2[:, t - 1], vq2[:, t - 1], vd2[:, t - 1] = ck, cks, cv, cvs
    assert np.array_equal(to_host(dkq), kq2) and np.array_equal(to_host(dkd), kd2)
    assert np.array_equal(to_host(dvq), vq2) and np.array_equal(to_host(dvd), vd2)
    assert_close(to_host(y), oracle.attn_decode(q, kq2, kd2, vq2, vd2, t, SCALE), f"append t={t}")


def test_attn_rejects_bad_arguments():
    q, kq, kd, vq, vd = cache(9400, 2, 10, 16)
    dq, dkq, dkd, dvq, dvd = (to_dev(a) for a in (q, kq, kd, vq, vd))
    with pytest.raises(q8.Q8Error) as e:
        q8.attn_decode(dq, dkq, dkd, dvq, dvd, 17, SCALE)          # t > t_cap
    assert e.value.status == 2
    with pytest.raises(q8.Q8Error):
        q8.attn_decode(dq, dkq, dkd, dvq, dvd, 0, SCALE)


@pytest.mark.parametrize("t", [1, 64, 65, 100, 128, 129, 511, 512, 513, 1000, 1024, 1025, 2048, 2049, 3001,
                               4096])
def test_partials_and_folded_combine_match_two_launches(t):
    """attn_decode_append_partials + gemm_attn_residual (the combine done in the
    o product's prologue) give bit for bit the residual of attn_decode_append
    followed by the fp32-prologue product with the residual add, and the same
    cache rows."""
    heads, t_cap, n = 12, 4096, 1536
    log(f"attn partials + folded combine t={t}")
    q, kq, kd, vq, vd = cache(9900 + t, heads, t_cap, t_cap)
    g = wl.rng(9901 + t)
    knew = to_dev(wl.f32_to_bf16_bits(g.standard_normal((heads, D)).astype(np.float32)))
    vnew = to_dev(wl.f32_to_bf16_bits(g.standard_normal((heads, D)).astype(np.float32)))
    wq, wd = q8.quantize_weights(to_dev(wl.normal_weights(9902, n, heads * D)))
    h0 = to_dev(g.standard_normal((1, n)).astype(np.float32))
    c1 = [to_dev(a) for a in (q, kq, kd, vq, vd)]
    c2 = [to_dev(a) for a in (q, kq, kd, vq, vd)]
    h1, h2 = h0.clone(), h0.clone()
    a = q8.attn_decode_append(*c1, t, SCALE, knew, vnew)
    q8.gemm_fused(wq, wd, a.view(1, -1), q8.PRO_F32, q8.EPI_ADD, out=h1)
    work = torch.full((q8.attn_partial_words(heads, t),), float("nan"), dtype=torch.float32, device=DEV)
    q8.attn_decode_append_partials(*c2, t, SCALE, knew, vnew, work=work)
    q8.gemm_attn_residual(wq, wd, work, t, h2)
    torch.cuda.synchronize()
    assert torch.equal(h1, h2)
    for x1, x2 in zip(c1, c2):
        assert torch.equal(x1, x2)


@pytest.mark.parametrize("heads,n,t", [(2, 300, 5), (2, 300, 700), (16, 4096, 900), (16, 4096, 3000)])
def test_folded_combine_other_widths(heads, n, t):
    """The folded combine for other head counts: 2 heads (k = 256) with a
    ragged number of output rows, and 16 heads (k = 2048, the widest row, a
    256-chunk K tile), against the two-launch form, bit for bit."""
    t_cap, k = 4096, heads * D
    log(f"folded combine heads={heads} n={n} t={t}")
    q, kq, kd, vq, vd = cache(9950 + heads + t, heads, t_cap, t_cap)
    g = wl.rng(9951 + t)
    knew = to_dev(wl.f32_to_bf16_bits(g.standard_normal((heads, D)).astype(np.float32)))
    vnew = to_dev(wl.f32_to_bf16_bits(g.standard_normal((heads, D)).astype(np.float32)))
    wq, wd = q8.quantize_weights(to_dev(wl.normal_weights(9952 + heads, n, k)))
    h0 = to_dev(g.standard_normal((1, n)).astype(np.float32))
    c1 = [to_dev(a) for a in (q, kq, kd, vq, vd)]
    c2 = [to_dev(a) for a in (q, kq, kd, vq, vd)]
    h1, h2 = h0.clone(), h0.clone()
    a = q8.attn_decode_append(*c1, t, SCALE, knew, vnew)
    q8.gemm_fused(wq, wd, a.view(1, -1), q8.PRO_F32, q8.EPI_ADD, out=h1)
    work = q8.attn_decode_append_partials(*c2, t, SCALE, knew, vnew)
    q8.gemm_attn_residual(wq, wd, work, t, h2)
    torch.cuda.synchronize()
    assert torch.equal(h1, h2)
    # and against the oracle: the product of the bf16 attention output
    ref = h0.cpu().numpy().astype(np.float64) + oracle.w8a16(to_host(wq), to_host(wd),
                                                              wl.f32_to_bf16_bits(to_host(a).reshape(1, -1)))
    assert_close(to_host(h2), ref, f"folded combine heads={heads} t={t}")
