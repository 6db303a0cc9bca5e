"""GPU parity of a whole batch-1 decode step with the glue fused into the
products (int8_weight_streaming_amd.decode_step), op by op against the oracle.

The step is run eagerly with a hook after every operation; each operation is
checked against the oracle given the inputs the GPU actually had at that point
(the residual stream, the bf16 activations, the cache), so rounding differences
cannot compound over layers.  Products and residual adds: max-abs 2e-3 and
relative L2 1e-5; bf16 outputs: the bounded-rounding rule of test_gpu_fused;
cache rows: bit-exact.  A reduced model (two blocks of the Mimir shapes, four
virtual layers in two module runs, a 4096-row vocabulary) is checked in full;
the full model (32 blocks, 128 virtual layers, 262,144-row lm_head) is run
eagerly and under graph replay and must give the same bits."""
import numpy as np
import pytest
import torch

import int8_weight_streaming_amd as q8
import oracle
import workloads as wl
from gpu_helpers import DEV, assert_close, log, oracle_threads, to_dev, to_host
from int8_weight_streaming_amd.decode_step import HEAD_DIM, HEADS, DecodeStep
from test_gpu_fused import assert_bf16_rounding_of, summation_bound

pytestmark = pytest.mark.gpu

SCALE = 1.0 / np.sqrt(HEAD_DIM)


@pytest.fixture(scope="module", autouse=True)
def _setup():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    q8.load_library()
    oracle.set_threads(oracle_threads())
    yield
    torch.cuda.synchronize()


def _perms():
    return wl.rope_pair_rows(2 * wl.HIDDEN, 3 * wl.HIDDEN), wl.swiglu_pair_rows(2 * wl.INTER)


def _norm_bf16(h_host):
    """bf16 of the GPU RMSNorm of h (the reduction the fused prologue uses)."""
    return wl.f32_to_bf16_bits(to_host(q8.rmsnorm(to_dev(h_host))))


def test_reduced_step_op_by_op():
    """Two consecutive tokens (context 300, then 301) of the reduced model,
    every operation checked; the second token attends over the first one's
    appended rows, which stay unchanged."""
    blocks, vocab, t, t_cap = 2, 4096, 300, 512
    order, module_ends = [0, 1, 0, 1], [1, 3]
    host, dev_w = {}, {}
    for blk in range(blocks):
        for proj, (_, n, k) in enumerate(wl.BLOCK_SHAPES):
            wq, wd = oracle.quantize_f32(wl.normal_weights(wl.mimir_weight_seed(blk, proj), n, k))
            host[(blk, proj)] = (wq, wd)
            dev_w[(blk, proj)] = (to_dev(wq), to_dev(wd))
    lq, ld = oracle.quantize_f32(wl.normal_weights(wl.LM_HEAD_SEED, vocab, wl.HIDDEN))
    rp, sp = _perms()
    st = DecodeStep(dev_w, (to_dev(lq), to_dev(ld)), order, module_ends, t_cap, rp, sp, fold_combine=False)
    # a context of t - 1 cached rows per virtual layer
    g = wl.rng(77)
    for v in range(len(order)):
        for c in (st.kq, st.vq):
            c[v].copy_(torch.from_numpy(g.integers(-127, 128, size=(HEADS, t_cap, HEAD_DIM), dtype=np.int8)).to(DEV))
        for c in (st.kd, st.vd):
            vals = (g.random((HEADS, t_cap, HEAD_DIM // 32)) * 0.02 + 0.005).astype(np.float16).view(np.uint16)
            c[v].copy_(to_dev(vals))
    h0 = (g.standard_normal((1, wl.HIDDEN)) * 1.0).astype(np.float32)
    st.h.copy_(to_dev(h0))
    torch.cuda.synchronize()

    state = {"h": h0.astype(np.float32), "t": t}
    checked = []

    def hook(stage, v):
        t = state["t"]
        torch.cuda.synchronize()
        h_prev = state["h"]
        h_now = to_host(st.h)
        blk = order[v] if v < len(order) else None
        if stage == "qkv":
            wq, wd = host[(blk, 0)]
            xb = _norm_bf16(h_prev)
            y = oracle.w8a16(wq, wd, xb)
            want, tol = y.copy(), summation_bound(wq, wd, xb)
            want[0, :2 * wl.HIDDEN] = oracle.rope(y[0, :2 * wl.HIDDEN], 2 * HEADS, HEAD_DIM, t - 1)
            bh = tol[0, :2 * wl.HIDDEN].reshape(-1, 2, 64)
            tol[0, :2 * wl.HIDDEN] = np.concatenate([bh[:, 0] + bh[:, 1]] * 2, axis=1).reshape(-1) + \
                2.0 ** -22 * np.abs(want[0, :2 * wl.HIDDEN])
            assert_bf16_rounding_of(to_host(st.qkv), want, tol, f"qkv v={v}")
        elif stage == "attn":
            qkv = to_host(st.qkv)[0]
            ck, cks = oracle.quantize_bf16(qkv[wl.HIDDEN:2 * wl.HIDDEN].reshape(HEADS, HEAD_DIM))
            cv, cvs = oracle.quantize_bf16(qkv[2 * wl.HIDDEN:].reshape(HEADS, HEAD_DIM))
            kq, kd, vq, vd = (to_host(c[v]) for c in (st.kq, st.kd, st.vq, st.vd))
            assert np.array_equal(kq[:, t - 1], ck) and np.array_equal(kd[:, t - 1], cks), f"K row v={v}"
            assert np.array_equal(vq[:, t - 1], cv) and np.array_equal(vd[:, t - 1], cvs), f"V row v={v}"
            ref = oracle.attn_decode(qkv[:wl.HIDDEN].reshape(HEADS, HEAD_DIM), kq, kd, vq, vd, t, SCALE)
            assert_close(to_host(st.attn), ref, f"attn v={v}")
        elif stage == "o":
            wq, wd = host[(blk, 1)]
            xb = wl.f32_to_bf16_bits(to_host(st.attn).reshape(1, -1))
            assert_close(h_now, h_prev.astype(np.float64) + oracle.w8a16(wq, wd, xb), f"o v={v}")
        elif stage == "gate_up":
            wq, wd = host[(blk, 2)]
            xb = _norm_bf16(h_prev)
            y = oracle.w8a16(wq, wd, xb)
            b = summation_bound(wq, wd, xb)
            gg, uu = y[:, :wl.INTER], y[:, wl.INTER:]
            tol = 1.1 * np.abs(uu) * b[:, :wl.INTER] + (np.abs(gg) + 0.3) * b[:, wl.INTER:]
            assert_bf16_rounding_of(to_host(st.s), oracle.swiglu(gg, uu), tol, f"swiglu v={v}")
        elif stage == "down":
            wq, wd = host[(blk, 3)]
            assert_close(h_now, h_prev.astype(np.float64) + oracle.w8a16(wq, wd, to_host(st.s)), f"down v={v}")
        elif stage == "norm":
            y64 = oracle.rmsnorm(h_prev)
            assert np.max(np.abs(h_now - y64) / (np.abs(y64) + 1e-30)) < 2e-6, f"norm v={v}"
        elif stage == "lm_head":
            assert_close(to_host(st.logits), oracle.w8a16(lq, ld, wl.f32_to_bf16_bits(h_prev)), "lm_head")
        state["h"] = h_now
        checked.append((stage, v))

    st.run(t, hook=hook)
    assert len(checked) == 5 * len(order) + len(module_ends) + 1
    # the next token: its attention reads the row this token appended
    appended = [(to_host(st.kq[v][:, t - 1]), to_host(st.vd[v][:, t - 1])) for v in range(len(order))]
    state["t"] = t + 1
    st.run(t + 1, hook=hook)
    assert len(checked) == 2 * (5 * len(order) + len(module_ends) + 1)
    for v, (kq_row, vd_row) in enumerate(appended):
        assert np.array_equal(to_host(st.kq[v][:, t - 1]), kq_row) and np.array_equal(to_host(st.vd[v][:, t - 1]), vd_row)


def test_full_step_graph_replay_bitwise():
    """The full Mimir-shaped step (128 virtual layers, context 64): eager run and
    graph replays from the same starting state give identical logits and
    caches; everything is finite."""
    log("full step: generating 32 blocks + lm_head")
    dev_w = {}
    for blk in range(wl.N_BLOCKS):
        for proj, (_, n, k) in enumerate(wl.BLOCK_SHAPES):
            w = to_dev(wl.normal_weights(wl.mimir_weight_seed(blk, proj), n, k))
            dev_w[(blk, proj)] = q8.quantize_weights(w)
            del w
    w = to_dev(wl.normal_weights(wl.LM_HEAD_SEED, *wl.LM_HEAD_SHAPE))
    lm = q8.quantize_weights(w)
    del w
    order = [blk for blk, _ in wl.mimir_step_order()[:-1:4]]
    module_ends = [v for v in range(len(order)) if v % 16 == 15]
    rp, sp = _perms()
    t, t_cap = 64, 64
    st = DecodeStep(dev_w, lm, order, module_ends, t_cap, rp, sp)
    h0 = to_dev((wl.rng(78).standard_normal((1, wl.HIDDEN))).astype(np.float32))
    st.h.copy_(h0)
    log("full step: eager")
    ref = st.run(t).clone()
    ref_k = st.kq.clone()
    torch.cuda.synchronize()
    assert torch.isfinite(ref).all()
    assert len(order) == 128
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    st.h.copy_(h0)
    with torch.cuda.stream(s):
        st.run(t)
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        st.run(t)
    for _ in range(2):
        st.h.copy_(h0)
        st.logits.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(st.logits, ref)
        assert torch.equal(st.kq, ref_k)


@pytest.mark.parametrize("t", [1, 129, 300, 1024, 2048, 4095])
def test_folded_combine_same_bits(t):
    """The step with the attention combine folded into the o product
    (contexts up to 4096 rows) gives the same bits -- residual stream, caches,
    logits -- as the step with the separate combine launch."""
    _folded_same_bits(t, 4100)


@pytest.mark.parametrize("t", [511, 512])
def test_folded_combine_tier_boundary(t):
    """A cache capacity between the attention's chunk tiers (600 rows: the
    workspaces are sized once from it) and two tokens across the 512-row
    boundary, where the chunk count drops from 8 to 5."""
    _folded_same_bits(t, 600)


def _folded_same_bits(t, t_cap):
    blocks, vocab = 2, 4096
    order, module_ends = [0, 1, 0, 1], [1, 3]
    dev_w = {}
    for blk in range(blocks):
        for proj, (_, n, k) in enumerate(wl.BLOCK_SHAPES):
            dev_w[(blk, proj)] = q8.quantize_weights(to_dev(wl.normal_weights(wl.mimir_weight_seed(blk, proj), n, k)))
    lm = q8.quantize_weights(to_dev(wl.normal_weights(wl.LM_HEAD_SEED, vocab, wl.HIDDEN)))
    rp, sp = _perms()
    steps = [DecodeStep(dev_w, lm, order, module_ends, t_cap, rp, sp, fold_combine=f) for f in (False, True)]
    g = wl.rng(500 + t)
    kq = torch.from_numpy(g.integers(-127, 128, size=(len(order), HEADS, t_cap, HEAD_DIM), dtype=np.int8)).to(DEV)
    kd = to_dev((g.random((len(order), HEADS, t_cap, HEAD_DIM // 32)) * 0.02 + 0.005).astype(np.float16).view(np.uint16))
    h0 = to_dev(g.standard_normal((1, wl.HIDDEN)).astype(np.float32))
    for st in steps:
        for c in (st.kq, st.vq):
            c.copy_(kq)
        for c in (st.kd, st.vd):
            c.copy_(kd)
        st.h.copy_(h0)
        st.run(t)
        st.run(t + 1)
    torch.cuda.synchronize()
    a, b = steps
    assert torch.equal(a.h, b.h) and torch.equal(a.logits, b.logits)
    assert torch.equal(a.kq, b.kq) and torch.equal(a.kd, b.kd) and torch.equal(a.vq, b.vq) and torch.equal(a.vd, b.vd)
    assert torch.isfinite(a.logits).all()
