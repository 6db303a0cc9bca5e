"""C ABI checks that need no GPU: the library loads, exports every function that
include/q8stream.h declares, and rejects bad arguments on the host before any HIP
call (so nothing is enqueued and no pointer is touched -- the pointers used here
are fake addresses that would fault if dereferenced)."""
import ctypes as C
import os
import re

import pytest

import int8_weight_streaming_amd as q8

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "q8stream.h")

OK, NULL, SHAPE, BATCH, ALIGN, ENUM, DEVICE = 0, 1, 2, 3, 4, 5, 6
A = 0x100000          # fake, 16-byte aligned "device" addresses (never dereferenced)
B = 0x200000
MIS = 0x300004        # misaligned


def declared_functions(header=HEADER):
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(q[48]_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return q8.load_library()


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert set(names) == set(q8.EXPORTED)
    for name in names:
        assert hasattr(lib, name), name
    # the measurement probes live in their own library, not in the product's
    from int8_weight_streaming_amd import probe as q8probe
    plib = q8probe.load()
    probe = declared_functions(os.path.join(ROOT, "include", "q8probe.h"))
    assert set(probe) == set(q8probe.EXPORTED)
    for name in probe:
        assert hasattr(plib, name), name
        assert not hasattr(lib, name), name


def test_version_and_status_strings(lib):
    assert lib.q8_abi_version() == 1
    assert [q8.status_str(s) for s in range(8)] == [
        "Q8_OK", "Q8_ERR_NULL", "Q8_ERR_SHAPE", "Q8_ERR_BATCH", "Q8_ERR_ALIGN",
        "Q8_ERR_ENUM", "Q8_ERR_DEVICE", "Q8_ERR_HIP"]
    assert q8.status_str(99) == "unknown"
    assert q8.status_str(-1) == "unknown"


def test_quantize_validation(lib):
    f = lib.q8_quantize_weights
    assert f(A, 4, 0, A, B, None) == SHAPE
    assert f(A, 4, 48, A, B, None) == SHAPE
    assert f(A, 4, 16, A, B, None) == SHAPE
    assert f(A, -1, 64, A, B, None) == SHAPE
    assert f(A, 1 << 31, 64, A, B, None) == SHAPE
    assert f(A, (1 << 30), 1 << 20, A, B, None) == SHAPE      # n*k overflow limit
    assert f(None, 4, 64, A, B, None) == NULL
    assert f(A, 4, 64, None, B, None) == NULL
    assert f(A, 4, 64, A, None, None) == NULL
    assert f(MIS, 4, 64, A, B, None) == ALIGN
    assert f(A, 4, 64, MIS, B, None) == ALIGN
    assert f(A, 4, 64, A, MIS, None) == ALIGN
    assert f(None, 0, 64, None, None, None) == OK              # empty: no pointer touched
    g = lib.q8_quantize_act
    assert g(A, 3, 33, A, B, None) == SHAPE
    assert g(None, 3, 64, A, B, None) == NULL
    assert g(A, 3, 64, A, MIS, None) == ALIGN
    assert g(None, 0, 64, None, None, None) == OK


def test_skinny_validation(lib):
    f = lib.q8_gemm_skinny
    # act enum and the xd / act agreement come first
    assert f(A, B, 8, 64, 1, 2, A, None, A, None) == ENUM
    assert f(A, B, 8, 64, 1, -1, A, None, A, None) == ENUM
    assert f(A, B, 8, 64, 1, 0, A, B, A, None) == ENUM         # bf16 with xd
    assert f(A, B, 8, 64, 1, 1, A, None, A, None) == ENUM      # q8 without xd
    assert f(A, B, 8, 40, 1, 0, A, None, A, None) == SHAPE
    assert f(A, B, -2, 64, 1, 0, A, None, A, None) == SHAPE
    assert f(A, B, 8, 64, 9, 0, A, None, A, None) == BATCH
    assert f(A, B, 8, 64, -1, 0, A, None, A, None) == BATCH
    assert f(None, B, 8, 64, 1, 0, A, None, A, None) == NULL
    assert f(A, None, 8, 64, 1, 0, A, None, A, None) == NULL
    assert f(A, B, 8, 64, 1, 0, None, None, A, None) == NULL
    assert f(A, B, 8, 64, 1, 0, A, None, None, None) == NULL
    assert f(MIS, B, 8, 64, 1, 0, A, None, A, None) == ALIGN
    assert f(A, B, 8, 64, 1, 0, MIS, None, A, None) == ALIGN
    assert f(A, B, 8, 64, 1, 0, A, None, MIS, None) == ALIGN
    assert f(A, B, 8, 64, 1, 1, A, MIS, A, None) == ALIGN
    assert f(None, None, 0, 64, 3, 0, None, None, None, None) == OK
    assert f(None, None, 5, 64, 0, 0, None, None, None, None) == OK
    g = lib.q8_gemv
    assert g(A, B, 8, 64, 7, A, None, A, None) == ENUM
    assert g(A, B, 8, 31, 0, A, None, A, None) == SHAPE
    assert g(None, B, 8, 64, 0, A, None, A, None) == NULL
    assert g(None, None, 0, 64, 0, None, None, None, None) == OK


def test_prefill_and_block_dots_validation(lib):
    f = lib.q8_gemm_prefill
    assert f(A, B, 8, 48, 4, A, B, A, None) == SHAPE
    assert f(A, B, 8, 64, 65535 * 64 + 1, A, B, A, None) == SHAPE
    assert f(A, B, 8, 64, 4, None, B, A, None) == NULL
    assert f(A, B, 8, 64, 4, A, None, A, None) == NULL
    assert f(A, B, 8, 64, 4, A, B, MIS, None) == ALIGN
    assert f(None, None, 8, 64, 0, None, None, None, None) == OK
    assert f(None, None, 0, 64, 9, None, None, None, None) == OK
    g = lib.q8_block_dots
    assert g(A, 8, 64, 9, A, A, None) == BATCH
    assert g(A, 8, 50, 1, A, A, None) == SHAPE
    assert g(A, 8, 64, 1, None, A, None) == NULL
    assert g(A, 8, 64, 1, A, MIS, None) == ALIGN
    assert g(None, 0, 64, 1, None, None, None) == OK


def test_frag_sizes_and_validation(lib):
    """Fragment order: rows rounded up to 64, K/32 blocks rounded up to 4; 32
    code bytes and 2 scale bytes per (row, block) of the padded matrix."""
    cb, sb = lib.q8_frag_code_bytes, lib.q8_frag_scale_bytes
    assert (cb(256, 1536), sb(256, 1536)) == (256 * 48 * 32, 256 * 48 * 2)
    assert (cb(1, 32), sb(1, 32)) == (64 * 4 * 32, 64 * 4 * 2)
    assert (cb(65, 96), sb(65, 96)) == (128 * 4 * 32, 128 * 4 * 2)
    assert (cb(4608, 4128), sb(4608, 4128)) == (4608 * 132 * 32, 4608 * 132 * 2)
    assert (cb(0, 64), sb(0, 64)) == (0, 0)
    for rows, k in ((4, 48), (4, 0), (-1, 64), (1 << 31, 64)):
        assert cb(rows, k) == -1 and sb(rows, k) == -1
    f = lib.q8_pack_frag
    assert f(A, B, 4, 48, A, B, None) == SHAPE
    assert f(A, B, -1, 64, A, B, None) == SHAPE
    assert f(None, B, 4, 64, A, B, None) == NULL
    assert f(A, B, 4, 64, A, None, None) == NULL
    assert f(A, B, 4, 64, MIS, B, None) == ALIGN
    assert f(A, MIS, 4, 64, A, B, None) == ALIGN
    assert f(None, None, 0, 64, None, None, None) == OK
    h = lib.q8_quantize_act_fused_frag
    assert h(A, 4, 64, 0, A, B, None) == ENUM                # the bf16 prologue is not a quantizer input
    assert h(A, 4, 48, 1, A, B, None) == SHAPE
    assert h(A, 65535 * 64 + 1, 64, 1, A, B, None) == SHAPE
    assert h(None, 4, 64, 2, A, B, None) == NULL
    assert h(A, 4, 64, 2, A, MIS, None) == ALIGN
    assert h(None, 0, 64, 2, None, None, None) == OK
    g = lib.q8_gemm_prefill_frag
    assert g(A, B, 8, 48, 4, A, B, A, None) == SHAPE
    assert g(A, B, 8, 64, 65535 * 64 + 1, A, B, A, None) == SHAPE
    assert g(A, B, -8, 64, 4, A, B, A, None) == SHAPE
    assert g(A, B, 8, (1 << 25) + 32, 4, A, B, A, None) == SHAPE      # K beyond 32-bit tile offsets
    assert g(A, B, 8, 64, 4, None, B, A, None) == NULL
    assert g(A, None, 8, 64, 4, A, B, A, None) == NULL
    assert g(A, B, 8, 64, 4, A, B, None, None) == NULL
    assert g(A, B, 8, 64, 4, A, MIS, A, None) == ALIGN
    assert g(A, B, 8, 64, 4, A, B, MIS, None) == ALIGN
    assert g(None, None, 8, 64, 0, None, None, None, None) == OK
    assert g(None, None, 0, 64, 9, None, None, None, None) == OK
    import torch
    if not torch.cuda.is_available():
        assert f(A, B, 4, 64, A, B, None) == DEVICE
        assert g(A, B, 8, 64, 4, A, B, A, None) == DEVICE


def test_q4_validation(lib):
    f = lib.q4_quantize_weights
    assert f(A, 4, 48, A, B, None) == SHAPE
    assert f(A, -1, 64, A, B, None) == SHAPE
    assert f(None, 4, 64, A, B, None) == NULL
    assert f(A, 4, 64, None, B, None) == NULL
    assert f(A, 4, 64, A, MIS, None) == ALIGN
    assert f(None, 0, 64, None, None, None) == OK
    g = lib.q4_gemm_skinny
    assert g(A, B, 8, 64, 1, 2, A, None, A, None) == ENUM
    assert g(A, B, 8, 64, 1, 0, A, B, A, None) == ENUM
    assert g(A, B, 8, 64, 1, 1, A, None, A, None) == ENUM
    assert g(A, B, 8, 40, 1, 0, A, None, A, None) == SHAPE
    assert g(A, B, 8, 64, 9, 0, A, None, A, None) == BATCH
    assert g(None, B, 8, 64, 1, 0, A, None, A, None) == NULL
    assert g(A, B, 8, 64, 1, 0, A, None, None, None) == NULL
    assert g(MIS, B, 8, 64, 1, 0, A, None, A, None) == ALIGN
    assert g(A, B, 8, 64, 1, 1, A, MIS, A, None) == ALIGN
    assert g(None, None, 0, 64, 3, 0, None, None, None, None) == OK
    assert g(None, None, 5, 64, 0, 1, None, B, None, None) == OK


def test_fused_validation(lib):
    f = lib.q8_gemm_fused
    # (prologue, epilogue) pairs outside the supported set
    assert f(A, B, 8, 64, 1, 0, A, 0, A, 0, 0, None) == ENUM      # BF16 + F32: the plain product
    assert f(A, B, 8, 64, 1, 1, A, 3, A, 0, 0, None) == ENUM
    assert f(A, B, 8, 64, 1, 3, A, 0, A, 0, 0, None) == ENUM
    assert f(A, B, 8, 64, 1, 2, A, 4, A, 0, 0, None) == ENUM
    assert f(A, B, 8, 40, 1, 2, A, 3, A, 0, 0, None) == SHAPE
    assert f(A, B, 8, 64, 9, 2, A, 3, A, 0, 0, None) == BATCH
    assert f(A, B, 7, 64, 1, 2, A, 2, A, 0, 0, None) == SHAPE     # odd n, paired epilogue
    assert f(A, B, 256, 64, 1, 2, A, 3, A, 64, 0, None) == SHAPE  # rope_rows not a multiple of 128
    assert f(A, B, 256, 64, 1, 2, A, 3, A, 384, 0, None) == SHAPE # rope_rows > n
    assert f(A, B, 256, 64, 1, 2, A, 3, A, 128, -1, None) == SHAPE
    assert f(A, B, 7, 64, 1, 1, A, 1, A, 0, 0, None) != SHAPE     # odd n is fine unpaired
    assert f(None, B, 8, 64, 1, 2, A, 3, A, 0, 0, None) == NULL
    assert f(A, B, 8, 64, 1, 2, A, 3, None, 0, 0, None) == NULL
    assert f(A, B, 8, 64, 1, 2, MIS, 3, A, 0, 0, None) == ALIGN
    assert f(None, None, 0, 64, 1, 2, None, 3, None, 0, 0, None) == OK
    g = lib.q8_rmsnorm
    assert g(A, 2, 0, B, None) == SHAPE
    assert g(A, 2, 48, B, None) == SHAPE                          # k not a multiple of 32
    assert g(A, -1, 64, B, None) == SHAPE
    assert g(None, 2, 64, B, None) == NULL
    assert g(A, 2, 64, MIS, None) == ALIGN
    assert g(None, 0, 64, None, None) == OK
    qf = lib.q8_quantize_act_fused
    assert qf(A, 2, 64, 0, A, B, None) == ENUM                     # bf16 prologue: q8_quantize_act
    assert qf(A, 2, 64, 7, A, B, None) == ENUM
    assert qf(A, 2, 48, 2, A, B, None) == SHAPE
    assert qf(A, -1, 64, 1, A, B, None) == SHAPE
    assert qf(A, 2, 64, 2, None, B, None) == NULL
    assert qf(A, 2, 64, 1, A, MIS, None) == ALIGN
    assert qf(None, 0, 64, 2, None, None, None) == OK


def test_attn_partials_and_residual_validation(lib):
    pw = lib.q8_attn_partial_words
    assert pw(12, 512) == 12 * 8 * 132 and pw(12, 1) == 12 * 132 and pw(12, 4096) == 12 * 16 * 132
    # sizes cover every shorter context (8 chunks of 64 rows at 512, 16 of 128 at 2048)
    assert pw(12, 600) == 12 * 8 * 132 and pw(12, 2049) == 12 * 16 * 132 and pw(12, 1500) == 12 * 12 * 132
    assert all(pw(3, t) <= pw(3, t + 1) for t in range(1, 4200))
    assert pw(-1, 5) == -1 and pw(2, 0) == -1
    f = lib.q8_attn_decode_append_partials
    need = pw(2, 200)
    base = [A, B, A, B, A, 2, 200, 256, 128, 0.088, A, B, A, need, None]

    def call(**kw):
        a = list(base)
        for i, v in kw.items():
            a[int(i[1:])] = v
        return f(*a)
    assert call(a8=64) == SHAPE
    assert call(a6=300) == SHAPE
    assert call(a13=need - 1) == SHAPE
    assert call(a12=None) == NULL                      # work is required (even for one chunk)
    assert call(a10=None) == NULL
    assert call(a12=MIS) == ALIGN
    assert call(a5=0) == OK
    g = lib.q8_gemm_attn_residual
    wneed = pw(12, 512)
    assert g(A, B, 1536, 1536, A, wneed, 512, A, None) != SHAPE
    assert g(A, B, 1536, 1600, A, wneed, 512, A, None) == SHAPE   # k not a multiple of 128
    assert g(A, B, 1536, 4096, A, 1 << 20, 512, A, None) == SHAPE # k > 2048
    assert g(A, B, 1536, 1536, A, 1 << 20, 4097, A, None) == SHAPE  # more than 16 chunks
    assert g(A, B, 1536, 1536, A, wneed, 0, A, None) == SHAPE
    assert g(A, B, 1536, 1536, A, wneed - 1, 512, A, None) == SHAPE
    assert g(A, B, 1536, 1536, None, wneed, 512, A, None) == NULL
    assert g(A, B, 1536, 1536, A, wneed, 512, MIS, None) == ALIGN
    assert g(None, None, 0, 1536, None, wneed, 512, None, None) == OK


def test_attn_append_validation(lib):
    f = lib.q8_attn_decode_append
    need = lib.q8_attn_work_words(2, 300)
    assert need > 0
    base = [A, B, A, B, A, 2, 300, 400, 128, 0.088, A, B, A, B, need, None]

    def call(**kw):
        a = list(base)
        for i, v in kw.items():
            a[int(i[1:])] = v
        return f(*a)
    assert call(a8=64) == SHAPE                        # head_dim
    assert call(a6=500) == SHAPE                       # t > t_cap
    assert call(a6=0) == SHAPE
    assert call(a10=None) == NULL                      # knew
    assert call(a11=None) == NULL                      # vnew
    assert call(a11=MIS) == ALIGN
    assert call(a14=need - 1) == SHAPE
    assert call(a5=0) == OK


def test_valid_arguments_without_gpu_report_device(lib):
    """With valid arguments the call reaches the device check; with no usable
    gfx950 it refuses with Q8_ERR_DEVICE instead of launching anything."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert lib.q8_gemm_skinny(A, B, 8, 64, 1, 0, A, None, A, None) == DEVICE
    assert lib.q8_quantize_weights(A, 4, 64, A, B, None) == DEVICE
    assert lib.q4_gemm_skinny(A, B, 8, 64, 2, 0, A, None, A, None) == DEVICE


def test_probe_validation():
    """The measurement probes check their arguments before any device call."""
    from int8_weight_streaming_amd import probe as q8probe
    plib = q8probe.load()
    assert plib.q8_probe_read(A, 0, 8, A, None) == SHAPE
    assert plib.q8_probe_read(A, 24, 8, A, None) == SHAPE
    assert plib.q8_probe_read(A, 64, 5, A, None) == SHAPE      # loads per thread not offered
    assert plib.q8_probe_read(None, 64, 8, A, None) == NULL
    assert plib.q8_probe_read(MIS, 64, 8, A, None) == ALIGN
    assert plib.q8_probe_barrier(None, 4, 1, None) == NULL
    assert plib.q8_probe_barrier(0x300002, 4, 1, None) == ALIGN   # flags need 4-byte alignment
    assert plib.q8_probe_barrier_words() > 8 * 1024
    assert plib.q8_probe_mfma_i8(0, 10, A, None) == SHAPE
    assert plib.q8_probe_mfma_i8(4, 0, A, None) == SHAPE
    assert plib.q8_probe_mfma_i8(4, 10, None, None) == NULL


def test_attn_validation(lib):
    f = lib.q8_attn_decode                                 # prototype set by load_library()
    need = lib.q8_attn_work_words(2, 300)
    assert need == 2 * 5 * 132                             # 64-row chunks above 256 rows
    assert lib.q8_attn_work_words(12, 256) == 0 and lib.q8_attn_work_words(12, 257) == 12 * 5 * 132
    assert lib.q8_attn_work_words(12, 4096) == 12 * 16 * 132
    assert all(lib.q8_attn_work_words(3, t) <= lib.q8_attn_work_words(3, t + 1) for t in range(1, 4200))
    assert lib.q8_attn_work_words(1, 0) == -1
    args = lambda **kw: dict(dict(q=A, kq=B, kd=A, vq=B, vd=A, heads=2, t=300, t_cap=400, d=128,
                                  scale=0.088, out=A, work=B, words=need), **kw)
    call = lambda a: f(a["q"], a["kq"], a["kd"], a["vq"], a["vd"], a["heads"], a["t"], a["t_cap"],
                       a["d"], a["scale"], a["out"], a["work"], a["words"], None)
    assert call(args(d=64)) == SHAPE
    assert call(args(t=0)) == SHAPE
    assert call(args(t=500)) == SHAPE                      # t > t_cap
    assert call(args(t_cap=1 << 24)) == SHAPE
    assert call(args(scale=float("nan"))) == SHAPE
    assert call(args(scale=float("inf"))) == SHAPE
    assert call(args(words=need - 1)) == SHAPE
    assert call(args(q=None)) == NULL
    assert call(args(work=None)) == NULL
    assert call(args(kd=MIS)) == ALIGN
    assert call(args(heads=0, q=None, kq=None, kd=None, vq=None, vd=None, out=None, work=None)) == OK
    # one chunk (up to 256 rows): no workspace needed
    assert call(args(t=256, work=None, words=0)) in (DEVICE, OK)
    assert call(args(t=257, work=None, words=0)) == SHAPE
    import torch
    if not torch.cuda.is_available():
        assert call(args()) == DEVICE


def test_attn_noalloc_validation(lib):
    """The allocation-free attention checks its arguments, and that the partials
    of (heads, t) fit its static scratch, before any device call."""
    f = lib.q8_attn_decode_noalloc
    assert q8.ATTN_SCRATCH_WORDS == 262144
    hdr = open(HEADER).read()
    assert "#define Q8_ATTN_SCRATCH_WORDS 262144" in hdr
    args = lambda **kw: dict(dict(q=A, kq=B, kd=A, vq=B, vd=A, heads=12, t=4096, t_cap=4096, d=128,
                                  scale=0.088, out=A), **kw)
    call = lambda a: f(a["q"], a["kq"], a["kd"], a["vq"], a["vd"], a["heads"], a["t"], a["t_cap"],
                       a["d"], a["scale"], a["out"], None)
    assert call(args(d=64)) == SHAPE
    assert call(args(t=0)) == SHAPE
    assert call(args(t=5000)) == SHAPE                     # t > t_cap
    assert call(args(scale=float("nan"))) == SHAPE
    assert call(args(q=None)) == NULL
    assert call(args(out=None)) == NULL
    assert call(args(vd=MIS)) == ALIGN
    assert call(args(heads=0, q=None, kq=None, kd=None, vq=None, vd=None, out=None)) == OK
    # the largest context of 12 heads whose partials fit, and the next one
    big = 1 << 20
    fits = [t for t in (42240, 42241) if lib.q8_attn_work_words(12, t) <= q8.ATTN_SCRATCH_WORDS]
    assert fits == [42240]
    assert call(args(t=42241, t_cap=big)) == SHAPE
    assert call(args(heads=1, t=(1 << 24) - 128, t_cap=(1 << 24) - 128)) == SHAPE
    import torch
    if not torch.cuda.is_available():
        assert call(args(t=42240, t_cap=big)) == DEVICE
        assert call(args()) == DEVICE


def test_kernel_name_validation(lib):
    f = lib.q8_kernel_name
    import ctypes
    buf = ctypes.create_string_buffer(96)
    p = ctypes.cast(buf, ctypes.c_void_p)
    assert f(4, 8, 64, 1, 0, p, 96) == ENUM                  # unknown op
    assert f(-1, 8, 64, 1, 0, p, 96) == ENUM
    assert f(0, 8, 64, 1, 2, p, 96) == ENUM                  # unknown activation type
    assert f(0, 8, 48, 1, 0, p, 96) == SHAPE
    assert f(0, 8, 64, 9, 0, p, 96) == BATCH
    assert f(2, 8, 64, -1, 1, p, 96) == BATCH
    assert f(1, 8, 64, -1, 0, p, 96) == SHAPE                # negative p
    assert f(1, 8, 64, 65535 * 64 + 1, 0, p, 96) == SHAPE
    assert f(0, 8, 64, 1, 0, None, 96) == NULL
    assert f(0, 8, 64, 1, 0, p, 0) == SHAPE
    import torch
    if not torch.cuda.is_available():
        assert f(0, 8, 64, 1, 0, p, 96) == DEVICE
        assert f(1, 8, 64, 5, 7, p, 96) == DEVICE            # act is ignored for prefill
        assert f(3, 8, 64, 5, 7, p, 96) == DEVICE            # and for the fragment-order prefill
    assert f(3, 8, 64, 65535 * 64 + 1, 0, p, 96) == SHAPE
