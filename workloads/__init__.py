"""Seeded synthetic inputs for the Q8_0 weight-streaming workloads.

This module is shared by the CPU oracle side and the GPU side, so it holds no
part of the method's arithmetic: it only draws numbers and lays them out.
Quantization, dot products and scale handling live elsewhere.

Recipe (numpy ``default_rng(PCG64(seed))``):

* weights: fp32 ``standard_normal`` times fp32 0.02, shape [N][K] row-major;
* activations: fp32 ``standard_normal`` rounded to bfloat16 (round to nearest,
  ties to even), returned as uint16 bit patterns, shape [M][K];
* the lm_head activation is additionally scaled to unit RMS (in fp64, then
  rounded to fp32 and to bf16);
* prefill activations carry seeded special rows (zero blocks, negative zeros,
  exact-half quotients, unit-scale rows) ahead of the N(0,1) rows.

The shapes follow the DFM-Mimir model described on the Frigg README ("The model,
as verified" table): hidden size 1536, SwiGLU intermediate 4096, 32 blocks,
vocabulary 262,144, and the recurrence that applies the 16-block L and H modules
in the order L L L H L L L H.
"""
from __future__ import annotations

import numpy as np

HIDDEN = 1536
INTER = 4096
VOCAB = 262144
N_BLOCKS = 32
# Per-block projections: (name, N = output rows, K = reduction length).
BLOCK_SHAPES = (
    ("qkv", 3 * HIDDEN, HIDDEN),        # [4608, 1536]
    ("o", HIDDEN, HIDDEN),              # [1536, 1536]
    ("gate_up", 2 * INTER, HIDDEN),     # [8192, 1536]
    ("down", HIDDEN, INTER),            # [1536, 4096]
)
LM_HEAD_SHAPE = (VOCAB, HIDDEN)
RECURRENCE = "LLLHLLLH"                 # L = blocks 0..15, H = blocks 16..31


def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round finite fp32 values to bfloat16 (nearest, ties to even); uint16 bits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = u + 0x7FFF + ((u >> 16) & 1)
    return (u >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def normal_weights(seed: int, n: int, k: int, std: float = 0.02) -> np.ndarray:
    """fp32 [n][k] ~ N(0, std^2)."""
    w = rng(seed).standard_normal((n, k), dtype=np.float32)
    w *= np.float32(std)
    return w


def normal_act_bf16(seed: int, m: int, k: int) -> np.ndarray:
    """bf16 bits [m][k] ~ N(0, 1)."""
    return f32_to_bf16_bits(rng(seed).standard_normal((m, k), dtype=np.float32))


def rms_unit_act_bf16(seed: int, k: int) -> np.ndarray:
    """bf16 bits [1][k]: z ~ N(0,1) scaled to unit RMS in fp64, then fp32, then bf16."""
    z = rng(seed).standard_normal(k).astype(np.float64)
    z = z / np.sqrt(np.mean(z * z))
    return f32_to_bf16_bits(z.astype(np.float32)).reshape(1, k)


def special_rows_f32(seed: int, k: int) -> np.ndarray:
    """Eleven fp32 rows of length k (k % 32 == 0), every value bf16-exact.

    row 0: +0.0; row 1: -0.0; row 2: every 4th 32-block zero, the rest N(0,1)
    rounded to bf16; rows 3-6: per block, element 0 is +-127*2^-e (e in 0..8)
    and the others +-(j + 1/2)*2^-e with j uniform in [0, 126]; rows 7-10: per
    block one element of magnitude 127 and the others integers or half-integers
    in [-127, 127].
    """
    g = rng(seed)
    nb = k // 32
    out = np.zeros((11, k), dtype=np.float32)
    out[1, :] = -0.0
    r2 = bf16_bits_to_f32(f32_to_bf16_bits(g.standard_normal(k, dtype=np.float32)))
    for b in range(0, nb, 4):
        r2[32 * b:32 * b + 32] = 0.0
    out[2] = r2
    for r in range(3, 7):
        for b in range(nb):
            e = int(g.integers(0, 9))
            sc = np.float32(2.0 ** -e)
            j = g.integers(0, 127, size=32).astype(np.float32)
            sg = np.where(g.integers(0, 2, size=32) == 0, -1.0, 1.0).astype(np.float32)
            blk = sg * (j + np.float32(0.5)) * sc
            pos = int(g.integers(0, 32))
            blk[pos] = sg[pos] * np.float32(127.0) * sc
            out[r, 32 * b:32 * b + 32] = blk
    for r in range(7, 11):
        for b in range(nb):
            v = g.integers(-254, 255, size=32).astype(np.float32) * np.float32(0.5)
            pos = int(g.integers(0, 32))
            v[pos] = np.float32(127.0) if g.integers(0, 2) else np.float32(-127.0)
            out[r, 32 * b:32 * b + 32] = v
    return out


def prefill_act_bf16(seed: int, p: int, k: int) -> np.ndarray:
    """bf16 bits [p][k]: the eleven special rows (as many as fit), then N(0,1)."""
    g = rng(seed)
    x = g.standard_normal((p, k), dtype=np.float32)
    sp = special_rows_f32(seed + 7919, k)
    nsp = min(p, sp.shape[0])
    x[:nsp] = sp[:nsp]
    return f32_to_bf16_bits(x)


def mimir_weight_seed(block: int, proj: int) -> int:
    """Seed of block `block` (0..31), projection `proj` (0..3, BLOCK_SHAPES order)."""
    return 3000 + 4 * block + proj


LM_HEAD_SEED = 3999


def mimir_step_order():
    """The 513 GEMVs of one decode token as (block, proj) pairs, then ('lm_head', None).

    Eight module runs in the order L L L H L L L H; the L module is blocks 0..15
    and the H module blocks 16..31; each block runs qkv, o, gate_up, down.
    """
    seq = []
    for run in RECURRENCE:
        base = 0 if run == "L" else 16
        for layer in range(16):
            for proj in range(4):
                seq.append((base + layer, proj))
    seq.append(("lm_head", None))
    return seq


# Row orders of the fused decode-step products (layout only: which stored row
# holds which natural row; the weights themselves are not changed).

def rope_pair_rows(rope_rows: int, n: int) -> np.ndarray:
    """Stored row s -> natural row, for a matrix whose first rope_rows rows are
    heads of 128 stored in pair order (dimension i of a head, then i + 64) and
    whose remaining rows keep their order."""
    assert rope_rows % 128 == 0 and rope_rows <= n
    perm = np.arange(n, dtype=np.int64)
    for h in range(rope_rows // 128):
        for i in range(64):
            perm[128 * h + 2 * i] = 128 * h + i
            perm[128 * h + 2 * i + 1] = 128 * h + i + 64
    return perm


def swiglu_pair_rows(n: int) -> np.ndarray:
    """Stored row s -> natural row, for a [gate; up] matrix of n rows stored
    interleaved (gate j, up j)."""
    assert n % 2 == 0
    perm = np.empty(n, dtype=np.int64)
    perm[0::2] = np.arange(n // 2)
    perm[1::2] = np.arange(n // 2) + n // 2
    return perm


# The five workloads, by what they are.
CONFIGS = {
    "gemv_1536x1536_b1": dict(n=1536, k=1536, m=1, w_seed=101, x_seed=102),
    "lm_head_gemv_262144x1536_b1": dict(n=VOCAB, k=HIDDEN, m=1, w_seed=201, x_seed=202),
    "mimir_decode_step_b1": dict(m=1),
    "mimir_skinny_b8": dict(m=8),
    "prefill_p256": dict(p=256, xa_seed=501, xb_seed=502),
}
