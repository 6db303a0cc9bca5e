"""One batch-1 decode step of the Mimir-shaped model through the library's calls.

The block is the one the Frigg README's model table describes -- pre-norm,
RMSNorm without a learnable weight (eps 1e-6), rotary embedding (theta 10,000),
multi-head attention with 12 heads of 128 over an int8 key/value cache, SwiGLU
MLP, a final norm at the end of every module run, the 16-block L and H modules
applied in the order L L L H L L L H -- with the glue fused into the products:

    qkv      q8_gemm_fused  RMSNORM prologue, ROPE epilogue      -> bf16 q | k | v
    attn     q8_attn_decode_append (k, v appended at row t - 1)   -> fp32 [12][128]
    o        q8_gemm_fused  F32 prologue, ADD epilogue            -> h += o(attn)
             (contexts up to 1024 rows: q8_attn_decode_append_partials leaves the
             chunk partials and q8_gemm_attn_residual combines them in its
             prologue -- one launch fewer, the same bits)
    gate_up  q8_gemm_fused  RMSNORM prologue, SWIGLU epilogue     -> bf16 s
    down     q8_gemm_fused  BF16 prologue, ADD epilogue           -> h += down(s)
    (end of a module run: q8_rmsnorm(h) in place)
    lm_head  q8_gemm_fused  F32 prologue, F32 epilogue            -> fp32 logits

This module only allocates buffers and issues those calls in order on the
current stream (capturable into one HIP graph): every operation runs in the
library's kernels.  The qkv matrices are stored with the query and key rows of
every head in pair order and the gate/up matrices interleaved (gate j, up j),
the row orders the fused epilogues read (workloads.rope_pair_rows,
workloads.swiglu_pair_rows).
"""
from __future__ import annotations

import math

import torch

import int8_weight_streaming_amd as q8

HEADS = 12
HEAD_DIM = 128
# contexts whose attention combine q8_gemm_attn_residual takes over: up to 8
# chunks it saves the combine launch; with 16 it measured slower than it
FOLD_MAX_T = 1024


class DecodeStep:
    """Weights, caches and activation buffers of batch-1 decode steps.

    weights: {(block, proj): (wq, wd)} in natural row order, proj 0..3 = qkv, o,
    gate_up, down; lm_head: (wq, wd); order: the block of every virtual layer;
    module_ends: the virtual layers after which the module-final norm runs;
    t_cap: cache rows per virtual layer."""

    def __init__(self, weights, lm_head, order, module_ends, t_cap: int, rope_perm, swiglu_perm,
                 fold_combine: bool = True):
        dev = lm_head[0].device
        self.order = list(order)
        self.module_ends = set(module_ends)
        self.t_cap = int(t_cap)
        self.w = {}
        for (blk, proj), (wq, wd) in weights.items():
            if proj == 0:
                idx = torch.as_tensor(rope_perm, device=dev)
                wq, wd = wq.index_select(0, idx).contiguous(), wd.index_select(0, idx).contiguous()
            elif proj == 2:
                idx = torch.as_tensor(swiglu_perm, device=dev)
                wq, wd = wq.index_select(0, idx).contiguous(), wd.index_select(0, idx).contiguous()
            self.w[(blk, proj)] = (wq, wd)
        self.lm = lm_head
        hidden = lm_head[0].shape[1]
        inter = self.w[(self.order[0], 3)][0].shape[1]
        nv = len(self.order)
        self.kq = torch.zeros((nv, HEADS, t_cap, HEAD_DIM), dtype=torch.int8, device=dev)
        self.vq = torch.zeros_like(self.kq)
        self.kd = torch.zeros((nv, HEADS, t_cap, HEAD_DIM // 32), dtype=torch.uint16, device=dev)
        self.vd = torch.zeros_like(self.kd)
        self.h = torch.zeros((1, hidden), dtype=torch.float32, device=dev)
        self.qkv = torch.empty((1, 3 * hidden), dtype=torch.uint16, device=dev)
        self.attn = torch.empty((HEADS, HEAD_DIM), dtype=torch.float32, device=dev)
        self.s = torch.empty((1, inter), dtype=torch.uint16, device=dev)
        self.logits = torch.empty((1, lm_head[0].shape[0]), dtype=torch.float32, device=dev)
        self.work = torch.empty((max(1, q8.attn_work_words(HEADS, t_cap)),), dtype=torch.float32, device=dev)
        self.fold = fold_combine
        self.pwork = torch.empty((q8.attn_partial_words(HEADS, min(t_cap, FOLD_MAX_T)),), dtype=torch.float32,
                                 device=dev)
        self.scale = 1.0 / math.sqrt(HEAD_DIM)

    def run(self, t: int, hook=None):
        """Issue one step for the token at position t - 1 (context t, 1 <= t <=
        t_cap) on the current stream, reading and updating self.h.  hook(stage,
        v), if given, is called after every operation (for checking; not under
        graph capture; the "attn" stage only where the attention output is
        formed, i.e. not when the combine is folded into the o product)."""
        fold = self.fold and t <= FOLD_MAX_T
        hidden = self.h.shape[1]
        q = self.qkv[0, :hidden].view(HEADS, HEAD_DIM)
        knew = self.qkv[0, hidden:2 * hidden].view(HEADS, HEAD_DIM)
        vnew = self.qkv[0, 2 * hidden:].view(HEADS, HEAD_DIM)
        for v, blk in enumerate(self.order):
            wq, wd = self.w[(blk, 0)]
            q8.gemm_fused(wq, wd, self.h, q8.PRO_RMSNORM, q8.EPI_ROPE, out=self.qkv,
                          rope_rows=2 * hidden, pos=t - 1)
            hook and hook("qkv", v)
            wq, wd = self.w[(blk, 1)]
            if fold:
                q8.attn_decode_append_partials(q, self.kq[v], self.kd[v], self.vq[v], self.vd[v], t, self.scale,
                                               knew, vnew, work=self.pwork)
                q8.gemm_attn_residual(wq, wd, self.pwork, t, self.h)
            else:
                q8.attn_decode_append(q, self.kq[v], self.kd[v], self.vq[v], self.vd[v], t, self.scale,
                                      knew, vnew, work=self.work, out=self.attn)
                hook and hook("attn", v)
                q8.gemm_fused(wq, wd, self.attn.view(1, hidden), q8.PRO_F32, q8.EPI_ADD, out=self.h)
            hook and hook("o", v)
            wq, wd = self.w[(blk, 2)]
            q8.gemm_fused(wq, wd, self.h, q8.PRO_RMSNORM, q8.EPI_SWIGLU, out=self.s)
            hook and hook("gate_up", v)
            wq, wd = self.w[(blk, 3)]
            q8.gemm_fused(wq, wd, self.s, q8.PRO_BF16, q8.EPI_ADD, out=self.h)
            hook and hook("down", v)
            if v in self.module_ends:
                q8.rmsnorm(self.h, out=self.h)
                hook and hook("norm", v)
        q8.gemm_fused(self.lm[0], self.lm[1], self.h, q8.PRO_F32, q8.EPI_F32, out=self.logits)
        hook and hook("lm_head", len(self.order))
        return self.logits
