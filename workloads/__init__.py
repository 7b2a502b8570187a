"""Seeded synthetic workloads for causal attention on one context-parallel rank.

This module only describes shapes and draws random inputs.  It holds none of
the attention arithmetic, so both the fp64 oracle tests and the GPU tests can
use it without sharing any of the method's code.

Workloads follow the shapes on the pages:

* TransformerEngine PR 3510 ("Add head-parallel FA4 backward for cuDNN CP
  attention"), section Validation: 32K sequence, BF16, 32 heads, QK/V head
  dims 192/128, CP2/4/8, balanced (dual-chunk) partitions.
* TransformerEngine PR 3699 ("Add cuDNN OSS backward dispatch for context
  parallel attention"), section "D128 initialization policy": compact THD,
  Hq32/Hkv8, D128.
* TransformerEngine PR 3527 ("cuDNN FROST attention backend for head_dim in
  (256, 512]"), section Performance: hq/hkv GQA at symmetric head dim 512.

Inputs are drawn in fp32 from N(0, 1) and then rounded to bf16 (round to
nearest even), as PR 3527's test commit describes: drawing already-rounded
values would collapse the error floor of the accuracy criterion.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

__all__ = [
    "Workload", "CONFIGS", "thd_doc_layout", "dual_chunk_segments",
    "draw_inputs", "poison_padding",
]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    layout: str            # "bshd" or "thd"
    batch: int
    heads_q: int
    heads_kv: int
    d_qk: int
    d_v: int
    seqlen_q: int          # bshd: per-batch query rows; thd: physical tokens
    seqlen_k: int          # bshd: per-batch key rows; thd: physical tokens
    in_dtype: str          # "bf16" or "fp32"
    seed: int
    causal: bool = True
    # dual-chunk context-parallel rank (bshd only): cp size and rank
    cp: int = 0
    cp_rank: int = 0
    # number of KV blocks the forward is split into (ring-step partials)
    kv_blocks: int = 1
    description: str = ""

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.d_qk))


CONFIGS = {
    "tiny": Workload(
        name="tiny", layout="bshd", batch=1, heads_q=2, heads_kv=2, d_qk=64,
        d_v=64, seqlen_q=256, seqlen_k=256, in_dtype="fp32", seed=0,
        description="B1 H2 S256 D64, fp32 inputs, dense BSHD"),
    "dense8k": Workload(
        name="dense8k", layout="bshd", batch=1, heads_q=32, heads_kv=32,
        d_qk=128, d_v=128, seqlen_q=8192, seqlen_k=8192, in_dtype="bf16",
        seed=1, description="B1 H32 S8192 D128 bf16 dense BSHD"),
    "cp4_rank": Workload(
        name="cp4_rank", layout="bshd", batch=1, heads_q=32, heads_kv=32,
        d_qk=192, d_v=128, seqlen_q=8192, seqlen_k=32768, in_dtype="bf16",
        seed=2, cp=4, cp_rank=0, kv_blocks=8,
        description="one CP4 rank of a 32768-token causal sequence: Q = "
                    "chunks r and 7-r (4096 each, global positions), K/V all "
                    "32768, H32, D 192/128, 8 KV-block partials merged by LSE"),
    "thd_gqa": Workload(
        name="thd_gqa", layout="thd", batch=1, heads_q=32, heads_kv=8,
        d_qk=128, d_v=128, seqlen_q=32768, seqlen_k=32768, in_dtype="bf16",
        seed=3, description="packed THD, 32768 physical tokens, docs "
                            "U[128,8192] padded to 64, Hq32/Hkv8, D128"),
    "d512": Workload(
        name="d512", layout="bshd", batch=1, heads_q=16, heads_kv=4,
        d_qk=512, d_v=512, seqlen_q=16384, seqlen_k=16384, in_dtype="bf16",
        seed=4, description="B1 S16384 Hq16/Hkv4 D512 bf16 dense BSHD"),
}


def thd_doc_layout(seed: int, total: int = 32768, lo: int = 128,
                   hi: int = 8192, align: int = 64):
    """Document lengths for the packed THD workload.

    Lengths are drawn in order from numpy's default_rng(seed).integers(lo,
    hi + 1); each document is padded to a multiple of ``align`` physical rows
    (physical padded offsets plus visible lengths, as in TransformerEngine PR
    3149 "Enable FA4 for context-parallel attention", Description).  Drawing
    stops when the physical total reaches ``total``; a document that would
    overflow is cut to the remaining space (then it has no padding).

    Returns (seqused, cu_seqlens) as int32 numpy arrays.
    """
    rng = np.random.default_rng(seed)
    used, cu = [], [0]
    while cu[-1] < total:
        n = int(rng.integers(lo, hi + 1))
        phys = (n + align - 1) // align * align
        if cu[-1] + phys > total:
            phys = total - cu[-1]
            n = phys
        used.append(n)
        cu.append(cu[-1] + phys)
    return np.asarray(used, np.int32), np.asarray(cu, np.int32)


def dual_chunk_segments(seq_len: int, cp: int, rank: int):
    """Query segments held by one rank under the dual-chunk load balance.

    The sequence is cut into 2*cp chunks; rank r holds chunks r and
    2*cp-1-r, so every rank gets the same amount of causal work (the
    "balanced CP partitions" of TransformerEngine PR 3510, Changes).

    Returns a list of (row_begin, pos_begin, rows) with local row offsets.
    """
    chunk = seq_len // (2 * cp)
    first = rank * chunk
    second = (2 * cp - 1 - rank) * chunk
    return [(0, first, chunk), (chunk, second, chunk)]


def _randn(gen, shape):
    import torch
    return torch.randn(*shape, generator=gen, dtype=torch.float32)


def draw_inputs(w: Workload, heads: Optional[slice] = None):
    """Draw fp32 N(0,1) inputs in the order Q, K, V, dO with a torch CPU
    generator seeded by ``w.seed``.

    Returns a dict of fp32 CPU torch tensors ``q, k, v, do`` with BSHD shape
    [B, S, H, D] or THD shape [T, H, D], plus ``seqused``/``cu_seqlens`` for
    THD.  ``heads`` is ignored here (draws are always full, so that any head
    subset sees the same numbers); callers slice afterwards.
    """
    import torch
    gen = torch.Generator().manual_seed(w.seed)
    out = {}
    if w.layout == "thd":
        used, cu = thd_doc_layout(w.seed, total=w.seqlen_q)
        out["seqused"] = used
        out["cu_seqlens"] = cu
        qs = (w.seqlen_q, w.heads_q, w.d_qk)
        ks = (w.seqlen_k, w.heads_kv, w.d_qk)
        vs = (w.seqlen_k, w.heads_kv, w.d_v)
        os_ = (w.seqlen_q, w.heads_q, w.d_v)
    else:
        qs = (w.batch, w.seqlen_q, w.heads_q, w.d_qk)
        ks = (w.batch, w.seqlen_k, w.heads_kv, w.d_qk)
        vs = (w.batch, w.seqlen_k, w.heads_kv, w.d_v)
        os_ = (w.batch, w.seqlen_q, w.heads_q, w.d_v)
    out["q"] = _randn(gen, qs)
    out["k"] = _randn(gen, ks)
    out["v"] = _randn(gen, vs)
    out["do"] = _randn(gen, os_)
    return out


def poison_padding(t, cu_seqlens, seqused, value=float("nan")):
    """Fill the padding rows of a THD tensor [T, ...] with ``value``."""
    for n in range(len(seqused)):
        a = int(cu_seqlens[n]) + int(seqused[n])
        b = int(cu_seqlens[n + 1])
        if b > a:
            t[a:b] = value
    return t
