"""One context-parallel rank's attention step on a single GPU.

The rank holds query chunks with their global positions (the dual-chunk
balanced partition of TransformerEngine PR 3510, "Add head-parallel FA4
backward for cuDNN CP attention", Changes) and the keys/values of the whole
sequence, cut into KV blocks the way a P2P ring would deliver them.  The
forward computes one partial attention per (query chunk, visible KV block)
and folds it into the chunk's fp32 accumulator with the LSE merge (the
per-step kernel call plus LSE correction of PR 3527's CP ring commits); the
last merge of a chunk writes the final O in the output dtype.  By default
the merge runs in the forward kernel's epilogue (attn_fwd_accum); with
fused_merge=False each partial goes to an fp32 buffer and attn_merge_lse
folds it in.  The backward
is one call over all the rank's query rows against all keys, with the
merged O and LSE.  The saved O and fp32 LSE are then packed into per-head-
group segments for the head-parallel exchange and unpacked again (PR 3510,
Description), bit-exactly.

Everything here is orchestration of the C-ABI calls on one stream; no
arithmetic of the method runs in Python.
"""
from __future__ import annotations

import dataclasses
from typing import List, Sequence, Tuple

import torch

from . import (CPA_FLAG_DQ_DIRECT, attn_bwd, attn_fwd, attn_merge_lse, pack_saved,
               pack_saved_size, unpack_saved)


@dataclasses.dataclass
class Chunk:
    row0: int    # first local query row
    rows: int
    pos0: int    # global position of row0


@dataclasses.dataclass
class Call:
    kind: str            # "fwd" or "merge"
    chunk: int
    block: int
    final: bool


class RankStep:
    """Buffers and call plan for one rank's forward + backward + pack.

    q [B, Sq, Hq, Dqk], k [B, Sk, Hkv, Dqk], v [B, Sk, Hkv, Dv], dout
    [B, Sq, Hq, Dv] on one device.  ``chunks`` lists (row0, rows, pos0) of
    the query chunks; keys have positions 0..Sk-1 and are split into
    ``kv_blocks`` equal blocks.
    """

    def __init__(self, q, k, v, dout, chunks: Sequence[Tuple[int, int, int]], kv_blocks: int,
                 *, scale=None, pack_groups: int = 4, out_dtype=None,
                 fused_merge: bool = True):
        self.q, self.k, self.v, self.dout = q, k, v, dout
        self.scale = scale
        self.fused_merge = fused_merge
        self.chunks = [Chunk(*c) for c in chunks]
        b, sq, hq, _ = q.shape
        sk = k.shape[1]
        dv = v.shape[-1]
        if sk % kv_blocks:
            raise ValueError("keys must split evenly into kv_blocks")
        self.block = sk // kv_blocks
        self.kv_blocks = kv_blocks
        self.pack_groups = pack_groups
        dev = q.device
        odt = out_dtype or q.dtype
        self.o = torch.empty(b, sq, hq, dv, dtype=odt, device=dev)
        self.lse = torch.empty(b, hq, sq, dtype=torch.float32, device=dev)
        self.o_acc = torch.empty(b, sq, hq, dv, dtype=torch.float32, device=dev)
        self.lse_acc = torch.empty(b, hq, sq, dtype=torch.float32, device=dev)
        maxrows = max(c.rows for c in self.chunks)
        self.o_part = torch.empty(b, maxrows, hq, dv, dtype=torch.float32, device=dev)
        self.lse_part = torch.empty(b, hq, maxrows, dtype=torch.float32, device=dev)
        self.dq = torch.empty_like(q, dtype=odt)
        self.dk = torch.empty_like(k, dtype=odt)
        self.dv = torch.empty_like(v, dtype=odt)
        self.segments = [(c.row0, c.pos0) for c in self.chunks]
        self.plan = self._plan()
        self.fwd_ws = torch.empty(256, dtype=torch.uint8, device=dev)
        from . import bwd_workspace_bytes
        self.bwd_ws = torch.empty(bwd_workspace_bytes(q, k, v), dtype=torch.uint8, device=dev)
        nbuf = pack_saved_size(self.o, self.lse, pack_groups)
        self.pack_buf = torch.empty(nbuf, dtype=torch.uint8, device=dev)
        self.o_recv = torch.empty_like(self.o)
        self.lse_recv = torch.empty_like(self.lse)

    def visible_blocks(self, c: Chunk) -> List[int]:
        last_pos = c.pos0 + c.rows - 1
        return [j for j in range(self.kv_blocks) if j * self.block <= last_pos]

    def _plan(self) -> List[Call]:
        plan = []
        for ci, c in enumerate(self.chunks):
            blocks = self.visible_blocks(c)
            for n, j in enumerate(blocks):
                last = n == len(blocks) - 1
                if self.fused_merge:
                    plan.append(Call("fwd", ci, j, final=last))
                    continue
                plan.append(Call("fwd", ci, j, final=(len(blocks) == 1)))
                if n > 0:
                    plan.append(Call("merge", ci, j, final=last))
        return plan

    def n_fwd_calls(self) -> int:
        return sum(1 for c in self.plan if c.kind == "fwd")

    def n_merges(self) -> int:
        return sum(1 for c in self.plan if c.kind == "merge")

    # ---------------------------------------------------------------- calls

    def forward(self, stream=None):
        blk = self.block
        for call in self.plan:
            c = self.chunks[call.chunk]
            rs = slice(c.row0, c.row0 + c.rows)
            ks = slice(call.block * blk, (call.block + 1) * blk)
            if call.kind == "fwd" and self.fused_merge and call.block != self.visible_blocks(c)[0]:
                acc = (self.o_acc[:, rs], self.lse_acc[:, :, rs])
                out = (self.o[:, rs], self.lse[:, :, rs]) if call.final else acc
                attn_fwd(self.q[:, rs], self.k[:, ks], self.v[:, ks], *out, causal=True,
                         scale=self.scale, q_segments=[(0, c.pos0)], k_pos_begin=ks.start,
                         workspace=self.fwd_ws, stream=stream, acc=acc)
            elif call.kind == "fwd":
                first = call.block == self.visible_blocks(c)[0]
                if call.final and first:
                    o, lse = self.o[:, rs], self.lse[:, :, rs]
                elif first:
                    o, lse = self.o_acc[:, rs], self.lse_acc[:, :, rs]
                else:
                    o, lse = self.o_part[:, :c.rows], self.lse_part[:, :, :c.rows]
                attn_fwd(self.q[:, rs], self.k[:, ks], self.v[:, ks], o, lse, causal=True,
                         scale=self.scale, q_segments=[(0, c.pos0)], k_pos_begin=ks.start,
                         workspace=self.fwd_ws, stream=stream)
            else:
                out_o = self.o[:, rs] if call.final else self.o_acc[:, rs]
                out_l = self.lse[:, :, rs] if call.final else self.lse_acc[:, :, rs]
                attn_merge_lse(self.o_acc[:, rs], self.lse_acc[:, :, rs],
                               self.o_part[:, :c.rows], self.lse_part[:, :, :c.rows],
                               out_o, out_l, stream=stream)
        return self.o, self.lse

    def backward(self, stream=None, main_events=None):
        """One backward over all query rows and keys.  ``main_events`` =
        (start, end) HIP events recorded around the key-outer main kernel
        only."""
        # one main and one dq over every key block with the full workspace:
        # the dq step writes dq itself (no accumulator clear, no post pass)
        kw = dict(causal=True, scale=self.scale, q_segments=self.segments, k_pos_begin=0,
                  workspace=self.bwd_ws, stream=stream, flags=CPA_FLAG_DQ_DIRECT)
        args = (self.q, self.k, self.v, self.o, self.dout, self.lse, self.dq, self.dk, self.dv)
        attn_bwd(*args, step="attn_bwd_pre", **kw)
        if main_events:
            main_events[0].record(stream)
        attn_bwd(*args, step="attn_bwd_main", **kw)
        if main_events:
            main_events[1].record(stream)
        attn_bwd(*args, step="attn_bwd_dq", **kw)
        attn_bwd(*args, step="attn_bwd_post", **kw)
        return self.dq, self.dk, self.dv

    def pack_roundtrip(self, stream=None):
        pack_saved(self.o, self.lse, self.pack_groups, self.pack_buf, stream=stream)
        unpack_saved(self.pack_buf, self.o_recv, self.lse_recv, self.pack_groups, stream=stream)
        return self.pack_buf

    def step(self, stream=None, main_events=None):
        self.forward(stream)
        self.pack_roundtrip(stream)
        self.backward(stream, main_events)


def cp_chunks(seq_len: int, cp: int, rank: int):
    """(row0, rows, pos0) of the two dual-chunk query chunks of a rank."""
    chunk = seq_len // (2 * cp)
    return [(0, chunk, rank * chunk), (chunk, chunk, (2 * cp - 1 - rank) * chunk)]
