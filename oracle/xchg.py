"""Byte-exact exchange buffers for the head-parallel all-to-alls.

Test infrastructure only (see the package docstring).

PR 3510 ("Add head-parallel FA4 backward for cuDNN CP attention",
Description and Diagram) moves the backward's inputs from the sequence
partition to a head partition with one all-to-all, runs a full-sequence
backward per head group, and sends dQ/dK/dV back the same way.  The pages
give no byte layout; this is the library's own convention (any layout is
correct if the round trip is exact), written here as plain array slicing:

A buffer holds ``groups`` segments, one per peer.  Segment g covers the
packed rows given by its row ranges [(row_begin, count), ...] (concatenated
in order, n_g rows) and, for each field in order, starting at a multiple of
256 bytes:

* a row field (array [B, R, H, D] of 2- or 4-byte elements): its heads
  [g*H/groups, (g+1)*H/groups) when ``split``, else all H heads (Hf of
  them); element (b, i, hh, d) of the packed rows at ((b*n_g + i)*Hf + hh)*D
  + d, raw bits;
* an LSE field (float32 [B, H, R]): element (b, hh, i) at (b*Hf + hh)*n_g
  + i, raw bits.

Segments follow each other, each padded to a multiple of 256 bytes.  Pad
bytes are never read.  Packing for the seq->heads exchange splits heads and
takes every local row; the receiver unpacks segment r (from sender r) into
the rows r holds, with all of the receiver's heads; the heads->seq return
swaps the two roles.
"""
from __future__ import annotations

import numpy as np


def _align(x, a=256):
    return (x + a - 1) // a * a


def _rows(ranges):
    return np.concatenate([np.arange(r0, r0 + n, dtype=np.int64) for r0, n in ranges]) \
        if ranges else np.zeros(0, np.int64)


def xchg_layout(batch, groups, ranges, fields):
    """fields: list of dicts {kind: 'rows'|'lse', heads, dim, elem_bytes,
    split}.  Returns (segment offsets [groups + 1], field offsets per
    segment [groups][nfields])."""
    seg_off = [0]
    field_off = []
    for g in range(groups):
        n = sum(c for _, c in ranges[g])
        off, offs = 0, []
        for f in fields:
            hf = f["heads"] // groups if f["split"] else f["heads"]
            off = _align(off)
            offs.append(off)
            if f["kind"] == "rows":
                off += batch * n * hf * f["dim"] * f["elem_bytes"]
            else:
                off += batch * hf * n * 4
        field_off.append(offs)
        seg_off.append(seg_off[-1] + _align(off))
    return seg_off, field_off


def _bits(a):
    a = np.ascontiguousarray(a)
    return a.view({2: np.uint16, 4: np.uint32}[a.dtype.itemsize])


def xchg_pack(arrays, groups, ranges, fields, batch):
    """arrays[f]: the field's local array.  Returns the uint8 buffer (pad
    bytes zero)."""
    seg_off, field_off = xchg_layout(batch, groups, ranges, fields)
    buf = np.zeros(seg_off[-1], dtype=np.uint8)
    for g in range(groups):
        rows = _rows(ranges[g])
        for f, a, fo in zip(fields, arrays, field_off[g]):
            hf = f["heads"] // groups if f["split"] else f["heads"]
            h0 = g * hf if f["split"] else 0
            if f["kind"] == "rows":
                part = _bits(a)[:, rows][:, :, h0:h0 + hf, :]
            else:
                part = np.asarray(a, np.float32).view(np.uint32)[:, h0:h0 + hf][:, :, rows]
            raw = np.ascontiguousarray(part).view(np.uint8).reshape(-1)
            base = seg_off[g] + fo
            buf[base:base + raw.size] = raw
    return buf


def xchg_unpack(buf, groups, ranges, fields, batch, outs):
    """Write each segment's packed rows and heads into ``outs`` (one array
    per field, modified in place; what no segment covers is left as is)."""
    seg_off, field_off = xchg_layout(batch, groups, ranges, fields)
    buf = np.asarray(buf, dtype=np.uint8)
    for g in range(groups):
        rows = _rows(ranges[g])
        n = rows.size
        for f, a, fo in zip(fields, outs, field_off[g]):
            hf = f["heads"] // groups if f["split"] else f["heads"]
            h0 = g * hf if f["split"] else 0
            base = seg_off[g] + fo
            if f["kind"] == "rows":
                cnt = batch * n * hf * f["dim"]
                bits = buf[base:base + cnt * f["elem_bytes"]].view(_bits(a).dtype)
                part = bits.reshape(batch, n, hf, f["dim"]).view(a.dtype)
                for i, r in enumerate(rows):
                    a[:, r, h0:h0 + hf, :] = part[:, i]
            else:
                cnt = batch * hf * n
                part = buf[base:base + cnt * 4].view(np.float32).reshape(batch, hf, n)
                for i, r in enumerate(rows):
                    a[:, h0:h0 + hf, r] = part[:, :, i]
    return outs
