"""Byte-exact pack/unpack of the saved forward outputs (O and fp32 LSE).

Test infrastructure only (see the package docstring).

PR 3510 ("Add head-parallel FA4 backward for cuDNN CP attention",
Description and Diagram) packs the saved attention tensors of each sequence
partition into one buffer for a single sequence-to-heads all-to-all; the
packing keeps the FP32 log-sum-exp bits and the receiver unpacks into the
send allocation.  The pages give no byte layout, so the layout below is this
library's own convention (any layout is correct if the round trip is exact):

The H heads are cut into G groups of Hg = H / G consecutive heads; group g
is the segment sent to destination g.  Segment g holds, in order:

* O of heads [g*Hg, (g+1)*Hg): element (b, s, hh, d) at
  ((b*S + s)*Hg + hh)*Dv + d, in O's own element type (raw bits);
* at the next multiple of 256 bytes, LSE of the same heads: element
  (b, hh, s) at (b*Hg + hh)*S + s, raw fp32 bits.

Each segment is padded to a multiple of 256 bytes; segment g starts at
g * segment_bytes.  Pad bytes are never read by unpack.
"""
from __future__ import annotations

import numpy as np


def _align(x, a=256):
    return (x + a - 1) // a * a


def pack_layout(batch, seqlen, heads, d_v, o_elem_bytes, groups):
    """Return (segment_bytes, o_bytes_per_segment, lse_offset_in_segment)."""
    assert heads % groups == 0
    hg = heads // groups
    o_bytes = batch * seqlen * hg * d_v * o_elem_bytes
    lse_off = _align(o_bytes)
    seg = _align(lse_off + batch * hg * seqlen * 4)
    return seg, o_bytes, lse_off


def _bits(a, nbytes):
    a = np.ascontiguousarray(a)
    return a.view(np.uint16 if nbytes == 2 else np.uint32)


def pack_saved(o, lse, groups):
    """o: [B, S, H, Dv] array of 2- or 4-byte elements (bf16 bits as uint16,
    or float32); lse: [B, H, S] float32.  Returns the uint8 buffer."""
    o = np.ascontiguousarray(o)
    lse = np.ascontiguousarray(lse, dtype=np.float32)
    b, s, h, dv = o.shape
    eb = o.dtype.itemsize
    seg, o_bytes, lse_off = pack_layout(b, s, h, dv, eb, groups)
    hg = h // groups
    buf = np.zeros(groups * seg, dtype=np.uint8)
    ob = _bits(o, eb)
    lb = lse.view(np.uint32)
    for g in range(groups):
        base = g * seg
        part = np.ascontiguousarray(ob[:, :, g * hg:(g + 1) * hg, :])
        buf[base:base + o_bytes] = part.view(np.uint8).reshape(-1)
        lpart = np.ascontiguousarray(lb[:, g * hg:(g + 1) * hg, :])
        n = lpart.size * 4
        buf[base + lse_off:base + lse_off + n] = lpart.view(np.uint8).reshape(-1)
    return buf


def unpack_saved(buf, batch, seqlen, heads, d_v, o_dtype, groups):
    """Inverse of pack_saved.  Returns (o [B,S,H,Dv] of o_dtype, lse
    [B,H,S] float32)."""
    o_dtype = np.dtype(o_dtype)
    eb = o_dtype.itemsize
    seg, o_bytes, lse_off = pack_layout(batch, seqlen, heads, d_v, eb, groups)
    hg = heads // groups
    o = np.empty((batch, seqlen, heads, d_v), dtype=o_dtype)
    lse = np.empty((batch, heads, seqlen), dtype=np.float32)
    buf = np.asarray(buf, dtype=np.uint8)
    for g in range(groups):
        base = g * seg
        part = buf[base:base + o_bytes].view(o_dtype).reshape(
            batch, seqlen, hg, d_v)
        o[:, :, g * hg:(g + 1) * hg, :] = part
        n = batch * hg * seqlen * 4
        lpart = buf[base + lse_off:base + lse_off + n].view(
            np.float32).reshape(batch, hg, seqlen)
        lse[:, g * hg:(g + 1) * hg, :] = lpart
    return o, lse
