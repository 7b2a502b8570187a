"""Causal attention forward/backward for one context-parallel rank, as HIP
kernels for AMD Instinct MI355X (gfx950) behind a small C ABI
(include/cpattn.h).

This module is the Python binding: it turns torch tensors into the C
descriptors (shapes, strides, device pointers, the current HIP stream) and
calls libcpattn.so.  PyTorch only provides device memory and streams; every
step of the computation runs in the library's kernels.  Entry points keep
the C names: attn_fwd, attn_bwd, attn_merge_lse, pack_saved, unpack_saved.

Tensor layouts
  BSHD: q [B, Sq, Hq, Dqk], k [B, Sk, Hkv, Dqk], v [B, Sk, Hkv, Dv],
        o/do [B, Sq, Hq, Dv], lse [B, Hq, Sq] (fp32)
  THD : q [Tq, Hq, Dqk], ..., lse [Hq, Tq]; sequence n occupies physical
        rows [cu_seqlens[n], cu_seqlens[n+1]) of which the first
        seqused[n] are real (TransformerEngine PR 3149, "Enable FA4 for
        context-parallel attention", Description).
"""
from __future__ import annotations

import ctypes
import dataclasses
import math
from typing import Optional, Sequence, Tuple

import torch

from . import _lib
from ._lib import (CPA_BF16, CPA_FP16, CPA_FP32, CPA_FLAG_DETERMINISTIC,  # noqa: F401
                   CPA_FLAG_DQ_DIRECT, CpaError, MergeDesc, PackDesc, Problem, STATUS_CODE)

__all__ = [
    "attn_fwd", "attn_bwd", "attn_bwd_static", "bwd_workspace_bytes", "attn_merge_lse", "pack_saved", "unpack_saved",
    "pack_saved_size", "Varlen", "CpaError", "forward", "backward",
    "workspace_error_flag", "library",
]


def library():
    """The loaded libcpattn (raises if it has not been built)."""
    return _lib.load()


@dataclasses.dataclass
class Varlen:
    """Packed-THD metadata (device int32 tensors, host max lengths)."""
    cu_seqlens_q: torch.Tensor
    cu_seqlens_k: torch.Tensor
    seqused_q: torch.Tensor
    seqused_k: torch.Tensor
    max_seqlen_q: int
    max_seqlen_k: int
    bottom_right: bool = False


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return CPA_BF16
    if t.dtype == torch.float32:
        return CPA_FP32
    if t.dtype == torch.float16:
        return CPA_FP16
    raise TypeError(f"unsupported dtype {t.dtype} (bf16, fp16 or fp32)")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream_handle(stream) -> ctypes.c_void_p:
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _strides3(t: torch.Tensor, thd: bool):
    if t is None:
        return (0, 0, 0)
    st = t.stride()
    if st[-1] != 1:
        raise ValueError("the head dim must be contiguous")
    return (0, st[0], st[1]) if thd else (st[0], st[1], st[2])


# ------------------------------------------------------------- validation
#
# The C ABI sees pointers and sizes only, so it cannot tell a tensor of the
# wrong shape or dtype, or a host pointer, from a good one.  Every entry point
# below checks its tensors against the problem before calling the library
# (the pages' validation of dtypes, shapes and LSE before dispatch: PR 3527
# "cuDNN FROST attention backend for head_dim in (256, 512]", commit notes on
# input validation).  Shapes and dtypes are checked first, devices last.

def _need(cond, msg, exc=ValueError):
    if not cond:
        raise exc(msg)


def _shape(t, name, shape):
    _need(isinstance(t, torch.Tensor), f"{name}: expected a tensor", TypeError)
    _need(tuple(t.shape) == tuple(int(x) for x in shape),
          f"{name}: shape {tuple(t.shape)}, expected {tuple(int(x) for x in shape)}")


def _dtype(t, name, dtypes):
    dtypes = dtypes if isinstance(dtypes, tuple) else (dtypes,)
    _need(t.dtype in dtypes, f"{name}: dtype {t.dtype}, expected {' or '.join(map(str, dtypes))}",
          TypeError)


def _same_device(named, ref):
    """Every tensor on ``ref``'s device, which must be a GPU."""
    _need(ref.is_cuda, f"tensors must be on a GPU (got {ref.device})")
    for name, t in named:
        if t is not None:
            _need(t.is_cuda and t.device == ref.device,
                  f"{name} is on {t.device}, expected {ref.device}")


def _check_qkv(q, k, v, varlen):
    thd = q.dim() == 3
    _need(q.dim() in (3, 4), "q must be [B, S, H, D] or [T, H, D]")
    _dtype(q, "q", (torch.bfloat16, torch.float16, torch.float32))
    _need(k.dim() == q.dim() and v.dim() == q.dim(), "q, k, v must have the same layout")
    _dtype(k, "k", q.dtype)
    _dtype(v, "v", q.dtype)
    if thd:
        _shape(v, "v", (k.shape[0], k.shape[1], v.shape[-1]))
        _shape(k, "k", (k.shape[0], k.shape[1], q.shape[-1]))
    else:
        _shape(k, "k", (q.shape[0], k.shape[1], k.shape[2], q.shape[-1]))
        _shape(v, "v", (q.shape[0], k.shape[1], k.shape[2], v.shape[-1]))
    if varlen is not None:
        n = varlen.seqused_q.numel()
        for name in ("cu_seqlens_q", "cu_seqlens_k", "seqused_q", "seqused_k"):
            t = getattr(varlen, name)
            _dtype(t, f"varlen.{name}", torch.int32)
            _need(t.dim() == 1 and t.is_contiguous(), f"varlen.{name} must be 1-D contiguous")
        _shape(varlen.seqused_k, "varlen.seqused_k", (n,))
        _shape(varlen.cu_seqlens_q, "varlen.cu_seqlens_q", (n + 1,))
        _shape(varlen.cu_seqlens_k, "varlen.cu_seqlens_k", (n + 1,))


def _varlen_tensors(varlen):
    if varlen is None:
        return []
    return [(f"varlen.{n}", getattr(varlen, n))
            for n in ("cu_seqlens_q", "cu_seqlens_k", "seqused_q", "seqused_k")]


def _lse_expected(q, thd):
    return (q.shape[1], q.shape[0]) if thd else (q.shape[0], q.shape[2], q.shape[1])


def _check_workspace(ws, q):
    if ws is not None:
        _dtype(ws, "workspace", torch.uint8)
        _need(ws.dim() == 1 and ws.is_contiguous(), "workspace must be 1-D contiguous")


def _fill_problem(q, k, v, *, causal, scale, out_dtype, q_segments, k_pos_begin,
                  varlen: Optional[Varlen], window=None) -> Problem:
    p = Problem()
    thd = q.dim() == 3
    if thd != (varlen is not None):
        raise ValueError("3-D (THD) tensors need varlen metadata, 4-D (BSHD) must not have it")
    _check_qkv(q, k, v, varlen)
    p.layout = 1 if thd else 0
    p.in_dtype = _dtype_code(q)
    p.out_dtype = out_dtype
    if thd:
        p.batch = 1
        p.seqlen_q, p.heads_q, p.d_qk = q.shape
        p.seqlen_k, p.heads_kv = k.shape[0], k.shape[1]
        p.num_seqs = varlen.seqused_q.numel()
        p.max_seqlen_q = int(varlen.max_seqlen_q)
        p.max_seqlen_k = int(varlen.max_seqlen_k)
        p.cu_seqlens_q = varlen.cu_seqlens_q.data_ptr()
        p.cu_seqlens_k = varlen.cu_seqlens_k.data_ptr()
        p.seqused_q = varlen.seqused_q.data_ptr()
        p.seqused_k = varlen.seqused_k.data_ptr()
        p.thd_bottom_right = int(bool(varlen.bottom_right))
    else:
        p.batch, p.seqlen_q, p.heads_q, p.d_qk = q.shape
        p.seqlen_k, p.heads_kv = k.shape[1], k.shape[2]
    p.d_v = v.shape[-1]
    p.q_stride = _strides3(q, thd)
    p.k_stride = _strides3(k, thd)
    p.v_stride = _strides3(v, thd)
    p.softmax_scale = float(1.0 / math.sqrt(p.d_qk) if scale is None else scale)
    p.causal = int(bool(causal))
    segs = list(q_segments or [])
    if len(segs) > _lib.CPA_MAX_SEGMENTS:
        raise ValueError("at most 8 query segments")
    p.num_q_segments = len(segs)
    for i, (r, pos) in enumerate(segs):
        p.q_seg_row[i] = int(r)
        p.q_seg_pos[i] = int(pos)
    p.k_pos_begin = int(k_pos_begin)
    if window is not None:
        p.window = 1
        p.window_left, p.window_right = (int(w) for w in window)
    return p


def _lse_strides(lse: torch.Tensor, thd: bool):
    st = lse.stride()
    if st[-1] != 1:
        raise ValueError("LSE rows must be contiguous")
    return (0, st[0]) if thd else (st[0], st[1])


def workspace_error_flag(ws: torch.Tensor) -> int:
    """The device metadata error flag (first int32 of a workspace); syncs."""
    return int(ws[:4].view(torch.int32).item())


def attn_fwd(q, k, v, o, lse, *, causal=True, scale=None, q_segments=None, k_pos_begin=0,
             varlen: Optional[Varlen] = None, workspace=None, stream=None,
             window=None, acc=None) -> torch.Tensor:
    """Forward into preallocated o (bf16 or fp32) and lse (fp32).

    q_segments: BSHD query positions as [(row_begin, pos_begin), ...]
    (default: one segment at 0, top-left causal); k_pos_begin: position of
    key row 0; window: (left, right) sliding window / band, -1 = unbounded
    on that side (None: no window).  acc = (o_acc, lse_acc): fp32 running
    accumulator laid out like (o, lse); the result is merged into it by LSE
    (attn_fwd_accum; o, lse may be o_acc, lse_acc themselves).  Returns the
    workspace (its first int32 is the THD metadata error flag).
    """
    p = _fill_problem(q, k, v, causal=causal, scale=scale, out_dtype=_dtype_code(o),
                      q_segments=q_segments, k_pos_begin=k_pos_begin, varlen=varlen,
                      window=window)
    thd = p.layout == 1
    _shape(o, "o", (*q.shape[:-1], v.shape[-1]))
    _shape(lse, "lse", _lse_expected(q, thd))
    _dtype(lse, "lse", torch.float32)
    _check_workspace(workspace, q)
    if acc is not None:
        _need(len(acc) == 2, "acc = (o_acc, lse_acc)")
        _shape(acc[0], "o_acc", o.shape)
        _shape(acc[1], "lse_acc", lse.shape)
    _same_device([("k", k), ("v", v), ("o", o), ("lse", lse), ("workspace", workspace),
                  *(("acc", t) for t in (acc or ())), *_varlen_tensors(varlen)], q)
    lib = _lib.load()
    p.o_stride = _strides3(o, thd)
    p.lse_stride = _lse_strides(lse, thd)
    need = lib.attn_fwd_workspace_size(ctypes.byref(p))
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    if acc is None:
        st = lib.attn_fwd(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                          _ptr(workspace), workspace.numel(), _stream_handle(stream))
        _lib.check(st, "attn_fwd")
    else:
        o_acc, lse_acc = acc
        if o_acc.dtype != torch.float32 or lse_acc.dtype != torch.float32:
            raise ValueError("the accumulator is fp32")
        if (o_acc.shape != o.shape or o_acc.stride() != o.stride() or
                lse_acc.shape != lse.shape or lse_acc.stride() != lse.stride()):
            raise ValueError("the accumulator must have the layout of o and lse")
        st = lib.attn_fwd_accum(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(o_acc),
                                _ptr(lse_acc), _ptr(o), _ptr(lse), _ptr(workspace),
                                workspace.numel(), _stream_handle(stream))
        _lib.check(st, "attn_fwd_accum")
    return workspace


def attn_bwd(q, k, v, o, dout, lse, dq, dk, dv, *, causal=True, scale=None, q_segments=None,
             k_pos_begin=0, varlen: Optional[Varlen] = None, workspace=None, flags=0,
             stream=None, step: str = "attn_bwd", window=None) -> torch.Tensor:
    """Backward into preallocated dq, dk, dv.  Returns the workspace.

    ``step`` selects the C entry point: "attn_bwd" (all four steps), or one
    of "attn_bwd_pre", "attn_bwd_main", "attn_bwd_dq", "attn_bwd_post".
    ``flags``: CPA_FLAG_DETERMINISTIC (always honoured), CPA_FLAG_DQ_DIRECT
    (given to all four steps of a backward that runs main and dq once over
    every key block: the dq step writes dq itself; "attn_bwd" with the full
    workspace does so without the flag)."""
    if step not in ("attn_bwd", "attn_bwd_pre", "attn_bwd_main", "attn_bwd_dq", "attn_bwd_post"):
        raise ValueError(step)
    if o.dtype != q.dtype or dout.dtype != q.dtype:
        raise TypeError("o and dout must have q's dtype")
    p = _fill_problem(q, k, v, causal=causal, scale=scale, out_dtype=_dtype_code(dq),
                      q_segments=q_segments, k_pos_begin=k_pos_begin, varlen=varlen,
                      window=window)
    thd = p.layout == 1
    ov = (*q.shape[:-1], v.shape[-1])
    _shape(o, "o", ov)
    _shape(dout, "dout", ov)
    _shape(lse, "lse", _lse_expected(q, thd))
    _dtype(lse, "lse", torch.float32)
    _shape(dq, "dq", q.shape)
    _shape(dk, "dk", k.shape)
    _shape(dv, "dv", v.shape)
    _dtype(dk, "dk", dq.dtype)
    _dtype(dv, "dv", dq.dtype)
    _check_workspace(workspace, q)
    _same_device([("k", k), ("v", v), ("o", o), ("dout", dout), ("lse", lse), ("dq", dq),
                  ("dk", dk), ("dv", dv), ("workspace", workspace),
                  *_varlen_tensors(varlen)], q)
    lib = _lib.load()
    p.o_stride = _strides3(o, thd)
    p.do_stride = _strides3(dout, thd)
    p.dq_stride = _strides3(dq, thd)
    p.dk_stride = _strides3(dk, thd)
    p.dv_stride = _strides3(dv, thd)
    p.lse_stride = _lse_strides(lse, thd)
    need = lib.attn_bwd_workspace_size(ctypes.byref(p))
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    fn = getattr(lib, step)
    st = fn(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(dq),
            _ptr(dk), _ptr(dv), _ptr(workspace), workspace.numel(), int(flags),
            _stream_handle(stream))
    _lib.check(st, step)
    return workspace


def attn_bwd_static(q, k, v, o, dout, lse, dq, dk, dv, *, err_flag=None, causal=True,
                    scale=None, q_segments=None, k_pos_begin=0,
                    varlen: Optional[Varlen] = None, flags=0, stream=None, window=None):
    """Backward into preallocated dq, dk, dv with the library's fixed
    per-GPU workspace (attn_bwd_static): no allocation.  ``err_flag``: a
    device int32 tensor of one element for the THD metadata flag (required
    for THD)."""
    if o.dtype != q.dtype or dout.dtype != q.dtype:
        raise TypeError("o and dout must have q's dtype")
    p = _fill_problem(q, k, v, causal=causal, scale=scale, out_dtype=_dtype_code(dq),
                      q_segments=q_segments, k_pos_begin=k_pos_begin, varlen=varlen,
                      window=window)
    thd = p.layout == 1
    ov = (*q.shape[:-1], v.shape[-1])
    _shape(o, "o", ov)
    _shape(dout, "dout", ov)
    _shape(lse, "lse", _lse_expected(q, thd))
    _dtype(lse, "lse", torch.float32)
    _shape(dq, "dq", q.shape)
    _shape(dk, "dk", k.shape)
    _shape(dv, "dv", v.shape)
    _dtype(dk, "dk", dq.dtype)
    _dtype(dv, "dv", dq.dtype)
    if err_flag is not None:
        _dtype(err_flag, "err_flag", torch.int32)
        _need(err_flag.numel() >= 1, "err_flag needs one element")
    _same_device([("k", k), ("v", v), ("o", o), ("dout", dout), ("lse", lse), ("dq", dq),
                  ("dk", dk), ("dv", dv), ("err_flag", err_flag), *_varlen_tensors(varlen)], q)
    lib = _lib.load()
    p.o_stride = _strides3(o, thd)
    p.do_stride = _strides3(dout, thd)
    p.dq_stride = _strides3(dq, thd)
    p.dk_stride = _strides3(dk, thd)
    p.dv_stride = _strides3(dv, thd)
    p.lse_stride = _lse_strides(lse, thd)
    st = lib.attn_bwd_static(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout),
                             _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(err_flag), int(flags),
                             _stream_handle(stream))
    _lib.check(st, "attn_bwd_static")


def bwd_workspace_bytes(q, k, v, *, varlen=None, minimum=False, **kw) -> int:
    """attn_bwd_workspace_size (or, with ``minimum``, attn_bwd_workspace_min)."""
    p = _fill_problem(q, k, v, causal=True, scale=None, out_dtype=0, q_segments=None,
                      k_pos_begin=0, varlen=varlen)
    lib = _lib.load()
    fn = lib.attn_bwd_workspace_min if minimum else lib.attn_bwd_workspace_size
    return int(fn(ctypes.byref(p)))


def _as4(o: torch.Tensor, lse: torch.Tensor):
    """Merge/pack tensors as [B, S, H, D] and LSE as [B, H, S]."""
    if o.dim() == 3:
        o = o.unsqueeze(0)
        lse = lse.unsqueeze(0)
    return o, lse


def attn_merge_lse(o_acc, lse_acc, o_part, lse_part, o_out=None, lse_out=None, *, stream=None):
    """(o_out, lse_out) = LSE merge of (o_acc, lse_acc) and (o_part,
    lse_part).  Defaults to in place on the accumulator.  O tensors are
    [B, S, H, D] or [S, H, D]; LSE [B, H, S] or [H, S]."""
    if o_out is None:
        o_out = o_acc
    if lse_out is None:
        lse_out = lse_acc
    _need(o_acc.dim() in (3, 4), "O tensors are [B, S, H, D] or [S, H, D]")
    for name, t in (("o_part", o_part), ("o_out", o_out)):
        _shape(t, name, o_acc.shape)
    lshape = (o_acc.shape[:-3] + (o_acc.shape[-2], o_acc.shape[-3]))
    for name, t in (("lse_acc", lse_acc), ("lse_part", lse_part), ("lse_out", lse_out)):
        _shape(t, name, lshape)
        _dtype(t, name, torch.float32)
    _same_device([("lse_acc", lse_acc), ("o_part", o_part), ("lse_part", lse_part),
                  ("o_out", o_out), ("lse_out", lse_out)], o_acc)
    lib = _lib.load()
    a4, la = _as4(o_acc, lse_acc)
    p4, lp = _as4(o_part, lse_part)
    o4, lo = _as4(o_out, lse_out)
    d = MergeDesc()
    d.batch, d.seqlen, d.heads, d.d_v = a4.shape
    d.acc_dtype, d.part_dtype, d.out_dtype = _dtype_code(a4), _dtype_code(p4), _dtype_code(o4)
    for name, t in (("acc_stride", a4), ("part_stride", p4), ("out_stride", o4)):
        if t.stride(-1) != 1:
            raise ValueError("last dim must be contiguous")
        setattr(d, name, tuple(t.stride()[:3]))
    for name, t in (("lse_acc_stride", la), ("lse_part_stride", lp), ("lse_out_stride", lo)):
        if t.stride(-1) != 1:
            raise ValueError("LSE rows must be contiguous")
        setattr(d, name, tuple(t.stride()[:2]))
    st = lib.attn_merge_lse(ctypes.byref(d), _ptr(a4), _ptr(la), _ptr(p4), _ptr(lp), _ptr(o4),
                            _ptr(lo), _stream_handle(stream))
    _lib.check(st, "attn_merge_lse")
    return o_out, lse_out


def _pack_desc(o, lse, groups, force_int64):
    _need(o.dim() in (3, 4), "o is [B, S, H, D] or [S, H, D]")
    _shape(lse, "lse", o.shape[:-3] + (o.shape[-2], o.shape[-3]))
    _dtype(lse, "lse", torch.float32)
    o4, l3 = _as4(o, lse)
    d = PackDesc()
    d.batch, d.seqlen, d.heads, d.d_v = o4.shape
    d.o_dtype = _dtype_code(o4)
    d.groups = int(groups)
    if o4.stride(-1) != 1 or l3.stride(-1) != 1:
        raise ValueError("last dims must be contiguous")
    d.o_stride = tuple(o4.stride()[:3])
    d.lse_stride = tuple(l3.stride()[:2])
    d.force_int64 = int(bool(force_int64))
    return d, o4, l3


def pack_saved_size(o, lse, groups) -> int:
    d, _, _ = _pack_desc(o, lse, groups, False)
    return int(_lib.load().pack_saved_size(ctypes.byref(d)))


def pack_saved(o, lse, groups, buf=None, *, force_int64=False, stream=None) -> torch.Tensor:
    """Pack O and the raw fp32 LSE into per-head-group segments; returns the
    uint8 buffer."""
    d, o4, l3 = _pack_desc(o, lse, groups, force_int64)
    if buf is not None:
        _dtype(buf, "buf", torch.uint8)
        _need(buf.dim() == 1 and buf.is_contiguous(), "buf must be 1-D contiguous")
    _same_device([("lse", lse), ("buf", buf)], o)
    lib = _lib.load()
    need = lib.pack_saved_size(ctypes.byref(d))
    if buf is None:
        buf = torch.empty(need, dtype=torch.uint8, device=o.device)
    st = lib.pack_saved(ctypes.byref(d), _ptr(o4), _ptr(l3), _ptr(buf), buf.numel(),
                        _stream_handle(stream))
    _lib.check(st, "pack_saved")
    return buf


def unpack_saved(buf, o, lse, groups, *, force_int64=False, stream=None):
    """Inverse of pack_saved, into preallocated o and lse."""
    d, o4, l3 = _pack_desc(o, lse, groups, force_int64)
    _dtype(buf, "buf", torch.uint8)
    _need(buf.dim() == 1 and buf.is_contiguous(), "buf must be 1-D contiguous")
    _same_device([("lse", lse), ("buf", buf)], o)
    lib = _lib.load()
    st = lib.unpack_saved(ctypes.byref(d), _ptr(buf), buf.numel(), _ptr(o4), _ptr(l3),
                          _stream_handle(stream))
    _lib.check(st, "unpack_saved")
    return o, lse


def xchg_desc(tensors, *, groups, ranges, split):
    """Exchange-buffer description (include/cpattn.h, cpa_xchg_desc).

    tensors: row tensors [B, R, H, D] (bf16 or fp32, moved as raw bits) and
    LSE tensors [B, H, R] (fp32), in buffer order; ranges: per segment a list
    of (row_begin, count); split: one bool for all fields or one per field
    (True: heads split over the segments)."""
    if not tensors or len(tensors) > _lib.CPA_XCHG_MAX_FIELDS:
        raise ValueError("1..8 tensors")
    if len(ranges) != groups or groups > _lib.CPA_XCHG_MAX_GROUPS:
        raise ValueError("one range list per segment, at most 8 segments")
    splits = list(split) if isinstance(split, (list, tuple)) else [split] * len(tensors)
    d = _lib.XchgDesc()
    d.groups, d.nfields = int(groups), len(tensors)
    rows = None
    for f, (x, sp) in enumerate(zip(tensors, splits)):
        fd = d.field[f]
        if x.stride(-1) != 1:
            raise ValueError("last dim must be contiguous")
        if x.dim() == 4:
            b, r, h, dim = x.shape
            fd.kind, fd.elem_bytes, fd.heads, fd.dim = (_lib.CPA_XCHG_ROWS, x.element_size(),
                                                        h, dim)
            fd.stride = tuple(x.stride()[:3])
        elif x.dim() == 3 and x.dtype == torch.float32:
            b, h, r = x.shape
            fd.kind, fd.elem_bytes, fd.heads, fd.dim = _lib.CPA_XCHG_LSE, 4, h, 1
            fd.stride = (x.stride(0), x.stride(1), 0)
        else:
            raise ValueError("row tensors are [B, R, H, D], LSE tensors fp32 [B, H, R]")
        fd.split = int(bool(sp))
        if rows is None:
            d.batch, rows = b, r
        elif (b, r) != (d.batch, rows):
            raise ValueError("all tensors need the same batch and rows")
    d.rows = rows
    for g, rg in enumerate(ranges):
        if len(rg) > _lib.CPA_XCHG_MAX_RANGES:
            raise ValueError("at most 4 ranges per segment")
        d.nranges[g] = len(rg)
        for i, (r0, n) in enumerate(rg):
            d.range_row[g][i], d.range_len[g][i] = int(r0), int(n)
    return d


def xchg_offsets(d) -> list:
    """Segment byte offsets [groups + 1] (the last is the buffer size)."""
    lib = _lib.load()
    offs = [int(lib.xchg_segment_offset(ctypes.byref(d), g)) for g in range(d.groups + 1)]
    if offs[-1] == 0 and d.rows > 0:
        raise ValueError("invalid exchange description")
    return offs


def _ptr_array(tensors):
    return (ctypes.c_void_p * len(tensors))(*[t.data_ptr() for t in tensors])


def xchg_pack(tensors, *, groups, ranges, split, buf=None, stream=None) -> torch.Tensor:
    """Pack every segment of ``tensors`` into one uint8 buffer (returned)."""
    d = xchg_desc(tensors, groups=groups, ranges=ranges, split=split)
    if buf is not None:
        _dtype(buf, "buf", torch.uint8)
        _need(buf.dim() == 1 and buf.is_contiguous(), "buf must be 1-D contiguous")
    _same_device([(f"tensors[{i}]", t) for i, t in enumerate(tensors)] + [("buf", buf)],
                 tensors[0])
    lib = _lib.load()
    need = xchg_offsets(d)[-1]
    if buf is None:
        buf = torch.empty(need, dtype=torch.uint8, device=tensors[0].device)
    st = lib.xchg_pack(ctypes.byref(d), _ptr_array(tensors), _ptr(buf), buf.numel(),
                       _stream_handle(stream))
    _lib.check(st, "xchg_pack")
    return buf


def xchg_unpack(buf, tensors, *, groups, ranges, split, stream=None):
    """Unpack a (received) buffer into ``tensors`` in place."""
    d = xchg_desc(tensors, groups=groups, ranges=ranges, split=split)
    _dtype(buf, "buf", torch.uint8)
    _need(buf.dim() == 1 and buf.is_contiguous(), "buf must be 1-D contiguous")
    _same_device([(f"tensors[{i}]", t) for i, t in enumerate(tensors)] + [("buf", buf)],
                 tensors[0])
    lib = _lib.load()
    st = lib.xchg_unpack(ctypes.byref(d), _ptr(buf), buf.numel(), _ptr_array(tensors),
                         _stream_handle(stream))
    _lib.check(st, "xchg_unpack")
    return tensors


# ------------------------------------------------------------- allocating

def _lse_shape(q, thd):
    return (q.shape[1], q.shape[0]) if thd else (q.shape[0], q.shape[2], q.shape[1])


def forward(q, k, v, *, out_dtype=None, causal=True, scale=None, q_segments=None,
            k_pos_begin=0, varlen=None, stream=None,
            window=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Allocate o, lse and run attn_fwd.  THD padding rows of the returned
    tensors are uninitialised (the kernels never write them)."""
    thd = q.dim() == 3
    o = torch.empty(*q.shape[:-1], v.shape[-1], dtype=out_dtype or q.dtype, device=q.device)
    lse = torch.empty(*_lse_shape(q, thd), dtype=torch.float32, device=q.device)
    attn_fwd(q, k, v, o, lse, causal=causal, scale=scale, q_segments=q_segments,
             k_pos_begin=k_pos_begin, varlen=varlen, stream=stream, window=window)
    return o, lse


def backward(q, k, v, o, dout, lse, *, out_dtype=None, causal=True, scale=None,
             q_segments=None, k_pos_begin=0, varlen=None, stream=None, window=None):
    """Allocate dq, dk, dv and run attn_bwd."""
    dt = out_dtype or q.dtype
    dq = torch.empty(q.shape, dtype=dt, device=q.device)
    dk = torch.empty(k.shape, dtype=dt, device=q.device)
    dv = torch.empty(v.shape, dtype=dt, device=q.device)
    attn_bwd(q, k, v, o, dout, lse, dq, dk, dv, causal=causal, scale=scale,
             q_segments=q_segments, k_pos_begin=k_pos_begin, varlen=varlen, stream=stream,
             window=window)
    return dq, dk, dv
