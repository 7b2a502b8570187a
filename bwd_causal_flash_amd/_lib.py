"""ctypes binding of libcpattn.so: the C structures and raw entry points.

Argument marshalling only; every computation runs in the HIP library.  The
library is loaded from this package directory; if it is missing the import
of the product API fails loudly (there is no fallback path).
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libcpattn.so")

CPA_BF16, CPA_FP32, CPA_FP16 = 0, 1, 2
CPA_LAYOUT_BSHD, CPA_LAYOUT_THD = 0, 1
CPA_MAX_SEGMENTS = 8
CPA_FLAG_DETERMINISTIC = 1
CPA_FLAG_DQ_DIRECT = 2
CPA_BWD_STATIC_WORKSPACE_BYTES = 256 << 20

STATUS = {
    0: "CPA_OK", 1: "CPA_ERR_NULL", 2: "CPA_ERR_SHAPE", 3: "CPA_ERR_DTYPE",
    4: "CPA_ERR_STRIDE", 5: "CPA_ERR_ALIGN", 6: "CPA_ERR_UNSUPPORTED",
    7: "CPA_ERR_WORKSPACE", 8: "CPA_ERR_OVERLAP", 9: "CPA_ERR_LAUNCH",
}
STATUS_CODE = {v: k for k, v in STATUS.items()}

I64x3 = ctypes.c_int64 * 3
I64x2 = ctypes.c_int64 * 2
I64xS = ctypes.c_int64 * CPA_MAX_SEGMENTS


class Problem(ctypes.Structure):
    """Mirror of struct cpa_problem (include/cpattn.h)."""
    _fields_ = [
        ("layout", ctypes.c_int32), ("in_dtype", ctypes.c_int32),
        ("out_dtype", ctypes.c_int32), ("batch", ctypes.c_int32),
        ("heads_q", ctypes.c_int32), ("heads_kv", ctypes.c_int32),
        ("d_qk", ctypes.c_int32), ("d_v", ctypes.c_int32),
        ("seqlen_q", ctypes.c_int64), ("seqlen_k", ctypes.c_int64),
        ("num_seqs", ctypes.c_int32), ("max_seqlen_q", ctypes.c_int32),
        ("max_seqlen_k", ctypes.c_int32),
        ("cu_seqlens_q", ctypes.c_void_p), ("cu_seqlens_k", ctypes.c_void_p),
        ("seqused_q", ctypes.c_void_p), ("seqused_k", ctypes.c_void_p),
        ("q_stride", I64x3), ("k_stride", I64x3), ("v_stride", I64x3),
        ("o_stride", I64x3), ("do_stride", I64x3),
        ("dq_stride", I64x3), ("dk_stride", I64x3), ("dv_stride", I64x3),
        ("lse_stride", I64x2),
        ("softmax_scale", ctypes.c_float), ("causal", ctypes.c_int32),
        ("thd_bottom_right", ctypes.c_int32),
        ("num_q_segments", ctypes.c_int32),
        ("q_seg_row", I64xS), ("q_seg_pos", I64xS),
        ("k_pos_begin", ctypes.c_int64),
        ("window", ctypes.c_int32), ("window_left", ctypes.c_int32),
        ("window_right", ctypes.c_int32),
    ]


class MergeDesc(ctypes.Structure):
    """Mirror of struct cpa_merge_desc."""
    _fields_ = [
        ("batch", ctypes.c_int32), ("heads", ctypes.c_int32),
        ("d_v", ctypes.c_int32), ("seqlen", ctypes.c_int64),
        ("acc_dtype", ctypes.c_int32), ("part_dtype", ctypes.c_int32),
        ("out_dtype", ctypes.c_int32),
        ("acc_stride", I64x3), ("part_stride", I64x3), ("out_stride", I64x3),
        ("lse_acc_stride", I64x2), ("lse_part_stride", I64x2),
        ("lse_out_stride", I64x2),
    ]


class PackDesc(ctypes.Structure):
    """Mirror of struct cpa_pack_desc."""
    _fields_ = [
        ("batch", ctypes.c_int32), ("heads", ctypes.c_int32),
        ("d_v", ctypes.c_int32), ("o_dtype", ctypes.c_int32),
        ("groups", ctypes.c_int32), ("seqlen", ctypes.c_int64),
        ("o_stride", I64x3), ("lse_stride", I64x2),
        ("force_int64", ctypes.c_int32),
    ]


CPA_XCHG_MAX_FIELDS, CPA_XCHG_MAX_GROUPS, CPA_XCHG_MAX_RANGES = 8, 8, 4
CPA_XCHG_ROWS, CPA_XCHG_LSE = 0, 1


class XchgField(ctypes.Structure):
    """Mirror of struct cpa_xchg_field."""
    _fields_ = [
        ("kind", ctypes.c_int32), ("elem_bytes", ctypes.c_int32),
        ("heads", ctypes.c_int32), ("dim", ctypes.c_int32), ("split", ctypes.c_int32),
        ("stride", I64x3),
    ]


class XchgDesc(ctypes.Structure):
    """Mirror of struct cpa_xchg_desc."""
    _fields_ = [
        ("batch", ctypes.c_int32), ("groups", ctypes.c_int32), ("nfields", ctypes.c_int32),
        ("rows", ctypes.c_int64),
        ("nranges", ctypes.c_int32 * CPA_XCHG_MAX_GROUPS),
        ("range_row", (ctypes.c_int64 * CPA_XCHG_MAX_RANGES) * CPA_XCHG_MAX_GROUPS),
        ("range_len", (ctypes.c_int64 * CPA_XCHG_MAX_RANGES) * CPA_XCHG_MAX_GROUPS),
        ("field", XchgField * CPA_XCHG_MAX_FIELDS),
    ]


EXPORTS = {
    "attn_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "attn_fwd_workspace_size": (ctypes.c_size_t, [ctypes.POINTER(Problem)]),
    "attn_bwd_workspace_size": (ctypes.c_size_t, [ctypes.POINTER(Problem)]),
    "attn_bwd_workspace_min": (ctypes.c_size_t, [ctypes.POINTER(Problem)]),
    "attn_fwd": (ctypes.c_int, [ctypes.POINTER(Problem)] + [ctypes.c_void_p] * 6 +
                 [ctypes.c_size_t, ctypes.c_void_p]),
    "attn_fwd_accum": (ctypes.c_int, [ctypes.POINTER(Problem)] + [ctypes.c_void_p] * 8 +
                       [ctypes.c_size_t, ctypes.c_void_p]),
    "attn_bwd": (ctypes.c_int, [ctypes.POINTER(Problem)] + [ctypes.c_void_p] * 10 +
                 [ctypes.c_size_t, ctypes.c_uint32, ctypes.c_void_p]),
    "attn_bwd_pre": (ctypes.c_int, [ctypes.POINTER(Problem)] + [ctypes.c_void_p] * 10 +
                     [ctypes.c_size_t, ctypes.c_uint32, ctypes.c_void_p]),
    "attn_bwd_main": (ctypes.c_int, [ctypes.POINTER(Problem)] + [ctypes.c_void_p] * 10 +
                      [ctypes.c_size_t, ctypes.c_uint32, ctypes.c_void_p]),
    "attn_bwd_dq": (ctypes.c_int, [ctypes.POINTER(Problem)] + [ctypes.c_void_p] * 10 +
                      [ctypes.c_size_t, ctypes.c_uint32, ctypes.c_void_p]),
    "attn_bwd_post": (ctypes.c_int, [ctypes.POINTER(Problem)] + [ctypes.c_void_p] * 10 +
                      [ctypes.c_size_t, ctypes.c_uint32, ctypes.c_void_p]),
    "attn_bwd_static": (ctypes.c_int, [ctypes.POINTER(Problem)] + [ctypes.c_void_p] * 10 +
                        [ctypes.c_uint32, ctypes.c_void_p]),
    "attn_merge_lse": (ctypes.c_int, [ctypes.POINTER(MergeDesc)] + [ctypes.c_void_p] * 7),
    "pack_saved_size": (ctypes.c_size_t, [ctypes.POINTER(PackDesc)]),
    "pack_saved": (ctypes.c_int, [ctypes.POINTER(PackDesc), ctypes.c_void_p, ctypes.c_void_p,
                                  ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "unpack_saved": (ctypes.c_int, [ctypes.POINTER(PackDesc), ctypes.c_void_p, ctypes.c_size_t,
                                    ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]),
    "xchg_segment_offset": (ctypes.c_size_t, [ctypes.POINTER(XchgDesc), ctypes.c_int32]),
    "xchg_pack": (ctypes.c_int, [ctypes.POINTER(XchgDesc), ctypes.POINTER(ctypes.c_void_p),
                                 ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "xchg_unpack": (ctypes.c_int, [ctypes.POINTER(XchgDesc), ctypes.c_void_p, ctypes.c_size_t,
                                   ctypes.POINTER(ctypes.c_void_p), ctypes.c_void_p]),
}

_lib = None


def load(path: str = LIB_PATH):
    """Load libcpattn.so once and declare every export's signature."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with `python -m bwd_causal_flash_amd.build` "
            "(there is no non-HIP fallback)")
    lib = ctypes.CDLL(path)
    for name, (res, args) in EXPORTS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


class CpaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        self.name = STATUS.get(status, str(status))
        super().__init__(f"{where}: {self.name}")


def check(status: int, where: str):
    if status != 0:
        raise CpaError(status, where)
