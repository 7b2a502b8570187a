"""Validation cases for the C ABI, run in a child process with no GPU
visible (HIP_VISIBLE_DEVICES=-1): every case must be rejected by host
validation before anything is enqueued; a case that slipped through would
only reach a launch error, never a device.  Prints one JSON object mapping
case name -> [expected status name, returned status name].
"""
import ctypes
import json
import os
import sys

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))

from bwd_causal_flash_amd import _lib  # noqa: E402

A = 1 << 20   # fake, 16-byte aligned device addresses (never dereferenced)


def good_problem(d_qk=128, d_v=128):
    p = _lib.Problem()
    p.layout, p.in_dtype, p.out_dtype = 0, 0, 0
    p.batch, p.heads_q, p.heads_kv, p.d_qk, p.d_v = 1, 4, 2, d_qk, d_v
    p.seqlen_q = p.seqlen_k = 256
    for name, d in (("q_stride", d_qk), ("k_stride", d_qk), ("v_stride", d_v),
                    ("o_stride", d_v), ("do_stride", d_v), ("dq_stride", d_qk),
                    ("dk_stride", d_qk), ("dv_stride", d_v)):
        h = 4 if name[0] in "qod" and name not in ("dk_stride", "dv_stride") else 2
        setattr(p, name, (256 * h * d, h * d, d))
    p.lse_stride = (4 * 256, 256)
    p.softmax_scale = 0.1
    p.causal = 1
    return p


def main():
    lib = _lib.load()
    out = {}
    ptr = lambda i: ctypes.c_void_p(A * (i + 1))  # disjoint 1 MiB-apart fakes

    def fwd(p, q=1, k=2, v=3, o=40, l=60, ws=80, wsb=256):
        args = [None if x is None else ptr(x) for x in (q, k, v, o, l, ws)]
        return lib.attn_fwd(ctypes.byref(p), *args[:5], args[5], wsb, None)

    def case(name, expect, status):
        out[name] = [expect, _lib.STATUS.get(status, str(status))]

    p = good_problem()
    case("null_q", "CPA_ERR_NULL", fwd(p, q=None))
    case("null_problem", "CPA_ERR_NULL",
         lib.attn_fwd(None, ptr(1), ptr(2), ptr(3), ptr(4), ptr(5), ptr(6), 256, None))
    p = good_problem(); p.in_dtype = 7
    case("bad_dtype", "CPA_ERR_DTYPE", fwd(p))
    p = good_problem(); p.in_dtype, p.out_dtype = 2, 0
    case("fp16_in_bf16_out_declined", "CPA_ERR_UNSUPPORTED", fwd(p))
    p = good_problem(); p.in_dtype, p.out_dtype = 0, 2
    case("bf16_in_fp16_out_declined", "CPA_ERR_UNSUPPORTED", fwd(p))
    p = good_problem(); p.heads_q = 3
    case("gqa_not_divisible", "CPA_ERR_SHAPE", fwd(p))
    p = good_problem(d_qk=96, d_v=96)
    case("head_dim_96_declined", "CPA_ERR_UNSUPPORTED", fwd(p))
    p = good_problem(d_qk=260, d_v=260)
    case("head_dim_not_multiple_of_8", "CPA_ERR_UNSUPPORTED", fwd(p))
    p = good_problem(d_qk=128, d_v=64)
    case("head_dims_pair_declined", "CPA_ERR_UNSUPPORTED", fwd(p))
    p = good_problem(); p.k_stride = (256 * 2 * 128, 2 * 128 + 4, 128)
    case("stride_not_multiple_of_8", "CPA_ERR_STRIDE", fwd(p))
    p = good_problem()
    case("misaligned_q", "CPA_ERR_ALIGN",
         lib.attn_fwd(ctypes.byref(p), ctypes.c_void_p(A + 8), ptr(2), ptr(3), ptr(40),
                      ptr(60), ptr(80), 256, None))
    p = good_problem()
    case("workspace_small", "CPA_ERR_WORKSPACE", fwd(p, wsb=16))
    case("workspace_null", "CPA_ERR_WORKSPACE", fwd(p, ws=None))
    p = good_problem()
    case("output_overlaps_input", "CPA_ERR_OVERLAP", fwd(p, o=1))
    p = good_problem(); p.num_q_segments = 2; p.q_seg_row[0] = 0; p.q_seg_row[1] = 0
    case("segments_not_increasing", "CPA_ERR_SHAPE", fwd(p))
    p = good_problem(); p.num_q_segments = 9
    case("too_many_segments", "CPA_ERR_SHAPE", fwd(p))
    p = good_problem(); p.softmax_scale = float("nan")
    case("nan_scale", "CPA_ERR_SHAPE", fwd(p))
    p = good_problem(); p.softmax_scale = -0.1
    case("negative_scale_declined", "CPA_ERR_UNSUPPORTED", fwd(p))
    p = good_problem(); p.layout = 1; p.num_seqs = 2
    case("thd_missing_metadata", "CPA_ERR_NULL", fwd(p))
    p = good_problem(); p.seqlen_q = 1 << 31
    case("seqlen_too_large", "CPA_ERR_SHAPE", fwd(p))
    p = good_problem(); p.window = 2
    case("window_flag_not_0_or_1", "CPA_ERR_SHAPE", fwd(p))
    p = good_problem(); p.window = 1; p.window_left = -2
    case("window_left_below_minus_1", "CPA_ERR_SHAPE", fwd(p))
    p = good_problem(); p.window = 1; p.window_right = 1 << 30
    case("window_right_too_large", "CPA_ERR_SHAPE", fwd(p))
    p = good_problem(); p.window = 1; p.window_left = 100; p.window_right = -1
    case("window_valid_reaches_launch", "CPA_ERR_LAUNCH", fwd(p))

    def acc_fwd(p, oa=100, la=120, o=40, l=60, ws=80, wsb=256):
        a = [None if x is None else ptr(x) for x in (oa, la, o, l, ws)]
        return lib.attn_fwd_accum(ctypes.byref(p), ptr(1), ptr(2), ptr(3), *a, wsb, None)

    p = good_problem()
    case("accum_null_o_acc", "CPA_ERR_NULL", acc_fwd(p, oa=None))
    case("accum_null_lse_acc", "CPA_ERR_NULL", acc_fwd(p, la=None))
    # o_acc is fp32: the same pointer as a bf16 o is an overlap, not in place
    case("accum_o_acc_is_bf16_o", "CPA_ERR_OVERLAP", acc_fwd(p, oa=40))
    case("accum_o_acc_overlaps_workspace", "CPA_ERR_OVERLAP", acc_fwd(p, oa=80))
    case("accum_lse_acc_overlaps_o", "CPA_ERR_OVERLAP", acc_fwd(p, la=40))
    case("accum_misaligned_o_acc", "CPA_ERR_ALIGN",
         lib.attn_fwd_accum(ctypes.byref(p), ptr(1), ptr(2), ptr(3), ctypes.c_void_p(A * 101 + 8),
                            ptr(120), ptr(40), ptr(60), ptr(80), 256, None))
    p = good_problem(); p.out_dtype = 1
    case("accum_in_place_fp32_reaches_launch", "CPA_ERR_LAUNCH", acc_fwd(p, oa=40, la=60))
    p = good_problem(512, 512); p.out_dtype = 1
    case("accum_lse_in_place_d512_declined", "CPA_ERR_OVERLAP", acc_fwd(p, oa=40, la=60))
    case("accum_d512_separate_lse_reaches_launch", "CPA_ERR_LAUNCH", acc_fwd(p, oa=40))

    def bwd(p, flags=0, wsb=1 << 30, dq=100, dk=120, dv=140):
        return lib.attn_bwd(ctypes.byref(p), ptr(1), ptr(2), ptr(3), ptr(40), ptr(50), ptr(60),
                            ptr(dq), ptr(dk), ptr(dv), ptr(200), wsb, flags, None)

    # The backward has no atomics at any head dim, so the flag is accepted:
    # validation passes and only the launch, with no GPU visible, fails.
    for d in (128, 256, 512):
        p = good_problem(d_qk=d, d_v=d)
        case(f"bwd_deterministic_accepted_d{d}", "CPA_ERR_LAUNCH", bwd(p, flags=1))
    p = good_problem()
    case("bwd_dq_direct_flag_accepted", "CPA_ERR_LAUNCH", bwd(p, flags=2))
    case("bwd_unknown_flag", "CPA_ERR_UNSUPPORTED", bwd(p, flags=4))
    need = lib.attn_bwd_workspace_size(ctypes.byref(p))
    least = lib.attn_bwd_workspace_min(ctypes.byref(p))
    case("bwd_workspace_small", "CPA_ERR_WORKSPACE", bwd(p, wsb=least - 1))
    case("bwd_workspace_min_accepted", "CPA_ERR_LAUNCH", bwd(p, wsb=least))
    step = lambda fn, wsb: fn(ctypes.byref(p), ptr(1), ptr(2), ptr(3), ptr(40), ptr(50), ptr(60),
                             ptr(100), ptr(120), ptr(140), ptr(200), wsb, 0, None)
    case("bwd_main_step_needs_full_workspace", "CPA_ERR_WORKSPACE", step(lib.attn_bwd_main, least))
    case("bwd_dq_step_needs_full_workspace", "CPA_ERR_WORKSPACE", step(lib.attn_bwd_dq, need - 1))
    case("bwd_outputs_overlap", "CPA_ERR_OVERLAP", bwd(p, dk=100))
    case("bwd_output_overlaps_input", "CPA_ERR_OVERLAP", bwd(p, dq=2))
    # launch grids past the device limits are declined by the host check
    p = good_problem(d_qk=256, d_v=256); p.batch = 20000
    case("bwd_d256_grid_z_declined", "CPA_ERR_UNSUPPORTED", bwd(p))
    far = lambda i: ctypes.c_void_p((i + 1) << 40)   # disjoint fakes for huge tensors
    fwd_far = lambda p: lib.attn_fwd(ctypes.byref(p), far(0), far(1), far(2), far(3), far(4),
                                     far(5), 256, None)
    case("fwd_d256_same_problem_reaches_launch", "CPA_ERR_LAUNCH", fwd_far(p))
    p = good_problem(); p.seqlen_q = 1 << 24
    case("fwd_grid_y_declined", "CPA_ERR_UNSUPPORTED", fwd(p))
    p = good_problem(); p.seqlen_k = 65536 * 128
    case("bwd_grid_y_key_blocks_declined", "CPA_ERR_UNSUPPORTED", bwd(p))
    case("fwd_long_keys_reaches_launch", "CPA_ERR_LAUNCH", fwd_far(p))
    # the backward with the library's own workspace array
    def bstatic(p, flag=300):
        f = None if flag is None else ctypes.c_void_p(A * flag if flag > 0 else -flag)
        return lib.attn_bwd_static(ctypes.byref(p), ptr(1), ptr(2), ptr(3), ptr(40), ptr(50),
                                   ptr(60), ptr(100), ptr(120), ptr(140), f, 0, None)
    p = good_problem()
    case("static_valid_reaches_device_lookup", "CPA_ERR_LAUNCH", bstatic(p))
    case("static_bshd_without_flag_accepted", "CPA_ERR_LAUNCH", bstatic(p, None))
    case("static_misaligned_flag", "CPA_ERR_ALIGN", bstatic(p, -(A * 300 + 2)))
    p = good_problem(); p.seqlen_q = p.seqlen_k = 1 << 16; p.heads_q = 64; p.heads_kv = 8
    case("static_too_large", "CPA_ERR_WORKSPACE", bstatic(p))
    p = good_problem(); p.layout = 1; p.num_seqs = 1
    p.cu_seqlens_q = p.cu_seqlens_k = p.seqused_q = p.seqused_k = A * 400
    case("static_thd_needs_flag", "CPA_ERR_NULL", bstatic(p, None))
    p = good_problem()
    out["bwd_workspace_bytes"] = ["int", int(need)]
    out["bwd_workspace_min_bytes"] = ["int", int(least)]
    p = good_problem(d_qk=512, d_v=512)
    out["bwd_workspace_d512"] = ["int", int(lib.attn_bwd_workspace_size(ctypes.byref(p))),
                                 int(lib.attn_bwd_workspace_min(ctypes.byref(p)))]

    md = _lib.MergeDesc()
    md.batch, md.heads, md.d_v, md.seqlen = 1, 4, 128, 64
    md.acc_stride = md.part_stride = md.out_stride = (64 * 4 * 128, 4 * 128, 128)
    md.lse_acc_stride = md.lse_part_stride = md.lse_out_stride = (4 * 64, 64)
    md.acc_dtype = md.part_dtype = md.out_dtype = 1
    st = lib.attn_merge_lse(ctypes.byref(md), ptr(1), ptr(2), ptr(3), ptr(4), ptr(3), ptr(5), None)
    case("merge_out_overlaps_part", "CPA_ERR_OVERLAP", st)
    md.out_dtype = 0
    st = lib.attn_merge_lse(ctypes.byref(md), ptr(1), ptr(2), ptr(3), ptr(4), ptr(1), ptr(2), None)
    case("merge_inplace_dtype_change", "CPA_ERR_OVERLAP", st)
    md.out_dtype = 9
    st = lib.attn_merge_lse(ctypes.byref(md), ptr(1), ptr(2), ptr(3), ptr(4), ptr(5), ptr(6), None)
    case("merge_bad_dtype", "CPA_ERR_DTYPE", st)

    pd = _lib.PackDesc()
    pd.batch, pd.heads, pd.d_v, pd.o_dtype, pd.groups, pd.seqlen = 1, 6, 128, 0, 4, 64
    pd.o_stride = (64 * 6 * 128, 6 * 128, 128)
    pd.lse_stride = (6 * 64, 64)
    case("pack_heads_not_divisible", "CPA_ERR_SHAPE",
         lib.pack_saved(ctypes.byref(pd), ptr(1), ptr(2), ptr(3), 1 << 24, None))
    out["pack_size_invalid_is_zero"] = ["int", int(lib.pack_saved_size(ctypes.byref(pd)))]
    pd.groups = 3
    n = lib.pack_saved_size(ctypes.byref(pd))
    out["pack_size_valid"] = ["int", int(n)]
    case("pack_buffer_small", "CPA_ERR_SHAPE",
         lib.pack_saved(ctypes.byref(pd), ptr(1), ptr(2), ptr(3), n - 1, None))
    case("pack_buffer_overlaps_o", "CPA_ERR_OVERLAP",
         lib.pack_saved(ctypes.byref(pd), ptr(1), ptr(2), ptr(1), n, None))
    case("unpack_buffer_overlaps_lse", "CPA_ERR_OVERLAP",
         lib.unpack_saved(ctypes.byref(pd), ptr(2), n, ptr(1), ptr(2), None))
    # exchange buffers: one row field and one LSE field, 2 segments
    def xdesc():
        d = _lib.XchgDesc()
        d.batch, d.groups, d.nfields, d.rows = 1, 2, 2, 64
        for g in range(2):
            d.nranges[g] = 1
            d.range_row[g][0], d.range_len[g][0] = 0, 64
        f0, f1 = d.field[0], d.field[1]
        f0.kind, f0.elem_bytes, f0.heads, f0.dim, f0.split = 0, 2, 4, 128, 1
        f0.stride = (64 * 4 * 128, 4 * 128, 128)
        f1.kind, f1.elem_bytes, f1.heads, f1.dim, f1.split = 1, 4, 4, 1, 1
        f1.stride = (4 * 64, 64, 0)
        return d
    ptrs = (ctypes.c_void_p * 2)(A * 1, A * 2)
    xpack = lambda d, buf=ptr(8), n=1 << 24: lib.xchg_pack(ctypes.byref(d), ptrs, buf, n, None)
    d = xdesc()
    seg1 = lib.xchg_segment_offset(ctypes.byref(d), 1)
    total = lib.xchg_segment_offset(ctypes.byref(d), 2)
    # segment: 64 rows x 2 heads x 128 bf16 = 32 KiB, LSE 2 x 64 x 4 = 512 B
    out["xchg_offsets"] = ["int", int(seg1), int(total)]
    case("xchg_valid_reaches_launch", "CPA_ERR_LAUNCH", xpack(d))
    case("xchg_buffer_small", "CPA_ERR_SHAPE", xpack(d, n=total - 1))
    case("xchg_buffer_overlaps_tensor", "CPA_ERR_OVERLAP", xpack(d, buf=ptr(0)))
    d = xdesc(); d.range_len[1][0] = 65
    case("xchg_range_past_rows", "CPA_ERR_SHAPE", xpack(d))
    d = xdesc(); d.field[0].heads = 3
    case("xchg_split_heads_not_divisible", "CPA_ERR_SHAPE", xpack(d))
    d = xdesc(); d.field[0].dim = 4
    case("xchg_row_bytes_not_16", "CPA_ERR_SHAPE", xpack(d))
    d = xdesc(); d.field[0].elem_bytes = 8
    case("xchg_bad_elem_bytes", "CPA_ERR_DTYPE", xpack(d))
    d = xdesc(); d.groups = 9
    case("xchg_too_many_groups", "CPA_ERR_SHAPE", xpack(d))
    out["xchg_invalid_offset_is_zero"] = ["int", int(lib.xchg_segment_offset(ctypes.byref(d), 1))]
    d = xdesc()
    case("xchg_misaligned_buffer", "CPA_ERR_ALIGN", xpack(d, buf=ctypes.c_void_p(A * 8 + 4)))
    print(json.dumps(out))


if __name__ == "__main__":
    main()
