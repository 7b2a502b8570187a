"""CPU checks of the C ABI: the library loads and exports every function the
header declares, the ctypes mirrors match the C struct layouts, and every
argument error is reported by host validation (run with no GPU visible, so
nothing can reach a device)."""
import ctypes
import json
import os
import re
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "cpattn.h")
LIB = os.path.join(ROOT, "bwd_causal_flash_amd", "libcpattn.so")

needs_lib = pytest.mark.skipif(not os.path.exists(LIB), reason="libcpattn.so not built")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^[A-Za-z_][\w\s\*]*?\b([a-z_]\w*)\s*\(", text, flags=re.M)
    return sorted(set(n for n in names if n not in ("if", "sizeof")))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("attn_fwd", "attn_bwd", "attn_merge_lse", "pack_saved", "unpack_saved",
              "attn_fwd_workspace_size", "attn_bwd_workspace_size", "pack_saved_size",
              "attn_status_string", "xchg_segment_offset", "xchg_pack", "xchg_unpack"):
        assert n in names, n


@needs_lib
def test_library_exports_every_declared_function():
    lib = ctypes.CDLL(LIB)
    for n in declared_functions():
        assert hasattr(lib, n), f"missing export {n}"
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True)
    exported = set(re.findall(r" T (\w+)$", out.stdout, flags=re.M))
    c_like = {e for e in exported if not e.startswith("_Z") and not e.startswith("_")}
    assert c_like == set(declared_functions()), c_like ^ set(declared_functions())


def test_ctypes_structs_match_c_layout():
    sys.path.insert(0, ROOT)
    from bwd_causal_flash_amd import _lib
    prog = r"""
#include <stdio.h>
#include <stddef.h>
#include "cpattn.h"
#define F(s, f) printf("%s.%s %zu\n", #s, #f, offsetof(struct s, f));
int main(void) {
  printf("cpa_problem %zu\n", sizeof(struct cpa_problem));
  printf("cpa_merge_desc %zu\n", sizeof(struct cpa_merge_desc));
  printf("cpa_pack_desc %zu\n", sizeof(struct cpa_pack_desc));
  printf("cpa_xchg_desc %zu\n", sizeof(struct cpa_xchg_desc));
  printf("cpa_xchg_field %zu\n", sizeof(struct cpa_xchg_field));
  F(cpa_xchg_desc, rows) F(cpa_xchg_desc, range_row) F(cpa_xchg_desc, range_len)
  F(cpa_xchg_desc, field) F(cpa_xchg_field, split) F(cpa_xchg_field, stride)
  F(cpa_problem, seqlen_q) F(cpa_problem, cu_seqlens_q) F(cpa_problem, q_stride)
  F(cpa_problem, lse_stride) F(cpa_problem, softmax_scale) F(cpa_problem, q_seg_row)
  F(cpa_problem, k_pos_begin) F(cpa_problem, window) F(cpa_problem, window_right)
  F(cpa_merge_desc, seqlen) F(cpa_merge_desc, acc_stride) F(cpa_merge_desc, lse_out_stride)
  F(cpa_pack_desc, seqlen) F(cpa_pack_desc, o_stride) F(cpa_pack_desc, force_int64)
  return 0;
}
"""
    with tempfile.TemporaryDirectory() as d:
        src = os.path.join(d, "t.c")
        exe = os.path.join(d, "t")
        open(src, "w").write(prog)
        subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), src, "-o", exe], check=True)
        lines = subprocess.run([exe], capture_output=True, text=True, check=True).stdout.split("\n")
    got = dict(l.split() for l in lines if l.strip())
    mirrors = {"cpa_problem": _lib.Problem, "cpa_merge_desc": _lib.MergeDesc,
               "cpa_pack_desc": _lib.PackDesc, "cpa_xchg_desc": _lib.XchgDesc,
               "cpa_xchg_field": _lib.XchgField}
    for k, v in got.items():
        if "." in k:
            s, f = k.split(".")
            assert getattr(mirrors[s], f).offset == int(v), k
        else:
            assert ctypes.sizeof(mirrors[k]) == int(v), k


@needs_lib
def test_argument_errors_are_rejected_before_launch():
    env = dict(os.environ, HIP_VISIBLE_DEVICES="-1", ROCR_VISIBLE_DEVICES="-1")
    r = subprocess.run([sys.executable, os.path.join(ROOT, "tests", "abi_cases.py")],
                       capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, r.stderr
    res = json.loads(r.stdout.strip().splitlines()[-1])
    bad = {k: v for k, v in res.items() if v[0] != "int" and v[0] != v[1]}
    assert not bad, bad
    assert res["pack_size_invalid_is_zero"][1] == 0
    assert res["xchg_offsets"][1:] == [32768 + 512, 2 * (32768 + 512)]
    assert res["xchg_invalid_offset_is_zero"][1] == 0
    assert res["pack_size_valid"][1] % 256 == 0 and res["pack_size_valid"][1] > 0
    # flag + D + fp32 dQ accumulator + query position tables (4 tiles x
    # (16 B + 64 rows x 4 B) = 1088 B, padded to 1280), then dS tiles: 4 heads
    # x 4 query tiles x 16 KiB per 128-key block; the problem has 256 keys =
    # 2 blocks.
    base = 256 + 4 * 256 * 4 + 256 * 4 * 128 * 4 + 1280
    block = 4 * 4 * 64 * 128 * 2
    assert res["bwd_workspace_min_bytes"][1] == base + block
    assert res["bwd_workspace_bytes"][1] == base + 2 * block
    # head dim 512: a larger fp32 accumulator, and the P tiles kept beside
    # the dS tiles (twice the tile bytes per key block)
    full, least = res["bwd_workspace_d512"][1:]
    base512 = 256 + 4 * 256 * 4 + 256 * 4 * 512 * 4 + 1280
    assert least == base512 + 2 * block and full == base512 + 4 * block
