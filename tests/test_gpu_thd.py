"""Packed THD varlen on the GPU: per-document parity with the oracle,
NaN-poisoned padding inputs, sentinel-filled padding outputs left bit for
bit unchanged, empty documents, bottom-right alignment with different query
and key lengths, and the device metadata check.

Padded THD = physical padded offsets plus visible lengths (PR 3149, "Enable
FA4 for context-parallel attention", Description); padding canaries and an
empty sequence follow PR 3699's review ("Add cuDNN OSS backward dispatch for
context parallel attention": physical gaps and an empty sequence).
"""
import math

import numpy as np
import pytest
import torch

import oracle
from tests import criteria
from tests.gpu_util import bits, dev, naive64, say, true64

pytestmark = pytest.mark.gpu

import bwd_causal_flash_amd as cpa  # noqa: E402

SENT_BF16 = 0x7FC1
SENT_F32 = 0x7FC00001


def _layout(lens, pitch=64):
    cu = [0]
    for L in lens:
        cu.append(cu[-1] + (L + pitch - 1) // pitch * pitch + (0 if L % pitch else 0))
    return np.asarray(lens, np.int32), np.asarray(cu, np.int32)


def _sentinel(shape, dtype, d):
    if dtype == torch.bfloat16:
        return torch.full(shape, SENT_BF16, dtype=torch.int16, device=d).view(torch.bfloat16)
    return torch.full(shape, SENT_F32, dtype=torch.int32, device=d).view(torch.float32)


def _pad_rows(cu, used):
    rows = []
    for n in range(len(used)):
        rows.extend(range(int(cu[n]) + int(used[n]), int(cu[n + 1])))
    return np.asarray(rows, np.int64)


def _thd_case(bottom_right, scale_mult=1.0):
    """Seven documents (one empty, one of one row) at a 64-row pitch, padding
    inputs NaN, padding outputs sentinel-filled; returns the GPU outputs, the
    oracle's true and naive results and the real-row masks."""
    used_q = np.array([37, 0, 130, 1, 200, 64, 5], np.int32)
    used_k = used_q.copy() if not bottom_right else np.array([50, 3, 100, 70, 200, 64, 0], np.int32)
    pitch = 64
    cu_q = np.concatenate([[0], np.cumsum([max(1, (max(a, b) + pitch - 1) // pitch) * pitch
                                           for a, b in zip(used_q, used_k)])]).astype(np.int32)
    cu_k = cu_q.copy()
    T = int(cu_q[-1])
    hq, hkv, d = 4, 2, 128
    g = torch.Generator().manual_seed(11 + bottom_right)
    q = torch.randn(T, hq, d, generator=g)
    k = torch.randn(T, hkv, d, generator=g)
    v = torch.randn(T, hkv, d, generator=g)
    do = torch.randn(T, hq, d, generator=g)
    dv_ = dev()
    pad_q = _pad_rows(cu_q, used_q)
    pad_k = _pad_rows(cu_k, used_k)
    qi, ki, vi, doi = (x.to(torch.bfloat16).to(dv_) for x in (q, k, v, do))
    # poison the padding rows of every input
    qi[pad_q] = float("nan"); doi[pad_q] = float("nan")
    ki[pad_k] = float("nan"); vi[pad_k] = float("nan")
    vl = cpa.Varlen(torch.tensor(cu_q, device=dv_), torch.tensor(cu_k, device=dv_),
                    torch.tensor(used_q, device=dv_), torch.tensor(used_k, device=dv_),
                    int(used_q.max()), int(used_k.max()), bottom_right)
    o = _sentinel((T, hq, d), torch.bfloat16, dv_)
    lse = _sentinel((hq, T), torch.float32, dv_)
    scale = 1 / math.sqrt(d)
    say(f"thd fwd br={bottom_right} scale x{scale_mult}")
    ws = cpa.attn_fwd(qi, ki, vi, o, lse, varlen=vl, scale=scale * scale_mult)
    dq = _sentinel((T, hq, d), torch.bfloat16, dv_)
    dk = _sentinel((T, hkv, d), torch.bfloat16, dv_)
    dvv = _sentinel((T, hkv, d), torch.bfloat16, dv_)
    say(f"thd bwd br={bottom_right} scale x{scale_mult}")
    ws2 = cpa.attn_bwd(qi, ki, vi, o, doi, lse, dq, dk, dvv, varlen=vl, scale=scale * scale_mult)
    torch.cuda.synchronize()
    assert cpa.workspace_error_flag(ws) == 0 and cpa.workspace_error_flag(ws2) == 0
    for t, rows in ((o, pad_q), (dq, pad_q), (dk, pad_k), (dvv, pad_k)):
        assert (bits(t)[rows] == np.int16(SENT_BF16)).all()
    assert (bits(lse)[:, pad_q] == np.int32(SENT_F32)).all()

    ref = {}
    for kind, f in (("true", true64), ("naive", naive64)):
        oo, ll = oracle.thd_forward(f(q), f(k), f(v), scale, cu_q, cu_k, used_q, used_k, True,
                                    bottom_right)
        a, b_, c = oracle.thd_backward(f(q), f(k), f(v), f(do), scale, cu_q, cu_k, used_q,
                                       used_k, True, bottom_right)
        ref[kind] = dict(o=oo, lse=ll, dq=a, dk=b_, dv=c)
    real_q = np.ones(T, bool); real_q[pad_q] = False
    real_k = np.ones(T, bool); real_k[pad_k] = False
    masks = dict(o=np.broadcast_to(real_q[:, None, None], (T, hq, d)),
                 dq=np.broadcast_to(real_q[:, None, None], (T, hq, d)),
                 dk=np.broadcast_to(real_k[:, None, None], (T, hkv, d)),
                 dv=np.broadcast_to(real_k[:, None, None], (T, hkv, d)),
                 lse=np.broadcast_to(real_q[None], (hq, T)))
    return dict(o=o, lse=lse, dq=dq, dk=dk, dv=dvv), ref, masks


@pytest.mark.parametrize("bottom_right", [False, True])
def test_thd_parity_and_padding_untouched(bottom_right):
    out, ref, masks = _thd_case(bottom_right)
    log = {}
    criteria.check("O", out["o"], ref["true"]["o"], ref["naive"]["o"], mask=masks["o"], log=log,
                   out_bf16=True)
    criteria.check_lse("LSE", out["lse"], ref["true"]["lse"], ref["naive"]["lse"],
                       mask=masks["lse"], log=log)
    for g in ("dq", "dk", "dv"):
        criteria.check(g, out[g], ref["true"][g], ref["naive"][g], mask=masks[g], grad=True,
                       log=log, out_bf16=True)
    print(log)


def test_thd_one_percent_scale_error_is_rejected():
    """The same THD case with the softmax scale 1% off must fail the
    criterion (PR 3527, Verification: the bound has to catch a 1% error)."""
    out, ref, masks = _thd_case(False, scale_mult=1.01)
    fails = {}
    for g in ("o", "dq", "dk", "dv"):
        r = criteria.evaluate(out[g], ref["true"][g], ref["naive"][g], mask=masks[g],
                              grad=(g != "o"), out_bf16=True)
        fails[g] = not criteria.passes(r)
    fin = masks["lse"] & np.isfinite(ref["naive"]["lse"])
    fails["lse"] = criteria.max_err(out["lse"], ref["naive"]["lse"], fin) > 1e-4
    print("thd 1% scale error caught by:", fails)
    assert fails["lse"]
    assert fails["o"] or fails["dq"] or fails["dk"] or fails["dv"], fails


def test_thd_malformed_metadata_sets_flag_and_skips_sequence():
    """A sequence whose visible length exceeds its physical span is treated
    as empty (none of its outputs written, nothing read out of bounds) and
    the workspace flag is raised; the other sequences are still computed."""
    d = dev()
    hq, dd = 2, 64
    cu = np.array([0, 64, 128], np.int32)
    used = np.array([40, 100], np.int32)       # 100 > 64: malformed
    T = 128
    g = torch.Generator().manual_seed(1)
    q, k, v = (torch.randn(T, hq, dd, generator=g) for _ in range(3))
    vl = cpa.Varlen(torch.tensor(cu, device=d), torch.tensor(cu, device=d),
                    torch.tensor(used, device=d), torch.tensor(used, device=d), 100, 100)
    o = _sentinel((T, hq, dd), torch.bfloat16, d)
    lse = _sentinel((hq, T), torch.float32, d)
    say("thd malformed metadata")
    ws = cpa.attn_fwd(q.to(torch.bfloat16).to(d), k.to(torch.bfloat16).to(d),
                      v.to(torch.bfloat16).to(d), o, lse, varlen=vl)
    torch.cuda.synchronize()
    assert cpa.workspace_error_flag(ws) == 1
    assert (bits(o)[64:] == np.int16(SENT_BF16)).all()
    assert not (bits(o)[:40] == np.int16(SENT_BF16)).any()


@pytest.mark.parametrize("dqk,d", [(192, 128), (256, 256), (512, 512)])
def test_thd_large_head_dims(dqk, d):
    """Packed THD at head dims 192/128 (the key-outer kernel of the CP rank
    shape) and 256/512 (scores and dS tiles materialised per document): five
    documents at a 64-row pitch (one empty, one of one row, one longer than
    a 128-row tile), GQA 4/2, NaN in the padding input rows, padding output
    rows untouched."""
    used = np.array([150, 0, 1, 70, 260], np.int32)
    pitch = 64
    cu = np.concatenate([[0], np.cumsum([max(1, (n + pitch - 1) // pitch) * pitch
                                         for n in used])]).astype(np.int32)
    T, hq, hkv = int(cu[-1]), 4, 2
    g = torch.Generator().manual_seed(80 + dqk + d)
    q, k, v, do = (torch.randn(T, h_, w_, generator=g)
                   for h_, w_ in ((hq, dqk), (hkv, dqk), (hkv, d), (hq, d)))
    pad = _pad_rows(cu, used)
    dv0 = dev()
    qi, ki, vi, doi = (x.to(torch.bfloat16).to(dv0) for x in (q, k, v, do))
    for t in (qi, ki, vi, doi):
        t[pad] = float("nan")
    vl = cpa.Varlen(torch.tensor(cu, device=dv0), torch.tensor(cu, device=dv0),
                    torch.tensor(used, device=dv0), torch.tensor(used, device=dv0),
                    int(used.max()), int(used.max()))
    o = _sentinel((T, hq, d), torch.bfloat16, dv0)
    lse = _sentinel((hq, T), torch.float32, dv0)
    dq = _sentinel((T, hq, dqk), torch.bfloat16, dv0)
    dk = _sentinel((T, hkv, dqk), torch.bfloat16, dv0)
    dvv = _sentinel((T, hkv, d), torch.bfloat16, dv0)
    scale = 1 / math.sqrt(dqk)
    say(f"thd d{dqk}/{d} fwd")
    ws = cpa.attn_fwd(qi, ki, vi, o, lse, varlen=vl, scale=scale)
    say(f"thd d{dqk}/{d} bwd")
    ws2 = cpa.attn_bwd(qi, ki, vi, o, doi, lse, dq, dk, dvv, varlen=vl, scale=scale)
    torch.cuda.synchronize()
    assert cpa.workspace_error_flag(ws) == 0 and cpa.workspace_error_flag(ws2) == 0
    for t in (o, dq, dk, dvv):
        assert (bits(t)[pad] == np.int16(SENT_BF16)).all()
    assert (bits(lse)[:, pad] == np.int32(SENT_F32)).all()
    ref = {}
    for kind, f in (("true", true64), ("naive", naive64)):
        oo, ll = oracle.thd_forward(f(q), f(k), f(v), scale, cu, cu, used, used)
        a, b_, c = oracle.thd_backward(f(q), f(k), f(v), f(do), scale, cu, cu, used, used)
        ref[kind] = dict(o=oo, lse=ll, dq=a, dk=b_, dv=c)
    real = np.ones(T, bool)
    real[pad] = False
    log = {}
    for name, val, h_, w_ in (("O", o, hq, d), ("dq", dq, hq, dqk), ("dk", dk, hkv, dqk),
                              ("dv", dvv, hkv, d)):
        key = "o" if name == "O" else name
        criteria.check(name, val, ref["true"][key], ref["naive"][key], grad=name != "O",
                       mask=np.broadcast_to(real[:, None, None], (T, h_, w_)), log=log,
                       out_bf16=True)
    criteria.check_lse("LSE", lse, ref["true"]["lse"], ref["naive"]["lse"],
                       mask=np.broadcast_to(real[None], (hq, T)), log=log)
    print(f"thd d{dqk}/{d}", {k_: round(v_["ratio"], 3) for k_, v_ in log.items() if "ratio" in v_})
