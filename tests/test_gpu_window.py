"""Sliding-window / band masks on the GPU vs the fp64 oracle, element by
element: causal windows, two-sided bands, the diagonal-only window (0, 0),
query segments with a KV-block offset, every head-dim path (the 8-wave and
4-wave key-outer kernels, the dq kernel's block ranges), a banded
workspace, and packed THD documents.

Window (left, right), -1 unbounded, a causal mask keeping the right bound
at the diagonal (PR 3527 "cuDNN FROST attention backend for head_dim in
(256, 512]", commits on sliding window: a window must change the output, and
the backward has to be checked under it, not only the forward).
"""
import math

import numpy as np
import pytest
import torch

import oracle
from tests import criteria
from tests.gpu_util import dev, naive64, say, true64

pytestmark = pytest.mark.gpu

import bwd_causal_flash_amd as cpa  # noqa: E402

# name, Sq, Sk, Hq, Hkv, Dqk, Dv, causal, window, segments, k_pos_begin
CASES = [
    ("d128_causal_left100", 300, 300, 4, 2, 128, 128, True, (100, -1), None, 0),
    ("d192_dual_chunk_left300", 256, 1024, 4, 4, 192, 128, True, (300, -1),
     [(0, 0), (128, 896)], 0),
    ("d128_band_70_40_rect", 200, 330, 2, 2, 128, 128, False, (70, 40), [(0, 130)], 0),
    ("d64_diagonal_only", 150, 150, 2, 1, 64, 64, False, (0, 0), None, 0),
    ("d192_kv_block_left500", 200, 384, 2, 2, 192, 128, True, (500, -1), [(0, 900)], 512),
    ("d256_causal_left90", 270, 270, 4, 2, 256, 256, True, (90, -1), None, 0),
    ("d512_causal_left64", 200, 200, 4, 2, 512, 512, True, (64, -1), None, 0),
    ("d128_right_only_noncausal", 180, 240, 2, 2, 128, 128, False, (-1, 30), None, 0),
]


def _draw(case, seed):
    name, sq, sk, hq, hkv, dqk, dv = case[:7]
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(1, sq, hq, dqk, generator=g), torch.randn(1, sk, hkv, dqk, generator=g),
            torch.randn(1, sk, hkv, dv, generator=g), torch.randn(1, sq, hq, dv, generator=g))


def _oracle(case, q, k, v, do):
    name, sq, sk, hq, hkv, dqk, dv, causal, win, segs, kp0 = case
    scale = 1.0 / math.sqrt(dqk)
    res = {}
    for kind, f in (("true", true64), ("naive", naive64)):
        o, lse = oracle.bshd_forward(f(q), f(k), f(v), scale, segs, kp0, causal, window=win)
        dq, dk, dv_ = oracle.bshd_backward(f(q), f(k), f(v), f(do), scale, segs, kp0, causal,
                                           window=win)
        res[kind] = dict(o=o, lse=lse, dq=dq, dk=dk, dv=dv_)
    return res


def _gpu(case, q, k, v, do, scale_mult=1.0, ws_min=False):
    name, sq, sk, hq, hkv, dqk, dv, causal, win, segs, kp0 = case
    d = dev()
    qi, ki, vi, doi = (x.to(torch.bfloat16).to(d) for x in (q, k, v, do))
    scale = scale_mult / math.sqrt(dqk)
    kw = dict(causal=causal, scale=scale, q_segments=segs, k_pos_begin=kp0, window=win)
    say(f"window fwd {name} x{scale_mult}")
    o, lse = cpa.forward(qi, ki, vi, **kw)
    dq, dk, dv_ = (torch.empty_like(qi), torch.empty_like(ki), torch.empty_like(vi))
    ws = None
    if ws_min:
        ws = torch.empty(cpa.bwd_workspace_bytes(qi, ki, vi, minimum=True), dtype=torch.uint8,
                         device=d)
    say(f"window bwd {name} x{scale_mult} ws_min={ws_min}")
    cpa.attn_bwd(qi, ki, vi, o, doi, lse, dq, dk, dv_, workspace=ws, **kw)
    torch.cuda.synchronize()
    return dict(o=o, lse=lse, dq=dq, dk=dk, dv=dv_)


def _check_all(tag, out, ref, grads=("dq", "dk", "dv")):
    log = {}
    criteria.check("O", out["o"], ref["true"]["o"], ref["naive"]["o"], log=log, out_bf16=True)
    criteria.check_lse("LSE", out["lse"], ref["true"]["lse"], ref["naive"]["lse"], log=log)
    for g in grads:
        criteria.check(g, out[g], ref["true"][g], ref["naive"][g], grad=True, log=log,
                       out_bf16=True)
    print(tag, {k_: round(v_["ratio"], 3) for k_, v_ in log.items() if "ratio" in v_})


@pytest.mark.parametrize("case", CASES, ids=lambda c: c[0])
def test_window_fwd_bwd_matches_oracle(case):
    q, k, v, do = _draw(case, 300 + CASES.index(case))
    ref = _oracle(case, q, k, v, do)
    out = _gpu(case, q, k, v, do)
    if case[0] == "d64_diagonal_only":
        # Only the diagonal key: P = 1, so O = V, dV = dO exactly, and dS =
        # dP - D = <dO, V> - <dO, O> is zero in exact arithmetic (the oracle's
        # floor is 0, so the 2x-floor criterion is degenerate for dQ, dK).
        # The device forms dP (matrix core) and D (pre kernel) in fp32 with
        # different summation orders: |dS| stays at fp32 rounding of |<dO, V>|.
        _check_all(case[0], out, ref, grads=("dv",))
        assert torch.equal(out["o"].float().cpu(),
                           v.to(torch.bfloat16).float().repeat_interleave(2, dim=2))
        assert torch.equal(out["dv"].float().cpu(),
                           do.to(torch.bfloat16).float().reshape(1, 150, 1, 2, 64).sum(3)
                           .to(torch.bfloat16).float())
        bound = 64 * 2 ** -22 * float((do.abs() * v.abs().repeat_interleave(2, dim=2)).sum(-1).max())
        assert float(out["dq"].abs().max()) < bound and float(out["dk"].abs().max()) < bound
        return
    _check_all(case[0], out, ref)
    # the window really changes the result (a dropped bound would still give
    # finite, plausible numbers)
    name, sq, sk, hq, hkv, dqk, dv, causal, win, segs, kp0 = case
    o_nowin, _ = oracle.bshd_forward(naive64(q), naive64(k), naive64(v), 1.0 / math.sqrt(dqk),
                                     segs, kp0, causal)
    assert np.abs(o_nowin - ref["naive"]["o"]).max() > 1e-2


@pytest.mark.parametrize("case", [CASES[1], CASES[5]], ids=lambda c: c[0])
def test_window_banded_workspace(case):
    """Smallest workspace (one dS key block per band): the dq kernel's block
    ranges meet band boundaries."""
    q, k, v, do = _draw(case, 300 + CASES.index(case))
    ref = _oracle(case, q, k, v, do)
    out = _gpu(case, q, k, v, do, ws_min=True)
    _check_all(case[0] + "_bands", out, ref)


def test_window_one_percent_scale_error_is_rejected():
    case = CASES[0]
    q, k, v, do = _draw(case, 300)
    ref = _oracle(case, q, k, v, do)
    out = _gpu(case, q, k, v, do, scale_mult=1.01)
    fails = [not criteria.passes(criteria.evaluate(out[g], ref["true"][g], ref["naive"][g],
                                                   grad=(g != "o"), out_bf16=True))
             for g in ("o", "dq", "dk", "dv")]
    assert any(fails)


def test_window_thd_documents():
    used = np.array([37, 0, 200, 130, 64], np.int32)
    pitch = 64
    cu = np.concatenate([[0], np.cumsum([max(1, (u + pitch - 1) // pitch) * pitch
                                         for u in used])]).astype(np.int32)
    T = int(cu[-1])
    hq, hkv, d = 4, 2, 128
    win = (45, -1)
    g = torch.Generator().manual_seed(41)
    q, k, v, do = (torch.randn(T, h, d, generator=g) for h in (hq, hkv, hkv, hq))
    scale = 1.0 / math.sqrt(d)
    ref = {}
    for kind, f in (("true", true64), ("naive", naive64)):
        o, lse = oracle.thd_forward(f(q), f(k), f(v), scale, cu, cu, used, used, window=win)
        dq, dk, dv_ = oracle.thd_backward(f(q), f(k), f(v), f(do), scale, cu, cu, used, used,
                                          window=win)
        ref[kind] = dict(o=o, lse=lse, dq=dq, dk=dk, dv=dv_)
    dv0 = dev()
    qi, ki, vi, doi = (x.to(torch.bfloat16).to(dv0) for x in (q, k, v, do))
    tcu, tused = torch.tensor(cu, device=dv0), torch.tensor(used, device=dv0)
    vl = cpa.Varlen(tcu, tcu, tused, tused, int(used.max()), int(used.max()), False)
    say("window thd fwd")
    o, lse = cpa.forward(qi, ki, vi, varlen=vl, window=win)
    say("window thd bwd")
    dq, dk, dvv = cpa.backward(qi, ki, vi, o, doi, lse, varlen=vl, window=win)
    torch.cuda.synchronize()
    real = np.concatenate([np.arange(cu[n], cu[n] + used[n]) for n in range(len(used))])
    log = {}
    criteria.check("O", o[real], ref["true"]["o"][real], ref["naive"]["o"][real], log=log,
                   out_bf16=True)
    criteria.check_lse("LSE", lse[:, real], ref["true"]["lse"][:, real],
                       ref["naive"]["lse"][:, real], log=log)
    for name, a, b in (("dq", dq, "dq"), ("dk", dk, "dk"), ("dv", dvv, "dv")):
        criteria.check(name, a[real], ref["true"][b][real], ref["naive"][b][real], grad=True,
                       log=log, out_bf16=True)
    print("thd window", {k_: round(v_["ratio"], 3) for k_, v_ in log.items() if "ratio" in v_})


# fp32 inputs (rounded to bf16 on the way into the kernels) and fp32 outputs
# through the banded kernels of each head-dim family: the fp32-input staging
# paths and the fp32-output epilogues of the windowed kernels.
# name, Sq, Sk, Hq, Hkv, Dqk, Dv, causal, window, segments, k_pos_begin, in, out
FP32_CASES = [
    ("d192_fp32_io_left300", 256, 512, 4, 2, 192, 128, True, (300, -1), None, 0, "fp32", "fp32"),
    ("d128_fp32_in_band_70_40", 200, 260, 2, 2, 128, 128, False, (70, 40), None, 0,
     "fp32", "bf16"),
    ("d256_fp32_io_left90", 200, 200, 2, 1, 256, 256, True, (90, -1), None, 0, "fp32", "fp32"),
    ("d512_fp32_io_left64", 130, 130, 2, 2, 512, 512, True, (64, -1), None, 0, "fp32", "fp32"),
    ("d512_bf16_in_fp32_out_left64", 150, 150, 2, 1, 512, 512, True, (64, -1), None, 0,
     "bf16", "fp32"),
]
_DT = {"bf16": torch.bfloat16, "fp32": torch.float32}


@pytest.mark.parametrize("case", FP32_CASES, ids=lambda c: c[0])
def test_window_fp32_io(case):
    name, sq, sk, hq, hkv, dqk, dv, causal, win, segs, kp0, idt, odt = case
    q, k, v, do = _draw(case, 400 + FP32_CASES.index(case))
    ref = _oracle(case[:11], q, k, v, do)
    d = dev()
    qi, ki, vi, doi = (x.to(_DT[idt]).to(d) for x in (q, k, v, do))
    kw = dict(causal=causal, scale=1.0 / math.sqrt(dqk), q_segments=segs, k_pos_begin=kp0,
              window=win)
    say(f"window fp32 fwd {name}")
    o, lse = cpa.forward(qi, ki, vi, out_dtype=_DT[odt], **kw)
    say(f"window fp32 bwd {name}")
    dq, dk, dv_ = cpa.backward(qi, ki, vi, o.to(_DT[idt]), doi, lse, out_dtype=_DT[odt], **kw)
    torch.cuda.synchronize()
    ob = odt == "bf16"
    log = {}
    criteria.check("O", o, ref["true"]["o"], ref["naive"]["o"], log=log, out_bf16=ob)
    criteria.check_lse("LSE", lse, ref["true"]["lse"], ref["naive"]["lse"], log=log)
    for g, val in (("dq", dq), ("dk", dk), ("dv", dv_)):
        criteria.check(g, val, ref["true"][g], ref["naive"][g], grad=True, log=log, out_bf16=ob)
    print(name, {k_: round(v_["ratio"], 3) for k_, v_ in log.items() if "ratio" in v_})
