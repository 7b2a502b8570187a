"""attn_bwd_static (the backward with the library's fixed per-GPU workspace,
for callers that cannot allocate) against attn_bwd, through the C ABI.

Two calls in a row on one GPU, the second with a smaller input, then a THD
call: the static array keeps the previous call's contents, so each result
must still equal attn_bwd's bit for bit (dK, dV always; dQ whenever the key
bands are the same, i.e. attn_bwd given a workspace of the array's size).
"""
import numpy as np
import pytest
import torch

from tests.gpu_util import dev, say

pytestmark = pytest.mark.gpu

import bwd_causal_flash_amd as cpa  # noqa: E402

BF = torch.bfloat16
CAP = cpa._lib.CPA_BWD_STATIC_WORKSPACE_BYTES


def _inputs(shape_q, shape_k, dv, seed, d):
    g = torch.Generator(device=d).manual_seed(seed)
    q = torch.randn(*shape_q, device=d, generator=g).to(BF)
    k = torch.randn(*shape_k, device=d, generator=g).to(BF)
    v = torch.randn(*shape_k[:-1], dv, device=d, generator=g).to(BF)
    do = torch.randn(*shape_q[:-1], dv, device=d, generator=g).to(BF)
    return q, k, v, do


def _same(a, b):
    return torch.equal(a.view(torch.int16), b.view(torch.int16))


def _run_both(q, k, v, do, *, varlen=None, ws_bytes=None, **kw):
    o, lse = cpa.forward(q, k, v, varlen=varlen, **kw)
    ref = [torch.zeros_like(t) for t in (q, k, v)]
    ws = None
    if ws_bytes is not None:
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
    cpa.attn_bwd(q, k, v, o, do, lse, *ref, varlen=varlen, workspace=ws, **kw)
    got = [torch.full_like(t, 3.0) for t in (q, k, v)]
    flag = torch.full((1,), 7, dtype=torch.int32, device=q.device)
    cpa.attn_bwd_static(q, k, v, o, do, lse, *got, varlen=varlen, err_flag=flag, **kw)
    torch.cuda.synchronize()
    return ref, got, int(flag.item())


def test_static_workspace_matches_attn_bwd():
    d = dev()
    # 1) B1 S8192 Hq16/Hkv8 D128: the full workspace (2.2 GB) is larger than
    #    the array, so both run in key bands; attn_bwd gets a workspace of
    #    the array's size, hence the same bands: bitwise equal
    q, k, v, do = _inputs((1, 8192, 16, 128), (1, 8192, 8, 128), 128, 1, d)
    assert cpa.bwd_workspace_bytes(q, k, v) > CAP >= cpa.bwd_workspace_bytes(q, k, v, minimum=True)
    say("static bwd: B1 S8192 Hq16/Hkv8 D128, banded")
    ref, got, flag = _run_both(q, k, v, do, ws_bytes=CAP)
    assert flag == 0
    for name, a, b in zip(("dq", "dk", "dv"), ref, got):
        assert _same(a, b), name
    # 2) smaller, dual-chunk positions, D 192/128: everything fits, no bands
    q, k, v, do = _inputs((1, 700, 4, 192), (1, 1500, 2, 192), 128, 2, d)
    say("static bwd: B1 Sq700 Sk1500 Hq4/Hkv2 D192/128, two segments")
    ref, got, flag = _run_both(q, k, v, do, q_segments=[(0, 100), (350, 1100)])
    assert flag == 0
    for name, a, b in zip(("dq", "dk", "dv"), ref, got):
        assert _same(a, b), name
    # 3) packed THD (documents of 300, 0 and 129 rows), metadata flag written
    used = torch.tensor([300, 0, 129], dtype=torch.int32)
    cu = torch.tensor([0, 320, 384, 576], dtype=torch.int32)
    vl = cpa.Varlen(cu.to(d), cu.to(d), used.to(d), used.to(d), 300, 300)
    q, k, v, do = _inputs((576, 4, 128), (576, 2, 128), 128, 3, d)
    say("static bwd: THD 3 documents")
    ref, got, flag = _run_both(q, k, v, do, varlen=vl)
    assert flag == 0
    real = np.concatenate([np.arange(0, 300), np.arange(384, 513)])
    for name, a, b in zip(("dq", "dk", "dv"), ref, got):
        assert _same(a[real], b[real]), name


def test_static_workspace_declines_too_large():
    """A problem whose smallest workspace exceeds the array is refused
    before anything runs."""
    d = dev()
    q = torch.zeros(1, 16384, 64, 128, dtype=BF, device=d)
    k = torch.zeros(1, 16384, 8, 128, dtype=BF, device=d)
    assert cpa.bwd_workspace_bytes(q, k, k, minimum=True) > CAP
    o = torch.zeros_like(q)
    lse = torch.zeros(1, 64, 16384, device=d)
    with pytest.raises(cpa.CpaError, match="CPA_ERR_WORKSPACE"):
        cpa.attn_bwd_static(q, k, k, o, o, lse, torch.empty_like(q), torch.empty_like(k),
                            torch.empty_like(k))
