"""Backward paths beyond one full call (head dims 192/128, and 256/512 below):

* CPA_FLAG_DETERMINISTIC: repeated calls, also on a side stream, give
  bitwise identical dQ, dK, dV;
* a workspace below attn_bwd_workspace_size: the keys are processed in
  bands; dK and dV do not depend on the band split (bitwise), dQ meets the
  accuracy criterion for every split;
* the ring-step use of the step entry points (the per-block backward of the
  pages' P2P ring): pre once, then main + dq per key block with that
  block's K, V, dK, dV and k_pos_begin, then post once;
* the single-pass dQ (whole workspace: the dq kernel writes dq itself) is
  bitwise the accumulating path's, zeros included.

Every result is checked against the fp64 oracle with the accuracy
criterion (tests/criteria.py).
"""
import math

import pytest
import torch

import oracle
from tests import criteria
from tests.gpu_util import dev, naive64, say, true64

pytestmark = pytest.mark.gpu

import bwd_causal_flash_amd as cpa  # noqa: E402

# Dual-chunk query rows (positions 0..127 and 896..1023), 1024 keys, GQA 4/2,
# head dims 192/128: 8 key blocks, two of them ragged in the ring split.
B, SQ, SK, HQ, HKV, DQK, DV = 1, 256, 1024, 4, 2, 192, 128
SEGS = [(0, 0), (128, 896)]
SCALE = 1.0 / math.sqrt(DQK)
DETERMINISTIC = 1


@pytest.fixture(scope="module")
def problem():
    g = torch.Generator().manual_seed(11)
    q = torch.randn(B, SQ, HQ, DQK, generator=g)
    k = torch.randn(B, SK, HKV, DQK, generator=g)
    v = torch.randn(B, SK, HKV, DV, generator=g)
    do = torch.randn(B, SQ, HQ, DV, generator=g)
    ref = {}
    for kind, f in (("true", true64), ("naive", naive64)):
        dq, dk, dv = oracle.bshd_backward(f(q), f(k), f(v), f(do), SCALE, SEGS, 0, True)
        ref[kind] = dict(dq=dq, dk=dk, dv=dv)
    d = dev()
    qi, ki, vi, doi = (x.to(torch.bfloat16).to(d) for x in (q, k, v, do))
    say("fwd for backward-path tests")
    o, lse = cpa.forward(qi, ki, vi, scale=SCALE, q_segments=SEGS)
    torch.cuda.synchronize()
    return dict(q=qi, k=ki, v=vi, do=doi, o=o, lse=lse, ref=ref)


def _outputs(p):
    return (torch.empty_like(p["q"]), torch.empty_like(p["k"]),
            torch.empty(p["v"].shape, dtype=torch.bfloat16, device=p["q"].device))


def _run(p, ws=None, flags=0, stream=None):
    dq, dk, dv = _outputs(p)
    cpa.attn_bwd(p["q"], p["k"], p["v"], p["o"], p["do"], p["lse"], dq, dk, dv, scale=SCALE,
                 q_segments=SEGS, workspace=ws, flags=flags, stream=stream)
    return dq, dk, dv


def _check(p, dq, dk, dv, tag):
    torch.cuda.synchronize()
    log = {}
    for name, val in (("dq", dq), ("dk", dk), ("dv", dv)):
        criteria.check(f"{tag}:{name}", val, p["ref"]["true"][name], p["ref"]["naive"][name],
                       grad=True, out_bf16=True, log=log)
    print(tag, {k_: round(v_["ratio"], 3) for k_, v_ in log.items()})


def _bits(x):
    return x.view(torch.int16)


def test_deterministic_flag_is_bitwise_reproducible(problem):
    p = problem
    say("bwd deterministic x20")
    first = _run(p, flags=DETERMINISTIC)
    _check(p, *first, "deterministic")
    for _ in range(19):
        again = _run(p, flags=DETERMINISTIC)
        for a, b in zip(first, again):
            assert torch.equal(_bits(a), _bits(b))
    side = torch.cuda.Stream()
    say("bwd deterministic on a side stream")
    with torch.cuda.stream(side):
        other = _run(p, flags=DETERMINISTIC, stream=side)
    side.synchronize()
    for a, b in zip(first, other):
        assert torch.equal(_bits(a), _bits(b))


def test_banded_workspace(problem):
    p = problem
    full = cpa.bwd_workspace_bytes(p["q"], p["k"], p["v"])
    least = cpa.bwd_workspace_bytes(p["q"], p["k"], p["v"], minimum=True)
    block = (full - least) // 7                 # 8 key blocks of 128
    assert full - least == 7 * block and block == HQ * (SQ // 64) * 64 * 128 * 2
    dev_ = p["q"].device
    results = {}
    for nblocks in (8, 3, 1):
        size = least + (nblocks - 1) * block
        ws = torch.empty(size, dtype=torch.uint8, device=dev_)
        say(f"bwd with room for {nblocks} dS key blocks")
        results[nblocks] = _run(p, ws=ws)
        _check(p, *results[nblocks], f"bands_of_{nblocks}")
    for nb in (3, 1):
        assert torch.equal(_bits(results[8][1]), _bits(results[nb][1]))   # dK
        assert torch.equal(_bits(results[8][2]), _bits(results[nb][2]))   # dV


def test_ring_step_backward(problem):
    """pre once, main + dq per key block (384, 384, 256 keys), post once."""
    p = problem
    blocks = [(0, 384), (384, 768), (768, 1024)]
    dq, dk, dv = _outputs(p)
    ws_bytes = max(cpa.bwd_workspace_bytes(p["q"], p["k"][:, a:b], p["v"][:, a:b])
                   for a, b in blocks)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=p["q"].device)
    common = dict(scale=SCALE, q_segments=SEGS, workspace=ws)

    def call(step, a, b):
        cpa.attn_bwd(p["q"], p["k"][:, a:b], p["v"][:, a:b], p["o"], p["do"], p["lse"], dq,
                     dk[:, a:b], dv[:, a:b], k_pos_begin=a, step=step, **common)

    say("ring-step bwd: pre")
    call("attn_bwd_pre", *blocks[0])
    for a, b in blocks:
        say(f"ring-step bwd: main + dq keys [{a}, {b})")
        call("attn_bwd_main", a, b)
        call("attn_bwd_dq", a, b)
    say("ring-step bwd: post")
    call("attn_bwd_post", *blocks[-1])
    _check(p, dq, dk, dv, "ring_step")


@pytest.mark.parametrize("d", [256, 512])
def test_large_head_dims_deterministic_and_banded(d):
    """Head dims 256/512 (the 4-wave key-outer kernel storing dS, the dq
    kernel in 256-column chunks): repeated calls are bitwise identical, and a
    one-key-block band split gives bitwise equal dK, dV; every result meets
    the accuracy criterion.  Ragged 200 queries and 330 keys, GQA 4/2."""
    b_, sq, sk, hq, hkv = 1, 200, 330, 4, 2
    scale = 1.0 / math.sqrt(d)
    segs = [(0, sk - sq)]
    g = torch.Generator().manual_seed(23 + d)
    q = torch.randn(b_, sq, hq, d, generator=g)
    k = torch.randn(b_, sk, hkv, d, generator=g)
    v = torch.randn(b_, sk, hkv, d, generator=g)
    do = torch.randn(b_, sq, hq, d, generator=g)
    ref = {}
    for kind, f in (("true", true64), ("naive", naive64)):
        dq, dk, dv = oracle.bshd_backward(f(q), f(k), f(v), f(do), scale, segs, 0, True)
        ref[kind] = dict(dq=dq, dk=dk, dv=dv)
    dv_ = dev()
    qi, ki, vi, doi = (x.to(torch.bfloat16).to(dv_) for x in (q, k, v, do))
    say(f"d{d} fwd for determinism test")
    o, lse = cpa.forward(qi, ki, vi, scale=scale, q_segments=segs)
    p = dict(q=qi, k=ki, v=vi, do=doi, o=o, lse=lse, ref=ref)

    def run(ws=None):
        dq, dk, dv = _outputs(p)
        cpa.attn_bwd(qi, ki, vi, o, doi, lse, dq, dk, dv, scale=scale, q_segments=segs,
                     workspace=ws, flags=DETERMINISTIC)
        return dq, dk, dv

    say(f"d{d} bwd x3")
    first = run()
    _check(p, *first, f"d{d}_full")
    for _ in range(2):
        for a, b in zip(first, run()):
            assert torch.equal(_bits(a), _bits(b))
    least = cpa.bwd_workspace_bytes(qi, ki, vi, minimum=True)
    say(f"d{d} bwd in one-block bands")
    banded = run(torch.empty(least, dtype=torch.uint8, device=dv_))
    _check(p, *banded, f"d{d}_bands")
    assert torch.equal(_bits(first[1]), _bits(banded[1]))
    assert torch.equal(_bits(first[2]), _bits(banded[2]))


@pytest.mark.parametrize("dqk,dv,out", [(128, 128, torch.bfloat16), (192, 128, torch.bfloat16),
                                         (192, 128, torch.float32), (512, 512, torch.bfloat16)])
def test_single_pass_dq_matches_accumulated(dqk, dv, out):
    """With a workspace for every key block, attn_bwd (and the four steps
    given CPA_FLAG_DQ_DIRECT) let the dq kernel write dq itself: dq, dk, dv
    are bitwise those of the accumulating steps (pre clears the
    accumulator, dq adds dS K, post scales).  The keys start at position 200
    and the queries at 0, so rows 0..199 see no key and their dq must be
    written as exact zeros; every output starts as NaN."""
    b_, sq, sk, hq, hkv, kpb = 1, 300, 450, 4, 2, 200
    scale = 1.0 / math.sqrt(dqk)
    g = torch.Generator().manual_seed(31 + dqk + dv)
    d = dev()
    q, k, v, do = (torch.randn(*sh, generator=g).to(torch.bfloat16).to(d)
                   for sh in ((b_, sq, hq, dqk), (b_, sk, hkv, dqk), (b_, sk, hkv, dv),
                              (b_, sq, hq, dv)))
    say(f"single-pass dq d{dqk}/{dv} {out}: fwd")
    o, lse = cpa.forward(q, k, v, scale=scale, k_pos_begin=kpb)
    ws = torch.empty(cpa.bwd_workspace_bytes(q, k, v), dtype=torch.uint8, device=d)
    common = dict(scale=scale, k_pos_begin=kpb, workspace=ws)
    ints = torch.int32 if out == torch.float32 else torch.int16

    def nan_outputs():
        return tuple(torch.full(t.shape, float("nan"), dtype=out, device=d) for t in (q, k, v))

    say(f"single-pass dq d{dqk}/{dv} {out}: attn_bwd")
    ref = nan_outputs()
    cpa.attn_bwd(q, k, v, o, do, lse, *ref, **common)
    for flags in (0, cpa.CPA_FLAG_DQ_DIRECT):
        say(f"single-pass dq d{dqk}/{dv} {out}: four steps, flags {flags}")
        got = nan_outputs()
        for step in ("attn_bwd_pre", "attn_bwd_main", "attn_bwd_dq", "attn_bwd_post"):
            cpa.attn_bwd(q, k, v, o, do, lse, *got, step=step, flags=flags, **common)
        torch.cuda.synchronize()
        for name, x, y in zip(("dq", "dk", "dv"), ref, got):
            assert torch.equal(x.view(ints), y.view(ints)), (name, flags)
    assert not ref[0].isnan().any()
    assert (ref[0][:, :kpb] == 0).all() and (ref[0][:, kpb:] != 0).any()
