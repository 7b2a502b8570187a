"""Exchange buffers on the GPU (xchg_pack / xchg_unpack through the C ABI).

* bit-exact against the oracle's byte layout (oracle/xchg.py) for bf16 and
  fp32 row fields and an LSE field holding NaN payloads, -0, -inf and
  denormals, with several row ranges per segment and split and unsplit
  fields; pad bytes untouched; unpack restores every covered element and
  leaves the rest alone;
* the head-parallel backward of PR 3510 ("Add head-parallel FA4 backward
  for cuDNN CP attention", Diagram) on CP = 4 simulated dual-chunk ranks:
  Q, K, V, O, dO, LSE go seq -> heads through one packed buffer per rank
  (the all-to-all itself is simulated by segment copies), every head group
  runs a full-sequence backward, dQ, dK, dV come back heads -> seq; the
  exchanged tensors are checked bit for bit by direct slicing and the
  gradients against the fp64 oracle with the accuracy criterion.
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


def _rand_bits(g, shape, dtype, d):
    if dtype == torch.bfloat16:
        x = torch.randint(-2**15, 2**15, shape, generator=g, dtype=torch.int16)
        return x.view(torch.bfloat16).to(d)
    x = torch.randint(-2**31, 2**31 - 1, shape, generator=g, dtype=torch.int32)
    return x.view(torch.float32).to(d)


def _np_bits(x):
    x = x.cpu()
    return x.view(torch.int16).numpy().view(np.uint16) if x.dtype == torch.bfloat16 \
        else x.view(torch.int32).numpy().view(np.uint32).view(np.float32)


def _fields(ts, split):
    out = []
    for t, sp in zip(ts, split):
        if t.dim() == 4:
            out.append(dict(kind="rows", heads=t.shape[2], dim=t.shape[3],
                            elem_bytes=t.element_size(), split=sp))
        else:
            out.append(dict(kind="lse", heads=t.shape[1], dim=1, elem_bytes=4, split=sp))
    return out


def test_pack_matches_oracle_bytes_and_unpack_restores():
    d = dev()
    g = torch.Generator().manual_seed(17)
    b, r = 2, 77
    a = _rand_bits(g, (b, r, 4, 64), torch.bfloat16, d)
    f32 = _rand_bits(g, (b, r, 2, 12), torch.float32, d)
    lse = _rand_bits(g, (b, 4, r), torch.float32, d)
    lse.view(torch.int32)[0, 0, :4] = torch.tensor([-8388608, -2**31, 0x7FC00123, 1],
                                                   dtype=torch.int32, device=d)
    # a strided view for the first field (every other head of a wider tensor)
    wide = _rand_bits(g, (b, r, 8, 64), torch.bfloat16, d)
    wide[:, :, ::2] = a
    a_view = wide[:, :, ::2]
    ts, split = [a_view, f32, lse], [True, False, True]
    ranges = [[(0, 77)], [(40, 37), (0, 40)], [(5, 3), (70, 7), (8, 62), (0, 5)], [(0, 77)]]
    ref = oracle.xchg_pack([_np_bits(a), _np_bits(f32), _np_bits(lse)], 4, ranges,
                           _fields([a, f32, lse], split), b)
    buf = torch.zeros(ref.size, dtype=torch.uint8, device=d)
    say("xchg pack vs oracle bytes")
    cpa.xchg_pack(ts, groups=4, ranges=ranges, split=split, buf=buf)
    torch.cuda.synchronize()
    assert np.array_equal(buf.cpu().numpy(), ref)
    outs = [torch.full_like(a, 7.0), torch.full_like(f32, 7.0), torch.full_like(lse, 7.0)]
    say("xchg unpack")
    cpa.xchg_unpack(buf, outs, groups=4, ranges=ranges, split=split)
    torch.cuda.synchronize()
    for x, y in zip((a, f32, lse), outs):
        assert torch.equal(x.view(torch.int16 if x.element_size() == 2 else torch.int32),
                           y.view(torch.int16 if y.element_size() == 2 else torch.int32))
    # rows no segment covers stay as they were
    part = [torch.full_like(a, 7.0)]
    cpa.xchg_unpack(cpa.xchg_pack([a], groups=1, ranges=[[(10, 5)]], split=[False]), part,
                    groups=1, ranges=[[(10, 5)]], split=[False])
    torch.cuda.synchronize()
    assert torch.equal(part[0][:, 10:15].view(torch.int16), a[:, 10:15].view(torch.int16))
    assert (part[0][:, :10] == 7).all() and (part[0][:, 15:] == 7).all()


def _a2a(sends, offs):
    n = len(sends)
    return [torch.cat([sends[r][offs[r][g]:offs[r][g + 1]] for r in range(n)]) for g in range(n)]


def test_head_parallel_backward_cp4():
    d = dev()
    cp, c, hq, hkv, dqk, dv = 4, 256, 8, 4, 192, 128
    total = 2 * cp * c
    hg, hkg = hq // cp, hkv // cp
    g = torch.Generator().manual_seed(23)
    q = torch.randn(1, total, hq, dqk, generator=g)
    k = torch.randn(1, total, hkv, dqk, generator=g)
    v = torch.randn(1, total, hkv, dv, generator=g)
    do = torch.randn(1, total, hq, dv, generator=g)
    scale = 1.0 / math.sqrt(dqk)
    Q, K, V, DO = (x.to(torch.bfloat16).to(d) for x in (q, k, v, do))
    say("head-parallel: full forward (saved O, LSE)")
    O, LSE = cpa.forward(Q, K, V, scale=scale)
    chunks = [[(r * c, c), ((2 * cp - 1 - r) * c, c)] for r in range(cp)]
    rows_of = [torch.cat([torch.arange(a0, a0 + n) for a0, n in ch]).to(d) for ch in chunks]
    local = [dict(q=Q[:, rw].contiguous(), k=K[:, rw].contiguous(), v=V[:, rw].contiguous(),
                  o=O[:, rw].contiguous(), do=DO[:, rw].contiguous(),
                  lse=LSE[:, :, rw].contiguous()) for rw in rows_of]
    names = ("q", "k", "v", "o", "do", "lse")
    every = [[(0, 2 * c)]] * cp
    say("head-parallel: pack seq -> heads")
    sends = [cpa.xchg_pack([x[n] for n in names], groups=cp, ranges=every, split=True)
             for x in local]
    offs = [cpa.xchg_offsets(cpa.xchg_desc([x[n] for n in names], groups=cp, ranges=every,
                                           split=True)) for x in local]
    recvs = _a2a(sends, offs)
    hp = []
    for gi in range(cp):
        dst = dict(q=torch.empty(1, total, hg, dqk, dtype=torch.bfloat16, device=d),
                   k=torch.empty(1, total, hkg, dqk, dtype=torch.bfloat16, device=d),
                   v=torch.empty(1, total, hkg, dv, dtype=torch.bfloat16, device=d),
                   o=torch.empty(1, total, hg, dv, dtype=torch.bfloat16, device=d),
                   do=torch.empty(1, total, hg, dv, dtype=torch.bfloat16, device=d),
                   lse=torch.empty(1, hg, total, dtype=torch.float32, device=d))
        say(f"head-parallel: unpack on head group {gi}")
        cpa.xchg_unpack(recvs[gi], [dst[n] for n in names], groups=cp, ranges=chunks, split=False)
        hs, ks = slice(gi * hg, (gi + 1) * hg), slice(gi * hkg, (gi + 1) * hkg)
        for n, full, sl in (("q", Q, hs), ("k", K, ks), ("v", V, ks), ("o", O, hs), ("do", DO, hs)):
            assert torch.equal(dst[n].view(torch.int16), full[:, :, sl].view(torch.int16)), n
        assert torch.equal(dst["lse"].view(torch.int32), LSE[:, hs].contiguous().view(torch.int32))
        say(f"head-parallel: full-sequence backward on head group {gi}")
        dq, dk, dv_ = cpa.backward(dst["q"], dst["k"], dst["v"], dst["o"], dst["do"], dst["lse"],
                                   scale=scale)
        hp.append(dict(dq=dq, dk=dk, dv=dv_))
    grads = ("dq", "dk", "dv")
    say("head-parallel: pack heads -> seq")
    back_send = [cpa.xchg_pack([hp[gi][n] for n in grads], groups=cp, ranges=chunks, split=False)
                 for gi in range(cp)]
    back_offs = [cpa.xchg_offsets(cpa.xchg_desc([hp[gi][n] for n in grads], groups=cp,
                                                ranges=chunks, split=False)) for gi in range(cp)]
    back = _a2a(back_send, back_offs)
    full_grads = dict(dq=torch.empty_like(Q), dk=torch.empty_like(K), dv=torch.empty_like(V))
    for r in range(cp):
        mine = dict(dq=torch.empty_like(local[r]["q"]), dk=torch.empty_like(local[r]["k"]),
                    dv=torch.empty_like(local[r]["v"]))
        say(f"head-parallel: unpack on rank {r}")
        cpa.xchg_unpack(back[r], [mine[n] for n in grads], groups=cp, ranges=every, split=True)
        for n in grads:
            direct = torch.cat([hp[gi][n][:, rows_of[r]] for gi in range(cp)], dim=2)
            assert torch.equal(mine[n].view(torch.int16), direct.view(torch.int16)), n
            full_grads[n][:, rows_of[r]] = mine[n]
    torch.cuda.synchronize()
    ref = {}
    for kind, f in (("true", true64), ("naive", naive64)):
        dq, dk, dv_ = oracle.bshd_backward(f(q), f(k), f(v), f(do), scale)
        ref[kind] = dict(dq=dq, dk=dk, dv=dv_)
    log = {}
    for n in grads:
        criteria.check(n, full_grads[n], ref["true"][n], ref["naive"][n], grad=True, log=log,
                       out_bf16=True)
    print("head-parallel", {k_: round(v_["ratio"], 3) for k_, v_ in log.items()})
