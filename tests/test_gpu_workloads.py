"""The five workloads at full size on the GPU, in the launch configuration
the benchmark times, against the fp64 oracle on outputs it can compute in
seconds: whole heads (heads are independent), sampled query rows (a row's O,
LSE and dQ depend only on that row), the last keys (their dK/dV depend only
on the last rows under causal masking), and sum identities that hold at any
size.  Same criterion as the small tests (tests/criteria.py).

Workloads (workloads.CONFIGS): tiny (B1 H2 S256 D64 fp32), dense8k (B1 H32
S8192 D128), cp4_rank (one CP4 rank of a 32768-token sequence, D 192/128,
8 KV-block partials merged by LSE, then the backward, plus pack/unpack),
thd_gqa (packed THD, Hq32/Hkv8, D128), d512 (S16384 Hq16/Hkv4 D512).
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads
from tests import criteria
from tests.gpu_util import bits, dev, naive64, say, true64

pytestmark = pytest.mark.gpu

import bwd_causal_flash_amd as cpa  # noqa: E402
from bwd_causal_flash_amd.pipeline import RankStep, cp_chunks  # noqa: E402

BF = torch.bfloat16


def _report(name, log):
    print(name, {k: {kk: (round(vv, 4) if isinstance(vv, float) else vv)
                     for kk, vv in v.items()} for k, v in log.items()}, flush=True)


def _check_all(log, g, t, n, out_bf16, names=("o", "dq", "dk", "dv"), masks=None):
    masks = masks or {}
    for x in names:
        criteria.check(x, g[x], t[x], n[x], grad=(x != "o"), log=log, out_bf16=out_bf16,
                       mask=masks.get(x))


def test_tiny_fp32():
    w = workloads.CONFIGS["tiny"]
    x = workloads.draw_inputs(w)
    d = dev()
    qi, ki, vi, doi = (x[n].to(d) for n in ("q", "k", "v", "do"))
    say("tiny fwd/bwd")
    o, lse = cpa.forward(qi, ki, vi, scale=w.scale)
    dq, dk, dv = cpa.backward(qi, ki, vi, o, doi, lse, scale=w.scale)
    torch.cuda.synchronize()
    g = dict(o=o, dq=dq, dk=dk, dv=dv)
    ref = {}
    for kind, f in (("true", true64), ("naive", naive64)):
        a = [f(x[n]) for n in ("q", "k", "v", "do")]
        oo, ll = oracle.bshd_forward(a[0], a[1], a[2], w.scale)
        gq, gk, gv = oracle.bshd_backward(*a, w.scale)
        ref[kind] = dict(o=oo, lse=ll, dq=gq, dk=gk, dv=gv)
    log = {}
    _check_all(log, g, ref["true"], ref["naive"], out_bf16=False)
    criteria.check_lse("lse", lse, ref["true"]["lse"], ref["naive"]["lse"], log=log)
    _report("tiny", log)


def test_dense8k_heads():
    w = workloads.CONFIGS["dense8k"]
    x = workloads.draw_inputs(w)
    d = dev()
    qi, ki, vi, doi = (x[n].to(BF).to(d) for n in ("q", "k", "v", "do"))
    say("dense8k fwd/bwd")
    o, lse = cpa.forward(qi, ki, vi, scale=w.scale)
    dq, dk, dv = cpa.backward(qi, ki, vi, o, doi, lse, scale=w.scale)
    torch.cuda.synchronize()
    for h in (0, 31):
        sl = slice(h, h + 1)
        g = dict(o=o[0, :, sl], dq=dq[0, :, sl], dk=dk[0, :, sl], dv=dv[0, :, sl])
        ref = {}
        for kind, f in (("true", true64), ("naive", naive64)):
            a = [f(x[n][0, :, sl]) for n in ("q", "k", "v", "do")]
            oo, ll = oracle.forward(a[0], a[1], a[2], w.scale)
            gq, gk, gv = oracle.backward(*a, w.scale)
            ref[kind] = dict(o=oo, lse=ll, dq=gq, dk=gk, dv=gv)
        log = {}
        _check_all(log, g, ref["true"], ref["naive"], out_bf16=True)
        criteria.check_lse("lse", lse[0, sl], ref["true"]["lse"], ref["naive"]["lse"], log=log)
        _report(f"dense8k head {h}", log)


def test_cp4_rank_pipeline():
    """Nine (chunk, KV block) forward partials, seven of them merged by LSE
    into their chunk's accumulator in the forward epilogue, the backward over
    both chunks, and the pack/unpack round trip, exactly as the benchmark
    runs them; the merged forward agrees with partials + separate merges to
    one bf16 ulp, and the step matches the unsplit oracle on two heads."""
    w = workloads.CONFIGS["cp4_rank"]
    x = workloads.draw_inputs(w)
    d = dev()
    qi, ki, vi, doi = (x[n].to(BF).to(d) for n in ("q", "k", "v", "do"))
    chunks = cp_chunks(w.seqlen_k, w.cp, w.cp_rank)
    ru = RankStep(qi, ki, vi, doi, chunks, w.kv_blocks, scale=w.scale, pack_groups=w.cp,
                  fused_merge=False)
    assert ru.n_fwd_calls() == 9 and ru.n_merges() == 7
    say("cp4_rank forward partials + separate merges")
    ru.forward()
    rs = RankStep(qi, ki, vi, doi, chunks, w.kv_blocks, scale=w.scale, pack_groups=w.cp)
    assert rs.n_fwd_calls() == 9 and rs.n_merges() == 0
    say("cp4_rank forward partials merged in the epilogue")
    rs.forward()
    torch.cuda.synchronize()
    lf, lu = rs.lse.cpu().numpy(), ru.lse.cpu().numpy()
    assert float(np.max(np.abs(lf - lu))) <= 2e-6
    of, ou = rs.o.float().cpu().numpy(), ru.o.float().cpu().numpy()
    ulp = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(ou), 2.0 ** -126))) - 7)
    assert np.all(np.abs(of - ou) <= ulp + 2e-6)   # one bf16 ulp + fp32 reordering
    del ru
    say("cp4_rank pack/unpack")
    rs.pack_roundtrip()
    say("cp4_rank backward")
    rs.backward()
    torch.cuda.synchronize()
    assert np.array_equal(bits(rs.o_recv), bits(rs.o))
    assert np.array_equal(bits(rs.lse_recv), bits(rs.lse))
    segs = [(c[0], c[2]) for c in chunks]
    qp = oracle.positions_from_segments(w.seqlen_q, segs)
    # heads 7 and 30 (no GQA here: kv head = query head), whose key blocks
    # the key kernel runs on different XCDs
    for h in (7, 30):
        sl = slice(h, h + 1)
        ref = {}
        for kind, f in (("true", true64), ("naive", naive64)):
            a = [f(x[n][0, :, sl]) for n in ("q", "k", "v", "do")]
            oo, ll = oracle.forward(a[0], a[1], a[2], w.scale, qp)
            gq, gk, gv = oracle.backward(*a, w.scale, qp)
            ref[kind] = dict(o=oo, lse=ll, dq=gq, dk=gk, dv=gv)
        g = dict(o=rs.o[0, :, sl], dq=rs.dq[0, :, sl], dk=rs.dk[0, :, sl], dv=rs.dv[0, :, sl])
        log = {}
        _check_all(log, g, ref["true"], ref["naive"], out_bf16=True)
        criteria.check_lse("lse", rs.lse[0, sl], ref["true"]["lse"], ref["naive"]["lse"],
                           log=log)
        _report(f"cp4_rank head {h}", log)
        # keys beyond the last position any query holds get exact zeros:
        # none here (chunk 7 ends at 32767), but blocks only chunk 7 sees
        # must still be nonzero for this head
        assert float(rs.dk[0, 8192:, h].float().abs().max()) > 0


def test_thd_gqa_full():
    w = workloads.CONFIGS["thd_gqa"]
    x = workloads.draw_inputs(w)
    used, cu = x["seqused"], x["cu_seqlens"]
    d = dev()
    T = w.seqlen_q
    pad = np.concatenate([np.arange(cu[n] + used[n], cu[n + 1]) for n in range(len(used))]
                         ).astype(np.int64)
    qi, ki, vi, doi = (x[n].to(BF).to(d) for n in ("q", "k", "v", "do"))
    if pad.size:
        for t_ in (qi, ki, vi, doi):
            t_[pad] = float("nan")
    vl = cpa.Varlen(torch.tensor(cu, device=d), torch.tensor(cu, device=d),
                    torch.tensor(used, device=d), torch.tensor(used, device=d),
                    int(used.max()), int(used.max()))
    sent = lambda shape: torch.full(shape, 0x7FC1, dtype=torch.int16, device=d).view(BF)
    o = sent((T, w.heads_q, w.d_v))
    lse = torch.full((w.heads_q, T), 0x7FC00001, dtype=torch.int32, device=d).view(torch.float32)
    say("thd_gqa fwd")
    ws = cpa.attn_fwd(qi, ki, vi, o, lse, varlen=vl, scale=w.scale)
    dq, dk, dv = sent(qi.shape), sent(ki.shape), sent(vi.shape)
    say("thd_gqa bwd")
    ws2 = cpa.attn_bwd(qi, ki, vi, o, doi, lse, dq, dk, dv, varlen=vl, scale=w.scale)
    torch.cuda.synchronize()
    assert cpa.workspace_error_flag(ws) == 0 and cpa.workspace_error_flag(ws2) == 0
    if pad.size:
        for t_ in (o, dq, dk, dv):
            assert (bits(t_)[pad] == np.int16(0x7FC1)).all()
        assert (bits(lse)[:, pad] == np.int32(0x7FC00001)).all()
    # q-head 0 over every document: O, LSE, dQ
    ref = {}
    for kind, f in (("true", true64), ("naive", naive64)):
        a = [f(x[n][:, :1]) for n in ("q", "k", "v", "do")]   # q-head 0 reads kv-head 0
        oo, ll = oracle.thd_forward(a[0], a[1], a[2], w.scale, cu, cu, used, used)
        gq, _, _ = oracle.thd_backward(*a, w.scale, cu, cu, used, used)
        ref[kind] = dict(o=oo, lse=ll, dq=gq)
    real = np.ones(T, bool)
    real[pad] = False
    m = np.broadcast_to(real[:, None, None], (T, 1, w.d_v))
    g = dict(o=o[:, :1], dq=dq[:, :1])
    log = {}
    _check_all(log, g, ref["true"], ref["naive"], out_bf16=True, names=("o", "dq"),
               masks={"o": m, "dq": m})
    criteria.check_lse("lse", lse[:1], ref["true"]["lse"], ref["naive"]["lse"],
                       mask=np.broadcast_to(real[None], (1, T)), log=log)
    # kv-head 1 (q heads 4..7) over every document: dK, dV
    refk = {}
    for kind, f in (("true", true64), ("naive", naive64)):
        a = [f(x[nm][:, sl]) for nm, sl in (("q", slice(4, 8)), ("k", slice(1, 2)),
                                            ("v", slice(1, 2)), ("do", slice(4, 8)))]
        _, gk, gv = oracle.thd_backward(*a, w.scale, cu, cu, used, used)
        refk[kind] = dict(dk=gk, dv=gv)
    gk = dict(dk=dk[:, 1:2], dv=dv[:, 1:2])
    _check_all(log, gk, refk["true"], refk["naive"], out_bf16=True, names=("dk", "dv"),
               masks={"dk": m, "dv": m})
    _report("thd_gqa", log)


def test_d512_sampled():
    w = workloads.CONFIGS["d512"]
    x = workloads.draw_inputs(w)
    d = dev()
    qi, ki, vi, doi = (x[n].to(BF).to(d) for n in ("q", "k", "v", "do"))
    say("d512 fwd/bwd")
    o, lse = cpa.forward(qi, ki, vi, scale=w.scale)
    dq, dk, dv = cpa.backward(qi, ki, vi, o, doi, lse, scale=w.scale)
    torch.cuda.synchronize()
    S = w.seqlen_q
    rows = np.concatenate([np.arange(0, 48), np.arange(8150, 8198), np.arange(S - 64, S)])
    ref = {}
    for kind, f in (("true", true64), ("naive", naive64)):
        a = [f(x[n][0]) for n in ("q", "k", "v", "do")]
        oo, ll = oracle.forward_rows(a[0], a[1], a[2], w.scale, rows)
        gq, _, _ = oracle.backward(a[0][rows], a[1], a[2], a[3][rows], w.scale, q_pos=rows)
        ref[kind] = dict(o=oo, lse=ll, dq=gq)
    g = dict(o=o[0, rows], dq=dq[0, rows])
    log = {}
    _check_all(log, g, ref["true"], ref["naive"], out_bf16=True, names=("o", "dq"))
    criteria.check_lse("lse", lse[0][:, rows], ref["true"]["lse"], ref["naive"]["lse"], log=log)
    # dK, dV of the last 2048 keys of kv head 2 (query heads 8..11): only
    # rows >= S-2048 see them, so the oracle over those rows gives them
    # exactly; they span 16 key blocks and 32 query tiles of the dK/dV kernel
    n = 2048
    r = np.arange(S - n, S)
    refk = {}
    for kind, f in (("true", true64), ("naive", naive64)):
        a = [f(x[nm][0][:, sl]) for nm, sl in (("q", slice(8, 12)), ("k", slice(2, 3)),
                                               ("v", slice(2, 3)), ("do", slice(8, 12)))]
        _, gk, gv = oracle.backward(a[0][r], a[1], a[2], a[3][r], w.scale, q_pos=r)
        refk[kind] = dict(dk=gk[S - n:], dv=gv[S - n:])
    gk = dict(dk=dk[0, S - n:, 2:3], dv=dv[0, S - n:, 2:3])
    _check_all(log, gk, refk["true"], refk["naive"], out_bf16=True, names=("dk", "dv"))
    # identities at full size: sum_j dK_j = 0; sum_j dV_j = sum_i dO_i per group
    dk64 = dk[0].double()
    dv64 = dv[0].double()
    g_ = w.heads_q // w.heads_kv
    assert float(dk64.sum(0).abs().max()) <= 1e-3 * float(dk64.abs().sum(0).max())
    dosum = doi[0].double().view(S, w.heads_kv, g_, w.d_v).sum(dim=(0, 2))
    assert float((dv64.sum(0) - dosum).abs().max()) <= 1e-3 * float(dv64.abs().sum(0).max())
    _report("d512", log)
