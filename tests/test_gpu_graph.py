"""HIP-graph capture of whole steps, replayed with changed inputs.

The library allocates nothing, keeps no per-call state and makes no host
synchronisation, and its metadata stays on the device, so a caller can
capture a step once and replay it (PR 3510 "Add head-parallel FA4 backward
for cuDNN CP attention", Validation: changed-input graph replay; PR 3699 "Add
cuDNN OSS backward dispatch for context parallel attention", Dependencies
and use: warm each call up before capture).  Each replay runs after eager
work and a synchronisation, with new input contents copied into the
captured tensors, and must equal the eager step bit for bit; a second graph
captured on other tensors (other addresses) must too.  Nothing in the
captured region clears memory with a memset: the kernels write every byte
they later read.
"""
import pytest
import torch

from tests.gpu_util import dev, say

pytestmark = pytest.mark.gpu

import bwd_causal_flash_amd as cpa  # noqa: E402
from bwd_causal_flash_amd.pipeline import RankStep, cp_chunks  # noqa: E402

BF = torch.bfloat16


def _same(a, b):
    return torch.equal(a.contiguous().view(torch.uint8), b.contiguous().view(torch.uint8))


def _capture(fn):
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for _ in range(2):        # warm up every call before capture
            fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def _replays(g, inputs, draws, outputs, expect):
    """Replay ``g`` once per draw (in an order that changes every time),
    copying the draw into ``inputs`` first and doing eager work and a
    synchronisation in between; compare every replay with ``expect``."""
    for n, i in enumerate([1, 0, 1, 0]):
        for dst, src in zip(inputs, draws[i]):
            dst.copy_(src)
        junk = torch.randn(1 << 20, device=inputs[0].device).sum()   # eager work
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert float(junk) == float(junk)
        for name, t in outputs().items():
            assert _same(t, expect[i][name]), f"replay {n} (draw {i}): {name} differs from eager"


def test_cp4_rank_step_graph_replay():
    """The whole cp4_rank step (9 forward partials, 7 of them merged in the
    epilogue, pack/unpack, backward) at its full size."""
    d = dev()
    S, cp, H, dqk, dv = 32768, 4, 32, 192, 128
    gens = [torch.Generator(device=d).manual_seed(s) for s in (21, 22)]
    draws = [[torch.randn(1, n, H, dd, device=d, generator=g).to(BF)
              for n, dd in ((8192, dqk), (S, dqk), (S, dv), (8192, dv))] for g in gens]
    chunks = cp_chunks(S, cp, 0)
    q, k, v, do = (t.clone() for t in draws[0])
    rs = RankStep(q, k, v, do, chunks, 8, pack_groups=cp)
    names = ("o", "lse", "dq", "dk", "dv", "o_recv", "lse_recv")
    outputs = lambda: {n: getattr(rs, n) for n in names}   # noqa: E731
    expect = []
    for i in (0, 1):
        for dst, src in zip((q, k, v, do), draws[i]):
            dst.copy_(src)
        say(f"cp4_rank eager step, draw {i}")
        rs.step()
        torch.cuda.synchronize()
        expect.append({n: t.clone() for n, t in outputs().items()})
    assert not _same(expect[0]["dq"], expect[1]["dq"])
    say("cp4_rank step: capture")
    g = _capture(lambda: rs.step())
    say("cp4_rank step: replays with changed inputs")
    _replays(g, (q, k, v, do), draws, outputs, expect)
    del g
    # a second graph on other tensors: other input and output addresses
    q2, k2, v2, do2 = (t.clone() for t in draws[1])
    rs2 = RankStep(q2, k2, v2, do2, chunks, 8, pack_groups=cp)
    say("cp4_rank step: capture on new addresses")
    g2 = _capture(lambda: rs2.step())
    _replays(g2, (q2, k2, v2, do2), draws, lambda: {n: getattr(rs2, n) for n in names}, expect)


def test_thd_fwd_bwd_graph_replay():
    """Packed THD (documents of 1000, 64, 0 and 300 rows at a 64-row pitch)
    GQA forward + backward; the metadata flags stay zero on every replay."""
    d = dev()
    used = torch.tensor([1000, 64, 0, 300], dtype=torch.int32)
    phys = [(int(u) + 63) // 64 * 64 or 64 for u in used]
    cu = torch.tensor([0] + list(torch.tensor(phys).cumsum(0)), dtype=torch.int32)
    T, hq, hkv, dd = int(cu[-1]), 8, 2, 128
    gens = [torch.Generator(device=d).manual_seed(s) for s in (31, 32)]
    draws = [[torch.randn(T, h, dd, device=d, generator=g).to(BF) for h in (hq, hkv, hkv, hq)]
             for g in gens]
    q, k, v, do = (t.clone() for t in draws[0])
    vl = cpa.Varlen(cu.to(d), cu.to(d), used.to(d), used.to(d), int(used.max()), int(used.max()))
    o = torch.zeros(T, hq, dd, dtype=BF, device=d)
    lse = torch.zeros(hq, T, device=d)
    dq, dk, dv = torch.zeros_like(q), torch.zeros_like(k), torch.zeros_like(v)
    fws = torch.empty(256, dtype=torch.uint8, device=d)
    bws = torch.empty(cpa.bwd_workspace_bytes(q, k, v, varlen=vl), dtype=torch.uint8, device=d)

    def step():
        cpa.attn_fwd(q, k, v, o, lse, varlen=vl, workspace=fws)
        cpa.attn_bwd(q, k, v, o, do, lse, dq, dk, dv, varlen=vl, workspace=bws)

    outputs = lambda: dict(o=o, lse=lse, dq=dq, dk=dk, dv=dv)   # noqa: E731
    expect = []
    for i in (0, 1):
        for dst, src in zip((q, k, v, do), draws[i]):
            dst.copy_(src)
        say(f"thd eager fwd+bwd, draw {i}")
        step()
        torch.cuda.synchronize()
        expect.append({n: t.clone() for n, t in outputs().items()})
    say("thd fwd+bwd: capture and replays")
    g = _capture(step)
    _replays(g, (q, k, v, do), draws, outputs, expect)
    assert cpa.workspace_error_flag(fws) == 0 and cpa.workspace_error_flag(bws) == 0
