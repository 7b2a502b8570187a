"""Forward merged into a running accumulator (attn_fwd_accum) on the GPU.

The LSE merge of ring-step partials (PR 3527, context-parallel commits: each
step's partial is corrected by its LSE and folded into the running result)
done in the forward kernel's epilogue must give what attn_fwd followed by
attn_merge_lse gives, and both must match the oracle run on all keys at
once.  Cases: GQA with a ragged query tile, the dual-chunk positions of a CP
rank with the 192/128 head dims, the 512 head dim (two output column chunks
per query tile, so the LSE cannot be updated in place), and rows that see no
key of the accumulated block or none at all.
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

# name, Sq, Sk, Hq, Hkv, Dqk, Dv, key blocks, query segments
CASES = [
    ("d128_gqa_3blocks", 300, 384, 4, 2, 128, 128, 3, None),
    ("d192_dual_chunk_4blocks", 256, 1024, 4, 4, 192, 128, 4, [(0, 0), (128, 896)]),
    ("d512_2blocks", 200, 256, 4, 2, 512, 512, 2, None),
]


def _draw(sq, sk, hq, hkv, dqk, dv, seed):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(1, sq, hq, dqk, generator=g), torch.randn(1, sk, hkv, dqk, generator=g),
            torch.randn(1, sk, hkv, dv, generator=g))


def _bf16_ulp(x: np.ndarray) -> np.ndarray:
    a = np.abs(x)
    return np.where(a > 0, 2.0 ** (np.floor(np.log2(np.where(a > 0, a, 1.0))) - 7), 2.0 ** -133)


def _run(qi, ki, vi, nb, segs, scale, fused):
    """Blocks in order; returns the final bf16 O and the LSE."""
    d = qi.device
    sq, hq, dv = qi.shape[1], qi.shape[2], vi.shape[-1]
    blk = ki.shape[1] // nb
    kb = lambda j: (ki[:, j * blk:(j + 1) * blk], vi[:, j * blk:(j + 1) * blk])
    kw = dict(causal=True, scale=scale, q_segments=segs)
    o_acc = torch.empty(1, sq, hq, dv, dtype=torch.float32, device=d)
    lse_acc = torch.empty(1, hq, sq, dtype=torch.float32, device=d)
    lse_alt = torch.empty_like(lse_acc)   # ping-pong when LSE cannot be in place
    o = torch.empty(1, sq, hq, dv, dtype=torch.bfloat16, device=d)
    lse = torch.empty_like(lse_acc)
    cpa.attn_fwd(qi, *kb(0), o_acc, lse_acc, k_pos_begin=0, **kw)
    for j in range(1, nb):
        last = j == nb - 1
        if fused:
            lse_out = lse if last else (lse_acc if dv <= 256 else lse_alt)
            cpa.attn_fwd(qi, *kb(j), o if last else o_acc, lse_out, k_pos_begin=j * blk,
                         acc=(o_acc, lse_acc), **kw)
            if not last and lse_out is not lse_acc:
                lse_acc, lse_alt = lse_out, lse_acc
        else:
            o_p = torch.empty_like(o_acc)
            l_p = torch.empty_like(lse_acc)
            cpa.attn_fwd(qi, *kb(j), o_p, l_p, k_pos_begin=j * blk, **kw)
            cpa.attn_merge_lse(o_acc, lse_acc, o_p, l_p, o if last else o_acc,
                               lse if last else lse_acc)
    torch.cuda.synchronize()
    return o, lse


@pytest.mark.parametrize("case", CASES, ids=lambda c: c[0])
def test_accum_matches_fwd_then_merge_and_oracle(case):
    name, sq, sk, hq, hkv, dqk, dv, nb, segs = case
    q, k, v = _draw(sq, sk, hq, hkv, dqk, dv, 700 + CASES.index(case))
    d = dev()
    qi, ki, vi = (x.to(torch.bfloat16).to(d) for x in (q, k, v))
    scale = 1.0 / math.sqrt(dqk)
    say(f"fwd_accum {name} fused")
    o_f, l_f = _run(qi, ki, vi, nb, segs, scale, True)
    say(f"fwd_accum {name} fwd + merge")
    o_u, l_u = _run(qi, ki, vi, nb, segs, scale, False)
    # The same fp32 arithmetic up to the order of one product: the fused path
    # scales the block's unnormalised O by (weight * 1/l), the separate merge
    # by weight after normalising.  Before the final bf16 rounding the two
    # differ by a few fp32 roundings of the operands, <= 2^-22 (|O_acc| +
    # |O_blk|) <= 2e-6 here (|O| < 4), so the bf16 outputs agree to one ulp
    # of the result plus that.
    lf, lu = l_f.cpu().numpy(), l_u.cpu().numpy()
    assert np.array_equal(np.isinf(lf), np.isinf(lu))
    fin = np.isfinite(lu)
    assert float(np.max(np.abs(lf[fin] - lu[fin]), initial=0.0)) <= 2e-6
    of, ou = o_f.float().cpu().numpy(), o_u.float().cpu().numpy()
    assert np.all(np.abs(of - ou) <= _bf16_ulp(ou) + 2e-6)
    # and the oracle on all keys at once
    ref = {}
    for kind, f in (("true", true64), ("naive", naive64)):
        ref[kind] = oracle.bshd_forward(f(q), f(k), f(v), scale, segs, 0, True)
    log = {}
    criteria.check("O", o_f, ref["true"][0], ref["naive"][0], log=log, out_bf16=True)
    criteria.check_lse("LSE", l_f, ref["true"][1], ref["naive"][1], log=log)
    print(name, {k_: round(v_["ratio"], 3) for k_, v_ in log.items() if "ratio" in v_})


def test_accum_keyless_rows_and_block_order():
    """Keys [0, 200) in two blocks, accumulated in reverse order (block 1,
    then block 0 merged in place, fp32).  Query rows 0..49 have positions
    -50..-1 and see no key at all: O = 0, LSE = -inf.  Rows whose position is
    below 100 see nothing of block 1, so the merge must return block 0's
    partial bit for bit; the rest must match the oracle."""
    sq, sk, h, dd = 200, 200, 2, 128
    segs = [(0, -50), (50, 0)]
    q, k, v = _draw(sq, sk, h, h, dd, dd, 777)
    d = dev()
    qi, ki, vi = (x.to(torch.bfloat16).to(d) for x in (q, k, v))
    scale = 1.0 / math.sqrt(dd)
    kw = dict(causal=True, scale=scale, q_segments=segs)
    acc_o = torch.empty(1, sq, h, dd, dtype=torch.float32, device=d)
    acc_l = torch.empty(1, h, sq, dtype=torch.float32, device=d)
    say("fwd_accum keyless: block 1 then block 0 in place")
    cpa.attn_fwd(qi, ki[:, 100:], vi[:, 100:], acc_o, acc_l, k_pos_begin=100, **kw)
    cpa.attn_fwd(qi, ki[:, :100], vi[:, :100], acc_o, acc_l, k_pos_begin=0,
                 acc=(acc_o, acc_l), **kw)
    b0_o = torch.empty_like(acc_o)
    b0_l = torch.empty_like(acc_l)
    cpa.attn_fwd(qi, ki[:, :100], vi[:, :100], b0_o, b0_l, k_pos_begin=0, **kw)
    torch.cuda.synchronize()
    o, l = acc_o.cpu(), acc_l.cpu()
    assert torch.all(o[0, :50] == 0) and torch.all(torch.isneginf(l[0, :, :50]))
    only0 = slice(50, 150)   # positions 0..99
    assert np.array_equal(bits(o[0, only0]), bits(b0_o[0, only0]))
    assert np.array_equal(bits(l[0, :, only0]), bits(b0_l[0, :, only0]))
    ref = {}
    for kind, f in (("true", true64), ("naive", naive64)):
        ref[kind] = oracle.bshd_forward(f(q), f(k), f(v), scale, segs, 0, True)
    rows = np.zeros((1, sq, h), dtype=bool)
    rows[0, 150:] = True
    log = {}
    criteria.check("O", acc_o, ref["true"][0], ref["naive"][0], log=log,
                   mask=np.broadcast_to(rows[..., None], (1, sq, h, dd)))
    criteria.check_lse("LSE", acc_l, ref["true"][1], ref["naive"][1], log=log,
                       mask=np.transpose(rows, (0, 2, 1)))
    print("keyless", {k_: round(v_["ratio"], 3) for k_, v_ in log.items() if "ratio" in v_})


def test_accum_rejects_in_place_lse_at_512():
    q, k, v = _draw(64, 64, 2, 2, 512, 512, 778)
    d = dev()
    qi, ki, vi = (x.to(torch.bfloat16).to(d) for x in (q, k, v))
    o = torch.zeros(1, 64, 2, 512, dtype=torch.float32, device=d)
    l = torch.zeros(1, 2, 64, dtype=torch.float32, device=d)
    with pytest.raises(cpa.CpaError) as e:
        cpa.attn_fwd(qi, ki, vi, o, l, acc=(o, l))
    assert e.value.name == "CPA_ERR_OVERLAP"
