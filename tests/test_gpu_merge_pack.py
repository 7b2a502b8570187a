"""GPU LSE merge vs the fp64 oracle merge, and bit-exact pack/unpack vs the
oracle's byte layout.

Merge tolerance: the kernel combines fp32 inputs with two exp, one log and
three multiply-adds in fp32, so each output is within a few fp32 ulps of the
exact value: |dO| <= 4e-6 * (|o_acc| + |o_part|) and |dLSE| <= 4e-6 *
max(1, |LSE|).  Exact identities (an empty partial leaves the other operand
bitwise unchanged; all-empty gives (0, -inf)) are checked bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
from tests.gpu_util import bits, dev, say

pytestmark = pytest.mark.gpu

import bwd_causal_flash_amd as cpa  # noqa: E402


def _parts(seed, b=2, s=77, h=3, d=128, ninf_frac=0.1):
    g = torch.Generator().manual_seed(seed)
    oa = torch.randn(b, s, h, d, generator=g)
    op = torch.randn(b, s, h, d, generator=g)
    la = torch.randn(b, h, s, generator=g) * 3
    lp = torch.randn(b, h, s, generator=g) * 3
    ma = torch.rand(b, h, s, generator=g) < ninf_frac
    mp = torch.rand(b, h, s, generator=g) < ninf_frac
    la[ma] = -float("inf")
    lp[mp] = -float("inf")
    la[0, 0, :3] = -float("inf")
    lp[0, 0, :3] = -float("inf")          # both empty
    return oa, la, op, lp


def _oracle_merge(oa, la, op, lp):
    # oracle merge over [B, H, S, D] with lse [B, H, S]
    o, l = oracle.merge([(oa.permute(0, 2, 1, 3).double().numpy(), la.double().numpy()),
                         (op.permute(0, 2, 1, 3).double().numpy(), lp.double().numpy())])
    return o.transpose(0, 2, 1, 3), l


@pytest.mark.parametrize("d", [64, 128, 512])
def test_merge_matches_oracle(d):
    oa, la, op, lp = _parts(d, d=d)
    ro, rl = _oracle_merge(oa, la, op, lp)
    g = dev()
    oa_d, la_d, op_d, lp_d = (x.to(g) for x in (oa, la, op, lp))
    oo = torch.empty_like(oa_d)
    lo = torch.empty_like(la_d)
    say(f"merge d={d}")
    cpa.attn_merge_lse(oa_d, la_d, op_d, lp_d, oo, lo)
    torch.cuda.synchronize()
    got_o, got_l = oo.double().cpu().numpy(), lo.double().cpu().numpy()
    bound = 4e-6 * (np.abs(oa.double().numpy()) + np.abs(op.double().numpy()))
    assert np.all(np.abs(got_o - ro) <= bound + 1e-30)
    fin = np.isfinite(rl)
    assert np.array_equal(np.isneginf(got_l), np.isneginf(rl))
    assert np.all(np.abs(got_l[fin] - rl[fin]) <= 4e-6 * np.maximum(1, np.abs(rl[fin])))
    # empty partial: the other operand passes through bit for bit
    pe = torch.isneginf(lp) & torch.isfinite(la)
    pe_o = pe.permute(0, 2, 1)
    assert np.array_equal(bits(lo.cpu())[pe.numpy()], bits(la)[pe.numpy()])
    assert np.array_equal(bits(oo.cpu())[pe_o.numpy()], bits(oa)[pe_o.numpy()])
    both = torch.isneginf(lp) & torch.isneginf(la)
    assert torch.isneginf(lo.cpu()[both]).all()
    assert (oo.cpu()[both.permute(0, 2, 1)] == 0).all()


def test_merge_in_place_and_bf16_output():
    oa, la, op, lp = _parts(5, b=1, s=300, h=4, d=128)
    ro, rl = _oracle_merge(oa, la, op, lp)
    g = dev()
    oa_d, la_d, op_d, lp_d = (x.to(g) for x in (oa, la, op, lp))
    say("merge in place")
    cpa.attn_merge_lse(oa_d, la_d, op_d, lp_d)          # in place on the accumulator
    torch.cuda.synchronize()
    assert np.all(np.abs(oa_d.double().cpu().numpy() - ro) <=
                  4e-6 * (np.abs(oa.double().numpy()) + np.abs(op.double().numpy())) + 1e-30)
    # bf16 output from fp32 inputs = the fp32 result rounded once
    oa_d2, la_d2 = oa.to(g), la.to(g)
    ob = torch.empty(oa.shape, dtype=torch.bfloat16, device=g)
    lb = torch.empty_like(la_d2)
    say("merge bf16 out")
    cpa.attn_merge_lse(oa_d2, la_d2, op_d, lp_d, ob, lb)
    torch.cuda.synchronize()
    assert torch.equal(ob.cpu().view(torch.int16), oa_d.cpu().to(torch.bfloat16).view(torch.int16))


def _pack_inputs(seed, b=1, s=500, h=8, d=128, dtype=torch.bfloat16):
    g = torch.Generator().manual_seed(seed)
    o = torch.randint(-32768, 32767, (b, s, h, d), generator=g, dtype=torch.int32)
    if dtype == torch.bfloat16:
        o = o.to(torch.int16).view(torch.bfloat16)
    else:
        o = (o * 65537).view(torch.float32)
    lse_bits = torch.randint(-2**31, 2**31 - 1, (b, h, s), generator=g, dtype=torch.int64)
    lse_bits = lse_bits.to(torch.int32)
    lse_bits[0, 0, :4] = torch.tensor([0xFF800000 - 2**32, 0, -2**31, 0x7FC00123], dtype=torch.int32)
    return o, lse_bits.view(torch.float32)


@pytest.mark.parametrize("groups,dtype,force64", [(4, torch.bfloat16, False),
                                                   (4, torch.bfloat16, True),
                                                   (2, torch.float32, False),
                                                   (8, torch.bfloat16, False)])
def test_pack_matches_oracle_bytes_and_roundtrips(groups, dtype, force64):
    o, lse = _pack_inputs(groups, dtype=dtype)
    g = dev()
    o_d, l_d = o.to(g), lse.to(g)
    say(f"pack groups={groups} {dtype} force64={force64}")
    buf = cpa.pack_saved(o_d, l_d, groups, force_int64=force64)
    torch.cuda.synchronize()
    ob = o.view(torch.int16).numpy().view(np.uint16) if dtype == torch.bfloat16 else o.numpy()
    ref = oracle.pack_saved(ob, lse.numpy(), groups)
    got = buf.cpu().numpy()
    seg, obytes, loff = oracle.pack_layout(1, 500, 8, 128, o.element_size(), groups)
    assert got.size == ref.size
    for s in range(groups):        # compare payload bytes (pads are unspecified)
        a = s * seg
        assert np.array_equal(got[a:a + obytes], ref[a:a + obytes])
        n = 8 // groups * 500 * 4
        assert np.array_equal(got[a + loff:a + loff + n], ref[a + loff:a + loff + n])
    o2 = torch.empty_like(o_d)
    l2 = torch.empty_like(l_d)
    say("unpack")
    cpa.unpack_saved(buf, o2, l2, groups, force_int64=force64)
    torch.cuda.synchronize()
    assert np.array_equal(bits(o2), bits(o))
    assert np.array_equal(bits(l2), bits(lse))


def test_pack_strided_source_and_reused_allocation():
    """Source O is a strided view (a slice of a larger tensor); unpack lands
    in a reused allocation."""
    o, lse = _pack_inputs(9, s=300)
    g = dev()
    big = torch.zeros(1, 600, 8, 136, dtype=torch.bfloat16, device=g)
    view = big[:, 100:400, :, :128]
    view.copy_(o.to(g))
    lbig = torch.zeros(1, 8, 512, dtype=torch.float32, device=g)
    lview = lbig[:, :, 10:310]
    lview.copy_(lse.to(g))
    say("pack strided")
    buf = cpa.pack_saved(view, lview, 4)
    recv = torch.full_like(big, 7.0)
    lrecv = torch.full_like(lbig, 3.0)
    cpa.unpack_saved(buf, recv[:, 100:400, :, :128], lrecv[:, :, 10:310], 4)
    torch.cuda.synchronize()
    assert np.array_equal(bits(recv[:, 100:400, :, :128]), bits(o))
    assert np.array_equal(bits(lrecv[:, :, 10:310]), bits(lse))
    # bytes outside the views are untouched
    assert (recv[:, :100].float() == 7).all() and (recv[..., 128:].float() == 7).all()
    assert (lrecv[..., :10] == 3).all() and (lrecv[..., 310:] == 3).all()


def test_pack_beyond_2gib_takes_the_wide_path():
    """A 2.7 GB O (bf16 [1, 81920, 64, 256]) in 4 head groups: segment 3
    lies past byte 2^31 of the buffer, so pack_saved must take its 64-bit
    offset path on its own (PR 3510, Validation: both index widths, with a
    real large-stride case).  The buffer equals the oracle's byte layout and
    the round trip is exact."""
    b, s, h, d, groups = 1, 81920, 64, 256, 4
    g = dev()
    gen = torch.Generator(device=g).manual_seed(77)
    o_d = torch.randint(-32768, 32767, (b, s, h, d), generator=gen, device=g,
                        dtype=torch.int32).to(torch.int16).view(torch.bfloat16)
    l_d = torch.randint(-2**31, 2**31 - 1, (b, h, s), generator=gen, device=g,
                        dtype=torch.int64).to(torch.int32).view(torch.float32)
    seg, obytes, loff = oracle.pack_layout(b, s, h, d, 2, groups)
    assert groups * seg > 2**31 and 3 * seg < 2**31 < 3 * seg + obytes
    say("pack > 2 GiB")
    buf = cpa.pack_saved(o_d, l_d, groups)
    torch.cuda.synchronize()
    ref = oracle.pack_saved(o_d.view(torch.int16).cpu().numpy().view(np.uint16),
                            l_d.cpu().numpy(), groups)
    got = buf.cpu().numpy()
    assert got.size == ref.size
    n = h // groups * s * 4
    for sg in range(groups):
        a = sg * seg
        assert np.array_equal(got[a:a + obytes], ref[a:a + obytes]), sg
        assert np.array_equal(got[a + loff:a + loff + n], ref[a + loff:a + loff + n]), sg
    del ref, got
    o2 = torch.empty_like(o_d)
    l2 = torch.empty_like(l_d)
    say("unpack > 2 GiB")
    cpa.unpack_saved(buf, o2, l2, groups)
    torch.cuda.synchronize()
    assert torch.equal(o2.view(torch.int16), o_d.view(torch.int16))
    assert torch.equal(l2.view(torch.int32), l_d.view(torch.int32))
