"""The Python binding refuses tensors that do not match the problem before
it calls the C library (which sees only pointers and sizes and so could not
tell): wrong shapes, dtypes, LSE layout, varlen metadata, and tensors that
are not on the GPU.  Run on the CPU with CPU tensors: shape and dtype
checks come first, the device check last, so every case below raises in
Python and nothing reaches the library."""
import pytest
import torch

import bwd_causal_flash_amd as cpa

BF = torch.bfloat16


def bshd(b=1, sq=64, sk=64, hq=4, hkv=2, dqk=128, dv=128, dt=BF):
    q = torch.zeros(b, sq, hq, dqk, dtype=dt)
    k = torch.zeros(b, sk, hkv, dqk, dtype=dt)
    v = torch.zeros(b, sk, hkv, dv, dtype=dt)
    o = torch.zeros(b, sq, hq, dv, dtype=dt)
    lse = torch.zeros(b, hq, sq, dtype=torch.float32)
    return q, k, v, o, lse


def thd(t=128, hq=4, hkv=2, d=128, nseq=2):
    q = torch.zeros(t, hq, d, dtype=BF)
    k = torch.zeros(t, hkv, d, dtype=BF)
    v = torch.zeros(t, hkv, d, dtype=BF)
    o = torch.zeros(t, hq, d, dtype=BF)
    lse = torch.zeros(hq, t, dtype=torch.float32)
    cu = torch.tensor([0, 64, 128], dtype=torch.int32)[: nseq + 1]
    used = torch.tensor([60, 64], dtype=torch.int32)[:nseq]
    vl = cpa.Varlen(cu, cu.clone(), used, used.clone(), 64, 64)
    return q, k, v, o, lse, vl


def test_fwd_declines():
    q, k, v, o, lse = bshd()
    with pytest.raises(TypeError, match="k: dtype"):
        cpa.attn_fwd(q, k.float(), v, o, lse)
    with pytest.raises(TypeError, match="v: dtype"):
        cpa.attn_fwd(q, k, v.half(), o, lse)
    with pytest.raises(TypeError, match="lse: dtype"):
        cpa.attn_fwd(q, k, v, o, lse.to(BF))
    with pytest.raises(ValueError, match="lse: shape"):
        cpa.attn_fwd(q, k, v, o, lse.transpose(1, 2).contiguous())
    with pytest.raises(ValueError, match="o: shape"):
        cpa.attn_fwd(q, k, v, o[:, :32], lse)
    with pytest.raises(ValueError, match="k: shape"):
        cpa.attn_fwd(q, k[..., :64], v, o, lse)
    with pytest.raises(ValueError, match="v: shape"):
        cpa.attn_fwd(q, k, v[:, :32], o, lse)
    with pytest.raises(ValueError, match="k: shape"):
        cpa.attn_fwd(q, torch.cat([k, k]), v, o, lse)            # batch mismatch
    with pytest.raises(ValueError, match="o_acc: shape"):
        cpa.attn_fwd(q, k, v, o.float(), lse, acc=(o[:, :3].float(), lse))
    with pytest.raises(TypeError, match="workspace: dtype"):
        cpa.attn_fwd(q, k, v, o, lse, workspace=torch.zeros(256, dtype=torch.int32))
    # everything consistent, but on the host: refused before any pointer is passed
    with pytest.raises(ValueError, match="must be on a GPU"):
        cpa.attn_fwd(q, k, v, o, lse)


def test_fwd_thd_varlen_declines():
    q, k, v, o, lse, vl = thd()
    bad = cpa.Varlen(vl.cu_seqlens_q.long(), vl.cu_seqlens_k, vl.seqused_q, vl.seqused_k, 64, 64)
    with pytest.raises(TypeError, match="cu_seqlens_q: dtype"):
        cpa.attn_fwd(q, k, v, o, lse, varlen=bad)
    bad = cpa.Varlen(vl.cu_seqlens_q[:2], vl.cu_seqlens_k, vl.seqused_q, vl.seqused_k, 64, 64)
    with pytest.raises(ValueError, match="cu_seqlens_q: shape"):
        cpa.attn_fwd(q, k, v, o, lse, varlen=bad)
    bad = cpa.Varlen(vl.cu_seqlens_q, vl.cu_seqlens_k, vl.seqused_q, vl.seqused_k[:1], 64, 64)
    with pytest.raises(ValueError, match="seqused_k: shape"):
        cpa.attn_fwd(q, k, v, o, lse, varlen=bad)
    with pytest.raises(ValueError, match="lse: shape"):
        cpa.attn_fwd(q, k, v, o, lse.t().contiguous(), varlen=vl)
    with pytest.raises(ValueError, match="varlen metadata"):
        cpa.attn_fwd(q, k, v, o, lse)
    with pytest.raises(ValueError, match="must be on a GPU"):
        cpa.attn_fwd(q, k, v, o, lse, varlen=vl)


def test_bwd_declines():
    q, k, v, o, lse = bshd()
    do, dq, dk, dv = torch.zeros_like(o), torch.zeros_like(q), torch.zeros_like(k), \
        torch.zeros_like(v)
    with pytest.raises(TypeError, match="lse: dtype"):
        cpa.attn_bwd(q, k, v, o, do, lse.double(), dq, dk, dv)
    with pytest.raises(ValueError, match="dq: shape"):
        cpa.attn_bwd(q, k, v, o, do, lse, dq[..., :64], dk, dv)
    with pytest.raises(ValueError, match="dk: shape"):
        cpa.attn_bwd(q, k, v, o, do, lse, dq, dk[:, :8], dv)
    with pytest.raises(TypeError, match="dv: dtype"):
        cpa.attn_bwd(q, k, v, o, do, lse, dq, dk, dv.float())
    with pytest.raises(ValueError, match="dout: shape"):
        cpa.attn_bwd(q, k, v, o, do[:, :, :2], lse, dq, dk, dv)
    with pytest.raises(TypeError, match="o and dout"):
        cpa.attn_bwd(q, k, v, o.float(), do, lse, dq, dk, dv)
    with pytest.raises(ValueError, match="must be on a GPU"):
        cpa.attn_bwd(q, k, v, o, do, lse, dq, dk, dv)


def test_merge_pack_xchg_declines():
    o = torch.zeros(1, 64, 4, 128)
    lse = torch.zeros(1, 4, 64)
    with pytest.raises(ValueError, match="o_part: shape"):
        cpa.attn_merge_lse(o, lse, o[:, :32], lse)
    with pytest.raises(TypeError, match="lse_part: dtype"):
        cpa.attn_merge_lse(o, lse, o, lse.to(BF))
    with pytest.raises(ValueError, match="lse_acc: shape"):
        cpa.attn_merge_lse(o, lse.transpose(1, 2).contiguous(), o, lse)
    with pytest.raises(ValueError, match="must be on a GPU"):
        cpa.attn_merge_lse(o, lse, o.clone(), lse.clone())
    ob = o.to(BF)
    with pytest.raises(TypeError, match="lse: dtype"):
        cpa.pack_saved(ob, lse.half(), 4)
    with pytest.raises(ValueError, match="lse: shape"):
        cpa.pack_saved(ob, lse[:, :2], 4)
    with pytest.raises(TypeError, match="buf: dtype"):
        cpa.pack_saved(ob, lse, 4, buf=torch.zeros(10, dtype=torch.float32))
    with pytest.raises(ValueError, match="must be on a GPU"):
        cpa.pack_saved(ob, lse, 4)
    with pytest.raises(ValueError, match="must be on a GPU"):
        cpa.unpack_saved(torch.zeros(10, dtype=torch.uint8), ob, lse, 4)
    with pytest.raises(ValueError, match="must be on a GPU"):
        cpa.xchg_pack([ob, lse], groups=1, ranges=[[(0, 64)]], split=True)
