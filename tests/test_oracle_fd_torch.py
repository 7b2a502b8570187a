"""Oracle gradients vs central finite differences, and the oracle vs torch's
own float64 scaled_dot_product_attention (forward and autograd backward).

Finite differences test the backward against the forward alone: with
L(Q, K, V) = sum(dO * O), the directional derivative along a random U must
equal <grad, U>.  A dropped term, a wrong sign or a transposed product in the
backward breaks this at O(1).  torch's SDPA is an independent library
implementation of the same definition (top-left causal, GQA).
"""
import math

import numpy as np
import pytest
import torch

import oracle


def _loss(q, k, v, do, scale, qp, kp, causal):
    o, _ = oracle.forward(q, k, v, scale, qp, kp, causal)
    return float(np.sum(do * o))


FD_CASES = [
    # sq, sk, hq, hkv, d, dv, causal, q offset (bottom-right style)
    (6, 6, 2, 2, 4, 3, True, 0),
    (5, 8, 4, 2, 3, 5, True, 3),      # rectangular, bottom-right, GQA
    (7, 4, 2, 1, 4, 4, True, -3),     # keyless leading rows
    (5, 6, 2, 2, 4, 4, False, 0),
]


@pytest.mark.parametrize("case", FD_CASES)
def test_backward_finite_differences(case):
    sq, sk, hq, hkv, d, dv, causal, off = case
    rng = np.random.default_rng(1234 + sq * 7 + sk)
    q = rng.standard_normal((sq, hq, d))
    k = rng.standard_normal((sk, hkv, d))
    v = rng.standard_normal((sk, hkv, dv))
    do = rng.standard_normal((sq, hq, dv))
    qp = np.arange(sq) + off
    kp = np.arange(sk)
    scale = 0.7
    dq, dk, dv_ = oracle.backward(q, k, v, do, scale, qp, kp, causal)
    h = 1e-5
    for name, x, gx in (("q", q, dq), ("k", k, dk), ("v", v, dv_)):
        for trial in range(3):
            u = rng.standard_normal(x.shape)
            xp, xm = x + h * u, x - h * u
            args_p = dict(q=q, k=k, v=v)
            args_m = dict(q=q, k=k, v=v)
            args_p[name] = xp
            args_m[name] = xm
            lp = _loss(args_p["q"], args_p["k"], args_p["v"], do, scale, qp, kp, causal)
            lm = _loss(args_m["q"], args_m["k"], args_m["v"], do, scale, qp, kp, causal)
            fd = (lp - lm) / (2 * h)
            an = float(np.sum(gx * u))
            assert abs(fd - an) <= 1e-7 * max(1.0, abs(an)), (name, fd, an)
    if off < 0:
        # keyless leading rows get exactly zero dQ
        assert (dq[:-off] == 0).all()


TORCH_CASES = [
    # b, s, hq, hkv, d, dv
    (1, 33, 2, 2, 16, 16),
    (2, 40, 4, 1, 8, 12),
    (1, 64, 6, 2, 24, 8),
]


@pytest.mark.parametrize("case", TORCH_CASES)
def test_matches_torch_sdpa_fp64(case):
    b, s, hq, hkv, d, dv = case
    g = torch.Generator().manual_seed(77 + s)
    q = torch.randn(b, s, hq, d, generator=g, dtype=torch.float64)
    k = torch.randn(b, s, hkv, d, generator=g, dtype=torch.float64)
    v = torch.randn(b, s, hkv, dv, generator=g, dtype=torch.float64)
    do = torch.randn(b, s, hq, dv, generator=g, dtype=torch.float64)
    scale = 1.0 / math.sqrt(d)
    qt = q.transpose(1, 2).clone().requires_grad_(True)
    kt = k.transpose(1, 2).clone().requires_grad_(True)
    vt = v.transpose(1, 2).clone().requires_grad_(True)
    ot = torch.nn.functional.scaled_dot_product_attention(
        qt, kt, vt, is_causal=True, scale=scale, enable_gqa=(hq != hkv))
    ot.backward(do.transpose(1, 2))
    o_ref = ot.detach().transpose(1, 2).numpy()
    o, lse = oracle.bshd_forward(q.numpy(), k.numpy(), v.numpy(), scale)
    np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-12)
    dq, dk, dv_ = oracle.bshd_backward(q.numpy(), k.numpy(), v.numpy(),
                                       do.numpy(), scale)
    np.testing.assert_allclose(dq, qt.grad.transpose(1, 2).numpy(), rtol=0, atol=1e-11)
    np.testing.assert_allclose(dk, kt.grad.transpose(1, 2).numpy(), rtol=0, atol=1e-11)
    np.testing.assert_allclose(dv_, vt.grad.transpose(1, 2).numpy(), rtol=0, atol=1e-11)


def test_matches_torch_sdpa_bottom_right_mask():
    """Rectangular shape where top-left and bottom-right differ (PR 3527,
    test commit: a rectangular shape where the two alignments differ);
    torch is given the bottom-right mask explicitly."""
    g = torch.Generator().manual_seed(5)
    sq, sk, h, d = 9, 21, 2, 8
    q = torch.randn(1, h, sq, d, generator=g, dtype=torch.float64)
    k = torch.randn(1, h, sk, d, generator=g, dtype=torch.float64)
    v = torch.randn(1, h, sk, d, generator=g, dtype=torch.float64)
    mask = (torch.arange(sk)[None, :] <= (torch.arange(sq)[:, None] + sk - sq))
    ot = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=mask)
    qp = np.arange(sq) + (sk - sq)
    o, _ = oracle.forward(q[0].transpose(0, 1).numpy(), k[0].transpose(0, 1).numpy(),
                          v[0].transpose(0, 1).numpy(), 1 / math.sqrt(d), qp,
                          np.arange(sk), True)
    np.testing.assert_allclose(o, ot[0].transpose(0, 1).numpy(), rtol=0, atol=1e-12)
    # and top-left really is different here
    o_tl, _ = oracle.forward(q[0].transpose(0, 1).numpy(), k[0].transpose(0, 1).numpy(),
                             v[0].transpose(0, 1).numpy(), 1 / math.sqrt(d))
    assert np.abs(o_tl - o).max() > 1e-2
