"""Pins for the oracle's sliding-window / band visibility.

The window (left, right) keeps key j visible to query i iff
q_pos - left <= k_pos <= q_pos + right, -1 leaving a side unbounded, and a
causal mask keeps the right bound at the diagonal (PR 3527 "cuDNN FROST
attention backend for head_dim in (256, 512]", commits on sliding window: a
diagonal alignment plus a two-sided band, -1 unbounded, a non-causal (w, 0)
window being the causal band of width w).

Each pin builds the mask, or the answer, without the oracle's arithmetic:
* a scalar brute force that tests each (row, key) pair with its own
  comparison;
* torch's float64 scaled_dot_product_attention and autograd with a band mask
  built from torch.tril / torch.triu diagonals;
* closed forms: window (0, 0) leaves only the diagonal key, so O_i = V_i,
  LSE_i = s <q_i, k_i>, dV_i = dO_i and dQ = dK = 0;
* a window wider than the sequence changes nothing, and a real window
  changes the output (a dropped bound would still give plausible numbers).
"""
import math

import numpy as np
import pytest
import torch

import oracle


def brute_window_forward(q, k, v, scale, qp, kp, causal, left, right):
    sq, hq, d = q.shape
    sk, hkv, dv = v.shape
    g = hq // hkv
    o = np.zeros((sq, hq, dv))
    lse = np.zeros((hq, sq))
    for h in range(hq):
        for i in range(sq):
            vis = []
            for j in range(sk):
                ok = True
                if causal and kp[j] > qp[i]:
                    ok = False
                if left != -1 and kp[j] < qp[i] - left:
                    ok = False
                if right != -1 and kp[j] > qp[i] + right:
                    ok = False
                if ok:
                    vis.append(j)
            if not vis:
                lse[h, i] = -math.inf
                continue
            s = {j: scale * math.fsum(float(q[i, h, t]) * float(k[j, h // g, t])
                                      for t in range(d)) for j in vis}
            m = max(s.values())
            l = m + math.log(math.fsum(math.exp(s[j] - m) for j in vis))
            lse[h, i] = l
            for e in range(dv):
                o[i, h, e] = math.fsum(math.exp(s[j] - l) * float(v[j, h // g, e]) for j in vis)
    return o, lse


WINDOW_CASES = [
    # name, sq, sk, causal, (left, right), q offset
    ("causal_left3", 9, 9, True, (3, -1), 0),
    ("causal_left0", 6, 6, True, (0, -1), 0),
    ("causal_right_ignored", 7, 7, True, (2, 5), 0),
    ("band_left2_right1", 8, 8, False, (2, 1), 0),
    ("noncausal_w_0_is_causal_band", 8, 8, False, (3, 0), 0),
    ("right_only", 6, 9, False, (-1, 2), 0),
    ("bottom_right_left2", 5, 11, True, (2, -1), 6),
    ("keyless_rows", 5, 4, True, (1, -1), -3),
]


@pytest.mark.parametrize("case", WINDOW_CASES, ids=lambda c: c[0])
def test_window_matches_bruteforce(case):
    name, sq, sk, causal, win, off = case
    rng = np.random.default_rng(sum(map(ord, name)))
    q = rng.standard_normal((sq, 2, 4))
    k = rng.standard_normal((sk, 1, 4))
    v = rng.standard_normal((sk, 1, 3))
    qp, kp = np.arange(sq) + off, np.arange(sk)
    o, lse = oracle.forward(q, k, v, 0.5, qp, kp, causal, window=win)
    ob, lb = brute_window_forward(q, k, v, 0.5, qp, kp, causal, *win)
    np.testing.assert_allclose(o, ob, rtol=0, atol=1e-13)
    assert np.array_equal(np.isneginf(lse), np.isneginf(lb))
    fin = np.isfinite(lb)
    np.testing.assert_allclose(lse[fin], lb[fin], rtol=0, atol=1e-13)


def _band_mask(sq, sk, left, right):
    """torch.tril / torch.triu band on the top-left diagonal."""
    ones = torch.ones(sq, sk, dtype=torch.bool)
    m = ones if right < 0 else torch.tril(ones, diagonal=right)
    if left >= 0:
        m = m & torch.triu(ones, diagonal=-left)
    return m


@pytest.mark.parametrize("causal,win", [(True, (5, -1)), (False, (4, 2)), (False, (0, 0)),
                                        (True, (0, 0)), (False, (-1, 3))])
def test_window_matches_torch_sdpa_fp64(causal, win):
    s, hq, hkv, d, dv = 37, 4, 2, 8, 6
    g = torch.Generator().manual_seed(123 + win[0] * 7 + win[1])
    q = torch.randn(1, s, hq, d, generator=g, dtype=torch.float64)
    k = torch.randn(1, s, hkv, d, generator=g, dtype=torch.float64)
    v = torch.randn(1, s, hkv, dv, generator=g, dtype=torch.float64)
    do = torch.randn(1, s, hq, dv, generator=g, dtype=torch.float64)
    scale = 1.0 / math.sqrt(d)
    right = 0 if causal else win[1]
    mask = _band_mask(s, s, win[0], right)
    rep = hq // hkv
    qt = q.transpose(1, 2).clone().requires_grad_(True)
    kt = k.transpose(1, 2).clone().requires_grad_(True)
    vt = v.transpose(1, 2).clone().requires_grad_(True)
    ot = torch.nn.functional.scaled_dot_product_attention(
        qt, kt.repeat_interleave(rep, dim=1), vt.repeat_interleave(rep, dim=1),
        attn_mask=mask, scale=scale)
    ot.backward(do.transpose(1, 2))
    o, _ = oracle.bshd_forward(q.numpy(), k.numpy(), v.numpy(), scale, causal=causal, window=win)
    np.testing.assert_allclose(o, ot.detach().transpose(1, 2).numpy(), rtol=0, atol=1e-12)
    dq, dk, dv_ = oracle.bshd_backward(q.numpy(), k.numpy(), v.numpy(), do.numpy(), scale,
                                       causal=causal, window=win)
    np.testing.assert_allclose(dq, qt.grad.transpose(1, 2).numpy(), rtol=0, atol=1e-11)
    np.testing.assert_allclose(dk, kt.grad.transpose(1, 2).numpy(), rtol=0, atol=1e-11)
    np.testing.assert_allclose(dv_, vt.grad.transpose(1, 2).numpy(), rtol=0, atol=1e-11)


def test_diagonal_only_window_closed_form():
    rng = np.random.default_rng(9)
    s, h, d = 12, 2, 5
    q = rng.standard_normal((s, h, d))
    k = rng.standard_normal((s, h, d))
    v = rng.standard_normal((s, h, 3))
    do = rng.standard_normal((s, h, 3))
    o, lse = oracle.forward(q, k, v, 0.7, causal=True, window=(0, -1))
    np.testing.assert_allclose(o, v, rtol=0, atol=1e-15)
    np.testing.assert_allclose(lse, 0.7 * np.einsum("shd,shd->hs", q, k), rtol=0, atol=1e-14)
    dq, dk, dv = oracle.backward(q, k, v, do, 0.7, causal=False, window=(0, 0))
    np.testing.assert_allclose(dv, do, rtol=0, atol=1e-15)
    assert np.abs(dq).max() < 1e-14 and np.abs(dk).max() < 1e-14


def test_wide_window_is_no_window_and_real_window_differs():
    rng = np.random.default_rng(4)
    s = 20
    q, k, v = (rng.standard_normal((s, 2, 4)) for _ in range(3))
    o_c, l_c = oracle.forward(q, k, v, 0.5, causal=True)
    o_w, l_w = oracle.forward(q, k, v, 0.5, causal=True, window=(s, s))
    assert np.array_equal(o_c, o_w) and np.array_equal(l_c, l_w)
    o_n, _ = oracle.forward(q, k, v, 0.5, causal=False, window=(-1, -1))
    o_f, _ = oracle.forward(q, k, v, 0.5, causal=False)
    assert np.array_equal(o_n, o_f)
    o_4, _ = oracle.forward(q, k, v, 0.5, causal=True, window=(4, -1))
    assert np.abs(o_4 - o_c).max() > 1e-2
