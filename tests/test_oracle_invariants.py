"""Invariants and structural identities of the oracle.

* softmax rows sum to one (read off with V = identity, so O = P);
* Q = 0 closed form: O_i is the mean of the visible V rows, LSE_i = ln n_i;
* sum_j dS_ij = 0 per row, hence sum_j dK_j = 0 per kv head;
* sum_j dV_j = sum over non-empty rows of dO_i (summed over the group);
* rowsum(P * dP) equals <dO_i, O_i> (the quantity the fast backward uses);
* merging partials over disjoint key blocks equals the unsplit result
  (including empty and fully masked blocks), and merge is symmetric;
* GQA equals MHA with K/V repeated per group (dK/dV summed over the group);
* THD equals per-document dense attention.
"""
import math

import numpy as np
import pytest

import oracle


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def test_rows_sum_to_one_and_zero_for_keyless():
    rng = np.random.default_rng(0)
    sq, sk, d = 7, 5, 4
    q = _rand(rng, sq, 2, d)
    k = _rand(rng, sk, 2, d)
    v = np.tile(np.eye(sk)[:, None, :], (1, 2, 1))     # O = P
    qp = np.arange(sq) - 2                               # rows 0,1 keyless
    p, lse = oracle.forward(q, k, v, 0.5, qp, np.arange(sk))
    rs = p.sum(axis=2)
    np.testing.assert_allclose(rs[2:], 1.0, rtol=0, atol=1e-14)
    assert (p[:2] == 0).all()
    assert np.isneginf(lse[:, :2]).all()
    # masked entries are exactly zero
    for i in range(sq):
        assert (p[i, :, max(0, qp[i] + 1):] == 0).all()


def test_zero_query_closed_form():
    rng = np.random.default_rng(1)
    s, d = 9, 3
    q = np.zeros((s, 1, d))
    k = _rand(rng, s, 1, d)
    v = _rand(rng, s, 1, 5)
    o, lse = oracle.forward(q, k, v, 0.3)
    for i in range(s):
        np.testing.assert_allclose(o[i, 0], v[:i + 1, 0].mean(axis=0), atol=1e-14)
        assert abs(lse[0, i] - math.log(i + 1)) < 1e-14
    # row 0 sees only key 0: O_0 = V_0, LSE_0 = S_00
    q2 = _rand(rng, s, 1, d)
    o2, l2 = oracle.forward(q2, k, v, 0.3)
    np.testing.assert_allclose(o2[0, 0], v[0, 0], atol=1e-14)
    assert abs(l2[0, 0] - 0.3 * q2[0, 0] @ k[0, 0]) < 1e-14


@pytest.mark.parametrize("hq,hkv", [(2, 2), (4, 2), (3, 1)])
def test_gradient_sum_invariants(hq, hkv):
    rng = np.random.default_rng(hq * 10 + hkv)
    sq, sk, d, dv = 11, 8, 5, 4
    q, k, v = _rand(rng, sq, hq, d), _rand(rng, sk, hkv, d), _rand(rng, sk, hkv, dv)
    do = _rand(rng, sq, hq, dv)
    qp = np.arange(sq) - 3          # 3 keyless rows
    dq, dk, dvv = oracle.backward(q, k, v, do, 0.4, qp, np.arange(sk))
    np.testing.assert_allclose(dk.sum(axis=0), 0.0, atol=1e-12)
    g = hq // hkv
    nonempty = qp >= 0
    for kh in range(hkv):
        expect = do[nonempty][:, kh * g:(kh + 1) * g, :].sum(axis=(0, 1))
        np.testing.assert_allclose(dvv[:, kh].sum(axis=0), expect, atol=1e-12)
    assert (dq[:3] == 0).all()


def test_rowsum_p_dp_equals_do_dot_o():
    rng = np.random.default_rng(3)
    sq, sk, d, dv = 6, 6, 4, 7
    q, k, v = _rand(rng, sq, 1, d), _rand(rng, sk, 1, d), _rand(rng, sk, 1, dv)
    do = _rand(rng, sq, 1, dv)
    o, _ = oracle.forward(q, k, v, 0.5)
    eye = np.tile(np.eye(sk)[:, None, :], (1, 1, 1))
    p, _ = oracle.forward(q, k, eye, 0.5)
    dp = do[:, 0] @ v[:, 0].T
    np.testing.assert_allclose((p[:, 0] * dp).sum(axis=1),
                               (do[:, 0] * o[:, 0]).sum(axis=1), atol=1e-13)


@pytest.mark.parametrize("cuts", [[0, 5, 9, 16], [0, 0, 16], [0, 12, 13, 16]])
def test_merge_equals_full(cuts):
    rng = np.random.default_rng(len(cuts))
    sq, sk, h, d = 10, 16, 2, 4
    q, k, v = _rand(rng, sq, h, d), _rand(rng, sk, h, d), _rand(rng, sk, h, d)
    qp = np.arange(sq) + 3          # rows 0..9 at positions 3..12
    kp = np.arange(sk)
    o_full, l_full = oracle.forward(q, k, v, 0.5, qp, kp)
    parts = []
    for a, b in zip(cuts[:-1], cuts[1:]):
        o, l = oracle.forward(q, k[a:b], v[a:b], 0.5, qp, kp[a:b])
        parts.append((o.transpose(1, 0, 2), l))   # [H, S, D] vs lse [H, S]
    om, lm = oracle.merge(parts)
    np.testing.assert_allclose(om.transpose(1, 0, 2), o_full, atol=1e-12)
    np.testing.assert_allclose(lm, l_full, atol=1e-12)
    # symmetric in its operands
    om2, lm2 = oracle.merge(parts[::-1])
    np.testing.assert_allclose(om2, om, atol=1e-13)
    np.testing.assert_allclose(lm2, lm, atol=1e-13)


def test_gqa_equals_repeated_mha():
    rng = np.random.default_rng(9)
    sq, sk, hq, hkv, d = 7, 9, 6, 2, 4
    g = hq // hkv
    q, k, v = _rand(rng, sq, hq, d), _rand(rng, sk, hkv, d), _rand(rng, sk, hkv, d)
    do = _rand(rng, sq, hq, d)
    qp = np.arange(sq) + 2
    kr, vr = np.repeat(k, g, axis=1), np.repeat(v, g, axis=1)
    o1, l1 = oracle.forward(q, k, v, 0.5, qp)
    o2, l2 = oracle.forward(q, kr, vr, 0.5, qp)
    np.testing.assert_allclose(o1, o2, atol=1e-14)
    np.testing.assert_allclose(l1, l2, atol=1e-14)
    dq1, dk1, dv1 = oracle.backward(q, k, v, do, 0.5, qp)
    dq2, dk2, dv2 = oracle.backward(q, kr, vr, do, 0.5, qp)
    np.testing.assert_allclose(dq1, dq2, atol=1e-13)
    np.testing.assert_allclose(dk1, dk2.reshape(sk, hkv, g, d).sum(axis=2), atol=1e-13)
    np.testing.assert_allclose(dv1, dv2.reshape(sk, hkv, g, d).sum(axis=2), atol=1e-13)


def test_thd_equals_per_document_dense():
    rng = np.random.default_rng(21)
    used = np.array([13, 1, 0, 20], np.int32)
    cu = np.array([0, 16, 32, 48, 72], np.int32)     # physical pitch, padding
    t, hq, hkv, d = 72, 4, 2, 8
    q, k, v = _rand(rng, t, hq, d), _rand(rng, t, hkv, d), _rand(rng, t, hkv, d)
    do = _rand(rng, t, hq, d)
    for br in (False, True):
        o, lse = oracle.thd_forward(q, k, v, 0.3, cu, cu, used, used, True, br)
        dq, dk, dvv = oracle.thd_backward(q, k, v, do, 0.3, cu, cu, used, used, True, br)
        for n in range(4):
            a, m = cu[n], used[n]
            if m == 0:
                continue
            od, ld = oracle.forward(q[a:a + m], k[a:a + m], v[a:a + m], 0.3)
            np.testing.assert_allclose(o[a:a + m], od, atol=1e-14)
            np.testing.assert_allclose(lse[:, a:a + m], ld, atol=1e-14)
            g1, g2, g3 = oracle.backward(q[a:a + m], k[a:a + m], v[a:a + m],
                                         do[a:a + m], 0.3)
            np.testing.assert_allclose(dq[a:a + m], g1, atol=1e-13)
            np.testing.assert_allclose(dk[a:a + m], g2, atol=1e-13)
            np.testing.assert_allclose(dvv[a:a + m], g3, atol=1e-13)
            assert np.isnan(o[a + m:cu[n + 1]]).all()
            assert np.isnan(dk[a + m:cu[n + 1]]).all()


def test_thd_different_q_and_k_lengths_bottom_right():
    """Per-document bottom-right alignment with S_q != S_k differs from
    top-left and equals the dense bottom-right result per document."""
    rng = np.random.default_rng(4)
    used_q = np.array([3, 6], np.int32)
    used_k = np.array([8, 2], np.int32)
    cu_q = np.array([0, 8, 16], np.int32)
    cu_k = np.array([0, 8, 16], np.int32)
    q, k, v = _rand(rng, 16, 2, 4), _rand(rng, 16, 2, 4), _rand(rng, 16, 2, 4)
    o, _ = oracle.thd_forward(q, k, v, 0.5, cu_q, cu_k, used_q, used_k, True, True)
    od, _ = oracle.forward(q[0:3], k[0:8], v[0:8], 0.5, np.arange(3) + 5)
    np.testing.assert_allclose(o[0:3], od, atol=1e-14)
    od2, _ = oracle.forward(q[8:14], k[8:10], v[8:10], 0.5, np.arange(6) - 4)
    np.testing.assert_allclose(o[8:14], od2, atol=1e-14)
    assert (o[8:12] == 0).all()      # keyless under bottom-right
