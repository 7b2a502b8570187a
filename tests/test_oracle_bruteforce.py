"""Oracle forward vs a scalar pure-Python evaluation on tiny inputs.

The brute force uses math.exp / math.log / math.fsum (exactly rounded sums)
and walks every (head, row, key) on its own, with no arrays, no blocking and
no shared helper, so an indexing slip in the vectorised oracle (a transposed
operand, a wrong GQA head, an off-by-one mask) shows up as a mismatch.
"""
import math

import numpy as np
import pytest

import oracle


def brute_forward(q, k, v, scale, qp, kp, causal):
    sq, hq, d = q.shape
    sk, hkv, dv = v.shape
    g = hq // hkv
    o = [[[0.0] * dv for _ in range(hq)] for _ in range(sq)]
    lse = [[0.0] * sq for _ in range(hq)]
    for h in range(hq):
        kh = h // g
        for i in range(sq):
            vis = [j for j in range(sk) if (not causal) or kp[j] <= qp[i]]
            if not vis:
                lse[h][i] = -math.inf
                continue
            s = {j: scale * math.fsum(float(q[i, h, t]) * float(k[j, kh, t])
                                      for t in range(d)) for j in vis}
            m = max(s.values())
            tot = math.fsum(math.exp(s[j] - m) for j in vis)
            l = m + math.log(tot)
            lse[h][i] = l
            for e in range(dv):
                o[i][h][e] = math.fsum(math.exp(s[j] - l) * float(v[j, kh, e])
                                       for j in vis)
    return np.asarray(o), np.asarray(lse)


CASES = [
    # name, sq, sk, hq, hkv, d, dv, causal, qp, kp
    ("square_topleft", 7, 7, 2, 2, 5, 4, True, None, None),
    ("rect_bottomright", 4, 9, 2, 1, 3, 6, True, "br", None),
    ("rect_topleft", 4, 9, 1, 1, 3, 3, True, None, None),
    ("q_longer_keyless", 9, 4, 3, 1, 4, 2, True, "br", None),
    ("noncausal", 5, 6, 4, 2, 3, 3, False, None, None),
    ("dual_chunk", 8, 16, 2, 2, 4, 4, True, "dc", None),
    ("offset_kv_block", 6, 5, 2, 2, 3, 3, True, "blk", "blk"),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: c[0])
def test_forward_matches_bruteforce(case):
    name, sq, sk, hq, hkv, d, dv, causal, qpk, kpk = case
    rng = np.random.default_rng(sum(map(ord, name)))
    q = rng.standard_normal((sq, hq, d))
    k = rng.standard_normal((sk, hkv, d))
    v = rng.standard_normal((sk, hkv, dv))
    scale = 1.0 / math.sqrt(d)
    qp = np.arange(sq)
    kp = np.arange(sk)
    if qpk == "br":
        qp = qp + (sk - sq)
    elif qpk == "dc":
        # two chunks of 4 rows at positions 0..3 and 12..15 of a 16-key span
        qp = oracle.positions_from_segments(sq, [(0, 0), (4, 12)])
        assert qp.tolist() == [0, 1, 2, 3, 12, 13, 14, 15]
    elif qpk == "blk":
        qp = np.arange(sq) + 10
    if kpk == "blk":
        kp = np.arange(sk) + 8
    o, lse = oracle.forward(q, k, v, scale, qp, kp, causal)
    ob, lb = brute_forward(q, k, v, scale, qp, kp, causal)
    np.testing.assert_allclose(o, ob, rtol=0, atol=1e-13)
    assert np.array_equal(np.isneginf(lse), np.isneginf(lb))
    fin = np.isfinite(lb)
    np.testing.assert_allclose(lse[fin], lb[fin], rtol=0, atol=1e-13)
    if qpk == "br" and sq > sk:
        # keyless leading rows: O = 0, LSE = -inf
        assert np.isneginf(lse[:, 0]).all()
        assert (o[0] == 0).all()


def test_thd_matches_bruteforce_per_doc():
    rng = np.random.default_rng(11)
    # docs with visible lengths 5, 0 (empty), 3 and physical pitch 8
    used = np.array([5, 0, 3], np.int32)
    cu = np.array([0, 8, 16, 24], np.int32)
    h, d = 2, 4
    q = rng.standard_normal((24, h, d))
    k = rng.standard_normal((24, h, d))
    v = rng.standard_normal((24, h, d))
    o, lse = oracle.thd_forward(q, k, v, 0.5, cu, cu, used, used)
    for n in range(3):
        a, m = cu[n], used[n]
        if m == 0:
            continue
        ob, lb = brute_forward(q[a:a + m], k[a:a + m], v[a:a + m], 0.5,
                               np.arange(m), np.arange(m), True)
        np.testing.assert_allclose(o[a:a + m], ob, rtol=0, atol=1e-13)
        np.testing.assert_allclose(lse[:, a:a + m], lb, rtol=0, atol=1e-13)
        # padding rows untouched (NaN in the oracle's output)
        assert np.isnan(o[a + m:cu[n + 1]]).all()
    assert np.isnan(o[8:16]).all()


def test_positions_from_segments_by_hand():
    """Positions written out by hand (dual-chunk CP ranks keep the global
    positions of both chunks: PR 3510 "Add head-parallel FA4 backward for
    cuDNN CP attention", Changes)."""
    assert oracle.positions_from_segments(8, [(0, 0), (4, 12)]).tolist() == \
        [0, 1, 2, 3, 12, 13, 14, 15]
    assert oracle.positions_from_segments(5, [(0, 7)]).tolist() == [7, 8, 9, 10, 11]
    # segments need not increase in position; the last runs to the end
    assert oracle.positions_from_segments(7, [(0, 3), (2, 0), (5, 100)]).tolist() == \
        [3, 4, 0, 1, 2, 100, 101]
    # CP4 rank 1 of a 32-token sequence: chunks 1 and 6 of 4 tokens
    assert oracle.positions_from_segments(8, [(0, 4), (4, 24)]).tolist() == \
        [4, 5, 6, 7, 24, 25, 26, 27]
    # CP4 rank 0 of 32768 tokens: rows 4096.. hold positions 28672..
    p = oracle.positions_from_segments(8192, [(0, 0), (4096, 28672)])
    assert p[0] == 0 and p[4095] == 4095 and p[4096] == 28672 and p[-1] == 32767


@pytest.mark.parametrize("explicit", [True, False])
def test_forward_rows_matches_bruteforce(explicit):
    """forward_rows on a scattered row subset against the scalar brute force
    given the rows' positions written out by hand (GQA, dual-chunk
    positions, keyless rows, rows out of order)."""
    rng = np.random.default_rng(29)
    sq, sk, hq, hkv, d, dv = 10, 12, 4, 2, 3, 5
    q = rng.standard_normal((sq, hq, d))
    k = rng.standard_normal((sk, hkv, d))
    v = rng.standard_normal((sk, hkv, dv))
    rows = [9, 0, 6, 3]
    if explicit:
        # rows 0..4 at positions 0..4, rows 5..9 at 7..11; keys start at 2
        qp = oracle.positions_from_segments(sq, [(0, 0), (5, 7)])
        kp = np.arange(sk) + 2
        qp_rows = [11, 0, 8, 3]            # by hand: row 0 sees no key
        o, lse = oracle.forward_rows(q, k, v, 0.6, rows, q_pos=qp, k_pos=kp)
    else:
        kp = np.arange(sk)
        qp_rows = [9, 0, 6, 3]
        o, lse = oracle.forward_rows(q, k, v, 0.6, rows)
    ob, lb = brute_forward(q[rows], k, v, 0.6, qp_rows, kp, True)
    assert o.shape == (4, hq, dv) and lse.shape == (hq, 4)
    np.testing.assert_allclose(o, ob, rtol=0, atol=1e-13)
    assert np.array_equal(np.isneginf(lse), np.isneginf(lb))
    fin = np.isfinite(lb)
    np.testing.assert_allclose(lse[fin], lb[fin], rtol=0, atol=1e-13)
    if explicit:
        assert np.isneginf(lse[:, 1]).all() and (o[1] == 0).all()
