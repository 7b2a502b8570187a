"""Plain float64 softmax attention, its exact gradient and the LSE merge.

Test infrastructure only (see the package docstring).  Everything here is
the textbook definition; the only concession to size is that query rows are
processed in blocks of ``row_block`` so that a 32K-key problem never forms an
S x S matrix.  Blocking over rows does not change any sum: each row's
softmax still sees all of its keys at once.
"""
from __future__ import annotations

import numpy as np

NEG_INF = -np.inf


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def positions_from_segments(n_rows, segments):
    """Query positions for rows made of contiguous segments.

    ``segments`` is a list of (row_begin, pos_begin); segment s covers rows
    [row_begin_s, row_begin_{s+1}) and row i in it has position
    pos_begin_s + (i - row_begin_s).  This is how a dual-chunk CP rank keeps
    the global positions of its two query chunks (PR 3510, Changes: balanced
    CP partitions).
    """
    pos = np.empty(n_rows, dtype=np.int64)
    bounds = [s[0] for s in segments] + [n_rows]
    for s, (r0, p0) in enumerate(segments):
        r1 = bounds[s + 1]
        pos[r0:r1] = p0 + np.arange(r1 - r0)
    return pos


def _visible(qp, kp, causal, window=None):
    """Boolean [rows, keys]: key j visible to query i.

    causal: k_pos[j] <= q_pos[i].  window = (left, right), -1 meaning no
    bound on that side: q_pos[i] - left <= k_pos[j] <= q_pos[i] + right, so
    ``left`` keys before the diagonal stay visible besides the diagonal
    itself (PR 3527, commits on sliding window: a diagonal alignment plus a
    two-sided band; the window applies to every mask type, -1 is unbounded,
    and a causal mask keeps the right bound at the diagonal, so a
    non-causal (w, 0) window is the causal band of width w).
    """
    d = kp[None, :] - qp[:, None]          # key position minus query position
    vis = np.ones(d.shape, dtype=bool)
    if causal:
        vis &= d <= 0
    if window is not None:
        left, right = window
        if left >= 0:
            vis &= d >= -left
        if right >= 0:
            vis &= d <= right
    return vis


def _row_softmax(s, vis):
    """Masked row softmax of scores ``s`` [r, n].

    Returns (P, LSE): LSE = m + ln(sum exp(s - m)) over visible keys (natural
    log), -inf for rows with no visible key; P = exp(s - LSE) on visible keys
    and 0 elsewhere (0 everywhere on keyless rows).
    """
    s = np.where(vis, s, NEG_INF)
    has = vis.any(axis=1)
    m = np.where(has, s.max(axis=1, initial=NEG_INF), 0.0)
    e = np.where(vis, np.exp(s - m[:, None]), 0.0)
    tot = e.sum(axis=1)
    lse = np.where(has, m + np.log(np.where(has, tot, 1.0)), NEG_INF)
    p = np.where(has[:, None], e / np.where(has, tot, 1.0)[:, None], 0.0)
    return p, lse


def forward(q, k, v, scale, q_pos=None, k_pos=None, causal=True,
            heads=None, row_block=512, window=None):
    """Attention forward for one sequence.

    q [Sq, Hq, Dqk], k [Sk, Hkv, Dqk], v [Sk, Hkv, Dv]; query head h reads
    kv head h // (Hq // Hkv) (GQA as K/V repeated Hq/Hkv times in order).
    Returns o [Sq, Hq, Dv] and lse [Hq, Sq] (float64).  ``heads`` restricts
    the computation to a subset of query heads (others are left NaN).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    sq, hq, _ = q.shape
    sk, hkv, dv = v.shape
    assert hq % hkv == 0
    g = hq // hkv
    qp = np.arange(sq) if q_pos is None else np.asarray(q_pos, np.int64)
    kp = np.arange(sk) if k_pos is None else np.asarray(k_pos, np.int64)
    o = np.full((sq, hq, dv), np.nan)
    lse = np.full((hq, sq), np.nan)
    for h in (range(hq) if heads is None else heads):
        kh = h // g
        for r0 in range(0, sq, row_block):
            r1 = min(sq, r0 + row_block)
            s = scale * (q[r0:r1, h, :] @ k[:, kh, :].T)
            p, l = _row_softmax(s, _visible(qp[r0:r1], kp, causal, window))
            o[r0:r1, h, :] = p @ v[:, kh, :]
            lse[h, r0:r1] = l
    return o, lse


def forward_rows(q, k, v, scale, rows, q_pos=None, k_pos=None, causal=True,
                 heads=None, window=None):
    """Forward for selected query rows only (sampled checks at full size).

    Returns o [len(rows), Hq, Dv] and lse [Hq, len(rows)].
    """
    rows = np.asarray(rows, np.int64)
    sq = q.shape[0]
    qp = np.arange(sq) if q_pos is None else np.asarray(q_pos, np.int64)
    return forward(np.asarray(q)[rows], k, v, scale, q_pos=qp[rows],
                   k_pos=k_pos, causal=causal, heads=heads, window=window)


def backward(q, k, v, do, scale, q_pos=None, k_pos=None, causal=True,
             heads=None, row_block=512, window=None):
    """Exact gradient of O = softmax(s Q K^T + mask) V for one sequence.

    With P the masked softmax, dP = dO V^T and the softmax Jacobian
    dS = P * (dP - rowsum(P * dP)):
        dQ = s dS K,  dK = s dS^T Q,  dV = P^T dO,
    with dK and dV of a kv head summed over its query-head group.  Keyless
    rows have P = 0, hence zero dQ; keys no query sees get dK = dV = 0.
    ``heads`` restricts to query heads (dK/dV then only hold those heads'
    contributions).
    """
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    sq, hq, dqk = q.shape
    sk, hkv, dv = v.shape
    g = hq // hkv
    qp = np.arange(sq) if q_pos is None else np.asarray(q_pos, np.int64)
    kp = np.arange(sk) if k_pos is None else np.asarray(k_pos, np.int64)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dvv = np.zeros_like(v)
    for h in (range(hq) if heads is None else heads):
        kh = h // g
        for r0 in range(0, sq, row_block):
            r1 = min(sq, r0 + row_block)
            s = scale * (q[r0:r1, h, :] @ k[:, kh, :].T)
            p, _ = _row_softmax(s, _visible(qp[r0:r1], kp, causal, window))
            dp = do[r0:r1, h, :] @ v[:, kh, :].T
            rs = (p * dp).sum(axis=1)
            ds = p * (dp - rs[:, None])
            dq[r0:r1, h, :] = scale * (ds @ k[:, kh, :])
            dk[:, kh, :] += scale * (ds.T @ q[r0:r1, h, :])
            dvv[:, kh, :] += p.T @ do[r0:r1, h, :]
    return dq, dk, dvv


def merge(parts):
    """Combine partial attentions over disjoint key sets.

    ``parts`` is a list of (o [..., Dv], lse [...]) with matching leading
    shapes (lse indexed like o without its last axis).  With M the max of the
    LSEs: M = -inf gives (0, -inf); else LSE = M + ln(sum_k exp(LSE_k - M))
    and O = sum_k exp(LSE_k - LSE) O_k.
    """
    os_ = [_f64(o) for o, _ in parts]
    ls = [_f64(l) for _, l in parts]
    m = np.maximum.reduce(ls)
    fin = np.isfinite(m)
    mm = np.where(fin, m, 0.0)
    tot = sum(np.exp(l - mm) for l in ls)
    lse = np.where(fin, mm + np.log(np.where(fin, tot, 1.0)), NEG_INF)
    lsafe = np.where(fin, lse, 0.0)
    o = sum(np.where(fin, np.exp(l - lsafe), 0.0)[..., None] * ok
            for ok, l in zip(os_, ls))
    return o, lse


# ---------------------------------------------------------------- layouts

def bshd_forward(q, k, v, scale, segments=None, k_pos_begin=0, causal=True,
                 heads=None, window=None):
    """Dense BSHD: q [B, Sq, Hq, D].  ``segments`` as in
    positions_from_segments (default: one segment at position 0, i.e.
    top-left); key j has position k_pos_begin + j.  Returns o [B, Sq, Hq,
    Dv], lse [B, Hq, Sq]."""
    b, sq = q.shape[:2]
    sk = k.shape[1]
    qp = positions_from_segments(sq, segments or [(0, 0)])
    kp = k_pos_begin + np.arange(sk)
    os_, ls = [], []
    for i in range(b):
        o, l = forward(q[i], k[i], v[i], scale, qp, kp, causal, heads,
                       window=window)
        os_.append(o)
        ls.append(l)
    return np.stack(os_), np.stack(ls)


def bshd_backward(q, k, v, do, scale, segments=None, k_pos_begin=0,
                  causal=True, heads=None, window=None):
    b, sq = q.shape[:2]
    sk = k.shape[1]
    qp = positions_from_segments(sq, segments or [(0, 0)])
    kp = k_pos_begin + np.arange(sk)
    res = [backward(q[i], k[i], v[i], do[i], scale, qp, kp, causal, heads,
                    window=window)
           for i in range(b)]
    return tuple(np.stack([r[j] for r in res]) for j in range(3))


def _thd_docs(cu_q, cu_k, used_q, used_k, bottom_right):
    for n in range(len(used_q)):
        q0, nq = int(cu_q[n]), int(used_q[n])
        k0, nk = int(cu_k[n]), int(used_k[n])
        off = (nk - nq) if bottom_right else 0
        yield q0, nq, k0, nk, np.arange(nq) + off, np.arange(nk)


def thd_forward(q, k, v, scale, cu_q, cu_k, used_q, used_k, causal=True,
                bottom_right=False, heads=None, window=None):
    """Packed THD: q [Tq, Hq, D] with document n on physical rows
    [cu_q[n], cu_q[n] + used_q[n]) (padded offsets plus visible lengths, PR
    3149 "Enable FA4 for context-parallel attention", Description).  Padding
    rows are left NaN.  Returns o [Tq, Hq, Dv], lse [Hq, Tq]."""
    tq, hq, _ = q.shape
    dv = v.shape[2]
    o = np.full((tq, hq, dv), np.nan)
    lse = np.full((hq, tq), np.nan)
    for q0, nq, k0, nk, qp, kp in _thd_docs(cu_q, cu_k, used_q, used_k,
                                            bottom_right):
        if nq == 0:
            continue
        od, ld = forward(q[q0:q0 + nq], k[k0:k0 + nk], v[k0:k0 + nk], scale,
                         qp, kp, causal, heads, window=window)
        o[q0:q0 + nq] = od
        lse[:, q0:q0 + nq] = ld
    return o, lse


def thd_backward(q, k, v, do, scale, cu_q, cu_k, used_q, used_k, causal=True,
                 bottom_right=False, heads=None, window=None):
    """Gradients for packed THD; padding rows are left NaN."""
    dq = np.full(q.shape, np.nan)
    dk = np.full(k.shape, np.nan)
    dvv = np.full(v.shape, np.nan)
    for q0, nq, k0, nk, qp, kp in _thd_docs(cu_q, cu_k, used_q, used_k,
                                            bottom_right):
        a, b_, c = backward(q[q0:q0 + nq], k[k0:k0 + nk], v[k0:k0 + nk],
                            do[q0:q0 + nq], scale, qp, kp, causal, heads,
                            window=window)
        dq[q0:q0 + nq] = a
        dk[k0:k0 + nk] = b_
        dvv[k0:k0 + nk] = c
    return dq, dk, dvv
