"""Pins for the exchange-buffer oracle (oracle/xchg.py).

* a hand-written layout example (byte offsets written out by hand);
* pack then unpack with the same description restores every covered byte,
  including NaN payloads, -0 and denormals;
* the head-parallel round trip of PR 3510 ("Add head-parallel FA4 backward
  for cuDNN CP attention", Diagram) on CP = 4 dual-chunk ranks, simulated
  with plain segment copies for the all-to-all: after seq->heads each
  receiver holds exactly its head slice of the full-sequence tensors (checked
  by direct slicing, independent of the byte layout), and heads->seq gives
  every rank back exactly its own rows.
"""
import numpy as np

import oracle

ROWS = dict(kind="rows", elem_bytes=2)
LSE = dict(kind="lse", elem_bytes=4, dim=1)


def test_hand_example():
    # B=1, 3 rows, 2 heads, dim 2 (uint16), LSE [1, 2, 3]; 2 groups, split.
    a = np.arange(1, 13, dtype=np.uint16).reshape(1, 3, 2, 2)
    lse = np.array([[[100, 101, 102], [200, 201, 202]]], np.uint32).view(np.float32)
    fields = [dict(ROWS, heads=2, dim=2, split=True), dict(LSE, heads=2, split=True)]
    ranges = [[(0, 3)], [(2, 1), (0, 1)]]
    seg, foff = oracle.xchg_layout(1, 2, ranges, fields)
    # segment 0: 3 rows x 1 head x 2 -> 12 bytes, LSE at 256 (12 bytes) -> 512
    # segment 1: rows 2, 0 -> 8 bytes, LSE at 256 (8 bytes) -> 512
    assert seg == [0, 512, 1024] and foff == [[0, 256], [0, 256]]
    buf = oracle.xchg_pack([a, lse], 2, ranges, fields, 1)
    assert list(buf[0:12].view(np.uint16)) == [1, 2, 5, 6, 9, 10]        # head 0, rows 0..2
    assert list(buf[256:268].view(np.uint32)) == [100, 101, 102]
    assert list(buf[512:520].view(np.uint16)) == [11, 12, 3, 4]          # head 1, rows 2, 0
    assert list(buf[768:776].view(np.uint32)) == [202, 200]


def _rand_bits(rng, shape, eb):
    if eb == 2:
        return rng.integers(0, 2**16, size=shape, dtype=np.uint16)
    return rng.integers(0, 2**32, size=shape, dtype=np.uint64).astype(np.uint32).view(np.float32)


def test_roundtrip_restores_bits():
    rng = np.random.default_rng(3)
    b, r, h = 2, 11, 4
    fields = [dict(ROWS, heads=h, dim=8, split=True), dict(kind="rows", elem_bytes=4, heads=2,
                                                            dim=4, split=False),
              dict(LSE, heads=h, split=True)]
    arrs = [_rand_bits(rng, (b, r, h, 8), 2), _rand_bits(rng, (b, r, 2, 4), 4),
            _rand_bits(rng, (b, h, r), 4)]
    arrs[2].view(np.uint32)[0, 0, :4] = [0xFF800000, 0x80000000, 0x7FC00123, 0x00000001]
    # every segment covers all rows, in a different order of ranges
    ranges = [[(0, 11)], [(6, 5), (0, 6)], [(10, 1), (0, 4), (4, 6)], [(0, 11)]]
    buf = oracle.xchg_pack(arrs, 4, ranges, fields, b)
    outs = [np.zeros_like(x) for x in arrs]
    oracle.xchg_unpack(buf, 4, ranges, fields, b, outs)
    for x, y in zip(arrs, outs):
        assert x.tobytes() == y.tobytes()


def _a2a(send, seg_offs):
    """recv[g] = concatenation over senders r of segment g of send[r]."""
    n = len(send)
    return [np.concatenate([send[r][seg_offs[r][g]:seg_offs[r][g + 1]] for r in range(n)])
            for g in range(n)]


def test_head_parallel_round_trip_cp4():
    rng = np.random.default_rng(5)
    cp, c, h, hkv, d = 4, 3, 8, 4, 8          # 8 chunks of 3 rows, 24 rows in all
    total = 2 * cp * c
    full = dict(q=_rand_bits(rng, (1, total, h, d), 2), k=_rand_bits(rng, (1, total, hkv, d), 2),
                lse=_rand_bits(rng, (1, h, total), 4))
    chunks = [[(r * c, c), ((2 * cp - 1 - r) * c, c)] for r in range(cp)]
    rows_of = [np.concatenate([np.arange(a, a + n) for a, n in ch]) for ch in chunks]
    local = [dict(q=full["q"][:, rw], k=full["k"][:, rw], lse=full["lse"][:, :, rw])
             for rw in rows_of]
    send_f = [dict(ROWS, heads=h, dim=d, split=True), dict(ROWS, heads=hkv, dim=d, split=True),
              dict(LSE, heads=h, split=True)]
    recv_f = [dict(ROWS, heads=h // cp, dim=d, split=False),
              dict(ROWS, heads=hkv // cp, dim=d, split=False),
              dict(LSE, heads=h // cp, split=False)]
    # seq -> heads
    every = [[(0, 2 * c)]] * cp
    sends = [oracle.xchg_pack([x["q"], x["k"], x["lse"]], cp, every, send_f, 1) for x in local]
    offs = [oracle.xchg_layout(1, cp, every, send_f)[0]] * cp
    recvs = _a2a(sends, offs)
    hp = []
    for g in range(cp):
        assert oracle.xchg_layout(1, cp, chunks, recv_f)[0][-1] == recvs[g].size
        outs = [np.zeros((1, total, h // cp, d), np.uint16),
                np.zeros((1, total, hkv // cp, d), np.uint16),
                np.zeros((1, h // cp, total), np.float32)]
        oracle.xchg_unpack(recvs[g], cp, chunks, recv_f, 1, outs)
        hs, ks = slice(g * h // cp, (g + 1) * h // cp), slice(g * hkv // cp, (g + 1) * hkv // cp)
        assert outs[0].tobytes() == np.ascontiguousarray(full["q"][:, :, hs]).tobytes()
        assert outs[1].tobytes() == np.ascontiguousarray(full["k"][:, :, ks]).tobytes()
        assert outs[2].view(np.uint32).tobytes() == \
            np.ascontiguousarray(full["lse"][:, hs]).view(np.uint32).tobytes()
        hp.append(outs)
    # heads -> seq (the return trip, with the roles swapped)
    back_send = [oracle.xchg_pack(hp[g], cp, chunks, recv_f, 1) for g in range(cp)]
    back_offs = [oracle.xchg_layout(1, cp, chunks, recv_f)[0]] * cp
    back = _a2a(back_send, back_offs)
    for r in range(cp):
        outs = [np.zeros_like(local[r]["q"]), np.zeros_like(local[r]["k"]),
                np.zeros_like(local[r]["lse"])]
        oracle.xchg_unpack(back[r], cp, every, send_f, 1, outs)
        assert outs[0].tobytes() == np.ascontiguousarray(local[r]["q"]).tobytes()
        assert outs[1].tobytes() == np.ascontiguousarray(local[r]["k"]).tobytes()
        assert outs[2].view(np.uint32).tobytes() == \
            np.ascontiguousarray(local[r]["lse"]).view(np.uint32).tobytes()
