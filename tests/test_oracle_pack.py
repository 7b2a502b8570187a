"""Oracle pack/unpack: exact round trip, raw-bit preservation, and a
hand-written layout example."""
import numpy as np

import oracle


def test_roundtrip_bits_bf16_and_fp32():
    rng = np.random.default_rng(0)
    for dt in (np.uint16, np.float32):
        b, s, h, dv = 2, 5, 4, 8
        if dt == np.uint16:
            o = rng.integers(0, 2**16, size=(b, s, h, dv), dtype=np.uint16)
        else:
            o = rng.integers(0, 2**32, size=(b, s, h, dv), dtype=np.uint64)
            o = o.astype(np.uint32).view(np.float32)
        lse_bits = rng.integers(0, 2**32, size=(b, h, s), dtype=np.uint64).astype(np.uint32)
        # include -inf, +0/-0, NaN payloads and denormals
        lse_bits[0, 0, :4] = [0xFF800000, 0x00000000, 0x80000000, 0x7FC00123]
        lse_bits[1, 2, 0] = 0x00000001
        lse = lse_bits.view(np.float32)
        for groups in (1, 2, 4):
            buf = oracle.pack_saved(o, lse, groups)
            o2, l2 = oracle.unpack_saved(buf, b, s, h, dv, o.dtype, groups)
            assert o2.tobytes() == o.tobytes()
            assert l2.view(np.uint32).tobytes() == lse_bits.tobytes()


def test_layout_hand_example():
    """B=1, S=2, H=2, Dv=2 bf16-sized elements, 2 groups.

    Segment g holds head g: O rows (s=0: d0 d1, s=1: d0 d1), then at byte 256
    the LSE of that head for s=0, 1.  Each segment is 512 bytes.
    """
    o = np.array([[[[1, 2], [3, 4]], [[5, 6], [7, 8]]]], dtype=np.uint16)  # [1,2,2,2]
    lse = np.array([[[10, 11], [12, 13]]], dtype=np.uint32).view(np.float32)  # [1,2,2]
    seg, ob, loff = oracle.pack_layout(1, 2, 2, 2, 2, 2)
    assert (seg, ob, loff) == (512, 8, 256)
    buf = oracle.pack_saved(o, lse, 2)
    assert buf.size == 1024
    assert list(buf[0:8].view(np.uint16)) == [1, 2, 5, 6]
    assert list(buf[256:264].view(np.uint32)) == [10, 11]
    assert list(buf[512:520].view(np.uint16)) == [3, 4, 7, 8]
    assert list(buf[768:776].view(np.uint32)) == [12, 13]
