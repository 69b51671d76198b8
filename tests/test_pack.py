"""The product packer / unpacker against the oracle's, bit for bit (CPU)."""
import numpy as np
import pytest

import binary_g128_bit_amd as tq
import oracle
from binary_g128_bit_amd import synth


@pytest.mark.parametrize("variant", [tq.TQ_TERNARY, tq.TQ_BINARY, tq.TQ_TERNARY5])
@pytest.mark.parametrize("N,K", [(1, 128), (3, 256), (17, 384), (64, 1024), (5, 5120),
                                 (2, 17408), (33, 640)])
def test_pack_matches_oracle(variant, N, K):
    g = synth.rng(100 + N + K + variant)
    t = synth.trits(g, N, K, variant)
    mine = tq.tq_pack(t, variant)
    ref = oracle.pack(t, variant)
    assert mine.dtype == np.uint8 and mine.shape == ref.shape
    assert np.array_equal(mine, ref)
    assert np.array_equal(tq.tq_unpack(mine, N, K, variant), t)
    assert np.array_equal(tq.tq_unpack(mine, N, K, variant), oracle.unpack(ref, N, K, variant))


def test_all_bytes_unpack_like_oracle():
    for b in range(256):
        row = np.full((1, 32), b, np.uint8)
        try:
            ref = oracle.unpack(row, 1, 128)
        except oracle.OracleError as e:
            with pytest.raises(tq.TQError) as me:
                tq.tq_unpack(row, 1, 128)
            assert me.value.status == 6 and me.value.index == e.index
            continue
        assert np.array_equal(tq.tq_unpack(row, 1, 128), ref)
        rowb = np.full((1, 16), b, np.uint8)
        assert np.array_equal(tq.tq_unpack(rowb, 1, 128, tq.TQ_BINARY),
                              oracle.unpack(rowb, 1, 128, oracle.BINARY))


def test_pack_large_rows_and_extremes():
    N, K = 4, 17408
    for fill in (-1, 0, 1):
        t = np.full((N, K), fill, np.int8)
        assert np.array_equal(tq.tq_pack(t), oracle.pack(t))
    for fill in (-1, 1):
        t = np.full((N, K), fill, np.int8)
        assert np.array_equal(tq.tq_pack(t, tq.TQ_BINARY), oracle.pack(t, oracle.BINARY))


def test_ternary5_all_bytes_unpack_like_oracle():
    """Every byte value at every position class of a group (even, odd, the
    three-trit last byte) and in the second group: same trits, or the same
    error and index, as the oracle."""
    K = 256
    for pos in (0, 1, 24, 25, 26, 51):
        for b in range(256):
            row = np.zeros((1, 64), np.uint8)
            row[0, pos] = b
            try:
                ref = oracle.unpack(row, 1, K, oracle.TERNARY5)
            except oracle.OracleError as e:
                with pytest.raises(tq.TQError) as me:
                    tq.tq_unpack(row, 1, K, tq.TQ_TERNARY5)
                assert me.value.status == 6 and me.value.index == e.index, (pos, b)
                continue
            assert np.array_equal(tq.tq_unpack(row, 1, K, tq.TQ_TERNARY5), ref), (pos, b)


def test_ternary5_sizes_and_errors():
    assert tq.tq_codes_bytes(1, 5120, tq.TQ_TERNARY5) == 1040
    assert tq.tq_codes_bytes(3, 384, tq.TQ_TERNARY5) == 3 * 80
    assert tq.tq_codes_bytes(248320, 5120, tq.TQ_TERNARY5) == 248320 * 1040
    t = np.zeros((3, 384), np.int8)
    t[2, 301] = -2
    with pytest.raises(tq.TQError) as e:
        tq.tq_pack(t, tq.TQ_TERNARY5)
    assert e.value.status == 5 and e.value.index == 2 * 384 + 301
    with pytest.raises(oracle.OracleError) as eo:
        oracle.pack(t, oracle.TERNARY5)
    assert eo.value.index == e.value.index
    # padding bytes are written as zeros and never read
    c = tq.tq_pack(np.ones((2, 384), np.int8), tq.TQ_TERNARY5)
    assert c.shape == (2, 80) and np.all(c[:, 78:] == 0)
    c[:, 78:] = 0xFF
    assert np.all(tq.tq_unpack(c, 2, 384, tq.TQ_TERNARY5) == 1)


def test_affine_levels_pack_like_oracle():
    g = synth.rng(4242)
    for N, K in ((1, 128), (9, 384), (33, 5120)):
        q = synth.levels(g, N, K)
        mine = tq.tq_pack(q, tq.TQ_AFFINE2)
        assert np.array_equal(mine, oracle.pack(q, oracle.AFFINE2))
        assert np.array_equal(tq.tq_unpack(mine, N, K, tq.TQ_AFFINE2), q)
    # the ternary bytes of t are the affine bytes of q = t + 1
    t = synth.trits(g, 4, 256)
    assert np.array_equal(tq.tq_pack(t), tq.tq_pack((t + 1).astype(np.int8), tq.TQ_AFFINE2))
    bad = np.zeros((2, 128), np.int8)
    bad[1, 3] = 4
    with pytest.raises(tq.TQError) as e:
        tq.tq_pack(bad, tq.TQ_AFFINE2)
    assert e.value.status == 5 and e.value.index == 131
    allb = np.arange(256, dtype=np.uint8).reshape(8, 32)
    assert np.array_equal(tq.tq_unpack(allb, 8, 128, tq.TQ_AFFINE2),
                          oracle.unpack(allb, 8, 128, oracle.AFFINE2))

