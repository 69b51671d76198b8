"""The product packer / unpacker against the oracle's, bit for bit (CPU)."""
import numpy as np
import pytest

import binary_g128_bit_amd as tq
import oracle
from binary_g128_bit_amd import synth


@pytest.mark.parametrize("variant", [tq.TQ_TERNARY, tq.TQ_BINARY])
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
