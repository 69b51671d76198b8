"""Embedding rows through tq_embed against the oracle (needs an MI355X).

Each output is s * t with t in {-1, 0, +1}, exact in FP16, so the bar is
bit-exact FP16 output (signed zeros included) against the oracle's float64
rows converted to FP16, which is exact for these values.
"""
import numpy as np
import pytest

import binary_g128_bit_amd as tq
import oracle
from binary_g128_bit_amd import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TERN, BIN = tq.TQ_TERNARY, tq.TQ_BINARY


def up(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def table(seed, N, K, variant):
    g = synth.rng(seed)
    t = synth.trits(g, N, K, variant)
    s = synth.scales(g, N, K)
    return oracle.pack(t, variant), s


def special_scales(s):
    """Negative, zero, negative-zero and subnormal scales in a few groups."""
    s = s.copy()
    G = s.shape[1]
    s[0, 0] = -s[0, 0]
    s[-1, G - 1] = np.float16(-0.0)
    s[s.shape[0] // 2, G // 2] = np.float16(0.0)
    s[1 % s.shape[0], 0] = np.float16(2.0 ** -20)
    s[1 % s.shape[0], G - 1] = np.float16(-(2.0 ** -24))
    return s


def run(codes, s, ids, variant):
    out = tq.tq_embed(up(codes), up(s), up(ids.astype(np.int32)), variant=variant)
    torch.cuda.synchronize()
    return out.cpu().numpy().view(np.uint16)


def expect(codes, s, ids, N, K, variant):
    ref = oracle.embed(codes, s, ids, N, K, variant)
    return ref.astype(np.float16).view(np.uint16)


@pytest.mark.parametrize("variant", [TERN, BIN])
@pytest.mark.parametrize("N,K,n_ids", [(1, 128, 1), (5, 128, 17), (9, 384, 40), (300, 640, 257),
                                       (1000, 5120, 700), (40, 17408, 65), (3, 65536, 5)])
def test_embed_bit_exact(N, K, n_ids, variant):
    codes, s = table(12000 + N + K, N, K, variant)
    s = special_scales(s)
    g = synth.rng(12500 + n_ids)
    ids = g.integers(0, N, n_ids).astype(np.int32)
    ids[0] = N - 1
    ids[-1] = 0
    got = run(codes, s, ids, variant)
    assert got.shape == (n_ids, K)
    assert np.array_equal(got, expect(codes, s, ids, N, K, variant))


def test_embed_lm_head_table_sampled():
    """The 248320 x 5120 ternary token table, 512 ids (a prefill chunk)."""
    N, K = synth.LM_HEAD
    codes, s = table(synth.seed_for(5, 0), N, K, TERN)
    g = synth.rng(12900)
    ids = np.concatenate([[0, N - 1], g.integers(0, N, 510)]).astype(np.int32)
    got = run(codes, s, ids, TERN)
    assert np.array_equal(got, expect(codes, s, ids, N, K, TERN))


@pytest.mark.parametrize("variant", [TERN, BIN])
def test_embed_out_of_range_ids_give_zero_rows(variant):
    N, K = 20, 384
    codes, s = table(13000 + variant, N, K, variant)
    ids = np.array([3, -1, N, 19, -(2 ** 31), 2 ** 31 - 1, 0], np.int32)
    got = run(codes, s, ids, variant)
    ok = (ids >= 0) & (ids < N)
    assert np.array_equal(got[ok], expect(codes, s, ids[ok], N, K, variant))
    assert np.all(got[~ok] == 0)


def test_embed_empty_and_repeat_calls():
    N, K = 10, 256
    codes, s = table(13100, N, K, TERN)
    cd, sd = up(codes), up(s)
    empty = tq.tq_embed(cd, sd, torch.zeros(0, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    assert empty.shape == (0, K)
    ids = up(np.array([4, 4, 9], np.int32))
    a = tq.tq_embed(cd, sd, ids)
    b = tq.tq_embed(cd, sd, ids)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    assert torch.equal(a[0].view(torch.int16), a[1].view(torch.int16))


def test_embed_row_feeds_gemv():
    """A row gathered by tq_embed is the FP16 activation for tq_gemv: the GEMV
    of the gathered row matches the oracle GEMV of the oracle's row."""
    Ne, K, N = 64, 5120, 512
    codes_e, s_e = table(13200, Ne, K, TERN)
    codes_w, s_w = table(13201, N, K, TERN)
    ids = np.array([17], np.int32)
    row = tq.tq_embed(up(codes_e), up(s_e), up(ids))
    y = tq.tq_gemv(up(codes_w), up(s_w), row[0])
    torch.cuda.synchronize()
    x = oracle.embed(codes_e, s_e, ids, Ne, K, TERN)[0].astype(np.float16)
    yref, A = oracle.gemv(codes_w, s_w, x, N, K, TERN)
    err = np.abs(y.cpu().numpy().astype(np.float64) - yref)
    assert np.all(err <= 2e-3 * A + 1e-5), err.max()
