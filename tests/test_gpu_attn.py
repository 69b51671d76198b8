"""4-bit KV cache and decode attention against the oracle (needs an MI355X).

The cache written by tq_kv_append is read back, turned from the physical
layout documented in include/tq.h into logical order (a restatement of that
layout here, in numpy) and compared with the oracle's quantizer bit for bit.
Attention outputs must satisfy |o - o_ref| <= 2e-3 * A + 1e-5 per element with
A = sum_t p_t |v_t| from the oracle.
"""
import numpy as np
import pytest

import binary_g128_bit_amd as tq
import oracle
from binary_g128_bit_amd import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _tau(c, s):
    return 4 * c + s if s < 4 else 12 + 4 * c + s


def logical_k(kc, n_kv, T):
    """K codes [n_kv][TC][32] uint32 -> nibbles [n_kv][T][256]."""
    w = kc.reshape(n_kv, -1, 32)[:, :T].astype(np.uint32)
    out = np.empty((n_kv, T, 256), np.uint8)
    for c in range(4):
        for g in range(8):
            word = w[:, :, 8 * c + g]
            for e in range(8):
                sh = 16 * (e & 1) + 4 * (e >> 1)
                out[:, :, 32 * g + 8 * c + e] = (word >> sh) & 0xF
    return out


def logical_v(vc, vs, n_kv, T, TC):
    """V codes [n_kv][TC/32][1024] uint32 and scales [n_kv][TC/32][256] ->
    nibbles [n_kv][T][256], scales [n_kv][T][8]."""
    nblk = TC // 32
    w = vc.reshape(n_kv, nblk, 4, 16, 16).astype(np.uint32)   # [h][blk][c][n][j]
    sc = vs.reshape(n_kv, nblk, 4, 8, 8)                       # [h][blk][c][g][s]
    nib = np.empty((n_kv, nblk * 32, 256), np.uint8)
    scales = np.empty((n_kv, nblk * 32, 8), np.float16)
    for c in range(4):
        for s in range(8):
            sh = 16 * (s & 1) + 4 * (s >> 1)
            tok = np.arange(nblk) * 32 + _tau(c, s)
            vals = (w[:, :, c] >> sh) & 0xF                         # [h][blk][n][j]
            nib[:, tok, :] = vals.transpose(0, 1, 3, 2).reshape(n_kv, nblk, 256)
            scales[:, tok, :] = sc[:, :, c, :, s]
    return nib[:, :T], scales[:, :T]


class Cache:
    def __init__(self, n_kv, TC):
        self.n_kv, self.TC = n_kv, TC
        mk = lambda part, dt: torch.zeros(tq.tq_kv_bytes(n_kv, TC, part) // np.dtype(dt).itemsize,
                                          dtype={np.uint8: torch.uint8, np.uint16: torch.int16}[dt],
                                          device="cuda")
        self.kc = mk(tq.TQ_KV_K_CODES, np.uint8)
        self.ks = mk(tq.TQ_KV_K_SCALES, np.uint16)
        self.vc = mk(tq.TQ_KV_V_CODES, np.uint8)
        self.vs = mk(tq.TQ_KV_V_SCALES, np.uint16)

    def append(self, k, v, pos):
        tq.tq_kv_append(up(k), up(v), pos, self.n_kv, self.TC, self.kc, self.ks, self.vc, self.vs)

    def logical(self, T):
        torch.cuda.synchronize()
        kn = logical_k(self.kc.cpu().numpy().view(np.uint32), self.n_kv, T)
        ks = self.ks.cpu().numpy().view(np.float16).reshape(self.n_kv, self.TC, 8)[:, :T]
        vn, vs = logical_v(self.vc.cpu().numpy().view(np.uint32),
                           self.vs.cpu().numpy().view(np.float16), self.n_kv, T, self.TC)
        return kn, ks, vn, vs


def up(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def kv_inputs(seed, T, n_kv):
    g = synth.rng(seed)
    k = (g.standard_normal((T, n_kv, 256)) * np.exp(g.normal(0, 1, (T, n_kv, 1)))).astype(np.float16)
    v = (g.standard_normal((T, n_kv, 256)) * np.exp(g.normal(0, 1, (T, n_kv, 1)))).astype(np.float16)
    return k, v


def oracle_cache(k, v):
    T, n_kv = k.shape[0], k.shape[1]
    kn, ks = oracle.kv_quant(k.transpose(1, 0, 2).reshape(-1, 256))
    vn, vs = oracle.kv_quant(v.transpose(1, 0, 2).reshape(-1, 256))
    return (kn.reshape(n_kv, T, 256), ks.reshape(n_kv, T, 8), vn.reshape(n_kv, T, 256),
            vs.reshape(n_kv, T, 8))


@pytest.mark.parametrize("T,n_kv,TC", [(1, 1, 32), (33, 2, 64), (100, 4, 128), (1000, 4, 1024)])
def test_kv_append_bit_exact(T, n_kv, TC):
    k, v = kv_inputs(19000 + T, T, n_kv)
    # special groups: zeros, ties at half steps, subnormals, a signed zero
    k[0, 0, :32] = 0
    k[0, 0, 32:64] = np.float16(7.0)
    k[0, 0, 32:40] = [7, -7, 3.5, 2.5, -2.5, 0.5, 1.5, -0.0]
    v[-1, -1, 64:96] = np.float16(2.0 ** -20)
    v[-1, -1, 64] = np.float16(-(2.0 ** -24))
    c = Cache(n_kv, TC)
    c.append(k, v, 0)
    got = c.logical(T)
    ref = oracle_cache(k, v)
    for a, b, name in zip(got, ref, ("K codes", "K scales", "V codes", "V scales")):
        assert np.array_equal(np.asarray(a).view(np.uint8), np.asarray(b).view(np.uint8)), name


def test_kv_append_token_by_token_and_overwrite():
    """Single-token appends share value dwords with earlier tokens; a rewrite
    of a position replaces only that token."""
    T, n_kv, TC = 70, 4, 96
    k, v = kv_inputs(19500, T, n_kv)
    c = Cache(n_kv, TC)
    c.append(k[:5], v[:5], 0)
    for t in range(5, T):
        c.append(k[t:t + 1], v[t:t + 1], t)
    k2, v2 = kv_inputs(19501, 3, n_kv)
    c.append(k2, v2, 40)
    k[40:43], v[40:43] = k2, v2
    got = c.logical(T)
    ref = oracle_cache(k, v)
    for a, b, name in zip(got, ref, ("K codes", "K scales", "V codes", "V scales")):
        assert np.array_equal(np.asarray(a).view(np.uint8), np.asarray(b).view(np.uint8)), name


def run_attention(q, c, T, n_q):
    ws_bytes = tq.tq_attn_workspace_bytes(T, n_q, c.n_kv)
    ws = torch.empty(ws_bytes // 4, dtype=torch.float32, device="cuda")
    out = tq.tq_attn_decode(up(q), c.kc, c.ks, c.vc, c.vs, T, c.n_kv, c.TC, ws)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


def attention_case(seed, T, n_kv, n_q, TC=None, qscale=1.0):
    TC = TC or (T + 31) // 32 * 32
    k, v = kv_inputs(seed, T, n_kv)
    g = synth.rng(seed + 1)
    q = (g.standard_normal((n_q, 256)) * qscale).astype(np.float16)
    c = Cache(n_kv, TC)
    c.append(k, v, 0)
    return q, c, oracle_cache(k, v)


def assert_attn(out, ref, A, what):
    err = np.abs(out - ref)
    bad = err > 2e-3 * A + 1e-5
    assert not bad.any(), "%s: %d bad, worst err %.3g (A %.3g)" % (what, bad.sum(), err.max(), A.max())


@pytest.mark.parametrize("T", [1, 2, 31, 32, 33, 127, 128, 129, 513, 1000, 4096, 4099])
def test_attn_decode_gqa6(T):
    n_kv, n_q = 4, 24
    q, c, (kn, ks, vn, vs) = attention_case(20000 + T, T, n_kv, n_q)
    ref, A = oracle.attn_decode(q, kn, ks, vn, vs)
    assert_attn(run_attention(q, c, T, n_q), ref, A, "T=%d" % T)


@pytest.mark.parametrize("n_kv,n_q", [(1, 1), (2, 2), (1, 16), (8, 64), (3, 12)])
def test_attn_decode_head_groups(n_kv, n_q):
    T = 300
    q, c, (kn, ks, vn, vs) = attention_case(20500 + n_q, T, n_kv, n_q, TC=320)
    ref, A = oracle.attn_decode(q, kn, ks, vn, vs)
    assert_attn(run_attention(q, c, T, n_q), ref, A, "n_kv=%d n_q=%d" % (n_kv, n_q))


def test_attn_decode_peaked_and_capacity():
    """Large query norms (near one-hot softmax), a cache whose capacity is far
    above T, and a second call reusing the workspace."""
    T, n_kv, n_q = 777, 4, 24
    q, c, (kn, ks, vn, vs) = attention_case(20600, T, n_kv, n_q, TC=4096, qscale=8.0)
    ref, A = oracle.attn_decode(q, kn, ks, vn, vs)
    assert_attn(run_attention(q, c, T, n_q), ref, A, "peaked")
    # a shorter prefix of the same cache
    ref2, A2 = oracle.attn_decode(q, kn[:, :100], ks[:, :100], vn[:, :100], vs[:, :100])
    assert_attn(run_attention(q, c, 100, n_q), ref2, A2, "prefix")


def test_attn_decode_long_context_sampled():
    """32K cached tokens at the model's 4 KV heads and 24 query heads: the
    oracle on two KV heads' query groups."""
    T, n_kv, n_q = 32768, 4, 24
    q, c, (kn, ks, vn, vs) = attention_case(20700, T, n_kv, n_q)
    out = run_attention(q, c, T, n_q)
    for h in (0, 3):
        ref, A = oracle.attn_decode(q[6 * h: 6 * h + 6], kn[h:h + 1], ks[h:h + 1], vn[h:h + 1],
                                    vs[h:h + 1])
        assert_attn(out[6 * h: 6 * h + 6], ref, A, "32K kv head %d" % h)


@pytest.mark.parametrize("T,n_q", [(32768, 4), (65536, 16)])
def test_attn_decode_one_kv_head_many_chunks(T, n_q):
    """One KV head splits into 256 and 512 chunks: the chunk merge folds
    several rounds of 32 chunks per wave."""
    q, c, (kn, ks, vn, vs) = attention_case(20800 + n_q, T, 1, n_q)
    ref, A = oracle.attn_decode(q, kn, ks, vn, vs)
    assert_attn(run_attention(q, c, T, n_q), ref, A, "T=%d n_q=%d" % (T, n_q))


def test_attn_decode_errors():
    c = Cache(4, 64)
    q = torch.zeros(24, 256, dtype=torch.float16, device="cuda")
    ws = torch.empty(16, dtype=torch.float32, device="cuda")
    with pytest.raises(tq.TQError) as e:
        tq.tq_attn_decode(q, c.kc, c.ks, c.vc, c.vs, 10, 4, 64, ws)   # workspace too small
    assert e.value.status == 2
    big = torch.empty(tq.tq_attn_workspace_bytes(64, 24, 4) // 4, dtype=torch.float32, device="cuda")
    with pytest.raises(tq.TQError) as e:
        tq.tq_attn_decode(q, c.kc, c.ks, c.vc, c.vs, 65, 4, 64, big)  # T above capacity
    assert e.value.status == 2
    with pytest.raises(tq.TQError) as e:
        tq.tq_kv_append(torch.zeros(2, 4, 256, dtype=torch.float16, device="cuda"),
                        torch.zeros(2, 4, 256, dtype=torch.float16, device="cuda"), 63, 4, 64,
                        c.kc, c.ks, c.vc, c.vs)                               # past the capacity
    assert e.value.status == 2


@pytest.mark.parametrize("T", [1, 37, 100, 4099])
def test_attn_decode_ignores_cache_contents_past_T(T):
    """The cache memory past T holds NaN and Inf scale patterns and random
    codes (as after torch.empty and an earlier sequence): the outputs must
    still match the oracle on the first T tokens.  Tokens past T only sit in
    the same 32-token blocks as the last real ones; nothing past t_cap is
    read."""
    n_kv, n_q = 4, 24
    TC = (T + 31) // 32 * 32 + 64
    k, v = kv_inputs(21000 + T, T, n_kv)
    g = synth.rng(21100 + T)
    q = g.standard_normal((n_q, 256)).astype(np.float16)
    c = Cache(n_kv, TC)
    specials = torch.tensor([0x7E00, 0x7C00, -1024, 0x7FFF], dtype=torch.int32)  # NaN, Inf, -Inf, NaN
    for arr in (c.ks, c.vs):
        idx = torch.from_numpy(g.integers(0, 4, arr.numel())).long()
        arr.copy_(specials[idx].to(torch.int16).cuda())
    for arr in (c.kc, c.vc):
        arr.copy_(torch.from_numpy(g.integers(0, 256, arr.numel()).astype(np.uint8)).cuda())
    c.append(k, v, 0)
    kn, ks, vn, vs = oracle_cache(k, v)
    ref, A = oracle.attn_decode(q, kn, ks, vn, vs)
    out = run_attention(q, c, T, n_q)
    assert np.isfinite(out).all(), "non-finite output"
    assert_attn(out, ref, A, "garbage past T=%d" % T)
