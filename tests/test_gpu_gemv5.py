"""Five-trit-per-byte ternary GEMV (TQ_TERNARY5) against the oracle, through
the C ABI (needs an MI355X).

Bars as for the 2-bit GEMV: bit-exact on the integer-exact sets (integer
activations in [-8, 8], power-of-two scales), elsewhere
|y - y_ref| <= 2e-3 * A + 1e-5 per element with A = sum |s * t * x|.
Codes come from the oracle's packer.
"""
import numpy as np
import pytest

import binary_g128_bit_amd as tq
import oracle
from binary_g128_bit_amd import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

T5 = tq.TQ_TERNARY5
THREADS = oracle.default_threads()


def up(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def case(seed, N, K, exact):
    t, s, X = synth.problem(seed, N, K, 1, T5, exact)
    return oracle.pack(t, T5), s, X[0]


def gpu(codes, s, x):
    y = tq.tq_gemv(up(codes), up(s), up(x), variant=T5)
    torch.cuda.synchronize()
    return y.cpu().numpy().astype(np.float64)


def assert_tol(y, yref, A, what=""):
    err = np.abs(y - yref)
    bad = err > 2e-3 * A + 1e-5
    assert not bad.any(), "%s: %d bad, worst err %.3g" % (what, bad.sum(), err.max())


# K spans odd group counts (128, 384, 640, 2176: the table kernel), every
# capacity class of the register kernel's shape table, exact and ragged shapes,
# its 20480 maximum (320 chunks, the most LDS) and the table kernel's 40960
SHAPES = [(1, 128), (7, 256), (33, 384), (100, 640), (1000, 1024), (65, 2176), (257, 5120),
          (129, 6144), (40, 17408), (9, 20480), (3, 29952), (5, 40960), (77, 10240), (300, 3072)]


@pytest.mark.parametrize("N,K", SHAPES)
def test_gemv5_integer_exact(N, K):
    codes, s, x = case(14000 + N + K, N, K, exact=True)
    yref, _ = oracle.gemv(codes, s, x, N, K, T5, threads=THREADS)
    assert np.array_equal(gpu(codes, s, x), yref)


@pytest.mark.parametrize("N,K", SHAPES)
def test_gemv5_random(N, K):
    codes, s, x = case(15000 + N + K, N, K, exact=False)
    yref, A = oracle.gemv(codes, s, x, N, K, T5, threads=THREADS)
    assert_tol(gpu(codes, s, x), yref, A, "N=%d K=%d" % (N, K))


def _sampled_rows(N, n, seed):
    g = synth.rng(seed)
    return np.unique(np.concatenate([[0, 1, N - 1], g.integers(0, N, n)]))


@pytest.mark.parametrize("N,K", [(2 * synth.GATE_UP[0], synth.GATE_UP[1]), synth.DOWN,
                                 synth.LM_HEAD])
def test_gemv5_full_size_sampled(N, K):
    """[gate;up] 34816 x 5120, down 5120 x 17408 and the 248320 x 5120 head at
    the launch shapes the bench times; the oracle on sampled rows."""
    codes, s, x = case(synth.seed_for(6, N % 97), N, K, exact=False)
    y = gpu(codes, s, x)
    rows = _sampled_rows(N, 384, N % 89)
    yref, A = oracle.gemv(codes[rows], s[rows], x, len(rows), K, T5, threads=THREADS)
    assert_tol(y[rows], yref, A, "%dx%d" % (N, K))


def test_gemv5_special_values():
    """Rows of zero trits stay within the bar (A = 0 there, so |y| <= 1e-5:
    the decode's slot offsets cancel up to fp32 rounding); negative, zero and
    subnormal scales and subnormal activations follow the oracle."""
    N, K = 64, 1024
    g = synth.rng(16000)
    t = synth.trits(g, N, K, T5)
    t[:8] = 0
    s = synth.scales(g, N, K)
    s[8, :] = -s[8, :]
    s[9, 2] = np.float16(0.0)
    s[10, 3] = np.float16(2.0 ** -20)
    x = synth.activations(g, 1, K)[0]
    x[5] = np.float16(2.0 ** -22)
    x[700] = np.float16(-(2.0 ** -24))
    codes = oracle.pack(t, T5)
    y = gpu(codes, s, x)
    yref, A = oracle.gemv(codes, s, x, N, K, T5)
    assert np.all(np.abs(y[:8]) <= 1e-5)
    assert_tol(y, yref, A, "special")


def test_gemv5_deterministic_and_stream():
    N, K = 4096, 5120
    codes, s, x = case(16100, N, K, exact=False)
    cd, sd, xd = up(codes), up(s), up(x)
    y0 = tq.tq_gemv(cd, sd, xd, variant=T5)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        y1 = tq.tq_gemv(cd, sd, xd, variant=T5, stream=side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    assert torch.equal(y0, y1)
    # M == 1 through tq_gemm forwards to the same kernel
    Y = tq.tq_gemm(cd, sd, xd.reshape(1, K), variant=T5)
    torch.cuda.synchronize()
    assert torch.equal(Y[0], y0)


def test_gemv5_limits():
    K = 40960 + 128
    codes = torch.zeros(tq.tq_codes_bytes(2, K, T5), dtype=torch.uint8, device="cuda")
    s = torch.zeros(2, K // 128, dtype=torch.float16, device="cuda")
    x = torch.zeros(K, dtype=torch.float16, device="cuda")
    with pytest.raises(tq.TQError) as e:
        tq.tq_gemv(codes, s, x, variant=T5)
    assert e.value.status == 2
    X = torch.zeros(2, 256, dtype=torch.float16, device="cuda")
    c2 = torch.zeros(tq.tq_codes_bytes(4, 256, T5), dtype=torch.uint8, device="cuda")
    with pytest.raises(tq.TQError) as e:
        tq.tq_gemm(c2, torch.zeros(4, 2, dtype=torch.float16, device="cuda"), X, variant=T5)
    assert e.value.status == 4


def test_gemv5_scales_2byte_aligned():
    """A scale array that is only 2-byte aligned takes the per-scale loads."""
    N, K = 96, 5120
    codes, s, x = case(16200, N, K, exact=False)
    big = torch.zeros(N * (K // 128) + 1, dtype=torch.float16, device="cuda")
    big[1:] = up(s).reshape(-1)
    sv = big[1:].view(N, K // 128)
    y = tq.tq_gemv(up(codes), sv, up(x), variant=T5)
    torch.cuda.synchronize()
    yref, A = oracle.gemv(codes, s, x, N, K, T5)
    assert_tol(y.cpu().numpy().astype(np.float64), yref, A, "2-byte aligned scales")
