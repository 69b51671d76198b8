"""Affine 2-bit GEMV (w = s * q + b per group) against the oracle, through
tq_gemv_affine (needs an MI355X).

Bars: bit-exact on the integer-exact sets (integer activations in [-8, 8],
power-of-two scales, biases -k 2^-j); elsewhere |y - y_ref| <= 2e-3 * A + 1e-5
with A = sum_g (|s| sum |q x| + |b| sum |x|) from the oracle.  Codes come from
the oracle's packer.
"""
import numpy as np
import pytest

import binary_g128_bit_amd as tq
import oracle
from binary_g128_bit_amd import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

THREADS = oracle.default_threads()


def up(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def case(seed, N, K, exact):
    q, s, b, X = synth.affine_problem(seed, N, K, 1, exact)
    return oracle.pack(q, oracle.AFFINE2), s, b, X[0]


def gpu(codes, s, b, x):
    y = tq.tq_gemv_affine(up(codes), up(s), up(b), up(x))
    torch.cuda.synchronize()
    return y.cpu().numpy().astype(np.float64)


def assert_tol(y, yref, A, what=""):
    err = np.abs(y - yref)
    bad = err > 2e-3 * A + 1e-5
    assert not bad.any(), "%s: %d bad, worst err %.3g" % (what, bad.sum(), err.max())


SHAPES = [(1, 128), (7, 256), (33, 384), (100, 640), (1000, 1024), (257, 5120), (129, 6144),
          (65, 17408), (3, 20480), (300, 2176), (300, 9216), (100, 4608), (2048, 6144), (6144, 5120)]


@pytest.mark.parametrize("N,K", SHAPES)
def test_affine_integer_exact(N, K):
    codes, s, b, x = case(17000 + N + K, N, K, exact=True)
    yref, _ = oracle.affine_gemm(codes, s, b, x, N, K, threads=THREADS)
    assert np.array_equal(gpu(codes, s, b, x), yref[0])


@pytest.mark.parametrize("N,K", [(64, 5120), (20, 17408)])
def test_affine_saturated_neighbour_dwords(N, K):
    """Code dwords of level 3 (every bit set) next to dwords of level 0 and
    the reverse, row by row, plus rows of one level-3 weight per dword: bits
    of one dword leaking into its neighbour's shifted copies would change
    these rows.  Integer-exact inputs, so the bar is bit-exact."""
    _, s, b, X = synth.affine_problem(17700 + N + K, N, K, 1, True)
    q = np.empty((N, K), np.int8)
    for n in range(N):
        hi, lo = (3, 0) if n % 2 == 0 else (0, 3)
        for d in range(K // 16):
            q[n, d * 16:(d + 1) * 16] = hi if d % 2 == 0 else lo
        if n % 4 == 3:
            q[n] = 0
            q[n, 15::16] = 3
    codes = oracle.pack(q, oracle.AFFINE2)
    yref, _ = oracle.affine_gemm(codes, s, b, X[0], N, K, threads=THREADS)
    assert np.array_equal(gpu(codes, s, b, X[0]), yref[0])


@pytest.mark.parametrize("N,K", SHAPES)
def test_affine_random(N, K):
    codes, s, b, x = case(18000 + N + K, N, K, exact=False)
    yref, A = oracle.affine_gemm(codes, s, b, x, N, K, threads=THREADS)
    assert_tol(gpu(codes, s, b, x), yref[0], A[0], "N=%d K=%d" % (N, K))


@pytest.mark.parametrize("N,K", [(2 * synth.GATE_UP[0], synth.GATE_UP[1]), synth.DOWN,
                                 synth.LM_HEAD])
def test_affine_full_size_sampled(N, K):
    codes, s, b, x = case(synth.seed_for(7, N % 97), N, K, exact=False)
    y = gpu(codes, s, b, x)
    g = synth.rng(N % 89)
    rows = np.unique(np.concatenate([[0, 1, N - 1], g.integers(0, N, 384)]))
    yref, A = oracle.affine_gemm(codes[rows], s[rows], b[rows], x, len(rows), K, threads=THREADS)
    assert_tol(y[rows], yref[0], A[0], "%dx%d" % (N, K))


def test_affine_matches_ternary_weights():
    """Ternary codes are affine codes with q = t + 1 and b = -s: the affine
    product of the same bytes follows the ternary oracle."""
    N, K = 512, 5120
    t, s, X = synth.problem(18500, N, K)
    codes = oracle.pack(t)
    y = gpu(codes, s, (-s.astype(np.float32)).astype(np.float16), X[0])
    yref, A = oracle.gemv(codes, s, X[0], N, K)
    # the affine bound: |s| sum |q x| + |s| sum |x| <= 3 |s| sum |x|
    Aaff = 3 * np.abs(np.repeat(s.astype(np.float64), 128, axis=1)) @ np.abs(X[0].astype(np.float64))
    assert_tol(y, yref, Aaff, "ternary as affine")


def test_affine_special_values():
    """Level-0 rows give sum_g b_g sum x_g; zero and subnormal scales and
    biases, negative scales, subnormal activations."""
    N, K = 64, 1024
    g = synth.rng(18600)
    q = synth.levels(g, N, K)
    q[:4] = 0
    s = synth.scales(g, N, K)
    b = synth.biases(g, N, K)
    s[5, :] = -s[5, :]
    s[6, 1] = np.float16(0.0)
    b[7, 2] = np.float16(0.0)
    s[8, 3] = np.float16(2.0 ** -20)
    b[9, 4] = np.float16(-(2.0 ** -22))
    x = synth.activations(g, 1, K)[0]
    x[3] = np.float16(2.0 ** -23)
    codes = oracle.pack(q, oracle.AFFINE2)
    y = gpu(codes, s, b, x)
    yref, A = oracle.affine_gemm(codes, s, b, x, N, K)
    assert_tol(y, yref[0], A[0], "special")


def test_affine_deterministic_and_limits():
    N, K = 2048, 5120
    codes, s, b, x = case(18700, N, K, exact=False)
    cd, sd, bd, xd = up(codes), up(s), up(b), up(x)
    y0 = tq.tq_gemv_affine(cd, sd, bd, xd)
    y1 = tq.tq_gemv_affine(cd, sd, bd, xd)
    torch.cuda.synchronize()
    assert torch.equal(y0, y1)
    K2 = 20480 + 128
    c2 = torch.zeros(2, K2 // 4, dtype=torch.uint8, device="cuda")
    s2 = torch.zeros(2, K2 // 128, dtype=torch.float16, device="cuda")
    with pytest.raises(tq.TQError) as e:
        tq.tq_gemv_affine(c2, s2, s2, torch.zeros(K2, dtype=torch.float16, device="cuda"))
    assert e.value.status == 2
    with pytest.raises(tq.TQError) as e:
        tq.tq_gemv(cd, sd, xd, variant=tq.TQ_AFFINE2)
    assert e.value.status == 4
