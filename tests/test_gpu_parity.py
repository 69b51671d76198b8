"""HIP path against the oracle, through the C ABI (needs an MI355X).

Bars: bit-exact on the integer-exact sets (integer activations in [-8, 8],
power-of-two scales: every partial sum is exact in fp32, so any summation order
gives the oracle's value); elsewhere |y - y_ref| <= 2e-3 * A + 1e-5 per element
with A = sum |s * t * x| from the oracle.
"""
import numpy as np
import pytest

import binary_g128_bit_amd as tq
import oracle
from binary_g128_bit_amd import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TERN, BIN = tq.TQ_TERNARY, tq.TQ_BINARY
THREADS = oracle.default_threads()


def up(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def gpu_gemm(codes, s, X, variant, N, K):
    """Y[M][N] through tq_gemv (M == 1) or tq_gemm."""
    cd, sd, Xd = up(codes), up(s), up(X)
    if X.shape[0] == 1:
        y = tq.tq_gemv(cd, sd, Xd[0], variant=variant)
        Y = y.reshape(1, N)
    else:
        Y = tq.tq_gemm(cd, sd, Xd, variant=variant)
    torch.cuda.synchronize()
    return Y.cpu().numpy()


def assert_tol(Y, Yref, A, what=""):
    err = np.abs(Y.astype(np.float64) - Yref)
    bound = 2e-3 * A + 1e-5
    bad = err > bound
    assert not bad.any(), "%s: %d bad, worst err %.3g vs bound %.3g; max err/A %.3g" % (
        what, bad.sum(), err[bad].max(), bound[bad][np.argmax(err[bad])], (err / np.maximum(A, 1e-30)).max())


def case(seed, N, K, M, variant, exact):
    t, s, X = synth.problem(seed, N, K, M, variant, exact)
    codes = oracle.pack(t, variant)
    return codes, s, X


SHAPES = [(1, 128), (7, 256), (33, 384), (100, 640), (1000, 1024), (257, 5120),
          (65, 17408), (9, 20480), (3, 29952), (129, 6144), (5, 65536), (70, 2176),
          (4096, 5120), (4100, 5120), (300, 9216), (97, 13312),
          (100, 4608), (99, 4608), (40, 14336), (2048, 6144), (1000, 10240), (6144, 5120), (8193, 5120)]


@pytest.mark.parametrize("variant", [TERN, BIN])
@pytest.mark.parametrize("N,K", SHAPES)
def test_gemv_integer_exact(N, K, variant):
    codes, s, X = case(7000 + N + K, N, K, 1, variant, exact=True)
    Y = gpu_gemm(codes, s, X, variant, N, K)
    Yref, _ = oracle.gemm(codes, s, X, N, K, variant, threads=THREADS)
    assert np.array_equal(Y.astype(np.float64), Yref)


@pytest.mark.parametrize("variant", [TERN, BIN])
@pytest.mark.parametrize("N,K", [(64, 5120), (20, 17408), (32, 6144)])
def test_gemv_saturated_neighbour_dwords(N, K, variant):
    """Every code dword all t = +1 (every bit of a dword set for binary)
    next to dwords of t = -1 or 0 and the reverse, row by row: a decode that
    let bits of one dword leak into its neighbour's shifted copies would
    change these rows.  Integer-exact inputs, so the bar is bit-exact."""
    _, s, X = synth.problem(7700 + N + K, N, K, 1, variant, exact=True)
    per = 16 if variant == TERN else 32              # weights per code dword
    lo = [-1, 0] if variant == TERN else [-1]
    t = np.empty((N, K), np.int8)
    for n in range(N):
        a, b = (1, lo[n % len(lo)]) if n % 2 == 0 else (lo[n % len(lo)], 1)
        for d in range(K // per):
            t[n, d * per:(d + 1) * per] = a if d % 2 == 0 else b
        if n % 4 == 3:                               # and a row of single set weights
            t[n] = lo[0]
            t[n, per - 1::per] = 1
    codes = oracle.pack(t, variant)
    Y = gpu_gemm(codes, s, X, variant, N, K)
    Yref, _ = oracle.gemm(codes, s, X, N, K, variant, threads=THREADS)
    assert np.array_equal(Y.astype(np.float64), Yref)


@pytest.mark.parametrize("variant", [TERN, BIN])
@pytest.mark.parametrize("N,K", SHAPES)
def test_gemv_random(N, K, variant):
    codes, s, X = case(8000 + N + K, N, K, 1, variant, exact=False)
    Y = gpu_gemm(codes, s, X, variant, N, K)
    Yref, A = oracle.gemm(codes, s, X, N, K, variant, threads=THREADS)
    assert_tol(Y, Yref, A, "N=%d K=%d" % (N, K))


def test_gemv_c1_ternary():
    N, K = synth.C1
    codes, s, X = case(synth.seed_for(1, 0), N, K, 1, TERN, exact=False)
    Y = gpu_gemm(codes, s, X, TERN, N, K)
    Yref, A = oracle.gemm(codes, s, X, N, K, TERN, threads=THREADS)
    assert_tol(Y, Yref, A, "C1")


# the decode shapes of the 27B-like stack, at full size
STACK_SHAPES = [synth.GATE_UP, synth.DOWN, (6144, 5120), (1024, 5120), (5120, 6144),
                (14336, 5120),
                # input-shared fusions: [gate; up], [q; k; v], [lin_qkv; lin_z]
                (34816, 5120), (8192, 5120), (20480, 5120)]


@pytest.mark.parametrize("variant", [TERN, BIN])
@pytest.mark.parametrize("N,K", STACK_SHAPES)
def test_gemv_full_size(N, K, variant):
    codes, s, X = case(synth.seed_for(2, N % 97 + K % 89), N, K, 1, variant, exact=False)
    Y = gpu_gemm(codes, s, X, variant, N, K)
    Yref, A = oracle.gemm(codes, s, X, N, K, variant, threads=THREADS)
    assert_tol(Y, Yref, A, "full %dx%d" % (N, K))
    # integer-exact at the same shape: bit for bit
    codes, s, X = case(synth.seed_for(2, 50 + N % 97), N, K, 1, variant, exact=True)
    Y = gpu_gemm(codes, s, X, variant, N, K)
    Yref, _ = oracle.gemm(codes, s, X, N, K, variant, threads=THREADS)
    assert np.array_equal(Y.astype(np.float64), Yref)


@pytest.mark.parametrize("K", [1024, 5120, 17408])
def test_gemv_special_values(K):
    """Negative and subnormal scales, subnormal and zero activations, all-zero
    and all-one trits (K = 5120 at 64 rows and K = 17408 run the tail-slot
    layouts)."""
    N = 64
    g = synth.rng(31)
    t = synth.trits(g, N, K, TERN)
    t[0] = 0
    t[1] = 1
    t[2] = -1
    s = synth.scales(g, N, K)
    s[3] = -s[3]
    s[4, :] = np.float16(2.0 ** -20)
    X = synth.activations(g, 1, K)
    X[0, :64] = np.float16(2.0 ** -24) * np.arange(64)
    X[0, 200:300] = 0
    codes = oracle.pack(t)
    Y = gpu_gemm(codes, s, X, TERN, N, K)
    Yref, A = oracle.gemm(codes, s, X, N, K, TERN)
    assert_tol(Y, Yref, A, "special")
    # all-zero trits: only the rounding residue of the per-group offsets
    # remains (it grows with the number of chunks summed)
    assert abs(Y[0, 0]) <= (1e-6 if K <= 1024 else 1e-5)


@pytest.mark.parametrize("p_zero", [0.9, 0.99, 1.0])
def test_gemv_sparse_rows(p_zero):
    """Mostly-zero trits make sum |s t x| small; the error must shrink with it."""
    N, K = 512, 5120
    g = synth.rng(int(p_zero * 1000))
    t = synth.trits(g, N, K, TERN)
    t[g.random((N, K)) < p_zero] = 0
    s = synth.scales(g, N, K)
    X = synth.activations(g, 1, K)
    codes = oracle.pack(t)
    Y = gpu_gemm(codes, s, X, TERN, N, K)
    Yref, A = oracle.gemm(codes, s, X, N, K, TERN)
    assert_tol(Y, Yref, A, "sparse %.2f" % p_zero)


def test_gemv_deterministic_and_canaries():
    N, K = synth.DOWN
    codes, s, X = case(9100, N, K, 1, TERN, exact=False)
    cd, sd, xd = up(codes), up(s), up(X[0])
    pad = 64
    ybig = torch.full((N + 2 * pad,), float("nan"), device="cuda")
    y = ybig[pad:pad + N]
    tq.tq_gemv(cd, sd, xd, y)
    torch.cuda.synchronize()
    first = y.clone()
    for _ in range(3):
        tq.tq_gemv(cd, sd, xd, y)
    torch.cuda.synchronize()
    assert torch.equal(first, y)
    assert torch.isnan(ybig[:pad]).all() and torch.isnan(ybig[pad + N:]).all()
    assert not torch.isnan(y).any()


@pytest.mark.parametrize("N,K", [(96, 5120), (65, 17408)])
def test_gemv_scales_2byte_aligned(N, K):
    """A scale array that is only 2-byte aligned (a view one half in) takes
    the per-scale loads instead of the aligned-dword ones; same results."""
    codes, s, X = case(9300 + N, N, K, 1, TERN, exact=False)
    big = torch.zeros(N * (K // 128) + 1, dtype=torch.float16, device="cuda")
    big[1:] = up(s).reshape(-1)
    sv = big[1:].view(N, K // 128)
    y = tq.tq_gemv(up(codes), sv, up(X[0]))
    y_al = tq.tq_gemv(up(codes), up(s), up(X[0]))
    torch.cuda.synchronize()
    yref, A = oracle.gemv(codes, s, X[0], N, K, threads=THREADS)
    assert_tol(y.cpu().numpy().astype(np.float64), yref, A, "2-byte aligned scales")
    assert_tol(y_al.cpu().numpy().astype(np.float64), yref, A, "aligned scales")


def test_gemv_rejects_k_above_limit():
    N, K = 4, 65536 + 128
    codes = torch.zeros(N * K // 4, dtype=torch.uint8, device="cuda")
    s = torch.zeros((N, K // 128), dtype=torch.float16, device="cuda")
    x = torch.zeros(K, dtype=torch.float16, device="cuda")
    with pytest.raises(tq.TQError) as e:
        tq.tq_gemv(codes, s, x)
    assert e.value.status == 2


def test_gemv_rejects_misaligned_device_pointer():
    N, K = 16, 256
    codes, s, X = case(9200, N, K, 1, TERN, exact=False)
    xbuf = torch.zeros(K + 8, dtype=torch.float16, device="cuda")
    with pytest.raises(tq.TQError) as e:
        tq.tq_gemv(up(codes), up(s), xbuf[1:1 + K])
    assert e.value.status == 7


@pytest.mark.parametrize("variant", [TERN, BIN])
@pytest.mark.parametrize("M", [2, 4, 8, 16, 64])
@pytest.mark.parametrize("N,K", [(33, 384), (300, 1024), (65, 5120)])
def test_gemm_small(M, N, K, variant):
    codes, s, X = case(9300 + M + N + K, N, K, M, variant, exact=True)
    Y = gpu_gemm(codes, s, X, variant, N, K)
    Yref, _ = oracle.gemm(codes, s, X, N, K, variant, threads=THREADS)
    assert np.array_equal(Y.astype(np.float64), Yref)
    codes, s, X = case(9400 + M + N + K, N, K, M, variant, exact=False)
    Y = gpu_gemm(codes, s, X, variant, N, K)
    Yref, A = oracle.gemm(codes, s, X, N, K, variant, threads=THREADS)
    assert_tol(Y, Yref, A, "gemm M=%d" % M)


def _sampled_rows(N, n, seed):
    g = synth.rng(seed)
    rows = np.unique(np.concatenate([[0, 1, N - 1], g.integers(0, N, n)]))
    return rows


@pytest.mark.parametrize("M", [2, 4, 8, 16, 64, 512])
@pytest.mark.parametrize("N,K", [synth.GATE_UP, synth.DOWN])
def test_gemm_full_size_sampled(M, N, K):
    """Speculative-verify / prefill widths on the MLP shapes: the full GEMM on
    the GPU, the oracle on sampled output rows."""
    codes, s, X = case(synth.seed_for(4, M + N % 7), N, K, M, TERN, exact=False)
    Y = gpu_gemm(codes, s, X, TERN, N, K)
    rows = _sampled_rows(N, 256 if M <= 64 else 64, M)
    Yref, A = oracle.gemm(codes[rows], s[rows], X, len(rows), K, TERN, threads=THREADS)
    assert_tol(Y[:, rows], Yref, A, "gemm M=%d %dx%d" % (M, N, K))


@pytest.mark.parametrize("M", [1, 8])
def test_lm_head_sampled(M):
    """Ternary LM head 5120 -> 248320 at batch 1 and 8."""
    N, K = synth.LM_HEAD
    codes, s, X = case(synth.seed_for(5, M), N, K, M, TERN, exact=False)
    Y = gpu_gemm(codes, s, X, TERN, N, K)
    rows = _sampled_rows(N, 512, 77 + M)
    Yref, A = oracle.gemm(codes[rows], s[rows], X, len(rows), K, TERN, threads=THREADS)
    assert_tol(Y[:, rows], Yref, A, "lm head M=%d" % M)


@pytest.mark.parametrize("variant", [TERN, BIN])
@pytest.mark.parametrize("M,N,K", [(3, 1, 128), (17, 70, 128), (31, 129, 256), (33, 64, 640),
                                   (100, 200, 2176), (5, 1000, 29952), (2, 77, 65536),
                                   (128, 128, 128), (130, 70, 384), (257, 300, 1024),
                                   (200, 129, 5120), (7, 33, 640), (6, 129, 17408),
                                   (8, 65, 5120), (6, 65600, 256), (2, 1001, 17408),
                                   (2, 33, 30080)])
def test_gemm_ragged(M, N, K, variant):
    """Ragged activation and weight tiles, K of one group (most waves of a
    workgroup idle), the largest K, 5..8 rows (eight staged rows) and two-row
    batches past the four-row kernel's staging (K = 30080: the two-row VALU
    kernel, near the capacity of its LDS tile)."""
    codes, s, X = case(9700 + M + N + K, N, K, M, variant, exact=True)
    Y = gpu_gemm(codes, s, X, variant, N, K)
    Yref, _ = oracle.gemm(codes, s, X, N, K, variant, threads=THREADS)
    assert np.array_equal(Y.astype(np.float64), Yref)
    codes, s, X = case(9800 + M + N + K, N, K, M, variant, exact=False)
    Y = gpu_gemm(codes, s, X, variant, N, K)
    Yref, A = oracle.gemm(codes, s, X, N, K, variant, threads=THREADS)
    assert_tol(Y, Yref, A, "gemm M=%d N=%d K=%d" % (M, N, K))


@pytest.mark.parametrize("variant", [TERN, BIN])
@pytest.mark.parametrize("M,N,K", [(200, 16500, 640), (128, 16384, 128), (300, 8200, 256)])
def test_gemm_tiled_ragged(M, N, K, variant):
    """Wide batches on the tiled kernel (at least 128 output tiles of 128 x 128):
    ragged activation and weight tiles, a single group of K, exact and
    tolerance cases."""
    codes, s, X = case(9850 + M + K, N, K, M, variant, exact=True)
    Y = gpu_gemm(codes, s, X, variant, N, K)
    Yref, _ = oracle.gemm(codes, s, X, N, K, variant, threads=THREADS)
    assert np.array_equal(Y.astype(np.float64), Yref)
    codes, s, X = case(9860 + M + K, N, K, M, variant, exact=False)
    Y = gpu_gemm(codes, s, X, variant, N, K)
    Yref, A = oracle.gemm(codes, s, X, N, K, variant, threads=THREADS)
    assert_tol(Y, Yref, A, "tiled gemm M=%d N=%d K=%d" % (M, N, K))


def _random_gemm_shapes():
    """Seeded shapes over every GEMM path: two-row VALU, staged, per-group and
    tiled MFMA kernels, with ragged M, N and K."""
    g = np.random.default_rng(4242)
    out = []
    for lo, hi, nlo, nhi, kmax in ((2, 3, 1, 3000, 160), (3, 9, 1, 3000, 100), (9, 128, 1, 2000, 60),
                                   (128, 400, 8200, 20000, 12)):
        for _ in range(3):
            out.append((int(g.integers(lo, hi)), int(g.integers(nlo, nhi)), 128 * int(g.integers(1, kmax))))
    return out


@pytest.mark.parametrize("variant", [TERN, BIN])
@pytest.mark.parametrize("M,N,K", _random_gemm_shapes())
def test_gemm_random_shapes(M, N, K, variant):
    codes, s, X = case(9990 + M + N + K, N, K, M, variant, exact=False)
    Y = gpu_gemm(codes, s, X, variant, N, K)
    Yref, A = oracle.gemm(codes, s, X, N, K, variant, threads=THREADS)
    assert_tol(Y, Yref, A, "random gemm M=%d N=%d K=%d" % (M, N, K))


@pytest.mark.parametrize("M", [2, 4, 16])
@pytest.mark.parametrize("N,K", [synth.GATE_UP, synth.DOWN])
def test_gemm_binary_full_size_sampled(M, N, K):
    codes, s, X = case(synth.seed_for(4, 50 + M + N % 7), N, K, M, BIN, exact=False)
    Y = gpu_gemm(codes, s, X, BIN, N, K)
    rows = _sampled_rows(N, 256, 100 + M)
    Yref, A = oracle.gemm(codes[rows], s[rows], X, len(rows), K, BIN, threads=THREADS)
    assert_tol(Y[:, rows], Yref, A, "binary gemm M=%d %dx%d" % (M, N, K))


@pytest.mark.parametrize("M", [2, 8])
def test_gemm_zero_rows_and_special_scales(M):
    """All-zero trit rows give |y| <= 1e-5 (the bound with A = 0); zero,
    subnormal and large scales pass through the FP32 group scaling."""
    N, K = 96, 1024
    t, s, X = synth.problem(9900, N, K, M, TERN, False)
    t[:32] = 0
    s[40, :] = 0
    s[41, :] = np.float16(6e-8)
    s[42, :] = np.float16(60000.0)
    codes = oracle.pack(t, TERN)
    Y = gpu_gemm(codes, s, X, TERN, N, K)
    Yref, A = oracle.gemm(codes, s, X, N, K, TERN, threads=THREADS)
    assert_tol(Y, Yref, A, "special")
    assert np.abs(Y[:, :32]).max() <= 1e-5
    assert np.all(Y[:, 40] == 0)


@pytest.mark.parametrize("variant", [TERN, BIN])
@pytest.mark.parametrize("M,N,K", [(3, 1, 128), (4, 5, 640), (4, 4097, 5120), (3, 33, 19456),
                                   (4, 7, 19584), (2, 1030, 1152), (4, 248, 17408), (4, 2000, 19456)])
def test_gemm_four_row_mfma_kernel(M, N, K, variant):
    """Batches of 3 and 4 rows (and two-row 1-bit batches) take the 4-row MFMA
    kernel: one weight row, a ragged chunk-group tail (K = 640), many blocks
    per workgroup, the largest K whose activations fit LDS (19456) and the
    first that does not (19584, another kernel).  Item partials are summed
    over 4, 2 (N = 33 at K = 19456) or 1 (N = 2000 at K = 19456) row groups
    before they go to LDS, by the LDS space left beside the activations."""
    codes, s, X = case(9870 + M + N + K, N, K, M, variant, exact=True)
    Y = gpu_gemm(codes, s, X, variant, N, K)
    Yref, _ = oracle.gemm(codes, s, X, N, K, variant, threads=THREADS)
    assert np.array_equal(Y.astype(np.float64), Yref)
    codes, s, X = case(9880 + M + N + K, N, K, M, variant, exact=False)
    Y = gpu_gemm(codes, s, X, variant, N, K)
    Yref, A = oracle.gemm(codes, s, X, N, K, variant, threads=THREADS)
    assert_tol(Y, Yref, A, "four-row gemm M=%d N=%d K=%d" % (M, N, K))


@pytest.mark.parametrize("variant", [TERN, BIN])
@pytest.mark.parametrize("M,N,K", [(5, 1, 128), (8, 5, 640), (6, 4097, 5120), (8, 33, 9216),
                                   (7, 7, 9728), (8, 32000, 5120), (8, 70000, 5120)])
def test_gemm_four_row_kernel_two_sets(M, N, K, variant):
    """Batches of 5 to 8 rows take the 4-row MFMA kernel with two row sets
    (one decode per weight for both) while both sets' activations fit LDS:
    one weight row, a ragged chunk-group tail, many blocks per workgroup, the
    largest K that fits (9216), the first that does not (9728: the K-split
    kernel), and two (N = 32000) or one (N = 70000) row-group partials per
    item."""
    codes, s, X = case(9890 + M + N + K, N, K, M, variant, exact=True)
    Y = gpu_gemm(codes, s, X, variant, N, K)
    Yref, _ = oracle.gemm(codes, s, X, N, K, variant, threads=THREADS)
    assert np.array_equal(Y.astype(np.float64), Yref)
    codes, s, X = case(9900 + M + N + K, N, K, M, variant, exact=False)
    Y = gpu_gemm(codes, s, X, variant, N, K)
    Yref, A = oracle.gemm(codes, s, X, N, K, variant, threads=THREADS)
    assert_tol(Y, Yref, A, "two-set four-row gemm M=%d N=%d K=%d" % (M, N, K))


def test_gemm_deterministic():
    """The K-split partial sums are added in a fixed order: repeated calls
    give identical bits."""
    N, K = 2048, 5120
    for M in (16, 4):
        codes, s, X = case(9950 + M, N, K, M, TERN, exact=False)
        cd, sd, Xd = up(codes), up(s), up(X)
        Y0 = tq.tq_gemm(cd, sd, Xd, variant=TERN)
        for _ in range(3):
            Y1 = tq.tq_gemm(cd, sd, Xd, variant=TERN)
            assert torch.equal(Y0, Y1), M


def test_graph_replay_matches_eager():
    """GEMV and GEMM launches captured in a HIP graph: every replay, with eager
    work and synchronisation between replays, gives the eager result's bits.
    The widths cover the four-row kernel with one and two row sets (2, 4, 8),
    the K-split kernel with the plain (16 rows, three slices) and the
    four-wide (64 rows, five slices) slice reduction."""
    N, K = 4096, 5120
    codes, s, X = case(9960, N, K, 64, TERN, exact=False)
    cd, sd, Xd = up(codes), up(s), up(X)
    y = torch.empty(N, dtype=torch.float32, device="cuda")
    widths = (2, 4, 8, 16, 64)
    Ys = [torch.empty(m, N, dtype=torch.float32, device="cuda") for m in widths]

    def calls():
        tq.tq_gemv(cd, sd, Xd[0], y)
        for m, Ym in zip(widths, Ys):
            tq.tq_gemm(cd, sd, Xd[:m], Ym)

    calls()
    torch.cuda.synchronize()
    y_ref, Y_refs = y.clone(), [t.clone() for t in Ys]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        calls()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        calls()
    for r in range(4):
        for t in [y] + Ys:
            t.fill_(float("nan"))
        tq.tq_gemv(cd, sd, Xd[1], torch.empty_like(y))   # unrelated eager work
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, y_ref), "GEMV replay %d" % r
        for m, Ym, Yr in zip(widths, Ys, Y_refs):
            assert torch.equal(Ym, Yr), "GEMM M=%d replay %d" % (m, r)


@pytest.mark.parametrize("M,N,K", [(5, 1, 256), (16, 33, 256), (8, 257, 2048), (13, 300, 2304),
                                   (16, 1000, 5120), (11, 129, 6144), (16, 65, 17408), (9, 4097, 5120),
                                   (16, 17, 19456), (6, 2049, 4608), (16, 40, 65536),
                                   (17, 33, 1024), (32, 1000, 5120), (29, 257, 2304), (33, 300, 5120),
                                   (64, 65, 17408), (48, 4097, 5120), (64, 17, 65536), (61, 129, 1280)])
def test_gemm_split_kernel(M, N, K):
    """5..64 rows of ternary weights on the K-split kernel (one, two or four
    16-row activation tiles): one slice (Y written directly), two to sixty-four
    slices added by the reduction kernel, ragged tiles, activation tiles and
    workgroup blocks, the largest K; bit-exact on the integer set, within
    tolerance elsewhere."""
    win = 8 if M <= 16 else 4
    slices = -(-(K // 256) // win)
    assert tq.tq_gemm_workspace_bytes(M, N, K) == (0 if slices == 1 else 4 * M * N * slices)
    codes, s, X = case(10100 + M + N + K, N, K, M, TERN, exact=True)
    Y = gpu_gemm(codes, s, X, TERN, N, K)
    Yref, _ = oracle.gemm(codes, s, X, N, K, TERN, threads=THREADS)
    assert np.array_equal(Y.astype(np.float64), Yref)
    codes, s, X = case(10200 + M + N + K, N, K, M, TERN, exact=False)
    Y = gpu_gemm(codes, s, X, TERN, N, K)
    Yref, A = oracle.gemm(codes, s, X, N, K, TERN, threads=THREADS)
    assert_tol(Y, Yref, A, "split gemm M=%d N=%d K=%d" % (M, N, K))


def test_gemm_ws_workspace_sizes():
    """tq_gemm_ws with the workspace it asks for, a larger one, and none (the
    call then takes the batched kernel): the same results within the bar, and
    bit-identical whenever the split kernel runs."""
    M, N, K = 16, 3000, 5120
    codes, s, X = case(10300, N, K, M, TERN, exact=False)
    cd, sd, Xd = up(codes), up(s), up(X)
    need = tq.tq_gemm_workspace_bytes(M, N, K)
    assert need == 3 * M * N * 4
    Yref, A = oracle.gemm(codes, s, X, N, K, TERN, threads=THREADS)
    ws_exact = torch.empty(need, dtype=torch.uint8, device="cuda")
    ws_big = torch.full((need + 4096,), 255, dtype=torch.uint8, device="cuda")
    Y1 = tq.tq_gemm(cd, sd, Xd, workspace=ws_exact)
    Y2 = tq.tq_gemm(cd, sd, Xd, workspace=ws_big)
    Y3 = tq.tq_gemm(cd, sd, Xd, workspace=ws_exact[: need - 4])  # too small: batched kernel
    Y4 = tq.tq_gemm(cd, sd, Xd)
    torch.cuda.synchronize()
    assert torch.equal(Y1, Y2) and torch.equal(Y1, Y4)
    for Y in (Y1, Y3):
        assert_tol(Y.cpu().numpy(), Yref, A, "tq_gemm_ws")


@pytest.mark.parametrize("M,N,K", [(32, 300, 5120), (64, 257, 17408), (16, 3000, 5120), (13, 129, 6144)])
def test_gemm_split_reduce_paths(M, N, K):
    """The slice reduction reads and writes four outputs per thread from five
    slices up when M * N is a multiple of 4 and Y is 16-byte aligned (5 slices
    at 32 x 5120, 17 = two batches of eight and one at 64 x 17408), else one
    (3 slices, or M * N odd): an output view one float into a buffer (4-byte
    aligned) takes the one-output path, with the same sums in the same order,
    so the bits are equal."""
    codes, s, X = case(10400 + M + N, N, K, M, TERN, exact=False)
    cd, sd, Xd = up(codes), up(s), up(X)
    need = tq.tq_gemm_workspace_bytes(M, N, K)
    assert need > 0
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    Ya = torch.empty(M, N, dtype=torch.float32, device="cuda")
    buf = torch.empty(M * N + 1, dtype=torch.float32, device="cuda")
    Yb = buf[1:].view(M, N)
    assert Yb.data_ptr() % 16 == 4
    tq.tq_gemm(cd, sd, Xd, Ya, workspace=ws)
    tq.tq_gemm(cd, sd, Xd, Yb, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(Ya, Yb)
    Yref, A = oracle.gemm(codes, s, X, N, K, TERN, threads=THREADS)
    assert_tol(Ya.cpu().numpy(), Yref, A, "split reduce paths")
