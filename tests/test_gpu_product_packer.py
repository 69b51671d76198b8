"""The product's packer feeding the product's kernels (needs an MI355X).

Every other GPU parity test packs with the oracle, so that a kernel is judged
against inputs the HIP side did not produce.  Here the codes come from the
library's own tq_pack instead: the packed bytes must equal the oracle's bit for
bit, and the kernel's output on them must match the oracle's product (computed
from the oracle's own packing and unpack) to the usual bars.
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


def check(Y, Yref, A, what):
    err = np.abs(Y.astype(np.float64) - Yref)
    bad = err > 2e-3 * A + 1e-5
    assert not bad.any(), "%s: %d bad, worst %.3g" % (what, bad.sum(), err.max())


@pytest.mark.parametrize("variant", [tq.TQ_TERNARY, tq.TQ_BINARY, tq.TQ_TERNARY5])
@pytest.mark.parametrize("N,K,M", [(1000, 5120, 1), (129, 17408, 1), (300, 1024, 1),
                                   (513, 5120, 4), (96, 1152, 16)])
def test_tq_pack_to_kernel(variant, N, K, M):
    if variant == tq.TQ_TERNARY5 and M > 1:
        pytest.skip("five-trit storage has a GEMV only")
    for exact in (False, True):
        t, s, X = synth.problem(synth.seed_for(3, N % 101 + M), N, K, M, variant, exact)
        codes = tq.tq_pack(t, variant)
        ref_codes = oracle.pack(t, variant)
        assert np.array_equal(codes, ref_codes), "tq_pack differs from the oracle"
        cd, sd, Xd = up(codes), up(s), up(X)
        if M == 1:
            Y = tq.tq_gemv(cd, sd, Xd[0], variant=variant).reshape(1, N)
        else:
            Y = tq.tq_gemm(cd, sd, Xd, variant=variant)
        torch.cuda.synchronize()
        Y = Y.cpu().numpy()
        Yref, A = oracle.gemm(ref_codes, s, X, N, K, variant, threads=THREADS)
        if exact:
            assert np.array_equal(Y.astype(np.float64), Yref), "integer-exact %dx%d M=%d" % (N, K, M)
        else:
            check(Y, Yref, A, "%dx%d M=%d" % (N, K, M))


@pytest.mark.parametrize("N,K", [(1000, 5120), (257, 17408), (64, 1024)])
def test_tq_pack_affine_to_kernel(N, K):
    for exact in (False, True):
        q, s, b, X = synth.affine_problem(synth.seed_for(3, 60 + N % 101), N, K, exact=exact)
        codes = tq.tq_pack(q, tq.TQ_AFFINE2)
        ref_codes = oracle.pack(q, oracle.AFFINE2)
        assert np.array_equal(codes, ref_codes), "tq_pack differs from the oracle"
        y = tq.tq_gemv_affine(up(codes), up(s), up(b), up(X[0]))
        torch.cuda.synchronize()
        y = y.cpu().numpy()
        Yref, A = oracle.affine_gemm(ref_codes, s, b, X[0], N, K, threads=THREADS)
        if exact:
            assert np.array_equal(y.astype(np.float64), Yref[0]), "affine integer-exact %dx%d" % (N, K)
        else:
            check(y, Yref[0], A[0], "affine %dx%d" % (N, K))
