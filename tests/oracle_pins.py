"""Pins that tie the oracle to something other than itself.

Each ``check_*`` takes a loaded oracle library (``oracle.load(path)``) and
raises AssertionError on a mismatch.  ``test_oracle_pins.py`` runs them on the
real oracle; ``test_oracle_mutants.py`` runs them on copies of the oracle with a
planted mistake and requires that some pin fails for every mistake.

What each pin rests on:
  * IEEE binary16 decoding: numpy's float16 -> float64 conversion (library).
  * Byte accounting: figures printed on the pages (tests/golden/page_figures.json).
  * Slot layout: hand-derived bytes (tests/golden/layout_examples.json).
  * The product itself: numpy float64 matmul of W = s * t built from the *input*
    trits (library routine), exact Python-integer arithmetic, and closed forms
    (one-hot, all-zero, all-one cases), plus a hand-evaluated worked example.
"""
import json
import math
import os

import numpy as np

import oracle
from binary_g128_bit_amd import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _dense(t, s):
    """W[n][k] = s[n][k/128] * t[n][k] from the input trits (not from unpack)."""
    s64 = np.asarray(s, dtype=np.float16).astype(np.float64)
    return np.repeat(s64, 128, axis=1) * t.astype(np.float64)


# ---------------------------------------------------------------- fp16 decode
def check_half_decode(lib):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([lib.oracle_half_to_double(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan), "NaN pattern differs"
    assert np.array_equal(got[~nan], ref[~nan]), "fp16 decode differs from numpy"


# ---------------------------------------------------------- byte accounting
def check_byte_counts(lib):
    pf = _golden("page_figures.json")
    # information content per weight (pages: log2(3) ~ 1.585, + 16/128 bit)
    bits_val = math.log2(3)
    assert round(bits_val, 3) == pf["ternary_bits_per_value"]["value"]
    ovh = pf["scale_overhead_bits"]["numerator"] / pf["scale_overhead_bits"]["denominator"]
    assert round(bits_val + ovh, 2) == pf["ternary_bpw"]["value"]
    assert 1 + ovh == pf["binary_bpw"]["value"]
    assert round(16 / (bits_val + ovh), 1) == pf["ternary_reduction_vs_fp16"]["value"]
    assert round(16 / (1 + ovh), 1) == pf["binary_reduction_vs_fp16"]["value"]

    # the oracle's own storage: 2-bit slots (or 1-bit) + one fp16 per 128
    shapes = [synth.C1, synth.GATE_UP, synth.DOWN, synth.LM_HEAD, (1024, 5120),
              (6144, 5120), (14336, 5120), (5120, 6144), (8, 128), (3, 384)]
    for N, K in shapes:
        sc = lib.oracle_scales_count(N, K, 128)
        assert sc == N * K // 128
        tb = lib.oracle_codes_bytes(N, K, 0)
        bb = lib.oracle_codes_bytes(N, K, 1)
        assert 8 * (tb + 2 * sc) == 2.125 * N * K, (N, K, tb)
        assert 8 * (bb + 2 * sc) == 1.125 * N * K, (N, K, bb)
    # five-trit bytes: ceil(128 / 5) = 26 bytes per group, rows padded to 16
    # bytes; with the scale that is (26 * 8 + 16) / 128 = 1.75 bpw whenever a
    # row's groups fill whole 16-byte units (G a multiple of 8)
    for N, K in shapes:
        G = K // 128
        rb = -(-26 * G // 16) * 16
        assert lib.oracle_codes_bytes(N, K, 2) == N * rb, (N, K)
        if G % 8 == 0:
            assert 8 * (N * rb + 2 * N * G) == 1.75 * N * K, (N, K)
    assert math.ceil(128 / 5) == 26 and 3 ** 5 <= 256 < 3 ** 6
    # the pages' deploy size follows from 2.125 bpw on the FP16 model's weights:
    # 54 GB at 16 bpw -> 27.0e9 weights -> 7.17 GB with 2-bit slots
    n_weights = pf["fp16_model_gb"]["value"] * 1e9 * 8 / 16
    N, K = 1024, 1024
    st_bpw = 8 * (lib.oracle_codes_bytes(N, K, 0) + 2 * lib.oracle_scales_count(N, K, 128)) / (N * K)
    deploy = n_weights * st_bpw / 8 / 1e9
    assert round(deploy, 2) == pf["ternary_deploy_gb_2bit_slots"]["value"], deploy
    # ideal sizes at the information bpw land within 3% of the printed ones
    assert abs(n_weights * (bits_val + ovh) / 8e9 / pf["ternary_ideal_gb"]["value"] - 1) < 0.03
    bin_bpw = 8 * (lib.oracle_codes_bytes(N, K, 1) + 2 * lib.oracle_scales_count(N, K, 128)) / (N * K)
    assert abs(n_weights * bin_bpw / 8e9 / pf["binary_ideal_gb"]["value"] - 1) < 0.03


# ------------------------------------------------------------- round trips
def check_roundtrip_bytes(lib):
    valid = 0
    for b in range(256):
        row = np.full((1, 32), b, dtype=np.uint8)        # K = 128, ternary
        try:
            t = oracle.unpack(row, 1, 128, oracle.TERNARY, lib=lib)
        except oracle.OracleError as e:
            assert e.code == 6
            # first bad slot of the first byte
            first = min(j for j in range(4) if (b >> (2 * j)) & 3 == 3)
            assert e.index == first, (b, e.index)
            continue
        valid += 1
        assert set(np.unique(t)) <= {-1, 0, 1}
        back = oracle.pack(t, oracle.TERNARY, lib=lib)
        assert np.array_equal(back, row), b
    assert valid == 81, valid                            # 3^4 valid bytes
    for b in range(256):
        row = np.full((1, 16), b, dtype=np.uint8)        # K = 128, binary
        t = oracle.unpack(row, 1, 128, oracle.BINARY, lib=lib)
        assert set(np.unique(t)) <= {-1, 1}
        assert np.array_equal(oracle.pack(t, oracle.BINARY, lib=lib), row), b
    # five-trit bytes: every byte below 3^5 round-trips at positions 0..24 of
    # a group; at position 25 only values below 3^3; all others are rejected
    # with the index of the byte's first trit
    for pos, limit in ((0, 243), (7, 243), (24, 243), (25, 27)):
        valid = 0
        for b in range(256):
            row = np.zeros((1, 16 * 4), dtype=np.uint8)  # K = 256: 2 groups, 64 bytes
            row[0, 26 + pos] = b
            try:
                t = oracle.unpack(row, 1, 256, oracle.TERNARY5, lib=lib)
            except oracle.OracleError as e:
                assert e.code == 6 and e.index == 128 + 5 * pos, (pos, b, e.index)
                assert b >= limit, (pos, b)
                continue
            valid += 1
            assert np.array_equal(oracle.pack(t, oracle.TERNARY5, lib=lib), row), (pos, b)
        assert valid == limit, (pos, valid)
    g = synth.rng(7)
    for variant in (oracle.TERNARY, oracle.BINARY, oracle.TERNARY5):
        for N, K in ((1, 128), (5, 384), (16, 1024)):
            t = synth.trits(g, N, K, variant)
            c = oracle.pack(t, variant, lib=lib)
            assert np.array_equal(oracle.unpack(c, N, K, variant, lib=lib), t)


def check_golden_layout(lib):
    lay = _golden("layout_examples.json")
    for key, variant in (("ternary_row", oracle.TERNARY), ("binary_row", oracle.BINARY)):
        ex = lay[key]
        K = ex["K"]
        t = np.full((1, K), ex["t_rest"], dtype=np.int8)
        t[0, :len(ex["t_prefix"])] = ex["t_prefix"]
        codes = oracle.pack(t, variant, lib=lib)[0]
        pre = [int(h, 16) for h in ex["bytes_prefix_hex"]]
        assert list(codes[:len(pre)]) == pre, (key, codes[:len(pre)])
        assert all(int(b) == int(ex["byte_rest_hex"], 16) for b in codes[len(pre):]), key
        assert np.array_equal(oracle.unpack(codes.reshape(1, -1), 1, K, variant, lib=lib), t)


def check_golden_ternary5(lib):
    ex = _golden("layout_examples.json")["ternary5_row"]
    K = ex["K"]
    t = np.ones((1, K), dtype=np.int8)
    for k in range(128):
        b, i = divmod(k, 5)
        t[0, k] = (b + i) % 3 - 1
    codes = oracle.pack(t, oracle.TERNARY5, lib=lib)[0]
    assert [int(h, 16) for h in ex["bytes_hex"]] == list(codes), list(codes)
    assert np.array_equal(oracle.unpack(codes.reshape(1, -1), 1, K, oracle.TERNARY5, lib=lib), t)
    for bad in ex["invalid"]:
        c = codes.copy()
        c[bad["byte_index"]] = bad["value"]
        try:
            oracle.unpack(c.reshape(1, -1), 1, K, oracle.TERNARY5, lib=lib)
            raise AssertionError("accepted %r" % bad)
        except oracle.OracleError as e:
            assert e.code == 6 and e.index == bad["error_index"], (bad, e.index)


def check_worked_gemv(lib):
    ex = _golden("layout_examples.json")["worked_gemv"]
    N, K = ex["N"], ex["K"]
    t = np.zeros((N, K), dtype=np.int8)
    t[0, :128] = 1
    t[1, 0:128:2] = -1
    t[1, 1:128:2] = 1
    t[1, 133] = 1
    s = np.array([r["scales"] for r in ex["rows"]], dtype=np.float16)
    x = np.where(np.arange(K) < 128, 1.0, 2.0).astype(np.float16)
    y, _ = oracle.gemv(oracle.pack(t, lib=lib), s, x, N, K, lib=lib)
    assert list(y) == ex["y"], y


# ------------------------------------------------------------ the product
def _thread_counts():
    """Row-split widths the oracle is pinned at: one thread, an odd count that
    leaves a remainder on the test shapes, and every core this process may
    use (what the GPU parity tests run the oracle with)."""
    return sorted({1, 3, max(2, oracle.default_threads())})


def check_bruteforce_numpy(lib):
    g = synth.rng(11)
    for variant in (oracle.TERNARY, oracle.BINARY, oracle.TERNARY5):
        for N, K, M in ((1, 128, 1), (3, 256, 2), (8, 384, 4), (5, 128, 3), (37, 256, 2)):
            t = synth.trits(g, N, K, variant)
            s = synth.scales(g, N, K)
            s[0, 0] = -s[0, 0]                       # negative scale
            if s.shape[1] > 1:
                s[-1, -1] = np.float16(2.0 ** -20)   # subnormal scale
            X = synth.activations(g, M, K)
            X[0, 0] = np.float16(2.0 ** -22)         # subnormal activation
            ref = X.astype(np.float64) @ _dense(t, s).T
            scale = np.abs(X.astype(np.float64)) @ np.abs(_dense(t, s)).T
            for threads in _thread_counts():
                Y, A = oracle.gemm(oracle.pack(t, variant, lib=lib), s, X, N, K, variant,
                                   threads=threads, lib=lib)
                err = np.abs(Y - ref)
                assert np.all(err <= 1e-12 * scale + 1e-300), (variant, N, K, M, threads, err.max())
                assert np.allclose(A, scale, rtol=1e-12, atol=0), (variant, N, K, M, threads)


def check_exact_integer(lib):
    g = synth.rng(13)
    for variant in (oracle.TERNARY, oracle.BINARY, oracle.TERNARY5):
        for N, K, M in ((4, 384, 3), (29, 256, 2)):
            t = synth.trits(g, N, K, variant)
            s = np.ones((N, K // 128), dtype=np.float16)
            X = synth.int_activations(g, M, K)
            xi = X.astype(np.int64)
            exact = [[sum(int(t[n, k]) * int(xi[m, k]) for k in range(K)) for n in range(N)]
                     for m in range(M)]
            for threads in _thread_counts():
                Y, _ = oracle.gemm(oracle.pack(t, variant, lib=lib), s, X, N, K, variant,
                                   threads=threads, lib=lib)
                for m in range(M):
                    for n in range(N):
                        assert Y[m, n] == exact[m][n], (variant, threads, m, n, Y[m, n], exact[m][n])


def check_special_cases(lib):
    g = synth.rng(17)
    N, K = 6, 384
    t = synth.trits(g, N, K, oracle.TERNARY)
    s = synth.scales(g, N, K)
    codes = oracle.pack(t, lib=lib)
    sv = s.astype(np.float64)
    # one-hot x = e_k: y[n] = s[n][k/128] * t[n][k] exactly
    for k in (0, 1, 2, 3, 4, 127, 128, 131, 255, 256, 383):
        x = np.zeros(K, dtype=np.float16)
        x[k] = 1
        y, _ = oracle.gemv(codes, s, x, N, K, lib=lib)
        assert np.array_equal(y, sv[:, k // 128] * t[:, k]), k
    # t == 0 -> y == 0
    z = oracle.pack(np.zeros((N, K), np.int8), lib=lib)
    x = synth.activations(g, 1, K)[0]
    y, _ = oracle.gemv(z, s, x, N, K, lib=lib)
    assert np.all(y == 0)
    # t == +1 and s == 1 -> y == sum(x)
    one = oracle.pack(np.ones((N, K), np.int8), lib=lib)
    y, _ = oracle.gemv(one, np.ones_like(s), x, N, K, lib=lib)
    assert np.all(y == np.sum(x.astype(np.float64)))
    # x == 1 -> y[n] = sum_g s_g * (#(+1) - #(-1)) in group g
    y, _ = oracle.gemv(codes, s, np.ones(K, np.float16), N, K, lib=lib)
    cnt = t.reshape(N, K // 128, 128).astype(np.int64).sum(axis=2)
    assert np.allclose(y, (sv * cnt).sum(axis=1), rtol=1e-15, atol=0)
    # binary one-hot: y[n] = s * (+-1)
    tb = synth.trits(g, N, K, oracle.BINARY)
    cb = oracle.pack(tb, oracle.BINARY, lib=lib)
    for k in (0, 7, 8, 129, 383):
        x = np.zeros(K, dtype=np.float16)
        x[k] = 1
        y, _ = oracle.gemv(cb, s, x, N, K, oracle.BINARY, lib=lib)
        assert np.array_equal(y, sv[:, k // 128] * tb[:, k]), k


def check_bound(lib):
    g = synth.rng(19)
    for variant in (oracle.TERNARY, oracle.BINARY):
        N, K, M = 5, 384, 2
        t = synth.trits(g, N, K, variant)
        s = synth.scales(g, N, K)
        s[1, 1] = -s[1, 1]
        X = synth.activations(g, M, K)
        Y, A = oracle.gemm(oracle.pack(t, variant, lib=lib), s, X, N, K, variant, lib=lib)
        refA = np.abs(X.astype(np.float64)) @ np.abs(_dense(t, s)).T
        assert np.allclose(A, refA, rtol=1e-12, atol=0), variant
        assert np.all(np.abs(Y) <= A * (1 + 1e-12))


def check_errors(lib):
    t = np.zeros((2, 128), np.int8)
    for bad_t, variant, idx in ((2, oracle.TERNARY, 5), (0, oracle.BINARY, 3), (-2, oracle.TERNARY, 200)):
        tt = np.zeros((2, 128), np.int8) if variant == oracle.TERNARY else np.ones((2, 128), np.int8)
        tt.flat[idx] = bad_t
        try:
            oracle.pack(tt, variant, lib=lib)
            raise AssertionError("pack accepted %d" % bad_t)
        except oracle.OracleError as e:
            assert e.code == 5 and e.index == idx, (e.code, e.index)
    for N, K, group, variant, code in ((2, 100, 128, 0, 2), (2, 192, 128, 0, 2), (0, 128, 128, 0, 2),
                                       (2, 128, 64, 0, 3), (2, 128, 128, 4, 4)):
        rc = lib.oracle_pack(t.ctypes.data, N, K, group, variant,
                             np.zeros(64, np.uint8).ctypes.data, None)
        assert rc == code, (N, K, group, variant, rc)
    codes = np.full((2, 32), 0x55, np.uint8)
    codes[1, 7] = 0x55 | (3 << 4)                       # slot 2 of byte 7 of row 1
    try:
        oracle.unpack(codes, 2, 128, lib=lib)
        raise AssertionError("code 3 accepted")
    except oracle.OracleError as e:
        assert e.code == 6 and e.index == 128 + 7 * 4 + 2, e.index


# ---------------------------------------------------------- embedding rows
def check_embed(lib):
    """Row id of W = s * t, built from the input trits with numpy."""
    g = synth.rng(23)
    for variant in (oracle.TERNARY, oracle.BINARY, oracle.TERNARY5):
        N, K = 9, 512
        t = synth.trits(g, N, K, variant)
        s = synth.scales(g, N, K)
        s[2, 1] = -s[2, 1]
        s[4, 3] = np.float16(2.0 ** -20)
        codes = oracle.pack(t, variant, lib=lib)
        ids = np.array([0, 8, 2, 2, 4, 5, 1], np.int32)
        got = oracle.embed(codes, s, ids, N, K, variant, lib=lib)
        assert np.array_equal(got, _dense(t, s)[ids]), variant
        empty = oracle.embed(codes, s, np.zeros(0, np.int32), N, K, variant, lib=lib)
        assert empty.shape == (0, K)
        for bad in (-1, N):
            try:
                oracle.embed(codes, s, np.array([0, bad], np.int32), N, K, variant, lib=lib)
                raise AssertionError("id %d accepted" % bad)
            except oracle.OracleError as e:
                assert e.code == 2, e.code


# ------------------------------------------------------------- affine 2-bit
def _affine_dense(q, s, b):
    """W[n][k] = s[n][k/128] * q[n][k] + b[n][k/128] from the inputs."""
    s64 = np.repeat(np.asarray(s, np.float16).astype(np.float64), 128, axis=1)
    b64 = np.repeat(np.asarray(b, np.float16).astype(np.float64), 128, axis=1)
    return s64 * q.astype(np.float64) + b64


def check_affine(lib):
    ex = _golden("layout_examples.json")["affine2_row"]
    q = np.full((1, ex["K"]), ex["q_rest"], np.int8)
    q[0, :len(ex["q_prefix"])] = ex["q_prefix"]
    codes = oracle.pack(q, oracle.AFFINE2, lib=lib)[0]
    pre = [int(h, 16) for h in ex["bytes_prefix_hex"]]
    assert list(codes[:len(pre)]) == pre, list(codes[:4])
    assert all(int(v) == int(ex["byte_rest_hex"], 16) for v in codes[len(pre):])
    # every byte is valid and round-trips
    allb = np.arange(256, dtype=np.uint8).reshape(8, 32)
    qa = oracle.unpack(allb, 8, 128, oracle.AFFINE2, lib=lib)
    assert qa.min() == 0 and qa.max() == 3
    assert np.array_equal(oracle.pack(qa, oracle.AFFINE2, lib=lib), allb)
    # worked example
    w = ex["worked"]
    s = np.full((1, 1), w["scale"], np.float16)
    b = np.full((1, 1), w["bias"], np.float16)
    qq = np.zeros((1, 128), np.int8)
    qq[0, :4] = [0, 1, 2, 3]
    x = np.zeros(128, np.float16)
    x[:4] = 1
    Y, _ = oracle.affine_gemm(oracle.pack(qq, oracle.AFFINE2, lib=lib), s, b, x, 1, 128, lib=lib)
    assert Y[0, 0] == w["y"], Y
    g = synth.rng(29)
    N, K, M = 6, 384, 3
    qr = g.integers(0, 4, size=(N, K)).astype(np.int8)
    s = synth.scales(g, N, K)
    b = (-synth.scales(g, N, K).astype(np.float32) * 1.5).astype(np.float16)
    s[0, 1] = -s[0, 1]
    b[2, 0] = np.float16(2.0 ** -21)
    X = synth.activations(g, M, K)
    c = oracle.pack(qr, oracle.AFFINE2, lib=lib)
    W = _affine_dense(qr, s, b)
    ref = X.astype(np.float64) @ W.T
    refA = (np.abs(X.astype(np.float64)) @ (np.abs(np.repeat(s.astype(np.float64), 128, 1)) * qr).T
            + np.abs(X.astype(np.float64)) @ np.abs(np.repeat(b.astype(np.float64), 128, 1)).T)
    for threads in _thread_counts():
        Y, A = oracle.affine_gemm(c, s, b, X, N, K, threads=threads, lib=lib)
        assert np.all(np.abs(Y - ref) <= 1e-12 * A), (threads, np.abs(Y - ref).max())
        assert np.allclose(A, refA, rtol=1e-12, atol=0), threads
    # a row count that leaves a remainder on every split
    N2 = 41
    q2 = g.integers(0, 4, size=(N2, K)).astype(np.int8)
    s2, b2 = synth.scales(g, N2, K), -synth.scales(g, N2, K)
    c2 = oracle.pack(q2, oracle.AFFINE2, lib=lib)
    ref2 = X.astype(np.float64) @ _affine_dense(q2, s2, b2).T
    for threads in _thread_counts():
        Y2, A2 = oracle.affine_gemm(c2, s2, b2, X, N2, K, threads=threads, lib=lib)
        assert np.all(np.abs(Y2 - ref2) <= 1e-12 * A2), (threads, np.abs(Y2 - ref2).max())
    # one-hot x: y = s * q_k + b exactly
    for k in (0, 5, 127, 128, 300, 383):
        x = np.zeros(K, np.float16)
        x[k] = 1
        y, _ = oracle.affine_gemm(c, s, b, x, N, K, lib=lib)
        exact = s[:, k // 128].astype(np.float64) * qr[:, k] + b[:, k // 128].astype(np.float64)
        assert np.array_equal(y[0], exact), k
    # q = 0: y = sum_g b_g * sum x_g
    z = oracle.pack(np.zeros((N, K), np.int8), oracle.AFFINE2, lib=lib)
    y, _ = oracle.affine_gemm(z, s, b, X[0], N, K, lib=lib)
    xg = X[0].astype(np.float64).reshape(-1, 128).sum(axis=1)
    assert np.allclose(y[0], b.astype(np.float64) @ xg, rtol=1e-13, atol=0)
    # ternary weights are the case q = t + 1, b = -s: the ternary product
    t = synth.trits(g, N, K)
    Yt, At = oracle.gemm(oracle.pack(t, lib=lib), s, X, N, K, lib=lib)
    Ya, _ = oracle.affine_gemm(oracle.pack((t + 1).astype(np.int8), oracle.AFFINE2, lib=lib), s,
                               -s, X, N, K, lib=lib)
    assert np.all(np.abs(Ya - Yt) <= 1e-12 * At + 1e-300)
    # the bias-free entry points refuse the affine variant
    for call in (lambda: oracle.gemm(c, s, X, N, K, oracle.AFFINE2, lib=lib),
                 lambda: oracle.embed(c, s, np.zeros(1, np.int32), N, K, oracle.AFFINE2, lib=lib)):
        try:
            call()
            raise AssertionError("affine accepted without biases")
        except oracle.OracleError as e:
            assert e.code == 4


# ------------------------------------------------------- 4-bit KV cache
def check_float_to_half(lib):
    g = np.random.default_rng(31)
    vals = g.standard_normal(4000).astype(np.float32) * np.float32(10.0) ** g.integers(-9, 4, 4000)
    vals = np.concatenate([vals, np.float32([0.0, -0.0, 2.0 ** -24, 2.0 ** -25, 3 * 2.0 ** -26,
                                             1 / 7, 65504.0, 6.1035156e-05, 6.0975552e-05])])
    vals = vals[np.abs(vals) < 65504]
    for v in vals:
        assert oracle.float_to_half(v, lib=lib) == int(np.float32(v).astype(np.float16).view(np.uint16)), v


def check_kv_quant(lib):
    ex = _golden("kv4_examples.json")
    x = np.zeros((1, 256), np.float16)
    for gi, grp in enumerate(ex["groups"]):
        x[0, 32 * gi: 32 * gi + len(grp["x"])] = grp["x"]
    nib, sc = oracle.kv_quant(x, lib=lib)
    for gi, grp in enumerate(ex["groups"]):
        assert int(sc[0, gi].view(np.uint16)) == int(grp["d_hex"], 16), (gi, sc[0, gi])
        n = len(grp["nibbles"])
        assert list(nib[0, 32 * gi: 32 * gi + n]) == grp["nibbles"], gi
        assert all(v == 8 for v in nib[0, 32 * gi + n: 32 * gi + 32]), gi
    # properties on random vectors: the largest element lands on +-7, every
    # element is within d / 2 of its dequantized value
    g = synth.rng(37)
    xr = (g.standard_normal((64, 256)) * np.exp(g.normal(0, 1.5, (64, 1)))).astype(np.float16)
    nib, sc = oracle.kv_quant(xr, lib=lib)
    xv = xr.astype(np.float64).reshape(64, 8, 32)
    q = nib.astype(np.int64).reshape(64, 8, 32) - 8
    d = sc.astype(np.float64)[:, :, None]
    assert q.min() >= -8 and q.max() <= 7
    assert np.all(np.abs(q * d - xv) <= d / 2 * (1 + 1e-12))
    am = np.abs(xv).argmax(axis=2)
    assert np.all(np.abs(np.take_along_axis(q, am[:, :, None], 2)) == 7)


def _dequant(nib, sc):
    return (nib.astype(np.float64) - 8.0) * np.repeat(sc.astype(np.float64), 32, axis=-1)


def check_attn_decode(lib):
    import scipy.special
    g = synth.rng(41)
    n_kv, n_q, T = 2, 8, 37
    q = synth.activations(g, n_q, 256)
    k = synth.activations(g, n_kv * T, 256)
    v = synth.activations(g, n_kv * T, 256)
    kn, ks = oracle.kv_quant(k, lib=lib)
    vn, vs = oracle.kv_quant(v, lib=lib)
    kn, ks = kn.reshape(n_kv, T, 256), ks.reshape(n_kv, T, 8)
    vn, vs = vn.reshape(n_kv, T, 256), vs.reshape(n_kv, T, 8)
    out, A = oracle.attn_decode(q, kn, ks, vn, vs, lib=lib)
    K, V = _dequant(kn, ks), _dequant(vn, vs)
    for h in range(n_q):
        kvh = h // (n_q // n_kv)
        p = scipy.special.softmax(K[kvh] @ q[h].astype(np.float64) / 16.0)
        ref = p @ V[kvh]
        assert np.allclose(out[h], ref, rtol=1e-12, atol=1e-14), h
        assert np.allclose(A[h], p @ np.abs(V[kvh]), rtol=1e-12, atol=1e-300)
    # one token: the output is that token's value; equal keys: the mean value
    o1, _ = oracle.attn_decode(q[:2], kn[:1, :1], ks[:1, :1], vn[:1, :1], vs[:1, :1], lib=lib)
    assert np.array_equal(o1, np.repeat(V[0, :1], 2, axis=0))
    ke = np.repeat(kn[:, :1], T, axis=1)
    kse = np.repeat(ks[:, :1], T, axis=1)
    oe, _ = oracle.attn_decode(q, ke, kse, vn, vs, lib=lib)
    for h in range(n_q):
        assert np.allclose(oe[h], V[h // (n_q // n_kv)].mean(axis=0), rtol=1e-12, atol=1e-15)


ALL_CHECKS = [check_half_decode, check_byte_counts, check_roundtrip_bytes,
              check_golden_layout, check_worked_gemv, check_bruteforce_numpy,
              check_exact_integer, check_special_cases, check_bound, check_errors,
              check_embed, check_golden_ternary5, check_affine, check_float_to_half,
              check_kv_quant, check_attn_decode]
