"""Runs the host code under AddressSanitizer and UndefinedBehaviorSanitizer.

Started by test_sanitizers.py in a child process whose LD_PRELOAD holds the
sanitizer runtimes: argv[1] is the packer (csrc/tq_host.cpp) built with
-fsanitize=address,undefined, argv[2] the oracle built the same way.  It runs
every variant's pack / unpack round trip and error paths through the packer's
C ABI, then every oracle pin against the sanitized oracle.  Any sanitizer
report aborts the process with a non-zero status."""
import ctypes
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(HERE))
sys.path.insert(0, HERE)

import oracle  # noqa: E402
import oracle_pins  # noqa: E402
from binary_g128_bit_amd import synth  # noqa: E402


def packer(path):
    L = ctypes.CDLL(path)
    i64, i32, vp = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p
    L.tq_codes_bytes.argtypes = [i64, i64, i32]
    L.tq_codes_bytes.restype = ctypes.c_size_t
    L.tq_pack.argtypes = [vp, i64, i64, i32, i32, vp]
    L.tq_pack.restype = i32
    L.tq_unpack.argtypes = [vp, i64, i64, i32, i32, vp]
    L.tq_unpack.restype = i32
    L.tq_last_error_index.restype = i64
    return L


def run_packer(L, olib):
    g = synth.rng(101)
    for variant in (0, 1, 2, 3):
        for N, K in ((1, 128), (3, 384), (7, 1152), (2, 5120)):
            if variant == 3:
                t = g.integers(0, 4, size=(N, K)).astype(np.int8)
            else:
                t = synth.trits(g, N, K, variant)
            nb = L.tq_codes_bytes(N, K, variant)
            codes = np.full(nb, 0xA5, np.uint8)  # every byte must be overwritten
            assert L.tq_pack(t.ctypes.data, N, K, 128, variant, codes.ctypes.data) == 0
            assert np.array_equal(codes, oracle.pack(t, variant, lib=olib).reshape(-1)), (variant, N, K)
            back = np.zeros((N, K), np.int8)
            assert L.tq_unpack(codes.ctypes.data, N, K, 128, variant, back.ctypes.data) == 0
            assert np.array_equal(back, t), (variant, N, K)
    # error paths: out-of-set values, code 3, bad five-trit bytes, bad shapes
    t = np.zeros((2, 256), np.int8)
    t[1, 77] = 2
    codes = np.zeros(L.tq_codes_bytes(2, 256, 0), np.uint8)
    assert L.tq_pack(t.ctypes.data, 2, 256, 128, 0, codes.ctypes.data) == 5
    assert L.tq_last_error_index() == 256 + 77
    codes = np.full(64, 0x55, np.uint8)
    codes[40] = 0xFF
    out = np.zeros((2, 128), np.int8)
    assert L.tq_unpack(codes.ctypes.data, 2, 128, 128, 0, out.ctypes.data) == 6
    c5 = np.zeros(L.tq_codes_bytes(1, 256, 2), np.uint8)
    c5[3] = 250
    out = np.zeros((1, 256), np.int8)
    assert L.tq_unpack(c5.ctypes.data, 1, 256, 128, 2, out.ctypes.data) == 6
    for N, K in ((0, 128), (2, 100), (2, 0)):
        assert L.tq_pack(t.ctypes.data, N, K, 128, 0, codes.ctypes.data) == 2
    assert L.tq_pack(None, 2, 128, 128, 0, codes.ctypes.data) == 1


def main():
    L = packer(sys.argv[1])
    olib = oracle.load(sys.argv[2])
    run_packer(L, olib)
    for check in oracle_pins.ALL_CHECKS:
        check(olib)
    print("sanitized host code: %d pins and the packer round trips clean" % len(oracle_pins.ALL_CHECKS))


if __name__ == "__main__":
    main()
