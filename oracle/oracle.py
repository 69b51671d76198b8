"""ctypes marshalling for the C oracle (``tq_oracle.c``).

TEST INFRASTRUCTURE ONLY (see the package docstring).  Every numeric step is in
the C file; this module converts numpy arrays to pointers and error codes to
exceptions.
"""
import ctypes
import os
import subprocess

import numpy as np

TERNARY = 0
BINARY = 1
TERNARY5 = 2  # five trits per byte, 26 bytes per group, rows padded to 16 bytes
AFFINE2 = 3   # unsigned 2-bit level q per weight, FP16 scale and bias per group

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "tq_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

_ERRORS = {1: "null pointer", 2: "bad shape", 3: "group must be 128",
           4: "unknown variant", 5: "value outside the variant's set",
           6: "invalid code (ternary code 3, or a five-trit byte out of range)",
           7: "out of memory"}


class OracleError(RuntimeError):
    def __init__(self, code, index=None):
        self.code = code
        self.index = index
        msg = _ERRORS.get(code, "error %d" % code)
        if index is not None:
            msg += " at flat index %d" % index
        super().__init__(msg)


def build(lib_path=_LIB, extra_flags=(), src=_SRC):
    """Compile the oracle with gcc (-O2 -fopenmp, no fast-math)."""
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
           *extra_flags, src, "-o", lib_path + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(lib_path + ".tmp", lib_path)
    return lib_path


_lib_cache = {}


def load(lib_path=_LIB):
    """Load (building first if absent) the oracle shared library."""
    if lib_path in _lib_cache:
        return _lib_cache[lib_path]
    if not os.path.exists(lib_path) or (
            lib_path == _LIB and os.path.getmtime(lib_path) < os.path.getmtime(_SRC)):
        build(lib_path)
    lib = ctypes.CDLL(lib_path)
    i64, i32, ci = ctypes.c_int64, ctypes.c_int32, ctypes.c_int
    vp = ctypes.c_void_p
    lib.oracle_half_to_double.argtypes = [ctypes.c_uint16]
    lib.oracle_half_to_double.restype = ctypes.c_double
    lib.oracle_codes_bytes.argtypes = [i64, i64, ci]
    lib.oracle_codes_bytes.restype = i64
    lib.oracle_scales_count.argtypes = [i64, i64, i32]
    lib.oracle_scales_count.restype = i64
    lib.oracle_pack.argtypes = [vp, i64, i64, i32, ci, vp, ctypes.POINTER(i64)]
    lib.oracle_pack.restype = ci
    lib.oracle_unpack.argtypes = [vp, i64, i64, i32, ci, vp, ctypes.POINTER(i64)]
    lib.oracle_unpack.restype = ci
    lib.oracle_gemm.argtypes = [vp, vp, vp, i64, i64, i64, i32, ci, vp, vp, ci]
    lib.oracle_gemm.restype = ci
    lib.oracle_embed.argtypes = [vp, vp, vp, i64, i64, i64, i32, ci, vp]
    lib.oracle_embed.restype = ci
    lib.oracle_affine_gemm.argtypes = [vp, vp, vp, vp, i64, i64, i64, i32, vp, vp, ci]
    lib.oracle_affine_gemm.restype = ci
    lib.oracle_float_to_half.argtypes = [ctypes.c_float]
    lib.oracle_float_to_half.restype = ctypes.c_uint16
    lib.oracle_kv_quant.argtypes = [vp, i64, vp, vp]
    lib.oracle_kv_quant.restype = ci
    lib.oracle_attn_decode.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, vp, vp]
    lib.oracle_attn_decode.restype = ci
    _lib_cache[lib_path] = lib
    return lib


def default_threads():
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def _ptr(a):
    return ctypes.c_void_p(a.ctypes.data) if a is not None else None


def half_to_double(bits, lib=None):
    lib = lib or load()
    return lib.oracle_half_to_double(int(bits) & 0xFFFF)


def codes_bytes(N, K, variant, lib=None):
    return (lib or load()).oracle_codes_bytes(N, K, variant)


def scales_count(N, K, group=128, lib=None):
    return (lib or load()).oracle_scales_count(N, K, group)


def pack(t, variant=TERNARY, group=128, lib=None):
    """t: int8 [N][K] -> uint8 codes [N][K/4] (ternary), [N][K/8] (binary) or
    [N][row bytes] (five-trit bytes)."""
    lib = lib or load()
    t = np.ascontiguousarray(t, dtype=np.int8)
    N, K = t.shape
    nb = lib.oracle_codes_bytes(N, K, variant)
    out = np.empty(max(nb, 0), dtype=np.uint8)
    bad = ctypes.c_int64(-1)
    rc = lib.oracle_pack(_ptr(t), N, K, group, variant, _ptr(out), ctypes.byref(bad))
    if rc:
        raise OracleError(rc, bad.value if rc == 5 else None)
    return out.reshape(N, -1)


def unpack(codes, N, K, variant=TERNARY, group=128, lib=None):
    """codes -> int8 t [N][K]; raises OracleError(code=6, index) on an invalid
    code (index of the first trit it holds)."""
    lib = lib or load()
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    t = np.empty((N, K), dtype=np.int8)
    bad = ctypes.c_int64(-1)
    rc = lib.oracle_unpack(_ptr(codes), N, K, group, variant, _ptr(t), ctypes.byref(bad))
    if rc:
        raise OracleError(rc, bad.value if rc == 6 else None)
    return t


def gemm(codes, scales, X, N, K, variant=TERNARY, group=128, threads=1, lib=None):
    """Y[M][N], A[M][N] in float64.  scales / X are float16 arrays (or their
    uint16 bit patterns); X has shape [M][K]."""
    lib = lib or load()
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    s = np.ascontiguousarray(scales)
    s = s.view(np.uint16) if s.dtype == np.float16 else s.astype(np.uint16)
    X = np.ascontiguousarray(X)
    X = X.view(np.uint16) if X.dtype == np.float16 else X.astype(np.uint16)
    if X.ndim == 1:
        X = X.reshape(1, -1)
    M = X.shape[0]
    if X.shape[1] != K:
        raise ValueError("X has %d columns, expected K=%d" % (X.shape[1], K))
    # NaN-filled, so an output the C code never writes cannot pass for a result
    Y = np.full((M, N), np.nan, dtype=np.float64)
    A = np.full((M, N), np.nan, dtype=np.float64)
    rc = lib.oracle_gemm(_ptr(codes), _ptr(s), _ptr(X), M, N, K, group, variant,
                         _ptr(Y), _ptr(A), int(threads))
    if rc:
        raise OracleError(rc)
    return Y, A


def gemv(codes, scales, x, N, K, variant=TERNARY, group=128, threads=1, lib=None):
    """y[N], A[N] for a single activation vector x[K]."""
    Y, A = gemm(codes, scales, np.asarray(x).reshape(1, -1), N, K, variant, group,
                threads, lib)
    return Y[0], A[0]


def embed(codes, scales, ids, N, K, variant=TERNARY, group=128, lib=None):
    """out[n_ids][K] float64: row ids[i] of W = s * t (ids in [0, N))."""
    lib = lib or load()
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    s = np.ascontiguousarray(scales)
    s = s.view(np.uint16) if s.dtype == np.float16 else s.astype(np.uint16)
    ids = np.ascontiguousarray(ids, dtype=np.int32).reshape(-1)
    out = np.empty((ids.size, K), dtype=np.float64)
    rc = lib.oracle_embed(_ptr(codes), _ptr(s), _ptr(ids), ids.size, N, K, group, variant, _ptr(out))
    if rc:
        raise OracleError(rc)
    return out


def _bits(a):
    a = np.ascontiguousarray(a)
    return a.view(np.uint16) if a.dtype == np.float16 else a.astype(np.uint16)


def affine_gemm(codes, scales, biases, X, N, K, group=128, threads=1, lib=None):
    """Y[M][N], A[M][N] float64 for the affine 2-bit weights w = s * q + b."""
    lib = lib or load()
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    s, b = _bits(scales), _bits(biases)
    X = _bits(X)
    if X.ndim == 1:
        X = X.reshape(1, -1)
    M = X.shape[0]
    Y = np.full((M, N), np.nan, dtype=np.float64)
    A = np.full((M, N), np.nan, dtype=np.float64)
    rc = lib.oracle_affine_gemm(_ptr(codes), _ptr(s), _ptr(b), _ptr(X), M, N, K, group,
                                _ptr(Y), _ptr(A), int(threads))
    if rc:
        raise OracleError(rc)
    return Y, A


def float_to_half(f, lib=None):
    """binary32 value -> binary16 bits, round to nearest even."""
    return (lib or load()).oracle_float_to_half(float(f))


def kv_quant(x, lib=None):
    """x float16 [n][256] -> (nibbles uint8 [n][256], scales float16 [n][8])."""
    lib = lib or load()
    xb = _bits(x).reshape(-1, 256)
    n = xb.shape[0]
    nib = np.empty((n, 256), dtype=np.uint8)
    sc = np.empty((n, 8), dtype=np.uint16)
    rc = lib.oracle_kv_quant(_ptr(xb), n, _ptr(nib), _ptr(sc))
    if rc:
        raise OracleError(rc)
    return nib, sc.view(np.float16)


def attn_decode(q, knib, ks, vnib, vs, lib=None):
    """Decode attention from the logical 4-bit cache: q float16 [n_q][256];
    knib / vnib uint8 [n_kv][T][256]; ks / vs float16 [n_kv][T][8].
    Returns (out [n_q][256], A [n_q][256]) float64."""
    lib = lib or load()
    qb = _bits(q).reshape(-1, 256)
    n_q = qb.shape[0]
    knib = np.ascontiguousarray(knib, dtype=np.uint8)
    vnib = np.ascontiguousarray(vnib, dtype=np.uint8)
    n_kv, T = knib.shape[0], knib.shape[1]
    ksb, vsb = _bits(ks), _bits(vs)
    out = np.empty((n_q, 256), dtype=np.float64)
    A = np.empty((n_q, 256), dtype=np.float64)
    rc = lib.oracle_attn_decode(_ptr(qb), _ptr(knib), _ptr(ksb), _ptr(vnib), _ptr(vsb), T, n_q,
                                n_kv, _ptr(out), _ptr(A))
    if rc:
        raise OracleError(rc)
    return out, A

