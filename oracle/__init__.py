"""Plain fp64 CPU oracle for the ternary / binary g128 packed-weight matmul.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by ``__graft_entry__.smoke()``
and by the CPU-baseline leg of ``bench.py``.  The product package never imports
it, and it imports nothing from the product.

The arithmetic lives in ``tq_oracle.c`` (plain C, built with gcc).  This module
only builds that file and marshals numpy arrays through ctypes.
"""
from .oracle import (  # noqa: F401
    TERNARY, BINARY, TERNARY5, AFFINE2, OracleError, build, load, half_to_double, codes_bytes,
    scales_count, pack, unpack, gemm, gemv, embed, affine_gemm, float_to_half, kv_quant,
    attn_decode, default_threads,
)
