"""Seeded synthetic inputs for the packed-weight matmul.

This module only draws random numbers and names workload shapes.  It holds none
of the method's arithmetic (no packing, no decoding, no products), so both the
oracle-side tests and the product-side tests and bench can share it.

Distributions (27B-shaped decode weights; the weights themselves are not public):
  * trits t: iid uniform over {-1, 0, +1} (ternary, either storage) or
    {-1, +1} (binary);
  * group scales: float16(exp(N(-4, 0.5))), one per 128 weights along K;
  * affine levels q: iid uniform over {0, 1, 2, 3}; group biases
    float16(-exp(N(-3.5, 0.5)));
  * activations: float16(N(0, 1)) drawn in float32, round-to-nearest-even;
  * integer-exact sets: activations uniform integers in [-8, 8], scales
    2^-j with j uniform in [0, 6] (affine biases -k 2^-j, k in [0, 3]), so
    every partial sum is exactly
    representable in fp32 and any summation order gives the same bits.

RNG: numpy PCG64, seed = 1000 * config_index + matrix_index; per matrix the
draw order is trits, then scales, then activations.
"""
import numpy as np

TERNARY = 0
BINARY = 1
TERNARY5 = 2  # ternary trits stored five to a byte
AFFINE2 = 3   # unsigned 2-bit levels with a scale and a bias per group
GROUP = 128

# Workload shapes (out N, in K).  The 27B-like projection shapes: MLP gate/up
# 5120 -> 17408 and down 17408 -> 5120; full attention q 5120 -> 6144,
# k/v 5120 -> 1024 (4 KV heads x head_dim 256), o 6144 -> 5120; linear
# attention projections 5120 -> 14336, 5120 -> 6144, 6144 -> 5120; LM head
# 5120 -> 248320.
C1 = (1024, 1024)
GATE_UP = (17408, 5120)
DOWN = (5120, 17408)
LM_HEAD = (248320, 5120)
GEMM_WIDTHS = (4, 16, 64, 512)
N_LAYERS = 64


def stack_layers():
    """Per-layer list of (name, N, K) for the 64-layer decode sweep: every
    fourth layer (l % 4 == 3) is full attention, the rest linear attention."""
    layers = []
    for l in range(N_LAYERS):
        mats = [("gate", 17408, 5120), ("up", 17408, 5120), ("down", 5120, 17408)]
        if l % 4 == 3:
            mats += [("q", 6144, 5120), ("k", 1024, 5120), ("v", 1024, 5120),
                     ("o", 5120, 6144)]
        else:
            mats += [("lin_qkv", 14336, 5120), ("lin_z", 6144, 5120),
                     ("lin_out", 5120, 6144)]
        layers.append(mats)
    return layers


def rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def seed_for(config_index, matrix_index):
    return 1000 * config_index + matrix_index


def trits(g, N, K, variant=TERNARY):
    """int8 [N][K] with values in the variant's set."""
    if variant in (TERNARY, TERNARY5):
        return (g.integers(0, 3, size=(N, K), dtype=np.int8) - 1).astype(np.int8)
    return (2 * g.integers(0, 2, size=(N, K), dtype=np.int8) - 1).astype(np.int8)


def scales(g, N, K, group=GROUP):
    """float16 [N][K/group], lognormal(mu=-4, sigma=0.5)."""
    return np.exp(g.normal(-4.0, 0.5, size=(N, K // group))).astype(np.float16)


def activations(g, M, K):
    """float16 [M][K], N(0, 1)."""
    return g.standard_normal(size=(M, K), dtype=np.float32).astype(np.float16)


def int_activations(g, M, K):
    """float16 [M][K], uniform integers in [-8, 8]."""
    return g.integers(-8, 9, size=(M, K)).astype(np.float16)


def pow2_scales(g, N, K, group=GROUP):
    """float16 [N][K/group] equal to 2^-j, j uniform in [0, 6]."""
    return np.ldexp(1.0, -g.integers(0, 7, size=(N, K // group))).astype(np.float16)


def levels(g, N, K):
    """int8 [N][K] affine levels, iid uniform over {0, 1, 2, 3}."""
    return g.integers(0, 4, size=(N, K), dtype=np.int8)


def biases(g, N, K, group=GROUP):
    """float16 [N][K/group] affine offsets, -exp(N(-3.5, 0.5)) (a group minimum)."""
    return (-np.exp(g.normal(-3.5, 0.5, size=(N, K // group)))).astype(np.float16)


def pow2_biases(g, N, K, group=GROUP):
    """float16 [N][K/group] equal to -k * 2^-j, k in [0, 3], j in [0, 6]."""
    k = g.integers(0, 4, size=(N, K // group))
    return (-k * np.ldexp(1.0, -g.integers(0, 7, size=(N, K // group)))).astype(np.float16)


def affine_problem(seed, N, K, M=1, exact=False):
    """(q int8 [N][K], scales f16, biases f16, X f16 [M][K])."""
    g = rng(seed)
    q = levels(g, N, K)
    if exact:
        return q, pow2_scales(g, N, K), pow2_biases(g, N, K), int_activations(g, M, K)
    return q, scales(g, N, K), biases(g, N, K), activations(g, M, K)


def problem(seed, N, K, M=1, variant=TERNARY, exact=False):
    """One seeded problem: (t int8 [N][K], scales f16 [N][G], X f16 [M][K])."""
    g = rng(seed)
    t = trits(g, N, K, variant)
    if exact:
        s = pow2_scales(g, N, K)
        X = int_activations(g, M, K)
    else:
        s = scales(g, N, K)
        X = activations(g, M, K)
    return t, s, X
