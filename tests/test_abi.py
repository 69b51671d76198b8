"""The C-ABI library loads without a GPU, exports every symbol include/tq.h
declares, and rejects bad arguments on the host before any HIP call."""
import ctypes
import os
import re

import numpy as np
import pytest

import binary_g128_bit_amd as tq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tq.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tq_\w+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    L = tq.lib()
    names = _declared()
    assert names, "no declarations parsed"
    for name in names:
        assert hasattr(L, name), name
    assert sorted(tq.EXPORTS) == names


def test_version_and_sizes():
    assert "gfx950" in tq.tq_version()
    assert tq.tq_codes_bytes(17408, 5120, tq.TQ_TERNARY) == 17408 * 5120 // 4
    assert tq.tq_codes_bytes(17408, 5120, tq.TQ_BINARY) == 17408 * 5120 // 8
    assert tq.tq_scales_count(5120, 17408) == 5120 * 136
    assert tq.tq_codes_bytes(4, 100, tq.TQ_TERNARY) == 0
    assert tq.tq_codes_bytes(4, 128, 7) == 0
    assert tq.tq_scales_count(4, 128, 64) == 0


FAKE = 0x7f0000000000  # 16-byte aligned address that is never dereferenced


@pytest.mark.parametrize("args,status", [
    # (codes, scales, x, y, M, N, K, group, variant)
    ((0, FAKE, FAKE, FAKE, 1, 8, 128, 128, 0), 1),
    ((FAKE, FAKE, FAKE, 0, 1, 8, 128, 128, 0), 1),
    ((FAKE, FAKE, FAKE, FAKE, 1, 0, 128, 128, 0), 2),
    ((FAKE, FAKE, FAKE, FAKE, 0, 8, 128, 128, 0), 2),
    ((FAKE, FAKE, FAKE, FAKE, 1, 8, 100, 128, 0), 2),
    ((FAKE, FAKE, FAKE, FAKE, 1, 8, 0, 128, 0), 2),
    ((FAKE, FAKE, FAKE, FAKE, 1, 8, 131072, 128, 0), 2),
    ((FAKE, FAKE, FAKE, FAKE, 1, 8, 256, 64, 0), 3),
    ((FAKE, FAKE, FAKE, FAKE, 1, 8, 256, 128, 3), 4),
    ((FAKE + 8, FAKE, FAKE, FAKE, 1, 8, 256, 128, 0), 7),
    ((FAKE + 8, FAKE, FAKE, FAKE, 1, 8, 256, 128, 2), 7),
    ((FAKE, FAKE, FAKE, FAKE, 2, 8, 256, 128, 2), 4),       # five-trit bytes: GEMV only
    ((FAKE, FAKE, FAKE, FAKE, 1, 8, 256, 128, 3), 4),       # affine levels need biases
    ((FAKE, FAKE, FAKE + 2, FAKE, 1, 8, 256, 128, 0), 7),
    ((FAKE, FAKE + 1, FAKE, FAKE, 1, 8, 256, 128, 0), 7),
    ((FAKE, FAKE, FAKE, FAKE + 2, 1, 8, 256, 128, 0), 7),
])
def test_device_entry_points_validate_on_host(args, status):
    L = tq.lib()
    codes, scales, x, y, M, N, K, group, variant = args
    p = ctypes.c_void_p
    rc = L.tq_gemm(p(codes), p(scales), p(x), p(y), M, N, K, group, variant, None)
    assert rc == status, L.tq_last_error()
    assert L.tq_last_error()
    if M == 1:
        rc = L.tq_gemv(p(codes), p(scales), p(x), p(y), N, K, group, variant, None)
        assert rc == status


@pytest.mark.parametrize("args,status", [
    # (codes, scales, ids, out, n_ids, N, K, group, variant)
    ((0, FAKE, FAKE, FAKE, 4, 8, 128, 128, 0), 1),
    ((FAKE, FAKE, 0, FAKE, 4, 8, 128, 128, 0), 1),
    ((FAKE, FAKE, FAKE, 0, 4, 8, 128, 128, 1), 1),
    ((FAKE, FAKE, FAKE, FAKE, -1, 8, 128, 128, 0), 2),
    ((FAKE, FAKE, FAKE, FAKE, 1 << 31, 8, 128, 128, 0), 2),
    ((FAKE, FAKE, FAKE, FAKE, 4, 0, 128, 128, 0), 2),
    ((FAKE, FAKE, FAKE, FAKE, 4, 8, 200, 128, 0), 2),
    ((FAKE, FAKE, FAKE, FAKE, 4, 8, 256, 64, 0), 3),
    ((FAKE, FAKE, FAKE, FAKE, 4, 8, 256, 128, 3), 4),
    ((FAKE, FAKE, FAKE, FAKE, 4, 8, 256, 128, 2), 4),       # five-trit tables: not for rows
    ((FAKE, FAKE, FAKE, FAKE, 4, 8, 256, 128, 3), 4),       # affine tables: not for rows
    ((FAKE + 2, FAKE, FAKE, FAKE, 4, 8, 256, 128, 0), 7),
    ((FAKE, FAKE + 1, FAKE, FAKE, 4, 8, 256, 128, 0), 7),
    ((FAKE, FAKE, FAKE + 2, FAKE, 4, 8, 256, 128, 0), 7),
    ((FAKE, FAKE, FAKE, FAKE + 8, 4, 8, 256, 128, 0), 7),
    # nothing to do: no pointer is looked at
    ((0, 0, 0, 0, 0, 8, 256, 128, 0), 0),
])
def test_embed_validates_on_host(args, status):
    L = tq.lib()
    codes, scales, ids, out, n_ids, N, K, group, variant = args
    p = ctypes.c_void_p
    rc = L.tq_embed(p(codes), p(scales), p(ids), p(out), n_ids, N, K, group, variant, None)
    assert rc == status, L.tq_last_error()
    if status:
        assert L.tq_last_error()
    # codes need only 4-byte alignment: an offset of 4 passes that check and
    # fails on the NULL output instead
    if status == 0:
        rc = L.tq_embed(p(FAKE + 4), p(FAKE), p(FAKE), p(0), 2, N, K, group, variant, None)
        assert rc == 1, L.tq_last_error()


@pytest.mark.parametrize("args,status", [
    # (codes, scales, biases, x, y, N, K, group)
    ((FAKE, FAKE, 0, FAKE, FAKE, 8, 256, 128), 1),
    ((0, FAKE, FAKE, FAKE, FAKE, 8, 256, 128), 1),
    ((FAKE, FAKE, FAKE, FAKE, FAKE, 0, 256, 128), 2),
    ((FAKE, FAKE, FAKE, FAKE, FAKE, 8, 200, 128), 2),
    ((FAKE, FAKE, FAKE, FAKE, FAKE, 8, 20480 + 128, 128), 2),   # above the affine limit
    ((FAKE, FAKE, FAKE, FAKE, FAKE, 8, 256, 64), 3),
    ((FAKE, FAKE, FAKE + 1, FAKE, FAKE, 8, 256, 128), 7),
    ((FAKE + 4, FAKE, FAKE, FAKE, FAKE, 8, 256, 128), 7),
    ((FAKE, FAKE, FAKE, FAKE + 8, FAKE, 8, 256, 128), 7),
])
def test_gemv_affine_validates_on_host(args, status):
    L = tq.lib()
    codes, scales, biases, x, y, N, K, group = args
    p = ctypes.c_void_p
    rc = L.tq_gemv_affine(p(codes), p(scales), p(biases), p(x), p(y), N, K, group, None)
    assert rc == status, L.tq_last_error()
    assert L.tq_last_error()


def test_kv_sizes_and_validation():
    L = tq.lib()
    assert tq.tq_kv_bytes(4, 262144, tq.TQ_KV_K_CODES) == 4 * 262144 * 128
    assert tq.tq_kv_bytes(4, 262144, tq.TQ_KV_V_SCALES) == 4 * 262144 * 16
    # 16 layers x 4 heads x (2 x 128 + 2 x 16) bytes per token: 4.5 bits per element
    per_token = 16 * sum(tq.tq_kv_bytes(4, 32, p) for p in range(4)) // 32
    assert per_token == 16 * 4 * 288 and 8 * per_token / (16 * 2 * 4 * 256) == 4.5
    assert tq.tq_kv_bytes(4, 100, 0) == 0 and tq.tq_kv_bytes(0, 64, 0) == 0
    assert tq.tq_kv_bytes(4, 64, 4) == 0
    assert tq.tq_attn_workspace_bytes(0, 24, 4) == 0
    assert tq.tq_attn_workspace_bytes(100, 25, 4) == 0          # not a multiple
    assert tq.tq_attn_workspace_bytes(100, 68, 4) == 0          # group above 16
    assert tq.tq_attn_workspace_bytes(100, 24, 4) > 0
    p = ctypes.c_void_p
    F = p(FAKE)
    ws = tq.tq_attn_workspace_bytes(64, 24, 4)
    cases = [  # (args to tq_attn_decode, status)
        ((F, F, F, F, F, 64, 24, 4, 64, F, F, ws, None), 0),
        ((F, F, F, F, F, 65, 24, 4, 64, F, F, ws, None), 2),
        ((F, F, F, F, F, 0, 24, 4, 64, F, F, ws, None), 2),
        ((F, F, F, F, F, 64, 24, 4, 60, F, F, ws, None), 2),
        ((F, F, F, F, F, 64, 20, 8, 64, F, F, ws, None), 2),
        ((F, F, F, F, F, 64, 24, 4, 64, F, F, ws - 4, None), 2),
        ((F, p(0), F, F, F, 64, 24, 4, 64, F, F, ws, None), 1),
        ((p(FAKE + 8), F, F, F, F, 64, 24, 4, 64, F, F, ws, None), 7),
        ((F, F, F, F, F, 64, 24, 4, 64, p(FAKE + 2), F, ws, None), 7),
    ]
    for args, status in cases:
        if status == 0:
            continue            # a valid call would launch
        assert L.tq_attn_decode(*args) == status, (args, L.tq_last_error())
    assert L.tq_kv_append(F, F, 0, 0, 4, 64, F, F, F, F, None) == 0       # nothing to do
    assert L.tq_kv_append(F, F, 2, 63, 4, 64, F, F, F, F, None) == 2
    assert L.tq_kv_append(F, F, 1, 0, 4, 64, F, F, F, p(0), None) == 1
    assert L.tq_kv_append(F, F, 1, 0, 4, 64, F, F, p(FAKE + 4), F, None) == 7
    assert L.tq_kv_append(F, F, 1, 0, 65, 64, F, F, F, F, None) == 2


def test_pack_errors():
    t = np.zeros((2, 128), np.int8)
    t[1, 5] = 2
    with pytest.raises(tq.TQError) as e:
        tq.tq_pack(t)
    assert e.value.status == 5 and e.value.index == 133
    tb = np.ones((2, 128), np.int8)
    tb[0, 9] = 0
    with pytest.raises(tq.TQError) as e:
        tq.tq_pack(tb, tq.TQ_BINARY)
    assert e.value.status == 5 and e.value.index == 9
    with pytest.raises(tq.TQError) as e:
        tq.tq_pack(np.zeros((2, 100), np.int8))
    assert e.value.status == 2
    with pytest.raises(tq.TQError) as e:
        tq.tq_pack(np.zeros((2, 128), np.int8), 4)
    assert e.value.status == 4
    assert tq.tq_codes_bytes(2, 128, 4) == 0
    L = tq.lib()
    assert L.tq_pack(None, 2, 128, 128, 0, None) == 1
    assert L.tq_pack(t.ctypes.data, 2, 128, 64, 0, t.ctypes.data) == 3


def test_unpack_rejects_code3_with_index():
    codes = np.full((3, 64), 0x55, np.uint8)       # N=3, K=256
    codes[2, 10] = 0x55 | (3 << 6)                  # slot 3 of byte 10 in row 2
    with pytest.raises(tq.TQError) as e:
        tq.tq_unpack(codes, 3, 256)
    assert e.value.status == 6
    assert e.value.index == 2 * 256 + 10 * 4 + 3
    assert "code 3" in str(e.value)


def _cpu_problem(N=8, K=256):
    import torch
    codes = torch.zeros(tq.tq_codes_bytes(N, K, tq.TQ_TERNARY), dtype=torch.uint8)
    scales = torch.zeros(N, K // 128, dtype=torch.float16)
    return codes, scales


def test_binding_checks_output_sizes_before_the_call():
    """Wrong-sized outputs and activations are refused in Python, before any
    pointer reaches the library (a short y would be written past its end on
    the device).  CPU tensors pass the size checks and then fail the
    device-tensor check, so no GPU is touched here."""
    import torch
    N, K = 8, 256
    codes, scales = _cpu_problem(N, K)
    x = torch.zeros(K, dtype=torch.float16)
    with pytest.raises(ValueError, match="y holds 7"):
        tq.tq_gemv(codes, scales, x, torch.zeros(N - 1))
    with pytest.raises(ValueError, match="device tensor"):
        tq.tq_gemv(codes, scales, x, torch.zeros(N))
    with pytest.raises(ValueError, match="x holds"):
        tq.tq_gemv(codes, scales, torch.zeros(2, K, dtype=torch.float16), torch.zeros(N))
    X = torch.zeros(4, K, dtype=torch.float16)
    with pytest.raises(ValueError, match="Y has shape"):
        tq.tq_gemm(codes, scales, X, torch.zeros(4, N - 1))
    with pytest.raises(ValueError, match="Y has shape"):
        tq.tq_gemm(codes, scales, X, torch.zeros(N, 4))
    with pytest.raises(ValueError, match="device tensor"):
        tq.tq_gemm(codes, scales, X, torch.zeros(4, N))
    with pytest.raises(ValueError, match="y holds"):
        tq.tq_gemv_affine(codes, scales, scales.clone(), x, torch.zeros(N + 1))


def test_binding_checks_attention_shapes():
    import torch
    n_kv, t_cap, n_q = 2, 64, 8
    parts = [torch.zeros(tq.tq_kv_bytes(n_kv, t_cap, p), dtype=torch.uint8) for p in range(4)]
    kc, ks, vc, vs = parts[0], parts[1].view(torch.int16), parts[2], parts[3].view(torch.int16)
    q = torch.zeros(n_q, 256, dtype=torch.float16)
    ws = torch.zeros(1 << 16, dtype=torch.float32)
    with pytest.raises(ValueError, match="q must be"):
        tq.tq_attn_decode(torch.zeros(n_q, 128, dtype=torch.float16), kc, ks, vc, vs, 10, n_kv, t_cap, ws)
    with pytest.raises(ValueError, match="out holds"):
        tq.tq_attn_decode(q, kc, ks, vc, vs, 10, n_kv, t_cap, ws, out=torch.zeros(n_q - 1, 256))
    with pytest.raises(ValueError, match="kc holds"):
        tq.tq_attn_decode(q, kc[:-16], ks, vc, vs, 10, n_kv, t_cap, ws)
    with pytest.raises(ValueError, match="vs holds"):
        tq.tq_attn_decode(q, kc, ks, vc, vs[:-8], 10, n_kv, t_cap, ws)
    with pytest.raises(ValueError, match="device tensor"):
        tq.tq_attn_decode(q, kc, ks, vc, vs, 10, n_kv, t_cap, ws)


def test_attn_noalloc_validates_on_host():
    """The no-allocation attention entry point checks shapes, pointers and its
    scratch limit before any HIP call (so this runs without a GPU)."""
    L = tq.lib()
    F = FAKE
    call = lambda T, n_q, n_kv, t_cap, q=F, out=F: L.tq_attn_decode_noalloc(
        q, F, F, F, F, T, n_q, n_kv, t_cap, out, None)
    assert call(10, 24, 4, 64, q=0) == 1
    assert call(10, 24, 4, 64, out=0) == 1
    assert call(65, 24, 4, 64) == 2          # T above the capacity
    assert call(10, 25, 4, 64) == 2          # n_q not a multiple of n_kv
    assert call(10, 24, 4, 64, q=F + 8) == 7
    # one KV head with 16 query heads at T = 65536: 8.06 MiB of partial rows,
    # above the 8 MiB scratch
    need = tq.tq_attn_workspace_bytes(65536, 16, 1)
    assert need > 8 << 20
    assert call(65536, 16, 1, 65536) == 2
    assert "scratch" in L.tq_last_error().decode()
    # the model's shape fits at every context length tried
    for T in (1, 4096, 32768, 102400, 262144, 1 << 20):
        assert tq.tq_attn_workspace_bytes(T, 24, 4) <= 8 << 20, T


def test_gemm_workspace_bytes_and_alignment():
    """The K-split workspace size (host only), and a misaligned workspace
    rejected before any launch."""
    assert tq.tq_gemm_workspace_bytes(4, 1000, 5120) == 0
    assert tq.tq_gemm_workspace_bytes(16, 1000, 384) == 0          # odd group count
    assert tq.tq_gemm_workspace_bytes(16, 1000, 2048) == 0         # one slice
    assert tq.tq_gemm_workspace_bytes(16, 1000, 5120) == 3 * 16 * 1000 * 4
    assert tq.tq_gemm_workspace_bytes(8, 5120, 17408) == 9 * 8 * 5120 * 4
    assert tq.tq_gemm_workspace_bytes(16, 1000, 5120, variant=tq.TQ_BINARY) == 0
    assert tq.tq_gemm_workspace_bytes(16, 1000, 100) == 0          # invalid K: no error
    assert tq.tq_gemm_workspace_bytes(16, 200000, 5120) == 0       # very tall: batched kernel
    assert tq.tq_gemm_workspace_bytes(64, 1000, 5120) == 5 * 64 * 1000 * 4
    assert tq.tq_gemm_workspace_bytes(65, 1000, 5120) == 0
    L = tq.lib()
    fake = 1 << 20
    rc = L.tq_gemm_ws(fake, fake, fake, fake, 16, 1000, 5120, 128, 0, fake + 8, 1 << 20, None)
    assert rc == 7 and b"workspace" in L.tq_last_error()
