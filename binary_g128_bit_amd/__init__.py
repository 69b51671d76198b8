"""Ternary / binary g128 packed-weight matmul for AMD MI355X (gfx950).

Thin ctypes binding over ``libtq.so`` (C ABI in ``include/tq.h``).  The
functions carry the C names and only marshal arguments: shapes are read off the
arrays, pointers and the current HIP stream are passed through, and a non-zero
status becomes a :class:`TQError`.  Every step of the computation runs in the
library.  PyTorch is used only for device memory and streams.

Build the library first: ``python -m binary_g128_bit_amd.build``.  There is no
fallback: calling a GPU entry point without the built library raises.
"""
import ctypes
import functools
import os

import numpy as np

TQ_TERNARY = 0
TQ_BINARY = 1
TQ_TERNARY5 = 2  # five trits per byte (GEMV only)
TQ_AFFINE2 = 3   # levels q in {0..3}, scale and bias per group (tq_gemv_affine)
GROUP = 128
TQ_KV_K_CODES, TQ_KV_K_SCALES, TQ_KV_V_CODES, TQ_KV_V_SCALES = 0, 1, 2, 3

_STATUS = {0: "TQ_OK", 1: "TQ_ERR_NULL", 2: "TQ_ERR_SHAPE", 3: "TQ_ERR_GROUP",
           4: "TQ_ERR_VARIANT", 5: "TQ_ERR_VALUE", 6: "TQ_ERR_CODE", 7: "TQ_ERR_ALIGN",
           8: "TQ_ERR_HIP"}

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libtq.so")

# every symbol include/tq.h declares
EXPORTS = ("tq_codes_bytes", "tq_scales_count", "tq_pack", "tq_unpack", "tq_gemv", "tq_gemm",
           "tq_gemm_workspace_bytes", "tq_gemm_ws", "tq_embed", "tq_gemv_affine", "tq_kv_bytes",
           "tq_kv_append", "tq_attn_workspace_bytes", "tq_attn_decode", "tq_attn_decode_noalloc",
           "tq_stream_read", "tq_last_error", "tq_last_error_index", "tq_version")


class TQError(RuntimeError):
    """A non-zero tq_status; ``.status`` is the code, ``.index`` the flat index
    attached to TQ_ERR_VALUE / TQ_ERR_CODE (else -1)."""

    def __init__(self, status, message, index=-1):
        self.status = status
        self.index = index
        super().__init__("%s: %s" % (_STATUS.get(status, str(status)), message))


_lib = None


def lib():
    """The loaded libtq.so; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("libtq.so is not built (%s); run `python -m binary_g128_bit_amd.build`"
                           % LIB_PATH)
    L = ctypes.CDLL(LIB_PATH)
    i64, i32, vp = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p
    L.tq_codes_bytes.argtypes = [i64, i64, i32]
    L.tq_codes_bytes.restype = ctypes.c_size_t
    L.tq_scales_count.argtypes = [i64, i64, i32]
    L.tq_scales_count.restype = ctypes.c_size_t
    L.tq_pack.argtypes = [vp, i64, i64, i32, i32, vp]
    L.tq_pack.restype = i32
    L.tq_unpack.argtypes = [vp, i64, i64, i32, i32, vp]
    L.tq_unpack.restype = i32
    L.tq_gemv.argtypes = [vp, vp, vp, vp, i64, i64, i32, i32, vp]
    L.tq_gemv.restype = i32
    L.tq_gemm.argtypes = [vp, vp, vp, vp, i64, i64, i64, i32, i32, vp]
    L.tq_gemm.restype = i32
    L.tq_gemm_workspace_bytes.argtypes = [i64, i64, i64, i32, i32]
    L.tq_gemm_workspace_bytes.restype = ctypes.c_size_t
    L.tq_gemm_ws.argtypes = [vp, vp, vp, vp, i64, i64, i64, i32, i32, vp, ctypes.c_size_t, vp]
    L.tq_gemm_ws.restype = i32
    L.tq_embed.argtypes = [vp, vp, vp, vp, i64, i64, i64, i32, i32, vp]
    L.tq_embed.restype = i32
    L.tq_gemv_affine.argtypes = [vp, vp, vp, vp, vp, i64, i64, i32, vp]
    L.tq_gemv_affine.restype = i32
    L.tq_kv_bytes.argtypes = [i64, i64, i32]
    L.tq_kv_bytes.restype = ctypes.c_size_t
    L.tq_kv_append.argtypes = [vp, vp, i64, i64, i64, i64, vp, vp, vp, vp, vp]
    L.tq_kv_append.restype = i32
    L.tq_attn_workspace_bytes.argtypes = [i64, i64, i64]
    L.tq_attn_workspace_bytes.restype = ctypes.c_size_t
    L.tq_attn_decode.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, vp, vp, ctypes.c_size_t, vp]
    L.tq_attn_decode.restype = i32
    L.tq_attn_decode_noalloc.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, vp, vp]
    L.tq_attn_decode_noalloc.restype = i32
    L.tq_stream_read.argtypes = [vp, ctypes.c_size_t, vp, i32, vp]
    L.tq_stream_read.restype = i32
    L.tq_last_error.argtypes = []
    L.tq_last_error.restype = ctypes.c_char_p
    L.tq_last_error_index.argtypes = []
    L.tq_last_error_index.restype = i64
    L.tq_version.argtypes = []
    L.tq_version.restype = ctypes.c_char_p
    _lib = L
    return L


def _check(status):
    if status != 0:
        L = lib()
        raise TQError(status, L.tq_last_error().decode(), L.tq_last_error_index())


def tq_version():
    return lib().tq_version().decode()


def tq_codes_bytes(N, K, variant=TQ_TERNARY):
    return lib().tq_codes_bytes(N, K, variant)


def tq_scales_count(N, K, group=GROUP):
    return lib().tq_scales_count(N, K, group)


# ------------------------------------------------------------------ host side
def tq_pack(t, variant=TQ_TERNARY, group=GROUP):
    """int8 t [N][K] (numpy) -> uint8 codes [N][row bytes]: K/4 (ternary),
    K/8 (binary) or 26*K/128 rounded up to 16 (five-trit bytes)."""
    t = np.ascontiguousarray(t, dtype=np.int8)
    if t.ndim != 2:
        raise ValueError("t must be 2-D [N][K]")
    N, K = t.shape
    nbytes = lib().tq_codes_bytes(N, K, variant) if N > 0 else 0
    out = np.empty((N, max(nbytes // max(N, 1), 1)), dtype=np.uint8)
    _check(lib().tq_pack(t.ctypes.data, N, K, group, variant, out.ctypes.data))
    return out


def tq_unpack(codes, N, K, variant=TQ_TERNARY, group=GROUP):
    """uint8 codes -> int8 t [N][K] (numpy)."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    need = lib().tq_codes_bytes(N, K, variant)
    if need and codes.size < need:
        raise ValueError("codes holds %d bytes, %d needed" % (codes.size, need))
    t = np.empty((N, K), dtype=np.int8)
    _check(lib().tq_unpack(codes.ctypes.data, N, K, group, variant, t.ctypes.data))
    return t


# ---------------------------------------------------------------- device side
def _dev(tensor, name, dtypes):
    if not tensor.is_cuda:
        raise ValueError("%s must be a device tensor" % name)
    if tensor.dtype not in dtypes:
        raise ValueError("%s has dtype %s, expected one of %s" % (name, tensor.dtype, dtypes))
    if not tensor.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return tensor.data_ptr()


def _stream(stream, tensor):
    """The HIP stream to launch on: `stream`, else the current stream of the
    device that holds `tensor` (read as a raw handle: building a torch Stream
    object per call costs about 2.5 us of host time)."""
    import torch
    if stream is not None:
        return ctypes.c_void_p(stream.cuda_stream)
    try:
        return ctypes.c_void_p(torch._C._cuda_getCurrentRawStream(tensor.get_device()))
    except AttributeError:  # a torch build without the raw accessor
        return ctypes.c_void_p(torch.cuda.current_stream(tensor.device).cuda_stream)


@functools.lru_cache(maxsize=1024)
def _codes_bytes(N, K, variant):
    # the library's byte count for a shape, asked once per shape: a ctypes
    # call costs about a microsecond of host time on every launch
    return lib().tq_codes_bytes(N, K, variant)


def _shape_checks(codes, scales, K, variant):
    N = scales.shape[0]
    if scales.dim() != 2 or scales.shape[1] * GROUP != K:
        raise ValueError("scales must be [N][K/128] with K=%d" % K)
    need = _codes_bytes(N, K, variant)
    if codes.numel() != need:
        raise ValueError("codes holds %d bytes, %d needed for N=%d K=%d" % (codes.numel(), need, N, K))
    return N


def _out_check(out, name, numel):
    if out.numel() != numel:
        raise ValueError("%s holds %d elements, %d needed" % (name, out.numel(), numel))


def tq_gemv(codes, scales, x, y=None, variant=TQ_TERNARY, group=GROUP, stream=None):
    """y[N] = W x on the current stream.  codes uint8, scales float16 [N][K/128],
    x float16 [K], y float32 [N] (allocated if None)."""
    import torch
    K = x.shape[-1]
    _out_check(x, "x", K)
    N = _shape_checks(codes, scales, K, variant)
    if y is None:
        y = torch.empty(N, dtype=torch.float32, device=x.device)
    _out_check(y, "y", N)
    half = (torch.float16, torch.int16)
    _check(lib().tq_gemv(_dev(codes, "codes", (torch.uint8,)), _dev(scales, "scales", half),
                         _dev(x, "x", half), _dev(y, "y", (torch.float32,)), N, K, group, variant,
                         _stream(stream, x)))
    return y


def tq_gemm_workspace_bytes(M, N, K, variant=TQ_TERNARY, group=GROUP):
    """Device workspace bytes tq_gemm can use for this shape (0: none)."""
    return lib().tq_gemm_workspace_bytes(M, N, K, group, variant)


def tq_gemm(codes, scales, X, Y=None, variant=TQ_TERNARY, group=GROUP, stream=None, workspace=None):
    """Y[M][N] = X W^T on the current stream (or `stream`).  X float16
    [M][K].  Shapes that can use a workspace (tq_gemm_workspace_bytes > 0)
    get `workspace` (a device tensor of at least that many bytes) or, when it
    is None, one from torch's allocator on the launch stream."""
    import torch
    M, K = X.shape
    N = _shape_checks(codes, scales, K, variant)
    if Y is None:
        Y = torch.empty((M, N), dtype=torch.float32, device=X.device)
    if tuple(Y.shape) != (M, N):
        raise ValueError("Y has shape %s, (%d, %d) needed" % (tuple(Y.shape), M, N))
    half = (torch.float16, torch.int16)
    args = (_dev(codes, "codes", (torch.uint8,)), _dev(scales, "scales", half), _dev(X, "X", half),
            _dev(Y, "Y", (torch.float32,)), M, N, K, group, variant)
    need = lib().tq_gemm_workspace_bytes(M, N, K, group, variant)
    if need == 0:
        _check(lib().tq_gemm(*args, _stream(stream, X)))
        return Y
    if workspace is None:
        # allocated on the launch stream, so that torch reuses it only after
        # this launch's work on that stream
        if stream is None:
            workspace = torch.empty(need, dtype=torch.uint8, device=X.device)
        else:
            with torch.cuda.stream(stream):
                workspace = torch.empty(need, dtype=torch.uint8, device=X.device)
    wbytes = workspace.numel() * workspace.element_size()
    _check(lib().tq_gemm_ws(*args, _dev(workspace, "workspace", (torch.uint8, torch.float32)), wbytes,
                            _stream(stream, X)))
    return Y


def tq_embed(codes, scales, ids, out=None, variant=TQ_TERNARY, group=GROUP, stream=None):
    """FP16 rows out[n_ids][K] = s[ids] * t[ids] on the current stream.
    codes uint8 table, scales float16 [N][K/128], ids int32 [n_ids]."""
    import torch
    N, G = scales.shape
    K = G * GROUP
    _shape_checks(codes, scales, K, variant)
    n_ids = ids.numel()
    if out is None:
        out = torch.empty((n_ids, K), dtype=torch.float16, device=ids.device)
    if out.numel() != n_ids * K:
        raise ValueError("out holds %d values, %d needed" % (out.numel(), n_ids * K))
    half = (torch.float16, torch.int16)
    _check(lib().tq_embed(_dev(codes, "codes", (torch.uint8,)), _dev(scales, "scales", half),
                          _dev(ids, "ids", (torch.int32,)), _dev(out, "out", half), n_ids, N, K,
                          group, variant, _stream(stream, codes)))
    return out


def tq_gemv_affine(codes, scales, biases, x, y=None, group=GROUP, stream=None):
    """y[N] = W x with w = s * q + b (affine 2-bit levels) on the current
    stream.  codes uint8 [N][K/4], scales / biases float16 [N][K/128]."""
    import torch
    K = x.shape[-1]
    _out_check(x, "x", K)
    N = _shape_checks(codes, scales, K, TQ_AFFINE2)
    if tuple(biases.shape) != tuple(scales.shape):
        raise ValueError("biases must have the shape of scales")
    if y is None:
        y = torch.empty(N, dtype=torch.float32, device=x.device)
    _out_check(y, "y", N)
    half = (torch.float16, torch.int16)
    _check(lib().tq_gemv_affine(_dev(codes, "codes", (torch.uint8,)), _dev(scales, "scales", half),
                                _dev(biases, "biases", half), _dev(x, "x", half),
                                _dev(y, "y", (torch.float32,)), N, K, group, _stream(stream, x)))
    return y


# ------------------------------------------------------- measurement aid
def tq_stream_read(buf, sink, blocks_per_cu=1, stream=None):
    """Plain streaming read of the whole device tensor `buf` (a multiple of 16
    bytes): the bandwidth ceiling for a launch of the same size.  `sink` is a
    device tensor of at least 4 bytes."""
    import torch
    if sink.numel() * sink.element_size() < 4:
        raise ValueError("sink needs 4 bytes")
    nbytes = buf.numel() * buf.element_size()
    _check(lib().tq_stream_read(_dev(buf, "buf", (torch.uint8, torch.int32, torch.int16, torch.float16,
                                                  torch.float32)),
                                nbytes, _dev(sink, "sink", (torch.int32, torch.uint8, torch.float32)),
                                blocks_per_cu, _stream(stream, buf)))


# ------------------------------------------------------- 4-bit KV cache
def tq_kv_bytes(n_kv, t_cap, part):
    return lib().tq_kv_bytes(n_kv, t_cap, part)


def tq_attn_workspace_bytes(T, n_q, n_kv):
    return lib().tq_attn_workspace_bytes(T, n_q, n_kv)


def _cache_checks(n_kv, t_cap, kc, ks, vc, vs):
    """Each cache array must hold exactly tq_kv_bytes(n_kv, t_cap, part) bytes."""
    for arr, part, name in ((kc, TQ_KV_K_CODES, "kc"), (ks, TQ_KV_K_SCALES, "ks"),
                            (vc, TQ_KV_V_CODES, "vc"), (vs, TQ_KV_V_SCALES, "vs")):
        need = tq_kv_bytes(n_kv, t_cap, part)
        if need and arr.numel() * arr.element_size() != need:  # 0: the C call reports the shape
            raise ValueError("%s holds %d bytes, %d needed" % (
                name, arr.numel() * arr.element_size(), need))


def tq_kv_append(k, v, pos, n_kv, t_cap, kc, ks, vc, vs, stream=None):
    """Quantize k, v (float16 [n_tok][n_kv][256]) into cache positions
    [pos, pos + n_tok).  kc / vc uint8 and ks / vs float16 (or int16) device
    arrays of tq_kv_bytes(n_kv, t_cap, part) bytes."""
    import torch
    if k.shape != v.shape or k.dim() != 3 or k.shape[1] != n_kv or k.shape[2] != 256:
        raise ValueError("k and v must be [n_tok][n_kv][256]")
    half = (torch.float16, torch.int16)
    _cache_checks(n_kv, t_cap, kc, ks, vc, vs)
    _check(lib().tq_kv_append(_dev(k, "k", half), _dev(v, "v", half), k.shape[0], pos, n_kv, t_cap,
                              _dev(kc, "kc", (torch.uint8,)), _dev(ks, "ks", half),
                              _dev(vc, "vc", (torch.uint8,)), _dev(vs, "vs", half), _stream(stream, k)))


def tq_attn_decode(q, kc, ks, vc, vs, T, n_kv, t_cap, workspace, out=None, stream=None):
    """Decode attention of q (float16 [n_q][256]) over cache positions [0, T).
    workspace: float32 device array of tq_attn_workspace_bytes(T, n_q, n_kv)
    bytes or more.  Returns out float32 [n_q][256]."""
    import torch
    if q.dim() != 2 or q.shape[1] != 256:
        raise ValueError("q must be [n_q][256], got %s" % (tuple(q.shape),))
    n_q = q.shape[0]
    if out is None:
        out = torch.empty(n_q, 256, dtype=torch.float32, device=q.device)
    _out_check(out, "out", n_q * 256)
    _cache_checks(n_kv, t_cap, kc, ks, vc, vs)
    half = (torch.float16, torch.int16)
    _check(lib().tq_attn_decode(_dev(q, "q", half), _dev(kc, "kc", (torch.uint8,)), _dev(ks, "ks", half),
                                _dev(vc, "vc", (torch.uint8,)), _dev(vs, "vs", half), T, n_q, n_kv,
                                t_cap, _dev(out, "out", (torch.float32,)),
                                _dev(workspace, "workspace", (torch.float32, torch.uint8)),
                                workspace.numel() * workspace.element_size(), _stream(stream, q)))
    return out


def tq_attn_decode_noalloc(q, kc, ks, vc, vs, T, n_kv, t_cap, out=None, stream=None):
    """tq_attn_decode on the library's own device scratch: no workspace
    argument, nothing allocated by the call (pass `out` to allocate nothing
    here either).  Calls that overlap on one GPU race."""
    import torch
    if q.dim() != 2 or q.shape[1] != 256:
        raise ValueError("q must be [n_q][256], got %s" % (tuple(q.shape),))
    n_q = q.shape[0]
    if out is None:
        out = torch.empty(n_q, 256, dtype=torch.float32, device=q.device)
    _out_check(out, "out", n_q * 256)
    _cache_checks(n_kv, t_cap, kc, ks, vc, vs)
    half = (torch.float16, torch.int16)
    _check(lib().tq_attn_decode_noalloc(_dev(q, "q", half), _dev(kc, "kc", (torch.uint8,)),
                                        _dev(ks, "ks", half), _dev(vc, "vc", (torch.uint8,)),
                                        _dev(vs, "vs", half), T, n_q, n_kv, t_cap,
                                        _dev(out, "out", (torch.float32,)), _stream(stream, q)))
    return out
