"""The no-allocation attention entry point against the one with a workspace
(needs an MI355X): same kernels, so the outputs must be identical bit for bit,
on two calls in a row, the second smaller than the first."""
import numpy as np
import pytest

import binary_g128_bit_amd as tq
from binary_g128_bit_amd import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _cache(seed, T, n_kv, TC):
    g = synth.rng(seed)
    parts = [torch.zeros(tq.tq_kv_bytes(n_kv, TC, p), dtype=torch.uint8, device="cuda") for p in range(4)]
    kc, ks, vc, vs = parts[0], parts[1].view(torch.int16), parts[2], parts[3].view(torch.int16)
    k = torch.from_numpy(g.standard_normal((T, n_kv, 256)).astype(np.float16)).cuda()
    v = torch.from_numpy(g.standard_normal((T, n_kv, 256)).astype(np.float16)).cuda()
    tq.tq_kv_append(k, v, 0, n_kv, TC, kc, ks, vc, vs)
    q = torch.from_numpy(g.standard_normal((6 * n_kv, 256)).astype(np.float16)).cuda()
    return q, kc, ks, vc, vs


def test_noalloc_matches_workspace_entry_point():
    n_kv, TC = 4, 40960
    q, kc, ks, vc, vs = _cache(31000, TC, n_kv, TC)
    n_q = q.shape[0]
    for T in (40000, 1000):                  # two calls in a row, the second smaller
        ws = torch.empty(tq.tq_attn_workspace_bytes(T, n_q, n_kv) // 4, dtype=torch.float32, device="cuda")
        ref = tq.tq_attn_decode(q, kc, ks, vc, vs, T, n_kv, TC, ws)
        out = torch.full((n_q, 256), float("nan"), dtype=torch.float32, device="cuda")
        tq.tq_attn_decode_noalloc(q, kc, ks, vc, vs, T, n_kv, TC, out=out)
        torch.cuda.synchronize()
        a, b = out.cpu().numpy(), ref.cpu().numpy()
        assert np.isfinite(a).all(), T
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), "T=%d differs" % T


def test_noalloc_rejects_above_scratch():
    n_kv, TC = 1, 65536
    q, kc, ks, vc, vs = _cache(31001, 32, n_kv, TC)
    q = torch.zeros(16, 256, dtype=torch.float16, device="cuda")
    with pytest.raises(tq.TQError) as e:
        tq.tq_attn_decode_noalloc(q, kc, ks, vc, vs, 65536, n_kv, TC)
    assert e.value.status == 2
