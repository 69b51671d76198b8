#!/usr/bin/env python3
"""Batch-1 ternary g128 decode GEMV on the 27B-like MLP shapes, one MI355X.

A step is one token's pass over one MLP block of packed ternary weights:
gate 5120->17408, up 5120->17408 and down 17408->5120.  gate and up read the
same activation, so they are stored as one 34816 x 5120 matrix (rows of gate,
then rows of up) and run as one GEMV launch; down is a second launch.  Both go
through the C ABI.  Weights rotate over >= 1 GiB of distinct device buffers so
that no step reads from the 256 MB last-level cache what the previous one left
there.  Inputs are resident in HBM before the timed region starts.

Prints ONE JSON line: packed-weight GB/s (value), % of the 8 TB/s HBM peak,
the roofline object of the dominant kernel (its launches timed one by one with
HIP events on its stream), the oracle's CPU baseline on a bounded sample of the
same workload, and context figures measured in the same run: the 64-layer
stack sweep (equivalent tokens/s, eager and graph-replayed), the small-batch
GEMM widths, the 1-bit variant and the LM head.

--only-step runs just the timed step (for counter collection); --copy-calibration
runs a plain 1 GiB device copy whose known byte count scales the HBM counters.
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0        # MI355X HBM3E, vendor figure
PEAK_F16_TFLOPS = 2500.0     # MI355X dense fp16/bf16 MFMA, vendor figure
STACK_BYTES = 6_595_543_040  # packed bytes of the 64-layer 24.83B-weight stack
COPY_BYTES = 1 << 30         # bytes read (and written) by the calibration copy


def packed_bytes(N, K, variant=0):
    return N * K // (8 if variant else 4) + 2 * N * K // 128


def parse():
    p = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=300)
    p.add_argument("--warmup", type=int, default=1000,
                   help="untimed steps first; the clocks take about 20 ms of load to settle")
    p.add_argument("--rotate-gib", type=float, default=1.0)
    p.add_argument("--cpu-seconds", type=float, default=10.0,
                   help="target duration of the oracle's CPU-baseline sample")
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU baseline")
    p.add_argument("--no-extras", action="store_true",
                   help="skip the stack sweep, GEMM, binary and LM-head figures")
    p.add_argument("--only-step", action="store_true",
                   help="run only the timed step (counter runs); implies --no-cpu --no-extras")
    p.add_argument("--copy-calibration", action="store_true",
                   help="run only a 1 GiB device-to-device copy, 5 times")
    return p.parse_args()


def source_hash(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def read_traffic(kernel_tag, src_hash):
    """Scaled HBM bytes per launch from a committed rocprofv3 --pmc summary,
    or None when absent or taken on a different kernel source."""
    path = os.path.join(ROOT, "profiles", "%s_counters.json" % kernel_tag)
    if not os.path.exists(path):
        return None
    try:
        with open(path) as f:
            d = json.load(f)
    except (OSError, ValueError):
        return None
    if d.get("source_sha256_16") != src_hash:
        return None
    return d.get("hbm_bytes_per_launch")


def cpu_baseline(mats, seconds):
    """The oracle, as it stands, on the step's matrices on all the host cores
    this process may use: whole passes over gate, up and down, repeated until
    about `seconds` have elapsed (or the first rows of each matrix if a single
    pass would take longer).  Returns the cpu_baseline object."""
    import oracle
    threads = oracle.default_threads()
    codes, s, x, N, K = mats[0]
    t0 = time.perf_counter()
    oracle.gemm(codes[:256], s[:256], x, 256, K, threads=threads)
    per_weight = (time.perf_counter() - t0) / (256 * K)
    total_weights = sum(m[3] * m[4] for m in mats)
    frac = min(1.0, seconds / max(per_weight * total_weights, 1e-12))
    done_bytes, passes = 0, 0
    t0 = time.perf_counter()
    while True:
        for codes, s, x, N, K in mats:
            n = max(64, int(N * frac))
            oracle.gemm(codes[:n], s[:n], x, n, K, threads=threads)
            done_bytes += packed_bytes(n, K)
        passes += 1
        dt = time.perf_counter() - t0
        if dt >= seconds or frac < 1.0 or passes >= 10000:
            break
    what = ("%d whole passes over gate, up and down (%d weights each pass)" % (passes, total_weights)
            if frac >= 1.0 else "the first %.1f%% of the rows of gate, up and down" % (100 * frac))
    return {"value": round(done_bytes / dt / 1e9, 4), "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "sample": "fp64 oracle GEMV, batch 1: %s, %.1f s" % (what, dt)}


class Dev:
    """Device-side synthetic weights for the timing-only figures (the parity
    tests check the same kernels on the same shapes against the oracle).
    Ternary code bytes are drawn uniformly from the 81 bytes whose four slots
    are valid codes, i.e. iid uniform trits; binary bytes are uniform; scales
    are float16(exp(N(-4, 0.5))); activations float16(N(0, 1))."""

    def __init__(self, torch, tq, dev, seed):
        import numpy as np
        self.torch, self.dev = torch, dev
        self.gen = torch.Generator(device=dev)
        self.gen.manual_seed(seed)
        t = np.zeros((81, 128), dtype=np.int8)  # row i: the i-th 4-trit tuple, then zeros
        t[:, :4] = [[a, b, c, d] for a in (-1, 0, 1) for b in (-1, 0, 1)
                    for c in (-1, 0, 1) for d in (-1, 0, 1)]
        self.lut = torch.from_numpy(np.ascontiguousarray(tq.tq_pack(t, tq.TQ_TERNARY)[:, 0])).to(dev)

    def codes(self, N, K, variant):
        torch = self.torch
        nbytes = N * K // (8 if variant else 4)
        out = torch.empty(N, nbytes // N, dtype=torch.uint8, device=self.dev)
        flat = out.view(-1)
        chunk = 1 << 26
        for i in range(0, nbytes, chunk):
            n = min(chunk, nbytes - i)
            if variant:
                flat[i:i + n] = torch.randint(0, 256, (n,), device=self.dev, generator=self.gen,
                                              dtype=torch.int32).to(torch.uint8)
            else:
                flat[i:i + n] = self.lut[torch.randint(0, 81, (n,), device=self.dev,
                                                       generator=self.gen)]
        return out

    def scales(self, N, K):
        torch = self.torch
        g = torch.randn(N, K // 128, device=self.dev, generator=self.gen)
        return torch.exp(g * 0.5 - 4.0).to(torch.float16)

    def act(self, M, K):
        return self.torch.randn(M, K, device=self.dev, generator=self.gen).to(self.torch.float16)


def per_launch_ms(torch, stream, launch, n, warm=10):
    """Average duration of `launch(i)` over n calls, each bracketed by its own
    pair of HIP events on `stream` (so host gaps between calls are excluded)."""
    for i in range(warm):
        launch(i)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(n)]
    for i in range(n):
        ev[i][0].record(stream)
        launch(i)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    return sum(a.elapsed_time(b) for a, b in ev) / n


def back_to_back_ms(torch, stream, launch, n, warm=10):
    """Average time per call of n back-to-back calls between two events."""
    for i in range(warm):
        launch(i)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for i in range(n):
        launch(i)
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / n


def graph_ms(torch, launch, n, replays=5):
    """Average time per call of n calls captured in one HIP graph and replayed
    (no host cost per call: for launches shorter than a Python call)."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for i in range(3):
            launch(i)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(n):
            launch(i)
    g.replay()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(replays):
        g.replay()
    b.record()
    torch.cuda.synchronize()
    del g
    return a.elapsed_time(b) / (n * replays)


def stack_sweep(torch, tq, gen, stream):
    """Configs' whole-stack decode sweep: 64 layers, ~24.83B packed ternary
    weights (6.60 GB), each read once per token.  Input-shared projections are
    fused (gate;up, q;k;v, lin_qkv;lin_z): 4 GEMV launches per layer."""
    from binary_g128_bit_amd import synth
    launches = []   # (codes, scales, x, y)
    total = 0
    for mats in synth.stack_layers():
        d = {name: (N, K) for name, N, K in mats}
        if "q" in d:
            groups = [["q", "k", "v"], ["o"], ["gate", "up"], ["down"]]
        else:
            groups = [["lin_qkv", "lin_z"], ["lin_out"], ["gate", "up"], ["down"]]
        for g in groups:
            N = sum(d[n][0] for n in g)
            K = d[g[0]][1]
            c, s = gen.codes(N, K, 0), gen.scales(N, K)
            x = gen.act(1, K)[0]
            y = torch.empty(N, dtype=torch.float32, device=gen.dev)
            launches.append((c, s, x, y))
            total += packed_bytes(N, K)

    def token():
        for c, s, x, y in launches:
            tq.tq_gemv(c, s, x, y)

    for _ in range(3):
        token()
    torch.cuda.synchronize()
    T = 20
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(T):
        token()
    b.record(stream)
    torch.cuda.synchronize()
    eager_ms = a.elapsed_time(b) / T
    ref = launches[-1][3].clone()

    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        token()          # warm the side stream before capture
    stream.wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        token()
    for _ in range(3):
        graph.replay()
    torch.cuda.synchronize()
    graph_ok = bool(torch.equal(launches[-1][3], ref))
    a.record(stream)
    for _ in range(T):
        graph.replay()
    b.record(stream)
    torch.cuda.synchronize()
    graph_ms = a.elapsed_time(b) / T
    graph_ok = graph_ok and bool(torch.equal(launches[-1][3], ref))
    kernel_ms = sum(per_launch_ms(torch, stream, lambda i, L=L: tq.tq_gemv(*L), 5, warm=2)
                    for L in launches)
    del graph
    return {
        "workload": "64-layer batch-1 ternary decode sweep, 24.83B weights, each read once "
                    "per token; 256 GEMV launches per token (input-shared projections fused)",
        "bytes_per_token": total,
        "launches_per_token": len(launches),
        "ms_per_token_eager": round(eager_ms, 4),
        "ms_per_token_graph": round(graph_ms, 4),
        "ms_per_token_kernels_only": round(kernel_ms, 4),
        "tok_s_eager": round(1e3 / eager_ms, 1),
        "tok_s_graph": round(1e3 / graph_ms, 1),
        "gbs_graph": round(total / graph_ms / 1e6, 1),
        "pct_of_hbm_peak_graph": round(100 * total / graph_ms / 1e6 / PEAK_HBM_GBS, 2),
        "graph_replay_matches_eager": graph_ok,
    }


def gemm_widths(torch, tq, gen, stream, bufs, slots):
    """Small-batch GEMM (speculative verify / prefill widths) on gate
    (17408 x 5120, the first half of the fused buffers) and down, rotating;
    back-to-back launches between two events."""
    from binary_g128_bit_amd import synth
    out = {}
    for name, m, (N, K) in (("gate_17408x5120", 0, synth.GATE_UP), ("down_5120x17408", 1, synth.DOWN)):
        pool = [(c[:N], s[:N]) for c, s in (bufs[r][m] for r in range(slots))]
        X = gen.act(512, K)
        Y = torch.empty(512, N, dtype=torch.float32, device=gen.dev)
        # the configured widths and a two-row batch (the VALU kernel's width)
        for M in (2,) + tuple(synth.GEMM_WIDTHS):
            Xm, Ym = X[:M], Y[:M]
            ms = back_to_back_ms(torch, stream,
                                 lambda i: tq.tq_gemm(pool[i % len(pool)][0], pool[i % len(pool)][1],
                                                    Xm, Ym), 50)
            tf = 2.0 * M * N * K / (ms * 1e-3) / 1e12
            gbs = packed_bytes(N, K) / (ms * 1e-3) / 1e9
            out["%s_M%d" % (name, M)] = {
                "us": round(ms * 1e3, 2), "weight_gbs": round(gbs, 1), "tflops": round(tf, 1),
                "frac_hbm": round(gbs / PEAK_HBM_GBS, 4),
                "frac_f16_mfma": round(tf / PEAK_F16_TFLOPS, 4)}
    return out


def binary_and_lm_head(torch, tq, gen, stream):
    from binary_g128_bit_amd import synth
    out = {}
    # 1-bit variant on the MLP shapes: [gate;up] fused and down, rotating >= 1 GiB
    for name, (N, K) in (("bin_gate_up_34816x5120", (2 * synth.GATE_UP[0], synth.GATE_UP[1])),
                         ("bin_down_5120x17408", synth.DOWN)):
        nb = packed_bytes(N, K, 1)
        copies = max(2, math.ceil((1 << 30) / nb))
        pool = [(gen.codes(N, K, 1), gen.scales(N, K)) for _ in range(copies)]
        x = gen.act(1, K)[0]
        y = torch.empty(N, dtype=torch.float32, device=gen.dev)
        ms = back_to_back_ms(torch, stream, lambda i: tq.tq_gemv(pool[i % copies][0], pool[i % copies][1],
                                                                 x, y, variant=tq.TQ_BINARY), 100)
        out[name] = {"us": round(ms * 1e3, 2), "gbs": round(nb / ms / 1e6, 1),
                     "frac_hbm": round(nb / ms / 1e6 / PEAK_HBM_GBS, 4)}
        del pool
    # LM head 5120 -> 248320, batch 1 (GEMV) and 8 (GEMM); 3 copies > last-level cache
    N, K = synth.LM_HEAD
    nb = packed_bytes(N, K)
    pool = [(gen.codes(N, K, 0), gen.scales(N, K)) for _ in range(3)]
    X = gen.act(8, K)
    Y = torch.empty(8, N, dtype=torch.float32, device=gen.dev)
    ms1 = back_to_back_ms(torch, stream, lambda i: tq.tq_gemv(pool[i % 3][0], pool[i % 3][1], X[0], Y[0]), 30)
    ms8 = back_to_back_ms(torch, stream, lambda i: tq.tq_gemm(pool[i % 3][0], pool[i % 3][1], X, Y), 30)
    out["lm_head_248320x5120_M1"] = {"us": round(ms1 * 1e3, 2), "gbs": round(nb / ms1 / 1e6, 1),
                                     "frac_hbm": round(nb / ms1 / 1e6 / PEAK_HBM_GBS, 4)}
    out["lm_head_248320x5120_M8"] = {"us": round(ms8 * 1e3, 2), "gbs": round(nb / ms8 / 1e6, 1),
                                     "frac_hbm": round(nb / ms8 / 1e6 / PEAK_HBM_GBS, 4)}
    # token-embedding rows from the same 248320 x 5120 ternary table: ids
    # uniform over the vocabulary; bytes = code row + scale row read, FP16 row
    # written, per id; timed as graph replays (a one-id gather is shorter than
    # the Python call that launches it)
    row_bytes = K // 4 + 2 * (K // 128) + 2 * K
    for n_ids in (1, 512, 8192):
        ids = torch.randint(0, N, (n_ids,), device=gen.dev, generator=gen.gen, dtype=torch.int32)
        rows = torch.empty(n_ids, K, dtype=torch.float16, device=gen.dev)
        ms = graph_ms(torch, lambda i: tq.tq_embed(pool[i % 3][0], pool[i % 3][1], ids, rows), 60)
        out["embed_248320x5120_ids%d" % n_ids] = {
            "us": round(ms * 1e3, 2), "gbs": round(n_ids * row_bytes / ms / 1e6, 1),
            "frac_hbm": round(n_ids * row_bytes / ms / 1e6 / PEAK_HBM_GBS, 4)}
    return out


def ternary5(torch, tq, gen, stream):
    """Five-trit-per-byte storage on the MLP and head shapes, next to the 2-bit
    figures: back-to-back launches over >= 1 GiB of rotating copies (graph
    replays as well).  Codes: bytes uniform over the 243 valid values (the
    three-trit last byte of a group over 27), i.e. iid uniform trits."""
    from binary_g128_bit_amd import synth
    out = {}
    for name, (N, K) in (("gate_up_34816x5120", (2 * synth.GATE_UP[0], synth.GATE_UP[1])),
                         ("down_5120x17408", synth.DOWN), ("lm_head_248320x5120", synth.LM_HEAD)):
        nb = tq.tq_codes_bytes(N, K, tq.TQ_TERNARY5)
        G = K // 128
        alg = nb + 2 * N * G
        copies = max(2, math.ceil((1 << 30) / alg))
        pool = []
        for _ in range(copies):
            c = torch.zeros(N, nb // N, dtype=torch.uint8, device=gen.dev)
            body = c[:, :26 * G].view(N, G, 26)
            body[:, :, :25] = torch.randint(0, 243, (N, G, 25), device=gen.dev, generator=gen.gen,
                                            dtype=torch.int32).to(torch.uint8)
            body[:, :, 25] = torch.randint(0, 27, (N, G), device=gen.dev, generator=gen.gen,
                                           dtype=torch.int32).to(torch.uint8)
            pool.append((c, gen.scales(N, K)))
        x = gen.act(1, K)[0]
        y = torch.empty(N, dtype=torch.float32, device=gen.dev)

        def launch(i):
            return tq.tq_gemv(pool[i % copies][0], pool[i % copies][1], x, y, variant=tq.TQ_TERNARY5)

        ms = back_to_back_ms(torch, stream, launch, 100 if N < 100000 else 30)
        msg = graph_ms(torch, launch, 4 * copies)
        out[name] = {"us": round(ms * 1e3, 2), "us_graph": round(msg * 1e3, 2),
                     "gbs": round(alg / ms / 1e6, 1), "frac_hbm": round(alg / ms / 1e6 / PEAK_HBM_GBS, 4),
                     "gweights_s": round(N * K / ms / 1e6, 1), "bytes": alg}
        del pool
        torch.cuda.empty_cache()
    return out


def affine2(torch, tq, gen, stream):
    """Affine 2-bit levels (scale and bias per group) on the MLP and head
    shapes: back-to-back launches over >= 1 GiB of rotating copies (graph
    replays as well).  Codes are uniform bytes (iid uniform levels)."""
    from binary_g128_bit_amd import synth
    out = {}
    for name, (N, K) in (("gate_up_34816x5120", (2 * synth.GATE_UP[0], synth.GATE_UP[1])),
                         ("down_5120x17408", synth.DOWN), ("lm_head_248320x5120", synth.LM_HEAD)):
        alg = N * K // 4 + 4 * N * (K // 128)
        copies = max(2, math.ceil((1 << 30) / alg))
        pool = []
        for _ in range(copies):
            c = torch.randint(0, 256, (N, K // 4), device=gen.dev, generator=gen.gen,
                              dtype=torch.int32).to(torch.uint8)
            pool.append((c, gen.scales(N, K), -gen.scales(N, K)))
        x = gen.act(1, K)[0]
        y = torch.empty(N, dtype=torch.float32, device=gen.dev)

        def launch(i):
            c, s, b = pool[i % copies]
            return tq.tq_gemv_affine(c, s, b, x, y)

        ms = back_to_back_ms(torch, stream, launch, 100 if N < 100000 else 30)
        msg = graph_ms(torch, launch, 4 * copies)
        out[name] = {"us": round(ms * 1e3, 2), "us_graph": round(msg * 1e3, 2),
                     "gbs": round(alg / ms / 1e6, 1), "frac_hbm": round(alg / ms / 1e6 / PEAK_HBM_GBS, 4),
                     "gweights_s": round(N * K / ms / 1e6, 1), "bytes": alg}
        del pool
        torch.cuda.empty_cache()
    return out


def kv_attention(torch, tq, gen, stream):
    """4-bit KV cache: decode attention of one token over T cached tokens at
    the full-attention shape (4 KV heads, 24 query heads, head_dim 256),
    graph-replayed; bytes = T * 4 heads * 288 (K and V codes 128 + 128, scales
    16 + 16).  Rotating copies of the cache keep it out of the last-level
    cache.  Also the append of 1 and 512 new tokens."""
    out = {}
    n_kv, n_q = 4, 24
    for T in (4096, 32768, 102400, 262144):
        per = n_kv * 288
        copies = max(2, math.ceil((1 << 30) / (T * per)))
        caches = []
        for _ in range(copies):
            parts = []
            for part in range(4):
                nb = tq.tq_kv_bytes(n_kv, T, part)
                a = torch.randint(0, 256, (nb,), device=gen.dev, generator=gen.gen,
                                  dtype=torch.int32).to(torch.uint8)
                if part in (tq.TQ_KV_K_SCALES, tq.TQ_KV_V_SCALES):
                    # finite positive scales: FP16 exponent fields 5..13
                    h = a.view(torch.int16)
                    h.copy_(torch.randint(0x1400, 0x3800, (nb // 2,), device=gen.dev,
                                          generator=gen.gen, dtype=torch.int32).to(torch.int16))
                parts.append(a)
            caches.append(parts)
        q = gen.act(n_q, 256)
        ws = torch.empty(tq.tq_attn_workspace_bytes(T, n_q, n_kv) // 4, dtype=torch.float32,
                         device=gen.dev)
        o = torch.empty(n_q, 256, dtype=torch.float32, device=gen.dev)

        def launch(i):
            kc, ks, vc, vs = caches[i % copies]
            tq.tq_attn_decode(q, kc, ks.view(torch.int16), vc, vs.view(torch.int16), T, n_kv, T, ws, o)

        ms = graph_ms(torch, launch, 4 * copies)
        nbytes = T * per
        out["T%d" % T] = {"us": round(ms * 1e3, 2), "gbs": round(nbytes / ms / 1e6, 1),
                          "frac_hbm": round(nbytes / ms / 1e6 / PEAK_HBM_GBS, 4), "bytes": nbytes,
                          "us_16_layers": round(16 * ms * 1e3, 1)}
        del caches
        torch.cuda.empty_cache()
    TC = 4096
    parts = [torch.zeros(tq.tq_kv_bytes(n_kv, TC, p), dtype=torch.uint8, device=gen.dev) for p in range(4)]
    for n_tok in (1, 512):
        k = gen.act(n_tok * n_kv, 256).view(n_tok, n_kv, 256)
        v = gen.act(n_tok * n_kv, 256).view(n_tok, n_kv, 256)
        ms = graph_ms(torch, lambda i: tq.tq_kv_append(k, v, (i * n_tok) % (TC - n_tok), n_kv, TC,
                                                       parts[0], parts[1].view(torch.int16), parts[2],
                                                       parts[3].view(torch.int16)), 32)
        out["append_%d_tokens" % n_tok] = {"us": round(ms * 1e3, 2)}
    return out


def copy_calibration():
    import torch
    dev = torch.device("cuda:0")
    a = torch.empty(COPY_BYTES, dtype=torch.uint8, device=dev)
    b = torch.empty_like(a)
    a.fill_(1)
    torch.cuda.synchronize()
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": COPY_BYTES, "launches": 5}), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py runs on one GPU only: this build has no multi-GPU path "
              "(got --gpus %d)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return
    if args.only_step:
        args.no_cpu = args.no_extras = True

    import numpy as np
    import torch

    import binary_g128_bit_amd as tq
    from binary_g128_bit_amd import synth

    tq.lib()  # raises if the library is not built
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()

    # ---- synthetic inputs: gate, up, down (seeds 2001..2003), packed on the host
    host = []
    for i, (N, K) in enumerate((synth.GATE_UP, synth.GATE_UP, synth.DOWN)):
        t, s, X = synth.problem(synth.seed_for(2, i + 1), N, K, 1)
        host.append((tq.tq_pack(t), s, X, N, K))
        del t
    (cg, sg, xg, Ng, Kg), (cu, su, _, Nu, _), (cd, sd, xd, Nd, Kd) = host
    # gate and up share x: one fused matrix [gate; up]
    fused = [(np.concatenate([cg, cu]), np.concatenate([sg, su]), xg, Ng + Nu, Kg),
             (cd, sd, xd, Nd, Kd)]
    dev_base = [(torch.from_numpy(c).to(dev), torch.from_numpy(s).to(dev),
                 torch.from_numpy(x[0]).to(dev), N) for c, s, x, N, K in fused]
    step_bytes = sum(packed_bytes(N, K) for _, _, _, N, K in fused)
    slots = max(2, math.ceil(args.rotate_gib * (1 << 30) / step_bytes))
    bufs = []  # bufs[slot][matrix] = (codes, scales)
    for r in range(slots):
        bufs.append([(c.clone(), s.clone()) for c, s, _, _ in dev_base])
    xs = [x for _, _, x, _ in dev_base]
    ys = [torch.empty(N, dtype=torch.float32, device=dev) for _, _, _, N in dev_base]

    def step(slot):
        for m in range(2):
            c, s = bufs[slot][m]
            tq.tq_gemv(c, s, xs[m], ys[m])

    # ---- timed region: K steps over rotating buffers
    for w in range(args.warmup):
        step(w % slots)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for k in range(args.steps):
        step(k % slots)
    e1.record(stream)
    torch.cuda.synchronize()
    ms_per_step = e0.elapsed_time(e1) / args.steps
    gbs = step_bytes / (ms_per_step * 1e-3) / 1e9

    # ---- dominant kernel: the fused 34816x5120 GEMV, each launch timed alone
    launches = max(200, args.steps)

    def gemv_launch(m, pool):
        return lambda i: tq.tq_gemv(pool[i % len(pool)][0], pool[i % len(pool)][1], xs[m],
                                    ys[m][:pool[0][1].shape[0]])

    gu_pool = [bufs[r][0] for r in range(slots)]
    gu_ms = per_launch_ms(torch, stream, gemv_launch(0, gu_pool), launches)
    down_ms = back_to_back_ms(torch, stream, gemv_launch(1, [bufs[r][1] for r in range(slots)]), launches)
    # context: gate alone (17408 x 5120, the unfused per-matrix launch)
    half = [(c[: c.shape[0] // 2], s[: s.shape[0] // 2]) for c, s in gu_pool]
    gate_ms = back_to_back_ms(torch, stream, gemv_launch(0, half), launches)
    gu_b2b_ms = back_to_back_ms(torch, stream, gemv_launch(0, gu_pool), launches)
    # the same launches replayed from a HIP graph (no Python cost per launch)
    graph_us = {"gate_up_34816x5120": graph_ms(torch, gemv_launch(0, gu_pool), 4 * slots) * 1e3,
                "down_5120x17408": graph_ms(torch, gemv_launch(1, [bufs[r][1] for r in range(slots)]),
                                            4 * slots) * 1e3,
                "gate_17408x5120_unfused": graph_ms(torch, gemv_launch(0, half), 4 * slots) * 1e3}
    gu_bytes = packed_bytes(Ng + Nu, Kg)
    # average launch duration: back-to-back launches between two events on the
    # kernel's stream (per-launch event pairs add the events' own cost)
    achieved = gu_bytes / (gu_b2b_ms * 1e-3) / 1e9
    src = os.path.join(ROOT, "binary_g128_bit_amd", "csrc", "tq_gemv.hip")
    traffic = read_traffic("gemv_tern_34816x5120", source_hash(src))

    line = {
        "metric": "packed-weight GB/s and % of HBM peak, batch-1 ternary GEMV; equiv tokens/s",
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": "batch-1 ternary g128 decode GEMV, one MLP block per step: "
                        "[gate;up] 5120->2x17408 as one launch, down 17408->5120; "
                        "fp16 activations, fp32 accumulate",
            "bytes_per_step": step_bytes,
            "rotation_slots": slots,
            "rotation_bytes": slots * step_bytes,
        },
        "pct_of_hbm_peak": round(100 * gbs / PEAK_HBM_GBS, 2),
        "equiv_tok_s": round(gbs * 1e9 / STACK_BYTES, 1),
        "per_launch_us": {"gate_up_34816x5120": round(gu_b2b_ms * 1e3, 3),
                          "gate_up_34816x5120_event_pairs": round(gu_ms * 1e3, 3),
                          "down_5120x17408": round(down_ms * 1e3, 3),
                          "gate_17408x5120_unfused": round(gate_ms * 1e3, 3)},
        "per_launch_us_graph": {k: round(v, 3) for k, v in graph_us.items()},
        "per_launch_gbs": {"gate_up_34816x5120": round(achieved, 1),
                           "down_5120x17408": round(packed_bytes(Nd, Kd) / down_ms / 1e6, 1),
                           "gate_17408x5120_unfused": round(packed_bytes(Ng, Kg) / gate_ms / 1e6, 1)},
        "roofline": {
            "bound": "hbm",
            "kernel": "gemv_xreg_kernel<0,16,5,8,false,true> (ternary, pipelined) on [gate;up] 34816x5120",
            "achieved": round(achieved, 2),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBS, 4),
            "traffic": traffic,
            "algorithmic_bytes_per_launch": gu_bytes,
        },
        "cpu_baseline": None if args.no_cpu else cpu_baseline(host, args.cpu_seconds),
    }
    if not args.no_extras:
        gen = Dev(torch, tq, dev, 12345)
        line["gemm"] = gemm_widths(torch, tq, gen, stream, bufs, slots)
        line["binary_and_lm_head"] = binary_and_lm_head(torch, tq, gen, stream)
        line["ternary5"] = ternary5(torch, tq, gen, stream)
        line["affine2"] = affine2(torch, tq, gen, stream)
        line["kv4_attention"] = kv_attention(torch, tq, gen, stream)
        del bufs
        torch.cuda.empty_cache()
        line["stack_sweep"] = stack_sweep(torch, tq, gen, stream)
        line["stack_sweep"]["equiv_tok_s_note"] = (
            "tok_s_graph is the whole stack's GEMVs per second; equiv_tok_s above "
            "scales the MLP step's GB/s to the stack's bytes")
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
