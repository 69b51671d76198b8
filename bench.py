#!/usr/bin/env python3
"""Batch-1 ternary g128 decode GEMV on the 27B-like MLP shapes, one MI355X.

A step is one token's pass over one MLP block of packed ternary weights:
gate 5120->17408, up 5120->17408 and down 17408->5120.  gate and up read the
same activation, so they are stored as one 34816 x 5120 matrix (rows of gate,
then rows of up) and run as one GEMV launch; down is a second launch.  Both go
through the C ABI.  Weights rotate over >= 1 GiB of distinct device buffers so
that no step reads from the 256 MB last-level cache what the previous one left
there.  Inputs are resident in HBM before the timed region starts, and the K
timed steps are enqueued behind a spin kernel, so that the events around them
time their GPU work back to back rather than the host's launch latency.

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
GEMV_KERNEL_NAME = ("gemv_xreg_kernel<0,16,5,8,false,true,0> (ternary, pipelined) "
                    "on [gate;up] 34816x5120")


def log(msg):
    """Progress on stderr (the JSON line alone goes to stdout)."""
    print("[bench %.1fs] %s" % (time.perf_counter() - _T0, msg), file=sys.stderr, flush=True)


_T0 = time.perf_counter()


def packed_bytes(N, K, variant=0):
    return N * K // (8 if variant else 4) + 2 * N * K // 128


def parse():
    p = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=300)
    p.add_argument("--warmup", type=int, default=100,
                   help="untimed steps first (see --warmup-ms)")
    p.add_argument("--warmup-ms", type=float, default=300.0,
                   help="the warm-up runs at least this long (wall clock) even past --warmup steps")
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
    p.add_argument("--only-gemm", action="store_true",
                   help="run only the GEMM widths 4, 8, 16 and 64 on both MLP shapes, 20 launches each "
                        "(counter runs)")
    p.add_argument("--trace-summary", metavar="CSV",
                   help="summarise a rocprofv3 kernel_trace.csv of this script's default run and exit")
    p.add_argument("--pmc-summary", metavar="CSV", nargs="+",
                   help="summarise rocprofv3 counter_collection.csv files (median per kernel and grid) "
                        "and exit")
    p.add_argument("--timed-steps-only", action="store_true",
                   help="run the warm-up and the timed steps only (the fused [gate;up] and down launches "
                        "and nothing else, for counter passes), print the step time and exit")
    p.add_argument("--traffic-json", metavar="CSV", nargs=4,
                   help="write the fused GEMV's HBM traffic summary from four rocprofv3 counter files: "
                        "FETCH_SIZE and WRITE_SIZE of `--only-step`, then of `--copy-calibration`; "
                        "print it as JSON and exit")
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


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_rate(oracle, codes, s, X, K, threads, seconds, min_rows=16):
    """Packed-weight GB/s of the oracle on leading rows of one matrix: a short
    probe sizes the sample to about `seconds`, then the sample is timed.
    Returns (gbs, rows, elapsed_s)."""
    n = min(codes.shape[0], min_rows)
    t0 = time.perf_counter()
    oracle.gemm(codes[:n], s[:n], X, n, K, threads=threads)
    per_row = max((time.perf_counter() - t0) / n, 1e-9)
    n = int(min(codes.shape[0], max(min_rows, seconds / per_row)))
    t0 = time.perf_counter()
    oracle.gemm(codes[:n], s[:n], X, n, K, threads=threads)
    dt = time.perf_counter() - t0
    return packed_bytes(n, K) / dt / 1e9, n, dt


def cpu_baseline(mats, seconds, c1):
    """The oracle, as it stands, on the GPU machine's host cores.  `value`: whole
    passes over the step's gate, up and down (all the cores this process may
    use), repeated for about `seconds`.  Beside it: a single-thread run of the
    same matrices and per-config rates on bounded row samples (each config's
    own activation width M; the LM head's rows have the gate's K = 5120, so
    its per-row cost is sampled on gate rows).  Rates are packed-weight GB/s
    over the rows processed, comparable with the GPU figures."""
    import numpy as np
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
    out = {"value": round(done_bytes / dt / 1e9, 4), "unit": "GB/s", "cores": threads,
           "kind": "oracle", "cpu_model": cpu_model(),
           "sample": "fp64 oracle GEMV, batch 1: %s, %.1f s" % (what, dt)}
    # single thread, same matrices, bounded sample
    st = [_oracle_rate(oracle, c, sc, xx, KK, 1, seconds / 6.0) for c, sc, xx, NN, KK in mats]
    out["single_thread"] = {"value": round(sum(r[0] * r[2] for r in st) / sum(r[2] for r in st), 4),
                            "unit": "GB/s", "cores": 1,
                            "sample": "rows %s of gate, up, down" % [r[1] for r in st]}
    # per config: (name, codes, scales, K, M); activations N(0, 1) fp16 of width M
    g = np.random.default_rng(2024)
    (cg, sg, _, _, Kg), _, (cd, sd, _, _, Kd) = mats
    c1_codes, c1_s, c1_K = c1
    confs = [("C1_1024x1024_M1", c1_codes, c1_s, c1_K, 1),
             ("C2a_gate_17408x5120_M1", cg, sg, Kg, 1),
             ("C2b_down_5120x17408_M1", cd, sd, Kd, 1),
             ("C5_lm_head_248320x5120_M1_rows_of_gate", cg, sg, Kg, 1),
             ("C5_lm_head_248320x5120_M8_rows_of_gate", cg, sg, Kg, 8)]
    for M in (4, 16, 64, 512):
        confs.append(("C4_gate_17408x5120_M%d" % M, cg, sg, Kg, M))
        confs.append(("C4_down_5120x17408_M%d" % M, cd, sd, Kd, M))
    full_rows = {"C5_lm_head_248320x5120_M1_rows_of_gate": 248320,
                 "C5_lm_head_248320x5120_M8_rows_of_gate": 248320}
    per = {}
    budget = seconds / (2.0 * len(confs))
    for name, c, sc, KK, M in confs:
        X = g.standard_normal((M, KK), dtype=np.float32).astype(np.float16)
        rows_full = full_rows.get(name, c.shape[0])
        entry = {}
        for label, th in (("all_cores", threads), ("single_thread", 1)):
            gbs, n, dt = _oracle_rate(oracle, c, sc, X, KK, th, budget, min_rows=4)
            entry[label + "_gbs"] = round(gbs, 4)
            entry[label + "_full_matrix_ms"] = round(dt / n * rows_full * 1e3, 2)
            entry[label + "_rows_timed"] = n
        per[name] = entry
    out["per_config"] = per
    return out


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


def back_to_back_ms(torch, stream, launch, n, warm=10, batches=20):
    """Time per call of back-to-back calls: `batches` batches of n calls, each
    batch between two events on `stream`; returns the median batch's average.
    The call index keeps counting across batches (rotating buffers keep
    rotating)."""
    for i in range(warm):
        launch(i)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(batches)]
    i = 0
    for a, b in ev:
        a.record(stream)
        for _ in range(n):
            launch(i)
            i += 1
        b.record(stream)
    torch.cuda.synchronize()
    per = sorted(a.elapsed_time(b) / n for a, b in ev)
    return per[len(per) // 2]


def spin_cycles_per_ms(torch, stream, cycles=200000):
    """Cycles of torch.cuda._sleep per millisecond on this GPU, timed with
    events (the spin counts the shader clock, whose rate the events measure)."""
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda._sleep(cycles)
    e0.record(stream)
    torch.cuda._sleep(cycles)
    e1.record(stream)
    torch.cuda.synchronize()
    return cycles / max(e0.elapsed_time(e1), 1e-3)


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
    replay_ms = a.elapsed_time(b) / T
    graph_ok = graph_ok and bool(torch.equal(launches[-1][3], ref))
    # per shape: that shape's launches of the token replayed from their own graph
    shapes = {}
    for L in launches:
        shapes.setdefault((L[3].shape[0], L[2].shape[0]), []).append(L)
    per_shape = {}
    for (N, K), Ls in shapes.items():
        us = graph_ms(torch, lambda i, Ls=Ls: tq.tq_gemv(*Ls[i % len(Ls)]), len(Ls)) * 1e3
        nb = packed_bytes(N, K)
        per_shape["%dx%d" % (N, K)] = {"launches_per_token": len(Ls), "us_graph": round(us, 3),
                                       "gbs": round(nb / us / 1e3, 1),
                                       "frac_hbm": round(nb / us / 1e3 / PEAK_HBM_GBS, 4)}
    kernel_ms = sum(v["launches_per_token"] * v["us_graph"] for v in per_shape.values()) / 1e3
    del graph
    return {
        "workload": "64-layer batch-1 ternary decode sweep, 24.83B weights, each read once "
                    "per token; 256 GEMV launches per token (input-shared projections fused)",
        "bytes_per_token": total,
        "launches_per_token": len(launches),
        "ms_per_token_eager": round(eager_ms, 4),
        "ms_per_token_graph": round(replay_ms, 4),
        "ms_per_token_sum_of_shapes": round(kernel_ms, 4),
        "per_shape": per_shape,
        "tok_s_eager": round(1e3 / eager_ms, 1),
        "tok_s_graph": round(1e3 / replay_ms, 1),
        "gbs_graph": round(total / replay_ms / 1e6, 1),
        "pct_of_hbm_peak_graph": round(100 * total / replay_ms / 1e6 / PEAK_HBM_GBS, 2),
        "graph_replay_matches_eager": graph_ok,
    }


def gemm_widths(torch, tq, gen, stream, bufs, slots, widths=None, launches=50):
    """Small-batch GEMM (speculative verify / prefill widths) on gate
    (17408 x 5120, the first half of the fused buffers) and down, rotating;
    back-to-back launches between two events.  Widths that take a K-split
    workspace get one allocated once, outside the timed launches."""
    from binary_g128_bit_amd import synth
    if widths is None:
        # the configured widths, a two-row batch (the VALU kernel's width) and
        # eight rows (the four-row kernel's two row sets)
        widths = tuple(sorted({2, 8} | set(synth.GEMM_WIDTHS)))
    out = {}
    for name, m, (N, K) in (("gate_17408x5120", 0, synth.GATE_UP), ("down_5120x17408", 1, synth.DOWN)):
        pool = [(c[:N], s[:N]) for c, s in (bufs[r][m] for r in range(slots))]
        X = gen.act(512, K)
        Y = torch.empty(512, N, dtype=torch.float32, device=gen.dev)
        for M in widths:
            Xm, Ym = X[:M], Y[:M]
            need = tq.tq_gemm_workspace_bytes(M, N, K)
            ws = torch.empty(max(need, 16), dtype=torch.uint8, device=gen.dev)
            ms = back_to_back_ms(torch, stream,
                                 lambda i: tq.tq_gemm(pool[i % len(pool)][0], pool[i % len(pool)][1],
                                                    Xm, Ym, workspace=ws), launches)
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
    del pool
    torch.cuda.empty_cache()
    # the 1-bit head, three copies
    nbb = packed_bytes(N, K, 1)
    bpool = [(gen.codes(N, K, 1), gen.scales(N, K)) for _ in range(3)]
    msb = back_to_back_ms(torch, stream, lambda i: tq.tq_gemv(bpool[i % 3][0], bpool[i % 3][1], X[0], Y[0],
                                                              variant=tq.TQ_BINARY), 30)
    out["bin_lm_head_248320x5120_M1"] = {"us": round(msb * 1e3, 2), "gbs": round(nbb / msb / 1e6, 1),
                                         "frac_hbm": round(nbb / msb / 1e6 / PEAK_HBM_GBS, 4)}
    del bpool
    torch.cuda.empty_cache()
    pool = [(gen.codes(N, K, 0), gen.scales(N, K)) for _ in range(3)]
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


def stream_ceiling(torch, tq, dev, stream):
    """A plain streaming read (tq_stream_read) of the dominant launches' byte
    counts, over windows rotating through 1.25 GiB, at 1, 2 and 4 workgroups
    per CU; the best of the three per size.  The ceiling a bandwidth-bound
    launch of that size is measured against."""
    total = 5 << 28
    buf = torch.empty(total, dtype=torch.uint8, device=dev)
    buf.fill_(0x5A)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    out = {}
    for nbytes in (47349760, 23674880, 337715200):
        copies = total // nbytes
        views = [buf[i * nbytes:(i + 1) * nbytes] for i in range(copies)]
        best = None
        for bpc in (1, 2, 4):
            ms = back_to_back_ms(torch, stream,
                                 lambda i: tq.tq_stream_read(views[i % copies], sink, bpc),
                                 50 if nbytes < 100_000_000 else 20)
            if best is None or ms < best[0]:
                best = (ms, bpc)
        ms, bpc = best
        out["bytes_%d" % nbytes] = {"us": round(ms * 1e3, 3), "gbs": round(nbytes / ms / 1e6, 1),
                                    "frac_hbm": round(nbytes / ms / 1e6 / PEAK_HBM_GBS, 4),
                                    "blocks_per_cu": bpc}
    del buf
    torch.cuda.empty_cache()
    return out


def c1_problems():
    """The 1024 x 1024 GEMV inputs, ternary and binary, packed on the host."""
    import binary_g128_bit_amd as tq
    from binary_g128_bit_amd import synth
    out = {}
    for name, variant, cfg in (("ternary", tq.TQ_TERNARY, 1), ("binary", tq.TQ_BINARY, 5)):
        N, K = synth.C1
        t, s, X = synth.problem(synth.seed_for(cfg, 0), N, K, 1, variant)
        out[name] = (tq.tq_pack(t, variant), s, X, variant)
    return out


def c1_latency(torch, tq, dev, stream, probs):
    """Microseconds per 1024 x 1024 GEMV call (the whole matrix fits in L2):
    back-to-back calls through Python, and graph-replayed (kernel only)."""
    out = {}
    N, K = 1024, 1024
    for name, (codes, s, X, variant) in probs.items():
        cd, sd = torch.from_numpy(codes).to(dev), torch.from_numpy(s).to(dev)
        x = torch.from_numpy(X[0]).to(dev)
        y = torch.empty(N, dtype=torch.float32, device=dev)

        def launch(i):
            return tq.tq_gemv(cd, sd, x, y, variant=variant)

        out[name] = {"us_per_call": round(back_to_back_ms(torch, stream, launch, 50) * 1e3, 3),
                     "us_graph": round(graph_ms(torch, launch, 60) * 1e3, 3),
                     "bytes": packed_bytes(N, K, variant)}
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


def _csv_rows(path):
    import csv
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def _col(row, *names):
    for n in names:
        if n in row:
            return row[n]
    raise KeyError("none of %s in %s" % (names, sorted(row)))


def trace_summary(path, min_run=90):
    """Runs of consecutive dispatches in a rocprofv3 kernel trace of the
    default run, in dispatch order: one kernel repeated, or two kernels
    alternating (a K-split GEMM and its reduction, or decode attention's two
    launches), at least min_run times.  The
    first long run of the fused GEMV is the back-to-back [gate;up] phase that
    `roofline.achieved` times.  The first 10 dispatches of a run (its
    warm-up) are left out of the averages."""
    rows = _csv_rows(path)
    rows.sort(key=lambda r: int(_col(r, "Start_Timestamp")))

    def grid_of(r):
        for c in ("Grid_Size_X", "Grid_Size"):
            if c in r:
                return r[c]
        return ""

    # a run is keyed by kernel and grid: launches of one kernel at different
    # sizes (batch widths, context lengths) are separate runs
    names = [(_col(r, "Kernel_Name"), grid_of(r)) for r in rows]
    durs = [int(_col(r, "End_Timestamp")) - int(_col(r, "Start_Timestamp")) for r in rows]
    n = len(rows)

    def short(name):
        return name.replace("(anonymous namespace)::", "").split("(")[0].replace("void ", "")

    def line(tag, key, d):
        body = sorted(d[10:])
        print("| %s | `%s` | %d | %.3f | %.3f | %.3f | %s |" % (tag, short(key[0]), len(d), sum(body) / len(body) / 1e3,
                                                               body[len(body) // 2] / 1e3, body[0] / 1e3, key[1]))

    print("| first dispatch | kernel | dispatches | avg us | median us | min us | grid |")
    print("|---|---|---|---|---|---|---|")
    i = 0
    while i < n:
        j = i
        while j < n and names[j] == names[i]:
            j += 1
        if j - i >= min_run:
            line(str(i), names[i], durs[i:j])
            i = j
            continue
        j = i
        while j + 1 < n and names[j] == names[i] and names[j + 1] == names[i + 1] and names[i] != names[i + 1]:
            j += 2
        if (j - i) // 2 >= min_run:
            line(str(i), names[i], durs[i:j:2])
            line("%d (alternating)" % (i + 1), names[i + 1], durs[i + 1:j:2])
            i = j
            continue
        i += 1


def pmc_summary(paths):
    """Median counter value per (kernel, grid size) over the dispatches of
    rocprofv3 counter_collection.csv files.  A dispatch directly followed by
    a slice reduction is also keyed by that reduction's grid, which tells
    apart batch widths that share a kernel and grid."""
    import collections
    agg = collections.OrderedDict()
    for path in paths:
        rows = list(_csv_rows(path))
        kernels = {}
        for r in rows:
            name = _col(r, "Kernel_Name").replace("(anonymous namespace)::", "").split("(")[0]
            kernels[int(_col(r, "Dispatch_Id"))] = (name, _col(r, "Grid_Size", "Grid_Size_X"))
        for r in rows:
            d = int(_col(r, "Dispatch_Id"))
            name, grid = kernels[d]
            nxt = kernels.get(d + 1)
            then = nxt[1] if nxt and "reduce" in nxt[0] and "reduce" not in name else None
            key = (name, grid, then)
            agg.setdefault(key, collections.defaultdict(list))[_col(r, "Counter_Name")].append(
                float(_col(r, "Counter_Value")))
    for (name, grid, then), cs in agg.items():
        print("%s grid=%s%s" % (name, grid, " then-reduce-grid=%s" % then if then else ""))
        for cn, vs in sorted(cs.items()):
            vs.sort()
            print("    %-28s median %.6g  (n=%d)" % (cn, vs[len(vs) // 2], len(vs)))


TRAFFIC_KERNEL = "gemv_xreg_kernel<0, 16, 5, 8, false, true, 0>"   # the fused [gate;up] launch's template
TRAFFIC_GRID = "131072"


def traffic_json(step_fetch, step_write, cal_fetch, cal_write, skip=5):
    """HBM bytes per fused [gate;up] launch from rocprofv3 FETCH_SIZE and
    WRITE_SIZE (KiB per dispatch): the mean over the `--only-step` run's
    launches of the fused GEMV (its first `skip` left out), each counter
    scaled by bytes / KiB read for the 1 GiB calibration copy."""
    def values(path, pick):
        rows = [r for r in _csv_rows(path) if pick(r)]
        rows.sort(key=lambda r: int(_col(r, "Dispatch_Id")))
        return [float(_col(r, "Counter_Value")) for r in rows]

    def fused(r):
        return TRAFFIC_KERNEL in _col(r, "Kernel_Name") and _col(r, "Grid_Size", "Grid_Size_X") == TRAFFIC_GRID

    def copy(r):
        return "copyBuffer" in _col(r, "Kernel_Name")

    out = {"kernel": TRAFFIC_KERNEL + " on [gate;up] 34816x5120 ternary",
           "source_sha256_16": source_hash(os.path.join(ROOT, "binary_g128_bit_amd", "csrc", "tq_gemv.hip")),
           "commands": [
               "cd /tmp && TMPDIR=/tmp rocprofv3 --pmc {FETCH_SIZE|WRITE_SIZE} -d /tmp/step_<ctr> -o run "
               "--output-format csv -- python3 $REPO/bench.py --only-step --steps 20 --warmup 2",
               "cd /tmp && TMPDIR=/tmp rocprofv3 --pmc {FETCH_SIZE|WRITE_SIZE} -d /tmp/cal_<ctr> -o run "
               "--output-format csv -- python3 $REPO/bench.py --copy-calibration",
               "python3 $REPO/bench.py --traffic-json <step FETCH_SIZE csv> <step WRITE_SIZE csv> "
               "<calibration FETCH_SIZE csv> <calibration WRITE_SIZE csv>"]}
    cal = {}
    for name, path in (("fetch", cal_fetch), ("write", cal_write)):
        v = sorted(values(path, copy))
        kib = v[len(v) // 2]
        cal[name] = (COPY_BYTES / 1024.0) / kib
        out.setdefault("copy_calibration", {"bytes": COPY_BYTES})["%s_size_kib" % name] = kib
        out["copy_calibration"]["%s_scale" % name] = cal[name]
    # the unfused 17408-row gate of the per-launch timings runs the same
    # template and grid on half the rows: its dispatches count about half
    # the bytes, and are left out by that
    def fused_only(v):
        top = max(v)
        return [x for x in v if x >= 0.75 * top]
    f = fused_only(values(step_fetch, fused)[skip:])
    w = fused_only(values(step_write, fused)[skip:])
    out["dispatches"] = {"fetch": len(f), "write": len(w),
                         "note": "fused launches only (grid %s, counts within 0.75 of the largest: the unfused "
                                 "gate on the same template counts about half); the first %d of each pass left "
                                 "out" % (TRAFFIC_GRID, skip)}
    fk, wk = sum(f) / len(f), sum(w) / len(w)
    out["fetch_size_kib_per_launch"] = fk
    out["write_size_kib_per_launch"] = wk
    out["hbm_fetch_bytes_per_launch"] = round(fk * 1024 * cal["fetch"])
    out["hbm_write_bytes_per_launch"] = round(wk * 1024 * cal["write"])
    out["hbm_bytes_per_launch"] = out["hbm_fetch_bytes_per_launch"] + out["hbm_write_bytes_per_launch"]
    N, K = 34816, 5120
    codes, scales = N * K // 4, N * (K // 128) * 2
    out["algorithmic_bytes_per_launch"] = codes + scales + 2 * K + 4 * N
    out["note"] = "algorithmic = codes %d + scales %d + x %d + y %d" % (codes, scales, 2 * K, 4 * N)
    print(json.dumps(out, indent=1))


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py runs on one GPU only: this build has no multi-GPU path "
              "(got --gpus %d)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return
    if args.trace_summary:
        trace_summary(args.trace_summary)
        return
    if args.pmc_summary:
        pmc_summary(args.pmc_summary)
        return
    if args.traffic_json:
        traffic_json(*args.traffic_json)
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

    if args.only_gemm:
        gen = Dev(torch, tq, dev, 12345)
        print(json.dumps(gemm_widths(torch, tq, gen, stream, bufs, slots, widths=(4, 8, 16, 64), launches=20)))
        return

    log("inputs ready; warm-up")
    # ---- untimed warm-up: the W steps asked for, continued until at least
    # --warmup-ms of wall time has passed (the clocks settle only after some
    # tens of milliseconds of load, whatever W is)
    w = 0
    t0 = time.perf_counter()
    while w < args.warmup or (time.perf_counter() - t0) * 1e3 < args.warmup_ms:
        step(w % slots)
        w += 1
        if w % 256 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    warmup_ms = (time.perf_counter() - t0) * 1e3
    warmup_steps = w

    # ---- timed region: K steps over rotating buffers.  A short spin kernel
    # holds the stream while the host starts enqueueing the K steps (two
    # launches each from Python), so that the events time the GPU's work on
    # the steps back to back, not the host's first launches.  The host
    # enqueues a step faster than the GPU runs one, so a head start keeps it
    # ahead; the JSON reports both rates.  (A spin as long as the whole
    # enqueue, milliseconds on one CU with the rest idle, let the clocks
    # drop: 21.0 against 18.5 us per step over 300 steps.)
    cycles_per_ms = spin_cycles_per_ms(torch, stream)
    prime_ms = 0.6
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda._sleep(int(prime_ms * cycles_per_ms))
    t_enq = time.perf_counter()
    e0.record(stream)
    for k in range(args.steps):
        step(k % slots)
    e1.record(stream)
    enqueue_ms = (time.perf_counter() - t_enq) * 1e3
    torch.cuda.synchronize()
    ms_per_step = e0.elapsed_time(e1) / args.steps
    gbs = step_bytes / (ms_per_step * 1e-3) / 1e9

    log("timed step done: %.3f us/step" % (ms_per_step * 1e3))
    if args.timed_steps_only:
        print(json.dumps({"timed_steps_only": True, "steps": args.steps, "warmup_steps": warmup_steps,
                          "us_per_step": round(ms_per_step * 1e3, 3), "gbs": round(gbs, 2)}), flush=True)
        return
    # ---- dominant kernel: the fused 34816x5120 GEMV
    launches = 100

    def gemv_launch(m, pool):
        return lambda i: tq.tq_gemv(pool[i % len(pool)][0], pool[i % len(pool)][1], xs[m],
                                    ys[m][:pool[0][1].shape[0]])

    gu_pool = [bufs[r][0] for r in range(slots)]
    down_pool = [bufs[r][1] for r in range(slots)]
    half = [(c[: c.shape[0] // 2], s[: s.shape[0] // 2]) for c, s in gu_pool]
    # average launch duration: back-to-back launches between two events on the
    # kernel's stream, median of 20 batches (per-launch event pairs add the
    # events' own cost and are printed for reference only)
    gu_b2b_ms = back_to_back_ms(torch, stream, gemv_launch(0, gu_pool), launches)
    down_ms = back_to_back_ms(torch, stream, gemv_launch(1, down_pool), launches)
    gate_ms = back_to_back_ms(torch, stream, gemv_launch(0, half), launches)
    gu_ms = per_launch_ms(torch, stream, gemv_launch(0, gu_pool), launches)
    # the same launches replayed from a HIP graph (no Python cost per launch)
    graph_us = {"gate_up_34816x5120": graph_ms(torch, gemv_launch(0, gu_pool), 4 * slots) * 1e3,
                "down_5120x17408": graph_ms(torch, gemv_launch(1, down_pool), 4 * slots) * 1e3,
                "gate_17408x5120_unfused": graph_ms(torch, gemv_launch(0, half), 4 * slots) * 1e3}
    gu_bytes = packed_bytes(Ng + Nu, Kg)
    achieved = gu_bytes / (gu_b2b_ms * 1e-3) / 1e9
    src = os.path.join(ROOT, "binary_g128_bit_amd", "csrc", "tq_gemv.hip")
    traffic = read_traffic("gemv_tern_34816x5120", source_hash(src))
    log("per-launch timings done")
    ceiling = stream_ceiling(torch, tq, dev, stream)
    log("stream ceiling done")
    c1_probs = c1_problems()
    c1 = c1_latency(torch, tq, dev, stream, c1_probs)
    c1_host = (c1_probs["ternary"][0], c1_probs["ternary"][1], 1024)

    line = {
        "metric": "packed-weight GB/s and % of HBM peak, batch-1 ternary GEMV; equiv tokens/s",
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_run": {"steps": warmup_steps, "ms": round(warmup_ms, 1)},
        "timed_region": {"steps": args.steps, "events": "on the launch stream around the K steps",
                         "queue_primed_ms": round(prime_ms, 3),
                         "host_us_per_step": round(enqueue_ms * 1e3 / args.steps, 3),
                         "gpu_us_per_step": round(ms_per_step * 1e3, 3),
                         "host_ahead": bool(enqueue_ms < prime_ms + ms_per_step * args.steps and
                                            enqueue_ms / args.steps < ms_per_step)},
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
        "timing": "per-launch figures: median of 20 event-timed batches of back-to-back launches",
        "per_launch_us": {"gate_up_34816x5120": round(gu_b2b_ms * 1e3, 3),
                          "gate_up_34816x5120_event_pairs": round(gu_ms * 1e3, 3),
                          "down_5120x17408": round(down_ms * 1e3, 3),
                          "gate_17408x5120_unfused": round(gate_ms * 1e3, 3)},
        "per_launch_us_graph": {k: round(v, 3) for k, v in graph_us.items()},
        "per_launch_gbs": {"gate_up_34816x5120": round(achieved, 1),
                           "down_5120x17408": round(packed_bytes(Nd, Kd) / down_ms / 1e6, 1),
                           "gate_17408x5120_unfused": round(packed_bytes(Ng, Kg) / gate_ms / 1e6, 1)},
        "stream_read_ceiling": ceiling,
        "frac_of_stream_ceiling": {
            "gate_up_34816x5120": round(ceiling["bytes_47349760"]["us"] / (gu_b2b_ms * 1e3), 4),
            "down_5120x17408": round(ceiling["bytes_23674880"]["us"] / (down_ms * 1e3), 4)},
        "c1_latency": c1,
        "roofline": {
            "bound": "hbm",
            "kernel": GEMV_KERNEL_NAME,
            "achieved": round(achieved, 2),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBS, 4),
            "traffic": traffic,
            "algorithmic_bytes_per_launch": gu_bytes,
        },
        "context": {
            "what": "the pages' whole-model single-batch decode through llama.cpp on other "
                    "machines (context only, not a target)",
            "source": "blog.devnsb.com, 'Ternary quantization: 27B in 7 GB', deploy size and "
                      "hardware section",
            "tok_s": {"H100": 98.0, "M5 Max": 44.0, "M5 Pro": 26.2},
        },
        "cpu_baseline": None if args.no_cpu else cpu_baseline(host, args.cpu_seconds, c1_host),
    }
    log("cpu baseline done" if not args.no_cpu else "cpu baseline skipped")
    if not args.no_extras:
        gen = Dev(torch, tq, dev, 12345)
        line["gemm"] = gemm_widths(torch, tq, gen, stream, bufs, slots)
        log("gemm widths done")
        line["binary_and_lm_head"] = binary_and_lm_head(torch, tq, gen, stream)
        log("binary and lm head done")
        line["ternary5"] = ternary5(torch, tq, gen, stream)
        line["affine2"] = affine2(torch, tq, gen, stream)
        log("ternary5 and affine2 done")
        line["kv4_attention"] = kv_attention(torch, tq, gen, stream)
        log("attention done")
        del bufs
        torch.cuda.empty_cache()
        line["stack_sweep"] = stack_sweep(torch, tq, gen, stream)
        log("stack sweep done")
        line["stack_sweep"]["equiv_tok_s_note"] = (
            "tok_s_graph is the whole stack's GEMVs per second; equiv_tok_s above "
            "scales the MLP step's GB/s to the stack's bytes")
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
