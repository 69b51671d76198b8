#!/usr/bin/env python3
"""Batch-1 ternary g128 decode GEMV on the 27B-like MLP shapes, one MI355X.

A step is one token's pass over one MLP block of packed ternary weights:
gate 5120->17408, up 5120->17408 and down 17408->5120.  gate and up read the
same activation, so they are stored as one 34816 x 5120 matrix (rows of gate,
then rows of up) and run as one GEMV launch; down is a second launch.  Both go
through the C ABI.  Weights rotate over >= 1 GiB of distinct device buffers so that no
step reads from the 256 MB last-level cache what the previous one left there.
Inputs are resident in HBM before the timed region starts.

Prints ONE JSON line: packed-weight GB/s (value), % of the 8 TB/s HBM peak,
equivalent tokens/s of the 6.60 GB 64-layer stack, the roofline object of the
dominant kernel (timed live with HIP events on its stream) and the oracle's
CPU baseline on a bounded sample of the same workload.
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

PEAK_HBM_GBS = 8000.0               # MI355X HBM3E, vendor figure
STACK_BYTES = 6_595_543_040         # packed bytes of the 64-layer 24.83B-weight stack
TERN_BYTES_PER_WEIGHT = 0.265625    # 2-bit slot + fp16 scale per 128


def packed_bytes(N, K):
    return N * K // 4 + 2 * N * K // 128


def parse():
    p = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=300)
    p.add_argument("--warmup", type=int, default=30)
    p.add_argument("--rotate-gib", type=float, default=1.0)
    p.add_argument("--cpu-seconds", type=float, default=10.0,
                   help="target duration of the oracle's CPU-baseline sample")
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU baseline")
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


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py runs on one GPU only: this build has no multi-GPU path "
              "(got --gpus %d)" % args.gpus, file=sys.stderr)
        sys.exit(2)

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

    # ---- dominant kernel: the fused 34816x5120 GEMV, timed alone on its stream
    def kernel_avg_ms(m, launches, views=None):
        pool = [bufs[r][m] for r in range(slots)] if views is None else views
        for i in range(20):
            c, s = pool[i % len(pool)]
            tq.tq_gemv(c, s, xs[m], ys[m][:s.shape[0]])
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for i in range(launches):
            c, s = pool[i % len(pool)]
            tq.tq_gemv(c, s, xs[m], ys[m][:s.shape[0]])
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / launches

    launches = max(200, args.steps)
    gu_ms = kernel_avg_ms(0, launches)
    down_ms = kernel_avg_ms(1, launches)
    # context: gate alone (17408 x 5120, the unfused per-matrix launch)
    half = [(c[: c.shape[0] // 2], s[: s.shape[0] // 2]) for c, s in (bufs[r][0] for r in range(slots))]
    gate_ms = kernel_avg_ms(0, launches, half)
    gu_bytes = packed_bytes(Ng + Nu, Kg)
    achieved = gu_bytes / (gu_ms * 1e-3) / 1e9
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
        "per_launch_us": {"gate_up_34816x5120": round(gu_ms * 1e3, 3),
                          "down_5120x17408": round(down_ms * 1e3, 3),
                          "gate_17408x5120_unfused": round(gate_ms * 1e3, 3)},
        "per_launch_gbs": {"gate_up_34816x5120": round(achieved, 1),
                           "down_5120x17408": round(packed_bytes(Nd, Kd) / down_ms / 1e6, 1),
                           "gate_17408x5120_unfused": round(packed_bytes(Ng, Kg) / gate_ms / 1e6, 1)},
        "roofline": {
            "bound": "hbm",
            "kernel": "gemv_kernel<0,8,5,1> on [gate;up] 34816x5120 ternary",
            "achieved": round(achieved, 2),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBS, 4),
            "traffic": traffic,
        },
        "cpu_baseline": None if args.no_cpu else cpu_baseline(host, args.cpu_seconds),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
