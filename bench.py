#!/usr/bin/env python3
"""ECF8 decode benchmark on one MI355X.

One step = one batched decode of a whole workload (default: the Llama-3-70B
transformer block, 7 FP8 E4M3 tensors, 855,638,016 elements) with every
input resident in HBM: the per-tensor decode-table kernel followed by the
persistent decode dispatch, into one reused output buffer.  The decoded
output is checked bit-exact against the original bytes before timing.

Prints ONE JSON line: value = decoded FP8 GB/s of the whole step; roofline =
algorithmic HBM bytes of the decode kernel (compressed bytes read + FP8 bytes
written) over its event-timed average duration; cpu_baseline = the plain C
oracle decoding a bounded sample on the host cores.
"""
from __future__ import annotations

import argparse
import concurrent.futures
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "ECF8 decoded GB/s on 1 MI355X, % of HBM roofline; bit-exact vs oracle"
WORKLOAD_TEXT = {
    "llama70b": "Llama-3-70B transformer block FP8 E4M3 (q,o 8192x8192; k,v 8192x1024; gate,up 8192x28672; "
                "down 28672x8192), alpha-stable alpha=1.9, per-tensor codebooks, one batched dispatch",
    "llama8b": "Llama-3-8B attention+MLP FP8 E4M3, alpha=1.8, per-tensor codebooks, one batched dispatch",
    "dit14b": "14B-DiT block FP8 E4M3 (hidden 5120), alpha=1.5 + 2% outliers, per-128x128 scaling, batched",
    "moe8": "MoE layer, 8 routed experts x (gate, up 7168x2048; down 2048x7168), per-expert codebooks, batched",
    "gauss1m": "single 1024x1024 N(0,0.02) FP8 E4M3 tensor",
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    """Hash of the decode kernel source with comments and blank lines removed."""
    import re
    p = os.path.join(ROOT, "lossless_entropy_coded_ecf8_amd", "csrc", "ecf8_decode.hip")
    text = re.sub(r"//[^\n]*", "", open(p).read())
    code = "\n".join(line.rstrip() for line in text.splitlines() if line.strip())
    return hashlib.sha256(code.encode()).hexdigest()[:16]


def load_traffic(workload: str, kernel_hash: str, launches_bytes: float):
    """HBM traffic per launch from committed rocprofv3 counter summaries, if they match this kernel."""
    p = os.path.join(ROOT, "profiles", "traffic_%s.json" % workload)
    if not os.path.exists(p):
        return None
    try:
        rec = json.load(open(p))
    except Exception:
        return None
    if rec.get("kernel_sha") != kernel_hash:
        return None
    return rec.get("traffic_bytes_per_launch")


def copy_ceiling(torch, d, gib: float = 1.0, reps: int = 5):
    """Event-timed plain streaming kernel (uint8 bitwise_not: reads and writes `gib` GiB each)."""
    n = int(gib * (1 << 30))
    a = torch.empty(n, dtype=torch.uint8, device=d).fill_(0x5A)
    b = torch.empty_like(a)
    torch.bitwise_not(a, out=b)
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(reps):
        torch.bitwise_not(a, out=b)
    e.record()
    torch.cuda.synchronize()
    ms = s.elapsed_time(e) / reps
    del a, b
    return 2.0 * n / (ms * 1e-3) / 1e9


def cpu_baseline(encs_host, seconds: float):
    """Time the C oracle decoding whole blocks of the largest tensor, all host cores."""
    import numpy as np
    import oracle
    enc = max(encs_host, key=lambda e: e.n)
    m = enc.meta
    C, TB = m.chunk_bytes, m.threads_per_block
    L = list(m.cb.len)
    stream, nib, gaps, blk = enc.stream, enc.nibbles, enc.gaps, enc.blk_off
    cores = len(os.sched_getaffinity(0))

    def one(b):
        t = b * TB
        gap = int(gaps[t >> 1] >> (4 * (t & 1))) & 15
        lo, hi = int(blk[b]), int(blk[b + 1])
        out, _ = oracle.decode_range(stream, nib, L, 8 * C * t + gap, lo, hi - lo)
        return hi - lo

    oracle.lib()
    # calibrate on 32 blocks per core, then size the sample to ~`seconds` of wall time
    cal = min(int(m.n_blocks) // 2, 32 * cores)
    t0 = time.perf_counter()
    with concurrent.futures.ThreadPoolExecutor(cores) as ex:
        done = sum(ex.map(one, range(cal)))
    dt = time.perf_counter() - t0
    nblk = int(max(cores, min(int(m.n_blocks) - cal, cal * seconds / max(dt, 1e-6))))
    blocks = list(range(cal, cal + nblk))
    t0 = time.perf_counter()
    with concurrent.futures.ThreadPoolExecutor(cores) as ex:
        done = sum(ex.map(one, blocks))
    dt = time.perf_counter() - t0
    return {"value": round(done / dt / 1e9, 6), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": "%d whole blocks (%d elements) of the largest tensor, bit-serial C oracle decode, "
                      "one thread per core, %.1f s" % (len(blocks), done, dt)}


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--workload", default="llama70b", choices=sorted(WORKLOAD_TEXT))
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: ECF8 decode is GPU-local (each GPU decodes its own "
              "shard); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import synth
    import lossless_entropy_coded_ecf8_amd as E
    from lossless_entropy_coded_ecf8_amd.workload import batch_bytes

    d = torch.device("cuda:0")
    t0 = time.time()
    wl = args.workload
    if wl == "moe8":
        gen = synth.workload_tensors("moe256", device=d, experts=synth.moe_routing())
    else:
        gen = synth.workload_tensors(wl, device=d)
    names, xs, encs_host, encs = [], [], [], []
    for name, x in gen:
        h = E.encode(x.cpu())
        names.append(name)
        xs.append(x.reshape(-1))
        encs_host.append(h)
        encs.append(h.to(d))
        log("encoded %-12s n=%d  %.3f bits/exponent" % (name, h.n, h.meta.total_bits / max(h.n, 1)))
    log("setup %.1f s" % (time.time() - t0))

    plan = E.DecodePlan(encs)
    plan.run()
    torch.cuda.synchronize()
    bad = plan.status()
    for i, x in enumerate(xs):
        if not torch.equal(plan.view(i), x):
            log("MISMATCH in tensor", names[i])
            sys.exit(1)
    if bad:
        log("block offset check failed on", bad, "blocks")
        sys.exit(1)
    log("bit-exact check passed on %d tensors" % len(xs))

    for _ in range(args.warmup):
        plan.run()
    torch.cuda.synchronize()
    K = args.steps
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for k in range(K):
        plan.build_tables()
        ev[k][0].record()
        plan.decode_blocks()
        ev[k][1].record()
    end.record()
    torch.cuda.synchronize()
    step_ms = start.elapsed_time(end) / K
    dec_ms = sum(a.elapsed_time(b) for a, b in ev) / K

    copy_gbs = copy_ceiling(torch, d)
    bb = batch_bytes(encs)
    n_total = bb["written"]
    value = n_total / (step_ms * 1e-3) / 1e9
    achieved = bb["total"] / (dec_ms * 1e-3) / 1e9
    khash = kernel_source_hash()
    traffic = load_traffic(wl, khash, bb["total"])
    res = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u8",
        "data": "synthetic",
        "config": {"workload": WORKLOAD_TEXT[wl], "name": wl, "tensors": len(encs), "elements": n_total,
                   "compressed_bytes": bb["read"], "bits_per_element": round(8.0 * bb["read"] / n_total, 4),
                   "chunk_bytes": 16, "lanes_per_block": 256, "grid": int(plan.plan.grid)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "kernel": "ecf8_decode_kernel", "kernel_ms": round(dec_ms, 5),
                     "algorithmic_bytes": bb["total"], "kernel_sha": khash,
                     "copy_ceiling_gbs": round(copy_gbs, 1), "frac_of_copy": round(achieved / copy_gbs, 4)},
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample ...")
        res["cpu_baseline"] = cpu_baseline(encs_host, args.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
