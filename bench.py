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


def kernel_source_hash(source: str = "ecf8_decode.hip") -> str:
    """Hash of a kernel source file with comments and blank lines removed."""
    import re
    p = os.path.join(ROOT, "lossless_entropy_coded_ecf8_amd", "csrc", source)
    text = re.sub(r"//[^\n]*", "", open(p).read())
    code = "\n".join(line.rstrip() for line in text.splitlines() if line.strip())
    return hashlib.sha256(code.encode()).hexdigest()[:16]


def load_traffic(workload: str, kernel_hash: str, launches_bytes: float = 0.0):
    """HBM traffic per launch from committed rocprofv3 counter summaries, if they match this kernel
    (`workload` names the summary: traffic_<workload>.json under profiles/)."""
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


def alpha_report(n: int = 1 << 24):
    """Tail index vs exponent entropy (ECF8 blog §2.2 bound, §6 estimator) on seeded CMS samples."""
    import math
    import numpy as np
    import torch
    import synth
    import lossless_entropy_coded_ecf8_amd as E

    d = torch.device("cuda:0") if torch.cuda.is_available() else torch.device("cpu")
    rows = []
    for alpha in (1.5, 1.6, 1.7, 1.8, 1.9, 2.0):
        g = torch.Generator(device=d).manual_seed(synth.seed_of("alpha-report", alpha))
        x = synth.alpha_stable(alpha, n, g, d, synth.GAMMA)
        ah = E.alpha_hat(x.float().cpu().numpy(), synth.GAMMA)
        # the pages' E = floor(log2 |x|) of the raw weight, and the E4M3 exponent field after scaling
        e_raw = torch.floor(torch.log2(x.abs().clamp_min(1e-300))).to(torch.int64).cpu().numpy()
        _, c = np.unique(e_raw, return_counts=True)
        p = c / c.sum()
        h_raw = float(-(p * np.log2(p)).sum())
        q = synth.to_e4m3_bytes(synth.maxabs_scale(x)).cpu().numpy()
        f = E.histogram(q).astype(np.float64)
        pf = f[f > 0] / f.sum()
        h_fp8 = float(-(pf * np.log2(pf)).sum())
        enc = E.encode(q)
        rows.append({"alpha": alpha, "n": n, "alpha_hat": round(ah, 4), "H_floor_log2": round(h_raw, 4),
                     "H_e4m3_exponent": round(h_fp8, 4), "huffman_bits": round(enc.meta.total_bits / n, 4),
                     "bound": round(E.exponent_entropy_bound(alpha), 4)})
        log(json.dumps(rows[-1]))
    print(json.dumps({"report": "alpha-stable tail index vs exponent entropy", "gamma": synth.GAMMA,
                      "estimator": "alpha_hat = log n / log(max|w| / gamma)",
                      "bound": "alpha / (1 - 2^-alpha)", "rows": rows}), flush=True)


def pipeline_bench(args):
    """Decode-on-use (ECF8 blog §3.2.2/§3.3): forward time of the block's linear layers with weights
    decoded ahead of use into a 3-slot pool, against the same FP8 GEMMs on resident FP8 weights."""
    import torch
    import synth
    import lossless_entropy_coded_ecf8_amd as E
    from lossless_entropy_coded_ecf8_amd import pipeline as P

    d = torch.device("cuda:0")
    names, ws, layers = [], [], []
    for name, x in synth.workload_tensors(args.workload, device=d):
        o, k = x.shape[-2], x.shape[-1]
        names.append(name)
        ws.append(x.reshape(o, k))
        layers.append(E.ECF8Linear(x.reshape(o, k), scale=1.0 / 64, device=d))
        log("compressed %-10s %d x %d" % (name, o, k))
    ws, layers = ws * args.repeats, layers * args.repeats
    resident = sum(w.numel() for w in ws)
    compressed = sum(l.compressed_bytes() for l in layers[: len(layers) // args.repeats]) * args.repeats
    configs = [("serial", 3, 0, None), ("ahead2", 3, 2, None), ("ahead2_wg256", 3, 2, 256)]
    chosen = args.pipe_configs.split(",")
    pipes = {nm: P.DecodePipeline(layers, slots=s, ahead=a, workgroups=wg) for nm, s, a, wg in configs
             if nm in chosen}
    results = []
    for T in [int(t) for t in args.tokens.split(",")]:
        g = torch.Generator(device=d).manual_seed(T)
        xs = [(torch.randn(T, l.in_features, device=d, generator=g) * 4).clamp(-448, 448)
              .to(torch.float8_e4m3fn) for l in layers]
        scs = [torch.tensor(0.25, dtype=torch.float32, device=d) for _ in layers]
        ref = [P.linear_fp8(x, s, w, l.w_scale) for x, s, w, l in zip(xs, scs, ws, layers)]
        for nm, pipe in pipes.items():                      # bit-exact against resident weights
            outs = pipe.run(xs, scs)
            torch.cuda.synchronize()
            if not all(torch.equal(o, r) for o, r in zip(outs, ref)):
                log("MISMATCH in pipeline", nm, "T", T)
                sys.exit(1)
        del ref

        def timed(fn, reps):
            for _ in range(3):
                fn()
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            for _ in range(reps):
                fn()
            b.record()
            torch.cuda.synchronize()
            return a.elapsed_time(b) / reps

        reps = max(3, min(20, args.steps))
        row = {"tokens": T, "resident_ms": round(timed(
            lambda: [P.linear_fp8(x, s, w, l.w_scale) for x, s, w, l in zip(xs, scs, ws, layers)], reps), 4)}
        for nm, pipe in pipes.items():
            row[nm + "_ms"] = round(timed(lambda: pipe.run(xs, scs), reps), 4)
            row[nm + "_vs_resident"] = round(row[nm + "_ms"] / row["resident_ms"], 4)
        log(json.dumps(row))
        results.append(row)
        del xs
    main_cfg = "ahead2" if "ahead2" in pipes else next(iter(pipes))
    pool = pipes[main_cfg].pool_bytes()
    res = {"metric": "ECF8 decode-on-use forward time / resident-FP8 forward time (FP8 GEMMs of the block's "
                     "linear layers, decode 2 layers ahead on a side stream into a 3-slot pool)",
           "value": results[-1][main_cfg + "_vs_resident"], "unit": "ratio", "n_gpus": 1,
           "higher_is_better": False, "dtype": "fp8 e4m3 GEMM, u8 decode", "data": "synthetic",
           "config": {"workload": WORKLOAD_TEXT[args.workload], "layers": len(layers), "repeats": args.repeats,
                      "gemm": "torch._scaled_mm" if P._scaled_mm_ok(d) else "bf16 matmul"},
           "memory": {"resident_fp8_bytes": resident, "compressed_bytes": compressed, "pool_bytes": pool,
                      "ecf8_total_bytes": compressed + pool},
           "results": results}
    print(json.dumps(res), flush=True)


def encode_bench(args):
    """GPU encode (ECF8 blog §3.1.1 / §3.2.1 on the device) of every tensor of the workload: histogram,
    then tile sums, scans and the encode kernel; output checked byte-identical to the host encoder."""
    import numpy as np
    import torch
    import synth
    import lossless_entropy_coded_ecf8_amd as E
    from lossless_entropy_coded_ecf8_amd import binding as B

    d = torch.device("cuda:0")
    names, xs = [], []
    for name, x in synth.workload_tensors(args.workload, device=d):
        names.append(name)
        xs.append(x.reshape(-1))
    encs = [E.encode_device(x) for x in xs]
    torch.cuda.synchronize()
    for nm, x, e in zip(names, xs, encs):                  # byte-identical to the host encoder
        h = E.encode(x.cpu())
        same = (B.meta_dict(h.meta) == B.meta_dict(e.meta) and np.array_equal(h.stream, e.stream.cpu().numpy())
                and np.array_equal(h.nibbles, e.nibbles.cpu().numpy()) and np.array_equal(h.gaps, e.gaps.cpu().numpy())
                and np.array_equal(h.blk_off.view(np.int64), e.blk_off.cpu().numpy()))
        if not same:
            log("MISMATCH device encode vs host encoder:", nm)
            sys.exit(1)
    log("device encode byte-identical to the host encoder on %d tensors" % len(xs))
    wss = [B.encode_workspace(x.numel(), d) for x in xs]     # per-tensor workspaces keep each tensor's tile counts
    freqs = [torch.empty(16, dtype=torch.int64, device=d) for _ in xs]

    def timed(fn, reps):
        for _ in range(max(2, args.warmup // 10)):
            fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    reps = max(3, args.steps // 5)
    hist_ms = timed(lambda: [B.histogram_device(x, f, w) for x, f, w in zip(xs, freqs, wss)], reps)
    enc_ms = timed(lambda: [B.encode_into(x, e, w) for x, e, w in zip(xs, encs, wss)], reps)
    torch.cuda.synchronize()
    for nm, x, e in zip(names, xs, encs):                  # the timed encodes rewrote the same bytes
        if not torch.equal(E.decode(e), x):
            log("MISMATCH after the timed encodes:", nm)
            sys.exit(1)
    e2e_ms = timed(lambda: [E.encode_device(x) for x in xs], reps)
    n = sum(x.numel() for x in xs)
    comp = sum(E.binding.compressed_bytes(e.meta) for e in encs)
    res = {"metric": "ECF8 GPU encode, FP8 GB/s encoded on 1 MI355X (histogram + encode kernels)",
           "value": round(n / ((hist_ms + enc_ms) * 1e-3) / 1e9, 3), "unit": "GB/s", "n_gpus": 1,
           "higher_is_better": True, "dtype": "u8", "data": "synthetic",
           "config": {"workload": WORKLOAD_TEXT[args.workload], "tensors": len(xs), "elements": n,
                      "compressed_bytes": comp},
           "histogram_ms": round(hist_ms, 4), "encode_ms": round(enc_ms, 4),
           "end_to_end_ms": round(e2e_ms, 4),
           "end_to_end_note": "encode_device per tensor: histogram, 128 B copy to the host and one "
                              "synchronisation, codebook and sizes on the host, buffer allocation, encode",
           "histogram_pass_gbs": round(n / (hist_ms * 1e-3) / 1e9, 2),
           "encode_pass_hbm_gbs": round((n + comp) / (enc_ms * 1e-3) / 1e9, 2),
           "encode_pass_note": "histogram pass: reads the input (per-tile counts out); encode pass: reads the "
                               "input once and writes the compressed form"}
    print(json.dumps(res), flush=True)


def variant_bench(args):
    """Batched GPU decode of a format variant (BF16 in the DFloat11 layout, or FP8 E5M2) on the workload:
    host encode, upload, one decode plan; output checked bit-exact against the input before timing."""
    import torch
    import synth
    from lossless_entropy_coded_ecf8_amd import binding as B

    d = torch.device("cuda:0")
    fmt = args.format
    names, xs, hs = [], [], []
    for name, x in synth.workload_tensors_as(args.workload, fmt, device=d):
        names.append(name)
        xs.append(x.reshape(-1).view(torch.int16) if fmt == "bf16" else x.reshape(-1))
        hs.append(B.v_encode(fmt, x.cpu()))
        log("encoded %-12s n=%d  %.3f code bits/element, max_len %d" % (name, hs[-1].n,
                                                                        hs[-1].meta.total_bits / hs[-1].n,
                                                                        hs[-1].meta.max_len))
    plan = B.DecodePlanV([h.to(d) for h in hs])
    plan.run()
    torch.cuda.synchronize()
    if plan.status() or not all(torch.equal(plan.view(i), x) for i, x in enumerate(xs)):
        log("MISMATCH in the variant decode")
        sys.exit(1)
    log("bit-exact check passed on %d tensors" % len(xs))
    for _ in range(args.warmup):
        plan.run()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(args.steps):
        plan.run()
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / args.steps
    eb = 2 if fmt == "bf16" else 1
    khash = kernel_source_hash("ecf8v_decode.hip")
    traffic = load_traffic("variant_%s_%s" % (fmt, args.workload), khash)
    n = sum(h.n for h in hs)
    read = sum(h.compressed_bytes() for h in hs)
    written = n * eb
    res = {"metric": "ECF8 variant decoded GB/s on 1 MI355X (%s, %s)" %
                     (fmt, "DFloat11 layout" if fmt == "bf16" else "5-bit exponent coded"),
           "value": round(written / (ms * 1e-3) / 1e9, 3), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True, "dtype": "u8",
           "data": "synthetic",
           "config": {"workload": WORKLOAD_TEXT[args.workload] + ", cast to " + fmt, "format": fmt,
                      "tensors": len(hs), "elements": n, "compressed_bytes": read,
                      "compressed_ratio": round(read / written, 4), "chunk_bytes": 16, "lanes_per_block": 256,
                      "grid": int(plan.plan.grid)},
           "roofline": {"bound": "hbm", "achieved": round((read + written) / (ms * 1e-3) / 1e9, 2),
                        "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": round((read + written) / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                        "traffic": traffic, "kernel": "ecf8v_decode_kernel (+ table kernel, one run)",
                        "algorithmic_bytes": read + written, "kernel_sha": khash}}
    print(json.dumps(res), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--workload", default="llama70b", choices=sorted(WORKLOAD_TEXT))
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--mode", default="decode", choices=["decode", "pipeline", "alpha", "encode", "variant"],
                    help="decode: the batched decode step (default); pipeline: decode-on-use of the "
                         "block's layers beside FP8 GEMMs, against resident FP8 weights")
    ap.add_argument("--format", default="bf16", choices=["bf16", "e5m2"], help="variant mode: the float format")
    ap.add_argument("--tokens", default="128,1024,4096", help="pipeline mode: GEMM rows (comma list)")
    ap.add_argument("--repeats", type=int, default=2, help="pipeline mode: copies of the block's 7 layers")
    ap.add_argument("--pipe-configs", default="serial,ahead2,ahead2_wg256",
                    help="pipeline mode: which decode schedules to run (comma list)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: ECF8 decode is GPU-local (each GPU decodes its own "
              "shard); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    if args.mode == "pipeline":
        pipeline_bench(args)
        return
    if args.mode == "alpha":
        alpha_report()
        return
    if args.mode == "encode":
        encode_bench(args)
        return
    if args.mode == "variant":
        variant_bench(args)
        return

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

    # the same decode with a 1 GiB read before each dispatch: the 256 MB Infinity Cache then holds
    # only clean lines of that buffer (a write would leave dirty lines for the decode to write back)
    scratch = torch.ones(1 << 27, dtype=torch.int64, device=d)
    kc = min(K, 20)
    evc = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(kc)]
    for k in range(kc):
        scratch.sum()
        plan.build_tables()
        evc[k][0].record()
        plan.decode_blocks()
        evc[k][1].record()
    torch.cuda.synchronize()
    cold_ms = sum(a.elapsed_time(b) for a, b in evc) / kc
    del scratch

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
                     "copy_ceiling_gbs": round(copy_gbs, 1), "frac_of_copy": round(achieved / copy_gbs, 4),
                     "cache": "kernel_ms: back-to-back dispatches (part of one step's data stays in the 256 MB "
                              "Infinity Cache for the next); kernel_ms_cache_evicted: each dispatch after a 1 GiB read",
                     "kernel_ms_cache_evicted": round(cold_ms, 5),
                     "frac_cache_evicted": round(bb["total"] / (cold_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample ...")
        res["cpu_baseline"] = cpu_baseline(encs_host, args.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
