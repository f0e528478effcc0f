#!/usr/bin/env python3
"""ECF8 decode benchmark on one MI355X.

One step = one batched decode of a whole workload (default: the Llama-3-70B
transformer block, 7 FP8 E4M3 tensors, 855,638,016 elements) with every
input resident in HBM: one persistent decode dispatch (the decode tables are
built once when the plan is prepared; each workgroup copies its tensor's
table into LDS) into one reused output buffer; the one-tensor-per-launch workloads make one such dispatch
per tensor.  The decoded output is checked bit-exact against the original
bytes before timing.

Prints ONE JSON line: value = decoded FP8 GB/s of the whole step (K timed
steps between two events); roofline = algorithmic HBM bytes of the decode
kernel (compressed bytes read + FP8 bytes written) over its average duration,
from events attached to the dispatch of each timed step (one-dispatch-per-
tensor workloads: of K more steps, since attached events would add launch
work to each of their dispatches); cpu_baseline = the plain C oracle decoding
a bounded sample on the host cores.
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
    "llama8b": "Llama-3-8B attention+MLP weights FP8 E4M3 (q,o 4096x4096; k,v 4096x1024; gate,up 4096x14336; "
               "down 14336x4096), alpha-stable alpha=1.8, per-tensor codebooks, one decode launch per tensor",
    "dit14b": "14B-DiT block FP8 E4M3 (hidden 5120: self/cross-attn qkvo 8x 5120x5120, FFN 5120x13824 and "
              "13824x5120), alpha-stable alpha=1.5 + 2% N(0,0.2) outliers, per-128x128-tile scaling, one batched dispatch",
    "moe8": "MoE layer, the 8 experts of a seeded routing draw x (gate, up 7168x2048; down 2048x7168), FP8 E4M3, "
            "alpha ~ U[1.5,2.0] per expert, per-expert codebooks, one batched dispatch",
    "moe256": "MoE layer, all 256 experts x (gate, up 7168x2048; down 2048x7168) = 11.27 G FP8 E4M3 weights, "
              "alpha ~ U[1.5,2.0] per expert, per-expert codebooks, one batched dispatch",
    "gauss1m": "single 1024x1024 FP8 E4M3 tensor, N(0,0.02), per-tensor max-abs scaling, one decode launch",
}
# configs whose decode reads and writes fit the 256 MB Infinity Cache: their timings are cache-resident
CACHE_RESIDENT = {"gauss1m"}
# configs decoded with one launch per tensor (the others: one batched dispatch per step)
PER_TENSOR = {"llama8b", "gauss1m"}


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


def dispatch_stats(ms_list):
    """Mean, median, min and max (ms) of per-dispatch times."""
    v = sorted(ms_list)
    n = len(v)
    med = v[n // 2] if n % 2 else 0.5 * (v[n // 2 - 1] + v[n // 2])
    return {"mean": round(sum(v) / n, 5), "median": round(med, 5), "min": round(v[0], 5), "max": round(v[-1], 5)}


def copy_ceiling(torch, d, gib: float = 1.0, reps: int = 10):
    """The plain dwordx4 streaming copy of the library (ecf8_hbm_copy), `gib` GiB in and out, back to back:
    median per-dispatch rate in GB/s (bytes read + written)."""
    from lossless_entropy_coded_ecf8_amd import binding as B
    n = int(gib * (1 << 30))
    a = torch.randint(0, 256, (n,), dtype=torch.uint8, device=d)
    b = torch.empty_like(a)
    B.hbm_copy(a, b)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for s, e in ev:
        s.record()
        B.hbm_copy(a, b)
        e.record()
    torch.cuda.synchronize()
    ok = torch.equal(a, b)
    del a, b
    if not ok:
        raise RuntimeError("copy kernel mismatch")
    st = dispatch_stats([s.elapsed_time(e) for s, e in ev])
    return 2.0 * n / (st["median"] * 1e-3) / 1e9


def stream_ceiling(torch, d, read_bytes: int, write_bytes: int, reps: int = 10):
    """The library's plain stream of the same byte mix (ecf8_hbm_stream): read_bytes read once and write_bytes
    written, rounded down to 16-byte units; median per-dispatch time in ms after a 1 GiB read."""
    from lossless_entropy_coded_ecf8_amd import binding as B
    rb, wb = read_bytes // 16 * 16, write_bytes // 16 * 16
    if rb == 0 or rb > wb:
        return None
    src = torch.randint(0, 256, (rb,), dtype=torch.uint8, device=d)
    dst = torch.empty(wb, dtype=torch.uint8, device=d)
    for _ in range(3):
        B.hbm_stream(src, rb, dst, wb)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for s, e in ev:
        s.record()
        B.hbm_stream(src, rb, dst, wb)
        e.record()
    torch.cuda.synchronize()
    u = (rb // 16 << 32) // (wb // 16)
    i = torch.tensor([0, wb // 16 // 2, wb // 16 - 1], dtype=torch.int64)
    j = (i * u) >> 32                                  # spot check of the mapping
    ok = all(torch.equal(dst[16 * int(a):16 * int(a) + 16], src[16 * int(b):16 * int(b) + 16]) for a, b in zip(i, j))
    del src, dst
    if not ok:
        raise RuntimeError("stream kernel mismatch")
    return dispatch_stats([s.elapsed_time(e) for s, e in ev])["median"]


def cpu_baseline(encs_host, seconds: float):
    """Time the C oracle decoding whole blocks of the largest tensor: all host cores (thread pool), then
    one core, each on a bounded sample sized to about `seconds` / 2 of wall time."""
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

    def timed(blocks, threads):
        t0 = time.perf_counter()
        with concurrent.futures.ThreadPoolExecutor(threads) as ex:
            done = sum(ex.map(one, blocks))
        return done, time.perf_counter() - t0

    oracle.lib()
    nb = int(m.n_blocks)
    # all cores: calibrate on 16 blocks per core, then size the sample
    cal = min(nb // 2, 16 * cores)
    _, dt = timed(range(cal), cores)
    nblk = int(max(cores, min(nb - cal, cal * 0.5 * seconds / max(dt, 1e-6))))
    done, dt = timed(range(cal, cal + nblk), cores)
    res = {"value": round(done / dt / 1e9, 6), "unit": "GB/s", "cores": cores, "kind": "oracle",
           "sample": "%d whole blocks (%d elements) of the largest tensor, bit-serial C oracle decode, "
                     "one thread per core, %.1f s" % (nblk, done, dt)}
    # one core
    _, dt1 = timed(range(4), 1)
    n1 = int(max(2, min(nb, 4 * 0.5 * seconds / max(dt1, 1e-6))))
    done1, dt1 = timed(range(n1), 1)
    res["single_core"] = {"value": round(done1 / dt1 / 1e9, 6), "unit": "GB/s", "cores": 1,
                          "sample": "%d whole blocks (%d elements), %.1f s" % (n1, done1, dt1)}
    return res


def copy_calibration(args):
    """The library's plain copy kernel (ecf8_hbm_copy) at several sizes, each dispatch preceded by a 1 GiB
    read that evicts the Infinity Cache: what FETCH_SIZE / WRITE_SIZE read for copies of known size
    calibrates the decode's traffic counters; the event-timed rates are the copy ceiling at each size."""
    import torch
    from lossless_entropy_coded_ecf8_amd import binding as B
    d = torch.device("cuda:0")
    scratch = torch.ones(1 << 27, dtype=torch.int64, device=d)
    rows = []
    for mib in [int(v) for v in args.copy_mib.split(",")]:
        n = mib << 20
        a = torch.randint(0, 256, (n,), dtype=torch.uint8, device=d)
        b = torch.empty_like(a)
        ms = []
        for _ in range(args.steps):
            scratch.sum()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            B.hbm_copy(a, b)
            e1.record()
            torch.cuda.synchronize()
            ms.append(e0.elapsed_time(e1))
        if not torch.equal(a, b):
            log("copy mismatch at", mib, "MiB")
            sys.exit(1)
        st = dispatch_stats(ms)
        rows.append({"mib": mib, "bytes_read": n, "bytes_written": n, "ms": st,
                     "gbs_median": round(2 * n / (st["median"] * 1e-3) / 1e9, 1)})
        log(json.dumps(rows[-1]))
        del a, b
    print(json.dumps({"report": "ecf8_hbm_copy calibration, each dispatch after a 1 GiB read", "rows": rows}),
          flush=True)


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
                      "gemm": "torch._scaled_mm (hipBLASLt FP8 E4M3)"},
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
        """Median over 7 samples of the mean time of `reps` back-to-back calls, after warm-up calls."""
        for _ in range(max(3, args.warmup)):
            fn()
        torch.cuda.synchronize()
        samples = []
        for _ in range(7):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            for _ in range(reps):
                fn()
            b.record()
            torch.cuda.synchronize()
            samples.append(a.elapsed_time(b) / reps)
        return sorted(samples)[3]

    reps = max(3, args.steps // 4)
    hist_ms = timed(lambda: [B.histogram_device(x, f, w) for x, f, w in zip(xs, freqs, wss)], reps)
    enc_ms = timed(lambda: B.encode_batched_into(xs, encs, wss), reps)
    enc_each_ms = timed(lambda: [B.encode_into(x, e, w) for x, e, w in zip(xs, encs, wss)], reps)
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
           "encode_ms_one_call_per_tensor": round(enc_each_ms, 4),
           "end_to_end_ms": round(e2e_ms, 4),
           "end_to_end_note": "encode_device per tensor: histogram, 128 B copy to the host and one "
                              "synchronisation, codebook and sizes on the host, buffer allocation, encode",
           "histogram_pass_gbs": round(n / (hist_ms * 1e-3) / 1e9, 2),
           "encode_pass_hbm_gbs": round((n + comp) / (enc_ms * 1e-3) / 1e9, 2),
           "encode_pass_frac_of_8tbs": round((n + comp) / (enc_ms * 1e-3) / 8e12, 4),
           "encode_pass_note": "histogram pass: reads the input (per-tile counts out); encode pass: reads the "
                               "input once and writes the compressed form, all tensors in one "
                               "ecf8_encode_batched_device call (encode_ms_one_call_per_tensor: one "
                               "ecf8_encode_device call each)"}
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
        hs.append(B.v_encode(fmt, x.cpu(), max_len=args.variant_max_code_len))
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
    del xs
    for _ in range(args.warmup):
        plan.run()
    torch.cuda.synchronize()
    # events attached to each timed dispatch (ecf8v_decode_run_timed): the kernel's start and end
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for e0, e1 in ev:                       # creates the events (outside the timed region)
        e0.record()
        e1.record()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record()
    for e0, e1 in ev:
        plan.run(events=(e0, e1))
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / args.steps
    st = dispatch_stats([e0.elapsed_time(e1) for e0, e1 in ev])
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
                      "grid": int(plan.plan.grid), "code_length_limit": args.variant_max_code_len,
                      "max_code_len": max(int(h.meta.max_len) for h in hs),
                      "short_code_form": bool(plan.plan.short_codes)},
           "roofline": {"bound": "hbm", "achieved": round((read + written) / (st["mean"] * 1e-3) / 1e9, 2),
                        "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": round((read + written) / (st["mean"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                        "frac_median": round((read + written) / (st["median"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                        "kernel_ms": st["mean"], "kernel_ms_median": st["median"], "kernel_ms_min": st["min"],
                        "kernel_ms_max": st["max"],
                        "traffic": traffic, "kernel": "ecf8v_decode_kernel (a run is this one dispatch)",
                        "algorithmic_bytes": read + written, "kernel_sha": khash}}
    print(json.dumps(res), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--workload", default="llama70b", choices=sorted(WORKLOAD_TEXT))
    ap.add_argument("--cpu-seconds", type=float, default=16.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--settled", action="store_true",
                    help="also time K decode steps after about 0.2 s of continuous decoding (kernel_ms_settled)")
    ap.add_argument("--copy-mib", default="512,2048", help="copycal mode: copy sizes in MiB (comma list)")
    ap.add_argument("--chunk-bytes", type=int, default=16, help="decode mode: stream bytes per lane (C)")
    ap.add_argument("--max-code-len", type=int, default=11,
                    help="decode mode: code length limit of the encoding (11: every codeword fits the decode's "
                         "11-bit table index; 16: plain Huffman)")
    ap.add_argument("--variant-max-code-len", type=int, default=10,
                    help="variant mode: code length limit of the encoding (10: every codeword fits the variant "
                         "decode's 10-bit table index; 16: the library default)")
    ap.add_argument("--lanes", type=int, default=256, help="decode mode: lanes per block (TB)")
    ap.add_argument("--experts", type=int, default=0,
                    help="decode mode, moe256: the first N experts only (a shorter dispatch of the same layer)")
    ap.add_argument("--claim-blocks", type=int, default=-1,
                    help="decode mode: block order (0 static, k >= 2 claims of k blocks; default: the library's choice)")
    ap.add_argument("--mode", default="decode", choices=["decode", "pipeline", "alpha", "encode", "variant", "copycal"],
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
    if args.mode == "copycal":
        copy_calibration(args)
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
    elif wl == "moe256" and args.experts:
        gen = synth.workload_tensors(wl, device=d, experts=list(range(args.experts)))
    else:
        gen = synth.workload_tensors(wl, device=d)
    names, xs, encs_host, encs = [], [], [], []
    for name, x in gen:
        h = E.encode(x.cpu(), chunk_bytes=args.chunk_bytes, threads_per_block=args.lanes, max_len=args.max_code_len)
        names.append(name)
        xs.append(x.reshape(-1))
        if wl != "moe256":
            encs_host.append(h)
        elif not encs_host or h.n > encs_host[0].n:
            encs_host = [h]                                   # the CPU leg needs one tensor only
        encs.append(h.to(d))
        if len(names) <= 16:
            log("encoded %-12s n=%d  %.3f bits/exponent" % (name, h.n, h.meta.total_bits / max(h.n, 1)))
    log("setup %.1f s, %d tensors" % (time.time() - t0, len(encs)))

    # one step: one batched dispatch of all tensors, or one dispatch per tensor (the decode tables are
    # built once per plan, so a run is one dispatch)
    claim = None if args.claim_blocks < 0 else args.claim_blocks
    plans = ([E.DecodePlan([e], claim_blocks=claim) for e in encs] if wl in PER_TENSOR
             else [E.DecodePlan(encs, claim_blocks=claim)])
    for p in plans:
        p.run()
    torch.cuda.synchronize()
    bad = sum(p.status() for p in plans)
    views = [p.view(0) for p in plans] if wl in PER_TENSOR else [plans[0].view(i) for i in range(len(encs))]
    for nm, v, x in zip(names, views, xs):
        if not torch.equal(v, x):
            log("MISMATCH in tensor", nm)
            sys.exit(1)
    if bad:
        log("block offset check failed on", bad, "blocks")
        sys.exit(1)
    log("bit-exact check passed on %d tensors" % len(xs))
    del xs, views

    def step(evs=None):
        # with events, they are attached to each decode dispatch itself (ecf8_decode_run_timed): they
        # hold the kernel's start and end, not the launch and completion latency of events recorded
        # around it
        for i, p in enumerate(plans):
            p.run(events=None if evs is None else evs[i])

    def new_events():
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in plans]
        for a, b in ev:                     # creates the events (outside any timed region)
            a.record()
            b.record()
        return ev

    # The timed region: K steps between two events.  A batched step is one dispatch, and its
    # attached events (about 10 us of launch work a step) are in the timed region, so `value` and
    # the kernel time come from the same steps.  A one-dispatch-per-tensor step would carry one
    # pair per tensor (about 18 us each): its K timed steps are plain launches, and the kernel
    # time comes from the K steps that follow, with events attached.
    separate = wl in PER_TENSOR
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    K = args.steps
    ev = [new_events() for _ in range(K)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for k in range(K):
        step(None if separate else ev[k])
    end.record()
    torch.cuda.synchronize()
    step_ms = start.elapsed_time(end) / K
    if separate:
        for k in range(K):
            step(ev[k])
        torch.cuda.synchronize()
    dec = [sum(a.elapsed_time(b) for a, b in e) for e in ev]      # decode time of each step
    st = dispatch_stats(dec)

    # --settled: the same decode once the device has run it without a pause for about 0.2 s (its
    # clocks have then left the start-up transient that a short timed region falls in); off by
    # default, so that a profiler's average over the run's dispatches is the timed region's
    sts = None
    if args.settled:
        t_end = time.time() + 0.2
        while time.time() < t_end:
            for _ in range(20):
                step()
            torch.cuda.synchronize()
        evs_ = [new_events() for _ in range(K)]
        for k in range(K):
            step(evs_[k])
        torch.cuda.synchronize()
        sts = dispatch_stats([sum(a.elapsed_time(b) for a, b in e) for e in evs_])

    # the same decode with a 1 GiB read before each step: the 256 MB Infinity Cache then holds only
    # clean lines of that buffer (a write would leave dirty lines for the decode to write back)
    scratch = torch.ones(1 << 27, dtype=torch.int64, device=d)
    kc = min(K, 20)
    evc = [new_events() for _ in range(kc)]
    for k in range(kc):
        scratch.sum()
        step(evc[k])
    torch.cuda.synchronize()
    stc = dispatch_stats([sum(a.elapsed_time(b) for a, b in e) for e in evc])
    del scratch

    copy_gbs = copy_ceiling(torch, d)
    bbs = batch_bytes(encs)
    stream_ms = stream_ceiling(torch, d, bbs["read"], bbs["written"])
    bb = batch_bytes(encs)
    n_total = bb["written"]
    value = n_total / (step_ms * 1e-3) / 1e9
    achieved = bb["total"] / (st["mean"] * 1e-3) / 1e9
    khash = kernel_source_hash()
    traffic = load_traffic(wl, khash, bb["total"])
    gbs = lambda ms: round(bb["total"] / (ms * 1e-3) / 1e9, 2)
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
        "config": {"workload": (WORKLOAD_TEXT[wl] if not (wl == "moe256" and args.experts) else
                                "MoE layer, the first %d of its 256 experts x (gate, up 7168x2048; down 2048x7168), "
                                "FP8 E4M3, alpha ~ U[1.5,2.0] per expert, per-expert codebooks, one batched dispatch"
                                % args.experts),
                   "name": wl if not (wl == "moe256" and args.experts) else "moe256_first%d" % args.experts,
                   "tensors": len(encs), "elements": n_total,
                   "compressed_bytes": bb["read"], "bits_per_element": round(8.0 * bb["read"] / n_total, 4),
                   "chunk_bytes": args.chunk_bytes, "lanes_per_block": args.lanes,
                   "max_code_len": max(max(int(v) for v in e.meta.cb.len) for e in encs),
                   "code_length_limit": args.max_code_len,
                   "short_code_form": all(int(p.plan.short_codes) for p in plans), "launches_per_step": len(plans),
                   "grid": int(max(p.plan.grid for p in plans)),
                   "claim_blocks": int(max(p.plan.claim_blocks for p in plans))},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "kernel": "ecf8_decode_kernel", "kernel_ms": st["mean"], "kernel_ms_median": st["median"],
                     "kernel_ms_min": st["min"], "kernel_ms_max": st["max"],
                     "frac_median": round(gbs(st["median"]) / HBM_PEAK_GBS, 4),
                     "algorithmic_bytes": bb["total"], "kernel_sha": khash,
                     "copy_ceiling_gbs": round(copy_gbs, 1), "frac_of_copy": round(achieved / copy_gbs, 4),
                     "stream_mix_ms": None if stream_ms is None else round(stream_ms, 5),
                     "frac_of_stream_mix": None if stream_ms is None else round(stream_ms / st["mean"], 4),
                     "stream_mix_note": "ecf8_hbm_stream: the same bytes read and written by a plain stream "
                                        "(no decode work); frac_of_stream_mix = its median time / the mean "
                                        "decode time",
                     "cache": ("every byte the decode reads and writes fits the 256 MB Infinity Cache: cache-resident "
                               "timings" if wl in CACHE_RESIDENT else
                               "kernel_ms*: back-to-back steps (part of one step's data stays in the 256 MB Infinity "
                               "Cache for the next); kernel_ms_cache_evicted*: each step after a 1 GiB read"),
                     "kernel_ms_cache_evicted": stc["mean"], "kernel_ms_cache_evicted_median": stc["median"],
                     "kernel_ms_cache_evicted_min": stc["min"], "kernel_ms_cache_evicted_max": stc["max"],
                     "frac_cache_evicted": round(gbs(stc["mean"]) / HBM_PEAK_GBS, 4),
                     "kernel_timing": ("a second series of K steps, events attached to each dispatch (the K "
                                       "timed steps are plain launches)" if separate else
                                       "events attached to the dispatch of each of the K timed steps"),
                     **({} if sts is None else {
                         "kernel_ms_settled": sts["mean"], "kernel_ms_settled_median": sts["median"],
                         "frac_settled": round(gbs(sts["mean"]) / HBM_PEAK_GBS, 4),
                         "settled_note": "--settled: K more steps after about 0.2 s of continuous decoding (the "
                                         "device leaves its start-up clock transient; context, not the "
                                         "headline)"}),
                     "decode_us_per_step": [round(1000 * t, 1) for t in dec[:50]]},
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample ...")
        res["cpu_baseline"] = cpu_baseline(encs_host, args.cpu_seconds)
    print(json.dumps(res), flush=True)

if __name__ == "__main__":
    main()
