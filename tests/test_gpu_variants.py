"""GPU decode of the BF16 (DFloat11 layout) and E5M2 variants: the HIP path (C ABI) against the oracle.

Bit-exact is the bar.  Small and edge cases compare every decoded element
with the oracle's bit-serial decode of the same stream and with the input,
with canary bytes around every output; full-size workloads compare every
element with the input on the GPU and sampled blocks with the oracle.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from lossless_entropy_coded_ecf8_amd import binding as B

pytestmark = pytest.mark.gpu

CANARY = 0xA5


def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def make(fmt, n, seed, kind="normal"):
    g = torch.Generator().manual_seed(seed)
    if kind == "all_exponents":                   # every exponent value (BF16: 256, E5M2: 32)
        v = torch.randint(0, 1 << 16 if fmt == "bf16" else 256, (n,), generator=g)
        return v.numpy().astype(np.uint16 if fmt == "bf16" else np.uint8)
    if kind == "single":
        return np.full(n, 0x3C11 if fmt == "bf16" else 0x3D, dtype=np.uint16 if fmt == "bf16" else np.uint8)
    x = torch.randn(n, generator=g) * (0.02 if fmt == "bf16" else 3.0)
    if kind == "heavy":
        x = x * torch.exp(torch.randn(n, generator=g) * 2.5)
    if fmt == "bf16":
        return x.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    return x.to(torch.float8_e5m2).view(torch.uint8).numpy()


def decode_checked(encs_host, d, pad=256):
    """Batched decode into a canary-filled buffer; returns per-tensor numpy outputs."""
    encs = [h.to(d) for h in encs_host]
    sizes = [h.n * (2 if h.meta.format == 1 else 1) for h in encs_host]
    offs, off = [], pad
    for s in sizes:
        offs.append(off)
        off += (s + pad + 15) // 16 * 16
    buf = torch.full((off + pad,), CANARY, dtype=torch.uint8, device=d)
    plan = B.DecodePlanV(encs, out=buf, offsets=offs)
    plan.run()
    torch.cuda.synchronize()
    assert plan.status() == 0
    b = buf.cpu().numpy()
    outs, prev = [], 0
    for o, s in zip(offs, sizes):
        assert (b[prev:o] == CANARY).all(), "write outside a tensor's output"
        outs.append(b[o:o + s])
        prev = o + s
    assert (b[prev:] == CANARY).all()
    return outs, plan


def as_elems(fmt, raw_bytes):
    return raw_bytes.view("<u2") if fmt == "bf16" else raw_bytes


SMALL = [(f, n, k) for f in ("bf16", "e5m2") for n, k in
         [(1, "normal"), (2, "normal"), (17, "normal"), (4095, "normal"), (4097, "heavy"), (65537, "normal"),
          (300_001, "heavy"), (1_000_003, "normal"), (50_000, "all_exponents"), (70_000, "single")]]


@pytest.mark.parametrize("fmt,n,kind", SMALL, ids=lambda v: str(v))
@pytest.mark.parametrize("tb", [256, 128, 64])
def test_small_and_edge_cases_bit_exact(fmt, n, kind, tb):
    d = dev()
    x = make(fmt, n, n + tb, kind)
    h = B.v_encode(fmt, x, threads_per_block=tb)
    (got,), _ = decode_checked([h], d)
    ref = oracle.v_decode(fmt, h.stream, h.raw, n, h.lengths)
    assert np.array_equal(ref, x)
    bad = np.nonzero(as_elems(fmt, got) != ref)[0]
    assert bad.size == 0, "first mismatch at %d of %d" % (bad[0], n)


@pytest.mark.parametrize("max_len", [16, 11, 9])
def test_length_limits_and_long_codes(max_len):
    """Heavy-tailed BF16 at several length limits: codes longer than the 10-bit window use the 16-bit region."""
    d = dev()
    x = make("bf16", 400_000, max_len, "heavy")
    h = B.v_encode("bf16", x, max_len=max_len)
    assert h.meta.max_len == max_len or max_len == 16
    (got,), _ = decode_checked([h], d)
    assert np.array_equal(as_elems("bf16", got), x)


@pytest.mark.parametrize("fmt", ["bf16", "e5m2"])
@pytest.mark.parametrize("kind,max_len", [("heavy", 16), ("heavy", 10), ("normal", 9), ("single", 16),
                                          ("all_exponents", 10)])
def test_short_code_form_selected_and_bit_exact(fmt, kind, max_len):
    """Plans whose codes are all at most 10 bits long take the one-shift table index (short_codes = 1),
    others the general one; both decode bit-exactly (the single-symbol code is incomplete: its unused
    prefixes decode nothing in either form)."""
    d = dev()
    x = make(fmt, 300_001, 13 + max_len, kind)
    h = B.v_encode(fmt, x, max_len=max_len)
    want_short = int(max(int(v) for v in h.lengths) <= 10)
    if kind == "heavy" and max_len == 16:
        assert not want_short, "the heavy-tailed case should need codes longer than 10 bits"
    (got,), plan = decode_checked([h], d)
    assert int(plan.plan.short_codes) == want_short
    ref = oracle.v_decode(fmt, h.stream, h.raw, h.n, h.lengths)
    assert np.array_equal(ref, x)
    bad = np.nonzero(as_elems(fmt, got) != ref)[0]
    assert bad.size == 0, "first mismatch at %d of %d" % (bad[0], h.n)


def test_short_form_needs_every_tensor_short():
    """One tensor with a code longer than 10 bits keeps the whole batch on the general form."""
    d = dev()
    hs = [B.v_encode("e5m2", make("e5m2", 200_000, 3, "normal"), max_len=10),
          B.v_encode("e5m2", make("e5m2", 200_000, 4, "heavy"))]
    assert max(int(v) for v in hs[1].lengths) > 10
    outs, plan = decode_checked(hs, d)
    assert int(plan.plan.short_codes) == 0
    for h, got in zip(hs, outs):
        assert np.array_equal(got, oracle.v_decode("e5m2", h.stream, h.raw, h.n, h.lengths))
    outs, plan = decode_checked(hs[:1], d)
    assert int(plan.plan.short_codes) == 1


def test_batched_mixed_formats_rejected_and_mixed_codebooks_ok():
    d = dev()
    hs = [B.v_encode("bf16", make("bf16", n, n, k)) for n, k in [(100_000, "normal"), (3, "normal"),
                                                                    (250_000, "heavy"), (64_001, "all_exponents")]]
    outs, plan = decode_checked(hs, d)
    for h, o in zip(hs, outs):
        assert np.array_equal(as_elems("bf16", o), oracle.v_decode("bf16", h.stream, h.raw, h.n, h.lengths))
    plan.run()                                   # a second run of the same plan is idempotent
    torch.cuda.synchronize()
    assert plan.status() == 0
    for i, h in enumerate(hs):
        assert np.array_equal(plan.view(i).cpu().numpy().view(np.uint16),
                              oracle.v_decode("bf16", h.stream, h.raw, h.n, h.lengths))
    e = B.v_encode("e5m2", make("e5m2", 1000, 1))
    with pytest.raises(B.Ecf8Error):
        B.DecodePlanV([hs[0].to(d), e.to(d)])


def test_corrupt_block_offset_is_flagged_and_contained():
    d = dev()
    x = make("bf16", 200_000, 9)
    h = B.v_encode("bf16", x, threads_per_block=64)
    assert h.meta.n_blocks > 4
    h.blk_off[2] += 5                            # block 1 and block 2 now disagree with their counts
    outs, plan = None, None
    encs = [h.to(d)]
    buf = torch.full((2 * x.size + 512,), CANARY, dtype=torch.uint8, device=d)
    plan = B.DecodePlanV(encs, out=buf, offsets=[256])
    plan.run()
    torch.cuda.synchronize()
    assert plan.status() == 2
    b = buf.cpu().numpy()
    assert (b[:256] == CANARY).all() and (b[256 + 2 * x.size:] == CANARY).all()
    got = b[256:256 + 2 * x.size].view("<u2")
    lo = int(h.blk_off[3])
    assert np.array_equal(got[lo:], x[lo:])      # later blocks unaffected


def test_status_counts_until_read_and_timed_run():
    """The variant block-check counter adds over runs and restarts when read; a run with events
    attached to its dispatch (ecf8v_decode_run_timed) decodes the same bytes, and its events hold
    a positive duration no longer than events recorded around the launch."""
    d = dev()
    x = make("e5m2", 300_000, 11)
    h = B.v_encode("e5m2", x, threads_per_block=64)
    good = B.DecodePlanV([h.to(d)])
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    o0, o1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for ev in (a, b):
        ev.record()
    good.out.fill_(CANARY)
    o0.record()
    good.run(events=(a, b))
    o1.record()
    torch.cuda.synchronize()
    assert good.status() == 0
    assert np.array_equal(as_elems("e5m2", good.view(0).cpu().numpy()), x)
    assert 0 < a.elapsed_time(b) <= o0.elapsed_time(o1) * 1.001 + 1e-3
    h.blk_off[2] += 5                            # blocks 1 and 2 disagree with their counts
    bad = B.DecodePlanV([h.to(d)])
    bad.run()
    assert bad.status() == 2
    assert bad.status() == 0
    bad.run()
    bad.run()
    assert bad.status() == 4
    assert bad.status() == 0


def dense_sparse_runs(fmt, n, dense_run, sparse_run, seed):
    """Runs of one exponent (a 1-bit code: 128 codewords per 16-byte chunk) between runs of ~100
    exponents (long codes), so that blocks stay under 16384 symbols while some chunks need more
    than 20 table lookups."""
    rng = np.random.default_rng(seed)
    bit = lambda k: rng.integers(0, 1 << k, size=n)
    if fmt == "bf16":
        sparse = (bit(1) << 15) | (rng.integers(60, 160, size=n) << 7) | bit(7)
        dense = (bit(1) << 15) | (127 << 7) | bit(7)
        dt = np.uint16
    else:
        sparse = (bit(1) << 7) | (rng.integers(2, 30, size=n) << 2) | bit(2)
        dense = (bit(1) << 7) | (15 << 2) | bit(2)
        dt = np.uint8
    return np.where(np.arange(n) % (dense_run + sparse_run) < dense_run, dense, sparse).astype(dt)


@pytest.mark.parametrize("fmt,sparse_run", [("bf16", 3300), ("e5m2", 5000)])
def test_lanes_past_the_recorded_lookups(fmt, sparse_run):
    """Chunks of 128 one-bit codewords take more lookups than a lane records; their lanes finish the
    replay from registers (blocks still fit the stage, so the round path is not taken)."""
    d = dev()
    x = dense_sparse_runs(fmt, 300_000, 8192, sparse_run, 7)
    h = B.v_encode(fmt, x)
    L = np.asarray(h.lengths, dtype=np.int64)
    sym = (x.astype(np.int64) >> 7) & 255 if fmt == "bf16" else (x.astype(np.int64) >> 2) & 31
    starts = np.concatenate([[0], np.cumsum(L[sym])])[:-1]
    per_chunk = np.bincount(starts // (8 * h.meta.chunk_bytes))
    assert per_chunk.max() > 3 * 20                                    # more than 20 three-symbol lookups
    assert np.diff(np.asarray(h.blk_off, dtype=np.int64)).max() <= 16384
    (got,), _ = decode_checked([h], d)
    assert np.array_equal(as_elems(fmt, got), x)
    assert np.array_equal(oracle.v_decode(fmt, h.stream, h.raw, h.n, h.lengths), x)


def test_window_with_no_codeword_is_flagged_and_contained():
    """A single-symbol code leaves half the code space unused: stream bits that start no codeword
    mark their block bad (not written); the other blocks decode exactly."""
    d = dev()
    x = make("bf16", 70_000, 5, "single")
    h = B.v_encode("bf16", x)
    assert int(np.count_nonzero(h.lengths)) == 1 and h.meta.n_blocks == 3
    h.stream[100] = 0xFF                         # inside block 0
    buf = torch.full((2 * x.size + 512,), CANARY, dtype=torch.uint8, device=d)
    plan = B.DecodePlanV([h.to(d)], out=buf, offsets=[256])
    plan.run()
    torch.cuda.synchronize()
    assert plan.status() == 1
    b = buf.cpu().numpy()
    assert (b[:256] == CANARY).all() and (b[256 + 2 * x.size:] == CANARY).all()
    got = b[256:256 + 2 * x.size].view("<u2")
    lo = int(h.blk_off[1])
    assert (b[256:256 + 2 * lo] == CANARY).all()    # the bad block is not written
    assert np.array_equal(got[lo:], x[lo:])


def test_empty_and_zero_tensor_plans():
    d = dev()
    h0 = B.v_encode("bf16", np.zeros(0, dtype=np.uint16))
    h1 = B.v_encode("bf16", make("bf16", 5000, 2))
    outs, plan = decode_checked([h0, h1], d)
    assert outs[0].size == 0
    assert np.array_equal(as_elems("bf16", outs[1]), make("bf16", 5000, 2))


# ---------------------------------------------------------------- full-size workload

def sampled_blocks(fmt, h, out_elems, rng, k=3):
    m = h.meta
    C, TB = m.chunk_bytes, m.threads_per_block
    for b in sorted({0, int(m.n_blocks) - 1} | set(int(v) for v in rng.integers(0, m.n_blocks, k))):
        t = b * TB
        gap = (int(h.gaps[t >> 1]) >> (4 * (t & 1))) & 15
        lo, hi = int(h.blk_off[b]), int(h.blk_off[b + 1])
        ref, _ = oracle.v_decode_range(fmt, h.stream, h.raw, h.lengths, 8 * C * t + gap, lo, hi - lo)
        assert np.array_equal(out_elems[lo:hi], ref), b


@pytest.mark.parametrize("fmt", ["bf16", "e5m2"])
def test_llama70b_block_batched(fmt):
    d = dev()
    names, xs, hs = [], [], []
    for name, x in synth.workload_tensors_as("llama70b", fmt, device=d):
        names.append(name)
        xs.append(x.reshape(-1))
        hs.append(B.v_encode(fmt, x.cpu()))
    plan = B.DecodePlanV([h.to(d) for h in hs])
    plan.run()
    torch.cuda.synchronize()
    assert plan.status() == 0
    rng = np.random.default_rng(0)
    for i, (nm, x, h) in enumerate(zip(names, xs, hs)):
        v = plan.view(i)
        ref = x.view(torch.int16) if fmt == "bf16" else x
        assert torch.equal(v, ref), nm
        if i in (0, 4):
            out = v.cpu().numpy()
            sampled_blocks(fmt, h, out.view(np.uint16) if fmt == "bf16" else out, rng)
