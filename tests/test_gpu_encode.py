"""GPU histogram and encode parity: the HIP path (through the C ABI) against the oracle.

Every buffer the device encode writes (stream with its zero padding, nibble
plane, gaps, block offsets) must equal the oracle's encode byte for byte, and
nothing may be written past the sizes the metadata gives.  Full-size
workloads check decode(encode_device(x)) = x on the GPU, the oracle's total
bit count, and the oracle's decode of sampled blocks from the stored gaps and
block offsets.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import lossless_entropy_coded_ecf8_amd as E
from lossless_entropy_coded_ecf8_amd import binding as B

pytestmark = pytest.mark.gpu

CANARY = 0xA5
PAD = 64

COMPLETE = {
    "uniform4": [4] * 16,
    "fib15": list(range(1, 16)) + [15],
    "long12x6": list(range(1, 10)) + [11] + [12] * 6,
    "two": [1, 1] + [0] * 14,
}


def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def make_input(kind, n, seed):
    rng = np.random.default_rng(seed)
    if kind == "stable":
        return synth.small_stable(max(n, 1), 1.7, seed)[:n], None
    if kind == "single":
        return np.full(n, 0x3B, dtype=np.uint8), None
    if kind == "bytes":
        return synth.random_bytes(n, seed), None
    L = COMPLETE[kind]
    present = [s for s in range(16) if L[s] > 0]
    e = rng.choice(present, n).astype(np.uint8)
    x = ((rng.integers(0, 2, n, dtype=np.uint8) << 7) | (e << 3) | rng.integers(0, 8, n, dtype=np.uint8))
    return x.astype(np.uint8), L


def canary_buffers(meta, d, out_offsets=(0, 0, 0, 0)):
    """Device buffers of meta's sizes inside larger canary-filled allocations, each starting
    out_offsets[i] bytes into its allocation (the ABI's least alignments: stream 4, nibbles 8,
    gaps 4, blk_off 8)."""
    def buf(nbytes, off):
        whole = torch.full((int(nbytes) + PAD + off,), CANARY, dtype=torch.uint8, device=d)
        return whole[off:], whole[off:off + int(nbytes)]
    sizes = [meta.stream_bytes, meta.nibble_bytes, meta.gap_bytes, 8 * (meta.n_blocks + 1)]
    parts = [buf(n, off) for n, off in zip(sizes, out_offsets)]
    enc = B.DeviceEncoded(meta, parts[0][1], parts[1][1], parts[2][1], parts[3][1].view(torch.int64))
    return enc, [p[0] for p in parts]


def encode_on_device(x_np, lengths, C, TB, d, offset=0, out_offsets=(0, 0, 0, 0)):
    """Device encode of x_np (uploaded at byte `offset` of a larger buffer) into canary buffers."""
    n = x_np.size
    up = torch.zeros(n + offset + 16, dtype=torch.uint8, device=d)
    up[offset:offset + n] = torch.from_numpy(np.ascontiguousarray(x_np)).to(d)
    x = up[offset:offset + n]
    ws = B.encode_workspace(n, d)
    freq = B.histogram_device(x, workspace=ws).cpu().numpy()
    if lengths is None:
        lengths = B.codebook_from_freq(freq.astype(np.uint64)) if n else [0] * 16
    m = B.meta_from_freq(freq.astype(np.uint64), n, lengths, C, TB)
    enc, wholes = canary_buffers(m, d, out_offsets)
    B.encode_into(x, enc, ws)
    torch.cuda.synchronize()
    return enc, wholes, freq


def assert_equal_to_oracle(x_np, lengths, C, TB, d, offset=0, out_offsets=(0, 0, 0, 0)):
    enc, wholes, freq = encode_on_device(x_np, lengths, C, TB, d, offset, out_offsets)
    assert np.array_equal(freq.astype(np.uint64), oracle.histogram(x_np).astype(np.uint64))
    ref = oracle.encode(x_np, lengths=lengths, chunk_bytes=C, tb=TB)
    assert int(enc.meta.total_bits) == ref["total_bits"]
    for whole, key in zip(wholes, ["stream", "nibbles", "gaps", "blk_off"]):
        got = whole.cpu().numpy()
        want = np.ascontiguousarray(ref[key]).view(np.uint8)
        k = want.size
        assert (got[k:] == CANARY).all(), "%s: write past the end" % key
        bad = np.nonzero(got[:k] != want)[0]
        assert bad.size == 0, "%s: first mismatch at byte %d of %d" % (key, bad[0], k)
    return enc


EDGE = [("stable", n) for n in (1, 2, 15, 16, 17, 31, 4095, 4096, 4097, 8191, 8193, 16385, 65537, 1_000_003)] + \
       [("uniform4", 8192 * 3), ("fib15", 200_000), ("long12x6", 200_000), ("two", 65536 + 7),
        ("single", 300_000), ("bytes", 123_457)]
PARAMS = [(16, 256), (4, 64), (12, 192), (64, 1024), (8, 128)]


@pytest.mark.parametrize("kind,n", EDGE, ids=lambda v: str(v))
@pytest.mark.parametrize("C,TB", PARAMS, ids=lambda v: str(v))
def test_encode_device_bytes_equal_oracle(kind, n, C, TB):
    d = dev()
    x, L = make_input(kind, n, n + C)
    assert_equal_to_oracle(x, L, C, TB, d)


@pytest.mark.parametrize("n", [4 * 64 * 32, 4 * 64 * 32 - 1, 4 * 64 * 32 + 1, 32, 33])
def test_encode_device_block_aligned_total_bits(n):
    """One present symbol of length 1: T = n lands exactly on chunk and block starts."""
    d = dev()
    L = [0] * 16
    L[7] = 1
    x = (0x38 | (np.arange(n) & 0x87)).astype(np.uint8)
    assert_equal_to_oracle(x, L, 4, 64, d)


@pytest.mark.parametrize("offset", [1, 3, 8])
def test_encode_device_unaligned_input(offset):
    d = dev()
    x, _ = make_input("stable", 100_003, offset)
    assert_equal_to_oracle(x, None, 16, 256, d, offset)


@pytest.mark.parametrize("n", [8192 * 5 + 100, 300_001])
def test_encode_device_outputs_at_least_alignment(n):
    """Stream and gaps 4 bytes, nibbles and blk_off 8 bytes past a 16-byte boundary: the
    encode's 16-byte stores fall back to narrower ones, same bytes."""
    d = dev()
    x, _ = make_input("stable", n, 7)
    assert_equal_to_oracle(x, None, 16, 256, d, out_offsets=(4, 8, 4, 8))
    assert_equal_to_oracle(x, None, 8, 128, d, out_offsets=(12, 8, 4, 8))


def test_encode_device_empty():
    d = dev()
    x = torch.zeros(0, dtype=torch.uint8, device=d)
    enc = E.encode_device(x)
    torch.cuda.synchronize()
    assert enc.n == 0
    assert (enc.stream.cpu().numpy() == 0).all() and int(enc.blk_off[0]) == 0
    assert (E.histogram_device(x).cpu().numpy() == 0).all()


def test_histogram_device_all_byte_values():
    d = dev()
    x = np.tile(np.arange(256, dtype=np.uint8), 1001)
    got = E.histogram_device(torch.from_numpy(x).to(d)).cpu().numpy()
    assert np.array_equal(got, np.full(16, 16 * 1001))


def test_encode_device_matches_host_encoder_and_round_trips():
    d = dev()
    x, _ = make_input("stable", 777_777, 5)
    xd = torch.from_numpy(x).to(d)
    enc = E.encode_device(xd)
    host = E.encode(x)
    torch.cuda.synchronize()
    assert B.meta_dict(enc.meta) == B.meta_dict(host.meta)
    assert np.array_equal(enc.stream.cpu().numpy(), host.stream)
    out = E.decode(enc)
    torch.cuda.synchronize()
    assert torch.equal(out, xd)


@pytest.mark.parametrize("counts_from", ["data", "other"])
def test_encode_device_mismatched_meta_or_counts_stays_in_bounds(counts_from):
    """Metadata (and, for "other", per-tile counts) of other data with fewer bits: the stream comes
    out wrong, but nothing is written past the buffers' sizes."""
    d = dev()
    x, _ = make_input("stable", 50_000, 9)
    L = list(oracle.huffman_lengths(oracle.histogram(x)))
    longest = int(max(L))
    s_long = int(np.argmax(L))
    y = ((x & 0x87) | (s_long << 3)).astype(np.uint8)     # every element the longest code
    m = B.meta_from_freq(oracle.histogram(x).astype(np.uint64), x.size, L, 16, 256)
    assert int(m.total_bits) < longest * x.size
    yd = torch.from_numpy(y).to(d)
    ws_whole = torch.full((E.encode_workspace_bytes(x.size) + PAD,), CANARY, dtype=torch.uint8, device=d)
    ws = ws_whole[:E.encode_workspace_bytes(x.size)]
    B.histogram_device(yd if counts_from == "data" else torch.from_numpy(x).to(d), workspace=ws)
    enc, wholes = canary_buffers(m, d)
    B.encode_into(yd, enc, ws)
    torch.cuda.synchronize()
    for whole, size in zip(wholes + [ws_whole], [m.stream_bytes, m.nibble_bytes, m.gap_bytes, 8 * (m.n_blocks + 1),
                                                 ws.numel()]):
        assert (whole.cpu().numpy()[int(size):] == CANARY).all()


def test_one_histogram_serves_several_encodes():
    """The per-tile counts survive an encode: the same workspace encodes under other codes and params."""
    d = dev()
    x, _ = make_input("stable", 300_001, 4)
    xd = torch.from_numpy(x).to(d)
    ws = B.encode_workspace(x.size, d)
    freq = B.histogram_device(xd, workspace=ws).cpu().numpy().astype(np.uint64)
    for L, C, TB in [(None, 16, 256), ([4] * 16, 4, 64), (None, 12, 192)]:
        L = B.codebook_from_freq(freq) if L is None else L
        m = B.meta_from_freq(freq, x.size, L, C, TB)
        enc = B.encode_into(xd, B.alloc_device(m, d), ws)
        torch.cuda.synchronize()
        ref = oracle.encode(x, lengths=L, chunk_bytes=C, tb=TB)
        assert np.array_equal(enc.stream.cpu().numpy(), ref["stream"])
        assert np.array_equal(enc.gaps.cpu().numpy(), ref["gaps"])
        assert np.array_equal(enc.blk_off.cpu().numpy().view(np.uint64), ref["blk_off"])


BATCH_CASES = [("stable", 100_003, 16, 256), ("stable", 0, 16, 256), ("stable", 1, 4, 64),
               ("fib15", 200_000, 12, 192), ("stable", 8193, 64, 1024), ("two", 65536 + 7, 8, 128),
               ("stable", 4097, 16, 256), ("single", 300_000, 4, 64), ("long12x6", 50_000, 16, 256),
               ("stable", 16385, 8, 128), ("bytes", 123_457, 16, 256), ("uniform4", 8192 * 3, 12, 192),
               ("stable", 31, 64, 1024), ("stable", 1_000_003, 16, 256), ("stable", 2, 16, 256),
               ("fib15", 70_001, 4, 64), ("stable", 8192, 16, 256), ("stable", 0, 8, 128),
               ("stable", 250_000, 16, 256)]


def prepare_job(kind, n, C, TB, seed, d):
    x_np, L = make_input(kind, n, seed)
    x = torch.from_numpy(np.ascontiguousarray(x_np)).to(d)
    ws = B.encode_workspace(max(n, 1), d)
    freq = B.histogram_device(x, workspace=ws).cpu().numpy().astype(np.uint64)
    if L is None:
        L = B.codebook_from_freq(freq) if n else [0] * 16
    m = B.meta_from_freq(freq, n, L, C, TB)
    enc, wholes = canary_buffers(m, d)
    return x_np, L, x, ws, enc, wholes


def check_against_oracle(x_np, L, C, TB, enc, wholes):
    ref = oracle.encode(x_np, lengths=L, chunk_bytes=C, tb=TB)
    assert int(enc.meta.total_bits) == ref["total_bits"]
    for whole, key in zip(wholes, ["stream", "nibbles", "gaps", "blk_off"]):
        got = whole.cpu().numpy()
        want = np.ascontiguousarray(ref[key]).view(np.uint8)
        k = want.size
        assert (got[k:] == CANARY).all(), "%s: write past the end" % key
        bad = np.nonzero(got[:k] != want)[0]
        assert bad.size == 0, "%s: first mismatch at byte %d of %d" % (key, bad[0], k)


def test_encode_batched_bytes_equal_oracle():
    """19 tensors of mixed sizes (two empty), symbol sets and (C, TB) in one batched call (eight
    tensors per set of launches, so three sets): every buffer equals the oracle's encode."""
    d = dev()
    jobs = [prepare_job(kind, n, C, TB, 11 * i + 5, d) for i, (kind, n, C, TB) in enumerate(BATCH_CASES)]
    B.encode_batched_into([j[2] for j in jobs], [j[4] for j in jobs], [j[3] for j in jobs])
    torch.cuda.synchronize()
    for (kind, n, C, TB), (x_np, L, x, ws, enc, wholes) in zip(BATCH_CASES, jobs):
        check_against_oracle(x_np, L, C, TB, enc, wholes)


def test_encode_batched_checks_every_job_first():
    """A misaligned stream in the third job: the call fails and no job's buffers are written."""
    d = dev()
    jobs = [prepare_job("stable", 50_000 + i, 16, 256, i, d) for i in range(4)]
    encs = [j[4] for j in jobs]
    whole = torch.full((int(encs[2].meta.stream_bytes) + PAD + 2,), CANARY, dtype=torch.uint8, device=d)
    encs[2].stream = whole[2:2 + int(encs[2].meta.stream_bytes)]
    with pytest.raises(E.Ecf8Error):
        B.encode_batched_into([j[2] for j in jobs], encs, [j[3] for j in jobs])
    torch.cuda.synchronize()
    for j in jobs:
        for w in j[5]:
            assert (w.cpu().numpy() == CANARY).all()
    assert (whole.cpu().numpy() == CANARY).all()


def test_encode_batched_empty_list():
    dev()
    assert B.encode_batched_into([], [], []) == []


def test_encode_device_rejects_bad_arguments():
    d = dev()
    x = torch.from_numpy(make_input("stable", 10_000, 1)[0]).to(d)
    enc = E.encode_device(x)
    ws = torch.empty(E.encode_workspace_bytes(x.numel()) + 512, dtype=torch.uint8, device=d)
    with pytest.raises(E.Ecf8Error, match="WORKSPACE"):
        B.encode_into(x, enc, workspace=ws[1:])
    with pytest.raises(E.Ecf8Error, match="WORKSPACE"):
        B.encode_into(x, enc, workspace=ws[:E.encode_workspace_bytes(x.numel()) - 1])
    with pytest.raises(E.Ecf8Error, match="WORKSPACE"):
        B.histogram_device(x, workspace=ws[:64])
    bad = B.Meta.from_buffer_copy(enc.meta)
    bad.n_blocks += 1
    enc2 = B.DeviceEncoded(bad, enc.stream, enc.nibbles, enc.gaps, enc.blk_off)
    with pytest.raises(E.Ecf8Error, match="META"):
        B.encode_into(x, enc2, workspace=ws)
    enc3 = B.DeviceEncoded(enc.meta, enc.stream[1:], enc.nibbles, enc.gaps, enc.blk_off)
    with pytest.raises(E.Ecf8Error, match="ARG"):
        B.encode_into(x, enc3, workspace=ws)


# ---------------------------------------------------------------- full-size workload

def test_llama70b_encode_device_round_trip():
    """Every tensor of the 70B-shaped workload: device encode, batched decode = input;
    T equals the oracle's; sampled blocks decode in the oracle from the device gaps and offsets;
    two tensors compared with the oracle's encode byte for byte."""
    d = dev()
    names, xs, encs = [], [], []
    for name, x in synth.workload_tensors("llama70b", device=d):
        names.append(name)
        xs.append(x.reshape(-1))
        encs.append(E.encode_device(x))
    plan = E.DecodePlan(encs)
    plan.run()
    torch.cuda.synchronize()
    assert plan.status() == 0
    rng = np.random.default_rng(2)
    full_checks = {0, len(xs) // 2}
    for i, (name, x, enc) in enumerate(zip(names, xs, encs)):
        assert torch.equal(plan.view(i), x), name
        xh = x.cpu().numpy()
        L = list(enc.meta.cb.len)
        assert np.array_equal(np.asarray(L), oracle.huffman_lengths(oracle.histogram(xh))), name
        stream = enc.stream.cpu().numpy()
        nib = enc.nibbles.cpu().numpy()
        gaps = enc.gaps.cpu().numpy()
        blk = enc.blk_off.cpu().numpy().view(np.uint64)
        C, TB = enc.meta.chunk_bytes, enc.meta.threads_per_block
        for b in sorted({0, int(enc.meta.n_blocks) - 1} | set(int(v) for v in rng.integers(0, enc.meta.n_blocks, 2))):
            t = b * TB
            gap = int(gaps[t >> 1] >> (4 * (t & 1))) & 15
            lo, hi = int(blk[b]), int(blk[b + 1])
            ref, _ = oracle.decode_range(stream, nib, L, 8 * C * t + gap, lo, hi - lo)
            assert np.array_equal(xh[lo:hi], ref), (name, b)
        if i in full_checks:
            ref = oracle.encode(xh, lengths=L, chunk_bytes=C, tb=TB)
            assert int(enc.meta.total_bits) == ref["total_bits"]
            assert np.array_equal(stream, ref["stream"]) and np.array_equal(nib, ref["nibbles"]), name
            assert np.array_equal(gaps, ref["gaps"]) and np.array_equal(blk, ref["blk_off"]), name
