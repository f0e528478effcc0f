"""GPU decode parity: the HIP path (through the C ABI) against the oracle.

Bit-exact is the only bar (integer / byte work).  Small and edge cases compare
every output byte with the oracle's bit-serial decode of the same stream and
with the original input; full-size workloads compare every byte with the
original input on the GPU (decode(encode(x)) = x is the oracle's pinned
property) and, on sampled blocks, with the oracle's own decode.
"""
import os

import numpy as np
import pytest
import torch

import oracle
import synth
import lossless_entropy_coded_ecf8_amd as E
from lossless_entropy_coded_ecf8_amd import binding as B

pytestmark = pytest.mark.gpu

CANARY = 0xA5


def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


COMPLETE = {
    "uniform4": [4] * 16,
    "fib15": list(range(1, 16)) + [15],
    "long12x6": list(range(1, 10)) + [11] + [12] * 6,
    "two": [1, 1] + [0] * 14,
}


def make_input(kind, n, seed):
    rng = np.random.default_rng(seed)
    if kind == "stable":
        return synth.small_stable(max(n, 1), 1.7, seed)[:n], None
    if kind == "gauss":
        return synth.gauss_tensor((n,), 0.02, seed).numpy(), None
    if kind == "single":
        return np.full(n, 0x3B, dtype=np.uint8), None
    if kind == "bytes":
        return synth.random_bytes(n, seed), None
    if kind == "special":
        v = np.array([0x7F, 0xFF, 0x00, 0x80, 0x7E, 0xFE, 0x01, 0x81], dtype=np.uint8)
        return v[rng.integers(0, v.size, n)], None
    L = COMPLETE[kind]
    present = [s for s in range(16) if L[s] > 0]
    e = rng.choice(present, n).astype(np.uint8)
    x = ((rng.integers(0, 2, n, dtype=np.uint8) << 7) | (e << 3) | rng.integers(0, 8, n, dtype=np.uint8))
    return x.astype(np.uint8), L


def decode_with_canaries(enc_host, d):
    n = enc_host.n
    buf = torch.full((n + 64,), CANARY, dtype=torch.uint8, device=d)
    out = buf[16:16 + n]
    E.decode(enc_host.to(d), out=out)
    torch.cuda.synchronize()
    b = buf.cpu().numpy()
    assert (b[:16] == CANARY).all() and (b[16 + n:] == CANARY).all(), "decode wrote outside [0, n)"
    return b[16:16 + n]


SMALL = ([("stable", n) for n in (1, 2, 3, 15, 16, 17, 100, 4095, 4096, 4097, 65535, 65536, 65537, 1_000_003)]
         + [("uniform4", n) for n in (8192, 8193, 8192 * 3, 8192 * 3 - 1)]
         + [("fib15", 200_000), ("long12x6", 200_000), ("two", 100_000), ("two", 65536 + 7),
            ("single", 300_000), ("single", 32768), ("bytes", 123_457), ("special", 50_001),
            ("gauss", 777_777)])


@pytest.mark.parametrize("kind,n", SMALL, ids=lambda v: str(v))
def test_small_and_edge_cases_bit_exact(kind, n):
    d = dev()
    x, L = make_input(kind, n, n)
    enc = E.encode(x, lengths=L)
    got = decode_with_canaries(enc, d)
    ref = oracle.decode(enc.stream, enc.nibbles, n, enc.lengths)
    assert np.array_equal(ref, x)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, "first mismatch at %d of %d (%s)" % (bad[0], n, kind)


SHAPES = [(32, 256), (64, 128), (16, 128), (8, 256), (16, 512)]
SHAPE_CASES = [("stable", 1), ("stable", 4097), ("stable", 1_000_003), ("gauss", 300_001), ("fib15", 200_000),
               ("long12x6", 100_000), ("two", 150_000), ("single", 200_000), ("bytes", 77_777), ("uniform4", 65_536)]


@pytest.mark.parametrize("C,TB", SHAPES, ids=lambda v: str(v))
@pytest.mark.parametrize("kind,n", SHAPE_CASES, ids=lambda v: str(v))
def test_other_shapes_bit_exact(C, TB, kind, n):
    """The decode kernels for other (C, TB) shapes, among them the pages' 64-byte chunks on 128 lanes:
    every byte equals the oracle's decode of the same stream, canaries intact (1-bit codes fill the
    staging; 15-bit codes use the long-code table region; long chunks walk past their records)."""
    d = dev()
    x, L = make_input(kind, n, n + C + TB)
    enc = E.encode(x, lengths=L, chunk_bytes=C, threads_per_block=TB)
    got = decode_with_canaries(enc, d)
    ref = oracle.decode(enc.stream, enc.nibbles, n, enc.lengths)
    assert np.array_equal(ref, x)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, "first mismatch at %d of %d (%s, C=%d, TB=%d)" % (bad[0], n, kind, C, TB)


@pytest.mark.parametrize("C,TB", SHAPES, ids=lambda v: str(v))
def test_other_shapes_batched_and_checked(C, TB):
    """A batched plan of one shape, run twice into a reused buffer; a corrupt gap is flagged exactly as
    the oracle's count step predicts, and contained."""
    d = dev()
    kinds = [("stable", 300_001), ("fib15", 70_000), ("single", 40_000), ("gauss", 1 << 20), ("stable", 5)]
    xs, encs, offs, off = [], [], [], 0
    for i, (k, n) in enumerate(kinds):
        x, L = make_input(k, n, 3000 + i)
        xs.append(x)
        encs.append(E.encode(x, lengths=L, chunk_bytes=C, threads_per_block=TB).to(d))
        offs.append(off)
        off += (n + 15) // 16 * 16 + 16
    out = torch.full((off + 64,), CANARY, dtype=torch.uint8, device=d)
    plan = E.DecodePlan(encs, out=out, offsets=offs)
    for rep in range(2):
        plan.run()
        torch.cuda.synchronize()
        for i, x in enumerate(xs):
            assert np.array_equal(plan.view(i).cpu().numpy(), x), (rep, kinds[i])
    assert plan.status() == 0
    x, _ = make_input("stable", 400_000, 21)
    enc = E.encode(x, chunk_bytes=C, threads_per_block=TB)
    t = TB + 37
    g0 = (int(enc.gaps[t >> 1]) >> (4 * (t & 1))) & 15
    for delta in range(1, 16):
        gaps = enc.gaps.copy()
        g1 = (g0 + delta) % 16
        gaps[t >> 1] = (gaps[t >> 1] & (0xF0 if t % 2 == 0 else 0x0F)) | (g1 << (4 * (t & 1)))
        want_bad = expected_bad_blocks(enc.stream, gaps, enc)
        if want_bad:
            break
    assert want_bad == [1]
    denc = enc.to(d)
    denc.gaps.copy_(torch.from_numpy(gaps).to(d))
    _, bad, buf = decode_plan_with_canaries(denc, d)
    assert bad == 1
    check_contained(buf, x, enc, want_bad)


def test_all_256_byte_values():
    d = dev()
    x = np.tile(np.arange(256, dtype=np.uint8), 1000)
    enc = E.encode(x)
    assert np.array_equal(decode_with_canaries(enc, d), x)


def test_gauss1m_config():
    """1024x1024 N(0, 0.02) tensor, max-abs scaled to 448, RNE E4M3; plain Huffman (max length 16)."""
    d = dev()
    x = synth.make_tensor("gauss1m", "w", (1024, 1024), "gauss", {"std": 0.02}).numpy().ravel()
    enc = E.encode(x)
    assert enc.meta.max_len <= 16
    got = decode_with_canaries(enc, d)
    ref = oracle.decode(enc.stream, enc.nibbles, enc.n, enc.lengths)
    assert np.array_equal(got, ref) and np.array_equal(ref, x)


def test_batched_mixed_tensors_and_buffer_reuse():
    """One dispatch decodes tensors with different codebooks; running it twice is idempotent;
    a second, smaller plan reuses the same output buffer and workspace."""
    d = dev()
    kinds = [("stable", 300_001), ("fib15", 70_000), ("single", 40_000), ("bytes", 99_999),
             ("two", 33_333), ("gauss", 1 << 20), ("stable", 5)]
    xs, encs, offs, off = [], [], [], 0
    for i, (k, n) in enumerate(kinds):
        x, L = make_input(k, n, 1000 + i)
        xs.append(x)
        encs.append(E.encode(x, lengths=L).to(d))
        offs.append(off)
        off += (n + 15) // 16 * 16 + 16 * (i % 3)
    out = torch.full((off + 64,), CANARY, dtype=torch.uint8, device=d)
    ws = torch.empty(E.workspace_bytes(len(encs)), dtype=torch.uint8, device=d)
    plan = E.DecodePlan(encs, out=out, offsets=offs, workspace=ws)
    for rep in range(2):
        plan.run()
        torch.cuda.synchronize()
        for i, x in enumerate(xs):
            assert np.array_equal(plan.view(i).cpu().numpy(), x), (rep, i, kinds[i])
    assert plan.status() == 0
    # second plan: smaller inputs into the same buffer and workspace
    plan2 = E.DecodePlan(encs[:2][::-1], out=out, offsets=[0, (kinds[1][1] + 15) // 16 * 16], workspace=ws)
    plan2.run()
    torch.cuda.synchronize()
    assert np.array_equal(plan2.view(0).cpu().numpy(), xs[1])
    assert np.array_equal(plan2.view(1).cpu().numpy(), xs[0])
    assert plan2.status() == 0


@pytest.mark.parametrize("claim,workgroups", [(2, 7), (3, 5), (5, None), (16, 13), (16, None), (1024, 3),
                                               (2, 1), (40, 64)], ids=lambda v: str(v))
def test_claimed_block_order_bit_exact(claim, workgroups):
    """The claimed block order (ecf8_plan.claim_blocks): tensors with different codebooks, claims
    of 2 to 1024 blocks, grids from 1 workgroup to full (some with more workgroups x claim than
    blocks), three runs into a reused buffer: every byte exact, canaries intact, no block flagged,
    and the claim counters back at zero after each run."""
    d = dev()
    kinds = [("stable", 1_300_001), ("fib15", 70_000), ("single", 40_000), ("bytes", 99_999),
             ("two", 33_333), ("gauss", 1 << 20), ("stable", 5), ("long12x6", 250_000)]
    xs, encs, offs, off = [], [], [], 0
    for i, (k, n) in enumerate(kinds):
        x, L = make_input(k, n, 5000 + i)
        xs.append(x)
        encs.append(E.encode(x, lengths=L).to(d))
        offs.append(off)
        off += (n + 15) // 16 * 16 + 16 * (i % 3)
    out = torch.full((off + 64,), CANARY, dtype=torch.uint8, device=d)
    plan = E.DecodePlan(encs, out=out, offsets=offs, workgroups=workgroups, claim_blocks=claim)
    assert int(plan.plan.claim_blocks) == claim
    for rep in range(3):
        out[:off].fill_(0)
        plan.run()
        torch.cuda.synchronize()
        for i, x in enumerate(xs):
            assert np.array_equal(plan.view(i).cpu().numpy(), x), (rep, i, kinds[i])
        assert (out[off:].cpu().numpy() == CANARY).all()
        assert int(plan.workspace[64:72].cpu().view(torch.int64)[0]) == 0, "claim counters not reset"
    assert plan.status() == 0


def test_claimed_order_on_the_llama70b_block():
    """The Llama-3-70B block (codes limited to 11 bits, as benchmarked) decoded in claims of 16
    blocks (the library keeps this block in the static order), twice: every tensor equals its
    input, sampled blocks equal the oracle's decode."""
    d = dev()
    names, xs, encs = encode_workload("llama70b", d, max_len=11)
    assert E.DecodePlan(encs).plan.claim_blocks == 0
    plan = E.DecodePlan(encs, claim_blocks=16)
    rng = np.random.default_rng(5)
    for rep in range(2):
        plan.out.fill_(CANARY)
        plan.run()
        torch.cuda.synchronize()
        for i, (nm, x) in enumerate(zip(names, xs)):
            assert torch.equal(plan.view(i), x), (rep, nm)
    assert plan.status() == 0
    for i in range(len(encs)):
        sampled_oracle_check(encs[i], plan.view(i), rng, 1)


def test_tables_switched_per_tensor_in_one_dispatch():
    """One dispatch over tensors whose tables differ in size and form (11-bit codes, 12-bit
    codes, 15-bit codes, two symbols, all 4-bit, 11-bit codes again): each workgroup copies the
    table of its next block's tensor into LDS whenever that tensor changes, at several workgroup
    counts (1 workgroup walks every tensor in turn); every tensor decodes exactly and no byte
    outside the tensors' ranges is written."""
    d = dev()
    kinds = [("stable", 500_001), ("long12x6", 300_000), ("fib15", 200_003), ("two", 150_000),
             ("uniform4", 262_144), ("gauss", 400_000)]
    xs, encs, offs, off = [], [], [], 0
    for i, (k, n) in enumerate(kinds):
        x, L = make_input(k, n, 2000 + i)
        xs.append(x)
        encs.append(E.encode(x, lengths=L).to(d))
        offs.append(off)
        off += (n + 15) // 16 * 16 + 32
    inside = np.zeros(off + 64, dtype=bool)
    for o, (_, n) in zip(offs, kinds):
        inside[o:o + n] = True
    for wgs in (None, 37, 1):
        out = torch.full((off + 64,), CANARY, dtype=torch.uint8, device=d)
        plan = E.DecodePlan(encs, out=out, offsets=offs, workgroups=wgs)
        plan.run()
        torch.cuda.synchronize()
        assert plan.status() == 0, wgs
        b = out.cpu().numpy()
        assert (b[~inside] == CANARY).all(), wgs
        for i, x in enumerate(xs):
            assert np.array_equal(b[offs[i]:offs[i] + x.size], x), (kinds[i], wgs)


def reference_table(lengths):
    """The decode table by its definition (ECF8 blog §3.1.2, table-driven decode of a canonical
    code), from the oracle's canonical codes: entry i < p_long stands for the 11-bit window i
    (11 known bits), entry i >= p_long for the 16-bit value i + 31 p_long (16 known bits, the
    region of codewords longer than 11 bits); each entry decodes greedily the whole codewords
    inside its known bits, at most 4, by prefix match.  Entry: 4 * symbols | bits consumed
    (1 when none) << 8 | symbols as nibbles << 16.  p_long = 11-bit prefixes of the codes of at
    most 11 bits; entries = min(65536 - 31 p_long, 2296)."""
    L = [int(v) for v in lengths]
    codes = oracle.canonical_codes(L)
    cw = [(int(codes[s]), L[s], s) for s in range(16) if L[s]]
    p_long = sum(1 << (16 - l) for l in L if 0 < l <= 11) >> 5
    ne = min(65536 - 31 * p_long, 2296)
    table = []
    for i in range(ne):
        v, known = (i << 5, 11) if i < p_long else (i + 31 * p_long, 16)
        pos = ns = sy = 0
        while ns < 4 and pos < known:
            x = (v << pos) & 0xFFFF
            hit = next(((l, s) for c, l, s in cw if x >> (16 - l) == c), None)
            if hit is None or pos + hit[0] > known:
                break
            sy |= hit[1] << (4 * ns)
            ns += 1
            pos += hit[0]
        table.append(4 * ns | max(pos, 1) << 8 | sy << 16)
    return np.array(table, dtype=np.uint32)


def test_decode_tables_match_definition():
    """The table kernel (run by ecf8_decode_prepare) writes, for each tensor of a plan, every
    entry the decode can index exactly as reference_table defines it: codes limited to 11 bits,
    all 4-bit, two 1-bit codes, 12- and 15-bit codewords (the 16-bit region), a single symbol
    (an incomplete code, 2296 entries) and plain Huffman codes of weight-like data.  The
    workspace holds a 256-byte counter, 144 bytes of descriptor per tensor rounded up to 256
    bytes in all, then 9216 bytes of table per tensor."""
    d = dev()
    kinds = [("stable", 11), ("uniform4", 16), ("two", 16), ("long12x6", 16), ("fib15", 16),
             ("single", 16), ("gauss", 16), ("stable", 16)]
    encs, lens = [], []
    for i, (k, ml) in enumerate(kinds):
        x, L = make_input(k, 40_000, 4000 + i)
        h = E.encode(x, lengths=L, max_len=ml) if L is not None else E.encode(x, max_len=ml)
        encs.append(h.to(d))
        lens.append(list(h.lengths))
    plan = E.DecodePlan(encs)
    torch.cuda.synchronize()
    ws = plan.workspace.cpu().numpy()
    off = 256 + (144 * len(encs) + 255) // 256 * 256
    for t, L in enumerate(lens):
        want = reference_table(L)
        got = ws[off + t * 9216: off + t * 9216 + 4 * want.size].view("<u4")
        bad = np.nonzero(got != want)[0]
        assert bad.size == 0, (kinds[t], L, bad[:5], got[bad[:5]], want[bad[:5]])
    # and the plan decodes every tensor exactly with those tables
    plan.run()
    assert plan.status() == 0


def test_status_counts_until_read():
    """The block-check counter adds over runs and restarts when read: two runs on a corrupt
    offset report twice one run's count, the next read reports 0."""
    d = dev()
    x, _ = make_input("stable", 400_000, 2100)
    enc = E.encode(x)
    denc = enc.to(d)
    denc.blk_off[1] += 5
    plan = E.DecodePlan([denc])
    plan.run()
    one = plan.status()
    assert one >= 1
    assert plan.status() == 0
    plan.run()
    plan.run()
    assert plan.status() == 2 * one
    assert plan.status() == 0


def test_short_code_form_selection_and_parity():
    """The plan picks the one-shift table index (short_codes) exactly when every tensor's code is
    complete with no codeword longer than 11 bits; both forms decode every tensor exactly."""
    d = dev()
    cases = [("stable", 400_001, 11),      # 0: codes limited to 11 bits
             ("gauss", 300_000, 11),       # 1: codes limited to 11 bits
             ("uniform4", 262_147, 16),    # 2: all 4 bits
             ("fib15", 200_000, 16),       # 3: codewords of 15 bits
             ("single", 70_000, 16),       # 4: one symbol, an incomplete code
             ("stable", 300_000, 16)]      # 5: the same kind of data with 13-bit codes
    xs, hosts, encs = [], [], []
    for i, (k, n, ml) in enumerate(cases):
        x, L = make_input(k, n, 3000 + i)
        xs.append(x)
        hosts.append(E.encode(x, lengths=L, max_len=ml))
        encs.append(hosts[-1].to(d))
    for i in (0, 1, 2):
        assert max(hosts[i].lengths) <= 11 and oracle.kraft_sum(hosts[i].lengths) == 1.0
    assert max(hosts[3].lengths) > 11 and max(hosts[5].lengths) > 11
    for batch, want_short in (([0, 1, 2], 1), ([0, 1, 2, 3], 0), ([4], 0), ([5], 0), ([2, 5, 0], 0)):
        plan = E.DecodePlan([encs[i] for i in batch])
        assert int(plan.plan.short_codes) == want_short, batch
        plan.out.fill_(CANARY)
        plan.run()
        torch.cuda.synchronize()
        assert plan.status() == 0
        for j, i in enumerate(batch):
            assert np.array_equal(plan.view(j).cpu().numpy(), xs[i]), (batch, i)


def test_short_code_form_refuses_long_codes():
    """A plan forced to the short form on a code with longer codewords decodes nothing wrong
    silently: every block is flagged and no byte outside the tensor is written."""
    d = dev()
    x, L = make_input("long12x6", 300_000, 3020)
    denc = E.encode(x, lengths=L).to(d)
    n = x.size
    buf = torch.full((n + 64,), CANARY, dtype=torch.uint8, device=d)
    plan = E.DecodePlan([denc], out=buf[16:16 + n], offsets=[0])
    assert int(plan.plan.short_codes) == 0
    plan.plan.short_codes = 1
    plan.run()
    assert plan.status() == int(plan.plan.total_blocks)
    b = buf.cpu().numpy()
    assert (b[:16] == CANARY).all() and (b[16 + n:] == CANARY).all()


def test_decode_run_with_dispatch_events():
    """ecf8_decode_run_timed: the same decode, with the events attached to the dispatch holding
    its start and end (a positive duration, no longer than events recorded around the launch)."""
    d = dev()
    x, _ = make_input("stable", 2_000_003, 3030)
    plan = E.DecodePlan([E.encode(x, max_len=11).to(d)])
    plan.out.fill_(CANARY)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    o0, o1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for ev in (a, b):
        ev.record()
    o0.record()
    plan.run(events=(a, b))
    o1.record()
    torch.cuda.synchronize()
    assert plan.status() == 0
    assert np.array_equal(plan.view(0).cpu().numpy(), x)
    inner, outer = a.elapsed_time(b), o0.elapsed_time(o1)
    assert 0 < inner <= outer * 1.001 + 1e-3, (inner, outer)


def test_corrupt_block_offset_is_flagged_and_contained():
    """Checked mode: a wrong blk_off entry is reported, and no byte outside [0, n) is written."""
    d = dev()
    x, _ = make_input("stable", 400_000, 7)
    enc = E.encode(x)
    assert enc.meta.n_blocks >= 3
    denc = enc.to(d)
    denc.blk_off[1] += 5
    n = enc.n
    buf = torch.full((n + 64,), CANARY, dtype=torch.uint8, device=d)
    plan = E.DecodePlan([denc], out=buf[16:16 + n], offsets=[0])
    plan.run()
    assert plan.status() >= 1
    b = buf.cpu().numpy()
    assert (b[:16] == CANARY).all() and (b[16 + n:] == CANARY).all()
    # blocks untouched by the corruption still decode exactly
    lo2 = int(enc.blk_off[2])
    assert np.array_equal(b[16 + lo2:16 + n], x[lo2:])


def decode_plan_with_canaries(denc, d):
    """Run a one-tensor plan into a canary-guarded buffer; returns (plan, host bytes of the buffer)."""
    n = denc.n
    buf = torch.full((n + 64,), CANARY, dtype=torch.uint8, device=d)
    plan = E.DecodePlan([denc], out=buf[16:16 + n], offsets=[0])
    plan.run()
    bad = plan.status()
    return plan, bad, buf


def expected_bad_blocks(stream, gaps, enc):
    """Blocks whose count-step total (oracle, from the stored gaps) disagrees with blk_off."""
    m = enc.meta
    bc = oracle.block_counts(stream, gaps, int(m.total_bits), enc.lengths, int(m.chunk_bytes),
                             int(m.threads_per_block), int(m.n_blocks))
    want = np.diff(enc.blk_off.astype(np.int64))
    return [b for b, c in enumerate(bc) if c is None or c != want[b]]


def check_contained(buf, x, enc, bad_blocks):
    """Canaries intact; every block outside bad_blocks decodes exactly."""
    n = x.size
    b = buf.cpu().numpy()
    assert (b[:16] == CANARY).all() and (b[16 + n:] == CANARY).all(), "decode wrote outside [0, n)"
    blk = enc.blk_off.astype(np.int64)
    for k in range(int(enc.meta.n_blocks)):
        if k not in bad_blocks:
            assert np.array_equal(b[16 + blk[k]:16 + blk[k + 1]], x[blk[k]:blk[k + 1]]), ("block", k)


def test_corrupt_gap_is_flagged_and_contained():
    """Checked mode (ECF8 blog §5.3: wrong output -> check the gap synchronisation): a corrupted gap
    nibble desynchronises one lane's walk.  The blocks the device flags are exactly those whose
    count-step totals, recomputed by the oracle from the corrupted gaps, disagree with blk_off; nothing
    is written outside [0, n); every other block decodes exactly."""
    d = dev()
    x, _ = make_input("stable", 400_000, 11)
    enc = E.encode(x)
    TB = int(enc.meta.threads_per_block)
    assert enc.meta.n_blocks >= 4
    for t in (TB + 37, 2 * TB + 200):
        g0 = (int(enc.gaps[t >> 1]) >> (4 * (t & 1))) & 15
        for delta in range(1, 16):
            gaps = enc.gaps.copy()
            g1 = (g0 + delta) % 16
            gaps[t >> 1] = (gaps[t >> 1] & (0xF0 if t % 2 == 0 else 0x0F)) | (g1 << (4 * (t & 1)))
            want_bad = expected_bad_blocks(enc.stream, gaps, enc)
            if want_bad:
                break
        assert want_bad == [t // TB]
        denc = enc.to(d)
        denc.gaps.copy_(torch.from_numpy(gaps).to(d))
        plan, bad, buf = decode_plan_with_canaries(denc, d)
        assert bad == len(want_bad), (t, g0, g1)
        check_contained(buf, x, enc, want_bad)


def test_corrupt_stream_byte_is_flagged_and_contained():
    """A corrupted stream byte (a complete code: every bit string still parses) changes the codewords
    one or two lanes find; the device flags exactly the blocks whose oracle count-step totals change,
    writes nothing outside [0, n), and decodes every other block exactly.  A later run on the repaired
    stream reports no corrupt block (the counter restarts with every run)."""
    d = dev()
    x, _ = make_input("stable", 400_000, 12)
    enc = E.encode(x)
    C, TB = int(enc.meta.chunk_bytes), int(enc.meta.threads_per_block)
    for pos in (C * TB + 16 * 5 + 3, 3 * C * TB + 16 * 100 + 9):
        for flip in (0x01, 0x10, 0x80, 0xFF, 0x5A):
            stream = enc.stream.copy()
            stream[pos] ^= flip
            want_bad = expected_bad_blocks(stream, enc.gaps, enc)
            if want_bad:
                break
        assert want_bad == [pos // (C * TB)]
        denc = enc.to(d)
        denc.stream.copy_(torch.from_numpy(stream).to(d))
        plan, bad, buf = decode_plan_with_canaries(denc, d)
        assert bad == len(want_bad), (pos, flip)
        check_contained(buf, x, enc, want_bad)
        denc.stream.copy_(torch.from_numpy(enc.stream).to(d))
        plan.run()
        assert plan.status() == 0
        assert np.array_equal(buf.cpu().numpy()[16:16 + x.size], x)


def test_corrupt_single_symbol_stream_is_flagged_and_contained():
    """The one incomplete code that validates (a single symbol, code '0'): a 1 bit in its stream is no
    codeword.  The decode table maps it to an entry that consumes the bit and decodes nothing, so the
    walk ends, the chunk counts one codeword fewer and the block is flagged; nothing is written outside
    [0, n) and the other blocks decode exactly."""
    d = dev()
    n = 300_000
    x, _ = make_input("single", n, 3)
    enc = E.encode(x)
    C, TB = int(enc.meta.chunk_bytes), int(enc.meta.threads_per_block)
    assert enc.meta.n_blocks >= 3 and sum(1 for l in enc.lengths if l) == 1
    stream = enc.stream.copy()
    stream[C * TB + 777] |= 0x08                     # one bit, block 1
    stream[2 * C * TB + 5] = 0xFF                    # eight bits, block 2
    denc = enc.to(d)
    denc.stream.copy_(torch.from_numpy(stream).to(d))
    plan, bad, buf = decode_plan_with_canaries(denc, d)
    assert bad == 2
    check_contained(buf, x, enc, [1, 2])


def test_out_buffer_checks():
    """The binding rejects an output buffer that is too small, not uint8, or whose ranges overlap, and a
    single-tensor decode whose output size is not n."""
    d = dev()
    x, _ = make_input("stable", 10_000, 13)
    e = E.encode(x).to(d)
    with pytest.raises(ValueError):
        E.DecodePlan([e], out=torch.empty(x.size - 1, dtype=torch.uint8, device=d), offsets=[0])
    with pytest.raises(ValueError):
        E.DecodePlan([e], out=torch.empty(x.size, dtype=torch.int16, device=d), offsets=[0])
    with pytest.raises(ValueError):
        E.DecodePlan([e, e], out=torch.empty(3 * x.size, dtype=torch.uint8, device=d), offsets=[0, x.size - 16])
    with pytest.raises(E.Ecf8Error) as ei:
        E.decode(e, out=torch.empty(x.size + 16, dtype=torch.uint8, device=d))
    assert ei.value.code == -2


def test_unsupported_and_misaligned_arguments():
    d = dev()
    x, _ = make_input("stable", 10_000, 8)
    e12 = E.encode(x, chunk_bytes=12).to(d)
    with pytest.raises(E.Ecf8Error) as ei:
        E.decode(e12)
    assert ei.value.code == -4
    # tensors of two supported shapes in one batch
    e8 = E.encode(x, chunk_bytes=8).to(d)
    with pytest.raises(E.Ecf8Error) as ei:
        E.DecodePlan([E.encode(x).to(d), e8])
    assert ei.value.code == -4
    e16 = E.encode(x).to(d)
    buf = torch.empty(x.size + 32, dtype=torch.uint8, device=d)
    with pytest.raises(E.Ecf8Error) as ei:
        E.decode(e16, out=buf[1:1 + x.size])
    assert ei.value.code == -1
    small_ws = torch.empty(64, dtype=torch.uint8, device=d)
    # the binding would replace an undersized workspace, so call the ABI directly
    s = e16.c_stream()
    m = e16.meta
    import ctypes
    rc = B.lib().ecf8_decode(ctypes.byref(s), ctypes.byref(m), ctypes.c_void_p(buf.data_ptr()), e16.n,
                             ctypes.c_void_p(small_ws.data_ptr()), 64, ctypes.c_void_p(0))
    assert rc == -7


def test_empty_tensor_is_a_no_op():
    d = dev()
    enc = E.encode(np.zeros(0, dtype=np.uint8)).to(d)
    out = torch.full((16,), CANARY, dtype=torch.uint8, device=d)
    E.decode(enc, out=out[:0])
    torch.cuda.synchronize()
    assert (out.cpu().numpy() == CANARY).all()


# ---------------------------------------------------------------- full-size workloads

def encode_workload(workload, d, experts=None, max_len=16):
    """Generate on the GPU, encode on the host, upload.  Returns (names, xs_gpu, device encs)."""
    names, xs, encs = [], [], []
    for name, x in synth.workload_tensors(workload, device=d, experts=experts):
        names.append(name)
        xs.append(x.reshape(-1))
        encs.append(E.encode(x.cpu(), max_len=max_len).to(d))
    return names, xs, encs


def sampled_oracle_check(enc_dev, out_view, rng, blocks=2):
    """Decode a few whole blocks with the oracle from the library's stream and compare."""
    m = enc_dev.meta
    stream = enc_dev.stream.cpu().numpy()
    nib = enc_dev.nibbles.cpu().numpy()
    gaps = enc_dev.gaps.cpu().numpy()
    blk = enc_dev.blk_off.cpu().numpy().view(np.uint64)
    L = list(m.cb.len)
    picks = {0, int(m.n_blocks) - 1} | set(int(v) for v in rng.integers(0, m.n_blocks, blocks))
    C, TB = m.chunk_bytes, m.threads_per_block
    for b in sorted(picks):
        t = b * TB
        gap = int(gaps[t >> 1] >> (4 * (t & 1))) & 15
        lo, hi = int(blk[b]), int(blk[b + 1])
        ref, _ = oracle.decode_range(stream, nib, L, 8 * C * t + gap, lo, hi - lo)
        assert np.array_equal(out_view[lo:hi].cpu().numpy(), ref), ("block", b)


def run_batched(workload, experts=None, check_blocks=2, max_len=16):
    d = dev()
    names, xs, encs = encode_workload(workload, d, experts, max_len)
    plan = E.DecodePlan(encs)
    plan.out.fill_(CANARY)
    plan.run()
    torch.cuda.synchronize()
    assert plan.status() == 0
    rng = np.random.default_rng(0)
    for i, (nm, x) in enumerate(zip(names, xs)):
        v = plan.view(i)
        assert torch.equal(v, x), nm
        if check_blocks:
            sampled_oracle_check(encs[i], v, rng, check_blocks)
    return plan


def test_llama8b_one_launch_per_tensor():
    d = dev()
    rng = np.random.default_rng(1)
    for name, x in synth.workload_tensors("llama8b", device=d):
        enc = E.encode(x.cpu()).to(d)
        out = E.decode(enc)
        torch.cuda.synchronize()
        assert torch.equal(out, x.reshape(-1)), name
        sampled_oracle_check(enc, out, rng)


def test_llama70b_block_batched():
    run_batched("llama70b")


def test_llama70b_block_batched_short_codes():
    """The block with codes limited to 11 bits (the bench's encoding): the one-shift form."""
    plan = run_batched("llama70b", max_len=11)
    assert int(plan.plan.short_codes) == 1


def test_dit14b_block_batched():
    run_batched("dit14b")


def test_moe_routed_experts_batched():
    run_batched("moe256", experts=synth.moe_routing(), check_blocks=1)


@pytest.mark.slow
def test_moe_full_layer_batched():
    """All 256 experts (11.27 G elements, > 2^32) in one dispatch into one 11.3 GB buffer."""
    if os.environ.get("ECF8_SKIP_FULL_MOE"):
        pytest.skip("ECF8_SKIP_FULL_MOE set")
    d = dev()
    names, xs, encs = encode_workload("moe256", d)
    plan = E.DecodePlan(encs)
    assert plan.out.numel() > 2 ** 32
    # a dispatch this long (515 blocks per workgroup) takes the claimed block order; two runs, the
    # second from the counters
    # the first left at zero
    assert int(plan.plan.claim_blocks) == 4
    for rep in range(2):
        plan.run()
    torch.cuda.synchronize()
    assert plan.status() == 0
    rng = np.random.default_rng(3)
    for i, (name, x) in enumerate(zip(names, xs)):
        assert torch.equal(plan.view(i), x), name
        if i % 97 == 0:
            sampled_oracle_check(encs[i], plan.view(i), rng, 1)
