"""Pins for the CPU oracle against facts the pages and mathematics fix.

Each test names what it pins.  None of them re-types the oracle's own code:
they use closed forms, a published worked example (RFC 1951 §3.2.2), brute
force over all prefix codes on tiny alphabets, and an independent bit-string
construction of the stream in Python.
"""
import itertools
import math
import os

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def load_rfc1951():
    rows = []
    with open(os.path.join(GOLDEN, "rfc1951_canonical.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            s, l, c = line.split()
            rows.append((int(s), int(l), int(c, 2)))
    return rows


def python_bits(x, lengths, codes):
    """Independent stream construction: concatenate binary strings, MSB first."""
    e = (np.asarray(x, dtype=np.uint8) >> 3) & 15
    return "".join(format(int(codes[s]), "0%db" % int(lengths[s])) for s in e)


def pack_msb_first(bits: str, nbytes: int) -> np.ndarray:
    out = np.zeros(nbytes, dtype=np.uint8)
    for k, ch in enumerate(bits):
        if ch == "1":
            out[k // 8] |= 1 << (7 - k % 8)
    return out


def make_bytes(exps, signs=None, mants=None, seed=0):
    rng = np.random.default_rng(seed)
    exps = np.asarray(exps, dtype=np.uint8)
    s = rng.integers(0, 2, exps.size, dtype=np.uint8) if signs is None else np.asarray(signs, np.uint8)
    m = rng.integers(0, 8, exps.size, dtype=np.uint8) if mants is None else np.asarray(mants, np.uint8)
    return ((s << 7) | (exps << 3) | m).astype(np.uint8)


# ---------------------------------------------------------------- codebook

def test_canonical_codes_rfc1951_example():
    """Canonical assignment equals the RFC 1951 §3.2.2 worked example."""
    rows = load_rfc1951()
    L = np.zeros(16, dtype=np.int64)
    for s, l, _ in rows:
        L[s] = l
    codes = oracle.canonical_codes(L)
    for s, l, c in rows:
        assert codes[s] == c, (s, l, codes[s], c)


def test_histogram_counts_exponent_field():
    x = make_bytes([3, 3, 0, 15, 7, 3], seed=1)
    f = oracle.histogram(x)
    assert f.tolist() == [1, 0, 0, 3, 0, 0, 0, 1, 0, 0, 0, 0, 0, 0, 0, 1]


def test_uniform_gives_all_length_4():
    """Closed form: equal frequencies over 16 symbols -> a complete code of depth 4."""
    L = oracle.huffman_lengths([100] * 16)
    assert L.tolist() == [4] * 16
    assert oracle.canonical_codes(L).tolist() == list(range(16))


def test_dyadic_lengths_and_average_equals_entropy():
    """Closed form: p = (1/2, 1/4, ..., 2^-15, 2^-15) -> lengths 1..15,15, average = H."""
    freq = [2 ** (14 - k) for k in range(15)] + [1]       # sums to 2^15: exactly dyadic
    L = oracle.huffman_lengths(freq)
    assert L.tolist() == list(range(1, 16)) + [15]
    H = oracle.entropy_bits(freq)
    assert abs(oracle.average_length(freq, L) - H) < 1e-12
    assert max(L) <= 16                                    # ECF8 blog §3.1.1 length limit


def test_single_and_empty_alphabet():
    L = oracle.huffman_lengths([0] * 5 + [42] + [0] * 10)
    assert L.tolist() == [0] * 5 + [1] + [0] * 10
    assert oracle.huffman_lengths([0] * 16).tolist() == [0] * 16


def brute_force_min_cost(freq):
    """Minimum sum f_i * l_i over all length vectors satisfying Kraft (<= 1)."""
    k = len(freq)
    best = None
    for ls in itertools.product(range(1, k + 1), repeat=k):
        if sum(2.0 ** -l for l in ls) <= 1.0 + 1e-12:
            c = sum(f * l for f, l in zip(freq, ls))
            best = c if best is None else min(best, c)
    return best


@pytest.mark.parametrize("seed", range(40))
def test_huffman_is_optimal_bruteforce(seed):
    """Brute force over every prefix code on alphabets of <= 6 symbols (random and tie-heavy)."""
    rng = np.random.default_rng(seed)
    k = int(rng.integers(2, 7))
    if seed % 3 == 0:
        freq_k = rng.integers(1, 4, k).tolist()            # many ties
    else:
        freq_k = rng.integers(1, 1000, k).tolist()
    syms = sorted(rng.choice(16, k, replace=False).tolist())
    freq = [0] * 16
    for s, f in zip(syms, freq_k):
        freq[s] = f
    L = oracle.huffman_lengths(freq)
    cost = sum(freq[s] * L[s] for s in range(16))
    assert cost == brute_force_min_cost(freq_k)
    assert abs(oracle.kraft_sum(L) - 1.0) < 1e-12           # complete code
    assert all(L[s] == 0 for s in range(16) if freq[s] == 0)


@pytest.mark.parametrize("seed", range(20))
def test_kraft_maxlen_and_length_bounds(seed):
    """Kraft equality, max length <= 16, H <= average < H + 1 on random histograms."""
    rng = np.random.default_rng(100 + seed)
    freq = (rng.pareto(1.0 + seed / 10, 16) * 1000).astype(np.int64)
    freq[rng.random(16) < 0.2] = 0
    if (freq > 0).sum() < 2:
        freq[:2] = [5, 7]
    L = oracle.huffman_lengths(freq)
    assert abs(oracle.kraft_sum(L) - 1.0) < 1e-12
    assert max(L) <= 16
    H = oracle.entropy_bits(freq)
    avg = oracle.average_length(freq, L)
    assert H - 1e-12 <= avg < H + 1


def test_codes_prefix_free_on_skewed_histogram():
    freq = [1, 1, 2, 3, 5, 8, 13, 21, 34, 55, 89, 144, 233, 377, 610, 987]  # Fibonacci: deepest tree
    L = oracle.huffman_lengths(freq)
    assert max(L) == 15
    C = oracle.canonical_codes(L)
    words = [format(int(C[s]), "0%db" % int(L[s])) for s in range(16)]
    for a, b in itertools.permutations(words, 2):
        assert not b.startswith(a)


# ---------------------------------------------------------------- encoder

def test_uniform_stream_is_packed_exponents():
    """Closed form: with all lengths 4, the MSB-first stream is the exponent
    fields packed two per byte, first element in the high nibble."""
    x = make_bytes(np.arange(64) % 16, seed=2)
    enc = oracle.encode(x, lengths=[4] * 16, chunk_bytes=4, tb=64)
    e = (x >> 3) & 15
    expect = (e[0::2] << 4) | e[1::2]
    assert enc["total_bits"] == 4 * x.size
    assert np.array_equal(enc["stream"][: x.size // 2], expect)
    assert not enc["stream"][x.size // 2:].any()


def test_nibble_plane_layout():
    """Sign and mantissa as (s << 3) | m, element j in byte j/2, low nibble for even j."""
    x = np.array([0b1_0101_011, 0b0_0011_110, 0b1_1111_111], dtype=np.uint8)
    enc = oracle.encode(x, chunk_bytes=4, tb=64)
    assert enc["nibbles"][0] == ((0b0110 << 4) | 0b1011)
    assert enc["nibbles"][1] == 0b1111
    assert not enc["nibbles"][2:].any()
    assert enc["nibble_bytes"] == 8


@pytest.mark.parametrize("seed", range(12))
def test_stream_matches_bitstring_construction(seed):
    """The oracle's bit writer agrees with an independent string-based construction."""
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 3000))
    x = synth.small_stable(n, 1.5 + 0.05 * seed, seed) if seed % 2 else synth.random_bytes(n, seed)
    enc = oracle.encode(x, chunk_bytes=8, tb=64)
    L = enc["lengths"]
    bits = python_bits(x, L, oracle.canonical_codes(L))
    assert len(bits) == enc["total_bits"]
    assert np.array_equal(enc["stream"], pack_msb_first(bits, enc["stream_bytes"]))


def brute_force_layout(x, lengths, C, TB):
    e = (np.asarray(x) >> 3) & 15
    lens = np.asarray(lengths)[e]
    starts = np.concatenate([[0], np.cumsum(lens)[:-1]]) if len(e) else np.zeros(0, np.int64)
    T = int(lens.sum())
    nc = -(-T // (8 * C))
    nb = -(-nc // TB)
    gaps = []
    for t in range(nb * TB):
        s = 8 * C * t
        if s >= T:
            gaps.append(0)
            continue
        cand = [p for p in starts if p >= s] + [T]
        gaps.append(min(cand) - s)
    blk = [int((starts < 8 * C * TB * b).sum()) for b in range(nb)] + [len(e)]
    return gaps, blk


@pytest.mark.parametrize("seed", range(10))
def test_gaps_and_block_offsets_by_definition(seed):
    """gap_t and blk_off_b recomputed by brute force from codeword starts."""
    rng = np.random.default_rng(50 + seed)
    n = int(rng.integers(1, 2500))
    x = synth.small_stable(n, 1.6, seed) if seed % 3 else synth.random_bytes(n, seed)
    C, TB = [(4, 64), (8, 64), (16, 64)][seed % 3]
    enc = oracle.encode(x, chunk_bytes=C, tb=TB)
    gaps, blk = brute_force_layout(x, enc["lengths"], C, TB)
    g = enc["gaps"]
    stored = [(g[t >> 1] >> (4 * (t & 1))) & 15 for t in range(len(gaps))]
    assert all(0 <= v <= 15 for v in gaps)
    assert stored == gaps
    assert enc["blk_off"].tolist() == blk
    assert oracle.check_layout(enc["stream"], n, enc["total_bits"], enc["lengths"], C, TB,
                               enc["gaps"], enc["blk_off"]) == 0


def set_gap(gaps, t, v):
    g = gaps.copy()
    g[t >> 1] = (g[t >> 1] & (0xF0 if t % 2 == 0 else 0x0F)) | (v << (4 * (t & 1)))
    return g


def test_check_layout_reports_the_first_corrupt_gap_and_offset():
    """oracle.check_layout names what it finds: t + 1 for a stored gap that is not the offset of chunk
    t's first codeword start (an interior chunk, a block's first chunk, a chunk past T), and -(b + 1) for
    a block offset that is not the count of codewords before block b (an interior and the final one)."""
    x = synth.small_stable(30_000, 1.7, 21)
    C, TB = 4, 64
    enc = oracle.encode(x, chunk_bytes=C, tb=TB)
    n, T, L = x.size, enc["total_bits"], enc["lengths"]
    assert enc["n_blocks"] >= 4 and enc["n_blocks"] * TB > enc["n_chunks"]
    chk = lambda gaps, blk: oracle.check_layout(enc["stream"], n, T, L, C, TB, gaps, blk)
    assert chk(enc["gaps"], enc["blk_off"]) == 0
    gaps_bf, _ = brute_force_layout(x, L, C, TB)
    for t in (5, 2 * TB, 3 * TB + 17, enc["n_chunks"] - 1, enc["n_blocks"] * TB - 1):
        bad = (gaps_bf[t] + 1) % 16
        assert chk(set_gap(enc["gaps"], t, bad), enc["blk_off"]) == t + 1, t
    for b in (1, 2, enc["n_blocks"]):
        blk = enc["blk_off"].copy()
        blk[b] += 1
        assert chk(enc["gaps"], blk) == -(b + 1), b
    # with both corrupt, the walk meets the earlier one first
    blk = enc["blk_off"].copy()
    blk[3] -= 1
    assert chk(set_gap(enc["gaps"], 3 * TB + 17, (gaps_bf[3 * TB + 17] + 3) % 16), blk) == -(3 + 1)


@pytest.mark.parametrize("seed", range(4))
def test_chunk_counts_by_definition(seed):
    """The count step from stored gaps (oracle.chunk_count) equals, per chunk, the number of codeword
    starts in [8Ct, min(8C(t+1), T)) counted by brute force; per block the counts sum to the block-offset
    difference.  A gap moved off its codeword changes the count the way a bit walk from there does."""
    rng = np.random.default_rng(90 + seed)
    n = int(rng.integers(500, 6000))
    x = synth.small_stable(n, 1.5 + 0.1 * seed, seed) if seed % 2 else synth.random_bytes(n, seed)
    C, TB = [(4, 64), (8, 64)][seed % 2]
    enc = oracle.encode(x, chunk_bytes=C, tb=TB)
    L = enc["lengths"]
    e = (x >> 3) & 15
    lens = np.asarray(L)[e]
    starts = np.concatenate([[0], np.cumsum(lens)[:-1]])
    T = enc["total_bits"]
    gaps = [(int(enc["gaps"][t >> 1]) >> (4 * (t & 1))) & 15 for t in range(enc["n_blocks"] * TB)]
    for t in range(enc["n_blocks"] * TB):
        lo, hi = 8 * C * t, min(8 * C * (t + 1), T)
        want = int(((starts >= lo) & (starts < hi)).sum()) if lo < T else 0
        assert oracle.chunk_count(enc["stream"], T, L, C, t, gaps[t]) == want, t
    bc = oracle.block_counts(enc["stream"], enc["gaps"], T, L, C, TB, enc["n_blocks"])
    assert bc == np.diff(enc["blk_off"].astype(np.int64)).tolist()
    # a gap one codeword later: one fewer codeword counted in that chunk
    t = next(t for t in range(1, enc["n_chunks"] - 1)
             if gaps[t] + int(lens[np.searchsorted(starts, 8 * C * t + gaps[t])]) < 16
             and 8 * C * t + gaps[t] + int(lens[np.searchsorted(starts, 8 * C * t + gaps[t])]) < 8 * C * (t + 1))
    j = int(np.searchsorted(starts, 8 * C * t + gaps[t]))
    c0 = oracle.chunk_count(enc["stream"], T, L, C, t, gaps[t])
    assert oracle.chunk_count(enc["stream"], T, L, C, t, gaps[t] + int(lens[j])) == c0 - 1


def test_sentinel_gap_for_chunk_without_codeword_start():
    """A last chunk that holds only the tail of the final codeword gets gap = T - 8Ct."""
    # lengths: symbol 0 -> 1 bit, symbol 1 -> 2 bits, symbol 2,3 -> 3 bits ... craft T = 33
    L = [1, 2, 3, 3] + [0] * 12
    exps = [0] * 30 + [2]          # 30 bits + one 3-bit code starting at bit 30 -> T = 33
    x = make_bytes(exps, seed=3)
    enc = oracle.encode(x, lengths=L, chunk_bytes=4, tb=64)    # chunk = 32 bits
    assert enc["total_bits"] == 33
    assert enc["n_chunks"] == 2
    g = enc["gaps"]
    assert (g[0] & 15) == 0
    assert (g[0] >> 4) == 1        # chunk 1 starts at 32; no start >= 32 before T = 33
    gaps, _ = brute_force_layout(x, L, 4, 64)
    assert gaps[1] == 1


# ---------------------------------------------------------------- decoder

@pytest.mark.parametrize("seed", range(16))
def test_round_trip_bit_exact(seed):
    """ECF8 paper abstract / blog §1: decode(encode(x)) == x byte for byte."""
    rng = np.random.default_rng(seed)
    n = int(rng.integers(0, 5000))
    kind = seed % 4
    if kind == 0:
        x = synth.random_bytes(n, seed)
    elif kind == 1:
        x = synth.small_stable(max(n, 1), 1.5 + seed / 40, seed)[:n]
    elif kind == 2:
        x = np.full(n, 0x38 if seed % 8 == 2 else 0x00, dtype=np.uint8)   # single symbol
    else:
        x = np.arange(n, dtype=np.uint8)                                    # every byte value
    enc = oracle.encode(x, chunk_bytes=16, tb=64)
    out = oracle.decode(enc["stream"], enc["nibbles"], n, enc["lengths"])
    assert np.array_equal(out, x)


def test_round_trip_special_bytes():
    """NaN (0x7F, 0xFF), +-0, max normal and subnormals pass through as data."""
    x = np.array([0x7F, 0xFF, 0x00, 0x80, 0x7E, 0xFE, 0x01, 0x81, 0x07, 0x87] * 37, dtype=np.uint8)
    enc = oracle.encode(x, chunk_bytes=4, tb=64)
    assert np.array_equal(oracle.decode(enc["stream"], enc["nibbles"], x.size, enc["lengths"]), x)


def test_decoder_reads_independently_built_stream():
    """Decode a stream built by the Python bit-string construction (not the oracle encoder)."""
    x = synth.small_stable(4000, 1.7, 9)
    L = oracle.huffman_lengths(oracle.histogram(x))
    bits = python_bits(x, L, oracle.canonical_codes(L))
    stream = pack_msb_first(bits, (len(bits) + 7) // 8 + 16)
    nib = np.zeros((x.size + 1) // 2, dtype=np.uint8)
    for j, b in enumerate(x):
        nib[j // 2] |= (((b >> 7) << 3) | (b & 7)) << (4 * (j % 2))
    assert np.array_equal(oracle.decode(stream, nib, x.size, L), x)


def test_decode_range_from_block_offset():
    """Decoding from a block boundary (gap of its first chunk) reproduces that block."""
    x = synth.small_stable(20000, 1.8, 4)
    C, TB = 4, 64
    enc = oracle.encode(x, chunk_bytes=C, tb=TB)
    for b in range(enc["n_blocks"]):
        t = b * TB
        gap = int(enc["gaps"][t >> 1] >> (4 * (t & 1))) & 15
        lo, hi = int(enc["blk_off"][b]), int(enc["blk_off"][b + 1])
        out, _ = oracle.decode_range(enc["stream"], enc["nibbles"], enc["lengths"],
                                     8 * C * t + gap, lo, hi - lo)
        assert np.array_equal(out, x[lo:hi])


def test_corrupted_stream_is_detected_or_differs():
    """Flipping a stream bit never passes silently as the original."""
    x = synth.small_stable(3000, 1.8, 5)
    enc = oracle.encode(x, chunk_bytes=16, tb=64)
    s = enc["stream"].copy()
    s[10] ^= 0x10
    try:
        out = oracle.decode(s, enc["nibbles"], x.size, enc["lengths"])
        assert not np.array_equal(out, x)
    except ValueError:
        pass


# ---------------------------------------------------------------- statistics the pages quote

def test_gaussian_exponent_entropy_and_short_codes():
    """ECF8 blog §2.2: exponent entropy of Gaussian-like FP8 weights 2.55-2.75 bits
    (bound 2.67 at alpha = 2); §3.1.1: > 90% of exponents coded in <= 6 bits."""
    x = synth.gauss_tensor((1024, 1024), 0.02, synth.seed_of("gauss1m", "w", 0)).numpy().ravel()
    f = oracle.histogram(x)
    H = oracle.entropy_bits(f)
    assert 2.5 <= H <= 2.8
    L = oracle.huffman_lengths(f)
    short = f[L <= 6].sum() / f.sum()
    assert short > 0.90
    avg = oracle.average_length(f, L)
    assert H <= avg < H + 1
    assert max(L) <= 16


# ---------------------------------------------------------------- alpha statistics (ECF8 blog §2.2, §6)

def test_alpha_hat_closed_form():
    """If max|w| = gamma * N^(1/alpha) exactly, the estimate returns alpha."""
    for alpha in (1.5, 1.8, 2.0):
        for n in (10, 1000, 123457):
            gamma = 0.01
            w = np.full(n, gamma * 0.5)
            w[n // 3] = -gamma * n ** (1.0 / alpha)
            assert abs(oracle.alpha_hat(w, gamma) - alpha) < 1e-12


def test_alpha_hat_ignores_nan_and_sign():
    w = np.array([0.5, -3.0, np.nan, 1.0])
    assert oracle.alpha_hat(w, 1.0) == np.log(4.0) / np.log(3.0)


def test_entropy_bound_values():
    """alpha / (1 - 2^-alpha): 8/3 at alpha = 2 (the page's 2.67 bits), 2 at alpha = 1,
    1/ln 2 in the limit alpha -> 0, increasing in alpha."""
    assert abs(oracle.entropy_bound(2.0) - 8.0 / 3.0) < 1e-15
    assert abs(round(oracle.entropy_bound(2.0), 2) - 2.67) < 1e-12
    assert oracle.entropy_bound(1.0) == 2.0
    assert abs(oracle.entropy_bound(1e-9) - 1.0 / np.log(2.0)) < 1e-6
    v = [oracle.entropy_bound(a) for a in np.linspace(0.1, 2.0, 20)]
    assert all(b > a for a, b in zip(v, v[1:]))
