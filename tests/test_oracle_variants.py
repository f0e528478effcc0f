"""Pins for the BF16 (DFloat11 layout) / FP8 E5M2 oracle (oracle/ecf8v_oracle.c).

Each check ties the oracle to something other than itself:
  * a worked example computed by hand (tests/golden/bf16_worked_example.txt);
  * the exponent field against numpy's frexp of the decoded value;
  * package-merge against brute-force optimal length-limited codes on tiny
    alphabets, against unlimited Huffman when the limit does not bind, and
    against closed forms (all-equal lengths for a power-of-two alphabet);
  * round trips and per-block decodes from the stored gaps and offsets.
"""
import itertools
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "bf16_worked_example.txt")
GOLDEN_E5M2 = os.path.join(os.path.dirname(__file__), "golden", "e5m2_worked_example.txt")


def read_golden(path=GOLDEN):
    d = {}
    for line in open(path):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        k, *v = line.split()
        d[k] = v
    return d


def test_bf16_worked_example():
    g = read_golden()
    x = np.array([int(v, 16) for v in g["values"]], dtype=np.uint16)
    f = oracle.v_histogram("bf16", x)
    assert [int(s) for s in g["symbols"]] == [int((v >> 7) & 255) for v in x]
    L = oracle.v_lengths("bf16", x)
    want = {int(a): int(b) for a, b in (kv.split(":") for kv in g["lengths"])}
    assert {int(s): int(L[s]) for s in np.nonzero(L)[0]} == want
    codes = oracle.v_canonical_codes(L)
    for kv in g["codes"]:
        s, bits = kv.split(":")
        assert int(codes[int(s)]) == int(bits, 2) and int(L[int(s)]) == len(bits)
    e = oracle.v_encode("bf16", x)
    assert e["total_bits"] == int(g["total_bits"][0])
    assert int(e["stream"][0]) == int(g["stream"][0], 16) and not e["stream"][1:].any()
    assert [int(v) for v in e["raw"][:4]] == [int(v, 16) for v in g["raw"]]
    assert np.array_equal(oracle.v_decode("bf16", e["stream"], e["raw"], 4, e["lengths"]), x)
    assert int(f.sum()) == 4


def test_bf16_symbol_is_the_biased_exponent():
    """For normal BF16 values the symbol is floor(log2|x|) + 127 (numpy frexp gives e with |x| = m 2^e)."""
    g = torch.Generator().manual_seed(0)
    x = (torch.randn(20000, generator=g) * torch.exp(torch.randn(20000, generator=g) * 3)).to(torch.bfloat16)
    bits = x.view(torch.int16).numpy().view(np.uint16)
    vals = x.float().numpy().astype(np.float64)
    normal = np.abs(vals) >= 2.0 ** -126
    _, ex = np.frexp(vals[normal])
    f = oracle.v_histogram("bf16", bits[normal])
    ref = np.bincount(ex + 126, minlength=256).astype(np.uint64)
    assert np.array_equal(f, ref)


def test_e5m2_symbol_is_the_biased_exponent():
    b = np.arange(256, dtype=np.uint8)
    vals = torch.from_numpy(b).view(torch.float8_e5m2).float().numpy().astype(np.float64)
    ok = np.isfinite(vals) & (np.abs(vals) >= 2.0 ** -14)
    _, ex = np.frexp(vals[ok])
    f = oracle.v_histogram("e5m2", b[ok])
    assert np.array_equal(f, np.bincount(ex + 14, minlength=32).astype(np.uint64))


def brute_force_cost(w, L):
    best = None
    for lens in itertools.product(range(1, L + 1), repeat=len(w)):
        if sum(2.0 ** -l for l in lens) <= 1.0 + 1e-12:
            c = sum(a * b for a, b in zip(w, lens))
            best = c if best is None else min(best, c)
    return best


@pytest.mark.parametrize("seed", range(40))
def test_package_merge_is_optimal_on_tiny_alphabets(seed):
    rng = np.random.default_rng(seed)
    m = int(rng.integers(2, 7))
    w = [int(v) for v in rng.integers(1, 60, m)]
    if seed % 3 == 0:
        w = [int(v) for v in np.cumsum(rng.integers(1, 4, m)) ** 2]      # skewed
    freq = np.zeros(8, dtype=np.uint64)
    pos = rng.choice(8, m, replace=False)
    freq[pos] = w
    for L in range(int(np.ceil(np.log2(m))), m):
        lens = oracle.v_package_merge(freq, L)
        got = oracle.code_cost(freq, lens)
        assert got == brute_force_cost(w, L), (w, L, list(lens))
        assert lens.max() <= L and all(lens[freq == 0] == 0) and all(lens[freq > 0] > 0)
        assert abs(oracle.kraft_sum(lens) - 1.0) < 1e-12


@pytest.mark.parametrize("seed", range(10))
def test_package_merge_equals_huffman_when_the_limit_does_not_bind(seed):
    rng = np.random.default_rng(100 + seed)
    freq = np.zeros(256, dtype=np.uint64)
    k = int(rng.integers(2, 200))
    freq[rng.choice(256, k, replace=False)] = rng.geometric(0.05, k)
    H = oracle.v_huffman_lengths(freq)
    if H.max() <= 16:
        P = oracle.v_package_merge(freq, 16)
        assert oracle.code_cost(freq, P) == oracle.code_cost(freq, H)


def test_package_merge_binds_on_a_geometric_alphabet():
    """Weights 2^0 .. 2^19: Huffman depth 19 (a chain); limiting to 16 costs more, to 5 forces a near-flat code."""
    freq = np.zeros(256, dtype=np.uint64)
    freq[:20] = [2 ** i for i in range(20)]
    H = oracle.v_huffman_lengths(freq)
    assert H.max() == 19
    P16 = oracle.v_package_merge(freq, 16)
    assert P16.max() == 16 and oracle.code_cost(freq, P16) > oracle.code_cost(freq, H)
    assert abs(oracle.kraft_sum(P16) - 1.0) < 1e-12
    P5 = oracle.v_package_merge(freq, 5)
    assert P5.max() <= 5 and abs(oracle.kraft_sum(P5) - 1.0) < 1e-12
    # heavier symbols never get longer codes
    order = np.argsort(freq[:20])
    assert all(np.diff(P16[order]) <= 0) and all(np.diff(P5[order]) <= 0)


def test_package_merge_closed_forms():
    freq = np.zeros(256, dtype=np.uint64)
    freq[:] = 7                                           # 256 equal weights, limit 8: all lengths 8
    assert (oracle.v_package_merge(freq, 8) == 8).all()
    with pytest.raises(ValueError):
        oracle.v_package_merge(freq, 7)                   # 2^7 < 256 symbols
    one = np.zeros(32, dtype=np.uint64)
    one[5] = 9
    assert list(np.nonzero(oracle.v_package_merge(one, 1))[0]) == [5]
    assert oracle.v_package_merge(np.zeros(32, dtype=np.uint64), 3).sum() == 0


def bf16_weights(n, seed, scale=0.02):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(n, generator=g) * scale).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("fmt,n", [("bf16", 1), ("bf16", 17), ("bf16", 50_001), ("e5m2", 1), ("e5m2", 33),
                                   ("e5m2", 40_003)])
@pytest.mark.parametrize("C,TB", [(16, 256), (4, 64)])
def test_round_trip_and_block_starts(fmt, n, C, TB):
    rng = np.random.default_rng(n + C)
    x = bf16_weights(n, n) if fmt == "bf16" else \
        torch.from_numpy(rng.standard_normal(n).astype(np.float32)).to(torch.float8_e5m2).view(torch.uint8).numpy()
    e = oracle.v_encode(fmt, x, chunk_bytes=C, tb=TB)
    assert np.array_equal(oracle.v_decode(fmt, e["stream"], e["raw"], n, e["lengths"]), x)
    blk = e["blk_off"]
    assert blk[0] == 0 and blk[-1] == n and np.all(np.diff(blk.astype(np.int64)) >= 0)
    for b in range(e["n_blocks"]):
        t = b * TB
        gap = (int(e["gaps"][t >> 1]) >> (4 * (t & 1))) & 15
        lo, hi = int(blk[b]), int(blk[b + 1])
        got, end = oracle.v_decode_range(fmt, e["stream"], e["raw"], e["lengths"], 8 * C * t + gap, lo, hi - lo)
        assert np.array_equal(got, x[lo:hi])
        assert end >= min(8 * C * TB * (b + 1), e["total_bits"])


def test_bf16_gaussian_compresses_to_about_eleven_bits():
    """DF11 blog §2: about 70% of the BF16 size; 8 raw bits + ~2.6-3 code bits on N(0, 0.02) weights."""
    x = bf16_weights(1 << 18, 7)
    e = oracle.v_encode("bf16", x)
    bits = (e["total_bits"] + 8 * x.size) / x.size
    assert 10.3 < bits < 11.2, bits


def test_e5m2_worked_example():
    """Hand-worked E5M2 example (tests/golden/e5m2_worked_example.txt): symbol (b >> 2) & 31, the raw
    nibble (s << 2) | m in the E4M3 nibble layout, canonical codes, stream bytes and T.  The byte values
    are also checked against torch's own E5M2 cast of the listed floats."""
    g = read_golden(GOLDEN_E5M2)
    x = np.array([int(v, 16) for v in g["values"]], dtype=np.uint8)
    fl = torch.tensor([float(v) for v in g["floats"]]).to(torch.float8_e5m2).view(torch.uint8).numpy()
    assert np.array_equal(fl, x)
    assert [int(s) for s in g["symbols"]] == [int((v >> 2) & 31) for v in x]
    L = oracle.v_lengths("e5m2", x)
    want = {int(a): int(b) for a, b in (kv.split(":") for kv in g["lengths"])}
    assert {int(s): int(L[s]) for s in np.nonzero(L)[0]} == want
    codes = oracle.v_canonical_codes(L)
    for kv in g["codes"]:
        s, bits = kv.split(":")
        assert int(codes[int(s)]) == int(bits, 2) and int(L[int(s)]) == len(bits)
    e = oracle.v_encode("e5m2", x)
    assert e["total_bits"] == int(g["total_bits"][0])
    assert int(e["stream"][0]) == int(g["stream"][0], 16) and not e["stream"][1:].any()
    raw = [int(v, 16) for v in g["raw"]]
    assert [int(v) for v in e["raw"][:len(raw)]] == raw and not e["raw"][len(raw):].any()
    assert e["blk_off"].tolist() == [0, x.size]
    assert np.array_equal(oracle.v_decode("e5m2", e["stream"], e["raw"], x.size, e["lengths"]), x)


def v_symbols(fmt, x):
    x = np.asarray(x)
    return ((x.astype(np.int64) >> 7) & 255) if fmt == "bf16" else ((x.astype(np.int64) >> 2) & 31)


def brute_force_layout_v(fmt, x, lengths, C, TB):
    """Gaps and block offsets from the definitions (ECF8 blog §3.2.1 per-thread gap), by brute force over
    the codeword start positions: gap_t = (first start >= 8Ct, T counting as a start) - 8Ct for 8Ct < T,
    else 0; blk_off_b = number of starts before 8*C*TB*b; blk_off[n_blocks] = n."""
    lens = np.asarray(lengths)[v_symbols(fmt, x)]
    starts = np.concatenate([[0], np.cumsum(lens)[:-1]]) if len(lens) else np.zeros(0, np.int64)
    T = int(lens.sum())
    nc = -(-T // (8 * C))
    nb = -(-nc // TB)
    gaps = []
    for t in range(nb * TB):
        s0 = 8 * C * t
        if s0 >= T:
            gaps.append(0)
            continue
        later = starts[starts >= s0]
        gaps.append(int(min(later.min(), T) if later.size else T) - s0)
    blk = [int((starts < 8 * C * TB * b).sum()) for b in range(nb)] + [len(lens)]
    return gaps, blk


@pytest.mark.parametrize("fmt", ["bf16", "e5m2"])
@pytest.mark.parametrize("seed", range(6))
def test_variant_gaps_and_block_offsets_by_definition(fmt, seed):
    """Every chunk's gap and every block offset of oraclev_encode equal a brute-force recomputation from
    codeword starts, interior chunks included, at several (C, TB) and sizes."""
    rng = np.random.default_rng(700 + seed)
    n = int(rng.integers(1, 4000))
    C, TB = [(4, 64), (8, 64), (16, 64)][seed % 3]
    if fmt == "bf16":
        x = bf16_weights(n, seed, scale=0.02 if seed % 2 else 3.0)
    else:
        x = torch.from_numpy((rng.standard_normal(n) * (10.0 ** rng.uniform(-3, 3, n))).astype(np.float32)) \
            .to(torch.float8_e5m2).view(torch.uint8).numpy()
    e = oracle.v_encode(fmt, x, chunk_bytes=C, tb=TB)
    gaps, blk = brute_force_layout_v(fmt, x, e["lengths"], C, TB)
    assert all(0 <= v <= 15 for v in gaps)
    g = e["gaps"]
    stored = [(int(g[t >> 1]) >> (4 * (t & 1))) & 15 for t in range(len(gaps))]
    assert stored == gaps
    assert e["blk_off"].tolist() == blk
    # every chunk decodes its own codewords from its stored gap: the first codeword it reads is the
    # element whose start the gap names
    starts = np.concatenate([[0], np.cumsum(np.asarray(e["lengths"])[v_symbols(fmt, x)])[:-1]])
    for t in range(0, e["n_chunks"], max(1, e["n_chunks"] // 40)):
        p = 8 * C * t + gaps[t]
        if p >= e["total_bits"]:
            continue
        j = int(np.searchsorted(starts, p))
        assert starts[j] == p
        got, _ = oracle.v_decode_range(fmt, e["stream"], e["raw"], e["lengths"], p, j, 1)
        assert int(got[0]) == int(x[j])
