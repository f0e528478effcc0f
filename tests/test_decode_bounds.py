"""Host-side checks of the E4M3 decode kernel's index and address arithmetic (no GPU).

The decode table (ecf8_decode.hip) has an 11-bit region (prefixes of codes up
to 11 bits) and a 16-bit region for the few prefixes of longer codes; a
lookup's index is max(prefix11, prefix16 - cd), clamped to the last entry.
These tests model that arithmetic in Python, exactly as the table kernel sizes
the table, and check on every 16-bit window that the index lands on a built
entry, for every kind of code that validates -- complete codes of every depth
and the one incomplete code (a single symbol of length 1).  A lookup that left
the built entries would read LDS that holds no entry; an entry consuming zero
bits would never end a walk.
"""
import numpy as np
import pytest

import oracle

K_WIN = 11
K_TABLE_MAX = (1 << K_WIN) + ((1 << (16 - K_WIN)) - 1) * 8     # 2296, as in the kernel


def table_geometry(lengths):
    """p_long, cdelta and the built entry count, as the table kernel computes them."""
    units = sum(1 << (16 - l) for l in lengths if 0 < l <= K_WIN)
    p_long = units >> (16 - K_WIN)
    cd = ((1 << (16 - K_WIN)) - 1) * p_long
    entries = min(65536 - cd, K_TABLE_MAX)
    return p_long, cd, entries


def indices(lengths):
    """Table index of every 16-bit window (the index only depends on the top 16 bits)."""
    _, cd, _ = table_geometry(lengths)
    w = np.arange(1 << 16, dtype=np.int64)
    return np.minimum(np.maximum(w >> (16 - K_WIN), w - cd), K_TABLE_MAX - 1)


def entry_bits(lengths, idx):
    """Bits the table entry at idx consumes (>= 1 by construction: 0 whole codewords -> 1)."""
    p_long, cd, _ = table_geometry(lengths)
    v, known = (idx << (16 - K_WIN), K_WIN) if idx < p_long else (idx + cd, 16)
    codes = oracle.canonical_codes(lengths)
    pos = 0
    for _ in range(4):
        x = (v << pos) & 0xFFFF
        hit = [l for s, l in enumerate(lengths) if l and (x >> (16 - l)) == codes[s]]
        if not hit or pos + hit[0] > known:
            break
        pos += hit[0]
    return pos if pos else 1


def codebooks():
    books = {"uniform4": [4] * 16, "fib15": list(range(1, 16)) + [15],
             "long12x6": list(range(1, 10)) + [11] + [12] * 6, "two": [1, 1] + [0] * 14}
    for s in (0, 7, 15):
        L = [0] * 16
        L[s] = 1
        books["single%d" % s] = L
    rng = np.random.default_rng(5)
    for i in range(40):
        k = int(rng.integers(2, 17))
        f = np.zeros(16, dtype=np.uint64)
        f[rng.choice(16, k, replace=False)] = (10 ** rng.uniform(0, 12, k)).astype(np.uint64) + 1
        books["huffman%d" % i] = oracle.huffman_lengths(f).tolist()
    return books


BOOKS = codebooks()


@pytest.mark.parametrize("name", sorted(BOOKS))
def test_every_window_indexes_a_built_entry(name):
    L = BOOKS[name]
    p_long, cd, entries = table_geometry(L)
    idx = indices(L)
    assert idx.min() >= 0
    assert idx.max() < entries, (name, int(idx.max()), entries)
    complete = abs(oracle.kraft_sum(L) - 1.0) < 1e-12
    if complete:
        # the clamp never binds for a complete code: the unclamped index is already in range
        w = np.arange(1 << 16, dtype=np.int64)
        assert np.maximum(w >> 5, w - cd).max() == entries - 1
        assert 2048 - p_long <= 8                 # long-code prefixes fit the 16-bit region
    else:
        assert sum(1 for l in L if l) == 1 and max(L) == 1


@pytest.mark.parametrize("name", ["single0", "single15", "fib15", "long12x6", "two"])
def test_every_reachable_entry_consumes_bits(name):
    L = BOOKS[name]
    for i in np.unique(indices(L)):
        assert entry_bits(L, int(i)) >= 1


def test_single_symbol_clamp_entry_decodes_nothing():
    """For the single 1-bit code '0', a window starting with 1 is no codeword: its (clamped) entry
    consumes one bit and decodes no symbol, so a corrupt single-symbol stream loses symbols (and
    fails the block check) instead of stalling."""
    L = BOOKS["single0"]
    p_long, cd, entries = table_geometry(L)
    assert (p_long, entries) == (1024, K_TABLE_MAX)
    top = indices(L)[1 << 15:]
    assert top.min() >= p_long and top.max() == K_TABLE_MAX - 1
    assert entry_bits(L, K_TABLE_MAX - 1) == 1


def test_staging_bound_under_any_counts():
    """Whatever the stream and gaps hold, a lane counts at most one codeword per bit of its chunk, so the
    block's counts sum to at most 8*C*TB; with the last lookup's at most 3 further symbols, a 15-element
    group offset and the pair emission touching the next dword, the highest staging dword the decode
    writes stays inside the kernel's staging area (C = 16, TB = 256)."""
    C, TB = 16, 256
    out_dw = ((8 * C * TB + 15 + 8 + 16) // 8 + 2 + 3) // 4 * 4          # the kernel's staging dwords
    max_nibble = 15 + 8 * C * TB + 3                                       # a0 + total + overshoot
    assert (4 * max_nibble) // 32 + 1 < out_dw
