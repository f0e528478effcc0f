"""A host-side model of one decode block's LDS arithmetic (no GPU).

The E4M3 decode kernel (ecf8_decode.hip) decodes a block of TB = 256 lanes,
C = 16 stream bytes each: a count pass in wave-uniform steps of table lookups
(entries recorded in registers; the second lookup of each pair takes the
first one's window shifted by the bits it consumed), an exclusive scan of the counts, then a
decode pass that ORs the recorded entries' symbols, two entries at a time,
into an LDS staging area of packed nibbles, and a write-back of whole
16-element groups.  This module re-enacts those steps in Python, with the
kernel's table layout, window positions, record count, step size, overshoot
correction, pair emission (one OR per pair plus a carried spill) and the
re-walk of lanes with more lookups than records, and checks on every case:

  * the staging nibbles equal the oracle's decode of the block (pinned
    independently), and the block's count matches blk_off;
  * every staging dword the decode touches lies below the kernel's staging
    size (the wave sums follow it in LDS), and the clearing range covers
    every dword written;
  * in a wave whose lanes all hold whole chunks, every lane is active for
    the first C / 2 lookups (rounded down to whole steps), which the kernel
    takes without activity tests;
  * the same for a variant that ORs four entries at a time with three
    dwords from one base (+0, +4, +8 bytes), a form once measured and left
    out: the model shows whether its addresses or its packing could explain
    wrong exponents.

The inputs include the worst cases for the staging (1-bit codes: 8 symbols
per stream byte), deep codes (15-bit and 12-bit codewords in the 16-bit table
region) and the 4-symbol cap (low-entropy tensors).
"""
import numpy as np
import pytest

import oracle
import synth
import lossless_entropy_coded_ecf8_amd as E

C, TB = 16, 256
K_WIN = 11
K_TABLE_MAX = (1 << K_WIN) + ((1 << (16 - K_WIN)) - 1) * 8
RECORDS, STEP = 20, 4
def out_dw(C, TB):
    """Staging dwords of the kernel's LDS for shape (C, TB)."""
    return ((8 * C * TB + 15 + 8 + 16) // 8 + 2 + 3) // 4 * 4


OUT_DW = out_dw(C, TB)


def build_table(lengths):
    """Entries as the table kernel writes them: [7:0] 4 * symbols, [15:8] bits, [31:16] symbols."""
    units = sum(1 << (16 - l) for l in lengths if 0 < l <= K_WIN)
    p_long = units >> (16 - K_WIN)
    cd = ((1 << (16 - K_WIN)) - 1) * p_long
    entries = min(65536 - cd, K_TABLE_MAX)
    codes = oracle.canonical_codes(lengths)
    book = [(int(codes[s]), int(l), s) for s, l in enumerate(lengths) if l]
    tab = np.zeros(K_TABLE_MAX, dtype=np.int64)
    for idx in range(entries):
        v, known = (idx << (16 - K_WIN), K_WIN) if idx < p_long else (idx + cd, 16)
        pos = ns = sy = 0
        while ns < 4 and pos < known:
            x = (v << pos) & 0xFFFF
            hit = [(l, s) for c, l, s in book if (x >> (16 - l)) == c]
            if not hit or pos + hit[0][0] > known:
                break
            l, s = hit[0]
            sy |= s << (4 * ns)
            ns += 1
            pos += l
        tab[idx] = (4 * ns) | ((pos if pos else 1) << 8) | (sy << 16)
    return tab, cd, lengths


def window(bits, bitpos):
    """The 32-bit window at bitpos of a lane's bit array."""
    w = 0
    for k in range(32):
        w = (w << 1) | int(bits[bitpos + k])
    return w


def entry(tab, cd, w):
    """Table entry for a 32-bit window."""
    idx = min(max(w >> (32 - K_WIN), (w >> 16) - cd), K_TABLE_MAX - 1)
    return int(tab[idx])


def lookup(tab, cd, bits, bitpos):
    """Entry for the 32-bit window at bitpos of a lane's bit array."""
    return entry(tab, cd, window(bits, bitpos))


def model_block(enc, tab, cd, b, quad=False):
    """Returns (staging dwords as python ints, max dword index touched, clear range in dwords, total)."""
    C, TB = int(enc.meta.chunk_bytes), int(enc.meta.threads_per_block)
    R0 = 32 * (C // 4 + 2)                        # r = R0 - bit position in the lane's chunk
    OUT_DW = out_dw(C, TB)
    stream = enc.stream
    T = int(enc.meta.total_bits)
    lens = [int(v) for v in enc.lengths]          # python ints: packets exceed 64 bits
    left = max(T - b * 8 * C * TB, 0)
    leftc = min(left, 8 * C * TB)
    lo, hi = int(enc.blk_off[b]), int(enc.blk_off[b + 1])
    a0 = lo & 15
    lanes = []
    for t in range(TB):
        g = b * TB + t
        gap = (int(enc.gaps[g >> 1]) >> (4 * (g & 1))) & 15
        E_ = min(max(leftc - t * 8 * C, 0), 8 * C)
        base = g * C
        raw = np.frombuffer(bytes(stream[base: base + C + 4]) + bytes(64), dtype=np.uint8)
        lanes.append(dict(bits=np.unpackbits(raw), r=R0 - gap, r0=R0 - gap, rend=R0 - E_, cnt4=0, lastex=0,
                          rec=[], raw=[], act=(R0 - gap) > (R0 - E_)))
    # count pass: wave-uniform steps, records, then lanes past the records keep walking.
    # A wave whose lanes all hold whole chunks takes its first `sure` lookups
    # without activity tests: check that every lane is indeed active there.
    sure = min(C // 2, RECORDS) // STEP * STEP
    for w0 in range(0, TB, 64):
        wave = lanes[w0:w0 + 64]
        wave_full = leftc >= 8 * C * (w0 + 64)
        for q in range(RECORDS // STEP):
            if not any(L["act"] for L in wave):
                break
            for L in wave:
                for j in range(STEP):
                    if wave_full and q * STEP + j < sure:
                        assert L["act"], ("unmasked lookup of an inactive lane", w0, q, j)
                    # pairs: the second lookup's window is the first's shifted
                    # by the bits the first consumed (zeros shifted in)
                    if j % 2 == 0:
                        w = window(L["bits"], R0 - L["r"])
                    else:
                        w = (w << ((L["rec"][-1] >> 8) & 0xFF)) & 0xFFFFFFFF
                    e = entry(tab, cd, w)
                    em = e if L["act"] else 0
                    if L["act"]:
                        L["lastex"] = e
                    L["raw"].append(em)
                    L["r"] -= (em >> 8) & 0xFF
                    if j % 2 == 0:
                        L["rec"].append(em)
                    else:
                        # a pair's second record carries the pair's nibble count in byte 0
                        L["rec"].append(em + (L["rec"][-1] & 0xFF))
                        assert (L["rec"][-1] & 0xFF) <= 32
                        L["cnt4"] += L["rec"][-1] & 0xFF
                    L["act"] = L["r"] > L["rend"]
        for L in wave:
            L["r_rec"] = L["r"]
            L["extra"] = []
            while L["r"] > L["rend"]:
                e = lookup(tab, cd, L["bits"], R0 - L["r"])
                L["extra"].append(e)
                L["lastex"] = e
                L["r"] -= (e >> 8) & 0xFF
                L["cnt4"] += e & 0xFF
    for L in lanes:
        cnt = L["cnt4"] >> 2
        if L["r"] != L["r0"]:
            ex = L["lastex"]
            ns = (ex & 0xFF) >> 2
            room = L["r"] + ((ex >> 8) & 0xFF) - L["rend"]
            sy, start, keep = ex >> 16, 0, 0
            for i in range(ns):
                keep += start < room
                start += lens[sy & 15]
                sy >>= 4
            cnt -= ns - keep
        L["cnt"] = int(cnt)
    total = sum(L["cnt"] for L in lanes)
    stage = [0] * (OUT_DW + 8)
    touched = [0]

    def OR(i, v):
        touched[0] = max(touched[0], i)
        stage[i] |= v & 0xFFFFFFFF

    pos = 0
    for L in lanes:
        ob = (a0 + pos) * 4
        pos += L["cnt"]
        rec = L["raw"] if quad else L["rec"]
        if quad:
            for k in range(0, len(rec) - 3, 4):
                pk, n = 0, 0
                for e in rec[k:k + 4]:
                    pk |= (e >> 16) << n
                    n += e & 0xFF
                v = pk << (ob & 31)
                OR(ob >> 5, v)
                OR((ob >> 5) + 1, v >> 32)
                OR((ob >> 5) + 2, v >> 64)
                ob += n
            for k in range(len(rec) - len(rec) % 4, len(rec), 2):
                p = (rec[k] >> 16) | ((rec[k + 1] >> 16) << (rec[k] & 31))
                v = p << (ob & 31)
                OR(ob >> 5, v)
                OR((ob >> 5) + 1, v >> 32)
                ob += (rec[k] & 0xFF) + (rec[k + 1] & 0xFF)
        else:
            carry = 0
            for k in range(0, len(rec), 2):
                p = (rec[k] >> 16) | ((rec[k + 1] >> 16) << (rec[k] & 31))
                v = p << (ob & 31)
                OR(ob >> 5, v | carry)
                carry = v >> 32
                ob += rec[k + 1] & 0xFF
            if rec:
                OR(ob >> 5, carry)
        for e in L["extra"]:
            v = (e >> 16) << (ob & 31)
            OR(ob >> 5, v)
            OR((ob >> 5) + 1, v >> 32)
            ob += e & 0xFF
    zend_groups = min((a0 + total + 3 + 15) >> 4, OUT_DW // 2)
    return stage, touched[0], 2 * zend_groups, total, a0, lo, hi


def staging_nibbles(stage, a0, count):
    out = np.zeros(count, dtype=np.uint8)
    for j in range(count):
        k = a0 + j
        out[j] = (stage[k >> 3] >> (4 * (k & 7))) & 15
    return out


CASES = {
    "stable17": lambda: (synth.small_stable(120_000, 1.7, 5), None),
    "lowentropy": lambda: (synth.small_stable(200_000, 1.5, 6), None),
    "two": lambda: (np.random.default_rng(1).choice([0x00, 0x08], 300_000).astype(np.uint8)
                    | np.random.default_rng(2).integers(0, 8, 300_000).astype(np.uint8), [1, 1] + [0] * 14),
    "single": lambda: (np.full(270_000, 0x3B, dtype=np.uint8), None),
    "fib15": lambda: (((np.random.default_rng(3).choice(16, 60_000, p=np.r_[0.5 ** np.arange(1, 16), 0.5 ** 15]))
                       << 3).astype(np.uint8), list(range(1, 16)) + [15]),
}


@pytest.mark.parametrize("quad", [False, True], ids=["pairs_with_carry", "four_at_a_time"])
@pytest.mark.parametrize("case", sorted(CASES))
def test_block_model(case, quad):
    check_model(case, quad, 16, 256)


@pytest.mark.parametrize("shape", [(32, 256), (64, 128), (8, 256)], ids=str)
@pytest.mark.parametrize("case", ["lowentropy", "two", "fib15"])
def test_block_model_other_shapes(case, shape):
    """The same model for other chunk sizes: longer chunks walk well past their 20 records."""
    check_model(case, False, *shape)


def check_model(case, quad, C, TB):
    x, L = CASES[case]()
    enc = E.encode(x, lengths=L, chunk_bytes=C, threads_per_block=TB)
    tab, cd, lens = build_table(list(enc.lengths))
    ref = oracle.decode(enc.stream, enc.nibbles, enc.n, enc.lengths)
    assert np.array_equal(ref, x)
    nb = int(enc.meta.n_blocks)
    for b in sorted({0, 1, nb - 1} & set(range(nb))):
        stage, top, clear_dw, total, a0, lo, hi = model_block(enc, tab, cd, b, quad=quad)
        assert total == hi - lo, ("count", b)
        assert top < out_dw(C, TB), ("staging dword out of range", top, out_dw(C, TB))
        assert top < clear_dw or all(v == 0 for v in stage[clear_dw:]), ("written past the cleared range", b)
        got = staging_nibbles(stage, a0, hi - lo)
        assert np.array_equal(got, (ref[lo:hi] >> 3) & 15), ("exponents", b)
