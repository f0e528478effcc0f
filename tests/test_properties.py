"""Property tests (hypothesis, CPU): invariants that hold for any input, on generated cases.

* decode(encode(x)) = x in the oracle for any bytes and any allowed (C, TB);
* the library's encoder writes the oracle's bytes (stream, nibbles, gaps, block offsets);
* length-limited codes (the library's E4M3 codebook and both package-merge implementations)
  satisfy the Kraft equality, respect the limit, cost no less than the unlimited Huffman code,
  and the two package-merge implementations find the same optimal cost;
* canonical codes are prefix-free.
The examples are derandomized, so every run checks the same cases.
"""
import numpy as np
from hypothesis import HealthCheck, given, settings, strategies as st

import oracle
import lossless_entropy_coded_ecf8_amd as E
from lossless_entropy_coded_ecf8_amd import binding as B

SETTINGS = dict(max_examples=60, deadline=None, derandomize=True,
                suppress_health_check=[HealthCheck.too_slow, HealthCheck.data_too_large])
SHAPES = [(16, 256), (4, 64), (8, 128), (12, 192), (64, 1024), (32, 256)]


def kraft(lengths):
    return sum(2.0 ** -int(l) for l in lengths if l)


@st.composite
def fp8_bytes(draw):
    """Bytes with a skewed exponent distribution (as weights have) or uniform bytes."""
    n = draw(st.integers(0, 3000))
    seed = draw(st.integers(0, 2 ** 31 - 1))
    rng = np.random.default_rng(seed)
    if draw(st.booleans()):
        e = np.minimum(rng.geometric(draw(st.floats(0.15, 0.9)), n) - 1 + draw(st.integers(0, 8)), 15)
        return ((rng.integers(0, 2, n) << 7) | (e << 3) | rng.integers(0, 8, n)).astype(np.uint8)
    return rng.integers(0, 256, n).astype(np.uint8)


@settings(**SETTINGS)
@given(x=fp8_bytes(), shape=st.sampled_from(SHAPES))
def test_oracle_round_trip_and_library_bytes(x, shape):
    C, TB = shape
    ref = oracle.encode(x, chunk_bytes=C, tb=TB)
    assert np.array_equal(oracle.decode(ref["stream"], ref["nibbles"], x.size, ref["lengths"]), x)
    h = E.encode(x, lengths=[int(v) for v in ref["lengths"]], chunk_bytes=C, threads_per_block=TB)
    assert np.array_equal(h.stream, ref["stream"])
    assert np.array_equal(h.nibbles, ref["nibbles"])
    assert np.array_equal(h.gaps, ref["gaps"])
    assert np.array_equal(h.blk_off.view(np.uint64), ref["blk_off"])


@st.composite
def histograms(draw, nsym):
    present = draw(st.integers(1, nsym))
    counts = draw(st.lists(st.integers(1, 10 ** 6), min_size=present, max_size=present))
    f = np.zeros(nsym, dtype=np.uint64)
    idx = np.random.default_rng(draw(st.integers(0, 2 ** 31 - 1))).permutation(nsym)[:present]
    f[idx] = counts
    return f


@settings(**SETTINGS)
@given(f=histograms(16), limit=st.integers(4, 16))
def test_e4m3_codebook_is_complete_limited_and_no_cheaper_than_huffman(f, limit):
    L = np.asarray(B.codebook_from_freq(f, limit), dtype=np.int64)
    present = int((f > 0).sum())
    assert ((L > 0) == (f > 0)).all()
    assert L.max() <= max(limit, 1)
    if present >= 2:
        assert abs(kraft(L) - 1.0) < 1e-12
    cost = int((f.astype(np.int64) * L).sum())
    huff = int((f.astype(np.int64) * oracle.huffman_lengths(f)).sum())
    assert cost >= huff
    if oracle.huffman_lengths(f).max() <= limit:
        assert cost == huff


@settings(**SETTINGS)
@given(data=st.data(), nsym=st.sampled_from([32, 256]))
def test_package_merge_implementations_agree_on_optimal_cost(data, nsym):
    f = data.draw(histograms(nsym))
    present = int((f > 0).sum())
    lo = max(1, int(np.ceil(np.log2(max(present, 2)))))
    limit = data.draw(st.integers(lo, 16))
    a = np.asarray(oracle.v_package_merge(f, limit), dtype=np.int64)
    b = np.asarray(B.v_code_lengths(f, limit), dtype=np.int64)
    for L in (a, b):
        assert ((L > 0) == (f > 0)).all() and L.max() <= limit
        if present >= 2:
            assert abs(kraft(L) - 1.0) < 1e-12
    fi = f.astype(np.int64)
    assert int((fi * a).sum()) == int((fi * b).sum())


@settings(**SETTINGS)
@given(f=histograms(16))
def test_canonical_codes_are_prefix_free(f):
    L = oracle.huffman_lengths(f)
    c = oracle.canonical_codes(L)
    words = [format(int(c[s]), "0%db" % int(L[s])) for s in range(16) if L[s]]
    for i, u in enumerate(words):
        for j, v in enumerate(words):
            if i != j:
                assert not v.startswith(u)
