"""Host half of libecf8 vs the oracle (CPU only), and the C ABI surface."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
import synth
import lossless_entropy_coded_ecf8_amd as E
from lossless_entropy_coded_ecf8_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    names = set()
    for h in sorted(os.listdir(os.path.join(ROOT, "include"))):
        if h.endswith(".h"):
            src = open(os.path.join(ROOT, "include", h)).read()
            names |= set(re.findall(r"^\s*(?:const\s+)?\w[\w\s\*]*?\b(ecf8v?_\w+)\s*\(", src, re.M))
    return sorted(names)


def test_every_header_function_is_exported():
    """libecf8.so loads on a CPU-only host and exports every declared entry point."""
    names = header_functions()
    assert len(names) >= 15
    lib = E.lib()
    for nm in names:
        assert hasattr(lib, nm), nm
    assert set(names) == set(B.EXPORTS) | set(B.EXPORTS_V)
    assert lib.ecf8_version() >= 100
    for code in (0, -1, -2, -3, -4, -5, -6, -7, -99):
        assert lib.ecf8_strerror(code)


@pytest.mark.parametrize("seed", range(60))
def test_codebook_matches_oracle_including_ties(seed):
    rng = np.random.default_rng(seed)
    k = int(rng.integers(1, 17))
    freq = np.zeros(16, dtype=np.uint64)
    syms = rng.choice(16, k, replace=False)
    if seed % 3 == 0:
        freq[syms] = rng.integers(1, 4, k)                      # heavy ties
    elif seed % 3 == 1:
        freq[syms] = (10 ** rng.uniform(0, 9, k)).astype(np.uint64)  # huge spread, deep trees
    else:
        freq[syms] = rng.integers(1, 10 ** 6, k)
    assert E.codebook_from_freq(freq).tolist() == oracle.huffman_lengths(freq).tolist()


def test_fibonacci_depth_15_and_length_limit():
    freq = [1, 1, 2, 3, 5, 8, 13, 21, 34, 55, 89, 144, 233, 377, 610, 987]
    assert max(E.codebook_from_freq(freq, 15)) == 15
    # a binding limit gives the optimal limited code (the oracle's package-merge)
    L14 = E.codebook_from_freq(freq, 14)
    assert L14.tolist() == oracle.v_package_merge(freq, 14).tolist() and max(L14) == 14
    assert oracle.kraft_sum(L14) == 1.0
    L4 = E.codebook_from_freq(freq, 4)
    assert L4.tolist() == [4] * 16                      # 16 symbols in 4 bits: the only code
    with pytest.raises(E.Ecf8Error) as ei:
        E.codebook_from_freq(freq, 3)                   # 2^3 < 16 present symbols
    assert ei.value.code == -4
    with pytest.raises(E.Ecf8Error):
        E.codebook_from_freq(freq, 17)


@pytest.mark.parametrize("seed", range(24))
def test_length_limited_codebook_matches_oracle(seed):
    """E4M3 codes under a length limit (the decode's one-shift table index needs codes of at most 11
    bits): the Huffman lengths when the tree is no deeper than the limit, otherwise the oracle's
    optimal length-limited lengths (package-merge, pinned by brute force on small alphabets)."""
    rng = np.random.default_rng(100 + seed)
    k = int(rng.integers(2, 17))
    freq = np.zeros(16, dtype=np.uint64)
    freq[rng.choice(16, k, replace=False)] = (10 ** rng.uniform(0, 9, k)).astype(np.uint64) + 1
    huff = oracle.huffman_lengths(freq)
    for limit in (16, 13, 11, 8, 5):
        if (1 << limit) < k:
            continue
        got = E.codebook_from_freq(freq, limit)
        want = huff if max(huff) <= limit else oracle.v_package_merge(freq, limit)
        assert got.tolist() == want.tolist(), (limit, freq.tolist())
        assert max(got) <= limit
        assert oracle.code_cost(freq, got) == oracle.code_cost(freq, want)


@pytest.mark.parametrize("lengths", [None, [4] * 16, list(range(1, 16)) + [15]])
def test_canonical_codes_match_oracle(lengths):
    if lengths is None:
        lengths = oracle.huffman_lengths(oracle.histogram(synth.small_stable(5000, 1.7, 1)))
    assert E.canonical_codes(lengths).tolist() == oracle.canonical_codes(lengths).tolist()


COMPLETE_CODES = {
    "uniform4": [4] * 16,
    "fib15": list(range(1, 16)) + [15],
    "long12x6": list(range(1, 10)) + [11] + [12] * 6,
    "two": [1, 1] + [0] * 14,
}


def cases():
    out = []
    for n in (0, 1, 2, 3, 7, 63, 64, 65, 1000, 4095, 4096, 4097, 33333):
        out.append(("stable", n, None))
    for name in COMPLETE_CODES:
        out.append((name, 5000, COMPLETE_CODES[name]))
    out.append(("single", 777, None))
    out.append(("bytes", 9999, None))
    return out


def make_input(kind, n, seed):
    rng = np.random.default_rng(seed)
    if kind == "stable":
        return synth.small_stable(max(n, 1), 1.75, seed)[:n]
    if kind == "single":
        return np.full(n, 0x3B, dtype=np.uint8)
    if kind == "bytes":
        return synth.random_bytes(n, seed)
    L = COMPLETE_CODES[kind]
    present = [s for s in range(16) if L[s] > 0]
    e = rng.choice(present, n).astype(np.uint8)
    return ((rng.integers(0, 2, n, dtype=np.uint8) << 7) | (e << 3) | rng.integers(0, 8, n, dtype=np.uint8)).astype(np.uint8)


@pytest.mark.parametrize("C,TB", [(16, 256), (4, 64), (8, 128), (32, 64)])
@pytest.mark.parametrize("case", cases(), ids=lambda c: "%s-%d" % (c[0], c[1]))
def test_encode_byte_identical_to_oracle(case, C, TB):
    kind, n, L = case
    x = make_input(kind, n, n + C)
    enc = E.encode(x, lengths=L, chunk_bytes=C, threads_per_block=TB)
    ref = oracle.encode(x, lengths=L, chunk_bytes=C, tb=TB)
    m = enc.meta
    assert m.n == n and m.total_bits == ref["total_bits"]
    for k in ("n_chunks", "n_blocks", "stream_bytes", "nibble_bytes", "gap_bytes"):
        assert getattr(m, k) == ref[k], k
    assert np.array_equal(enc.stream, ref["stream"])
    assert np.array_equal(enc.nibbles, ref["nibbles"])
    assert np.array_equal(enc.gaps, ref["gaps"])
    assert np.array_equal(enc.blk_off, ref["blk_off"])
    assert B.validate_meta(m) == 0
    # the oracle decodes the library's stream back to x
    assert np.array_equal(oracle.decode(enc.stream, enc.nibbles, n, enc.lengths), x)


@pytest.mark.parametrize("threads", ["1", "3", "8"])
def test_multithreaded_encoder_is_deterministic(threads, monkeypatch):
    x = synth.small_stable(3_000_001, 1.6, 2)
    monkeypatch.setenv("ECF8_THREADS", threads)
    enc = E.encode(x)
    ref = oracle.encode(x)
    assert np.array_equal(enc.stream, ref["stream"])
    assert np.array_equal(enc.gaps, ref["gaps"])
    assert np.array_equal(enc.blk_off, ref["blk_off"])
    assert np.array_equal(enc.nibbles, ref["nibbles"])


def test_validate_meta_rejects_corruption():
    x = synth.small_stable(50000, 1.8, 3)
    m = E.encode(x).meta

    def bad(mutate):
        mm = B.Meta.from_buffer_copy(m)
        mutate(mm)
        return B.validate_meta(mm)

    assert B.validate_meta(m) == 0
    assert bad(lambda mm: setattr(mm, "n_blocks", mm.n_blocks + 1)) == -3
    assert bad(lambda mm: setattr(mm, "total_bits", mm.total_bits + 4096)) == -3
    assert bad(lambda mm: setattr(mm, "stream_bytes", mm.stream_bytes - 1)) == -3
    assert bad(lambda mm: setattr(mm, "max_len", mm.max_len + 1)) == -3
    assert bad(lambda mm: setattr(mm, "chunk_bytes", 6)) == -3

    def kill_kraft(mm):
        mm.cb.len[0] = mm.cb.len[0] + 1
    assert bad(kill_kraft) == -3

    def too_long(mm):
        mm.cb.len[0] = 17
    assert bad(too_long) == -3


def test_encode_rejects_bad_arguments():
    x = synth.small_stable(1000, 1.8, 4)
    with pytest.raises(E.Ecf8Error) as ei:
        E.encode(x, chunk_bytes=6)
    assert ei.value.code == -1
    with pytest.raises(E.Ecf8Error) as ei:
        E.encode(x, threads_per_block=100)
    assert ei.value.code == -1
    L = oracle.huffman_lengths(oracle.histogram(x)).copy()
    present = int(np.nonzero(L)[0][0])
    L2 = [4] * 16
    L2[present] = 0                       # a present symbol without a code
    with pytest.raises(E.Ecf8Error) as ei:
        E.encode(x, lengths=L2)
    assert ei.value.code == -3


def test_workspace_size_grows_with_count():
    a, b = E.workspace_bytes(1), E.workspace_bytes(768)
    assert 0 < a < b
    assert b % 256 == 0


# ---------------------------------------------------------------- device encode (host-side logic)

@pytest.mark.parametrize("C,TB", [(16, 256), (4, 64), (12, 192), (64, 1024)])
def test_meta_from_freq_equals_encode_sizes_and_oracle(C, TB):
    for n in (1, 17, 4097, 100_003):
        x = synth.small_stable(n, 1.8, n)
        L = oracle.huffman_lengths(oracle.histogram(x))
        m = E.meta_from_freq(oracle.histogram(x).astype(np.uint64), n, L, C, TB)
        host = E.encode(x, lengths=L, chunk_bytes=C, threads_per_block=TB).meta
        assert B.meta_dict(m) == B.meta_dict(host)
        ref = oracle.encode(x, lengths=L, chunk_bytes=C, tb=TB)
        assert int(m.total_bits) == ref["total_bits"]
        for k in ("n_chunks", "n_blocks", "stream_bytes", "nibble_bytes", "gap_bytes"):
            assert int(getattr(m, k)) == ref[k], k
        assert B.validate_meta(m) == 0


def test_meta_from_freq_rejects_inconsistent_counts():
    x = synth.small_stable(1000, 1.8, 2)
    f = oracle.histogram(x).astype(np.uint64)
    L = oracle.huffman_lengths(f)
    with pytest.raises(E.Ecf8Error) as ei:
        E.meta_from_freq(f, 999, L)                   # counts do not sum to n
    assert ei.value.code == -2
    L2 = list(L)
    L2[int(np.nonzero(f)[0][0])] = 0                 # a counted symbol without a code
    with pytest.raises(E.Ecf8Error):
        E.meta_from_freq(f, 1000, L2)
    with pytest.raises(E.Ecf8Error) as ei:
        E.meta_from_freq(f, 1000, L, chunk_bytes=6)
    assert ei.value.code == -1


def test_encode_workspace_bytes():
    assert E.encode_workspace_bytes(0) >= 256
    sizes = [E.encode_workspace_bytes(n) for n in (1, 4096, 4097, 10 ** 9, 11_300_000_000)]
    assert sizes == sorted(sizes) and all(v % 256 == 0 for v in sizes)
    # per-tile counts (32 B) and tile offsets (8 B) per 4096-element tile, at least
    assert sizes[-2] >= 40 * (10 ** 9 // 4096)


def test_encode_device_argument_checks_need_no_gpu():
    """Every rejection happens on the host before any launch (fake device pointers)."""
    x = synth.small_stable(10_000, 1.8, 3)
    m = E.encode(x).meta
    L = E.lib()
    ws_need = E.encode_workspace_bytes(m.n)
    P = lambda v: ctypes.c_void_p(v)
    good = dict(fp8=0x100000, stream=0x200000, nib=0x300000, gaps=0x400000, blk=0x500000, ws=0x600000)

    def call(meta=m, ws_bytes=ws_need, **kw):
        a = dict(good, **kw)
        return L.ecf8_encode_device(P(a["fp8"]), ctypes.byref(meta) if meta is not None else None,
                                    P(a["stream"]), P(a["nib"]), P(a["gaps"]), P(a["blk"]), P(a["ws"]),
                                    ws_bytes, None)
    assert call(meta=None) == -1
    assert call(stream=0) == -1 and call(stream=0x200002) == -1
    assert call(blk=0x500004) == -1 and call(nib=0x300004) == -1 and call(gaps=0x400002) == -1
    assert call(fp8=0) == -1
    assert call(ws=0x600010) == -7 and call(ws_bytes=ws_need - 1) == -7
    bad = B.Meta.from_buffer_copy(m)
    bad.total_bits += 1 << 20
    assert call(meta=bad) == -3
    assert L.ecf8_histogram_device(P(0), 5, P(0x100000), P(0), 0, None) == -1
    assert L.ecf8_histogram_device(P(0x100000), 5, P(0x100004), P(0), 0, None) == -1
    assert L.ecf8_histogram_device(P(0x100000), 5, P(0x100000), P(0x600010), 1 << 20, None) == -7
    assert L.ecf8_histogram_device(P(0x100000), 5, P(0x100000), P(0x600000), 255, None) == -7


def test_encode_batched_checks_every_job_before_any_launch():
    """ecf8_encode_batched_device rejects a batch on the host when any job is bad (fake device pointers,
    so a launch would fail with a HIP error instead of the argument error)."""
    x = synth.small_stable(10_000, 1.8, 3)
    m = E.encode(x).meta
    L = E.lib()
    ws_need = E.encode_workspace_bytes(m.n)

    def job(k, **kw):
        base = 0x1000000 * (k + 1)
        a = dict(fp8=base, stream=base + 0x100000, nib=base + 0x200000, gaps=base + 0x300000,
                 blk=base + 0x400000, ws=base + 0x500000, ws_bytes=ws_need, meta=m)
        a.update(kw)
        return B.EncodeJob(a["fp8"], a["meta"], a["stream"], a["nib"], a["gaps"], a["blk"], a["ws"], a["ws_bytes"])

    def call(jobs, count=None):
        arr = (B.EncodeJob * max(len(jobs), 1))(*jobs)
        return L.ecf8_encode_batched_device(arr, len(jobs) if count is None else count, None)
    assert L.ecf8_encode_batched_device(None, 2, None) == -1
    assert call([job(0)], count=-1) == -1
    assert call([job(0), job(1, stream=0x2100002)]) == -1
    assert call([job(0), job(1), job(2, nib=0x3200004)]) == -1
    assert call([job(0), job(1, ws_bytes=ws_need - 1)]) == -7
    bad = B.Meta.from_buffer_copy(m)
    bad.total_bits += 1 << 20
    assert call([job(0), job(1, meta=bad)]) == -3
    assert call([job(k) for k in range(9)] + [job(9, fp8=0)]) == -1


def test_measurement_kernels_reject_bad_arguments_without_a_gpu():
    L = E.lib()
    P = lambda v: ctypes.c_void_p(v)
    assert L.ecf8_hbm_copy(P(0), P(0x200000), 16, None) == -1
    assert L.ecf8_hbm_copy(P(0x100008), P(0x200000), 16, None) == -1
    assert L.ecf8_hbm_copy(P(0), P(0), 0, None) == 0
    assert L.ecf8_hbm_stream(P(0x100000), 32, P(0x200000), 16, None) == -1       # reads more than it writes
    assert L.ecf8_hbm_stream(P(0x100000), 0, P(0x200000), 16, None) == -1
    assert L.ecf8_hbm_stream(P(0x100000), 24, P(0x200000), 32, None) == -1       # not whole 16-byte units
    assert L.ecf8_hbm_stream(P(0x100004), 16, P(0x200000), 32, None) == -1       # misaligned
    assert L.ecf8_hbm_stream(P(0), 16, P(0x200000), 32, None) == -1
    assert L.ecf8_hbm_stream(P(0x100000), 16, P(0x200000), 16 << 32, None) == -2
    assert L.ecf8_hbm_stream(P(0), 0, P(0), 0, None) == 0


# ---------------------------------------------------------------- alpha statistics

def test_alpha_hat_matches_oracle():
    rng = np.random.default_rng(11)
    for n in (2, 17, 1000, 100003):
        w = (rng.standard_cauchy(n) * 0.01).astype(np.float32)
        w[rng.integers(0, n)] = np.nan
        gamma = 0.001
        got = E.alpha_hat(w, gamma)
        ref = oracle.alpha_hat(w.astype(np.float64), gamma)
        assert abs(got - ref) <= 1e-12 * abs(ref), (n, got, ref)


def test_alpha_hat_rejects_undefined_cases():
    with pytest.raises(E.Ecf8Error):
        E.alpha_hat(np.ones(1, dtype=np.float32), 0.5)          # n < 2
    with pytest.raises(E.Ecf8Error):
        E.alpha_hat(np.ones(8, dtype=np.float32), 0.0)          # gamma <= 0
    with pytest.raises(E.Ecf8Error):
        E.alpha_hat(np.full(8, 0.5, dtype=np.float32), 0.5)     # max|w| <= gamma


def test_entropy_bound_matches_oracle():
    for a in (0.5, 1.0, 1.5, 1.9, 2.0):
        assert abs(E.exponent_entropy_bound(a) - oracle.entropy_bound(a)) < 1e-15
    assert np.isnan(E.exponent_entropy_bound(0.0))


def test_plan_block_order_checks_need_no_gpu():
    """ecf8_decode_run checks a plan's claim size before any launch: 1 and more than 1024 blocks
    per claim, and a claim counter that could pass 2^32, are argument errors."""
    ws = (ctypes.c_uint8 * 256)()
    base = dict(workspace=ctypes.cast(ws, ctypes.c_void_p), workspace_bytes=1 << 20, total_blocks=1000, count=1,
                chunk_bytes=16, threads_per_block=256, grid=100, short_codes=1)
    for claim, blocks, grid in ((1, 1000, 100), (1025, 1000, 100), (16, (1 << 32) - 100 * 16, 100),
                                (1024, 1 << 20, (1 << 22) + 1)):
        p = B.Plan(**dict(base, total_blocks=blocks, grid=grid))
        p.claim_blocks = claim
        assert B.lib().ecf8_decode_run(ctypes.byref(p), None) == -1, (claim, blocks, grid)  # ECF8_ERR_ARG
    assert ctypes.sizeof(B.Plan) == 48
