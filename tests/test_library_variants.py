"""Host half of the BF16 (DFloat11 layout) / E5M2 variants in libecf8 against the oracle (CPU only).

Code lengths: where several length-limited codes are optimal, the total
coded bits (unique) must equal the oracle's package-merge and the lengths
must form a complete prefix code within the limit.  Encode: byte-identical
buffers to the oracle's encode under the same code lengths.
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from lossless_entropy_coded_ecf8_amd import binding as B


def bf16(n, seed, scale=0.02, heavy=False):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(n, generator=g) * scale
    if heavy:
        x = x * torch.exp(torch.randn(n, generator=g) * 2.5)
    return x.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def e5m2(n, seed):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(n, generator=g) * 3).to(torch.float8_e5m2).view(torch.uint8).numpy()


def make(fmt, n, seed, heavy=False):
    return bf16(n, seed, heavy=heavy) if fmt == "bf16" else e5m2(n, seed)


@pytest.mark.parametrize("fmt", ["bf16", "e5m2"])
def test_histogram_matches_oracle(fmt):
    for n in (0, 1, 999, 123_457):
        x = make(fmt, n, n, heavy=True)
        assert np.array_equal(B.v_histogram(fmt, x), oracle.v_histogram(fmt, x))


@pytest.mark.parametrize("seed", range(40))
def test_code_lengths_optimal_like_the_oracle(seed):
    rng = np.random.default_rng(seed)
    nsym = 256 if seed % 2 == 0 else 32
    freq = np.zeros(nsym, dtype=np.uint64)
    k = int(rng.integers(2, nsym + 1))
    kind = seed % 4
    if kind == 0:
        w = rng.geometric(0.3, k)
    elif kind == 1:
        w = 2 ** rng.integers(0, 40, k)
    elif kind == 2:
        w = rng.integers(1, 1000, k)
    else:
        w = np.full(k, 5)
    freq[rng.choice(nsym, k, replace=False)] = w.astype(np.uint64)
    lo = int(np.ceil(np.log2(k))) if k > 1 else 1
    for L in sorted({max(lo, 1), max(lo, 8), 11, 16}):
        if L < lo:
            continue
        got = B.v_code_lengths(freq, L)
        ref = oracle.v_package_merge(freq, L)
        assert oracle.code_cost(freq, got) == oracle.code_cost(freq, ref), (seed, L)
        assert got.max() <= L and all(got[freq == 0] == 0) and all(got[freq > 0] > 0)
        assert abs(oracle.kraft_sum(got) - 1.0) < 1e-12


def test_code_lengths_errors_and_degenerate_cases():
    f = np.zeros(256, dtype=np.uint64)
    f[:] = 3
    with pytest.raises(B.Ecf8Error) as ei:
        B.v_code_lengths(f, 7)
    assert ei.value.code == -4
    with pytest.raises(B.Ecf8Error):
        B.v_code_lengths(f, 17)
    one = np.zeros(32, dtype=np.uint64)
    one[9] = 4
    assert list(B.v_code_lengths(one, 16)) == [1 if s == 9 else 0 for s in range(32)]
    assert B.v_code_lengths(np.zeros(32, dtype=np.uint64), 16).sum() == 0


@pytest.mark.parametrize("lengths", [[8] * 256, list(range(1, 16)) + [16, 16] + [0] * 239])
def test_canonical_codes_match_oracle(lengths):
    assert np.array_equal(B.v_canonical_codes(lengths), oracle.v_canonical_codes(lengths))


@pytest.mark.parametrize("fmt,n,heavy", [("bf16", 1, False), ("bf16", 17, False), ("bf16", 100_003, True),
                                         ("bf16", 400_000, False), ("e5m2", 1, False), ("e5m2", 33, False),
                                         ("e5m2", 250_001, False)])
@pytest.mark.parametrize("C,TB", [(16, 256), (16, 128), (4, 64), (12, 192)])
def test_encode_byte_identical_to_oracle(fmt, n, heavy, C, TB):
    x = make(fmt, n, n + C, heavy)
    L = oracle.v_lengths(fmt, x, 16)
    h = B.v_encode(fmt, x, lengths=L, chunk_bytes=C, threads_per_block=TB)
    r = oracle.v_encode(fmt, x, lengths=L, chunk_bytes=C, tb=TB)
    assert h.meta.total_bits == r["total_bits"]
    for k in ("n_chunks", "n_blocks", "stream_bytes", "raw_bytes", "gap_bytes"):
        assert getattr(h.meta, k) == r[k], k
    assert np.array_equal(h.stream, r["stream"])
    assert np.array_equal(h.raw, r["raw"])
    assert np.array_equal(h.gaps, r["gaps"])
    assert np.array_equal(h.blk_off, r["blk_off"])
    assert B.v_validate_meta(h.meta) == 0


@pytest.mark.parametrize("fmt", ["bf16", "e5m2"])
def test_default_lengths_decode_in_the_oracle(fmt):
    x = make(fmt, 77_777, 3, heavy=True)
    h = B.v_encode(fmt, x)
    assert h.meta.max_len <= 16
    assert np.array_equal(oracle.v_decode(fmt, h.stream, h.raw, x.size, h.lengths), x)


def test_length_limit_binds_on_heavy_bf16():
    """Heavy-tailed BF16 weights: the unlimited Huffman depth passes 11, a limit of 11 is met optimally."""
    x = bf16(1 << 18, 5, heavy=True)
    f = oracle.v_histogram("bf16", x)
    assert oracle.v_huffman_lengths(f).max() > 11
    h = B.v_encode("bf16", x, max_len=11)
    assert h.meta.max_len == 11
    assert oracle.code_cost(f, h.lengths) == oracle.code_cost(f, oracle.v_package_merge(f, 11))
    assert np.array_equal(oracle.v_decode("bf16", h.stream, h.raw, x.size, h.lengths), x)


def test_validate_meta_rejects_corruption():
    x = make("bf16", 5000, 1)
    m = B.v_encode("bf16", x).meta

    def bad(mut):
        mm = B.MetaV.from_buffer_copy(m)
        mut(mm)
        return B.v_validate_meta(mm)
    assert bad(lambda mm: None) == 0
    assert bad(lambda mm: setattr(mm, "format", 3)) == -3
    assert bad(lambda mm: setattr(mm, "total_bits", mm.total_bits + 1000)) == -3
    assert bad(lambda mm: setattr(mm, "max_len", mm.max_len + 1)) == -3
    assert bad(lambda mm: setattr(mm, "chunk_bytes", 6)) == -3

    def kraft(mm):
        s = int(np.argmax(list(mm.len)))
        mm.len[s] = mm.len[s] + 1
    assert bad(kraft) == -3
    e = B.v_encode("e5m2", make("e5m2", 100, 2)).meta
    mm = B.MetaV.from_buffer_copy(e)
    mm.len[40] = 3                                   # past E5M2's 32 symbols
    assert B.v_validate_meta(mm) == -3


def test_encode_rejects_bad_arguments():
    x = make("bf16", 1000, 4)
    with pytest.raises(B.Ecf8Error) as ei:
        B.v_encode("bf16", x, chunk_bytes=6)
    assert ei.value.code == -1
    L = oracle.v_lengths("bf16", x)
    L2 = L.copy()
    L2[int(np.nonzero(L)[0][0])] = 0                 # a present symbol without a code
    with pytest.raises(B.Ecf8Error) as ei:
        B.v_encode("bf16", x, lengths=L2)
    assert ei.value.code == -3
    assert B.lib().ecf8v_nsym(7) == -1


def test_variant_workspace_and_prepare_checks_need_no_gpu():
    """Rejections before any device work (fake device pointers)."""
    lib = B.lib()
    assert lib.ecf8v_workspace_bytes(0) < lib.ecf8v_workspace_bytes(3)
    x = make("bf16", 3000, 6)
    h = B.v_encode("bf16", x)
    d = (B.TensorDescV * 1)()
    d[0].stream, d[0].raw, d[0].gaps, d[0].blk_off = 0x100000, 0x200000, 0x300000, 0x400000
    d[0].meta = h.meta
    plan = B.PlanV()
    ws_bytes = lib.ecf8v_workspace_bytes(1)
    call = lambda ws, wsb, desc=d: lib.ecf8v_decode_prepare(desc, 1, ctypes.c_void_p(0x500000), ctypes.c_void_p(ws),
                                                            wsb, None, ctypes.byref(plan))
    assert call(0x600010, ws_bytes) == -7
    assert call(0x600000, ws_bytes - 1) == -7
    d2 = (B.TensorDescV * 1)()
    ctypes.memmove(ctypes.addressof(d2), ctypes.addressof(d), ctypes.sizeof(d))
    d2[0].meta.chunk_bytes = 8
    assert call(0x600000, ws_bytes, d2) == -3                     # chunk_bytes disagrees with the layout
    h8 = B.v_encode("bf16", x, chunk_bytes=8)
    d2[0].meta = h8.meta
    assert call(0x600000, ws_bytes, d2) == -4                     # valid, no kernel for C = 8
    d2[0].meta = h.meta
    d2[0].stream = 0x100008
    assert call(0x600000, ws_bytes, d2) == -1                     # misaligned stream
