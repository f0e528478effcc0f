"""CPU oracle for ECF8 -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product (``lossless_entropy_coded_ecf8_amd``)
never imports it, and this package never imports the product: the two are
independent implementations of the same format so that each can check the other.

The arithmetic lives in ``ecf8_oracle.c`` (E4M3) and ``ecf8v_oracle.c`` (the
BF16 / DFloat11 and E5M2 variants, with package-merge length limiting), plain
C, one bit at a time; this module only marshals numpy arrays into them and
adds the fp64 statistics the pages quote (entropy, average code length).

Sources: the ECF8 technical blog (codearts.csdn.net), sections 2.2 (exponent
entropy), 3.1.1 (Huffman coding of the exponent) and 3.2.1 (chunked parallel
decode with per-thread gaps); the ECF8 paper abstract (arXiv 2510.02676,
lossless / bit-exact).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ecf8_oracle.c")
_SRCV = os.path.join(_HERE, "ecf8v_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

_u8p = ctypes.POINTER(ctypes.c_uint8)
_u64p = ctypes.POINTER(ctypes.c_uint64)
_intp = ctypes.POINTER(ctypes.c_int)
_u32p = ctypes.POINTER(ctypes.c_uint32)


def build(force: bool = False) -> str:
    """Compile the oracle with gcc into oracle/liboracle.so."""
    newest = max(os.path.getmtime(_SRC), os.path.getmtime(_SRCV))
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < newest:
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c99", "-Wall", "-Wextra", "-shared", "-fPIC",
                               _SRC, _SRCV, "-o", tmp])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        L = ctypes.CDLL(_LIB)
        L.oracle_histogram.argtypes = [_u8p, ctypes.c_uint64, _u64p]
        L.oracle_huffman_lengths.argtypes = [_u64p, _intp]
        L.oracle_huffman_lengths.restype = ctypes.c_int
        L.oracle_canonical_codes.argtypes = [_intp, _u32p]
        L.oracle_canonical_codes.restype = ctypes.c_int
        L.oracle_total_bits.argtypes = [_u8p, ctypes.c_uint64, _intp]
        L.oracle_total_bits.restype = ctypes.c_uint64
        L.oracle_sizes.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint32,
                                   _u64p, _u64p, _u64p, _u64p, _u64p]
        L.oracle_encode.argtypes = [_u8p, ctypes.c_uint64, _intp, ctypes.c_uint32, ctypes.c_uint32,
                                    _u8p, _u8p, _u8p, _u64p]
        L.oracle_encode.restype = ctypes.c_uint64
        L.oracle_decode_range.argtypes = [_u8p, ctypes.c_uint64, _u8p, _intp, ctypes.c_uint64,
                                          ctypes.c_uint64, ctypes.c_uint64, _u8p]
        L.oracle_decode_range.restype = ctypes.c_uint64
        L.oracle_decode.argtypes = [_u8p, ctypes.c_uint64, _u8p, ctypes.c_uint64, _intp, _u8p]
        L.oracle_decode.restype = ctypes.c_uint64
        L.oracle_check_layout.argtypes = [_u8p, ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint64,
                                          _intp, ctypes.c_uint32, ctypes.c_uint32, _u8p, _u64p]
        L.oracle_check_layout.restype = ctypes.c_int64
        L.oracle_chunk_count.argtypes = [_u8p, ctypes.c_uint64, ctypes.c_uint64, _intp, ctypes.c_uint32,
                                         ctypes.c_uint64, ctypes.c_uint32]
        L.oracle_chunk_count.restype = ctypes.c_int64
        # format variants (ecf8v_oracle.c)
        L.oraclev_nsym.argtypes = [ctypes.c_int]
        L.oraclev_nsym.restype = ctypes.c_int
        L.oraclev_histogram.argtypes = [ctypes.c_int, _u8p, ctypes.c_uint64, _u64p]
        L.oraclev_huffman_lengths.argtypes = [_u64p, ctypes.c_int, _intp]
        L.oraclev_huffman_lengths.restype = ctypes.c_int
        L.oraclev_package_merge.argtypes = [_u64p, ctypes.c_int, ctypes.c_int, _intp]
        L.oraclev_package_merge.restype = ctypes.c_int
        L.oraclev_canonical_codes.argtypes = [_intp, ctypes.c_int, _u32p]
        L.oraclev_canonical_codes.restype = ctypes.c_int
        L.oraclev_total_bits.argtypes = [ctypes.c_int, _u8p, ctypes.c_uint64, _intp]
        L.oraclev_total_bits.restype = ctypes.c_uint64
        L.oraclev_raw_bytes.argtypes = [ctypes.c_int, ctypes.c_uint64]
        L.oraclev_raw_bytes.restype = ctypes.c_uint64
        L.oraclev_sizes.argtypes = [ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint32, _u64p, _u64p, _u64p, _u64p]
        L.oraclev_encode.argtypes = [ctypes.c_int, _u8p, ctypes.c_uint64, _intp, ctypes.c_uint32, ctypes.c_uint32,
                                     _u8p, _u8p, _u8p, _u64p]
        L.oraclev_encode.restype = ctypes.c_uint64
        L.oraclev_decode_range.argtypes = [ctypes.c_int, _u8p, ctypes.c_uint64, _u8p, _intp, ctypes.c_uint64,
                                           ctypes.c_uint64, ctypes.c_uint64, _u8p]
        L.oraclev_decode_range.restype = ctypes.c_uint64
        L.oraclev_decode.argtypes = [ctypes.c_int, _u8p, ctypes.c_uint64, _u8p, ctypes.c_uint64, _intp, _u8p]
        L.oraclev_decode.restype = ctypes.c_uint64
        _lib = L
    return _lib


def _p(a, t):
    return a.ctypes.data_as(t)


def _c8(a):
    a = np.ascontiguousarray(a, dtype=np.uint8)
    return a


def histogram(x: np.ndarray) -> np.ndarray:
    x = _c8(x)
    f = np.zeros(16, dtype=np.uint64)
    lib().oracle_histogram(_p(x, _u8p), x.size, _p(f, _u64p))
    return f


def huffman_lengths(freq) -> np.ndarray:
    f = np.ascontiguousarray(np.asarray(freq, dtype=np.uint64))
    assert f.size == 16
    L = np.zeros(16, dtype=np.intc)
    lib().oracle_huffman_lengths(_p(f, _u64p), _p(L, _intp))
    return L.astype(np.int64)


def canonical_codes(lengths) -> np.ndarray:
    L = np.ascontiguousarray(np.asarray(lengths, dtype=np.intc))
    c = np.zeros(16, dtype=np.uint32)
    rc = lib().oracle_canonical_codes(_p(L, _intp), _p(c, _u32p))
    if rc != 0:
        raise ValueError("bad code lengths")
    return c.astype(np.int64)


def sizes(n: int, total_bits: int, chunk_bytes: int, tb: int) -> dict:
    out = [ctypes.c_uint64() for _ in range(5)]
    lib().oracle_sizes(n, total_bits, chunk_bytes, tb, *[ctypes.byref(o) for o in out])
    keys = ["n_chunks", "n_blocks", "stream_bytes", "nibble_bytes", "gap_bytes"]
    return {k: int(o.value) for k, o in zip(keys, out)}


def encode(x: np.ndarray, lengths=None, chunk_bytes: int = 16, tb: int = 256) -> dict:
    """Histogram -> Huffman lengths (unless given) -> canonical code -> encode."""
    x = _c8(x).ravel()
    n = x.size
    if lengths is None:
        lengths = huffman_lengths(histogram(x))
    L = np.ascontiguousarray(np.asarray(lengths, dtype=np.intc))
    T = int(lib().oracle_total_bits(_p(x, _u8p), n, _p(L, _intp)))
    sz = sizes(n, T, chunk_bytes, tb)
    stream = np.zeros(sz["stream_bytes"], dtype=np.uint8)
    nib = np.zeros(sz["nibble_bytes"], dtype=np.uint8)
    gaps = np.zeros(sz["gap_bytes"], dtype=np.uint8)
    blk = np.zeros(sz["n_blocks"] + 1, dtype=np.uint64)
    T2 = lib().oracle_encode(_p(x, _u8p), n, _p(L, _intp), chunk_bytes, tb,
                             _p(stream, _u8p), _p(nib, _u8p), _p(gaps, _u8p), _p(blk, _u64p))
    if T2 == (1 << 64) - 1:
        raise ValueError("oracle_encode: element with a zero-length code")
    assert T2 == T
    return dict(n=n, total_bits=T, lengths=L.astype(np.int64), chunk_bytes=chunk_bytes, tb=tb,
                stream=stream, nibbles=nib, gaps=gaps, blk_off=blk, **sz)


def decode(stream, nibbles, n: int, lengths) -> np.ndarray:
    stream = _c8(stream)
    nibbles = _c8(nibbles)
    L = np.ascontiguousarray(np.asarray(lengths, dtype=np.intc))
    out = np.zeros(max(n, 1), dtype=np.uint8)
    r = lib().oracle_decode(_p(stream, _u8p), stream.size, _p(nibbles, _u8p), n, _p(L, _intp),
                            _p(out, _u8p))
    if r == (1 << 64) - 1:
        raise ValueError("oracle_decode: invalid code in stream")
    return out[:n]


def decode_range(stream, nibbles, lengths, start_bit: int, first_elem: int, count: int):
    """Decode `count` elements starting at codeword bit `start_bit`.
    Returns (bytes, end_bit)."""
    stream = _c8(stream)
    nibbles = _c8(nibbles)
    L = np.ascontiguousarray(np.asarray(lengths, dtype=np.intc))
    out = np.zeros(max(count, 1), dtype=np.uint8)
    r = lib().oracle_decode_range(_p(stream, _u8p), stream.size, _p(nibbles, _u8p), _p(L, _intp),
                                  start_bit, first_elem, count, _p(out, _u8p))
    if r == (1 << 64) - 1:
        raise ValueError("oracle_decode_range: invalid code in stream")
    return out[:count], int(r)


def check_layout(stream, n: int, total_bits: int, lengths, chunk_bytes: int, tb: int,
                 gaps, blk_off) -> int:
    """0 if the stored gaps / block offsets match a fresh bit walk."""
    stream = _c8(stream)
    gaps = _c8(gaps)
    blk = np.ascontiguousarray(np.asarray(blk_off, dtype=np.uint64))
    L = np.ascontiguousarray(np.asarray(lengths, dtype=np.intc))
    return int(lib().oracle_check_layout(_p(stream, _u8p), stream.size, n, total_bits, _p(L, _intp),
                                         chunk_bytes, tb, _p(gaps, _u8p), _p(blk, _u64p)))


def chunk_count(stream, total_bits: int, lengths, chunk_bytes: int, t: int, gap: int) -> int:
    """Codewords a thread counts in chunk t from stored gap `gap` (ECF8 blog §3.2.1 count step);
    -1 on an invalid codeword."""
    stream = _c8(stream)
    L = np.ascontiguousarray(np.asarray(lengths, dtype=np.intc))
    return int(lib().oracle_chunk_count(_p(stream, _u8p), stream.size, total_bits, _p(L, _intp), chunk_bytes,
                                        t, gap))


def block_counts(stream, gaps, total_bits: int, lengths, chunk_bytes: int, tb: int, n_blocks: int):
    """Per block, the sum of its chunks' counts from their stored gaps (what a block-wide reduction of
    the count step gives); None for a block with an invalid codeword."""
    gaps = _c8(gaps)
    out = []
    for b in range(n_blocks):
        tot = 0
        for t in range(b * tb, (b + 1) * tb):
            c = chunk_count(stream, total_bits, lengths, chunk_bytes, t, (int(gaps[t >> 1]) >> (4 * (t & 1))) & 15)
            if c < 0:
                tot = None
                break
            tot += c
        out.append(tot)
    return out


# ---- format variants: BF16 (DFloat11 layout) and FP8 E5M2 (ecf8v_oracle.c) ----

BF16, E5M2 = 1, 2
FORMATS = {"bf16": BF16, "e5m2": E5M2}


def _fmt(fmt) -> int:
    return FORMATS[fmt] if isinstance(fmt, str) else int(fmt)


def _elems(fmt, x):
    """(bytes, n): a BF16 input is uint16 values (or their little-endian bytes); E5M2 is bytes."""
    f = _fmt(fmt)
    a = np.ascontiguousarray(x)
    if f == BF16:
        a = np.ascontiguousarray(a.view(np.uint16) if a.dtype != np.uint16 else a).astype("<u2")
        return a.view(np.uint8), a.size
    a = _c8(a)
    return a, a.size


def v_nsym(fmt) -> int:
    return int(lib().oraclev_nsym(_fmt(fmt)))


def v_histogram(fmt, x) -> np.ndarray:
    b, n = _elems(fmt, x)
    f = np.zeros(v_nsym(fmt), dtype=np.uint64)
    lib().oraclev_histogram(_fmt(fmt), _p(b, _u8p), n, _p(f, _u64p))
    return f


def v_huffman_lengths(freq) -> np.ndarray:
    f = np.ascontiguousarray(np.asarray(freq, dtype=np.uint64))
    L = np.zeros(f.size, dtype=np.intc)
    lib().oraclev_huffman_lengths(_p(f, _u64p), f.size, _p(L, _intp))
    return L.astype(np.int64)


def v_package_merge(freq, max_len: int) -> np.ndarray:
    """Optimal code lengths no longer than max_len (package-merge); raises if impossible."""
    f = np.ascontiguousarray(np.asarray(freq, dtype=np.uint64))
    L = np.zeros(f.size, dtype=np.intc)
    r = lib().oraclev_package_merge(_p(f, _u64p), f.size, int(max_len), _p(L, _intp))
    if r < 0:
        raise ValueError("no prefix code with lengths <= %d for %d symbols" % (max_len, int((f > 0).sum())))
    return L.astype(np.int64)


def v_lengths(fmt, x, max_len: int = 16) -> np.ndarray:
    """Huffman lengths of x's exponent histogram, length-limited to max_len by package-merge."""
    return v_package_merge(v_histogram(fmt, x), max_len)


def v_canonical_codes(lengths) -> np.ndarray:
    L = np.ascontiguousarray(np.asarray(lengths, dtype=np.intc))
    c = np.zeros(L.size, dtype=np.uint32)
    if lib().oraclev_canonical_codes(_p(L, _intp), L.size, _p(c, _u32p)) != 0:
        raise ValueError("bad code lengths")
    return c.astype(np.int64)


def v_encode(fmt, x, lengths=None, chunk_bytes: int = 16, tb: int = 256, max_len: int = 16) -> dict:
    f = _fmt(fmt)
    b, n = _elems(fmt, x)
    if lengths is None:
        lengths = v_lengths(fmt, x, max_len)
    L = np.ascontiguousarray(np.asarray(lengths, dtype=np.intc))
    T = int(lib().oraclev_total_bits(f, _p(b, _u8p), n, _p(L, _intp)))
    out = [ctypes.c_uint64() for _ in range(4)]
    lib().oraclev_sizes(T, chunk_bytes, tb, *[ctypes.byref(o) for o in out])
    keys = ["n_chunks", "n_blocks", "stream_bytes", "gap_bytes"]
    sz = {k: int(o.value) for k, o in zip(keys, out)}
    sz["raw_bytes"] = int(lib().oraclev_raw_bytes(f, n))
    stream = np.zeros(sz["stream_bytes"], dtype=np.uint8)
    raw = np.zeros(max(sz["raw_bytes"], 1), dtype=np.uint8)
    gaps = np.zeros(max(sz["gap_bytes"], 1), dtype=np.uint8)
    blk = np.zeros(sz["n_blocks"] + 1, dtype=np.uint64)
    T2 = lib().oraclev_encode(f, _p(b, _u8p), n, _p(L, _intp), chunk_bytes, tb, _p(stream, _u8p), _p(raw, _u8p),
                              _p(gaps, _u8p), _p(blk, _u64p))
    if T2 == (1 << 64) - 1:
        raise ValueError("oraclev_encode: element with a zero-length code")
    assert T2 == T
    return dict(fmt=f, n=n, total_bits=T, lengths=L.astype(np.int64), chunk_bytes=chunk_bytes, tb=tb,
                stream=stream, raw=raw[:sz["raw_bytes"]], gaps=gaps[:sz["gap_bytes"]], blk_off=blk, **sz)


def v_decode(fmt, stream, raw, n: int, lengths) -> np.ndarray:
    """Bit-serial decode; returns uint16 values (BF16) or bytes (E5M2)."""
    f = _fmt(fmt)
    stream, raw = _c8(stream), _c8(raw)
    L = np.ascontiguousarray(np.asarray(lengths, dtype=np.intc))
    eb = 2 if f == BF16 else 1
    out = np.zeros(max(n * eb, 1), dtype=np.uint8)
    r = lib().oraclev_decode(f, _p(stream, _u8p), stream.size, _p(raw, _u8p), n, _p(L, _intp), _p(out, _u8p))
    if r == (1 << 64) - 1:
        raise ValueError("oraclev_decode: invalid code in stream")
    out = out[: n * eb]
    return out.view("<u2") if f == BF16 else out


def v_decode_range(fmt, stream, raw, lengths, start_bit: int, first_elem: int, count: int):
    f = _fmt(fmt)
    stream, raw = _c8(stream), _c8(raw)
    L = np.ascontiguousarray(np.asarray(lengths, dtype=np.intc))
    eb = 2 if f == BF16 else 1
    out = np.zeros(max(count * eb, 1), dtype=np.uint8)
    r = lib().oraclev_decode_range(f, _p(stream, _u8p), stream.size, _p(raw, _u8p), _p(L, _intp), start_bit,
                                   first_elem, count, _p(out, _u8p))
    if r == (1 << 64) - 1:
        raise ValueError("oraclev_decode_range: invalid code in stream")
    out = out[: count * eb]
    return (out.view("<u2") if f == BF16 else out), int(r)


def code_cost(freq, lengths) -> int:
    """Total coded bits sum freq_s * len_s (exact integer)."""
    return int(sum(int(f) * int(l) for f, l in zip(freq, lengths)))


# ---- fp64 statistics quoted by the pages (ECF8 blog §2.2, §3.1.1) ----

def entropy_bits(freq) -> float:
    """Shannon entropy H = -sum p log2 p of the exponent histogram (fp64)."""
    f = np.asarray(freq, dtype=np.float64)
    tot = f.sum()
    if tot == 0:
        return 0.0
    p = f[f > 0] / tot
    return float(-(p * np.log2(p)).sum())


def average_length(freq, lengths) -> float:
    """Expected code length sum p_s * len_s (fp64)."""
    f = np.asarray(freq, dtype=np.float64)
    tot = f.sum()
    if tot == 0:
        return 0.0
    return float((f * np.asarray(lengths, dtype=np.float64)).sum() / tot)


def kraft_sum(lengths) -> float:
    L = [int(l) for l in lengths if int(l) > 0]
    return float(sum(2.0 ** -l for l in L))


# ---------------------------------------------------------------- alpha statistics

def alpha_hat(w, gamma: float) -> float:
    """ECF8 blog §6: alpha_hat = log N / log(max |w_i| / gamma), fp64 (NaN weights skipped)."""
    a = np.abs(np.asarray(w, dtype=np.float64).ravel())
    a = a[~np.isnan(a)]
    return float(np.log(np.float64(np.asarray(w).size)) / np.log(a.max() / gamma))


def entropy_bound(alpha: float) -> float:
    """ECF8 blog §2.2: H(E) <= alpha / (1 - 2^-alpha) bits for an alpha-stable weight."""
    return float(alpha / (1.0 - 2.0 ** (-alpha)))
