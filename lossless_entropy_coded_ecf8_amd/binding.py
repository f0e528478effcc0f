"""ctypes binding of libecf8.so (include/ecf8.h).

Argument marshalling only: every step of encode runs in the library's host
code and every step of decode runs in its HIP kernels.  PyTorch provides
device memory and the current HIP stream.  If the library is not built the
import fails loudly -- there is no Python or CPU fallback.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
from typing import List, Optional, Sequence

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libecf8.so")

NSYM = 16
DEFAULT_CHUNK_BYTES = 16
DEFAULT_THREADS_PER_BLOCK = 256

ERRORS = {0: "ok", -1: "ECF8_ERR_ARG", -2: "ECF8_ERR_SIZE", -3: "ECF8_ERR_META",
          -4: "ECF8_ERR_UNSUPPORTED", -5: "ECF8_ERR_CORRUPT", -6: "ECF8_ERR_HIP",
          -7: "ECF8_ERR_WORKSPACE"}


class Ecf8Error(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__("%s failed: %s (%d)" % (where, ERRORS.get(code, "?"), code))


class Codebook(ctypes.Structure):
    _fields_ = [("len", ctypes.c_uint8 * NSYM)]


class Params(ctypes.Structure):
    _fields_ = [("chunk_bytes", ctypes.c_uint32), ("threads_per_block", ctypes.c_uint32)]


class Meta(ctypes.Structure):
    _fields_ = [("n", ctypes.c_uint64), ("total_bits", ctypes.c_uint64), ("n_chunks", ctypes.c_uint64),
                ("n_blocks", ctypes.c_uint64), ("stream_bytes", ctypes.c_uint64),
                ("nibble_bytes", ctypes.c_uint64), ("gap_bytes", ctypes.c_uint64),
                ("chunk_bytes", ctypes.c_uint32), ("threads_per_block", ctypes.c_uint32),
                ("cb", Codebook), ("max_len", ctypes.c_uint32), ("reserved", ctypes.c_uint32)]


class Stream(ctypes.Structure):
    _fields_ = [("stream", ctypes.c_void_p), ("nibbles", ctypes.c_void_p), ("gaps", ctypes.c_void_p),
                ("blk_off", ctypes.c_void_p)]


class TensorDesc(ctypes.Structure):
    _fields_ = [("s", Stream), ("meta", Meta), ("out_offset", ctypes.c_uint64)]


class EncodeJob(ctypes.Structure):
    _fields_ = [("fp8", ctypes.c_void_p), ("meta", Meta), ("stream", ctypes.c_void_p), ("nibbles", ctypes.c_void_p),
                ("gaps", ctypes.c_void_p), ("blk_off", ctypes.c_void_p), ("workspace", ctypes.c_void_p),
                ("workspace_bytes", ctypes.c_uint64)]


class Plan(ctypes.Structure):
    _fields_ = [("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_uint64),
                ("total_blocks", ctypes.c_uint64), ("count", ctypes.c_uint32),
                ("chunk_bytes", ctypes.c_uint32), ("threads_per_block", ctypes.c_uint32),
                ("grid", ctypes.c_uint32), ("short_codes", ctypes.c_uint32),
                ("claim_blocks", ctypes.c_uint32)]


MAXSYM_V = 256
FORMAT_V = {"bf16": 1, "e5m2": 2}


class MetaV(ctypes.Structure):
    _fields_ = [("n", ctypes.c_uint64), ("total_bits", ctypes.c_uint64), ("n_chunks", ctypes.c_uint64),
                ("n_blocks", ctypes.c_uint64), ("stream_bytes", ctypes.c_uint64), ("raw_bytes", ctypes.c_uint64),
                ("gap_bytes", ctypes.c_uint64), ("chunk_bytes", ctypes.c_uint32),
                ("threads_per_block", ctypes.c_uint32), ("format", ctypes.c_uint32), ("max_len", ctypes.c_uint32),
                ("len", ctypes.c_uint8 * MAXSYM_V)]


class TensorDescV(ctypes.Structure):
    _fields_ = [("stream", ctypes.c_void_p), ("raw", ctypes.c_void_p), ("gaps", ctypes.c_void_p),
                ("blk_off", ctypes.c_void_p), ("meta", MetaV), ("out_offset", ctypes.c_uint64)]


class PlanV(ctypes.Structure):
    _fields_ = [("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_uint64),
                ("total_blocks", ctypes.c_uint64), ("count", ctypes.c_uint32), ("format", ctypes.c_uint32),
                ("threads_per_block", ctypes.c_uint32), ("grid", ctypes.c_uint32),
                ("table_entries", ctypes.c_uint32), ("short_codes", ctypes.c_uint32)]


EXPORTS_V = ["ecf8v_nsym", "ecf8v_histogram", "ecf8v_code_lengths", "ecf8v_canonical_codes", "ecf8v_encode_sizes",
             "ecf8v_encode", "ecf8v_validate_meta", "ecf8v_workspace_bytes", "ecf8v_decode_prepare",
             "ecf8v_decode_run", "ecf8v_decode_run_timed", "ecf8v_decode_status"]

EXPORTS = ["ecf8_histogram", "ecf8_codebook_from_freq", "ecf8_build_codebook", "ecf8_canonical_codes",
           "ecf8_encode_sizes", "ecf8_encode", "ecf8_validate_meta", "ecf8_workspace_bytes",
           "ecf8_decode_prepare", "ecf8_decode_run", "ecf8_decode_run_timed", "ecf8_decode_batched", "ecf8_decode", "ecf8_decode_batched_noalloc",
           "ecf8_decode_status", "ecf8_histogram_device", "ecf8_meta_from_freq", "ecf8_encode_workspace_bytes",
           "ecf8_encode_device", "ecf8_encode_batched_device", "ecf8_alpha_hat", "ecf8_exponent_entropy_bound", "ecf8_hbm_copy", "ecf8_hbm_stream",
           "ecf8_strerror", "ecf8_version"]

_lib = None


def lib() -> ctypes.CDLL:
    """Load libecf8.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("libecf8.so is not built; run `python -m lossless_entropy_coded_ecf8_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    u8p, u64p, u32p, vp = (ctypes.POINTER(ctypes.c_uint8), ctypes.POINTER(ctypes.c_uint64),
                           ctypes.POINTER(ctypes.c_uint32), ctypes.c_void_p)
    i = ctypes.c_int
    sig = {
        "ecf8_histogram": (i, [vp, ctypes.c_uint64, u64p]),
        "ecf8_codebook_from_freq": (i, [u64p, ctypes.c_uint32, ctypes.POINTER(Codebook)]),
        "ecf8_build_codebook": (i, [vp, ctypes.c_uint64, ctypes.c_uint32, ctypes.POINTER(Codebook)]),
        "ecf8_canonical_codes": (i, [ctypes.POINTER(Codebook), u32p]),
        "ecf8_encode_sizes": (i, [vp, ctypes.c_uint64, ctypes.POINTER(Codebook), ctypes.POINTER(Params),
                                  ctypes.POINTER(Meta)]),
        "ecf8_encode": (i, [vp, ctypes.c_uint64, ctypes.POINTER(Codebook), ctypes.POINTER(Params),
                            vp, ctypes.c_uint64, vp, ctypes.c_uint64, vp, ctypes.c_uint64, vp,
                            ctypes.c_uint64, ctypes.POINTER(Meta)]),
        "ecf8_validate_meta": (i, [ctypes.POINTER(Meta)]),
        "ecf8_workspace_bytes": (ctypes.c_uint64, [i]),
        "ecf8_decode_prepare": (i, [ctypes.POINTER(TensorDesc), i, vp, vp, ctypes.c_uint64, vp,
                                    ctypes.POINTER(Plan)]),
        "ecf8_decode_run": (i, [ctypes.POINTER(Plan), vp]),
        "ecf8_decode_run_timed": (i, [ctypes.POINTER(Plan), vp, vp, vp]),
        "ecf8_decode_batched": (i, [ctypes.POINTER(TensorDesc), i, vp, vp, ctypes.c_uint64, vp]),
        "ecf8_decode": (i, [ctypes.POINTER(Stream), ctypes.POINTER(Meta), vp, ctypes.c_uint64, vp,
                            ctypes.c_uint64, vp]),
        "ecf8_decode_batched_noalloc": (i, [ctypes.POINTER(TensorDesc), i, vp, vp, vp]),
        "ecf8_decode_status": (i, [vp, vp, u64p]),
        "ecf8_histogram_device": (i, [vp, ctypes.c_uint64, vp, vp, ctypes.c_uint64, vp]),
        "ecf8_meta_from_freq": (i, [u64p, ctypes.c_uint64, ctypes.POINTER(Codebook), ctypes.POINTER(Params),
                                    ctypes.POINTER(Meta)]),
        "ecf8_encode_workspace_bytes": (ctypes.c_uint64, [ctypes.c_uint64]),
        "ecf8_encode_device": (i, [vp, ctypes.POINTER(Meta), vp, vp, vp, vp, vp, ctypes.c_uint64, vp]),
        "ecf8_encode_batched_device": (i, [ctypes.POINTER(EncodeJob), i, vp]),
        "ecf8_alpha_hat": (i, [vp, ctypes.c_uint64, ctypes.c_double, ctypes.POINTER(ctypes.c_double)]),
        "ecf8_exponent_entropy_bound": (ctypes.c_double, [ctypes.c_double]),
        "ecf8_hbm_copy": (i, [vp, vp, ctypes.c_uint64, vp]),
        "ecf8_hbm_stream": (i, [vp, ctypes.c_uint64, vp, ctypes.c_uint64, vp]),
        "ecf8_strerror": (ctypes.c_char_p, [i]),
        "ecf8_version": (i, []),
    }
    sig.update({
        "ecf8v_nsym": (i, [ctypes.c_uint32]),
        "ecf8v_histogram": (i, [ctypes.c_uint32, vp, ctypes.c_uint64, u64p]),
        "ecf8v_code_lengths": (i, [u64p, ctypes.c_uint32, ctypes.c_uint32, u8p]),
        "ecf8v_canonical_codes": (i, [u8p, ctypes.c_uint32, u32p]),
        "ecf8v_encode_sizes": (i, [ctypes.c_uint32, vp, ctypes.c_uint64, u8p, ctypes.POINTER(Params),
                                   ctypes.POINTER(MetaV)]),
        "ecf8v_encode": (i, [ctypes.c_uint32, vp, ctypes.c_uint64, u8p, ctypes.POINTER(Params), vp, ctypes.c_uint64,
                             vp, ctypes.c_uint64, vp, ctypes.c_uint64, vp, ctypes.c_uint64, ctypes.POINTER(MetaV)]),
        "ecf8v_validate_meta": (i, [ctypes.POINTER(MetaV)]),
        "ecf8v_workspace_bytes": (ctypes.c_uint64, [i]),
        "ecf8v_decode_prepare": (i, [ctypes.POINTER(TensorDescV), i, vp, vp, ctypes.c_uint64, vp,
                                     ctypes.POINTER(PlanV)]),
        "ecf8v_decode_run": (i, [ctypes.POINTER(PlanV), vp]),
        "ecf8v_decode_run_timed": (i, [ctypes.POINTER(PlanV), vp, vp, vp]),
        "ecf8v_decode_status": (i, [vp, vp, u64p]),
    })
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args
    _lib = L
    return L


def _check(rc: int, where: str):
    if rc != 0:
        raise Ecf8Error(rc, where)


def _u8(x) -> np.ndarray:
    if hasattr(x, "detach"):  # torch tensor on the CPU
        x = x.detach().cpu().contiguous().view(-1).numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.uint8).reshape(-1))


def _ptr(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data) if a.size else ctypes.c_void_p(0)


# ------------------------------------------------------------------ host side

def histogram(x) -> np.ndarray:
    a = _u8(x)
    f = (ctypes.c_uint64 * NSYM)()
    _check(lib().ecf8_histogram(_ptr(a), a.size, f), "ecf8_histogram")
    return np.array(list(f), dtype=np.uint64)


def codebook_from_freq(freq, max_len: int = 16) -> np.ndarray:
    f = (ctypes.c_uint64 * NSYM)(*[int(v) for v in freq])
    cb = Codebook()
    _check(lib().ecf8_codebook_from_freq(f, max_len, ctypes.byref(cb)), "ecf8_codebook_from_freq")
    return np.array(list(cb.len), dtype=np.int64)


def build_codebook(x, max_len: int = 16) -> np.ndarray:
    a = _u8(x)
    cb = Codebook()
    _check(lib().ecf8_build_codebook(_ptr(a), a.size, max_len, ctypes.byref(cb)), "ecf8_build_codebook")
    return np.array(list(cb.len), dtype=np.int64)


def _codebook(lengths) -> Codebook:
    cb = Codebook()
    for s, l in enumerate(lengths):
        cb.len[s] = int(l)
    return cb


def canonical_codes(lengths) -> np.ndarray:
    out = (ctypes.c_uint32 * NSYM)()
    cb = _codebook(lengths)
    _check(lib().ecf8_canonical_codes(ctypes.byref(cb), out), "ecf8_canonical_codes")
    return np.array(list(out), dtype=np.int64)


def meta_dict(m: Meta) -> dict:
    d = {k: getattr(m, k) for k, _ in Meta._fields_ if k not in ("cb", "reserved")}
    d["lengths"] = list(m.cb.len)
    return d


def compressed_bytes(m: Meta) -> int:
    """Bytes one decode must read: stream payload, nibble plane, gaps, block offsets."""
    return int((m.total_bits + 7) // 8 + (m.n + 1) // 2 + (m.n_chunks + 1) // 2 + 8 * (m.n_blocks + 1))


@dataclasses.dataclass
class Encoded:
    """Host-side encoded tensor (numpy buffers in the include/ecf8.h layout)."""
    meta: Meta
    stream: np.ndarray
    nibbles: np.ndarray
    gaps: np.ndarray
    blk_off: np.ndarray
    shape: tuple = ()

    @property
    def n(self) -> int:
        return int(self.meta.n)

    @property
    def lengths(self) -> np.ndarray:
        return np.array(list(self.meta.cb.len), dtype=np.int64)

    def compressed_bytes(self) -> int:
        return compressed_bytes(self.meta)

    def to(self, device) -> "DeviceEncoded":
        import torch
        t = lambda a: torch.from_numpy(a).to(device)
        return DeviceEncoded(self.meta, t(self.stream), t(self.nibbles), t(self.gaps),
                             t(self.blk_off.view(np.int64)), self.shape)


def encode(x, lengths=None, chunk_bytes: int = DEFAULT_CHUNK_BYTES,
           threads_per_block: int = DEFAULT_THREADS_PER_BLOCK, max_len: int = 16) -> Encoded:
    """Histogram -> Huffman code (unless `lengths` given) -> encode, all in libecf8."""
    shape = tuple(x.shape) if hasattr(x, "shape") else ()
    a = _u8(x)
    cb = _codebook(build_codebook(a, max_len) if lengths is None else lengths)
    p = Params(chunk_bytes, threads_per_block)
    m = Meta()
    _check(lib().ecf8_encode_sizes(_ptr(a), a.size, ctypes.byref(cb), ctypes.byref(p), ctypes.byref(m)),
           "ecf8_encode_sizes")
    stream = np.empty(m.stream_bytes, dtype=np.uint8)
    nib = np.empty(m.nibble_bytes, dtype=np.uint8)
    gaps = np.empty(m.gap_bytes, dtype=np.uint8)
    blk = np.empty(m.n_blocks + 1, dtype=np.uint64)
    m2 = Meta()
    _check(lib().ecf8_encode(_ptr(a), a.size, ctypes.byref(cb), ctypes.byref(p), _ptr(stream), stream.size,
                             _ptr(nib), nib.size, _ptr(gaps), gaps.size, _ptr(blk), blk.size,
                             ctypes.byref(m2)), "ecf8_encode")
    return Encoded(m2, stream, nib, gaps, blk, shape)


def alpha_hat(w, gamma: float) -> float:
    """Tail-index estimate log n / log(max|w| / gamma) of float32 weights (ecf8_alpha_hat)."""
    if hasattr(w, "detach"):
        w = w.detach().float().cpu().numpy()
    a = np.ascontiguousarray(np.asarray(w, dtype=np.float32).ravel())
    out = ctypes.c_double(0.0)
    _check(lib().ecf8_alpha_hat(a.ctypes.data_as(ctypes.c_void_p), a.size, float(gamma), ctypes.byref(out)),
           "ecf8_alpha_hat")
    return float(out.value)


def exponent_entropy_bound(alpha: float) -> float:
    """alpha / (1 - 2^-alpha), the pages' bound on the exponent entropy in bits."""
    return float(lib().ecf8_exponent_entropy_bound(float(alpha)))


def meta_from_freq(freq, n: int, lengths, chunk_bytes: int = DEFAULT_CHUNK_BYTES,
                   threads_per_block: int = DEFAULT_THREADS_PER_BLOCK) -> Meta:
    """Metadata for n elements with exponent histogram freq under code lengths (ecf8_meta_from_freq)."""
    f = (ctypes.c_uint64 * NSYM)(*[int(v) for v in freq])
    cb = _codebook(lengths)
    p = Params(chunk_bytes, threads_per_block)
    m = Meta()
    _check(lib().ecf8_meta_from_freq(f, int(n), ctypes.byref(cb), ctypes.byref(p), ctypes.byref(m)),
           "ecf8_meta_from_freq")
    return m


def encode_workspace_bytes(n: int) -> int:
    return int(lib().ecf8_encode_workspace_bytes(int(n)))


def validate_meta(m: Meta) -> int:
    return int(lib().ecf8_validate_meta(ctypes.byref(m)))


def workspace_bytes(count: int) -> int:
    return int(lib().ecf8_workspace_bytes(count))


# ------------------------------------------------------------------ device side

@dataclasses.dataclass
class DeviceEncoded:
    """Device-resident encoded tensor: four torch uint8/int64 tensors + metadata."""
    meta: Meta
    stream: "object"
    nibbles: "object"
    gaps: "object"
    blk_off: "object"
    shape: tuple = ()

    @property
    def n(self) -> int:
        return int(self.meta.n)

    def compressed_bytes(self) -> int:
        return compressed_bytes(self.meta)

    def c_stream(self) -> Stream:
        return Stream(self.stream.data_ptr(), self.nibbles.data_ptr(), self.gaps.data_ptr(),
                      self.blk_off.data_ptr())


def _stream_handle(stream) -> ctypes.c_void_p:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _torch_stream(stream):
    import torch
    return torch.cuda.current_stream() if stream is None else stream


def _workspace(count: int, device, workspace=None, stream=None):
    """A caller's workspace if it is large enough, else a new one.  A new one is
    allocated while `stream` (the launch stream) is current, so that the caching
    allocator does not hand its memory to other work before the launch ends."""
    import torch
    need = workspace_bytes(count)
    if workspace is None or workspace.numel() < need:
        with torch.cuda.stream(_torch_stream(stream)):
            workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=device)
    else:
        _check_buffer(workspace, device, "workspace")
    return workspace


def _check_buffer(t, device, what: str):
    """A device buffer handed to the library: uint8, contiguous, on `device`."""
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch tensor" % what)
    if t.dtype != torch.uint8 or not t.is_contiguous():
        raise ValueError("%s must be a contiguous uint8 tensor (got %s, contiguous=%s)"
                         % (what, t.dtype, t.is_contiguous()))
    if t.device != torch.device(device):
        raise ValueError("%s is on %s, the encoded tensors on %s" % (what, t.device, device))


def _check_out_ranges(out, offsets, sizes, device):
    """out must hold every tensor's range [offset, offset + n) and the ranges must not overlap."""
    _check_buffer(out, device, "out")
    spans = sorted((int(o), int(o) + int(n)) for o, n in zip(offsets, sizes) if int(n) > 0)
    for o, n in zip(offsets, sizes):
        if int(o) < 0:
            raise ValueError("negative output offset %d" % int(o))
    if spans and spans[-1][1] > out.numel():
        raise ValueError("out holds %d bytes; the tensors need %d" % (out.numel(), max(e for _, e in spans)))
    for (a0, a1), (b0, b1) in zip(spans, spans[1:]):
        if b0 < a1:
            raise ValueError("output ranges [%d, %d) and [%d, %d) overlap" % (a0, a1, b0, b1))


def encode_workspace(n: int, device):
    """Device workspace for histogram_device / encode_into of n elements."""
    import torch
    return torch.empty(encode_workspace_bytes(n), dtype=torch.uint8, device=device)


def histogram_device(x, freq=None, workspace=None, stream=None):
    """Exponent histogram of a device uint8 tensor (ecf8_histogram_device); returns 16 int64 counts on the
    device.  With `workspace` (encode_workspace) the per-tile counts an encode_into of x needs are kept there."""
    import torch
    x = x.contiguous().view(-1)
    if freq is None:
        freq = torch.empty(NSYM, dtype=torch.int64, device=x.device)
    ws_ptr, ws_n = (ctypes.c_void_p(workspace.data_ptr()), workspace.numel()) if workspace is not None \
        else (ctypes.c_void_p(0), 0)
    _check(lib().ecf8_histogram_device(ctypes.c_void_p(x.data_ptr()), x.numel(), ctypes.c_void_p(freq.data_ptr()),
                                       ws_ptr, ws_n, _stream_handle(stream)), "ecf8_histogram_device")
    return freq


def alloc_device(meta: Meta, device, shape=()) -> DeviceEncoded:
    """Uninitialised device buffers of meta's sizes (stream, nibbles, gaps, blk_off)."""
    import torch
    e = lambda k, dt=torch.uint8: torch.empty(max(int(k), 1), dtype=dt, device=device)
    return DeviceEncoded(meta, e(meta.stream_bytes), e(meta.nibble_bytes), e(meta.gap_bytes),
                         e(meta.n_blocks + 1, torch.int64), shape)


def encode_into(x, enc: DeviceEncoded, workspace, stream=None) -> DeviceEncoded:
    """Encode device bytes x into enc's buffers under enc.meta (ecf8_encode_device); `workspace` is the one a
    histogram_device of the same x filled."""
    x = x.contiguous().view(-1)
    m = enc.meta
    _check(lib().ecf8_encode_device(ctypes.c_void_p(x.data_ptr()), ctypes.byref(m),
                                    ctypes.c_void_p(enc.stream.data_ptr()), ctypes.c_void_p(enc.nibbles.data_ptr()),
                                    ctypes.c_void_p(enc.gaps.data_ptr()), ctypes.c_void_p(enc.blk_off.data_ptr()),
                                    ctypes.c_void_p(workspace.data_ptr()), workspace.numel(),
                                    _stream_handle(stream)), "ecf8_encode_device")
    return enc


def encode_batched_into(xs, encs, workspaces, stream=None):
    """Encode several device byte tensors at once (ecf8_encode_batched_device): xs[i] into encs[i]'s buffers
    under encs[i].meta, workspaces[i] being the one a histogram_device of xs[i] filled."""
    if not (len(xs) == len(encs) == len(workspaces)):
        raise ValueError("xs, encs and workspaces differ in length")
    jobs = (EncodeJob * max(len(xs), 1))()
    keep = []
    for k, (x, enc, ws) in enumerate(zip(xs, encs, workspaces)):
        x = x.contiguous().view(-1)
        keep.append(x)
        jobs[k] = EncodeJob(x.data_ptr(), enc.meta, enc.stream.data_ptr(), enc.nibbles.data_ptr(),
                            enc.gaps.data_ptr(), enc.blk_off.data_ptr(), ws.data_ptr(), ws.numel())
    _check(lib().ecf8_encode_batched_device(jobs, len(xs), _stream_handle(stream)), "ecf8_encode_batched_device")
    return encs


def encode_device(x, lengths=None, chunk_bytes: int = DEFAULT_CHUNK_BYTES,
                  threads_per_block: int = DEFAULT_THREADS_PER_BLOCK, max_len: int = 16,
                  stream=None, workspace=None) -> DeviceEncoded:
    """GPU encode of a device uint8 (FP8 E4M3 bytes) tensor.

    Histogram pass on the GPU; the 16 counts come to the host (one
    synchronisation) for the code lengths and buffer sizes; the encode pass
    runs on the GPU.  The buffers equal those of encode() on the same bytes.
    """
    import torch
    shape = tuple(x.shape)
    x = x.contiguous().view(-1)
    if x.dtype != torch.uint8:
        x = x.view(torch.uint8)
    n = x.numel()
    if workspace is None or workspace.numel() < encode_workspace_bytes(n):
        workspace = encode_workspace(n, x.device)
    freq = histogram_device(x, workspace=workspace, stream=stream)
    if stream is not None:
        stream.synchronize()
    freq = freq.cpu().numpy().astype(np.uint64)
    if lengths is None:
        lengths = codebook_from_freq(freq, max_len) if n else [0] * NSYM
    m = meta_from_freq(freq, n, lengths, chunk_bytes, threads_per_block)
    enc = alloc_device(m, x.device, shape)
    return encode_into(x, enc, workspace, stream=stream)


def decode(enc: DeviceEncoded, out=None, workspace=None, stream=None):
    """Single-tensor GPU decode (ecf8_decode).  Returns the uint8 output tensor.

    out, if given, must be a contiguous uint8 tensor of exactly n bytes on the
    encoded tensor's device (its size is passed as n and checked against the
    metadata).  Buffers allocated here are allocated on the launch stream."""
    import torch
    dev = enc.stream.device
    if out is None:
        with torch.cuda.stream(_torch_stream(stream)):
            out = torch.empty(max(enc.n, 1), dtype=torch.uint8, device=dev)[: enc.n]
    else:
        _check_buffer(out, dev, "out")
    ws = _workspace(1, dev, workspace, stream)
    s = enc.c_stream()
    m = enc.meta
    _check(lib().ecf8_decode(ctypes.byref(s), ctypes.byref(m), ctypes.c_void_p(out.data_ptr()), out.numel(),
                             ctypes.c_void_p(ws.data_ptr()), ws.numel(), _stream_handle(stream)),
           "ecf8_decode")
    return out


class DecodePlan:
    """A prepared batched decode (ecf8_decode_prepare / ecf8_decode_run).

    All tensors decode in one persistent dispatch into `out` (a reused uint8
    buffer); tensor i lands at out[offsets[i] : offsets[i] + n_i].
    """

    def __init__(self, encs: Sequence[DeviceEncoded], out=None, offsets: Optional[List[int]] = None,
                 workspace=None, stream=None, workgroups: Optional[int] = None,
                 claim_blocks: Optional[int] = None):
        """workgroups: upper bound on the persistent decode's workgroups (default:
        every compute unit at full occupancy); a smaller grid leaves compute units
        to kernels running concurrently on other streams.  claim_blocks: the block
        order (ecf8_plan.claim_blocks: 0 static, 2..1024 blocks per claim; default:
        the library's choice)."""
        import torch
        self.encs = list(encs)
        dev = self.encs[0].stream.device if self.encs else torch.device("cuda")
        if offsets is None:
            offsets, off = [], 0
            for e in self.encs:
                offsets.append(off)
                off += (e.n + 255) // 256 * 256
            total = off
        else:
            total = max([o + e.n for o, e in zip(offsets, self.encs)] + [0])
        self.offsets = list(offsets)
        if len(self.offsets) != len(self.encs):
            raise ValueError("%d offsets for %d tensors" % (len(self.offsets), len(self.encs)))
        if out is None:
            with torch.cuda.stream(_torch_stream(stream)):
                out = torch.empty(max(total, 1), dtype=torch.uint8, device=dev)
        _check_out_ranges(out, self.offsets, [e.n for e in self.encs], dev)
        self.out = out
        self.workspace = _workspace(len(self.encs), dev, workspace, stream)
        arr = (TensorDesc * max(1, len(self.encs)))()
        for i, (e, o) in enumerate(zip(self.encs, self.offsets)):
            arr[i].s = e.c_stream()
            arr[i].meta = e.meta
            arr[i].out_offset = o
        self._descs = arr
        self.plan = Plan()
        _check(lib().ecf8_decode_prepare(arr, len(self.encs), ctypes.c_void_p(self.out.data_ptr()),
                                         ctypes.c_void_p(self.workspace.data_ptr()), self.workspace.numel(),
                                         _stream_handle(stream), ctypes.byref(self.plan)),
               "ecf8_decode_prepare")
        if workgroups is not None:
            self.plan.grid = max(1, min(int(self.plan.grid), int(workgroups)))
        if claim_blocks is not None:
            self.plan.claim_blocks = int(claim_blocks)
        # the descriptor upload is ordered on the prepare stream; a launch on
        # another stream first waits for it (once per stream)
        self._prep_stream = _torch_stream(stream)
        self._ready = torch.cuda.Event()
        self._ready.record(self._prep_stream)
        self._synced = {self._prep_stream.cuda_stream}

    def _launch_stream(self, stream):
        s = _torch_stream(stream)
        if s.cuda_stream not in self._synced:
            s.wait_event(self._ready)
            self._synced.add(s.cuda_stream)
        return ctypes.c_void_p(s.cuda_stream)

    def run(self, stream=None, events=None):
        """The decode dispatch (each workgroup copies its tensor's decode table, built when the
        plan was prepared, into LDS).  events:
        optional (start, stop) torch.cuda.Event pair (timing enabled) attached to the dispatch
        itself (ecf8_decode_run_timed), so that start.elapsed_time(stop) is the kernel's own
        duration."""
        st = self._launch_stream(stream)
        if events is None:
            _check(lib().ecf8_decode_run(ctypes.byref(self.plan), st), "ecf8_decode_run")
            return self.out
        handles = []
        for ev in events:
            if not ev.cuda_event:                  # torch creates its event on the first record
                ev.record()
            handles.append(ctypes.c_void_p(ev.cuda_event))
        _check(lib().ecf8_decode_run_timed(ctypes.byref(self.plan), st, handles[0], handles[1]),
               "ecf8_decode_run_timed")
        return self.out

    def status(self, stream=None) -> int:
        """Synchronize and return the number of blocks whose counts disagreed with blk_off in
        the runs since the plan was prepared or since the previous status() (which restarts
        the count)."""
        bad = ctypes.c_uint64(0)
        rc = lib().ecf8_decode_status(ctypes.c_void_p(self.workspace.data_ptr()), _stream_handle(stream),
                                      ctypes.byref(bad))
        if rc not in (0, -5):
            _check(rc, "ecf8_decode_status")
        return int(bad.value)

    def view(self, i: int):
        return self.out[self.offsets[i]: self.offsets[i] + self.encs[i].n]


def hbm_stream(src, read_bytes: int, dst, write_bytes: int, stream=None):
    """A plain stream with a decode's byte mix (ecf8_hbm_stream): write_bytes to dst, reading read_bytes of src
    once; output 16-byte unit i takes input unit (i * m) >> 32, m = floor(2^32 * read_units / write_units)."""
    if src.numel() * src.element_size() < read_bytes or dst.numel() * dst.element_size() < write_bytes:
        raise ValueError("buffers smaller than the sizes")
    _check(lib().ecf8_hbm_stream(ctypes.c_void_p(src.data_ptr()), int(read_bytes), ctypes.c_void_p(dst.data_ptr()),
                                 int(write_bytes), _stream_handle(stream)), "ecf8_hbm_stream")
    return dst


def hbm_copy(src, dst, stream=None):
    """Plain streaming device copy src -> dst (ecf8_hbm_copy), the HBM ceiling the decode is compared with."""
    n = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() < n:
        raise ValueError("dst holds fewer bytes than src")
    _check(lib().ecf8_hbm_copy(ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(dst.data_ptr()), n,
                               _stream_handle(stream)), "ecf8_hbm_copy")
    return dst


def decode_batched_noalloc(encs: Sequence[DeviceEncoded], out, offsets, bad_blocks=None, stream=None):
    """ecf8_decode_batched_noalloc: decode up to 16 tensors into out[offsets[i]:] with no workspace and no
    allocation (the library's fixed device scratch).  bad_blocks: None or a device int64 tensor of one
    element that receives the block-check count."""
    encs = list(encs)
    dev = encs[0].stream.device if encs else out.device
    if len(offsets) != len(encs):
        raise ValueError("%d offsets for %d tensors" % (len(offsets), len(encs)))
    _check_out_ranges(out, offsets, [e.n for e in encs], dev)
    arr = (TensorDesc * max(1, len(encs)))()
    for i, (e, o) in enumerate(zip(encs, offsets)):
        arr[i].s = e.c_stream()
        arr[i].meta = e.meta
        arr[i].out_offset = o
    bb = ctypes.c_void_p(bad_blocks.data_ptr()) if bad_blocks is not None else ctypes.c_void_p(0)
    _check(lib().ecf8_decode_batched_noalloc(arr, len(encs), ctypes.c_void_p(out.data_ptr()), bb,
                                             _stream_handle(stream)), "ecf8_decode_batched_noalloc")
    return out


def decode_batched(encs: Sequence[DeviceEncoded], out=None, offsets=None, workspace=None, stream=None):
    """prepare + run in one call (ecf8_decode_batched semantics)."""
    p = DecodePlan(encs, out, offsets, workspace, stream)
    p.run(stream)
    return p


# ------------------------------------------------------------------ format variants (include/ecf8v.h)

def _fmt_v(fmt) -> int:
    return FORMAT_V[fmt] if isinstance(fmt, str) else int(fmt)


def _elems_v(fmt, x) -> np.ndarray:
    """Host elements of the format: uint16 BF16 bit patterns, or E5M2 bytes."""
    if hasattr(x, "detach"):
        import torch
        t = x.detach().cpu().contiguous().view(-1)
        if t.dtype == torch.bfloat16:
            t = t.view(torch.int16)
        elif t.dtype == torch.float8_e5m2:
            t = t.view(torch.uint8)
        x = t.numpy()
    a = np.ascontiguousarray(np.asarray(x).reshape(-1))
    if _fmt_v(fmt) == 1:
        return np.ascontiguousarray(a.view(np.uint16) if a.dtype.itemsize == 2 else a.astype(np.uint16))
    return np.ascontiguousarray(a.view(np.uint8) if a.dtype.itemsize == 1 else a.astype(np.uint8))


def v_nsym(fmt) -> int:
    r = int(lib().ecf8v_nsym(_fmt_v(fmt)))
    _check(min(r, 0), "ecf8v_nsym")
    return r


def v_histogram(fmt, x) -> np.ndarray:
    a = _elems_v(fmt, x)
    f = np.zeros(v_nsym(fmt), dtype=np.uint64)
    _check(lib().ecf8v_histogram(_fmt_v(fmt), _ptr(a), a.size, f.ctypes.data_as(ctypes.POINTER(ctypes.c_uint64))),
           "ecf8v_histogram")
    return f


def v_code_lengths(freq, max_len: int = 16) -> np.ndarray:
    """Optimal prefix-code lengths no longer than max_len (ecf8v_code_lengths, package-merge)."""
    f = np.ascontiguousarray(np.asarray(freq, dtype=np.uint64))
    L = np.zeros(f.size, dtype=np.uint8)
    _check(lib().ecf8v_code_lengths(f.ctypes.data_as(ctypes.POINTER(ctypes.c_uint64)), f.size, int(max_len),
                                    L.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8))), "ecf8v_code_lengths")
    return L.astype(np.int64)


def v_canonical_codes(lengths) -> np.ndarray:
    L = np.ascontiguousarray(np.asarray(lengths, dtype=np.uint8))
    c = np.zeros(L.size, dtype=np.uint32)
    _check(lib().ecf8v_canonical_codes(L.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8)), L.size,
                                       c.ctypes.data_as(ctypes.POINTER(ctypes.c_uint32))), "ecf8v_canonical_codes")
    return c.astype(np.int64)


def meta_v_dict(m: MetaV) -> dict:
    d = {k: getattr(m, k) for k, _ in MetaV._fields_ if k != "len"}
    d["lengths"] = list(m.len)
    return d


def compressed_bytes_v(m: MetaV) -> int:
    """Bytes one decode reads: stream payload, raw plane, gaps, block offsets."""
    raw = m.n if m.format == 1 else (m.n + 1) // 2
    return int((m.total_bits + 7) // 8 + raw + (m.n_chunks + 1) // 2 + 8 * (m.n_blocks + 1))


@dataclasses.dataclass
class EncodedV:
    """Host-side encoded tensor of a format variant."""
    meta: MetaV
    stream: np.ndarray
    raw: np.ndarray
    gaps: np.ndarray
    blk_off: np.ndarray
    shape: tuple = ()

    @property
    def n(self) -> int:
        return int(self.meta.n)

    @property
    def lengths(self) -> np.ndarray:
        return np.array(list(self.meta.len)[: v_nsym(self.meta.format)], dtype=np.int64)

    def compressed_bytes(self) -> int:
        return compressed_bytes_v(self.meta)

    def to(self, device) -> "DeviceEncodedV":
        import torch
        t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(device)
        return DeviceEncodedV(self.meta, t(self.stream), t(self.raw if self.raw.size else np.zeros(1, np.uint8)),
                              t(self.gaps if self.gaps.size else np.zeros(1, np.uint8)),
                              t(self.blk_off.view(np.int64)), self.shape)


def v_encode(fmt, x, lengths=None, chunk_bytes: int = DEFAULT_CHUNK_BYTES,
             threads_per_block: int = DEFAULT_THREADS_PER_BLOCK, max_len: int = 16) -> EncodedV:
    """Histogram -> package-merge lengths (unless given) -> encode, all in libecf8."""
    f = _fmt_v(fmt)
    shape = tuple(x.shape) if hasattr(x, "shape") else ()
    a = _elems_v(f, x)
    ns = v_nsym(f)
    if lengths is None:
        lengths = v_code_lengths(v_histogram(f, a), max_len)
    L = np.zeros(MAXSYM_V, dtype=np.uint8)
    L[:ns] = np.asarray(lengths, dtype=np.uint8)[:ns]
    Lp = L.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8))
    p = Params(chunk_bytes, threads_per_block)
    m = MetaV()
    _check(lib().ecf8v_encode_sizes(f, _ptr(a), a.size, Lp, ctypes.byref(p), ctypes.byref(m)), "ecf8v_encode_sizes")
    stream = np.empty(m.stream_bytes, dtype=np.uint8)
    raw = np.empty(m.raw_bytes, dtype=np.uint8)
    gaps = np.empty(m.gap_bytes, dtype=np.uint8)
    blk = np.empty(m.n_blocks + 1, dtype=np.uint64)
    m2 = MetaV()
    _check(lib().ecf8v_encode(f, _ptr(a), a.size, Lp, ctypes.byref(p), _ptr(stream), stream.size, _ptr(raw),
                              raw.size, _ptr(gaps), gaps.size, _ptr(blk), blk.size, ctypes.byref(m2)), "ecf8v_encode")
    return EncodedV(m2, stream, raw, gaps, blk, shape)


def v_validate_meta(m: MetaV) -> int:
    return int(lib().ecf8v_validate_meta(ctypes.byref(m)))


@dataclasses.dataclass
class DeviceEncodedV:
    """Device-resident encoded tensor of a format variant."""
    meta: MetaV
    stream: "object"
    raw: "object"
    gaps: "object"
    blk_off: "object"
    shape: tuple = ()

    @property
    def n(self) -> int:
        return int(self.meta.n)

    @property
    def elem_bytes(self) -> int:
        return 2 if self.meta.format == 1 else 1

    def compressed_bytes(self) -> int:
        return compressed_bytes_v(self.meta)


class DecodePlanV:
    """A prepared batched decode of variant tensors (ecf8v_decode_prepare / ecf8v_decode_run).

    All tensors decode in one persistent dispatch into `out` (uint8 bytes);
    tensor i lands at byte offset offsets[i] (n_i elements of the format).
    """

    def __init__(self, encs, out=None, offsets=None, workspace=None, stream=None, workgroups=None):
        import torch
        self.encs = list(encs)
        dev = self.encs[0].stream.device if self.encs else torch.device("cuda")
        if offsets is None:
            offsets, off = [], 0
            for e in self.encs:
                offsets.append(off)
                off += (e.n * e.elem_bytes + 255) // 256 * 256
            total = off
        else:
            total = max([o + e.n * e.elem_bytes for o, e in zip(offsets, self.encs)] + [0])
        self.offsets = list(offsets)
        if len(self.offsets) != len(self.encs):
            raise ValueError("%d offsets for %d tensors" % (len(self.offsets), len(self.encs)))
        if out is None:
            with torch.cuda.stream(_torch_stream(stream)):
                out = torch.empty(max(total, 1), dtype=torch.uint8, device=dev)
        _check_out_ranges(out, self.offsets, [e.n * e.elem_bytes for e in self.encs], dev)
        self.out = out
        need = int(lib().ecf8v_workspace_bytes(len(self.encs)))
        if workspace is None or workspace.numel() < need:
            with torch.cuda.stream(_torch_stream(stream)):
                workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
        else:
            _check_buffer(workspace, dev, "workspace")
        self.workspace = workspace
        arr = (TensorDescV * max(1, len(self.encs)))()
        for i, (e, o) in enumerate(zip(self.encs, self.offsets)):
            arr[i].stream = e.stream.data_ptr()
            arr[i].raw = e.raw.data_ptr()
            arr[i].gaps = e.gaps.data_ptr()
            arr[i].blk_off = e.blk_off.data_ptr()
            arr[i].meta = e.meta
            arr[i].out_offset = o
        self._descs = arr
        self.plan = PlanV()
        _check(lib().ecf8v_decode_prepare(arr, len(self.encs), ctypes.c_void_p(self.out.data_ptr()),
                                          ctypes.c_void_p(self.workspace.data_ptr()), self.workspace.numel(),
                                          _stream_handle(stream), ctypes.byref(self.plan)), "ecf8v_decode_prepare")
        if workgroups is not None:
            self.plan.grid = max(1, min(int(self.plan.grid), int(workgroups)))
        self._prep_stream = _torch_stream(stream)
        self._ready = torch.cuda.Event()
        self._ready.record(self._prep_stream)
        self._synced = {self._prep_stream.cuda_stream}

    _launch_stream = DecodePlan._launch_stream

    def run(self, stream=None, events=None):
        """The decode dispatch.  events: optional (start, stop) torch.cuda.Event pair (timing
        enabled) attached to the dispatch itself (ecf8v_decode_run_timed)."""
        st = self._launch_stream(stream)
        if events is None:
            _check(lib().ecf8v_decode_run(ctypes.byref(self.plan), st), "ecf8v_decode_run")
            return self.out
        handles = []
        for ev in events:
            if not ev.cuda_event:                  # torch creates its event on the first record
                ev.record()
            handles.append(ctypes.c_void_p(ev.cuda_event))
        _check(lib().ecf8v_decode_run_timed(ctypes.byref(self.plan), st, handles[0], handles[1]),
               "ecf8v_decode_run_timed")
        return self.out

    def status(self, stream=None) -> int:
        """Synchronize and return the bad blocks of the runs since prepare or the previous
        status() (which restarts the count)."""
        bad = ctypes.c_uint64(0)
        rc = lib().ecf8v_decode_status(ctypes.c_void_p(self.workspace.data_ptr()), _stream_handle(stream),
                                       ctypes.byref(bad))
        if rc not in (0, -5):
            _check(rc, "ecf8v_decode_status")
        return int(bad.value)

    def view(self, i: int):
        """Tensor i's decoded elements (uint16 bit patterns for BF16, bytes for E5M2)."""
        import torch
        e = self.encs[i]
        b = self.out[self.offsets[i]: self.offsets[i] + e.n * e.elem_bytes]
        return b.view(torch.int16) if e.elem_bytes == 2 else b
