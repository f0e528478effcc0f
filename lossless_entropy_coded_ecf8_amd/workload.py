"""Encode a set of FP8 tensors (one codebook each) and make them device resident.

ECF8 blog (codearts.csdn.net) §5.1: statistics and codebooks are kept per
layer (per expert for MoE), built once after training and frozen; §3.3: on
datacenter GPUs the compressed model stays resident and whole blocks are
decoded in batches.  These helpers do the offline part (host encode through
libecf8) and the upload; decoding is `binding.DecodePlan`.
"""
from __future__ import annotations

from typing import Iterable, List, Tuple

from . import binding


def encode_tensors(named: Iterable[Tuple[str, "object"]], chunk_bytes: int = binding.DEFAULT_CHUNK_BYTES,
                   threads_per_block: int = binding.DEFAULT_THREADS_PER_BLOCK):
    """[(name, uint8 tensor or ndarray)] -> [(name, binding.Encoded)] (host encode, per-tensor codebook)."""
    out = []
    for name, x in named:
        if hasattr(x, "is_cuda") and x.is_cuda:
            x = x.cpu()
        out.append((name, binding.encode(x, chunk_bytes=chunk_bytes, threads_per_block=threads_per_block)))
    return out


def upload(encoded: List[Tuple[str, binding.Encoded]], device) -> List[Tuple[str, binding.DeviceEncoded]]:
    return [(nm, e.to(device)) for nm, e in encoded]


def batch_bytes(encs) -> dict:
    """Algorithmic bytes of one decode of `encs`: what must be read and written."""
    read = sum(e.compressed_bytes() for e in encs)
    written = sum(e.n for e in encs)
    return {"read": read, "written": written, "total": read + written}
