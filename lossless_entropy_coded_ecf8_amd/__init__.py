"""lossless_entropy_coded_ecf8_amd -- ECF8 lossless FP8 E4M3 coding with
MI355X (gfx950) GPU decode.

The 4-bit exponent of every FP8 E4M3 weight is Huffman coded per tensor; the
sign and mantissa stay raw as packed nibbles (ECF8 technical blog,
codearts.csdn.net, §3.1.1).  Decode runs in hand-written HIP kernels behind a
C ABI (include/ecf8.h); this package is a thin ctypes binding over it.
"""
from .binding import (DecodePlan, alpha_hat, exponent_entropy_bound, DeviceEncoded, Ecf8Error, Encoded, build_codebook, canonical_codes,
                      codebook_from_freq, decode, decode_batched, encode, encode_batched_into, encode_device,
                      encode_into, encode_workspace_bytes, histogram, histogram_device, lib, meta_from_freq, validate_meta,
                      workspace_bytes)

from .pipeline import DecodePipeline, ECF8Linear, fp8_e4m3_bytes, linear_fp8

__all__ = ["alpha_hat", "exponent_entropy_bound", "DecodePipeline", "ECF8Linear", "fp8_e4m3_bytes", "linear_fp8", "DecodePlan", "DeviceEncoded", "Ecf8Error", "Encoded", "build_codebook", "canonical_codes",
           "codebook_from_freq", "decode", "decode_batched", "encode", "encode_batched_into", "encode_device",
           "encode_into",
           "encode_workspace_bytes", "histogram", "histogram_device", "lib", "meta_from_freq", "validate_meta",
           "workspace_bytes"]
