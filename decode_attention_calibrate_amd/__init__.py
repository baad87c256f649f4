"""Lossless compressed-KV decode attention for AMD MI355X (gfx950).

The method is GAAC's (page "GAAC: Lossless KV Compression for Bandwidth-Efficient LLM Inference
on Personal Devices"): calibrated per-(head, channel) exponent bases, 3-bit / 4-bit / raw
exponent modes per 16-token (or 8-token) group, sign and mantissa stored raw, fixed-capacity slots behind a
paged block table, and a decode-attention kernel that rebuilds tiles on chip.

Everything runs in hand-written HIP kernels behind the C ABI of include/kvc.h (libkvc.so);
this package only marshals arguments.  Creating a KVCache (or calling load()) raises if
libkvc.so has not been built; there is no CPU fallback.
"""
from ._lib import (BF16, FP8_E4M3, FP8_E5M2, KVCError, LIB_PATH, STATUS_COMP_EXHAUSTED, STATUS_CORRUPT,
                   STATUS_MISSING_BLOCK, STATUS_RAW_EXHAUSTED, load)
from .cache import KVCache, admit_fcfs, read_probe

__all__ = ["KVCache", "admit_fcfs", "read_probe", "KVCError", "load", "LIB_PATH", "BF16", "FP8_E5M2", "FP8_E4M3", "STATUS_COMP_EXHAUSTED",
           "STATUS_RAW_EXHAUSTED", "STATUS_MISSING_BLOCK", "STATUS_CORRUPT"]
