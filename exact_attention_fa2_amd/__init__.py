"""MI355X-native exact attention: FlashAttention-2 forward and backward, and
flash-decoding.

The compute lives in libfa2.so (hand-written HIP for gfx950, C ABI in
include/fa2.h).  This package is its ctypes binding plus the seeded input
generator used by tests and bench.  Importing the package never loads the
library; the first call does, and raises if it is missing.
"""
from .fa2 import (FA2Error, attn_bwd, attn_decode, attn_decode_combine, attn_decode_split, attn_fwd,
                  default_splits, lib, status_string)

__all__ = ["attn_fwd", "attn_bwd", "attn_decode_split", "attn_decode_combine", "attn_decode",
           "default_splits", "status_string", "lib", "FA2Error"]
