"""LSB-first bit packing of per-vector code and sign fields.

"How 0xsero/turboquant works", "Value Compression": value payloads are stored
bit-packed, with several low-bit codes sharing a byte (a byte holds 4 codes at
2 bits, 2 at 4 bits).  "5x Faster LLM Inference?
...", "Example 4: Kernel-Level Operations": the last compression step packs the
bits.  The pages fix no 3-bit format; the reading used everywhere here is a
little-endian bitstream per field: element j of a b-bit field occupies stream
bits [b*j, b*j + b), stream bit i is bit (i mod 8) of byte floor(i / 8).
For b = 2 and b = 4 this is exactly "four / two values per byte", lowest
element in the lowest bits.
"""

import numpy as np


def pack(values, b):
    """Pack the last axis of `values` (ints in [0, 2**b)) into uint8 bytes."""
    v = np.asarray(values, dtype=np.int64)
    if v.size and (v.min() < 0 or v.max() >= (1 << b)):
        raise ValueError("value out of range for %d bits" % b)
    n = v.shape[-1]
    if (n * b) % 8:
        raise ValueError("field length must be a whole number of bytes")
    bitplanes = (v[..., :, None] >> np.arange(b)) & 1           # [..., n, b]
    stream = bitplanes.reshape(v.shape[:-1] + (n * b,)).astype(np.uint8)
    return np.packbits(stream, axis=-1, bitorder="little")


def unpack(data, b, n):
    """Inverse of pack: uint8 bytes -> n ints of b bits (last axis)."""
    d = np.asarray(data, dtype=np.uint8)
    stream = np.unpackbits(d, axis=-1, bitorder="little")[..., : n * b]
    planes = stream.reshape(d.shape[:-1] + (n, b)).astype(np.int64)
    return (planes << np.arange(b)).sum(axis=-1)
