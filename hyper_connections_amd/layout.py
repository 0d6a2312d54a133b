"""Host-side layout helpers: pack logical INT4 codes into the library's byte format.

Weight preparation, done once when weights are loaded; never on the per-token path.
The format (declared in include/decodehp.h): uint8 [rows][cols/2], row-major, byte j of a
row holding k = 2j in bits 0..3 and k = 2j+1 in bits 4..7; bf16 scales and biases
[rows][cols/64] stored as their 16-bit patterns.
"""
from __future__ import annotations

import numpy as np


def pack_int4_codes(q) -> np.ndarray:
    """uint8 codes [rows, cols] in 0..15 -> packed uint8 [rows, cols/2]."""
    q = np.asarray(q)
    if q.ndim != 2 or q.shape[1] % 2:
        raise ValueError("codes must be [rows, cols] with even cols")
    if q.dtype != np.uint8:
        q = q.astype(np.uint8)
    if q.size and q.max() > 15:
        raise ValueError("codes must lie in 0..15")
    return np.ascontiguousarray(q[:, 0::2] | (q[:, 1::2] << 4))


def bf16_bits_to_tensor(bits):
    """uint16 bf16 bit patterns -> a torch int16 tensor with the same bits (CPU)."""
    import torch
    b = np.ascontiguousarray(np.asarray(bits, dtype=np.uint16))
    return torch.from_numpy(b.view(np.int16).copy())
