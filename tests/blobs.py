"""Hand-built Q4_K blobs for exactness tests (byte layout of a 144-byte block: fp16 d, fp16 dmin,
12 bytes of packed 6-bit sub-block scales and mins, 128 bytes of nibbles)."""
import numpy as np

import synth


def unit_scales(blob: np.ndarray) -> np.ndarray:
    """Every 6-bit sub-block scale 1 and every min 0 (in place; returns the blob)."""
    blocks = blob.reshape(-1, 144)
    blocks[:, 4:8] = 1    # scales of sub-blocks 0..3 (high bits 0)
    blocks[:, 8:12] = 0   # mins of sub-blocks 0..3
    blocks[:, 12:16] = 1  # sub-blocks 4..7: low nibble scale 1, high nibble min 0
    return blob


def lattice(g, n: int, k: int) -> np.ndarray:
    """d = 1, dmin = 0, unit scales: every weight is its 4-bit quant, 0..15."""
    return unit_scales(synth.blob("q4_k", g, n, k, d_value=1.0, dmin_value=0.0))


def identity(n: int) -> np.ndarray:
    """An n x n Q4_K matrix equal to the identity (n a multiple of 256)."""
    nb = n // 256
    b = np.zeros((n, nb, 144), np.uint8)
    b[:, :, 0:2] = np.frombuffer(np.float16(1.0).tobytes(), np.uint8)
    unit_scales(b)
    for i in range(n):
        blk, r = divmod(i, 256)
        c, l = divmod(r, 64)  # group c: low nibbles are weights 64c..64c+31, high 64c+32..
        b[i, blk, 16 + 32 * c + (l % 32)] = 1 if l < 32 else 0x10
    return b.reshape(-1)
