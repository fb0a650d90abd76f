"""The GPU library's FP8 plane order (include/kvq.h, FP8 cache: 16-byte
pieces, channel c of token j of a group at byte
((2 (c mod 2) + j div 16) (D/2) + c div 2) 16 + j mod 16 of the group's
block) permuted to the oracle's logical [group][channel][token] order.  The
oracle never sees the piece order: the tests bring GPU planes to its order
before comparing."""
import numpy as np


def piece_offset(D, c, j):
    """Byte of channel c, token j (< 32) inside a group block of the GPU planes."""
    return ((2 * (c % 2) + j // 16) * (D // 2) + c // 2) * 16 + j % 16


def to_logical(pieces):
    """uint8[nb][Hkv][Gcap][2][2][D/2][16] (channel parity, token half,
    channel pair, token mod 16) -> uint8[nb][Hkv][Gcap][D][32]."""
    nb, hkv, gcap, _, _, np2, _ = pieces.shape
    x = pieces.transpose(0, 1, 2, 5, 3, 4, 6)        # nb hkv g pair parity half byte
    return np.ascontiguousarray(x.reshape(nb, hkv, gcap, 2 * np2, 32))
