"""Where the product library keeps packed weight bytes, stated from its header (bitnet.h,
bitnet_packed_bytes) and applied to canonical row-major packed bytes.

The oracle packs row-major: byte b of 320-weight block B of row n is byte
n * 64 * nblk + 64 B + b (nblk = ceil(K / 320)).  The product keeps the same bytes in 1 KB
tiles: rows in groups of 16 (the last group padded with rows of zero weights, whose bytes are
the code of digits 1,1,1,1,1 = 121); group G and block B form the tile at (G * nblk + B) * 1024,
and inside it byte b of row n sits at ((b / 16) * 16 + n % 16) * 16 + b % 16.  So the device
buffer is a permutation of the canonical bytes plus pad rows; nothing else changes.

Test helper only: it uses numpy reshapes, none of the product's or the oracle's code.
"""
import numpy as np

ZERO_BYTE = 121  # five digits 1 (t = 0): 81 + 27 + 9 + 3 + 1


def nblocks(K: int) -> int:
    return (K + 319) // 320


def to_device(canonical, N: int, K: int) -> np.ndarray:
    """Canonical N x (64 nblk) packed bytes -> the product's tiled buffer (16 ceil(N/16) rows)."""
    nb = nblocks(K)
    c = np.asarray(canonical, np.uint8).reshape(N, nb * 64)
    rows = (N + 15) // 16 * 16
    pad = np.full((rows, nb * 64), ZERO_BYTE, np.uint8)
    pad[:N] = c
    # (group, row-in-group, block, chunk b/16, byte b%16) -> (group, block, chunk, row, byte)
    t = pad.reshape(rows // 16, 16, nb, 4, 16).transpose(0, 2, 3, 1, 4)
    return np.ascontiguousarray(t).reshape(-1)


def from_device(device, N: int, K: int) -> np.ndarray:
    """Inverse of to_device: the canonical N x (64 nblk) bytes (pad rows dropped)."""
    nb = nblocks(K)
    rows = (N + 15) // 16 * 16
    t = np.asarray(device, np.uint8).reshape(rows // 16, nb, 4, 16, 16).transpose(0, 3, 1, 2, 4)
    return np.ascontiguousarray(t).reshape(rows, nb * 64)[:N].reshape(-1)


def device_groups(device, K: int) -> np.ndarray:
    """The tiled buffer viewed as its 16-row groups (one row of 1024 * nblk bytes each)."""
    return np.asarray(device, np.uint8).reshape(-1, 1024 * nblocks(K))
