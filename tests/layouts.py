"""Host-side conversions between row-major weight storage and the tiled storage of the
library's MX formats (include/moe.h: 16-row x 128-K tiles).  Test infrastructure; NumPy only.

Scale tiles: a matrix [N, K] (N a multiple of 16) has N/16 x ceil(K/128) tiles of 64 bytes,
tile (n, j) holding row 16 n + r's four E8M0 codes of K-block j at byte 4 r (codes of blocks
past K are 127).  MXFP4 code tiles: 1024 bytes, row r at byte 64 r holding K [128 j, 128 j +
128) two codes a byte (element 2i in the low nibble of byte i), zeros past K.
"""
from __future__ import annotations

import numpy as np


def kb(n: int) -> int:
    return -(-n // 128)


def pad_scale_rows(codes: np.ndarray, K: int) -> np.ndarray:
    """E8M0 codes [..., K/32] -> padded rows [..., 4 ceil(K/128)] (pads 127)."""
    out = np.full(codes.shape[:-1] + (4 * kb(K),), 127, np.uint8)
    out[..., :K // 32] = codes
    return out


def tile_scales(rows: np.ndarray, N: int, K: int) -> np.ndarray:
    """Padded E8M0 rows [E, N, 4 ceil(K/128)] -> scale tiles [E, N/16, ceil(K/128), 16, 4]."""
    E = rows.shape[0]
    return np.ascontiguousarray(rows.reshape(E, N // 16, 16, kb(K), 4).transpose(0, 1, 3, 2, 4))


def untile_scales(tiles: np.ndarray, N: int, K: int) -> np.ndarray:
    """Scale tiles [E, N/16, KB, 16, 4] -> padded E8M0 rows [E, N, 4 KB]."""
    E = tiles.shape[0]
    return tiles.reshape(E, N // 16, kb(K), 16, 4).transpose(0, 1, 3, 2, 4).reshape(E, N, 4 * kb(K))


def tile_fp4(packed: np.ndarray, N: int, K: int) -> np.ndarray:
    """Row-major packed e2m1 codes [E, N, K/2] -> code tiles [E, N/16, KB, 16, 64]."""
    E = packed.shape[0]
    rows = np.zeros((E, N, kb(K) * 64), np.uint8)
    rows[..., :K // 2] = packed
    return np.ascontiguousarray(rows.reshape(E, N // 16, 16, kb(K), 64).transpose(0, 1, 3, 2, 4))


def untile_fp4(tiles: np.ndarray, N: int, K: int):
    """Code tiles [E, N/16, KB, 16, 64] -> (row-major packed codes [E, N, K/2], the bytes past K)."""
    E = tiles.shape[0]
    c = tiles.reshape(E, N // 16, kb(K), 16, 64).transpose(0, 1, 3, 2, 4).reshape(E, N, kb(K) * 64)
    return c[..., :K // 2], c[..., K // 2:]
