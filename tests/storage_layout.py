"""Host-side definitions of the library's storage layouts (include/svgemm.h)
and of the canonical row-major layouts its import/export calls convert from
and to -- test infrastructure, not part of the oracle: the oracle computes
codes, scales and zeros as plain arrays; these functions only place them.

Canonical layouts (the plainest row-major reading; the pages fix none):
  W4 codes [N][K/2] bytes, low nibble = even k; scales and fp16 zeros
  [N][K/group]; 4-bit zeros [N][ceil(K/group/2)] bytes, low nibble = even
  group; W8 codes [N][K]; activation codes [M][K].
"""
import numpy as np

BLOCK = 32


def canonical_w4_codes(q):
    """W4 codes q[N, K] (0..15) as [N][K/2] bytes: code k in the low nibble of
    byte k/2 if k is even, in the high nibble if odd."""
    q = np.asarray(q, dtype=np.uint8)
    return (q[:, 0::2] | (q[:, 1::2] << 4)).astype(np.uint8)


def canonical_z4(z):
    """Zero points z[N, G] (0..15) as [N][ceil(G/2)] bytes, group j in the low
    nibble of byte j/2 if j is even."""
    z = np.asarray(z, dtype=np.uint8)
    N, G = z.shape
    zp = np.zeros((N, G + (G & 1)), np.uint8)
    zp[:, :G] = z
    return (zp[:, 0::2] | (zp[:, 1::2] << 4)).astype(np.uint8)


# ------------------------------------------------------- library storage
# These functions place arrays in the library's layout (include/svgemm.h) so
# that encoded weights can be compared byte for byte.
# W4 scales and zeros are blocked per (16-row tile, 512-k block, row); W8
# scales are a plain [N] array.
TILE_ROWS = 16


def _up(a: int, b: int) -> int:
    return (a + b - 1) // b * b


def w4_tiled_shape(N: int, K: int) -> tuple:
    """(padded rows, padded K) of the W4 storage: rows to 16, K to 128."""
    return _up(N, TILE_ROWS), _up(K, 128)


def pack_w4_codes(q: np.ndarray) -> np.ndarray:
    """W4 codes q[N, K] (0..15) in the library's tiled byte order.

    Rows are padded to a multiple of 16 and K to a multiple of 128 with code 0.
    Tile (i, j) -- rows 16i..16i+15, k 128j..128j+127 -- is 1024 consecutive
    bytes at offset (i * K/128 + j) * 1024.  Inside a tile, the 16-byte piece
    p = 16*b + r (b = 0..3, r = 0..15) belongs to row 16i + r: its first 8
    bytes hold k in [128j + 16b, 128j + 16b + 16), its last 8 bytes k in
    [128j + 64 + 16b, 128j + 64 + 16b + 16).  Each 4-byte word covering k0..k0+7
    holds code k0+t in the low nibble and code k0+t+4 in the high nibble of
    byte t (t = 0..3).  Returns a flat uint8 array."""
    q = np.asarray(q, dtype=np.uint8)
    N, K = q.shape
    Np, Kp = w4_tiled_shape(N, K)
    qp = np.zeros((Np, Kp), np.uint8)
    qp[:N, :K] = q
    # k = 128 j + 64 h + 16 b + 8 w + 4 e + t   (e selects the nibble)
    a = qp.reshape(Np // 16, 16, Kp // 128, 2, 4, 2, 2, 4)      # i r j h b w e t
    byte = a[..., 0, :] | (a[..., 1, :] << 4)                     # i r j h b w t
    return byte.transpose(0, 2, 4, 1, 3, 5, 6).reshape(-1).copy()  # i j b r h w t


META_K = 512   # k extent of one block of group parameters


def group_param_shape(N: int, K: int, group: int) -> tuple:
    """(padded rows, groups per row incl. padding) of the W4 scale/zero storage:
    rows to 16, K to 512."""
    return _up(N, TILE_ROWS), _up(K, META_K) // group


def tile_group_params(a: np.ndarray, K: int, group: int) -> np.ndarray:
    """Per-group parameters a[N, K/group] (W4 scales, or fp16 zeros) in the
    library's blocked order: rows padded to 16 and K to 512 with 0; the
    512/group values of (16-row tile i, 512-k block jb, row r) are contiguous,
    blocks ordered (i, jb, r).  Returns a flat array."""
    a = np.asarray(a)
    N, G = a.shape
    Np, Gp = group_param_shape(N, K, group)
    gpb = META_K // group
    ap = np.zeros((Np, Gp), a.dtype)
    ap[:N, :G] = a
    return ap.reshape(Np // 16, 16, Gp // gpb, gpb).transpose(0, 2, 1, 3).reshape(-1).copy()


def pack_z4(z: np.ndarray, K: int, group: int) -> np.ndarray:
    """Zero points (0..15) as 4-bit values in the blocked order of
    tile_group_params: group 2c of a block in the low nibble of byte c,
    group 2c + 1 in the high nibble."""
    zt = tile_group_params(np.asarray(z, np.uint8), K, group)
    return (zt[0::2] | (zt[1::2] << 4)).astype(np.uint8)


def zeros_as_f16(z: np.ndarray, K: int, group: int) -> np.ndarray:
    """Zero points stored as fp16 (integers 0..15 are exact), blocked order."""
    return tile_group_params(np.asarray(z).astype(np.float16), K, group)


def w8_tiled_shape(N: int, K: int) -> tuple:
    """(padded rows, padded K) of the W8 storage: rows to 16, K to 64."""
    return _up(N, TILE_ROWS), _up(K, 64)


def pack_w8_codes(q: np.ndarray) -> np.ndarray:
    """W8 codes q[N, K] (int8) in the library's tiled byte order: rows padded to
    16 and K to 64 with 0; tile (i, j) -- rows 16i.., k 64j.. -- is 1024 bytes at
    (i * K/64 + j) * 1024; piece p = 16*b + r holds row 16i + r, k in
    [64j + 16b, 64j + 16b + 16) in natural order.  Returns flat int8."""
    q = np.asarray(q, dtype=np.int8)
    N, K = q.shape
    Np, Kp = w8_tiled_shape(N, K)
    qp = np.zeros((Np, Kp), np.int8)
    qp[:N, :K] = q
    a = qp.reshape(Np // 16, 16, Kp // 64, 4, 16)                # i r j b t
    return a.transpose(0, 2, 3, 1, 4).reshape(-1).copy()


def pack_act_codes(qx: np.ndarray) -> np.ndarray:
    """int8 activation codes qx[M, K] in the library's slab byte order (the
    pages give no layout): K is cut into slabs of 32 values (one transform
    block each), slabs in k order, and within a slab the M rows' 32 bytes one
    after another -- byte (m, k) at ((k // 32) * M + m) * 32 + k % 32.  Same
    size as [M][K]; for M = 1 it is the row itself.  Returns flat int8."""
    qx = np.asarray(qx, dtype=np.int8)
    M, K = qx.shape
    if K % BLOCK:
        raise ValueError("K must be a multiple of 32")
    return qx.reshape(M, K // BLOCK, BLOCK).transpose(1, 0, 2).reshape(-1).copy()
