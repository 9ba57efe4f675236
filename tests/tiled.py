"""Test-side reader of libft's expert blob (a restatement of include/ft.h's description of
the layout, independent of the library): 4096-byte header, then gate codes, gate scales,
up codes, up scales, down codes, down scales, each starting on a 4096-byte boundary.  A
matrix [R][K] is stored in tiles of 16 rows x 128 K, row-tile major; lane l of a tile owns
16 code bytes (row l % 16, K from 32 (l / 16)) and one E8M0 byte (MXFP4) or two E4M3 bytes
(NVFP4) of scales."""
import numpy as np


def blob_offsets(fmt, H, I):
    sb = 64 if fmt == "mxfp4" else 128
    sizes = [I * H // 2, (I // 16) * (H // 128) * sb] * 2 + [H * I // 2, (H // 16) * (I // 128) * sb]
    offs, o = [], 4096
    for s in sizes:
        offs.append(o)
        o = (o + s + 4095) // 4096 * 4096
    return offs, o


def unpack_tiled(blob, off_codes, off_scales, R, K, fmt):
    """(codes uint8 [R][K/2] packed low nibble first, scales uint8 [R][K/B])."""
    KC = K // 128
    B = 32 if fmt == "mxfp4" else 16
    sb = 64 if fmt == "mxfp4" else 128
    nt = (R // 16) * KC
    c = np.asarray(blob[off_codes:off_codes + nt * 1024]).reshape(R // 16, KC, 4, 16, 16)
    # [rt][kc][g][n][16 bytes] -> [rt][n][kc][g][16 bytes] -> rows, K/2 bytes
    codes = c.transpose(0, 3, 1, 2, 4).reshape(R, K // 2)
    s = np.asarray(blob[off_scales:off_scales + nt * sb])
    if fmt == "mxfp4":
        s = s.reshape(R // 16, KC, 4, 16).transpose(0, 3, 1, 2).reshape(R, K // B)
    else:
        s = s.reshape(R // 16, KC, 4, 16, 2).transpose(0, 3, 1, 2, 4).reshape(R, K // B)
    return codes.copy(), s.copy()


def matrices(blob, fmt, H, I):
    """[(codes, scales)] of gate, up and down."""
    offs, _ = blob_offsets(fmt, H, I)
    dims = [(I, H), (I, H), (H, I)]
    return [unpack_tiled(blob, offs[2 * m], offs[2 * m + 1], R, K, fmt)
            for m, (R, K) in enumerate(dims)]
