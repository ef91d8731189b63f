"""Test-side Q4_K block packer, written from the public GGUF Q4_K layout
described byte by byte (the oracle's decoder describes it field by field).

Scale area (12 bytes):
  byte j,   j = 0..3 : bits 0-5 = scale of sub-block j,   bits 6-7 = bits 4-5 of the scale of sub-block j+4
  byte 4+j, j = 0..3 : bits 0-5 = min of sub-block j,     bits 6-7 = bits 4-5 of the min of sub-block j+4
  byte 8+j, j = 0..3 : bits 0-3 = bits 0-3 of the scale of sub-block j+4, bits 4-7 = bits 0-3 of its min
Quant area (128 bytes): byte 32c + l holds weight 64c + l in its low nibble and
weight 64c + 32 + l in its high nibble.
"""
import numpy as np


def pack_scales(sc, mn):
    sc = [int(v) for v in sc]
    mn = [int(v) for v in mn]
    b = [0] * 12
    for j in range(4):
        b[j] = (sc[j] & 63) | ((sc[j + 4] >> 4) << 6)
        b[4 + j] = (mn[j] & 63) | ((mn[j + 4] >> 4) << 6)
        b[8 + j] = (sc[j + 4] & 15) | ((mn[j + 4] & 15) << 4)
    return np.array(b, np.uint8)


def pack_quants(q):
    q = np.asarray(q, np.int64)
    out = np.zeros(128, np.uint8)
    for c in range(4):
        for l in range(32):
            out[32 * c + l] = (q[64 * c + l] & 15) | ((q[64 * c + 32 + l] & 15) << 4)
    return out


def make_block(d, dmin, sc, mn, q):
    blk = np.zeros(144, np.uint8)
    blk[0:2] = np.array([d], np.float16).view(np.uint8)
    blk[2:4] = np.array([dmin], np.float16).view(np.uint8)
    blk[4:16] = pack_scales(sc, mn)
    blk[16:] = pack_quants(q)
    return blk
