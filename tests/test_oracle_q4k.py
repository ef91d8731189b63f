"""Pins of the oracle's binary16 and Q4_K decoding (CPU only).

The Q4_K layout is the public GGUF k-quant block; the pages name the format only
(the Q4_K_M model file in forward_qwen3_moe.rs's serve contract note). Pins:
every fp16 bit pattern against numpy, a byte-by-byte bit map of the 12 packed
scale bytes, the nibble map of the 128 quant bytes, closed-form blocks, and
pack/unpack round trips. Interop with a real GGUF file is parity unpinned:
there is none here.
"""
import numpy as np
import pytest

import oracle
from tests.q4k_pack import make_block, pack_quants, pack_scales


def test_half_all_bit_patterns():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = oracle.half_to_double(bits)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # signed zero and subnormal edge
    assert np.signbit(got[0x8000]) and got[0x8000] == 0.0
    assert got[0x0001] == 2.0 ** -24
    assert got[0x7BFF] == 65504.0


# (byte, bit) -> (field, field bit); field = ("sc"|"m", sub-block), from the
# byte-by-byte layout in tests/q4k_pack.py's docstring.
def _expected_bitmap():
    m = {}
    for j in range(4):
        for b in range(6):
            m[(j, b)] = (("sc", j), b)
            m[(4 + j, b)] = (("m", j), b)
        for b in (6, 7):
            m[(j, b)] = (("sc", j + 4), b - 2)
            m[(4 + j, b)] = (("m", j + 4), b - 2)
        for b in range(4):
            m[(8 + j, b)] = (("sc", j + 4), b)
            m[(8 + j, 4 + b)] = (("m", j + 4), b)
    return m


def test_scale_bytes_bit_map():
    expected = _expected_bitmap()
    seen = set()
    for byte in range(12):
        for bit in range(8):
            blk = np.zeros(144, np.uint8)
            blk[4 + byte] = 1 << bit
            _, _, sc, mn, q = oracle.q4k_fields(blk)
            nz = [(("sc", j), int(sc[j])) for j in range(8) if sc[j]] + [(("m", j), int(mn[j])) for j in range(8) if mn[j]]
            assert len(nz) == 1, (byte, bit, nz)
            field, val = nz[0]
            efield, ebit = expected[(byte, bit)]
            assert field == efield and val == (1 << ebit), (byte, bit, field, val)
            seen.add((field, ebit))
            assert not q.any()
    assert len(seen) == 96  # the 16 six-bit fields use every bit exactly once


def test_quant_nibble_map():
    for byte in range(128):
        blk = make_block(1.0, 0.0, [1] * 8, [0] * 8, np.zeros(256, np.int64))
        blk[16:] = 0
        blk[16 + byte] = 0x21  # low nibble 1, high nibble 2
        w = oracle.q4k_dequant(blk.reshape(1, 144))
        c, l = divmod(byte, 32)
        exp = np.zeros(256)
        exp[64 * c + l] = 1.0
        exp[64 * c + 32 + l] = 2.0
        assert np.array_equal(w, exp), byte


def test_closed_form_block():
    # d = 1, dmin = 0.5, scale_j = j + 1, min_j = 2j, q_i = (i // 8) mod 16:
    # w_i = (j + 1) * q_i - j with j = i // 32. q differs between the two nibbles
    # of every quant byte and the fields differ between sub-blocks, so a swapped
    # nibble, sub-block or scale/min fails.
    i = np.arange(256)
    q = (i // 8) % 16
    j = i // 32
    blk = make_block(1.0, 0.5, [jj + 1 for jj in range(8)], [2 * jj for jj in range(8)], q)
    w = oracle.q4k_dequant(blk.reshape(1, 144))
    assert np.array_equal(w, (j + 1) * q - j)


def test_all_max_block():
    blk = np.full(144, 0xFF, np.uint8)
    blk[0:2] = np.array([1.0], np.float16).view(np.uint8)
    blk[2:4] = np.array([1.0], np.float16).view(np.uint8)
    w = oracle.q4k_dequant(blk.reshape(1, 144))
    assert np.all(w == 63 * 15 - 63)  # 882


def test_zero_scale_gives_minus_min():
    rng = np.random.default_rng(1)
    mn = rng.integers(0, 64, 8)
    blk = make_block(3.0, 0.25, [0] * 8, mn, rng.integers(0, 16, 256))
    w = oracle.q4k_dequant(blk.reshape(1, 144))
    assert np.array_equal(w, -0.25 * np.repeat(mn, 32))


def test_subnormal_scales():
    blk = make_block(0.0, 0.0, [63] * 8, [5] * 8, np.full(256, 15))
    blk[0:2] = np.array([0x0001], np.uint16).view(np.uint8)  # d = 2^-24
    blk[2:4] = np.array([0x0003], np.uint16).view(np.uint8)  # dmin = 3 * 2^-24
    w = oracle.q4k_dequant(blk.reshape(1, 144))
    assert np.all(w == (63 * 15 - 3 * 5) * 2.0 ** -24)


def test_pack_unpack_round_trip_random_scale_bytes():
    rng = np.random.default_rng(7)
    for _ in range(500):
        s = rng.integers(0, 256, 12).astype(np.uint8)
        blk = np.zeros(144, np.uint8)
        blk[4:16] = s
        _, _, sc, mn, _ = oracle.q4k_fields(blk)
        assert np.array_equal(pack_scales(sc, mn), s)


@pytest.mark.parametrize("field", range(16))
def test_unpack_pack_each_field_sweep(field):
    rng = np.random.default_rng(field)
    for v in range(64):
        sc = rng.integers(0, 64, 8)
        mn = rng.integers(0, 64, 8)
        if field < 8:
            sc[field] = v
        else:
            mn[field - 8] = v
        blk = np.zeros(144, np.uint8)
        blk[4:16] = pack_scales(sc, mn)
        _, _, sc2, mn2, _ = oracle.q4k_fields(blk)
        assert np.array_equal(sc2, sc) and np.array_equal(mn2, mn)


def test_quants_round_trip():
    rng = np.random.default_rng(3)
    q = rng.integers(0, 16, 256)
    blk = np.zeros(144, np.uint8)
    blk[16:] = pack_quants(q)
    _, _, _, _, q2 = oracle.q4k_fields(blk)
    assert np.array_equal(q2, q)


def test_matrix_dequant_row_major_blocks():
    # A [2][512] matrix = 2 rows x 2 blocks; each block holds a distinct constant.
    blocks = np.zeros((2, 2, 144), np.uint8)
    for r in range(2):
        for b in range(2):
            blocks[r, b] = make_block(1.0, 0.0, [1] * 8, [0] * 8, np.full(256, 1 + 2 * r + b))
    w = oracle.q4k_dequant(blocks)
    assert w.shape == (2, 512)
    assert np.all(w[0, :256] == 1) and np.all(w[0, 256:] == 2)
    assert np.all(w[1, :256] == 3) and np.all(w[1, 256:] == 4)
