"""Pins for the oracle's packing units and layouts.

Sources: pwwt.cn 2/3/5/6-bit mixed quantization page, s3.1 (units: smallest n with n*b
divisible by 8) and s3.2 (little-endian unit reads; 3-bit shifts 0,3,...,21 with value 2
straddling a byte boundary; 5-bit read as a 64-bit integer; 6-bit shifts 0,6,12,18;
the all-0x07 test)."""
import json
import os

import numpy as np
import pytest

import oracle

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_values.json")))
BITS = (2, 3, 4, 5, 6)


@pytest.mark.parametrize("case", GOLD["packing_units"], ids=lambda c: f"b{c['bits']}")
def test_units_match_pages(case):
    assert oracle.unit_values(case["bits"]) == case["values"]
    assert oracle.unit_bytes(case["bits"]) == case["bytes"]


@pytest.mark.parametrize("case", GOLD["unpack_all_ones"], ids=lambda c: f"b{c['bits']}")
def test_all_ones_pattern(case):
    codes = np.array([case["codes"]], np.uint8)
    packed = oracle.pack_canonical(codes, case["bits"])
    assert list(packed) == case["bytes"]
    assert np.array_equal(oracle.unpack_canonical(packed, 1, codes.shape[1], case["bits"]), codes)


def test_hand_derived_units():
    # 3-bit codes 0..7, LSB-first: bit stream 000 100 010 110 001 101 011 111
    # -> bytes 0b10001000, 0b11000110, 0b11111010.
    assert list(oracle.pack_canonical(np.array([range(8)], np.uint8), 3)) == [0x88, 0xC6, 0xFA]
    # 6-bit codes 1,1,1,1: v = 1 + 2^6 + 2^12 + 2^18 = 0x041041 -> 41 10 04.
    assert list(oracle.pack_canonical(np.array([[1, 1, 1, 1]], np.uint8), 6)) == [0x41, 0x10, 0x04]
    # 5-bit codes 31,0,31,0,...: ones at bit runs 0-4, 10-14, 20-24, 30-34.
    assert list(oracle.pack_canonical(np.array([[31, 0] * 4], np.uint8), 5)) == \
        [0x1F, 0x7C, 0xF0, 0xC1, 0x07]
    # 2-bit 1,2,3,0 -> 1 + 2*4 + 3*16 = 0x39; 4-bit low nibble first: 5,10 -> 0xA5.
    assert list(oracle.pack_canonical(np.array([[1, 2, 3, 0]], np.uint8), 2)) == [0x39]
    assert list(oracle.pack_canonical(np.array([[5, 10]], np.uint8), 4)) == [0xA5]


@pytest.mark.parametrize("bits", BITS)
def test_bitstream_equivalence(bits):
    """Unit packing with LSB-first values and little-endian unit bytes is the same as
    one continuous LSB-first bit stream of the codes.  A wrong shift, mask, unit size
    or byte order breaks this."""
    rng = np.random.default_rng(bits)
    N, K = 5, 512
    codes = rng.integers(0, 1 << bits, (N, K)).astype(np.uint8)
    bitplanes = np.unpackbits(codes[..., None], axis=-1, bitorder="little")[..., :bits]
    stream = np.packbits(bitplanes.reshape(N, K * bits), axis=-1, bitorder="little")
    assert np.array_equal(oracle.pack_canonical(codes, bits), stream.reshape(-1))


def test_three_bit_straddle_closed_form():
    """Value 2 of a 3-bit unit is bits 6..8: the top two bits of byte 0 and the lowest
    bit of byte 1."""
    rng = np.random.default_rng(3)
    units = rng.integers(0, 256, (1000, 3)).astype(np.uint8)
    codes = oracle.unpack_canonical(units.reshape(-1), 1000, 8, 3)
    expect = (units[:, 0] >> 6) | ((units[:, 1] & 1) << 2)
    assert np.array_equal(codes[:, 2], expect)
    # 5-bit value 6 is bits 30..34: top two bits of byte 3, low three of byte 4.
    u5 = rng.integers(0, 256, (1000, 5)).astype(np.uint8)
    c5 = oracle.unpack_canonical(u5.reshape(-1), 1000, 8, 5)
    assert np.array_equal(c5[:, 6], (u5[:, 3] >> 6) | ((u5[:, 4] & 7) << 2))


@pytest.mark.parametrize("bits", (3, 6))
def test_exhaustive_three_byte_roundtrip(bits):
    """Every 24-bit pattern unpacks and repacks to itself (3-bit and 6-bit units)."""
    pats = np.arange(1 << 24, dtype=np.uint32)
    raw = pats.view(np.uint8).reshape(-1, 4)[:, :3].copy().reshape(-1)
    nv = oracle.unit_values(bits)
    codes = oracle.unpack_canonical(raw, 1 << 24, nv, bits)
    assert codes.max() == (1 << bits) - 1
    assert np.array_equal(oracle.pack_canonical(codes, bits), raw)


@pytest.mark.parametrize("bits", (2, 4))
def test_exhaustive_byte_roundtrip(bits):
    raw = np.arange(256, dtype=np.uint8)
    codes = oracle.unpack_canonical(raw, 256, 8 // bits, bits)
    assert np.array_equal(oracle.pack_canonical(codes, bits), raw)
    # low bits first: the first value of byte v is v & mask
    assert np.array_equal(codes[:, 0], raw & ((1 << bits) - 1))


def test_random_forty_bit_roundtrip():
    rng = np.random.default_rng(5)
    raw = rng.integers(0, 256, 2_000_000 * 5).astype(np.uint8)
    codes = oracle.unpack_canonical(raw, 2_000_000, 8, 5)
    assert np.array_equal(oracle.pack_canonical(codes, 5), raw)


@pytest.mark.parametrize("bits", BITS)
def test_device_layout_byte_map(bits):
    """The byte map of the device layout moves whole canonical bytes of the group-reordered
    codes (so every page unit stays intact) and keeps each 16-row x 256-k tile in its own
    512*b byte range; the reordering is a permutation inside each group."""
    N, K = 32, 512
    rowbytes = K * bits // 8
    offs = np.array([[oracle.device_offset(n, cb, K, bits) for cb in range(rowbytes)]
                     for n in range(N)])
    assert np.array_equal(np.sort(offs.reshape(-1)), np.arange(N * rowbytes))
    for n in range(N):
        for cb in range(rowbytes):
            k0 = (cb // bits) * 8
            tile = (n // 16) * (K // 256) + k0 // 256
            assert tile * 512 * bits <= offs[n, cb] < (tile + 1) * 512 * bits
    rng = np.random.default_rng(bits)
    codes = rng.integers(0, 1 << bits, (N, K)).astype(np.uint8)
    reord = oracle.device_reorder(codes, bits)
    assert np.array_equal(np.sort(reord, axis=1), np.sort(codes, axis=1))
    assert np.array_equal(oracle.device_reorder(reord, bits, inverse=True), codes)
    dev = oracle.pack_device(codes, bits)
    assert np.array_equal(dev[offs.reshape(-1)], oracle.pack_canonical(reord, bits))
    assert np.array_equal(oracle.unpack_device(dev, N, K, bits), codes)


# Distance in bits between the two values of a pair (G/2 values of b bits).
PAIR_GAP = {2: 16, 3: 12, 4: 16, 5: 20, 6: 12}


def chunk_int(dev, bits, tile, lane):
    """The lane's 8*b chunk bytes (documented offsets) as one little-endian integer."""
    F = 16 * (bits // 2)
    base = tile * 512 * bits
    by = [dev[base + (1024 * (c // 16) + 16 * lane + c % 16 if c < F else 64 * F + 8 * lane + (c - F))]
          for c in range(8 * bits)]
    return int.from_bytes(bytes(by), "little")


def pair_position(bits, j, i):
    """Chunk bit of the low value of pair i (values 2i, 2i+1) of block j."""
    if bits == 2:
        return 32 * (j // 2) + 2 * (4 * (j % 2) + i)
    if bits == 6:
        return 48 * j + 24 * (i // 2) + 6 * (i % 2)
    return 8 * bits * j + bits * i


@pytest.mark.parametrize("bits", BITS)
def test_device_layout_pair_rule(bits):
    """Independent decoder of the documented rule the GPU unpack relies on: the values 2i and
    2i+1 of every 8-k block sit PAIR_GAP bits apart in the lane chunk, so one mask yields an
    fp16 pair.  Checked value by value against the codes."""
    N, K = 16, 512
    rng = np.random.default_rng(100 + bits)
    codes = rng.integers(0, 1 << bits, (N, K)).astype(np.uint8)
    dev = oracle.pack_device(codes, bits)
    mask = (1 << bits) - 1
    for kt in range(K // 256):
        for lane in range(64):
            t, r = lane // 16, lane % 16
            v = chunk_int(dev, bits, kt, lane)
            for j in range(8):
                k0 = 256 * kt + 128 * (j // 4) + 32 * (j % 4) + 8 * t
                for i in range(4):
                    p = pair_position(bits, j, i)
                    assert (v >> p) & mask == codes[r, k0 + 2 * i]
                    assert (v >> (p + PAIR_GAP[bits])) & mask == codes[r, k0 + 2 * i + 1]


def test_device_layout_lane_chunks():
    """Documented lane chunk: lane l = 16*t + r of a tile holds, in order, the eight
    8-k blocks of row r starting at k0 = 128*(j//4) + 32*(j%4) + 8*t, j = 0..7; the
    first 16*floor(b/2) chunk bytes are in 16-byte slabs (1 KB apart), the rest in an
    8-byte tail slab."""
    K = 256
    for bits in BITS:
        F = 16 * (bits // 2)
        for lane in (0, 5, 17, 38, 63):
            t, r = lane // 16, lane % 16
            chunk = []
            for j in range(8):
                k0 = 128 * (j // 4) + 32 * (j % 4) + 8 * t
                for bib in range(bits):
                    chunk.append(oracle.device_offset(r, k0 * bits // 8 + bib, K, bits))
            want = [1024 * (c // 16) + 16 * lane + c % 16 if c < F else 64 * F + 8 * lane + (c - F)
                    for c in range(8 * bits)]
            assert chunk == want


# ---- zero points stored in b bits (mixed-bit page, s2.3) --------------------------------

@pytest.mark.parametrize("bits", [2, 3, 4, 5, 6])
@pytest.mark.parametrize("G", [1, 5, 32, 86, 128])
def test_packed_zeros_round_trip_and_size(bits, G):
    rng = np.random.default_rng(bits * 100 + G)
    z = rng.integers(0, 1 << bits, (7, G), dtype=np.uint8)
    p = oracle.pack_zeros(z, bits)
    assert p.shape == (7, 4 * ((G * bits + 31) // 32))
    assert (oracle.unpack_zeros(p, 7, G, bits) == z).all()


@pytest.mark.parametrize("bits", [2, 3, 5, 6])
def test_packed_zeros_bit_positions(bits):
    """Field g of a row is bits [g*b, g*b + b) of the little-endian row stream: a single
    all-ones field lands exactly there, every other bit of the row stays zero."""
    G = 40
    for g in (0, 1, 7, 10, 31, 39):
        z = np.zeros((1, G), np.uint8)
        z[0, g] = (1 << bits) - 1
        p = oracle.pack_zeros(z, bits)[0]
        stream = int.from_bytes(p.tobytes(), "little")
        assert stream == ((1 << bits) - 1) << (g * bits)


def test_packed_zeros_bits_per_weight():
    """The page's 2-bit, 32-weight block with an fp16 scale and a 2-bit zero point (about 2.56
    bits per weight): the zero-point bytes this layout stores for a 4096-wide row are exactly
    b bits per group, so codes + scales + packed zero points give that figure."""
    c = [c for c in GOLD["bits_per_weight"] if c["zp_bits"] == 2][0]
    G = 4096 // c["group"]
    row_bytes = 4096 * c["bits"] / 8 + G * c["scale_bytes"] + oracle.zero_row_bytes(G, c["zp_bits"])
    assert oracle.zero_row_bytes(G, c["zp_bits"]) == G * c["zp_bits"] // 8
    assert abs(row_bytes * 8 / 4096 - c["value_approx"]) <= c["tol"]
