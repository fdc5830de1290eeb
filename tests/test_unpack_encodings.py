"""The weight unpack encodings of the HIP kernels, checked on the CPU.

The kernels turn packed int4/int8 weights into 16-bit matrix-core operands by
OR-ing exponent bits around the raw bits (moe_device.h).  Each form must give
q + (a fixed offset) exactly, and the constant fragments that remove the
offsets must hold exactly minus that offset.  This emulates the byte permute
(v_perm_b32: selector bytes 0-3 pick bytes of the second operand, 4-7 of the
first, 0x0C gives zero) and the bit operations, and checks every value.
Packing follows the int4 reading of the pages (element 2c in the low nibble,
two's complement).
"""
import random
import struct

import numpy as np
import pytest


def perm(s0, s1, sel):
    b = list(s1.to_bytes(4, "little")) + list(s0.to_bytes(4, "little"))
    out = 0
    for k in range(4):
        c = (sel >> (8 * k)) & 0xFF
        v = b[c] if c < 8 else {0x0C: 0x00, 0x0D: 0xFF}[c]
        out |= v << (8 * k)
    return out


def bf16(h):
    return struct.unpack("<f", struct.pack("<I", h << 16))[0]


def f16(h):
    return float(np.frombuffer(struct.pack("<H", h), dtype=np.float16)[0])


def f32bits(x):
    return struct.unpack("<I", struct.pack("<f", x))[0]


def nibbles(w):
    q = [(w >> (4 * j)) & 0xF for j in range(8)]
    return [v - 16 if v >= 8 else v for v in q]


def int8s(w):
    q = [(w >> (8 * j)) & 0xFF for j in range(4)]
    return [v - 256 if v >= 128 else v for v in q]


WORDS = [0, 0xFFFFFFFF, 0x88888888, 0x77777777, 0x80808080, 0x7F7F7F7F, 0x01234567, 0xFEDCBA98] + \
    [random.Random(7).getrandbits(32) for _ in range(3000)]


@pytest.mark.parametrize("w", WORDS[:8])
def test_int4_bf16_natural_order_named_words(w):
    _check_int4_bf16_nat(w)


def _check_int4_bf16_nat(w):
    q = nibbles(w)
    u = w >> 4
    for i, sel in enumerate([0x0C040C00, 0x0C050C01, 0x0C060C02, 0x0C070C03]):
        r = ((perm(u, w, sel) ^ 0x00080008) & 0x000F000F) | 0x43004300
        assert bf16(r & 0xFFFF) == q[2 * i] + 136
        assert bf16(r >> 16) == q[2 * i + 1] + 136


def test_int4_forms_random_words():
    for w in WORDS:
        _check_int4_bf16_nat(w)
        q = nibbles(w)
        for i in range(4):
            # k-slot order (e_i, e_{i+4}): bf16 q + 136 and f16 q + 1032
            t = ((w >> (4 * i)) ^ 0x00080008) & 0x000F000F
            assert bf16((t | 0x43004300) & 0xFFFF) == q[i] + 136
            assert bf16((t | 0x43004300) >> 16) == q[i + 4] + 136
            assert f16((t | 0x64006400) & 0xFFFF) == q[i] + 1032
            assert f16((t | 0x64006400) >> 16) == q[i + 4] + 1032


def test_int8_forms_random_words():
    for w in WORDS:
        q = int8s(w)
        t = w ^ 0x80808080
        # bf16 q + 128 from byte converts: the upper halves of exact f32 values
        fb = [f32bits(float((t >> (8 * j)) & 0xFF)) for j in range(4)]
        r0, r1 = perm(fb[1], fb[0], 0x07060302), perm(fb[3], fb[2], 0x07060302)
        assert [bf16(r0 & 0xFFFF), bf16(r0 >> 16), bf16(r1 & 0xFFFF), bf16(r1 >> 16)] == [v + 128 for v in q]
        # f16 q + 1152: 0x64 high bytes from a constant operand
        a0, a1 = perm(0x64646464, t, 0x04010400), perm(0x64646464, t, 0x04030402)
        assert [f16(a0 & 0xFFFF), f16(a0 >> 16), f16(a1 & 0xFFFF), f16(a1 >> 16)] == [v + 1152 for v in q]


def test_offset_constants():
    assert bf16(0xC308) == -136.0 and bf16(0xC300) == -128.0
    assert f16(0xE408) == -1032.0 and f16(0xE480) == -1152.0


def test_int4_into_int8_code_shifted():
    """The Q8 GEMM's int4 form (unpack_int4x8_i8): two masks and two byte
    permutes give byte j = code j << 4 as a signed byte, i.e. sixteen times the
    two's-complement code, for every nibble value in every position."""
    rng = np.random.default_rng(3)
    words = [0x76543210, 0xFEDCBA98, 0x0F0F0F0F, 0xF0F0F0F0] + [int(x) for x in rng.integers(0, 2**32, 2000)]
    for w in words:
        lo = (w << 4) & 0xF0F0F0F0
        hi = w & 0xF0F0F0F0
        r = [perm(hi, lo, 0x05010400), perm(hi, lo, 0x07030602)]
        got = [((r[j // 4] >> (8 * (j % 4))) & 0xFF) for j in range(8)]
        got = [b - 256 if b >= 128 else b for b in got]
        assert got == [16 * q for q in nibbles(w)], hex(w)


def test_int2_forms_every_word():
    """unpack_int2x8: pair i holds elements 2i (low half) and 2i + 1, each
    2^e + code + 2 with 2^e = 128 (bf16 0x4300) or 1024 (f16 0x6400): the int2
    encodings are code + 130 in bf16 and code + 1026 in f16, for all 65536
    eight-code words."""
    for w in range(1 << 16):
        t = (w & 0xFFFF) | ((w & 0xFFFF) << 14)
        codes = [((w >> (2 * j)) & 3) - (4 if (w >> (2 * j)) & 2 else 0) for j in range(8)]
        for hi, fn, off in ((0x4300, bf16, 130), (0x6400, f16, 1026)):
            vals = []
            for i in range(4):
                r = (((t >> (4 * i)) & 0x00030003) ^ 0x00020002) | (hi | (hi << 16))
                vals += [fn(r & 0xFFFF), fn(r >> 16)]
            assert vals == [float(c + off) for c in codes], hex(w)


def test_int2_small_batch_form_matches_int4_bits():
    """unpack_int2x8_ks (the small-batch kernel's int2 unpack): for every one
    of the 65536 eight-code words, the same 32-bit words that unpack_int4x8
    (bf16, 0x4300) and unpack_int4x8_f16 (0x6400) give for the same eight
    values packed as int4 (nibble j = element j, two's complement), so an
    int2 expert runs the int4 path's arithmetic bit for bit.  The k-slot
    order pairs elements (i, i + 4); the int2 field of element j sits at
    bits 2j..2j+1."""
    for w in range(1 << 16):
        t = w | (w << 8)
        codes = [((w >> (2 * j)) & 3) - (4 if (w >> (2 * j)) & 2 else 0) for j in range(8)]
        w4 = 0
        for j, c in enumerate(codes):
            w4 |= (c & 0xF) << (4 * j)
        for hi in (0x4300, 0x6400):
            h2 = hi | (hi << 16)
            r2 = [((((t >> (2 * i)) & 0x00030003) ^ 0x00020002) + 0x00060006) | h2 for i in range(4)]
            r4 = [(((w4 >> (4 * i)) ^ 0x00080008) & 0x000F000F) | h2 for i in range(4)]
            assert r2 == r4, hex(w)
        # and the int4 form is q + 136 in bf16, pair i = (element i, element i + 4)
        vals = []
        for i in range(4):
            r = (((w4 >> (4 * i)) ^ 0x00080008) & 0x000F000F) | 0x43004300
            vals += [bf16(r & 0xFFFF), bf16(r >> 16)]
        assert vals == [float(codes[j] + 136) for i in range(4) for j in (i, i + 4)], hex(w)
