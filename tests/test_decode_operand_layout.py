"""Byte algebra of the matrix-core decode's 8-bit V operand (no GPU).

For the output product O += P V, lane (lr, kg) needs, for each of its dims e, the values of
its four tokens 4kg .. 4kg+3 in token order: two 16-bit pairs (tokens 0, 1 | 2, 3).  Over an
E4M3 cache the lane holds four rows of codes, word w of row j being dims 4w .. 4w+3 of token
j, one byte each.  csrc/pa_decode_mfma.h gathers the codes with v_perm_b32 before converting:
x01 = perm(row1[w], row0[w], sel_k), x23 = perm(row3[w], row2[w], sel_k) with sel_0 =
0x05010400 and sel_2 = 0x07030602, then converts half word b of x01 / x23 (a scaled packed
conversion turns bytes 2b, 2b+1 of a word into the low / high 16-bit value) for dim 4w + k + b.
These tests emulate v_perm_b32 and the half-word choice and check, for every dim and every
possible byte value, that the pairs are exactly the four tokens' codes of that dim in order --
the same operand the 16-bit path builds by transposing converted rows.
"""

import random

import pytest


def v_perm_b32(s0, s1, sel):
    """Byte i of the result is byte sel_i of the 8-byte value {s0, s1} (s1 the low word);
    only selectors 0-7 occur here."""
    src = s1 | (s0 << 32)
    out = 0
    for i in range(4):
        b = (sel >> (8 * i)) & 0xFF
        assert b < 8
        out |= ((src >> (8 * b)) & 0xFF) << (8 * i)
    return out


def half_word_codes(word, hi):
    """The two codes a scaled packed conversion reads: bytes 0, 1 (hi false) or 2, 3."""
    sh = 16 if hi else 0
    return ((word >> sh) & 0xFF, (word >> (sh + 8)) & 0xFF)


def operand_codes(rows, w, k, b):
    sel = 0x05010400 if k == 0 else 0x07030602
    x01 = v_perm_b32(rows[1][w], rows[0][w], sel)
    x23 = v_perm_b32(rows[3][w], rows[2][w], sel)
    return half_word_codes(x01, b) + half_word_codes(x23, b)


@pytest.mark.parametrize("VW", [1, 2, 4])   # head dims 64, 128, 256: D/16 dims per lane
def test_fp8_v_operand_is_the_token_column(VW):
    rng = random.Random(77 + VW)
    for _ in range(200):
        rows = [[rng.getrandbits(32) for _ in range(VW)] for _ in range(4)]
        for w in range(VW):
            for k in (0, 2):
                for b in (0, 1):
                    e = 4 * w + k + b
                    want = tuple((rows[j][e // 4] >> (8 * (e % 4))) & 0xFF for j in range(4))
                    assert operand_codes(rows, w, k, b) == want


def test_fp8_v_operand_every_byte_value():
    """Each byte position of each token row reaches the right operand slot for all 256 values
    (the permutes move bytes; nothing depends on their value)."""
    for v in range(256):
        for j in range(4):
            for e in range(4):
                rows = [[0] for _ in range(4)]
                rows[j][0] = v << (8 * e)
                got = operand_codes(rows, 0, e & 2, e & 1)
                want = tuple(v if jj == j else 0 for jj in range(4))
                assert got == want, (v, j, e)
