"""Index algebra of the prefill kernel's LDS tiles (no GPU).

The kernel (csrc/pa_prefill.h) defines its swizzled layouts by two functions of a row, and then
computes the addresses of its stores and MFMA operand reads from a per-lane part XOR a
compile-time part.  These tests restate both forms in Python and check, over every thread,
lane, token and step, that they name the same slot, that the loader threads' stores cover each
slot of a tile exactly once, and that the MFMA reads see the token order the stores wrote.
Head dims 128 (16 chunks of 8 dims a K row) and 64 (8 chunks).
"""

import pytest

KTILE = 64  # tokens per LDS tile


def kswz(t, ch):
    return (t & 15) if ch == 16 else ((t ^ (t >> 3)) & 7)


def vswz(d):
    return (d ^ (d >> 3)) & 7


def loader_role(tid, ch):
    """(tg, dc) of loader thread tid: tokens 4tg..4tg+3, dims 8dc..8dc+7."""
    p16, l16 = tid >> 4, tid & 15
    if ch == 16:
        dc = (l16 & 7) | ((p16 & 1) << 3)
        tg = ((p16 >> 1) & 3) | ((l16 >> 3) << 2) | ((p16 >> 3) << 3)
    else:
        dc = l16 & 7
        tg = ((p16 >> 1) & 3) | ((l16 >> 3) << 2) | ((p16 & 1) << 3)
    return tg, dc


def loaders(ch):
    return range(256 if ch == 16 else 128)


@pytest.mark.parametrize("D", [128, 64])
def test_k_tile_stores_and_reads_agree(D):
    ch = D // 8
    written = {}
    for tid in loaders(ch):
        tg, dc = loader_role(tid, ch)
        sk = dc ^ kswz(4 * tg, ch)
        for i in range(4):
            t = 4 * tg + i
            slot = t * ch + (sk ^ i)
            assert slot == t * ch + (dc ^ kswz(t, ch))
            assert slot not in written
            written[slot] = (t, dc)
    assert sorted(written) == list(range(KTILE * ch))
    # score operand: lane (lr, lg) of token block j at depth step c reads token 16j + lr,
    # dims 32c + 8lg .. +8 (chunk 4c + lg)
    for lane in range(64):
        lr, lg = lane & 15, lane >> 4
        klane = lg ^ (lr if ch == 16 else ((lr & 7) ^ (lr >> 3)))
        for j in range(4):
            for c in range(D // 32):
                slot = (16 * j + lr) * ch + (klane ^ (4 * c) ^ (0 if ch == 16 else (2 * j) & 7))
                assert slot == (16 * j + lr) * ch + ((4 * c + lg) ^ kswz(16 * j + lr, ch))
                assert written[slot] == (16 * j + lr, 4 * c + lg)


@pytest.mark.parametrize("D", [128, 64])
def test_v_tile_stores_and_reads_agree(D):
    ch = D // 8
    written = {}   # (16-byte slot, 8-byte half) -> (dim, 4 token positions)
    for tid in loaders(ch):
        tg, dc = loader_role(tid, ch)
        v_chunk, v_half = 4 * (tg >> 3) + (tg & 3), (tg >> 2) & 1
        sv = v_chunk ^ (dc & 7)
        # V^T position of token 32h + 16b + 4g + i is 32h + 8g + 4b + i
        toks = [4 * tg + i for i in range(4)]
        pos = [32 * (t >> 5) + 8 * ((t >> 2) & 3) + 4 * ((t >> 4) & 1) + (t & 3) for t in toks]
        for e in range(8):
            d = 8 * dc + e
            slot = d * 8 + (sv ^ e)
            assert slot == d * 8 + (v_chunk ^ vswz(d))
            key = (slot, v_half)
            assert key not in written
            # the 4 tokens land on consecutive positions of one 8-token chunk
            assert pos == list(range(8 * v_chunk + 4 * v_half, 8 * v_chunk + 4 * v_half + 4))
            written[key] = (d, tuple(toks))
    assert len(written) == D * 8 * 2
    # output operand: lane (lr, lg) of half h, dim block b reads dim 16b + lr, V^T positions
    # 32h + 8lg .. +8: tokens 4lg + i of 16-token blocks 2h and 2h + 1 (the lane's scores)
    for lane in range(64):
        lr, lg = lane & 15, lane >> 4
        for h in range(2):
            vlane = (4 * h + lg) ^ (lr & 7) ^ (lr >> 3)
            for b in range(D // 16):
                d = 16 * b + lr
                slot = d * 8 + (vlane ^ ((2 * b) & 7))
                assert slot == d * 8 + ((4 * h + lg) ^ vswz(d))
                got = written[(slot, 0)][1] + written[(slot, 1)][1]
                assert all(written[(slot, x)][0] == d for x in (0, 1))
                want = tuple(32 * h + 16 * blk + 4 * lg + i for blk in (0, 1) for i in range(4))
                assert got == want
