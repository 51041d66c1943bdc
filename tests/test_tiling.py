"""Host-side replay of the prefill kernel's tile geometry (no GPU).

Mirrors the arithmetic of prefill.hpp: query tiles of TQ = 128*MB/G tokens,
KV tiles of 32 keys from the first key a row may see up to the tile holding
the workgroup's last token, padded up to a multiple of the LDS ring depth; each
tile is loaded through a buffer resource covering rows kv0 .. kv0+rows-1 of
one KV head.  Checks that every byte a load may touch lies inside the tensor
and that padding tiles hold only masked keys.  Regression test: padding tiles
past the end of the sequence once produced a negative row count, hence a
wrapped resource size and loads past the end of K.
"""
import pytest

BN = 32


def wg_tiles(S, G, MB, W):
    TQ = 4 * 32 * MB // G
    for qt in range((S + TQ - 1) // TQ):
        t0 = qt * TQ
        t_end = min(t0 + TQ, S)
        klo = max(0, t0 - W + 1) if W > 0 else 0
        yield t0, t_end, klo // BN, (t_end - 1) // BN


def tile_rows(kt, S):
    kv0 = min(kt * BN, ((S - 1) // BN) * BN)
    return kv0, min(S - kv0, BN)


SHAPES = [  # S, Hkv, D, G, MB, W, NST
    (300, 1, 512, 8, 1, 0, 3), (77, 2, 512, 8, 1, 0, 3), (333, 2, 256, 2, 2, 64, 3),
    (129, 1, 512, 2, 1, 0, 3), (190, 2, 512, 4, 1, 40, 2), (1, 1, 512, 8, 1, 0, 3),
    (33, 8, 256, 1, 2, 1, 3), (262144, 2, 512, 8, 1, 0, 3), (262144, 8, 256, 2, 2, 1024, 3),
    (8192, 8, 256, 2, 2, 1024, 3), (32768, 4, 512, 8, 1, 0, 3),
]


@pytest.mark.parametrize("shape", SHAPES)
def test_every_tile_load_stays_inside_k(shape):
    S, Hkv, D, G, MB, W, NST = shape
    rb = Hkv * D * 2
    for t0, t_end, kt0, kt1 in wg_tiles(S, G, MB, W):
        ktp = kt0 + (kt1 - kt0 + NST) // NST * NST - 1
        assert (ktp - kt0 + 1) % NST == 0 and ktp - kt1 < NST
        # interior tiles lie well inside the sequence; check the edges
        for kt in sorted(set(range(kt0, min(kt0 + 3, ktp + 1))) | set(range(max(kt0, kt1 - 3), ktp + 1))):
            kv0, rows = tile_rows(kt, S)
            assert 1 <= rows <= BN
            extent = rows * rb - (rb - 2 * D)   # bytes the resource covers
            assert 0 < extent <= BN * rb
            assert kv0 * rb + extent <= S * rb
            if kt > kt1:  # padding tile: every key is past the last token
                assert kt * BN > t_end - 1
