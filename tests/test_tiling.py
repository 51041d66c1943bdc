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
    # the shipped d = 256 instance (local layers and the vision encoder): one
    # 32-row block per wave, 2-stage ring, two workgroups per CU
    (8192, 8, 256, 2, 1, 1024, 2), (262144, 8, 256, 2, 1, 1024, 2), (131072, 8, 256, 2, 1, 512, 2),
    (1100, 8, 256, 2, 1, 512, 2), (333, 2, 256, 2, 1, 64, 2), (97, 8, 256, 1, 1, 0, 2),
    (2520, 8, 256, 1, 1, 0, 2), (10080, 8, 256, 1, 1, 0, 2), (700, 1, 256, 8, 1, 0, 2),
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


def rotated_order(kt0, ktp, rot=True):
    """Tiles in the order the 2-deep loop of the d = 256 windowed instances
    visits them: step i takes tile kt0 + (i + off) mod n, off = -kt0 mod n."""
    n = ktp - kt0 + 1
    off = (n - kt0 % n) % n if rot else 0
    return [kt0 + (i + off - n if i + off >= n else i + off) for i in range(n)]


@pytest.mark.parametrize("S,G,W", [(262144, 2, 1024), (8192, 2, 1024), (131072, 2, 512),
                                   (1100, 2, 512), (333, 2, 64), (700, 8, 1024), (97, 1, 0)])
def test_rotated_tile_order(S, G, W):
    """Every span is visited exactly once; without a window the order is the
    plain one; and two workgroups whose spans have the same length visit every
    tile they share at the same step (the point of the rotation: the
    workgroups that run together read a shared tile together)."""
    NST = 2
    TQ = 4 * 32 // G
    step_of = {}  # span length -> {tile: step}
    interior = set()  # span lengths of workgroups whose window starts inside the sequence
    for t0, t_end, kt0, kt1 in wg_tiles(S, G, 1, W):
        ktp = kt0 + (kt1 - kt0 + NST) // NST * NST - 1
        order = rotated_order(kt0, ktp)
        assert sorted(order) == list(range(kt0, ktp + 1))
        if W == 0:
            assert order == list(range(kt0, ktp + 1))
        n = len(order)
        seen = step_of.setdefault(n, {})
        for i, kt in enumerate(order):
            assert seen.setdefault(kt, i) == i, (t0, kt)
        if W > 0 and t0 - W + 1 > 0 and t_end == t0 + TQ:
            interior.add(n)
    # query tiles aligned to key tiles give every interior workgroup the same
    # span, so all of them share their tiles step for step
    assert len(interior) <= (1 if TQ % BN == 0 else 2)


VISION_SHAPES = [  # S, Hkv, G, valid patches per image
    (2520, 8, 1, [2520, 2520, 2520, 2496]), (10080, 8, 1, [10080]), (300, 2, 2, [300, 1, 0, 33]),
    (1100, 1, 8, [1099, 1100, 64, 65]),
]


@pytest.mark.parametrize("shape", VISION_SHAPES)
def test_vision_tile_loads_stay_inside_k(shape):
    """Vision instance (no causal mask): every query tile walks key tiles 0 ..
    (n_b - 1) / 32 of its image, padded to the 2-deep ring; an empty image
    loads nothing."""
    S, Hkv, G, lengths = shape
    D, NST = 256, 2
    rb = Hkv * D * 2
    for nv in lengths:
        if nv == 0:
            continue
        kt0, kt1 = 0, (nv - 1) // BN
        ktp = kt0 + (kt1 - kt0 + NST) // NST * NST - 1
        for kt in range(kt0, ktp + 1):
            kv0, rows = tile_rows(kt, S)
            assert 1 <= rows <= BN
            extent = rows * rb - (rb - 2 * D)
            assert 0 < extent <= BN * rb and kv0 * rb + extent <= S * rb
            if kt > kt1:  # padding tile: every key is past the image's patches
                assert kt * BN >= nv


# ---- decode grid numbering (unit_of_block in decode_common.hpp) ----
# Blocks map densely onto the (sequence, KV head, chunk) units that hold a
# visible row: the active chunks of sequence b are those up to its last
# visible row, none for an out-of-range position (the merge kernel writes its
# NaN rows), and with one chunk per sequence every (b, KV head) is a unit.
# The replay follows the kernel's scan 64 sequences at a time and checks that
# each active unit gets exactly one block per column block and no block gets
# anything else.

def active_chunks(P, window, capacity, chunk, nchunk):
    if P < 0 or (window == 0 and P >= capacity):
        return 0
    last = min(P, capacity - 1) if window > 0 else P
    return min(last // chunk + 1, nchunk)


def unit_of_block(blk, pos, Hkv, chunk, nchunk, window, capacity, ncb):
    B = len(pos)
    if nchunk == 1:
        nunit = B * Hkv
    else:
        nunit = Hkv * sum(active_chunks(p, window, capacity, chunk, nchunk) for p in pos)
    grp = blk // (8 * ncb)
    gsz = min(8, nunit - 8 * grp)
    if gsz <= 0:
        return None
    within = blk - grp * 8 * ncb
    if within >= gsz * ncb:
        return None
    unit, cb = 8 * grp + within % gsz, within // gsz
    if nchunk == 1:
        return cb, 0, unit // Hkv, unit % Hkv
    acc = 0
    for b0 in range(0, B, 64):
        n = [active_chunks(pos[b], window, capacity, chunk, nchunk) if b < B else 0
             for b in range(b0, b0 + 64)]
        incl, run = [], 0
        for x in n:
            run += x * Hkv
            incl.append(run)
        hits = [l for l in range(64) if acc + incl[l] > unit]
        if hits:
            l = hits[0]
            rem = unit - acc - incl[l] + n[l] * Hkv
            return cb, rem % n[l], b0 + l, rem // n[l]
        acc += incl[63]
    raise AssertionError("unit past every sequence")


DECODE_GRIDS = [  # B, Hkv, capacity, window, chunk, ncb, positions (seeded)
    (64, 2, 65536, 0, 1024, 1, "lengths"),
    (130, 1, 2500, 0, 1024, 1, "mixed"),
    (70, 1, 2200, 0, 1024, 4, "mixed"),
    (3, 2, 3000, 0, 1024, 3, [5000, -1, 2999]),
    (64, 8, 512, 512, 512, 1, "mixed"),
    (5, 2, 4096, 0, 1024, 1, [-1, -1, -1, -1, -1]),
    (200, 2, 4096, 0, 1024, 2, "edges"),
]


@pytest.mark.parametrize("grid", DECODE_GRIDS, ids=[f"B{g[0]}-C{g[2]}-ncb{g[5]}" for g in DECODE_GRIDS])
def test_decode_units_dense_and_complete(grid):
    import random
    B, Hkv, C, W, chunk, ncb, kind = grid
    rnd = random.Random(B * 7 + C)
    if kind == "lengths":
        pos = [rnd.randint(4096, 65536) - 1 for _ in range(B)]
    elif kind == "mixed":
        pos = [rnd.randint(-3, C + 50) for _ in range(B)]
    elif kind == "edges":
        pos = [rnd.choice([-1, 0, chunk - 1, chunk, C - 1, C]) for _ in range(B)]
    else:
        pos = kind
    nchunk = (C + chunk - 1) // chunk if W == 0 else 1
    seen = set()
    for blk in range(B * Hkv * ncb * nchunk):  # the launch's grid
        u = unit_of_block(blk, pos, Hkv, chunk, nchunk, W, C, ncb)
        if u is None:
            continue
        assert u not in seen, u
        seen.add(u)
    want = set()
    for b, P in enumerate(pos):
        n = 1 if nchunk == 1 else active_chunks(P, W, C, chunk, nchunk)
        want |= {(cb, c, b, h) for cb in range(ncb) for c in range(n) for h in range(Hkv)}
    assert seen == want
