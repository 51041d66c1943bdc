"""Host-side replay of the prefill kernel's LDS layout (no GPU).

Replays the index arithmetic of prefill.hpp for one KV tile of 32 keys:
  - direct HBM->LDS loads: lane ln of a load instruction reads global chunk
    ln ^ swz(row) (16 bytes) and the hardware stores it at LDS byte 16*ln of
    the instruction's destination;
  - score operand (ds_read_b128): lane l reads key row l % 32, 8 dims starting
    at 16*s + 8*(l // 32), for k-step s;
  - value operand (ds_read_b64_tr_b16, 2 reads per fragment): within a
    16-lane group, destination lane i receives 16-bit element i % 4 of the
    8 bytes addressed by source lanes i // 4 + 4*k, k = 0..3 (the lane map
    measured on gfx950);
and checks that every MFMA operand lane receives the (key, dim) element the
matrix layout asks for, and that each group of lanes the LDS serves together
(16 lanes for 16-byte reads, 32 lanes for 8-byte reads, 64 banks of 4 bytes)
touches 64 distinct banks.
"""
import pytest

BN = 32


def swz(r):
    return ((r & 3) << 2) | ((r >> 2) & 3)


def lds_tile(D):
    """LDS bytes of one tile of rows of D bf16 dims, as a dict chunk-position ->
    (key, first dim).  Replays the kernel's load offsets: lane ln of the load
    whose first row is r0 takes row r0 + lr, lr = ln // CPR, and global chunk
    A ^ swz(r0) with A = (ln % CPR) ^ (lr << 2), which must equal the chunk
    (ln % CPR) ^ swz(row) the layout stores at LDS byte 16*ln."""
    RB = 2 * D
    CPR, RPI = RB // 16, 1024 // RB
    lds = {}
    for r0 in range(0, BN, RPI):
        for ln in range(64):
            lr = ln // CPR
            a = (ln % CPR) ^ (lr << 2)
            row, chunk = r0 + lr, a ^ swz(r0)
            assert chunk == (ln % CPR) ^ swz(row)
            pos = r0 * RB + 16 * ln  # destination byte of this lane
            assert pos not in lds
            lds[pos] = (row, 8 * chunk)
    assert len(lds) == BN * D // 8
    return lds


def element(lds, byte):
    """(key, dim) of the bf16 element stored at LDS byte offset `byte`."""
    key, dim0 = lds[byte - byte % 16]
    return key, dim0 + (byte % 16) // 2


def score_offsets(D, lane, s):
    """The kernel's form: P ^ ((s % 8) << 5) + 256*(s // 8), with
    P = row + 16*((hl ^ swz) & 1) + 32*(swz >> 1)."""
    l32, hl = lane & 31, lane >> 5
    sw = swz(l32)
    p = l32 * (2 * D) + (((hl ^ sw) & 1) << 4) + ((sw >> 1) << 5)
    off = (p ^ ((s % 8) << 5)) + 256 * (s // 8)
    # the layout's definition: chunk 2s + hl of row l32 at 16*(s//8) + ((2(s%8) + hl) ^ swz)
    assert off == l32 * (2 * D) + 256 * (s // 8) + (((2 * (s % 8) + hl) ^ sw) << 4)
    return off


def value_offsets(D, lane, db, k2, h):
    """The kernel's form: V_h ^ ((db % 4) << 6) + 256*(db // 4) + 16*k2 rows,
    V_0 = tr_row*2D + 8*(tr_i & 1) + ((tr_x ^ swz(tr_row)) << 4),
    V_1 = (V_0 ^ 32) + 8 rows."""
    tr_i, tr_g = lane & 15, lane >> 4
    tr_row = 4 * (tr_g >> 1) + (tr_i >> 2)
    tr_x = 2 * (tr_g & 1) + ((tr_i & 3) >> 1)
    v0 = tr_row * (2 * D) + (tr_i & 1) * 8 + ((tr_x ^ swz(tr_row)) << 4)
    v = v0 if h == 0 else (v0 ^ 32) + 8 * (2 * D)
    off = (v ^ ((db % 4) << 6)) + 256 * (db // 4) + 16 * k2 * (2 * D)
    # the layout's definition: chunk 4*db + tr_x of row tr_row + 8h at its swizzled place
    want = ((tr_row + 8 * h) * (2 * D) + (tr_i & 1) * 8
            + (((4 * (db % 4) + tr_x) ^ swz(tr_row + 8 * h)) << 4))
    assert off == want + 256 * (db // 4) + 16 * k2 * (2 * D)
    return off


def banks16(addrs):
    return {(a >> 2) & 63 for a in addrs for a in (a, a + 4, a + 8, a + 12)}


@pytest.mark.parametrize("D", [128, 256, 512])
def test_score_operand_reads(D):
    """D = 128 is the rotated-key slab of the d = 512 K=V layer (256-byte rows,
    four rows per direct load)."""
    lds = lds_tile(D)
    for s in range(D // 16):
        offs = [score_offsets(D, lane, s) for lane in range(64)]
        for lane, off in enumerate(offs):
            for e in range(8):
                # A operand of the 32x32x16 product: row = key lane%32, k = 8*(lane//32) + e
                assert element(lds, off + 2 * e) == (lane & 31, 16 * s + 8 * (lane >> 5) + e)
        for g in range(4):  # 16 lanes served together: 16 chunks x 4 banks
            assert len(banks16(offs[16 * g:16 * g + 16])) == 64, (D, s, g)


@pytest.mark.parametrize("D", [256, 512])
def test_value_operand_transpose_reads(D):
    lds = lds_tile(D)
    for db in range(D // 32):
        for k2 in range(2):
            for h in range(2):
                src = [value_offsets(D, lane, db, k2, h) for lane in range(64)]
                for half in range(2):  # 32 lanes served together, 8 bytes = 2 banks each
                    banks = {(a >> 2) & 63 for a in src[32 * half:32 * half + 32] for a in (a, a + 4)}
                    assert len(banks) == 64, (D, db, k2, h, half)
                for lane in range(64):
                    grp, i = lane // 16, lane % 16
                    got = [element(lds, src[16 * grp + i // 4 + 4 * k] + 2 * (i % 4)) for k in range(4)]
                    # A operand of O^T += V^T P^T: row = dim 32*db + lane%32; k slots 4h..4h+3
                    # hold keys 16*k2 + 8*h + 4*(lane//32) + 0..3 (the score-register order)
                    want = [(16 * k2 + 8 * h + 4 * (lane >> 5) + k, 32 * db + (lane & 31)) for k in range(4)]
                    assert got == want, (D, db, k2, h, lane)


@pytest.mark.parametrize("D,SW", [(512, 128), (256, 256), (512, 512)])
def test_rotation_items_cover_slab_once(D, SW):
    """Rotation items (chunk tid % SWC of row tid // SWC + m*RDR) cover every
    slab chunk once, and each 16 lanes write 16 distinct bank groups."""
    SWC = SW // 8
    IPT = BN * SWC // 256
    RDR = 256 // SWC
    seen = set()
    for m in range(IPT):
        for tid in range(256):
            c, r = tid % SWC, tid // SWC + m * RDR
            pos = r * (2 * SW) + ((c ^ swz(r)) << 4)
            assert pos not in seen
            seen.add(pos)
        for g in range(16):
            addrs = [(tid // SWC + m * RDR) * (2 * SW) + (((tid % SWC) ^ swz(tid // SWC + m * RDR)) << 4)
                     for tid in range(16 * g, 16 * g + 16)]
            assert len(banks16(addrs)) == 64
    assert len(seen) == BN * SWC


# ---- decode tiles: 16 contiguous cache rows, chunk c of row r at c ^ dswz(r) ----

TRD = 16


def dswz(r):
    return ((r & 7) << 1) | ((r >> 3) & 1)


def decode_tile(D):
    CPR = D // 8
    RPI = 64 // CPR
    lds = {}
    for n in range(TRD // RPI):
        for ln in range(64):
            row = n * RPI + ln // CPR
            chunk = (ln % CPR) ^ dswz(row)
            pos = n * 1024 + 16 * ln
            assert pos not in lds and 0 <= chunk < CPR
            lds[pos] = (row, 8 * chunk)
    assert len(lds) == TRD * D // 8
    return lds


@pytest.mark.parametrize("D", [256, 512])
def test_decode_score_operand_reads(D):
    """16x16x32 A operand: lane l holds key row l % 16, dims 32*s + 8*(l // 16) .. +7."""
    lds = decode_tile(D)
    for s in range(D // 32):
        offs = []
        for lane in range(64):
            row, gq = lane & 15, lane >> 4
            c = 4 * s + gq
            off = row * (2 * D) + 256 * (c >> 4) + (((c & 15) ^ dswz(row)) << 4)
            offs.append(off)
            for e in range(8):
                assert element(lds, off + 2 * e) == (row, 32 * s + 8 * gq + e)
        for g in range(4):
            assert len(banks16(offs[16 * g:16 * g + 16])) == 64, (D, s, g)


@pytest.mark.parametrize("D", [256, 512])
def test_decode_value_operand_transpose_reads(D):
    """16x16x16 A operand V^T: lane l holds dim 16*db + l % 16, keys 4*(l // 16) .. +3."""
    lds = decode_tile(D)
    for db in range(D // 16):
        src = []
        for lane in range(64):
            row, gq = lane & 15, lane >> 4
            trow, tch = 4 * gq + (row >> 2), (row & 3) >> 1
            c = 2 * db + tch
            src.append(trow * (2 * D) + (row & 1) * 8 + 256 * (c >> 4) + (((c & 15) ^ dswz(trow)) << 4))
        for half in range(2):
            banks = {(a >> 2) & 63 for a in src[32 * half:32 * half + 32] for a in (a, a + 4)}
            assert len(banks) == 64, (D, db, half)
        for lane in range(64):
            grp, i = lane // 16, lane % 16
            got = [element(lds, src[16 * grp + i // 4 + 4 * k] + 2 * (i % 4)) for k in range(4)]
            assert got == [(4 * grp + k, 16 * db + i) for k in range(4)], (D, db, lane)


# ---- fp8 decode tiles: 32 rows of D one-byte codes, chunk c of row r at c ^ fswz(r) ----

TR8 = 32


def fswz(r):
    return (r & 3) | ((((r >> 3) + 2 * ((r >> 2) & 1)) & 3) << 2)


def fp8_tile(D):
    CPR = D // 16
    RPI = 64 // CPR
    lds = {}
    for n in range(TR8 // RPI):
        for ln in range(64):
            row = n * RPI + ln // CPR
            chunk = (ln % CPR) ^ fswz(row)
            pos = n * 1024 + 16 * ln
            assert pos not in lds and 0 <= chunk < CPR
            lds[pos] = (row, 16 * chunk)
    assert len(lds) == TR8 * D // 16
    return lds


def code_at(lds, byte):
    """(key, dim) of the code stored at LDS byte offset `byte`."""
    key, dim0 = lds[byte - byte % 16]
    return key, dim0 + byte % 16


def kchunk(s, gq):
    return 8 * (s >> 1) + 2 * gq + (s & 1)


@pytest.mark.parametrize("D", [256, 512])
def test_fp8_decode_score_operand_reads(D):
    """Half h of the score product: operand row r is key 8*(r//4) + 4h + r%4, so
    output register j of lane group g is key 8g + 4h + j; k-step s of lane group
    gq takes dims 8*kchunk(s, gq) .. +7 (the query operand uses the same map),
    and over all k-steps every dim is taken exactly once."""
    lds = fp8_tile(D)
    for g in range(4):
        for j in range(4):
            for h in range(2):
                r = 4 * g + j
                assert 8 * (r >> 2) + 4 * h + (r & 3) == 8 * g + 4 * h + j
    for gq in range(4):
        dims = sorted(8 * kchunk(s, gq) + j for s in range(D // 32) for j in range(8))
        assert len(set(dims)) == len(dims) == D // 4
    assert sorted(8 * kchunk(s, gq) + j for s in range(D // 32) for gq in range(4)
                  for j in range(8)) == list(range(D))
    for h in range(2):
        for u2 in range(D // 64):
            offs = []
            for lane in range(64):
                row, gq = lane & 15, lane >> 4
                kr = 8 * (row >> 2) + 4 * h + (row & 3)
                off = kr * D + (((4 * u2 + gq) ^ fswz(kr)) << 4)
                offs.append(off)
                for e in range(2):
                    for j in range(8):
                        assert code_at(lds, off + 8 * e + j) == (kr, 8 * kchunk(2 * u2 + e, gq) + j)
            for g in range(4):
                assert len(banks16(offs[16 * g:16 * g + 16])) == 64, (D, h, u2, g)


@pytest.mark.parametrize("D", [256, 512])
def test_fp8_decode_value_operand_transpose_reads(D):
    """8-bit transpose reads (gfx950 lane map: within 16 lanes, source lane n
    holds row n // 2, bytes 8*(n % 2) .. +7 of an 8 x 16 byte block, and
    destination lane i gets column i): lane l holds dim 16*db + l % 16 of keys
    8*(l // 16) .. +7, the keys its P^T operand holds."""
    lds = fp8_tile(D)
    for db in range(D // 16):
        src = []
        for lane in range(64):
            n, gq = lane & 15, lane >> 4
            kk = 8 * gq + (n >> 1)
            src.append(kk * D + (n & 1) * 8 + ((db ^ fswz(kk)) << 4))
        for half in range(2):
            banks = {(a >> 2) & 63 for a in src[32 * half:32 * half + 32] for a in (a, a + 4)}
            assert len(banks) == 64, (D, db, half)
        for lane in range(64):
            grp, i = lane // 16, lane % 16
            got = [code_at(lds, src[16 * grp + 2 * k + i // 8] + i % 8) for k in range(8)]
            assert got == [(8 * grp + k, 16 * db + i) for k in range(8)], (D, db, lane)


# ---- staged output rows of the d = 256 prefill epilogue ----
# A wave writes 16 rows of fp32 output into LDS (lane (l32, hl) writes the
# 16-byte chunks c = 8*db + 2*g4 + hl of its row l32 - 16p, at chunk c ^ r),
# then reads each row back whole (lane l reads chunk l of row r, at l ^ r).

@pytest.mark.parametrize("p", [0, 1])
def test_staged_output_rows(p):
    D = 256
    CPR = D * 4 // 16  # 16-byte chunks per fp32 row
    written = {}
    for db in range(D // 32):
        for g4 in range(4):
            banks = []
            for lane in range(64):
                l32, hl = lane & 31, lane >> 5
                r = l32 - 16 * p
                if not 0 <= r < 16:
                    continue
                c = 8 * db + 2 * g4 + hl
                pos = r * CPR + (c ^ r)
                assert pos not in written
                written[pos] = (r, c)
                banks.append((lane // 16, ((c ^ r) % 16)))
            # the 16 lanes served together (one hl, 16 rows) hit 16 distinct bank quads
            for grp in set(g for g, _ in banks):
                quads = [q for g, q in banks if g == grp]
                assert len(quads) == len(set(quads)) == 16
    assert len(written) == 16 * CPR
    for r in range(16):
        got = [written[r * CPR + (lane ^ r)] for lane in range(64)]
        assert got == [(r, lane) for lane in range(64)]  # row r, chunks in order
        # a 16-byte read is served 16 lanes at a time: 16 distinct bank quads
        for g in range(4):
            assert len({(lane ^ r) % 16 for lane in range(16 * g, 16 * g + 16)}) == 16


# ---- fp8 K=V decode tiles: 16 rows of D one-byte codes, chunk c of row r at c ^ (r & 15) ----

TRK = 16


def kswz(r):
    return r & 15


def fp8_kv_tile(D):
    CPR = D // 16
    RPI = 64 // CPR
    lds = {}
    for n in range(TRK // RPI):
        for ln in range(64):
            row = n * RPI + ln // CPR
            chunk = (ln % CPR) ^ kswz(row)
            pos = n * 1024 + 16 * ln
            assert pos not in lds and 0 <= chunk < CPR
            lds[pos] = (row, 16 * chunk)
    assert len(lds) == TRK * D // 16
    return lds


@pytest.mark.parametrize("D", [256, 512])
def test_fp8_kv_decode_score_operand_reads(D):
    """One key row per lane (row = lane % 16): the 16-byte read of chunk
    4*u2 + gq holds the dims of k-steps 2*u2 and 2*u2 + 1 in kchunk order, and
    each 16-lane read covers all 64 banks."""
    lds = fp8_kv_tile(D)
    for u2 in range(D // 64):
        offs = []
        for lane in range(64):
            row, gq = lane & 15, lane >> 4
            off = row * D + (((4 * u2 + gq) ^ kswz(row)) << 4)
            offs.append(off)
            for e in range(2):
                for j in range(8):
                    assert code_at(lds, off + 8 * e + j) == (row, 8 * kchunk(2 * u2 + e, gq) + j)
        for g in range(4):
            assert len(banks16(offs[16 * g:16 * g + 16])) == 64, (D, u2, g)


@pytest.mark.parametrize("D", [256, 512])
def test_fp8_kv_decode_value_operand_transpose_reads(D):
    """8-bit transpose reads whose eight source rows are keys 4g .. 4g+3 twice:
    the first four bytes lane l receives are dim 16*db + l % 16 of keys
    4*(l // 16) .. +3, the keys its P^T operand holds (score register j of
    lane group g is key 4g + j); no two different words share a bank."""
    lds = fp8_kv_tile(D)
    for db in range(D // 16):
        src = []
        for lane in range(64):
            n, gq = lane & 15, lane >> 4
            kr = 4 * gq + ((n >> 1) & 3)
            src.append(kr * D + (n & 1) * 8 + ((db ^ kswz(kr)) << 4))
        for half in range(2):
            words = {w for a in src[32 * half:32 * half + 32] for w in (a >> 2, (a >> 2) + 1)}
            banks = {}
            for wd in words:
                banks.setdefault(wd & 63, set()).add(wd)
            assert all(len(v) == 1 for v in banks.values()), (D, db, half)
        for lane in range(64):
            grp, i = lane // 16, lane % 16
            got = [code_at(lds, src[16 * grp + 2 * k + i // 8] + i % 8) for k in range(8)]
            assert got[:4] == [(4 * grp + k, 16 * db + i) for k in range(4)], (D, db, lane)
            assert got[4:] == got[:4]
