"""CPU model of the LDS tile layouts of the matrix-core kernels.

gfx950's LDS has 64 banks of 4 bytes.  A wave's LDS read is served in
passes: a 128-bit read (``ds_read_b128``) serves 16 lanes per pass (16 x 16 B
= 256 B), a transposing ``ds_read_b64_tr_b16`` 32 lanes (32 x 8 B).  A pass is
conflict-free when the dwords its lanes touch fall in distinct banks.

The address functions below restate the kernels' own (the GEMM's
K-contiguous and M/N-contiguous operand tiles, and the attention kernels'
row-major K/V/Q/dO tiles); the tests check, for every tile height the
kernels instantiate, that

* every fragment read is conflict-free in every pass,
* the chunk swizzle is a bijection on each row (or k-row), and
* the LDS-direct loader's map (which LDS chunk each lane fills from which
  source row and column) is the inverse of the readers' map,

and that the earlier M/N swizzle ``c ^ 2 (k mod 8)`` of the 256- and
512-byte k-rows fails the transposing read, which is why it was replaced.
"""
import itertools

import pytest

BANKS = 64


def banks_of(addr, nbytes):
    return [((addr >> 2) + i) % BANKS for i in range(nbytes // 4)]


def conflict_free(addrs, nbytes, lanes_per_pass):
    """addrs: the 64 lanes' byte addresses of one instruction."""
    for p in range(0, 64, lanes_per_pass):
        seen = []
        for lane in range(p, p + lanes_per_pass):
            seen += banks_of(addrs[lane], nbytes)
        if len(seen) != len(set(seen)):
            return False
    return True


# ----------------------------------------------------------- GEMM operand tiles

def kofs(bk, row, c):
    """K-contiguous [ROWS][BK] tile: byte offset of 16-byte chunk c of row `row`."""
    if bk == 32:
        return row * 64 + ((c ^ ((row >> 2) & 3)) << 4)
    return row * 128 + ((c ^ ((row ^ (row >> 3)) & 7)) << 4)


def mswz(nch, k):
    if nch >= 16:
        return ((k & 3) << 2) & (nch - 1)
    return ((k & 7) << 1) & (nch - 1)


def mswz_previous(nch, k):
    """The swizzle the M/N tiles used before: c ^ 2 (k mod 8) at every height."""
    return ((k & 7) << 1) & (nch - 1)


def mofs(rows, k, c, swz=mswz):
    """M/N-contiguous [BK][ROWS] tile: byte offset of chunk c of k-row k."""
    nch = rows // 8
    return k * rows * 2 + ((c ^ swz(nch, k)) << 4)


def kmajor_fragment_addrs(bk, tr, kk):
    return [kofs(bk, tr + (lane & 31), kk * 2 + (lane >> 5)) for lane in range(64)]


def mnmajor_fragment_addrs(rows, tr, kk, half, swz=mswz):
    out = []
    for lane in range(64):
        g, R = lane >> 4, lane & 15
        m = tr + 16 * (g & 1) + 4 * (R & 3)
        k = kk * 16 + 8 * (g >> 1) + 4 * half + (R >> 2)
        out.append(mofs(rows, k, m >> 3, swz) + (m & 7) * 2)
    return out


# Tile heights (rows of an operand tile) the GEMM instantiates: 256 x 256 and
# 256 x 128 tiles (eight waves), 128 x 128 and 128 x 64 (four waves), 64 x 64,
# and the 256 x 128 half-width tail of a pair.
GEMM_ROWS = [64, 128, 256]


@pytest.mark.parametrize("rows", GEMM_ROWS)
@pytest.mark.parametrize("bk", [32, 64])
def test_gemm_kmajor_fragments_conflict_free(rows, bk):
    for tr in range(0, rows, 32):
        for kk in range(bk // 16):
            assert conflict_free(kmajor_fragment_addrs(bk, tr, kk), 16, 16), (tr, kk)


@pytest.mark.parametrize("rows", GEMM_ROWS)
@pytest.mark.parametrize("bk", [32, 64])
def test_gemm_mnmajor_transposing_fragments_conflict_free(rows, bk):
    for tr in range(0, rows, 32):
        for kk in range(bk // 16):
            for half in (0, 1):
                assert conflict_free(mnmajor_fragment_addrs(rows, tr, kk, half), 8, 32), (tr, kk, half)


@pytest.mark.parametrize("rows", [128, 256])
def test_previous_mn_swizzle_conflicts(rows):
    """k-rows of 256 and 512 bytes start on the same bank; c ^ 2 (k mod 8)
    leaves k-rows 4j and 4j+1 in one group of four chunks: a two-way
    conflict on the transposing read."""
    bad = [not conflict_free(mnmajor_fragment_addrs(rows, tr, kk, half, mswz_previous), 8, 32)
           for tr in range(0, rows, 32) for kk in range(4) for half in (0, 1)]
    assert all(bad)


@pytest.mark.parametrize("rows", GEMM_ROWS)
@pytest.mark.parametrize("bk", [32, 64])
def test_gemm_swizzles_are_bijections(rows, bk):
    for row in range(rows):
        got = sorted(kofs(bk, row, c) for c in range(bk // 8))
        assert got == [row * bk * 2 + 16 * c for c in range(bk // 8)]
    for k in range(bk):
        got = sorted(mofs(rows, k, c) for c in range(rows // 8))
        assert got == [k * rows * 2 + 16 * c for c in range(rows // 8)]


def dma_loader_map(rows, layout, nw, bk):
    """(lds byte offset, source row r, source k) of every chunk the LDS-direct
    loader fills, as the kernel's DmaLoader computes them."""
    instr = rows * bk * 2 // 1024
    per = instr // nw
    out = []
    for wave in range(nw):
        for i in range(per):
            for lane in range(64):
                q = (wave * per + i) * 64 + lane
                if layout == "k" and bk == 32:
                    row, p = q >> 2, q & 3
                    r, k = row, (p ^ ((row >> 2) & 3)) * 8
                elif layout == "k":
                    row, p = q >> 3, q & 7
                    r, k = row, (p ^ ((row ^ (row >> 3)) & 7)) * 8
                else:
                    nch = rows // 8
                    kk, p = q // nch, q % nch
                    k, r = kk, (p ^ mswz(nch, kk)) * 8
                out.append((q * 16, r, k))
    return out


@pytest.mark.parametrize("rows,nw", [(256, 8), (128, 8), (128, 4), (64, 4)])
@pytest.mark.parametrize("bk", [32, 64])
@pytest.mark.parametrize("layout", ["k", "mn"])
def test_gemm_loader_is_inverse_of_readers(rows, nw, bk, layout):
    if rows * bk * 2 // 1024 % nw:
        pytest.skip("tile instructions do not divide over the waves (not instantiated)")
    m = dma_loader_map(rows, layout, nw, bk)
    assert sorted(o for o, _, _ in m) == list(range(0, rows * bk * 2, 16))
    for off, r, k in m:
        assert k % 8 == 0 if layout == "k" else r % 8 == 0
        expect = kofs(bk, r, k // 8) if layout == "k" else mofs(rows, k, r // 8)
        assert off == expect, (off, r, k)


# ----------------------------------------------------- attention row-major tiles

def aswz(d, r):
    if d == 128:
        return ((r & 3) << 2) | ((r >> 2) & 3)
    return (((r >> 1) & 1) << 2) | ((r >> 2) & 3)


def tile_off(d, r, c):
    return r * d * 2 + ((c ^ aswz(d, r)) << 4)


def row_frag_addrs(d, r0, kk):
    return [tile_off(d, r0 + (lane & 31), kk * 2 + (lane >> 5)) for lane in range(64)]


def tr_frag_addrs(d, r0, dt, jj, half):
    out = []
    for lane in range(64):
        g4, R, h = lane >> 4, lane & 15, lane >> 5
        col = 32 * dt + 16 * (g4 & 1) + 4 * (R & 3)
        row = r0 + 16 * jj + 4 * h + 8 * half + (R >> 2)
        out.append(tile_off(d, row, col >> 3) + (col & 7) * 2)
    return out


@pytest.mark.parametrize("d", [64, 128])
def test_attention_tile_reads_conflict_free(d):
    rows = 64     # K/V blocks of 64 keys; Q and dO tiles of 32 rows use rows 0..31 of the same map
    for r0, kk in itertools.product(range(0, rows, 32), range(d // 16)):
        assert conflict_free(row_frag_addrs(d, r0, kk), 16, 16), (r0, kk)
    for r0, dt, jj, half in itertools.product(range(0, rows, 32), range(d // 32), range(2), range(2)):
        assert conflict_free(tr_frag_addrs(d, r0, dt, jj, half), 8, 32), (r0, dt, jj, half)


@pytest.mark.parametrize("d", [64, 128])
def test_attention_swizzle_bijection_and_loader_inverse(d):
    for r in range(64):
        assert sorted(tile_off(d, r, c) for c in range(d // 8)) == [r * d * 2 + 16 * c for c in range(d // 8)]
    # the loader: lane `lane` of instruction i fills LDS bytes o = 1024 i + 16 lane with
    # logical chunk pos ^ swz(r) of row r, where (r, pos) is o's place in the row-major tile
    for i in range(64 * d * 2 // 1024):
        for lane in range(64):
            o = i * 1024 + 16 * lane
            r, pos = o // (2 * d), (o % (2 * d)) >> 4
            c = pos ^ aswz(d, r)
            assert tile_off(d, r, c) == o


def test_unswizzled_attention_tile_would_conflict():
    """Without the swizzle, 256-byte rows put every row's chunk c on the same
    banks: the 16 lanes of a 128-bit pass collide."""
    plain = [r * 256 + 16 * ((lane >> 5)) for lane, r in zip(range(64), [(l & 31) for l in range(64)])]
    assert not conflict_free(plain, 16, 16)
