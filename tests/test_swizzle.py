"""CPU pins of the LDS swizzle maps ("Optimizing Blackwell matrix multiplication in Mojo (part 2)",
section "Kernel 3: Swizzling" and its appendix: XOR row bits into the 16-byte-chunk bits of an LDS address so
that the rows one wave instruction touches fall in different banks).

The maps come from the kernels' own header functions, printed on the host by tests/swizzle_dump.cpp.  The
access patterns are those of the kernels' LDS instructions on gfx950, whose LDS has 64 banks of 4 bytes
(256 bytes per clock): a ds_read_b128 / ds_write_b128 is served in four passes of 16 consecutive lanes, a
ds_read_b64_tr_b16 / ds_write_b64 in two passes of 32.  A pass is conflict-free when no bank is addressed
twice; the count below is the largest number of accesses any one bank receives in any pass.
"""
import collections
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
DUMP = os.path.join(ROOT, "tests", "swizzle_dump")
BANKS, BANK_BYTES = 64, 4


@pytest.fixture(scope="module")
def maps():
    if not os.path.exists(DUMP):
        from dense_tiled_gemm_amd import build

        build.build_swizzle_dump()
    out = subprocess.run([DUMP], capture_output=True, text=True, check=True, timeout=60).stdout
    swz, kouter, epi = {}, {}, {}
    for line in out.splitlines():
        f = line.split()
        if f[0] == "swz":
            swz[(int(f[1]), int(f[2]), int(f[3]))] = int(f[4])
        elif f[0] == "kouter":
            kouter[int(f[1])] = int(f[2])
        elif f[0] == "epi":
            epi[(int(f[1]), int(f[2]), int(f[3]))] = int(f[4])
    return swz, kouter, epi


def worst_bank(passes):
    """passes: lists of (byte address, bytes) accesses; the largest per-bank count over all passes."""
    worst = 0
    for acc in passes:
        count = collections.Counter()
        for addr, nbytes in acc:
            assert addr % 4 == 0 and nbytes % 4 == 0
            for w in range(nbytes // 4):
                count[(addr // BANK_BYTES + w) % BANKS] += 1
        worst = max(worst, max(count.values()))
    return worst


def split(lanes, per_pass):
    return [lanes[i:i + per_pass] for i in range(0, len(lanes), per_pass)]


@pytest.mark.parametrize("cpr", [16, 8, 4])
@pytest.mark.parametrize("swz_kind", [0, 1, 2])
def test_row_swizzle_is_a_bijection_on_each_window(maps, cpr, swz_kind):
    swz, _, _ = maps
    for row in range(256):
        s = swz[(cpr, swz_kind, row)]
        assert 0 <= s < cpr
        assert sorted(c ^ s for c in range(cpr)) == list(range(cpr))
    # the DMA write: one wave instruction fills 1 KiB of LDS, lane L at physical chunk L % cpr of row L // cpr
    # (plus the block's first row); it fetches logical chunk (L % cpr) ^ swz(row), so every logical chunk of
    # every row arrives exactly once, and the LDS writes themselves are contiguous
    rows_per_block = 64 // cpr
    for first in range(0, 256, rows_per_block):
        got = {(first + lane // cpr, (lane % cpr) ^ swz[(cpr, swz_kind, first + lane // cpr)]) for lane in range(64)}
        assert got == {(first + r, c) for r in range(rows_per_block) for c in range(cpr)}
        writes = [((first + lane // cpr) * cpr * 16 + (lane % cpr) * 16, 16) for lane in range(64)]
        assert worst_bank(split(writes, 16)) == 1


def mfma_read_passes(swz, cpr, swz_kind, mf, ks, block):
    """ds_read_b128 of an MFMA operand: lane l reads row block + l % mf, logical chunk (16 / mf... ) of k-substep
    ks: 16x16x32 (mf 16) chunk 4 ks + l // 16, 32x32x16 (mf 32) chunk 2 ks + l // 32 (128-byte rows); 64-byte
    rows (cpr 4) hold one substep of the 16x16x32 form: chunk 2 ks + l // 16 within a pair of substeps."""
    lanes = []
    for lane in range(64):
        row = block + lane % mf
        if cpr == 16:  # 256-byte rows (16x16x32 only): four substeps per row
            chunk = 4 * ks + lane // 16
        elif cpr == 8:
            chunk = (4 * ks + lane // 16) if mf == 16 else (2 * ks + lane // 32)
        else:
            chunk = (2 * (ks % 2) + lane // 16) % 4 if mf == 16 else (ks % 2) * 2 + lane // 32
        phys = chunk ^ swz[(cpr, swz_kind, row)]
        lanes.append((row * cpr * 16 + phys * 16, 16))
    return split(lanes, 16)


@pytest.mark.parametrize("mf", [16, 32])
def test_mfma_operand_reads(maps, mf):
    swz, _, _ = maps
    worst = {}
    for kind in (0, 1, 2):
        worst[kind] = max(worst_bank(mfma_read_passes(swz, 8, kind, mf, ks, block))
                          for ks in range(2 if mf == 16 else 4) for block in range(0, 256, mf))
    # the production swizzle (row bits 1..3, for 64 banks) is conflict-free; the 32-bank form (row bits 0..2)
    # leaves two-way conflicts; without a swizzle the 16 rows of a pass share two 16-byte bank groups (8-way)
    assert worst[2] == 1
    assert worst[1] == 2
    assert worst[0] == 8


def test_mfma_operand_reads_256_byte_rows(maps):
    """256-byte rows (the thin split tiles): each row spans all 64 banks, so without a swizzle the 16 rows of a pass
    all read the same 16-byte bank group; XORing row bits 0..3 spreads them over the 16 groups."""
    swz, _, _ = maps
    worst = {kind: max(worst_bank(mfma_read_passes(swz, 16, kind, 16, ks, block))
                       for ks in range(4) for block in range(0, 256, 16)) for kind in (0, 1, 2)}
    assert worst[2] == 1 and worst[1] == 2 and worst[0] == 16


def test_mfma_operand_reads_64_byte_rows(maps):
    swz, _, _ = maps
    worst = {kind: max(worst_bank(mfma_read_passes(swz, 4, kind, 16, ks, block))
                       for ks in range(2) for block in range(0, 256, 16)) for kind in (0, 1, 2)}
    assert worst[2] == 1 and worst[1] == 2 and worst[0] == 4


@pytest.mark.parametrize("bx", [128, 256])
def test_kouter_pair_swizzle_and_transpose_reads(maps, bx):
    _, kouter, _ = maps
    cr = 2 * bx // 16  # 16-byte chunks per K-outer row (bx 16-bit elements)
    for row in range(64):
        s = kouter[row]
        assert s % 2 == 0 and 0 <= s < cr  # whole pairs: the two 8-byte halves of a read stay together
        assert sorted(c ^ s for c in range(cr)) == list(range(cr))
    # ds_read_b64_tr_b16 of the 16 rows x 32 bytes behind one 16x16x32 operand fragment: lane = 16 g4 + 4 e + a,
    # rows r0 = 32 ks + 8 g4 + e (and r0 + 4 for the second read), column chunk (x / 8 + a // 2), 8-byte half a % 2
    rowb = 2 * bx
    for ks in range(2):
        for x in range(0, bx, 16):
            for h in (0, 4):
                lanes = []
                for lane in range(64):
                    g4, q = lane >> 4, lane & 15
                    e, a = q >> 2, q & 3
                    r0 = 32 * ks + 8 * g4 + e + h
                    c = (x >> 3) + (a >> 1)
                    lanes.append((r0 * rowb + (c ^ kouter[r0]) * 16 + (a & 1) * 8, 8))
                assert worst_bank(split(lanes, 32)) == 1, (bx, ks, x, h)
    # without the swizzle the same reads conflict
    plain = max(worst_bank(split([((32 * ks + 8 * (l >> 4) + ((l & 15) >> 2)) * rowb + ((x >> 3) + ((l & 3) >> 1)) * 16
                                   + (l & 1) * 8, 8) for l in range(64)], 32))
                for ks in range(2) for x in range(0, bx, 16))
    assert plain > 1


@pytest.mark.parametrize("osz,bn", [(4, 256), (4, 128), (2, 256), (2, 128), (2, 64), (4, 64), (4, 96), (2, 96)])
def test_epilogue_park_and_copy(maps, osz, bn):
    """The output tile parked in LDS: each wave writes its 16x16 accumulator blocks (lane l: row l % 16, 4
    columns from 4 (l // 16)) as 16 bytes (fp32) or 8 bytes (16-bit) per lane; then the workgroup copies whole
    rows, thread t reading chunk t % cpr of row t // cpr."""
    _, _, epi = maps
    rowb = bn * osz
    cpr = rowb // 16
    for row in range(64):
        assert sorted(epi[(cpr, row, c)] for c in range(cpr)) == list(range(cpr))
    per_pass = 16 if osz == 4 else 32
    worst_park = 0
    for rbase in range(0, 64, 16):
        for cbase in range(0, bn, 16):
            lanes = []
            for lane in range(64):
                r = rbase + lane % 16
                col = cbase + 4 * (lane // 16)
                c = col * osz // 16
                off = 8 * ((col >> 2) & 1) if osz == 2 else 0
                lanes.append((r * rowb + epi[(cpr, r, c)] * 16 + off, 16 if osz == 4 else 8))
            worst_park = max(worst_park, worst_bank(split(lanes, per_pass)))
    assert worst_park == 1
    reads = [((t // cpr) * rowb + epi[(cpr, t // cpr, t % cpr)] * 16, 16) for t in range(64 * cpr) if t // cpr < 64]
    assert worst_bank(split(reads, 16)) == 1
