"""Host-side check of the LDS tile layouts of the bf16 attention kernel.

The kernel (`ra_kernels.hip`: `KvTile128`, `KvTileDma128` and the operand
reads of `attn_bf16_mfma`, and `BfTile` / `swz` in `ra_device.h`) places each
64-key K or V tile in LDS so that the two operand reads of the MFMAs are free
of bank conflicts. The formulas below restate the kernel's per-lane address
arithmetic (the dk/dv kernel of `ra_bwd.hip` stores its 32-row Q / dO tiles
in the same padded groups and reads them with the same formulas, which are
the half-tile-0 cases here); the tests enumerate every lane and step and check that

* each read lands on the key row and head dims the MFMA formulation needs
  (K operand: row `col` + 32 per half tile, chunk 2t + half; transposed V
  read: keys 4*(grp/2) + sl/4 (+16 per chunk, +8 for the second read), dims
  32*db + 16*(grp%2) + 4*(sl%4));
* the 16 lanes of a 16-byte K read and the 32 lanes of an 8-byte transposed
  read each touch all 64 four-byte banks exactly once;
* the DMA writes cover every (row, chunk) of the tile once and stay inside it,
  and every group of four DMA lanes reads 64 contiguous bytes of one row
  (padded layout only).
"""
import pytest

BANKS = 64          # gfx950 LDS: 64 banks of 4 bytes
D = 128
ROWB = 2 * D        # bytes per unpadded key row
CPR = D // 8        # 16-byte chunks per row


# ---- padded layout (d = 128, 8 waves) ------------------------------------
SEGP = 1040          # bytes per group of 4 rows (1 KiB + 64 bytes of padding)
TB_PAD = 16 * SEGP   # one 64-key tile
HALF_PAD = 8 * SEGP  # 32 keys


def pad_dma(seg, lane):
    """(LDS byte offset within the tile, row, chunk) written by DMA lane `lane` of group `seg`."""
    c = 4 * (lane >> 4) + (lane & 3)
    r4 = (lane >> 2) & 3
    return seg * SEGP + 16 * lane, 4 * seg + r4, c


def pad_k_read(lane, uh, t):
    col, half = lane & 31, lane >> 5
    kbase = (col >> 2) * SEGP + 16 * (4 * (col & 3) + half)
    return uh * HALF_PAD + kbase + 256 * (t >> 1) + 32 * (t & 1)


def pad_v_read(lane, uh, c, db, second):
    grp, sl = lane >> 4, lane & 15
    lowc = 2 * (grp & 1) + ((sl >> 1) & 1)
    vbase = (grp >> 1) * SEGP + 16 * (4 * (sl >> 2) + lowc) + 8 * (sl & 1)
    lo = uh * HALF_PAD + vbase + 4 * SEGP * c + 256 * db
    return lo + 2 * SEGP if second else lo


# ---- swizzled layout (other head sizes; checked here at d = 128) ---------
def swz(r):
    return ((r & 3) << 2) | ((r >> 2) & 3)


def swz_k_read(lane, uh, t):
    col, half = lane & 31, lane >> 5
    fr = swz(col) & (CPR - 1)
    return uh * 32 * ROWB + col * ROWB + (((2 * t + half) ^ fr) & (CPR - 1)) * 16


def swz_v_read(lane, uh, c, db, second):
    grp, sl = lane >> 4, lane & 15
    r = 4 * (grp >> 1) + (sl >> 2) + (8 if second else 0)
    ch = (4 * db + 2 * (grp & 1) + ((sl >> 1) & 1)) & (CPR - 1)
    return uh * 32 * ROWB + r * ROWB + ((ch ^ swz(r)) & (CPR - 1)) * 16 + 8 * (sl & 1) + c * 16 * ROWB


def swz_content():
    # chunk c of row r at position c ^ swz(r)
    return {r * ROWB + ((c ^ swz(r)) & (CPR - 1)) * 16: (r, c) for r in range(64) for c in range(CPR)}


def pad_content():
    out = {}
    for seg in range(16):
        for lane in range(64):
            off, row, ch = pad_dma(seg, lane)
            assert off not in out
            out[off] = (row, ch)
    return out


def _banks(addrs, nbytes):
    return [((a // 4) + w) % BANKS for a in addrs for w in range(nbytes // 4)]


LAYOUTS = {
    "padded": (pad_content, pad_k_read, pad_v_read, TB_PAD),
    "swizzled": (swz_content, swz_k_read, swz_v_read, 64 * ROWB),
}


@pytest.mark.parametrize("name", sorted(LAYOUTS))
def test_k_operand_reads(name):
    content_fn, k_read, _, tb = LAYOUTS[name]
    content = content_fn()
    for uh in range(2):
        for t in range(D // 16):
            addrs = [k_read(lane, uh, t) for lane in range(64)]
            for lane, a in enumerate(addrs):
                assert 0 <= a and a + 16 <= tb
                assert content[a] == ((lane & 31) + 32 * uh, 2 * t + (lane >> 5)), (name, lane, uh, t)
            for ph in range(4):  # 16 lanes x 16 bytes per bank cycle
                assert sorted(_banks(addrs[16 * ph:16 * ph + 16], 16)) == list(range(BANKS)), (name, uh, t, ph)


@pytest.mark.parametrize("name", sorted(LAYOUTS))
def test_transposed_v_reads(name):
    content_fn, _, v_read, tb = LAYOUTS[name]
    content = content_fn()
    for uh in range(2):
        for c in range(2):
            for db in range(D // 32):
                for second in (False, True):
                    addrs = [v_read(lane, uh, c, db, second) for lane in range(64)]
                    for lane, a in enumerate(addrs):
                        grp, sl = lane >> 4, lane & 15
                        assert 0 <= a and a + 8 <= tb
                        row, ch = content[a - a % 16]
                        want_row = 4 * (grp >> 1) + (sl >> 2) + 16 * c + 32 * uh + (8 if second else 0)
                        want_dim = 32 * db + 16 * (grp & 1) + 4 * (sl % 4)
                        assert (row, 8 * ch + (a % 16) // 2) == (want_row, want_dim), (name, lane)
                    for ph in range(2):  # 32 lanes x 8 bytes per bank cycle
                        assert sorted(_banks(addrs[32 * ph:32 * ph + 32], 8)) == list(range(BANKS))


def test_padded_dma_covers_tile_and_reads_rows_in_runs():
    content = pad_content()
    assert sorted(content.values()) == [(r, c) for r in range(64) for c in range(CPR)]
    assert max(content) + 16 <= TB_PAD
    for seg in range(16):
        for q in range(16):  # groups of four lanes: one row, four consecutive chunks
            cells = [pad_dma(seg, 4 * q + i)[1:] for i in range(4)]
            assert len({r for r, _ in cells}) == 1
            assert [c for _, c in cells] == list(range(cells[0][1], cells[0][1] + 4))


def test_padded_immediates_fit_the_ds_offset_field():
    # every per-step offset is added to one base register as a 16-bit immediate
    k_imm = max(HALF_PAD + 256 * (t >> 1) + 32 * (t & 1) for t in range(8))
    v_imm = HALF_PAD + 4 * SEGP + 2 * SEGP + 256 * 3
    assert k_imm < 65536 and v_imm < 65536
