"""CPU model of the tiled GEMM's LDS placement (csrc/gemm_bf16.hip, tile_body).

Two operand forms are staged in LDS by buffer loads with the LDS flag (lane l
of a load instruction writes its 16 bytes at the instruction's base + 16 l):

* K-contiguous rows (weights [out][in], gathered token rows): 128-byte rows of
  one 64-deep K step, the 16-byte chunk XOR-swizzled by (row / 2) % 8; read
  with 16-byte reads, lane l taking row l % 32 and K 8 (l / 32) .. + 7 of a
  16-deep sub-step -- the operand layout of v_mfma_f32_32x32x16_bf16.
* K-row tiles ([K][columns], for the backward's products): rows of BX
  columns, the 16-byte chunk XOR-swizzled by 4 (row % 4); read with the
  transposing read ds_read_b64_tr_b16, whose lane layout was measured on the
  GPU: in each group of 16 lanes, lanes 4r .. 4r + 3 point at 4 consecutive
  bf16 each (16 values of "row" r), and result lane j receives the j-th value
  of each of the 4 rows.

The model fills a tagged LDS image exactly as the loader's address arithmetic
says, then evaluates every fragment read and checks that each lane receives
the (row, K) elements the MFMA expects, that every address stays inside the
stage, and that the reads of one bank sweep hit distinct banks (64 banks of
4 bytes).
"""
import pytest

ROW_BYTES = 128          # one K step of a K-contiguous row (64 bf16)
CH = 8                   # 16-byte chunks per row
RPB = 2                  # rows per 256-byte bank sweep
ROWS_LD = 8              # rows per 1 KB load instruction
BANKS = 64


def bank(addr):
    return (addr // 4) % BANKS


# ---- K-contiguous operand ---------------------------------------------------
def fill_kcontig(rows_total, nwaves, row_of_load):
    """LDS image {byte address -> (tile row, K element)} of one operand tile
    of rows_total rows, filled by nwaves waves; row_of_load(wid, i) is the
    first LDS row of load i of wave wid."""
    lds = {}
    loads = rows_total * ROW_BYTES // 1024 // nwaves
    for wid in range(nwaves):
        for i in range(loads):
            base = row_of_load(wid, i) * ROW_BYTES
            for lane in range(64):
                r = row_of_load(wid, i) + lane // CH
                pc = lane % CH
                c = pc ^ ((r // RPB) % CH)           # logical chunk this lane fetches
                addr = base + 16 * lane
                assert addr == r * ROW_BYTES + pc * 16
                for e in range(8):
                    a = addr + 2 * e
                    assert a not in lds, "two lanes write one LDS element"
                    lds[a] = (r, 8 * c + e)
    assert len(lds) == rows_total * 64
    return lds


@pytest.mark.parametrize("BM,WM,nwaves", [(256, 2, 4), (128, 1, 4), (64, 1, 4), (256, 2, 8)])
def test_kcontig_reads_give_mfma_layout(BM, WM, nwaves):
    loads = BM * ROW_BYTES // 1024 // nwaves
    lds = fill_kcontig(BM, nwaves, lambda wid, i: (wid * loads + i) * ROWS_LD)
    WTM = BM // WM
    TM = WTM // 32
    for wm in range(WM):
        for kk in range(4):
            for i in range(TM):
                addrs = []
                for lane in range(64):
                    l32, khalf = lane & 31, lane >> 5
                    sw = (l32 // RPB) % CH
                    kofs = ((kk * 2 + khalf) ^ sw) << 4
                    addr = (wm * WTM + l32) * ROW_BYTES + kofs + i * 32 * ROW_BYTES
                    assert 0 <= addr and addr + 16 <= BM * ROW_BYTES
                    got = [lds[addr + 2 * e] for e in range(8)]
                    row = wm * WTM + 32 * i + l32
                    want = [(row, 16 * kk + 8 * khalf + e) for e in range(8)]
                    assert got == want, (wm, kk, i, lane)
                    addrs.append(addr)
                # 16 consecutive lanes (one 256-byte sweep) hit 64 distinct banks
                for g in range(4):
                    bk = {bank(a + 4 * w) for a in addrs[16 * g:16 * g + 16] for w in range(4)}
                    assert len(bk) == BANKS, (wm, kk, i, g)


def test_gate_up_b_tile_halves():
    """Gate/up's B tile: loads i < B_LD / 2 fill W1 rows 0..127, the others
    the matching W3 rows 128..255 (same output columns)."""
    BN, nwaves = 256, 4
    B_LD = BN * ROW_BYTES // 1024 // nwaves
    H = B_LD // 2

    def b_lrow(wid, i):
        return (0 if i < H else BN // 2) + (wid * H + (i if i < H else i - H)) * ROWS_LD

    lds = fill_kcontig(BN, nwaves, b_lrow)
    rows = sorted({r for (r, _) in lds.values()})
    assert rows == list(range(BN))
    # column of each B row: W1 half and W3 half map to the same 128 columns
    col = [r - BN // 2 if r >= BN // 2 else r for r in rows]
    assert sorted(col[:128]) == sorted(col[128:]) == list(range(128))


# ---- K-row operand (transposing read) ---------------------------------------
def fill_krow(BX, KD, nwaves):
    """LDS image of a [KD][BX] K-row tile: {address -> (K row, column)}."""
    pitch = 2 * BX
    cpr = BX // 8                  # 16-byte chunks per K row
    rpi = 64 // cpr                # K rows per load instruction
    loads = BX * KD * 2 // 1024 // nwaves
    assert loads * 1024 * nwaves == BX * KD * 2
    lds = {}
    for wid in range(nwaves):
        for i in range(loads):
            base = (wid * loads + i) * 1024
            for lane in range(64):
                kr = (wid * loads + i) * rpi + lane // cpr
                c = (lane % cpr) ^ (4 * (kr & 3))
                addr = base + 16 * lane
                assert addr == kr * pitch + (lane % cpr) * 16
                assert kr < KD
                for e in range(8):
                    a = addr + 2 * e
                    assert a not in lds
                    lds[a] = (kr, 8 * c + e)
    assert len(lds) == BX * KD
    return lds


def kr_off(lane, c0, f, pitch):
    g, i16 = lane >> 4, lane & 15
    row = 8 * (g >> 1) + (i16 >> 2)
    chunk = ((c0 + 32 * f) >> 3) + 2 * (g & 1) + ((i16 & 3) >> 1)
    return row * pitch + ((chunk ^ (4 * (row & 3))) << 4) + (i16 & 1) * 8


def read_tr(lds, addrs):
    """ds_read_b64_tr_b16 on per-lane addresses: lane j of each 16-lane group
    gets value j of rows r = 0..3 of its group (row r = the 16 values the
    lanes 4r..4r+3 point at, in lane order)."""
    out = []
    for lane in range(64):
        g0, j = lane & ~15, lane & 15
        vals = []
        for r in range(4):
            row16 = []
            for q in range(4):
                a = addrs[g0 + 4 * r + q]
                row16 += [lds[a + 2 * e] for e in range(4)]
            vals.append(row16[j])
        out.append(vals)
    return out


@pytest.mark.parametrize("BX,WX,KD,nwaves",
                         [(256, 2, 64, 8), (256, 4, 64, 8), (512, 8, 64, 8), (128, 1, 64, 8),
                          (128, 1, 32, 4), (256, 4, 32, 4)])
def test_krow_transposing_reads_give_mfma_layout(BX, WX, KD, nwaves):
    """WX waves side by side along the tile's columns (wave tile BX / WX
    columns, 32-column fragments f)."""
    pitch = 2 * BX
    lds = fill_krow(BX, KD, nwaves)
    WT = BX // WX
    for w in range(WX):
        c0 = w * WT
        for f in range(WT // 32):
            for kk in range(KD // 16):
                lo = [kr_off(l, c0, f, pitch) + kk * 16 * pitch for l in range(64)]
                hi = [a + 4 * pitch for a in lo]
                for addrs in (lo, hi):
                    for a in addrs:
                        assert 0 <= a and a + 8 <= BX * KD * 2
                    # each half wave reads 256 bytes spread over all 64 banks
                    for h in range(2):
                        bk = {bank(a + 4 * u) for a in addrs[32 * h:32 * h + 32] for u in range(2)}
                        assert len(bk) == BANKS, (BX, w, f, kk, h)
                v_lo, v_hi = read_tr(lds, lo), read_tr(lds, hi)
                for lane in range(64):
                    col = c0 + 32 * f + (lane % 32)
                    k0 = 16 * kk + 8 * (lane // 32)
                    got = v_lo[lane] + v_hi[lane]
                    want = [(k0 + e, col) for e in range(8)]
                    assert got == want, (BX, w, f, kk, lane, got[:2], want[:2])


def test_krow_tiles_need_sixteen_chunks_per_row():
    """The swizzle XORs the chunk index with 4 (row % 4), up to 12: a K-row
    tile of 64 columns (8 chunks) would fetch chunks past its row, which is
    why the kernel only builds K-row tiles of >= 128 columns (a static_assert
    in tile_body)."""
    lds = fill_krow(64, 64, 8)
    assert max(col for (_, col) in lds.values()) >= 64
    src = open(__file__.replace("tests/test_lds_placement.py",
                                "sparse_mixture_experts_14_amd/csrc/gemm_bf16.hip")).read()
    assert "(!AKR || BM >= 128) && (!BKR || BN >= 128)" in src
