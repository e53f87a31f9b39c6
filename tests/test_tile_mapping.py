"""CPU mirror of the tiled grouped GEMM's block -> tile mapping.

The kernel (csrc/gemm_bf16.hip, gemm_bf16_kernel) finds its tile on the
device from the expert offsets: square 256-row tiles, a wide (<= 128 rows) or
narrow (<= 64 rows) tail tile per expert, row groups and column pairs, the
per-XCD order, and -- for the down projection and the backward's dx product --
the K splits of the last round's tiles only (rows from R0 on, Sr splits, the
partial sums past the first packed after buffer 0).  This file restates that
index arithmetic in Python, step for step, and checks on many routings that:

* every output element is written exactly once per K split it needs: once,
  with the whole K range, below R0; Sr times, with K ranges that partition
  the whole range, from R0 on;
* every tile lies inside one expert, within the row limits of its shape;
* split tiles start at or after R0 and whole-K tiles end at or before it;
* the partial-sum rows stay inside the workspace's `splits` buffers of A rows
  and no two (split, row) pairs share one;
* the launch grid (the host's upper bound) reaches every real tile, and each
  block's expert search stays inside the n experts;
* the whole-K tiles are spread evenly over the 8 XCDs (block b on XCD b % 8).

The mirror is a line-by-line restatement of the kernel's integer logic, so it
checks that logic against these properties, not against itself.
"""
import math

import numpy as np
import pytest

SQ_BM = 256
WD_BM = 128
NARROW_BM = 64
BK = 64


def cdiv(a, b):
    return -(-a // b)


class Mapping:
    """The tile mapping of one launch: gate/up (splits 1, no remainder
    split) or the down projection (cus > 0: the last round split)."""

    def __init__(self, offsets, N, Kdim, gateup, splits=1, cus=0, GM=8, down_wide_max=128):
        self.off = [int(v) for v in offsets]
        self.n = len(offsets) - 1
        self.N, self.Kdim, self.gateup = N, Kdim, gateup
        self.splits, self.cus, self.GM = splits, cus, GM
        self.BNO_S = 128 if gateup else 256          # output columns of a square tile
        self.ntn_s = cdiv(N, self.BNO_S)
        self.npair = (self.ntn_s + 1) // 2
        self.WIDE_MAX = WD_BM if gateup else down_wide_max
        self.tiles = sum(self.expert_tiles(self.off[q + 1] - self.off[q])[0]
                         for q in range(self.n))
        self.A = self.off[self.n]
        self._remainder_split()

    def expert_tiles(self, m):
        rem = m % SQ_BM
        nsq = m // SQ_BM + (1 if rem > self.WIDE_MAX else 0)
        nwide = 1 if 0 < rem <= self.WIDE_MAX else 0
        return nsq * self.ntn_s + nwide * self.npair, nsq, nwide

    def _remainder_split(self):
        off, n = self.off, self.n
        self.R0, self.Sr, self.Trem = off[n], 1, 0
        if self.cus <= 0:
            return
        R0, Sr, Trem = off[n], 1, 0
        r = self.tiles % self.cus
        if r > 0 and self.splits > 1:
            q = n - 1
            while q >= 0 and Trem < r:
                _, nsq_q, nw_q = self.expert_tiles(off[q + 1] - off[q])
                s0 = off[q]
                if nw_q:
                    Trem += self.npair
                    R0 = s0 + nsq_q * SQ_BM
                if Trem >= r:
                    break
                take = min(cdiv(r - Trem, self.ntn_s), nsq_q)
                Trem += take * self.ntn_s
                if take > 0:
                    R0 = s0 + (nsq_q - take) * SQ_BM
                q -= 1
            rows_rem = off[n] - R0
            fit = 1 + (self.splits - 1) * off[n] // max(1, rows_rem)
            nk = cdiv(self.Kdim, BK)
            Sr = min(min(min(self.cus // Trem, nk), 16), fit)
            if Sr < 2:
                Sr, R0, Trem = 1, off[n], 0
        self.R0, self.Sr, self.Trem = R0, Sr, Trem

    def grid(self, A_rows):
        """The launch's block count (launch_tiled's upper bound)."""
        mslots = A_rows // SQ_BM + self.n
        ntn = cdiv(self.N, self.BNO_S)
        if self.cus > 0:
            return cdiv(mslots * ntn, 8) * 8 + cdiv(self.cus, 8) * 8
        return cdiv(mslots * ntn * self.splits, 8) * 8

    def block(self, b):
        """Tile of block b: None (block exits) or a dict."""
        off, n = self.off, self.n
        lo, hi, ks, nsplit, part0 = off[0], off[n], 0, self.splits, 0
        if self.cus > 0:
            Tdp = self.tiles - self.Trem
            per_xcd = cdiv(Tdp, 8)
            if b < 8 * per_xcd:
                L = (b & 7) * per_xcd + (b >> 3)
                if L >= Tdp:
                    return None
                hi, nsplit = self.R0, 1
            else:
                u = b - 8 * per_xcd
                if u >= self.Trem * self.Sr:
                    return None
                ks = u // self.Trem
                L = u - ks * self.Trem
                lo, nsplit = self.R0, self.Sr
                if ks > 0:
                    part0 = off[n] + (ks - 1) * (off[n] - self.R0) - self.R0
        else:
            per_xcd = cdiv(self.tiles * self.splits, 8)
            jx = b >> 3
            L0 = (b & 7) * per_xcd + jx
            if jx >= per_xcd or L0 >= self.tiles * self.splits:
                return None
            ks = L0 // self.tiles
            L = L0 - ks * self.tiles
            part0 = self.A * ks
        e = 0
        while True:
            assert e < n, f"block {b}: expert search ran past the last expert"
            start, end = max(off[e], lo), min(off[e + 1], hi)
            cnt, nsq, nwide = self.expert_tiles(max(0, end - start))
            if L < cnt:
                break
            L -= cnt
            e += 1
        GM = self.GM
        ngroups = max(1, cdiv(nsq, GM))
        g = min(L // (GM * self.ntn_s), ngroups - 1)
        L -= g * GM * self.ntn_s
        gm = min(GM, nsq - g * GM)
        w = nwide if g == ngroups - 1 else 0
        c = min(L // (2 * gm + w), self.npair - 1)
        L -= c * (2 * gm + w)
        ncol = min(2, self.ntn_s - 2 * c)
        nk_all = cdiv(self.Kdim, BK)
        per_split = cdiv(nk_all, nsplit)
        k_begin = min(nk_all, ks * per_split)
        k_end = min(nk_all, k_begin + per_split)
        if L < gm * ncol:
            mt = g * GM + L % gm
            row0 = start + mt * SQ_BM
            rows = min(SQ_BM, end - row0)
            n0 = (2 * c + L // gm) * self.BNO_S
            kind, width = "square", self.BNO_S
        else:
            assert w == 1 and L == gm * ncol, f"block {b}: no tile left in its column pair"
            row0 = start + nsq * SQ_BM
            rows = end - row0
            n0 = 2 * c * self.BNO_S
            kind = "narrow" if rows <= NARROW_BM else "wide"
            width = 2 * self.BNO_S
        return dict(e=e, row0=row0, rows=rows, n0=n0, width=width, kind=kind, ks=ks,
                    nsplit=nsplit, k_begin=k_begin, k_end=k_end, part0=part0, lo=lo, hi=hi)


def check_mapping(offsets, N, Kdim, gateup, splits=1, cus=0, GM=8):
    m = Mapping(offsets, N, Kdim, gateup, splits, cus, GM)
    A, n = m.A, m.n
    CU = 128  # column unit: every tile edge is a multiple of 128 output columns
    ncu = cdiv(N, CU)
    nk = cdiv(Kdim, BK)
    # per (row, column unit): the K steps covered by each split index
    cover = {}
    whole = np.zeros((A, ncu), np.int32)
    part_rows = {}
    nblocks = m.grid(A)
    found = 0
    xcd = np.zeros(8, np.int64)
    for b in range(nblocks):
        t = m.block(b)
        if t is None:
            continue
        found += 1
        e, r0, rows = t["e"], t["row0"], t["rows"]
        assert rows >= 1, t
        assert m.off[e] <= r0 and r0 + rows <= m.off[e + 1], ("tile outside its expert", t)
        lim = {"square": SQ_BM, "wide": WD_BM, "narrow": NARROW_BM}[t["kind"]]
        assert rows <= lim, t
        assert t["n0"] < N and t["n0"] % CU == 0, t
        c0, c1 = t["n0"] // CU, min(cdiv(t["n0"] + t["width"], CU), ncu)
        if t["nsplit"] == 1:
            assert t["k_begin"] == 0 and t["k_end"] == nk, t
            assert r0 + rows <= m.R0, ("whole-K tile past R0", t)
            whole[r0:r0 + rows, c0:c1] += 1
            xcd[b % 8] += 1
        else:
            assert r0 >= m.R0, ("split tile below R0", t)
            for p in range(r0, r0 + rows):
                for cu in range(c0, c1):
                    cover.setdefault((p, cu), []).append((t["ks"], t["k_begin"], t["k_end"]))
        if t["ks"] > 0:
            for p in range(r0, r0 + rows):
                dst = t["part0"] + p
                assert A <= dst < splits * A, ("partial row outside the workspace", t, dst)
                prev = part_rows.setdefault(dst, (t["ks"], p))
                assert prev == (t["ks"], p), ("two partial sums share a row", prev, t)
    assert found == (m.tiles - m.Trem) + m.Trem * m.Sr, "grid misses real tiles"
    # rows below R0: exactly one whole-K tile per column unit; from R0 on, none
    assert (whole[:m.R0] == 1).all(), "rows below R0 not covered exactly once"
    assert (whole[m.R0:] == 0).all()
    for p in range(m.R0, A):
        for cu in range(ncu):
            got = sorted(cover.get((p, cu), []))
            assert [s for s, _, _ in got] == list(range(m.Sr)), (p, cu, got)
            ks = [(a, z) for _, a, z in got]
            assert ks[0][0] == 0 and ks[-1][1] == nk, (p, cu, ks)
            assert all(ks[i][1] == ks[i + 1][0] for i in range(len(ks) - 1)), (p, cu, ks)
    if m.cus == 0:
        assert not cover
    # whole-K tiles: a contiguous share per XCD, all but the last share full
    Tdp = m.tiles - m.Trem
    per = cdiv(Tdp, 8)
    assert xcd.sum() == Tdp and xcd.max() <= per
    assert (np.sort(xcd)[::-1][:Tdp // per if per else 0] == per).all()
    return m


def routing_offsets(rng, A, n, kind):
    if kind == "uniform":
        counts = rng.multinomial(A, np.full(n, 1.0 / n))
    elif kind == "skew":
        p = np.array([0.48] + [0.095] * 5 + [0.0175, 0.0175])[:n]
        counts = rng.multinomial(A, p / p.sum())
    elif kind == "sparse":  # some experts empty, some tiny
        w = rng.random(n) * (rng.random(n) < 0.6)
        w[rng.integers(n)] += 0.1
        counts = rng.multinomial(A, w / w.sum())
    else:  # tails of every size around the tile boundaries
        counts = rng.integers(0, 4, n) * SQ_BM + rng.choice([0, 1, 63, 64, 65, 127, 128, 129,
                                                              255], n)
    return np.concatenate([[0], np.cumsum(counts)])


@pytest.mark.parametrize("kind", ["uniform", "skew", "sparse", "edges"])
def test_down_projection_mapping_random_routings(kind):
    rng = np.random.default_rng(["uniform", "skew", "sparse", "edges"].index(kind))
    for trial in range(25):
        n = 8 if kind == "skew" else int(rng.choice([1, 3, 8, 13, 64]))
        A = int(rng.choice([1, 40, 300, 700, 2048, 4096, 8192]))
        off = routing_offsets(rng, A, n, kind)
        N = int(rng.choice([256, 264, 1024, 4096]))
        Kdim = int(rng.choice([64, 200, 1024, 14336]))
        cus = int(rng.choice([256, 304, 80]))
        check_mapping(off, N, Kdim, gateup=False, splits=4, cus=cus)


@pytest.mark.parametrize("kind", ["uniform", "skew", "sparse", "edges"])
def test_gate_up_mapping_random_routings(kind):
    rng = np.random.default_rng(10 + ["uniform", "skew", "sparse", "edges"].index(kind))
    for trial in range(25):
        n = 8 if kind == "skew" else int(rng.choice([1, 3, 8, 13, 64]))
        A = int(rng.choice([1, 40, 300, 700, 2048, 4096]))
        off = routing_offsets(rng, A, n, kind)
        N = int(rng.choice([128, 136, 2048, 14336]))
        check_mapping(off, N, 4096, gateup=True)


def test_workload_shapes():
    """The benchmark's shapes: prefill (A = 8192, ~1024 rows per expert), the
    stack layer (A = 4096), the skewed routing (A = 32768, one expert with
    ~48%); a left-over partial round of the down projection is always split."""
    rng = np.random.default_rng(3)
    for A, kind in ((8192, "uniform"), (4096, "uniform"), (32768, "skew")):
        off = routing_offsets(rng, A, 8, kind)
        check_mapping(off, 14336, 4096, gateup=True)
        m = check_mapping(off, 4096, 14336, gateup=False, splits=4, cus=256)
        if m.tiles % 256:
            assert m.Sr >= 2 and m.Trem >= m.tiles % 256, (m.tiles, m.Trem, m.Sr)
        assert (m.Sr == 1) == (m.R0 == A)


def test_empty_and_single_expert():
    check_mapping([0, 0, 0, 0], 4096, 14336, gateup=False, splits=4, cus=256)
    check_mapping([0, 0, 5000, 5000], 4096, 14336, gateup=False, splits=4, cus=256)
    check_mapping([0, 0, 5000, 5000], 14336, 4096, gateup=True)
    check_mapping([0, 1], 256, 64, gateup=False, splits=4, cus=256)
