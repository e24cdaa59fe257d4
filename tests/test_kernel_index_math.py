"""CPU checks of the pass-1 kernels' index arithmetic (no GPU needed).

The kernels' LDS layout and buffer-resource bounds are restated here in plain
Python from the kernels' own formulas and checked exhaustively on small plans
produced by the library's planner. bf16 matrix engine:

* the row stores and the transposing reads (ds_read_b64_tr_b16, whose lane
  layout was probed on MI355X: in each 16-lane group, output lane i element k
  comes from source lane 4k + i/4, element i mod 4) hand lane (g, m) of a wave
  the B operand V[8g + j][16t + m], j = 0..7;
* a lane's V and attn accesses are inside the buffer resource exactly when the
  row is inside the split (rows past it read as zero), the resources lie inside
  the tensors, every row of a split is consumed once per KV head, and every
  output is written once.

VALU engine: the same bounds, rows and outputs for its lane layout (row slots,
lane chunks, KV heads per tile, D-tiles, weight windows), in reuse and
per-head mode, for every V dtype.
"""
import numpy as np
import pytest

import gqa_reuse_attn_amd as ga

ENGINE_BF16 = 3


def _swz(PR, row):
    return ((row & 3) ^ (row >> 3)) & 3 if PR == 8 else ((row & 3) | ((row >> 3) << 2)) & (PR // 2 - 1)


@pytest.mark.parametrize("PR", [8, 16, 32])
def test_lds_transpose_layout(PR):
    RB, RPI, LPI, D = PR * 16, 64 // PR, PR // 2, PR * 8
    mem = {}
    for i in range(LPI):                       # row stores: load i, lane -> (row, 16-byte piece)
        for lane in range(64):
            prow, pp = lane // PR, lane % PR
            row = RPI * i + prow
            off = row * RB + 32 * ((pp >> 1) ^ _swz(PR, row)) + 16 * (pp & 1)
            assert 0 <= off and off + 16 <= 32 * RB
            for e in range(8):
                assert off + 2 * e not in mem
                mem[off + 2 * e] = (row, 8 * pp + e)
    assert len(mem) == 32 * D
    for t in range(D // 16):
        for h in range(2):
            addr = []
            for lane in range(64):                 # transposing reads: source addresses
                g = lane >> 4
                row = 8 * g + 4 * h + ((lane & 15) >> 2)
                addr.append(row * RB + 32 * (t ^ _swz(PR, row)) + 8 * (lane & 3))
            for lane in range(64):
                g, i = lane >> 4, lane & 15
                for k in range(4):
                    got = mem[addr[16 * g + 4 * k + i // 4] + 2 * (i % 4)]
                    assert got == (8 * g + 4 * h + k, 16 * t + i)
            # 512 bytes per read: at best two passes over 64 banks of 4 bytes
            banks = {}
            for a in addr:
                for w in (a // 4, a // 4 + 1):
                    banks.setdefault(w % 64, set()).add(w)
            assert max(len(v) for v in banks.values()) <= 2


@pytest.mark.parametrize("PR,NSET", [(8, 1), (8, 2), (16, 1), (16, 2), (32, 1)])
def test_attention_lds_reads(PR, NSET):
    """Fused attention in the bf16 matrix engine: with K rows stored like V rows,
    lane 16 g + n's 16-byte read for row 16 t2 + n and d-block kk returns
    K[row][32 kk + 8 g .. + 7]; the scores pass through the region as
    [16 NSET heads][32 rows] floats, inside the region, and each lane reads
    back head m + 16 s, rows 8 g .. 8 g + 7 of what the MFMA result layout
    wrote (register i of lane 16 g' + n': head 4 g' + i, row n')."""
    RB, RPI, LPI, D = PR * 16, 64 // PR, PR // 2, PR * 8
    mem = {}
    for i in range(LPI):
        for lane in range(64):
            prow, pp = lane // PR, lane % PR
            row = RPI * i + prow
            off = row * RB + 32 * ((pp >> 1) ^ _swz(PR, row)) + 16 * (pp & 1)
            for e in range(8):
                mem[off + 2 * e] = (row, 8 * pp + e)
    for t2 in range(2):
        for kk in range(D // 32):
            for lane in range(64):
                g, n = lane >> 4, lane & 15
                row, piece = 16 * t2 + n, 4 * kk + g
                off = row * RB + 32 * ((piece >> 1) ^ _swz(PR, row)) + 16 * (piece & 1)
                assert off % 16 == 0 and off + 16 <= 32 * RB
                assert [mem[off + 2 * e] for e in range(8)] == [(row, 32 * kk + 8 * g + e) for e in range(8)]
    # scores: written [head][32 rows], read back by (g, m)
    assert 16 * NSET * 32 * 4 <= 32 * RB, "the score tile fits in the wave's region"
    wrote = {}
    for s_ in range(NSET):
        for t2 in range(2):
            for lane in range(64):
                gp, npr = lane >> 4, lane & 15
                for i in range(4):
                    idx = (16 * s_ + 4 * gp + i) * 32 + 16 * t2 + npr
                    assert idx not in wrote
                    wrote[idx] = (16 * s_ + 4 * gp + i, 16 * t2 + npr)
    assert len(wrote) == 16 * NSET * 32
    for s_ in range(NSET):
        for lane in range(64):
            g, m = lane >> 4, lane & 15
            base = (16 * s_ + m) * 32 + 8 * g
            assert (base * 4) % 16 == 0
            assert [wrote[base + j] for j in range(8)] == [(16 * s_ + m, 8 * g + j) for j in range(8)]


def _remap(i, n):
    per, rem = n // 8, n % 8
    x, k = i % 8, i // 8
    return x * (per + 1) + k if x < rem else rem * (per + 1) + (x - rem) * per + k


def _check_plan(p, B, C, Hq, Hkv, D, es=2):
    """es: bytes of a V element (2: bf16; 1: fp8, loaded as 8-byte pieces of 8 values)."""
    assert p.engine == ENGINE_BF16 and p.vec_bytes == 8 * es
    PR, HT, NW = D // 8, p.kv_heads_per_tile, p.threads // 64
    assert NW in (4, 8) and NW % HT == 0 and (NW == 4 or not p.softmax or HT == 8)
    RPI, LPI, WPH = 64 // PR, PR // 2, NW // HT
    NSET = p.heads_per_tile // 16
    RSTEP, vrow, G = 32 * WPH, Hkv * D * es, Hq // Hkv
    GT, nsg, ns = 16 * NSET, p.subgroups, p.nsplit
    assert p.lanes_per_row == HT * D // 8 and p.row_slots == 32 * WPH
    lanes = np.arange(64)
    cnt = np.zeros((B, Hq, D), np.int64)
    scnt = np.zeros((ns, B, Hq), np.int64)          # fused softmax: split statistics written
    seen = {}                                       # rows each (b, KV head, head set) is streamed for, all splits
    nkvt = Hkv // HT
    for blk in range(p.grid):
        t = _remap(blk, p.grid)
        sg = t % nsg; t //= nsg
        kv = (t % nkvt) * HT; t //= nkvt
        s = t % ns; t //= ns
        b = t % B
        qf, nq = kv * G + sg * GT, min(GT, G - sg * GT)
        il = bool(p.interleave) and not p.page_size
        assert p.interleave in (0, 1) and not (p.interleave and p.page_size)
        if il:
            # interleaved: split s takes the steps s, s + ns, ... of RSTEP rows of the sequence
            assert p.rows_per_split == RSTEP and 2 <= ns <= -(-C // RSTEP)
            cb, ce = 0, C
        else:
            cb = s * p.rows_per_split
            ce = min(C, cb + p.rows_per_split)
        nrows = ce - cb
        assert nrows > 0
        if p.page_size:
            # paged V: the split's page list and every loaded row's entry in
            # it, including the pipeline's reloads past the split (clamped to
            # its last valid row), for full and shorter sequences
            P = p.page_size
            shift = P.bit_length() - 1
            for ln in {C, C // 2, cb + 1, cb}:
                nr = max(0, min(ce, ln) - cb)
                if nr == 0:
                    continue
                pg0 = cb >> shift
                npg = ((cb + nr - 1) >> shift) - pg0 + 1
                assert npg <= 1024 and (cb + nr - 1) // P < -(-C // P)
                ns_ = -(-nr // RSTEP)
                uniform = es == 1 and P >= RPI and cb % RPI == 0 and P * vrow <= 2 ** 31 - 1   # fp8 only
                for step in range(ns_ + (1 if ns_ > 1 else 0)):
                    for wave in range(NW):
                        r0 = 32 * (step * WPH + wave % WPH)
                        rows = np.minimum(r0 + RPI * np.arange(LPI)[:, None] + lanes[None, :] // PR, nr - 1)
                        idx = ((cb + rows) >> shift) - pg0
                        assert idx.min() >= 0 and idx.max() < npg
                        if not uniform:
                            continue
                        # pages of >= RPI rows: one page per load, through a
                        # resource from the page's row 0 (head kv) that ends
                        # with the split's last row in it
                        kvl = wave // WPH
                        vlane = (lanes // PR) * vrow + kvl * D * es + (lanes % PR) * 8 * es
                        for i in range(LPI):
                            r = cb + r0 + RPI * i
                            assert r % RPI == 0
                            pidx = min((r >> shift) - pg0, npg - 1)
                            assert 0 <= pidx < npg
                            pstart = r & ~(P - 1)
                            vr = min(P, cb + nr - pstart)
                            nrec = vr * vrow - kv * D * es if vr > 0 else 0
                            assert 0 <= nrec <= P * vrow - kv * D * es and nrec < 2 ** 31
                            off = vlane + (r & (P - 1)) * vrow
                            c = r + lanes // PR                  # the rows the lanes load
                            live = c < cb + nr
                            assert np.array_equal(off + 8 * es <= nrec, live)
                            # a live lane reads its own row's piece of its page
                            assert (c[live] >> shift == r >> shift).all()
                            assert np.array_equal(off[live], ((c[live] & (P - 1)) * vrow + kvl * D * es
                                                              + (lanes[live] % PR) * 8 * es))
        vrec = (nrows - 1) * vrow + HT * D * es
        assert ((b * C + cb) * Hkv + kv) * D * es + vrec <= B * C * Hkv * D * es and vrec < 2 ** 31
        wrec = ((nrows - 1) * Hq + (HT - 1) * G + nq) * 4
        assert ((b * C + cb) * Hq + qf) * 4 + wrec <= B * C * Hq * 4 and wrec < 2 ** 31
        nblk = -(-nrows // RSTEP)
        nsteps = (-(-(nblk - s) // ns) if nblk > s else 0) if il else nblk
        step_row = (lambda st: (st * ns + s) * RSTEP) if il else (lambda st: st * RSTEP)
        loaded, st = ([0] if nsteps else []), 0
        while st + 1 < nsteps:                  # the pipeline's loads, including its unconditional reload
            loaded += [st + 1, st + 2]
            st += 2
        for k in range(HT):
            seen.setdefault((b, kv + k, sg), [])
        for step in loaded:
            for wave in range(NW):
                kvl, wh = wave // WPH, wave % WPH
                r0 = step_row(step) + 32 * wh
                assert (r0 + 32 + 2 * RSTEP) * max(vrow, Hq * 4) < 2 ** 31
                rows = r0 + RPI * np.arange(LPI)[:, None] + lanes[None, :] // PR
                off = ((lanes // PR) * vrow + kvl * D * es + (lanes % PR) * 8 * es
                       + (r0 + RPI * np.arange(LPI)[:, None]) * vrow)
                assert np.array_equal(off + 8 * es <= vrec, rows < nrows)
                wrows = r0 + 8 * (lanes >> 4)[None, :] + np.arange(8)[:, None]
                for sset in range(NSET):
                    woff = np.minimum((lanes & 15) + 16 * sset, nq - 1)
                    wo = ((8 * (lanes >> 4)[None, :] * Hq + kvl * G + woff[None, :]) * 4
                          + (r0 + np.arange(8)[:, None]) * Hq * 4)
                    assert np.array_equal(wo + 4 <= wrec, wrows < nrows)
                if step < nsteps:
                    seen[(b, kv + kvl, sg)] += [cb + r for r in range(r0, r0 + 32) if r < nrows]
        if s == 0:
            # the final sum: wave w writes head row 16 s + 4 (l / 16) + i, column
            # 16 t + l % 16 of its [GH][RP] region; thread q then adds four
            # columns of head hh over its KV head's waves and stores them
            RP = D + 4
            lw = np.arange(64)
            for w in range(NW):
                for sset in range(NSET):
                    for t in range(D // 16):
                        for i in range(4):
                            off = (w * GT + 16 * sset + 4 * (lw >> 4) + i) * RP + 16 * t + (lw & 15)
                            assert off.min() >= 0 and off.max() < NW * GT * RP
                            # the four lane groups of one store land on different banks (64 banks)
                            assert len(set(off % 64)) == 64
            Q4 = D // 4
            q = np.arange(HT * GT * Q4)
            k, hh, c4 = q // (GT * Q4), (q // Q4) % GT, q % Q4
            for w in range(WPH):
                off = ((k * WPH + w) * GT + hh) * RP + 4 * c4
                assert off.min() >= 0 and off.max() + 3 < NW * GT * RP and (off % 4 == 0).all()
            ok = hh < nq
            for c in range(4):
                np.add.at(cnt, (b, qf + k[ok] * G + hh[ok], 4 * c4[ok] + c), 1)
        if p.softmax and ns > 1:
            for t2 in range(HT * GT):
                k2, hh = t2 // GT, t2 % GT
                if hh < nq:
                    scnt[s, b, qf + k2 * G + hh] += 1
    assert (cnt == 1).all()
    if p.softmax and ns > 1:
        assert (scnt == 1).all(), "each split's statistics of each (b, q_h) are written once"
    for key, rows in seen.items():
        assert sorted(rows) == list(range(C)), f"{key}: every row streamed by exactly one split"


@pytest.mark.parametrize("B,C,Hq,Hkv,D", [(1, 300, 16, 1, 128), (2, 1000, 16, 2, 64), (2, 130, 40, 2, 64),
                                         (1, 257, 24, 1, 256), (2, 31, 16, 1, 128), (1, 1, 16, 1, 64),
                                         (2, 700, 32, 4, 128), (1, 300, 48, 4, 256), (3, 1500, 16, 2, 64),
                                         (2, 700, 64, 8, 128), (1, 300, 16, 8, 64), (1, 200, 128, 16, 128)])
def test_bf16_engine_plan_bounds(B, C, Hq, Hkv, D):
    for ns in (0, 1, 3, 7):
        for comb, sm in (("kernel", False), ("auto", False), ("kernel", True)):
            for ht in (0, 1, 2, 4, 8):
                if ht > 1 and Hkv % ht:
                    continue
                for dt, es in (("bf16", 2), ("fp8", 1)):
                    for P in (0,) + ((16,) if ht in (0, 2, 8) else ()) + ((1, 256) if ns in (0, 3) and ht == 0 else ()):
                        for nw, order in (((0, "auto"), (0, "interleaved")) if sm else
                                          ((0, "auto"), (8, "auto"), (0, "contiguous"), (8, "contiguous"))):
                            if ht == 8 and nw not in (0, 8):
                                continue
                            try:
                                p = ga.make_plan(B, C, Hq, Hkv, D, dt, "reuse", engine="mfma_bf16", nsplit=ns,
                                                 combine=comb, kv_tile=ht, softmax=sm, page_size=P, waves=nw,
                                                 split_order=order)
                            except ga.GqaAvError as e:     # a forced split over more than 1024 pages, or
                                assert e.name == "UNSUPPORTED" and P and (   # interleaved splits of paged V
                                    (ns and -(-C // ns) > 1023 * P) or order == "interleaved")
                                continue
                            assert p.softmax == int(sm) and p.page_size == P
                            assert nw == 0 or p.threads == 64 * nw
                            assert p.interleave == ((order == "interleaved" or (order == "auto" and not sm))
                                                    and not P and p.nsplit > 1)
                            _check_plan(p, B, C, Hq, Hkv, D, es)


ENGINE_VALU = 1


def _esize(dt):
    return {"f32": 4, "fp8": 1}.get(dt, 2)


def _check_valu_plan(p, B, C, Hq, Hkv, D, dt):
    assert p.engine == ENGINE_VALU
    es, G = _esize(dt), Hq // Hkv
    VB, Lc, rps, ndt, HT = p.vec_bytes, p.lanes_per_row, p.row_slots, p.d_tiles, p.kv_heads_per_tile
    E, L = VB // es, D * es // VB
    per_head = p.mode == 0
    GT = 1 if per_head else p.heads_per_tile
    # rows per lane and step (valu_unroll): eight for three-head tiles over dense fp16 V
    U = 8 if (GT == 3 and dt == "f16" and not p.softmax and not p.page_size) else (
        4 if GT <= 4 else (2 if GT <= 8 else 1))
    R, vrow, ns = rps * U, Hkv * D * es, p.nsplit
    assert rps * Lc <= 256 and GT <= Hq
    nminor = ndt if per_head else p.subgroups * ndt
    nkvt = Hkv // HT
    tid = np.arange(256)
    r, j = tid // Lc, tid % Lc
    kvl = j // L
    cnt = np.zeros((B, Hq, D), np.int64)
    scnt = np.zeros((ns, B, Hq), np.int64)          # fused softmax: split statistics written
    rows_of = {}                                    # rows each tile's splits stream, over all splits
    if p.softmax:
        CH = min(GT * E, 32)
        assert HT <= 4 and rps * HT * GT <= CH * 256, "row-slot statistics must fit the reduction buffer"
    for blk in range(p.grid):
        t = _remap(blk, p.grid)
        minor = t % nminor; t //= nminor
        kvt = t % nkvt; t //= nkvt
        kv = kvt * HT
        s = t % ns; t //= ns
        b = t % B; major = t // B
        if per_head:
            dtile, qf, nq = minor, kv * G + major, 1
        else:
            sg, dtile = minor // ndt, minor % ndt
            qf, nq = kv * G + sg * GT, min(GT, G - sg * GT)
        lane_d = dtile * Lc + (j - kvl * L)
        active = (r < rps) & (lane_d < L)
        il = bool(p.interleave) and not p.page_size
        assert p.interleave in (0, 1) and not (p.interleave and p.page_size)
        if il:
            # interleaved: split s takes the blocks s, s + ns, ... of R rows of the sequence
            assert p.rows_per_split == R and 2 <= ns <= -(-C // R)
            cb, ce = 0, C
        else:
            cb = s * p.rows_per_split
            ce = min(C, cb + p.rows_per_split)
        nrows = ce - cb
        assert nrows > 0
        if p.page_size:
            # paged V: the split's page list (one entry per page its rows touch,
            # at most 1024) and every loaded row's entry in it, for a full-length
            # sequence and for shorter ones (rows past the length read the
            # split's last valid row)
            P = p.page_size
            shift = P.bit_length() - 1
            for ln in {C, C // 2, cb + 1, cb}:
                nr = max(0, min(ce, ln) - cb)
                if nr == 0:
                    continue
                pg0 = cb >> shift
                npg = ((cb + nr - 1) >> shift) - pg0 + 1
                assert npg <= 1024 and (cb + nr - 1) // P < -(-C // P)
                for step in range(-(-nr // R)):
                    for u in range(U):
                        rows = np.minimum(step * R + u * rps + r, nr - 1)
                        idx = ((cb + rows) >> shift) - pg0
                        assert idx.min() >= 0 and idx.max() < npg
        vrec = (nrows - 1) * vrow + HT * D * es
        assert ((b * C + cb) * Hkv + kv) * D * es + vrec <= B * C * Hkv * D * es and vrec < 2 ** 31
        wrec = nrows * Hq * 4
        assert (b * C + cb) * Hq * 4 + wrec <= B * C * Hq * 4
        q_lo = np.minimum(qf + kvl * G, Hq - GT)
        voff = r * vrow + kvl * D * es + lane_d * VB
        woff = (r * Hq + q_lo) * 4
        nblk = -(-nrows // R)
        nsteps = (-(-(nblk - s) // ns) if nblk > s else 0) if il else nblk
        step_row = (lambda st: (st * ns + s) * R) if il else (lambda st: st * R)
        loaded, st = ([0] if nsteps else []), 0
        while st + 1 < nsteps:
            loaded += [st + 1, st + 2]
            st += 2
        tile = (b, kvt, minor, major)
        rows_of.setdefault(tile, [])
        for step in loaded:
            for u in range(U):
                row = step_row(step) + u * rps
                assert (row + 2 * R) * vrow < 2 ** 31 and (row + 2 * R) * Hq * 4 < 2 ** 31
                inrow = (row + r) < nrows
                if step < nsteps:
                    rows_of[tile] += [cb + row + rr for rr in range(rps) if row + rr < nrows]
                off = voff + row * vrow
                assert np.array_equal((off + VB <= vrec)[active], inrow[active])
                assert (off[active] >= 0).all()
                wo = woff + row * Hq * 4
                for k0 in range(0, GT, 4):
                    n = min(4, GT - k0)
                    assert np.array_equal((wo + 4 * k0 + 4 * n <= wrec)[active], inrow[active])
        if s == 0:
            # epilogue: writers put their E columns of CHH heads at a time into
            # LDS rows [slot][KV head][head][RL columns]; readers add QW columns
            # of one head over the slots and store them at (b, ql + g, d)
            CHH = min(32 // E, GT) if E < 32 else 1
            QW = 4 if E % 4 == 0 else 1
            Lh = Lc // HT
            RL = Lh * E
            assert Lc % HT == 0 and RL % QW == 0
            jl = j - kvl * L
            red = min(GT * E, 32) * 256
            for g0 in range(0, GT, CHH):
                for gl in range(min(CHH, GT - g0)):
                    dst = ((r * HT + kvl) * CHH + gl) * RL + jl * E
                    assert (dst[active] >= 0).all() and (dst[active] + E <= red).all()
                    if QW == 4:
                        assert (dst[active] % 4 == 0).all()
                    # no two active lanes share an LDS word
                    assert len(set(dst[active].tolist())) == int(active.sum())
                nh = min(CHH, GT - g0)
                q = np.arange(HT * nh * (RL // QW))
                kl, gl = q // (nh * (RL // QW)), (q // (RL // QW)) % nh
                dl = (q % (RL // QW)) * QW
                d = (0 if HT > 1 else dtile * Lc * E) + dl
                g = g0 + gl
                ql = np.minimum(qf + kl * G, Hq - GT)
                go = qf + kl * G - ql
                keep = (d < D) & (g >= go) & (g < go + nq)
                assert (d[keep] + QW <= D).all()
                # the last slot's words of the kept units lie in the buffer, and
                # the lane that wrote them (slot rr, chunk kl * L + dl / E) is active
                src = (((rps - 1) * HT + kl) * CHH + gl) * RL + dl
                assert (src[keep] + QW <= red).all()
                assert (dtile * Lc + dl[keep] // E < L).all()
                for c in range(QW):
                    np.add.at(cnt, (b, (ql + g)[keep], d[keep] + c), 1)
        if p.softmax and ns > 1 and dtile == 0:
            # every row slot has an active first lane per KV head of the tile
            lead = active & (j - kvl * L == 0)
            assert sorted(zip(r[lead], kvl[lead])) == [(rr, k) for rr in range(rps) for k in range(HT)]
            for t2 in range(HT * GT):
                kl, g = t2 // GT, t2 % GT
                ql = min(qf + kl * G, Hq - GT)
                go = qf + kl * G - ql
                if go <= g < go + nq:
                    scnt[s, b, ql + g] += 1
    assert (cnt == 1).all()
    if p.softmax and ns > 1:
        assert (scnt == 1).all(), "each split's statistics of each (b, q_h) are written once"
    if not p.page_size:
        for tile, rows in rows_of.items():
            assert sorted(rows) == list(range(C)), f"tile {tile}: every row streamed by exactly one split"


@pytest.mark.parametrize("B,C,Hq,Hkv,D,dt", [
    (2, 1000, 8, 4, 128, "bf16"), (1, 300, 4, 2, 127, "bf16"), (2, 129, 6, 3, 1, "f16"), (1, 200, 1, 1, 64, "f32"),
    (2, 150, 64, 1, 64, "bf16"), (1, 90, 4, 2, 2048, "f32"), (3, 257, 10, 5, 80, "f16"), (2, 333, 24, 8, 96, "f16"),
    (1, 64, 32, 8, 128, "bf16"), (2, 500, 14, 2, 256, "bf16"), (1, 777, 12, 3, 128, "f32"),
    (2, 300, 16, 8, 128, "fp8"), (1, 129, 6, 3, 96, "fp8"), (2, 65, 64, 1, 2, "fp8"), (1, 200, 8, 2, 46, "fp8")])
def test_valu_engine_plan_bounds(B, C, Hq, Hkv, D, dt):
    modes = ("reuse", "per_head") if Hq // Hkv >= 2 else ("per_head",)
    for mode in modes:
        for ns in (0, 1, 3, 7):
            for ht in (0, 1, 2, 4):
                if ht > 1 and (Hkv % ht or mode == "per_head"):
                    continue
                for align, P in ((0, 0), (2, 0), (0, 1), (0, 16), (0, 64)):
                    for sm in (False, True):
                        # contiguous splits of paged or narrowed V are the automatic plan already
                        for order in (("auto", "contiguous") if (align, P) == (0, 0) else ("auto",)):
                            try:
                                p = ga.make_plan(B, C, Hq, Hkv, D, dt, mode, engine="valu", nsplit=ns, kv_tile=ht,
                                                 v_align=align, softmax=sm, page_size=P, split_order=order)
                            except ga.GqaAvError as e:
                                assert e.name == "UNSUPPORTED"
                                continue
                            assert p.softmax == int(sm)
                            assert p.interleave == (order == "auto" and not P and p.nsplit > 1 and not sm)
                            _check_valu_plan(p, B, C, Hq, Hkv, D, dt)


# ---- decode score step -------------------------------------------------------

QK_BLOCKS = 1   # 16-row blocks per wave and buffer in the score kernel
QK_BLOCKS_FP8 = 2   # the same for fp8 K
OUT_OF_RANGE = 0x40000000   # kOutOfRange: a buffer offset past every resource


def _check_qk_plan(p, B, C, Hq, Hkv, D, dt, UB=QK_BLOCKS, vec4=False):
    es, G = _esize(dt), Hq // Hkv
    per_head = p.mode == 0
    NBLK = D // 32
    NSET = 1 if per_head else p.heads_per_tile // 16
    HT = p.kv_heads_per_tile
    WPH = 4 // HT
    assert HT in (1, 2, 4) and Hkv % HT == 0 and (HT == 1 or not per_head)
    rows = p.rows_per_block
    assert rows % 64 == 0 and D % 32 == 0
    nchunk = -(-C // rows)
    nminor = G if per_head else p.subgroups
    nkvt = Hkv // HT
    assert p.grid == B * nkvt * nminor * nchunk
    krow = Hkv * D * es
    NP = D * es // 16
    lanes = np.arange(64)
    m, g = lanes & 15, lanes >> 4
    written = np.zeros((B, C, Hq), np.int64)
    for blk_id in range(p.grid):
        t = _remap(blk_id, p.grid)
        minor = t % nminor; t //= nminor
        kv0 = (t % nkvt) * HT; t //= nkvt
        chunk = t % nchunk; t //= nchunk
        b = t
        assert b < B
        r0 = chunk * rows
        nrows = min(rows, C - r0)
        assert nrows > 0
        if p.page_size:
            # paged K: the chunk's page list (at most 1024 entries) and every
            # loaded row's entry in it, reloads past the chunk clamped to its
            # last row, for full and shorter sequences
            P = p.page_size
            shift = P.bit_length() - 1
            for ln in {C, C // 2, r0 + 1, r0}:
                nr = max(0, min(r0 + rows, C, ln) - r0)
                if nr == 0:
                    continue
                pg0 = r0 >> shift
                npg = ((r0 + nr - 1) >> shift) - pg0 + 1
                assert npg <= 1024 and (r0 + nr - 1) // P < -(-C // P)
                nsteps_ = -(-(-(-nr // 16)) // (WPH * UB))
                for step in range(nsteps_ + (1 if nsteps_ > 1 else 0)):
                    for u in range(UB):
                        for wh in range(WPH):
                            j = (step * UB + u) * WPH + wh
                            for i in range(NP // 4):
                                rows_ = np.minimum(16 * j + (64 * i + lanes) // NP, nr - 1)
                                idx = ((r0 + rows_) >> shift) - pg0
                                assert idx.min() >= 0 and idx.max() < npg
        kbase = ((b * C + r0) * Hkv + kv0) * D * es
        krec = (nrows - 1) * krow + HT * D * es
        assert kbase + krec <= B * C * Hkv * D * es
        nrb = -(-nrows // 16)
        nsteps = -(-nrb // (WPH * UB))
        loaded, st = ([0] if nsteps else []), 0
        while st + 1 < nsteps:
            loaded += [st + 1, st + 2]
            st += 2
        for wave in range(4):
            kvl, wh = wave // WPH, wave % WPH
            kv = kv0 + kvl
            q_first = kv * G + minor if per_head else kv * G + minor * 16 * NSET
            nq = 1 if per_head else min(16 * NSET, G - minor * 16 * NSET)
            assert nq >= 1 and q_first + nq <= Hq
            for s in range(NSET):                      # q operand reads
                head = q_first + np.minimum(m + 16 * s, nq - 1)
                qidx = (b * Hq + head) * D + 8 * g
                assert qidx.min() >= 0 and (qidx + 32 * (NBLK - 1) + 7).max() < B * Hq * D
            for step, u in ((st_, u_) for st_ in loaded for u_ in range(UB)):
                j = (step * UB + u) * WPH + wh
                assert 16 * (j + 1) * krow < 2 ** 31
                for i in range(NP // 4):               # whole-row loads: piece f = 64 i + lane
                    f = 64 * i + lanes
                    off = (f // NP) * krow + kvl * D * es + (f % NP) * 16 + 16 * j * krow
                    assert np.array_equal(off + 16 <= krec, (16 * j + f // NP) < nrows)
        # Scores: each step's LDS tile (R rows x W columns), filled by the
        # waves, then stored with unconditional stores that the score
        # resource masks: row r by wave r % 4, VE heads per lane.
        R, WMAX = 16 * WPH * UB, HT * 16 * (1 if per_head else NSET)
        OP, NSR = WMAX + 4, R // 4 * WMAX // 64
        nq = 1 if per_head else min(16 * NSET, G - minor * 16 * NSET)
        q_tile = kv0 * G + (minor if per_head else minor * 16 * NSET)
        W, srow = HT * nq, 4 * Hq
        sbase = ((b * C + r0) * Hq + q_tile) * 4
        srec = (nrows - 1) * srow + 4 * ((HT - 1) * G + nq)
        assert sbase + srec <= 4 * B * C * Hq and srec <= 2 ** 30
        VE = 4 if vec4 else 1
        nsr = -(-(R // 4 * W) // (64 * VE))
        assert nsr <= NSR
        for step in range(nsteps):
            tile = {}
            for wave in range(4):
                kvl, wh = wave // WPH, wave % WPH
                for u in range(UB):
                    j = (step * UB + u) * WPH + wh
                    for s in range(NSET):
                        h = m + 16 * s
                        col = np.where(h < nq, kvl * nq + h, WMAX + (m & 3))
                        for i in range(4):
                            r = 16 * (j - step * UB * WPH) + 4 * g + i
                            assert r.max() < R and col.max() < OP
                            for rr, cc, hh in zip(r, col, h):
                                if hh < nq:
                                    assert (rr, cc) not in tile
                                    tile[(rr, cc)] = (16 * j + rr - 16 * (j - step * UB * WPH),
                                                      (kv0 + kvl) * G + (minor if per_head else minor * 16 * NSET) + hh)
            for wave in range(4):
                for k in range(nsr):
                    e = 64 * k + lanes
                    rq, c = e // (W // VE), (e % (W // VE)) * VE
                    r = 4 * rq + wave
                    kc = c // nq
                    ok = r < R
                    lds = np.where(ok, r * OP + c, 0)
                    assert (lds + VE <= R * OP).all() and (lds % VE == 0).all()
                    off = np.where(ok, r * srow + 4 * (kc * G + c - kc * nq), OUT_OF_RANGE) + step * R * srow
                    assert off.max() < 2 ** 31
                    inr = off + 4 * VE <= srec
                    assert np.array_equal(inr, ok & (step * R + r < nrows))
                    for rr, cc, oo in zip(r[inr], c[inr], off[inr]):
                        assert (sbase + oo) % (4 * VE) == 0
                        for v in range(VE):
                            row, head = tile[(rr, cc + v)]
                            assert (sbase + oo) // 4 + v == (b * C + r0 + row) * Hq + head
                            written[b, r0 + row, head] += 1
    assert (written == 1).all()


@pytest.mark.parametrize("B,C,Hq,Hkv,D,dt", [
    (2, 300, 8, 2, 64, "bf16"), (1, 65, 16, 1, 128, "f16"), (2, 129, 6, 3, 32, "f32"), (1, 1, 4, 4, 96, "bf16"),
    (2, 500, 64, 2, 256, "bf16"), (1, 1000, 40, 1, 128, "f16"), (3, 77, 24, 8, 96, "f32"), (1, 257, 68, 2, 160, "bf16"),
    (2, 700, 32, 4, 128, "bf16"), (1, 333, 24, 8, 96, "f16"), (2, 300, 16, 8, 128, "fp8"), (1, 129, 64, 1, 64, "fp8"),
    (2, 77, 12, 2, 256, "fp8"), (2, 300, 16, 1, 128, "fp8"), (1, 200, 64, 2, 64, "bf16")])
def test_qk_plan_bounds(B, C, Hq, Hkv, D, dt):
    modes = ("auto", "per_head") if Hq // Hkv >= 2 else ("auto",)
    for mode in modes:
        for rows, P in ((0, 0), (64, 0), (128, 0), (192, 0), (0, 1), (192, 16), (0, 64)):
            for ht in ((0, 1, 2, 4) if not P else (0,)):
                if ht > 1 and (Hkv % ht or mode == "per_head" or Hq // Hkv < 2):
                    continue
                p = ga.qk_make_plan(B, C, Hq, Hkv, D, dt, mode, rows_per_block=rows, kv_tile=ht, page_size=P)
                assert p.page_size == P
                # 16-byte score stores when the host would choose them (scores
                # 16-byte aligned), 4-byte stores always possible
                v4 = p.mode == 1 and p.subgroups == 1 and (p.kv_heads_per_tile * (Hq // Hkv)) % 4 == 0 and Hq % 4 == 0
                for vec4 in ((False, True) if v4 else (False,)):
                    _check_qk_plan(p, B, C, Hq, Hkv, D, dt, UB=QK_BLOCKS_FP8 if dt == "fp8" else QK_BLOCKS, vec4=vec4)


@pytest.mark.parametrize("D,dt", [(32, "bf16"), (96, "f16"), (128, "bf16"), (160, "f32"), (256, "f32"), (224, "f16"),
                                  (64, "fp8"), (128, "fp8"), (192, "fp8"), (256, "fp8")])
def test_qk_lds_relayout(D, dt):
    """The score kernel's LDS re-layout: every 16-byte piece of the 16-row block
    is stored once inside the wave's region (fp8: a 16-byte piece of 16 values
    becomes two 16-byte bf16 pieces), and lane (m, g) reads back row m's
    d-range [32 blk + 8 g, +8) for each block of 32 d (16-row reads in
    distinct 16-byte bank groups)."""
    es = _esize(dt)
    esl = 2 if dt == "fp8" else es                       # LDS element size
    NP, RBP = D * es // 16, D * esl + 16
    assert NP % 4 == 0
    where = {}
    for i in range(NP // 4):
        for lane in range(64):
            f = 64 * i + lane
            row, piece = f // NP, f % NP
            for half in range(esl // es):               # fp8: the widened piece's two halves
                off = row * RBP + piece * 16 * (esl // es) + 16 * half
                assert 0 <= off and off + 16 <= 16 * RBP and off not in where.values()
                where[(row, piece * (esl // es) + half)] = off
    assert len(where) == 16 * NP * (esl // es)
    es = esl                                             # the operand reads see LDS elements
    pieces_per_op = 2 if dt == "f32" else 1
    for blk in range(D // 32):
        for pc in range(pieces_per_op):
            groups = set()
            for lane in range(64):
                m, g = lane & 15, lane >> 4
                off = m * RBP + (32 * blk + 8 * g) * es + 16 * pc
                byte = (32 * blk + 8 * g) * es + 16 * pc
                assert where[(m, byte // 16)] == off       # the piece holding d = 32 blk + 8 g (+ 4 pc for fp32)
                if g == 0:
                    groups.add((off // 16) % 16)
            assert len(groups) == 16                      # the 16 rows of one lane group: distinct bank groups


@pytest.mark.parametrize("D,es", [(64, 2), (128, 2), (256, 2)])
def test_attention_direct_k_loads(D, es):
    """Dense bf16 fused attention loads K straight into the score MFMA's B layout:
    load i of a chunk gives lane 16 g + n piece 4 kk + g of row 16 t2 + n
    (t2 = i / NKK, kk = i % NKK) of its KV head, through the K resource that
    ends with the split's last row; rows past the split read as zero."""
    PR, NKK = D // 8, D // 32
    LPI, PB = PR // 2, 8 * es
    assert LPI == 2 * NKK
    lanes = np.arange(64)
    g, n = lanes >> 4, lanes & 15
    for Hkv, HT in ((1, 1), (4, 2), (8, 4)):
        vrow = Hkv * D * es
        for kv in range(0, Hkv, HT):
            for nrows in (1, 17, 32, 45, 100):
                krec = (nrows - 1) * vrow + HT * D * es
                for kvl in range(HT):
                    klane = n * vrow + kvl * D * es + g * PB
                    for r0 in range(0, ((nrows + 31) // 32 + 1) * 32, 32):   # with the pipeline's reload past the end
                        for i in range(LPI):
                            t2, kk = i // NKK, i % NKK
                            off = klane + (r0 + 16 * t2) * vrow + 4 * kk * PB
                            row = r0 + 16 * t2 + n
                            piece = 4 * kk + g
                            # the element the lane must hold: row, KV head kv + kvl, d = 8 piece .. + 7
                            assert np.array_equal(off, row * vrow + kvl * D * es + piece * PB)
                            assert (piece < D // 8).all()
                            assert np.array_equal(off + PB <= krec, row < nrows)
                            assert (off[row < nrows] >= 0).all()
