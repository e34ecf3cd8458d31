"""Host model of the LDS layout of an N-contiguous GEMM stage (the X operand
of Q X in the 256 x 256 kernel, gemm.hip: nslot / nchunk / swzn and the
transposing fragment reads).  Checked on the CPU: the slot map is a
bijection per row, the DMA placement (lane L of a row fetches chunk
nchunk(kr, L mod 32) into slot L mod 32) and the read addresses agree, and no
read phase has a bank conflict, whether the LDS serves 16 lanes over 32 banks
or 32 lanes over 64 banks of 4 bytes per cycle."""


def t(ch):
    return ch ^ (((ch >> 1) & 1) << 3)


def nslot(kr, ch):
    return t(ch) ^ (2 * (kr & 3))


def nchunk(kr, s):
    return t(s ^ (2 * (kr & 3)))


def swzn(kr, n):
    return kr * 512 + (nslot(kr, n >> 3) << 4) + ((n & 4) << 1)


def read_addrs(wn, j, st, half):
    """Byte addresses of the 64 lanes of one ds_read_b64_tr_b16 of fragment j
    (k-step st, second read of the pair when half = 1)."""
    out = []
    for lane in range(64):
        gg, q, tt = lane >> 4, (lane >> 2) & 3, lane & 3
        n = wn * 128 + j * 32 + 16 * (gg & 1) + 4 * tt
        kr0 = 16 * st + 8 * (gg >> 1) + q + 4 * half
        out.append(swzn(kr0, n))
    return out


def worst_conflict(addrs, lanes, banks):
    worst = 1
    for g0 in range(0, 64, lanes):
        cnt = {}
        for a in addrs[g0:g0 + lanes]:
            for w in range(2):
                b = (a // 4 + w) % banks
                cnt[b] = cnt.get(b, 0) + 1
        worst = max(worst, max(cnt.values()))
    return worst


def test_slot_map_is_a_bijection_and_matches_the_dma():
    for kr in range(32):
        assert sorted(nslot(kr, c) for c in range(32)) == list(range(32))
        for s in range(32):
            assert nslot(kr, nchunk(kr, s)) == s


def test_transposing_reads_are_conflict_free():
    for wn in range(2):
        for j in range(4):
            for st in range(2):
                for half in range(2):
                    a = read_addrs(wn, j, st, half)
                    assert len(set(a)) == 64
                    assert worst_conflict(a, 16, 32) == 1
                    assert worst_conflict(a, 32, 64) == 1


def test_plain_xor_layout_conflicts_on_64_banks():
    # the layout without t: 2-way conflicts when 32 lanes share 64 banks
    global t
    saved = t
    t = lambda ch: ch  # noqa: E731
    try:
        assert max(worst_conflict(read_addrs(0, j, 0, 0), 32, 64) for j in range(4)) == 2
    finally:
        t = saved


# ---------------------------------------------------------------------------
# Symmetric epilogue of the 256 x 256 kernel (gemm.hip: epilogue_sym): which
# entry of C each lane stores, modelled from the accumulator layout.


def _acc(m0, n0, wm, wn, i, j, lane, g, q):
    """(row, column) of C held by accumulator 4 g + q of block (i, j)."""
    lc, lh = lane & 31, lane >> 5
    return (m0 + wm * 128 + 32 * i + lc, n0 + wn * 128 + 32 * j + 8 * g + 4 * lh + q)


def _butterfly(X):
    """Transpose of 8 dwords across each group of 8 lanes (distances 4, 2, 1)."""
    for s in (4, 2, 1):
        new = [list(r) for r in X]
        for lane in range(64):
            up = (lane & 7) & s
            partner = lane ^ s
            for k in range(8):
                if k & s:
                    continue
                kk = k | s
                sent = X[partner][k] if ((partner & 7) & s) else X[partner][kk]
                if up:
                    new[lane][k] = sent
                else:
                    new[lane][kk] = sent
        X = new
    return X


def _mirror_chunks(m0, n0, wm, wn, i, j):
    """Butterfly output of block (i, j): Y[lane][e][b] is the entry of block row
    8 o + e and column c0 + b that lane holds for the mirrored store."""
    d = [[(_acc(m0, n0, wm, wn, i, j, L, k >> 1, 2 * (k & 1)),
           _acc(m0, n0, wm, wn, i, j, L, k >> 1, 2 * (k & 1) + 1)) for k in range(8)]
         for L in range(64)]
    return _butterfly(d)


def _symmetric_epilogue_writes(n, paired):
    written = {}
    T = n // 256
    for ti in range(T):
        for tj in range(ti + 1):
            m0, n0, diag = 256 * ti, 256 * tj, ti == tj
            for wm in range(2):
                for wn in range(2):
                    if diag and wm < wn:
                        continue
                    dq = diag and wm == wn
                    if paired and not dq:
                        # a full quadrant of the symmetric product: direct stores of
                        # blocks (i, j), (i, j + 1) together (lanes L and L ^ 8
                        # exchange one chunk each)
                        for i in range(4):
                            for j in (0, 2):
                                ra0, rb0 = _qx_chunks(wm, wn, i, j)
                                ra1, rb1 = _qx_chunks(wm, wn, i, j + 1)
                                for hh in range(2):
                                    x0 = rb0 if hh else ra0
                                    x1 = rb1 if hh else ra1
                                    send = [x0[L] if (L >> 3) & 1 else x1[L] for L in range(64)]
                                    recv = [send[(L & ~15) | ((L + 8) & 15)] for L in range(64)]
                                    for L in range(64):
                                        lc, lh = L & 31, L >> 5
                                        hi8 = (lc >> 3) & 1
                                        col = n0 + wn * 128 + 32 * j + 32 * hi8 + 16 * ((lc >> 4) & 1) + 8 * lh
                                        for rowoff, chunk in ((0, recv[L] if hi8 else x0[L]), (8, x1[L] if hi8 else recv[L])):
                                            row = m0 + wm * 128 + 32 * i + 16 * hh + (lc & 7) + rowoff
                                            for e in range(8):
                                                pos = (row, col + e)
                                                src = (chunk[e][0] + m0, chunk[e][1] + n0)
                                                assert src == pos
                                                assert pos not in written
                                                written[pos] = src
                        # mirror stores of blocks (i, j) and (i + 1, j) together (lanes
                        # t and t ^ 1 exchange one chunk each)
                        for i in (0, 2):
                            for j in range(4):
                                Y0 = _mirror_chunks(m0, n0, wm, wn, i, j)
                                Y1 = _mirror_chunks(m0, n0, wm, wn, i + 1, j)
                                for rr in range(2):
                                    x0 = [[Y0[L][e][rr] for e in range(8)] for L in range(64)]
                                    x1 = [[Y1[L][e][rr] for e in range(8)] for L in range(64)]
                                    send = [x0[L] if L & 1 else x1[L] for L in range(64)]
                                    recv = [send[L ^ 1] for L in range(64)]
                                    for L in range(64):
                                        lc, lh = L & 31, L >> 5
                                        o, t = lc >> 3, lc & 7
                                        t1 = t & 1
                                        c0 = 8 * (t >> 1) + 4 * lh + 2 * t1
                                        col = m0 + wm * 128 + 32 * (i + t1) + 8 * o
                                        for rowoff, chunk in ((0, recv[L] if t1 else x0[L]), (2, x1[L] if t1 else recv[L])):
                                            row = n0 + wn * 128 + 32 * j + c0 - 2 * t1 + rr + rowoff
                                            for e in range(8):
                                                pos = (row, col + e)
                                                assert chunk[e] == (pos[1], pos[0])   # the mirrored entry
                                                assert pos not in written
                                                written[pos] = chunk[e]
                    for i in range(4):
                        for j in range(4):
                            if dq and i < j:
                                continue
                            dblk = dq and i == j
                            # direct: after the half-wave swap lane L holds columns
                            # 16 pr + 8 (L/32) .. +7 of row L mod 32 (w[pr][L]); the
                            # 16-lane swap (rows64) then gives lane L the chunks of
                            # rows L mod 16 and 16 + L mod 16 at column 16 ((L/16) mod 2) + 8 (L/32)
                            w = [[[_acc(m0, n0, wm, wn, i, j, 32 * (((16 * pr + 8 * (L >> 5) + e) % 8) // 4) + (L & 31),
                                        (16 * pr + 8 * (L >> 5) + e) // 8, (16 * pr + 8 * (L >> 5) + e) % 4)
                                   for e in range(8)] for L in range(64)] for pr in range(2)]
                            for lane in range(64 if dq or not paired else 0):
                                lc, lh = lane & 31, lane >> 5
                                odd = (lane >> 4) & 1
                                a = w[1][lane - 16] if odd else w[0][lane]
                                b = w[1][lane] if odd else w[0][lane + 16]
                                y0 = 16 * ((lc >> 4) & 1) + 8 * lh
                                for hh, chunk in ((0, a), (1, b)):
                                    r = 16 * hh + (lc & 15)
                                    for e in range(8):
                                        if dblk and y0 + e > r:
                                            continue
                                        pos = (m0 + wm * 128 + 32 * i + r, n0 + wn * 128 + 32 * j + y0 + e)
                                        assert chunk[e] == pos       # a direct store holds its own entry
                                        assert pos not in written
                                        written[pos] = chunk[e]
                            # mirror
                            Y = _mirror_chunks(m0, n0, wm, wn, i, j)
                            for lane in range(64 if dq or not paired else 0):
                                lc, lh = lane & 31, lane >> 5
                                o, t = lc >> 3, lc & 7
                                c0 = 8 * (t >> 1) + 4 * lh + 2 * (t & 1)
                                for b in range(2):
                                    for e in range(8):
                                        if dblk and not (8 * o + e > c0 + b):
                                            continue
                                        pos = (n0 + wn * 128 + 32 * j + c0 + b, m0 + wm * 128 + 32 * i + 8 * o + e)
                                        assert pos not in written
                                        written[pos] = Y[lane][e][b]
    return written


def test_symmetric_epilogue_writes_every_entry_once_from_the_lower_triangle():
    for n, paired in ((256, False), (768, False), (768, True)):
        w = _symmetric_epilogue_writes(n, paired)
        assert len(w) == n * n
        for (x, y), (r, c) in w.items():
            assert r >= c                      # computed at or below the diagonal
            assert (x, y) in ((r, c), (c, r))  # stored at its place or the mirrored one


# ---------------------------------------------------------------------------
# Q X epilogue of the 256 x 256 kernel (gemm.hip: epilogue_swap, 16-bit
# output): half-wave swap, 16-lane swap (rows64) and the exchange between
# lanes L and L ^ 8 (DPP rotation by 8 within 16 lanes), then 8 rows x 128
# bytes per store.  Every entry of the tile is written once, with its own value.


def _qx_chunks(wm, wn, i, j):
    """rows64 output per lane: (ra, rb), each 8 (row, column) entries of the tile."""
    w = [[[_acc(0, 0, wm, wn, i, j, 32 * (((16 * pr + 8 * (L >> 5) + e) % 8) // 4) + (L & 31),
                (16 * pr + 8 * (L >> 5) + e) // 8, (16 * pr + 8 * (L >> 5) + e) % 4)
           for e in range(8)] for L in range(64)] for pr in range(2)]
    ra, rb = [], []
    for L in range(64):
        odd = (L >> 4) & 1
        ra.append(w[1][L - 16] if odd else w[0][L])
        rb.append(w[1][L] if odd else w[0][L + 16])
    return ra, rb


def test_qx_epilogue_writes_every_entry_once():
    written = {}
    for wm in range(2):
        for wn in range(2):
            for i in range(4):
                for j in (0, 2):
                    ra0, rb0 = _qx_chunks(wm, wn, i, j)
                    ra1, rb1 = _qx_chunks(wm, wn, i, j + 1)
                    for hh in range(2):
                        x0 = rb0 if hh else ra0
                        x1 = rb1 if hh else ra1
                        send = [x0[L] if (L >> 3) & 1 else x1[L] for L in range(64)]
                        recv = [send[(L & ~15) | ((L + 8) & 15)] for L in range(64)]   # row_ror:8
                        for L in range(64):
                            lc, lh = L & 31, L >> 5
                            hi8 = (lc >> 3) & 1
                            col = 32 * j + 32 * hi8 + 16 * ((lc >> 4) & 1) + 8 * lh
                            for rowoff, chunk in ((0, recv[L] if hi8 else x0[L]), (8, x1[L] if hi8 else recv[L])):
                                row = wm * 128 + 32 * i + 16 * hh + (lc & 7) + rowoff
                                for e in range(8):
                                    pos = (row, wn * 128 + col + e)
                                    assert chunk[e] == pos
                                    assert pos not in written
                                    written[pos] = True
    assert len(written) == 256 * 256
    # one store: 8 rows x 64 columns (128 contiguous bytes per row)
