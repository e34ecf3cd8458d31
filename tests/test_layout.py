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
