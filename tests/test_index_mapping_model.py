"""CPU model of the chunked prefill's work mapping: which workspace unit and which token rows
each prep and scan workgroup touches, checked for every workgroup of the grid.

The prep grid covers the chunk bound rounded up to 8 (heads of one chunk on one XCD, since
workgroups are dealt round-robin over the 8 XCDs); the scan runs one chain per
(sequence, head). The model restates the index arithmetic of the kernels and checks that
  - with cu_seqlens as the header requires (cu[0] = 0, non-decreasing, cu[n] = T), every
    chunk of every sequence is prepared by exactly one workgroup into the unit the scan reads,
    and the rows touched are the chunk's own;
  - with cu_seqlens that break that contract (decreasing, negative, past T, describing more
    chunks than the workspace bound), no workgroup reads or writes a workspace unit at or past
    the bound, and no token row outside [0, T) is read or written.
The same holds for the two-segment scan (first segment [c0, mid), second [mid, c_end) with
mid = c0 + ceil(35 n / 64) for n >= 40 chunks) and its combine pass, whose chunk workgroups
are numbered over the second segments' chunks of all sequences: with valid cu_seqlens every
second-segment chunk of every (sequence, head) is combined by exactly one workgroup within
the grid bound, and the first segments and the combine together write every output row
once.
"""
import random

import pytest

WAVE = 64


def max_chunks(T, n, C):
    return (T + n * (C - 1)) // C


def seq_table(cu, n, C):
    """Each wave's inline table (up to 64 sequences): exclusive / inclusive prefix sums of
    ceil(max(0, len) / C)."""
    excl, incl, run = [], [], 0
    for s in range(n):
        cnt = (max(0, cu[s + 1] - cu[s]) + C - 1) // C
        excl.append(run)
        run += cnt
        incl.append(run)
    return excl, incl


def locate_chunk(c, cu, n, C, T):
    excl, incl = seq_table(cu, n, C)
    hits = [s for s in range(n) if excl[s] <= c < incl[s]]
    if not hits:
        return None
    s = hits[0]
    tok0 = cu[s] + (c - excl[s]) * C
    ln = min(C, min(cu[s + 1], T) - tok0)
    if tok0 < 0 or ln <= 0:
        return None
    return s, tok0, ln


def seg_prep_group(i, NG, a64=35):
    """The two-segment scan's prep order: dispatch slot i -> chunk group."""
    sg = (NG * a64 + 63) // 64
    na, nb = sg, NG - sg
    mn = min(na, nb)
    r = NG - 1 - i
    if r < 2 * mn:
        return r // 2 if r % 2 == 0 else sg + r // 2
    return r - mn if na > nb else sg + (r - mn)


def prep_touch(cu, n, T, H, C, conv, seg=False):
    """For every prep workgroup: (unit, rows read, rows of the conv halo read). seg: the
    chunk-group order of a call that runs the two-segment scan."""
    mc = max_chunks(T, n, C)
    grid = (mc if conv else (mc + 7) // 8 * 8) * H
    out = []
    for b in range(grid):
        if conv:
            c, h = b // H, b % H
        else:
            xcd, jj = b & 7, b >> 3
            grp = seg_prep_group(jj // H, (mc + 7) // 8) if seg else jj // H
            c, h = grp * 8 + xcd, jj % H
        if c >= mc:
            continue
        loc = locate_chunk(c, cu, n, C, T)
        if loc is None:
            continue
        s, tok0, ln = loc
        rows = list(range(tok0, tok0 + ln))
        halo = []
        if conv:
            ss = cu[s]
            for w in range(C // 16):
                for r16 in (13, 14, 15):
                    hrow = tok0 + w * 16 + r16 - 16
                    if hrow >= ss and hrow >= 0 and hrow < tok0 + ln:
                        halo.append(hrow)
        out.append((c * H + h, (c, h), rows, halo))
    return out


def scan_touch(cu, n, T, H, C):
    """For every (sequence, head) chain: units read and token rows touched. A chain reads the
    workspace units of its chunks and, one and three chunks ahead (clamped to its last
    chunk), the units and the v and q rows of later chunks (wide value tiles); it writes the
    output rows of its chunks. Every row index goes through the same test (row within the
    chunk's length, token index not negative) before it is used."""
    mc = max_chunks(T, n, C)
    excl, incl = seq_table(cu, n, C)
    out = []
    for s in range(n):
        c_begin, c_end = excl[s], min(incl[s], mc)
        clast = c_end - 1
        t_begin, t_end = cu[s], min(cu[s + 1], T)

        def rows_of(cc):
            tok0 = t_begin + (cc - c_begin) * C
            ln = min(C, t_end - tok0)
            return [tok0 + i for i in range(C) if i < ln and tok0 + i >= 0]

        for h in range(H):
            units, rows = [], []
            for c in range(c_begin, c_end):
                for cc in sorted({c, min(c + 1, clast), min(c + 3, clast)}):
                    units.append(cc * H + h)
                    rows += rows_of(cc)
            out.append((s, h, units, rows))
    return out


def _valid_cu(rng, n, maxlen):
    lens = [rng.randrange(0, maxlen) for _ in range(n)]
    cu = [0]
    for L in lens:
        cu.append(cu[-1] + L)
    return cu


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("C", [16, 64])
@pytest.mark.parametrize("conv", [False, True])
def test_valid_cu_seqlens_exact_cover(seed, C, conv):
    rng = random.Random(seed)
    n, H = rng.randrange(1, 9), rng.choice([1, 3, 16])
    cu = _valid_cu(rng, n, 300)
    T = cu[-1]
    prep = prep_touch(cu, n, T, H, C, conv)
    units = [u for u, _, _, _ in prep]
    assert len(units) == len(set(units))  # one workgroup per unit
    excl, incl = seq_table(cu, n, C)
    expect = {(c, h) for s in range(n) for c in range(excl[s], incl[s]) for h in range(H)}
    assert {ch for _, ch, _, _ in prep} == expect
    for u, (c, h), rows, halo in prep:
        s = next(s for s in range(n) if excl[s] <= c < incl[s])
        assert rows and cu[s] <= rows[0] and rows[-1] < cu[s + 1]
        assert all(cu[s] <= r < rows[-1] + 1 for r in halo)
    for s, h, su, rows in scan_touch(cu, n, T, H, C):
        assert set(su) == {c * H + h for c in range(excl[s], incl[s])}
        assert set(rows) == set(range(cu[s], cu[s + 1]))


BROKEN = [
    [0, 1000, 0, 1000],          # decreasing: more chunks than the workspace bound
    [0, 70, 30, 200, 150],       # overlapping, decreasing
    [-64, 10, 300],              # negative start
    [0, 50, 900],                # past total_tokens
    [5, 5, 5],                   # cu[0] != 0
    [0, 300, 100, 400, 0, 500],
]


@pytest.mark.parametrize("cu", BROKEN)
@pytest.mark.parametrize("C", [16, 64])
@pytest.mark.parametrize("conv", [False, True])
def test_broken_cu_seqlens_stay_in_bounds(cu, C, conv):
    n, H = len(cu) - 1, 3
    T = 400 if cu != BROKEN[0] else 1000
    mc = max_chunks(T, n, C)
    for u, _, rows, halo in prep_touch(cu, n, T, H, C, conv):
        assert 0 <= u < mc * H
        assert all(0 <= r < T for r in rows + halo)
    for _, _, units, rows in scan_touch(cu, n, T, H, C):
        assert all(0 <= u < mc * H for u in units)
        assert all(0 <= r < T for r in rows)


def test_random_broken_cu_seqlens_stay_in_bounds():
    rng = random.Random(7)
    for _ in range(200):
        n, H, C = rng.randrange(1, 7), rng.choice([1, 2, 5]), rng.choice([16, 32, 64])
        T = rng.randrange(0, 500)
        cu = [rng.randrange(-100, 700) for _ in range(n + 1)]
        mc = max_chunks(T, n, C)
        for u, _, rows, halo in prep_touch(cu, n, T, H, C, rng.random() < 0.5):
            assert 0 <= u < mc * H and all(0 <= r < T for r in rows + halo)
        for _, _, units, rows in scan_touch(cu, n, T, H, C):
            assert all(0 <= u < mc * H for u in units) and all(0 <= r < T for r in rows)


# ------------------------------------------------------------------ two-segment scan
SEG_MIN_CHUNKS, SEG_A_64 = 40, 35


def seg_mid(c0, c1):
    n = c1 - c0
    return c1 if n < SEG_MIN_CHUNKS else c0 + (n * SEG_A_64 + 63) // 64


def seg_scan_touch(cu, n, T, H, C):
    """Both segments' workgroups: (sequence, head, units read, units written, rows written).
    A second-segment workgroup writes its chunks' zero-state outputs over their U and their
    L, both in the unit's own workspace slots, and no token rows."""
    mc = max_chunks(T, n, C)
    excl, incl = seq_table(cu, n, C)
    out = []
    for s in range(n):
        c0, c_end = excl[s], min(incl[s], mc)
        mid = seg_mid(c0, c_end)
        t_begin, t_end = cu[s], min(cu[s + 1], T)

        def rows_of(cc):
            tok0 = t_begin + (cc - c0) * C
            ln = min(C, t_end - tok0)
            return [tok0 + i for i in range(C) if i < ln and tok0 + i >= 0]

        for h in range(H):
            for lo, hi, second in ((c0, mid, False), (mid, c_end, True)):
                if second and lo >= hi:
                    continue
                clast = hi - 1
                rd, wr, rows = [], [], []
                for c in range(lo, hi):
                    rd += [cc * H + h for cc in {c, min(c + 1, clast)}]
                    if second:
                        wr.append(c * H + h)
                    else:
                        rows += rows_of(c)
                out.append((s, h, rd, wr, rows))
    return out


def combine_touch(cu, n, T, H, C):
    """Chunk workgroups of the combine: (sequence, head, chunk, unit, rows written)."""
    mc = max_chunks(T, n, C)
    excl, incl = seq_table(cu, n, C)
    c1l = [min(x, mc) for x in incl]
    nbl = [max(0, c1l[s] - seg_mid(excl[s], c1l[s])) for s in range(n)]
    pin, run = [], 0
    for x in nbl:
        run += x
        pin.append(run)
    pex = [pin[s] - nbl[s] for s in range(n)]
    bound = (mc * (64 - SEG_A_64) + 63) // 64 + 1
    out = []
    for b in range(bound * H):
        h, k = b % H, b // H
        hits = [s for s in range(n) if pex[s] <= k < pin[s]]
        if not hits:
            continue
        s = hits[0]
        c = seg_mid(excl[s], c1l[s]) + (k - pex[s])
        tok0 = cu[s] + (c - excl[s]) * C
        ln = min(C, min(cu[s + 1], T) - tok0)
        rows = [tok0 + i for i in range(C) if i < ln and tok0 + i >= 0]
        out.append((s, h, c, c * H + h, rows))
    return out


def _long_cu(rng, n):
    lens = [rng.choice([0, rng.randrange(1, 900), rng.randrange(1000, 9000)]) for _ in range(n)]
    cu = [0]
    for L in lens:
        cu.append(cu[-1] + L)
    return cu


@pytest.mark.parametrize("seed", range(8))
def test_two_segment_exact_cover(seed):
    rng = random.Random(100 + seed)
    n, H, C = rng.randrange(1, 17), rng.choice([1, 2, 4]), 64
    cu = _long_cu(rng, n)
    T = cu[-1]
    excl, incl = seq_table(cu, n, C)
    written = {}
    for s, h, rd, wr, rows in seg_scan_touch(cu, n, T, H, C):
        assert set(rd) <= {c * H + h for c in range(excl[s], incl[s])}
        for r in rows:
            written[(r, h)] = written.get((r, h), 0) + 1
    comb = combine_touch(cu, n, T, H, C)
    seen = set()
    for s, h, c, u, rows in comb:
        assert seg_mid(excl[s], incl[s]) <= c < incl[s]
        assert (s, h, c) not in seen
        seen.add((s, h, c))
        for r in rows:
            written[(r, h)] = written.get((r, h), 0) + 1
    expect = {(s, h, c) for s in range(n) for h in range(H)
              for c in range(seg_mid(excl[s], incl[s]), incl[s])}
    assert seen == expect
    assert written == {(r, h): 1 for r in range(T) for h in range(H)}


@pytest.mark.parametrize("cu", BROKEN)
def test_two_segment_broken_cu_seqlens_stay_in_bounds(cu):
    n, H, C = len(cu) - 1, 3, 64
    for T in (400, 1000, 5000):
        mc = max_chunks(T, n, C)
        for _, _, rd, wr, rows in seg_scan_touch(cu, n, T, H, C):
            assert all(0 <= u < mc * H for u in rd + wr)
            assert all(0 <= r < T for r in rows)
        for _, _, _, u, rows in combine_touch(cu, n, T, H, C):
            assert 0 <= u < mc * H and all(0 <= r < T for r in rows)


def test_two_segment_random_broken_cu_seqlens_stay_in_bounds():
    rng = random.Random(11)
    for _ in range(200):
        n, H, C = rng.randrange(1, 9), rng.choice([1, 2, 5]), 64
        T = rng.randrange(0, 6000)
        cu = [rng.randrange(-500, 7000) for _ in range(n + 1)]
        mc = max_chunks(T, n, C)
        for _, _, rd, wr, rows in seg_scan_touch(cu, n, T, H, C):
            assert all(0 <= u < mc * H for u in rd + wr) and all(0 <= r < T for r in rows)
        for _, _, _, u, rows in combine_touch(cu, n, T, H, C):
            assert 0 <= u < mc * H and all(0 <= r < T for r in rows)


def test_seg_prep_order_is_a_permutation():
    for NG in range(1, 200):
        assert sorted(seg_prep_group(i, NG) for i in range(NG)) == list(range(NG))


@pytest.mark.parametrize("seed", range(6))
def test_two_segment_prep_exact_cover(seed):
    rng = random.Random(200 + seed)
    n, H, C = rng.randrange(1, 9), rng.choice([1, 3, 16]), 64
    cu = _long_cu(rng, n)
    T = cu[-1]
    prep = prep_touch(cu, n, T, H, C, False, seg=True)
    units = [u for u, _, _, _ in prep]
    assert len(units) == len(set(units))
    excl, incl = seq_table(cu, n, C)
    expect = {(c, h) for s in range(n) for c in range(excl[s], incl[s]) for h in range(H)}
    assert {ch for _, ch, _, _ in prep} == expect


@pytest.mark.parametrize("cu", BROKEN)
def test_two_segment_prep_broken_cu_seqlens_stay_in_bounds(cu):
    n, H, C = len(cu) - 1, 3, 64
    for T in (400, 1000, 5000):
        mc = max_chunks(T, n, C)
        for u, _, rows, _ in prep_touch(cu, n, T, H, C, False, seg=True):
            assert 0 <= u < mc * H and all(0 <= r < T for r in rows)
