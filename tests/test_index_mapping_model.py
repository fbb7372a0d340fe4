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
The same holds for the segmented scan (a sequence of n >= 40 chunks cut into
k = min(K, n / 20) segments, at least 2, at seg_bound) and its chain and combine passes,
whose chunk workgroups are numbered over the later segments' chunks of all sequences: with
valid cu_seqlens every later-segment chunk of every (sequence, head) is combined by exactly
one workgroup within the grid bound, the first segments and the combine together write every
output row once, and every boundary state is written (once) before it is read.
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
    """The two-segment scan's prep order (K = 2): dispatch slot i -> chunk group."""
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


# ------------------------------------------------------------------ segmented scan
SEG_MIN_CHUNKS, SEG_MULTI_CHUNKS, SEG_PER_CHUNKS, SEG_MAX = 40, 80, 20, 8


def seg_segments(H, n, T, cus=256, C=64, d=128):
    """K, the most segments a sequence is cut into (bf16, d = 64 or 128, C = 64), or 0."""
    units = n * H
    if not (units > 0 and n <= 64 and T >= n * SEG_MIN_CHUNKS * C and d in (64, 128)):
        return 0
    k = cus // (units * (d // 16))
    if k < 2:
        return 0
    return seg_count(min(-(-T // C), SEG_MAX * SEG_PER_CHUNKS), min(k, SEG_MAX))


def seg_count(nch, kmax):
    if nch < SEG_MIN_CHUNKS or kmax < 2:
        return 1
    if nch < SEG_MULTI_CHUNKS:
        return 2
    return min(kmax, nch // SEG_PER_CHUNKS)


def seg_first_64(k):
    d = 29 * k + 6
    return (2240 + d // 2) // d


def cdiv_int(a, b):
    """C integer division (truncates toward zero), as the device code divides."""
    q = abs(a) // abs(b)
    return q if (a >= 0) == (b >= 0) else -q


def seg_bound(c0, c1, j, k):
    if j <= 0:
        return c0
    if j >= k:
        return c1
    b1 = c0 + cdiv_int((c1 - c0) * seg_first_64(k) + 63, 64)
    return b1 + cdiv_int((j - 1) * (c1 - b1), k - 1)


def test_seg_split_rules():
    assert [seg_first_64(k) for k in range(1, 9)] == [64, 35, 24, 18, 15, 12, 11, 9]
    for kmax in range(2, SEG_MAX + 1):
        for nch in range(0, 3000):
            k = seg_count(nch, kmax)
            assert (k == 1) == (nch < SEG_MIN_CHUNKS) and k <= kmax
            assert k <= 2 or nch >= SEG_MULTI_CHUNKS
            b = [seg_bound(5, 5 + nch, j, k) for j in range(k + 1)]
            assert b[0] == 5 and b[-1] == 5 + nch
            assert all(b[j] < b[j + 1] for j in range(k)) or nch == 0  # no empty segment
            if k == 2:  # the two-segment split at ceil(35 n / 64)
                assert b[1] == 5 + (nch * 35 + 63) // 64
            later = nch - (b[1] - b[0]) if k > 1 else 0
            assert later <= (nch * (64 - seg_first_64(kmax)) + 63) // 64


def seg_scan_touch(cu, n, T, H, C, kmax=2):
    """Every segment's workgroups: (sequence, head, units read, units written, rows written,
    boundary slots written). A later segment's workgroup writes its chunks' zero-state
    outputs over their U and their L, both in the unit's own workspace slots, no token rows,
    and its transition and Delta at boundary slot (segment - 1)."""
    mc = max_chunks(T, n, C)
    excl, incl = seq_table(cu, n, C)
    out = []
    for s in range(n):
        c0, c_end = excl[s], min(incl[s], mc)
        k = seg_count(c_end - c0, kmax)
        t_begin, t_end = cu[s], min(cu[s + 1], T)

        def rows_of(cc):
            tok0 = t_begin + (cc - c0) * C
            ln = min(C, t_end - tok0)
            return [tok0 + i for i in range(C) if i < ln and tok0 + i >= 0]

        for h in range(H):
            for j in range(k):
                lo, hi = seg_bound(c0, c_end, j, k), seg_bound(c0, c_end, j + 1, k)
                clast = hi - 1
                rd, wr, rows = [], [], []
                for c in range(lo, hi):
                    rd += [cc * H + h for cc in {c, min(c + 1, clast)}]
                    if j > 0:
                        wr.append(c * H + h)
                    else:
                        rows += rows_of(c)
                # P and Delta of segment j, or (first segment of a split sequence) S_1
                slots = ([("P", (j - 1) * n * H + s * H + h)] if j > 0 else
                         [("S", s * H + h)] if k > 1 else [])
                out.append((s, h, rd, wr, rows, slots))
    return out


def combine_touch(cu, n, T, H, C, kmax=2):
    """Chunk workgroups of the combine: (sequence, head, chunk, unit, rows written, the
    boundary slot of S_j read)."""
    mc = max_chunks(T, n, C)
    excl, incl = seq_table(cu, n, C)
    c1l = [min(x, mc) for x in incl]
    ks = [seg_count(c1l[s] - excl[s], kmax) for s in range(n)]
    nbl = [max(0, c1l[s] - seg_bound(excl[s], c1l[s], 1, ks[s])) if ks[s] > 1 else 0
           for s in range(n)]
    pin, run = [], 0
    for x in nbl:
        run += x
        pin.append(run)
    pex = [pin[s] - nbl[s] for s in range(n)]
    bound = (mc * (64 - seg_first_64(kmax)) + 63) // 64 + 1
    out = []
    for b in range(bound * H):
        h, kc = b % H, b // H
        hits = [s for s in range(n) if pex[s] <= kc < pin[s]]
        if not hits:
            continue
        s = hits[0]
        k = ks[s]
        c = seg_bound(excl[s], c1l[s], 1, k) + (kc - pex[s])
        j = 1
        while j + 1 < k and seg_bound(excl[s], c1l[s], j + 1, k) <= c:
            j += 1
        tok0 = cu[s] + (c - excl[s]) * C
        ln = min(C, min(cu[s + 1], T) - tok0)
        rows = [tok0 + i for i in range(C) if i < ln and tok0 + i >= 0]
        out.append((s, h, c, c * H + h, rows, ("S", (j - 1) * n * H + s * H + h)))
    return out


def chain_slots(cu, n, T, H, C, kmax):
    """Boundary slots ("P": transition and Delta, "S": S_j) that the chain pass reads
    (P_j, S_j for j < k - 1) and writes (S_{j+1}) and that the combine's state rows read
    (j = k - 1), per (sequence, head)."""
    mc = max_chunks(T, n, C)
    excl, incl = seq_table(cu, n, C)
    out = []
    for s in range(n):
        k = seg_count(min(incl[s], mc) - excl[s], kmax)
        for h in range(H):
            u = s * H + h
            rd = [(b, (j - 1) * n * H + u) for j in range(1, k) for b in "PS"]
            wr = [("S", j * n * H + u) for j in range(1, k - 1)]
            out.append((rd, wr))
    return out


def seg_grid_cover(n, H, kmax, NVT=8):
    """The segmented scan kernel's workgroup -> (segment, unit, value tile) map (NVT value
    tiles of 16 columns per head: d / 16)."""
    units = n * H
    grid = (kmax * units + 7) // 8 * 8 * NVT
    seen = []
    for b in range(grid):
        xcd, jj = b & 7, b >> 3
        vu, vt = (jj // NVT) * 8 + xcd, jj % NVT
        if vu >= kmax * units:
            continue
        seen.append((vu // units, vu % units, vt))
    return seen


def test_seg_grid_covers_every_segment_tile_once():
    for d in (64, 128):
        NT = d // 16
        for n in (1, 2, 3, 5, 8):
            for H in (1, 2, 3, 4, 8, 16):
                kmax = seg_segments(H, n, 10 ** 7, d=d)
                if kmax == 0:
                    continue
                seen = seg_grid_cover(n, H, kmax, NT)
                assert sorted(seen) == [(s, u, v) for s in range(kmax) for u in range(n * H)
                                        for v in range(NT)]
                # the chain pass: every (unit, 16-column slice) once, a unit's slices on one
                # XCD
                grid = (n * H + 7) // 8 * 8 * NT
                cover = {}
                for b in range(grid):
                    xcd, jj = b & 7, b >> 3
                    u, tv = (jj // NT) * 8 + xcd, jj % NT
                    if u < n * H:
                        assert (u, tv) not in cover
                        cover[(u, tv)] = xcd
                assert sorted(cover) == [(u, tv) for u in range(n * H) for tv in range(NT)]
                assert all(len({cover[(u, tv)] for tv in range(NT)}) == 1 for u in range(n * H))
    # the 16-head call: two segments, on all 256 CUs
    assert seg_segments(16, 1, 8192) == 2 and len(seg_grid_cover(1, 16, 2)) == 256
    assert seg_segments(8, 1, 8192) == 4 and seg_segments(4, 1, 8192) == 6
    assert seg_segments(4, 1, 12000) == 8 and seg_segments(4, 1, 5057) == 4
    assert seg_segments(4, 1, 5056) == 2  # 79 chunks: no sequence takes more than 2
    assert seg_segments(3, 3, 20000) == 3  # 9 units: K = 3
    # d = 64: 4 value tiles per head, so twice the units fit
    assert seg_segments(16, 2, 20000, d=64) == 2 and seg_segments(32, 1, 8192, d=64) == 2
    assert seg_segments(16, 1, 8192, d=64) == 4 and seg_segments(33, 1, 8192, d=64) == 0
    assert seg_segments(4, 1, 8192, d=32) == 0
    assert seg_segments(17, 1, 8192) == 0 and seg_segments(16, 1, 40 * 64 - 1) == 0
    # K only bounds the segment count: every sequence of a call gets what the CUs allow
    for T in range(2560, 20000, 97):
        kcu = 256 // (2 * 8)
        for nch in range(0, -(-T // 64) + 1):
            assert seg_count(nch, seg_segments(2, 1, T)) == seg_count(nch, min(kcu, SEG_MAX))


def _long_cu(rng, n):
    lens = [rng.choice([0, rng.randrange(1, 900), rng.randrange(1000, 9000)]) for _ in range(n)]
    cu = [0]
    for L in lens:
        cu.append(cu[-1] + L)
    return cu


@pytest.mark.parametrize("seed", range(8))
def test_segmented_exact_cover(seed):
    rng = random.Random(100 + seed)
    n, H, C = rng.randrange(1, 17), rng.choice([1, 2, 4]), 64
    kmax = rng.choice([2, 3, 4, 8])
    cu = _long_cu(rng, n)
    T = cu[-1]
    excl, incl = seq_table(cu, n, C)
    nslot = (kmax - 1) * n * H
    written = {}
    bslots = []
    for s, h, rd, wr, rows, slots in seg_scan_touch(cu, n, T, H, C, kmax):
        assert set(rd) <= {c * H + h for c in range(excl[s], incl[s])}
        assert all(0 <= x < nslot for _, x in slots)
        bslots += slots
        for r in rows:
            written[(r, h)] = written.get((r, h), 0) + 1
    chain = chain_slots(cu, n, T, H, C, kmax)
    chain_written = [x for _, wr in chain for x in wr]
    writes = bslots + chain_written
    assert len(writes) == len(set(writes))  # each boundary slot has one writer
    comb = combine_touch(cu, n, T, H, C, kmax)
    seen = set()
    for s, h, c, u, rows, sl in comb:
        k = seg_count(incl[s] - excl[s], kmax)
        assert seg_bound(excl[s], incl[s], 1, k) <= c < incl[s]
        assert sl in writes  # S_j of the chunk's segment: the first segment's or the chain's
        assert (s, h, c) not in seen
        seen.add((s, h, c))
        for r in rows:
            written[(r, h)] = written.get((r, h), 0) + 1
    expect = set()
    for s in range(n):
        k = seg_count(incl[s] - excl[s], kmax)
        if k > 1:
            expect |= {(s, h, c) for h in range(H)
                       for c in range(seg_bound(excl[s], incl[s], 1, k), incl[s])}
    assert seen == expect
    assert written == {(r, h): 1 for r in range(T) for h in range(H)}
    done = set(bslots)  # the scan's writes, then the chain's steps in order
    for rd, wr in chain:
        assert all(0 <= x < nslot for _, x in rd + wr)
        for j, x in enumerate(wr):  # step j + 1 reads P_{j+1} and S_{j+1}, writes S_{j+2}
            assert ("P", rd[2 * j][1]) in done and ("S", rd[2 * j + 1][1]) in done
            done.add(x)
        assert set(rd) <= done  # the combine's state rows: the last P and S_{k-1}


@pytest.mark.parametrize("cu", BROKEN)
@pytest.mark.parametrize("kmax", [2, 8])
def test_segmented_broken_cu_seqlens_stay_in_bounds(cu, kmax):
    n, H, C = len(cu) - 1, 3, 64
    for T in (400, 1000, 5000):
        mc = max_chunks(T, n, C)
        nslot = (kmax - 1) * n * H
        for _, _, rd, wr, rows, slots in seg_scan_touch(cu, n, T, H, C, kmax):
            assert all(0 <= u < mc * H for u in rd + wr)
            assert all(0 <= r < T for r in rows) and all(0 <= x < nslot for _, x in slots)
        for _, _, _, u, rows, sl in combine_touch(cu, n, T, H, C, kmax):
            assert 0 <= u < mc * H and all(0 <= r < T for r in rows) and 0 <= sl[1] < nslot
        for rd, wr in chain_slots(cu, n, T, H, C, kmax):
            assert all(0 <= x < nslot for _, x in rd + wr)


def test_segmented_random_broken_cu_seqlens_stay_in_bounds():
    rng = random.Random(11)
    for _ in range(200):
        n, H, C = rng.randrange(1, 9), rng.choice([1, 2, 5]), 64
        kmax = rng.choice([2, 3, 5, 8])
        T = rng.randrange(0, 6000)
        cu = [rng.randrange(-500, 7000) for _ in range(n + 1)]
        mc = max_chunks(T, n, C)
        nslot = (kmax - 1) * n * H
        for _, _, rd, wr, rows, slots in seg_scan_touch(cu, n, T, H, C, kmax):
            assert all(0 <= u < mc * H for u in rd + wr) and all(0 <= r < T for r in rows)
            assert all(0 <= x < nslot for _, x in slots)
        for _, _, _, u, rows, sl in combine_touch(cu, n, T, H, C, kmax):
            assert 0 <= u < mc * H and all(0 <= r < T for r in rows) and 0 <= sl[1] < nslot
        for rd, wr in chain_slots(cu, n, T, H, C, kmax):
            assert all(0 <= x < nslot for _, x in rd + wr)


def seg_prep_group_k(i, NG, k):
    """The prep order of a call cut into k > 2 segments: slot i -> chunk group (the device's
    bisection over passes, written out)."""
    b = [seg_bound(0, NG, min(s, k), k) for s in range(SEG_MAX + 1)]

    def before(m):
        return sum(min(b[s + 1] - b[s], m) for s in range(SEG_MAX))

    r = NG - 1 - i
    lo, hi = 0, NG
    while hi - lo > 1:
        mid = (lo + hi) >> 1
        if before(mid) <= r:
            lo = mid
        else:
            hi = mid
    t, grp = r - before(lo), i
    for s in range(SEG_MAX):
        has = b[s + 1] - b[s] > lo
        if has and t == 0:
            grp = b[s] + lo
        t -= 1 if has else 0
    return grp


def test_seg_prep_order_is_a_permutation():
    for NG in range(1, 200):
        assert sorted(seg_prep_group(i, NG) for i in range(NG)) == list(range(NG))
        for k in range(1, SEG_MAX + 1):
            order = [seg_prep_group_k(i, NG, k) for i in range(NG)]
            assert sorted(order) == list(range(NG))
            if k == 2:  # the same order as the two-segment form
                assert order == [seg_prep_group(i, NG) for i in range(NG)]
            # the last slots go to each segment's first group, first segment first
            firsts = [g for g in (seg_bound(0, NG, s, k) for s in range(k)) if g < NG]
            firsts = sorted(set(firsts))
            assert order[::-1][:len(firsts)] == firsts


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
