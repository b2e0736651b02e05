"""The blocked factorisation's schedule, checked on the host through
chol_potrf_plan (the list of operations chol_potrf enqueues, with the joins
between its two streams).  Two properties, on cells of g x g elements
(g = gcd(nb, 128), so every operation covers whole cells):

* panel bookkeeping: every lower cell is brought over from A exactly once,
  before anything else touches it (by the copy, or by the far-triangle
  update that reads A, which must then be the cell's first update); every
  trailing-update operation subtracts each panel's product from a cell at
  most once, each tile column holds exactly the products of the panels left
  of it when its diagonal tile is factored and when its panel is solved, and
  at the end every lower cell holds exactly the panels left of its tile
  column;
* ordering: any two operations that touch the same data (a cell of the
  matrix or an inverse slot), at least one of them writing it, are ordered
  by stream order or by a join.

No GPU call is made."""
import math

import pytest

dc = pytest.importorskip("differentiable_cholesky_amd")
from differentiable_cholesky_amd import _lib  # noqa: E402

COPY, DIAG, PANEL, UPDATE, TRI, JOIN, ZERO = range(7)
CHAIN, WIDE = 0, 1


def _cells(n, g):
    return (n + g - 1) // g


def _mask(C, rows, cols, lower_only):
    """Bitmask of cells (a, b) with a in rows, b in cols (cell ranges)."""
    m = 0
    for a in range(*rows):
        for b in range(*cols):
            if not lower_only or a >= b:
                m |= 1 << (a * C + b)
    return m


def _check(n, nb, plan=None, slots=480):
    if plan is None:
        plan = dc.chol_potrf_plan(n, nb, copy=True, slots=slots)
    nbe = nb or 128
    g = math.gcd(nbe, 128)
    C = _cells(n, g)
    cell = lambda x: (x + g - 1) // g          # first cell at or after element x (x aligned)
    K = (n + nbe - 1) // nbe
    SLOT = [1 << (C * C), 1 << (C * C + 1)]   # the two inverse slots as extra resources
    lower_all = _mask(C, (0, C), (0, C), True)

    applied = {}                               # lower cell -> bitmask of panels applied
    loaded = set()                             # lower cells that hold A's values (or later ones)
    if not any(int(row[0]) == COPY for row in plan):
        loaded = {(a, b) for a in range(C) for b in range(a + 1)}   # in place: L is A
    clock = [[0, 0], [0, 0]]                   # per stream: known positions of (chain, wide)
    pos = [0, 0]
    done = []                                  # (stream, position, clock, reads, writes)

    def col_complete(k):
        k0 = k * nbe
        for b in range(cell(k0), cell(min(k0 + nbe, n))):
            for a in range(b, C):
                assert (a, b) in loaded, (n, nb, "tile column", k, "cell never loaded from A", (a, b))
                got = applied.get((a, b), 0)
                assert got == (1 << k) - 1, (n, nb, "tile column", k, "cell", (a, b), bin(got))

    def apply(rows_c, cols_c, f, np_, lower_rule, from_a=False):
        pm = ((1 << np_) - 1) << f
        for a in range(*rows_c):
            for b in range(*cols_c):
                if a >= b and lower_rule(a, b):
                    if from_a:
                        assert (a, b) not in loaded, (n, nb, "cell loaded from A twice", (a, b))
                        loaded.add((a, b))
                    assert (a, b) in loaded, (n, nb, "cell updated before it holds A", (a, b))
                    got = applied.get((a, b), 0)
                    assert not got & pm, (n, nb, "panel applied twice", (a, b), f, np_)
                    applied[(a, b)] = got | pm

    for row in plan:
        kind, stream, k, c, w, f, np_, t0, tn, slot = (int(x) for x in row)
        reads = writes = 0
        if kind == JOIN:
            other = 1 - stream
            clock[stream][other] = max(clock[stream][other], pos[other])
            clock[stream] = [max(x, y) for x, y in zip(clock[stream], clock[other])]
            clock[stream][other] = max(clock[stream][other], pos[other])
            continue
        if kind == COPY:
            assert 0 < w <= n, (n, nb, "copy width", w)
            for a in range(C):
                for b in range(min(a + 1, cell(w))):
                    assert (a, b) not in loaded, (n, nb, "cell loaded from A twice", (a, b))
                    loaded.add((a, b))
            writes = _mask(C, (0, C), (0, cell(w)), True)
        elif kind == ZERO:
            writes = _mask(C, (0, C), (0, C), False) & ~_mask(C, (0, C), (0, C), True) | \
                sum(1 << (a * C + a) for a in range(C))
        elif kind == DIAG:
            k0 = k * nbe
            kb = min(nbe, n - k0)
            col_complete(k)
            assert (slot >= 0) == (k0 + kb < n), (n, nb, "inverse slot", k, slot)
            writes = _mask(C, (cell(k0), cell(k0 + kb)), (cell(k0), cell(k0 + kb)), True)
            if slot >= 0:
                assert slot == k % 2
                writes |= SLOT[slot]
        elif kind == PANEL:
            k0 = k * nbe
            r0 = k0 + min(nbe, n - k0)
            col_complete(k)
            assert slot == k % 2
            writes = _mask(C, (cell(r0), C), (cell(k0), cell(r0)), False)
            reads = SLOT[slot]
        elif kind == UPDATE:
            assert f + np_ <= K and c % nbe == 0 and (f + np_) * nbe <= c
            rows_c, cols_c = (cell(c), C), (cell(c), cell(min(c + w, n)))
            apply(rows_c, cols_c, f, np_, lambda a, b: True)
            writes = _mask(C, rows_c, cols_c, True)
            reads = _mask(C, rows_c, (cell(f * nbe), cell((f + np_) * nbe)), False)
        elif kind == TRI:
            assert f + np_ <= K and c % nbe == 0 and (f + np_) * nbe <= c
            M = n - c
            TI = (M + 127) // 128
            tiles = [(I, J) for I in range(TI) for J in range(I + 1)]
            assert 0 <= t0 and t0 + tn <= len(tiles) and tn > 0
            assert slot in (-1, 1), (n, nb, "far-triangle source", slot)
            for I, J in tiles[t0:t0 + tn]:
                rows_c = (cell(c + 128 * I), cell(min(c + 128 * I + 128, n)))
                cols_c = (cell(c + 128 * J), cell(min(c + 128 * J + 128, n)))
                apply(rows_c, cols_c, f, np_, lambda a, b: True, from_a=slot == 1)
                writes |= _mask(C, rows_c, cols_c, True)
            reads = _mask(C, (cell(c), C), (cell(f * nbe), cell((f + np_) * nbe)), False)
        else:
            raise AssertionError(f"unknown operation kind {kind}")
        pos[stream] += 1
        me = (stream, pos[stream], list(clock[stream]), reads, writes)
        clock[stream][stream] = pos[stream]
        for (s2, p2, _, r2, w2) in done:
            if (writes & (r2 | w2)) or (reads & w2):
                ordered = s2 == stream or me[2][s2] >= p2
                assert ordered, (n, nb, "unordered conflict", (s2, p2), (stream, pos[stream], kind))
        done.append(me)

    for a in range(C):
        for b in range(a + 1):
            assert (a, b) in loaded, (n, nb, "final: cell never loaded from A", (a, b))
            want = (1 << ((b * g) // nbe)) - 1
            assert applied.get((a, b), 0) == want, (n, nb, "final", (a, b))


@pytest.mark.parametrize("n,nb", [(65, 32), (100, 32), (127, 64), (128, 64), (129, 128), (200, 64),
                                  (255, 128), (256, 128), (300, 16), (384, 128), (513, 128), (700, 64),
                                  (1000, 0), (1030, 32), (1300, 128), (2100, 96)])
@pytest.mark.parametrize("slots", [0, 5, 480])
def test_forward_schedule(n, nb, slots):
    # slots 0: equal parts; 5: far triangles cut at multiples of 5 tiles, with
    # empty parts where a group has fewer rounds than parts; 480: MI355X
    _check(n, nb, slots=slots)


def test_forward_schedule_benchmark_size():
    # the schedule the n = 16384 benchmark runs (128 tile columns)
    _check(16384, 128)


def test_far_triangle_cut_at_whole_rounds():
    # each group's far triangle: parts in order, covering its tiles once, and
    # every part but the group's last one a whole number of rounds
    slots = 480
    plan = dc.chol_potrf_plan(16384, 128, copy=True, slots=slots)
    groups = {}
    for row in plan:
        if row[0] == TRI:
            groups.setdefault((row[3], row[5], row[6]), []).append((row[7], row[8]))
    assert groups
    for (c, f, np_), parts in groups.items():
        T = (16384 - c + 127) // 128
        tiles = T * (T + 1) // 2
        assert parts[0][0] == 0 and sum(tn for _, tn in parts) == tiles
        for (t0, tn), (t1, _) in zip(parts, parts[1:]):
            assert t0 + tn == t1
        for t0, tn in parts[:-1]:
            assert tn % slots == 0, (c, parts)
        assert len(parts) <= 4


def _mutants(plan):
    import numpy as np
    kinds = plan[:, 0]
    out = []
    # the join before the second panel solve dropped: the solve would read an
    # inverse slot the chain stream may still be writing
    joins = [i for i in range(len(plan) - 1) if kinds[i] == JOIN and kinds[i + 1] == PANEL]
    out.append(("join dropped", np.delete(plan, joins[1], axis=0)))
    # one part of a far triangle dropped: its tiles miss their group's panels
    tri = [i for i in range(len(plan)) if kinds[i] == TRI]
    out.append(("triangle part dropped", np.delete(plan, tri[len(tri) // 2], axis=0)))
    # an update run twice: its panels subtracted twice
    upd = [i for i in range(len(plan)) if kinds[i] == UPDATE]
    out.append(("update doubled", np.insert(plan, upd[3], plan[upd[3]], axis=0)))
    # an update with one panel too few
    bad = plan.copy()
    i = next(i for i in upd if plan[i, 6] > 1)
    bad[i, 5] += 1
    bad[i, 6] -= 1
    out.append(("panel missing", bad))
    # the copy one tile column short: the first far triangle's tiles are
    # read from A, but that column's cells are never brought over
    bad = plan.copy()
    assert bad[0, 0] == COPY
    bad[0, 4] -= nb_of(plan)
    out.append(("copy short", bad))
    # a later far-triangle part that reads A: it would discard earlier updates
    bad = plan.copy()
    late = [i for i in tri if plan[i, 9] != 1]
    bad[late[0], 9] = 1
    out.append(("late part reads A", bad))
    return out


def nb_of(plan):
    return int(next(row[4] for row in plan if row[0] == UPDATE and row[6] == 1))


@pytest.mark.parametrize("n,nb", [(1300, 128), (2100, 96)])
def test_schedule_check_catches_planted_mistakes(n, nb):
    # the checker must reject schedules with a planted mistake
    for name, bad in _mutants(dc.chol_potrf_plan(n, nb, copy=True)):
        with pytest.raises(AssertionError):
            _check(n, nb, bad)
        assert name


def test_first_far_triangle_read_from_a():
    # with A apart from L only the columns left of the first far triangle are
    # copied; the first group's parts read A.  In place (copy=False), nothing
    # reads A.
    for n, nb in [(16384, 128), (2100, 96)]:
        plan = dc.chol_potrf_plan(n, nb, copy=True)
        assert plan[0, 0] == COPY and plan[0, 4] == 5 * nb
        tri = plan[plan[:, 0] == TRI]
        first = tri[:, 5] == 0                    # the first group's parts: panel 0 alone
        assert first.any() and (tri[first, 9] == 1).all() and (tri[~first, 9] == -1).all()
        inplace = dc.chol_potrf_plan(n, nb, copy=False)
        assert (inplace[:, 0] != COPY).all() and (inplace[inplace[:, 0] == TRI][:, 9] == -1).all()
        _check(n, nb, inplace)
    plan = dc.chol_potrf_plan(600, 128, copy=True)     # no far triangle: everything copied
    assert plan[0, 4] == 600 and not (plan[:, 0] == TRI).any()


def test_plan_argument_errors():
    assert _lib.lib.chol_potrf_plan(-1, 0, 1, 480, None, 0) == -1
    assert _lib.lib.chol_potrf_plan(100, 129, 1, 480, None, 0) == -1
    assert _lib.lib.chol_potrf_plan(100, -1, 1, 480, None, 0) == -1
    assert _lib.lib.chol_potrf_plan(100, 0, 1, -1, None, 0) == -1
    assert _lib.lib.chol_potrf_plan(0, 0, 1, 480, None, 0) == 0
