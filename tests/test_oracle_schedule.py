"""Pins for the schedule simulator (CPU only): the pages' closed forms and
printed table values, plus an independent rule checker that re-derives the
greedy rules and the dependencies from the simulator's op list alone."""
import os
from fractions import Fraction

import pytest

from oracle import schedule as S
from oracle.schedule import simulate

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
COSTS = [(1, 1, 1), (1, 2, 0), (2, 3, 1), (3, 5, 2)]


def _rows(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return [ln.split() for ln in f if ln.strip() and not ln.startswith("#")]


@pytest.mark.parametrize("kind", ["gpipe", "1f1b"])
def test_atomic_schedules_closed_forms(kind):
    """[Guide]: GPipe and 1F1B bubble = (p-1)/(m+p-1) of the makespan, i.e.
    (p-1)/m of the busy time, for every stage."""
    for costs in COSTS:
        for p in range(2, 13):
            for m in range(1, 49):
                r = simulate(kind, p, m, costs=costs)
                for i in range(p):
                    assert r.idle_over_makespan(i) == Fraction(p - 1, m + p - 1)
                    assert r.idle_over_busy(i) == Fraction(p - 1, m)


def test_printed_1f1b_table():
    for p, m, pct in _rows("guide_1f1b_bubble_table.txt"):
        r = simulate("1f1b", int(p), int(m))
        assert round(float(r.idle_over_makespan(0)) * 100, 1) == float(pct)


def test_printed_closed_form_values():
    for kind, p, m, num, den, what in _rows("guide_closed_forms.txt"):
        r = simulate(kind, int(p), int(m))
        got = r.idle_over_makespan(0) if what == "idle_over_makespan" else r.idle_over_busy(0)
        assert got == Fraction(int(num), int(den))


def test_1f1b_peak_memory_bounded_by_p():
    """[Guide] "2. The 1F1B Schedule": peak activation memory <= p."""
    for p in range(2, 10):
        for m in range(1, 30):
            r = simulate("1f1b", p, m)
            for i in range(p):
                assert r.stats[i].peak_active == min(p - i, m)


def test_zb_2p_bubble_closed_form_and_zero_in_window():
    """[Guide] "2. Zero-Bubble ZB-1F1B Bubble Duration" and "ZB-2p": for
    m >= 2p the bubble is (p-1)/(3m) of the busy time and ZB-2p leaves no
    idle time between a stage's first and last op."""
    for p in range(2, 13):
        for m in range(2 * p, 49):
            r = simulate("zb", p, m, M=2 * p)
            for i in range(p):
                assert r.idle_over_busy(i) == Fraction(p - 1, 3 * m)
                assert r.stats[i].in_window_idle == 0


def test_zb_makespan_equals_lower_bound_at_2p():
    r = simulate("zb", 8, 16, M=16)
    assert r.makespan == 7 * 1 + 16 * 3 == 55


def _check_valid_and_greedy(r):
    """Independent checker: dependencies, no overlap, memory limit, and for
    zb the greedy priority rule at every decision instant."""
    p, m, M = r.p, r.m, r.M
    cF, cB, cW = r.costs
    end = {}
    start = {}
    for i in range(p):
        for o in r.ops[i]:
            end[(o.type, i, o.mb)] = o.end
            start[(o.type, i, o.mb)] = o.start
    for i in range(p):
        ops = r.ops[i]
        assert sorted((o.type, o.mb) for o in ops) == sorted(
            [(t, j) for t in "FBW" for j in range(m)])
        for a, b in zip(ops, ops[1:]):
            assert a.end <= b.start
        for o in ops:
            if o.type == "F" and i > 0:
                assert start[("F", i, o.mb)] >= end[("F", i - 1, o.mb)]
            if o.type == "B":
                assert o.start >= end[("F", i, o.mb)]
                if i < p - 1:
                    assert o.start >= end[("B", i + 1, o.mb)] if r.kind == "zb" else True
            if o.type == "W":
                assert o.start >= end[("B", i, o.mb)]
    if r.kind != "zb":
        return
    for i in range(p):
        active = 0
        ops = r.ops[i]
        decision_times = sorted({0} | {e for (t, s, j), e in end.items()})
        k = 0
        free_at = 0
        for t in decision_times:
            if t < free_at:
                continue
            # state of this stage at time t, from the op list only
            fdone = lambda s, j: end.get(("F", s, j), 1 << 60) <= t
            bdone = lambda s, j: end.get(("B", s, j), 1 << 60) <= t
            started = {(o.type, o.mb) for o in ops if o.start < t}
            act = sum(1 for o in ops if o.start < t and o.type == "F") - \
                sum(1 for o in ops if o.start < t and o.type == "W")
            readyB = [j for j in range(m) if ("B", j) not in started and fdone(i, j)
                      and (i == p - 1 or bdone(i + 1, j))]
            readyF = [j for j in range(m) if ("F", j) not in started and (i == 0 or fdone(i - 1, j))]
            readyW = [j for j in range(m) if ("W", j) not in started and bdone(i, j)]
            if readyB:
                want = ("B", min(readyB))
            elif readyF and act < M:
                want = ("F", min(readyF))
            elif readyW:
                want = ("W", min(readyW))
            else:
                want = None
            at_t = [o for o in ops if o.start == t]
            if want is None:
                assert not at_t
            else:
                assert len(at_t) == 1 and (at_t[0].type, at_t[0].mb) == want, (i, t, want, at_t)
                free_at = at_t[0].end
        assert max(0, act) <= M
        assert r.stats[i].peak_active <= M


@pytest.mark.parametrize("costs", [(1, 1, 1), (2, 3, 1), (3, 2, 2), (1, 1, 3)])
def test_zb_greedy_rule_checker(costs):
    for p in (2, 3, 4, 6):
        for m in (1, 3, 2 * p, 2 * p + 3):
            for M in range(p, 2 * p + 1):
                _check_valid_and_greedy(simulate("zb", p, m, M=M, costs=costs))


def test_atomic_schedules_valid():
    for kind in ("gpipe", "1f1b"):
        for p in (2, 5):
            for m in (1, 4, 9):
                _check_valid_and_greedy(simulate(kind, p, m, costs=(2, 3, 1)))


def test_1f1b_stage_order_matches_figure():
    """[Guide] "Conventional 1F1B Pipeline Schedule" figure (p = 4)."""
    r = simulate("1f1b", 4, 8)
    fig = {0: "F0 F1 F2 F3 B0 F4 B1 F5 B2", 1: "F0 F1 F2 B0 F3 B1 F4 B2",
           2: "F0 F1 B0 F2 B1 F3 B2", 3: "F0 B0 F1 B1 F2 B2"}
    for i, want in fig.items():
        got = " ".join(f"{t}{j}" for t, j in r.order(i) if t != "W")
        assert got.startswith(want)


def test_zb_memory_limit_respected_and_deadlock_free():
    for p in range(2, 9):
        for M in range(p, 2 * p + 1):
            r = simulate("zb", p, 3 * p, M=M)
            assert all(s.peak_active <= M for s in r.stats)


# ---------------------------------------------------- several iterations ---

ITER_CASES = [(8, 16, 16, (1, 1, 1), 1, 3), (4, 8, 8, (2, 2, 2), 1, 2), (4, 8, 8, (1, 1, 1), 3, 2),
              (8, 24, 16, (1, 1, 1), 1, 2), (4, 6, 8, (1, 1, 1), 1, 2), (8, 16, 8, (1, 1, 1), 1, 2),
              (8, 16, 16, (63, 84, 63), 1, 3), (8, 16, 12, (2, 3, 2), 2, 3), (3, 2, 3, (1, 1, 1), 1, 3),
              (2, 1, 1, (1, 1, 1), 1, 3)]


def _check_iteration_dependencies(r):
    """Independent of the simulator's bookkeeping: every op once, no overlap
    on a stage, every dependency ended before its op starts, the memory
    limit never exceeded."""
    p, m, n = r.p, r.m, r.n_iter
    G = n * m
    # the gradient a stage sends upstream: after B (zero bubble), after the
    # whole backward B + W (1F1B, M = 0)
    down = "W" if r.M == 0 else "B"
    end = {}
    for i in range(p):
        seen = set()
        last = 0
        for o in r.ops[i]:
            assert o.start >= last, ("overlap", i, o)
            last = o.end
            assert (o.type, o.mb) not in seen
            seen.add((o.type, o.mb))
            end[(o.type, i, o.mb)] = (o.start, o.end)
        assert seen == ({(t, g) for t in "FBW" for g in range(G)} | {("O", it) for it in range(n)})
    for i in range(p):
        active = 0
        for o in r.ops[i]:
            s = o.start
            if o.type == "F":
                g, it = o.mb, o.mb // m
                if i > 0:
                    assert end[("F", i - 1, g)][1] <= s
                if it > 0:
                    assert end[("O", i, it - 1)][1] <= s
                active += 1
                assert r.M == 0 or active <= r.M   # M = 0: 1F1B, no memory limit
            elif o.type == "B":
                assert end[("F", i, o.mb)][1] <= s
                if i < p - 1:
                    assert end[(down, i + 1, o.mb)][1] <= s
            elif o.type == "W":
                assert end[("B", i, o.mb)][1] <= s
                active -= 1
            else:
                for j in range(m):
                    assert end[("W", i, o.mb * m + j)][1] <= s
        for g in range(G):
            if i > 0:
                assert r.arrive_f[i][g] == end[("F", i - 1, g)][1]
            if i < p - 1:
                assert r.arrive_b[i][g] == end[(down, i + 1, g)][1]


ITER_KIND_CASES = [("zb",) + c for c in ITER_CASES] + [("1f1b", p, m, 0, costs, c_opt, n) for p, m, _, costs, c_opt, n in ITER_CASES]


@pytest.mark.parametrize("kind,p,m,M,costs,c_opt,n", ITER_KIND_CASES)
def test_iterations_dependencies_and_memory(kind, p, m, M, costs, c_opt, n):
    _check_iteration_dependencies(S.simulate_iterations(p, m, M, costs, n, c_opt, kind=kind))


@pytest.mark.parametrize("kind,p,m,M,costs,c_opt,n", ITER_KIND_CASES)
def test_one_iteration_is_the_single_iteration_schedule(kind, p, m, M, costs, c_opt, n):
    r = S.simulate_iterations(p, m, M, costs, 1, c_opt, kind=kind)
    single = S.simulate(kind, p, m, M, costs)
    for i in range(p):
        got = [(o.type, o.mb, o.start, o.end) for o in r.ops[i]]
        last_w = single.ops[i][-1].end
        assert got == [(o.type, o.mb, o.start, o.end) for o in single.ops[i]] + [("O", 0, last_w, last_w + c_opt)]


@pytest.mark.parametrize("kind,p,m,M,costs,c_opt,n", ITER_KIND_CASES)
def test_iterations_repeat_with_stage0_period(kind, p, m, M, costs, c_opt, n):
    """Every stage's iteration k is its iteration 0 shifted by k * T, with
    T = stage 0's single-iteration end + c_opt (stage 0 starts iteration k+1
    right after its optimizer step, and nothing else gates it), so the
    makespan is (n-1) T + makespan(1) + c_opt."""
    r = S.simulate_iterations(p, m, M, costs, n, c_opt, kind=kind)
    single = S.simulate(kind, p, m, M, costs)
    T = single.stats[0].last_end + c_opt
    for i in range(p):
        base = [(o.type, o.mb, o.start, o.end) for o in single.ops[i]]
        for it in range(n):
            got = [(o.type, o.mb - m * it, o.start - it * T, o.end - it * T) for o in r.ops[i]
                   if o.type != "O" and m * it <= o.mb < m * (it + 1)]
            assert got == base, (i, it)
    assert r.makespan == (n - 1) * T + single.makespan + c_opt


@pytest.mark.parametrize("p,m,n", [(8, 16, 2), (8, 16, 3), (4, 8, 3), (8, 24, 2)])
def test_iterations_tile_without_idle_at_equal_costs(p, m, n):
    """Equal F, B, W costs, memory limit 2p, m >= 2p: the iterations tile
    (each stage starts its next iteration's first F exactly when it would
    otherwise fall idle), so in-window idle stays zero over the whole run."""
    r = S.simulate_iterations(p, m, 2 * p, (1, 1, 1), n, 1)
    for s in r.stats:
        assert s.busy == s.last_end - s.first_start


def test_iterations_reject_bad_arguments():
    for bad in (dict(n_iter=0), dict(c_opt=0), dict(M=0)):
        kw = dict(p=4, m=8, M=8, costs=(1, 1, 1), n_iter=2, c_opt=1)
        kw.update(bad)
        with pytest.raises(ValueError):
            S.simulate_iterations(**kw)


@pytest.mark.parametrize("p,m,n", [(8, 16, 2), (4, 8, 3)])
def test_1f1b_iterations_keep_a_bubble_where_zero_bubble_has_none(p, m, n):
    """Equal costs, m >= 2p: over several iterations every 1F1B stage but the
    first and the last idles inside its window (its ramp-up and ramp-down
    gaps sit between iterations), while ZB(2p) tiles without idle."""
    r1 = S.simulate_iterations(p, m, 0, (1, 1, 1), n, 1, kind="1f1b")
    rz = S.simulate_iterations(p, m, 2 * p, (1, 1, 1), n, 1, kind="zb")
    for i in range(p):
        assert rz.stats[i].busy == rz.stats[i].last_end - rz.stats[i].first_start
        if 0 < i < p - 1:
            assert r1.stats[i].busy < r1.stats[i].last_end - r1.stats[i].first_start


# ------------------------------------------------------ degenerate cases ---

@pytest.mark.parametrize("costs", [(1, 1, 1), (2, 3, 1), (3, 1, 2)])
@pytest.mark.parametrize("kind,M", [("gpipe", 0), ("1f1b", 0), ("zb", 1), ("zb", 3)])
def test_single_stage_has_no_bubble(kind, M, costs):
    """p = 1: nothing to wait for, so every order runs back to back."""
    m = 5
    r = simulate(kind, 1, m, M, costs)
    assert r.stats[0].busy == r.makespan == m * sum(costs)
    assert r.stats[0].first_start == 0


def test_single_stage_zero_bubble_with_limit_one_is_f_b_w_per_microbatch():
    r = simulate("zb", 1, 4, 1, (2, 3, 1))
    assert r.order(0) == [(t, j) for j in range(4) for t in "FBW"]


@pytest.mark.parametrize("p", [2, 4, 8])
@pytest.mark.parametrize("costs", [(1, 1, 1), (2, 3, 1), (1, 2, 3)])
def test_single_microbatch_runs_the_critical_path(p, costs):
    """m = 1: F through every stage, B back through every stage, then the
    first stage's W (zero bubble: W off the path except the last one); the
    atomic backward orders carry W on the path at every stage."""
    cF, cB, cW = costs
    assert simulate("zb", p, 1, 1, costs).makespan == p * cF + p * cB + cW
    for kind in ("gpipe", "1f1b"):
        assert simulate(kind, p, 1, 0, costs).makespan == p * cF + p * (cB + cW)


# ------------------------------------------------- survey-derived regressions
# Stage 3 of p = 8, m = 16 at costs 1:1:1, derived from the rules by an
# independent simulation before this one was written; they pin the greedy's
# behaviour below the memory limit 2p, which the closed forms do not cover.

def _ops(s):
    return [(t[0], int(t[1:])) for t in s.split()]


def test_zb_p_limit_regression_values():
    r = simulate("zb", 8, 16, M=8)
    assert r.makespan == 57
    for i in range(8):
        assert r.idle_over_busy(i) == Fraction(3, 16)
    assert r.order(3) == _ops("F0 F1 F2 F3 F4 F5 F6 F7 B0 W0 B1 W1 B2 W2 B3 W3 B4 F8 B5 W4 B6 F9 B7 W5 W6 F10 "
                              "B8 W7 W8 F11 B9 F12 W9 B10 F13 W10 F14 B11 F15 B12 W11 W12 B13 W13 B14 W14 B15 W15")
    assert (r.stats[3].first_start, r.stats[3].last_end) == (3, 54)
    assert r.stats[3].in_window_idle == Fraction(3, 51)
    assert r.arrive_f[3] == list(range(3, 11)) + [21, 25, 29, 33, 35, 39, 41, 43]
    assert r.arrive_b[3] == list(range(12, 27, 2)) + [30, 34, 38, 42, 44, 48, 50, 52]


def test_zb_2p_and_1f1b_stage3_regression_values():
    z = simulate("zb", 8, 16, M=16)
    assert z.order(3) == (_ops("F0 F1 F2 F3 F4 F5 F6 F7 F8") +
                          [x for k in range(7) for x in (("B", k), ("F", 9 + k))] +
                          [("B", 7)] + [x for k in range(7) for x in (("W", k), ("B", 8 + k))] +
                          [("W", 7), ("B", 15)] + [("W", k) for k in range(8, 16)])
    assert z.arrive_f[3] == list(range(3, 14)) + [15, 17, 19, 21, 23]
    assert z.arrive_b[3] == list(range(12, 43, 2))
    assert (z.stats[3].first_start, z.stats[3].last_end) == (3, 51)
    o = simulate("1f1b", 8, 16)
    assert o.arrive_f[3] == [3, 4, 5, 6, 7, 8] + list(range(21, 49, 3))
    assert o.arrive_b[3] == list(range(16, 62, 3))
    assert (o.stats[3].first_start, o.stats[3].last_end) == (3, 63)
    assert o.stats[3].in_window_idle == Fraction(12, 60)


# ------------------------------------------------------- interleaved 1F1B

INTERLEAVED_COSTS = COSTS + [(1, 1, 0), (5, 1, 1)]


def test_interleaved_bubble_closed_form():
    """Virtual stages: the bubble over the makespan is (p-1)/(vm + p-1) on
    every device ([Guide] "2. The 1F1B Schedule": virtual stages lower the
    1F1B bubble, which is (p-1)/(m+p-1); with v chunks per device each
    warm-up and cool-down step is 1/v of a stage)."""
    n = 0
    for costs in INTERLEAVED_COSTS:
        for p in range(2, 10):
            for v in (2, 3, 4):
                for m in range(p, 6 * p + 1, p):
                    r = S.simulate_interleaved(p, m, v, costs)
                    for i in range(p):
                        assert r.idle_over_makespan(i) == Fraction(p - 1, v * m + p - 1), (costs, p, m, v, i)
                    n += 1
    assert n > 500


def test_interleaved_printed_table():
    """The Quantitative Comparison table: 1F1B 30.4% and interleaved (v = 2)
    17.9% at p = 8, m = 16, both with a memory limit of p microbatches
    (a chunk holds 1/v of a stage's stash, so the peak of chunk-microbatches
    divided by v)."""
    for kind, v, p, m, pct, mem in _rows("guide_schedule_comparison_table.txt"):
        v, p, m, mem = int(v), int(p), int(m), int(mem)
        if kind == "interleaved":
            r = S.simulate_interleaved(p, m, v)
            peak = max(s.peak_active for s in r.stats)
            assert Fraction(peak, v) == mem
        else:
            r = simulate(kind, p, m)
            assert max(s.peak_active for s in r.stats) == mem
        assert round(float(r.idle_over_makespan(0)) * 100, 1) == float(pct)


def test_interleaved_one_chunk_is_1f1b():
    """With one chunk per device the interleaved simulator is the plain 1F1B
    one: the same ops at the same times and the same arrivals."""
    for costs in COSTS:
        for p in range(1, 9):
            for m in range(1, 25):
                a = S.simulate_interleaved(p, m, 1, costs)
                b = simulate("1f1b", p, m, costs=costs)
                assert a.makespan == b.makespan
                for i in range(p):
                    assert [(o.type, o.mb, o.start, o.end) for o in a.ops[i]] == \
                           [(o.type, o.mb, o.start, o.end) for o in b.ops[i]]
                    assert a.arrive_f[i][0] == b.arrive_f[i]
                    assert a.arrive_b[i][0] == b.arrive_b[i]


def _check_interleaved(r):
    """Independent of the simulator's loop: every (chunk, mb) forward and
    backward of every device exactly once; no overlap on a device; every op
    after its inputs; every op as early as possible (it starts when its
    device's previous op ended or when its last input arrived); arrivals
    are the upstream / downstream op ends; peak stash as counted from the
    list."""
    p, m, v = r.p, r.m, r.v
    cF, cB, cW = r.costs
    fend, bend = {}, {}
    for i in range(p):
        for o in r.ops[i]:
            s = o.chunk * p + i
            if o.type == "F":
                fend[(s, o.mb)] = o.end
            elif o.type == "W":
                bend[(s, o.mb)] = o.end
    assert len(fend) == len(bend) == v * p * m
    for i in range(p):
        prev_end, active, peak = 0, 0, 0
        ops = r.ops[i]
        k = 0
        while k < len(ops):
            o = ops[k]
            s = o.chunk * p + i
            if o.type == "F":
                deps = [fend[(s - 1, o.mb)]] if s > 0 else []
                assert o.end - o.start == cF
                active += 1
                peak = max(peak, active)
                k += 1
            else:
                w = ops[k + 1]
                assert o.type == "B" and w.type == "W" and (w.chunk, w.mb) == (o.chunk, o.mb)
                assert o.end - o.start == cB and w.start == o.end and w.end - w.start == cW
                deps = [fend[(s, o.mb)]] + ([bend[(s + 1, o.mb)]] if s < v * p - 1 else [])
                active -= 1
                k += 2
            assert o.start >= prev_end and all(o.start >= d for d in deps)
            assert o.start == max([prev_end] + deps)
            prev_end = ops[k - 1].end
        assert peak == r.stats[i].peak_active
        for c in range(v):
            s = c * p + i
            for j in range(m):
                assert r.arrive_f[i][c][j] == (fend[(s - 1, j)] if s > 0 else 0)
                assert r.arrive_b[i][c][j] == (bend[(s + 1, j)] if s < v * p - 1 else 0)


def test_interleaved_valid_and_as_soon_as_possible():
    for costs in INTERLEAVED_COSTS:
        for p, m, v in ((2, 2, 2), (4, 8, 2), (8, 16, 2), (3, 9, 3), (5, 10, 4), (8, 8, 2), (1, 4, 3)):
            _check_interleaved(S.simulate_interleaved(p, m, v, costs))


def test_interleaved_peak_stash():
    """Device i holds at most (p-1-i) + (v-1)p + 1 chunk-microbatches: its
    warm-up forwards and one more; the first device holds v*p chunks, p whole
    microbatches, the 1F1B bound."""
    for p in range(2, 9):
        for v in (2, 3):
            for m in (p, 2 * p, 4 * p):
                r = S.simulate_interleaved(p, m, v)
                for i in range(p):
                    assert r.stats[i].peak_active == min((p - 1 - i) + (v - 1) * p + 1, v * m)
                assert r.stats[0].peak_active == min(v * p, v * m)


def test_interleaved_stage3_of_8():
    """Stage 3 of p = 8, m = 16, v = 2 (chunk costs 1:1:1): window and
    in-window idle, beside 1F1B's 20% and zero bubble's 0."""
    r = S.simulate_interleaved(8, 16, 2)
    st = r.stats[3]
    assert (st.first_start, st.last_end, st.busy) == (3, 111, 96)
    assert st.in_window_idle == Fraction(12, 108)
    assert r.makespan == 117


def test_interleaved_rejects_bad_arguments():
    for bad in ((8, 12, 2), (8, 16, 0), (0, 16, 2)):
        with pytest.raises(ValueError):
            S.simulate_interleaved(*bad)
    with pytest.raises(ValueError):
        S.simulate_interleaved(4, 8, 2, (0, 1, 1))
