"""Integer-time pipeline schedule simulator.  TEST INFRASTRUCTURE ONLY.

Model ([Guide] "Mathematical Modeling: Bubble Fractions, Memory Bounds,
and Speedups" and "The Mechanics of Pipeline Bubbles"):

* p stages, m microbatches, integer op costs (cF, cB, cW); the model has no
  communication term, so a dependency is satisfied the instant it ends.
* Dependencies: F(i,j) after F(i-1,j);  B(i,j) after F(i,j) and B(i+1,j);
  W(i,j) after B(i,j).
* GPipe and 1F1B keep the backward atomic ([Guide] "Core Innovation 1",
  the "Backward Decomposition" box): one op "BW" of cost cB + cW, and the
  upstream stage's backward waits for the whole of it.
* GPipe ("1. The GPipe Bubble"): each stage runs F0..F(m-1), then the
  backwards in ascending microbatch order.
* 1F1B ("2. The 1F1B Schedule" and the "Conventional 1F1B" figure): stage i
  runs w = min(p-1-i, m) warm-up forwards, then pairs (F(w+k), BW(k)), then
  the remaining backwards.  Every op starts at max(stage free, deps done).
* ZB(M) greedy ("Core Innovation 2" and the scheduler listing): event
  driven.  At each completion time all completions are applied first; then
  every idle stage picks, in order:
    1. the lowest-microbatch ready B;
    2. else the lowest-microbatch ready F if its active count < M
       (the count then rises by one);
    3. else the lowest-microbatch ready W (the count then falls by one --
       the W releases that microbatch's stashed activations);
    4. else it stays idle until the next completion.
  The listing's fourth rule (start a forward regardless of the limit) is
  dropped: it contradicts the hard ceiling on in-flight activations stated
  under "Memory Management & Activation Rollback".  [Ghost]'s prose ranks F
  above B, but both code listings (the [Guide] scheduler and [Ghost]'s
  "The Code Behind the Curtain") try B first; the code is followed.

Results are exact (``fractions.Fraction``).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from fractions import Fraction
from typing import Dict, List, Tuple

GPIPE, ONE_F_ONE_B, ZB = "gpipe", "1f1b", "zb"


@dataclass
class Op:
    type: str      # "F", "B", "W" ("B" of an atomic backward is followed by its "W")
    mb: int
    start: int
    end: int


@dataclass
class StageStats:
    busy: int
    first_start: int
    last_end: int
    peak_active: int

    @property
    def window(self) -> int:
        return self.last_end - self.first_start

    @property
    def in_window_idle(self) -> Fraction:
        return Fraction(self.window - self.busy, self.window)


@dataclass
class Result:
    kind: str
    p: int
    m: int
    M: int
    costs: Tuple[int, int, int]
    ops: List[List[Op]]                 # per stage, in execution order
    stats: List[StageStats]
    makespan: int
    arrive_f: List[List[int]] = field(default_factory=list)   # [stage][mb]
    arrive_b: List[List[int]] = field(default_factory=list)

    def idle_over_makespan(self, i: int) -> Fraction:
        return Fraction(self.makespan - self.stats[i].busy, self.makespan)

    def idle_over_busy(self, i: int) -> Fraction:
        return Fraction(self.makespan - self.stats[i].busy, self.stats[i].busy)

    def order(self, i: int) -> List[Tuple[str, int]]:
        return [(o.type, o.mb) for o in self.ops[i]]


def _fixed_orders(kind: str, p: int, m: int) -> List[List[Tuple[str, int]]]:
    orders = []
    for i in range(p):
        if kind == GPIPE:
            seq = [("F", j) for j in range(m)] + [("BW", j) for j in range(m)]
        else:
            w = min(p - 1 - i, m)
            seq = [("F", j) for j in range(w)]
            for k in range(m - w):
                seq += [("F", w + k), ("BW", k)]
            seq += [("BW", j) for j in range(m - w, m)]
        orders.append(seq)
    return orders


def _simulate_fixed(kind, p, m, costs):
    cF, cB, cW = costs
    orders = _fixed_orders(kind, p, m)
    end: Dict[Tuple[str, int, int], int] = {}
    free = [0] * p
    pos = [0] * p
    placed: List[List[Tuple[str, int, int, int]]] = [[] for _ in range(p)]
    remaining = sum(len(o) for o in orders)
    while remaining:
        progressed = False
        for i in range(p):
            while pos[i] < len(orders[i]):
                t, j = orders[i][pos[i]]
                if t == "F":
                    deps = [("F", i - 1, j)] if i > 0 else []
                    cost = cF
                else:
                    deps = [("F", i, j)] + ([("BW", i + 1, j)] if i < p - 1 else [])
                    cost = cB + cW
                if any(d not in end for d in deps):
                    break
                s = max([free[i]] + [end[d] for d in deps])
                end[(t, i, j)] = s + cost
                free[i] = s + cost
                placed[i].append((t, j, s, s + cost))
                pos[i] += 1
                remaining -= 1
                progressed = True
        if not progressed:
            raise RuntimeError("fixed order deadlocked")
    ops, stats = [], []
    for i in range(p):
        lst, active, peak = [], 0, 0
        for t, j, s, e in placed[i]:
            if t == "F":
                active += 1
                peak = max(peak, active)
                lst.append(Op("F", j, s, e))
            else:
                active -= 1
                lst.append(Op("B", j, s, s + cB))
                lst.append(Op("W", j, s + cB, e))
        busy = m * (cF + cB + cW)
        ops.append(lst)
        stats.append(StageStats(busy, lst[0].start, lst[-1].end, peak))
    arrive_f = [[end[("F", i - 1, j)] if i > 0 else 0 for j in range(m)] for i in range(p)]
    arrive_b = [[end[("BW", i + 1, j)] if i < p - 1 else 0 for j in range(m)] for i in range(p)]
    return ops, stats, arrive_f, arrive_b


def _simulate_zb(p, m, M, costs):
    cF, cB, cW = costs
    cost = {"F": cF, "B": cB, "W": cW}
    done: Dict[Tuple[str, int, int], int] = {}
    started = {("F", i, j): False for i in range(p) for j in range(m)}
    started.update({("B", i, j): False for i in range(p) for j in range(m)})
    started.update({("W", i, j): False for i in range(p) for j in range(m)})
    running: List[Tuple[int, str, int, int]] = []   # (end, type, stage, mb)
    busy_stage = [False] * p
    active = [0] * p
    peak = [0] * p
    ops: List[List[Op]] = [[] for _ in range(p)]
    t = 0
    total = 3 * p * m
    n_done = 0
    while n_done < total:
        # 1) apply every completion at time t
        still = []
        for (e, ty, i, j) in running:
            if e == t:
                done[(ty, i, j)] = e
                busy_stage[i] = False
                n_done += 1
            else:
                still.append((e, ty, i, j))
        running = still
        # 2) every idle stage picks an op
        for i in range(p):
            if busy_stage[i]:
                continue
            pick = None
            for j in range(m):          # rule 1: lowest ready B
                if (not started[("B", i, j)] and ("F", i, j) in done
                        and (i == p - 1 or ("B", i + 1, j) in done)):
                    pick = ("B", j)
                    break
            if pick is None and active[i] < M:   # rule 2: lowest ready F
                for j in range(m):
                    if not started[("F", i, j)] and (i == 0 or ("F", i - 1, j) in done):
                        pick = ("F", j)
                        break
            if pick is None:               # rule 3: lowest ready W
                for j in range(m):
                    if not started[("W", i, j)] and ("B", i, j) in done:
                        pick = ("W", j)
                        break
            if pick is None:
                continue
            ty, j = pick
            started[(ty, i, j)] = True
            if ty == "F":
                active[i] += 1
                peak[i] = max(peak[i], active[i])
            elif ty == "W":
                active[i] -= 1
            e = t + cost[ty]
            running.append((e, ty, i, j))
            busy_stage[i] = True
            ops[i].append(Op(ty, j, t, e))
        if n_done == total:
            break
        if not running:
            raise RuntimeError("zero-bubble greedy deadlocked (memory limit too small?)")
        t = min(e for (e, _, _, _) in running)
    stats = []
    for i in range(p):
        busy = sum(o.end - o.start for o in ops[i])
        stats.append(StageStats(busy, ops[i][0].start, ops[i][-1].end, peak[i]))
    arrive_f = [[done[("F", i - 1, j)] if i > 0 else 0 for j in range(m)] for i in range(p)]
    arrive_b = [[done[("B", i + 1, j)] if i < p - 1 else 0 for j in range(m)] for i in range(p)]
    return ops, stats, arrive_f, arrive_b


def simulate(kind: str, p: int, m: int, M: int = 0, costs=(1, 1, 1)) -> Result:
    """Simulate one iteration of a p-stage pipeline over m microbatches.

    kind: "gpipe", "1f1b" or "zb" (M = memory limit in microbatches, p..2p
    on the pages; any M >= 1 is accepted).  Costs are integers with
    cF >= 1 and cB >= 1; cW >= 0 for the atomic schedules and >= 1 for zb.
    """
    cF, cB, cW = (int(c) for c in costs)
    if p < 1 or m < 1 or cF < 1 or cB < 1 or cW < 0:
        raise ValueError("bad arguments")
    if kind in (GPIPE, ONE_F_ONE_B):
        ops, stats, af, ab = _simulate_fixed(kind, p, m, (cF, cB, cW))
    elif kind == ZB:
        if M < 1 or cW < 1:
            raise ValueError("zb needs M >= 1 and cW >= 1")
        ops, stats, af, ab = _simulate_zb(p, m, M, (cF, cB, cW))
    else:
        raise ValueError(kind)
    makespan = max(s.last_end for s in stats)
    return Result(kind, p, m, M, (cF, cB, cW), ops, stats, makespan, af, ab)


# ---------------------------------------------------------------------------
# Several iterations back to back (zero-bubble greedy only).
#
# Each stage closes iteration `it` with an optimizer op O(it) of cost cO once
# all of its own W of that iteration have completed; its first F of
# iteration it+1 waits for that O and for the upstream stage's F, and for
# nothing else: there is no synchronization across stages between
# iterations.  [Abstract] says the method bypasses the synchronizations of
# the optimizer step without describing how; this is the plainest reading
# (each stage updates its own weights as soon as its own gradients are
# complete).  Microbatch j of
# iteration it has the global index g = it*m + j; "lowest microbatch" in the
# greedy rules is the lowest g, and the memory limit counts in-flight
# microbatches of any iteration.  Rule 0 (before B, F, W): a ready O.
# ---------------------------------------------------------------------------

@dataclass
class IterResult:
    p: int
    m: int
    M: int
    n_iter: int
    costs: Tuple[int, int, int]
    c_opt: int
    ops: List[List[Op]]                 # per stage; O ops carry the iteration in .mb
    stats: List[StageStats]
    makespan: int
    arrive_f: List[List[int]]           # [stage][g], g = it*m + j
    arrive_b: List[List[int]]

    def order(self, i: int) -> List[Tuple[str, int]]:
        return [(o.type, o.mb) for o in self.ops[i]]


def _simulate_1f1b_iterations(p, m, costs, n_iter, c_opt):
    """1F1B over several iterations: each stage runs its fixed 1F1B sequence
    of iteration it (microbatches g = it*m + j, whole backwards), then its
    optimizer step O(it), then the sequence of iteration it+1; an op starts
    when its stage is free and its inputs exist (the step follows the
    stage's last backward by sequence order, and the next iteration's F
    waits for the step the same way)."""
    cF, cB, cW = costs
    G = n_iter * m
    seqs = []
    for i in range(p):
        seq = []
        for it in range(n_iter):
            seq += [(t, it * m + j) for t, j in _fixed_orders(ONE_F_ONE_B, p, m)[i]] + [("O", it)]
        seqs.append(seq)
    end: Dict[Tuple[str, int, int], int] = {}
    free = [0] * p
    pos = [0] * p
    ops: List[List[Op]] = [[] for _ in range(p)]
    active, peak = [0] * p, [0] * p
    remaining = sum(len(q) for q in seqs)
    while remaining:
        progressed = False
        for i in range(p):
            while pos[i] < len(seqs[i]):
                t, k = seqs[i][pos[i]]
                if t == "F":
                    deps, cost = ([("F", i - 1, k)] if i > 0 else []), cF
                elif t == "BW":
                    deps, cost = [("F", i, k)] + ([("BW", i + 1, k)] if i < p - 1 else []), cB + cW
                else:
                    deps, cost = [], c_opt
                if any(d not in end for d in deps):
                    break
                st = max([free[i]] + [end[d] for d in deps])
                end[(t, i, k)] = st + cost
                free[i] = st + cost
                if t == "F":
                    ops[i].append(Op("F", k, st, st + cF))
                    active[i] += 1
                    peak[i] = max(peak[i], active[i])
                elif t == "BW":
                    ops[i].append(Op("B", k, st, st + cB))
                    ops[i].append(Op("W", k, st + cB, st + cB + cW))
                    active[i] -= 1
                else:
                    ops[i].append(Op("O", k, st, st + cost))
                pos[i] += 1
                remaining -= 1
                progressed = True
        if not progressed:
            raise RuntimeError("fixed order deadlocked")
    stats = [StageStats(sum(o.end - o.start for o in ops[i]), ops[i][0].start, ops[i][-1].end, peak[i])
             for i in range(p)]
    arrive_f = [[end[("F", i - 1, g)] if i > 0 else 0 for g in range(G)] for i in range(p)]
    arrive_b = [[end[("BW", i + 1, g)] if i < p - 1 else 0 for g in range(G)] for i in range(p)]
    return ops, stats, arrive_f, arrive_b


def simulate_iterations(p: int, m: int, M: int, costs=(1, 1, 1), n_iter: int = 2, c_opt: int = 1,
                        kind: str = ZB) -> IterResult:
    """Several iterations back to back: kind "zb" (the greedy below, memory
    limit M) or "1f1b" (fixed sequences, M unused)."""
    cF, cB, cW = (int(c) for c in costs)
    c_opt = int(c_opt)
    if kind == ONE_F_ONE_B:
        if p < 1 or m < 1 or cF < 1 or cB < 1 or cW < 0 or n_iter < 1 or c_opt < 1:
            raise ValueError("bad arguments")
        ops, stats, af, ab = _simulate_1f1b_iterations(p, m, (cF, cB, cW), n_iter, c_opt)
        return IterResult(p, m, M, n_iter, (cF, cB, cW), c_opt, ops, stats, max(s.last_end for s in stats), af, ab)
    if kind != ZB:
        raise ValueError(kind)
    if p < 1 or m < 1 or M < 1 or cF < 1 or cB < 1 or cW < 1 or n_iter < 1 or c_opt < 1:
        raise ValueError("bad arguments")
    G = n_iter * m
    cost = {"F": cF, "B": cB, "W": cW, "O": c_opt}
    done: Dict[Tuple[str, int, int], int] = {}
    started = set()
    w_left = [[m] * n_iter for _ in range(p)]   # W of iteration it still to complete at stage i
    running: List[Tuple[int, str, int, int]] = []
    busy_stage = [False] * p
    active = [0] * p
    peak = [0] * p
    ops: List[List[Op]] = [[] for _ in range(p)]
    t = 0
    total = p * (3 * G + n_iter)
    n_done = 0
    while n_done < total:
        still = []
        for (e, ty, i, k) in running:
            if e == t:
                done[(ty, i, k)] = e
                busy_stage[i] = False
                n_done += 1
                if ty == "W":
                    w_left[i][k // m] -= 1
            else:
                still.append((e, ty, i, k))
        running = still
        for i in range(p):
            if busy_stage[i]:
                continue
            pick = None
            for it in range(n_iter):                 # rule 0: a ready optimizer step
                if ("O", i, it) not in started and w_left[i][it] == 0:
                    pick = ("O", it)
                    break
            if pick is None:                         # rule 1: lowest ready B
                for g in range(G):
                    if (("B", i, g) not in started and ("F", i, g) in done
                            and (i == p - 1 or ("B", i + 1, g) in done)):
                        pick = ("B", g)
                        break
            if pick is None and active[i] < M:       # rule 2: lowest ready F
                for g in range(G):
                    it = g // m
                    if (("F", i, g) not in started and (i == 0 or ("F", i - 1, g) in done)
                            and (it == 0 or ("O", i, it - 1) in done)):
                        pick = ("F", g)
                        break
            if pick is None:                         # rule 3: lowest ready W
                for g in range(G):
                    if ("W", i, g) not in started and ("B", i, g) in done:
                        pick = ("W", g)
                        break
            if pick is None:
                continue
            ty, k = pick
            started.add((ty, i, k))
            if ty == "F":
                active[i] += 1
                peak[i] = max(peak[i], active[i])
            elif ty == "W":
                active[i] -= 1
            e = t + cost[ty]
            running.append((e, ty, i, k))
            busy_stage[i] = True
            ops[i].append(Op(ty, k, t, e))
        if n_done == total:
            break
        if not running:
            raise RuntimeError("zero-bubble greedy deadlocked (memory limit too small?)")
        t = min(e for (e, _, _, _) in running)
    stats = []
    for i in range(p):
        busy = sum(o.end - o.start for o in ops[i])
        stats.append(StageStats(busy, ops[i][0].start, ops[i][-1].end, peak[i]))
    arrive_f = [[done[("F", i - 1, g)] if i > 0 else 0 for g in range(G)] for i in range(p)]
    arrive_b = [[done[("B", i + 1, g)] if i < p - 1 else 0 for g in range(G)] for i in range(p)]
    makespan = max(s.last_end for s in stats)
    return IterResult(p, m, M, n_iter, (cF, cB, cW), c_opt, ops, stats, makespan, arrive_f, arrive_b)


# ---------------------------------------------------------------------------
# Interleaved 1F1B (virtual stages), the comparison schedule of [Guide] "2.
# The 1F1B Schedule" (virtual stages lower the bubble) and of the "Quantitative
# Comparison: LLaMA-3-70B on 8 Pipeline Stages" table (v = 2).  The pages
# give no algorithm; this is the published interleaved schedule of Megatron-LM
# (Narayanan et al., 2021), restated:
#
# * each of the p devices holds v model chunks; chunk c of device i is the
#   virtual stage s = c*p + i of a pipeline of v*p virtual stages, so
#   microbatch j's forward runs s = 0, 1, ..., v*p - 1 across the devices and
#   its backward runs back down.  Op costs (cF, cB, cW) are per chunk.
# * Dependencies: F(s, j) after F(s-1, j); the backward BW(s, j) (atomic,
#   cost cB + cW, as in 1F1B) after F(s, j) and BW(s+1, j).
# * The microbatches go p at a time (m must be a multiple of p): the k-th
#   forward of a device is chunk (k mod vp) div p of microbatch
#   (k div vp)*p + k mod p; the k-th backward the same microbatch of chunk
#   v - 1 - (k mod vp) div p.
# * Device i runs w_i = min((p-1-i) + (v-1)p, vm) warm-up forwards, then
#   pairs (next forward, next backward), then the remaining backwards; each
#   op starts at max(device free, inputs done).  w_i is the fewest warm-up
#   forwards that never deadlock: the first backward that reaches device i
#   needs the forwards of all v chunks of the first microbatch group.
#   Megatron-LM adds another p-1-i warm-up forwards, which pair its sends and
#   receives; the pages' model has no communication, and there they change
#   no op time but keep more microbatch-chunks stashed.  With v = 1 the
#   sequence is the plain 1F1B one.
#
# The idle time over the makespan is (p-1)/(vm + p-1), the bubble the [Guide]
# table prints for v = 2 (17.9% at p = 8, m = 16).
# ---------------------------------------------------------------------------

INTERLEAVED = "interleaved"


@dataclass
class ChunkOp:
    type: str      # "F", "B", "W" (the atomic backward's B, then its W)
    chunk: int
    mb: int
    start: int
    end: int


@dataclass
class InterleavedResult:
    p: int
    m: int
    v: int
    costs: Tuple[int, int, int]
    ops: List[List[ChunkOp]]            # per device, in execution order
    stats: List[StageStats]             # peak_active counts chunk-microbatches
    makespan: int
    arrive_f: List[List[List[int]]]     # [device][chunk][mb]: end of F(s-1, j), 0 for s = 0
    arrive_b: List[List[List[int]]]     # [device][chunk][mb]: end of BW(s+1, j), 0 for the last s

    def order(self, i: int) -> List[Tuple[str, int, int]]:
        return [(o.type, o.chunk, o.mb) for o in self.ops[i]]

    def idle_over_makespan(self, i: int) -> Fraction:
        return Fraction(self.makespan - self.stats[i].busy, self.makespan)


def interleaved_sequence(p: int, m: int, v: int, i: int) -> List[Tuple[str, int, int]]:
    """Device i's op sequence: ("F" | "BW", chunk, microbatch)."""
    n = v * m

    def mb_of(k):
        return (k // (p * v)) * p + k % p

    def fwd(k):
        return ("F", (k % (p * v)) // p, mb_of(k))

    def bwd(k):
        return ("BW", v - 1 - (k % (p * v)) // p, mb_of(k))

    warm = min((p - 1 - i) + (v - 1) * p, n)
    seq = [fwd(k) for k in range(warm)]
    for k in range(n - warm):
        seq += [fwd(warm + k), bwd(k)]
    seq += [bwd(k) for k in range(n - warm, n)]
    return seq


def simulate_interleaved(p: int, m: int, v: int, costs=(1, 1, 1)) -> InterleavedResult:
    cF, cB, cW = (int(c) for c in costs)
    if p < 1 or m < 1 or v < 1 or (v > 1 and m % p) or cF < 1 or cB < 1 or cW < 0:
        raise ValueError("bad arguments (v >= 1; with v > 1, m must be a multiple of p)")
    seqs = [interleaved_sequence(p, m, v, i) for i in range(p)]
    last = v * p - 1
    end: Dict[Tuple[str, int, int], int] = {}
    free = [0] * p
    pos = [0] * p
    ops: List[List[ChunkOp]] = [[] for _ in range(p)]
    active, peak = [0] * p, [0] * p
    remaining = sum(len(q) for q in seqs)
    while remaining:
        progressed = False
        for i in range(p):
            while pos[i] < len(seqs[i]):
                t, c, j = seqs[i][pos[i]]
                s = c * p + i
                if t == "F":
                    deps, cost = ([("F", s - 1, j)] if s > 0 else []), cF
                else:
                    deps, cost = [("F", s, j)] + ([("BW", s + 1, j)] if s < last else []), cB + cW
                if any(d not in end for d in deps):
                    break
                st = max([free[i]] + [end[d] for d in deps])
                end[(t, s, j)] = st + cost
                free[i] = st + cost
                if t == "F":
                    ops[i].append(ChunkOp("F", c, j, st, st + cF))
                    active[i] += 1
                    peak[i] = max(peak[i], active[i])
                else:
                    ops[i].append(ChunkOp("B", c, j, st, st + cB))
                    ops[i].append(ChunkOp("W", c, j, st + cB, st + cB + cW))
                    active[i] -= 1
                pos[i] += 1
                remaining -= 1
                progressed = True
        if not progressed:
            raise RuntimeError("interleaved order deadlocked")
    stats = [StageStats(v * m * (cF + cB + cW), ops[i][0].start, ops[i][-1].end, peak[i]) for i in range(p)]
    arrive_f = [[[end[("F", c * p + i - 1, j)] if c * p + i > 0 else 0 for j in range(m)] for c in range(v)]
                for i in range(p)]
    arrive_b = [[[end[("BW", c * p + i + 1, j)] if c * p + i < last else 0 for j in range(m)] for c in range(v)]
                for i in range(p)]
    return InterleavedResult(p, m, v, (cF, cB, cW), ops, stats, max(s.last_end for s in stats), arrive_f, arrive_b)
