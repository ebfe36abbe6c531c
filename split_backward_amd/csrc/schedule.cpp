// Host schedule generator: per-stage op order for GPipe, 1F1B and the
// memory-limited zero-bubble greedy, by integer-time simulation of the whole
// p-stage pipeline (the model of "Zero-Bubble Pipeline Parallelism Guide for
// LLMs", "Mathematical Modeling: Bubble Fractions, Memory Bounds, and
// Speedups": no communication term, integer op costs).
//
// Zero-bubble greedy ("Core Innovation 2" and the Guide's scheduler
// listing): whenever a stage is idle it takes the ready input-gradient op
// (B) of the lowest microbatch; otherwise the next forward (F) if fewer than
// mem_limit microbatches hold stashed activations; otherwise the ready
// weight-gradient op (W) of the lowest microbatch, which releases that
// microbatch's stash; otherwise it waits for the next completion.  All
// completions at a time instant are applied before any stage chooses.  The
// listing's last-resort rule (a forward regardless of the limit) is left out
// because it would break the hard ceiling on stashed activations described
// under "Memory Management & Activation Rollback".
#include <algorithm>
#include <cstdint>
#include <limits>
#include <queue>
#include <vector>

#include "../../include/zb.h"

namespace {

constexpr int64_t NOT_DONE = std::numeric_limits<int64_t>::max();

struct Placed {
    int type;  // ZB_OP_F / ZB_OP_B / ZB_OP_W
    int mb;
    int64_t start, end;
};

struct Pipeline {
    int p, m;
    // completion times, NOT_DONE until finished: index stage * m + mb
    std::vector<int64_t> f_end, b_end, w_end;
    std::vector<std::vector<Placed>> placed;
    std::vector<int> peak;
    Pipeline(int p_, int m_)
        : p(p_), m(m_), f_end((size_t)p_ * m_, NOT_DONE), b_end((size_t)p_ * m_, NOT_DONE),
          w_end((size_t)p_ * m_, NOT_DONE), placed(p_), peak(p_, 0) {}
    int64_t& F(int i, int j) { return f_end[(size_t)i * m + j]; }
    int64_t& B(int i, int j) { return b_end[(size_t)i * m + j]; }
    int64_t& W(int i, int j) { return w_end[(size_t)i * m + j]; }
};

// GPipe / 1F1B: fixed per-stage sequences of F and whole backwards (B then W
// back to back); each op starts when its stage is free and its inputs exist.
bool run_fixed(Pipeline& P, bool one_f_one_b, int64_t cF, int64_t cB, int64_t cW) {
    const int p = P.p, m = P.m;
    std::vector<std::vector<std::pair<int, int>>> seq(p);  // (is_backward, mb)
    for (int i = 0; i < p; ++i) {
        auto& s = seq[i];
        if (!one_f_one_b) {
            for (int j = 0; j < m; ++j) s.push_back({0, j});
            for (int j = 0; j < m; ++j) s.push_back({1, j});
        } else {
            const int warm = std::min(p - 1 - i, m);
            for (int j = 0; j < warm; ++j) s.push_back({0, j});
            for (int j = warm; j < m; ++j) {
                s.push_back({0, j});
                s.push_back({1, j - warm});
            }
            for (int j = m - warm; j < m; ++j) s.push_back({1, j});
        }
    }
    std::vector<size_t> next(p, 0);
    std::vector<int64_t> free_at(p, 0);
    std::vector<int> active(p, 0);
    size_t left = (size_t)2 * p * m;
    while (left > 0) {
        bool moved = false;
        for (int i = 0; i < p; ++i) {
            while (next[i] < seq[i].size()) {
                const auto [bwd, j] = seq[i][next[i]];
                int64_t ready;
                if (!bwd) {
                    ready = (i == 0) ? 0 : P.F(i - 1, j);
                } else {
                    const int64_t down = (i == p - 1) ? 0 : P.W(i + 1, j);  // whole backward downstream
                    ready = std::max(P.F(i, j), down);
                }
                if (ready == NOT_DONE) break;
                const int64_t st = std::max(ready, free_at[i]);
                if (!bwd) {
                    P.F(i, j) = st + cF;
                    free_at[i] = st + cF;
                    P.placed[i].push_back({ZB_OP_F, j, st, st + cF});
                    P.peak[i] = std::max(P.peak[i], ++active[i]);
                } else {
                    P.B(i, j) = st + cB;
                    P.W(i, j) = st + cB + cW;
                    free_at[i] = st + cB + cW;
                    P.placed[i].push_back({ZB_OP_B, j, st, st + cB});
                    P.placed[i].push_back({ZB_OP_W, j, st + cB, st + cB + cW});
                    --active[i];
                }
                ++next[i];
                --left;
                moved = true;
            }
        }
        if (!moved) return false;
    }
    return true;
}

bool run_greedy(Pipeline& P, int M, int64_t cF, int64_t cB, int64_t cW) {
    const int p = P.p, m = P.m;
    struct Running { int64_t end; int type, stage, mb; };
    auto later = [](const Running& a, const Running& b) { return a.end > b.end; };
    std::priority_queue<Running, std::vector<Running>, decltype(later)> heap(later);
    std::vector<char> busy(p, 0);
    std::vector<int> active(p, 0), next_f(p, 0);
    std::vector<std::vector<char>> b_started(p, std::vector<char>(m, 0)), w_started(p, std::vector<char>(m, 0));
    int64_t now = 0;
    size_t finished = 0;
    const size_t total = (size_t)3 * p * m;
    while (true) {
        while (!heap.empty() && heap.top().end == now) {
            const Running r = heap.top();
            heap.pop();
            if (r.type == ZB_OP_F) P.F(r.stage, r.mb) = r.end;
            else if (r.type == ZB_OP_B) P.B(r.stage, r.mb) = r.end;
            else P.W(r.stage, r.mb) = r.end;
            busy[r.stage] = 0;
            ++finished;
        }
        if (finished == total) break;
        for (int i = 0; i < p; ++i) {
            if (busy[i]) continue;
            int type = -1, mb = -1;
            for (int j = 0; j < m && type < 0; ++j)
                if (!b_started[i][j] && P.F(i, j) != NOT_DONE && (i == p - 1 || P.B(i + 1, j) != NOT_DONE)) {
                    type = ZB_OP_B;
                    mb = j;
                }
            if (type < 0 && active[i] < M && next_f[i] < m &&
                (i == 0 || P.F(i - 1, next_f[i]) != NOT_DONE)) {
                type = ZB_OP_F;
                mb = next_f[i];
            }
            if (type < 0)
                for (int j = 0; j < m && type < 0; ++j)
                    if (!w_started[i][j] && P.B(i, j) != NOT_DONE) {
                        type = ZB_OP_W;
                        mb = j;
                    }
            if (type < 0) continue;
            int64_t cost;
            if (type == ZB_OP_F) {
                ++next_f[i];
                P.peak[i] = std::max(P.peak[i], ++active[i]);
                cost = cF;
            } else if (type == ZB_OP_B) {
                b_started[i][mb] = 1;
                cost = cB;
            } else {
                w_started[i][mb] = 1;
                --active[i];
                cost = cW;
            }
            busy[i] = 1;
            heap.push({now + cost, type, i, mb});
            P.placed[i].push_back({type, mb, now, now + cost});
        }
        if (heap.empty()) return false;  // nothing can run: limit too small
        now = heap.top().end;
    }
    return true;
}

}  // namespace

extern "C" int32_t zb_schedule_generate(int32_t kind, int32_t p, int32_t m, int32_t mem_limit, int32_t cF,
                                        int32_t cB, int32_t cW, int32_t stage, zb_op* ops, int64_t* start,
                                        int64_t* end, int32_t cap, int64_t* arrive_f, int64_t* arrive_b,
                                        zb_sched_stats* stats) {
    if (p < 1 || m < 1 || stage < 0 || stage >= p || cF < 1 || cB < 1 || cW < 0) return ZB_EINVAL;
    if ((ops || start || end) && cap < 3 * m) return ZB_EINVAL;
    if (kind != ZB_SCHED_GPIPE && kind != ZB_SCHED_1F1B && kind != ZB_SCHED_ZB) return ZB_EINVAL;
    if ((int64_t)p * m > 1 << 22) return ZB_EINVAL;
    Pipeline P(p, m);
    bool ok;
    if (kind == ZB_SCHED_ZB) {
        if (mem_limit < 1 || cW < 1) return ZB_EINVAL;
        ok = run_greedy(P, mem_limit, cF, cB, cW);
    } else {
        ok = run_fixed(P, kind == ZB_SCHED_1F1B, cF, cB, cW);
    }
    if (!ok) return ZB_EINVAL;
    const auto& mine = P.placed[stage];
    for (size_t k = 0; k < mine.size(); ++k) {
        if (ops) ops[k] = zb_op{mine[k].type, mine[k].mb};
        if (start) start[k] = mine[k].start;
        if (end) end[k] = mine[k].end;
    }
    for (int j = 0; j < m; ++j) {
        if (arrive_f) arrive_f[j] = stage == 0 ? 0 : P.F(stage - 1, j);
        if (arrive_b) {
            if (stage == p - 1) arrive_b[j] = 0;
            else arrive_b[j] = (kind == ZB_SCHED_ZB) ? P.B(stage + 1, j) : P.W(stage + 1, j);
        }
    }
    if (stats) {
        int64_t mk = 0;
        for (int i = 0; i < p; ++i) mk = std::max(mk, P.placed[i].back().end);
        int64_t busy = 0;
        for (const auto& o : mine) busy += o.end - o.start;
        stats->makespan = mk;
        stats->busy = busy;
        stats->first_start = mine.front().start;
        stats->last_end = mine.back().end;
        stats->peak_active = P.peak[stage];
        stats->n_ops = (int32_t)mine.size();
    }
    return (int32_t)mine.size();
}

// ---------------------------------------------------------------------------
// Several iterations of the zero-bubble greedy.  Each stage runs an optimizer
// step O(it) (cost c_opt) once all of its own W of iteration it have
// completed; its F of iteration it+1 waits for that step and for the
// upstream F only (no synchronization across stages between iterations: the
// abstract page "Zero Bubble Pipeline Parallelism" states that the method
// bypasses the optimizer step's synchronizations).  Microbatch j of
// iteration it is g = it*m + j; "lowest microbatch" is the lowest g and the
// memory limit counts stashed microbatches of any iteration.  A ready O is
// taken before any B, F or W.
namespace {
// 1F1B over several iterations: each stage runs its fixed 1F1B sequence of
// iteration it (whole backwards, microbatches g = it*m + j), then its
// optimizer step, then iteration it+1; an op starts when its stage is free
// and its inputs exist.  Fills the stage's ops and the arrival times.
bool run_fixed_iters(int p, int m, int n_iter, int64_t cF, int64_t cB, int64_t cW, int64_t c_opt,
                     std::vector<std::vector<Placed>>& placed, std::vector<int>& peak, std::vector<int64_t>& Fe,
                     std::vector<int64_t>& BWe) {
    const int G = m * n_iter;
    enum { S_F = 0, S_BW = 1, S_O = 2 };
    std::vector<std::vector<std::pair<int, int>>> seq(p);  // (kind, index)
    for (int i = 0; i < p; ++i) {
        const int warm = std::min(p - 1 - i, m);
        for (int it = 0; it < n_iter; ++it) {
            const int b = it * m;
            for (int j = 0; j < warm; ++j) seq[i].push_back({S_F, b + j});
            for (int j = warm; j < m; ++j) {
                seq[i].push_back({S_F, b + j});
                seq[i].push_back({S_BW, b + j - warm});
            }
            for (int j = m - warm; j < m; ++j) seq[i].push_back({S_BW, b + j});
            seq[i].push_back({S_O, it});
        }
    }
    auto at = [G](int i, int g) { return (size_t)i * G + g; };
    std::vector<size_t> next(p, 0);
    std::vector<int64_t> free_at(p, 0);
    std::vector<int> active(p, 0);
    size_t left = 0;
    for (auto& q : seq) left += q.size();
    while (left > 0) {
        bool moved = false;
        for (int i = 0; i < p; ++i) {
            while (next[i] < seq[i].size()) {
                const auto [kind, k] = seq[i][next[i]];
                int64_t ready = 0;
                if (kind == S_F) ready = (i == 0) ? 0 : Fe[at(i - 1, k)];
                else if (kind == S_BW) ready = std::max(Fe[at(i, k)], (i == p - 1) ? int64_t(0) : BWe[at(i + 1, k)]);
                if (ready == NOT_DONE) break;
                const int64_t st = std::max(ready, free_at[i]);
                if (kind == S_F) {
                    Fe[at(i, k)] = st + cF;
                    free_at[i] = st + cF;
                    placed[i].push_back({ZB_OP_F, k, st, st + cF});
                    peak[i] = std::max(peak[i], ++active[i]);
                } else if (kind == S_BW) {
                    BWe[at(i, k)] = st + cB + cW;
                    free_at[i] = st + cB + cW;
                    placed[i].push_back({ZB_OP_B, k, st, st + cB});
                    placed[i].push_back({ZB_OP_W, k, st + cB, st + cB + cW});
                    --active[i];
                } else {
                    free_at[i] = st + c_opt;
                    placed[i].push_back({ZB_OP_O, k, st, st + c_opt});
                }
                ++next[i];
                --left;
                moved = true;
            }
        }
        if (!moved) return false;
    }
    return true;
}
}  // namespace

extern "C" int32_t zb_schedule_generate_iters(int32_t kind, int32_t p, int32_t m, int32_t mem_limit, int32_t cF,
                                              int32_t cB, int32_t cW, int32_t c_opt, int32_t n_iter, int32_t stage,
                                              zb_op* ops, int64_t* start, int64_t* end, int32_t cap,
                                              int64_t* arrive_f, int64_t* arrive_b, zb_sched_stats* stats) {
    if (kind != ZB_SCHED_ZB && kind != ZB_SCHED_1F1B) return ZB_EINVAL;
    if (p < 1 || m < 1 || n_iter < 1 || stage < 0 || stage >= p || cF < 1 || cB < 1 || c_opt < 1) return ZB_EINVAL;
    if (kind == ZB_SCHED_ZB && (cW < 1 || mem_limit < 1)) return ZB_EINVAL;
    if (cW < 0) return ZB_EINVAL;
    if ((int64_t)p * m * n_iter > 1 << 22) return ZB_EINVAL;
    const int G = m * n_iter;
    const int n_stage_ops = 3 * G + n_iter;
    if ((ops || start || end) && cap < n_stage_ops) return ZB_EINVAL;
    if (kind == ZB_SCHED_1F1B) {
        std::vector<std::vector<Placed>> placed(p);
        std::vector<int> peak(p, 0);
        std::vector<int64_t> Fe((size_t)p * G, NOT_DONE), BWe((size_t)p * G, NOT_DONE);
        if (!run_fixed_iters(p, m, n_iter, cF, cB, cW, c_opt, placed, peak, Fe, BWe)) return ZB_EINVAL;
        const auto& mine = placed[stage];
        for (size_t q = 0; q < mine.size(); ++q) {
            if (ops) ops[q] = zb_op{mine[q].type, mine[q].mb};
            if (start) start[q] = mine[q].start;
            if (end) end[q] = mine[q].end;
        }
        for (int g = 0; g < G; ++g) {
            if (arrive_f) arrive_f[g] = stage == 0 ? 0 : Fe[(size_t)(stage - 1) * G + g];
            if (arrive_b) arrive_b[g] = stage == p - 1 ? 0 : BWe[(size_t)(stage + 1) * G + g];
        }
        if (stats) {
            int64_t mk = 0, b = 0;
            for (int i = 0; i < p; ++i) mk = std::max(mk, placed[i].back().end);
            for (const auto& o : mine) b += o.end - o.start;
            stats->makespan = mk;
            stats->busy = b;
            stats->first_start = mine.front().start;
            stats->last_end = mine.back().end;
            stats->peak_active = peak[stage];
            stats->n_ops = (int32_t)mine.size();
        }
        return (int32_t)mine.size();
    }
    std::vector<int64_t> Fe((size_t)p * G, NOT_DONE), Be((size_t)p * G, NOT_DONE), Oe((size_t)p * n_iter, NOT_DONE);
    auto at = [G](int i, int g) { return (size_t)i * G + g; };
    std::vector<std::vector<char>> b_started(p, std::vector<char>(G, 0)), w_started(p, std::vector<char>(G, 0));
    std::vector<std::vector<char>> o_started(p, std::vector<char>(n_iter, 0));
    std::vector<std::vector<int>> w_left(p, std::vector<int>(n_iter, m));
    std::vector<int> active(p, 0), next_f(p, 0), peak(p, 0);
    std::vector<char> busy(p, 0);
    std::vector<std::vector<Placed>> placed(p);
    struct Running { int64_t end; int type, stage, k; };
    auto later = [](const Running& a, const Running& b) { return a.end > b.end; };
    std::priority_queue<Running, std::vector<Running>, decltype(later)> heap(later);
    int64_t now = 0;
    size_t finished = 0;
    const size_t total = (size_t)p * n_stage_ops;
    while (true) {
        while (!heap.empty() && heap.top().end == now) {
            const Running r = heap.top();
            heap.pop();
            if (r.type == ZB_OP_F) Fe[at(r.stage, r.k)] = r.end;
            else if (r.type == ZB_OP_B) Be[at(r.stage, r.k)] = r.end;
            else if (r.type == ZB_OP_W) --w_left[r.stage][r.k / m];
            else Oe[(size_t)r.stage * n_iter + r.k] = r.end;
            busy[r.stage] = 0;
            ++finished;
        }
        if (finished == total) break;
        for (int i = 0; i < p; ++i) {
            if (busy[i]) continue;
            int type = -1, k = -1;
            for (int it = 0; it < n_iter && type < 0; ++it)
                if (!o_started[i][it] && w_left[i][it] == 0) {
                    type = ZB_OP_O;
                    k = it;
                }
            for (int g = 0; g < G && type < 0; ++g)
                if (!b_started[i][g] && Fe[at(i, g)] != NOT_DONE && (i == p - 1 || Be[at(i + 1, g)] != NOT_DONE)) {
                    type = ZB_OP_B;
                    k = g;
                }
            if (type < 0 && active[i] < mem_limit && next_f[i] < G) {
                const int g = next_f[i], it = g / m;
                if ((i == 0 || Fe[at(i - 1, g)] != NOT_DONE) && (it == 0 || Oe[(size_t)i * n_iter + it - 1] != NOT_DONE)) {
                    type = ZB_OP_F;
                    k = g;
                }
            }
            for (int g = 0; g < G && type < 0; ++g)
                if (!w_started[i][g] && Be[at(i, g)] != NOT_DONE) {
                    type = ZB_OP_W;
                    k = g;
                }
            if (type < 0) continue;
            int64_t cost;
            if (type == ZB_OP_F) {
                ++next_f[i];
                peak[i] = std::max(peak[i], ++active[i]);
                cost = cF;
            } else if (type == ZB_OP_B) {
                b_started[i][k] = 1;
                cost = cB;
            } else if (type == ZB_OP_W) {
                w_started[i][k] = 1;
                --active[i];
                cost = cW;
            } else {
                o_started[i][k] = 1;
                cost = c_opt;
            }
            busy[i] = 1;
            heap.push({now + cost, type, i, k});
            placed[i].push_back({type, k, now, now + cost});
        }
        if (heap.empty()) return ZB_EINVAL;  // nothing can run: limit too small
        now = heap.top().end;
    }
    const auto& mine = placed[stage];
    for (size_t q = 0; q < mine.size(); ++q) {
        if (ops) ops[q] = zb_op{mine[q].type, mine[q].mb};
        if (start) start[q] = mine[q].start;
        if (end) end[q] = mine[q].end;
    }
    for (int g = 0; g < G; ++g) {
        if (arrive_f) arrive_f[g] = stage == 0 ? 0 : Fe[at(stage - 1, g)];
        if (arrive_b) arrive_b[g] = stage == p - 1 ? 0 : Be[at(stage + 1, g)];
    }
    if (stats) {
        int64_t mk = 0;
        for (int i = 0; i < p; ++i) mk = std::max(mk, placed[i].back().end);
        int64_t b = 0;
        for (const auto& o : mine) b += o.end - o.start;
        stats->makespan = mk;
        stats->busy = b;
        stats->first_start = mine.front().start;
        stats->last_end = mine.back().end;
        stats->peak_active = peak[stage];
        stats->n_ops = (int32_t)mine.size();
    }
    return (int32_t)mine.size();
}

// ---------------------------------------------------------------------------
// Interleaved 1F1B (virtual stages): the comparison schedule of the Guide's
// "2. The 1F1B Schedule" and of its "Quantitative Comparison" table (v = 2).
// Each device holds v model chunks; chunk c of device i is virtual stage
// s = c*p + i of a v*p-stage pipeline.  Microbatches go p at a time (m a
// multiple of p when v > 1): the k-th forward of a device is chunk
// (k mod vp) div p of microbatch (k div vp)*p + k mod p, the k-th backward
// the same microbatch of chunk v-1 - (k mod vp) div p.  Device i runs
// (p-1-i) + (v-1)p warm-up forwards (the fewest that cannot deadlock: the
// first backward to reach it needs all v chunks of the first microbatch
// group), then pairs (forward, backward), then the rest of the backwards;
// backwards stay whole (B then W), as in 1F1B, and each op starts when its
// device is free and its inputs exist.  With v = 1 this is 1F1B.
namespace {
struct ChunkPlaced {
    int type, chunk, mb;
    int64_t start, end;
};
}  // namespace

extern "C" int32_t zb_schedule_generate_interleaved(int32_t p, int32_t m, int32_t v, int32_t cF, int32_t cB,
                                                    int32_t cW, int32_t stage, zb_chunk_op* ops, int64_t* start,
                                                    int64_t* end, int32_t cap, int64_t* arrive_f, int64_t* arrive_b,
                                                    zb_sched_stats* stats) {
    if (p < 1 || m < 1 || v < 1 || (v > 1 && m % p) || stage < 0 || stage >= p || cF < 1 || cB < 1 || cW < 0)
        return ZB_EINVAL;
    if ((int64_t)p * m * v > 1 << 22) return ZB_EINVAL;
    const int n = v * m;  // forwards (and backwards) per device
    if ((ops || start || end) && cap < 3 * n) return ZB_EINVAL;
    const int S = v * p;  // virtual stages
    auto mb_of = [&](int k) { return (k / (p * v)) * p + k % p; };
    // per device: (is_backward, chunk, mb)
    struct Step { int bwd, chunk, mb; };
    std::vector<std::vector<Step>> seq(p);
    for (int i = 0; i < p; ++i) {
        const int warm = std::min((p - 1 - i) + (v - 1) * p, n);
        auto fwd = [&](int k) { return Step{0, (k % (p * v)) / p, mb_of(k)}; };
        auto bwd = [&](int k) { return Step{1, v - 1 - (k % (p * v)) / p, mb_of(k)}; };
        for (int k = 0; k < warm; ++k) seq[i].push_back(fwd(k));
        for (int k = 0; k < n - warm; ++k) {
            seq[i].push_back(fwd(warm + k));
            seq[i].push_back(bwd(k));
        }
        for (int k = n - warm; k < n; ++k) seq[i].push_back(bwd(k));
    }
    std::vector<int64_t> Fe((size_t)S * m, NOT_DONE), BWe((size_t)S * m, NOT_DONE);
    auto at = [m](int s, int j) { return (size_t)s * m + j; };
    std::vector<std::vector<ChunkPlaced>> placed(p);
    std::vector<size_t> next(p, 0);
    std::vector<int64_t> free_at(p, 0);
    std::vector<int> active(p, 0), peak(p, 0);
    size_t left = (size_t)2 * n * p;
    while (left > 0) {
        bool moved = false;
        for (int i = 0; i < p; ++i) {
            while (next[i] < seq[i].size()) {
                const Step q = seq[i][next[i]];
                const int s = q.chunk * p + i;
                int64_t ready;
                if (!q.bwd) ready = s == 0 ? 0 : Fe[at(s - 1, q.mb)];
                else ready = std::max(Fe[at(s, q.mb)], s == S - 1 ? int64_t(0) : BWe[at(s + 1, q.mb)]);
                if (ready == NOT_DONE) break;
                const int64_t st = std::max(ready, free_at[i]);
                if (!q.bwd) {
                    Fe[at(s, q.mb)] = st + cF;
                    free_at[i] = st + cF;
                    placed[i].push_back({ZB_OP_F, q.chunk, q.mb, st, st + cF});
                    peak[i] = std::max(peak[i], ++active[i]);
                } else {
                    BWe[at(s, q.mb)] = st + cB + cW;
                    free_at[i] = st + cB + cW;
                    placed[i].push_back({ZB_OP_B, q.chunk, q.mb, st, st + cB});
                    placed[i].push_back({ZB_OP_W, q.chunk, q.mb, st + cB, st + cB + cW});
                    --active[i];
                }
                ++next[i];
                --left;
                moved = true;
            }
        }
        if (!moved) return ZB_EINVAL;
    }
    const auto& mine = placed[stage];
    for (size_t k = 0; k < mine.size(); ++k) {
        if (ops) ops[k] = zb_chunk_op{mine[k].type, mine[k].chunk, mine[k].mb};
        if (start) start[k] = mine[k].start;
        if (end) end[k] = mine[k].end;
    }
    for (int c = 0; c < v; ++c) {
        const int s = c * p + stage;
        for (int j = 0; j < m; ++j) {
            if (arrive_f) arrive_f[(size_t)c * m + j] = s == 0 ? 0 : Fe[at(s - 1, j)];
            if (arrive_b) arrive_b[(size_t)c * m + j] = s == S - 1 ? 0 : BWe[at(s + 1, j)];
        }
    }
    if (stats) {
        int64_t mk = 0;
        for (int i = 0; i < p; ++i) mk = std::max(mk, placed[i].back().end);
        stats->makespan = mk;
        stats->busy = (int64_t)n * (cF + cB + cW);
        stats->first_start = mine.front().start;
        stats->last_end = mine.back().end;
        stats->peak_active = peak[stage];
        stats->n_ops = (int32_t)mine.size();
    }
    return (int32_t)mine.size();
}
