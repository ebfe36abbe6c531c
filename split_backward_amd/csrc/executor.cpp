// One-GPU stage executor: replays a generated per-stage schedule with the
// arrivals of upstream activations and downstream gradients emulated by GPU
// waits on the device's constant-rate wall clock.  A stage may hold several
// model chunks (interleaved 1F1B), each its own zb_stage; an op names the
// chunk it runs on.
//
// F and B (the critical path of the Guide's "Core Innovation 1") run on the
// high stream behind their arrival waits; W runs on the low (filler) stream
// ("Core Innovation 2": W fills what would otherwise be idle time).  Both
// streams keep the default priority; the ordering the schedule asks for is
// enforced with events instead:
//   ORDERED: every op waits for the end of the op before it in the list, so
//            the GPU executes exactly the generated order.
//   FILLER:  W waits only for its own B (and F of a reused ring slot waits
//            for the W that frees it), so W soaks up whatever gaps remain.
// Optimizer-step ops (several iterations back to back) run on the high
// stream after every W issued before them.  Each op is bracketed by two
// clock-stamp kernels, the first issued after the op's dependency and
// arrival waits, so an interval covers only the time the op could run; idle
// time is the part of the stage's window [first op start, last op end] that
// no op interval covers.
#include <algorithm>
#include <cmath>
#include <vector>

#include "common.h"
#include "stage.h"

using namespace zb;

namespace {

struct StreamGuard {
    hipStream_t s = nullptr;
    bool own = false;
    ~StreamGuard() {
        if (own && s) (void)hipStreamDestroy(s);
    }
};

struct EventPool {
    std::vector<hipEvent_t> ev;
    ~EventPool() {
        for (auto e : ev) (void)hipEventDestroy(e);
    }
};

// An op of the run: type, chunk (index into the stage objects), microbatch.
struct RunOp {
    int type, chunk, mb;
};

// The replay behind both entry points.  Arrays x, y, dy, dx and the
// arrivals are indexed chunk * per_chunk + mb.
int32_t run_ops(const std::vector<zb_stage*>& chunks, const std::vector<RunOp>& ops, int per_chunk,
                const double* arrive_f, const double* arrive_b, double unit_ms, const void* const* x,
                void* const* y, const void* const* dy, void* const* dx, void* hi_stream, void* lo_stream, int32_t mode,
                zb_run_stats* stats, double* op_ms) {
    const int n = (int)ops.size();
    const int v = (int)chunks.size();
    // F, B and W ops carry a microbatch index into x, y, dy, dx and the
    // arrivals; an optimizer-step op (ZB_OP_O, from
    // zb_schedule_generate_iters) closes an iteration and resets every
    // chunk, whose own numbering then starts again at 0 with the next F.
    // local[k] is op k's microbatch in the chunks' numbering, checked here
    // before any work is issued.
    std::vector<int> local(n, 0);
    {
        int base = 0;
        bool reset = false;
        for (int k = 0; k < n; ++k) {
            const RunOp& o = ops[k];
            if (o.type < ZB_OP_F || o.type > ZB_OP_O || o.mb < 0 || o.chunk < 0 || o.chunk >= v)
                return fail(ZB_EINVAL, "zb_stage_run_schedule: malformed op " + std::to_string(k));
            if (o.type == ZB_OP_O) {
                reset = true;
                continue;
            }
            if (o.mb >= per_chunk)
                return fail(ZB_EINVAL, "zb_stage_run_schedule: op " + std::to_string(k) + " has a microbatch beyond the arrays");
            if (o.type == ZB_OP_F && reset) {
                base = o.mb;
                reset = false;
            }
            local[k] = o.mb - base;
            if (local[k] < 0 || reset)
                return fail(ZB_EINVAL, "zb_stage_run_schedule: op " + std::to_string(k) +
                                           " belongs to an iteration an optimizer step has closed");
        }
    }
    constexpr double MAX_ARRIVAL_MS = 30000.0;  // the wait kernel's cap
    for (int k = 0; k < n; ++k) {
        if (ops[k].type == ZB_OP_O) continue;
        const size_t a = (size_t)ops[k].chunk * per_chunk + ops[k].mb;
        if (!(arrive_f[a] >= 0.0) || !(arrive_b[a] >= 0.0) || arrive_f[a] > 1e6 || arrive_b[a] > 1e6)
            return fail(ZB_EINVAL, "zb_stage_run_schedule: arrival times must be in [0, 1e6] units");
        if (arrive_f[a] * unit_ms > MAX_ARRIVAL_MS || arrive_b[a] * unit_ms > MAX_ARRIVAL_MS)
            return fail(ZB_EINVAL, "zb_stage_run_schedule: an arrival lies more than 30 s after the run's start");
    }
    for (zb_stage* c : chunks)
        if (!c) return fail(ZB_EINVAL, "zb_stage_run_schedule: bad argument");
    if (!x || !y || !dy || !dx) return fail(ZB_EINVAL, "zb_stage_run_schedule: bad argument");

    StreamGuard hi, lo;
    hi.s = static_cast<hipStream_t>(hi_stream);
    lo.s = static_cast<hipStream_t>(lo_stream);
    if (!hi.s) {
        ZB_HIP(hipStreamCreateWithFlags(&hi.s, hipStreamNonBlocking));
        hi.own = true;
    }
    if (!lo.s) {
        ZB_HIP(hipStreamCreateWithFlags(&lo.s, hipStreamNonBlocking));
        lo.own = true;
    }
    EventPool pool;
    pool.ev.resize(n + 1, nullptr);
    for (auto& e : pool.ev) ZB_HIP(hipEventCreateWithFlags(&e, hipEventDisableTiming));

    const double hz = (double)wall_clock_hz();
    const double ticks_per_ms = hz / 1000.0;
    zb_stage* st0 = chunks[0];  // its workspace holds the run's clock stamps
    uint64_t* t0 = st0->stamps;
    uint64_t* stamp = st0->stamps + 1;           // 2 per op
    uint64_t* wait_end = st0->stamps + 1 + 2 * n;  // 1 per op

    int32_t rc = stamp_now(t0, hi.s);
    if (rc) return rc;
    ZB_HIP(hipEventRecord(pool.ev[n], hi.s));
    ZB_HIP(hipStreamWaitEvent(lo.s, pool.ev[n], 0));

    int prev = -1;
    hipStream_t prev_stream = nullptr;
    for (int k = 0; k < n && rc == ZB_OK; ++k) {
        const RunOp op = ops[k];
        const bool is_w = op.type == ZB_OP_W;
        hipStream_t s = is_w ? lo.s : hi.s;
        const size_t a = (size_t)op.chunk * per_chunk + op.mb;
        if (mode == ZB_EXEC_ORDERED && prev >= 0 && prev_stream != s) {
            hipError_t e = hipStreamWaitEvent(s, pool.ev[prev], 0);
            if (e != hipSuccess) { rc = fail(ZB_EHIP, "hipStreamWaitEvent failed"); break; }
        }
        // the op's own dependencies (on the other stream too) before its start stamp
        if (op.type == ZB_OP_O) {
            for (zb_stage* c : chunks)
                if ((rc = c->wait_deps(op.type, 0, s))) break;
        } else {
            rc = chunks[op.chunk]->wait_deps(op.type, local[k], s);
        }
        if (rc) break;
        if (op.type == ZB_OP_F || op.type == ZB_OP_B) {
            const double t = op.type == ZB_OP_F ? arrive_f[a] : arrive_b[a];
            const uint64_t delta = (uint64_t)std::llround(t * unit_ms * ticks_per_ms);
            rc = wait_until(t0, delta, wait_end + k, s);
            if (rc) break;
        }
        rc = stamp_now(stamp + 2 * k, s);
        if (rc) break;
        zb_stage* c = chunks[op.chunk];
        if (op.type == ZB_OP_F) rc = zb_fwd(c, local[k], x[a], y[a], s);
        else if (op.type == ZB_OP_B) rc = zb_bwd_input(c, local[k], dy[a], dx[a], s);
        else if (op.type == ZB_OP_W) rc = zb_bwd_weight_accum(c, local[k], s);
        else
            for (zb_stage* cc : chunks)  // waits for every W issued on the other stream
                if ((rc = zb_stage_sgd_step(cc, cc->lr, s))) break;
        if (rc) break;
        rc = stamp_now(stamp + 2 * k + 1, s);
        if (rc) break;
        hipError_t e = hipEventRecord(pool.ev[k], s);
        if (e != hipSuccess) { rc = fail(ZB_EHIP, "hipEventRecord failed"); break; }
        prev = k;
        prev_stream = s;
    }
    // Drain both streams whether or not the issue loop completed.
    hipError_t e1 = hipStreamSynchronize(hi.s);
    hipError_t e2 = hipStreamSynchronize(lo.s);
    if (rc) return rc;
    if (e1 != hipSuccess || e2 != hipSuccess) return fail(ZB_EHIP, "stream synchronize failed after the run");

    std::vector<uint64_t> host(1 + 3 * (size_t)n);
    ZB_HIP(hipMemcpy(host.data(), st0->stamps, host.size() * sizeof(uint64_t), hipMemcpyDeviceToHost));
    const uint64_t base = host[0];
    auto ms = [&](uint64_t t) { return ((double)(int64_t)(t - base)) / ticks_per_ms; };
    std::vector<std::pair<double, double>> iv(n);
    double late = 0.0;
    for (int k = 0; k < n; ++k) {
        iv[k] = {ms(host[1 + 2 * k]), ms(host[2 + 2 * k])};
        if (op_ms) {
            op_ms[2 * k] = iv[k].first;
            op_ms[2 * k + 1] = iv[k].second;
        }
        if (ops[k].type == ZB_OP_F || ops[k].type == ZB_OP_B) {
            const size_t a = (size_t)ops[k].chunk * per_chunk + ops[k].mb;
            const double t = (ops[k].type == ZB_OP_F ? arrive_f[a] : arrive_b[a]) * unit_ms;
            late += std::max(0.0, ms(host[1 + 2 * n + k]) - t);
        }
    }
    if (stats) {
        std::vector<std::pair<double, double>> srt = iv;
        std::sort(srt.begin(), srt.end());
        double busy = 0.0, cs = srt[0].first, ce = srt[0].second;
        for (size_t i = 1; i < srt.size(); ++i) {
            if (srt[i].first > ce) {
                busy += ce - cs;
                cs = srt[i].first;
                ce = srt[i].second;
            } else {
                ce = std::max(ce, srt[i].second);
            }
        }
        busy += ce - cs;
        double first = srt[0].first, last = 0.0;
        for (auto& q : iv) last = std::max(last, q.second);
        stats->t_first_start_ms = first;
        stats->t_last_end_ms = last;
        stats->window_ms = last - first;
        stats->busy_ms = busy;
        stats->in_window_idle = stats->window_ms > 0 ? (stats->window_ms - busy) / stats->window_ms : 0.0;
        stats->wait_late_ms = late;
    }
    return ZB_OK;
}

// Checks every entry point makes before anything else (host only, before
// the stages are looked at).
int32_t check_common(const void* ops, int32_t n, const double* arrive_f, const double* arrive_b, double unit_ms,
                     int32_t mode) {
    if (!ops || n < 1 || n > MAX_RUN_OPS || !arrive_f || !arrive_b)
        return fail(ZB_EINVAL, "zb_stage_run_schedule: bad op list or arrival arrays");
    if (!std::isfinite(unit_ms) || unit_ms < 0.0)
        return fail(ZB_EINVAL, "zb_stage_run_schedule: unit_ms must be finite and >= 0");
    if (mode != ZB_EXEC_ORDERED && mode != ZB_EXEC_FILLER) return fail(ZB_EINVAL, "zb_stage_run_schedule: bad mode");
    return ZB_OK;
}

}  // namespace

// The op list and the times are checked first (host only, before the stage
// is looked at): every wait the run would issue must end within the wait
// kernel's 30 s cap.
extern "C" int32_t zb_stage_run_schedule(zb_stage* st, const zb_op* ops, int32_t n, const double* arrive_f,
                                         const double* arrive_b, double unit_ms, const void* const* x, void* const* y,
                                         const void* const* dy, void* const* dx, void* hi_stream, void* lo_stream,
                                         int32_t mode, zb_run_stats* stats, double* op_ms) {
    int32_t rc = check_common(ops, n, arrive_f, arrive_b, unit_ms, mode);
    if (rc) return rc;
    std::vector<RunOp> run(n);
    int nmb = 0;
    for (int k = 0; k < n; ++k) {
        run[k] = RunOp{ops[k].type, 0, ops[k].mb};
        if (ops[k].type != ZB_OP_O) nmb = std::max(nmb, ops[k].mb + 1);
    }
    return run_ops({st}, run, nmb, arrive_f, arrive_b, unit_ms, x, y, dy, dx, hi_stream, lo_stream, mode, stats,
                   op_ms);
}

extern "C" int32_t zb_run_schedule_chunks(zb_stage* const* chunks, int32_t v, const zb_chunk_op* ops, int32_t n,
                                          int32_t m, const double* arrive_f, const double* arrive_b, double unit_ms,
                                          const void* const* x, void* const* y, const void* const* dy,
                                          void* const* dx, void* hi_stream, void* lo_stream, int32_t mode,
                                          zb_run_stats* stats, double* op_ms) {
    int32_t rc = check_common(ops, n, arrive_f, arrive_b, unit_ms, mode);
    if (rc) return rc;
    if (v < 1 || v > 64 || m < 1) return fail(ZB_EINVAL, "zb_run_schedule_chunks: bad chunk or microbatch count");
    if (!chunks) return fail(ZB_EINVAL, "zb_run_schedule_chunks: bad argument");
    std::vector<zb_stage*> cs(chunks, chunks + v);
    for (int a = 0; a < v; ++a)
        for (int b = a + 1; b < v; ++b)
            if (cs[a] && cs[a] == cs[b]) return fail(ZB_EINVAL, "zb_run_schedule_chunks: a stage object given twice");
    std::vector<RunOp> run(n);
    for (int k = 0; k < n; ++k) run[k] = RunOp{ops[k].type, ops[k].chunk, ops[k].mb};
    return run_ops(cs, run, m, arrive_f, arrive_b, unit_ms, x, y, dy, dx, hi_stream, lo_stream, mode, stats, op_ms);
}
