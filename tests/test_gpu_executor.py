"""Stage executor on the GPU (zb_stage_run_schedule through the C ABI).

* A replayed schedule computes exactly (bitwise) what issuing the same ops
  one by one computes: the executor only adds waits and clock stamps.
* ORDERED mode starts ops strictly in list order and never overlaps them.
* Emulated arrivals are honoured: no F or B starts before its arrival time.
* With the zero-bubble memory limit equal to the ring size, the ring is
  reused under the executor without corrupting results (slot reuse waits for
  the W that frees it).
* A malformed op list is rejected before anything is launched.
"""
import numpy as np
import pytest
import torch

import split_backward_amd as zb
import synth
from tests.gpu_helpers import make_stage, to_dev, to_f64

pytestmark = pytest.mark.gpu

SHAPE = synth.StageShape("llama", 256, 256, 344, n_layers=2, n_heads=2, n_kv_heads=1, head_dim=128)


def _inputs(m):
    xs = [to_dev(synth.make_x(SHAPE, j)) for j in range(m)]
    dys = [to_dev(synth.make_dy(SHAPE, j)) for j in range(m)]
    ys = [torch.empty((SHAPE.tokens, SHAPE.hidden), dtype=torch.bfloat16, device="cuda") for _ in range(m)]
    dxs = [torch.empty((SHAPE.tokens, SHAPE.hidden), dtype=torch.bfloat16, device="cuda") for _ in range(m)]
    return xs, ys, dys, dxs


def _sequential(ops, ring, m):
    st, _ = make_stage(SHAPE, ring)
    xs, ys, dys, dxs = _inputs(m)
    st.zero_grad()
    for t, j in ops:
        if t == "F":
            st.fwd(j, xs[j], ys[j])
        elif t == "B":
            st.bwd_input(j, dys[j], dxs[j])
        else:
            st.bwd_weight(j)
    torch.cuda.synchronize()
    return [to_f64(y) for y in ys], [to_f64(d) for d in dxs], [to_f64(w) for w in st.dw]


@pytest.mark.parametrize("kind,M,mode", [("1f1b", 0, zb.EXEC_ORDERED), ("zb", 8, zb.EXEC_ORDERED),
                                         ("zb", 4, zb.EXEC_ORDERED), ("zb", 8, zb.EXEC_FILLER)])
def test_replay_matches_sequential_and_honours_arrivals(kind, M, mode):
    p, stage, m = 4, 1, 8
    g = zb.schedule_generate(kind, p, m, M, (1, 1, 1), stage)
    ring = max(g["peak_active"], 1)
    unit_ms = 0.5
    st, _ = make_stage(SHAPE, ring)
    xs, ys, dys, dxs = _inputs(m)
    st.zero_grad()
    torch.cuda.synchronize()
    r = st.run_schedule(g["ops"], g["arrive_f"], g["arrive_b"], unit_ms, xs, ys, dys, dxs, mode=mode)
    torch.cuda.synchronize()
    y_ref, dx_ref, dw_ref = _sequential(g["ops"], ring, m)
    for a, b in zip([to_f64(y) for y in ys] + [to_f64(d) for d in dxs] + [to_f64(w) for w in st.dw],
                    y_ref + dx_ref + dw_ref):
        assert np.array_equal(a, b)
    iv = r["op_ms"]
    tol = 0.02  # ms of clock granularity and stamp-kernel placement
    for (t, j), (s, e) in zip(g["ops"], iv):
        assert e >= s
        if t == "F":
            assert s >= g["arrive_f"][j] * unit_ms - tol
        if t == "B":
            assert s >= g["arrive_b"][j] * unit_ms - tol
    if mode == zb.EXEC_ORDERED:
        for (s0, e0), (s1, e1) in zip(iv, iv[1:]):
            assert s1 >= e0 - 1e-6
    # every op's interval starts after its dependencies ended (the start stamp
    # follows the dependency waits, on either stream): W(j) after B(j), B(j)
    # after F(j), W(j) after W(j-1), F(j) after the W that freed its slot
    where = {(t, j): k for k, (t, j) in enumerate(g["ops"])}
    for (t, j), (s, e) in zip(g["ops"], iv):
        deps = {"W": [("B", j), ("W", j - 1)], "B": [("F", j)], "F": [("W", j - ring), ("F", j - 1)]}[t]
        for dep in deps:
            if dep in where:
                assert s >= iv[where[dep]][1] - 1e-3, ((t, j), dep)
    assert 0.0 <= r["in_window_idle"] < 1.0
    assert r["busy_ms"] <= r["window_ms"] + 1e-6


@pytest.mark.parametrize("mode", [zb.EXEC_ORDERED, zb.EXEC_FILLER], ids=["ordered", "filler"])
def test_replay_with_slot_reuse_matches_oracle(mode):
    """A replayed zero-bubble order whose ring is smaller than the number of
    microbatches (slots reused, W on the second stream in FILLER mode)
    against the fp64 oracle stage run on the same inputs, whole tensors:
    every y_j, dx_j and dW, relative Frobenius error <= 2e-2 and the element
    bound |got - ref| <= 2e-2 (|ref| + 5 rms(ref))."""
    from tests.gpu_helpers import oracle_stage
    from tests.stage_checks import Sampler
    p, stage, m, M = 4, 1, 10, 4
    g = zb.schedule_generate("zb", p, m, M, (1, 1, 1), stage)
    assert g["peak_active"] == M < m
    st, weights = make_stage(SHAPE, M)
    xs, ys, dys, dxs = _inputs(m)
    st.zero_grad()
    torch.cuda.synchronize()
    st.run_schedule(g["ops"], g["arrive_f"], g["arrive_b"], 0.3, xs, ys, dys, dxs, mode=mode)
    torch.cuda.synchronize()
    ref = oracle_stage(SHAPE, weights)
    xh = [synth.make_x(SHAPE, j).f64 for j in range(m)]
    dyh = [synth.make_dy(SHAPE, j).f64 for j in range(m)]
    oy = [ref.fwd(j, xh[j]) for j in range(m)]
    odx = [ref.bwd_input(j, dyh[j]) for j in range(m)]
    for j in range(m):
        ref.bwd_weight(j)
    S = Sampler(0)
    for j in range(m):
        S.record("y", to_f64(ys[j]), oy[j], 2e-2)
        S.record("dx", to_f64(dxs[j]), odx[j], 2e-2)
    for i, (d, o) in enumerate(zip(st.dw, ref.grad)):
        S.record(f"dw{i}", to_f64(d), o, 2e-2)


def test_zero_bubble_leaves_less_idle_than_1f1b():
    """[Guide] "Core Innovation 2": with W free to fill gaps, the stage's
    in-window idle under the zero-bubble order (M = 2p) is below 1F1B's."""
    p, stage, m = 4, 1, 8
    res = {}
    for kind, M in (("1f1b", 0), ("zb", 8)):
        g = zb.schedule_generate(kind, p, m, M, (1, 1, 1), stage)
        st, _ = make_stage(SHAPE, 8)
        xs, ys, dys, dxs = _inputs(m)
        # calibrate the unit to this stage's mean op time
        st.zero_grad()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        ev[0].record(); st.fwd(0, xs[0], ys[0]); ev[1].record()
        st.bwd_input(0, dys[0], dxs[0]); ev[2].record(); st.bwd_weight(0); ev[3].record()
        torch.cuda.synchronize()
        unit = sum(ev[i].elapsed_time(ev[i + 1]) for i in range(3)) / 3
        st.zero_grad()
        torch.cuda.synchronize()
        r = st.run_schedule(g["ops"], g["arrive_f"], g["arrive_b"], max(unit, 0.2), xs, ys, dys, dxs)
        res[kind] = r["in_window_idle"]
    assert res["zb"] < res["1f1b"], res


def test_malformed_schedule_rejected():
    import ctypes
    st, _ = make_stage(SHAPE, 2)
    xs, ys, dys, dxs = _inputs(2)
    with pytest.raises(ValueError):
        st.run_schedule([("F", 0), ("B", 5)], [0, 0], [0, 0], 0.1, xs, ys, dys, dxs)
    with pytest.raises(zb.ZbError) as e:
        st.run_schedule([("F", 0)], [-1.0, 0], [0, 0], 0.1, xs, ys, dys, dxs)
    assert e.value.code == zb.EINVAL
    # an unknown op type, straight through the C ABI
    ops = (zb.Op * 1)(zb.Op(7, 0))
    dbl = lambda v: (ctypes.c_double * 2)(*v)
    P = lambda ts: (ctypes.c_void_p * 2)(*[t.data_ptr() for t in ts])
    rc = zb.lib().zb_stage_run_schedule(st.handle, ops, 1, dbl([0, 0]), dbl([0, 0]), 0.1, P(xs), P(ys), P(dys),
                                        P(dxs), None, None, zb.EXEC_ORDERED, None, None)
    assert rc == zb.EINVAL
    torch.cuda.synchronize()


@pytest.mark.parametrize("mode", [zb.EXEC_ORDERED, zb.EXEC_FILLER], ids=["ordered", "filler"])
def test_interleaved_replay_over_two_chunks_matches_oracle(mode):
    """Interleaved 1F1B (zb_schedule_generate_interleaved, v = 2 chunks of
    one decoder layer each, stage 1 of p = 4, m = 8) replayed over two stage
    objects with zb_run_schedule_chunks: every chunk's y, dx and dW against
    the fp64 oracle of that chunk (whole tensors, 2e-2 and the element
    bound), arrivals honoured, and in ordered mode the list order kept."""
    from tests.gpu_helpers import oracle_stage
    from tests.stage_checks import Sampler
    p, stage, m, v = 4, 1, 8, 2
    chunk = synth.StageShape("llama", 256, 256, 344, n_layers=1, n_heads=2, n_kv_heads=1, head_dim=128)
    g = zb.schedule_generate_interleaved(p, m, v, (1, 1, 1), stage)
    peaks = []
    for c in range(v):  # stashed microbatches of each chunk at once, from the op list
        live = peak = 0
        for t, cc, _ in g["ops"]:
            if cc == c and t in "FW":
                live += 1 if t == "F" else -1
                peak = max(peak, live)
        peaks.append(peak)
    stages, weights = [], []
    for c in range(v):
        w = synth.make_weights(chunk, seed=c)
        st, _ = make_stage(chunk, peaks[c], weights=w)
        stages.append(st)
        weights.append(w)
    xin = [[synth.make_x(chunk, 100 * c + j) for j in range(m)] for c in range(v)]
    dyin = [[synth.make_dy(chunk, 100 * c + j) for j in range(m)] for c in range(v)]
    xs = [[to_dev(t) for t in row] for row in xin]
    dys = [[to_dev(t) for t in row] for row in dyin]
    ys = [[torch.empty((chunk.tokens, chunk.hidden), dtype=torch.bfloat16, device="cuda") for _ in range(m)]
          for _ in range(v)]
    dxs = [[torch.empty_like(t) for t in row] for row in ys]
    for st in stages:
        st.zero_grad()
    torch.cuda.synchronize()
    unit_ms = 0.3
    r = zb.run_schedule_chunks(stages, g["ops"], g["arrive_f"], g["arrive_b"], unit_ms, xs, ys, dys, dxs, mode=mode)
    torch.cuda.synchronize()
    S = Sampler(0)
    for c in range(v):
        ref = oracle_stage(chunk, weights[c])
        oy = [ref.fwd(j, xin[c][j].f64) for j in range(m)]
        odx = [ref.bwd_input(j, dyin[c][j].f64) for j in range(m)]
        for j in range(m):
            ref.bwd_weight(j)
            S.record("y", to_f64(ys[c][j]), oy[j], 2e-2)
            S.record("dx", to_f64(dxs[c][j]), odx[j], 2e-2)
        for i, (d, o) in enumerate(zip(stages[c].dw, ref.grad)):
            S.record(f"dw{i}", to_f64(d), o, 2e-2)
    iv = r["op_ms"]
    for (t, c, j), (s, e) in zip(g["ops"], iv):
        if t == "F":
            assert s >= g["arrive_f"][c][j] * unit_ms - 0.02
        if t == "B":
            assert s >= g["arrive_b"][c][j] * unit_ms - 0.02
    if mode == zb.EXEC_ORDERED:
        for (s0, e0), (s1, e1) in zip(iv, iv[1:]):
            assert s1 >= e0 - 1e-6
    assert 0.0 <= r["in_window_idle"] < 1.0


def test_chunk_executor_rejects_chunk_out_of_range():
    st, _ = make_stage(SHAPE, 2)
    xs, ys, dys, dxs = _inputs(1)
    with pytest.raises(zb.ZbError) as e:
        zb.run_schedule_chunks([st], [("F", 1, 0)], [[0.0]], [[0.0]], 0.1, [xs], [ys], [dys], [dxs])
    assert e.value.code == zb.EINVAL
    with pytest.raises(zb.ZbError) as e:
        zb.run_schedule_chunks([st, st], [("F", 0, 0)], [[0.0]] * 2, [[0.0]] * 2, 0.1, [xs] * 2, [ys] * 2, [dys] * 2,
                               [dxs] * 2)
    assert e.value.code == zb.EINVAL
    torch.cuda.synchronize()


def test_memory_limit_sweep_stash_matches_simulator():
    """ZB(M) for M = p .. 2p ([Guide] "Core Innovation 2": the memory limit
    between p and 2p in-flight microbatches): the simulator's peak of
    stashed microbatches equals the peak counted from its op list, a ring of
    exactly that many slots replays the order (result bit for bit that of
    sequential issue, which here is the oracle-checked path), and one slot
    fewer refuses it with ZB_ERING_FULL before any work of the refused op."""
    p, stage, m = 4, 1, 10
    for M in range(p, 2 * p + 1):
        g = zb.schedule_generate("zb", p, m, M, (1, 1, 1), stage)
        live = peak = 0
        for t, _ in g["ops"]:
            live += {"F": 1, "W": -1}.get(t, 0)
            peak = max(peak, live)
        assert peak == g["peak_active"] <= M
        st, _ = make_stage(SHAPE, peak)
        xs, ys, dys, dxs = _inputs(m)
        st.zero_grad()
        torch.cuda.synchronize()
        st.run_schedule(g["ops"], g["arrive_f"], g["arrive_b"], 0.05, xs, ys, dys, dxs)
        torch.cuda.synchronize()
        y_ref, dx_ref, dw_ref = _sequential(g["ops"], peak, m)
        for a, b in zip([to_f64(y) for y in ys] + [to_f64(d) for d in dxs] + [to_f64(w) for w in st.dw],
                        y_ref + dx_ref + dw_ref):
            assert np.array_equal(a, b)
        if peak > 1:
            small, _ = make_stage(SHAPE, peak - 1)
            small.zero_grad()
            with pytest.raises(zb.ZbError) as e:
                for t, j in g["ops"]:
                    if t == "F":
                        small.fwd(j, xs[j], ys[j])
                    elif t == "B":
                        small.bwd_input(j, dys[j], dxs[j])
                    else:
                        small.bwd_weight(j)
            assert e.value.code == zb.ERING_FULL
            torch.cuda.synchronize()
