"""Several iterations on the GPU: the optimizer step (zb_stage_sgd_step) and
the executor replaying the multi-iteration zero-bubble order
(zb_schedule_generate_iters) through the C ABI.

* The step equals the oracle's sgd_step bit for bit (bf16 and fp32 stages),
  clears dW and resets the stage for the next iteration.
* A two-iteration replay, ordered or filler, computes bit for bit what
  issuing the same ops one by one computes (optimizer steps included, so the
  second iteration runs on the updated weights), and honours the arrivals.
* An op list with an op of an iteration an optimizer step has closed is
  rejected before anything is launched.
"""
import numpy as np
import pytest
import torch

import split_backward_amd as zb
import synth
from oracle import dense as od
from tests.gpu_helpers import make_stage, to_dev, to_f64

pytestmark = pytest.mark.gpu

SHAPE = synth.StageShape("llama", 256, 256, 344, n_layers=2, n_heads=2, n_kv_heads=1, head_dim=128)
LR = 0.05


def setup_module(module):
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    zb.lib()


@pytest.mark.parametrize("shape", [SHAPE, synth.StageShape("linear", 128, 256, 264, dtype="f32")])
def test_sgd_step_matches_oracle_bitwise(shape):
    st, _ = make_stage(shape, 2)
    st.zero_grad()
    for j in range(2):
        st.fwd(j, to_dev(synth.make_x(shape, j)))
    for j in range(2):
        st.bwd_input(j, to_dev(synth.make_dy(shape, j)))
    for j in range(2):
        st.bwd_weight(j)
    torch.cuda.synchronize()
    w0 = [to_f64(w) for w in st.weights]
    dw0 = [d.detach().cpu().numpy().copy() for d in st.dw]
    st.sgd_step(LR)
    torch.cuda.synchronize()
    moved = False
    for i, (w, ref_w, d) in enumerate(zip(st.weights, w0, dw0)):
        ref = od.sgd_step(ref_w, d, LR, shape.dtype)
        assert np.array_equal(to_f64(w), ref), i
        # (an RMSNorm gain of 1 may not move: lr * dgamma is below half a bf16 unit of 1)
        moved = moved or not np.array_equal(ref, ref_w)
    assert moved
    for d in st.dw:
        assert not d.any()
    st.fwd(0, to_dev(synth.make_x(shape, 0)))  # the stage starts a new iteration at microbatch 0
    torch.cuda.synchronize()


def test_sgd_step_orders_the_next_forward_on_another_stream():
    """The optimizer step and the next iteration's first F issued on two
    different streams compute bit for bit what issuing both on one stream
    computes: the next F waits for the step on the device, whatever stream
    it is issued on."""
    outs = []
    for two_streams in (False, True):
        st, _ = make_stage(SHAPE, 2)
        st.zero_grad()
        xs = [to_dev(synth.make_x(SHAPE, j)) for j in range(2)]
        for j in range(2):
            st.fwd(j, xs[j])
        for j in range(2):
            st.bwd_input(j, to_dev(synth.make_dy(SHAPE, j)))
        for j in range(2):
            st.bwd_weight(j)
        torch.cuda.synchronize()
        s1 = torch.cuda.Stream()
        s2 = torch.cuda.Stream() if two_streams else s1
        st.sgd_step(LR, stream=s1)
        y = st.fwd(0, xs[0], stream=s2)
        torch.cuda.synchronize()
        outs.append((to_f64(y), [to_f64(w) for w in st.weights]))
    assert np.array_equal(outs[0][0], outs[1][0])
    for a, b in zip(outs[0][1], outs[1][1]):
        assert np.array_equal(a, b)


def _inputs(m):
    xs = [to_dev(synth.make_x(SHAPE, j)) for j in range(m)]
    dys = [to_dev(synth.make_dy(SHAPE, j)) for j in range(m)]
    ys = [torch.empty((SHAPE.tokens, SHAPE.hidden), dtype=torch.bfloat16, device="cuda") for _ in range(m)]
    dxs = [torch.empty((SHAPE.tokens, SHAPE.hidden), dtype=torch.bfloat16, device="cuda") for _ in range(m)]
    return xs, ys, dys, dxs


def _snapshot(st, ys, dxs):
    return ([to_f64(w) for w in st.weights], [to_f64(d) for d in st.dw], [to_f64(y) for y in ys],
            [to_f64(d) for d in dxs])


@pytest.mark.parametrize("kind,mode", [("zb", zb.EXEC_ORDERED), ("zb", zb.EXEC_FILLER), ("1f1b", zb.EXEC_ORDERED)])
def test_two_iteration_replay_matches_sequential(kind, mode):
    p, stage, m, n_iter = 4, 1, 4, 2
    g = zb.schedule_generate_iters(p, m, 4 if kind == "zb" else 0, (2, 2, 2), 1, n_iter, stage, kind=kind)
    M = max(g["peak_active"], 1)  # ring slots
    ops = g["ops"]
    assert [t for t, _ in ops].count("O") == n_iter
    # one set of per-microbatch buffers per iteration (iteration 2 reuses the inputs of iteration 1)
    xs, ys, dys, dxs = _inputs(m)
    ys2 = [torch.empty_like(y) for y in ys]
    dxs2 = [torch.empty_like(d) for d in dxs]
    X, Y, DY, DX = xs + xs, ys + ys2, dys + dys, dxs + dxs2

    # sequential issue of the same ops
    st, _ = make_stage(SHAPE, M)
    st.zero_grad()
    base = 0
    for t, k in ops:
        if t == "O":
            st.sgd_step(LR)
            base = None
            continue
        if base is None:
            base = k
        j = k - base
        if t == "F":
            st.fwd(j, X[k], Y[k])
        elif t == "B":
            st.bwd_input(j, DY[k], DX[k])
        else:
            st.bwd_weight(j)
    torch.cuda.synchronize()
    ref = _snapshot(st, Y, DX)

    # the executor
    unit_ms = 0.25
    st2, _ = make_stage(SHAPE, M)
    st2.set_lr(LR)
    st2.zero_grad()
    ys_b = [torch.empty_like(y) for y in Y]
    dxs_b = [torch.empty_like(d) for d in DX]
    torch.cuda.synchronize()
    r = st2.run_schedule(ops, g["arrive_f"], g["arrive_b"], unit_ms, X, ys_b, DY, dxs_b, mode=mode)
    torch.cuda.synchronize()
    got = _snapshot(st2, ys_b, dxs_b)
    for a_list, b_list in zip(got, ref):
        for a, b in zip(a_list, b_list):
            assert np.array_equal(a, b)
    # the second iteration ran on updated weights: its outputs differ from the first's
    assert not np.array_equal(got[2][0], got[2][m])
    # arrivals honoured: no F or B starts before its arrival
    for (t, k), (s, _) in zip(ops, r["op_ms"]):
        if t in "FB":
            a = (g["arrive_f"] if t == "F" else g["arrive_b"])[k] * unit_ms
            assert s >= a - 0.05, (t, k, s, a)
    if mode == zb.EXEC_ORDERED:
        ends = [e for _, e in r["op_ms"]]
        starts = [s for s, _ in r["op_ms"]]
        assert all(starts[i + 1] >= ends[i] - 1e-3 for i in range(len(ops) - 1))


def test_replay_rejects_op_of_closed_iteration():
    st, _ = make_stage(SHAPE, 2)
    xs, ys, dys, dxs = _inputs(2)
    bad = [("F", 0), ("B", 0), ("W", 0), ("O", 0), ("B", 0)]  # B of the closed iteration after its step
    with pytest.raises(zb.ZbError) as e:
        st.run_schedule(bad, [0, 0], [0, 0], 0.1, xs, ys, dys, dxs)
    assert e.value.code == zb.EINVAL
    # after the step the stage's numbering restarts at the next F (global 5):
    # a B of global index 4 would be microbatch -1 of the new iteration
    bad2 = [("F", 0), ("B", 0), ("W", 0), ("O", 0), ("F", 5), ("B", 4)]
    X, Y, DY, DX = xs * 3, ys * 3, dys * 3, dxs * 3
    with pytest.raises(zb.ZbError) as e:
        st.run_schedule(bad2, [0] * 6, [0] * 6, 0.1, X, Y, DY, DX)
    assert e.value.code == zb.EINVAL
    torch.cuda.synchronize()
