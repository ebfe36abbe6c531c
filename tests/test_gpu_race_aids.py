"""Debug aids of the stage on the GPU (zb_stage_set_debug, zb_stage_debug_report),
through the C ABI.

The ring discipline under test: a microbatch's stash is freed only once its
W has run, so a slot is reused only after that W ("Zero-Bubble Pipeline
Parallelism Guide for LLMs", "Memory Management & Activation Rollback").

* Slow W: every W pass first waits 2 ms on the device.  In FILLER mode (W on
  the second stream) with a ring smaller than the number of microbatches, an
  F that reused a slot before the delayed W had read it would corrupt that
  W's operands.  The slot tags find no mismatch, every F into a reused slot
  starts after the W that freed it ended, and y, dx and dW equal bit for bit
  those of the same order replayed without delay in ORDERED mode.
* Serialize mode computes the same bits as plain issue.
* The tags do detect a wrong slot state: enabling them while a microbatch is
  in flight resets its tag to "unused", and its B and W then report.
* Arrival delays injected from the host move only the timing: the results
  stay bitwise equal, the delayed F starts after its new arrival.
"""
import numpy as np
import pytest
import torch

import split_backward_amd as zb
import synth
from tests.gpu_helpers import make_stage, to_dev, to_f64

pytestmark = pytest.mark.gpu

SHAPE = synth.StageShape("llama", 256, 256, 344, n_layers=2, n_heads=2, n_kv_heads=1, head_dim=128)
P, STAGE, M_MB, RING = 4, 1, 10, 4


def _inputs(m):
    xs = [to_dev(synth.make_x(SHAPE, j)) for j in range(m)]
    dys = [to_dev(synth.make_dy(SHAPE, j)) for j in range(m)]
    ys = [torch.empty((SHAPE.tokens, SHAPE.hidden), dtype=torch.bfloat16, device="cuda") for _ in range(m)]
    dxs = [torch.empty((SHAPE.tokens, SHAPE.hidden), dtype=torch.bfloat16, device="cuda") for _ in range(m)]
    return xs, ys, dys, dxs


def _replay(g, mode, unit_ms, arrive_f=None, **debug):
    st, _ = make_stage(SHAPE, RING)
    xs, ys, dys, dxs = _inputs(M_MB)
    st.zero_grad()
    if debug:
        st.set_debug(**debug)
    torch.cuda.synchronize()
    r = st.run_schedule(g["ops"], arrive_f if arrive_f is not None else g["arrive_f"], g["arrive_b"], unit_ms,
                        xs, ys, dys, dxs, mode=mode)
    torch.cuda.synchronize()
    out = [to_f64(y) for y in ys] + [to_f64(d) for d in dxs] + [to_f64(w) for w in st.dw]
    return st, r, out


def _zb_order():
    g = zb.schedule_generate("zb", P, M_MB, RING, (1, 1, 1), STAGE)
    assert g["peak_active"] == RING < M_MB
    return g


def test_slow_w_never_loses_its_slot():
    g = _zb_order()
    _, _, ref = _replay(g, zb.EXEC_ORDERED, 0.3)
    delay_us = 2000
    st, r, got = _replay(g, zb.EXEC_FILLER, 0.3, slot_tags=True, w_delay_us=delay_us)
    n, last = st.debug_report()
    assert n == 0, last
    for a, b in zip(got, ref):
        assert np.array_equal(a, b)
    iv = {op: se for op, se in zip(map(tuple, g["ops"]), r["op_ms"])}
    for j in range(M_MB):
        s, e = iv[("W", j)]
        assert e - s >= delay_us * 1e-3 * 0.95  # the delay ran inside W's interval
        if j + RING < M_MB:  # F(j + R) reuses W(j)'s slot
            assert iv[("F", j + RING)][0] >= e - 1e-3


def test_serialize_mode_computes_the_same_bits():
    g = _zb_order()
    _, _, ref = _replay(g, zb.EXEC_ORDERED, 0.3)
    st, _, got = _replay(g, zb.EXEC_FILLER, 0.3, slot_tags=True, serialize=True)
    assert st.debug_report()[0] == 0
    for a, b in zip(got, ref):
        assert np.array_equal(a, b)


def test_tags_report_a_slot_in_the_wrong_state():
    st, _ = make_stage(SHAPE, 2)
    xs, ys, dys, dxs = _inputs(3)
    st.zero_grad()
    st.set_debug(slot_tags=True)
    st.fwd(0, xs[0], ys[0])
    st.bwd_input(0, dys[0], dxs[0])
    assert st.debug_report() == (0, None)
    st.set_debug(slot_tags=False)
    st.fwd(1, xs[1], ys[1])  # in flight (slot 1 tagged "F done") when the tags are reset
    st.set_debug(slot_tags=True)  # every tag back to "unused"
    st.bwd_weight(0)  # slot 0 expected "B(0) done" = 2
    n, last = st.debug_report()
    assert n == 1 and last == {"op": "W", "mb": 0, "slot": 0, "found": -1, "expected": 2}
    st.bwd_input(1, dys[1], dxs[1])  # slot 1 expected "F(1) done" = 5
    n, last = st.debug_report()
    assert n == 2 and last == {"op": "B", "mb": 1, "slot": 1, "found": -1, "expected": 5}
    st.bwd_weight(1)  # B(1) set the tag to 6 after its check: W(1) finds what it expects
    st.fwd(2, xs[2], ys[2])  # slot 0, W(0) done: free
    assert st.debug_report()[0] == 2
    with pytest.raises(zb.ZbError):
        st.set_debug(w_delay_us=-1)
    st.set_debug()
    with pytest.raises(zb.ZbError):
        st.debug_report()  # tags disabled


def test_injected_arrival_delay_changes_timing_only():
    g = _zb_order()
    unit = 0.3
    _, r0, ref = _replay(g, zb.EXEC_ORDERED, unit)
    late = list(g["arrive_f"])
    j, extra = 6, 40  # F(6) arrives 40 units (12 ms) late
    late[j] += extra
    _, r1, got = _replay(g, zb.EXEC_ORDERED, unit, arrive_f=late)
    for a, b in zip(got, ref):
        assert np.array_equal(a, b)
    iv = {op: se for op, se in zip(map(tuple, g["ops"]), r1["op_ms"])}
    assert iv[("F", j)][0] >= late[j] * unit - 0.02
    # the stage's end moves by at most the delay (plus clock slack)
    assert r1["t_last_end_ms"] <= r0["t_last_end_ms"] + extra * unit + 1.0
