"""The stage executor at the benchmark shape, checked against the fp64 oracle.

The Llama-7B-shape stage (4 decoder layers, 4096 tokens, h 4096, ffn 11008,
32 heads) replays stage 3 of an emulated 8-stage pipeline for 16
microbatches in the zero-bubble order with memory limit 8, through
zb_stage_run_schedule, with an 8-slot stash ring: microbatches 8..15 reuse
the ring slots of 0..7, so F(j + 8) may start only once W(j) has finished
reading the slot ([Guide] "Memory Management & Activation Rollback": a
microbatch's activations are released by its weight-gradient pass).  In
FILLER mode W runs on the second stream, beside F and B.

The replay's outputs are then compared with the oracle ([Guide]
"Convergence and Numerical Stability": the split computes the same
gradients):

* microbatches 8..15: every F and B step of every layer from the stash the
  replay left, the replay's y_j and dx_j included;
* microbatches 0..7, whose stash the replay overwrote: the stage is reset
  and their F and B are issued again one by one (no W), every step is
  checked from that stash, and the replay's own y_j and dx_j are checked
  against the oracle's recomputation from it;
* dW of every linear and dgamma of every RMSNorm, summed by the oracle over
  all 16 microbatches from those stashes, against the replay's buffers.

A W that read a slot already refilled by a later F, or an F that overwrote a
slot before its W finished, puts another microbatch's activations into dW
and fails the last check.
"""
import pytest
import torch

import split_backward_amd as zb
import synth
from tests.gpu_helpers import make_stage, to_dev
from tests.stage_checks import Sampler, WeightGradAccumulator, check_microbatch_layer

pytestmark = pytest.mark.gpu

WL = synth.WORKLOADS["llama7b_stage4"]
SHAPE = WL["shape"]
M_MB = 16
RING = 8


def _replay(mode):
    st, _ = make_stage(SHAPE, RING)
    xs = [to_dev(synth.make_x(SHAPE, j)) for j in range(M_MB)]
    dys = [to_dev(synth.make_dy(SHAPE, j)) for j in range(M_MB)]
    ys = [torch.empty((SHAPE.tokens, SHAPE.hidden), dtype=torch.bfloat16, device="cuda") for _ in range(M_MB)]
    dxs = [torch.empty_like(y) for y in ys]
    g = zb.schedule_generate("zb", 8, M_MB, RING, (1, 1, 1), 3)
    assert g["peak_active"] == RING  # the order fills the ring, so slots are reused
    st.zero_grad()
    torch.cuda.synchronize()
    # unit of 5 ms: arrivals leave gaps (about the pass time at this shape)
    r = st.run_schedule(g["ops"], g["arrive_f"], g["arrive_b"], 5.0, xs, ys, dys, dxs, mode=mode)
    torch.cuda.synchronize()
    # dependency order of the replay's intervals: W(j) after B(j), F(j + 8) after W(j)
    where = {op: k for k, op in enumerate(g["ops"])}
    iv = r["op_ms"]
    for j in range(M_MB):
        assert iv[where[("W", j)]][0] >= iv[where[("B", j)]][1] - 1e-3
        if j + RING < M_MB:
            assert iv[where[("F", j + RING)]][0] >= iv[where[("W", j)]][1] - 1e-3
    return st, xs, dys, ys, dxs


@pytest.mark.timeout(900)
@pytest.mark.parametrize("mode", [zb.EXEC_ORDERED, zb.EXEC_FILLER], ids=["ordered", "filler"])
def test_replay_with_ring_reuse_matches_oracle(mode):
    print(f"executor full-size replay, mode {mode}", flush=True)
    st, xs, dys, ys, dxs = _replay(mode)
    dw = [d.clone() for d in st.dw]  # the replay's dW and dgamma, before the stage is reset
    L = SHAPE.n_layers
    S = Sampler(11)
    acc = WeightGradAccumulator(S, st, SHAPE)

    def check(j):
        for l in range(L):
            out = ys[j] if l == L - 1 else st.stash(j, l + 1, zb.L_X)
            dxl = dxs[j] if l == 0 else st.stash(j, l - 1, zb.L_DOUT)
            # a whole head's attention backward for two microbatches (it is the slow check)
            check_microbatch_layer(S, st, SHAPE, j, l, out, dxl, x_in=xs[j] if l == 0 else None,
                                   dy_in=dys[j] if l == L - 1 else None, attn_bwd=(j in (0, M_MB - 1) and l == 0))
        acc.add(j)

    for j in range(RING, M_MB):  # still resident after the replay
        check(j)
    # microbatches 0..7 again, F and B only, into the slots the replay refilled
    st.zero_grad()
    for j in range(RING):
        st.fwd(j, xs[j], torch.empty_like(ys[j]))
    for j in range(RING):
        st.bwd_input(j, dys[j], torch.empty_like(dxs[j]))
    torch.cuda.synchronize()
    for j in range(RING):
        check(j)  # the replay's y_j, dx_j against the oracle from this stash
    acc.check(dw)
    print({k: f"{v:.2e}" for k, v in S.err.items()})
