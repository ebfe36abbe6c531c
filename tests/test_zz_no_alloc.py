"""zb_bwd_weight_accum_noalloc (the W pass with its scratch in the library's
fixed device array) against zb_bwd_weight_accum, through the C ABI.

Two Llama stages in a row, the second smaller (fewer tokens, narrower), two
microbatches each: every dW and dgamma after the no-allocation W calls
equals bit for bit what the ordinary W calls give on a twin stage with the
same weights and inputs.  The array keeps the previous call's partials, so
the smaller stage's calls also show that stale contents are never read.  A
stage whose dgamma partials exceed the array is rejected before anything
is launched."""
import numpy as np
import pytest
import torch

import split_backward_amd as zb
import synth
from tests.gpu_helpers import make_stage, to_dev, to_f64

pytestmark = pytest.mark.gpu

BIG = synth.StageShape("llama", 1024, 1024, 1376, n_layers=2, n_heads=8, n_kv_heads=4, head_dim=128)
SMALL = synth.StageShape("llama", 256, 512, 688, n_layers=1, n_heads=4, n_kv_heads=4, head_dim=128)


def _w(shape, noalloc):
    st, _ = make_stage(shape, 2)
    st.zero_grad()
    for j in range(2):
        st.fwd(j, to_dev(synth.make_x(shape, j)))
    for j in range(2):
        st.bwd_input(j, to_dev(synth.make_dy(shape, j)))
    for j in range(2):
        if noalloc:
            rc = zb.lib().zb_bwd_weight_accum_noalloc(st.handle, j, None)
            assert rc == zb.OK, zb.last_error()
        else:
            st.bwd_weight(j)
    torch.cuda.synchronize()
    return [to_f64(d) for d in st.dw]


def test_noalloc_w_equals_w_bitwise_two_stages_second_smaller():
    for shape in (BIG, SMALL):
        ref = _w(shape, False)
        got = _w(shape, True)
        assert any(np.any(r != 0) for r in ref)
        for i, (a, b) in enumerate(zip(got, ref)):
            assert np.array_equal(a, b), (shape.tokens, i)


def test_noalloc_rejects_a_stage_beyond_the_array():
    # ceil(16512 / 64) * 8192 * 4 bytes = 8.45 MB of partials > 8 MiB
    T, H, F = 16512, 8192, 8
    shapes = zb.weight_shapes("llama", H, F, 1, 64, 8, 128)
    w = [torch.zeros(s, dtype=torch.bfloat16, device="cuda") for s in shapes]
    st = zb.Stage("llama", T, H, F, w, n_layers=1, n_heads=64, n_kv_heads=8, head_dim=128, ring_slots=1)
    assert zb.lib().zb_bwd_weight_accum_noalloc(st.handle, 0, None) == zb.EINVAL
    assert "scratch" in zb.last_error()
    torch.cuda.synchronize()
