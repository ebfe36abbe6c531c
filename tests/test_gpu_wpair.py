"""W over two microbatches in one pass (zb_bwd_weight_accum_pair), on the GPU.

The weight-gradient pass only reads stashed operands and adds into dW, so two
ready microbatches can share one pass: each product runs once with K
spanning both microbatches' tokens.  Checked here:

* the pair equals W(mb) then W(mb + 1) within the fp32-accumulate tolerance
  (the two contributions are summed before they reach dW, so the rounding
  differs), and RMSNorm dgamma bit for bit (it is reduced per microbatch in
  the same order);
* stages whose products cannot take the two-segment kernel (fp32 linear,
  tokens not a multiple of 32) run the two single passes: bit for bit equal;
* the whole stage against the fp64 oracle;
* the state errors of the pair call.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import split_backward_amd as zb
import synth
from oracle import dense as od
from tests.gpu_helpers import make_stage, oracle_stage, to_dev, to_f64

pytestmark = pytest.mark.gpu

F32_TOL = 1e-5
BF16_TOL = 2e-2


def setup_module(module):
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    zb.lib()


def _run(shape, m, w_plan, ring=None):
    """All F, all B, then W as w_plan: ("W", j) single, ("P", j) pair j, j+1."""
    st, weights = make_stage(shape, ring or m)
    xs = [synth.make_x(shape, j) for j in range(m)]
    dys = [synth.make_dy(shape, j) for j in range(m)]
    st.zero_grad()
    for j in range(m):
        st.fwd(j, to_dev(xs[j]))
    for j in range(m):
        st.bwd_input(j, to_dev(dys[j]))
    for op, j in w_plan:
        if op == "W":
            st.bwd_weight(j)
        else:
            st.bwd_weight_pair(j)
    torch.cuda.synchronize()
    return [to_f64(d) for d in st.dw], weights, xs, dys


def _is_gain(shape, i):
    return shape.kind == "llama" and i % 6 >= 4


SINGLES4 = [("W", 0), ("W", 1), ("W", 2), ("W", 3)]


@pytest.mark.parametrize("shape,plan", [
    (synth.StageShape("llama", 256, 256, 344, n_layers=2, n_heads=2, n_kv_heads=1, head_dim=128),
     [("P", 0), ("P", 2)]),
    (synth.StageShape("llama", 384, 512, 1032, n_layers=1, n_heads=4, n_kv_heads=2, head_dim=128),
     [("W", 0), ("P", 1), ("W", 3)]),
    (synth.StageShape("mlp", 320, 136, 520), [("P", 0), ("P", 2)]),
])
def test_pair_matches_two_single_passes(shape, plan):
    single, _, _, _ = _run(shape, 4, SINGLES4)
    pair, _, _, _ = _run(shape, 4, plan)
    differs = False
    for i, (a, b) in enumerate(zip(pair, single)):
        if _is_gain(shape, i):
            assert np.array_equal(a, b), i
        else:
            assert od.rel_fro(a, b) <= F32_TOL, i
            differs = differs or not np.array_equal(a, b)
    assert differs  # the two-segment kernel ran (not the fallback, which is bitwise the singles)


@pytest.mark.parametrize("shape", [
    synth.StageShape("linear", 128, 256, 256, dtype="f32"),   # fp32 stage: no bf16 two-segment kernel
    synth.StageShape("mlp", 296, 136, 520),                   # 296 tokens: not a multiple of 32
])
def test_pair_falls_back_to_two_single_passes_bitwise(shape):
    single, _, _, _ = _run(shape, 4, SINGLES4)
    pair, _, _, _ = _run(shape, 4, [("P", 0), ("P", 2)])
    for i, (a, b) in enumerate(zip(pair, single)):
        assert np.array_equal(a, b), i


def test_pair_stage_against_oracle():
    shape = synth.StageShape("llama", 256, 256, 344, n_layers=2, n_heads=2, n_kv_heads=1, head_dim=128)
    dw, weights, xs, dys = _run(shape, 4, [("P", 0), ("P", 2)])
    ref = oracle_stage(shape, weights)
    for j in range(4):
        ref.fwd(j, xs[j].f64)
    for j in range(4):
        ref.bwd_input(j, dys[j].f64)
    for j in range(4):
        ref.bwd_weight(j)
    for i, (a, b) in enumerate(zip(dw, ref.grad)):
        assert od.rel_fro(a, b) <= BF16_TOL, i


def test_pair_at_llama7b_widths():
    """One decoder layer at the Llama-7B widths (h=4096, ffn=11008, 32 heads),
    256 tokens, two microbatches: pair against the two single passes."""
    shape = synth.StageShape("llama", 256, 4096, 11008, n_layers=1, n_heads=32, n_kv_heads=32, head_dim=128)
    single, _, _, _ = _run(shape, 2, [("W", 0), ("W", 1)])
    pair, _, _, _ = _run(shape, 2, [("P", 0)])
    for i, (a, b) in enumerate(zip(pair, single)):
        if _is_gain(shape, i):
            assert np.array_equal(a, b), i
        else:
            assert od.rel_fro(a, b) <= F32_TOL, i


def test_pair_state_errors():
    shape = synth.StageShape("mlp", 64, 64, 64)
    st, _ = make_stage(shape, ring=3)
    x = to_dev(synth.make_x(shape, 0))
    dy = to_dev(synth.make_dy(shape, 0))
    st.zero_grad()
    for j in range(3):
        st.fwd(j, x)
    st.bwd_input(0, dy)
    with pytest.raises(zb.ZbError) as e:
        st.bwd_weight_pair(0)         # B(1) not issued
    assert e.value.code == zb.ESTATE
    st.bwd_input(1, dy)
    st.bwd_input(2, dy)
    with pytest.raises(zb.ZbError) as e:
        st.bwd_weight_pair(1)         # W(0) is next
    assert e.value.code == zb.ESTATE
    st.bwd_weight_pair(0)
    with pytest.raises(zb.ZbError) as e:
        st.bwd_weight(1)              # already covered by the pair
    assert e.value.code == zb.ESTATE
    with pytest.raises(zb.ZbError) as e:
        st.bwd_weight_pair(2)         # microbatch 3 was never run
    assert e.value.code == zb.ESTATE
    st.bwd_weight(2)
    st.fwd(3, x)                      # slots freed by the pair and W(2)
    torch.cuda.synchronize()
    one, _ = make_stage(shape, ring=1)
    one.fwd(0, x)
    one.bwd_input(0, dy)
    with pytest.raises(zb.ZbError) as e:
        one.bwd_weight_pair(0)        # a one-slot ring never holds two microbatches
    assert e.value.code == zb.ESTATE
    torch.cuda.synchronize()
