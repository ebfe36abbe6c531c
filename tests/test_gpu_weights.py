"""The stage's own weight copies follow the caller's weights (GPU, through
the C ABI).

A bf16 Llama stage's B pass multiplies by transposed copies [in][out] of its
linear weights that it keeps in its workspace; an fp8 stage's F and B
multiply by E4M3 copies.  Both are made by the first pass that needs them.
After the caller writes new values into its weight tensors and calls
zb_stage_weights_changed, a full F, B and W matches the oracle run on the
new values (the old values would miss it by far: the two weight sets are
independent draws).
"""
import pytest
import torch

import split_backward_amd as zb
import synth
from oracle import dense as od
from oracle import fp8 as o8
from tests.gpu_helpers import make_stage, oracle_stage, to_dev, to_f64

pytestmark = pytest.mark.gpu

SHAPE = synth.StageShape("llama", 256, 256, 384, n_layers=2, n_heads=2, n_kv_heads=1, head_dim=128)


def _pass(st, m, xs, dys):
    st.zero_grad()
    ys = [st.fwd(j, to_dev(xs[j])) for j in range(m)]
    dxs = [st.bwd_input(j, to_dev(dys[j])) for j in range(m)]
    for j in range(m):
        st.bwd_weight(j)
    torch.cuda.synchronize()
    return [to_f64(y) for y in ys] + [to_f64(d) for d in dxs] + [to_f64(d) for d in st.dw]


def _oracle(ref, m, xs, dys):
    oy = [ref.fwd(j, xs[j].f64) for j in range(m)]
    odx = [ref.bwd_input(j, dys[j].f64) for j in range(m)]
    for j in range(m):
        ref.bwd_weight(j)
    return oy + odx + list(ref.grad)


@pytest.mark.parametrize("dtype,tol", [("bf16", 2e-2), ("fp8", 0.25)])
def test_weights_changed_refreshes_the_stage_copies(dtype, tol):
    shape = synth.StageShape(**{**SHAPE.__dict__, "dtype": "bf16"})
    m = 2
    first = synth.make_weights(shape)
    second = synth.make_weights(shape, seed=1234)
    if dtype == "bf16":
        st, _ = make_stage(shape, m, weights=first)
    else:
        st = zb.Stage("llama", shape.tokens, shape.hidden, shape.ffn, [to_dev(w) for w in first], dtype="fp8",
                      n_layers=shape.n_layers, n_heads=shape.n_heads, n_kv_heads=shape.n_kv_heads,
                      head_dim=shape.head_dim, ring_slots=m)
    xs = [synth.make_x(shape, j) for j in range(m)]
    dys = [synth.make_dy(shape, j) for j in range(m)]
    _pass(st, m, xs, dys)  # the copies now hold the first weights

    with torch.no_grad():
        for dev, w in zip(st.weights, second):
            dev.copy_(to_dev(w))
    st.weights_changed()
    got = _pass(st, m, xs, dys)

    dims = od.LlamaDims(shape.hidden, shape.ffn, shape.n_heads, shape.n_kv_heads, shape.head_dim, shape.rms_eps)
    if dtype == "bf16":
        ref_new, ref_old = oracle_stage(shape, second), oracle_stage(shape, first)
    else:
        ref_new = o8.Fp8LlamaStage([w.f64 for w in second], dims, shape.n_layers)
        ref_old = o8.Fp8LlamaStage([w.f64 for w in first], dims, shape.n_layers)
    new = _oracle(ref_new, m, xs, dys)
    old = _oracle(ref_old, m, xs, dys)
    errs = [od.rel_fro(a, b) for a, b in zip(got, new)]
    assert max(errs) <= tol, errs
    # the check discriminates: the weight gradients under the first weights
    # are far away (the outputs less so: the residual stream dominates them)
    assert min(od.rel_fro(a, b) for a, b in zip(got[2 * m:], old[2 * m:])) > 0.5
