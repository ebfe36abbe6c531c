"""Helpers of the GPU parity tests: move synth inputs to the device, build a
libzb stage through the Python binding, run the fp64 oracle on the same
values."""
from __future__ import annotations

import numpy as np
import torch

import split_backward_amd as zb
import synth
from oracle import dense as od


to_dev = synth.to_device


def to_f64(x: torch.Tensor) -> np.ndarray:
    return x.detach().float().cpu().numpy().astype(np.float64)


def make_stage(shape: synth.StageShape, ring: int, weights=None):
    weights = weights or synth.make_weights(shape)
    dev_w = [to_dev(w) for w in weights]
    st = zb.Stage(shape.kind, shape.tokens, shape.hidden, shape.ffn, dev_w, dtype=shape.dtype,
                  n_layers=shape.n_layers, n_heads=shape.n_heads, n_kv_heads=shape.n_kv_heads,
                  head_dim=shape.head_dim if shape.kind == "llama" else 128, rms_eps=shape.rms_eps,
                  ring_slots=ring)
    return st, weights


def oracle_stage(shape: synth.StageShape, weights):
    dims = None
    if shape.kind == "llama":
        dims = od.LlamaDims(shape.hidden, shape.ffn, shape.n_heads, shape.n_kv_heads, shape.head_dim,
                            shape.rms_eps)
    return od.Stage(shape.kind, [w.f64 for w in weights], dims, shape.n_layers)


def run_both(shape: synth.StageShape, m: int, ring: int = None, order: str = "deferred"):
    """Run F/B/W for m microbatches on the GPU and in the oracle.
    order: "deferred" (all F, all B, then all W) or "immediate" (F B W per mb).
    Returns (gpu dict, oracle dict) of float64 arrays."""
    ring = ring or m
    st, weights = make_stage(shape, ring)
    ref = oracle_stage(shape, weights)
    xs = [synth.make_x(shape, j) for j in range(m)]
    dys = [synth.make_dy(shape, j) for j in range(m)]
    dxs_dev = [to_dev(x) for x in xs]
    dys_dev = [to_dev(d) for d in dys]
    st.zero_grad()
    ys, dxs = {}, {}
    if order == "deferred":
        for j in range(m):
            ys[j] = st.fwd(j, dxs_dev[j])
        for j in range(m):
            dxs[j] = st.bwd_input(j, dys_dev[j])
        for j in range(m):
            st.bwd_weight(j)
    else:
        for j in range(m):
            ys[j] = st.fwd(j, dxs_dev[j])
            dxs[j] = st.bwd_input(j, dys_dev[j])
            st.bwd_weight(j)
    torch.cuda.synchronize()
    gpu = {"y": [to_f64(ys[j]) for j in range(m)], "dx": [to_f64(dxs[j]) for j in range(m)],
           "dw": [to_f64(d) for d in st.dw]}
    oy = [ref.fwd(j, xs[j].f64) for j in range(m)]
    odx = [ref.bwd_input(j, dys[j].f64) for j in range(m)]
    for j in range(m):
        ref.bwd_weight(j)
    orc = {"y": oy, "dx": odx, "dw": ref.grad}
    return gpu, orc, st


def max_rel(gpu, orc):
    out = {}
    for key in ("y", "dx", "dw"):
        out[key] = max(od.rel_fro(a, b) for a, b in zip(gpu[key], orc[key]))
    return out
