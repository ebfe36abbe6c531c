"""The attention backward of a Llama stage (GPU, through the C ABI).

S and dP are computed once, by the kernel that owns a key block; it forms
dK and dV and stores dS^T, from which the dq kernel then forms dQ = dS K.
Checked on one-layer stages whose token counts span several key blocks: 640
tokens (128-key and 128-query blocks, an odd number of them, so the middle
block pairs with itself in the mirrored launch) and 256, 512 and 1024 (the
256-key and 256-query workgroups), with and without grouped-query heads (the
grouped shapes split a KV head's query heads over workgroups and add their
partial dK, dV in a fixed order):

* every head's dq and every KV head's dk and dv against the fp64 oracle
  ("Zero-Bubble Pipeline Parallelism Guide for LLMs", "Core Innovation 1":
  the attention backward lies wholly in B), computed from the GPU's own
  stashed q, k, v and output-projection gradient, per element as well as in
  norm;
* determinism: two stages on the same inputs give bitwise-equal dq, dk, dv
  and dx.  The first stage's workspace starts filled with NaN bit patterns
  and the second's with large finite ones, so a dS^T entry the dq kernel
  read without the dk/dv kernel having written it would show in either
  check.
"""
import numpy as np
import pytest
import torch

import split_backward_amd as zb
import synth
from oracle import dense as od
from tests.gpu_helpers import make_stage, to_dev
from tests.stage_checks import Sampler, f64

pytestmark = pytest.mark.gpu

D = 128


@pytest.mark.parametrize("T,nq,nkv", [(640, 2, 2), (640, 2, 1), (1024, 4, 2), (512, 2, 2), (256, 2, 1)])
def test_attention_backward_every_head_and_deterministic(T, nq, nkv):
    shape = synth.StageShape("llama", T, 256, 384, n_layers=1, n_heads=nq, n_kv_heads=nkv, head_dim=D)
    weights = synth.make_weights(shape)
    x, dy = synth.make_x(shape, 0), synth.make_dy(shape, 0)
    runs = []
    for fill in (0xFF, 0x7F):
        st, _ = make_stage(shape, 1, weights=weights)
        st.ws.fill_(fill)
        st.fwd(0, to_dev(x))
        dx = st.bwd_input(0, to_dev(dy))
        torch.cuda.synchronize()
        runs.append({"dx": dx.clone(), "dqkv": st.stash(0, 0, zb.L_DQKV).clone(),
                     "qkv": st.stash(0, 0, zb.L_QKV).clone(), "dh1": st.stash(0, 0, zb.L_DH1).clone(),
                     "wo": st.weights[1]})
    a, b = runs
    assert torch.equal(a["dqkv"], b["dqkv"])
    assert torch.equal(a["dx"], b["dx"])

    QD, KVD = nq * D, nkv * D
    qkv = f64(a["qkv"])
    q, k, v = qkv[:, :QD], qkv[:, QD:QD + KVD], qkv[:, QD + KVD:]
    da = f64(a["dh1"]) @ f64(a["wo"])  # the output projection's input gradient, [T][QD]
    dq = np.zeros((T, QD))
    dk = np.zeros((T, KVD))
    dv = np.zeros((T, KVD))
    for h in range(nq):
        g = h // (nq // nkv)
        dqh, dkp, dvp = od.attn_head_bwd(q, k, v, da, h, nq, nkv, D)
        dq[:, h * D:(h + 1) * D] = dqh
        dk[:, g * D:(g + 1) * D] += dkp
        dv[:, g * D:(g + 1) * D] += dvp
    got = f64(a["dqkv"])
    S = Sampler(0)
    for h in range(nq):
        S.record(f"dq head {h}", got[:, h * D:(h + 1) * D], dq[:, h * D:(h + 1) * D], 2e-2)
    for g in range(nkv):
        S.record(f"dk kv head {g}", got[:, QD + g * D:QD + (g + 1) * D], dk[:, g * D:(g + 1) * D], 2e-2)
        S.record(f"dv kv head {g}", got[:, QD + KVD + g * D:QD + KVD + (g + 1) * D], dv[:, g * D:(g + 1) * D], 2e-2)
    assert np.isfinite(got).all()
