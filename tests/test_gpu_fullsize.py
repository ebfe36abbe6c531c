"""Full-size Llama stage parity (GPU, through the C ABI).

1. Full widths (hidden, ffn, heads) with the token count reduced so the fp64
   oracle finishes in seconds: whole-stage parity, element by element.
2. The exact configuration the benchmark times (all layers, 4096 tokens, the
   benchmark's ring size, W per microbatch and W over a pair of microbatches):
   every F / B / W product, the RMSNorms and the attention core are checked
   on sampled outputs that the oracle recomputes
   one by one in fp64 from the GPU's own stashed operands (the inputs of
   each step), so a wrong tile, epilogue or index anywhere shows up.

Tolerances (relative Frobenius error over the samples): 5e-3 for products
and norms computed from the GPU's own bf16 operands (bf16 output rounding
<= 2^-9 plus fp32 accumulation), 1e-2 for attention rows (bf16 probabilities
in the second product), 2e-2 (the stage bar) for whole-stage comparisons and
the attention backward.
"""
import math

import numpy as np
import pytest
import torch

import split_backward_amd as zb
import synth
from oracle import dense as od
from tests.gpu_helpers import make_stage, max_rel, run_both, to_dev

pytestmark = pytest.mark.gpu


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name,tokens,layers", [("llama7b_stage4", 256, 1), ("llama70b_slice2", 128, 1)])
def test_full_width_reduced_tokens(name, tokens, layers):
    s = synth.WORKLOADS[name]["shape"]
    shape = synth.StageShape("llama", tokens, s.hidden, s.ffn, n_layers=layers, n_heads=s.n_heads,
                             n_kv_heads=s.n_kv_heads, head_dim=s.head_dim)
    gpu, orc, _ = run_both(shape, 2 if name == "llama7b_stage4" else 1)
    r = max_rel(gpu, orc)
    assert max(r.values()) <= 2e-2, r


class Sampler:
    def __init__(self, seed):
        self.rng = np.random.default_rng(seed)
        self.err = {}

    def idx(self, n, k=64):
        return self.rng.integers(0, n, size=k)

    def record(self, key, got, ref, tol):
        e = od.rel_fro(got, ref)
        self.err[key] = max(self.err.get(key, 0.0), e)
        assert e <= tol, (key, e)


def _nt_samples(S: Sampler, key, A, B, C, tol=5e-3, R=None):
    """C[r, c] (+ R[r, c]) == A[r] . B[c] on 64 random entries."""
    rows = S.idx(A.shape[0])
    cols = S.idx(B.shape[0])
    rt = torch.as_tensor(rows, device=A.device)
    ct = torch.as_tensor(cols, device=A.device)
    ref = od.gemm_nt_entries(f64(A[rt]), f64(B[ct]), range(len(rows)), range(len(cols)))
    if R is not None:
        ref = ref + f64(R[rt, ct])
    S.record(key, f64(C[rt, ct]), ref, tol)


def _nn_samples(S: Sampler, key, A, W, C, tol=5e-3):
    """C[r, c] == sum_k A[r, k] W[k, c]  (W stored [K, N])."""
    rows = S.idx(A.shape[0])
    cols = S.idx(W.shape[1])
    rt = torch.as_tensor(rows, device=A.device)
    ct = torch.as_tensor(cols, device=A.device)
    ref = od.gemm_nt_entries(f64(A[rt]), f64(W[:, ct]).T, range(len(rows)), range(len(cols)))
    S.record(key, f64(C[rt, ct]), ref, tol)


def _w_samples(S: Sampler, key, dYs, Xs, dW, tol=5e-3):
    """dW[o, i] == sum_j sum_t dY_j[t, o] X_j[t, i]."""
    o = S.idx(dW.shape[0])
    i = S.idx(dW.shape[1])
    ot = torch.as_tensor(o, device=dW.device)
    it = torch.as_tensor(i, device=dW.device)
    ref = np.zeros(len(o))
    for dY, X in zip(dYs, Xs):
        ref += np.sum(f64(dY[:, ot]) * f64(X[:, it]), axis=0)
    S.record(key, f64(dW[ot, it]), ref, tol)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name,w_pair", [("llama7b_stage4", False), ("llama7b_stage4", True),
                                         ("llama70b_slice2", False), ("llama70b_slice2", True)])
def test_benchmark_configuration_sampled(name, w_pair):
    """w_pair: W of the two microbatches as one pass (two K segments), as the
    benchmark issues adjacent W ops; otherwise one W per microbatch."""
    wl = synth.WORKLOADS[name]
    shape = wl["shape"]
    ring = wl.get("ring", wl["m"])
    st, _ = make_stage(shape, ring)
    T, H, F = shape.tokens, shape.hidden, shape.ffn
    nq, nkv, d = shape.n_heads, shape.n_kv_heads, shape.head_dim
    QD, KVD = nq * d, nkv * d
    eps = shape.rms_eps
    m = 2
    xs = [to_dev(synth.make_x(shape, j)) for j in range(m)]
    dys = [to_dev(synth.make_dy(shape, j)) for j in range(m)]
    st.zero_grad()
    ys = [st.fwd(j, xs[j]) for j in range(m)]
    dxs = [st.bwd_input(j, dys[j]) for j in range(m)]
    if w_pair:
        st.bwd_weight_pair(0)
    else:
        for j in range(m):
            st.bwd_weight(j)
    torch.cuda.synchronize()

    S = Sampler(7)
    L = shape.n_layers
    for l in range(L):
        wqkv, wo, wgu, wd, g1, g2 = st.weights[6 * l:6 * l + 6]
        for j in range(m):
            T_ = lambda which: st.stash(j, l, which)
            x, r1, n1, qkv, a = T_(zb.L_X), T_(zb.L_R1), T_(zb.L_N1), T_(zb.L_QKV), T_(zb.L_A)
            h1, r2, n2, gu, sw = T_(zb.L_H1), T_(zb.L_R2), T_(zb.L_N2), T_(zb.L_GU), T_(zb.L_S)
            dout, dgu, dn2, dh1, dqkv, dn1 = (T_(zb.L_DOUT), T_(zb.L_DGU), T_(zb.L_DN2), T_(zb.L_DH1),
                                              T_(zb.L_DQKV), T_(zb.L_DN1))
            out = ys[j] if l == L - 1 else st.stash(j, l + 1, zb.L_X)
            dxl = dxs[j] if l == 0 else st.stash(j, l - 1, zb.L_DOUT)
            if l == 0:
                S.record("x copy", f64(x[:4]), f64(xs[j][:4]), 0.0)
            if l == L - 1:
                S.record("dy copy", f64(dout[:4]), f64(dys[j][:4]), 0.0)
            rows = S.idx(T, 8)
            rt = torch.as_tensor(rows, device=x.device)
            # ---- F ----
            nref, _, _ = od.rms_fwd(f64(x[rt]), f64(g1), eps)
            S.record("rms1", f64(n1[rt]), nref, 5e-3)
            _nt_samples(S, "qkv", n1, wqkv, qkv)
            qf, kf, vf = f64(qkv[:, :QD]), f64(qkv[:, QD:QD + KVD]), f64(qkv[:, QD + KVD:])
            for h in (0, nq - 1):
                arows = np.concatenate([[0, 1, T - 1], S.idx(T, 5)])
                o_ref, _ = od.attn_rows_fwd(qf, kf, vf, h, arows, nq, nkv, d)
                S.record("attn fwd", f64(a[torch.as_tensor(arows, device=a.device), h * d:(h + 1) * d]), o_ref, 1e-2)
            _nt_samples(S, "o proj + residual", a, wo, h1, R=x)
            nref, _, _ = od.rms_fwd(f64(h1[rt]), f64(g2), eps)
            S.record("rms2", f64(n2[rt]), nref, 5e-3)
            _nt_samples(S, "gate/up", n2, wgu, gu)
            gsel, fsel = S.idx(T), S.idx(F)
            gt, ft = torch.as_tensor(gsel, device=x.device), torch.as_tensor(fsel, device=x.device)
            gg, uu = f64(gu[gt, ft]), f64(gu[gt, ft + F])
            S.record("swiglu fwd", f64(sw[gt, ft]), od.swiglu(gg, uu), 5e-3)
            _nt_samples(S, "down + residual", sw, wd, out, R=h1)
            # ---- B ----
            ds_ref = od.gemm_nt_entries(f64(dout[gt]), f64(wd[:, ft]).T, range(64), range(64))
            dg_ref, du_ref = od.swiglu_bwd(gg, uu, ds_ref)
            S.record("swiglu bwd (dg)", f64(dgu[gt, ft]), dg_ref, 5e-3)
            S.record("swiglu bwd (du)", f64(dgu[gt, ft + F]), du_ref, 5e-3)
            _nn_samples(S, "gate/up bwd", dgu, wgu, dn2)
            h1r = f64(h1[rt])
            _, xh2, rr2 = od.rms_fwd(h1r, f64(g2), eps)
            S.record("rms2 bwd", f64(dh1[rt]), f64(dout[rt]) + od.rms_bwd_input(xh2, rr2, f64(g2), f64(dn2[rt])), 5e-3)
            rep = nq // nkv
            da = f64(dh1) @ f64(wo[:, :rep * d])  # heads 0..rep-1 of da, fp64 from the GPU's dh1
            dq_ref, dk_sum, dv_sum = None, 0.0, 0.0
            for hh in range(rep):  # head 0 and its KV group 0
                dqh, dkp, dvp = od.attn_head_bwd(qf, kf, vf, da, hh, nq, nkv, d)
                if hh == 0:
                    dq_ref = dqh
                dk_sum = dk_sum + dkp
                dv_sum = dv_sum + dvp
            S.record("attn bwd dq", f64(dqkv[:, :d]), dq_ref, 2e-2)
            S.record("attn bwd dk", f64(dqkv[:, QD:QD + d]), dk_sum, 2e-2)
            S.record("attn bwd dv", f64(dqkv[:, QD + KVD:QD + KVD + d]), dv_sum, 2e-2)
            _nn_samples(S, "qkv bwd", dqkv, wqkv, dn1)
            _, xh1, rr1 = od.rms_fwd(f64(x[rt]), f64(g1), eps)
            S.record("rms1 bwd", f64(dxl[rt]), f64(dh1[rt]) + od.rms_bwd_input(xh1, rr1, f64(g1), f64(dn1[rt])), 5e-3)
        # ---- W (over both microbatches) ----
        stl = lambda which: [st.stash(j, l, which) for j in range(m)]
        dw = st.dw[6 * l:6 * l + 6]
        _w_samples(S, "dWqkv", stl(zb.L_DQKV), stl(zb.L_N1), dw[0])
        _w_samples(S, "dWo", stl(zb.L_DH1), stl(zb.L_A), dw[1])
        _w_samples(S, "dWgu", stl(zb.L_DGU), stl(zb.L_N2), dw[2])
        _w_samples(S, "dWd", stl(zb.L_DOUT), stl(zb.L_S), dw[3])
        cols = S.idx(H)
        ct = torch.as_tensor(cols, device=dw[4].device)
        for gi, (xw, rw, dnw) in ((4, (zb.L_X, zb.L_R1, zb.L_DN1)), (5, (zb.L_H1, zb.L_R2, zb.L_DN2))):
            ref = np.zeros(len(cols))
            for j in range(m):
                xv = f64(st.stash(j, l, xw)[:, ct]) * f64(st.stash(j, l, rw))
                ref += np.sum(f64(st.stash(j, l, dnw)[:, ct]) * xv, axis=0)
            S.record(f"dgamma{gi - 3}", f64(dw[gi][ct]), ref, 5e-3)
    print({k: f"{v:.2e}" for k, v in S.err.items()})
