"""Sampled oracle checks of a Llama stage at full size (GPU tests' helper).

At the benchmark sizes the fp64 oracle cannot run a whole stage, so each
step of F, B and W is checked on sampled outputs that the oracle recomputes
in fp64 from the GPU's own stashed inputs of that step: a wrong tile,
epilogue, index or stale operand anywhere shows up in the step that
produced it.

Every sampled set of rows and columns includes the first and last index and
the indices on each side of the 128- and 256-wide tile boundaries, beside
random ones.  Each check applies two bars: the relative Frobenius error over
the samples, and per element |got - ref| <= tol * (|ref| + 5 * rms(ref)),
so a few wrong entries cannot hide in a good norm.
"""
from __future__ import annotations

import numpy as np
import torch

import split_backward_amd as zb
from oracle import dense as od


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


class Lazy:
    """A device tensor read as fp64 one slice at a time (t[idx] converts only
    what is indexed), for oracle routines that select a head's columns."""

    def __init__(self, t: torch.Tensor):
        self.t = t
        self.shape = tuple(t.shape)

    def __getitem__(self, idx):
        return f64(self.t[idx])


def edge_indices(n: int):
    """First and last index and both sides of the 128/256 tile edges."""
    cand = [0, n - 1]
    for b in (128, 256):
        for e in (b, 2 * b, (n // b) * b):
            cand += [e - 1, e]
    return sorted({c for c in cand if 0 <= c < n})


class Sampler:
    def __init__(self, seed):
        self.rng = np.random.default_rng(seed)
        self.err = {}

    def idx(self, n, k=64):
        """k indices in [0, n): the edge indices first, then random ones."""
        e = edge_indices(n)[:k]
        return np.concatenate([np.asarray(e, dtype=np.int64), self.rng.integers(0, n, size=k - len(e))])

    def record(self, key, got, ref, tol):
        got = np.asarray(got, np.float64)
        ref = np.asarray(ref, np.float64)
        e = od.rel_fro(got, ref)
        self.err[key] = max(self.err.get(key, 0.0), e)
        assert e <= tol, (key, e)
        rms = float(np.sqrt(np.mean(ref * ref))) if ref.size else 0.0
        bad = np.abs(got - ref) > tol * (np.abs(ref) + 5.0 * rms)
        assert not bad.any(), (key, "element bound", int(bad.sum()), np.argwhere(bad)[:4].tolist())


def nt_samples(S: Sampler, key, A, B, C, tol=5e-3, R=None):
    """C[r, c] (+ R[r, c]) == A[r] . B[c] on sampled entries."""
    rows = S.idx(A.shape[0])
    cols = S.idx(B.shape[0])
    rt = torch.as_tensor(rows, device=A.device)
    ct = torch.as_tensor(cols, device=A.device)
    ref = od.gemm_nt_entries(f64(A[rt]), f64(B[ct]), range(len(rows)), range(len(cols)))
    if R is not None:
        ref = ref + f64(R[rt, ct])
    S.record(key, f64(C[rt, ct]), ref, tol)


def nn_samples(S: Sampler, key, A, W, C, tol=5e-3):
    """C[r, c] == sum_k A[r, k] W[k, c]  (W stored [K, N])."""
    rows = S.idx(A.shape[0])
    cols = S.idx(W.shape[1])
    rt = torch.as_tensor(rows, device=A.device)
    ct = torch.as_tensor(cols, device=A.device)
    ref = od.gemm_nt_entries(f64(A[rt]), f64(W[:, ct]).T, range(len(rows)), range(len(cols)))
    S.record(key, f64(C[rt, ct]), ref, tol)


def check_microbatch_layer(S: Sampler, st, shape, j: int, l: int, out, dxl, x_in=None, dy_in=None,
                           attn_bwd=True):
    """Every F and B step of decoder layer l of microbatch j, from the
    stage's stash of j (which must still be resident): RMSNorms, the QKV,
    output, gate/up and down products with their epilogues, attention rows,
    and (attn_bwd) a whole head's attention backward.  `out` is the layer's
    output (the stage output y_j for the last layer), `dxl` its input
    gradient (the stage's dx_j for layer 0); x_in / dy_in, when given, are
    the caller's inputs the stash must hold exact copies of."""
    T, H, F = shape.tokens, shape.hidden, shape.ffn
    nq, nkv, d = shape.n_heads, shape.n_kv_heads, shape.head_dim
    QD, KVD = nq * d, nkv * d
    eps = shape.rms_eps
    wqkv, wo, wgu, wd, g1, g2 = st.weights[6 * l:6 * l + 6]
    T_ = lambda which: st.stash(j, l, which)
    x, qkv, a = T_(zb.L_X), T_(zb.L_QKV), T_(zb.L_A)
    n1, h1, n2, gu, sw = T_(zb.L_N1), T_(zb.L_H1), T_(zb.L_N2), T_(zb.L_GU), T_(zb.L_S)
    dout, dgu, dn2, dh1, dqkv, dn1 = (T_(zb.L_DOUT), T_(zb.L_DGU), T_(zb.L_DN2), T_(zb.L_DH1), T_(zb.L_DQKV),
                                      T_(zb.L_DN1))
    if x_in is not None:
        S.record("x copy", f64(x[:4]), f64(x_in[:4]), 0.0)
        S.record("x copy (last rows)", f64(x[-4:]), f64(x_in[-4:]), 0.0)
    if dy_in is not None:
        S.record("dy copy", f64(dout[:4]), f64(dy_in[:4]), 0.0)
        S.record("dy copy (last rows)", f64(dout[-4:]), f64(dy_in[-4:]), 0.0)
    rows = S.idx(T, 16)
    rt = torch.as_tensor(rows, device=x.device)
    # ---- F ----
    nref, _, _ = od.rms_fwd(f64(x[rt]), f64(g1), eps)
    S.record("rms1", f64(n1[rt]), nref, 5e-3)
    nt_samples(S, "qkv", n1, wqkv, qkv)
    qf, kf, vf = Lazy(qkv[:, :QD]), Lazy(qkv[:, QD:QD + KVD]), Lazy(qkv[:, QD + KVD:])
    for h in (0, nq - 1):
        arows = np.concatenate([[0, 1, 127, 128, T - 1], S.idx(T, 8)[-3:]])
        o_ref, _ = od.attn_rows_fwd(qf, kf, vf, h, arows, nq, nkv, d)
        S.record("attn fwd", f64(a[torch.as_tensor(arows, device=a.device), h * d:(h + 1) * d]), o_ref, 1e-2)
    nt_samples(S, "o proj + residual", a, wo, h1, R=x)
    nref, _, _ = od.rms_fwd(f64(h1[rt]), f64(g2), eps)
    S.record("rms2", f64(n2[rt]), nref, 5e-3)
    nt_samples(S, "gate/up", n2, wgu, gu)
    gsel, fsel = S.idx(T), S.idx(F)
    gt, ft = torch.as_tensor(gsel, device=x.device), torch.as_tensor(fsel, device=x.device)
    gg, uu = f64(gu[gt, ft]), f64(gu[gt, ft + F])
    S.record("swiglu fwd", f64(sw[gt, ft]), od.swiglu(gg, uu), 5e-3)
    nt_samples(S, "down + residual", sw, wd, out, R=h1)
    # ---- B ----
    ds_ref = od.gemm_nt_entries(f64(dout[gt]), f64(wd[:, ft]).T, range(len(gsel)), range(len(fsel)))
    dg_ref, du_ref = od.swiglu_bwd(gg, uu, ds_ref)
    S.record("swiglu bwd (dg)", f64(dgu[gt, ft]), dg_ref, 5e-3)
    S.record("swiglu bwd (du)", f64(dgu[gt, ft + F]), du_ref, 5e-3)
    nn_samples(S, "gate/up bwd", dgu, wgu, dn2)
    _, xh2, rr2 = od.rms_fwd(f64(h1[rt]), f64(g2), eps)
    S.record("rms2 bwd", f64(dh1[rt]), f64(dout[rt]) + od.rms_bwd_input(xh2, rr2, f64(g2), f64(dn2[rt])), 5e-3)
    if attn_bwd:
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
    nn_samples(S, "qkv bwd", dqkv, wqkv, dn1)
    _, xh1, rr1 = od.rms_fwd(f64(x[rt]), f64(g1), eps)
    S.record("rms1 bwd", f64(dxl[rt]), f64(dh1[rt]) + od.rms_bwd_input(xh1, rr1, f64(g1), f64(dn1[rt])), 5e-3)


# The weight-gradient products of a decoder layer: (dW index within the
# layer's six, output-gradient stash, input stash).
W_PRODUCTS = ((0, zb.L_DQKV, zb.L_N1), (1, zb.L_DH1, zb.L_A), (2, zb.L_DGU, zb.L_N2), (3, zb.L_DOUT, zb.L_S))
GAMMAS = ((4, zb.L_X, zb.L_R1, zb.L_DN1), (5, zb.L_H1, zb.L_R2, zb.L_DN2))


class WeightGradAccumulator:
    """fp64 sums over microbatches of the sampled entries of every dW and
    dgamma of a Llama stage: dW[o, i] = sum_j sum_t dY_j[t, o] X_j[t, i] and
    dgamma[c] = sum_j sum_t dn_j[t, c] x_j[t, c] r_j[t], taken from each
    microbatch's stash while it is resident (add(j)), then compared with the
    GPU's accumulated buffers (check)."""

    def __init__(self, S: Sampler, st, shape):
        self.S, self.st, self.shape = S, st, shape
        self.sel, self.ref = {}, {}
        for l in range(shape.n_layers):
            for wi, _, _ in W_PRODUCTS:
                M, N = st.dw[6 * l + wi].shape
                self.sel[(l, wi)] = (S.idx(M), S.idx(N))
                self.ref[(l, wi)] = np.zeros(len(self.sel[(l, wi)][0]))
            for gi, _, _, _ in GAMMAS:
                self.sel[(l, gi)] = S.idx(shape.hidden)
                self.ref[(l, gi)] = np.zeros(len(self.sel[(l, gi)]))
        self.seen = []

    def add(self, j: int):
        st = self.st
        for l in range(self.shape.n_layers):
            for wi, dyw, xw in W_PRODUCTS:
                o, i = self.sel[(l, wi)]
                dY, X = st.stash(j, l, dyw), st.stash(j, l, xw)
                ot, it = torch.as_tensor(o, device=dY.device), torch.as_tensor(i, device=dY.device)
                self.ref[(l, wi)] += np.sum(f64(dY[:, ot]) * f64(X[:, it]), axis=0)
            for gi, xw, rw, dnw in GAMMAS:
                c = self.sel[(l, gi)]
                ct = torch.as_tensor(c, device=st.dw[0].device)
                xv = f64(st.stash(j, l, xw)[:, ct]) * f64(st.stash(j, l, rw))
                self.ref[(l, gi)] += np.sum(f64(st.stash(j, l, dnw)[:, ct]) * xv, axis=0)
        self.seen.append(j)

    def check(self, dws, tol=5e-3):
        """dws: the GPU's dW / dgamma tensors (the stage's order)."""
        for (l, wi), ref in self.ref.items():
            dw = dws[6 * l + wi]
            if wi < 4:
                o, i = self.sel[(l, wi)]
                got = f64(dw[torch.as_tensor(o, device=dw.device), torch.as_tensor(i, device=dw.device)])
                key = ("dWqkv", "dWo", "dWgu", "dWd")[wi]
            else:
                got = f64(dw[torch.as_tensor(self.sel[(l, wi)], device=dw.device)])
                key = f"dgamma{wi - 3}"
            self.S.record(key, got, ref, tol)
