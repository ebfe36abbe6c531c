"""fp64 oracle for the stage's forward (F), input-gradient (B) and
weight-gradient (W) passes.  TEST INFRASTRUCTURE ONLY (see package header).

Conventions
-----------
[Guide] "Core Innovation 1" writes the layer as Y = X.W with W[in, out], so
dX = dY.W^T and dW = X^T.dY.  Its PyTorch stage listing ("Step-by-Step
Implementation") stores the weight as [out, in] and computes y = x.weight^T,
dx = dy.weight, grad_weight = dy^T.x.  The two are the same mathematics with
W_eq = weight^T.  This oracle, like the GPU path, stores weights [out, in]
(the listing's convention), so every formula below is the listing's form.

All arrays are float64 and nothing is rounded between steps.  A library
matmul (numpy) serves as the product step; there is no blocking or fusion.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Dict, List, Optional

import numpy as np

GELU_C = math.sqrt(2.0 / math.pi)
GELU_K = 0.044715


# =============================================================== linear ====
# [Guide] "Core Innovation 1: Mathematical Decomposition of the Backward
# Pass" (equations for the input gradient and the weight gradient) and the
# listing's forward_microbatch / backward_input_bx / backward_weight_bw.

def linear_fwd(x: np.ndarray, w: np.ndarray) -> np.ndarray:
    """Y = X . W^T  (w is [out, in])."""
    return x @ w.T


def linear_bwd_input(dy: np.ndarray, w: np.ndarray) -> np.ndarray:
    """B_X: dX = dY . W  (critical path: sent to the previous stage)."""
    return dy @ w


def linear_bwd_weight(x: np.ndarray, dy: np.ndarray) -> np.ndarray:
    """B_W: dW = dY^T . X  (local; deferrable until the optimizer step)."""
    return dy.T @ x


# ========================================================== activations ====

def gelu_tanh(a: np.ndarray) -> np.ndarray:
    """GeLU, tanh form (Hendrycks & Gimpel): 0.5 a (1 + tanh(c (a + k a^3)))."""
    return 0.5 * a * (1.0 + np.tanh(GELU_C * (a + GELU_K * a ** 3)))


def gelu_tanh_grad(a: np.ndarray) -> np.ndarray:
    """d gelu_tanh / da = 0.5 (1 + t) + 0.5 a (1 - t^2) c (1 + 3 k a^2)."""
    t = np.tanh(GELU_C * (a + GELU_K * a ** 3))
    return 0.5 * (1.0 + t) + 0.5 * a * (1.0 - t * t) * GELU_C * (1.0 + 3.0 * GELU_K * a * a)


def sigmoid(z: np.ndarray) -> np.ndarray:
    return 1.0 / (1.0 + np.exp(-z))


def swiglu(g: np.ndarray, u: np.ndarray) -> np.ndarray:
    """s = silu(g) * u with silu(g) = g . sigmoid(g)."""
    return g * sigmoid(g) * u


def swiglu_bwd(g: np.ndarray, u: np.ndarray, ds: np.ndarray):
    """dg = ds . u . sig(g)(1 + g(1 - sig(g))),  du = ds . g . sig(g)."""
    sg = sigmoid(g)
    dg = ds * u * sg * (1.0 + g * (1.0 - sg))
    du = ds * g * sg
    return dg, du


# ============================================================== RMSNorm ====

def rms_fwd(x: np.ndarray, gamma: np.ndarray, eps: float):
    """y = x . r . gamma with r = (mean(x^2) + eps)^(-1/2) per row.
    Returns (y, xhat, r) where xhat = x . r."""
    r = 1.0 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    xhat = x * r
    return xhat * gamma, xhat, r


def rms_bwd_input(xhat: np.ndarray, r: np.ndarray, gamma: np.ndarray, dy: np.ndarray) -> np.ndarray:
    """dx = r (dxhat - xhat . mean(dxhat . xhat)), dxhat = dy . gamma."""
    dxh = dy * gamma
    return r * (dxh - xhat * np.mean(dxh * xhat, axis=-1, keepdims=True))


def rms_bwd_gamma(xhat: np.ndarray, dy: np.ndarray) -> np.ndarray:
    """dgamma = sum over tokens of dy . xhat (a weight gradient)."""
    return np.sum(dy * xhat, axis=0)


# ============================================================ attention ====
# Causal multi-head attention with grouped KV heads: query head h reads KV
# head floor(h * n_kv / n_q) (contiguous groups).  Scale 1/sqrt(head_dim),
# no rotary embedding, no dropout.  q, k, v are [T, heads * d].

def _kv_of(h: int, n_q: int, n_kv: int) -> int:
    return (h * n_kv) // n_q


def attn_fwd(q, k, v, n_q: int, n_kv: int, d: int):
    """Returns (o [T, n_q d], P list per head) with P = softmax(S) and
    S = q k^T / sqrt(d) masked to key index <= query index."""
    T = q.shape[0]
    scale = 1.0 / math.sqrt(d)
    mask = np.tril(np.ones((T, T), dtype=bool))
    o = np.zeros((T, n_q * d))
    probs = []
    for h in range(n_q):
        g = _kv_of(h, n_q, n_kv)
        qh = q[:, h * d:(h + 1) * d]
        kh = k[:, g * d:(g + 1) * d]
        vh = v[:, g * d:(g + 1) * d]
        s = (qh @ kh.T) * scale
        s = np.where(mask, s, -np.inf)
        s = s - np.max(s, axis=1, keepdims=True)
        e = np.exp(s)
        p = e / np.sum(e, axis=1, keepdims=True)
        o[:, h * d:(h + 1) * d] = p @ vh
        probs.append(p)
    return o, probs


def attn_bwd(q, k, v, o, probs, do, n_q: int, n_kv: int, d: int):
    """Gradients of the causal attention w.r.t. q, k, v.

    dP = dO v^T;  dS = P . (dP - rowsum(dO . O));  dq = dS k / sqrt(d);
    dk = dS^T q / sqrt(d);  dv = P^T dO  (dk, dv summed over the query
    heads of each KV group)."""
    scale = 1.0 / math.sqrt(d)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for h in range(n_q):
        g = _kv_of(h, n_q, n_kv)
        sl = slice(h * d, (h + 1) * d)
        gl = slice(g * d, (g + 1) * d)
        p = probs[h]
        doh = do[:, sl]
        dp = doh @ v[:, gl].T
        delta = np.sum(doh * o[:, sl], axis=1, keepdims=True)
        ds = p * (dp - delta)
        dq[:, sl] = (ds @ k[:, gl]) * scale
        dk[:, gl] += (ds.T @ q[:, sl]) * scale
        dv[:, gl] += p.T @ doh
    return dq, dk, dv


# =========================================================== GPT MLP =======
# fc1 -> GeLU(tanh) -> fc2, no bias, no norm, no residual.

def mlp_fwd(x, w1, w2):
    a = linear_fwd(x, w1)
    hact = gelu_tanh(a)
    y = linear_fwd(hact, w2)
    return y, {"x": x, "a": a, "h": hact}


def mlp_bwd_input(st, dy, w1, w2):
    """B: dH = dY W2, dA = dH . gelu'(A), dX = dA W1.  Returns (dx, bstash)."""
    dh = linear_bwd_input(dy, w2)
    da = dh * gelu_tanh_grad(st["a"])
    dx = linear_bwd_input(da, w1)
    return dx, {"dy": dy, "da": da}


def mlp_bwd_weight(st, bst):
    """W: dW2 = dY^T H,  dW1 = dA^T X."""
    return [linear_bwd_weight(st["x"], bst["da"]), linear_bwd_weight(st["h"], bst["dy"])]


def mlp_bwd_fused(x, dy, w1, w2):
    """One-piece backward of the MLP (B and W together, layer by layer in
    reverse), written out on its own for the B+W invariant."""
    a = x @ w1.T
    t = np.tanh(GELU_C * (a + GELU_K * a ** 3))
    hact = 0.5 * a * (1.0 + t)
    dw2 = dy.T @ hact
    dh = dy @ w2
    da = dh * (0.5 * (1.0 + t) + 0.5 * a * (1.0 - t * t) * GELU_C * (1.0 + 3.0 * GELU_K * a * a))
    dw1 = da.T @ x
    dx = da @ w1
    return dx, [dw1, dw2]


# ====================================================== Llama decoder ======

@dataclass
class LlamaDims:
    hidden: int
    ffn: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    eps: float = 1e-5

    @property
    def q_dim(self):
        return self.n_heads * self.head_dim

    @property
    def kv_dim(self):
        return self.n_kv_heads * self.head_dim


def llama_layer_fwd(x, wts, dm: LlamaDims):
    """Pre-norm decoder layer.  wts = (wqkv, wo, wgu, wd, g1, g2).

    n1 = RMS(x; g1);  [q|k|v] = n1 Wqkv^T;  a = Attn(q,k,v);  h1 = x + a Wo^T;
    n2 = RMS(h1; g2);  [g|u] = n2 Wgu^T;  s = silu(g) u;  out = h1 + s Wd^T.
    """
    wqkv, wo, wgu, wd, g1, g2 = wts
    qd, kvd = dm.q_dim, dm.kv_dim
    n1, xh1, r1 = rms_fwd(x, g1, dm.eps)
    qkv = linear_fwd(n1, wqkv)
    q, k, v = qkv[:, :qd], qkv[:, qd:qd + kvd], qkv[:, qd + kvd:]
    a, probs = attn_fwd(q, k, v, dm.n_heads, dm.n_kv_heads, dm.head_dim)
    h1 = x + linear_fwd(a, wo)
    n2, xh2, r2 = rms_fwd(h1, g2, dm.eps)
    gu = linear_fwd(n2, wgu)
    g, u = gu[:, :dm.ffn], gu[:, dm.ffn:]
    s = swiglu(g, u)
    out = h1 + linear_fwd(s, wd)
    st = dict(x=x, n1=n1, xh1=xh1, r1=r1, q=q, k=k, v=v, a=a, probs=probs, h1=h1,
              n2=n2, xh2=xh2, r2=r2, g=g, u=u, s=s)
    return out, st


def llama_layer_bwd_input(st, dout, wts, dm: LlamaDims):
    """B pass of one layer; returns (dx, bstash).  The attention backward
    has no weights and sits wholly in B."""
    wqkv, wo, wgu, wd, g1, g2 = wts
    ds = linear_bwd_input(dout, wd)
    dg, du = swiglu_bwd(st["g"], st["u"], ds)
    dgu = np.concatenate([dg, du], axis=1)
    dn2 = linear_bwd_input(dgu, wgu)
    dh1 = dout + rms_bwd_input(st["xh2"], st["r2"], g2, dn2)
    da = linear_bwd_input(dh1, wo)
    dq, dk, dv = attn_bwd(st["q"], st["k"], st["v"], st["a"], st["probs"], da,
                          dm.n_heads, dm.n_kv_heads, dm.head_dim)
    dqkv = np.concatenate([dq, dk, dv], axis=1)
    dn1 = linear_bwd_input(dqkv, wqkv)
    dx = dh1 + rms_bwd_input(st["xh1"], st["r1"], g1, dn1)
    return dx, dict(dout=dout, dgu=dgu, dn2=dn2, dh1=dh1, dqkv=dqkv, dn1=dn1)


def llama_layer_bwd_weight(st, bst):
    """W pass of one layer, in the weight order (wqkv, wo, wgu, wd, g1, g2)."""
    return [
        linear_bwd_weight(st["n1"], bst["dqkv"]),
        linear_bwd_weight(st["a"], bst["dh1"]),
        linear_bwd_weight(st["n2"], bst["dgu"]),
        linear_bwd_weight(st["s"], bst["dout"]),
        rms_bwd_gamma(st["xh1"], bst["dn1"]),
        rms_bwd_gamma(st["xh2"], bst["dn2"]),
    ]


def llama_layer_bwd_fused(x, dout, wts, dm: LlamaDims):
    """One-piece backward of a decoder layer (recomputes its own forward),
    interleaving input and weight gradients the way an autograd engine
    would.  Written separately from the split routines for the B+W
    invariant."""
    wqkv, wo, wgu, wd, g1, g2 = wts
    out, st = llama_layer_fwd(x, wts, dm)
    dwd = dout.T @ st["s"]
    ds = dout @ wd
    sg = 1.0 / (1.0 + np.exp(-st["g"]))
    dg = ds * st["u"] * sg * (1.0 + st["g"] * (1.0 - sg))
    du = ds * st["g"] * sg
    dgu = np.concatenate([dg, du], axis=1)
    dwgu = dgu.T @ st["n2"]
    dn2 = dgu @ wgu
    dgam2 = np.sum(dn2 * st["xh2"], axis=0)
    dxh = dn2 * g2
    dh1 = dout + st["r2"] * (dxh - st["xh2"] * np.mean(dxh * st["xh2"], axis=-1, keepdims=True))
    dwo = dh1.T @ st["a"]
    da = dh1 @ wo
    dq, dk, dv = attn_bwd(st["q"], st["k"], st["v"], st["a"], st["probs"], da,
                          dm.n_heads, dm.n_kv_heads, dm.head_dim)
    dqkv = np.concatenate([dq, dk, dv], axis=1)
    dwqkv = dqkv.T @ st["n1"]
    dn1 = dqkv @ wqkv
    dgam1 = np.sum(dn1 * st["xh1"], axis=0)
    dxh = dn1 * g1
    dx = dh1 + st["r1"] * (dxh - st["xh1"] * np.mean(dxh * st["xh1"], axis=-1, keepdims=True))
    return dx, [dwqkv, dwo, dwgu, dwd, dgam1, dgam2]


# ======================================================= stage object ======
# [Guide] "Step-by-Step Implementation" listing: F stashes its input, B
# stashes the output gradient and returns the input gradient, W pops both
# stashes and adds the weight gradient into a fixed buffer (the first W
# assigns, later ones add; [Guide] "Memory Management & Activation Rollback",
# in-place weight-gradient accumulation).

class Stage:
    """Host fp64 stage of ``kind`` in {"linear", "mlp", "llama"}.

    weights: list of float64 arrays in the stage's documented weight order.
    """

    def __init__(self, kind: str, weights: List[np.ndarray], dims: Optional[LlamaDims] = None,
                 n_layers: int = 1):
        self.kind = kind
        self.w = [np.asarray(t, np.float64) for t in weights]
        self.dims = dims
        self.n_layers = n_layers
        self.saved_f: Dict[int, object] = {}
        self.saved_b: Dict[int, object] = {}
        self.grad: List[Optional[np.ndarray]] = [None] * len(self.w)

    def _layer_w(self, l):
        return self.w[6 * l:6 * l + 6]

    def fwd(self, mb: int, x: np.ndarray) -> np.ndarray:
        if self.kind == "linear":
            self.saved_f[mb] = x
            return linear_fwd(x, self.w[0])
        if self.kind == "mlp":
            y, st = mlp_fwd(x, self.w[0], self.w[1])
            self.saved_f[mb] = st
            return y
        sts = []
        h = x
        for l in range(self.n_layers):
            h, st = llama_layer_fwd(h, self._layer_w(l), self.dims)
            sts.append(st)
        self.saved_f[mb] = sts
        return h

    def bwd_input(self, mb: int, dy: np.ndarray) -> np.ndarray:
        if mb not in self.saved_f or mb in self.saved_b:
            raise KeyError(f"B({mb}) out of order")
        if self.kind == "linear":
            self.saved_b[mb] = dy
            return linear_bwd_input(dy, self.w[0])
        if self.kind == "mlp":
            dx, bst = mlp_bwd_input(self.saved_f[mb], dy, self.w[0], self.w[1])
            self.saved_b[mb] = bst
            return dx
        bsts = [None] * self.n_layers
        d = dy
        for l in reversed(range(self.n_layers)):
            d, bsts[l] = llama_layer_bwd_input(self.saved_f[mb][l], d, self._layer_w(l), self.dims)
        self.saved_b[mb] = bsts
        return d

    def bwd_weight(self, mb: int) -> None:
        st = self.saved_f.pop(mb)
        bst = self.saved_b.pop(mb)
        if self.kind == "linear":
            gs = [linear_bwd_weight(st, bst)]
        elif self.kind == "mlp":
            gs = mlp_bwd_weight(st, bst)
        else:
            gs = []
            for l in range(self.n_layers):
                gs += llama_layer_bwd_weight(st[l], bst[l])
        for i, g in enumerate(gs):
            if self.grad[i] is None:
                self.grad[i] = g
            else:
                self.grad[i] = self.grad[i] + g


def stage_bwd_fused(kind: str, weights, x, dy, dims: Optional[LlamaDims] = None, n_layers: int = 1):
    """Fused (atomic) backward of a whole stage for one microbatch: returns
    (dx, [dW...]) computed layer by layer in reverse in one routine."""
    w = [np.asarray(t, np.float64) for t in weights]
    if kind == "linear":
        return dy @ w[0], [dy.T @ x]
    if kind == "mlp":
        return mlp_bwd_fused(x, dy, w[0], w[1])
    xs = [x]
    for l in range(n_layers):
        xs.append(llama_layer_fwd(xs[-1], w[6 * l:6 * l + 6], dims)[0])
    grads = [None] * (6 * n_layers)
    d = dy
    for l in reversed(range(n_layers)):
        d, gl = llama_layer_bwd_fused(xs[l], d, w[6 * l:6 * l + 6], dims)
        grads[6 * l:6 * l + 6] = gl
    return d, grads


# =================================================== sampled entries =======

def gemm_nt_entries(a: np.ndarray, b: np.ndarray, rows, cols) -> np.ndarray:
    """Entries C[r, c] of C = A . B^T computed one by one in fp64
    (A [M, K], B [N, K]); used to check full-size products on samples."""
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return np.array([float(np.dot(a[r], b[c])) for r, c in zip(rows, cols)])


def rel_fro(got: np.ndarray, ref: np.ndarray) -> float:
    """Relative Frobenius error ||got - ref||_F / ||ref||_F in fp64."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.linalg.norm(ref.ravel())
    num = np.linalg.norm((got - ref).ravel())
    if den == 0.0:
        return 0.0 if num == 0.0 else float("inf")
    return float(num / den)


# ====================================================== sampled attention ===
# Single rows / columns of the causal attention at full sequence length,
# each from its plain definition in fp64 (the same formulas as attn_fwd /
# attn_bwd, restricted to what one output entry depends on).

def attn_rows_fwd(q, k, v, h: int, rows, n_q: int, n_kv: int, d: int):
    """Output rows o[t, head h] and their log-sum-exp for query rows `rows`."""
    g = _kv_of(h, n_q, n_kv)
    scale = 1.0 / math.sqrt(d)
    kh = np.asarray(k[:, g * d:(g + 1) * d], np.float64)
    vh = np.asarray(v[:, g * d:(g + 1) * d], np.float64)
    out, lse = [], []
    for t in rows:
        s = (kh[:t + 1] @ np.asarray(q[t, h * d:(h + 1) * d], np.float64)) * scale
        mx = np.max(s)
        e = np.exp(s - mx)
        out.append((e / e.sum()) @ vh[:t + 1])
        lse.append(mx + math.log(e.sum()))
    return np.array(out), np.array(lse)


def attn_head_bwd(q, k, v, do, h: int, n_q: int, n_kv: int, d: int):
    """Full backward of one query head (all rows): (dq_h, dk_part, dv_part)
    where dk_part / dv_part are this head's contributions to its KV group."""
    g = _kv_of(h, n_q, n_kv)
    qh = np.asarray(q[:, h * d:(h + 1) * d], np.float64)
    kh = np.asarray(k[:, g * d:(g + 1) * d], np.float64)
    vh = np.asarray(v[:, g * d:(g + 1) * d], np.float64)
    doh = np.asarray(do[:, h * d:(h + 1) * d], np.float64)
    T = qh.shape[0]
    scale = 1.0 / math.sqrt(d)
    s = (qh @ kh.T) * scale
    s = np.where(np.tril(np.ones((T, T), dtype=bool)), s, -np.inf)
    s = s - np.max(s, axis=1, keepdims=True)
    p = np.exp(s)
    p /= p.sum(axis=1, keepdims=True)
    o = p @ vh
    dp = doh @ vh.T
    ds = p * (dp - np.sum(doh * o, axis=1, keepdims=True))
    return (ds @ kh) * scale, (ds.T @ qh) * scale, p.T @ doh


# ====================================================== optimizer step ====
# The pages name an optimizer step after each iteration's weight gradients
# ([Guide] listing: the weight gradient accumulates into weight.grad, which
# an optimizer then consumes; [Abstract]: the optimizer step) but no
# optimizer.  The stage applies plain SGD, w <- w - lr * dW, and its result
# is a rounded value, so here the step is written at the precision the
# stage defines for it: the product lr * dW and the difference are float32
# operations (one rounding each), then the weight is rounded once to its
# storage type.  Unlike the rest of this module this is not fp64: the
# result is a bf16 / fp32 bit pattern that is compared exactly.

def bf16_round(x: np.ndarray) -> np.ndarray:
    """float32 values -> nearest bfloat16 values (ties to even), as float64.
    Finite inputs only."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    keep = u >> 16                       # sign, exponent and top 7 mantissa bits
    rest = u & 0xFFFF                    # the 16 bits rounded away
    up = (rest > 0x8000) | ((rest == 0x8000) & ((keep & 1) == 1))
    r = ((keep + up.astype(np.uint64)) << 16).astype(np.uint32)
    return r.view(np.float32).astype(np.float64)


def sgd_step(w: np.ndarray, dw: np.ndarray, lr: float, dtype: str) -> np.ndarray:
    """w - lr * dW as the stage computes it: float32 product, float32
    difference, then one rounding to dtype ("bf16" or "f32")."""
    w32 = np.asarray(w, dtype=np.float64).astype(np.float32)  # exact: w is bf16 or fp32
    t = np.float32(lr) * np.asarray(dw, dtype=np.float32)
    r = (w32 - t).astype(np.float32)
    return bf16_round(r) if dtype == "bf16" else r.astype(np.float64)
