"""Pins for the fp64 dense oracle (CPU only).

Each oracle function is tied to something other than itself:
* brute-force Python loops on tiny inputs (products);
* central finite differences of a scalar loss (every backward);
* library routines that compute the same textbook function in fp64
  (torch gelu/silu/rms_norm/scaled_dot_product_attention and torch autograd);
* the B+W = fused and deferred = immediate invariants, bitwise in fp64
  ([Guide] "Convergence and Numerical Stability": splitting the backward
  performs the very same multiplications, so results are identical).
"""
import math

import numpy as np
import pytest
import torch

from oracle import dense as od

RNG = np.random.default_rng(12345)


def rnd(*shape, std=1.0):
    return RNG.standard_normal(shape) * std


# ------------------------------------------------------------------ linear --

def test_linear_forward_brute_force():
    x, w = rnd(3, 4), rnd(5, 4)
    y = od.linear_fwd(x, w)
    for t in range(3):
        for o in range(5):
            acc = 0.0
            for i in range(4):
                acc += x[t, i] * w[o, i]
            assert abs(y[t, o] - acc) < 1e-13


def test_linear_backward_finite_differences():
    """L = sum(Y . G): dL/dX must be B's output, dL/dW must be W's output."""
    x, w, g = rnd(3, 4), rnd(5, 4), rnd(3, 5)
    loss = lambda xx, ww: float(np.sum(od.linear_fwd(xx, ww) * g))
    dx = od.linear_bwd_input(g, w)
    dw = od.linear_bwd_weight(x, g)
    eps = 1e-6
    for arr, grad, f in ((x, dx, lambda a: loss(a, w)), (w, dw, lambda a: loss(x, a))):
        num = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            p, m = arr.copy(), arr.copy()
            p[idx] += eps
            m[idx] -= eps
            num[idx] = (f(p) - f(m)) / (2 * eps)
        assert od.rel_fro(grad, num) < 1e-6


def test_linear_shapes_transposes_distinguished():
    """Non-square tiny shapes: a transposed operand fails to broadcast."""
    x, w, g = rnd(2, 3), rnd(5, 3), rnd(2, 5)
    assert od.linear_fwd(x, w).shape == (2, 5)
    assert od.linear_bwd_input(g, w).shape == (2, 3)
    assert od.linear_bwd_weight(x, g).shape == (5, 3)


def test_accumulation_equals_one_big_gemm():
    """sum_j dY_j^T X_j == [dY_0;..]^T [X_0;..]  (fp64, rel <= 1e-13)."""
    xs = [rnd(7, 6) for _ in range(4)]
    dys = [rnd(7, 5) for _ in range(4)]
    acc = sum(od.linear_bwd_weight(x, d) for x, d in zip(xs, dys))
    big = od.linear_bwd_weight(np.concatenate(xs), np.concatenate(dys))
    assert od.rel_fro(acc, big) < 1e-13


# ------------------------------------------------------------- activations --

def test_gelu_tanh_matches_torch():
    a = np.linspace(-8, 8, 2001)
    ref = torch.nn.functional.gelu(torch.tensor(a), approximate="tanh").numpy()
    assert np.max(np.abs(od.gelu_tanh(a) - ref)) < 1e-14
    assert od.gelu_tanh(np.array([0.0]))[0] == 0.0


def test_gelu_tanh_grad_fd_and_autograd():
    a = np.linspace(-6, 6, 1001)
    eps = 1e-6
    num = (od.gelu_tanh(a + eps) - od.gelu_tanh(a - eps)) / (2 * eps)
    assert np.max(np.abs(od.gelu_tanh_grad(a) - num)) < 1e-8
    ta = torch.tensor(a, requires_grad=True)
    torch.nn.functional.gelu(ta, approximate="tanh").sum().backward()
    assert np.max(np.abs(od.gelu_tanh_grad(a) - ta.grad.numpy())) < 1e-13


def test_swiglu_matches_torch_and_fd():
    g, u, ds = rnd(5, 7), rnd(5, 7), rnd(5, 7)
    tg, tu = torch.tensor(g, requires_grad=True), torch.tensor(u, requires_grad=True)
    s = torch.nn.functional.silu(tg) * tu
    assert np.max(np.abs(od.swiglu(g, u) - s.detach().numpy())) < 1e-14
    (s * torch.tensor(ds)).sum().backward()
    dg, du = od.swiglu_bwd(g, u, ds)
    assert np.max(np.abs(dg - tg.grad.numpy())) < 1e-13
    assert np.max(np.abs(du - tu.grad.numpy())) < 1e-13
    z = np.linspace(-8, 8, 1001)
    eps = 1e-6
    num = ((z + eps) * od.sigmoid(z + eps) - (z - eps) * od.sigmoid(z - eps)) / (2 * eps)
    dg1, _ = od.swiglu_bwd(z, np.ones_like(z), np.ones_like(z))
    assert np.max(np.abs(dg1 - num)) < 1e-8


# ------------------------------------------------------------------ RMSNorm --

def test_rmsnorm_matches_torch():
    x, gam, dy = rnd(6, 8), rnd(8), rnd(6, 8)
    tx, tg = torch.tensor(x, requires_grad=True), torch.tensor(gam, requires_grad=True)
    ty = torch.nn.functional.rms_norm(tx, (8,), tg, 1e-5)
    y, xh, r = od.rms_fwd(x, gam, 1e-5)
    assert np.max(np.abs(y - ty.detach().numpy())) < 1e-13
    (ty * torch.tensor(dy)).sum().backward()
    assert np.max(np.abs(od.rms_bwd_input(xh, r, gam, dy) - tx.grad.numpy())) < 1e-12
    assert np.max(np.abs(od.rms_bwd_gamma(xh, dy) - tg.grad.numpy())) < 1e-12


def test_rmsnorm_special_case_constant_row():
    """A constant row c normalises to c / sqrt(c^2 + eps) exactly."""
    x = np.full((1, 8), 3.0)
    y, _, _ = od.rms_fwd(x, np.ones(8), 1e-5)
    assert np.allclose(y, 3.0 / math.sqrt(9.0 + 1e-5), rtol=0, atol=1e-15)


# ---------------------------------------------------------------- attention --

@pytest.mark.parametrize("nq,nkv", [(2, 1), (4, 2), (2, 2)])
def test_attention_matches_torch_sdpa(nq, nkv):
    T, d = 6, 4
    q, k, v, do = rnd(T, nq * d), rnd(T, nkv * d), rnd(T, nkv * d), rnd(T, nq * d)
    o, probs = od.attn_fwd(q, k, v, nq, nkv, d)
    tq = torch.tensor(q.reshape(T, nq, d).transpose(1, 0, 2)[None], requires_grad=True)
    tk = torch.tensor(k.reshape(T, nkv, d).transpose(1, 0, 2)[None], requires_grad=True)
    tv = torch.tensor(v.reshape(T, nkv, d).transpose(1, 0, 2)[None], requires_grad=True)
    to = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True,
                                                          enable_gqa=(nq != nkv))
    to_flat = to[0].detach().numpy().transpose(1, 0, 2).reshape(T, nq * d)
    assert np.max(np.abs(o - to_flat)) < 1e-13
    tdo = torch.tensor(do.reshape(T, nq, d).transpose(1, 0, 2)[None])
    (to * tdo).sum().backward()
    dq, dk, dv = od.attn_bwd(q, k, v, o, probs, do, nq, nkv, d)
    flat = lambda t, h: t.grad[0].numpy().transpose(1, 0, 2).reshape(T, h * d)
    assert np.max(np.abs(dq - flat(tq, nq))) < 1e-12
    assert np.max(np.abs(dk - flat(tk, nkv))) < 1e-12
    assert np.max(np.abs(dv - flat(tv, nkv))) < 1e-12


def test_attention_first_token_sees_only_itself():
    """Causal special case: output row 0 is exactly v row 0 of its group."""
    q, k, v = rnd(5, 8), rnd(5, 4), rnd(5, 4)
    o, _ = od.attn_fwd(q, k, v, 2, 1, 4)
    assert np.array_equal(o[0, :4], v[0]) and np.array_equal(o[0, 4:], v[0])


# ------------------------------------------------------------- full blocks --

def _fd_check(loss_fn, arrays, grads, eps=1e-6, tol=1e-6, max_entries=60):
    for arr, grad in zip(arrays, grads):
        idxs = list(np.ndindex(arr.shape))
        if len(idxs) > max_entries:
            sel = RNG.choice(len(idxs), max_entries, replace=False)
            idxs = [idxs[i] for i in sel]
        num, ana = [], []
        for idx in idxs:
            old = arr[idx]
            arr[idx] = old + eps
            lp = loss_fn()
            arr[idx] = old - eps
            lm = loss_fn()
            arr[idx] = old
            num.append((lp - lm) / (2 * eps))
            ana.append(grad[idx])
        assert od.rel_fro(np.array(ana), np.array(num)) < tol


def test_mlp_finite_differences():
    T, h, f = 4, 8, 12
    x, w1, w2, g = rnd(T, h), rnd(f, h, std=0.5), rnd(h, f, std=0.5), rnd(T, h)
    y, st = od.mlp_fwd(x, w1, w2)
    dx, bst = od.mlp_bwd_input(st, g, w1, w2)
    dw1, dw2 = od.mlp_bwd_weight(st, bst)
    loss = lambda: float(np.sum(od.mlp_fwd(x, w1, w2)[0] * g))
    _fd_check(loss, [x, w1, w2], [dx, dw1, dw2])


DIMS = od.LlamaDims(hidden=8, ffn=12, n_heads=2, n_kv_heads=1, head_dim=4)


def _llama_weights(n_layers, dims=DIMS, std=0.4):
    ws = []
    for _ in range(n_layers):
        ws += [rnd(dims.q_dim + 2 * dims.kv_dim, dims.hidden, std=std),
               rnd(dims.hidden, dims.q_dim, std=std),
               rnd(2 * dims.ffn, dims.hidden, std=std),
               rnd(dims.hidden, dims.ffn, std=std),
               1.0 + rnd(dims.hidden, std=0.2), 1.0 + rnd(dims.hidden, std=0.2)]
    return ws


def test_llama_two_layer_finite_differences():
    T, L = 4, 2
    ws = _llama_weights(L)
    x, g = rnd(T, DIMS.hidden), rnd(T, DIMS.hidden)
    st = od.Stage("llama", ws, DIMS, L)
    st.w = ws  # same array objects so FD perturbations reach the stage
    y = st.fwd(0, x)
    dx = st.bwd_input(0, g)
    st.bwd_weight(0)
    grads = st.grad

    def loss():
        s2 = od.Stage("llama", ws, DIMS, L)
        s2.w = ws
        return float(np.sum(s2.fwd(0, x) * g))

    _fd_check(loss, [x] + ws, [dx] + grads, tol=2e-6)


def _torch_llama_layer(x, w, dims):
    """Independent torch fp64 rendition of the decoder layer (autograd
    supplies every derivative)."""
    wqkv, wo, wgu, wd, g1, g2 = w
    T = x.shape[0]
    qd, kvd, d = dims.q_dim, dims.kv_dim, dims.head_dim
    n1 = torch.nn.functional.rms_norm(x, (dims.hidden,), g1, dims.eps)
    qkv = n1 @ wqkv.T
    q = qkv[:, :qd].reshape(T, dims.n_heads, d).transpose(0, 1)[None]
    k = qkv[:, qd:qd + kvd].reshape(T, dims.n_kv_heads, d).transpose(0, 1)[None]
    v = qkv[:, qd + kvd:].reshape(T, dims.n_kv_heads, d).transpose(0, 1)[None]
    a = torch.nn.functional.scaled_dot_product_attention(
        q, k, v, is_causal=True, enable_gqa=dims.n_heads != dims.n_kv_heads)
    a = a[0].transpose(0, 1).reshape(T, qd)
    h1 = x + a @ wo.T
    n2 = torch.nn.functional.rms_norm(h1, (dims.hidden,), g2, dims.eps)
    gu = n2 @ wgu.T
    s = torch.nn.functional.silu(gu[:, :dims.ffn]) * gu[:, dims.ffn:]
    return h1 + s @ wd.T


def test_llama_stage_matches_torch_autograd():
    dims = od.LlamaDims(hidden=16, ffn=24, n_heads=4, n_kv_heads=2, head_dim=4)
    T, L = 7, 2
    ws = _llama_weights(L, dims, std=0.2)
    x, g = rnd(T, dims.hidden), rnd(T, dims.hidden)
    st = od.Stage("llama", ws, dims, L)
    y = st.fwd(0, x)
    dx = st.bwd_input(0, g)
    st.bwd_weight(0)
    tws = [torch.tensor(w, requires_grad=True) for w in ws]
    tx = torch.tensor(x, requires_grad=True)
    h = tx
    for l in range(L):
        h = _torch_llama_layer(h, tws[6 * l:6 * l + 6], dims)
    assert np.max(np.abs(y - h.detach().numpy())) < 1e-12
    (h * torch.tensor(g)).sum().backward()
    assert od.rel_fro(dx, tx.grad.numpy()) < 1e-12
    for a, b in zip(st.grad, tws):
        assert od.rel_fro(a, b.grad.numpy()) < 1e-12


# -------------------------------------------------------------- invariants --

def _stage_inputs(kind):
    if kind == "linear":
        return [rnd(6, 5)], None, 1, (3, 5), (3, 6)
    if kind == "mlp":
        return [rnd(8, 4, std=0.5), rnd(4, 8, std=0.5)], None, 1, (3, 4), (3, 4)
    return _llama_weights(2), DIMS, 2, (4, 8), (4, 8)


@pytest.mark.parametrize("kind", ["linear", "mlp", "llama"])
def test_invariant_split_equals_fused_bitwise(kind):
    """I1: B followed by W gives exactly the fused backward (fp64, bitwise)."""
    ws, dims, L, xs, ys = _stage_inputs(kind)
    x, g = rnd(*xs), rnd(*ys)
    st = od.Stage(kind, ws, dims, L)
    st.fwd(0, x)
    dx = st.bwd_input(0, g)
    st.bwd_weight(0)
    fdx, fgr = od.stage_bwd_fused(kind, ws, x, g, dims, L)
    assert np.array_equal(dx, fdx)
    for a, b in zip(st.grad, fgr):
        assert np.array_equal(a, b)


@pytest.mark.parametrize("kind", ["linear", "mlp", "llama"])
def test_invariant_deferred_equals_immediate_bitwise(kind):
    """I2: F0 F1 B0 B1 W0 W1 == F0 B0 W0 F1 B1 W1 (same W order), bitwise."""
    ws, dims, L, xs, ys = _stage_inputs(kind)
    xs_ = [rnd(*xs) for _ in range(2)]
    gs = [rnd(*ys) for _ in range(2)]
    a = od.Stage(kind, ws, dims, L)
    b = od.Stage(kind, ws, dims, L)
    ya = [a.fwd(j, xs_[j]) for j in range(2)]
    da = [a.bwd_input(j, gs[j]) for j in range(2)]
    for j in range(2):
        a.bwd_weight(j)
    yb, db = [], []
    for j in range(2):
        yb.append(b.fwd(j, xs_[j]))
        db.append(b.bwd_input(j, gs[j]))
        b.bwd_weight(j)
    for u, v in zip(ya + da + a.grad, yb + db + b.grad):
        assert np.array_equal(u, v)


def test_stage_state_errors():
    """B needs F first; W needs B first (dict lookups of the listing)."""
    st = od.Stage("linear", [rnd(3, 2)])
    with pytest.raises(KeyError):
        st.bwd_input(0, rnd(1, 3))
    st.fwd(0, rnd(1, 2))
    with pytest.raises(KeyError):
        st.bwd_weight(0)


def test_flop_ratio_linear_one_to_one_to_one():
    """[Guide] "Core Innovation 1": F : B_X : B_W = 1 : 1 : 1 for a linear
    layer; each pass is one product of 2*T*in*out flops."""
    T, i, o = 3, 4, 5
    x, w, g = rnd(T, i), rnd(o, i), rnd(T, o)
    # count multiply-adds of each product by its operand shapes
    f = 2 * x.shape[0] * x.shape[1] * w.shape[0]
    b = 2 * g.shape[0] * g.shape[1] * w.shape[1]
    wflops = 2 * g.shape[1] * g.shape[0] * x.shape[1]
    assert f == b == wflops == 2 * T * i * o


@pytest.mark.parametrize("kind", ["linear", "mlp", "llama"])
def test_stage_accumulates_over_microbatches(kind):
    """[Guide] "Memory Management & Activation Rollback": W adds each
    microbatch's gradient into one fixed buffer.  The result must equal the
    sum of single-microbatch gradients (each pinned by FD above), and for the
    linear layer the single big product over all tokens."""
    ws, dims, L, xs, ys = _stage_inputs(kind)
    xs_ = [rnd(*xs) for _ in range(3)]
    gs = [rnd(*ys) for _ in range(3)]
    st = od.Stage(kind, ws, dims, L)
    for j in range(3):
        st.fwd(j, xs_[j])
        st.bwd_input(j, gs[j])
        st.bwd_weight(j)
    singles = []
    for j in range(3):
        s1 = od.Stage(kind, ws, dims, L)
        s1.fwd(0, xs_[j])
        s1.bwd_input(0, gs[j])
        s1.bwd_weight(0)
        singles.append(s1.grad)
    for i, g in enumerate(st.grad):
        assert od.rel_fro(g, sum(s[i] for s in singles)) < 1e-14
        assert od.rel_fro(g, singles[0][i]) > 1e-3
    if kind == "linear":
        big = od.linear_bwd_weight(np.concatenate(xs_), np.concatenate(gs))
        assert od.rel_fro(st.grad[0], big) < 1e-13


@pytest.mark.parametrize("nq,nkv", [(4, 2), (2, 2)])
def test_sampled_attention_helpers_match_torch(nq, nkv):
    """Row-wise forward and per-head backward (used for full-size sampled
    checks) against torch SDPA / autograd in fp64."""
    T, d = 9, 4
    q, k, v, do = rnd(T, nq * d), rnd(T, nkv * d), rnd(T, nkv * d), rnd(T, nq * d)
    tq = torch.tensor(q.reshape(T, nq, d).transpose(1, 0, 2)[None], requires_grad=True)
    tk = torch.tensor(k.reshape(T, nkv, d).transpose(1, 0, 2)[None], requires_grad=True)
    tv = torch.tensor(v.reshape(T, nkv, d).transpose(1, 0, 2)[None], requires_grad=True)
    to = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True, enable_gqa=nq != nkv)
    (to * torch.tensor(do.reshape(T, nq, d).transpose(1, 0, 2)[None])).sum().backward()
    for h in range(nq):
        rows = [0, 3, T - 1]
        o, _ = od.attn_rows_fwd(q, k, v, h, rows, nq, nkv, d)
        assert np.max(np.abs(o - to[0, h].detach().numpy()[rows])) < 1e-13
    dk_sum = np.zeros((T, nkv * d))
    dv_sum = np.zeros((T, nkv * d))
    for h in range(nq):
        dq, dkp, dvp = od.attn_head_bwd(q, k, v, do, h, nq, nkv, d)
        assert np.max(np.abs(dq - tq.grad[0, h].numpy())) < 1e-12
        g = (h * nkv) // nq
        dk_sum[:, g * d:(g + 1) * d] += dkp
        dv_sum[:, g * d:(g + 1) * d] += dvp
    assert np.max(np.abs(dk_sum - tk.grad[0].numpy().transpose(1, 0, 2).reshape(T, nkv * d))) < 1e-12
    assert np.max(np.abs(dv_sum - tv.grad[0].numpy().transpose(1, 0, 2).reshape(T, nkv * d))) < 1e-12


def test_gemm_entries_brute_force():
    a, b = rnd(5, 7), rnd(6, 7)
    rows, cols = [0, 4, 2], [5, 0, 3]
    got = od.gemm_nt_entries(a, b, rows, cols)
    for i, (r, c) in enumerate(zip(rows, cols)):
        assert abs(got[i] - sum(a[r, k] * b[c, k] for k in range(7))) < 1e-13


# ------------------------------------------------------- optimizer step ---

def test_bf16_round_matches_torch_conversion():
    """The oracle's round-to-nearest-even equals torch's float32 -> bfloat16
    conversion (a library routine) on random values and on constructed ties."""
    import torch
    rng = np.random.default_rng(3)
    x = (rng.standard_normal(100000) * np.exp(rng.uniform(-20, 20, 100000))).astype(np.float32)
    ties = (np.array([1.0, -1.0, 3.0, 0.5], np.float32).view(np.uint32)[:, None]
            + np.array([0x8000, 0x18000, 0x7FFF, 0x8001], np.uint32)[None, :]).ravel().view(np.float32)
    for v in (x, ties):
        ref = torch.from_numpy(v.copy()).to(torch.bfloat16).to(torch.float64).numpy()
        assert np.array_equal(od.bf16_round(v), ref)


def test_bf16_round_ties_to_even():
    assert od.bf16_round(np.array([1 + 2 ** -8], np.float32))[0] == 1.0             # halfway, even below
    assert od.bf16_round(np.array([1 + 3 * 2 ** -8], np.float32))[0] == 1 + 2 ** -6  # halfway, even above
    assert od.bf16_round(np.array([-(1 + 2 ** -8)], np.float32))[0] == -1.0
    assert od.bf16_round(np.array([1 + 2 ** -8 + 2 ** -20], np.float32))[0] == 1 + 2 ** -7


def test_sgd_step_special_cases():
    rng = np.random.default_rng(4)
    w = od.bf16_round(rng.standard_normal(4096).astype(np.float32))
    dw = rng.standard_normal(4096).astype(np.float32)
    assert np.array_equal(od.sgd_step(w, dw, 0.0, "bf16"), w)                    # lr = 0: unchanged
    assert od.sgd_step(np.array([1.0]), np.array([0.5]), 0.5, "bf16")[0] == 0.75  # exact
    assert od.sgd_step(np.array([1.0]), np.array([3.0]), 0.25, "f32")[0] == 0.25
    # the result is the exact value rounded twice: within half a bf16 unit of it
    exact = w - np.float64(np.float32(1e-2)) * dw.astype(np.float64)
    got = od.sgd_step(w, dw, 1e-2, "bf16")
    ulp = 2.0 ** (np.floor(np.log2(np.abs(exact))) - 7)
    assert np.all(np.abs(got - exact) <= 0.5 * ulp * (1 + 2 ** -15))
    # a step against the gradient lowers a quadratic loss sum(w^2)/2 (dW = w)
    ww = od.bf16_round(rng.standard_normal(4096).astype(np.float32))
    assert np.sum(od.sgd_step(ww, ww.astype(np.float32), 0.1, "bf16") ** 2) < np.sum(ww ** 2)


def test_sgd_step_rounds_the_product_to_float32_first():
    """A case built by hand where the stage's reading (float32 product, then
    float32 difference, then bf16) and an exact or fp64 formulation part:
    lr = 1 + 2^-12 and dW = 2^-9 (1 - 2^-12 + 2^-24), both float32 values,
    have the exact product 2^-9 + 2^-45, which float32 rounds to 2^-9.  Then
    w - t = 1 - 2^-9 exactly, a bf16 tie between 1 - 2^-8 (odd) and 1.0
    (even): 1.0.  Rounded once from the exact 1 - 2^-9 - 2^-45 it would be
    1 - 2^-8."""
    lr = 1.0 + 2.0 ** -12
    dw = np.array([2.0 ** -9 * (1.0 - 2.0 ** -12 + 2.0 ** -24)])
    assert float(np.float32(lr)) == lr and float(np.float32(dw[0])) == dw[0]
    assert od.sgd_step(np.array([1.0]), dw, lr, "bf16")[0] == 1.0
    exact = 1.0 - lr * dw[0]
    assert exact == 1.0 - 2.0 ** -9 - 2.0 ** -45
    # float32 cannot hold the exact difference (it rounds it to the tie), so
    # the single-rounding formulation is checked in float64 against the bf16
    # grid directly: the exact value lies below the midpoint 1 - 2^-9, so its
    # nearest bf16 is 1 - 2^-8
    lo, hi = 1.0 - 2.0 ** -8, 1.0
    assert abs(exact - lo) < abs(exact - hi)
    # the fp32 formulation's difference for the f32 dtype
    assert od.sgd_step(np.array([1.0]), dw, lr, "f32")[0] == 1.0 - 2.0 ** -9


def test_sgd_step_f32_rounds_the_product_exact_arithmetic():
    """fp32 stage, w = 1: near cancellation the product's float32 rounding
    error is far above the spacing of the difference, so the reading
    (product rounded to float32, then an exact difference) and a formulation
    that rounds only the difference give different float32 results.  The
    expected value is worked out in exact rational arithmetic:
    lr dW = 1 - 2^-12 + 2^-20 + 2^-21 - 2^-23 - 2^-31 + 2^-33 + 2^-41, whose
    float32 (spacing 2^-24 in [1/2, 1)) drops the last three terms."""
    from fractions import Fraction as Fr
    lr = 1.0 + 2.0 ** -12 + 2.0 ** -20
    dw = 1.0 - 2.0 ** -11 + 2.0 ** -21
    exact = Fr(lr) * Fr(dw)
    assert exact == 1 - Fr(2) ** -12 + Fr(2) ** -20 + Fr(2) ** -21 - Fr(2) ** -23 - Fr(2) ** -31 + Fr(2) ** -33 + Fr(2) ** -41
    t32 = Fr(round(exact / Fr(2) ** -24)) * Fr(2) ** -24
    assert t32 == 1 - Fr(2) ** -12 + Fr(2) ** -20 + Fr(2) ** -21 - Fr(2) ** -23
    want = 1 - t32  # exactly representable: the difference of two nearby float32 values
    got = od.sgd_step(np.array([1.0]), np.array([dw]), lr, "f32")[0]
    assert Fr(got) == want
    # rounding only the difference (from the exact product) lands elsewhere
    assert Fr(float(np.float32(float(1 - exact)))) != want
