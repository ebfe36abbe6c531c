"""The loop-nest fp64 oracle of a linear layer's F, B and W products
(oracle/loopnest.c) against what fixes them independently of its code
(CPU):

* brute-force Python loops over the defining sums on tiny inputs;
* numpy's matrix product at a moderate, ragged shape (a library routine);
* the adjoint identities that tie the three products together, so that a
  transposed operand or a wrong index in any one of them fails:
  <dY, F(X)> = <B(dY), X> = <W(dY, X), W>  ("Zero-Bubble Pipeline
  Parallelism Guide for LLMs", "Core Innovation 1": B and W are the two
  halves of one backward);
* deferred accumulation: W over two microbatches into one dW equals the
  sum of the two separate weight gradients (the Guide's deferred W);
* agreement with the numpy oracle's linear functions (oracle/dense.py).
"""
import numpy as np
import pytest

from oracle import dense as od
from oracle import loopnest as ln


def _rng(seed=0):
    return np.random.default_rng(seed)


def test_tiny_shapes_equal_brute_force_sums():
    r = _rng(1)
    T, n_in, n_out = 3, 5, 4
    X, W, dY = r.standard_normal((T, n_in)), r.standard_normal((n_out, n_in)), r.standard_normal((T, n_out))
    dW0 = r.standard_normal((n_out, n_in))
    Y = np.zeros((T, n_out))
    dX = np.zeros((T, n_in))
    dW = dW0.copy()
    for t in range(T):
        for o in range(n_out):
            s = 0.0
            for i in range(n_in):
                s += X[t, i] * W[o, i]
            Y[t, o] = s
    for t in range(T):
        for i in range(n_in):
            s = 0.0
            for o in range(n_out):
                s += dY[t, o] * W[o, i]
            dX[t, i] = s
    for o in range(n_out):
        for i in range(n_in):
            s = dW[o, i]
            for t in range(T):
                s += dY[t, o] * X[t, i]
            dW[o, i] = s
    got_dw = dW0.copy()
    ln.linear_bwd_weight(dY, X, got_dw)
    for got, ref in ((ln.linear_fwd(X, W), Y), (ln.linear_bwd_input(dY, W), dX), (got_dw, dW)):
        assert np.allclose(got, ref, rtol=1e-14, atol=1e-14)


@pytest.mark.parametrize("T,n_in,n_out", [(37, 29, 53), (64, 128, 96)])
def test_against_numpy_products(T, n_in, n_out):
    r = _rng(2)
    X, W, dY = r.standard_normal((T, n_in)), r.standard_normal((n_out, n_in)), r.standard_normal((T, n_out))
    assert od.rel_fro(ln.linear_fwd(X, W), X @ W.T) < 1e-13
    assert od.rel_fro(ln.linear_bwd_input(dY, W), dY @ W) < 1e-13
    dW = np.zeros((n_out, n_in))
    assert od.rel_fro(ln.linear_bwd_weight(dY, X, dW), dY.T @ X) < 1e-13


def test_adjoint_identities():
    r = _rng(3)
    T, n_in, n_out = 41, 33, 27
    X, W, dY = r.standard_normal((T, n_in)), r.standard_normal((n_out, n_in)), r.standard_normal((T, n_out))
    a = float(np.sum(dY * ln.linear_fwd(X, W)))
    b = float(np.sum(ln.linear_bwd_input(dY, W) * X))
    c = float(np.sum(ln.linear_bwd_weight(dY, X, np.zeros((n_out, n_in))) * W))
    scale = float(np.sum(np.abs(dY) * np.abs(X @ W.T)))
    assert abs(a - b) <= 1e-12 * scale and abs(a - c) <= 1e-12 * scale


def test_deferred_accumulation_over_two_microbatches():
    r = _rng(4)
    T, n_in, n_out = 16, 24, 20
    X = [r.standard_normal((T, n_in)) for _ in range(2)]
    dY = [r.standard_normal((T, n_out)) for _ in range(2)]
    dW = np.zeros((n_out, n_in))
    for j in range(2):
        ln.linear_bwd_weight(dY[j], X[j], dW)
    ref = dY[0].T @ X[0] + dY[1].T @ X[1]
    assert od.rel_fro(dW, ref) < 1e-13


def test_agrees_with_numpy_oracle():
    r = _rng(5)
    T, n_in, n_out = 48, 40, 56
    X, W, dY = r.standard_normal((T, n_in)), r.standard_normal((n_out, n_in)), r.standard_normal((T, n_out))
    assert od.rel_fro(ln.linear_fwd(X, W), od.linear_fwd(X, W)) < 1e-13
    assert od.rel_fro(ln.linear_bwd_input(dY, W), od.linear_bwd_input(dY, W)) < 1e-13
    assert od.rel_fro(ln.linear_bwd_weight(dY, X, np.zeros((n_out, n_in))), od.linear_bwd_weight(X, dY)) < 1e-13


def test_threads_reported():
    assert ln.threads() >= 1
