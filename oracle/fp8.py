"""FP8 operands of the linear products, in fp64.  TEST INFRASTRUCTURE ONLY.

[Ghost] "Memory Pressure: The Hidden Cost of Efficiency" names FP8 as what
halves the memory of many buffers and makes room for a pipeline schedule's
extra stash.  The pages give no format, scaling or rounding, so the reading
here (the plainest one a gfx950 matrix core supports) is:

* format: 8-bit floating point E4M3 of the OCP 8-bit FP specification
  (sign, 4 exponent bits with bias 7, 3 mantissa bits; subnormals; largest
  finite value 448; no infinities; S.1111.111 is NaN);
* scaling: one power of two per tensor, 2^e with e the smallest integer
  such that max|x| <= 448 * 2^e (e = 0 for an all-zero tensor), so that
  x * 2^-e is exact and lies in [-448, 448];
* rounding: x * 2^-e rounded to the nearest E4M3 value, ties to the even
  code;
* a product C = A . B^T of two quantized operands is the fp64 product of
  their dequantized values; the GPU accumulates it in fp32.

Every linear product of the fp8 stage (F, B and W) takes both operands in
this form; RMSNorm, attention and the activation epilogues stay as in the
bf16 stage.
"""
from __future__ import annotations

import math

import numpy as np

from . import dense as od

E4M3_MAX = 448.0
_MAX_EXP = 8          # 448 = 1.75 * 2^8
_MIN_NORMAL_EXP = -6  # smallest normal 2^-6; subnormals are multiples of 2^-9


def e4m3_decode(codes) -> np.ndarray:
    """Exact values of E4M3 codes (uint8) as float64 (NaN for S.1111.111)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c >> 7, -1.0, 1.0)
    e = (c >> 3) & 15
    m = c & 7
    normal = np.ldexp(1.0 + m / 8.0, e - 7)
    sub = np.ldexp(m / 8.0, _MIN_NORMAL_EXP)
    v = sign * np.where(e == 0, sub, normal)
    return np.where((e == 15) & (m == 7), np.nan, v)


def e4m3_round(x) -> np.ndarray:
    """Nearest E4M3 code of each value (|x| <= 448), ties to the even code.

    The E4M3 values with exponent field E are spaced 2^(E-10) apart
    (E >= 1) and the subnormals 2^-9 apart, so x is divided by the spacing
    of its binade, rounded half-to-even to an integer (np.rint), and
    re-encoded; rounding up across a binade edge carries into the exponent
    naturally because the code is sign | (E << 3 | m) with consecutive codes
    consecutive in value.
    """
    x = np.asarray(x, dtype=np.float64)
    if np.any(~np.isfinite(x)) or np.any(np.abs(x) > E4M3_MAX):
        raise ValueError("e4m3_round: values must be finite with |x| <= 448")
    a = np.abs(x)
    # binade exponent of |x| (floor(log2)), clamped to the subnormal binade
    ex = np.where(a > 0, np.floor(np.log2(np.where(a > 0, a, 1.0))), _MIN_NORMAL_EXP)
    ex = np.maximum(ex, _MIN_NORMAL_EXP)
    # guard against log2 rounding at exact powers of two
    ex = np.where(np.ldexp(1.0, ex.astype(np.int64)) > a, ex - 1, ex)
    ex = np.where(np.ldexp(1.0, (ex + 1).astype(np.int64)) <= a, ex + 1, ex)
    ex = np.maximum(ex, _MIN_NORMAL_EXP)
    step = np.ldexp(1.0, (ex - 3).astype(np.int64))    # value spacing in this binade
    n = np.rint(a / step)                                # multiples of the spacing, ties to even
    # code magnitude: subnormal binade -> n directly (n = 0..8); normal ->
    # (E << 3) + (n - 8) with E = ex + 7
    mag = np.where(ex <= _MIN_NORMAL_EXP, n, ((ex + 7) * 8 + (n - 8)))
    mag = mag.astype(np.int64)
    assert np.all(mag <= 0x7E), "rounded past 448"
    return (np.where(np.signbit(x), 0x80, 0) | mag).astype(np.uint8)


def scale_exponent(amax: float) -> int:
    """Smallest integer e with amax <= 448 * 2^e (0 when amax == 0)."""
    amax = float(amax)
    if amax == 0.0:
        return 0
    if not math.isfinite(amax) or amax < 0:
        raise ValueError("amax must be finite and >= 0")
    e = math.ceil(math.log2(amax / E4M3_MAX))
    while amax > math.ldexp(E4M3_MAX, e):      # log2 rounding guards
        e += 1
    while amax <= math.ldexp(E4M3_MAX, e - 1):
        e -= 1
    return e


def quantize(x: np.ndarray):
    """Per-tensor E4M3 quantization: (codes uint8, exponent e), x ~ codes * 2^e."""
    x = np.asarray(x, dtype=np.float64)
    e = scale_exponent(np.max(np.abs(x)) if x.size else 0.0)
    return e4m3_round(np.ldexp(x, -e)), e


def dequantize(codes: np.ndarray, e: int) -> np.ndarray:
    return np.ldexp(e4m3_decode(codes), e)


def fake_quant(x: np.ndarray) -> np.ndarray:
    """x replaced by its per-tensor E4M3 value (quantize then dequantize)."""
    q, e = quantize(x)
    return dequantize(q, e)


def product_nt(qa: np.ndarray, ea: int, qb: np.ndarray, eb: int) -> np.ndarray:
    """C = A . B^T from quantized operands A [M, K], B [N, K], in fp64."""
    return dequantize(qa, ea) @ dequantize(qb, eb).T


# ======================================================== fp8 Llama stage ===
# The decoder layer of oracle.dense with every linear product taking both of
# its operands through fake_quant (per-tensor scaling of the whole operand
# tensor, as the GPU quantizes it): F's activation and weight, B's output
# gradient and weight, W's output gradient and activation.

def llama_layer_fwd_fp8(x, wts, dm: od.LlamaDims):
    wqkv, wo, wgu, wd, g1, g2 = wts
    fq = fake_quant
    qd, kvd = dm.q_dim, dm.kv_dim
    n1, xh1, r1 = od.rms_fwd(x, g1, dm.eps)
    qkv = fq(n1) @ fq(wqkv).T
    q, k, v = qkv[:, :qd], qkv[:, qd:qd + kvd], qkv[:, qd + kvd:]
    a, probs = od.attn_fwd(q, k, v, dm.n_heads, dm.n_kv_heads, dm.head_dim)
    h1 = x + fq(a) @ fq(wo).T
    n2, xh2, r2 = od.rms_fwd(h1, g2, dm.eps)
    gu = fq(n2) @ fq(wgu).T
    g, u = gu[:, :dm.ffn], gu[:, dm.ffn:]
    s = od.swiglu(g, u)
    out = h1 + fq(s) @ fq(wd).T
    st = dict(x=x, n1=n1, xh1=xh1, r1=r1, q=q, k=k, v=v, a=a, probs=probs, h1=h1,
              n2=n2, xh2=xh2, r2=r2, g=g, u=u, s=s)
    return out, st


def llama_layer_bwd_input_fp8(st, dout, wts, dm: od.LlamaDims):
    wqkv, wo, wgu, wd, g1, g2 = wts
    fq = fake_quant
    ds = fq(dout) @ fq(wd)
    dg, du = od.swiglu_bwd(st["g"], st["u"], ds)
    dgu = np.concatenate([dg, du], axis=1)
    dn2 = fq(dgu) @ fq(wgu)
    dh1 = dout + od.rms_bwd_input(st["xh2"], st["r2"], g2, dn2)
    da = fq(dh1) @ fq(wo)
    dq, dk, dv = od.attn_bwd(st["q"], st["k"], st["v"], st["a"], st["probs"], da,
                             dm.n_heads, dm.n_kv_heads, dm.head_dim)
    dqkv = np.concatenate([dq, dk, dv], axis=1)
    dn1 = fq(dqkv) @ fq(wqkv)
    dx = dh1 + od.rms_bwd_input(st["xh1"], st["r1"], g1, dn1)
    return dx, dict(dout=dout, dgu=dgu, dn2=dn2, dh1=dh1, dqkv=dqkv, dn1=dn1)


def llama_layer_bwd_weight_fp8(st, bst):
    fq = fake_quant
    return [
        fq(bst["dqkv"]).T @ fq(st["n1"]),
        fq(bst["dh1"]).T @ fq(st["a"]),
        fq(bst["dgu"]).T @ fq(st["n2"]),
        fq(bst["dout"]).T @ fq(st["s"]),
        od.rms_bwd_gamma(st["xh1"], bst["dn1"]),
        od.rms_bwd_gamma(st["xh2"], bst["dn2"]),
    ]


class Fp8LlamaStage(od.Stage):
    """oracle.dense.Stage of kind "llama" with fp8 linear products."""

    def __init__(self, weights, dims: od.LlamaDims, n_layers: int):
        super().__init__("llama", weights, dims, n_layers)

    def fwd(self, mb, x):
        sts, h = [], x
        for l in range(self.n_layers):
            h, st = llama_layer_fwd_fp8(h, self._layer_w(l), self.dims)
            sts.append(st)
        self.saved_f[mb] = sts
        return h

    def bwd_input(self, mb, dy):
        if mb not in self.saved_f or mb in self.saved_b:
            raise KeyError(f"B({mb}) out of order")
        bsts = [None] * self.n_layers
        d = dy
        for l in reversed(range(self.n_layers)):
            d, bsts[l] = llama_layer_bwd_input_fp8(self.saved_f[mb][l], d, self._layer_w(l), self.dims)
        self.saved_b[mb] = bsts
        return d

    def bwd_weight(self, mb):
        st = self.saved_f.pop(mb)
        bst = self.saved_b.pop(mb)
        gs = []
        for l in range(self.n_layers):
            gs += llama_layer_bwd_weight_fp8(st[l], bst[l])
        for i, g in enumerate(gs):
            self.grad[i] = g if self.grad[i] is None else self.grad[i] + g
