"""The fp8 stage (ZB_FP8) on the GPU against oracle.fp8, through the C ABI.

Bars (fixed with the oracle, before the kernels):
* quantization: codes and exponent bit for bit equal to the oracle's
  quantization of the GPU's own bf16 input;
* each fp8 product: relative Frobenius error <= 5e-3, and the element bound
  |got - ref| <= 5e-3 (|ref| + 5 rms(ref)), against the oracle's fp64 product
  of the GPU's own codes and exponents (bf16 output rounding 2^-9 plus the
  fp8 MFMA's in-block sum);
* the whole stage: <= 0.25 of oracle.fp8.Fp8LlamaStage and of the exact
  dense oracle (the E4M3 bound pinned on the oracle itself).  The GPU
  quantizes bf16-rounded tensors, the oracle its fp64 ones, so the two take
  neighbouring codes wherever a value lies between them and an E4M3
  midpoint.  Once two tensors differ by a relative d, their codes differ by
  about sqrt(d * s), s the E4M3 step (about 9%): 2^-9 of bf16 rounding
  becomes about 1.3% after the first quantization, and after a few
  quantized products the two fp8 computations differ by the quantization
  noise itself, as much as either differs from the exact stage (measured:
  0.4-4% at h 256, 6-8% at the Llama-7B widths).  So the whole-stage
  comparison can only bound the fp8 error; the exact checks are the
  per-step ones on the GPU's own codes (bit for bit, 5e-3).
"""
import numpy as np
import pytest
import torch

import split_backward_amd as zb
import synth
from oracle import dense as od
from oracle import fp8 as o8
from tests.gpu_helpers import to_dev, to_f64
from tests.stage_checks import Sampler

pytestmark = pytest.mark.gpu


def _bf16(rng, shape, std):
    t = torch.from_numpy(rng.standard_normal(shape) * std).to(torch.bfloat16)
    return t, t.to(torch.float64).numpy()


def _u8(t):
    return t.cpu().numpy().astype(np.uint8)


@pytest.mark.parametrize("shape,std", [((64, 64), 1.0), ((80, 48), 1e-2), ((256, 1024), 3.0), ((4096, 16), 1e-5),
                                       ((128, 4096), 0.02)])
def test_quantize_matches_oracle_bitwise(shape, std):
    rng = np.random.default_rng(sum(shape))
    x, x64 = _bf16(rng, shape, std)
    x[3, 5] = 7.0 * std  # a clear maximum, and exact ties at the tensor's scale
    x64[3, 5] = 7.0 * std
    x64 = x.to(torch.float64).numpy()
    xd = x.cuda()
    rows, cols = shape
    q = torch.empty((rows, cols), dtype=torch.uint8, device="cuda")
    qt = torch.empty((cols, rows), dtype=torch.uint8, device="cuda")
    _, _, e = zb.quantize_e4m3(xd, q, qt)
    torch.cuda.synchronize()
    codes, e_ref = o8.quantize(x64)
    assert int(e.item()) == e_ref
    assert np.array_equal(_u8(q), codes)
    assert np.array_equal(_u8(qt), codes.T)


def test_quantize_zero_and_single_outputs():
    x = torch.zeros((32, 48), dtype=torch.bfloat16, device="cuda")
    q = torch.full((32, 48), 7, dtype=torch.uint8, device="cuda")
    _, _, e = zb.quantize_e4m3(x, q, None)
    torch.cuda.synchronize()
    assert int(e.item()) == 0 and not q.any()
    rng = np.random.default_rng(1)
    x2, x64 = _bf16(rng, (48, 32), 1.0)
    qt = torch.empty((32, 48), dtype=torch.uint8, device="cuda")
    zb.quantize_e4m3(x2.cuda(), None, qt)
    torch.cuda.synchronize()
    assert np.array_equal(_u8(qt), o8.quantize(x64)[0].T)


def _codes(rng, shape):
    c = rng.integers(0, 256, size=shape, dtype=np.uint8)
    c[(c & 0x7F) == 0x7F] = 0x3C  # no NaN codes
    return c


@pytest.mark.parametrize("M,N,K,out_f32", [(300, 200, 256, 0), (512, 256, 1024, 0), (64, 96, 128, 1),
                                           (1000, 520, 384, 1), (256, 256, 4096, 0)])
def test_gemm_fp8_matches_oracle(M, N, K, out_f32):
    rng = np.random.default_rng(M + N + K)
    a, b = _codes(rng, (M, K)), _codes(rng, (N, K))
    ea, eb = -7, -9
    ref = o8.product_nt(a, ea, b, eb)
    A, B = torch.from_numpy(a).cuda(), torch.from_numpy(b).cuda()
    EA = torch.tensor([ea], dtype=torch.int32, device="cuda")
    EB = torch.tensor([eb], dtype=torch.int32, device="cuda")
    if out_f32:
        c0 = rng.standard_normal((M, N)).astype(np.float32)
        C = torch.from_numpy(c0).cuda()
        ref = ref + c0
    else:
        C = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    zb.gemm_fp8(A, EA, B, EB, C)
    torch.cuda.synchronize()
    S = Sampler(0)
    S.record("fp8 product", to_f64(C), ref, 5e-3)


SMALL = synth.StageShape("llama", 256, 256, 384, n_layers=2, n_heads=2, n_kv_heads=1, head_dim=128)


def _run_fp8(shape, m, ring=None):
    weights = synth.make_weights(shape)
    st = zb.Stage("llama", shape.tokens, shape.hidden, shape.ffn, [to_dev(w) for w in weights], dtype="fp8",
                  n_layers=shape.n_layers, n_heads=shape.n_heads, n_kv_heads=shape.n_kv_heads,
                  head_dim=shape.head_dim, ring_slots=ring or m)
    xs = [synth.make_x(shape, j) for j in range(m)]
    dys = [synth.make_dy(shape, j) for j in range(m)]
    xd = [to_dev(t) for t in xs]
    dyd = [to_dev(t) for t in dys]
    st.zero_grad()
    ys = [st.fwd(j, xd[j]) for j in range(m)]
    dxs = [st.bwd_input(j, dyd[j]) for j in range(m)]
    torch.cuda.synchronize()
    return st, weights, xs, dys, xd, dyd, ys, dxs


def _oracle(cls, shape, weights, xs, dys):
    dims = od.LlamaDims(shape.hidden, shape.ffn, shape.n_heads, shape.n_kv_heads, shape.head_dim, shape.rms_eps)
    w = [t.f64 for t in weights]
    ref = o8.Fp8LlamaStage(w, dims, shape.n_layers) if cls == "fp8" else od.Stage("llama", w, dims, shape.n_layers)
    m = len(xs)
    oy = [ref.fwd(j, xs[j].f64) for j in range(m)]
    odx = [ref.bwd_input(j, dys[j].f64) for j in range(m)]
    for j in range(m):
        ref.bwd_weight(j)
    return oy, odx, ref.grad


@pytest.mark.parametrize("shape", [SMALL, synth.StageShape("llama", 256, 512, 768, n_layers=1, n_heads=4,
                                                           n_kv_heads=4, head_dim=128)])
def test_fp8_stage_against_oracles(shape):
    m = 2
    st, weights, xs, dys, *_ , ys, dxs = _run_fp8(shape, m)
    for j in range(m):
        st.bwd_weight(j)
    torch.cuda.synchronize()
    got = [to_f64(y) for y in ys] + [to_f64(d) for d in dxs] + [to_f64(d) for d in st.dw]
    worst = {}
    for cls, tol in (("fp8", 0.25), ("dense", 0.25)):
        oy, odx, og = _oracle(cls, shape, weights, xs, dys)
        errs = [od.rel_fro(a, b) for a, b in zip(got, oy + odx + og)]
        worst[cls] = max(errs)
        assert max(errs) <= tol, (cls, errs)
    print(worst)


# 384 tokens: 128-token attention blocks (4-wave kernels), no split of the
# dk/dv work; the small stage's grouped heads take the split and its
# reduction kernel, so both kernels that store dk, dv leave maxima here.
S384 = synth.StageShape("llama", 384, 256, 384, n_layers=1, n_heads=2, n_kv_heads=2, head_dim=128)


@pytest.mark.parametrize("shape", [SMALL, S384], ids=["small", "t384"])
def test_fp8_stage_products_from_its_own_codes(shape):
    """Every fp8 product of the small stage against the oracle's product of
    the codes and exponents the GPU stashed (transposed codes of n1, a, n2,
    s, dout, dgu, dh1, dqkv; E4M3 weight copies), and the weight copies
    against the oracle's quantization of the bf16 weights."""
    m = 2
    st, weights, xs, dys, xd, dyd, ys, dxs = _run_fp8(shape, m)
    T, H, F = shape.tokens, shape.hidden, shape.ffn
    S = Sampler(1)
    W = {}
    for i in range(6 * shape.n_layers):
        if i % 6 >= 4:
            continue
        q, qt, e = st.fp8_weight(i)
        codes, e_ref = o8.quantize(weights[i].f64)
        assert int(e.item()) == e_ref and np.array_equal(_u8(q), codes) and np.array_equal(_u8(qt), codes.T)
        W[i] = (codes, e_ref)
    L = shape.n_layers
    for j in range(m):
        for l in range(L):
            T_ = lambda which: st.stash(j, l, which)
            ex = T_(zb.L_QEXP).cpu().numpy().ravel()
            codes = {k: _u8(T_(k)).T for k in (zb.L_N1T, zb.L_AT, zb.L_N2T, zb.L_ST, zb.L_DOUTT, zb.L_DGUT,
                                               zb.L_DH1T, zb.L_DQKVT)}
            e_of = dict(zip((zb.L_N1T, zb.L_AT, zb.L_N2T, zb.L_ST, zb.L_DOUTT, zb.L_DGUT, zb.L_DH1T, zb.L_DQKVT),
                            ex.tolist()))
            # Each exponent is the smallest with max|x| <= 448 * 2^e, so
            # max|x| 2^-e lies in (224, 448] and the largest code, its E4M3
            # rounding, in [224, 448]: an exponent one too large leaves it at
            # most 224, one too small saturates.  This holds whichever kernel
            # found the maximum (a pass over the tensor, or the partial
            # maxima its producer left).
            for k, c in codes.items():
                top = float(np.max(np.abs(o8.e4m3_decode(c))))
                assert 224.0 <= top <= 448.0, (j, l, k, e_of[k], top)
            prod = lambda k, wi, tr=False: o8.product_nt(codes[k], e_of[k], W[wi][0].T if tr else W[wi][0], W[wi][1])
            w0 = 6 * l
            x = to_f64(T_(zb.L_X))
            S.record("qkv", to_f64(T_(zb.L_QKV)), prod(zb.L_N1T, w0), 5e-3)
            h1 = to_f64(T_(zb.L_H1))
            S.record("o + residual", h1, x + prod(zb.L_AT, w0 + 1), 5e-3)
            gu = to_f64(T_(zb.L_GU))
            S.record("gate/up", gu, prod(zb.L_N2T, w0 + 2), 5e-3)
            out = to_f64(ys[j]) if l == L - 1 else to_f64(st.stash(j, l + 1, zb.L_X))
            S.record("down + residual", out, h1 + prod(zb.L_ST, w0 + 3), 5e-3)
            # s codes hold silu(g) u of the GPU's own [g | u]
            s_ref = od.swiglu(gu[:, :F], gu[:, F:])
            S.record("s codes", o8.dequantize(codes[zb.L_ST], e_of[zb.L_ST]), s_ref, 2.0 ** -4)
            # B: dg|du from the dout codes through Wd, against the dgu codes
            ds = prod(zb.L_DOUTT, w0 + 3, tr=True)
            dg, du = od.swiglu_bwd(gu[:, :F], gu[:, F:], ds)
            S.record("dgu codes", o8.dequantize(codes[zb.L_DGUT], e_of[zb.L_DGUT]), np.concatenate([dg, du], 1),
                     2.0 ** -4 + 5e-3)
            S.record("gate/up bwd", to_f64(T_(zb.L_DN2)), prod(zb.L_DGUT, w0 + 2, tr=True), 5e-3)
            # the attention outputs' codes against what they encode (their
            # exponents come from the attention kernels' partial maxima: one
            # that missed the wave holding the maximum would leave the
            # exponent too small, and the largest values saturated): a against
            # the stashed bf16 a, dq|dk|dv against the oracle's attention
            # backward of the stashed q, k, v with da = q(dh1) q(Wo)
            S.record("a codes", o8.dequantize(codes[zb.L_AT], e_of[zb.L_AT]), to_f64(T_(zb.L_A)), 2.0 ** -4)
            nq, nkv, hd = shape.n_heads, shape.n_kv_heads, shape.head_dim
            qkv = to_f64(T_(zb.L_QKV))
            QD, KVD = nq * hd, nkv * hd
            q_, k_, v_ = qkv[:, :QD], qkv[:, QD:QD + KVD], qkv[:, QD + KVD:]
            da = prod(zb.L_DH1T, w0 + 1, tr=True)
            dqkv = np.zeros_like(qkv)
            for h in range(nq):
                g = h // (nq // nkv)
                dqh, dkp, dvp = od.attn_head_bwd(q_, k_, v_, da, h, nq, nkv, hd)
                dqkv[:, h * hd:(h + 1) * hd] = dqh
                dqkv[:, QD + g * hd:QD + (g + 1) * hd] += dkp
                dqkv[:, QD + KVD + g * hd:QD + KVD + (g + 1) * hd] += dvp
            S.record("dqkv codes", o8.dequantize(codes[zb.L_DQKVT], e_of[zb.L_DQKVT]), dqkv, 2.0 ** -4 + 2e-2)
            S.record("qkv bwd", to_f64(T_(zb.L_DN1)), prod(zb.L_DQKVT, w0, tr=True), 5e-3)
            if l == L - 1:
                S.record("dout codes", o8.dequantize(codes[zb.L_DOUTT], e_of[zb.L_DOUTT]), to_f64(dyd[j]), 2.0 ** -4)
    # W over both microbatches from the stashed codes
    ref = {}
    for j in range(2):
        for l in range(L):
            T_ = lambda which: st.stash(j, l, which)
            ex = T_(zb.L_QEXP).cpu().numpy().ravel()
            e_of = dict(zip((zb.L_N1T, zb.L_AT, zb.L_N2T, zb.L_ST, zb.L_DOUTT, zb.L_DGUT, zb.L_DH1T, zb.L_DQKVT),
                            ex.tolist()))
            for wi, (dyk, xk) in enumerate(((zb.L_DQKVT, zb.L_N1T), (zb.L_DH1T, zb.L_AT), (zb.L_DGUT, zb.L_N2T),
                                            (zb.L_DOUTT, zb.L_ST))):
                p = o8.product_nt(_u8(T_(dyk)), e_of[dyk], _u8(T_(xk)), e_of[xk])
                ref[6 * l + wi] = ref.get(6 * l + wi, 0.0) + p
    st.bwd_weight(0)
    st.bwd_weight(1)
    torch.cuda.synchronize()
    for i, r in ref.items():
        S.record(f"dW{i}", to_f64(st.dw[i]), r, 5e-3)
    print({k: f"{v:.2e}" for k, v in S.err.items()})


def test_fp8_weights_requantized_after_an_optimizer_step():
    shape = SMALL
    st, weights, xs, dys, xd, dyd, ys, dxs = _run_fp8(shape, 1)
    st.bwd_weight(0)
    st.sgd_step(0.5)
    st.fwd(0, xd[0])
    torch.cuda.synchronize()
    q, qt, e = st.fp8_weight(0)
    codes, e_ref = o8.quantize(to_f64(st.weights[0]))
    assert int(e.item()) == e_ref and np.array_equal(_u8(q), codes) and np.array_equal(_u8(qt), codes.T)
    assert not np.array_equal(codes, o8.quantize(weights[0].f64)[0])


def test_fp8_stash_is_smaller_than_bf16():
    """The fp8 ring slot holds the W-only operands as 1-byte codes."""
    s7 = synth.WORKLOADS["llama7b_stage4"]["shape"]
    import ctypes
    L = zb.lib()
    sizes = {}
    for dt in (zb.BF16, zb.FP8):
        d1 = zb.StageDesc(zb.LLAMA, dt, 4, s7.tokens, s7.hidden, s7.ffn, 32, 32, 128, 1e-5, 1)
        d2 = zb.StageDesc(zb.LLAMA, dt, 4, s7.tokens, s7.hidden, s7.ffn, 32, 32, 128, 1e-5, 2)
        sizes[dt] = L.zb_stage_workspace_bytes(ctypes.byref(d2)) - L.zb_stage_workspace_bytes(ctypes.byref(d1))
    assert sizes[zb.FP8] < 0.8 * sizes[zb.BF16], sizes


@pytest.mark.timeout(900)
def test_fp8_stage_at_llama7b_widths_reduced_tokens():
    """Full Llama-7B widths (h 4096, ffn 11008, 32 heads), one layer, 256
    tokens: the whole fp8 stage against both oracles."""
    s = synth.WORKLOADS["llama7b_stage4"]["shape"]
    shape = synth.StageShape("llama", 256, s.hidden, s.ffn, n_layers=1, n_heads=s.n_heads, n_kv_heads=s.n_kv_heads,
                             head_dim=s.head_dim)
    st, weights, xs, dys, *_, ys, dxs = _run_fp8(shape, 1)
    st.bwd_weight(0)
    torch.cuda.synchronize()
    got = [to_f64(ys[0]), to_f64(dxs[0])] + [to_f64(d) for d in st.dw]
    for cls, tol in (("fp8", 0.25), ("dense", 0.25)):
        oy, odx, og = _oracle(cls, shape, weights, xs, dys)
        errs = [od.rel_fro(a, b) for a, b in zip(got, oy + odx + og)]
        print(cls, [f"{e:.3f}" for e in errs])
        assert max(errs) <= tol, (cls, errs)


def _codes_rows(t_T, idx):
    """Rows idx of the codes whose transposed copy [features][tokens] is t_T."""
    it = torch.as_tensor(idx, device=t_T.device)
    return _u8(t_T[:, it]).T


@pytest.mark.timeout(900)
def test_fp8_benchmark_configuration_sampled():
    """The Llama-7B-shape stage exactly as the fp8 benchmark line runs it
    (4 layers, 4096 tokens), two microbatches: every fp8 product of F, B and
    W on sampled outputs (edge and random rows and columns) against the
    oracle's product of the GPU's own stashed codes and exponents, and the
    weight copies against the oracle's quantization of sampled rows."""
    shape = synth.WORKLOADS["llama7b_stage4"]["shape"]
    m = 2
    st, weights, xs, dys, xd, dyd, ys, dxs = _run_fp8(shape, m)
    T, H, F = shape.tokens, shape.hidden, shape.ffn
    S = Sampler(3)
    L = shape.n_layers
    W8 = {}
    for i in range(6 * L):
        if i % 6 >= 4:
            continue
        q, qt, e = st.fp8_weight(i)
        e = int(e.item())
        wf = weights[i].f64
        rows = S.idx(wf.shape[0], 16)
        e_ref = o8.scale_exponent(np.max(np.abs(wf)))  # the whole weight decides the exponent
        codes = o8.e4m3_round(np.ldexp(wf[rows], -e_ref))
        assert e == e_ref
        assert np.array_equal(_u8(q[torch.as_tensor(rows, device=q.device)]), codes)
        assert np.array_equal(_u8(qt[:, torch.as_tensor(rows, device=q.device)]).T, codes)
        W8[i] = (q, qt, e)

    def check(key, C, A_T, ea, Bq, eb, R=None, tol=5e-3, cols_of=None):
        """C[r, c] (+ R) == sum_k A[r, k] B[c, k] * 2^(ea + eb), A from its transposed codes."""
        rows = S.idx(A_T.shape[1])
        cols = S.idx(Bq.shape[0] if cols_of is None else cols_of)
        a = _codes_rows(A_T, rows)
        b = _u8(Bq[torch.as_tensor(cols, device=Bq.device)])
        ref = np.einsum("ik,ik->i", o8.dequantize(a, ea), o8.dequantize(b, eb))
        if R is not None:
            ref = ref + to_f64(R[torch.as_tensor(rows, device=R.device), torch.as_tensor(cols, device=R.device)])
        got = to_f64(C[torch.as_tensor(rows, device=C.device), torch.as_tensor(cols, device=C.device)])
        S.record(key, got, ref, tol)

    for j in range(m):
        for l in range(L):
            T_ = lambda which: st.stash(j, l, which)
            ex = T_(zb.L_QEXP).cpu().numpy().ravel().tolist()
            e_n1, e_a, e_n2, e_s, e_dout, e_dgu, e_dh1, e_dqkv = ex
            # every exponent the smallest that fits (largest code in [224, 448],
            # as in the small-stage test), over each whole tensor; E4M3
            # magnitudes order as their 7-bit codes (0x7f is NaN)
            for k in (zb.L_N1T, zb.L_AT, zb.L_N2T, zb.L_ST, zb.L_DOUTT, zb.L_DGUT, zb.L_DH1T, zb.L_DQKVT):
                top_code = int((T_(k) & 0x7F).max().item())
                top = float(o8.e4m3_decode(np.array([top_code], dtype=np.uint8))[0])
                assert 224.0 <= top <= 448.0, (j, l, k, top_code)
            w = 6 * l
            out = ys[j] if l == L - 1 else st.stash(j, l + 1, zb.L_X)
            check("qkv", T_(zb.L_QKV), T_(zb.L_N1T), e_n1, W8[w][0], W8[w][2])
            check("o + residual", T_(zb.L_H1), T_(zb.L_AT), e_a, W8[w + 1][0], W8[w + 1][2], R=T_(zb.L_X))
            check("gate/up", T_(zb.L_GU), T_(zb.L_N2T), e_n2, W8[w + 2][0], W8[w + 2][2])
            check("down + residual", out, T_(zb.L_ST), e_s, W8[w + 3][0], W8[w + 3][2], R=T_(zb.L_H1))
            check("gate/up bwd", T_(zb.L_DN2), T_(zb.L_DGUT), e_dgu, W8[w + 2][1], W8[w + 2][2])
            check("qkv bwd", T_(zb.L_DN1), T_(zb.L_DQKVT), e_dqkv, W8[w][1], W8[w][2])
    # W over both microbatches, sampled entries from the stashed codes
    prods = ((0, zb.L_DQKVT, zb.L_N1T, 7, 0), (1, zb.L_DH1T, zb.L_AT, 6, 1), (2, zb.L_DGUT, zb.L_N2T, 5, 2),
             (3, zb.L_DOUTT, zb.L_ST, 4, 3))
    sel, ref = {}, {}
    for l in range(L):
        for wi, dyk, xk, ey, ex_ in prods:
            M_, N_ = st.dw[6 * l + wi].shape
            o, i = S.idx(M_), S.idx(N_)
            sel[(l, wi)] = (o, i)
            r = np.zeros(len(o))
            for j in range(m):
                ee = st.stash(j, l, zb.L_QEXP).cpu().numpy().ravel()
                A = st.stash(j, l, dyk)  # [M][T] codes
                B = st.stash(j, l, xk)   # [N][T] codes
                a = _u8(A[torch.as_tensor(o, device=A.device)])
                b = _u8(B[torch.as_tensor(i, device=B.device)])
                r += np.einsum("ik,ik->i", o8.dequantize(a, int(ee[ey])), o8.dequantize(b, int(ee[ex_])))
            ref[(l, wi)] = r
    for j in range(m):
        st.bwd_weight(j)
    torch.cuda.synchronize()
    for (l, wi), (o, i) in sel.items():
        dw = st.dw[6 * l + wi]
        got = to_f64(dw[torch.as_tensor(o, device=dw.device), torch.as_tensor(i, device=dw.device)])
        S.record(f"dW{wi}", got, ref[(l, wi)], 5e-3)
    print({k: f"{v:.2e}" for k, v in S.err.items()})
