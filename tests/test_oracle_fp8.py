"""Pins of oracle.fp8 (CPU): the E4M3 decoding and rounding against torch's
float8_e4m3fn conversion (a library routine of the same OCP format) and
hand-computed codes, the per-tensor scale's defining inequality, the
quantization error bound, the fp8 product against brute-force loops, and
the fp8 Llama stage against the already-pinned dense stage."""
import math

import numpy as np
import pytest
import torch

from oracle import dense as od
from oracle import fp8

F8 = torch.float8_e4m3fn


def _torch_codes(x_f32: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(x_f32, dtype=np.float32)).to(F8).view(torch.uint8).numpy()


def test_decode_every_code():
    codes = np.arange(256, dtype=np.uint8)
    ours = fp8.e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(F8).to(torch.float32).numpy().astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan) and nan.sum() == 2  # S.1111.111 only
    assert np.array_equal(ours[~nan], ref[~nan])
    # hand values: 1, 448, the smallest subnormal and normal, -2, -0
    assert fp8.e4m3_decode([0x38, 0x7E, 0x01, 0x08, 0xC0]).tolist() == [1.0, 448.0, 2.0 ** -9, 2.0 ** -6, -2.0]
    assert math.copysign(1.0, fp8.e4m3_decode([0x80])[0]) == -1.0


def _finite_values():
    v = fp8.e4m3_decode(np.arange(256, dtype=np.uint8))
    return np.unique(v[np.isfinite(v)])


def test_round_trip_of_every_value():
    v = _finite_values()
    assert np.array_equal(fp8.e4m3_decode(fp8.e4m3_round(v)), v)


def test_round_ties_and_neighbours_like_torch():
    v = _finite_values()
    v = v[v >= 0]
    mids = (v[:-1] + v[1:]) / 2
    xs = np.concatenate([mids, -mids, np.nextafter(mids.astype(np.float32), np.float32(0)),
                         np.nextafter(mids.astype(np.float32), np.float32(1e9))]).astype(np.float32)
    assert np.array_equal(fp8.e4m3_round(xs.astype(np.float64)), _torch_codes(xs))
    # a tie goes to the even code: 1 + 1/16 lies between codes 0x38 (1) and 0x39 (1.125)
    assert fp8.e4m3_round([1.0625, 1.1875])[0] == 0x38 and fp8.e4m3_round([1.1875])[0] == 0x3A


@pytest.mark.parametrize("seed", [0, 1])
def test_round_random_like_torch(seed):
    rng = np.random.default_rng(seed)
    x = np.concatenate([rng.uniform(-448, 448, 50000), rng.standard_normal(50000),
                        rng.uniform(-2.0 ** -6, 2.0 ** -6, 20000)]).astype(np.float32)
    assert np.array_equal(fp8.e4m3_round(x.astype(np.float64)), _torch_codes(x))


def test_round_rejects_out_of_range():
    for bad in ([449.0], [np.inf], [np.nan]):
        with pytest.raises(ValueError):
            fp8.e4m3_round(bad)


def test_scale_exponent_definition():
    assert fp8.scale_exponent(0.0) == 0
    assert fp8.scale_exponent(448.0) == 0
    assert fp8.scale_exponent(449.0) == 1
    assert fp8.scale_exponent(224.0) == -1
    assert fp8.scale_exponent(448.0 * 2 ** -20) == -20
    rng = np.random.default_rng(3)
    for a in np.exp(rng.uniform(-30, 30, 2000)):
        e = fp8.scale_exponent(a)
        assert a <= math.ldexp(448.0, e) and a > math.ldexp(448.0, e - 1)


@pytest.mark.parametrize("std", [1.0, 1e-2, 3e-5, 40.0])
def test_quantize_error_bound(std):
    rng = np.random.default_rng(4)
    x = rng.standard_normal((64, 96)) * std
    q, e = fp8.quantize(x)
    d = fp8.dequantize(q, e)
    assert np.max(np.abs(x)) <= 448.0 * 2.0 ** e and np.max(np.abs(x)) > 224.0 * 2.0 ** e
    scaled = np.abs(x) * 2.0 ** -e
    normal = scaled >= 2.0 ** -6
    # half an E4M3 spacing: 2^-4 relative for normal values, 2^-10 (times the scale) below
    assert np.all(np.abs(d - x)[normal] <= 2.0 ** -4 * np.abs(x)[normal])
    assert np.all(np.abs(d - x)[~normal] <= 2.0 ** -10 * 2.0 ** e)
    assert np.array_equal(fp8.fake_quant(x), d)


def test_quantize_zero_tensor():
    q, e = fp8.quantize(np.zeros((3, 4)))
    assert e == 0 and not q.any()


def test_product_nt_brute_force():
    rng = np.random.default_rng(5)
    qa = fp8.e4m3_round(rng.uniform(-448, 448, (3, 5)))
    qb = fp8.e4m3_round(rng.uniform(-448, 448, (4, 5)))
    c = fp8.product_nt(qa, 2, qb, -3)
    for i in range(3):
        for j in range(4):
            s = 0.0
            for k in range(5):
                s += float(fp8.e4m3_decode([qa[i, k]])[0]) * 4.0 * float(fp8.e4m3_decode([qb[j, k]])[0]) / 8.0
            assert c[i, j] == pytest.approx(s, rel=1e-14)


DIMS = od.LlamaDims(8, 12, 2, 1, 4)


def _tiny_stage(cls, **kw):
    rng = np.random.default_rng(6)
    w = []
    for _ in range(2):
        w += [rng.standard_normal((16, 8)) * 0.3, rng.standard_normal((8, 8)) * 0.3,
              rng.standard_normal((24, 8)) * 0.3, rng.standard_normal((8, 12)) * 0.3,
              1 + 0.1 * rng.standard_normal(8), 1 + 0.1 * rng.standard_normal(8)]
    return (cls(w, DIMS, 2, **kw) if cls is fp8.Fp8LlamaStage else cls("llama", w, DIMS, 2)), rng


def _run(st, rng):
    x = [rng.standard_normal((6, 8)) for _ in range(2)]
    dy = [rng.standard_normal((6, 8)) for _ in range(2)]
    ys = [st.fwd(j, x[j]) for j in range(2)]
    dxs = [st.bwd_input(j, dy[j]) for j in range(2)]
    for j in range(2):
        st.bwd_weight(j)
    return ys, dxs, st.grad


def test_fp8_stage_without_quantization_is_the_dense_stage(monkeypatch):
    """With the quantizer replaced by the identity, the fp8 stage is the
    dense stage bit for bit: no term of the layer is dropped or reordered."""
    monkeypatch.setattr(fp8, "fake_quant", lambda t: t)
    a = _run(*_tiny_stage(fp8.Fp8LlamaStage))
    b = _run(*_tiny_stage(od.Stage))
    for xa, xb in zip(a[0] + a[1] + a[2], b[0] + b[1] + b[2]):
        assert np.array_equal(xa, xb)


def test_fp8_stage_within_the_e4m3_bound_of_the_dense_stage():
    """E4M3 keeps 3 mantissa bits (unit roundoff 2^-4, rms error 2^-4/sqrt(3)
    = 3.6% per rounded operand): every output and gradient of the fp8 stage
    lies within 0.25 relative (Frobenius) of the exact stage, and is not
    identical to it.  A gradient of the first layer passes through up to
    five rounded products along the backward chain, and at these tiny widths
    (K = 6..24) nothing averages out."""
    a = _run(*_tiny_stage(fp8.Fp8LlamaStage))
    b = _run(*_tiny_stage(od.Stage))
    worst = 0.0
    for xa, xb in zip(a[0] + a[1] + a[2], b[0] + b[1] + b[2]):
        worst = max(worst, od.rel_fro(xa, xb))
    assert 1e-4 < worst < 0.25, worst


def test_fp8_stage_quantizes_both_operands_of_every_product(monkeypatch):
    """Per layer and microbatch, F, B and W each run four linear products,
    each on two quantized operands: 8 quantizer calls per pass per layer,
    with the operand shapes of the products."""
    calls = []

    def counting(t):
        calls.append(t.shape)
        return t

    monkeypatch.setattr(fp8, "fake_quant", counting)
    st, rng = _tiny_stage(fp8.Fp8LlamaStage)
    x, dy = rng.standard_normal((6, 8)), rng.standard_normal((6, 8))
    st.fwd(0, x)
    assert len(calls) == 2 * 8
    assert calls[:8] == [(6, 8), (16, 8), (6, 8), (8, 8), (6, 8), (24, 8), (6, 12), (8, 12)]
    calls.clear()
    st.bwd_input(0, dy)
    assert len(calls) == 2 * 8
    assert calls[:8] == [(6, 8), (8, 12), (6, 24), (24, 8), (6, 8), (8, 8), (6, 16), (16, 8)]
    calls.clear()
    st.bwd_weight(0)
    assert len(calls) == 2 * 8
    assert calls[:8] == [(6, 16), (6, 8), (6, 8), (6, 8), (6, 24), (6, 8), (6, 8), (6, 12)]
