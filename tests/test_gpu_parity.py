"""GPU parity: libzb's F / B / W against the fp64 oracle, element by element,
on the same seeded inputs (through the C ABI via the Python binding).

Tolerances (relative Frobenius error per tensor, max over tensors):
* fp32 linear stage: 1e-5.
* bf16 stages (bf16 operands and stored activations, fp32 accumulation):
  2e-2.
* bare GEMM with bf16 output: 2.5e-3 -- the only error is the final
  round-to-nearest to bf16 (relative error <= 2^-9 = 1.95e-3 per element)
  plus fp32 accumulation error (~1e-6 at these K).
* bare GEMM accumulating into fp32: 1e-5 (inputs are exact bf16 values; only
  fp32 accumulation rounding remains).
"""
import numpy as np
import pytest
import torch

import split_backward_amd as zb
import synth
from oracle import dense as od
from tests.gpu_helpers import make_stage, max_rel, run_both, to_dev, to_f64

pytestmark = pytest.mark.gpu

BF16_TOL = 2e-2
F32_TOL = 1e-5


def setup_module(module):
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    zb.lib()  # loud failure if the library was not built


# ------------------------------------------------------------- bare GEMM ---

def _bf16(name, shape, seed, std=1.0):
    return synth.make_tensor(name, seed, shape, std, "bf16")


@pytest.mark.parametrize("M,N,K", [(264, 136, 72), (512, 512, 512), (8, 8, 8), (1000, 24, 64), (256, 776, 1032)])
def test_gemm_nt_bf16(M, N, K):
    """F form: C = A . B^T with both operands K-contiguous."""
    a, b = _bf16("a", (M, K), 11), _bf16("b", (N, K), 12)
    c = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    zb.gemm(to_dev(a), to_dev(b), c, a_kmajor=True, b_kmajor=True, M=M, N=N, K=K)
    torch.cuda.synchronize()
    assert od.rel_fro(to_f64(c), a.f64 @ b.f64.T) <= 2.5e-3


@pytest.mark.parametrize("M,N,K,b_kmajor", [
    (500, 129 * 256 + 40, 64, True),   # 2 x 130 tiles: 256-row tiles fill one round, 128-row tiles the rest
    (512, 128 * 256, 32, False),       # 2 x 128 tiles, exactly one round: 256-row tiles only
    (1000, 24, 64, False),             # under one round: 128-row tiles only
])
def test_gemm_tile_heights_bitwise_and_parity(M, N, K, b_kmajor, monkeypatch):
    """Products with a K-contiguous A mix 256-row and 128-row tiles by how
    the tile count fills the chip's rounds (the cases above are for 256 CUs).
    The result equals, bit for bit, the one with every tile 256 rows high
    (ZB_GEMM_FULL_TILES=1), and the oracle's product."""
    a = _bf16("a", (M, K), 21)
    b = _bf16("b", (N, K) if b_kmajor else (K, N), 22)
    outs = []
    for full in (False, True):
        if full:
            monkeypatch.setenv("ZB_GEMM_FULL_TILES", "1")
        c = torch.full((M, N), 7.0, dtype=torch.bfloat16, device="cuda")
        zb.gemm(to_dev(a), to_dev(b), c, a_kmajor=True, b_kmajor=b_kmajor, M=M, N=N, K=K)
        torch.cuda.synchronize()
        outs.append(c.cpu())
    assert torch.equal(outs[0], outs[1])
    ref = a.f64 @ (b.f64.T if b_kmajor else b.f64)
    assert od.rel_fro(to_f64(outs[0]), ref) <= 2.5e-3


@pytest.mark.parametrize("M,N,K", [(264, 136, 72), (512, 512, 512), (8, 8, 8), (300, 1032, 24)])
def test_gemm_nn_bf16(M, N, K):
    """B form: C = A . W with W stored [K, N] (N contiguous)."""
    a, w = _bf16("a", (M, K), 13), _bf16("w", (K, N), 14)
    c = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    zb.gemm(to_dev(a), to_dev(w), c, a_kmajor=True, b_kmajor=False, M=M, N=N, K=K)
    torch.cuda.synchronize()
    assert od.rel_fro(to_f64(c), a.f64 @ w.f64) <= 2.5e-3


@pytest.mark.parametrize("M,N,K", [(264, 136, 72), (512, 512, 512), (8, 8, 8), (136, 1032, 296)])
def test_gemm_tn_accumulate_f32(M, N, K):
    """W form: dW[M,N] += dY[K,M]^T . X[K,N], fp32 in place, twice."""
    dy, x = _bf16("dy", (K, M), 15), _bf16("x", (K, N), 16)
    c0 = synth.normal(17, (M, N), 1.0).astype(np.float32)
    c = torch.from_numpy(c0.copy()).cuda()
    for _ in range(2):
        zb.gemm(to_dev(dy), to_dev(x), c, a_kmajor=False, b_kmajor=False, M=M, N=N, K=K, accumulate=True)
    torch.cuda.synchronize()
    ref = c0.astype(np.float64) + 2.0 * (dy.f64.T @ x.f64)
    assert od.rel_fro(to_f64(c), ref) <= F32_TOL


def test_wgrad_group_matches_single_launches_and_oracle():
    """Grouped W-pass launch: 18 products (two launches of at most 16, one
    ragged in every dimension, one too wide for 16-byte epilogue accesses so
    it takes the fallback kernel) equal the single launches bit for bit, and
    the oracle within the fp32-accumulate tolerance."""
    shapes = [(264, 136, 72), (512, 512, 512), (8, 8, 8), (136, 1032, 296), (1024, 256, 64), (40, 264, 24)] * 3
    padded = 5  # C with leading dimension N + 2: no 16-byte epilogue, first-generation kernel inside the group call
    As, Bs, C1, C2, refs = [], [], [], [], []
    for i, (M, N, K) in enumerate(shapes):
        dy, x = _bf16(f"gdy{i}", (K, M), 40 + i), _bf16(f"gx{i}", (K, N), 80 + i)
        c0 = synth.normal(120 + i, (M, N), 1.0).astype(np.float32)
        As.append(to_dev(dy)); Bs.append(to_dev(x))
        for lst in (C1, C2):
            if i == padded:
                big = torch.zeros((M, N + 2), dtype=torch.float32, device="cuda")
                big[:, :N] = torch.from_numpy(c0)
                lst.append(big[:, :N])
            else:
                lst.append(torch.from_numpy(c0.copy()).cuda())
        refs.append(c0.astype(np.float64) + dy.f64.T @ x.f64)
    Ms, Ns, Ks = [s_[0] for s_ in shapes], [s_[1] for s_ in shapes], [s_[2] for s_ in shapes]
    zb.gemm_wgrad_group(As, Bs, C1, Ms, Ns, Ks)
    for A, B, C, (M, N, K) in zip(As, Bs, C2, shapes):
        zb.gemm(A, B, C, a_kmajor=False, b_kmajor=False, M=M, N=N, K=K, accumulate=True, ldc=C.stride(0))
    torch.cuda.synchronize()
    for i, (c1, c2, ref) in enumerate(zip(C1, C2, refs)):
        assert torch.equal(c1, c2), i
        assert od.rel_fro(to_f64(c1), ref) <= F32_TOL, i


def test_gemm_fp32_all_layouts():
    M, N, K = 200, 136, 72
    rng = np.random.default_rng(5)
    a = rng.standard_normal((M, K)).astype(np.float32)
    b = rng.standard_normal((K, N)).astype(np.float32)
    A, B = torch.from_numpy(a).cuda(), torch.from_numpy(b).cuda()
    ref = a.astype(np.float64) @ b.astype(np.float64)
    for ak in (True, False):
        for bk in (True, False):
            Ad = A if ak else A.t().contiguous()
            Bd = B.t().contiguous() if bk else B
            c = torch.zeros((M, N), dtype=torch.float32, device="cuda")
            zb.gemm(Ad, Bd, c, a_kmajor=ak, b_kmajor=bk, M=M, N=N, K=K)
            torch.cuda.synchronize()
            assert od.rel_fro(to_f64(c), ref) <= F32_TOL, (ak, bk)


# ---------------------------------------------------------------- stages ---

def test_linear_fp32_workload_parity():
    """fp32 linear layer X[128x256] W[256x256], m = 2, deferred W."""
    wl = synth.WORKLOADS["linear_f32"]
    gpu, orc, _ = run_both(wl["shape"], wl["m"])
    r = max_rel(gpu, orc)
    assert max(r.values()) <= F32_TOL, r


def test_linear_fp32_ragged_parity():
    shape = synth.StageShape("linear", 200, 136, 72, dtype="f32")
    gpu, orc, _ = run_both(shape, 3, ring=3)
    r = max_rel(gpu, orc)
    assert max(r.values()) <= F32_TOL, r


def test_linear_bf16_ragged_parity():
    shape = synth.StageShape("linear", 296, 136, 520)
    gpu, orc, _ = run_both(shape, 3)
    r = max_rel(gpu, orc)
    assert max(r.values()) <= BF16_TOL, r


@pytest.mark.parametrize("kind_shape", [
    synth.StageShape("linear", 128, 256, 256, dtype="f32"),
    synth.StageShape("mlp", 296, 136, 520),
])
def test_deferred_equals_immediate_bitwise(kind_shape):
    """F0 F1 B0 B1 W0 W1 == F0 B0 W0 F1 B1 W1 on the GPU, bit for bit: the W
    kernel adds each microbatch into dW in issue order, without atomics."""
    g1, _, _ = run_both(kind_shape, 2, order="deferred")
    g2, _, _ = run_both(kind_shape, 2, order="immediate")
    for k in ("y", "dx", "dw"):
        for a, b in zip(g1[k], g2[k]):
            assert np.array_equal(a, b), k


def test_mlp_ragged_parity():
    shape = synth.StageShape("mlp", 296, 136, 520)
    gpu, orc, _ = run_both(shape, 3)
    r = max_rel(gpu, orc)
    assert max(r.values()) <= BF16_TOL, r


def test_mlp_split_k_ragged_parity():
    """264 tokens at h=1024, ffn=2048: every product's half-height tiles fill
    few CUs, so all four run split along K (fc1 and its input gradient in 2
    slices, fc2 and the stage's input gradient in 4), with a ragged last
    tile row."""
    shape = synth.StageShape("mlp", 264, 1024, 2048)
    gpu, orc, _ = run_both(shape, 2)
    r = max_rel(gpu, orc)
    assert max(r.values()) <= BF16_TOL, r


def test_mlp_split_k_bitwise_deterministic():
    """The split-K slices overwrite every partial sum they own: two stages on
    the same inputs, whose workspaces start filled with NaN and with large
    finite bit patterns, give bitwise-equal y, dx and dW."""
    shape = synth.StageShape("mlp", 264, 1024, 2048)
    weights = synth.make_weights(shape)
    xs = [to_dev(synth.make_x(shape, j)) for j in range(2)]
    dys = [to_dev(synth.make_dy(shape, j)) for j in range(2)]
    outs = []
    for fill in (0xFF, 0x7F):
        st, _ = make_stage(shape, 2, weights=weights)
        st.ws.fill_(fill)
        st.zero_grad()
        ys = [st.fwd(j, xs[j]).clone() for j in range(2)]
        dxs = [st.bwd_input(j, dys[j]).clone() for j in range(2)]
        for j in range(2):
            st.bwd_weight(j)
        torch.cuda.synchronize()
        outs.append(ys + dxs + [d.clone() for d in st.dw])
    for a, b in zip(*outs):
        assert torch.equal(a, b)
        assert torch.isfinite(a.float()).all()


def test_mlp_full_width_parity():
    """GPT MLP at its full shape (s=2048, h=1024, ffn=4096), 2 microbatches
    (fc2 and the stage's input gradient run split along K)."""
    shape = synth.WORKLOADS["gpt_mlp_h1024"]["shape"]
    gpu, orc, _ = run_both(shape, 2)
    r = max_rel(gpu, orc)
    assert max(r.values()) <= BF16_TOL, r


@pytest.mark.parametrize("shape", [
    synth.StageShape("llama", 256, 256, 344, n_layers=2, n_heads=2, n_kv_heads=1, head_dim=128),
    synth.StageShape("llama", 384, 512, 1032, n_layers=1, n_heads=4, n_kv_heads=2, head_dim=128),
    synth.StageShape("llama", 128, 384, 256, n_layers=1, n_heads=3, n_kv_heads=3, head_dim=128),
])
def test_llama_small_parity(shape):
    gpu, orc, _ = run_both(shape, 2)
    r = max_rel(gpu, orc)
    assert max(r.values()) <= BF16_TOL, r


def test_one_slot_ring_reused_by_every_microbatch():
    """Ring of one slot (memory limit 1): F B W of each microbatch in turn,
    every F reusing the slot the previous W released.  Equal to the oracle,
    and bit for bit to the same order with a slot per microbatch."""
    shape = synth.StageShape("llama", 256, 256, 344, n_layers=2, n_heads=2, n_kv_heads=1, head_dim=128)
    g1, orc, _ = run_both(shape, 3, ring=1, order="immediate")
    g3, _, _ = run_both(shape, 3, ring=3, order="immediate")
    r = max_rel(g1, orc)
    assert max(r.values()) <= BF16_TOL, r
    for k in ("y", "dx", "dw"):
        for a, b in zip(g1[k], g3[k]):
            assert np.array_equal(a, b), k


# ------------------------------------------------------------ state errors --

def test_stage_state_machine_errors():
    shape = synth.StageShape("linear", 64, 64, 64)
    st, _ = make_stage(shape, ring=2)
    x = to_dev(synth.make_x(shape, 0))
    dy = to_dev(synth.make_dy(shape, 0))
    with pytest.raises(zb.ZbError) as e:
        st.bwd_input(0, dy)
    assert e.value.code == zb.ESTATE
    st.fwd(0, x)
    with pytest.raises(zb.ZbError) as e:
        st.bwd_weight(0)
    assert e.value.code == zb.ESTATE
    with pytest.raises(zb.ZbError) as e:
        st.fwd(2, x)              # out of order
    assert e.value.code == zb.ESTATE
    st.fwd(1, x)
    with pytest.raises(zb.ZbError) as e:
        st.fwd(2, x)              # ring of 2 is full: W(0) not issued
    assert e.value.code == zb.ERING_FULL
    st.bwd_input(0, dy)
    with pytest.raises(zb.ZbError) as e:
        st.bwd_input(0, dy)       # twice
    assert e.value.code == zb.ESTATE
    st.bwd_weight(0)
    st.fwd(2, x)                  # slot freed by W(0)
    with pytest.raises(zb.ZbError) as e:
        st.zero_grad()            # microbatches 1 and 2 still in flight
    assert e.value.code == zb.ESTATE
    torch.cuda.synchronize()
