"""Seeded synthetic inputs shared by the oracle-side tests and the GPU path.

This module draws random numbers and rounds them once to the storage type.
It holds none of the stage's arithmetic (no products, activations or norms),
so both sides of every parity check can take their inputs from here.

Recipe (the pages fix only the weight scale of their PyTorch stage listing,
a standard normal times 0.02; everything else here is a stated reading):

* every value is drawn in float64 from ``numpy.random.default_rng(seed)``
  (PCG64) as a normal variate with the stated standard deviation;
* it is then rounded ONCE, round-to-nearest-even, to the storage type:
  float32 for the fp32 linear workload, bfloat16 for the others;
* weights use seed 0 (drawn in the documented order of the stage's weight
  list), the input activation of microbatch j uses seed 1000 + j and the
  output gradient of microbatch j uses seed 2000 + j;
* weights ~ N(0, 0.02), inputs ~ N(0, 1), output gradients ~ N(0, 1e-2),
  except the fp32 linear workload where all three are N(0, 1);
* RMSNorm gains start at exactly 1.

bf16 values are carried as ``uint16`` bit patterns; ``bf16_to_f64`` widens
them exactly so the fp64 oracle sees the very same numbers.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List

import numpy as np

WEIGHT_SEED = 0
X_SEED_BASE = 1000
DY_SEED_BASE = 2000


# ---------------------------------------------------------------- rounding --

def round_to_bf16_f64(x: np.ndarray) -> np.ndarray:
    """Round float64 values once, to nearest-even, onto the bfloat16 grid.

    bfloat16 keeps 8 significant bits.  ``frexp`` gives a mantissa in
    [0.5, 1); scaling it by 2**8 and rounding half-to-even (``np.rint``)
    keeps exactly 8 significant bits.  Inputs here are far from the bf16
    overflow and subnormal ranges; that is asserted.
    """
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)
    q = np.rint(m * 256.0) / 256.0
    out = np.ldexp(q, e)
    nz = out[out != 0]
    if nz.size:
        a = np.abs(nz)
        assert a.max() < 3.0e38 and a.min() > 1.2e-38, "value outside bf16 normal range"
    return out


def f64_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) of values already on the bf16 grid."""
    f32 = np.asarray(x, dtype=np.float32)
    assert np.array_equal(f32.astype(np.float64), np.asarray(x, np.float64)), "not on the bf16 grid"
    bits = f32.view(np.uint32)
    assert np.all((bits & 0xFFFF) == 0), "not on the bf16 grid"
    return (bits >> 16).astype(np.uint16)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float64."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def normal(seed: int, shape, std: float) -> np.ndarray:
    rng = np.random.default_rng(seed)
    return rng.standard_normal(size=shape, dtype=np.float64) * std


# ------------------------------------------------------------ tensor sets --

@dataclass
class Tensor:
    """One stored tensor: float64 values (exactly representable in the
    storage type) plus the raw storage array handed to the GPU path."""
    name: str
    f64: np.ndarray
    storage: np.ndarray          # float32 array or uint16 bf16 bit patterns
    dtype: str                   # "f32" or "bf16"


def make_tensor(name: str, seed_or_values, shape=None, std=None, dtype="bf16") -> Tensor:
    if isinstance(seed_or_values, np.ndarray):
        vals = seed_or_values.astype(np.float64)
    else:
        vals = normal(seed_or_values, shape, std)
    if dtype == "f32":
        st = vals.astype(np.float32)
        f64 = st.astype(np.float64)
    elif dtype == "bf16":
        f64 = round_to_bf16_f64(vals)
        st = f64_to_bf16_bits(f64)
    else:
        raise ValueError(dtype)
    return Tensor(name, f64, st, dtype)


@dataclass
class StageShape:
    """Shape of one pipeline stage.

    kind: "linear" (one Y = X W^T layer; ``ffn`` is its output width),
          "mlp" (fc1 -> GeLU(tanh) -> fc2), or "llama" (pre-norm decoder
          layers: RMSNorm, causal GQA attention, RMSNorm, SwiGLU).
    """
    kind: str
    tokens: int
    hidden: int
    ffn: int
    n_layers: int = 1
    n_heads: int = 1
    n_kv_heads: int = 1
    head_dim: int = 1
    dtype: str = "bf16"
    rms_eps: float = 1e-5

    @property
    def q_dim(self) -> int:
        return self.n_heads * self.head_dim

    @property
    def kv_dim(self) -> int:
        return self.n_kv_heads * self.head_dim


def weight_shapes(s: StageShape):
    """Documented weight order (storage layout [out, in], PyTorch's linear
    convention).  RMSNorm gains are 1-D [hidden]."""
    if s.kind == "linear":
        return [("w", (s.ffn, s.hidden))]
    if s.kind == "mlp":
        return [("w1", (s.ffn, s.hidden)), ("w2", (s.hidden, s.ffn))]
    if s.kind == "llama":
        out = []
        for l in range(s.n_layers):
            out += [
                (f"l{l}.wqkv", (s.q_dim + 2 * s.kv_dim, s.hidden)),
                (f"l{l}.wo", (s.hidden, s.q_dim)),
                (f"l{l}.wgu", (2 * s.ffn, s.hidden)),
                (f"l{l}.wd", (s.hidden, s.ffn)),
                (f"l{l}.g1", (s.hidden,)),
                (f"l{l}.g2", (s.hidden,)),
            ]
        return out
    raise ValueError(s.kind)


def make_weights(s: StageShape, seed: int = WEIGHT_SEED, std: float = None) -> List[Tensor]:
    """All weights of a stage, drawn in the documented order from one seed."""
    if std is None:
        std = 1.0 if s.kind == "linear" and s.dtype == "f32" else 0.02
    rng = np.random.default_rng(seed)
    out = []
    for name, shape in weight_shapes(s):
        if name.endswith(".g1") or name.endswith(".g2"):
            out.append(make_tensor(name, np.ones(shape), dtype=s.dtype))
        else:
            vals = rng.standard_normal(size=shape, dtype=np.float64) * std
            out.append(make_tensor(name, vals, dtype=s.dtype))
    return out


def out_width(s: StageShape) -> int:
    return s.ffn if s.kind == "linear" else s.hidden


def make_x(s: StageShape, mb: int, std: float = 1.0) -> Tensor:
    return make_tensor(f"x{mb}", X_SEED_BASE + mb, (s.tokens, s.hidden), std, s.dtype)


def make_dy(s: StageShape, mb: int, std: float = None) -> Tensor:
    if std is None:
        std = 1.0 if s.dtype == "f32" else 1e-2
    return make_tensor(f"dy{mb}", DY_SEED_BASE + mb, (s.tokens, out_width(s)), std, s.dtype)


def to_device(t: Tensor, device="cuda"):
    """The tensor's storage bytes as a torch tensor on `device` (float32, or
    bfloat16 from the bit patterns): a copy of the very values the oracle
    reads, nothing computed."""
    import torch
    if t.dtype == "f32":
        return torch.from_numpy(t.storage.copy()).to(device)
    return torch.from_numpy(t.storage.view(np.int16).copy()).view(torch.bfloat16).to(device)


# Named workloads (the pages' stage shapes; sizes only, no arithmetic).
WORKLOADS = {
    # fp32 single linear layer, X[128x256] W[256x256], 2 microbatches
    "linear_f32": dict(shape=StageShape("linear", 128, 256, 256, dtype="f32"), m=2),
    # GPT-style MLP block, h=1024, ffn=4096, s=2048, 8 microbatches
    "gpt_mlp_h1024": dict(shape=StageShape("mlp", 2048, 1024, 4096), m=8),
    # Llama-7B-shape stage: 4 decoder layers, h=4096, 32 heads, ffn 11008, s=4096, 16 microbatches
    "llama7b_stage4": dict(shape=StageShape("llama", 4096, 4096, 11008, n_layers=4,
                                            n_heads=32, n_kv_heads=32, head_dim=128), m=16),
    # the same stage with every linear product on E4M3 operands (stage dtype fp8)
    "llama7b_stage4_fp8": dict(shape=StageShape("llama", 4096, 4096, 11008, n_layers=4,
                                                n_heads=32, n_kv_heads=32, head_dim=128), m=16, stage_dtype="fp8"),
    # Llama-70B-shape slice: 2 layers, h=8192, 64/8 heads, ffn 28672, s=4096, 24 microbatches, 8-slot ring
    "llama70b_slice2": dict(shape=StageShape("llama", 4096, 8192, 28672, n_layers=2,
                                             n_heads=64, n_kv_heads=8, head_dim=128), m=24, ring=8),
}
