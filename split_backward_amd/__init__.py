"""Python binding of libzb (the split-backward pipeline stage for MI355X).

Argument marshalling only: every step of F, B and W runs in the HIP kernels
of libzb.so.  PyTorch supplies device memory (tensors) and streams; tensors
are passed to the C ABI as raw device pointers.  If libzb.so is missing the
import of this module still works, but every call raises -- there is no CPU
fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import List, Optional, Sequence

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libzb.so")

# ---- constants mirrored from include/zb.h ---------------------------------
OK, EINVAL, ESTATE, ERING_FULL, EHIP, ENOMEM = 0, -1, -2, -3, -4, -5
F32, BF16, FP8, E4M3, I32 = 0, 1, 2, 3, 4
DTYPE = {"f32": F32, "bf16": BF16, "fp8": FP8}
LINEAR, MLP_GELU, LLAMA = 0, 1, 2
OP_F, OP_B, OP_W, OP_O = 0, 1, 2, 3
DEBUG_SLOT_TAGS, DEBUG_SERIALIZE = 1, 2
SCHED_GPIPE, SCHED_1F1B, SCHED_ZB = 0, 1, 2
EXEC_ORDERED, EXEC_FILLER = 0, 1

KIND = {"linear": LINEAR, "mlp": MLP_GELU, "llama": LLAMA}
SCHED = {"gpipe": SCHED_GPIPE, "1f1b": SCHED_1F1B, "zb": SCHED_ZB}
OPNAME = {OP_F: "F", OP_B: "B", OP_W: "W", OP_O: "O"}

# stash tensor indices ("which")
LIN_X, LIN_DY = 0, 1
MLP_X, MLP_A, MLP_H, MLP_DY, MLP_DA = 0, 1, 2, 3, 4
(L_X, L_R1, L_N1, L_QKV, L_A, L_LSE, L_H1, L_R2, L_N2, L_GU, L_S,
 L_DOUT, L_DGU, L_DN2, L_DH1, L_DQKV, L_DN1,
 L_N1T, L_AT, L_N2T, L_ST, L_DOUTT, L_DGUT, L_DH1T, L_DQKVT, L_QEXP) = range(26)


class ZbError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"libzb error {code}: {msg}")
        self.code = code


class StageDesc(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("dtype", ctypes.c_int32), ("n_layers", ctypes.c_int32),
                ("tokens", ctypes.c_int32), ("hidden", ctypes.c_int32), ("ffn", ctypes.c_int32),
                ("n_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("rms_eps", ctypes.c_float), ("ring_slots", ctypes.c_int32)]


class Op(ctypes.Structure):
    _fields_ = [("type", ctypes.c_int32), ("mb", ctypes.c_int32)]


class ChunkOp(ctypes.Structure):
    _fields_ = [("type", ctypes.c_int32), ("chunk", ctypes.c_int32), ("mb", ctypes.c_int32)]


class SchedStats(ctypes.Structure):
    _fields_ = [("makespan", ctypes.c_int64), ("busy", ctypes.c_int64), ("first_start", ctypes.c_int64),
                ("last_end", ctypes.c_int64), ("peak_active", ctypes.c_int32), ("n_ops", ctypes.c_int32)]


class RunStats(ctypes.Structure):
    _fields_ = [("t_first_start_ms", ctypes.c_double), ("t_last_end_ms", ctypes.c_double),
                ("window_ms", ctypes.c_double), ("busy_ms", ctypes.c_double),
                ("in_window_idle", ctypes.c_double), ("wait_late_ms", ctypes.c_double)]


_vp, _i32, _i64, _sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
_PROTOS = {
    "zb_stage_num_weights": (_i32, [ctypes.POINTER(StageDesc)]),
    "zb_stage_workspace_bytes": (_sz, [ctypes.POINTER(StageDesc)]),
    "zb_stage_create": (_i32, [ctypes.POINTER(StageDesc), ctypes.POINTER(_vp), ctypes.POINTER(_vp), _vp, _sz,
                               ctypes.POINTER(_vp)]),
    "zb_stage_destroy": (None, [_vp]),
    "zb_fwd": (_i32, [_vp, _i32, _vp, _vp, _vp]),
    "zb_bwd_input": (_i32, [_vp, _i32, _vp, _vp, _vp]),
    "zb_bwd_weight_accum": (_i32, [_vp, _i32, _vp]),
    "zb_bwd_weight_accum_pair": (_i32, [_vp, _i32, _vp]),
    "zb_bwd_weight_accum_noalloc": (_i32, [_vp, _i32, _vp]),
    "zb_stage_zero_grad": (_i32, [_vp, _vp]),
    "zb_stage_sgd_step": (_i32, [_vp, ctypes.c_float, _vp]),
    "zb_stage_set_lr": (_i32, [_vp, ctypes.c_float]),
    "zb_stage_weights_changed": (_i32, [_vp]),
    "zb_stage_set_debug": (_i32, [_vp, _i32, _i32, _vp]),
    "zb_stage_debug_report": (_i32, [_vp, ctypes.POINTER(_i32)]),
    "zb_stage_stash_tensor": (_i32, [_vp, _i32, _i32, _i32, ctypes.POINTER(_vp), ctypes.POINTER(_i32),
                                     ctypes.POINTER(_i32), ctypes.POINTER(_i32)]),
    "zb_schedule_generate": (_i32, [_i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, ctypes.POINTER(Op),
                                    ctypes.POINTER(_i64), ctypes.POINTER(_i64), _i32, ctypes.POINTER(_i64),
                                    ctypes.POINTER(_i64), ctypes.POINTER(SchedStats)]),
    "zb_schedule_generate_iters": (_i32, [_i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, ctypes.POINTER(Op),
                                          ctypes.POINTER(_i64), ctypes.POINTER(_i64), _i32, ctypes.POINTER(_i64),
                                          ctypes.POINTER(_i64), ctypes.POINTER(SchedStats)]),
    "zb_stage_run_schedule": (_i32, [_vp, ctypes.POINTER(Op), _i32, ctypes.POINTER(ctypes.c_double),
                                     ctypes.POINTER(ctypes.c_double), ctypes.c_double, ctypes.POINTER(_vp),
                                     ctypes.POINTER(_vp), ctypes.POINTER(_vp), ctypes.POINTER(_vp), _vp, _vp, _i32,
                                     ctypes.POINTER(RunStats), ctypes.POINTER(ctypes.c_double)]),
    "zb_schedule_generate_interleaved": (_i32, [_i32, _i32, _i32, _i32, _i32, _i32, _i32, ctypes.POINTER(ChunkOp),
                                                ctypes.POINTER(_i64), ctypes.POINTER(_i64), _i32, ctypes.POINTER(_i64),
                                                ctypes.POINTER(_i64), ctypes.POINTER(SchedStats)]),
    "zb_run_schedule_chunks": (_i32, [ctypes.POINTER(_vp), _i32, ctypes.POINTER(ChunkOp), _i32, _i32,
                                      ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_double), ctypes.c_double,
                                      ctypes.POINTER(_vp), ctypes.POINTER(_vp), ctypes.POINTER(_vp),
                                      ctypes.POINTER(_vp), _vp, _vp, _i32, ctypes.POINTER(RunStats),
                                      ctypes.POINTER(ctypes.c_double)]),
    "zb_stage_fp8_weight": (_i32, [_vp, _i32, ctypes.POINTER(_vp), ctypes.POINTER(_vp), ctypes.POINTER(_vp)]),
    "zb_quantize_e4m3": (_i32, [_vp, _i32, _i32, _i64, _vp, _i64, _vp, _i64, _vp, _vp, _vp]),
    "zb_gemm_fp8": (_i32, [_i32, _i32, _i32, _vp, _i64, _vp, _vp, _i64, _vp, _vp, _i64, _i32, _vp]),
    "zb_gemm_fp8_wgrad_group": (_i32, [_i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    "zb_gemm": (_i32, [_i32, _i32, _i32, _i32, _vp, _i64, _i32, _vp, _i64, _i32, _vp, _i64, _i32, _i32, _vp]),
    "zb_gemm_wgrad_group": (_i32, [_i32, _vp, _vp, _vp, _vp, _vp, _i32, _vp, _vp, _i32, _vp, _vp, _vp]),
    "zb_last_error": (ctypes.c_char_p, []),
    "zb_version": (ctypes.c_char_p, []),
}
EXPORTS = tuple(_PROTOS)

_lib = None


def lib() -> ctypes.CDLL:
    """Load libzb.so once.  Raises if it has not been built: there is no
    fallback path."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m split_backward_amd.build`")
        l = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _PROTOS.items():
            fn = getattr(l, name)
            fn.restype = res
            fn.argtypes = args
        _lib = l
    return _lib


def last_error() -> str:
    return lib().zb_last_error().decode()


def check(rc: int) -> int:
    if rc < 0:
        raise ZbError(rc, last_error())
    return rc


# ---- schedules (host only) -------------------------------------------------

def schedule_generate(kind: str, p: int, m: int, mem_limit: int = 0, costs=(1, 1, 1), stage: int = 0) -> dict:
    """Per-stage op order from the library's generator (no GPU needed)."""
    n = 3 * m
    ops = (Op * n)()
    st = (ctypes.c_int64 * n)()
    en = (ctypes.c_int64 * n)()
    af = (ctypes.c_int64 * m)()
    ab = (ctypes.c_int64 * m)()
    stats = SchedStats()
    cnt = lib().zb_schedule_generate(SCHED[kind], p, m, mem_limit, costs[0], costs[1], costs[2], stage, ops, st,
                                     en, n, af, ab, ctypes.byref(stats))
    check(cnt)
    return {
        "ops": [(OPNAME[ops[i].type], ops[i].mb) for i in range(cnt)],
        "start": list(st[:cnt]), "end": list(en[:cnt]),
        "arrive_f": list(af), "arrive_b": list(ab),
        "makespan": stats.makespan, "busy": stats.busy, "first_start": stats.first_start,
        "last_end": stats.last_end, "peak_active": stats.peak_active,
    }


def schedule_generate_iters(p: int, m: int, mem_limit: int, costs=(1, 1, 1), c_opt: int = 1, n_iter: int = 2,
                            stage: int = 0, kind: str = "zb") -> dict:
    """Zero-bubble (or 1F1B) order of n_iter iterations for one stage, with
    an optimizer step ("O", iteration) closing each (no GPU needed).  F, B, W
    ops carry the global microbatch index it * m + j; arrivals are indexed
    by it."""
    G = m * n_iter
    n = 3 * G + n_iter
    ops = (Op * n)()
    st = (ctypes.c_int64 * n)()
    en = (ctypes.c_int64 * n)()
    af = (ctypes.c_int64 * G)()
    ab = (ctypes.c_int64 * G)()
    stats = SchedStats()
    cnt = lib().zb_schedule_generate_iters(SCHED[kind], p, m, mem_limit, costs[0], costs[1], costs[2], c_opt, n_iter,
                                           stage, ops, st, en, n, af, ab, ctypes.byref(stats))
    check(cnt)
    return {
        "ops": [(OPNAME[ops[i].type], ops[i].mb) for i in range(cnt)],
        "start": list(st[:cnt]), "end": list(en[:cnt]),
        "arrive_f": list(af), "arrive_b": list(ab),
        "makespan": stats.makespan, "busy": stats.busy, "first_start": stats.first_start,
        "last_end": stats.last_end, "peak_active": stats.peak_active,
    }


def schedule_generate_interleaved(p: int, m: int, v: int, costs=(1, 1, 1), stage: int = 0) -> dict:
    """Interleaved 1F1B order of one stage holding v model chunks (no GPU
    needed): ops are (type, chunk, microbatch); arrivals are lists of v
    lists of m entries ([chunk][mb])."""
    n = 3 * v * m
    ops = (ChunkOp * n)()
    st = (ctypes.c_int64 * n)()
    en = (ctypes.c_int64 * n)()
    af = (ctypes.c_int64 * (v * m))()
    ab = (ctypes.c_int64 * (v * m))()
    stats = SchedStats()
    cnt = lib().zb_schedule_generate_interleaved(p, m, v, costs[0], costs[1], costs[2], stage, ops, st, en, n, af, ab,
                                                 ctypes.byref(stats))
    check(cnt)
    return {
        "ops": [(OPNAME[ops[i].type], ops[i].chunk, ops[i].mb) for i in range(cnt)],
        "start": list(st[:cnt]), "end": list(en[:cnt]),
        "arrive_f": [list(af[c * m:(c + 1) * m]) for c in range(v)],
        "arrive_b": [list(ab[c * m:(c + 1) * m]) for c in range(v)],
        "makespan": stats.makespan, "busy": stats.busy, "first_start": stats.first_start,
        "last_end": stats.last_end, "peak_active": stats.peak_active,
    }


def run_schedule_chunks(stages: Sequence["Stage"], ops, arrive_f, arrive_b, unit_ms: float, xs, ys, dys, dxs,
                        mode: int = EXEC_ORDERED, hi_stream=None, lo_stream=None) -> dict:
    """Replay an op list over a stage made of several model chunks
    (zb_run_schedule_chunks).  ops: (type, chunk, mb); arrive_f / arrive_b:
    [chunk][mb]; xs, ys, dys, dxs: [chunk][mb] device tensors."""
    v = len(stages)
    m = len(xs[0])
    if not all(len(a) == v for a in (arrive_f, arrive_b, xs, ys, dys, dxs)):
        raise ValueError("arrivals and tensors need one list per chunk")
    if not all(len(q) == m for q in list(arrive_f) + list(arrive_b) + list(xs) + list(ys) + list(dys) + list(dxs)):
        raise ValueError("every per-chunk list needs m entries")
    n = len(ops)
    code = {"F": OP_F, "B": OP_B, "W": OP_W, "O": OP_O}
    opa = (ChunkOp * n)(*[ChunkOp(code[t], c, j) for t, c, j in ops])
    flat = lambda L: [q for row in L for q in row]
    af = (ctypes.c_double * (v * m))(*[float(a) for a in flat(arrive_f)])
    ab = (ctypes.c_double * (v * m))(*[float(a) for a in flat(arrive_b)])
    P = lambda ts: (ctypes.c_void_p * (v * m))(*[_ptr(t) for t in flat(ts)])
    hs = (ctypes.c_void_p * v)(*[s_.handle.value for s_ in stages])
    stats = RunStats()
    op_ms = (ctypes.c_double * (2 * n))()
    hi = hi_stream.cuda_stream if hi_stream is not None else None
    lo = lo_stream.cuda_stream if lo_stream is not None else None
    check(lib().zb_run_schedule_chunks(hs, v, opa, n, m, af, ab, unit_ms, P(xs), P(ys), P(dys), P(dxs), hi, lo, mode,
                                       ctypes.byref(stats), op_ms))
    return {"window_ms": stats.window_ms, "busy_ms": stats.busy_ms, "in_window_idle": stats.in_window_idle,
            "t_first_start_ms": stats.t_first_start_ms, "t_last_end_ms": stats.t_last_end_ms,
            "wait_late_ms": stats.wait_late_ms,
            "op_ms": [(op_ms[2 * i], op_ms[2 * i + 1]) for i in range(n)]}


# ---- device side (needs torch + a GPU) -------------------------------------

def _ptr(t) -> int:
    return t.data_ptr()


def _stream_ptr(stream) -> Optional[int]:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def weight_shapes(kind: str, hidden: int, ffn: int, n_layers: int = 1, n_heads: int = 1, n_kv_heads: int = 1,
                  head_dim: int = 128) -> List[tuple]:
    if kind == "linear":
        return [(ffn, hidden)]
    if kind == "mlp":
        return [(ffn, hidden), (hidden, ffn)]
    qd, kvd = n_heads * head_dim, n_kv_heads * head_dim
    out = []
    for _ in range(n_layers):
        out += [(qd + 2 * kvd, hidden), (hidden, qd), (2 * ffn, hidden), (hidden, ffn), (hidden,), (hidden,)]
    return out


class Stage:
    """One pipeline stage on the current GPU.

    weights: device tensors in the kind's weight order (bf16, or fp32 for an
    fp32 linear stage).  The fp32 dW buffers and the workspace (stash ring +
    scratch) are allocated here with torch and handed to the library.
    """

    def __init__(self, kind: str, tokens: int, hidden: int, ffn: int, weights: Sequence, *, dtype: str = "bf16",
                 n_layers: int = 1, n_heads: int = 1, n_kv_heads: int = 1, head_dim: int = 128,
                 rms_eps: float = 1e-5, ring_slots: int = 2, device=None):
        import torch
        self.torch = torch
        self.desc = StageDesc(KIND[kind], DTYPE[dtype], n_layers, tokens, hidden, ffn,
                              n_heads, n_kv_heads, head_dim, rms_eps, ring_slots)
        self.kind = kind
        self.dtype = dtype
        L = lib()
        nw = check(L.zb_stage_num_weights(ctypes.byref(self.desc)))
        if len(weights) != nw:
            raise ValueError(f"expected {nw} weights, got {len(weights)}")
        device = device or weights[0].device
        self.device = device
        want = torch.float32 if dtype == "f32" else torch.bfloat16  # fp8 stages keep bf16 weights
        for w in weights:
            if w.dtype != want or not w.is_contiguous() or w.device != device:
                raise ValueError("weights must be contiguous device tensors of the stage dtype")
        self.weights = list(weights)
        self.dw = [torch.zeros(w.shape, dtype=torch.float32, device=device) for w in weights]
        nbytes = L.zb_stage_workspace_bytes(ctypes.byref(self.desc))
        if nbytes == 0:
            raise ZbError(EINVAL, last_error())
        self.ws = torch.empty(nbytes + 256, dtype=torch.uint8, device=device)
        off = (-self.ws.data_ptr()) % 256
        self.ws_off = off
        wp = (ctypes.c_void_p * nw)(*[_ptr(w) for w in self.weights])
        dp = (ctypes.c_void_p * nw)(*[_ptr(d) for d in self.dw])
        h = ctypes.c_void_p()
        check(L.zb_stage_create(ctypes.byref(self.desc), wp, dp, ctypes.c_void_p(self.ws.data_ptr() + off), nbytes,
                                ctypes.byref(h)))
        self.handle = h

    def __del__(self):
        h = getattr(self, "handle", None)
        if h is not None and h.value:
            try:
                self.torch.cuda.synchronize(self.device)
            except Exception:
                pass
            try:
                lib().zb_stage_destroy(h)
            except Exception:  # interpreter shutdown: module globals may already be gone
                pass
            self.handle = None

    def slot_bytes(self) -> int:
        """Bytes of one stash-ring slot (one microbatch's F and B stash):
        the workspace size's growth per added slot."""
        L = lib()
        d1, d2 = StageDesc.from_buffer_copy(self.desc), StageDesc.from_buffer_copy(self.desc)
        d1.ring_slots, d2.ring_slots = 1, 2
        return int(L.zb_stage_workspace_bytes(ctypes.byref(d2)) - L.zb_stage_workspace_bytes(ctypes.byref(d1)))

    @property
    def act_dtype(self):
        return self.torch.float32 if self.dtype == "f32" else self.torch.bfloat16

    @property
    def out_width(self) -> int:
        return self.desc.ffn if self.kind == "linear" else self.desc.hidden

    def fwd(self, mb: int, x, y=None, stream=None):
        if y is None:
            y = self.torch.empty((self.desc.tokens, self.out_width), dtype=self.act_dtype, device=self.device)
        check(lib().zb_fwd(self.handle, mb, _ptr(x), _ptr(y), _stream_ptr(stream)))
        return y

    def bwd_input(self, mb: int, dy, dx=None, stream=None):
        if dx is None:
            dx = self.torch.empty((self.desc.tokens, self.desc.hidden), dtype=self.act_dtype, device=self.device)
        check(lib().zb_bwd_input(self.handle, mb, _ptr(dy), _ptr(dx), _stream_ptr(stream)))
        return dx

    def bwd_weight(self, mb: int, stream=None):
        check(lib().zb_bwd_weight_accum(self.handle, mb, _stream_ptr(stream)))

    def bwd_weight_noalloc(self, mb: int, stream=None):
        """W for microbatch mb with its scratch in the library's fixed device
        array (zb_bwd_weight_accum_noalloc)."""
        check(lib().zb_bwd_weight_accum_noalloc(self.handle, mb, _stream_ptr(stream)))

    def bwd_weight_pair(self, mb: int, stream=None):
        """W for microbatches mb and mb + 1 in one pass (zb_bwd_weight_accum_pair)."""
        check(lib().zb_bwd_weight_accum_pair(self.handle, mb, _stream_ptr(stream)))

    def sgd_step(self, lr: float, stream=None):
        """w -= lr * dW for every weight, then zero_grad (zb_stage_sgd_step)."""
        check(lib().zb_stage_sgd_step(self.handle, lr, _stream_ptr(stream)))

    def weights_changed(self):
        """The caller wrote the weights: refresh the stage's copies of them
        (zb_stage_weights_changed)."""
        check(lib().zb_stage_weights_changed(self.handle))

    def set_lr(self, lr: float):
        """Rate of the optimizer steps the executor runs for "O" ops."""
        check(lib().zb_stage_set_lr(self.handle, lr))

    def zero_grad(self, stream=None):
        check(lib().zb_stage_zero_grad(self.handle, _stream_ptr(stream)))

    def set_debug(self, slot_tags: bool = False, serialize: bool = False, w_delay_us: int = 0, stream=None):
        """Debug aids (zb_stage_set_debug): device-side ring-slot tags,
        a device synchronization after every op, a delay before every W."""
        flags = (DEBUG_SLOT_TAGS if slot_tags else 0) | (DEBUG_SERIALIZE if serialize else 0)
        check(lib().zb_stage_set_debug(self.handle, flags, int(w_delay_us), _stream_ptr(stream)))

    def debug_report(self):
        """(mismatch count, last mismatch as a dict or None) of the slot
        tags (zb_stage_debug_report; waits for the device)."""
        info = (_i32 * 5)()
        n = lib().zb_stage_debug_report(self.handle, info)
        if n < 0:
            check(n)
        last = None
        if n:
            last = {"op": "FBW"[info[0]] if 0 <= info[0] < 3 else info[0], "mb": info[1], "slot": info[2],
                    "found": info[3], "expected": info[4]}
        return n, last

    def stash(self, mb: int, layer: int, which: int):
        """Torch view of a stashed tensor (valid until W(mb) completes)."""
        p, r, c, dt = ctypes.c_void_p(), ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
        check(lib().zb_stage_stash_tensor(self.handle, mb, layer, which, ctypes.byref(p), ctypes.byref(r),
                                          ctypes.byref(c), ctypes.byref(dt)))
        torch = self.torch
        off = p.value - self.ws.data_ptr()
        tdt, esz = {F32: (torch.float32, 4), BF16: (torch.bfloat16, 2), E4M3: (torch.uint8, 1),
                    I32: (torch.int32, 4)}[dt.value]
        nbytes = r.value * c.value * esz
        return self.ws[off:off + nbytes].view(tdt).view(r.value, c.value)

    def fp8_weight(self, i: int):
        """(codes [out][in], codes [in][out], exponent) of linear weight i of
        an fp8 stage, as torch views (uint8, uint8, int32 of one element)."""
        q, qt, e = ctypes.c_void_p(), ctypes.c_void_p(), ctypes.c_void_p()
        check(lib().zb_stage_fp8_weight(self.handle, i, ctypes.byref(q), ctypes.byref(qt), ctypes.byref(e)))
        out_, in_ = self.weights[i].shape
        base = self.ws.data_ptr()
        view = lambda p, n: self.ws[p - base:p - base + n]
        return (view(q.value, out_ * in_).view(out_, in_), view(qt.value, out_ * in_).view(in_, out_),
                view(e.value, 4).view(self.torch.int32))

    def run_schedule(self, ops, arrive_f, arrive_b, unit_ms: float, xs, ys, dys, dxs, mode: int = EXEC_ORDERED,
                     hi_stream=None, lo_stream=None):
        n = len(ops)
        m = len(xs)
        if not (len(ys) == len(dys) == len(dxs) == m and len(arrive_f) >= m and len(arrive_b) >= m):
            raise ValueError("xs, ys, dys, dxs and the arrival lists need one entry per microbatch")
        if any(j < 0 or (t != "O" and j >= m) for t, j in ops):
            raise ValueError("op microbatch outside the given per-microbatch lists")
        opa = (Op * n)(*[Op({"F": OP_F, "B": OP_B, "W": OP_W, "O": OP_O}[t], j) for t, j in ops])
        af = (ctypes.c_double * m)(*[float(a) for a in arrive_f])
        ab = (ctypes.c_double * m)(*[float(a) for a in arrive_b])
        P = lambda ts: (ctypes.c_void_p * m)(*[_ptr(t) for t in ts])
        stats = RunStats()
        op_ms = (ctypes.c_double * (2 * n))()
        hs = hi_stream.cuda_stream if hi_stream is not None else None
        ls = lo_stream.cuda_stream if lo_stream is not None else None
        check(lib().zb_stage_run_schedule(self.handle, opa, n, af, ab, unit_ms, P(xs), P(ys), P(dys), P(dxs), hs, ls,
                                          mode, ctypes.byref(stats), op_ms))
        return {"window_ms": stats.window_ms, "busy_ms": stats.busy_ms, "in_window_idle": stats.in_window_idle,
                "t_first_start_ms": stats.t_first_start_ms, "t_last_end_ms": stats.t_last_end_ms,
                "wait_late_ms": stats.wait_late_ms,
                "op_ms": [(op_ms[2 * i], op_ms[2 * i + 1]) for i in range(n)]}


def gemm(A, B, C, *, a_kmajor: bool, b_kmajor: bool, M: int, N: int, K: int, accumulate: bool = False,
         lda: int = None, ldb: int = None, ldc: int = None, stream=None):
    """C (op)= opA(A) . opB(B) through the library's GEMM kernels."""
    import torch
    dt = F32 if A.dtype == torch.float32 else BF16
    out_f32 = 1 if C.dtype == torch.float32 else 0
    lda = lda if lda is not None else A.shape[-1]
    ldb = ldb if ldb is not None else B.shape[-1]
    ldc = ldc if ldc is not None else C.shape[-1]
    check(lib().zb_gemm(dt, M, N, K, _ptr(A), lda, int(a_kmajor), _ptr(B), ldb, int(b_kmajor), _ptr(C), ldc,
                        out_f32, int(accumulate), _stream_ptr(stream)))
    return C


def quantize_e4m3(x, q=None, qt=None, stream=None):
    """Per-tensor E4M3 quantization of a bf16 matrix through the library's
    kernels: returns (q [rows][cols] uint8 or None, qt [cols][rows] or None,
    exponent int32 tensor of one element)."""
    import torch
    rows, cols = x.shape
    e = torch.zeros(1, dtype=torch.int32, device=x.device)
    part = torch.empty(512, dtype=torch.float32, device=x.device)
    check(lib().zb_quantize_e4m3(_ptr(x), rows, cols, x.stride(0), _ptr(q) if q is not None else None, cols,
                                 _ptr(qt) if qt is not None else None, rows, _ptr(e), _ptr(part),
                                 _stream_ptr(stream)))
    return q, qt, e


def gemm_fp8(A, ea, B, eb, C, stream=None):
    """C (op)= (A . B^T) * 2^(ea + eb) over E4M3 codes A [M][K], B [N][K];
    C bf16 (assigned) or fp32 (accumulated)."""
    import torch
    M, K = A.shape
    N = B.shape[0]
    out_f32 = 1 if C.dtype == torch.float32 else 0
    check(lib().zb_gemm_fp8(M, N, K, _ptr(A), A.stride(0), _ptr(ea), _ptr(B), B.stride(0), _ptr(eb), _ptr(C),
                            C.stride(0), out_f32, _stream_ptr(stream)))


def gemm_fp8_wgrad_group(As, eas, Bs, ebs, Cs, stream=None):
    """C_i += (A_i . B_i^T) * 2^(ea_i + eb_i) over E4M3 codes, fp32 C_i, in
    grouped launches (zb_gemm_fp8_wgrad_group)."""
    n = len(As)
    i32 = lambda v: (ctypes.c_int32 * n)(*v)
    i64 = lambda v: (ctypes.c_int64 * n)(*v)
    P = lambda ts: (ctypes.c_void_p * n)(*[_ptr(t) for t in ts])
    check(lib().zb_gemm_fp8_wgrad_group(n, i32([a.shape[0] for a in As]), i32([b.shape[0] for b in Bs]),
                                        i32([a.shape[1] for a in As]), P(As), i64([a.stride(0) for a in As]), P(eas),
                                        P(Bs), i64([b.stride(0) for b in Bs]), P(ebs), P(Cs),
                                        i64([c.stride(0) for c in Cs]), _stream_ptr(stream)))


def gemm_wgrad_group(As, Bs, Cs, Ms, Ns, Ks, a_kmajor=False, b_kmajor=False, stream=None):
    """C_i (fp32) += opA_i . opB_i for every i in one grouped launch
    (zb_gemm_wgrad_group); bf16 A_i, B_i with one orientation for all."""
    import torch
    n = len(As)
    if not (len(Bs) == len(Cs) == len(Ms) == len(Ns) == len(Ks) == n):
        raise ValueError("gemm_wgrad_group: list lengths differ")
    for t in list(As) + list(Bs):
        if t.dtype != torch.bfloat16:
            raise ValueError("gemm_wgrad_group: A and B are bf16")
    for t in Cs:
        if t.dtype != torch.float32:
            raise ValueError("gemm_wgrad_group: C is fp32")
    i32 = ctypes.c_int32 * n
    i64 = ctypes.c_int64 * n
    vp = ctypes.c_void_p * n
    check(lib().zb_gemm_wgrad_group(n, i32(*Ms), i32(*Ns), i32(*Ks), vp(*[a.data_ptr() for a in As]),
                                    i64(*[a.stride(0) for a in As]), int(a_kmajor),
                                    vp(*[b.data_ptr() for b in Bs]), i64(*[b.stride(0) for b in Bs]), int(b_kmajor),
                                    vp(*[c.data_ptr() for c in Cs]), i64(*[c.stride(0) for c in Cs]),
                                    _stream_ptr(stream)))
