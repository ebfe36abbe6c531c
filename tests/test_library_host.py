"""Host-side tests of libzb (no GPU): the library loads and exports every
symbol include/zb.h declares, the schedule generator matches the oracle
simulator bit for bit, and argument validation rejects bad calls before
anything is launched."""
import ctypes
import os
import re

import pytest

import split_backward_amd as zb
from oracle.schedule import simulate

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_symbols():
    with open(os.path.join(ROOT, "include", "zb.h")) as f:
        src = f.read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(zb_[a-z0-9_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    L = zb.lib()
    declared = _declared_symbols()
    assert len(declared) >= 14
    for name in declared:
        assert hasattr(L, name), name
    assert set(declared) == set(zb.EXPORTS)


def test_version_string():
    assert b"gfx950" in zb.lib().zb_version()


def _grid():
    for p in (1, 2, 3, 5, 8, 12, 16):
        for m in (1, 2, 7, 16, 33, 48):
            for kind in ("gpipe", "1f1b", "zb"):
                Ms = sorted({p, p + 1, (3 * p) // 2, 2 * p}) if kind == "zb" else [0]
                for M in Ms:
                    yield kind, p, m, M


@pytest.mark.parametrize("costs", [(1, 1, 1), (2, 3, 1)])
def test_generator_matches_oracle_bit_exact(costs):
    n = 0
    for kind, p, m, M in _grid():
        if p * m > 400 and costs != (1, 1, 1):
            continue
        ref = simulate(kind, p, m, M=M, costs=costs)
        for stage in sorted({0, p // 2, p - 1}):
            got = zb.schedule_generate(kind, p, m, M, costs, stage)
            assert got["ops"] == ref.order(stage), (kind, p, m, M, stage)
            assert got["start"] == [o.start for o in ref.ops[stage]]
            assert got["end"] == [o.end for o in ref.ops[stage]]
            assert got["arrive_f"] == ref.arrive_f[stage]
            assert got["arrive_b"] == ref.arrive_b[stage]
            assert got["makespan"] == ref.makespan
            assert got["busy"] == ref.stats[stage].busy
            assert got["peak_active"] == ref.stats[stage].peak_active
            n += 1
    assert n > 100


def test_generator_headline_stage():
    """Stage 3 of p=8, m=16: 1F1B and ZB(2p) orders and windows."""
    one = zb.schedule_generate("1f1b", 8, 16, 0, (1, 1, 1), 3)
    z16 = zb.schedule_generate("zb", 8, 16, 16, (1, 1, 1), 3)
    assert one["makespan"] == 69 and z16["makespan"] == 55
    assert (one["first_start"], one["last_end"]) == (3, 63)
    assert (z16["first_start"], z16["last_end"]) == (3, 51)
    assert z16["busy"] == z16["last_end"] - z16["first_start"]  # zero in-window idle


def test_generator_rejects_bad_arguments():
    L = zb.lib()
    assert L.zb_schedule_generate(zb.SCHED_ZB, 4, 8, 0, 1, 1, 1, 0, None, None, None, 0, None, None, None) == zb.EINVAL
    assert L.zb_schedule_generate(zb.SCHED_ZB, 4, 8, 4, 1, 1, 0, 0, None, None, None, 0, None, None, None) == zb.EINVAL
    assert L.zb_schedule_generate(zb.SCHED_1F1B, 4, 8, 0, 1, 1, 1, 4, None, None, None, 0, None, None, None) == zb.EINVAL
    ops = (zb.Op * 3)()
    assert L.zb_schedule_generate(zb.SCHED_1F1B, 4, 8, 0, 1, 1, 1, 0, ops, None, None, 3, None, None, None) == zb.EINVAL
    assert L.zb_schedule_generate(9, 4, 8, 0, 1, 1, 1, 0, None, None, None, 0, None, None, None) == zb.EINVAL
    # memory limit 1 with p = 3 still makes progress (one microbatch at a time)
    assert L.zb_schedule_generate(zb.SCHED_ZB, 3, 4, 1, 1, 1, 1, 0, None, None, None, 0, None, None, None) == 12


def _desc(**kw):
    base = dict(kind=zb.LLAMA, dtype=zb.BF16, n_layers=4, tokens=4096, hidden=4096, ffn=11008, n_heads=32,
                n_kv_heads=32, head_dim=128, rms_eps=1e-5, ring_slots=16)
    base.update(kw)
    return zb.StageDesc(*[base[f] for f, _ in zb.StageDesc._fields_])


def test_workspace_sizes_and_weight_counts():
    L = zb.lib()
    d = _desc()
    assert L.zb_stage_num_weights(ctypes.byref(d)) == 24
    ws = L.zb_stage_workspace_bytes(ctypes.byref(d))
    # 16 slots of 4 layers of stash, roughly 1.06 GB per layer per microbatch
    assert 60e9 < ws < 75e9
    lin = _desc(kind=zb.LINEAR, dtype=zb.F32, n_layers=1, tokens=128, hidden=256, ffn=256, ring_slots=2)
    assert L.zb_stage_num_weights(ctypes.byref(lin)) == 1
    assert L.zb_stage_workspace_bytes(ctypes.byref(lin)) >= 2 * (128 * 256 * 4 * 2)


def test_workspace_grows_by_one_slot_per_ring_slot():
    """The workspace is the stash ring plus fixed scratch, so its size is
    affine in ring_slots; the bench's stash figures (peak resident
    microbatches x slot bytes) rely on it."""
    L = zb.lib()
    for kw in (dict(), dict(kind=zb.MLP_GELU, n_layers=1, tokens=2048, hidden=1024, ffn=4096),
               dict(n_layers=2, hidden=8192, ffn=28672, n_heads=64, n_kv_heads=8)):
        sizes = [L.zb_stage_workspace_bytes(ctypes.byref(_desc(ring_slots=r, **kw))) for r in range(1, 6)]
        steps = {b - a for a, b in zip(sizes, sizes[1:])}
        assert len(steps) == 1, kw
        slot = steps.pop()
        d = _desc(**kw)
        T, h, f = d.tokens, d.hidden, d.ffn
        if d.kind == zb.LLAMA:
            # per layer, bf16: the F stash x, n1, q|k|v, attention output, h1,
            # n2, g|u, s and the B stash d_out, dg|du, dn2, dh1, dq|dk|dv,
            # dn1; fp32: two rms factors per token and the attention lse per
            # head and token; each tensor 256-byte aligned
            qd, qkv = d.n_heads * d.head_dim, (d.n_heads + 2 * d.n_kv_heads) * d.head_dim
            bf16 = d.n_layers * 2 * T * (8 * h + qd + 2 * qkv + 5 * f)
            f32 = d.n_layers * 4 * T * (2 + d.n_heads)
            assert bf16 + f32 <= slot < bf16 + f32 + d.n_layers * 17 * 256, kw
        else:
            # x, a, gelu(a), dy, da in bf16
            assert 2 * T * (2 * h + 3 * f) <= slot < 2 * T * (2 * h + 3 * f) + 5 * 256, kw


@pytest.mark.parametrize("bad", [dict(head_dim=64), dict(n_kv_heads=5), dict(ring_slots=0), dict(hidden=4100),
                                 dict(dtype=zb.F32), dict(tokens=0), dict(kind=7), dict(tokens=4000),
                                 dict(tokens=200)])
def test_invalid_descs_rejected(bad):
    L = zb.lib()
    d = _desc(**bad)
    assert L.zb_stage_workspace_bytes(ctypes.byref(d)) == 0
    assert L.zb_stage_num_weights(ctypes.byref(d)) == zb.EINVAL
    assert len(zb.last_error()) > 5


def test_gemm_rejects_bad_shapes_before_launch():
    L = zb.lib()
    fake = ctypes.c_void_p(0x1000)
    # K not a multiple of 8 (bf16 vector loads)
    assert L.zb_gemm(zb.BF16, 64, 64, 12, fake, 16, 1, fake, 16, 1, fake, 64, 0, 0, None) == zb.EINVAL
    # leading dimension smaller than the row
    assert L.zb_gemm(zb.BF16, 64, 64, 64, fake, 32, 1, fake, 64, 1, fake, 64, 0, 0, None) == zb.EINVAL
    # bf16 output cannot accumulate
    assert L.zb_gemm(zb.BF16, 64, 64, 64, fake, 64, 1, fake, 64, 1, fake, 64, 0, 1, None) == zb.EINVAL
    # empty shape
    assert L.zb_gemm(zb.BF16, 0, 64, 64, fake, 64, 1, fake, 64, 1, fake, 64, 0, 0, None) == zb.EINVAL
    assert L.zb_gemm(zb.F32, 8, 8, 8, None, 8, 1, fake, 8, 1, fake, 8, 1, 0, None) == zb.EINVAL


def test_compute_calls_reject_null_stage():
    L = zb.lib()
    assert L.zb_fwd(None, 0, ctypes.c_void_p(16), ctypes.c_void_p(16), None) == zb.EINVAL
    assert L.zb_bwd_input(None, 0, ctypes.c_void_p(16), ctypes.c_void_p(16), None) == zb.EINVAL
    assert L.zb_bwd_weight_accum(None, 0, None) == zb.EINVAL
    assert L.zb_stage_zero_grad(None, None) == zb.EINVAL


@pytest.mark.parametrize("kind", ["zb", "1f1b"])
@pytest.mark.parametrize("p,m,M,costs,c_opt,n", [(8, 16, 16, (1, 1, 1), 1, 3), (4, 8, 8, (2, 3, 2), 2, 2),
                                                (8, 16, 8, (63, 84, 63), 1, 2), (4, 6, 5, (1, 2, 1), 3, 3),
                                                (2, 1, 1, (1, 1, 1), 1, 2), (1, 4, 1, (2, 3, 1), 1, 3),
                                                (4, 1, 1, (1, 2, 3), 2, 2)])
def test_iteration_generator_matches_oracle_bit_exact(kind, p, m, M, costs, c_opt, n):
    from oracle.schedule import simulate_iterations
    M = M if kind == "zb" else 0
    ref = simulate_iterations(p, m, M, costs, n, c_opt, kind=kind)
    for stage in range(p):
        g = zb.schedule_generate_iters(p, m, M, costs, c_opt, n, stage, kind=kind)
        assert g["ops"] == ref.order(stage)
        assert g["start"] == [o.start for o in ref.ops[stage]]
        assert g["end"] == [o.end for o in ref.ops[stage]]
        assert g["arrive_f"] == ref.arrive_f[stage]
        assert g["arrive_b"] == ref.arrive_b[stage]
        assert g["makespan"] == ref.makespan
        assert g["peak_active"] == ref.stats[stage].peak_active
        assert g["busy"] == ref.stats[stage].busy


def test_iteration_generator_rejects_bad_arguments():
    for bad in (dict(n_iter=0), dict(c_opt=0), dict(mem_limit=0), dict(stage=4), dict(kind="gpipe")):
        kw = dict(p=4, m=8, mem_limit=8, costs=(1, 1, 1), c_opt=1, n_iter=2, stage=0)
        kw.update(bad)
        with pytest.raises(zb.ZbError):
            zb.schedule_generate_iters(**kw)


def _run_args(n=2, af=(0.0, 0.0), ab=(0.0, 0.0), unit_ms=0.1):
    ops = (zb.Op * n)(*([zb.Op(zb.OP_F, 0), zb.Op(zb.OP_B, 0)][:n]))
    dbl = lambda v: (ctypes.c_double * len(v))(*v)
    return ops, n, dbl(af), dbl(ab), unit_ms


@pytest.mark.parametrize("unit_ms,af,msg", [(float("inf"), (0.0, 0.0), "unit_ms"), (float("nan"), (0.0, 0.0), "unit_ms"),
                                            (-1.0, (0.0, 0.0), "unit_ms"), (1e12, (1.0, 0.0), "30 s"),
                                            (100.0, (301.0, 0.0), "30 s"), (float("inf"), (0.0, 0.0), "unit_ms")])
def test_executor_rejects_unbounded_waits_before_any_work(unit_ms, af, msg):
    """Every arrival wait must end within the wait kernel's 30 s cap: a unit
    that is not finite, or an arrival x unit beyond 30 s, is rejected while
    checking the arguments, before the stage is looked at (so no GPU is
    needed to see it)."""
    L = zb.lib()
    ops, n, a_f, a_b, u = _run_args(af=af, unit_ms=unit_ms)
    rc = L.zb_stage_run_schedule(None, ops, n, a_f, a_b, u, None, None, None, None, None, None, zb.EXEC_ORDERED,
                                 None, None)
    assert rc == zb.EINVAL
    assert msg in zb.last_error()


def test_executor_bounded_waits_pass_argument_checks():
    """A finite unit with every arrival within 30 s gets past the time checks
    (and then fails on the NULL stage)."""
    L = zb.lib()
    ops, n, a_f, a_b, u = _run_args(af=(299.0, 0.0), unit_ms=100.0)
    rc = L.zb_stage_run_schedule(None, ops, n, a_f, a_b, u, None, None, None, None, None, None, zb.EXEC_ORDERED,
                                 None, None)
    assert rc == zb.EINVAL
    assert "bad argument" in zb.last_error()


@pytest.mark.parametrize("costs", [(1, 1, 1), (2, 3, 1), (1, 2, 0)])
def test_interleaved_generator_matches_oracle_bit_exact(costs):
    from oracle.schedule import simulate_interleaved
    n = 0
    for p in (1, 2, 3, 4, 8):
        for v in (1, 2, 3):
            for m in sorted({p, 2 * p, 3 * p, 16 if 16 % p == 0 else p}):
                ref = simulate_interleaved(p, m, v, costs)
                for stage in sorted({0, p // 2, p - 1}):
                    got = zb.schedule_generate_interleaved(p, m, v, costs, stage)
                    assert got["ops"] == ref.order(stage), (p, m, v, stage)
                    assert got["start"] == [o.start for o in ref.ops[stage]]
                    assert got["end"] == [o.end for o in ref.ops[stage]]
                    assert got["arrive_f"] == ref.arrive_f[stage]
                    assert got["arrive_b"] == ref.arrive_b[stage]
                    assert got["makespan"] == ref.makespan
                    assert got["busy"] == ref.stats[stage].busy
                    assert got["peak_active"] == ref.stats[stage].peak_active
                    n += 1
    assert n > 60


def test_interleaved_generator_rejects_bad_arguments():
    L = zb.lib()
    for args in ((8, 12, 2, 1, 1, 1, 0), (8, 16, 0, 1, 1, 1, 0), (8, 16, 2, 0, 1, 1, 0), (8, 16, 2, 1, 1, 1, 8)):
        assert L.zb_schedule_generate_interleaved(*args, None, None, None, 0, None, None, None) == zb.EINVAL
    ops = (zb.ChunkOp * 10)()
    assert L.zb_schedule_generate_interleaved(2, 2, 2, 1, 1, 1, 0, ops, None, None, 10, None, None, None) == zb.EINVAL


def test_chunk_executor_rejects_bad_op_lists_before_any_work():
    L = zb.lib()
    ops = (zb.ChunkOp * 2)(zb.ChunkOp(zb.OP_F, 0, 0), zb.ChunkOp(zb.OP_B, 0, 0))
    d = lambda v: (ctypes.c_double * len(v))(*v)
    rc = L.zb_run_schedule_chunks(None, 2, ops, 2, 1, d([0.0, 0.0]), d([0.0, 0.0]), float("inf"), None, None, None,
                                  None, None, None, zb.EXEC_ORDERED, None, None)
    assert rc == zb.EINVAL and "unit_ms" in zb.last_error()
    rc = L.zb_run_schedule_chunks(None, 0, ops, 2, 1, d([0.0, 0.0]), d([0.0, 0.0]), 1.0, None, None, None,
                                  None, None, None, zb.EXEC_ORDERED, None, None)
    assert rc == zb.EINVAL
