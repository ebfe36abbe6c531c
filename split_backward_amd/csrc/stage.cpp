// The stage object behind the C ABI: stash ring, per-microbatch state
// machine, and the F / B / W passes of each stage kind.
//
// The pass structure follows "Zero-Bubble Pipeline Parallelism Guide for
// LLMs": F keeps what the backward needs (the listing's saved inputs), B
// computes the input gradient and keeps the output gradients (saved grad
// outputs), W consumes both and adds the weight gradient into a fixed fp32
// buffer, then releases the microbatch's activations ("Memory Management &
// Activation Rollback").  The stash lives in a ring of R slots in the caller's
// workspace; microbatch mb uses slot mb % R, which is valid because F and W
// are both issued in ascending microbatch order, so the live microbatches
// always form a contiguous range.
#include <algorithm>
#include <cmath>
#include <cstring>
#include <string>
#include <vector>

#include "common.h"
#include "stage.h"

using namespace zb;

namespace {

constexpr size_t ALIGN = 256;
size_t align_up(size_t v) { return (v + ALIGN - 1) / ALIGN * ALIGN; }

size_t elem_bytes(int dtype) { return dtype == ZB_F32 || dtype == ZB_I32 ? 4 : dtype == ZB_E4M3 ? 1 : 2; }

bool valid_desc(const zb_stage_desc* d, std::string& why) {
    if (!d) { why = "desc is NULL"; return false; }
    if (d->tokens < 1 || d->hidden < 1 || d->ffn < 1 || d->ring_slots < 1) { why = "tokens, hidden, ffn, ring_slots must be >= 1"; return false; }
    if (d->dtype != ZB_F32 && d->dtype != ZB_BF16 && d->dtype != ZB_FP8) { why = "dtype must be ZB_F32, ZB_BF16 or ZB_FP8"; return false; }
    if (d->dtype == ZB_FP8 && d->kind != ZB_LLAMA) { why = "ZB_FP8 is a Llama stage dtype"; return false; }
    if (d->dtype == ZB_FP8 && (d->hidden % 128 || d->ffn % 128)) { why = "ZB_FP8 needs hidden and ffn multiples of 128"; return false; }
    if (d->kind == ZB_LINEAR) {
        if (d->dtype == ZB_BF16 && (d->hidden % 8 || d->ffn % 8)) { why = "bf16 linear needs hidden, ffn multiples of 8"; return false; }
        return true;
    }
    if (d->dtype == ZB_F32) { why = "only the linear kind supports fp32"; return false; }
    if (d->hidden % 8 || d->ffn % 8) { why = "hidden and ffn must be multiples of 8"; return false; }
    if (d->kind == ZB_MLP_GELU) return true;
    if (d->kind != ZB_LLAMA) { why = "unknown kind"; return false; }
    if (d->n_layers < 1 || d->n_heads < 1 || d->n_kv_heads < 1 || d->n_heads % d->n_kv_heads) { why = "bad head counts"; return false; }
    if (d->head_dim != 128) { why = "head_dim must be 128"; return false; }
    if (d->hidden > 8192) { why = "hidden must be <= 8192"; return false; }
    if (!(d->rms_eps > 0.f)) { why = "rms_eps must be > 0"; return false; }
    if (d->tokens % 128) { why = "the Llama stage's attention needs tokens to be a multiple of 128"; return false; }
    return true;
}

}  // namespace

// ----------------------------------------------------------------- layout --

void Layout::build(const zb_stage_desc& d) {
    const size_t T = d.tokens, H = d.hidden, F = d.ffn;
    off.clear();
    slot_bytes = 0;
    auto add = [&](int layer, int which, int rows, int cols, int dtype) {
        Tensor t;
        t.layer = layer; t.which = which; t.rows = rows; t.cols = cols; t.dtype = dtype;
        t.offset = slot_bytes;
        slot_bytes += align_up((size_t)rows * cols * elem_bytes(dtype));
        off.push_back(t);
    };
    if (d.kind == ZB_LINEAR) {
        add(0, LIN_X, T, H, d.dtype);
        add(0, LIN_DY, T, F, d.dtype);
    } else if (d.kind == ZB_MLP_GELU) {
        add(0, MLP_X, T, H, ZB_BF16);
        add(0, MLP_A, T, F, ZB_BF16);
        add(0, MLP_H, T, F, ZB_BF16);
        add(0, MLP_DY, T, H, ZB_BF16);
        add(0, MLP_DA, T, F, ZB_BF16);
    } else if (d.dtype == ZB_FP8) {
        const int QD = d.n_heads * d.head_dim, KVD = d.n_kv_heads * d.head_dim, QKV = QD + 2 * KVD;
        for (int l = 0; l < d.n_layers; ++l) {
            add(l, L_X, T, H, ZB_BF16);
            add(l, L_R1, T, 1, ZB_F32);
            add(l, L_QKV, T, QKV, ZB_BF16);
            add(l, L_A, T, QD, ZB_BF16);
            add(l, L_LSE, d.n_heads, T, ZB_F32);
            add(l, L_H1, T, H, ZB_BF16);
            add(l, L_R2, T, 1, ZB_F32);
            add(l, L_GU, T, 2 * F, ZB_BF16);
            add(l, L_DN2, T, H, ZB_BF16);
            add(l, L_DN1, T, H, ZB_BF16);
            add(l, L_N1T, H, T, ZB_E4M3);
            add(l, L_AT, QD, T, ZB_E4M3);
            add(l, L_N2T, H, T, ZB_E4M3);
            add(l, L_ST, F, T, ZB_E4M3);
            add(l, L_DOUTT, H, T, ZB_E4M3);
            add(l, L_DGUT, 2 * F, T, ZB_E4M3);
            add(l, L_DH1T, H, T, ZB_E4M3);
            add(l, L_DQKVT, QKV, T, ZB_E4M3);
            add(l, L_QEXP, 1, NQ8, ZB_I32);
        }
    } else {
        const int QD = d.n_heads * d.head_dim, KVD = d.n_kv_heads * d.head_dim;
        for (int l = 0; l < d.n_layers; ++l) {
            add(l, L_X, T, H, ZB_BF16);
            add(l, L_R1, T, 1, ZB_F32);
            add(l, L_N1, T, H, ZB_BF16);
            add(l, L_QKV, T, QD + 2 * KVD, ZB_BF16);
            add(l, L_A, T, QD, ZB_BF16);
            add(l, L_LSE, d.n_heads, T, ZB_F32);
            add(l, L_H1, T, H, ZB_BF16);
            add(l, L_R2, T, 1, ZB_F32);
            add(l, L_N2, T, H, ZB_BF16);
            add(l, L_GU, T, 2 * F, ZB_BF16);
            add(l, L_S, T, F, ZB_BF16);
            add(l, L_DOUT, T, H, ZB_BF16);
            add(l, L_DGU, T, 2 * F, ZB_BF16);
            add(l, L_DN2, T, H, ZB_BF16);
            add(l, L_DH1, T, H, ZB_BF16);
            add(l, L_DQKV, T, QD + 2 * KVD, ZB_BF16);
            add(l, L_DN1, T, H, ZB_BF16);
        }
    }
    // per-pass scratch (not per slot)
    scratch_b = 0;
    scratch_w = 0;
    if (d.kind == ZB_LLAMA) {
        const size_t QD = (size_t)d.n_heads * d.head_dim;
        // da + delta + the attention backward's scratch (dS^T, and the dk/dv
        // partials of split query-head groups)
        scratch_b = align_up(T * QD * 2) + align_up((size_t)d.n_heads * T * 4) +
                    align_up(attn_bwd_scratch_bytes(d.tokens, d.n_heads, d.n_kv_heads));
        scratch_w = align_up(rmsnorm_dgamma_scratch_floats(d.tokens, d.hidden) * 4);
    }
    scratch_f = 0;
    if (d.kind == ZB_MLP_GELU && d.dtype == ZB_BF16) {
        // split-K partial sums of the products whose tiles would fill little
        // of the chip (the pass code asks gemm_splitk_factor the same), one
        // set per pass: F's fc1 [T, ffn] (K = hidden) and fc2 [T, hidden]
        // (K = ffn), B's products of the same shapes
        auto need = [&](int N, int K, int epi) {
            GemmDesc g{};
            g.M = d.tokens;
            g.N = N;
            g.K = K;
            g.a_kmajor = 1;
            g.epi = epi;
            return gemm_splitk_scratch_bytes(g.M, g.N, gemm_splitk_factor(g));
        };
        scratch_f = align_up(std::max(need(d.ffn, d.hidden, EPI_GELU_FWD), need(d.hidden, d.ffn, EPI_STORE)));
        scratch_b = align_up(std::max(need(d.ffn, d.hidden, EPI_GELU_BWD), need(d.hidden, d.ffn, EPI_STORE)));
    }
    w8_bytes = 0;
    w8_q.clear();
    w8_qt.clear();
    w8_e.clear();
    if (d.kind == ZB_LLAMA && d.dtype == ZB_FP8) {
        const size_t QD = (size_t)d.n_heads * d.head_dim, QKV = QD + 2 * (size_t)d.n_kv_heads * d.head_dim;
        // partial maxima: the amax pass's, T of an RMSNorm, 4 per workgroup
        // of a SwiGLU product (at most ceil(T/128) x ceil(F/128) half-height
        // tiles) or one per storing wave of the attention kernels, then the
        // reduced value
        amax_cap = std::max({(size_t)AMAX_PARTS, T, ((T + 127) / 128) * ((F + 127) / 128) * 4,
                             (size_t)attn_amax_parts((int)T, d.n_heads, d.n_kv_heads)});
        // F: one bf16 activation (n1, n2 or s), its row-major codes, amax partials
        f_act = 0;
        f_q = align_up(T * std::max(H, F) * 2);
        f_part = f_q + align_up(T * std::max({H, QD, F}));
        scratch_f = f_part + align_up((amax_cap + 1) * 4);
        // B: after the bf16 stage's scratch, dg|du, dh1, dq|dk|dv, two
        // ping-pong output gradients, row-major codes, amax partials
        b_dgu = scratch_b;
        b_dh1 = b_dgu + align_up(T * 2 * F * 2);
        b_dqkv = b_dh1 + align_up(T * H * 2);
        b_dout[0] = b_dqkv + align_up(T * QKV * 2);
        b_dout[1] = b_dout[0] + align_up(T * H * 2);
        b_q = b_dout[1] + align_up(T * H * 2);
        b_part = b_q + align_up(T * std::max({2 * F, QKV, H}));
        scratch_b = b_part + align_up((amax_cap + 1) * 4);
        // E4M3 copies [out][in] and [in][out] of every linear weight, one exponent each
        const int nw = 6 * d.n_layers;
        w8_q.assign(nw, 0);
        w8_qt.assign(nw, 0);
        w8_e.assign(nw, 0);
        for (int i = 0; i < nw; ++i) {
            if (i % 6 >= 4) continue;  // RMSNorm gains stay bf16
            const size_t n = weight_elems(d, i);
            w8_q[i] = w8_bytes;
            w8_qt[i] = w8_bytes + align_up(n);
            w8_e[i] = w8_qt[i] + align_up(n);
            w8_bytes = w8_e[i] + ALIGN;
        }
    }
    wt_bytes = 0;
    wt_off.clear();
    if (d.kind == ZB_LLAMA && d.dtype == ZB_BF16) {
        const int nw = 6 * d.n_layers;
        wt_off.assign(nw, 0);
        for (int i = 0; i < nw; ++i) {
            if (i % 6 >= 4) continue;  // RMSNorm gains
            wt_off[i] = wt_bytes;
            wt_bytes += align_up(weight_elems(d, i) * 2);
        }
    }
    stamps_bytes = align_up(sizeof(uint64_t) * (3 * (size_t)MAX_RUN_OPS + 8));
    // debug area: the delay stamp (8 bytes), the mismatch record, one tag per slot
    debug_bytes = align_up(8 + 4 * (size_t)DEBUG_REC + 4 * (size_t)d.ring_slots);
    ring_bytes = slot_bytes * d.ring_slots;
    total = ring_bytes + scratch_b + scratch_w + scratch_f + w8_bytes + wt_bytes + stamps_bytes + debug_bytes;
}

const Layout::Tensor* Layout::find(int layer, int which) const {
    for (const auto& t : off)
        if (t.layer == layer && t.which == which) return &t;
    return nullptr;
}

// ----------------------------------------------------------------- stage ---

zb_stage::~zb_stage() {
    for (auto& s : slots) {
        if (s.evF) (void)hipEventDestroy(s.evF);
        if (s.evB) (void)hipEventDestroy(s.evB);
        if (s.evW) (void)hipEventDestroy(s.evW);
    }
    for (auto& e : chain) if (e) (void)hipEventDestroy(e);
}

void* zb_stage::slot_tensor(int mb, int layer, int which) const {
    const Layout::Tensor* t = lay.find(layer, which);
    if (!t) return nullptr;
    return ws + (size_t)(mb % desc.ring_slots) * lay.slot_bytes + t->offset;
}

// Make `s` wait for the last op of kind k (scratch of that pass is shared),
// and for `dep` (the microbatch's previous op) if it was recorded.
int32_t zb_stage::order_after(int k, hipEvent_t dep, bool dep_valid, hipStream_t s) {
    if (chain_valid[k]) ZB_HIP(hipStreamWaitEvent(s, chain[k], 0));
    if (dep_valid) ZB_HIP(hipStreamWaitEvent(s, dep, 0));
    return ZB_OK;
}

int32_t zb_stage::wait_deps(int type, int mb, hipStream_t s) {
    if (mb < 0) return ZB_OK;
    const Slot& sl = slots[mb % desc.ring_slots];
    switch (type) {
        case ZB_OP_F:
            if (sl.mb >= 0 && !sl.w_issued) return ZB_OK;  // zb_fwd reports the full ring
            return order_after(PASS_F, sl.evW, sl.w_event_valid, s);
        case ZB_OP_B:
            if (sl.mb != mb || sl.b_issued) return ZB_OK;
            return order_after(PASS_B, sl.evF, true, s);
        case ZB_OP_W:
            if (sl.mb != mb || !sl.b_issued || sl.w_issued) return ZB_OK;
            return order_after(PASS_W, sl.evB, true, s);
        case ZB_OP_O:
            return order_after(PASS_W, nullptr, false, s);
        default:
            return ZB_OK;
    }
}

int32_t zb_stage::tag(int op, int mb, int expect, int set, hipStream_t s) {
    if (!(debug_flags & ZB_DEBUG_SLOT_TAGS)) return ZB_OK;
    return slot_tag(tags, dbg_rec, mb % desc.ring_slots, op, mb, expect, set, s);
}

int32_t zb_stage::delay_w(hipStream_t s) {
    if (w_delay_us <= 0) return ZB_OK;
    int32_t rc = stamp_now(dbg_t0, s);
    if (rc) return rc;
    return wait_until(dbg_t0, wall_clock_hz() / 1000000ull * (uint64_t)w_delay_us, nullptr, s);
}

int32_t zb_stage::serialize() {
    if (!(debug_flags & ZB_DEBUG_SERIALIZE)) return ZB_OK;
    ZB_HIP(hipDeviceSynchronize());
    ZB_HIP(hipGetLastError());
    return ZB_OK;
}

int32_t zb_stage::finish(int k, hipEvent_t ev, hipStream_t s) {
    ZB_HIP(hipEventRecord(ev, s));
    ZB_HIP(hipEventRecord(chain[k], s));
    chain_valid[k] = true;
    return ZB_OK;
}

// ------------------------------------------------------------- C ABI -------

extern "C" int32_t zb_stage_num_weights(const zb_stage_desc* d) {
    std::string why;
    if (!valid_desc(d, why)) return fail(ZB_EINVAL, why);
    if (d->kind == ZB_LINEAR) return 1;
    if (d->kind == ZB_MLP_GELU) return 2;
    return 6 * d->n_layers;
}

extern "C" size_t zb_stage_workspace_bytes(const zb_stage_desc* d) {
    std::string why;
    if (!valid_desc(d, why)) {
        set_error(why);
        return 0;
    }
    Layout l;
    l.build(*d);
    return l.total;
}

extern "C" int32_t zb_stage_create(const zb_stage_desc* d, void* const* weights, float* const* dw, void* workspace,
                                   size_t ws_bytes, zb_stage** out) {
    std::string why;
    if (!out) return fail(ZB_EINVAL, "out is NULL");
    *out = nullptr;
    if (!valid_desc(d, why)) return fail(ZB_EINVAL, why);
    if (!weights || !dw || !workspace) return fail(ZB_EINVAL, "weights, dw and workspace must be non-NULL");
    if (reinterpret_cast<uintptr_t>(workspace) % ALIGN) return fail(ZB_EINVAL, "workspace must be 256-byte aligned");
    const int nw = zb_stage_num_weights(d);
    for (int i = 0; i < nw; ++i)
        if (!weights[i] || !dw[i]) return fail(ZB_EINVAL, "NULL weight or dW pointer " + std::to_string(i));
    auto st = new zb_stage();
    st->desc = *d;
    if (hipGetDevice(&st->device) != hipSuccess) st->device = 0;
    st->lay.build(*d);
    if (ws_bytes < st->lay.total) {
        const size_t need = st->lay.total;
        delete st;
        return fail(ZB_ENOMEM, "workspace too small: need " + std::to_string(need) + " bytes");
    }
    st->w.assign(weights, weights + nw);
    st->dw.assign(dw, dw + nw);
    st->ws = static_cast<char*>(workspace);
    st->scratch_b = st->ws + st->lay.ring_bytes;
    st->scratch_w = st->scratch_b + st->lay.scratch_b;
    st->scratch_f = st->scratch_w + st->lay.scratch_w;
    st->w8 = st->scratch_f + st->lay.scratch_f;
    st->wt = st->w8 + st->lay.w8_bytes;
    st->stamps = reinterpret_cast<uint64_t*>(st->wt + st->lay.wt_bytes);
    char* dbg = reinterpret_cast<char*>(st->stamps) + st->lay.stamps_bytes;
    st->dbg_t0 = reinterpret_cast<uint64_t*>(dbg);
    st->dbg_rec = reinterpret_cast<int32_t*>(dbg + 8);
    st->tags = st->dbg_rec + DEBUG_REC;
    st->slots.resize(d->ring_slots);
    auto mk = [&](hipEvent_t* e) { return hipEventCreateWithFlags(e, hipEventDisableTiming); };
    for (auto& s : st->slots) {
        if (mk(&s.evF) != hipSuccess || mk(&s.evB) != hipSuccess || mk(&s.evW) != hipSuccess) {
            delete st;
            return fail(ZB_EHIP, "hipEventCreate failed");
        }
    }
    for (auto& e : st->chain)
        if (mk(&e) != hipSuccess) {
            delete st;
            return fail(ZB_EHIP, "hipEventCreate failed");
        }
    *out = st;
    return ZB_OK;
}

extern "C" void zb_stage_destroy(zb_stage* st) { delete st; }

extern "C" int32_t zb_fwd(zb_stage* st, int32_t mb, const void* x, void* y, void* stream) {
    if (!st || !x || !y || mb < 0) return fail(ZB_EINVAL, "zb_fwd: bad argument");
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (mb != st->next_f) return fail(ZB_ESTATE, "zb_fwd: F must be issued in ascending microbatch order; expected mb " + std::to_string(st->next_f));
    Slot& sl = st->slots[mb % st->desc.ring_slots];
    if (sl.mb >= 0 && !sl.w_issued)
        return fail(ZB_ERING_FULL, "zb_fwd: ring slot still holds microbatch " + std::to_string(sl.mb) + " (its W has not been issued)");
    int32_t rc = st->order_after(PASS_F, sl.evW, sl.w_event_valid, s);
    if (rc) return rc;
    if ((rc = st->tag(ZB_OP_F, mb, TAG_FREE, TAG_KEEP, s))) return rc;
    rc = run_forward(*st, mb, x, y, s);
    if (rc) return rc;
    if ((rc = st->tag(ZB_OP_F, mb, TAG_ANY, 4 * mb + 1, s))) return rc;
    sl.mb = mb;
    sl.b_issued = sl.w_issued = false;
    rc = st->finish(PASS_F, sl.evF, s);
    if (rc) return rc;
    ++st->next_f;
    return st->serialize();
}

extern "C" int32_t zb_bwd_input(zb_stage* st, int32_t mb, const void* dy, void* dx, void* stream) {
    if (!st || !dy || !dx || mb < 0) return fail(ZB_EINVAL, "zb_bwd_input: bad argument");
    hipStream_t s = static_cast<hipStream_t>(stream);
    Slot& sl = st->slots[mb % st->desc.ring_slots];
    if (sl.mb != mb || sl.b_issued) return fail(ZB_ESTATE, "zb_bwd_input: needs F(mb) issued and B(mb) not yet issued");
    int32_t rc = st->order_after(PASS_B, sl.evF, true, s);
    if (rc) return rc;
    if ((rc = st->tag(ZB_OP_B, mb, 4 * mb + 1, TAG_KEEP, s))) return rc;
    rc = run_backward_input(*st, mb, dy, dx, s);
    if (rc) return rc;
    if ((rc = st->tag(ZB_OP_B, mb, TAG_ANY, 4 * mb + 2, s))) return rc;
    sl.b_issued = true;
    if ((rc = st->finish(PASS_B, sl.evB, s))) return rc;
    return st->serialize();
}

extern "C" int32_t zb_bwd_weight_accum(zb_stage* st, int32_t mb, void* stream) {
    if (!st || mb < 0) return fail(ZB_EINVAL, "zb_bwd_weight_accum: bad argument");
    return bwd_weight_accum(st, mb, static_cast<hipStream_t>(stream), nullptr);
}

int32_t zb::bwd_weight_accum(zb_stage* st, int mb, hipStream_t s, float* dg_part) {
    Slot& sl = st->slots[mb % st->desc.ring_slots];
    if (sl.mb != mb || !sl.b_issued || sl.w_issued) return fail(ZB_ESTATE, "zb_bwd_weight_accum: needs B(mb) issued and W(mb) not yet issued");
    if (mb != st->next_w) return fail(ZB_ESTATE, "zb_bwd_weight_accum: W must be issued in ascending microbatch order; expected mb " + std::to_string(st->next_w));
    int32_t rc = st->order_after(PASS_W, sl.evB, true, s);
    if (rc) return rc;
    if ((rc = st->delay_w(s))) return rc;
    if ((rc = st->tag(ZB_OP_W, mb, 4 * mb + 2, TAG_KEEP, s))) return rc;
    rc = run_backward_weight(*st, mb, s, dg_part);
    if (rc) return rc;
    if ((rc = st->tag(ZB_OP_W, mb, TAG_ANY, 4 * mb + 3, s))) return rc;
    sl.w_issued = true;
    sl.w_event_valid = true;
    ++st->next_w;
    if ((rc = st->finish(PASS_W, sl.evW, s))) return rc;
    return st->serialize();
}

extern "C" int32_t zb_bwd_weight_accum_pair(zb_stage* st, int32_t mb, void* stream) {
    if (!st || mb < 0) return fail(ZB_EINVAL, "zb_bwd_weight_accum_pair: bad argument");
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int R = st->desc.ring_slots;
    if (R < 2) return fail(ZB_ESTATE, "zb_bwd_weight_accum_pair: a ring of one slot never holds two microbatches");
    Slot& s0 = st->slots[mb % R];
    Slot& s1 = st->slots[(mb + 1) % R];
    for (const Slot* sl : {&s0, &s1})
        if (sl->mb < 0 || !sl->b_issued || sl->w_issued)
            return fail(ZB_ESTATE, "zb_bwd_weight_accum_pair: needs B issued and W not yet issued for mb and mb + 1");
    if (s0.mb != mb || s1.mb != mb + 1)
        return fail(ZB_ESTATE, "zb_bwd_weight_accum_pair: mb and mb + 1 must both be resident");
    if (mb != st->next_w) return fail(ZB_ESTATE, "zb_bwd_weight_accum_pair: W must be issued in ascending microbatch order; expected mb " + std::to_string(st->next_w));
    int32_t rc = st->order_after(PASS_W, s0.evB, true, s);
    if (rc) return rc;
    ZB_HIP(hipStreamWaitEvent(s, s1.evB, 0));
    if ((rc = st->delay_w(s))) return rc;
    for (int j : {mb, mb + 1})
        if ((rc = st->tag(ZB_OP_W, j, 4 * j + 2, TAG_KEEP, s))) return rc;
    rc = run_backward_weight_pair(*st, mb, s);
    if (rc) return rc;
    for (int j : {mb, mb + 1})
        if ((rc = st->tag(ZB_OP_W, j, TAG_ANY, 4 * j + 3, s))) return rc;
    for (Slot* sl : {&s0, &s1}) {
        sl->w_issued = true;
        sl->w_event_valid = true;
    }
    st->next_w += 2;
    ZB_HIP(hipEventRecord(s1.evW, s));
    if ((rc = st->finish(PASS_W, s0.evW, s))) return rc;
    return st->serialize();
}

extern "C" int32_t zb_stage_zero_grad(zb_stage* st, void* stream) {
    if (!st) return fail(ZB_EINVAL, "zb_stage_zero_grad: NULL stage");
    hipStream_t s = static_cast<hipStream_t>(stream);
    for (auto& sl : st->slots)
        if (sl.mb >= 0 && !sl.w_issued) return fail(ZB_ESTATE, "zb_stage_zero_grad: microbatch " + std::to_string(sl.mb) + " still in flight");
    if (st->chain_valid[PASS_W]) ZB_HIP(hipStreamWaitEvent(s, st->chain[PASS_W], 0));
    const zb_stage_desc& d = st->desc;
    const int nw = zb_stage_num_weights(&d);
    for (int i = 0; i < nw; ++i) {
        const size_t n = weight_elems(d, i);
        int32_t rc = fill_f32(st->dw[i], n, 0.f, s);
        if (rc) return rc;
    }
    ZB_HIP(hipEventRecord(st->chain[PASS_W], s));
    st->chain_valid[PASS_W] = true;
    for (auto& sl : st->slots) sl.mb = -1;
    st->next_f = st->next_w = 0;
    return ZB_OK;
}

extern "C" int32_t zb_stage_sgd_step(zb_stage* st, float lr, void* stream) {
    if (!st || !std::isfinite(lr)) return fail(ZB_EINVAL, "zb_stage_sgd_step: bad argument");
    hipStream_t s = static_cast<hipStream_t>(stream);
    for (auto& sl : st->slots)
        if (sl.mb >= 0 && !sl.w_issued) return fail(ZB_ESTATE, "zb_stage_sgd_step: microbatch " + std::to_string(sl.mb) + " still in flight");
    if (st->chain_valid[PASS_W]) ZB_HIP(hipStreamWaitEvent(s, st->chain[PASS_W], 0));
    const zb_stage_desc& d = st->desc;
    const int nw = zb_stage_num_weights(&d);
    if (d.dtype == ZB_F32) {  // the fp32 linear stage: per weight, then the clearing fill
        for (int i = 0; i < nw; ++i) {
            const int32_t rc = sgd_step_f32(static_cast<float*>(st->w[i]), st->dw[i], weight_elems(d, i), lr, s);
            if (rc) return rc;
        }
        const int32_t rc = zb_stage_zero_grad(st, stream);
        if (rc) return rc;
        for (int k : {PASS_F, PASS_B}) {  // the next F reads the updated weights
            ZB_HIP(hipEventRecord(st->chain[k], s));
            st->chain_valid[k] = true;
        }
        return ZB_OK;
    }
    // bf16: every weight in grouped launches that also clear dW
    for (int i0 = 0; i0 < nw; i0 += SGD_GROUP_MAX) {
        SgdGroup g{};
        g.lr = lr;
        g.n = std::min(SGD_GROUP_MAX, nw - i0);
        for (int k = 0; k < g.n; ++k) {
            const size_t n = weight_elems(d, i0 + k);
            if (n % 4) return fail(ZB_EINVAL, "zb_stage_sgd_step: weight size not divisible by 4");
            g.seg[k] = SgdSeg{st->w[i0 + k], st->dw[i0 + k], n / 4};
        }
        const int32_t rc = sgd_step_group_bf16(g, s);
        if (rc) return rc;
    }
    st->w8_dirty = true;  // ZB_FP8: the next F re-quantizes the updated weights
    st->wt_dirty = true;  // bf16 Llama: the next B re-transposes them
    // the same reset as zb_stage_zero_grad, without its fill; the step's
    // completion also becomes the last op of F and B, so the next
    // iteration's first F (on any stream) reads the updated weights
    for (int k : {PASS_F, PASS_B, PASS_W}) {
        ZB_HIP(hipEventRecord(st->chain[k], s));
        st->chain_valid[k] = true;
    }
    for (auto& sl : st->slots) sl.mb = -1;
    st->next_f = st->next_w = 0;
    return st->serialize();
}

extern "C" int32_t zb_stage_set_debug(zb_stage* st, int32_t flags, int32_t w_delay_us, void* stream) {
    if (!st || (flags & ~(ZB_DEBUG_SLOT_TAGS | ZB_DEBUG_SERIALIZE)) || w_delay_us < 0 || w_delay_us > 1000000)
        return fail(ZB_EINVAL, "zb_stage_set_debug: bad argument");
    hipStream_t s = static_cast<hipStream_t>(stream);
    if ((flags & ZB_DEBUG_SLOT_TAGS) && !(st->debug_flags & ZB_DEBUG_SLOT_TAGS)) {
        // tags start at "unused"; they must not be reset under a pass that
        // is still running, so the reset follows the last op of every pass
        for (int k : {PASS_F, PASS_B, PASS_W})
            if (st->chain_valid[k]) ZB_HIP(hipStreamWaitEvent(s, st->chain[k], 0));
        const int32_t rc = tag_reset(st->tags, st->desc.ring_slots, st->dbg_rec, s);
        if (rc) return rc;
        for (int k : {PASS_F, PASS_B, PASS_W}) {  // and every later pass follows the reset
            ZB_HIP(hipEventRecord(st->chain[k], s));
            st->chain_valid[k] = true;
        }
    }
    st->debug_flags = flags;
    st->w_delay_us = w_delay_us;
    return ZB_OK;
}

extern "C" int32_t zb_stage_debug_report(zb_stage* st, int32_t* info) {
    if (!st) return fail(ZB_EINVAL, "zb_stage_debug_report: NULL stage");
    if (!(st->debug_flags & ZB_DEBUG_SLOT_TAGS)) return fail(ZB_ESTATE, "zb_stage_debug_report: slot tags are not enabled");
    int32_t rec[DEBUG_REC];
    ZB_HIP(hipDeviceSynchronize());
    ZB_HIP(hipMemcpy(rec, st->dbg_rec, sizeof(rec), hipMemcpyDeviceToHost));
    if (info)
        for (int i = 0; i < 5; ++i) info[i] = rec[i + 1];
    return rec[0];
}

extern "C" int32_t zb_stage_weights_changed(zb_stage* st) {
    if (!st) return fail(ZB_EINVAL, "zb_stage_weights_changed: NULL stage");
    st->w8_dirty = true;
    st->wt_dirty = true;
    return ZB_OK;
}

extern "C" int32_t zb_stage_set_lr(zb_stage* st, float lr) {
    if (!st || !std::isfinite(lr)) return fail(ZB_EINVAL, "zb_stage_set_lr: bad argument");
    st->lr = lr;
    return ZB_OK;
}

extern "C" int32_t zb_stage_stash_tensor(zb_stage* st, int32_t mb, int32_t layer, int32_t which, void** ptr,
                                         int32_t* rows, int32_t* cols, int32_t* dtype) {
    if (!st || mb < 0 || !ptr) return fail(ZB_EINVAL, "zb_stage_stash_tensor: bad argument");
    const Layout::Tensor* t = st->lay.find(layer, which);
    if (!t) return fail(ZB_EINVAL, "zb_stage_stash_tensor: no such tensor");
    if (st->slots[mb % st->desc.ring_slots].mb != mb) return fail(ZB_ESTATE, "zb_stage_stash_tensor: microbatch not resident");
    *ptr = st->slot_tensor(mb, layer, which);
    if (rows) *rows = t->rows;
    if (cols) *cols = t->cols;
    if (dtype) *dtype = t->dtype;
    return ZB_OK;
}

extern "C" int32_t zb_stage_fp8_weight(zb_stage* st, int32_t i, void** q, void** qt, void** e) {
    if (!st || st->desc.dtype != ZB_FP8 || i < 0 || i >= (int)st->lay.w8_e.size() || i % 6 >= 4)
        return fail(ZB_EINVAL, "zb_stage_fp8_weight: not a linear weight of a ZB_FP8 stage");
    if (q) *q = st->w8 + st->lay.w8_q[i];
    if (qt) *qt = st->w8 + st->lay.w8_qt[i];
    if (e) *e = st->w8 + st->lay.w8_e[i];
    return ZB_OK;
}

extern "C" int32_t zb_quantize_e4m3(const void* x, int32_t rows, int32_t cols, int64_t ld, void* q, int64_t ldq,
                                    void* qt, int64_t ldqt, void* e_out, void* part, void* stream) {
    return quantize_e4m3(static_cast<const bf16_t*>(x), rows, cols, ld, static_cast<uint8_t*>(q), ldq,
                         static_cast<uint8_t*>(qt), ldqt, static_cast<int32_t*>(e_out), static_cast<float*>(part),
                         static_cast<hipStream_t>(stream));
}

extern "C" int32_t zb_gemm_fp8(int32_t M, int32_t N, int32_t K, const void* A, int64_t lda, const void* ea,
                               const void* B, int64_t ldb, const void* eb, void* C, int64_t ldc, int32_t out_f32,
                               void* stream) {
    if (!A || !B || !C || !ea || !eb || M < 1 || N < 1 || K < 1 || lda < K || ldb < K || ldc < N)
        return fail(ZB_EINVAL, "zb_gemm_fp8: bad argument");
    GemmDesc g{};
    g.M = M; g.N = N; g.K = K;
    g.A = A; g.lda = lda; g.a_kmajor = 1;
    g.B = B; g.ldb = ldb; g.b_kmajor = 1;
    g.C = C; g.ldc = ldc;
    g.ea = static_cast<const int32_t*>(ea);
    g.eb = static_cast<const int32_t*>(eb);
    g.epi = out_f32 ? EPI_ACCUM_F32 : EPI_STORE;
    return gemm_fp8(g, static_cast<hipStream_t>(stream));
}

extern "C" int32_t zb_gemm_fp8_wgrad_group(int32_t count, const int32_t* M, const int32_t* N, const int32_t* K,
                                           const void* const* A, const int64_t* lda, const void* const* ea,
                                           const void* const* B, const int64_t* ldb, const void* const* eb,
                                           void* const* C, const int64_t* ldc, void* stream) {
    if (count < 1 || count > 256 || !M || !N || !K || !A || !lda || !ea || !B || !ldb || !eb || !C || !ldc)
        return fail(ZB_EINVAL, "zb_gemm_fp8_wgrad_group: bad argument");
    std::vector<GemmDesc> g(count);
    for (int i = 0; i < count; ++i) {
        if (!A[i] || !B[i] || !C[i] || !ea[i] || !eb[i] || M[i] < 1 || N[i] < 1 || K[i] < 1 || lda[i] < K[i] ||
            ldb[i] < K[i] || ldc[i] < N[i])
            return fail(ZB_EINVAL, "zb_gemm_fp8_wgrad_group: bad product");
        GemmDesc& d = g[i];
        d = GemmDesc{};
        d.M = M[i]; d.N = N[i]; d.K = K[i];
        d.A = A[i]; d.lda = lda[i]; d.a_kmajor = 1;
        d.B = B[i]; d.ldb = ldb[i]; d.b_kmajor = 1;
        d.C = C[i]; d.ldc = ldc[i];
        d.ea = static_cast<const int32_t*>(ea[i]);
        d.eb = static_cast<const int32_t*>(eb[i]);
        d.epi = EPI_ACCUM_F32;
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    for (int i = 0; i < count; i += 16) {
        const int32_t rc = gemm_fp8_group(&g[i], std::min(16, count - i), s);
        if (rc != ZB_OK) return rc;
    }
    return ZB_OK;
}

size_t zb::weight_elems(const zb_stage_desc& d, int i) {
    const size_t H = d.hidden, F = d.ffn;
    if (d.kind == ZB_LINEAR) return H * F;
    if (d.kind == ZB_MLP_GELU) return H * F;
    const size_t QD = (size_t)d.n_heads * d.head_dim, KVD = (size_t)d.n_kv_heads * d.head_dim;
    switch (i % 6) {
        case 0: return (QD + 2 * KVD) * H;
        case 1: return H * QD;
        case 2: return 2 * F * H;
        case 3: return H * F;
        default: return H;
    }
}

extern "C" int32_t zb_gemm(int32_t dtype, int32_t M, int32_t N, int32_t K, const void* A, int64_t lda,
                           int32_t a_kmajor, const void* B, int64_t ldb, int32_t b_kmajor, void* C, int64_t ldc,
                           int32_t out_f32, int32_t accumulate, void* stream) {
    if (!A || !B || !C || M < 1 || N < 1 || K < 1) return fail(ZB_EINVAL, "zb_gemm: bad argument");
    GemmDesc g{};
    g.M = M; g.N = N; g.K = K;
    g.A = A; g.lda = lda; g.a_kmajor = a_kmajor;
    g.B = B; g.ldb = ldb; g.b_kmajor = b_kmajor;
    g.C = C; g.ldc = ldc;
    const int64_t minlda = a_kmajor ? K : M, minldb = b_kmajor ? K : N;
    if (lda < minlda || ldb < minldb || ldc < N) return fail(ZB_EINVAL, "zb_gemm: leading dimension too small");
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (dtype == ZB_F32) {
        if (!out_f32) return fail(ZB_EINVAL, "zb_gemm: fp32 GEMM writes fp32");
        return gemm_f32(g, accumulate, s);
    }
    if (dtype != ZB_BF16) return fail(ZB_EINVAL, "zb_gemm: bad dtype");
    if (out_f32) {
        if (!accumulate) return fail(ZB_EINVAL, "zb_gemm: bf16 with fp32 output accumulates (C += A.B)");
        g.epi = EPI_ACCUM_F32;
    } else {
        if (accumulate) return fail(ZB_EINVAL, "zb_gemm: bf16 output does not accumulate");
        g.epi = EPI_STORE;
    }
    return gemm_bf16(g, s);
}

extern "C" int32_t zb_gemm_wgrad_group(int32_t count, const int32_t* M, const int32_t* N, const int32_t* K,
                                       const void* const* A, const int64_t* lda, int32_t a_kmajor,
                                       const void* const* B, const int64_t* ldb, int32_t b_kmajor, void* const* C,
                                       const int64_t* ldc, void* stream) {
    if (count < 1 || count > 256 || !M || !N || !K || !A || !lda || !B || !ldb || !C || !ldc)
        return fail(ZB_EINVAL, "zb_gemm_wgrad_group: bad argument");
    std::vector<GemmDesc> g(count);
    for (int i = 0; i < count; ++i) {
        if (!A[i] || !B[i] || !C[i] || M[i] < 1 || N[i] < 1 || K[i] < 1)
            return fail(ZB_EINVAL, "zb_gemm_wgrad_group: bad product");
        const int64_t minlda = a_kmajor ? K[i] : M[i], minldb = b_kmajor ? K[i] : N[i];
        if (lda[i] < minlda || ldb[i] < minldb || ldc[i] < N[i])
            return fail(ZB_EINVAL, "zb_gemm_wgrad_group: leading dimension too small");
        GemmDesc& d = g[i];
        d = GemmDesc{};
        d.M = M[i]; d.N = N[i]; d.K = K[i];
        d.A = A[i]; d.lda = lda[i]; d.a_kmajor = a_kmajor;
        d.B = B[i]; d.ldb = ldb[i]; d.b_kmajor = b_kmajor;
        d.C = C[i]; d.ldc = ldc[i];
        d.epi = EPI_ACCUM_F32;
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    constexpr int GROUP = 16;  // products per launch
    for (int i = 0; i < count; i += GROUP) {
        const int32_t rc = gemm_bf16_group(&g[i], std::min(GROUP, count - i), s);
        if (rc != ZB_OK) return rc;
    }
    return ZB_OK;
}
