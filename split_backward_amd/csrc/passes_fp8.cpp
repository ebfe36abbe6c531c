// F, B and W of the ZB_FP8 Llama stage: every linear product on E4M3
// operands with per-tensor power-of-two scales (fp32 accumulation, fp32 dW);
// RMSNorm, attention and the SwiGLU epilogues as in the bf16 stage.
//
// "The Ghost in the Machine: Scaling Zero-Bubble Pipeline Parallelism",
// "Memory Pressure: The Hidden Cost of Efficiency": FP8 halves buffers and so
// makes room for the stash a zero-bubble schedule keeps until its deferred
// weight-gradient pass ("Zero-Bubble Pipeline Parallelism Guide for LLMs",
// "Core Innovation 1").  Layout choices:
//
// * Each activation or output gradient that feeds a product is quantized
//   once, as it is produced, into two code arrays: row-major [T][features]
//   (pass scratch, the K-contiguous A operand of F's or B's product) and
//   transposed [features][T] (ring slot, the K-contiguous operand of W's
//   product).  The same tensor, the same exponent, the same codes.
// * Its maximum comes from the kernel that wrote it where that kernel can
//   give it cheaply: the RMSNorm kernels (forward and backward) leave one
//   per row, the SwiGLU GEMM epilogues and the attention kernels one per
//   storing wave, and a one-workgroup kernel reduces them.  Only the
//   stage's incoming gradient, written outside the stage, takes a pass over
//   the tensor instead.
// * Weights are quantized once per iteration (first F after creation or an
//   optimizer step) into [out][in] codes (F's B operand, K = in) and
//   [in][out] codes (B's B operand, K = out).
// * So every product is C = A . B^T with both operands K-contiguous, one
//   kernel layout, no transposed LDS reads; W reads 1-byte codes from the
//   ring instead of 2-byte bf16.
//
// Per layer (weights [out, in]; q(.) = E4M3 codes, e(.) = exponent):
//   F: n1 = RMS(x)            -> q(n1) row-major + n1^T codes
//      qkv = q(n1) q(Wqkv)^T   (bf16, kept for the attention backward)
//      a = attention(qkv)      -> q(a) row-major + a^T codes; a (bf16) kept
//      h1 = x + q(a) q(Wo)^T
//      n2 = RMS(h1)            -> q(n2) row-major + n2^T codes
//      [g|u] = q(n2) q(Wgu)^T, s = silu(g) u  -> q(s) row-major + s^T codes
//      out = h1 + q(s) q(Wd)^T
//   B: q(dout) row-major + dout^T codes
//      [dg|du] = SwiGLU'(q(dout) q(Wd^T)^T)  -> row-major + dgu^T codes
//      dn2 = q(dgu) q(Wgu^T)^T (kept for dgamma2);  dh1 = dout + RMS'(dn2)
//      q(dh1) row-major + dh1^T codes;  da = q(dh1) q(Wo^T)^T
//      [dq|dk|dv] = attention'(da) -> row-major + dqkv^T codes
//      dn1 = q(dqkv) q(Wqkv^T)^T (kept for dgamma1);  dx = dh1 + RMS'(dn1)
//   W: dWqkv += dqkv^T n1, dWo += dh1^T a, dWgu += dgu^T n2, dWd += dout^T s
//      from the transposed codes (K = tokens contiguous in both), one
//      grouped launch; dgamma as in the bf16 stage.
#include <algorithm>
#include <vector>

#include "common.h"
#include "stage.h"

namespace zb {
namespace {

#define ZB_TRY(expr)                     \
    do {                                 \
        int32_t rc_ = (expr);            \
        if (rc_ != ZB_OK) return rc_;    \
    } while (0)

enum { Q_N1 = 0, Q_A, Q_N2, Q_S, Q_DOUT, Q_DGU, Q_DH1, Q_DQKV };  // exponent slots (L_QEXP)

struct Dims {
    int T, H, F, QD, KVD, QKV;
};
Dims dims_of(const zb_stage_desc& d) {
    const int QD = d.n_heads * d.head_dim, KVD = d.n_kv_heads * d.head_dim;
    return {d.tokens, d.hidden, d.ffn, QD, KVD, QD + 2 * KVD};
}

bf16_t* bf(void* p) { return static_cast<bf16_t*>(p); }
const bf16_t* cbf(const void* p) { return static_cast<const bf16_t*>(p); }
uint8_t* u8(void* p) { return static_cast<uint8_t*>(p); }
int32_t* i32(void* p) { return static_cast<int32_t*>(p); }

// C = A . B^T * 2^(ea + eb) over E4M3 codes, A [M][K], B [N][K].
GemmDesc q8(int M, int N, int K, const void* A, const int32_t* ea, const void* B, const int32_t* eb, void* C,
            int64_t ldc, int epi = EPI_STORE) {
    GemmDesc g{};
    g.M = M; g.N = N; g.K = K;
    g.A = A; g.lda = K; g.a_kmajor = 1;
    g.B = B; g.ldb = K; g.b_kmajor = 1;
    g.C = C; g.ldc = ldc; g.epi = epi;
    g.ea = ea;
    g.eb = eb;
    return g;
}

struct W8 {
    const uint8_t* q;   // [out][in]
    const uint8_t* qt;  // [in][out]
    const int32_t* e;
};
W8 w8(const zb_stage& st, int i) {
    return {reinterpret_cast<const uint8_t*>(st.w8 + st.lay.w8_q[i]),
            reinterpret_cast<const uint8_t*>(st.w8 + st.lay.w8_qt[i]),
            reinterpret_cast<const int32_t*>(st.w8 + st.lay.w8_e[i])};
}

// Weight i [out][in] bf16 -> codes [out][in] and [in][out], one exponent.
int32_t quantize_weights(zb_stage& st, hipStream_t s) {
    const zb_stage_desc& d = st.desc;
    const Dims D = dims_of(d);
    float* part = reinterpret_cast<float*>(st.scratch_f + st.lay.f_part);
    for (int l = 0; l < d.n_layers; ++l) {
        const int outs[4] = {D.QKV, D.H, 2 * D.F, D.H}, ins[4] = {D.H, D.QD, D.H, D.F};
        for (int k = 0; k < 4; ++k) {
            const int i = 6 * l + k;
            ZB_TRY(quantize_e4m3(cbf(st.w[i]), outs[k], ins[k], ins[k], u8(st.w8 + st.lay.w8_q[i]), ins[k],
                                 u8(st.w8 + st.lay.w8_qt[i]), outs[k], i32(st.w8 + st.lay.w8_e[i]), part, s));
        }
    }
    st.w8_dirty = false;
    return ZB_OK;
}

}  // namespace

// Codes (row-major into q, transposed into qt) and exponent of a [rows, cols]
// tensor whose producer wrote n partial maxima to part (capacity
// st.lay.amax_cap, the reduced value right after it).
static int32_t quantize_from(zb_stage& st, const bf16_t* x, int rows, int cols, uint8_t* q, uint8_t* qt, int32_t* e,
                      float* part, int n, hipStream_t s) {
    if (n > (int)st.lay.amax_cap) return fail(ZB_EINVAL, "fp8 stage: more partial maxima than the scratch holds");
    return quantize_e4m3_from_partials(x, rows, cols, cols, q, cols, qt, rows, e, part, n, part + st.lay.amax_cap, s);
}

// The attention forward with its output's partial maxima, after checking
// that they fit.
static int32_t attn_fwd_tracked(zb_stage& st, const bf16_t* qkv, bf16_t* a, float* lse, float* part, int* n,
                                hipStream_t s) {
    const zb_stage_desc& d = st.desc;
    const int T = dims_of(d).T;
    if (attn_amax_parts(T, d.n_heads, d.n_kv_heads) > (int64_t)st.lay.amax_cap)
        return fail(ZB_EINVAL, "fp8 stage: more partial maxima than the scratch holds");
    return attn_fwd(qkv, a, lse, T, d.n_heads, d.n_kv_heads, s, part, n);
}

int32_t run_forward_fp8(zb_stage& st, int mb, const void* x, void* y, hipStream_t s) {
    const zb_stage_desc& d = st.desc;
    const Dims D = dims_of(d);
    const int T = D.T, H = D.H, F = D.F;
    if (st.w8_dirty) ZB_TRY(quantize_weights(st, s));
    bf16_t* act = bf(st.scratch_f + st.lay.f_act);       // n1, n2 or s (bf16)
    uint8_t* qrow = u8(st.scratch_f + st.lay.f_q);       // its row-major codes
    float* part = reinterpret_cast<float*>(st.scratch_f + st.lay.f_part);
    for (int l = 0; l < d.n_layers; ++l) {
        void* const* w = &st.w[6 * l];
        const W8 wqkv = w8(st, 6 * l), wo = w8(st, 6 * l + 1), wgu = w8(st, 6 * l + 2), wd = w8(st, 6 * l + 3);
        bf16_t* xl = bf(st.slot_tensor(mb, l, L_X));
        float* r1 = static_cast<float*>(st.slot_tensor(mb, l, L_R1));
        bf16_t* qkv = bf(st.slot_tensor(mb, l, L_QKV));
        bf16_t* a = bf(st.slot_tensor(mb, l, L_A));
        float* lse = static_cast<float*>(st.slot_tensor(mb, l, L_LSE));
        bf16_t* h1 = bf(st.slot_tensor(mb, l, L_H1));
        float* r2 = static_cast<float*>(st.slot_tensor(mb, l, L_R2));
        bf16_t* gu = bf(st.slot_tensor(mb, l, L_GU));
        int32_t* ex = i32(st.slot_tensor(mb, l, L_QEXP));
        void* out = (l == d.n_layers - 1) ? y : st.slot_tensor(mb, l + 1, L_X);

        // layer 0 stashes the stage input as its norm reads it; the norms,
        // and the SwiGLU product, leave the partial maxima of their outputs
        if (l == 0) ZB_TRY(rmsnorm_fwd(cbf(x), cbf(w[4]), act, r1, T, H, d.rms_eps, s, xl, part));
        else ZB_TRY(rmsnorm_fwd(xl, cbf(w[4]), act, r1, T, H, d.rms_eps, s, nullptr, part));
        ZB_TRY(quantize_from(st, act, T, H, qrow, u8(st.slot_tensor(mb, l, L_N1T)), ex + Q_N1, part, T, s));
        ZB_TRY(gemm_fp8(q8(T, D.QKV, H, qrow, ex + Q_N1, wqkv.q, wqkv.e, qkv, D.QKV), s));
        int n_parts = 0;
        ZB_TRY(attn_fwd_tracked(st, qkv, a, lse, part, &n_parts, s));
        ZB_TRY(quantize_from(st, a, T, D.QD, qrow, u8(st.slot_tensor(mb, l, L_AT)), ex + Q_A, part, n_parts, s));
        GemmDesc go = q8(T, H, D.QD, qrow, ex + Q_A, wo.q, wo.e, h1, H, EPI_RESID);
        go.R = xl;
        go.ldr = H;
        ZB_TRY(gemm_fp8(go, s));
        ZB_TRY(rmsnorm_fwd(h1, cbf(w[5]), act, r2, T, H, d.rms_eps, s, nullptr, part));
        ZB_TRY(quantize_from(st, act, T, H, qrow, u8(st.slot_tensor(mb, l, L_N2T)), ex + Q_N2, part, T, s));
        GemmDesc gg = q8(T, 2 * F, H, qrow, ex + Q_N2, wgu.q, wgu.e, gu, 2 * F, EPI_SWIGLU_FWD);
        gg.C2 = act;  // s = silu(g) u
        gg.ldc2 = F;
        gg.half_n = F;
        gg.amax = part;
        ZB_TRY(gemm_fp8(gg, s, &n_parts, (int)st.lay.amax_cap));
        ZB_TRY(quantize_from(st, act, T, F, qrow, u8(st.slot_tensor(mb, l, L_ST)), ex + Q_S, part, n_parts, s));
        GemmDesc gd = q8(T, H, F, qrow, ex + Q_S, wd.q, wd.e, out, H, EPI_RESID);
        gd.R = h1;
        gd.ldr = H;
        ZB_TRY(gemm_fp8(gd, s));
    }
    return ZB_OK;
}

int32_t run_backward_input_fp8(zb_stage& st, int mb, const void* dy, void* dx, hipStream_t s) {
    const zb_stage_desc& d = st.desc;
    const Dims D = dims_of(d);
    const int T = D.T, H = D.H, F = D.F;
    char* sb = st.scratch_b;
    bf16_t* da = bf(sb);
    float* delta = reinterpret_cast<float*>(sb + ((size_t)T * D.QD * 2 + 255) / 256 * 256);
    void* ascratch = reinterpret_cast<char*>(delta) + ((size_t)d.n_heads * T * 4 + 255) / 256 * 256;
    bf16_t* dgu = bf(sb + st.lay.b_dgu);
    bf16_t* dh1 = bf(sb + st.lay.b_dh1);
    bf16_t* dqkv = bf(sb + st.lay.b_dqkv);
    bf16_t* pingpong[2] = {bf(sb + st.lay.b_dout[0]), bf(sb + st.lay.b_dout[1])};
    uint8_t* qrow = u8(sb + st.lay.b_q);
    float* part = reinterpret_cast<float*>(sb + st.lay.b_part);
    const bf16_t* dout = cbf(dy);
    for (int l = d.n_layers - 1; l >= 0; --l) {
        void* const* w = &st.w[6 * l];
        const W8 wqkv = w8(st, 6 * l), wo = w8(st, 6 * l + 1), wgu = w8(st, 6 * l + 2), wd = w8(st, 6 * l + 3);
        bf16_t* xl = bf(st.slot_tensor(mb, l, L_X));
        float* r1 = static_cast<float*>(st.slot_tensor(mb, l, L_R1));
        bf16_t* qkv = bf(st.slot_tensor(mb, l, L_QKV));
        bf16_t* a = bf(st.slot_tensor(mb, l, L_A));
        float* lse = static_cast<float*>(st.slot_tensor(mb, l, L_LSE));
        bf16_t* h1 = bf(st.slot_tensor(mb, l, L_H1));
        float* r2 = static_cast<float*>(st.slot_tensor(mb, l, L_R2));
        bf16_t* gu = bf(st.slot_tensor(mb, l, L_GU));
        bf16_t* dn2 = bf(st.slot_tensor(mb, l, L_DN2));
        bf16_t* dn1 = bf(st.slot_tensor(mb, l, L_DN1));
        int32_t* ex = i32(st.slot_tensor(mb, l, L_QEXP));
        bf16_t* dest = (l == 0) ? bf(dx) : pingpong[l & 1];

        // the incoming gradient gets a pass for its maximum; the other
        // quantized tensors come with the partial maxima their producer left
        // (below the last layer, dout is the previous layer's norm backward)
        if (l == d.n_layers - 1)
            ZB_TRY(quantize_e4m3(dout, T, H, H, qrow, H, u8(st.slot_tensor(mb, l, L_DOUTT)), T, ex + Q_DOUT, part, s));
        else
            ZB_TRY(quantize_from(st, dout, T, H, qrow, u8(st.slot_tensor(mb, l, L_DOUTT)), ex + Q_DOUT, part, T, s));
        // ds = dout . Wd  (Wd^T codes [F][H]), SwiGLU backward into [dg | du]
        GemmDesc gd = q8(T, F, H, qrow, ex + Q_DOUT, wd.qt, wd.e, dgu, 2 * F, EPI_SWIGLU_BWD);
        gd.R = gu;
        gd.ldr = 2 * F;
        gd.half_n = F;
        gd.amax = part;
        int n_parts = 0;
        ZB_TRY(gemm_fp8(gd, s, &n_parts, (int)st.lay.amax_cap));
        ZB_TRY(quantize_from(st, dgu, T, 2 * F, qrow, u8(st.slot_tensor(mb, l, L_DGUT)), ex + Q_DGU, part, n_parts, s));
        ZB_TRY(gemm_fp8(q8(T, H, 2 * F, qrow, ex + Q_DGU, wgu.qt, wgu.e, dn2, H), s));
        ZB_TRY(rmsnorm_bwd(h1, r2, cbf(w[5]), dn2, dout, dh1, T, H, s, nullptr, part));
        ZB_TRY(quantize_from(st, dh1, T, H, qrow, u8(st.slot_tensor(mb, l, L_DH1T)), ex + Q_DH1, part, T, s));
        ZB_TRY(gemm_fp8(q8(T, D.QD, H, qrow, ex + Q_DH1, wo.qt, wo.e, da, D.QD), s));
        if (attn_amax_parts(T, d.n_heads, d.n_kv_heads) > (int64_t)st.lay.amax_cap)
            return fail(ZB_EINVAL, "fp8 stage: more partial maxima than the scratch holds");
        ZB_TRY(attn_bwd(qkv, a, lse, da, dqkv, delta, ascratch, T, d.n_heads, d.n_kv_heads, s, part, &n_parts));
        ZB_TRY(quantize_from(st, dqkv, T, D.QKV, qrow, u8(st.slot_tensor(mb, l, L_DQKVT)), ex + Q_DQKV, part, n_parts,
                             s));
        ZB_TRY(gemm_fp8(q8(T, H, D.QKV, qrow, ex + Q_DQKV, wqkv.qt, wqkv.e, dn1, H), s));
        ZB_TRY(rmsnorm_bwd(xl, r1, cbf(w[4]), dn1, dh1, dest, T, H, s, nullptr, l > 0 ? part : nullptr));
        dout = dest;
    }
    return ZB_OK;
}

int32_t run_backward_weight_fp8(zb_stage& st, int mb, hipStream_t s, float* dg_part) {
    const zb_stage_desc& d = st.desc;
    const Dims D = dims_of(d);
    const int T = D.T, H = D.H, F = D.F;
    float* part = dg_part ? dg_part : reinterpret_cast<float*>(st.scratch_w);
    std::vector<GemmDesc> g;
    g.reserve(4 * d.n_layers);
    for (int l = 0; l < d.n_layers; ++l) {
        float* const* dw = &st.dw[6 * l];
        const int32_t* ex = i32(st.slot_tensor(mb, l, L_QEXP));
        auto t = [&](int which) { return st.slot_tensor(mb, l, which); };
        g.push_back(q8(D.QKV, H, T, t(L_DQKVT), ex + Q_DQKV, t(L_N1T), ex + Q_N1, dw[0], H, EPI_ACCUM_F32));
        g.push_back(q8(H, D.QD, T, t(L_DH1T), ex + Q_DH1, t(L_AT), ex + Q_A, dw[1], D.QD, EPI_ACCUM_F32));
        g.push_back(q8(2 * F, H, T, t(L_DGUT), ex + Q_DGU, t(L_N2T), ex + Q_N2, dw[2], H, EPI_ACCUM_F32));
        g.push_back(q8(H, F, T, t(L_DOUTT), ex + Q_DOUT, t(L_ST), ex + Q_S, dw[3], F, EPI_ACCUM_F32));
    }
    constexpr int GROUP = 16;
    for (size_t i = 0; i < g.size(); i += GROUP)
        ZB_TRY(gemm_fp8_group(&g[i], (int)std::min<size_t>(GROUP, g.size() - i), s));
    for (int l = 0; l < d.n_layers; ++l) {
        float* const* dw = &st.dw[6 * l];
        ZB_TRY(rmsnorm_dgamma(cbf(st.slot_tensor(mb, l, L_X)), static_cast<const float*>(st.slot_tensor(mb, l, L_R1)),
                              cbf(st.slot_tensor(mb, l, L_DN1)), dw[4], part, T, H, s));
        ZB_TRY(rmsnorm_dgamma(cbf(st.slot_tensor(mb, l, L_H1)), static_cast<const float*>(st.slot_tensor(mb, l, L_R2)),
                              cbf(st.slot_tensor(mb, l, L_DN2)), dw[5], part, T, H, s));
    }
    return ZB_OK;
}

}  // namespace zb
