// F, B and W passes of each stage kind, as sequences of kernel launches on
// one stream.  Shapes use T tokens, H = hidden, F = ffn; weights are [out, in].
//
// Per linear layer (the "Core Innovation 1" decomposition of "Zero-Bubble
// Pipeline Parallelism Guide for LLMs", in the listing's [out, in] layout):
//   F: Y = X W^T     B: dX = dY W     W: dW += dY^T X  (fp32, in place)
#include "common.h"
#include "stage.h"

#include <algorithm>
#include <vector>

namespace zb {
namespace {

GemmDesc nt(int M, int N, int K, const void* X, int64_t ldx, const void* W, int64_t ldw, void* C, int64_t ldc,
            int epi = EPI_STORE) {
    GemmDesc g{};
    g.M = M; g.N = N; g.K = K;
    g.A = X; g.lda = ldx; g.a_kmajor = 1;
    g.B = W; g.ldb = ldw; g.b_kmajor = 1;
    g.C = C; g.ldc = ldc; g.epi = epi;
    return g;
}
// C[M,N] = A[M,K] . W[K,N] with W stored [K=out, N=in]
GemmDesc nn(int M, int N, int K, const void* A, int64_t lda, const void* W, int64_t ldw, void* C, int64_t ldc,
            int epi = EPI_STORE) {
    GemmDesc g = nt(M, N, K, A, lda, W, ldw, C, ldc, epi);
    g.b_kmajor = 0;
    return g;
}
// dW[M=out, N=in] += dY[T, out]^T . X[T, in]
GemmDesc tn(int M, int N, int T, const void* dY, int64_t ldy, const void* X, int64_t ldx, float* dW) {
    GemmDesc g{};
    g.M = M; g.N = N; g.K = T;
    g.A = dY; g.lda = ldy; g.a_kmajor = 0;
    g.B = X; g.ldb = ldx; g.b_kmajor = 0;
    g.C = dW; g.ldc = N; g.epi = EPI_ACCUM_F32;
    return g;
}

#define ZB_TRY(expr)                     \
    do {                                 \
        int32_t rc_ = (expr);            \
        if (rc_ != ZB_OK) return rc_;    \
    } while (0)

int32_t linear_gemm(const zb_stage& st, const GemmDesc& g, hipStream_t s) {
    if (st.desc.dtype == ZB_F32) return gemm_f32(g, g.epi == EPI_ACCUM_F32, s);
    return gemm_bf16(g, s);
}

// A product whose tiles would fill little of the chip runs split along K
// when the pass scratch holds the partial sums.
int32_t gemm_split_if_small(const GemmDesc& g, char* scratch, size_t bytes, hipStream_t s) {
    const int split = gemm_splitk_factor(g);
    if (split > 1 && scratch != nullptr && gemm_splitk_scratch_bytes(g.M, g.N, split) <= bytes)
        return gemm_bf16_splitk(g, split, reinterpret_cast<float*>(scratch), s);
    return gemm_bf16(g, s);
}

const bf16_t* cbf(const void* p) { return static_cast<const bf16_t*>(p); }
bf16_t* bf(void* p) { return static_cast<bf16_t*>(p); }

}  // namespace

int32_t run_forward(zb_stage& st, int mb, const void* x, void* y, hipStream_t s) {
    const zb_stage_desc& d = st.desc;
    if (d.dtype == ZB_FP8) return run_forward_fp8(st, mb, x, y, s);
    const int T = d.tokens, H = d.hidden, F = d.ffn;
    if (d.kind == ZB_LINEAR) {
        void* xs = st.slot_tensor(mb, 0, LIN_X);
        ZB_TRY(copy_bytes(xs, x, (size_t)T * H * (d.dtype == ZB_F32 ? 4 : 2), s));
        return linear_gemm(st, nt(T, F, H, xs, H, st.w[0], H, y, F), s);
    }
    if (d.kind == ZB_MLP_GELU) {
        void* xs = st.slot_tensor(mb, 0, MLP_X);
        void* a = st.slot_tensor(mb, 0, MLP_A);
        void* h = st.slot_tensor(mb, 0, MLP_H);
        ZB_TRY(copy_bytes(xs, x, (size_t)T * H * 2, s));
        GemmDesc g1 = nt(T, F, H, xs, H, st.w[0], H, a, F, EPI_GELU_FWD);
        g1.C2 = h;
        g1.ldc2 = F;
        ZB_TRY(gemm_split_if_small(g1, st.scratch_f, st.lay.scratch_f, s));
        return gemm_split_if_small(nt(T, H, F, h, F, st.w[1], F, y, H), st.scratch_f, st.lay.scratch_f, s);
    }
    const int QD = d.n_heads * d.head_dim, KVD = d.n_kv_heads * d.head_dim, QKV = QD + 2 * KVD;
    for (int l = 0; l < d.n_layers; ++l) {
        void* const* w = &st.w[6 * l];
        bf16_t* xl = bf(st.slot_tensor(mb, l, L_X));
        float* r1 = static_cast<float*>(st.slot_tensor(mb, l, L_R1));
        bf16_t* n1 = bf(st.slot_tensor(mb, l, L_N1));
        bf16_t* qkv = bf(st.slot_tensor(mb, l, L_QKV));
        bf16_t* a = bf(st.slot_tensor(mb, l, L_A));
        float* lse = static_cast<float*>(st.slot_tensor(mb, l, L_LSE));
        bf16_t* h1 = bf(st.slot_tensor(mb, l, L_H1));
        float* r2 = static_cast<float*>(st.slot_tensor(mb, l, L_R2));
        bf16_t* n2 = bf(st.slot_tensor(mb, l, L_N2));
        bf16_t* gu = bf(st.slot_tensor(mb, l, L_GU));
        bf16_t* sw = bf(st.slot_tensor(mb, l, L_S));
        void* out = (l == d.n_layers - 1) ? y : st.slot_tensor(mb, l + 1, L_X);

        // layer 0 stashes the stage input as its norm reads it
        if (l == 0) ZB_TRY(rmsnorm_fwd(cbf(x), cbf(w[4]), n1, r1, T, H, d.rms_eps, s, xl));
        else ZB_TRY(rmsnorm_fwd(xl, cbf(w[4]), n1, r1, T, H, d.rms_eps, s));
        ZB_TRY(gemm_bf16(nt(T, QKV, H, n1, H, w[0], H, qkv, QKV), s));
        ZB_TRY(attn_fwd(qkv, a, lse, T, d.n_heads, d.n_kv_heads, s));
        GemmDesc go = nt(T, H, QD, a, QD, w[1], QD, h1, H, EPI_RESID);
        go.R = xl;
        go.ldr = H;
        ZB_TRY(gemm_bf16(go, s));
        ZB_TRY(rmsnorm_fwd(h1, cbf(w[5]), n2, r2, T, H, d.rms_eps, s));
        GemmDesc gg = nt(T, 2 * F, H, n2, H, w[2], H, gu, 2 * F, EPI_SWIGLU_FWD);
        gg.C2 = sw;
        gg.ldc2 = F;
        gg.half_n = F;
        ZB_TRY(gemm_bf16(gg, s));
        GemmDesc gd = nt(T, H, F, sw, F, w[3], F, out, H, EPI_RESID);
        gd.R = h1;
        gd.ldr = H;
        ZB_TRY(gemm_bf16(gd, s));
    }
    return ZB_OK;
}

int32_t run_backward_input(zb_stage& st, int mb, const void* dy, void* dx, hipStream_t s) {
    const zb_stage_desc& d = st.desc;
    if (d.dtype == ZB_FP8) return run_backward_input_fp8(st, mb, dy, dx, s);
    const int T = d.tokens, H = d.hidden, F = d.ffn;
    if (d.kind == ZB_LINEAR) {
        void* dys = st.slot_tensor(mb, 0, LIN_DY);
        ZB_TRY(copy_bytes(dys, dy, (size_t)T * F * (d.dtype == ZB_F32 ? 4 : 2), s));
        return linear_gemm(st, nn(T, H, F, dys, F, st.w[0], H, dx, H), s);
    }
    if (d.kind == ZB_MLP_GELU) {
        void* dys = st.slot_tensor(mb, 0, MLP_DY);
        void* a = st.slot_tensor(mb, 0, MLP_A);
        void* da = st.slot_tensor(mb, 0, MLP_DA);
        ZB_TRY(copy_bytes(dys, dy, (size_t)T * H * 2, s));
        GemmDesc g2 = nn(T, F, H, dys, H, st.w[1], F, da, F, EPI_GELU_BWD);
        g2.R = a;
        g2.ldr = F;
        ZB_TRY(gemm_split_if_small(g2, st.scratch_b, st.lay.scratch_b, s));
        return gemm_split_if_small(nn(T, H, F, da, F, st.w[0], H, dx, H), st.scratch_b, st.lay.scratch_b, s);
    }
    const int QD = d.n_heads * d.head_dim, KVD = d.n_kv_heads * d.head_dim, QKV = QD + 2 * KVD;
    if (st.wt_dirty) ZB_TRY(transpose_weights(st, s));
    bf16_t* da = bf(st.scratch_b);
    float* delta = reinterpret_cast<float*>(st.scratch_b + ((size_t)T * QD * 2 + 255) / 256 * 256);
    void* ascratch = reinterpret_cast<char*>(delta) + ((size_t)d.n_heads * T * 4 + 255) / 256 * 256;
    for (int l = d.n_layers - 1; l >= 0; --l) {
        void* const* w = &st.w[6 * l];
        bf16_t* xl = bf(st.slot_tensor(mb, l, L_X));
        float* r1 = static_cast<float*>(st.slot_tensor(mb, l, L_R1));
        bf16_t* qkv = bf(st.slot_tensor(mb, l, L_QKV));
        bf16_t* a = bf(st.slot_tensor(mb, l, L_A));
        float* lse = static_cast<float*>(st.slot_tensor(mb, l, L_LSE));
        bf16_t* h1 = bf(st.slot_tensor(mb, l, L_H1));
        float* r2 = static_cast<float*>(st.slot_tensor(mb, l, L_R2));
        bf16_t* gu = bf(st.slot_tensor(mb, l, L_GU));
        bf16_t* dout = bf(st.slot_tensor(mb, l, L_DOUT));
        bf16_t* dgu = bf(st.slot_tensor(mb, l, L_DGU));
        bf16_t* dn2 = bf(st.slot_tensor(mb, l, L_DN2));
        bf16_t* dh1 = bf(st.slot_tensor(mb, l, L_DH1));
        bf16_t* dqkv = bf(st.slot_tensor(mb, l, L_DQKV));
        bf16_t* dn1 = bf(st.slot_tensor(mb, l, L_DN1));
        void* dest = (l == 0) ? dx : st.slot_tensor(mb, l - 1, L_DOUT);
        // the last layer reads the incoming gradient itself and stashes it
        // (for W) in its second norm's backward, which reads it whole
        const bool last = l == d.n_layers - 1;
        const bf16_t* gin = last ? cbf(dy) : dout;

        // transposed weights [in][out]: every product below is A . B^T
        const void* wqkv_t = st.wt + st.lay.wt_off[6 * l];      // [H][QKV]
        const void* wo_t = st.wt + st.lay.wt_off[6 * l + 1];    // [QD][H]
        const void* wgu_t = st.wt + st.lay.wt_off[6 * l + 2];   // [H][2F]
        const void* wd_t = st.wt + st.lay.wt_off[6 * l + 3];    // [F][H]
        GemmDesc gd = nt(T, F, H, gin, H, wd_t, H, dgu, 2 * F, EPI_SWIGLU_BWD);
        gd.R = gu;
        gd.ldr = 2 * F;
        gd.half_n = F;
        ZB_TRY(gemm_bf16(gd, s));
        ZB_TRY(gemm_bf16(nt(T, H, 2 * F, dgu, 2 * F, wgu_t, 2 * F, dn2, H), s));
        ZB_TRY(rmsnorm_bwd(h1, r2, cbf(w[5]), dn2, gin, dh1, T, H, s, last ? dout : nullptr));
        ZB_TRY(gemm_bf16(nt(T, QD, H, dh1, H, wo_t, H, da, QD), s));
        ZB_TRY(attn_bwd(qkv, a, lse, da, dqkv, delta, ascratch, T, d.n_heads, d.n_kv_heads, s));
        ZB_TRY(gemm_bf16(nt(T, H, QKV, dqkv, QKV, wqkv_t, QKV, dn1, H), s));
        ZB_TRY(rmsnorm_bwd(xl, r1, cbf(w[4]), dn1, dh1, bf(dest), T, H, s));
    }
    return ZB_OK;
}

// The B pass of a bf16 Llama stage multiplies by each linear weight with its
// output index as the reduction index; from a transposed copy [in][out] that
// product has both operands K-contiguous (the F-layout GEMM).  Refreshed after
// the weights change (zb_stage_create, zb_stage_sgd_step,
// zb_stage_weights_changed), on the B stream, before the B that reads them.
int32_t transpose_weights(zb_stage& st, hipStream_t s) {
    const zb_stage_desc& d = st.desc;
    const int H = d.hidden, F = d.ffn;
    const int QD = d.n_heads * d.head_dim, QKV = QD + 2 * d.n_kv_heads * d.head_dim;
    const int rows[4] = {QKV, H, 2 * F, H}, cols[4] = {H, QD, H, F};  // Wqkv, Wo, Wgu, Wd as stored [out][in]
    for (int l = 0; l < d.n_layers; ++l)
        for (int k = 0; k < 4; ++k) {
            const int i = 6 * l + k;
            ZB_TRY(transpose_bf16(cbf(st.w[i]), bf(st.wt + st.lay.wt_off[i]), rows[k], cols[k], s));
        }
    st.wt_dirty = false;
    return ZB_OK;
}

size_t dgamma_scratch_bytes(const zb_stage_desc& d) {
    return d.kind == ZB_LLAMA ? rmsnorm_dgamma_scratch_floats(d.tokens, d.hidden) * sizeof(float) : 0;
}

int32_t run_backward_weight(zb_stage& st, int mb, hipStream_t s, float* dg_part) {
    const zb_stage_desc& d = st.desc;
    if (d.dtype == ZB_FP8) return run_backward_weight_fp8(st, mb, s, dg_part);
    const int T = d.tokens, H = d.hidden, F = d.ffn;
    if (d.kind == ZB_LINEAR)
        return linear_gemm(st, tn(F, H, T, st.slot_tensor(mb, 0, LIN_DY), F, st.slot_tensor(mb, 0, LIN_X), H, st.dw[0]), s);
    // Every weight-gradient product of the microbatch is independent of the
    // others (distinct dW buffers, stashed operands): they run as one grouped
    // launch (16 products at most per launch), so the partial last round of
    // one product's tiles overlaps the next product's tiles.
    constexpr int GROUP = 16;
    if (d.kind == ZB_MLP_GELU) {
        const GemmDesc g[2] = {tn(F, H, T, st.slot_tensor(mb, 0, MLP_DA), F, st.slot_tensor(mb, 0, MLP_X), H, st.dw[0]),
                               tn(H, F, T, st.slot_tensor(mb, 0, MLP_DY), H, st.slot_tensor(mb, 0, MLP_H), F, st.dw[1])};
        return gemm_bf16_group(g, 2, s);
    }
    const int QD = d.n_heads * d.head_dim, KVD = d.n_kv_heads * d.head_dim, QKV = QD + 2 * KVD;
    float* part = dg_part ? dg_part : reinterpret_cast<float*>(st.scratch_w);
    std::vector<GemmDesc> g;
    g.reserve(4 * d.n_layers);
    for (int l = 0; l < d.n_layers; ++l) {
        float* const* dw = &st.dw[6 * l];
        g.push_back(tn(QKV, H, T, st.slot_tensor(mb, l, L_DQKV), QKV, st.slot_tensor(mb, l, L_N1), H, dw[0]));
        g.push_back(tn(H, QD, T, st.slot_tensor(mb, l, L_DH1), H, st.slot_tensor(mb, l, L_A), QD, dw[1]));
        g.push_back(tn(2 * F, H, T, st.slot_tensor(mb, l, L_DGU), 2 * F, st.slot_tensor(mb, l, L_N2), H, dw[2]));
        g.push_back(tn(H, F, T, st.slot_tensor(mb, l, L_DOUT), H, st.slot_tensor(mb, l, L_S), F, dw[3]));
    }
    for (size_t i = 0; i < g.size(); i += GROUP)
        ZB_TRY(gemm_bf16_group(&g[i], (int)std::min<size_t>(GROUP, g.size() - i), s));
    for (int l = 0; l < d.n_layers; ++l) {
        float* const* dw = &st.dw[6 * l];
        ZB_TRY(rmsnorm_dgamma(cbf(st.slot_tensor(mb, l, L_X)), static_cast<const float*>(st.slot_tensor(mb, l, L_R1)),
                              cbf(st.slot_tensor(mb, l, L_DN1)), dw[4], part, T, H, s));
        ZB_TRY(rmsnorm_dgamma(cbf(st.slot_tensor(mb, l, L_H1)), static_cast<const float*>(st.slot_tensor(mb, l, L_R2)),
                              cbf(st.slot_tensor(mb, l, L_DN2)), dw[5], part, T, H, s));
    }
    return ZB_OK;
}

// W for microbatches mb and mb + 1 together: each weight-gradient product
// runs once with K spanning both microbatches' tokens (two K segments, one
// per ring slot), so dW is read and written once for the pair.  When a
// product cannot take the two-segment kernel the pair is issued as two
// ordinary W passes.  The RMSNorm dgamma reductions run per microbatch, in
// the same order as two W passes.
int32_t run_backward_weight_pair(zb_stage& st, int mb, hipStream_t s) {
    const zb_stage_desc& d = st.desc;
    if (d.dtype == ZB_FP8) {  // no two-segment fp8 kernel: two single passes
        ZB_TRY(run_backward_weight(st, mb, s));
        return run_backward_weight(st, mb + 1, s);
    }
    const int T = d.tokens, H = d.hidden, F = d.ffn;
    std::vector<GemmDesc> g;
    auto two = [&](GemmDesc a, const void* dy1, const void* x1) {
        a.K = 2 * T;
        a.K1 = T;
        a.A2 = dy1;
        a.B2 = x1;
        g.push_back(a);
    };
    const int m1 = mb + 1;
    if (d.kind == ZB_MLP_GELU && d.dtype == ZB_BF16) {
        two(tn(F, H, T, st.slot_tensor(mb, 0, MLP_DA), F, st.slot_tensor(mb, 0, MLP_X), H, st.dw[0]),
            st.slot_tensor(m1, 0, MLP_DA), st.slot_tensor(m1, 0, MLP_X));
        two(tn(H, F, T, st.slot_tensor(mb, 0, MLP_DY), H, st.slot_tensor(mb, 0, MLP_H), F, st.dw[1]),
            st.slot_tensor(m1, 0, MLP_DY), st.slot_tensor(m1, 0, MLP_H));
    } else if (d.kind == ZB_LLAMA) {
        const int QD = d.n_heads * d.head_dim, KVD = d.n_kv_heads * d.head_dim, QKV = QD + 2 * KVD;
        for (int l = 0; l < d.n_layers; ++l) {
            float* const* dw = &st.dw[6 * l];
            two(tn(QKV, H, T, st.slot_tensor(mb, l, L_DQKV), QKV, st.slot_tensor(mb, l, L_N1), H, dw[0]),
                st.slot_tensor(m1, l, L_DQKV), st.slot_tensor(m1, l, L_N1));
            two(tn(H, QD, T, st.slot_tensor(mb, l, L_DH1), H, st.slot_tensor(mb, l, L_A), QD, dw[1]),
                st.slot_tensor(m1, l, L_DH1), st.slot_tensor(m1, l, L_A));
            two(tn(2 * F, H, T, st.slot_tensor(mb, l, L_DGU), 2 * F, st.slot_tensor(mb, l, L_N2), H, dw[2]),
                st.slot_tensor(m1, l, L_DGU), st.slot_tensor(m1, l, L_N2));
            two(tn(H, F, T, st.slot_tensor(mb, l, L_DOUT), H, st.slot_tensor(mb, l, L_S), F, dw[3]),
                st.slot_tensor(m1, l, L_DOUT), st.slot_tensor(m1, l, L_S));
        }
    }
    // The products as segmented groups of at most 16; all must take that path.
    constexpr int GROUP = 16;
    bool handled = !g.empty();
    for (size_t i = 0; i < g.size() && handled; i += GROUP) {
        // probe each group before launching any, so a fallback issues nothing twice
        const int n = (int)std::min<size_t>(GROUP, g.size() - i);
        for (int j = 0; j < n && handled; ++j)
            handled = g[i + j].K1 % 32 == 0 && g[i + j].M % 8 == 0 && g[i + j].N % 8 == 0;
    }
    if (!handled) {
        ZB_TRY(run_backward_weight(st, mb, s));
        return run_backward_weight(st, m1, s);
    }
    for (size_t i = 0; i < g.size(); i += GROUP) {
        bool h = false;
        ZB_TRY(gemm_bf16_group_segmented(&g[i], (int)std::min<size_t>(GROUP, g.size() - i), s, &h));
        if (!h) {
            // A group the segmented kernel did not take (operand spans beyond
            // one buffer range): its products as one-segment products, per
            // microbatch.
            for (size_t j = i; j < std::min(g.size(), i + GROUP); ++j) {
                GemmDesc a = g[j], b = g[j];
                a.K = b.K = T;
                a.K1 = b.K1 = 0;
                a.A2 = a.B2 = b.A2 = b.B2 = nullptr;
                b.A = g[j].A2;
                b.B = g[j].B2;
                ZB_TRY(gemm_bf16(a, s));
                ZB_TRY(gemm_bf16(b, s));
            }
        }
    }
    if (d.kind == ZB_LLAMA) {
        float* part = reinterpret_cast<float*>(st.scratch_w);
        for (int m : {mb, m1})
            for (int l = 0; l < d.n_layers; ++l) {
                float* const* dw = &st.dw[6 * l];
                ZB_TRY(rmsnorm_dgamma(cbf(st.slot_tensor(m, l, L_X)), static_cast<const float*>(st.slot_tensor(m, l, L_R1)),
                                      cbf(st.slot_tensor(m, l, L_DN1)), dw[4], part, T, H, s));
                ZB_TRY(rmsnorm_dgamma(cbf(st.slot_tensor(m, l, L_H1)), static_cast<const float*>(st.slot_tensor(m, l, L_R2)),
                                      cbf(st.slot_tensor(m, l, L_DN2)), dw[5], part, T, H, s));
            }
    }
    return ZB_OK;
}

}  // namespace zb
