// Causal grouped-query attention core of the Llama stage (head_dim 128), a
// weightless op: its forward runs in F and its whole backward in B.
//
//   S = q k^T / sqrt(d) (key index <= query index),  P = softmax(S),  o = P v
//   dP = do v^T,  dS = P (dP - rowsum(do o)),  dq = dS k / sqrt(d),
//   dk = dS^T q / sqrt(d),  dv = P^T do   (dk, dv summed over each KV group)
//
// CDNA4 design.  Every product is a v_mfma_f32_32x32x16_bf16.  The forward and
// the dq kernel compute the TRANSPOSED score block S^T = K Q^T, so each lane
// owns one query column: the softmax row statistics are per-lane scalars
// (combined with the partner lane 32 away), and the probabilities already sit
// in the B-operand layout of the next product O^T += V^T P^T.  The MFMA
// reduction index of that product is the key index in the order the score
// accumulator holds it; the V^T operand is read from a transposed LDS tile in
// the same order, so no shuffle of P is needed.  The dk/dv kernel owns a key
// block per workgroup and sweeps the query blocks, accumulating dK^T and dV^T
// in registers, so the backward needs no atomics and is deterministic.
// Softmax runs in fp32 in the base-2 domain; the stashed row statistic is
// lse2 = max + log2(sum) of the scaled scores.
#include "common.h"

namespace zb {
namespace {

constexpr int D = 128;          // head dim
constexpr float LOG2E = 1.4426950408889634f;

__device__ __forceinline__ floatx16 zero16() {
    floatx16 z;
#pragma unroll
    for (int i = 0; i < 16; ++i) z[i] = 0.f;
    return z;
}

__device__ __forceinline__ floatx16 mfma(const bf16x8& a, const bf16x8& b, const floatx16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Pack 8 fp32 into a bf16x8 operand.
__device__ __forceinline__ bf16x8 pack_bf16x8(float a0, float a1, float a2, float a3, float a4, float a5, float a6,
                                              float a7) {
    bf16x8 v;
    v[0] = (__bf16)a0; v[1] = (__bf16)a1; v[2] = (__bf16)a2; v[3] = (__bf16)a3;
    v[4] = (__bf16)a4; v[5] = (__bf16)a5; v[6] = (__bf16)a6; v[7] = (__bf16)a7;
    return v;
}

// Accumulator slots [8h, 8h+8) of a 32x32 block as a bf16 B/A operand.  Slot s
// of lane group g holds reduction index 16h' + 8(s/4) + 4g + s%4 relative to
// the block (h' = half), matching the C layout rows (r/4)*8 + 4g + r%4.
__device__ __forceinline__ bf16x8 acc_half_to_bf16(const floatx16& c, int half) {
    const int b = half * 8;
    return pack_bf16x8(c[b], c[b + 1], c[b + 2], c[b + 3], c[b + 4], c[b + 5], c[b + 6], c[b + 7]);
}

// ---- LDS tile helpers ----------------------------------------------------
// Row-major tile with 128 bf16 (256 B) per row, 16-byte chunks swizzled by row.
__device__ __forceinline__ int rm_off(int row, int chunk) { return row * D + ((chunk ^ (row & 7)) << 3); }
// Transposed tile [128 d][NK keys] with NK*2 bytes per row, 8-byte units swizzled.
template <int NK>
__device__ __forceinline__ int tr_off(int d, int unit) {
    constexpr int UNITS = NK / 4;
    return d * NK + ((unit ^ (d & (UNITS - 1) & 15)) << 2);
}

// Operand read from a transposed tile: row d, keys 16*step + {4g..4g+3} and
// 16*step + 8 + {4g..4g+3}.
template <int NK>
__device__ __forceinline__ bf16x8 read_tr_operand(const bf16_t* t, int d, int step, int g) {
    const u32x2 lo = *reinterpret_cast<const u32x2*>(t + tr_off<NK>(d, 4 * step + g));
    const u32x2 hi = *reinterpret_cast<const u32x2*>(t + tr_off<NK>(d, 4 * step + 2 + g));
    u32x4 v{lo[0], lo[1], hi[0], hi[1]};
    return __builtin_bit_cast(bf16x8, v);
}

// Write a 4 (rows = keys) x 8 (d) register block transposed into a [128][NK] tile.
template <int NK>
__device__ __forceinline__ void store_tr_block(const u32x4 (&reg)[4], bf16_t* t, int key0, int d0) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        const uint32_t a0 = reg[0][w], a1 = reg[1][w], a2 = reg[2][w], a3 = reg[3][w];
        const u32x2 lo{(a0 & 0xffffu) | (a1 << 16), (a2 & 0xffffu) | (a3 << 16)};
        const u32x2 hi{(a0 >> 16) | (a1 & 0xffff0000u), (a2 >> 16) | (a3 & 0xffff0000u)};
        const int d = d0 + 2 * w;
        *reinterpret_cast<u32x2*>(t + tr_off<NK>(d, key0 / 4)) = lo;
        *reinterpret_cast<u32x2*>(t + tr_off<NK>(d + 1, key0 / 4)) = hi;
    }
}

// ======================================================== forward ========
constexpr int FQ = 128, FKV = 64, FTHR = 256;

struct FwdSmem {
    bf16_t k[2][FKV * D];
    bf16_t vt[2][D * FKV];
};

__global__ __launch_bounds__(FTHR) void attn_fwd_kernel(const bf16_t* __restrict__ qkv, bf16_t* __restrict__ o,
                                                        float* __restrict__ lse, int T, int nq, int nkv) {
    __shared__ __attribute__((aligned(16))) FwdSmem sm;
    const int ld = (nq + 2 * nkv) * D;
    const int h = blockIdx.y;
    const int grp = h / (nq / nkv);
    const int nqb = T / FQ;
    const int qb = nqb - 1 - blockIdx.x;  // heaviest (longest causal range) first
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 5, col = lane & 31;
    const int qw0 = qb * FQ + wave * 32;
    const int q = qw0 + col;
    const bf16_t* kbase = qkv + nq * D + grp * D;
    const bf16_t* vbase = qkv + (nq + nkv) * D + grp * D;

    bf16x8 qf[8];
#pragma unroll
    for (int kk = 0; kk < 8; ++kk)
        qf[kk] = *reinterpret_cast<const bf16x8*>(qkv + (int64_t)q * ld + h * D + kk * 16 + g * 8);

    floatx16 oacc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) oacc[i] = zero16();
    float m = -INFINITY, l = 0.f;
    const float c = LOG2E / sqrtf((float)D);

    const int nkb = (qb * FQ + FQ) / FKV;  // key blocks up to the diagonal
    u32x4 rk[4], rv[4];
    auto fetch = [&](int kb) {
        const int k0 = kb * FKV;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int cidx = tid + i * FTHR;  // 1024 chunks of 16 B
            const int r = cidx >> 4, ch = cidx & 15;
            rk[i] = *reinterpret_cast<const u32x4*>(kbase + (int64_t)(k0 + r) * ld + ch * 8);
        }
        const int kg = tid >> 4, dq = tid & 15;  // 4 keys x 8 d per thread
#pragma unroll
        for (int r = 0; r < 4; ++r)
            rv[r] = *reinterpret_cast<const u32x4*>(vbase + (int64_t)(k0 + kg * 4 + r) * ld + dq * 8);
    };
    auto stash = [&](int buf) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int cidx = tid + i * FTHR;
            const int r = cidx >> 4, ch = cidx & 15;
            *reinterpret_cast<u32x4*>(sm.k[buf] + rm_off(r, ch)) = rk[i];
        }
        store_tr_block<FKV>(rv, sm.vt[buf], (tid >> 4) * 4, (tid & 15) * 8);
    };

    fetch(0);
    stash(0);
    __syncthreads();
    for (int kb = 0; kb < nkb; ++kb) {
        const int cur = kb & 1;
        if (kb + 1 < nkb) fetch(kb + 1);
        const int k0 = kb * FKV;
        if (k0 <= qw0 + 31) {  // some key of this block is visible to the wave
            const bf16_t* kt = sm.k[cur];
            floatx16 s[2];
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                s[j] = zero16();
#pragma unroll
                for (int kk = 0; kk < 8; ++kk) {
                    const int row = j * 32 + col;
                    const bf16x8 a = *reinterpret_cast<const bf16x8*>(kt + rm_off(row, kk * 2 + g));
                    s[j] = mfma(a, qf[kk], s[j]);
                }
            }
            // scale, mask, running max
            float mx = -INFINITY;
            const bool diag = (k0 + FKV - 1 > qw0);
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    float v = s[j][r] * c;
                    if (diag) {
                        const int key = k0 + j * 32 + (r >> 2) * 8 + g * 4 + (r & 3);
                        if (key > q) v = -INFINITY;
                    }
                    s[j][r] = v;
                    mx = fmaxf(mx, v);
                }
            mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
            const float mnew = fmaxf(m, mx);
            const float alpha = exp2f(m - mnew);
            float rs = 0.f;
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float p = exp2f(s[j][r] - mnew);
                    s[j][r] = p;
                    rs += p;
                }
            rs += __shfl_xor(rs, 32, 64);
            l = l * alpha + rs;
            m = mnew;
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int e = 0; e < 16; ++e) oacc[i][e] *= alpha;
            bf16x8 pb[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) pb[t] = acc_half_to_bf16(s[t >> 1], t & 1);
            const bf16_t* vt = sm.vt[cur];
#pragma unroll
            for (int db = 0; db < 4; ++db)
#pragma unroll
                for (int t = 0; t < 4; ++t)
                    oacc[db] = mfma(read_tr_operand<FKV>(vt, db * 32 + col, t, g), pb[t], oacc[db]);
        }
        if (kb + 1 < nkb) stash(cur ^ 1);
        __syncthreads();
    }
    const float inv = 1.f / l;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
            const int d = db * 32 + rg * 8 + g * 4;
            u32x2 v;
            v[0] = uint32_t(f2bf(oacc[db][rg * 4] * inv)) | (uint32_t(f2bf(oacc[db][rg * 4 + 1] * inv)) << 16);
            v[1] = uint32_t(f2bf(oacc[db][rg * 4 + 2] * inv)) | (uint32_t(f2bf(oacc[db][rg * 4 + 3] * inv)) << 16);
            *reinterpret_cast<u32x2*>(o + (int64_t)q * (nq * D) + h * D + d) = v;
        }
    if (g == 0) lse[(int64_t)h * T + q] = m + log2f(l);
}

// ===================================================== delta = rowsum(do o)
__global__ __launch_bounds__(256) void attn_delta_kernel(const bf16_t* __restrict__ o, const bf16_t* __restrict__ dout,
                                                         float* __restrict__ delta, int T, int nq) {
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6);  // (q, h) pair
    const int lane = threadIdx.x & 63;
    if (row >= T * nq) return;
    const int q = row / nq, h = row % nq;
    const int64_t base = (int64_t)q * nq * D + h * D + lane * 2;
    const uint32_t ov = *reinterpret_cast<const uint32_t*>(o + base);
    const uint32_t dv = *reinterpret_cast<const uint32_t*>(dout + base);
    float s = __uint_as_float(ov << 16) * __uint_as_float(dv << 16) +
              __uint_as_float(ov & 0xffff0000u) * __uint_as_float(dv & 0xffff0000u);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off, 64);
    if (lane == 0) delta[(int64_t)h * T + q] = s;
}

// ====================================================== dq kernel ========
// Per (query block of 128, query head).  Mirrors the forward: S^T = K Q^T,
// dP^T = V dO^T, dS^T = P^T (dP^T - delta), dQ^T += K^T dS^T.
struct DqSmem {
    bf16_t k[2][FKV * D];
    bf16_t v[2][FKV * D];
    bf16_t kt[2][D * FKV];
};

__global__ __launch_bounds__(FTHR) void attn_dq_kernel(const bf16_t* __restrict__ qkv, const bf16_t* __restrict__ dout,
                                                       const float* __restrict__ lse, const float* __restrict__ delta,
                                                       bf16_t* __restrict__ dqkv, int T, int nq, int nkv) {
    extern __shared__ __attribute__((aligned(16))) char dyn_smem[];
    DqSmem& sm = *reinterpret_cast<DqSmem*>(dyn_smem);
    const int ld = (nq + 2 * nkv) * D;
    const int h = blockIdx.y;
    const int grp = h / (nq / nkv);
    const int nqb = T / FQ;
    const int qb = nqb - 1 - blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 5, col = lane & 31;
    const int qw0 = qb * FQ + wave * 32;
    const int q = qw0 + col;
    const bf16_t* kbase = qkv + nq * D + grp * D;
    const bf16_t* vbase = qkv + (nq + nkv) * D + grp * D;
    const int ldo = nq * D;

    bf16x8 qf[8], dof[8];
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
        qf[kk] = *reinterpret_cast<const bf16x8*>(qkv + (int64_t)q * ld + h * D + kk * 16 + g * 8);
        dof[kk] = *reinterpret_cast<const bf16x8*>(dout + (int64_t)q * ldo + h * D + kk * 16 + g * 8);
    }
    const float lq = lse[(int64_t)h * T + q];
    const float dq_delta = delta[(int64_t)h * T + q];
    const float c = LOG2E / sqrtf((float)D);

    floatx16 dacc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) dacc[i] = zero16();

    const int nkb = (qb * FQ + FQ) / FKV;
    u32x4 rk[4], rv[4], rt[4];
    auto fetch = [&](int kb) {
        const int k0 = kb * FKV;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int cidx = tid + i * FTHR;
            const int r = cidx >> 4, ch = cidx & 15;
            rk[i] = *reinterpret_cast<const u32x4*>(kbase + (int64_t)(k0 + r) * ld + ch * 8);
            rv[i] = *reinterpret_cast<const u32x4*>(vbase + (int64_t)(k0 + r) * ld + ch * 8);
        }
        const int kg = tid >> 4, dq = tid & 15;
#pragma unroll
        for (int r = 0; r < 4; ++r)
            rt[r] = *reinterpret_cast<const u32x4*>(kbase + (int64_t)(k0 + kg * 4 + r) * ld + dq * 8);
    };
    auto stash = [&](int buf) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int cidx = tid + i * FTHR;
            const int r = cidx >> 4, ch = cidx & 15;
            *reinterpret_cast<u32x4*>(sm.k[buf] + rm_off(r, ch)) = rk[i];
            *reinterpret_cast<u32x4*>(sm.v[buf] + rm_off(r, ch)) = rv[i];
        }
        store_tr_block<FKV>(rt, sm.kt[buf], (tid >> 4) * 4, (tid & 15) * 8);
    };

    fetch(0);
    stash(0);
    __syncthreads();
    for (int kb = 0; kb < nkb; ++kb) {
        const int cur = kb & 1;
        if (kb + 1 < nkb) fetch(kb + 1);
        const int k0 = kb * FKV;
        if (k0 <= qw0 + 31) {
            floatx16 s[2], dp[2];
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                s[j] = zero16();
                dp[j] = zero16();
                const int row = j * 32 + col;
#pragma unroll
                for (int kk = 0; kk < 8; ++kk) {
                    const bf16x8 ak = *reinterpret_cast<const bf16x8*>(sm.k[cur] + rm_off(row, kk * 2 + g));
                    s[j] = mfma(ak, qf[kk], s[j]);
                    const bf16x8 av = *reinterpret_cast<const bf16x8*>(sm.v[cur] + rm_off(row, kk * 2 + g));
                    dp[j] = mfma(av, dof[kk], dp[j]);
                }
            }
            const bool diag = (k0 + FKV - 1 > qw0);
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    float p = exp2f(s[j][r] * c - lq);
                    if (diag) {
                        const int key = k0 + j * 32 + (r >> 2) * 8 + g * 4 + (r & 3);
                        if (key > q) p = 0.f;
                    }
                    s[j][r] = p * (dp[j][r] - dq_delta);  // dS^T
                }
            bf16x8 sb[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) sb[t] = acc_half_to_bf16(s[t >> 1], t & 1);
#pragma unroll
            for (int db = 0; db < 4; ++db)
#pragma unroll
                for (int t = 0; t < 4; ++t)
                    dacc[db] = mfma(read_tr_operand<FKV>(sm.kt[cur], db * 32 + col, t, g), sb[t], dacc[db]);
        }
        if (kb + 1 < nkb) stash(cur ^ 1);
        __syncthreads();
    }
    const float scale = 1.f / sqrtf((float)D);
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
            const int d = db * 32 + rg * 8 + g * 4;
            u32x2 v;
            v[0] = uint32_t(f2bf(dacc[db][rg * 4] * scale)) | (uint32_t(f2bf(dacc[db][rg * 4 + 1] * scale)) << 16);
            v[1] = uint32_t(f2bf(dacc[db][rg * 4 + 2] * scale)) | (uint32_t(f2bf(dacc[db][rg * 4 + 3] * scale)) << 16);
            *reinterpret_cast<u32x2*>(dqkv + (int64_t)q * ld + h * D + d) = v;
        }
}

// ===================================================== dk / dv kernel ====
// Per (key block of 128, KV head).  Each wave owns 32 keys (K and V rows in
// registers as B operands).  Sweeps the query heads of the group and the
// query blocks of 32 rows at or after the diagonal:
//   S = Q K^T, P = exp2(S c - lse2), dP = dO V^T, dS = P (dP - delta),
//   dV^T += dO^T P,  dK^T += Q^T dS.
constexpr int BKV = 128, BQB = 32;

struct DkvSmem {
    bf16_t q[2][BQB * D];
    bf16_t dO[2][BQB * D];
    bf16_t qt[2][D * BQB];
    bf16_t dot[2][D * BQB];
    float lse[2][BQB];
    float delta[2][BQB];
};

__global__ __launch_bounds__(FTHR) void attn_dkv_kernel(const bf16_t* __restrict__ qkv, const bf16_t* __restrict__ dout,
                                                        const float* __restrict__ lse, const float* __restrict__ delta,
                                                        bf16_t* __restrict__ dqkv, int T, int nq, int nkv) {
    extern __shared__ __attribute__((aligned(16))) char dyn_smem[];
    DkvSmem& sm = *reinterpret_cast<DkvSmem*>(dyn_smem);
    const int ld = (nq + 2 * nkv) * D;
    const int ldo = nq * D;
    const int grp = blockIdx.y;
    const int rep = nq / nkv;
    const int nkb = T / BKV;
    const int kb = blockIdx.x;  // low key blocks have the most query blocks; launch them first
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 5, col = lane & 31;
    const int kw0 = kb * BKV + wave * 32;
    const int key = kw0 + col;
    (void)nkb;

    bf16x8 kf[8], vf[8];
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
        kf[kk] = *reinterpret_cast<const bf16x8*>(qkv + (int64_t)key * ld + nq * D + grp * D + kk * 16 + g * 8);
        vf[kk] = *reinterpret_cast<const bf16x8*>(qkv + (int64_t)key * ld + (nq + nkv) * D + grp * D + kk * 16 + g * 8);
    }
    floatx16 dk[4], dv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        dk[i] = zero16();
        dv[i] = zero16();
    }
    const float c = LOG2E / sqrtf((float)D);
    const int qb0 = (kb * BKV) / BQB;
    const int nqb = T / BQB;
    const int per_head = nqb - qb0;
    const int total = per_head * rep;

    u32x4 rq[4];
    float rl = 0.f;
    auto fetch = [&](int it) {
        const int hh = grp * rep + it / per_head;
        const int q0 = (qb0 + it % per_head) * BQB;
        // threads 0..127: Q block (4 rows x 8 d); 128..255: dO block
        const int t = tid & 127;
        const int rg = t >> 4, dq = t & 15;  // rows 4rg..4rg+3, d 8dq..8dq+7
        if (tid < 128) {
#pragma unroll
            for (int r = 0; r < 4; ++r)
                rq[r] = *reinterpret_cast<const u32x4*>(qkv + (int64_t)(q0 + rg * 4 + r) * ld + hh * D + dq * 8);
        } else {
#pragma unroll
            for (int r = 0; r < 4; ++r)
                rq[r] = *reinterpret_cast<const u32x4*>(dout + (int64_t)(q0 + rg * 4 + r) * ldo + hh * D + dq * 8);
        }
        if (tid < BQB) rl = lse[(int64_t)hh * T + q0 + tid];
        else if (tid >= 64 && tid < 64 + BQB) rl = delta[(int64_t)hh * T + q0 + tid - 64];
    };
    auto stash = [&](int buf) {
        const int t = tid & 127;
        const int rg = t >> 4, dq = t & 15;
        bf16_t* rowt = tid < 128 ? sm.q[buf] : sm.dO[buf];
        bf16_t* trt = tid < 128 ? sm.qt[buf] : sm.dot[buf];
#pragma unroll
        for (int r = 0; r < 4; ++r) *reinterpret_cast<u32x4*>(rowt + rm_off(rg * 4 + r, dq)) = rq[r];
        store_tr_block<BQB>(rq, trt, rg * 4, dq * 8);
        if (tid < BQB) sm.lse[buf][tid] = rl;
        else if (tid >= 64 && tid < 64 + BQB) sm.delta[buf][tid - 64] = rl;
    };

    fetch(0);
    stash(0);
    __syncthreads();
    for (int it = 0; it < total; ++it) {
        const int cur = it & 1;
        if (it + 1 < total) fetch(it + 1);
        const int q0 = (qb0 + it % per_head) * BQB;
        if (q0 + BQB - 1 >= kw0) {  // some query of the block sees some key of the wave
            floatx16 s = zero16(), dp = zero16();
#pragma unroll
            for (int kk = 0; kk < 8; ++kk) {
                const bf16x8 aq = *reinterpret_cast<const bf16x8*>(sm.q[cur] + rm_off(col, kk * 2 + g));
                s = mfma(aq, kf[kk], s);
                const bf16x8 ad = *reinterpret_cast<const bf16x8*>(sm.dO[cur] + rm_off(col, kk * 2 + g));
                dp = mfma(ad, vf[kk], dp);
            }
            const bool diag = (q0 < kw0 + 31);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int qr = (r >> 2) * 8 + g * 4 + (r & 3);
                float p = exp2f(s[r] * c - sm.lse[cur][qr]);
                if (diag && key > q0 + qr) p = 0.f;
                s[r] = p;
                dp[r] = p * (dp[r] - sm.delta[cur][qr]);
            }
            const bf16x8 p0 = acc_half_to_bf16(s, 0), p1 = acc_half_to_bf16(s, 1);
            const bf16x8 s0 = acc_half_to_bf16(dp, 0), s1 = acc_half_to_bf16(dp, 1);
#pragma unroll
            for (int db = 0; db < 4; ++db) {
                const int d = db * 32 + col;
                dv[db] = mfma(read_tr_operand<BQB>(sm.dot[cur], d, 0, g), p0, dv[db]);
                dv[db] = mfma(read_tr_operand<BQB>(sm.dot[cur], d, 1, g), p1, dv[db]);
                dk[db] = mfma(read_tr_operand<BQB>(sm.qt[cur], d, 0, g), s0, dk[db]);
                dk[db] = mfma(read_tr_operand<BQB>(sm.qt[cur], d, 1, g), s1, dk[db]);
            }
        }
        if (it + 1 < total) stash(cur ^ 1);
        __syncthreads();
    }
    const float scale = 1.f / sqrtf((float)D);
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
            const int d = db * 32 + rg * 8 + g * 4;
            u32x2 vk, vv;
            vk[0] = uint32_t(f2bf(dk[db][rg * 4] * scale)) | (uint32_t(f2bf(dk[db][rg * 4 + 1] * scale)) << 16);
            vk[1] = uint32_t(f2bf(dk[db][rg * 4 + 2] * scale)) | (uint32_t(f2bf(dk[db][rg * 4 + 3] * scale)) << 16);
            vv[0] = uint32_t(f2bf(dv[db][rg * 4])) | (uint32_t(f2bf(dv[db][rg * 4 + 1])) << 16);
            vv[1] = uint32_t(f2bf(dv[db][rg * 4 + 2])) | (uint32_t(f2bf(dv[db][rg * 4 + 3])) << 16);
            *reinterpret_cast<u32x2*>(dqkv + (int64_t)key * ld + nq * D + grp * D + d) = vk;
            *reinterpret_cast<u32x2*>(dqkv + (int64_t)key * ld + (nq + nkv) * D + grp * D + d) = vv;
        }
}

bool shapes_ok(int T, int nq, int nkv) { return T > 0 && T % FQ == 0 && nq > 0 && nkv > 0 && nq % nkv == 0; }

}  // namespace

int32_t attn_fwd(const bf16_t* qkv, bf16_t* o, float* lse, int T, int nq, int nkv, hipStream_t s) {
    if (!shapes_ok(T, nq, nkv)) return fail(ZB_EINVAL, "attention: tokens must be a multiple of 128");
    hipLaunchKernelGGL(attn_fwd_kernel, dim3(T / FQ, nq), dim3(FTHR), 0, s, qkv, o, lse, T, nq, nkv);
    ZB_HIP(hipGetLastError());
    return ZB_OK;
}

int32_t attn_bwd(const bf16_t* qkv, const bf16_t* o, const float* lse, const bf16_t* dout, bf16_t* dqkv, float* delta,
                 int T, int nq, int nkv, hipStream_t s) {
    if (!shapes_ok(T, nq, nkv)) return fail(ZB_EINVAL, "attention: tokens must be a multiple of 128");
    hipLaunchKernelGGL(attn_delta_kernel, dim3((T * nq + 3) / 4), dim3(256), 0, s, o, dout, delta, T, nq);
    ZB_HIP(hipGetLastError());
    static bool attr_set = false;
    if (!attr_set) {
        ZB_HIP(hipFuncSetAttribute(reinterpret_cast<const void*>(attn_dq_kernel),
                                   hipFuncAttributeMaxDynamicSharedMemorySize, (int)sizeof(DqSmem)));
        ZB_HIP(hipFuncSetAttribute(reinterpret_cast<const void*>(attn_dkv_kernel),
                                   hipFuncAttributeMaxDynamicSharedMemorySize, (int)sizeof(DkvSmem)));
        attr_set = true;
    }
    hipLaunchKernelGGL(attn_dq_kernel, dim3(T / FQ, nq), dim3(FTHR), sizeof(DqSmem), s, qkv, dout, lse, delta, dqkv, T,
                       nq, nkv);
    ZB_HIP(hipGetLastError());
    hipLaunchKernelGGL(attn_dkv_kernel, dim3(T / BKV, nkv), dim3(FTHR), sizeof(DkvSmem), s, qkv, dout, lse, delta,
                       dqkv, T, nq, nkv);
    ZB_HIP(hipGetLastError());
    return ZB_OK;
}

}  // namespace zb
