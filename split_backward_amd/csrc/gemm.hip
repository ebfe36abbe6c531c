// GEMM kernels of the stage: F (Y = X W^T), B (dX = dY W) and W (dW += dY^T X).
//
// bf16 path: one CDNA4 kernel template, v_mfma_f32_32x32x16_bf16 with fp32
// accumulation.  Workgroup tile 256 x 256 x 64, 512 threads = 8 waves laid out
// 2 (M) x 4 (N); each wave owns a 128 x 64 sub-tile = 4 x 2 MFMA blocks.
// Both operands are staged through LDS in a "K-contiguous" layout ([row][64 k],
// 16-byte chunks XOR-swizzled so MFMA fragment reads and tile writes avoid
// bank conflicts), double buffered with one barrier per K step; the next
// K tile is fetched into registers while the current one is consumed.
//
// An operand that is contiguous along M or N in HBM (B's W operand, both
// operands of the W pass, where the reduction runs over tokens) is read as
// 4 (k) x 8 (m) blocks per thread and transposed in registers to 8 x 4 before
// it is written to LDS, so every pass feeds the same MFMA inner loop.
//
// The workgroup -> tile map is XCD aware: consecutive workgroup ids are
// spread over the 8 XCDs by the dispatcher, so tiles are renumbered such that
// each XCD works on a contiguous, M-grouped range (shared A/B panels stay in
// that XCD's L2).
//
// Epilogues fuse the activation forward/backward of the Guide's split
// ("Core Innovation 1"): GeLU(tanh) forward and backward, SwiGLU forward
// (paired gate/up tiles) and backward, the residual add and the in-place fp32
// weight-gradient accumulation of the W pass.
#include <cstdlib>

#include "common.h"

namespace zb {
namespace {

constexpr int BM = 256, BN = 256, BK = 64, NTHR = 512;
constexpr int TILE_ELEMS = 256 * BK;  // one operand tile in LDS (bf16 elements)

// 16-byte chunk index inside a 128-byte LDS row, XOR-swizzled by the row.
__device__ __forceinline__ int swz(int row, int chunk) { return chunk ^ ((row ^ (row >> 3)) & 7); }

__device__ __forceinline__ float gelu_tanh_f(float a) {
    const float c = 0.7978845608028654f, k = 0.044715f;
    float t = tanhf(c * (a + k * a * a * a));
    return 0.5f * a * (1.f + t);
}
__device__ __forceinline__ float gelu_tanh_grad_f(float a) {
    const float c = 0.7978845608028654f, k = 0.044715f;
    float t = tanhf(c * (a + k * a * a * a));
    return 0.5f * (1.f + t) + 0.5f * a * (1.f - t * t) * c * (1.f + 3.f * k * a * a);
}
__device__ __forceinline__ float sigmoid_f(float z) { return 1.f / (1.f + __expf(-z)); }

// Tile id for workgroup `bid`: spread over XCDs contiguously, then grouped
// along M in groups of G tile rows.
__device__ __forceinline__ void tile_of(int bid, int tiles_m, int tiles_n, int& tm, int& tn) {
    const int nwg = tiles_m * tiles_n;
    const int xcd = bid & 7, local = bid >> 3;
    const int q = nwg >> 3, r = nwg & 7;
    const int tile = (xcd < r) ? xcd * (q + 1) + local : r * (q + 1) + (xcd - r) * q + local;
    constexpr int G = 4;
    const int per_group = G * tiles_n;
    const int group = tile / per_group;
    const int first_m = group * G;
    const int gsize = min(tiles_m - first_m, G);
    const int in_group = tile - group * per_group;
    tm = first_m + in_group % gsize;
    tn = in_group / gsize;
}

// ---- global -> register loads ---------------------------------------------
// K-major operand: tile rows [row0, row0+256) x k [k0, k0+64).  Thread t loads
// 16-byte chunks c = t + 512 i: row c/8, chunk c%8.  `paired` maps tile rows
// 128..255 to rows half_n + ... (gate/up pairs of the SwiGLU forward).
template <bool PAIRED>
__device__ __forceinline__ void load_kmaj(u32x4 (&reg)[4], const bf16_t* __restrict__ base, int64_t ld,
                                          int row0, int rows_total, int half_n, int k0, int K, int tid) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int c = tid + i * NTHR;
        const int r = c >> 3, kc = c & 7;
        int grow;
        bool ok;
        if (PAIRED) {
            const int rr = row0 + (r & 127);
            ok = rr < half_n;
            grow = (r < 128) ? rr : half_n + rr;
        } else {
            grow = row0 + r;
            ok = grow < rows_total;
        }
        const int gk = k0 + kc * 8;
        if (ok && gk < K)
            reg[i] = *reinterpret_cast<const u32x4*>(base + (int64_t)grow * ld + gk);
        else
            reg[i] = u32x4{0u, 0u, 0u, 0u};
    }
}

__device__ __forceinline__ void store_kmaj(const u32x4 (&reg)[4], bf16_t* lds, int tid) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int c = tid + i * NTHR;
        const int r = c >> 3, kc = c & 7;
        *reinterpret_cast<u32x4*>(lds + r * BK + swz(r, kc) * 8) = reg[i];
    }
}

// M/N-major operand: HBM rows are k, columns are m.  Thread t covers k rows
// k0 + 4 g .. +3 (g = t/32) and columns col0 + 8 q .. +7 (q = t%32).
__device__ __forceinline__ void load_mnmaj(u32x4 (&reg)[4], const bf16_t* __restrict__ base, int64_t ld,
                                           int col0, int cols_total, int k0, int K, int tid) {
    const int g = tid >> 5, q = tid & 31;
    const int gc = col0 + q * 8;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int gk = k0 + g * 4 + r;
        if (gk < K && gc < cols_total)
            reg[r] = *reinterpret_cast<const u32x4*>(base + (int64_t)gk * ld + gc);
        else
            reg[r] = u32x4{0u, 0u, 0u, 0u};
    }
}

// Transpose the thread's 4 x 8 block to 8 rows of 4 k values and write them
// (8 bytes each) to the K-contiguous LDS tile.
__device__ __forceinline__ void store_mnmaj(const u32x4 (&reg)[4], bf16_t* lds, int tid) {
    const int g = tid >> 5, q = tid & 31;
    const int chunk = g >> 1, half = g & 1;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        const uint32_t a0 = reg[0][w], a1 = reg[1][w], a2 = reg[2][w], a3 = reg[3][w];
        const u32x2 lo{(a0 & 0xffffu) | (a1 << 16), (a2 & 0xffffu) | (a3 << 16)};
        const u32x2 hi{(a0 >> 16) | (a1 & 0xffff0000u), (a2 >> 16) | (a3 & 0xffff0000u)};
        const int r0 = q * 8 + 2 * w, r1 = r0 + 1;
        *reinterpret_cast<u32x2*>(lds + r0 * BK + swz(r0, chunk) * 8 + half * 4) = lo;
        *reinterpret_cast<u32x2*>(lds + r1 * BK + swz(r1, chunk) * 8 + half * 4) = hi;
    }
}

template <bool A_KMAJ, bool B_KMAJ, int EPI>
__global__ __launch_bounds__(NTHR) void gemm_bf16_kernel(GemmDesc d, int tiles_m, int tiles_n) {
    constexpr bool PAIRED = (EPI == EPI_SWIGLU_FWD);
    __shared__ __attribute__((aligned(16))) bf16_t smem[2 * 2 * TILE_ELEMS];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 2, wn = wave & 3;
    int tm, tn;
    tile_of(blockIdx.x, tiles_m, tiles_n, tm, tn);
    const int m0 = tm * BM;
    const int n0 = PAIRED ? tn * (BN / 2) : tn * BN;

    const bf16_t* __restrict__ A = reinterpret_cast<const bf16_t*>(d.A);
    const bf16_t* __restrict__ B = reinterpret_cast<const bf16_t*>(d.B);

    u32x4 ra[4], rb[4];
    auto fetch = [&](int k0) {
        if (A_KMAJ) load_kmaj<false>(ra, A, d.lda, m0, d.M, 0, k0, d.K, tid);
        else load_mnmaj(ra, A, d.lda, m0, d.M, k0, d.K, tid);
        if (B_KMAJ) load_kmaj<PAIRED>(rb, B, d.ldb, n0, d.N, d.half_n, k0, d.K, tid);
        else load_mnmaj(rb, B, d.ldb, n0, d.N, k0, d.K, tid);
    };
    auto stash = [&](int buf) {
        bf16_t* la = smem + buf * 2 * TILE_ELEMS;
        bf16_t* lb = la + TILE_ELEMS;
        if (A_KMAJ) store_kmaj(ra, la, tid); else store_mnmaj(ra, la, tid);
        if (B_KMAJ) store_kmaj(rb, lb, tid); else store_mnmaj(rb, lb, tid);
    };

    floatx16 acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

    const int nk = (d.K + BK - 1) / BK;
    fetch(0);
    stash(0);
    __syncthreads();

    const int lrow = lane & 31, lk = lane >> 5;
    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < nk) fetch((kt + 1) * BK);
        const bf16_t* la = smem + cur * 2 * TILE_ELEMS;
        const bf16_t* lb = la + TILE_ELEMS;
#pragma unroll
        for (int kk = 0; kk < BK / 16; ++kk) {
            const int chunk = kk * 2 + lk;
            bf16x8 fa[4], fb[2];
#pragma unroll
            for (int mi = 0; mi < 4; ++mi) {
                const int row = wm * 128 + mi * 32 + lrow;
                fa[mi] = *reinterpret_cast<const bf16x8*>(la + row * BK + swz(row, chunk) * 8);
            }
#pragma unroll
            for (int ni = 0; ni < 2; ++ni) {
                const int row = PAIRED ? (ni * 128 + wn * 32 + lrow) : (wn * 64 + ni * 32 + lrow);
                fb[ni] = *reinterpret_cast<const bf16x8*>(lb + row * BK + swz(row, chunk) * 8);
            }
#pragma unroll
            for (int mi = 0; mi < 4; ++mi)
#pragma unroll
                for (int ni = 0; ni < 2; ++ni)
                    acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[mi], fb[ni], acc[mi][ni], 0, 0, 0);
        }
        if (kt + 1 < nk) stash(cur ^ 1);
        __syncthreads();
    }

    // ---- epilogue: lane holds rows (r/4)*8 + (lane/32)*4 + r%4, column lane%32
    const int lcol = lane & 31;
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int row = m0 + wm * 128 + mi * 32 + (r >> 2) * 8 + lk * 4 + (r & 3);
            if (row >= d.M) continue;
            if (PAIRED) {
                const int col = n0 + wn * 32 + lcol;
                if (col >= d.half_n) continue;
                const float g = acc[mi][0][r], u = acc[mi][1][r];
                bf16_t* C = reinterpret_cast<bf16_t*>(d.C) + (int64_t)row * d.ldc;
                C[col] = f2bf(g);
                C[d.half_n + col] = f2bf(u);
                reinterpret_cast<bf16_t*>(d.C2)[(int64_t)row * d.ldc2 + col] = f2bf(g * sigmoid_f(g) * u);
                continue;
            }
#pragma unroll
            for (int ni = 0; ni < 2; ++ni) {
                const int col = n0 + wn * 64 + ni * 32 + lcol;
                if (col >= d.N) continue;
                const float v = acc[mi][ni][r];
                if (EPI == EPI_STORE) {
                    reinterpret_cast<bf16_t*>(d.C)[(int64_t)row * d.ldc + col] = f2bf(v);
                } else if (EPI == EPI_RESID) {
                    const float res = bf2f(reinterpret_cast<const bf16_t*>(d.R)[(int64_t)row * d.ldr + col]);
                    reinterpret_cast<bf16_t*>(d.C)[(int64_t)row * d.ldc + col] = f2bf(v + res);
                } else if (EPI == EPI_ACCUM_F32) {
                    float* c = reinterpret_cast<float*>(d.C) + (int64_t)row * d.ldc + col;
                    *c = *c + v;
                } else if (EPI == EPI_GELU_FWD) {
                    reinterpret_cast<bf16_t*>(d.C)[(int64_t)row * d.ldc + col] = f2bf(v);
                    reinterpret_cast<bf16_t*>(d.C2)[(int64_t)row * d.ldc2 + col] = f2bf(gelu_tanh_f(v));
                } else if (EPI == EPI_GELU_BWD) {
                    const float a = bf2f(reinterpret_cast<const bf16_t*>(d.R)[(int64_t)row * d.ldr + col]);
                    reinterpret_cast<bf16_t*>(d.C)[(int64_t)row * d.ldc + col] = f2bf(v * gelu_tanh_grad_f(a));
                } else if (EPI == EPI_SWIGLU_BWD) {
                    const bf16_t* R = reinterpret_cast<const bf16_t*>(d.R) + (int64_t)row * d.ldr;
                    const float g = bf2f(R[col]), u = bf2f(R[d.half_n + col]);
                    const float sg = sigmoid_f(g);
                    bf16_t* C = reinterpret_cast<bf16_t*>(d.C) + (int64_t)row * d.ldc;
                    C[col] = f2bf(v * u * sg * (1.f + g * (1.f - sg)));
                    C[d.half_n + col] = f2bf(v * g * sg);
                }
            }
        }
    }
}

template <bool AK, bool BKM>
int32_t launch_epi(const GemmDesc& d, hipStream_t s, int tiles_m, int tiles_n) {
    dim3 grid(tiles_m * tiles_n), block(NTHR);
    switch (d.epi) {
#define ZB_CASE(E) case E: hipLaunchKernelGGL((gemm_bf16_kernel<AK, BKM, E>), grid, block, 0, s, d, tiles_m, tiles_n); break;
        ZB_CASE(EPI_STORE)
        ZB_CASE(EPI_RESID)
        ZB_CASE(EPI_ACCUM_F32)
        ZB_CASE(EPI_GELU_FWD)
        ZB_CASE(EPI_GELU_BWD)
        ZB_CASE(EPI_SWIGLU_FWD)
        ZB_CASE(EPI_SWIGLU_BWD)
#undef ZB_CASE
        default: return fail(ZB_EINVAL, "gemm: unknown epilogue");
    }
    ZB_HIP(hipGetLastError());
    return ZB_OK;
}

// ---- fp32 path (the fp32 linear workload): LDS-tiled FMA GEMM ----------------
// 64 x 64 tile, K step 16, 256 threads with 4 x 4 outputs each.  Any operand
// layout; fp32 accumulation in the order k = 0, 1, ..., K-1 per output.
constexpr int FT = 64, FK = 16;

__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmDesc d, int accumulate) {
    __shared__ float As[FK][FT + 1];
    __shared__ float Bs[FK][FT + 1];
    const float* A = reinterpret_cast<const float*>(d.A);
    const float* B = reinterpret_cast<const float*>(d.B);
    float* C = reinterpret_cast<float*>(d.C);
    const int tid = threadIdx.x;
    const int m0 = blockIdx.y * FT, n0 = blockIdx.x * FT;
    const int tr = tid / 16, tc = tid % 16;
    float acc[4][4] = {};
    for (int k0 = 0; k0 < d.K; k0 += FK) {
        for (int e = tid; e < FK * FT; e += 256) {
            const int kk = e / FT, mm = e % FT;
            const int gm = m0 + mm, gk = k0 + kk;
            float av = 0.f, bv = 0.f;
            if (gm < d.M && gk < d.K)
                av = d.a_kmajor ? A[(int64_t)gm * d.lda + gk] : A[(int64_t)gk * d.lda + gm];
            const int gn = n0 + mm;
            if (gn < d.N && gk < d.K)
                bv = d.b_kmajor ? B[(int64_t)gn * d.ldb + gk] : B[(int64_t)gk * d.ldb + gn];
            As[kk][mm] = av;
            Bs[kk][mm] = bv;
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < FK; ++kk) {
            float a[4], b[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) a[i] = As[kk][tr + 16 * i];
#pragma unroll
            for (int j = 0; j < 4; ++j) b[j] = Bs[kk][tc + 16 * j];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int gm = m0 + tr + 16 * i, gn = n0 + tc + 16 * j;
            if (gm < d.M && gn < d.N) {
                float* c = C + (int64_t)gm * d.ldc + gn;
                *c = accumulate ? *c + acc[i][j] : acc[i][j];
            }
        }
}

}  // namespace

int32_t gemm_bf16(const GemmDesc& d, hipStream_t s) {
    if (d.M <= 0 || d.N <= 0 || d.K <= 0) return fail(ZB_EINVAL, "gemm_bf16: empty shape");
    if (d.K1 != 0) return fail(ZB_EINVAL, "gemm_bf16: a second K segment needs gemm_bf16_group_segmented");
    if (d.K % 8 || d.lda % 8 || d.ldb % 8) return fail(ZB_EINVAL, "gemm_bf16: K and leading dims must be multiples of 8");
    if ((!d.a_kmajor && d.M % 8) || (!d.b_kmajor && d.N % 8))
        return fail(ZB_EINVAL, "gemm_bf16: contiguous M/N extent must be a multiple of 8");
    if ((reinterpret_cast<uintptr_t>(d.A) | reinterpret_cast<uintptr_t>(d.B)) & 15)
        return fail(ZB_EINVAL, "gemm_bf16: operands must be 16-byte aligned");
    const bool paired = d.epi == EPI_SWIGLU_FWD;
    if (paired && (!d.b_kmajor || d.half_n <= 0)) return fail(ZB_EINVAL, "gemm_bf16: bad SwiGLU pairing");
    static const bool force_v1 = getenv("ZB_GEMM_V1") != nullptr;
    if (!force_v1) {
        bool handled = false;
        const int32_t rc = gemm_bf16_v2(d, s, &handled);
        if (handled || rc != ZB_OK) return rc;
    }
    const int tiles_m = (d.M + BM - 1) / BM;
    const int tiles_n = paired ? (d.half_n + BN / 2 - 1) / (BN / 2) : (d.N + BN - 1) / BN;
    if (d.a_kmajor && d.b_kmajor) return launch_epi<true, true>(d, s, tiles_m, tiles_n);
    if (d.a_kmajor && !d.b_kmajor) return launch_epi<true, false>(d, s, tiles_m, tiles_n);
    if (!d.a_kmajor && !d.b_kmajor) return launch_epi<false, false>(d, s, tiles_m, tiles_n);
    return launch_epi<false, true>(d, s, tiles_m, tiles_n);
}

int32_t gemm_f32(const GemmDesc& d, int accumulate, hipStream_t s) {
    if (d.M <= 0 || d.N <= 0 || d.K <= 0) return fail(ZB_EINVAL, "gemm_f32: empty shape");
    if (d.K1 != 0) return fail(ZB_EINVAL, "gemm_f32: no second K segment");
    dim3 grid((d.N + FT - 1) / FT, (d.M + FT - 1) / FT), block(256);
    hipLaunchKernelGGL(gemm_f32_kernel, grid, block, 0, s, d, accumulate);
    ZB_HIP(hipGetLastError());
    return ZB_OK;
}

}  // namespace zb
