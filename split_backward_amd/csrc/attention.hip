// Causal grouped-query attention core of the Llama stage (head_dim 128), a
// weightless op: its forward runs in F and its whole backward in B.
//
//   S = q k^T / sqrt(d) (key index <= query index),  P = softmax(S),  o = P v
//   dP = do v^T,  dS = P (dP - rowsum(do o)),  dq = dS k / sqrt(d),
//   dk = dS^T q / sqrt(d),  dv = P^T do   (dk, dv summed over each KV group)
//
// CDNA4 design.  Every product is a v_mfma_f32_32x32x16_bf16.  The wave
// index is read into a scalar register so that LDS DMA destinations (M0) are
// computed by scalar instructions.
// * Tiles of K, V (forward, dq) and of Q, dO (dk/dv) are DMA'd HBM -> LDS
//   with buffer_load ... lds in their natural [rows][128 d] layout (256-byte
//   rows, 16-byte chunks XOR-swizzled by the row), double buffered.
// * Operands whose reduction index is the row of such a tile (V^T in o,
//   K^T in dq, dO^T and Q^T in dv / dk) are read with the gfx950 transpose
//   read ds_read_b64_tr_b16; the row addresses are chosen so the lane receives
//   the keys (or queries) in exactly the order the score accumulator holds
//   them (8(s/4) + 4g + s%4 within a 16-row step), so probabilities go from
//   the accumulator into the next MFMA without any shuffle.
// * The forward and dq kernels compute the transposed score block S^T = K Q^T:
//   each lane owns one query column, so softmax statistics are per-lane
//   scalars combined with the partner lane 32 away.  The forward rescales its
//   running output only when a row maximum grows by more than 2^8 (exact:
//   output and normaliser always share one reference maximum), and skips the
//   rescale entirely when no lane of the wave needs it.
// * The dk/dv kernel owns a key block per workgroup and sweeps query blocks,
//   accumulating dK^T and dV^T in registers: no atomics, deterministic.
// Softmax runs in fp32 in base 2; the stashed row statistic is
// lse2 = max + log2(sum) of the scaled scores.
#include "common.h"

namespace zb {
namespace {

constexpr int D = 128;          // head dim
constexpr float LOG2E = 1.4426950408889634f;
constexpr float RESCALE_TAU = 8.0f;  // log2 growth of a row max tolerated without rescaling

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8;
constexpr uint32_t OOB = 0x80000000u;

__device__ __forceinline__ floatx16 zero16() {
    floatx16 z;
#pragma unroll
    for (int i = 0; i < 16; ++i) z[i] = 0.f;
    return z;
}

// 2^x with the hardware instruction alone: results below 2^-126 flush to
// zero, which is harmless for softmax weights (exp2f adds a denormal range
// fix-up of four more instructions per call).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ floatx16 mfma(const bf16x8& a, const bf16x8& b, const floatx16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}

// Accumulator slots [8h, 8h+8) of a 32x32 block as a bf16 operand: slot s of
// lane group g holds row 16h + 8(s/4) + 4g + s%4 of the block.
__device__ __forceinline__ bf16x8 acc_half_to_bf16(const floatx16& c, int half) {
    const int b = half * 8;
    bf16x8 v;
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = (__bf16)c[b + i];
    return v;
}

// ---- [rows][128] tiles in LDS ---------------------------------------------
// 256-byte rows of 16 chunks (16 B); chunk c of row r sits at c ^ swz(r).
// With b_i the bits of r, swz = (b0^b1^b3, b0, b1, b2) is a bijection of the
// low 4 row bits (row reads: 8 or 16 consecutive rows at one chunk hit
// distinct bank windows), and for the 4 consecutive rows a 16-lane group of a
// transpose read touches, bits (2,1) and bits (3,2) of swz are bijections of
// (b1, b0), so their 32-byte pieces also hit distinct windows for 32 and 64
// four-byte banks.  It depends on r & 15 only.
__device__ __forceinline__ int swz(int r) {
    const int b0 = r & 1, b1 = (r >> 1) & 1, b2 = (r >> 2) & 1, b3 = (r >> 3) & 1;
    return ((b0 ^ b1 ^ b3) << 3) | (b0 << 2) | (b1 << 1) | b2;
}
__device__ __forceinline__ uint32_t tile_off(int row, int chunk) { return row * 256 + ((chunk ^ swz(row)) << 4); }

// DMA of `rows` rows (multiple of 16) starting at global row `row0` of a
// [*, ld] bf16 matrix, columns col0..col0+127, into `tile`.  Each wave
// instruction writes 1 KB = 4 rows; instruction i of wave w covers rows
// 4(nw*i + w) .. +3.  Rows >= rows_total read as zero.  A call that is not
// `live` issues the same instructions over an empty range (zeros, no memory
// traffic), which keeps every wave's count of outstanding loads uniform.
template <int ROWS, int NW>
__device__ __forceinline__ void dma_rows(const bf16_t* base, int64_t ld, int row0, int rows_total, int col0,
                                         lds_void* tile, int lane, int wave, bool live = true) {
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(base, live ? 0x7fffffffu : 0u);
#pragma unroll
    for (int i = 0; i < ROWS / 4 / NW; ++i) {
        const int b = NW * i + wave;
        const int r = b * 4 + (lane >> 4);
        const int chunk = (lane & 15) ^ swz(r);
        const int grow = row0 + r;
        const uint32_t off = grow < rows_total ? (uint32_t)(((int64_t)grow * ld + col0 + chunk * 8) * 2) : OOB;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)((lds_char*)tile + b * 1024), 16, off, 0, 0, 0);
    }
}

// Row fragment: row `row`, 8 consecutive d at 16 kk + 8 g.
__device__ __forceinline__ bf16x8 frag_row(const lds_void* tile, int row, int kk, int g) {
    return *(const lds_bf16x8*)((const lds_char*)tile + tile_off(row, kk * 2 + g));
}

// Transposed fragment: column d = dblk*32 + lane%32 of the tile, reduction
// over tile rows 16 t + 8(s/4) + 4g + s%4 (slot s, g = lane/32), i.e. the
// score-accumulator order.  Two ds_read_b64_tr_b16: in each 16-lane group
// the lane j reads 4 columns at row offset j/4; output lane i, slot s takes
// column i of the row read by lane 4s + i/4.  The row's low 4 bits do not
// depend on t, so the per-lane byte offsets of (dblk, lo/hi) are computed
// once (tr_bases) and t enters as the instruction's immediate offset.
struct TrBases {
    uint32_t lo[4], hi[4];
};
__device__ __forceinline__ TrBases tr_bases(int lane) {
    const int G = lane >> 4, j = lane & 15;
    const int s = j >> 2, q = j & 3;
    const int row_lo = (G >> 1) * 4 + s, row_hi = row_lo + 8;
    TrBases b;
#pragma unroll
    for (int db = 0; db < 4; ++db) {
        const int d = db * 32 + (G & 1) * 16 + q * 4;
        b.lo[db] = row_lo * 256 + (((d >> 3) ^ swz(row_lo)) << 4) + (d & 7) * 2;
        b.hi[db] = row_hi * 256 + (((d >> 3) ^ swz(row_hi)) << 4) + (d & 7) * 2;
    }
    return b;
}
template <int T16>
__device__ __forceinline__ bf16x8 frag_tr(uint32_t tile, const TrBases& b, int db) {
    u32x2 lo, hi;
    asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(lo) : "v"(tile + b.lo[db]), "i"(T16 * 4096));
    asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(hi) : "v"(tile + b.hi[db]), "i"(T16 * 4096));
    return __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
}

// Wait for all LDS reads; `v` becomes an output so its uses stay below.
template <int N>
__device__ __forceinline__ void lds_wait(bf16x8 (&v)[N]) {
#pragma unroll
    for (int i = 0; i < N; ++i) asm volatile("" : "+v"(v[i]));
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int i = 0; i < N; ++i) asm volatile("" : "+v"(v[i]));
}

// s_waitcnt lgkmcnt(N) (N a compile-time count of LDS reads allowed to stay
// in flight); the fragments passed become outputs of the wait so their uses
// stay below it.  Only LDS reads issued by this code are outstanding where
// it is used (no scalar memory loads), so the in-order count is exact.
template <int N>
__device__ __forceinline__ void lgkm_wait() {
    static_assert(N >= 0 && N <= 15, "lgkmcnt");
    if constexpr (N == 0) asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    else if constexpr (N == 1) asm volatile("s_waitcnt lgkmcnt(1)" ::: "memory");
    else if constexpr (N == 2) asm volatile("s_waitcnt lgkmcnt(2)" ::: "memory");
    else if constexpr (N == 3) asm volatile("s_waitcnt lgkmcnt(3)" ::: "memory");
    else if constexpr (N == 4) asm volatile("s_waitcnt lgkmcnt(4)" ::: "memory");
    else if constexpr (N == 6) asm volatile("s_waitcnt lgkmcnt(6)" ::: "memory");
    else if constexpr (N == 8) asm volatile("s_waitcnt lgkmcnt(8)" ::: "memory");
    else static_assert(N == 0, "unsupported lgkmcnt");
}
template <typename F>
__device__ __forceinline__ void pin(F& f) {
    asm volatile("" : "+v"(f));
}
template <int N, typename... F>
__device__ __forceinline__ void lds_wait_keep(F&... f) {
    (pin(f), ...);
    lgkm_wait<N>();
    (pin(f), ...);
}

// s_waitcnt vmcnt(N) for a compile-time N.
template <int N>
__device__ __forceinline__ void vm_wait() {
    if constexpr (N == 0) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    else if constexpr (N == 6) asm volatile("s_waitcnt vmcnt(6)" ::: "memory");
    else if constexpr (N == 8) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
    else if constexpr (N == 12) asm volatile("s_waitcnt vmcnt(12)" ::: "memory");
    else if constexpr (N == 16) asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
    else if constexpr (N == 18) asm volatile("s_waitcnt vmcnt(18)" ::: "memory");
    else if constexpr (N == 24) asm volatile("s_waitcnt vmcnt(24)" ::: "memory");
    else static_assert(N == 0, "unsupported vmcnt");
}

__device__ __forceinline__ void wg_barrier() { asm volatile("s_barrier" ::: "memory"); }

// ======================================================== forward ========
constexpr int FQ = 128, FKV = 64, FTHR = 256;
constexpr int KV_TILE = FKV * D * 2;  // 16 KB

// One query block qb (128 queries) of head blockIdx.y.
__device__ __forceinline__ void attn_fwd_block(int qb, char (*sm)[2 * KV_TILE], const bf16_t* __restrict__ qkv,
                                               bf16_t* __restrict__ o, float* __restrict__ lse, int T, int nq,
                                               int nkv) {
    const int ld = (nq + 2 * nkv) * D;
    const int h = blockIdx.y;
    const int grp = h / (nq / nkv);
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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
    const TrBases trb = tr_bases(lane);
    const float c = LOG2E / sqrtf((float)D);

    const int nkb = (qb * FQ + FQ) / FKV;
    auto dma = [&](int kb) {
        char* st = sm[kb & 1];
        dma_rows<FKV, 4>(kbase, ld, kb * FKV, T, 0, (lds_void*)st, lane, wave);
        dma_rows<FKV, 4>(vbase, ld, kb * FKV, T, 0, (lds_void*)(st + KV_TILE), lane, wave);
    };
    dma(0);
    for (int kb = 0; kb < nkb; ++kb) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        wg_barrier();  // tile kb landed for every wave; the other stage is free
        if (kb + 1 < nkb) dma(kb + 1);
        const int k0 = kb * FKV;
        if (k0 > qw0 + 31) continue;  // every key of this block is in the future of every query of the wave
        const lds_void* kt = (const lds_void*)sm[kb & 1];
        const lds_void* vt = (const lds_void*)(sm[kb & 1] + KV_TILE);
        floatx16 s[2];
        s[0] = s[1] = zero16();
        {
            // K row fragment of step (j, kk) + 1 is read while step (j, kk) multiplies
            const uint32_t ka = (uint32_t)(uintptr_t)kt;
            bf16x8 fk[2];
            auto rd = [&](int st, int slot) {
                asm volatile("ds_read_b128 %0, %1" : "=v"(fk[slot]) : "v"(ka + tile_off((st >> 3) * 32 + col, (st & 7) * 2 + g)));
            };
            rd(0, 0);
#pragma unroll
            for (int st = 0; st < 16; ++st) {
                const int cur = st & 1;
                if (st + 1 < 16) {
                    rd(st + 1, cur ^ 1);
                    lds_wait_keep<1>(fk[cur]);
                } else {
                    lds_wait_keep<0>(fk[cur]);
                }
                s[st >> 3] = mfma(fk[cur], qf[st & 7], s[st >> 3]);
            }
        }
        if (k0 + FKV - 1 > qw0) {  // diagonal block: mask keys after the query
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = k0 + j * 32 + (r >> 2) * 8 + g * 4 + (r & 3);
                    if (key > q) s[j][r] = -INFINITY;
                }
        }
        float mx = -INFINITY;
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[j][r]);
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64)) * c;
        const bool grow = mx > m + RESCALE_TAU;
        if (__any(grow)) {  // rare after the first block
            const float mnew = grow ? mx : m;
            const float alpha = fast_exp2(m - mnew);
            l *= alpha;
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int e = 0; e < 16; ++e) oacc[i][e] *= alpha;
            m = mnew;
        }
        float rs = 0.f;
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float p = fast_exp2(fmaf(s[j][r], c, -m));
                s[j][r] = p;
                rs += p;
            }
        l += rs + __shfl_xor(rs, 32, 64);
        bf16x8 pb[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) pb[t] = acc_half_to_bf16(s[t >> 1], t & 1);
        const uint32_t vaddr = (uint32_t)(uintptr_t)vt;
        {
            // V^T fragments of d block db + 1 are read while block db multiplies
            bf16x8 vf[2][4];
            auto rd = [&](int db) {
                vf[db & 1][0] = frag_tr<0>(vaddr, trb, db);
                vf[db & 1][1] = frag_tr<1>(vaddr, trb, db);
                vf[db & 1][2] = frag_tr<2>(vaddr, trb, db);
                vf[db & 1][3] = frag_tr<3>(vaddr, trb, db);
            };
            rd(0);
#pragma unroll
            for (int db = 0; db < 4; ++db) {
                bf16x8(&cur)[4] = vf[db & 1];
                if (db + 1 < 4) {
                    rd(db + 1);
                    lds_wait_keep<8>(cur[0], cur[1], cur[2], cur[3]);
                } else {
                    lds_wait_keep<0>(cur[0], cur[1], cur[2], cur[3]);
                }
#pragma unroll
                for (int t = 0; t < 4; ++t) oacc[db] = mfma(cur[t], pb[t], oacc[db]);
            }
        }
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

// Causal query blocks differ in length up to nb-fold: each workgroup runs
// block nb-1-x and then its mirror x, so every workgroup does the same work
// and the two resident per CU finish together.
__global__ __launch_bounds__(FTHR, 2) void attn_fwd_kernel(const bf16_t* __restrict__ qkv, bf16_t* __restrict__ o,
                                                           float* __restrict__ lse, int T, int nq, int nkv) {
    __shared__ __attribute__((aligned(1024))) char sm[2][2 * KV_TILE];  // [stage][K | V]
    const int nb = T / FQ;
    const int a = nb - 1 - (int)blockIdx.x, b = (int)blockIdx.x;
    for (int pass = 0; pass < (b < a ? 2 : 1); ++pass) {
        if (pass) wg_barrier();  // every wave is done with the stages
        attn_fwd_block(pass ? b : a, sm, qkv, o, lse, T, nq, nkv);
    }
}

// ====================================================== dq kernel ========
// Per (query block of 128, query head).  Mirrors the forward: S^T = K Q^T,
// dP^T = V dO^T, dS^T = P^T (dP^T - delta), dQ^T += K^T dS^T.
// Two workgroups per CU as in the dk/dv kernel (64 KB of LDS each).
constexpr int DQ_STAGES = 2;
__device__ __forceinline__ void attn_dq_block(int qb, char (*sm)[2 * KV_TILE], const bf16_t* __restrict__ qkv,
                                              const bf16_t* __restrict__ o, const bf16_t* __restrict__ dout,
                                              const float* __restrict__ lse, float* __restrict__ delta,
                                              bf16_t* __restrict__ dqkv, int T, int nq, int nkv) {
    const int ld = (nq + 2 * nkv) * D;
    const int h = blockIdx.y;
    const int grp = h / (nq / nkv);
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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
    // delta = rowsum(dO o) of the lane's query: half of the row's 128 products
    // in each of the lanes q and q+32; stored for the dk/dv kernel.
    float dsum = 0.f;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
        const bf16x8 ov = *reinterpret_cast<const bf16x8*>(o + (int64_t)q * ldo + h * D + kk * 16 + g * 8);
#pragma unroll
        for (int e = 0; e < 8; ++e) dsum = fmaf((float)ov[e], (float)dof[kk][e], dsum);
    }
    dsum += __shfl_xor(dsum, 32, 64);
    const float dq_delta = dsum;
    if (g == 0) delta[(int64_t)h * T + q] = dsum;
    const float c = LOG2E / sqrtf((float)D);

    floatx16 dacc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) dacc[i] = zero16();
    const TrBases trb = tr_bases(lane);

    const int nkb = (qb * FQ + FQ) / FKV;
    // Ring of DQ_STAGES K/V blocks: the DMA of blocks kb+1 .. kb+DQ_STAGES-1
    // is issued while block kb is used (8 loads per wave per block; blocks
    // past the last are empty).
    auto dma = [&](int kb) {
        char* st = sm[kb % DQ_STAGES];
        const bool live = kb < nkb;
        dma_rows<FKV, 4>(kbase, ld, kb * FKV, T, 0, (lds_void*)st, lane, wave, live);
        dma_rows<FKV, 4>(vbase, ld, kb * FKV, T, 0, (lds_void*)(st + KV_TILE), lane, wave, live);
    };
#pragma unroll
    for (int t = 0; t < DQ_STAGES - 1; ++t) dma(t);
    for (int kb = 0; kb < nkb; ++kb) {
        vm_wait<8 * (DQ_STAGES - 2)>();  // block kb landed
        wg_barrier();
        dma(kb + DQ_STAGES - 1);  // into the stage block kb-1 used
        const int k0 = kb * FKV;
        if (k0 > qw0 + 31) continue;
        const lds_void* kt = (const lds_void*)sm[kb % DQ_STAGES];
        const lds_void* vt = (const lds_void*)(sm[kb % DQ_STAGES] + KV_TILE);
        floatx16 s[2], dp[2];
        s[0] = s[1] = dp[0] = dp[1] = zero16();
        {
            // K and V row fragments of step (j, kk) + 1 are read while step (j, kk) multiplies
            const uint32_t ka = (uint32_t)(uintptr_t)kt;
            bf16x8 fk[2], fv[2];
            auto rd = [&](int st, int slot) {
                const uint32_t ro = tile_off((st >> 3) * 32 + col, (st & 7) * 2 + g);
                asm volatile("ds_read_b128 %0, %1" : "=v"(fk[slot]) : "v"(ka + ro));
                asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(fv[slot]) : "v"(ka + ro), "i"(KV_TILE));
            };
            rd(0, 0);
#pragma unroll
            for (int st = 0; st < 16; ++st) {
                const int cur = st & 1, j = st >> 3, kk = st & 7;
                if (st + 1 < 16) {
                    rd(st + 1, cur ^ 1);
                    lds_wait_keep<2>(fk[cur], fv[cur]);
                } else {
                    lds_wait_keep<0>(fk[cur], fv[cur]);
                }
                s[j] = mfma(fk[cur], qf[kk], s[j]);
                dp[j] = mfma(fv[cur], dof[kk], dp[j]);
            }
        }
        const bool diag = (k0 + FKV - 1 > qw0);
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float p = fast_exp2(fmaf(s[j][r], c, -lq));
                if (diag) {
                    const int key = k0 + j * 32 + (r >> 2) * 8 + g * 4 + (r & 3);
                    if (key > q) p = 0.f;
                }
                s[j][r] = p * (dp[j][r] - dq_delta);  // dS^T
            }
        bf16x8 sb[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) sb[t] = acc_half_to_bf16(s[t >> 1], t & 1);
        const uint32_t kaddr = (uint32_t)(uintptr_t)kt;
        {
            // K^T fragments of d block db, read one block ahead (8 reads each)
            bf16x8 kf[2][4];
            auto rd = [&](int db) {
                kf[db & 1][0] = frag_tr<0>(kaddr, trb, db);
                kf[db & 1][1] = frag_tr<1>(kaddr, trb, db);
                kf[db & 1][2] = frag_tr<2>(kaddr, trb, db);
                kf[db & 1][3] = frag_tr<3>(kaddr, trb, db);
            };
            rd(0);
#pragma unroll
            for (int db = 0; db < 4; ++db) {
                bf16x8(&cur)[4] = kf[db & 1];
                if (db + 1 < 4) {
                    rd(db + 1);
                    lds_wait_keep<8>(cur[0], cur[1], cur[2], cur[3]);
                } else {
                    lds_wait_keep<0>(cur[0], cur[1], cur[2], cur[3]);
                }
#pragma unroll
                for (int t = 0; t < 4; ++t) dacc[db] = mfma(cur[t], sb[t], dacc[db]);
            }
        }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the empty trailing blocks still write LDS
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

// Paired query blocks as in the forward kernel.
__global__ __launch_bounds__(FTHR, 2) void attn_dq_kernel(const bf16_t* __restrict__ qkv,
                                                          const bf16_t* __restrict__ o,
                                                          const bf16_t* __restrict__ dout,
                                                          const float* __restrict__ lse,
                                                          float* __restrict__ delta,
                                                          bf16_t* __restrict__ dqkv, int T, int nq, int nkv) {
    __shared__ __attribute__((aligned(1024))) char sm[DQ_STAGES][2 * KV_TILE];
    const int nb = T / FQ;
    const int a = nb - 1 - (int)blockIdx.x, b = (int)blockIdx.x;
    for (int pass = 0; pass < (b < a ? 2 : 1); ++pass) {
        if (pass) wg_barrier();
        attn_dq_block(pass ? b : a, sm, qkv, o, dout, lse, delta, dqkv, T, nq, nkv);
    }
}

// ===================================================== dk / dv kernel ====
// Per (key block of 128, KV head).  Each wave owns 32 keys (K and V rows in
// registers as B operands).  Sweeps the query heads of the group and the
// query blocks of 32 rows at or after the diagonal:
//   S = Q K^T, P = exp2(S c - lse2), dP = dO V^T, dS = P (dP - delta),
//   dV^T += dO^T P,  dK^T += Q^T dS.
constexpr int BKV = 128, BQB = 32;
constexpr int Q_TILE = BQB * D * 2;  // 8 KB
// Two workgroups per CU (two waves per SIMD, at most 256 registers per
// lane, 64.5 KB of LDS each): one workgroup's softmax, barrier and LDS
// latency overlap the other's MFMAs.  Double-buffered query blocks suffice
// with that overlap.
constexpr int KV_STAGES = 2;

__device__ __forceinline__ void attn_dkv_block(int kb, char (*sm)[2 * Q_TILE], char* svt, float (*sl)[2][BQB],
                                               const bf16_t* __restrict__ qkv, const bf16_t* __restrict__ dout,
                                               const float* __restrict__ lse, const float* __restrict__ delta,
                                               bf16_t* __restrict__ dqkv, float* __restrict__ part, int T, int nq,
                                               int nkv) {
    const int ld = (nq + 2 * nkv) * D;
    const int ldo = nq * D;
    const int grp = blockIdx.y;
    // The group's query heads split over gridDim.z workgroups (head subset
    // blockIdx.z); with more than one, each writes fp32 partial dK, dV to
    // `part` and attn_dkv_reduce_kernel adds them in subset order.
    const int rep = nq / nkv / (int)gridDim.z;
    const int head0 = (grp * (int)gridDim.z + (int)blockIdx.z) * rep;
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 5, col = lane & 31;
    const int kw0 = kb * BKV + wave * 32;
    const int key = kw0 + col;

    // K rows of the wave's keys stay in registers; V rows of the block's 128
    // keys go to LDS once (8 loads per wave, waited for with the first block).
    bf16x8 kf[8];
#pragma unroll
    for (int kk = 0; kk < 8; ++kk)
        kf[kk] = *reinterpret_cast<const bf16x8*>(qkv + (int64_t)key * ld + nq * D + grp * D + kk * 16 + g * 8);
    dma_rows<BKV, 4>(qkv + (nq + nkv) * D + grp * D, ld, kb * BKV, T, 0, (lds_void*)svt, lane, wave);
    floatx16 dk[4], dv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        dk[i] = zero16();
        dv[i] = zero16();
    }
    const float c = LOG2E / sqrtf((float)D);
    const TrBases trb = tr_bases(lane);
    const int qb0 = (kb * BKV) / BQB;
    const int nqb = T / BQB;
    const int per_head = nqb - qb0;
    const int total = per_head * rep;

    // Ring of KV_STAGES query blocks: the DMA of blocks it+1 .. it+KV_STAGES-1
    // is issued while block it is used.  Every wave issues 6 loads per block
    // (2 + 2 DMA of Q and dO, and the 32 row statistics of lse and delta,
    // written identically by each wave's lanes 0..31); blocks past the last
    // are empty.
    auto fetch = [&](int it) {
        const bool live = it < total;
        const int itc = live ? it : 0;
        const int hh = head0 + itc / per_head;
        const int q0 = (qb0 + itc % per_head) * BQB;
        char* st = sm[it % KV_STAGES];
        dma_rows<BQB, 4>(qkv + hh * D, ld, q0, T, 0, (lds_void*)st, lane, wave, live);
        dma_rows<BQB, 4>(dout + hh * D, ldo, q0, T, 0, (lds_void*)(st + Q_TILE), lane, wave, live);
        if (lane < BQB) {
            const __amdgpu_buffer_rsrc_t rl = make_rsrc(lse + (int64_t)hh * T + q0, live ? BQB * 4 : 0);
            const __amdgpu_buffer_rsrc_t rd = make_rsrc(delta + (int64_t)hh * T + q0, live ? BQB * 4 : 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rl, (lds_void*)&sl[it % KV_STAGES][0][0], 4, lane * 4, 0, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rd, (lds_void*)&sl[it % KV_STAGES][1][0], 4, lane * 4, 0, 0, 0);
        }
    };

#pragma unroll
    for (int t = 0; t < KV_STAGES - 1; ++t) fetch(t);
    for (int it = 0; it < total; ++it) {
        vm_wait<6 * (KV_STAGES - 2)>();  // block it landed
        wg_barrier();
        fetch(it + KV_STAGES - 1);  // into the stage block it-1 used
        const int q0 = (qb0 + it % per_head) * BQB;
        if (q0 + BQB - 1 < kw0) continue;  // every query of the block precedes every key of the wave
        const int stg = it % KV_STAGES;
        const lds_void* qt = (const lds_void*)sm[stg];
        const lds_void* ot = (const lds_void*)(sm[stg] + Q_TILE);
        // Fragment reads as asm (explicit waits): the compiler would otherwise
        // wait for the DMA of the next block, issued just above, before them.
        floatx16 s = zero16(), dp = zero16();
        {
            const uint32_t qa = (uint32_t)(uintptr_t)qt, va = (uint32_t)(uintptr_t)svt + wave * 32 * 256;
            // Q, dO and V row fragments of k step kk + 1 are read while step kk multiplies
            bf16x8 fq[2], fo[2], fv[2];
            auto rd = [&](int kk, int slot) {
                const uint32_t ro = tile_off(col, kk * 2 + g);
                asm volatile("ds_read_b128 %0, %1" : "=v"(fq[slot]) : "v"(qa + ro));
                asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(fo[slot]) : "v"(qa + ro), "i"(Q_TILE));
                asm volatile("ds_read_b128 %0, %1" : "=v"(fv[slot]) : "v"(va + ro));
            };
            rd(0, 0);
#pragma unroll
            for (int kk = 0; kk < 8; ++kk) {
                const int cur = kk & 1;
                if (kk + 1 < 8) {
                    rd(kk + 1, cur ^ 1);
                    lds_wait_keep<3>(fq[cur], fo[cur], fv[cur]);
                } else {
                    lds_wait_keep<0>(fq[cur], fo[cur], fv[cur]);
                }
                s = mfma(fq[cur], kf[kk], s);
                dp = mfma(fo[cur], fv[cur], dp);
            }
        }
        const bool diag = (q0 < kw0 + 31);
        // row statistics of the accumulator rows (r/4)*8 + 4g + r%4, 16-byte
        // reads issued as asm (see frag_tr), two row groups at a time
        const uint32_t lb = (uint32_t)(uintptr_t)&sl[stg][0][0] + g * 16;
        const uint32_t db = (uint32_t)(uintptr_t)&sl[stg][1][0] + g * 16;
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) {
            floatx4 lsv, dsv;
            asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(lsv) : "v"(lb), "i"(rb * 32));
            asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(dsv) : "v"(db), "i"(rb * 32));
            lds_wait_keep<0>(lsv, dsv);
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const int r = rb * 4 + r4;
                const int qr = rb * 8 + g * 4 + r4;
                float p = fast_exp2(fmaf(s[r], c, -lsv[r4]));
                if (diag && key > q0 + qr) p = 0.f;
                s[r] = p;
                dp[r] = p * (dp[r] - dsv[r4]);
            }
        }
        const bf16x8 p0 = acc_half_to_bf16(s, 0), p1 = acc_half_to_bf16(s, 1);
        const bf16x8 s0 = acc_half_to_bf16(dp, 0), s1 = acc_half_to_bf16(dp, 1);
        const uint32_t oaddr = (uint32_t)(uintptr_t)ot, qaddr = (uint32_t)(uintptr_t)qt;
        {
            // dO^T and Q^T fragments of d block db, read one block ahead
            bf16x8 fr[2][4];
            auto rd = [&](int db) {
                fr[db & 1][0] = frag_tr<0>(oaddr, trb, db);
                fr[db & 1][1] = frag_tr<1>(oaddr, trb, db);
                fr[db & 1][2] = frag_tr<0>(qaddr, trb, db);
                fr[db & 1][3] = frag_tr<1>(qaddr, trb, db);
            };
            rd(0);
#pragma unroll
            for (int db = 0; db < 4; ++db) {
                bf16x8(&cur)[4] = fr[db & 1];
                if (db + 1 < 4) {
                    rd(db + 1);
                    lds_wait_keep<8>(cur[0], cur[1], cur[2], cur[3]);
                } else {
                    lds_wait_keep<0>(cur[0], cur[1], cur[2], cur[3]);
                }
                dv[db] = mfma(cur[0], p0, dv[db]);
                dv[db] = mfma(cur[1], p1, dv[db]);
                dk[db] = mfma(cur[2], s0, dk[db]);
                dk[db] = mfma(cur[3], s1, dk[db]);
            }
        }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the empty trailing blocks still write LDS
    if (part) {  // fp32 partials [subset][key][kv head][dK | dV][D], dK not yet scaled
        float* pk = part + (((int64_t)blockIdx.z * T + key) * nkv + grp) * 2 * D;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int rg = 0; rg < 4; ++rg) {
                const int d = db * 32 + rg * 8 + g * 4;
                *reinterpret_cast<floatx4*>(pk + d) =
                    floatx4{dk[db][rg * 4], dk[db][rg * 4 + 1], dk[db][rg * 4 + 2], dk[db][rg * 4 + 3]};
                *reinterpret_cast<floatx4*>(pk + D + d) =
                    floatx4{dv[db][rg * 4], dv[db][rg * 4 + 1], dv[db][rg * 4 + 2], dv[db][rg * 4 + 3]};
            }
        return;
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

// Key block kb sweeps the query blocks at or after it: pairs kb with its
// mirror so every workgroup does the same work.
__global__ __launch_bounds__(FTHR, 2) void attn_dkv_kernel(const bf16_t* __restrict__ qkv,
                                                           const bf16_t* __restrict__ dout,
                                                           const float* __restrict__ lse,
                                                           const float* __restrict__ delta,
                                                           bf16_t* __restrict__ dqkv, float* __restrict__ part,
                                                           int T, int nq, int nkv) {
    __shared__ __attribute__((aligned(1024))) char sm[KV_STAGES][2 * Q_TILE];  // [stage][Q | dO]
    __shared__ __attribute__((aligned(1024))) char svt[BKV * D * 2];           // V rows of the block
    __shared__ float sl[KV_STAGES][2][BQB];                                     // [stage][lse | delta]
    const int nb = T / BKV;
    const int a = (int)blockIdx.x, b = nb - 1 - (int)blockIdx.x;  // a: the longer sweep
    for (int pass = 0; pass < (b > a ? 2 : 1); ++pass) {
        if (pass) wg_barrier();
        attn_dkv_block(pass ? b : a, sm, svt, sl, qkv, dout, lse, delta, dqkv, part, T, nq, nkv);
    }
}

// dK = scale * sum_z part[z][.][.][0], dV = sum_z part[z][.][.][1], summed in
// subset order (deterministic); one thread per 4 consecutive elements.
__global__ __launch_bounds__(256) void attn_dkv_reduce_kernel(const float* __restrict__ part, bf16_t* __restrict__ dqkv,
                                                              int T, int nq, int nkv, int nsplit) {
    const int64_t per = (int64_t)T * nkv * 2 * D;  // floats per subset
    const int64_t i4 = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
    if (i4 >= per) return;
    floatx4 acc = *reinterpret_cast<const floatx4*>(part + i4);
    for (int z = 1; z < nsplit; ++z) acc += *reinterpret_cast<const floatx4*>(part + z * per + i4);
    const int d = (int)(i4 % D);
    const int which = (int)((i4 / D) % 2);
    const int grp = (int)((i4 / (2 * D)) % nkv);
    const int key = (int)(i4 / (2 * D * nkv));
    const float sc = which == 0 ? 1.f / sqrtf((float)D) : 1.f;
    u32x2 v;
    v[0] = uint32_t(f2bf(acc[0] * sc)) | (uint32_t(f2bf(acc[1] * sc)) << 16);
    v[1] = uint32_t(f2bf(acc[2] * sc)) | (uint32_t(f2bf(acc[3] * sc)) << 16);
    const int ld = (nq + 2 * nkv) * D;
    *reinterpret_cast<u32x2*>(dqkv + (int64_t)key * ld + (nq + which * nkv + grp) * D + d) = v;
}

bool shapes_ok(int T, int nq, int nkv) { return T > 0 && T % FQ == 0 && nq > 0 && nkv > 0 && nq % nkv == 0; }

// Query-head subsets per KV head for the dk/dv kernel: the smallest divisor
// of the group size that gives at least 512 workgroups (two per CU on a
// 256-CU part).  A group of 8 query heads per KV head (Llama-70B: 8 KV heads,
// 16 key-block pairs) would otherwise run 128 workgroups.
int dkv_split(int T, int nq, int nkv) {
    const int rep = nq / nkv, wgs = (T / BKV + 1) / 2 * nkv;
    for (int z = 1; z < rep; ++z)
        if (rep % z == 0 && wgs * z >= 512) return z;
    return rep;
}

}  // namespace

int32_t attn_fwd(const bf16_t* qkv, bf16_t* o, float* lse, int T, int nq, int nkv, hipStream_t s) {
    if (!shapes_ok(T, nq, nkv)) return fail(ZB_EINVAL, "attention: tokens must be a multiple of 128");
    hipLaunchKernelGGL(attn_fwd_kernel, dim3((T / FQ + 1) / 2, nq), dim3(FTHR), 0, s, qkv, o, lse, T, nq, nkv);
    ZB_HIP(hipGetLastError());
    return ZB_OK;
}

size_t attn_bwd_scratch_bytes(int T, int nq, int nkv) {
    if (!shapes_ok(T, nq, nkv)) return 0;
    const int z = dkv_split(T, nq, nkv);
    return z > 1 ? (size_t)z * T * nkv * 2 * D * 4 : 0;
}

int32_t attn_bwd(const bf16_t* qkv, const bf16_t* o, const float* lse, const bf16_t* dout, bf16_t* dqkv, float* delta,
                 float* part, int T, int nq, int nkv, hipStream_t s) {
    if (!shapes_ok(T, nq, nkv)) return fail(ZB_EINVAL, "attention: tokens must be a multiple of 128");
    // the dq kernel also computes delta = rowsum(dO o), which the dk/dv kernel reads
    hipLaunchKernelGGL(attn_dq_kernel, dim3((T / FQ + 1) / 2, nq), dim3(FTHR), 0, s, qkv, o, dout, lse, delta, dqkv, T,
                       nq, nkv);
    ZB_HIP(hipGetLastError());
    const int z = dkv_split(T, nq, nkv);
    if (z > 1 && part == nullptr) return fail(ZB_EINVAL, "attention: missing dk/dv partial scratch");
    hipLaunchKernelGGL(attn_dkv_kernel, dim3((T / BKV + 1) / 2, nkv, z), dim3(FTHR), 0, s, qkv, dout, lse, delta, dqkv,
                       z > 1 ? part : nullptr, T, nq, nkv);
    ZB_HIP(hipGetLastError());
    if (z > 1) {
        const int64_t n4 = (int64_t)T * nkv * 2 * D / 4;
        hipLaunchKernelGGL(attn_dkv_reduce_kernel, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, s, part, dqkv, T,
                           nq, nkv, z);
        ZB_HIP(hipGetLastError());
    }
    return ZB_OK;
}

}  // namespace zb
