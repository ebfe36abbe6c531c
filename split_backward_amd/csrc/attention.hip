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
// * Tiles of K, V (forward, dq), of Q, dO (dk/dv) and of dS^T (dq) are DMA'd
//   HBM -> LDS with buffer_load ... lds in their natural [rows][128] layout
//   (256-byte rows, 16-byte chunks XOR-swizzled by the row), double buffered.
// * Operands whose reduction index is the row of such a tile (V^T in o,
//   K^T and dS^T in dq, dO^T and Q^T in dv / dk) are read with the gfx950
//   transpose read ds_read_b64_tr_b16; the row addresses are chosen so the
//   lane receives the keys (or queries) in exactly the order the score
//   accumulator holds them (8(s/4) + 4g + s%4 within a 16-row step), so
//   probabilities go from the accumulator into the next MFMA without any
//   shuffle.
// * The forward computes the transposed score block S^T = K Q^T: each lane
//   owns one query column, so softmax statistics are per-lane scalars
//   combined with the partner lane 32 away.  It rescales its running output
//   only when a row maximum grows by more than 2^8 (exact: output and
//   normaliser always share one reference maximum), and skips the rescale
//   entirely when no lane of the wave needs it.
// * The backward computes S and dP once.  The dk/dv kernel owns a key block
//   per workgroup and sweeps query blocks, accumulating dK^T and dV^T in
//   registers (no atomics, deterministic); it also writes dS^T in bf16 (the
//   operand its own dK product uses) to a scratch [head][key][query].  The
//   dq kernel then forms dQ = dS K from that scratch and K alone, summing
//   over keys in a fixed order.  delta = rowsum(dO o) comes from a small
//   kernel before both.
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
constexpr int CPOL_NT = 2;  // cache-policy operand of buffer loads and stores: non-temporal

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

// x as three bf16 terms hi + mid + lo whose sum is x to within fp32 rounding
// (slots 0..2; the rest zero).
__device__ __forceinline__ bf16x8 split3(float x) {
    const __bf16 hi = (__bf16)x;
    const float r1 = x - (float)hi;
    const __bf16 mid = (__bf16)r1;
    const __bf16 lo = (__bf16)(r1 - (float)mid);
    const __bf16 z = (__bf16)0.f;
    return bf16x8{hi, mid, lo, z, z, z, z, z};
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
struct TrCol {
    uint32_t lo, hi;
};
// Offsets of the 32-column block cb (0..3) of the tile.
__device__ __forceinline__ TrCol tr_col(int lane, int cb) {
    const int G = lane >> 4, j = lane & 15;
    const int s = j >> 2, q = j & 3;
    const int row_lo = (G >> 1) * 4 + s, row_hi = row_lo + 8;
    const int d = cb * 32 + (G & 1) * 16 + q * 4;
    return TrCol{(uint32_t)(row_lo * 256 + (((d >> 3) ^ swz(row_lo)) << 4) + (d & 7) * 2),
                 (uint32_t)(row_hi * 256 + (((d >> 3) ^ swz(row_hi)) << 4) + (d & 7) * 2)};
}
struct TrBases {
    uint32_t lo[4], hi[4];
};
__device__ __forceinline__ TrBases tr_bases(int lane) {
    TrBases b;
#pragma unroll
    for (int db = 0; db < 4; ++db) {
        const TrCol c = tr_col(lane, db);
        b.lo[db] = c.lo;
        b.hi[db] = c.hi;
    }
    return b;
}
template <int T16>
__device__ __forceinline__ bf16x8 frag_tr(uint32_t tile, uint32_t lo_off, uint32_t hi_off) {
    u32x2 lo, hi;
    asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(lo) : "v"(tile + lo_off), "i"(T16 * 4096));
    asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(hi) : "v"(tile + hi_off), "i"(T16 * 4096));
    return __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
}
template <int T16>
__device__ __forceinline__ bf16x8 frag_tr(uint32_t tile, const TrBases& b, int db) {
    return frag_tr<T16>(tile, b.lo[db], b.hi[db]);
}
template <int T16>
__device__ __forceinline__ bf16x8 frag_tr(uint32_t tile, const TrCol& c) {
    return frag_tr<T16>(tile, c.lo, c.hi);
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
    else if constexpr (N == 2) asm volatile("s_waitcnt vmcnt(2)" ::: "memory");
    else if constexpr (N == 4) asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
    else if constexpr (N == 6) asm volatile("s_waitcnt vmcnt(6)" ::: "memory");
    else if constexpr (N == 8) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
    else if constexpr (N == 12) asm volatile("s_waitcnt vmcnt(12)" ::: "memory");
    else if constexpr (N == 16) asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
    else if constexpr (N == 18) asm volatile("s_waitcnt vmcnt(18)" ::: "memory");
    else if constexpr (N == 24) asm volatile("s_waitcnt vmcnt(24)" ::: "memory");
    else static_assert(N == 0, "unsupported vmcnt");
}

__device__ __forceinline__ void wg_barrier() { asm volatile("s_barrier" ::: "memory"); }

// Item of workgroup b in a 1-D grid of n: the hardware deals workgroups to
// the 8 XCDs round-robin (XCD b % 8), and this gives each XCD a contiguous
// range of items, so the workgroups sharing an XCD's L2 work on the same few
// heads (items are numbered head-major).
__device__ __forceinline__ int xcd_item(int b, int n) {
    const int xcd = b & 7, local = b >> 3;
    const int q = n >> 3, r = n & 7;
    return xcd < r ? xcd * (q + 1) + local : r * (q + 1) + (xcd - r) * q + local;
}

// Largest bf16 magnitude among the four values of two packed words (sign
// bits cleared: magnitudes order as their bit patterns).  TRACK kernels (the
// fp8 stage) fold it over every value they store and leave one maximum per
// wave, from which the next product's quantization takes its exponent.
__device__ __forceinline__ uint32_t mag_max(uint32_t m, const u32x2& v) {
    const uint32_t a = v[0] & 0x7fff7fffu, b = v[1] & 0x7fff7fffu;
    m = max(m, max(a & 0xffffu, a >> 16));
    return max(m, max(b & 0xffffu, b >> 16));
}
// Wave maximum of m, written by lane 0 to *out as the bf16 value (a float).
__device__ __forceinline__ void wave_mag_out(uint32_t m, float* out) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, o, 64));
    if ((threadIdx.x & 63) == 0) *out = __uint_as_float(m << 16);
}

// ======================================================== forward ========
constexpr int FQ = 128, FKV = 64, FTHR = 256;
constexpr int KV_TILE = FKV * D * 2;  // 16 KB

// One query block qb (32 NW queries, a wave's 32 each) of head h.
template <int NW, bool TRACK = false>
__device__ __forceinline__ void attn_fwd_block(int qb, int h, char (*sm)[2 * KV_TILE], const bf16_t* __restrict__ qkv,
                                               bf16_t* __restrict__ o, float* __restrict__ lse, int T, int nq,
                                               int nkv, uint32_t& mx) {
    constexpr int QB = 32 * NW;  // queries per block
    const int ld = (nq + 2 * nkv) * D;
    const int grp = h / (nq / nkv);
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 5, col = lane & 31;
    const int qw0 = qb * QB + wave * 32;
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

    const int nkb = (qb * QB + QB) / FKV;
    auto dma = [&](int kb) {
        char* st = sm[kb & 1];
        dma_rows<FKV, NW>(kbase, ld, kb * FKV, T, 0, (lds_void*)st, lane, wave);
        dma_rows<FKV, NW>(vbase, ld, kb * FKV, T, 0, (lds_void*)(st + KV_TILE), lane, wave);
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
            if constexpr (TRACK) mx = mag_max(mx, v);
        }
    if (g == 0) lse[(int64_t)h * T + q] = m + log2f(l);
}

// Causal query blocks differ in length up to nb-fold: each workgroup runs
// block nb-1-x and then its mirror x, so every workgroup does the same work
// and the workgroups resident on a CU finish together.  Grid: (nb + 1) / 2
// pairs per head, 1-D, items head-major (xcd_item).  NW = 8: one workgroup
// of 256 queries per CU, whose eight waves share each K/V tile (half the
// DMA per query of two 128-query workgroups); NW = 4 for token counts that
// are not a multiple of 256.
template <int NW, bool TRACK = false>
__global__ __launch_bounds__(NW * 64, 8 / NW) void attn_fwd_kernel(const bf16_t* __restrict__ qkv,
                                                                   bf16_t* __restrict__ o, float* __restrict__ lse,
                                                                   int T, int nq, int nkv, float* __restrict__ amax) {
    __shared__ __attribute__((aligned(1024))) char sm[2][2 * KV_TILE];  // [stage][K | V]
    const int nb = T / (32 * NW), npair = (nb + 1) / 2;
    const int item = xcd_item(blockIdx.x, gridDim.x);
    const int h = item / npair, x = item % npair;
    const int a = nb - 1 - x, b = x;
    uint32_t mx = 0;
    for (int pass = 0; pass < (b < a ? 2 : 1); ++pass) {
        if (pass) wg_barrier();  // every wave is done with the stages
        attn_fwd_block<NW, TRACK>(pass ? b : a, h, sm, qkv, o, lse, T, nq, nkv, mx);
    }
    if constexpr (TRACK) wave_mag_out(mx, amax + blockIdx.x * NW + (threadIdx.x >> 6));
}

// =================================================== delta kernel ========
// delta[h][q] = sum_d dO[q][h][d] o[q][h][d] in fp32, the row statistic of
// dS = P (dP - delta).  16 lanes per (query, head): 8 products each, then a
// sum across the 16 lanes.
__global__ __launch_bounds__(256) void attn_delta_kernel(const bf16_t* __restrict__ o, const bf16_t* __restrict__ dout,
                                                         float* __restrict__ delta, int T, int nq) {
    const int64_t pair = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
    if (pair >= (int64_t)T * nq) return;  // whole 16-lane groups
    const int q = (int)(pair / nq), h = (int)(pair % nq);
    const int j = threadIdx.x & 15;
    const int64_t e = (int64_t)q * nq * D + h * D + j * 8;
    const bf16x8 ov = *reinterpret_cast<const bf16x8*>(o + e);
    const bf16x8 dv = *reinterpret_cast<const bf16x8*>(dout + e);
    float sum = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) sum = fmaf((float)ov[i], (float)dv[i], sum);
#pragma unroll
    for (int m = 8; m >= 1; m >>= 1) sum += __shfl_xor(sum, m, 16);
    if (j == 0) delta[(int64_t)h * T + q] = sum;
}

// ====================================================== dq kernel ========
// dS^T scratch layout: 2 KB chunks [head][query block of 32][key block of 32],
// each holding dS^T of 32 keys x 32 queries in the order the dk/dv kernel's
// lanes hold it, so that kernel stores 1 KB contiguous per instruction: half
// j (queries 16j .. 16j+15), then for key kk and lane half g the 16 bytes at
// 32 kk + 16 g: queries 16j + 4g + 0..3, then 16j + 8 + 4g + 0..3.
constexpr int DS_CHUNK = 2048;
// Byte offset, in a wave's 4 KB of two consecutive chunks (64 keys, 32
// queries), at which lane `lane` starts its transpose reads of dS^T: source
// lane j = 4s + c of 16-lane group G reads key 4(G/2) + s of a 16-key step
// at queries 16(G%2) + 4c .. +3, which lands output lane i of the group, slot
// s, on query 16(G%2) + i and key 4(G/2) + s: the score-accumulator order of
// the keys.  A group's 16 reads cover one contiguous 128-byte range.
__device__ __forceinline__ uint32_t ds_gather_base(int lane) {
    const int G = lane >> 4, j = lane & 15, s = j >> 2, c = j & 3;
    return (uint32_t)((G & 1) * 1024 + (4 * (G >> 1) + s) * 32 + (c & 1) * 16 + (c >> 1) * 8);
}
// Fragment of 16-key step t (keys 16t .. 16t+15 of the 64): keys 16t + 4g + s
// in slots 0..3 and 16t + 8 + 4g + s in slots 4..7.
template <int T16>
__device__ __forceinline__ bf16x8 frag_ds(uint32_t tile, uint32_t base) {
    constexpr int off = (T16 >> 1) * DS_CHUNK + (T16 & 1) * 512;
    u32x2 lo, hi;
    asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(lo) : "v"(tile + base), "i"(off));
    asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(hi) : "v"(tile + base), "i"(off + 256));
    return __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
}

// Per (query block of 128, query head): dQ^T += K^T dS^T over the key
// blocks of 64 at or before the block's queries, both operands from LDS by
// transpose reads.  dS^T of the head was written by the dk/dv kernel (bf16,
// zero where the key follows the query); each wave DMAs the two chunks of
// its 32 queries per key block (4 KB) and reads nothing else of it, so the
// kernel streams dS^T from HBM once while K comes mostly from L2.  dS^T
// stages sit in a ring of three (two in flight while one is used), K tiles
// in a ring of two: 80 KB of LDS, two workgroups per CU.
constexpr int DQ_K_STAGES = 2, DQ_S_STAGES = 3;
constexpr int DS_STAGE = 4 * 2 * DS_CHUNK;  // four waves x 64 keys x 32 queries: 16 KB
struct DqSmem {
    char k[DQ_K_STAGES][KV_TILE];
    char s[DQ_S_STAGES][DS_STAGE];
};
template <bool TRACK = false>
__device__ __forceinline__ void attn_dq_block(int qb, int h, DqSmem& sm, const bf16_t* __restrict__ qkv,
                                              const bf16_t* __restrict__ dst, bf16_t* __restrict__ dqkv, int T, int nq,
                                              int nkv, uint32_t& mx) {
    const int ld = (nq + 2 * nkv) * D;
    const int grp = h / (nq / nkv);
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 5, col = lane & 31;
    const int qw0 = qb * FQ + wave * 32;
    const int q = qw0 + col;
    const int nq32 = T / 32;
    const bf16_t* kbase = qkv + nq * D + grp * D;
    // the wave's chunks: [h][query block qw0 / 32][key block 0 ..]
    const bf16_t* dsw = dst + ((int64_t)h * nq32 + qw0 / 32) * nq32 * (DS_CHUNK / 2);

    floatx16 dacc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) dacc[i] = zero16();
    const TrBases trb = tr_bases(lane);
    const uint32_t sgat = ds_gather_base(lane);

    const int nkb = (qb * FQ + FQ) / FKV;
    // 4 loads per wave for either tile; blocks past the last are empty.
    auto dma_k = [&](int kb) {
        dma_rows<FKV, 4>(kbase, ld, kb * FKV, T, 0, (lds_void*)sm.k[kb % DQ_K_STAGES], lane, wave, kb < nkb);
    };
    auto dma_s = [&](int kb) {
        const bool live = kb < nkb;
        const __amdgpu_buffer_rsrc_t rs =
            make_rsrc(dsw + (int64_t)(live ? kb : 0) * 2 * (DS_CHUNK / 2), live ? 2 * DS_CHUNK : 0);
        lds_char* dstl = (lds_char*)sm.s[kb % DQ_S_STAGES] + wave * 2 * DS_CHUNK;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(dstl + i * 1024), 16, i * 1024 + lane * 16, 0, 0,
                                                     CPOL_NT);  // read once: non-temporal
    };
    // Issue order K(0) S(0) S(1), then per iteration kb: K(kb+1) S(kb+2).  At
    // the top of iteration kb only S(kb+1) (4 loads) may still be in flight.
    dma_k(0);
    dma_s(0);
    dma_s(1);
    for (int kb = 0; kb < nkb; ++kb) {
        vm_wait<4>();  // K(kb) and S(kb) landed
        wg_barrier();  // and every wave is done with block kb-1's stages
        dma_k(kb + 1);
        dma_s(kb + 2);
        const int k0 = kb * FKV;
        if (k0 > qw0 + 31) continue;  // every key of the block follows every query of the wave
        const uint32_t kaddr = (uint32_t)(uintptr_t)sm.k[kb % DQ_K_STAGES];
        const uint32_t saddr = (uint32_t)(uintptr_t)sm.s[kb % DQ_S_STAGES] + wave * 2 * DS_CHUNK;
        // dS^T fragments: the wave's queries, the block's keys in accumulator order
        bf16x8 sb[4];
        sb[0] = frag_ds<0>(saddr, sgat);
        sb[1] = frag_ds<1>(saddr, sgat);
        sb[2] = frag_ds<2>(saddr, sgat);
        sb[3] = frag_ds<3>(saddr, sgat);
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
                    lds_wait_keep<8>(cur[0], cur[1], cur[2], cur[3], sb[0], sb[1], sb[2], sb[3]);
                } else {
                    lds_wait_keep<0>(cur[0], cur[1], cur[2], cur[3], sb[0], sb[1], sb[2], sb[3]);
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
            if constexpr (TRACK) mx = mag_max(mx, v);
        }
}

// Paired query blocks as in the forward kernel; 1-D grid, items head-major.
template <bool TRACK = false>
__global__ __launch_bounds__(FTHR, 2) void attn_dq_kernel(const bf16_t* __restrict__ qkv,
                                                          const bf16_t* __restrict__ dst,
                                                          bf16_t* __restrict__ dqkv, int T, int nq, int nkv,
                                                          float* __restrict__ amax) {
    __shared__ __attribute__((aligned(1024))) DqSmem sm;
    const int nb = T / FQ, npair = (nb + 1) / 2;
    const int item = xcd_item(blockIdx.x, gridDim.x);
    const int h = item / npair, x = item % npair;
    const int a = nb - 1 - x, b = x;
    uint32_t mx = 0;
    for (int pass = 0; pass < (b < a ? 2 : 1); ++pass) {
        if (pass) wg_barrier();
        attn_dq_block<TRACK>(pass ? b : a, h, sm, qkv, dst, dqkv, T, nq, nkv, mx);
    }
    if constexpr (TRACK) wave_mag_out(mx, amax + blockIdx.x * (FTHR / 64) + (threadIdx.x >> 6));
}

// ===================================================== dk / dv kernel ====
// Per (key block of 32 NW keys, KV head).  Each of the NW waves owns 32 keys
// (K rows in registers, V rows in LDS, as B operands).  Sweeps the query
// heads of the group and the query blocks of 32 rows at or after the
// diagonal:
//   S = Q K^T, P = exp2(S c - lse2), dP = dO V^T, dS = P (dP - delta),
//   dV^T += dO^T P,  dK^T += Q^T dS,  and stores dS^T (bf16) for dQ.
// NW = 4: two workgroups per CU (two waves per SIMD, at most 256 registers
// per lane, 64.5 KB of LDS each), so one workgroup's softmax, barrier and
// LDS latency overlap the other's MFMAs.  NW = 8: one workgroup of 256 keys
// per CU (97 KB of LDS), whose eight waves share each Q and dO block.
// Double-buffered query blocks suffice with that overlap.
constexpr int BQB = 32;
constexpr int Q_TILE = BQB * D * 2;  // 8 KB
constexpr int KV_STAGES = 2;

template <int NW, bool TRACK = false>
__device__ __forceinline__ void attn_dkv_block(int kb, char (*sm)[2 * Q_TILE], char* svt, float (*sl)[2][BQB],
                                               const bf16_t* __restrict__ qkv, const bf16_t* __restrict__ dout,
                                               const float* __restrict__ lse, const float* __restrict__ delta,
                                               bf16_t* __restrict__ dqkv, float* __restrict__ part,
                                               bf16_t* __restrict__ dst, int T, int nq, int nkv, int grp, int zi,
                                               int nz, uint32_t& mx) {
    const int ld = (nq + 2 * nkv) * D;
    const int ldo = nq * D;
    // The group's query heads split over nz workgroups (head subset zi);
    // with more than one, each writes fp32 partial dK, dV to `part` and
    // attn_dkv_reduce_kernel adds them in subset order.
    const int rep = nq / nkv / nz;
    const int head0 = (grp * nz + zi) * rep;
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 5, col = lane & 31;
    constexpr int BKV = 32 * NW;
    const int kw0 = kb * BKV + wave * 32;
    const int key = kw0 + col;

    // K rows of the wave's keys stay in registers; V rows of the block's keys
    // go to LDS once (8 loads per wave, waited for with the first block).
    bf16x8 kf[8];
#pragma unroll
    for (int kk = 0; kk < 8; ++kk)
        kf[kk] = *reinterpret_cast<const bf16x8*>(qkv + (int64_t)key * ld + nq * D + grp * D + kk * 16 + g * 8);
    dma_rows<BKV, NW>(qkv + (nq + nkv) * D + grp * D, ld, kb * BKV, T, 0, (lds_void*)svt, lane, wave);
    floatx16 dk[4], dv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        dk[i] = zero16();
        dv[i] = zero16();
    }
    const float c = LOG2E / sqrtf((float)D);
    const float inv_c = 1.f / c;
    const TrBases trb = tr_bases(lane);
    // B operand that adds k = 0..2 of an A fragment into every column: ones
    // at k 0..2 (lane group 0), zeros elsewhere.
    bf16x8 ones3;
#pragma unroll
    for (int i = 0; i < 8; ++i) ones3[i] = (__bf16)((g == 0 && i < 3) ? 1.f : 0.f);
    const int qb0 = (kb * BKV) / BQB;
    const int nqb = T / BQB;
    const int per_head = nqb - qb0;
    const int total = per_head * rep;

    // Ring of KV_STAGES query blocks: the DMA of blocks it+1 .. it+KV_STAGES-1
    // is issued while block it is used.  Every wave issues 2 (8 / NW) + 2
    // loads per block (DMA of Q and dO, and the 32 row statistics of lse and
    // delta, written identically by each wave's lanes 0..31); blocks past the
    // last are empty.  Block it is query block qi of head hh: the fetch and
    // the sweep each step their own (hh, qi) rather than divide it by the
    // blocks per head (the divisions were 3% of the kernel's time).
    auto fetch = [&](int it, int hh, int qi) {
        const bool live = it < total;
        const int q0 = (qb0 + (live ? qi : 0)) * BQB;
        hh = live ? hh : head0;
        char* st = sm[it % KV_STAGES];
        dma_rows<BQB, NW>(qkv + hh * D, ld, q0, T, 0, (lds_void*)st, lane, wave, live);
        dma_rows<BQB, NW>(dout + hh * D, ldo, q0, T, 0, (lds_void*)(st + Q_TILE), lane, wave, live);
        if (lane < BQB) {
            const __amdgpu_buffer_rsrc_t rl = make_rsrc(lse + (int64_t)hh * T + q0, live ? BQB * 4 : 0);
            const __amdgpu_buffer_rsrc_t rd = make_rsrc(delta + (int64_t)hh * T + q0, live ? BQB * 4 : 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rl, (lds_void*)&sl[it % KV_STAGES][0][0], 4, lane * 4, 0, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rd, (lds_void*)&sl[it % KV_STAGES][1][0], 4, lane * 4, 0, 0, 0);
        }
    };

    // dS^T of the wave's 32 keys x the block's 32 queries: one 2 KB chunk
    // (layout above the dq kernel), two 1 KB stores.  Slots 0..7 of the
    // lane's accumulator are queries 4g + 0..3 and 8 + 4g + 0..3, slots 8..15
    // the same plus 16.
    const int nq32 = T / 32;
    auto ds_store = [&](int hh, int q0, const u32x4& w0, const u32x4& w1) {
        const __amdgpu_buffer_rsrc_t rds =
            make_rsrc(dst + ((int64_t)hh * nq32 + q0 / 32) * nq32 * (DS_CHUNK / 2), nq32 * DS_CHUNK);
        const uint32_t off = (uint32_t)((kb * NW + wave) * DS_CHUNK + (2 * col + g) * 16);
        // non-temporal: left dirty in the caches, the 537 MB (Llama-7B shape)
        // would still be written back while the dq kernel reads it
        __builtin_amdgcn_raw_buffer_store_b128(w0, rds, off, 0, CPOL_NT);
        __builtin_amdgcn_raw_buffer_store_b128(w1, rds, off + 1024, 0, CPOL_NT);
    };
    // Each iteration ends with its 2 dS^T stores, so the DMA of the next
    // block is waited for with those 2 stores still in flight (vector memory
    // operations complete in issue order).  A wave whose keys all follow the
    // block's queries runs the block anyway: the causal mask makes its P and
    // dS zero, which is what dS^T must hold there, and the iteration count
    // of stores stays exact.
    static_assert(KV_STAGES == 2, "the wait below counts one block of DMA and one of stores");
    int f_hh = head0, f_qi = 0;  // the next block to fetch
    auto fetch_next = [&](int it) {
        fetch(it, f_hh, f_qi);
        if (++f_qi == per_head) {
            f_qi = 0;
            ++f_hh;
        }
    };
    fetch_next(0);
    int c_hh = head0, c_qi = 0;  // block it
    for (int it = 0; it < total; ++it) {
        if (it == 0) vm_wait<0>();
        else vm_wait<2>();  // block it landed (the previous block's 2 stores may be in flight)
        wg_barrier();
        fetch_next(it + 1);  // into the stage block it-1 used
        const int hh = c_hh;
        const int q0 = (qb0 + c_qi) * BQB;
        if (++c_qi == per_head) {
            c_qi = 0;
            ++c_hh;
        }
        const int stg = it % KV_STAGES;
        const lds_void* qt = (const lds_void*)sm[stg];
        const lds_void* ot = (const lds_void*)(sm[stg] + Q_TILE);
        // Fragment reads as asm (explicit waits): the compiler would otherwise
        // wait for the DMA of the next block, issued just above, before them.
        // The row statistics enter as the accumulators' initial values: an MFMA
        // of an A fragment holding query row l's value in k = 0..2 (lane l,
        // split3) with ones3 writes -lse2/c into every key column of S's row
        // l and -delta into dP's, in the accumulator's own row order, so no
        // lane gathers its rows' statistics.
        floatx16 s, dp;
        {
            const uint32_t la = (uint32_t)(uintptr_t)&sl[stg][0][0] + col * 4;
            float ls, ds;
            asm volatile("ds_read_b32 %0, %1" : "=v"(ls) : "v"(la));
            asm volatile("ds_read_b32 %0, %1 offset:%2" : "=v"(ds) : "v"(la), "i"(BQB * 4));
            lds_wait_keep<0>(ls, ds);
            s = mfma(split3(-ls * inv_c), ones3, zero16());
            dp = mfma(split3(-ds), ones3, zero16());
        }
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
        // accumulator row of slot r: query (r/4)*8 + 4g + r%4 of the block
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int qr = (r >> 2) * 8 + g * 4 + (r & 3);
            float p = fast_exp2(s[r] * c);  // s = S - lse2/c
            if (diag && key > q0 + qr) p = 0.f;
            s[r] = p;
            dp[r] = p * dp[r];  // dp = dP - delta
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
        ds_store(hh, q0, __builtin_bit_cast(u32x4, s0), __builtin_bit_cast(u32x4, s1));
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the empty trailing blocks still write LDS
    if (part) {  // fp32 partials [subset][key][kv head][dK | dV][D], dK not yet scaled
        float* pk = part + (((int64_t)zi * T + key) * nkv + grp) * 2 * D;
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
            if constexpr (TRACK) mx = mag_max(mag_max(mx, vk), vv);
        }
}

// Key block kb sweeps the query blocks at or after it: pairs kb with its
// mirror so every workgroup does the same work.
// TRACK (with part null): the waves' maxima of the dK, dV they store go to
// amax[NW * workgroup + wave].
template <int NW, bool TRACK = false>
__global__ __launch_bounds__(NW * 64, 8 / NW) void attn_dkv_kernel(const bf16_t* __restrict__ qkv,
                                                                   const bf16_t* __restrict__ dout,
                                                                   const float* __restrict__ lse,
                                                                   const float* __restrict__ delta,
                                                                   bf16_t* __restrict__ dqkv, float* __restrict__ part,
                                                                   bf16_t* __restrict__ dst, int T, int nq, int nkv,
                                                                   int nz, float* __restrict__ amax) {
    __shared__ __attribute__((aligned(1024))) char sm[KV_STAGES][2 * Q_TILE];  // [stage][Q | dO]
    __shared__ __attribute__((aligned(1024))) char svt[32 * NW * D * 2];       // V rows of the block
    __shared__ float sl[KV_STAGES][2][BQB];                                     // [stage][lse | delta]
    const int nb = T / (32 * NW), npair = (nb + 1) / 2;
    // 1-D grid of npair x nz x nkv items, KV-head-major (xcd_item)
    const int item = xcd_item(blockIdx.x, gridDim.x);
    const int x = item % npair, zi = (item / npair) % nz, grp = item / (npair * nz);
    const int a = x, b = nb - 1 - x;  // a: the longer sweep
    uint32_t mx = 0;
    for (int pass = 0; pass < (b > a ? 2 : 1); ++pass) {
        if (pass) wg_barrier();
        attn_dkv_block<NW, TRACK>(pass ? b : a, sm, svt, sl, qkv, dout, lse, delta, dqkv, part, dst, T, nq, nkv, grp,
                                  zi, nz, mx);
    }
    if constexpr (TRACK) wave_mag_out(mx, amax + blockIdx.x * NW + (threadIdx.x >> 6));
}

// dK = scale * sum_z part[z][.][.][0], dV = sum_z part[z][.][.][1], summed in
// subset order (deterministic); one thread per 4 consecutive elements.
// TRACK: the waves' maxima of what they store go to amax[4 * workgroup + wave].
template <bool TRACK = false>
__global__ __launch_bounds__(256) void attn_dkv_reduce_kernel(const float* __restrict__ part, bf16_t* __restrict__ dqkv,
                                                              int T, int nq, int nkv, int nsplit,
                                                              float* __restrict__ amax) {
    const int64_t per = (int64_t)T * nkv * 2 * D;  // floats per subset
    const int64_t i4 = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
    if (TRACK) {
        // every lane reaches the wave's maximum: lanes past the end add zero
        uint32_t mx = 0;
        if (i4 < per) {
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
            mx = mag_max(mx, v);
        }
        wave_mag_out(mx, amax + blockIdx.x * 4 + (threadIdx.x >> 6));
        return;
    }
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

// Waves per dk/dv workgroup: 8 (256 keys) when the key blocks tile T.
int dkv_waves(int T) { return T % 256 == 0 ? 8 : 4; }

// Query-head subsets per KV head for the dk/dv kernel: the smallest divisor
// of the group size that fills a 256-CU part (512 workgroups of 128 keys,
// two per CU, or 256 of 256 keys).  A group of 8 query heads per KV head
// (Llama-70B: 8 KV heads, 8 key-block pairs of 256) would otherwise run 64
// workgroups.
int dkv_split(int T, int nq, int nkv) {
    const int nw = dkv_waves(T);
    const int rep = nq / nkv, wgs = (T / (32 * nw) + 1) / 2 * nkv;
    for (int z = 1; z < rep; ++z)
        if (rep % z == 0 && wgs * z >= 2048 / nw) return z;
    return rep;
}

size_t ds_bytes(int T, int nq) { return ((size_t)nq * T * T * 2 + 255) / 256 * 256; }

}  // namespace

// Grids of the launches below (workgroups), shared with the partial-maxima counts.
namespace {
int fwd_grid(int T, int nq) { return T % 256 == 0 ? (T / 256 + 1) / 2 * nq : (T / 128 + 1) / 2 * nq; }
int dkv_grid(int T, int nkv, int z) { return dkv_waves(T) == 8 ? (T / 256 + 1) / 2 * nkv * z : (T / 128 + 1) / 2 * nkv * z; }
int64_t reduce_grid(int T, int nkv) { return ((int64_t)T * nkv * 2 * D / 4 + 255) / 256; }
int dq_grid(int T, int nq) { return (T / FQ + 1) / 2 * nq; }
int fwd_parts(int T, int nq) { return fwd_grid(T, nq) * (T % 256 == 0 ? 8 : 4); }
int64_t bwd_parts(int T, int nq, int nkv) {
    const int z = dkv_split(T, nq, nkv);
    return (z > 1 ? reduce_grid(T, nkv) * 4 : (int64_t)dkv_grid(T, nkv, z) * dkv_waves(T)) + dq_grid(T, nq) * (FTHR / 64);
}
}  // namespace

int64_t attn_amax_parts(int T, int nq, int nkv) {
    if (!shapes_ok(T, nq, nkv)) return 0;
    return std::max<int64_t>(fwd_parts(T, nq), bwd_parts(T, nq, nkv));
}

int32_t attn_fwd(const bf16_t* qkv, bf16_t* o, float* lse, int T, int nq, int nkv, hipStream_t s, float* amax,
                 int* amax_n) {
    if (!shapes_ok(T, nq, nkv)) return fail(ZB_EINVAL, "attention: tokens must be a multiple of 128");
    const dim3 grid(fwd_grid(T, nq));
    if (amax) {
        if (T % 256 == 0)
            hipLaunchKernelGGL((attn_fwd_kernel<8, true>), grid, dim3(512), 0, s, qkv, o, lse, T, nq, nkv, amax);
        else
            hipLaunchKernelGGL((attn_fwd_kernel<4, true>), grid, dim3(256), 0, s, qkv, o, lse, T, nq, nkv, amax);
    } else if (T % 256 == 0) {
        hipLaunchKernelGGL(attn_fwd_kernel<8>, grid, dim3(512), 0, s, qkv, o, lse, T, nq, nkv, nullptr);
    } else {
        hipLaunchKernelGGL(attn_fwd_kernel<4>, grid, dim3(256), 0, s, qkv, o, lse, T, nq, nkv, nullptr);
    }
    ZB_HIP(hipGetLastError());
    if (amax_n) *amax_n = amax ? fwd_parts(T, nq) : 0;
    return ZB_OK;
}

size_t attn_bwd_scratch_bytes(int T, int nq, int nkv) {
    if (!shapes_ok(T, nq, nkv)) return 0;
    const int z = dkv_split(T, nq, nkv);
    return ds_bytes(T, nq) + (z > 1 ? (size_t)z * T * nkv * 2 * D * 4 : 0);
}

int32_t attn_bwd(const bf16_t* qkv, const bf16_t* o, const float* lse, const bf16_t* dout, bf16_t* dqkv, float* delta,
                 void* scratch, int T, int nq, int nkv, hipStream_t s, float* amax, int* amax_n) {
    if (!shapes_ok(T, nq, nkv)) return fail(ZB_EINVAL, "attention: tokens must be a multiple of 128");
    if (scratch == nullptr) return fail(ZB_EINVAL, "attention: missing backward scratch");
    bf16_t* dst = static_cast<bf16_t*>(scratch);
    const int z = dkv_split(T, nq, nkv);
    float* part = z > 1 ? reinterpret_cast<float*>(static_cast<char*>(scratch) + ds_bytes(T, nq)) : nullptr;
    // delta = rowsum(dO o), read by the dk/dv kernel
    const int64_t pairs = (int64_t)T * nq;
    hipLaunchKernelGGL(attn_delta_kernel, dim3((unsigned)((pairs + 15) / 16)), dim3(256), 0, s, o, dout, delta, T, nq);
    ZB_HIP(hipGetLastError());
    // dK, dV (or their per-subset partials) and dS^T; with amax, the kernel
    // that stores dK, dV (this one, or the reduction) leaves its maxima first,
    // the dq kernel's follow
    const bool track_dkv = amax && z == 1;
    const dim3 g_dkv(dkv_grid(T, nkv, z));
    if (dkv_waves(T) == 8) {
        if (track_dkv)
            hipLaunchKernelGGL((attn_dkv_kernel<8, true>), g_dkv, dim3(512), 0, s, qkv, dout, lse, delta, dqkv, part,
                               dst, T, nq, nkv, z, amax);
        else
            hipLaunchKernelGGL(attn_dkv_kernel<8>, g_dkv, dim3(512), 0, s, qkv, dout, lse, delta, dqkv, part, dst, T,
                               nq, nkv, z, nullptr);
    } else {
        if (track_dkv)
            hipLaunchKernelGGL((attn_dkv_kernel<4, true>), g_dkv, dim3(256), 0, s, qkv, dout, lse, delta, dqkv, part,
                               dst, T, nq, nkv, z, amax);
        else
            hipLaunchKernelGGL(attn_dkv_kernel<4>, g_dkv, dim3(256), 0, s, qkv, dout, lse, delta, dqkv, part, dst, T,
                               nq, nkv, z, nullptr);
    }
    ZB_HIP(hipGetLastError());
    int64_t n_parts = track_dkv ? (int64_t)dkv_grid(T, nkv, z) * dkv_waves(T) : 0;
    if (z > 1) {
        const dim3 g_red((unsigned)reduce_grid(T, nkv));
        if (amax) {
            hipLaunchKernelGGL((attn_dkv_reduce_kernel<true>), g_red, dim3(256), 0, s, part, dqkv, T, nq, nkv, z, amax);
            n_parts = reduce_grid(T, nkv) * 4;
        } else {
            hipLaunchKernelGGL(attn_dkv_reduce_kernel<false>, g_red, dim3(256), 0, s, part, dqkv, T, nq, nkv, z,
                               nullptr);
        }
        ZB_HIP(hipGetLastError());
    }
    // dQ = dS K from the scratch
    const dim3 g_dq(dq_grid(T, nq));
    if (amax)
        hipLaunchKernelGGL((attn_dq_kernel<true>), g_dq, dim3(FTHR), 0, s, qkv, dst, dqkv, T, nq, nkv, amax + n_parts);
    else
        hipLaunchKernelGGL(attn_dq_kernel<false>, g_dq, dim3(FTHR), 0, s, qkv, dst, dqkv, T, nq, nkv, nullptr);
    ZB_HIP(hipGetLastError());
    if (amax_n) *amax_n = amax ? (int)(n_parts + (int64_t)dq_grid(T, nq) * (FTHR / 64)) : 0;
    return ZB_OK;
}

}  // namespace zb
