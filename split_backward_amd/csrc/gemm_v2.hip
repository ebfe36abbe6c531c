// bf16 GEMM, second generation: direct-to-LDS operand staging.
//
// Workgroup tile 256 x 256, 256 threads = 4 waves in a 2 x 2 grid, each wave
// owning a 128 x 128 sub-tile (256 fp32 accumulators per lane, held in
// AGPRs): 4 x 4 blocks of v_mfma_f32_32x32x16_bf16, or, for products with
// both operands K-contiguous (the F pass, and the B pass on transposed
// weights), 8 x 8 blocks of v_mfma_f32_16x16x32_bf16 (gemm_64_tile16).
// For a K-contiguous A the tile may instead be 128 x 256 (each wave 64 x 128),
// used where a launch's last round of tiles would leave most CUs idle.
//
// The description below is that of the 32-k loop of the W pass; the loops
// of products with a K-contiguous A (64-k parts in a ring of five LDS slots)
// are described where they are defined.
//
// Operands go HBM -> LDS with buffer_load ... lds (16 bytes per lane): no
// VGPR staging, no ds_write, and out-of-range rows / columns / k read as zero
// through the buffer range check.  Each operand keeps its HBM orientation in
// LDS:
//   K-contiguous operand  -> LDS [rows][32 k], 64-byte rows, 16-byte chunks
//                            XOR-swizzled by the row; an MFMA fragment (8
//                            consecutive k of one row) is one ds_read_b128.
//   M/N-contiguous operand -> LDS [32 k][256 cols], 512-byte rows, 32-byte
//                            pieces XOR-swizzled by k; a fragment is two
//                            ds_read_b64_tr_b16, the gfx950 LDS transpose
//                            read (in each 16-lane group, output lane i,
//                            slot s takes element i%4 of the load of lane
//                            4s + i/4), so the lane receives 8 consecutive k
//                            of its column.
// Four LDS stages of 32-k tiles (128 KB): the DMA of the next k-tiles is in
// flight while tile t is multiplied (three tiles of prefetch hide HBM latency
// with one wave per SIMD), fragments of the next 16-k step are read while the
// MFMAs of the current step issue, and the per-tile barrier sits in the
// middle of a tile so fragment reads never wait behind it.  DMA addressing
// costs no VALU: each lane's offset is fixed once, and the buffer base
// advances in scalar registers from tile to tile.
#include "common.h"

namespace zb {
namespace {

constexpr int BM = 256, BN = 256, BK = 32, NTHR = 256, STAGES = 4;
constexpr int TILE_BYTES = 256 * BK * 2;  // 16 KB per operand tile
constexpr int STAGE_BYTES = 2 * TILE_BYTES;

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8;
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

// 16-byte chunk swizzle of a K-contiguous tile (64-byte rows): the rows a
// ds_read_b128 serves together (8 or 16 lanes) hit distinct bank windows.
__device__ __forceinline__ int key_km(int row) { return ((row >> 1) ^ (row >> 3)) & 3; }
// 32-byte piece swizzle of an M/N-contiguous tile row k: the 4 rows a 16-lane
// group reads in one transpose instruction land in 4 distinct 32-byte bank
// windows (and the 8 pieces of a 32-lane half in 8), conflict-free for both
// 32 and 64 four-byte banks.  Depends only on k & 3, so it is the same for
// every 16-k step and the step offsets fold into the instruction offset.
__device__ __forceinline__ int key_mn(int k) { return ((k & 3) << 1) | ((k >> 1) & 1); }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}

constexpr uint32_t OOB = 0x80000000u;  // any offset >= the buffer size reads as zero

// ---- DMA of one operand tile (NI instructions per wave, 1 KB each) --------
// Per-lane byte offsets relative to the tile's first k are computed once;
// rows / columns outside the operand get OOB.  K-contiguous: instruction i of
// wave w covers tile rows 16b..16b+15 with b = 4i + w (NI = 4: 256 rows,
// NI = 2: 128 rows).  `k_lim` (elements, relative to the tile's first k)
// marks k beyond K as OOB; a full tile passes BK and needs no check.
template <bool PAIRED, int NI>
__device__ __forceinline__ void dma_offsets_kmaj(uint32_t (&off)[NI], int64_t ld, int row0, int rows_total,
                                                 int half_n, int k_lim, int lane, int wave) {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const int b = i * 4 + wave;
        const int r = b * 16 + (lane >> 2);
        const int kc = (lane & 3) ^ key_km(r);
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
        off[i] = (ok && kc * 8 < k_lim) ? (uint32_t)(((int64_t)grow * ld + kc * 8) * 2) : OOB;
    }
}

// M/N-contiguous: instruction i of wave w covers k rows 2b, 2b+1 (b = 4i + w);
// k beyond K falls past the end of the (advanced) buffer range.
__device__ __forceinline__ void dma_offsets_mnmaj(uint32_t (&off)[4], int64_t ld, int col0, int cols_total, int lane,
                                                  int wave) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int b = i * 4 + wave;
        const int k = b * 2 + (lane >> 5);
        const int piece = ((lane & 31) >> 1) ^ key_mn(k);  // logical 32-byte piece at this slot
        const int col = piece * 16 + (lane & 1) * 8;
        const int gc = col0 + col;
        off[i] = (gc < cols_total) ? (uint32_t)(((int64_t)k * ld + gc) * 2) : OOB;
    }
}

// Instruction i of wave w writes LDS bytes [1024 b, 1024 b + 1024), b = 4i + w.
__device__ __forceinline__ void dma_issue_one(__amdgpu_buffer_rsrc_t rs, lds_void* tile, uint32_t off, int b) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)((__attribute__((address_space(3))) char*)tile + b * 1024),
                                             16, off, 0, 0, 0);
}
__device__ __forceinline__ void dma_issue(__amdgpu_buffer_rsrc_t rs, lds_void* tile, const uint32_t (&off)[4],
                                          int wave) {
#pragma unroll
    for (int i = 0; i < 4; ++i) dma_issue_one(rs, tile, off[i], i * 4 + wave);
}
__device__ __forceinline__ void dma_issue(__amdgpu_buffer_rsrc_t rs, lds_void* tile, const uint32_t (&off)[2],
                                          int wave) {
#pragma unroll
    for (int i = 0; i < 2; ++i) dma_issue_one(rs, tile, off[i], i * 4 + wave);
}

// ---- fragment reads ------------------------------------------------------
// K-contiguous tile: row `row`, k step kk, lane group g = lane/32.
__device__ __forceinline__ bf16x8 frag_kmaj(const lds_void* tile, int row, int kk, int g) {
    const int chunk = (kk * 2 + g) ^ key_km(row);
    return *(const lds_bf16x8*)((const __attribute__((address_space(3))) char*)tile + row * (BK * 2) + chunk * 16);
}

// M/N-contiguous tile ([BK][256], 512-byte rows): 32-wide block `blk` (0..7), k step kk.
// The two transpose reads are issued as inline asm: the compiler cannot tell
// the intrinsic form from the in-flight LDS DMA of later stages and would wait
// for all of it.  The caller waits for the results with lds_wait().
__device__ __forceinline__ bf16x8 frag_mnmaj(const lds_void* tile, int blk, int kk, int lane) {
    const int G = lane >> 4, j = lane & 15;
    const int s = j >> 2, q = j & 3;
    const int piece = (blk * 2 + (G & 1)) ^ key_mn(s);  // k & 3 == s for both reads
    const int r0 = (G >> 1) * 8 + s;                     // row within the 16-k step
    const uint32_t addr = (uint32_t)(uintptr_t)tile + kk * 16 * 512 + r0 * 512 + piece * 32 + q * 8;
    u32x2 lo, hi;
    asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(lo) : "v"(addr));
    asm volatile("ds_read_b64_tr_b16 %0, %1 offset:2048" : "=v"(hi) : "v"(addr));
    return __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
}

// Wait for every outstanding LDS read; the fragments become outputs of the
// wait so no use of them is scheduled above it.
template <int NA>
__device__ __forceinline__ void lds_wait(bf16x8 (&a)[NA], bf16x8 (&b)[4]) {
    if constexpr (NA == 4)
        asm volatile("s_waitcnt lgkmcnt(0)"
                     : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]), "+v"(b[0]), "+v"(b[1]), "+v"(b[2]), "+v"(b[3]));
    else
        asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(a[0]), "+v"(a[1]), "+v"(b[0]), "+v"(b[1]), "+v"(b[2]), "+v"(b[3]));
}

// Scheduling pattern for one 16-k step of NM MFMAs: NM/2 slots, each
// holding its share of the RD LDS reads followed by 2 MFMAs.
template <int RD, int NM, int SLOT>
__device__ __forceinline__ void interleave_reads_mfma() {
    constexpr int NS = NM / 2;
    if constexpr (SLOT < NS) {
        constexpr int n = ((SLOT + 1) * RD) / NS - (SLOT * RD) / NS;
        if constexpr (n > 0) __builtin_amdgcn_sched_group_barrier(0x100, n, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        interleave_reads_mfma<RD, NM, SLOT + 1>();
    }
}

// Region B of the main loop: RD fragment reads, then ND DMA loads, spread
// over the NM MFMAs of the step (reads first: they come before the DMA in
// program order and must stay there).
template <int RD, int ND, int NM, int SLOT>
__device__ __forceinline__ void interleave_reads_dma_mfma() {
    if constexpr (SLOT < NM) {
        constexpr int T = RD + ND;
        constexpr int lo = (SLOT * T) / NM, hi = ((SLOT + 1) * T) / NM;
        constexpr int nr = (hi < RD ? hi : RD) - (lo < RD ? lo : RD);
        constexpr int nd = (hi - lo) - nr;
        if constexpr (nr > 0) __builtin_amdgcn_sched_group_barrier(0x100, nr, 0);
        if constexpr (nd > 0) __builtin_amdgcn_sched_group_barrier(0x020, nd, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        interleave_reads_dma_mfma<RD, ND, NM, SLOT + 1>();
    }
}

// Wait until at most N buffer loads of this wave are outstanding.
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N == 0 || N == 4 || N == 8 || N == 12 || N == 14 || N == 16 || N == 18 || N == 20 || N == 24 || N == 32,
                  "vmcnt");
    if constexpr (N == 0) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    else if constexpr (N == 4) asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
    else if constexpr (N == 12) asm volatile("s_waitcnt vmcnt(12)" ::: "memory");
    else if constexpr (N == 14) asm volatile("s_waitcnt vmcnt(14)" ::: "memory");
    else if constexpr (N == 18) asm volatile("s_waitcnt vmcnt(18)" ::: "memory");
    else if constexpr (N == 20) asm volatile("s_waitcnt vmcnt(20)" ::: "memory");
    else if constexpr (N == 8) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
    else if constexpr (N == 16) asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
    else if constexpr (N == 24) asm volatile("s_waitcnt vmcnt(24)" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(32)" ::: "memory");
}

// Workgroup barrier without the memory fence __syncthreads() implies: that
// fence waits for every outstanding load, including the DMA of tiles that are
// meant to stay in flight.  Callers wait for exactly the tile they need
// (s_waitcnt vmcnt(n)) first; every LDS read of the stage being recycled has
// been consumed by an MFMA, so it has completed.
__device__ __forceinline__ void workgroup_barrier() { asm volatile("s_barrier" ::: "memory"); }

// Branch-free activations for the epilogues (results are rounded to bf16):
// tanh(y) = 1 - 2 / (e^{2y} + 1) and sigmoid(z) = 1 / (1 + e^{-z}), with the
// hardware base-2 exponential and reciprocal.  At large |y| the exponential
// saturates to 0 or inf and the reciprocal to 1/1 or 0, so the limits -1, 1
// (tanh) and 0, 1 (sigmoid) come out exactly.
__device__ __forceinline__ float exp_f(float x) { return __builtin_amdgcn_exp2f(x * 1.4426950408889634f); }
__device__ __forceinline__ float tanh_f(float y) { return 1.f - 2.f * __builtin_amdgcn_rcpf(exp_f(2.f * y) + 1.f); }
__device__ __forceinline__ float gelu_tanh_f(float a) {
    const float c = 0.7978845608028654f, k = 0.044715f;
    return 0.5f * a * (1.f + tanh_f(c * (a + k * a * a * a)));
}
__device__ __forceinline__ float gelu_tanh_grad_f(float a) {
    const float c = 0.7978845608028654f, k = 0.044715f;
    const float t = tanh_f(c * (a + k * a * a * a));
    return 0.5f * (1.f + t) + 0.5f * a * (1.f - t * t) * c * (1.f + 3.f * k * a * a);
}
__device__ __forceinline__ float sigmoid_f(float z) { return __builtin_amdgcn_rcpf(1.f + exp_f(-z)); }

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
// Four floats -> four bf16 (round to nearest even), two per conversion instruction.
__device__ __forceinline__ u32x2 pack_bf16x4(const float (&f)[4]) {
    return u32x2{__builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{f[0], f[1]}, bf16x2_t)),
                 __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{f[2], f[3]}, bf16x2_t))};
}

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

// Byte lengths of the buffer ranges through which a product's operands are
// read and its outputs written (A, B, C, the epilogue input R, the second
// output C2).  Each is below 2^31: an offset at or past a range reads zero or
// drops the store, which is how rows and columns outside the matrices are
// handled without branches.
struct BufSpans {
    uint32_t a, b, c, r, c2;
};

// One TBM x 256 output tile (tm, tn) of the product `d`; `smem` is the
// workgroup's 128 KB of LDS.  TBM = 256: each wave computes 128 x 128;
// TBM = 128 (K-contiguous A only): each wave computes 64 x 128, for tiles
// that would otherwise leave most of the chip idle in a launch's last round.
// Epilogue of a TBM x 256 tile: the accumulators go through LDS (the
// k-tile stages are free by then) and out with the fused operation EPI.
// Called once every DMA into LDS has been issued: the waits below count the
// loads still in flight.
// Staging of the 32-row block mi of a wave's accumulators into `stage`
// (32 rows of P floats, 128 columns), from either MFMA layout.
// 32x32 blocks: slot r of lane l is row 8 (r / 4) + 4 (l / 32) + r % 4,
// column l % 32.
template <int MI, int P>
__device__ __forceinline__ void stage_block(floatx16 (&acc)[MI][4], int mi, float* stage, int lane) {
    const int g = lane >> 5, lrow = lane & 31;
#pragma unroll
    for (int ni = 0; ni < 4; ++ni)
#pragma unroll
        for (int r = 0; r < 16; ++r) stage[((r >> 2) * 8 + g * 4 + (r & 3)) * P + ni * 32 + lrow] = acc[mi][ni][r];
}
// 16x16 blocks (two per 32 rows): slot i of lane l is row 4 (l / 16) + i,
// column l % 16.
template <int MB, int P>
__device__ __forceinline__ void stage_block(floatx4 (&acc)[MB][8], int mi, float* stage, int lane) {
    const int kg = lane >> 4, r16 = lane & 15;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int ni = 0; ni < 8; ++ni)
#pragma unroll
            for (int i = 0; i < 4; ++i) stage[(h * 16 + kg * 4 + i) * P + ni * 16 + r16] = acc[2 * mi + h][ni][i];
}

// TRACK (the fp8 kernels): the SwiGLU epilogues also leave the per-wave
// maxima of their quantized output at d.amax when it is set.
template <bool A_KMAJ, bool B_KMAJ, int EPI, int TBM, bool TRACK = false, class ACC>
__device__ __forceinline__ void gemm_epilogue(const GemmDesc& d, const BufSpans& sp, ACC& acc, int m0, int n0,
                                              char* smem) {
    constexpr bool PAIRED = (EPI == EPI_SWIGLU_FWD);
    constexpr int MI = TBM / 64;                              // 32-row blocks per wave
    constexpr int MI_ACC = sizeof(ACC) / sizeof(acc[0]);     // first extent of the accumulator array
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    __builtin_amdgcn_sched_barrier(0);
    const int c4 = (lane & 31) * 4;
    const int gcol = n0 + wn * 128 + c4;
    const bool col_ok = gcol < d.N;
    floatx4 cin[2][16];
    // Every epilogue access is a buffer access, issued whether or not its row
    // and columns are inside the matrix (outside, the offset is OOB: loads
    // read zero, stores are dropped).  The code is then free of branches and
    // the compiler counts outstanding loads exactly, so a wait for a block's
    // inputs does not also wait for the stores issued before it.
    const __amdgpu_buffer_rsrc_t rc = make_rsrc(d.C, sp.c);
    auto load_block = [&](int mi, floatx4 (&dst)[16]) {
        const int rbase = m0 + wm * (TBM / 2) + mi * 32;
#pragma unroll
        for (int it = 0; it < 16; ++it) {
            const int row = rbase + 2 * it + (lane >> 5);
            const uint32_t off = (row < d.M && col_ok) ? (uint32_t)(((int64_t)row * d.ldc + gcol) * 4) : OOB;
            dst[it] = __builtin_bit_cast(floatx4, __builtin_amdgcn_raw_buffer_load_b128(rc, off, 0, 0));
        }
    };
    // Epilogues that read a bf16 input (residual, activation input): the
    // rows of block mi+1 are loaded while block mi is computed and stored.
    constexpr bool HAS_R = EPI == EPI_RESID || EPI == EPI_GELU_BWD || EPI == EPI_SWIGLU_BWD;
    constexpr int IT = 16;  // rows 2*it + lane/32 of a 32-row block
    const __amdgpu_buffer_rsrc_t rr = make_rsrc(d.R, HAS_R ? sp.r : 0u);
    u32x2 rin[2][IT], rin2[2][IT];
    auto load_r = [&](int mi, int buf) {
        const int rbase = m0 + wm * (TBM / 2) + mi * 32;
#pragma unroll
        for (int it = 0; it < IT; ++it) {
            const int row = rbase + 2 * it + (lane >> 5);
            const bool ok = row < d.M && col_ok;
            const int64_t e = (int64_t)row * d.ldr + gcol;
            rin[buf][it] = __builtin_amdgcn_raw_buffer_load_b64(rr, ok ? (uint32_t)(e * 2) : OOB, 0, 0);
            if (EPI == EPI_SWIGLU_BWD)
                rin2[buf][it] = __builtin_amdgcn_raw_buffer_load_b64(rr, ok ? (uint32_t)((e + d.half_n) * 2) : OOB, 0, 0);
        }
    };
    // The empty tiles' DMA still writes (zeros) into the stages, and every
    // wave must be done with them before the epilogue reuses the memory.  The
    // first block's epilogue inputs are requested before that wait, so their
    // latency overlaps the drain.
    if constexpr (EPI == EPI_ACCUM_F32) {
        load_block(0, cin[0]);
        asm volatile("s_waitcnt vmcnt(16) lgkmcnt(0)" ::: "memory");  // all DMA done; dW loads in flight
    } else if constexpr (EPI == EPI_SWIGLU_BWD) {
        load_r(0, 0);
        asm volatile("s_waitcnt vmcnt(32) lgkmcnt(0)" ::: "memory");
    } else if constexpr (HAS_R) {
        load_r(0, 0);
        asm volatile("s_waitcnt vmcnt(16) lgkmcnt(0)" ::: "memory");
    } else {
        asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
    }
    workgroup_barrier();

    // ---- epilogue ---------------------------------------------------------
    // The accumulators of a 32-row block (mi) go through the wave's own LDS
    // region (the k-tile stages are free now) so that each lane then owns 4
    // consecutive columns of a row: global traffic is 16-byte (fp32) or
    // 8-byte (bf16) per lane, and every global load of a block is issued
    // before any of its values is needed.  Same-wave LDS accesses are ordered,
    // so no barrier is needed.  (Unaligned leading dimensions or widths not
    // divisible by 4 are routed to the first-generation kernel instead.)
    constexpr int P = 132;  // floats per staged row: 128 + 4 padding
    float* stage = reinterpret_cast<float*>(smem) + wave * 32 * P;
    if constexpr (EPI == EPI_ACCUM_F32 || EPI == EPI_STORE_F32) {
        // dW += acc: the old values of block mi+1 are loaded while block mi
        // is added and stored, so at most one HBM round trip is exposed.
        // (EPI_STORE_F32: the same stores, nothing loaded.)
#pragma unroll
        for (int mi = 0; mi < MI; ++mi) {
            if (EPI == EPI_ACCUM_F32 && mi + 1 < MI) load_block(mi + 1, cin[(mi + 1) & 1]);
            const int rbase = m0 + wm * (TBM / 2) + mi * 32;
            stage_block<MI_ACC, P>(acc, mi, stage, lane);
#pragma unroll
            for (int it = 0; it < 16; ++it) {
                const int lr = 2 * it + (lane >> 5);
                const int row = rbase + lr;
                const uint32_t off = (row < d.M && col_ok) ? (uint32_t)(((int64_t)row * d.ldc + gcol) * 4) : OOB;
                floatx4 v = *reinterpret_cast<const floatx4*>(stage + lr * P + c4);
                if constexpr (EPI == EPI_ACCUM_F32) v += cin[mi & 1][it];
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), rc, off, 0, 0);  // dropped outside C
            }
        }
        return;
    }
    constexpr bool HAS_C2 = EPI == EPI_GELU_FWD || PAIRED;
    const __amdgpu_buffer_rsrc_t rc2 = make_rsrc(d.C2, HAS_C2 ? sp.c2 : 0u);
    // SwiGLU epilogues: the largest |value| of the quantized output, as bf16
    // magnitudes (sign bit cleared; for them integer order is value order)
    // of the packed words stored, two per register; rows and columns outside
    // the matrix hold zeros
    u16x2 mxb = {0, 0};
    auto track = [&](const u32x2& w) {
        mxb = __builtin_elementwise_max(mxb, __builtin_bit_cast(u16x2, w[0] & 0x7fff7fffu));
        mxb = __builtin_elementwise_max(mxb, __builtin_bit_cast(u16x2, w[1] & 0x7fff7fffu));
    };
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
        const int rbase = m0 + wm * (TBM / 2) + mi * 32;
        if (!PAIRED) {
            if (HAS_R && mi + 1 < MI) load_r(mi + 1, (mi + 1) & 1);
            stage_block<MI_ACC, P>(acc, mi, stage, lane);
#pragma unroll
            for (int it = 0; it < IT; ++it) {
                const int lr = 2 * it + (lane >> 5);
                const int row = rbase + lr;
                const bool ok = row < d.M && col_ok;
                const floatx4 v = *reinterpret_cast<const floatx4*>(stage + lr * P + c4);
                float o[4], o2[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float x = v[e];
                    const uint32_t rw = HAS_R ? rin[mi & 1][it][e >> 1] : 0u;
                    const float rv = (e & 1) ? __uint_as_float(rw & 0xffff0000u) : __uint_as_float(rw << 16);
                    if (EPI == EPI_STORE) o[e] = x;
                    else if (EPI == EPI_RESID) o[e] = x + rv;
                    else if (EPI == EPI_GELU_FWD) { o[e] = x; o2[e] = gelu_tanh_f(x); }
                    else if (EPI == EPI_GELU_BWD) o[e] = x * gelu_tanh_grad_f(rv);
                    else if (EPI == EPI_SWIGLU_BWD) {
                        const uint32_t uw = rin2[mi & 1][it][e >> 1];
                        const float u = (e & 1) ? __uint_as_float(uw & 0xffff0000u) : __uint_as_float(uw << 16);
                        // dg = ds u sg (1 + g (1 - sg)) = ds u (sg + a - a sg), du = ds a, a = g sg
                        const float sg = sigmoid_f(rv), a = rv * sg;
                        o[e] = x * u * fmaf(-a, sg, a + sg);
                        o2[e] = x * a;
                    }
                }
                const int64_t ec = (int64_t)row * d.ldc + gcol;
                const u32x2 wo = pack_bf16x4(o);
                __builtin_amdgcn_raw_buffer_store_b64(wo, rc, ok ? (uint32_t)(ec * 2) : OOB, 0, 0);
                if (EPI == EPI_GELU_FWD)
                    __builtin_amdgcn_raw_buffer_store_b64(
                        pack_bf16x4(o2), rc2, ok ? (uint32_t)(((int64_t)row * d.ldc2 + gcol) * 2) : OOB, 0, 0);
                if constexpr (EPI == EPI_SWIGLU_BWD) {
                    const u32x2 wo2 = pack_bf16x4(o2);
                    __builtin_amdgcn_raw_buffer_store_b64(wo2, rc, ok ? (uint32_t)((ec + d.half_n) * 2) : OOB, 0, 0);
                    if constexpr (TRACK) {
                        track(wo);
                        track(wo2);
                    }
                }
            }
        } else {
            // paired SwiGLU forward: staged columns 0..63 are gate, 64..127 up
            const int c4 = (lane & 15) * 4;
            const int gcol = n0 + wn * 64 + c4;
            const bool col_ok = gcol < d.half_n;
            stage_block<MI_ACC, P>(acc, mi, stage, lane);
#pragma unroll
            for (int it = 0; it < 8; ++it) {
                const int lr = 4 * it + (lane >> 4);
                const int row = rbase + lr;
                const bool ok = row < d.M && col_ok;
                const floatx4 gv = *reinterpret_cast<const floatx4*>(stage + lr * P + c4);
                const floatx4 uv = *reinterpret_cast<const floatx4*>(stage + lr * P + 64 + c4);
                float og[4], ou[4], os[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    og[e] = gv[e];
                    ou[e] = uv[e];
                    os[e] = gv[e] * sigmoid_f(gv[e]) * uv[e];
                }
                const int64_t ec = (int64_t)row * d.ldc + gcol;
                __builtin_amdgcn_raw_buffer_store_b64(pack_bf16x4(og), rc, ok ? (uint32_t)(ec * 2) : OOB, 0, 0);
                __builtin_amdgcn_raw_buffer_store_b64(pack_bf16x4(ou), rc, ok ? (uint32_t)((ec + d.half_n) * 2) : OOB, 0, 0);
                const u32x2 ws = pack_bf16x4(os);
                __builtin_amdgcn_raw_buffer_store_b64(
                    ws, rc2, ok ? (uint32_t)(((int64_t)row * d.ldc2 + gcol) * 2) : OOB, 0, 0);
                if constexpr (TRACK && EPI == EPI_SWIGLU_FWD) track(ws);
            }
        }
    }
    if constexpr (TRACK && (EPI == EPI_SWIGLU_FWD || EPI == EPI_SWIGLU_BWD)) {
        if (d.amax) {
            uint32_t m = mxb[0] > mxb[1] ? mxb[0] : mxb[1];
#pragma unroll
            for (int o = 32; o > 0; o >>= 1) {
                const uint32_t t = (uint32_t)__shfl_xor((int)m, o, 64);
                m = t > m ? t : m;
            }
            if (lane == 0) d.amax[blockIdx.x * (NTHR / 64) + wave] = __uint_as_float(m << 16);
        }
    }
}

template <bool A_KMAJ, bool B_KMAJ, int EPI, int TBM = BM>
__device__ __forceinline__ void gemm_v2_tile(const GemmDesc& d, int tm, int tn, const BufSpans& sp, char* smem) {
    constexpr bool PAIRED = (EPI == EPI_SWIGLU_FWD);
    static_assert(TBM == BM || (TBM == BM / 2 && A_KMAJ), "half-height tiles need a K-contiguous A");
    constexpr int MI = TBM / 64;  // 32-row A fragments per wave; also A DMA instructions per wave
    constexpr int DPT = MI + 4;   // DMA instructions per wave per k-tile
    constexpr bool SEGMENTED = !A_KMAJ && !B_KMAJ && EPI == EPI_ACCUM_F32;

    // wave index as a scalar: every LDS address derived from it (the DMA
    // destinations in M0) is then computed by scalar instructions.
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const int g = lane >> 5, lrow = lane & 31;
    const int m0 = tm * TBM;
    const int n0 = PAIRED ? tn * (BN / 2) : tn * BN;
    const int nk = (d.K + BK - 1) / BK;
    const int k_tail = d.K - (nk - 1) * BK;  // k extent of the last tile (1..BK)

    uint32_t offa[MI], offb[4];
    if constexpr (A_KMAJ) dma_offsets_kmaj<false, MI>(offa, d.lda, m0, d.M, 0, BK, lane, wave);
    else dma_offsets_mnmaj(offa, d.lda, m0, d.M, lane, wave);
    if constexpr (B_KMAJ) dma_offsets_kmaj<PAIRED, 4>(offb, d.ldb, n0, d.N, d.half_n, BK, lane, wave);
    else dma_offsets_mnmaj(offb, d.ldb, n0, d.N, lane, wave);
    // Byte step of the buffer base per k-tile.
    const int64_t step_a = A_KMAJ ? BK * 2 : (int64_t)BK * d.lda * 2;
    const int64_t step_b = B_KMAJ ? BK * 2 : (int64_t)BK * d.ldb * 2;

    // Two K segments (W over two microbatches): k-tiles from K1 / BK on come
    // from A2 / B2.  K1 is a multiple of BK, so no k-tile straddles them.
    const int nk1 = (SEGMENTED && d.K1 > 0) ? d.K1 / BK : nk;

    // part 0: the A tile only, 1: the B tile only, 2: both.
    auto dma_tile = [&](int kt, int part = 2) {
        char* st = smem + (kt % STAGES) * STAGE_BYTES;
        // A tile past the end of K gets an empty range: its loads read zeros,
        // fetch nothing, and keep the per-iteration DMA count uniform.
        const bool live = kt < nk;
        const bool seg2 = SEGMENTED && kt >= nk1;
        const int ktl = seg2 ? kt - nk1 : kt;
        const char* base_a = static_cast<const char*>(seg2 ? d.A2 : d.A);
        const char* base_b = static_cast<const char*>(seg2 ? d.B2 : d.B);
        const uint32_t adv_a = live ? (uint32_t)(ktl * step_a) : 0u, adv_b = live ? (uint32_t)(ktl * step_b) : 0u;
        const __amdgpu_buffer_rsrc_t ra = make_rsrc(base_a + adv_a, live ? sp.a - adv_a : 0u);
        const __amdgpu_buffer_rsrc_t rb = make_rsrc(base_b + adv_b, live ? sp.b - adv_b : 0u);
        if (kt == nk - 1 && k_tail < BK) {  // partial last tile: mask k >= K on K-contiguous operands
            uint32_t ta[MI], tb[4];
            if constexpr (A_KMAJ) dma_offsets_kmaj<false, MI>(ta, d.lda, m0, d.M, 0, k_tail, lane, wave);
            else dma_offsets_mnmaj(ta, d.lda, m0, d.M, lane, wave);
            if constexpr (B_KMAJ) dma_offsets_kmaj<PAIRED, 4>(tb, d.ldb, n0, d.N, d.half_n, k_tail, lane, wave);
            else dma_offsets_mnmaj(tb, d.ldb, n0, d.N, lane, wave);
            if (part != 1) dma_issue(ra, (lds_void*)st, ta, wave);
            if (part != 0) dma_issue(rb, (lds_void*)(st + TILE_BYTES), tb, wave);
        } else {
            if (part != 1) dma_issue(ra, (lds_void*)st, offa, wave);
            if (part != 0) dma_issue(rb, (lds_void*)(st + TILE_BYTES), offb, wave);
        }
    };

    floatx16 acc[MI][4];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

    auto frag_a = [&](const lds_void* ta, int mi, int kk) -> bf16x8 {
        if (A_KMAJ) return frag_kmaj(ta, wm * (TBM / 2) + mi * 32 + lrow, kk, g);
        return frag_mnmaj(ta, wm * 4 + mi, kk, lane);
    };
    auto frag_b = [&](const lds_void* tb, int ni, int kk) -> bf16x8 {
        if (B_KMAJ) {
            const int row = PAIRED ? ((ni >> 1) * 128 + wn * 64 + (ni & 1) * 32 + lrow) : (wn * 128 + ni * 32 + lrow);
            return frag_kmaj(tb, row, kk, g);
        }
        return frag_mnmaj(tb, wn * 4 + ni, kk, lane);
    };

    constexpr int RD_A = A_KMAJ ? 1 : 2, RD_B = B_KMAJ ? 1 : 2;
    // With an M/N-contiguous operand (transpose reads, twice the LDS read
    // instructions) the DMA of a tile is split: its A half is issued in
    // region B, its B half in the next region A, which spreads the address
    // unit's work over the whole tile.  Both-K-contiguous kernels measure
    // faster with the whole tile in region B.
    constexpr bool SPLIT_DMA = !A_KMAJ || !B_KMAJ;
    constexpr int RD = MI * RD_A + 4 * RD_B;  // LDS read instructions per 16-k step
    constexpr int NM = MI * 4;                // MFMAs per wave per 16-k step

    // Software pipeline across tiles.  Iteration kt:
    //   region A: MFMAs of k step 0 of tile kt, while the step-1 fragments of
    //             tile kt are read;
    //   every read of tile kt has completed and tile kt+1 has landed, then a
    //             barrier (mid-tile, so no wave idles at a tile boundary);
    //   region B: MFMAs of step 1 of tile kt, while the step-0 fragments of
    //             tile kt+1 are read and the DMA of tile kt+4 is issued into
    //             the stage tile kt just vacated (with SPLIT_DMA its A half;
    //             the B half follows in region A of iteration kt+1, when that
    //             stage is still free).
    // Every iteration issues the same DMA count (tiles past K are empty), so
    // the waits are constants: after region A of iteration kt the DMA of
    // tiles kt+2 and kt+3 (16 loads per wave) may stay in flight.
    if (SPLIT_DMA) {
#pragma unroll
        for (int t = 0; t < STAGES - 1; ++t) dma_tile(t);
        dma_tile(STAGES - 1, 0);
        wait_vm<(STAGES - 2) * DPT + MI>();  // tile 0 landed (tiles 1, 2 and the A half of 3 may not)
    } else {
#pragma unroll
        for (int t = 0; t < STAGES; ++t) dma_tile(t);
        wait_vm<(STAGES - 1) * DPT>();  // tile 0 landed
    }
    workgroup_barrier();
    bf16x8 fa0[MI], fb0[4], fa1[MI], fb1[4];
    {
        const lds_void* ta = (const lds_void*)smem;
        const lds_void* tb = (const lds_void*)(smem + TILE_BYTES);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (i < MI) fa0[i] = frag_a(ta, i, 0);
            fb0[i] = frag_b(tb, i, 0);
        }
    }
    for (int kt = 0; kt < nk; ++kt) {
        const char* st = smem + (kt % STAGES) * STAGE_BYTES;
        const lds_void* ta = (const lds_void*)st;
        const lds_void* tb = (const lds_void*)(st + TILE_BYTES);
        __builtin_amdgcn_sched_barrier(0);
        if (!A_KMAJ || !B_KMAJ) lds_wait(fa0, fb0);
        // region A
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (i < MI) fa1[i] = frag_a(ta, i, 1);
            fb1[i] = frag_b(tb, i, 1);
        }
        if (!A_KMAJ || !B_KMAJ) __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int mi = 0; mi < MI; ++mi)
#pragma unroll
            for (int ni = 0; ni < 4; ++ni)
                acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa0[mi], fb0[ni], acc[mi][ni], 0, 0, 0);
        if (SPLIT_DMA) dma_tile(kt + STAGES - 1, 1);  // B half of tile kt+3
        if (A_KMAJ && B_KMAJ) interleave_reads_mfma<RD, NM, 0>();
        __builtin_amdgcn_sched_barrier(0);
        lds_wait(fa1, fb1);  // tile kt fully read: its stage may be overwritten
        wait_vm<(STAGES - 2) * DPT>();  // tile kt+1 landed
        workgroup_barrier();

        // region B (the fragments read past the last tile are never used)
        {
            const char* sn = smem + ((kt + 1) % STAGES) * STAGE_BYTES;
            const lds_void* na = (const lds_void*)sn;
            const lds_void* nb = (const lds_void*)(sn + TILE_BYTES);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                if (i < MI) fa0[i] = frag_a(na, i, 0);
                fb0[i] = frag_b(nb, i, 0);
            }
        }
        dma_tile(kt + STAGES, SPLIT_DMA ? 0 : 2);  // into the stage tile kt vacated
#pragma unroll
        for (int mi = 0; mi < MI; ++mi)
#pragma unroll
            for (int ni = 0; ni < 4; ++ni)
                acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa1[mi], fb1[ni], acc[mi][ni], 0, 0, 0);
        if (A_KMAJ && B_KMAJ) interleave_reads_dma_mfma<RD, DPT, NM, 0>();
    }
    // The last iteration read fragments of a k-tile past K that are never
    // used.  Waiting for them with the fragments as operands keeps their
    // registers reserved until the reads have landed, so no later value can
    // be placed in a register an LDS read is still writing.
    lds_wait(fa0, fb0);
    gemm_epilogue<A_KMAJ, B_KMAJ, EPI, TBM>(d, sp, acc, m0, n0, smem);
}

// ---- K-contiguous A: 64-k parts in a ring of five --------------------------
// A 32-k K-contiguous tile row is a 64-byte segment, half a cache line, and
// its DMA keeps the address unit waiting on the vector L1.  With a
// K-contiguous A (the F and B passes) the k-tile is 64 deep instead: a
// K-contiguous part of a k-tile (rows x 128 bytes) fills whole lines (an
// M/N-contiguous part is 64 rows of 512 bytes).  The parts sit in a ring of
// five 32 KB LDS slots (part p, the A (p even) or B (p odd) half of k-tile
// p/2, in slot p % 5), so about three parts are in flight while a k-tile is
// multiplied, the prefetch depth of four 32-k stages.
// Swizzle of the 16-byte chunks of a 128-byte row (conflict-free b128 reads).
__device__ __forceinline__ int key8(int row) { return (row >> 1) & 7; }

// Instruction i of wave w covers part rows 8b..8b+7 (b = 4i + w); NI = 8:
// 256 rows, NI = 4: 128 rows.
template <bool PAIRED, int NI>
__device__ __forceinline__ void dma_offsets_k64(uint32_t (&off)[NI], int64_t ld, int row0, int rows_total, int half_n,
                                                int k_lim, int lane, int wave) {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const int b = i * 4 + wave;
        const int r = b * 8 + (lane >> 3);
        const int kc = (lane & 7) ^ key8(r);
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
        off[i] = (ok && kc * 8 < k_lim) ? (uint32_t)(((int64_t)grow * ld + kc * 8) * 2) : OOB;
    }
}

template <int NI>
__device__ __forceinline__ void dma_issue_n(__amdgpu_buffer_rsrc_t rs, lds_void* tile, const uint32_t (&off)[NI],
                                            int wave) {
#pragma unroll
    for (int i = 0; i < NI; ++i) dma_issue_one(rs, tile, off[i], i * 4 + wave);
}


__device__ __forceinline__ bf16x8 frag_k64(const lds_void* tile, int row, int kk, int g) {
    const int chunk = (kk * 2 + g) ^ key8(row);
    return *(const lds_bf16x8*)((const __attribute__((address_space(3))) char*)tile + row * 128 + chunk * 16);
}

constexpr int BK64 = 64, PART_BYTES = 32768, NSLOT = 5;

__device__ __forceinline__ void dma_offsets_mn64(uint32_t (&off)[8], int64_t ld, int col0, int cols_total, int lane,
                                                 int wave) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int b = i * 4 + wave;
        const int k = b * 2 + (lane >> 5);
        const int piece = ((lane & 31) >> 1) ^ key_mn(k);
        const int col = piece * 16 + (lane & 1) * 8;
        const int gc = col0 + col;
        off[i] = (gc < cols_total) ? (uint32_t)(((int64_t)k * ld + gc) * 2) : OOB;
    }
}
template <bool A_KMAJ, bool B_KMAJ, int EPI, int TBM>
__device__ __forceinline__ void gemm_64_tile(const GemmDesc& d, int tm, int tn, const BufSpans& sp, char* smem) {
    constexpr bool PAIRED = (EPI == EPI_SWIGLU_FWD);
    constexpr int MI = TBM / 64;
    constexpr int NA = TBM / 32, NB = 8;  // DMA instructions per wave per part
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const int g = lane >> 5, lrow = lane & 31;
    const int m0 = tm * TBM;
    const int n0 = PAIRED ? tn * (BN / 2) : tn * BN;
    const int nk = (d.K + BK64 - 1) / BK64;
    const int k_tail = d.K - (nk - 1) * BK64;  // k extent of the last k-tile (1..64)

    uint32_t offa[NA], offb[NB], offa_t[NA], offb_t[NB];  // full k-tiles, and the last one
    if constexpr (A_KMAJ) {
        dma_offsets_k64<false, NA>(offa, d.lda, m0, d.M, 0, BK64, lane, wave);
        dma_offsets_k64<false, NA>(offa_t, d.lda, m0, d.M, 0, k_tail, lane, wave);
    } else {
        dma_offsets_mn64(offa, d.lda, m0, d.M, lane, wave);
    }
    if constexpr (B_KMAJ) {
        dma_offsets_k64<PAIRED, NB>(offb, d.ldb, n0, d.N, d.half_n, BK64, lane, wave);
        dma_offsets_k64<PAIRED, NB>(offb_t, d.ldb, n0, d.N, d.half_n, k_tail, lane, wave);
    } else {
        dma_offsets_mn64(offb, d.ldb, n0, d.N, lane, wave);
    }
    const int64_t step_a = A_KMAJ ? BK64 * 2 : (int64_t)BK64 * d.lda * 2;
    const int64_t step_b = B_KMAJ ? BK64 * 2 : (int64_t)BK64 * d.ldb * 2;
    // Part p of the sequence; parts past the last k-tile get an empty range
    // (zeros, nothing fetched) so every iteration issues the same loads.
    auto dma_part = [&](int p) {
        const int kt = p >> 1;
        char* dst = smem + (p % NSLOT) * PART_BYTES;
        const bool live = kt < nk, tail = kt == nk - 1;
        if ((p & 1) == 0) {
            const uint32_t adv = live ? (uint32_t)(kt * step_a) : 0u;
            const __amdgpu_buffer_rsrc_t rs = make_rsrc(static_cast<const char*>(d.A) + adv, live ? sp.a - adv : 0u);
            uint32_t t[NA];
#pragma unroll
            for (int i = 0; i < NA; ++i) t[i] = (A_KMAJ && tail) ? offa_t[i] : offa[i];
            dma_issue_n<NA>(rs, (lds_void*)dst, t, wave);
        } else {
            const uint32_t adv = live ? (uint32_t)(kt * step_b) : 0u;
            const __amdgpu_buffer_rsrc_t rs = make_rsrc(static_cast<const char*>(d.B) + adv, live ? sp.b - adv : 0u);
            uint32_t t[NB];
#pragma unroll
            for (int i = 0; i < NB; ++i) t[i] = (B_KMAJ && tail) ? offb_t[i] : offb[i];
            dma_issue_n<NB>(rs, (lds_void*)dst, t, wave);
        }
    };

    floatx16 acc[MI][4];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
    auto frag_a = [&](const lds_void* ta, int mi, int kk) -> bf16x8 {
        if constexpr (A_KMAJ) return frag_k64(ta, wm * (TBM / 2) + mi * 32 + lrow, kk, g);
        else return frag_mnmaj(ta, wm * 4 + mi, kk, lane);
    };
    auto frag_b = [&](const lds_void* tb, int ni, int kk) -> bf16x8 {
        if constexpr (B_KMAJ) {
            const int row = PAIRED ? ((ni >> 1) * 128 + wn * 64 + (ni & 1) * 32 + lrow) : (wn * 128 + ni * 32 + lrow);
            return frag_k64(tb, row, kk, g);
        } else {
            return frag_mnmaj(tb, wn * 4 + ni, kk, lane);
        }
    };
    constexpr bool KK = A_KMAJ && B_KMAJ;
    constexpr int RD = MI * (A_KMAJ ? 1 : 2) + 4 * (B_KMAJ ? 1 : 2);  // LDS reads per 16-k step
    constexpr int NM = MI * 4;  // MFMAs per 16-k step

    // Iteration kt multiplies the four 16-k steps of k-tile kt, each while
    // the next step's fragments are read.  During step 0 the A part of
    // k-tile kt+2 goes into the slot k-tile kt-1's B part left.  Before the
    // last step every read of kt has completed and k-tile kt+1 has landed
    // (the A part of kt+2 may still be in flight), then a barrier; during the
    // last step the first fragments of kt+1 are read and the B part of kt+2
    // goes into the slot kt's A part left.  Splitting the two parts' DMA
    // between steps 3 and 0 spreads the address unit's work.
#pragma unroll
    for (int p = 0; p < NSLOT - 1; ++p) dma_part(p);
    wait_vm<NA + NB>();  // parts 0 and 1 (k-tile 0) landed
    workgroup_barrier();
    bf16x8 fa0[MI], fb0[4], fa1[MI], fb1[4];
    {
        const lds_void* ta = (const lds_void*)smem;
        const lds_void* tb = (const lds_void*)(smem + PART_BYTES);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (i < MI) fa0[i] = frag_a(ta, i, 0);
            fb0[i] = frag_b(tb, i, 0);
        }
    }
    for (int kt = 0; kt < nk; ++kt) {
        const lds_void* ta = (const lds_void*)(smem + ((2 * kt) % NSLOT) * PART_BYTES);
        const lds_void* tb = (const lds_void*)(smem + ((2 * kt + 1) % NSLOT) * PART_BYTES);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int st = 0; st < 3; ++st) {
            bf16x8(&ca)[MI] = (st & 1) ? fa1 : fa0;
            bf16x8(&cb)[4] = (st & 1) ? fb1 : fb0;
            bf16x8(&na)[MI] = (st & 1) ? fa0 : fa1;
            bf16x8(&nb)[4] = (st & 1) ? fb0 : fb1;
            if constexpr (!KK) lds_wait(ca, cb);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                if (i < MI) na[i] = frag_a(ta, i, st + 1);
                nb[i] = frag_b(tb, i, st + 1);
            }
            if constexpr (!KK) __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int mi = 0; mi < MI; ++mi)
#pragma unroll
                for (int ni = 0; ni < 4; ++ni)
                    acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ca[mi], cb[ni], acc[mi][ni], 0, 0, 0);
            if (st == 0) dma_part(2 * kt + 4);  // the A part of k-tile kt+2, into the slot kt-1's B part left
            if constexpr (KK) {
                if (st == 0) interleave_reads_dma_mfma<RD, NA, NM, 0>();
                else interleave_reads_mfma<RD, NM, 0>();
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        lds_wait(fa1, fb1);  // every read of k-tile kt has completed: its slots may be overwritten
        wait_vm<NA>();       // k-tile kt+1 landed
        workgroup_barrier();
        {
            const lds_void* na = (const lds_void*)(smem + ((2 * kt + 2) % NSLOT) * PART_BYTES);
            const lds_void* nb = (const lds_void*)(smem + ((2 * kt + 3) % NSLOT) * PART_BYTES);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                if (i < MI) fa0[i] = frag_a(na, i, 0);
                fb0[i] = frag_b(nb, i, 0);
            }
        }
        dma_part(2 * kt + 5);  // the B part of k-tile kt+2, into the slot kt's A part left
#pragma unroll
        for (int mi = 0; mi < MI; ++mi)
#pragma unroll
            for (int ni = 0; ni < 4; ++ni)
                acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa1[mi], fb1[ni], acc[mi][ni], 0, 0, 0);
        if constexpr (KK) interleave_reads_dma_mfma<RD, NB, NM, 0>();
    }
    lds_wait(fa0, fb0);  // the unused reads of k-tile nk (see the 32-k loop)
    gemm_epilogue<A_KMAJ, B_KMAJ, EPI, TBM>(d, sp, acc, m0, n0, smem);
}


// 16x16x32 fragments of a 64-k part.  K-contiguous part (128-byte rows):
// lane l holds row `row`, k = 8 (l / 16) .. + 7 of 32-k step kk.
__device__ __forceinline__ bf16x8 frag16_k64(const lds_void* tile, int row, int kk, int kg) {
    const int chunk = (kk * 4 + kg) ^ key8(row);
    return *(const lds_bf16x8*)((const __attribute__((address_space(3))) char*)tile + row * 128 + chunk * 16);
}
// One TBM x 256 tile with both operands K-contiguous (the F pass) on 64-k
// parts, every product a v_mfma_f32_16x16x32_bf16: each wave computes
// (TBM / 2) x 128 as (TBM / 32) x 8 blocks of 16 x 16 (256 or 128
// accumulators).  Same parts, ring, DMA schedule and epilogues as the 32x32
// loop above; per 32-k step a wave reads TBM / 32 + 8 fragments (16 bytes
// per lane each) and issues (TBM / 32) x 8 MFMAs.  On the F products this
// keeps the matrix units busier than the 32x32x16 loop (+5-7% on one box);
// on the B pass (transpose reads of B) it was slower and is not used.  K
// must be a multiple of 64 (every k-tile full); other K take the 32x32 loop,
// whose last k-tile masks k >= K.
template <bool A_KMAJ, bool B_KMAJ, int EPI, int TBM>
__device__ __forceinline__ void gemm_64_tile16(const GemmDesc& d, int tm, int tn, const BufSpans& sp, char* smem) {
    static_assert(A_KMAJ && B_KMAJ, "16x16x32 loop: both operands K-contiguous");
    constexpr bool PAIRED = (EPI == EPI_SWIGLU_FWD);
    constexpr int MB = TBM / 32;          // 16-row blocks per wave
    constexpr int NA = TBM / 32, NB = 8;  // DMA instructions per wave per part
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const int kg = lane >> 4, r16 = lane & 15;
    const int m0 = tm * TBM;
    const int n0 = PAIRED ? tn * (BN / 2) : tn * BN;
    const int nk = (d.K + BK64 - 1) / BK64;  // K is a multiple of 64 here (no partial k-tile)

    uint32_t offa[NA], offb[NB];
    dma_offsets_k64<false, NA>(offa, d.lda, m0, d.M, 0, BK64, lane, wave);
    dma_offsets_k64<PAIRED, NB>(offb, d.ldb, n0, d.N, d.half_n, BK64, lane, wave);
    const int64_t step_a = BK64 * 2, step_b = BK64 * 2;
    // Part p of the sequence; parts past the last k-tile get an empty range
    // (zeros, nothing fetched) so every iteration issues the same loads.
    auto dma_part = [&](int p) {
        const int kt = p >> 1;
        char* dst = smem + (p % NSLOT) * PART_BYTES;
        const bool live = kt < nk;
        if ((p & 1) == 0) {
            const uint32_t adv = live ? (uint32_t)(kt * step_a) : 0u;
            const __amdgpu_buffer_rsrc_t rs = make_rsrc(static_cast<const char*>(d.A) + adv, live ? sp.a - adv : 0u);
            dma_issue_n<NA>(rs, (lds_void*)dst, offa, wave);
        } else {
            const uint32_t adv = live ? (uint32_t)(kt * step_b) : 0u;
            const __amdgpu_buffer_rsrc_t rs = make_rsrc(static_cast<const char*>(d.B) + adv, live ? sp.b - adv : 0u);
            dma_issue_n<NB>(rs, (lds_void*)dst, offb, wave);
        }
    };

    floatx4 acc[MB][8];
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};
    auto frag_a = [&](const lds_void* ta, int mi, int kk) -> bf16x8 {
        return frag16_k64(ta, wm * (TBM / 2) + mi * 16 + r16, kk, kg);
    };
    // B columns of block ni: with the SwiGLU pairing, blocks 0..3 are the
    // wave's 64 gate columns and 4..7 the matching up columns (staged as
    // columns 0..63 and 64..127, which the epilogue expects).
    auto frag_b = [&](const lds_void* tb, int ni, int kk) -> bf16x8 {
        const int row = PAIRED ? ((ni >> 2) * 128 + wn * 64 + (ni & 3) * 16 + r16) : (wn * 128 + ni * 16 + r16);
        return frag16_k64(tb, row, kk, kg);
    };
    constexpr int RD = MB + 8;  // LDS read instructions per 32-k step
    constexpr int NM = MB * 8;  // MFMAs per 32-k step

    // Iteration kt multiplies the two 32-k steps of k-tile kt, each while the
    // next step's fragments are read.  During step 0 the A part of k-tile
    // kt+2 goes into the slot k-tile kt-1's B part left.  Before step 1 every
    // read of kt has completed and k-tile kt+1 has landed (the A part of kt+2
    // may still be in flight), then a barrier; during step 1 the first
    // fragments of kt+1 are read and the B part of kt+2 goes into the slot
    // kt's A part left.
#pragma unroll
    for (int p = 0; p < NSLOT - 1; ++p) dma_part(p);
    wait_vm<NA + NB>();  // parts 0 and 1 (k-tile 0) landed
    workgroup_barrier();
    bf16x8 fa0[MB], fb0[8], fa1[MB], fb1[8];
    {
        const lds_void* ta = (const lds_void*)smem;
        const lds_void* tb = (const lds_void*)(smem + PART_BYTES);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            if (i < MB) fa0[i] = frag_a(ta, i, 0);
            fb0[i] = frag_b(tb, i, 0);
        }
    }
    for (int kt = 0; kt < nk; ++kt) {
        const lds_void* ta = (const lds_void*)(smem + ((2 * kt) % NSLOT) * PART_BYTES);
        const lds_void* tb = (const lds_void*)(smem + ((2 * kt + 1) % NSLOT) * PART_BYTES);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            if (i < MB) fa1[i] = frag_a(ta, i, 1);
            fb1[i] = frag_b(tb, i, 1);
        }
#pragma unroll
        for (int mi = 0; mi < MB; ++mi)
#pragma unroll
            for (int ni = 0; ni < 8; ++ni)
                acc[mi][ni] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa0[mi], fb0[ni], acc[mi][ni], 0, 0, 0);
        dma_part(2 * kt + 4);  // the A part of k-tile kt+2, into the slot kt-1's B part left
        interleave_reads_dma_mfma<RD, NA, NM, 0>();
        __builtin_amdgcn_sched_barrier(0);
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // every read of k-tile kt has completed
        wait_vm<NA>();                                        // k-tile kt+1 landed
        workgroup_barrier();
        {
            const lds_void* na = (const lds_void*)(smem + ((2 * kt + 2) % NSLOT) * PART_BYTES);
            const lds_void* nb = (const lds_void*)(smem + ((2 * kt + 3) % NSLOT) * PART_BYTES);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                if (i < MB) fa0[i] = frag_a(na, i, 0);
                fb0[i] = frag_b(nb, i, 0);
            }
        }
        dma_part(2 * kt + 5);  // the B part of k-tile kt+2, into the slot kt's A part left
#pragma unroll
        for (int mi = 0; mi < MB; ++mi)
#pragma unroll
            for (int ni = 0; ni < 8; ++ni)
                acc[mi][ni] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa1[mi], fb1[ni], acc[mi][ni], 0, 0, 0);
        interleave_reads_dma_mfma<RD, NB, NM, 0>();
        __builtin_amdgcn_sched_barrier(0);
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the unused reads of k-tile nk
    gemm_epilogue<A_KMAJ, B_KMAJ, EPI, TBM>(d, sp, acc, m0, n0, smem);
}

// ---- fp8 (E4M3) products: both operands K-contiguous, 128-k parts ------
// v_mfma_f32_32x32x64_f8f6f4 with E4M3 operands: each lane holds 32 codes of
// one row (A) or column (B), the 32 consecutive k of its lane group (lane
// l: row l % 32, k 32 (l / 32) .. + 31 of a 64-k step); A and B use the same
// lane-to-k assignment, so every product pairs A[i][k] with B[k][j].  A
// 128-k part row is 128 bytes, the same LDS geometry as the bf16 kernel's
// 64-k parts: the five-slot ring, its DMA schedule and its swizzle carry
// over; a k-tile is two 64-k MFMA steps.
typedef int v8i32 __attribute__((ext_vector_type(8)));
constexpr int BK8 = 128;  // k per fp8 k-tile (bytes per part row)

template <bool PAIRED, int NI>
__device__ __forceinline__ void dma_offsets_f8(uint32_t (&off)[NI], int64_t ld, int row0, int rows_total,
                                               int half_n, int k_lim, int lane, int wave) {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const int b = i * 4 + wave;
        const int r = b * 8 + (lane >> 3);
        const int kc = (lane & 7) ^ key8(r);  // 16-byte chunk = 16 codes
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
        off[i] = (ok && kc * 16 < k_lim) ? (uint32_t)((int64_t)grow * ld + kc * 16) : OOB;
    }
}

// Fragment of 32 codes: row `row`, 64-k step kk, lane group g (chunks
// 4kk + 2g and 4kk + 2g + 1 of the 128-byte row).
__device__ __forceinline__ v8i32 frag_f8(const lds_void* tile, int row, int kk, int g) {
    typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
    const __attribute__((address_space(3))) char* base =
        (const __attribute__((address_space(3))) char*)tile + row * 128;
    const int c0 = (kk * 4 + g * 2) ^ key8(row), c1 = (kk * 4 + g * 2 + 1) ^ key8(row);
    const u32x4 lo = *(const lds_u32x4*)(base + c0 * 16);
    const u32x4 hi = *(const lds_u32x4*)(base + c1 * 16);
    return v8i32{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
}

__device__ __forceinline__ floatx16 mfma_f8(const v8i32& a, const v8i32& b, const floatx16& c) {
    // formats 0 / 0: both operands E4M3; block scales 127 = 2^0 (unscaled)
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

template <int EPI, int TBM>
__device__ __forceinline__ void gemm_f8_tile(const GemmDesc& d, int tm, int tn, const BufSpans& sp, char* smem) {
    constexpr bool PAIRED = (EPI == EPI_SWIGLU_FWD);
    constexpr int MI = TBM / 64;
    constexpr int NA = TBM / 32, NB = 8;  // DMA instructions per wave per part
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const int g = lane >> 5, lrow = lane & 31;
    const int m0 = tm * TBM;
    const int n0 = PAIRED ? tn * (BN / 2) : tn * BN;
    const int nk = d.K / BK8;  // K is a multiple of 128 (checked on the host)

    uint32_t offa[NA], offb[NB];
    dma_offsets_f8<false, NA>(offa, d.lda, m0, d.M, 0, BK8, lane, wave);
    dma_offsets_f8<PAIRED, NB>(offb, d.ldb, n0, d.N, d.half_n, BK8, lane, wave);
    auto dma_part = [&](int p) {
        const int kt = p >> 1;
        char* dst = smem + (p % NSLOT) * PART_BYTES;
        const bool live = kt < nk;
        const uint32_t adv = live ? (uint32_t)(kt * BK8) : 0u;
        if ((p & 1) == 0) {
            const __amdgpu_buffer_rsrc_t rs = make_rsrc(static_cast<const char*>(d.A) + adv, live ? sp.a - adv : 0u);
            dma_issue_n<NA>(rs, (lds_void*)dst, offa, wave);
        } else {
            const __amdgpu_buffer_rsrc_t rs = make_rsrc(static_cast<const char*>(d.B) + adv, live ? sp.b - adv : 0u);
            dma_issue_n<NB>(rs, (lds_void*)dst, offb, wave);
        }
    };

    floatx16 acc[MI][4];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
    auto frag_a = [&](const lds_void* ta, int mi, int kk) { return frag_f8(ta, wm * (TBM / 2) + mi * 32 + lrow, kk, g); };
    auto frag_b = [&](const lds_void* tb, int ni, int kk) {
        const int row = PAIRED ? ((ni >> 1) * 128 + wn * 64 + (ni & 1) * 32 + lrow) : (wn * 128 + ni * 32 + lrow);
        return frag_f8(tb, row, kk, g);
    };
    constexpr int RD = 2 * (MI + 4);  // LDS reads per 64-k step
    constexpr int NM = MI * 4;        // MFMAs per 64-k step

    // Iteration kt multiplies the two 64-k steps of k-tile kt, each while
    // the next step's fragments are read.  During step 0 the A part of
    // k-tile kt+2 goes into the slot k-tile kt-1's B part left; then every
    // read of kt has completed and k-tile kt+1 has landed, a barrier, and
    // during step 1 the first fragments of kt+1 are read and the B part of
    // kt+2 goes into the slot kt's A part left.
#pragma unroll
    for (int p = 0; p < NSLOT - 1; ++p) dma_part(p);
    wait_vm<NA + NB>();  // parts 0 and 1 (k-tile 0) landed
    workgroup_barrier();
    v8i32 fa0[MI], fb0[4], fa1[MI], fb1[4];
    {
        const lds_void* ta = (const lds_void*)smem;
        const lds_void* tb = (const lds_void*)(smem + PART_BYTES);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (i < MI) fa0[i] = frag_a(ta, i, 0);
            fb0[i] = frag_b(tb, i, 0);
        }
    }
    for (int kt = 0; kt < nk; ++kt) {
        const lds_void* ta = (const lds_void*)(smem + ((2 * kt) % NSLOT) * PART_BYTES);
        const lds_void* tb = (const lds_void*)(smem + ((2 * kt + 1) % NSLOT) * PART_BYTES);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (i < MI) fa1[i] = frag_a(ta, i, 1);
            fb1[i] = frag_b(tb, i, 1);
        }
#pragma unroll
        for (int mi = 0; mi < MI; ++mi)
#pragma unroll
            for (int ni = 0; ni < 4; ++ni) acc[mi][ni] = mfma_f8(fa0[mi], fb0[ni], acc[mi][ni]);
        dma_part(2 * kt + 4);  // the A part of k-tile kt+2, into the slot kt-1's B part left
        interleave_reads_dma_mfma<RD, NA, NM, 0>();
        __builtin_amdgcn_sched_barrier(0);
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // every read of k-tile kt has completed
        wait_vm<NA>();                                      // k-tile kt+1 landed
        workgroup_barrier();
        {
            const lds_void* na = (const lds_void*)(smem + ((2 * kt + 2) % NSLOT) * PART_BYTES);
            const lds_void* nb = (const lds_void*)(smem + ((2 * kt + 3) % NSLOT) * PART_BYTES);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                if (i < MI) fa0[i] = frag_a(na, i, 0);
                fb0[i] = frag_b(nb, i, 0);
            }
        }
        dma_part(2 * kt + 5);  // the B part of k-tile kt+2, into the slot kt's A part left
#pragma unroll
        for (int mi = 0; mi < MI; ++mi)
#pragma unroll
            for (int ni = 0; ni < 4; ++ni) acc[mi][ni] = mfma_f8(fa1[mi], fb1[ni], acc[mi][ni]);
        interleave_reads_dma_mfma<RD, NB, NM, 0>();
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the unused reads of k-tile nk
    // dequantization: both scales are powers of two, so this multiply is exact
    const float sc = __builtin_ldexpf(1.f, *d.ea + *d.eb);
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int ni = 0; ni < 4; ++ni)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[mi][ni][e] *= sc;
    gemm_epilogue<true, true, EPI, TBM, true>(d, sp, acc, m0, n0, smem);
}

// LDS of one workgroup: five 32 KB slots for products with a K-contiguous A
// (64-k parts), four 32 KB stages otherwise (the epilogue reuses the first
// 68 KB).
template <bool A_KMAJ, bool B_KMAJ>
constexpr int gemm_lds_bytes() { return A_KMAJ ? NSLOT * PART_BYTES : STAGES * STAGE_BYTES; }

// Products with a K-contiguous A (the F and B passes) run on 64-k parts;
// those with an M/N-contiguous A (the W pass) measured faster on 32-k tiles.
// K16: both operands K-contiguous and K a multiple of 64, the 16x16x32 loop
// (a kernel of its own: sharing one function with the 32x32 loop costs the
// register allocator its room).
template <bool A_KMAJ, bool B_KMAJ, int EPI, int TBM, bool K16 = false>
__device__ __forceinline__ void gemm_tile(const GemmDesc& d, int tm, int tn, const BufSpans& sp, char* smem) {
    if constexpr (K16) gemm_64_tile16<A_KMAJ, B_KMAJ, EPI, TBM>(d, tm, tn, sp, smem);
    else if constexpr (A_KMAJ) gemm_64_tile<A_KMAJ, B_KMAJ, EPI, TBM>(d, tm, tn, sp, smem);
    else gemm_v2_tile<A_KMAJ, B_KMAJ, EPI, TBM>(d, tm, tn, sp, smem);
}

// Tiles (tm, tn_base + tn) for tm < tiles_m, tn < tiles_n, of height TBM.
template <bool A_KMAJ, bool B_KMAJ, int EPI, int TBM, bool K16 = false>
__global__ __launch_bounds__(NTHR) void gemm_v2_kernel(GemmDesc d, int tiles_m, int tiles_n, int tn_base,
                                                       BufSpans sp) {
    __shared__ __attribute__((aligned(1024))) char smem[gemm_lds_bytes<A_KMAJ, B_KMAJ>()];
    int tm, tn;
    tile_of(blockIdx.x, tiles_m, tiles_n, tm, tn);
    gemm_tile<A_KMAJ, B_KMAJ, EPI, TBM, K16>(d, tm, tn_base + tn, sp, smem);
}

// Up to GROUP_MAX independent products of one layout and epilogue in one
// launch (the W pass of a whole stage: every weight gradient of every layer).
// Product g owns workgroups [off[g], off[g+1]); each range is a multiple of 8
// so that a workgroup's XCD (blockIdx & 7) is the same in the product's own
// numbering, and the padding workgroups of a range exit at once.
constexpr int GROUP_MAX = 16;
struct GemmGroup {
    GemmDesc d[GROUP_MAX];
    int tiles_m[GROUP_MAX], tiles_n[GROUP_MAX];
    BufSpans sp[GROUP_MAX];
    int off[GROUP_MAX + 1];
    int n;
};
static_assert(sizeof(GemmGroup) <= 3072, "kernel argument block");

template <bool A_KMAJ, bool B_KMAJ, int EPI, int TBM = BM>
__global__ __launch_bounds__(NTHR) void gemm_v2_group_kernel(GemmGroup grp) {
    __shared__ __attribute__((aligned(1024))) char smem[gemm_lds_bytes<A_KMAJ, B_KMAJ>()];
    const int bid = blockIdx.x;
    int g = 0;
    while (g + 1 < grp.n && bid >= grp.off[g + 1]) ++g;
    const int local = bid - grp.off[g];
    const int nwg = grp.tiles_m[g] * grp.tiles_n[g];
    const int q = nwg >> 3, r = nwg & 7, xcd = local & 7;
    if ((local >> 3) >= (xcd < r ? q + 1 : q)) return;  // padding workgroup
    int tm, tn;
    tile_of(local, grp.tiles_m[g], grp.tiles_n[g], tm, tn);
    const GemmDesc d = grp.d[g];  // a value copy: its fields stay in scalar registers
    const BufSpans sp = grp.sp[g];
    gemm_tile<A_KMAJ, B_KMAJ, EPI, TBM>(d, tm, tn, sp, smem);
}

// fp8 products (both operands K-contiguous E4M3): single and grouped.
template <int EPI, int TBM>
__global__ __launch_bounds__(NTHR) void gemm_f8_kernel(GemmDesc d, int tiles_m, int tiles_n, int tn_base,
                                                       BufSpans sp) {
    __shared__ __attribute__((aligned(1024))) char smem[NSLOT * PART_BYTES];
    int tm, tn;
    tile_of(blockIdx.x, tiles_m, tiles_n, tm, tn);
    gemm_f8_tile<EPI, TBM>(d, tm, tn_base + tn, sp, smem);
}

template <int EPI>
__global__ __launch_bounds__(NTHR) void gemm_f8_group_kernel(GemmGroup grp) {
    __shared__ __attribute__((aligned(1024))) char smem[NSLOT * PART_BYTES];
    const int bid = blockIdx.x;
    int g = 0;
    while (g + 1 < grp.n && bid >= grp.off[g + 1]) ++g;
    const int local = bid - grp.off[g];
    const int nwg = grp.tiles_m[g] * grp.tiles_n[g];
    const int q = nwg >> 3, r = nwg & 7, xcd = local & 7;
    if ((local >> 3) >= (xcd < r ? q + 1 : q)) return;  // padding workgroup
    int tm, tn;
    tile_of(local, grp.tiles_m[g], grp.tiles_n[g], tm, tn);
    const GemmDesc d = grp.d[g];
    const BufSpans sp = grp.sp[g];
    gemm_f8_tile<EPI, BM>(d, tm, tn, sp, smem);
}

// The 16x16x32 loop runs full-height tiles of both-K-contiguous products
// with K a multiple of 64 and the F pass's epilogues.  The other cases keep
// the 32x32 loop: for them (half-height tiles, the fp32-accumulate and
// GeLU-backward epilogues) the register allocator moves accumulators between
// registers on every iteration of the 16x16 loop (checked in the generated
// code: the 256-row F-epilogue loops copy at most 16 registers per
// iteration, those cases 128-350).
template <bool AK, bool BKM, int TBM>
int32_t launch_v2(const GemmDesc& d, hipStream_t s, int tiles_m, int tiles_n, int tn_base, const BufSpans& sp) {
    if constexpr (AK && BKM && TBM == BM) {
        if (d.K % BK64 == 0 && d.epi != EPI_ACCUM_F32 && d.epi != EPI_GELU_BWD) {
            dim3 grid(tiles_m * tiles_n), block(NTHR);
            switch (d.epi) {
#define ZB_CASE(E) case E: hipLaunchKernelGGL((gemm_v2_kernel<AK, BKM, E, TBM, true>), grid, block, 0, s, d, tiles_m, tiles_n, tn_base, sp); break;
                ZB_CASE(EPI_STORE)
                ZB_CASE(EPI_RESID)
                ZB_CASE(EPI_GELU_FWD)
                ZB_CASE(EPI_SWIGLU_FWD)
                ZB_CASE(EPI_SWIGLU_BWD)
#undef ZB_CASE
                default: return fail(ZB_EINVAL, "gemm: unknown epilogue");
            }
            ZB_HIP(hipGetLastError());
            return ZB_OK;
        }
    }
    dim3 grid(tiles_m * tiles_n), block(NTHR);
    switch (d.epi) {
#define ZB_CASE(E) case E: hipLaunchKernelGGL((gemm_v2_kernel<AK, BKM, E, TBM>), grid, block, 0, s, d, tiles_m, tiles_n, tn_base, sp); break;
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

}  // namespace

// Bytes spanned by an operand: rows x ld elements (last row counted to its
// logical end).  Must stay below 2^31 for the buffer range check.
static uint64_t span_bytes(int64_t rows, int64_t ld, int64_t cols) { return (uint64_t)((rows - 1) * ld + cols) * 2; }

namespace {
// Whether the direct-to-LDS kernel can run `d`, and its buffer spans and grid.
struct V2Plan {
    bool ok;
    BufSpans sp;
    int tiles_m, tiles_n;
};
V2Plan plan_v2(const GemmDesc& d) {
    V2Plan p{};
    const bool paired = d.epi == EPI_SWIGLU_FWD;
    const int64_t krows = d.K1 > 0 ? d.K1 : d.K;  // k extent of one segment
    const uint64_t ab = d.a_kmajor ? span_bytes(d.M, d.lda, d.K) : span_bytes(krows, d.lda, d.M);
    const uint64_t bb = d.b_kmajor ? span_bytes(d.N, d.ldb, d.K) : span_bytes(krows, d.ldb, d.N);
    const bool has_r = d.epi == EPI_RESID || d.epi == EPI_GELU_BWD || d.epi == EPI_SWIGLU_BWD;
    const bool has_c2 = d.epi == EPI_GELU_FWD || paired;
    // Row widths touched by the epilogue: [g | u] and [dg | du] rows hold
    // their second half half_n elements after the first.
    const int64_t c_w = paired ? 2 * (int64_t)d.half_n : d.epi == EPI_SWIGLU_BWD ? (int64_t)d.half_n + d.N : d.N;
    const int64_t r_w = d.epi == EPI_SWIGLU_BWD ? (int64_t)d.half_n + d.N : d.N;
    const int64_t c2_w = paired ? d.half_n : d.N;
    const bool c_f32 = d.epi == EPI_ACCUM_F32 || d.epi == EPI_STORE_F32;
    const uint64_t cb = c_f32 ? (uint64_t)((int64_t)(d.M - 1) * d.ldc + d.N) * 4 : span_bytes(d.M, d.ldc, c_w);
    const uint64_t rb = has_r ? span_bytes(d.M, d.ldr, r_w) : 0;
    const uint64_t c2b = has_c2 ? span_bytes(d.M, d.ldc2, c2_w) : 0;
    if (ab >= OOB || bb >= OOB || cb >= OOB || rb >= OOB || c2b >= OOB) return p;  // too large for one buffer range
    // 16-byte (fp32) / 8-byte (bf16) epilogue accesses need widths and leading
    // dimensions divisible by 4 and aligned base pointers.
    auto al = [](const void* q, int a) { return (reinterpret_cast<uintptr_t>(q) % a) == 0; };
    bool vec = (d.N % 4 == 0) && (d.ldc % 4 == 0) && al(d.C, c_f32 ? 16 : 8);
    if (has_r) vec = vec && (d.ldr % 4 == 0) && al(d.R, 8);
    if (has_c2) vec = vec && (d.ldc2 % 4 == 0) && al(d.C2, 8);
    if (d.epi == EPI_SWIGLU_BWD || paired) vec = vec && (d.half_n % 4 == 0);
    if (!vec) return p;
    p.ok = true;
    p.sp = BufSpans{(uint32_t)ab, (uint32_t)bb, (uint32_t)cb, (uint32_t)rb, (uint32_t)c2b};
    p.tiles_m = (d.M + BM - 1) / BM;
    p.tiles_n = paired ? (d.half_n + BN / 2 - 1) / (BN / 2) : (d.N + BN - 1) / BN;
    return p;
}

template <bool AK, bool BKM>
int32_t launch_group(const GemmGroup& g, int epi, hipStream_t s) {
    dim3 grid(g.off[g.n]), block(NTHR);
    switch (epi) {
#define ZB_CASE(E) case E: hipLaunchKernelGGL((gemm_v2_group_kernel<AK, BKM, E>), grid, block, 0, s, g); break;
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
}  // namespace

namespace {
int cu_count() {
    static int cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cached[dev] <= 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cached[dev] = n;
    }
    return cached[dev];
}

// How the tile columns of a K-contiguous-A product split between 256-row
// and 128-row tiles.  With one workgroup per CU a launch runs in rounds of
// `cus` tiles, and a last round with at most half the CUs busy costs as long
// as a full one.  Columns [0, n_full) use 256-row tiles and fill whole rounds;
// columns [n_full, tiles_n) use 128-row tiles, twice as many of half the
// work, so the remainder finishes in about half a round.
struct TileSplit {
    int n_full;
};
TileSplit split_columns(int tiles_m, int tiles_n, int tiles_m_half, int cus) {
    const int tiles = tiles_m * tiles_n;
    if (tiles_m_half * tiles_n <= cus) return {0};  // under one round: all half-height
    const int rounds = tiles / cus, rem = tiles % cus;
    if (rem == 0 || rem > cus / 2) return {tiles_n};
    const int n_full = rounds * cus / tiles_m;
    if (tiles_m_half * (tiles_n - n_full) > cus) return {tiles_n};
    return {n_full};
}

template <bool AK, bool BKM>
int32_t launch_v2_split(const GemmDesc& d, hipStream_t s, const V2Plan& p) {
    if constexpr (!AK) {
        return launch_v2<AK, BKM, BM>(d, s, p.tiles_m, p.tiles_n, 0, p.sp);
    } else {
        const int tiles_m_half = (d.M + BM / 2 - 1) / (BM / 2);
        // ZB_GEMM_FULL_TILES=1 keeps every tile 256 rows high (the results are
        // the same bit for bit: a tile's height does not change the order in
        // which any output element is accumulated).
        const TileSplit t = getenv("ZB_GEMM_FULL_TILES") ? TileSplit{p.tiles_n}
                                                         : split_columns(p.tiles_m, p.tiles_n, tiles_m_half, cu_count());
        if (t.n_full > 0) {
            const int32_t rc = launch_v2<AK, BKM, BM>(d, s, p.tiles_m, t.n_full, 0, p.sp);
            if (rc != ZB_OK) return rc;
        }
        if (t.n_full < p.tiles_n) return launch_v2<AK, BKM, BM / 2>(d, s, tiles_m_half, p.tiles_n - t.n_full, t.n_full, p.sp);
        return ZB_OK;
    }
}
}  // namespace

int32_t gemm_bf16_v2(const GemmDesc& d, hipStream_t s, bool* handled) {
    *handled = false;
    if (d.K1 != 0) return fail(ZB_EINVAL, "gemm: a second K segment needs gemm_bf16_group_segmented");
    const V2Plan p = plan_v2(d);
    if (!p.ok) return ZB_OK;  // caller uses the first-generation kernel
    *handled = true;
    if (d.a_kmajor && d.b_kmajor) return launch_v2_split<true, true>(d, s, p);
    if (d.a_kmajor && !d.b_kmajor) return launch_v2_split<true, false>(d, s, p);
    if (!d.a_kmajor && !d.b_kmajor) return launch_v2_split<false, false>(d, s, p);
    return launch_v2_split<false, true>(d, s, p);
}

int32_t gemm_bf16_group_segmented(const GemmDesc* ds, int n, hipStream_t s, bool* handled) {
    *handled = false;
    if (n <= 0 || n > GROUP_MAX || getenv("ZB_GEMM_V1")) return ZB_OK;
    GemmGroup g{};
    g.n = n;
    g.off[0] = 0;
    for (int i = 0; i < n; ++i) {
        const GemmDesc& d = ds[i];
        if (d.K1 <= 0 || d.K1 % BK != 0 || d.K != 2 * d.K1 || !d.A2 || !d.B2) return ZB_OK;
        const V2Plan p = plan_v2(d);
        const bool ok = p.ok && !d.a_kmajor && !d.b_kmajor && d.epi == EPI_ACCUM_F32 && d.M % 8 == 0 &&
                        d.N % 8 == 0 && d.lda % 8 == 0 && d.ldb % 8 == 0 &&
                        ((reinterpret_cast<uintptr_t>(d.A) | reinterpret_cast<uintptr_t>(d.B) |
                          reinterpret_cast<uintptr_t>(d.A2) | reinterpret_cast<uintptr_t>(d.B2)) & 15) == 0;
        if (!ok) return ZB_OK;
        g.d[i] = d;
        g.tiles_m[i] = p.tiles_m;
        g.tiles_n[i] = p.tiles_n;
        g.sp[i] = p.sp;
        g.off[i + 1] = g.off[i] + ((p.tiles_m * p.tiles_n + 7) & ~7);
    }
    *handled = true;
    return launch_group<false, false>(g, EPI_ACCUM_F32, s);
}

namespace {
// Whether an fp8 product fits the kernel: spans (bytes) below 2^31, K and
// the leading dimensions multiples of 16 codes, 16-byte aligned operands,
// vector-friendly epilogue outputs (as for the bf16 kernel).
V2Plan plan_f8(const GemmDesc& d) {
    V2Plan p{};
    if (!d.a_kmajor || !d.b_kmajor || d.K1 != 0 || !d.ea || !d.eb) return p;
    if (d.K % 128 || d.lda % 16 || d.ldb % 16) return p;
    if ((reinterpret_cast<uintptr_t>(d.A) | reinterpret_cast<uintptr_t>(d.B)) & 15) return p;
    GemmDesc b = d;  // the epilogue spans and checks of the bf16 plan, operand spans replaced below
    b.K = 1;
    b.lda = 1;
    b.ldb = 1;
    V2Plan q = plan_v2(b);
    if (!q.ok) return p;
    const uint64_t ab = (uint64_t)((int64_t)(d.M - 1) * d.lda + d.K);
    const uint64_t bb = (uint64_t)((int64_t)((d.epi == EPI_SWIGLU_FWD ? 2 * d.half_n : d.N) - 1) * d.ldb + d.K);
    if (ab >= OOB || bb >= OOB) return p;
    q.sp.a = (uint32_t)ab;
    q.sp.b = (uint32_t)bb;
    return q;
}

template <int TBM>
int32_t launch_f8(const GemmDesc& d, hipStream_t s, int tiles_m, int tiles_n, int tn_base, const BufSpans& sp) {
    dim3 grid(tiles_m * tiles_n), block(NTHR);
    switch (d.epi) {
#define ZB_CASE(E) case E: hipLaunchKernelGGL((gemm_f8_kernel<E, TBM>), grid, block, 0, s, d, tiles_m, tiles_n, tn_base, sp); break;
        ZB_CASE(EPI_STORE)
        ZB_CASE(EPI_RESID)
        ZB_CASE(EPI_ACCUM_F32)
        ZB_CASE(EPI_GELU_FWD)
        ZB_CASE(EPI_GELU_BWD)
        ZB_CASE(EPI_SWIGLU_FWD)
        ZB_CASE(EPI_SWIGLU_BWD)
#undef ZB_CASE
        default: return fail(ZB_EINVAL, "gemm_fp8: unknown epilogue");
    }
    ZB_HIP(hipGetLastError());
    return ZB_OK;
}
}  // namespace

int32_t gemm_fp8(const GemmDesc& d, hipStream_t s, int* amax_n, int amax_cap) {
    if (d.M <= 0 || d.N <= 0 || d.K <= 0) return fail(ZB_EINVAL, "gemm_fp8: empty shape");
    if (d.epi == EPI_SWIGLU_FWD && d.half_n <= 0) return fail(ZB_EINVAL, "gemm_fp8: bad SwiGLU pairing");
    if (d.amax && (d.epi != EPI_SWIGLU_FWD && d.epi != EPI_SWIGLU_BWD))
        return fail(ZB_EINVAL, "gemm_fp8: output maxima only from the SwiGLU epilogues");
    const V2Plan p = plan_f8(d);
    if (!p.ok)
        return fail(ZB_EINVAL, "gemm_fp8: needs K-contiguous operands, K a multiple of 128, leading dimensions multiples of 16, "
                               "16-byte aligned operands, exponent pointers, and spans below 2 GiB");
    const int tiles_m_half = (d.M + BM / 2 - 1) / (BM / 2);
    const TileSplit t = getenv("ZB_GEMM_FULL_TILES") ? TileSplit{p.tiles_n}
                                                     : split_columns(p.tiles_m, p.tiles_n, tiles_m_half, cu_count());
    constexpr int WAVES = NTHR / 64;  // partial maxima per workgroup
    if (d.amax && (int64_t)(p.tiles_m * t.n_full + tiles_m_half * (p.tiles_n - t.n_full)) * WAVES > amax_cap)
        return fail(ZB_EINVAL, "gemm_fp8: more partial maxima than amax_cap");
    int n_parts = 0;
    if (t.n_full > 0) {
        const int32_t rc = launch_f8<BM>(d, s, p.tiles_m, t.n_full, 0, p.sp);
        if (rc != ZB_OK) return rc;
        n_parts += p.tiles_m * t.n_full * WAVES;
    }
    if (t.n_full < p.tiles_n) {
        GemmDesc h = d;  // the half-height launch writes its maxima after the first launch's
        if (h.amax) h.amax += n_parts;
        const int32_t rc = launch_f8<BM / 2>(h, s, tiles_m_half, p.tiles_n - t.n_full, t.n_full, p.sp);
        if (rc != ZB_OK) return rc;
        n_parts += tiles_m_half * (p.tiles_n - t.n_full) * WAVES;
    }
    if (amax_n) *amax_n = d.amax ? n_parts : 0;
    return ZB_OK;
}

int32_t gemm_fp8_group(const GemmDesc* ds, int n, hipStream_t s) {
    if (n <= 0) return ZB_OK;
    if (n > GROUP_MAX) return fail(ZB_EINVAL, "gemm_fp8_group: at most 16 products");
    GemmGroup g{};
    g.n = n;
    g.off[0] = 0;
    for (int i = 0; i < n; ++i) {
        const V2Plan p = plan_f8(ds[i]);
        if (!p.ok || ds[i].epi != ds[0].epi || ds[i].M <= 0 || ds[i].N <= 0 || ds[i].K <= 0 ||
            ds[i].epi == EPI_SWIGLU_FWD)
            return fail(ZB_EINVAL, "gemm_fp8_group: a product does not fit the grouped fp8 kernel");
        g.d[i] = ds[i];
        g.tiles_m[i] = p.tiles_m;
        g.tiles_n[i] = p.tiles_n;
        g.sp[i] = p.sp;
        g.off[i + 1] = g.off[i] + ((p.tiles_m * p.tiles_n + 7) & ~7);
    }
    dim3 grid(g.off[n]), block(NTHR);
    switch (ds[0].epi) {
#define ZB_CASE(E) case E: hipLaunchKernelGGL((gemm_f8_group_kernel<E>), grid, block, 0, s, g); break;
        ZB_CASE(EPI_STORE)
        ZB_CASE(EPI_RESID)
        ZB_CASE(EPI_ACCUM_F32)
        ZB_CASE(EPI_GELU_FWD)
        ZB_CASE(EPI_GELU_BWD)
        ZB_CASE(EPI_SWIGLU_BWD)
#undef ZB_CASE
        default: return fail(ZB_EINVAL, "gemm_fp8_group: unknown epilogue");
    }
    ZB_HIP(hipGetLastError());
    return ZB_OK;
}

namespace {
// Sum of the split-K slices in slice order, then the product's epilogue (the
// same operations as the GEMM epilogue on an unsplit product); one thread per
// 4 consecutive columns of a row.
template <int EPI>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ part, int split, int M, int N,
                                                            bf16_t* __restrict__ C, int64_t ldc,
                                                            const bf16_t* __restrict__ R, int64_t ldr,
                                                            bf16_t* __restrict__ C2, int64_t ldc2) {
    const int64_t n4 = N / 4;
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= (int64_t)M * n4) return;
    const int64_t row = i / n4;
    const int col = (int)(i % n4) * 4;
    const int64_t slice = (int64_t)M * N;
    const float* p = part + row * N + col;
    floatx4 acc = *reinterpret_cast<const floatx4*>(p);
    for (int k = 1; k < split; ++k) acc += *reinterpret_cast<const floatx4*>(p + k * slice);
    u32x2 rw{0u, 0u};
    if constexpr (EPI == EPI_RESID || EPI == EPI_GELU_BWD) rw = *reinterpret_cast<const u32x2*>(R + row * ldr + col);
    float o[4], o2[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const float x = acc[e];
        const uint32_t w = rw[e >> 1];
        const float rv = (e & 1) ? __uint_as_float(w & 0xffff0000u) : __uint_as_float(w << 16);
        if (EPI == EPI_STORE) o[e] = x;
        else if (EPI == EPI_RESID) o[e] = x + rv;
        else if (EPI == EPI_GELU_FWD) { o[e] = x; o2[e] = gelu_tanh_f(x); }
        else if (EPI == EPI_GELU_BWD) o[e] = x * gelu_tanh_grad_f(rv);
    }
    *reinterpret_cast<u32x2*>(C + row * ldc + col) = pack_bf16x4(o);
    if constexpr (EPI == EPI_GELU_FWD) *reinterpret_cast<u32x2*>(C2 + row * ldc2 + col) = pack_bf16x4(o2);
}

bool splitk_epilogue(int epi) {
    return epi == EPI_STORE || epi == EPI_RESID || epi == EPI_GELU_FWD || epi == EPI_GELU_BWD;
}
}  // namespace

// K slices for a product whose half-height tiles would fill little of a
// 256-CU part: the largest power of two that keeps the slices' tiles within
// one round of 256 workgroups, each slice at least 512 deep and a multiple of
// the 64-k part.
int gemm_splitk_factor(const GemmDesc& d) {
    constexpr int64_t TARGET = 256;
    if (!d.a_kmajor || d.K1 != 0 || d.M <= 0 || d.N <= 0 || d.K <= 0 || d.N % 4 != 0 || !splitk_epilogue(d.epi))
        return 1;
    const int64_t tiles = (int64_t)((d.M + BM / 2 - 1) / (BM / 2)) * ((d.N + BN - 1) / BN);
    int split = 1;
    while (tiles * split * 2 <= TARGET && split * 2 <= GROUP_MAX && d.K % (split * 2 * BK64) == 0 &&
           d.K / (split * 2) >= 512)
        split *= 2;
    return split;
}

size_t gemm_splitk_scratch_bytes(int M, int N, int split) {
    return split > 1 ? (size_t)split * (size_t)M * (size_t)N * 4 : 0;
}

int32_t gemm_bf16_splitk(const GemmDesc& d, int split, float* part, hipStream_t s) {
    if (split <= 1) return gemm_bf16(d, s);
    if (split > GROUP_MAX || part == nullptr || !d.a_kmajor || d.K1 != 0 || d.K % (split * BK64) != 0 ||
        d.N % 4 != 0 || !splitk_epilogue(d.epi) || d.lda % 8 != 0 || d.ldb % 8 != 0 || (!d.b_kmajor && d.N % 8 != 0) ||
        ((reinterpret_cast<uintptr_t>(d.A) | reinterpret_cast<uintptr_t>(d.B) | reinterpret_cast<uintptr_t>(part)) & 15))
        return fail(ZB_EINVAL, "gemm: unsupported split-K product");
    const V2Plan whole = plan_v2(d);  // the epilogue's outputs must suit the vector accesses
    if (!whole.ok) return fail(ZB_EINVAL, "gemm: split-K product does not fit the kernel");
    const int ks = d.K / split;
    GemmGroup g{};
    g.n = split;
    g.off[0] = 0;
    for (int i = 0; i < split; ++i) {
        GemmDesc q = d;
        q.K = ks;
        q.A = static_cast<const char*>(d.A) + (size_t)i * ks * 2;
        q.B = static_cast<const char*>(d.B) + (d.b_kmajor ? (size_t)i * ks * 2 : (size_t)i * ks * d.ldb * 2);
        q.C = part + (size_t)i * d.M * d.N;
        q.ldc = d.N;
        q.epi = EPI_STORE_F32;
        q.R = nullptr;
        q.ldr = 0;
        q.C2 = nullptr;
        q.ldc2 = 0;
        q.half_n = 0;
        const V2Plan p = plan_v2(q);
        if (!p.ok) return fail(ZB_EINVAL, "gemm: split-K slice does not fit the kernel");
        const int tiles_m = (d.M + BM / 2 - 1) / (BM / 2);
        g.d[i] = q;
        g.tiles_m[i] = tiles_m;
        g.tiles_n[i] = p.tiles_n;
        g.sp[i] = p.sp;
        g.off[i + 1] = g.off[i] + ((tiles_m * p.tiles_n + 7) & ~7);
    }
    if (d.b_kmajor)
        hipLaunchKernelGGL((gemm_v2_group_kernel<true, true, EPI_STORE_F32, BM / 2>), dim3(g.off[g.n]), dim3(NTHR), 0, s, g);
    else
        hipLaunchKernelGGL((gemm_v2_group_kernel<true, false, EPI_STORE_F32, BM / 2>), dim3(g.off[g.n]), dim3(NTHR), 0, s,
                           g);
    ZB_HIP(hipGetLastError());
    const int64_t threads = (int64_t)d.M * (d.N / 4);
    const dim3 grid((unsigned)((threads + 255) / 256)), block(256);
    bf16_t* C = static_cast<bf16_t*>(d.C);
    const bf16_t* R = static_cast<const bf16_t*>(d.R);
    bf16_t* C2 = static_cast<bf16_t*>(d.C2);
    switch (d.epi) {
#define ZB_CASE(E) case E: hipLaunchKernelGGL((splitk_reduce_kernel<E>), grid, block, 0, s, part, split, d.M, d.N, C, d.ldc, R, d.ldr, C2, d.ldc2); break;
        ZB_CASE(EPI_STORE)
        ZB_CASE(EPI_RESID)
        ZB_CASE(EPI_GELU_FWD)
        ZB_CASE(EPI_GELU_BWD)
#undef ZB_CASE
        default: return fail(ZB_EINVAL, "gemm: unsupported split-K epilogue");
    }
    ZB_HIP(hipGetLastError());
    return ZB_OK;
}

int32_t gemm_bf16_group(const GemmDesc* ds, int n, hipStream_t s) {
    if (n <= 0) return ZB_OK;
    for (int i = 0; i < n; ++i)
        if (ds[i].K1 != 0) return fail(ZB_EINVAL, "gemm: a second K segment needs gemm_bf16_group_segmented");
    bool grouped = n <= GROUP_MAX && getenv("ZB_GEMM_V1") == nullptr;
    GemmGroup g{};
    g.n = n;
    g.off[0] = 0;
    for (int i = 0; i < n && grouped; ++i) {
        const GemmDesc& d = ds[i];
        const V2Plan p = plan_v2(d);
        // same layout and epilogue for every product; each must be valid for the single-product path too
        grouped = p.ok && d.a_kmajor == ds[0].a_kmajor && d.b_kmajor == ds[0].b_kmajor && d.epi == ds[0].epi &&
                  d.M > 0 && d.N > 0 && d.K > 0 && d.K % 8 == 0 && d.lda % 8 == 0 && d.ldb % 8 == 0 &&
                  (d.a_kmajor || d.M % 8 == 0) && (d.b_kmajor || d.N % 8 == 0) &&
                  ((reinterpret_cast<uintptr_t>(d.A) | reinterpret_cast<uintptr_t>(d.B)) & 15) == 0 &&
                  (d.epi != EPI_SWIGLU_FWD || (d.b_kmajor && d.half_n > 0));
        if (!grouped) break;
        g.d[i] = d;
        g.tiles_m[i] = p.tiles_m;
        g.tiles_n[i] = p.tiles_n;
        g.sp[i] = p.sp;
        g.off[i + 1] = g.off[i] + ((p.tiles_m * p.tiles_n + 7) & ~7);
    }
    if (!grouped) {  // one launch per product (validated there)
        for (int i = 0; i < n; ++i) {
            const int32_t rc = gemm_bf16(ds[i], s);
            if (rc != ZB_OK) return rc;
        }
        return ZB_OK;
    }
    const bool ak = ds[0].a_kmajor, bk = ds[0].b_kmajor;
    if (ak && bk) return launch_group<true, true>(g, ds[0].epi, s);
    if (ak && !bk) return launch_group<true, false>(g, ds[0].epi, s);
    if (!ak && !bk) return launch_group<false, false>(g, ds[0].epi, s);
    return launch_group<false, true>(g, ds[0].epi, s);
}

}  // namespace zb
