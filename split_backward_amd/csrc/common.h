// Shared declarations of libzb: error reporting, launch helpers and the
// kernel launchers each translation unit provides.
#pragma once

#include <hip/hip_runtime.h>
#include <cstddef>
#include <cstdint>
#include <string>

#include "../../include/zb.h"

namespace zb {

// ---------------------------------------------------------------- errors --
void set_error(const std::string& msg);
int32_t fail(int32_t code, const std::string& msg);

#define ZB_HIP(expr)                                                             \
    do {                                                                         \
        hipError_t e_ = (expr);                                                  \
        if (e_ != hipSuccess)                                                    \
            return ::zb::fail(ZB_EHIP, std::string(#expr) + ": " + hipGetErrorString(e_)); \
    } while (0)

// Device types used by every kernel file.
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint16_t bf16_t;  // bfloat16 bit pattern in memory

__device__ __forceinline__ float bf2f(bf16_t v) { return __uint_as_float(uint32_t(v) << 16); }
// fp32 -> bf16, round to nearest even (gfx950 converts in hardware).
__device__ __forceinline__ bf16_t f2bf(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

// ------------------------------------------------------------ GEMM API ----
// Epilogues of the bf16 MFMA GEMM.  acc is the fp32 tile of A.B.
enum Epi : int {
    EPI_STORE = 0,        // C(bf16) = acc
    EPI_RESID = 1,        // C(bf16) = acc + R(bf16)                    (residual add)
    EPI_ACCUM_F32 = 2,    // C(f32) += acc                              (W pass)
    EPI_GELU_FWD = 3,     // C(bf16) = acc (pre-activation), C2(bf16) = gelu_tanh(acc)
    EPI_GELU_BWD = 4,     // C(bf16) = acc * gelu_tanh'(R)              (R = stashed pre-activation)
    EPI_SWIGLU_FWD = 5,   // paired tiles: C = [g | u] (bf16), C2 = silu(g) * u (bf16)
    EPI_SWIGLU_BWD = 6,   // acc = ds; R = [g | u]; C = [dg | du] (bf16)
    EPI_STORE_F32 = 7,    // C(f32) = acc                               (split-K partial sums)
};

struct GemmDesc {
    int M, N, K;
    int a_kmajor;                              // opA[m][k] = a_kmajor ? A[m*lda+k] : A[k*lda+m]
    int b_kmajor;                              // opB[k][n] = b_kmajor ? B[n*ldb+k] : B[k*ldb+n]
    int epi;
    int half_n;                                // EPI_SWIGLU_*: width of g (= ffn)
    // Second K segment (W over two microbatches): with K1 > 0, k < K1 reads
    // A and B and k >= K1 reads A2 and B2 at row k - K1 (same leading
    // dimensions, K = 2 * K1).  Only the grouped direct-to-LDS kernel with
    // both operands M/N-contiguous and EPI_ACCUM_F32 takes it
    // (gemm_bf16_group_segmented); every other path rejects K1 != 0.
    int K1;
    const void* A; int64_t lda;
    const void* B; int64_t ldb;
    void* C; int64_t ldc;
    const void* R; int64_t ldr;                // residual / stash operand of the epilogue
    void* C2; int64_t ldc2;                    // second output of the epilogue
    const void* A2;
    const void* B2;
    // fp8 products (gemm_fp8 / gemm_fp8_group): A and B hold E4M3 codes
    // (K-contiguous both) with per-tensor power-of-two scales 2^*ea, 2^*eb
    // read on the device; the epilogue sees acc * 2^(*ea + *eb).
    const int32_t* ea;
    const int32_t* eb;
    // fp8 stages, the SwiGLU epilogues only: per-wave max|output| (of the
    // tensor the next product quantizes: C2 = silu(g) u for EPI_SWIGLU_FWD,
    // C = [dg | du] for EPI_SWIGLU_BWD, as the bf16 values stored) to
    // amax[4 * workgroup + wave] of each launch; null elsewhere.
    float* amax;
};

int32_t gemm_bf16(const GemmDesc& d, hipStream_t s);
// Split-K for products whose tiles would fill little of the chip (K-contiguous
// A, epilogues STORE, RESID, GELU_FWD, GELU_BWD): gemm_splitk_factor(d) K
// slices (1 = none; chosen for 256 workgroups of half-height tiles), each
// storing its fp32 partial product in part[slice][M][N], then one pass that
// adds the slices in slice order and applies d's epilogue.  part holds
// gemm_splitk_scratch_bytes(d.M, d.N, split) bytes.
int gemm_splitk_factor(const GemmDesc& d);
size_t gemm_splitk_scratch_bytes(int M, int N, int split);
int32_t gemm_bf16_splitk(const GemmDesc& d, int split, float* part, hipStream_t s);
// Direct-to-LDS kernel; sets *handled = false (and does nothing) when an
// operand is too large for one buffer range or the epilogue cannot use
// vector accesses (the first-generation kernel then runs).
int32_t gemm_bf16_v2(const GemmDesc& d, hipStream_t s, bool* handled);
int32_t gemm_f32(const GemmDesc& d, int accumulate, hipStream_t s);
// n independent products of one layout and epilogue in a single launch when
// every one fits the direct-to-LDS kernel (else one gemm_bf16 each).
int32_t gemm_bf16_group(const GemmDesc* ds, int n, hipStream_t s);
// The same for products with a second K segment (K1 > 0).  Launches nothing
// and sets *handled = false unless every product fits one grouped launch of
// the direct-to-LDS kernel (both operands M/N-contiguous, EPI_ACCUM_F32,
// K = 2 * K1, K1 a multiple of 32); the caller then issues the segments as
// separate products.
int32_t gemm_bf16_group_segmented(const GemmDesc* ds, int n, hipStream_t s, bool* handled);
// C (epi)= (A . B^T) * 2^(ea + eb) with A [M, K], B [N, K] E4M3 codes, both
// K-contiguous (a_kmajor = b_kmajor = 1), K a multiple of 128, leading
// dimensions multiples of 16 bytes; any epilogue of the bf16 kernel.
// With d.amax set, *amax_n = the number of partial maxima written there; a
// product that would write more than amax_cap is rejected before any launch.
int32_t gemm_fp8(const GemmDesc& d, hipStream_t s, int* amax_n = nullptr, int amax_cap = 0);
// Up to 16 such products of one epilogue in one launch.
int32_t gemm_fp8_group(const GemmDesc* ds, int n, hipStream_t s);

// ------------------------------------------------------- fp8 operands ----
// Per-tensor E4M3 quantization of a bf16 [rows, cols] matrix (leading
// dimension ld): *e_out = the smallest e with max|x| <= 448 * 2^e, codes of
// x * 2^-e (round to nearest even) row-major into q (ldq) and/or transposed
// ([cols][rows]) into qt (ldqt); either may be null.  rows and cols are
// multiples of 16.  part: AMAX_PARTS floats of scratch.
constexpr int AMAX_PARTS = 512;
int32_t quantize_e4m3(const bf16_t* x, int rows, int cols, int64_t ld, uint8_t* q, int64_t ldq, uint8_t* qt,
                      int64_t ldqt, int32_t* e_out, float* part, hipStream_t s);
// The same for a tensor whose producer already wrote partial maxima of
// |x| (part[0..nparts), every element of x covered by one of them): one
// small kernel reduces them into *amax, then the codes; no pass over x for
// its maximum.
int32_t quantize_e4m3_from_partials(const bf16_t* x, int rows, int cols, int64_t ld, uint8_t* q, int64_t ldq,
                                    uint8_t* qt, int64_t ldqt, int32_t* e_out, const float* part, int nparts,
                                    float* amax, hipStream_t s);

// ------------------------------------------------- elementwise / norms ----
int32_t fill_f32(float* p, size_t n, float v, hipStream_t s);
// fp32 w -= lr * dw, elementwise, the product and the difference each
// rounded once.
int32_t sgd_step_f32(float* w, const float* dw, size_t n, float lr, hipStream_t s);
// bf16 w -= lr * dw for up to SGD_GROUP_MAX weights in one launch: fp32
// product and difference each rounded once, then rounded once to bf16
// (round to nearest even); each dW is cleared as it is consumed.
// n4 = elements / 4 (bf16 stages have widths divisible by 8).
constexpr int SGD_GROUP_MAX = 64;
struct SgdSeg {
    void* w;
    float* dw;
    size_t n4;
};
struct SgdGroup {
    SgdSeg seg[SGD_GROUP_MAX];
    int n;
    float lr;
};
int32_t sgd_step_group_bf16(const SgdGroup& g, hipStream_t s);
int32_t copy_bytes(void* dst, const void* src, size_t n, hipStream_t s);
// dst [cols, rows] = transpose of the bf16 matrix src [rows, cols].
int32_t transpose_bf16(const bf16_t* src, bf16_t* dst, int rows, int cols, hipStream_t s);
// n = RMS(x) * g, r = 1/sqrt(mean(x^2)+eps) per row; x, n bf16 [T, H]; r f32 [T].
// xcopy (optional): receives a copy of x.
// amax_rows (optional): max|n| of each row (the stored bf16 values), T floats.
int32_t rmsnorm_fwd(const bf16_t* x, const bf16_t* g, bf16_t* n, float* r, int T, int H, float eps,
                    hipStream_t s, bf16_t* xcopy = nullptr, float* amax_rows = nullptr);
// dx = dres + r * (dn*g - xhat * mean(dn*g*xhat)), xhat = x*r.
// rescopy (optional): receives a copy of dres.
// amax_rows (optional): max|dx| of each row (the stored bf16 values), T floats.
int32_t rmsnorm_bwd(const bf16_t* x, const float* r, const bf16_t* g, const bf16_t* dn,
                    const bf16_t* dres, bf16_t* dx, int T, int H, hipStream_t s, bf16_t* rescopy = nullptr,
                    float* amax_rows = nullptr);
// dgamma[h] += sum_t dn[t,h] * x[t,h] * r[t]   (partials in scratch, fixed order)
int32_t rmsnorm_dgamma(const bf16_t* x, const float* r, const bf16_t* dn, float* dgamma,
                       float* scratch, int T, int H, hipStream_t s);
size_t rmsnorm_dgamma_scratch_floats(int T, int H);

// -------------------------------------------------------------- attention --
// Causal GQA attention, head_dim 128.  q/k/v are column blocks of the packed
// qkv [T, (nq + 2 nkv) * 128] buffer; o [T, nq*128]; lse f32 [nq, T].
// With `amax` set, every wave that stores o also leaves the largest magnitude
// it stored (a bf16 value widened to f32) in amax[0 .. *amax_n); the count is
// at most attn_amax_parts(T, nq, nkv).
int32_t attn_fwd(const bf16_t* qkv, bf16_t* o, float* lse, int T, int nq, int nkv, hipStream_t s,
                 float* amax = nullptr, int* amax_n = nullptr);
int64_t attn_amax_parts(int T, int nq, int nkv);
// dqkv [T, (nq + 2 nkv)*128]; delta scratch f32 [nq, T]; scratch: device
// memory of attn_bwd_scratch_bytes(T, nq, nkv) bytes (dS^T in bf16
// [nq][T][T], then fp32 partial dK, dV when the query heads of a KV head are
// split over workgroups).
size_t attn_bwd_scratch_bytes(int T, int nq, int nkv);
// `amax`, `amax_n`: as for attn_fwd, over every element of dqkv.
int32_t attn_bwd(const bf16_t* qkv, const bf16_t* o, const float* lse, const bf16_t* dout,
                 bf16_t* dqkv, float* delta, void* scratch, int T, int nq, int nkv, hipStream_t s,
                 float* amax = nullptr, int* amax_n = nullptr);

// ---------------------------------------------------------------- debug ---
// Ring-slot tags (debug.hip): tags[slot] = 4 * mb + phase (1 F, 2 B, 3 W
// done), -1 = unused.  slot_tag checks tags[slot] against `expect` (a tag,
// TAG_FREE = unused or phase 3, TAG_ANY = no check), records a mismatch in
// rec[0..5] = {count, op, mb, slot, found, expected}, then stores `set`
// unless it is TAG_KEEP.
constexpr int TAG_FREE = -2, TAG_ANY = -3, TAG_KEEP = -4;
constexpr int DEBUG_REC = 8;  // int32 words of the mismatch record
int32_t slot_tag(int32_t* tags, int32_t* rec, int slot, int op, int mb, int expect, int set, hipStream_t s);
// tags[0..n) = -1, rec[0..DEBUG_REC) = 0.
int32_t tag_reset(int32_t* tags, int n, int32_t* rec, hipStream_t s);

// --------------------------------------------------------------- timing ---
int32_t stamp_now(uint64_t* dst, hipStream_t s);
int32_t wait_until(const uint64_t* t0, uint64_t delta_ticks, uint64_t* wait_end, hipStream_t s);
uint64_t wall_clock_hz();

}  // namespace zb
