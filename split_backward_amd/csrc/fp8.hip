// Per-tensor E4M3 quantization of bf16 tensors for the fp8 stage's linear
// products.
//
// The pages name FP8 buffers as what makes room for a zero-bubble schedule's
// extra stash ("The Ghost in the Machine: Scaling Zero-Bubble Pipeline
// Parallelism", "Memory Pressure: The Hidden Cost of Efficiency") but give
// no format or scaling.  Here: OCP E4M3 codes (the gfx950 matrix core's
// fp8), one power-of-two scale 2^e per tensor with e the smallest integer
// such that max|x| <= 448 * 2^e, codes = x * 2^-e rounded to nearest, ties
// to even (the hardware conversion v_cvt_pk_fp8_f32).  x * 2^-e is exact in
// fp32, so the E4M3 rounding is the only rounding.
//
// Three kernels, all HBM-bound:
//   amax_partial_kernel   max|x| of row groups -> AMAX_PARTS partials
//   amax_final_kernel     max of the partials -> the exponent e (int32)
//   quantize_kernel       64 x 64 tiles: codes row-major [rows][cols] and/or
//                         transposed [cols][rows] (through LDS), so that a
//                         product's K index is contiguous whichever operand
//                         the tensor becomes.
#include <cmath>

#include "common.h"

namespace zb {
namespace {

constexpr int QT = 64;  // quantize tile (rows x cols)

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}

// Rows blockIdx.x, blockIdx.x + gridDim.x, ...; 8 columns per thread.
__global__ __launch_bounds__(256) void amax_partial_kernel(const bf16_t* __restrict__ x, int rows, int cols,
                                                           int64_t ld, float* __restrict__ part) {
    __shared__ float red[4];
    float m = 0.f;
    const int per_row = cols / 8;
    for (int r = blockIdx.x; r < rows; r += gridDim.x) {
        const bf16_t* row = x + (int64_t)r * ld;
        for (int c = threadIdx.x; c < per_row; c += 256) {
            const u32x4 v = *reinterpret_cast<const u32x4*>(row + c * 8);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                m = fmaxf(m, fabsf(__uint_as_float(v[i] << 16)));
                m = fmaxf(m, fabsf(__uint_as_float(v[i] & 0xffff0000u)));
            }
        }
    }
    m = wave_max(m);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) part[blockIdx.x] = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

// Smallest e with amax <= 448 * 2^e: amax = f * 2^x with f in [0.5, 1), so
// amax = (2f) * 2^(x-1) with 2f in [1, 2); 448 = 1.75 * 2^8, hence
// e = x - 9 if 2f <= 1.75, else x - 8.  0 for amax == 0.
__device__ __forceinline__ int scale_exponent(float amax) {
    if (!(amax > 0.f)) return 0;
    int x;
    const float f = __builtin_frexpf(amax, &x);
    return f <= 0.875f ? x - 9 : x - 8;
}

__global__ __launch_bounds__(256) void amax_final_kernel(const float* __restrict__ part, int nparts,
                                                         int32_t* __restrict__ e_out) {
    __shared__ float red[4];
    float m = 0.f;
    for (int i = threadIdx.x; i < nparts; i += 256) m = fmaxf(m, part[i]);
    m = wave_max(m);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) *e_out = scale_exponent(fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3])));
}

// One 64 x 64 tile per block (blockIdx.x: column tile, blockIdx.y: row
// tile); thread t converts 16 consecutive columns of row t / 4.  rows and
// cols are multiples of 16.  Codes of four values go into one dword with two
// packed conversions.
__global__ __launch_bounds__(256) void quantize_kernel(const bf16_t* __restrict__ x, int rows, int cols, int64_t ld,
                                                       const int32_t* __restrict__ e_in, uint8_t* __restrict__ q,
                                                       int64_t ldq, uint8_t* __restrict__ qt, int64_t ldqt) {
    __shared__ uint32_t tile[QT][QT / 4 + 1];  // codes, 4 per word, padded row
    const int tid = threadIdx.x;
    const int ne = -*e_in;  // x * 2^-e with v_ldexp_f32: exact, whatever the range of 2^-e
    const int r0 = blockIdx.y * QT, c0 = blockIdx.x * QT;
    const int rr = tid >> 2, cc = (tid & 3) * 16;
    const int r = r0 + rr, c = c0 + cc;
    uint32_t w[4] = {0u, 0u, 0u, 0u};
    if (r < rows && c < cols) {
        const bf16_t* src = x + (int64_t)r * ld + c;
        const u32x4 a = *reinterpret_cast<const u32x4*>(src);
        const u32x4 b = *reinterpret_cast<const u32x4*>(src + 8);
        const uint32_t v[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const float f0 = __builtin_ldexpf(__uint_as_float(v[2 * k] << 16), ne);
            const float f1 = __builtin_ldexpf(__uint_as_float(v[2 * k] & 0xffff0000u), ne);
            const float f2 = __builtin_ldexpf(__uint_as_float(v[2 * k + 1] << 16), ne);
            const float f3 = __builtin_ldexpf(__uint_as_float(v[2 * k + 1] & 0xffff0000u), ne);
            int p = __builtin_amdgcn_cvt_pk_fp8_f32(f0, f1, 0, false);
            p = __builtin_amdgcn_cvt_pk_fp8_f32(f2, f3, p, true);
            w[k] = (uint32_t)p;
        }
        if (q) *reinterpret_cast<u32x4*>(q + (int64_t)r * ldq + c) = u32x4{w[0], w[1], w[2], w[3]};
    }
    if (!qt) return;
#pragma unroll
    for (int k = 0; k < 4; ++k) tile[rr][cc / 4 + k] = w[k];
    __syncthreads();
    // transposed: thread t writes 16 codes of output row c0 + t / 4 (input
    // column), input rows r0 + (t % 4) * 16 .. + 15
    const int oc = tid >> 2, orow = (tid & 3) * 16;
    const int gc = c0 + oc, gr = r0 + orow;
    if (gc < cols && gr < rows) {
        uint32_t o[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            uint32_t acc = 0u;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t word = tile[orow + 4 * k + j][oc >> 2];
                acc |= ((word >> (8 * (oc & 3))) & 0xffu) << (8 * j);
            }
            o[k] = acc;
        }
        *reinterpret_cast<u32x4*>(qt + (int64_t)gc * ldqt + gr) = u32x4{o[0], o[1], o[2], o[3]};
    }
}

}  // namespace

int32_t quantize_e4m3(const bf16_t* x, int rows, int cols, int64_t ld, uint8_t* q, int64_t ldq, uint8_t* qt,
                      int64_t ldqt, int32_t* e_out, float* part, hipStream_t s) {
    if (!x || !e_out || !part || rows < 1 || cols < 1 || (!q && !qt))
        return fail(ZB_EINVAL, "quantize_e4m3: bad argument");
    if (rows % 16 || cols % 16 || ld % 8 || (q && ldq % 16) || (qt && ldqt % 16) || ld < cols || (q && ldq < cols) ||
        (qt && ldqt < rows))
        return fail(ZB_EINVAL, "quantize_e4m3: rows and cols must be multiples of 16, leading dimensions aligned");
    if ((reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(qt)) & 15)
        return fail(ZB_EINVAL, "quantize_e4m3: pointers must be 16-byte aligned");
    const int nparts = rows < AMAX_PARTS ? rows : AMAX_PARTS;
    hipLaunchKernelGGL(amax_partial_kernel, dim3(nparts), dim3(256), 0, s, x, rows, cols, ld, part);
    ZB_HIP(hipGetLastError());
    hipLaunchKernelGGL(amax_final_kernel, dim3(1), dim3(256), 0, s, part, nparts, e_out);
    ZB_HIP(hipGetLastError());
    hipLaunchKernelGGL(quantize_kernel, dim3((cols + QT - 1) / QT, (rows + QT - 1) / QT), dim3(256), 0, s, x, rows,
                       cols, ld, e_out, q, ldq, qt, ldqt);
    ZB_HIP(hipGetLastError());
    return ZB_OK;
}

}  // namespace zb
