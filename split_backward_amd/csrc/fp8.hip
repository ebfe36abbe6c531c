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
// Two kernels, both HBM-bound:
//   amax_partial_kernel   max|x| of grid-strided 16-byte chunks -> up to
//                         AMAX_PARTS partial maxima
//   quantize_kernel       the exponent from the partials (every block), then
//                         128 x 64 tiles: codes row-major [rows][cols] and/or
//                         transposed [cols][rows] (through LDS), so that a
//                         product's K index is contiguous whichever operand
//                         the tensor becomes.
// Where the kernel that wrote x already produced partial maxima (the RMSNorm
// kernels per row, the SwiGLU GEMM epilogues and the attention kernels per
// storing wave), amax_reduce_kernel
// folds them into one value instead of the pass over x.
#include <algorithm>
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

// max|x| over the matrix in 16-byte chunks (8 values), chunk c of a grid
// stride loop at row c / (cols / 8); four loads in flight per thread.
__global__ __launch_bounds__(256) void amax_partial_kernel(const bf16_t* __restrict__ x, int rows, int cols,
                                                           int64_t ld, float* __restrict__ part) {
    __shared__ float red[4];
    float m = 0.f;
    const uint32_t per_row = (uint32_t)cols / 8, total = (uint32_t)rows * per_row;
    const uint32_t stride = gridDim.x * 256u;
    auto at = [&](uint32_t c) {
        const uint32_t r = c / per_row, k = c - r * per_row;
        return *reinterpret_cast<const u32x4*>(x + (int64_t)r * ld + (int64_t)k * 8);
    };
    auto fold = [&](const u32x4& v) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            m = fmaxf(m, fabsf(__uint_as_float(v[i] << 16)));
            m = fmaxf(m, fabsf(__uint_as_float(v[i] & 0xffff0000u)));
        }
    };
    uint32_t c = blockIdx.x * 256u + threadIdx.x;
    for (; c + 3 * stride < total; c += 4 * stride) {
        const u32x4 v0 = at(c), v1 = at(c + stride), v2 = at(c + 2 * stride), v3 = at(c + 3 * stride);
        fold(v0);
        fold(v1);
        fold(v2);
        fold(v3);
    }
    for (; c < total; c += stride) fold(at(c));
    m = wave_max(m);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) part[blockIdx.x] = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

// max of n partial maxima into *out (one workgroup; max is exact, so the
// order does not matter)
__global__ __launch_bounds__(1024) void amax_reduce_kernel(const float* __restrict__ part, int n,
                                                          float* __restrict__ out) {
    __shared__ float red[16];
    float m = 0.f;
    for (int i = threadIdx.x; i < n; i += 1024) m = fmaxf(m, part[i]);
    m = wave_max(m);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
        float t = red[0];
        for (int i = 1; i < 16; ++i) t = fmaxf(t, red[i]);
        *out = t;
    }
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

// One QR x 64 tile per block (QR = 64 RG; blockIdx.x: column tile,
// blockIdx.y: row tile); thread t converts 16 consecutive columns of rows
// t / 4 + 64 g, g < RG.  rows and cols are multiples of 16.  Codes of four
// values go into one dword with two packed conversions.
template <int RG>
__global__ __launch_bounds__(256) void quantize_kernel(const bf16_t* __restrict__ x, int rows, int cols, int64_t ld,
                                                       const float* __restrict__ part, int nparts,
                                                       int32_t* __restrict__ e_out, uint8_t* __restrict__ q,
                                                       int64_t ldq, uint8_t* __restrict__ qt, int64_t ldqt) {
    constexpr int QR = 64 * RG;
    __shared__ uint32_t tile[QR][QT / 4 + 1];  // codes, 4 per word, padded row
    __shared__ float red[4];
    const int tid = threadIdx.x;
    const int r0 = blockIdx.y * QR, c0 = blockIdx.x * QT;
    const int rr = tid >> 2, cc = (tid & 3) * 16;
    const int c = c0 + cc;
    // the tile's values are requested before the partial maxima, so that a
    // block waits for one memory round trip, not two in a row
    u32x4 a[RG], b[RG];
    bool in[RG];
#pragma unroll
    for (int g = 0; g < RG; ++g) {
        const int r = r0 + rr + 64 * g;
        in[g] = r < rows && c < cols;
        a[g] = u32x4{0u, 0u, 0u, 0u};
        b[g] = u32x4{0u, 0u, 0u, 0u};
        if (in[g]) {
            const bf16_t* src = x + (int64_t)r * ld + c;
            a[g] = *reinterpret_cast<const u32x4*>(src);
            b[g] = *reinterpret_cast<const u32x4*>(src + 8);
        }
    }
    // every block reduces the partial maxima itself (the same values in the
    // same order, so the same exponent); block (0, 0) publishes it
    float am = 0.f;
    for (int i = tid; i < nparts; i += 256) am = fmaxf(am, part[i]);
    am = wave_max(am);
    if ((tid & 63) == 0) red[tid >> 6] = am;
    __syncthreads();
    const int e = scale_exponent(fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3])));
    if (tid == 0 && blockIdx.x == 0 && blockIdx.y == 0) *e_out = e;
    const int ne = -e;  // x * 2^-e with v_ldexp_f32: exact, whatever the range of 2^-e
#pragma unroll
    for (int g = 0; g < RG; ++g) {
        uint32_t w[4] = {0u, 0u, 0u, 0u};
        if (in[g]) {
            const uint32_t v[8] = {a[g][0], a[g][1], a[g][2], a[g][3], b[g][0], b[g][1], b[g][2], b[g][3]};
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
            if (q) *reinterpret_cast<u32x4*>(q + (int64_t)(r0 + rr + 64 * g) * ldq + c) = u32x4{w[0], w[1], w[2], w[3]};
        }
        if (qt) {
#pragma unroll
            for (int k = 0; k < 4; ++k) tile[rr + 64 * g][cc / 4 + k] = w[k];
        }
    }
    if (!qt) return;
    __syncthreads();
    // transposed: thread t writes 16 codes of output row c0 + t / 4 (input
    // column) for each g: input rows r0 + (t % 4) * 16 + 64 g .. + 15
    const int oc = tid >> 2, gc = c0 + oc;
#pragma unroll
    for (int g = 0; g < RG; ++g) {
        const int orow = (tid & 3) * 16 + 64 * g, gr = r0 + orow;
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
}

// Rows per quantize tile: 64 QRG.
constexpr int QRG = 2;

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
    const int64_t chunks = (int64_t)rows * (cols / 8);
    if (chunks >= (int64_t)1 << 31) return fail(ZB_EINVAL, "quantize_e4m3: tensor too large");
    const int nparts = (int)std::min<int64_t>(AMAX_PARTS, (chunks + 1023) / 1024);
    hipLaunchKernelGGL(amax_partial_kernel, dim3(nparts), dim3(256), 0, s, x, rows, cols, ld, part);
    ZB_HIP(hipGetLastError());
    hipLaunchKernelGGL(quantize_kernel<QRG>, dim3((cols + QT - 1) / QT, (rows + 64 * QRG - 1) / (64 * QRG)), dim3(256), 0, s, x, rows,
                       cols, ld, part, nparts, e_out, q, ldq, qt, ldqt);
    ZB_HIP(hipGetLastError());
    return ZB_OK;
}

int32_t quantize_e4m3_from_partials(const bf16_t* x, int rows, int cols, int64_t ld, uint8_t* q, int64_t ldq,
                                    uint8_t* qt, int64_t ldqt, int32_t* e_out, const float* part, int nparts,
                                    float* amax, hipStream_t s) {
    if (!x || !e_out || !part || !amax || nparts < 1 || rows < 1 || cols < 1 || (!q && !qt))
        return fail(ZB_EINVAL, "quantize_e4m3_from_partials: bad argument");
    if (rows % 16 || cols % 16 || ld % 8 || (q && ldq % 16) || (qt && ldqt % 16) || ld < cols || (q && ldq < cols) ||
        (qt && ldqt < rows))
        return fail(ZB_EINVAL, "quantize_e4m3: rows and cols must be multiples of 16, leading dimensions aligned");
    if ((reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(qt)) & 15)
        return fail(ZB_EINVAL, "quantize_e4m3: pointers must be 16-byte aligned");
    hipLaunchKernelGGL(amax_reduce_kernel, dim3(1), dim3(1024), 0, s, part, nparts, amax);
    ZB_HIP(hipGetLastError());
    hipLaunchKernelGGL(quantize_kernel<QRG>, dim3((cols + QT - 1) / QT, (rows + 64 * QRG - 1) / (64 * QRG)), dim3(256), 0, s, x, rows,
                       cols, ld, amax, 1, e_out, q, ldq, qt, ldqt);
    ZB_HIP(hipGetLastError());
    return ZB_OK;
}

}  // namespace zb
