// Memory-bound kernels of the Llama stage: RMSNorm forward / input backward,
// the RMSNorm gain gradient (a weight gradient, so it belongs to W), fills,
// and the executor's clock kernels.
//
// RMSNorm: y = x r g with r = (mean(x^2) + eps)^(-1/2);
//          dx = r (dy g - xhat mean(dy g xhat)), xhat = x r;  dg = sum_t dy xhat.
#include <algorithm>

#include "common.h"

namespace zb {
namespace {

constexpr int RT = 256;  // threads per row block

__device__ __forceinline__ float block_sum(float v, float* red) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
    if (l == 0) red[w] = v;
    __syncthreads();
    float t = 0.f;
#pragma unroll
    for (int i = 0; i < RT / 64; ++i) t += red[i];
    __syncthreads();
    return t;
}

// max over the workgroup, written by thread 0 to *out as the bf16 value it
// rounds to (rounding is monotonic, so that is the largest stored |value|)
__device__ __forceinline__ void block_max_to(float v, float* red, float* out) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
    if (l == 0) red[w] = v;
    __syncthreads();
    if (threadIdx.x == 0) {
        float t = red[0];
#pragma unroll
        for (int i = 1; i < RT / 64; ++i) t = fmaxf(t, red[i]);
        *out = __uint_as_float((uint32_t)f2bf(t) << 16);
    }
}

__device__ __forceinline__ void unpack8(const u32x4 v, float (&f)[8]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[2 * i] = __uint_as_float(v[i] << 16);
        f[2 * i + 1] = __uint_as_float(v[i] & 0xffff0000u);
    }
}
__device__ __forceinline__ u32x4 pack8(const float (&f)[8]) {
    u32x4 v;
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = uint32_t(f2bf(f[2 * i])) | (uint32_t(f2bf(f[2 * i + 1])) << 16);
    return v;
}

// One workgroup per row; H is a multiple of 8 and at most 8 * RT * 4.
// xcopy (optional): a copy of x written as it is read (the stage stashes
// its input this way instead of with a separate copy).  amax (optional):
// max|n| of the row at amax[row].
template <int CH>
__global__ __launch_bounds__(RT) void rms_fwd_kernel(const bf16_t* __restrict__ x, const bf16_t* __restrict__ g,
                                                     bf16_t* __restrict__ n, float* __restrict__ r,
                                                     bf16_t* __restrict__ xcopy, float* __restrict__ amax, int H,
                                                     float eps) {
    __shared__ float red[RT / 64];
    const int64_t row = blockIdx.x;
    const bf16_t* xr = x + row * H;
    float v[CH][8];
    float ss = 0.f;
#pragma unroll
    for (int c = 0; c < CH; ++c) {
        const int col = (threadIdx.x + c * RT) * 8;
        if (col < H) {
            const u32x4 raw = *reinterpret_cast<const u32x4*>(xr + col);
            if (xcopy) *reinterpret_cast<u32x4*>(xcopy + row * H + col) = raw;
            unpack8(raw, v[c]);
#pragma unroll
            for (int i = 0; i < 8; ++i) ss += v[c][i] * v[c][i];
        }
    }
    const float tot = block_sum(ss, red);
    const float rr = 1.f / sqrtf(tot / float(H) + eps);
    if (threadIdx.x == 0) r[row] = rr;
    float mx = 0.f;
#pragma unroll
    for (int c = 0; c < CH; ++c) {
        const int col = (threadIdx.x + c * RT) * 8;
        if (col < H) {
            float gg[8], o[8];
            unpack8(*reinterpret_cast<const u32x4*>(g + col), gg);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                o[i] = v[c][i] * rr * gg[i];
                mx = fmaxf(mx, fabsf(o[i]));
            }
            *reinterpret_cast<u32x4*>(n + row * H + col) = pack8(o);
        }
    }
    if (amax) block_max_to(mx, red, amax + row);
}

// rescopy (optional): a copy of dres written as it is read.  amax
// (optional): max|dx| of the row at amax[row].
template <int CH>
__global__ __launch_bounds__(RT) void rms_bwd_kernel(const bf16_t* __restrict__ x, const float* __restrict__ r,
                                                     const bf16_t* __restrict__ g, const bf16_t* __restrict__ dn,
                                                     const bf16_t* __restrict__ dres, bf16_t* __restrict__ dx,
                                                     bf16_t* __restrict__ rescopy, float* __restrict__ amax, int H) {
    __shared__ float red[RT / 64];
    const int64_t row = blockIdx.x;
    const float rr = r[row];
    float xh[CH][8], dg[CH][8];
    float dot = 0.f;
#pragma unroll
    for (int c = 0; c < CH; ++c) {
        const int col = (threadIdx.x + c * RT) * 8;
        if (col < H) {
            float gg[8];
            unpack8(*reinterpret_cast<const u32x4*>(x + row * H + col), xh[c]);
            unpack8(*reinterpret_cast<const u32x4*>(dn + row * H + col), dg[c]);
            unpack8(*reinterpret_cast<const u32x4*>(g + col), gg);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                xh[c][i] *= rr;
                dg[c][i] *= gg[i];
                dot += dg[c][i] * xh[c][i];
            }
        }
    }
    const float mean = block_sum(dot, red) / float(H);
    float mx = 0.f;
#pragma unroll
    for (int c = 0; c < CH; ++c) {
        const int col = (threadIdx.x + c * RT) * 8;
        if (col < H) {
            float res[8], o[8];
            const u32x4 raw = *reinterpret_cast<const u32x4*>(dres + row * H + col);
            if (rescopy) *reinterpret_cast<u32x4*>(rescopy + row * H + col) = raw;
            unpack8(raw, res);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                o[i] = res[i] + rr * (dg[c][i] - xh[c][i] * mean);
                mx = fmaxf(mx, fabsf(o[i]));
            }
            *reinterpret_cast<u32x4*>(dx + row * H + col) = pack8(o);
        }
    }
    if (amax) block_max_to(mx, red, amax + row);
}

// dgamma partials.  Block (column block of 512, row chunk of DG_ROWS rows):
// each lane owns 8 consecutive columns (16-byte loads of x and dn), each of
// the 4 waves a quarter of the chunk's rows with all its loads in flight;
// the waves' sums are combined in LDS in a fixed order (deterministic).
constexpr int DG_ROWS = 64, DG_WROWS = DG_ROWS / 4;
__global__ __launch_bounds__(256) void dgamma_partial_kernel(const bf16_t* __restrict__ x, const float* __restrict__ r,
                                                             const bf16_t* __restrict__ dn, float* __restrict__ part,
                                                             int T, int H) {
    __shared__ float red[4][512];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int c0 = blockIdx.x * 512 + lane * 8;
    const int t0 = blockIdx.y * DG_ROWS + wave * DG_WROWS;
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.f;
    if (c0 < H) {
        u32x4 xv[DG_WROWS], dv[DG_WROWS];
        float rv[DG_WROWS];
#pragma unroll
        for (int i = 0; i < DG_WROWS; ++i) {
            const int t = t0 + i;
            if (t < T) {
                xv[i] = *reinterpret_cast<const u32x4*>(x + (int64_t)t * H + c0);
                dv[i] = *reinterpret_cast<const u32x4*>(dn + (int64_t)t * H + c0);
                rv[i] = r[t];
            } else {
                xv[i] = dv[i] = u32x4{0, 0, 0, 0};
                rv[i] = 0.f;
            }
        }
#pragma unroll
        for (int i = 0; i < DG_WROWS; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t xw = xv[i][e], dw = dv[i][e];
                acc[2 * e] += __uint_as_float(dw << 16) * (__uint_as_float(xw << 16) * rv[i]);
                acc[2 * e + 1] += __uint_as_float(dw & 0xffff0000u) * (__uint_as_float(xw & 0xffff0000u) * rv[i]);
            }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) red[wave][lane * 8 + e] = acc[e];
    __syncthreads();
    for (int j = threadIdx.x; j < 512; j += 256) {
        const int col = blockIdx.x * 512 + j;
        if (col < H) part[(int64_t)blockIdx.y * H + col] = ((red[0][j] + red[1][j]) + red[2][j]) + red[3][j];
    }
}

// dgamma += sum of the chunk partials.  A workgroup owns 64 columns; its four
// waves each sum a quarter of the chunks (in ascending order, four
// independent partial sums per column to keep loads in flight) and the
// quarters are added in order: a fixed order, so deterministic, with four
// times the loads in flight of one wave per column.
__global__ __launch_bounds__(256) void dgamma_reduce_kernel(const float* __restrict__ part, float* __restrict__ dgamma,
                                                            int nchunks, int H) {
    __shared__ float red[4][64];
    const int lc = threadIdx.x & 63, q = threadIdx.x >> 6;
    const int col = blockIdx.x * 64 + lc;
    const int per = (nchunks + 3) / 4;
    const int c1 = min(nchunks, (q + 1) * per);
    float s[4] = {0.f, 0.f, 0.f, 0.f};
    if (col < H) {
        int c = q * per;
        for (; c + 4 <= c1; c += 4)
#pragma unroll
            for (int k = 0; k < 4; ++k) s[k] += part[(int64_t)(c + k) * H + col];
        for (; c < c1; ++c) s[0] += part[(int64_t)c * H + col];
    }
    red[q][lc] = (s[0] + s[1]) + (s[2] + s[3]);
    __syncthreads();
    if (q == 0 && col < H) dgamma[col] += ((red[0][lc] + red[1][lc]) + red[2][lc]) + red[3][lc];
}

__global__ void fill_f32_kernel(float* p, size_t n, float v) {
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) p[i] = v;
}

// Optimizer step w -= lr * dW, in fp32 with the product and the difference
// each rounded once (no fused multiply-add: contraction is switched off in
// these kernels; the __fmul_rn / __fsub_rn helpers are fused regardless,
// because they are inlined from headers that allow it), then w rounded once
// to the weight's type (bf16: round to nearest even).
// All bf16 weights of a stage in one launch: segment blockIdx.y, grid-stride
// over its groups of four; dW is cleared as it is consumed (the step ends
// an iteration), so no separate fill pass follows.
__global__ void sgd_bf16_group_kernel(SgdGroup g) {
#pragma clang fp contract(off)
    const SgdSeg sg = g.seg[blockIdx.y];
    bf16_t* __restrict__ w = static_cast<bf16_t*>(sg.w);
    float* __restrict__ dw = sg.dw;
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < sg.n4; i += stride) {
        const floatx4 d = reinterpret_cast<const floatx4*>(dw)[i];
        u32x2 v = reinterpret_cast<const u32x2*>(w)[i];
        float x[4] = {__uint_as_float(v[0] << 16), __uint_as_float(v[0] & 0xffff0000u), __uint_as_float(v[1] << 16),
                      __uint_as_float(v[1] & 0xffff0000u)};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float t = g.lr * d[e];
            x[e] = x[e] - t;
        }
        v[0] = uint32_t(f2bf(x[0])) | (uint32_t(f2bf(x[1])) << 16);
        v[1] = uint32_t(f2bf(x[2])) | (uint32_t(f2bf(x[3])) << 16);
        reinterpret_cast<u32x2*>(w)[i] = v;
        reinterpret_cast<floatx4*>(dw)[i] = floatx4{0.f, 0.f, 0.f, 0.f};
    }
}

__global__ void sgd_f32_kernel(float* __restrict__ w, const float* __restrict__ dw, size_t n, float lr) {
#pragma clang fp contract(off)
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
        const float t = lr * dw[i];
        w[i] = w[i] - t;
    }
}

__global__ void stamp_kernel(uint64_t* dst) {
    if (threadIdx.x == 0) *dst = wall_clock64();
}

// Spin until the device wall clock reaches *t0 + delta.  The deadline is at
// most `delta` ticks after the kernel starts (t0 lies in the past), and a
// hard cap ends the wait regardless, so every launch finishes.
__global__ void wait_kernel(const uint64_t* t0, uint64_t delta, uint64_t cap, uint64_t* wait_end) {
    if (threadIdx.x != 0) return;
    const uint64_t start = wall_clock64();
    const uint64_t deadline = __atomic_load_n(t0, __ATOMIC_RELAXED) + delta;
    const uint64_t limit = start + cap;
    uint64_t now = start;
    while (now < deadline && now < limit) {
        __builtin_amdgcn_s_sleep(1);
        now = wall_clock64();
    }
    if (wait_end) *wait_end = now;
}

// dst[c][r] = src[r][c] for a bf16 [rows, cols] matrix, through a 64 x 64
// LDS tile per workgroup: each thread reads 16 consecutive columns of one
// row (two 16-byte loads when they lie inside the matrix and its rows are
// 16-byte aligned, else element by element) and writes 16 consecutive
// columns of one output row the same way.
__global__ __launch_bounds__(256) void transpose_bf16_kernel(const bf16_t* __restrict__ src, bf16_t* __restrict__ dst,
                                                             int rows, int cols) {
    __shared__ bf16_t tile[64][64 + 2];
    const int r0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
    const int tr = threadIdx.x >> 2, tc = (threadIdx.x & 3) * 16;
    {
        const int r = r0 + tr, c = c0 + tc;
        if (r < rows && c + 16 <= cols && (cols & 7) == 0 && (reinterpret_cast<uintptr_t>(src) & 15) == 0) {
            const u32x4* p = reinterpret_cast<const u32x4*>(src + (int64_t)r * cols + c);
            const u32x4 v0 = p[0], v1 = p[1];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                tile[tr][tc + 2 * j] = (bf16_t)(v0[j] & 0xffffu);
                tile[tr][tc + 2 * j + 1] = (bf16_t)(v0[j] >> 16);
                tile[tr][tc + 8 + 2 * j] = (bf16_t)(v1[j] & 0xffffu);
                tile[tr][tc + 8 + 2 * j + 1] = (bf16_t)(v1[j] >> 16);
            }
        } else {
#pragma unroll
            for (int j = 0; j < 16; ++j)
                tile[tr][tc + j] = (r < rows && c + j < cols) ? src[(int64_t)r * cols + c + j] : (bf16_t)0;
        }
    }
    __syncthreads();
    const int orow = c0 + tr, ocol = r0 + tc;  // dst[orow][ocol + j] = src[ocol + j][orow]
    if (orow < cols && ocol + 16 <= rows && (rows & 7) == 0 && (reinterpret_cast<uintptr_t>(dst) & 15) == 0) {
        u32x4 v0, v1;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            v0[j] = uint32_t(tile[tc + 2 * j][tr]) | (uint32_t(tile[tc + 2 * j + 1][tr]) << 16);
            v1[j] = uint32_t(tile[tc + 8 + 2 * j][tr]) | (uint32_t(tile[tc + 8 + 2 * j + 1][tr]) << 16);
        }
        u32x4* q = reinterpret_cast<u32x4*>(dst + (int64_t)orow * rows + ocol);
        q[0] = v0;
        q[1] = v1;
    } else if (orow < cols) {
#pragma unroll
        for (int j = 0; j < 16; ++j)
            if (ocol + j < rows) dst[(int64_t)orow * rows + ocol + j] = tile[tc + j][tr];
    }
}

template <int CH>
int32_t launch_rms_fwd(const bf16_t* x, const bf16_t* g, bf16_t* n, float* r, bf16_t* xcopy, float* amax, int T, int H,
                       float eps, hipStream_t s) {
    hipLaunchKernelGGL(rms_fwd_kernel<CH>, dim3(T), dim3(RT), 0, s, x, g, n, r, xcopy, amax, H, eps);
    ZB_HIP(hipGetLastError());
    return ZB_OK;
}
template <int CH>
int32_t launch_rms_bwd(const bf16_t* x, const float* r, const bf16_t* g, const bf16_t* dn, const bf16_t* dres,
                       bf16_t* dx, bf16_t* rescopy, float* amax, int T, int H, hipStream_t s) {
    hipLaunchKernelGGL(rms_bwd_kernel<CH>, dim3(T), dim3(RT), 0, s, x, r, g, dn, dres, dx, rescopy, amax, H);
    ZB_HIP(hipGetLastError());
    return ZB_OK;
}

}  // namespace

int32_t rmsnorm_fwd(const bf16_t* x, const bf16_t* g, bf16_t* n, float* r, int T, int H, float eps, hipStream_t s,
                    bf16_t* xcopy, float* amax_rows) {
    if (H % 8 || H > 8 * RT * 4 || T <= 0) return fail(ZB_EINVAL, "rmsnorm: hidden must be a multiple of 8 and <= 8192");
    const int ch = (H / 8 + RT - 1) / RT;
    if (ch <= 1) return launch_rms_fwd<1>(x, g, n, r, xcopy, amax_rows, T, H, eps, s);
    if (ch <= 2) return launch_rms_fwd<2>(x, g, n, r, xcopy, amax_rows, T, H, eps, s);
    return launch_rms_fwd<4>(x, g, n, r, xcopy, amax_rows, T, H, eps, s);
}

int32_t rmsnorm_bwd(const bf16_t* x, const float* r, const bf16_t* g, const bf16_t* dn, const bf16_t* dres,
                    bf16_t* dx, int T, int H, hipStream_t s, bf16_t* rescopy, float* amax_rows) {
    if (H % 8 || H > 8 * RT * 4 || T <= 0) return fail(ZB_EINVAL, "rmsnorm: hidden must be a multiple of 8 and <= 8192");
    const int ch = (H / 8 + RT - 1) / RT;
    if (ch <= 1) return launch_rms_bwd<1>(x, r, g, dn, dres, dx, rescopy, amax_rows, T, H, s);
    if (ch <= 2) return launch_rms_bwd<2>(x, r, g, dn, dres, dx, rescopy, amax_rows, T, H, s);
    return launch_rms_bwd<4>(x, r, g, dn, dres, dx, rescopy, amax_rows, T, H, s);
}

int32_t transpose_bf16(const bf16_t* src, bf16_t* dst, int rows, int cols, hipStream_t s) {
    if (!src || !dst || rows < 1 || cols < 1) return fail(ZB_EINVAL, "transpose_bf16: bad argument");
    hipLaunchKernelGGL(transpose_bf16_kernel, dim3((cols + 63) / 64, (rows + 63) / 64), dim3(256), 0, s, src, dst, rows,
                       cols);
    ZB_HIP(hipGetLastError());
    return ZB_OK;
}

size_t rmsnorm_dgamma_scratch_floats(int T, int H) { return (size_t)((T + DG_ROWS - 1) / DG_ROWS) * H; }

int32_t rmsnorm_dgamma(const bf16_t* x, const float* r, const bf16_t* dn, float* dgamma, float* scratch, int T,
                       int H, hipStream_t s) {
    if (H % 8 || T <= 0) return fail(ZB_EINVAL, "dgamma: hidden size must be a multiple of 8");
    const int nch = (T + DG_ROWS - 1) / DG_ROWS;
    hipLaunchKernelGGL(dgamma_partial_kernel, dim3((H + 511) / 512, nch), dim3(256), 0, s, x, r, dn, scratch, T, H);
    ZB_HIP(hipGetLastError());
    hipLaunchKernelGGL(dgamma_reduce_kernel, dim3((H + 63) / 64), dim3(256), 0, s, scratch, dgamma, nch, H);
    ZB_HIP(hipGetLastError());
    return ZB_OK;
}

int32_t fill_f32(float* p, size_t n, float v, hipStream_t s) {
    if (n == 0) return ZB_OK;
    size_t blocks = (n + 255) / 256;
    if (blocks > 8192) blocks = 8192;
    hipLaunchKernelGGL(fill_f32_kernel, dim3((unsigned)blocks), dim3(256), 0, s, p, n, v);
    ZB_HIP(hipGetLastError());
    return ZB_OK;
}

int32_t sgd_step_f32(float* w, const float* dw, size_t n, float lr, hipStream_t s) {
    if (n == 0) return ZB_OK;
    size_t blocks = std::min<size_t>((n + 255) / 256, 8192);
    hipLaunchKernelGGL(sgd_f32_kernel, dim3((unsigned)blocks), dim3(256), 0, s, w, dw, n, lr);
    ZB_HIP(hipGetLastError());
    return ZB_OK;
}

int32_t sgd_step_group_bf16(const SgdGroup& g, hipStream_t s) {
    if (g.n < 1 || g.n > SGD_GROUP_MAX) return fail(ZB_EINVAL, "sgd_step_group_bf16: bad segment count");
    size_t most = 0;
    for (int i = 0; i < g.n; ++i) {
        const SgdSeg& sg = g.seg[i];
        if ((reinterpret_cast<uintptr_t>(sg.w) & 7) || (reinterpret_cast<uintptr_t>(sg.dw) & 15))
            return fail(ZB_EINVAL, "sgd_step_group_bf16: weights need 8-byte and dW 16-byte alignment");
        most = std::max<size_t>(most, sg.n4);
    }
    if (most == 0) return ZB_OK;
    const size_t bx = std::min<size_t>((most + 255) / 256, 2048);
    hipLaunchKernelGGL(sgd_bf16_group_kernel, dim3((unsigned)bx, (unsigned)g.n), dim3(256), 0, s, g);
    ZB_HIP(hipGetLastError());
    return ZB_OK;
}

int32_t copy_bytes(void* dst, const void* src, size_t n, hipStream_t s) {
    if (n == 0 || dst == src) return ZB_OK;
    ZB_HIP(hipMemcpyAsync(dst, src, n, hipMemcpyDeviceToDevice, s));
    return ZB_OK;
}

int32_t stamp_now(uint64_t* dst, hipStream_t s) {
    hipLaunchKernelGGL(stamp_kernel, dim3(1), dim3(64), 0, s, dst);
    ZB_HIP(hipGetLastError());
    return ZB_OK;
}

uint64_t wall_clock_hz() {
    int dev = 0, khz = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 100000000ull;
    if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess || khz <= 0)
        return 100000000ull;
    return (uint64_t)khz * 1000ull;
}

int32_t wait_until(const uint64_t* t0, uint64_t delta_ticks, uint64_t* wait_end, hipStream_t s) {
    const uint64_t cap = wall_clock_hz() * 30ull;  // never spin longer than 30 s
    hipLaunchKernelGGL(wait_kernel, dim3(1), dim3(64), 0, s, t0, delta_ticks, cap, wait_end);
    ZB_HIP(hipGetLastError());
    return ZB_OK;
}

}  // namespace zb
