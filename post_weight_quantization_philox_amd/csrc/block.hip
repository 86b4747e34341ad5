// Kernels of a synthetic decoder block's forward pass, used by the staged
// schedule (the pages quantize a block in stages, each stage's calibration
// inputs computed from the block with the earlier stages already quantized:
// agihunt.info, optimizer paragraph). Everything here is bf16 in and out
// with fp32 arithmetic; the projections and attention products use the NT
// GEMM of gemm.hip.
#include "gsq_internal.hpp"

namespace gsq {

namespace {

constexpr int kT = 256;

__device__ __forceinline__ float ld_bf16(const uint16_t* p, int64_t i) { return bf16_lo(p[i]); }

__device__ __forceinline__ uint16_t to_bf16(float v) {
    return static_cast<uint16_t>(pack_bf16x2(v, 0.0f) & 0xFFFFu);
}

// Fixed-order sum of one value per thread over the workgroup.
__device__ __forceinline__ float block_sum(float v, float* red) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    const float s = ((red[0] + red[1]) + red[2]) + red[3];
    __syncthreads();
    return s;
}

__device__ __forceinline__ float block_max(float v, float* red) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, 64));
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    const float s = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    __syncthreads();
    return s;
}

// y = x / sqrt(mean(x^2) + eps) * gamma, one workgroup per row.
__global__ __launch_bounds__(kT) void rmsnorm_kernel(const uint16_t* __restrict__ x,
                                                     const float* __restrict__ gamma, int64_t cols,
                                                     float eps, uint16_t* __restrict__ y) {
    __shared__ float red[kT / 64];
    const int64_t r = blockIdx.x;
    const uint16_t* xr = x + r * cols;
    float ss = 0.0f;
    for (int64_t j = threadIdx.x; j < cols; j += kT) {
        const float v = ld_bf16(xr, j);
        ss = __builtin_fmaf(v, v, ss);
    }
    ss = block_sum(ss, red);
    const float inv = 1.0f / sqrtf(ss / static_cast<float>(cols) + eps);
    for (int64_t j = threadIdx.x; j < cols; j += kT)
        y[r * cols + j] = to_bf16(ld_bf16(xr, j) * inv * gamma[j]);
}

// Row i of P = softmax(scale * S) over columns 0..i (causal), zeros after.
__global__ __launch_bounds__(kT) void softmax_causal_kernel(const uint16_t* __restrict__ S,
                                                            int64_t n, float scale,
                                                            uint16_t* __restrict__ P) {
    __shared__ float red[kT / 64];
    const int64_t i = blockIdx.x;
    const uint16_t* sr = S + i * n;
    float mx = -INFINITY;
    for (int64_t j = threadIdx.x; j <= i; j += kT) mx = fmaxf(mx, ld_bf16(sr, j) * scale);
    mx = block_max(mx, red);
    float sum = 0.0f;
    for (int64_t j = threadIdx.x; j <= i; j += kT) sum += expf(ld_bf16(sr, j) * scale - mx);
    sum = block_sum(sum, red);
    const float inv = 1.0f / sum;
    for (int64_t j = threadIdx.x; j < n; j += kT)
        P[i * n + j] = (j <= i) ? to_bf16(expf(ld_bf16(sr, j) * scale - mx) * inv) : 0;
}

// act = silu(gate) * up, silu(z) = z / (1 + exp(-z)).
__global__ __launch_bounds__(kT) void silu_mul_kernel(const uint16_t* __restrict__ gate,
                                                      const uint16_t* __restrict__ up, int64_t n,
                                                      uint16_t* __restrict__ act) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * kT + threadIdx.x;
    if (i >= n) return;
    const float g = ld_bf16(gate, i);
    act[i] = to_bf16(g / (1.0f + expf(-g)) * ld_bf16(up, i));
}

// out = a + b (SUB: a - b), one fp32 operation rounded to bf16.
template <bool SUB>
__global__ __launch_bounds__(kT) void add_kernel(const uint16_t* __restrict__ a,
                                                 const uint16_t* __restrict__ b, int64_t n,
                                                 uint16_t* __restrict__ out) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * kT + threadIdx.x;
    if (i >= n) return;
    out[i] = to_bf16(SUB ? ld_bf16(a, i) - ld_bf16(b, i) : ld_bf16(a, i) + ld_bf16(b, i));
}

// Hard weights s * v(code) in bf16 from stored codes and fp16 scales.
__global__ __launch_bounds__(kT) void dequant_kernel(const uint8_t* __restrict__ codes,
                                                     const uint16_t* __restrict__ s16, int64_t mk,
                                                     int64_t cols, int grid,
                                                     uint16_t* __restrict__ W) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * kT + threadIdx.x;
    if (i >= mk) return;
    const int64_t r = i / cols, j = i - r * cols;
    const _Float16 h = __builtin_bit_cast(_Float16, s16[r * (cols / 128) + j / 128]);
    const int c = codes[i];
    const int v = (grid == GSQ_GRID_TERNARY) ? c - 1
                  : (grid == GSQ_GRID_INT2)  ? 2 * c - 3
                                             : 2 * c - 7;
    W[i] = to_bf16(static_cast<float>(h) * static_cast<float>(v));
}

inline unsigned nblk(int64_t n) { return static_cast<unsigned>((n + kT - 1) / kT); }

}  // namespace

hipError_t launch_rmsnorm(int64_t rows, int64_t cols, const uint16_t* x, const float* gamma,
                          float eps, uint16_t* y, hipStream_t st) {
    hipLaunchKernelGGL(rmsnorm_kernel, dim3(static_cast<unsigned>(rows)), dim3(kT), 0, st, x, gamma,
                       cols, eps, y);
    return hipGetLastError();
}

hipError_t launch_softmax_causal(int64_t n, const uint16_t* S, float scale, uint16_t* P,
                                 hipStream_t st) {
    hipLaunchKernelGGL(softmax_causal_kernel, dim3(static_cast<unsigned>(n)), dim3(kT), 0, st, S, n,
                       scale, P);
    return hipGetLastError();
}

hipError_t launch_silu_mul(int64_t n, const uint16_t* gate, const uint16_t* up, uint16_t* act,
                           hipStream_t st) {
    hipLaunchKernelGGL(silu_mul_kernel, dim3(nblk(n)), dim3(kT), 0, st, gate, up, n, act);
    return hipGetLastError();
}

hipError_t launch_add(int64_t n, const uint16_t* a, const uint16_t* b, uint16_t* out,
                      hipStream_t st) {
    hipLaunchKernelGGL(add_kernel<false>, dim3(nblk(n)), dim3(kT), 0, st, a, b, n, out);
    return hipGetLastError();
}

hipError_t launch_sub(int64_t n, const uint16_t* a, const uint16_t* b, uint16_t* out,
                      hipStream_t st) {
    hipLaunchKernelGGL(add_kernel<true>, dim3(nblk(n)), dim3(kT), 0, st, a, b, n, out);
    return hipGetLastError();
}

hipError_t launch_dequant(const LayerDesc& d, const uint8_t* codes, const uint16_t* s16,
                          uint16_t* W, hipStream_t st) {
    hipLaunchKernelGGL(dequant_kernel, dim3(nblk(static_cast<int64_t>(d.mk))), dim3(kT), 0, st, codes,
                       s16, static_cast<int64_t>(d.mk), static_cast<int64_t>(d.cols), d.grid, W);
    return hipGetLastError();
}

}  // namespace gsq
