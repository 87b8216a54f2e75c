// Calibration kernels for the roofline figures bench.py reports (measurement only; not part of
// libkda): the issue rate of the bf16 MFMA instruction the prefill kernel uses, and a plain
// device copy, both measured on the machine the benchmark runs on.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

namespace {

constexpr int kChains = 8;   // independent accumulators per wave: enough to keep the pipe full

// Every wave runs kChains independent chains of v_mfma_f32_16x16x32_bf16 for `iters` rounds.
// The operands are nonzero and fixed, the results are summed and stored only if they equal a
// value they cannot reach, so nothing is optimised away and nothing is written.
__global__ __launch_bounds__(256) void mfma_loop(float* __restrict__ out, int iters) {
    bf16x8 a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        a[e] = (__bf16)(1.0f + 0.001f * (threadIdx.x & 7));
        b[e] = (__bf16)(0.5f - 0.001f * e);
    }
    // distinct starting values keep the eight accumulators in eight register quads
    const float l = (float)(threadIdx.x & 3);
    f32x4 c0{l, 0.f, 0.f, 0.f}, c1{l + 1.f, 0.f, 0.f, 0.f}, c2{l + 2.f, 0.f, 0.f, 0.f},
        c3{l + 3.f, 0.f, 0.f, 0.f}, c4{l + 4.f, 0.f, 0.f, 0.f}, c5{l + 5.f, 0.f, 0.f, 0.f},
        c6{l + 6.f, 0.f, 0.f, 0.f}, c7{l + 7.f, 0.f, 0.f, 0.f};
    for (int i = 0; i < iters; ++i) {
        c0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c1, 0, 0, 0);
        c2 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c2, 0, 0, 0);
        c3 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c3, 0, 0, 0);
        c4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c4, 0, 0, 0);
        c5 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c5, 0, 0, 0);
        c6 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c6, 0, 0, 0);
        c7 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c7, 0, 0, 0);
    }
    const f32x4 t = ((c0 + c1) + (c2 + c3)) + ((c4 + c5) + (c6 + c7));
    const float s = t[0] + t[1] + t[2] + t[3];
    if (s == -1.0f) out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

__global__ __launch_bounds__(256) void copy16(const f32x4* __restrict__ x, f32x4* __restrict__ y, size_t n) {
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += stride) y[i] = x[i];
}

}  // namespace

extern "C" {

// Flops one calib_mfma launch performs: blocks x 4 waves x iters x chains x (2 x 16 x 16 x 32).
double calib_mfma_flops(int blocks, int iters) {
    return (double)blocks * 4.0 * iters * kChains * (2.0 * 16 * 16 * 32);
}

// blocks workgroups of 256 threads; `out` is a device float buffer of blocks * 256 (never
// written in practice).  Returns a hipError_t code.
int calib_mfma(float* out, int blocks, int iters, hipStream_t stream) {
    if (!out || blocks < 1 || iters < 1) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(mfma_loop, dim3(blocks), dim3(256), 0, stream, out, iters);
    return (int)hipGetLastError();
}

// Copies n16 16-byte elements from x to y (device pointers, 16-byte aligned, not overlapping)
// with a grid-stride loop over `blocks` workgroups of 256 threads.  Returns a hipError_t code.
int calib_copy(const void* x, void* y, size_t n16, int blocks, hipStream_t stream) {
    if (!x || !y || blocks < 1) return (int)hipErrorInvalidValue;
    if ((reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(y)) & 15) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(copy16, dim3(blocks), dim3(256), 0, stream, static_cast<const f32x4*>(x),
                       static_cast<f32x4*>(y), n16);
    return (int)hipGetLastError();
}

}  // extern "C"
