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

// The contraction sequence of one 16-column state slice for one 32-token chunk, as the prefill
// kernel's consumer waves issue it, with the elementwise work left out: operand rows read from LDS
// as 16-byte fragments (K~ 4 steps x 2 tiles, T_b, Q~ hi/lo, A_qk hi/lo, K_end hi/lo), 68
// v_mfma_f32_16x16x32_bf16 per wave per chunk (K~ S 8, T_b R 4, Q~ S 24, A_qk V~ 6, state update
// 24, two transposes), the accumulators chained as in the kernel and the state carried from chunk
// to chunk.  B operands stay in registers.  8 waves per workgroup, one workgroup per CU.
constexpr int kRB = 136, kTB = 40;   // the kernel's bf16 row strides ([token][dk], [*][token])
constexpr int kOffKt = 0, kOffQt = kOffKt + 32 * kRB, kOffTb = kOffQt + 2 * 32 * kRB;
constexpr int kOffAq = kOffTb + 32 * kTB, kOffKe = kOffAq + 2 * 32 * kTB, kLdsElems = kOffKe + 2 * 128 * kTB;
constexpr int kContractionMfmas = 68;

__global__ __launch_bounds__(512) void contraction_loop(float* __restrict__ out, int chunks) {
    __shared__ __attribute__((aligned(16))) __bf16 lds[kLdsElems];
    for (int i = threadIdx.x; i < kLdsElems; i += 512) lds[i] = (__bf16)(0.001f * (float)(i % 97) - 0.04f);
    __syncthreads();
    const int lane = threadIdx.x & 63, i16 = lane & 15, g4 = lane >> 4;
    int base = 0;   // made opaque every chunk below, so the reads stay inside the loop
    auto frag = [&](int off, int row, int stride, int col) -> bf16x8 {
        return *reinterpret_cast<const bf16x8*>(lds + base + off + row * stride + col + 8 * g4);
    };
    auto mma = [](bf16x8 a, bf16x8 b, f32x4 c) { return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0); };
    bf16x8 Bs[4], Br, Bv, Bq;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        Br[e] = (__bf16)(0.01f * (e + 1));
        Bv[e] = (__bf16)(0.02f * (e - 3));
        Bq[e] = (__bf16)(0.005f * (lane & 7));
#pragma unroll
        for (int k = 0; k < 4; ++k) Bs[k][e] = (__bf16)(0.001f * (k + e));
    }
    const f32x4 z{0.f, 0.f, 0.f, 0.f};
    f32x4 S[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) S[c] = f32x4{0.01f * c, 0.f, 0.f, 0.f};
    for (int it = 0; it < chunks; ++it) {
        base = 0;
        asm volatile("" : "+v"(base));
        f32x4 V[2], R[2], Vt[2], O[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) V[t] = mma(t ? Br : Bv, Bq, z);              // transposes
#pragma unroll
        for (int ta = 0; ta < 2; ++ta) {                                          // R = V - K~ S
            f32x4 acc = z;
#pragma unroll
            for (int k = 0; k < 4; ++k) acc = mma(frag(kOffKt, 16 * ta + i16, kRB, 32 * k), Bs[k], acc);
            R[ta] = V[ta] - acc;
        }
#pragma unroll
        for (int ta = 0; ta < 2; ++ta) {                                          // V~ = T_b R (split R)
            const bf16x8 tb = frag(kOffTb, 16 * ta + i16, kTB, 0);
            Vt[ta] = mma(tb, Br, mma(tb, Bv, R[ta]));
        }
#pragma unroll
        for (int ta = 0; ta < 2; ++ta) {                                          // O = Q~ S (split x split)
            f32x4 acc = z;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const bf16x8 qh = frag(kOffQt, 16 * ta + i16, kRB, 32 * k);
                const bf16x8 ql = frag(kOffQt + 32 * kRB, 16 * ta + i16, kRB, 32 * k);
                acc = mma(qh, Bs[k], acc);
                acc = mma(ql, Bs[k], acc);
                acc = mma(qh, Br, acc);
            }
            const bf16x8 ah = frag(kOffAq, 16 * ta + i16, kTB, 0);                // + A_qk V~ (split)
            const bf16x8 al = frag(kOffAq + 32 * kTB, 16 * ta + i16, kTB, 0);
            acc = mma(ah, Bv, acc);
            acc = mma(al, Bv, acc);
            O[ta] = mma(ah, Bq, acc) + Vt[ta];
        }
#pragma unroll
        for (int c = 0; c < 8; ++c) {                                             // S += K_end^T V~ (split x split)
            const bf16x8 kh = frag(kOffKe, 16 * c + i16, kTB, 0);
            const bf16x8 kl = frag(kOffKe + 128 * kTB, 16 * c + i16, kTB, 0);
            S[c] = mma(kh, Bv, mma(kl, Bv, mma(kh, Bq, S[c])));
        }
        S[0] += O[0] + O[1];
    }
    f32x4 t = z;
#pragma unroll
    for (int c = 0; c < 8; ++c) t += S[c];
    const float sum = t[0] + t[1] + t[2] + t[3];
    if (sum == -1.0f) out[blockIdx.x * blockDim.x + threadIdx.x] = sum;
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

// Flops one calib_contraction launch issues: blocks x 8 waves x chunks x 68 MFMAs x 16384.
double calib_contraction_flops(int blocks, int chunks) {
    return (double)blocks * 8.0 * chunks * kContractionMfmas * (2.0 * 16 * 16 * 32);
}

// blocks workgroups of 512 threads running `chunks` rounds of the contraction sequence; `out` as
// for calib_mfma (blocks * 512 floats, never written in practice).  Returns a hipError_t code.
int calib_contraction(float* out, int blocks, int chunks, hipStream_t stream) {
    if (!out || blocks < 1 || chunks < 1) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(contraction_loop, dim3(blocks), dim3(512), 0, stream, out, chunks);
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
