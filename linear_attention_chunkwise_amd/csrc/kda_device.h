// Device-side helpers shared by the libkda kernels (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16;
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
// g_min of the bounded decay map, g = g_min Sigmoid(exp(A_h) z), and g_min in log2 units
constexpr float kGmin = -5.0f;
constexpr float kGminLog2e = -7.2134752044448170f;

// D = A * B + C on one 16x16x32 bf16 tile (v_mfma_f32_16x16x32_bf16, fp32 accumulation).
// With lane l, i16 = l % 16 and g4 = l / 16: the A operand of lane l holds row i16 and the B
// operand holds column i16, each for eight positions of the 32-long contraction selected by
// (g4, element index); A and B use the same selection, so any bijection of the contraction index
// onto (g4, element) gives the same product.  The result holds rows 4*g4 .. 4*g4+3 of column
// i16 in its four elements.
__device__ __forceinline__ f32x4 mma(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// The same tile shape on float16 operands (v_mfma_f32_16x16x32_f16), same lane layout.
__device__ __forceinline__ f32x4 mma_h(f16x8 a, f16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// Debug builds only (-DKDA_POISON_LDS): every kernel first fills its LDS with 0x7FC07FC0, a
// float32 NaN whose two 16-bit halves are bf16 NaNs, so a value read before any wave wrote it
// reaches the results as NaN.  The library build compiles both macros to nothing.
#ifdef KDA_POISON_LDS
__device__ __forceinline__ void poison_lds(void* p, size_t bytes) {
    uint32_t* w = static_cast<uint32_t*>(p);
    for (size_t i = threadIdx.x; i < bytes / 4; i += blockDim.x) w[i] = 0x7FC07FC0u;
}
#define KDA_POISON(p, bytes) ::kda::poison_lds((p), (bytes))
#define KDA_POISON_DONE() __syncthreads()
#else
#define KDA_POISON(p, bytes) ((void)0)
#define KDA_POISON_DONE() ((void)0)
#endif

__device__ __forceinline__ float bf2f(bf16 x) { return static_cast<float>(x); }
__device__ __forceinline__ bf16 f2bf(float x) { return static_cast<bf16>(x); }  // round to nearest even

// x = hi + lo with hi = bf16(x) and lo = bf16(x - hi): 16 significant bits in two bf16 halves.
__device__ __forceinline__ void split_bf16(float x, bf16& hi, bf16& lo) {
    hi = f2bf(x);
    lo = f2bf(x - bf2f(hi));
}

template <typename T>
__device__ __forceinline__ T ld(const void* p) { return *reinterpret_cast<const T*>(p); }
template <typename T>
__device__ __forceinline__ void st(void* p, T v) { *reinterpret_cast<T*>(p) = v; }

// Two 4-element bf16 vectors (8 bytes each) packed into one MFMA operand.
__device__ __forceinline__ bf16x8 cat44(bf16x4 a, bf16x4 b) {
    return bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

}  // namespace kda
