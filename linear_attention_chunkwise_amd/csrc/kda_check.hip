// Optional input-domain checks (enabled by the environment variable KDA_CHECK_RANGE=1): the decay
// g must lie in [g_min, 0] with g_min = -5 (Kimi K3: Open Frontier Intelligence, §2.1.1, eq. (5)
// and the bound stated after it), which the prefill kernel relies on for the bf16 range of its
// 16-token rescale factors; packed-sequence offsets must run from 0 to T without decreasing.  A
// debug aid: each check synchronises the stream to read its result.
#include <stdint.h>

#include <mutex>

#include "kda_launch.h"

namespace kda {

namespace {

// One flag per device, cleared before each check.  Checks in one process take turns (the lock
// below), so concurrent checked calls from several host threads do not see each other's flag.
__device__ uint32_t g_violations;
std::mutex g_check_lock;

__global__ __launch_bounds__(256) void range_kernel(const float* __restrict__ g, size_t n, float lo, float hi) {
    uint32_t bad = 0;
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += stride) {
        const float x = g[i];
        bad |= !(x >= lo && x <= hi);   // NaN fails too
    }
    if (bad) atomicOr(&g_violations, 1u);
}

// cu[0] = 0, cu[i] >= cu[i-1], cu[n-1] = T over the n = N + 1 entries
__global__ __launch_bounds__(256) void offsets_kernel(const int32_t* __restrict__ cu, int64_t n, int64_t T) {
    uint32_t bad = 0;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += stride) {
        const int64_t c = cu[i];
        bad |= i == 0 ? c != 0 : c < cu[i - 1];
        bad |= i == n - 1 && c != T;
    }
    if (bad) atomicOr(&g_violations, 1u);
}

// Clears the flag, enqueues `launch` on the stream, reads the flag back and waits for it.
template <typename Launch>
hipError_t flag_check(hipStream_t stream, bool& ok, Launch launch) {
    ok = true;
    const std::lock_guard<std::mutex> hold(g_check_lock);
    static const uint32_t zero = 0;
    hipError_t e = hipMemcpyToSymbolAsync(HIP_SYMBOL(g_violations), &zero, sizeof zero, 0,
                                          hipMemcpyHostToDevice, stream);
    if (e != hipSuccess) return e;
    launch();
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    uint32_t v = 0;
    e = hipMemcpyFromSymbolAsync(&v, HIP_SYMBOL(g_violations), sizeof v, 0, hipMemcpyDeviceToHost, stream);
    if (e != hipSuccess) return e;
    e = hipStreamSynchronize(stream);
    ok = v == 0;
    return e;
}

unsigned grid_for(int64_t n) {
    const int64_t want = (n + 255) / 256;
    return (unsigned)(want < 2048 ? want : 2048);
}

}  // namespace

hipError_t check_range(const float* g, size_t n, float lo, float hi, hipStream_t stream, bool& ok) {
    ok = true;
    if (n == 0) return hipSuccess;
    return flag_check(stream, ok, [&] {
        hipLaunchKernelGGL(range_kernel, dim3(grid_for((int64_t)n)), dim3(256), 0, stream, g, n, lo, hi);
    });
}

hipError_t check_offsets(const int32_t* cu, int32_t N, int64_t T, hipStream_t stream, bool& ok) {
    ok = true;
    const int64_t n = (int64_t)N + 1;
    return flag_check(stream, ok, [&] {
        hipLaunchKernelGGL(offsets_kernel, dim3(grid_for(n)), dim3(256), 0, stream, cu, n, T);
    });
}

}  // namespace kda
