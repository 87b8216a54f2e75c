// Optional input-domain check (enabled by the environment variable KDA_CHECK_RANGE=1): the decay
// g must lie in [g_min, 0] with g_min = -5 (Kimi K3: Open Frontier Intelligence, §2.1.1, eq. (5)
// and the bound stated after it), which the prefill kernel relies on for the bf16 range of its
// 16-token rescale factors.  A debug aid: the check synchronises the stream to read its result.
#include <stdint.h>

#include <mutex>

#include "kda_launch.h"

namespace kda {

// One flag per device, cleared before each check.  Checks in one process take turns (the lock
// below), so concurrent checked calls from several host threads do not see each other's flag.
__device__ uint32_t g_range_violations;

__global__ __launch_bounds__(256) void range_kernel(const float* __restrict__ g, size_t n, float lo, float hi) {
    uint32_t bad = 0;
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += stride) {
        const float x = g[i];
        bad |= !(x >= lo && x <= hi);   // NaN fails too
    }
    if (bad) atomicOr(&g_range_violations, 1u);
}

hipError_t check_range(const float* g, size_t n, float lo, float hi, hipStream_t stream, bool& ok) {
    ok = true;
    if (n == 0) return hipSuccess;
    static std::mutex lock;
    const std::lock_guard<std::mutex> hold(lock);
    static const uint32_t zero = 0;
    hipError_t e = hipMemcpyToSymbolAsync(HIP_SYMBOL(g_range_violations), &zero, sizeof zero, 0,
                                          hipMemcpyHostToDevice, stream);
    if (e != hipSuccess) return e;
    const size_t want = (n + 255) / 256;
    hipLaunchKernelGGL(range_kernel, dim3((unsigned)(want < 2048 ? want : 2048)), dim3(256), 0, stream, g, n, lo, hi);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    uint32_t v = 0;
    e = hipMemcpyFromSymbolAsync(&v, HIP_SYMBOL(g_range_violations), sizeof v, 0, hipMemcpyDeviceToHost, stream);
    if (e != hipSuccess) return e;
    e = hipStreamSynchronize(stream);
    ok = v == 0;
    return e;
}

}  // namespace kda
