// Host-side launch interface between the C ABI (kda_api.hip) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

struct PrefillArgs {
    const void* q;
    const void* k;
    const void* v;
    const float* g;
    const void* beta;
    const float* S0;          // may be null
    const int32_t* cu;        // may be null
    int64_t T;                // tokens per row of the [B, T, ...] tensors
    int32_t H, N, dk, dv;
    bool in_f32, out_f32;
    float scale;
    void* o;
    float* ST;                // may be null
    float* ckpt;              // may be null: [N, H, ckpt_cap, dk, dv] states at interval ends
    int32_t ckpt_every;       // checkpoint interval in 32-token chunks (>= 1 when ckpt is set)
    int32_t ckpt_cap;         // checkpoints kept per (sequence, head)
    hipStream_t stream;
};

struct DecodeArgs {
    const void* q;
    const void* k;
    const void* v;
    const float* g;
    const void* beta;
    float* S;
    int32_t NH, dk, dv;
    bool in_f32, out_f32;
    float scale;
    void* o;
    hipStream_t stream;
};

hipError_t launch_chunk_fwd(const PrefillArgs& a);
hipError_t launch_decode_step(const DecodeArgs& a);

}  // namespace kda
