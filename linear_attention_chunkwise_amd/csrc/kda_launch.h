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
    // Segmented (context-parallel) runs over nseg time segments of seg_len tokens per sequence:
    //   mode 0: plain prefill (nseg, seg_len, ws unused);
    //   mode 1: segment summaries: for segments j < nseg - 1 the state after the segment,
    //           entered with S0 (j = 0) or 0, and the segment's transition (extra dk columns
    //           entered with the identity, value 0) -> ws;
    //   mode 2: outputs: each segment rebuilds its entering state from the summaries of the
    //           segments before it, then runs as mode 0 (the last one writes S_T).
    int32_t mode;
    int32_t nseg;
    int64_t seg_len;          // multiple of 32
    float* ws;                // [N, nseg - 1, H, dk, dv + dk] float32 (modes 1, 2)
    hipStream_t stream;
    // decay map in the kernel (g unused): g = -5 Sigmoid(exp(A_log[h]) z), z [.., H, dk] stored
    // like q
    const void* z = nullptr;
    const float* A_log = nullptr;
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
    // several tokens per (sequence, head) when K > 0: inputs [N, K, H, d], o [N, K, H, dv] or
    // null, the state written after n_commit[n] tokens (null: all K)
    int32_t K = 0, N = 0, H = 0;
    const int32_t* n_commit = nullptr;
    // decay map in the kernel (g unused), as in PrefillArgs; H must be set
    const void* z = nullptr;
    const float* A_log = nullptr;
    // fused prologue/epilogue (K > 0, z set): q, k L2-normalised, beta holds logits, outputs
    // Sigmoid(G) * RMSNorm(o~) with weight norm_w (null: ones) and eps
    bool fused = false;
    const void* G = nullptr;
    const float* norm_w = nullptr;
    float eps = 0.f;
    // eq. (2)'s short convolution before Swish (fused only): taps [H, 2 dk + dv, conv_width]
    // float32, window [N, H, 2 dk + dv, conv_width - 1] in the input dtype, updated at the commit
    const float* conv_w = nullptr;
    void* conv_state = nullptr;
    int32_t conv_width = 1;
};

hipError_t launch_chunk_fwd(const PrefillArgs& a);
// ok = every g[i], i < n, lies in [lo, hi] (NaN does not); synchronises `stream`
hipError_t check_range(const float* g, size_t n, float lo, float hi, hipStream_t stream, bool& ok);
// ok = cu[0] == 0, cu non-decreasing, cu[N] == T (the N + 1 packed-sequence offsets); synchronises
hipError_t check_offsets(const int32_t* cu, int32_t N, int64_t T, hipStream_t stream, bool& ok);
hipError_t launch_decode_step(const DecodeArgs& a);

}  // namespace kda
