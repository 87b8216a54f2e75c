// C ABI of libkda (declared in include/kda.h): host-side argument checks and dispatch.
//
// Every check runs before anything is enqueued, so an error return leaves the stream untouched.
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>

#include "kda.h"
#include "kda_launch.h"

namespace {

// Segment summaries of kda_chunk_fwd_cp_noalloc: a fixed array in each device's copy of the code
// object, so that the call itself allocates nothing.  Host code never uses the name as an
// address (on the host it is only a stand-in): the device address comes from
// hipGetSymbolAddress, looked up once per device and kept in g_scratch_dev.
constexpr size_t kScratchBytes = KDA_NOALLOC_SCRATCH_BYTES;
__device__ __align__(256) unsigned char scratch[kScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_lock;
void* g_scratch_dev[kMaxDevices] = {};

thread_local char g_last_error[512] = "";

kda_status fail(kda_status s, const char* fmt, const char* what, long long x = 0) {
    snprintf(g_last_error, sizeof g_last_error, fmt, what, x);
    return s;
}

kda_status ok() {
    g_last_error[0] = '\0';
    return KDA_OK;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
    if (!a || !b || na == 0 || nb == 0) return false;
    const char* x = static_cast<const char*>(a);
    const char* y = static_cast<const char*>(b);
    return x < y + nb && y < x + na;
}

// A byte range of one argument.  A null pointer or an empty range takes part in no overlap.
struct Span {
    const void* p;
    size_t n;
    const char* name;
};

// Outputs may overlap no input and no other output: workgroups read inputs while others write
// outputs.  Read-only inputs may alias one another.
template <size_t NO, size_t NI>
kda_status check_disjoint(const Span (&outs)[NO], const Span (&ins)[NI]) {
    for (size_t i = 0; i < NO; ++i) {
        const Span* hit = nullptr;
        for (size_t j = 0; j < NI && !hit; ++j)
            if (overlaps(outs[i].p, outs[i].n, ins[j].p, ins[j].n)) hit = &ins[j];
        for (size_t j = i + 1; j < NO && !hit; ++j)
            if (overlaps(outs[i].p, outs[i].n, outs[j].p, outs[j].n)) hit = &outs[j];
        if (hit) {
            snprintf(g_last_error, sizeof g_last_error, "%s overlaps %s", outs[i].name, hit->name);
            return KDA_ERR_INVALID_ARGUMENT;
        }
    }
    return KDA_OK;
}

// Concurrent prefill workgroups on the current device: one per compute unit.
int device_slots() {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 256;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1) return 256;
    return cus;
}

// Bytes of `count` segment summaries per head ([dk][dv + dk] float32 each) and of their stop
// counts (one int32 per 64 transition columns), which follow them in a workspace.
size_t summary_bytes(int64_t count, int32_t H, int32_t dk, int32_t dv) {
    return (size_t)count * H * ((size_t)dk * (dv + dk) + dk / 64) * 4;
}

// Bytes of the plan in front of the summaries in an automatic split, 256-aligned.
size_t plan_bytes(int32_t N, int64_t Smax) {
    return ((size_t)kda::PlanLayout{N, (int32_t)Smax}.ints() * 4 + 255) / 256 * 256;
}

kda_status hip_status(hipError_t e) {
    if (e == hipSuccess) return ok();
    snprintf(g_last_error, sizeof g_last_error, "HIP error %d: %s", (int)e, hipGetErrorString(e));
    return KDA_ERR_HIP;
}

size_t dsize(kda_dtype d) { return d == KDA_F32 ? 4 : 2; }

kda_status check_dtype(kda_dtype d, const char* what) {
    if (d != KDA_BF16 && d != KDA_F32)
        return fail(KDA_ERR_INVALID_ARGUMENT, "%s: unknown dtype code %lld", what, (long long)d);
    return KDA_OK;
}

kda_status check_ptr(const void* p, size_t align, const char* what) {
    if (!p) return fail(KDA_ERR_INVALID_ARGUMENT, "%s is NULL%.0lld", what);
    if (!aligned(p, align))
        return fail(KDA_ERR_INVALID_ARGUMENT, "%s is not %lld-byte aligned", what, (long long)align);
    return KDA_OK;
}

// KDA_CHECK_RANGE=1: check g against [-5, 0] before launching (synchronises the stream)
kda_status check_g(const float* g, size_t n, hipStream_t stream) {
    const char* env = getenv("KDA_CHECK_RANGE");
    if (!env || env[0] != '1' || !g || n == 0) return KDA_OK;
    bool in_range = true;
    const hipError_t e = kda::check_range(g, n, -5.0f, 0.0f, stream, in_range);
    if (e != hipSuccess) {
        snprintf(g_last_error, sizeof g_last_error, "HIP error %d: %s", (int)e, hipGetErrorString(e));
        return KDA_ERR_HIP;
    }
    if (!in_range) return fail(KDA_ERR_RANGE, "%s: a value lies outside [-5, 0] or is NaN%.0lld", "g");
    return KDA_OK;
}

// KDA_CHECK_RANGE=1: check the packed-sequence offsets before launching (synchronises the stream)
kda_status check_cu(const int32_t* cu, int32_t N, int64_t T, hipStream_t stream) {
    const char* env = getenv("KDA_CHECK_RANGE");
    if (!env || env[0] != '1' || !cu) return KDA_OK;
    bool fine = true;
    const hipError_t e = kda::check_offsets(cu, N, T, stream, fine);
    if (e != hipSuccess) {
        snprintf(g_last_error, sizeof g_last_error, "HIP error %d: %s", (int)e, hipGetErrorString(e));
        return KDA_ERR_HIP;
    }
    if (!fine)
        return fail(KDA_ERR_INVALID_ARGUMENT, "%s: the offsets do not run from 0 to T without decreasing%.0lld",
                    "cu_seqlens");
    return KDA_OK;
}

#define KDA_TRY(expr)                      \
    do {                                   \
        kda_status _s = (expr);            \
        if (_s != KDA_OK) return _s;       \
    } while (0)

}  // namespace

extern "C" {

int32_t kda_version(void) { return (1 << 16) | 2; }

const char* kda_status_string(kda_status s) {
    switch (s) {
        case KDA_OK: return "KDA_OK";
        case KDA_ERR_INVALID_ARGUMENT: return "KDA_ERR_INVALID_ARGUMENT";
        case KDA_ERR_UNSUPPORTED: return "KDA_ERR_UNSUPPORTED";
        case KDA_ERR_RANGE: return "KDA_ERR_RANGE";
        case KDA_ERR_HIP: return "KDA_ERR_HIP";
    }
    return "KDA_ERR_UNKNOWN";
}

const char* kda_last_error(void) { return g_last_error; }

static kda_status chunk_fwd_impl(const void* q, const void* k, const void* v, const float* g,
                                 const void* z, const float* A_log, const void* beta, const float* S0, const int32_t* cu_seqlens,
                                 int32_t B, int64_t T, int32_t H, int32_t N, int32_t dk, int32_t dv,
                                 kda_dtype in_dtype, kda_dtype out_dtype, float scale, void* o,
                                 float* S_T, int32_t ckpt_interval, int32_t ckpt_capacity,
                                 float* ckpt, int32_t segments, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream) {
    KDA_TRY(check_dtype(in_dtype, "in_dtype"));
    KDA_TRY(check_dtype(out_dtype, "out_dtype"));
    if (B < 1) return fail(KDA_ERR_INVALID_ARGUMENT, "%s must be >= 1 (got %lld)", "B", B);
    if (H < 1) return fail(KDA_ERR_INVALID_ARGUMENT, "%s must be >= 1 (got %lld)", "H", H);
    if (T < 0) return fail(KDA_ERR_INVALID_ARGUMENT, "%s must be >= 0 (got %lld)", "T", T);
    if (dk < 1 || dv < 1) return fail(KDA_ERR_INVALID_ARGUMENT, "%s must be >= 1 (got %lld)", "dk/dv", dk < 1 ? dk : dv);
    if (cu_seqlens) {
        if (B != 1) return fail(KDA_ERR_INVALID_ARGUMENT, "%s: packed sequences need B == 1 (got %lld)", "cu_seqlens", B);
        if (N < 0) return fail(KDA_ERR_INVALID_ARGUMENT, "%s must be >= 0 (got %lld)", "N", N);
        if (!aligned(cu_seqlens, 4)) return fail(KDA_ERR_INVALID_ARGUMENT, "%s is not %lld-byte aligned", "cu_seqlens", 4);
    } else if (N != B) {
        return fail(KDA_ERR_INVALID_ARGUMENT, "%s must equal B without cu_seqlens (got %lld)", "N", N);
    }
    if (!(dk == 64 || dk == 128)) return fail(KDA_ERR_UNSUPPORTED, "%s = %lld is not supported (64 or 128)", "dk", dk);
    if (!(dv == 64 || dv == 128)) return fail(KDA_ERR_UNSUPPORTED, "%s = %lld is not supported (64 or 128)", "dv", dv);
    if ((int64_t)N * H > (int64_t)1 << 30) return fail(KDA_ERR_UNSUPPORTED, "%s = %lld too large", "N*H", (long long)N * H);
    // the kernel addresses one 32-token chunk of a head's rows with 32-bit byte offsets
    if ((int64_t)H * (dk > dv ? dk : dv) > (int64_t)1 << 22)
        return fail(KDA_ERR_UNSUPPORTED, "%s = %lld too large", "H*d", (long long)H * (dk > dv ? dk : dv));

    const int64_t tokens = (int64_t)B * T;
    const size_t es = dsize(in_dtype);
    const size_t nqk = (size_t)tokens * H * dk, nv = (size_t)tokens * H * dv;
    if (tokens > 0) {
        KDA_TRY(check_ptr(q, 16, "q"));
        KDA_TRY(check_ptr(k, 16, "k"));
        KDA_TRY(check_ptr(v, 16, "v"));
        if (z) {
            KDA_TRY(check_ptr(z, 16, "z"));
            KDA_TRY(check_ptr(A_log, 4, "A_log"));
        } else {
            KDA_TRY(check_ptr(g, 16, "g"));
        }
        KDA_TRY(check_ptr(beta, es, "beta"));
        KDA_TRY(check_ptr(o, 16, "o"));
    }
    if (cu_seqlens == nullptr && N == 0) return ok();
    const size_t nst = (size_t)N * H * dk * dv * 4;
    if (S0) KDA_TRY(check_ptr(S0, 16, "S0"));
    if (S_T) {
        KDA_TRY(check_ptr(S_T, 16, "S_T"));
        if (S_T != S0 && overlaps(S_T, nst, S0, nst))
            return fail(KDA_ERR_INVALID_ARGUMENT, "%s partially overlaps S0 (only exact aliasing is allowed)%.0lld", "S_T");
    }
    if (ckpt_capacity < 0)
        return fail(KDA_ERR_INVALID_ARGUMENT, "%s must be >= 0 (got %lld)", "ckpt_capacity", ckpt_capacity);
    const size_t nck = (size_t)N * H * (size_t)ckpt_capacity * dk * dv * 4;
    if (ckpt_capacity > 0) {
        if (ckpt_interval < 1 || ckpt_interval % 32 != 0)
            return fail(KDA_ERR_UNSUPPORTED, "%s = %lld: checkpoints sit on 32-token chunk ends (a positive multiple of 32)",
                        "ckpt_interval", ckpt_interval);
        KDA_TRY(check_ptr(ckpt, 16, "ckpt"));
    }
    int64_t seg_len = 0;
    size_t need = 0;
    // automatic split (segments == 0, kda_chunk_fwd with a workspace): planned on the device (a
    // decay probe, then one planning workgroup), fixed-length rows and packed sequences alike;
    // the host checks only that a split can pay (the workspace size is 0 otherwise)
    bool device_plan = false;
    kda::SplitLimits lim;
    int slots = 0;
    if (segments == 0) {
        segments = 1;
        if (workspace && workspace_bytes > 0 && ckpt_capacity == 0 && N > 0 && !(S_T && S_T == S0)) {
            slots = device_slots();
            const size_t want = kda_chunk_fwd_workspace_size(N, tokens, H, dk, dv, cu_seqlens ? 1 : 0);
            if (want > 0 && workspace_bytes >= want) {
                // the device planner (fixed rows too: its decay probe chooses the layout)
                lim = kda::split_limits(N, tokens, H, dv, slots);
                if (lim.Smax > 0 && kda::plan_packed(N, H, dv, slots)) {
                    device_plan = true;
                    segments = lim.Pmax;
                }
            }
        }
    }
    if (segments < 1) return fail(KDA_ERR_INVALID_ARGUMENT, "%s must be >= 1 (got %lld)", "segments", segments);
    if (segments > 1) {
        // one workgroup per (sequence, head, segment, 64-column slice): keep the grid and the
        // kernel's 32-bit unit index in range
        if ((int64_t)N * H * segments > (int64_t)1 << 28)
            return fail(KDA_ERR_UNSUPPORTED, "%s = %lld too large", "N*H*segments", (long long)N * H * segments);
        if (ckpt_capacity > 0)
            return fail(KDA_ERR_UNSUPPORTED, "%s: checkpoints are not emitted by segmented runs%.0lld", "segments");
        // segment length: the whole row split evenly, rounded up to whole 32-token chunks
        seg_len = ((T + segments - 1) / segments + 31) / 32 * 32;
        if (seg_len == 0) seg_len = 32;
        // the first segment reads S0 while the last one writes S_T, in the same launch
        if (S_T && S_T == S0)
            return fail(KDA_ERR_INVALID_ARGUMENT, "%s may not alias S0 in a segmented run%.0lld", "S_T");
        need = device_plan ? plan_bytes(N, lim.Smax) + summary_bytes(lim.Smax, H, dk, dv)
                           : kda_chunk_fwd_cp_workspace_size(N, H, dk, dv, segments);
        if (workspace_bytes < need)
            return fail(KDA_ERR_INVALID_ARGUMENT, "%s: %lld bytes given, the workspace size asks for more",
                        "workspace_bytes", (long long)workspace_bytes);
        KDA_TRY(check_ptr(workspace, 16, "workspace"));
    }
    {
        // S_T may be S0 itself (in place: each workgroup reads its S0 block before writing it)
        const Span outs[] = {{tokens > 0 ? o : nullptr, nv * dsize(out_dtype), "o"},
                             {S_T, nst, "S_T"},
                             {ckpt_capacity > 0 ? ckpt : nullptr, nck, "ckpt"},
                             {segments > 1 ? workspace : nullptr, need, "workspace"}};
        const Span ins[] = {{q, nqk * es, "q"},
                            {k, nqk * es, "k"},
                            {v, nv * es, "v"},
                            {z ? nullptr : g, nqk * 4, "g"},
                            {z, nqk * es, "z"},
                            {z ? A_log : nullptr, (size_t)H * 4, "A_log"},
                            {beta, (size_t)tokens * H * es, "beta"},
                            {cu_seqlens, cu_seqlens ? ((size_t)N + 1) * 4 : 0, "cu_seqlens"},
                            {S_T == S0 ? nullptr : S0, nst, "S0"}};
        KDA_TRY(check_disjoint(outs, ins));
    }
    if (N == 0) return ok();

    KDA_TRY(check_cu(cu_seqlens, N, T, stream));
    if (!z) KDA_TRY(check_g(g, (size_t)tokens * H * dk, stream));
    kda::PrefillArgs a{q, k, v, g, beta, S0, cu_seqlens, T, H, N, dk, dv,
                       in_dtype == KDA_F32, out_dtype == KDA_F32, scale, o, S_T,
                       ckpt_capacity > 0 ? ckpt : nullptr, ckpt_interval / 32, ckpt_capacity,
                       /*mode*/ 0, /*nseg*/ 1, /*seg_len*/ 0, /*ws*/ nullptr, stream};
    if (z) {
        a.g = nullptr;
        a.z = z;
        a.A_log = A_log;
    }
    if (segments <= 1) return hip_status(kda::launch_chunk_fwd(a));
    // segmented: every segment with its outputs and the summaries of all but the last, then the
    // later segments again over the chunks whose outputs depend on their entering state
    a.nseg = segments;
    a.seg_len = seg_len;
    a.ws = static_cast<float*>(workspace);
    int64_t nsum = (int64_t)N * (segments - 1);
    const kda::PlanLayout lay{N, (int32_t)lim.Smax};
    if (device_plan) {
        int32_t* plan = static_cast<int32_t*>(workspace);
        a.ws = reinterpret_cast<float*>(static_cast<char*>(workspace) + plan_bytes(N, lim.Smax));
        const hipError_t e = kda::launch_plan(a, plan, slots, lim);
        if (e != hipSuccess) return hip_status(e);
        a.plan = plan;
        a.plan_smax = (int32_t)lim.Smax;
        nsum = lim.Smax;
    }
    a.stops = reinterpret_cast<int32_t*>(a.ws + (size_t)nsum * H * dk * (dv + dk));
    a.mode = 1;
    a.plan_items = lay.max_items1();
    const hipError_t e = kda::launch_chunk_fwd(a);
    if (e != hipSuccess) return hip_status(e);
    a.mode = 2;
    a.plan_items = lay.max_items2();
    return hip_status(kda::launch_chunk_fwd(a));
}

kda_status kda_chunk_fwd(const void* q, const void* k, const void* v, const float* g,
                         const void* beta, const float* S0, const int32_t* cu_seqlens,
                         int32_t B, int64_t T, int32_t H, int32_t N, int32_t dk, int32_t dv,
                         kda_dtype in_dtype, kda_dtype out_dtype, float scale, void* o,
                         float* S_T, void* workspace, size_t workspace_bytes, hipStream_t stream) {
    return chunk_fwd_impl(q, k, v, g, nullptr, nullptr, beta, S0, cu_seqlens, B, T, H, N, dk, dv, in_dtype, out_dtype,
                          scale, o, S_T, 0, 0, nullptr, 0, workspace, workspace_bytes, stream);
}

size_t kda_chunk_fwd_workspace_size(int32_t n_seq, int64_t total_tokens, int32_t H, int32_t dk, int32_t dv,
                                    int32_t packed) {
    if (n_seq < 1 || total_tokens <= 0 || H < 1 || !(dk == 64 || dk == 128) || !(dv == 64 || dv == 128)) return 0;
    const int slots = device_slots();
    if (!packed && (total_tokens % n_seq || !kda::split_may_pay(n_seq, total_tokens / n_seq, H, dk, dv, slots)))
        return 0;
    const kda::SplitLimits lim = kda::split_limits(n_seq, total_tokens, H, dv, slots);
    if (lim.Smax <= 0 || !kda::plan_packed(n_seq, H, dv, slots)) return 0;
    return plan_bytes(n_seq, lim.Smax) + summary_bytes(lim.Smax, H, dk, dv);
}

kda_status kda_chunk_fwd_ckpt(const void* q, const void* k, const void* v, const float* g,
                              const void* beta, const float* S0, const int32_t* cu_seqlens,
                              int32_t B, int64_t T, int32_t H, int32_t N, int32_t dk, int32_t dv,
                              kda_dtype in_dtype, kda_dtype out_dtype, float scale, void* o,
                              float* S_T, int32_t ckpt_interval, int32_t ckpt_capacity, float* ckpt,
                              hipStream_t stream) {
    return chunk_fwd_impl(q, k, v, g, nullptr, nullptr, beta, S0, cu_seqlens, B, T, H, N, dk, dv, in_dtype, out_dtype,
                          scale, o, S_T, ckpt_interval, ckpt_capacity, ckpt, 1, nullptr, 0, stream);
}

kda_status kda_chunk_fwd_gate(const void* q, const void* k, const void* v, const void* z,
                              const float* A_log, const void* beta, const float* S0,
                              const int32_t* cu_seqlens, int32_t B, int64_t T, int32_t H, int32_t N,
                              int32_t dk, int32_t dv, kda_dtype in_dtype, kda_dtype out_dtype,
                              float scale, void* o, float* S_T, void* workspace,
                              size_t workspace_bytes, hipStream_t stream) {
    if (!z) return fail(KDA_ERR_INVALID_ARGUMENT, "%s is NULL%.0lld", "z");
    return chunk_fwd_impl(q, k, v, nullptr, z, A_log, beta, S0, cu_seqlens, B, T, H, N, dk, dv,
                          in_dtype, out_dtype, scale, o, S_T, 0, 0, nullptr, 0, workspace,
                          workspace_bytes, stream);
}

size_t kda_chunk_fwd_cp_workspace_size(int32_t N, int32_t H, int32_t dk, int32_t dv, int32_t segments) {
    if (N < 1 || H < 1 || dk < 1 || dv < 1 || segments <= 1) return 0;
    // saturate rather than wrap for sizes no device could hold
    size_t n = 4;
    const size_t per = (size_t)dk * ((size_t)dv + (size_t)dk) + (size_t)dk / 64;   // summary, stop counts
    const size_t factors[4] = {(size_t)N, (size_t)(segments - 1), (size_t)H, per};
    for (size_t f : factors)
        if (__builtin_mul_overflow(n, f, &n)) return SIZE_MAX;
    return n;
}

int32_t kda_chunk_fwd_cp_segments(int32_t N, int32_t H, int32_t dk, int32_t dv, int32_t slots) {
    if (N < 1 || H < 1 || dk < 1 || dv < 1 || slots < 1) return 1;
    // the value workgroups of pass 1 (every segment) in one round; its transition workgroups
    // stop early where the keys' channels decay
    const int64_t units = (int64_t)N * H * (dv / 64);
    const int64_t p = units > 0 ? slots / units : 0;
    return (int32_t)(p < 1 ? 1 : (p > 64 ? 64 : p));
}

kda_status kda_chunk_fwd_cp(const void* q, const void* k, const void* v, const float* g,
                            const void* beta, const float* S0, const int32_t* cu_seqlens, int32_t B,
                            int64_t T, int32_t H, int32_t N, int32_t dk, int32_t dv,
                            kda_dtype in_dtype, kda_dtype out_dtype, float scale, void* o,
                            float* S_T, int32_t segments, void* workspace, size_t workspace_bytes,
                            hipStream_t stream) {
    if (segments < 1) return fail(KDA_ERR_INVALID_ARGUMENT, "%s must be >= 1 (got %lld)", "segments", segments);
    return chunk_fwd_impl(q, k, v, g, nullptr, nullptr, beta, S0, cu_seqlens, B, T, H, N, dk, dv, in_dtype, out_dtype,
                          scale, o, S_T, 0, 0, nullptr, segments, workspace, workspace_bytes, stream);
}

// The scratch array's address on the current device (looked up on the first call there).
static kda_status scratch_on_current_device(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_status(e);
    if (dev < 0 || dev >= kMaxDevices)
        return fail(KDA_ERR_UNSUPPORTED, "%s = %lld: beyond the devices this library tracks", "device", dev);
    const std::lock_guard<std::mutex> hold(g_scratch_lock);
    if (!g_scratch_dev[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_status(e);
        if (!p) return fail(KDA_ERR_HIP, "%s: hipGetSymbolAddress gave no address%.0lld", "scratch");
        g_scratch_dev[dev] = p;
    }
    *out = g_scratch_dev[dev];
    return KDA_OK;
}

kda_status kda_chunk_fwd_cp_noalloc(const void* q, const void* k, const void* v, const float* g,
                                    const void* beta, const float* S0, const int32_t* cu_seqlens,
                                    int32_t B, int64_t T, int32_t H, int32_t N, int32_t dk,
                                    int32_t dv, kda_dtype in_dtype, kda_dtype out_dtype, float scale,
                                    void* o, float* S_T, int32_t segments, hipStream_t stream) {
    if (segments < 1) return fail(KDA_ERR_INVALID_ARGUMENT, "%s must be >= 1 (got %lld)", "segments", segments);
    void* ws = nullptr;
    if (segments > 1) {
        const size_t need = kda_chunk_fwd_cp_workspace_size(N, H, dk, dv, segments);
        if (need > kScratchBytes)
            return fail(KDA_ERR_UNSUPPORTED,
                        "%s: the summaries need %lld bytes, beyond the fixed 32 MiB of the no-allocation "
                        "variant (use kda_chunk_fwd_cp with a workspace, or fewer segments)",
                        "segments", need == SIZE_MAX ? -1LL : (long long)need);
        if (need > 0) KDA_TRY(scratch_on_current_device(&ws));
    }
    return chunk_fwd_impl(q, k, v, g, nullptr, nullptr, beta, S0, cu_seqlens, B, T, H, N, dk, dv,
                          in_dtype, out_dtype, scale, o, S_T, 0, 0, nullptr, segments, ws,
                          ws ? kScratchBytes : 0, stream);
}

static kda_status recurrent_step_impl(const void* q, const void* k, const void* v, const float* g,
                                      const void* z, const float* A_log, const void* beta, float* S,
                                      int32_t N, int32_t H, int32_t dk, int32_t dv,
                                      kda_dtype in_dtype, kda_dtype out_dtype, float scale,
                                      void* o, hipStream_t stream) {
    KDA_TRY(check_dtype(in_dtype, "in_dtype"));
    KDA_TRY(check_dtype(out_dtype, "out_dtype"));
    if (N < 0) return fail(KDA_ERR_INVALID_ARGUMENT, "%s must be >= 0 (got %lld)", "N", N);
    if (H < 1) return fail(KDA_ERR_INVALID_ARGUMENT, "%s must be >= 1 (got %lld)", "H", H);
    if (!(dk == 64 || dk == 128)) return fail(KDA_ERR_UNSUPPORTED, "%s = %lld is not supported (64 or 128)", "dk", dk);
    if (!(dv == 64 || dv == 128)) return fail(KDA_ERR_UNSUPPORTED, "%s = %lld is not supported (64 or 128)", "dv", dv);
    if ((int64_t)N * H > (int64_t)1 << 30) return fail(KDA_ERR_UNSUPPORTED, "%s = %lld too large", "N*H", (long long)N * H);
    if (N == 0) return ok();
    const size_t es = dsize(in_dtype);
    KDA_TRY(check_ptr(q, 16, "q"));
    KDA_TRY(check_ptr(k, 16, "k"));
    KDA_TRY(check_ptr(v, 16, "v"));
    if (z) {
        KDA_TRY(check_ptr(z, 16, "z"));
        KDA_TRY(check_ptr(A_log, 4, "A_log"));
    } else {
        KDA_TRY(check_ptr(g, 16, "g"));
    }
    KDA_TRY(check_ptr(beta, es, "beta"));
    KDA_TRY(check_ptr(S, 16, "S"));
    KDA_TRY(check_ptr(o, 16, "o"));
    const size_t nh = (size_t)N * H;
    {
        const Span outs[] = {{S, nh * dk * dv * 4, "S"}, {o, nh * dv * dsize(out_dtype), "o"}};
        const Span ins[] = {{q, nh * dk * es, "q"},
                            {k, nh * dk * es, "k"},
                            {v, nh * dv * es, "v"},
                            {z ? nullptr : g, nh * dk * 4, "g"},
                            {z, nh * dk * es, "z"},
                            {z ? A_log : nullptr, (size_t)H * 4, "A_log"},
                            {beta, nh * es, "beta"}};
        KDA_TRY(check_disjoint(outs, ins));
    }
    if (!z) KDA_TRY(check_g(g, nh * dk, stream));
    kda::DecodeArgs a{q, k, v, z ? nullptr : g, beta, S, (int32_t)nh, dk, dv,
                      in_dtype == KDA_F32, out_dtype == KDA_F32, scale, o, stream};
    a.H = H;
    a.z = z;
    a.A_log = z ? A_log : nullptr;
    return hip_status(kda::launch_decode_step(a));
}

kda_status kda_recurrent_step(const void* q, const void* k, const void* v, const float* g,
                              const void* beta, float* S, int32_t N, int32_t H, int32_t dk,
                              int32_t dv, kda_dtype in_dtype, kda_dtype out_dtype, float scale,
                              void* o, hipStream_t stream) {
    return recurrent_step_impl(q, k, v, g, nullptr, nullptr, beta, S, N, H, dk, dv, in_dtype,
                               out_dtype, scale, o, stream);
}

kda_status kda_recurrent_step_gate(const void* q, const void* k, const void* v, const void* z,
                                   const float* A_log, const void* beta, float* S, int32_t N,
                                   int32_t H, int32_t dk, int32_t dv, kda_dtype in_dtype,
                                   kda_dtype out_dtype, float scale, void* o, hipStream_t stream) {
    if (!z) return fail(KDA_ERR_INVALID_ARGUMENT, "%s is NULL%.0lld", "z");
    return recurrent_step_impl(q, k, v, nullptr, z, A_log, beta, S, N, H, dk, dv, in_dtype,
                               out_dtype, scale, o, stream);
}

kda_status kda_recurrent_multi(const void* q, const void* k, const void* v, const float* g,
                               const void* beta, float* S, const int32_t* n_commit, int32_t N,
                               int32_t K, int32_t H, int32_t dk, int32_t dv, kda_dtype in_dtype,
                               kda_dtype out_dtype, float scale, void* o, hipStream_t stream) {
    KDA_TRY(check_dtype(in_dtype, "in_dtype"));
    KDA_TRY(check_dtype(out_dtype, "out_dtype"));
    if (N < 0) return fail(KDA_ERR_INVALID_ARGUMENT, "%s must be >= 0 (got %lld)", "N", N);
    if (K < 0) return fail(KDA_ERR_INVALID_ARGUMENT, "%s must be >= 0 (got %lld)", "K", K);
    if (H < 1) return fail(KDA_ERR_INVALID_ARGUMENT, "%s must be >= 1 (got %lld)", "H", H);
    if (!(dk == 64 || dk == 128)) return fail(KDA_ERR_UNSUPPORTED, "%s = %lld is not supported (64 or 128)", "dk", dk);
    if (!(dv == 64 || dv == 128)) return fail(KDA_ERR_UNSUPPORTED, "%s = %lld is not supported (64 or 128)", "dv", dv);
    if ((int64_t)N * H > (int64_t)1 << 30) return fail(KDA_ERR_UNSUPPORTED, "%s = %lld too large", "N*H", (long long)N * H);
    if (N == 0 || K == 0) return ok();
    const size_t es = dsize(in_dtype);
    KDA_TRY(check_ptr(q, 16, "q"));
    KDA_TRY(check_ptr(k, 16, "k"));
    KDA_TRY(check_ptr(v, 16, "v"));
    KDA_TRY(check_ptr(g, 16, "g"));
    KDA_TRY(check_ptr(beta, es, "beta"));
    KDA_TRY(check_ptr(S, 16, "S"));
    if (n_commit) KDA_TRY(check_ptr(n_commit, 4, "n_commit"));
    const size_t nh = (size_t)N * H, nt = nh * (size_t)K;
    if (o) KDA_TRY(check_ptr(o, 16, "o"));
    {
        const Span outs[] = {{S, nh * dk * dv * 4, "S"}, {o, nt * dv * dsize(out_dtype), "o"}};
        const Span ins[] = {{q, nt * dk * es, "q"}, {k, nt * dk * es, "k"},    {v, nt * dv * es, "v"},
                            {g, nt * dk * 4, "g"},  {beta, nt * es, "beta"}, {n_commit, (size_t)N * 4, "n_commit"}};
        KDA_TRY(check_disjoint(outs, ins));
    }
    KDA_TRY(check_g(g, nt * dk, stream));
    kda::DecodeArgs a{q, k, v, g, beta, S, (int32_t)nh, dk, dv,
                      in_dtype == KDA_F32, out_dtype == KDA_F32, scale, o, stream};
    a.K = K;
    a.N = N;
    a.H = H;
    a.n_commit = n_commit;
    return hip_status(kda::launch_decode_step(a));
}

kda_status kda_recurrent_multi_fused(const void* q, const void* k, const void* v, const void* z,
                                     const float* A_log, const void* beta_logit, const void* G,
                                     const float* norm_weight, float eps, const float* conv_weight,
                                     void* conv_state, int32_t conv_width, float* S,
                                     const int32_t* n_commit, int32_t N, int32_t K, int32_t H,
                                     int32_t dk, int32_t dv, kda_dtype in_dtype,
                                     kda_dtype out_dtype, float scale, void* y, hipStream_t stream) {
    KDA_TRY(check_dtype(in_dtype, "in_dtype"));
    KDA_TRY(check_dtype(out_dtype, "out_dtype"));
    if (N < 0) return fail(KDA_ERR_INVALID_ARGUMENT, "%s must be >= 0 (got %lld)", "N", N);
    if (K < 0) return fail(KDA_ERR_INVALID_ARGUMENT, "%s must be >= 0 (got %lld)", "K", K);
    if (H < 1) return fail(KDA_ERR_INVALID_ARGUMENT, "%s must be >= 1 (got %lld)", "H", H);
    if (!(eps >= 0.f)) return fail(KDA_ERR_INVALID_ARGUMENT, "%s must be >= 0%.0lld", "eps");
    if (!(dk == 64 || dk == 128)) return fail(KDA_ERR_UNSUPPORTED, "%s = %lld is not supported (64 or 128)", "dk", dk);
    if (!(dv == 64 || dv == 128)) return fail(KDA_ERR_UNSUPPORTED, "%s = %lld is not supported (64 or 128)", "dv", dv);
    if ((int64_t)N * H > (int64_t)1 << 30) return fail(KDA_ERR_UNSUPPORTED, "%s = %lld too large", "N*H", (long long)N * H);
    if (conv_weight && (conv_width < 1 || conv_width > 4))
        return fail(KDA_ERR_UNSUPPORTED, "%s = %lld: the short convolution is 1 to 4 taps wide", "conv_width", conv_width);
    if (N == 0 || K == 0) return ok();
    const size_t es = dsize(in_dtype);
    KDA_TRY(check_ptr(q, 16, "q"));
    KDA_TRY(check_ptr(k, 16, "k"));
    KDA_TRY(check_ptr(v, 16, "v"));
    KDA_TRY(check_ptr(z, 16, "z"));
    KDA_TRY(check_ptr(A_log, 4, "A_log"));
    KDA_TRY(check_ptr(beta_logit, es, "beta_logit"));
    KDA_TRY(check_ptr(S, 16, "S"));
    if (n_commit) KDA_TRY(check_ptr(n_commit, 4, "n_commit"));
    if (norm_weight) KDA_TRY(check_ptr(norm_weight, 16, "norm_weight"));
    const size_t nh = (size_t)N * H, nt = nh * (size_t)K;
    if (y) {
        KDA_TRY(check_ptr(y, 16, "y"));
        KDA_TRY(check_ptr(G, es, "G"));
    }
    const size_t nch = (size_t)(2 * dk + dv);
    size_t ncw = 0, ncs = 0;
    if (conv_weight) {
        KDA_TRY(check_ptr(conv_weight, 4, "conv_weight"));
        ncw = (size_t)H * nch * conv_width * 4;
        if (conv_width > 1) {
            KDA_TRY(check_ptr(conv_state, 16, "conv_state"));
            ncs = nh * nch * (conv_width - 1) * es;
        }
    }
    {
        const Span outs[] = {{S, nh * dk * dv * 4, "S"}, {y, nt * dv * dsize(out_dtype), "y"},
                             {ncs ? conv_state : nullptr, ncs, "conv_state"}};
        const Span ins[] = {{q, nt * dk * es, "q"},
                            {k, nt * dk * es, "k"},
                            {v, nt * dv * es, "v"},
                            {z, nt * dk * es, "z"},
                            {A_log, (size_t)H * 4, "A_log"},
                            {beta_logit, nt * es, "beta_logit"},
                            {y ? G : nullptr, nt * dv * es, "G"},
                            {norm_weight, (size_t)dv * 4, "norm_weight"},
                            {n_commit, (size_t)N * 4, "n_commit"},
                            {conv_weight, ncw, "conv_weight"}};
        KDA_TRY(check_disjoint(outs, ins));
    }
    kda::DecodeArgs a{q, k, v, nullptr, beta_logit, S, (int32_t)nh, dk, dv,
                      in_dtype == KDA_F32, out_dtype == KDA_F32, scale, y, stream};
    a.K = K;
    a.N = N;
    a.H = H;
    a.n_commit = n_commit;
    a.z = z;
    a.A_log = A_log;
    a.fused = true;
    a.G = G;
    a.norm_w = norm_weight;
    a.eps = eps;
    a.conv_w = conv_weight;
    a.conv_state = conv_state;
    a.conv_width = conv_weight ? conv_width : 1;
    return hip_status(kda::launch_decode_step(a));
}

}  // extern "C"
