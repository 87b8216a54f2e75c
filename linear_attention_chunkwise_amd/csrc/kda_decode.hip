// KDA decode step: one token per (sequence, head), state advanced in place.
//
// Kimi K3: Open Frontier Intelligence, §2.1.1 eq. (1) with a single token, as used at decode
// time (§5.4.2: the recurrent state is updated in place at every step, and at large batch the
// state traffic is the cost):
//     S' = Diag(exp(g)) S;  u = beta (v - S'^T k);  S <- S' + k u^T;  o = S^T (scale q)
//        = scale (S'^T q + (q . k) u).
//
// Bound: HBM.  Per (sequence, head) the algorithmic traffic is the state read once and written
// once (2 * dk * dv * 4 bytes) plus q, k, v, g, beta and o; the arithmetic is ~7 dk dv fp32 ops.
// The state, touched once per launch, is read and written with nontemporal loads and stores:
// measured 11 % faster than plain accesses at 1024 sequences x 32 heads (each hint about half).
//
// The decay is either given (g) or computed here from the logits z and the per-head log-scales by
// the bounded map of §2.1.1, eq. (5), g = g_min Sigmoid(exp(A_h) z) with g_min = -5.
//
// Mapping: one 256-thread workgroup per (sequence, head).  Thread t owns four adjacent value
// columns (one float4 per state row) and a contiguous group of dk / (1024 / dv) state rows, so
// every state row is read and written by full 16-byte lanes, 512 contiguous bytes per row at
// dv = 128.  The two column reductions over dk (S'^T k and S'^T q) and the scalar q . k are
// finished across the row groups through LDS in a fixed order (deterministic).
#include "kda_device.h"
#include "kda_launch.h"

namespace kda {

// Per-channel decay exp(g) of element idx: g as given, or (GATE) the bounded map of the logit,
// g = g_min Sigmoid(exp(A_h) z), with ea = exp(A_h).
template <bool IN_F32, bool GATE>
__device__ __forceinline__ float decay_at(const float* __restrict__ g, const void* __restrict__ z,
                                          float ea, size_t idx) {
    if constexpr (GATE) {
        float zv;
        if constexpr (IN_F32) zv = reinterpret_cast<const float*>(z)[idx];
        else zv = bf2f(reinterpret_cast<const bf16*>(z)[idx]);
        return __expf(kGmin * __builtin_amdgcn_rcpf(1.f + __expf(-ea * zv)));
    } else {
        return __expf(g[idx]);
    }
}

template <int DK, int DV, bool IN_F32, bool OUT_F32, bool GATE>
__global__ __launch_bounds__(256) void decode_kernel(const void* __restrict__ qp,
                                                     const void* __restrict__ kp,
                                                     const void* __restrict__ vp,
                                                     const float* __restrict__ g,
                                                     const void* __restrict__ zp,
                                                     const float* __restrict__ A_log, int32_t H,
                                                     const void* __restrict__ betap,
                                                     float* __restrict__ S, int32_t NH,
                                                     float scale, void* __restrict__ op) {
    constexpr int CG = DV / 4;          // column groups (float4 each)
    constexpr int NRG = 256 / CG;       // row groups
    constexpr int RPG = DK / NRG;       // state rows per thread
    static_assert(RPG >= 1 && DK % NRG == 0, "decode tiling");
    __shared__ f32x4 red_y[NRG][CG];
    __shared__ f32x4 red_z[NRG][CG];
    __shared__ float red_qk[NRG];

    const int unit = blockIdx.x;        // sequence * H + head
    if (unit >= NH) return;
    const int t = threadIdx.x;
    const int cg = t % CG, rg = t / CG;
    const int r0 = rg * RPG;

    float* Su = S + (size_t)unit * DK * DV;
    f32x4 s[RPG];
#pragma unroll
    for (int i = 0; i < RPG; ++i) s[i] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(Su + (size_t)(r0 + i) * DV + 4 * cg));

    auto in_at = [&](const void* p, size_t idx) -> float {
        if constexpr (IN_F32) return reinterpret_cast<const float*>(p)[idx];
        else return bf2f(reinterpret_cast<const bf16*>(p)[idx]);
    };
    const size_t kb = (size_t)unit * DK;
    // decay map (GATE): once per channel through LDS rather than in each of the CG threads that
    // hold the channel's row (the state loads above are already in flight)
    __shared__ float dec[GATE ? DK : 1];
    KDA_POISON(red_y, sizeof red_y);
    KDA_POISON(red_z, sizeof red_z);
    KDA_POISON(red_qk, sizeof red_qk);
    KDA_POISON(dec, sizeof dec);
    KDA_POISON_DONE();
    if constexpr (GATE) {
        if (t < DK) dec[t] = decay_at<IN_F32, true>(g, zp, __expf(A_log[unit % H]), kb + t);
        __syncthreads();
    }
    f32x4 y = zero4(), z = zero4();
    float qk = 0.f;
#pragma unroll
    for (int i = 0; i < RPG; ++i) {
        const float a = GATE ? dec[r0 + i] : __expf(g[kb + r0 + i]);
        const float kv = in_at(kp, kb + r0 + i);
        const float qv = in_at(qp, kb + r0 + i);
        s[i] *= a;
        y += kv * s[i];
        z += qv * s[i];
        qk += qv * kv;
    }
    red_y[rg][cg] = y;
    red_z[rg][cg] = z;
    if (cg == 0) red_qk[rg] = qk;  // every column group holds the same partial dot product
    __syncthreads();
    f32x4 yt = zero4(), zt = zero4();
    float qkt = 0.f;
#pragma unroll
    for (int j = 0; j < NRG; ++j) {
        yt += red_y[j][cg];
        zt += red_z[j][cg];
        qkt += red_qk[j];
    }
    const float b = in_at(betap, (size_t)unit);
    const size_t vb = (size_t)unit * DV + 4 * cg;
    f32x4 u;
#pragma unroll
    for (int c = 0; c < 4; ++c) u[c] = b * (in_at(vp, vb + c) - yt[c]);
#pragma unroll
    for (int i = 0; i < RPG; ++i) {
        const float kv = in_at(kp, kb + r0 + i);
        __builtin_nontemporal_store(s[i] + kv * u, reinterpret_cast<f32x4*>(Su + (size_t)(r0 + i) * DV + 4 * cg));
    }
    if (rg == 0) {
        const f32x4 o = scale * (zt + qkt * u);
        if constexpr (OUT_F32) {
            st<f32x4>(reinterpret_cast<float*>(op) + vb, o);
        } else {
            bf16x4 ob{f2bf(o[0]), f2bf(o[1]), f2bf(o[2]), f2bf(o[3])};
            st<bf16x4>(reinterpret_cast<bf16*>(op) + vb, ob);
        }
    }
}

// Several tokens per (sequence, head) with the state read once (speculative verification and
// replay of accepted tokens, §5.4.2): the state stays in registers across the K tokens; it is
// written back after the first `commit` tokens (commit = 0: outputs only, state untouched).
// Tokens are laid out [N, K, H, d]; the reductions use two LDS buffers by token parity, one
// workgroup barrier per token.  The per-channel decay of token tok + 1 is computed once per
// channel into LDS while token tok is processed (the barrier of token tok publishes it), instead
// of in each of the CG threads holding the channel's row: 822 -> 765 us for 4 tokens at
// 1024 x 32 heads.
template <int DK, int DV, bool IN_F32, bool OUT_F32, bool GATE>
__global__ __launch_bounds__(256) void decode_multi_kernel(const void* __restrict__ qp,
                                                           const void* __restrict__ kp,
                                                           const void* __restrict__ vp,
                                                           const float* __restrict__ g,
                                                           const void* __restrict__ zp,
                                                           const float* __restrict__ A_log,
                                                           const void* __restrict__ betap,
                                                           float* __restrict__ S,
                                                           const int32_t* __restrict__ n_commit,
                                                           int32_t N, int32_t H, int32_t K,
                                                           float scale, void* __restrict__ op) {
    constexpr int CG = DV / 4;
    constexpr int NRG = 256 / CG;
    constexpr int RPG = DK / NRG;
    static_assert(RPG >= 1 && DK % NRG == 0, "decode tiling");
    __shared__ f32x4 red_y[2][NRG][CG];
    __shared__ f32x4 red_z[2][NRG][CG];
    __shared__ float red_qk[2][NRG];
    __shared__ float dec[2][DK];

    const int unit = blockIdx.x;        // sequence * H + head
    if (unit >= N * H) return;
    KDA_POISON(red_y, sizeof red_y);
    KDA_POISON(red_z, sizeof red_z);
    KDA_POISON(red_qk, sizeof red_qk);
    KDA_POISON(dec, sizeof dec);
    KDA_POISON_DONE();
    const int n = unit / H, h = unit % H;
    const int t = threadIdx.x;
    const int cg = t % CG, rg = t / CG;
    const int r0 = rg * RPG;
    int commit = n_commit ? n_commit[n] : K;
    commit = commit < 0 ? 0 : (commit > K ? K : commit);
    const float ea = GATE ? __expf(A_log[h]) : 0.f;

    float* Su = S + (size_t)unit * DK * DV;
    f32x4 s[RPG];
#pragma unroll
    for (int i = 0; i < RPG; ++i) s[i] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(Su + (size_t)(r0 + i) * DV + 4 * cg));

    auto in_at = [&](const void* p, size_t idx) -> float {
        if constexpr (IN_F32) return reinterpret_cast<const float*>(p)[idx];
        else return bf2f(reinterpret_cast<const bf16*>(p)[idx]);
    };
    // the buffer a token writes was last read before the previous token's barrier
    auto decay_into = [&](int tok, int buf) {
        if (t < DK) dec[buf][t] = decay_at<IN_F32, GATE>(g, zp, ea, (((size_t)n * K + tok) * H + h) * DK + t);
    };
    decay_into(0, 0);
    __syncthreads();
    for (int tok = 0; tok < K; ++tok) {
        const int pb = tok & 1;
        const size_t row = ((size_t)n * K + tok) * H + h;   // token row of [N, K, H, *]
        const size_t kb = row * DK;
        if (tok + 1 < K) decay_into(tok + 1, pb ^ 1);
        f32x4 y = zero4(), z = zero4();
        float qk = 0.f;
        float kv[RPG];
#pragma unroll
        for (int i = 0; i < RPG; ++i) {
            const float a = dec[pb][r0 + i];
            kv[i] = in_at(kp, kb + r0 + i);
            const float qv = in_at(qp, kb + r0 + i);
            s[i] *= a;
            y += kv[i] * s[i];
            z += qv * s[i];
            qk += qv * kv[i];
        }
        red_y[pb][rg][cg] = y;
        red_z[pb][rg][cg] = z;
        if (cg == 0) red_qk[pb][rg] = qk;
        __syncthreads();   // the other parity's buffers were last read before this barrier
        f32x4 yt = zero4(), zt = zero4();
        float qkt = 0.f;
#pragma unroll
        for (int j = 0; j < NRG; ++j) {
            yt += red_y[pb][j][cg];
            zt += red_z[pb][j][cg];
            qkt += red_qk[pb][j];
        }
        const float b = in_at(betap, row);
        const size_t vb = row * DV + 4 * cg;
        f32x4 u;
#pragma unroll
        for (int c = 0; c < 4; ++c) u[c] = b * (in_at(vp, vb + c) - yt[c]);
#pragma unroll
        for (int i = 0; i < RPG; ++i) s[i] += kv[i] * u;
        if (tok + 1 == commit) {
#pragma unroll
            for (int i = 0; i < RPG; ++i) __builtin_nontemporal_store(s[i], reinterpret_cast<f32x4*>(Su + (size_t)(r0 + i) * DV + 4 * cg));
        }
        if (op && rg == 0) {
            const f32x4 o = scale * (zt + qkt * u);
            if constexpr (OUT_F32) {
                st<f32x4>(reinterpret_cast<float*>(op) + vb, o);
            } else {
                bf16x4 ob{f2bf(o[0]), f2bf(o[1]), f2bf(o[2]), f2bf(o[3])};
                st<bf16x4>(reinterpret_cast<bf16*>(op) + vb, ob);
            }
        }
    }
}

// The multi-token step fused with the weight-free steps around it (§2.1.1): before the recurrence,
// eq. (2)'s L2Norm of q and k (x / max(||x||, 1e-12)), beta = Sigmoid of its logit and the bounded
// decay map of eq. (5); after it, eq. (6) without W_o: y = Sigmoid(G) * RMSNorm(o~) per head, with
// RMSNorm(o~) = o~ / sqrt(mean(o~^2) + eps) * w.  The normalisations need two more dk
// reductions per token (q . q, k . k, finished with the others) and one dv reduction (o~ . o~,
// inside each row group's lanes).  Same mapping and commit rule as decode_multi_kernel.  The
// decay map runs once per (token, channel) into LDS instead of in every thread that holds the
// channel's row, and k is read again for the state update rather than held across the barrier:
// with those, three waves per SIMD fit (1194 -> 882 us for 4 tokens at 1024 x 32 heads).
template <int DK, int DV, bool IN_F32, bool OUT_F32>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3))) void decode_fused_kernel(const void* __restrict__ qp,
                                                           const void* __restrict__ kp,
                                                           const void* __restrict__ vp,
                                                           const void* __restrict__ zp,
                                                           const float* __restrict__ A_log,
                                                           const void* __restrict__ bp,
                                                           const void* __restrict__ Gp,
                                                           const float* __restrict__ norm_w, float eps,
                                                           float* __restrict__ S,
                                                           const int32_t* __restrict__ n_commit,
                                                           int32_t N, int32_t H, int32_t K,
                                                           float scale, void* __restrict__ op) {
    constexpr int CG = DV / 4;
    constexpr int NRG = 256 / CG;
    constexpr int RPG = DK / NRG;
    static_assert(RPG >= 1 && DK % NRG == 0 && 64 % CG == 0, "decode tiling");
    __shared__ f32x4 red_y[2][NRG][CG];
    __shared__ f32x4 red_z[2][NRG][CG];
    __shared__ f32x4 red_s[2][NRG];   // q . k, q . q, k . k (and one spare) per row group
    __shared__ float dec[2][DK];      // per-channel decay exp(g) of a token, by token parity

    const int unit = blockIdx.x;        // sequence * H + head
    if (unit >= N * H) return;
    KDA_POISON(red_y, sizeof red_y);
    KDA_POISON(red_z, sizeof red_z);
    KDA_POISON(red_s, sizeof red_s);
    KDA_POISON(dec, sizeof dec);
    KDA_POISON_DONE();
    const int n = unit / H, h = unit % H;
    const int t = threadIdx.x;
    const int cg = t % CG, rg = t / CG;
    const int r0 = rg * RPG;
    int commit = n_commit ? n_commit[n] : K;
    commit = commit < 0 ? 0 : (commit > K ? K : commit);
    const float ea = __expf(A_log[h]);
    f32x4 w = f32x4{1.f, 1.f, 1.f, 1.f};
    if (norm_w) w = ld<f32x4>(norm_w + 4 * cg);

    float* Su = S + (size_t)unit * DK * DV;
    f32x4 s[RPG];
#pragma unroll
    for (int i = 0; i < RPG; ++i) s[i] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(Su + (size_t)(r0 + i) * DV + 4 * cg));

    auto in_at = [&](const void* p, size_t idx) -> float {
        if constexpr (IN_F32) return reinterpret_cast<const float*>(p)[idx];
        else return bf2f(reinterpret_cast<const bf16*>(p)[idx]);
    };
    auto sigm = [](float x) { return __builtin_amdgcn_rcpf(1.f + __expf(-x)); };
    // the decay map once per (token, channel), a token ahead: written before the barrier that
    // precedes its use; the buffer it overwrites was last read before the previous barrier
    auto decay_into = [&](int tok, int buf) {
        if (t < DK) dec[buf][t] = decay_at<IN_F32, true>(nullptr, zp, ea, (((size_t)n * K + tok) * H + h) * DK + t);
    };
    decay_into(0, 0);
    __syncthreads();
    for (int tok = 0; tok < K; ++tok) {
        const int pb = tok & 1;
        const size_t row = ((size_t)n * K + tok) * H + h;   // token row of [N, K, H, *]
        const size_t kb = row * DK;
        if (tok + 1 < K) decay_into(tok + 1, pb ^ 1);
        f32x4 y = zero4(), z = zero4();
        float qk = 0.f, qq = 0.f, kk = 0.f;
#pragma unroll
        for (int i = 0; i < RPG; ++i) {
            const float a = dec[pb][r0 + i];
            const float kvi = in_at(kp, kb + r0 + i);
            const float qv = in_at(qp, kb + r0 + i);
            s[i] *= a;
            y += kvi * s[i];
            z += qv * s[i];
            qk += qv * kvi;
            qq += qv * qv;
            kk += kvi * kvi;
        }
        red_y[pb][rg][cg] = y;
        red_z[pb][rg][cg] = z;
        if (cg == 0) red_s[pb][rg] = f32x4{qk, qq, kk, 0.f};
        __syncthreads();   // the other parity's buffers were last read before this barrier
        f32x4 yt = zero4(), zt = zero4(), st4 = zero4();
#pragma unroll
        for (int j = 0; j < NRG; ++j) {
            yt += red_y[pb][j][cg];
            zt += red_z[pb][j][cg];
            st4 += red_s[pb][j];
        }
        // L2Norm of q and k as scale factors on the sums (and on k in the state update)
        const float rq = 1.f / fmaxf(sqrtf(st4[1]), 1e-12f);
        const float rk = 1.f / fmaxf(sqrtf(st4[2]), 1e-12f);
        const float b = sigm(in_at(bp, row));
        const size_t vb = row * DV + 4 * cg;
        f32x4 u;
#pragma unroll
        for (int c = 0; c < 4; ++c) u[c] = b * (in_at(vp, vb + c) - yt[c] * rk);
#pragma unroll
        for (int i = 0; i < RPG; ++i) s[i] += (in_at(kp, kb + r0 + i) * rk) * u;   // k re-read (cached)
        if (tok + 1 == commit) {
#pragma unroll
            for (int i = 0; i < RPG; ++i) __builtin_nontemporal_store(s[i], reinterpret_cast<f32x4*>(Su + (size_t)(r0 + i) * DV + 4 * cg));
        }
        if (op) {
            // o~ for this thread's 4 columns, then RMSNorm over dv across the CG lanes of the row
            // group (one wave holds whole row groups) and the gate
            const f32x4 o = scale * (zt * rq + (st4[0] * rq * rk) * u);
            float ss = o[0] * o[0] + o[1] * o[1] + o[2] * o[2] + o[3] * o[3];
#pragma unroll
            for (int m = 1; m < CG; m *= 2) ss += __shfl_xor(ss, m, 64);
            const float inv = rsqrtf(ss / DV + eps);
            if (rg == 0) {
                f32x4 yo;
#pragma unroll
                for (int c = 0; c < 4; ++c) yo[c] = sigm(in_at(Gp, vb + c)) * (o[c] * inv * w[c]);
                if constexpr (OUT_F32) {
                    st<f32x4>(reinterpret_cast<float*>(op) + vb, yo);
                } else {
                    bf16x4 ob{f2bf(yo[0]), f2bf(yo[1]), f2bf(yo[2]), f2bf(yo[3])};
                    st<bf16x4>(reinterpret_cast<bf16*>(op) + vb, ob);
                }
            }
        }
    }
}

template <int DK, int DV, bool IN_F32, bool OUT_F32>
static hipError_t launch_fused(const DecodeArgs& a) {
    const int64_t units = (int64_t)a.N * a.H;
    if (units == 0 || a.K == 0) return hipSuccess;
    hipLaunchKernelGGL((decode_fused_kernel<DK, DV, IN_F32, OUT_F32>), dim3((unsigned)units), dim3(256), 0,
                       a.stream, a.q, a.k, a.v, a.z, a.A_log, a.beta, a.G, a.norm_w, a.eps, a.S,
                       a.n_commit, a.N, a.H, a.K, a.scale, a.o);
    return hipGetLastError();
}

template <int DK, int DV, bool IN_F32, bool OUT_F32, bool GATE>
static hipError_t launch_decode(const DecodeArgs& a) {
    if (a.NH == 0) return hipSuccess;
    hipLaunchKernelGGL((decode_kernel<DK, DV, IN_F32, OUT_F32, GATE>), dim3(a.NH), dim3(256), 0,
                       a.stream, a.q, a.k, a.v, a.g, a.z, a.A_log, a.H, a.beta, a.S, a.NH, a.scale,
                       a.o);
    return hipGetLastError();
}

template <int DK, int DV, bool IN_F32, bool OUT_F32, bool GATE>
static hipError_t launch_multi(const DecodeArgs& a) {
    const int64_t units = (int64_t)a.N * a.H;
    if (units == 0 || a.K == 0) return hipSuccess;
    hipLaunchKernelGGL((decode_multi_kernel<DK, DV, IN_F32, OUT_F32, GATE>), dim3((unsigned)units),
                       dim3(256), 0, a.stream, a.q, a.k, a.v, a.g, a.z, a.A_log, a.beta, a.S,
                       a.n_commit, a.N, a.H, a.K, a.scale, a.o);
    return hipGetLastError();
}

template <int DK, int DV, bool GATE>
static hipError_t dispatch_io(const DecodeArgs& a) {
    if (a.K > 0) {
        if (a.in_f32)
            return a.out_f32 ? launch_multi<DK, DV, true, true, GATE>(a) : launch_multi<DK, DV, true, false, GATE>(a);
        return a.out_f32 ? launch_multi<DK, DV, false, true, GATE>(a) : launch_multi<DK, DV, false, false, GATE>(a);
    }
    if (a.in_f32)
        return a.out_f32 ? launch_decode<DK, DV, true, true, GATE>(a) : launch_decode<DK, DV, true, false, GATE>(a);
    return a.out_f32 ? launch_decode<DK, DV, false, true, GATE>(a) : launch_decode<DK, DV, false, false, GATE>(a);
}

template <int DK, int DV>
static hipError_t dispatch_gate(const DecodeArgs& a) {
    if (a.fused) {
        if (a.in_f32) return a.out_f32 ? launch_fused<DK, DV, true, true>(a) : launch_fused<DK, DV, true, false>(a);
        return a.out_f32 ? launch_fused<DK, DV, false, true>(a) : launch_fused<DK, DV, false, false>(a);
    }
    return a.z ? dispatch_io<DK, DV, true>(a) : dispatch_io<DK, DV, false>(a);
}

hipError_t launch_decode_step(const DecodeArgs& a) {
    if (a.dk == 128 && a.dv == 128) return dispatch_gate<128, 128>(a);
    if (a.dk == 128 && a.dv == 64) return dispatch_gate<128, 64>(a);
    if (a.dk == 64 && a.dv == 128) return dispatch_gate<64, 128>(a);
    if (a.dk == 64 && a.dv == 64) return dispatch_gate<64, 64>(a);
    return hipErrorInvalidValue;
}

}  // namespace kda
