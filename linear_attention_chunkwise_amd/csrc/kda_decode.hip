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

// The multi-token step fused with the steps the model applies around it (§2.1.1): before the
// recurrence, optionally eq. (2)'s short convolution and Swish on q, k, v (CONV), then its L2Norm
// of q and k (x / max(||x||, 1e-12)), beta = Sigmoid of its logit and the bounded decay map of
// eq. (5); after it, eq. (6) without W_o: y = Sigmoid(G) * RMSNorm(o~) per head, with
// RMSNorm(o~) = o~ / sqrt(mean(o~^2) + eps) * w.  Same mapping and commit rule as
// decode_multi_kernel.
//
// None of the steps before the recurrence depend on the state, so they run for a group of KB
// tokens at once, ahead of the serial token loop, and leave LDS holding the recurrence's inputs
// ready to use (normalised q and k, v, exp(g), beta, q . k, Sigmoid(G)).  For the first group
// the input loads are issued before the state's, and the preparation runs while the state is
// still arriving from HBM (vector loads complete in issue order, so loads issued after the
// state's would wait for it).  The token loop is then the plain multi-token loop plus the
// output norm.
//
// CONV: thread t owns channels t and t + 256 (when < 2 dk + dv; q's channels, then k's, then
// v's).  A channel's taps and window sit in its own row of cwt, used by its owner only, kept
// right-aligned (zeros on the left when W < 4): y = w3 x_t + w2 x_{t-1} + w1 x_{t-2} + w0 x_{t-3},
// cwt[c] = {w0, w1, w2, w3, x_{t-3}, x_{t-2}, x_{t-1}, unused}.  The window is written back to
// conv_state after the committed prefix, together with S.
template <int DK, int DV, bool IN_F32, bool OUT_F32, bool CONV>
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
                                                           float scale, void* __restrict__ op,
                                                           const float* __restrict__ conv_w,
                                                           void* __restrict__ conv_state, int32_t W) {
    constexpr int CG = DV / 4;
    constexpr int NRG = 256 / CG;
    constexpr int RPG = DK / NRG;
    constexpr int NCH = 2 * DK + DV;   // q, k, v channels
    constexpr int KB = 4;              // tokens prepared per group: one wave each for the norms
    constexpr int ZPT = KB * DK / 256; // decay logits per thread in a group
    constexpr int GPT = KB * DV / 256; // gate inputs per thread in a group
    static_assert(RPG >= 4 && RPG % 4 == 0 && DK % NRG == 0 && 64 % CG == 0, "decode tiling");
    static_assert(NCH <= 512 && ZPT >= 1 && GPT >= 1, "two channels per thread at most");
    __shared__ f32x4 red_y[2][NRG][CG];
    __shared__ f32x4 red_z[2][NRG][CG];
    // Rows are padded to the 512 channels two per thread can name, and tb to one beta slot per
    // thread, so that the preparation stores unconditionally: a loaded value used only under a
    // per-thread condition gets sunk past the state's loads, and waiting for it would then wait
    // for the state as well.
    constexpr int XS = 512;
    __shared__ __align__(16) float xin[KB][XS];    // q^, k^ (normalised) and v of the group
    __shared__ __align__(16) float dec[KB][DK];    // exp(g)
    __shared__ __align__(16) float sgate[KB][DV];  // Sigmoid(G)
    __shared__ float bsig[256];                    // beta of the group's tokens (first KB)
    __shared__ float tqk[KB];                      // q^ . k^
    __shared__ __align__(16) float cwt[CONV ? XS : 1][8];
    // the committed windows of the unit, staged in conv_state's own layout [NCH][W - 1] so that
    // they leave as whole 16-byte stores instead of scattered 2- or 4-byte ones
    __shared__ __align__(16) char cst[CONV ? NCH * 3 * (IN_F32 ? 4 : 2) : 16];

    const int unit = blockIdx.x;        // sequence * H + head
    if (unit >= N * H) return;
    KDA_POISON(red_y, sizeof red_y);
    KDA_POISON(red_z, sizeof red_z);
    KDA_POISON(xin, sizeof xin);
    KDA_POISON(dec, sizeof dec);
    KDA_POISON(sgate, sizeof sgate);
    KDA_POISON(bsig, sizeof bsig);
    KDA_POISON(tqk, sizeof tqk);
    KDA_POISON(cwt, sizeof cwt);
    KDA_POISON(cst, sizeof cst);
    KDA_POISON_DONE();
    const int n = unit / H, h = unit % H;
    const int t = threadIdx.x;
    const int cg = t % CG, rg = t / CG;
    const int r0 = rg * RPG;
    const int wv = t / 64, lane = t % 64;
    int commit = n_commit ? n_commit[n] : K;
    commit = commit < 0 ? 0 : (commit > K ? K : commit);
    const float ea = __expf(A_log[h]);

    // Addressing: every tensor is reached from a workgroup-uniform base (the unit's token 0,
    // head h) plus a 32-bit per-thread offset, so that addresses live in scalar registers and
    // the loads take the base + 32-bit offset form; the vector registers go to the state.
    constexpr int ES = IN_F32 ? 4 : 2;
    const size_t tok0 = (size_t)n * K * H + h;            // row of (n, token 0, h) in [N, K, H]
    const uint32_t HDK = (uint32_t)H * DK, HDV = (uint32_t)H * DV;
    const char* const qb = static_cast<const char*>(qp) + tok0 * DK * ES;
    const char* const kbp = static_cast<const char*>(kp) + tok0 * DK * ES;
    const char* const vbp = static_cast<const char*>(vp) + tok0 * DV * ES;
    const char* const zb = static_cast<const char*>(zp) + tok0 * DK * ES;
    const char* const bb = static_cast<const char*>(bp) + tok0 * ES;
    // without outputs G may be absent: z stands in (read, never used)
    const char* const gb = op ? static_cast<const char*>(Gp) + tok0 * DV * ES : zb;
    // element i past a uniform base; the byte offset is formed in 32 bits (the host keeps a
    // unit's K tokens under 2^30 elements)
    auto ldx = [&](const char* base, uint32_t i) -> float {
        const char* p = base + i * (uint32_t)ES;
        if constexpr (IN_F32) return *reinterpret_cast<const float*>(p);
        else return bf2f(*reinterpret_cast<const bf16*>(p));
    };
    auto sigm = [](float x) { return __builtin_amdgcn_rcpf(1.f + __expf(-x)); };
    // channel c of q | k | v: its base (uniform across a wave, as the three ranges are whole
    // waves: dk and dv are multiples of 64), its offset within a token and the token stride
    auto chan = [&](int c, const char*& src, uint32_t& off, uint32_t& stride) {
        const int part = __builtin_amdgcn_readfirstlane(c < DK ? 0 : (c < 2 * DK ? 1 : 2));
        src = part == 0 ? qb : (part == 1 ? kbp : vbp);
        stride = part < 2 ? HDK : HDV;
        off = (uint32_t)(c - part * DK);
    };

    // a group's inputs, loaded to registers.  Every load is unconditional, at an index clamped
    // into range (values past the group or the channels are never used): a load under a
    // per-thread condition is waited for where the branches join, one at a time.
    float xr[2][KB], zr[ZPT], gr[GPT], br = 0.f;
    auto load_group = [&](int t0, int kb) {
        const int last = t0 + kb - 1;
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const int c = t + 256 * e;
            const char* src;
            uint32_t off, stride;
            chan(c < NCH ? c : NCH - 1, src, off, stride);
#pragma unroll
            for (int j = 0; j < KB; ++j) xr[e][j] = ldx(src, (uint32_t)(t0 + j < last ? t0 + j : last) * stride + off);
        }
#pragma unroll
        for (int i = 0; i < ZPT; ++i) {
            const int idx = t + 256 * i, j = idx / DK, c = idx % DK;
            zr[i] = ldx(zb, (uint32_t)(t0 + j < last ? t0 + j : last) * HDK + c);
        }
#pragma unroll
        for (int i = 0; i < GPT; ++i) {
            const int idx = t + 256 * i, j = idx / DV, c = idx % DV;
            gr[i] = ldx(gb, op ? (uint32_t)(t0 + j < last ? t0 + j : last) * HDV + c : 0u);
        }
        br = ldx(bb, (uint32_t)(t0 + t < last ? t0 + t : last) * H);
    };
    // the unit's conv window rows: [N, H, NCH, W - 1]
    char* const csb = CONV && W > 1 ? static_cast<char*>(conv_state) + ((size_t)n * H + h) * NCH * (W - 1) * ES : nullptr;
    // everything before the recurrence for the group's tokens, into LDS (rows past the group
    // and channels past NCH receive values that are never read)
    auto prep_group = [&](int t0, int kb) {
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const int c = t + 256 * e;
            if constexpr (CONV) {
                const f32x4 tp = *reinterpret_cast<const f32x4*>(&cwt[c][0]);
                f32x4 wn = *reinterpret_cast<const f32x4*>(&cwt[c][4]);
#pragma unroll
                for (int j = 0; j < KB; ++j) {
                    const float x = xr[e][j];
                    const float y = tp[3] * x + tp[2] * wn[2] + tp[1] * wn[1] + tp[0] * wn[0];
                    xin[j][c] = y * sigm(y);   // Swish
                    const f32x4 rolled = f32x4{wn[1], wn[2], x, 0.f};
                    wn = j < kb ? rolled : wn;
                    if (c < NCH && t0 + j + 1 == commit) {
#pragma unroll
                        for (int m = 0; m < 3; ++m) {
                            if (m >= 4 - W) {
                                char* const o = cst + ((uint32_t)c * (W - 1) + (m - (4 - W))) * (uint32_t)ES;
                                if constexpr (IN_F32) *reinterpret_cast<float*>(o) = wn[m];
                                else *reinterpret_cast<bf16*>(o) = f2bf(wn[m]);
                            }
                        }
                    }
                }
                *reinterpret_cast<f32x4*>(&cwt[c][4]) = wn;
            } else {
#pragma unroll
                for (int j = 0; j < KB; ++j) xin[j][c] = xr[e][j];
            }
        }
#pragma unroll
        for (int i = 0; i < ZPT; ++i) {
            const int idx = t + 256 * i, j = idx / DK, c = idx % DK;
            dec[j][c] = __expf(kGmin * sigm(ea * zr[i]));
        }
#pragma unroll
        for (int i = 0; i < GPT; ++i) {
            const int idx = t + 256 * i, j = idx / DV, c = idx % DV;
            sgate[j][c] = sigm(gr[i]);
        }
        bsig[t] = sigm(br);
        __syncthreads();
        if constexpr (CONV) {
            // the group holds the commit (block-uniform): the staged windows go out whole
            if (W > 1 && t0 < commit && commit <= t0 + kb) {
                const uint32_t bytes = (uint32_t)NCH * (W - 1) * ES;
                for (uint32_t i = 16 * t; i + 16 <= bytes; i += 16 * 256)
                    *reinterpret_cast<uint4*>(csb + i) = *reinterpret_cast<const uint4*>(cst + i);
                for (uint32_t i = bytes / 16 * 16 + ES * t; i < bytes; i += ES * 256) {
                    if constexpr (IN_F32) *reinterpret_cast<float*>(csb + i) = *reinterpret_cast<const float*>(cst + i);
                    else *reinterpret_cast<bf16*>(csb + i) = *reinterpret_cast<const bf16*>(cst + i);
                }
            }
        }
        // L2Norm of q and k: wave wv normalises token wv of the group in place
        if (wv < kb) {
            float qq = 0.f, kk = 0.f, qk = 0.f;
#pragma unroll
            for (int c = lane; c < DK; c += 64) {
                const float qv = xin[wv][c], kv = xin[wv][DK + c];
                qq += qv * qv;
                kk += kv * kv;
                qk += qv * kv;
            }
#pragma unroll
            for (int m = 32; m >= 1; m /= 2) {
                qq += __shfl_xor(qq, m, 64);
                kk += __shfl_xor(kk, m, 64);
                qk += __shfl_xor(qk, m, 64);
            }
            const float rq = 1.f / fmaxf(sqrtf(qq), 1e-12f);
            const float rk = 1.f / fmaxf(sqrtf(kk), 1e-12f);
#pragma unroll
            for (int c = lane; c < DK; c += 64) {
                xin[wv][c] *= rq;
                xin[wv][DK + c] *= rk;
            }
            if (lane == 0) tqk[wv] = qk * rq * rk;
        }
        __syncthreads();
    };

    // CONV: taps and entering window to registers (stored to cwt only after the state's loads
    // are issued, so that nothing waits for them before); unconditional loads at clamped
    // indices, as in load_group; with W = 1 there is no window (conv_state may be absent) and a
    // tap stands in (read, never used)
    f32x4 tp0[2], wn0[2];
    if constexpr (CONV) {
        const float* const cwb = conv_w + (size_t)h * NCH * W;
        const char* const wsb = W > 1 ? csb : reinterpret_cast<const char*>(cwb);
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const uint32_t c = t + 256 * e < NCH ? t + 256 * e : NCH - 1;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int m = j - (4 - W);
                const float x = *reinterpret_cast<const float*>(reinterpret_cast<const char*>(cwb) + (c * W + (m > 0 ? m : 0)) * 4u);
                tp0[e][j] = m >= 0 ? x : 0.f;
            }
#pragma unroll
            for (int j = 0; j < 3; ++j) {
                const int m = j - (4 - W);
                const float x = ldx(wsb, W > 1 ? c * (W - 1) + (m > 0 ? m : 0) : 0u);
                wn0[e][j] = m >= 0 ? x : 0.f;
            }
            wn0[e][3] = 0.f;
        }
    }
    load_group(0, K < KB ? K : KB);
    // the state, after the first group's inputs (see above)
    float* const Su = S + (size_t)unit * DK * DV;
    const uint32_t so0 = (uint32_t)r0 * DV + 4 * cg;
    f32x4 s[RPG];
#pragma unroll
    for (int i = 0; i < RPG; ++i) s[i] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(Su + so0 + i * DV));
    if constexpr (CONV) {
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            *reinterpret_cast<f32x4*>(&cwt[t + 256 * e][0]) = tp0[e];
            *reinterpret_cast<f32x4*>(&cwt[t + 256 * e][4]) = wn0[e];
        }
    }

    char* const yb = op ? static_cast<char*>(op) + tok0 * DV * (OUT_F32 ? 4 : 2) : nullptr;
    // the first group is prepared outside the loop: its waits then count only the loads issued
    // before the state's, where inside the loop they would be merged with the later groups'
    prep_group(0, K < KB ? K : KB);
    for (int t0 = 0;;) {
        const int kb = K - t0 < KB ? K - t0 : KB;
        for (int j = 0; j < kb; ++j) {
            const int tok = t0 + j;
            const int pb = tok & 1;
            f32x4 y = zero4(), z = zero4();
#pragma unroll
            for (int i4 = 0; i4 < RPG; i4 += 4) {
                const f32x4 a = *reinterpret_cast<const f32x4*>(&dec[j][r0 + i4]);
                const f32x4 kv = *reinterpret_cast<const f32x4*>(&xin[j][DK + r0 + i4]);
                const f32x4 qv = *reinterpret_cast<const f32x4*>(&xin[j][r0 + i4]);
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    s[i4 + m] *= a[m];
                    y += kv[m] * s[i4 + m];
                    z += qv[m] * s[i4 + m];
                }
            }
            red_y[pb][rg][cg] = y;
            red_z[pb][rg][cg] = z;
            __syncthreads();   // the other parity's buffers were last read before this barrier
            f32x4 yt = zero4(), zt = zero4();
#pragma unroll
            for (int m = 0; m < NRG; ++m) {
                yt += red_y[pb][m][cg];
                zt += red_z[pb][m][cg];
            }
            const f32x4 vv = *reinterpret_cast<const f32x4*>(&xin[j][2 * DK + 4 * cg]);
            const f32x4 u = bsig[j] * (vv - yt);
#pragma unroll
            for (int i4 = 0; i4 < RPG; i4 += 4) {
                const f32x4 kv = *reinterpret_cast<const f32x4*>(&xin[j][DK + r0 + i4]);
#pragma unroll
                for (int m = 0; m < 4; ++m) s[i4 + m] += kv[m] * u;
            }
            if (tok + 1 == commit) {
#pragma unroll
                for (int i = 0; i < RPG; ++i) __builtin_nontemporal_store(s[i], reinterpret_cast<f32x4*>(Su + so0 + i * DV));
            }
            if (op && rg == (tok * (64 / CG)) % NRG) {
                // o~ for this thread's 4 columns, then RMSNorm over dv across the CG lanes of one
                // row group (within one wave) and the gate; the waves take turns by token, so
                // that no wave carries this on every token's critical path
                const f32x4 o = scale * (zt + tqk[j] * u);
                float ss = o[0] * o[0] + o[1] * o[1] + o[2] * o[2] + o[3] * o[3];
#pragma unroll
                for (int m = 1; m < CG; m *= 2) ss += __shfl_xor(ss, m, 64);
                const float inv = rsqrtf(ss / DV + eps);
                const f32x4 gt = *reinterpret_cast<const f32x4*>(&sgate[j][4 * cg]);
                const f32x4 w = norm_w ? ld<f32x4>(norm_w + 4 * cg) : f32x4{1.f, 1.f, 1.f, 1.f};
                const f32x4 yo = gt * (o * inv * w);
                const uint32_t yo_at = (uint32_t)tok * HDV + 4 * cg;
                if constexpr (OUT_F32) {
                    st<f32x4>(reinterpret_cast<float*>(yb) + yo_at, yo);
                } else {
                    bf16x4 ob{f2bf(yo[0]), f2bf(yo[1]), f2bf(yo[2]), f2bf(yo[3])};
                    st<bf16x4>(reinterpret_cast<bf16*>(yb) + yo_at, ob);
                }
            }
        }
        t0 += KB;
        if (t0 >= K) break;
        load_group(t0, K - t0 < KB ? K - t0 : KB);
        __syncthreads();   // the group's LDS is rewritten next
        prep_group(t0, K - t0 < KB ? K - t0 : KB);
    }
}

template <int DK, int DV, bool IN_F32, bool OUT_F32>
static hipError_t launch_fused(const DecodeArgs& a) {
    const int64_t units = (int64_t)a.N * a.H;
    if (units == 0 || a.K == 0) return hipSuccess;
    if (a.conv_w)
        hipLaunchKernelGGL((decode_fused_kernel<DK, DV, IN_F32, OUT_F32, true>), dim3((unsigned)units), dim3(256), 0,
                           a.stream, a.q, a.k, a.v, a.z, a.A_log, a.beta, a.G, a.norm_w, a.eps, a.S,
                           a.n_commit, a.N, a.H, a.K, a.scale, a.o, a.conv_w, a.conv_state, a.conv_width);
    else
        hipLaunchKernelGGL((decode_fused_kernel<DK, DV, IN_F32, OUT_F32, false>), dim3((unsigned)units), dim3(256), 0,
                           a.stream, a.q, a.k, a.v, a.z, a.A_log, a.beta, a.G, a.norm_w, a.eps, a.S,
                           a.n_commit, a.N, a.H, a.K, a.scale, a.o, nullptr, nullptr, 1);
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
