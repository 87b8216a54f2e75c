// KDA chunkwise prefill, one fused kernel: intra-chunk work and the inter-chunk state scan.
//
// Kimi K3: Open Frontier Intelligence, §2.1.1, eqs. (3)-(4): recurrent across chunks, parallel
// inside a chunk.  For a chunk entered with state S (positions r = 0..C-1), G_r is the running
// sum of g inside the chunk (log of the cumulative decay gamma of eq. (3)), and unrolling eq. (1)
// over the chunk gives (the UT transform the pages defer to Kimi Linear):
//     A_kk[r,i] = beta_r sum_c k_rc k_ic exp(G_rc - G_ic)        i < r   (strictly lower)
//     T = (I + A_kk)^-1,  T_b = T Diag(beta),  K~ = K * exp(G)
//     V~ = T_b (V - K~ S)            (pseudo-values; the same as U - W S with U = T_b V and
//                                     W = T_b K~, computed without forming W)
//     A_qk[r,i] = sum_c q_rc k_ic exp(G_rc - G_ic)             i <= r  (eq. (4): Tril keeps
//                                                                        the diagonal)
//     O = (Q * exp(G)) S + A_qk V~                                        (eq. (4))
//     S <- Diag(exp(G_last)) S + (K * exp(G_last - G))^T V~.
//
// Decayed products inside a chunk use 16-token sub-tiles (§2.1.1, "lower-bounded decay"): for the
// row tile a with reference E = G at the end of tile a-1 (0 for a = 0),
//     A[r,i] = sum_c (x_rc exp(G_rc - E_c)) (k_ic exp(E_c - G_ic)),
// the row factor is <= 1 and the column factor is <= exp(80) on the diagonal tile (g >= -5 over
// 16 tokens), <= 1 off it: both representable in bf16, so every causal tile, diagonal included,
// is a dense MFMA product.
//
// Grid: one 512-thread workgroup per (sequence, head, 64-column slice of dv); the slices of one
// head go to the same XCD so their reads of q, k, g share L2.  Only the last of the steps below
// depends on the state, so the workgroup is a two-stage pipeline: four producer waves prepare
// chunk i while four consumer waves advance the state through chunk i - 1.  Each SIMD runs one
// wave of each kind, so one kind's latency hides behind the other's issue.  Two workgroup
// barriers per iteration; every hand-off buffer is written after the barrier that ends its last
// read, so one copy of each suffices.
//   interval 1  producers: inputs of chunk i (prefetched one chunk ahead), in-tile decay prefix
//               (DPP scan over the 16 token lanes of a row), decayed operands in registers and the
//               partial Gram tiles of A_kk and A_qk over each wave's 32 key channels.
//               consumers: the inter-chunk step of chunk i - 1 on their 16 value columns:
//               V~ = T_b (V - K~ S), O = Q~ S + A_qk V~ (written out),
//               S <- Diag(gamma) S + K_end^T V~.  The state slice (dk x 16, fp32) stays in MFMA
//               accumulators for the whole sequence.
//   interval 2  producers: Q~, K~, K_end^T ("transposed" by a product with an identity block)
//               and the decay of the chunk to LDS.
//               consumer 0: T_b from the reduced Gram tiles by block elimination with
//               16x16x16 MFMA products (closed-form 4x4 diagonal blocks, then 8x8, 16x16, 32x32).
//               consumers 1-3: one masked A_qk tile each.
//
// Precision: bf16 MFMA with fp32 accumulation.  Operands whose rounding would dominate the error
// are carried as hi + lo bf16 pairs (products hi*hi + lo*hi + hi*lo): the decayed operands of
// A_qk, A_qk itself, V - K~ S, V~ in both of its uses, K_end (its rounding would dominate the
// state's error), both operands of (Q * exp(G)) S, which dominates short sequences entered with a
// large state.  A_kk, T_b, K~ and the state as the operand of K~ S are single bf16; the state
// stays fp32.  Float32 inputs (kFull) carry T_b and K~ as pairs too.  The scale on q is applied to
// the outputs (everything is linear in q).
//
// Precise-solve instantiation (PREC): T_b as a pair, and both operands of every product inside the
// UT solve as pairs.  With beta near 1 and keys close to one direction, A_kk's entries are near 1,
// the inverse's entries are of order one, and the single-bf16 rounding of the solve's operands
// then dominates the output's error (about 6e-3 relative instead of 1e-4 for random keys); the
// pairs bring it to 7e-4 .. 1e-3 at about 24 % more time, as the solve lies on the critical path
// of its pipeline interval.
#include <atomic>
#include <type_traits>

#include "kda_device.h"
#include "kda_launch.h"

namespace kda {

constexpr int kC = 32;     // chunk length (two 16-token sub-tiles)
constexpr int kDVT = 64;   // value columns per workgroup
constexpr int kNW = 4;     // producer waves = consumer waves
constexpr int kNT = 128 * kNW;

template <int DK, bool F32IN, bool PREC>
struct Layout {
    static constexpr bool kFull = F32IN;
    static constexpr bool kPrec = PREC;
    static constexpr int kNP = kFull ? 2 : 1;               // bf16 planes of K~
    static constexpr int kTP = kFull || kPrec ? 2 : 1;      // bf16 planes of T_b
    static constexpr int NCB = DK / 32;                       // 32-channel blocks = intra waves
    static constexpr int RB = DK + 8;                         // bf16 [token][DK] row stride
    static constexpr int TB = kC + 8;                         // bf16 [*][token] row stride
    static constexpr int SB = 16 * 20 + 16;                   // fp32 16x16 block stride (banks +16)
    static constexpr int o_Gp = 0;                            // fp32 [NCB][6][64][4] partials
    static constexpr int o_N = o_Gp + NCB * 6 * 64 * 16;      // fp32 2 blocks [16][20]: A_kk diag
    static constexpr int o_Tb = o_N + 2 * SB * 4;             // bf16 planes [C][TB]
    static constexpr int o_Aq = o_Tb + kTP * kC * TB * 2;     // bf16 hi, lo [C][TB]
    static constexpr int o_Kt = o_Aq + 2 * kC * TB * 2;       // bf16 planes [C][RB]: K~
    static constexpr int o_Qt = o_Kt + kNP * kC * RB * 2;     // bf16 hi, lo [C][RB]: Q~
    static constexpr int o_Ke = o_Qt + 2 * kC * RB * 2;       // bf16 hi, lo [DK][TB] (K_end^T)
    static constexpr int o_gam = o_Ke + 2 * DK * TB * 2;      // fp32 [DK]
    static constexpr int o_beta = o_gam + DK * 4;             // fp32 [C]
    static constexpr int total = o_beta + kC * 4;
    static_assert(total <= 160 * 1024, "LDS budget");
    static_assert(o_N - o_Gp >= 4 * (1024 + 1), "sequence ranking scratch fits the Gram region");
};

// DPP row shift right by N lanes inside each 16-lane row, zero fill.
template <int N>
__device__ __forceinline__ float row_shr(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x),
                                                                 0x110 + N, 0xF, 0xF, true));
}

__device__ __forceinline__ float row_scan16(float x) {   // inclusive prefix sum over a row
    x += row_shr<1>(x);
    x += row_shr<2>(x);
    x += row_shr<4>(x);
    x += row_shr<8>(x);
    return x;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Two floats to two bf16 (round to nearest even) in one v_cvt_pk_bf16_f32, as a packed word.
__device__ __forceinline__ uint32_t cvt_pk(float a, float b) {
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}

__device__ __forceinline__ bf16x8 to_bf16x8(const float* x) {
    const uint4 w{cvt_pk(x[0], x[1]), cvt_pk(x[2], x[3]), cvt_pk(x[4], x[5]), cvt_pk(x[6], x[7])};
    return __builtin_bit_cast(bf16x8, w);
}

// x = hi + lo, hi = bf16(x), lo = bf16(x - hi): pairs are converted together and hi is widened
// back with a shift or a mask, three operations per element.
__device__ __forceinline__ void split8(const float* x, bf16x8& hi, bf16x8& lo) {
    uint32_t h[4], l[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        h[i] = cvt_pk(x[2 * i], x[2 * i + 1]);
        const float h0 = __builtin_bit_cast(float, h[i] << 16);
        const float h1 = __builtin_bit_cast(float, h[i] & 0xffff0000u);
        l[i] = cvt_pk(x[2 * i] - h0, x[2 * i + 1] - h1);
    }
    hi = __builtin_bit_cast(bf16x8, uint4{h[0], h[1], h[2], h[3]});
    lo = __builtin_bit_cast(bf16x8, uint4{l[0], l[1], l[2], l[3]});
}

// Fragment of an f32x4 accumulator pair as an operand with the accumulator-compatible contraction
// order (element e < 4 from `a`, e >= 4 from `b`).
__device__ __forceinline__ bf16x8 acc_pair(f32x4 a, f32x4 b) {
    const float x[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    return to_bf16x8(x);
}
__device__ __forceinline__ void acc_pair_split(f32x4 a, f32x4 b, bf16x8& hi, bf16x8& lo) {
    const float x[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    split8(x, hi, lo);
}
__device__ __forceinline__ bf16x4 to_bf16x4(f32x4 a) {
    return __builtin_bit_cast(bf16x4, uint2{cvt_pk(a[0], a[1]), cvt_pk(a[2], a[3])});
}
__device__ __forceinline__ void split4(f32x4 a, bf16x4& hi, bf16x4& lo) {
    const float x[8] = {a[0], a[1], a[2], a[3], 0.f, 0.f, 0.f, 0.f};
    bf16x8 h, l;
    split8(x, h, l);
    hi = bf16x4{h[0], h[1], h[2], h[3]};
    lo = bf16x4{l[0], l[1], l[2], l[3]};
}

// 16x16x16 product, single bf16 operands: lane (i16, g4) supplies row (A) / column (B) i16 at
// contraction positions 4 g4 .. 4 g4 + 3; the result is laid out as for mma().
__device__ __forceinline__ f32x4 mma16(bf16x4 a, bf16x4 b, f32x4 c) {
    typedef short s16x4 __attribute__((ext_vector_type(4)));
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a), __builtin_bit_cast(s16x4, b), c, 0, 0, 0);
}

// The same product on fp32 operands carried as hi + lo bf16 pairs (hi*hi + lo*hi + hi*lo).
__device__ __forceinline__ f32x4 mma16x(f32x4 a, f32x4 b) {
    bf16x4 ah, al, bh, bl;
    split4(a, ah, al);
    split4(b, bh, bl);
    f32x4 c = mma16(ah, bh, zero4());
    c = mma16(al, bh, c);
    return mma16(ah, bl, c);
}

// Storage order of every 32-long contraction index in LDS: position pm(c) puts the elements one
// lane feeds to a 16x16x32 MFMA with the accumulator-compatible order (4 g4 + e for e < 4,
// 16 + 4 g4 + e - 4 for e >= 4) next to each other, so an operand is one 16-byte read.
__device__ __forceinline__ constexpr int pm(int c) {
    return (c & 16) ? ((c & 15) >> 2) * 8 + 4 + (c & 3) : (c >> 2) * 8 + (c & 3);
}

// One block of the grid -> (unit, column slice), slices of a unit on one XCD (the dispatcher
// places consecutive workgroups on consecutive XCDs, 8 of them).
__device__ __forceinline__ void block_coords(int nslices, int& unit, int& slice) {
    const int b = blockIdx.x;
    const int xcd = b & 7, slot = b >> 3;
    unit = (slot / nslices) * 8 + xcd;
    slice = slot % nslices;
}

// Buffer resource over [base, base + bytes): loads at or past `bytes` return zero, so the ragged
// tail of a sequence needs neither branches nor clamped addresses.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ uint4 bload16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
constexpr uint32_t kOOB = 0x80000000u;   // an offset past every resource: reads zero

// Redefine a prefetched register at the point of use.  Without this the compiler moves the
// conversions of next-chunk data up to the loads at the end of the previous iteration, which
// forces an immediate wait for HBM there instead of one chunk later.
__device__ __forceinline__ void pin(uint4& u) {
    asm volatile("" : "+v"(u.x), "+v"(u.y), "+v"(u.z), "+v"(u.w));
}
__device__ __forceinline__ void pin(uint32_t& u) { asm volatile("" : "+v"(u)); }
// Forces loaded values to be complete here: the loads of a batch are then issued together
// instead of each right before its first use.
__device__ __forceinline__ void pin(f32x4& u) { asm volatile("" : "+v"(u)); }
__device__ __forceinline__ void pin(bf16x8& u) { asm volatile("" : "+v"(u)); }

// Keeps the compiler from moving LDS accesses across this point; the hardware executes one
// wave's LDS instructions in order, so lanes of a wave then see each other's earlier writes.
__device__ __forceinline__ void wave_lds_order() { asm volatile("" ::: "memory"); }

// Raw 8-element fragment of one token row as stored (bf16: one 16-byte piece; f32: two).
template <bool F32IN>
struct Raw8 {
    uint4 p[F32IN ? 2 : 1];
    __device__ void load(__amdgpu_buffer_rsrc_t r, uint32_t off) {
#pragma unroll
        for (int i = 0; i < (F32IN ? 2 : 1); ++i) p[i] = bload16(r, off + 16 * i);
    }
    __device__ void pin_all() {
#pragma unroll
        for (int i = 0; i < (F32IN ? 2 : 1); ++i) pin(p[i]);
    }
    __device__ void to_f32(float* x) const {
        if constexpr (F32IN) {
            const float* f = reinterpret_cast<const float*>(p);
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] = f[e];
        } else {
            // whole 32-bit words: element 2i is the low half, 2i+1 the high half
            const uint32_t w[4] = {p[0].x, p[0].y, p[0].z, p[0].w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                x[2 * i] = __builtin_bit_cast(float, w[i] << 16);
                x[2 * i + 1] = __builtin_bit_cast(float, w[i] & 0xffff0000u);
            }
        }
    }
};

// Sequence bounds (clamped: malformed cu_seqlens never produce out-of-bounds accesses).
__device__ __forceinline__ void seq_bounds(const PrefillArgs& a, int n, int64_t& row0, int64_t& len) {
    if (a.cu) {
        int64_t s0 = a.cu[n], s1 = a.cu[n + 1];
        s0 = s0 < 0 ? 0 : (s0 > a.T ? a.T : s0);
        s1 = s1 < s0 ? s0 : (s1 > a.T ? a.T : s1);
        row0 = s0;
        len = s1 - s0;
    } else {
        row0 = (int64_t)n * a.T;
        len = a.T;
    }
}

// ==================================== producer waves =========================================
// Wave p owns key channels [32 p, 32 p + 32) (none when p >= DK / 32).  Per chunk: the decayed
// operands and the partial Gram tiles (interval 1); Q~, K~, K_end^T and gamma (interval 2).
template <int DK, bool F32IN, bool GATE, bool PREC>
__device__ __forceinline__ void producer(const PrefillArgs& a, char* smem, int p, int lane,
                                         int64_t row0, int64_t len, int h) {
    using Lay = Layout<DK, F32IN, PREC>;
    using IT = typename std::conditional<F32IN, float, bf16>::type;
    constexpr bool kFull = Lay::kFull;
    constexpr int RB = Lay::RB, TB = Lay::TB;
    auto bfp = [&](int off) { return reinterpret_cast<bf16*>(smem + off); };
    auto f32p = [&](int off) { return reinterpret_cast<float*>(smem + off); };
    const int i16 = lane & 15, g4 = lane >> 4;
    const bool intra = p < Lay::NCB;
    const int ch0 = 32 * p + 8 * g4;          // this lane's 8 key channels
    const size_t sq = (size_t)a.H * DK;       // token stride of q, k, g (elements)

    const IT* qh = reinterpret_cast<const IT*>(a.q) + (size_t)row0 * sq + (size_t)h * DK;
    const IT* kh = reinterpret_cast<const IT*>(a.k) + (size_t)row0 * sq + (size_t)h * DK;
    const float* gh = GATE ? nullptr : a.g + (size_t)row0 * sq + (size_t)h * DK;
    const IT* zh = GATE ? reinterpret_cast<const IT*>(a.z) + (size_t)row0 * sq + (size_t)h * DK : nullptr;
    // decay map of the logits: g log2(e) = g_min log2(e) / (1 + 2^(zsc z)), zsc = -exp(A_h) log2(e)
    float zsc = 0.f;
    if constexpr (GATE) zsc = -__expf(a.A_log[h]) * kLog2e;
    const IT* bh = reinterpret_cast<const IT*>(a.beta) + (size_t)row0 * a.H + h;
    uint32_t off_qk[2], off_g[2], off_b[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        const uint32_t r = 16 * t + i16;
        off_qk[t] = (uint32_t)((r * sq + ch0) * sizeof(IT));
        off_g[t] = (uint32_t)((r * sq + ch0) * 4);
        off_b[t] = (p == 0 && g4 == 0) ? (uint32_t)(r * a.H * sizeof(IT)) : kOOB;   // beta: wave 0
    }

    // identity blocks: B operand selecting channel half hh of a 32-long contraction step
    bf16x8 Id[2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int e = 0; e < 8; ++e) Id[hh][e] = f2bf((8 * g4 + e == 16 * hh + i16) ? 1.f : 0.f);

    // prefetch registers (one chunk ahead): token 16 t + i16 of tile t
    Raw8<F32IN> pq[2], pk[2], pz[2];
    uint4 pg[2][2];
    uint32_t pb[2];
    auto prefetch = [&](int64_t c0) {
        const uint32_t nv = (uint32_t)((len - c0) < kC ? (len - c0) : kC);
        const __amdgpu_buffer_rsrc_t rq = make_rsrc(qh + (size_t)c0 * sq, nv * (uint32_t)(sq * sizeof(IT)));
        const __amdgpu_buffer_rsrc_t rk = make_rsrc(kh + (size_t)c0 * sq, nv * (uint32_t)(sq * sizeof(IT)));
        const __amdgpu_buffer_rsrc_t rb = make_rsrc(bh + (size_t)c0 * a.H, nv * (uint32_t)(a.H * sizeof(IT)));
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            pq[t].load(rq, off_qk[t]);
            pk[t].load(rk, off_qk[t]);
            if constexpr (GATE) {
                pz[t].load(make_rsrc(zh + (size_t)c0 * sq, nv * (uint32_t)(sq * sizeof(IT))), off_qk[t]);
            } else {
                const __amdgpu_buffer_rsrc_t rg = make_rsrc(gh + (size_t)c0 * sq, nv * (uint32_t)(sq * 4));
                pg[t][0] = bload16(rg, off_g[t]);
                pg[t][1] = bload16(rg, off_g[t] + 16);
            }
            if (p == 0) {
                if constexpr (F32IN) pb[t] = __builtin_amdgcn_raw_buffer_load_b32(rb, off_b[t], 0, 0);
                else pb[t] = __builtin_amdgcn_raw_buffer_load_b16(rb, off_b[t], 0, 0);
            }
        }
    };

    // GATE: the log2 decay of a chunk is mapped from its logits one interval ahead, in interval 2
    // of the chunk before (the producers' shorter interval), so interval 1 only reads Lg.
    float Lg[2][8];
    auto gate_map = [&](int64_t c0) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            pz[t].pin_all();
            // tokens past the end read z = 0, whose map is not 0: they must not decay
            const bool valid = 16 * t + i16 < len - c0;
            float zv[8];
            pz[t].to_f32(zv);
#pragma unroll
            for (int e = 0; e < 8; ++e)
                Lg[t][e] = valid ? kGminLog2e * __builtin_amdgcn_rcpf(1.f + fast_exp2(zsc * zv[e])) : 0.f;
        }
    };

    const int64_t nchunks = (len + kC - 1) / kC;
    if (intra && nchunks > 0) {
        prefetch(0);
        if constexpr (GATE) gate_map(0);
    }

    for (int64_t it = 0; it <= nchunks; ++it) {
        const bool work = intra && it < nchunks;   // wave-uniform
        float F0[8], F1[8], Qs1[8], Kr[2][8], Kd1[8], Kc[8];
        bf16x8 Qh0, Ql0;

        // ---- interval 1: decay prefix, decayed operands, partial Gram tiles
        if (work) {
            float qv[2][8], kv[2][8], L[2][8];
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                pq[t].pin_all();
                pk[t].pin_all();
                if constexpr (!GATE) {
                    pin(pg[t][0]);
                    pin(pg[t][1]);
                }
            }
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                pq[t].to_f32(qv[t]);
                pk[t].to_f32(kv[t]);
                if constexpr (GATE) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) L[t][e] = Lg[t][e];
                } else {
                    const float* gl = reinterpret_cast<const float*>(pg[t]);
#pragma unroll
                    for (int e = 0; e < 8; ++e) L[t][e] = gl[e] * kLog2e;
                }
            }
            if (p == 0) {   // beta of the chunk for the solve
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    pin(pb[t]);
                    if (g4 == 0)
                        f32p(Lay::o_beta)[16 * t + i16] =
                            F32IN ? __builtin_bit_cast(float, pb[t]) : __builtin_bit_cast(float, pb[t] << 16);
                }
            }
            // the raw registers are consumed: fetch the next chunk while this one is computed
            if (it + 1 < nchunks) prefetch((it + 1) * kC);

            float P[2][8], Pi[2][8], Qs[2][8], Kd0[8];
            // in-tile prefix of the log2 decay (DPP scan across the 16 token lanes of a row)
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    L[t][e] = row_scan16(L[t][e]);
                    P[t][e] = fast_exp2(L[t][e]);        // tile start -> token, <= 1
                    Pi[t][e] = fast_exp2(-L[t][e]);      // token -> tile start, >= 1
                }
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                F0[e] = __shfl(P[0][e], (lane & ~15) | 15, 64);   // decay over tile 0
                F1[e] = __shfl(P[1][e], (lane & ~15) | 15, 64);   // decay over tile 1
            }
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    Qs[t][e] = qv[t][e] * P[t][e];
                    Kr[t][e] = kv[t][e] * P[t][e];
                }
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                Kd0[e] = kv[0][e] * Pi[0][e];
                Kd1[e] = kv[1][e] * Pi[1][e];
                Kc[e] = Kd0[e] * F0[e];                  // tile 0 seen from tile 1
                Qs1[e] = Qs[1][e];
            }
            bf16x8 Qh1, Ql1, Krh[2], Kdh[2], Kdl[2], Kch, Kcl;
            split8(Qs[0], Qh0, Ql0);
            split8(Qs[1], Qh1, Ql1);
            Krh[0] = to_bf16x8(Kr[0]);
            Krh[1] = to_bf16x8(Kr[1]);
            split8(Kd0, Kdh[0], Kdl[0]);
            split8(Kd1, Kdh[1], Kdl[1]);
            split8(Kc, Kch, Kcl);
            // Gram tiles transposed (column side as the A operand): the accumulator of lane
            // (row r = i16, g4) holds A[r][16 b + 4 g4 + j].  m: 0 qk00, 1 qk11, 2 qk10,
            // 3 kk00, 4 kk11, 5 kk10.  A_qk with split operands (3 products); A_kk feeds only the
            // triangular inverse, where single bf16 operands cost no measurable accuracy.
#pragma unroll
            for (int m = 0; m < 6; ++m) {
                const int ta = (m % 3 == 0) ? 0 : 1;
                const bf16x8 ch = (m % 3 == 2) ? Kch : Kdh[ta];
                const bf16x8 cl = (m % 3 == 2) ? Kcl : Kdl[ta];
                f32x4 acc;
                if (m < 3) {
                    const bf16x8 rh = ta ? Qh1 : Qh0, rl = ta ? Ql1 : Ql0;
                    acc = mma(ch, rh, zero4());
                    acc = mma(cl, rh, acc);
                    acc = mma(ch, rl, acc);
                } else {
                    acc = mma(ch, Krh[ta], zero4());
                }
                st<f32x4>(smem + Lay::o_Gp + ((p * 6 + m) * 64 + lane) * 16, acc);
            }
        }
        __syncthreads();

        // ---- interval 2: Q~ (split), K~ and K_end^T to LDS, and the decay of the chunk
        if (work) {
            if (i16 == 0) {
#pragma unroll
                for (int e = 0; e < 8; ++e) f32p(Lay::o_gam)[ch0 + e] = F0[e] * F1[e];
            }
            // 8 channels of token 16 t + i16 into [token][pm(channel)] storage
            auto put_row = [&](int off, int t, bf16x8 v) {
                bf16* d = bfp(off) + (16 * t + i16) * RB + 32 * p;
                st<bf16x4>(d + pm(8 * g4), bf16x4{v[0], v[1], v[2], v[3]});
                st<bf16x4>(d + pm(8 * g4 + 4), bf16x4{v[4], v[5], v[6], v[7]});
            };
            // Q~ = Q exp(G), K~ = K exp(G) from the chunk start; tile 1 carries the tile-0 decay
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                bf16x8 hh = Qh0, ll = Ql0;
                float xt[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) xt[e] = t ? Kr[1][e] * F0[e] : Kr[0][e];
                if (t == 1) {
                    float x[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) x[e] = Qs1[e] * F0[e];
                    split8(x, hh, ll);
                }
                put_row(Lay::o_Qt, t, hh);
                put_row(Lay::o_Qt + kC * RB * 2, t, ll);
                if constexpr (kFull) {
                    bf16x8 th, tl;
                    split8(xt, th, tl);
                    put_row(Lay::o_Kt, t, th);
                    put_row(Lay::o_Kt + kC * RB * 2, t, tl);
                } else {
                    put_row(Lay::o_Kt, t, to_bf16x8(xt));
                }
            }
            // K_end = K exp(G_last - G), transposed through the identity: the accumulator of lane
            // (channel i16 of half hh, g4) holds tokens 16 t + 4 g4 + j.
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                float xe[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) xe[e] = t ? Kd1[e] * F1[e] : Kc[e] * F1[e];
                bf16x8 eh, el;
                split8(xe, eh, el);
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    bf16* dst = bfp(Lay::o_Ke) + (32 * p + 16 * hh + i16) * TB + pm(16 * t + 4 * g4);
                    st<bf16x4>(dst, to_bf16x4(mma(eh, Id[hh], zero4())));          // exact: bf16 in
                    st<bf16x4>(dst + DK * TB, to_bf16x4(mma(el, Id[hh], zero4())));
                }
            }
            if constexpr (GATE) {
                if (it + 1 < nchunks) gate_map((it + 1) * kC);
            }
        }
        __syncthreads();
    }
}

// ==================================== consumer waves =========================================
// Wave 4 + cw owns value columns [16 cw, 16 cw + 16) of the slice and its dk x 16 state slice.
// Interval 1 of iteration i: the inter-chunk step of chunk i - 1.  Interval 2: chunk i's T_b
// (cw = 0) or one A_qk tile (cw = 1..3).
template <int DK, bool F32IN, bool OUT_F32, bool PREC>
__device__ __forceinline__ void consumer(const PrefillArgs& a, char* smem, int cw, int lane,
                                         int64_t row0, int64_t len, int n, int h, int slice, int seg) {
    using Lay = Layout<DK, F32IN, PREC>;
    using IT = typename std::conditional<F32IN, float, bf16>::type;
    constexpr bool kFull = Lay::kFull;
    constexpr int KS = DK / 32;          // 32-channel contraction steps
    constexpr int CT = DK / 16;          // 16-channel tiles of the state
    constexpr int NCB = Lay::NCB;
    constexpr int RB = Lay::RB, TB = Lay::TB, SB = Lay::SB;
    auto bfp = [&](int off) { return reinterpret_cast<bf16*>(smem + off); };
    auto f32p = [&](int off) { return reinterpret_cast<float*>(smem + off); };
    const int i16 = lane & 15, g4 = lane >> 4;
    const int H = a.H;
    const size_t sv = (size_t)H * a.dv;        // token stride of v, o
    const int col0 = slice * kDVT + 16 * cw;   // first value column of this wave
    // segment summaries: columns >= dv carry the segment's transition (value 0); no outputs
    const bool tcols = a.mode == 1 && col0 >= a.dv;
    const bool vlane = g4 < 2 && !tcols;       // lanes that load this wave's 16 v columns

    const IT* vh = reinterpret_cast<const IT*>(a.v) + (size_t)row0 * sv + (size_t)h * a.dv + col0;
    using OT = typename std::conditional<OUT_F32, float, bf16>::type;
    OT* ob = reinterpret_cast<OT*>(a.o) + (size_t)row0 * sv + (size_t)h * a.dv + col0;
    uint32_t off_v[2], off_o[2][4];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        const uint32_t r = 16 * t + i16;
        off_v[t] = vlane ? (uint32_t)((r * sv + 8 * g4) * sizeof(IT)) : kOOB;
#pragma unroll
        for (int j = 0; j < 4; ++j)   // output row 16 t + 4 g4 + j, column i16
            off_o[t][j] = (uint32_t)(((16 * t + 4 * g4 + j) * sv + i16) * sizeof(OT));
    }

    // ---- state slice in accumulators: Sacc[ct][j] = S[16 ct + 4 g4 + j][col0 + i16]
    f32x4 Sacc[CT];
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) Sacc[ct] = zero4();
    const int wcols = a.dv + DK;   // row length of a segment summary [dk][dv + dk]
    auto summary = [&](int j) {    // summary of segment j of this (sequence, head)
        return a.ws + (((size_t)n * (a.nseg - 1) + j) * H + h) * DK * wcols;
    };
    if (tcols) {
        // transition columns start as the identity
        const int c = col0 - a.dv + i16;
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
#pragma unroll
            for (int j = 0; j < 4; ++j) Sacc[ct][j] = (16 * ct + 4 * g4 + j == c) ? 1.f : 0.f;
    } else if (a.mode == 2 && seg > 0) {
        // entering state of segment seg: the state after segment 0 (entered with S0), carried
        // through segments 1 .. seg-1 by S <- M_j S + S~_j (products on split bf16 operands)
        const float* W0 = summary(0);
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
#pragma unroll
            for (int j = 0; j < 4; ++j) Sacc[ct][j] = W0[(size_t)(16 * ct + 4 * g4 + j) * wcols + col0 + i16];
        for (int jseg = 1; jseg < seg; ++jseg) {
            const float* Wj = summary(jseg);
            bf16x8 Sh[KS], Sl[KS];
#pragma unroll
            for (int s2 = 0; s2 < KS; ++s2) acc_pair_split(Sacc[2 * s2], Sacc[2 * s2 + 1], Sh[s2], Sl[s2]);
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) {
                f32x4 acc;
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[j] = Wj[(size_t)(16 * ct + 4 * g4 + j) * wcols + col0 + i16];
                // A operand: row 16 ct + i16 of M_j, contraction positions of the B operand
                const float* Mr = Wj + (size_t)(16 * ct + i16) * wcols + a.dv;
#pragma unroll
                for (int s2 = 0; s2 < KS; ++s2) {
                    const f32x4 m0 = ld<f32x4>(Mr + 32 * s2 + 4 * g4);
                    const f32x4 m1 = ld<f32x4>(Mr + 32 * s2 + 16 + 4 * g4);
                    bf16x8 mh, ml;
                    acc_pair_split(m0, m1, mh, ml);
                    acc = mma(mh, Sh[s2], acc);
                    acc = mma(ml, Sh[s2], acc);
                    acc = mma(mh, Sl[s2], acc);
                }
                Sacc[ct] = acc;
            }
        }
    } else if (a.S0 && !(a.mode == 1 && seg > 0)) {
        const float* S0 = a.S0 + ((size_t)n * H + h) * DK * a.dv;
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                Sacc[ct][j] = S0[(size_t)(16 * ct + 4 * g4 + j) * a.dv + col0 + i16];
    }

    // the upper-right 16x16 blocks of T_b and A_qk are zero for every chunk
    if (cw == 1) {
        const bf16x4 z{f2bf(0.f), f2bf(0.f), f2bf(0.f), f2bf(0.f)};
        bf16* ad = bfp(Lay::o_Aq) + i16 * TB + pm(16 + 4 * g4);
        st<bf16x4>(ad, z);
        st<bf16x4>(ad + kC * TB, z);
        bf16* td = bfp(Lay::o_Tb) + i16 * TB + pm(16 + 4 * g4);
#pragma unroll
        for (int pl = 0; pl < Lay::kTP; ++pl) st<bf16x4>(td + pl * kC * TB, z);
    }

    bf16x8 Id0;   // identity block: B operand selecting columns 0..15 of a 32-long step
#pragma unroll
    for (int e = 0; e < 8; ++e) Id0[e] = f2bf((8 * g4 + e == i16) ? 1.f : 0.f);

    Raw8<F32IN> pv[2];
    auto prefetch_v = [&](int64_t c0) {
        const uint32_t nv = (uint32_t)((len - c0) < kC ? (len - c0) : kC);
        const __amdgpu_buffer_rsrc_t rv = make_rsrc(vh + (size_t)c0 * sv, nv * (uint32_t)(sv * sizeof(IT)));
#pragma unroll
        for (int t = 0; t < 2; ++t) pv[t].load(rv, off_v[t]);
    };
    auto reduce = [&](int m) -> f32x4 {   // sum of the producers' partial Gram tiles
        f32x4 acc = ld<f32x4>(smem + Lay::o_Gp + (m * 64 + lane) * 16);
#pragma unroll
        for (int w = 1; w < NCB; ++w) acc += ld<f32x4>(smem + Lay::o_Gp + ((w * 6 + m) * 64 + lane) * 16);
        return acc;
    };
    auto put_tb = [&](int r, int c, float v) {   // T_b[r][c] (one or two bf16 planes)
        bf16* Tb = bfp(Lay::o_Tb);
        if constexpr (Lay::kTP == 2) {
            bf16 hh, ll;
            split_bf16(v, hh, ll);
            Tb[r * TB + pm(c)] = hh;
            Tb[kC * TB + r * TB + pm(c)] = ll;
        } else {
            Tb[r * TB + pm(c)] = f2bf(v);
        }
    };

    const int64_t nchunks = (len + kC - 1) / kC;
    if (nchunks > 0) prefetch_v(0);

    for (int64_t it = 0; it <= nchunks; ++it) {
        // ---- interval 1: inter-chunk step of chunk it - 1 on this wave's 16 state columns.
        // LDS operands come in three batches, each issued ahead of independent work and pinned
        // at its first use (without this each MFMA waits for its own read).
        if (it > 0) {
            const int64_t c0 = (it - 1) * kC;
            const uint32_t nvalid = a.mode == 1 ? 0u : (uint32_t)((len - c0) < kC ? (len - c0) : kC);
            // output rows of the chunk: stores at or past row nvalid fall outside the resource
            // (summaries write no outputs)
            const __amdgpu_buffer_rsrc_t ro = make_rsrc(ob + (size_t)c0 * sv, nvalid * (uint32_t)(sv * sizeof(OT)));
            // operand fragments read from [row][pm(index)] storage: elements 4 g4 + e (e < 4) and
            // 16 + 4 g4 + e - 4 (e >= 4) of each 32-long contraction step are one 16-byte read
            auto frag = [&](int off, int row, int stride, int col) -> bf16x8 {
                return ld<bf16x8>(bfp(off) + row * stride + col + 8 * g4);
            };
            // batch 1: rows of K~ (for K~ S) and of T_b
            constexpr int kPL = Lay::kTP > Lay::kNP ? Lay::kTP : Lay::kNP;
            bf16x8 tbr[2][Lay::kTP], kt[2][KS][Lay::kNP];
#pragma unroll
            for (int ta = 0; ta < 2; ++ta)
#pragma unroll
                for (int pl = 0; pl < kPL; ++pl) {
                    if (pl < Lay::kTP) tbr[ta][pl] = frag(Lay::o_Tb + pl * kC * TB * 2, 16 * ta + i16, TB, 0);
                    if (pl < Lay::kNP)
#pragma unroll
                        for (int s = 0; s < KS; ++s) kt[ta][s][pl] = frag(Lay::o_Kt + pl * kC * RB * 2, 16 * ta + i16, RB, 32 * s);
                }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int t = 0; t < 2; ++t) pv[t].pin_all();
            Raw8<F32IN> vr[2] = {pv[0], pv[1]};
            if (it < nchunks) prefetch_v(it * kC);

            // V: token-per-lane -> column-per-lane through a product with the identity; the
            // accumulator of lane (column i16, g4) holds tokens 16 t + 4 g4 + j
            f32x4 Vf[2];
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                if constexpr (kFull) {
                    float vv[8];
                    vr[t].to_f32(vv);
                    bf16x8 vh, vl;
                    split8(vv, vh, vl);
                    Vf[t] = mma(vl, Id0, mma(vh, Id0, zero4()));
                } else {
                    Vf[t] = mma(__builtin_bit_cast(bf16x8, vr[t].p[0]), Id0, zero4());   // bf16 as stored
                }
            }
            // state as B operand: contraction index (32-channel step s, g4, e) ->
            // channel 32 s + 4 g4 + e (e < 4), 32 s + 16 + 4 g4 + (e - 4) (e >= 4)
            bf16x8 Sh[KS], Sl[KS];
#pragma unroll
            for (int s = 0; s < KS; ++s) acc_pair_split(Sacc[2 * s], Sacc[2 * s + 1], Sh[s], Sl[s]);
#pragma unroll
            for (int ta = 0; ta < 2; ++ta)
#pragma unroll
                for (int pl = 0; pl < kPL; ++pl) {
                    if (pl < Lay::kTP) pin(tbr[ta][pl]);
                    if (pl < Lay::kNP)
#pragma unroll
                        for (int s = 0; s < KS; ++s) pin(kt[ta][s][pl]);
                }
            // batch 2: rows of Q~ (hi, lo) and of A_qk (hi, lo)
            bf16x8 qr[2][KS][2], ar[2][2];
#pragma unroll
            for (int ta = 0; ta < 2; ++ta)
#pragma unroll
                for (int pl = 0; pl < 2; ++pl) {
                    ar[ta][pl] = frag(Lay::o_Aq + pl * kC * TB * 2, 16 * ta + i16, TB, 0);
#pragma unroll
                    for (int s = 0; s < KS; ++s) qr[ta][s][pl] = frag(Lay::o_Qt + pl * kC * RB * 2, 16 * ta + i16, RB, 32 * s);
                }
            __builtin_amdgcn_sched_barrier(0);
            // V~ = T_b (V - K~ S): the residual R = V - K~ S in fp32, then one product with T_b
            // (R split, so only T_b's own planes are rounded)
            f32x4 Vt[2];
            {
                f32x4 R[2];
#pragma unroll
                for (int ta = 0; ta < 2; ++ta) {
                    f32x4 acc = zero4();
#pragma unroll
                    for (int s = 0; s < KS; ++s) {
                        acc = mma(kt[ta][s][0], Sh[s], acc);
                        if constexpr (kFull) {
                            acc = mma(kt[ta][s][1], Sh[s], acc);
                            acc = mma(kt[ta][s][0], Sl[s], acc);
                        }
                    }
                    R[ta] = Vf[ta] - acc;
                }
                bf16x8 Rh, Rl;   // R as B operand: token index (g4, e) as for V~ below
                acc_pair_split(R[0], R[1], Rh, Rl);
#pragma unroll
                for (int ta = 0; ta < 2; ++ta) {
                    f32x4 v = mma(tbr[ta][0], Rh, zero4());
                    v = mma(tbr[ta][0], Rl, v);
                    if constexpr (Lay::kTP == 2) v = mma(tbr[ta][1], Rh, v);
                    Vt[ta] = v;
                }
            }
            // V~ as B operand: token index (g4, e) -> 4 g4 + e (e < 4), 16 + 4 g4 + (e - 4)
            bf16x8 Vh, Vl;
            acc_pair_split(Vt[0], Vt[1], Vh, Vl);
#pragma unroll
            for (int ta = 0; ta < 2; ++ta)
#pragma unroll
                for (int pl = 0; pl < 2; ++pl) {
                    pin(ar[ta][pl]);
#pragma unroll
                    for (int s = 0; s < KS; ++s) pin(qr[ta][s][pl]);
                }
            // outputs O = Q~ S + A_qk V~
            f32x4 Oacc[2];
#pragma unroll
            for (int ta = 0; ta < 2; ++ta) {
                f32x4 acc = zero4();
#pragma unroll
                for (int s = 0; s < KS; ++s) {
                    acc = mma(qr[ta][s][0], Sh[s], acc);
                    acc = mma(qr[ta][s][1], Sh[s], acc);
                    acc = mma(qr[ta][s][0], Sl[s], acc);
                }
                Oacc[ta] = acc;
            }
            // batch 3, in two halves (registers): rows of K_end^T (hi, lo) and the chunk decay
            // gamma for state tiles [0, CT/2), then [CT/2, CT)
            constexpr int CH = CT / 2;
            bf16x8 kr[CH][2];
            f32x4 gm[CH];
            auto load_half = [&](int c0h) {
#pragma unroll
                for (int c = 0; c < CH; ++c) {
#pragma unroll
                    for (int pl = 0; pl < 2; ++pl) kr[c][pl] = frag(Lay::o_Ke + pl * DK * TB * 2, 16 * (c0h + c) + i16, TB, 0);
                    gm[c] = ld<f32x4>(f32p(Lay::o_gam) + 16 * (c0h + c) + 4 * g4);
                }
            };
            // state: S <- Diag(gamma_last) S + K_end^T V~ on tiles [c0h, c0h + CH)
            auto update_half = [&](int c0h) {
#pragma unroll
                for (int c = 0; c < CH; ++c) {
                    pin(kr[c][0]);
                    pin(kr[c][1]);
                    pin(gm[c]);
                }
#pragma unroll
                for (int c = 0; c < CH; ++c) {
                    f32x4 st = Sacc[c0h + c] * gm[c];
                    st = mma(kr[c][0], Vh, st);
                    st = mma(kr[c][0], Vl, st);
                    st = mma(kr[c][1], Vh, st);
                    Sacc[c0h + c] = st;
                }
            };
            load_half(0);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int ta = 0; ta < 2; ++ta) {
                f32x4 acc = Oacc[ta];
                acc = mma(ar[ta][0], Vh, acc);
                acc = mma(ar[ta][1], Vh, acc);
                acc = mma(ar[ta][0], Vl, acc);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    if constexpr (OUT_F32)
                        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, a.scale * acc[j]), ro,
                                                              off_o[ta][j], 0, 0);
                    else
                        __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(uint16_t, f2bf(a.scale * acc[j])), ro,
                                                              off_o[ta][j], 0, 0);
                }
            }
            update_half(0);
            load_half(CH);
            update_half(CH);
            // state checkpoint after every ckpt_every full chunks (prefix states for reuse)
            if (a.ckpt && it % a.ckpt_every == 0 && it * kC <= len) {
                const int64_t j = it / a.ckpt_every - 1;
                if (j < a.ckpt_cap) {
                    float* C = a.ckpt + (((size_t)n * H + h) * a.ckpt_cap + j) * DK * a.dv;
                    // 32-bit lane offset, opaque so that the 32 store addresses are formed here
                    // rather than hoisted out of the chunk loop into registers
                    int lo = 4 * g4 * a.dv + col0 + i16;
                    asm volatile("" : "+v"(lo));
#pragma unroll
                    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                        for (int jj = 0; jj < 4; ++jj) C[lo + (16 * ct + jj) * a.dv] = Sacc[ct][jj];
                }
            }
        }
        __syncthreads();

        // ---- interval 2: the UT solve (cw = 0) and the A_qk tiles (cw = 1..3) of chunk it
        if (it < nchunks) {
            if (cw == 0) {
                // T = (I + N)^-1, N = A_kk with rows scaled by beta (strictly lower, 32 x 32).
                // Each diagonal 16x16 block B = L0 + L1 + L2 (L0: inside the 4x4 diagonal
                // blocks; L1: the 4x4 blocks just below them within each 8x8 diagonal block; L2:
                // the lower-left 8x8 block) is inverted by block elimination,
                //     D = (I + L0)^-1 (closed form, fp32),  E = D - D L1 D,  X = E - E L2 E,
                // each product filling blocks that are zero in the previous level (no
                // cancellation), and T10 = -T11 N10 T00.  Products are 16x16x16 MFMAs on single
                // bf16 operands (on hi + lo pairs in the precise-solve instantiation), and the
                // diagonal 4x4 blocks stay fp32.  Forms: row form of M in lane (i16, g4) = M[i16][4 g4 + j], column
                // form = M[4 g4 + j][i16]; mma16(row form of X, column form of Y) is the column
                // form of X Y, and the row form of M is the column form of M^T.
                const float bt[2] = {f32p(Lay::o_beta)[i16], f32p(Lay::o_beta)[16 + i16]};
                // an opaque lane index: keeps the compiler from hoisting lane-constant masks out
                // of the chunk loop into registers held across it
                int lid = i16;
                asm volatile("" : "+v"(lid));
                const int rb = lid >> 2;                       // 4-row block of this lane's row / column
                f32x4 Nr[2];
                Nr[0] = reduce(3);
                Nr[1] = reduce(4);
                f32x4 N10r = reduce(5);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const bool low = 4 * g4 + j < lid;
                    Nr[0][j] = low ? Nr[0][j] * bt[0] : 0.f;
                    Nr[1][j] = low ? Nr[1][j] * bt[1] : 0.f;
                    N10r[j] *= bt[1];
                }
                float* Nb = f32p(Lay::o_N);
                st<f32x4>(Nb + i16 * 20 + 4 * g4, Nr[0]);
                st<f32x4>(Nb + SB + i16 * 20 + 4 * g4, Nr[1]);
                wave_lds_order();
                f32x4 Nc[2], n1[2], n2[2], n3[2];
#pragma unroll
                for (int q = 0; q < 2; ++q) {
#pragma unroll
                    for (int j = 0; j < 4; ++j) Nc[q][j] = Nb[q * SB + (4 * g4 + j) * 20 + i16];
                    // rows 1..3 of the 4x4 diagonal block g4 (strictly lower entries)
                    n1[q] = ld<f32x4>(Nb + q * SB + (4 * g4 + 1) * 20 + 4 * g4);
                    n2[q] = ld<f32x4>(Nb + q * SB + (4 * g4 + 2) * 20 + 4 * g4);
                    n3[q] = ld<f32x4>(Nb + q * SB + (4 * g4 + 3) * 20 + 4 * g4);
                    pin(n1[q]);   // whole rows in separate registers, read together
                    pin(n2[q]);
                    pin(n3[q]);
                }
                const bool on_diag = g4 == rb;                 // this lane's 4-block holds D entries
                const int kk = lid & 3;
                const float d0 = kk == 0 ? 1.f : 0.f, d1 = kk == 1 ? 1.f : 0.f;
                const float d2 = kk == 2 ? 1.f : 0.f, d3 = kk == 3 ? 1.f : 0.f;
                // whole-vector masks: L1 and L2 in row form (row i16, columns 4 g4 + j) and in
                // column form (rows 4 g4 + j, column i16)
                const bool l1r = (rb == 1 || rb == 3) && g4 == rb - 1;
                const bool l1c = (g4 == 1 || g4 == 3) && rb == g4 - 1;
                const bool l2r = lid >= 8 && g4 < 2;
                const bool l2c = g4 >= 2 && lid < 8;
                auto mask = [](f32x4 v, bool keep) { return keep ? v : zero4(); };
                f32x4 Xc0, Xr1;
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    // D = (I + L0)^-1: column kk (column form) and row kk (row form) of the
                    // inverse of the unit lower 4x4 block g4
                    const float x1 = d1 - n1[q][0] * d0;
                    const float x2 = d2 - n2[q][0] * d0 - n2[q][1] * x1;
                    const float x3 = d3 - n3[q][0] * d0 - n3[q][1] * x1 - n3[q][2] * x2;
                    const float y2 = d2 - d3 * n3[q][2];
                    const float y1 = d1 - y2 * n2[q][1] - d3 * n3[q][1];
                    const float y0 = d0 - y1 * n1[q][0] - y2 * n2[q][0] - d3 * n3[q][0];
                    const f32x4 Dc = on_diag ? f32x4{d0, x1, x2, x3} : zero4();
                    const f32x4 Dr = on_diag ? f32x4{y0, y1, y2, d3} : zero4();
                    if constexpr (Lay::kPrec) {
                        // E = D - D L1 D (column form), E^T = D^T - D^T L1^T D^T (row form of E)
                        const f32x4 Ec = Dc - mma16x(Dr, mma16x(mask(Nr[q], l1r), Dc));
                        const f32x4 Er = Dr - mma16x(Dc, mma16x(mask(Nc[q], l1c), Dr));
                        // X = E - E L2 E: column form for T00, row form for T11
                        if (q == 0)
                            Xc0 = Ec - mma16x(Er, mma16x(mask(Nr[q], l2r), Ec));
                        else
                            Xr1 = Er - mma16x(Ec, mma16x(mask(Nc[q], l2c), Er));
                    } else {
                        const bf16x4 Dcb = to_bf16x4(Dc), Drb = to_bf16x4(Dr);
                        const f32x4 Ec = Dc - mma16(Drb, to_bf16x4(mma16(to_bf16x4(mask(Nr[q], l1r)), Dcb, zero4())), zero4());
                        const f32x4 Er = Dr - mma16(Dcb, to_bf16x4(mma16(to_bf16x4(mask(Nc[q], l1c)), Drb, zero4())), zero4());
                        const bf16x4 Ecb = to_bf16x4(Ec), Erb = to_bf16x4(Er);
                        if (q == 0)
                            Xc0 = Ec - mma16(Erb, to_bf16x4(mma16(to_bf16x4(mask(Nr[q], l2r)), Ecb, zero4())), zero4());
                        else
                            Xr1 = Er - mma16(Ecb, to_bf16x4(mma16(to_bf16x4(mask(Nc[q], l2c)), Erb, zero4())), zero4());
                    }
                }
                // T10 = -T11 (N10 T00), column form
                f32x4 T10c;
                if constexpr (Lay::kPrec)
                    T10c = -mma16x(Xr1, mma16x(N10r, Xc0));
                else
                    T10c = -mma16(to_bf16x4(Xr1), to_bf16x4(mma16(to_bf16x4(N10r), to_bf16x4(Xc0), zero4())), zero4());
                // T_b = T Diag(beta): T00 and T10 from column forms (column i16), T11 from its row
                // form (row 16 + i16, four adjacent columns)
                const f32x4 bcol = ld<f32x4>(f32p(Lay::o_beta) + 16 + 4 * g4);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    put_tb(4 * g4 + j, i16, Xc0[j] * bt[0]);
                    put_tb(16 + 4 * g4 + j, i16, T10c[j] * bt[0]);
                }
                const f32x4 t11 = Xr1 * bcol;
                bf16* tr = bfp(Lay::o_Tb) + (16 + i16) * TB + pm(16 + 4 * g4);
                if constexpr (Lay::kTP == 2) {
                    bf16x4 hv, lv;
                    split4(t11, hv, lv);
                    st<bf16x4>(tr, hv);
                    st<bf16x4>(tr + kC * TB, lv);
                } else {
                    st<bf16x4>(tr, to_bf16x4(t11));
                }
            } else {
                // A_qk tile m (masked) -> split bf16 [row][pm(col)]
                const int m = cw - 1;   // 0: rows 0-15 x cols 0-15, 1: 16-31 x 16-31, 2: 16-31 x 0-15
                f32x4 acc = reduce(m);
                const int ta = (m == 0) ? 0 : 1, tb = (m == 1) ? 1 : 0;
                const int r = 16 * ta + i16;
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[j] = (16 * tb + 4 * g4 + j <= r) ? acc[j] : 0.f;
                bf16x4 hv, lv;
                split4(acc, hv, lv);
                bf16* ad = bfp(Lay::o_Aq) + r * TB + pm(16 * tb + 4 * g4);
                st<bf16x4>(ad, hv);
                st<bf16x4>(ad + kC * TB, lv);
            }
        }
        __syncthreads();
    }

    if (a.mode == 1) {
        float* W = summary(seg);
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
#pragma unroll
            for (int j = 0; j < 4; ++j) W[(size_t)(16 * ct + 4 * g4 + j) * wcols + col0 + i16] = Sacc[ct][j];
    } else if (a.ST && (a.mode == 0 || seg == a.nseg - 1)) {
        float* ST = a.ST + ((size_t)n * H + h) * DK * a.dv;
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                ST[(size_t)(16 * ct + 4 * g4 + j) * a.dv + col0 + i16] = Sacc[ct][j];
    }
}

// Packed sequences run longest first: the workgroups of rank r take the r-th longest sequence
// (ties in index order), so a long sequence does not start only after the short ones before it
// in the batch have been through the machine.  Every thread of the workgroup calls this; the
// lengths are ranked in LDS (the Gram-partials region, not yet in use), 1024 sequences at most.
constexpr int kRankMax = 1024;
__device__ int seq_of_rank(const PrefillArgs& a, int r, char* smem) {
    int* L = reinterpret_cast<int*>(smem);
    int* found = L + kRankMax;
    const int n4 = (a.N + 3) / 4;
    for (int m = threadIdx.x; m < 4 * n4; m += kNT) {
        int64_t row0 = 0, len = -1;       // padding ranks below every real length
        if (m < a.N) seq_bounds(a, m, row0, len);
        L[m] = (int)len;
    }
    if (threadIdx.x == 0) *found = r;     // unreachable for a valid r; keeps the result in range
    __syncthreads();
    for (int m = threadIdx.x; m < a.N; m += kNT) {
        const int lm = L[m];
        int rank = 0;
        for (int j4 = 0; j4 < n4; ++j4) {
            const int4 v = reinterpret_cast<const int4*>(L)[j4];
            const int j = 4 * j4;
            rank += (v.x > lm) | ((v.x == lm) & (j < m));
            rank += (v.y > lm) | ((v.y == lm) & (j + 1 < m));
            rank += (v.z > lm) | ((v.z == lm) & (j + 2 < m));
            rank += (v.w > lm) | ((v.w == lm) & (j + 3 < m));
        }
        if (rank == r) *found = m;
    }
    __syncthreads();
    const int n = *found;
    __syncthreads();   // the region is reused by the pipeline
    return n;
}

// Both roles run the same number of iterations (chunks + 1) with two barriers each.  RANK: packed
// sequences (at most kRankMax) in longest-first order; a separate instantiation, so that the
// fixed-length kernel's code is not changed by the ranking.  PREC: the precise solve.
template <int DK, bool F32IN, bool OUT_F32, bool GATE, bool RANK, bool PREC>
__global__ __launch_bounds__(kNT) void prefill_kernel(PrefillArgs a) {
    extern __shared__ __attribute__((aligned(16))) char smem[];
    const int nslices = (a.mode == 1 ? a.dv + a.dk : a.dv) / kDVT;
    const int nseg = a.mode == 0 ? 1 : a.nseg;
    int unit, slice;
    block_coords(nslices, unit, slice);
    if (unit >= a.N * a.H * nseg) return;
    const int h = unit % a.H;
    const int seg = (unit / a.H) % nseg;
    const int rank = unit / (a.H * nseg);
    if (a.mode == 1 && (seg == nseg - 1 || (seg == 0 && slice * kDVT >= a.dv))) return;   // not needed
    KDA_POISON(smem, (Layout<DK, F32IN, PREC>::total));
    KDA_POISON_DONE();
    int n = rank;
    if constexpr (RANK) n = seq_of_rank(a, rank, smem);
    int64_t row0, len;
    seq_bounds(a, n, row0, len);
    if (a.mode != 0) {   // this segment's tokens
        const int64_t lo = (int64_t)seg * a.seg_len;
        const int64_t hi = lo + a.seg_len < len ? lo + a.seg_len : len;
        row0 += lo;
        len = hi > lo ? hi - lo : 0;
    }
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform (scalar)
    if (wave < kNW) producer<DK, F32IN, GATE, PREC>(a, smem, wave, lane, row0, len, h);
    else consumer<DK, F32IN, OUT_F32, PREC>(a, smem, wave - kNW, lane, row0, len, n, h, slice, seg);
}

template <int DK, bool F32IN, bool OUT_F32, bool GATE, bool RANK, bool PREC>
static hipError_t launch_one(const PrefillArgs& a) {
    using Lay = Layout<DK, F32IN, PREC>;
    auto kern = prefill_kernel<DK, F32IN, OUT_F32, GATE, RANK, PREC>;
    // The LDS limit is a per-device attribute of the kernel: set it once on each device this
    // instantiation launches on (devices past 63 set it on every launch).  Concurrent first calls
    // may both set it; the value is the same.
    static std::atomic<uint64_t> attr_set{0};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const uint64_t bit = (dev >= 0 && dev < 64) ? (uint64_t{1} << dev) : 0;
    if (!(attr_set.load(std::memory_order_relaxed) & bit) || !bit) {
        e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                                Lay::total);
        if (e != hipSuccess) return e;
        attr_set.fetch_or(bit, std::memory_order_relaxed);
    }
    const int nslices = (a.mode == 1 ? a.dv + a.dk : a.dv) / kDVT;
    const int64_t units = (int64_t)a.N * a.H * (a.mode == 0 ? 1 : a.nseg);
    const int64_t blocks = ((units + 7) / 8) * 8 * nslices;
    if (blocks == 0) return hipSuccess;
    hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(kNT), Lay::total, a.stream, a);
    return hipGetLastError();
}

template <int DK, bool F32IN, bool OUT_F32, bool GATE, bool PREC>
static hipError_t launch_ranked(const PrefillArgs& a) {
    if (a.cu && a.N > 1 && a.N <= kRankMax) return launch_one<DK, F32IN, OUT_F32, GATE, true, PREC>(a);
    return launch_one<DK, F32IN, OUT_F32, GATE, false, PREC>(a);
}

template <int DK, bool F32IN, bool OUT_F32, bool GATE>
static hipError_t launch_prefill(const PrefillArgs& a) {
    return a.precise ? launch_ranked<DK, F32IN, OUT_F32, GATE, true>(a)
                     : launch_ranked<DK, F32IN, OUT_F32, GATE, false>(a);
}

template <bool GATE>
static hipError_t dispatch_prefill(const PrefillArgs& a) {
    if (a.dk == 128) {
        // float32 inputs are supported at dk = 64 (the ABI rejects them at dk = 128)
        if (a.in_f32) return hipErrorInvalidValue;
        return a.out_f32 ? launch_prefill<128, false, true, GATE>(a) : launch_prefill<128, false, false, GATE>(a);
    }
    if (a.dk == 64) {
        if (a.in_f32)
            return a.out_f32 ? launch_prefill<64, true, true, GATE>(a) : launch_prefill<64, true, false, GATE>(a);
        return a.out_f32 ? launch_prefill<64, false, true, GATE>(a) : launch_prefill<64, false, false, GATE>(a);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_chunk_fwd(const PrefillArgs& a) {
    return a.z ? dispatch_prefill<true>(a) : dispatch_prefill<false>(a);
}

}  // namespace kda
