// KDA chunkwise prefill, one fused kernel: intra-chunk work and the inter-chunk state scan.
//
// Kimi K3: Open Frontier Intelligence, §2.1.1, eqs. (3)-(4): recurrent across chunks, parallel
// inside a chunk.  For a chunk entered with state S (positions r = 0..C-1), G_r is the running
// sum of g inside the chunk (log of the cumulative decay gamma of eq. (3)), and unrolling eq. (1)
// over the chunk gives (the UT transform the pages defer to Kimi Linear):
//     A_kk[r,i] = sum_c k_rc k_ic exp(G_rc - G_ic)                 i < r   (strictly lower)
//     T = (I + Diag(beta) A_kk)^-1,  T_b = T Diag(beta),  K~ = K * exp(G)
//     V~ = T_b (V - K~ S)            (pseudo-values, the U - W S of §2.1.1)
//     A_qk[r,i] = sum_c q_rc k_ic exp(G_rc - G_ic)                 i <= r  (eq. (4): Tril keeps
//                                                                            the diagonal)
//     O = (Q * exp(G)) S + A_qk V~                                            (eq. (4))
//     S <- Diag(exp(G_last)) S + (K * exp(G_last - G))^T V~.
// The kernel never forms V~: with R = V - K~ S, M = A_qk T_b (C x C) and W = K_end^T T_b
// (dk x C, K_end = K * exp(G_last - G)), associativity gives
//     O = Q~ S + M R,      S <- Diag(gamma) S + W R.
// M and W depend on the chunk only, not on the state, so they are formed a pipeline stage ahead
// of the state step and shared by every value column.  This is also what keeps the rounding
// small: with keys bunched around one direction and beta near 1, V~ is a sequence of
// differences whose running sums (A_qk V~, K_end^T V~) cancel almost completely, while M and W
// are formed once from accurate factors and the state step multiplies well-scaled R.
//
// Decayed products inside a chunk use 16-token sub-tiles (§2.1.1, "lower-bounded decay"): for the
// row tile a with reference E = G at the end of tile a-1 (0 for a = 0),
//     A[r,i] = sum_c (x_rc exp(G_rc - E_c)) (k_ic exp(E_c - G_ic)),
// the row factor is <= 1 and the column factor is <= exp(80) on the diagonal tile (g >= -5 over
// 16 tokens), <= 1 off it: both representable in bf16, so every causal tile, diagonal included,
// is a dense MFMA product.
//
// Grid: one 512-thread workgroup per (sequence, head, 64-column slice of dv); the slices of one
// head go to the same XCD so their reads of q, k, g share L2.  Four producer waves (channel
// slices) and four consumer waves (16 value columns each), one of each per SIMD.  Iteration it
// has two intervals separated by workgroup barriers and works on four chunks at once:
//   interval 1  producers, chunk it: the decayed operands (prepared in the interval before)
//                   split into bf16 pairs, partial Gram tiles of A_kk and A_qk over the wave's
//                   32 key channels, the rows of Q~ and K~ and gamma (into one of three LDS
//                   buffers), K_end.
//                   Producer 1 also completes T_b of chunk it - 1 with its off-diagonal block
//                   T10 = -T11 N10 T00.
//               consumers, chunk it - 2: the state step on their 16 columns: R = V - K~ S,
//                   O = Q~ S + M R (written out), S <- gamma S + W R.
//   interval 2  producers: the rows of W over the wave's channels (and M) for chunk it - 1, from
//                   the K_end fragments they kept (with float32 inputs, the K_end fragments of
//                   chunk it are formed here rather than in interval 1); then the decay prefix
//                   (DPP scan over the 16 token lanes of a row) and the decayed operands of chunk
//                   it + 1 (kept in registers).
//               consumers, chunk it: the diagonal blocks T00 (consumer 0) and T11 (consumer 1) of
//                   the UT transform, beta N10 and the A_qk tiles (consumers 2, 3); every
//                   consumer sets the scale of its value path for chunk it - 1.
// A wave issues at most one instruction every four cycles, so each interval lasts about as long
// as its busiest wave's instruction stream: the producers' elementwise work (several hundred
// instructions per chunk) is split between the two intervals so that each producer interval
// stays within the consumers' (the state step in interval 1, the UT solve in interval 2).
// The state slice (dk x 16, fp32) stays in MFMA accumulators for the whole sequence.  Every
// hand-off buffer is read at least one barrier after it was written and written again only after
// its last read; buffers whose writer runs ahead of the reader are doubled.
//
// Precision: Gram tiles on bf16 hi + lo pairs (products hi*hi + lo*hi + hi*lo, fp32
// accumulation: the column factors reach exp(80), beyond float16); the UT solve on the fp32
// MFMA; M and W from float16 hi + lo pairs of A_qk, T_b and K_end; the state step on single
// float16 operands (Q~, K~, S, M, W, R).  To keep the value path inside float16's range each
// consumer wave carries its state as S 2^-e with a power-of-two exponent e chosen, per chunk,
// from the largest |S| and |V| alone (history-free, so a run resumed from a checkpoint repeats
// the same arithmetic); V is scaled by 2^-e and the outputs by 2^e.  The scale on q is applied to
// the outputs (everything is linear in q).
#include <atomic>
#include <type_traits>

#include "kda_device.h"
#include "kda_launch.h"

namespace kda {

constexpr int kC = 32;     // chunk length (two 16-token sub-tiles)
constexpr int kDVT = 64;   // value columns per workgroup
constexpr int kNW = 4;     // producer waves = consumer waves
constexpr int kNT = 128 * kNW;

template <int DK>
struct Layout {
    static constexpr int NCB = DK / 32;                     // 32-channel blocks = producer waves
    static constexpr int RB = DK + 8;                       // f16 [token][DK] row stride
    static constexpr int TB = kC + 8;                       // f16 [*][token] row stride
    static constexpr int SB = 16 * 20 + 16;                 // fp32 16x16 block stride (banks +16)
    static constexpr int GPB = NCB * 6 * 64 * 16;           // one set of partial Gram tiles
    static constexpr int QKB = 2 * kC * RB * 2 + DK * 4;    // Q~, K~ rows, gamma
    static constexpr int CPL = kC * TB * 2;                 // one C x C plane
    static constexpr int o_Gp = 0;                          // fp32 [NCB][6][64][4]
    static constexpr int o_beta = o_Gp + GPB;               // fp32 [2][C]
    static constexpr int o_QK = o_beta + 2 * kC * 4;        // [3] x {Q~ [C][RB], K~ [C][RB] f16, gamma [DK]}
    static constexpr int o_Tb = o_QK + 3 * QKB;             // [2] x T_b^T hi, lo [C][TB] f16
    static constexpr int o_Aq = o_Tb + 2 * 2 * CPL;         // [2] x A_qk hi, lo [C][TB] f16
    static constexpr int o_M = o_Aq + 2 * 2 * CPL;          // M [C][TB] f16
    static constexpr int o_W = o_M + CPL;                   // W [DK][TB] f16
    static constexpr int o_N = o_W + DK * TB * 2;           // fp32 2 blocks [16][20]: solve scratch
    static constexpr int o_Pub = o_N + 2 * SB * 4;          // fp32 3 blocks [16][20]: T00, T11, N10
    static constexpr int total = o_Pub + 3 * SB * 4;
    static constexpr int o_stop = total;                    // int [4]: consumer votes to stop early
    static constexpr int total_summ = total + 16;           // (first pass of a split in time)
    static_assert(total + 16 <= 160 * 1024, "LDS budget");
    static_assert(GPB >= 4 * (1024 + 1), "sequence ranking scratch fits the Gram region");
    static_assert(o_QK % 16 == 0 && QKB % 16 == 0 && o_Tb % 16 == 0 && o_W % 16 == 0 && o_N % 16 == 0,
                  "16-byte aligned regions");
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

template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL,
                                                                 0xF, 0xF, false));
}

// Maximum over the 64 lanes of a wave (wave-uniform result): quad swaps, half-row and row
// mirrors inside each 16-lane row, then the four rows.
__device__ __forceinline__ float wave_max(float x) {
    x = fmaxf(x, dpp_f<0xB1>(x));    // quad_perm [1,0,3,2]
    x = fmaxf(x, dpp_f<0x4E>(x));    // quad_perm [2,3,0,1]
    x = fmaxf(x, dpp_f<0x141>(x));   // row_half_mirror
    x = fmaxf(x, dpp_f<0x140>(x));   // row_mirror
    const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 0));
    const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 16));
    const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 32));
    const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 48));
    return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Two floats to two bf16 (round to nearest even) in one v_cvt_pk_bf16_f32, as a packed word.
__device__ __forceinline__ uint32_t cvt_pk(float a, float b) {
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}
// Two floats to two float16 (round to nearest even) in one v_cvt_pk_f16_f32.
__device__ __forceinline__ uint32_t cvt_pk_h(float a, float b) {
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, f16x2));
}

__device__ __forceinline__ bf16x8 to_bf16x8(const float* x) {
    const uint4 w{cvt_pk(x[0], x[1]), cvt_pk(x[2], x[3]), cvt_pk(x[4], x[5]), cvt_pk(x[6], x[7])};
    return __builtin_bit_cast(bf16x8, w);
}
__device__ __forceinline__ f16x8 to_f16x8(const float* x) {
    const uint4 w{cvt_pk_h(x[0], x[1]), cvt_pk_h(x[2], x[3]), cvt_pk_h(x[4], x[5]), cvt_pk_h(x[6], x[7])};
    return __builtin_bit_cast(f16x8, w);
}
__device__ __forceinline__ f16x4 to_f16x4(f32x4 a) {
    return __builtin_bit_cast(f16x4, uint2{cvt_pk_h(a[0], a[1]), cvt_pk_h(a[2], a[3])});
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

// The same split on float16 halves (22 significant bits for values of order one).
__device__ __forceinline__ void split_h4(f32x4 a, f16x4& hi, f16x4& lo) {
    hi = to_f16x4(a);
    const f32x4 r{a[0] - (float)hi[0], a[1] - (float)hi[1], a[2] - (float)hi[2], a[3] - (float)hi[3]};
    lo = to_f16x4(r);
}
__device__ __forceinline__ void split_h8(const float* x, f16x8& hi, f16x8& lo) {
    f16x4 h0, l0, h1, l1;
    split_h4(f32x4{x[0], x[1], x[2], x[3]}, h0, l0);
    split_h4(f32x4{x[4], x[5], x[6], x[7]}, h1, l1);
    hi = f16x8{h0[0], h0[1], h0[2], h0[3], h1[0], h1[1], h1[2], h1[3]};
    lo = f16x8{l0[0], l0[1], l0[2], l0[3], l1[0], l1[1], l1[2], l1[3]};
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
__device__ __forceinline__ f16x8 acc_pair_h(f32x4 a, f32x4 b) {
    const float x[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    return to_f16x8(x);
}

// 16x16x16 product on fp32 operands with the fp32 MFMA (four v_mfma_f32_16x16x4_f32): `xr` is
// the row form of X (lane (i16, g4) holds X[i16][4 g4 + e]), `yc` the column form of Y (lane
// (j16, g4) holds Y[4 g4 + e][j16]); MFMA e contracts over the positions 4 g4 + e, and the
// result is the column form of X Y.
__device__ __forceinline__ f32x4 mm16(f32x4 xr, f32x4 yc, f32x4 c) {
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(xr[0], yc[0], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(xr[1], yc[1], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(xr[2], yc[2], c, 0, 0, 0);
    return __builtin_amdgcn_mfma_f32_16x16x4f32(xr[3], yc[3], c, 0, 0, 0);
}

// hi*hi + lo*hi + hi*lo on float16 pairs
__device__ __forceinline__ f32x4 mma_h3(f16x8 ah, f16x8 al, f16x8 bh, f16x8 bl, f32x4 c) {
    c = mma_h(ah, bh, c);
    c = mma_h(al, bh, c);
    return mma_h(ah, bl, c);
}
__device__ __forceinline__ f32x4 mma3(bf16x8 ah, bf16x8 al, bf16x8 bh, bf16x8 bl, f32x4 c) {
    c = mma(ah, bh, c);
    c = mma(al, bh, c);
    return mma(ah, bl, c);
}

// Storage order of every 32-long contraction index in LDS: position pm(c) puts the elements one
// lane feeds to a 16x16x32 MFMA with the accumulator-compatible order (4 g4 + e for e < 4,
// 16 + 4 g4 + e - 4 for e >= 4) next to each other, so an operand is one 16-byte read.
__device__ __forceinline__ constexpr int pm(int c) {
    return (c & 16) ? ((c & 15) >> 2) * 8 + 4 + (c & 3) : (c >> 2) * 8 + (c & 3);
}

// One block of the grid -> (unit, column slice), slices of a unit on one XCD (the dispatcher
// places consecutive workgroups on consecutive XCDs, 8 of them).
// Workgroups are dispatched in order, round-robin over the 8 XCDs (block b to XCD b mod 8); the
// slices of one unit stay on one XCD so that their reads of q, k, g share its L2.  SUMM (the first
// pass of a split in time, nv value slices and nslices - nv transition slices per unit): all
// transition slices come first.  Their workgroups are short (a sequence's first and last
// segments have none; the others stop once the transition is zero).  As measured (start times of
// every workgroup of such a pass), an XCD dispatches in order and the k-th workgroup it receives
// goes to its shader engine k mod 4 (8 CUs each), waiting while that engine is full: placed after
// the long-running value slices, a short workgroup held back every later value slice until a long
// one ended (two rounds instead of one).
template <bool SUMM>
__device__ __forceinline__ void block_coords(int nslices, int nv, int& unit, int& slice) {
    const int b = blockIdx.x;
    const int xcd = b & 7, slot = b >> 3;
    if (SUMM && nslices > nv) {
        const int per_xcd = gridDim.x / (8 * nslices);   // units per XCD (the grid is a multiple)
        const int nt = nslices - nv;
        if (slot < per_xcd * nt) {
            unit = (slot / nt) * 8 + xcd;
            slice = nv + slot % nt;
        } else {
            const int s2 = slot - per_xcd * nt;
            unit = (s2 / nv) * 8 + xcd;
            slice = s2 % nv;
        }
        return;
    }
    unit = (slot / nslices) * 8 + xcd;
    slice = slot % nslices;
}

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
__device__ __forceinline__ void pin(f16x8& u) { asm volatile("" : "+v"(u)); }

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
// Every consumer wave of the workgroup voted to stop (read after the barrier that ends the
// interval in which the votes were written; a scalar result).
__device__ __forceinline__ bool stop_voted(const char* votes) {
    const int4 f = *reinterpret_cast<const int4*>(votes);
    return __builtin_amdgcn_readfirstlane(f.x & f.y & f.z & f.w) != 0;
}

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
// Wave p owns key channels [32 p, 32 p + 32) (none when p >= DK / 32).  Iteration it: the decayed
// operands and the partial Gram tiles of chunk it (interval 1); the rows of W over the wave's
// channels and a row tile of M for chunk it - 1, then Q~, K~, gamma and K_end of chunk it
// (interval 2).  TSL: a workgroup of transition columns (first pass of a split in time), which
// stops when its consumers vote that the transition is zero.
template <int DK, bool F32IN, bool GATE, bool TSL>
__device__ __forceinline__ void producer(const PrefillArgs& a, char* smem, int p, int lane,
                                         int64_t row0, int64_t len, int h) {
    using Lay = Layout<DK>;
    using IT = typename std::conditional<F32IN, float, bf16>::type;
    constexpr int RB = Lay::RB, TB = Lay::TB;
    auto hp = [&](int off) { return reinterpret_cast<f16*>(smem + off); };
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
    f16x8 Id[2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int e = 0; e < 8; ++e) Id[hh][e] = (f16)((8 * g4 + e == 16 * hh + i16) ? 1.f : 0.f);

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

    const int64_t nchunks = (len + kC - 1) / kC;

    // Decayed operands of the next chunk (float), held from their preparation in interval 2 to
    // interval 1, where they are split for its Gram tiles and turned into its rows and K_end.
    float Qs[2][8], Kr[2][8], Kd0[8], Kd1[8], Kc[8], F0[8], F1[8];
    // K_end of the chunk of this iteration (float, before its split)
    float Xe[2][8];

    // The part of chunk c that comes first: the decay prefix and the decayed operands; beta into
    // o_beta[c & 1] (wave 0); and the fetch of chunk c + 1.
    auto prep = [&](int64_t c) {
        const int64_t c0 = c * kC;
        float qv[2][8], kv[2][8], L[2][8];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            pq[t].pin_all();
            pk[t].pin_all();
            if constexpr (GATE) {
                pz[t].pin_all();
            } else {
                pin(pg[t][0]);
                pin(pg[t][1]);
            }
        }
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            pq[t].to_f32(qv[t]);
            pk[t].to_f32(kv[t]);
            if constexpr (GATE) {
                // decay map of the logits; tokens past the end read z = 0, whose map is not 0:
                // they must not decay
                const bool valid = 16 * t + i16 < len - c0;
                float zv[8];
                pz[t].to_f32(zv);
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    L[t][e] = valid ? kGminLog2e * __builtin_amdgcn_rcpf(1.f + fast_exp2(zsc * zv[e])) : 0.f;
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
                    f32p(Lay::o_beta)[(int)(c & 1) * kC + 16 * t + i16] =
                        F32IN ? __builtin_bit_cast(float, pb[t]) : __builtin_bit_cast(float, pb[t] << 16);
            }
        }
        // the raw registers are consumed: fetch the next chunk while this one is computed
        if (c + 1 < nchunks) prefetch(c0 + kC);

        float P[2][8], Pi[2][8];
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
        }
    };

    // The rest of chunk c before its products, from the operands above: the rows of Q~ and K~
    // and the chunk decay gamma into QK[c % 3], K_end.
    auto rows = [&](int64_t c) {
        char* qk = smem + Lay::o_QK + (int)(c % 3) * Lay::QKB;
        if (i16 == 0) {
#pragma unroll
            for (int e = 0; e < 8; ++e) reinterpret_cast<float*>(qk + 2 * kC * RB * 2)[ch0 + e] = F0[e] * F1[e];
        }
        // 8 channels of token 16 t + i16 into [token][pm(channel)] storage
        auto put_row = [&](char* base, int t, f16x8 v) {
            f16* d = reinterpret_cast<f16*>(base) + (16 * t + i16) * RB + 32 * p;
            st<f16x4>(d + pm(8 * g4), f16x4{v[0], v[1], v[2], v[3]});
            st<f16x4>(d + pm(8 * g4 + 4), f16x4{v[4], v[5], v[6], v[7]});
        };
        // Q~ = Q exp(G), K~ = K exp(G) from the chunk start; tile 1 carries the tile-0 decay
        {
            float x[8], y[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                x[e] = Qs[1][e] * F0[e];
                y[e] = Kr[1][e] * F0[e];
            }
            put_row(qk, 0, to_f16x8(Qs[0]));
            put_row(qk, 1, to_f16x8(x));
            put_row(qk + kC * RB * 2, 0, to_f16x8(Kr[0]));
            put_row(qk + kC * RB * 2, 1, to_f16x8(y));
        }
        // K_end = K exp(G_last - G)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            Xe[0][e] = Kc[e] * F1[e];
            Xe[1][e] = Kd1[e] * F1[e];
        }
    };

    // K_end of the last chunk as B operands (channel half hh, plane hi / lo), kept for one
    // iteration until M and W of that chunk are formed.  With bf16 inputs the fragments of a
    // chunk are formed in interval 1 (KeN), beside its products, and move to Ke after W; with
    // float32 inputs (more registers in flight) they are formed in interval 2 directly into Ke.
    constexpr bool KE_EARLY = !F32IN;
    f16x8 Ke[2][2], KeN[2][2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int pl = 0; pl < 2; ++pl) Ke[hh][pl] = KeN[hh][pl] = f16x8{};
    // K_end split and transposed through the identity: lane (channel i16 of half hh, g4) gets
    // tokens 16 t + 4 g4 + j of tile t, i.e. the B operand of a contraction over the chunk's
    // tokens in pm order
    auto ke_frags = [&](f16x8 (&K)[2][2]) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            f16x8 eh, el;
            split_h8(Xe[t], eh, el);
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const f16x4 vh = to_f16x4(mma_h(eh, Id[hh], zero4()));   // exact: f16 in
                const f16x4 vl = to_f16x4(mma_h(el, Id[hh], zero4()));
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    K[hh][0][4 * t + j] = vh[j];
                    K[hh][1][4 * t + j] = vl[j];
                }
            }
        }
    };

    if (intra && nchunks > 0) {
        prefetch(0);
        prep(0);
    }

    for (int64_t it = 0; it <= nchunks + 1; ++it) {
        const bool work = intra && it < nchunks;   // wave-uniform

        // ---- interval 1: partial Gram tiles of chunk it, from the operands prepared in the
        // previous interval 2, split here.  Transposed (column side as the A operand): the
        // accumulator of lane (row r = i16, g4) holds A[r][16 b + 4 g4 + j].  m: 0 qk00,
        // 1 qk11, 2 qk10, 3 kk00, 4 kk11, 5 kk10; every tile on split operands (3 products).
        // Then the rows, gamma and K_end of the chunk.
        if (work) {
            bf16x8 Qh[2], Ql[2], Krh[2], Krl[2], Kdh[2], Kdl[2], Kch, Kcl;
            split8(Qs[0], Qh[0], Ql[0]);
            split8(Qs[1], Qh[1], Ql[1]);
            split8(Kr[0], Krh[0], Krl[0]);
            split8(Kr[1], Krh[1], Krl[1]);
            split8(Kd0, Kdh[0], Kdl[0]);
            split8(Kd1, Kdh[1], Kdl[1]);
            split8(Kc, Kch, Kcl);
#pragma unroll
            for (int m = 0; m < 6; ++m) {
                const int ta = (m % 3 == 0) ? 0 : 1;
                const bf16x8 ch = (m % 3 == 2) ? Kch : Kdh[ta];
                const bf16x8 cl = (m % 3 == 2) ? Kcl : Kdl[ta];
                const bf16x8 rh = m < 3 ? Qh[ta] : Krh[ta];
                const bf16x8 rl = m < 3 ? Ql[ta] : Krl[ta];
                const f32x4 acc = mma3(ch, cl, rh, rl, zero4());
                st<f32x4>(smem + Lay::o_Gp + ((p * 6 + m) * 64 + lane) * 16, acc);
            }
            rows(it);
            if constexpr (KE_EARLY) ke_frags(KeN);
        }
        // ---- interval 1, producer wave 1: T10 = -T11 (beta N10) T00 of chunk it - 1 (column
        // form, times beta of its columns) completes T_b^T in the buffer of that chunk
        if (p == 1 && it >= 1 && it <= nchunks) {
            const int tb = (int)((it - 1) & 1);
            const float* pub = f32p(Lay::o_Pub);
            const f32x4 T00c = ld<f32x4>(pub + i16 * 20 + 4 * g4);
            const f32x4 T11r = ld<f32x4>(pub + Lay::SB + i16 * 20 + 4 * g4);
            const f32x4 N10r = ld<f32x4>(pub + 2 * Lay::SB + i16 * 20 + 4 * g4);
            const float b0 = f32p(Lay::o_beta)[tb * kC + i16];
            const f32x4 T10c = mm16(T11r, mm16(N10r, T00c, zero4()), zero4()) * (-b0);
            f16x4 hv, lv;
            split_h4(T10c, hv, lv);
            f16* t = hp(Lay::o_Tb + 2 * tb * Lay::CPL) + i16 * TB + pm(16 + 4 * g4);
            st<f16x4>(t, hv);
            st<f16x4>(t + Lay::CPL / 2, lv);
        }
        __syncthreads();

        // ---- interval 2: M and W of chunk it - 1 (formed from the K_end fragments held since
        // the previous interval 2 and T_b, A_qk from LDS), the K_end fragments of chunk it, then
        // the preparation of chunk it + 1.
        if (it >= 1 && it <= nchunks) {
            // W = K_end^T T_b and M = A_qk T_b on float16 pairs, formed transposed:
            // D[i][x] = sum_j T_b[j][i] X[x][j], whose accumulator (lane (column x, g4) holding
            // tokens i = 4 g4 + j) is the row fragment of W or M.
            const int tbuf = (int)((it - 1) & 1);
            f16x8 tA[2][2];   // rows of T_b^T for token tiles 0, 1, planes hi, lo
#pragma unroll
            for (int ai = 0; ai < 2; ++ai)
#pragma unroll
                for (int pl = 0; pl < 2; ++pl)
                    tA[ai][pl] = ld<f16x8>(hp(Lay::o_Tb + (2 * tbuf + pl) * Lay::CPL) + (16 * ai + i16) * TB + 8 * g4);
            if (intra) {
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    const f32x4 d0 = mma_h3(tA[0][0], tA[0][1], Ke[hh][0], Ke[hh][1], zero4());
                    const f32x4 d1 = mma_h3(tA[1][0], tA[1][1], Ke[hh][0], Ke[hh][1], zero4());
                    st<f16x8>(hp(Lay::o_W) + (32 * p + 16 * hh + i16) * TB + 8 * g4, acc_pair_h(d0, d1));
                }
            }
            // M: row tile 0 by producer wave 2, row tile 1 by producer wave 3
            const int b = p - (kNW - 2);
            if (b >= 0) {
                const f16x8 ah = ld<f16x8>(hp(Lay::o_Aq + (2 * tbuf) * Lay::CPL) + (16 * b + i16) * TB + 8 * g4);
                const f16x8 al = ld<f16x8>(hp(Lay::o_Aq + (2 * tbuf + 1) * Lay::CPL) + (16 * b + i16) * TB + 8 * g4);
                const f32x4 d0 = mma_h3(tA[0][0], tA[0][1], ah, al, zero4());
                const f32x4 d1 = b ? mma_h3(tA[1][0], tA[1][1], ah, al, zero4()) : zero4();
                st<f16x8>(hp(Lay::o_M) + (16 * b + i16) * TB + 8 * g4, acc_pair_h(d0, d1));
            }
        }
        if (work) {
            if constexpr (KE_EARLY) {
#pragma unroll
                for (int hh = 0; hh < 2; ++hh)
#pragma unroll
                    for (int pl = 0; pl < 2; ++pl) Ke[hh][pl] = KeN[hh][pl];
            } else {
                ke_frags(Ke);
            }
        }
        if (intra && it + 1 < nchunks) prep(it + 1);
        __syncthreads();
        if constexpr (TSL) {
            if (stop_voted(smem + Lay::o_stop)) {
                __builtin_amdgcn_s_waitcnt(0);   // the next chunk's loads are abandoned
                return;
            }
        }
    }
}

// ==================================== consumer waves =========================================
// Wave 4 + cw owns value columns [16 cw, 16 cw + 16) of the slice and its dk x 16 state slice.
// Iteration it: the state step of chunk it - 2 (interval 1); for chunk it the diagonal blocks of
// the UT transform (cw = 0, 1), beta N10 and the A_qk tiles (cw = 2, 3), and the scale of the
// value path for chunk it - 1 (interval 2).  SUMM: the first pass of a split in time (every
// segment writes its outputs, from S0 or 0); TSL: a workgroup of its transition columns, whose
// waves vote each iteration whether their columns are all zero and stop together.  full: false
// where a second pass runs a segment only over the chunks whose outputs depend on its entering
// state (the first pass wrote the rest and, for the last segment, S_T).
template <int DK, bool F32IN, bool OUT_F32, bool SUMM, bool TSL>
__device__ __forceinline__ void consumer(const PrefillArgs& a, char* smem, int cw, int lane,
                                         int64_t row0, int64_t len, int n, int h, int slice, int seg,
                                         int mode, int nseg_n, int64_t sbase, bool full, int jfrom) {
    using Lay = Layout<DK>;
    using IT = typename std::conditional<F32IN, float, bf16>::type;
    constexpr int KS = DK / 32;          // 32-channel contraction steps
    constexpr int CT = DK / 16;          // 16-channel tiles of the state
    constexpr int NCB = Lay::NCB;
    constexpr int RB = Lay::RB, TB = Lay::TB, SB = Lay::SB;
    auto hp = [&](int off) { return reinterpret_cast<f16*>(smem + off); };
    auto f32p = [&](int off) { return reinterpret_cast<float*>(smem + off); };
    const int i16 = lane & 15, g4 = lane >> 4;
    const int H = a.H;
    const size_t sv = (size_t)H * a.dv;        // token stride of v, o
    const int col0 = slice * kDVT + 16 * cw;   // first value column of this wave
    // segment summaries: columns >= dv carry the segment's transition (value 0); no outputs
    const bool tcols = mode == 1 && col0 >= a.dv;
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

    // ---- state slice in accumulators: Sacc[ct][j] = S[16 ct + 4 g4 + j][col0 + i16] 2^-esc
    f32x4 Sacc[CT];
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) Sacc[ct] = zero4();
    const int wcols = a.dv + DK;   // row length of a segment summary [dk][dv + dk]
    auto summary = [&](int j) {    // summary of segment j of this (sequence, head)
        return a.ws + ((size_t)(sbase + j) * H + h) * DK * wcols;
    };
    if (tcols) {
        // transition columns start as the identity
        const int c = col0 - a.dv + i16;
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
#pragma unroll
            for (int j = 0; j < 4; ++j) Sacc[ct][j] = (16 * ct + 4 * g4 + j == c) ? 1.f : 0.f;
    } else if (mode == 2 && seg > 0) {
        // entering state of segment seg: the state after segment jfrom (after segment 0, entered
        // with S0, or S~ of a segment whose transition is zero), carried through segments
        // jfrom + 1 .. seg-1 by S <- M_j S + S~_j (products on split bf16 operands)
        const float* W0 = summary(jfrom);
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
#pragma unroll
            for (int j = 0; j < 4; ++j) Sacc[ct][j] = W0[(size_t)(16 * ct + 4 * g4 + j) * wcols + col0 + i16];
        for (int jseg = jfrom + 1; jseg < seg; ++jseg) {
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
                    acc = mma3(mh, ml, Sh[s2], Sl[s2], acc);
                }
                Sacc[ct] = acc;
            }
        }
    } else if (a.S0 && !(mode == 1 && seg > 0)) {
        const float* S0 = a.S0 + ((size_t)n * H + h) * DK * a.dv;
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                Sacc[ct][j] = S0[(size_t)(16 * ct + 4 * g4 + j) * a.dv + col0 + i16];
    }
    // power-of-two scale of the value path: Sacc = S 2^-esc, V enters as V 2^-esc
    int esc = 0;
    float vsc = 1.f, osc = a.scale;

    // blocks that are zero for every chunk (both buffers): rows 16..31 x columns 0..15 of T_b^T
    // (T_b is lower triangular) and rows 0..15 x columns 16..31 of A_qk
    if (cw == 1) {
        const f16x4 z{(f16)0.f, (f16)0.f, (f16)0.f, (f16)0.f};
#pragma unroll
        for (int pl = 0; pl < 4; ++pl) {
            st<f16x4>(hp(Lay::o_Aq + pl * Lay::CPL) + i16 * TB + pm(16 + 4 * g4), z);
            st<f16x4>(hp(Lay::o_Tb + pl * Lay::CPL) + (16 + i16) * TB + pm(4 * g4), z);
        }
    }

    bf16x8 Id0;   // identity block: B operand selecting columns 0..15 of a 32-long step
#pragma unroll
    for (int e = 0; e < 8; ++e) Id0[e] = f2bf((8 * g4 + e == i16) ? 1.f : 0.f);

    // v fetched two chunks ahead: pa holds the chunk of the next state step, pb the one after;
    // the sets rotate after each step (named registers: an indexed pair would live in scratch)
    const IT* vhc = vh;   // rows of the next chunk to fetch
    OT* obc = ob;         // rows of the next chunk to write
    Raw8<F32IN> pa[2], pb[2];
    auto prefetch_v = [&](Raw8<F32IN>* pv, int64_t c0) {
        const uint32_t nv = (uint32_t)((len - c0) < kC ? (len - c0) : kC);
        const __amdgpu_buffer_rsrc_t rv = make_rsrc(vhc, nv * (uint32_t)(sv * sizeof(IT)));
        vhc += (size_t)kC * sv;
#pragma unroll
        for (int t = 0; t < 2; ++t) pv[t].load(rv, off_v[t]);
    };
    auto reduce = [&](int m) -> f32x4 {   // sum of the producers' partial Gram tiles
        const char* base = smem + Lay::o_Gp;
        f32x4 acc = ld<f32x4>(base + (m * 64 + lane) * 16);
#pragma unroll
        for (int w = 1; w < NCB; ++w) acc += ld<f32x4>(base + ((w * 6 + m) * 64 + lane) * 16);
        return acc;
    };
    auto frag = [&](int off, int row, int stride) -> f16x8 {   // 8 contraction positions of a row
        return ld<f16x8>(hp(off) + row * stride + 8 * g4);
    };

    const int64_t nchunks = (len + kC - 1) / kC;
    int64_t dep = nchunks;   // transition columns: chunks before they vanish
    if (nchunks > 0) prefetch_v(pa, 0);
    if (nchunks > 1) prefetch_v(pb, kC);

    for (int64_t it = 0; it <= nchunks + 1; ++it) {
        // ---- interval 1: state step of chunk it - 2 on this wave's 16 state columns.
        if (it >= 2) {
            const int64_t c = it - 2, c0 = c * kC;
            const char* qk = smem + Lay::o_QK + (int)(c % 3) * Lay::QKB;
            const uint32_t nvalid = (TSL || tcols) ? 0u : (uint32_t)((len - c0) < kC ? (len - c0) : kC);
            // output rows of the chunk: stores at or past row nvalid fall outside the resource
            // (transition columns write no outputs)
            const __amdgpu_buffer_rsrc_t ro = make_rsrc(obc, nvalid * (uint32_t)(sv * sizeof(OT)));
            obc += (size_t)kC * sv;
            // batch 1: rows of K~, Q~ and M
            f16x8 kt[2][KS], qr[2][KS], mr[2];
#pragma unroll
            for (int ta = 0; ta < 2; ++ta) {
#pragma unroll
                for (int s = 0; s < KS; ++s) {
                    kt[ta][s] = ld<f16x8>(reinterpret_cast<const f16*>(qk + kC * RB * 2) + (16 * ta + i16) * RB + 32 * s + 8 * g4);
                    qr[ta][s] = ld<f16x8>(reinterpret_cast<const f16*>(qk) + (16 * ta + i16) * RB + 32 * s + 8 * g4);
                }
                mr[ta] = frag(Lay::o_M, 16 * ta + i16, TB);
            }
            __builtin_amdgcn_sched_barrier(0);
            // V: token-per-lane -> column-per-lane through a product with the identity; the
            // accumulator of lane (column i16, g4) holds tokens 16 t + 4 g4 + j
            f32x4 Vf[2];
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                pa[t].pin_all();
                if constexpr (F32IN) {
                    float vv[8];
                    pa[t].to_f32(vv);
                    bf16x8 vh, vl;
                    split8(vv, vh, vl);
                    Vf[t] = mma(vl, Id0, mma(vh, Id0, zero4()));
                } else {
                    Vf[t] = mma(__builtin_bit_cast(bf16x8, pa[t].p[0]), Id0, zero4());   // bf16 as stored
                }
            }
            // rotate: the next chunk's v (fetched one step ago) moves up, the one after is fetched
#pragma unroll
            for (int t = 0; t < 2; ++t) pa[t] = pb[t];
            if (c + 2 < nchunks) prefetch_v(pb, (c + 2) * kC);
            // state as B operand: contraction index (32-channel step s, g4, e) ->
            // channel 32 s + 4 g4 + e (e < 4), 32 s + 16 + 4 g4 + (e - 4) (e >= 4)
            f16x8 Sh[KS];
#pragma unroll
            for (int s = 0; s < KS; ++s) Sh[s] = acc_pair_h(Sacc[2 * s], Sacc[2 * s + 1]);
#pragma unroll
            for (int ta = 0; ta < 2; ++ta) {
                pin(mr[ta]);
#pragma unroll
                for (int s = 0; s < KS; ++s) {
                    pin(kt[ta][s]);
                    pin(qr[ta][s]);
                }
            }
            // K~ S and Q~ S, four independent chains
            f32x4 KSa[2] = {zero4(), zero4()}, QSa[2] = {zero4(), zero4()};
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                KSa[0] = mma_h(kt[0][s], Sh[s], KSa[0]);
                KSa[1] = mma_h(kt[1][s], Sh[s], KSa[1]);
                QSa[0] = mma_h(qr[0][s], Sh[s], QSa[0]);
                QSa[1] = mma_h(qr[1][s], Sh[s], QSa[1]);
            }
            // batch 2, in two halves (registers): rows of W and the chunk decay gamma for state
            // tiles [0, CT/2), then [CT/2, CT)
            constexpr int CH = CT / 2;
            f16x8 wr[CH];
            f32x4 gm[CH];
            auto load_half = [&](int c0h) {
#pragma unroll
                for (int cc = 0; cc < CH; ++cc) {
                    wr[cc] = frag(Lay::o_W, 16 * (c0h + cc) + i16, TB);
                    gm[cc] = ld<f32x4>(reinterpret_cast<const float*>(qk + 2 * kC * RB * 2) + 16 * (c0h + cc) + 4 * g4);
                }
            };
            load_half(0);
            __builtin_amdgcn_sched_barrier(0);
            // R = V 2^-esc - K~ S, as the B operand of M R and W R
            f32x4 R[2];
#pragma unroll
            for (int ta = 0; ta < 2; ++ta)
#pragma unroll
                for (int j = 0; j < 4; ++j) R[ta][j] = __builtin_fmaf(Vf[ta][j], vsc, -KSa[ta][j]);
            const f16x8 Rh = acc_pair_h(R[0], R[1]);
            // outputs O = Q~ S + M R
#pragma unroll
            for (int ta = 0; ta < 2; ++ta) {
                const f32x4 acc = mma_h(mr[ta], Rh, QSa[ta]);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    if constexpr (OUT_F32)
                        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, osc * acc[j]), ro,
                                                              off_o[ta][j], 0, 0);
                    else
                        __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(uint16_t, f2bf(osc * acc[j])), ro,
                                                              off_o[ta][j], 0, 0);
                }
            }
            // state: S <- Diag(gamma_last) S + W R on tiles [c0h, c0h + CH)
            auto update_half = [&](int c0h) {
#pragma unroll
                for (int cc = 0; cc < CH; ++cc) {
                    pin(wr[cc]);
                    pin(gm[cc]);
                }
#pragma unroll
                for (int cc = 0; cc < CH; ++cc) Sacc[c0h + cc] = mma_h(wr[cc], Rh, Sacc[c0h + cc] * gm[cc]);
            };
            update_half(0);
            load_half(CH);
            update_half(CH);
            // state checkpoint after every ckpt_every full chunks (prefix states for reuse)
            const int64_t done = c + 1;   // chunks folded into the state
            if (a.ckpt && done % a.ckpt_every == 0 && done * kC <= len) {
                const int64_t j = done / a.ckpt_every - 1;
                if (j < a.ckpt_cap) {
                    float* Cp = a.ckpt + (((size_t)n * H + h) * a.ckpt_cap + j) * DK * a.dv;
                    // 32-bit lane offset, opaque so that the 32 store addresses are formed here
                    // rather than hoisted out of the chunk loop into registers
                    int lo = 4 * g4 * a.dv + col0 + i16;
                    asm volatile("" : "+v"(lo));
                    const float un = __builtin_ldexpf(1.f, esc);
#pragma unroll
                    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                        for (int jj = 0; jj < 4; ++jj) Cp[lo + (16 * ct + jj) * a.dv] = Sacc[ct][jj] * un;
                }
            }
        }
        __syncthreads();

        // ---- interval 2, chunk it: diagonal blocks of the UT transform (cw = 0: T00, cw = 1:
        // T11), beta N10 and the A_qk tiles (cw = 2, 3), from the Gram tiles of interval 1
        if (it < nchunks) {
            const int tb = (int)(it & 1);
            const float* bet = f32p(Lay::o_beta) + tb * kC;
            float* pub = f32p(Lay::o_Pub);   // [0] T00 (column form rows), [1] T11 (rows), [2] beta N10 (rows)
            if (cw < 2) {
                // T_qq = (I + N_qq)^-1 for the diagonal 16x16 block q of N = Diag(beta) A_kk
                // (strictly lower) by block elimination: B = L0 + L1 + L2 (L0: inside the 4x4
                // diagonal blocks; L1: the 4x4 blocks just below them within each 8x8 diagonal
                // block; L2: the lower-left 8x8 block),
                //     D = (I + L0)^-1 (closed form),  E = D - D L1 D,  X = E - E L2 E,
                // each product filling blocks that are zero in the previous level (no
                // cancellation).  Products on the fp32 MFMA.  Forms: row form of M in lane
                // (i16, g4) = M[i16][4 g4 + j], column form = M[4 g4 + j][i16]; mm16(row form of
                // X, column form of Y) is the column form of X Y; a row form is read back from LDS
                // where a column form was stored.
                const int q = cw;
                const float bq = bet[16 * q + i16];
                // an opaque lane index: keeps the compiler from hoisting lane-constant masks out
                // of the chunk loop into registers held across it
                int lid = i16;
                asm volatile("" : "+v"(lid));
                const int rb = lid >> 2;                       // 4-row block of this lane's row / column
                f32x4 Nr = reduce(3 + q);
#pragma unroll
                for (int j = 0; j < 4; ++j) Nr[j] = 4 * g4 + j < lid ? Nr[j] * bq : 0.f;
                float* Nb = f32p(Lay::o_N) + q * SB;
                st<f32x4>(Nb + i16 * 20 + 4 * g4, Nr);
                wave_lds_order();
                // rows 1..3 of the 4x4 diagonal block g4 (strictly lower entries)
                f32x4 n1 = ld<f32x4>(Nb + (4 * g4 + 1) * 20 + 4 * g4);
                f32x4 n2 = ld<f32x4>(Nb + (4 * g4 + 2) * 20 + 4 * g4);
                f32x4 n3 = ld<f32x4>(Nb + (4 * g4 + 3) * 20 + 4 * g4);
                pin(n1);   // whole rows in separate registers, read together
                pin(n2);
                pin(n3);
                wave_lds_order();
                const bool on_diag = g4 == rb;                 // this lane's 4-block holds D entries
                const int kk = lid & 3;
                const float d0 = kk == 0 ? 1.f : 0.f, d1 = kk == 1 ? 1.f : 0.f;
                const float d2 = kk == 2 ? 1.f : 0.f, d3 = kk == 3 ? 1.f : 0.f;
                // whole-vector masks of L1 and L2 in row form (row i16, columns 4 g4 + j)
                const bool l1r = (rb == 1 || rb == 3) && g4 == rb - 1;
                const bool l2r = lid >= 8 && g4 < 2;
                auto mask = [](f32x4 v, bool keep) { return keep ? v : zero4(); };
                // D = (I + L0)^-1: column kk (column form) and row kk (row form) of the inverse of
                // the unit lower 4x4 block g4
                const float x1 = d1 - n1[0] * d0;
                const float x2 = d2 - n2[0] * d0 - n2[1] * x1;
                const float x3 = d3 - n3[0] * d0 - n3[1] * x1 - n3[2] * x2;
                const float y2 = d2 - d3 * n3[2];
                const float y1 = d1 - y2 * n2[1] - d3 * n3[1];
                const float y0 = d0 - y1 * n1[0] - y2 * n2[0] - d3 * n3[0];
                const f32x4 Dc = on_diag ? f32x4{d0, x1, x2, x3} : zero4();
                const f32x4 Dr = on_diag ? f32x4{y0, y1, y2, d3} : zero4();
                // E = D - D L1 D (column form); its row form through LDS (Nb is free again)
                const f32x4 Ec = Dc - mm16(Dr, mm16(mask(Nr, l1r), Dc, zero4()), zero4());
#pragma unroll
                for (int j = 0; j < 4; ++j) Nb[(4 * g4 + j) * 20 + i16] = Ec[j];
                wave_lds_order();
                f32x4 Er = ld<f32x4>(Nb + i16 * 20 + 4 * g4);
                pin(Er);
                // X = E - E L2 E, column form
                const f32x4 Xc = Ec - mm16(Er, mm16(mask(Nr, l2r), Ec, zero4()), zero4());
                // T_b^T [i][pm(j)] = T[j][i] beta_i (float16 hi, lo) for this block: lane
                // (column i16, g4) holds T[16 q + 4 g4 + j][16 q + i16]
                f16x4 hv, lv;
                split_h4(Xc * bq, hv, lv);
                f16* t = hp(Lay::o_Tb + 2 * tb * Lay::CPL) + (16 * q + i16) * TB + pm(16 * q + 4 * g4);
                st<f16x4>(t, hv);
                st<f16x4>(t + Lay::CPL / 2, lv);
                // for T10: T00 in column form, T11 in row form
                if (q == 0) {
                    st<f32x4>(pub + i16 * 20 + 4 * g4, Xc);
                } else {
#pragma unroll
                    for (int j = 0; j < 4; ++j) pub[SB + (4 * g4 + j) * 20 + i16] = Xc[j];
                }
            } else {
                // A_qk tiles (masked) -> float16 hi, lo [row][pm(col)]; m: 0 rows 0-15 x cols
                // 0-15, 1: 16-31 x 16-31, 2: 16-31 x 0-15.  cw = 2 also forms beta N10 (row form).
                auto aqk_tile = [&](int m) {
                    f32x4 acc = reduce(m);
                    const int ta = (m == 0) ? 0 : 1, tbb = (m == 1) ? 1 : 0;
                    const int r = 16 * ta + i16;
#pragma unroll
                    for (int j = 0; j < 4; ++j) acc[j] = (16 * tbb + 4 * g4 + j <= r) ? acc[j] : 0.f;
                    f16x4 hv, lv;
                    split_h4(acc, hv, lv);
                    f16* ad = hp(Lay::o_Aq + 2 * tb * Lay::CPL) + r * TB + pm(16 * tbb + 4 * g4);
                    st<f16x4>(ad, hv);
                    st<f16x4>(ad + Lay::CPL / 2, lv);
                };
                if (cw == 2) {
                    const f32x4 N10r = reduce(5) * bet[16 + i16];
                    st<f32x4>(pub + 2 * SB + i16 * 20 + 4 * g4, N10r);
                    aqk_tile(2);
                } else {
                    aqk_tile(0);
                    aqk_tile(1);
                }
            }
        }
        // ---- interval 2: scale of the value path for the state step of chunk it - 1, from the
        // largest |S| and |V| only, in steps of 2^4, so that the scaled values lie in [2^6, 2^10)
        if (it >= 1 && it <= nchunks) {
            float mV = 0.f;   // pa holds v of chunk it - 1
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                pa[t].pin_all();
                float vv[8];
                pa[t].to_f32(vv);
                mV = fmaxf(mV, fmaxf(fmaxf(fmaxf(fabsf(vv[0]), fabsf(vv[1])), fmaxf(fabsf(vv[2]), fabsf(vv[3]))),
                                     fmaxf(fmaxf(fabsf(vv[4]), fabsf(vv[5])), fmaxf(fabsf(vv[6]), fabsf(vv[7])))));
            }
            float mS0 = 0.f, mS1 = 0.f;
#pragma unroll
            for (int ct = 0; ct < CT; ct += 2) {
                mS0 = fmaxf(fmaxf(mS0, fabsf(Sacc[ct][0])), fabsf(Sacc[ct][1]));
                mS0 = fmaxf(fmaxf(mS0, fabsf(Sacc[ct][2])), fabsf(Sacc[ct][3]));
                mS1 = fmaxf(fmaxf(mS1, fabsf(Sacc[ct + 1][0])), fabsf(Sacc[ct + 1][1]));
                mS1 = fmaxf(fmaxf(mS1, fabsf(Sacc[ct + 1][2])), fabsf(Sacc[ct + 1][3]));
            }
            const float m = wave_max(fmaxf(mV * vsc, fmaxf(mS0, mS1)));
            if (m > 0.f && m < 3.0e38f) {
                // m in [2^(ex-1), 2^ex) in scaled units; the unscaled exponent is ex + esc
                const int ex = __builtin_amdgcn_frexp_expf(m) + esc;
                int want = ((ex - 7) >> 2) << 2;                 // floor to a multiple of 4
                want = want < -120 ? -120 : (want > 120 ? 120 : want);
                if (want != esc) {
                    const float f = __builtin_ldexpf(1.f, esc - want);
#pragma unroll
                    for (int ct = 0; ct < CT; ++ct) Sacc[ct] *= f;
                    esc = want;
                    vsc = __builtin_ldexpf(1.f, -esc);
                    osc = a.scale * __builtin_ldexpf(1.f, esc);
                }
            }
        }
        if (TSL) {
            // transition columns: V is 0, so once every entry is exactly zero every later step
            // leaves them zero (R = 0 - K~ 0, S <- gamma 0 + W 0).  Entries that small in value
            // need not reach zero: with the scale at its floor (2^-120) their float16 operands sit
            // on the subnormal grid, where the rounded update can hold them near 2^-24 instead of
            // letting them decay.  So below 2^-20 there (2^-140 of the identity the transition
            // starts from) they count as zero too.  This wave's vote to stop (NaN never votes).
            uint32_t nz = 0;
            bool tiny = true;
#pragma unroll
            for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    nz |= __builtin_bit_cast(uint32_t, Sacc[ct][j]) & 0x7fffffffu;
                    tiny = tiny && fabsf(Sacc[ct][j]) < 0x1p-20f;
                }
            const bool zero = __builtin_amdgcn_ballot_w64(nz != 0) == 0 ||
                              (esc <= -120 && __builtin_amdgcn_ballot_w64(!tiny) == 0);
            if (lane == 0) reinterpret_cast<int*>(smem + Lay::o_stop)[cw] = zero ? 1 : 0;
        }
        __syncthreads();
        if constexpr (TSL) {
            if (stop_voted(smem + Lay::o_stop)) {
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) Sacc[ct] = zero4();   // +0
                // the state after chunks 0 .. it - 2 is zero: from chunk it - 1 on, the outputs of
                // the segment do not depend on the state it is entered with
                dep = it - 1 < nchunks ? it - 1 : nchunks;
                break;
            }
        }
    }

    const float un = __builtin_ldexpf(1.f, esc);
    if (mode == 1 && seg < nseg_n - 1) {
        float* Wsum = summary(seg);
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
#pragma unroll
            for (int j = 0; j < 4; ++j) Wsum[(size_t)(16 * ct + 4 * g4 + j) * wcols + col0 + i16] = Sacc[ct][j] * un;
    }
    if (tcols) {
        // chunks of this segment whose outputs depend on its entering state (all of them unless
        // the transition reached zero), per 64-column transition slice
        if (cw == 0 && lane == 0)
            a.stops[((size_t)(sbase + seg - 1) * H + h) * (DK / kDVT) + (col0 - a.dv) / kDVT] = (int32_t)dep;
    } else if (a.ST && full && (mode == 0 || seg == nseg_n - 1)) {
        float* ST = a.ST + ((size_t)n * H + h) * DK * a.dv;
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                ST[(size_t)(16 * ct + 4 * g4 + j) * a.dv + col0 + i16] = Sacc[ct][j] * un;
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

// Both roles run the same number of iterations (chunks + 2) with two barriers each.  PASS: 0 a
// whole-sequence run, 1 the first pass of a split in time (every segment with its outputs, the
// later ones entered with 0; segment summaries; transition workgroups may stop early), 2 its
// second pass (the later segments again from their true entering state, over the chunks whose
// outputs depend on it); a.mode equals PASS.  RANK: packed sequences (at
// most kRankMax) in longest-first order.  Separate instantiations, so that the plain kernel
// carries none of the split's code.
template <int DK, bool F32IN, bool OUT_F32, bool GATE, bool RANK, int PASS>
__global__ __launch_bounds__(kNT) void prefill_kernel(PrefillArgs a) {
    extern __shared__ __attribute__((aligned(16))) char smem[];
    constexpr bool SUMM = PASS == 1;
    const int nslices = (SUMM ? a.dv + a.dk : a.dv) / kDVT;
    const int nseg = PASS == 0 ? 1 : a.nseg;   // segments per sequence in the grid (at most)
    int unit, slice;
    block_coords<SUMM>(nslices, a.dv / kDVT, unit, slice);
    int n, seg, mode = PASS, nseg_n = 1;
    int64_t sbase = 0, row0, len;
    int64_t seqlen = 0, segL = 0;   // split runs: the sequence's tokens and its segment length
    const int h = unit % a.H;
    if (PASS != 0 && a.plan) {
        // a planned split: the workgroup's item of this pass's list
        const PlanLayout lay{a.N, a.plan_smax};
        const int item = unit / a.H;
        if (item >= a.plan[PASS]) return;
        const int32_t* it = a.plan + (SUMM ? lay.items1() : lay.items2()) + 2 * (int64_t)item;
        n = it[0];
        seg = it[1];
        nseg_n = a.plan[lay.segs() + n];
        sbase = a.plan[lay.first() + n];
        const int64_t L = a.plan[lay.seglen() + n];
        if (nseg_n <= 1) {
            // a sequence the plan leaves whole runs completely, in either pass
            if (SUMM && slice * kDVT >= a.dv) return;
            mode = 0;
        } else if (SUMM && seg == 0 && slice * kDVT >= a.dv) {
            return;   // the first segment is entered with S0: no transition columns
        }
        KDA_POISON(smem, (SUMM ? Layout<DK>::total_summ : Layout<DK>::total));
        KDA_POISON_DONE();
        seq_bounds(a, n, row0, len);
        seqlen = len;
        segL = L;
        if (mode != 0) {   // this segment's tokens
            const int64_t lo = (int64_t)seg * L;
            const int64_t hi = lo + L < len ? lo + L : len;
            row0 += lo;
            len = hi > lo ? hi - lo : 0;
        }
    } else {
        if (unit >= a.N * a.H * nseg) return;
        seg = (unit / a.H) % nseg;
        const int rank = unit / (a.H * nseg);
        // every sequence has nseg segments, each run in pass 1 with the transition columns of all
        // but the first
        if (SUMM && seg == 0 && slice * kDVT >= a.dv) return;   // entered with S0: no transition
        if (PASS == 2 && seg == 0) return;   // the first segment wrote its outputs in pass 1
        KDA_POISON(smem, (SUMM ? Layout<DK>::total_summ : Layout<DK>::total));
        KDA_POISON_DONE();
        n = rank;
        if constexpr (RANK) n = seq_of_rank(a, rank, smem);
        seq_bounds(a, n, row0, len);
        if (PASS != 0) {
            // nseg segments of ceil(len / nseg) tokens rounded up to whole chunks
            nseg_n = nseg;
            sbase = (int64_t)n * (nseg - 1);
            int64_t L = ((len + nseg - 1) / nseg + kC - 1) / kC * kC;
            if (L == 0) L = kC;
            seqlen = len;
            segL = L;
            const int64_t lo = (int64_t)seg * L;
            const int64_t hi = lo + L < len ? lo + L : len;
            row0 += lo;
            len = hi > lo ? hi - lo : 0;
        }
    }
    // Second pass: eq. (17) gives the state of segment seg at each chunk as M S_in + S~, M the
    // transition from the segment's start.  Once M has vanished (both of its 64-column slices
    // stopped in the first pass: zero, or below 2^-140 of the identity), the outputs from there
    // on are those of the first pass, run from 0: only the chunks before it run again.
    bool full = true;
    // (a deferred plan's last segment has no transition: it runs whole)
    if (PASS == 2 && mode == 2 && !(a.plan && !a.plan[3] && seg == nseg_n - 1)) {
        const int32_t* st = a.stops + ((size_t)(sbase + seg - 1) * a.H + h) * (DK / kDVT);
        int64_t dep = 0;
        for (int ts = 0; ts < DK / kDVT; ++ts) dep = dep > st[ts] ? dep : st[ts];
        if (dep * kC < len) {
            len = dep * kC;
            full = false;
        }
    }
    // The entering state S_in(seg) = M_{seg-1} S_in(seg-1) + S~_{seg-1} is rebuilt from the last
    // earlier segment whose transition vanished (its chunks before that are fewer than its
    // chunks): the state after it is its S~, and the products with the earlier ones are +-0.
    int jfrom = 0;
    if (PASS == 2 && mode == 2) {
        for (int jj = seg - 1; jj >= 1; --jj) {
            const int64_t lo = (int64_t)jj * segL, rest = seqlen - lo;
            const int64_t chunks = ((rest < segL ? (rest > 0 ? rest : 0) : segL) + kC - 1) / kC;
            const int32_t* st = a.stops + ((size_t)(sbase + jj - 1) * a.H + h) * (DK / kDVT);
            int64_t dep = 0;
            for (int ts = 0; ts < DK / kDVT; ++ts) dep = dep > st[ts] ? dep : st[ts];
            if (dep < chunks) {
                jfrom = jj;
                break;
            }
        }
    }
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform (scalar)
    // a workgroup of transition columns (segment summaries) may stop once they are all zero
    const bool tslice = SUMM && mode == 1 && slice * kDVT >= a.dv;
    if constexpr (SUMM) {
        if (tslice) {   // its own code: the vote and the stop stay out of the value workgroups
            if (wave < kNW) producer<DK, F32IN, GATE, true>(a, smem, wave, lane, row0, len, h);
            else consumer<DK, F32IN, OUT_F32, true, true>(a, smem, wave - kNW, lane, row0, len, n, h, slice, seg,
                                                           mode, nseg_n, sbase, full, jfrom);
            return;
        }
    }
    if (wave < kNW) producer<DK, F32IN, GATE, false>(a, smem, wave, lane, row0, len, h);
    else consumer<DK, F32IN, OUT_F32, SUMM, false>(a, smem, wave - kNW, lane, row0, len, n, h, slice, seg, mode,
                                                   nseg_n, sbase, full, jfrom);
}

template <int DK, bool F32IN, bool OUT_F32, bool GATE, bool RANK, int PASS>
static hipError_t launch_one(const PrefillArgs& a) {
    using Lay = Layout<DK>;
    constexpr bool SUMM = PASS == 1;
    auto kern = prefill_kernel<DK, F32IN, OUT_F32, GATE, RANK, PASS>;
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
                                SUMM ? Lay::total_summ : Lay::total);
        if (e != hipSuccess) return e;
        attr_set.fetch_or(bit, std::memory_order_relaxed);
    }
    const int nslices = (a.mode == 1 ? a.dv + a.dk : a.dv) / kDVT;
    const int64_t units = a.plan ? (int64_t)a.plan_items * a.H : (int64_t)a.N * a.H * (a.mode == 0 ? 1 : a.nseg);
    const int64_t blocks = ((units + 7) / 8) * 8 * nslices;
    if (blocks == 0) return hipSuccess;
    hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(kNT), SUMM ? Lay::total_summ : Lay::total, a.stream, a);
    return hipGetLastError();
}

template <int DK, bool F32IN, bool OUT_F32, bool GATE>
static hipError_t launch_prefill(const PrefillArgs& a) {
    const bool rank = a.cu && !a.plan && a.N > 1 && a.N <= kRankMax;
    if (a.mode == 1 || a.mode == 2) {
        // the passes of a split in time
        if (a.mode == 1)
            return rank ? launch_one<DK, F32IN, OUT_F32, GATE, true, 1>(a)
                        : launch_one<DK, F32IN, OUT_F32, GATE, false, 1>(a);
        return rank ? launch_one<DK, F32IN, OUT_F32, GATE, true, 2>(a)
                    : launch_one<DK, F32IN, OUT_F32, GATE, false, 2>(a);
    }
    if (rank) return launch_one<DK, F32IN, OUT_F32, GATE, true, 0>(a);
    return launch_one<DK, F32IN, OUT_F32, GATE, false, 0>(a);
}

template <bool GATE>
static hipError_t dispatch_prefill(const PrefillArgs& a) {
    if (a.dk == 128) {
        if (a.in_f32)
            return a.out_f32 ? launch_prefill<128, true, true, GATE>(a) : launch_prefill<128, true, false, GATE>(a);
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

// The best candidate of one layout: its segment length (0: none qualifies) and its score.
// price(L, eager, c) fills c with the batch's cost for segment length L.  A candidate must be
// expected to beat the whole schedule by kSplitGain and, should no transition vanish after all,
// take at most kSplitRisk times as long as it; the lowest expected time wins, near ties going to
// the lower worst case.
constexpr double kSplitRisk = 1.5, kSplitTie = 0.05;
template <class Price>
__host__ __device__ inline int64_t split_best(Price&& price, int64_t longest, const SplitLimits& lim,
                                              double base, int H, int slots, bool eager, double& best) {
    best = 0.0;
    int64_t bestL = 0;
    for (int p = 2; p <= lim.Pmax; ++p) {
        const int64_t L = split_candidate(longest, p);
        if (L < lim.Lmin) break;
        SplitCost c;
        price(L, eager, c);
        if (c.summaries > lim.Smax) continue;
        const double m = split_makespan(c, L, H, slots, false), f = split_makespan(c, L, H, slots, true);
        const double score = m + kSplitTie * f;
        if (m < base * kSplitGain && f <= base * kSplitRisk && (bestL == 0 || score < best)) {
            best = score;
            bestL = L;
        }
    }
    return bestL;
}

bool split_may_pay(int32_t N, int64_t T, int32_t H, int32_t dk, int32_t dv, int slots) {
    const SplitLimits lim = split_limits(N, (int64_t)N * T, H, dv, slots);
    const int nsl = dv / kDVT, nslt = (dv + dk) / kDVT;
    if (lim.Smax <= 0 || N < 1 || T <= 0) return false;
    auto price = [&](int64_t L, bool eager, SplitCost& c) {
        int P;
        int64_t Ls;
        split_of(T, L, lim.Pmax, P, Ls);
        split_add(c, T, P, Ls, L, nsl, nslt, eager, kTransSteps);
        split_times(c, N);
    };
    SplitCost whole;
    price(0, false, whole);
    const double base = split_makespan(whole, 0, H, slots, false);
    double score;
    return split_best(price, T, lim, base, H, slots, true, score) > 0 ||
           split_best(price, T, lim, base, H, slots, false, score) > 0;
}

// Decay probe: workgroup (sample j, channel group) sums g over the 32 tokens that start at
// j / kProbeChunks of the batch (rounded down to a multiple of 32) for its channels and records
// the smallest decay among them (nats; 0 for a NaN sum, +inf for an empty sample).  With logits
// z instead of g, g is formed by the map of eq. (5) first.
__global__ __launch_bounds__(256) void probe_kernel(PrefillArgs a, int32_t* __restrict__ probe, int64_t tokens) {
    __shared__ float red[256];
    const int j = blockIdx.x / kProbeGroups, grp = blockIdx.x % kProbeGroups;
    const int64_t nch = (int64_t)a.H * a.dk;
    const int64_t t0 = tokens * j / kProbeChunks / 32 * 32, t1 = t0 + 32 < tokens ? t0 + 32 : tokens;
    float dmin = __builtin_inff();
    for (int64_t c = (int64_t)grp * 256 + threadIdx.x; c < nch && t0 < t1; c += 256 * kProbeGroups) {
        float x[32];
        if (a.z) {
            const float es = __expf(a.A_log[c / a.dk]);
#pragma unroll
            for (int i = 0; i < 32; ++i) {
                const int64_t idx = (t0 + i) * nch + c;
                const float zv = t0 + i >= t1 ? 0.f
                                 : a.in_f32 ? static_cast<const float*>(a.z)[idx]
                                            : __builtin_bit_cast(float, (uint32_t)static_cast<const uint16_t*>(a.z)[idx] << 16);
                x[i] = t0 + i < t1 ? kGmin / (1.f + __expf(-es * zv)) : 0.f;
            }
        } else {
#pragma unroll
            for (int i = 0; i < 32; ++i) x[i] = t0 + i < t1 ? a.g[(t0 + i) * nch + c] : 0.f;   // loads in flight together
        }
        float sum = 0.f;
#pragma unroll
        for (int i = 0; i < 32; ++i) sum += x[i];
        const float d = -sum;
        dmin = d >= 0.f ? (d < dmin ? d : dmin) : 0.f;   // NaN or growth: no decay
    }
    red[threadIdx.x] = dmin;
    __syncthreads();
    for (int k = 128; k > 0; k >>= 1) {
        if (threadIdx.x < k) red[threadIdx.x] = red[threadIdx.x + k] < red[threadIdx.x] ? red[threadIdx.x + k] : red[threadIdx.x];
        __syncthreads();
    }
    if (threadIdx.x == 0) probe[blockIdx.x] = __builtin_bit_cast(int32_t, red[0]);
}

// One workgroup of 256 threads estimates from the probe how many chunks a transition runs
// before it vanishes, prices every candidate segment length (the longest sequence cut into
// 2 .. Pmax pieces) in both layouts with the model above and writes the plan of the best.
__global__ __launch_bounds__(256) void plan_kernel(PrefillArgs a, int32_t* __restrict__ plan, int slots,
                                                   SplitLimits lim) {
    const int t = threadIdx.x, wave = t >> 6, lane = t & 63;
    const int N = a.N, H = a.H, nsl = a.dv / kDVT, nslt = (a.dv + a.dk) / kDVT;
    const PlanLayout lay{N, (int32_t)lim.Smax};
    // the lengths, staged once in LDS (up to kRankMax sequences; read from memory beyond)
    __shared__ int32_t order[kRankMax];
    __shared__ int64_t lens[kRankMax];
    const bool ranked = N <= kRankMax;
    if (ranked) {
        for (int n = t; n < N; n += 256) {
            int64_t row0, len;
            seq_bounds(a, n, row0, len);
            lens[n] = len;
        }
    }
    // the weakest decay per chunk the probe saw: transitions fall below 2^-140 of the identity
    // within about kZeroNats / d chunks (the delta rule's own contraction only shortens that)
    __shared__ float pd[kProbeBlocks];
    if (t < kProbeBlocks) pd[t] = __builtin_bit_cast(float, plan[lay.probe() + t]);
    __syncthreads();
    float dmin = __builtin_inff();
    for (int i = 0; i < kProbeBlocks; ++i) dmin = pd[i] < dmin ? pd[i] : dmin;
    const double tr = dmin > 0.f ? kZeroNats / dmin + 2.0 : 1e18;
    const int64_t trans = tr < 1e9 ? (int64_t)tr : (int64_t)1000000000;
    auto length = [&](int n) {
        int64_t row0, len;
        if (ranked) return lens[n];
        seq_bounds(a, n, row0, len);
        return len;
    };
    // The cost of every sequence for the candidate L, priced by one wave: its lanes take the
    // sequences in turn and a butterfly over the 64 lanes sums them (maxima for the critical
    // paths), leaving the total in every lane.  The sums are of whole chunk counts, exact in
    // double, so the result does not depend on the order.
    auto price_wave = [&](int64_t L, bool eg) {
        SplitCost m;
        for (int n = lane; n < N; n += 64) {
            const int64_t len = length(n);
            int P;
            int64_t Ls;
            split_of(len, L, lim.Pmax, P, Ls);
            split_add(m, len, P, Ls, L, nsl, nslt, eg, trans);
        }
        for (int k = 32; k > 0; k >>= 1) {
            m.work1 += __shfl_xor(m.work1, k, 64);
            m.work2 += __shfl_xor(m.work2, k, 64);
            m.work1f += __shfl_xor(m.work1f, k, 64);
            m.work2f += __shfl_xor(m.work2f, k, 64);
            m.big += __shfl_xor(m.big, k, 64);
            m.crit1 = max_i64(m.crit1, (int64_t)__shfl_xor((long long)m.crit1, k, 64));
            m.crit2 = max_i64(m.crit2, (int64_t)__shfl_xor((long long)m.crit2, k, 64));
            m.crit2f = max_i64(m.crit2f, (int64_t)__shfl_xor((long long)m.crit2f, k, 64));
            m.summaries += (int64_t)__shfl_xor((long long)m.summaries, k, 64);
        }
        return m;
    };
    // every wave prices the whole schedule (the same total in each)
    const SplitCost whole = price_wave(0, false);
    const int64_t longest = whole.crit1 * 32;   // in tokens, rounded up to whole chunks
    const double base = split_makespan(whole, 0, H, slots, false);
    // the candidates, P = 2 .. Pmax in each layout (eager first), one wave each, four at a time;
    // then the rule of split_best on each layout, in P order, and the better layout
    constexpr int kMaxCand = 2 * 15;
    __shared__ double cscore[kMaxCand];
    __shared__ int64_t cL[kMaxCand];
    __shared__ int cok[kMaxCand];
    const int per = lim.Pmax - 1, ncand = 2 * per;
    for (int i = wave; i < ncand; i += 4) {
        const bool eg = i < per;
        const int64_t L = split_candidate(longest, 2 + (eg ? i : i - per));
        bool ok = false;
        double score = 0.0;
        if (L >= lim.Lmin) {
            const SplitCost c = price_wave(L, eg);
            const double m = split_makespan(c, L, H, slots, false), f = split_makespan(c, L, H, slots, true);
            ok = c.summaries <= lim.Smax && m < base * kSplitGain && f <= base * kSplitRisk;
            score = m + kSplitTie * f;
        }
        if (lane == 0) {
            cok[i] = ok;
            cscore[i] = score;
            cL[i] = L;
        }
    }
    __syncthreads();
    int64_t Le = 0, Ld = 0;
    double se = 0.0, sd = 0.0;
    for (int i = 0; i < ncand; ++i) {
        if (!cok[i]) continue;
        int64_t& Lb = i < per ? Le : Ld;
        double& sb = i < per ? se : sd;
        if (Lb == 0 || cscore[i] < sb) {
            Lb = cL[i];
            sb = cscore[i];
        }
    }
    const bool eager = Le > 0 && (Ld == 0 || se <= sd);
    const int64_t bestL = eager ? Le : Ld;
    // The plan of bestL.  Sequences are taken longest first (ranked here for up to kRankMax of
    // them, in index order beyond): their summaries' first index and their pass-1 and pass-2
    // items follow from exclusive prefix sums in that order.
    if (ranked) {
        for (int n = t; n < N; n += 256) {
            int r = 0;
            for (int m = 0; m < N; ++m) r += (lens[m] > lens[n]) | ((lens[m] == lens[n]) & (m < n));
            order[r] = n;
        }
        __syncthreads();
    }
    int32_t c_sum = 0, c_a = 0, c_b = 0;
    __shared__ int32_t sc[3][256];
    for (int base = 0; base < N; base += 256) {
        const int r = base + t;
        int P = 0;
        int64_t Ls = 0;
        int n = 0;
        if (r < N) {
            n = ranked ? order[r] : r;
            split_of(length(n), bestL, lim.Pmax, P, Ls);
            plan[lay.segs() + n] = P;
            plan[lay.seglen() + n] = (int32_t)(P > 1 ? Ls : (Ls > 0 ? Ls : kC));
        }
        // pass-1 items: every segment (deferred: all but the last; a whole run: one)
        const int na = r < N ? (P > 1 && !eager ? P - 1 : P) : 0;
        const int nb = r < N ? P - 1 : 0;   // pass-2 items: segments 1 .. P - 1
        const int ns = r < N ? P - 1 : 0;   // summaries
        sc[0][t] = ns;
        sc[1][t] = na;
        sc[2][t] = nb;
        __syncthreads();
        for (int k = 1; k < 256; k <<= 1) {
            const int32_t x0 = t >= k ? sc[0][t - k] : 0, x1 = t >= k ? sc[1][t - k] : 0,
                          x2 = t >= k ? sc[2][t - k] : 0;
            __syncthreads();
            sc[0][t] += x0;
            sc[1][t] += x1;
            sc[2][t] += x2;
            __syncthreads();
        }
        if (r < N) {
            plan[lay.first() + n] = c_sum + sc[0][t] - ns;
            const int32_t ia = c_a + sc[1][t] - na, ib = c_b + sc[2][t] - nb;
            int32_t* A = plan + lay.items1();
            int32_t* B = plan + lay.items2();
            for (int j = 0; j < na; ++j) {
                A[2 * (ia + j)] = n;
                A[2 * (ia + j) + 1] = j;
            }
            for (int j = 0; j < nb; ++j) {
                B[2 * (ib + j)] = n;
                B[2 * (ib + j) + 1] = j + 1;
            }
        }
        c_sum += sc[0][255];
        c_a += sc[1][255];
        c_b += sc[2][255];
        __syncthreads();
    }
    if (t == 0) {
        plan[0] = (int32_t)bestL;
        plan[1] = c_a;
        plan[2] = c_b;
        plan[3] = eager ? 1 : 0;
    }
}

hipError_t launch_plan(const PrefillArgs& a, int32_t* plan, int slots, SplitLimits lim) {
    const PlanLayout lay{a.N, (int32_t)lim.Smax};
    const int64_t tokens = a.cu ? a.T : (int64_t)a.N * a.T;
    hipLaunchKernelGGL(probe_kernel, dim3(kProbeBlocks), dim3(256), 0, a.stream, a, plan + lay.probe(), tokens);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(256), 0, a.stream, a, plan, slots, lim);
    return hipGetLastError();
}

}  // namespace kda
