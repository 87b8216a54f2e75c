// KDA chunkwise prefill, one fused kernel: intra-chunk work and the inter-chunk state scan.
//
// Kimi K3: Open Frontier Intelligence, §2.1.1, eqs. (3)-(4): recurrent across chunks, parallel
// inside a chunk.  For a chunk entered with state S (positions r = 0..C-1), G_r is the running
// sum of g inside the chunk (log of the cumulative decay gamma of eq. (3)), and unrolling eq. (1)
// over the chunk gives (the UT transform the pages defer to Kimi Linear):
//     A_kk[r,i] = beta_r sum_c k_rc k_ic exp(G_rc - G_ic)        i < r   (strictly lower)
//     T = (I + A_kk)^-1,  T_b = T Diag(beta)
//     W = T_b (K * exp(G)),  U = T_b V,  V~ = U - W S                      (pseudo-values)
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
// Grid: one 256-thread workgroup (4 waves) per (sequence, head, 64-column slice of dv).  Wave w
// owns value columns [16w, 16w + 16) of the slice: its slice of the state S (dk x 16, fp32) lives
// in MFMA accumulator registers for the whole sequence and doubles as the B operand of W S and
// Q~ S, so the state never leaves the chip between chunks.  The state-independent intra-chunk work
// (decay prefix, Gram tiles, the triangular inverse, W) is recomputed by each column slice of a
// head; the slices of one head are placed on the same XCD so their re-reads of q, k, g hit L2.
//
// Precision: bf16 MFMA with fp32 accumulation.  Operands whose rounding would dominate the error
// are carried as hi + lo bf16 pairs (products hi*hi + lo*hi + hi*lo): the decayed Gram operands,
// A_qk, V~ in both of its uses, and both operands of the inter-chunk output term (Q * exp(G)) S,
// which dominates short sequences entered with a large state.  T_b, K~, W and K_end, and the
// state as the operand of W S, are single bf16; U and the state stay fp32.  Float32 inputs
// (kFull) carry every operand as a pair.
#include <type_traits>

#include "kda_device.h"
#include "kda_launch.h"

namespace kda {

constexpr int kC = 32;     // chunk length (two 16-token sub-tiles)
constexpr int kDVT = 64;   // value columns per workgroup
constexpr int kNT = 256;   // threads per workgroup (4 waves)

template <int DK, bool F32IN>
struct Layout {
    static constexpr bool kFull = F32IN;
    static constexpr int kNP = kFull ? 2 : 1;            // bf16 planes of "single" operands
    using IT = typename std::conditional<F32IN, float, bf16>::type;
    static constexpr int RB = DK + 8;                      // bf16 row-major [token][DK] stride
    static constexpr int RF = DK + 4;                      // fp32 row-major stride
    static constexpr int RI = F32IN ? RF : RB;             // raw input row stride
    static constexpr int TB = kC + 8;                      // bf16 [*][token] stride
    static constexpr int AB = kC + 8;                      // bf16 [C][C] stride
    static constexpr int AF = kC + 4;                      // fp32 [C][C] stride
    // Group A (raw chunk and decay factors; dead after the operand pass), later reused.
    static constexpr int o_rq = 0;
    static constexpr int o_rk = o_rq + kC * RI * (int)sizeof(IT);
    static constexpr int o_P = o_rk + kC * RI * (int)sizeof(IT);
    static constexpr int o_Pi = o_P + kC * RF * 4;
    static constexpr int endA1 = o_Pi + kC * RF * 4;
    static constexpr int o_Akk = 0;                        // fp32 [C][AF]
    static constexpr int o_Tm = o_Akk + kC * AF * 4;       // fp32 [C][AF]
    static constexpr int o_Tb = o_Tm + kC * AF * 4;        // bf16 planes [C][AB]
    static constexpr int o_W = o_Tb + kNP * kC * AB * 2;   // bf16 planes [C][RB]
    static constexpr int endA2 = o_W + kNP * kC * RB * 2;
    static constexpr int endA = endA1 > endA2 ? endA1 : endA2;
    // Group G: split Gram operands (hi plane, lo plane).
    static constexpr int o_Qs = endA;
    static constexpr int o_Kr = o_Qs + 2 * kC * RB * 2;
    static constexpr int o_Kd = o_Kr + 2 * kC * RB * 2;
    static constexpr int o_Kc = o_Kd + 2 * kC * RB * 2;    // 16 rows
    static constexpr int endG = o_Kc + 2 * 16 * RB * 2;
    // Persistent within a chunk (the split Qs of group G also stays live until the outputs).
    static constexpr int o_Kt = endG;                      // bf16 planes [DK][TB]  (K~ transposed)
    static constexpr int o_Ke = o_Kt + kNP * DK * TB * 2;  // bf16 planes [DK][TB]  (K_end transp.)
    static constexpr int o_Vt = o_Ke + kNP * DK * TB * 2;  // bf16 planes [DVT][TB] (V transposed)
    static constexpr int o_Aq = o_Vt + kNP * kDVT * TB * 2;// bf16 hi, lo [C][AB]
    static constexpr int o_beta = o_Aq + 2 * kC * AB * 2;  // fp32 [C]
    static constexpr int o_gam = o_beta + kC * 4;          // fp32 [DK]
    static constexpr int o_D = o_gam + DK * 4;             // fp32 [2][DK] tile log2-decay totals
    static constexpr int o_F0 = o_D + 2 * DK * 4;          // fp32 [DK] exp of tile-0 total
    static constexpr int total = o_F0 + DK * 4;
    static_assert(total <= 160 * 1024, "LDS budget");
};

template <typename L>
struct Smem {
    char* base;
    __device__ bf16* bfp(int off) const { return reinterpret_cast<bf16*>(base + off); }
    __device__ float* f32p(int off) const { return reinterpret_cast<float*>(base + off); }
};

// One block of the grid -> (unit, column slice), slices of a unit on one XCD (the dispatcher
// places consecutive workgroups on consecutive XCDs, 8 of them).
__device__ __forceinline__ void block_coords(int nslices, int& unit, int& slice) {
    const int b = blockIdx.x;
    const int xcd = b & 7, slot = b >> 3;
    unit = (slot / nslices) * 8 + xcd;
    slice = slot % nslices;
}

template <int DK, bool F32IN, bool OUT_F32>
__global__ __launch_bounds__(kNT, 1) void prefill_kernel(PrefillArgs a) {
    using Lay = Layout<DK, F32IN>;
    using IT = typename Lay::IT;
    constexpr bool kFull = Lay::kFull;
    constexpr int KS = DK / 32;          // 32-channel contraction steps
    constexpr int CT = DK / 16;          // 16-channel tiles of the state
    constexpr int RB = Lay::RB, RF = Lay::RF, RI = Lay::RI, TB = Lay::TB, AB = Lay::AB,
                  AF = Lay::AF;
    extern __shared__ __attribute__((aligned(16))) char smem_raw[];
    Smem<Lay> sm{smem_raw};

    const int nslices = a.dv / kDVT;
    int unit, slice;
    block_coords(nslices, unit, slice);
    if (unit >= a.N * a.H) return;
    const int n = unit / a.H, h = unit % a.H;

    // Sequence bounds (clamped: malformed cu_seqlens never produce out-of-bounds accesses).
    int64_t row0, len;
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
    const int H = a.H;
    const size_t sq = (size_t)H * DK;          // token stride of q, k, g (elements)
    const size_t sv = (size_t)H * a.dv;        // token stride of v, o
    const IT* qg = reinterpret_cast<const IT*>(a.q) + (size_t)row0 * sq + (size_t)h * DK;
    const IT* kg = reinterpret_cast<const IT*>(a.k) + (size_t)row0 * sq + (size_t)h * DK;
    const float* gg = a.g + (size_t)row0 * sq + (size_t)h * DK;
    const IT* vg = reinterpret_cast<const IT*>(a.v) + (size_t)row0 * sv + (size_t)h * a.dv +
                   (size_t)slice * kDVT;
    const IT* bg = reinterpret_cast<const IT*>(a.beta) + (size_t)row0 * H + h;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int i16 = lane & 15, g4 = lane >> 4;
    const int col0 = slice * kDVT + 16 * wave;  // first value column of this wave

    // ---- state slice in accumulators: Sacc[ct][j] = S[16 ct + 4 g4 + j][col0 + i16]
    f32x4 Sacc[CT];
    {
        const float* S0 = a.S0 ? a.S0 + ((size_t)n * H + h) * DK * a.dv : nullptr;
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                Sacc[ct][j] = S0 ? S0[(size_t)(16 * ct + 4 * g4 + j) * a.dv + col0 + i16] : 0.f;
    }

    // ---- prefetch plan (registers), loaded one chunk ahead
    constexpr int PPR = DK * (int)sizeof(IT) / 16;        // 16-byte pieces per q/k row
    constexpr int NQK = 2 * kC * PPR / kNT;                // q and k pieces per thread
    static_assert((2 * kC * PPR) % kNT == 0, "q/k piece split");
    constexpr int PPV = kDVT * (int)sizeof(IT) / 16;      // pieces per v row
    constexpr int NV = (kC * PPV + kNT - 1) / kNT;         // v pieces per thread
    const bool gcol = tid < 2 * DK;                         // column-pass threads
    const int gc = tid % DK, ga = tid / DK;                 // (channel, 16-row tile)
    uint4 pqk[NQK];
    uint4 pv[NV];
    float pg[16];
    float pb = 0.f;

    auto prefetch = [&](int64_t c0) {
        const int nvalid = (int)((len - c0) < kC ? (len - c0) : kC);
#pragma unroll
        for (int i = 0; i < NQK; ++i) {
            const int p = tid + kNT * i;
            const int arr = p / (kC * PPR), rem = p % (kC * PPR);
            const int r = rem / PPR, pc = rem % PPR;
            const IT* src = (arr ? kg : qg) + (size_t)(c0 + r) * sq;
            pqk[i] = r < nvalid ? ld<uint4>(reinterpret_cast<const char*>(src) + 16 * pc)
                                : uint4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int p = tid + kNT * i;
            const int r = p / PPV, pc = p % PPV;
            pv[i] = (p < kC * PPV && r < nvalid)
                        ? ld<uint4>(reinterpret_cast<const char*>(vg + (size_t)(c0 + r) * sv) +
                                    16 * pc)
                        : uint4{0u, 0u, 0u, 0u};
        }
        if (gcol) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int rr = 16 * ga + r;
                pg[r] = rr < nvalid ? gg[(size_t)(c0 + rr) * sq + gc] : 0.f;
            }
        }
        if (tid < kC) pb = tid < nvalid ? static_cast<float>(bg[(size_t)(c0 + tid) * H]) : 0.f;
    };

    const int64_t nchunks = (len + kC - 1) / kC;
    if (nchunks > 0) prefetch(0);

    for (int64_t ci = 0; ci < nchunks; ++ci) {
        const int64_t c0 = ci * kC;
        const int nvalid = (int)((len - c0) < kC ? (len - c0) : kC);

        // ---------------- step 0: raw chunk -> LDS
#pragma unroll
        for (int i = 0; i < NQK; ++i) {
            const int p = tid + kNT * i;
            const int arr = p / (kC * PPR), rem = p % (kC * PPR);
            const int r = rem / PPR, pc = rem % PPR;
            char* dst = sm.base + (arr ? Lay::o_rk : Lay::o_rq) + (r * RI) * (int)sizeof(IT) + 16 * pc;
            st<uint4>(dst, pqk[i]);
        }
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int p = tid + kNT * i;
            if (p < kC * PPV) {
                const int r = p / PPV, pc = p % PPV;
                if constexpr (F32IN) {
                    const float* x = reinterpret_cast<const float*>(&pv[i]);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        bf16 hi, lo;
                        split_bf16(x[e], hi, lo);
                        const int col = 4 * pc + e;
                        sm.bfp(Lay::o_Vt)[col * TB + r] = hi;
                        sm.bfp(Lay::o_Vt + kDVT * TB * 2)[col * TB + r] = lo;
                    }
                } else {
                    const bf16* x = reinterpret_cast<const bf16*>(&pv[i]);
#pragma unroll
                    for (int e = 0; e < 8; ++e) sm.bfp(Lay::o_Vt)[(8 * pc + e) * TB + r] = x[e];
                }
            }
        }
        if (tid < kC) sm.f32p(Lay::o_beta)[tid] = pb;

        // ---------------- step 1: per-channel decay prefix inside each 16-token tile (log2 units)
        float Pc[16], Pic[16];
        if (gcol) {
            float L = 0.f;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                L += pg[r] * kLog2e;
                Pc[r] = exp2f(L);
                Pic[r] = exp2f(-L);
                sm.f32p(Lay::o_P)[(16 * ga + r) * RF + gc] = Pc[r];
                sm.f32p(Lay::o_Pi)[(16 * ga + r) * RF + gc] = Pic[r];
            }
            sm.f32p(Lay::o_D)[ga * DK + gc] = L;
            if (ga == 0) sm.f32p(Lay::o_F0)[gc] = exp2f(L);
        }
        __syncthreads();
        // the column values are consumed: fetch the next chunk while this one is computed
        if (ci + 1 < nchunks) prefetch(c0 + kC);

        // ---------------- step 2a: transposed K~ = k exp(G) and K_end = k exp(G_last - G)
        if (gcol) {
            const float D0 = sm.f32p(Lay::o_D)[gc], D1 = sm.f32p(Lay::o_D)[DK + gc];
            const float Eprev = ga ? D0 : 0.f;       // log2 decay from chunk start to tile start
            const float fK = exp2f(Eprev), fE = exp2f(D0 + D1 - Eprev);
            if (ga == 0) sm.f32p(Lay::o_gam)[gc] = exp2f(D0 + D1);
            bf16 kt_h[16], ke_h[16], kt_l[16], ke_l[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float kv =
                    static_cast<float>(reinterpret_cast<const IT*>(sm.base + Lay::o_rk)[(16 * ga + r) * RI + gc]);
                const float xt = kv * Pc[r] * fK, xe = kv * Pic[r] * fE;
                if constexpr (kFull) {
                    split_bf16(xt, kt_h[r], kt_l[r]);
                    split_bf16(xe, ke_h[r], ke_l[r]);
                } else {
                    kt_h[r] = f2bf(xt);
                    ke_h[r] = f2bf(xe);
                }
            }
            bf16* Kt = sm.bfp(Lay::o_Kt) + gc * TB + 16 * ga;
            bf16* Ke = sm.bfp(Lay::o_Ke) + gc * TB + 16 * ga;
#pragma unroll
            for (int r = 0; r < 16; r += 8) {
                st<bf16x8>(Kt + r, bf16x8{kt_h[r], kt_h[r + 1], kt_h[r + 2], kt_h[r + 3],
                                          kt_h[r + 4], kt_h[r + 5], kt_h[r + 6], kt_h[r + 7]});
                st<bf16x8>(Ke + r, bf16x8{ke_h[r], ke_h[r + 1], ke_h[r + 2], ke_h[r + 3],
                                          ke_h[r + 4], ke_h[r + 5], ke_h[r + 6], ke_h[r + 7]});
                if constexpr (kFull) {
                    st<bf16x8>(Kt + DK * TB + r,
                               bf16x8{kt_l[r], kt_l[r + 1], kt_l[r + 2], kt_l[r + 3], kt_l[r + 4],
                                      kt_l[r + 5], kt_l[r + 6], kt_l[r + 7]});
                    st<bf16x8>(Ke + DK * TB + r,
                               bf16x8{ke_l[r], ke_l[r + 1], ke_l[r + 2], ke_l[r + 3], ke_l[r + 4],
                                      ke_l[r + 5], ke_l[r + 6], ke_l[r + 7]});
                }
            }
        }

        // ---------------- step 2b: row-major decayed operands (split Gram operands, Q~)
        {
            constexpr int NG8 = DK / 8;
            constexpr int NTASK = kC * NG8;
#pragma unroll
            for (int it = 0; it < (NTASK + kNT - 1) / kNT; ++it) {
                const int id = tid + kNT * it;
                if (NTASK % kNT == 0 || id < NTASK) {
                    const int r = id / NG8, c8 = 8 * (id % NG8);
                    const int tile = r >> 4;
                    float qv[8], kv[8];
                    const IT* rq = reinterpret_cast<const IT*>(sm.base + Lay::o_rq) + r * RI + c8;
                    const IT* rk = reinterpret_cast<const IT*>(sm.base + Lay::o_rk) + r * RI + c8;
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        qv[e] = static_cast<float>(rq[e]) * a.scale;
                        kv[e] = static_cast<float>(rk[e]);
                    }
                    const float* P = sm.f32p(Lay::o_P) + r * RF + c8;
                    const float* Pi = sm.f32p(Lay::o_Pi) + r * RF + c8;
                    const float* F0 = sm.f32p(Lay::o_F0) + c8;
                    bf16x8 qh, ql, krh, krl, kdh, kdl, kch, kcl;
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const float p = P[e], pi = Pi[e];
                        const float qs = qv[e] * p, kr = kv[e] * p, kd = kv[e] * pi;
                        bf16 h_, l_;
                        split_bf16(qs, h_, l_); qh[e] = h_; ql[e] = l_;
                        split_bf16(kr, h_, l_); krh[e] = h_; krl[e] = l_;
                        split_bf16(kd, h_, l_); kdh[e] = h_; kdl[e] = l_;
                        if (tile == 0) { split_bf16(kd * F0[e], h_, l_); kch[e] = h_; kcl[e] = l_; }
                    }
                    const int off = r * RB + c8;
                    st<bf16x8>(sm.bfp(Lay::o_Qs) + off, qh);
                    st<bf16x8>(sm.bfp(Lay::o_Qs) + kC * RB + off, ql);
                    st<bf16x8>(sm.bfp(Lay::o_Kr) + off, krh);
                    st<bf16x8>(sm.bfp(Lay::o_Kr) + kC * RB + off, krl);
                    st<bf16x8>(sm.bfp(Lay::o_Kd) + off, kdh);
                    st<bf16x8>(sm.bfp(Lay::o_Kd) + kC * RB + off, kdl);
                    if (tile == 0) {
                        st<bf16x8>(sm.bfp(Lay::o_Kc) + off, kch);
                        st<bf16x8>(sm.bfp(Lay::o_Kc) + 16 * RB + off, kcl);
                    }
                }
            }
        }
        __syncthreads();

        // ---------------- step 3: Gram tiles A_qk, A_kk (split operands, 3 MFMAs per step)
        if (wave < 3) {
            const int ta = wave == 0 ? 0 : 1;             // row tile
            const int tb = wave == 1 ? 1 : 0;             // column tile
            const bf16* Qh = sm.bfp(Lay::o_Qs) + (16 * ta + i16) * RB + 8 * g4;
            const bf16* Kh = sm.bfp(Lay::o_Kr) + (16 * ta + i16) * RB + 8 * g4;
            const bf16* Bh = (ta == tb) ? sm.bfp(Lay::o_Kd) + (16 * tb + i16) * RB + 8 * g4
                                        : sm.bfp(Lay::o_Kc) + i16 * RB + 8 * g4;
            const int Blo = (ta == tb) ? kC * RB : 16 * RB;
            f32x4 aq = zero4(), ak = zero4();
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                const bf16x8 qh = ld<bf16x8>(Qh + 32 * s), ql = ld<bf16x8>(Qh + kC * RB + 32 * s);
                const bf16x8 kh = ld<bf16x8>(Kh + 32 * s), kl = ld<bf16x8>(Kh + kC * RB + 32 * s);
                const bf16x8 bh = ld<bf16x8>(Bh + 32 * s), bl = ld<bf16x8>(Bh + Blo + 32 * s);
                aq = mma(qh, bh, aq);
                aq = mma(ql, bh, aq);
                aq = mma(qh, bl, aq);
                ak = mma(kh, bh, ak);
                ak = mma(kl, bh, ak);
                ak = mma(kh, bl, ak);
            }
            const int col = 16 * tb + i16;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int row = 16 * ta + 4 * g4 + j;
                const float vq = (col <= row) ? aq[j] : 0.f;
                const float vk = (col < row) ? ak[j] * sm.f32p(Lay::o_beta)[row] : 0.f;
                bf16 hq, lq;
                split_bf16(vq, hq, lq);
                sm.bfp(Lay::o_Aq)[row * AB + col] = hq;
                sm.bfp(Lay::o_Aq + kC * AB * 2)[row * AB + col] = lq;
                sm.f32p(Lay::o_Akk)[row * AF + col] = vk;
            }
        } else {
            // upper-right block of A_qk (row tile 0, column tile 1) is zero
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int row = 4 * g4 + j, col = 16 + i16;
                sm.bfp(Lay::o_Aq)[row * AB + col] = f2bf(0.f);
                sm.bfp(Lay::o_Aq + kC * AB * 2)[row * AB + col] = f2bf(0.f);
            }
        }
        __syncthreads();

        // ---------------- step 4: inverses of the two unit-lower-triangular diagonal blocks
        if (wave == 0 && lane < 32) {
            const int bb = lane >> 4, c = i16;
            const float* Ab = sm.f32p(Lay::o_Akk) + (16 * bb) * AF + 16 * bb;
            float x[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float s = 0.f;
#pragma unroll
                for (int j = 0; j < r; ++j) s += Ab[r * AF + j] * x[j];
                x[r] = (r == c) ? 1.f : ((r > c) ? -s : 0.f);
            }
            float* Tb = sm.f32p(Lay::o_Tm) + (16 * bb) * AF + 16 * bb;
#pragma unroll
            for (int r = 0; r < 16; ++r) Tb[r * AF + c] = x[r];
        }
        __syncthreads();

        // ---------------- step 5: X = A_kk[1,0] T00, kept in the unused upper block of A_kk
        {
            const int r = tid >> 4, c = tid & 15;
            const float* A10 = sm.f32p(Lay::o_Akk) + (16 + r) * AF;
            const float* T00 = sm.f32p(Lay::o_Tm);
            float s = 0.f;
#pragma unroll
            for (int m = 0; m < 16; ++m) s += A10[m] * T00[m * AF + c];
            sm.f32p(Lay::o_Akk)[r * AF + 16 + c] = s;
        }
        __syncthreads();

        // ---------------- step 6: T10 = -T11 X, then T_b = T Diag(beta) in bf16
        {
            const int r = tid >> 4, c = tid & 15;
            const float* T11 = sm.f32p(Lay::o_Tm) + (16 + r) * AF + 16;
            float s = 0.f;
#pragma unroll
            for (int m = 0; m < 16; ++m) s += T11[m] * sm.f32p(Lay::o_Akk)[m * AF + 16 + c];
            const float* beta = sm.f32p(Lay::o_beta);
            const float t00 = sm.f32p(Lay::o_Tm)[r * AF + c] * beta[c];
            const float t11 = sm.f32p(Lay::o_Tm)[(16 + r) * AF + 16 + c] * beta[16 + c];
            const float t10 = -s * beta[c];
            bf16* Tb = sm.bfp(Lay::o_Tb);
            if constexpr (kFull) {
                bf16 hh, ll;
                split_bf16(t00, hh, ll); Tb[r * AB + c] = hh; Tb[kC * AB + r * AB + c] = ll;
                split_bf16(t11, hh, ll); Tb[(16 + r) * AB + 16 + c] = hh; Tb[kC * AB + (16 + r) * AB + 16 + c] = ll;
                split_bf16(t10, hh, ll); Tb[(16 + r) * AB + c] = hh; Tb[kC * AB + (16 + r) * AB + c] = ll;
                Tb[r * AB + 16 + c] = f2bf(0.f); Tb[kC * AB + r * AB + 16 + c] = f2bf(0.f);
            } else {
                Tb[r * AB + c] = f2bf(t00);
                Tb[(16 + r) * AB + 16 + c] = f2bf(t11);
                Tb[(16 + r) * AB + c] = f2bf(t10);
                Tb[r * AB + 16 + c] = f2bf(0.f);
            }
        }
        __syncthreads();

        // ---------------- step 7: W^T = K~^T T_b^T (all waves) and U = T_b V (own columns)
        {
            const bf16* Tb = sm.bfp(Lay::o_Tb);
            constexpr int NWT = CT * 2;                    // output tiles of W^T
#pragma unroll
            for (int tt = wave; tt < NWT; tt += 4) {
                const int ct = tt >> 1, tk = tt & 1;
                const bf16* Ka = sm.bfp(Lay::o_Kt) + (16 * ct + i16) * TB + 8 * g4;
                const bf16* Bt = Tb + (16 * tk + i16) * AB + 8 * g4;
                f32x4 acc = mma(ld<bf16x8>(Ka), ld<bf16x8>(Bt), zero4());
                if constexpr (kFull) {
                    acc = mma(ld<bf16x8>(Ka + DK * TB), ld<bf16x8>(Bt), acc);
                    acc = mma(ld<bf16x8>(Ka), ld<bf16x8>(Bt + kC * AB), acc);
                }
                // acc[j] = W[16 tk + i16][16 ct + 4 g4 + j]
                bf16* Wd = sm.bfp(Lay::o_W) + (16 * tk + i16) * RB + 16 * ct + 4 * g4;
                if constexpr (kFull) {
                    bf16x4 hv, lv;
#pragma unroll
                    for (int j = 0; j < 4; ++j) { bf16 hh, ll; split_bf16(acc[j], hh, ll); hv[j] = hh; lv[j] = ll; }
                    st<bf16x4>(Wd, hv);
                    st<bf16x4>(Wd + kC * RB, lv);
                } else {
                    st<bf16x4>(Wd, bf16x4{f2bf(acc[0]), f2bf(acc[1]), f2bf(acc[2]), f2bf(acc[3])});
                }
            }
        }
        f32x4 U[2];
        {
            const bf16* Tb = sm.bfp(Lay::o_Tb);
            const bf16* Vb = sm.bfp(Lay::o_Vt) + (16 * wave + i16) * TB + 8 * g4;
            const bf16x8 vh = ld<bf16x8>(Vb);
#pragma unroll
            for (int ta = 0; ta < 2; ++ta) {
                const bf16* Ta = Tb + (16 * ta + i16) * AB + 8 * g4;
                U[ta] = mma(ld<bf16x8>(Ta), vh, zero4());
                if constexpr (kFull) {
                    U[ta] = mma(ld<bf16x8>(Ta + kC * AB), vh, U[ta]);
                    U[ta] = mma(ld<bf16x8>(Ta), ld<bf16x8>(Vb + kDVT * TB), U[ta]);
                }
            }
        }
        __syncthreads();

        // ---------------- step 8: inter-chunk part on this wave's 16 state columns
        {
            // state as B operand: contraction index (32-channel step s, g4, e) ->
            // channel 32 s + 4 g4 + e (e < 4), 32 s + 16 + 4 g4 + (e - 4) (e >= 4).
            // Sh/Sl: the state split hi + lo; Fh/Fl: Diag(exp(G at the end of tile 0)) S, the
            // entering state seen from the start of tile 1, so that tile 1's (Q * exp(G)) S is
            // Qs S' with the same split Qs operand as the Gram tiles.
            bf16x8 Sh[KS], Sl[KS], Fh[KS], Fl[KS];
            const float* F0 = sm.f32p(Lay::o_F0);
#pragma unroll
            for (int s = 0; s < KS; ++s)
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int ct = 2 * s + (e >> 2), j = e & 3;
                    const float x = Sacc[ct][j];
                    bf16 hh, ll;
                    split_bf16(x, hh, ll);
                    Sh[s][e] = hh;
                    Sl[s][e] = ll;
                    split_bf16(x * F0[16 * ct + 4 * g4 + j], hh, ll);
                    Fh[s][e] = hh;
                    Fl[s][e] = ll;
                }
            auto ldA = [&](const bf16* rowp, int s) -> bf16x8 {   // same channel selection
                return cat44(ld<bf16x4>(rowp + 32 * s + 4 * g4), ld<bf16x4>(rowp + 32 * s + 16 + 4 * g4));
            };
            f32x4 Vt[2];
#pragma unroll
            for (int ta = 0; ta < 2; ++ta) {
                const bf16* Wr = sm.bfp(Lay::o_W) + (16 * ta + i16) * RB;
                f32x4 acc = zero4();
#pragma unroll
                for (int s = 0; s < KS; ++s) {
                    const bf16x8 wa = ldA(Wr, s);
                    acc = mma(wa, Sh[s], acc);
                    if constexpr (kFull) {
                        acc = mma(ldA(Wr + kC * RB, s), Sh[s], acc);
                        acc = mma(wa, Sl[s], acc);
                    }
                }
                Vt[ta] = U[ta] - acc;
            }
            // V~ as B operand: token index (g4, e) -> 4 g4 + e (e < 4), 16 + 4 g4 + (e - 4)
            bf16x8 Vh, Vl;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                bf16 hh, ll;
                split_bf16(Vt[e >> 2][e & 3], hh, ll);
                Vh[e] = hh;
                Vl[e] = ll;
            }
            // outputs O = Q~ S + A_qk V~ (Q~ S as split Qs times the split (rescaled) state)
#pragma unroll
            for (int ta = 0; ta < 2; ++ta) {
                const bf16* Qr = sm.bfp(Lay::o_Qs) + (16 * ta + i16) * RB;
                f32x4 acc = zero4();
#pragma unroll
                for (int s = 0; s < KS; ++s) {
                    const bf16x8 qa = ldA(Qr, s), ql = ldA(Qr + kC * RB, s);
                    const bf16x8 bh = ta ? Fh[s] : Sh[s], bl = ta ? Fl[s] : Sl[s];
                    acc = mma(qa, bh, acc);
                    acc = mma(ql, bh, acc);
                    acc = mma(qa, bl, acc);
                }
                const bf16* Ar = sm.bfp(Lay::o_Aq) + (16 * ta + i16) * AB;
                const bf16x8 ah = cat44(ld<bf16x4>(Ar + 4 * g4), ld<bf16x4>(Ar + 16 + 4 * g4));
                const bf16x8 al = cat44(ld<bf16x4>(Ar + kC * AB + 4 * g4),
                                        ld<bf16x4>(Ar + kC * AB + 16 + 4 * g4));
                acc = mma(ah, Vh, acc);
                acc = mma(al, Vh, acc);
                acc = mma(ah, Vl, acc);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int r = 16 * ta + 4 * g4 + j;
                    if (r < nvalid) {
                        const size_t off = (size_t)(row0 + c0 + r) * sv + (size_t)h * a.dv + col0 + i16;
                        if constexpr (OUT_F32) reinterpret_cast<float*>(a.o)[off] = acc[j];
                        else reinterpret_cast<bf16*>(a.o)[off] = f2bf(acc[j]);
                    }
                }
            }
            // state: S <- Diag(gamma_last) S + K_end^T V~
            const float* gam = sm.f32p(Lay::o_gam);
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) {
                const bf16* Kr = sm.bfp(Lay::o_Ke) + (16 * ct + i16) * TB;
                const bf16x8 ka = cat44(ld<bf16x4>(Kr + 4 * g4), ld<bf16x4>(Kr + 16 + 4 * g4));
                f32x4 s = Sacc[ct];
#pragma unroll
                for (int j = 0; j < 4; ++j) s[j] *= gam[16 * ct + 4 * g4 + j];
                s = mma(ka, Vh, s);
                s = mma(ka, Vl, s);
                if constexpr (kFull)
                    s = mma(cat44(ld<bf16x4>(Kr + DK * TB + 4 * g4), ld<bf16x4>(Kr + DK * TB + 16 + 4 * g4)), Vh, s);
                Sacc[ct] = s;
            }
        }
        __syncthreads();
    }

    if (a.ST) {
        float* ST = a.ST + ((size_t)n * H + h) * DK * a.dv;
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                ST[(size_t)(16 * ct + 4 * g4 + j) * a.dv + col0 + i16] = Sacc[ct][j];
    }
}

template <int DK, bool F32IN, bool OUT_F32>
static hipError_t launch_prefill(const PrefillArgs& a) {
    using Lay = Layout<DK, F32IN>;
    auto kern = prefill_kernel<DK, F32IN, OUT_F32>;
    static bool attr_set = false;   // benign race: the attribute value is idempotent
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, Lay::total);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    const int nslices = a.dv / kDVT;
    const int64_t units = (int64_t)a.N * a.H;
    const int64_t blocks = ((units + 7) / 8) * 8 * nslices;
    if (blocks == 0) return hipSuccess;
    hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(kNT), Lay::total, a.stream, a);
    return hipGetLastError();
}

hipError_t launch_chunk_fwd(const PrefillArgs& a) {
    if (a.dk == 128) {
        // float32 inputs at dk = 128 would not fit the 160 KB LDS (rejected by the ABI)
        if (a.in_f32) return hipErrorInvalidValue;
        return a.out_f32 ? launch_prefill<128, false, true>(a) : launch_prefill<128, false, false>(a);
    }
    if (a.dk == 64) {
        if (a.in_f32) return a.out_f32 ? launch_prefill<64, true, true>(a) : launch_prefill<64, true, false>(a);
        return a.out_f32 ? launch_prefill<64, false, true>(a) : launch_prefill<64, false, false>(a);
    }
    return hipErrorInvalidValue;
}

}  // namespace kda
