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
    // Segmented (context-parallel) runs over nseg time segments per sequence:
    //   mode 0: plain prefill (nseg, ws, stops unused);
    //   mode 1: every segment from its entering state (S0 for the first, 0 for the others) with
    //           its outputs; the state after segments j < nseg - 1 -> ws (the last writes S_T),
    //           and for segments j >= 1 the transition (extra dk columns entered with the
    //           identity, value 0) -> ws for j < nseg - 1, with the number of its chunks before it
    //           vanishes -> stops;
    //   mode 2: segments j >= 1 rebuild their entering state from the summaries of the segments
    //           before them and run again over the chunks whose outputs depend on it (all of
    //           them, and S_T for the last, where the transition never reaches zero).
    //   Without a plan every sequence has nseg segments of ceil(len / nseg) tokens rounded up
    //   to whole chunks.  With one (plan != null, from launch_plan), sequence n has
    //   plan[1 + n] <= nseg segments of plan[1 + 2N + n] tokens, its summaries start at index
    //   plan[1 + N + n], and a sequence with one segment runs whole in mode 1 (outputs and S_T).
    int32_t mode;
    int32_t nseg;
    int64_t seg_len;          // unused (kept for the layout of this record)
    float* ws;                // summaries [index, H, dk, dv + dk] float32 (modes 1, 2)
    hipStream_t stream;
    // decay map in the kernel (g unused): g = -5 Sigmoid(exp(A_log[h]) z), z [.., H, dk] stored
    // like q
    const void* z = nullptr;
    const float* A_log = nullptr;
    const int32_t* plan = nullptr;   // see PlanLayout
    int32_t plan_smax = 0;           // summaries the plan may use (per head)
    int32_t plan_items = 0;          // grid bound of this pass: work items of the plan
    // modes 1, 2: per (summary index, head, transition slice of 64 columns) the chunks of segment
    // j >= 1 (summary index of segment j - 1) whose outputs depend on its entering state
    int32_t* stops = nullptr;
};

// Layout of a device plan (int32), for N sequences and at most Smax summaries:
//   [0] segment length (0: no split), [1] items of pass 1, [2] items of pass 2, [3] 1 for the
//   eager layout, 0 for the deferred one (below, at the split cost model),
//   segs[N], first summary[N], segment length[N] per sequence,
//   pass-1 items [N + Smax] x {sequence, segment}: the segments of the split sequences that pass
//   1 runs and the whole runs of the others, longest sequences first,
//   pass-2 items [N + Smax] x {sequence, segment}: the segments after the first of the split
//   sequences,
//   probe[kProbeBlocks]: per workgroup of the decay probe, the smallest decay (nats, float bits)
//   of a key channel over one of kProbeChunks 32-token samples spread evenly over the batch.
constexpr int kProbeChunks = 8, kProbeGroups = 8, kProbeBlocks = kProbeChunks * kProbeGroups;
struct PlanLayout {
    int32_t N, Smax;
    __host__ __device__ int64_t segs() const { return 4; }
    __host__ __device__ int64_t first() const { return 4 + (int64_t)N; }
    __host__ __device__ int64_t seglen() const { return 4 + 2 * (int64_t)N; }
    __host__ __device__ int64_t items1() const { return 4 + 3 * (int64_t)N; }
    __host__ __device__ int64_t items2() const { return items1() + 2 * ((int64_t)N + Smax); }
    __host__ __device__ int64_t probe() const { return items2() + 2 * ((int64_t)N + Smax); }
    __host__ __device__ int64_t ints() const { return probe() + kProbeBlocks; }
    __host__ __device__ int32_t max_items1() const { return N + Smax; }
    __host__ __device__ int32_t max_items2() const { return Smax; }   // one per summary
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

// ---- Splitting sequences in time (in-device context parallelism).  Costs are in chunk steps
// of one workgroup (one 32-token chunk of one 64-column slice).  A sequence of len tokens left
// whole costs nsl workgroups x ceil(len / 32) steps, in pass 1.  A sequence split into P
// segments of Ls tokens (the last one shorter or equal) runs, in pass 1, its first segment from
// S0 and later ones from 0, each with its outputs (nsl x ceil(Ls_j / 32)), and the transitions
// of the segments j >= 1 it runs (nslt - nsl workgroups x ceil(Ls_j / 32)); in pass 2 each
// segment j >= 1 again from its true entering state, over c_j + j steps: c_j chunks whose outputs
// depend on that state (the chunks until the segment's transition is negligible) and the j
// summaries it composes.  Two layouts:
//   eager:    pass 1 runs every segment, so pass 2 runs only the c_j chunks of each;
//   deferred: pass 1 runs all but the last, which pass 2 runs whole (c = its length).
// Transitions stop, and c_j ends, once every entry of the transition is below 2^-140 of the
// identity it starts from, which a decay of every key channel by d nats per chunk brings about
// within about kZeroNats / d chunks: the expected cost counts `trans` chunks for both (the
// planner's estimate from the decay probe), the full cost (no transition vanishes) the whole
// segment.  A pass on `slots` concurrent workgroups takes at least its longest workgroup, at least
// its total work / slots and, where more than `slots` segment workgroups of about the candidate
// length run in pass 1, at least two of them in a row.
constexpr int64_t kTransSteps = 8;          // the host's estimate (it cannot see g)
constexpr double kZeroNats = 140 * 0.6931471805599453;   // ln 2^140
struct SplitCost {
    double work1 = 0, work2 = 0;     // per head, expected
    double work1f = 0, work2f = 0;   // per head, if no transition reaches zero
    double big = 0;                  // per head: pass-1 segment workgroups of >= 0.9 of the candidate
    int64_t crit1 = 0, crit2 = 0, crit2f = 0;
    int64_t summaries = 0;           // per head
};
__host__ __device__ inline int64_t chunks_of(int64_t x) { return (x + 31) / 32; }
__host__ __device__ inline int64_t min_i64(int64_t a, int64_t b) { return a < b ? a : b; }
__host__ __device__ inline int64_t max_i64(int64_t a, int64_t b) { return a > b ? a : b; }
// segments of one sequence for the segment length L (L <= 0: whole), at most Pmax of them
__host__ __device__ inline void split_of(int64_t len, int64_t L, int Pmax, int& P, int64_t& Ls) {
    if (L <= 0 || len <= L) {
        P = 1;
        Ls = len;
        return;
    }
    int64_t p = (len + L - 1) / L;
    Ls = L;
    if (p > Pmax) {
        p = Pmax;
        Ls = ((len + p - 1) / p + 31) / 32 * 32;
    }
    P = (int)p;
}
// Adds one sequence of len tokens cut into P segments of Ls tokens (candidate length L).
__host__ __device__ inline void split_add(SplitCost& c, int64_t len, int P, int64_t Ls, int64_t L, int nsl,
                                          int nslt, bool eager, int64_t trans) {
    if (P <= 1) {
        const double w = (double)nsl * chunks_of(len);
        c.work1 += w;
        c.work1f += w;
        c.crit1 = max_i64(c.crit1, chunks_of(len));
        return;
    }
    const int64_t ch = chunks_of(Ls), chl = chunks_of(max_i64(0, len - (int64_t)(P - 1) * Ls));   // full, last
    const int ntsl = nslt - nsl;
    const int64_t e = min_i64(ch, trans), el = min_i64(chl, trans);
    const double comp = (double)P * (P - 1) / 2;   // summaries composed by segments 1 .. P - 1
    const int64_t tall = chunks_of(L) * 9 / 10;
    c.crit1 = max_i64(c.crit1, ch);
    c.summaries += P - 1;
    if (eager) {
        const double value = (double)nsl * ((double)(P - 1) * ch + chl);
        c.work1 += value + (double)ntsl * ((double)(P - 2) * e + el);
        c.work1f += value + (double)ntsl * ((double)(P - 2) * ch + chl);
        c.work2 += (double)nsl * ((double)(P - 2) * e + el + comp);
        c.work2f += (double)nsl * ((double)(P - 2) * ch + chl + comp);
        c.crit2 = max_i64(c.crit2, e + P - 1);
        c.big += (double)nsl * ((ch >= tall ? P - 1 : 0) + (chl >= tall ? 1 : 0));
    } else {
        const double value = (double)nsl * (P - 1) * ch;
        c.work1 += value + (double)ntsl * (P - 2) * e;
        c.work1f += value + (double)ntsl * (P - 2) * ch;
        c.work2 += (double)nsl * ((double)(P - 2) * e + chl + comp);
        c.work2f += (double)nsl * ((double)(P - 2) * ch + chl + comp);
        c.crit2 = max_i64(c.crit2, max_i64(e + P - 2, chl + P - 1));
        c.big += (double)nsl * (ch >= tall ? P - 1 : 0);
    }
    c.crit2f = max_i64(c.crit2f, ch + P - 1);
}
// The same for n sequences alike.
__host__ __device__ inline void split_times(SplitCost& c, double n) {
    c.work1 *= n;
    c.work2 *= n;
    c.work1f *= n;
    c.work2f *= n;
    c.big *= n;
    c.summaries = (int64_t)(c.summaries * n);
}
__host__ __device__ inline double split_pass(double crit, double work, int H, int slots) {
    const double w = work * H / slots;
    return crit > w ? crit : w;
}
// Expected (full = false) or worst-case (full = true) time of a plan, for the candidate L.
__host__ __device__ inline double split_makespan(const SplitCost& c, int64_t L, int H, int slots, bool full) {
    double m1 = split_pass((double)c.crit1, full ? c.work1f : c.work1, H, slots);
    if (c.summaries) {
        const double rounds = (double)(int64_t)((c.big * H + slots - 1) / slots);
        const double r = rounds * (double)(chunks_of(L) * 9 / 10);
        m1 = m1 > r ? m1 : r;
    }
    const double m2 = c.summaries ? (full ? split_pass((double)c.crit2f, c.work2f, H, slots)
                                          : split_pass((double)c.crit2, c.work2, H, slots))
                                  : 0.0;
    return m1 + m2;
}
// The candidate segment length that cuts a sequence of `longest` tokens into P pieces (whole
// chunks); the planners try P = 2 .. Pmax for the longest sequence of the batch.
__host__ __device__ inline int64_t split_candidate(int64_t longest, int P) {
    return ((longest + P - 1) / P + 31) / 32 * 32;
}
// A split must beat the whole-sequence schedule by this factor (extra launch, rough chain cost).
constexpr double kSplitGain = 0.95;
// Packed batches are planned on the device up to this many sequences (one workgroup prices them).
constexpr int32_t kPlanMaxSeqs = 65536;
// ... and only when their whole-sequence grid (N H dv / 64 workgroups) is at most kPlanWgsPerCu
// per compute unit: the planned launches carry a grid sized for the largest plan, whose unused
// workgroups pass through the dispatcher, while a batch that many times the GPU's size is rarely
// bound by one sequence's chain.
constexpr int32_t kPlanWgsPerCu = 16;
__host__ __device__ inline bool plan_packed(int32_t N, int32_t H, int32_t dv, int slots) {
    return N <= kPlanMaxSeqs && (int64_t)N * H * (dv / 64) <= (int64_t)kPlanWgsPerCu * slots;
}
// Limits of the automatic plan on a GPU with `slots` concurrent workgroups: segments per
// sequence, the shortest segment, and the number of summaries the workspace holds per head.
struct SplitLimits {
    int Pmax = 1;
    int64_t Lmin = 0;
    int64_t Smax = 0;
};
__host__ __device__ inline SplitLimits split_limits(int32_t N, int64_t total, int32_t H, int32_t dv, int slots) {
    SplitLimits l;
    const int64_t units = (int64_t)H * (dv / 64);
    int64_t p = (2 * (int64_t)slots + units - 1) / units;
    l.Pmax = (int)(p < 1 ? 1 : (p > 16 ? 16 : p));
    int64_t lm = ((total + 63) / 64 + 31) / 32 * 32;
    l.Lmin = lm < 1024 ? 1024 : lm;
    const int64_t s1 = (int64_t)N * (l.Pmax - 1), s2 = total / l.Lmin;
    l.Smax = s1 < s2 ? s1 : s2;
    if (l.Pmax <= 1 || total >= ((int64_t)1 << 31)) l.Smax = 0;
    return l;
}
// Whether a split in time can pay for N sequences of T tokens in either layout (the device
// planner makes the choice).
bool split_may_pay(int32_t N, int64_t T, int32_t H, int32_t dk, int32_t dv, int slots);
// The device planner (a decay probe over 8 chunks of the batch, then one workgroup), writing the
// plan laid out as PlanLayout{N, lim.Smax}.  a supplies g, cu (or fixed rows of T tokens), N, T, H,
// dk, dv and the stream.
hipError_t launch_plan(const PrefillArgs& a, int32_t* plan, int slots, SplitLimits lim);
// ok = every g[i], i < n, lies in [lo, hi] (NaN does not); synchronises `stream`
hipError_t check_range(const float* g, size_t n, float lo, float hi, hipStream_t stream, bool& ok);
// ok = cu[0] == 0, cu non-decreasing, cu[N] == T (the N + 1 packed-sequence offsets); synchronises
hipError_t check_offsets(const int32_t* cu, int32_t N, int64_t T, hipStream_t stream, bool& ok);
hipError_t launch_decode_step(const DecodeArgs& a);

}  // namespace kda
