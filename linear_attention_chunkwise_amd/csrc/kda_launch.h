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
};

// Layout of a device plan (int32), for N sequences and at most Smax summaries:
//   [0] segment length (0: no split), [1] items of pass 1, [2] items of pass 2, [3] unused,
//   segs[N], first summary[N], segment length[N] per sequence,
//   pass-1 items [N + Smax] x {sequence, segment}: the summaries of the split sequences and the
//   whole runs of the others, longest sequences first,
//   pass-2 items [N + Smax] x {sequence, segment}: the segments after the first of the split
//   sequences (the first segment writes its outputs in pass 1), then the whole runs moved into
//   the second pass's idle slots.
struct PlanLayout {
    int32_t N, Smax;
    __host__ __device__ int64_t segs() const { return 4; }
    __host__ __device__ int64_t first() const { return 4 + (int64_t)N; }
    __host__ __device__ int64_t seglen() const { return 4 + 2 * (int64_t)N; }
    __host__ __device__ int64_t items1() const { return 4 + 3 * (int64_t)N; }
    __host__ __device__ int64_t items2() const { return items1() + 2 * ((int64_t)N + Smax); }
    __host__ __device__ int64_t ints() const { return items2() + 2 * ((int64_t)N + Smax); }
    __host__ __device__ int32_t max_items1() const { return N + Smax; }
    __host__ __device__ int32_t max_items2() const { return N + Smax; }
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
// whole costs nsl workgroups x ceil(len / 32) steps, in pass 1 (beside the summaries) unless the
// plan moves it into pass 2 (below).  Split into P segments of Ls tokens it costs, in pass 1,
// nsl x ceil(Ls / 32) for its first segment (its outputs and the summary of its value columns)
// and nslt x ceil(Ls / 32) for each of the
// next P - 2 (value and transition columns; the transition workgroups stop early once their
// columns are exactly zero, which the model does not count on), and in pass 2
// nsl x (ceil(Ls_j / 32) + j) for segment j >= 1 (its tokens and the j summaries it composes).
// A pass on `slots` concurrent workgroups takes at least its longest workgroup and at least its
// total work / slots; a plan is priced at the sum of the two passes' bounds.  Where the second
// pass leaves slots idle (slots x its longest workgroup above its work), sequences left whole
// run there instead of in the first pass, up to the idle capacity: each is no longer than the
// segment length, so it fits under the second pass's longest workgroup.
struct SplitCost {
    double work1 = 0, work2 = 0;   // per head
    double whole = 0;              // per head: the part of work1 in sequences left whole
    int64_t crit1 = 0, crit2 = 0;
    int64_t summaries = 0;         // per head
};
__host__ __device__ inline int64_t chunks_of(int64_t x) { return (x + 31) / 32; }
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
__host__ __device__ inline void split_add(SplitCost& c, int64_t len, int P, int64_t Ls, int nsl, int nslt) {
    if (P <= 1) {
        c.work1 += (double)nsl * chunks_of(len);
        c.whole += (double)nsl * chunks_of(len);
        c.crit1 = c.crit1 > chunks_of(len) ? c.crit1 : chunks_of(len);
        return;
    }
    const int64_t ch = chunks_of(Ls);
    c.work1 += (double)ch * (nsl + (double)nslt * (P - 2));
    c.crit1 = c.crit1 > ch ? c.crit1 : ch;
    c.work2 += (double)nsl * ((double)(chunks_of(len) - ch) + (double)P * (P - 1) / 2);
    c.crit2 = c.crit2 > ch + P - 1 ? c.crit2 : ch + P - 1;
    c.summaries += P - 1;
}
// The idle capacity of the second pass, in work per head (0 without a split).
__host__ __device__ inline double split_idle2(const SplitCost& c, int H, int slots) {
    if (!c.summaries) return 0.0;
    const double idle = (double)slots * (double)c.crit2 / H - c.work2;
    return idle > 0.0 ? idle : 0.0;
}
__host__ __device__ inline double split_makespan(const SplitCost& c, int H, int slots) {
    const double idle = split_idle2(c, H, slots);
    const double x = c.whole < idle ? c.whole : idle;
    const double w1 = (c.work1 - x) * H / slots, w2 = (c.work2 + x) * H / slots;
    const double m1 = (double)c.crit1 > w1 ? (double)c.crit1 : w1;
    const double m2 = c.summaries ? ((double)c.crit2 > w2 ? (double)c.crit2 : w2) : 0.0;
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
// The whole-sequence plan for N sequences of T tokens: the segment count (1: no split).
int32_t plan_fixed_segments(int32_t N, int64_t T, int32_t H, int32_t dk, int32_t dv, int slots);
// The device planner for packed sequences (one workgroup), writing the plan laid out as
// PlanLayout{N, lim.Smax}.  a supplies cu, N, T, H, dk, dv and the stream.
hipError_t launch_plan(const PrefillArgs& a, int32_t* plan, int slots, SplitLimits lim);
// ok = every g[i], i < n, lies in [lo, hi] (NaN does not); synchronises `stream`
hipError_t check_range(const float* g, size_t n, float lo, float hi, hipStream_t stream, bool& ok);
// ok = cu[0] == 0, cu non-decreasing, cu[N] == T (the N + 1 packed-sequence offsets); synchronises
hipError_t check_offsets(const int32_t* cu, int32_t N, int64_t T, hipStream_t stream, bool& ok);
hipError_t launch_decode_step(const DecodeArgs& a);

}  // namespace kda
