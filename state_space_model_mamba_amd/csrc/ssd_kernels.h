// Internal launchers of libssd (not part of the C ABI; see include/ssd.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace ssd {

// Up to this many HIP events bracket the kernels of one scan (timed entry point).
constexpr int kMaxTimedKernels = 8;

struct EventLog {
    hipEvent_t ev[kMaxTimedKernels + 1];
    const char *name[kMaxTimedKernels];
    int n = 0;          // kernels recorded
    bool on = false;    // record events around launches
};

// Record the start event before the first kernel and one event after each kernel.
hipError_t log_begin(EventLog *log, hipStream_t s);
hipError_t log_kernel(EventLog *log, const char *name, hipStream_t s);

// Step-size prep fused into the kernels: with softplus set, the dt argument
// holds u and the step size of head h is softplus(u + bias[h]) (bias NULL: 0),
// evaluated in fp32 as max(v, 0) + log1p(exp(-|v|)), which neither overflows
// for large v nor loses the small values of very negative v.  With
// w = fl(1 + e), log1p(e) = log(w) - log(w / (1 + e)), and the rounding error
// d = (w - 1) - e is exact in fp32 (w - 1 is exact for w in [1, 2], and so is
// the difference of the two nearby values), so log1p(e) = log(w) - d / (1 + e)
// to first order in d.  Dropping the 1 / (1 + e) changes the result by at most
// |d| e <= 2^-24 e, i.e. 2^-24 of log1p(e) ~ e: no reciprocal, and w = 1
// (e below 2^-24) needs no branch (d = -e).  The exp and log are the hardware
// exp2 / log2 (log(w) = log2(w) ln 2; w in [1, 2] needs none of the denormal
// handling of the library log).  Positions past the end of a sequence keep a
// step size of 0.
struct DtPrep {
    const float *bias;
    int softplus;
};

__device__ __forceinline__ float softplus_dt(float u, float bias)
{
    const float v = u + bias;
    const float e = __expf(-fabsf(v));   // (0, 1]
    const float w = 1.f + e;             // [1, 2]: no denormal handling needed
    const float d = (w - 1.f) - e;       // the rounding error of 1 + e, exactly
    return fmaxf(v, 0.f) + (__builtin_amdgcn_logf(w) * 0.6931471806f - d);
}

// Sum of a wave value with its partner lane across lane bit 4 or 5 (the lane
// 16 or 32 away), every lane keeping the sum: one permlane swap and one add.
// When one instruction read both results of the swap builtin directly, hipcc
// (ROCm 7.2) emitted it reading the first result twice; passing the second
// through an empty asm statement keeps them apart.
__device__ __forceinline__ float swap_sum(unsigned first, unsigned second)
{
    asm volatile("" : "+v"(second));
    return __builtin_bit_cast(float, first) + __builtin_bit_cast(float, second);
}
template <int kBit>
__device__ __forceinline__ float lane_pair_sum(float v)
{
    static_assert(kBit == 4 || kBit == 5, "lane bit 4 or 5");
    const unsigned u = __builtin_bit_cast(unsigned, v);
    const auto s = kBit == 5 ? __builtin_amdgcn_permlane32_swap(u, u, false, false)
                             : __builtin_amdgcn_permlane16_swap(u, u, false, false);
    return swap_sum(s[0], s[1]);
}

// state[i] = src ? src[i] : 0 for i < n (fill/copy kernel, graph-capturable).
hipError_t launch_state_init(float *state, const float *src, int64_t n, hipStream_t s);

// One decode step over B*H (batch row, head) pairs; io is bf16 when bf16 != 0.
hipError_t launch_decode(int bf16, int64_t B, int64_t H, int64_t P, int64_t N, int64_t G,
                         const void *x, const float *dt, const float *A, const void *Bm,
                         const void *Cm, const float *D, float *state, void *y, DtPrep prep,
                         hipStream_t s);

// S consecutive decode steps in one launch (state kept in registers across
// them); x, y [S, B, H, P], dt [S, B, H], B/C [S, B, G, N].
hipError_t launch_decode_steps(int bf16, int64_t S, int64_t B, int64_t H, int64_t P, int64_t N,
                               int64_t G, const void *x, const float *dt, const float *A,
                               const void *Bm, const void *Cm, const float *D, float *state,
                               void *y, DtPrep prep, hipStream_t s);

// Gated DeltaNet decode step over B x Hv value heads: q, k [B, Hk, dk],
// v, o [B, Hv, dv], g, beta [B, Hv], state [B, Hv, dk, dv] (updated in place).
hipError_t launch_gdn_decode(int bf16, int64_t B, int64_t Hk, int64_t Hv, int64_t dk, int64_t dv,
                             const void *q, const void *k, const void *v, const float *g,
                             const float *beta, float *state, void *o, hipStream_t s);

// S Gated DeltaNet steps in one launch, the state held in registers across
// them: q, k [S, B, Hk, dk], v, o [S, B, Hv, dv], g, beta [S, B, Hv].
hipError_t launch_gdn_decode_steps(int bf16, int64_t S, int64_t B, int64_t Hk, int64_t Hv,
                                   int64_t dk, int64_t dv, const void *q, const void *k,
                                   const void *v, const float *g, const float *beta, float *state,
                                   void *o, hipStream_t s);

// fp32 chunked scan (VALU), P <= 64, N <= 128, Q <= 256.
hipError_t launch_scan_f32(int64_t B, int64_t L, int64_t H, int64_t P, int64_t N, int64_t G,
                           int64_t Q, const float *x, const float *dt, const float *A,
                           const float *Bm, const float *Cm, const float *D, const float *init,
                           float *y, float *fin, DtPrep prep, hipStream_t s, EventLog *log);

// bf16 MFMA chunked scan, P = 64, N = 128, Q % 64 == 0, Q <= 512.
// The workspace holds the segment states and their decays.
struct Bf16Plan {
    int64_t nchunks;       // ceil(L / Q)
    int64_t quads;         // work-groups per (batch row, segment): G * ceil(H / G / 4)
    int64_t chunks_per_seg;  // ceil(seg_tokens / Q), for reports
    int64_t seg_tokens;    // tokens per segment (a multiple of 64; the last may be shorter)
    int64_t nseg;          // segments per (b, h) of the scan kernel
    int64_t nsub;          // state-kernel units per segment (each segment but the last)
    int64_t unit_tokens;   // tokens per unit (a multiple of 64)
    int64_t nslot;         // state slots per (b, h): one per unit + one spare (0 if nseg == 1)
    size_t state_bytes;    // B*H*nslot*P*N*4
    size_t decay_bytes;    // B*H*nslot*4
    size_t ws_bytes;       // total workspace
};
// cus: the CUs the problem may count on (fewer when it shares a launch);
// nseg > 0 fixes the segment count.  With use_env the SSD_NSEG / SSD_NSUB
// environment variables, when set, override the segment and unit counts.
Bf16Plan plan_scan_bf16(int64_t B, int64_t L, int64_t H, int64_t G, int64_t Q, int64_t cus = 256,
                        int64_t nseg = 0, bool use_env = true);

hipError_t launch_scan_bf16(const Bf16Plan &plan, int64_t B, int64_t L, int64_t H, int64_t G,
                            int64_t Q, const void *x, const float *dt, const float *A,
                            const void *Bm, const void *Cm, const float *D, const float *init,
                            void *y, float *fin, void *ws, DtPrep prep, hipStream_t s,
                            EventLog *log);

// Up to kMaxRuns independent bf16 scans (batch B, length L > 0 each; same H, G,
// Q, A, D, step-size prep) in one state-kernel and one scan-kernel launch.
constexpr int kMaxRuns = 8;
struct Bf16Run {
    Bf16Plan plan;
    int64_t B, L;
    const void *x;
    const float *dt;
    const void *Bm, *Cm;
    const float *init;
    void *y;
    float *fin;
    void *ws;   // plan.ws_bytes of workspace for this run
};
hipError_t launch_scan_bf16_multi(const Bf16Run *runs, int nruns, int64_t H, int64_t G, int64_t Q,
                                  const float *A, const float *D, DtPrep prep, hipStream_t s);

}  // namespace ssd
