// S consecutive cached decode steps in one launch, the state held in
// registers across all of them.
//
// "Compiler-First State Space Duality and Portable O(1) Autoregressive
// Caching for Inference", section 2: generation runs as a loop compiled onto
// the device around the fixed-size state cache, with no host round trip per
// step.  "A Persistent-State Dataflow Accelerator for Memory-Bound Linear
// Attention Decode on FPGA", section 2A: a recurrent state that stays on-chip
// across decode steps is no longer re-read from external memory, which turns
// decode from memory-bound into compute-bound.  Here each wave loads its rows
// of the state once, advances them through every step of the recurrence of
// ssd_decode_step,
//     alpha = exp(dt A_h);  H <- alpha H + (dt x) (outer) B_g;  y = H . C_g + D_h x,
// and stores them once.  Per step only that step's x, dt, B, C come in and y
// goes out, so the work is fp32 VALU arithmetic on registers.
//
// Layout of a wave: a state row (N floats) is spread over LPR lanes with
// CPL = N / LPR consecutive columns each: LPR = 16 (one DPP row) for
// N <= 128, LPR = 64 for N = 256.  A wave holds RPW = 64 / LPR row groups of
// R rows, so every lane owns R x CPL state elements.  The reduction of y over
// n is done per lane over its CPL columns, then across the LPR lanes of a row
// group without going through LDS: first log2(R) halving exchanges
// (permlane32 / permlane16 swaps, then DPP mirrors and quad permutations),
// each of which leaves a lane with half as many rows summed over twice as
// many lanes, then plain DPP sums over the remaining lane bits.  Afterwards
// the lanes of row group `grp` with lane-in-row index lr hold the full sum
// for row slot lr >> SHIFT.  Fewer lanes per row make that reduction short
// (4 exchanges for 4 rows over 16 lanes, against 35 instructions for 16 rows
// over 64 lanes) at the price of unpacking more B and C values per lane.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "ssd_kernels.h"

namespace ssd {
namespace {

constexpr int kStepsThreads = 256;   // four independent waves per work-group

template <int N, int CPL, int R>
struct StepsGeom {
    static constexpr int LPR = N / CPL;            // lanes per state row
    static constexpr int RPW = 64 / LPR;           // row groups per wave
    static constexpr int LOG_LPR = __builtin_ctz(LPR);
    static constexpr int HALVE = __builtin_ctz(R); // halving exchanges of the y reduction
    static constexpr int SHIFT = LOG_LPR - HALVE;  // a row's sum ends on 1 << SHIFT lanes
    static constexpr int ROWS = R * RPW;           // state rows per wave
    static_assert(LPR == 16 || LPR == 64, "a row spans one DPP row or the whole wave");
    static_assert((R & (R - 1)) == 0 && R >= 1 && R <= LPR, "R: power of two <= LPR");
};

typedef __amdgpu_buffer_rsrc_t rsrc_t;
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// Raw buffer resource over `bytes` bytes at `base` (gfx9-family data word):
// loads past the end return zero and stores there are dropped, so a step past
// the last one (bytes = 0) or a row past P costs no branch.
__device__ __forceinline__ rsrc_t buf(const void *base, int bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, bytes, 0x00020000);
}

// kBytes (2, 4, 8, 16 or 32) bytes at byte offset off, as raw 32-bit words.
template <int kBytes>
struct Raw {
    static constexpr int W = kBytes < 4 ? 1 : kBytes / 4;
    unsigned w[W];
};

template <int kBytes>
__device__ __forceinline__ Raw<kBytes> load_raw(rsrc_t r, unsigned off);

template <int kBytes>
__device__ __forceinline__ Raw<kBytes> load_raw(rsrc_t r, unsigned off)
{
    Raw<kBytes> v;
    if constexpr (kBytes == 2) {
        v.w[0] = __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
    } else if constexpr (kBytes == 4) {
        v.w[0] = __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
    } else if constexpr (kBytes == 8) {
        const u32x2 t = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
        v.w[0] = t[0];
        v.w[1] = t[1];
    } else if constexpr (kBytes == 16) {
        const u32x4 t = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i)
            v.w[i] = t[i];
    } else {
        static_assert(kBytes == 32, "2, 4, 8, 16 or 32 bytes");
        const u32x4 t0 = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
        const u32x4 t1 = __builtin_amdgcn_raw_buffer_load_b128(r, off + 16, 0, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v.w[i] = t0[i];
            v.w[4 + i] = t1[i];
        }
    }
    return v;
}

// Element i of K consecutive io values held as raw words, widened to fp32.
template <typename T, int K, int kBytes>
__device__ __forceinline__ float elem(const Raw<kBytes> &v, int i)
{
    if constexpr (sizeof(T) == 2) {
        const unsigned w = v.w[i / 2];
        return __builtin_bit_cast(float, (i & 1) ? (w & 0xffff0000u) : (w << 16));
    } else {
        return __builtin_bit_cast(float, v.w[i]);
    }
}

template <typename T> __device__ __forceinline__ void store_y(rsrc_t r, unsigned off, float v);
template <> __device__ __forceinline__ void store_y<float>(rsrc_t r, unsigned off, float v)
{
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, v), r, off, 0, 0);
}
template <> __device__ __forceinline__ void store_y<__bf16>(rsrc_t r, unsigned off, float v)
{
    __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, (__bf16)v), r, off, 0, 0);
}

template <int kCtrl>
__device__ __forceinline__ float dpp(float v)
{
    return __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), kCtrl, 0xf, 0xf, true));
}

// Lane kLane of each 16-lane row, broadcast to the row (gfx90a+ DPP row_newbcast).
template <int kLane>
__device__ __forceinline__ float row_bcast(float v)
{
    return dpp<0x150 + kLane>(v);
}

// DPP control of the exchange partner for lane bits 0..3: quad permutations
// [1,0,3,2] and [2,3,0,1], the half-row mirror (lane ^ 7) and the row mirror
// (lane ^ 15).  Each partner differs in the named bit and in no higher one.
template <int kBit>
__device__ __forceinline__ float partner(float v)
{
    if constexpr (kBit == 0)
        return dpp<0xB1>(v);
    else if constexpr (kBit == 1)
        return dpp<0x4E>(v);
    else if constexpr (kBit == 2)
        return dpp<0x141>(v);
    else
        return dpp<0x140>(v);
}

// Halving exchange on lane bit kBit: a lane whose bit is 0 keeps row `lo`,
// one whose bit is 1 keeps `hi`, each summed with the partner lane's value.
template <int kBit>
__device__ __forceinline__ float halve(float lo, float hi, int lane)
{
    if constexpr (kBit >= 4) {
        const u32x2 s = kBit == 5
            ? __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, lo),
                                               __builtin_bit_cast(unsigned, hi), false, false)
            : __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(unsigned, lo),
                                               __builtin_bit_cast(unsigned, hi), false, false);
        return swap_sum(s[0], s[1]);   // (ssd_kernels.h)
    } else {
        const bool up = (lane >> kBit) & 1;
        const float mine = up ? hi : lo, send = up ? lo : hi;
        return mine + partner<kBit>(send);
    }
}

// Plain sum with the partner lane on bit kBit (all lanes keep the sum).
template <int kBit>
__device__ __forceinline__ float pair_sum(float v)
{
    if constexpr (kBit >= 4) {
        return lane_pair_sum<kBit>(v);
    } else {
        return v + partner<kBit>(v);
    }
}

template <class Gm, int kStep, int R>
__device__ __forceinline__ void halvings(float (&v)[R], int lane)
{
    if constexpr (kStep < Gm::HALVE) {
        constexpr int half = (R >> kStep) / 2;
#pragma unroll
        for (int j = 0; j < half; ++j)
            v[j] = halve<Gm::LOG_LPR - 1 - kStep>(v[j], v[j + half], lane);
        halvings<Gm, kStep + 1>(v, lane);
    }
}

template <int kBit, int kEnd>
__device__ __forceinline__ float pair_sums(float v)
{
    if constexpr (kBit < kEnd)
        return pair_sums<kBit + 1, kEnd>(pair_sum<kBit>(v));
    else
        return v;
}

// Sum of v[s] over the LPR lanes of each row group, transposed: returns the
// total of row slot (lane % LPR) >> SHIFT of the lane's group.
template <class Gm, int R>
__device__ __forceinline__ float reduce_rows(float (&v)[R], int lane)
{
    halvings<Gm, 0>(v, lane);
    return pair_sums<0, Gm::SHIFT>(v[0]);
}

// u[s] = v of lane s << SHIFT of the lane's row group, s < R.
template <class Gm, int kS, int R>
__device__ __forceinline__ void bcast_rows(float (&u)[R], float v)
{
    if constexpr (kS < R) {
        if constexpr (Gm::LPR == 64)
            u[kS] = __builtin_bit_cast(
                float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), kS << Gm::SHIFT));
        else
            u[kS] = row_bcast<(kS << Gm::SHIFT)>(v);
        bcast_rows<Gm, kS + 1>(u, v);
    }
}

// The inputs of one decode step as this lane needs them.
template <typename T, int CPL>
struct StepIn {
    Raw<sizeof(T)> x;          // x of the lane's reduced row
    Raw<4> dt;                 // dt of the (b, h) pair
    Raw<CPL * sizeof(T)> B, C; // the lane's CPL columns of B_g and C_g
};

// One work-group = four waves, each an independent block of ROWS state rows of
// one (batch row, head); `wpb` waves cover the P rows of a pair.
// Waves per SIMD the compiler must leave room for: the bf16 kernels are held
// to three (168 registers) so that the large row blocking still overlaps three
// waves on a SIMD; the fp32 ones keep their larger prefetch ring in registers.
template <typename T>
constexpr int kStepsMinWaves = sizeof(T) == 2 ? 3 : 1;

// kSp: the dt inputs hold u and the step size is softplus(u + bias[h]).
template <typename T, int N, int CPL, int R, bool kSp>
__global__ __attribute__((amdgpu_flat_work_group_size(1, kStepsThreads),
                          amdgpu_waves_per_eu(kStepsMinWaves<T>))) void decode_steps_kernel(
    int S, int Bn, int H, int P, int G, int wpb, const T *__restrict__ x,
    const float *__restrict__ dt, const float *__restrict__ A, const T *__restrict__ Bm,
    const T *__restrict__ Cm, const float *__restrict__ D, float *__restrict__ state,
    T *__restrict__ y, const float *__restrict__ dt_bias)
{
    using Gm = StepsGeom<N, CPL, R>;
    constexpr int esz = (int)sizeof(T);
    const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x / 64);
    const int lane = (int)threadIdx.x % 64;
    const int gw = (int)blockIdx.x * (kStepsThreads / 64) + wave;
    const int bh = gw / wpb;
    if (bh >= Bn * H)
        return;
    const int p0 = (gw - bh * wpb) * Gm::ROWS;
    const int b = bh / H, h = bh - b * H, g = h / (H / G);
    const int grp = lane / Gm::LPR, lr = lane % Gm::LPR;
    const int rbase = p0 + grp * R;               // first state row of the lane's group
    const int myrow = rbase + (lr >> Gm::SHIFT);  // row whose y this lane holds
    const float Ah = A[h], Dh = D[h];
    const float dtb = kSp && dt_bias ? dt_bias[h] : 0.f;

    // the lane's R x CPL state elements, loaded once
    float st[R][CPL];
    float *sp = state + (int64_t)bh * P * N + CPL * lr;
#pragma unroll
    for (int s = 0; s < R; ++s) {
        const int row = rbase + s;
        if (row < P) {
#pragma unroll
            for (int k = 0; k < CPL; ++k)
                st[s][k] = sp[(int64_t)row * N + k];
        } else {
#pragma unroll
            for (int k = 0; k < CPL; ++k)
                st[s][k] = 0.f;
        }
    }

    const int64_t xstep = (int64_t)Bn * H * P, bstep = (int64_t)Bn * G * N, dstep = (int64_t)Bn * H;
    const T *xb = x + (int64_t)bh * P;
    const float *db = dt + bh;
    const T *bb = Bm + (int64_t)(b * G + g) * N;
    const T *cb = Cm + (int64_t)(b * G + g) * N;
    T *yb = y + (int64_t)bh * P;
    const unsigned xoff = (unsigned)myrow * esz, boff = (unsigned)(CPL * lr * esz);
    // a lane that does not write y points past the end of the step's row
    const bool writer = (lr & ((1 << Gm::SHIFT) - 1)) == 0;
    const unsigned yoff = writer ? xoff : 0x7fffffffu;

    // Running pointers at the next step to issue.  A checked issue may be past
    // the last step: its pointers stay at the last step and its resources are
    // empty (its loads read zeros); an unchecked one is known to be in range.
    const T *xi = xb, *bi = bb, *ci = cb;
    const float *di = db;
    int ti = 0;
    auto issue = [&](StepIn<T, CPL> &in, auto checked) {
        bool ok = true, more = true;
        if constexpr (decltype(checked)::value) {
            ok = ti < S;
            more = ti + 1 < S;
        }
        in.x = load_raw<esz>(buf(xi, ok ? P * esz : 0), xoff);
        in.dt = load_raw<4>(buf(di, ok ? 4 : 0), 0);
        in.B = load_raw<CPL * esz>(buf(bi, ok ? N * esz : 0), boff);
        in.C = load_raw<CPL * esz>(buf(ci, ok ? N * esz : 0), boff);
        xi = more ? xi + xstep : xi;
        di = more ? di + dstep : di;
        bi = more ? bi + bstep : bi;
        ci = more ? ci + bstep : ci;
        ++ti;
    };
    using checked_t = std::integral_constant<bool, true>;
    using unchecked_t = std::integral_constant<bool, false>;

    // With the large row blocking (throughput-bound; 16 or more state elements
    // per lane) the lanes keep H / sc, sc
    // being the product of the decays since the last renormalisation (the
    // same on every lane of the wave), so that a step is one fused
    // multiply-add per element: H/sc' += (dt x / sc') B with sc' = sc alpha,
    // and y = sc' (H/sc' . C) + D x.  A step that would take sc outside
    // [2^-64, 2^64] (alpha = 0 included) instead multiplies the state by sc
    // and alpha and restarts sc at 1.  1 / sc' is the hardware reciprocal
    // (within 1 ulp).  The small blocking runs one wave per SIMD and is bound
    // by the latency of a step, so it applies alpha directly (two operations
    // per element, none of the bookkeeping).
    constexpr bool kLazy = R * CPL >= 16;
    float sc = 1.f;
    T *yp = yb;   // y of the step being computed
    auto step = [&](const StepIn<T, CPL> &in) {
        const float xv = elem<T, 1>(in.x, 0);
        float d = elem<float, 1>(in.dt, 0);
        if constexpr (kSp)
            d = softplus_dt(d, dtb);
        const float alpha = __expf(d * Ah);
        float ux = d * xv, scn = 1.f;
        if constexpr (kLazy) {
            scn = sc * alpha;
            if (__builtin_amdgcn_readfirstlane(!(scn >= 0x1p-64f && scn <= 0x1p64f))) {
#pragma unroll
                for (int s = 0; s < R; ++s)
#pragma unroll
                    for (int k = 0; k < CPL; ++k)
                        st[s][k] = st[s][k] * sc * alpha;
                scn = 1.f;
            }
            sc = scn;
            ux *= __builtin_amdgcn_rcpf(scn);
        }
        // dt x (/ sc) of row slot s of this lane's group, held by the group's
        // lane s << SHIFT: a readlane when a row spans the wave, a DPP row
        // broadcast when it spans a 16-lane row
        float u[R];
        bcast_rows<Gm, 0>(u, ux);
        float part[R];
#pragma unroll
        for (int s = 0; s < R; ++s) {
            float acc = 0.f;
#pragma unroll
            for (int k = 0; k < CPL; ++k) {
                const float o = kLazy ? __builtin_fmaf(u[s], elem<T, CPL>(in.B, k), st[s][k])
                                      : alpha * st[s][k] + u[s] * elem<T, CPL>(in.B, k);
                st[s][k] = o;
                acc = k == 0 ? o * elem<T, CPL>(in.C, k) : acc + o * elem<T, CPL>(in.C, k);
            }
            part[s] = acc;
        }
        const float sum = reduce_rows<Gm>(part, lane);
        const float yv = (kLazy ? sum * scn : sum) + Dh * xv;
        store_y<T>(buf(yp, P * esz), yoff, yv);
        yp += xstep;
    };

    // Inputs are issued kStepsAhead steps ahead of the one computed: a ring of
    // loads in flight.  Groups of steps whose issues all stay in range run
    // unchecked.  Four steps ahead cover the memory latency of a wave that is
    // alone on its SIMD (small blocking); with the large blocking three waves
    // share a SIMD, and two steps ahead, with fewer registers, measured ~3%
    // faster.
    constexpr int kStepsAhead = kLazy ? 2 : 4;
    StepIn<T, CPL> ring[kStepsAhead];
#pragma unroll
    for (int k = 0; k < kStepsAhead; ++k)
        issue(ring[k], checked_t{});
    int t0 = 0;
    // a slot is refilled right after the step that consumed it, so the loads
    // land in the registers it frees (no copies around the loop)
    for (; t0 + 2 * kStepsAhead <= S; t0 += kStepsAhead) {
#pragma unroll
        for (int k = 0; k < kStepsAhead; ++k) {
            step(ring[k]);
            issue(ring[k], unchecked_t{});
        }
    }
    if (t0 + kStepsAhead <= S) {
#pragma unroll
        for (int k = 0; k < kStepsAhead; ++k) {
            step(ring[k]);
            issue(ring[k], checked_t{});
        }
        t0 += kStepsAhead;
    }
#pragma unroll
    for (int k = 0; k < kStepsAhead - 1; ++k)
        if (t0 + k < S)
            step(ring[k]);

#pragma unroll
    for (int s = 0; s < R; ++s) {
        const int row = rbase + s;
        if (row < P) {
#pragma unroll
            for (int k = 0; k < CPL; ++k)
                sp[(int64_t)row * N + k] = st[s][k] * sc;
        }
    }
}

// Layouts: a state row spans one 16-lane DPP row (CPL = N / 16 columns per
// lane) for N <= 128, the whole wave for N = 256.  Rows per lane: the larger
// choice keeps 32 state elements per lane (16 for N = 16); the smaller one, a
// quarter of it, spreads a small batch over four times as many waves, and is
// used while the larger would leave the chip with fewer than two waves per
// SIMD.
constexpr int kSmallBatchWaves = 2048;

template <typename T, int N, int CPL, int R>
hipError_t launch_steps(int64_t S, int64_t B, int64_t H, int64_t P, int64_t G, const void *x,
                        const float *dt, const float *A, const void *Bm, const void *Cm,
                        const float *D, float *state, void *y, DtPrep prep, hipStream_t s)
{
    using Gm = StepsGeom<N, CPL, R>;
    const int64_t wpb = (P + Gm::ROWS - 1) / Gm::ROWS;
    const int64_t waves = B * H * wpb;
    if (waves > INT32_MAX - 4)
        return hipErrorInvalidValue;
    const int64_t blocks = (waves + kStepsThreads / 64 - 1) / (kStepsThreads / 64);
    if (prep.softplus)
        decode_steps_kernel<T, N, CPL, R, true><<<(unsigned)blocks, kStepsThreads, 0, s>>>(
            (int)S, (int)B, (int)H, (int)P, (int)G, (int)wpb, static_cast<const T *>(x), dt, A,
            static_cast<const T *>(Bm), static_cast<const T *>(Cm), D, state,
            static_cast<T *>(y), prep.bias);
    else
        decode_steps_kernel<T, N, CPL, R, false><<<(unsigned)blocks, kStepsThreads, 0, s>>>(
            (int)S, (int)B, (int)H, (int)P, (int)G, (int)wpb, static_cast<const T *>(x), dt, A,
            static_cast<const T *>(Bm), static_cast<const T *>(Cm), D, state,
            static_cast<T *>(y), nullptr);
    return hipGetLastError();
}

template <typename T, int N, int CPL, int RBig>
hipError_t steps_select(int64_t S, int64_t B, int64_t H, int64_t P, int64_t G, const void *x,
                        const float *dt, const float *A, const void *Bm, const void *Cm,
                        const float *D, float *state, void *y, DtPrep prep, hipStream_t s)
{
    constexpr int RSmall = RBig / 4;
    const int64_t rows = StepsGeom<N, CPL, RBig>::ROWS;
    if (B * H * ((P + rows - 1) / rows) < kSmallBatchWaves)
        return launch_steps<T, N, CPL, RSmall>(S, B, H, P, G, x, dt, A, Bm, Cm, D, state, y,
                                               prep, s);
    return launch_steps<T, N, CPL, RBig>(S, B, H, P, G, x, dt, A, Bm, Cm, D, state, y, prep, s);
}

template <typename T>
hipError_t steps_dispatch(int64_t S, int64_t B, int64_t H, int64_t P, int64_t N, int64_t G,
                          const void *x, const float *dt, const float *A, const void *Bm,
                          const void *Cm, const float *D, float *state, void *y, DtPrep prep,
                          hipStream_t s)
{
    switch (N) {
    case 16: return steps_select<T, 16, 1, 16>(S, B, H, P, G, x, dt, A, Bm, Cm, D, state, y, prep, s);
    case 32: return steps_select<T, 32, 2, 16>(S, B, H, P, G, x, dt, A, Bm, Cm, D, state, y, prep, s);
    case 64: return steps_select<T, 64, 4, 8>(S, B, H, P, G, x, dt, A, Bm, Cm, D, state, y, prep, s);
    case 128: return steps_select<T, 128, 8, 4>(S, B, H, P, G, x, dt, A, Bm, Cm, D, state, y, prep, s);
    case 256: return steps_select<T, 256, 4, 8>(S, B, H, P, G, x, dt, A, Bm, Cm, D, state, y, prep, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_decode_steps(int bf16, int64_t S, int64_t B, int64_t H, int64_t P, int64_t N,
                               int64_t G, const void *x, const float *dt, const float *A,
                               const void *Bm, const void *Cm, const float *D, float *state,
                               void *y, DtPrep prep, hipStream_t s)
{
    if (S == 0 || B * H == 0)
        return hipSuccess;
    if (bf16)
        return steps_dispatch<__bf16>(S, B, H, P, N, G, x, dt, A, Bm, Cm, D, state, y, prep, s);
    return steps_dispatch<float>(S, B, H, P, N, G, x, dt, A, Bm, Cm, D, state, y, prep, s);
}

}  // namespace ssd
