// Gated DeltaNet (GDN) decode step: one read and one write of the state.
//
// "A Persistent-State Dataflow Accelerator for Memory-Bound Linear Attention
// Decode on FPGA", section 2B: the standard step reads the recurrent state
// three times (retrieval, update, output); with the identity
//     S_t^T q = g S_{t-1}^T q + (q^T k) dv
// the output follows from what the retrieval pass already read, so one read
// pass and one write pass suffice.  Per (batch row b, value head j), with
// query/key head i = j / (Hv / Hk) (section 2C: value heads grouped onto
// query/key heads):
//     r  = S^T k,  p = S^T q                       (one read of S)
//     dv = beta (v - g r)                          (the gated delta rule)
//     o  = g p + (q . k) dv
//     S <- g S + k dv^T                            (one write of S)
// S is [dk, dv] fp32 per value head.  A work-group of four waves owns one
// value head's 128-column tile of S (all dk rows): each lane holds four
// consecutive columns of dk / (4 * RPI) rows in registers between the two
// passes, RPI = 64 / (CT / 4) rows being covered by one load instruction.
#include <hip/hip_runtime.h>

#include "ssd_kernels.h"

namespace ssd {
namespace {

constexpr int kGdnThreads = 256;

template <typename T> __device__ __forceinline__ float gdn_f(T v);
template <> __device__ __forceinline__ float gdn_f<float>(float v) { return v; }
template <> __device__ __forceinline__ float gdn_f<__bf16>(__bf16 v) { return (float)v; }

template <typename T> __device__ __forceinline__ T gdn_t(float v);
template <> __device__ __forceinline__ float gdn_t<float>(float v) { return v; }
template <> __device__ __forceinline__ __bf16 gdn_t<__bf16>(float v) { return (__bf16)v; }

// State above the 256 MB MALL streams through HBM on every step: its loads and
// stores carry non-temporal hints (measured 9% faster at batch 256 of the
// page's shape, 537 MB of state); a smaller state is accessed normally and
// stays cache-resident between steps.
constexpr int64_t kGdnNTBytes = 256ll << 20;

typedef float gdn_f4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

template <bool kNT>
__device__ __forceinline__ float4 gdn_ld(const float *p)
{
    if constexpr (kNT) {
        const gdn_f4 t = __builtin_nontemporal_load(reinterpret_cast<const gdn_f4 *>(p));
        return make_float4(t.x, t.y, t.z, t.w);
    }
    return *reinterpret_cast<const float4 *>(p);
}

template <bool kNT>
__device__ __forceinline__ void gdn_st(float *p, float4 v)
{
    if constexpr (kNT) {
        const gdn_f4 t = {v.x, v.y, v.z, v.w};
        __builtin_nontemporal_store(t, reinterpret_cast<gdn_f4 *>(p));
        return;
    }
    *reinterpret_cast<float4 *>(p) = v;
}

// DK state rows, CT columns per work-group (a tile of the dv columns).
template <typename T, int DK, int CT, bool kNT>
__global__ __launch_bounds__(kGdnThreads) void gdn_decode_kernel(
    int Hk, int Hv, int dv, const T *__restrict__ q, const T *__restrict__ k,
    const T *__restrict__ v, const float *__restrict__ g, const float *__restrict__ beta,
    float *__restrict__ state, T *__restrict__ o)
{
    constexpr int LPR = CT / 4;             // lanes per state row (4 columns each)
    constexpr int RPI = 64 / LPR;           // rows covered by one load instruction of a wave
    constexpr int ROWS = DK / (4 * RPI);    // rows per lane
    static_assert(ROWS >= 1 && ROWS * 4 * RPI == DK, "DK rows split over 4 waves x RPI");
    __shared__ float4 part[4 * RPI][LPR][2];   // per (wave, lane group): r and p of 4 columns
    __shared__ float4 sdv[LPR];
    __shared__ float sqk;

    const int tiles = dv / CT;
    const int bj = blockIdx.x / tiles, tile = blockIdx.x - bj * tiles;
    const int b = bj / Hv, j = bj - b * Hv, i = j / (Hv / Hk);
    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid / 64), lane = tid % 64;
    const int lg = lane / LPR, lc = lane % LPR;
    const int c0 = tile * CT + 4 * lc;                  // first of the lane's 4 columns
    const int r0 = (w * RPI + lg) * ROWS;               // first of the lane's ROWS rows

    // q and k of the lane's rows, widened into registers straight from memory
    // (not through LDS: no barrier before the first pass, so a wave starts as
    // soon as its own state loads land; 3% faster at batch 256, although the
    // kernel then runs two waves per SIMD instead of three)
    const T *qi = q + ((int64_t)b * Hk + i) * DK, *ki = k + ((int64_t)b * Hk + i) * DK;
    float kr_[ROWS], qr_[ROWS];
#pragma unroll
    for (int r = 0; r < ROWS; ++r) {
        kr_[r] = gdn_f<T>(ki[r0 + r]);
        qr_[r] = gdn_f<T>(qi[r0 + r]);
    }
    float *S = state + ((int64_t)bj * DK + r0) * dv + c0;
    float4 s[ROWS];
#pragma unroll
    for (int r = 0; r < ROWS; ++r)
        s[r] = gdn_ld<kNT>(S + (int64_t)r * dv);
    const float gj = g[bj], bt = beta[bj];

    // pass 1 (read): partial retrieval r = S^T k and readout p = S^T q
    float4 pr = make_float4(0.f, 0.f, 0.f, 0.f), pp = pr;
#pragma unroll
    for (int r = 0; r < ROWS; ++r) {
        const float kr = kr_[r], qr = qr_[r];
        pr.x += kr * s[r].x; pr.y += kr * s[r].y; pr.z += kr * s[r].z; pr.w += kr * s[r].w;
        pp.x += qr * s[r].x; pp.y += qr * s[r].y; pp.z += qr * s[r].z; pp.w += qr * s[r].w;
    }
    part[w * RPI + lg][lc][0] = pr;
    part[w * RPI + lg][lc][1] = pp;
    if (w == 0) {   // q . k over the wave: DK / 64 products per lane, then a lane sum
        float d = 0.f;
#pragma unroll
        for (int e = lane; e < DK; e += 64)
            d += gdn_f<T>(qi[e]) * gdn_f<T>(ki[e]);
#pragma unroll
        for (int off = 32; off > 0; off >>= 1)
            d += __shfl_xor(d, off, 64);
        if (lane == 0)
            sqk = d;
    }
    __syncthreads();

    // the delta and the output, once per column
    if (tid < LPR) {
        float4 R = part[0][tid][0], Pq = part[0][tid][1];
#pragma unroll
        for (int m = 1; m < 4 * RPI; ++m) {
            const float4 a = part[m][tid][0], c = part[m][tid][1];
            R.x += a.x; R.y += a.y; R.z += a.z; R.w += a.w;
            Pq.x += c.x; Pq.y += c.y; Pq.z += c.z; Pq.w += c.w;
        }
        const T *vj = v + (int64_t)bj * dv + c0;
        float4 d;
        d.x = bt * (gdn_f<T>(vj[0]) - gj * R.x);
        d.y = bt * (gdn_f<T>(vj[1]) - gj * R.y);
        d.z = bt * (gdn_f<T>(vj[2]) - gj * R.z);
        d.w = bt * (gdn_f<T>(vj[3]) - gj * R.w);
        sdv[tid] = d;
        T *oj = o + (int64_t)bj * dv + c0;
        oj[0] = gdn_t<T>(gj * Pq.x + sqk * d.x);
        oj[1] = gdn_t<T>(gj * Pq.y + sqk * d.y);
        oj[2] = gdn_t<T>(gj * Pq.z + sqk * d.z);
        oj[3] = gdn_t<T>(gj * Pq.w + sqk * d.w);
    }
    __syncthreads();

    // pass 2 (write): S <- g S + k dv^T from the registers
    const float4 d = sdv[lc];
#pragma unroll
    for (int r = 0; r < ROWS; ++r) {
        const float kr = kr_[r];
        float4 n;
        n.x = gj * s[r].x + kr * d.x;
        n.y = gj * s[r].y + kr * d.y;
        n.z = gj * s[r].z + kr * d.z;
        n.w = gj * s[r].w + kr * d.w;
        gdn_st<kNT>(S + (int64_t)r * dv, n);
    }
}

// S consecutive steps in one launch (tokens of every step given): the
// work-group keeps its tile of S in registers across all of them, so the state
// is read once and written once per launch -- the GPU form of the page's
// on-chip persistent state (section 2A), which turns decode from memory-bound
// into compute-bound.  Per step the same arithmetic as above, with one
// barrier: a wave first sums its row groups' partials across lanes (lane
// swaps) and stores them, and after the barrier every thread sums the four
// waves' partials for its own four columns and forms their delta itself (the
// first LPR threads also store o).  q and k reach LDS a step ahead of their
// use, through three buffers; the partials alternate between two.
//
// The registers hold S / sc, sc being the product of the gates since the last
// renormalisation: a step is then one fused multiply-add per element,
// S / sc' += k (dv / sc'), with sc' = sc g, instead of a multiply by g and a
// multiply-add; the retrieval and readout are scaled by sc after the
// reduction.  A step that would take sc' outside [2^-64, 2^64] (g = 0
// included) multiplies the registers by sc' and restarts sc at 1.  g is one
// value per work-group and step, so the test is uniform.  1 / sc' is the
// hardware reciprocal (within 1 ulp).
// q, k [S, B, Hk, DK], v, o [S, B, Hv, dv], g, beta [S, B, Hv].
// Occupancy: a thread holds DK * CT / 256 state elements.  At 64 (dk = dv =
// 128, or dk = 256 on 64-column tiles) the kernel is held to four waves per
// SIMD (128 VGPRs, no spill inside the step loop; the compiler alone took 160
// and three waves, 18% slower at batch 256); smaller slices need fewer
// registers anyway.
// NH value heads of one query/key head per work-group (NH = 2 when the value
// heads per query/key head come in pairs; section 2C of the page: the two
// value heads of a pair share the q/k datapath).  Waves 4 h .. 4 h + 3 serve
// value head h of the group; q and k are fetched once per step for all of
// them, and q . k is formed once.
template <typename T, int DK, int CT, int NH>
__global__ __launch_bounds__(kGdnThreads * NH) __attribute__((amdgpu_waves_per_eu(DK * CT <= 128 * 128 ? 4 : 1)))
void gdn_steps_kernel(
    int nsteps, int Bn, int Hk, int Hv, int dv, const T *__restrict__ q,
    const T *__restrict__ k, const T *__restrict__ v, const float *__restrict__ g,
    const float *__restrict__ beta, float *__restrict__ state, T *__restrict__ o)
{
    constexpr int kThreads = kGdnThreads * NH;
    constexpr int LPR = CT / 4, RPI = 64 / LPR, ROWS = DK / (4 * RPI);
    static_assert(ROWS >= 1 && ROWS * 4 * RPI == DK, "DK rows split over 4 waves x RPI");
    constexpr int QK = DK / kThreads > 0 ? DK / kThreads : 1;   // q/k elements per thread
    // q and k in three buffers (step t reads t % 3 and writes step t + 1's
    // into the next); the partials and q . k in two (by step parity)
    __shared__ float sk[3][DK], sq[3][DK];
    __shared__ float4 part[2][NH][4][LPR][2];   // per wave: r (row group 0) and p (row group 1)
    static_assert(RPI == 2 || RPI == 4, "row groups of a wave on lane bit 5 (and 4)");
    __shared__ float sqk[2];

    const int tiles = dv / CT;
    const int bp = blockIdx.x / tiles, tile = blockIdx.x - bp * tiles;   // (b, head group)
    const int tid = threadIdx.x;
    const int wg = __builtin_amdgcn_readfirstlane(tid / 64), lane = tid % 64;
    const int hs = wg / 4, w = wg % 4;                   // value head in the group, wave of its four
    const int b = bp / (Hv / NH), j = (bp - b * (Hv / NH)) * NH + hs, i = j / (Hv / Hk);
    const int bj = b * Hv + j;
    const int lg = lane / LPR, lc = lane % LPR;
    const int c0 = tile * CT + 4 * lc;
    const int r0 = (w * RPI + lg) * ROWS;
    const int64_t qks = (int64_t)Bn * Hk * DK, vs = (int64_t)Bn * Hv * dv, gs = (int64_t)Bn * Hv;
    const T *qb = q + ((int64_t)b * Hk + i) * DK, *kb = k + ((int64_t)b * Hk + i) * DK;
    const T *vb = v + (int64_t)bj * dv + c0;
    T *ob = o + (int64_t)bj * dv + c0;

    // The value head's state block through a buffer resource: one 32-bit lane
    // offset, the row stride in the scalar offset, so that no per-row address
    // stays live across the step loop for the final store.
    const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc(
        state + (int64_t)bj * DK * dv, (short)0, DK * dv * 4, 0x00020000);
    const unsigned soff = ((unsigned)r0 * (unsigned)dv + (unsigned)c0) * 4u;
    float4 s[ROWS];
#pragma unroll
    for (int r = 0; r < ROWS; ++r)
        s[r] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(
                                              srs, soff, r * dv * 4, 0));

    // A step's q and k (this thread's share, for the LDS copy), fetched two
    // steps ahead since they go to LDS one step ahead; its v (this thread's
    // four columns), g and beta, fetched one step ahead.
    struct QkIn {
        float qv[QK], kv[QK];
    };
    struct VIn {
        float vv[4], gg, bb;
    };
    auto fetch_qk = [&](QkIn &in, int t) {
        const int64_t tt = t < nsteps ? t : nsteps - 1;
#pragma unroll
        for (int e = 0; e < QK; ++e) {
            const int idx = tid + e * kThreads;
            in.qv[e] = idx < DK ? gdn_f<T>(qb[tt * qks + idx]) : 0.f;
            in.kv[e] = idx < DK ? gdn_f<T>(kb[tt * qks + idx]) : 0.f;
        }
    };
    auto fetch_v = [&](VIn &in, int t) {
        const int64_t tt = t < nsteps ? t : nsteps - 1;
#pragma unroll
        for (int e = 0; e < 4; ++e)
            in.vv[e] = gdn_f<T>(vb[tt * vs + e]);
        in.gg = g[tt * gs + bj];
        in.bb = beta[tt * gs + bj];
    };
    auto put_qk = [&](const QkIn &in, int buf) {
#pragma unroll
        for (int e = 0; e < QK; ++e) {
            const int idx = tid + e * kThreads;
            if (idx < DK) {
                sq[buf][idx] = in.qv[e];
                sk[buf][idx] = in.kv[e];
            }
        }
    };

    QkIn qkn;
    VIn cur, nxt;
    fetch_qk(qkn, 0);
    put_qk(qkn, 0);
    fetch_qk(qkn, 1);
    fetch_v(cur, 0);
    __syncthreads();   // step 0's q, k in LDS
    float sc = 1.f;
    for (int t = 0; t < nsteps; ++t) {
        const int pb = t % 3, nb = pb == 2 ? 0 : pb + 1, hb = t & 1;
        // Step t + 1's q and k go to the next buffer now; they are read after
        // this step's barrier.  That buffer was last read in step t - 2, which
        // every thread finished before it reached step t - 1's barrier, and
        // part[hb] / sqk[hb] were last read in step t - 2 the same way, so one
        // barrier per step suffices.
        put_qk(qkn, nb);
        fetch_qk(qkn, t + 2);
        fetch_v(nxt, t + 1);
        float4 pr = make_float4(0.f, 0.f, 0.f, 0.f), pp = pr;
#pragma unroll
        for (int r = 0; r < ROWS; ++r) {
            const float kr = sk[pb][r0 + r], qr = sq[pb][r0 + r];
            pr.x += kr * s[r].x; pr.y += kr * s[r].y; pr.z += kr * s[r].z; pr.w += kr * s[r].w;
            pp.x += qr * s[r].x; pp.y += qr * s[r].y; pp.z += qr * s[r].z; pp.w += qr * s[r].w;
        }
        // the wave's RPI row groups (lane bits 4 and 5) summed in every lane;
        // lanes of row group 0 store the retrieval, row group 1 the readout
        auto wave_sum = [&](float4 &v) {
            if constexpr (RPI == 4) {
                v.x = lane_pair_sum<4>(v.x); v.y = lane_pair_sum<4>(v.y);
                v.z = lane_pair_sum<4>(v.z); v.w = lane_pair_sum<4>(v.w);
            }
            v.x = lane_pair_sum<5>(v.x); v.y = lane_pair_sum<5>(v.y);
            v.z = lane_pair_sum<5>(v.z); v.w = lane_pair_sum<5>(v.w);
        };
        wave_sum(pr);
        wave_sum(pp);
        if (lg == 0)
            part[hb][hs][w][lc][0] = pr;
        else if (lg == 1)
            part[hb][hs][w][lc][1] = pp;
        if (wg == 1) {   // q . k, once for the group (wave 1, so wave 0 is free for the delta below)
            float d = 0.f;
#pragma unroll
            for (int e = lane; e < DK; e += 64)
                d += sq[pb][e] * sk[pb][e];
#pragma unroll
            for (int off = 32; off > 0; off >>= 1)
                d += __shfl_xor(d, off, 64);
            if (lane == 0)
                sqk[hb] = d;
        }
        __syncthreads();   // partials, q . k and step t + 1's q, k in LDS
        float4 R = part[hb][hs][0][lc][0], Pq = part[hb][hs][0][lc][1];
#pragma unroll
        for (int m = 1; m < 4; ++m) {
            const float4 a = part[hb][hs][m][lc][0], c = part[hb][hs][m][lc][1];
            R.x += a.x; R.y += a.y; R.z += a.z; R.w += a.w;
            Pq.x += c.x; Pq.y += c.y; Pq.z += c.z; Pq.w += c.w;
        }
        R.x *= sc; R.y *= sc; R.z *= sc; R.w *= sc;
        Pq.x *= sc; Pq.y *= sc; Pq.z *= sc; Pq.w *= sc;
        float4 d;
        d.x = cur.bb * (cur.vv[0] - cur.gg * R.x);
        d.y = cur.bb * (cur.vv[1] - cur.gg * R.y);
        d.z = cur.bb * (cur.vv[2] - cur.gg * R.z);
        d.w = cur.bb * (cur.vv[3] - cur.gg * R.w);
        if (w == 0 && lane < LPR) {
            T *oj = ob + (int64_t)t * vs;
            const float qk = sqk[hb];
            oj[0] = gdn_t<T>(cur.gg * Pq.x + qk * d.x);
            oj[1] = gdn_t<T>(cur.gg * Pq.y + qk * d.y);
            oj[2] = gdn_t<T>(cur.gg * Pq.z + qk * d.z);
            oj[3] = gdn_t<T>(cur.gg * Pq.w + qk * d.w);
        }
        float scn = sc * cur.gg;
        if (__builtin_amdgcn_readfirstlane(!(scn >= 0x1p-64f && scn <= 0x1p64f))) {
#pragma unroll
            for (int r = 0; r < ROWS; ++r) {
                s[r].x *= scn; s[r].y *= scn; s[r].z *= scn; s[r].w *= scn;
            }
            scn = 1.f;
        }
        sc = scn;
        const float ri = __builtin_amdgcn_rcpf(scn);
        d.x *= ri; d.y *= ri; d.z *= ri; d.w *= ri;
#pragma unroll
        for (int r = 0; r < ROWS; ++r) {
            const float kr = sk[pb][r0 + r];
            s[r].x = __builtin_fmaf(kr, d.x, s[r].x);
            s[r].y = __builtin_fmaf(kr, d.y, s[r].y);
            s[r].z = __builtin_fmaf(kr, d.z, s[r].z);
            s[r].w = __builtin_fmaf(kr, d.w, s[r].w);
        }
        cur = nxt;
    }
#pragma unroll
    for (int r = 0; r < ROWS; ++r)
        __builtin_amdgcn_raw_buffer_store_b128(
            __builtin_bit_cast(u32x4_t, make_float4(s[r].x * sc, s[r].y * sc, s[r].z * sc, s[r].w * sc)),
            srs, soff, r * dv * 4, 0);
}

template <typename T, int DK, int CT>
hipError_t gdn_steps_launch(int64_t S, int64_t B, int64_t Hk, int64_t Hv, int64_t dv,
                            const void *q, const void *k, const void *v, const float *g,
                            const float *beta, float *state, void *o, hipStream_t s)
{
    const T *qq = static_cast<const T *>(q), *kk = static_cast<const T *>(k),
            *vv = static_cast<const T *>(v);
    T *oo = static_cast<T *>(o);
    const int n = (int)S, b = (int)B, hk = (int)Hk, hv = (int)Hv, d = (int)dv;
    // value heads in pairs when every query/key head has an even number of
    // them and the pairs still give every CU a work-group (a small batch is
    // latency-bound per step, and twice the work-groups of one value head each
    // finish a step sooner)
    if ((Hv / Hk) % 2 == 0 && B * (Hv / 2) * (dv / CT) >= 256) {
        const unsigned grid = (unsigned)(B * (Hv / 2) * (dv / CT));
        gdn_steps_kernel<T, DK, CT, 2><<<grid, 2 * kGdnThreads, 0, s>>>(n, b, hk, hv, d, qq, kk, vv,
                                                                         g, beta, state, oo);
    } else {
        const unsigned grid = (unsigned)(B * Hv * (dv / CT));
        gdn_steps_kernel<T, DK, CT, 1><<<grid, kGdnThreads, 0, s>>>(n, b, hk, hv, d, qq, kk, vv, g,
                                                                     beta, state, oo);
    }
    return hipGetLastError();
}

template <typename T, int DK>
hipError_t gdn_steps_dispatch_dv(int64_t S, int64_t B, int64_t Hk, int64_t Hv, int64_t dv,
                                 const void *q, const void *k, const void *v, const float *g,
                                 const float *beta, float *state, void *o, hipStream_t s)
{
    // 64-column tiles at dk = 256, so that a thread holds 64 state elements
    // and the kernel runs four waves per SIMD (128-column tiles: 128 elements,
    // 256 VGPRs, one wave)
    if constexpr (DK == 256) {
        return gdn_steps_launch<T, DK, 64>(S, B, Hk, Hv, dv, q, k, v, g, beta, state, o, s);
    } else {
        if (dv < 128)
            return gdn_steps_launch<T, DK, 64>(S, B, Hk, Hv, dv, q, k, v, g, beta, state, o, s);
        return gdn_steps_launch<T, DK, 128>(S, B, Hk, Hv, dv, q, k, v, g, beta, state, o, s);
    }
}

template <typename T>
hipError_t gdn_steps_dispatch(int64_t S, int64_t B, int64_t Hk, int64_t Hv, int64_t dk, int64_t dv,
                              const void *q, const void *k, const void *v, const float *g,
                              const float *beta, float *state, void *o, hipStream_t s)
{
    switch (dk) {
    case 64: return gdn_steps_dispatch_dv<T, 64>(S, B, Hk, Hv, dv, q, k, v, g, beta, state, o, s);
    case 128: return gdn_steps_dispatch_dv<T, 128>(S, B, Hk, Hv, dv, q, k, v, g, beta, state, o, s);
    case 256: return gdn_steps_dispatch_dv<T, 256>(S, B, Hk, Hv, dv, q, k, v, g, beta, state, o, s);
    default: return hipErrorInvalidValue;
    }
}

template <typename T, int DK>
hipError_t gdn_dispatch_dv(int64_t B, int64_t Hk, int64_t Hv, int64_t dv, const void *q,
                           const void *k, const void *v, const float *g, const float *beta,
                           float *state, void *o, hipStream_t s)
{
    const int64_t ct = dv < 128 ? dv : 128;
    const unsigned grid = (unsigned)(B * Hv * (dv / ct));
    const T *qq = static_cast<const T *>(q), *kk = static_cast<const T *>(k),
            *vv = static_cast<const T *>(v);
    T *oo = static_cast<T *>(o);
    const bool nt = B * Hv * DK * dv * 4 > kGdnNTBytes;
    const int hk = (int)Hk, hv = (int)Hv, d = (int)dv;
    if (ct == 64 && nt)
        gdn_decode_kernel<T, DK, 64, true><<<grid, kGdnThreads, 0, s>>>(hk, hv, d, qq, kk, vv, g,
                                                                        beta, state, oo);
    else if (ct == 64)
        gdn_decode_kernel<T, DK, 64, false><<<grid, kGdnThreads, 0, s>>>(hk, hv, d, qq, kk, vv, g,
                                                                         beta, state, oo);
    else if (nt)
        gdn_decode_kernel<T, DK, 128, true><<<grid, kGdnThreads, 0, s>>>(hk, hv, d, qq, kk, vv, g,
                                                                         beta, state, oo);
    else
        gdn_decode_kernel<T, DK, 128, false><<<grid, kGdnThreads, 0, s>>>(hk, hv, d, qq, kk, vv,
                                                                          g, beta, state, oo);
    return hipGetLastError();
}

template <typename T>
hipError_t gdn_dispatch(int64_t B, int64_t Hk, int64_t Hv, int64_t dk, int64_t dv, const void *q,
                        const void *k, const void *v, const float *g, const float *beta,
                        float *state, void *o, hipStream_t s)
{
    switch (dk) {
    case 64: return gdn_dispatch_dv<T, 64>(B, Hk, Hv, dv, q, k, v, g, beta, state, o, s);
    case 128: return gdn_dispatch_dv<T, 128>(B, Hk, Hv, dv, q, k, v, g, beta, state, o, s);
    case 256: return gdn_dispatch_dv<T, 256>(B, Hk, Hv, dv, q, k, v, g, beta, state, o, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_gdn_decode(int bf16, int64_t B, int64_t Hk, int64_t Hv, int64_t dk, int64_t dv,
                             const void *q, const void *k, const void *v, const float *g,
                             const float *beta, float *state, void *o, hipStream_t s)
{
    if (B * Hv == 0)
        return hipSuccess;
    if (bf16)
        return gdn_dispatch<__bf16>(B, Hk, Hv, dk, dv, q, k, v, g, beta, state, o, s);
    return gdn_dispatch<float>(B, Hk, Hv, dk, dv, q, k, v, g, beta, state, o, s);
}

}  // namespace ssd

namespace ssd {

hipError_t launch_gdn_decode_steps(int bf16, int64_t S, int64_t B, int64_t Hk, int64_t Hv,
                                   int64_t dk, int64_t dv, const void *q, const void *k,
                                   const void *v, const float *g, const float *beta, float *state,
                                   void *o, hipStream_t s)
{
    if (S == 0 || B * Hv == 0)
        return hipSuccess;
    if (bf16)
        return gdn_steps_dispatch<__bf16>(S, B, Hk, Hv, dk, dv, q, k, v, g, beta, state, o, s);
    return gdn_steps_dispatch<float>(S, B, Hk, Hv, dk, dv, q, k, v, g, beta, state, o, s);
}

}  // namespace ssd
