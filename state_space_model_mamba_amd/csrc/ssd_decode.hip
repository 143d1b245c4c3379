// O(1) cached decode step and state initialisation.
//
// "Compiler-First State Space Duality and Portable O(1) Autoregressive
// Caching for Inference", section 2: a fixed-size per-sequence state lives on
// the device and each generated token updates it in place; section 4: this
// step is bandwidth-bound.  One step per (batch row b, head h):
//     alpha = exp(dt * A_h)                       (fp32 exponentiation)
//     H    <- alpha * H + (dt * x) (outer) B_g    (P x N, in place)
//     y     = H . C_g + D_h * x
// The kernel streams the fp32 state once: every element is loaded once,
// updated, stored once, and its contribution to y is reduced in the same pass
// (the one-read/one-write arrangement the FPGA decode page, section 2B,
// reaches for its recurrence).
#include <hip/hip_runtime.h>

#include <algorithm>

#include "ssd_kernels.h"

namespace ssd {
namespace {

template <typename T> __device__ __forceinline__ float to_f(T v);
template <> __device__ __forceinline__ float to_f<float>(float v) { return v; }
template <> __device__ __forceinline__ float to_f<__bf16>(__bf16 v) { return (float)v; }

template <typename T> __device__ __forceinline__ T from_f(float v);
template <> __device__ __forceinline__ float from_f<float>(float v) { return v; }
template <> __device__ __forceinline__ __bf16 from_f<__bf16>(float v) { return (__bf16)v; }

// Four consecutive elements of B or C, widened to fp32.
template <typename T> __device__ __forceinline__ float4 load4(const T *p);
template <> __device__ __forceinline__ float4 load4<float>(const float *p)
{
    return *reinterpret_cast<const float4 *>(p);
}
template <> __device__ __forceinline__ float4 load4<__bf16>(const __bf16 *p)
{
    typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
    const bf16x4 v = *reinterpret_cast<const bf16x4 *>(p);
    return make_float4((float)v[0], (float)v[1], (float)v[2], (float)v[3]);
}

// A state larger than the 256 MB MALL is streamed through HBM every step:
// non-temporal loads and stores (kNT; both together measured ~12% faster than
// plain ones at the 2.7B shape, batch 256) keep it from displacing other data
// on its way through.  A smaller state stays cache-resident across steps, so
// it is accessed normally.
constexpr int64_t kNTStateBytes = 256ll << 20;

template <bool kNT>
__device__ __forceinline__ float4 ld_state(const float *p)
{
    if constexpr (kNT) {
        typedef float f4 __attribute__((ext_vector_type(4)));
        const f4 v = __builtin_nontemporal_load(reinterpret_cast<const f4 *>(p));
        return make_float4(v.x, v.y, v.z, v.w);
    }
    return *reinterpret_cast<const float4 *>(p);
}
template <bool kNT>
__device__ __forceinline__ void st_state(float *p, float4 v)
{
    if constexpr (kNT) {
        typedef float f4 __attribute__((ext_vector_type(4)));
        const f4 w = {v.x, v.y, v.z, v.w};
        __builtin_nontemporal_store(w, reinterpret_cast<f4 *>(p));
        return;
    }
    *reinterpret_cast<float4 *>(p) = v;
}

constexpr int kDecodeThreads = 256;
constexpr int kDecodeUnroll = 8;   // state rows in flight per thread

// One work-group per (b, h).  A row of the state (N floats) is covered by
// N/4 consecutive lanes, each owning one float4; a pass covers 256/(N/4) rows
// and kDecodeUnroll passes are loaded before any is updated, so each thread
// keeps kDecodeUnroll 16-byte loads in flight.
template <typename T, int N, bool kNT>
__global__ __launch_bounds__(kDecodeThreads) void decode_kernel(
    int64_t H, int64_t P, int64_t G, const T *__restrict__ x, const float *__restrict__ dt,
    const float *__restrict__ A, const T *__restrict__ Bm, const T *__restrict__ Cm,
    const float *__restrict__ D, float *__restrict__ state, T *__restrict__ y, DtPrep prep)
{
    constexpr int LPR = N / 4;                 // lanes per state row
    constexpr int RPP = kDecodeThreads / LPR;  // rows per pass
    const int64_t bh = blockIdx.x;
    const int64_t b = bh / H, h = bh - b * H, g = h / (H / G);
    const int tid = threadIdx.x, lr = tid % LPR, rr = tid / LPR;
    const int n0 = lr * 4;

    const float4 Bv = load4<T>(Bm + (b * G + g) * N + n0);
    const float4 Cv = load4<T>(Cm + (b * G + g) * N + n0);
    float d = dt[bh];
    if (prep.softplus)
        d = softplus_dt(d, prep.bias ? prep.bias[h] : 0.f);
    const float alpha = __expf(d * A[h]);
    const float Dh = D[h];
    float *S = state + bh * P * N;
    const T *xr = x + bh * P;
    T *yr = y + bh * P;

    for (int64_t p0 = 0; p0 < P; p0 += (int64_t)RPP * kDecodeUnroll) {
        float4 s[kDecodeUnroll];
        float xv[kDecodeUnroll];
#pragma unroll
        for (int u = 0; u < kDecodeUnroll; ++u) {
            const int64_t p = p0 + u * RPP + rr;
            if (p < P) {
                s[u] = ld_state<kNT>(S + p * N + n0);
                xv[u] = to_f<T>(xr[p]);
            } else {
                s[u] = make_float4(0.f, 0.f, 0.f, 0.f);
                xv[u] = 0.f;
            }
        }
#pragma unroll
        for (int u = 0; u < kDecodeUnroll; ++u) {
            const int64_t p = p0 + u * RPP + rr;
            const float du = d * xv[u];
            float4 o;
            o.x = alpha * s[u].x + du * Bv.x;
            o.y = alpha * s[u].y + du * Bv.y;
            o.z = alpha * s[u].z + du * Bv.z;
            o.w = alpha * s[u].w + du * Bv.w;
            if (p < P)
                st_state<kNT>(S + p * N + n0, o);
            float part = o.x * Cv.x + o.y * Cv.y + o.z * Cv.z + o.w * Cv.w;
#pragma unroll
            for (int off = LPR / 2; off > 0; off >>= 1)
                part += __shfl_xor(part, off, 64);
            if (lr == 0 && p < P)
                yr[p] = from_f<T>(part + Dh * xv[u]);
        }
    }
}

// Rows of N >= 64: each lane owns 16 floats of a row (four float4 at
// n = 4 lr + 4 LPR k, so that each load instruction covers whole 64 LPR-byte
// row pieces), so the y reduction over n is mostly inside the thread and the
// remaining LPR (4, 8 or 16) lanes of a row are combined with DPP lane swaps
// (quad permutations, then the half-row and row mirrors) instead of shuffles
// through LDS.  Two row slots per thread keep eight 16-byte loads in flight;
// rows past P are clamped for the loads and not stored.
template <int kCtrl>
__device__ __forceinline__ float dpp_f(float v)
{
    return __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), kCtrl, 0xf, 0xf, true));
}

template <typename T, int N, bool kNT>
__global__ __launch_bounds__(kDecodeThreads) void decode_rows_kernel(
    int H, int P, int G, const T *__restrict__ x, const float *__restrict__ dt,
    const float *__restrict__ A, const T *__restrict__ Bm, const T *__restrict__ Cm,
    const float *__restrict__ D, float *__restrict__ state, T *__restrict__ y, DtPrep prep)
{
    constexpr int LPR = N / 16;                // lanes per state row
    constexpr int RPP = kDecodeThreads / LPR;  // rows per pass
    constexpr int U = 2;                       // row slots per thread
    const int bh = blockIdx.x;
    const int b = bh / H, h = bh - b * H, g = h / (H / G);
    const int tid = threadIdx.x, lr = tid % LPR, rr = tid / LPR;

    float4 Bv[4], Cv[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        Bv[k] = load4<T>(Bm + (int64_t)(b * G + g) * N + 4 * lr + 4 * LPR * k);
        Cv[k] = load4<T>(Cm + (int64_t)(b * G + g) * N + 4 * lr + 4 * LPR * k);
    }
    float d = dt[bh];
    if (prep.softplus)
        d = softplus_dt(d, prep.bias ? prep.bias[h] : 0.f);
    const float alpha = __expf(d * A[h]);
    const float Dh = D[h];
    float *S = state + (int64_t)bh * P * N + 4 * lr;
    const T *xr = x + (int64_t)bh * P;
    T *yr = y + (int64_t)bh * P;

    for (int p0 = 0; p0 < P; p0 += RPP * U) {
        float4 s[U][4];
        float xv[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int p = min(p0 + u * RPP + rr, P - 1);
#pragma unroll
            for (int k = 0; k < 4; ++k)
                s[u][k] = ld_state<kNT>(S + (int64_t)p * N + 4 * LPR * k);
            xv[u] = to_f<T>(xr[p]);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int p = p0 + u * RPP + rr;
            const float du = d * xv[u];
            float part = 0.f;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                float4 o;
                o.x = alpha * s[u][k].x + du * Bv[k].x;
                o.y = alpha * s[u][k].y + du * Bv[k].y;
                o.z = alpha * s[u][k].z + du * Bv[k].z;
                o.w = alpha * s[u][k].w + du * Bv[k].w;
                s[u][k] = o;
                part += o.x * Cv[k].x + o.y * Cv[k].y + o.z * Cv[k].z + o.w * Cv[k].w;
            }
            if (p < P) {
#pragma unroll
                for (int k = 0; k < 4; ++k)
                    st_state<kNT>(S + (int64_t)p * N + 4 * LPR * k, s[u][k]);
            }
            part += dpp_f<0xB1>(part);                 // quad_perm [1,0,3,2]
            part += dpp_f<0x4E>(part);                 // quad_perm [2,3,0,1]
            if constexpr (LPR >= 8)
                part += dpp_f<0x141>(part);            // row_half_mirror
            if constexpr (LPR >= 16)
                part += dpp_f<0x140>(part);            // row_mirror
            if (lr == 0 && p < P)
                yr[p] = from_f<T>(part + Dh * xv[u]);
        }
    }
}

__global__ void fill_kernel(float *__restrict__ dst, const float *__restrict__ src, int64_t n)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
        dst[i] = src ? src[i] : 0.f;
}

__global__ void fill4_kernel(float4 *__restrict__ dst, const float4 *__restrict__ src, int64_t n4)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride)
        dst[i] = src ? src[i] : make_float4(0.f, 0.f, 0.f, 0.f);
}

template <typename T, bool kNT>
hipError_t decode_dispatch(int64_t B, int64_t H, int64_t P, int64_t N, int64_t G, const void *x,
                           const float *dt, const float *A, const void *Bm, const void *Cm,
                           const float *D, float *state, void *y, DtPrep prep, hipStream_t s)
{
    const dim3 grid((unsigned)(B * H)), block(kDecodeThreads);
    const T *xx = static_cast<const T *>(x);
    const T *bb = static_cast<const T *>(Bm);
    const T *cc = static_cast<const T *>(Cm);
    T *yy = static_cast<T *>(y);
    const int h = (int)H, p = (int)P, g = (int)G;
    switch (N) {
    case 16:
        decode_kernel<T, 16, kNT><<<grid, block, 0, s>>>(H, P, G, xx, dt, A, bb, cc, D, state, yy, prep);
        break;
    case 32:
        decode_kernel<T, 32, kNT><<<grid, block, 0, s>>>(H, P, G, xx, dt, A, bb, cc, D, state, yy, prep);
        break;
    case 64:
        decode_rows_kernel<T, 64, kNT><<<grid, block, 0, s>>>(h, p, g, xx, dt, A, bb, cc, D, state, yy, prep);
        break;
    case 128:
        decode_rows_kernel<T, 128, kNT><<<grid, block, 0, s>>>(h, p, g, xx, dt, A, bb, cc, D, state, yy, prep);
        break;
    case 256:
        decode_rows_kernel<T, 256, kNT><<<grid, block, 0, s>>>(h, p, g, xx, dt, A, bb, cc, D, state, yy, prep);
        break;
    default:
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <typename T>
hipError_t decode_select(int64_t B, int64_t H, int64_t P, int64_t N, int64_t G, const void *x,
                         const float *dt, const float *A, const void *Bm, const void *Cm,
                         const float *D, float *state, void *y, DtPrep prep, hipStream_t s)
{
    if (B * H * P * N * 4 > kNTStateBytes)
        return decode_dispatch<T, true>(B, H, P, N, G, x, dt, A, Bm, Cm, D, state, y, prep, s);
    return decode_dispatch<T, false>(B, H, P, N, G, x, dt, A, Bm, Cm, D, state, y, prep, s);
}

}  // namespace

hipError_t launch_state_init(float *state, const float *src, int64_t n, hipStream_t s)
{
    if (n <= 0 || state == src)
        return hipSuccess;
    const int threads = 256;
    const bool vec = (n % 4 == 0) && (reinterpret_cast<uintptr_t>(state) % 16 == 0) &&
                     (reinterpret_cast<uintptr_t>(src) % 16 == 0);
    const int64_t work = vec ? n / 4 : n;
    const int64_t blocks = std::min<int64_t>((work + threads - 1) / threads, 65536);
    if (vec)
        fill4_kernel<<<(unsigned)blocks, threads, 0, s>>>(reinterpret_cast<float4 *>(state),
                                                          reinterpret_cast<const float4 *>(src),
                                                          work);
    else
        fill_kernel<<<(unsigned)blocks, threads, 0, s>>>(state, src, n);
    return hipGetLastError();
}

hipError_t launch_decode(int bf16, int64_t B, int64_t H, int64_t P, int64_t N, int64_t G,
                         const void *x, const float *dt, const float *A, const void *Bm,
                         const void *Cm, const float *D, float *state, void *y, DtPrep prep,
                         hipStream_t s)
{
    if (B * H == 0)
        return hipSuccess;
    if (bf16)
        return decode_select<__bf16>(B, H, P, N, G, x, dt, A, Bm, Cm, D, state, y, prep, s);
    return decode_select<float>(B, H, P, N, G, x, dt, A, Bm, Cm, D, state, y, prep, s);
}

}  // namespace ssd
