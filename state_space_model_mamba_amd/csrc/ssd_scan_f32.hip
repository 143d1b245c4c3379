// fp32 chunked SSD scan (VALU), for fp32 inputs with P <= 64, N <= 128, Q <= 256.
//
// "Compiler-First State Space Duality and Portable O(1) Autoregressive
// Caching for Inference", section 2: the recurrence is cut into fixed-size
// chunks; inside a chunk the output is a causal (lower-triangular, statically
// masked) quadratic form, across chunks a state is passed along; the decay is
// exponentiated in float32.  Per chunk of Qc <= Q tokens, with
// a_t = dt_t * A_h and Lam_t the inclusive sum of a over the chunk:
//     M[t,s]  = (C_t . B_s) * exp(Lam_t - Lam_s) * dt_s       for s <= t, else 0
//     y_t     = sum_s M[t,s] x_s + exp(Lam_t) * (S_in C_t) + D_h x_t
//     S_out   = exp(Lam_end) S_in + sum_s exp(Lam_end - Lam_s) dt_s x_s (outer) B_s
// All products and sums are fp32.  Lam is accumulated in fp64 so that the
// differences Lam_t - Lam_s do not lose the ~1e-5 absolute accuracy a long
// fp32 running sum would (the fp32 workload is held to 1e-5 relative); the
// exponentials themselves are fp32.
//
// One work-group per (b, h) walks its chunks in order; the state lives in LDS.
#include <hip/hip_runtime.h>

#include "ssd_kernels.h"

namespace ssd {
namespace {

constexpr int kF32Threads = 256;
constexpr int kF32MaxP = 64, kF32MaxN = 128, kF32MaxQ = 256, kF32TT = 16;

__global__ __launch_bounds__(kF32Threads) void scan_f32_kernel(
    int64_t L, int64_t H, int64_t P, int64_t N, int64_t G, int64_t Q,
    const float *__restrict__ x, const float *__restrict__ dt, const float *__restrict__ A,
    const float *__restrict__ Bm, const float *__restrict__ Cm, const float *__restrict__ D,
    const float *__restrict__ init, float *__restrict__ y, float *__restrict__ fin, DtPrep prep)
{
    __shared__ float S[kF32MaxP * kF32MaxN];
    __shared__ double lam[kF32MaxQ];
    __shared__ float dts[kF32MaxQ];
    __shared__ float wts[kF32MaxQ];   // exp(Lam_end - Lam_s) * dt_s
    __shared__ float M[kF32TT * kF32MaxQ];

    const int tid = threadIdx.x;
    const int64_t bh = blockIdx.x, b = bh / H, h = bh - b * H, g = h / (H / G);
    const float Ah = A[h], Dh = D[h];
    const float dtb = prep.softplus && prep.bias ? prep.bias[h] : 0.f;
    const int64_t PN = P * N;

    for (int64_t e = tid; e < PN; e += kF32Threads)
        S[e] = init ? init[bh * PN + e] : 0.f;

    for (int64_t c0 = 0; c0 < L; c0 += Q) {
        const int64_t Qc = (L - c0 < Q) ? (L - c0) : Q;
        __syncthreads();
        for (int64_t i = tid; i < Qc; i += kF32Threads) {
            const float u = dt[(b * L + c0 + i) * H + h];
            dts[i] = prep.softplus ? softplus_dt(u, dtb) : u;
        }
        __syncthreads();
        if (tid == 0) {
            double acc = 0.0;
            for (int64_t i = 0; i < Qc; ++i) {
                acc += (double)(dts[i] * Ah);
                lam[i] = acc;
            }
        }
        __syncthreads();
        const double lam_end = lam[Qc - 1];
        for (int64_t i = tid; i < Qc; i += kF32Threads)
            wts[i] = expf((float)(lam_end - lam[i])) * dts[i];

        for (int64_t t0 = 0; t0 < Qc; t0 += kF32TT) {
            const int64_t nt = (Qc - t0 < kF32TT) ? (Qc - t0) : kF32TT;
            __syncthreads();
            // masked, decayed C.B^T rows of this t-tile
            for (int64_t e = tid; e < nt * Qc; e += kF32Threads) {
                const int64_t tt = e / Qc, s = e - tt * Qc, t = t0 + tt;
                float v = 0.f;
                if (s <= t) {
                    const float *Cr = Cm + ((b * L + c0 + t) * G + g) * N;
                    const float *Br = Bm + ((b * L + c0 + s) * G + g) * N;
                    float dot = 0.f;
                    for (int64_t n = 0; n < N; ++n)
                        dot += Cr[n] * Br[n];
                    v = dot * expf((float)(lam[t] - lam[s])) * dts[s];
                }
                M[tt * Qc + s] = v;
            }
            __syncthreads();
            for (int64_t e = tid; e < nt * P; e += kF32Threads) {
                const int64_t tt = e / P, p = e - tt * P, t = t0 + tt;
                float intra = 0.f;
                for (int64_t s = 0; s <= t; ++s)
                    intra += M[tt * Qc + s] * x[((b * L + c0 + s) * H + h) * P + p];
                const float *Cr = Cm + ((b * L + c0 + t) * G + g) * N;
                float off = 0.f;
                for (int64_t n = 0; n < N; ++n)
                    off += Cr[n] * S[p * N + n];
                const float xv = x[((b * L + c0 + t) * H + h) * P + p];
                y[((b * L + c0 + t) * H + h) * P + p] =
                    intra + expf((float)lam[t]) * off + Dh * xv;
            }
        }
        __syncthreads();
        const float dec = expf((float)lam_end);
        for (int64_t e = tid; e < PN; e += kF32Threads) {
            const int64_t p = e / N, n = e - p * N;
            float acc = 0.f;
            for (int64_t s = 0; s < Qc; ++s)
                acc += wts[s] * x[((b * L + c0 + s) * H + h) * P + p] *
                       Bm[((b * L + c0 + s) * G + g) * N + n];
            S[e] = dec * S[e] + acc;
        }
    }
    __syncthreads();
    for (int64_t e = tid; e < PN; e += kF32Threads)
        fin[bh * PN + e] = S[e];
}

}  // namespace

hipError_t launch_scan_f32(int64_t B, int64_t L, int64_t H, int64_t P, int64_t N, int64_t G,
                           int64_t Q, const float *x, const float *dt, const float *A,
                           const float *Bm, const float *Cm, const float *D, const float *init,
                           float *y, float *fin, DtPrep prep, hipStream_t s, EventLog *log)
{
    if (P > kF32MaxP || N > kF32MaxN || Q > kF32MaxQ)
        return hipErrorInvalidValue;
    if (B * H == 0)
        return hipSuccess;
    hipError_t e = log_begin(log, s);
    if (e != hipSuccess)
        return e;
    scan_f32_kernel<<<(unsigned)(B * H), kF32Threads, 0, s>>>(L, H, P, N, G, Q, x, dt, A, Bm, Cm,
                                                             D, init, y, fin, prep);
    e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    return log_kernel(log, "scan_f32_kernel", s);
}

}  // namespace ssd
