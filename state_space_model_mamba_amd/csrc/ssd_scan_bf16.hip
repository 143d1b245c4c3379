// bf16 chunked SSD scan on gfx950 MFMA (P = 64, N = 128, Q % 64 == 0).
//
// Source of the method: "Compiler-First State Space Duality and Portable O(1)
// Autoregressive Caching for Inference", section 2 -- the SSD recurrence is
// diagonal per head and chunkable; inside a chunk it is a causal quadratic
// form built from einsum-style contractions under a static lower-triangular
// mask, across chunks a state is passed along, and the decay is exponentiated
// in float32.  With a_t = dt_t A_h and Lam_t the inclusive sum of a over the
// current chunk (reset to 0 at every chunk start):
//
//   segsum      Lseg[t,s] = exp(Lam_t - Lam_s) for s <= t, else 0
//   intra-chunk Y_diag   = (C B^T o Lseg) (dt x)
//   chunk state S_out    = exp(Lam_end) S_in + sum_s exp(Lam_end - Lam_s) dt_s x_s (outer) B_s
//   state->out  Y_off[t] = exp(Lam_t) S_in C_t
//   output      y = Y_diag + Y_off + D_h x
//
// How it maps onto the chip (the page's XLA formulation is prior art only):
//
// * A chunk is processed as 64-token tiles.  The quadratic form is evaluated
//   on the diagonal 64 x 64 tiles only; an off-diagonal tile (s in an earlier
//   tile of the same chunk) factorises as exp(Lam_t - Lam_e) exp(Lam_e - Lam_s)
//   with e the last token before t's tile, so its contribution is C_t times a
//   running state R that already holds exp(Lam_e) S_in plus the in-chunk
//   terms.  Every exponent is <= 0, so nothing can overflow.  Per tile:
//       Yt^T = (dt x)^T (C B^T o Lseg)^T + exp(Lam_t - Lam_e) R C^T    (MFMA)
//       R    = exp(Lam_tile_end - Lam_e) R + (B o w)^T (dt x),         (MFMA)
//       w_s  = exp(Lam_tile_end - Lam_s)
// * The contractions over tokens (dt x and B along s) need those operands
//   with s running along the MFMA K lanes, but x and B arrive token-major.
//   They are transposed in registers by a 16x16x16 MFMA against the identity
//   (exact: one product with 1, the rest with 0), whose output layout is
//   exactly the K-major operand layout; the per-token scale (dt_s or w_s) is
//   applied to the fp32 output before rounding to bf16.  The masked
//   C B^T tile is produced by an MFMA in the layout the next MFMA consumes,
//   so it never touches LDS.
// * Sequence parallelism: a (b, h) sequence is cut into segments of whole
//   chunks.  Kernel 1 computes each segment's end state from a zero start
//   (contractions for R only), kernel 2 chains the segment states
//   (S_in[k+1] = decay_k S_in[k] + S_loc[k]), kernel 3 re-walks every segment
//   from its true entering state and writes y (and the final state).  The
//   last segment is never needed by kernel 1.
// * Work-groups are remapped so that all heads of one (batch row, segment)
//   run on the same XCD and share its L2 for the B/C tiles.
//
// MFMA operand conventions (16x16 tiles, wave64): lane l = c + 16 g holds
// row/column c of A/B and K-group g; the fp32 result holds D[4g + i][c].
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdlib>

#include "ssd_kernels.h"

namespace ssd {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kP = 64, kN = 128, kT = 64;     // headdim, dstate, tile tokens
constexpr int kThreads = 256;                 // 4 waves
constexpr int kBRow = kN * 2 + 16;            // padded LDS row pitch (bytes) of B tile
constexpr int kXRow = kP * 2 + 16;            // of x tile
constexpr int kSRow = kN * 2 + 16;            // of bf16 state copy

struct __align__(16) TileSmem {
    unsigned char Bt[kT * kBRow];   // B[s][n] of the tile
    unsigned char Xt[kT * kXRow];   // x[s][p] of the tile
    unsigned char Sb[kP * kSRow];   // bf16(R)[p][n]
    float lam[kT];                  // chunk-referenced Lam of each token
    float dtv[kT];                  // dt of each token (0 past the end)
    float wout[kT];                 // exp(Lam_tile_end - Lam_s)
    float scal[4];                  // [0] Lam_e (before tile), [1] tile decay
};

struct SegArgs {
    const __bf16 *x;
    const float *dt;
    const float *A;
    const __bf16 *B;
    const __bf16 *C;
    const float *D;
    const float *init;   // S_in of segment 0 (nullable = zero state)
    __bf16 *y;
    float *fin;
    float *ws_state;     // [B*H][nslot][P][N]
    float *ws_decay;     // [B*H][nslot]
    int64_t L;
    int H, G, Q;
    int cps;             // chunks per segment
    int nseg;            // segments per (b, h)
    int nseg_launch;     // segments this launch covers
    int nslot;
    int seg0_from_ws;    // segment 0 reads its entering state from slot nseg-1
};

__device__ __forceinline__ f32x4 mfma32(bf16x8 a, bf16x8 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(bf16x4 a, bf16x4 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

// Hardware places work-group i on XCD i % 8; give each XCD a contiguous range
// of logical ids so that neighbouring logical work shares one L2.
__device__ __forceinline__ int64_t xcd_remap(int64_t i, int64_t n)
{
    const int64_t per = n / 8;
    if (i >= per * 8)
        return i;
    return (i % 8) * per + i / 8;
}

// Global -> LDS staging of one 64-token tile; wave 0 also scans the decay.
__device__ __forceinline__ void stage_tile(TileSmem &sm, const SegArgs &a, int64_t b, int h,
                                           int grp, int64_t t0, float Ah, float &lamE, int tid)
{
    const int64_t L = a.L;
    uint4 bv[4], xv[2];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int ci = tid + kThreads * r, row = ci >> 4, col = ci & 15;
        const int64_t t = t0 + row;
        bv[r] = make_uint4(0u, 0u, 0u, 0u);
        if (t < L)
            bv[r] = *reinterpret_cast<const uint4 *>(a.B + ((b * L + t) * a.G + grp) * kN + col * 8);
    }
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        const int ci = tid + kThreads * r, row = ci >> 3, col = ci & 7;
        const int64_t t = t0 + row;
        xv[r] = make_uint4(0u, 0u, 0u, 0u);
        if (t < L)
            xv[r] = *reinterpret_cast<const uint4 *>(a.x + ((b * L + t) * a.H + h) * kP + col * 8);
    }
    if (tid < 64) {   // wave 0: inclusive scan of a_t = dt_t A_h over the tile
        const int lane = tid;
        const int64_t t = t0 + lane;
        if (t0 % a.Q == 0)
            lamE = 0.f;                        // chunk start: Lam restarts
        const float d = (t < L) ? a.dt[(b * L + t) * a.H + h] : 0.f;
        float s = d * Ah;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const float v = __shfl_up(s, o, 64);
            if (lane >= o)
                s += v;
        }
        const float lam = lamE + s;
        const float lam_end = __shfl(lam, 63, 64);
        sm.lam[lane] = lam;
        sm.dtv[lane] = d;
        sm.wout[lane] = __expf(lam_end - lam);
        if (lane == 0) {
            sm.scal[0] = lamE;
            sm.scal[1] = __expf(lam_end - lamE);
        }
        lamE = lam_end;
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int ci = tid + kThreads * r, row = ci >> 4, col = ci & 15;
        *reinterpret_cast<uint4 *>(sm.Bt + row * kBRow + col * 16) = bv[r];
    }
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        const int ci = tid + kThreads * r, row = ci >> 3, col = ci & 7;
        *reinterpret_cast<uint4 *>(sm.Xt + row * kXRow + col * 16) = xv[r];
    }
}

// kOut = false: kernel 1 (segment end state from zero, written to the workspace).
// kOut = true : kernel 3 (y and, for the last segment, the final state).
template <bool kOut>
__global__ __launch_bounds__(kThreads, 2) void seg_kernel(SegArgs a)
{
    __shared__ TileSmem sm;
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, g = l >> 4, c = l & 15;
    const int64_t j = xcd_remap(blockIdx.x, gridDim.x);
    const int h = (int)(j % a.H);
    const int64_t r = j / a.H;
    const int seg = (int)(r % a.nseg_launch);
    const int64_t b = r / a.nseg_launch;
    const int grp = h / (a.H / a.G);
    const int64_t bh = b * a.H + h;
    const int64_t L = a.L;
    const int64_t tseg0 = (int64_t)seg * a.cps * a.Q;
    const int64_t tseg1 = std::min<int64_t>(L, tseg0 + (int64_t)a.cps * a.Q);
    const float Ah = a.A[h];
    const float Dh = kOut ? a.D[h] : 0.f;

    bf16x4 ident;
#pragma unroll
    for (int e = 0; e < 4; ++e)
        ident[e] = (__bf16)((4 * g + e == c) ? 1.f : 0.f);
    const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};

    // Running state R, held transposed: R[ni][pi][i] = R[p = 16 pi + c][n = 32 w + 16 ni + 4 g + i].
    f32x4 R[2][4];
    {
        const float *src = nullptr;
        if (kOut) {
            if (seg == 0)
                src = a.seg0_from_ws ? a.ws_state + (bh * a.nslot + (a.nseg - 1)) * kP * kN : a.init;
            else
                src = a.ws_state + (bh * a.nslot + (seg - 1)) * kP * kN;
        }
        if (src)
            src += (src == a.init) ? bh * kP * kN : 0;
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
#pragma unroll
            for (int pi = 0; pi < 4; ++pi) {
                R[ni][pi] = zero4;
                if (src)
                    R[ni][pi] = *reinterpret_cast<const f32x4 *>(
                        src + (16 * pi + c) * kN + 32 * w + 16 * ni + 4 * g);
            }
    }
    if (kOut) {
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
#pragma unroll
            for (int pi = 0; pi < 4; ++pi) {
                bf16x4 v;
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    v[i] = (__bf16)R[ni][pi][i];
                *reinterpret_cast<bf16x4 *>(sm.Sb + (16 * pi + c) * kSRow +
                                            (32 * w + 16 * ni + 4 * g) * 2) = v;
            }
    }

    float lamE = 0.f;       // wave 0 only: Lam at the end of the previous tile
    float decprod = 1.f;    // product of tile decays over the segment

    for (int64_t t0 = tseg0; t0 < tseg1; t0 += kT) {
        stage_tile(sm, a, b, h, grp, t0, Ah, lamE, tid);

        // C rows of this wave's 16 tokens, in MFMA operand layout (K = n).
        bf16x8 cop[4];
        const int tl = 16 * w + c;           // token of this lane within the tile
        const int64_t tg = t0 + tl;
        if (kOut) {
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                cop[ks] = bf16x8{};
                if (tg < L)
                    cop[ks] = *reinterpret_cast<const bf16x8 *>(
                        a.C + ((b * L + tg) * a.G + grp) * kN + 32 * ks + 8 * g);
            }
        }
        __syncthreads();

        // (dt x) transposed: xop[j][pi] lane (c, g) element 4 (si & 1) + i
        //   = dt_s x[s][16 pi + c],  s = 16 si + 4 g + i,  si in {2j, 2j+1}.
        bf16x8 xop[2][4];
#pragma unroll
        for (int si = 0; si < 4; ++si) {
            const f32x4 dv = *reinterpret_cast<const f32x4 *>(&sm.dtv[16 * si + 4 * g]);
#pragma unroll
            for (int pi = 0; pi < 4; ++pi) {
                const bf16x4 av = *reinterpret_cast<const bf16x4 *>(
                    sm.Xt + (16 * si + c) * kXRow + (16 * pi + 4 * g) * 2);
                const f32x4 d = mfma16(av, ident, zero4);
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    xop[si >> 1][pi][(si & 1) * 4 + i] = (__bf16)(d[i] * dv[i]);
            }
        }
        // (B o w) transposed for this wave's n-range: bop[j][ni] lane (c, g)
        //   element 4 (si & 1) + i = w_s B[s][32 w + 16 ni + c].
        bf16x8 bop[2][2];
#pragma unroll
        for (int si = 0; si < 4; ++si) {
            const f32x4 wv = *reinterpret_cast<const f32x4 *>(&sm.wout[16 * si + 4 * g]);
#pragma unroll
            for (int ni = 0; ni < 2; ++ni) {
                const bf16x4 av = *reinterpret_cast<const bf16x4 *>(
                    sm.Bt + (16 * si + c) * kBRow + (32 * w + 16 * ni + 4 * g) * 2);
                const f32x4 d = mfma16(av, ident, zero4);
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    bop[si >> 1][ni][(si & 1) * 4 + i] = (__bf16)(d[i] * wv[i]);
            }
        }

        if (kOut) {
            // (C B^T)^T for s-tiles si <= w (this wave's t-tile is w): lane (c, g)
            // holds [s = 16 si + 4 g + i][t = 16 w + c].
            f32x4 mt[4];
#pragma unroll
            for (int si = 0; si < 4; ++si) {
                mt[si] = zero4;
                if (si <= w) {
#pragma unroll
                    for (int ks = 0; ks < 4; ++ks) {
                        const bf16x8 av = *reinterpret_cast<const bf16x8 *>(
                            sm.Bt + (16 * si + c) * kBRow + (32 * ks + 8 * g) * 2);
                        mt[si] = mfma32(av, cop[ks], mt[si]);
                    }
                }
            }
            // Static causal mask on the exponent and the decay, rounded to bf16 in
            // the B-operand layout of the next product (dt_s is already in xop).
            const float lamt = sm.lam[tl];
            bf16x8 mop[2];
#pragma unroll
            for (int si = 0; si < 4; ++si) {
                const f32x4 lv = *reinterpret_cast<const f32x4 *>(&sm.lam[16 * si + 4 * g]);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int s = 16 * si + 4 * g + i;
                    float v = 0.f;
                    if (si <= w && s <= tl)
                        v = mt[si][i] * __expf(lamt - lv[i]);
                    mop[si >> 1][(si & 1) * 4 + i] = (__bf16)v;
                }
            }
            // Y^T[p][t] = sum_s (dt x)^T[p][s] Lmask[s][t]   (diagonal tile)
            f32x4 yacc[4];
#pragma unroll
            for (int pi = 0; pi < 4; ++pi) {
                yacc[pi] = mfma32(xop[0][pi], mop[0], zero4);
                if (w >= 2)
                    yacc[pi] = mfma32(xop[1][pi], mop[1], yacc[pi]);
            }
            // + exp(Lam_t - Lam_e) R C^T   (earlier tiles and earlier chunks)
            const float dec_in = __expf(lamt - sm.scal[0]);
#pragma unroll
            for (int pi = 0; pi < 4; ++pi) {
                f32x4 yo = zero4;
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) {
                    const bf16x8 av = *reinterpret_cast<const bf16x8 *>(
                        sm.Sb + (16 * pi + c) * kSRow + (32 * ks + 8 * g) * 2);
                    yo = mfma32(av, cop[ks], yo);
                }
                yacc[pi] += yo * dec_in;
            }
            // y = Y + D_h x, one rounding to bf16.
            if (tg < L) {
#pragma unroll
                for (int pi = 0; pi < 4; ++pi) {
                    const bf16x4 xv = *reinterpret_cast<const bf16x4 *>(
                        sm.Xt + tl * kXRow + (16 * pi + 4 * g) * 2);
                    bf16x4 o;
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        o[i] = (__bf16)(yacc[pi][i] + Dh * (float)xv[i]);
                    *reinterpret_cast<bf16x4 *>(a.y + ((b * L + tg) * a.H + h) * kP + 16 * pi +
                                                4 * g) = o;
                }
            }
        }

        // R <- exp(Lam_tile_end - Lam_e) R + (B o w)^T (dt x)
        const float dtile = sm.scal[1];
        decprod *= dtile;
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
#pragma unroll
            for (int pi = 0; pi < 4; ++pi) {
                f32x4 acc = R[ni][pi] * dtile;
                acc = mfma32(bop[0][ni], xop[0][pi], acc);
                acc = mfma32(bop[1][ni], xop[1][pi], acc);
                R[ni][pi] = acc;
            }
        __syncthreads();
        if (kOut) {
#pragma unroll
            for (int ni = 0; ni < 2; ++ni)
#pragma unroll
                for (int pi = 0; pi < 4; ++pi) {
                    bf16x4 v;
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        v[i] = (__bf16)R[ni][pi][i];
                    *reinterpret_cast<bf16x4 *>(sm.Sb + (16 * pi + c) * kSRow +
                                                (32 * w + 16 * ni + 4 * g) * 2) = v;
                }
        }
    }

    float *dst = nullptr;
    if (kOut) {
        if (seg == a.nseg - 1)
            dst = a.fin + bh * kP * kN;
    } else {
        dst = a.ws_state + (bh * a.nslot + seg) * kP * kN;
        if (tid == 0)
            a.ws_decay[bh * a.nslot + seg] = decprod;
    }
    if (dst) {
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
#pragma unroll
            for (int pi = 0; pi < 4; ++pi)
                *reinterpret_cast<f32x4 *>(dst + (16 * pi + c) * kN + 32 * w + 16 * ni + 4 * g) =
                    R[ni][pi];
    }
}

// Kernel 2: chain the segment states of every (b, h), elementwise over P x N.
//   S_in[0] = init (or 0);  S_in[k+1] = decay_k S_in[k] + S_loc[k]
// slot k (k < nseg-1) holds S_loc[k] on entry and S_in[k+1] on exit; when the
// final state aliases the initial state, slot nseg-1 receives a copy of S_in[0].
__global__ __launch_bounds__(256) void seg_pass_kernel(const float *__restrict__ init,
                                                      float *__restrict__ ws_state,
                                                      const float *__restrict__ ws_decay,
                                                      int64_t BH, int nseg, int nslot,
                                                      int seg0_to_ws)
{
    constexpr int PN4 = kP * kN / 4;
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= BH * PN4)
        return;
    const int64_t bh = idx / PN4;
    const int e = (int)(idx - bh * PN4);
    float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
    if (init)
        s = reinterpret_cast<const float4 *>(init)[bh * PN4 + e];
    float4 *base = reinterpret_cast<float4 *>(ws_state) + bh * nslot * PN4;
    if (seg0_to_ws)
        base[(int64_t)(nseg - 1) * PN4 + e] = s;
    for (int k = 0; k < nseg - 1; ++k) {
        const float d = ws_decay[bh * nslot + k];
        const float4 v = base[(int64_t)k * PN4 + e];
        s.x = d * s.x + v.x;
        s.y = d * s.y + v.y;
        s.z = d * s.z + v.z;
        s.w = d * s.w + v.w;
        base[(int64_t)k * PN4 + e] = s;
    }
}

int64_t env_int(const char *name, int64_t dflt)
{
    const char *v = std::getenv(name);
    if (!v || !*v)
        return dflt;
    const long long x = std::atoll(v);
    return x > 0 ? (int64_t)x : dflt;
}

}  // namespace

Bf16Plan plan_scan_bf16(int64_t B, int64_t L, int64_t H, int64_t Q)
{
    Bf16Plan p{};
    p.nchunks = (L + Q - 1) / Q;
    const int64_t bh = std::max<int64_t>(B * H, 1);
    // Segments per sequence: enough work-groups to fill 256 CUs a few times over.
    const int64_t target = env_int("SSD_SEG_TARGET_WG", 1024);
    int64_t nseg = std::max<int64_t>(1, std::min<int64_t>(p.nchunks, (target + bh - 1) / bh));
    p.chunks_per_seg = std::max<int64_t>(1, (p.nchunks + nseg - 1) / nseg);
    p.nseg = std::max<int64_t>(1, (p.nchunks + p.chunks_per_seg - 1) / p.chunks_per_seg);
    p.nslot = p.nseg > 1 ? p.nseg : 0;
    p.state_bytes = (size_t)(B * H * p.nslot) * kP * kN * sizeof(float);
    const size_t decay_bytes = (size_t)(B * H * p.nslot) * sizeof(float);
    p.ws_bytes = p.nslot ? ((p.state_bytes + 255) / 256) * 256 + decay_bytes : 0;
    return p;
}

hipError_t launch_scan_bf16(const Bf16Plan &plan, int64_t B, int64_t L, int64_t H, int64_t G,
                            int64_t Q, const void *x, const float *dt, const float *A,
                            const void *Bm, const void *Cm, const float *D, const float *init,
                            void *y, float *fin, void *ws, hipStream_t s, EventLog *log)
{
    if (B * H == 0 || L == 0)
        return hipSuccess;
    SegArgs a{};
    a.x = static_cast<const __bf16 *>(x);
    a.dt = dt;
    a.A = A;
    a.B = static_cast<const __bf16 *>(Bm);
    a.C = static_cast<const __bf16 *>(Cm);
    a.D = D;
    a.init = init;
    a.y = static_cast<__bf16 *>(y);
    a.fin = fin;
    a.L = L;
    a.H = (int)H;
    a.G = (int)G;
    a.Q = (int)Q;
    a.cps = (int)plan.chunks_per_seg;
    a.nseg = (int)plan.nseg;
    a.nslot = (int)plan.nslot;
    const bool alias = init != nullptr && init == fin;
    a.seg0_from_ws = (alias && plan.nseg > 1) ? 1 : 0;
    if (plan.nslot) {
        a.ws_state = static_cast<float *>(ws);
        a.ws_decay = reinterpret_cast<float *>(static_cast<char *>(ws) +
                                               ((plan.state_bytes + 255) / 256) * 256);
    }
    hipError_t e = log_begin(log, s);
    if (e != hipSuccess)
        return e;
    if (plan.nseg > 1) {
        a.nseg_launch = a.nseg - 1;
        seg_kernel<false><<<(unsigned)(B * H * (plan.nseg - 1)), kThreads, 0, s>>>(a);
        if ((e = hipGetLastError()) != hipSuccess || (e = log_kernel(log, "seg_state_kernel", s)) != hipSuccess)
            return e;
        const int64_t n = B * H * (kP * kN / 4);
        seg_pass_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(
            init, a.ws_state, a.ws_decay, B * H, a.nseg, a.nslot, a.seg0_from_ws);
        if ((e = hipGetLastError()) != hipSuccess || (e = log_kernel(log, "seg_pass_kernel", s)) != hipSuccess)
            return e;
    }
    a.nseg_launch = a.nseg;
    seg_kernel<true><<<(unsigned)(B * H * plan.nseg), kThreads, 0, s>>>(a);
    if ((e = hipGetLastError()) != hipSuccess)
        return e;
    return log_kernel(log, "chunk_scan_kernel", s);
}

}  // namespace ssd
