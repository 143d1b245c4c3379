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
// * The contractions over tokens need (dt x) and B with s running along the
//   MFMA K lanes, but both arrive token-major.  They are staged token-major in
//   LDS and read K-major with gfx950's transpose read (ds_read_b64_tr_b16);
//   the per-token scale dt_s w_s of the state update is applied once while
//   staging a second, scaled bf16 copy of the x tile, and dt_s of the
//   diagonal block is applied to the masked C B^T tile.  That tile is produced
//   by an MFMA in the layout the next MFMA consumes, so it never touches LDS.
// * The next tile's global loads are issued before the current tile is
//   computed and land in registers (software pipelining); they are written to
//   LDS after the tile's closing barrier.
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
typedef short s16x4 __attribute__((__vector_size__(8)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr int kP = 64, kN = 128, kT = 64;     // headdim, dstate, tile tokens
constexpr int kThreads = 256;                 // 4 waves
// Padded LDS row pitches (bytes): a 32-byte pad spreads the 16 rows one
// transpose read touches over all banks.
constexpr int kBRow = kN * 2 + 32;            // B tile [s][n]
constexpr int kXRow = kP * 2 + 32;            // x tiles [s][p]
constexpr int kSRow = kN * 2 + 16;            // bf16 copy of the state [p][n]

// LDS of one work-group.  The state-only kernel needs only the B tile, the
// scaled x tile and the tile decay.
template <bool kOut> struct TileSmem;
template <> struct __align__(16) TileSmem<true> {
    unsigned char Bt[kT * kBRow];   // B[s][n] of the tile
    unsigned char Xt[kT * kXRow];   // x[s][p] of the tile (raw)
    unsigned char Xw[kT * kXRow];   // bf16(dt_s w_s x[s][p]), w_s = exp(Lam_tile_end - Lam_s)
    unsigned char Sb[kP * kSRow];   // bf16(R)[p][n]
    float lam[kT];                  // chunk-referenced Lam of each token
    float dtv[kT];                  // dt of each token (0 past the end)
    float ed[kT];                   // exp(Lam_q - Lam_s) dt_s, q = last token of s's 16-row block
    float scal[4];                  // [0] Lam_e (before tile), [1] tile decay
};
template <> struct __align__(16) TileSmem<false> {
    unsigned char Bt[kT * kBRow];
    unsigned char Xw[kT * kXRow];
    float scal[4];
};

struct SegArgs {
    const __bf16 *x;
    const float *dt;
    const float2 *ld;    // [B*H][L]: (Lam_t chunk-referenced, dt_t), from decay_prep_kernel
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

// Hardware places work-group i on XCD i % 8; give each XCD a contiguous range
// of logical ids so that neighbouring logical work shares one L2.
__device__ __forceinline__ int64_t xcd_remap(int64_t i, int64_t n)
{
    const int64_t per = n / 8;
    if (i >= per * 8)
        return i;
    return (i % 8) * per + i / 8;
}

// Work-group barrier for LDS hand-offs only.  __syncthreads() also fences
// global memory, which would make every barrier wait for the next tile's
// in-flight global loads and this tile's y stores; here only LDS traffic has
// to be complete (lgkmcnt), and the memory clobber keeps the compiler from
// moving LDS accesses across the barrier.
__device__ __forceinline__ void lds_barrier()
{
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Inclusive prefix sum across the 64 lanes of a wave: Hillis-Steele inside
// each 16-lane row with DPP row shifts (bound_ctrl: lanes with no source add
// 0), then the three lower rows' totals are added with readlane.  A few cycles
// per step, against ~100 for a shuffle through the LDS crossbar.
template <int kCtrl>
__device__ __forceinline__ float dpp_row_shr(float v)
{
    return __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), kCtrl, 0xf, 0xf, true));
}
__device__ __forceinline__ float lane_f(float v, int lane)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}
__device__ __forceinline__ float wave_inclusive_sum(float v, int lane)
{
    v += dpp_row_shr<0x111>(v);   // row_shr:1
    v += dpp_row_shr<0x112>(v);   // row_shr:2
    v += dpp_row_shr<0x114>(v);   // row_shr:4
    v += dpp_row_shr<0x118>(v);   // row_shr:8
    const float r0 = lane_f(v, 15), r1 = lane_f(v, 31), r2 = lane_f(v, 47);
    const int row = lane >> 4;
    return v + (row == 0 ? 0.f : row == 1 ? r0 : row == 2 ? r0 + r1 : r0 + r1 + r2);
}

// K-major MFMA operand from a token-major LDS tile with gfx950's transpose read
// (ds_read_b64_tr_b16).  Within each 16-lane group the instruction hands
// output lane i, element e, the element (i % 4) of the 8 bytes input lane
// 4e + i/4 addressed.  Input lane (c, g) therefore addresses row
// 32 j + 16 h + 4 g + c/4 and columns col0 + 4 (c % 4) .. +3, so that output
// lane (c, g) receives column col0 + c at rows s = 32 j + 16 h + 4 g + e
// (elements 4 h + e of the 8-element operand): the same token-to-K-slot map
// as the C B^T tiles produced by the MFMA of the causal block.
__device__ __forceinline__ bf16x8 tr_operand(const unsigned char *tile, int pitch, int j,
                                             int col0, int g, int c)
{
    const unsigned char *p = tile + (32 * j + 4 * g + (c >> 2)) * pitch + (col0 + 4 * (c & 3)) * 2;
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)p);
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(p + 16 * pitch));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Per-work-group view of the inputs: pointers at token 0 of this (b, h) and
// per-lane element offsets that are the same for every tile.
struct WgIo {
    const __bf16 *x, *B, *C;
    const float2 *ld;                     // (Lam, dt) of this (b, h), token-contiguous
    __bf16 *y;
    int64_t xstride, bstride;             // elements per token
    int offB[4], offX[2], offC;
};

// One 64-token tile's global inputs, held in registers while the previous tile
// is being computed (software pipelining across tiles).
struct TileRegs {
    uint4 b[4];      // B rows: chunks tid + 256 r of the [64][16 x 16 B] tile
    uint4 x[2];      // x rows: chunks tid + 256 r of the [64][8 x 16 B] tile
    bf16x8 c[4];     // C row 16 w + c, n = 32 ks + 8 g .. +8 (MFMA operand layout)
    float2 ld;       // (Lam, dt) of token t0 + lane
};

// Issue the global loads of the tile starting at t0.  Always the same
// instructions with no branches (rows past the end are clamped to the last
// valid token and zeroed later, in store_tile), so the compiler's wait-count
// analysis sees exactly which loads are outstanding and lets a prefetched tile
// stay in flight while earlier tiles are consumed.  t0 itself may lie past the
// end of the segment: the caller then simply never stores that tile.
template <bool kOut>
__device__ __forceinline__ void load_tile(TileRegs &tr, const WgIo &io, int64_t t0, int64_t L,
                                          int tid)
{
    const int w = tid >> 6, l = tid & 63, c = l & 15, g = l >> 4;
    t0 = (t0 < L) ? t0 : (L - 1) & ~(int64_t)(kT - 1);
    const int rem = (int)((L - t0 < kT) ? (L - t0) : kT);   // valid tokens, 1 .. 64
    const __bf16 *Bp = io.B + t0 * io.bstride;
    const __bf16 *xp = io.x + t0 * io.xstride;
    const __bf16 *Cp = io.C + t0 * io.bstride;
    const float2 *lp = io.ld + t0;
    int oB[4], oX[2], oC = io.offC, oD = l;
#pragma unroll
    for (int r = 0; r < 4; ++r)
        oB[r] = io.offB[r];
#pragma unroll
    for (int r = 0; r < 2; ++r)
        oX[r] = io.offX[r];
    if (rem < kT) {                           // ragged tile: clamp rows (no loads here)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int ci = tid + kThreads * r, row = ci >> 4;
            oB[r] = ((row < rem) ? row : rem - 1) * (int)io.bstride + (ci & 15) * 8;
        }
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            const int ci = tid + kThreads * r, row = ci >> 3;
            oX[r] = ((row < rem) ? row : rem - 1) * (int)io.xstride + (ci & 7) * 8;
        }
        const int rc = 16 * w + c;
        oC = ((rc < rem) ? rc : rem - 1) * (int)io.bstride + 8 * g;
        oD = (l < rem) ? l : rem - 1;
    }
#pragma unroll
    for (int r = 0; r < 4; ++r)
        tr.b[r] = *reinterpret_cast<const uint4 *>(Bp + oB[r]);
#pragma unroll
    for (int r = 0; r < 2; ++r)
        tr.x[r] = *reinterpret_cast<const uint4 *>(xp + oX[r]);
    if constexpr (kOut) {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
            tr.c[ks] = *reinterpret_cast<const bf16x8 *>(Cp + oC + 32 * ks);
    }
    tr.ld = lp[oD];
}

// Registers -> LDS for one tile.  Every wave scans a_t = dt_t A_h over the 64
// tokens (lane = token) to get the chunk-referenced Lam and w_s; wave 0 also
// publishes the per-token tables.  lamE (Lam before the tile) is carried in
// every wave and restarts at 0 at a chunk boundary.
template <bool kOut>
__device__ __forceinline__ void store_tile(TileSmem<kOut> &sm, TileRegs &tr, int64_t t0, int64_t L,
                                           int Q, float &lamE, int tid)
{
    const int w = tid >> 6, l = tid & 63;
    if (t0 % Q == 0)
        lamE = 0.f;
    const int rem = (int)((L - t0 < kT) ? (L - t0) : kT);
    if (rem < kT) {                           // ragged tile: zero the clamped rows
        const uint4 z = make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
        for (int r = 0; r < 4; ++r)
            if (((tid + kThreads * r) >> 4) >= rem)
                tr.b[r] = z;
#pragma unroll
        for (int r = 0; r < 2; ++r)
            if (((tid + kThreads * r) >> 3) >= rem)
                tr.x[r] = z;
        if constexpr (kOut) {
            if (16 * w + (l & 15) >= rem) {
#pragma unroll
                for (int ks = 0; ks < 4; ++ks)
                    tr.c[ks] = bf16x8{};
            }
        }
        if (l >= rem)
            tr.ld.y = 0.f;                    // clamped lanes repeat the last token's Lam
    }
    const float lam = tr.ld.x, dtl = tr.ld.y;
    const float lam_end = lane_f(lam, 63);
    const float fx = dtl * __expf(lam_end - lam);     // dt_s w_s of token l
    if (w == 0) {
        if constexpr (kOut) {
            const float lam_q = __shfl(lam, l | 15, 64);
            sm.lam[l] = lam;
            sm.dtv[l] = dtl;
            sm.ed[l] = __expf(lam_q - lam) * dtl;
        }
        if (l == 0) {
            sm.scal[0] = lamE;
            sm.scal[1] = __expf(lam_end - lamE);
        }
    }
    lamE = lam_end;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int ci = tid + kThreads * r, row = ci >> 4, col = ci & 15;
        *reinterpret_cast<uint4 *>(sm.Bt + row * kBRow + col * 16) = tr.b[r];
    }
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        const int ci = tid + kThreads * r, row = ci >> 3, col = ci & 7;
        const float f = __shfl(fx, row, 64);
        const bf16x8 xv = __builtin_bit_cast(bf16x8, tr.x[r]);
        bf16x8 xs;
#pragma unroll
        for (int e = 0; e < 8; ++e)
            xs[e] = (__bf16)((float)xv[e] * f);
        *reinterpret_cast<bf16x8 *>(sm.Xw + row * kXRow + col * 16) = xs;
        if constexpr (kOut)
            *reinterpret_cast<uint4 *>(sm.Xt + row * kXRow + col * 16) = tr.x[r];
    }
}

// kOut = false: kernel 1 (segment end state from zero, written to the workspace).
// kOut = true : kernel 3 (y and, for the last segment, the final state).
template <bool kOut>
__device__ __forceinline__ void seg_body(const SegArgs &a, TileSmem<kOut> &sm)
{
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
    const float Dh = kOut ? a.D[h] : 0.f;
    const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};

    WgIo io;
    io.xstride = (int64_t)a.H * kP;
    io.bstride = (int64_t)a.G * kN;
    io.x = a.x + (b * L * a.H + h) * kP;
    io.B = a.B + (b * L * a.G + grp) * kN;
    io.C = a.C + (b * L * a.G + grp) * kN;
    io.ld = a.ld + bh * L;
    io.y = kOut ? a.y + (b * L * a.H + h) * kP : nullptr;
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
        const int ci = tid + kThreads * rr;
        io.offB[rr] = (ci >> 4) * (int)io.bstride + (ci & 15) * 8;
    }
#pragma unroll
    for (int rr = 0; rr < 2; ++rr) {
        const int ci = tid + kThreads * rr;
        io.offX[rr] = (ci >> 3) * (int)io.xstride + (ci & 7) * 8;
    }
    io.offC = (16 * w + c) * (int)io.bstride + 8 * g;

    // Running state R, held transposed: R[ni][pi][i] = R[p = 16 pi + c][n = 32 w + 16 ni + 4 g + i].
    f32x4 R[2][4];
    {
        const float *src = nullptr;
        if (kOut) {
            if (seg > 0)
                src = a.ws_state + (bh * a.nslot + (seg - 1)) * kP * kN;
            else if (a.seg0_from_ws)
                src = a.ws_state + (bh * a.nslot + (a.nseg - 1)) * kP * kN;
            else if (a.init)
                src = a.init + bh * kP * kN;
        }
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
    if constexpr (kOut) {
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

    float lamE = 0.f;       // Lam at the end of the previous tile (every wave)
    float decprod = 1.f;    // product of tile decays over the segment

    // One tile: the state update always; for kOut also y of the tile, returned
    // in yout (bf16, lane (c, g): token 16 w + c, p = 16 pi + 4 g .. +4) and
    // stored by the caller later, so that the stores do not sit between the
    // next tile's loads and their first use (one vmcnt counter on gfx9).
    auto compute_tile = [&](const bf16x8 (&cop)[4], bf16x4 (&yout)[4]) {
        // R <- exp(Lam_tile_end - Lam_e) R + B^T (dt w x): A = B^T (n rows), B = (dt w x) (p cols)
        const float dtile = sm.scal[1];
        decprod *= dtile;
#pragma unroll
        for (int ni = 0; ni < 2; ++ni) {
            const bf16x8 bo0 = tr_operand(sm.Bt, kBRow, 0, 32 * w + 16 * ni, g, c);
            const bf16x8 bo1 = tr_operand(sm.Bt, kBRow, 1, 32 * w + 16 * ni, g, c);
#pragma unroll
            for (int pi = 0; pi < 4; ++pi) {
                const bf16x8 xo0 = tr_operand(sm.Xw, kXRow, 0, 16 * pi, g, c);
                const bf16x8 xo1 = tr_operand(sm.Xw, kXRow, 1, 16 * pi, g, c);
                f32x4 acc = R[ni][pi] * dtile;
                acc = mfma32(bo0, xo0, acc);
                acc = mfma32(bo1, xo1, acc);
                R[ni][pi] = acc;
            }
        }
        if constexpr (kOut) {
            const int tl = 16 * w + c;        // token of this lane within the tile
            // (C B^T)^T for s-blocks si <= w (this wave's 16 tokens are block w):
            // lane (c, g) holds [s = 16 si + 4 g + i][t = 16 w + c].
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
            // Decay exp(Lam_t - Lam_s) dt_s under the static causal mask.  For an
            // earlier 16-token block it factorises through that block's last
            // token q: exp(Lam_t - Lam_q) (one exp per block per lane) times the
            // per-token table exp(Lam_q - Lam_s) dt_s; both factors are <= 1.
            // The diagonal block takes exp(Lam_t - Lam_s) directly and masks
            // s > t to zero before any exponential is formed.
            const float lamt = sm.lam[tl];
            bf16x8 mop[2];
#pragma unroll
            for (int si = 0; si < 4; ++si) {
                f32x4 v = zero4;
                if (si < w) {
                    const float f = __expf(lamt - sm.lam[16 * si + 15]);
                    const f32x4 ev = *reinterpret_cast<const f32x4 *>(&sm.ed[16 * si + 4 * g]);
                    v = mt[si] * (ev * f);
                } else if (si == w) {
                    const f32x4 lv = *reinterpret_cast<const f32x4 *>(&sm.lam[16 * si + 4 * g]);
                    const f32x4 dv = *reinterpret_cast<const f32x4 *>(&sm.dtv[16 * si + 4 * g]);
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        v[i] = (4 * g + i <= c) ? mt[si][i] * __expf(lamt - lv[i]) * dv[i] : 0.f;
                }
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    mop[si >> 1][(si & 1) * 4 + i] = (__bf16)v[i];
            }
            // Y^T[p][t] = sum_s x^T[p][s] Lmask[s][t]   (diagonal tile)
            f32x4 yacc[4];
#pragma unroll
            for (int pi = 0; pi < 4; ++pi) {
                yacc[pi] = mfma32(tr_operand(sm.Xt, kXRow, 0, 16 * pi, g, c), mop[0], zero4);
                if (w >= 2)
                    yacc[pi] = mfma32(tr_operand(sm.Xt, kXRow, 1, 16 * pi, g, c), mop[1], yacc[pi]);
            }
            // + exp(Lam_t - Lam_e) R_old C^T   (earlier tiles and earlier chunks)
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
#pragma unroll
            for (int pi = 0; pi < 4; ++pi) {
                const bf16x4 xv = *reinterpret_cast<const bf16x4 *>(
                    sm.Xt + tl * kXRow + (16 * pi + 4 * g) * 2);
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    yout[pi][i] = (__bf16)(yacc[pi][i] + Dh * (float)xv[i]);
            }
        }
    };
    auto write_sb = [&]() {
        if constexpr (kOut) {
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
    };
    auto store_y = [&](const bf16x4 (&yv)[4], int64_t t0y) {
        const int64_t t = t0y + 16 * w + c;
        if (t < L) {
            __bf16 *yp = io.y + t * io.xstride + 4 * g;
#pragma unroll
            for (int pi = 0; pi < 4; ++pi)
                *reinterpret_cast<bf16x4 *>(yp + 16 * pi) = yv[pi];
        }
    };

    if constexpr (kOut) {
        // One tile of loads in flight; y of a tile is stored at the top of the
        // next iteration, before that iteration's loads are issued.  The C rows
        // are consumed from the register set before the next loads overwrite it.
        TileRegs pre;
        load_tile<kOut>(pre, io, tseg0, L, tid);
        store_tile<kOut>(sm, pre, tseg0, L, a.Q, lamE, tid);
        bf16x4 ypend[4];
        for (int64_t t0 = tseg0; t0 < tseg1; t0 += kT) {
            lds_barrier();                        // tile t0 (and Sb) visible in LDS
            bf16x8 cop[4];
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
                cop[ks] = pre.c[ks];
            if (t0 != tseg0)
                store_y(ypend, t0 - kT);
            load_tile<kOut>(pre, io, t0 + kT, L, tid);   // next tile (clamped past the end)
            compute_tile(cop, ypend);
            lds_barrier();                        // every read of this tile's LDS is done
            write_sb();
            if (t0 + kT < tseg1)
                store_tile<kOut>(sm, pre, t0 + kT, L, a.Q, lamE, tid);
        }
        store_y(ypend, tseg0 + ((tseg1 - tseg0 - 1) / kT) * kT);
    } else {
        // State only: two tiles of loads in flight (ring of two register sets).
        TileRegs p0, p1;
        bf16x8 cdummy[4];
        bf16x4 ydummy[4];
        load_tile<kOut>(p0, io, tseg0, L, tid);
        load_tile<kOut>(p1, io, tseg0 + kT, L, tid);
        store_tile<kOut>(sm, p0, tseg0, L, a.Q, lamE, tid);
        for (int64_t t0 = tseg0; t0 < tseg1; t0 += 2 * kT) {
            // tile t0 is in LDS, p1 holds t0 + 64 (in flight), p0 is free
            lds_barrier();
            load_tile<kOut>(p0, io, t0 + 2 * kT, L, tid);
            compute_tile(cdummy, ydummy);
            lds_barrier();
            if (t0 + kT >= tseg1)
                break;
            store_tile<kOut>(sm, p1, t0 + kT, L, a.Q, lamE, tid);
            // tile t0 + 64 is in LDS, p0 holds t0 + 128 (in flight), p1 is free
            lds_barrier();
            load_tile<kOut>(p1, io, t0 + 3 * kT, L, tid);
            compute_tile(cdummy, ydummy);
            lds_barrier();
            store_tile<kOut>(sm, p0, t0 + 2 * kT, L, a.Q, lamE, tid);
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

// Decay preparation: for every (b, h) and token t, the chunk-referenced
// inclusive log-decay Lam_t = sum over the chunk's tokens r <= t of dt_r A_h
// (fp32), stored with dt_t as float2 in [B][H][L] order so that the scan
// kernels read 64 consecutive tokens of one head as one coalesced 512-byte
// row instead of gathering dt with a stride of H floats.  One work-group per
// (b, chunk, 16 heads): dt of the chunk is staged in LDS with 64-byte
// coalesced loads; each wave then scans its heads in 64-token steps (lane =
// token), carrying the running sum across steps.
constexpr int kPrepHeads = 16;
constexpr int kPrepMaxQ = 512;

__global__ __launch_bounds__(256) void decay_prep_kernel(const float *__restrict__ dt,
                                                         const float *__restrict__ A,
                                                         float2 *__restrict__ ld, int64_t L,
                                                         int H, int Q)
{
    __shared__ float sdt[kPrepMaxQ][kPrepHeads + 1];
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
    const int nhg = (H + kPrepHeads - 1) / kPrepHeads;
    const int64_t nc = (L + Q - 1) / Q;
    const int64_t j = blockIdx.x;
    const int hg = (int)(j % nhg);
    const int64_t c = (j / nhg) % nc;
    const int64_t b = j / (nhg * nc);
    const int64_t t0 = c * Q;
    const int qc = (int)((L - t0 < Q) ? (L - t0) : Q);
    const int h0 = hg * kPrepHeads;
    for (int e = tid; e < qc * kPrepHeads; e += 256) {
        const int t = e / kPrepHeads, hh = e % kPrepHeads;
        sdt[t][hh] = (h0 + hh < H) ? dt[(b * L + t0 + t) * H + h0 + hh] : 0.f;
    }
    __syncthreads();
    for (int hh = w; hh < kPrepHeads && h0 + hh < H; hh += 4) {
        const int h = h0 + hh;
        const float Ah = A[h];
        float carry = 0.f;
        float2 *out = ld + ((b * H + h) * L + t0);
        for (int k0 = 0; k0 < qc; k0 += 64) {
            const float d = (k0 + l < qc) ? sdt[k0 + l][hh] : 0.f;
            const float lam = carry + wave_inclusive_sum(d * Ah, l);
            if (k0 + l < qc)
                out[k0 + l] = make_float2(lam, d);
            carry = lane_f(lam, 63);
        }
    }
}

// Kernel 1: end state of segments 0 .. nseg-2 from a zero start.
__global__ __launch_bounds__(kThreads, 2) void seg_state_kernel(SegArgs a)
{
    __shared__ TileSmem<false> sm;
    seg_body<false>(a, sm);
}

// Kernel 3: y of every segment from its entering state, and the final state.
__global__ __launch_bounds__(kThreads, 2) void chunk_scan_kernel(SegArgs a)
{
    __shared__ TileSmem<true> sm;
    seg_body<true>(a, sm);
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

static size_t align256(size_t n)
{
    return (n + 255) / 256 * 256;
}

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
    p.decay_bytes = (size_t)(B * H * p.nslot) * sizeof(float);
    p.ld_bytes = (size_t)(B * H * L) * sizeof(float2);
    p.ws_bytes = align256(p.state_bytes) + align256(p.decay_bytes) + align256(p.ld_bytes);
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
    char *wsb = static_cast<char *>(ws);
    a.ws_state = reinterpret_cast<float *>(wsb);
    a.ws_decay = reinterpret_cast<float *>(wsb + align256(plan.state_bytes));
    float2 *ld = reinterpret_cast<float2 *>(wsb + align256(plan.state_bytes) +
                                            align256(plan.decay_bytes));
    a.ld = ld;
    hipError_t e = log_begin(log, s);
    if (e != hipSuccess)
        return e;
    {
        const int64_t nhg = (H + kPrepHeads - 1) / kPrepHeads;
        decay_prep_kernel<<<(unsigned)(B * plan.nchunks * nhg), 256, 0, s>>>(dt, A, ld, L, (int)H,
                                                                           (int)Q);
        if ((e = hipGetLastError()) != hipSuccess || (e = log_kernel(log, "decay_prep_kernel", s)) != hipSuccess)
            return e;
    }
    if (plan.nseg > 1) {
        a.nseg_launch = a.nseg - 1;
        seg_state_kernel<<<(unsigned)(B * H * (plan.nseg - 1)), kThreads, 0, s>>>(a);
        if ((e = hipGetLastError()) != hipSuccess || (e = log_kernel(log, "seg_state_kernel", s)) != hipSuccess)
            return e;
        const int64_t n = B * H * (kP * kN / 4);
        seg_pass_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(
            init, a.ws_state, a.ws_decay, B * H, a.nseg, a.nslot, a.seg0_from_ws);
        if ((e = hipGetLastError()) != hipSuccess || (e = log_kernel(log, "seg_pass_kernel", s)) != hipSuccess)
            return e;
    }
    a.nseg_launch = a.nseg;
    chunk_scan_kernel<<<(unsigned)(B * H * plan.nseg), kThreads, 0, s>>>(a);
    if ((e = hipGetLastError()) != hipSuccess)
        return e;
    return log_kernel(log, "chunk_scan_kernel", s);
}

}  // namespace ssd
