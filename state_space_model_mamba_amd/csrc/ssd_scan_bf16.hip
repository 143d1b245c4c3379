// bf16 chunked SSD scan on gfx950 MFMA (P = 64, N = 128, Q % 64 == 0).
//
// Source of the method: "Compiler-First State Space Duality and Portable O(1)
// Autoregressive Caching for Inference", section 2 -- the SSD recurrence is
// diagonal per head and chunkable; inside a chunk it is a causal quadratic
// form built from einsum-style contractions under a static lower-triangular
// mask, across chunks a state is passed along, and the decay is exponentiated
// in float32.  With a_t = dt_t A_h and Lam_t the inclusive sum of a over a
// block of tokens:
//
//   segsum      Lseg[t,s] = exp(Lam_t - Lam_s) for s <= t, else 0
//   intra-block Y_diag   = (C B^T o Lseg) (dt x)
//   block state S_out    = exp(Lam_end) S_in + sum_s exp(Lam_end - Lam_s) dt_s x_s (outer) B_s
//   state->out  Y_off[t] = exp(Lam_t) S_in C_t
//   output      y = Y_diag + Y_off + D_h x
//
// The result does not depend on the block length, so the kernels use 64-token
// tiles with Lam referenced to the tile start (every exponent they form is a
// difference Lam_t - Lam_s with s <= t, hence <= 0) and use the chunk length Q
// only to place segment boundaries.  How it maps onto the chip (the page's
// XLA formulation is prior art only):
//
// * Two waves own one head, each half of its P rows.  A wave's 32 x 128 fp32
//   slice of the state R lives in MFMA accumulators for the whole segment,
//   laid out so that the state->output contraction takes its operand straight
//   from those registers, and every product of a tile is local to the P half
//   (y rows and state rows are both indexed by p).  Per tile:
//       Y^T  = exp(Lam_t) R C^T + (x)^T (C B^T o Lseg o dt)^T          (MFMA)
//       R    = exp(Lam_end) R + (B)^T (w o dt o x),  w_s = exp(Lam_end - Lam_s)
//   with D_h folded into the diagonal of the masked C B^T tile.
// * A work-group is four heads of one B/C group (eight waves, two per SIMD):
//   the B and C tiles are staged once in LDS and shared, x of a head is
//   staged by its two waves; all of it double-buffered, one barrier per tile.
//   Each wave scans dt A of its head over the 64 tokens (lane = token), so Lam
//   is one wave-wide prefix sum and the decay tables are private to the wave.
// * K-major operands (B^T and x^T over tokens) come from the token-major LDS
//   tiles through gfx950's transpose read (ds_read_b64_tr_b16); the masked
//   C B^T tile is produced by an MFMA in the layout the next MFMA consumes.
// * The next tile's global loads are issued before the current tile is
//   computed and land in registers (software pipelining).
// * Sequence parallelism: a (b, h) sequence is cut into segments of whole
//   chunks, and segments 0 .. nseg-2 into units.  The state kernel computes
//   each unit's end state from a zero start, with its B and x tiles loaded
//   straight into a three-slot LDS ring two tiles ahead; the scan kernel
//   chains those into the state entering its own segment (S_in[k+1] =
//   decay_k S_in[k] + S_loc[k]) and re-walks the segment from it, writing y
//   (and the final state).  The segment count is chosen so that the scan
//   kernel fills the chip in as few rounds as possible while every extra
//   segment costs one more pass of its x through HBM.
// * Work-groups are remapped so that neighbouring (batch row, segment, head
//   quad) work lands on one XCD and shares its L2 for the B/C tiles.
//
// MFMA operand conventions (v_mfma_f32_16x16x32_bf16, wave64): lane l = c + 16 g
// holds row c of A / column c of B and the K-slots 8 g .. 8 g + 7; the fp32
// result holds D[4 g + i][c].  The K index of a contraction may be assigned to
// slots in any order as long as both operands agree; the maps used here are
// stated where the operands are built.
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
// Heads per scan work-group (two waves, one per P half, per head), which
// share its B/C tiles and C B^T blocks.
constexpr int kScanHeads = 4;
template <int kH> struct Geom {
    static constexpr int kHeads = kH;
    static constexpr int kWaves = 2 * kH;
    static constexpr int kThreads = 64 * kWaves;
    static constexpr int kBPer = kT * 16 / kThreads;  // 16-byte B (and C) chunks per thread
};
// LDS row pitches (bytes).  C is read only row-major (16 bytes per lane from
// rows 16 tb + c, after the permutation below): a 16-byte pad spreads the 16
// rows of a lane group over all banks.
// B is read both row-major and by transpose reads, which no single pitch
// serves, so its rows are unpadded and their 16-byte chunks are permuted by an
// XOR with bswz(row), which makes both patterns conflict-free; x (transpose
// reads only) is unpadded and permuted by xswz(row) the same way.
constexpr int kBRow = kN * 2;                 // B tile [s][n], swizzled
constexpr int kCRow = kN * 2 + 16;            // C tile [t][n]
constexpr int kXRow = kP * 2;                 // x tile [s][p], swizzled
constexpr int kGBlocks = 10;                  // causal 16 x 16 blocks of a 64-token tile
constexpr float kLog2e = 1.4426950408889634f;

template <int kH> struct __align__(16) ScanSmem {
    static constexpr int kHeads = kH, kWaves = 2 * kH;
    unsigned char Bt[2][kT * kBRow];          // B[s][n], ring of two tiles
    unsigned char Ct[2][kT * kCRow];          // C[t][n]
    unsigned char Xt[2][kHeads][kT * kXRow];  // x[s][p] of each head
    f32x4 Gs[kGBlocks][64];                   // (C B^T)^T blocks of the tile, MFMA fragment order
    float lam[kWaves][kT];                    // log2(e) Lam_s, tile-referenced
    float dtv[kWaves][kT];                    // dt_s (0 past the end)
    float vt[kWaves][kT];                     // exp(Lam_q - Lam_s) dt_s, q = last token of s's 16-block
    float gt[kWaves][kT];                     // exp(Lam_t - Lam_p), p = last token of the 16-block before t's
    float wd[kWaves][kT];                     // dt_s 2^(bias - log2(e) Lam_s), see stage_tile
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
    int H, G;
    int hg;              // heads per group
    int nq;              // work-groups (head quads) per group
    int64_t seg_tokens;  // tokens per segment (whole 64-token tiles)
    int64_t unit_tokens; // tokens per state-kernel unit
    int nseg;            // segments per (b, h)
    int nsub;            // state-kernel units per segment
    int nseg_launch;     // segments (scan kernel) or units (state kernel) this launch covers
    int nslot;           // units of segments 0 .. nseg-2, then the spare slot
    int seg0_from_ws;    // segment 0 reads its entering state from slot nseg-1
    const float *dt_bias;  // step-size prep (kSp kernels): dt = softplus(u + dt_bias[h])
};

__device__ __forceinline__ f32x4 mfma32(bf16x8 a, bf16x8 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float fast_exp2(float v)
{
    return __builtin_amdgcn_exp2f(v);
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
// 0), then the three lower rows' totals are added with readlane.
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
// Inclusive prefix sum over the wave's 64 lanes: DPP shifts within each
// 16-lane row, then the earlier rows' totals added as three independent
// selects (no branch; a nested select became divergent branches on this
// dependent chain).
__device__ __forceinline__ float wave_inclusive_sum(float v, int lane)
{
    v += dpp_row_shr<0x111>(v);   // row_shr:1
    v += dpp_row_shr<0x112>(v);   // row_shr:2
    v += dpp_row_shr<0x114>(v);   // row_shr:4
    v += dpp_row_shr<0x118>(v);   // row_shr:8
    const float r0 = lane_f(v, 15), r1 = lane_f(v, 31), r2 = lane_f(v, 47);
    const int row = lane >> 4;
    return v + (((row >= 1 ? r0 : 0.f) + (row >= 2 ? r1 : 0.f)) + (row >= 3 ? r2 : 0.f));
}

// K-major MFMA operand from a token-major LDS tile with gfx950's transpose read
// (ds_read_b64_tr_b16).  Within each 16-lane group the instruction hands
// output lane i, element e, the element (i % 4) of the 8 bytes input lane
// 4e + i/4 addressed.  Input lane (c, g) therefore addresses row
// 32 j + 16 h + 4 g + c/4 and columns col0 + 4 (c % 4) .. +3, so that output
// lane (c, g) receives column col0 + c at rows s = 32 j + 16 h + 4 g + e in
// K-slot 4 h + e -- the token-to-slot map of every contraction over tokens.
__device__ __forceinline__ bf16x8 tr_operand(const unsigned char *tile, int pitch, int j,
                                             int col0, int g, int c)
{
    const unsigned char *p = tile + (32 * j + 4 * g + (c >> 2)) * pitch + (col0 + 4 * (c & 3)) * 2;
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)p);
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(p + 16 * pitch));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

__device__ __forceinline__ int bswz(int row)
{
    return ((row & 7) << 1) | ((row >> 3) & 1);
}
// Byte offset of element n of row `row` in the swizzled B tile.
__device__ __forceinline__ int boff(int row, int n)
{
    return row * kBRow + (((n >> 3) ^ bswz(row)) << 4) + (n & 7) * 2;
}

__device__ __forceinline__ int xswz(int row)
{
    return row & 7;
}

// tr_operand on the swizzled x tile (the swizzle repeats every 8 rows).
__device__ __forceinline__ bf16x8 tr_operand_x(const unsigned char *tile, int j, int col0, int g,
                                               int c)
{
    const int row = 32 * j + 4 * g + (c >> 2), n = col0 + 4 * (c & 3);
    const unsigned char *p = tile + row * kXRow + (((n >> 3) ^ xswz(row)) << 4) + (n & 7) * 2;
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)p);
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(p + 16 * kXRow));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Index of the causal block (sb <= tb) in the shared block array.
constexpr int gblock(int sb, int tb)
{
    return sb * 4 - sb * (sb - 1) / 2 + (tb - sb);
}

// tr_operand on the swizzled B tile (the row's swizzle repeats every 16 rows,
// so the upper half of the operand sits 16 rows further down unchanged).
__device__ __forceinline__ bf16x8 tr_operand_b(const unsigned char *tile, int j, int col0, int g,
                                               int c)
{
    const unsigned char *p = tile + boff(32 * j + 4 * g + (c >> 2), col0 + 4 * (c & 3));
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)p);
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(p + 16 * kBRow));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// n_operand on the swizzled B tile.
__device__ __forceinline__ bf16x8 n_operand_b(const unsigned char *tile, int row, int kk, int g)
{
    const bf16x4 lo = *reinterpret_cast<const bf16x4 *>(tile + boff(row, 32 * kk + 4 * g));
    const bf16x4 hi = *reinterpret_cast<const bf16x4 *>(tile + boff(row, 32 * kk + 16 + 4 * g));
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// The C tile is stored with each 32-element block of n permuted so that the
// operand's K-slots (n = 32 kk + 16 h + 4 g + i at slot 4 h + i of lane group
// g) are 8 contiguous elements: n_local = 16 h + 4 g + i sits at 8 g + 4 h + i.
// Staging: the 16-byte chunk `col` (n = 8 col .. +7, m = col % 4 within its
// block) splits into two 8-byte halves (g = 2 (m % 2) and g + 1, h = m / 2).
__device__ __forceinline__ void cstage(unsigned char *row, int col, uint4 v)
{
    const int m = col & 3;
    const int p0 = (col & ~3) * 8 + 16 * (m & 1) + 4 * (m >> 1);   // element position
    *reinterpret_cast<uint2 *>(row + p0 * 2) = make_uint2(v.x, v.y);
    *reinterpret_cast<uint2 *>(row + (p0 + 8) * 2) = make_uint2(v.z, v.w);
}
// The operand from the permuted C tile: one 16-byte read.
__device__ __forceinline__ bf16x8 c_operand(const unsigned char *tile, int row, int kk, int g)
{
    return *reinterpret_cast<const bf16x8 *>(tile + row * kCRow + (32 * kk + 8 * g) * 2);
}

// Row-major MFMA operand over n from a [row][n] LDS tile.  K-slot 4 h + i of
// lane group g is n = 32 kk + 16 h + 4 g + i -- the map under which the state
// accumulators (rows n = 16 nb + 4 g + i) are directly an operand.
__device__ __forceinline__ bf16x8 n_operand(const unsigned char *tile, int pitch, int row, int kk,
                                            int g)
{
    const unsigned char *p = tile + row * pitch + (32 * kk + 4 * g) * 2;
    const bf16x4 lo = *reinterpret_cast<const bf16x4 *>(p);
    const bf16x4 hi = *reinterpret_cast<const bf16x4 *>(p + 32);
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// One tile's global inputs, held in registers while the previous tile is being
// computed.  B and C are loaded by the whole work-group (16-byte chunk
// tid + 512 r of the [64][16 x 16 B] tile); x by the two waves of its head
// (chunk pt + 128 r of the [64][8 x 16 B] tile, pt = thread within the pair);
// dt by every wave, lane = token.
template <int kH> struct Prefetch {
    uint4 b[Geom<kH>::kBPer];
    uint4 c[Geom<kH>::kBPer];
    uint4 x[4];
    float dt;
};

struct WaveIo {
    const __bf16 *x, *B, *C;   // at token 0 of this (b, head) / (b, group)
    const float *dt;
    int64_t xstride, bstride;  // elements per token
    int dtstride;
};

typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __amdgpu_buffer_rsrc_t rsrc_t;

// Buffer resource (raw, 32-bit data: the gfx9-family descriptor word) over
// the rows of a tile starting at `base` of which min(rows, kT) are valid
// (none if rows <= 0).  Buffer loads past its end return zero and stores
// there are dropped, so one resource per tile both bounds and zero-fills a
// ragged tile without per-lane arithmetic.  It is computed without branches:
// a select around the loads would make the compiler duplicate them and lose
// track of which are in flight.  A tile spans at most kT rows, so its byte
// count is 32-bit.
__device__ __forceinline__ rsrc_t tile_rsrc(const void *base, int64_t rows, unsigned pitch,
                                            unsigned row_bytes)
{
    const int r = (int)std::max<int64_t>(0, std::min<int64_t>(rows, kT));
    const int bytes = std::max(r * (int)pitch - (int)pitch + (int)row_bytes, 0);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, bytes, 0x00020000);
}

// Issue the global loads of the tile starting at t0, through buffer resources
// that end at token L (the caller passes the segment's end), so a ragged tile
// reads zeros and a tile past the end reads nothing.  Always the same
// instructions with no branches, so the compiler's wait-count analysis sees
// exactly which loads are outstanding and a prefetched tile stays in flight
// while the current one is computed.  Offsets are 32-bit (a tile spans at
// most 64 rows of H*P or G*N elements).  kPart: 1 = B, C and dt; 2 = x; 3 =
// all of them.
template <int kH, int kPart = 3>
__device__ __forceinline__ void load_tile(Prefetch<kH> &pf, const WaveIo &io, int64_t t0,
                                          int64_t L, int tid)
{
    constexpr int kPer = Geom<kH>::kBPer, kRows = Geom<kH>::kThreads / 16;
    const int l = tid & 63, pt = tid & 127;
    const int64_t rows = L - t0;
    if constexpr ((kPart & 1) != 0) {
        // dt first: it is consumed mid-tile (the fused step-size prep) while
        // the B and C loads issued after it may still be in flight
        const unsigned dp = (unsigned)io.dtstride * 4u;
        const rsrc_t rd = tile_rsrc(io.dt + t0 * io.dtstride, rows, dp, 4);
        pf.dt = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rd, (unsigned)l * dp, 0, 0));
        const unsigned bp = (unsigned)io.bstride * 2u;
        const rsrc_t rb = tile_rsrc(io.B + t0 * io.bstride, rows, bp, kN * 2);
#pragma unroll
        for (int r = 0; r < kPer; ++r) {
            const unsigned off = (unsigned)((tid >> 4) + kRows * r) * bp + (tid & 15) * 16u;
            pf.b[r] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rb, off, 0, 0));
        }
        const rsrc_t rc = tile_rsrc(io.C + t0 * io.bstride, rows, bp, kN * 2);
#pragma unroll
        for (int r = 0; r < kPer; ++r) {
            const unsigned off = (unsigned)((tid >> 4) + kRows * r) * bp + (tid & 15) * 16u;
            pf.c[r] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rc, off, 0, 0));
        }
    }
    if constexpr ((kPart & 2) != 0) {
        const unsigned xp = (unsigned)io.xstride * 2u;
        const rsrc_t rx = tile_rsrc(io.x + t0 * io.xstride, rows, xp, kP * 2);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const unsigned off = (unsigned)((pt >> 3) + 16 * r) * xp + (pt & 7) * 16u;
            pf.x[r] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rx, off, 0, 0));
        }
    }
}

// The state is held scaled: R = 2^ls Z with a wave-uniform ls in [-kRenorm, 0].
// A tile's decay 2^lam_end then only moves ls (and the per-token weights of
// the update absorb 2^-ls), instead of multiplying all of Z; Z is rescaled
// only when ls would fall below -kRenorm, and a tile whose own decay exceeds
// that is applied to Z directly.  Every factor formed stays within 2^(2 kRenorm).
constexpr float kRenorm = 48.f;

// The wave's index in the work-group, as a scalar: everything derived from it
// (head, pointers, buffer descriptors) then stays in scalar registers.
__device__ __forceinline__ int wave_id()
{
    return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
}

// A wave-uniform condition as a scalar branch (the values it derives from are
// wave-uniform, but the compiler cannot always prove it through the loop).
__device__ __forceinline__ bool uniform(bool v)
{
    return __builtin_amdgcn_readfirstlane((int)v) != 0;
}

struct TileMode {
    float ly;       // ls of the state entering the tile (decay of Y_off)
    float eyl;      // 2^ly
    float zscale;   // direct mode: Z <- zscale Z + update
    bool direct;
    bool renorm;    // before the tile: Z <- rscale Z
    float rscale;
};

// How a tile with total log2 decay lam_end treats the state R = 2^ls Z (see
// kRenorm); updates ls and lsum (the unit's total log2 decay).  The tile's
// update weights are wd_s = dt_s 2^(bias - lam_s).
__device__ __forceinline__ TileMode tile_mode(float lam_end, float &ls, float &lsum, float &bias)
{
    // (selects rather than branches: the decision ends a dependent chain from
    // the step sizes, and branches here would split the code that follows
    // from that chain)
    lsum += lam_end;
    TileMode md;
    const bool direct = lam_end < -kRenorm;
    const bool renorm = !direct && ls + lam_end < -kRenorm;
    const float ls_in = renorm ? 0.f : ls;       // ls after a renormalisation
    md.direct = direct;
    md.renorm = renorm;
    md.rscale = renorm ? fast_exp2(ls) : 1.f;
    md.ly = direct ? ls : ls_in;
    md.zscale = direct ? fast_exp2(ls + lam_end) : 1.f;
    bias = direct ? lam_end : -ls_in;
    ls = direct ? 0.f : ls_in + lam_end;
    md.eyl = fast_exp2(md.ly);
    return md;
}

// Z <- zscale Z + B^T (wd x) over one tile, with Z[nb][q][i] the state rows
// n = 16 nb + 4 g + i, column p = 32 ph + 16 q + c (lane (c, g)) of this
// wave's P half.  A = B^T (rows n) from the swizzled B tile, B = x^T scaled by
// the tile's weights wd (64 floats, token-indexed).  The B^T operands are read
// kAhead blocks ahead of their MFMAs, so that their LDS latency overlaps the
// x scaling and the previous blocks' MFMAs.
// The B operand of the state update: x^T scaled by the tile's weights wd
// (64 floats, token-indexed; K-slot 4 h + i <-> token 32 jj + 16 h + 4 g + i).
__device__ __forceinline__ void scale_x(bf16x8 (&XS)[2][2], const bf16x8 (&XT)[2][2],
                                        const float *wd, int g)
{
    f32x4 wv[2][2];
#pragma unroll
    for (int jj = 0; jj < 2; ++jj)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
            wv[jj][hh] = *reinterpret_cast<const f32x4 *>(&wd[32 * jj + 16 * hh + 4 * g]);
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
        for (int jj = 0; jj < 2; ++jj)
#pragma unroll
            for (int e = 0; e < 8; ++e)
                XS[q][jj][e] = (__bf16)((float)XT[q][jj][e] * wv[jj][e >> 2][e & 3]);
}

// Z <- zscale Z + B^T (wd x) over one tile, with Z[nb][q][i] the state rows
// n = 16 nb + 4 g + i, column p = 32 ph + 16 q + c (lane (c, g)) of this
// wave's P half.  A = B^T (rows n) from the swizzled B tile, B = XS (scale_x).
// The B^T operands are read kAhead blocks ahead of their MFMAs, so that their
// LDS latency overlaps the previous blocks' MFMAs.
template <int kAhead>
__device__ __forceinline__ void state_update(f32x4 (&Z)[8][2], const unsigned char *Bs,
                                             const bf16x8 (&XS)[2][2], const TileMode &md,
                                             int g, int c)
{
    bf16x8 BT[8][2];
#pragma unroll
    for (int nb = 0; nb < kAhead; ++nb) {
        BT[nb][0] = tr_operand_b(Bs, 0, 16 * nb, g, c);
        BT[nb][1] = tr_operand_b(Bs, 1, 16 * nb, g, c);
    }
    if (uniform(md.direct)) {
#pragma unroll
        for (int nb = 0; nb < 8; ++nb)
#pragma unroll
            for (int q = 0; q < 2; ++q)
                Z[nb][q] *= md.zscale;
    }
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) {
        if (nb + kAhead < 8) {
            BT[nb + kAhead][0] = tr_operand_b(Bs, 0, 16 * (nb + kAhead), g, c);
            BT[nb + kAhead][1] = tr_operand_b(Bs, 1, 16 * (nb + kAhead), g, c);
        }
#pragma unroll
        for (int q = 0; q < 2; ++q)
            Z[nb][q] = mfma32(BT[nb][1], XS[q][1], mfma32(BT[nb][0], XS[q][0], Z[nb][q]));
    }
}

// The state update of state_update on B^T operands read beforehand (all of
// them, so that their LDS latency overlaps whatever comes between).
__device__ __forceinline__ void state_update_pre(f32x4 (&Z)[8][2], const bf16x8 (&BT)[8][2],
                                                 const bf16x8 (&XS)[2][2], const TileMode &md)
{
    if (uniform(md.direct)) {
#pragma unroll
        for (int nb = 0; nb < 8; ++nb)
#pragma unroll
            for (int q = 0; q < 2; ++q)
                Z[nb][q] *= md.zscale;
    }
#pragma unroll
    for (int nb = 0; nb < 8; ++nb)
#pragma unroll
        for (int q = 0; q < 2; ++q)
            Z[nb][q] = mfma32(BT[nb][1], XS[q][1], mfma32(BT[nb][0], XS[q][0], Z[nb][q]));
}

// A tile's decay tables, formed in registers from its step sizes (lane =
// token) before they are staged: each wave scans a_t = dt_t A_h over its 64
// tokens, in log2 units.  Updates ls (and lsum, the segment's total log2
// decay) and returns how the tile treats the state.  No other use of ls comes
// between this and the tile, so the tables of tile k + 1 can be formed while
// tile k is computed.
struct Tables {
    float lam, dtv, vt, wd, gt;
    TileMode md;
};
__device__ __forceinline__ Tables tile_tables(float dtl, int64_t t0, int64_t L, float Ah2, float &ls,
                                              float &lsum, int l)
{
    Tables tb;
    const float lam = wave_inclusive_sum(dtl * Ah2, l);
    // Lam at the last valid token (in a ragged tile the zero-dt lanes after it
    // hold the same sum only up to the summation order, which matters when
    // the decay is extreme and Lam is large)
    // (a scalar: readlane needs a uniform lane)
    const int last = __builtin_amdgcn_readfirstlane(
        (int)std::min<int64_t>(std::max<int64_t>(L - t0, 1), kT) - 1);
    const float lam_end = lane_f(lam, last);
    float bias;
    tb.md = tile_mode(lam_end, ls, lsum, bias);
    tb.wd = fast_exp2(bias - lam) * dtl;
    const float q0 = lane_f(lam, 15), q1 = lane_f(lam, 31), q2 = lane_f(lam, 47);
    const int row = l >> 4;
    const float lq = row == 0 ? q0 : row == 1 ? q1 : row == 2 ? q2 : lam_end;
    tb.lam = lam;
    tb.dtv = dtl;
    tb.vt = fast_exp2(lq - lam) * dtl;
    // the decay from the end of the previous 16-token block (Lam = 0 before
    // the tile): every factor of the tile's row decays is a product of these
    const float lp = row == 0 ? 0.f : row == 1 ? q0 : row == 2 ? q1 : q2;
    tb.gt = fast_exp2(lam - lp);
    return tb;
}

// Registers -> LDS for one tile: B, C, this head's x, and the wave's tables.
template <int kH>
__device__ __forceinline__ void stage_tile(ScanSmem<kH> &sm, Prefetch<kH> &pf, int slot,
                                           const Tables &tb, int tid)
{
    constexpr int kPer = Geom<kH>::kBPer, kRows = Geom<kH>::kThreads / 16;
    const int w = wave_id(), l = tid & 63, pt = tid & 127;
    // (rows past the end were loaded as zeros)
#pragma unroll
    for (int r = 0; r < kPer; ++r) {
        const int row = (tid >> 4) + kRows * r, col = tid & 15;
        *reinterpret_cast<uint4 *>(sm.Bt[slot] + row * kBRow + ((col ^ bswz(row)) << 4)) = pf.b[r];
        cstage(sm.Ct[slot] + row * kCRow, col, pf.c[r]);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int row = (pt >> 3) + 16 * r;
        *reinterpret_cast<uint4 *>(sm.Xt[slot][w >> 1] + row * kXRow +
                                   (((pt & 7) ^ xswz(row)) << 4)) = pf.x[r];
    }
    sm.wd[w][l] = tb.wd;
    sm.lam[w][l] = tb.lam;
    sm.dtv[w][l] = tb.dtv;
    sm.vt[w][l] = tb.vt;
    sm.gt[w][l] = tb.gt;
}

// The fused step-size prep on a prefetched tile at t0 (lane = token): the
// step size from u, tokens past the end L keep 0.
template <int kH, bool kSp>
__device__ __forceinline__ void prep_dt(Prefetch<kH> &pf, int64_t t0, int64_t L, float dtb, int l)
{
    if constexpr (kSp)
        pf.dt = l < L - t0 ? softplus_dt(pf.dt, dtb) : 0.f;
}

// The scan kernel: y of segment `seg` from the state entering it and, for the
// last segment, the final state.
// `bid` of `nblk` is the work-group's index among those of its launch (or of
// its run, when one launch covers several problems).
template <int kH, bool kSp>
__device__ __forceinline__ void scan_body(const SegArgs &a, ScanSmem<kH> &sm, int64_t bid,
                                          int64_t nblk)
{
    constexpr int kHeads = kH, kWaves = 2 * kH;
    const int tid = threadIdx.x, w = wave_id(), l = tid & 63, g = l >> 4, c = l & 15;
    const int hs = w >> 1;                                // head slot in the work-group
    // One wave of each pair that shares a SIMD (w and w + 4, or 2k and 2k + 1:
    // the even-parity wave indices 0, 3, 5, 6 hold one of each either way)
    // takes issue priority from the mid-tile barrier until its y stores are
    // issued (before the state update), so that the pair's VALU-bound
    // masked-operand builds and MFMA-bound products drift apart instead of
    // running side by side.
    const bool lead = (__builtin_popcount(w) & 1) == 0;
    const int ph = w & 1;                                 // P half: p = 32 ph .. 32 ph + 31
    const int64_t j = xcd_remap(bid, nblk);
    const int nquad = a.G * a.nq;
    const int quad = (int)(j % nquad);
    const int64_t r = j / nquad;
    const int seg = (int)(r % a.nseg_launch);
    const int64_t b = r / a.nseg_launch;
    const int grp = quad / a.nq;
    const int hw = (quad % a.nq) * kHeads + hs;           // head within the group
    const bool active = hw < a.hg;                        // idle slots mirror the last head
    const int h = grp * a.hg + (active ? hw : a.hg - 1);
    const int64_t bh = b * a.H + h;
    const int64_t L = a.L;
    const int64_t tseg0 = (int64_t)seg * a.seg_tokens;
    const int64_t tseg1 = std::min<int64_t>(L, tseg0 + a.seg_tokens);
    const float Ah2 = a.A[h] * kLog2e;
    const float dtb = kSp && a.dt_bias ? a.dt_bias[h] : 0.f;
    const float Dh = a.D[h];
    const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};

    WaveIo io;
    io.xstride = (int64_t)a.H * kP;
    io.bstride = (int64_t)a.G * kN;
    io.dtstride = a.H;
    io.x = a.x + (b * L * a.H + h) * kP;
    io.B = a.B + (b * L * a.G + grp) * kN;
    io.C = a.C + (b * L * a.G + grp) * kN;
    io.dt = a.dt + b * L * a.H + h;
    // y as stored: lane (c, g) of token block tb writes row 16 tb + c, columns
    // 32 ph + 8 g .. +7; byte offsets from the tile's first row (a tile spans 64
    // rows of H * P elements)
    const int64_t ystride = (int64_t)a.H * kP;
    __bf16 *ybase = a.y + (b * L * a.H + h) * kP;
    const unsigned ylane = ((unsigned)c * (unsigned)ystride + 32u * ph + 8u * g) * 2u;

    // State accumulators: Z[nb][q][i] = R[p = 32 ph + 16 q + c][n = 16 nb + 4 g + i] / 2^ls.
    const int zoff = (32 * ph + c) * kN + 4 * g;      // + 16 q kN + 16 nb
    f32x4 Z[8][2];
    {
        // The state entering the segment, from the initial state and the end
        // states S_k of the earlier units (state kernel), i.e. the
        // chain S <- d_k S + S_k written out as
        //   S_in = (prod_k d_k) S_init + sum_k (prod_{j > k} d_j) S_k,
        // summed from the last unit backwards so that the loads of all units
        // are independent and can be in flight together (fp32, fixed order).
        // When the final state aliases the initial state, the state kernel has
        // copied the initial state to the spare slot.
        const float *src = nullptr;
        if (a.seg0_from_ws)
            src = a.ws_state + (bh * a.nslot + (a.nslot - 1)) * kP * kN;
        else if (a.init)
            src = a.init + bh * kP * kN;
#pragma unroll
        for (int nb = 0; nb < 8; ++nb)
#pragma unroll
            for (int q = 0; q < 2; ++q)
                Z[nb][q] = zero4;
        float wgt = 1.f;                              // prod_{j > k} d_j
#pragma unroll 2
        for (int k = seg * a.nsub - 1; k >= 0; --k) {
            const float *sl = a.ws_state + (bh * a.nslot + k) * kP * kN;
#pragma unroll
            for (int nb = 0; nb < 8; ++nb)
#pragma unroll
                for (int q = 0; q < 2; ++q)
                    Z[nb][q] += *reinterpret_cast<const f32x4 *>(sl + zoff + 16 * q * kN + 16 * nb) * wgt;
            wgt *= a.ws_decay[bh * a.nslot + k];
        }
        if (src) {
#pragma unroll
            for (int nb = 0; nb < 8; ++nb)
#pragma unroll
                for (int q = 0; q < 2; ++q)
                    Z[nb][q] += *reinterpret_cast<const f32x4 *>(src + zoff + 16 * q * kN + 16 * nb) * wgt;
        }
    }
    float ls = 0.f;         // R = 2^ls Z
    float lsum = 0.f;       // log2 of the product of tile decays over the segment

    // R <- zscale R + B^T (w dt x); the prefetched tile is live here, so the
    // B^T operands are read half a tile ahead
    auto update_state = [&](const unsigned char *Bs, const bf16x8 (&XS)[2][2], const TileMode &md) {
        state_update<4>(Z, Bs, XS, md, g, c);
    };

    // y of the tile at t0 from the state entering it, then the state update.
    Prefetch<kH> pf;
    Tables tnext;
    auto compute_tile = [&](int slot, const TileMode &md, int64_t t0) {
        const unsigned char *Xs = sm.Xt[slot][hs];
        const unsigned char *Bs = sm.Bt[slot];
        bf16x8 XT[2][2];      // x^T: rows p (this wave's half), K over tokens
        bf16x8 XS[2][2];      // x^T scaled by the update weights
        {
            const unsigned char *Cs = sm.Ct[slot];
            // (C B^T)^T causal blocks, shared by the four heads: wave w computes
            // blocks w and w + 8 of the ten; lane (c, g) of block (sb, tb) holds
            // [s = 16 sb + 4 g + i][t = 16 tb + c].
#pragma unroll
            for (int bi0 = 0; bi0 < kGBlocks; bi0 += kWaves) {
                const int bi = bi0 + w;
                if (bi < kGBlocks) {
                    const int sb = bi < 4 ? 0 : bi < 7 ? 1 : bi < 9 ? 2 : 3;
                    const int tb = bi - gblock(sb, sb) + sb;
                    f32x4 gacc = zero4;
#pragma unroll
                    for (int kk = 0; kk < 4; ++kk)
                        gacc = mfma32(n_operand_b(Bs, 16 * sb + c, kk, g),
                                      c_operand(Cs, 16 * tb + c, kk, g), gacc);
                    sm.Gs[bi][l] = gacc;
                }
            }
            // x of the next tile goes out now, so that its registers are not
            // live across the C B^T blocks.
            load_tile<kH, 2>(pf, io, t0 + kT, tseg1, tid);
            // Y^T[p][t] = 2^ls exp(Lam_t) sum_n Z[p][n] C[t][n]   (A = Z straight from the accumulators)
            f32x4 Y[2][4];
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                bf16x8 CF[4];
#pragma unroll
                for (int tb = 0; tb < 4; ++tb)
                    CF[tb] = c_operand(Cs, 16 * tb + c, kk, g);
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    bf16x8 za;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        za[i] = (__bf16)Z[2 * kk][q][i];
                        za[4 + i] = (__bf16)Z[2 * kk + 1][q][i];
                    }
#pragma unroll
                    for (int tb = 0; tb < 4; ++tb)
                        Y[q][tb] = mfma32(za, CF[tb], kk == 0 ? zero4 : Y[q][tb]);
                }
            }
            // Row decays 2^(Lam_t + ly) and the off-diagonal factors
            // 2^(Lam_t - Lam_q(sb)) as products of the tables' block decays
            // (all factors at most 1): pt = 2^(Lam_t - Lam_p) for t's row,
            // bj = the decay across block j, eb = 2^(Lam_p + ly).
            float lamt[4], pt[4];
            const float b1 = sm.gt[w][31], b2 = sm.gt[w][47];
            float eb[4];
            eb[0] = md.eyl;
            eb[1] = eb[0] * sm.gt[w][15];
            eb[2] = eb[1] * b1;
            eb[3] = eb[2] * b2;
#pragma unroll
            for (int tb = 0; tb < 4; ++tb) {
                lamt[tb] = sm.lam[w][16 * tb + c];
                pt[tb] = sm.gt[w][16 * tb + c];
                const float dec = pt[tb] * eb[tb];
#pragma unroll
                for (int q = 0; q < 2; ++q)
                    Y[q][tb] *= dec;
            }
            lds_barrier();                            // every block of the tile is in Gs
            if (lead)
                __builtin_amdgcn_s_setprio(2);
            // the next tile's step sizes and decay tables, well before they
            // are staged at the end of this tile
            prep_dt<kH, kSp>(pf, t0 + kT, tseg1, dtb, l);
            tnext = tile_tables(pf.dt, t0 + kT, tseg1, Ah2, ls, lsum, l);
            // Mask and decay, B-operand over tokens s (slot 4 h + i <-> s = 32 jj + 16 h + 4 g + i):
            //   s in an earlier 16-block: exp(Lam_t - Lam_q) * [exp(Lam_q - Lam_s) dt_s]
            //   s in t's 16-block      : exp(Lam_t - Lam_s) dt_s for s <= t (exponent
            //                            masked to -inf above the diagonal), + D_h at s = t
            bf16x8 MOP[4][2];
#pragma unroll
            for (int tb = 0; tb < 4; ++tb) {
#pragma unroll
                for (int jj = 0; jj < 2; ++jj) {
#pragma unroll
                    for (int hh = 0; hh < 2; ++hh) {
                        const int sb = 2 * jj + hh;
                        f32x4 v = zero4;
                        if (sb < tb) {
                            // 2^(Lam_t - Lam_q(sb)): blocks sb + 1 .. tb - 1 lie between
                            const float u = sb + 1 == tb ? pt[tb] : sb + 2 == tb ? pt[tb] * (tb == 2 ? b1 : b2)
                                                                                 : pt[tb] * (b1 * b2);
                            const f32x4 vt = *reinterpret_cast<const f32x4 *>(&sm.vt[w][16 * sb + 4 * g]);
                            v = sm.Gs[gblock(sb, tb)][l] * (vt * u);
                        } else if (sb == tb) {
                            const f32x4 gd = sm.Gs[gblock(sb, tb)][l];
                            const f32x4 lsv = *reinterpret_cast<const f32x4 *>(&sm.lam[w][16 * sb + 4 * g]);
                            const f32x4 ds = *reinterpret_cast<const f32x4 *>(&sm.dtv[w][16 * sb + 4 * g]);
#pragma unroll
                            for (int i = 0; i < 4; ++i) {
                                const bool causal = 4 * g + i <= c;
                                const float e = fast_exp2(causal ? lamt[tb] - lsv[i] : -INFINITY);
                                v[i] = gd[i] * e * ds[i] + ((4 * g + i == c) ? Dh : 0.f);
                            }
                        }
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            MOP[tb][jj][4 * hh + i] = (__bf16)v[i];
                    }
                }
            }
#pragma unroll
            for (int q = 0; q < 2; ++q)
#pragma unroll
                for (int jj = 0; jj < 2; ++jj)
                    XT[q][jj] = tr_operand_x(Xs, jj, 32 * ph + 16 * q, g, c);
            // Y^T += x^T (masked C B^T)^T over the causal token blocks, then y = bf16(Y)
#pragma unroll
            for (int q = 0; q < 2; ++q)
#pragma unroll
                for (int tb = 0; tb < 4; ++tb) {
                    Y[q][tb] = mfma32(XT[q][0], MOP[tb][0], Y[q][tb]);
                    if (tb >= 2)
                        Y[q][tb] = mfma32(XT[q][1], MOP[tb][1], Y[q][tb]);
                }
            // the update's operand, formed while the products above run
            scale_x(XS, XT, sm.wd[w], g);
            // Lane (c, g) holds columns 16 q + 4 g .. +3 (q = 0, 1) of the wave's
            // half of row 16 tb + c.  Swapping the upper and lower 32 lanes of the
            // q = 1 and q = 0 registers, then the odd and even 16-lane rows, leaves
            // lane (c, g) with columns 8 g .. 8 g + 7 in (r0, r1), so one store
            // writes 16 rows x 64 contiguous bytes.  Rows past the end fall
            // outside the descriptor and are dropped, and an idle wave's
            // descriptor is empty.  The stores are issued on every path: under a
            // branch, the wait for the next tile's loads in stage_tile would also
            // wait for these stores to complete.
            const rsrc_t ry = tile_rsrc(ybase + t0 * ystride, active ? L - t0 : 0, (unsigned)ystride * 2u, kP * 2);
#pragma unroll
            for (int tb = 0; tb < 4; ++tb) {
                bf16x4 y0, y1;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    y0[i] = (__bf16)Y[0][tb][i];
                    y1[i] = (__bf16)Y[1][tb][i];
                }
                u32x2 r0 = __builtin_bit_cast(u32x2, y0), r1 = __builtin_bit_cast(u32x2, y1);
#pragma unroll
                for (int d = 0; d < 2; ++d) {
                    const u32x2 s32 = __builtin_amdgcn_permlane32_swap(r0[d], r1[d], false, false);
                    const u32x2 s16 = __builtin_amdgcn_permlane16_swap(s32[0], s32[1], false, false);
                    r0[d] = s16[0];
                    r1[d] = s16[1];
                }
                const u32x4 v = {r0[0], r0[1], r1[0], r1[1]};
                __builtin_amdgcn_raw_buffer_store_b128(v, ry, ylane + 32u * tb * (unsigned)ystride, 0, 0);
            }
        }
        if (lead)
            __builtin_amdgcn_s_setprio(0);
        update_state(Bs, XS, md);
    };

    // Z <- 2^ls Z, ls restarting at 0, before a tile that would take ls below
    // -kRenorm (a uniform branch)
    auto renorm = [&](const TileMode &md) {
        if (uniform(md.renorm)) {
#pragma unroll
            for (int nb = 0; nb < 8; ++nb)
#pragma unroll
                for (int q = 0; q < 2; ++q)
                    Z[nb][q] *= md.rscale;
        }
    };
    // Tile k is staged in ring slot k & 1 (B, C, x) and in the wave's own
    // tables; tile k + 1's loads are in flight in `pf` while tile k is
    // computed.  The barrier at the top of an iteration publishes the slot
    // written at the end of the previous one and guarantees every wave is done
    // reading the slot the current iteration will overwrite.  Loads end at
    // the segment's last token: the tile after it reads as zeros, and staging
    // it leaves ls unchanged, so every iteration stages without a branch
    // (which lets the compiler interleave the staging with the update).
    load_tile<kH>(pf, io, tseg0, tseg1, tid);
    prep_dt<kH, kSp>(pf, tseg0, tseg1, dtb, l);
    tnext = tile_tables(pf.dt, tseg0, tseg1, Ah2, ls, lsum, l);
    stage_tile<kH>(sm, pf, 0, tnext, tid);
    int slot = 0;
    for (int64_t t0 = tseg0; t0 < tseg1; t0 += kT) {
        lds_barrier();
        const TileMode md = tnext.md;
        renorm(md);
        // next tile (nothing past the end); x follows mid-tile
        load_tile<kH, 1>(pf, io, t0 + kT, tseg1, tid);
        compute_tile(slot, md, t0);
        slot ^= 1;
        stage_tile<kH>(sm, pf, slot, tnext, tid);
    }

    if (!active || seg != a.nseg - 1)
        return;
    {
        float *dst = a.fin + bh * kP * kN;
        const float sc = fast_exp2(ls);
#pragma unroll
        for (int nb = 0; nb < 8; ++nb)
#pragma unroll
            for (int q = 0; q < 2; ++q)
                *reinterpret_cast<f32x4 *>(dst + (32 * ph + 16 * q + c) * kN + 16 * nb + 4 * g) =
                    Z[nb][q] * sc;
    }
}

// State kernel: the end state of every unit (part of segments 0 .. nseg-2)
// from a zero start, and the unit's total decay.  A unit is a plain sequence
// of tile updates, so what bounds it is how much of HBM's latency its loads
// can hide: its B and x tiles go straight from memory into a ring of three
// LDS slots (buffer loads with an LDS destination, no registers in between),
// two tiles ahead of the one being computed, with one barrier per tile.
// Four heads per work-group share each B tile; wave w = (head w / 2, P half
// w % 2) loads half of its own head's x tile, and the step sizes of 8 tokens
// for all four heads (16 contiguous bytes per token: one cache line per token,
// not one per token and wave).
constexpr int kStHeads = 4, kStWaves = 2 * kStHeads, kStThreads = 64 * kStWaves;
constexpr int kStBBlocks = kT * kBRow / 1024 / kStWaves;   // 1 KB B blocks per wave per tile
constexpr int kStXBlocks = kT * kXRow / 1024 / 2;          // 1 KB x blocks per wave per tile
constexpr int kStLoads = kStBBlocks + kStXBlocks + 1;      // memory instructions per wave per tile (+ dt)
constexpr size_t kStSmemBytes = 3 * (size_t)kT * (kBRow + kStHeads * kXRow + kStHeads * 4) + (size_t)kStWaves * kT * 4;
static_assert(kStWaves * 8 == kT && kStHeads == 4, "each wave loads the dt of 8 tokens x 4 heads");

struct StIo {
    const __bf16 *B, *x;       // this (b, group) / (b, head) at token 0
    const float *dt;
    int64_t bp, xp, dp;        // bytes per token
    unsigned boff[kStBBlocks]; // this lane's source offset within a tile, per block
    unsigned xoff[kStXBlocks];
    unsigned doff;
    unsigned dbytes;           // bytes of dt per token for this quad's heads (4 per head)
};

// Buffer resource words over the valid rows of a tile (as tile_rsrc), for
// the loads below.
__device__ __forceinline__ u32x4 tile_words(const void *base, int64_t rows, unsigned pitch,
                                            unsigned row_bytes)
{
    const int r = (int)std::max<int64_t>(0, std::min<int64_t>(rows, kT));
    const uint64_t p = reinterpret_cast<uint64_t>(base);
    u32x4 d;
    d.x = __builtin_amdgcn_readfirstlane((unsigned)p);
    d.y = __builtin_amdgcn_readfirstlane((unsigned)(p >> 32)) & 0xffffu;
    d.z = __builtin_amdgcn_readfirstlane((unsigned)std::max(r * (int)pitch - (int)pitch + (int)row_bytes, 0));
    d.w = 0x00020000u;
    return d;
}

// Buffer loads with an LDS destination: lane l's 16 (4) bytes land at
// dst + 16 l (4 l).  They are written out here so that the compiler does not
// insert its own waits for them (it cannot tell the ring slots apart and
// would wait for every one in flight); their reader waits with wait_vmcnt and
// a barrier.  Nothing is written to registers.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void lds_load16(unsigned dst, u32x4 rsrc, unsigned voff)
{
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :: "s"(dst), "v"(voff), "s"(rsrc) : "memory", "m0");
}
__device__ __forceinline__ void lds_load4(unsigned dst, u32x4 rsrc, unsigned voff)
{
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, 0 offen lds"
                 :: "s"(dst), "v"(voff), "s"(rsrc) : "memory", "m0");
}
#pragma clang diagnostic pop

// The next tile a wave loads: where its rows start, and how many tokens are
// left from it to the unit's end.  Advanced by one tile per issue, so that a
// tile's descriptors take a 64-bit add and 32-bit clamps (no 64-bit index
// arithmetic or compares per tile).
struct StCursor {
    uint64_t b, x, d;   // byte addresses of the tile's first row of B, x, dt
    int rows;           // tokens from the tile to the unit's end (<= 0: past it)
};

// tile_words on a byte address and a 32-bit row count.
// (the clamp is written out as scalar min and max: as C, the compiler folds
// it into a vector median, and the products after it then run on the vector
// unit too.  Both instructions write SCC, which the statement declares.)
__device__ __forceinline__ u32x4 tile_words32(uint64_t p, int rows, unsigned pitch, unsigned row_bytes)
{
    int r;
    asm("s_max_i32 %0, %1, 0\n\ts_min_i32 %0, %0, %2" : "=&s"(r) : "s"(rows), "n"(kT) : "scc");
    const int bytes = r * (int)pitch - (int)pitch + (int)row_bytes;
    u32x4 d;
    d.x = __builtin_amdgcn_readfirstlane((unsigned)p);
    d.y = __builtin_amdgcn_readfirstlane((unsigned)(p >> 32)) & 0xffffu;
    d.z = __builtin_amdgcn_readfirstlane((unsigned)(bytes < 0 ? 0 : bytes));
    d.w = 0x00020000u;
    return d;
}

// Loads of the cursor's tile into one ring slot, bounded by the unit's end (a
// tile past it reads as zeros): kStLoads instructions per wave; then the
// cursor moves to the next tile.  Lane l of a 1 KB block writes bytes
// 16 l .. 16 l + 15 of it, so the swizzle of the B and x tiles is applied to
// the source offsets.
__device__ __forceinline__ void st_issue(const StIo &io, StCursor &cur, unsigned Bslot, unsigned Xslot,
                                         unsigned Dslot, int w)
{
    const u32x4 rb = tile_words32(cur.b, cur.rows, (unsigned)io.bp, kN * 2);
#pragma unroll
    for (int k = 0; k < kStBBlocks; ++k)
        lds_load16(Bslot + 1024 * (kStBBlocks * w + k), rb, io.boff[k]);
    const u32x4 rx = tile_words32(cur.x, cur.rows, (unsigned)io.xp, kP * 2);
#pragma unroll
    for (int k = 0; k < kStXBlocks; ++k)
        lds_load16(Xslot + 1024 * (kStXBlocks * (w & 1) + k), rx, io.xoff[k]);
    const u32x4 rd = tile_words32(cur.d, cur.rows, (unsigned)io.dp, io.dbytes);
    if ((threadIdx.x & 63) < 32)
        lds_load4(Dslot + 128 * w, rd, io.doff);
    cur.b += (uint64_t)kT * (uint64_t)io.bp;
    cur.x += (uint64_t)kT * (uint64_t)io.xp;
    cur.d += (uint64_t)kT * (uint64_t)io.dp;
    cur.rows -= kT;
}

// The LDS location at byte address a, as a pointer.
__device__ __forceinline__ const unsigned char *lds_ptr(unsigned a)
{
    return (const unsigned char *)(const __attribute__((address_space(3))) unsigned char *)(uintptr_t)a;
}

// s_waitcnt vmcnt(n), other counters untouched (gfx9 encoding)
template <int n> __device__ __forceinline__ void wait_vmcnt()
{
    static_assert(n >= 0 && n < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (0x7 << 4) | (0xf << 8));
}

template <bool kSp>
__device__ __forceinline__ void seg_state_body(const SegArgs &a, int64_t bid, int64_t nblk)
{
    __shared__ __align__(16) unsigned char sB0[kT * kBRow], sB1[kT * kBRow], sB2[kT * kBRow];
    __shared__ __align__(16) unsigned char sX0[kStHeads][kT * kXRow], sX1[kStHeads][kT * kXRow],
        sX2[kStHeads][kT * kXRow];
    __shared__ __align__(16) unsigned char sD0[kT * kStHeads * 4], sD1[kT * kStHeads * 4], sD2[kT * kStHeads * 4];
    __shared__ __align__(16) float swd[kStWaves][kT];

    const int tid = threadIdx.x, w = wave_id(), l = tid & 63, g = l >> 4, c = l & 15;
    const int hs = w >> 1, ph = w & 1;
    // Work-groups in dispatch order, without the XCD remap of the scan kernel:
    // the head quads of one token range then run on different XCDs, which
    // streams x faster (B, shared by the quads, is small and comes from the
    // memory-side cache).
    const int64_t j = bid;
    const int nquad = a.G * a.nq;
    const int quad = (int)(j % nquad);
    const int64_t r = j / nquad;
    const int unit = (int)(r % a.nseg_launch);
    const int64_t b = r / a.nseg_launch;
    const int grp = quad / a.nq;
    const int hw = (quad % a.nq) * kStHeads + hs;
    const bool active = hw < a.hg;                        // idle slots mirror the last head
    const int h = grp * a.hg + (active ? hw : a.hg - 1);
    const int64_t bh = b * a.H + h;
    const int64_t L = a.L;
    const int64_t sbeg = (int64_t)(unit / a.nsub) * a.seg_tokens;
    const int64_t tseg0 = sbeg + (int64_t)(unit % a.nsub) * a.unit_tokens;
    const int64_t tseg1 = std::min<int64_t>(std::min<int64_t>(L, sbeg + a.seg_tokens), tseg0 + a.unit_tokens);
    const float Ah2 = a.A[h] * kLog2e;
    const float dtb = kSp && a.dt_bias ? a.dt_bias[h] : 0.f;
    const int zoff = (32 * ph + c) * kN + 4 * g;          // + 16 q kN + 16 nb

    if (unit == 0 && a.seg0_from_ws && active) {
        // alias of final and initial state: keep a copy of the initial state
        const float *ini = a.init + bh * kP * kN;
        float *cp = a.ws_state + (bh * a.nslot + (a.nslot - 1)) * kP * kN;
#pragma unroll
        for (int nb = 0; nb < 8; ++nb)
#pragma unroll
            for (int q = 0; q < 2; ++q)
                *reinterpret_cast<f32x4 *>(cp + zoff + 16 * q * kN + 16 * nb) =
                    *reinterpret_cast<const f32x4 *>(ini + zoff + 16 * q * kN + 16 * nb);
    }

    StIo io;
    io.bp = (int64_t)a.G * kN * 2;
    io.xp = (int64_t)a.H * kP * 2;
    io.dp = (int64_t)a.H * 4;
    io.B = a.B + (b * L * a.G + grp) * kN;
    io.x = a.x + (b * L * a.H + h) * kP;
    const int hq = (quad % a.nq) * kStHeads;               // the quad's first head in the group
    io.dt = a.dt + b * L * a.H + grp * a.hg + hq;
    io.dbytes = 4u * (unsigned)std::min(kStHeads, a.hg - hq);
#pragma unroll
    for (int k = 0; k < kStBBlocks; ++k) {
        const int row = 4 * (kStBBlocks * w + k) + (l >> 4), pc = l & 15;
        io.boff[k] = (unsigned)row * (unsigned)io.bp + (unsigned)((pc ^ bswz(row)) << 4);
    }
#pragma unroll
    for (int k = 0; k < kStXBlocks; ++k) {
        const int row = 8 * (kStXBlocks * ph + k) + (l >> 3), pc = l & 7;
        io.xoff[k] = (unsigned)row * (unsigned)io.xp + (unsigned)((pc ^ xswz(row)) << 4);
    }
    // lanes 0..31 of wave w: token 8 w + l / 4, head l % 4 of the quad
    io.doff = (unsigned)(8 * w + (l >> 2)) * (unsigned)io.dp + 4u * (unsigned)(l & 3);

    // Zero the ring once: rows past a unit's end then hold zeros or an older
    // tile's finite values, which its zero weights cancel.
    {
        uint4 *z0 = reinterpret_cast<uint4 *>(sB0), *z1 = reinterpret_cast<uint4 *>(sB1),
              *z2 = reinterpret_cast<uint4 *>(sB2);
        for (int i = tid; i < kT * kBRow / 16; i += kStThreads)
            z0[i] = z1[i] = z2[i] = make_uint4(0, 0, 0, 0);
        uint4 *x0 = reinterpret_cast<uint4 *>(&sX0[0][0]), *x1 = reinterpret_cast<uint4 *>(&sX1[0][0]),
              *x2 = reinterpret_cast<uint4 *>(&sX2[0][0]);
        for (int i = tid; i < kStHeads * kT * kXRow / 16; i += kStThreads)
            x0[i] = x1[i] = x2[i] = make_uint4(0, 0, 0, 0);
    }
    lds_barrier();

    f32x4 Z[8][2];
    const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int nb = 0; nb < 8; ++nb)
#pragma unroll
        for (int q = 0; q < 2; ++q)
            Z[nb][q] = zero4;
    float ls = 0.f, lsum = 0.f;
    // LDS byte addresses of the slots (scalars; the loads take them in M0)
#define SSD_LDS(p) __builtin_amdgcn_readfirstlane( \
    (unsigned)reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) unsigned char *)(p)))
    const unsigned aB0 = SSD_LDS(sB0), aB1 = SSD_LDS(sB1), aB2 = SSD_LDS(sB2);
    const unsigned aX0 = SSD_LDS(&sX0[hs][0]), aX1 = SSD_LDS(&sX1[hs][0]), aX2 = SSD_LDS(&sX2[hs][0]);
    const unsigned aD0 = SSD_LDS(sD0), aD1 = SSD_LDS(sD1), aD2 = SSD_LDS(sD2);
#undef SSD_LDS
    StCursor cur;
    cur.b = reinterpret_cast<uint64_t>(io.B + tseg0 * (io.bp / 2));
    cur.x = reinterpret_cast<uint64_t>(io.x + tseg0 * (io.xp / 2));
    cur.d = reinterpret_cast<uint64_t>(io.dt + tseg0 * (io.dp / 4));
    cur.rows = (int)std::min<int64_t>(tseg1 - tseg0, int64_t(1) << 30);
    st_issue(io, cur, aB0, aX0, aD0, w);
    st_issue(io, cur, aB1, aX1, aD1, w);

    // tile t0 in slot (Bs, Xs, Ds); tile t0 + 2 kT goes to (Bn, Xn, Dn)
    auto step = [&](unsigned aB, unsigned aX, unsigned aD, unsigned Bn, unsigned Xn, unsigned Dn,
                    int64_t t0) {
        wait_vmcnt<kStLoads>();                   // this wave's loads of tile t0 are in
        lds_barrier();                            // ... and every wave's; slot of t0 - kT free
        st_issue(io, cur, Bn, Xn, Dn, w);      // tile t0 + 2 kT
        const unsigned char *Bs = lds_ptr(aB), *Xs = lds_ptr(aX), *Ds = lds_ptr(aD);
        float dtc = reinterpret_cast<const float *>(Ds)[kStHeads * l + hs];
        // the update's operands, read while the decay scan below runs
        bf16x8 XT[2][2], BT[8][2];
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
            for (int jj = 0; jj < 2; ++jj)
                XT[q][jj] = tr_operand_x(Xs, jj, 32 * ph + 16 * q, g, c);
#pragma unroll
        for (int nb = 0; nb < 8; ++nb) {
            BT[nb][0] = tr_operand_b(Bs, 0, 16 * nb, g, c);
            BT[nb][1] = tr_operand_b(Bs, 1, 16 * nb, g, c);
        }
        if constexpr (kSp) {
            // the step size from u, tokens past the end keep 0: formed in
            // every lane and then selected (as a conditional it became a
            // divergent branch ahead of the decay scan; 3 us slower)
            float sp = softplus_dt(dtc, dtb);
            asm volatile("" : "+v"(sp));
            dtc = l < tseg1 - t0 ? sp : 0.f;
        }
        const float lam = wave_inclusive_sum(dtc * Ah2, l);
        // (a scalar: readlane needs a uniform lane)
        const int last = __builtin_amdgcn_readfirstlane(
            (int)std::min<int64_t>(std::max<int64_t>(tseg1 - t0, 1), kT) - 1);
        float bias;
        const TileMode md = tile_mode(lane_f(lam, last), ls, lsum, bias);
        swd[w][l] = fast_exp2(bias - lam) * dtc;
        bf16x8 XS[2][2];
        scale_x(XS, XT, swd[w], g);
        if (uniform(md.renorm)) {
#pragma unroll
            for (int nb = 0; nb < 8; ++nb)
#pragma unroll
                for (int q = 0; q < 2; ++q)
                    Z[nb][q] *= md.rscale;
        }
        state_update_pre(Z, BT, XS, md);
    };
    // the ring's slots: c = tile t0, m = tile t0 + kT (in flight), f = free
    unsigned cB = aB0, cX = aX0, cD = aD0, mB = aB1, mX = aX1, mD = aD1, fB = aB2, fX = aX2, fD = aD2;
    for (int64_t t0 = tseg0; t0 < tseg1; t0 += kT) {
        step(cB, cX, cD, fB, fX, fD, t0);
        const unsigned oB = cB, oX = cX, oD = cD;
        cB = mB, cX = mX, cD = mD;
        mB = fB, mX = fX, mD = fD;
        fB = oB, fX = oX, fD = oD;
    }
    wait_vmcnt<0>();   // the loads past the end land before the work-group's LDS is released

    if (!active)
        return;
    float *dst = a.ws_state + (bh * a.nslot + unit) * kP * kN;
    if (tid == 128 * hs)
        a.ws_decay[bh * a.nslot + unit] = fast_exp2(lsum);
    const float sc = fast_exp2(ls);
#pragma unroll
    for (int nb = 0; nb < 8; ++nb)
#pragma unroll
        for (int q = 0; q < 2; ++q)
            *reinterpret_cast<f32x4 *>(dst + zoff + 16 * q * kN + 16 * nb) = Z[nb][q] * sc;
}

// State kernel: the end state of every unit of segments 0 .. nseg-2, and its decay.
template <bool kSp>
__global__ __launch_bounds__(kStThreads, 1) void seg_state_kernel(SegArgs a)
{
    seg_state_body<kSp>(a, blockIdx.x, gridDim.x);
}

// Scan kernel: y of every segment from its entering state, and the final state.
// kSp: the dt input holds u and the step size is softplus(u + dt_bias[h]).
template <bool kSp>
__global__ __launch_bounds__(Geom<kScanHeads>::kThreads, 1) void chunk_scan_kernel(SegArgs a)
{
    __shared__ ScanSmem<kScanHeads> sm;
    scan_body<kScanHeads, kSp>(a, sm, blockIdx.x, gridDim.x);
}

// Several independent problems (the runs of equal length of a packed batch)
// in one launch: run r owns work-groups wg0[r] .. wg0[r] + nwg[r] - 1, its
// start a multiple of 8 so that the work-group -> XCD mapping inside a run is
// the same as in a launch of its own; the padding work-groups return.
struct MultiArgs {
    SegArgs run[kMaxRuns];
    int wg0[kMaxRuns + 1];
    int nwg[kMaxRuns];
    int nruns;
};

__device__ __forceinline__ int multi_run(const MultiArgs &m, int bid)
{
    int r = 0;
#pragma unroll
    for (int k = 1; k < kMaxRuns; ++k)
        r += (k < m.nruns && bid >= m.wg0[k]) ? 1 : 0;
    return r;
}

template <bool kSp>
__global__ __launch_bounds__(kStThreads, 1) void seg_state_multi_kernel(MultiArgs m)
{
    const int r = multi_run(m, blockIdx.x);
    const int local = (int)blockIdx.x - m.wg0[r];
    if (local >= m.nwg[r])
        return;
    seg_state_body<kSp>(m.run[r], local, m.nwg[r]);
}

template <bool kSp>
__global__ __launch_bounds__(Geom<kScanHeads>::kThreads, 1) void chunk_scan_multi_kernel(MultiArgs m)
{
    __shared__ ScanSmem<kScanHeads> sm;
    const int r = multi_run(m, blockIdx.x);
    const int local = (int)blockIdx.x - m.wg0[r];
    if (local >= m.nwg[r])
        return;
    scan_body<kScanHeads, kSp>(m.run[r], sm, local, m.nwg[r]);
}

int64_t env_int(const char *name, int64_t dflt)
{
    const char *v = std::getenv(name);
    if (!v || !*v)
        return dflt;
    const long long x = std::atoll(v);
    return x > 0 ? (int64_t)x : dflt;
}

constexpr int64_t kCUs = 256;

}  // namespace

static size_t align256(size_t n)
{
    return (n + 255) / 256 * 256;
}

Bf16Plan plan_scan_bf16(int64_t B, int64_t L, int64_t H, int64_t G, int64_t Q, int64_t cus,
                        int64_t nseg_fixed, bool use_env)
{
    const int64_t kCUs = std::max<int64_t>(1, cus);
    Bf16Plan p{};
    p.nchunks = (L + Q - 1) / Q;
    const int64_t hg = G > 0 ? H / G : 1;
    p.quads = std::max<int64_t>(1, G * ((hg + kScanHeads - 1) / kScanHeads));
    const int64_t per_seg = std::max<int64_t>(1, B * p.quads);     // scan work-groups per segment
    // state work-groups per segment, and how many fit on the chip at once (LDS)
    const int64_t per_seg1 = std::max<int64_t>(1, B * G * ((hg + kStHeads - 1) / kStHeads));
    const int64_t slots1 = kCUs * (int64_t)(160 * 1024 / kStSmemBytes);
    // Segments per sequence, in whole 64-token tiles (the kernels' step; the
    // result does not depend on where the segments end).  The scan kernel runs
    // one work-group per CU, so its time is ~ rounds * tiles per segment; the
    // state kernel (about half the work per tile) re-reads x for all but the
    // last segment, and every segment adds one unit state, which the last
    // segment's work-groups chain before their first tile (~2.75 us, 0.6 of a
    // tile at the 2.7B layer) and which passes through the workspace: about a
    // tile's worth.  When the scan fits one round of work-groups, only such
    // plans are taken: a second round measured slower than this cost says
    // (131072 tokens, 80 heads in 8 groups: 21 segments 1.39 ms, 10 segments
    // 1.33 ms), while within one round more segments paid (the 130M-shaped
    // layer: 5 segments 63.3 us, 4 segments 70.0 us).
    const int64_t tiles = std::max<int64_t>(1, (L + kT - 1) / kT);
    int64_t nseg = use_env ? env_int("SSD_NSEG", 0) : 0;
    if (nseg <= 0)
        nseg = nseg_fixed;
    if (nseg <= 0) {
        const bool one_round = per_seg <= kCUs;
        double best = 1e300;
        for (int64_t k = 1; k <= tiles; ++k) {
            const int64_t tps = (tiles + k - 1) / k;
            const int64_t ns = (tiles + tps - 1) / tps;
            if (ns != k || (one_round && per_seg * ns > kCUs))
                continue;
            const double r3 = (double)((per_seg * ns + kCUs - 1) / kCUs);
            const double r1 = (double)((per_seg1 * (ns - 1) + slots1 - 1) / slots1);
            const double cost = (r3 + 0.5 * r1) * (double)tps + 1.0 * (double)ns;
            if (cost < best) {
                best = cost;
                nseg = ns;
            }
        }
    }
    nseg = std::max<int64_t>(1, std::min<int64_t>(nseg, tiles));
    const int64_t seg_tiles = (tiles + nseg - 1) / nseg;
    p.seg_tokens = seg_tiles * kT;
    p.nseg = (tiles + seg_tiles - 1) / seg_tiles;
    p.chunks_per_seg = (p.seg_tokens + Q - 1) / Q;
    // The state kernel may cut each of its segments into units to fill the
    // chip; every unit adds one more state to write, and the scan kernel's
    // last segment chains (nseg-1) * nsub states before its first tile.  Cost
    // in microseconds, from times measured at the 2.7B layer for 1 to 4 units
    // per segment: the state kernel runs in rounds of `slots1` work-groups; a
    // tile costs a work-group ~1.9 us when few run, and their HBM traffic
    // (~49 KB per tile and work-group) caps a round at ~5 TB/s; each chained
    // unit state adds ~2.75 us to the scan kernel's prologue.
    p.nsub = 1;
    p.unit_tokens = p.seg_tokens;
    if (p.nseg > 1) {
        constexpr double kTileUs = 1.9, kChainUs = 2.75, kHbmBytesPerUs = 5.0e6;
        constexpr double kTileBytes = (double)kT * (kStHeads * kP * 2 + kN * 2 + kStHeads * 4);
        int64_t want = use_env ? env_int("SSD_NSUB", 0) : 0;
        double best = 1e300;
        for (int64_t k = 1; k <= 8; ++k) {
            const int64_t ut = (seg_tiles + k - 1) / k;             // tiles per unit
            const int64_t nk = (seg_tiles + ut - 1) / ut;           // non-empty units
            if (nk != k)
                continue;
            const int64_t wgs = per_seg1 * (p.nseg - 1) * nk;
            const double rounds = (double)((wgs + slots1 - 1) / slots1);
            const double active = (double)std::min(wgs, slots1);
            const double tile_us = std::max(kTileUs, active * kTileBytes / kHbmBytesPerUs);
            const double cost = rounds * (double)ut * tile_us + kChainUs * (double)((p.nseg - 1) * nk);
            if (want > 0 ? k == want : cost < best) {
                best = cost;
                p.nsub = nk;
                p.unit_tokens = ut * kT;
            }
        }
    }
    p.nslot = p.nseg > 1 ? (p.nseg - 1) * p.nsub + 1 : 0;
    p.state_bytes = (size_t)(B * H * p.nslot) * kP * kN * sizeof(float);
    p.decay_bytes = (size_t)(B * H * p.nslot) * sizeof(float);
    p.ws_bytes = align256(p.state_bytes) + align256(p.decay_bytes);
    return p;
}

namespace {

// The kernel arguments of one problem; nq and nseg_launch are set per kernel.
SegArgs seg_args(const Bf16Plan &plan, int64_t B, int64_t L, int64_t H, int64_t G, int64_t Q,
                 const void *x, const float *dt, const float *A, const void *Bm, const void *Cm,
                 const float *D, const float *init, void *y, float *fin, void *ws, DtPrep prep)
{
    (void)B;
    SegArgs a{};
    a.x = static_cast<const __bf16 *>(x);
    a.dt = dt;
    a.dt_bias = prep.bias;
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
    a.hg = (int)(H / G);
    a.seg_tokens = plan.seg_tokens;
    a.unit_tokens = plan.unit_tokens;
    a.nseg = (int)plan.nseg;
    a.nsub = (int)plan.nsub;
    a.nslot = (int)plan.nslot;
    const bool alias = init != nullptr && init == fin;
    a.seg0_from_ws = (alias && plan.nseg > 1) ? 1 : 0;
    char *wsb = static_cast<char *>(ws);
    a.ws_state = reinterpret_cast<float *>(wsb);
    a.ws_decay = reinterpret_cast<float *>(wsb + align256(plan.state_bytes));
    return a;
}

int state_quads(const SegArgs &a)
{
    return (a.hg + kStHeads - 1) / kStHeads;
}

int scan_quads(const SegArgs &a)
{
    return (a.hg + kScanHeads - 1) / kScanHeads;
}

}  // namespace

hipError_t launch_scan_bf16(const Bf16Plan &plan, int64_t B, int64_t L, int64_t H, int64_t G,
                            int64_t Q, const void *x, const float *dt, const float *A,
                            const void *Bm, const void *Cm, const float *D, const float *init,
                            void *y, float *fin, void *ws, DtPrep prep, hipStream_t s,
                            EventLog *log)
{
    if (B * H == 0 || L == 0)
        return hipSuccess;
    SegArgs a = seg_args(plan, B, L, H, G, Q, x, dt, A, Bm, Cm, D, init, y, fin, ws, prep);
    const int nq3 = scan_quads(a);
    const int nq1 = state_quads(a);
    hipError_t e = log_begin(log, s);
    if (e != hipSuccess)
        return e;
    if (plan.nseg > 1) {
        a.nq = nq1;
        a.nseg_launch = (a.nseg - 1) * a.nsub;
        const unsigned grid = (unsigned)(B * G * nq1 * a.nseg_launch);
        if (prep.softplus)
            seg_state_kernel<true><<<grid, kStThreads, 0, s>>>(a);
        else
            seg_state_kernel<false><<<grid, kStThreads, 0, s>>>(a);
        if ((e = hipGetLastError()) != hipSuccess || (e = log_kernel(log, "seg_state_kernel", s)) != hipSuccess)
            return e;
    }
    a.nq = nq3;
    a.nseg_launch = a.nseg;
    const unsigned grid = (unsigned)(B * G * nq3 * plan.nseg);
    if (prep.softplus)
        chunk_scan_kernel<true><<<grid, Geom<kScanHeads>::kThreads, 0, s>>>(a);
    else
        chunk_scan_kernel<false><<<grid, Geom<kScanHeads>::kThreads, 0, s>>>(a);
    if ((e = hipGetLastError()) != hipSuccess)
        return e;
    return log_kernel(log, "chunk_scan_kernel", s);
}

hipError_t launch_scan_bf16_multi(const Bf16Run *runs, int nruns, int64_t H, int64_t G, int64_t Q,
                                  const float *A, const float *D, DtPrep prep, hipStream_t s)
{
    if (nruns < 1 || nruns > kMaxRuns)
        return hipErrorInvalidValue;
    MultiArgs m1{}, m3{};   // state kernel, scan kernel
    int wg1 = 0, wg3 = 0;
    for (int r = 0; r < nruns; ++r) {
        const Bf16Run &u = runs[r];
        SegArgs a = seg_args(u.plan, u.B, u.L, H, G, Q, u.x, u.dt, A, u.Bm, u.Cm, D, u.init, u.y,
                             u.fin, u.ws, prep);
        SegArgs a1 = a, a3 = a;
        a1.nq = state_quads(a);
        a1.nseg_launch = (a.nseg - 1) * a.nsub;
        a3.nq = scan_quads(a);
        a3.nseg_launch = a.nseg;
        const int64_t n1 = u.plan.nseg > 1 ? u.B * G * a1.nq * a1.nseg_launch : 0;
        const int64_t n3 = u.B * G * a3.nq * a3.nseg_launch;
        if (wg1 + n1 + 8 > INT32_MAX / 2 || wg3 + n3 + 8 > INT32_MAX / 2)
            return hipErrorInvalidValue;
        m1.run[r] = a1;
        m1.wg0[r] = wg1;
        m1.nwg[r] = (int)n1;
        wg1 += (int)((n1 + 7) / 8 * 8);
        m3.run[r] = a3;
        m3.wg0[r] = wg3;
        m3.nwg[r] = (int)n3;
        wg3 += (int)((n3 + 7) / 8 * 8);
    }
    m1.nruns = m3.nruns = nruns;
    for (int r = nruns; r <= kMaxRuns; ++r) {
        if (r < kMaxRuns) {
            m1.nwg[r] = m3.nwg[r] = 0;
        }
        m1.wg0[r] = wg1;
        m3.wg0[r] = wg3;
    }
    hipError_t e;
    if (wg1 > 0) {
        if (prep.softplus)
            seg_state_multi_kernel<true><<<(unsigned)wg1, kStThreads, 0, s>>>(m1);
        else
            seg_state_multi_kernel<false><<<(unsigned)wg1, kStThreads, 0, s>>>(m1);
        if ((e = hipGetLastError()) != hipSuccess)
            return e;
    }
    if (prep.softplus)
        chunk_scan_multi_kernel<true><<<(unsigned)wg3, Geom<kScanHeads>::kThreads, 0, s>>>(m3);
    else
        chunk_scan_multi_kernel<false><<<(unsigned)wg3, Geom<kScanHeads>::kThreads, 0, s>>>(m3);
    return hipGetLastError();
}

}  // namespace ssd
