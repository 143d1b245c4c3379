/*
 * ssd.h -- C ABI of libssd: the Mamba-2 state-space-duality (SSD) layer on one
 * AMD Instinct MI355X (gfx950): chunked prefill scan (also over packed batches
 * of different lengths), O(1) cached decode (one step, or many known steps in
 * one launch with the state on-chip), an optional fused step-size prep, and
 * the Gated DeltaNet decode step of the FPGA decode page (ssd_gdn_*).
 *
 * The operation.  "Compiler-First State Space Duality and Portable O(1)
 * Autoregressive Caching for Inference" (section 2, methodology) describes
 * the SSD layer as a per-head diagonal state recurrence that is cut into
 * fixed-size chunks and evaluated with einsum-style contractions and static
 * causal (lower-triangular) masks, the decay being exponentiated in float32,
 * and a fixed-size per-sequence state cache that decoding updates in place
 * on the device (sections 2 and 3).  The page never writes the recurrence;
 * this library computes the Mamba-2 SSD layer with a scalar-times-identity
 * state matrix per head.  For batch row b, head h, group g = h / (H / G):
 *
 *     alpha_t = exp(dt[b,t,h] * A[h])
 *     H_t     = alpha_t * H_{t-1} + dt[b,t,h] * x[b,t,h,:] (outer) B[b,t,g,:]
 *     y[b,t,h,:] = H_t . C[b,t,g,:] + D[h] * x[b,t,h,:]
 *
 * H_t is the P x N state (headdim x dstate).  ssd_chunk_scan evaluates this
 * for t = 1..L with the chunked (state-space-duality) algorithm: inside each
 * chunk of Q tokens a causal quadratic form, across chunks a state passed from
 * chunk to chunk.  ssd_decode_step is exactly one more step t on the cached
 * state, ssd_decode_steps S of them.  dt is taken as given (already
 * softplus-ed, positive) unless ssd_dims.flags has SSD_DT_SOFTPLUS; A should
 * be <= 0 (A > 0 is not rejected, but exp(dt*A) may overflow and is
 * unsupported).
 *
 * Conventions shared by every call:
 *   - Every tensor pointer is a DEVICE pointer to contiguous row-major memory
 *     owned by the caller; the library allocates no device memory and keeps
 *     no pointer after a call returns.
 *   - stream is a hipStream_t passed as void* (NULL = the default stream).
 *     Calls enqueue work asynchronously and return without synchronising.
 *   - Arguments are validated before any device call; on an error nothing is
 *     launched and a status code is returned.  No call aborts or throws.
 *   - Alignment: x, B, C, y and the state / workspace buffers must be 16-byte
 *     aligned (x and y of ssd_decode_step(s): element-aligned); dt, A, D
 *     4-byte.  Otherwise SSD_ERR_ALIGNMENT.
 *   - Float inputs must be finite.  Outputs for non-finite inputs are undefined.
 *   - State kept between calls: each host thread caches its last eight
 *     variable-length launch plans (a pure function of the sizes, so results
 *     never depend on it), and ssd_chunk_scan_noalloc keeps one scratch
 *     array per device.  Apart from ssd_chunk_scan_noalloc (see there), calls
 *     on different streams may run concurrently if their buffers do not
 *     overlap.
 *   - Environment: SSD_NSEG and SSD_NSUB, when set to positive integers,
 *     override the bf16 scan's segment and unit counts (a test hook: the
 *     result changes only by rounding, the workspace size with the plan).
 *   - Shapes (x, y : [B, L, H, P] of io_dtype; dt : [B, L, H] fp32;
 *     A, D : [H] fp32; B, C : [B, L, G, N] of io_dtype;
 *     state : [B, H, P, N] fp32, n fastest).
 */
#ifndef SSD_H
#define SSD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum ssd_status {
    SSD_OK = 0,
    SSD_ERR_NULL = 1,        /* a required pointer is NULL                        */
    SSD_ERR_SHAPE = 2,       /* a size is out of range, or nheads % ngroups != 0  */
    SSD_ERR_UNSUPPORTED = 3, /* valid, but not an implemented (P, N, Q, dtype)    */
    SSD_ERR_ALIAS = 4,       /* an output overlaps a buffer it must not overlap   */
    SSD_ERR_WORKSPACE = 5,   /* workspace NULL or smaller than required           */
    SSD_ERR_DEVICE = 6,      /* a HIP runtime call or kernel launch failed        */
    SSD_ERR_ALIGNMENT = 7    /* a pointer is not aligned as required              */
} ssd_status;

typedef enum ssd_dtype {
    SSD_F32 = 0,             /* x, B, C, y in float32                             */
    SSD_BF16 = 1             /* x, B, C, y in bfloat16                            */
} ssd_dtype;

/* flags of ssd_dims: fused step-size prep.  With SSD_DT_SOFTPLUS the dt
 * argument of every call holds u instead of the step size, and the step size
 * of head h is softplus(u + dt_bias[h]) = log(1 + exp(u + dt_bias[h])),
 * evaluated in fp32 inside the kernels (the workloads draw dt through a
 * softplus; fusing it saves a pass over dt).  Positions past the end of a
 * sequence still contribute nothing. */
#define SSD_DT_SOFTPLUS 1

/* Problem sizes.  seqlen and chunk are ignored by ssd_decode_step(s) and
 * ssd_state_init. */
typedef struct ssd_dims {
    int64_t batch;     /* B >= 0                                              */
    int64_t seqlen;    /* L >= 0 tokens per sequence                          */
    int64_t nheads;    /* H >= 1                                              */
    int64_t headdim;   /* P >= 1                                              */
    int64_t dstate;    /* N >= 1                                              */
    int64_t ngroups;   /* G >= 1, H % G == 0; head h reads B/C group h/(H/G)  */
    int64_t chunk;     /* Q >= 1, chunk length of the chunked scan            */
    int32_t io_dtype;  /* ssd_dtype of x, B, C, y                             */
    int32_t flags;     /* 0 or SSD_DT_SOFTPLUS; other bits: SSD_ERR_SHAPE     */
    const float *dt_bias; /* [H] fp32 device pointer or NULL (bias 0); read
                             only with SSD_DT_SOFTPLUS; 4-byte aligned, must
                             not overlap an output                          */
} ssd_dims;

/* Human-readable name of a status code (static storage; never NULL). */
const char *ssd_status_string(ssd_status status);

/* Library version, major * 10000 + minor * 100 + patch. */
int ssd_version(void);

/*
 * ssd_state_init -- set the cached state of every (batch row, head).
 *   state : [B, H, P, N] fp32, written.
 *   src   : [B, H, P, N] fp32 to copy from, or NULL for the zero state
 *           (the empty cache: H_0 = 0).  src == state is a no-op; any other
 *           overlap of src and state returns SSD_ERR_ALIAS.
 * Implemented with a fill/copy kernel (no hipMemsetAsync), so it may be
 * captured in a HIP graph.  Section 2 of the page: the cache lives on the
 * device and is initialised there.
 */
ssd_status ssd_state_init(const ssd_dims *dims, float *state, const float *src, void *stream);

/*
 * ssd_chunk_scan_workspace_size -- bytes of device workspace ssd_chunk_scan
 * needs for these sizes (0 is possible).  *bytes is written on SSD_OK.  The
 * result depends on dims only (and on the environment variables SSD_NSEG /
 * SSD_NSUB, which override the planner's segment and unit counts when set
 * to a positive integer; the tests use them).
 */
ssd_status ssd_chunk_scan_workspace_size(const ssd_dims *dims, size_t *bytes);

/*
 * ssd_chunk_scan -- prefill: run the recurrence over L tokens of every
 * sequence with the chunked algorithm of chunk length Q (section 2 of the
 * page: chunked recurrence, static causal masks, float32 decay exponentials).
 *   x [B,L,H,P], dt [B,L,H], A [H], B [B,L,G,N], C [B,L,G,N], D [H]   inputs
 *   initial_state [B,H,P,N] fp32, or NULL for the zero state            input
 *   y [B,L,H,P] (io_dtype)                                               output
 *   final_state [B,H,P,N] fp32 = H_L                                     output
 *   workspace : device buffer of >= ssd_chunk_scan_workspace_size bytes,
 *               16-byte aligned; contents on entry are ignored.
 * final_state may be the same pointer as initial_state (resume a cache in
 * place); y must not overlap any input, the state buffers or the workspace.
 * L need not be a multiple of Q (the last chunk is then shorter); L == 0
 * writes final_state = initial_state (or zeros); B == 0 does nothing.
 * Supported: io_dtype SSD_BF16 with (P, N) = (64, 128) and Q a multiple of
 * 64 up to 512 (bf16 MFMA path, fp32 accumulation); io_dtype SSD_F32 with
 * P <= 64, N <= 128, Q <= 256 (fp32 path).  Others: SSD_ERR_UNSUPPORTED.
 */
ssd_status ssd_chunk_scan(const ssd_dims *dims, const void *x, const float *dt, const float *A,
                          const void *B, const void *C, const float *D,
                          const float *initial_state, void *y, float *final_state,
                          void *workspace, size_t workspace_bytes, void *stream);

/*
 * ssd_chunk_scan_noalloc -- ssd_chunk_scan without a workspace argument, for
 * callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc.  It allocates nothing
 * (no hipMalloc, no hipFree, no allocating library call); the workspace is a
 * scratch array inside the library, SSD_NOALLOC_SCRATCH_BYTES per device,
 * which each device the library runs on holds from its first call there until
 * the process ends.  The caller still passes every input and output.
 *   Arguments, shapes, results and errors as for ssd_chunk_scan (the same
 *   plan and kernels: the results are identical to ssd_chunk_scan's).
 *   SSD_ERR_WORKSPACE, before any device call, when the workspace that
 *   ssd_chunk_scan_workspace_size reports for dims exceeds
 *   SSD_NOALLOC_SCRATCH_BYTES (use ssd_chunk_scan with a caller workspace).
 * Every call on one device shares that device's scratch array, which keeps the
 * last call's contents (nothing in it needs to start at zero): calls that can
 * overlap in time on one device (other streams, other threads) race on it and
 * must be ordered by the caller.  The stream must belong to the current device.
 */
#define SSD_NOALLOC_SCRATCH_BYTES ((size_t)96 << 20)
ssd_status ssd_chunk_scan_noalloc(const ssd_dims *dims, const void *x, const float *dt,
                                  const float *A, const void *B, const void *C, const float *D,
                                  const float *initial_state, void *y, float *final_state,
                                  void *stream);

/*
 * ssd_chunk_scan_varlen -- prefill of a packed batch of sequences of
 * different lengths, each its own recurrence with its own cache (section 2 of
 * the page, per sequence, as ssd_chunk_scan).  dims->batch = number of sequences S, dims->seqlen = total
 * tokens T; cu_seqlens is a HOST array of S + 1 offsets (cu[0] = 0,
 * non-decreasing, cu[S] = T): sequence i is tokens cu[i] .. cu[i+1]-1.
 *   x [T,H,P], dt [T,H], B [T,G,N], C [T,G,N]    packed inputs (io_dtype / fp32)
 *   A [H], D [H]                                  as for ssd_chunk_scan
 *   initial_states [S,H,P,N] fp32 or NULL         input
 *   y [T,H,P]                                     output
 *   final_states [S,H,P,N] fp32                   output (may alias initial_states)
 *   workspace : >= ssd_chunk_scan_varlen_workspace_size bytes
 * Zero-length sequences pass their state through.  Consecutive sequences of
 * equal length form one run, laid out like a batched scan; with bf16 I/O up
 * to eight runs share one launch of each scan kernel (the workspace holds a
 * region per run), with fp32 I/O each run is one scan call.  Every run is
 * validated before anything is enqueued.  Supported shapes and the alignment
 * of each sequence's slices as for ssd_chunk_scan.
 */
ssd_status ssd_chunk_scan_varlen_workspace_size(const ssd_dims *dims, const int64_t *cu_seqlens,
                                                size_t *bytes);
ssd_status ssd_chunk_scan_varlen(const ssd_dims *dims, const int64_t *cu_seqlens, const void *x,
                                 const float *dt, const float *A, const void *B, const void *C,
                                 const float *D, const float *initial_states, void *y,
                                 float *final_states, void *workspace, size_t workspace_bytes,
                                 void *stream);

/*
 * ssd_decode_step -- one O(1) cached decode step for every sequence (section
 * 2 of the page: the fixed-size on-device cache, updated per generated token
 * with no host round trip; section 4: decode is bandwidth-bound).  Each
 * state element is read once and written once, and y is reduced in the same
 * pass.
 *   x [B,H,P], dt [B,H], A [H], B [B,G,N], C [B,G,N], D [H]   one token per sequence
 *   state [B,H,P,N] fp32, updated in place: H <- alpha*H + dt * x (outer) B
 *   y [B,H,P] (io_dtype) = H_new . C + D * x
 * y must not overlap the state or any input.  Supported: N in {16, 32, 64,
 * 128, 256}, 1 <= P <= 2^24, io_dtype SSD_F32 or SSD_BF16.
 */
ssd_status ssd_decode_step(const ssd_dims *dims, const void *x, const float *dt, const float *A,
                           const void *B, const void *C, const float *D, float *state, void *y,
                           void *stream);

/*
 * ssd_decode_steps -- nsteps consecutive cached decode steps in one launch:
 * the result of calling ssd_decode_step nsteps times, step k on the k-th
 * slice of each input, up to rounding (between steps the state may be held
 * divided by the product of the decays since its last rescale, which rounds
 * differently; both forms meet the same tolerance against the exact
 * recurrence), but the state is read once, kept on-chip (in
 * registers) across all steps and written once (section 2 of the page: the
 * decode loop runs on the device around the state cache; "A Persistent-State
 * Dataflow Accelerator for Memory-Bound Linear Attention Decode on FPGA",
 * section 2A: a state that persists on-chip across steps is not re-read
 * from external memory).  The tokens of all steps must be known in advance
 * (teacher-forced steps, appending a short known segment to a cache).
 *   x [S,B,H,P], dt [S,B,H], A [H], B [S,B,G,N], C [S,B,G,N], D [H]   inputs, S = nsteps
 *   state [B,H,P,N] fp32, updated in place (H after step S)
 *   y [S,B,H,P] (io_dtype), y[k] = output of step k
 * Step-major layout: slice k of x, dt, B, C, y is exactly what one
 * ssd_decode_step call takes.  nsteps == 0 or B == 0 does nothing; nsteps < 0
 * is SSD_ERR_SHAPE.  y must not overlap the state or any input; the state
 * must not overlap an input.  Supported: N in {16, 32, 64, 128, 256},
 * 1 <= P <= 2^24, io_dtype SSD_F32 or SSD_BF16, nsteps <= INT32_MAX.
 */
ssd_status ssd_decode_steps(const ssd_dims *dims, int64_t nsteps, const void *x, const float *dt,
                            const float *A, const void *B, const void *C, const float *D,
                            float *state, void *y, void *stream);

/*
 * ssd_gdn_decode_step -- one Gated DeltaNet decode step, the second
 * fixed-state recurrence the pages treat ("A Persistent-State Dataflow
 * Accelerator for Memory-Bound Linear Attention Decode on FPGA", section 2).
 * Per batch row b and value head j, with query/key head i = j / (Hv / Hk)
 * (value heads grouped onto query/key heads, section 2C):
 *     dv  = beta[b,j] (v[b,j] - g[b,j] S^T k[b,i])
 *     S  <- g[b,j] S + k[b,i] dv^T          (S is [dk, dv] fp32, in place)
 *     o[b,j] = S^T q[b,i]                   (computed as g S_old^T q + (q.k) dv,
 *                                            section 2B: one read, one write of S)
 * The page writes the update and the output identity; dv is the gated delta
 * rule's.
 *   q, k  [B, Hk, dk]   io_dtype          v, o [B, Hv, dv]   io_dtype
 *   g, beta [B, Hv]     fp32 (decay gate and write strength, taken as given)
 *   state [B, Hv, dk, dv] fp32, updated in place
 * o must not overlap the state or any input; the state must not overlap an
 * input.  Alignment: state 16 bytes; q, k, v, o element-aligned; g, beta 4.
 * Supported: dk in {64, 128, 256}, dv in {64, 128, 256}, io_dtype SSD_F32 or
 * SSD_BF16.  B == 0 does nothing.
 */
typedef struct ssd_gdn_dims {
    int64_t batch;     /* B >= 0                                              */
    int64_t qk_heads;  /* Hk >= 1                                             */
    int64_t v_heads;   /* Hv >= 1, Hv % Hk == 0                               */
    int64_t dk;        /* key dimension (state rows)                          */
    int64_t dv;        /* value dimension (state columns)                     */
    int32_t io_dtype;  /* ssd_dtype of q, k, v, o                             */
    int32_t reserved;  /* must be 0                                           */
} ssd_gdn_dims;

ssd_status ssd_gdn_decode_step(const ssd_gdn_dims *dims, const void *q, const void *k,
                               const void *v, const float *g, const float *beta, float *state,
                               void *o, void *stream);

/*
 * ssd_gdn_decode_steps -- nsteps Gated DeltaNet decode steps in one launch:
 * the result of nsteps ssd_gdn_decode_step calls on consecutive slices, up
 * to rounding (between steps the state is held divided by the product of the
 * gates since its last rescale), with the state read once, kept on-chip (in
 * registers) across the steps and written once (section 2A of the FPGA page:
 * a state persistent on-chip is not re-read from external memory between
 * steps).
 *   q, k [S, B, Hk, dk]; v, o [S, B, Hv, dv]; g, beta [S, B, Hv]; S = nsteps
 *   state [B, Hv, dk, dv] fp32, updated in place
 * nsteps == 0 or B == 0 does nothing; nsteps < 0 is SSD_ERR_SHAPE.  Shapes,
 * dtypes, alignment and aliasing rules as for ssd_gdn_decode_step.
 */
ssd_status ssd_gdn_decode_steps(const ssd_gdn_dims *dims, int64_t nsteps, const void *q,
                                const void *k, const void *v, const float *g, const float *beta,
                                float *state, void *o, void *stream);

/*
 * ssd_chunk_scan_timed -- measurement entry point: the same computation as
 * ssd_chunk_scan (same arguments and results), run synchronously; the device
 * time of each kernel the scan launched is written to kernel_ms[0 ..
 * *n_kernels-1] (HIP events on the given stream) and their names to
 * kernel_names (static strings; may be NULL).  On input *n_kernels is the
 * capacity of the arrays; on SSD_OK it is the number of kernels launched.
 */
ssd_status ssd_chunk_scan_timed(const ssd_dims *dims, const void *x, const float *dt,
                                const float *A, const void *B, const void *C, const float *D,
                                const float *initial_state, void *y, float *final_state,
                                void *workspace, size_t workspace_bytes, void *stream,
                                float *kernel_ms, const char **kernel_names, int *n_kernels);

#ifdef __cplusplus
}
#endif

#endif /* SSD_H */
