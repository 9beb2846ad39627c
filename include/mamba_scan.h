/*
 * mamba_scan.h -- C ABI of the MI355X (gfx950) selective-scan library.
 *
 * The library computes Mamba's selective state-space scan: the forward pass
 * over a whole sequence and the single-token recurrent step used in O(1)
 * decoding.  For every batch row b, channel d and state n, with a diagonal
 * real A[d,n] = -exp(A_log[d,n]):
 *
 *   Delta_t   = softplus(delta[b,d,t] + delta_bias[d])      (or without softplus)
 *   Abar_t    = exp(Delta_t * A[d,n])                       zero-order hold
 *   Bbar_t    = (exp(Delta_t * A[d,n]) - 1) / A[d,n] * B[b,n,t]
 *               (or Delta_t * B[b,n,t] with MAMBA_SCAN_FLAG_EULER)
 *   h_t[n]    = Abar_t * h_{t-1}[n] + Bbar_t * u[b,d,t]      h_{-1} = initial_state or 0
 *   y[b,d,t]  = (sum_n C[b,n,t] * h_t[n] + D[d] * u[b,d,t]) * SiLU(z[b,d,t])
 *
 * Sources (page and section): the selection mechanism and ZOH discretization,
 * Mamba notes (awesome.papernotes.org), 设计 1; A = -exp(A_log) and the
 * softplus-plus-bias step, same notes, 训练策略, and State space models and
 * Mamba (jonathanding.github.io), §1.5 and §4; the ZOH formula
 * Bbar = A^-1 (exp(Delta A) - I) B, State space models and Mamba, §2; the D
 * skip, Mamba notes 设计 1 pseudo-code; the SiLU gate, Mamba notes 设计 3
 * pseudo-code and 整体框架 figure; the Euler input term Delta B u, the same
 * notes' 设计 1 pseudo-code; the single-token recurrence with a fixed
 * (d, N) state, State space models and Mamba, §3 (recurrence mode) and Mamba
 * notes 设计 2.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every tensor pointer is a caller-owned DEVICE pointer to contiguous,
 *   row-major memory on the current HIP device.  The library never allocates
 *   or frees device memory, never keeps a pointer after returning, and holds
 *   no mutable global state; calls on different streams may run concurrently.
 * - Element types: tensors marked "io" are float32 (MAMBA_SCAN_F32) or
 *   bfloat16 (MAMBA_SCAN_BF16) according to io_dtype; tensors marked "f32"
 *   are always float32.  Each pointer must be aligned to its element size.
 * - All arithmetic is float32 on the device (state included); bfloat16
 *   outputs are rounded to nearest even.
 * - Validation (null pointers, sizes, dtype, alignment, workspace size) is
 *   done on the host before any HIP call.  A failing call returns a non-zero
 *   mamba_scan_status and launches nothing.  After launching, a launch error
 *   reported by hipGetLastError() is returned as MAMBA_SCAN_ERR_HIP.
 * - Work is queued asynchronously on `stream` (a hipStream_t; NULL means the
 *   null stream).  The host never synchronizes.
 * - No output may overlap any input, except `state` in mamba_scan_step,
 *   which is updated in place by design.
 * - NaN and Inf in inputs propagate; they are not checked.  A_log must be
 *   finite (A = 0 is not supported).
 */
#ifndef MAMBA_SCAN_H
#define MAMBA_SCAN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MAMBA_SCAN_ABI_VERSION 2
#define MAMBA_SCAN_MAX_DSTATE 64     /* forward scan and decode step */
#define MAMBA_SCAN_MAX_DSTATE_BWD 64 /* backward pass */

/* Bits of the `flags` argument; any other bit set returns MAMBA_SCAN_ERR_UNSUPPORTED. */
#define MAMBA_SCAN_FLAG_SOFTPLUS 1 /* Delta = softplus(delta + bias); without it Delta = delta + bias */
#define MAMBA_SCAN_FLAG_EULER 2    /* Bbar u = Delta B u (Euler) instead of the zero-order hold      */

typedef enum { MAMBA_SCAN_F32 = 0, MAMBA_SCAN_BF16 = 1 } mamba_scan_dtype;

typedef enum {
  MAMBA_SCAN_OK = 0,
  MAMBA_SCAN_ERR_NULL = 1,        /* a required pointer is NULL                          */
  MAMBA_SCAN_ERR_SHAPE = 2,       /* a size is out of range                              */
  MAMBA_SCAN_ERR_DTYPE = 3,       /* io_dtype is not a mamba_scan_dtype                  */
  MAMBA_SCAN_ERR_ALIGN = 4,       /* a pointer is not aligned to its element size        */
  MAMBA_SCAN_ERR_UNSUPPORTED = 5, /* a size beyond a documented limit or a bad tuning knob */
  MAMBA_SCAN_ERR_WORKSPACE = 6,   /* workspace NULL or smaller than required             */
  MAMBA_SCAN_ERR_HIP = 7          /* the HIP runtime reported an error at launch         */
} mamba_scan_status;

/*
 * Forward selective scan over a whole sequence.
 *
 *   u            (batch, dim, seqlen) io     input sequence, seqlen contiguous
 *   delta        (batch, dim, seqlen) io     pre-activation step size
 *   A_log        (dim, dstate)        f32    A = -exp(A_log)
 *   B, C         (batch, dstate, seqlen) io  input / output projections, shared by all channels
 *   D            (dim)                f32    skip weight, NULL means 0
 *   z            (batch, dim, seqlen) io     gate, NULL means no gate (y is not multiplied)
 *   delta_bias   (dim)                f32    added to delta before softplus, NULL means 0
 *   initial_state(batch, dim, dstate) f32    h_{-1}, NULL means 0
 *   final_state  (batch, dim, dstate) f32    OUT: h after the last token, NULL means not written
 *   y            (batch, dim, seqlen) io     OUT: gated output
 *   flags        MAMBA_SCAN_FLAG_SOFTPLUS and/or MAMBA_SCAN_FLAG_EULER (see above)
 *   workspace    device scratch of at least mamba_scan_fwd_workspace_size(...) bytes,
 *                256-byte aligned; its contents on entry are ignored and on exit undefined.
 *                It holds the chunk carry of a chunked scan (with per-range sums of Delta),
 *                for the plan that splits each row into a head and a shorter tail (129-204
 *                groups of 64 channels) the tail's y in fp32 (batch x dim x tail tokens x 4
 *                bytes), and, for dstate > 16 (run as one pass per 16 states), the fp32
 *                readout summed over the passes (batch x dim x seqlen x 4 bytes)
 *
 * Sizes: batch >= 1, dim >= 1, 1 <= dstate <= 64, seqlen >= 0, and
 * 64 * (seqlen + 8) * sizeof(io element) < 2^31 (seqlen < 4,194,296 for
 * bf16, 8,388,600 for fp32; larger returns MAMBA_SCAN_ERR_UNSUPPORTED).  Every
 * launch must fit a dispatch's 32-bit work-item count: batch * ceil(dim / 64) *
 * chunks * 512 and batch * dim * dstate below 2^32 (else MAMBA_SCAN_ERR_UNSUPPORTED).  seqlen == 0
 * writes no y and sets final_state to initial_state (or zeros); the tensors
 * with a seqlen dimension (u, delta, B, C, z, y) are then empty and may be NULL.
 */
int mamba_scan_fwd(const void* u, const void* delta, const float* A_log, const void* B, const void* C,
                   const float* D, const void* z, const float* delta_bias, const float* initial_state,
                   float* final_state, void* y, int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen,
                   int io_dtype, int flags, void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of workspace mamba_scan_fwd needs for these sizes (0 when it needs none: seqlen == 0,
 * or a one-pass scan with dstate <= 16).
 * Returns (size_t)-1 for sizes mamba_scan_fwd would reject. */
size_t mamba_scan_fwd_workspace_size(int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen, int io_dtype);

/* Scratch held by the library for mamba_scan_fwd_noalloc: one array of this many
 * bytes in each GPU's memory, from the first call on that GPU until the process ends. */
#define MAMBA_SCAN_NOALLOC_SCRATCH_BYTES (64u << 20)

/*
 * mamba_scan_fwd without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).  It calls no hipMalloc, hipFree or other allocating routine:
 * the chunk carry and the multi-pass readout sum live in a static device array of
 * MAMBA_SCAN_NOALLOC_SCRATCH_BYTES bytes per GPU, whose device address is looked up
 * once per device (on the first call with that device current).  The caller still
 * passes every input and output; arguments, layouts, status codes and results are
 * those of mamba_scan_fwd with the automatic launch plan (bit-identical results).
 * The device is the current HIP device; the stream must belong to it.
 *
 * Limit: calls whose mamba_scan_fwd_workspace_size(...) exceeds
 * MAMBA_SCAN_NOALLOC_SCRATCH_BYTES return MAMBA_SCAN_ERR_WORKSPACE and launch
 * nothing (the automatic plan's chunk carry is at most ~7 MB for any size, its per-range
 * sums of Delta at most 16 x seqlen bytes + 1.5 MB more; for 129-204 channel groups of 64
 * with short sequences the plan's tail chunk keeps its y in fp32, at most ~54 MB; a
 * dstate > 16 call adds batch x dim x seqlen x 4 bytes).  Every call on one GPU shares that GPU's array
 * and leaves its contents behind (each call writes what it reads, so nothing needs
 * clearing): calls that overlap in time on one GPU -- on different streams or
 * threads -- race on it and must be serialized by the caller.
 */
int mamba_scan_fwd_noalloc(const void* u, const void* delta, const float* A_log, const void* B, const void* C,
                           const float* D, const void* z, const float* delta_bias, const float* initial_state,
                           float* final_state, void* y, int64_t batch, int64_t dim, int64_t dstate,
                           int64_t seqlen, int io_dtype, int flags, void* stream);

/*
 * Same as mamba_scan_fwd with two explicit launch choices (0 = automatic):
 *   nchunks          number of time chunks scanned in parallel, joined by an
 *                    inter-chunk carry of the state (1 = one sequential pass);
 *                    chunks are whole tiles of 64 tokens, and a request for
 *                    more chunks than tiles is reduced to one chunk per tile.
 *   states_per_wave  states held per lane: 0 or 2 (eight waves per workgroup,
 *                    two per SIMD, the only layout); any other value returns
 *                    MAMBA_SCAN_ERR_UNSUPPORTED.
 * The result is the same function; only rounding order differs.  The
 * workspace must be at least mamba_scan_fwd_workspace_size_ex(...) bytes.
 * Used for testing the chunked path at small sizes and for tuning.
 */
int mamba_scan_fwd_ex(const void* u, const void* delta, const float* A_log, const void* B, const void* C,
                      const float* D, const void* z, const float* delta_bias, const float* initial_state,
                      float* final_state, void* y, int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen,
                      int io_dtype, int flags, int64_t nchunks, int states_per_wave, void* workspace,
                      size_t workspace_bytes, void* stream);

size_t mamba_scan_fwd_workspace_size_ex(int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen, int io_dtype,
                                        int64_t nchunks, int states_per_wave);

/*
 * Causal depthwise conv1d (4 taps) + SiLU fused into the forward scan's load
 * stage: the scan input u is computed on chip from x and never round-trips
 * through HBM (conv, SiLU, then the SSM: Mamba concept page §3.3 flow; State
 * space models and Mamba, Mamba block architecture; the Mamba notes' 设计 3
 * pseudo-code puts SiLU before the conv and is not followed).  Exactly
 * mamba_conv1d_fwd(x, conv_weight, conv_bias, conv_state_in, conv_state_out,
 * kernel_size 4, silu on) followed by mamba_scan_fwd on its output u: u is
 * rounded to the io dtype before the scan uses it, as a stored u would be, so
 * the results are identical to the two calls.
 *
 *   x               (batch, dim, seqlen)  io    conv input
 *   conv_weight     (dim, 4)              f32   taps, oldest input first
 *   conv_bias       (dim)                 f32   NULL means 0
 *   conv_state_in   (batch, dim, 3)       io    the 3 inputs before x, oldest first; NULL means 0
 *   conv_state_out  (batch, dim, 3)       io    OUT: the last 3 inputs; NULL: not written; may
 *                                               equal conv_state_in
 *   u_out           (batch, dim, seqlen)  io    OUT: the conv output (what the scan consumed);
 *                                               NULL: not written
 *   delta, A_log, B, C, D, z, delta_bias, initial_state, final_state, y, flags,
 *   workspace (mamba_scan_fwd_workspace_size bytes): as for mamba_scan_fwd.
 * Sizes and limits as for mamba_scan_fwd, except 1 <= dstate <= 16 (larger returns
 * MAMBA_SCAN_ERR_UNSUPPORTED).  No output may overlap x.
 */
int mamba_scan_fwd_conv(const void* x, const float* conv_weight, const float* conv_bias, const void* conv_state_in,
                        void* conv_state_out, const void* delta, const float* A_log, const void* B, const void* C,
                        const float* D, const void* z, const float* delta_bias, const float* initial_state,
                        float* final_state, void* u_out, void* y, int64_t batch, int64_t dim, int64_t dstate,
                        int64_t seqlen, int io_dtype, int flags, void* workspace, size_t workspace_bytes,
                        void* stream);

/*
 * Forward scan over a variable-length batch: nseq sequences packed one after
 * another along the time axis, sequence s on tokens [cu_seqlens[s],
 * cu_seqlens[s+1]).  Each sequence is scanned exactly as mamba_scan_fwd scans
 * one batch row -- from its own initial state, with its own final state;
 * nothing crosses a sequence boundary.  (The pages define the scan of one
 * sequence: Mamba notes, 设计 1 and 设计 2; State space models and Mamba, §3.
 * Packing unequal lengths without padding restarts the recurrence at every
 * sequence start.)
 *
 *   u, delta, z, y    (dim, total_len)          io   one packed row per channel
 *   B, C              (dstate, total_len)       io
 *   cu_seqlens        (nseq + 1)                int64, DEVICE memory, 8-byte aligned:
 *                     0 = cu[0] <= cu[1] <= ... <= cu[nseq] = total_len (empty
 *                     sequences allowed).  Not checked on the host (it is device
 *                     memory); offsets outside [0, total_len] are clamped, so a bad
 *                     array gives wrong results but no out-of-bounds access.
 *   initial_states    (nseq, dim, dstate) f32   NULL means zeros
 *   final_states      (nseq, dim, dstate) f32   OUT, NULL means not written
 *   A_log, D, delta_bias, flags: as for mamba_scan_fwd
 *   workspace         at least mamba_scan_fwd_varlen_workspace_size(...) bytes (never 0),
 *                     256-byte aligned: the number of pieces per sequence, the state
 *                     entering each piece, and for dstate > 16 a readout sum
 * Sequences are cut into pieces of at most 2048 tokens that are scanned in
 * parallel and joined through their carried states (as the time chunks of
 * mamba_scan_fwd), so one long sequence is not one long serial scan.
 * Sizes: nseq >= 1, dim >= 1, 1 <= dstate <= 64, total_len >= 0 with the seqlen
 * limit of mamba_scan_fwd; (nseq + ceil(total_len / 2048)) * ceil(dim / 64) * 512 < 2^32
 * (the launches' work-items) and nseq * dim * dstate < 2^31 (else MAMBA_SCAN_ERR_UNSUPPORTED).
 */
int mamba_scan_fwd_varlen(const void* u, const void* delta, const float* A_log, const void* B, const void* C,
                          const float* D, const void* z, const float* delta_bias, const int64_t* cu_seqlens,
                          const float* initial_states, float* final_states, void* y, int64_t nseq, int64_t dim,
                          int64_t dstate, int64_t total_len, int io_dtype, int flags, void* workspace,
                          size_t workspace_bytes, void* stream);

/* Bytes of workspace mamba_scan_fwd_varlen needs (> 0); (size_t)-1 for rejected sizes. */
size_t mamba_scan_fwd_varlen_workspace_size(int64_t nseq, int64_t dim, int64_t dstate, int64_t total_len,
                                            int io_dtype);

/*
 * One recurrent step for one token per (batch, channel); the state is updated
 * IN PLACE and y is written.  Exactly one iteration of the forward recurrence.
 *
 *   state     (batch, dim, dstate) f32   IN/OUT
 *   x, dt     (batch, dim)         io    token input and pre-activation step size
 *   A_log     (dim, dstate)        f32
 *   B, C      (batch, dstate)      io
 *   D         (dim)                f32   NULL means 0
 *   z         (batch, dim)         io    NULL means no gate
 *   dt_bias   (dim)                f32   NULL means 0
 *   flags        as for mamba_scan_fwd (softplus of dt + dt_bias; Euler input term)
 *   y         (batch, dim)         io    OUT
 *
 * Sizes: batch >= 1, dim >= 1, 1 <= dstate <= 64, batch <= 262140 (a
 * launch covers four batch rows per grid row) and dim * (4, 8 or 16 lanes for
 * dstate up to 16, 32, 64) < 2^32 (a grid row's work-items); larger returns
 * MAMBA_SCAN_ERR_UNSUPPORTED.
 */
int mamba_scan_step(float* state, const void* x, const void* dt, const float* A_log, const void* B, const void* C,
                    const float* D, const void* z, const float* dt_bias, int flags, void* y, int64_t batch,
                    int64_t dim, int64_t dstate, int io_dtype, void* stream);

/*
 * Backward pass: gradients of a scalar loss through mamba_scan_fwd, given the
 * gradient of its outputs (dy and, optionally, the final state).  Inputs are
 * those of the forward call (same meaning, layout and NULL conventions).  The
 * pages describe the backward pass as recomputing the states instead of
 * storing them (State space models and Mamba, Parallel Scan; Mamba notes,
 * 设计 2); the gradients are the chain rule through the forward recurrence.
 *
 *   dy               (batch, dim, seqlen) io    dL/dy
 *   d_final_state    (batch, dim, dstate) f32   dL/d(final state), NULL means 0
 * Outputs (written in full; no accumulation into existing values):
 *   du, ddelta       (batch, dim, seqlen) io
 *   dA_log           (dim, dstate)        f32
 *   dB, dC           (batch, dstate, seqlen) io
 *   dD               (dim)                f32   NULL: not computed
 *   dz               (batch, dim, seqlen) io    required iff z is given
 *   ddelta_bias      (dim)                f32   NULL: not computed
 *   d_initial_state  (batch, dim, dstate) f32   NULL: not computed
 *   workspace        at least mamba_scan_bwd_workspace_size(...) bytes, 256-byte aligned:
 *                    the state entering every 8-token sub-chunk (batch x ceil(seqlen/8) x 16 x
 *                    dim fp32, for one group of 16 states at a time), per-channel-group /
 *                    per-row partial sums, and for dstate > 16 three (batch, dim, seqlen) fp32
 *                    running sums over state groups
 *   flags            as for mamba_scan_fwd: MAMBA_SCAN_FLAG_SOFTPLUS, MAMBA_SCAN_FLAG_EULER
 * Sizes and limits as for mamba_scan_fwd (1 <= dstate <= 64, MAMBA_SCAN_MAX_DSTATE_BWD;
 * dstate > 16 runs one pass per 16 states), and batch * dstate * seqlen < 2^32 (the dB/dC
 * reduction's work-items; else MAMBA_SCAN_ERR_UNSUPPORTED).  Sums over channels (dB, dC) and
 * over batch rows (dA_log, dD, ddelta_bias) are taken in a fixed order, so
 * repeated calls give identical results.
 */
int mamba_scan_bwd(const void* u, const void* delta, const float* A_log, const void* B, const void* C,
                   const float* D, const void* z, const float* delta_bias, const float* initial_state,
                   const void* dy, const float* d_final_state, void* du, void* ddelta, float* dA_log, void* dB,
                   void* dC, float* dD, void* dz, float* ddelta_bias, float* d_initial_state, int64_t batch,
                   int64_t dim, int64_t dstate, int64_t seqlen, int io_dtype, int flags, void* workspace,
                   size_t workspace_bytes, void* stream);

/* Bytes of workspace mamba_scan_bwd needs (0 only for seqlen == 0); (size_t)-1 for rejected sizes. */
size_t mamba_scan_bwd_workspace_size(int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen, int io_dtype);

/*
 * Multi-head SSM with a scalar decay per head -- the state-space-duality form
 * (State space models and Mamba, §5: head dim P > 1, the P channels of a head
 * share A, the dual matrix carries Lambda_ij = prod_{t=j+1..i} a_t; computed
 * chunk-wise with matrix products inside a chunk and the N x P state passed
 * between chunks).  Per batch row b, head h, head channel p, state n, with
 * A_h = -exp(A_log[h]) and Delta_t = softplus(dt[b,t,h] + dt_bias[h]):
 *
 *   a_t = exp(Delta_t A_h),  w_t = (a_t - 1) / A_h  (Delta_t with MAMBA_SCAN_FLAG_EULER)
 *   h_t[p,n] = a_t h_{t-1}[p,n] + w_t B[b,t,n] x[b,t,h,p]
 *   y[b,t,h,p] = (sum_n C[b,t,n] h_t[p,n] + D[h] x[b,t,h,p]) * SiLU(z[b,t,h,p])
 *
 * i.e. the selective scan above with A and Delta shared by a head's channels.
 * Token-major layouts (as the projections that feed the layer produce them):
 *   x, z, y          (batch, seqlen, nheads, headdim)  bf16, 16-byte aligned
 *   dt               (batch, seqlen, nheads)           bf16
 *   B, C             (batch, seqlen, dstate)           bf16, 16-byte aligned (shared by all heads)
 *   A_log, D, dt_bias (nheads)                          f32 (D, dt_bias may be NULL)
 *   initial_state, final_state (batch, nheads, headdim, dstate) f32, 16-byte aligned, NULL allowed
 *   z                NULL means no gate
 * Supported: io_dtype MAMBA_SCAN_BF16, headdim a multiple of 32 up to 256, dstate 64 or 128
 * (others return MAMBA_SCAN_ERR_UNSUPPORTED); batch * nheads * headdim / 32 * 1024 < 2^32 (the
 * launch's work-items, at most 1024 per slice) and
 * nheads * headdim <= 2^24.  Products take bf16 operands with fp32 accumulation, and the state is
 * carried in fp32.  Where a product reads the fp32 state, or x times its decayed input weight,
 * that operand is split as bf16 hi + bf16 (rest), which gives 16 significant bits over fp32's
 * range.  No workspace.
 */
int mamba_ssd_fwd(const void* x, const void* dt, const float* A_log, const void* B, const void* C, const float* D,
                  const void* z, const float* dt_bias, const float* initial_state, float* final_state, void* y,
                  int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim, int64_t dstate, int io_dtype,
                  int flags, void* stream);

/*
 * Causal depthwise 1-D convolution + SiLU, the step in front of the scan in the
 * Mamba block: conv, then SiLU, then the SSM (Mamba concept page §3.3 flow;
 * State space models and Mamba, Mamba block architecture; the Mamba notes' 设计 3
 * pseudo-code applies SiLU first and is not followed), kernel size 4 (Mamba
 * notes, 设计 3).  Per
 * (batch, channel) with K = kernel_size taps:
 *
 *   a[t] = bias[d] + sum_{k<K} weight[d,k] * x[t - (K-1) + k],   u[t] = a[t] * sigmoid(a[t])
 *
 * (u = a when silu is zero); x at negative times is read from conv_state_in.
 *
 *   x               (batch, dim, seqlen)  io    input
 *   weight          (dim, kernel_size)    f32   taps, oldest input first
 *   bias            (dim)                 f32   NULL means 0
 *   conv_state_in   (batch, dim, K-1)     io    the K-1 inputs before x, oldest first; NULL means 0
 *   conv_state_out  (batch, dim, K-1)     io    OUT: the last K-1 inputs (older ones from conv_state_in
 *                                               when seqlen < K-1); NULL: not written; may equal
 *                                               conv_state_in (updated in place)
 *   u               (batch, dim, seqlen)  io    OUT; must not overlap x
 * Sizes: batch, dim >= 1, seqlen >= 0, 1 <= kernel_size <= 4 (else MAMBA_SCAN_ERR_UNSUPPORTED).
 * Arithmetic in fp32; u is rounded to the io dtype (RNE for bf16).
 */
int mamba_conv1d_fwd(const void* x, const float* weight, const float* bias, const void* conv_state_in,
                     void* conv_state_out, void* u, int64_t batch, int64_t dim, int64_t seqlen, int64_t kernel_size,
                     int io_dtype, int silu, void* stream);

/* Static, NUL-terminated description of a status code (never NULL). */
const char* mamba_scan_status_str(int status);

/* MAMBA_SCAN_ABI_VERSION of the built library. */
int mamba_scan_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MAMBA_SCAN_H */
