/*
 * ss_scan.h -- C ABI of the MI355X (gfx950) selective-scan library (libssscan.so).
 *
 * The operation (Mamba walk-through, section 3.3 "selective_scan" and the
 * discrete recurrence of section 2.2; D skip and silu(z) gate of the Mamba
 * block, section 3.4; LTI chapter 3.1, section 0.4.2 for the shapes):
 *
 *   for every lane (b, d) and state index n, from h = h0 (zeros if absent):
 *     h_t[n] = exp(delta[b,t,d] * A[d,n]) * h_{t-1}[n] + delta[b,t,d] * B[b,t,n] * u[b,t,d]
 *     y[b,t,d] = sum_n C[b,t,n] * h_t[n]                       (state after the update)
 *              + Dskip[d] * u[b,t,d]                           (if Dskip != NULL)
 *     y[b,t,d] *= z[b,t,d] / (1 + exp(-z[b,t,d]))              (if z != NULL: silu gate)
 *
 * delta is taken as given (already positive); no softplus is applied.
 *
 * Conventions shared by every entry point
 *  - Every tensor pointer is a DEVICE pointer, caller-owned, contiguous and
 *    row-major in the shape stated next to it.  The library allocates no
 *    memory and keeps no state besides a thread-local "last HIP error".
 *  - `dtype` (ss_dtype) is the element type of u, delta, B, C, z and y.
 *    bf16 is the 16-bit brain-float pattern; y is rounded once from fp32 with
 *    round-to-nearest-even.  A, Dskip and every state (h0, h_last, h) are fp32.
 *    All arithmetic is fp32.
 *  - Alignment: A, h0, h_last and h must be 16-byte aligned, the workspace
 *    256-byte aligned; every other tensor must be aligned to its element size.
 *  - Calls are asynchronous on `stream` (NULL = the default stream): SS_OK
 *    means every kernel was enqueued.  Arguments are validated on the host,
 *    synchronously, before anything is enqueued; a rejected call enqueues
 *    nothing.  NaN/Inf inputs are not checked and propagate.
 *  - Errors: SS_ERR_INVALID_ARG (NULL required pointer, size <= 0, size
 *    overflow, misalignment, forbidden overlap), SS_ERR_UNSUPPORTED (dstate
 *    other than 16, unknown dtype), SS_ERR_WORKSPACE (workspace too small or
 *    NULL), SS_ERR_HIP (a HIP call or launch failed; see
 *    ss_last_hip_error()).  No exceptions cross the ABI.
 */
#ifndef SS_SCAN_H
#define SS_SCAN_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    SS_OK = 0,
    SS_ERR_INVALID_ARG = 1,
    SS_ERR_UNSUPPORTED = 2,
    SS_ERR_WORKSPACE = 3,
    SS_ERR_HIP = 4
} ss_status;

typedef enum { SS_F32 = 0, SS_BF16 = 1 } ss_dtype;

/*
 * Option bits of ss_scan_fwd_ex / ss_step_ex (0 = the plain ss_scan_fwd /
 * ss_step behaviour):
 *  SS_DELTA_SOFTPLUS  the step size is softplus(delta + delta_bias[d]),
 *                     softplus(v) = log(1 + e^v) (LTI chapter, section
 *                     3.1.4.2: softplus of a per-channel parameter plus a
 *                     projection of the input).  Without it a given
 *                     delta_bias is added as is.
 *  SS_B_ZOH           the zero-order-hold input term of the walk-through's
 *                     section 2.2, Bbar = (delta*A)^-1 (exp(delta*A) - 1) *
 *                     delta*B, elementwise for the diagonal A and equal to
 *                     delta*B where delta*A = 0; instead of the Euler term
 *                     delta*B.
 * Unknown bits return SS_ERR_UNSUPPORTED.
 */
typedef enum { SS_DELTA_SOFTPLUS = 1, SS_B_ZOH = 2 } ss_option;

/*
 * ss_scan_plan -- how ss_scan_fwd splits the sequence axis for this shape.
 *
 * The scan is cut into n_chunks_K = ceil(seqlen / chunk_len_T) chunks; chunk c
 * covers timesteps [c*chunk_len_T, min((c+1)*chunk_len_T, seqlen)).  Chunks
 * are joined by an exact associative combine of affine pairs (LTI chapter
 * 3.1, section 3.1.5.2, parallel scan over an associative operator):
 * (a1, b1) then (a2, b2) gives (a2*a1, a2*b1 + b2).  Chunks shorter than
 * 1024 rows (or with checkpoints): every chunk but the last first has its end
 * state from a zero start found (its affine pair), the pairs are combined
 * into each chunk's carry (with at most 16 chunks by the pass that produces
 * y, at the start of each chunk), and every chunk is run from its carry to
 * produce y.  Chunks of 1024 rows or more (a multiple of 16), without
 * checkpoints: every chunk is first run from its own start (h0 for the
 * first, zero for the others), writing y and its end state; the carries
 * follow; then each later chunk is rerun from its carry until the carry's
 * effect has decayed below fp32 resolution (all step sizes of the chunk >= 0,
 * A <= 0, and exp(A * sum of delta) * |carry| <= 2^-24 of the lane's largest
 * state entry, checked after 128 rows and then every 64 rows for each 32 or
 * 64 channels), else to its end.  Either way the result is the one-pass
 * recurrence up to fp32 rounding.
 *
 * The chunk length is a power of two chosen from the shape only: pure,
 * host-only, deterministic.  Writes *chunk_len_T and *n_chunks_K (either may
 * be NULL).  Returns SS_ERR_INVALID_ARG for sizes <= 0 or sizes whose element
 * counts overflow int64.
 */
ss_status ss_scan_plan(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate,
                       int64_t* chunk_len_T, int64_t* n_chunks_K);

/*
 * ss_scan_plan_ex -- ss_scan_plan with a chunk length request:
 * chunk_len_request 0 is ss_scan_plan's choice; a positive value forces that
 * chunk length (any value >= 1, not only powers of two); a negative one is
 * SS_ERR_INVALID_ARG.  This is the plan ss_scan_fwd_ex and ss_scan_fwd_ckpt
 * use for the same request.
 */
ss_status ss_scan_plan_ex(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate,
                          int64_t chunk_len_request, int64_t* chunk_len_T, int64_t* n_chunks_K);

/*
 * ss_scan_workspace_bytes -- device workspace ss_scan_fwd needs for this
 * shape ((size_t)-1 for invalid sizes).  Always > 0: even a one-chunk plan
 * needs the fp32 copy of B and C described below.
 *
 * Workspace layout (fp32 words, K = n_chunks, BD = batch*dim, N = dstate),
 * valid after the call completes:
 *   when K > 1:
 *   [0, K*BD*N)            state slots (K, batch, dim, N): slot 0 holds the
 *                          initial state (h0, or zeros); slot c, 1 <= c < K,
 *                          holds the state right after timestep c*chunk_len-1,
 *                          i.e. the carry into chunk c.  (With a checkpoint
 *                          output the chunked plans always take the
 *                          aggregate pass.)
 *   [K*BD*N, +K*BD)        sum of delta over chunk c, (K, batch, dim).
 *   then, when chunk_len >= 1024 and a multiple of 16 (emit first, see
 *   ss_scan_plan): (K-1, batch, ceil(dim/32)) uint32 words, 1 where chunk c+1
 *   was rerun over its whole length, 0 where the rerun stopped early;
 *   then (K, batch, ceil(dim/32)) uint32 words, 1 where chunk c has a
 *   negative step size.
 *   otherwise (the aggregate pass), when K <= 16: (K-1, batch, dim, N), the
 *   end state of chunk c from a zero start (the pass that produces y forms
 *   the carries from these itself).
 *   always, from the next multiple of 256 bytes to the end:
 *                          an fp32 copy of B and C, per (batch row, chunk),
 *                          regrouped in the order the scan kernels read it
 *                          and zero-padded past each chunk's end; its
 *                          arrangement is internal to the library.  (The
 *                          aggregate-pass plans without checkpoints read B
 *                          and C directly and leave this region untouched;
 *                          it stays in the size so that the size depends on
 *                          the shape alone.)
 */
size_t ss_scan_workspace_bytes(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate);

/*
 * ss_scan_workspace_bytes_ex -- the workspace of ss_scan_fwd_ex and
 * ss_scan_fwd_ckpt for a chunk length request (as ss_scan_plan_ex; 0 gives
 * ss_scan_workspace_bytes).  (size_t)-1 for invalid sizes or a negative
 * request.  Same layout.
 */
size_t ss_scan_workspace_bytes_ex(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate,
                                  int64_t chunk_len_request);

/*
 * ss_scan_fwd -- the selective scan over full sequences (Mamba walk-through,
 * section 3.3; fused as the hardware-aware path of section 3.3 and LTI chapter
 * section 3.1.5.3 describe: the discretised operands and the per-timestep
 * states are never written to memory).
 *
 *   u, delta, z : (batch, seqlen, dim)   dtype      (z NULL: no gate)
 *   A           : (dim, dstate)          fp32
 *   B, C        : (batch, seqlen, dstate) dtype
 *   Dskip       : (dim,)                 fp32       (NULL: no skip term)
 *   h0          : (batch, dim, dstate)   fp32       (NULL: zero initial state)
 *   y           : (batch, seqlen, dim)   dtype      output
 *   h_last      : (batch, dim, dstate)   fp32       output, state after the
 *                                                   last timestep (NULL: not written)
 *   workspace   : ss_scan_workspace_bytes(...) bytes of device memory,
 *                 256-byte aligned, caller-owned (contents on entry unused)
 *
 * The sequence is split as ss_scan_plan says.
 * y must not overlap any other tensor; h_last must not overlap any input
 * except that it may be exactly h0 (in-place continuation of a state).  The
 * workspace must not overlap any tensor.  dstate must be 16.
 */
ss_status ss_scan_fwd(const void* u, const void* delta, const float* A, const void* B, const void* C,
                      const float* Dskip, const void* z, const float* h0,
                      void* y, float* h_last,
                      void* workspace, size_t workspace_bytes,
                      int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate,
                      ss_dtype dtype, hipStream_t stream);

/*
 * ss_scan_fwd_ex -- ss_scan_fwd with the step-size and input-term options and
 * a chunk length request:
 *   delta_bias : (dim,) fp32, 4-byte aligned, or NULL (no bias); an input, so
 *                y and h_last must not overlap it
 *   options    : SS_DELTA_SOFTPLUS and/or SS_B_ZOH (see ss_option)
 *   chunk_len_request : as for ss_scan_plan_ex (0 = ss_scan_plan's choice);
 *                the workspace is then ss_scan_workspace_bytes_ex(...) bytes
 * Every other argument, the validation and the errors are as for ss_scan_fwd,
 * which is ss_scan_fwd_ex with delta_bias = NULL, options = 0 and
 * chunk_len_request = 0.
 */
ss_status ss_scan_fwd_ex(const void* u, const void* delta, const float* A, const void* B, const void* C,
                         const float* Dskip, const void* z, const float* h0,
                         const float* delta_bias, uint32_t options,
                         void* y, float* h_last,
                         void* workspace, size_t workspace_bytes,
                         int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate,
                         int64_t chunk_len_request, ss_dtype dtype, hipStream_t stream);

/* Size in bytes of ss_scan_fwd_noalloc's per-GPU array (the largest workspace it serves). */
#define SS_NOALLOC_MAX_WORKSPACE_BYTES ((size_t)32 << 20)

/*
 * ss_scan_fwd_noalloc -- ss_scan_fwd for callers that cannot allocate device
 * memory: code under stream (graph) capture, tight serving loops, harnesses
 * that forbid allocation.  It takes no workspace: the library keeps one static
 * device array of SS_NOALLOC_MAX_WORKSPACE_BYTES (32 MiB) per GPU,
 * created with the code object and held until the process ends, and the call
 * allocates nothing (no hipMalloc, no allocating library routine).  The first
 * call on a device looks up that device's array address (one HIP symbol query
 * per device, kept for later calls).
 *
 * Arguments, results, validation and errors are as for ss_scan_fwd, plus:
 * a shape whose ss_scan_workspace_bytes exceeds the array returns
 * SS_ERR_WORKSPACE (before any HIP call); SS_ERR_HIP if the symbol query
 * fails.  Every call on one GPU shares that GPU's array and leaves its own
 * contents there: calls that overlap in time on one GPU (two streams, or two
 * host threads) race and must be ordered by the caller.  Nothing in the array
 * needs clearing between calls: each call writes every word it reads.
 */
ss_status ss_scan_fwd_noalloc(const void* u, const void* delta, const float* A, const void* B, const void* C,
                              const float* Dskip, const void* z, const float* h0, void* y, float* h_last,
                              int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, ss_dtype dtype,
                              hipStream_t stream);

/*
 * ss_scan_ckpt_bytes -- size of the state checkpoints of a (batch, seqlen,
 * dim, dstate) scan: ceil(seqlen/16) * batch * dim * dstate fp32 words, in
 * bytes ((size_t)-1 for invalid sizes).
 *
 * ss_scan_fwd_ckpt -- ss_scan_fwd_ex that also keeps the states the backward
 * needs, so that ss_scan_bwd_ckpt can reuse them instead of recomputing them
 * (the walk-through's section 3.3 recomputes the per-timestep states in the
 * backward; here only every 16th is kept, the way the chunked forward keeps
 * only its chunk carries, LTI chapter section 3.1.5.2):
 *   ckpt : (ceil(seqlen/16), batch, dstate, dim) fp32 output, 16-byte aligned;
 *          ckpt[j, b, n, d] = the state h[n] of lane (b, d) entering timestep
 *          16*j, i.e. after timestep 16*j - 1 (h0, or zero, for j = 0)
 * ckpt must not overlap any input, y, h_last or the workspace.  With more than
 * one chunk the chunk length must be a multiple of 16 (SS_ERR_UNSUPPORTED
 * otherwise).  Every other argument, the validation and the errors are as for
 * ss_scan_fwd_ex; y and h_last are the same as ss_scan_fwd_ex's.
 */
size_t ss_scan_ckpt_bytes(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate);

ss_status ss_scan_fwd_ckpt(const void* u, const void* delta, const float* A, const void* B, const void* C,
                           const float* Dskip, const void* z, const float* h0,
                           const float* delta_bias, uint32_t options,
                           void* y, float* h_last, float* ckpt,
                           void* workspace, size_t workspace_bytes,
                           int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate,
                           int64_t chunk_len_request, ss_dtype dtype, hipStream_t stream);

/*
 * ss_step -- one token of the recurrent (constant-state) mode: the walk-
 * through's section 6 (O(1) state per generated token) and the interactive
 * demo page (the state is all that is carried from one token to the next).
 * The same update as one timestep of ss_scan_fwd, applied in place to h:
 *
 *   h     : (batch, dim, dstate) fp32, read and overwritten
 *   u, delta, z : (batch, dim)    dtype   (z NULL: no gate)
 *   A     : (dim, dstate)         fp32
 *   B, C  : (batch, dstate)       dtype
 *   Dskip : (dim,)                fp32    (NULL: no skip term)
 *   y     : (batch, dim)          dtype   output
 *
 * h and y must not overlap each other or any input.  dstate must be 16.
 */
ss_status ss_step(float* h, const void* u, const void* delta, const float* A, const void* B,
                  const void* C, const float* Dskip, const void* z, void* y,
                  int64_t batch, int64_t dim, int64_t dstate, ss_dtype dtype, hipStream_t stream);

/*
 * ss_step_ex -- ss_step with delta_bias ((dim,) fp32 or NULL) and the options
 * of ss_scan_fwd_ex; a token of ss_step_ex matches one timestep of
 * ss_scan_fwd_ex with the same options.  ss_step is ss_step_ex with
 * delta_bias = NULL and options = 0.
 */
ss_status ss_step_ex(float* h, const void* u, const void* delta, const float* A, const void* B,
                     const void* C, const float* Dskip, const void* z,
                     const float* delta_bias, uint32_t options, void* y,
                     int64_t batch, int64_t dim, int64_t dstate, ss_dtype dtype, hipStream_t stream);

/*
 * ss_scan_bwd_workspace_bytes -- device workspace ss_scan_bwd needs for this
 * shape ((size_t)-1 for invalid sizes).  It holds the fp32 B/C panel, state
 * checkpoints every 16 timesteps (ceil(seqlen/16) * batch * dim * dstate
 * words), per-64-channel partial sums of dB and dC (2 * ceil(dim/64) * batch *
 * seqlen * dstate words) and per-batch-row partial sums of dA, dD and the
 * delta bias; its arrangement is internal to the library.
 */
size_t ss_scan_bwd_workspace_bytes(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate);

/*
 * ss_scan_bwd -- gradients of the scan (reverse mode), recomputing the states
 * from the inputs instead of storing them (the backward of the walk-through's
 * section 3.3 and the LTI chapter's section 3.1.5.3).  With out = ss_scan_fwd_ex
 * of the same inputs and options, it returns the gradients of
 *     sum(dy * out) + sum(dh_last * h_last)
 * with respect to every input:
 *
 *   forward inputs : as ss_scan_fwd_ex, options included (SS_DELTA_SOFTPLUS,
 *                    SS_B_ZOH: the input coefficient beta = (e^{delta A} - 1)/A
 *                    has dbeta/ddelta = e^{delta A} and dbeta/dA =
 *                    delta^2 psi(delta A), psi(x) = (x e^x - e^x + 1)/x^2)
 *   dy          : (batch, seqlen, dim)   dtype   gradient of out
 *   dh_last     : (batch, dim, dstate)   fp32    gradient of h_last (NULL: zero)
 *   du, ddelta  : (batch, seqlen, dim)   dtype   output; ddelta is with respect
 *                                                to delta as passed (the raw
 *                                                value under SS_DELTA_SOFTPLUS)
 *   dz          : (batch, seqlen, dim)   dtype   output, required iff z is given
 *   dA          : (dim, dstate)          fp32    output
 *   dB, dC      : (batch, seqlen, dstate) dtype  output (sums over channels in
 *                                                fp32, rounded once)
 *   dD          : (dim,)                 fp32    output, required iff Dskip is given
 *   ddelta_bias : (dim,)                 fp32    output, required iff delta_bias is given
 *   dh0         : (batch, dim, dstate)   fp32    output, gradient of the initial
 *                                                state (NULL: not written)
 *   workspace   : ss_scan_bwd_workspace_bytes(...) bytes, 256-byte aligned
 *
 * Sums over channels, timesteps and batch rows are taken in a fixed order:
 * the results are the same from run to run.  Outputs must not overlap the
 * inputs or each other; the workspace overlaps nothing.  One batch row's
 * (seqlen, dim) slab must stay below 2 GiB (SS_ERR_UNSUPPORTED otherwise).
 * Alignment and the other errors are as for ss_scan_fwd.
 */
ss_status ss_scan_bwd(const void* u, const void* delta, const float* A, const void* B, const void* C,
                      const float* Dskip, const void* z, const float* h0,
                      const float* delta_bias, uint32_t options,
                      const void* dy, const float* dh_last,
                      void* du, void* ddelta, float* dA, void* dB, void* dC,
                      float* dD, void* dz, float* ddelta_bias, float* dh0,
                      void* workspace, size_t workspace_bytes,
                      int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate,
                      ss_dtype dtype, hipStream_t stream);

/*
 * ss_scan_bwd_ckpt -- ss_scan_bwd from the checkpoints of a forward pass:
 *   ckpt : (ceil(seqlen/16), batch, dstate, dim) fp32, 16-byte aligned, as
 *          written by ss_scan_fwd_ckpt for the same inputs, h0 and options;
 *          read only.  Any other contents give the gradients of a scan whose
 *          state entering every 16th timestep is ckpt's.
 *   workspace : ss_scan_bwd_ckpt_workspace_bytes(...) bytes, 256-byte aligned
 *          (the checkpoint region of ss_scan_bwd's workspace is not needed)
 * The pass that recomputes the checkpoints is skipped.  With ss_scan_fwd_ckpt's
 * checkpoints of a one-chunk forward the results are ss_scan_bwd's bit for
 * bit; a chunked forward's checkpoints come from its chunk carries and differ
 * from the sequential ones by rounding only.  ckpt is an input: outputs
 * and the workspace must not overlap it.  Every other argument, the
 * validation and the errors are as for ss_scan_bwd.
 */
size_t ss_scan_bwd_ckpt_workspace_bytes(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate);

ss_status ss_scan_bwd_ckpt(const void* u, const void* delta, const float* A, const void* B, const void* C,
                           const float* Dskip, const void* z, const float* h0,
                           const float* delta_bias, uint32_t options,
                           const void* dy, const float* dh_last, const float* ckpt,
                           void* du, void* ddelta, float* dA, void* dB, void* dC,
                           float* dD, void* dz, float* ddelta_bias, float* dh0,
                           void* workspace, size_t workspace_bytes,
                           int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate,
                           ss_dtype dtype, hipStream_t stream);

/*
 * ss_conv1d_silu -- the Mamba block's causal depthwise convolution and SiLU
 * that produce the scan's input u (walk-through, section 3.4: a Conv1d with
 * one filter of `width` taps per channel, padding width-1, only the first L
 * outputs kept, then silu):
 *   u[b,t,d] = silu(bias[d] + sum_{k<width} weight[d,k] * x[b, t-width+1+k, d]),
 * with x = 0 before t = 0.
 *
 *   x      : (batch, seqlen, dim) dtype, rows x_row_stride (>= dim) elements
 *            apart: the x half of the in-projection output xz (batch, seqlen,
 *            2*dim) is read in place with x_row_stride = 2*dim
 *   weight : (dim, width) fp32;  bias : (dim,) fp32 or NULL (no bias)
 *   u      : (batch, seqlen, dim) dtype, contiguous; must not overlap x,
 *            weight or bias
 *   width  : 2, 3 or 4 (SS_ERR_UNSUPPORTED otherwise)
 * x and u are aligned to their element size; weight and bias to 4 bytes.
 */
ss_status ss_conv1d_silu(const void* x, int64_t x_row_stride, const float* weight, const float* bias,
                         void* u, int64_t batch, int64_t seqlen, int64_t dim, int64_t width,
                         ss_dtype dtype, hipStream_t stream);

/*
 * ss_ssd_fwd -- the multi-head state-space recurrence of Mamba-2 (walk-through,
 * section 4.1: h_t = A_t h_{t-1} + B_t x_t, y_t = C_t h_t with a state per
 * head, and its dual form, a causal structured matrix applied to the inputs;
 * section 5.2: heads of 64 channels, d_state 64-256).  Per batch row b and
 * head h, with an (dstate x headdim) state S and a scalar decay per head:
 *   S_t = exp(dt[b,t,h] A[h]) S_{t-1} + dt[b,t,h] B[b,t,:] x[b,t,h,:]^T
 *   y[b,t,h,:] = S_t^T C[b,t,:] + D[h] x[b,t,h,:]
 * (the discretisation of ss_scan_fwd applied per head; B and C shared by all
 * heads).  Computed chunk by chunk on the matrix cores: bf16 products with
 * fp32 accumulation, the state kept in fp32.
 *
 *   x, y   : (batch, seqlen, heads, headdim)  bf16, 16-byte aligned
 *   dt     : (batch, seqlen, heads)           bf16 (positive step sizes)
 *   A      : (heads,) fp32;  D : (heads,) fp32 or NULL
 *   B, C   : (batch, seqlen, dstate)          bf16, 16-byte aligned
 *   h0     : (batch, heads, dstate, headdim)  fp32 or NULL (zero state)
 *   h_last : (batch, heads, dstate, headdim)  fp32 output or NULL
 * Supported: dtype SS_BF16, headdim 64, dstate 64, 128 or 256, and one batch
 * row of x (seqlen*heads*headdim*2 bytes) and of B (seqlen*dstate*2 bytes)
 * below 2 GiB (SS_ERR_UNSUPPORTED otherwise).  y and h_last must not overlap
 * the inputs or each other.  dstate 256 needs a workspace: ss_ssd_fwd returns
 * SS_ERR_WORKSPACE for it; call ss_ssd_fwd_ex.
 */
ss_status ss_ssd_fwd(const void* x, const void* dt, const float* A, const void* B, const void* C,
                     const float* D, const float* h0, void* y, float* h_last,
                     int64_t batch, int64_t seqlen, int64_t heads, int64_t headdim, int64_t dstate,
                     ss_dtype dtype, hipStream_t stream);

/*
 * ss_ssd_workspace_bytes -- device workspace ss_ssd_fwd_ex needs: 0 for dstate
 * 64 and 128; for dstate 256, batch*seqlen*heads*headdim*4 bytes (the fp32
 * part of y from the first half of the state entries, which the pass over the
 * second half adds to its own).  (size_t)-1 for sizes <= 0 or overflowing.
 */
size_t ss_ssd_workspace_bytes(int64_t batch, int64_t seqlen, int64_t heads, int64_t headdim, int64_t dstate);

/*
 * ss_ssd_fwd_ex -- ss_ssd_fwd with a workspace (ss_ssd_workspace_bytes(...)
 * bytes, 256-byte aligned, overlapping no argument; NULL when that is 0).
 * dstate 256 also requires (seqlen + 64) * heads * headdim * 2 <= 2^31.
 */
ss_status ss_ssd_fwd_ex(const void* x, const void* dt, const float* A, const void* B, const void* C,
                        const float* D, const float* h0, void* y, float* h_last,
                        void* workspace, size_t workspace_bytes,
                        int64_t batch, int64_t seqlen, int64_t heads, int64_t headdim, int64_t dstate,
                        ss_dtype dtype, hipStream_t stream);

/* Static, human-readable name of a status code ("unknown status" otherwise). */
const char* ss_status_string(ss_status s);

/* hipError_t value behind the last SS_ERR_HIP returned on this thread (0 if none). */
int ss_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* SS_SCAN_H */
