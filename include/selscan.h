/*
 * selscan.h -- C ABI of libselscan, the selective state-space scan for AMD
 * Instinct MI355X (gfx950).
 *
 * The operation is the selective (S6) state-space recurrence of Mamba as the
 * pages on state-space models describe it:
 *
 *   delta_t = softplus(raw_t + bias)            (optional bias and softplus)
 *   Abar_t  = exp(delta_t * A)                  (zero-order hold, diagonal A)
 *   Bbar_t  = delta_t * B_t                     (default rule)   or
 *             A^-1 (exp(delta_t * A) - 1) B_t   (exact zero-order hold)
 *   h_t     = Abar_t h_{t-1} + Bbar_t u_t,   h_{-1} = h0 or 0
 *   y_t     = (C_t . h_t + D u_t) * silu(z_t)   (gate optional)
 *
 * Sources: "State-space models" (rayaq.ca), sections "Discretization",
 * "Recurrence and convolution", "Mamba: selection" and "The parallel scan";
 * "State Space Models: Mamba and Beyond", section "Discretization:
 * zero-order hold"; "Structured State Space Models and Mamba: Mathematical
 * Foundations, Continuous Discretization, and Hardware-Aware Associative
 * Scans", sections "The Linear Time-Invariance Bottleneck and the Selective
 * State Space (S6)" (delta with bias) and "Hardware-Aware Parallel
 * Associative Scan" (the pair-composition operator).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Pointers are DEVICE pointers (memory of the current HIP device) unless a
 *    comment says otherwise.  The caller allocates and owns every buffer;
 *    the library allocates nothing, keeps no pointer after it returns and has
 *    no mutable global state, so calls from several host threads are safe.
 *  - Tensors are dense, row-major, innermost index last.  Sequence tensors
 *    keep time innermost: u, delta, z, y are [batch, dim, seqlen] and the
 *    selective B, C are [batch, dstate, seqlen] (shared by all channels of a
 *    sequence).  A is [dim, dstate]; D and delta_bias are [dim]; states are
 *    [batch, dim, dstate].
 *  - io_dtype (ssm_dtype) is the element type of u, delta, B, C, z and y.
 *    A, D, delta_bias and every state are float32.  All arithmetic is float32.
 *  - Work is enqueued on `hip_stream` (a hipStream_t; NULL = the legacy
 *    default stream) and the call returns without waiting.  Device-side
 *    faults surface at the caller's next synchronization.
 *  - Arguments are validated on the host before anything is enqueued.  On
 *    error nothing is enqueued, the return value is the ssm_status code and
 *    ssm_last_error() (thread-local) describes the argument at fault.
 *  - Sequence-tensor base pointers must be 16-byte aligned (every torch
 *    allocation is).  Any seqlen >= 1 is accepted; the fastest path needs
 *    seqlen to be a multiple of 8 (bf16) or 4 (float32).
 *  - Non-finite inputs are not trapped: NaN and Inf propagate.
 */
#ifndef SELSCAN_H
#define SELSCAN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SSM_ABI_VERSION 3

typedef enum { SSM_DTYPE_F32 = 0, SSM_DTYPE_BF16 = 1 } ssm_dtype;

/* Discretization rule (the bbar_mode argument), per ("State-space models",
 * section "Discretization"; "Implementation" for the default):
 *  SSM_BBAR_DELTA_B    Abar = exp(delta A), Bbar = delta B  (Mamba's simplified
 *                      input matrix, the default)
 *  SSM_BBAR_ZOH_EXACT  Abar = exp(delta A), Bbar = A^-1 (exp(delta A) - 1) B
 *  SSM_DISC_EULER      Abar = 1 + delta A,  Bbar = delta B
 *  SSM_DISC_BILINEAR   Abar = (1 + delta A/2) / (1 - delta A/2),
 *                      Bbar = delta B / (1 - delta A/2)
 * The scan, the decode step and the LTI kernel take all four; the backward
 * takes the first two (SSM_E_UNSUPPORTED otherwise). */
typedef enum {
  SSM_BBAR_DELTA_B = 0,
  SSM_BBAR_ZOH_EXACT = 1,
  SSM_DISC_EULER = 2,
  SSM_DISC_BILINEAR = 3
} ssm_bbar_mode;

typedef enum {
  SSM_OK = 0,
  SSM_E_NULL = 1,        /* a required pointer is NULL                         */
  SSM_E_SHAPE = 2,       /* an extent is <= 0 or too large                      */
  SSM_E_DTYPE = 3,       /* io_dtype or bbar_mode is not a known value          */
  SSM_E_ALIGN = 4,       /* a sequence tensor is not 16-byte aligned            */
  SSM_E_ALIAS = 5,       /* an output overlaps an input it must not overlap     */
  SSM_E_UNSUPPORTED = 6, /* a size or mode the entry point does not implement    */
  SSM_E_HIP = 7          /* the HIP runtime refused the launch                  */
} ssm_status;

/*
 * Forward selective scan over whole sequences (prefill / training forward).
 *
 *  u           [batch, dim, seqlen]     io_dtype   input x_t per channel
 *  delta       [batch, dim, seqlen]     io_dtype   raw step; the step used is
 *                                                  softplus(delta + delta_bias)
 *                                                  if delta_softplus, else
 *                                                  delta + delta_bias
 *  A           [dim, dstate]            float32    diagonal of A (negative reals
 *                                                  for a stable system)
 *  Bm, Cm      [batch, dstate, seqlen]  io_dtype   input-dependent B_t and C_t
 *  Dskip       [dim] float32 or NULL (= 0)         skip term D u_t
 *  z           [batch, dim, seqlen] io_dtype or NULL: gate y * silu(z)
 *  delta_bias  [dim] float32 or NULL (= 0)
 *  h0          [batch, dim, dstate] float32 or NULL (= 0): initial state, so a
 *              long sequence can be scanned in pieces (pass the previous
 *              piece's final_state)
 *  y           [batch, dim, seqlen] io_dtype, out.  Must not overlap any input.
 *  final_state [batch, dim, dstate] float32 out, or NULL.  May be exactly h0
 *              (in-place resume) but must not otherwise overlap it.
 *  checkpoints [batch, dim, ceil(seqlen / 128), dstate] float32 out, or NULL:
 *              the state entering every 128-step block (block 0: h0), which
 *              ssm_selective_scan_bwd can take instead of recomputing them.
 *              Must not overlap any input or output.
 *
 * The expanded state [batch, seqlen, dim, dstate] is never written to memory.
 */
int ssm_selective_scan_fwd(const void* u, const void* delta, const float* A, const void* Bm,
                           const void* Cm, const float* Dskip, const void* z,
                           const float* delta_bias, int delta_softplus, const float* h0, void* y,
                           float* final_state, float* checkpoints, int64_t batch, int64_t dim,
                           int64_t dstate, int64_t seqlen, int io_dtype, int bbar_mode,
                           void* hip_stream);

/*
 * One decode step: every sequence advances by one token at constant cost,
 * reading and writing its [dim, dstate] state in place ("State-space
 * models", section "Recurrence and convolution": generation advances the
 * state by one token).
 *
 *  state       [batch, dim, dstate] float32, in/out
 *  u, delta, z [batch, dim]   io_dtype (z may be NULL)
 *  Bm, Cm      [batch, dstate] io_dtype
 *  A, Dskip, delta_bias, delta_softplus, bbar_mode: as for the forward scan
 *  y           [batch, dim] io_dtype out; must not overlap any input or state
 * state, Bm and Cm must be 16-byte aligned (SSM_E_ALIGN otherwise); A is read
 * with 16-byte accesses when it is aligned and dstate is a multiple of 16,
 * element by element otherwise.
 */
int ssm_state_update(float* state, const void* u, const void* delta, const float* A,
                     const void* Bm, const void* Cm, const float* Dskip, const void* z,
                     const float* delta_bias, int delta_softplus, void* y, int64_t batch,
                     int64_t dim, int64_t dstate, int io_dtype, int bbar_mode, void* hip_stream);

/*
 * Time-invariant convolution kernel K[d, k] = sum_n C[d,n] Abar[d,n]^k Bbar[d,n]
 * for k in [0, L), with Abar = exp(delta[d] A[d,n]) and Bbar by bbar_mode.
 * With delta, B and C fixed in time the recurrence equals the causal
 * convolution y = K * u + D u ("State-space models", section "Recurrence and
 * convolution"; "S4: a structured state matrix": with a diagonal A the powers
 * are elementwise).  Used to check the scan against its time-invariant case.
 *
 *  A      [dim, dstate] float32
 *  Bv, Cv rows of dstate float32; row d starts at Bv + d*b_row_stride
 *         (stride 0: one row shared by every channel)
 *  delta  [dim] float32: the step actually used (no softplus applied here)
 *  K      [dim, L] float32 out
 */
int ssm_lti_kernel(const float* A, const float* Bv, const float* Cv, const float* delta, float* K,
                   int64_t dim, int64_t dstate, int64_t L, int64_t b_row_stride,
                   int64_t c_row_stride, int bbar_mode, void* hip_stream);

/*
 * Backward of ssm_selective_scan_fwd: gradients of the loss
 * sum(dy * y) + sum(dfinal_state * final_state) with respect to every input,
 * by reverse-mode differentiation of the recurrence with the states
 * recomputed rather than stored ("State-space models", section "The
 * parallel scan": the fused kernel recomputes the expanded state in the
 * backward pass).  The adjoint lambda_t = dL/dh_t obeys the same recurrence
 * run backwards, lambda_t = dyc_t C_t + Abar_{t+1} lambda_{t+1}, and is
 * scanned the same way.
 *
 * Inputs: the forward's inputs (same layouts, dtypes and rules; y and the
 * final state are not needed), and
 *  dy           [batch, dim, seqlen] io_dtype: gradient of y
 *  dfinal_state [batch, dim, dstate] float32 or NULL (= 0)
 *  checkpoints  the forward's checkpoints for these same inputs, or NULL:
 *               then the backward recomputes them (one more forward pass)
 * Outputs (overwritten; none may overlap an input or another output):
 *  du, ddelta   [batch, dim, seqlen] io_dtype; ddelta is the gradient of the
 *               raw step (before bias and softplus)
 *  dA           [dim, dstate] float32
 *  dB, dC       [batch, dstate, seqlen] io_dtype (summed over channels)
 *  dD           [dim] float32 or NULL (not computed)
 *  dz           [batch, dim, seqlen] io_dtype; required when z is given
 *  ddelta_bias  [dim] float32 or NULL (not computed)
 *  dh0          [batch, dim, dstate] float32 or NULL (not computed)
 *  workspace    device memory of at least
 *               ssm_selective_scan_bwd_workspace_size(batch, dim, dstate, seqlen)
 *               bytes, 16-byte aligned, owned by the caller; its contents on
 *               entry do not matter.  Calls that share a workspace must not
 *               run concurrently.
 * dstate must be 1..64 (SSM_E_UNSUPPORTED otherwise); above 16 the states
 * are taken in tiles of 16, one kernel launch each, and the workspace also
 * holds three float32 [batch, dim, seqlen] sums carried between them.  dA,
 * dD, ddelta_bias, dB and dC are sums accumulated in float32 with atomic
 * adds, so they can differ in the last bits from run to run.
 */
int ssm_selective_scan_bwd(const void* u, const void* delta, const float* A, const void* Bm,
                           const void* Cm, const float* Dskip, const void* z,
                           const float* delta_bias, int delta_softplus, const float* h0,
                           const void* dy, const float* dfinal_state, const float* checkpoints,
                           void* du, void* ddelta, float* dA, void* dB, void* dC, float* dD, void* dz,
                           float* ddelta_bias, float* dh0, void* workspace,
                           int64_t workspace_bytes, int64_t batch, int64_t dim, int64_t dstate,
                           int64_t seqlen, int io_dtype, int bbar_mode, void* hip_stream);

/* Bytes of workspace ssm_selective_scan_bwd needs for these extents (-1 if
 * an extent is out of range).  Host-only, enqueues nothing. */
int64_t ssm_selective_scan_bwd_workspace_size(int64_t batch, int64_t dim, int64_t dstate,
                                              int64_t seqlen);

/*
 * Depthwise causal convolution of width W (1..4) with an optional silu, the
 * step in front of the scan in the Mamba block ("State-space models",
 * section "Mamba: selection": a depthwise causal convolution of width 4 and
 * a silu on one half of the projection).  Per sequence b and channel d:
 *
 *   pre_t = bias_d + sum_{k<W} weight_{d,k} x_{t-(W-1)+k},  out_t = silu(pre_t) or pre_t
 *
 * the cross-correlation of the sequence padded on the left, the convention of
 * the page's F.conv1d snippet ("State-space models", section
 * "Implementation").  The W-1 inputs before t = 0 are state_in or zero.
 *
 *  x, out      [batch, dim, seqlen] io_dtype, 16-byte aligned
 *  weight      [dim, W] float32;  bias [dim] float32 or NULL
 *  state_in    [batch, dim, W-1] float32 (oldest first) or NULL (zeros)
 *  state_out   [batch, dim, W-1] float32 or NULL: the last W-1 inputs of the
 *              extended sequence, what ssm_causal_conv1d_update or a later
 *              call continues from; it may be state_in itself
 * Outputs must not overlap inputs (except state_out == state_in).  Returns
 * SSM_E_UNSUPPORTED for W outside 1..4.  Arithmetic in float32.
 */
int ssm_causal_conv1d_fwd(const void* x, const float* weight, const float* bias,
                          const float* state_in, void* out, float* state_out, int64_t batch,
                          int64_t dim, int64_t seqlen, int64_t width, int apply_silu,
                          int io_dtype, void* hip_stream);

/*
 * One token per (sequence, channel): out = act(bias + sum_k weight_k
 * [conv_state, x]_k), then conv_state (float32 [batch, dim, W-1], updated in
 * place) drops its oldest input and appends x.  x, out are [batch, dim].
 * Equal to ssm_causal_conv1d_fwd with seqlen 1 and state_out = state_in.
 */
int ssm_causal_conv1d_update(const void* x, float* conv_state, const float* weight,
                             const float* bias, void* out, int64_t batch, int64_t dim,
                             int64_t width, int apply_silu, int io_dtype, void* hip_stream);

/*
 * Backward of ssm_causal_conv1d_fwd for the loss sum(dout * out):
 *  dx        [batch, dim, seqlen] io_dtype
 *  dweight   [dim, W] float32, overwritten (sum over sequences and steps)
 *  dbias     [dim] float32 or NULL, overwritten
 *  dstate_in [batch, dim, W-1] float32 or NULL: gradient of state_in
 * pre is recomputed from x.  dweight and dbias are float32 sums with atomic
 * adds, so they can differ in the last bits from run to run.
 */
int ssm_causal_conv1d_bwd(const void* x, const float* weight, const float* bias,
                          const float* state_in, const void* dout, void* dx, float* dweight,
                          float* dbias, float* dstate_in, int64_t batch, int64_t dim,
                          int64_t seqlen, int64_t width, int apply_silu, int io_dtype,
                          void* hip_stream);

/*
 * Mamba-2 scan: the selective scan with A restricted to a scalar per head
 * ("State-space models", section "The parallel scan"; "Structured State
 * Space Models and Mamba ...", section "State Space Duality and Mamba-2").
 * Heads of headdim channels share a step dt and a decay A_h; groups of
 * nheads / ngroups heads share B and C.  Per sequence b, head h, channel p,
 * state n (g = h / (nheads / ngroups)):
 *
 *   dt_t     = softplus(dt_raw_t + dt_bias_h)   (or without the softplus)
 *   h_t[p,n] = exp(dt_t A_h) h_{t-1}[p,n] + dt_t B_t[g,n] x_t[h,p]
 *   y_t[h,p] = (sum_n C_t[g,n] h_t[p,n] + D_h x_t[h,p]) * silu(z_t[h,p])
 *
 * computed in chunks of 64 steps as block matrix products on MFMA (bf16
 * operands, float32 accumulation and state).
 *
 *  x, z, y      [batch, nheads * headdim, seqlen] bf16 (z may be NULL)
 *  dt           [batch, nheads, seqlen] bf16, raw step
 *  Bm, Cm       [batch, ngroups * dstate, seqlen] bf16
 *  A            [nheads] float32 (negative);  Dskip, dt_bias [nheads] or NULL
 *  h0           [batch, nheads, headdim, dstate] float32 or NULL (zeros)
 *  final_state  [batch, nheads, headdim, dstate] float32 or NULL
 *  workspace    at least ssm_ssd_workspace_size(...) bytes of device memory,
 *               16-byte aligned, owned by the caller; calls sharing it must
 *               not run concurrently
 * io_dtype must be SSM_DTYPE_BF16, headdim 64 and dstate one of 32, 64, 128,
 * 256 (SSM_E_UNSUPPORTED otherwise); nheads a multiple of ngroups; seqlen at
 * most 65535 x 64 (SSM_E_SHAPE otherwise).  Outputs must not overlap inputs.
 */
int ssm_ssd_fwd(const void* x, const void* dt, const float* A, const void* Bm, const void* Cm,
                const float* Dskip, const void* z, const float* dt_bias, int dt_softplus,
                const float* h0, void* y, float* final_state, void* workspace,
                int64_t workspace_bytes, int64_t batch, int64_t seqlen, int64_t nheads,
                int64_t headdim, int64_t ngroups, int64_t dstate, int io_dtype, void* hip_stream);

/* Bytes of workspace ssm_ssd_fwd needs (-1 if an extent is out of range). */
int64_t ssm_ssd_workspace_size(int64_t batch, int64_t seqlen, int64_t ngroups, int64_t dstate);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * ssm_ssd_fwd with its workspace in a static scratch array of the library,
 * ssm_ssd_scratch_bytes() = 32 MiB per GPU (held from the first call on that
 * GPU until the process ends).  It allocates and frees nothing.  Arguments,
 * layouts, results and errors are those of ssm_ssd_fwd, plus:
 *  - SSM_E_SHAPE when ssm_ssd_workspace_size(batch, seqlen, ngroups, dstate)
 *    exceeds the scratch (refused before any HIP call; the Mamba-2 2.7B layer
 *    at batch 4, L 8192, N 128 needs 14.7 MB);
 *  - SSM_E_HIP when hip_stream belongs to a device other than the current
 *    one, or the scratch's address cannot be looked up.
 * Every call on one GPU uses the same scratch: calls that overlap in time on
 * one GPU (other streams, other threads) race and must be serialized by the
 * caller.  Nothing in the scratch needs clearing between calls: each call
 * writes all of it that it reads.
 */
int ssm_ssd_fwd_noalloc(const void* x, const void* dt, const float* A, const void* Bm,
                        const void* Cm, const float* Dskip, const void* z, const float* dt_bias,
                        int dt_softplus, const float* h0, void* y, float* final_state,
                        int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                        int64_t ngroups, int64_t dstate, int io_dtype, void* hip_stream);

/* Bytes of the static scratch that ssm_ssd_fwd_noalloc uses (per GPU). */
int64_t ssm_ssd_scratch_bytes(void);

/*
 * Time-invariant path: y = K * u + D u, the causal convolution of every
 * channel with its kernel K_k = C Abar^k Bbar (from ssm_lti_kernel), which is
 * what the recurrence computes when delta, B and C do not depend on the
 * input ("State-space models", section "Recurrence and convolution").
 *  K      [dim, seqlen] float32
 *  u, y   [batch, dim, seqlen] io_dtype;  Dskip [dim] float32 or NULL
 * Direct sum in float32: O(seqlen^2) work per channel.
 */
int ssm_lti_conv(const float* K, const void* u, const float* Dskip, void* y, int64_t batch,
                 int64_t dim, int64_t seqlen, int io_dtype, void* hip_stream);

/*
 * The same y = K * u + D u by FFT ("State-space models", section
 * "Recurrence and convolution": the precomputed kernel applied with an FFT in
 * O(L log L)): per channel, K and each sequence are zero-padded to a power of
 * two M >= 2 seqlen - 1, transformed, multiplied and transformed back, in
 * float32.  Arguments as for ssm_lti_conv, plus a workspace: up to seqlen
 * 4096 the transforms stay in on-chip memory and workspace may be NULL; from
 * 4097 to 2^20 they go through workspace, at least
 * ssm_lti_conv_fft_workspace_size(dim, seqlen) bytes of device memory,
 * 16-byte aligned, owned by the caller, not overlapping any argument (calls
 * sharing it must not run concurrently).  seqlen beyond 2^20:
 * SSM_E_UNSUPPORTED (the direct sum takes any length).
 */
int ssm_lti_conv_fft(const float* K, const void* u, const float* Dskip, void* y, void* workspace,
                     int64_t workspace_bytes, int64_t batch, int64_t dim, int64_t seqlen,
                     int io_dtype, void* hip_stream);

/* Bytes of workspace ssm_lti_conv_fft needs: 0 up to seqlen 4096, -1 if an
 * extent is out of range. */
int64_t ssm_lti_conv_fft_workspace_size(int64_t dim, int64_t seqlen);

/* Static description of a status code (never NULL). */
const char* ssm_status_str(int status);

/* Detail of the last error raised on the calling host thread ("" if none). */
const char* ssm_last_error(void);

/* SSM_ABI_VERSION of the loaded library. */
int ssm_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SELSCAN_H */
