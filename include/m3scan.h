/*
 * m3scan.h -- C ABI of libm3scan, the MI355X (gfx950) implementation of the
 * Mamba-3 sequence mixer: chunked prefill (m3_scan_fwd) and one autoregressive
 * step (m3_decode_step).
 *
 * The operation (per batch row b and head h, t = 1..L):
 *
 *   h_t = alpha_t R_t h_{t-1} + beta_t R_t B_{t-1} X_{t-1} + gamma_t B_t X_t
 *   y_t = C_t^T h_t
 *   alpha_t = exp(dt_t A_h),  beta_t = (1 - lam_t) dt_t alpha_t,  gamma_t = lam_t dt_t
 *
 *   - Exponential-trapezoidal discretization: Mamba-3 summary on b-lab.team,
 *     section 1 "Exponential-Trapezoidal Discretization" (recurrence and the
 *     alpha/beta/gamma shorthand; lam = 1 is Mamba-2's Euler rule, lam = 1/2
 *     the classic trapezoid).
 *   - R_t: block-diagonal rotation with N/2 blocks R(dt_t theta_t[i]) =
 *     [[cos, -sin], [sin, cos]] on adjacent state rows (2i, 2i+1): same page,
 *     section 2 "Complex-Valued SSM" (real form of the complex SSM,
 *     Proposition 2).  The library applies it as data-dependent RoPE on B and
 *     C (Proposition 3, the "RoPE trick").  R_t also carries the previous
 *     endpoint B_{t-1} X_{t-1} across the step (the trapezoid's left endpoint
 *     is propagated by the same flow as the state).
 *   - MIMO: B_t, C_t are N x R, X_t is R x P; the input term B_t X_t sums the
 *     R ranks and the readout C_t^T h_t gives R outputs of length P: same
 *     page, section 3 "MIMO".
 *
 * Data layout.  Every tensor is dense, row-major, contiguous:
 *   x, y            [batch, seqlen, nheads, rank, headdim]     io dtype
 *   B, C            [batch, seqlen, nheads, rank, dstate]      io dtype
 *   dt, lam         [batch, seqlen, nheads]                    float32
 *   theta           [batch, seqlen, nheads, dstate/2]          float32
 *   A               [nheads]                                   float32
 *   state record:
 *     h             [batch, nheads, dstate, headdim]           float32
 *     B_prev        [batch, nheads, rank, dstate]              io dtype
 *     x_prev        [batch, nheads, rank, headdim]             io dtype
 * The state record (h_t, B_t, X_t) is everything needed to continue: a scan
 * split into several calls, or a scan followed by decode steps, equals one
 * scan.  h is the true state after the last token; the record's (B, X) pair is
 * the last token's input, which the next token's trapezoid term needs.
 *
 * io dtype is M3_F32 (float) or M3_BF16 (bfloat16).  Arithmetic is float32
 * (bf16 products on matrix cores accumulate in float32 for M3_BF16).
 *
 * Ownership and execution.  All pointers are device pointers owned by the
 * caller; the library keeps none of them after a call returns.  m3_scan_fwd
 * and m3_decode_step allocate nothing, never synchronise, and enqueue their
 * kernels on the caller's stream (a hipStream_t passed as void*, NULL = the
 * default stream); the results are ready when that stream reaches them.
 * Calls are reentrant; the library holds no global mutable state besides a
 * thread-local record of the last HIP error.
 *
 * Options (m3_options, zero-initialised = none of them; both entry points):
 *   - per-token decay rate A_t: the Mamba-3 summary on b-lab.team, section 1,
 *     writes the decay as exp(dt_t A_t); A is then [batch, seqlen, nheads]
 *     (decode: [batch, nheads]) instead of one value per head;
 *   - head groups: B and C given once per group of nheads/ngroups consecutive
 *     heads, [batch, seqlen, ngroups, rank, dstate] (decode: [batch, ngroups,
 *     rank, dstate]); head h reads group h / (nheads / ngroups);
 *   - phase interventions of "Understanding Mamba-3 Through Oscillatory
 *     Dynamics" (section 5.3, appendix D.4): the phase increments dt_t theta_t
 *     are zeroed, negated, or shuffled across the rotary pairs (pair i uses
 *     theta[..., perm[i]] at every step); the decay is untouched;
 *   - packed sequences (m3_scan_fwd only): cu_seqlens[batch + 1] gives the
 *     token offsets of `batch` sequences of different lengths packed along
 *     one token axis; the token arrays are then [seqlen, nheads, ...] with
 *     seqlen the total, and each sequence has its own state record;
 *   - pre-mixer: the Towards AI explainer of Mamba-3 (section II) pairs the
 *     mixer with QKNorm-style RMSNorm and channel-wise biases on B and C.
 *     With premix set, dt and lam are raw projections and the mixer uses
 *         dt  = softplus(dt_raw + dt_bias[h]),   lam = sigmoid(lam_raw),
 *         B'  = B / sqrt(mean_n(B^2) + eps) * B_norm_w[n] + B_bias[h, r, n]
 *     (and C' alike), the mean over the dstate entries of one (token, head,
 *     rank) row.  The state record's B_prev holds B' (what the recurrence
 *     consumed), so a record can be continued with or without the pre-mixer.
 *
 * Errors.  Every entry point validates all arguments before making any HIP
 * call and returns M3_OK or one of the negative m3_status codes below.  On an
 * error nothing has been enqueued.  NaN or Inf inputs are not errors: they
 * propagate into the outputs (within the dense chunk form a non-finite input
 * may reach outputs of earlier tokens of the same chunk).  The waves of one
 * prefill workgroup hand chunk totals to each other through a counter with a
 * bounded wait (so that no defect can hang the device); if such a wait ever
 * ran out, that (batch, head)'s y and final state are NaN rather than
 * silently wrong.
 */
#ifndef M3SCAN_H
#define M3SCAN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define M3_ABI_VERSION 6

typedef enum {
    M3_F32 = 0,
    M3_BF16 = 1
} m3_dtype;

typedef enum {
    M3_PHASE_NATIVE = 0,   /* theta as given */
    M3_PHASE_ZERO = 1,     /* no rotation; theta is not read and may be NULL */
    M3_PHASE_REVERSE = 2,  /* theta negated */
    M3_PHASE_SHUFFLE = 3,  /* pair i uses theta[..., phase_perm[i]] */
    /* m3_decode_step only: the rotation removed from writing, from readout, or
     * from both, for prediction steps after a native context ("Understanding
     * Mamba-3 Through Oscillatory Dynamics", section 5.3 and appendix D.4).
     * In the frame that turns with the accumulated angle Phi (phase_in plus
     * this step's dt theta), the native model writes R(Phi)^T B and reads
     * R(Phi)^T C; these modes use B, C unrotated there.  In the state's own
     * frame: the write terms beta B_prev x_prev + gamma B x are rotated by
     * R(Phi) instead of (R(dt theta) on the first, none on the second), and
     * the readout uses R(Phi) C.  theta is used as given. */
    M3_PHASE_NO_WRITE = 4,
    M3_PHASE_NO_READ = 5,
    M3_PHASE_NO_WRITE_READ = 6
} m3_phase_mode;

typedef enum {
    M3_BWD_AUTO = 0,       /* chunked where supported, else step by step */
    M3_BWD_STEP = 1,       /* adjoint recurrence step by step */
    M3_BWD_CHUNKED = 2     /* reverse mode of the chunked form */
} m3_bwd_method;

typedef enum {
    M3_OK = 0,
    M3_ERR_NULL = -1,        /* a required pointer is NULL, or the state record is partial */
    M3_ERR_SHAPE = -2,       /* a negative dimension, zero headdim/dstate/rank, odd dstate */
    M3_ERR_UNSUPPORTED = -3, /* dstate, headdim, rank or chunk outside the compiled set */
    M3_ERR_DTYPE = -4,       /* io_dtype is not an m3_dtype */
    M3_ERR_ALIGN = -5,       /* a pointer is not 16-byte aligned */
    M3_ERR_WORKSPACE = -6,   /* workspace missing or smaller than m3_scan_workspace_bytes */
    M3_ERR_ALIAS = -7,       /* an output overlaps an input it must not overlap */
    M3_ERR_HIP = -8,         /* a HIP call failed; see m3_last_hip_error() */
    M3_ERR_OPTION = -9,      /* an m3_options field or the gradient method is out of range */
    M3_ERR_SCRATCH = -10     /* m3_scan_fwd_noalloc: the call needs more scratch than the library holds */
} m3_status;

/*
 * Options shared by m3_scan_fwd and m3_decode_step, a subset of them also by
 * m3_scan_bwd (all zero = the plain mixer).  Pointers are device pointers
 * owned by the caller.
 *   ngroups      0 = one B and C per head; else a divisor of nheads
 *   A_per_token  0: A is [nheads]; 1: A is [batch, seqlen, nheads] in a scan,
 *                [batch, nheads] in a decode step
 *   phase_mode   an m3_phase_mode; phase_perm ([dstate/2] int32) is required
 *                for M3_PHASE_SHUFFLE and must hold each of 0 .. dstate/2-1
 *                once (entries are clamped into that range, never checked)
 *   premix       1 = apply the pre-mixer; B_norm_w, C_norm_w [dstate] (NULL =
 *                all ones), B_bias, C_bias [nheads, rank, dstate] and dt_bias
 *                [nheads] (NULL = zeros), norm_eps >= 0
 *   cu_seqlens   m3_scan_fwd only (NULL in a decode step): int32 [batch + 1],
 *                nondecreasing from 0 to seqlen; sequence b is tokens
 *                cu_seqlens[b] .. cu_seqlens[b+1]-1 of x, B, C, dt, lam,
 *                theta, y (and of A when it is per token, [seqlen, nheads]).
 *                max_seqlen bounds every sequence's length (it sizes the
 *                launch).  Offsets are clamped into [0, seqlen] and lengths
 *                to max_seqlen on the device: bad entries give wrong
 *                results, never accesses outside the arrays.
 *   phase_in     float32 [batch, nheads, dstate/2] or NULL (zero): the
 *                accumulated rotation angle Phi per (batch row or sequence,
 *                head, pair) before the call's first token -- the sum of
 *                dt theta (after the phase transform and the pre-mixer) over
 *                every earlier token of the sequence, in radians
 *   phase_out    float32 [batch, nheads, dstate/2] or NULL (not written):
 *                receives Phi after the call's last token, reduced into
 *                [-pi, pi).  May be the same array as phase_in (updated in
 *                place); no other overlap.  A scan that writes it needs the
 *                workspace m3_scan_workspace_bytes reports for it.
 */
typedef struct {
    int64_t ngroups;
    int32_t A_per_token;
    int32_t phase_mode;
    const int32_t *phase_perm;
    int32_t premix;
    float norm_eps;
    const float *B_norm_w, *C_norm_w;
    const float *B_bias, *C_bias;
    const float *dt_bias;
    const int32_t *cu_seqlens;
    int64_t max_seqlen;
    const float *phase_in;
    float *phase_out;
} m3_options;

/*
 * Arguments of m3_scan_fwd.
 *
 * Sizes: batch >= 0, seqlen >= 0, nheads >= 0 (a zero batch or head count is a
 * no-op); headdim P, dstate N (even), rank R >= 1.  Supported sets are listed
 * by m3_scan_supported().
 *
 * chunk: chunk length Q of the chunked (SSD) form, or 0 for the library's
 * choice.  Results do not depend on Q beyond float32 rounding.
 * p_split, segments: work decomposition (0 = library's choice).  p_split
 * divides headdim into independent column slices; segments > 1 splits the
 * sequence into that many pieces whose boundary states are combined through a
 * workspace.  Neither changes the result beyond float32 rounding.
 *
 * State record in (h_in, B_prev_in, x_prev_in): all three NULL means a zero
 * state and no previous token; otherwise all three must be given.
 * State record out (h_out, B_prev_out, x_prev_out): all three NULL, or all
 * three given.  They may be exactly the input record (h_out == h_in,
 * B_prev_out == B_prev_in, x_prev_out == x_prev_in: the record is updated in
 * place, as a decode step does -- the fixed-size state that a sequence split
 * into calls carries, "Unlocking Rotational Dynamics via data-RoPE", TL;DR);
 * then the call first copies the input record into its workspace, which
 * m3_scan_workspace_bytes sizes for it.  Any other overlap with an input of
 * the call is rejected.  With seqlen = 0 the record is copied through (or
 * zeroed when no input record is given).
 * y may be NULL only when seqlen * batch * nheads == 0.
 * workspace: device memory of at least m3_scan_workspace_bytes(args) bytes,
 * 256-byte aligned (may be NULL when that size is 0).
 */
typedef struct {
    int64_t batch, seqlen, nheads, headdim, dstate, rank;
    int32_t chunk;
    int32_t io_dtype;                 /* m3_dtype */
    int32_t p_split;                  /* 0 = auto */
    int32_t segments;                 /* 0 = auto */
    const void *x, *B, *C;            /* io dtype */
    const float *dt, *A, *theta, *lam;
    const float *h_in;                /* optional state record in */
    const void *B_prev_in, *x_prev_in;
    void *y;                          /* io dtype */
    float *h_out;                     /* optional state record out */
    void *B_prev_out, *x_prev_out;
    void *workspace;
    size_t workspace_bytes;
    m3_options opt;
} m3_scan_args;

/*
 * Arguments of m3_decode_step: one token for every (batch, head).
 *   x [batch, nheads, rank, headdim], B, C [batch, nheads, rank, dstate] (io dtype)
 *   dt, lam [batch, nheads], theta [batch, nheads, dstate/2], A [nheads] (float32)
 *   h [batch, nheads, dstate, headdim] float32, B_prev, x_prev: the state
 *   record, read and then overwritten in place with (h_t, B_t, X_t).
 *   y [batch, nheads, rank, headdim] (io dtype) receives C_t^T h_t.
 * y must not overlap the state record or the step inputs.
 */
typedef struct {
    int64_t batch, nheads, headdim, dstate, rank;
    int32_t io_dtype;
    int32_t reserved;
    const void *x, *B, *C;
    const float *dt, *A, *theta, *lam;
    float *h;
    void *B_prev, *x_prev;
    void *y;
    m3_options opt;
} m3_decode_args;

/*
 * Arguments of m3_scan_bwd: the gradient of a scan (m3_scan_fwd, with or
 * without the options below) for training.  Given dy = dLoss/dy and optionally dh_out =
 * dLoss/dh_L, it returns the gradients of Loss = sum(dy * y) + sum(dh_out *
 * h_L) with respect to every input, by one of two methods (see below).
 *   inputs   as m3_scan_args: x, B, C (io dtype), dt, A [nheads], theta, lam
 *            (float32), optional state record h_in, B_prev_in, x_prev_in
 *   dy       [batch, seqlen, nheads, rank, headdim] io dtype
 *   dh_out   [batch, nheads, dstate, headdim] float32, or NULL (zero)
 *   dB_prev_out, dx_prev_out  float32 [batch, nheads, rank, dstate] and
 *            [batch, nheads, rank, headdim], or NULL (zero): the gradient
 *            with respect to the output record's (B_L, x_L), e.g. a later
 *            call's dB_prev, dx_prev when a sequence is split into calls.
 *            Added to the last token's gradients (B_L is B as the recurrence
 *            used it: per head, pre-mixed), or, for a sequence without
 *            tokens, to the input record's.
 *   outputs  float32, same shapes as their inputs: dx, dB, dC, ddt, dtheta,
 *            dlam, dA [nheads]; optionally all of dh_in [batch, nheads,
 *            dstate, headdim], dB_prev [batch, nheads, rank, dstate],
 *            dx_prev [batch, nheads, rank, headdim] (gradients with respect to
 *            the input state record, zero record when none was given)
 *   workspace  m3_scan_bwd_workspace_bytes(args) bytes, 256-byte aligned
 *   method   an m3_bwd_method: how the gradient is computed (below)
 * Methods:
 *   M3_BWD_STEP     the adjoint recurrence step by step, backward in time,
 *                   forward states recomputed from checkpoints every few
 *                   steps.  Supported: dstate a multiple of 8 up to 128,
 *                   headdim 16, 32 or 64, rank 1, 2 or 4.
 *   M3_BWD_CHUNKED  the reverse mode of the chunked (SSD) form the prefill
 *                   evaluates: chunk-local sums, a scan of the chunk-boundary
 *                   states forward and of their adjoints backward, then every
 *                   gradient of a chunk from its boundary states on matrix
 *                   cores (64 operand rows per chunk: 64 / rank tokens).
 *                   Supported: dstate 32, 64 or 128 (float32: 32 or 64),
 *                   headdim 32 or 64, rank 1, 2 or 4.
 *   M3_BWD_AUTO     chunked where supported, else step by step.
 * A method that does not support the sizes returns M3_ERR_UNSUPPORTED; any
 * other value returns M3_ERR_OPTION.  The methods agree to rounding.
 * Options (opt, as m3_options for m3_scan_fwd; all zero = the plain mixer):
 *   A_per_token  A and dA are [batch, seqlen, nheads] (dA per token)
 *   ngroups      B, C and dB, dC are [batch, seqlen, ngroups, rank, dstate];
 *                a group's gradient sums those of its heads
 *   phase_mode   M3_PHASE_ZERO, _REVERSE or _SHUFFLE: dtheta is the gradient
 *                with respect to theta as given (zero: theta is not read and
 *                may be NULL, dtheta may be NULL, else it is zero-filled;
 *                shuffle: phase_perm must be a permutation -- entries are
 *                clamped, never checked -- and pair j receives the gradient of
 *                every pair i with phase_perm[i] = j)
 *   premix       dt and lam are the raw projections and ddt, dlam, dB, dC the
 *                gradients with respect to them and to the raw B, C; the
 *                pre-mixer's parameter gradients go to dB_norm_w, dC_norm_w
 *                [dstate], dB_bias, dC_bias [nheads, rank, dstate] and
 *                ddt_bias [nheads], each optional (NULL = not computed; a
 *                NULL parameter is differentiated at its default, ones or
 *                zeros).  The state record (B_prev_in) holds the pre-mixed B,
 *                as m3_scan_fwd writes it, and dB_prev is with respect to it.
 *   cu_seqlens   packed sequences as in m3_scan_fwd: token arrays and their
 *                gradients [seqlen, nheads, ...], one state record, dh_out
 *                and record gradient per sequence; the gradient runs on a
 *                padded batch of max_seqlen tokens per sequence (zero steps
 *                past each end, which leave the state unchanged), so the
 *                workspace grows with batch * max_seqlen
 *   phase_in and phase_out are not supported here (M3_ERR_UNSUPPORTED), nor
 *   the decode-only phase modes (M3_ERR_OPTION).
 * With options, the inputs are first materialised in the workspace as the
 * recurrence uses them, and the gradients are mapped back afterwards.
 * Every output is written (no accumulation into the caller's buffers); the
 * result is deterministic.
 */
typedef struct {
    int64_t batch, seqlen, nheads, headdim, dstate, rank;
    int32_t io_dtype;
    int32_t method;                     /* m3_bwd_method */
    const void *x, *B, *C;
    const float *dt, *A, *theta, *lam;
    const float *h_in;
    const void *B_prev_in, *x_prev_in;
    const void *dy;
    const float *dh_out;
    float *dx, *dB, *dC, *ddt, *dA, *dtheta, *dlam;
    float *dh_in, *dB_prev, *dx_prev;
    void *workspace;
    size_t workspace_bytes;
    m3_options opt;
    float *dB_norm_w, *dC_norm_w, *dB_bias, *dC_bias, *ddt_bias;
    const float *dB_prev_out, *dx_prev_out;
} m3_scan_bwd_args;

/* Chunked prefill: y and (optionally) the state record after the last token.
 * Enqueued on `stream`; returns before the work completes. */
m3_status m3_scan_fwd(const m3_scan_args *args, void *stream);

/* m3_scan_fwd for callers that cannot allocate (code under HIP graph capture,
 * tight serving loops, harnesses that forbid device allocation): the same
 * scan, but every byte of scratch the call needs (the segment records, the
 * accumulated angle's partial sums, the copy of an in-place state record) is
 * taken from one static device array of M3_NOALLOC_SCRATCH_BYTES bytes inside
 * the library instead of a workspace argument; args->workspace and
 * args->workspace_bytes are ignored.  The caller still provides the inputs
 * and outputs.  A call whose m3_scan_workspace_bytes exceeds
 * M3_NOALLOC_SCRATCH_BYTES returns M3_ERR_SCRATCH (checked, like every other
 * argument, before any HIP call).  It calls no allocating routine; each GPU
 * it runs on holds the array until the process ends, and the first call on a
 * device looks its address up there.  `stream` must belong to the current
 * device (else M3_ERR_HIP with hipErrorInvalidDevice).  Every call on one GPU
 * shares that GPU's array: calls that may overlap on one GPU (different
 * streams, or threads) race and must be serialised by the caller.  Nothing in
 * the array needs clearing: every call writes the scratch it reads. */
#define M3_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
m3_status m3_scan_fwd_noalloc(const m3_scan_args *args, void *stream);

/* Workspace bytes that m3_scan_fwd needs for these arguments (0 when the call
 * runs in a single pass).  Depends only on sizes, dtype, chunk, p_split and
 * segments, on whether phase_out is given and on whether the output state
 * record is the input record (in place).  Returns 0 for arguments that
 * m3_scan_fwd would reject. */
size_t m3_scan_workspace_bytes(const m3_scan_args *args);

/* Gradient of a scan.  Enqueued on `stream`; allocates nothing. */
m3_status m3_scan_bwd(const m3_scan_bwd_args *args, void *stream);

/* Workspace bytes m3_scan_bwd needs for these arguments and their method
 * (step by step: states checkpointed every few steps per (batch, head);
 * chunked: the chunk-local sums and the state and adjoint at every chunk
 * boundary); 0 for arguments it would reject. */
size_t m3_scan_bwd_workspace_bytes(const m3_scan_bwd_args *args);

/* 1 when (dstate, headdim, rank, io_dtype) is supported by m3_scan_bwd with
 * some method (M3_BWD_AUTO), else 0. */
int m3_scan_bwd_supported(int64_t dstate, int64_t headdim, int64_t rank, int32_t io_dtype);

/* 1 when m3_scan_bwd supports (dstate, headdim, rank, io_dtype) with the
 * given m3_bwd_method, else 0. */
int m3_scan_bwd_method_supported(int64_t dstate, int64_t headdim, int64_t rank, int32_t io_dtype,
                                 int32_t method);

/* One decode step, state record updated in place.  Enqueued on `stream`. */
m3_status m3_decode_step(const m3_decode_args *args, void *stream);

/* 1 when (dstate, headdim, rank, chunk, io_dtype) is in the compiled set of
 * m3_scan_fwd (chunk 0 = the default chunk), else 0. */
int m3_scan_supported(int64_t dstate, int64_t headdim, int64_t rank, int32_t chunk,
                      int32_t io_dtype);

/* 1 when (dstate, headdim, rank, io_dtype) is supported by m3_decode_step. */
int m3_decode_supported(int64_t dstate, int64_t headdim, int64_t rank, int32_t io_dtype);

/* Static description of a status code.  Never NULL. */
const char *m3_status_string(m3_status status);

/* hipError_t value of the last failed HIP call on this thread (0 if none). */
int m3_last_hip_error(void);

/* M3_ABI_VERSION of the built library. */
int m3_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* M3SCAN_H */
