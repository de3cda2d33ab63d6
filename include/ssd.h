/*
 * ssd.h -- C ABI of libssd: the Mamba-2 SSD (state-space duality) chunked
 * forward pass and the single-token decode state update, as hand-written
 * HIP kernels for gfx950 (MI355X).
 *
 * The operation.  For every batch b and head h, with group g = h / (nheads /
 * ngroups) and a state h_t of shape [headdim x dstate]:
 *
 *     h_t = exp(dt_t * A_h) * h_{t-1} + dt_t * x_t (outer) B_t
 *     y_t = h_t C_t + D_h * x_t
 *
 * (fla `layers/mamba2.py`, `Mamba2.torch_forward`: the decode branch is one
 * step of this recurrence and the naive branch computes the same thing chunk
 * by chunk; burn-mamba `Mamba2SsdInput` rustdoc, `ssd_minimal`, Steps 1-4 and
 * the D skip connection.)  `ssd_chunk_scan_fwd` evaluates it chunk by chunk:
 * intra-chunk outputs (L o C B^T) X, per-chunk states, an inter-chunk
 * state-passing scan and the state-to-output term, following the five
 * kernels of burn-mamba `mamba2/ssd/serial.rs` (`k1_ssd_chunk_cumsum` ..
 * `k5_ssd_chunk_scan`).  `ssd_state_update` is one token of the recurrence
 * applied in place to a cached state (the `selective_state_update` call of
 * the fla layer's decode path).
 *
 * Conventions shared by every entry point:
 *  - All pointers except `stream` are DEVICE pointers to dense row-major
 *    arrays; the library never dereferences them on the host.
 *  - dt is the processed time step (already non-negative: bias, softplus
 *    and any clamp are applied by the caller), except in the `_ex` entry
 *    points, which apply that processing themselves (see ssd_dt_proc).  A is
 *    the per-head decay rate and must be <= 0: the layer stores it as
 *    A = -exp(A_log) (fla Mamba2 page, the mixer's A_log parameter), so every
 *    factor exp(dt A) is a decay in (0, 1].  A > 0 is outside the method; the
 *    forward's factored decays then overflow, and its outputs are undefined
 *    (no error is reported: A stays on the device, unread by the host).
 *  - x, B, C and y share one element type, `io_dtype` (fp32 or bf16).
 *    dt, A, D and every state are fp32.  Accumulation is fp32.
 *  - The caller owns every buffer.  The library allocates no device memory
 *    and is reentrant.  Work is enqueued on `stream` (a hipStream_t; NULL =
 *    the legacy default stream) and nothing synchronises the host: results
 *    are ready when the stream is.  The one state it keeps: a forward on
 *    the fused path that cuts a long sequence of a narrow layer into
 *    segments (see ssd_chunk_scan_fwd), and the gradient pass
 *    (ssd_chunk_scan_bwd, not its _timed form), fork part of their work onto
 *    an auxiliary stream of the library's and join it back to `stream` with
 *    events; that stream and three events are created per device at the
 *    first such call (default priority) and kept until the process ends.
 *  - Errors are reported as status codes, never by exceptions or aborts.
 *    Argument validation happens before anything is enqueued, so a call that
 *    returns SSD_ERR_INVALID_ARGUMENT, SSD_ERR_UNSUPPORTED or
 *    SSD_ERR_WORKSPACE has touched no device memory.  SSD_ERR_HIP means a
 *    launch failed (hipGetLastError); earlier kernels of that call may have
 *    run, so outputs are undefined.  SSD_ERR_NONFINITE comes only from the
 *    opt-in check described below (SSD_CHECK_FINITE).
 *
 * Supported shapes (anything else returns SSD_ERR_UNSUPPORTED):
 *    chunk_len in {16, 32, 64, 128, 256};  headdim a multiple of 16, <= 128;
 *    dstate a multiple of 16, <= 256.
 */
#ifndef LIBSSD_SSD_H
#define LIBSSD_SSD_H

#include <stddef.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SSD_ABI_VERSION 1

typedef enum ssd_status {
    SSD_OK = 0,
    SSD_ERR_INVALID_ARGUMENT = 1, /* NULL required pointer, size <= 0,
                                     nheads % ngroups != 0, unknown dtype   */
    SSD_ERR_UNSUPPORTED = 2,      /* valid but outside the supported shapes */
    SSD_ERR_WORKSPACE = 3,        /* workspace NULL or smaller than needed  */
    SSD_ERR_HIP = 4,              /* a kernel launch failed                 */
    SSD_ERR_NONFINITE = 5         /* opt-in check (SSD_CHECK_FINITE): a NaN
                                     or infinity in an input or an output  */
} ssd_status;

/* The element type of x, B, C, y (and z).  Any other value a caller passes
 * is SSD_ERR_INVALID_ARGUMENT; the two sentinels give the type the range of
 * int, so that every value a C caller can pass is one of its values (a C++
 * implementation may then compare it without undefined behaviour). */
typedef enum ssd_dtype {
    SSD_DTYPE_RANGE_MIN_ = -0x7FFFFFFF - 1,
    SSD_F32 = 0,
    SSD_BF16 = 1,
    SSD_DTYPE_RANGE_MAX_ = 0x7FFFFFFF
} ssd_dtype;

/*
 * The opt-in non-finite check.  burn-mamba's `ssd_serial`
 * (`mamba2/ssd/serial.rs`) guards every intermediate of its five kernels
 * against NaN and infinity (its `san` calls), and the `Mamba2SsdInput`
 * rustdoc gives the input a `sanity()` check; libssd offers the same guard
 * on the values that cross its boundary.  With the environment variable
 * SSD_CHECK_FINITE set to anything but "" or "0", every entry point below
 * (forward, decode, convolution, normalisation) also scans its
 * floating-point inputs before its work and its outputs after it, on
 * `stream`, and returns SSD_ERR_NONFINITE if any value is a NaN or an
 * infinity (exponent bits all ones).  The outputs are still written.  In
 * that mode the call waits for `stream` (it reads the result back), so it
 * cannot be captured in a graph, and checked calls on one device share one
 * result word: they must not run concurrently.  With the variable unset or
 * "0" the call reads it and nothing else changes: no extra kernel runs and
 * nothing synchronises.  The variable is read on every call.
 *
 * A second debug mode, SSD_POISON_WORKSPACE (anything but "" or "0"), makes
 * a forward that uses its workspace (the split path, and the fused path when
 * it cuts the sequence into segments) first fill the whole workspace with
 * quiet NaNs, on `stream`, so that any intermediate read before a kernel of
 * the same call wrote it reaches the outputs (where SSD_CHECK_FINITE, or the
 * caller, sees it).  It adds one fill kernel and nothing else.
 */

/* Version of this ABI (SSD_ABI_VERSION of the built library). */
int ssd_abi_version(void);

/* Static, NUL-terminated description of a status code. */
const char *ssd_status_string(ssd_status status);

/*
 * Bytes of device workspace `ssd_chunk_scan_fwd` needs for this problem,
 * written to *bytes.  The same validation as `ssd_chunk_scan_fwd` is applied
 * (pointers aside); on error *bytes is left unchanged.  The workspace holds
 * the per-chunk intermediates of the chunked algorithm and needs no
 * initialisation.  It depends on the forward path (see
 * ssd_chunk_scan_fwd_timed): the split path keeps the decay prefix sums,
 * the C B^T blocks and every chunk state (batch * nchunks * nheads *
 * headdim * dstate fp32); the fused path keeps every intermediate on chip
 * and needs none (0 bytes), except when it cuts the sequence into segments
 * (below): then it keeps the state each segment but the last leaves,
 * (nsegments - 1) * batch * nheads * headdim * dstate fp32, and their log
 * decays.
 */
ssd_status ssd_chunk_scan_fwd_workspace_size(int batch, int seqlen, int nheads,
                                             int headdim, int dstate,
                                             int ngroups, int chunk_len,
                                             ssd_dtype io_dtype,
                                             size_t *bytes);

/*
 * Chunked SSD forward.
 *
 *   x             [batch, seqlen, nheads, headdim]    io_dtype   in
 *   dt            [batch, seqlen, nheads]             fp32       in
 *   A             [nheads]                            fp32       in
 *   B, C          [batch, seqlen, ngroups, dstate]    io_dtype   in
 *   D             [nheads]                            fp32       in, NULL = 0
 *   initial_state [batch, nheads, headdim, dstate]    fp32       in, NULL = 0
 *   y             [batch, seqlen, nheads, headdim]    io_dtype   out
 *   final_state   [batch, nheads, headdim, dstate]    fp32       out, NULL = skip
 *   workspace     >= ssd_chunk_scan_fwd_workspace_size bytes, 256-byte aligned
 *                 (ignored, and may be NULL, when that size is 0)
 *
 * chunk_len is the chunk length Q of the chunked algorithm; the sequence is
 * processed as ceil(seqlen / Q) chunks and a ragged last chunk behaves as if
 * zero-padded (dt = x = B = C = 0 past seqlen), so the final state is that
 * of token seqlen-1.  y is rounded to io_dtype (round to nearest even for
 * bf16).  final_state may alias initial_state (a cache updated in place);
 * no other buffers may overlap.
 *
 * Sequence segments (fused path).  When the layer has fewer than 128
 * groups of 128 columns (batch * nheads * headdim / 128) and a long enough
 * sequence, the fused forward cuts the sequence into segments so that every
 * compute unit has work: segment 0 runs while a state-only pass forms the
 * state each later segment but the last leaves from zero (on the auxiliary
 * stream, see above), then the other segments run, each from the state
 * entering it, chained from those states (the inter-chunk recurrence of the
 * burn-mamba rustdoc's Step 3, Eq. 22, over segments).  The results differ
 * from a single pass by rounding only.
 */
ssd_status ssd_chunk_scan_fwd(const void *x, const float *dt, const float *A,
                              const void *B, const void *C, const float *D,
                              const float *initial_state, int chunk_len,
                              int ngroups, int batch, int seqlen, int nheads,
                              int headdim, int dstate, ssd_dtype io_dtype,
                              void *y, float *final_state, void *workspace,
                              size_t workspace_bytes, hipStream_t stream);

/*
 * ssd_chunk_scan_fwd for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Same arguments without the workspace; the call itself
 * allocates nothing.  Where the forward path needs a workspace (the split
 * path, see ssd_chunk_scan_fwd_timed) it uses a scratch array of
 * SSD_NOALLOC_SCRATCH_BYTES that the library holds on every GPU it runs on,
 * from the library's load until the process ends; a problem whose workspace
 * (ssd_chunk_scan_fwd_workspace_size) exceeds it returns SSD_ERR_WORKSPACE
 * before anything is enqueued.  Every call on one GPU shares that GPU's
 * array and it keeps the last call's contents (the forward needs none of
 * them: no kernel reads workspace that the same call has not written), so
 * calls that overlap on one GPU, from several streams or host threads, race
 * and must be serialised by the caller.  The first call on a device looks
 * the array's address up once (SSD_ERR_HIP if that fails).
 */
#define SSD_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

ssd_status ssd_chunk_scan_fwd_noalloc(const void *x, const float *dt, const float *A,
                                      const void *B, const void *C, const float *D,
                                      const float *initial_state, int chunk_len,
                                      int ngroups, int batch, int seqlen, int nheads,
                                      int headdim, int dstate, ssd_dtype io_dtype,
                                      void *y, float *final_state, hipStream_t stream);

/*
 * Upper bound on the number of kernels one `ssd_chunk_scan_fwd` call
 * launches (fixed for a library build).
 */
int ssd_chunk_scan_fwd_max_kernels(void);

/*
 * Diagnostic twin of `ssd_chunk_scan_fwd`: identical arguments, identical
 * work and results.  In addition, with k the number of kernels this call
 * launches, events[i] (caller-created hipEvent_t handles) is recorded on
 * `stream` immediately before kernel i for i < k and events[k] right after
 * the last kernel; events[k+1 .. max] are recorded after that, so every
 * handle passed in is recorded.  The caller reads each kernel's GPU time
 * with hipEventElapsedTime.  *nkernels receives k and kernel_names[0..k-1]
 * static kernel names (both may be NULL; kernel_names must have room for
 * ssd_chunk_scan_fwd_max_kernels() entries).  nevents must be at least
 * ssd_chunk_scan_fwd_max_kernels() + 1 with every handle non-NULL, else
 * SSD_ERR_INVALID_ARGUMENT.  A failed event record returns SSD_ERR_HIP.
 *
 * Forward path.  bf16 shapes with dstate 128 and headdim a multiple of 32
 * run the fused path: one kernel that walks the sequence in 32-token
 * blocks with the fp32 state in registers, forms each block's decay
 * prefix sums and diagonal 32x32 block of C B^T on chip, and writes y;
 * inside a chunk it contracts the off-diagonal blocks of L o C B^T through
 * the running state (their rank-dstate factorisation), so its work and
 * result do not depend on chunk_len.  Other shapes run the five-kernel split
 * (k1 .. k5) with the given chunk_len as its chunk size.  The environment variable
 * SSD_FORWARD_PATH=split|fused overrides the choice for diagnostics
 * (forcing "fused" where it does not apply returns SSD_ERR_UNSUPPORTED);
 * the workspace size depends on the path, so query it under the same
 * setting.
 */
ssd_status ssd_chunk_scan_fwd_timed(const void *x, const float *dt, const float *A,
                                    const void *B, const void *C, const float *D,
                                    const float *initial_state, int chunk_len,
                                    int ngroups, int batch, int seqlen, int nheads,
                                    int headdim, int dstate, ssd_dtype io_dtype,
                                    void *y, float *final_state, void *workspace,
                                    size_t workspace_bytes, hipStream_t stream,
                                    hipEvent_t *events, int nevents, int *nkernels,
                                    const char **kernel_names);

/*
 * Gradients of the chunked forward (the recompute-backward path: the pages
 * name it, burn-mamba `Mamba2SsdInput::ssd_serial_recalculated`, and say
 * nothing of its steps; these are the derivative of the four steps of the
 * rustdoc's `ssd_minimal`, Eqs. 20-23, and their sum over a chunk is the
 * reverse-mode loop of the serial recurrence).  For a loss with gradients
 * dy = dLoss/dy and dfinal_state = dLoss/d final_state, it returns the
 * gradients of that loss with respect to every input of ssd_chunk_scan_fwd:
 *
 *   x, dt, A, B, C, D, initial_state, chunk_len ... io_dtype   as for
 *                   ssd_chunk_scan_fwd (no time-step preprocessing, gate or
 *                   packed sequences: dt is the processed time step)
 *   dy            [batch, seqlen, nheads, headdim]    io_dtype   in
 *   dfinal_state  [batch, nheads, headdim, dstate]    fp32       in, NULL = 0
 *   dx            [batch, seqlen, nheads, headdim]    io_dtype   out
 *   ddt           [batch, seqlen, nheads]             fp32       out
 *   dA            [nheads]                            fp32       out
 *   dB, dC        [batch, seqlen, ngroups, dstate]    io_dtype   out (summed
 *                                                                over the group's heads)
 *   dD            [nheads]                            fp32       out, NULL = skip
 *                 (written also when D is NULL: the gradient at D = 0)
 *   dinitial_state [batch, nheads, headdim, dstate]   fp32       out, NULL = skip
 *                 (written also when initial_state is NULL)
 *   workspace     >= ssd_chunk_scan_bwd_workspace_size bytes, 256-byte aligned
 *
 * The call recomputes the forward's prefix sums, C B^T blocks and chunk
 * states (the split path's first four kernels, with this chunk_len), then
 * runs the gradient kernels; nothing from a forward call is needed.  The
 * score tiles and dC run on the library's auxiliary stream of the device
 * (see above), joined back to `stream` before dB.  The outputs must not
 * overlap the inputs or each other.  dA and dD are summed
 * in a fixed order: the results are deterministic.  Accumulation is fp32;
 * bf16 runs round the products' operands to bf16 like the forward.  Errors
 * as for ssd_chunk_scan_fwd (dy and the seven outputs but dD and
 * dinitial_state are required); SSD_CHECK_FINITE and SSD_POISON_WORKSPACE
 * apply.
 */
ssd_status ssd_chunk_scan_bwd_workspace_size(int batch, int seqlen, int nheads,
                                             int headdim, int dstate, int ngroups,
                                             int chunk_len, ssd_dtype io_dtype,
                                             size_t *bytes);

ssd_status ssd_chunk_scan_bwd(const void *x, const float *dt, const float *A,
                              const void *B, const void *C, const float *D,
                              const float *initial_state, const void *dy,
                              const float *dfinal_state, int chunk_len, int ngroups,
                              int batch, int seqlen, int nheads, int headdim,
                              int dstate, ssd_dtype io_dtype, void *dx, float *ddt,
                              float *dA, void *dB, void *dC, float *dD,
                              float *dinitial_state, void *workspace,
                              size_t workspace_bytes, hipStream_t stream);

/* Number of timed kernel groups of one ssd_chunk_scan_bwd call. */
int ssd_chunk_scan_bwd_max_kernels(void);

/*
 * Diagnostic twin of ssd_chunk_scan_bwd with per-kernel events, as
 * ssd_chunk_scan_fwd_timed: events[i] is recorded before kernel group i and
 * events[k] after the last (k = ssd_chunk_scan_bwd_max_kernels(); the first
 * group is the four recompute kernels).  nevents >= k + 1, every handle
 * non-NULL.
 */
ssd_status ssd_chunk_scan_bwd_timed(const void *x, const float *dt, const float *A,
                                    const void *B, const void *C, const float *D,
                                    const float *initial_state, const void *dy,
                                    const float *dfinal_state, int chunk_len, int ngroups,
                                    int batch, int seqlen, int nheads, int headdim,
                                    int dstate, ssd_dtype io_dtype, void *dx, float *ddt,
                                    float *dA, void *dB, void *dC, float *dD,
                                    float *dinitial_state, void *workspace,
                                    size_t workspace_bytes, hipStream_t stream,
                                    hipEvent_t *events, int nevents, int *nkernels,
                                    const char **kernel_names);

/*
 * One decode step, in place.
 *
 *   state  [batch, nheads, headdim, dstate]  fp32      in/out
 *   x      [batch, nheads, headdim]          io_dtype  in
 *   dt     [batch, nheads]                   fp32      in
 *   A      [nheads]                          fp32      in
 *   B, C   [batch, ngroups, dstate]          io_dtype  in
 *   D      [nheads]                          fp32      in, NULL = 0
 *   y      [batch, nheads, headdim]          io_dtype  out
 *
 * state <- exp(dt A) state + dt x (outer) B, then y = state C + D x, read from
 * the UPDATED state (the order of the fla decode branch).  y must not
 * overlap state.  No workspace is needed.
 */
ssd_status ssd_state_update(float *state, const void *x, const float *dt,
                            const float *A, const void *B, const void *C,
                            const float *D, int ngroups, int batch, int nheads,
                            int headdim, int dstate, ssd_dtype io_dtype,
                            void *y, hipStream_t stream);

/*
 * Time-step preprocessing inside the kernels.  The Mamba-2 layer does not
 * feed its projected time step to the recurrence directly: it passes
 * `dt_bias`, `dt_softplus` and `dt_limit` to `mamba_chunk_scan_combined`
 * and `selective_state_update`, and its reference branches compute
 * dt = clamp(softplus(dt + dt_bias), time_step_limit) (fla
 * `layers/mamba2.py`, `Mamba2.forward` and `Mamba2.torch_forward`).  With
 * this struct the library does the same, per element of dt, in fp32:
 *
 *     dt_used = min(max(f(dt + dt_bias_h), dt_min), dt_max)
 *     f(v)    = log(1 + e^v) when dt_softplus != 0 (v itself above 20),
 *               else v
 *
 *   dt_bias      [nheads] fp32 device pointer, 4-byte aligned; NULL = 0
 *   dt_softplus  0 or nonzero
 *   dt_min       lower bound, >= 0 (so dt_used >= 0); the layer's default 0
 *   dt_max       upper bound, >= dt_min; +INFINITY for none (the default)
 *
 * Tokens past seqlen (the ragged last chunk) keep dt_used = 0, as in the
 * entry points without preprocessing.  Any bound that is NaN, dt_min < 0 or
 * dt_min > dt_max returns SSD_ERR_INVALID_ARGUMENT.
 */
typedef struct ssd_dt_proc {
    const float *dt_bias;
    int dt_softplus;
    float dt_min;
    float dt_max;
} ssd_dt_proc;

/*
 * ssd_chunk_scan_fwd with dt the raw time step [batch, seqlen, nheads],
 * processed as *dt_proc says.  A NULL dt_proc makes it exactly
 * ssd_chunk_scan_fwd.  Same arguments, workspace (size and path) and errors
 * otherwise.
 */
ssd_status ssd_chunk_scan_fwd_ex(const void *x, const float *dt, const float *A,
                                 const void *B, const void *C, const float *D,
                                 const float *initial_state, int chunk_len,
                                 int ngroups, int batch, int seqlen, int nheads,
                                 int headdim, int dstate, ssd_dtype io_dtype,
                                 void *y, float *final_state, void *workspace,
                                 size_t workspace_bytes, hipStream_t stream,
                                 const ssd_dt_proc *dt_proc);

/*
 * Packed variable-length sequences: each batch row holds several sequences
 * one after the other, told apart by seq_idx [batch, seqlen] (int32 device
 * pointer, 4-byte aligned), the `seq_idx` argument of the pages'
 * `mamba_chunk_scan_combined`.  Token t > 0 whose seq_idx differs from token
 * t-1's starts a new sequence: the state entering it is zero, so no output
 * or state depends on an earlier sequence.  initial_state enters the row's
 * first sequence; final_state is that of the row's last token.  Otherwise
 * as ssd_chunk_scan_fwd_ex (dt_proc may be NULL).  Both forward paths take
 * it, every io type and supported shape; the workspace is the same as for
 * ssd_chunk_scan_fwd.  A NULL or misaligned seq_idx is
 * SSD_ERR_INVALID_ARGUMENT.
 */
ssd_status ssd_chunk_scan_fwd_varlen(const void *x, const float *dt, const float *A,
                                     const void *B, const void *C, const float *D,
                                     const float *initial_state, int chunk_len, int ngroups,
                                     int batch, int seqlen, int nheads, int headdim,
                                     int dstate, ssd_dtype io_dtype, void *y,
                                     float *final_state, void *workspace,
                                     size_t workspace_bytes, hipStream_t stream,
                                     const int *seq_idx, const ssd_dt_proc *dt_proc);

/*
 * The output gate and the shape of the skip term.  The pages' scan and
 * decode kernels take `D` and `z` (`mamba_chunk_scan_combined(x, dt, A, B,
 * C, chunk_size, D, z, seq_idx, ...)`, `selective_state_update(state, x, dt,
 * A, B, C, D, z, dt_bias, dt_softplus)` in fla `layers/mamba2.py`), and the
 * lrnnx scan spells out what they do to the output (`selective_scan_ref`,
 * "Final Output Processing"): the skip term is added, then the sum is
 * multiplied by SiLU of the gate,
 *
 *     y_t = (h_t C_t + D (*) x_t) * silu(z_t),    silu(v) = v / (1 + e^-v),
 *
 * per element, with D either one value per head or one per head and
 * headdim column (the fla decode branch passes D expanded to [nheads,
 * headdim]).
 *
 *   z              like x: [batch, seqlen, nheads, headdim] for the forward,
 *                  [batch, nheads, headdim] for the decode step; io_dtype,
 *                  aligned like x (16 bytes for the forward); NULL = no gate
 *   D_per_channel  0: D is [nheads] (as in the plain calls); nonzero: D is
 *                  [nheads, headdim] fp32 (ignored when D is NULL)
 *
 * The state and final_state are not gated.  A misaligned z returns
 * SSD_ERR_INVALID_ARGUMENT.
 */
typedef struct ssd_gate {
    const void *z;
    int D_per_channel;
} ssd_gate;

/*
 * The forward with every optional argument of the pages' scan call: packed
 * sequences (seq_idx, as ssd_chunk_scan_fwd_varlen; NULL = one sequence per
 * row), the time-step preprocessing (dt_proc, as ssd_chunk_scan_fwd_ex; NULL =
 * dt as given) and the gate and per-channel D (gate; NULL = neither).  With
 * all three NULL it is ssd_chunk_scan_fwd.  Both forward paths take all
 * three.
 */
ssd_status ssd_chunk_scan_fwd_full(const void *x, const float *dt, const float *A,
                                   const void *B, const void *C, const float *D,
                                   const float *initial_state, int chunk_len, int ngroups,
                                   int batch, int seqlen, int nheads, int headdim,
                                   int dstate, ssd_dtype io_dtype, void *y,
                                   float *final_state, void *workspace,
                                   size_t workspace_bytes, hipStream_t stream,
                                   const int *seq_idx, const ssd_dt_proc *dt_proc,
                                   const ssd_gate *gate);

/*
 * The decode step with every optional argument of the pages' decode call:
 * the time-step preprocessing (dt_proc) and the gate and per-channel D
 * (gate), both nullable.  With both NULL it is ssd_state_update.  y is the
 * gated output; the state is updated as in ssd_state_update.
 */
ssd_status ssd_state_update_full(float *state, const void *x, const float *dt,
                                 const float *A, const void *B, const void *C,
                                 const float *D, int ngroups, int batch, int nheads,
                                 int headdim, int dstate, ssd_dtype io_dtype,
                                 void *y, hipStream_t stream,
                                 const ssd_dt_proc *dt_proc, const ssd_gate *gate);

/*
 * ssd_state_update with dt the raw time step [batch, nheads], processed as
 * *dt_proc says (the `dt_bias` and `dt_softplus` arguments of the layer's
 * `selective_state_update` call).  A NULL dt_proc makes it exactly
 * ssd_state_update.
 */
ssd_status ssd_state_update_ex(float *state, const void *x, const float *dt,
                               const float *A, const void *B, const void *C,
                               const float *D, int ngroups, int batch, int nheads,
                               int headdim, int dstate, ssd_dtype io_dtype,
                               void *y, hipStream_t stream,
                               const ssd_dt_proc *dt_proc);

/*
 * The causal depthwise convolution that precedes the scan in the Mamba-2
 * layer (fla `layers/mamba2.py`, `Mamba2.torch_forward`: the x | B | C
 * channels go through `nn.Conv1d(conv_dim, conv_dim, kernel_size=width,
 * groups=conv_dim, padding=width-1)`, truncated to the first seqlen outputs,
 * then SiLU).  Per channel c, with x_t = 0 for t < 0:
 *
 *     out_t[c] = act(bias[c] + sum_{k<width} weight[c][k] * x_{t-width+1+k}[c])
 *
 * act is the identity (SSD_ACT_NONE) or SiLU, v / (1 + e^-v) (SSD_ACT_SILU).
 */
typedef enum ssd_activation {
    SSD_ACT_NONE = 0,
    SSD_ACT_SILU = 1
} ssd_activation;

/*
 * Convolution over a sequence, starting from an empty (zero) cache.
 *
 *   x           [batch, seqlen, dim]    io_dtype   in, 16-byte aligned
 *   weight      [dim, width]            fp32       in (the conv1d weight with
 *                                                  its singleton axis dropped)
 *   bias        [dim]                   fp32       in, NULL = 0
 *   out         [batch, seqlen, dim]    io_dtype   out, 16-byte aligned; may
 *                                                  not overlap x
 *   conv_state  [batch, dim, width]     io_dtype   out, NULL = skip: the cache
 *               the decode path continues from, the last `width` inputs of
 *               every channel, zeros before the first token (the layer's
 *               cache initialisation, a left pad of the transposed inputs)
 *
 * width is 2, 3 or 4 and dim a multiple of 8 (else SSD_ERR_UNSUPPORTED).
 * Accumulation is fp32; out is rounded to io_dtype.
 */
ssd_status ssd_causal_conv1d_fwd(const void *x, const float *weight, const float *bias,
                                 int batch, int seqlen, int dim, int width, int activation,
                                 ssd_dtype io_dtype, void *out, void *conv_state,
                                 hipStream_t stream);

/*
 * One decode token, the cache updated in place (the layer's single-token
 * branch: `update_conv_state` rolls the cache left by one and appends the
 * new input; the output is the same dot product, bias and activation).
 *
 *   conv_state  [batch, dim, width]  io_dtype  in/out
 *   x           [batch, dim]         io_dtype  in
 *   weight, bias                     as above
 *   out         [batch, dim]         io_dtype  out, may not overlap the cache
 */
ssd_status ssd_causal_conv1d_update(void *conv_state, const void *x, const float *weight,
                                    const float *bias, int batch, int dim, int width,
                                    int activation, ssd_dtype io_dtype, void *out,
                                    hipStream_t stream);

/*
 * The gated RMS normalisation that follows the scan in the Mamba-2 layer
 * (fla `layers/mamba2.py`: `RMSNormGated(intermediate_size, eps=norm_eps,
 * norm_before_gate=False)`, applied as `norm(y, gate)` to the scan output).
 * Per row of dim values, with silu(v) = v / (1 + e^-v):
 *
 *   norm_before_gate == 0 (the layer's):  g = y * silu(z),
 *                                        out = g / sqrt(mean(g^2) + eps) * weight
 *   norm_before_gate != 0:               out = y / sqrt(mean(y^2) + eps) * weight * silu(z)
 *   z == NULL:                           out = y / sqrt(mean(y^2) + eps) * weight
 *
 * The mean runs over the whole row (the module as the layer builds it has
 * no group size).
 *
 *   y, z    [rows, dim]  io_dtype  in, 16-byte aligned (z may be NULL)
 *   weight  [dim]        fp32      in, 16-byte aligned
 *   out     [rows, dim]  io_dtype  out, 16-byte aligned; may alias y
 *   eps     >= 0 (the layer's norm_eps, 1e-5 by default)
 *
 * dim must be a multiple of 8 and at most 8192 (else SSD_ERR_UNSUPPORTED).
 * Sums and scaling are fp32; out is rounded to io_dtype.
 */
ssd_status ssd_gated_rmsnorm_fwd(const void *y, const void *z, const float *weight, int rows,
                                 int dim, float eps, int norm_before_gate, ssd_dtype io_dtype,
                                 void *out, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* LIBSSD_SSD_H */
