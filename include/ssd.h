/*
 * ssd.h -- C ABI of libssd.so, the gfx950 (MI355X) Mamba-2 SSD mixer core.
 *
 * Nine operations, each a few HIP kernel launches on the caller's stream:
 *
 *   ssd_conv_fwd        causal depthwise conv (k = 4) + SiLU over the
 *                       [x | B | C] columns, and dt = softplus(dt_raw + dt_bias)
 *   ssd_chunk_scan_fwd  the SSD selective scan in chunks of 64 tokens, with
 *                       B/C groups, document resets, initial/final state, the
 *                       D skip and the y * silu(z) gate
 *   ssd_mixer_fwd       both of the above in one pass: the scan reads the raw
 *                       columns and convolves each chunk on chip
 *   ssd_resume_fwd      decode tokens appended to the working chunk and
 *                       rescanned with the forward kernels: bit-identical to
 *                       the forward
 *   ssd_step            one decode token per sequence: conv from a rolling
 *                       buffer, state update, output and gate
 *   ssd_s6_scan_fwd     the Mamba-1 selective scan (S6): a per-channel
 *                       diagonal state, B and C shared by the channels
 *   ssd_chunk_scan_bwd  backward (VJP) of the scan for a zero-state prefill
 *   ssd_conv_bwd        backward of the conv prologue
 *   ssd_mixer_bwd       backward of conv + scan, recomputing the forward
 *
 * The operation (per batch row b and head h, token t, head h in group
 * g = h / (H/G)):
 *     a_t = exp(dt_t * A_h)
 *     h_t = a_t * h_{t-1} + dt_t * B_t x_t^T            (h_t is N x P)
 *     y_t = (C_t^T h_t + D_h * x_t) * silu(z_t)          (h_t after token t)
 * is the Mamba-2 SSD layer whose tensors the Codestral-Mamba weight port
 * lists (builderforce-memory-engine diff, codestral_mamba.ts header: in_proj
 * rows [z | x | B | C | dt], conv1d weight [conv_dim, 1, d_conv] with
 * conv_dim = d_inner + 2*n_groups*d_state, per-head A_log, D and dt_bias,
 * A = -exp(A_log), gate norm(y * silu(z))), in the mixer shape of the
 * Mini-K3-1H-mamba2-n64-g8 card ("Architecture": 32 heads x 64 channels,
 * state 64, 8 B/C groups, conv kernel 4).  dt_bias goes inside the softplus
 * (falcon_mamba.ts header).  Document ids reset both the conv history and
 * the recurrent state (Mini-K3-1H card, "Checkpoint and training").  State
 * is caller-owned, read at entry and written at exit, and a step is the
 * forward at length 1 with the state carried (mojolearn.Mamba3Block docs,
 * forward() and step()).  Chunk size 64 follows the same mojolearn page.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - All pointers are DEVICE pointers, allocated and owned by the caller,
 *   and must stay valid until the work queued on `stream` has finished.
 *   The library allocates nothing, frees nothing, keeps no pointer and
 *   never synchronises.  `stream` is a hipStream_t (NULL = default stream).
 * - Activation tensors are [B][L][row] with rows `*_row_stride` ELEMENTS
 *   apart (stride >= row width) and batch rows L * stride elements apart.
 *   The innermost dimension is contiguous.
 * - dtype (ssd_dtype_t) is the storage type of the activation tensors
 *   marked "T".  Parameters (conv_w, conv_b, dt_bias, A, D), dt after the
 *   prologue, y and the SSM state are always fp32.  Other dtypes are
 *   refused by name, never converted.
 * - Column layouts: x and z are head-major [h][p] (H*P wide); B and C are
 *   group-major [g][n] (G*N wide); the conv tensors are [x | B | C]
 *   (conv_dim = H*P + 2*G*N wide).  The SSM state is [B][H][P][N] with n
 *   fastest (entry (p, n) holds h[n][p] of the equations).  The conv state
 *   is [B][K-1][conv_dim]: the last K-1 raw input rows, oldest first.
 * - Document ids (int32 [B][L], optional): a new document starts at t > 0
 *   exactly where doc[b][t] != doc[b][t-1].  t = 0 always continues the
 *   carried state; a caller starting a fresh document passes NULL (zero)
 *   states for it.
 * - Supported sizes: P = 64, N in {16, 32, 64, 128}, K = 4, chunk = 64,
 *   G divides H, B >= 1, 0 <= L <= 2^30 = 1073741824 tokens per row (L = 0
 *   is a no-op apart from copying the states through; a partial last chunk
 *   is handled; a larger L is refused with SSD_ERR_BAD_SHAPE), and one batch
 *   row of the widest activation -- L * max(conv_dim * sizeof(T),
 *   H * P * 4) bytes -- below 2^31 bytes (refused with SSD_ERR_BAD_SHAPE).
 * - Alignment: every tensor base must be 16-byte aligned, and row strides
 *   of T tensors must be multiples of 16 bytes (8 bf16 or 4 fp32 elements).
 * - Errors: arguments are validated on the host before anything is
 *   launched and device memory is never touched on failure.  The return
 *   value is an ssd_status_t; ssd_last_error() gives a message naming the
 *   argument and its value(s) (thread-local, valid until the next call on
 *   that thread).  A failed launch returns SSD_ERR_HIP with the HIP error
 *   string.  Inputs are not scanned for NaN/Inf.
 */
#ifndef SSD_H
#define SSD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SSD_ABI_VERSION 2

typedef enum { SSD_F32 = 0, SSD_BF16 = 1 } ssd_dtype_t;

/* Activation after the depthwise conv: SiLU (the Mamba-2 default) or none. */
typedef enum { SSD_ACT_SILU = 0, SSD_ACT_NONE = 1 } ssd_act_t;

typedef enum {
    SSD_OK = 0,
    SSD_ERR_NULL_ARG = 1,     /* a required pointer is NULL                  */
    SSD_ERR_BAD_SHAPE = 2,    /* negative/zero size, H % G != 0, stride < row */
    SSD_ERR_UNSUPPORTED = 3,  /* P, N, K, chunk or dtype outside the set above */
    SSD_ERR_ALIGNMENT = 4,    /* base pointer or row stride breaks 16 B loads */
    SSD_ERR_WORKSPACE = 5,    /* workspace smaller than the size query says  */
    SSD_ERR_HIP = 6           /* the kernel launch failed                     */
} ssd_status_t;

/* Message of the last failing call on this thread ("" after a success). */
const char *ssd_last_error(void);
/* Name of a status code ("SSD_OK", "SSD_ERR_BAD_SHAPE", ...). */
const char *ssd_status_string(int status);
/* SSD_ABI_VERSION of the loaded library. */
int ssd_version(void);

/*
 * ssd_conv_fwd -- causal depthwise conv + activation, and the dt prologue.
 *
 *   xbc_out[b,t,c] = act(conv_b[c] + sum_{k<K} conv_w[c][k] * src(b, t-K+1+k, c))
 *   dt_out[b,t,h]  = softplus(dt_raw[b,t,h] + dt_bias[h])
 *
 * src(b, tau, c) is xbc_raw[b,tau,c] if tau >= 0 and tau lies in t's
 * document; conv_state_in[b][K-1+tau][c] if tau < 0 and t is still in the
 * row's first document; else 0.  conv_w[c][K-1] multiplies the current
 * token (the port pages store the upstream [conv_dim,1,d_conv] weight with
 * the tap axis reversed; this is the un-reversed, upstream order).
 *
 *   xbc_raw        T  [B][L][conv_dim], row stride xbc_raw_row_stride
 *   conv_w         f32 [conv_dim][K]
 *   conv_b         f32 [conv_dim] or NULL (zero bias)
 *   dt_raw         T  [B][L][H], row stride dt_raw_row_stride, or NULL (no dt output)
 *   dt_bias        f32 [H] or NULL (zero)
 *   doc_ids        i32 [B][L] or NULL (one document per row)
 *   conv_state_in  T  [B][K-1][conv_dim] or NULL (zero history)
 *   conv_state_out T  [B][K-1][conv_dim] or NULL; may equal conv_state_in
 *                  (in place).  Holds the K-1 raw rows the next call's first
 *                  token reads, judged from the last token's document.
 *   act            ssd_act_t
 *   xbc_out        T  [B][L][conv_dim], row stride xbc_out_row_stride; must not
 *                  overlap xbc_raw (the halo rows are re-read)
 *   dt_out         f32 [B][L][H] contiguous; required iff dt_raw != NULL
 * Values are computed in fp32 and rounded to T (round to nearest even).
 */
int ssd_conv_fwd(int B, int L, int H, int P, int N, int G, int K, int dtype,
                 const void *xbc_raw, int64_t xbc_raw_row_stride,
                 const float *conv_w, const float *conv_b,
                 const void *dt_raw, int64_t dt_raw_row_stride,
                 const float *dt_bias, const int32_t *doc_ids,
                 const void *conv_state_in, void *conv_state_out, int act,
                 void *xbc_out, int64_t xbc_out_row_stride, float *dt_out,
                 void *stream);

/*
 * ssd_chunk_scan_fwd -- the SSD selective scan, chunk = 64.
 *
 * Computes y (and the final state) of the recurrence above for every
 * (b, h).  Inside a chunk the dual (quadratic) form is used.
 *
 * Without a workspace (NULL, 0) chunk states are passed strictly in chunk
 * order with the state kept on chip in fp32, so a prefill split at a
 * multiple of 64 tokens with the state carried is bitwise identical to one
 * call.  With a workspace of ssd_chunk_scan_workspace_size() bytes the
 * sequence may additionally be cut into superchunks scanned in parallel:
 * a first pass stores each superchunk's local end state (scanned from a zero
 * state) and total decay in the workspace, and the main pass folds the
 * preceding superchunks' states into its starting state, in order, exactly
 * as chunk states are passed between chunks.  Results then agree with the
 * sequential pass to fp32 rounding, not bitwise.  The first pass also copies
 * init_state into the workspace and the main pass reads only that copy, so
 * final_state may alias init_state on either path.
 *
 *   x       T   [B][L][H*P]  row stride x_row_stride
 *   Bm, Cm  T   [B][L][G*N]  row strides B_row_stride, C_row_stride
 *               (x, Bm, Cm may be column slices of one ssd_conv_fwd output)
 *   dt      f32 [B][L][H]    row stride dt_row_stride; dt_softplus = 0: dt is
 *               already activated (>= 0); 1: dt := softplus(dt + dt_bias)
 *   dt_bias f32 [H] or NULL (only read when dt_softplus = 1)
 *   A       f32 [H], A <= 0 (the caller computes A = -exp(A_log))
 *   D       f32 [H] or NULL (no skip)
 *   z       T   [B][L][H*P] row stride z_row_stride, or NULL (no gate)
 *   doc_ids i32 [B][L] or NULL
 *   lengths i32 [B] or NULL: a ragged batch (mojolearn.Mamba3Block docs,
 *               forward(): row b is real at positions t < lengths[b]).  Every
 *               output at t >= lengths[b] is exactly +0.0; real positions are
 *               causal and equal the row run alone at its own length
 *               (bitwise without a workspace).  Values are read on the
 *               device and clamped to [0, L]; padding inputs must be finite.
 *               Not allowed with init_state / final_state (SSD_ERR_BAD_SHAPE).
 *   init_state  f32 [B][H][P][N] or NULL (zero)
 *   final_state f32 [B][H][P][N] or NULL; may equal init_state (in place)
 *   y       f32 [B][L][H*P]  row stride y_row_stride; must not overlap inputs
 *   workspace, workspace_bytes: NULL, 0 (sequential pass) or device scratch
 *               of at least ssd_chunk_scan_workspace_size() bytes, 16-byte
 *               aligned, owned by the caller and not read before it is
 *               written; SSD_ERR_WORKSPACE if too small or misaligned.
 *               Concurrent calls must not share one workspace.
 * Row strides are in elements, >= the row width and <= 4194304.
 */
int ssd_chunk_scan_fwd(int B, int L, int H, int P, int N, int G, int chunk, int dtype,
                       const void *x, int64_t x_row_stride,
                       const void *Bm, int64_t B_row_stride,
                       const void *Cm, int64_t C_row_stride,
                       const float *dt, int64_t dt_row_stride,
                       int dt_softplus, const float *dt_bias,
                       const float *A, const float *D,
                       const void *z, int64_t z_row_stride,
                       const int32_t *doc_ids, const int32_t *lengths,
                       const float *init_state, float *final_state,
                       float *y, int64_t y_row_stride,
                       void *workspace, size_t workspace_bytes, void *stream);

/* Bytes of workspace that let ssd_chunk_scan_fwd split the sequence for
 * these sizes; 0 when no split pays (then the workspace is ignored). */
size_t ssd_chunk_scan_workspace_size(int B, int L, int H, int P, int N, int G, int dtype);

/* Size of the library's static scratch buffer (per GPU) used by
 * ssd_chunk_scan_fwd_static. */
#define SSD_STATIC_SCRATCH_BYTES ((size_t)32 << 20)

/*
 * ssd_chunk_scan_fwd_static -- ssd_chunk_scan_fwd for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).
 *
 * Arguments and results are those of ssd_chunk_scan_fwd called with a
 * workspace of ssd_chunk_scan_workspace_size() bytes (bit for bit the same
 * outputs), except that the workspace is a file-scope device array of the
 * library, SSD_STATIC_SCRATCH_BYTES bytes, one per GPU, held until the
 * process ends.  The call allocates nothing: no hipMalloc, hipFree or
 * allocating library routine.  Sizes whose workspace exceeds the static
 * buffer are refused with SSD_ERR_WORKSPACE before any launch (the call
 * without a workspace, ssd_chunk_scan_fwd(..., NULL, 0, stream), needs
 * none).  Every call on one GPU shares that GPU's buffer and leaves its
 * contents behind (nothing in it needs to start at zero): calls that may
 * overlap in time on one GPU -- on different streams, or from different
 * threads -- race and must be ordered by the caller.
 */
int ssd_chunk_scan_fwd_static(int B, int L, int H, int P, int N, int G, int chunk, int dtype,
                              const void *x, int64_t x_row_stride,
                              const void *Bm, int64_t B_row_stride,
                              const void *Cm, int64_t C_row_stride,
                              const float *dt, int64_t dt_row_stride,
                              int dt_softplus, const float *dt_bias,
                              const float *A, const float *D,
                              const void *z, int64_t z_row_stride,
                              const int32_t *doc_ids, const int32_t *lengths,
                              const float *init_state, float *final_state,
                              float *y, int64_t y_row_stride, void *stream);

/*
 * ssd_mixer_fwd -- the conv prologue and the scan in one pass.
 *
 * Computes what ssd_conv_fwd followed by ssd_chunk_scan_fwd computes -- the
 * conv (k = 4) + act over the raw [x | B | C] columns, dt = softplus(dt_raw +
 * dt_bias), the scan with groups, documents and states, the D skip and the
 * gate (the Codestral-Mamba port header for the in_proj row layout and the
 * conv weight).  Two plans, chosen by the workspace size:
 *   staged  workspace_bytes >= ssd_mixer_workspace_size(): the conv kernel
 *           writes the convolved columns and dt into the workspace and the
 *           scan reads them, with the sequence split (the faster plan).
 *   fused   a smaller workspace, or NULL (bf16 only): the scan kernels read
 *           the raw tiles and convolve each chunk in LDS with the conv
 *           kernel's fp32 arithmetic, so the convolved columns never reach
 *           memory; the split is used when the workspace holds
 *           ssd_chunk_scan_workspace_size() bytes.  It needs no staging
 *           buffer but is slower on MI355X: the conv's SiLU arithmetic then
 *           runs inside the scan kernels at one workgroup per CU.
 * Either way y, final_state and conv_state_out are bit-identical to the
 * two-call composition (ssd_chunk_scan_fwd with dt_softplus = 0 on
 * ssd_conv_fwd's outputs) with the same split choice.
 *
 *   xbc_raw      T  [B][L][conv_dim], row stride xbc_raw_row_stride
 *   conv_w       f32 [conv_dim][K], conv_b f32 [conv_dim] or NULL; act as in
 *                ssd_conv_fwd
 *   dt_raw       T  [B][L][H], row stride dt_raw_row_stride (even for bf16:
 *                read in 4-byte words; base 4-byte aligned)
 *   dt_bias      f32 [H] or NULL; A, D, z, doc_ids, lengths, init_state,
 *                final_state and y as in ssd_chunk_scan_fwd (final_state may
 *                equal init_state; lengths excludes every carried state,
 *                the conv states included)
 *   conv_state_in, conv_state_out  T [B][K-1][conv_dim] or NULL, as in
 *                ssd_conv_fwd, except that they must not overlap
 *                (SSD_ERR_BAD_SHAPE): several workgroups read the incoming
 *                B/C history while another writes the outgoing one
 *   workspace    device scratch selecting the plan (above); fp32 requires
 *                the staged plan (SSD_ERR_WORKSPACE otherwise).  16-byte
 *                aligned, owned by the caller, not read before it is
 *                written, not shared by concurrent calls.
 * Row strides are in elements, >= the row width and <= 4194304.  L = 0
 * copies both carried states through.
 */
int ssd_mixer_fwd(int B, int L, int H, int P, int N, int G, int K, int chunk, int dtype,
                  const void *xbc_raw, int64_t xbc_raw_row_stride,
                  const float *conv_w, const float *conv_b,
                  const void *dt_raw, int64_t dt_raw_row_stride, const float *dt_bias,
                  const float *A, const float *D,
                  const void *z, int64_t z_row_stride,
                  const int32_t *doc_ids, const int32_t *lengths,
                  const void *conv_state_in, void *conv_state_out,
                  const float *init_state, float *final_state,
                  int act, float *y, int64_t y_row_stride,
                  void *workspace, size_t workspace_bytes, void *stream);

/* Bytes of workspace of ssd_mixer_fwd's staged plan for these sizes: the
 * conv output [B][L][conv_dim] (T) and dt [B][L][H] (fp32), each padded to
 * 256 bytes, plus the scan's split state (ssd_chunk_scan_workspace_size()). */
size_t ssd_mixer_workspace_size(int B, int L, int H, int P, int N, int G, int dtype);

/*
 * ssd_resume_fwd -- append n tokens to each sequence's working chunk and
 * return their outputs exactly as the sequential forward computes them.
 *
 * The working chunk is the tokens after a sequence's last multiple of 64
 * (pos of them, the same for every sequence).  Decoding resumes it (the
 * mojolearn.Mamba3Block step() description: decoding resumes the working
 * chunk, so step and forward continue a prefill bit for bit): the new tokens
 * are convolved by the conv kernel into rows pos .. pos+n-1 of the working
 * chunk, and the scan kernel reruns the chunk's rows 0 .. pos+n-1 from the
 * state at the chunk's start.  A token's output depends only on the chunk's
 * rows up to it, so y is bit-identical (up to the sign of zero) to
 * ssd_conv_fwd + ssd_chunk_scan_fwd without a workspace over the whole
 * sequence, and so is the state each time a chunk completes.  A step costs a
 * rerun of the working chunk; ssd_step is the cheaper recurrent step.
 *
 *   pos, n       0 <= pos <= 63, n >= 1, pos + n <= 64
 *   xbc_raw      T [B][n][conv_dim], dt_raw T [B][n][H], z T [B][n][H*P] or
 *                NULL, all contiguous: the new tokens' raw inputs
 *   conv_w, conv_b, dt_bias, A, D, act   as in ssd_conv_fwd / ssd_chunk_scan_fwd
 *   conv_state   T [B][K-1][conv_dim], read and advanced in place
 *   chunk_xbc    T [B][64][conv_dim], chunk_dt f32 [B][64][H], chunk_z T
 *                [B][64][H*P] (given iff z is): the working chunk's
 *                convolved rows, dt and gate rows; rows < pos as earlier
 *                calls left them, rows pos .. pos+n-1 written
 *   chunk_state  f32 [B][H][P][N]: the SSM state at the working chunk's
 *                start; when pos + n = 64 it becomes the state at its end
 *                (the next chunk's start, pos = 0)
 *   chunk_y      f32 [B][64][H*P] scratch
 *   y            f32 [B][n][H*P]: the new tokens' outputs
 * To continue a forward over L0 tokens (a multiple of 64): chunk_state = its
 * final_state, conv_state = its conv_state_out, pos = 0; a prefill whose
 * length is not a multiple of 64 passes its last L mod 64 tokens through
 * this call.  No document ids: appended tokens continue the working chunk's
 * document.  All buffers 16-byte aligned (chunk_dt, dt_raw: 4-byte).
 * conv_dim at most 4194304 (the working chunk's row width).
 */
int ssd_resume_fwd(int B, int H, int P, int N, int G, int K, int dtype, int pos, int n,
                   const void *xbc_raw, const void *dt_raw, const void *z,
                   const float *conv_w, const float *conv_b, const float *dt_bias,
                   const float *A, const float *D, int act,
                   void *conv_state, void *chunk_xbc, float *chunk_dt, void *chunk_z,
                   float *chunk_state, float *chunk_y, float *y, void *stream);

/*
 * ssd_step -- one decode token for each of B sequences.
 *
 * window = [conv_state[b][0..K-2], xbc_raw[b]]; xbc = act(conv over window),
 * rounded to T; conv_state shifts by one row (the new raw row enters last);
 * dt = softplus(dt_raw + dt_bias); then one token of the recurrence and the
 * gate.  This is ssd_conv_fwd + ssd_chunk_scan_fwd at L = 1 with both
 * states carried, so it continues a prefill's conv_state_out/final_state
 * buffers as they are.
 *
 *   xbc_raw    T   [B][conv_dim]     dt_raw T [B][H]     z T [B][H*P] or NULL
 *   conv_w     f32 [conv_dim][K]     conv_b f32 [conv_dim] or NULL
 *   dt_bias    f32 [H] or NULL       A f32 [H]           D f32 [H] or NULL
 *   conv_state T   [B][K-1][conv_dim], read and updated in place
 *   ssm_state  f32 [B][H][P][N],     read and updated in place
 *   y          f32 [B][H*P]
 * Rows are contiguous.  xbc_raw, z, conv_w, conv_state and ssm_state must be
 * 16-byte aligned (they are read in 16-byte pieces); dt_raw, the parameter
 * vectors and y 4-byte aligned.  A misaligned pointer is refused with
 * SSD_ERR_ALIGNMENT before any launch.
 * One workgroup serves one sequence, so B should be >= the CU count (256)
 * for full-device bandwidth.  Deterministic and batch-invariant: a row's
 * result does not depend on B or on the other rows.  The conv row, the gate
 * row and four per-head values are staged in LDS: sizes with
 * conv_dim + H*P + 4*H > 16384 floats are refused (SSD_ERR_UNSUPPORTED).
 */
int ssd_step(int B, int H, int P, int N, int G, int K, int dtype,
             const void *xbc_raw, const void *dt_raw, const void *z,
             const float *conv_w, const float *conv_b, const float *dt_bias,
             const float *A, const float *D,
             void *conv_state, float *ssm_state, int act, float *y, void *stream);

/*
 * ssd_s6_scan_fwd -- the Mamba-1 selective scan (S6).
 *
 * Per batch row b and channel d (D channels), with a state of N entries:
 *     a_t[d][n] = exp(dt_t[d] * A[d][n])
 *     h_t[d][n] = a_t[d][n] * h_{t-1}[d][n] + dt_t[d] * B_t[n] * x_t[d]
 *     y_t[d]    = (sum_n C_t[n] h_t[d][n] + D_skip[d] * x_t[d]) * silu(z_t[d])
 * (builderforce-memory-engine diff, falcon_mamba.ts header: x_proj rows
 * [dt, B, C] give one B and one C per token for all channels, dt_proj gives
 * dt per channel with its bias inside the softplus, A_log is [d_inner,
 * d_state] and A = -exp(A_log)).  Document ids, states and the gate follow
 * the conventions above; the state is [B][D][N] with n fastest.  The decay
 * differs per (d, n), so the scan runs token by token (no chunked matrix
 * form); with a workspace of ssd_s6_workspace_size() bytes the sequence is
 * cut into superchunks scanned in parallel, a first pass storing each one's
 * local end state and sum of dt, and the main pass folding them in (results
 * agree with the sequential pass to fp32 rounding, not bitwise; final_state
 * may equal init_state either way).  exp and softplus use the hardware exp2 /
 * log2 (a few ulp); softplus(v) for v below about -17 reads as 0.
 *
 *   x, dt   T   [B][L][D]   row strides x_row_stride, dt_row_stride;
 *               dt_softplus = 0: dt is already activated; 1: dt :=
 *               softplus(dt + dt_bias)
 *   dt_bias f32 [D] or NULL (read only when dt_softplus = 1)
 *   A       f32 [D][N], A <= 0 (the caller computes A = -exp(A_log))
 *   Bm, Cm  T   [B][L][N]   row strides B_row_stride, C_row_stride (column
 *               slices of the x_proj output are fine)
 *   D_skip  f32 [D] or NULL; z T [B][L][D] or NULL; doc_ids i32 [B][L] or NULL
 *   init_state, final_state  f32 [B][D][N] or NULL
 *   y       f32 [B][L][D]   row stride y_row_stride; must not overlap inputs
 *   workspace, workspace_bytes: NULL, 0 (one sequential pass per channel)
 *               or device scratch of at least ssd_s6_workspace_size()
 *               bytes, 16-byte aligned, caller-owned, not shared by
 *               concurrent calls
 * Supported: N in {8, 16, 32}, any D >= 1, B, L >= 0.  Tensor bases 16-byte
 * aligned and T row strides multiples of 16 bytes, as above; row strides in
 * elements, >= the row width and <= 4194304.
 */
int ssd_s6_scan_fwd(int B, int L, int D, int N, int dtype,
                    const void *x, int64_t x_row_stride,
                    const void *dt, int64_t dt_row_stride,
                    int dt_softplus, const float *dt_bias,
                    const float *A,
                    const void *Bm, int64_t B_row_stride,
                    const void *Cm, int64_t C_row_stride,
                    const float *D_skip,
                    const void *z, int64_t z_row_stride,
                    const int32_t *doc_ids,
                    const float *init_state, float *final_state,
                    float *y, int64_t y_row_stride,
                    void *workspace, size_t workspace_bytes, void *stream);

/* Bytes of workspace that let ssd_s6_scan_fwd split the sequence for these
 * sizes: hloc [B][D][K-1][N] and sdt [B][D][K-1] (fp32) and a copy of the
 * initial state; 0 when no split pays. */
size_t ssd_s6_workspace_size(int B, int L, int D, int N, int dtype);

/*
 * ssd_chunk_scan_bwd -- backward (vector-Jacobian product) of
 * ssd_chunk_scan_fwd for a prefill from a zero state.
 *
 * Given grad_y = dLoss/dy, writes the gradients of every input of the scan.
 * The forward is recomputed from the inputs; no earlier forward's state is
 * used.  As the mojolearn.Mamba3Block backward() describes, there is no
 * gradient for a carried initial state and no cotangent for the final state.
 * Document ids cut gradients exactly as they cut the forward: a loss on a
 * later document gives exactly zero gradient on earlier-document inputs
 * (Mini-K3-1H card, "Checkpoint and training").  bf16 inputs are widened to
 * fp32; all gradients are fp32.  Results are deterministic: dB and dC are
 * summed over a group's heads in one workgroup, and dA, dD, ddt_bias through
 * per-chunk partial sums added in a fixed order.
 *
 *   x, Bm, Cm, dt, dt_softplus, dt_bias, A, D, z, doc_ids   as in
 *               ssd_chunk_scan_fwd (no init_state)
 *   grad_y  f32 [B][L][H*P], row stride grad_y_row_stride
 *   dx      f32 [B][L][H*P];  dB, dC f32 [B][L][G*N] (row strides in
 *               elements, multiples of 4)
 *   ddt     f32 [B][L][H]: with respect to the dt input (the raw value when
 *               dt_softplus = 1)
 *   ddt_bias f32 [H] or NULL (written when dt_softplus = 1)
 *   dA      f32 [H]: with respect to A (the caller chains A = -exp(A_log))
 *   dD      f32 [H] or NULL (zero when D is NULL)
 *   dz      f32 [B][L][H*P] or NULL (only with z)
 *   workspace, workspace_bytes: required, at least
 *               ssd_chunk_scan_bwd_workspace_size() bytes, 16-byte aligned,
 *               caller-owned, not shared by concurrent calls
 * Outputs must not overlap the inputs or each other.  Supported: N in
 * {16, 32, 64, 128}, P = 64, chunk = 64.  L = 0 writes zero parameter
 * gradients.
 */
int ssd_chunk_scan_bwd(int B, int L, int H, int P, int N, int G, int chunk, int dtype,
                       const void *x, int64_t x_row_stride,
                       const void *Bm, int64_t B_row_stride,
                       const void *Cm, int64_t C_row_stride,
                       const float *dt, int64_t dt_row_stride,
                       int dt_softplus, const float *dt_bias,
                       const float *A, const float *D,
                       const void *z, int64_t z_row_stride,
                       const int32_t *doc_ids,
                       const float *grad_y, int64_t grad_y_row_stride,
                       float *dx, int64_t dx_row_stride,
                       float *dB, int64_t dB_row_stride,
                       float *dC, int64_t dC_row_stride,
                       float *ddt, int64_t ddt_row_stride,
                       float *ddt_bias, float *dA, float *dD,
                       float *dz, int64_t dz_row_stride,
                       void *workspace, size_t workspace_bytes, void *stream);

/* Bytes of workspace ssd_chunk_scan_bwd needs: the state entering and the
 * adjoint of the state leaving every chunk ([B][H][L/64][N][P] fp32 each),
 * the chunk decays and per-chunk partial sums. */
size_t ssd_chunk_scan_bwd_workspace_size(int B, int L, int H, int P, int N, int G, int dtype);

/*
 * ssd_conv_bwd -- backward of ssd_conv_fwd's conv + act for a zero conv
 * state: given grad_xbc = dLoss/d(conv output) (f32 [B][L][conv_dim]),
 * writes dxbc_raw (f32 [B][L][conv_dim]), dconv_w (f32 [conv_dim][K]) and
 * dconv_b (f32 [conv_dim] or NULL).  Taps across a document start carry no
 * gradient, as they carry no value forward.  The softplus of dt is not part
 * of this call: ssd_chunk_scan_bwd with dt_softplus = 1 (or ssd_mixer_bwd)
 * returns dt_raw's gradient.  The workspace (ssd_conv_bwd_workspace_size()
 * bytes, required) holds per-64-token partial sums of dconv_w and dconv_b.
 */
int ssd_conv_bwd(int B, int L, int H, int P, int N, int G, int K, int dtype,
                 const void *xbc_raw, int64_t xbc_raw_row_stride,
                 const float *conv_w, const float *conv_b, const int32_t *doc_ids, int act,
                 const float *grad_xbc, int64_t grad_xbc_row_stride,
                 float *dxbc_raw, int64_t dxbc_raw_row_stride,
                 float *dconv_w, float *dconv_b,
                 void *workspace, size_t workspace_bytes, void *stream);

size_t ssd_conv_bwd_workspace_size(int B, int L, int H, int P, int N, int G, int dtype);

/*
 * ssd_mixer_bwd -- backward of ssd_mixer_fwd (conv + act, dt softplus, scan,
 * D skip, gate) for a prefill from zero states.
 *
 * Recomputes the conv output and dt with the conv kernel (a bf16 pipeline's
 * rounding of the conv output is taken as the identity in the backward),
 * runs ssd_chunk_scan_bwd's passes on them, then the conv backward.  Writes
 * dxbc_raw (f32 [B][L][conv_dim]), dconv_w, dconv_b, ddt_raw (f32 [B][L][H]),
 * ddt_bias, dA, dD and dz as above.  workspace: required,
 * ssd_mixer_bwd_workspace_size() bytes.
 */
int ssd_mixer_bwd(int B, int L, int H, int P, int N, int G, int K, int chunk, int dtype,
                  const void *xbc_raw, int64_t xbc_raw_row_stride,
                  const float *conv_w, const float *conv_b,
                  const void *dt_raw, int64_t dt_raw_row_stride, const float *dt_bias,
                  const float *A, const float *D,
                  const void *z, int64_t z_row_stride,
                  const int32_t *doc_ids, int act,
                  const float *grad_y, int64_t grad_y_row_stride,
                  float *dxbc_raw, int64_t dxbc_raw_row_stride,
                  float *dconv_w, float *dconv_b,
                  float *ddt_raw, int64_t ddt_raw_row_stride, float *ddt_bias,
                  float *dA, float *dD,
                  float *dz, int64_t dz_row_stride,
                  void *workspace, size_t workspace_bytes, void *stream);

/* Bytes of workspace of ssd_mixer_bwd: the recomputed conv output (T) and dt,
 * the conv output's gradient (fp32), and the two backward calls' scratch. */
size_t ssd_mixer_bwd_workspace_size(int B, int L, int H, int P, int N, int G, int dtype);

#ifdef __cplusplus
}
#endif

#endif /* SSD_H */
