/*
 * wkv7.h -- C ABI of the MI355X (gfx950) WKV7 library.
 *
 * The operation: the RWKV-7 "Goose" WKV state recurrence, a generalised delta
 * rule with a diagonal-plus-rank-one transition, vector-valued data-dependent
 * decay and separate removal and replacement keys ("Paper Review: RWKV-7
 * Goose", sections Architecture and The approach; "RWKV-7 Goose with
 * Expressive Dynamic State Evolution", Abstract).  Per batch row b and head h
 * the state S is an N x N fp32 matrix, row i = value channel, column j = key
 * channel, and every token t applies
 *
 *     S <- S (diag(w_t) + a_t b_t^T) + v_t k_t^T,      y_t = S r_t
 *
 * i.e. z = S a_t (old state), S[i][j] = S[i][j] w_t[j] + z[i] b_t[j] +
 * v_t[i] k_t[j], then the receptance reads the updated state ("once the WKV
 * state is updated", The approach).  In RWKV-7, a = -kappa (removal key),
 * b = kappa * alpha (in-context learning rate), k = the replacement key; the
 * library takes a and b as general vectors and never assumes that form.
 *
 * Conventions shared by every entry point
 *   - Tensor pointers are DEVICE pointers owned by the caller.  The library
 *     never allocates, frees or synchronises, and keeps no pointer after the
 *     call returns.  All work is enqueued asynchronously on `stream` (a
 *     hipStream_t passed as void*; NULL = the default stream).
 *   - Layouts are row-major, last index fastest:
 *       token tensors r, w, k, v, a, b, y, dy, dr..db   [B][T][H][N]
 *       states s0, sT, dsT, ds0, decode state           [B][H][N][N] (fp32)
 *       tape (forward -> backward), see wkv7_tape_bytes
 *   - `dtype` selects the element type of the token tensors and gradients:
 *     WKV7_F32 (IEEE float) or WKV7_BF16 (bfloat16, outputs rounded to
 *     nearest even).  States are always fp32; the tape is always bf16.
 *   - w is the multiplicative decay itself (not its logarithm).  The
 *     sequential scan and the decode step accept any finite w.  The chunked
 *     form (chunk_len > 0) divides by running products of w inside a chunk
 *     and requires 0 < w <= 1 with w^chunk_len above ~1e-30.
 *   - Validation is synchronous and launches nothing on error:
 *       WKV7_ERR_INVALID_ARG  negative sizes, NULL required pointers, pointers
 *                             not 16-byte aligned, NULL desc;
 *       WKV7_ERR_UNSUPPORTED  unsupported head size (below), unknown dtype,
 *                             unsupported chunk_len, T above INT32_MAX - 64,
 *                             more than 2^28 heads (B*H);
 *       WKV7_ERR_WORKSPACE    workspace smaller than wkv7_workspace_bytes();
 *       WKV7_ERR_LAUNCH       the HIP runtime reported a launch error.
 *     No exception crosses the ABI.  There is no global mutable state, so
 *     concurrent calls on different streams are safe.
 *   - a and b may both be NULL (with tokens; never just one of them): then
 *     a = b = 0 and the transition is diagonal, S <- S diag(w_t) + v_t k_t^T,
 *     the vector-decay recurrence that RWKV-7 extends ("Paper Review: RWKV-7
 *     Goose", Background information on delta rule: RWKV-6 decays the state
 *     with a diagonal transition).  Every entry point then runs kernels
 *     specialised for it, which skip the removal terms; the forward does not
 *     write the tape's Z part (the backward does not read it) and the
 *     backward leaves da and db unwritten (they may be NULL).
 *   - Inputs must not alias outputs, except the decode state (in place).
 *   - Empty problems (B, H or T equal to 0) are valid.  With T = 0 the forward
 *     copies s0 (or zeros) to sT; y may then be NULL.
 */
#ifndef WKV7_H
#define WKV7_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define WKV7_ABI_VERSION 1
/* Head sizes: the sequential forms (chunk_len = 0: the scan and the reverse
   pass of wkv7_backward), the decode step and the chunked forward (chunk_len =
   16: wkv7_forward, _ckpt, _split, _static, _epilogue) take N = 32, 64 or 128
   (a larger N is the state expansion of "Millions of States: Designing a
   Scalable MoE Architecture with RWKV-7 Meta-learner", Abstract); the chunked
   backward entry points take N = 32 or WKV7_HEAD_SIZE.  At N = 128 the chunked
   forward writes no tape (tape must be NULL, else WKV7_ERR_UNSUPPORTED) and
   splits in time by maps only (wkv7_forward_split: segments <= -2 return
   WKV7_ERR_UNSUPPORTED); it writes fp32 checkpoints (wkv7_forward_ckpt), from
   which wkv7_backward_ckpt (chunk_len = 0) trains.  It splits each head's
   value rows over two workgroups, which form the chunk factors each, while
   those fit the device at once (else one workgroup per head). */
#define WKV7_HEAD_SIZE 64
#define WKV7_TAPE_CHUNK 16       /* tokens per chunk of the backward */
#define WKV7_TAPE_BLOCK 32       /* tokens per state saved in the forward tape */

typedef enum {
    WKV7_OK = 0,
    WKV7_ERR_INVALID_ARG = 1,
    WKV7_ERR_UNSUPPORTED = 2,
    WKV7_ERR_WORKSPACE = 3,
    WKV7_ERR_LAUNCH = 4,
    WKV7_ERR_STATIC_SCRATCH = 5   /* the call needs more than WKV7_STATIC_SCRATCH_BYTES */
} wkv7_status;

/* Size of the device scratch that wkv7_forward_split_static uses in place of a
   workspace (one copy per device, held until the process ends). */
#define WKV7_STATIC_SCRATCH_BYTES (16u << 20)

typedef enum { WKV7_F32 = 0, WKV7_BF16 = 1 } wkv7_dtype;

/* Problem descriptor.  chunk_len = 0 selects the sequential forms (one token
   at a time, state rows in registers, fp32 arithmetic: the scan forward, the
   reverse recurrence backward); 16 selects the chunked forms, whose
   intra-chunk products run on bf16 matrix cores with the carried state kept
   in fp32 (the pages state that training remains parallelisable: Abstract;
   Elamur summary, Summary). */
typedef struct {
    int32_t B, T, H, N;
    int32_t dtype;      /* wkv7_dtype */
    int32_t chunk_len;  /* 0 or 16 */
} wkv7_desc;

/* Returns WKV7_ABI_VERSION. */
int wkv7_abi_version(void);

/* Static, never-NULL description of a status code. */
const char *wkv7_status_string(int status);

/* Bytes of the tape that wkv7_forward can write for wkv7_backward:
     Z   [B][T][H][N]              bf16: z_t = S_{t-1} a_t, the removal read-outs;
     S   [B][H][ceil(T/32)][N][N]  bf16: the state entering every 32-token block
                                   (tokens 32m ..), stored key-major (element
                                   [j][i] = S[i][j]).
   0 on an invalid descriptor, and at N = 128 with chunk_len = 16 (that form
   writes no tape). */
size_t wkv7_tape_bytes(const wkv7_desc *desc);

/* Bytes of the fp32 checkpoints that wkv7_forward_ckpt writes and the
   sequential reverse pass (wkv7_backward with chunk_len = 0) reads:
     S   [B][H][ceil(T/16)][N][N]  fp32: the state entering every 16-token
                                   chunk (tokens 16m ..), element [i][j] =
                                   S[i][j] (row = value channel).
   This is the per-head state of "Paper Review: RWKV-7 Goose", The approach,
   kept at chunk boundaries for the backward.  0 on an invalid descriptor. */
size_t wkv7_ckpt_bytes(const wkv7_desc *desc);

/* Bytes of device scratch that wkv7_backward needs when the caller supplies
   nothing the forward wrote (no tape, no checkpoints): the size that always
   suffices.  Equal to wkv7_backward_workspace_bytes(desc, 0). */
size_t wkv7_workspace_bytes(const wkv7_desc *desc);

/* Bytes of device scratch wkv7_backward needs, given whether the caller passes
   a tape.
   chunk_len = 16: with_tape != 0 when the caller passes a tape written by
   wkv7_forward (the backward then keeps one per-token intermediate adjoint and
   the adjoint of the state leaving every 32-token block there, as much again as
   the tape, plus 256 bytes of work queues); with_tape = 0 when it passes none
   (then a forward re-run also writes its tape into the workspace: twice the
   tape); and, when the adjoint chain runs in time segments (below, at
   wkv7_backward), from the next 256-byte boundary 3 * nseg fp32 N x N states
   per head.  That choice depends on the current device: query the size and
   call on the same one.
   chunk_len = 0 (the sequential reverse pass, which writes fp32 checkpoints
   itself): wkv7_ckpt_bytes(desc), whatever with_tape is (wkv7_backward_ckpt,
   which reads the caller's checkpoints, needs none).
   0 on an invalid descriptor or one the backward does not take (chunk_len = 16
   with fp32, or at N = 128). */
size_t wkv7_backward_workspace_bytes(const wkv7_desc *desc, int with_tape);

/*
 * Forward over a whole sequence.
 *   r, w, k, v, a, b  [B][T][H][N] inputs (dtype).
 *   s0                [B][H][N][N] fp32 initial state, or NULL for zeros.
 *   y                 [B][T][H][N] output y_t = S_t r_t (dtype).
 *   sT                [B][H][N][N] fp32 final state, or NULL.
 *   tape              NULL, or wkv7_tape_bytes(desc) bytes: receives the
 *                     removal read-outs and chunk entry states for
 *                     wkv7_backward (layout at wkv7_tape_bytes).  NULL for
 *                     the chunked form at N = 128 (else WKV7_ERR_UNSUPPORTED).
 */
int wkv7_forward(const wkv7_desc *desc, const void *r, const void *w, const void *k,
                 const void *v, const void *a, const void *b, const float *s0, void *y,
                 float *sT, void *tape, void *stream);

/*
 * wkv7_forward writing fp32 checkpoints instead of the tape: the same y and sT,
 * and in `ckpt` (NULL, or wkv7_ckpt_bytes(desc) bytes) the fp32 state entering
 * every 16-token chunk, layout at wkv7_ckpt_bytes.  Either form writes them
 * (the scan from its registers every 16 tokens, the chunked form from its fp32
 * carried state), and either form's checkpoints feed wkv7_backward_ckpt.
 */
int wkv7_forward_ckpt(const wkv7_desc *desc, const void *r, const void *w, const void *k,
                      const void *v, const void *a, const void *b, const float *s0, void *y,
                      float *sT, float *ckpt, void *stream);

/*
 * wkv7_forward with each head's sequence split in time, for the two shapes
 * where one workgroup per head leaves the device idle on serial chains of
 * T/16 chunks: few heads, and more heads than compute units (whose last,
 * partial round of heads runs mostly alone).  Same arguments and results as
 * wkv7_forward (y, sT and tape agree with it to rounding), plus:
 *   segments   0: the library chooses from the device's compute-unit count
 *                 (B*H at most a third of it: every head by maps, below; more
 *                 heads than compute units: the heads of the last, partial
 *                 round by maps when they fill at most a fifth of it; the
 *                 scan: every head by maps when B*H*N/16 workgroups fill at
 *                 most half of it; the chunked form at N = 128: every head
 *                 by maps when its two workgroups per head fill at most a
 *                 third of it, and with more heads than compute units those
 *                 of the last round when they fill at most a quarter of it;
 *                 at N = 128 in at most 4 segments; else, or
 *                 when T is too short for segments of 128 tokens, no split);
 *              1 or -1: no split (exactly wkv7_forward);
 *              n >= 2: every head in up to n segments by maps;
 *              n <= -2: every head in up to -n sequential segments.
 *              At most 16 segments; below -16: WKV7_ERR_INVALID_ARG.  The
 *              chunked form (chunk_len = 16) at N = 32 and 64 splits both
 *              ways; at N = 128, and the sequential scan (chunk_len = 0, N =
 *              32, 64 or 128), by maps only (n <= -2: WKV7_ERR_UNSUPPORTED).
 *   workspace  wkv7_forward_split_workspace_bytes(desc, segments) bytes of
 *              device scratch, or NULL when that is 0; else WKV7_ERR_WORKSPACE.
 * Segments start at multiples of 32 tokens (the tape's state blocks).
 * Maps: the state update is affine in the state, S <- S M_t + v_t k_t^T with
 * M_t = diag(w_t) + a_t b_t^T (the transition of "Paper Review: RWKV-7 Goose",
 * The approach), so a segment maps its entry state as S_out = S_in P + Hm,
 * P = the product of its transitions (a run from the identity with v = 0) and
 * Hm = its final state from zero.  A first launch runs segment 0 with its
 * outputs and the two map runs of segments 1 .. n-2 side by side; a small
 * kernel composes the entry states in fp32; a second launch re-runs segments
 * 1 .. n-1 from them with their outputs.  The serial chain per head falls
 * from T to about 2T/n tokens.
 * Sequential: one workgroup per segment, numbered segment by segment over all
 * heads; each waits for its head's previous segment to publish its final state
 * (fp32, in the workspace) and publishes its own.  No extra work: the device
 * takes segments as they come instead of whole heads.  This relies on the
 * device dispatching a grid's workgroups in order (a segment waits only for
 * one dispatched before it).  The wait is bounded (about a second; the
 * environment variable WKV7_SEGMENT_SPIN_LIMIT sets the number of polls): a
 * segment whose wait expires starts from a NaN state, so its y, tape and
 * final state, and those of the head's later segments, are NaN -- an expired
 * wait never yields plausible but wrong results.  The status stays WKV7_OK
 * (the launch cannot report it); check the outputs when in doubt.
 * The automatic choice depends on the current device: query the size and call
 * on the same one.
 */
size_t wkv7_forward_split_workspace_bytes(const wkv7_desc *desc, int32_t segments);

/* The plan wkv7_forward_split would run for `segments` on the current device,
 * returned without running it (for logs and tuning): heads [split_from, B*H)
 * run in nseg segments of seg_len tokens (the last takes the rest), by maps or
 * sequentially; with no split, split_from = B*H, nseg = 1 and seg_len = T.
 * Returns WKV7_OK, or the status wkv7_forward_split returns for that desc and
 * segments (plan NULL: WKV7_ERR_INVALID_ARG). */
enum { WKV7_SPLIT_NONE = 0, WKV7_SPLIT_MAPS = 1, WKV7_SPLIT_SEQUENTIAL = 2 };
typedef struct {
    int32_t kind;         /* WKV7_SPLIT_* */
    int32_t split_from;
    int32_t nseg;
    int32_t seg_len;
} wkv7_split_plan;
int wkv7_forward_split_plan(const wkv7_desc *desc, int32_t segments, wkv7_split_plan *plan);
int wkv7_forward_split(const wkv7_desc *desc, const void *r, const void *w, const void *k,
                       const void *v, const void *a, const void *b, const float *s0, void *y,
                       float *sT, void *tape, int32_t segments, void *workspace,
                       size_t workspace_bytes, void *stream);

/*
 * wkv7_forward_split without a workspace, for callers that cannot allocate
 * device memory (code under stream capture, tight serving loops, harnesses
 * that forbid allocation).  Same arguments (minus the workspace) and results
 * as wkv7_forward_split: the segment plan's scratch (the entry states and maps,
 * or the sequential segments' states and flags) lives in a fixed device buffer
 * of WKV7_STATIC_SCRATCH_BYTES inside the library, one per device.  A call
 * whose plan needs more returns WKV7_ERR_STATIC_SCRATCH and launches nothing
 * (wkv7_forward_split_workspace_bytes gives the need).  The call allocates
 * nothing: the buffer's device address is looked up on the first call on each
 * device.  Every call on a device shares that device's buffer, so calls that
 * overlap on one device (other streams, other threads) race: serialise them.
 * The buffer keeps the previous call's contents; nothing in it is read before
 * the call writes it (the sequential segments' flags are cleared by a kernel).
 */
int wkv7_forward_split_static(const wkv7_desc *desc, const void *r, const void *w,
                              const void *k, const void *v, const void *a, const void *b,
                              const float *s0, void *y, float *sT, void *tape, int32_t segments,
                              void *stream);

/*
 * Gradients of the scalar  L = sum_t <dy_t, y_t> + <dsT, S_T>  with respect to
 * r, w, k, v, a, b (written in dtype) and s0 (fp32).  This is the adjoint of
 * the same recurrence: the adjoint state G = dL/dS runs backwards in time as
 * G <- G (diag(w_t) + b_t a_t^T) + dy_{t-1} r_{t-1}^T.
 *   s0          as given to the forward (NULL = zeros).
 *   dy          [B][T][H][N] upstream gradient of y (dtype).
 *   dsT         [B][H][N][N] fp32 upstream gradient of S_T, or NULL (= 0).
 *   tape        chunked form: the tape written by wkv7_forward with the same
 *               inputs and s0 (by either forward form), or NULL; then the
 *               backward first re-runs the chunked forward to write it.  Not
 *               used by the sequential form (chunk_len = 0).
 *   dr..db      [B][T][H][N] outputs (dtype).  ds0: [B][H][N][N] fp32 or NULL.
 *   workspace   at least wkv7_backward_workspace_bytes(desc, tape != NULL)
 *               bytes of device scratch (contents on entry are ignored); else
 *               WKV7_ERR_WORKSPACE.  Required whenever B*T*H > 0.
 * desc->chunk_len selects the form:
 *   16  chunk by chunk (16 tokens) on bf16 matrix cores: dtype = WKV7_BF16 and
 *       N = 32 or 64 (WKV7_ERR_UNSUPPORTED otherwise); uses the tape.  The
 *       adjoint chain (a serial run per head from the last chunk to the
 *       first) runs in time segments when wkv7_forward_split's automatic plan
 *       for the same desc splits every head (few heads; see there): the
 *       adjoint is affine in itself, so a segment maps the adjoint at its
 *       right edge as dS_left = dS_right P + H (P: the run from the identity
 *       with dy = 0, H: the run from zero), and a first launch runs the last
 *       segment and the maps of the middle ones, a small kernel composes the
 *       entry adjoints in fp32, a second launch runs the other segments
 *       (gradients agree with the unsplit chain to rounding).
 *   0   the sequential reverse recurrence token by token in fp32 on the vector
 *       ALU (one workgroup per head): either dtype, N = 32, 64 or 128.  It
 *       first re-runs the sequential forward to write fp32 states every 16
 *       tokens into the workspace (wkv7_ckpt_bytes); wkv7_backward_ckpt
 *       takes them from the caller instead.
 */
int wkv7_backward(const wkv7_desc *desc, const void *r, const void *w, const void *k,
                  const void *v, const void *a, const void *b, const float *s0,
                  const void *dy, const float *dsT, const void *tape, void *dr, void *dw,
                  void *dk, void *dv, void *da, void *db, float *ds0, void *workspace,
                  size_t workspace_bytes, void *stream);

/*
 * The sequential reverse pass (desc->chunk_len = 0, else WKV7_ERR_UNSUPPORTED)
 * from the caller's fp32 checkpoints instead of a re-run of the scan: `ckpt`
 * (required when B*T*H > 0) holds what wkv7_forward_ckpt wrote for the same
 * inputs and s0, by either forward form, wkv7_ckpt_bytes(desc) bytes.  Other
 * arguments and results as wkv7_backward; no workspace.
 */
int wkv7_backward_ckpt(const wkv7_desc *desc, const void *r, const void *w, const void *k,
                       const void *v, const void *a, const void *b, const float *s0,
                       const void *dy, const float *dsT, const float *ckpt, void *dr, void *dw,
                       void *dk, void *dv, void *da, void *db, float *ds0, void *stream);

/*
 * The two stages of wkv7_backward as separate calls, for callers that schedule
 * or time them apart; both take exactly wkv7_backward's arguments, and calling
 * wkv7_backward_adjoint then wkv7_backward_gradients on one stream with the
 * same arguments computes what wkv7_backward computes.  `tape` is required
 * (WKV7_ERR_INVALID_ARG when NULL and B*T*H > 0): the workspace carries the
 * first stage's results to the second, so both calls must receive the same
 * workspace, untouched in between.  Chunked form only (chunk_len = 0:
 * WKV7_ERR_UNSUPPORTED).
 *   wkv7_backward_adjoint    the sequential part: the adjoint state carried
 *                            backwards through the chunks (the transposed
 *                            transition of "Paper Review: RWKV-7 Goose", The
 *                            approach), one chunk at a time.  Writes dv and
 *                            ds0 (if not NULL) and fills the workspace with the
 *                            adjoint entering every chunk and the per-token
 *                            intermediate adjoint.  dr, dw, dk, da, db are not
 *                            touched.
 *   wkv7_backward_gradients  the parallel part: every chunk independently,
 *                            from the tape and the workspace.  Writes dr, dw,
 *                            dk, da, db; dv, ds0 and the workspace are not
 *                            touched.
 */
int wkv7_backward_adjoint(const wkv7_desc *desc, const void *r, const void *w, const void *k,
                          const void *v, const void *a, const void *b, const float *s0,
                          const void *dy, const float *dsT, const void *tape, void *dr,
                          void *dw, void *dk, void *dv, void *da, void *db, float *ds0,
                          void *workspace, size_t workspace_bytes, void *stream);
int wkv7_backward_gradients(const wkv7_desc *desc, const void *r, const void *w, const void *k,
                            const void *v, const void *a, const void *b, const float *s0,
                            const void *dy, const float *dsT, const void *tape, void *dr,
                            void *dw, void *dk, void *dv, void *da, void *db, float *ds0,
                            void *workspace, size_t workspace_bytes, void *stream);

/*
 * wkv7_backward on two streams, for callers that have a second one: same
 * arguments and results, plus `aux_stream` (a hipStream_t as void*, or NULL =
 * plain wkv7_backward on `stream`).  When B*H exceeds the device's compute
 * units and B > 1, the batch rows split into a first group that fills the
 * device with one workgroup per head and the rest; the first group's per-key
 * pass runs on aux_stream beside the second group's adjoint chain (the chain
 * is one workgroup per head, so it alone would leave most of the device idle
 * in its last round).  All work has finished, as seen from `stream`, when the
 * work enqueued on `stream` has: `stream` waits for aux_stream's part.  The
 * library creates and destroys two events per call; it never synchronises.
 * With chunk_len = 0 the sequential reverse pass runs on `stream` alone.
 */
int wkv7_backward_overlapped(const wkv7_desc *desc, const void *r, const void *w, const void *k,
                             const void *v, const void *a, const void *b, const float *s0,
                             const void *dy, const float *dsT, const void *tape, void *dr,
                             void *dw, void *dk, void *dv, void *da, void *db, float *ds0,
                             void *workspace, size_t workspace_bytes, void *stream,
                             void *aux_stream);

/*
 * One token on B*H resident states, in place: constant memory and constant
 * time per token at inference (Abstract).
 *   r, w, k, v, a, b  [B][H][N] this step's inputs (dtype).
 *   state             [B][H][N][N] fp32, read and overwritten.
 *   y                 [B][H][N] output (dtype).
 */
int wkv7_decode_step(int32_t B, int32_t H, int32_t N, int32_t dtype, const void *r,
                     const void *w, const void *k, const void *v, const void *a,
                     const void *b, float *state, void *y, void *stream);

/*
 * The step after the read-out ("Paper Review: RWKV-7 Goose", The approach:
 * the receptance also attends to the current token without storing it in the
 * state, and the result is normalised per head and gated; combining the heads
 * through the output projection is not part of it).  The pages fix neither the
 * current-token formula, the normalisation nor their order; the library takes
 * them with the learned parts as inputs.  Per token t and head h, over the
 * head's N channels:
 *     s       = r_t . (u_h * k_t)                         (a scalar)
 *     norm(x) = gamma_h * (x - mean(x)) / sqrt(var(x) + eps) + beta_h,
 *               var = the mean squared deviation (divisor N)
 *     WKV7_EPI_PLAIN:     out_t = g_t * (y_t + s v_t)
 *     WKV7_EPI_NORM_TERM: out_t = g_t * (norm(y_t) + s v_t)
 *     WKV7_EPI_TERM_NORM: out_t = g_t * norm(y_t + s v_t)
 * (* elementwise).  The arithmetic is fp32; the result is written in dtype.
 */
typedef enum { WKV7_EPI_PLAIN = 0, WKV7_EPI_NORM_TERM = 1, WKV7_EPI_TERM_NORM = 2 } wkv7_epi_mode;

/* The learned parts and settings (device pointers to fp32 [H][N], each
   16-byte aligned, or NULL). */
typedef struct {
    const float *u;      /* current-token weights; NULL: no current-token term */
    const float *gamma;  /* scale after normalising; NULL = 1 */
    const float *beta;   /* shift after normalising; NULL = 0 */
    float eps;           /* added to the variance: finite, >= 0 */
    int32_t mode;        /* wkv7_epi_mode */
} wkv7_epilogue_params;

/*
 * The step after the read-out on its own, over [B][T][H][N] tensors in
 * desc->dtype with N = 32, 64 or 128 (desc->chunk_len is ignored): reads y (a
 * read-out such as wkv7_forward's), r, k and v (only with params->u), g (the
 * gate; NULL = 1) and writes out, which may be y itself (in place) but must
 * not overlap the other inputs.  params must not be NULL.  WKV7_ERR_INVALID_ARG
 * for an unknown mode, a negative or non-finite eps, or a missing pointer.
 */
int wkv7_epilogue(const wkv7_desc *desc, const void *y, const void *r, const void *k,
                  const void *v, const void *g, const wkv7_epilogue_params *params, void *out,
                  void *stream);

/*
 * wkv7_forward followed by the step after the read-out: out receives the
 * result in place of y (y itself is not written), sT the final state (may be
 * NULL); no tape.  With chunk_len = 16 and N = 64 the step is fused into the
 * chunked forward kernel, which applies it to the fp32 read-outs before
 * anything is stored (y never reaches memory) when T * H * N * 2 < 2^31 (its
 * per-head offsets are 32-bit); otherwise (and with chunk_len = 0) the forward
 * writes y (in dtype) into out and wkv7_epilogue runs on it in place.  Arguments otherwise as
 * wkv7_forward and wkv7_epilogue.
 */
int wkv7_forward_epilogue(const wkv7_desc *desc, const void *r, const void *w, const void *k,
                          const void *v, const void *a, const void *b, const float *s0,
                          const void *g, const wkv7_epilogue_params *params, void *out,
                          float *sT, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* WKV7_H */
