/*
 * ipttt.h - C ABI of the In-Place Test-Time Training (In-Place TTT) layer
 * forward on AMD Instinct MI355X (gfx950).
 *
 * The layer is the gated MLP whose down projection W_down acts as a fast
 * weight that is updated chunk by chunk while a sequence is read:
 *
 *   Z      = SiLU(H W_gate^T) * (H W_up^T)                     (ipttt_z)
 *   V_hat  = Conv1D_k5(X0) W_target                            (ipttt_target)
 *   dW_i   = clip(eta V_hat_[i]^T Z_[i])                       (ipttt_chunk_delta)
 *   O_[i]  = Z_[i] (W_down + sum_{j<i} dW_j)^T                 (ipttt_scan_apply)
 *
 * Sources: lijianxiong.blog "In-Place Test-Time Training", sections
 * 方法 > 原地自适应 (gated MLP), 高效的块状更新机制 (chunks; apply, then update),
 * 对齐语言模型的目标函数 (target and update rule) and 工程实现 (exclusive prefix
 * sum); developer.cloud.tencent.com "榨干MLP的剩余价值", 详细步骤 3-4 (k=5 conv
 * with padding, chunk-parallel deltas, prefix sum, 1e-5 norm clip);
 * iplexlaw.co.kr In-Place TTT review, sections 3 and 6 (pre-update state per
 * chunk, exclusive scan, reset at document boundaries).
 *
 * Conventions shared by every call
 * --------------------------------
 * - All tensor pointers are DEVICE pointers unless stated otherwise, row-major
 *   and contiguous, 16-byte aligned.  Token axes are flattened: token t of
 *   row b sits at flat index b*T + t.
 * - dtype selects the element type of H, X0, all weights, Z, V_hat and O:
 *   IPTTT_F32 (float) or IPTTT_BF16 (bfloat16, round-to-nearest-even on every
 *   store).  alpha and dW are always float.
 *   Accumulation is fp32 in every kernel.
 * - Chunks form a fixed grid per row: chunk i of a row covers row-relative
 *   tokens [i*C, min((i+1)*C, T)); the last one may be short.  N = ceil(T/C).
 * - Documents: every row start is a document start, except in rows flagged
 *   in `continues`; doc_starts lists the others.  A document start resets the
 *   fast weight to W_down for the tokens from that start on, and the conv
 *   window never reads across it or across a chunk end.
 * - Streaming (one long sequence read in pieces): a row flagged in continues
 *   begins inside the document that was open at the end of the same row of
 *   the previous call; ipttt_scan_apply_carry takes that document's state in
 *   and hands the new one out.  Pieces that are whole numbers of chunks give
 *   exactly the result of one call over the whole sequence.
 * - Every call only enqueues work on `stream` (a hipStream_t; NULL = the
 *   default stream) and returns; device faults surface at the caller's next
 *   synchronisation.  Arguments are validated first: on any error nothing is
 *   launched and no buffer is written.
 * - Ownership: the caller allocates and frees every buffer, including the
 *   workspace; the library allocates no device memory and keeps no state
 *   between calls, so calls on different streams with different buffers may
 *   run concurrently.  Outputs must not alias inputs.
 */
#ifndef IPTTT_H
#define IPTTT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define IPTTT_ABI_VERSION 10

typedef enum {
  IPTTT_OK = 0,
  IPTTT_ERR_NULL = 1,       /* a required pointer is NULL                       */
  IPTTT_ERR_SHAPE = 2,      /* a size is < 1, too large, or d/f not a multiple of 8 */
  IPTTT_ERR_DTYPE = 3,      /* dtype is neither IPTTT_F32 nor IPTTT_BF16         */
  IPTTT_ERR_ALIGN = 4,      /* a tensor pointer is not 16-byte aligned           */
  IPTTT_ERR_SEGMENTS = 5,   /* doc_starts not strictly increasing or out of range */
  IPTTT_ERR_WORKSPACE = 6,  /* ws is NULL or smaller than ipttt_workspace_bytes(),
                               or saved smaller than ipttt_saved_bytes()        */
  IPTTT_ERR_HIP = 7,        /* a HIP runtime call or kernel launch failed         */
  IPTTT_ERR_ARG = 8,        /* eta or tau not finite, an unknown target kind, or
                               S_out overlapping S_in without being S_in         */
  IPTTT_ERR_SCRATCH = 9     /* the problem needs more scratch than the
                               allocation-free call's static array holds
                               (IPTTT_NOALLOC_SCRATCH_BYTES)                     */
} ipttt_status;

typedef enum { IPTTT_F32 = 0, IPTTT_BF16 = 1 } ipttt_dtype;

/* Which target V_hat the fast weights learn (lijianxiong.blog, 对齐语言模型的
 * 目标函数; the ablation of its two parts: tencent article "榨干MLP的剩余价值",
 * 验证模块三, objective decoupling, figure 3(c)):
 *   IPTTT_TARGET_LM       V_hat = Conv1D(X0) W_target   (the method)
 *   IPTTT_TARGET_NO_CONV  V_hat = X0 W_target           (no Conv1D)
 *   IPTTT_TARGET_NO_PROJ  V_hat = Conv1D(X0)            (no W_target)
 * A reconstruction target (the current token only) is IPTTT_TARGET_LM or
 * IPTTT_TARGET_NO_PROJ with conv weights that are zero outside tap 0. */
typedef enum { IPTTT_TARGET_LM = 0, IPTTT_TARGET_NO_CONV = 1, IPTTT_TARGET_NO_PROJ = 2 } ipttt_target_kind;

/* The problem: sizes, element type and document boundaries. */
typedef struct {
  int64_t rows;               /* B: independent sequences (at most 65535)          */
  int64_t seq_len;            /* T: tokens per row                                 */
  int64_t d_model;            /* d: width of H, X0, V_hat, O (multiple of 8)       */
  int64_t d_ff;               /* f: width of Z (multiple of 8)                     */
  int64_t chunk;              /* C: tokens per chunk; rows * ceil(T / C), the
                                 chunks of all rows, at most 65535              */
  int32_t dtype;              /* ipttt_dtype                                       */
  int32_t target;             /* ipttt_target_kind (0 = the LM target of the method) */
  const int64_t *doc_starts;  /* HOST array of flat token offsets in [0, B*T),
                                 strictly increasing; row starts may be listed
                                 or omitted.  NULL (with n_doc_starts = 0) means
                                 one document per row.  Read during the call only. */
  int64_t n_doc_starts;
  const uint8_t *continues;   /* HOST array of `rows` flags, or NULL (no row
                                 continues).  continues[b] != 0: row b's first
                                 tokens, up to its first listed start, continue
                                 a document of the previous call, whose state
                                 ipttt_scan_apply_carry takes as S_in[b]
                                 (the other calls treat it as zero).  A listed
                                 start at b*T wins over the flag.  Read during
                                 the call only. */
  /* Prepared segment descriptors, optional: both NULL (each call then builds
   * its own in its workspace) or both DEVICE arrays that
   * ipttt_segments_device filled for this same problem (sizes, doc_starts,
   * continues), done in stream order before the call: seg_table B*N*3 int32
   * (4-byte aligned), seg_bytes B*T uint8.  The calls then read them and
   * launch no descriptor kernel, so a layer step of several calls builds them
   * once.  Owned by the caller; the library does not check that they match
   * the problem (stale ones give wrong results). */
  const int32_t *seg_table;
  const uint8_t *seg_bytes;
} ipttt_problem;

/* Version of this ABI (IPTTT_ABI_VERSION). */
int ipttt_abi_version(void);

/* Static description of a status code; never NULL. */
const char *ipttt_status_string(int status);

/* Validates a problem description on the host; touches no device. */
ipttt_status ipttt_validate(const ipttt_problem *p);

/* Bytes of device workspace that ipttt_target, ipttt_chunk_delta and
 * ipttt_scan_apply need for this problem (the maximum over the three; one
 * buffer of this size serves all of them in turn).  0 for an invalid problem.
 * Dominated by the per-chunk fast weights of the scan.  On the bf16 path with
 * d and f multiples of 64 the scan and apply run in passes whose weights fit
 * a budget of 4 GiB: as many whole rows as fit, or, when one row's N*d*f
 * weights exceed it, windows of a row's chunks that hand the fp32 state on
 * through the workspace (d*f*4 more bytes); a larger workspace than this
 * minimum gives larger passes.  The environment variable IPTTT_PASS_BYTES
 * (bytes, read at each call) replaces the budget.  Passes compute exactly
 * what one pass would.  Other shapes take B*N*d*f elements at once.  The
 * workspace must be 256-byte aligned; its contents between calls are
 * scratch. */
size_t ipttt_workspace_bytes(const ipttt_problem *p);

/* Host-side segment table, for inspection and tests.  table[(b*N + i)*3 + k]
 * for k = 0, 1, 2 receives, for chunk i of row b with length L:
 *   r0    offset of the first document start inside the chunk (L if none;
 *         0 for chunk 0 of a row that does not continue);
 *         tokens at offsets >= r0 use the reset fast weight W_down;
 *   l0    offset of the last document start inside the chunk (0 if none);
 *         tokens [l0, L) form the segment whose delta can carry on;
 *   carry 1 if chunk i+1 exists and does not begin with a document start.
 * table is a HOST array of B*N*3 int32.  Reset rule: iplexlaw review section 6. */
ipttt_status ipttt_segment_table(const ipttt_problem *p, int32_t *table);

/* Device-side version of the same table plus one descriptor byte per token:
 * table (device, B*N*3 int32, as above; may be NULL) and segs (device, B*T
 * uint8, required): bit 7 of segs[t] is set when token t starts a document
 * (row starts included) and segs[t] & 7 = min(5, end(t) - t) with
 * end(t) = min(chunk end, next document start, T), the number of conv taps
 * token t reads.  Every other call builds the same descriptors in its
 * workspace; this entry point exposes them. */
ipttt_status ipttt_segments_device(const ipttt_problem *p, int32_t *table, uint8_t *segs,
                                   void *stream);

/* Z = SiLU(H W_gate^T) * (H W_up^T)  (lijianxiong.blog, 高效的块状更新机制,
 * definition of the intermediate activation; phi = SiLU).
 *   H      [B*T, d]          W_gate, W_up [f, d]   (torch Linear layout)
 *   Z      [B*T, f]  out
 * One dual GEMM on the matrix cores with a fused SiLU*mul epilogue. */
ipttt_status ipttt_z(const ipttt_problem *p, const void *H, const void *W_gate,
                     const void *W_up, void *Z, void *stream);

/* ipttt_z that also keeps, for the backward, the two products before the
 * gate: GU [2, B*T, f] (dtype) out, G = H W_gate^T in GU[0], U = H W_up^T in
 * GU[1], each rounded once from its fp32 accumulator.  Caller-owned;
 * errors as ipttt_z (GU NULL: IPTTT_ERR_NULL). */
ipttt_status ipttt_z_save(const ipttt_problem *p, const void *H, const void *W_gate,
                          const void *W_up, void *Z, void *GU, void *stream);

/* V_hat = Conv1D(X0) W_target  (lijianxiong.blog, 对齐语言模型的目标函数;
 * tencent article 详细步骤 3; iplexlaw review section 6).  Depthwise conv with
 * k = 5 taps read forward and zero-padded at chunk ends and document starts:
 * Y[t, c] = sum_{k < wlen[t]} conv_w[c, k] X0[t+k, c];  V_hat = Y W_target.
 *   X0     [B*T, d]     conv_w [d, 5]     W_target [d_in = d, d_out = d]
 *   V      [B*T, d] out
 *   ws     workspace of ws_bytes >= ipttt_workspace_bytes(p)
 * With p->target = IPTTT_TARGET_NO_CONV, Y = X0 and conv_w may be NULL; with
 * IPTTT_TARGET_NO_PROJ, V_hat = Y and W_target may be NULL.                 */
ipttt_status ipttt_target(const ipttt_problem *p, const void *X0, const void *conv_w,
                          const void *W_target, void *V, void *ws, size_t ws_bytes, void *stream);

/* Clip scale of each chunk's carried delta (tencent article 详细步骤 4 note;
 * iplexlaw review section 6: Frobenius threshold).  For chunk i of row b, the
 * carried segment is tokens [l0, L) (see ipttt_segment_table) and
 *   n = |eta| * || V_hat_seg^T Z_seg ||_F,
 *   alpha[b*N + i] = tau / n if tau > 0 and n > tau, else 1.
 * The norm comes from the Gram identity ||V^T Z||_F^2 = <V V^T, Z Z^T>_F, so
 * the d x f delta is never formed.  With tau <= 0 alpha is all ones.
 *   V, Z      outputs of ipttt_target / ipttt_z
 *   alpha     [B*N] float out
 *   dW        NULL, or [B*N, d, f] float out: alpha * eta * V_hat_seg^T Z_seg
 *             materialised (diagnostic; large)                               */
ipttt_status ipttt_chunk_delta(const ipttt_problem *p, const void *V, const void *Z, float eta,
                               float tau, float *alpha, float *dW, void *ws, size_t ws_bytes,
                               void *stream);

/* Exclusive segmented scan of the fp32 fast-weight state fused with the
 * apply (lijianxiong.blog 步骤一/步骤二 and 工程实现; iplexlaw review sections 3
 * and 6): with S_0 = 0 and, per row,
 *   S_{i+1} = carry_i * ((r0_i == L_i ? S_i : 0) + alpha_i eta V_hat_seg^T Z_seg),
 *   O_[i][c] = Z_[i][c] (W_down + S_i)^T   for c <  r0_i,
 *   O_[i][c] = Z_[i][c]  W_down^T          for c >= r0_i.
 *   Z      [B*T, f]   V [B*T, d]   W_down [d, f]
 *   alpha  [B*N] float (from ipttt_chunk_delta)         O [B*T, d] out
 * A first kernel walks the chunks with the state tile resident in registers and
 * writes each chunk's effective weight W_down + S_i (dtype) to the workspace; a
 * second kernel applies them on the matrix cores.  On the bf16 path with d and
 * f multiples of 64, the state is cut into as many 256 x 256 tiles as the
 * device has CUs and 256 x 128 tiles for the rest; the environment variable
 * IPTTT_SCAN_CUS (a positive integer, read at each call) replaces that CU
 * count, for this call's forward scan and the backward's reverse scan alike.
 * The plan changes no result: both tile kinds accumulate every state element
 * in the same order. */
ipttt_status ipttt_scan_apply(const ipttt_problem *p, const void *Z, const void *V,
                              const void *W_down, const float *alpha, float eta, void *O,
                              void *ws, size_t ws_bytes, void *stream);

/* ipttt_scan_apply with the state carried across calls (the streamed reading
 * of one long sequence; the unrolled sum of lijianxiong.blog 工程实现 split at
 * a chunk boundary; document reset as in iplexlaw review section 6).  The
 * scan keeps S itself in fp32 (not W_down + S), so the state keeps full fp32
 * resolution however small it is next to W_down; each chunk applies the
 * weight W_down + S_i rounded to dtype once.
 *   S_in   [B, d, f] float (device) or NULL (zeros): row b of a problem with
 *          continues[b] set starts from S_0 = S_in[b]; other rows start
 *          from 0 and do not read S_in.
 *   S_out  [B, d, f] float out (device) or NULL: per row, the state of the
 *          document open at the row's end, after the update of the last
 *          chunk (whose delta the plain call never forms):
 *            S_out[b] = (r0 == L ? S_{N-1} : 0) + alpha eta V_hat_seg^T Z_seg
 *          for the last chunk N-1, its segment [l0, L) and alpha[b*N + N-1].
 *          S_out may equal S_in (updated in place); it must not overlap it
 *          otherwise.
 * The other arguments, the outputs O and the errors are those of
 * ipttt_scan_apply; with S_in = NULL and S_out = NULL the result equals
 * ipttt_scan_apply's up to the rounding of W_down + S.
 * Decode (tokens one at a time; the delta of a chunk lands once the chunk
 * is complete): each new token is a call over that token alone with
 * S_in = S and S_out = NULL (it applies W_down + S); when a chunk is
 * complete, one call over its C tokens with S_in = S_out = S folds its
 * clipped delta into S.  The outputs equal those of one call over the
 * whole sequence. */
ipttt_status ipttt_scan_apply_carry(const ipttt_problem *p, const void *Z, const void *V,
                                    const void *W_down, const float *alpha, float eta,
                                    const float *S_in, float *S_out, void *O, void *ws,
                                    size_t ws_bytes, void *stream);

/* ---------------------------------------------------------------- backward
 *
 * Reverse mode of the forward: given dO, the cotangent of O, the gradients
 * of <O, dO> with respect to every input, in three calls that mirror the
 * forward's in reverse order:
 *   ipttt_scan_apply_backward  dO -> dZ, dV (= d V_hat), dW_down
 *   ipttt_target_backward      dV -> dX0, dconv_w, dW_target
 *   ipttt_z_backward           dZ -> dH, dW_gate, dW_up
 * The pages train the layer further (lijianxiong.blog, 工程实现) but give no
 * gradient formulas; these are the chain rule through each forward step,
 * including the clip (the derivative of tau D/|D| where it applies) and the
 * document resets.  Rows flagged in `continues` start from a zero state, as
 * in ipttt_scan_apply; no gradient flows to a carried-in state.
 * Gradients of the dtype tensors come out in dtype; weight gradients are
 * float.  Every call is built on general batched MFMA products (any d, f
 * multiple of 8, fp32 or bf16).  One workspace of
 * ipttt_backward_workspace_bytes(p) (256-byte aligned) serves the three calls
 * in turn; the errors are those of the forward calls. */
size_t ipttt_backward_workspace_bytes(const ipttt_problem *p);

/* Gradients through the chunk deltas, their clip, the segmented scan and the
 * apply (the reverse of ipttt_chunk_delta + ipttt_scan_apply).
 *   Z [B*T, f], V [B*T, d]   the forward's intermediates
 *   W_down [d, f], eta, tau  as in the forward
 *   dO [B*T, d]              cotangent of O
 *   dZ [B*T, f] out, dV [B*T, d] out (dtype), dW_down [d, f] float out
 * The state adjoints G_i (the gradient with respect to the state chunk i
 * applies) run backwards: G_i = dO_head^T Z_head + (r0 == L and carry ?
 * G_{i+1} : 0), and chunk i's delta receives carry_i G_{i+1}. */
ipttt_status ipttt_scan_apply_backward(const ipttt_problem *p, const void *Z, const void *V,
                                       const void *W_down, float eta, float tau, const void *dO,
                                       void *dZ, void *dV, float *dW_down, void *ws, size_t ws_bytes,
                                       void *stream);

/* ------------------------------------------------------------ saved state
 *
 * A training step can keep, from the forward, what the scan/apply backward
 * would otherwise recompute: the per-chunk weights W_down + S_i that the scan
 * forms (dtype, in the library's internal fragment layout) and W_down in the
 * same layout.  The caller owns the buffer; its bytes are opaque.
 * ipttt_saved_bytes(p) is its size (0 for an invalid problem, and for the
 * shapes whose kernels keep no such state: fp32, or d or f not a multiple
 * of 64; there ipttt_scan_apply_save is ipttt_scan_apply and the saved
 * backward recomputes the weights). */
size_t ipttt_saved_bytes(const ipttt_problem *p);

/* ipttt_scan_apply that also leaves its per-chunk weights in `saved`
 * (saved_bytes >= ipttt_saved_bytes(p), 256-byte aligned; NULL allowed only
 * where ipttt_saved_bytes(p) is 0).  O and the errors are ipttt_scan_apply's. */
ipttt_status ipttt_scan_apply_save(const ipttt_problem *p, const void *Z, const void *V,
                                   const void *W_down, const float *alpha, float eta, void *O,
                                   void *saved, size_t saved_bytes, void *ws, size_t ws_bytes,
                                   void *stream);

/* ipttt_scan_apply_backward from the forward's own results instead of
 * recomputing them:
 *   alpha [B*N] float   the clip scales the forward applied (ipttt_chunk_delta's
 *                       output for the same Z, V, eta, tau); where a chunk was
 *                       clipped its delta norm is tau / (|eta| alpha)
 *   saved, saved_bytes  the buffer ipttt_scan_apply_save filled for the same
 *                       p, Z, V, W_down, alpha and eta, or NULL (recomputed)
 * The gradients equal ipttt_scan_apply_backward's up to rounding. */
ipttt_status ipttt_scan_apply_backward_saved(const ipttt_problem *p, const void *Z, const void *V,
                                             const void *W_down, float eta, float tau,
                                             const float *alpha, const void *saved,
                                             size_t saved_bytes, const void *dO, void *dZ,
                                             void *dV, float *dW_down, void *ws, size_t ws_bytes,
                                             void *stream);

/* Gradients through V_hat = Conv1D(X0) W_target and its ablations (p->target).
 *   dV [B*T, d]                   gradient of V_hat
 *   dX0 [B*T, d] out (dtype)
 *   dconv_w [d, 5] float out      (may be NULL with IPTTT_TARGET_NO_CONV)
 *   dW_target [d, d] float out    (may be NULL with IPTTT_TARGET_NO_PROJ)
 * conv_w and W_target may be NULL where the forward allows it. */
ipttt_status ipttt_target_backward(const ipttt_problem *p, const void *X0, const void *conv_w,
                                   const void *W_target, const void *dV, void *dX0, float *dconv_w,
                                   float *dW_target, void *ws, size_t ws_bytes, void *stream);

/* Gradients through Z = SiLU(H W_gate^T) * (H W_up^T); G = H W_gate^T and
 * U = H W_up^T are recomputed.
 *   dZ [B*T, f]                         gradient of Z
 *   dH [B*T, d] out (dtype)
 *   dW_gate, dW_up [f, d] float out */
ipttt_status ipttt_z_backward(const ipttt_problem *p, const void *H, const void *W_gate,
                              const void *W_up, const void *dZ, void *dH, float *dW_gate,
                              float *dW_up, void *ws, size_t ws_bytes, void *stream);

/* ipttt_z_backward from the G and U that ipttt_z_save kept for the same H,
 * W_gate and W_up (GU [2, B*T, f], not NULL) instead of recomputing them:
 * dG = dZ * U * SiLU'(G) and dU = dZ * SiLU(G) elementwise, then dH,
 * dW_gate and dW_up as in ipttt_z_backward.  The gradients equal
 * ipttt_z_backward's up to the dtype rounding of the saved G and U. */
ipttt_status ipttt_z_backward_saved(const ipttt_problem *p, const void *H, const void *W_gate,
                                    const void *W_up, const void *GU, const void *dZ, void *dH,
                                    float *dW_gate, float *dW_up, void *ws, size_t ws_bytes,
                                    void *stream);

/* ---- measurement aid (not a step of the method) --------------------------
 *
 * When a hook is set, every entry point calls hook(kernel, stream, user) on
 * the calling thread immediately before it enqueues each kernel (or group of
 * small kernels) on `stream`, with a short name: "gated_z", "segments",
 * "target_prep", "conv", "target_gemm", "gram_v", "gram", "alpha",
 * "scale_rows", "scan", "apply", and the backward's "rscan_fast", "nt",
 * "tn_fast", ...  A
 * profiler records a stream event in the hook and times each kernel between
 * consecutive events on the stream's own timeline.  The hook must not call
 * back into the library.  NULL (the default) disables it.  The setting is
 * process-wide: change it only while no other thread is inside the library. */
typedef void (*ipttt_launch_hook)(const char *kernel, void *stream, void *user);
void ipttt_set_launch_hook(ipttt_launch_hook hook, void *user);

/* ---- allocation-free variant -------------------------------------------
 *
 * For callers that cannot allocate device memory or hand over a workspace:
 * code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  ipttt_chunk_delta_noalloc computes exactly what
 * ipttt_chunk_delta computes with dW = NULL (the same kernels, the same clip
 * scales bit for bit), taking its scratch -- per-token segment bytes
 * (B*T), the segment table (B*N*3 int32) and the Gram partial sums (B*N times
 * the chunk's token-tile pairs, fp32), each region 256-byte aligned -- from
 * a static device array of IPTTT_NOALLOC_SCRATCH_BYTES that the library
 * holds on every GPU it runs on until the process ends.  It calls no
 * hipMalloc, hipFree or allocating library routine.
 *   V, Z, eta, tau, alpha, stream   as for ipttt_chunk_delta
 * Errors: as ipttt_chunk_delta (no workspace errors), and IPTTT_ERR_SCRATCH,
 * before any launch, when the scratch above exceeds the array.  The array of
 * a GPU is shared by every call on that GPU and keeps the last call's
 * contents (each call rewrites all it reads): calls that overlap on one GPU
 * (other streams, other threads) race and must be serialised by the caller. */
#define IPTTT_NOALLOC_SCRATCH_BYTES (8u << 20)
ipttt_status ipttt_chunk_delta_noalloc(const ipttt_problem *p, const void *V, const void *Z, float eta,
                                       float tau, float *alpha, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* IPTTT_H */
