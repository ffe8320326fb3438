/*
 * flce.h - fused linear + cross-entropy loss head for AMD Instinct MI355X
 * (CDNA4, gfx950): C ABI.
 *
 * The operation (page 2, "Liger-Kernel: Triton kernels that replace Hugging
 * Face training ops", section "What actually gets replaced, and how the patch
 * mechanism works"; page 3, "Complete Guide to Liger Kernel", section
 * "LigerFusedLinearCrossEntropyLoss"): given hidden states h[N,H], the
 * LM-head weight W[V,H] and class labels t[N], return the cross-entropy loss
 * of the logits h W^T directly, without a [N,V] logit tensor, together with
 * its gradients (page 1, "Liger Kernel explained", section "What does Liger
 * Kernel actually fuse, and why does that cut memory?": loss and gradient
 * are produced in the same pass, working through the logits in chunks).
 *
 *   Z      = h W^T                                   (never resident whole)
 *   loss   = (1/N) sum_i ( logsumexp_j Z_ij - Z_{i,t_i} )
 *   G      = (softmax(Z) - onehot(t)) / N
 *   grad_h = G W,     grad_W = G^T h
 *
 * Conventions shared by every entry point:
 *  - Every pointer is a DEVICE pointer unless stated otherwise; arrays are
 *    row-major and contiguous; the caller allocates and owns every buffer.
 *  - Work is enqueued on `stream` (a hipStream_t; NULL is the legacy default
 *    stream).  No call synchronises, allocates device memory, or reads
 *    device data on the host; results are valid once the stream has
 *    completed.  Calls on different streams are independent when their
 *    output and workspace buffers are distinct.
 *  - Arguments are checked on the host before anything is enqueued; a
 *    failed check returns a status and enqueues nothing.
 *  - Requirements: H % 8 == 0 and 16-byte aligned h, W, grad_h, grad_W and
 *    workspace (FLCE_ERR_UNSUPPORTED otherwise); all sizes below 2^31 and
 *    N, H, V, chunk >= 1 (FLCE_ERR_INVALID_ARG otherwise).  A chunk whose
 *    logits or hidden rows would exceed 2^56 elements is FLCE_ERR_UNSUPPORTED
 *    (the workspace functions return 0 for it), so every size and offset is
 *    exact in 64-bit arithmetic.
 *  - Targets must lie in [0, V).  An out-of-range target is not read
 *    through: it makes that token's loss, and so the returned loss, NaN.
 */
#ifndef FLCE_H_
#define FLCE_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Storage type of h, W and grad_h.  grad_W and the loss are always fp32. */
typedef enum flce_dtype {
  FLCE_BF16 = 0, /* bfloat16: MFMA contractions, fp32 accumulation      */
  FLCE_F32 = 1   /* float32 operands and fp32 gradient of the logits    */
} flce_dtype;

typedef enum flce_status {
  FLCE_OK = 0,
  FLCE_ERR_INVALID_ARG = 1, /* null pointer, size < 1 or >= 2^31, bad dtype */
  FLCE_ERR_WORKSPACE = 2,   /* workspace smaller than flce_workspace_bytes   */
  FLCE_ERR_UNSUPPORTED = 3, /* H % 8 != 0, a pointer not 16-byte aligned,
                               or a shape the entry point does not run    */
  FLCE_ERR_HIP = 4,         /* the HIP runtime reported a launch error       */
  FLCE_ERR_SCRATCH = 5      /* flce_fwd_bwd_noalloc: the sizes need more
                               workspace than FLCE_NOALLOC_SCRATCH_BYTES    */
} flce_status;

/* Size of the static device scratch flce_fwd_bwd_noalloc works in. */
#define FLCE_NOALLOC_SCRATCH_BYTES ((size_t)512 << 20)

/*
 * Bytes of device workspace flce_fwd_bwd needs, with C = min(chunk, N);
 * never more than C * V * 4 (the fp32 logits of one chunk; the logits of
 * all N tokens would take N * V * 4):
 *   bf16 inputs, H % 64 == 0, V % 8 == 0, H and V below 2^22:
 *        C * V * 2 + C * ceil(V / 128) * 8   (the logits of one token chunk
 *        kept as bf16 exponentials, plus two floats per row and 128-column
 *        slice; each region rounded up to 256 bytes)
 *        + P * H * 4 when the grad_h product of a chunk of r rows (H x r,
 *        in tiles of 256 x 256) would leave the 256 CUs partly idle: its
 *        K = V contraction is split into s fp32 parts, s in {1, 2, 4, 8}
 *        minimising ceil(tiles * s / 256) / s / (tiles / 256) + 560 s / V
 *        (rounds of the chip over a perfect fill, plus the pass summing the
 *        parts; s = 1 adds nothing), with V % 64 == 0, V >= 1024 s and the
 *        parts within what remains of C * V * 4 bytes; P is the larger of
 *        s * r over r = C and r = N mod C (e.g. 2 parts at H = 4096 and
 *        2048 rows, 4 at 1024 rows, 8 at H = 3584 and 4096 rows)
 *        (when the two regions alone would exceed C * V * 4, a handful of
 *        rows of a tiny vocabulary, the second form is used)
 *   otherwise:
 *        C * V * 4                           (the fp32 logits of one chunk)
 * Returns 0 when a size is < 1.  Pure host function.
 */
size_t flce_workspace_bytes(int64_t N, int64_t H, int64_t V, int64_t chunk,
                            flce_dtype dt);

/*
 * Forward and backward of the fused head in one call.
 *
 *  h          [N, H]  dt     hidden states (read only)
 *  W          [V, H]  dt     LM-head weight, nn.Linear layout (read only)
 *  targets    [N]     int32  class of each token, 0 <= t < V (read only)
 *  chunk             tokens whose logits are live at once (clamped to N)
 *  loss       [1]     fp32   overwritten with the mean token loss
 *  grad_h     [N, H]  dt     overwritten with dloss/dh
 *  grad_W     [V, H]  fp32   overwritten with dloss/dW (fp32 accumulation
 *                            over token chunks)
 *  workspace                 >= flce_workspace_bytes(N, H, V, chunk, dt)
 *                            bytes of scratch, contents undefined on return
 *
 * The gradients are those of the mean loss with an upstream gradient of 1.
 * Outputs must not alias inputs, the workspace or each other.
 * Returns FLCE_OK once everything is enqueued.
 */
flce_status flce_fwd_bwd(const void* h, const void* W, const int32_t* targets,
                         int64_t N, int64_t H, int64_t V, int64_t chunk,
                         float* loss, void* grad_h, float* grad_W,
                         void* workspace, size_t workspace_bytes,
                         flce_dtype dt, hipStream_t stream);

/*
 * flce_fwd_bwd for gradient accumulation over micro-batches (page 3,
 * "Complete Guide to Liger Kernel", the training-loop example: the loss of
 * each micro-batch is backpropagated and the optimizer steps every few
 * micro-batches): identical, except that grad_W is ADDED to, i.e. on
 * return grad_W = (its previous contents) + dloss/dW, accumulated in fp32
 * from the first token chunk on.  loss and grad_h are overwritten as in
 * flce_fwd_bwd.  grad_W must hold initialised values.
 */
flce_status flce_fwd_bwd_accumulate(const void* h, const void* W, const int32_t* targets,
                                    int64_t N, int64_t H, int64_t V, int64_t chunk,
                                    float* loss, void* grad_h, float* grad_W,
                                    void* workspace, size_t workspace_bytes,
                                    flce_dtype dt, hipStream_t stream);

/*
 * Multiplies precomputed gradients in place by the upstream gradient of
 * the loss, for a backward pass whose loss was scaled after the fused call
 * (page 3's training loop divides it by the accumulation steps):
 *   grad_h[0 .. n_h) *= *scale   (dt; bf16 rounded to nearest even)
 *   grad_W[0 .. n_W) *= *scale   (fp32)
 * scale is a DEVICE pointer to one fp32 value, read by the kernel, so the
 * host never synchronises to learn it.  A buffer with n = 0 may be null;
 * non-null buffers must be 16-byte aligned (FLCE_ERR_UNSUPPORTED),
 * negative counts or a null scale give FLCE_ERR_INVALID_ARG.
 */
flce_status flce_scale_grads(void* grad_h, int64_t n_h, float* grad_W, int64_t n_W,
                             const float* scale, flce_dtype dt, hipStream_t stream);

/*
 * Steps flce_fwd_bwd runs for these sizes: FLCE_STEPS per token chunk,
 * i.e. FLCE_STEPS * ceil(N / min(chunk, N)).  0 if a size is < 1.  A step
 * is one or two kernel launches (on the exponentiated bf16 path the row
 * step is a statistics launch and a rewrite launch, and a K-split grad_h
 * adds a summing launch).
 */
#define FLCE_STEPS 5
int64_t flce_launch_count(int64_t N, int64_t chunk);

/*
 * flce_fwd_bwd that also records, on `stream`, events[2k] just before and
 * events[2k + 1] just after its k-th step, so a caller can time each step
 * with hipEventElapsedTime.  Step k belongs to token chunk k / FLCE_STEPS
 * and is step k % FLCE_STEPS of that chunk: 0 logits GEMM,
 * 1 row log-sum-exp + gradient rewrite, 2 loss sum, 3 grad_h GEMM,
 * 4 grad_W GEMM.  `events` is a HOST array of n_events handles the caller
 * created (hipEventCreate) and owns; n_events must be at least
 * 2 * flce_launch_count(N, chunk) (FLCE_ERR_INVALID_ARG otherwise).  The
 * computation and every other rule are those of flce_fwd_bwd.
 */
flce_status flce_fwd_bwd_timed(const void* h, const void* W, const int32_t* targets,
                               int64_t N, int64_t H, int64_t V, int64_t chunk,
                               float* loss, void* grad_h, float* grad_W,
                               void* workspace, size_t workspace_bytes,
                               flce_dtype dt, hipStream_t stream,
                               hipEvent_t* events, int64_t n_events);

/*
 * Step 1 alone: the logits of `rows` tokens, z[i * ldz + j] = sum_k
 * h[i, k] W[j, k] in fp32 (MFMA, fp32 accumulation), for 0 <= i < rows,
 * 0 <= j < V.  ldz >= V, in floats; z must be 16-byte aligned and, for the
 * vectorised path, ldz % 4 == 0.  Same alignment rules as flce_fwd_bwd.
 */
flce_status flce_logits(const void* h, const void* W, int64_t rows, int64_t H,
                        int64_t V, float* z, int64_t ldz, flce_dtype dt,
                        hipStream_t stream);

/*
 * Steps 2-3 alone, on given fp32 logits (cross entropy with the gradient
 * written in place, page 3 section "LigerCrossEntropyLoss"): for each of
 * `rows` rows of z (pitch ldz floats, ldz >= V), computes
 *   row_loss[i] = logsumexp_j z[i, j] - z[i, t_i]
 * and rewrites the row in place as
 *   G[i, j] = (exp(z[i, j] - lse_i) - [j == t_i]) * scale,
 * stored as dt: for FLCE_F32 at the same positions; for FLCE_BF16 as bf16
 * (round to nearest even) at element offset i * 2 * ldz + j of
 * (uint16_t*)z, i.e. in the first half of the row's own bytes.
 * row_loss [rows] fp32 is written with a stride of loss_stride floats.
 * scale is the upstream factor (1/N for a mean over N tokens).
 */
flce_status flce_ce_rows(float* z, int64_t ldz, const int32_t* targets,
                         int64_t rows, int64_t V, float scale,
                         float* row_loss, int64_t loss_stride, flce_dtype dt,
                         hipStream_t stream);

/*
 * Cross entropy on given logits, the gradient written over them (page 3,
 * "Complete Guide to Liger Kernel", section "LigerCrossEntropyLoss": the
 * loss of [B*S, V] logits against labels, computed chunk-wise with the
 * gradient formed in the same pass): for the `rows` rows of `logits`
 * (dt: bf16 or fp32, row pitch ld >= V elements)
 *   *loss      = (1/rows) sum_i (logsumexp_j z[i, j] - z[i, t_i])   (fp32)
 *   row_loss[i] = logsumexp_j z[i, j] - z[i, t_i]   [rows] fp32, caller-owned
 *   z[i, j]   <- (softmax(z[i, :])_j - [j == t_i]) / rows, in place, same
 *               dtype and positions (bf16 rounded to nearest even)
 * i.e. the logits become dloss/dlogits of the mean loss.  Two passes over
 * each row (max / sum, then the rewrite): bf16 rows that start 16-byte
 * aligned (ld % 8 == 0) take one 512-thread workgroup per row, other bf16
 * rows and fp32 rows one wave64 per row; the mean is summed in fp64 in a
 * fixed order.  logits must be aligned to its element size (fp32 rows
 * 16-byte aligned with ld % 4 == 0 take a vector path); targets 0 <= t < V (an out-of-range target is
 * never dereferenced and makes the loss NaN).  Null pointers or bad sizes
 * give FLCE_ERR_INVALID_ARG, misalignment FLCE_ERR_UNSUPPORTED.
 */
flce_status flce_cross_entropy(void* logits, int64_t ld, const int32_t* targets,
                               int64_t rows, int64_t V, float* loss, float* row_loss,
                               flce_dtype dt, hipStream_t stream);

/*
 * The fused head behind an RMSNorm of its input (page 3, "Complete Guide to
 * Liger Kernel", section "LigerRMSNorm"; the epsilon convention of page 2,
 * section "The support surface is narrower than the pitch suggests", is eps
 * added to the mean square):
 *   r_i    = 1 / sqrt(mean_k x[i, k]^2 + eps)
 *   h      = x * r * gamma           (per row; rounded once to dt)
 * followed by flce_fwd_bwd on h, and the chain rule back through the norm:
 *   grad_x[i, k]  = r_i gamma_k g[i, k] - x[i, k] r_i^3 / H sum_k gamma_k g[i, k] x[i, k]
 *   grad_gamma[k] = sum_i g[i, k] x[i, k] r_i
 * with g = dloss/dh.  Each token chunk is normalised into the workspace just
 * before its logits and the norm's backward runs right after the chunk's
 * gradients, so h and dloss/dh exist for one chunk at a time.
 *
 *  x          [N, H]  dt     pre-norm hidden states (read only)
 *  gamma      [H]     dt     norm weight (read only, 16-byte aligned)
 *  eps               fp32   >= 0 and finite (FLCE_ERR_INVALID_ARG otherwise);
 *                            with eps = 0 an all-zero row gives a non-finite
 *                            result
 *  W, targets, N, H, V, chunk, loss, grad_W, stream: as flce_fwd_bwd
 *  grad_x     [N, H]  dt     overwritten with dloss/dx
 *  grad_gamma [H]     fp32   overwritten with dloss/dgamma (4-byte aligned)
 *  workspace                 >= flce_rmsnorm_workspace_bytes(N, H, V, chunk, dt)
 * The gradients are those of the mean loss with an upstream gradient of 1.
 */
flce_status flce_fwd_bwd_rmsnorm(const void* x, const void* gamma, float eps, const void* W,
                                 const int32_t* targets, int64_t N, int64_t H, int64_t V,
                                 int64_t chunk, float* loss, void* grad_x, float* grad_gamma,
                                 float* grad_W, void* workspace, size_t workspace_bytes,
                                 flce_dtype dt, hipStream_t stream);

/*
 * Bytes of workspace flce_fwd_bwd_rmsnorm needs, with C = min(chunk, N) and
 * es the element size of dt: flce_workspace_bytes(N, H, V, chunk, dt), then
 * (each region starting on a 256-byte boundary) C * H * es for the chunk's
 * h, C * H * es for its dloss/dh, C * 4 for the per-row 1/rms, and
 * ceil(C / 64) * H * 4 for the grad_gamma partial sums.  0 when a size is
 * < 1.  Pure host function.
 */
size_t flce_rmsnorm_workspace_bytes(int64_t N, int64_t H, int64_t V, int64_t chunk,
                                    flce_dtype dt);

/*
 * Vocabulary-chunked variant of flce_fwd_bwd (page 1, "Liger Kernel
 * explained", section "What does Liger Kernel actually fuse, and why does
 * that cut memory?": the logits are worked through in chunks over the
 * vocabulary dimension), for few tokens and a large vocabulary, where token
 * chunks would be short.  All N tokens are processed together and the
 * vocabulary in column chunks of Vc = min(vchunk, V):
 *   pass 1  the logits of every column chunk are formed only for their
 *           per-row (max, sum of exponentials) statistics, which give every
 *           row's log-sum-exp and loss;
 *   pass 2  each chunk's logits are formed again and become
 *           G = (softmax - onehot) / N with the global log-sum-exp; then
 *           grad_h += G W_c (fp32 accumulator in the workspace) and
 *           grad_W[chunk rows] = G^T h.
 * The logits are computed twice (8 N V H flops instead of 6 N V H).  The
 * arguments, outputs and rules are those of flce_fwd_bwd with `vchunk` in
 * place of `chunk`; loss, grad_h and grad_W are overwritten.
 * Supported: FLCE_BF16, H % 64 == 0, V % 64 == 0, vchunk >= V or
 * vchunk % 128 == 0, H and V below 2^22; otherwise FLCE_ERR_UNSUPPORTED
 * (flce_fwd_bwd covers every shape).
 */
flce_status flce_fwd_bwd_vocab(const void* h, const void* W, const int32_t* targets,
                               int64_t N, int64_t H, int64_t V, int64_t vchunk,
                               float* loss, void* grad_h, float* grad_W,
                               void* workspace, size_t workspace_bytes,
                               flce_dtype dt, hipStream_t stream);

/*
 * Bytes of device workspace flce_fwd_bwd_vocab needs, with Vc = min(vchunk,
 * V), each region rounded up to 256 bytes:
 *   N * Vc * 2            bf16 logits of one vocabulary chunk
 * + N * ceil(V/128) * 8   (max, sum) per row and 128-column slice
 * + N * 16                per-row log-sum-exp, p_t - 1, loss and the
 *                         mass of the target's 128-column slice
 * + N * H * 4             fp32 grad_h accumulator
 * Returns 0 when a size is < 1 or the shape is not supported by this entry
 * point.  Pure host function.
 */
size_t flce_vocab_workspace_bytes(int64_t N, int64_t H, int64_t V, int64_t vchunk,
                                  flce_dtype dt);

/*
 * Odds-ratio preference (ORPO) loss over the same head.  Page 2,
 * "Liger-Kernel: Triton kernels that replace Hugging Face training ops",
 * section "Installation and the one-line patch", lists ORPO among the chunked
 * post-training losses called with the LM-head weight, the hidden states
 * and the targets that return the loss itself; the pages give no formula,
 * so the objective is the published one of ORPO (Hong, Lee and Thorne,
 * 2024):
 *   rows       N = 2 * pairs * seq_len rows of h [N, H] and targets [N]:
 *              sequence s = row / seq_len; sequences [0, pairs) are the
 *              chosen responses, [pairs, 2 pairs) the rejected ones, pair b
 *              = (b, pairs + b)
 *   counted    a row counts when its target is >= 0; a negative target
 *              marks a prompt or padding row (no loss, zero gradient row)
 *   l_s        mean of log softmax(h_r W^T)[t_r] over the counted rows of s
 *              (each log p formed as -ln(1 + S), S the other classes' mass
 *              relative to the target's from the fp32 logits, so 1 - exp(l)
 *              keeps its relative precision for a confident model; a
 *              sequence whose every token has S below fp32's range, logit
 *              margins beyond about 100, counts as certain: l = 0, which
 *              leaves finite terms for a chosen sequence and an infinite
 *              loss for a rejected one, the objective's own limits)
 *   loss       -(1/M) sum over counted chosen rows of log p
 *              + beta * (1/pairs) sum_b ln(1 + exp(-(lo_b - lo_{pairs+b})))
 *              with lo_s = l_s - ln(1 - exp(l_s)) and M the counted chosen
 *              rows of the batch
 * Outputs (overwritten): *loss; seq_logp[2 pairs] = l_s (optional, may be
 * NULL); grad_h [N, H] bf16 = dloss/dh; grad_W [V, H] fp32 = dloss/dW.
 * The batch is processed in chunks of min(chunk_pairs, pairs) pairs, each
 * pair's two sequences in the same chunk; the logits of one chunk are the
 * only [rows, V] array.  A sequence with no counted row, or a target >= V,
 * makes the loss NaN (targets are never read on the host).
 * Supported: FLCE_BF16 with H % 64 == 0, V % 8 == 0 and H and V below 2^22;
 * otherwise FLCE_ERR_UNSUPPORTED.  FLCE_ERR_INVALID_ARG for a null required
 * pointer, pairs, seq_len or chunk_pairs < 1, more than 2^31 - 1 rows, a
 * chunk of logits or hidden rows beyond 2^56 elements, or a beta that is not
 * finite.  Alignment, workspace and stream rules as
 * flce_fwd_bwd (seq_logp 4-byte aligned).
 */
flce_status flce_orpo_fwd_bwd(const void* h, const void* W, const int32_t* targets,
                              int64_t pairs, int64_t seq_len, int64_t H, int64_t V,
                              int64_t chunk_pairs, float beta, float* loss, float* seq_logp,
                              void* grad_h, float* grad_W, void* workspace,
                              size_t workspace_bytes, flce_dtype dt, hipStream_t stream);

/*
 * Bytes of device workspace flce_orpo_fwd_bwd needs, with R = 2 * Pc *
 * seq_len rows per chunk (Pc = min(chunk_pairs, pairs)), each region
 * rounded up to 256 bytes:
 *   R * V * 2             bf16 logits of one chunk
 * + R * ceil(V/128) * 8   (max, sum) per row and 128-column slice
 * + K-split rows * H * 4  fp32 grad_h parts when a chunk has few H x R tiles
 * + R * 20                per-row log-sum-exp, p_t - 1, loss, scale and the
 *                         mass of the target's 128-column slice
 * + 2 * R * H * 2         the chunk's h rows and grad_h rows
 * + R * 4                 the chunk's targets
 * + pairs * 8             per-pair loss terms
 * + 256                   the count of counted chosen rows
 * Returns 0 when an argument is invalid or the shape unsupported.  Pure
 * host function.
 */
size_t flce_orpo_workspace_bytes(int64_t pairs, int64_t seq_len, int64_t H, int64_t V,
                                 int64_t chunk_pairs, flce_dtype dt);

/*
 * Matrix-core rate microbenchmark.  This is a measurement aid, not a step
 * of the loss: it gives the bf16 MFMA rate and shader clock the part
 * sustains when it runs the contractions' instruction stream with no memory
 * traffic.  The loss head's GEMMs are compared against that ceiling as well
 * as against the published dense peak.
 *
 * It launches `workgroups` workgroups of 4 waves, one wave per SIMD as in
 * the head's GEMMs.  Each wave loads eight 16-byte operand fragments once.
 * Lane l of wave w reads the 128-byte group g = (w*64 + l) mod G, where
 * G = min(floor(operand_bytes / 128), 2^30); the group's pieces 0-3 are its
 * A fragments and pieces 4-7 its B fragments.  It then runs `iters`
 * rounds of the 4 x 4 products acc[i][j] += A_i B_j^T, each one
 * v_mfma_f32_32x32x16_bf16: 32x16 by 16x32 blocks, with lane l holding
 * row (or column) l % 32 and k = 8*(l/32) .. 8*(l/32)+7 of its block.
 * One call performs workgroups * 4 * iters * 16 * 32768 flop.
 * Outputs, per wave w = 4 * workgroup + wave index:
 *   sink[w]          fp32 sum, over the wave's 64 lanes and 16 blocks, of
 *                    each lane's element 0 of the block: row 4*(l/32),
 *                    column l % 32 of that block's 32x32 result;
 *   clocks[2w]       shader clocks the wave spent in its loop (s_memtime);
 *   clocks[2w + 1]   ticks of the constant-rate reference counter
 *                    (s_memrealtime, 100 MHz) over the same interval.
 *                    Their ratio is the wave's clock.
 * Requires: operands 16-byte aligned with operand_bytes >= 8192 and a
 * multiple of 16; sink [4 * workgroups] fp32 (4-byte aligned); clocks
 * [8 * workgroups] uint64 (8-byte aligned); 1 <= iters <= 2^40;
 * 1 <= workgroups <= 65535.  Otherwise it returns INVALID_ARG or
 * UNSUPPORTED and enqueues nothing.
 */
flce_status flce_mfma_rate(const void* operands, int64_t operand_bytes, int64_t iters,
                           int64_t workgroups, float* sink, uint64_t* clocks,
                           hipStream_t stream);

/* A static, human-readable name for a status code (host only). */
/*
 * flce_fwd_bwd for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments, results and rules as flce_fwd_bwd, minus the workspace:
 * the call works in a static device array of FLCE_NOALLOC_SCRATCH_BYTES
 * that the library holds on every GPU it runs on until the process ends.
 * Its address on a device is looked up once, on the first call whose
 * `stream` belongs to that device (the current device for the null
 * stream), with that device made current for the lookup and the caller's
 * current device restored; no call makes a hipMalloc, hipFree or other
 * allocation.
 *  - Returns FLCE_ERR_SCRATCH, enqueuing nothing, when
 *    flce_workspace_bytes(N, H, V, chunk, dt) exceeds
 *    FLCE_NOALLOC_SCRATCH_BYTES (use a smaller chunk: the Llama-3-8B head,
 *    H = 4096 and V = 128256, fits chunks of up to 1024 tokens).
 *  - Every call on one GPU shares that GPU's array: calls that overlap in
 *    time on one GPU (other streams, other host threads) race and give
 *    undefined results.  Calls serialised on one stream are safe; the
 *    array needs no clearing between calls (every byte a call reads it
 *    has written first).
 *  - FLCE_ERR_HIP when the array's address cannot be obtained.
 * This entry point keeps the per-device address as global state, unlike
 * the others.
 */
flce_status flce_fwd_bwd_noalloc(const void* h, const void* W, const int32_t* targets,
                                 int64_t N, int64_t H, int64_t V, int64_t chunk,
                                 float* loss, void* grad_h, float* grad_W,
                                 flce_dtype dt, hipStream_t stream);

const char* flce_status_string(flce_status s);

#ifdef __cplusplus
}
#endif

#endif /* FLCE_H_ */
