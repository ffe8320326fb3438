// Internal launch helpers of the fused linear + cross-entropy library.
// Not part of the public ABI (include/flce.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace flce {

// Contraction D[m][n] = sum_k A(m, k) * B(n, k), stored transposed as
// out[n * ldo + m] (each lane of an MFMA output tile then holds runs of
// consecutive m, which become vector stores).
//   A(m, k) = a_kc ? A[m * lda + k] : A[k * lda + m]
//   B(n, k) = b_kc ? B[n * ldb + k] : B[k * ldb + n]
// "kc" means the contraction index is the contiguous one.
enum Epilogue : int {
  kStoreF32 = 0,   // out (fp32) = D
  kStoreOut = 1,   // out (operand dtype: bf16 or fp32) = D
  kAccumF32 = 2,   // out (fp32) = D + (beta ? out : 0)
  // Exponentiated logits (direct-to-LDS kernel, k/k operands only): with
  // y = D * log2(e) and, per output column n and 128-row half tile q of m,
  // mx = max of y over the half tile's rows m < M:
  //   out (bf16) = 2^(y - mx)
  //   row_part[n * ldp + 2q] = mx,  row_part[n * ldp + 2q + 1] = sum of 2^(y - mx)
  kExpBF16 = 3,
};

// Rows of m per (max, sum) pair of the kExpBF16 epilogue.
constexpr int kHalfTile = 128;

struct GemmArgs {
  const void* A;
  int64_t lda;
  const void* B;
  int64_t ldb;
  void* out;
  int64_t ldo;
  int M, N, K;
  int beta;
  // Tile order (direct-to-LDS kernel): tiles are walked in groups of
  // group_m row panels (m fastest inside a group); 0 picks a default.
  int group_m = 0;
  // K-start rotation per tile group: group g starts its K walk at slab
  // (g * stagger) mod (K / 64); 0 disables it.
  int stagger = 0;
  // (max, sum) pairs of the kExpBF16 epilogue; ldp in floats.
  float* row_part = nullptr;
  int64_t ldp = 0;
  // K split (direct-to-LDS kernel): the K slabs are cut into `splits`
  // consecutive parts; part s is computed by its own workgroups and stored
  // at out + s * split_stride (elements), to be summed by the caller.
  int splits = 1;
  int64_t split_stride = 0;
};

// Whether a grid of ceil(M/bm) * ceil(N/bn) tiles (times `parts`) fits the
// int tile indices the kernels use (launchers return hipErrorInvalidValue
// otherwise).
inline bool tile_count_ok(int M, int N, int bm, int bn, int parts) {
  const int64_t t = (int64_t)((M + bm - 1) / bm) * ((N + bn - 1) / bn) * (parts > 1 ? parts : 1);
  return t <= 0x7fffffff;
}

// bf16 operands, MFMA 32x32x16, fp32 accumulation.  `vec` selects the
// 16-byte load/store path, valid when every dimension that is contiguous in
// memory (and every leading dimension) is a multiple of 8 elements and the
// base pointers are 16-byte aligned.
hipError_t launch_gemm_bf16(bool a_kc, bool b_kc, int epi, bool vec,
                            const GemmArgs& g, hipStream_t s);

// The same bf16 contraction through the direct-to-LDS pipeline of
// gemm_bf16_dma.hip; valid when gemm_bf16_dma_supported() holds.
bool gemm_bf16_dma_supported(bool a_kc, bool b_kc, const GemmArgs& g);
// True when launch_gemm_bf16 with these arguments runs the direct-to-LDS
// kernel (the only one with the kExpBF16 epilogue).
bool gemm_bf16_uses_dma(bool a_kc, bool b_kc, bool vec, const GemmArgs& g);
hipError_t launch_gemm_bf16_dma(bool a_kc, bool b_kc, int epi, const GemmArgs& g,
                                hipStream_t s);

// fp32 operands, same index semantics (used by FLCE_F32).
hipError_t launch_gemm_f32(bool a_kc, bool b_kc, int epi, const GemmArgs& g,
                           hipStream_t s);

// Cross entropy of `rows` fp32 logit rows with the gradient rewritten in
// place (bf16 at pitch 2*ldz elements, or fp32 at pitch ldz).
hipError_t launch_ce_rows(float* z, int64_t ldz, const int32_t* targets,
                          int rows, int V, float scale, float* row_loss,
                          int64_t loss_stride, bool out_bf16, hipStream_t s);

// The same on bf16 logits at pitch ldz elements, rewritten in place as the
// bf16 gradient (same positions).
hipError_t launch_ce_rows_bf16(uint16_t* z, int64_t ldz, const int32_t* targets, int rows,
                               int V, float scale, float* row_loss, int64_t loss_stride,
                               hipStream_t s);

// The same from exponentiated logits (kExpBF16 output u at pitch ldu, with
// its (max, sum) pairs): u is rewritten in place as the bf16 gradient.  The
// target logit of row i is recomputed as the dot product of h[i] and
// W[targets[i]] (bf16 rows of H elements, fp32 accumulation); the row loss
// is ln(1 + S) with S = sum over j != t of exp(z_j - z_t), formed from the
// other half tiles' pairs and the target's half tile's u values without the
// target (positive terms only), and G[i, t] = -S / (1 + S) * scale.  Two
// launches: the row statistics, staged per row as loss, lse2 and pt1 at
// row_loss[i * loss_stride + 0, 1, 2] (loss_stride >= 3), then the
// elementwise rewrite in memory order.
hipError_t launch_ce_rows_exp(uint16_t* u, int64_t ldu, const float* row_part, int64_t ldp,
                              const uint16_t* h, const uint16_t* W, int H,
                              const int32_t* targets, int rows, int V, float scale,
                              float* row_loss, int64_t loss_stride, hipStream_t s);

// Split form of the same (vocabulary chunks, preference loss).
//   ce_target_mass: for a chunk [v0, v0 + n) of columns (v0 % 128 == 0; u
//     rows at pitch ldu hold the chunk's columns from 0), every row whose
//     target falls in the chunk gets rt[row] = the sum of u over its
//     target's half tile without the target.
//   ce_stats_exp: once every chunk's pairs (row pitch ldp floats,
//     2 * ceil(V / 128) used) and rt exist: per row lse2 over all V columns,
//     pt1 = p_t - 1 and row_loss = ln(1 + S) = -log p_t, [rows] each.  A
//     row whose target is outside [0, V) gets the log-sum-exp of all
//     columns, pt1 = 0 and a NaN loss.
hipError_t launch_ce_target_mass(const uint16_t* u, int64_t ldu, const int32_t* targets,
                                 int rows, int v0, int n, float* rt, hipStream_t s);
hipError_t launch_ce_stats_exp(const float* row_part, int64_t ldp, const float* rt,
                               const uint16_t* h, const uint16_t* W, int H,
                               const int32_t* targets, int rows, int V, float* lse2, float* pt1,
                               float* row_loss, hipStream_t s);
// Vocabulary-chunked path, gradient of columns [v0, v0 + n) (v0 % 128 == 0,
// n % 8 == 0): u (row pitch ldu) -> (u 2^(mx_q - lse2) - [j == t]) * scale
// in place, the target's element (when it falls in the chunk) being
// pt1 * scale; row_part points at the chunk's first pair of row 0.  A
// non-null row_scale gives each row its own scale (any sign) in place of
// `scale`.
hipError_t launch_ce_rewrite_exp(uint16_t* u, int64_t ldu, const float* row_part, int64_t ldp,
                                 const float* lse2, const float* pt1, const int32_t* targets,
                                 int rows, int v0, int n, float scale, const float* row_scale,
                                 hipStream_t s);

// Odds-ratio preference loss (orpo.hip).  Rows of a batch of 2B sequences of
// T tokens: sequences [0, B) chosen, [B, 2B) rejected; a negative target
// marks a row that does not count.
//   orpo_count: *count = number of rows r < n with targets[r] >= 0.
//   orpo_coef:  for the Pc pairs [p0, p0 + Pc) staged as one chunk (chosen
//     rows [0, Pc T), rejected rows [Pc T, 2 Pc T), with each row's
//     -log p_t from launch_ce_stats_exp in row_loss): each row's gradient scale
//     c = -dloss/dlog p (0 for rows that do not count) into coef, each
//     sequence's mean log-probability into seq_logp[p] and seq_logp[B + p]
//     (when non-null), and per pair the chosen rows' -sum log p and the
//     odds-ratio term ln(1 + exp(-ratio)) into stage[2p], stage[2p + 1].
//   orpo_loss:  *loss = sum_p stage[2p] / count + beta / B sum_p stage[2p+1],
//     fixed-order fp64 sums.
hipError_t launch_orpo_count(const int32_t* targets, int64_t n, int* count, hipStream_t s);
hipError_t launch_orpo_coef(const float* row_loss, const int32_t* targets, int Pc,
                            int T, int B, int p0, float beta, const int* count, float* coef,
                            float* seq_logp, float* stage, hipStream_t s);
hipError_t launch_orpo_loss(const float* stage, int B, float beta, const int* count, float* loss,
                            hipStream_t s);

// RMSNorm in front of the head (rmsnorm.hip), one wave per row, H % 8 == 0,
// 16-byte aligned rows: h = x * r * gamma with r = 1/sqrt(mean x^2 + eps)
// (r stored per row in rinv), and its backward from g = dloss/dh: grad_x
// rows, and grad_gamma (fp32 [H]) = (first ? 0 : grad_gamma) + sum_i
// g_i * x_i * r_i through `part` (rmsnorm_groups(rows) * H floats).
int rmsnorm_groups(int rows);
hipError_t launch_rmsnorm_fwd(const void* x, const void* gamma, float eps, int rows, int H,
                              void* h, float* rinv, bool bf16, hipStream_t s);
hipError_t launch_rmsnorm_bwd(const void* x, const void* gamma, const void* g, const float* rinv,
                              int rows, int H, void* grad_x, float* part, float* grad_gamma,
                              int first, bool bf16, hipStream_t s);

// out[i] = bf16(sum over s < S of parts[s * stride + i]) for i < n, summed
// in the order s = 0, 1, ... (deterministic); parts and out 16-byte aligned.
hipError_t launch_sum_parts_bf16(const float* parts, int S, int64_t stride, uint16_t* out,
                                 int64_t n, hipStream_t st);

// x[0 .. n) *= *s in place (bf16 with round to nearest even, or fp32); x
// 16-byte aligned, s a device pointer.
hipError_t launch_scale(void* x, int64_t n, bool bf16, const float* s, hipStream_t st);

// loss[0] = (first ? 0 : loss[0]) + (sum of rows staged losses) * scale,
// summed in fp64 in a fixed order.
hipError_t launch_loss_sum(const float* row_loss, int64_t loss_stride,
                           int rows, float scale, int first, float* loss,
                           hipStream_t s);

// Matrix-core rate microbenchmark (mfma_rate.hip): `workgroups` x 4 waves,
// each running `iters` rounds of 16 v_mfma_f32_32x32x16_bf16 on fragments
// read from the first n_groups 128-byte groups at ops (16-byte aligned);
// per wave w, sink[w] = sum of element 0 of its 16 accumulator blocks over
// its lanes, clocks[2w] = shader clocks
// and clocks[2w + 1] = reference-counter ticks spent in the loop.
hipError_t launch_mfma_rate(const void* ops, int n_groups, int64_t iters, int workgroups,
                            float* sink, uint64_t* clocks, hipStream_t s);

}  // namespace flce
