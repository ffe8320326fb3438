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
};

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
  // Optional (kStoreF32 through the direct-to-LDS kernel only): for every
  // output column n and every 256-row tile t of m, row_part[n * ldp + t] =
  // log2(sum over the tile's rows m < M of 2^(D[m][n] * log2 e)), the
  // tile's share of a row log-sum-exp, with D[m][n] * log2 e rounded once.
  float* row_part = nullptr;
  int64_t ldp = 0;
};

// Rows of m per tile of the direct-to-LDS kernel (granularity of row_part).
constexpr int kRowPartTile = 256;

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
// kernel (the only one that fills GemmArgs::row_part).
bool gemm_bf16_uses_dma(bool a_kc, bool b_kc, bool vec, const GemmArgs& g);
hipError_t launch_gemm_bf16_dma(bool a_kc, bool b_kc, int epi, const GemmArgs& g,
                                hipStream_t s);

// fp32 operands, same index semantics (used by FLCE_F32).
hipError_t launch_gemm_f32(bool a_kc, bool b_kc, int epi, const GemmArgs& g,
                           hipStream_t s);

// Cross entropy of `rows` fp32 logit rows with the gradient rewritten in
// place (bf16 at pitch 2*ldz elements, or fp32 at pitch ldz).  With
// row_part != nullptr the row log-sum-exp is assembled from the n_part
// per-tile partials row_part[row * ldp + t] (GemmArgs::row_part) and each
// row is read once; otherwise it is read twice (online max / sum first).
hipError_t launch_ce_rows(float* z, int64_t ldz, const int32_t* targets,
                          int rows, int V, float scale, float* row_loss,
                          int64_t loss_stride, bool out_bf16, hipStream_t s,
                          const float* row_part = nullptr, int64_t ldp = 0,
                          int n_part = 0);

// loss[0] = (first ? 0 : loss[0]) + (sum of rows staged losses) * scale,
// summed in fp64 in a fixed order.
hipError_t launch_loss_sum(const float* row_loss, int64_t loss_stride,
                           int rows, float scale, int first, float* loss,
                           hipStream_t s);

}  // namespace flce
