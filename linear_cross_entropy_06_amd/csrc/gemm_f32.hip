// fp32 contractions of the fused linear + cross-entropy head (FLCE_F32).
//
// Same index semantics as the bf16 MFMA kernel (D[m][n] = sum_k A(m,k)
// B(n,k), stored as out[n * ldo + m]); used for fp32 operands, where the
// path is small and fp32 FMA on the vector ALUs reaches the same peak as the
// fp32 matrix instructions.  64x64 output tile per 256-thread workgroup, each
// thread a 4x4 register block, K walked in 32-wide slabs staged in LDS in
// [k][row] order so the inner loop reads broadcast-free float4s.  The next
// slab's operands are loaded into registers while the current slab's FMAs
// run: at the head's fp32 shapes the grid is a few workgroups with a long K
// (grad_h of 256 tokens: 8 tiles, K = V), so each slab's memory round trip,
// not arithmetic, sets the time.
#include "flce_internal.h"

namespace flce {
namespace {

constexpr int kBM = 64, kBN = 64, kBK = 32, kNT = 256;
constexpr int kLA = (kBM * kBK) / kNT, kLB = (kBN * kBK) / kNT;  // loads per thread and slab

template <bool KC>
__device__ __forceinline__ float ld_op(const float* __restrict__ p, int64_t ld, int row,
                                       int rows, int k, int K) {
  if (row >= rows || k >= K) return 0.0f;
  return KC ? p[(int64_t)row * ld + k] : p[(int64_t)k * ld + row];
}

template <bool A_KC, bool B_KC, int EPI>
__global__ void __launch_bounds__(kNT) gemm_f32_kernel(GemmArgs g) {
  __shared__ float As[kBK][kBM + 4];
  __shared__ float Bs[kBK][kBN + 4];
  const int tid = threadIdx.x;
  const int tiles_n = (g.N + kBN - 1) / kBN;
  const int m0 = (blockIdx.x / tiles_n) * kBM;
  const int n0 = (blockIdx.x % tiles_n) * kBN;
  const float* __restrict__ A = static_cast<const float*>(g.A);
  const float* __restrict__ B = static_cast<const float*>(g.B);
  const int tx = tid % 16, ty = tid / 16;

  // Element i of a thread's share of a slab: tile row r, slab column k.
  // k-contiguous operands: consecutive threads walk k; otherwise rows.
  float ra[kLA], rb[kLB];
  auto fetch = [&](int k0) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < kLA; ++i) {
      const int q = tid + kNT * i;
      const int r = A_KC ? q / kBK : q % kBM;
      const int k = A_KC ? q % kBK : q / kBM;
      ra[i] = ld_op<A_KC>(A, g.lda, m0 + r, g.M, k0 + k, g.K);
    }
#pragma unroll
    for (int i = 0; i < kLB; ++i) {
      const int q = tid + kNT * i;
      const int r = B_KC ? q / kBK : q % kBN;
      const int k = B_KC ? q % kBK : q / kBN;
      rb[i] = ld_op<B_KC>(B, g.ldb, n0 + r, g.N, k0 + k, g.K);
    }
  };
  auto stage = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < kLA; ++i) {
      const int q = tid + kNT * i;
      As[A_KC ? q % kBK : q / kBM][A_KC ? q / kBK : q % kBM] = ra[i];
    }
#pragma unroll
    for (int i = 0; i < kLB; ++i) {
      const int q = tid + kNT * i;
      Bs[B_KC ? q % kBK : q / kBN][B_KC ? q / kBK : q % kBN] = rb[i];
    }
  };

  float acc[4][4] = {};
  fetch(0);
  for (int k0 = 0; k0 < g.K; k0 += kBK) {
    stage();
    __syncthreads();
    if (k0 + kBK < g.K) fetch(k0 + kBK);  // in flight during this slab's FMAs
#pragma unroll
    for (int k = 0; k < kBK; ++k) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[k][tx * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = Bs[k][ty * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
  float* __restrict__ out = static_cast<float*>(g.out);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int n = n0 + ty * 4 + j;
    if (n >= g.N) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = m0 + tx * 4 + i;
      if (m >= g.M) continue;
      float* o = out + (int64_t)n * g.ldo + m;
      *o = (EPI == kAccumF32 && g.beta) ? *o + acc[i][j] : acc[i][j];
    }
  }
}

template <bool A_KC, bool B_KC, int EPI>
hipError_t launch_one(const GemmArgs& g, hipStream_t s) {
  if (!tile_count_ok(g.M, g.N, kBM, kBN, 1)) return hipErrorInvalidValue;
  const int tiles = ((g.M + kBM - 1) / kBM) * ((g.N + kBN - 1) / kBN);
  hipLaunchKernelGGL((gemm_f32_kernel<A_KC, B_KC, EPI>), dim3(tiles), dim3(kNT), 0, s, g);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_f32(bool a_kc, bool b_kc, int epi, const GemmArgs& g,
                           hipStream_t s) {
  if (g.M <= 0 || g.N <= 0) return hipSuccess;
  if (g.splits > 1 || epi == kExpBF16) return hipErrorInvalidValue;  // bf16 kernel only
  if (a_kc && b_kc && (epi == kStoreF32 || epi == kStoreOut))
    return launch_one<true, true, kStoreF32>(g, s);
  if (!a_kc && b_kc && (epi == kStoreF32 || epi == kStoreOut))
    return launch_one<false, true, kStoreF32>(g, s);
  if (!a_kc && !b_kc && epi == kAccumF32) return launch_one<false, false, kAccumF32>(g, s);
  return hipErrorInvalidValue;
}

}  // namespace flce
