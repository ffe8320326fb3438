// Odds-ratio preference loss over the fused head (gfx950): the per-row and
// per-pair steps between the head's row statistics and its gradient GEMMs.
//
// Page 2, "Liger-Kernel: Triton kernels that replace Hugging Face training
// ops", section "Installation and the one-line patch", lists ORPO among the
// chunked post-training losses that take the LM-head weight, the hidden
// states and the targets and return the loss; the objective is the
// published one of ORPO (Hong, Lee and Thorne, 2024):
//   l_s      = mean over the counted rows of sequence s of log p(t_r)
//   lo_s     = l_s - ln(1 - exp(l_s))                       (log odds)
//   L_OR     = (1/B) sum_b ln(1 + exp(-(lo_b - lo_{B+b})))
//   L_SFT    = -(1/M) sum over counted chosen rows of log p(t_r)
//   loss     = L_SFT + beta L_OR
// and every row's logit gradient is c_r (softmax - onehot) with
//   c_r = [chosen] / M + (+/-) beta / B * sigmoid(-(lo_b - lo_{B+b}))
//         / ((1 - exp(l_s)) n_s)
// (+ for the chosen, - for the rejected row of pair b; n_s counted rows of
// the row's sequence).  With P = exp(l), Q = 1 - P and odds P / Q, the
// odds-ratio factor is evaluated as
//   sigmoid(-ratio) / Q_w = 1 / (Q_w + P_w Q_l / P_l)
//   sigmoid(-ratio) / Q_l = 1 / (Q_l + Q_l^2 P_w / (Q_w P_l))
// (exp(ratio) = odds_w / odds_l), which equal the chain-rule forms and
// reach their limits as a sequence becomes certain (Q -> 0): a certain
// chosen sequence leaves finite terms, a certain rejected one an infinite
// loss, as the objective itself does.  Each log p(t_r) comes from the row pass as
// -ln(1 + S_r), S_r the other classes' mass relative to the target's, so
// l and Q = -expm1(l) keep their relative precision near P = 1.  Sums run
// in fp64 in a fixed order (deterministic).
#include "flce_internal.h"

#include <math.h>

namespace flce {
namespace {

constexpr int kWaves = 4;
constexpr int kCountThreads = 1024;
constexpr int kLossThreads = 256;

__global__ void __launch_bounds__(kCountThreads)
orpo_count_kernel(const int32_t* __restrict__ targets, int64_t n, int* __restrict__ count) {
  __shared__ int part[kCountThreads];
  int c = 0;
  for (int64_t i = threadIdx.x; i < n; i += kCountThreads) c += targets[i] >= 0 ? 1 : 0;
  part[threadIdx.x] = c;
  __syncthreads();
  for (int w = kCountThreads / 2; w >= 1; w >>= 1) {
    if ((int)threadIdx.x < w) part[threadIdx.x] += part[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) count[0] = part[0];
}

// Sum over the wave in a fixed butterfly order: every lane gets the total.
__device__ __forceinline__ double wave_sum(double x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}
__device__ __forceinline__ int wave_sum(int x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}

// One wave per pair q of the chunk.
__global__ void __launch_bounds__(64 * kWaves)
orpo_coef_kernel(const float* __restrict__ row_loss, const int32_t* __restrict__ targets, int Pc,
                 int T, int B, int p0, float beta, const int* __restrict__ count,
                 float* __restrict__ coef, float* __restrict__ seq_logp,
                 float* __restrict__ stage) {
  const int lane = threadIdx.x & 63;
  const int q = blockIdx.x * kWaves + (threadIdx.x >> 6);
  if (q >= Pc) return;
  const int64_t rw = (int64_t)q * T;         // chosen rows of the pair
  const int64_t rl = (int64_t)(Pc + q) * T;  // rejected rows
  double sw = 0.0, sl = 0.0;                 // sums of log p over counted rows
  int nw = 0, nl = 0;
  for (int k = lane; k < T; k += 64) {
    if (targets[rw + k] >= 0) {
      sw -= (double)row_loss[rw + k];
      ++nw;
    }
    if (targets[rl + k] >= 0) {
      sl -= (double)row_loss[rl + k];
      ++nl;
    }
  }
  sw = wave_sum(sw);
  sl = wave_sum(sl);
  nw = wave_sum(nw);
  nl = wave_sum(nl);
  // Mean log-probabilities (0 / 0 = NaN for a sequence with no counted row).
  const double lw = sw / (double)nw, ll = sl / (double)nl;
  const double pw = exp(lw), pl = exp(ll);
  const double qw = -expm1(lw), ql = -expm1(ll);  // 1 - P, accurate near P = 1
  const double ratio = (lw - log(qw)) - (ll - log(ql));
  const double or_term = ratio > 0.0 ? log1p(exp(-ratio)) : -ratio + log1p(exp(ratio));
  const double k_or = (double)beta / (double)B;
  const double cw_or = k_or / ((double)nw * (qw + pw * ql / pl));
  const double cl_or = -k_or / ((double)nl * (ql + ql * ql * pw / (qw * pl)));
  const float cw = (float)(1.0 / (double)count[0] + cw_or);
  const float cl = (float)cl_or;
  for (int k = lane; k < T; k += 64) {
    coef[rw + k] = targets[rw + k] >= 0 ? cw : 0.0f;
    coef[rl + k] = targets[rl + k] >= 0 ? cl : 0.0f;
  }
  if (lane == 0) {
    const int p = p0 + q;
    stage[2 * p] = (float)(-sw);
    stage[2 * p + 1] = (float)or_term;
    if (seq_logp) {
      seq_logp[p] = (float)lw;
      seq_logp[B + p] = (float)ll;
    }
  }
}

__global__ void __launch_bounds__(kLossThreads)
orpo_loss_kernel(const float* __restrict__ stage, int B, float beta,
                 const int* __restrict__ count, float* __restrict__ loss) {
  __shared__ double sft[kLossThreads], orr[kLossThreads];
  double a = 0.0, b = 0.0;
  for (int p = threadIdx.x; p < B; p += kLossThreads) {
    a += (double)stage[2 * p];
    b += (double)stage[2 * p + 1];
  }
  sft[threadIdx.x] = a;
  orr[threadIdx.x] = b;
  __syncthreads();
  for (int w = kLossThreads / 2; w >= 1; w >>= 1) {
    if ((int)threadIdx.x < w) {
      sft[threadIdx.x] += sft[threadIdx.x + w];
      orr[threadIdx.x] += orr[threadIdx.x + w];
    }
    __syncthreads();
  }
  if (threadIdx.x == 0)
    loss[0] = (float)(sft[0] / (double)count[0] + (double)beta / (double)B * orr[0]);
}

}  // namespace

hipError_t launch_orpo_count(const int32_t* targets, int64_t n, int* count, hipStream_t s) {
  if (n < 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL(orpo_count_kernel, dim3(1), dim3(kCountThreads), 0, s, targets, n, count);
  return hipGetLastError();
}

hipError_t launch_orpo_coef(const float* row_loss, const int32_t* targets, int Pc, int T, int B,
                            int p0, float beta, const int* count, float* coef, float* seq_logp,
                            float* stage, hipStream_t s) {
  if (Pc <= 0) return hipSuccess;
  if (T <= 0 || B <= 0 || p0 < 0 || p0 + Pc > B) return hipErrorInvalidValue;
  hipLaunchKernelGGL(orpo_coef_kernel, dim3((Pc + kWaves - 1) / kWaves), dim3(64 * kWaves), 0, s,
                     row_loss, targets, Pc, T, B, p0, beta, count, coef, seq_logp, stage);
  return hipGetLastError();
}

hipError_t launch_orpo_loss(const float* stage, int B, float beta, const int* count, float* loss,
                            hipStream_t s) {
  if (B <= 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL(orpo_loss_kernel, dim3(1), dim3(kLossThreads), 0, s, stage, B, beta, count,
                     loss);
  return hipGetLastError();
}

}  // namespace flce
