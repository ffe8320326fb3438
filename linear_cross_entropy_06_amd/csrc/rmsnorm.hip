// RMSNorm in front of the loss head (page 3, "Complete Guide to Liger
// Kernel", section "LigerRMSNorm": the normalisation of the hidden states
// that feed the LM head; eps added to the mean square, the convention page 2
// warns to check, section "The support surface is narrower than the pitch
// suggests").  Per token row x_i of H elements:
//
//   r_i  = 1 / sqrt(mean_k x_ik^2 + eps)
//   h_ik = x_ik r_i gamma_k                      (fp32, rounded once on store)
//
// and, from g = dloss/dh as stored by the grad_h step:
//
//   grad_x_ik   = r_i gamma_k g_ik - x_ik (r_i^3 / H) sum_k gamma_k g_ik x_ik
//   grad_gamma_k (+)= sum_i g_ik x_ik r_i
//
// One wave64 per row for the row passes (8 elements per lane and step);
// grad_gamma sums fixed groups of 64 rows per column in fp32, then the
// groups in index order (deterministic), added to the running value over
// token chunks.  HBM-bound: the forward reads x twice (the second time from
// cache) and writes h; the backward reads x, g and writes grad_x.
#include "flce_internal.h"

#include <math.h>

namespace flce {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

constexpr int kWaves = 4;        // rows per 256-thread block
constexpr int kGroupRows = 64;   // rows per grad_gamma partial
constexpr int kThreads = 256;

__device__ __forceinline__ float lo16(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float hi16(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }
__device__ __forceinline__ uint32_t pack2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
}

// Elements 8v .. 8v+7 of a row: bf16 (one 16-byte piece) or fp32 (two).
template <bool BF16>
__device__ __forceinline__ void load8(const void* row, int v, float (&f)[8]) {
  if constexpr (BF16) {
    const u32x4 p = reinterpret_cast<const u32x4*>(row)[v];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      f[2 * e] = lo16(p[e]);
      f[2 * e + 1] = hi16(p[e]);
    }
  } else {
    const f32x4 a = reinterpret_cast<const f32x4*>(row)[2 * v];
    const f32x4 b = reinterpret_cast<const f32x4*>(row)[2 * v + 1];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      f[e] = a[e];
      f[4 + e] = b[e];
    }
  }
}

template <bool BF16>
__device__ __forceinline__ void store8(void* row, int v, const float (&f)[8]) {
  if constexpr (BF16) {
    u32x4 p;
#pragma unroll
    for (int e = 0; e < 4; ++e) p[e] = pack2(f[2 * e], f[2 * e + 1]);
    reinterpret_cast<u32x4*>(row)[v] = p;
  } else {
    reinterpret_cast<f32x4*>(row)[2 * v] = f32x4{f[0], f[1], f[2], f[3]};
    reinterpret_cast<f32x4*>(row)[2 * v + 1] = f32x4{f[4], f[5], f[6], f[7]};
  }
}

__device__ __forceinline__ float wave_sum(float a) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) a += __shfl_xor(a, off, 64);
  return a;
}

template <bool BF16>
__global__ void __launch_bounds__(64 * kWaves)
rmsnorm_fwd_kernel(const void* __restrict__ x, const void* __restrict__ gamma, float eps, int rows,
                   int H, void* __restrict__ h, float* __restrict__ rinv) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * kWaves + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int64_t es = BF16 ? 2 : 4;
  const char* xr = static_cast<const char*>(x) + (int64_t)row * H * es;
  char* hr = static_cast<char*>(h) + (int64_t)row * H * es;
  const int n8 = H / 8;
  float ss = 0.0f;
  for (int v = lane; v < n8; v += 64) {
    float f[8];
    load8<BF16>(xr, v, f);
#pragma unroll
    for (int e = 0; e < 8; ++e) ss = __builtin_fmaf(f[e], f[e], ss);
  }
  ss = wave_sum(ss);
  const float r = 1.0f / sqrtf(ss / (float)H + eps);
  for (int v = lane; v < n8; v += 64) {
    float f[8], gm[8];
    load8<BF16>(xr, v, f);
    load8<BF16>(gamma, v, gm);
#pragma unroll
    for (int e = 0; e < 8; ++e) f[e] = f[e] * r * gm[e];
    store8<BF16>(hr, v, f);
  }
  if (lane == 0) rinv[row] = r;
}

template <bool BF16>
__global__ void __launch_bounds__(64 * kWaves)
rmsnorm_bwd_kernel(const void* __restrict__ x, const void* __restrict__ gamma,
                   const void* __restrict__ g, const float* __restrict__ rinv, int rows, int H,
                   void* __restrict__ grad_x) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * kWaves + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int64_t es = BF16 ? 2 : 4;
  const char* xr = static_cast<const char*>(x) + (int64_t)row * H * es;
  const char* gr = static_cast<const char*>(g) + (int64_t)row * H * es;
  char* outr = static_cast<char*>(grad_x) + (int64_t)row * H * es;
  const int n8 = H / 8;
  const float r = rinv[row];
  float dot = 0.0f;
  for (int v = lane; v < n8; v += 64) {
    float xf[8], gf[8], gm[8];
    load8<BF16>(xr, v, xf);
    load8<BF16>(gr, v, gf);
    load8<BF16>(gamma, v, gm);
#pragma unroll
    for (int e = 0; e < 8; ++e) dot = __builtin_fmaf(gm[e] * gf[e], xf[e], dot);
  }
  dot = wave_sum(dot);
  const float c = r * r * r / (float)H * dot;
  for (int v = lane; v < n8; v += 64) {
    float xf[8], gf[8], gm[8], o[8];
    load8<BF16>(xr, v, xf);
    load8<BF16>(gr, v, gf);
    load8<BF16>(gamma, v, gm);
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = r * gm[e] * gf[e] - xf[e] * c;
    store8<BF16>(outr, v, o);
  }
}

// part[grp][k] = sum over the rows of group grp of g_ik x_ik r_i; each
// thread owns 4 consecutive columns; block b covers column block
// b % col_blocks of row group b / col_blocks.
template <bool BF16>
__global__ void __launch_bounds__(kThreads)
gamma_part_kernel(const void* __restrict__ x, const void* __restrict__ g,
                  const float* __restrict__ rinv, int rows, int H, int col_blocks,
                  float* __restrict__ part) {
  const int grp = (int)blockIdx.x / col_blocks;
  const int c4 = ((int)blockIdx.x - grp * col_blocks) * kThreads + threadIdx.x;
  if (4 * c4 >= H) return;
  const int i0 = grp * kGroupRows;
  const int i1 = min(rows, i0 + kGroupRows);
  float a[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int i = i0; i < i1; ++i) {
    const float r = rinv[i];
    float xf[4], gf[4];
    if constexpr (BF16) {
      const u32x2 xp = reinterpret_cast<const u32x2*>(static_cast<const uint16_t*>(x) +
                                                      (int64_t)i * H)[c4];
      const u32x2 gp = reinterpret_cast<const u32x2*>(static_cast<const uint16_t*>(g) +
                                                      (int64_t)i * H)[c4];
      xf[0] = lo16(xp[0]); xf[1] = hi16(xp[0]); xf[2] = lo16(xp[1]); xf[3] = hi16(xp[1]);
      gf[0] = lo16(gp[0]); gf[1] = hi16(gp[0]); gf[2] = lo16(gp[1]); gf[3] = hi16(gp[1]);
    } else {
      const f32x4 xp = reinterpret_cast<const f32x4*>(static_cast<const float*>(x) +
                                                      (int64_t)i * H)[c4];
      const f32x4 gp = reinterpret_cast<const f32x4*>(static_cast<const float*>(g) +
                                                      (int64_t)i * H)[c4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        xf[e] = xp[e];
        gf[e] = gp[e];
      }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) a[e] = __builtin_fmaf(gf[e] * xf[e], r, a[e]);
  }
  f32x4* out = reinterpret_cast<f32x4*>(part + (int64_t)grp * H);
  out[c4] = f32x4{a[0], a[1], a[2], a[3]};
}

__global__ void __launch_bounds__(kThreads)
gamma_sum_kernel(const float* __restrict__ part, int groups, int H,
                 float* __restrict__ grad_gamma, int first) {
  const int k = blockIdx.x * kThreads + threadIdx.x;
  if (k >= H) return;
  float s = 0.0f;
  for (int q = 0; q < groups; ++q) s += part[(int64_t)q * H + k];
  grad_gamma[k] = first ? s : grad_gamma[k] + s;
}

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

int rmsnorm_groups(int rows) { return (rows + kGroupRows - 1) / kGroupRows; }

hipError_t launch_rmsnorm_fwd(const void* x, const void* gamma, float eps, int rows, int H,
                              void* h, float* rinv, bool bf16, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if ((H % 8) || !aligned16(x) || !aligned16(gamma) || !aligned16(h)) return hipErrorInvalidValue;
  const dim3 grid((rows + kWaves - 1) / kWaves), block(64 * kWaves);
  if (bf16)
    hipLaunchKernelGGL(rmsnorm_fwd_kernel<true>, grid, block, 0, s, x, gamma, eps, rows, H, h,
                       rinv);
  else
    hipLaunchKernelGGL(rmsnorm_fwd_kernel<false>, grid, block, 0, s, x, gamma, eps, rows, H, h,
                       rinv);
  return hipGetLastError();
}

hipError_t launch_rmsnorm_bwd(const void* x, const void* gamma, const void* g, const float* rinv,
                              int rows, int H, void* grad_x, float* part, float* grad_gamma,
                              int first, bool bf16, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if ((H % 8) || !aligned16(x) || !aligned16(gamma) || !aligned16(g) || !aligned16(grad_x) ||
      !aligned16(part))
    return hipErrorInvalidValue;
  const dim3 grid((rows + kWaves - 1) / kWaves), block(64 * kWaves);
  const int col_blocks = (H / 4 + kThreads - 1) / kThreads;
  if ((int64_t)col_blocks * rmsnorm_groups(rows) > 0x7fffffff) return hipErrorInvalidValue;
  const dim3 pgrid(col_blocks * rmsnorm_groups(rows));
  const dim3 sgrid((H + kThreads - 1) / kThreads);
  if (bf16) {
    hipLaunchKernelGGL(rmsnorm_bwd_kernel<true>, grid, block, 0, s, x, gamma, g, rinv, rows, H,
                       grad_x);
    hipLaunchKernelGGL(gamma_part_kernel<true>, pgrid, dim3(kThreads), 0, s, x, g, rinv, rows,
                       H, col_blocks, part);
  } else {
    hipLaunchKernelGGL(rmsnorm_bwd_kernel<false>, grid, block, 0, s, x, gamma, g, rinv, rows, H,
                       grad_x);
    hipLaunchKernelGGL(gamma_part_kernel<false>, pgrid, dim3(kThreads), 0, s, x, g, rinv, rows,
                       H, col_blocks, part);
  }
  hipLaunchKernelGGL(gamma_sum_kernel, sgrid, dim3(kThreads), 0, s, part, rmsnorm_groups(rows), H,
                     grad_gamma, first);
  return hipGetLastError();
}

}  // namespace flce
