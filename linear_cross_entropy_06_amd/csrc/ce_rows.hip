// Row kernels of the fused linear + cross-entropy head (gfx950).
//
// ce_rows: per token row of fp32 logits (page 3, "Complete Guide to Liger
// Kernel", section "LigerCrossEntropyLoss": cross entropy of the logits
// against the labels; page 1, "Liger Kernel explained", section "What does
// Liger Kernel actually fuse": the gradient comes out of the same pass and
// is recomputed from the logits instead of being stored separately):
//   pass 1  online maximum / sum of exponentials over the row, one wave64
//           per row, lanes combined with cross-lane shuffles
//           -> lse_i, row loss lse_i - z[i, t_i]
//           (or, when the logits kernel left one log-sum-exp per 256-wide
//           slice of the row, the same online reduction over those
//           partials: the row is then read only once, by pass 2)
//   pass 2  G[i, j] = (exp(z[i, j] - lse_i) - [j == t_i]) * scale, written
//           back over the row itself (bf16 into the first half of the row's
//           bytes, or fp32 in place).
// The exponentials run in base 2 on the hardware v_exp_f32 / v_log_f32.
//
// In-place safety: a wave owns its row, reads a slab of the row into
// registers and only then writes the slab's results, whose bytes (2 per
// element, starting at the row's first byte) lie at or below bytes the wave
// has already read (4 per element).  Within one wave, memory operations are
// issued in program order and every store depends on the loads it follows,
// so no barrier is needed.
//
// loss_sum: the per-row losses of a chunk, summed in fp64 in a fixed order
// (deterministic), scaled and added to the running fp32 loss.
#include "flce_internal.h"

#include <math.h>

namespace flce {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kWavesPerBlock = 4;
constexpr int kUnroll = 4;  // float4 loads in flight per lane

// Two floats rounded to nearest-even bf16 and packed (first in the low
// half): one v_cvt_pk_bf16_f32 on gfx950.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}

__device__ __forceinline__ uint32_t bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// z * log2(e), rounded once and never fused into a following add, so that
// both passes see bit-identical base-2 logits (the row maximum then maps to
// exactly 2^0 = 1 in pass 2).
__device__ __forceinline__ float to_log2(float z) {
#pragma clang fp contract(off)
  return z * kLog2e;
}
__device__ __forceinline__ float log2_hw(float x) { return __builtin_amdgcn_logf(x); }

// Online update of (m, s) = (running max, sum of 2^(y - m)) with y = z*log2e.
__device__ __forceinline__ void online_add(float y, float& m, float& s) {
  if (y > m) {
    s = s * exp2_hw(m - y) + 1.0f;
    m = y;
  } else {
    s += exp2_hw(y - m);
  }
}

__device__ __forceinline__ void online_add4(f32x4 z, float& m, float& s) {
  const float y0 = to_log2(z[0]), y1 = to_log2(z[1]);
  const float y2 = to_log2(z[2]), y3 = to_log2(z[3]);
  const float mx = fmaxf(fmaxf(y0, y1), fmaxf(y2, y3));
  if (mx > m) {
    s *= exp2_hw(m - mx);
    m = mx;
  }
  s += exp2_hw(y0 - m) + exp2_hw(y1 - m) + exp2_hw(y2 - m) + exp2_hw(y3 - m);
}

// Combine two (m, s) pairs.
__device__ __forceinline__ void combine(float& m, float& s, float m2, float s2) {
  const float mm = fmaxf(m, m2);
  if (mm == -INFINITY) return;  // both empty
  s = s * exp2_hw(m - mm) + s2 * exp2_hw(m2 - mm);
  m = mm;
}

template <bool VEC4, bool OUT_BF16, bool PARTS>
__global__ void __launch_bounds__(64 * kWavesPerBlock)
ce_rows_kernel(float* __restrict__ z, int64_t ldz, const int32_t* __restrict__ targets,
               int rows, int V, float scale, float* __restrict__ row_loss,
               int64_t loss_stride, const float* __restrict__ row_part, int64_t ldp,
               int n_part) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  if (row >= rows) return;
  float* zr = z + (int64_t)row * ldz;
  const int t = targets[row];
  const bool t_ok = (t >= 0) && (t < V);
  const float zt = t_ok ? zr[t] : __builtin_nanf("");

  // ---- pass 1: online max / sum of exponentials (base 2) ----
  float m = -INFINITY, s = 0.0f;
  int j0 = 0;
  if constexpr (PARTS) {
    // The logits kernel already reduced each 256-wide slice of the row to
    // log2(sum 2^y); their log-sum-exp is the row's.
    const float* pr = row_part + (int64_t)row * ldp;
    for (int p = lane; p < n_part; p += 64) online_add(pr[p], m, s);
  } else if constexpr (VEC4) {
    const int nvec = V >> 2;
    const f32x4* zv = reinterpret_cast<const f32x4*>(zr);
    int v = lane;
    for (; v + 64 * (kUnroll - 1) < nvec; v += 64 * kUnroll) {
      f32x4 x[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) x[u] = zv[v + 64 * u];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) online_add4(x[u], m, s);
    }
    for (; v < nvec; v += 64) online_add4(zv[v], m, s);
    j0 = nvec << 2;
  }
  if constexpr (!PARTS)
    for (int j = j0 + lane; j < V; j += 64) online_add(to_log2(zr[j]), m, s);

#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const float m2 = __shfl_xor(m, off, 64);
    const float s2 = __shfl_xor(s, off, 64);
    combine(m, s, m2, s2);
  }
  const float lse2 = m + log2_hw(s);  // log2 of sum_j 2^(z_j log2e)
  // loss = lse - z_t, formed as (m - z_t log2e + log2 s) ln2 so that the
  // target's own term cancels exactly when it is the row maximum.
  if (lane == 0)
    row_loss[(int64_t)row * loss_stride] = ((m - to_log2(zt)) + log2_hw(s)) * kLn2;

  // ---- pass 2: rewrite the row as (softmax - onehot) * scale ----
  uint16_t* gb = reinterpret_cast<uint16_t*>(zr);
  if constexpr (PARTS) {
    // (bf16 output, V % 8 == 0.)  Every element becomes
    // 2^(z log2 e - lse2 + log2 scale): one fma and one exp per logit; the
    // target's element is then rewritten as (p_t - 1) * scale.
    const float shift = lse2 - log2_hw(scale);
    const int nvec = V >> 2;
    const f32x4* zv = reinterpret_cast<const f32x4*>(zr);
    for (int v0 = 0; v0 < nvec; v0 += 64 * kUnroll) {
      f32x4 x[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int v = v0 + lane + 64 * u;
        // Streaming: the row is read once here and its G is consumed by
        // the next GEMM long after other rows have gone through the caches.
        if (v < nvec) x[u] = __builtin_nontemporal_load(&zv[v]);
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int v = v0 + lane + 64 * u;
        if (v >= nvec) continue;
        float g[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) g[e] = exp2_hw(__builtin_fmaf(x[u][e], kLog2e, -shift));
        u32x2 w;
        w[0] = pack_bf16x2(g[0], g[1]);
        w[1] = pack_bf16x2(g[2], g[3]);
        __builtin_nontemporal_store(w, &reinterpret_cast<u32x2*>(gb)[v]);
      }
    }
    if (t_ok && lane == 0) {
      // After this wave's stores of the row have completed (the target's
      // element among them), overwrite that element.
      __builtin_amdgcn_s_waitcnt(0);
      const float pt = exp2_hw(to_log2(zt) - lse2);
      gb[t] = (uint16_t)bf16_bits((pt - 1.0f) * scale);
    }
    return;
  }
  if constexpr (VEC4) {
    const int nvec = V >> 2;
    f32x4* zv = reinterpret_cast<f32x4*>(zr);
    for (int v0 = 0; v0 < nvec; v0 += 64 * kUnroll) {
      f32x4 x[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int v = v0 + lane + 64 * u;
        // Streaming: the row is read once here and its G is consumed by
        // the next GEMM long after other rows have gone through the caches.
        if (v < nvec) x[u] = __builtin_nontemporal_load(&zv[v]);
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int v = v0 + lane + 64 * u;
        if (v >= nvec) continue;
        f32x4 g;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float p = exp2_hw(to_log2(x[u][e]) - lse2);
          g[e] = (p - ((4 * v + e) == t ? 1.0f : 0.0f)) * scale;
        }
        if constexpr (OUT_BF16) {
          u32x2 w;
          w[0] = pack_bf16x2(g[0], g[1]);
          w[1] = pack_bf16x2(g[2], g[3]);
          __builtin_nontemporal_store(w, &reinterpret_cast<u32x2*>(gb)[v]);
        } else {
          zv[v] = g;
        }
      }
    }
    j0 = nvec << 2;
  } else {
    j0 = 0;
  }
  // Scalar remainder (or the whole row when V % 4 != 0), walked in slabs of
  // 64 elements: every lane reads before any lane of the wave writes.
  for (int jb = j0; jb < V; jb += 64) {
    const int j = jb + lane;
    float x = 0.0f;
    if (j < V) x = zr[j];
    if (j < V) {
      const float p = exp2_hw(to_log2(x) - lse2);
      const float g = (p - (j == t ? 1.0f : 0.0f)) * scale;
      if constexpr (OUT_BF16)
        gb[j] = (uint16_t)bf16_bits(g);
      else
        zr[j] = g;
    }
  }
}

constexpr int kSumThreads = 256;

__global__ void __launch_bounds__(kSumThreads)
loss_sum_kernel(const float* __restrict__ row_loss, int64_t loss_stride, int rows,
                float scale, int first, float* __restrict__ loss) {
  __shared__ double part[kSumThreads];
  double acc = 0.0;
  for (int i = threadIdx.x; i < rows; i += kSumThreads)
    acc += (double)row_loss[(int64_t)i * loss_stride];
  part[threadIdx.x] = acc;
  __syncthreads();
  for (int w = kSumThreads / 2; w >= 1; w >>= 1) {
    if (threadIdx.x < w) part[threadIdx.x] += part[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const double prev = first ? 0.0 : (double)loss[0];
    loss[0] = (float)(prev + part[0] * (double)scale);
  }
}

}  // namespace

hipError_t launch_ce_rows(float* z, int64_t ldz, const int32_t* targets, int rows,
                          int V, float scale, float* row_loss, int64_t loss_stride,
                          bool out_bf16, hipStream_t s, const float* row_part, int64_t ldp,
                          int n_part) {
  if (rows <= 0) return hipSuccess;
  const dim3 grid((rows + kWavesPerBlock - 1) / kWavesPerBlock);
  const dim3 block(64 * kWavesPerBlock);
  // float4 path: row starts 16-byte aligned (base aligned, pitch % 4 == 0).
  const bool vec4 = ((ldz & 3) == 0) && ((reinterpret_cast<uintptr_t>(z) & 15) == 0);
  if (row_part) {
    // Partials come from the bf16 logits kernel, whose shapes give float4 rows.
    if (!(vec4 && out_bf16) || n_part < 1) return hipErrorInvalidValue;
    hipLaunchKernelGGL((ce_rows_kernel<true, true, true>), grid, block, 0, s, z, ldz, targets,
                       rows, V, scale, row_loss, loss_stride, row_part, ldp, n_part);
  } else if (vec4 && out_bf16) {
    hipLaunchKernelGGL((ce_rows_kernel<true, true, false>), grid, block, 0, s, z, ldz, targets,
                       rows, V, scale, row_loss, loss_stride, nullptr, 0, 0);
  } else if (vec4) {
    hipLaunchKernelGGL((ce_rows_kernel<true, false, false>), grid, block, 0, s, z, ldz,
                       targets, rows, V, scale, row_loss, loss_stride, nullptr, 0, 0);
  } else if (out_bf16) {
    hipLaunchKernelGGL((ce_rows_kernel<false, true, false>), grid, block, 0, s, z, ldz,
                       targets, rows, V, scale, row_loss, loss_stride, nullptr, 0, 0);
  } else {
    hipLaunchKernelGGL((ce_rows_kernel<false, false, false>), grid, block, 0, s, z, ldz,
                       targets, rows, V, scale, row_loss, loss_stride, nullptr, 0, 0);
  }
  return hipGetLastError();
}

hipError_t launch_loss_sum(const float* row_loss, int64_t loss_stride, int rows,
                           float scale, int first, float* loss, hipStream_t s) {
  hipLaunchKernelGGL(loss_sum_kernel, dim3(1), dim3(kSumThreads), 0, s, row_loss,
                     loss_stride, rows, scale, first, loss);
  return hipGetLastError();
}

}  // namespace flce
