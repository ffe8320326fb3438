// Elementwise kernels of the head (gfx950): scaling of precomputed
// gradients by the loss's upstream gradient, and the sum of K-split parts.
//
// Scaling:
//
// The fused head forms dloss/dh and dloss/dW during the forward call (page
// 1, "Liger Kernel explained", section "What does Liger Kernel actually
// fuse": the gradient of each chunk is produced while its logits exist);
// when the loss is then scaled, e.g. divided by the number of accumulation
// steps as in page 3's training loop ("Complete Guide to Liger Kernel",
// the training-loop example), the backward pass only multiplies them by
// that factor.  The factor is read from device memory, so the caller never
// synchronises to learn it.
#include "flce_internal.h"

namespace flce {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

constexpr int kThreads = 256;

// n16: number of 16-byte pieces (8 bf16 values); tail: trailing values.
__global__ void __launch_bounds__(kThreads)
scale_bf16_kernel(uint16_t* __restrict__ x, int64_t n16, int tail, const float* __restrict__ s) {
  const float c = *s;
  u32x4* xv = reinterpret_cast<u32x4*>(x);
  for (int64_t i = blockIdx.x * (int64_t)kThreads + threadIdx.x; i < n16;
       i += (int64_t)gridDim.x * kThreads) {
    const u32x4 v = xv[i];
    u32x4 w;
#pragma unroll
    for (int e = 0; e < 4; ++e) w[e] = pack_bf16x2(bf16_lo(v[e]) * c, bf16_hi(v[e]) * c);
    xv[i] = w;
  }
  if (blockIdx.x == 0 && threadIdx.x < tail) {
    uint16_t* p = x + n16 * 8 + threadIdx.x;
    *p = (uint16_t)(pack_bf16x2(__uint_as_float((uint32_t)*p << 16) * c, 0.0f) & 0xffffu);
  }
}

// n16: number of 16-byte pieces (4 floats); tail: trailing values.
__global__ void __launch_bounds__(kThreads)
scale_f32_kernel(float* __restrict__ x, int64_t n16, int tail, const float* __restrict__ s) {
  const float c = *s;
  f32x4* xv = reinterpret_cast<f32x4*>(x);
  for (int64_t i = blockIdx.x * (int64_t)kThreads + threadIdx.x; i < n16;
       i += (int64_t)gridDim.x * kThreads)
    xv[i] = xv[i] * c;
  if (blockIdx.x == 0 && threadIdx.x < tail) x[n16 * 4 + threadIdx.x] *= c;
}

inline dim3 grid_for(int64_t n16) {
  // enough workgroups to cover every CU several times, grid-stride beyond
  int64_t g = (n16 + kThreads - 1) / kThreads;
  if (g > 4096) g = 4096;
  if (g < 1) g = 1;
  return dim3(static_cast<unsigned>(g));
}

// out[i] = bf16(parts[i] + parts[stride + i] + ...), 4 values per thread and
// step, parts summed in index order.
__global__ void __launch_bounds__(kThreads)
sum_parts_kernel(const float* __restrict__ parts, int S, int64_t stride,
                 uint16_t* __restrict__ out, int64_t n4, int tail) {
  for (int64_t i = blockIdx.x * (int64_t)kThreads + threadIdx.x; i < n4;
       i += (int64_t)gridDim.x * kThreads) {
    f32x4 a = reinterpret_cast<const f32x4*>(parts)[i];
    for (int s = 1; s < S; ++s) a += reinterpret_cast<const f32x4*>(parts + s * stride)[i];
    uint2 w;
    w.x = pack_bf16x2(a[0], a[1]);
    w.y = pack_bf16x2(a[2], a[3]);
    reinterpret_cast<uint2*>(out)[i] = w;
  }
  if (blockIdx.x == 0 && threadIdx.x < tail) {
    const int64_t i = n4 * 4 + threadIdx.x;
    float a = parts[i];
    for (int s = 1; s < S; ++s) a += parts[s * stride + i];
    out[i] = (uint16_t)(pack_bf16x2(a, 0.0f) & 0xffffu);
  }
}

}  // namespace

hipError_t launch_sum_parts_bf16(const float* parts, int S, int64_t stride, uint16_t* out,
                                 int64_t n, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  const int64_t n4 = n / 4;
  hipLaunchKernelGGL(sum_parts_kernel, grid_for(n4), dim3(kThreads), 0, st, parts, S, stride,
                     out, n4, static_cast<int>(n % 4));
  return hipGetLastError();
}

hipError_t launch_scale(void* x, int64_t n, bool bf16, const float* s, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  if (bf16) {
    const int64_t n16 = n / 8;
    hipLaunchKernelGGL(scale_bf16_kernel, grid_for(n16), dim3(kThreads), 0, st,
                       static_cast<uint16_t*>(x), n16, static_cast<int>(n % 8), s);
  } else {
    const int64_t n16 = n / 4;
    hipLaunchKernelGGL(scale_f32_kernel, grid_for(n16), dim3(kThreads), 0, st,
                       static_cast<float*>(x), n16, static_cast<int>(n % 4), s);
  }
  return hipGetLastError();
}

}  // namespace flce
