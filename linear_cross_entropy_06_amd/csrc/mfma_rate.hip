// Matrix-core rate microbenchmark (gfx950): the bf16 MFMA rate this part
// sustains for given operand bits, and the shader clock it sustains it at.
//
// The head's three contractions run one 256-thread workgroup per CU; each
// wave issues 4 x 4 v_mfma_f32_32x32x16_bf16 per 16-wide k step into 256
// fp32 accumulators.  This kernel issues that same instruction stream from
// registers alone: the operand fragments are loaded once and the loop has
// no LDS or memory traffic.  Its rate is therefore the ceiling the GEMMs
// approach, i.e. 4096 flop per clock and CU at the clock the chip holds
// under this load.  The clock depends on the operand bits, because the
// matrix cores draw more power when their inputs toggle.
//
// Each wave times its own loop with two counters: s_memtime counts shader
// clocks and s_memrealtime counts a constant-rate reference.  The ratio of
// the two over the loop gives the clock that wave ran at.
#include "flce_internal.h"

namespace flce {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Wave w, lane l reads the 128-byte group g = (w * 64 + l) mod n_groups:
// its 16-byte pieces 0-3 are the lane's A fragments, 4-7 its B fragments.
// With the 32x32x16 operand layout, lane l holds row (or column) l % 32 and
// k = 8 * (l / 32) .. 8 * (l / 32) + 7 of its 32 x 16 block.
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
mfma_rate_kernel(const u32x4* __restrict__ ops, int n_groups, int64_t iters,
                 float* __restrict__ sink, uint64_t* __restrict__ clocks) {
  const int lane = threadIdx.x & 63;
  const int wave = blockIdx.x * 4 + (threadIdx.x >> 6);
  const u32x4* const grp = ops + 8 * (int64_t)((wave * 64 + lane) % n_groups);
  bf16x8 a[4], b[4];
#pragma unroll
  for (int f = 0; f < 4; ++f) {
    a[f] = __builtin_bit_cast(bf16x8, grp[f]);
    b[f] = __builtin_bit_cast(bf16x8, grp[4 + f]);
  }
  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const uint64_t c0 = __builtin_amdgcn_s_memtime();
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
  // iters >= 1 (checked on the host): no zero-trip path to compile.
  int64_t n = iters;
  do {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
  } while (--n > 0);
  const uint64_t c1 = __builtin_amdgcn_s_memtime();
  const uint64_t t1 = __builtin_amdgcn_s_memrealtime();

  // One accumulator of every block, summed over the wave, keeps all 16
  // MFMA chains live (each instruction writes its whole block) and lets a
  // caller check what was computed.  Element 0 of a lane's block is row
  // 4 * (lane / 32), column lane % 32 of that 32 x 32 product.  Reading all
  // 256 accumulators out here instead makes the register allocator spill
  // the operand fragments inside the loop.
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) s += acc[i][j][0];
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off, 64);
  if (lane == 0) {
    sink[wave] = s;
    clocks[2 * wave] = c1 - c0;
    clocks[2 * wave + 1] = t1 - t0;
  }
}

}  // namespace

hipError_t launch_mfma_rate(const void* ops, int n_groups, int64_t iters, int workgroups,
                            float* sink, uint64_t* clocks, hipStream_t s) {
  if (n_groups < 1 || workgroups < 1 || workgroups > 65535) return hipErrorInvalidValue;
  hipLaunchKernelGGL(mfma_rate_kernel, dim3(workgroups), dim3(256), 0, s,
                     static_cast<const u32x4*>(ops), n_groups, iters, sink, clocks);
  return hipGetLastError();
}

}  // namespace flce
