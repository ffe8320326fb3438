// Row kernels of the fused linear + cross-entropy head (gfx950).
//
// Per token row (page 3, "Complete Guide to Liger Kernel", section
// "LigerCrossEntropyLoss": cross entropy of the logits against the labels;
// page 1, "Liger Kernel explained", section "What does Liger Kernel actually
// fuse": the gradient comes out of the same pass and is recomputed from the
// logits instead of being stored separately), one wave64 per row:
//
// ce_rows (from fp32 logits)
//   pass 1  online maximum / sum of exponentials over the row, lanes
//           combined with cross-lane shuffles -> lse_i, row loss
//           lse_i - z[i, t_i]
//   pass 2  G[i, j] = (exp(z[i, j] - lse_i) - [j == t_i]) * scale, written
//           back over the row itself (bf16 into the first half of the row's
//           bytes, or fp32 in place).
//   In-place safety: a wave reads a slab of its row into registers and only
//   then writes the slab's results, whose bytes (2 per element, starting at
//   the row's first byte) lie at or below bytes the wave has already read
//   (4 per element); within one wave, memory operations are issued in
//   program order and every store depends on the loads it follows.
//
// ce_rows_exp (from the logits kernel's exponentiated output: bf16
// u = 2^(y - mx_q) with y = z log2 e, and one (mx_q, s_q = sum of u) pair
// per 128-column half tile q of the row, both from the kernel's fp32
// accumulators)
//   y_t     = log2(e) h_i . W_t, recomputed (bf16 rows, fp32 accumulation)
//   S       = sum over j != t of 2^(y_j - y_t): the probability mass of
//             every other class relative to the target's, a sum of positive
//             terms, from the pairs of the other half tiles and, for the
//             target's own half tile q_t, from its stored u values without
//             the target's (2^(mx_{q_t} - y_t) sum over j in q_t, j != t of
//             u_j)
//   loss_i  = ln(1 + S) = -log p_t (log1p: every digit kept as p_t -> 1)
//   lse2_i  = y_t + log2(1 + S)
//   G[i, j] = u * 2^(mx_q - lse2_i) * scale, written over u element by
//             element (same place, same size), except G[i, t] =
//             (p_t - 1) * scale = -S / (1 + S) * scale.
// Two kernels: one wave per row forms the statistics (loss, lse2, pt1,
// staged per row), then the rewrite walks u in memory order, one block of a
// row per workgroup.
// Writing log p_t through S rather than as lse - z_t keeps its relative
// precision when the model is confident (the odds-ratio loss divides by
// 1 - p).  y_t enters S only as a factor, so the rounding difference
// between the recomputed and the GEMM's target logit shifts S relatively
// (by about |y| 2^-24), never absolutely; the target's half tile adds the
// bf16 rounding of its other u values (at most 2^-9 relatively, on that
// half tile's share of S only).
//
// The exponentials run in base 2 on the hardware v_exp_f32 / v_log_f32.
//
// ce_target_mass / ce_stats_exp / ce_rewrite_exp (vocabulary chunks,
// preference loss): the same steps split in time.  After each chunk's
// logits, the target's half-tile mass of the rows whose target falls in the
// chunk; after every chunk's pairs exist, lse2_i, p_t - 1 and the row loss;
// then, chunk by chunk, G over that chunk's columns, with the target's
// element rewritten when it falls in the chunk.
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

template <bool VEC4, bool OUT_BF16>
__global__ void __launch_bounds__(64 * kWavesPerBlock)
ce_rows_kernel(float* __restrict__ z, int64_t ldz, const int32_t* __restrict__ targets,
               int rows, int V, float scale, float* __restrict__ row_loss,
               int64_t loss_stride) {
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
  if constexpr (VEC4) {
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

// bf16 -> fp32 (exact).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// (max, sum) over a row's nq pairs except half tile q_skip (one wave;
// every lane gets it).
__device__ __forceinline__ void combine_pairs(const float* pr, int nq, int q_skip, int lane,
                                              float& m, float& a) {
  m = -INFINITY;
  a = 0.0f;
  // Eight pairs per lane are requested before any is combined (the
  // statistics kernel is bound by these round trips); the combining order
  // is the plain one, q = lane, lane + 64, ...
  constexpr int kBatch = 8;
  for (int q0 = lane; q0 < nq; q0 += 64 * kBatch) {
    float pm[kBatch], ps[kBatch];
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      const int q = q0 + 64 * k;
      pm[k] = q < nq ? pr[2 * q] : -INFINITY;
      ps[k] = q < nq ? pr[2 * q + 1] : 0.0f;
    }
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      const int q = q0 + 64 * k;
      if (q < nq && q != q_skip) combine(m, a, pm[k], ps[k]);
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const float m2 = __shfl_xor(m, off, 64);
    const float a2 = __shfl_xor(a, off, 64);
    combine(m, a, m2, a2);
  }
}

// Sum of u over the elements [j0, j1) of a row (j0 even, j1 - j0 <= 128),
// without element t; two elements per lane, every lane gets the sum.
__device__ __forceinline__ float half_tile_mass(const uint16_t* ur, int j0, int j1, int t,
                                                int lane) {
  const int j = j0 + 2 * lane;
  float x = 0.0f;
  if (j < j1) {
    const uint32_t w = *reinterpret_cast<const uint32_t*>(ur + j);
    x = (j != t ? bf16_lo(w) : 0.0f) + (j + 1 < j1 && j + 1 != t ? bf16_hi(w) : 0.0f);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}

// Statistics of a row with a valid target t: from the pairs of every half
// tile but the target's, that half tile's (max, mass without the target)
// (mxt, rt), and the target's base-2 logit yt: lse2, the row loss
// ln(1 + S) and pt1 = p_t - 1 = -S / (1 + S).
struct RowStats {
  float lse2, loss, pt1;
};
__device__ __forceinline__ RowStats row_stats(const float* pr, int nq, int qt, float rt, float yt,
                                              int lane) {
  float m, a;
  combine_pairs(pr, nq, qt, lane, m, a);
  combine(m, a, pr[2 * qt], rt);  // (m, a): max and mass of every class but t
  const float d = m - yt;
  RowStats r;
  if (d <= 64.0f) {
    const float S = a * exp2_hw(d);
    r.loss = log1pf(S);
    r.pt1 = -S / (1.0f + S);
  } else {
    // another class exceeds the target by 2^64: S > 2^64, p_t = 0 in fp32
    r.loss = (d + log2_hw(a + exp2_hw(-d))) * kLn2;
    r.pt1 = -1.0f;
  }
  r.lse2 = yt + r.loss * kLog2e;
  return r;
}

// Target logit z_t = h_row . W_t (bf16 rows, fp32 accumulation; every lane
// gets it).
__device__ __forceinline__ float target_logit(const uint16_t* h_row, const uint16_t* w_row, int H,
                                              int lane) {
  const u32x4* hv = reinterpret_cast<const u32x4*>(h_row);
  const u32x4* wv = reinterpret_cast<const u32x4*>(w_row);
  float acc = 0.0f;
  // Four pieces of each row requested at a time; accumulated in the plain
  // order k = lane, lane + 64, ...
  constexpr int kBatch = 4;
  const int n8 = H / 8;
  for (int k0 = lane; k0 < n8; k0 += 64 * kBatch) {
    u32x4 a[kBatch], b[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const int k = k0 + 64 * j;
      if (k < n8) {
        a[j] = hv[k];
        b[j] = wv[k];
      }
    }
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      if (k0 + 64 * j >= n8) continue;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        acc += bf16_lo(a[j][e]) * bf16_lo(b[j][e]) + bf16_hi(a[j][e]) * bf16_hi(b[j][e]);
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off, 64);
  return acc;
}

// Row statistics of a chunk's exponentiated logits: per row the loss, lse2
// and pt1 = p_t - 1 into stats[row * stride + 0, 1, 2] (the caller's staging
// area), read by the rewrite below and by the loss sum.
__global__ void __launch_bounds__(64 * kWavesPerBlock)
ce_rows_exp_kernel(const uint16_t* __restrict__ u, int64_t ldu,
                   const float* __restrict__ row_part, int64_t ldp,
                   const uint16_t* __restrict__ h, const uint16_t* __restrict__ W, int H,
                   const int32_t* __restrict__ targets, int rows, int V,
                   float* __restrict__ stats, int64_t stride) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int t = targets[row];
  const bool t_ok = (t >= 0) && (t < V);
  const int nq = (V + kHalfTile - 1) / kHalfTile;
  const float* pr = row_part + (int64_t)row * ldp;

  // An out-of-range target is never dereferenced: the loss becomes NaN.
  RowStats st;
  if (t_ok) {
    const int qt = t / kHalfTile;
    const float rt = half_tile_mass(u + (int64_t)row * ldu, kHalfTile * qt,
                                    min(kHalfTile * (qt + 1), V), t, lane);
    const float yt = to_log2(target_logit(h + (int64_t)row * H, W + (int64_t)t * H, H, lane));
    st = row_stats(pr, nq, qt, rt, yt, lane);
  } else {
    float m, a;
    combine_pairs(pr, nq, -1, lane, m, a);
    st = RowStats{m + log2_hw(a), __builtin_nanf(""), 0.0f};
  }
  if (lane == 0) {
    float* o = stats + (int64_t)row * stride;
    o[0] = st.loss;
    o[1] = st.lse2;
    o[2] = st.pt1;
  }
}

// u -> G over columns [v0, v0 + n) of rows row0 .. (the chunk's own columns
// from u's first element), elementwise: every workgroup takes 16-byte pieces
// kRewritePieces * kRewriteThreads of one row, so consecutive workgroups
// sweep consecutive memory (a row-per-wave walk measured 20% slower than
// this order).  Piece v (elements 8v .. 8v + 7, half tile v / 16) becomes
// sign * u * 2^(mx_q - shift) with shift = lse2 - log2 |scale|, and the
// target's element, when the piece holds it, (p_t - 1) * scale.  With
// row_scale, row i takes the scale row_scale[i] (any sign; 0 clears the
// row); lse2 and pt1 of row i are read at i * stat_stride.
constexpr int kRewriteThreads = 256;
constexpr int kRewritePieces = 4;
constexpr int kRewriteBlockPieces = kRewriteThreads * kRewritePieces;

__global__ void __launch_bounds__(kRewriteThreads)
ce_rewrite_exp_kernel(uint16_t* __restrict__ u, int64_t ldu, const float* __restrict__ row_part,
                      int64_t ldp, const float* __restrict__ lse2_in,
                      const float* __restrict__ pt1_in, int64_t stat_stride,
                      const int32_t* __restrict__ targets, int row0, int v0, int n, int nb,
                      float scale, const float* __restrict__ row_scale) {
  const int rb = (int)blockIdx.x / nb;
  const int row = row0 + rb;
  const int cb = (int)blockIdx.x - rb * nb;
  const float lse2 = lse2_in[(int64_t)row * stat_stride];
  float sign = 1.0f;
  if (row_scale) {
    scale = row_scale[row];
    sign = scale < 0.0f ? -1.0f : 1.0f;
  }
  // |scale| folds into the exponent (log2 0 = -inf clears the row).
  const float shift = lse2 - log2_hw(__builtin_fabsf(scale));
  const int tt = targets[row] - v0;  // the target's column in the chunk
  u32x4* uv = reinterpret_cast<u32x4*>(u + (int64_t)row * ldu);
  const float* pr = row_part + (int64_t)row * ldp;
  const int nvec = n >> 3;
  const int first = cb * kRewriteBlockPieces + (int)threadIdx.x;
  u32x4 x[kRewritePieces];
  float f[kRewritePieces];
#pragma unroll
  for (int k = 0; k < kRewritePieces; ++k) {
    const int v = first + kRewriteThreads * k;
    if (v < nvec) {
      x[k] = __builtin_nontemporal_load(&uv[v]);
      f[k] = pr[2 * (v >> 4)];  // mx of the half tile holding elements 8v .. 8v+7
    }
  }
#pragma unroll
  for (int k = 0; k < kRewritePieces; ++k) {
    const int v = first + kRewriteThreads * k;
    if (v >= nvec) continue;
    const float c = exp2_hw(f[k] - shift) * sign;
    u32x4 w;
#pragma unroll
    for (int e = 0; e < 4; ++e) w[e] = pack_bf16x2(bf16_lo(x[k][e]) * c, bf16_hi(x[k][e]) * c);
    if (tt >= 0 && tt < n && (tt >> 3) == v) {
      const uint32_t g = bf16_bits(pt1_in[(int64_t)row * stat_stride] * scale);
      const int e = tt & 7;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if ((e >> 1) == q)
          w[q] = (e & 1) ? ((w[q] & 0xffffu) | (g << 16)) : ((w[q] & 0xffff0000u) | g);
      }
    }
    __builtin_nontemporal_store(w, &uv[v]);
  }
}

// Rewrite launches over rows [0, rows) in batches whose block count fits
// the 1-D grid.
hipError_t launch_rewrite_blocks(uint16_t* u, int64_t ldu, const float* row_part, int64_t ldp,
                                 const float* lse2, const float* pt1, int64_t stat_stride,
                                 const int32_t* targets, int rows, int v0, int n, float scale,
                                 const float* row_scale, hipStream_t s) {
  const int nb = (n / 8 + kRewriteBlockPieces - 1) / kRewriteBlockPieces;
  if (nb <= 0) return hipSuccess;
  const int per = (int)(((int64_t{1} << 31) - 1) / nb);
  for (int r0 = 0; r0 < rows; r0 += per) {
    const int rc = rows - r0 < per ? rows - r0 : per;
    hipLaunchKernelGGL(ce_rewrite_exp_kernel, dim3((unsigned)((int64_t)rc * nb)),
                       dim3(kRewriteThreads), 0, s, u, ldu, row_part, ldp, lse2, pt1,
                       stat_stride, targets, r0, v0, n, nb, scale, row_scale);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// Vocabulary chunk [v0, v0 + n) of rows' exponentiated logits (row pitch
// ldu, chunk-local columns; v0 % 128 == 0): for each row whose target falls
// in the chunk, the mass of its half tile without the target, into rt[row].
__global__ void __launch_bounds__(64 * kWavesPerBlock)
ce_target_mass_kernel(const uint16_t* __restrict__ u, int64_t ldu,
                      const int32_t* __restrict__ targets, int rows, int v0, int n,
                      float* __restrict__ rt) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int t = targets[row] - v0;
  if (t < 0 || t >= n) return;
  const int qt = t / kHalfTile;
  const float m = half_tile_mass(u + (int64_t)row * ldu, kHalfTile * qt,
                                 min(kHalfTile * (qt + 1), n), t, lane);
  if (lane == 0) rt[row] = m;
}

// Statistics only: after the exponentiated logits of every vocabulary chunk
// have left their (max, sum) pairs and the target's half-tile mass rt, per
// row lse2 (all V columns), p_t - 1 and the row loss.
__global__ void __launch_bounds__(64 * kWavesPerBlock)
ce_stats_exp_kernel(const float* __restrict__ row_part, int64_t ldp, const float* __restrict__ rt,
                    const uint16_t* __restrict__ h, const uint16_t* __restrict__ W, int H,
                    const int32_t* __restrict__ targets, int rows, int V,
                    float* __restrict__ lse2_out, float* __restrict__ pt1_out,
                    float* __restrict__ row_loss) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int t = targets[row];
  const bool t_ok = (t >= 0) && (t < V);
  const int nq = (V + kHalfTile - 1) / kHalfTile;
  const float* pr = row_part + (int64_t)row * ldp;
  RowStats st;
  if (t_ok) {
    const float yt = to_log2(target_logit(h + (int64_t)row * H, W + (int64_t)t * H, H, lane));
    st = row_stats(pr, nq, t / kHalfTile, rt[row], yt, lane);
  } else {
    float m, a;
    combine_pairs(pr, nq, -1, lane, m, a);
    st = RowStats{m + log2_hw(a), __builtin_nanf(""), 0.0f};
  }
  if (lane == 0) {
    lse2_out[row] = st.lse2;
    pt1_out[row] = st.pt1;
    row_loss[row] = st.loss;
  }
}

// Cross entropy of given bf16 logit rows (the standalone loss on logits):
// pass 1 online (max, sum) over the row, pass 2 rewrites every logit in
// place with (2^(y - lse2) - [j == t]) * scale in bf16 (same place, same
// size).  This form, one wave per row and one logit per lane and step,
// serves rows that are not 16-byte aligned.
__global__ void __launch_bounds__(64 * kWavesPerBlock)
ce_rows_bf16_kernel(uint16_t* __restrict__ z, int64_t ldz, const int32_t* __restrict__ targets,
                    int rows, int V, float scale, float* __restrict__ row_loss,
                    int64_t loss_stride) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  if (row >= rows) return;
  uint16_t* zr = z + (int64_t)row * ldz;
  const int t = targets[row];
  const bool t_ok = (t >= 0) && (t < V);
  const float zt = t_ok ? __uint_as_float((uint32_t)zr[t] << 16) : __builtin_nanf("");

  float m = -INFINITY, s = 0.0f;
  for (int j = lane; j < V; j += 64)
    online_add(to_log2(__uint_as_float((uint32_t)zr[j] << 16)), m, s);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const float m2 = __shfl_xor(m, off, 64);
    const float s2 = __shfl_xor(s, off, 64);
    combine(m, s, m2, s2);
  }
  const float lse2 = m + log2_hw(s);
  if (lane == 0)
    row_loss[(int64_t)row * loss_stride] = ((m - to_log2(zt)) + log2_hw(s)) * kLn2;
  for (int j = lane; j < V; j += 64) {
    const float p = exp2_hw(to_log2(__uint_as_float((uint32_t)zr[j] << 16)) - lse2);
    zr[j] = (uint16_t)bf16_bits((p - (j == t ? 1.0f : 0.0f)) * scale);
  }
}

// The same for rows that start 16-byte aligned, one 512-thread workgroup
// per row: pass 1 spreads the row's 16-byte pieces over the workgroup's
// threads, each thread's (max, sum) is combined over its wave with
// shuffles and over the waves through LDS in a fixed order, and pass 2 has
// every thread rewrite the pieces it read (after the barrier that ends
// pass 1, so no thread writes before every read of the row is done).  Eight
// waves per row keep enough requests in flight when a batch has few rows
// (a single wave per row left a 1024-row batch with four waves per CU).
constexpr int kRowBlockThreads = 512;
constexpr int kRowBlockWaves = kRowBlockThreads / 64;

template <int UNROLL>
__global__ void __launch_bounds__(kRowBlockThreads)
ce_rows_bf16_block_kernel(uint16_t* __restrict__ z, int64_t ldz,
                          const int32_t* __restrict__ targets, int V, float scale,
                          float* __restrict__ row_loss, int64_t loss_stride) {
  __shared__ float wm[kRowBlockWaves], ws[kRowBlockWaves];
  const int row = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  uint16_t* zr = z + (int64_t)row * ldz;
  const int t = targets[row];
  const bool t_ok = (t >= 0) && (t < V);
  const float zt = t_ok ? __uint_as_float((uint32_t)zr[t] << 16) : __builtin_nanf("");

  float m = -INFINITY, s = 0.0f;
  const int nvec = V >> 3;
  const u32x4* zv = reinterpret_cast<const u32x4*>(zr);
  for (int v0 = 0; v0 < nvec; v0 += kRowBlockThreads * UNROLL) {
    u32x4 x[UNROLL];
#pragma unroll
    for (int k = 0; k < UNROLL; ++k)
      if (v0 + tid + kRowBlockThreads * k < nvec) x[k] = zv[v0 + tid + kRowBlockThreads * k];
#pragma unroll
    for (int k = 0; k < UNROLL; ++k) {
      if (v0 + tid + kRowBlockThreads * k >= nvec) continue;
      online_add4(f32x4{bf16_lo(x[k][0]), bf16_hi(x[k][0]), bf16_lo(x[k][1]), bf16_hi(x[k][1])},
                  m, s);
      online_add4(f32x4{bf16_lo(x[k][2]), bf16_hi(x[k][2]), bf16_lo(x[k][3]), bf16_hi(x[k][3])},
                  m, s);
    }
  }
  for (int j = 8 * nvec + tid; j < V; j += kRowBlockThreads)
    online_add(to_log2(__uint_as_float((uint32_t)zr[j] << 16)), m, s);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const float m2 = __shfl_xor(m, off, 64);
    const float s2 = __shfl_xor(s, off, 64);
    combine(m, s, m2, s2);
  }
  if (lane == 0) {
    wm[tid >> 6] = m;
    ws[tid >> 6] = s;
  }
  __syncthreads();
  m = wm[0];
  s = ws[0];
#pragma unroll
  for (int w = 1; w < kRowBlockWaves; ++w) combine(m, s, wm[w], ws[w]);
  const float lse2 = m + log2_hw(s);
  if (tid == 0) row_loss[(int64_t)row * loss_stride] = ((m - to_log2(zt)) + log2_hw(s)) * kLn2;

  u32x4* zw = reinterpret_cast<u32x4*>(zr);
  for (int v0 = 0; v0 < nvec; v0 += kRowBlockThreads * UNROLL) {
    u32x4 x[UNROLL];
#pragma unroll
    for (int k = 0; k < UNROLL; ++k)
      if (v0 + tid + kRowBlockThreads * k < nvec) x[k] = zw[v0 + tid + kRowBlockThreads * k];
#pragma unroll
    for (int k = 0; k < UNROLL; ++k) {
      const int v = v0 + tid + kRowBlockThreads * k;
      if (v >= nvec) continue;
      u32x4 w;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int j = 8 * v + 2 * e;
        const float g0 =
            (exp2_hw(to_log2(bf16_lo(x[k][e])) - lse2) - (j == t ? 1.0f : 0.0f)) * scale;
        const float g1 =
            (exp2_hw(to_log2(bf16_hi(x[k][e])) - lse2) - (j + 1 == t ? 1.0f : 0.0f)) * scale;
        w[e] = pack_bf16x2(g0, g1);
      }
      zw[v] = w;
    }
  }
  for (int j = 8 * nvec + tid; j < V; j += kRowBlockThreads) {
    const float p = exp2_hw(to_log2(__uint_as_float((uint32_t)zr[j] << 16)) - lse2);
    zr[j] = (uint16_t)bf16_bits((p - (j == t ? 1.0f : 0.0f)) * scale);
  }
}

constexpr int kSumThreads = 1024;

// Thread j adds rows j, j + 1024, ... in that order (four loads in flight:
// the staged losses sit a row of grad_h apart, one cache line each), then
// a fixed tree combines the threads.
__global__ void __launch_bounds__(kSumThreads)
loss_sum_kernel(const float* __restrict__ row_loss, int64_t loss_stride, int rows,
                float scale, int first, float* __restrict__ loss) {
  __shared__ double part[kSumThreads];
  double acc = 0.0;
  int i = threadIdx.x;
  for (; i + 3 * kSumThreads < rows; i += 4 * kSumThreads) {
    const float a0 = row_loss[(int64_t)i * loss_stride];
    const float a1 = row_loss[(int64_t)(i + kSumThreads) * loss_stride];
    const float a2 = row_loss[(int64_t)(i + 2 * kSumThreads) * loss_stride];
    const float a3 = row_loss[(int64_t)(i + 3 * kSumThreads) * loss_stride];
    acc += (double)a0;
    acc += (double)a1;
    acc += (double)a2;
    acc += (double)a3;
  }
  for (; i < rows; i += kSumThreads) acc += (double)row_loss[(int64_t)i * loss_stride];
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
                          bool out_bf16, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  const dim3 grid((rows + kWavesPerBlock - 1) / kWavesPerBlock);
  const dim3 block(64 * kWavesPerBlock);
  // float4 path: row starts 16-byte aligned (base aligned, pitch % 4 == 0).
  const bool vec4 = ((ldz & 3) == 0) && ((reinterpret_cast<uintptr_t>(z) & 15) == 0);
  if (vec4 && out_bf16)
    hipLaunchKernelGGL((ce_rows_kernel<true, true>), grid, block, 0, s, z, ldz, targets,
                       rows, V, scale, row_loss, loss_stride);
  else if (vec4)
    hipLaunchKernelGGL((ce_rows_kernel<true, false>), grid, block, 0, s, z, ldz, targets,
                       rows, V, scale, row_loss, loss_stride);
  else if (out_bf16)
    hipLaunchKernelGGL((ce_rows_kernel<false, true>), grid, block, 0, s, z, ldz, targets,
                       rows, V, scale, row_loss, loss_stride);
  else
    hipLaunchKernelGGL((ce_rows_kernel<false, false>), grid, block, 0, s, z, ldz, targets,
                       rows, V, scale, row_loss, loss_stride);
  return hipGetLastError();
}

hipError_t launch_ce_rows_bf16(uint16_t* z, int64_t ldz, const int32_t* targets, int rows,
                               int V, float scale, float* row_loss, int64_t loss_stride,
                               hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  const dim3 grid((rows + kWavesPerBlock - 1) / kWavesPerBlock);
  const dim3 block(64 * kWavesPerBlock);
  const bool vec = ((ldz & 7) == 0) && ((reinterpret_cast<uintptr_t>(z) & 15) == 0);
  if (vec)
    hipLaunchKernelGGL((ce_rows_bf16_block_kernel<4>), dim3(rows), dim3(kRowBlockThreads), 0, s,
                       z, ldz, targets, V, scale, row_loss, loss_stride);
  else
    hipLaunchKernelGGL(ce_rows_bf16_kernel, grid, block, 0, s, z, ldz, targets, rows, V, scale,
                       row_loss, loss_stride);
  return hipGetLastError();
}

hipError_t launch_ce_rows_exp(uint16_t* u, int64_t ldu, const float* row_part, int64_t ldp,
                              const uint16_t* h, const uint16_t* W, int H,
                              const int32_t* targets, int rows, int V, float scale,
                              float* row_loss, int64_t loss_stride, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  // 16-byte pieces of u, h and W rows; one (max, sum) pair per half tile;
  // three floats (loss, lse2, pt1) staged per row.
  if ((V % 8) || (ldu % 8) || (H % 8) || loss_stride < 3 ||
      (reinterpret_cast<uintptr_t>(u) & 15) || (reinterpret_cast<uintptr_t>(h) & 15) ||
      (reinterpret_cast<uintptr_t>(W) & 15) || ldp < 2 * ((V + kHalfTile - 1) / kHalfTile))
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(ce_rows_exp_kernel, dim3((rows + kWavesPerBlock - 1) / kWavesPerBlock),
                     dim3(64 * kWavesPerBlock), 0, s, u, ldu, row_part, ldp, h, W, H, targets,
                     rows, V, row_loss, loss_stride);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_rewrite_blocks(u, ldu, row_part, ldp, row_loss + 1, row_loss + 2, loss_stride,
                               targets, rows, 0, V, scale, nullptr, s);
}

hipError_t launch_ce_target_mass(const uint16_t* u, int64_t ldu, const int32_t* targets,
                                 int rows, int v0, int n, float* rt, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if ((v0 % kHalfTile) || (ldu % 2) || (reinterpret_cast<uintptr_t>(u) & 3) || n < 1)
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(ce_target_mass_kernel, dim3((rows + kWavesPerBlock - 1) / kWavesPerBlock),
                     dim3(64 * kWavesPerBlock), 0, s, u, ldu, targets, rows, v0, n, rt);
  return hipGetLastError();
}

hipError_t launch_ce_stats_exp(const float* row_part, int64_t ldp, const float* rt,
                               const uint16_t* h, const uint16_t* W, int H,
                               const int32_t* targets, int rows, int V, float* lse2, float* pt1,
                               float* row_loss, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if ((H % 8) || (reinterpret_cast<uintptr_t>(h) & 15) || (reinterpret_cast<uintptr_t>(W) & 15) ||
      !rt || ldp < 2 * ((V + kHalfTile - 1) / kHalfTile))
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(ce_stats_exp_kernel, dim3((rows + kWavesPerBlock - 1) / kWavesPerBlock),
                     dim3(64 * kWavesPerBlock), 0, s, row_part, ldp, rt, h, W, H, targets, rows,
                     V, lse2, pt1, row_loss);
  return hipGetLastError();
}

hipError_t launch_ce_rewrite_exp(uint16_t* u, int64_t ldu, const float* row_part, int64_t ldp,
                                 const float* lse2, const float* pt1, const int32_t* targets,
                                 int rows, int v0, int n, float scale, const float* row_scale,
                                 hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  // 16-byte pieces of u rows; the chunk starts on a half tile.
  if ((n % 8) || (v0 % kHalfTile) || (ldu % 8) || (reinterpret_cast<uintptr_t>(u) & 15) ||
      ldp < 2 * ((n + kHalfTile - 1) / kHalfTile))
    return hipErrorInvalidValue;
  return launch_rewrite_blocks(u, ldu, row_part, ldp, lse2, pt1, 1, targets, rows, v0, n, scale,
                               row_scale, s);
}

hipError_t launch_loss_sum(const float* row_loss, int64_t loss_stride, int rows,
                           float scale, int first, float* loss, hipStream_t s) {
  hipLaunchKernelGGL(loss_sum_kernel, dim3(1), dim3(kSumThreads), 0, s, row_loss,
                     loss_stride, rows, scale, first, loss);
  return hipGetLastError();
}

}  // namespace flce
