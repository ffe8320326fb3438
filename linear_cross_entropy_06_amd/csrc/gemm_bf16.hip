// bf16 MFMA contractions of the fused linear + cross-entropy head (gfx950).
//
// One kernel template serves the three dense contractions of the head
// (page 1, "Liger Kernel explained", section "What does Liger Kernel
// actually fuse": the logits and the gradient both come from the LM-head
// matmul, taken chunk by chunk):
//   logits    Z^T      = W   . h_c^T   (A = W   k-contiguous, B = h_c k-contiguous)
//   grad_h    grad_h^T = W^T . G^T     (A = W   m-contiguous, B = G   k-contiguous)
//   grad_W    grad_W^T = h^T . G       (A = h_c m-contiguous, B = G   n-contiguous)
// Every product is computed as D[m][n] = sum_k A(m,k) B(n,k) and written
// transposed, out[n * ldo + m], so each lane of a 32x32 MFMA output block
// holds runs of 4 consecutive m and stores them as one vector.
//
// Design (CDNA4):
//  * 256-thread workgroups (4 wave64s) on a 256x256 output tile, each wave
//    owning a 128x128 quarter = 4x4 blocks of v_mfma_f32_32x32x16_bf16 with
//    the 256 fp32 accumulators resident in registers.
//  * K is walked in 64-wide slabs staged in LDS (two 256x64 bf16 operand
//    tiles per slab, double buffered: 128 KiB of the 160 KiB LDS).  The next
//    slab's global loads are in flight while the current slab is multiplied.
//  * Both operands are stored in LDS as [row][k] with k contiguous, so every
//    MFMA fragment (8 consecutive k of one row) is one 16-byte LDS read.
//    Operands whose contraction index is NOT contiguous in memory are loaded
//    as 8x8 bf16 blocks (eight 16-byte row loads along m) and transposed in
//    registers with v_perm_b32 before the LDS write: no transposed copy of W,
//    h or G ever exists in HBM.
//  * 16-byte LDS chunks are XOR-swizzled by row so that the fragment reads
//    and both kinds of tile writes touch distinct banks within 8 lanes.
//  * Workgroup ids are remapped so that each of the 8 XCDs (one L2 each)
//    works on a contiguous range of tiles, and the tile order walks the
//    small operand's dimension fastest, so a panel of the large operand is
//    reused from L2 by consecutive tiles.
#include "flce_internal.h"

namespace flce {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kXcds = 8;

// Workgroups are dispatched round-robin over the XCDs: give XCD x the
// contiguous tile range [x * per, (x + 1) * per); the tail keeps its id.
__device__ __forceinline__ int xcd_remap(int b, int total) {
  const int per = total / kXcds;
  if (b >= per * kXcds) return b;
  return (b % kXcds) * per + b / kXcds;
}

// fp32 -> bf16 bits, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint32_t bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

template <int CPR>
__device__ __forceinline__ int swz(int row) {
  return (row ^ (row >> 3)) & (CPR - 1);
}

__device__ __forceinline__ u32x4 pack8(const uint16_t* e) {
  u32x4 r;
  r[0] = e[0] | ((uint32_t)e[1] << 16);
  r[1] = e[2] | ((uint32_t)e[3] << 16);
  r[2] = e[4] | ((uint32_t)e[5] << 16);
  r[3] = e[6] | ((uint32_t)e[7] << 16);
  return r;
}

// Global -> register -> LDS staging of one R x BK operand tile.
// KC: the tile's contraction index k is contiguous in memory
//     (element (row, k) at base[row * ld + k]).
// otherwise: the row index is contiguous (element (row, k) at
//     base[k * ld + row]); loaded as 8x8 blocks and transposed in registers.
template <int R, int BK, int NT, bool KC, bool VEC>
struct TileLoader {
  static constexpr int CPR = BK / 8;            // 16-byte chunks per LDS row
  static constexpr int KC_CHUNKS = R * CPR;
  static constexpr int KC_PT = (KC_CHUNKS + NT - 1) / NT;
  static constexpr int MB = R / 8;              // 8-row blocks
  static constexpr int NBLK = MB * (BK / 8);    // 8x8 blocks per tile
  static constexpr int BPT = (NBLK + NT - 1) / NT;
  static constexpr int NREG = KC ? KC_PT : BPT * 8;
  static_assert(R % 32 == 0 && BK % 16 == 0, "tile shape");

  u32x4 r[NREG];

  __device__ __forceinline__ void load(const uint16_t* __restrict__ base,
                                       int64_t ld, int row0, int rows_total,
                                       int k0, int K, int tid) {
    if constexpr (KC) {
#pragma unroll
      for (int i = 0; i < KC_PT; ++i) {
        const int q = tid + NT * i;
        const int row = q / CPR, c = q % CPR;
        const int grow = row0 + row, gk = k0 + c * 8;
        const bool ok = (q < KC_CHUNKS) && grow < rows_total;
        if constexpr (VEC) {
          if (ok && gk < K)
            r[i] = *reinterpret_cast<const u32x4*>(base + (int64_t)grow * ld + gk);
          else
            r[i] = u32x4{0u, 0u, 0u, 0u};
        } else {
          uint16_t e[8];
#pragma unroll
          for (int j = 0; j < 8; ++j)
            e[j] = (ok && gk + j < K) ? base[(int64_t)grow * ld + gk + j] : (uint16_t)0;
          r[i] = pack8(e);
        }
      }
    } else {
#pragma unroll
      for (int bi = 0; bi < BPT; ++bi) {
        const int blk = tid + NT * bi;
        const int mb = blk % MB, kb = blk / MB;
        const int gm = row0 + mb * 8;
        const bool okb = blk < NBLK;
        u32x4 v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int gk = k0 + kb * 8 + e;
          if constexpr (VEC) {
            if (okb && gk < K && gm < rows_total)
              v[e] = *reinterpret_cast<const u32x4*>(base + (int64_t)gk * ld + gm);
            else
              v[e] = u32x4{0u, 0u, 0u, 0u};
          } else {
            uint16_t x[8];
#pragma unroll
            for (int j = 0; j < 8; ++j)
              x[j] = (okb && gk < K && gm + j < rows_total)
                         ? base[(int64_t)gk * ld + gm + j] : (uint16_t)0;
            v[e] = pack8(x);
          }
        }
        // 8x8 transpose: output q (row gm + q) holds k = kb*8 + 0..7; its
        // 32-bit word p packs k = 2p (low half) and k = 2p + 1 (high half),
        // i.e. element q of input rows 2p and 2p + 1.
#pragma unroll
        for (int q = 0; q < 8; ++q) {
#pragma unroll
          for (int p = 0; p < 4; ++p) {
            const uint32_t lo = v[2 * p][q >> 1];
            const uint32_t hi = v[2 * p + 1][q >> 1];
            r[bi * 8 + q][p] = (q & 1) ? __builtin_amdgcn_perm(hi, lo, 0x07060302u)
                                       : __builtin_amdgcn_perm(hi, lo, 0x05040100u);
          }
        }
      }
    }
  }

  __device__ __forceinline__ void store(uint16_t* __restrict__ S, int tid) const {
    if constexpr (KC) {
#pragma unroll
      for (int i = 0; i < KC_PT; ++i) {
        const int q = tid + NT * i;
        if (q < KC_CHUNKS) {
          const int row = q / CPR, c = q % CPR;
          *reinterpret_cast<u32x4*>(S + row * BK + ((c ^ swz<CPR>(row)) * 8)) = r[i];
        }
      }
    } else {
#pragma unroll
      for (int bi = 0; bi < BPT; ++bi) {
        const int blk = tid + NT * bi;
        if (blk < NBLK) {
          const int mb = blk % MB, kb = blk / MB;
#pragma unroll
          for (int q = 0; q < 8; ++q) {
            const int row = mb * 8 + q;
            *reinterpret_cast<u32x4*>(S + row * BK + ((kb ^ swz<CPR>(row)) * 8)) =
                r[bi * 8 + q];
          }
        }
      }
    }
  }
};

template <int BM, int BN, int BK, int WM, int WN>
struct Tile {
  static constexpr int kBM = BM, kBN = BN, kBK = BK, kWM = WM, kWN = WN;
  static constexpr int WAVES_M = BM / WM, WAVES_N = BN / WN;
  static constexpr int NT = 64 * WAVES_M * WAVES_N;
  static constexpr int TM = WM / 32, TN = WN / 32;
  static constexpr int CPR = BK / 8;
  static constexpr int LDS_ELEMS = 2 * (BM + BN) * BK;  // double buffered
};

template <class T, bool A_KC, bool B_KC, bool VEC, int EPI, typename OutT>
__global__ void __launch_bounds__(T::NT)
__attribute__((amdgpu_waves_per_eu(1, 1)))
gemm_bf16_kernel(GemmArgs g, int m_fastest) {
  constexpr int BM = T::kBM, BN = T::kBN, BK = T::kBK;
  constexpr int NT = T::NT, TM = T::TM, TN = T::TN, CPR = T::CPR;
  __shared__ __attribute__((aligned(16))) uint16_t smem[T::LDS_ELEMS];
  // stage s: A tile at smem + s * STAGE, B tile right after it
  constexpr int STAGE = (BM + BN) * BK;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave % T::WAVES_M, wn = wave / T::WAVES_M;

  const int tiles_m = (g.M + BM - 1) / BM;
  const int tiles_n = (g.N + BN - 1) / BN;
  const int t = xcd_remap(blockIdx.x, tiles_m * tiles_n);
  int tmi, tni;
  if (m_fastest) {
    tmi = t % tiles_m;
    tni = t / tiles_m;
  } else {
    tmi = t / tiles_n;
    tni = t % tiles_n;
  }
  const int m0 = tmi * BM, n0 = tni * BN;

  const uint16_t* __restrict__ Ap = static_cast<const uint16_t*>(g.A);
  const uint16_t* __restrict__ Bp = static_cast<const uint16_t*>(g.B);

  TileLoader<BM, BK, NT, A_KC, VEC> la;
  TileLoader<BN, BK, NT, B_KC, VEC> lb;

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const int KT = (g.K + BK - 1) / BK;
  la.load(Ap, g.lda, m0, g.M, 0, g.K, tid);
  lb.load(Bp, g.ldb, n0, g.N, 0, g.K, tid);
  la.store(smem, tid);
  lb.store(smem + BM * BK, tid);
  __syncthreads();

  for (int kt = 0; kt < KT; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < KT) {
      la.load(Ap, g.lda, m0, g.M, (kt + 1) * BK, g.K, tid);
      lb.load(Bp, g.ldb, n0, g.N, (kt + 1) * BK, g.K, tid);
    }
    const uint16_t* __restrict__ Sa = smem + cur * STAGE;
    const uint16_t* __restrict__ Sb = smem + cur * STAGE + BM * BK;
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      const int c = 2 * kk + (lane >> 5);
      bf16x8 a[TM], b[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int row = wm * T::kWM + i * 32 + (lane & 31);
        a[i] = __builtin_bit_cast(
            bf16x8, *reinterpret_cast<const u32x4*>(Sa + row * BK + ((c ^ swz<CPR>(row)) * 8)));
      }
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int row = wn * T::kWN + j * 32 + (lane & 31);
        b[j] = __builtin_bit_cast(
            bf16x8, *reinterpret_cast<const u32x4*>(Sb + row * BK + ((c ^ swz<CPR>(row)) * 8)));
      }
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < KT) {
      la.store(smem + (cur ^ 1) * STAGE, tid);
      lb.store(smem + (cur ^ 1) * STAGE + BM * BK, tid);
    }
    __syncthreads();
  }

  // Epilogue.  Accumulator r of lane l in block (i, j) is
  // D[m = 8*(r/4) + 4*(l/32) + r%4][n = l%32] of that 32x32 block.
#pragma unroll
  for (int i = 0; i < TM; ++i) {
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int n = n0 + wn * T::kWN + j * 32 + (lane & 31);
      if (n >= g.N) continue;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int m = m0 + wm * T::kWM + i * 32 + 8 * q + 4 * (lane >> 5);
        const f32x4 v = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                         acc[i][j][4 * q + 3]};
        const int64_t off = (int64_t)n * g.ldo + m;
        if constexpr (EPI == kStoreOut && sizeof(OutT) == 2) {
          uint16_t* o = static_cast<uint16_t*>(g.out) + off;
          if (VEC && m + 3 < g.M) {
            u32x2 w;
            w[0] = bf16_bits(v[0]) | (bf16_bits(v[1]) << 16);
            w[1] = bf16_bits(v[2]) | (bf16_bits(v[3]) << 16);
            *reinterpret_cast<u32x2*>(o) = w;
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (m + e < g.M) o[e] = (uint16_t)bf16_bits(v[e]);
          }
        } else {
          float* o = static_cast<float*>(g.out) + off;
          if (VEC && m + 3 < g.M) {
            f32x4 w = v;
            if (EPI == kAccumF32 && g.beta) w += *reinterpret_cast<const f32x4*>(o);
            *reinterpret_cast<f32x4*>(o) = w;
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (m + e < g.M)
                o[e] = (EPI == kAccumF32 && g.beta) ? o[e] + v[e] : v[e];
          }
        }
      }
    }
  }
}

using TileBig = Tile<256, 256, 64, 128, 128>;

template <class T, bool A_KC, bool B_KC, bool VEC, int EPI, typename OutT>
hipError_t launch_t(const GemmArgs& g, int m_fastest, hipStream_t s) {
  if (!tile_count_ok(g.M, g.N, T::kBM, T::kBN, 1)) return hipErrorInvalidValue;
  const int tiles = ((g.M + T::kBM - 1) / T::kBM) * ((g.N + T::kBN - 1) / T::kBN);
  hipLaunchKernelGGL((gemm_bf16_kernel<T, A_KC, B_KC, VEC, EPI, OutT>), dim3(tiles),
                     dim3(T::NT), 0, s, g, m_fastest);
  return hipGetLastError();
}

template <bool A_KC, bool B_KC, int EPI, typename OutT>
hipError_t launch_layout(bool vec, const GemmArgs& g, int m_fastest, hipStream_t s) {
  if (vec) return launch_t<TileBig, A_KC, B_KC, true, EPI, OutT>(g, m_fastest, s);
  return launch_t<TileBig, A_KC, B_KC, false, EPI, OutT>(g, m_fastest, s);
}

}  // namespace

// The direct-to-LDS pipeline serves every shape it supports; this
// register-staged kernel takes the rest.
bool gemm_bf16_uses_dma(bool a_kc, bool b_kc, bool vec, const GemmArgs& g) {
  return vec && gemm_bf16_dma_supported(a_kc, b_kc, g);
}

hipError_t launch_gemm_bf16(bool a_kc, bool b_kc, int epi, bool vec,
                            const GemmArgs& g, hipStream_t s) {
  if (g.M <= 0 || g.N <= 0) return hipSuccess;
  // Walk the dimension of the smaller operand fastest, so that a panel of
  // the larger operand stays in L2 across consecutive tiles.
  const int m_fastest = g.M < g.N ? 1 : 0;
  if (gemm_bf16_uses_dma(a_kc, b_kc, vec, g)) return launch_gemm_bf16_dma(a_kc, b_kc, epi, g, s);
  // Exponentiated logits and K splits exist on the direct-to-LDS kernel only.
  if (epi == kExpBF16 || g.splits > 1) return hipErrorInvalidValue;
  if (a_kc && b_kc && epi == kStoreF32)       // logits
    return launch_layout<true, true, kStoreF32, float>(vec, g, m_fastest, s);
  if (!a_kc && b_kc && epi == kStoreOut)      // grad_h (bf16 out)
    return launch_layout<false, true, kStoreOut, uint16_t>(vec, g, m_fastest, s);
  if (!a_kc && !b_kc && epi == kAccumF32)     // grad_W
    return launch_layout<false, false, kAccumF32, float>(vec, g, m_fastest, s);
  return hipErrorInvalidValue;
}

}  // namespace flce
