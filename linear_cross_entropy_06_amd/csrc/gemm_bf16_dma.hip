// bf16 MFMA contraction with a direct-to-LDS operand pipeline (gfx950).
//
// Same contract as the generic kernel in gemm_bf16.hip (D[m][n] =
// sum_k A(m,k) B(n,k), stored as out[n * ldo + m]) for the shapes the
// loss head runs at scale: K a multiple of 64 unless both operands are
// m-contiguous, every contiguous extent and leading dimension a multiple of
// 8 elements, 16-byte aligned bases.
//
// CDNA4 design:
//  * 256x256 output tile per 256-thread workgroup; each wave64 owns a
//    128x128 quarter = 4x4 v_mfma_f32_32x32x16_bf16 blocks (256 fp32
//    accumulators per lane, one wave per SIMD).
//  * Operand tiles move L2 -> LDS with buffer_load_dwordx4 ... lds (no VGPR
//    staging).  A buffer (not global) load keeps the compiler's wait-count
//    model exact: it counts these requests on vmcnt only, so fragment reads
//    wait on partial lgkmcnt values instead of draining every LDS read.
//  * K advances in 64-wide slabs; an operand's slab is one 32 KiB tile.  LDS
//    holds a ring of five tile slots (160 KiB): while slab kt is multiplied,
//    B of slab kt+1 and A of slab kt+2 stream into the two slots that slab
//    kt-1 freed.  So every request has one to two slabs of MFMA work to
//    land in, and the 16 requests per thread are spread over the slab's
//    first three k steps (6/5/5) instead of bursting.
//  * Each operand stays in its memory layout in LDS:
//      k-contiguous  tile [row][64 k]   128 B rows, fragment = ds_read_b128
//      m-contiguous  tile [k][256 rows] 512 B rows, fragment = two
//                    ds_read_b64_tr_b16: a 16-lane group reads a 4(k) x 16(m)
//                    block as sixteen 8-byte pieces and each lane receives
//                    4 consecutive k of one m, i.e. an MFMA operand slice.
//    16-byte chunks are XOR-swizzled per row (the DMA source address is
//    permuted to match) so fragment reads hit distinct LDS banks.  The LDS
//    has 64 four-byte banks (256 B a cycle).  A k-contiguous row is 128 B,
//    so rows r and r + 1 fill the two bank halves.  XOR-ing the chunk with
//    (r >> 1) & 7 gives the 16 consecutive rows of a ds_read_b128 lane group
//    16 distinct (half, chunk) positions.  XOR-ing with r & 7 left rows r
//    and r + 8 on the same banks, a 2-way conflict measured at 2-3% of the
//    GEMM time.  An m-contiguous row is 512 B; its XOR,
//    4 (k & 3) ^ 2 ((k >> 3) & 1) of k-row k, makes lane groups 0/1, 2/3,
//    0/2 and 1/3 of a ds_read_b64_tr_b16 cover complementary bank sets.
//  * MFMA operands are double-buffered in registers: the fragments of the
//    next 16-wide k step are read while the current step's 16 MFMAs run.
//  * Tiles are walked in groups of 4 row panels (each XCD's ~32 concurrent
//    tiles form a 4 x 8 block sharing operand slabs in L2); optionally each
//    group starts its K walk at a rotated slab to spread L2 channel load.
//  * One barrier per slab, placed in the middle of the slab's last k step
//    so the MFMAs queued before it cover the wait.
//  * Rows beyond M/N are loaded from a clamped (valid) address and their
//    results are never stored.
//  * Epilogues go through LDS (each wave transposes 32 x 128 blocks in its
//    own 16 KiB) so every store covers whole 128-byte lines; edge tests and
//    the accumulate decision are taken once per tile, so a full tile's
//    stores carry no branches and no per-store waits.
#include "flce_internal.h"

#include <type_traits>

namespace flce {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int kBM = 256, kBN = 256, kBK = 64;
constexpr int kKSteps = kBK / 16;              // MFMA k steps per slab
constexpr int kTileBytes = 256 * kBK * 2;      // one operand slab: 32 KiB
constexpr int kSlots = 5;                      // LDS ring of operand tiles: 160 KiB
constexpr int kDmaPerOp = kTileBytes / (256 * 16);  // 8 DMA instructions per thread
constexpr int kXcds = 8;
// Buffer resource for the operand loads: raw (stride 0) addressing with a
// 2 GiB range (every piece offset is below 64 rows x the leading dimension,
// checked by gemm_bf16_dma_supported) and the dword data format.
constexpr int kBufferRange = 0x7fffffff;
constexpr int kBufferFlags = 0x00020000;

__device__ __forceinline__ int xcd_remap(int b, int total) {
  const int per = total / kXcds;
  if (b >= per * kXcds) return b;
  return (b % kXcds) * per + b / kXcds;
}

// Two floats rounded to nearest-even bf16 and packed (first in the low
// half): one v_cvt_pk_bf16_f32 on gfx950.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}

// z * log2(e) rounded once (never fused into a following operation).
__device__ __forceinline__ float to_log2(float z) {
#pragma clang fp contract(off)
  return z * 1.4426950408889634f;
}

// s_waitcnt with only vmcnt constrained (expcnt / lgkmcnt left open).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}
__device__ __forceinline__ void wait_lgkmcnt0() {
  __builtin_amdgcn_s_waitcnt(0xF | (0x3 << 14) | (0x7 << 4) | (0x0 << 8));
}

// Workgroup barrier without a memory fence (a fence would wait for every
// outstanding DMA).  The signal fences only stop the compiler from moving
// memory operations across the barrier; the hardware waits are explicit.
__device__ __forceinline__ void block_barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Per-thread DMA sources of one operand slab (kDmaPerOp 16-byte pieces).
// Instruction i of wave w fills 1 KiB block b = kDmaPerOp * w + i of the
// slab; lane l of that instruction lands at byte 16 * l of the block.  The
// pieces are addressed as 32-bit offsets from a per-tile panel base, which
// a buffer resource turns into loads.
template <bool KC>
struct DmaOperand {
  const char* base;            // panel origin: first row (kc) or first m (mc), k slab 0
  uint32_t voff[kDmaPerOp];    // per-lane byte offset of each piece from base
  int64_t kstep;               // bytes to advance per k slab
  int start = 0;               // first K slab of this tile (rotation)
  int kt_total = 1;            // K slabs
  int tail_range = kBufferRange;  // buffer range of the last slab (bytes)

  __device__ __forceinline__ void init(const uint16_t* ptr, int64_t ld, int row0,
                                       int rows_total, int wave, int lane) {
    base = reinterpret_cast<const char*>(ptr + (KC ? (int64_t)row0 * ld : (int64_t)row0));
#pragma unroll
    for (int i = 0; i < kDmaPerOp; ++i) {
      const int b = kDmaPerOp * wave + i;
      int64_t elem;
      if constexpr (KC) {
        // 8 rows of 64 k (128 B) per block; 8 chunks per row.
        const int row = 8 * b + (lane >> 3);
        const int c = (lane & 7) ^ ((row >> 1) & 7);  // bank swizzle, see the header
        int grow = row0 + row;
        grow = grow < rows_total ? grow : rows_total - 1;
        elem = (int64_t)(grow - row0) * ld + 8 * c;
      } else {
        // 2 k-rows of 256 m (512 B) per block; 32 chunks per row.
        const int krow = 2 * b + (lane >> 5);
        const int c = (lane & 31) ^ (4 * (krow & 3) ^ 2 * ((krow >> 3) & 1));  // see the header
        int gm = row0 + 8 * c;
        gm = gm <= rows_total - 8 ? gm : rows_total - 8;
        elem = (int64_t)krow * ld + (gm - row0);
      }
      voff[i] = (uint32_t)(elem * 2);
    }
    kstep = KC ? (int64_t)kBK * 2 : (int64_t)kBK * ld * 2;
  }

  // K % 64 valid k rows in the last slab (m-contiguous operands; 0: full).
  __device__ __forceinline__ void set_tail(int ktail, int64_t ld) {
    if (!KC && ktail != 0) tail_range = (int)((int64_t)ktail * ld * 2);
  }

  // Request slab kt (before rotation) into `slot`.  A partial last slab
  // (m-contiguous operands only, K % 64 != 0) gets a buffer range that ends
  // at its last valid k row: the pieces of later rows lie beyond it, and
  // the hardware's range check returns zeros for them (no memory is read),
  // so the missing k contribute exact zeros to the products.
  __device__ __forceinline__ void issue(int kt, char* slot, int wave) const {
    kt += start;
    if (kt >= kt_total) kt -= kt_total;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char*>(base + kt * kstep), (short)0,
        kt == kt_total - 1 ? tail_range : kBufferRange, kBufferFlags);
#pragma unroll
    for (int i = 0; i < kDmaPerOp; ++i) {
      const int b = kDmaPerOp * wave + i;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(slot + 1024 * b), 16, voff[i], 0,
                                               0, 0);
    }
  }
};

// Fragment reads of one operand for one 16-wide k step: 4 blocks of 32 rows.
template <bool KC>
struct FragOperand {
  uint32_t off[4];  // per-lane byte offsets inside a slab (see init)

  __device__ __forceinline__ void init(int wrow0, int lane) {
    if constexpr (KC) {
      // row = wrow0 + 32 i + (lane & 31); chunk = 2 kk + (lane >> 5).
      const int row = wrow0 + (lane & 31);
      const int x = (row >> 1) & 7;
      const int h = lane >> 5;
#pragma unroll
      for (int kk = 0; kk < kKSteps; ++kk) off[kk] = row * 128 + (((2 * kk + h) ^ x) * 16);
    } else {
      // 16-lane group G reads k rows 8 (G >> 1) + 4 t + (j >> 2) and
      // m = 16 (G & 1) + 4 (j & 3) .. + 3 of each 32-row block.
      const int G = lane >> 4, j = lane & 15;
      const int krow = 8 * (G >> 1) + (j >> 2);
      const int x = 4 * (krow & 3) ^ 2 * ((krow >> 3) & 1);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = wrow0 + 32 * i + 16 * (G & 1) + 4 * (j & 3);
        off[i] = krow * 512 + (((m >> 3) ^ x) * 16) + 8 * ((m >> 2) & 1);
      }
    }
  }

  // Ring slot s sits at LDS byte s * kTileBytes (the five slots are
  // declared in order), but ds_read's immediate offset holds 16 bits only.
  // For slots at 64 KiB and 128 KiB, off_hi[b - 1] = off + b * 64 KiB is
  // kept in registers, opaque to the compiler, and the read address is
  // written as slot + (off_hi - b * 64 KiB): the constant parts cancel into
  // the immediate, the slot object still names what is read (so loads into
  // other slots are known not to interfere), and no address is recomputed
  // inside the K loop.  Were the slots laid out otherwise, the addresses
  // would still be exact, only computed with extra adds.
  uint32_t off_hi[2][4];

  __device__ __forceinline__ void pin() {
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        off_hi[b][x] = off[x] + (uint32_t)(b + 1) * 65536u;
        asm volatile("" : "+v"(off_hi[b][x]));
      }
  }

  // Byte offset of piece x inside slot s (a compile-time index).
  __device__ __forceinline__ int piece(int s, int x) const {
    const int b = s * kTileBytes / 65536;
    return b == 0 ? (int)off[x] : (int)off_hi[b - 1][x] - b * 65536;
  }

  // Fragments of k step kk from `slab`, ring slot s.
  __device__ __forceinline__ void read(const char* slab, int s, int kk,
                                       bf16x8 (&f)[4]) const {
    if constexpr (KC) {
      const char* p = slab + piece(s, kk);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        f[i] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p + 4096 * i));
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const char* p = slab + piece(s, i) + kk * 8192;
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p + 2048));
        const u32x2 l2 = __builtin_bit_cast(u32x2, lo);
        const u32x2 h2 = __builtin_bit_cast(u32x2, hi);
        f[i] = __builtin_bit_cast(bf16x8, u32x4{l2[0], l2[1], h2[0], h2[1]});
      }
    }
  }
};

// 32x32x16 MFMAs over the 4x4 blocks, rows i0 .. i1 - 1 of the block grid.
// JO: B fragment outer (consecutive MFMAs share b[j]); the kernels with a
// k-contiguous B ran 0.3-0.8% faster that way (alternating runs), grad_W
// (both operands m-contiguous) 1.6% slower.  Every accumulator sees the
// same sequence of products either way.
template <int I0, int I1, bool JO = false>
__device__ __forceinline__ void mma(f32x16 (&acc)[4][4], const bf16x8 (&a)[4],
                                    const bf16x8 (&b)[4]) {
  if constexpr (JO) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int i = I0; i < I1; ++i)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
  } else {
#pragma unroll
    for (int i = I0; i < I1; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
  }
}

// Epilogues that may run with a K split (plain fp32 stores of each part).
template <int EPI>
constexpr bool kSplitK = EPI == kStoreF32;

template <bool A_KC, bool B_KC, int EPI, typename OutT>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
gemm_bf16_dma_kernel(GemmArgs g, int group_m) {
  // Five distinct LDS objects, one per ring slot: every DMA and every
  // fragment read names its slot statically (the K loop is unrolled by
  // five), so the compiler can tell which reads a DMA may overwrite and
  // never waits for an unrelated one.
  __shared__ __attribute__((aligned(1024))) char slot0[kTileBytes];
  __shared__ __attribute__((aligned(1024))) char slot1[kTileBytes];
  __shared__ __attribute__((aligned(1024))) char slot2[kTileBytes];
  __shared__ __attribute__((aligned(1024))) char slot3[kTileBytes];
  __shared__ __attribute__((aligned(1024))) char slot4[kTileBytes];
  char* const slots[kSlots] = {slot0, slot1, slot2, slot3, slot4};

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 1, wn = wave >> 1;

  const int tiles_m = (g.M + kBM - 1) / kBM;
  const int tiles_n = (g.N + kBN - 1) / kBN;
  const int t = xcd_remap(blockIdx.x, tiles_m * tiles_n);
  // Grouped order: group = group_m row panels x all column panels, row
  // panel fastest, so the ~32 tiles an XCD runs at once form a compact
  // block and share operand slabs in its L2.
  const int gm = group_m;
  const int per_group = gm * tiles_n;
  const int grp = t / per_group;
  const int first_m = grp * gm;
  const int gsize = min(tiles_m - first_m, gm);
  const int r = t - grp * per_group;
  // The integer divisions run on the vector unit; readfirstlane states that
  // the results are wave-uniform, so every address derived from them (the
  // DMA buffer resources above all) stays in scalar registers.
  const int tmi = __builtin_amdgcn_readfirstlane(first_m + r % gsize);
  const int tni = __builtin_amdgcn_readfirstlane(r / gsize);
  const int m0 = tmi * kBM, n0 = tni * kBN;

  // K split (fp32 part stores only): workgroup row blockIdx.y takes its own
  // run of slabs and its own output slice.  Compiled out of the other
  // epilogues, whose register budget has no room for it.
  // K slabs, the last one partial when K % 64 != 0 (its missing k read as
  // zeros).
  int KT = (g.K + kBK - 1) / kBK;
  int ktail = g.K % kBK;
  if (kSplitK<EPI> && g.splits > 1) {
    const int per = (KT + g.splits - 1) / g.splits;
    const int kt0 = (int)blockIdx.y * per;
    if (kt0 + per < KT) ktail = 0;  // only the last part holds the partial slab
    KT = min(per, KT - kt0);        // >= 1: checked on the host
    const int64_t k0 = (int64_t)kt0 * kBK;
    g.A = static_cast<const uint16_t*>(g.A) + (A_KC ? k0 : k0 * g.lda);
    g.B = static_cast<const uint16_t*>(g.B) + (B_KC ? k0 : k0 * g.ldb);
    g.out = static_cast<OutT*>(g.out) + (int64_t)blockIdx.y * g.split_stride;
  }

  DmaOperand<A_KC> da;
  DmaOperand<B_KC> db;
  da.init(static_cast<const uint16_t*>(g.A), g.lda, m0, g.M, wave, lane);
  db.init(static_cast<const uint16_t*>(g.B), g.ldb, n0, g.N, wave, lane);
  FragOperand<A_KC> fa;
  FragOperand<B_KC> fb;
  fa.init(wm * 128, lane);
  fb.init(wn * 128, lane);
  fa.pin();
  fb.pin();

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  da.kt_total = db.kt_total = KT;
  da.set_tail(ktail, g.lda);
  db.set_tail(ktail, g.ldb);
  da.start = db.start = __builtin_amdgcn_readfirstlane(
      g.stagger > 0 ? (int)(((unsigned)grp * (unsigned)g.stagger) % (unsigned)KT) : 0);
  // Prologue: A_0 -> slot 0, B_0 -> slot 1, A_1 -> slot 2; wait for the
  // first two (the A_1 requests, issued last, may still be in flight).
  da.issue(0, slots[0], wave);
  db.issue(0, slots[1], wave);
  da.issue(KT > 1 ? 1 : 0, slots[2], wave);
  wait_vmcnt<kDmaPerOp>();
  block_barrier();

  bf16x8 a0[4], b0[4], a1[4], b1[4];
  fa.read(slots[0], 0, 0, a0);
  fb.read(slots[1], 1, 0, b0);

  // LDS fragment reads per k step (ds_read_b128 per 32-row block, or two
  // ds_read_b64_tr_b16 for m-contiguous operands).
  constexpr int kReads = (A_KC ? 4 : 8) + (B_KC ? 4 : 8);
  // One slab kt.  Ring: A_kt sits in slot 2kt mod 5 and B_kt in slot
  // 2kt+1 mod 5.  During the slab, B_{kt+1} goes to slot 2kt+3 and A_{kt+2}
  // to slot 2kt+4 (mod 5): the slots of A_{kt-1} and B_{kt-1}, whose last
  // reads finished before the barrier that ended slab kt-1.  Requests past
  // the last slab re-fetch the last slab (L2 hits, never read) so the body
  // stays one basic block.
  auto slab_step = [&](int kt, int sa, int sb, int sa1, int sb1, int sa2)
      __attribute__((always_inline)) {
    const int kn1 = kt + 1 < KT ? kt + 1 : KT - 1;
    const int kn2 = kt + 2 < KT ? kt + 2 : KT - 1;
    fa.read(slots[sa], sa, 1, a1);
    fb.read(slots[sb], sb, 1, b1);
    db.issue(kn1, slots[sb1], wave);
    da.issue(kn2, slots[sa2], wave);
    mma<0, 4, B_KC>(acc, a0, b0);
    fa.read(slots[sa], sa, 2, a0);
    fb.read(slots[sb], sb, 2, b0);
    mma<0, 4, B_KC>(acc, a1, b1);
    fa.read(slots[sa], sa, 3, a1);
    fb.read(slots[sb], sb, 3, b1);
    mma<0, 4, B_KC>(acc, a0, b0);
    mma<0, 2, B_KC>(acc, a1, b1);
    // Issue order: each k step requests the fragments of the next step
    // while its 16 MFMAs run, and the 16 DMA requests are spread over the
    // first three steps (6, 5, 5), one per two or three MFMAs.  With an
    // m-contiguous A (two transposing reads per fragment) half the reads
    // go up front and the rest one per MFMA over the first eight (fewer
    // cycles per slab, measured); the k/k kernel issues all eight first.
    constexpr int kDma[3] = {6, 5, 5};
    constexpr int kPre = A_KC ? kReads : kReads / 2;
    constexpr int kSpread = kReads - kPre;
#pragma unroll
    for (int s = 0; s < 3; ++s) {
      __builtin_amdgcn_sched_group_barrier(0x100, kPre, 0);
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if ((q + 1) * kDma[s] / 16 > q * kDma[s] / 16)
          __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
        if (kSpread && q < 8) {
          const int nr = (q + 1) * kSpread / 8 - q * kSpread / 8;
          for (int r = 0; r < nr; ++r) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
      }
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
    // B_{kt+1} and everything before it landed (A_{kt+2}, the last
    // kDmaPerOp requests, may not have); every read of slab kt is done.
    __builtin_amdgcn_sched_barrier(0);
    wait_vmcnt<kDmaPerOp>();
    wait_lgkmcnt0();
    block_barrier();
    __builtin_amdgcn_sched_barrier(0);
    fa.read(slots[sa1], sa1, 0, a0);
    fb.read(slots[sb1], sb1, 0, b0);
    mma<2, 4, B_KC>(acc, a1, b1);
    __builtin_amdgcn_sched_group_barrier(0x100, kReads, 1);
    __builtin_amdgcn_sched_group_barrier(0x008, 8, 1);
  };
  // Slab kt with p = kt mod 5.
  auto step = [&](int kt, int p) __attribute__((always_inline)) {
    slab_step(kt, (2 * p) % kSlots, (2 * p + 1) % kSlots, (2 * p + 2) % kSlots,
              (2 * p + 3) % kSlots, (2 * p + 4) % kSlots);
  };
  int kt = 0;
  for (; kt + kSlots <= KT; kt += kSlots) {
    step(kt, 0);
    step(kt + 1, 1);
    step(kt + 2, 2);
    step(kt + 3, 3);
    step(kt + 4, 4);
  }
  if (kt < KT) step(kt, 0);
  if (kt + 1 < KT) step(kt + 1, 1);
  if (kt + 2 < KT) step(kt + 2, 2);
  if (kt + 3 < KT) step(kt + 3, 3);
  // The last slab's look-ahead requests must land before the workgroup's
  // LDS can be handed to another workgroup.
  wait_vmcnt<0>();
  // The epilogue works from an opaque copy of the lane index, so none of its
  // address arithmetic is hoisted above the K loop, where it would hold
  // registers the loop needs.
  int lane_ep = lane;
  asm volatile("" : "+v"(lane_ep));

  // Epilogue.  Accumulator r of lane l in block (i, j) is
  // D[m = 8*(r/4) + 4*(l/32) + r%4][n = l%32] of that 32x32 block.
  {
    // Each lane holds 16-byte pieces of 32 different output rows, so direct
    // stores would send 32 partial-line requests per instruction.  Each wave
    // instead transposes its results a block at a time through its own
    // 16 KiB of LDS, laid out [128 n][128 bytes of m] with the 16-byte chunk
    // index XOR-swizzled by row pair (conflict-free both ways), and reads it
    // back with 8 lanes per 128-byte row segment: every store (and, when
    // accumulating, every load of the previous value) covers whole lines.
    // All look-ahead DMA requests of every wave have landed once all waves
    // pass this barrier; the operand ring is free.
    const int lane = lane_ep;
    block_barrier();
    char* const buf = wave == 0 ? slot0 : wave == 1 ? slot1 : wave == 2 ? slot2 : slot3;
    const int c_rd = lane & 7;  // 16-byte chunk this lane reads back
    auto lds_off = [](int nl, int c) { return nl * 128 + ((c ^ ((nl >> 1) & 7)) << 4); };
    if constexpr (EPI == kExpBF16 || (EPI == kStoreOut && sizeof(OutT) == 2)) {
      // bf16 output, 32(m) x 128(n) blocks i = 2p, 2p+1 filling one
      // 128-byte row segment of m per row n; addresses are 32-bit offsets
      // from the wave's corner of the output (ldo < 2^22).  For the
      // exponentiated logits the values are 2^(z log2 e - mx) with mx the
      // column maximum over each 128-row half tile, and the (max, sum) pair
      // of every column and half tile is written too: lanes l and l ^ 32
      // hold the two halves of every 32-row block, so one shuffle completes
      // a column over the wave's 128 rows.  Tiles wholly inside the output
      // skip every per-element edge test.
      constexpr bool kExp = EPI == kExpBF16;
      auto bf16_body = [&](auto guard_tag) __attribute__((always_inline)) {
        constexpr bool kGuard = decltype(guard_tag)::value;
        constexpr float kL2e = 1.4426950408889634f;
        const int hl = lane >> 5;
        uint16_t* const corner = static_cast<uint16_t*>(g.out) +
                                 ((int64_t)(n0 + wn * 128) * g.ldo + (m0 + wm * 128));
        const uint32_t row8 = 8u * (uint32_t)g.ldo;
        const uint32_t lane_off = (uint32_t)(lane >> 3) * (uint32_t)g.ldo + 8u * c_rd;
        const int n_lane = n0 + wn * 128 + (lane >> 3);
        float mneg[4], ssum[4];
        if constexpr (kExp) {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            float mz = -__builtin_inff();
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
              for (int q = 0; q < 4; ++q)
                if (!kGuard || m0 + wm * 128 + i * 32 + 8 * q + 4 * hl < g.M)
#pragma unroll
                  for (int e = 0; e < 4; ++e) mz = fmaxf(mz, acc[i][j][4 * q + e]);
            mz = fmaxf(mz, __shfl_xor(mz, 32, 64));
            // No row of this half tile below M: nothing is stored for it.
            mneg[j] = mz == -__builtin_inff() ? 0.0f : -to_log2(mz);
            ssum[j] = 0.0f;
          }
        }
#pragma unroll
        for (int p = 0; p < 2; ++p) {
#pragma unroll
          for (int ii = 0; ii < 2; ++ii) {
            const int i = 2 * p + ii;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const int nl = 32 * j + (lane & 31);
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                float u[4];
                if constexpr (kExp) {
                  const bool ok = !kGuard || m0 + wm * 128 + i * 32 + 8 * q + 4 * hl < g.M;
#pragma unroll
                  for (int e = 0; e < 4; ++e)
                    u[e] = ok ? __builtin_amdgcn_exp2f(
                                    __builtin_fmaf(acc[i][j][4 * q + e], kL2e, mneg[j]))
                              : 0.0f;
                  ssum[j] += (u[0] + u[1]) + (u[2] + u[3]);
                } else {
#pragma unroll
                  for (int e = 0; e < 4; ++e) u[e] = acc[i][j][4 * q + e];
                }
                const u32x2 w = {pack_bf16x2(u[0], u[1]), pack_bf16x2(u[2], u[3])};
                *reinterpret_cast<u32x2*>(buf + lds_off(nl, 4 * ii + q) + 8 * hl) = w;
              }
            }
          }
          const bool m_ok = !kGuard || m0 + wm * 128 + 64 * p + 8 * c_rd < g.M;
#pragma unroll
          for (int t = 0; t < 16; ++t) {
            const int nl = 8 * t + (lane >> 3);
            const u32x4 v = *reinterpret_cast<const u32x4*>(buf + lds_off(nl, c_rd));
            // M % 8 == 0: a run of 8 is all in or all out
            if (!kGuard || (m_ok && n_lane + 8 * t < g.N))
              *reinterpret_cast<u32x4*>(corner + (lane_off + (uint32_t)t * row8 + 64u * p)) = v;
          }
        }
        if constexpr (kExp) {
#pragma unroll
          for (int j = 0; j < 4; ++j) ssum[j] += __shfl_xor(ssum[j], 32, 64);
          if (lane < 32 && m0 + wm * 128 < g.M) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const int n = n0 + wn * 128 + 32 * j + lane;
              if (!kGuard || n < g.N) {
                float* pr = g.row_part + (int64_t)n * g.ldp + 2 * (2 * tmi + wm);
                pr[0] = -mneg[j];
                pr[1] = ssum[j];
              }
            }
          }
        }
      };
      if (m0 + kBM <= g.M && n0 + kBN <= g.N)
        bf16_body(std::integral_constant<bool, false>{});
      else
        bf16_body(std::integral_constant<bool, true>{});
    } else {
      // fp32 output: one 32(m) x 128(n) block i at a time, double-buffered.
      // Addresses are 32-bit offsets from the wave's corner of the output
      // (its 128 x 128 block spans < 2^32 bytes: ldo < 2^22 floats).  The
      // accumulate and edge decisions are made once per tile, so a full
      // tile's stores carry no branches; without accumulation no memory
      // read is pending and the stores stream with no waits, and with it
      // each block's 16 previous values are fetched in one batch (loads and
      // stores share one completion counter, so a later wait drains both).
      auto f32_body = [&](auto guard_tag, auto acc_tag) __attribute__((always_inline)) {
        constexpr bool kGuard = decltype(guard_tag)::value;
        constexpr bool kAcc = decltype(acc_tag)::value;
        float* const corner = static_cast<float*>(g.out) +
                              ((int64_t)(n0 + wn * 128) * g.ldo + (m0 + wm * 128));
        const uint32_t row8 = 8u * (uint32_t)g.ldo;
        const uint32_t lane_off = (uint32_t)(lane >> 3) * (uint32_t)g.ldo + 4u * c_rd;
        const int n_lane = n0 + wn * 128 + (lane >> 3);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          char* const b = buf + (i & 1) * 16384;
          const int m = m0 + wm * 128 + i * 32 + 4 * c_rd;
          const bool m_ok = !kGuard || m < g.M;
          f32x4 old[16];
          if constexpr (kAcc) {
#pragma unroll
            for (int t = 0; t < 16; ++t) {
              const float* src = corner + (lane_off + (uint32_t)t * row8 + 32u * i);
              if (!kGuard || (m_ok && n_lane + 8 * t < g.N))
                old[t] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(src));
              else
                old[t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
            }
          }
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int nl = 32 * j + (lane & 31);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const f32x4 v = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                               acc[i][j][4 * q + 3]};
              *reinterpret_cast<f32x4*>(b + lds_off(nl, 2 * q + (lane >> 5))) = v;
            }
          }
#pragma unroll
          for (int t = 0; t < 16; ++t) {
            const int nl = 8 * t + (lane >> 3);
            f32x4 v = *reinterpret_cast<const f32x4*>(b + lds_off(nl, c_rd));
            if constexpr (kAcc) v += old[t];
            float* dst = corner + (lane_off + (uint32_t)t * row8 + 32u * i);
            if (!kGuard || (m_ok && n_lane + 8 * t < g.N)) {
              // The accumulated fp32 output is next read a whole chunk later
              // (or by the caller): streamed past the caches, measured 1-2%
              // faster for grad_W.  K-split parts, read back right away by
              // the summing pass, stay cached.
              if constexpr (EPI == kAccumF32)
                __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(dst));
              else
                *reinterpret_cast<f32x4*>(dst) = v;
            }
          }
        }
      };
      const bool full = m0 + kBM <= g.M && n0 + kBN <= g.N;
      if (EPI == kAccumF32 && g.beta) {
        if (full)
          f32_body(std::integral_constant<bool, false>{}, std::integral_constant<bool, true>{});
        else
          f32_body(std::integral_constant<bool, true>{}, std::integral_constant<bool, true>{});
      } else {
        if (full)
          f32_body(std::integral_constant<bool, false>{}, std::integral_constant<bool, false>{});
        else
          f32_body(std::integral_constant<bool, true>{}, std::integral_constant<bool, false>{});
      }
    }
  }
}

template <bool A_KC, bool B_KC, int EPI, typename OutT>
hipError_t launch_dma(const GemmArgs& g, hipStream_t s) {
  const int tiles_m = (g.M + kBM - 1) / kBM;
  const int tiles_n = (g.N + kBN - 1) / kBN;
  int gm = g.group_m > 0 ? g.group_m : 4;
  if (gm > tiles_m) gm = tiles_m;
  if (g.splits > 1 && !kSplitK<EPI>) return hipErrorInvalidValue;
  if (!tile_count_ok(g.M, g.N, kBM, kBN, 1) || g.splits > 65535) return hipErrorInvalidValue;
  hipLaunchKernelGGL((gemm_bf16_dma_kernel<A_KC, B_KC, EPI, OutT>),
                     dim3(tiles_m * tiles_n, g.splits > 1 ? g.splits : 1), dim3(256), 0, s, g,
                     gm);
  return hipGetLastError();
}

}  // namespace

bool gemm_bf16_dma_supported(bool a_kc, bool b_kc, const GemmArgs& g) {
  if (g.K <= 0 || g.M <= 0 || g.N <= 0) return false;
  // K % 64 != 0 (a partial last slab, zero-filled through the buffer
  // range) needs both operands m-contiguous, whose slab offsets grow with
  // the k row; the last slab's range (rows x leading dimension) stays
  // below 2^31 bytes.
  if (g.K % kBK != 0 && (a_kc || b_kc)) return false;
  // m runs of 8 (stores, m-contiguous A chunks); n runs of 8 only when B
  // is n-contiguous.
  if (g.M % 8 != 0 || (!b_kc && g.N % 8 != 0)) return false;
  if ((g.lda % 8) || (g.ldb % 8) || (g.ldo % 4)) return false;
  // Operand pieces are addressed by 32-bit offsets within 256 rows (k-
  // contiguous) or 64 k-rows (m-contiguous) of a leading dimension.
  if (g.lda >= (int64_t{1} << 22) || g.ldb >= (int64_t{1} << 22)) return false;
  // fp32 epilogue offsets within a wave's 128 output rows are 32-bit.
  if (g.ldo >= (int64_t{1} << 22)) return false;
  if (g.splits > 1) {  // every part gets at least one slab
    const int kt = (g.K + kBK - 1) / kBK, per = (kt + g.splits - 1) / g.splits;
    if ((g.splits - 1) * per >= kt || g.splits > 65535) return false;
  }
  const uintptr_t al = reinterpret_cast<uintptr_t>(g.A) | reinterpret_cast<uintptr_t>(g.B) |
                       reinterpret_cast<uintptr_t>(g.out);
  if (al & 15u) return false;
  return true;
}

hipError_t launch_gemm_bf16_dma(bool a_kc, bool b_kc, int epi, const GemmArgs& g,
                                hipStream_t s) {
  if (a_kc && b_kc && epi == kStoreF32) return launch_dma<true, true, kStoreF32, float>(g, s);
  if (a_kc && b_kc && epi == kExpBF16) {
    // 16-byte bf16 row pieces, (max, sum) pairs for every half tile
    if ((g.ldo % 8) || !g.row_part || g.ldp < 2 * ((g.M + kHalfTile - 1) / kHalfTile))
      return hipErrorInvalidValue;
    return launch_dma<true, true, kExpBF16, uint16_t>(g, s);
  }
  if (!a_kc && b_kc && epi == kStoreOut)
    return launch_dma<false, true, kStoreOut, uint16_t>(g, s);
  if (!a_kc && b_kc && epi == kStoreF32)  // K-split parts of grad_h
    return launch_dma<false, true, kStoreF32, float>(g, s);
  if (!a_kc && b_kc && epi == kAccumF32)  // fp32 grad_h over vocabulary chunks
    return launch_dma<false, true, kAccumF32, float>(g, s);
  if (!a_kc && !b_kc && epi == kAccumF32)
    return launch_dma<false, false, kAccumF32, float>(g, s);
  return hipErrorInvalidValue;
}

}  // namespace flce
