// C ABI of the fused linear + cross-entropy head: argument checks, the token
// chunk loop and the kernel launches.  Host code, plus the one static device
// array of the allocation-free entry point at the end of the file; nothing
// here allocates, synchronises or reads device memory.
//
// Per token chunk of C rows (page 1, "Liger Kernel explained", section
// "What does Liger Kernel actually fuse": only a chunk of logits is ever
// resident, and its gradient is formed before the next chunk):
//   1. logits   Z[C, V] = h_c W^T (workspace)                 MFMA
//               bf16 inputs on the direct-to-LDS kernel: stored as
//               u = 2^(Z log2 e - mx) in bf16 with one (mx, sum u) pair per
//               128-column half tile, so the row pass reads 2 bytes per
//               logit and the workspace is chunk * V * 2 bytes plus the
//               pairs; otherwise fp32 Z
//   2. rows     lse, row loss -> staged in grad_h's rows of the chunk;
//               the logits rewritten in place as G = (softmax - onehot) / N
//   3. loss     *loss (+)= sum(staged row losses) / N         fixed order
//   4. grad_h   grad_h_c = G W      (overwrites the staged losses)
//   5. grad_W   grad_W (+)= G^T h_c (written by the first chunk, then
//               accumulated in fp32)
#include "flce.h"
#include "flce_internal.h"

#include <stdint.h>

#include <mutex>

namespace {

constexpr int64_t kMaxDim = (int64_t(1) << 31) - 1;

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline bool dims_ok(int64_t a) { return a >= 1 && a <= kMaxDim; }

// rows x cols elements stay below 2^56, so every workspace size (a few such
// areas times at most 8 bytes) is exact in int64.  Positive arguments.
inline bool area_ok(int64_t rows, int64_t cols) { return rows <= (int64_t{1} << 56) / cols; }

inline bool dtype_ok(flce_dtype dt) { return dt == FLCE_BF16 || dt == FLCE_F32; }

inline int64_t esize(flce_dtype dt) { return dt == FLCE_BF16 ? 2 : 4; }

inline hipError_t gemm(flce_dtype dt, bool a_kc, bool b_kc, int epi, bool vec,
                       const flce::GemmArgs& g, hipStream_t s) {
  return dt == FLCE_BF16 ? flce::launch_gemm_bf16(a_kc, b_kc, epi, vec, g, s)
                         : flce::launch_gemm_f32(a_kc, b_kc, epi, g, s);
}

// The bf16 path whose logits kernel writes exponentiated bf16 logits and
// their (max, sum) pairs (direct-to-LDS kernel: K = H a multiple of 64,
// V a multiple of 8, both leading dimensions below 2^22).  Every other case
// keeps fp32 logits.
inline bool exp_path(int64_t H, int64_t V, flce_dtype dt) {
  return dt == FLCE_BF16 && V % 8 == 0 && H % 64 == 0 && H < (int64_t{1} << 22) &&
         V < (int64_t{1} << 22);
}

// (max, sum) pairs per row on the exponentiated path.
inline int64_t n_half_tiles(int64_t V) { return (V + flce::kHalfTile - 1) / flce::kHalfTile; }

// K split of the grad_h contraction (H x rows output, K = V: few output
// tiles, each a long run of K slabs).  Each of s consecutive K runs is a
// work item with its own fp32 part, summed afterwards in a fixed order.
// The split s in {1, 2, 4, 8} minimises the estimated time relative to a
// perfectly filled chip: the rounds of 256 CUs the tiles * s items take,
// over s, plus the summing pass (it reads s fp32 parts at about 5 TB/s
// while the contraction runs at about 1.4 PFLOP/s: 560 s / V of the
// contraction's time).  V % 64 == 0, each part keeps at least 16 slabs of
// 64 and the parts fit in `room` bytes.  At H = 4096: 64 tiles take 4 parts, 128 take
// 2, 256 none; at H = 3584 and 4096 rows, 224 tiles take 8 (7 full
// rounds).
constexpr int64_t kCUs = 256;
inline int grad_h_splits(int64_t H, int64_t rows, int64_t V, int64_t room) {
  const int64_t tiles = ((H + 255) / 256) * ((rows + 255) / 256);
  if (V % 64 != 0) return 1;  // the split runs on the direct-to-LDS kernel only
  int best = 1;
  double best_t = 1e300;
  for (int s = 1; s <= 8; s *= 2) {
    if (s > 1 && (V / 64 < 16 * s || s * rows * H * 4 > room)) break;
    const int64_t items = tiles * s;
    const double rounds = static_cast<double>((items + kCUs - 1) / kCUs);
    const double t = rounds / s / (static_cast<double>(tiles) / kCUs) +
                     (s > 1 ? 560.0 * s / static_cast<double>(V) : 0.0);
    if (t < best_t - 1e-9) {
      best_t = t;
      best = s;
    }
  }
  return best;
}

// Rows of the fp32 [rows][H] part buffer the K split needs: the larger of
// splits(rows) * rows over the chunk sizes that occur (C, and N mod C).
inline int64_t split_scratch_rows(int64_t N, int64_t H, int64_t C, int64_t V, int64_t room) {
  int64_t best = 0;
  for (int64_t r : {C, N % C}) {
    if (r <= 0) continue;
    const int s = grad_h_splits(H, r, V, room);
    if (s > 1 && s * r > best) best = s * r;
  }
  return best;
}

inline int64_t round_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

// Byte offsets of the exponentiated path's workspace regions: u [C][V]
// bf16, the pairs [C][ceil(V/128)][2], then the grad_h K-split parts in
// whatever remains of C * V * 4 bytes (`room`).
struct ExpLayout {
  int64_t pairs, parts, room, total;
};
inline ExpLayout exp_layout(int64_t N, int64_t C, int64_t H, int64_t V) {
  ExpLayout l;
  l.pairs = round_up(C * V * 2, 256);
  l.parts = round_up(l.pairs + C * n_half_tiles(V) * 8, 256);
  l.room = C * V * 4 > l.parts ? C * V * 4 - l.parts : 0;
  l.total = l.parts + split_scratch_rows(N, H, C, V, l.room) * H * 4;
  return l;
}

// The token-chunked path runs exponentiated when its layout fits the fp32
// logits' C * V * 4 bytes (it does unless the chunk is a handful of rows of
// a tiny vocabulary), so the workspace never exceeds C * V * 4.
inline bool use_exp(int64_t N, int64_t C, int64_t H, int64_t V, flce_dtype dt) {
  return exp_path(H, V, dt) && exp_layout(N, C, H, V).parts <= C * V * 4;
}

}  // namespace

extern "C" size_t flce_workspace_bytes(int64_t N, int64_t H, int64_t V, int64_t chunk,
                                       flce_dtype dt) {
  if (!dims_ok(N) || !dims_ok(H) || !dims_ok(V) || chunk < 1 || !dtype_ok(dt)) return 0;
  const int64_t C = chunk < N ? chunk : N;
  if (!area_ok(C, V) || !area_ok(C, H)) return 0;
  // bf16 logits of one chunk + 2 floats per row and half tile (+ grad_h
  // K-split parts for short chunks)
  if (use_exp(N, C, H, V, dt)) return static_cast<size_t>(exp_layout(N, C, H, V).total);
  return static_cast<size_t>(C) * static_cast<size_t>(V) * 4u;  // fp32 logits of one chunk
}

extern "C" int64_t flce_launch_count(int64_t N, int64_t chunk) {
  if (!dims_ok(N) || chunk < 1) return 0;
  const int64_t C = chunk < N ? chunk : N;
  return FLCE_STEPS * ((N + C - 1) / C);
}

namespace {

// Records events[2k] / events[2k+1] around step k when events != nullptr.
struct Marks {
  hipEvent_t* ev;
  hipStream_t s;
  int64_t k = 0;
  void before() {
    if (ev) (void)hipEventRecord(ev[2 * k], s);
  }
  void after() {
    if (ev) (void)hipEventRecord(ev[2 * k + 1], s);
    ++k;
  }
};

// An RMSNorm in front of the head (flce_fwd_bwd_rmsnorm): per token chunk,
// h_c = rmsnorm(x_c) is formed into h_buf before step 1, step 4 writes
// grad_h_c into g_buf, and after step 5 the norm's backward turns g_buf into
// the chunk's grad_x rows and adds to grad_gamma.
struct NormSide {
  const void* x;
  const void* gamma;
  float eps;
  void* grad_x;
  float* grad_gamma;
  char* h_buf;   // [C][H] dt
  char* g_buf;   // [C][H] dt
  float* rinv;   // [C]
  float* part;   // [rmsnorm_groups(C)][H]
};

flce_status fwd_bwd_impl(const void* h, const void* W, const int32_t* targets, int64_t N,
                         int64_t H, int64_t V, int64_t chunk, float* loss, void* grad_h,
                         float* grad_W, void* workspace, size_t workspace_bytes,
                         flce_dtype dt, hipStream_t stream, hipEvent_t* events,
                         int64_t n_events, bool accumulate, const NormSide* ns = nullptr) {
  if (!h || !W || !targets || !loss || !grad_h || !grad_W || !workspace)
    return FLCE_ERR_INVALID_ARG;
  if (!dims_ok(N) || !dims_ok(H) || !dims_ok(V) || chunk < 1 || !dtype_ok(dt))
    return FLCE_ERR_INVALID_ARG;
  if (H % 8 != 0) return FLCE_ERR_UNSUPPORTED;
  if (!aligned16(h) || !aligned16(W) || !aligned16(grad_h) || !aligned16(grad_W) ||
      !aligned16(workspace) || (reinterpret_cast<uintptr_t>(targets) & 3u) ||
      (reinterpret_cast<uintptr_t>(loss) & 3u))
    return FLCE_ERR_UNSUPPORTED;
  if (events && n_events < 2 * flce_launch_count(N, chunk)) return FLCE_ERR_INVALID_ARG;
  const size_t need = flce_workspace_bytes(N, H, V, chunk, dt);
  if (need == 0) return FLCE_ERR_UNSUPPORTED;  // a chunk of logits beyond 2^56 elements
  if (workspace_bytes < need) return FLCE_ERR_WORKSPACE;

  Marks mk{events, stream};
  const int64_t C = chunk < N ? chunk : N;
  const int64_t es = esize(dt);
  const bool bf16 = dt == FLCE_BF16;
  const bool vec = (V % 8) == 0;
  const bool expo = use_exp(N, C, H, V, dt);
  const float inv_n = static_cast<float>(1.0 / static_cast<double>(N));
  // Workspace: fp32 logits Z (row pitch V) that become G in place (bf16 G in
  // the first half of each row, fp32 G over the row), or on the
  // exponentiated path bf16 u (row pitch V) that becomes bf16 G in place,
  // followed by the rows' (max, sum) pairs.
  const int64_t ldg = expo ? V : (bf16 ? 2 * V : V);
  float* z = static_cast<float*>(workspace);
  uint16_t* u = static_cast<uint16_t*>(workspace);
  const int64_t ldp = 2 * n_half_tiles(V);
  const ExpLayout lay = exp_layout(N, C, H, V);
  float* pairs = reinterpret_cast<float*>(static_cast<char*>(workspace) + lay.pairs);
  float* parts = reinterpret_cast<float*>(static_cast<char*>(workspace) + lay.parts);
  void* g_base = workspace;
  const int64_t loss_stride = H * es / 4;  // floats between staged row losses

  for (int64_t r0 = 0; r0 < N; r0 += C) {
    const int rows = static_cast<int>((N - r0) < C ? (N - r0) : C);
    const char* hc = static_cast<const char*>(h) + r0 * H * es;
    char* ghc = static_cast<char*>(grad_h) + r0 * H * es;
    hipError_t e;
    if (ns) {
      // 0. h_c = rmsnorm(x_c) into the workspace; grad_h_c goes there too.
      if (flce::launch_rmsnorm_fwd(hc, ns->gamma, ns->eps, rows, static_cast<int>(H), ns->h_buf,
                                   ns->rinv, bf16, stream) != hipSuccess)
        return FLCE_ERR_HIP;
      hc = ns->h_buf;
      ghc = ns->g_buf;
    }
    float* staged = reinterpret_cast<float*>(ghc);

    // 1. Z^T = W . h_c^T, stored as Z[i][j] (row pitch V), or as its
    //    exponentiated bf16 form with (max, sum) pairs.
    flce::GemmArgs g1{W, H, hc, H, workspace, V, static_cast<int>(V), rows, static_cast<int>(H),
                      0};
    g1.group_m = 4;
    g1.stagger = 37;
    if (expo) {
      g1.row_part = pairs;
      g1.ldp = ldp;
    }
    mk.before();
    e = expo ? flce::launch_gemm_bf16(true, true, flce::kExpBF16, vec, g1, stream)
             : gemm(dt, true, true, flce::kStoreF32, vec, g1, stream);
    mk.after();
    if (e != hipSuccess) return FLCE_ERR_HIP;

    // 2. lse and row losses (staged in the chunk's grad_h rows); the logits
    //    become G in place.
    mk.before();
    e = expo ? flce::launch_ce_rows_exp(u, V, pairs, ldp, static_cast<const uint16_t*>(
                                            static_cast<const void*>(hc)),
                                        static_cast<const uint16_t*>(W), static_cast<int>(H),
                                        targets + r0, rows, static_cast<int>(V), inv_n, staged,
                                        loss_stride, stream)
             : flce::launch_ce_rows(z, V, targets + r0, rows, static_cast<int>(V), inv_n,
                                    staged, loss_stride, bf16, stream);
    mk.after();
    if (e != hipSuccess) return FLCE_ERR_HIP;

    // 3. running mean loss.
    mk.before();
    e = flce::launch_loss_sum(staged, loss_stride, rows, inv_n, r0 == 0 ? 1 : 0, loss, stream);
    mk.after();
    if (e != hipSuccess) return FLCE_ERR_HIP;

    // 4. grad_h_c^T = W^T . G^T: A(m = hidden, k = vocab) = W[k][m],
    //    B(n = token, k = vocab) = G[n][k].
    //    Few output tiles (short chunks): K split into fp32 parts in the
    //    workspace, then summed into grad_h in a fixed order (both launches
    //    are this step).
    flce::GemmArgs g4{W, H, g_base, ldg, ghc, H, static_cast<int>(H), rows, static_cast<int>(V),
                      0};
    g4.group_m = 4;
    const int splits = expo ? grad_h_splits(H, rows, V, lay.room) : 1;
    mk.before();
    if (splits > 1) {
      g4.out = parts;
      g4.splits = splits;
      g4.split_stride = static_cast<int64_t>(rows) * H;
      e = flce::launch_gemm_bf16(false, true, flce::kStoreF32, vec, g4, stream);
      if (e == hipSuccess)
        e = flce::launch_sum_parts_bf16(parts, splits, static_cast<int64_t>(rows) * H,
                                        reinterpret_cast<uint16_t*>(ghc),
                                        static_cast<int64_t>(rows) * H, stream);
    } else {
      e = gemm(dt, false, true, flce::kStoreOut, vec, g4, stream);
    }
    mk.after();
    if (e != hipSuccess) return FLCE_ERR_HIP;

    // 5. grad_W^T (+)= h_c^T . G: A(m = hidden, k = token) = h_c[k][m],
    //    B(n = vocab, k = token) = G[k][n].
    flce::GemmArgs g5{hc, H, g_base, ldg, grad_W, H, static_cast<int>(H), static_cast<int>(V),
                      rows, (r0 == 0 && !accumulate) ? 0 : 1};
    g5.group_m = 4;
    g5.stagger = 37;
    mk.before();
    e = gemm(dt, false, false, flce::kAccumF32, vec, g5, stream);
    mk.after();
    if (e != hipSuccess) return FLCE_ERR_HIP;

    if (ns) {
      // 6. the norm's backward: grad_x rows of the chunk, grad_gamma (+)=.
      const char* xc = static_cast<const char*>(ns->x) + r0 * H * es;
      char* gxc = static_cast<char*>(ns->grad_x) + r0 * H * es;
      if (flce::launch_rmsnorm_bwd(xc, ns->gamma, ns->g_buf, ns->rinv, rows, static_cast<int>(H),
                                   gxc, ns->part, ns->grad_gamma, r0 == 0 ? 1 : 0, bf16,
                                   stream) != hipSuccess)
        return FLCE_ERR_HIP;
    }
  }
  return FLCE_OK;
}

}  // namespace

extern "C" flce_status flce_fwd_bwd(const void* h, const void* W, const int32_t* targets,
                                    int64_t N, int64_t H, int64_t V, int64_t chunk,
                                    float* loss, void* grad_h, float* grad_W,
                                    void* workspace, size_t workspace_bytes, flce_dtype dt,
                                    hipStream_t stream) {
  return fwd_bwd_impl(h, W, targets, N, H, V, chunk, loss, grad_h, grad_W, workspace,
                      workspace_bytes, dt, stream, nullptr, 0, false);
}

extern "C" flce_status flce_fwd_bwd_accumulate(const void* h, const void* W,
                                               const int32_t* targets, int64_t N, int64_t H,
                                               int64_t V, int64_t chunk, float* loss,
                                               void* grad_h, float* grad_W, void* workspace,
                                               size_t workspace_bytes, flce_dtype dt,
                                               hipStream_t stream) {
  return fwd_bwd_impl(h, W, targets, N, H, V, chunk, loss, grad_h, grad_W, workspace,
                      workspace_bytes, dt, stream, nullptr, 0, true);
}

extern "C" flce_status flce_scale_grads(void* grad_h, int64_t n_h, float* grad_W, int64_t n_W,
                                        const float* scale, flce_dtype dt,
                                        hipStream_t stream) {
  if (!scale || n_h < 0 || n_W < 0 || !dtype_ok(dt)) return FLCE_ERR_INVALID_ARG;
  if ((n_h > 0 && !grad_h) || (n_W > 0 && !grad_W)) return FLCE_ERR_INVALID_ARG;
  if ((n_h > 0 && !aligned16(grad_h)) || (n_W > 0 && !aligned16(grad_W)) ||
      (reinterpret_cast<uintptr_t>(scale) & 3u))
    return FLCE_ERR_UNSUPPORTED;
  if (flce::launch_scale(grad_h, n_h, dt == FLCE_BF16, scale, stream) != hipSuccess ||
      flce::launch_scale(grad_W, n_W, false, scale, stream) != hipSuccess)
    return FLCE_ERR_HIP;
  return FLCE_OK;
}

extern "C" flce_status flce_fwd_bwd_timed(const void* h, const void* W,
                                          const int32_t* targets, int64_t N, int64_t H,
                                          int64_t V, int64_t chunk, float* loss, void* grad_h,
                                          float* grad_W, void* workspace,
                                          size_t workspace_bytes, flce_dtype dt,
                                          hipStream_t stream, hipEvent_t* events,
                                          int64_t n_events) {
  if (!events) return FLCE_ERR_INVALID_ARG;
  return fwd_bwd_impl(h, W, targets, N, H, V, chunk, loss, grad_h, grad_W, workspace,
                      workspace_bytes, dt, stream, events, n_events, false);
}

extern "C" flce_status flce_logits(const void* h, const void* W, int64_t rows, int64_t H,
                                   int64_t V, float* z, int64_t ldz, flce_dtype dt,
                                   hipStream_t stream) {
  if (!h || !W || !z) return FLCE_ERR_INVALID_ARG;
  if (!dims_ok(rows) || !dims_ok(H) || !dims_ok(V) || ldz < V || !dtype_ok(dt))
    return FLCE_ERR_INVALID_ARG;
  if (H % 8 != 0) return FLCE_ERR_UNSUPPORTED;
  if (!aligned16(h) || !aligned16(W) || !aligned16(z)) return FLCE_ERR_UNSUPPORTED;
  const bool vec = (ldz % 4) == 0;
  flce::GemmArgs g{W, H, h, H, z, ldz, static_cast<int>(V), static_cast<int>(rows),
                   static_cast<int>(H), 0};
  return gemm(dt, true, true, flce::kStoreF32, vec, g, stream) == hipSuccess ? FLCE_OK
                                                                             : FLCE_ERR_HIP;
}

extern "C" flce_status flce_ce_rows(float* z, int64_t ldz, const int32_t* targets,
                                    int64_t rows, int64_t V, float scale, float* row_loss,
                                    int64_t loss_stride, flce_dtype dt, hipStream_t stream) {
  if (!z || !targets || !row_loss) return FLCE_ERR_INVALID_ARG;
  if (!dims_ok(rows) || !dims_ok(V) || ldz < V || loss_stride < 1 || !dtype_ok(dt))
    return FLCE_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(z) & 3u) || (reinterpret_cast<uintptr_t>(targets) & 3u) ||
      (reinterpret_cast<uintptr_t>(row_loss) & 3u))
    return FLCE_ERR_UNSUPPORTED;
  return flce::launch_ce_rows(z, ldz, targets, static_cast<int>(rows), static_cast<int>(V),
                              scale, row_loss, loss_stride, dt == FLCE_BF16, stream) ==
                 hipSuccess
             ? FLCE_OK
             : FLCE_ERR_HIP;
}

extern "C" flce_status flce_cross_entropy(void* logits, int64_t ld, const int32_t* targets,
                                          int64_t rows, int64_t V, float* loss,
                                          float* row_loss, flce_dtype dt, hipStream_t stream) {
  if (!logits || !targets || !loss || !row_loss) return FLCE_ERR_INVALID_ARG;
  if (!dims_ok(rows) || !dims_ok(V) || ld < V || !dtype_ok(dt)) return FLCE_ERR_INVALID_ARG;
  const uintptr_t es_mask = dt == FLCE_BF16 ? 1u : 3u;
  if ((reinterpret_cast<uintptr_t>(logits) & es_mask) ||
      (reinterpret_cast<uintptr_t>(targets) & 3u) ||
      (reinterpret_cast<uintptr_t>(row_loss) & 3u) || (reinterpret_cast<uintptr_t>(loss) & 3u))
    return FLCE_ERR_UNSUPPORTED;
  const float inv = static_cast<float>(1.0 / static_cast<double>(rows));
  const int r = static_cast<int>(rows);
  hipError_t e =
      dt == FLCE_BF16
          ? flce::launch_ce_rows_bf16(static_cast<uint16_t*>(logits), ld, targets, r,
                                      static_cast<int>(V), inv, row_loss, 1, stream)
          : flce::launch_ce_rows(static_cast<float*>(logits), ld, targets, r,
                                 static_cast<int>(V), inv, row_loss, 1, false, stream);
  if (e != hipSuccess) return FLCE_ERR_HIP;
  return flce::launch_loss_sum(row_loss, 1, r, inv, 1, loss, stream) == hipSuccess
             ? FLCE_OK
             : FLCE_ERR_HIP;
}

// ---------------------------------------------------------------------------
// The head behind an RMSNorm (page 3, "Complete Guide to Liger Kernel",
// section "LigerRMSNorm"): the caller passes the pre-norm hidden states x and
// the norm weight gamma; each token chunk is normalised into the workspace
// just before its logits, and the norm's backward runs right after the
// chunk's gradients, so neither h nor grad_h exists for more than one chunk.
// ---------------------------------------------------------------------------
namespace {

struct NormLayout {
  int64_t h_buf, g_buf, rinv, part, total;
};
inline NormLayout norm_layout(size_t base, int64_t C, int64_t H, int64_t es) {
  NormLayout l;
  l.h_buf = round_up(static_cast<int64_t>(base), 256);
  l.g_buf = round_up(l.h_buf + C * H * es, 256);
  l.rinv = round_up(l.g_buf + C * H * es, 256);
  l.part = round_up(l.rinv + C * 4, 256);
  l.total = l.part + static_cast<int64_t>(flce::rmsnorm_groups(static_cast<int>(C))) * H * 4;
  return l;
}

}  // namespace

extern "C" size_t flce_rmsnorm_workspace_bytes(int64_t N, int64_t H, int64_t V, int64_t chunk,
                                               flce_dtype dt) {
  const size_t base = flce_workspace_bytes(N, H, V, chunk, dt);
  if (base == 0) return 0;
  const int64_t C = chunk < N ? chunk : N;
  return static_cast<size_t>(norm_layout(base, C, H, esize(dt)).total);
}

extern "C" flce_status flce_fwd_bwd_rmsnorm(const void* x, const void* gamma, float eps,
                                            const void* W, const int32_t* targets, int64_t N,
                                            int64_t H, int64_t V, int64_t chunk, float* loss,
                                            void* grad_x, float* grad_gamma, float* grad_W,
                                            void* workspace, size_t workspace_bytes,
                                            flce_dtype dt, hipStream_t stream) {
  if (!x || !gamma || !grad_gamma || !W || !targets || !loss || !grad_x || !grad_W ||
      !workspace)
    return FLCE_ERR_INVALID_ARG;
  if (!dims_ok(N) || !dims_ok(H) || !dims_ok(V) || chunk < 1 || !dtype_ok(dt))
    return FLCE_ERR_INVALID_ARG;
  if (!(eps >= 0.0f) || eps > 3.0e38f) return FLCE_ERR_INVALID_ARG;  // NaN, negative or inf
  if (H % 8 != 0) return FLCE_ERR_UNSUPPORTED;
  if (!aligned16(x) || !aligned16(gamma) || !aligned16(grad_x) || !aligned16(grad_W) ||
      !aligned16(workspace) || (reinterpret_cast<uintptr_t>(grad_gamma) & 3u))
    return FLCE_ERR_UNSUPPORTED;
  const size_t need = flce_rmsnorm_workspace_bytes(N, H, V, chunk, dt);
  if (need == 0) return FLCE_ERR_UNSUPPORTED;
  if (workspace_bytes < need) return FLCE_ERR_WORKSPACE;
  const int64_t C = chunk < N ? chunk : N;
  const NormLayout lay = norm_layout(flce_workspace_bytes(N, H, V, chunk, dt), C, H, esize(dt));
  char* ws = static_cast<char*>(workspace);
  const NormSide ns{x,
                    gamma,
                    eps,
                    grad_x,
                    grad_gamma,
                    ws + lay.h_buf,
                    ws + lay.g_buf,
                    reinterpret_cast<float*>(ws + lay.rinv),
                    reinterpret_cast<float*>(ws + lay.part)};
  return fwd_bwd_impl(x, W, targets, N, H, V, chunk, loss, grad_x, grad_W, workspace,
                      workspace_bytes, dt, stream, nullptr, 0, false, &ns);
}

// ---------------------------------------------------------------------------
// Vocabulary-chunked variant (page 1, "Liger Kernel explained", section
// "What does Liger Kernel actually fuse, and why does that cut memory?":
// the logits are worked through in chunks over the vocabulary dimension).
// All N tokens at once, the vocabulary in column chunks of Vc:
//   pass 1  per chunk: exponentiated bf16 logits and their (max, sum) pairs
//           (the values are not kept); then per row lse2 over all V columns,
//           log2 of the target logit, the row loss; the mean loss
//   pass 2  per chunk: the logits again, G over the chunk's columns with the
//           global lse, grad_h (+)= G W_c into an fp32 [N, H] accumulator,
//           grad_W[chunk rows] = G^T h
//   finally grad_h = bf16(accumulator).
// The logits are computed twice: 8 N V H flops instead of 6 N V H, for a
// workspace of N Vc (not C V) bf16 logits.
// ---------------------------------------------------------------------------
namespace {

struct VocabLayout {
  int64_t pairs, stats, acc, total;
};
inline VocabLayout vocab_layout(int64_t N, int64_t H, int64_t V, int64_t Vc) {
  VocabLayout l;
  l.pairs = round_up(N * Vc * 2, 256);                         // u [N][Vc] bf16
  l.stats = round_up(l.pairs + N * n_half_tiles(V) * 8, 256);  // pairs [N][2 ceil(V/128)]
  l.acc = round_up(l.stats + 4 * N * 4, 256);                  // lse2, pt1, loss, rt [N]
  l.total = l.acc + N * H * 4;                                 // grad_h accumulator fp32
  return l;
}

// Shapes the vocabulary-chunked path runs: bf16, K = H and every chunk's
// K = Vc a multiple of 64 on the direct-to-LDS kernel, chunks starting on
// 128-column half tiles.
inline bool vocab_path_ok(int64_t H, int64_t V, int64_t vchunk, flce_dtype dt) {
  return dt == FLCE_BF16 && H % 64 == 0 && H < (int64_t{1} << 22) && V % 64 == 0 &&
         V < (int64_t{1} << 22) && (vchunk >= V || vchunk % flce::kHalfTile == 0);
}

}  // namespace

extern "C" size_t flce_vocab_workspace_bytes(int64_t N, int64_t H, int64_t V, int64_t vchunk,
                                             flce_dtype dt) {
  if (!dims_ok(N) || !dims_ok(H) || !dims_ok(V) || vchunk < 1 || !dtype_ok(dt)) return 0;
  if (!vocab_path_ok(H, V, vchunk, dt)) return 0;
  const int64_t Vc = vchunk < V ? vchunk : V;
  if (!area_ok(N, Vc) || !area_ok(N, H) || !area_ok(N, V)) return 0;
  return static_cast<size_t>(vocab_layout(N, H, V, Vc).total);
}

extern "C" flce_status flce_fwd_bwd_vocab(const void* h, const void* W, const int32_t* targets,
                                          int64_t N, int64_t H, int64_t V, int64_t vchunk,
                                          float* loss, void* grad_h, float* grad_W,
                                          void* workspace, size_t workspace_bytes,
                                          flce_dtype dt, hipStream_t stream) {
  if (!h || !W || !targets || !loss || !grad_h || !grad_W || !workspace)
    return FLCE_ERR_INVALID_ARG;
  if (!dims_ok(N) || !dims_ok(H) || !dims_ok(V) || vchunk < 1 || !dtype_ok(dt))
    return FLCE_ERR_INVALID_ARG;
  if (!aligned16(h) || !aligned16(W) || !aligned16(grad_h) || !aligned16(grad_W) ||
      !aligned16(workspace) || (reinterpret_cast<uintptr_t>(targets) & 3u) ||
      (reinterpret_cast<uintptr_t>(loss) & 3u))
    return FLCE_ERR_UNSUPPORTED;
  if (!vocab_path_ok(H, V, vchunk, dt)) return FLCE_ERR_UNSUPPORTED;
  const size_t need = flce_vocab_workspace_bytes(N, H, V, vchunk, dt);
  if (need == 0) return FLCE_ERR_UNSUPPORTED;
  if (workspace_bytes < need) return FLCE_ERR_WORKSPACE;

  const int64_t Vc = vchunk < V ? vchunk : V;
  const VocabLayout lay = vocab_layout(N, H, V, Vc);
  char* ws = static_cast<char*>(workspace);
  uint16_t* u = reinterpret_cast<uint16_t*>(ws);
  float* pairs = reinterpret_cast<float*>(ws + lay.pairs);
  float* lse2 = reinterpret_cast<float*>(ws + lay.stats);
  float* pt1 = lse2 + N;
  float* row_loss = pt1 + N;
  float* rt = row_loss + N;
  float* gacc = reinterpret_cast<float*>(ws + lay.acc);
  const int64_t ldp = 2 * n_half_tiles(V);
  const int rows = static_cast<int>(N);
  const float inv_n = static_cast<float>(1.0 / static_cast<double>(N));
  const uint16_t* h16 = static_cast<const uint16_t*>(h);
  const uint16_t* W16 = static_cast<const uint16_t*>(W);

  // Exponentiated logits of columns [v0, v0 + n) for all tokens.
  auto logits = [&](int64_t v0, int64_t n) {
    flce::GemmArgs g{W16 + v0 * H, H, h, H, u, Vc, static_cast<int>(n), rows,
                     static_cast<int>(H), 0};
    g.group_m = 4;
    g.stagger = 37;
    g.row_part = pairs + 2 * (v0 / flce::kHalfTile);
    g.ldp = ldp;
    return flce::launch_gemm_bf16(true, true, flce::kExpBF16, true, g, stream);
  };

  // Pass 1: statistics (the target's half-tile mass taken from the chunk
  // that holds the target, while its u values are in the workspace).
  for (int64_t v0 = 0; v0 < V; v0 += Vc) {
    const int64_t n = (V - v0) < Vc ? (V - v0) : Vc;
    if (logits(v0, n) != hipSuccess ||
        flce::launch_ce_target_mass(u, Vc, targets, rows, static_cast<int>(v0),
                                    static_cast<int>(n), rt, stream) != hipSuccess)
      return FLCE_ERR_HIP;
  }
  if (flce::launch_ce_stats_exp(pairs, ldp, rt, h16, W16, static_cast<int>(H), targets, rows,
                                static_cast<int>(V), lse2, pt1, row_loss, stream) != hipSuccess ||
      flce::launch_loss_sum(row_loss, 1, rows, inv_n, 1, loss, stream) != hipSuccess)
    return FLCE_ERR_HIP;

  // Pass 2: gradients, chunk by chunk.
  for (int64_t v0 = 0; v0 < V; v0 += Vc) {
    const int64_t n = (V - v0) < Vc ? (V - v0) : Vc;
    if (logits(v0, n) != hipSuccess) return FLCE_ERR_HIP;
    if (flce::launch_ce_rewrite_exp(u, Vc, pairs + 2 * (v0 / flce::kHalfTile), ldp, lse2, pt1,
                                    targets, rows, static_cast<int>(v0), static_cast<int>(n),
                                    inv_n, nullptr, stream) != hipSuccess)
      return FLCE_ERR_HIP;
    // grad_h^T (+)= W_c^T . G^T: A(m = hidden, k = vocab) = W[v0 + k][m],
    // B(n = token, k = vocab) = G[n][k]; fp32, accumulated after chunk 0.
    flce::GemmArgs g4{W16 + v0 * H, H, u, Vc, gacc, H, static_cast<int>(H), rows,
                      static_cast<int>(n), v0 > 0 ? 1 : 0};
    g4.group_m = 4;
    if (flce::launch_gemm_bf16(false, true, flce::kAccumF32, true, g4, stream) != hipSuccess)
      return FLCE_ERR_HIP;
    // grad_W[v0 + n][m] = sum over tokens k of G[k][n] h[k][m]:
    // A(m = hidden, k = token) = h[k][m], B(n = vocab, k = token) = G[k][n].
    flce::GemmArgs g5{h, H, u, Vc, grad_W + v0 * H, H, static_cast<int>(H), static_cast<int>(n),
                      rows, 0};
    g5.group_m = 4;
    g5.stagger = 37;
    if (flce::launch_gemm_bf16(false, false, flce::kAccumF32, true, g5, stream) != hipSuccess)
      return FLCE_ERR_HIP;
  }
  return flce::launch_sum_parts_bf16(gacc, 1, N * H, static_cast<uint16_t*>(grad_h), N * H,
                                     stream) == hipSuccess
             ? FLCE_OK
             : FLCE_ERR_HIP;
}

// ---------------------------------------------------------------------------
// Odds-ratio preference loss over the same head (page 2, "Liger-Kernel:
// Triton kernels that replace Hugging Face training ops", section
// "Installation and the one-line patch": ORPO is one of the chunked
// post-training losses called with the LM-head weight, the hidden states
// and the targets; the objective is the published one, see orpo.hip).
// Rows: 2B sequences of T tokens, sequences [0, B) chosen, [B, 2B) rejected.  The batch is worked
// through in chunks of Pc pairs; a chunk's chosen and rejected rows are
// copied next to each other into the workspace, so every pair's two
// sequences are in one chunk and the head's kernels run unchanged:
//   0. count of counted chosen rows (once)
//   1. h_c, t_c  <- the chunk's chosen rows, then its rejected rows
//   2. exponentiated logits and (max, sum) pairs of h_c           MFMA
//   3. per row lse2 and log2 of the target logit
//   4. per pair: mean log-probabilities, log odds, the loss terms; per row
//      the gradient scale c = -dloss/dlog p
//   5. u -> G = c (softmax - onehot) in place
//   6. grad_h_c = G W, copied back to the chunk's rows of grad_h     MFMA
//   7. grad_W (+)= G^T h_c                                           MFMA
// and finally the loss from the staged per-pair terms.
// ---------------------------------------------------------------------------
namespace {

struct OrpoLayout {
  int64_t pairs, parts, stats, hc, ghc, tc, stage, count, total;
};
// The preference loss sizes its K-split parts without a cap (its workspace
// also stages the chunk's hidden rows and gradients).
constexpr int64_t kOrpoSplitRoom = int64_t{1} << 62;
inline OrpoLayout orpo_layout(int64_t B, int64_t T, int64_t Pc, int64_t H, int64_t V) {
  const int64_t R = 2 * Pc * T;        // rows of a full chunk
  const int64_t Rl = 2 * (B % Pc) * T; // rows of a shorter last chunk (0: none)
  int64_t split_rows = 0;
  for (int64_t r : {R, Rl}) {
    if (r <= 0) continue;
    const int sp = grad_h_splits(H, r, V, kOrpoSplitRoom);
    if (sp > 1 && sp * r > split_rows) split_rows = sp * r;
  }
  OrpoLayout l;
  l.pairs = round_up(R * V * 2, 256);                             // u [R][V] bf16
  l.parts = round_up(l.pairs + R * n_half_tiles(V) * 8, 256);     // (max, sum) pairs
  l.stats = round_up(l.parts + split_rows * H * 4, 256);          // grad_h K-split parts
  l.hc = round_up(l.stats + 5 * R * 4, 256);                      // lse2, pt1, loss, coef, rt
  l.ghc = round_up(l.hc + R * H * 2, 256);                        // h_c [R][H] bf16
  l.tc = round_up(l.ghc + R * H * 2, 256);                        // grad_h_c [R][H] bf16
  l.stage = round_up(l.tc + R * 4, 256);                          // t_c [R]
  l.count = round_up(l.stage + 2 * B * 4, 256);                   // per-pair terms [B][2]
  l.total = l.count + 256;                                        // counted chosen rows
  return l;
}

// Sizes the preference loss runs: bf16 on the exponentiated-logits path,
// int-sized row counts.
inline bool orpo_args_ok(int64_t B, int64_t T, int64_t H, int64_t V, int64_t Pc,
                         flce_dtype dt) {
  if (B < 1 || T < 1 || Pc < 1 || !dims_ok(H) || !dims_ok(V) || !dtype_ok(dt)) return false;
  if (B > kMaxDim / 2 || T > kMaxDim / (2 * B)) return false;  // 2 B T rows fit an int
  const int64_t R = 2 * (Pc < B ? Pc : B) * T;                 // rows of a chunk
  return area_ok(R, V) && area_ok(R, H);
}

}  // namespace

extern "C" size_t flce_orpo_workspace_bytes(int64_t pairs, int64_t seq_len, int64_t H,
                                            int64_t V, int64_t chunk_pairs, flce_dtype dt) {
  if (!orpo_args_ok(pairs, seq_len, H, V, chunk_pairs, dt) || !exp_path(H, V, dt)) return 0;
  const int64_t Pc = chunk_pairs < pairs ? chunk_pairs : pairs;
  return static_cast<size_t>(orpo_layout(pairs, seq_len, Pc, H, V).total);
}

extern "C" flce_status flce_orpo_fwd_bwd(const void* h, const void* W, const int32_t* targets,
                                         int64_t pairs, int64_t seq_len, int64_t H, int64_t V,
                                         int64_t chunk_pairs, float beta, float* loss,
                                         float* seq_logp, void* grad_h, float* grad_W,
                                         void* workspace, size_t workspace_bytes,
                                         flce_dtype dt, hipStream_t stream) {
  if (!h || !W || !targets || !loss || !grad_h || !grad_W || !workspace)
    return FLCE_ERR_INVALID_ARG;
  if (!orpo_args_ok(pairs, seq_len, H, V, chunk_pairs, dt)) return FLCE_ERR_INVALID_ARG;
  if (!(beta == beta) || beta > 3.0e38f || beta < -3.0e38f) return FLCE_ERR_INVALID_ARG;
  if (!aligned16(h) || !aligned16(W) || !aligned16(grad_h) || !aligned16(grad_W) ||
      !aligned16(workspace) || (reinterpret_cast<uintptr_t>(targets) & 3u) ||
      (reinterpret_cast<uintptr_t>(loss) & 3u) || (reinterpret_cast<uintptr_t>(seq_logp) & 3u))
    return FLCE_ERR_UNSUPPORTED;
  if (!exp_path(H, V, dt)) return FLCE_ERR_UNSUPPORTED;
  if (workspace_bytes < flce_orpo_workspace_bytes(pairs, seq_len, H, V, chunk_pairs, dt))
    return FLCE_ERR_WORKSPACE;

  const int64_t B = pairs, T = seq_len;
  const int64_t Pc = chunk_pairs < B ? chunk_pairs : B;
  const OrpoLayout lay = orpo_layout(B, T, Pc, H, V);
  char* ws = static_cast<char*>(workspace);
  uint16_t* u = reinterpret_cast<uint16_t*>(ws);
  float* rpairs = reinterpret_cast<float*>(ws + lay.pairs);
  float* parts = reinterpret_cast<float*>(ws + lay.parts);
  const int64_t R = 2 * Pc * T;
  float* lse2 = reinterpret_cast<float*>(ws + lay.stats);
  float* pt1 = lse2 + R;
  float* row_loss = pt1 + R;
  float* coef = row_loss + R;
  float* rt = coef + R;
  uint16_t* hc = reinterpret_cast<uint16_t*>(ws + lay.hc);
  uint16_t* ghc = reinterpret_cast<uint16_t*>(ws + lay.ghc);
  int32_t* tc = reinterpret_cast<int32_t*>(ws + lay.tc);
  float* stage = reinterpret_cast<float*>(ws + lay.stage);
  int* count = reinterpret_cast<int*>(ws + lay.count);
  const int64_t ldp = 2 * n_half_tiles(V);
  const uint16_t* h16 = static_cast<const uint16_t*>(h);
  const uint16_t* W16 = static_cast<const uint16_t*>(W);
  uint16_t* gh16 = static_cast<uint16_t*>(grad_h);
  const hipMemcpyKind d2d = hipMemcpyDeviceToDevice;

  // 0. counted chosen rows over the whole batch (the SFT term's mean).
  if (flce::launch_orpo_count(targets, B * T, count, stream) != hipSuccess) return FLCE_ERR_HIP;

  for (int64_t p0 = 0; p0 < B; p0 += Pc) {
    const int64_t pc = (B - p0) < Pc ? (B - p0) : Pc;
    const int64_t half = pc * T;  // chosen rows of the chunk (as many rejected)
    const int rows = static_cast<int>(2 * half);
    const int64_t cw = p0 * T, cr = (B + p0) * T;  // first chosen / rejected row in the batch

    // 1. stage the chunk's rows contiguously.
    if (hipMemcpyAsync(hc, h16 + cw * H, half * H * 2, d2d, stream) != hipSuccess ||
        hipMemcpyAsync(hc + half * H, h16 + cr * H, half * H * 2, d2d, stream) != hipSuccess ||
        hipMemcpyAsync(tc, targets + cw, half * 4, d2d, stream) != hipSuccess ||
        hipMemcpyAsync(tc + half, targets + cr, half * 4, d2d, stream) != hipSuccess)
      return FLCE_ERR_HIP;

    // 2. exponentiated logits of h_c and their (max, sum) pairs.
    flce::GemmArgs g1{W, H, hc, H, u, V, static_cast<int>(V), rows, static_cast<int>(H), 0};
    g1.group_m = 4;
    g1.stagger = 37;
    g1.row_part = rpairs;
    g1.ldp = ldp;
    if (flce::launch_gemm_bf16(true, true, flce::kExpBF16, true, g1, stream) != hipSuccess)
      return FLCE_ERR_HIP;

    // 3.-5. row statistics, per-pair terms and row scales, G in place.
    if (flce::launch_ce_target_mass(u, V, tc, rows, 0, static_cast<int>(V), rt, stream) !=
            hipSuccess ||
        flce::launch_ce_stats_exp(rpairs, ldp, rt, hc, W16, static_cast<int>(H), tc, rows,
                                  static_cast<int>(V), lse2, pt1, row_loss, stream) !=
            hipSuccess ||
        flce::launch_orpo_coef(row_loss, tc, static_cast<int>(pc), static_cast<int>(T),
                               static_cast<int>(B), static_cast<int>(p0), beta, count, coef,
                               seq_logp, stage, stream) != hipSuccess ||
        flce::launch_ce_rewrite_exp(u, V, rpairs, ldp, lse2, pt1, tc, rows, 0,
                                    static_cast<int>(V), 1.0f, coef, stream) != hipSuccess)
      return FLCE_ERR_HIP;

    // 6. grad_h_c^T = W^T . G^T (K split for few output tiles), then back
    //    to the chunk's rows of grad_h.
    flce::GemmArgs g4{W, H, u, V, ghc, H, static_cast<int>(H), rows, static_cast<int>(V), 0};
    g4.group_m = 4;
    const int splits = grad_h_splits(H, rows, V, kOrpoSplitRoom);
    hipError_t e;
    if (splits > 1) {
      g4.out = parts;
      g4.splits = splits;
      g4.split_stride = static_cast<int64_t>(rows) * H;
      e = flce::launch_gemm_bf16(false, true, flce::kStoreF32, true, g4, stream);
      if (e == hipSuccess)
        e = flce::launch_sum_parts_bf16(parts, splits, static_cast<int64_t>(rows) * H, ghc,
                                        static_cast<int64_t>(rows) * H, stream);
    } else {
      e = flce::launch_gemm_bf16(false, true, flce::kStoreOut, true, g4, stream);
    }
    if (e != hipSuccess ||
        hipMemcpyAsync(gh16 + cw * H, ghc, half * H * 2, d2d, stream) != hipSuccess ||
        hipMemcpyAsync(gh16 + cr * H, ghc + half * H, half * H * 2, d2d, stream) != hipSuccess)
      return FLCE_ERR_HIP;

    // 7. grad_W^T (+)= h_c^T . G.
    flce::GemmArgs g5{hc, H, u, V, grad_W, H, static_cast<int>(H), static_cast<int>(V), rows,
                      p0 == 0 ? 0 : 1};
    g5.group_m = 4;
    g5.stagger = 37;
    if (flce::launch_gemm_bf16(false, false, flce::kAccumF32, true, g5, stream) != hipSuccess)
      return FLCE_ERR_HIP;
  }
  return flce::launch_orpo_loss(stage, static_cast<int>(B), beta, count, loss, stream) ==
                 hipSuccess
             ? FLCE_OK
             : FLCE_ERR_HIP;
}

extern "C" flce_status flce_mfma_rate(const void* operands, int64_t operand_bytes,
                                     int64_t iters, int64_t workgroups, float* sink,
                                     uint64_t* clocks, hipStream_t stream) {
  if (!operands || !sink || !clocks) return FLCE_ERR_INVALID_ARG;
  if (operand_bytes < 8192 || operand_bytes % 16 != 0 || iters < 1 ||
      iters > (int64_t{1} << 40) || workgroups < 1 || workgroups > 65535)
    return FLCE_ERR_INVALID_ARG;
  if (!aligned16(operands) || (reinterpret_cast<uintptr_t>(sink) & 3u) ||
      (reinterpret_cast<uintptr_t>(clocks) & 7u))
    return FLCE_ERR_UNSUPPORTED;
  const int64_t groups = operand_bytes / 128;
  return flce::launch_mfma_rate(operands,
                                static_cast<int>(groups < (int64_t{1} << 30) ? groups
                                                                             : int64_t{1} << 30),
                                iters,
                                static_cast<int>(workgroups), sink, clocks,
                                stream) == hipSuccess
             ? FLCE_OK
             : FLCE_ERR_HIP;
}

// ---------------------------------------------------------------------------
// Allocation-free entry point: flce_fwd_bwd over a static device array
// instead of a caller-provided workspace, for callers that cannot allocate.
// This translation unit defines no kernel, so the array's code object is
// loaded on a device only when its address is first looked up there.
// ---------------------------------------------------------------------------
namespace {

static __device__ __align__(256) char scratch[FLCE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch` per device

// Device address of `scratch` on the device that `stream` belongs to (the
// current device for the null stream), looked up once per device with that
// device current and restored afterwards.  In host code the array's name is a
// host-side stand-in: only this address may reach a kernel or a copy.
hipError_t scratch_for_stream(hipStream_t stream, void** out) {
  int cur = -1;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return e;
  int dev = cur;
  if (stream) {
    hipDevice_t sd = -1;
    e = hipStreamGetDevice(stream, &sd);
    if (e != hipSuccess) return e;
    dev = static_cast<int>(sd);
  }
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (dev != cur) {
      const hipError_t r = hipSetDevice(cur);
      if (e == hipSuccess) e = r;
    }
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" flce_status flce_fwd_bwd_noalloc(const void* h, const void* W,
                                            const int32_t* targets, int64_t N, int64_t H,
                                            int64_t V, int64_t chunk, float* loss,
                                            void* grad_h, float* grad_W, flce_dtype dt,
                                            hipStream_t stream) {
  // Sizes the workspace functions reject (0) are reported by the full
  // argument checks below; sizes beyond the array are refused here.
  if (flce_workspace_bytes(N, H, V, chunk, dt) > FLCE_NOALLOC_SCRATCH_BYTES)
    return FLCE_ERR_SCRATCH;
  void* ws = nullptr;
  if (scratch_for_stream(stream, &ws) != hipSuccess) return FLCE_ERR_HIP;
  return fwd_bwd_impl(h, W, targets, N, H, V, chunk, loss, grad_h, grad_W, ws,
                      FLCE_NOALLOC_SCRATCH_BYTES, dt, stream, nullptr, 0, false);
}

extern "C" const char* flce_status_string(flce_status s) {
  switch (s) {
    case FLCE_OK: return "FLCE_OK";
    case FLCE_ERR_INVALID_ARG: return "FLCE_ERR_INVALID_ARG: null pointer, bad size or dtype";
    case FLCE_ERR_WORKSPACE: return "FLCE_ERR_WORKSPACE: workspace smaller than required";
    case FLCE_ERR_UNSUPPORTED:
      return "FLCE_ERR_UNSUPPORTED: H % 8 != 0, a pointer not 16-byte aligned, or a shape "
             "this entry point does not run";
    case FLCE_ERR_HIP: return "FLCE_ERR_HIP: the HIP runtime reported a launch error";
    case FLCE_ERR_SCRATCH:
      return "FLCE_ERR_SCRATCH: these sizes need more workspace than the allocation-free "
             "entry point's static scratch (FLCE_NOALLOC_SCRATCH_BYTES); use a smaller chunk";
  }
  return "unknown flce_status";
}
