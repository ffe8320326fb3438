// Stub HIP runtime and kernel launchers for the CPU sanitizer build of the
// library's host layer.  TEST INFRASTRUCTURE: linked with flce_api.hip (built
// by g++ with AddressSanitizer and UndefinedBehaviorSanitizer) in place of the
// HIP runtime and the kernels.  No launcher computes anything: each checks
// that every byte range the real kernel would read or write lies inside one
// buffer the test registered (the caller's inputs, outputs and workspace),
// and counts a violation otherwise.  Pointers are never dereferenced, so the
// test can pass arbitrary, never-allocated addresses.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <vector>

#include "flce.h"
#include "flce_internal.h"

namespace {

struct Range {
  uintptr_t base;
  size_t bytes;
};

std::mutex g_mu;
std::vector<Range> g_buffers;
Range g_symbol{0, 0};  // the device symbol looked up once per process, kept across resets
int64_t g_launches = 0;
int64_t g_violations = 0;
char g_last[256] = "";

// [p, p + bytes) must lie inside one registered buffer.
void need(const void* p, int64_t bytes, const char* what) {
  if (bytes <= 0) return;
  const uintptr_t a = reinterpret_cast<uintptr_t>(p);
  if (a >= g_symbol.base && a - g_symbol.base <= g_symbol.bytes &&
      static_cast<uint64_t>(bytes) <= g_symbol.bytes - (a - g_symbol.base))
    return;
  for (const Range& r : g_buffers)
    if (a >= r.base && a - r.base <= r.bytes &&
        static_cast<uint64_t>(bytes) <= r.bytes - (a - r.base))
      return;
  ++g_violations;
  snprintf(g_last, sizeof g_last, "%s: [%#llx, +%lld) outside every buffer", what,
           static_cast<unsigned long long>(a), static_cast<long long>(bytes));
}

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Extents of D[m][n] = sum_k A(m, k) B(n, k), out[n * ldo + m] (flce_internal.h).
void check_gemm(bool a_kc, bool b_kc, int epi, const flce::GemmArgs& g, int64_t es,
                const char* what) {
  ++g_launches;
  if (g.M <= 0 || g.N <= 0) return;
  if (g.K <= 0) {
    ++g_violations;
    snprintf(g_last, sizeof g_last, "%s: K = %d", what, g.K);
    return;
  }
  const int64_t M = g.M, N = g.N, K = g.K;
  need(g.A, (a_kc ? (M - 1) * g.lda + K : (K - 1) * g.lda + M) * es, "gemm A");
  need(g.B, (b_kc ? (N - 1) * g.ldb + K : (K - 1) * g.ldb + N) * es, "gemm B");
  const int64_t oes = (epi == flce::kStoreF32 || epi == flce::kAccumF32) ? 4
                      : epi == flce::kExpBF16                            ? 2
                                                                         : es;
  const int64_t parts = g.splits > 1 ? g.splits : 1;
  need(g.out, ((parts - 1) * g.split_stride + (N - 1) * g.ldo + M) * oes, "gemm out");
  if (epi == flce::kExpBF16)
    need(g.row_part, ((N - 1) * g.ldp + 2 * cdiv(M, flce::kHalfTile)) * 4, "gemm pairs");
}

}  // namespace

extern "C" {

// Test hooks (exported by this stub library only).
void flce_stub_reset(void) {
  std::lock_guard<std::mutex> l(g_mu);
  g_buffers.clear();
  g_launches = 0;
  g_violations = 0;
  g_last[0] = 0;
}
void flce_stub_add_buffer(uint64_t base, uint64_t bytes) {
  std::lock_guard<std::mutex> l(g_mu);
  g_buffers.push_back(Range{static_cast<uintptr_t>(base), static_cast<size_t>(bytes)});
}
int64_t flce_stub_launches(void) { return g_launches; }
int64_t flce_stub_violations(void) { return g_violations; }
const char* flce_stub_last_violation(void) { return g_last; }

hipError_t hipEventRecord(hipEvent_t, hipStream_t) { return hipSuccess; }
hipError_t hipMemcpyAsync(void* dst, const void* src, size_t bytes, hipMemcpyKind, hipStream_t) {
  ++g_launches;
  need(dst, static_cast<int64_t>(bytes), "memcpy dst");
  need(src, static_cast<int64_t>(bytes), "memcpy src");
  return hipSuccess;
}
hipError_t hipGetDevice(int* device) {
  *device = 0;
  return hipSuccess;
}
hipError_t hipSetDevice(int device) { return device == 0 ? hipSuccess : hipErrorInvalidDevice; }
hipError_t hipStreamGetDevice(hipStream_t, hipDevice_t* device) {
  *device = 0;
  return hipSuccess;
}
// The host stand-in of a device symbol is its own address; the scratch the
// allocation-free entry point asks for counts as a buffer from then on (the
// library looks it up once per device, so it survives flce_stub_reset).
hipError_t hipGetSymbolAddress(void** dev_ptr, const void* symbol) {
  *dev_ptr = const_cast<void*>(symbol);
  std::lock_guard<std::mutex> l(g_mu);
  g_symbol = Range{reinterpret_cast<uintptr_t>(symbol), FLCE_NOALLOC_SCRATCH_BYTES};
  return hipSuccess;
}

}  // extern "C"

namespace flce {

hipError_t launch_gemm_bf16(bool a_kc, bool b_kc, int epi, bool, const GemmArgs& g,
                            hipStream_t) {
  check_gemm(a_kc, b_kc, epi, g, 2, "gemm_bf16");
  return hipSuccess;
}
hipError_t launch_gemm_bf16_dma(bool a_kc, bool b_kc, int epi, const GemmArgs& g, hipStream_t) {
  check_gemm(a_kc, b_kc, epi, g, 2, "gemm_bf16_dma");
  return hipSuccess;
}
hipError_t launch_gemm_f32(bool a_kc, bool b_kc, int epi, const GemmArgs& g, hipStream_t) {
  check_gemm(a_kc, b_kc, epi, g, 4, "gemm_f32");
  return hipSuccess;
}

hipError_t launch_ce_rows(float* z, int64_t ldz, const int32_t* targets, int rows, int V, float,
                          float* row_loss, int64_t loss_stride, bool, hipStream_t) {
  ++g_launches;
  need(z, ((rows - 1) * ldz + V) * 4, "ce_rows z");
  need(targets, rows * int64_t{4}, "ce_rows targets");
  need(row_loss, ((rows - 1) * loss_stride + 1) * 4, "ce_rows loss");
  return hipSuccess;
}
hipError_t launch_ce_rows_bf16(uint16_t* z, int64_t ldz, const int32_t* targets, int rows, int V,
                               float, float* row_loss, int64_t loss_stride, hipStream_t) {
  ++g_launches;
  need(z, ((rows - 1) * ldz + V) * 2, "ce_rows_bf16 z");
  need(targets, rows * int64_t{4}, "ce_rows_bf16 targets");
  need(row_loss, ((rows - 1) * loss_stride + 1) * 4, "ce_rows_bf16 loss");
  return hipSuccess;
}
hipError_t launch_ce_rows_exp(uint16_t* u, int64_t ldu, const float* row_part, int64_t ldp,
                              const uint16_t* h, const uint16_t* W, int H,
                              const int32_t* targets, int rows, int V, float, float* row_loss,
                              int64_t loss_stride, hipStream_t) {
  ++g_launches;
  need(u, ((rows - 1) * ldu + V) * 2, "ce_rows_exp u");
  need(row_part, ((rows - 1) * ldp + 2 * cdiv(V, kHalfTile)) * 4, "ce_rows_exp pairs");
  need(h, int64_t{rows} * H * 2, "ce_rows_exp h");
  need(W, int64_t{V} * H * 2, "ce_rows_exp W");
  need(targets, rows * int64_t{4}, "ce_rows_exp targets");
  need(row_loss, ((rows - 1) * loss_stride + 3) * 4, "ce_rows_exp loss, lse2, pt1");
  return hipSuccess;
}
hipError_t launch_ce_target_mass(const uint16_t* u, int64_t ldu, const int32_t* targets, int rows,
                                 int, int n, float* rt, hipStream_t) {
  ++g_launches;
  need(u, ((rows - 1) * ldu + n) * 2, "ce_target_mass u");
  need(targets, rows * int64_t{4}, "ce_target_mass targets");
  need(rt, rows * int64_t{4}, "ce_target_mass rt");
  return hipSuccess;
}
hipError_t launch_ce_stats_exp(const float* row_part, int64_t ldp, const float* rt,
                               const uint16_t* h, const uint16_t* W, int H,
                               const int32_t* targets, int rows, int V, float* lse2, float* pt1,
                               float* row_loss, hipStream_t) {
  ++g_launches;
  need(row_part, ((rows - 1) * ldp + 2 * cdiv(V, kHalfTile)) * 4, "ce_stats_exp pairs");
  for (const void* p : {static_cast<const void*>(rt), static_cast<const void*>(targets),
                        static_cast<const void*>(lse2), static_cast<const void*>(pt1),
                        static_cast<const void*>(row_loss)})
    need(p, rows * int64_t{4}, "ce_stats_exp per-row array");
  need(h, int64_t{rows} * H * 2, "ce_stats_exp h");
  need(W, int64_t{V} * H * 2, "ce_stats_exp W");
  return hipSuccess;
}
hipError_t launch_ce_rewrite_exp(uint16_t* u, int64_t ldu, const float* row_part, int64_t ldp,
                                 const float* lse2, const float* pt1, const int32_t* targets,
                                 int rows, int, int n, float, const float* row_scale,
                                 hipStream_t) {
  ++g_launches;
  need(u, ((rows - 1) * ldu + n) * 2, "ce_rewrite_exp u");
  need(row_part, ((rows - 1) * ldp + 2 * cdiv(n, kHalfTile)) * 4, "ce_rewrite_exp pairs");
  need(lse2, rows * int64_t{4}, "ce_rewrite_exp lse2");
  need(pt1, rows * int64_t{4}, "ce_rewrite_exp pt1");
  need(targets, rows * int64_t{4}, "ce_rewrite_exp targets");
  if (row_scale) need(row_scale, rows * int64_t{4}, "ce_rewrite_exp row_scale");
  return hipSuccess;
}

hipError_t launch_orpo_count(const int32_t* targets, int64_t n, int* count, hipStream_t) {
  ++g_launches;
  need(targets, n * 4, "orpo_count targets");
  need(count, 4, "orpo_count count");
  return hipSuccess;
}
hipError_t launch_orpo_coef(const float* row_loss, const int32_t* targets, int Pc, int T, int B,
                            int p0, float, const int* count, float* coef, float* seq_logp,
                            float* stage, hipStream_t) {
  ++g_launches;
  const int64_t R = 2 * int64_t{Pc} * T;
  need(row_loss, R * 4, "orpo_coef row_loss");
  need(targets, R * 4, "orpo_coef targets");
  need(coef, R * 4, "orpo_coef coef");
  need(count, 4, "orpo_coef count");
  if (seq_logp) need(seq_logp, 2 * int64_t{B} * 4, "orpo_coef seq_logp");
  need(stage + 2 * int64_t{p0}, 2 * int64_t{Pc} * 4, "orpo_coef stage");
  return hipSuccess;
}
hipError_t launch_orpo_loss(const float* stage, int B, float, const int* count, float* loss,
                            hipStream_t) {
  ++g_launches;
  need(stage, 2 * int64_t{B} * 4, "orpo_loss stage");
  need(count, 4, "orpo_loss count");
  need(loss, 4, "orpo_loss loss");
  return hipSuccess;
}

// The same grouping as rmsnorm.hip: partial sums over 64-row groups.
int rmsnorm_groups(int rows) { return (rows + 63) / 64; }
hipError_t launch_rmsnorm_fwd(const void* x, const void* gamma, float, int rows, int H, void* h,
                              float* rinv, bool bf16, hipStream_t) {
  ++g_launches;
  const int64_t es = bf16 ? 2 : 4;
  need(x, int64_t{rows} * H * es, "rmsnorm_fwd x");
  need(gamma, H * es, "rmsnorm_fwd gamma");
  need(h, int64_t{rows} * H * es, "rmsnorm_fwd h");
  need(rinv, rows * int64_t{4}, "rmsnorm_fwd rinv");
  return hipSuccess;
}
hipError_t launch_rmsnorm_bwd(const void* x, const void* gamma, const void* g, const float* rinv,
                              int rows, int H, void* grad_x, float* part, float* grad_gamma, int,
                              bool bf16, hipStream_t) {
  ++g_launches;
  const int64_t es = bf16 ? 2 : 4;
  need(x, int64_t{rows} * H * es, "rmsnorm_bwd x");
  need(g, int64_t{rows} * H * es, "rmsnorm_bwd g");
  need(grad_x, int64_t{rows} * H * es, "rmsnorm_bwd grad_x");
  need(gamma, H * es, "rmsnorm_bwd gamma");
  need(rinv, rows * int64_t{4}, "rmsnorm_bwd rinv");
  need(part, int64_t{rmsnorm_groups(rows)} * H * 4, "rmsnorm_bwd part");
  need(grad_gamma, H * int64_t{4}, "rmsnorm_bwd grad_gamma");
  return hipSuccess;
}

hipError_t launch_sum_parts_bf16(const float* parts, int S, int64_t stride, uint16_t* out,
                                 int64_t n, hipStream_t) {
  ++g_launches;
  need(parts, ((S - 1) * stride + n) * 4, "sum_parts parts");
  need(out, n * 2, "sum_parts out");
  return hipSuccess;
}
hipError_t launch_scale(void* x, int64_t n, bool bf16, const float* s, hipStream_t) {
  ++g_launches;
  need(x, n * (bf16 ? 2 : 4), "scale x");
  need(s, 4, "scale factor");
  return hipSuccess;
}
hipError_t launch_loss_sum(const float* row_loss, int64_t loss_stride, int rows, float, int,
                           float* loss, hipStream_t) {
  ++g_launches;
  need(row_loss, ((rows - 1) * loss_stride + 1) * 4, "loss_sum rows");
  need(loss, 4, "loss_sum loss");
  return hipSuccess;
}
hipError_t launch_mfma_rate(const void* ops, int n_groups, int64_t, int workgroups, float* sink,
                            uint64_t* clocks, hipStream_t) {
  ++g_launches;
  need(ops, int64_t{n_groups} * 128, "mfma_rate operands");
  need(sink, int64_t{workgroups} * 4 * 4, "mfma_rate sink");
  need(clocks, int64_t{workgroups} * 4 * 2 * 8, "mfma_rate clocks");
  return hipSuccess;
}

}  // namespace flce
