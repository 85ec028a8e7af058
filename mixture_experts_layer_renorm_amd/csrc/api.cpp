// C ABI of the MoE layer library: host-side validation, then the kernel launchers.
#include "moe_rocm.h"

#include <stdarg.h>
#include <stdio.h>

#include "internal.hpp"

namespace {

thread_local char g_err[512] = "";

moe_status fail(moe_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return st;
}

moe_status ok() {
  g_err[0] = '\0';
  return MOE_OK;
}

moe_status hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

bool bad_dt(moe_dtype dt) { return dt != MOE_F32 && dt != MOE_BF16; }

constexpr int kMaxE = 1024;
constexpr int kMaxK = 32;

#define REQUIRE(cond, st, ...) \
  do {                         \
    if (!(cond)) return fail(st, __VA_ARGS__); \
  } while (0)

}  // namespace

extern "C" {

const char* moe_last_error(void) { return g_err; }

int moe_abi_version(void) { return 1; }

moe_status moe_router_logits(const void* x, const void* w_gate, moe_dtype dt, int T, int H, int E, float* logits,
                             hipStream_t stream) {
  REQUIRE(!bad_dt(dt), MOE_ERR_INVALID_ARG, "moe_router_logits: unknown dtype %d", (int)dt);
  REQUIRE(T >= 0 && H >= 0, MOE_ERR_INVALID_ARG, "moe_router_logits: T=%d H=%d must be >= 0", T, H);
  REQUIRE(E >= 1 && E <= kMaxE, MOE_ERR_INVALID_ARG, "moe_router_logits: E=%d outside [1, %d]", E, kMaxE);
  if (T == 0) return ok();
  REQUIRE(x && w_gate && logits, MOE_ERR_INVALID_ARG, "moe_router_logits: null pointer");
  return hip_status(moe::launch_router_logits(x, w_gate, (int)dt, T, H, E, logits, stream), "moe_router_logits");
}

moe_status moe_router_topk(const float* logits, int T, int E, int k, int renorm, int32_t* topk_idx, float* topk_w,
                           hipStream_t stream) {
  REQUIRE(T >= 0, MOE_ERR_INVALID_ARG, "moe_router_topk: T=%d must be >= 0", T);
  REQUIRE(E >= 1 && E <= kMaxE, MOE_ERR_INVALID_ARG, "moe_router_topk: E=%d outside [1, %d]", E, kMaxE);
  REQUIRE(k >= 1 && k <= E && k <= kMaxK, MOE_ERR_INVALID_ARG, "moe_router_topk: k=%d outside [1, min(E=%d, %d)]", k,
          E, kMaxK);
  REQUIRE(renorm == 0 || renorm == 1, MOE_ERR_INVALID_ARG, "moe_router_topk: renorm=%d must be 0 or 1", renorm);
  if (T == 0) return ok();
  REQUIRE(logits && topk_idx && topk_w, MOE_ERR_INVALID_ARG, "moe_router_topk: null pointer");
  return hip_status(moe::launch_router_topk(logits, T, E, k, renorm, topk_idx, topk_w, stream), "moe_router_topk");
}

size_t moe_router_stats_workspace_bytes(int T, int E) {
  if (T <= 0 || E <= 0) return 0;
  return moe::router_stats_workspace_bytes(T, E);
}

moe_status moe_router_stats(const float* logits, const int32_t* topk_idx, int T, int E, int k, float* probs,
                            float* mean_prob, int32_t* load, void* workspace, size_t workspace_bytes,
                            hipStream_t stream) {
  const char* fn = "moe_router_stats";
  REQUIRE(T >= 0, MOE_ERR_INVALID_ARG, "%s: T=%d must be >= 0", fn, T);
  REQUIRE(E >= 1 && E <= kMaxE, MOE_ERR_INVALID_ARG, "%s: E=%d outside [1, %d]", fn, E, kMaxE);
  REQUIRE(k >= 1 && k <= E && k <= kMaxK, MOE_ERR_INVALID_ARG, "%s: k=%d outside [1, min(E=%d, %d)]", fn, k, E, kMaxK);
  REQUIRE(mean_prob && load, MOE_ERR_INVALID_ARG, "%s: null mean_prob/load", fn);
  if (T == 0) {  // no tokens: zero statistics (fill kernels; 0.0f is all-zero bits)
    hipError_t e = moe::launch_fill_i32((int32_t*)mean_prob, E, 0, stream);
    if (e == hipSuccess) e = moe::launch_fill_i32(load, E, 0, stream);
    return hip_status(e, fn);
  }
  REQUIRE(logits && topk_idx, MOE_ERR_INVALID_ARG, "%s: null pointer", fn);
  const size_t need = moe::router_stats_workspace_bytes(T, E);
  REQUIRE(workspace && workspace_bytes >= need, MOE_ERR_WORKSPACE, "%s: workspace of %zu bytes given, %zu needed", fn,
          workspace ? workspace_bytes : (size_t)0, need);
  return hip_status(moe::launch_router_stats(logits, topk_idx, T, E, k, probs, mean_prob, load, workspace, stream), fn);
}

size_t moe_permute_workspace_bytes(int T, int k, int E) {
  (void)k;
  if (T <= 0 || E <= 0) return 0;
  return moe::permute_workspace_bytes(T, E);
}

moe_status moe_permute(const void* x, moe_dtype dt, int T, int H, const int32_t* topk_idx, int k, int E, void* x_perm,
                       int32_t* counts, int32_t* offsets, int32_t* row_of_slot, int32_t* slot_of_row, void* workspace,
                       size_t workspace_bytes, hipStream_t stream) {
  REQUIRE(!bad_dt(dt), MOE_ERR_INVALID_ARG, "moe_permute: unknown dtype %d", (int)dt);
  REQUIRE(T >= 0 && H >= 0, MOE_ERR_INVALID_ARG, "moe_permute: T=%d H=%d must be >= 0", T, H);
  REQUIRE(E >= 1 && E <= kMaxE, MOE_ERR_INVALID_ARG, "moe_permute: E=%d outside [1, %d]", E, kMaxE);
  REQUIRE(k >= 1 && k <= E && k <= kMaxK, MOE_ERR_INVALID_ARG, "moe_permute: k=%d outside [1, min(E=%d, %d)]", k, E,
          kMaxK);
  REQUIRE((int64_t)T * k <= 0x7fffffffLL, MOE_ERR_INVALID_ARG, "moe_permute: T*k overflows int32");
  REQUIRE(counts && offsets, MOE_ERR_INVALID_ARG, "moe_permute: null counts/offsets");
  if (T == 0) {
    // nothing routed: counts = 0, offsets = 0 are still produced (a fill kernel, safe in a captured graph)
    hipError_t e = moe::launch_fill_i32(counts, E, 0, stream);
    if (e == hipSuccess) e = moe::launch_fill_i32(offsets, E + 1, 0, stream);
    return hip_status(e, "moe_permute");
  }
  REQUIRE(topk_idx && row_of_slot && slot_of_row, MOE_ERR_INVALID_ARG, "moe_permute: null pointer");
  REQUIRE(!x_perm || x, MOE_ERR_INVALID_ARG, "moe_permute: x is NULL but x_perm is not");
  const size_t need = moe::permute_workspace_bytes(T, E);
  REQUIRE(workspace && workspace_bytes >= need, MOE_ERR_WORKSPACE,
          "moe_permute: workspace of %zu bytes given, %zu needed", workspace ? workspace_bytes : (size_t)0, need);
  return hip_status(moe::launch_permute(x, (int)dt, T, H, topk_idx, k, E, x_perm, counts, offsets, row_of_slot,
                                        slot_of_row, (int32_t*)workspace, stream),
                    "moe_permute");
}

moe_status moe_permute_noalloc(const void* x, moe_dtype dt, int T, int H, const int32_t* topk_idx, int k, int E,
                               void* x_perm, int32_t* counts, int32_t* offsets, int32_t* row_of_slot,
                               int32_t* slot_of_row, hipStream_t stream) {
  const char* fn = "moe_permute_noalloc";
  REQUIRE(!bad_dt(dt), MOE_ERR_INVALID_ARG, "%s: unknown dtype %d", fn, (int)dt);
  REQUIRE(T >= 0 && H >= 0, MOE_ERR_INVALID_ARG, "%s: T=%d H=%d must be >= 0", fn, T, H);
  REQUIRE(E >= 1 && E <= kMaxE, MOE_ERR_INVALID_ARG, "%s: E=%d outside [1, %d]", fn, E, kMaxE);
  REQUIRE(k >= 1 && k <= E && k <= kMaxK, MOE_ERR_INVALID_ARG, "%s: k=%d outside [1, min(E=%d, %d)]", fn, k, E,
          kMaxK);
  REQUIRE((int64_t)T * k <= 0x7fffffffLL, MOE_ERR_INVALID_ARG, "%s: T*k overflows int32", fn);
  const int64_t need = (int64_t)moe::permute_ncount(T) * E;
  REQUIRE(need <= moe::kPermuteScratchInts, MOE_ERR_WORKSPACE,
          "%s: ceil(T/16)*E = %lld chunk counts exceed the fixed scratch of %lld (T=%d E=%d); use moe_permute with a "
          "workspace",
          fn, (long long)need, (long long)moe::kPermuteScratchInts, T, E);
  REQUIRE(counts && offsets, MOE_ERR_INVALID_ARG, "%s: null counts/offsets", fn);
  if (T == 0) {
    hipError_t e = moe::launch_fill_i32(counts, E, 0, stream);
    if (e == hipSuccess) e = moe::launch_fill_i32(offsets, E + 1, 0, stream);
    return hip_status(e, fn);
  }
  REQUIRE(topk_idx && row_of_slot && slot_of_row, MOE_ERR_INVALID_ARG, "%s: null pointer", fn);
  REQUIRE(!x_perm || x, MOE_ERR_INVALID_ARG, "%s: x is NULL but x_perm is not", fn);
  int32_t* scratch = nullptr;
  hipError_t e = moe::permute_noalloc_scratch(&scratch);
  if (e == hipSuccess)
    e = moe::launch_permute(x, (int)dt, T, H, topk_idx, k, E, x_perm, counts, offsets, row_of_slot, slot_of_row,
                            scratch, stream);
  return hip_status(e, fn);
}

moe_status moe_router_topk_permute(const float* logits, int T, int E, int k, int renorm, int32_t* topk_idx,
                                   float* topk_w, const void* x, moe_dtype dt, int H, void* x_perm, int32_t* counts,
                                   int32_t* offsets, int32_t* row_of_slot, int32_t* slot_of_row, void* workspace,
                                   size_t workspace_bytes, hipStream_t stream) {
  const char* fn = "moe_router_topk_permute";
  REQUIRE(!bad_dt(dt), MOE_ERR_INVALID_ARG, "%s: unknown dtype %d", fn, (int)dt);
  REQUIRE(T >= 0 && H >= 0, MOE_ERR_INVALID_ARG, "%s: T=%d H=%d must be >= 0", fn, T, H);
  REQUIRE(E >= 1 && E <= kMaxE, MOE_ERR_INVALID_ARG, "%s: E=%d outside [1, %d]", fn, E, kMaxE);
  REQUIRE(k >= 1 && k <= E && k <= kMaxK, MOE_ERR_INVALID_ARG, "%s: k=%d outside [1, min(E=%d, %d)]", fn, k, E,
          kMaxK);
  REQUIRE(renorm == 0 || renorm == 1, MOE_ERR_INVALID_ARG, "%s: renorm=%d must be 0 or 1", fn, renorm);
  REQUIRE((int64_t)T * k <= 0x7fffffffLL, MOE_ERR_INVALID_ARG, "%s: T*k overflows int32", fn);
  REQUIRE(counts && offsets, MOE_ERR_INVALID_ARG, "%s: null counts/offsets", fn);
  if (T == 0) {
    hipError_t e = moe::launch_fill_i32(counts, E, 0, stream);
    if (e == hipSuccess) e = moe::launch_fill_i32(offsets, E + 1, 0, stream);
    return hip_status(e, fn);
  }
  REQUIRE(logits && topk_idx && topk_w && row_of_slot && slot_of_row, MOE_ERR_INVALID_ARG, "%s: null pointer", fn);
  REQUIRE(!x_perm || x, MOE_ERR_INVALID_ARG, "%s: x is NULL but x_perm is not", fn);
  const size_t need = moe::permute_workspace_bytes(T, E);
  REQUIRE(workspace && workspace_bytes >= need, MOE_ERR_WORKSPACE, "%s: workspace of %zu bytes given, %zu needed", fn,
          workspace ? workspace_bytes : (size_t)0, need);
  int32_t* chunk_counts = (int32_t*)workspace;
  bool counted = false;
  hipError_t e = moe::launch_router_topk(logits, T, E, k, renorm, topk_idx, topk_w, stream, chunk_counts, &counted);
  if (e == hipSuccess)
    e = counted ? moe::launch_permute_counted(x, (int)dt, T, H, topk_idx, k, E, x_perm, counts, offsets, row_of_slot,
                                              slot_of_row, chunk_counts, stream)
                : moe::launch_permute(x, (int)dt, T, H, topk_idx, k, E, x_perm, counts, offsets, row_of_slot,
                                      slot_of_row, chunk_counts, stream);
  return hip_status(e, fn);
}

namespace {
moe_status check_ffn(const char* fn, moe_dtype dt, int N, int H, int I, int E) {
  REQUIRE(!bad_dt(dt), MOE_ERR_INVALID_ARG, "%s: unknown dtype %d", fn, (int)dt);
  REQUIRE(N >= 0 && H >= 1 && I >= 1, MOE_ERR_INVALID_ARG, "%s: N=%d H=%d I=%d out of range", fn, N, H, I);
  REQUIRE(E >= 1 && E <= kMaxE, MOE_ERR_INVALID_ARG, "%s: E=%d outside [1, %d]", fn, E, kMaxE);
  // the bf16 kernels address one expert's weight block with 32-bit byte offsets
  REQUIRE((int64_t)H * 2 * I * 4 < 0x7fffffffLL, MOE_ERR_UNSUPPORTED, "%s: H*I=%lld too large", fn,
          (long long)H * I);
  return MOE_OK;
}
}  // namespace

moe_status moe_grouped_gemm_swiglu(const void* x_perm, const void* gate_up, moe_dtype dt, int N, int H, int I, int E,
                                   const int32_t* expert_offsets, void* h, void* gu_saved, hipStream_t stream) {
  const char* fn = "moe_grouped_gemm_swiglu";
  moe_status st = check_ffn(fn, dt, N, H, I, E);
  if (st != MOE_OK) return st;
  if (N == 0) return ok();
  REQUIRE(x_perm && gate_up && expert_offsets && h, MOE_ERR_INVALID_ARG, "%s: null pointer", fn);
  return hip_status(moe::launch_gemm_gate_up(x_perm, gate_up, (int)dt, N, H, I, E, expert_offsets, h, gu_saved, stream),
                    fn);
}

namespace {
moe_status check_gather(const char* fn, moe_dtype dt, int T, int k, int N, int H) {
  REQUIRE(T >= 0 && k >= 1 && k <= kMaxK, MOE_ERR_INVALID_ARG, "%s: T=%d k=%d (need T >= 0, 1 <= k <= %d)", fn, T, k,
          kMaxK);
  REQUIRE((int64_t)N <= (int64_t)T * k, MOE_ERR_INVALID_ARG, "%s: N=%d rows but only T*k=%lld slots", fn, N,
          (long long)T * k);
  REQUIRE((int64_t)T * H * (int64_t)moe::dtype_bytes((int)dt) < (1LL << 31), MOE_ERR_UNSUPPORTED, "%s: x [T=%d, H=%d] exceeds 2 GiB", fn, T,
          H);
  return MOE_OK;
}
}  // namespace

moe_status moe_grouped_gemm_swiglu_gather(const void* x, const int32_t* slot_of_row, int T, int k, const void* gate_up,
                                          moe_dtype dt, int N, int H, int I, int E, const int32_t* expert_offsets,
                                          void* h, void* gu_saved, hipStream_t stream) {
  const char* fn = "moe_grouped_gemm_swiglu_gather";
  moe_status st = check_ffn(fn, dt, N, H, I, E);
  if (st == MOE_OK) st = check_gather(fn, dt, T, k, N, H);
  if (st != MOE_OK) return st;
  if (N == 0) return ok();
  REQUIRE(x && slot_of_row && gate_up && expert_offsets && h, MOE_ERR_INVALID_ARG, "%s: null pointer", fn);
  return hip_status(moe::launch_gemm_gate_up(x, gate_up, (int)dt, N, H, I, E, expert_offsets, h, gu_saved, stream,
                                             slot_of_row, k, T),
                    fn);
}

moe_status moe_grouped_swiglu_ffn_gather(const void* x, const int32_t* slot_of_row, int T, int k, const void* gate_up,
                                         const void* down, moe_dtype dt, int N, int H, int I, int E,
                                         const int32_t* expert_offsets, void* h, void* gu_saved, void* y,
                                         hipStream_t stream) {
  const char* fn = "moe_grouped_swiglu_ffn_gather";
  moe_status st = check_ffn(fn, dt, N, H, I, E);
  if (st == MOE_OK) st = check_gather(fn, dt, T, k, N, H);
  if (st != MOE_OK) return st;
  if (N == 0) return ok();
  REQUIRE(x && slot_of_row && gate_up && down && expert_offsets && h && y, MOE_ERR_INVALID_ARG, "%s: null pointer", fn);
  hipError_t e = moe::launch_gemm_gate_up(x, gate_up, (int)dt, N, H, I, E, expert_offsets, h, gu_saved, stream,
                                          slot_of_row, k, T);
  if (e == hipSuccess) e = moe::launch_gemm_down(h, down, (int)dt, N, H, I, E, expert_offsets, y, stream);
  return hip_status(e, fn);
}

moe_status moe_grouped_gemm_down(const void* h, const void* down, moe_dtype dt, int N, int H, int I, int E,
                                 const int32_t* expert_offsets, void* y, hipStream_t stream) {
  const char* fn = "moe_grouped_gemm_down";
  moe_status st = check_ffn(fn, dt, N, H, I, E);
  if (st != MOE_OK) return st;
  if (N == 0) return ok();
  REQUIRE(h && down && expert_offsets && y, MOE_ERR_INVALID_ARG, "%s: null pointer", fn);
  return hip_status(moe::launch_gemm_down(h, down, (int)dt, N, H, I, E, expert_offsets, y, stream), fn);
}

moe_status moe_grouped_swiglu_ffn(const void* x_perm, const void* gate_up, const void* down, moe_dtype dt, int N, int H,
                                  int I, int E, const int32_t* expert_offsets, void* h, void* gu_saved, void* y,
                                  hipStream_t stream) {
  const char* fn = "moe_grouped_swiglu_ffn";
  moe_status st = check_ffn(fn, dt, N, H, I, E);
  if (st != MOE_OK) return st;
  if (N == 0) return ok();
  REQUIRE(x_perm && gate_up && down && expert_offsets && h && y, MOE_ERR_INVALID_ARG, "%s: null pointer", fn);
  hipError_t e = moe::launch_gemm_gate_up(x_perm, gate_up, (int)dt, N, H, I, E, expert_offsets, h, gu_saved, stream);
  if (e == hipSuccess) e = moe::launch_gemm_down(h, down, (int)dt, N, H, I, E, expert_offsets, y, stream);
  return hip_status(e, fn);
}

moe_status moe_unpermute_combine(const void* y, moe_dtype dt, int T, int H, int k, const int32_t* row_of_slot,
                                 const float* topk_w, const void* residual, void* out, hipStream_t stream) {
  REQUIRE(!bad_dt(dt), MOE_ERR_INVALID_ARG, "moe_unpermute_combine: unknown dtype %d", (int)dt);
  REQUIRE(T >= 0 && H >= 0, MOE_ERR_INVALID_ARG, "moe_unpermute_combine: T=%d H=%d must be >= 0", T, H);
  REQUIRE(k >= 1 && k <= kMaxK, MOE_ERR_INVALID_ARG, "moe_unpermute_combine: k=%d outside [1, %d]", k, kMaxK);
  if (T == 0 || H == 0) return ok();
  REQUIRE(y && row_of_slot && topk_w && out, MOE_ERR_INVALID_ARG, "moe_unpermute_combine: null pointer");
  return hip_status(moe::launch_combine(y, (int)dt, T, H, k, row_of_slot, topk_w, residual, out, stream),
                    "moe_unpermute_combine");
}

// ---- backward ---------------------------------------------------------------------------------
moe_status moe_unpermute_combine_bwd(const void* d_out, const void* y, moe_dtype dt, int T, int H, int k,
                                     const int32_t* row_of_slot, const float* topk_w, void* d_y, float* d_w,
                                     hipStream_t stream) {
  const char* fn = "moe_unpermute_combine_bwd";
  REQUIRE(!bad_dt(dt), MOE_ERR_INVALID_ARG, "%s: unknown dtype %d", fn, (int)dt);
  REQUIRE(T >= 0 && H >= 0, MOE_ERR_INVALID_ARG, "%s: T=%d H=%d must be >= 0", fn, T, H);
  REQUIRE(k >= 1 && k <= kMaxK, MOE_ERR_INVALID_ARG, "%s: k=%d outside [1, %d]", fn, k, kMaxK);
  if (T == 0) return ok();
  REQUIRE(d_out && y && row_of_slot && topk_w && d_y && d_w, MOE_ERR_INVALID_ARG, "%s: null pointer", fn);
  return hip_status(moe::launch_combine_bwd(d_out, y, (int)dt, T, H, k, row_of_slot, topk_w, d_y, d_w, stream), fn);
}

moe_status moe_grouped_swiglu_ffn_bwd(const void* d_y, const void* x_perm, const void* gu_saved, const void* h,
                                      const void* gate_up, const void* down, moe_dtype dt, int N, int H, int I, int E,
                                      const int32_t* expert_offsets, void* d_x_perm, void* d_gate_up, void* d_down,
                                      void* d_gu, hipStream_t stream) {
  const char* fn = "moe_grouped_swiglu_ffn_bwd";
  moe_status st = check_ffn(fn, dt, N, H, I, E);
  if (st != MOE_OK) return st;
  // the weight-gradient products address all rows of one expert with 32-bit byte offsets
  REQUIRE((int64_t)N * (H > 2 * I ? H : 2 * I) * 2 < 0x7fffffffLL, MOE_ERR_UNSUPPORTED,
          "%s: N*max(H, 2I) too large for one call (N=%d H=%d I=%d)", fn, N, H, I);
  REQUIRE(d_gate_up && d_down && expert_offsets, MOE_ERR_INVALID_ARG, "%s: null pointer", fn);
  if (N > 0) REQUIRE(d_y && x_perm && gu_saved && h && gate_up && down && d_x_perm && d_gu, MOE_ERR_INVALID_ARG,
                     "%s: null pointer", fn);
  hipError_t e = hipSuccess;
  if (moe::mfma_shapes_ok((int)dt, H, I, d_y, x_perm, gu_saved, h, gate_up, down, d_x_perm, d_gu) &&
      moe::mfma_shapes_ok((int)dt, H, I, d_gate_up, d_down)) {
    if (N > 0) {
      e = moe::launch_gemm_down_bwd(d_y, down, gu_saved, N, H, I, E, expert_offsets, d_gu, stream);
      if (e == hipSuccess) e = moe::launch_gemm_gate_up_bwd(d_gu, gate_up, N, H, I, E, expert_offsets, d_x_perm, stream);
    }
    // weight gradients cover every expert (zeros for experts without rows, and for N == 0)
    if (e == hipSuccess) e = moe::launch_gemm_wgrad(h, d_y, I, H, E, expert_offsets, d_down, stream);
    if (e == hipSuccess) e = moe::launch_gemm_wgrad(x_perm, d_gu, H, 2 * I, E, expert_offsets, d_gate_up, stream);
  } else {  // fp32, or bf16 widths / alignments the matrix-core kernels do not take
    if (N > 0) {
      e = moe::launch_gen_down_bwd(d_y, down, gu_saved, (int)dt, N, H, I, E, expert_offsets, d_gu, stream);
      if (e == hipSuccess)
        e = moe::launch_gen_gate_up_bwd(d_gu, gate_up, (int)dt, N, H, I, E, expert_offsets, d_x_perm, stream);
    }
    if (e == hipSuccess) e = moe::launch_gen_wgrad(h, d_y, (int)dt, I, H, E, expert_offsets, d_down, stream);
    if (e == hipSuccess) e = moe::launch_gen_wgrad(x_perm, d_gu, (int)dt, H, 2 * I, E, expert_offsets, d_gate_up, stream);
  }
  return hip_status(e, fn);
}

namespace {
moe_status check_bwd(const char* fn, moe_dtype dt, int N, int H, int I, int E) {
  moe_status st = check_ffn(fn, dt, N, H, I, E);
  if (st != MOE_OK) return st;
  return MOE_OK;
}
}  // namespace

moe_status moe_grouped_gemm_down_bwd(const void* d_y, const void* down, const void* gu_saved, moe_dtype dt, int N,
                                     int H, int I, int E, const int32_t* expert_offsets, void* d_gu,
                                     hipStream_t stream) {
  const char* fn = "moe_grouped_gemm_down_bwd";
  moe_status st = check_bwd(fn, dt, N, H, I, E);
  if (st != MOE_OK) return st;
  if (N == 0) return ok();
  REQUIRE(d_y && down && gu_saved && expert_offsets && d_gu, MOE_ERR_INVALID_ARG, "%s: null pointer", fn);
  if (!moe::mfma_shapes_ok((int)dt, H, I, d_y, down, gu_saved, d_gu))
    return hip_status(moe::launch_gen_down_bwd(d_y, down, gu_saved, (int)dt, N, H, I, E, expert_offsets, d_gu, stream),
                      fn);
  return hip_status(moe::launch_gemm_down_bwd(d_y, down, gu_saved, N, H, I, E, expert_offsets, d_gu, stream), fn);
}

moe_status moe_grouped_gemm_gate_up_bwd(const void* d_gu, const void* gate_up, moe_dtype dt, int N, int H, int I,
                                        int E, const int32_t* expert_offsets, void* d_x_perm, hipStream_t stream) {
  const char* fn = "moe_grouped_gemm_gate_up_bwd";
  moe_status st = check_bwd(fn, dt, N, H, I, E);
  if (st != MOE_OK) return st;
  if (N == 0) return ok();
  REQUIRE(d_gu && gate_up && expert_offsets && d_x_perm, MOE_ERR_INVALID_ARG, "%s: null pointer", fn);
  if (!moe::mfma_shapes_ok((int)dt, H, I, d_gu, gate_up, d_x_perm))
    return hip_status(moe::launch_gen_gate_up_bwd(d_gu, gate_up, (int)dt, N, H, I, E, expert_offsets, d_x_perm, stream),
                      fn);
  return hip_status(moe::launch_gemm_gate_up_bwd(d_gu, gate_up, N, H, I, E, expert_offsets, d_x_perm, stream), fn);
}

moe_status moe_grouped_gemm_wgrad(const void* P, const void* Q, moe_dtype dt, int N, int M, int Nq, int E,
                                  const int32_t* expert_offsets, void* d_w, int max_workgroups, hipStream_t stream) {
  const char* fn = "moe_grouped_gemm_wgrad";
  REQUIRE(!bad_dt(dt), MOE_ERR_INVALID_ARG, "%s: unknown dtype %d", fn, (int)dt);
  REQUIRE(N >= 0 && M >= 1 && Nq >= 1, MOE_ERR_INVALID_ARG, "%s: N=%d M=%d Nq=%d out of range", fn, N, M, Nq);
  REQUIRE(E >= 1 && E <= kMaxE, MOE_ERR_INVALID_ARG, "%s: E=%d outside [1, %d]", fn, E, kMaxE);
  // rows of one expert and one expert's output block are addressed with 32-bit byte offsets
  REQUIRE((int64_t)N * (M > Nq ? M : Nq) * 2 < 0x7fffffffLL && (int64_t)M * Nq * 2 < 0x7fffffffLL,
          MOE_ERR_UNSUPPORTED, "%s: N*max(M, Nq) or M*Nq too large for one call (N=%d M=%d Nq=%d)", fn, N, M, Nq);
  REQUIRE(expert_offsets && d_w, MOE_ERR_INVALID_ARG, "%s: null pointer", fn);
  if (N > 0) REQUIRE(P && Q, MOE_ERR_INVALID_ARG, "%s: null pointer", fn);
  if (!moe::mfma_shapes_ok((int)dt, M, Nq, P, Q, d_w))
    return hip_status(moe::launch_gen_wgrad(P, Q, (int)dt, M, Nq, E, expert_offsets, d_w, stream), fn);
  return hip_status(moe::launch_gemm_wgrad(P, Q, M, Nq, E, expert_offsets, d_w, stream, max_workgroups), fn);
}

moe_status moe_permute_bwd(const void* d_x_perm, moe_dtype dt, int T, int H, int k, const int32_t* row_of_slot,
                           const void* d_x_add, void* d_x, hipStream_t stream) {
  const char* fn = "moe_permute_bwd";
  REQUIRE(!bad_dt(dt), MOE_ERR_INVALID_ARG, "%s: unknown dtype %d", fn, (int)dt);
  REQUIRE(T >= 0 && H >= 0, MOE_ERR_INVALID_ARG, "%s: T=%d H=%d must be >= 0", fn, T, H);
  REQUIRE(k >= 1 && k <= kMaxK, MOE_ERR_INVALID_ARG, "%s: k=%d outside [1, %d]", fn, k, kMaxK);
  if (T == 0 || H == 0) return ok();
  REQUIRE(d_x_perm && row_of_slot && d_x, MOE_ERR_INVALID_ARG, "%s: null pointer", fn);
  return hip_status(moe::launch_permute_bwd(d_x_perm, (int)dt, T, H, k, row_of_slot, d_x_add, d_x, stream), fn);
}

moe_status moe_router_topk_bwd(const float* logits, const int32_t* topk_idx, const float* topk_w, const float* d_w,
                               int T, int E, int k, int renorm, float* d_logits, hipStream_t stream) {
  const char* fn = "moe_router_topk_bwd";
  REQUIRE(T >= 0, MOE_ERR_INVALID_ARG, "%s: T=%d must be >= 0", fn, T);
  REQUIRE(E >= 1 && E <= kMaxE, MOE_ERR_INVALID_ARG, "%s: E=%d outside [1, %d]", fn, E, kMaxE);
  REQUIRE(k >= 1 && k <= E && k <= kMaxK, MOE_ERR_INVALID_ARG, "%s: k=%d outside [1, min(E=%d, %d)]", fn, k, E, kMaxK);
  REQUIRE(renorm == 0 || renorm == 1, MOE_ERR_INVALID_ARG, "%s: renorm=%d must be 0 or 1", fn, renorm);
  if (T == 0) return ok();
  REQUIRE(topk_idx && topk_w && d_w && d_logits, MOE_ERR_INVALID_ARG, "%s: null pointer", fn);
  REQUIRE(renorm || logits, MOE_ERR_INVALID_ARG, "%s: the raw-softmax gradient needs the logits", fn);
  return hip_status(moe::launch_router_topk_bwd(logits, topk_idx, topk_w, d_w, T, E, k, renorm, d_logits, stream), fn);
}

moe_status moe_router_logits_bwd(const void* x, const void* w_gate, const float* d_logits, moe_dtype dt, int T, int H,
                                 int E, float* d_w_gate, const void* d_x_in, void* d_x, hipStream_t stream) {
  const char* fn = "moe_router_logits_bwd";
  REQUIRE(!bad_dt(dt), MOE_ERR_INVALID_ARG, "%s: unknown dtype %d", fn, (int)dt);
  REQUIRE(T >= 0 && H >= 1, MOE_ERR_INVALID_ARG, "%s: T=%d H=%d out of range", fn, T, H);
  REQUIRE(E >= 1 && E <= kMaxE, MOE_ERR_INVALID_ARG, "%s: E=%d outside [1, %d]", fn, E, kMaxE);
  REQUIRE(d_w_gate || d_x, MOE_ERR_INVALID_ARG, "%s: nothing to compute (d_w_gate and d_x are both NULL)", fn);
  if (T == 0) {  // no tokens: x^T dl over an empty K is zero (a fill kernel); d_x has no rows
    const int64_t n = (int64_t)H * E;
    REQUIRE(n <= 0x7fffffffLL, MOE_ERR_INVALID_ARG, "%s: H*E too large", fn);
    return hip_status(d_w_gate ? moe::launch_fill_i32((int32_t*)d_w_gate, (int)n, 0, stream) : hipSuccess, fn);
  }
  REQUIRE(x && w_gate && d_logits, MOE_ERR_INVALID_ARG, "%s: null pointer", fn);
  return hip_status(
      moe::launch_router_logits_bwd(x, w_gate, d_logits, (int)dt, T, H, E, d_w_gate, d_x_in, d_x, stream), fn);
}

}  // extern "C"
