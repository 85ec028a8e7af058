// Kernel launchers behind the C ABI. Each enqueues on the given stream and returns
// hipGetLastError() after the launch. Arguments are validated by the ABI layer beforehand.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

enum { kF32 = 0, kBF16 = 1 };

inline size_t dtype_bytes(int dt) { return dt == kF32 ? 4 : 2; }

// router.hip
hipError_t launch_router_logits(const void* x, const void* w_gate, int dt, int T, int H, int E, float* logits,
                                hipStream_t s);
size_t router_stats_workspace_bytes(int T, int E);
hipError_t launch_router_stats(const float* logits, const int32_t* topk_idx, int T, int E, int k, float* probs,
                               float* mean_prob, int32_t* load, void* workspace, hipStream_t s);
// chunk_counts (may be NULL): the expert histogram of every kCountTok tokens, [permute_ncount(T), E],
// as permute_count_kernel writes it; returns false in *counted when this E takes the separate count
hipError_t launch_router_topk(const float* logits, int T, int E, int k, int renorm, int32_t* idx, float* w,
                              hipStream_t s, int32_t* chunk_counts = nullptr, bool* counted = nullptr);

// permute.hip
constexpr int kPermuteChunk = 64;   // tokens per plan chunk (64 measured faster than 128 or 256)
inline int permute_nchunks(int T) { return (T + kPermuteChunk - 1) / kPermuteChunk; }
// The expert histograms are kept per kCountTok tokens (four rows per plan chunk), the granularity at
// which the top-k kernel's workgroups own tokens: 16-token workgroups spread the top-k over every CU.
constexpr int kCountTok = 16;
constexpr int kCountPerChunk = kPermuteChunk / kCountTok;
inline int permute_ncount(int T) { return (T + kCountTok - 1) / kCountTok; }
inline size_t permute_workspace_bytes(int T, int E) { return (size_t)permute_ncount(T) * (size_t)E * sizeof(int32_t); }
hipError_t launch_fill_i32(int32_t* p, int n, int32_t v, hipStream_t s);
// allocation-free permute: its chunk counts in a fixed device array of kPermuteScratchInts int32
// (4 MiB) per GPU; *out = this device's address of it (looked up once per device)
constexpr int64_t kPermuteScratchInts = 1 << 20;
hipError_t permute_noalloc_scratch(int32_t** out);
hipError_t launch_permute(const void* x, int dt, int T, int H, const int32_t* topk_idx, int k, int E, void* x_perm,
                          int32_t* counts, int32_t* offsets, int32_t* row_of_slot, int32_t* slot_of_row,
                          int32_t* chunk_counts, hipStream_t s);
// the same from chunk counts already computed (by the top-k kernel)
hipError_t launch_permute_counted(const void* x, int dt, int T, int H, const int32_t* topk_idx, int k, int E,
                                  void* x_perm, int32_t* counts, int32_t* offsets, int32_t* row_of_slot,
                                  int32_t* slot_of_row, const int32_t* chunk_counts, hipStream_t s);

// grouped_gemm.hip
hipError_t launch_gemm_gate_up(const void* x_perm, const void* gate_up, int dt, int N, int H, int I, int E,
                               const int32_t* offsets, void* h, void* gu_saved, hipStream_t s,
                               const int32_t* slot_of_row = nullptr, int k = 1, int T = 0);
hipError_t launch_gemm_down(const void* h, const void* down, int dt, int N, int H, int I, int E, const int32_t* offsets,
                            void* y, hipStream_t s);
hipError_t launch_gemm_down_bwd(const void* d_y, const void* down, const void* gu_saved, int N, int H, int I, int E,
                                const int32_t* offsets, void* d_gu, hipStream_t s);
hipError_t launch_gemm_gate_up_bwd(const void* d_gu, const void* gate_up, int N, int H, int I, int E,
                                   const int32_t* offsets, void* d_x, hipStream_t s);
// max_wg > 0 caps the workgroups (one per CU) of the persistent weight-gradient kernels, so that
// another stream's kernels can run on the remaining CUs
hipError_t launch_gemm_wgrad(const void* P, const void* Q, int M, int Nq, int E, const int32_t* offsets, void* d_w,
                             hipStream_t s, int max_wg = 0);

// generic.hip: the expert FFN products for fp32 and for bf16 shapes the matrix-core kernels do not
// take (H or I not a multiple of 8, buffers not 16-byte aligned); one thread per output element
hipError_t launch_gen_ffn1(const void* A, const void* W, int dt, const int32_t* offsets, int E, int N, int H, int I,
                           void* h, void* gu_saved, const int32_t* a_slot, int a_div, hipStream_t s);
hipError_t launch_gen_ffn2(const void* Hh, const void* D, int dt, const int32_t* offsets, int E, int N, int H, int I,
                           void* y, hipStream_t s);
hipError_t launch_gen_down_bwd(const void* d_y, const void* down, const void* gu_saved, int dt, int N, int H, int I,
                               int E, const int32_t* offsets, void* d_gu, hipStream_t s);
hipError_t launch_gen_gate_up_bwd(const void* d_gu, const void* gate_up, int dt, int N, int H, int I, int E,
                                  const int32_t* offsets, void* d_x, hipStream_t s);
hipError_t launch_gen_wgrad(const void* P, const void* Q, int dt, int M, int Nq, int E, const int32_t* offsets,
                            void* d_w, hipStream_t s);
// the matrix-core kernels take bf16 with every width a multiple of 8 and 16-byte aligned buffers
inline bool mfma_shapes_ok(int dt, int a, int b, const void* p0, const void* p1 = nullptr, const void* p2 = nullptr,
                           const void* p3 = nullptr, const void* p4 = nullptr, const void* p5 = nullptr,
                           const void* p6 = nullptr, const void* p7 = nullptr) {
  const uintptr_t m = (uintptr_t)p0 | (uintptr_t)p1 | (uintptr_t)p2 | (uintptr_t)p3 | (uintptr_t)p4 | (uintptr_t)p5 |
                      (uintptr_t)p6 | (uintptr_t)p7;
  return dt == kBF16 && a % 8 == 0 && b % 8 == 0 && (m & 15u) == 0;
}

// backward.hip
hipError_t launch_combine_bwd(const void* d_out, const void* y, int dt, int T, int H, int k, const int32_t* row_of_slot,
                              const float* topk_w, void* d_y, float* d_w, hipStream_t s);
hipError_t launch_permute_bwd(const void* d_x_perm, int dt, int T, int H, int k, const int32_t* row_of_slot,
                              const void* d_x_add, void* d_x, hipStream_t s);
hipError_t launch_router_topk_bwd(const float* logits, const int32_t* idx, const float* w, const float* d_w, int T,
                                  int E, int k, int renorm, float* d_logits, hipStream_t s);
hipError_t launch_router_logits_bwd(const void* x, const void* w_gate, const float* d_logits, int dt, int T, int H,
                                    int E, float* d_w_gate, const void* d_x_in, void* d_x, hipStream_t s);

// combine.hip
hipError_t launch_combine(const void* y, int dt, int T, int H, int k, const int32_t* row_of_slot, const float* topk_w,
                          const void* residual, void* out, hipStream_t s);

}  // namespace moe
