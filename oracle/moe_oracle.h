/*
 * moe_oracle.h — CPU oracle for the MoE expert layer with renormalised top-k routing.
 *
 * TEST INFRASTRUCTURE ONLY. This is a plain, slow, obviously-correct CPU implementation used to
 * check the GPU library. Only the tests, the smoke check and the benchmark's CPU-baseline leg
 * may load it. It shares no code, header, table or helper with the GPU path.
 *
 * What it computes (sources: the web pages on the fused MoE layer):
 *   - MindSpeed-MM issue 625, "InternVL3.5 pure FSDP2" practice doc, section 8.2/8.3: the MoE
 *     block's router is gate -> FP32 softmax -> top-k -> weight normalisation, then the experts
 *     run permute -> grouped_matmul -> SwiGLU -> grouped_matmul -> unpermute.
 *   - same doc, section 2 (model integration): fused weights gate_up [E*H, 2*I], down [E*I, H].
 *   - "DeepSeek MoE: EP and FSDP" guide (gsyq.cn), Expert Parallelism section: the naive MoE
 *     forward ends by summing the experts' outputs weighted by the gate weights; its VeOmni
 *     section orders the permuted rows expert-major, tokens ascending inside an expert.
 *
 * Precision: fp64 throughout, except the router logits, which are fp32 fused-multiply-add
 * chains over four fixed blocks of h (ascending inside a block), added in block order, so that
 * both sides take the top-k decision on identical fp32 values.
 * bf16 inputs are passed as raw 16-bit patterns and widened exactly.
 *
 * Every function returns 0 on success and a negative value on a bad argument.
 */
#ifndef MOE_ORACLE_H
#define MOE_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Threads the OpenMP loops below use (n > 0), and the current maximum. */
void orc_set_threads(int n);
int orc_max_threads(void);

enum { ORC_F32 = 0, ORC_BF16 = 1 };

/* logits[t*E+e] = ((c0 + c1) + c2) + c3 in fp32, where c_b is the chain acc = 0;
 * for h in block b ascending: acc = fmaf(x[t,h], w_gate[h,e], acc); block b = [b*HB, min((b+1)*HB, H)),
 * HB = orc_router_logit_block(H) = 128 * ceil(H / 512) (empty blocks give +0.0). */
int orc_router_logit_block(int64_t H);
int orc_router_logits(const void* x, const void* w_gate, int dt, int64_t T, int64_t H, int64_t E,
                      float* logits);

/* Router statistics for an auxiliary load-balance loss (the practice doc's section 8.1 names an
 * auxiliary-loss capture; the DeepSeek guide's Automodel section keeps the full softmax):
 *   probs[t*E+e]  = exp(l_e - m) / sum_{e'} exp(l_e' - m)      (m = max_e l_e; full softmax)
 *   mean_prob[e]  = (1/T) sum_t probs[t*E+e]
 *   load[e]       = #{(t, j) : topk_idx[t*k+j] == e}          (indices outside [0, E) ignored)
 * probs may be NULL. */
int orc_router_stats(const float* logits, const int32_t* topk_idx, int64_t T, int64_t E, int64_t k,
                     double* probs, double* mean_prob, int64_t* load);

/* Top-k by (logit descending, expert index ascending); slot j = rank j.
 * renorm=1: w_j = exp(l_j - m) / sum_{i in S} exp(l_i - m)   (softmax renormalised over S)
 * renorm=0: w_j = exp(l_j - m) / sum_{all e} exp(l_e - m)     (raw softmax probability) */
int orc_router_topk(const float* logits, int64_t T, int64_t E, int64_t k, int renorm,
                    int32_t* topk_idx, double* topk_w);

/* counts[e], exclusive offsets[0..E], rows ordered by (expert, token, slot) ascending.
 * row_of_slot[t*k+j] = row, slot_of_row[row] = t*k+j. A slot whose index is outside [0, E) is
 * dropped (not counted, row_of_slot = -1); slot_of_row entries past offsets[E] are -1. */
int orc_permute_plan(const int32_t* topk_idx, int64_t T, int64_t k, int64_t E, int32_t* counts,
                     int32_t* offsets, int32_t* row_of_slot, int32_t* slot_of_row);

/* x_perm[r, :] = x[slot_of_row[r] / k, :]  (byte copy, elem_bytes per element) */
int orc_permute_rows(const void* x, int64_t elem_bytes, int64_t H, const int32_t* slot_of_row,
                     int64_t k, int64_t N, void* x_perm);

/* Expert FFN on rows of an expert-grouped buffer. For each requested row r (rows[0..nrows)),
 * e is the expert with offsets[e] <= r < offsets[e+1] and
 *   g = x_perm[r] @ gate_up[e*H:(e+1)*H, 0:I], u = x_perm[r] @ gate_up[e*H:(e+1)*H, I:2I],
 *   a = silu(g) * u,  y = a @ down[e*I:(e+1)*I, :].
 * Outputs (fp64, one row per requested row): y_out [nrows, H]; a_out [nrows, I] and
 * gu_out [nrows, 2I] (g then u) when non-null. */
int orc_expert_rows(const void* x_perm, int dt, int64_t H, int64_t I, int64_t E,
                    const int32_t* offsets, const void* gate_up, const void* down,
                    const int64_t* rows, int64_t nrows, double* y_out, double* a_out, double* gu_out);

/* out[t] = sum_{j<k} w[t,j] * y[row_of_slot[t*k+j]] (+ residual[t]) for each requested token.
 * A slot whose row map is negative has been dropped and contributes nothing (here and in the
 * two backward functions below). */
int orc_combine(const void* y, int dt, int64_t H, int64_t k, const int32_t* row_of_slot,
                const float* topk_w, const void* residual, const int64_t* tokens, int64_t ntok,
                double* out);

/* Whole layer for the requested tokens, per token: out[t] = sum_j w[t,j] * FFN_{idx[t,j]}(x[t])
 * (+ FFN_shared(x[t]) with weight 1 when shared_gate_up is non-null; its intermediate is Is). */
int orc_moe_forward_tokens(const void* x, int dt, int64_t H, int64_t I, int64_t E, int64_t k,
                           const int32_t* topk_idx, const double* topk_w, const void* gate_up,
                           const void* down, const void* shared_gate_up, const void* shared_down,
                           int64_t Is, const int64_t* tokens, int64_t ntok, double* out);

/* ---- backward (loss L with dL/dout = d_out) ----
 * The incoming gradients (d_y, and y in the combine backward) carry their own data type, so that
 * fp32 intermediates can meet bf16 parameters. */

/* d_y[t*k+j] = w[t,j] * d_out[t];  d_w[t,j] = <d_out[t], y[row_of_slot[t*k+j]]> */
int orc_combine_bwd(const void* d_out, int dt, const void* y, int dt_y, int64_t H, int64_t k,
                    const int32_t* row_of_slot, const float* topk_w, const int64_t* tokens,
                    int64_t ntok, double* d_y_slots, double* d_w);

/* Per grouped row r: da = d_y[r] @ down_e^T; dg = da*u*s*(1+g*(1-s)), du = da*g*s (s = sigmoid g);
 * d_x[r] = dg @ gate_up_e[:, :I]^T + du @ gate_up_e[:, I:]^T.  Outputs fp64: d_x_out [nrows,H],
 * d_gu_out [nrows, 2I] (dg then du) when non-null. */
int orc_expert_rows_bwd(const void* x_perm, const void* d_y, int dt, int dt_dy, int64_t H, int64_t I,
                        int64_t E, const int32_t* offsets, const void* gate_up, const void* down,
                        const int64_t* rows, int64_t nrows, double* d_x_out, double* d_gu_out);

/* Weight gradients of expert e: d_gate_up_e [H, 2I] = sum_r x_perm[r]^T (dg|du)[r],
 * d_down_e [I, H] = sum_r a[r]^T d_y[r], over rows r of expert e (zeros when it has none). */
int orc_expert_weight_grads(const void* x_perm, const void* d_y, int dt, int dt_dy, int64_t H, int64_t I,
                            int64_t E, const int32_t* offsets, const void* gate_up,
                            const void* down, int64_t e, double* d_gate_up_e, double* d_down_e);

/* The entries of expert e's weight gradients that belong to intermediate units[q] (0 <= q < nunits):
 * d_gate_up_cols [nunits, 2, H] = columns units[q] and I+units[q] of d_gate_up_e,
 * d_down_rows [nunits, H] = row units[q] of d_down_e. */
int orc_expert_weight_grads_units(const void* x_perm, const void* d_y, int dt, int dt_dy, int64_t H, int64_t I,
                                  int64_t E, const int32_t* offsets, const void* gate_up,
                                  const void* down, int64_t e, const int64_t* units, int64_t nunits,
                                  double* d_gate_up_cols, double* d_down_rows);

/* d_x[t] = sum_j d_x_perm[row_of_slot[t*k+j]] (+ d_x_add[t]) */
int orc_permute_bwd(const void* d_x_perm, int dt, int64_t H, int64_t k, const int32_t* row_of_slot,
                    const void* d_x_add, const int64_t* tokens, int64_t ntok, double* d_x);

/* Gradient through the routing weights (selection has none).
 * renorm=1: dl[t,S_i] = w_i (dw_i - sum_j w_j dw_j), 0 off S.
 * renorm=0: dl[t,e] = p_e (1[e in S] dw_e - sum_{j in S} p_j dw_j) with p the full softmax. */
int orc_router_topk_bwd(const float* logits, const int32_t* topk_idx, const double* d_w,
                        int64_t T, int64_t E, int64_t k, int renorm, double* d_logits);

/* d_w_gate = x^T dl  [H, E]; d_x = dl @ w_gate^T  [T, H] (both fp64, over all T tokens) */
int orc_router_logits_bwd(const void* x, const void* w_gate, int dt, const double* d_logits,
                          int64_t T, int64_t H, int64_t E, double* d_w_gate, double* d_x);

#ifdef __cplusplus
}
#endif
#endif
