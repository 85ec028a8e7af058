/*
 * moe_rocm.h — C ABI of the MI355X (gfx950) MoE expert layer with renormalised top-k routing.
 *
 * The layer (one GPU):
 *   forward:  moe_router_logits -> moe_router_topk -> moe_permute -> moe_grouped_swiglu_ffn -> moe_unpermute_combine
 *   backward: moe_unpermute_combine_bwd -> moe_grouped_swiglu_ffn_bwd -> moe_permute_bwd, and
 *             moe_router_topk_bwd -> moe_router_logits_bwd
 *
 * Sources for what each call computes (web pages on the fused MoE layer):
 *   [MM]  MindSpeed-MM issue 625, "InternVL3.5 pure FSDP2" practice doc: section 8.2/8.3 (router is
 *         gate -> FP32 softmax -> top-k -> weight normalisation; experts run permute -> grouped_matmul
 *         -> SwiGLU -> grouped_matmul -> unpermute), section 2 (fused weights gate_up [E*H, 2*I],
 *         down [E*I, H]); optimisation doc section 2.1 (experts grouped into one call).
 *   [DS]  "DeepSeek MoE: EP and FSDP" guide (gsyq.cn): Expert Parallelism section (gate scores,
 *         expert choice, dispatch, expert compute, gate-weighted sum of the outputs), VeOmni section
 *         (per-expert token counts; permuted rows expert-major, tokens ascending inside an expert),
 *         Automodel/DeepEP section (fp32 top-k weights; the dispatch "handle" reused by combine).
 *   [FT]  LLaMA-Factory "FSDPTurbo EP/EFSDP" design note, section 3 (the fused dispatcher's device
 *         permute / grouped matmul / unpermute; empty experts must be handled).
 *
 * Conventions for every call:
 *   - Pointers are DEVICE pointers unless marked "host". The caller allocates and owns every buffer;
 *     the library never allocates, frees, synchronises or copies to the host on these paths.
 *   - Every call only enqueues kernels on `stream` (0 = the null stream) and returns; results are
 *     ready when the stream reaches them.
 *   - Tensors are contiguous and row-major. bf16 data is raw bfloat16 (16-bit) storage.
 *     Routing weights are always fp32; indices and row maps are int32.
 *   - Sizes: T, H, I, N >= 0 (a zero size enqueues nothing); 1 <= E <= 1024; 1 <= k <= min(E, 32).
 *     Any H, I >= 1 in either dtype: the grouped FFN and its backward run on the matrix cores for
 *     bf16 with H and I multiples of 8 and 16-byte aligned buffers, and on generic kernels (one
 *     thread per output element, fp32 accumulation, much slower) for everything else.
 *   - Results are bitwise deterministic run to run (no floating-point atomics).
 *   - Errors: a moe_status is returned; arguments are checked on the host before any launch and a
 *     failed check enqueues nothing. moe_last_error() gives the calling thread's last message.
 *     A launch failure reports MOE_ERR_HIP. Nothing aborts and nothing falls back silently.
 *     Device-side values are not checked on the host: expert indices outside [0, E) are dropped by the
 *     permute (no row, not counted), a token may name one expert in several slots (one row per slot),
 *     and negative row maps are skipped; expert_offsets must be non-decreasing with offsets[E] <= the
 *     buffer's rows, and row maps must index existing rows.
 *   - Sizing: the permute's layout handle is four caller-owned int32 arrays (counts [E], offsets [E+1],
 *     row_of_slot [T*k], slot_of_row [T*k]) rather than one packed plan buffer, because the FFN and the
 *     combine take them one by one and a caller that already holds grouped rows (one expert-parallel
 *     rank after its exchange) passes its own offsets and row maps; the permute's scratch is sized by
 *     moe_permute_workspace_bytes. The FFN backward's only intermediate, d_gu [N, 2I], is also one of
 *     its outputs, so the caller allocates it like the other outputs instead of sizing a workspace.
 */
#ifndef MOE_ROCM_H
#define MOE_ROCM_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1, /* null pointer, size out of range, misaligned buffer */
  MOE_ERR_UNSUPPORTED = 2, /* legal request this build does not implement (e.g. sizes past 32-bit offsets) */
  MOE_ERR_WORKSPACE = 3,   /* workspace missing or smaller than required */
  MOE_ERR_HIP = 4          /* a HIP runtime call or kernel launch failed */
} moe_status;

/* Element type of inputs, weights and activations. A plain int, so that any value a caller passes
 * is a valid argument value: values other than these two are rejected with MOE_ERR_INVALID_ARG. */
typedef int moe_dtype;
enum { MOE_F32 = 0, MOE_BF16 = 1 };

/* Message for the calling thread's last non-OK status ("" if none). Never NULL. */
const char* moe_last_error(void);

/* Version of this ABI (incremented on incompatible change). */
int moe_abi_version(void);

/* ---- (1) router logits -------------------------------------------------------------------------
 * [MM 8.2/8.3] the gate: logits = x @ w_gate, consumed by the FP32 softmax.
 * logits[t, e] = ((c_0 + c_1) + c_2) + c_3 in fp32, where c_b is acc after `acc = fmaf(x[t,h],
 * w_gate[h,e], acc)` from acc = 0 over the h of block b = [b*HB, min((b+1)*HB, H)) in ascending order,
 * HB = 128 * ceil(H / 512) (IEEE fused multiply-add; empty blocks give 0) — a fixed order, so that the
 * top-k decision is reproducible bit for bit, with four independent chains per logit.
 *   x      [T, H]  dt       w_gate [H, E] dt       logits [T, E] fp32 (output)                       */
moe_status moe_router_logits(const void* x, const void* w_gate, moe_dtype dt, int T, int H, int E,
                             float* logits, hipStream_t stream);

/* ---- (2) softmax -> top-k -> renormalise ---------------------------------------------------------
 * [MM 8.2/8.3] FP32 softmax, top-k, weight normalisation; [DS Automodel] fp32 top-k weights.
 * Selection: the k largest logits (softmax is monotone), ties to the lower expert index; slot j holds
 * the j-th largest. With m = max_e logits[t, e]:
 *   renorm = 1:  topk_w[t, j] = exp(l_j - m) / sum_{i selected} exp(l_i - m)   (sums to 1)
 *   renorm = 0:  topk_w[t, j] = exp(l_j - m) / sum_{all e} exp(l_e - m)        (raw probability)
 *   logits [T, E] fp32 (finite)     topk_idx [T, k] int32 (out)     topk_w [T, k] fp32 (out)        */
moe_status moe_router_topk(const float* logits, int T, int E, int k, int renorm, int32_t* topk_idx,
                           float* topk_w, hipStream_t stream);

/* Router statistics for an auxiliary load-balance loss ([MM 8.1]: the trainer installs an
 * auxiliary-loss capture; [DS Automodel] keeps the full softmax probabilities):
 *   probs[t, e]  = exp(l[t,e] - m_t) / sum_e' exp(l[t,e'] - m_t)    (full softmax, fp32; may be NULL)
 *   mean_prob[e] = (1/T) sum_t probs[t, e]                           (fp32, fixed summation order)
 *   load[e]      = #{(t, j) : topk_idx[t, j] == e}                   (int32; indices outside [0, E)
 *                                                                      are not counted)
 *   logits [T, E] fp32 (finite); topk_idx [T, k] int32; workspace: device scratch of at least
 *   moe_router_stats_workspace_bytes(T, E) bytes (no initialisation needed). T = 0 gives zeros.   */
size_t moe_router_stats_workspace_bytes(int T, int E);
moe_status moe_router_stats(const float* logits, const int32_t* topk_idx, int T, int E, int k, float* probs,
                            float* mean_prob, int32_t* load, void* workspace, size_t workspace_bytes,
                            hipStream_t stream);

/* ---- (3) permute ----------------------------------------------------------------------------------
 * [DS VeOmni] group the N = T*k rows by expert: counts[e] = #slots choosing e, offsets = exclusive
 * scan (offsets[E] = number of valid slots), rows ordered by (expert, token, slot) ascending:
 *   row_of_slot[t*k + j] = row of slot j of token t,  slot_of_row[row] = t*k + j,
 *   x_perm[row, :] = x[t, :]  (bit copy).
 * Slots whose index is outside [0, E) get no row: row_of_slot = -1, they are not counted, and
 * slot_of_row past offsets[E] is left untouched. A token that names one expert in several slots
 * gets one row per slot.
 *   x [T, H] dt; topk_idx [T, k] int32; x_perm [T*k, H] dt (out); counts [E], offsets [E+1],
 *   row_of_slot [T*k], slot_of_row [T*k] int32 (out); workspace: device scratch of at least
 *   moe_permute_workspace_bytes(T, k, E) bytes (contents need no initialisation).
 * x_perm may be NULL (then x may be too): only the plan (counts, offsets, row maps) is computed, for
 * the gathering FFN below, which reads the rows from x through slot_of_row.
 * The (counts, offsets, row_of_slot) triple is the layout handle that the FFN and combine take.  */
size_t moe_permute_workspace_bytes(int T, int k, int E);
moe_status moe_permute(const void* x, moe_dtype dt, int T, int H, const int32_t* topk_idx, int k, int E,
                       void* x_perm, int32_t* counts, int32_t* offsets, int32_t* row_of_slot,
                       int32_t* slot_of_row, void* workspace, size_t workspace_bytes, hipStream_t stream);

/* moe_permute without a workspace argument, for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc). Same arguments and
 * results as moe_permute; its scratch (the expert counts per 16 tokens) is a fixed 4 MiB device array
 * inside the library, one per GPU, held until the process ends. Limit: ceil(T/16) * E <= 1048576
 * (e.g. T <= 131072 at E = 128, T <= 16384 at E = 1024), else MOE_ERR_WORKSPACE. The call allocates
 * nothing; its first call on a device looks the array's address up. Every call on one GPU shares the
 * array: calls that overlap on one GPU (concurrent streams, threads) race and must be ordered by the
 * caller.                                                                                            */
moe_status moe_permute_noalloc(const void* x, moe_dtype dt, int T, int H, const int32_t* topk_idx, int k, int E,
                               void* x_perm, int32_t* counts, int32_t* offsets, int32_t* row_of_slot,
                               int32_t* slot_of_row, hipStream_t stream);

/* (2)+(3) in one call: the selection and weights of moe_router_topk, then the layout handle (and
 * x_perm unless NULL) of moe_permute, with the same results bit for bit. For E <= 256 the top-k
 * kernel also counts the expert choices of every 16 tokens, so the permute skips its counting pass.
 * Arguments as in (2) and (3); workspace: moe_permute_workspace_bytes(T, k, E) bytes.           */
moe_status moe_router_topk_permute(const float* logits, int T, int E, int k, int renorm, int32_t* topk_idx,
                                   float* topk_w, const void* x, moe_dtype dt, int H, void* x_perm, int32_t* counts,
                                   int32_t* offsets, int32_t* row_of_slot, int32_t* slot_of_row, void* workspace,
                                   size_t workspace_bytes, hipStream_t stream);

/* ---- (4) grouped SwiGLU expert FFN -----------------------------------------------------------------
 * [MM 2, 8.3; opt. 2.1] for each expert e with rows [offsets[e], offsets[e+1]) of x_perm:
 *   g = x_perm[r] @ gate_up[e*H:(e+1)*H, 0:I],  u = x_perm[r] @ gate_up[e*H:(e+1)*H, I:2I],
 *   h[r] = silu(g) * u  (silu(z) = z / (1 + exp(-z))),   y[r] = h[r] @ down[e*I:(e+1)*I, :].
 * fp32 accumulation; in bf16, h is stored as bf16 between the two matmuls and y is rounded once.
 * Experts with no rows cost nothing. Rows outside [offsets[0], offsets[E]) are left untouched.
 *   x_perm [N, H] dt; gate_up [E*H, 2*I] dt; down [E*I, H] dt; expert_offsets [E+1] int32 (device,
 *   non-decreasing, offsets[E] <= N); h [N, I] dt (out, scratch for the caller); gu_saved [N, 2*I] dt
 *   (out, optional: the pre-activations g | u, kept for a backward pass; may be NULL); y [N, H] dt (out).
 * A shared expert is the same call with E = 1 and expert_offsets = {0, T}.                        */
moe_status moe_grouped_swiglu_ffn(const void* x_perm, const void* gate_up, const void* down, moe_dtype dt,
                                  int N, int H, int I, int E, const int32_t* expert_offsets, void* h,
                                  void* gu_saved, void* y, hipStream_t stream);

/* The two halves of moe_grouped_swiglu_ffn, same arguments and rules:
 *   moe_grouped_gemm_swiglu: the first grouped matmul with SwiGLU fused in its epilogue -> h (+ gu_saved);
 *   moe_grouped_gemm_down:   the second grouped matmul h @ down_e -> y.
 * moe_grouped_swiglu_ffn(...) == moe_grouped_gemm_swiglu(...) then moe_grouped_gemm_down(...).        */
moe_status moe_grouped_gemm_swiglu(const void* x_perm, const void* gate_up, moe_dtype dt, int N, int H, int I,
                                   int E, const int32_t* expert_offsets, void* h, void* gu_saved,
                                   hipStream_t stream);
moe_status moe_grouped_gemm_down(const void* h, const void* down, moe_dtype dt, int N, int H, int I, int E,
                                 const int32_t* expert_offsets, void* y, hipStream_t stream);

/* Gathering variants ([FT 3] fused dispatcher: the permute folded into the grouped matmul, so the
 * permuted copy of x is never written): grouped row r is token slot_of_row[r] / k of x, i.e.
 *   x_perm[r, :] = x[slot_of_row[r] / k, :]
 * and the result is bit-identical to moe_permute(x -> x_perm) followed by the calls above.
 *   x [T, H] dt; slot_of_row [>= N] int32 from moe_permute (device; entries of rows below
 *   offsets[E] must lie in [0, T*k)); other arguments as moe_grouped_swiglu_ffn. N <= T*k and
 *   T*H*sizeof(dt) < 2 GiB (MOE_ERR_UNSUPPORTED otherwise).                                        */
moe_status moe_grouped_gemm_swiglu_gather(const void* x, const int32_t* slot_of_row, int T, int k,
                                          const void* gate_up, moe_dtype dt, int N, int H, int I, int E,
                                          const int32_t* expert_offsets, void* h, void* gu_saved,
                                          hipStream_t stream);
moe_status moe_grouped_swiglu_ffn_gather(const void* x, const int32_t* slot_of_row, int T, int k,
                                         const void* gate_up, const void* down, moe_dtype dt, int N, int H,
                                         int I, int E, const int32_t* expert_offsets, void* h, void* gu_saved,
                                         void* y, hipStream_t stream);

/* ---- (5) unpermute + gate-weighted combine ---------------------------------------------------------
 * [DS Expert Parallelism] weighted sum of the expert outputs by the gate weights; [MM 8.3] unpermute.
 *   out[t] = residual[t] + sum_{j<k} topk_w[t, j] * y[row_of_slot[t*k + j]]   (fp32, j ascending,
 *   rounded once to dt; slots with row_of_slot < 0 are skipped; residual may be NULL).
 *   y [N, H] dt with N > every row_of_slot entry; topk_w [T, k] fp32; residual, out [T, H] dt.   */
moe_status moe_unpermute_combine(const void* y, moe_dtype dt, int T, int H, int k, const int32_t* row_of_slot,
                                 const float* topk_w, const void* residual, void* out, hipStream_t stream);

/* ==== backward =====================================================================================
 * Gradients of a loss L given dL/dout, for the forward above. [DS Automodel/DeepEP]: the combine is
 * the dispatch's backward and vice versa. All reductions in fp32; weight gradients are written, not
 * accumulated. */

/* ---- (6) combine backward ------------------------------------------------------------------------
 * [DS Automodel/DeepEP] the combine is the dispatch's backward: the gradient of the gate-weighted sum
 * goes back along the layout handle of the forward's dispatch to each slot's row, and the gradient of
 * the fp32 top-k weights is the row's dot product with the upstream gradient.
 *   d_y[row_of_slot[t*k+j]] = topk_w[t,j] * d_out[t]        (dt; rows without a slot are untouched)
 *   d_w[t,j] = <d_out[t], y[row_of_slot[t*k+j]]>            (fp32)
 *   d_out [T,H] dt; y [N,H] dt; row_of_slot [T*k]; topk_w [T,k] fp32; d_y [N,H] dt; d_w [T,k] fp32.  */
moe_status moe_unpermute_combine_bwd(const void* d_out, const void* y, moe_dtype dt, int T, int H, int k,
                                     const int32_t* row_of_slot, const float* topk_w, void* d_y, float* d_w,
                                     hipStream_t stream);

/* ---- (7) grouped SwiGLU FFN backward ------------------------------------------------------------------
 * [MM 2, 8.3] the transposed products of the experts' permute -> grouped_matmul -> SwiGLU ->
 * grouped_matmul path over the same fused weights; [FT 3] experts without rows get zero weight
 * gradients. For each expert e and its rows r (g, u = the forward pre-activations saved in gu_saved, s = sigmoid(g)):
 *   dh[r] = d_y[r] @ down_e^T;  dg = dh * u * s * (1 + g (1 - s));  du = dh * g * s;   d_gu[r] = dg | du
 *   d_x_perm[r] = d_gu[r] @ gate_up_e^T
 *   d_down_e    = h_e^T @ d_y_e        [I, H]   (zeros for an expert without rows)
 *   d_gate_up_e = x_perm_e^T @ d_gu_e  [H, 2I]  (zeros for an expert without rows)
 *   d_y, x_perm [N,H]; gu_saved, d_gu [N,2I] (d_gu: caller scratch, also an output); h [N,I];
 *   gate_up, d_gate_up [E*H, 2I]; down, d_down [E*I, H]; d_x_perm [N,H]. All of dtype dt.
 * A shared expert is the same call with E = 1 and expert_offsets = {0, T}.
 * fp32 and bf16 shapes outside the matrix-core kernels' (see the conventions) take the generic kernels. */
moe_status moe_grouped_swiglu_ffn_bwd(const void* d_y, const void* x_perm, const void* gu_saved, const void* h,
                                      const void* gate_up, const void* down, moe_dtype dt, int N, int H, int I, int E,
                                      const int32_t* expert_offsets, void* d_x_perm, void* d_gate_up, void* d_down,
                                      void* d_gu, hipStream_t stream);

/* ---- (7a-c) the products of (7) one at a time, for callers that put them on streams of their own ---
 * moe_grouped_swiglu_ffn_bwd(...) == 7a, 7b, then 7c for (h, d_y) -> d_down and (x_perm, d_gu) -> d_gate_up.
 *   7a  d_gu = dg | du from d_y, down and gu_saved as in (7)           (layouts as in (7))
 *   7b  d_x_perm = d_gu @ gate_up_e^T
 *   7c  d_w_e = P_e^T @ Q_e over the rows of expert e, for every expert (zeros without rows):
 *       P [N, M] and Q [N, Nq] row-major with the rows grouped by expert; d_w [E*M, Nq].
 *       max_workgroups > 0 caps the product's workgroups (rounded down to a multiple of 8, at least 8;
 *       each holds one CU until the product ends), leaving the other CUs to kernels on other streams;
 *       0 = one per CU (the generic kernels ignore it). N*max(M, Nq)*2 and M*Nq*2 below 2^31, else
 *       MOE_ERR_UNSUPPORTED. fp32, or bf16 with M or Nq not a multiple of 8 or unaligned buffers, take
 *       the generic kernels.                                                                        */
moe_status moe_grouped_gemm_down_bwd(const void* d_y, const void* down, const void* gu_saved, moe_dtype dt, int N,
                                     int H, int I, int E, const int32_t* expert_offsets, void* d_gu,
                                     hipStream_t stream);
moe_status moe_grouped_gemm_gate_up_bwd(const void* d_gu, const void* gate_up, moe_dtype dt, int N, int H, int I,
                                        int E, const int32_t* expert_offsets, void* d_x_perm, hipStream_t stream);
moe_status moe_grouped_gemm_wgrad(const void* P, const void* Q, moe_dtype dt, int N, int M, int Nq, int E,
                                  const int32_t* expert_offsets, void* d_w, int max_workgroups, hipStream_t stream);

/* ---- (8) permute backward (gather-sum of a token's k rows) ----------------------------------------
 * [DS Automodel/DeepEP] the dispatch's backward is a combine: each token's k row gradients are
 * gathered through the same layout handle and summed (unweighted).
 *   d_x[t] = d_x_add[t] + sum_{j<k} d_x_perm[row_of_slot[t*k+j]]   (fp32, rounded once; d_x_add may
 *   be NULL; slots with row_of_slot < 0 are skipped).  d_x_perm [N,H], d_x_add, d_x [T,H] dt.         */
moe_status moe_permute_bwd(const void* d_x_perm, moe_dtype dt, int T, int H, int k, const int32_t* row_of_slot,
                           const void* d_x_add, void* d_x, hipStream_t stream);

/* ---- (9) top-k / renormalisation backward ----------------------------------------------------------
 * [MM 8.2/8.3] gradient of the FP32 softmax -> top-k -> weight normalisation of (2) with respect to
 * the logits. Selection has no gradient. With w the forward weights and s = sum_j w_j d_w_j:
 *   renorm = 1:  d_logits[t, S_j] = w_j (d_w_j - s), 0 for experts outside the selection;
 *   renorm = 0:  d_logits[t, e] = p_e (1[e selected] d_w_e - s), p = softmax(logits[t]) recomputed
 *                (logits may be NULL when renorm = 1).   d_logits [T,E] fp32, every entry written.     */
moe_status moe_router_topk_bwd(const float* logits, const int32_t* topk_idx, const float* topk_w, const float* d_w,
                               int T, int E, int k, int renorm, float* d_logits, hipStream_t stream);

/* ---- (10) router logits backward -------------------------------------------------------------------
 * [MM 8.2/8.3] gradient of the gate logits = x @ w_gate of (1):
 *   d_w_gate = x^T @ d_logits   [H,E] fp32   (skipped when NULL; zeros when T = 0)
 *   d_x      = d_x_in + d_logits @ w_gate^T   [T,H] dt   (skipped when NULL; d_x_in may be NULL)
 * fp32 accumulation on the matrix cores (fp32 MFMA); d_x on the vector ALU when E is not a multiple
 * of 8 or the buffers are not 16-byte aligned.                                                       */
moe_status moe_router_logits_bwd(const void* x, const void* w_gate, const float* d_logits, moe_dtype dt, int T,
                                 int H, int E, float* d_w_gate, const void* d_x_in, void* d_x, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_ROCM_H */
