// Expert FFN products for every dtype and shape the matrix-core kernels do not take: fp32, and bf16
// with H or I not a multiple of 8 or buffers not 16-byte aligned.
//
// The products are the ones of the MindSpeed-MM InternVL3.5 practice doc (issue 625, section 8.3:
// permute -> grouped_matmul -> SwiGLU -> grouped_matmul -> unpermute) over the fused weights of its
// section 2 (gate_up [E*H, 2*I], down [E*I, H]), and their gradients. One thread per output element,
// fp32 fused multiply-adds over the contraction index in ascending order, one rounding to the
// storage type at the end (bf16: h and the gradients are stored as bf16, as on the matrix-core path).
// These kernels trade speed for generality: they read their operands straight from global memory.
#include "common.hpp"
#include "internal.hpp"

namespace moe {

constexpr int kGenThreads = 256;

// the expert whose rows [offsets[e], offsets[e+1]) contain row r, or -1
__device__ __forceinline__ int gen_expert_of_row(const int32_t* __restrict__ offsets, int E, int r) {
  if (r < offsets[0] || r >= offsets[E]) return -1;
  int lo = 0, hi = E;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (offsets[mid] <= r)
      lo = mid;
    else
      hi = mid;
  }
  return lo;
}

__device__ __forceinline__ float gen_sigmoid(float g) { return 1.0f / (1.0f + expf(-g)); }

// h[r, j] = silu(g) * u, g = A_r . W_e[:, j], u = A_r . W_e[:, I + j]; A_r = A[a_slot[r] / a_div] when
// a_slot is given (rows gathered from the token matrix), else A[r]
template <typename TE>
__global__ __launch_bounds__(kGenThreads) void gen_ffn1_kernel(const TE* __restrict__ A, const TE* __restrict__ W,
                                                               const int32_t* __restrict__ offsets, int E, int N, int K,
                                                               int I, TE* __restrict__ h, TE* __restrict__ gu_saved,
                                                               const int32_t* __restrict__ a_slot, int a_div) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (int64_t)N * I) return;
  const int r = (int)(gid / I), j = (int)(gid % I);
  const int e = gen_expert_of_row(offsets, E, r);
  if (e < 0) return;
  const int64_t a0 = (int64_t)(a_slot ? a_slot[r] / a_div : r) * K;
  const int64_t w0 = (int64_t)e * K * 2 * I;
  float g = 0.0f, u = 0.0f;
  for (int k = 0; k < K; ++k) {
    const float a = Elem<TE>::load(A, a0 + k);
    g = __builtin_fmaf(a, Elem<TE>::load(W, w0 + (int64_t)k * 2 * I + j), g);
    u = __builtin_fmaf(a, Elem<TE>::load(W, w0 + (int64_t)k * 2 * I + I + j), u);
  }
  Elem<TE>::store(h, (int64_t)r * I + j, g * gen_sigmoid(g) * u);
  if (gu_saved) {
    Elem<TE>::store(gu_saved, (int64_t)r * 2 * I + j, g);
    Elem<TE>::store(gu_saved, (int64_t)r * 2 * I + I + j, u);
  }
}

// y[r, c] = h_r . D_e[:, c]
template <typename TE>
__global__ __launch_bounds__(kGenThreads) void gen_ffn2_kernel(const TE* __restrict__ Hh, const TE* __restrict__ D,
                                                               const int32_t* __restrict__ offsets, int E, int N, int I,
                                                               int H, TE* __restrict__ y) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (int64_t)N * H) return;
  const int r = (int)(gid / H), c = (int)(gid % H);
  const int e = gen_expert_of_row(offsets, E, r);
  if (e < 0) return;
  const int64_t a0 = (int64_t)r * I, d0 = (int64_t)e * I * H;
  float acc = 0.0f;
  for (int i = 0; i < I; ++i) acc = __builtin_fmaf(Elem<TE>::load(Hh, a0 + i), Elem<TE>::load(D, d0 + (int64_t)i * H + c), acc);
  Elem<TE>::store(y, (int64_t)r * H + c, acc);
}

// d_gu[r, j] = dh * u * s * (1 + g (1 - s)), d_gu[r, I + j] = dh * g * s with dh = dY_r . D_e[j, :],
// s = sigmoid(g), (g, u) = gu_saved[r, j], gu_saved[r, I + j]: the derivatives of silu(g) * u
template <typename TE>
__global__ __launch_bounds__(kGenThreads) void gen_down_bwd_kernel(const TE* __restrict__ d_y, const TE* __restrict__ D,
                                                                   const TE* __restrict__ gu, const int32_t* __restrict__ offsets,
                                                                   int E, int N, int H, int I, TE* __restrict__ d_gu) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (int64_t)N * I) return;
  const int r = (int)(gid / I), j = (int)(gid % I);
  const int e = gen_expert_of_row(offsets, E, r);
  if (e < 0) return;
  const int64_t y0 = (int64_t)r * H, d0 = ((int64_t)e * I + j) * H;
  float dh = 0.0f;
  for (int c = 0; c < H; ++c) dh = __builtin_fmaf(Elem<TE>::load(d_y, y0 + c), Elem<TE>::load(D, d0 + c), dh);
  const float g = Elem<TE>::load(gu, (int64_t)r * 2 * I + j), u = Elem<TE>::load(gu, (int64_t)r * 2 * I + I + j);
  const float s = gen_sigmoid(g);
  Elem<TE>::store(d_gu, (int64_t)r * 2 * I + j, dh * u * s * (1.0f + g * (1.0f - s)));
  Elem<TE>::store(d_gu, (int64_t)r * 2 * I + I + j, dh * g * s);
}

// d_x[r, c] = d_gu_r . GU_e[c, :] (over the 2I gate and up columns)
template <typename TE>
__global__ __launch_bounds__(kGenThreads) void gen_gate_up_bwd_kernel(const TE* __restrict__ d_gu,
                                                                      const TE* __restrict__ GU,
                                                                      const int32_t* __restrict__ offsets, int E, int N,
                                                                      int H, int I, TE* __restrict__ d_x) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (int64_t)N * H) return;
  const int r = (int)(gid / H), c = (int)(gid % H);
  const int e = gen_expert_of_row(offsets, E, r);
  if (e < 0) return;
  const int64_t g0 = (int64_t)r * 2 * I, w0 = ((int64_t)e * H + c) * 2 * I;
  float acc = 0.0f;
  for (int j = 0; j < 2 * I; ++j) acc = __builtin_fmaf(Elem<TE>::load(d_gu, g0 + j), Elem<TE>::load(GU, w0 + j), acc);
  Elem<TE>::store(d_x, (int64_t)r * H + c, acc);
}

// d_w[e, m, n] = sum over the rows r of expert e (ascending) of P[r, m] * Q[r, n]; zero without rows
template <typename TE>
__global__ __launch_bounds__(kGenThreads) void gen_wgrad_kernel(const TE* __restrict__ P, const TE* __restrict__ Q,
                                                                const int32_t* __restrict__ offsets, int E, int M, int Nq,
                                                                TE* __restrict__ d_w) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t per = (int64_t)M * Nq;
  if (gid >= (int64_t)E * per) return;
  const int e = (int)(gid / per);
  const int m = (int)((gid % per) / Nq), n = (int)(gid % Nq);
  float acc = 0.0f;
  for (int r = offsets[e]; r < offsets[e + 1]; ++r)
    acc = __builtin_fmaf(Elem<TE>::load(P, (int64_t)r * M + m), Elem<TE>::load(Q, (int64_t)r * Nq + n), acc);
  Elem<TE>::store(d_w, gid, acc);
}

namespace {
inline dim3 gen_grid(int64_t n) { return dim3((unsigned)((n + kGenThreads - 1) / kGenThreads)); }
}  // namespace

hipError_t launch_gen_ffn1(const void* A, const void* W, int dt, const int32_t* offsets, int E, int N, int H, int I,
                           void* h, void* gu_saved, const int32_t* a_slot, int a_div, hipStream_t s) {
  const int64_t n = (int64_t)N * I;
  if (n == 0) return hipSuccess;
  if (dt == kF32)
    hipLaunchKernelGGL(gen_ffn1_kernel<float>, gen_grid(n), dim3(kGenThreads), 0, s, (const float*)A, (const float*)W,
                       offsets, E, N, H, I, (float*)h, (float*)gu_saved, a_slot, a_div);
  else
    hipLaunchKernelGGL(gen_ffn1_kernel<uint16_t>, gen_grid(n), dim3(kGenThreads), 0, s, (const uint16_t*)A,
                       (const uint16_t*)W, offsets, E, N, H, I, (uint16_t*)h, (uint16_t*)gu_saved, a_slot, a_div);
  return hipGetLastError();
}

hipError_t launch_gen_ffn2(const void* Hh, const void* D, int dt, const int32_t* offsets, int E, int N, int H, int I,
                           void* y, hipStream_t s) {
  const int64_t n = (int64_t)N * H;
  if (n == 0) return hipSuccess;
  if (dt == kF32)
    hipLaunchKernelGGL(gen_ffn2_kernel<float>, gen_grid(n), dim3(kGenThreads), 0, s, (const float*)Hh, (const float*)D,
                       offsets, E, N, I, H, (float*)y);
  else
    hipLaunchKernelGGL(gen_ffn2_kernel<uint16_t>, gen_grid(n), dim3(kGenThreads), 0, s, (const uint16_t*)Hh,
                       (const uint16_t*)D, offsets, E, N, I, H, (uint16_t*)y);
  return hipGetLastError();
}

hipError_t launch_gen_down_bwd(const void* d_y, const void* down, const void* gu_saved, int dt, int N, int H, int I,
                               int E, const int32_t* offsets, void* d_gu, hipStream_t s) {
  const int64_t n = (int64_t)N * I;
  if (n == 0) return hipSuccess;
  if (dt == kF32)
    hipLaunchKernelGGL(gen_down_bwd_kernel<float>, gen_grid(n), dim3(kGenThreads), 0, s, (const float*)d_y,
                       (const float*)down, (const float*)gu_saved, offsets, E, N, H, I, (float*)d_gu);
  else
    hipLaunchKernelGGL(gen_down_bwd_kernel<uint16_t>, gen_grid(n), dim3(kGenThreads), 0, s, (const uint16_t*)d_y,
                       (const uint16_t*)down, (const uint16_t*)gu_saved, offsets, E, N, H, I, (uint16_t*)d_gu);
  return hipGetLastError();
}

hipError_t launch_gen_gate_up_bwd(const void* d_gu, const void* gate_up, int dt, int N, int H, int I, int E,
                                  const int32_t* offsets, void* d_x, hipStream_t s) {
  const int64_t n = (int64_t)N * H;
  if (n == 0) return hipSuccess;
  if (dt == kF32)
    hipLaunchKernelGGL(gen_gate_up_bwd_kernel<float>, gen_grid(n), dim3(kGenThreads), 0, s, (const float*)d_gu,
                       (const float*)gate_up, offsets, E, N, H, I, (float*)d_x);
  else
    hipLaunchKernelGGL(gen_gate_up_bwd_kernel<uint16_t>, gen_grid(n), dim3(kGenThreads), 0, s, (const uint16_t*)d_gu,
                       (const uint16_t*)gate_up, offsets, E, N, H, I, (uint16_t*)d_x);
  return hipGetLastError();
}

hipError_t launch_gen_wgrad(const void* P, const void* Q, int dt, int M, int Nq, int E, const int32_t* offsets,
                            void* d_w, hipStream_t s) {
  const int64_t n = (int64_t)E * M * Nq;
  if (n == 0) return hipSuccess;
  if (dt == kF32)
    hipLaunchKernelGGL(gen_wgrad_kernel<float>, gen_grid(n), dim3(kGenThreads), 0, s, (const float*)P, (const float*)Q,
                       offsets, E, M, Nq, (float*)d_w);
  else
    hipLaunchKernelGGL(gen_wgrad_kernel<uint16_t>, gen_grid(n), dim3(kGenThreads), 0, s, (const uint16_t*)P,
                       (const uint16_t*)Q, offsets, E, M, Nq, (uint16_t*)d_w);
  return hipGetLastError();
}

}  // namespace moe
