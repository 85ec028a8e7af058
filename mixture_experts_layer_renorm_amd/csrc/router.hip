// Router: gate logits, then softmax -> top-k -> renormalised weights.
//
// The MoE block of the MindSpeed-MM InternVL3.5 practice doc (issue 625, sections 8.2 and 8.3)
// routes each token with gate -> FP32 softmax -> top-k -> weight normalisation. The logits are an
// fp32 fused-multiply-add chain over the hidden dimension in ascending order, so that the top-k
// decision is reproducible bit for bit by a sequential CPU implementation. Selection works on the
// logits (softmax is monotone); ties go to the lower expert index.
#include "common.hpp"
#include "internal.hpp"

namespace moe {

// ---------------------------------------------------------------------------------------------
// logits[t, e] = fp32 chain over h = 0..H-1 of fma(x[t,h], w_gate[h,e], acc).
// Lanes map to experts (64 per wave); each wave owns kTokPerWave consecutive tokens, whose x
// values are wave-uniform (scalar loads); blockIdx.y selects the block of 64 experts.
constexpr int kTokPerWave = 8;
constexpr int kLogitWaves = 4;

template <typename TIn>
__global__ __launch_bounds__(kLogitWaves * kWave) void router_logits_kernel(
    const TIn* __restrict__ x, const TIn* __restrict__ wg, int T, int H, int E,
    float* __restrict__ logits) {
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int e = blockIdx.y * kWave + lane;
  const int t0 = (blockIdx.x * kLogitWaves + wave) * kTokPerWave;
  if (t0 >= T) return;
  const int nt = min(kTokPerWave, T - t0);
  const int ec = e < E ? e : E - 1;
  const TIn* xr[kTokPerWave];
#pragma unroll
  for (int i = 0; i < kTokPerWave; ++i) xr[i] = x + (int64_t)(t0 + (i < nt ? i : nt - 1)) * H;
  const TIn* wcol = wg + ec;
  float acc[kTokPerWave];
#pragma unroll
  for (int i = 0; i < kTokPerWave; ++i) acc[i] = 0.0f;
  for (int h = 0; h < H; ++h) {
    const float w = Elem<TIn>::load(wcol, (int64_t)h * E);
#pragma unroll
    for (int i = 0; i < kTokPerWave; ++i) acc[i] = __builtin_fmaf(Elem<TIn>::load(xr[i], h), w, acc[i]);
  }
  if (e < E) {
#pragma unroll
    for (int i = 0; i < kTokPerWave; ++i)
      if (i < nt) logits[(int64_t)(t0 + i) * E + e] = acc[i];
  }
}

// ---------------------------------------------------------------------------------------------
// One wave per token. k rounds of a wave-wide argmax over the still-available experts; lane j
// keeps the round-j winner. Weights: exp(l_j - max) over the selected set (renorm) or over all
// experts (raw softmax probability).
constexpr int kTopkWaves = 4;

template <int VPL>
__global__ __launch_bounds__(kTopkWaves * kWave) void router_topk_kernel(
    const float* __restrict__ logits, int T, int E, int k, int renorm, int32_t* __restrict__ topk_idx,
    float* __restrict__ topk_w) {
  const int lane = lane_id();
  const int t = blockIdx.x * kTopkWaves + (int)(threadIdx.x / kWave);
  if (t >= T) return;
  const float* l = logits + (int64_t)t * E;
  float v[VPL];
  uint32_t avail = 0;
#pragma unroll
  for (int q = 0; q < VPL; ++q) {
    const int e = q * kWave + lane;
    v[q] = e < E ? l[e] : 0.0f;
    if (e < E) avail |= 1u << q;
  }
  float my_v = 0.0f;
  int my_e = -1;
  for (int j = 0; j < k; ++j) {
    float bv = 0.0f;
    int be = 0x7fffffff;
#pragma unroll
    for (int q = 0; q < VPL; ++q) {
      const int e = q * kWave + lane;
      if ((avail >> q) & 1u) {
        if (be == 0x7fffffff || v[q] > bv) {  // ascending e per lane: strict > keeps lower index on ties
          bv = v[q];
          be = e;
        }
      }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      const float ov = __shfl_xor(bv, off, kWave);
      const int oe = __shfl_xor(be, off, kWave);
      const bool take = (oe != 0x7fffffff) && (be == 0x7fffffff || ov > bv || (ov == bv && oe < be));
      if (take) {
        bv = ov;
        be = oe;
      }
    }
    if (lane == j) {
      my_v = bv;
      my_e = be;
    }
    if ((be & (kWave - 1)) == lane) avail &= ~(1u << (be / kWave));
  }
  const float m = __shfl(my_v, 0, kWave);
  float ex = lane < k ? expf(my_v - m) : 0.0f;
  float den;
  if (renorm) {
    den = wave_sum(ex);
  } else {
    float s = 0.0f;
#pragma unroll
    for (int q = 0; q < VPL; ++q) {
      const int e = q * kWave + lane;
      if (e < E) s += expf(v[q] - m);
    }
    den = wave_sum(s);
  }
  if (lane < k) {
    topk_idx[(int64_t)t * k + lane] = my_e;
    topk_w[(int64_t)t * k + lane] = ex / den;
  }
}

// ---------------------------------------------------------------------------------------------
hipError_t launch_router_logits(const void* x, const void* w_gate, int dt, int T, int H, int E, float* logits,
                                hipStream_t s) {
  dim3 grid((T + kLogitWaves * kTokPerWave - 1) / (kLogitWaves * kTokPerWave), (E + kWave - 1) / kWave);
  dim3 block(kLogitWaves * kWave);
  if (dt == kF32)
    hipLaunchKernelGGL(router_logits_kernel<float>, grid, block, 0, s, (const float*)x, (const float*)w_gate, T, H,
                       E, logits);
  else
    hipLaunchKernelGGL(router_logits_kernel<uint16_t>, grid, block, 0, s, (const uint16_t*)x,
                       (const uint16_t*)w_gate, T, H, E, logits);
  return hipGetLastError();
}

hipError_t launch_router_topk(const float* logits, int T, int E, int k, int renorm, int32_t* idx, float* w,
                              hipStream_t s) {
  dim3 grid((T + kTopkWaves - 1) / kTopkWaves), block(kTopkWaves * kWave);
  const int vpl = (E + kWave - 1) / kWave;
#define MOE_TOPK_CASE(V)                                                                                  \
  case V:                                                                                                 \
    hipLaunchKernelGGL(router_topk_kernel<V>, grid, block, 0, s, logits, T, E, k, renorm, idx, w); \
    break;
  switch (vpl) {
    MOE_TOPK_CASE(1)
    MOE_TOPK_CASE(2)
    MOE_TOPK_CASE(4)
    MOE_TOPK_CASE(8)
    MOE_TOPK_CASE(16)
    case 3:
      hipLaunchKernelGGL(router_topk_kernel<4>, grid, block, 0, s, logits, T, E, k, renorm, idx, w);
      break;
    default:
      if (vpl <= 8)
        hipLaunchKernelGGL(router_topk_kernel<8>, grid, block, 0, s, logits, T, E, k, renorm, idx, w);
      else
        hipLaunchKernelGGL(router_topk_kernel<16>, grid, block, 0, s, logits, T, E, k, renorm, idx, w);
  }
#undef MOE_TOPK_CASE
  return hipGetLastError();
}

}  // namespace moe
