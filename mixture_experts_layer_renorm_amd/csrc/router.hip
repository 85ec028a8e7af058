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
//
// A workgroup (4 waves) owns 16 tokens x 64*EQ experts; each lane owns 4 tokens x EQ adjacent
// experts, i.e. 4*EQ independent chains. The hidden dimension is walked in chunks of HB: the
// chunk's x tile [16 x HB] and W_g tile [HB x 64*EQ] are loaded cooperatively (16-byte loads when
// the rows allow), widened to fp32 once, and staged in LDS (double buffered, the next chunk's
// global loads in flight during this chunk's FMAs). Within a lane, every chain still consumes
// h = 0, 1, ..., H-1 in order.
constexpr int kLogitWaves = 4;
constexpr int kTokPerWave = 4;
constexpr int kTokPerBlock = kLogitWaves * kTokPerWave;

template <typename TIn, int EQ>
struct LogitTile {
  static constexpr int EB = kWave * EQ;              // experts per workgroup
  static constexpr int HB = EQ >= 4 ? 32 : 64;       // hidden chunk
  static constexpr int VEC = 16 / sizeof(TIn);       // elements per 16-byte load
  static constexpr int XCH = kTokPerBlock * HB / VEC;  // 16-byte chunks of the x tile
  static constexpr int WCH = HB * EB / VEC;            // 16-byte chunks of the W tile
  static constexpr int XPT = (XCH + 255) / 256;        // per thread
  static constexpr int WPT = (WCH + 255) / 256;
};

template <typename TIn>
__device__ __forceinline__ void widen(const uint4& v, float* f);
template <>
__device__ __forceinline__ void widen<uint16_t>(const uint4& v, float* f) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(w[i] << 16);
    f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}
template <>
__device__ __forceinline__ void widen<float>(const uint4& v, float* f) {
  f[0] = __uint_as_float(v.x);
  f[1] = __uint_as_float(v.y);
  f[2] = __uint_as_float(v.z);
  f[3] = __uint_as_float(v.w);
}

// 16 bytes (VEC elements) of row `row` from column `col`; columns >= ncols read as zero.
template <typename TIn>
__device__ __forceinline__ uint4 load_chunk(const TIn* __restrict__ row, int col, int ncols, bool vec) {
  constexpr int VEC = 16 / sizeof(TIn);
  if (vec && col + VEC <= ncols) return *reinterpret_cast<const uint4*>(row + col);
  TIn tmp[VEC];
#pragma unroll
  for (int i = 0; i < VEC; ++i) tmp[i] = col + i < ncols ? row[col + i] : TIn(0);
  uint4 v;
  __builtin_memcpy(&v, tmp, 16);
  return v;
}

template <typename TIn, int EQ>
__global__ __launch_bounds__(kLogitWaves * kWave) void router_logits_kernel(
    const TIn* __restrict__ x, const TIn* __restrict__ wg, int T, int H, int E, float* __restrict__ logits, int vec_x,
    int vec_w) {
  using P = LogitTile<TIn, EQ>;
  constexpr int EB = P::EB, HB = P::HB, VEC = P::VEC;
  __shared__ __attribute__((aligned(16))) float xs[2][kTokPerBlock][HB];
  __shared__ __attribute__((aligned(16))) float ws[2][HB][EB];
  const int tid = threadIdx.x, lane = lane_id(), wave = tid / kWave;
  const int t0 = blockIdx.x * kTokPerBlock;
  const int e0 = blockIdx.y * EB;
  const int nh_chunks = (H + HB - 1) / HB;

  uint4 rx[P::XPT], rw[P::WPT];
  auto load = [&](int hc) {
    const int h0 = hc * HB;
#pragma unroll
    for (int i = 0; i < P::XPT; ++i) {
      const int c = tid + 256 * i;
      if (c < P::XCH) {
        const int tt = c / (HB / VEC), hh = (c % (HB / VEC)) * VEC;
        const int t = min(t0 + tt, T - 1);
        rx[i] = load_chunk<TIn>(x + (int64_t)t * H, h0 + hh, H, vec_x);
      }
    }
#pragma unroll
    for (int i = 0; i < P::WPT; ++i) {
      const int c = tid + 256 * i;
      if (c < P::WCH) {
        const int hh = c / (EB / VEC), ee = (c % (EB / VEC)) * VEC;
        const int h = min(h0 + hh, H - 1);
        rw[i] = load_chunk<TIn>(wg + (int64_t)h * E, e0 + ee, E, vec_w);
      }
    }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int i = 0; i < P::XPT; ++i) {
      const int c = tid + 256 * i;
      if (c < P::XCH) {
        const int tt = c / (HB / VEC), hh = (c % (HB / VEC)) * VEC;
        float f[VEC];
        widen<TIn>(rx[i], f);
#pragma unroll
        for (int q = 0; q < VEC; q += 4)
          *reinterpret_cast<float4*>(&xs[buf][tt][hh + q]) = make_float4(f[q], f[q + 1], f[q + 2], f[q + 3]);
      }
    }
#pragma unroll
    for (int i = 0; i < P::WPT; ++i) {
      const int c = tid + 256 * i;
      if (c < P::WCH) {
        const int hh = c / (EB / VEC), ee = (c % (EB / VEC)) * VEC;
        float f[VEC];
        widen<TIn>(rw[i], f);
#pragma unroll
        for (int q = 0; q < VEC; q += 4)
          *reinterpret_cast<float4*>(&ws[buf][hh][ee + q]) = make_float4(f[q], f[q + 1], f[q + 2], f[q + 3]);
      }
    }
  };

  float acc[kTokPerWave][EQ];
#pragma unroll
  for (int i = 0; i < kTokPerWave; ++i)
#pragma unroll
    for (int q = 0; q < EQ; ++q) acc[i][q] = 0.0f;

  load(0);
  store(0);
  __syncthreads();
  for (int hc = 0; hc < nh_chunks; ++hc) {
    const int buf = hc & 1;
    if (hc + 1 < nh_chunks) load(hc + 1);
    const int nh = min(HB, H - hc * HB);
    const float* xw = &xs[buf][wave * kTokPerWave][0];
    const float* wl = &ws[buf][0][lane * EQ];
    // four h at a time: one broadcast float4 of x per token, EQ weights per lane per h
    auto quad = [&](int hh) {
      float4 xv[kTokPerWave];
#pragma unroll
      for (int i = 0; i < kTokPerWave; ++i) xv[i] = *reinterpret_cast<const float4*>(xw + i * HB + hh);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        float wv[EQ];
#pragma unroll
        for (int q = 0; q < EQ; ++q) wv[q] = wl[(hh + u) * EB + q];
#pragma unroll
        for (int i = 0; i < kTokPerWave; ++i) {
          const float xe = u == 0 ? xv[i].x : u == 1 ? xv[i].y : u == 2 ? xv[i].z : xv[i].w;
#pragma unroll
          for (int q = 0; q < EQ; ++q) acc[i][q] = __builtin_fmaf(xe, wv[q], acc[i][q]);
        }
      }
    };
    int hh = 0;
    if (nh == HB) {
      // full chunk: unrolled so that the next reads are issued under the current FMAs
#pragma unroll
      for (int h4 = 0; h4 < HB; h4 += 4) quad(h4);
      hh = HB;
    } else {
      for (; hh + 4 <= nh; hh += 4) quad(hh);
    }
    for (; hh < nh; ++hh) {
#pragma unroll
      for (int i = 0; i < kTokPerWave; ++i) {
        const float xe = xw[i * HB + hh];
#pragma unroll
        for (int q = 0; q < EQ; ++q) acc[i][q] = __builtin_fmaf(xe, wl[hh * EB + q], acc[i][q]);
      }
    }
    if (hc + 1 < nh_chunks) store(buf ^ 1);
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < kTokPerWave; ++i) {
    const int t = t0 + wave * kTokPerWave + i;
    if (t >= T) continue;
#pragma unroll
    for (int q = 0; q < EQ; ++q) {
      const int e = e0 + lane * EQ + q;
      if (e < E) logits[(int64_t)t * E + e] = acc[i][q];
    }
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
template <typename TIn, int EQ>
static void launch_logits_t(const void* x, const void* w_gate, int T, int H, int E, float* logits, hipStream_t s) {
  constexpr int EB = kWave * EQ;
  const bool vec_x = H % (16 / sizeof(TIn)) == 0 && ((uintptr_t)x & 15) == 0;
  const bool vec_w = E % (16 / sizeof(TIn)) == 0 && ((uintptr_t)w_gate & 15) == 0;
  dim3 grid((T + kTokPerBlock - 1) / kTokPerBlock, (E + EB - 1) / EB);
  hipLaunchKernelGGL((router_logits_kernel<TIn, EQ>), grid, dim3(kLogitWaves * kWave), 0, s, (const TIn*)x,
                     (const TIn*)w_gate, T, H, E, logits, (int)vec_x, (int)vec_w);
}

template <typename TIn>
static void launch_logits_dt(const void* x, const void* w_gate, int T, int H, int E, float* logits, hipStream_t s) {
  if (E <= 64)
    launch_logits_t<TIn, 1>(x, w_gate, T, H, E, logits, s);
  else if (E <= 128)
    launch_logits_t<TIn, 2>(x, w_gate, T, H, E, logits, s);
  else
    launch_logits_t<TIn, 4>(x, w_gate, T, H, E, logits, s);
}

hipError_t launch_router_logits(const void* x, const void* w_gate, int dt, int T, int H, int E, float* logits,
                                hipStream_t s) {
  if (dt == kF32)
    launch_logits_dt<float>(x, w_gate, T, H, E, logits, s);
  else
    launch_logits_dt<uint16_t>(x, w_gate, T, H, E, logits, s);
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
