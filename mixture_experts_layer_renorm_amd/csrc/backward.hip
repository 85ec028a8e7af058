// Backward pass of the MoE layer (everything except the grouped GEMMs).
//
// The forward is router -> permute -> grouped SwiGLU FFN -> unpermute/combine (MindSpeed-MM
// InternVL3.5 practice doc, issue 625, section 8.3), with the router renormalising the top-k
// softmax weights (same doc, section 8.2). The "DeepSeek MoE: EP and FSDP" guide (gsyq.cn,
// Automodel/DeepEP section) notes that the combine is the dispatch's backward and vice versa; here:
//   combine backward : dY[row(t,j)] = w[t,j] * dOut[t],   dw[t,j] = <dOut[t], y[row(t,j)]>
//   permute backward : dX[t] = dX_add[t] + sum_j dX_perm[row(t,j)]
//   top-k backward   : renorm: dl[t,S_i] = w_i (dw_i - sum_j w_j dw_j), 0 off the selected set;
//                      raw softmax: dl[t,e] = p_e (1[e in S] dw_e - sum_j w_j dw_j)
//   logits backward  : dW_g = x^T dl,   dX_router = dl W_g^T (+ an incoming dX)
// All reductions accumulate in fp32; nothing uses floating-point atomics.
#include "common.hpp"
#include "internal.hpp"

namespace moe {

constexpr int kBwdWaves = 4;

template <typename T>
__device__ __forceinline__ void load8(const T* p, float* f);
template <>
__device__ __forceinline__ void load8<uint16_t>(const uint16_t* p, float* f) {
  const uint4 v = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(w[i] << 16);
    f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}
template <>
__device__ __forceinline__ void load8<float>(const float* p, float* f) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
  f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
}
template <typename T>
__device__ __forceinline__ void store8(T* p, const float* f);
template <>
__device__ __forceinline__ void store8<uint16_t>(uint16_t* p, const float* f) {
  *reinterpret_cast<uint4*>(p) =
      make_uint4(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]), pack_bf16x2(f[6], f[7]));
}
template <>
__device__ __forceinline__ void store8<float>(float* p, const float* f) {
  *reinterpret_cast<float4*>(p) = make_float4(f[0], f[1], f[2], f[3]);
  *reinterpret_cast<float4*>(p + 4) = make_float4(f[4], f[5], f[6], f[7]);
}

// ---------------------------------------------------------------------------------------------
// combine backward: one wave per token; lane owns 8 consecutive features per 512-wide chunk.
// VEC: 8-element vector path (H % 8 == 0 and aligned) or one element at a time.
template <typename TE, bool VEC>
__global__ __launch_bounds__(kBwdWaves * kWave) void combine_bwd_kernel(
    const TE* __restrict__ d_out, const TE* __restrict__ y, int T, int H, int k, const int32_t* __restrict__ row_of_slot,
    const float* __restrict__ topk_w, TE* __restrict__ d_y, float* __restrict__ d_w) {
  const int lane = lane_id();
  const int t = blockIdx.x * kBwdWaves + (int)(threadIdx.x / kWave);
  if (t >= T) return;
  const int my_row = lane < k ? row_of_slot[(int64_t)t * k + lane] : -1;
  const float my_w = lane < k ? topk_w[(int64_t)t * k + lane] : 0.0f;
  float dot[32];  // k <= 32: per-slot partial dot products of this lane
#pragma unroll
  for (int j = 0; j < 32; ++j) dot[j] = 0.0f;
  const TE* go = d_out + (int64_t)t * H;
  constexpr int W = VEC ? 8 : 1;
  // every lane runs every iteration (lanes past H only skip their memory accesses), so the
  // shuffles below always read from active lanes, however few features a lane row covers
  for (int base = 0; base < H; base += kWave * W) {
    const int c0 = base + lane * W;
    const bool act = c0 < H;
    float g[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) g[i] = 0.0f;
    if (act) {
      if (VEC) load8<TE>(go + c0, g);
      else g[0] = Elem<TE>::load(go, c0);
    }
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      if (j >= k) break;
      const int r = __shfl(my_row, j, kWave);
      const float w = __shfl(my_w, j, kWave);
      if (r < 0 || !act) continue;
      float yv[8], dy[8];
      if (VEC) load8<TE>(y + (int64_t)r * H + c0, yv);
      else yv[0] = Elem<TE>::load(y, (int64_t)r * H + c0);
#pragma unroll
      for (int i = 0; i < W; ++i) {
        dot[j] = __builtin_fmaf(g[i], yv[i], dot[j]);
        dy[i] = w * g[i];
      }
      if (VEC) store8<TE>(d_y + (int64_t)r * H + c0, dy);
      else Elem<TE>::store(d_y, (int64_t)r * H + c0, dy[0]);
    }
  }
#pragma unroll
  for (int j = 0; j < 32; ++j) {
    if (j >= k) break;
    const float s = wave_sum(dot[j]);
    if (lane == 0) d_w[(int64_t)t * k + j] = s;
  }
}

// permute backward: one wave per token, fp32 accumulation, rounded once.
template <typename TE, bool VEC>
__global__ __launch_bounds__(kBwdWaves * kWave) void permute_bwd_kernel(
    const TE* __restrict__ d_x_perm, int T, int H, int k, const int32_t* __restrict__ row_of_slot,
    const TE* __restrict__ d_x_add, TE* __restrict__ d_x) {
  const int lane = lane_id();
  const int t = blockIdx.x * kBwdWaves + (int)(threadIdx.x / kWave);
  if (t >= T) return;
  const int my_row = lane < k ? row_of_slot[(int64_t)t * k + lane] : -1;
  constexpr int W = VEC ? 8 : 1;
  for (int base = 0; base < H; base += kWave * W) {   // uniform trip count: the shuffles read active lanes
    const int c0 = base + lane * W;
    const bool act = c0 < H;
    float acc[8];
    if (d_x_add && act) {
      if (VEC) load8<TE>(d_x_add + (int64_t)t * H + c0, acc);
      else acc[0] = Elem<TE>::load(d_x_add, (int64_t)t * H + c0);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
    }
    for (int j = 0; j < k; ++j) {
      const int r = __shfl(my_row, j, kWave);
      if (r < 0 || !act) continue;
      float v[8];
      if (VEC) load8<TE>(d_x_perm + (int64_t)r * H + c0, v);
      else v[0] = Elem<TE>::load(d_x_perm, (int64_t)r * H + c0);
#pragma unroll
      for (int i = 0; i < W; ++i) acc[i] += v[i];
    }
    if (!act) continue;
    if (VEC) store8<TE>(d_x + (int64_t)t * H + c0, acc);
    else Elem<TE>::store(d_x, (int64_t)t * H + c0, acc[0]);
  }
}

// top-k backward: one wave per token; writes the whole logits-gradient row.
template <int VPL>
__global__ __launch_bounds__(kBwdWaves * kWave) void router_topk_bwd_kernel(
    const float* __restrict__ logits, const int32_t* __restrict__ topk_idx, const float* __restrict__ topk_w,
    const float* __restrict__ d_w, int T, int E, int k, int renorm, float* __restrict__ d_logits) {
  const int lane = lane_id();
  const int t = blockIdx.x * kBwdWaves + (int)(threadIdx.x / kWave);
  if (t >= T) return;
  const int my_e = lane < k ? topk_idx[(int64_t)t * k + lane] : -1;
  const float my_w = lane < k ? topk_w[(int64_t)t * k + lane] : 0.0f;
  const float my_dw = lane < k ? d_w[(int64_t)t * k + lane] : 0.0f;
  const float s = wave_sum(my_w * my_dw);  // sum_j w_j dw_j
  float* dl = d_logits + (int64_t)t * E;
  if (renorm) {
#pragma unroll
    for (int q = 0; q < VPL; ++q) {
      const int e = q * kWave + lane;
      if (e < E) dl[e] = 0.0f;
    }
    // the selected entries overwrite their zeros; the same lane wrote both, so program order holds
#pragma unroll
    for (int q = 0; q < VPL; ++q) {
      const int e = q * kWave + lane;
      float v = 0.0f;
      bool sel = false;
      for (int j = 0; j < k; ++j) {
        const int ej = __shfl(my_e, j, kWave);
        const float wj = __shfl(my_w, j, kWave);
        const float dwj = __shfl(my_dw, j, kWave);
        if (ej == e) {
          v = wj * (dwj - s);
          sel = true;
        }
      }
      if (e < E && sel) dl[e] = v;
    }
  } else {
    const float* l = logits + (int64_t)t * E;
    float lv[VPL];
    float m = -INFINITY;
#pragma unroll
    for (int q = 0; q < VPL; ++q) {
      const int e = q * kWave + lane;
      lv[q] = e < E ? l[e] : -INFINITY;
      m = fmaxf(m, lv[q]);
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, kWave));
    float z = 0.0f;
#pragma unroll
    for (int q = 0; q < VPL; ++q) {
      const int e = q * kWave + lane;
      if (e < E) z += expf(lv[q] - m);
    }
    z = wave_sum(z);
#pragma unroll
    for (int q = 0; q < VPL; ++q) {
      const int e = q * kWave + lane;
      float dsel = 0.0f;
      for (int j = 0; j < k; ++j) {  // every lane takes part in the shuffles
        const int ej = __shfl(my_e, j, kWave);
        const float dwj = __shfl(my_dw, j, kWave);
        if (ej == e) dsel = dwj;
      }
      if (e < E) dl[e] = expf(lv[q] - m) / z * (dsel - s);
    }
  }
}

// ---------------------------------------------------------------------------------------------
// Small fp32-accumulating products of the router backward, C[M,N] = sum_k A(m,k) B(k,n):
//   dW_g [H,E]   = x^T dl :  A(h,t) = x[t,h],  B(t,e) = dl[t,e]
//   dX   [T,H]   = dl W_g^T:  A(t,e) = dl[t,e], B(e,h) = W_g[h,e]   (+ incoming dX)
// A 64 x 64 tile per workgroup, 4 x 4 outputs per thread, K staged in LDS 16 at a time as fp32.
template <typename TA, typename TB, typename TC>
struct SmallGemm {
  const TA* a;
  int64_t a_m, a_k;  // element (m,k) at a[m * a_m + k * a_k]
  const TB* b;
  int64_t b_k, b_n;
  TC* c;
  const TC* c_add;  // optional, same layout as c
  int M, N, K;
};

template <typename TA, typename TB, typename TC>
__global__ __launch_bounds__(256) void small_gemm_kernel(const SmallGemm<TA, TB, TC> p) {
  __shared__ float as[16][64 + 1];
  __shared__ float bs[16][64 + 1];
  const int tid = threadIdx.x;
  const int m0 = blockIdx.y * 64, n0 = blockIdx.x * 64;
  const int tm = (tid >> 4) * 4, tn = (tid & 15) * 4;
  float acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.0f;
  for (int k0 = 0; k0 < p.K; k0 += 16) {
    // consecutive threads walk whichever index is contiguous in memory
    for (int i = tid; i < 16 * 64; i += 256) {
      const int kk = p.a_k == 1 ? i % 16 : i / 64, mm = p.a_k == 1 ? i / 16 : i % 64;
      const int m = m0 + mm, k = k0 + kk;
      as[kk][mm] = (m < p.M && k < p.K) ? Elem<TA>::load(p.a, (int64_t)m * p.a_m + (int64_t)k * p.a_k) : 0.0f;
    }
    for (int i = tid; i < 16 * 64; i += 256) {
      const int kk = p.b_k == 1 ? i % 16 : i / 64, nn = p.b_k == 1 ? i / 16 : i % 64;
      const int n = n0 + nn, k = k0 + kk;
      bs[kk][nn] = (n < p.N && k < p.K) ? Elem<TB>::load(p.b, (int64_t)k * p.b_k + (int64_t)n * p.b_n) : 0.0f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      float av[4], bv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) av[i] = as[kk][tm + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) bv[j] = bs[kk][tn + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_fmaf(av[i], bv[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + tm + i;
    if (m >= p.M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + tn + j;
      if (n >= p.N) continue;
      const int64_t o = (int64_t)m * p.N + n;
      const float add = p.c_add ? Elem<TC>::load(p.c_add, o) : 0.0f;
      Elem<TC>::store(p.c, o, acc[i][j] + add);
    }
  }
}

template <typename TA, typename TB, typename TC>
static void launch_small_gemm(const SmallGemm<TA, TB, TC>& p, hipStream_t s) {
  dim3 grid((p.N + 63) / 64, (p.M + 63) / 64);
  hipLaunchKernelGGL((small_gemm_kernel<TA, TB, TC>), grid, dim3(256), 0, s, p);
}

// The same products on the matrix cores (used for dW_g, whose K = T is long): v_mfma_f32_32x32x2_f32
// takes fp32 operands (bf16 inputs widen exactly) and accumulates in fp32. A 64 x 64 tile per workgroup, four waves of 32 x 32; K is
// staged 32 at a time in a double-buffered LDS tile ([k][m] and [k][n], rows padded to 96 floats so
// that the two half-waves of a read, one k-row apart, fall on different banks), and the next chunk
// is loaded into registers while the current one is multiplied.
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
constexpr int kMmK = 32, kMmPitch = 96;

// 8 consecutive elements from a 16-byte aligned address, as fp32
__device__ __forceinline__ void load8(const uint16_t* p, float* v) {
  const uint4 q = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = bf16_to_f32(w[i] & 0xffffu);
    v[2 * i + 1] = bf16_to_f32(w[i] >> 16);
  }
}
__device__ __forceinline__ void load8(const float* p, float* v) {
  const float4 a = *reinterpret_cast<const float4*>(p), b = *reinterpret_cast<const float4*>(p + 4);
  v[0] = a.x, v[1] = a.y, v[2] = a.z, v[3] = a.w, v[4] = b.x, v[5] = b.y, v[6] = b.z, v[7] = b.w;
}

// VEC = 1: A contiguous in m and B contiguous in n (dW_g = x^T dl), M and N multiples of 8; a thread
// loads 8 consecutive m (n) of one k. VEC = 2: both contiguous in k (dX = dl W_g^T), K a multiple of
// 8; a thread loads 8 consecutive k of one m (n). Every 8-element group is 16-byte aligned.
template <typename TA, typename TB, typename TC, int VEC>
__global__ __launch_bounds__(256) void small_gemm_mfma_kernel(const SmallGemm<TA, TB, TC> p) {
  __shared__ float as[2][kMmK][kMmPitch];
  __shared__ float bs[2][kMmK][kMmPitch];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 1, wn = wave >> 1;
  const int m0 = blockIdx.y * 64, n0 = blockIdx.x * 64;
  const int nch = (p.K + kMmK - 1) / kMmK;
  // chunk c -> register set (consecutive threads walk whichever index is contiguous in memory);
  // two sets, so that a chunk's loads are issued two chunks of multiply-adds before their use
  float ra[2][8], rb[2][8];
  auto load = [&](int c, float* pa, float* pb) {
    const int k0 = c * kMmK;
    if constexpr (VEC == 2) {
      const int k = k0 + (tid & 3) * 8, m = m0 + (tid >> 2), n = n0 + (tid >> 2);
      if (k < p.K && m < p.M)
        load8(p.a + (int64_t)m * p.a_m + (int64_t)k, pa);
      else
#pragma unroll
        for (int j = 0; j < 8; ++j) pa[j] = 0.0f;
      if (k < p.K && n < p.N)
        load8(p.b + (int64_t)k + (int64_t)n * p.b_n, pb);
      else
#pragma unroll
        for (int j = 0; j < 8; ++j) pb[j] = 0.0f;
      return;
    }
    if constexpr (VEC == 1) {
      const int k = k0 + (tid >> 3), m = m0 + (tid & 7) * 8, n = n0 + (tid & 7) * 8;
      if (k < p.K && m < p.M)
        load8(p.a + (int64_t)m + (int64_t)k * p.a_k, pa);
      else
#pragma unroll
        for (int j = 0; j < 8; ++j) pa[j] = 0.0f;
      if (k < p.K && n < p.N)
        load8(p.b + (int64_t)k * p.b_k + (int64_t)n, pb);
      else
#pragma unroll
        for (int j = 0; j < 8; ++j) pb[j] = 0.0f;
      return;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int i = tid + 256 * j;
      const int kk = p.a_k == 1 ? i % kMmK : i / 64, mm = p.a_k == 1 ? i / kMmK : i % 64;
      const int m = m0 + mm, k = k0 + kk;
      pa[j] = (m < p.M && k < p.K) ? Elem<TA>::load(p.a, (int64_t)m * p.a_m + (int64_t)k * p.a_k) : 0.0f;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int i = tid + 256 * j;
      const int kk = p.b_k == 1 ? i % kMmK : i / 64, nn = p.b_k == 1 ? i / kMmK : i % 64;
      const int n = n0 + nn, k = k0 + kk;
      pb[j] = (n < p.N && k < p.K) ? Elem<TB>::load(p.b, (int64_t)k * p.b_k + (int64_t)n * p.b_n) : 0.0f;
    }
  };
  auto put = [&](int buf, const float* pa, const float* pb) {
    if constexpr (VEC == 2) {
      const int kk = (tid & 3) * 8, o = tid >> 2;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        as[buf][kk + j][o] = pa[j];
        bs[buf][kk + j][o] = pb[j];
      }
      return;
    }
    if constexpr (VEC == 1) {
      const int kk = tid >> 3, o = (tid & 7) * 8;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        as[buf][kk][o + j] = pa[j];
        bs[buf][kk][o + j] = pb[j];
      }
      return;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int i = tid + 256 * j;
      const int kk = p.a_k == 1 ? i % kMmK : i / 64, mm = p.a_k == 1 ? i / kMmK : i % 64;
      as[buf][kk][mm] = pa[j];
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int i = tid + 256 * j;
      const int kk = p.b_k == 1 ? i % kMmK : i / 64, nn = p.b_k == 1 ? i / kMmK : i % 64;
      bs[buf][kk][nn] = pb[j];
    }
  };
  f32x16_t acc;
#pragma unroll
  for (int q = 0; q < 16; ++q) acc[q] = 0.0f;
  // lane l supplies A(m = l % 32, k = l / 32) and B(k = l / 32, n = l % 32) of each 2-deep MFMA
  const int lm = wm * 32 + (lane & 31), ln = wn * 32 + (lane & 31), lk = lane >> 5;
  // all of the chunk's operands are read before its MFMAs (read one by one ahead of each MFMA, every
  // multiply waited for the LDS)
  auto mul = [&](int buf) {
    float av[kMmK / 2], bv[kMmK / 2];
#pragma unroll
    for (int k = 0; k < kMmK; k += 2) {
      av[k / 2] = as[buf][k + lk][lm];
      bv[k / 2] = bs[buf][k + lk][ln];
    }
#pragma unroll
    for (int k = 0; k < kMmK / 2; ++k) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(av[k], bv[k], acc, 0, 0, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, kMmK, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, kMmK / 2, 0);
  };
  // chunk c sits in LDS buffer c % 2; when it is multiplied, chunk c + 1 waits in register set
  // (c + 1) % 2 and chunk c + 2 is being loaded into set c % 2 (which held chunk c)
  load(0, ra[0], rb[0]);
  if (nch > 1) load(1, ra[1], rb[1]);
  put(0, ra[0], rb[0]);
  __syncthreads();
  for (int c = 0; c < nch; c += 2) {
    if (c + 2 < nch) load(c + 2, ra[0], rb[0]);
    mul(0);
    if (c + 1 < nch) put(1, ra[1], rb[1]);
    __syncthreads();
    if (c + 1 >= nch) break;
    if (c + 3 < nch) load(c + 3, ra[1], rb[1]);
    mul(1);
    if (c + 2 < nch) put(0, ra[0], rb[0]);
    __syncthreads();
  }
  // lane l holds column n = l % 32 and rows (q / 4) * 8 + (l / 32) * 4 + q % 4 of the wave's block
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const int m = m0 + wm * 32 + (q >> 2) * 8 + (lane >> 5) * 4 + (q & 3), n = n0 + ln;
    if (m < p.M && n < p.N) {
      const int64_t o = (int64_t)m * p.N + n;
      const float add = p.c_add ? Elem<TC>::load(p.c_add, o) : 0.0f;
      Elem<TC>::store(p.c, o, acc[q] + add);
    }
  }
}

template <typename TA, typename TB, typename TC>
static void launch_small_gemm_mfma(const SmallGemm<TA, TB, TC>& p, hipStream_t s) {
  dim3 grid((p.N + 63) / 64, (p.M + 63) / 64);
  const bool aligned = ((uintptr_t)p.a & 15) == 0 && ((uintptr_t)p.b & 15) == 0;
  const bool mn = aligned && p.a_m == 1 && p.b_n == 1 && p.M % 8 == 0 && p.N % 8 == 0 &&
                  (p.a_k * (int64_t)sizeof(TA)) % 16 == 0 && (p.b_k * (int64_t)sizeof(TB)) % 16 == 0;
  const bool kc = aligned && p.a_k == 1 && p.b_k == 1 && p.K % 8 == 0 && (p.a_m * (int64_t)sizeof(TA)) % 16 == 0 &&
                  (p.b_n * (int64_t)sizeof(TB)) % 16 == 0;
  if (mn)
    hipLaunchKernelGGL((small_gemm_mfma_kernel<TA, TB, TC, 1>), grid, dim3(256), 0, s, p);
  else if (kc)
    hipLaunchKernelGGL((small_gemm_mfma_kernel<TA, TB, TC, 2>), grid, dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL((small_gemm_mfma_kernel<TA, TB, TC, 0>), grid, dim3(256), 0, s, p);
}

// ---------------------------------------------------------------------------------------------
template <typename TE>
static void combine_bwd_t(const void* d_out, const void* y, int T, int H, int k, const int32_t* ros, const float* w,
                          void* d_y, float* d_w, hipStream_t s) {
  dim3 grid((T + kBwdWaves - 1) / kBwdWaves), block(kBwdWaves * kWave);
  const bool vec = H % 8 == 0 && (((uintptr_t)d_out | (uintptr_t)y | (uintptr_t)d_y) & 31) == 0;
  if (vec)
    hipLaunchKernelGGL((combine_bwd_kernel<TE, true>), grid, block, 0, s, (const TE*)d_out, (const TE*)y, T, H, k, ros,
                       w, (TE*)d_y, d_w);
  else
    hipLaunchKernelGGL((combine_bwd_kernel<TE, false>), grid, block, 0, s, (const TE*)d_out, (const TE*)y, T, H, k, ros,
                       w, (TE*)d_y, d_w);
}

hipError_t launch_combine_bwd(const void* d_out, const void* y, int dt, int T, int H, int k, const int32_t* row_of_slot,
                              const float* topk_w, void* d_y, float* d_w, hipStream_t s) {
  if (dt == kBF16)
    combine_bwd_t<uint16_t>(d_out, y, T, H, k, row_of_slot, topk_w, d_y, d_w, s);
  else
    combine_bwd_t<float>(d_out, y, T, H, k, row_of_slot, topk_w, d_y, d_w, s);
  return hipGetLastError();
}

template <typename TE>
static void permute_bwd_t(const void* d_xp, int T, int H, int k, const int32_t* ros, const void* add, void* d_x,
                          hipStream_t s) {
  dim3 grid((T + kBwdWaves - 1) / kBwdWaves), block(kBwdWaves * kWave);
  const bool vec = H % 8 == 0 && (((uintptr_t)d_xp | (uintptr_t)add | (uintptr_t)d_x) & 31) == 0;
  if (vec)
    hipLaunchKernelGGL((permute_bwd_kernel<TE, true>), grid, block, 0, s, (const TE*)d_xp, T, H, k, ros,
                       (const TE*)add, (TE*)d_x);
  else
    hipLaunchKernelGGL((permute_bwd_kernel<TE, false>), grid, block, 0, s, (const TE*)d_xp, T, H, k, ros,
                       (const TE*)add, (TE*)d_x);
}

hipError_t launch_permute_bwd(const void* d_x_perm, int dt, int T, int H, int k, const int32_t* row_of_slot,
                              const void* d_x_add, void* d_x, hipStream_t s) {
  if (dt == kBF16)
    permute_bwd_t<uint16_t>(d_x_perm, T, H, k, row_of_slot, d_x_add, d_x, s);
  else
    permute_bwd_t<float>(d_x_perm, T, H, k, row_of_slot, d_x_add, d_x, s);
  return hipGetLastError();
}

hipError_t launch_router_topk_bwd(const float* logits, const int32_t* idx, const float* w, const float* d_w, int T,
                                  int E, int k, int renorm, float* d_logits, hipStream_t s) {
  dim3 grid((T + kBwdWaves - 1) / kBwdWaves), block(kBwdWaves * kWave);
  const int vpl = (E + kWave - 1) / kWave;
  if (vpl <= 1)
    hipLaunchKernelGGL(router_topk_bwd_kernel<1>, grid, block, 0, s, logits, idx, w, d_w, T, E, k, renorm, d_logits);
  else if (vpl <= 2)
    hipLaunchKernelGGL(router_topk_bwd_kernel<2>, grid, block, 0, s, logits, idx, w, d_w, T, E, k, renorm, d_logits);
  else if (vpl <= 4)
    hipLaunchKernelGGL(router_topk_bwd_kernel<4>, grid, block, 0, s, logits, idx, w, d_w, T, E, k, renorm, d_logits);
  else if (vpl <= 8)
    hipLaunchKernelGGL(router_topk_bwd_kernel<8>, grid, block, 0, s, logits, idx, w, d_w, T, E, k, renorm, d_logits);
  else
    hipLaunchKernelGGL(router_topk_bwd_kernel<16>, grid, block, 0, s, logits, idx, w, d_w, T, E, k, renorm, d_logits);
  return hipGetLastError();
}

template <typename TE>
static void router_logits_bwd_t(const void* x, const void* w_gate, const float* dl, int T, int H, int E,
                                float* d_w_gate, const void* d_x_in, void* d_x, hipStream_t s) {
  if (d_w_gate) {
    SmallGemm<TE, float, float> p{};
    p.a = (const TE*)x;  // A(h, t) = x[t, h]
    p.a_m = 1;
    p.a_k = H;
    p.b = dl;            // B(t, e) = dl[t, e]
    p.b_k = E;
    p.b_n = 1;
    p.c = d_w_gate;
    p.M = H;
    p.N = E;
    p.K = T;
    launch_small_gemm_mfma(p, s);
  }
  if (d_x) {
    SmallGemm<float, TE, TE> p{};
    p.a = dl;            // A(t, e) = dl[t, e]
    p.a_m = E;
    p.a_k = 1;
    p.b = (const TE*)w_gate;  // B(e, h) = W_g[h, e]
    p.b_k = 1;
    p.b_n = E;
    p.c = (TE*)d_x;
    p.c_add = (const TE*)d_x_in;
    p.M = T;
    p.N = H;
    p.K = E;
    // on the matrix cores with 16-byte loads along K when the rows allow them; else the vector-ALU tiles
    const bool kc = E % 8 == 0 && ((uintptr_t)dl & 15) == 0 && ((uintptr_t)w_gate & 15) == 0;
    if (kc)
      launch_small_gemm_mfma(p, s);
    else
      launch_small_gemm(p, s);
  }
}

hipError_t launch_router_logits_bwd(const void* x, const void* w_gate, const float* d_logits, int dt, int T, int H,
                                    int E, float* d_w_gate, const void* d_x_in, void* d_x, hipStream_t s) {
  if (dt == kBF16)
    router_logits_bwd_t<uint16_t>(x, w_gate, d_logits, T, H, E, d_w_gate, d_x_in, d_x, s);
  else
    router_logits_bwd_t<float>(x, w_gate, d_logits, T, H, E, d_w_gate, d_x_in, d_x, s);
  return hipGetLastError();
}

}  // namespace moe
