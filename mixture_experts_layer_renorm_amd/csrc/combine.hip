// Unpermute + gate-weighted combine.
//
// The naive MoE forward of the "DeepSeek MoE: EP and FSDP" guide (gsyq.cn, Expert Parallelism
// section) ends by summing the experts' outputs weighted by the gate scores and passing the sum
// on; the InternVL3.5 practice doc (MindSpeed-MM issue 625, section 8.3) calls this last step of
// the fused expert path "unpermute".
//
//   out[t] = residual[t] + sum_{j<k} topk_w[t,j] * y[row_of_slot[t*k+j]]     (fp32, j ascending)
//
// One wave per token: each lane owns 8 consecutive features, gathers the k rows with 16-byte
// loads (bf16) and accumulates in fp32; the result is rounded once to the output dtype.
#include "common.hpp"
#include "internal.hpp"

namespace moe {

constexpr int kCombineWaves = 4;

__device__ __forceinline__ void unpack8(const uint4& v, float* f) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(w[i] << 16);
    f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

// bf16, H % 8 == 0, 16-byte aligned rows. The loads of up to kCombineBatch rows are all issued
// before the multiply-adds that consume them (a dropped slot loads row 0 and skips its
// multiply-add); a lane covers kCombineVec 16-byte pieces of each row per pass (the whole 4 KB row
// of H = 2048 in one pass), so it keeps kCombineVec * kCombineBatch = 32 loads in flight. Every
// byte of y is read once and every byte of out written once, so both go through non-temporal
// (streaming) accesses that do not displace other lines from the caches (measured on 537 MB of y:
// 128 -> 104 us).
constexpr int kCombineBatch = 8;
constexpr int kCombineVec = 4;
typedef __attribute__((ext_vector_type(4))) unsigned int cu32x4;
__device__ __forceinline__ uint4 nt_load16(const uint4* p) {
  const cu32x4 r = __builtin_nontemporal_load(reinterpret_cast<const cu32x4*>(p));
  return make_uint4(r.x, r.y, r.z, r.w);
}
__device__ __forceinline__ void nt_store16(const uint4& o, uint4* p) {
  const cu32x4 r = {o.x, o.y, o.z, o.w};
  __builtin_nontemporal_store(r, reinterpret_cast<cu32x4*>(p));
}

__global__ __launch_bounds__(kCombineWaves * kWave) void combine_bf16_kernel(
    const uint16_t* __restrict__ y, int T, int H, int k, const int32_t* __restrict__ row_of_slot,
    const float* __restrict__ topk_w, const uint16_t* __restrict__ residual, uint16_t* __restrict__ out) {
  const int lane = lane_id();
  const int t = blockIdx.x * kCombineWaves + (int)(threadIdx.x / kWave);
  if (t >= T) return;
  const int my_row = lane < k ? row_of_slot[(int64_t)t * k + lane] : -1;
  const float my_w = lane < k ? topk_w[(int64_t)t * k + lane] : 0.0f;
  const int nvec = H >> 3;
  const uint4* y4 = reinterpret_cast<const uint4*>(y);
  for (int v0 = 0; v0 < nvec; v0 += kCombineVec * kWave) {
    float acc[kCombineVec][8];
    bool live[kCombineVec];
#pragma unroll
    for (int u = 0; u < kCombineVec; ++u) {
      const int v = v0 + u * kWave + lane;
      live[u] = v < nvec;
      if (residual && live[u]) {
        unpack8(reinterpret_cast<const uint4*>(residual + (int64_t)t * H)[v], acc[u]);
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[u][i] = 0.0f;
      }
    }
    for (int j0 = 0; j0 < k; j0 += kCombineBatch) {
      uint4 buf[kCombineBatch][kCombineVec];
      int rows[kCombineBatch];
#pragma unroll
      for (int jj = 0; jj < kCombineBatch; ++jj) {
        rows[jj] = j0 + jj < k ? __shfl(my_row, j0 + jj, kWave) : -1;
        const int64_t rr = max(rows[jj], 0);
#pragma unroll
        for (int u = 0; u < kCombineVec; ++u) {
          const int v = v0 + u * kWave + lane;
          if (j0 + jj < k && live[u]) buf[jj][u] = nt_load16(&y4[rr * nvec + v]);
        }
      }
#pragma unroll
      for (int jj = 0; jj < kCombineBatch; ++jj) {
        if (rows[jj] < 0) continue;  // also j >= k
        const float w = __shfl(my_w, j0 + jj, kWave);
#pragma unroll
        for (int u = 0; u < kCombineVec; ++u) {
          if (live[u]) {
            float f[8];
            unpack8(buf[jj][u], f);
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[u][i] = __builtin_fmaf(w, f[i], acc[u][i]);
          }
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kCombineVec; ++u) {
      const int v = v0 + u * kWave + lane;
      if (live[u]) {
        uint4 o;
        o.x = pack_bf16x2(acc[u][0], acc[u][1]);
        o.y = pack_bf16x2(acc[u][2], acc[u][3]);
        o.z = pack_bf16x2(acc[u][4], acc[u][5]);
        o.w = pack_bf16x2(acc[u][6], acc[u][7]);
        nt_store16(o, &reinterpret_cast<uint4*>(out + (int64_t)t * H)[v]);
      }
    }
  }
}

// any dtype / width: one element per lane step
template <typename TE>
__global__ __launch_bounds__(kCombineWaves * kWave) void combine_generic_kernel(
    const TE* __restrict__ y, int T, int H, int k, const int32_t* __restrict__ row_of_slot,
    const float* __restrict__ topk_w, const TE* __restrict__ residual, TE* __restrict__ out) {
  const int lane = lane_id();
  const int t = blockIdx.x * kCombineWaves + (int)(threadIdx.x / kWave);
  if (t >= T) return;
  const int my_row = lane < k ? row_of_slot[(int64_t)t * k + lane] : -1;
  const float my_w = lane < k ? topk_w[(int64_t)t * k + lane] : 0.0f;
  for (int base = 0; base < H; base += kWave) {   // uniform trip count: the shuffles read active lanes
    const int c = base + lane;
    const bool act = c < H;
    float acc = residual && act ? Elem<TE>::load(residual, (int64_t)t * H + c) : 0.0f;
    for (int j = 0; j < k; ++j) {
      const int r = __shfl(my_row, j, kWave);
      const float w = __shfl(my_w, j, kWave);
      if (r >= 0 && act) acc = __builtin_fmaf(w, Elem<TE>::load(y, (int64_t)r * H + c), acc);
    }
    if (act) Elem<TE>::store(out, (int64_t)t * H + c, acc);
  }
}

hipError_t launch_combine(const void* y, int dt, int T, int H, int k, const int32_t* row_of_slot, const float* topk_w,
                          const void* residual, void* out, hipStream_t s) {
  dim3 grid((T + kCombineWaves - 1) / kCombineWaves), block(kCombineWaves * kWave);
  const bool aligned = (((uintptr_t)y | (uintptr_t)out | (uintptr_t)residual) & 15) == 0;
  if (dt == kBF16 && H % 8 == 0 && aligned) {
    hipLaunchKernelGGL(combine_bf16_kernel, grid, block, 0, s, (const uint16_t*)y, T, H, k, row_of_slot, topk_w,
                       (const uint16_t*)residual, (uint16_t*)out);
  } else if (dt == kBF16) {
    hipLaunchKernelGGL(combine_generic_kernel<uint16_t>, grid, block, 0, s, (const uint16_t*)y, T, H, k, row_of_slot,
                       topk_w, (const uint16_t*)residual, (uint16_t*)out);
  } else {
    hipLaunchKernelGGL(combine_generic_kernel<float>, grid, block, 0, s, (const float*)y, T, H, k, row_of_slot, topk_w,
                       (const float*)residual, (float*)out);
  }
  return hipGetLastError();
}

}  // namespace moe
