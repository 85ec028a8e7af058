// Device helpers shared by the MoE layer kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kWave = 64;

// bf16 is carried as its raw 16-bit pattern.
__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// fp32 -> bf16, round to nearest, ties to even, fp32 subnormals kept; NaN stays NaN (quieted). One
// v_cvt_pk_bf16_f32 per pair: for every non-NaN fp32 pattern the same bits as rounding in integer
// arithmetic (add 0x7fff plus the lowest kept bit, drop the low half).
typedef __bf16 bf16x2_hw __attribute__((ext_vector_type(2)));
typedef float f32x2_hw __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2_hw f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_hw));
}
__device__ __forceinline__ uint32_t f32_to_bf16(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

template <typename T> struct Elem;
template <> struct Elem<float> {
  static __device__ __forceinline__ float load(const float* p, int64_t i) { return p[i]; }
  static __device__ __forceinline__ void store(float* p, int64_t i, float v) { p[i] = v; }
};
template <> struct Elem<uint16_t> {
  static __device__ __forceinline__ float load(const uint16_t* p, int64_t i) { return bf16_to_f32(p[i]); }
  static __device__ __forceinline__ void store(uint16_t* p, int64_t i, float v) { p[i] = (uint16_t)f32_to_bf16(v); }
};

__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & (kWave - 1)); }

// Inclusive prefix sum across the 64 lanes of a wave.
__device__ __forceinline__ int wave_incl_scan(int v) {
  const int lane = lane_id();
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    int n = __shfl_up(v, off, kWave);
    if (lane >= off) v += n;
  }
  return v;
}

__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

// Exclusive prefix sum of a[0..n) held in LDS, in place; a[n] receives the total.
// Every thread of the block must call it; NT = blockDim.x (a multiple of 64); n <= 4 * NT.
template <int NT>
__device__ void block_exclusive_scan(int* a, int n, int* wave_tot /* LDS, NT/64 ints */) {
  static_assert(NT % kWave == 0 && NT <= 1024, "block size");
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = tid / kWave;
  int v[4];
  int s = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int i = tid * 4 + q;
    v[q] = i < n ? a[i] : 0;
    s += v[q];
  }
  const int incl = wave_incl_scan(s);
  if (lane == kWave - 1) wave_tot[wave] = incl;
  __syncthreads();
  int before = 0, total = 0;
  for (int w = 0; w < NT / kWave; ++w) {
    const int t = wave_tot[w];
    if (w < wave) before += t;
    total += t;
  }
  int run = before + incl - s;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int i = tid * 4 + q;
    if (i < n) a[i] = run;
    run += v[q];
  }
  if (tid == 0) a[n] = total;
  __syncthreads();
}

}  // namespace moe
