// Grouped SwiGLU expert FFN over the fused expert weights.
//
// The fused layout is the one of the MindSpeed-MM InternVL3.5 practice doc (issue 625, section 2,
// model integration): gate_up [E*H, 2*I] and down [E*I, H], row-major; its section 8.3 runs the
// experts as permute -> grouped_matmul -> SwiGLU -> grouped_matmul -> unpermute, and its
// optimisation doc (section 2.1) groups the experts into one call to avoid per-expert launches.
// Gate columns are [0, I) and up columns [I, 2I) of an expert's block; h = silu(gate) * up.
//
//   GEMM-1 (MODE 0): for each expert e, rows r of segment e:  h[r, :] = silu(x_perm[r] @ Wg_e) * (x_perm[r] @ Wu_e)
//   GEMM-2 (MODE 1): y[r, :] = h[r] @ down_e
//
// bf16 path: v_mfma_f32_32x32x16_bf16 with fp32 accumulation. A workgroup (4 waves) owns a
// 256-row x 128-column tile of one expert; each wave owns 64 rows x all 128 columns. Tiles are
// derived on the device from expert_offsets (empty experts own no tile), so no host sync is needed.
// K is staged through a double-buffered LDS ring in steps of 64. The weights are row-major [K, N]
// (N contiguous) while the matrix cores want K contiguous per lane, so each thread loads a 4 x 8
// block of the weight tile and transposes it in registers before writing it to LDS. LDS rows are
// 128 bytes; 16-byte chunks are XOR-swizzled by (row ^ row >> 3) & 7 so that both the 16-byte
// fragment reads (32 consecutive rows) and the transposed 8-byte writes stay conflict-light.
// The MFMA is issued with the weight fragment as its first operand, so each lane ends up holding
// four consecutive output columns of one row, which become one 8-byte store.
#include "common.hpp"
#include "internal.hpp"

namespace moe {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;

constexpr int kBM = 256;
constexpr int kBN = 128;
constexpr int kBK = 64;
constexpr int kGemmThreads = 256;
constexpr int kTileA = kBM * kBK * 2;
constexpr int kTileB = kBN * kBK * 2;
constexpr int kStage = kTileA + kTileB;
constexpr int kGemmMaxE = 1024;

__device__ __forceinline__ int lds_swz(int r) { return (r ^ (r >> 3)) & 7; }
// byte offset of 16-byte chunk c (8 consecutive k) of row r in a [rows][64] bf16 LDS tile
__device__ __forceinline__ int lds_off(int r, int c) { return r * 128 + ((c ^ lds_swz(r)) << 4); }

__device__ __forceinline__ float silu_f(float g) { return g / (1.0f + __expf(-g)); }

// Shared tile schedule: linear workgroup index -> (expert, row range, column tile).
// Returns false when this workgroup has no tile.
struct TileInfo {
  int e, row0, row_end, nt;
};

__device__ __forceinline__ bool tile_of_block(const int32_t* __restrict__ offsets, int E, int bm, int ntiles_n,
                                              int* s_pref, int* s_wtot, int* s_e, TileInfo& ti) {
  const int tid = threadIdx.x;
  const int G = gridDim.x;  // a multiple of 8
  const int b = blockIdx.x;
  // consecutive logical tiles land on the same XCD (blocks are dealt round-robin over 8 XCDs)
  const int L = (b & 7) * (G >> 3) + (b >> 3);
  const int mt_g = L / ntiles_n;
  ti.nt = L - mt_g * ntiles_n;
  for (int e = tid; e < E; e += kGemmThreads) {
    const int n = offsets[e + 1] - offsets[e];
    s_pref[e] = n > 0 ? (n + bm - 1) / bm : 0;
  }
  __syncthreads();
  block_exclusive_scan<kGemmThreads>(s_pref, E, s_wtot);
  if (mt_g >= s_pref[E]) return false;
  for (int e = tid; e < E; e += kGemmThreads)
    if (s_pref[e] <= mt_g && mt_g < s_pref[e + 1]) *s_e = e;
  __syncthreads();
  ti.e = *s_e;
  ti.row0 = offsets[ti.e] + (mt_g - s_pref[ti.e]) * bm;
  ti.row_end = min(ti.row0 + bm, (int)offsets[ti.e + 1]);
  return true;
}

template <int MODE>
__global__ __launch_bounds__(kGemmThreads, 1) void grouped_gemm_bf16_kernel(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ W, const int32_t* __restrict__ offsets, int E, int K,
    int ncols, int ldw, int ntiles_n, uint16_t* __restrict__ out, int ldo, uint16_t* __restrict__ gu_saved) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * kStage];
  __shared__ int s_pref[kGemmMaxE + 1];
  __shared__ int s_wtot[kGemmThreads / kWave];
  __shared__ int s_e;

  TileInfo ti;
  if (!tile_of_block(offsets, E, kBM, ntiles_n, s_pref, s_wtot, &s_e, ti)) return;

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int row0 = ti.row0, row_end = ti.row_end, nt = ti.nt;
  const uint16_t* Wexp = W + (int64_t)ti.e * K * ldw;

  // weight-tile loader: thread owns 8 columns x 4 consecutive k rows
  const int ng = tid & 15, kg = tid >> 4;
  int bcol;
  bool bcol_ok;
  if (MODE == 0) {
    const int nl = ng * 8;
    const int j = nt * 64 + (nl & 63);
    bcol = (nl < 64 ? 0 : ncols) + j;
    bcol_ok = j < ncols;
  } else {
    bcol = nt * kBN + ng * 8;
    bcol_ok = bcol < ncols;
  }

  uint4 ra[8], rb[4];
  auto load_tiles = [&](int kt) {
    const int k0 = kt * kBK;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int idx = tid + kGemmThreads * i;
      const int r = idx >> 3, c = idx & 7;
      const int grow = row0 + r;
      const int kc = k0 + c * 8;
      if (grow < row_end && kc < K)
        ra[i] = *reinterpret_cast<const uint4*>(A + (int64_t)grow * K + kc);
      else
        ra[i] = make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int kr = k0 + kg * 4 + i;
      if (bcol_ok && kr < K)
        rb[i] = *reinterpret_cast<const uint4*>(Wexp + (int64_t)kr * ldw + bcol);
      else
        rb[i] = make_uint4(0u, 0u, 0u, 0u);
    }
  };
  auto store_tiles = [&](uint8_t* st) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int idx = tid + kGemmThreads * i;
      *reinterpret_cast<uint4*>(st + lds_off(idx >> 3, idx & 7)) = ra[i];
    }
    uint8_t* sb = st + kTileA;
    const uint32_t b0[4] = {rb[0].x, rb[0].y, rb[0].z, rb[0].w};
    const uint32_t b1[4] = {rb[1].x, rb[1].y, rb[1].z, rb[1].w};
    const uint32_t b2[4] = {rb[2].x, rb[2].y, rb[2].z, rb[2].w};
    const uint32_t b3[4] = {rb[3].x, rb[3].y, rb[3].z, rb[3].w};
    const int koff = (kg & 1) * 8;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const uint32_t lo01 = (b0[d] & 0xffffu) | (b1[d] << 16);
      const uint32_t hi01 = (b0[d] >> 16) | (b1[d] & 0xffff0000u);
      const uint32_t lo23 = (b2[d] & 0xffffu) | (b3[d] << 16);
      const uint32_t hi23 = (b2[d] >> 16) | (b3[d] & 0xffff0000u);
      const int n0 = ng * 8 + 2 * d;
      *reinterpret_cast<uint2*>(sb + lds_off(n0, kg >> 1) + koff) = make_uint2(lo01, lo23);
      *reinterpret_cast<uint2*>(sb + lds_off(n0 + 1, kg >> 1) + koff) = make_uint2(hi01, hi23);
    }
  };

  f32x16 acc[2][4];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[mb][nb][q] = 0.0f;

  const int wrows = row_end - (row0 + wave * 64);
  const int nmb = wrows <= 0 ? 0 : (wrows <= 32 ? 1 : 2);  // m-blocks of this wave holding real rows

  const int KT = (K + kBK - 1) / kBK;
  load_tiles(0);
  store_tiles(smem);
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    const uint8_t* cur = smem + (kt & 1) * kStage;
    if (kt + 1 < KT) load_tiles(kt + 1);
    if (nmb > 0) {
#pragma unroll
      for (int kk = 0; kk < kBK / 16; ++kk) {
        const int c = kk * 2 + (lane >> 5);
        bf16x8 af[2], bfr[4];
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
          af[mb] = *reinterpret_cast<const bf16x8*>(cur + lds_off(wave * 64 + mb * 32 + (lane & 31), c));
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
          bfr[nb] = *reinterpret_cast<const bf16x8*>(cur + kTileA + lds_off(nb * 32 + (lane & 31), c));
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) acc[0][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[nb], af[0], acc[0][nb], 0, 0, 0);
        if (nmb > 1) {
#pragma unroll
          for (int nb = 0; nb < 4; ++nb)
            acc[1][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[nb], af[1], acc[1][nb], 0, 0, 0);
        }
      }
    }
    if (kt + 1 < KT) store_tiles(smem + ((kt + 1) & 1) * kStage);
    __syncthreads();
  }

  // epilogue: lane holds row m = .. + (lane & 31) and columns (q/4)*8 + (lane/32)*4 + q%4 of each block
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
    const int m = row0 + wave * 64 + mb * 32 + (lane & 31);
    if (m >= row_end) continue;
    if (MODE == 0) {
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int col = nt * 64 + nb * 32 + g * 8 + (lane >> 5) * 4;
          if (col >= ncols) continue;
          float hv[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) hv[q] = silu_f(acc[mb][nb][g * 4 + q]) * acc[mb][nb + 2][g * 4 + q];
          *reinterpret_cast<uint2*>(out + (int64_t)m * ldo + col) =
              make_uint2(pack_bf16x2(hv[0], hv[1]), pack_bf16x2(hv[2], hv[3]));
          if (gu_saved) {
            uint16_t* gs = gu_saved + (int64_t)m * 2 * ncols;
            *reinterpret_cast<uint2*>(gs + col) =
                make_uint2(pack_bf16x2(acc[mb][nb][g * 4 + 0], acc[mb][nb][g * 4 + 1]),
                           pack_bf16x2(acc[mb][nb][g * 4 + 2], acc[mb][nb][g * 4 + 3]));
            *reinterpret_cast<uint2*>(gs + ncols + col) =
                make_uint2(pack_bf16x2(acc[mb][nb + 2][g * 4 + 0], acc[mb][nb + 2][g * 4 + 1]),
                           pack_bf16x2(acc[mb][nb + 2][g * 4 + 2], acc[mb][nb + 2][g * 4 + 3]));
          }
        }
      }
    } else {
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int col = nt * kBN + nb * 32 + g * 8 + (lane >> 5) * 4;
          if (col >= ncols) continue;
          *reinterpret_cast<uint2*>(out + (int64_t)m * ldo + col) =
              make_uint2(pack_bf16x2(acc[mb][nb][g * 4 + 0], acc[mb][nb][g * 4 + 1]),
                         pack_bf16x2(acc[mb][nb][g * 4 + 2], acc[mb][nb][g * 4 + 3]));
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------------------------
// fp32 path: one thread per output element, fp32 fused multiply-add over k ascending.
__device__ __forceinline__ int expert_of_row(const int32_t* __restrict__ offsets, int E, int r) {
  int lo = 0, hi = E;  // find e with offsets[e] <= r < offsets[e+1]
  if (r < offsets[0] || r >= offsets[E]) return -1;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (offsets[mid] <= r)
      lo = mid;
    else
      hi = mid;
  }
  return lo;
}

__global__ __launch_bounds__(256) void grouped_ffn1_f32_kernel(const float* __restrict__ A, const float* __restrict__ W,
                                                               const int32_t* __restrict__ offsets, int E, int N, int K,
                                                               int I, float* __restrict__ h, float* __restrict__ gu_saved) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (int64_t)N * I) return;
  const int r = (int)(gid / I), j = (int)(gid % I);
  const int e = expert_of_row(offsets, E, r);
  if (e < 0) return;
  const float* a = A + (int64_t)r * K;
  const float* w = W + (int64_t)e * K * 2 * I;
  float g = 0.0f, u = 0.0f;
  for (int k = 0; k < K; ++k) {
    g = __builtin_fmaf(a[k], w[(int64_t)k * 2 * I + j], g);
    u = __builtin_fmaf(a[k], w[(int64_t)k * 2 * I + I + j], u);
  }
  h[(int64_t)r * I + j] = g / (1.0f + expf(-g)) * u;
  if (gu_saved) {
    gu_saved[(int64_t)r * 2 * I + j] = g;
    gu_saved[(int64_t)r * 2 * I + I + j] = u;
  }
}

__global__ __launch_bounds__(256) void grouped_ffn2_f32_kernel(const float* __restrict__ Hh, const float* __restrict__ D,
                                                               const int32_t* __restrict__ offsets, int E, int N, int I,
                                                               int H, float* __restrict__ y) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (int64_t)N * H) return;
  const int r = (int)(gid / H), c = (int)(gid % H);
  const int e = expert_of_row(offsets, E, r);
  if (e < 0) return;
  const float* a = Hh + (int64_t)r * I;
  const float* d = D + (int64_t)e * I * H;
  float acc = 0.0f;
  for (int i = 0; i < I; ++i) acc = __builtin_fmaf(a[i], d[(int64_t)i * H + c], acc);
  y[(int64_t)r * H + c] = acc;
}

// ---------------------------------------------------------------------------------------------
static inline int round_up8(int64_t v) { return (int)((v + 7) / 8 * 8); }

hipError_t launch_gemm_gate_up(const void* x_perm, const void* gate_up, int dt, int N, int H, int I, int E,
                               const int32_t* offsets, void* h, void* gu_saved, hipStream_t s) {
  if (dt == kBF16) {
    const int64_t mt_bound = ((int64_t)N + (int64_t)E * (kBM - 1)) / kBM;
    const int nt1 = (I + 63) / 64;
    hipLaunchKernelGGL(grouped_gemm_bf16_kernel<0>, dim3(round_up8(mt_bound * nt1)), dim3(kGemmThreads), 0, s,
                       (const uint16_t*)x_perm, (const uint16_t*)gate_up, offsets, E, H, I, 2 * I, nt1, (uint16_t*)h, I,
                       (uint16_t*)gu_saved);
  } else {
    const int64_t n1 = (int64_t)N * I;
    hipLaunchKernelGGL(grouped_ffn1_f32_kernel, dim3((unsigned)((n1 + 255) / 256)), dim3(256), 0, s,
                       (const float*)x_perm, (const float*)gate_up, offsets, E, N, H, I, (float*)h, (float*)gu_saved);
  }
  return hipGetLastError();
}

hipError_t launch_gemm_down(const void* h, const void* down, int dt, int N, int H, int I, int E, const int32_t* offsets,
                            void* y, hipStream_t s) {
  if (dt == kBF16) {
    const int64_t mt_bound = ((int64_t)N + (int64_t)E * (kBM - 1)) / kBM;
    const int nt2 = (H + kBN - 1) / kBN;
    hipLaunchKernelGGL(grouped_gemm_bf16_kernel<1>, dim3(round_up8(mt_bound * nt2)), dim3(kGemmThreads), 0, s,
                       (const uint16_t*)h, (const uint16_t*)down, offsets, E, I, H, H, nt2, (uint16_t*)y, H,
                       (uint16_t*)nullptr);
  } else {
    const int64_t n2 = (int64_t)N * H;
    hipLaunchKernelGGL(grouped_ffn2_f32_kernel, dim3((unsigned)((n2 + 255) / 256)), dim3(256), 0, s, (const float*)h,
                       (const float*)down, offsets, E, N, I, H, (float*)y);
  }
  return hipGetLastError();
}

}  // namespace moe
