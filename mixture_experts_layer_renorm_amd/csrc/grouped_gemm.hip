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
#include <type_traits>

#include "common.hpp"
#include "internal.hpp"

namespace moe {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) short i16x4;
typedef __attribute__((ext_vector_type(8))) short i16x8;
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int kBufferWord3 = 0x00020000;  // gfx9 raw buffer descriptor: 32-bit data, offset addressing
constexpr int kOutOfRange = 0x7ffffff0;    // an offset past every descriptor's end: loads return zero

constexpr int kBM = 256;            // rows of one expert per workgroup tile
constexpr int kBN = 256;            // weight columns per tile (GEMM-1: 128 gate + 128 up)
constexpr int kBK = 32;             // K per pipeline step
constexpr int kStages = 4;          // LDS ring depth: steps s+1..s+3 are in flight while s computes
constexpr int kGemmThreads = 512;   // 8 waves (2 per SIMD): 4 along M (64 rows each) x 2 along N (128 columns each)
constexpr int kTileA = kBM * kBK * 2;  // 16 KB: [256 rows][32 k], 64-byte rows
constexpr int kTileB = kBK * kBN * 2;  // 16 KB: [32 k][256 n], 512-byte rows (natural weight layout)
constexpr int kWaves = kGemmThreads / 64;
constexpr int kDmaPerWave = (kTileA + kTileB) / 1024 / kWaves;  // 1 KB per wave-wide DMA instruction
constexpr int kDmaA = kTileA / 1024 / kWaves;  // row-tile DMA instructions per wave per step
constexpr int kDmaB = kTileB / 1024 / kWaves;
constexpr int kGemmMaxE = 1024;

// LDS swizzles, applied when choosing which global chunk each DMA lane fetches. They keep the
// fragment reads free of bank conflicts whether the LDS serves 128 or 256 bytes per clock:
//  - row tile (64-byte rows): 16-byte chunk c (8 k) of row r lives at chunk c ^ g(r) with
//    g(r) = ((r >> 1) ^ (r >> 2)) & 3; the 8 (or 16) consecutive rows read together at one logical
//    chunk then land on distinct banks;
//  - weight tile (512-byte k-rows): 16-byte chunk c (8 n) of k-row r lives at chunk c ^ f(r) with
//    f(r) = 4 (r & 3) + 2 ((r >> 1) & 1); the transpose read of four consecutive k-rows x 32 bytes
//    (x 64 bytes for two lane groups) then lands on distinct banks. f is even and below 16, so a
//    16-byte pair stays adjacent and the gate / up halves of a GEMM-1 row never mix.
__device__ __forceinline__ int swz_a(int r) { return ((r >> 1) ^ (r >> 2)) & 3; }
__device__ __forceinline__ int swz_b(int r) { return 4 * (r & 3) + 2 * ((r >> 1) & 1); }

__device__ __forceinline__ float silu_f(float g) { return g / (1.0f + __expf(-g)); }

// Linear workgroup index -> (expert, row range, column tile). Returns false when the workgroup
// has no tile (the grid is sized for the worst case over any distribution of rows).
struct TileInfo {
  int e, row0, row_end, nt;
};

template <int NT>
__device__ __forceinline__ bool tile_of_block(const int32_t* __restrict__ offsets, int E, int bm, int ntiles_n,
                                              int* s_pref, int* s_wtot, int* s_e, TileInfo& ti) {
  const int tid = threadIdx.x;
  const int G = gridDim.x;  // a multiple of 8
  const int b = blockIdx.x;
  // consecutive logical tiles land on the same XCD (blocks are dealt round-robin over 8 XCDs),
  // so the column tiles of one row tile share its rows through that XCD's L2
  const int L = (b & 7) * (G >> 3) + (b >> 3);
  const int mt_g = L / ntiles_n;
  ti.nt = L - mt_g * ntiles_n;
  for (int e = tid; e < E; e += NT) {
    const int n = offsets[e + 1] - offsets[e];
    s_pref[e] = n > 0 ? (n + bm - 1) / bm : 0;
  }
  __syncthreads();
  block_exclusive_scan<NT>(s_pref, E, s_wtot);
  if (mt_g >= s_pref[E]) return false;
  for (int e = tid; e < E; e += NT)
    if (s_pref[e] <= mt_g && mt_g < s_pref[e + 1]) *s_e = e;
  __syncthreads();
  ti.e = __builtin_amdgcn_readfirstlane(*s_e);
  ti.row0 = __builtin_amdgcn_readfirstlane(offsets[ti.e] + (mt_g - s_pref[ti.e]) * bm);
  ti.row_end = __builtin_amdgcn_readfirstlane(min(ti.row0 + bm, (int)offsets[ti.e + 1]));
  return true;
}

template <int MODE>
__global__ __launch_bounds__(kGemmThreads) void grouped_gemm_bf16_kernel(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ W, const int32_t* __restrict__ offsets, int E, int K,
    int ncols, int ldw, int ntiles_n, uint16_t* __restrict__ out, int ldo, uint16_t* __restrict__ gu_saved) {
  // one LDS object per ring slot, so that the compiler can tell a DMA into one slot from reads of another
  __shared__ __attribute__((aligned(1024))) uint8_t sA0[kTileA], sA1[kTileA], sA2[kTileA], sA3[kTileA];
  __shared__ __attribute__((aligned(1024))) uint8_t sB0[kTileB], sB1[kTileB], sB2[kTileB], sB3[kTileB];
  __shared__ int s_pref[kGemmMaxE + 1];
  __shared__ int s_wtot[kGemmThreads / kWave];
  __shared__ int s_e;

  TileInfo ti;
  if (!tile_of_block<kGemmThreads>(offsets, E, kBM, ntiles_n, s_pref, s_wtot, &s_e, ti)) return;

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int wm = wave & 3, wn = wave >> 2;
  const int row0 = ti.row0, row_end = ti.row_end, nt = ti.nt;

  // Buffer descriptors: the row tile covers exactly rows [row0, row_end) and the weight block exactly
  // expert e's K rows, so rows past either end read as zero.
  const __amdgpu_buffer_rsrc_t rsA = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(A + (int64_t)row0 * K), (short)0, (row_end - row0) * K * 2, kBufferWord3);
  const __amdgpu_buffer_rsrc_t rsW = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(W + (int64_t)ti.e * K * ldw), (short)0, K * ldw * 2, kBufferWord3);

  // ---- DMA lanes. Row tile: wave w, instruction i fills rows (kDmaA w + i) * 16 .. + 16, four lanes
  // per row. Weight tile: instruction i fills k-rows (kDmaB w + i) * 2 .. + 2, 32 lanes per row.
  int a_off[kDmaA], a_kc[kDmaA], b_off[kDmaB];
  bool b_ok[kDmaB];
#pragma unroll
  for (int i = 0; i < kDmaA; ++i) {
    const int r = (wave * kDmaA + i) * 16 + (lane >> 2);
    const int c = (lane & 3) ^ swz_a(r);
    a_kc[i] = c * 8;
    a_off[i] = (r * K + c * 8) * 2;
  }
#pragma unroll
  for (int i = 0; i < kDmaB; ++i) {
    const int kr = (wave * kDmaB + i) * 2 + (lane >> 5);
    const int cb = (lane & 31) ^ swz_b(kr);
    int col;
    if (MODE == 0) {
      const int j = nt * 128 + (cb & 15) * 8;
      b_ok[i] = j < ncols;
      col = (cb < 16 ? 0 : ncols) + j;
    } else {
      col = nt * kBN + cb * 8;
      b_ok[i] = col < ncols;
    }
    b_off[i] = (kr * ldw + col) * 2;
  }
  auto dma = [&](int kt, uint8_t* sa, uint8_t* sb) {
    const int k0 = kt * kBK;
#pragma unroll
    for (int i = 0; i < kDmaA; ++i) {
      const int off = (k0 + a_kc[i] < K) ? a_off[i] + k0 * 2 : kOutOfRange;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsA, (lds_void*)(sa + (wave * kDmaA + i) * 1024), 16, off, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < kDmaB; ++i) {
      const int off = b_ok[i] ? b_off[i] + k0 * ldw * 2 : kOutOfRange;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsW, (lds_void*)(sb + (wave * kDmaB + i) * 1024), 16, off, 0, 0, 0);
    }
  };

  // ---- fragments. Row block mb: lane reads row (lane & 31) of the block, k = kk*16 + (lane/32)*8
  // .. +8. Weight block nb (32 columns from brow[nb]): two transpose reads give column
  // brow + (lane & 31) at k = kk*16 + (lane/32)*8 + 0..3 and + 4..7.
  int brow[4];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb)
    brow[nb] = MODE == 0 ? ((nb >> 1) * 128 + wn * 64 + (nb & 1) * 32) : (wn * 128 + nb * 32);
  const int q = lane >> 4, sl = lane & 15;
  int a_rd[2][2], b_rd[2][4][2];
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      const int r = wm * 64 + mb * 32 + (lane & 31);
      const int c = kk * 2 + (lane >> 5);
      a_rd[kk][mb] = r * 64 + ((c ^ swz_a(r)) << 4);
    }
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
      for (int ri = 0; ri < 2; ++ri) {
        const int kr = kk * 16 + (q >> 1) * 8 + ri * 4 + (sl >> 2);
        const int col = brow[nb] + (q & 1) * 16 + 4 * (sl & 3);
        b_rd[kk][nb][ri] = kr * 512 + (((col >> 3) ^ swz_b(kr)) << 4) + (col & 7) * 2;
      }
  }

  f32x16 acc[2][4];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
      for (int qq = 0; qq < 16; ++qq) acc[mb][nb][qq] = 0.0f;

  struct Frags {
    bf16x8 a[2], b[4];
  };
  // NMB = number of this wave's 32-row blocks that hold rows (0..2, wave-uniform). Waves of one
  // tile may run different NMB variants: every variant issues the same DMAs and barriers.
  auto read_frags = [&](auto nmb_c, const uint8_t* sa, const uint8_t* sb, int kk, Frags& f) {
    constexpr int NMB = decltype(nmb_c)::value;
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(sb + b_rd[kk][nb][0]));
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(sb + b_rd[kk][nb][1]));
      const i16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      f.b[nb] = __builtin_bit_cast(bf16x8, v);
    }
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb) f.a[mb] = *reinterpret_cast<const bf16x8*>(sa + a_rd[kk][mb]);
  };
  auto mfmas = [&](auto nmb_c, const Frags& f) {
    constexpr int NMB = decltype(nmb_c)::value;
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
        acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.b[nb], f.a[mb], acc[mb][nb], 0, 0, 0);
  };
  // One step: prefetch step kt+3 into the slot freed by step kt-1, compute step kt, then wait for
  // this wave's DMA of step kt+1 (the two later steps stay in flight) and meet at the barrier.
  // The scheduler is told to interleave: the first sub-step's fragment reads, then MFMAs with the
  // DMA issues and the second sub-step's fragment reads threaded between them.
  auto step = [&](auto nmb_c, int kt, const uint8_t* sa, const uint8_t* sb, uint8_t* pa, uint8_t* pb) {
    constexpr int NMB = decltype(nmb_c)::value;
    if constexpr (NMB == 0) {
      dma(kt + 3, pa, pb);
    } else {
      Frags f0, f1;
      read_frags(nmb_c, sa, sb, 0, f0);
      read_frags(nmb_c, sa, sb, 1, f1);
      dma(kt + 3, pa, pb);
      mfmas(nmb_c, f0);
      mfmas(nmb_c, f1);
      constexpr int R = 8 + NMB;  // fragment reads per sub-step
      constexpr int M = 4 * NMB;  // MFMAs per sub-step
      __builtin_amdgcn_sched_group_barrier(0x100, R, 0);
#pragma unroll
      for (int i = 0; i < kDmaPerWave; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x100, R > 2 * kDmaPerWave ? R - 2 * kDmaPerWave : 0, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 2 * M - kDmaPerWave, 0);
    }
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(2 * kDmaPerWave) : "memory");
  };
  auto main_loop = [&](auto nmb_c) {
    // Steps past the last real one load zeros (out-of-range offsets) and add nothing, so the step
    // count is padded to a multiple of the ring depth and the loop body has no memory branches.
    const int KT = (K + kBK - 1) / kBK;
    const int KT4 = (KT + kStages - 1) / kStages * kStages;
    dma(0, sA0, sB0);
    dma(1, sA1, sB1);
    dma(2, sA2, sB2);
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(2 * kDmaPerWave) : "memory");
    for (int kt = 0; kt < KT4; kt += kStages) {
      step(nmb_c, kt + 0, sA0, sB0, sA3, sB3);
      step(nmb_c, kt + 1, sA1, sB1, sA0, sB0);
      step(nmb_c, kt + 2, sA2, sB2, sA1, sB1);
      step(nmb_c, kt + 3, sA3, sB3, sA2, sB2);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  };
  const int wrows = row_end - (row0 + wm * 64);
  const int nmb = __builtin_amdgcn_readfirstlane(wrows <= 0 ? 0 : min(2, (wrows + 31) / 32));
  switch (nmb) {
    case 2: main_loop(std::integral_constant<int, 2>{}); break;
    case 1: main_loop(std::integral_constant<int, 1>{}); break;
    default: main_loop(std::integral_constant<int, 0>{}); break;
  }

  // ---- epilogue: lane holds row (lane & 31) of each 32-row block and, per 32-column block,
  // columns (q / 4) * 8 + (lane / 32) * 4 + q % 4 for accumulator element q
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
    const int m = row0 + wm * 64 + mb * 32 + (lane & 31);
    if (m >= row_end) continue;
    if (MODE == 0) {
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int col = nt * 128 + wn * 64 + nb * 32 + g * 8 + (lane >> 5) * 4;
          if (col >= ncols) continue;
          float hv[4];
#pragma unroll
          for (int qq = 0; qq < 4; ++qq) hv[qq] = silu_f(acc[mb][nb][g * 4 + qq]) * acc[mb][nb + 2][g * 4 + qq];
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
          const int col = nt * kBN + wn * 128 + nb * 32 + g * 8 + (lane >> 5) * 4;
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
    const int nt1 = (I + 127) / 128;
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
