// Grouped GEMMs of the expert FFN (forward and backward) over the fused expert weights.
//
// The fused layout is the one of the MindSpeed-MM InternVL3.5 practice doc (issue 625, section 2,
// model integration): gate_up [E*H, 2*I] and down [E*I, H], row-major; its section 8.3 runs the
// experts as permute -> grouped_matmul -> SwiGLU -> grouped_matmul -> unpermute, and its
// optimisation doc (section 2.1) groups the experts into one call to avoid per-expert launches.
// Gate columns are [0, I) and up columns [I, 2I) of an expert's block; h = silu(gate) * up.
//
// The grouped products of the layer, for each expert e with rows [offsets[e], offsets[e+1]) of the
// expert-grouped buffers:
//   forward   h  = silu(X_e Wg_e) * (X_e Wu_e)            (SwiGLU epilogue, optional saved g|u)
//             y  = h_e D_e
//   backward  dGU = SwiGLU'(dY_e D_e^T, g, u)              (SwiGLU-backward epilogue)
//             dX  = dGU_e GU_e^T
// run as one row-grouped kernel template (grouped_gemm_bf16_kernel); the weight gradients
//             dD_e  = h_e^T dY_e,   dGU_e = X_e^T dGU_e   (K = rows of expert e, experts without
//                                                          rows get zeros)
// have persistent kernels of their own (grouped_wgrad_res_kernel, grouped_wgrad_kernel).
//
// gfx950 design: v_mfma_f32_32x32x16_bf16, fp32 accumulation. A workgroup of 8 waves (2 per SIMD)
// computes a 256 x 256 tile; each wave 64 x 128. Both operand tiles go global -> LDS by 16-byte
// buffer DMA in 32-deep K steps. An operand whose K dimension is contiguous in memory is staged as
// a "row tile" ([rows][k], read with ds_read_b128); an operand whose M or N dimension is contiguous
// is staged in its natural layout as a "k-row tile" ([32 k][256 cols], 512-byte rows) and read with
// the LDS transpose read ds_read_b64_tr_b16, so no operand is ever repacked. In the row-grouped
// products the grouped operand A is loaded two K steps at a time (128-byte row pieces) into two
// alternating stages and the weights B one step at a time into a 4-slot ring. The MFMA takes the
// B fragment first, so a lane ends up holding four consecutive output columns of one row; the
// forward epilogues stage the tile through the (then free) operand buffers and store whole rows.
#include <algorithm>
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

constexpr int kBM = 256;            // output rows per workgroup tile
constexpr int kBN = 256;            // output columns per tile (forward GEMM-1: 128 gate + 128 up)
constexpr int kBK = 32;             // K per pipeline step
constexpr int kStages = 4;          // LDS ring depth: steps s+1..s+3 are in flight while s computes
constexpr int kGemmThreads = 512;   // 8 waves (2 per SIMD): 4 along M (64 rows each) x 2 along N (128 columns each)
constexpr int kTileA = kBM * kBK * 2;  // 16 KB per operand tile, either layout
constexpr int kTileB = kBK * kBN * 2;
constexpr int kWaves = kGemmThreads / 64;
constexpr int kDmaB = kTileB / 1024 / kWaves;  // DMA instructions (1 KB each) per wave per step, operand B
constexpr int kGemmMaxE = 1024;
constexpr int kSortMaxE = 256;  // the persistent forward lists its experts tallest first up to this many
// Row-grouped products: a tile holds up to kBMX = 320 rows, the regular 256 plus an extra band of
// up to 64 rows, so an expert with 257..320 rows (E = 128, k = 8, T = 4096 gives counts of 256 with
// a standard deviation near 16) is one tile instead of a full tile plus a nearly empty one that
// streams the same weight panel again, and the tile count stays a multiple of the CU count. The
// extra band is one or two 32-row blocks (as many as the tile's rows need), each spread over the
// eight waves against a 32-column slice per wave (16 gate + 16 up output columns with SwiGLU).
constexpr int kBMX = kBM + 64;
// The row-grouped operand A is staged two K steps at a time: [320 rows][64 k], 128-byte rows, so every
// DMA lane group fetches whole 128-byte lines of a row (one request per line instead of two 64-byte
// halves a step apart). Two such stages (40 KB each) alternate; stage s + 1 is loaded while stage s
// is read, so A arrives two K steps ahead and B, from HBM, keeps its three-step lead in a 4-slot ring.
constexpr int kBK2 = 2 * kBK;                              // K depth of one A stage
constexpr int kTileA2 = kBMX * kBK2 * 2;                   // 40 KB per A stage
constexpr int kDmaA2 = kBM * kBK2 * 2 / 1024 / kWaves;     // 4 DMA instructions per wave per A stage (+1 band)

// LDS swizzles, applied when choosing which global chunk each DMA lane fetches. They keep the
// fragment reads free of bank conflicts whether the LDS serves 128 or 256 bytes per clock:
//  - row tile (64-byte rows): 16-byte chunk c (8 k) of row r lives at chunk c ^ g(r) with
//    g(r) = ((r >> 1) ^ (r >> 2)) & 3; the 8 (or 16) consecutive rows read together at one logical
//    chunk then land on distinct banks;
//  - k-row tile (512-byte k-rows): 16-byte chunk c (8 columns) of k-row r lives at chunk c ^ f(r) with
//    f(r) = 4 (r & 3) + 2 ((r >> 1) & 1); the transpose read of four consecutive k-rows x 32 bytes
//    (x 64 bytes for two lane groups) then lands on distinct banks. f is even and below 16, so a
//    16-byte pair stays adjacent and the gate / up halves of a forward GEMM-1 row never mix.
__device__ __forceinline__ int swz_a(int r) { return ((r >> 1) ^ (r >> 2)) & 3; }
__device__ __forceinline__ int swz_b(int r) { return 4 * (r & 3) + 2 * ((r >> 1) & 1); }
// A stage (128-byte rows): chunk c of row r lives at chunk c ^ h(r), h(r) = (r & 7) ^ ((r >> 3) & 1). Eight
// consecutive rows (one 128-byte LDS cycle) get eight distinct chunks; of sixteen (one 256-byte cycle),
// the even and the odd rows each get eight distinct chunks, and the two parities sit in opposite halves
// of the 256 bytes. Chunks 0-3 (the stage's first K step) map to 0-3 or 4-7 as a block per row, so the
// second step's address is the first's with bit 6 flipped.
__device__ __forceinline__ int swz_a2(int r) { return (r & 7) ^ ((r >> 3) & 1); }

// sigmoid with the hardware reciprocal (1 ulp) instead of an IEEE division (about ten instructions
// each): the results are rounded to bf16, and the division sequence was most of the epilogue's time
__device__ __forceinline__ float sigmoid_f(float g) { return __builtin_amdgcn_rcpf(1.0f + __expf(-g)); }
__device__ __forceinline__ float silu_f(float g) { return g * sigmoid_f(g); }

// Row-grouped schedule: linear workgroup index -> (expert, row range, column tile). Returns false
// when the workgroup has no tile (the grid is sized for the worst case over any row distribution).
struct TileInfo {
  int e, row0, row_end, nt;
};

// An expert with c rows gets ceil(c / bm) tiles of near-equal height.

template <int NT>
__device__ __forceinline__ bool tile_of_block(const int32_t* __restrict__ offsets, int E, int bm, int ntiles_n,
                                              int* s_pref, int* s_wtot, int* s_e, TileInfo& ti) {
  const int tid = threadIdx.x;
  const int b = blockIdx.x;
  // each thread keeps the offsets it loaded; the one whose expert owns the tile hands them over
  // through LDS (reloading them from global memory would add a dependent round trip per tile)
  constexpr int PER = (kGemmMaxE + NT - 1) / NT;
  int my_o0[PER], my_n[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int e = tid + i * NT;
    my_o0[i] = e < E ? offsets[e] : 0;
    my_n[i] = e < E ? offsets[e + 1] - my_o0[i] : 0;
    if (e < E) s_pref[e] = my_n[i] > 0 ? (my_n[i] + bm - 1) / bm : 0;
  }
  __syncthreads();
  block_exclusive_scan<NT>(s_pref, E, s_wtot);
  // The grid is sized for the worst row distribution; only the first `total` tiles exist. Blocks
  // are dealt round-robin over the 8 XCDs, so block b runs on XCD b % 8: give XCD x the
  // contiguous tile range [x Q, (x+1) Q) with Q = ceil(total / 8), which keeps the column tiles
  // of one row tile (and the row tiles of one expert) in one XCD's L2 and uses every XCD.
  const int total = s_pref[E] * ntiles_n;
  const int Q = (total + 7) >> 3;
  const int L = (b & 7) * Q + (b >> 3);
  if ((b >> 3) >= Q || L >= total) return false;
  const int mt_g = L / ntiles_n;
  ti.nt = L - mt_g * ntiles_n;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int e = tid + i * NT;
    if (e < E && s_pref[e] <= mt_g && mt_g < s_pref[e + 1]) {
      s_e[0] = e;
      s_e[1] = my_o0[i];
      s_e[2] = my_n[i];
    }
  }
  __syncthreads();
  ti.e = __builtin_amdgcn_readfirstlane(s_e[0]);
  const int p0 = __builtin_amdgcn_readfirstlane(s_pref[ti.e]), p1 = __builtin_amdgcn_readfirstlane(s_pref[ti.e + 1]);
  const int j = mt_g - p0, nte = p1 - p0;
  const int o0 = __builtin_amdgcn_readfirstlane(s_e[1]), c = __builtin_amdgcn_readfirstlane(s_e[2]);
  ti.row0 = __builtin_amdgcn_readfirstlane(o0 + (int)((int64_t)j * c / nte));
  ti.row_end = __builtin_amdgcn_readfirstlane(o0 + (int)((int64_t)(j + 1) * c / nte));
  return true;
}


enum { kEpiSwiglu = 0, kEpiStore = 1, kEpiSwigluBwd = 2 };

// Arguments of one grouped product C = A B (per expert). Sizes in elements.
struct GemmArgs {
  const uint16_t* A;   // row-grouped operand (row-grouped products) or P, whose rows are K (weight gradients)
  const uint16_t* B;   // weights (row-grouped products) or Q (weight gradients)
  uint16_t* C;
  const uint16_t* gu;  // saved g|u [rows, 2*N] read by the SwiGLU-backward epilogue
  uint16_t* gu_out;    // optional g|u written by the SwiGLU epilogue [rows, 2*N]
  const int32_t* offsets;
  const int32_t* a_slot;  // optional (row-grouped A): A row r is row a_slot[r] / a_div of A, i.e. the
  int a_div;              // grouped rows are gathered from the token matrix through the slot map
  int E;
  int M, N, K;         // row-grouped: N output columns, K (M = tokens when gathering); weight gradients: M, N per expert
  int lda, ldb, ldc;
  int64_t b_expert;    // row-grouped: elements between two experts' weight blocks
  int64_t c_expert;    // weight gradients: elements between two experts' output blocks
  int b_rows;          // row-grouped: rows of one expert's weight block (K for a k-row B, N for a row B)
  int ntiles_m, ntiles_n;
};

// dL/dh -> (dL/dg, dL/du) for four consecutive columns of row m, with s = sigmoid(g):
// dL/dg = v * u * s * (1 + g (1 - s)), dL/du = v * g * s; writes dG | dU into C (row stride ldc).
__device__ __forceinline__ void store_swiglu_bwd(const GemmArgs& g, uint16_t* cbase, int64_t m, int col,
                                                 const float* v) {
  const uint16_t* gr = g.gu + m * 2 * g.N;
  const uint2 gp = *reinterpret_cast<const uint2*>(gr + col);
  const uint2 up = *reinterpret_cast<const uint2*>(gr + g.N + col);
  const float gv[4] = {bf16_to_f32(gp.x & 0xffffu), bf16_to_f32(gp.x >> 16), bf16_to_f32(gp.y & 0xffffu),
                       bf16_to_f32(gp.y >> 16)};
  const float uv[4] = {bf16_to_f32(up.x & 0xffffu), bf16_to_f32(up.x >> 16), bf16_to_f32(up.y & 0xffffu),
                       bf16_to_f32(up.y >> 16)};
  float dg[4], du[4];
#pragma unroll
  for (int qq = 0; qq < 4; ++qq) {
    const float sg = sigmoid_f(gv[qq]);
    dg[qq] = v[qq] * uv[qq] * sg * (1.0f + gv[qq] * (1.0f - sg));
    du[qq] = v[qq] * gv[qq] * sg;
  }
  uint16_t* dr = cbase + m * g.ldc;
  *reinterpret_cast<uint2*>(dr + col) = make_uint2(pack_bf16x2(dg[0], dg[1]), pack_bf16x2(dg[2], dg[3]));
  *reinterpret_cast<uint2*>(dr + g.N + col) = make_uint2(pack_bf16x2(du[0], du[1]), pack_bf16x2(du[2], du[3]));
}

// Epilogue of extra-band block xb (row-grouped products): lane holds tile row 256 + 32 xb + (lane & 31)
// and, for accumulator element q, slice column (q / 4) * 8 + (lane / 32) * 4 + q % 4: gate columns
// 0..15 and up columns 16..31 of the SwiGLU slice g0, else columns wn*128 + wm*32 + 0..31.
template <int EPI>
__device__ __forceinline__ void store_extra(const GemmArgs& g, const f32x16& acc, int xb, int m0, int mvalid, int n0,
                                            int nt, int g0, int wm, int wn, int lane) {
  const int mloc = kBM + xb * 32 + (lane & 31);
  if (mloc >= mvalid) return;
  const int64_t m = m0 + mloc;
  if constexpr (EPI == kEpiSwiglu) {
#pragma unroll
    for (int gq = 0; gq < 2; ++gq) {
      const int col = nt * 128 + g0 + gq * 8 + (lane >> 5) * 4;
      if (col >= g.N) continue;
      float hv[4];
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) hv[qq] = silu_f(acc[gq * 4 + qq]) * acc[(gq + 2) * 4 + qq];
      *reinterpret_cast<uint2*>(g.C + m * g.ldc + col) = make_uint2(pack_bf16x2(hv[0], hv[1]), pack_bf16x2(hv[2], hv[3]));
      if (g.gu_out) {
        uint16_t* gs = g.gu_out + m * 2 * g.N;
        *reinterpret_cast<uint2*>(gs + col) =
            make_uint2(pack_bf16x2(acc[gq * 4 + 0], acc[gq * 4 + 1]), pack_bf16x2(acc[gq * 4 + 2], acc[gq * 4 + 3]));
        *reinterpret_cast<uint2*>(gs + g.N + col) = make_uint2(pack_bf16x2(acc[gq * 4 + 8], acc[gq * 4 + 9]),
                                                               pack_bf16x2(acc[gq * 4 + 10], acc[gq * 4 + 11]));
      }
    }
  } else {
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      const int col = n0 + wn * 128 + wm * 32 + gq * 8 + (lane >> 5) * 4;
      if (col >= g.N) continue;
      float v[4];
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) v[qq] = acc[gq * 4 + qq];
      if constexpr (EPI == kEpiSwigluBwd) {
        store_swiglu_bwd(g, g.C, m, col, v);
      } else {
        *reinterpret_cast<uint2*>(g.C + m * g.ldc + col) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
      }
    }
  }
}

// A_ROWS: A is a row tile (K contiguous) - else a k-row tile (M contiguous).
// B_ROWS: B is a row tile (K contiguous) - else a k-row tile (N contiguous).
template <bool A_ROWS, bool B_ROWS, int EPI>
__global__ __launch_bounds__(kGemmThreads) void grouped_gemm_bf16_kernel(const GemmArgs g) {
  static_assert(A_ROWS, "the row-grouped operand is staged as a row tile");
  // one LDS object per A stage and per B ring slot, so that the compiler can tell a DMA into one
  // buffer from reads of another
  __shared__ __attribute__((aligned(1024))) uint8_t sA0[kTileA2], sA1[kTileA2];
  __shared__ __attribute__((aligned(1024))) uint8_t sB0[kTileB], sB1[kTileB], sB2[kTileB], sB3[kTileB];
  __shared__ int s_pref[kGemmMaxE + 1];
  __shared__ int s_wtot[kGemmThreads / kWave];
  __shared__ int s_e[3];  // the tile's expert, its first row and its row count

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int wm = (wave >> 1) & 3, wn = wave & 1;  // a tile with few rows still spreads over two SIMDs

  // ---- tile, rows and K of this workgroup
  int e, m0, n0, mvalid, K, nt;
  const uint16_t* abase;
  const uint16_t* bbase;
  int a_records, b_records;
  {
    TileInfo ti;
    if (!tile_of_block<kGemmThreads>(g.offsets, g.E, kBMX, g.ntiles_n, s_pref, s_wtot, s_e, ti)) return;
    e = ti.e;
    m0 = ti.row0;
    mvalid = ti.row_end - ti.row0;
    nt = ti.nt;
    n0 = nt * kBN;
    K = g.K;
    if (g.a_slot) {                          // gathered: rows come from the token matrix
      abase = g.A;
      a_records = g.M * g.lda * 2;           // g.M = tokens
    } else {
      abase = g.A + (int64_t)m0 * g.lda;     // rows [row0, row_end) of the grouped operand
      a_records = mvalid * g.lda * 2;
    }
    bbase = g.B + (int64_t)e * g.b_expert;   // expert e's weight block
    b_records = g.b_rows * g.ldb * 2;
  }
  const __amdgpu_buffer_rsrc_t rsA =
      __builtin_amdgcn_make_buffer_rsrc((void*)abase, (short)0, a_records, kBufferWord3);
  const __amdgpu_buffer_rsrc_t rsB =
      __builtin_amdgcn_make_buffer_rsrc((void*)bbase, (short)0, b_records, kBufferWord3);

  // ---- DMA lanes (offsets in bytes from the descriptor base, for k0 = 0)
  // A stage: instruction i fills rows (kDmaA2 w + i) * 8 .. +8, eight lanes (16-byte chunks) per row.
  // B row tile: instruction i fills rows (kDmaB w + i) * 16 .. +16, four lanes per row.
  // B k-row tile: instruction i fills k-rows (kDmaB w + i) * 2 .. +2, 32 lanes per row.
  // A: a row past the tile gets an offset at or past the descriptor's end, so every stage loads zeros
  // for it (rows of the grouped operand past the tile are past their descriptor already). The lane's
  // chunk depends only on the lane and on i % 2 (rows 8 i .. 8 i + 7 share h(r) up to bit 0).
  int a_off[kDmaA2], b_off[kDmaB];
  bool b_ok[kDmaB];
  int b_kc[kDmaB];  // row tiles: k offset of the lane's chunk (for the K tail)
  const int a_c0 = (lane & 7) ^ swz_a2(lane >> 3);
  const int a_kc[2] = {a_c0 * 8, (a_c0 ^ 1) * 8};
#pragma unroll
  for (int i = 0; i < kDmaA2; ++i) {
    const int r = (wave * kDmaA2 + i) * 8 + (lane >> 3);
    const int c = a_c0 ^ (i & 1);
    if (g.a_slot)
      a_off[i] = r < mvalid ? (g.a_slot[m0 + r] / g.a_div * g.lda + c * 8) * 2 : a_records;
    else
      a_off[i] = (r * g.lda + c * 8) * 2;
  }
#pragma unroll
  for (int i = 0; i < kDmaB; ++i) {
    if constexpr (B_ROWS) {
      const int r = (wave * kDmaB + i) * 16 + (lane >> 2);
      const int c = (lane & 3) ^ swz_a(r);
      const int n = n0 + r;
      b_kc[i] = c * 8;
      b_ok[i] = n < g.N;
      b_off[i] = ((b_ok[i] ? n : 0) * g.ldb + c * 8) * 2;
    } else {
      const int kr = (wave * kDmaB + i) * 2 + (lane >> 5);
      const int cb = (lane & 31) ^ swz_b(kr);
      int col;
      if constexpr (EPI == kEpiSwiglu) {  // 128 gate columns then the matching 128 up columns
        const int j = nt * 128 + (cb & 15) * 8;
        b_ok[i] = j < g.N;
        col = (cb < 16 ? 0 : g.N) + (b_ok[i] ? j : 0);
      } else {
        col = n0 + cb * 8;
        b_ok[i] = col < g.N;
        if (!b_ok[i]) col = 0;
      }
      b_kc[i] = 0;
      b_off[i] = (kr * g.ldb + col) * 2;
    }
  }
  // extra-band rows 256 + 8 w .. + 7 of an A stage: one DMA instruction per wave
  const int x_r = kBM + wave * 8 + (lane >> 3);
  const int xch = (lane & 7) ^ swz_a2(x_r);
  const int x_kc = xch * 8;
  const int x_off = !g.a_slot ? (x_r * g.lda + xch * 8) * 2
                    : x_r < mvalid ? (g.a_slot[m0 + x_r] / g.a_div * g.lda + xch * 8) * 2 : a_records;
  // A stage st (K 64 st .. 64 st + 63 of the tile's rows) into buffer sa; the band rows only in tiles
  // that have them
  auto dma_a = [&](auto x_c, int st, uint8_t* sa) {
    const int k0 = st * kBK2;
    if constexpr (decltype(x_c)::value > 0) {
      const int off = k0 + x_kc < K ? (int)((uint32_t)x_off + (uint32_t)(k0 * 2)) : kOutOfRange;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsA, (lds_void*)(sa + kBM * kBK2 * 2 + wave * 1024), 16, off, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < kDmaA2; ++i) {
      // unsigned: a missing gathered row's offset is the descriptor's size, which k0 may push past 2^31
      const int off = k0 + a_kc[i & 1] < K ? (int)((uint32_t)a_off[i] + (uint32_t)(k0 * 2)) : kOutOfRange;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsA, (lds_void*)(sa + (wave * kDmaA2 + i) * 1024), 16, off, 0, 0, 0);
    }
  };
  // B step kt (K 32 kt .. 32 kt + 31) into ring slot sb
  auto dma_b = [&](int kt, uint8_t* sb) {
    const int k0 = kt * kBK;
#pragma unroll
    for (int i = 0; i < kDmaB; ++i) {
      int off;
      if constexpr (B_ROWS)
        off = (b_ok[i] && k0 + b_kc[i] < K) ? b_off[i] + k0 * 2 : kOutOfRange;
      else
        off = b_ok[i] ? b_off[i] + k0 * g.ldb * 2 : kOutOfRange;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsB, (lds_void*)(sb + (wave * kDmaB + i) * 1024), 16, off, 0, 0, 0);
    }
  };

  // ---- fragment addresses. A block mb: rows wm*64 + mb*32 + (lane & 31), one ds_read_b128 at
  // k = kk*16 + (lane/32)*8 of the stage's first K step (the second step: address bit 6 flipped).
  // B block nb: 32 tile columns from bcol[nb]. Row tile: one ds_read_b128 at k = kk*16 + (lane/32)*8.
  // k-row tile: two transpose reads at k = kk*16 + (lane/32)*8 + {0..3, 4..7}.
  int bcol[4];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb)
    bcol[nb] = EPI == kEpiSwiglu ? ((nb >> 1) * 128 + wn * 64 + (nb & 1) * 32) : (wn * 128 + nb * 32);
  const int q = lane >> 4, sl = lane & 15;
  auto row_rd = [&](int r, int kk) {
    const int c = kk * 2 + (lane >> 5);
    return r * 64 + ((c ^ swz_a(r)) << 4);
  };
  auto arow_rd = [&](int r, int kk) {
    const int c = kk * 2 + (lane >> 5);
    return r * (kBK2 * 2) + ((c ^ swz_a2(r)) << 4);
  };
  auto krow_rd = [&](int col32, int kk, int ri) {
    const int kr = kk * 16 + (q >> 1) * 8 + ri * 4 + (sl >> 2);
    const int col = col32 + (q & 1) * 16 + 4 * (sl & 3);
    return kr * 512 + (((col >> 3) ^ swz_b(kr)) << 4) + (col & 7) * 2;
  };
  int a_rd[2][2][2], b_rd[2][4][2];
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      a_rd[kk][mb][0] = arow_rd(wm * 64 + mb * 32 + (lane & 31), kk);
      a_rd[kk][mb][1] = 0;
    }
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      if constexpr (B_ROWS) {
        b_rd[kk][nb][0] = row_rd(bcol[nb] + (lane & 31), kk);
        b_rd[kk][nb][1] = 0;
      } else {
        b_rd[kk][nb][0] = krow_rd(bcol[nb], 0, 0);  // + kk * 8192 at the read
        b_rd[kk][nb][1] = 0;
      }
    }
  }

  // Extra band (row-grouped products): A blocks = tile rows 256..287 and 288..319; B block = this wave's
  // 32-column slice: columns wn*128 + wm*32 of its half, or for SwiGLU the 16 gate columns
  // g0 .. g0+15 (lanes with column index < 16) and the matching 16 up columns, g0 = (wn*4+wm)*16.
  const int g0 = (wn * 4 + wm) * 16;
  // (the second band block's addresses are the first's + 32 rows: the row swizzle repeats every 16 rows)
  int xa_rd[2], xb_rd[2][2];
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
    xa_rd[kk] = arow_rd(kBM + (lane & 31), kk);
    if constexpr (B_ROWS) {
      xb_rd[kk][0] = row_rd(wn * 128 + wm * 32 + (lane & 31), kk);
      xb_rd[kk][1] = 0;
    } else if constexpr (EPI == kEpiSwiglu) {
#pragma unroll
      for (int ri = 0; ri < 2; ++ri) {
        const int kr = (q >> 1) * 8 + (sl >> 2);  // k-row of kk = 0, ri = 0 (+ kk * 8192 at the read)
        const int col = (q & 1) * 128 + g0 + 4 * (sl & 3);
        xb_rd[kk][ri] = ri ? 0 : kr * 512 + (((col >> 3) ^ swz_b(kr)) << 4) + (col & 7) * 2;
      }
    } else {
      xb_rd[kk][0] = krow_rd(wn * 128 + wm * 32, 0, 0);
      xb_rd[kk][1] = 0;
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
    bf16x8 a[2], b[4], xa[2], xb;
  };
  // k-row tiles: the swizzle depends on the k-row mod 4 only, so the lane's address for k-rows +4
  // (second half of its 8 k) is +2048 bytes and for sub-step kk = 1 (+16 k-rows) +8192: one base
  // register per 32-column block, the rest in the instructions' offset fields
  auto frag = [&](const uint8_t* base, const int* rd, bool rows, int kk) -> bf16x8 {
    if (rows) return *reinterpret_cast<const bf16x8*>(base + rd[0]);
    const uint8_t* p = base + rd[0] + kk * 8192;
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p);
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p + 2048));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  // NMB = number of this wave's 32-row blocks that hold rows (0..2, wave-uniform); NX = number of
  // extra-band blocks of the tile (0..2). Waves of one tile may run different NMB variants: every
  // variant issues the same DMAs and barriers.
  // AX: 0 in the first K step of an A stage, 64 (address bit 6) in the second
  auto read_frags = [&](auto nmb_c, auto nx_c, const uint8_t* sa, const uint8_t* sb, int kk, int AX, Frags& f) {
    constexpr int NMB = decltype(nmb_c)::value;
    constexpr int NX = decltype(nx_c)::value;
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) f.b[nb] = frag(sb, b_rd[kk][nb], B_ROWS, kk);
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb) f.a[mb] = *reinterpret_cast<const bf16x8*>(sa + (a_rd[kk][mb][0] ^ AX));
    if constexpr (NX > 0) {
#pragma unroll
      for (int xb = 0; xb < NX; ++xb)
        f.xa[xb] = *reinterpret_cast<const bf16x8*>(sa + xb * 32 * kBK2 * 2 + (xa_rd[kk] ^ AX));
      f.xb = frag(sb, xb_rd[kk], B_ROWS, kk);
    }
  };
  auto mfmas = [&](auto nmb_c, auto nx_c, const Frags& f, f32x16* acc_x) {
    constexpr int NMB = decltype(nmb_c)::value;
    constexpr int NX = decltype(nx_c)::value;
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
        acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.b[nb], f.a[mb], acc[mb][nb], 0, 0, 0);
#pragma unroll
    for (int xb = 0; xb < NX; ++xb)
      acc_x[xb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.xb, f.xa[xb], acc_x[xb], 0, 0, 0);
  };
  // One step kt (P = kt % 2: first or second K step of the A stage in sa): at P = 0 load the next A
  // stage into pa, the buffer every wave finished with at the last barrier; load B step kt + 3 into
  // the slot freed by step kt - 1; compute step kt; then wait for this wave's DMAs of step kt + 1
  // (after P = 1 that includes the A stage issued one step earlier: two steps of lead for A, three
  // for B) and meet at the barrier. The scheduler is told to interleave: the first sub-step's
  // fragment reads, then MFMAs with the DMA issues and the second sub-step's reads between them.
  auto step = [&](auto nmb_c, auto x_c, auto p_c, f32x16* acc_x, int kt, const uint8_t* sa, const uint8_t* sb,
                  uint8_t* pa, uint8_t* pb) {
    constexpr int NMB = decltype(nmb_c)::value;
    constexpr int NX = decltype(x_c)::value;
    constexpr int P = decltype(p_c)::value;
    constexpr int X = NX > 0 ? 1 : 0;
    constexpr int DA = kDmaA2 + X;                    // DMAs of an A stage
    constexpr int DPW = (P == 0 ? DA : 0) + kDmaB;    // DMAs issued in this step
    constexpr int AX = P * 64;
    auto issue = [&]() {
      if constexpr (P == 0) dma_a(x_c, kt / 2 + 1, pa);
      dma_b(kt + 3, pb);
    };
    if constexpr (NMB == 0) {
      issue();
    } else if constexpr (NX > 0) {
      // band blocks: the sub-steps one after the other, so that one set of fragments is live
      // (both sets with the band's accumulators do not fit in the register budget)
      Frags f;
      read_frags(nmb_c, x_c, sa, sb, 0, AX, f);
      issue();
      mfmas(nmb_c, x_c, f, acc_x);
      read_frags(nmb_c, x_c, sa, sb, 1, AX, f);
      mfmas(nmb_c, x_c, f, acc_x);
    } else {
      Frags f0, f1;
      read_frags(nmb_c, x_c, sa, sb, 0, AX, f0);
      read_frags(nmb_c, x_c, sa, sb, 1, AX, f1);
      issue();
      mfmas(nmb_c, x_c, f0, acc_x);
      mfmas(nmb_c, x_c, f1, acc_x);
      constexpr int R = (B_ROWS ? 4 : 8) + (A_ROWS ? 1 : 2) * NMB + NX + X * (B_ROWS ? 1 : 2);  // LDS reads per sub-step
      constexpr int M = 4 * NMB + NX;                                                          // MFMAs per sub-step
      __builtin_amdgcn_sched_group_barrier(0x100, R, 0);
#pragma unroll
      for (int i = 0; i < DPW; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x100, R > 2 * DPW ? R - 2 * DPW : 0, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 2 * M > DPW ? 2 * M - DPW : 0, 0);
    }
    // ops issued after the B DMA of step kt + 1: P = 0: B kt + 2, then this step's A stage and B kt + 3;
    // P = 1: B kt + 2 and B kt + 3 (the A stage of step kt + 1 went out just before B kt + 2)
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(P == 0 ? 2 * kDmaB + DA : 2 * kDmaB) : "memory");
  };
  auto main_loop = [&](auto nmb_c, auto x_c) {
    // Steps past the last real one load zeros (out-of-range offsets) and add nothing, so the step
    // count is padded to a multiple of the ring depth and the loop body has no memory branches.
    const int KT = (K + kBK - 1) / kBK;
    const int KT4 = (KT + kStages - 1) / kStages * kStages;
    f32x16 acc_x[2];
#pragma unroll
    for (int xb = 0; xb < 2; ++xb)
#pragma unroll
      for (int qq = 0; qq < 16; ++qq) acc_x[xb][qq] = 0.0f;
    using P0 = std::integral_constant<int, 0>;
    using P1 = std::integral_constant<int, 1>;
    dma_a(x_c, 0, sA0);
    dma_b(0, sB0);
    dma_b(1, sB1);
    dma_b(2, sB2);
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(2 * kDmaB) : "memory");  // A stage 0 and B step 0
    for (int kt = 0; kt < KT4; kt += kStages) {
      step(nmb_c, x_c, P0{}, acc_x, kt + 0, sA0, sB0, sA1, sB3);
      step(nmb_c, x_c, P1{}, acc_x, kt + 1, sA0, sB1, nullptr, sB0);
      step(nmb_c, x_c, P0{}, acc_x, kt + 2, sA1, sB2, sA0, sB1);
      step(nmb_c, x_c, P1{}, acc_x, kt + 3, sA1, sB3, nullptr, sB2);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#pragma unroll
    for (int xb = 0; xb < decltype(x_c)::value; ++xb)
      store_extra<EPI>(g, acc_x[xb], xb, m0, mvalid, n0, nt, g0, wm, wn, lane);
  };
  const int wrows = mvalid - wm * 64;
  const int nmb = __builtin_amdgcn_readfirstlane(wrows <= 0 ? 0 : min(2, (wrows + 31) / 32));
  using F = std::integral_constant<int, 0>;
  if (mvalid > kBM) {  // the extra band holds rows: every regular band is full
    if (mvalid > kBM + 32)
      main_loop(std::integral_constant<int, 2>{}, std::integral_constant<int, 2>{});
    else
      main_loop(std::integral_constant<int, 2>{}, std::integral_constant<int, 1>{});
  } else {
    switch (nmb) {
      case 2: main_loop(std::integral_constant<int, 2>{}, F{}); break;
      case 1: main_loop(std::integral_constant<int, 1>{}, F{}); break;
      default: main_loop(std::integral_constant<int, 0>{}, F{}); break;
    }
  }

  // ---- epilogue: lane holds output row (lane & 31) of each 32-row block and, per 32-column
  // block, columns (q / 4) * 8 + (lane / 32) * 4 + q % 4 for accumulator element q
  if constexpr (EPI == kEpiStore) {
    // Staged: after the K loop every operand buffer is free, so the tile's 256 regular rows go to LDS
    // as bf16 (32-row block j in 16 KB block j: the halves of sA0 and sA1, then sB0..sB3; 16-byte
    // chunk c of row r at chunk c ^ r) and out as whole 512-byte rows, two rows per 1 KB store. Straight from the
    // accumulators each 8-byte-per-lane store touches 32 rows, and with every CU reaching its
    // epilogue at about the same time that was a quarter of the down product's tile time. The
    // stores are plain: the combine reads y right after, partly from the last-level cache (with
    // non-temporal stores the down product was 5 us faster and the combine 9 us slower).
    auto blk = [&](int j) -> uint8_t* {
      return j == 0 ? sA0 : j == 1 ? sA0 + 16384 : j == 2 ? sA1 : j == 3 ? sA1 + 16384 : j == 4 ? sB0 : j == 5 ? sB1 : j == 6 ? sB2 : sB3;
    };
    asm volatile("s_barrier" ::: "memory");  // every wave is done with the operand buffers
    const int lr = lane & 31;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      uint8_t* st = blk(wm * 2 + mb) + lr * 512 + (lane >> 5) * 8;
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          const int chunk = (wn * 16 + nb * 4 + gq) ^ lr;
          *reinterpret_cast<uint2*>(st + (chunk << 4)) =
              make_uint2(pack_bf16x2(acc[mb][nb][gq * 4 + 0], acc[mb][nb][gq * 4 + 1]),
                         pack_bf16x2(acc[mb][nb][gq * 4 + 2], acc[mb][nb][gq * 4 + 3]));
        }
    }
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    const uint8_t* src = blk(wave);
    const int c = lane & 31;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int r = 2 * i + (lane >> 5);
      const int mloc = wave * 32 + r, col = n0 + c * 8;
      if (mloc < mvalid && col < g.N) {
        const uint4 v = *reinterpret_cast<const uint4*>(src + r * 512 + ((c ^ r) << 4));
        *reinterpret_cast<uint4*>(g.C + (int64_t)(m0 + mloc) * g.ldc + col) = v;
      }
    }
    return;
  }
  if constexpr (EPI == kEpiSwiglu) {
    // Staged as above: h of the 256 regular rows (128 columns, 256-byte rows) goes to LDS (32-row
    // block j in the first 8 KB of 16 KB block j; 16-byte chunk c of row r at chunk c ^ (r & 15)) and out as
    // whole rows, four per 1 KB store; the saved g | u (training only) are stored straight
    auto blk = [&](int j) -> uint8_t* {
      return j == 0 ? sA0 : j == 1 ? sA0 + 16384 : j == 2 ? sA1 : j == 3 ? sA1 + 16384 : j == 4 ? sB0 : j == 5 ? sB1 : j == 6 ? sB2 : sB3;
    };
    asm volatile("s_barrier" ::: "memory");  // every wave is done with the operand buffers
    const int lr = lane & 31;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      uint8_t* st = blk(wm * 2 + mb) + lr * 256 + (lane >> 5) * 8;
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          float hv[4];
#pragma unroll
          for (int qq = 0; qq < 4; ++qq) hv[qq] = silu_f(acc[mb][nb][gq * 4 + qq]) * acc[mb][nb + 2][gq * 4 + qq];
          const int chunk = (wn * 8 + nb * 4 + gq) ^ (lr & 15);
          *reinterpret_cast<uint2*>(st + (chunk << 4)) = make_uint2(pack_bf16x2(hv[0], hv[1]), pack_bf16x2(hv[2], hv[3]));
        }
      if (g.gu_out) {
        const int mloc = wm * 64 + mb * 32 + lr;
        if (mloc < mvalid) {
          uint16_t* gs = g.gu_out + (int64_t)(m0 + mloc) * 2 * g.N;
#pragma unroll
          for (int nb = 0; nb < 2; ++nb)
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
              const int col = nt * 128 + wn * 64 + nb * 32 + gq * 8 + (lane >> 5) * 4;
              if (col >= g.N) continue;
              *reinterpret_cast<uint2*>(gs + col) =
                  make_uint2(pack_bf16x2(acc[mb][nb][gq * 4 + 0], acc[mb][nb][gq * 4 + 1]),
                             pack_bf16x2(acc[mb][nb][gq * 4 + 2], acc[mb][nb][gq * 4 + 3]));
              *reinterpret_cast<uint2*>(gs + g.N + col) =
                  make_uint2(pack_bf16x2(acc[mb][nb + 2][gq * 4 + 0], acc[mb][nb + 2][gq * 4 + 1]),
                             pack_bf16x2(acc[mb][nb + 2][gq * 4 + 2], acc[mb][nb + 2][gq * 4 + 3]));
            }
        }
      }
    }
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    const uint8_t* src = blk(wave);
    const int c = lane & 15;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = 4 * i + (lane >> 4);
      const int mloc = wave * 32 + r, col = nt * 128 + c * 8;
      if (mloc < mvalid && col < g.N) {
        const uint4 v = *reinterpret_cast<const uint4*>(src + r * 256 + ((c ^ (r & 15)) << 4));
        typedef __attribute__((ext_vector_type(4))) unsigned int v4u;
        __builtin_nontemporal_store(v4u{v.x, v.y, v.z, v.w}, reinterpret_cast<v4u*>(g.C + (int64_t)(m0 + mloc) * g.ldc + col));
      }
    }
    return;
  }
  // SwiGLU backward: dG | dU from the accumulators and the saved g, u (read in 8-byte pieces), staged
  // like the plain store, in two rounds (accumulator half mb = 0, then 1): each wave writes dG of its
  // 32 rows into 16 KB block wm and dU into block 4 + wm, then wave w copies block w out as whole
  // 512-byte rows (dG into columns [0, N), dU into [N, 2N)).
  if constexpr (EPI == kEpiSwigluBwd) {
    auto blk = [&](int j) -> uint8_t* {
      return j == 0 ? sA0 : j == 1 ? sA0 + 16384 : j == 2 ? sA1 : j == 3 ? sA1 + 16384 : j == 4 ? sB0 : j == 5 ? sB1 : j == 6 ? sB2 : sB3;
    };
    const int lr = lane & 31, c = lane & 31;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      asm volatile("s_barrier" ::: "memory");  // the operand buffers (or the previous round's rows) are free
      const int mloc = wm * 64 + mb * 32 + lr;
      const uint16_t* gr = g.gu + (int64_t)(m0 + min(mloc, max(mvalid - 1, 0))) * 2 * g.N;
      uint8_t* sg_ = blk(wm) + lr * 512 + (lane >> 5) * 8;
      uint8_t* su_ = blk(4 + wm) + lr * 512 + (lane >> 5) * 8;
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          const int col = n0 + wn * 128 + nb * 32 + gq * 8 + (lane >> 5) * 4;
          uint2 gp = make_uint2(0u, 0u), up = make_uint2(0u, 0u);
          if (mloc < mvalid && col < g.N) {
            gp = *reinterpret_cast<const uint2*>(gr + col);
            up = *reinterpret_cast<const uint2*>(gr + g.N + col);
          }
          const float gv[4] = {bf16_to_f32(gp.x & 0xffffu), bf16_to_f32(gp.x >> 16), bf16_to_f32(gp.y & 0xffffu),
                               bf16_to_f32(gp.y >> 16)};
          const float uv[4] = {bf16_to_f32(up.x & 0xffffu), bf16_to_f32(up.x >> 16), bf16_to_f32(up.y & 0xffffu),
                               bf16_to_f32(up.y >> 16)};
          float dg[4], du[4];
#pragma unroll
          for (int qq = 0; qq < 4; ++qq) {
            const float v = acc[mb][nb][gq * 4 + qq];
            const float sg = sigmoid_f(gv[qq]);
            dg[qq] = v * uv[qq] * sg * (1.0f + gv[qq] * (1.0f - sg));
            du[qq] = v * gv[qq] * sg;
          }
          const int chunk = (wn * 16 + nb * 4 + gq) ^ lr;
          *reinterpret_cast<uint2*>(sg_ + (chunk << 4)) = make_uint2(pack_bf16x2(dg[0], dg[1]), pack_bf16x2(dg[2], dg[3]));
          *reinterpret_cast<uint2*>(su_ + (chunk << 4)) = make_uint2(pack_bf16x2(du[0], du[1]), pack_bf16x2(du[2], du[3]));
        }
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      const uint8_t* src = blk(wave);
      const int wb = wave & 3, coff = wave < 4 ? 0 : g.N;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int r = 2 * i + (lane >> 5);
        const int ml = wb * 64 + mb * 32 + r, col = n0 + c * 8;
        if (ml < mvalid && col < g.N) {
          const uint4 v = *reinterpret_cast<const uint4*>(src + r * 512 + ((c ^ r) << 4));
          *reinterpret_cast<uint4*>(g.C + (int64_t)(m0 + ml) * g.ldc + coff + col) = v;
        }
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    }
  }
}


// ---------------------------------------------------------------------------------------------
// Weight gradients, persistent. dW_e = P_e^T Q_e with K = the rows of expert e (about 128 for
// the fine-grained shape), so a 256 x 256 output tile is only a few K steps followed by 128 KB of
// stores, and the kernel is bound by writing the gradients. A fixed grid of workgroups (one per
// CU) walks the tile list; tiles of one XCD are contiguous in the list (an expert's tiles share
// its P and Q rows in that XCD's L2).
//
// The waves split the memory work: waves 0-3 issue every global -> LDS DMA, waves 4-7 every
// global store; all eight compute a 64 x 128 block of the tile. Loads and stores share one
// in-order counter per wave, so if one wave did both, waiting for a K step's loads would also
// wait for the previous tile's stores; split this way the stores of tile i drain while tile i+1
// loads and computes. During the last three K steps of a tile the DMAs for the first three steps
// of the next tile are issued. The epilogue (wgrad_store_tile) is staged through the two 16 KB
// halves of ring slot 3: slot 3 held the last K step, which every wave has read by that step's
// barrier, while slots 0-2 already receive the next tile's first steps.
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;
constexpr int kWgLoaders = 4;                              // waves 0-3 load, waves 4-7 store
constexpr int kWgDmaA = kTileA / 1024 / kWgLoaders;        // DMA instructions per loader per step
constexpr int kWgDmaB = kTileB / 1024 / kWgLoaders;
constexpr int kWgDma = kWgDmaA + kWgDmaB;
constexpr int kWgStoresPerEighth = 32 / (kWaves - kWgLoaders) / 2;  // 1 KB stores per store wave per 32 rows

constexpr int kMaxExperts = 1024;  // the library's limit on E (checked on the host)
typedef __attribute__((ext_vector_type(4))) int i32x4;

// raw buffer descriptor over [p, p + bytes): 32-bit offsets, loads past the end return zero
__device__ __forceinline__ i32x4 buffer_rsrc(const void* p, int bytes) {
  const uint64_t a = (uint64_t)p;
  i32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  r[1] = __builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32) & 0xffff);
  r[2] = __builtin_amdgcn_readfirstlane(bytes);
  r[3] = kBufferWord3;
  return r;
}
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
// 16 bytes per lane from rsrc + voff into LDS at lds + 16 * lane (one wave-wide 1 KB DMA)
__device__ __forceinline__ void dma_16(const i32x4& rsrc, int voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff), "s"(rsrc), "s"(lds)
               : "memory", "m0");
}

constexpr int kResSteps = 5;             // K steps of a P slice kept in LDS
constexpr int kResK = kResSteps * kBK;   // experts with up to this many rows use the resident kernel

// Loads the expert offsets into s_off, sets s_pref[e] to the exclusive prefix over experts of
// units(K_e) (units of work the calling kernel does for expert e) and returns the total.
template <typename F>
__device__ int wgrad_units(const GemmArgs& g, int* s_off, int* s_pref, int* s_wtot, F units) {
  for (int i = threadIdx.x; i <= g.E; i += kGemmThreads) s_off[i] = g.offsets[i];
  __syncthreads();
  for (int e = threadIdx.x; e < g.E; e += kGemmThreads) s_pref[e] = units(max(0, s_off[e + 1] - s_off[e]));
  __syncthreads();
  block_exclusive_scan<kGemmThreads>(s_pref, g.E, s_wtot);
  return __builtin_amdgcn_readfirstlane(s_pref[g.E]);
}
// the expert whose units contain unit u (s_pref[e] <= u < s_pref[e + 1]; experts with no units skipped)
__device__ __forceinline__ int unit_expert(const int* s_pref, int E, int u) {
  int lo = 0, hi = E;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (s_pref[mid] <= u)
      lo = mid;
    else
      hi = mid;
  }
  return __builtin_amdgcn_readfirstlane(lo);
}

// Epilogue of a weight-gradient tile: rows m0 .. m0 + 255, columns n0 .. n0 + 255 of dW_e (rsC),
// through two free 16 KB LDS buffers, in eighths of 32 rows. Eighth i (rows 32 i ..) is held by the
// waves with wm = i / 2, accumulator half i % 2. While its owners write eighth i + 1 into one buffer
// as bf16 rows (16-byte chunk c of row r at chunk position c ^ r, so the 32 rows of one write fall on
// different banks), the store waves copy eighth i out of the other as whole 512-byte rows, two rows
// (1 KB) per buffer store, non-temporal (the gradients are not re-read); one barrier per eighth. A
// lane's accumulator holds 4-column runs of one row: lanes l and l + 32 hold the two halves of each
// 8-column chunk, and one v_permlane32_swap per register pair gives every lane a whole 16-byte chunk
// (of an even run pair on lanes 0-31, an odd one on lanes 32-63), written with one 16-byte LDS store.
// Every wave of the workgroup calls it (one barrier per eighth, nine in all); the caller has made sure
// that nothing else reads or writes the two buffers until it returns.
template <bool LOADER>
__device__ __forceinline__ void wgrad_store_tile(const f32x16 (&acc)[2][4], uint8_t* buf0, uint8_t* buf1,
                                                 const __amdgpu_buffer_rsrc_t& rsC, int m0, int n0, int M, int N,
                                                 int ldc, int wave, int lane, int wm, int wn) {
  int z;  // (lane offsets computed here, not hoisted out of the caller's tile loop)
  asm volatile("v_mov_b32 %0, 0" : "=v"(z));
  const int lr = (lane & 31) + z;
  // round to bf16 first: 64 packed registers stay live through the eighths, not 128
  u32x4 pw[2][4][2];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
      for (int gp = 0; gp < 2; ++gp) {
        const uint32_t x0 = pack_bf16x2(acc[mb][nb][gp * 8 + 0], acc[mb][nb][gp * 8 + 1]);
        const uint32_t x1 = pack_bf16x2(acc[mb][nb][gp * 8 + 2], acc[mb][nb][gp * 8 + 3]);
        const uint32_t y0 = pack_bf16x2(acc[mb][nb][gp * 8 + 4], acc[mb][nb][gp * 8 + 5]);
        const uint32_t y1 = pack_bf16x2(acc[mb][nb][gp * 8 + 6], acc[mb][nb][gp * 8 + 7]);
        const auto s0 = __builtin_amdgcn_permlane32_swap(x0, y0, false, false);
        const auto s1 = __builtin_amdgcn_permlane32_swap(x1, y1, false, false);
        pw[mb][nb][gp] = u32x4{(uint32_t)s0[0], (uint32_t)s1[0], (uint32_t)s0[1], (uint32_t)s1[1]};
      }
#pragma unroll
  for (int e8 = -1; e8 < 8; ++e8) {
    if (e8 + 1 < 8 && wm == ((e8 + 1) >> 1)) {  // stage eighth e8 + 1
      uint8_t* rowp = (((e8 + 1) & 1) ? buf1 : buf0) + lr * 512;
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
#pragma unroll
        for (int gp = 0; gp < 2; ++gp) {
          const int chunk = (wn * 16 + nb * 4 + gp * 2 + (lane >> 5)) ^ lr;
          *reinterpret_cast<u32x4*>(rowp + (chunk << 4)) = pw[(e8 + 1) & 1][nb][gp];
        }
    }
    if constexpr (!LOADER) {
      if (e8 >= 0) {  // store eighth e8
        const uint8_t* sp = (e8 & 1) ? buf1 : buf0;
#pragma unroll
        for (int j = 0; j < kWgStoresPerEighth; ++j) {
          const int r = ((wave - kWgLoaders) * kWgStoresPerEighth + j) * 2 + (lane >> 5) + z;
          const int c = lane & 31;
          const u32x4 v = *reinterpret_cast<const u32x4*>(sp + r * 512 + ((c ^ r) << 4));
          const int m = m0 + e8 * 32 + r, col = n0 + c * 8;
          const int off = (m < M && col < N) ? (m * ldc + col) * 2 : kOutOfRange;
          __builtin_amdgcn_raw_buffer_store_b128(v, rsC, off, 0, 2);
        }
      }
    }
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  }
}

struct WgTile {
  const uint16_t* a;  // P rows of the expert, from its first row
  const uint16_t* b;  // Q rows of the expert
  int e, m0, n0, K, KT4;
};

__global__ __launch_bounds__(kGemmThreads) void grouped_wgrad_kernel(const GemmArgs g) {
  __shared__ __attribute__((aligned(1024))) uint8_t sA0[kTileA], sA1[kTileA], sA2[kTileA], sA3[kTileA];
  __shared__ __attribute__((aligned(1024))) uint8_t sB0[kTileB], sB1[kTileB], sB2[kTileB], sB3[kTileB];
  __shared__ int s_off[kMaxExperts + 1];  // expert offsets, read once (LDS reads do not touch vmcnt)
  __shared__ int s_pref[kMaxExperts + 1];
  __shared__ int s_wtot[kGemmThreads / kWave];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int wm = (wave >> 1) & 3, wn = wave & 1;
  const int b = blockIdx.x;
  // this kernel takes the experts with more than kResK rows (the others keep their P slice in LDS,
  // grouped_wgrad_res_kernel); tiles are numbered over those experts only
  const int per_e = g.ntiles_m * g.ntiles_n;
  const int total = wgrad_units(g, s_off, s_pref, s_wtot, [&](int K) { return K > kResK ? per_e : 0; });
  const int Q = (total + 7) >> 3;
  const int t_end = min(((b & 7) + 1) * Q, total);
  const int stride = gridDim.x >> 3;
  const int t0 = (b & 7) * Q + (b >> 3);
  if (t0 >= t_end) return;

  // tile tt -> expert, output origin, K rows and operand rows. A tile past the end has K = 0.
  auto setup = [&](int tt, WgTile& w) {
    const bool real = tt < t_end;
    const int e = real ? unit_expert(s_pref, g.E, tt) : 0;
    const int rem = real ? tt - s_pref[e] : 0;
    const int mt = rem / g.ntiles_n;
    w.e = e;
    w.m0 = mt * kBM;
    w.n0 = (rem - mt * g.ntiles_n) * kBN;
    const int r0 = __builtin_amdgcn_readfirstlane(s_off[e]);
    const int K = real ? __builtin_amdgcn_readfirstlane(max(0, s_off[e + 1] - r0)) : 0;
    w.K = K;
    w.KT4 = max(kStages, (K + kBK * kStages - 1) / (kBK * kStages) * kStages);
    w.a = g.A + (int64_t)r0 * g.lda;
    w.b = g.B + (int64_t)r0 * g.ldb;
  };

  // fragment addresses (both operands k-row tiles, read with the transpose read)
  const int q = lane >> 4, sl = lane & 15;
  auto krow_rd = [&](int col32, int kk, int ri) {
    const int kr = kk * 16 + (q >> 1) * 8 + ri * 4 + (sl >> 2);
    const int col = col32 + (q & 1) * 16 + 4 * (sl & 3);
    return kr * 512 + (((col >> 3) ^ swz_b(kr)) << 4) + (col & 7) * 2;
  };
  int a_rd[2][2][2], b_rd[2][4][2];
#pragma unroll
  for (int kk = 0; kk < 2; ++kk)
#pragma unroll
    for (int ri = 0; ri < 2; ++ri) {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) a_rd[kk][mb][ri] = krow_rd(wm * 64 + mb * 32, kk, ri);
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) b_rd[kk][nb][ri] = krow_rd(wn * 128 + nb * 32, kk, ri);
    }
  auto frag = [&](const uint8_t* base, const int* rd) -> bf16x8 {
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(base + rd[0]));
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(base + rd[1]));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };

  f32x16 acc[2][4];
  auto zero_acc = [&]() {
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
#pragma unroll
        for (int qq = 0; qq < 16; ++qq) acc[mb][nb][qq] = 0.0f;
  };

  // The whole walk, once per role, so that each role's loop is scheduled on its own. Both roles
  // meet the same barriers in the same order: one per K step, nine per epilogue.
  auto walk = [&](auto loader_tag) {
    constexpr bool LOADER = decltype(loader_tag)::value;
    const int lw = wave & (kWgLoaders - 1);
    // loader lane offsets within a k-row tile: instruction i fills k-rows (lw*n + i)*2 .. +2, 32
    // lanes per 512-byte row; rows of P are g.lda elements apart, rows of Q g.ldb
    int a_lane[kWgDmaA], b_lane[kWgDmaB];
#pragma unroll
    for (int i = 0; i < kWgDmaA; ++i) {
      const int kr = (lw * kWgDmaA + i) * 2 + (lane >> 5);
      a_lane[i] = kr * g.lda * 2 + (((lane & 31) ^ swz_b(kr)) * 16);
    }
#pragma unroll
    for (int i = 0; i < kWgDmaB; ++i) {
      const int kr = (lw * kWgDmaB + i) * 2 + (lane >> 5);
      b_lane[i] = kr * g.ldb * 2 + (((lane & 31) ^ swz_b(kr)) * 16);
    }
    // Step kt of tile w: the descriptors start at the step's first k-row and end at the expert's
    // last row, so k-rows past K (the step count is padded to the ring depth) read as zero; they
    // are rebuilt per step in scalar registers, which keeps the per-step offsets out of vector
    // registers. Columns past M or N are not masked: they read other elements of the same
    // operands and only reach outputs that are never stored.
    //
    // The DMAs are written as inline assembly: the compiler then does not track them, and only
    // the explicit waits below order them against the fragment reads. (Tracked, its own
    // conservative waits before the fragment reads cut the prefetch depth from three steps to
    // two.)
    auto dma = [&](const WgTile& w, int kt, uint8_t* sa, uint8_t* sb) {
      if constexpr (LOADER) {
        const int k0 = kt * kBK, rows = max(0, w.K - k0);
        const i32x4 rsA = buffer_rsrc(w.a + (int64_t)k0 * g.lda, rows * g.lda * 2);
        const i32x4 rsB = buffer_rsrc(w.b + (int64_t)k0 * g.ldb, rows * g.ldb * 2);
        const uint32_t da = lds_addr(sa) + lw * kWgDmaA * 1024, db = lds_addr(sb) + lw * kWgDmaB * 1024;
#pragma unroll
        for (int i = 0; i < kWgDmaA; ++i) dma_16(rsA, a_lane[i] + w.m0 * 2, da + i * 1024);
#pragma unroll
        for (int i = 0; i < kWgDmaB; ++i) dma_16(rsB, b_lane[i] + w.n0 * 2, db + i * 1024);
      }
    };
    // end of a step: loaders wait until only the two newer steps' DMAs are outstanding
    auto meet = [&]() {
      if constexpr (LOADER)
        asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(2 * kWgDma) : "memory");
      else
        asm volatile("s_barrier" ::: "memory");
    };
    // One step: fragments of step kt, one prefetch (this tile's step kt+3, or the next tile's
    // step kt+3-KT4 in the last three steps), MFMAs, then meet. Padded steps (past K) keep only
    // the prefetch and the barrier.
    auto step = [&](int kt, const WgTile& cur, const WgTile& nxt, const uint8_t* sa, const uint8_t* sb, uint8_t* pa,
                    uint8_t* pb) {
      if (kt * kBK < cur.K) {
        bf16x8 fa[2][2], fb[2][4];
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
          for (int nb = 0; nb < 4; ++nb) fb[kk][nb] = frag(sb, b_rd[kk][nb]);
#pragma unroll
          for (int mb = 0; mb < 2; ++mb) fa[kk][mb] = frag(sa, a_rd[kk][mb]);
        }
        if (kt + 3 < cur.KT4)
          dma(cur, kt + 3, pa, pb);
        else
          dma(nxt, kt + 3 - cur.KT4, pa, pb);
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
          for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int nb = 0; nb < 4; ++nb)
              acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[kk][nb], fa[kk][mb], acc[mb][nb], 0, 0, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 24, 0);
        if constexpr (LOADER) {
#pragma unroll
          for (int i = 0; i < kWgDma; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
          }
          __builtin_amdgcn_sched_group_barrier(0x008, 16 - kWgDma, 0);
        } else {
          __builtin_amdgcn_sched_group_barrier(0x008, 16, 0);
        }
      } else {
        if (kt + 3 < cur.KT4)
          dma(cur, kt + 3, pa, pb);
        else
          dma(nxt, kt + 3 - cur.KT4, pa, pb);
      }
      meet();
    };
    // Epilogue: the previous tile's stores are waited for first (the store waves' counter then
    // holds only this tile's), then wgrad_store_tile through ring slot 3.
    auto store = [&](const WgTile& w) {
      const __amdgpu_buffer_rsrc_t rsC = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(g.C + (int64_t)w.e * g.c_expert), (short)0, g.M * g.N * 2, kBufferWord3);
      if constexpr (!LOADER) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      wgrad_store_tile<LOADER>(acc, sA3, sB3, rsC, w.m0, w.n0, g.M, g.N, g.ldc, wave, lane, wm, wn);
    };

    int t = t0;
    WgTile cur, nxt;
    setup(t, cur);
    zero_acc();
    dma(cur, 0, sA0, sB0);
    dma(cur, 1, sA1, sB1);
    dma(cur, 2, sA2, sB2);
    meet();
    for (;;) {
      setup(t + stride, nxt);
      for (int kb = 0; kb < cur.KT4; kb += kStages) {
        step(kb + 0, cur, nxt, sA0, sB0, sA3, sB3);
        step(kb + 1, cur, nxt, sA1, sB1, sA0, sB0);
        step(kb + 2, cur, nxt, sA2, sB2, sA1, sB1);
        step(kb + 3, cur, nxt, sA3, sB3, sA2, sB2);
      }
      store(cur);
      t += stride;
      if (t >= t_end) break;
      cur = nxt;
      zero_acc();
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  };
  if (wave < kWgLoaders)
    walk(std::true_type{});
  else
    walk(std::false_type{});
}

// ---------------------------------------------------------------------------------------------
// Weight gradients of experts with at most kResK rows, P slice resident. A unit of work is (expert
// e, 256-row block mt of dW_e): its P slice (K x 256, at most kResSteps K steps) is loaded into LDS
// once, and the workgroup then computes all ntiles_n column tiles of that block, streaming only
// Q (K x 256 per tile) through a 4-slot ring; per K step that is 16 KB of global -> LDS traffic
// instead of 32. The Q steps of the unit form one sequence (tile nt, step kt -> nt * KT + kt),
// prefetched three steps ahead across tile boundaries, except that a tile's last step prefetches
// only two ahead: the epilogue then has two free ring slots (the step just read and the one not yet
// loaded) for staging 64 output rows at a time, and the next tile's first step issues two steps
// to catch up. Roles as in grouped_wgrad_kernel: waves 0-3 issue the DMAs, waves 4-7 the stores.
__global__ __launch_bounds__(kGemmThreads) void grouped_wgrad_res_kernel(const GemmArgs g) {
  __shared__ __attribute__((aligned(1024))) uint8_t sR0[kTileA], sR1[kTileA], sR2[kTileA], sR3[kTileA], sR4[kTileA];
  __shared__ __attribute__((aligned(1024))) uint8_t sB0[kTileB], sB1[kTileB], sB2[kTileB], sB3[kTileB];
  __shared__ int s_off[kMaxExperts + 1];
  __shared__ int s_pref[kMaxExperts + 1];
  __shared__ int s_wtot[kGemmThreads / kWave];
  static_assert(kResSteps == 5, "five resident slots");

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int wm = (wave >> 1) & 3, wn = wave & 1;
  const int b = blockIdx.x;
  const int total = wgrad_units(g, s_off, s_pref, s_wtot, [&](int K) { return K <= kResK ? g.ntiles_m : 0; });
  const int Q = (total + 7) >> 3;
  const int u_end = min(((b & 7) + 1) * Q, total);
  const int stride = gridDim.x >> 3;
  const int u0 = (b & 7) * Q + (b >> 3);
  if (u0 >= u_end) return;

  auto rslot = [&](int kt) -> uint8_t* { return kt == 0 ? sR0 : kt == 1 ? sR1 : kt == 2 ? sR2 : kt == 3 ? sR3 : sR4; };
  auto bslot = [&](int s4) -> uint8_t* { return s4 == 0 ? sB0 : s4 == 1 ? sB1 : s4 == 2 ? sB2 : sB3; };

  const int q = lane >> 4, sl = lane & 15;
  auto krow_rd = [&](int col32, int kk, int ri) {
    const int kr = kk * 16 + (q >> 1) * 8 + ri * 4 + (sl >> 2);
    const int col = col32 + (q & 1) * 16 + 4 * (sl & 3);
    return kr * 512 + (((col >> 3) ^ swz_b(kr)) << 4) + (col & 7) * 2;
  };
  int a_rd[2][2][2], b_rd[2][4][2];
#pragma unroll
  for (int kk = 0; kk < 2; ++kk)
#pragma unroll
    for (int ri = 0; ri < 2; ++ri) {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) a_rd[kk][mb][ri] = krow_rd(wm * 64 + mb * 32, kk, ri);
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) b_rd[kk][nb][ri] = krow_rd(wn * 128 + nb * 32, kk, ri);
    }
  auto frag = [&](const uint8_t* base, const int* rd) -> bf16x8 {
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(base + rd[0]));
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(base + rd[1]));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  f32x16 acc[2][4];

  auto walk = [&](auto loader_tag) {
    constexpr bool LOADER = decltype(loader_tag)::value;
    const int lw = wave & (kWgLoaders - 1);
    int a_lane[kWgDmaA], b_lane[kWgDmaB];
#pragma unroll
    for (int i = 0; i < kWgDmaA; ++i) {
      const int kr = (lw * kWgDmaA + i) * 2 + (lane >> 5);
      a_lane[i] = kr * g.lda * 2 + (((lane & 31) ^ swz_b(kr)) * 16);
    }
#pragma unroll
    for (int i = 0; i < kWgDmaB; ++i) {
      const int kr = (lw * kWgDmaB + i) * 2 + (lane >> 5);
      b_lane[i] = kr * g.ldb * 2 + (((lane & 31) ^ swz_b(kr)) * 16);
    }
    // the unit being computed
    int e = 0, m0 = 0, K = 0, KT = 0, G = 0;
    const uint16_t* pa = g.A;
    const uint16_t* pb = g.B;
    // P step kt into its resident slot; Q step j of the unit's sequence into ring slot j % 4
    // (descriptors from the step's first k-row to the expert's last row: rows past K read zero)
    auto dma_a = [&](int kt) {
      if constexpr (LOADER) {
        const int k0 = kt * kBK;
        const i32x4 rs = buffer_rsrc(pa + (int64_t)k0 * g.lda, max(0, K - k0) * g.lda * 2);
        const uint32_t d = lds_addr(rslot(kt)) + lw * kWgDmaA * 1024;
#pragma unroll
        for (int i = 0; i < kWgDmaA; ++i) dma_16(rs, a_lane[i] + m0 * 2, d + i * 1024);
      }
    };
    auto dma_b = [&](int j) {
      if constexpr (LOADER) {
        const int nt = j / KT, k0 = (j - nt * KT) * kBK;
        const i32x4 rs = buffer_rsrc(pb + (int64_t)k0 * g.ldb, max(0, K - k0) * g.ldb * 2);
        const uint32_t d = lds_addr(bslot(j & 3)) + lw * kWgDmaB * 1024;
#pragma unroll
        for (int i = 0; i < kWgDmaB; ++i) dma_16(rs, b_lane[i] + nt * kBN * 2, d + i * 1024);
      }
    };
    // loaders wait until at most n Q steps (n = 0, 1, 2) issued after the one needed are pending
    auto meet = [&](int n) {
      if constexpr (LOADER) {
        if (n >= 2)
          asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(2 * kWgDmaB) : "memory");
        else if (n == 1)
          asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(kWgDmaB) : "memory");
        else
          asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
      } else {
        asm volatile("s_barrier" ::: "memory");
      }
    };
    // epilogue of tile nt through the free ring slots st0 and st1
    auto store = [&](int nt, uint8_t* st0, uint8_t* st1) {
      const __amdgpu_buffer_rsrc_t rsC = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(g.C + (int64_t)e * g.c_expert), (short)0, g.M * g.N * 2, kBufferWord3);
      if constexpr (!LOADER) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      wgrad_store_tile<LOADER>(acc, st0, st1, rsC, m0, nt * kBN, g.M, g.N, g.ldc, wave, lane, wm, wn);
    };

    for (int u = u0; u < u_end; u += stride) {
      e = unit_expert(s_pref, g.E, u);
      const int mt = u - s_pref[e];
      m0 = mt * kBM;
      const int r0 = __builtin_amdgcn_readfirstlane(s_off[e]);
      K = __builtin_amdgcn_readfirstlane(max(0, s_off[e + 1] - r0));
      KT = (K + kBK - 1) / kBK;  // 0 .. kResSteps
      G = g.ntiles_n * KT;
      pa = g.A + (int64_t)r0 * g.lda;
      pb = g.B + (int64_t)r0 * g.ldb;
      // prologue: the resident P steps, then the first Q steps; wait for all of P and Q step 0
      for (int kt = 0; kt < KT; ++kt) dma_a(kt);
      int issued = min(3, G);
      for (int j = 0; j < issued; ++j) dma_b(j);
      meet(issued - 1);
      int s = 0;  // Q step being computed
      for (int nt = 0; nt < g.ntiles_n; ++nt) {
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int nb = 0; nb < 4; ++nb)
#pragma unroll
            for (int qq = 0; qq < 16; ++qq) acc[mb][nb][qq] = 0.0f;
        for (int kt = 0; kt < KT; ++kt, ++s) {
          const uint8_t* sa = rslot(kt);
          const uint8_t* sb = bslot(s & 3);
          bf16x8 fa[2][2], fb[2][4];
#pragma unroll
          for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
            for (int nb = 0; nb < 4; ++nb) fb[kk][nb] = frag(sb, b_rd[kk][nb]);
#pragma unroll
            for (int mb = 0; mb < 2; ++mb) fa[kk][mb] = frag(sa, a_rd[kk][mb]);
          }
          // prefetch: up to s + 3 (s + 2 on the tile's last step), never past the unit
          const int target = min(G - 1, kt == KT - 1 ? s + 2 : s + 3);
          for (; issued <= target; ++issued) dma_b(issued);
#pragma unroll
          for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int mb = 0; mb < 2; ++mb)
#pragma unroll
              for (int nb = 0; nb < 4; ++nb)
                acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[kk][nb], fa[kk][mb], acc[mb][nb], 0, 0, 0);
          // step s + 1 must have landed: at most issued - (s + 2) later steps may stay pending
          meet(issued - (s + 2));
        }
        // staging: the slot of the step just computed and the slot of step s + 2 (not yet loaded;
        // its predecessor in the slot, step s - 2, is done). With no steps, every slot is free.
        const int sl0 = KT > 0 ? (s - 1) & 3 : 0, sl1 = KT > 0 ? (s + 2) & 3 : 1;
        store(nt, bslot(sl0), bslot(sl1));
      }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  };
  if (wave < kWgLoaders)
    walk(std::true_type{});
  else
    walk(std::false_type{});
}

// 16 bytes per lane from rsrc + voff into LDS at lds + IMM + 16 * lane; the immediate keeps one
// scalar register per LDS buffer instead of one per DMA instruction. The add writes SCC, which the
// clobber list must say: the compiler keeps loop conditions in SCC across code like this.
template <int IMM>
__device__ __forceinline__ void dma_16i(const i32x4& rsrc, int voff, uint32_t lds) {
  asm volatile("s_add_u32 m0, %2, %3\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff), "s"(rsrc),
               "s"(lds),
               "n"(IMM)
               : "memory", "m0", "scc");
}
// The same with the non-temporal hint, for the expert weights: every byte of them is read once per
// call, so they are marked as streaming and leave the caches to the row operands (x, h), which are
// read once per column tile (step time -2 to -4 % measured).
template <int IMM>
__device__ __forceinline__ void dma_16i_nt(const i32x4& rsrc, int voff, uint32_t lds) {
  asm volatile("s_add_u32 m0, %2, %3\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen nt lds" ::"v"(voff), "s"(rsrc),
               "s"(lds), "n"(IMM)
               : "memory", "m0", "scc");
}
// The descriptor of the same buffer starting `bytes` further on (bytes >= 0, wave-uniform): base +
// bytes, records - bytes (at least 0), so every offset keeps its range check against the buffer's
// original end and the per-lane offsets need no per-step arithmetic.
__device__ __forceinline__ i32x4 rsrc_advance(const i32x4& r, int bytes) {
  const uint64_t b = ((uint64_t)(uint32_t)r[0] | ((uint64_t)((uint32_t)r[1] & 0xffffu) << 32)) + (uint32_t)bytes;
  i32x4 o;
  o[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)b);
  o[1] = __builtin_amdgcn_readfirstlane((int)(((uint32_t)r[1] & 0xffff0000u) | ((uint32_t)(b >> 32) & 0xffffu)));
  o[2] = __builtin_amdgcn_readfirstlane(max(0, r[2] - bytes));
  o[3] = r[3];
  return o;
}

// ---------------------------------------------------------------------------------------------
// Forward row-grouped products, persistent: gate_up + SwiGLU (EPI = kEpiSwiglu) and down
// (EPI = kEpiStore), the rows from the grouped buffer or (GATHER) from the token matrix through
// the slot map.
//
// One workgroup per CU walks the tiles of grouped_gemm_bf16_kernel's list: each XCD takes an
// eighth of the list and deals it to its workgroups in rounds, back and forth; when a few rounds
// would end in a partial one, the experts are listed tallest first and the row tiles dealt
// round-robin to the XCDs instead (see the tile list and the walk below), so that skewed expert
// sizes end in a last round of short tiles. Per tile the K loop is the one above. What changes is the tile boundary, where the one-tile kernel leaves every CU
// idle at once (set-up, pipeline fill, epilogue):
//  - the tile list is built once per workgroup (expert offsets, list order and row-tile prefix
//    in LDS);
//  - the last three K steps issue the next tile's first A stage and B steps 0-2 (where the
//    one-tile kernel issues zero-filling DMAs past K), so the next tile's data is on its way
//    during the epilogue;
//  - the epilogue stages the finished tile through the A stage the last two steps used, each
//    wave its own block through its own part of it (no workgroup barrier but one at the end),
//    and writes whole 128-byte row segments with buffer stores. Every wave issues the same
//    number of stores (rows past the tile are dropped by the descriptor), and the stores are
//    issued after the prefetches, so the next tile's first wait leaves exactly them in flight:
//    they drain while the next tile computes;
//  - with gathered rows, the slot map of the next tile's rows is brought into LDS by one DMA of
//    wave 0 in the current tile's first step.
// BR: the weights are a row tile (K contiguous: row n of the expert's block holds column n of the
// product, as in the backward input gradient dX = dGU gate_up_e^T), staged [256 n][32 k] per step in
// 64-byte rows and read with ds_read_b128; only with K a multiple of four steps and the plain store.
template <int EPI, bool GATHER, bool KF, bool BR = false>
__global__ __launch_bounds__(kGemmThreads) void grouped_gemm_fwd_kernel(const GemmArgs g) {
  static_assert(EPI == kEpiSwiglu || EPI == kEpiStore, "the forward epilogues");
  static_assert(!BR || (KF && EPI == kEpiStore && !GATHER), "row-tile weights: whole K steps, plain store");
  __shared__ __attribute__((aligned(1024))) uint8_t sA0[kTileA2], sA1[kTileA2];
  __shared__ __attribute__((aligned(1024))) uint8_t sB0[kTileB], sB1[kTileB], sB2[kTileB], sB3[kTileB];
  __shared__ __attribute__((aligned(1024))) int s_slot[512];  // slot map of the next tile's rows (gathered)
  __shared__ int s_off[kGemmMaxE + 1];
  __shared__ __attribute__((aligned(16))) int s_pref[kGemmMaxE + 4];
  __shared__ short s_ord[kGemmMaxE];  // the expert at each position of the tile list
  __shared__ int s_wtot[kGemmThreads / kWave];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int wm = (wave >> 1) & 3, wn = wave & 1;

  // ---- the tile list: expert e owns n_e = ceil(c_e / hm) row tiles of near-equal height (at most
  // h_e = ceil(c_e / n_e) rows), each with ntiles_n column tiles; s_pref = exclusive prefix of the
  // row tiles over the list. The tile height limit hm is kBMX (band tiles: fewest row tiles), or, for
  // one expert (a dense product, whose weights every row tile reads whichever the height), kBM when
  // the kBM list takes as many rounds of the grid and either only it splits into whole rounds on
  // every XCD (see the walk below) or there are two or more. E.g. 4096 rows with 16 column tiles on
  // 256 workgroups: 256 tiles of 256 rows instead of 208 of 315 (a fifth of the chip idle, each tile a
  // fifth more work); with 28 column tiles, two rounds either way: 11-15 % faster measured. Not for
  // several experts: one split into more row tiles streams its weights into more XCDs (one
  // expert-parallel rank's Zipf share: 14 % slower with kBM in its two rounds).
  // The experts are listed in index order, or tallest first (ties by index) when the walk below
  // balances (and there are at most kSortMaxE experts).
  const int ntn = g.ntiles_n;
  const int nbx = (int)(gridDim.x >> 3);  // workgroups per XCD (the grid is a multiple of 8)
  for (int i = tid; i <= g.E; i += kGemmThreads) s_off[i] = g.offsets[i];
  __syncthreads();
  int hm = kBMX;
  if (g.E == 1) {  // one expert: a dense product
    auto whole_rounds = [&](int rt) { return (rt & 7) == 0 && ((rt >> 3) * ntn) % nbx == 0; };
    const int c = __builtin_amdgcn_readfirstlane(s_off[1] - s_off[0]), G = (int)gridDim.x;
    const int rt_x = (c + kBMX - 1) / kBMX, rt_b = (c + kBM - 1) / kBM;
    const int rounds_x = (rt_x * ntn + G - 1) / G, rounds_b = (rt_b * ntn + G - 1) / G;
    if (c > 0 && rt_b != rt_x && rounds_b == rounds_x &&
        ((whole_rounds(rt_b) && !whole_rounds(rt_x)) || rounds_x >= 2))
      hm = kBM;
  }
  for (int i = tid; i < g.E; i += kGemmThreads) {
    const int c = s_off[i + 1] - s_off[i];
    s_ord[i] = (short)i;
    s_pref[i] = c <= 0 ? 0 : hm == kBM ? (c + kBM - 1) / kBM : (c + kBMX - 1) / kBMX;
  }
  __syncthreads();
  block_exclusive_scan<kGemmThreads>(s_pref, g.E, s_wtot);
  const int RT = __builtin_amdgcn_readfirstlane(s_pref[g.E]);  // row tiles in the list
  const int total = RT * ntn;
  // The walk deals each XCD's tiles to its nbx workgroups in rounds. With whole rounds on every XCD,
  // or more than four rounds on average, XCD x takes the contiguous eighth [x Q, (x + 1) Q) of the
  // list in index order, Q = ceil(tiles / 8): an expert's row tiles share one XCD's L2 (its weights
  // are streamed once per XCD) and both forward products split the experts alike. Otherwise the
  // last round is partial and, with few rounds, costs a large share of the product: then the walk
  // balances. The experts are listed tallest first and row tile R goes to XCD R mod 8, so each XCD
  // gets every eighth of the heights and its partial last round holds its shortest tiles.
  const bool whole = (RT & 7) == 0 && ((RT >> 3) * ntn) % nbx == 0;
  const bool balance = !whole && total <= 4 * (int)gridDim.x;
  if (balance && g.E <= kSortMaxE) {
    static_assert(kSortMaxE <= kGemmThreads, "one expert per thread");
    __syncthreads();  // every thread has read the row-tile total
    if (tid < g.E) {
      const int c = s_off[tid + 1] - s_off[tid];
      const int n = c <= 0 ? 0 : hm == kBM ? (c + kBM - 1) / kBM : (c + kBMX - 1) / kBMX;
      s_pref[tid] = n > 0 ? (c + n - 1) / n : 0;
    }
    __syncthreads();
    int rk = 0;  // the expert's position: taller experts, then equal ones of lower index
    if (tid < g.E) {
      const int h = s_pref[tid];
#pragma unroll 4
      for (int j0 = 0; j0 < g.E; j0 += 4) {  // four heights per LDS read (entries past E are masked)
        const int4 hv = *reinterpret_cast<const int4*>(s_pref + j0);
        const int hs[4] = {hv.x, hv.y, hv.z, hv.w};
#pragma unroll
        for (int k4 = 0; k4 < 4; ++k4) {
          const int j = j0 + k4;
          rk += (j < g.E && (hs[k4] > h || (hs[k4] == h && j < tid))) ? 1 : 0;
        }
      }
    }
    __syncthreads();
    if (tid < g.E) s_ord[rk] = (short)tid;
    __syncthreads();
    if (tid < g.E) {
      const int e = s_ord[tid];
      const int c = s_off[e + 1] - s_off[e];
      s_pref[tid] = c <= 0 ? 0 : hm == kBM ? (c + kBM - 1) / kBM : (c + kBMX - 1) / kBMX;
    }
    __syncthreads();
    block_exclusive_scan<kGemmThreads>(s_pref, g.E, s_wtot);
  }

  // ---- the walk. Workgroup b runs on XCD b mod 8 and is workgroup j = b div 8 of that XCD; of the
  // XCD's n_x tiles it takes tile r nbx + j in an even round r and r nbx + nbx - 1 - j in an odd
  // one (back and forth: a workgroup that took one of the last tiles of a round takes one of the
  // first of the next).
  const int xcd = (int)(blockIdx.x & 7);
  const int wj = (int)(blockIdx.x >> 3);
  const int Q = (total + 7) >> 3;
  const int n_x = balance ? (RT > xcd ? (RT - xcd + 7) >> 3 : 0) * ntn : max(0, min(Q, total - xcd * Q));
  // the list index (row tile * ntn + column tile) of this workgroup's tile in round r, or -1
  auto pos = [&](int r) -> int {
    const int q = r * nbx + ((r & 1) ? nbx - 1 - wj : wj);
    if (q >= n_x) return -1;
    if (!balance) return xcd * Q + q;
    int dn;
    asm volatile("s_mov_b32 %0, %1" : "=s"(dn) : "s"(ntn));
    const int l = (int)((uint32_t)q / (uint32_t)dn);
    return (l * 8 + xcd) * ntn + (q - l * dn);
  };
  int rnd = 0;
  int L = pos(0);
  if (L < 0) return;

  struct Tile {
    int e, m0, mvalid, nt;
  };
  // (32-bit arithmetic on operands the compiler cannot see through: it would otherwise hoist the
  // division constants out of the tile loop and keep them in registers through every K loop)
  auto decode = [&](int LL, Tile& t) {
    int dn;
    asm volatile("s_mov_b32 %0, %1" : "=s"(dn) : "s"(ntn));
    const int mt_g = (int)((uint32_t)LL / (uint32_t)dn);
    t.nt = __builtin_amdgcn_readfirstlane(LL - mt_g * dn);
    int lo = 0, hi = g.E;  // the last list position whose row tiles start at or before mt_g
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (s_pref[mid] <= mt_g)
        lo = mid;
      else
        hi = mid;
    }
    const int e = __builtin_amdgcn_readfirstlane((int)s_ord[lo]);
    const int p0 = __builtin_amdgcn_readfirstlane(s_pref[lo]);
    const int nte = __builtin_amdgcn_readfirstlane(s_pref[lo + 1]) - p0;
    const int o0 = __builtin_amdgcn_readfirstlane(s_off[e]);
    const int c = __builtin_amdgcn_readfirstlane(s_off[e + 1]) - o0;
    // the expert's c rows in nte contiguous pieces, the first c % nte one row longer
    const int j = mt_g - p0;
    const int base = (int)((uint32_t)c / (uint32_t)nte), rem = c - base * nte;
    t.e = e;
    t.m0 = __builtin_amdgcn_readfirstlane(o0 + j * base + min(j, rem));
    t.mvalid = __builtin_amdgcn_readfirstlane(base + (j < rem ? 1 : 0));
  };

  // ---- operand DMAs (inline assembly, so that only the explicit waits below order them)
  const int K = g.K;
  const int a_c0 = (lane & 7) ^ swz_a2(lane >> 3);
  const int a_kc[2] = {a_c0 * 8, (a_c0 ^ 1) * 8};
  const int x_r = kBM + wave * 8 + (lane >> 3);       // extra-band row of this DMA lane
  const int x_kc = ((lane & 7) ^ swz_a2(x_r)) * 8;
  struct Ops {
    i32x4 rsA, rsB;
    int a_off[kDmaA2];   // byte offsets for k = 0 (kOutOfRange: no row)
    int x_off;
    int b_off[kDmaB];
    int band;            // the tile has rows in the extra band: one more DMA per A stage
  };
  // slots: the tile's slot map (LDS), for gathered rows
  auto set_ops = [&](const Tile& t, const int* slots, Ops& o) {
    int zo;
    asm volatile("v_mov_b32 %0, 0" : "=v"(zo));
    const int lane = (int)(threadIdx.x & (kWave - 1)) + zo;
    if constexpr (GATHER) {
      o.rsA = buffer_rsrc(g.A, g.M * g.lda * 2);
    } else {
      o.rsA = buffer_rsrc(g.A + (int64_t)t.m0 * g.lda, t.mvalid * g.lda * 2);
    }
    o.rsB = buffer_rsrc(g.B + (int64_t)t.e * g.b_expert, g.b_rows * g.ldb * 2);
#pragma unroll
    for (int i = 0; i < kDmaA2; ++i) {
      const int r = (wave * kDmaA2 + i) * 8 + (lane >> 3);
      const int c = a_c0 ^ (i & 1);
      if constexpr (GATHER)
        o.a_off[i] = r < t.mvalid ? (slots[r] / g.a_div * g.lda + c * 8) * 2 : kOutOfRange;
      else
        o.a_off[i] = (r * g.lda + c * 8) * 2;
    }
    const int xc = x_kc / 8;
    if constexpr (GATHER)
      o.x_off = x_r < t.mvalid ? (slots[x_r] / g.a_div * g.lda + xc * 8) * 2 : kOutOfRange;
    else
      o.x_off = (x_r * g.lda + xc * 8) * 2;
#pragma unroll
    for (int i = 0; i < kDmaB; ++i) {
      if constexpr (BR) {  // rows (wave kDmaB + i) 16 .. +16 of the tile's 256 weight rows, 4 lanes per row
        const int r = (wave * kDmaB + i) * 16 + (lane >> 2);
        const int c = (lane & 3) ^ swz_a(r);
        const int n = t.nt * kBN + r;
        o.b_off[i] = n < g.N ? (n * g.ldb + c * 8) * 2 : kOutOfRange;
        continue;
      }
      const int kr = (wave * kDmaB + i) * 2 + (lane >> 5);
      const int cb = (lane & 31) ^ swz_b(kr);
      int col;
      bool ok;
      if constexpr (EPI == kEpiSwiglu) {  // 128 gate columns then the matching 128 up columns
        const int j = t.nt * 128 + (cb & 15) * 8;
        ok = j < g.N;
        col = (cb < 16 ? 0 : g.N) + j;
      } else {
        col = t.nt * kBN + cb * 8;
        ok = col < g.N;
      }
      o.b_off[i] = ok ? (kr * g.ldb + col) * 2 : kOutOfRange;
    }
    o.band = __builtin_amdgcn_readfirstlane(t.mvalid > kBM ? 1 : 0);
  };
  // A stage st (K 64 st .. 64 st + 63) into sa; B step kt (K 32 kt .. 32 kt + 31) into sb.
  // Offsets are unsigned: a missing row's kOutOfRange plus k may pass 2^31 and stays out of range.
  static_assert(kDmaA2 == 4 && kDmaB == 2, "DMA instruction counts per wave");
  const uint32_t wa = __builtin_amdgcn_readfirstlane(wave * kDmaA2 * 1024);
  const uint32_t wx = __builtin_amdgcn_readfirstlane(kBM * kBK2 * 2 + wave * 1024);
  const uint32_t wb = __builtin_amdgcn_readfirstlane(wave * kDmaB * 1024);
  auto dma_a = [&](const Ops& o, int st, uint8_t* sa) {
    const int k0 = st * kBK2;
    const uint32_t base = lds_addr(sa) + wa;
    if constexpr (KF) {
      // K a multiple of 128: no K tail. The step moves the descriptor (scalar arithmetic) instead of
      // every lane's offset; rows past the tile keep their out-of-range offset
      const i32x4 rs = rsrc_advance(o.rsA, k0 * 2);
      if (o.band) dma_16i<0>(rs, o.x_off, lds_addr(sa) + wx);
      dma_16i<0>(rs, o.a_off[0], base);
      dma_16i<1024>(rs, o.a_off[1], base);
      dma_16i<2048>(rs, o.a_off[2], base);
      dma_16i<3072>(rs, o.a_off[3], base);
      return;
    }
    if (o.band) {
      const int off = k0 + x_kc < K ? (int)((uint32_t)o.x_off + (uint32_t)(k0 * 2)) : kOutOfRange;
      dma_16i<0>(o.rsA, off, lds_addr(sa) + wx);
    }
    int off[kDmaA2];
#pragma unroll
    for (int i = 0; i < kDmaA2; ++i)
      off[i] = k0 + a_kc[i & 1] < K ? (int)((uint32_t)o.a_off[i] + (uint32_t)(k0 * 2)) : kOutOfRange;
    dma_16i<0>(o.rsA, off[0], base);
    dma_16i<1024>(o.rsA, off[1], base);
    dma_16i<2048>(o.rsA, off[2], base);
    dma_16i<3072>(o.rsA, off[3], base);
  };
  auto dma_b = [&](const Ops& o, int kt, uint8_t* sb) {
    const int kb = kt * kBK * g.ldb * 2;  // k-rows past K are past the expert's block
    const uint32_t base = lds_addr(sb) + wb;
    if constexpr (BR) {  // the step's 32 k of every row: the descriptor moves 64 bytes along the rows
      // (plain loads: an expert's rows are read by each of its row tiles)
      const i32x4 rs = rsrc_advance(o.rsB, kt * kBK * 2);
      dma_16i<0>(rs, o.b_off[0], base);
      dma_16i<1024>(rs, o.b_off[1], base);
      return;
    }
    if constexpr (KF) {
      const i32x4 rs = rsrc_advance(o.rsB, kb);
      dma_16i_nt<0>(rs, o.b_off[0], base);
      dma_16i_nt<1024>(rs, o.b_off[1], base);
      return;
    }
    const int off0 = o.b_off[0] == kOutOfRange ? kOutOfRange : o.b_off[0] + kb;
    const int off1 = o.b_off[1] == kOutOfRange ? kOutOfRange : o.b_off[1] + kb;
    dma_16i_nt<0>(o.rsB, off0, base);
    dma_16i_nt<1024>(o.rsB, off1, base);
  };
  // wave 0: the slot map of tile t's rows into s_slot (entries past the tile read as zero)
  auto dma_slots = [&](const Tile& t) {
    if constexpr (GATHER) {
      if (wave == 0) {
        int zs;  // (computed here, not kept from the kernel's start)
        asm volatile("v_mov_b32 %0, 0" : "=v"(zs));
        const int lo = (lane + zs) * 16;
        const i32x4 rs = buffer_rsrc(g.a_slot + t.m0, t.mvalid * 4);
        dma_16i<0>(rs, lo, lds_addr(s_slot));
        dma_16i<1024>(rs, lo + 1024, lds_addr(s_slot));
      }
    }
  };

  // ---- fragment addresses (as in grouped_gemm_bf16_kernel)
  int bcol[4];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb)
    bcol[nb] = EPI == kEpiSwiglu ? ((nb >> 1) * 128 + wn * 64 + (nb & 1) * 32) : (wn * 128 + nb * 32);
  const int q = lane >> 4, sl = lane & 15;
  auto arow_rd = [&](int r, int kk) {
    const int c = kk * 2 + (lane >> 5);
    return r * (kBK2 * 2) + ((c ^ swz_a2(r)) << 4);
  };
  auto krow_rd = [&](int col32) {
    const int kr = (q >> 1) * 8 + (sl >> 2);
    const int col = col32 + (q & 1) * 16 + 4 * (sl & 3);
    return kr * 512 + (((col >> 3) ^ swz_b(kr)) << 4) + (col & 7) * 2;
  };
  // row-tile weights: row r's 16-byte chunk c (k = 8 c) at chunk c ^ swz_a(r) of its 64-byte row; the
  // lane's chunk is kk * 2 + lane / 32, so the second 16-deep sub-step's address is the first's with
  // bit 5 flipped
  auto brow_rd = [&](int r) { return r * 64 + (((lane >> 5) ^ swz_a(r)) << 4); };
  int a_rd[2][2], b_rd[4];
#pragma unroll
  for (int kk = 0; kk < 2; ++kk)
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) a_rd[kk][mb] = arow_rd(wm * 64 + mb * 32 + (lane & 31), kk);
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) b_rd[nb] = BR ? brow_rd(bcol[nb] + (lane & 31)) : krow_rd(bcol[nb]);
  const int g0 = (wn * 4 + wm) * 16;
  int xa_rd[2], xb_rd;
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) xa_rd[kk] = arow_rd(kBM + (lane & 31), kk);
  if constexpr (EPI == kEpiSwiglu) {
    const int kr = (q >> 1) * 8 + (sl >> 2);
    const int col = (q & 1) * 128 + g0 + 4 * (sl & 3);
    xb_rd = kr * 512 + (((col >> 3) ^ swz_b(kr)) << 4) + (col & 7) * 2;
  } else if constexpr (BR) {
    xb_rd = brow_rd(wn * 128 + wm * 32 + (lane & 31));
  } else {
    xb_rd = krow_rd(wn * 128 + wm * 32);
  }

  f32x16 acc[2][4];
  struct Frags {
    bf16x8 a[2], b[4], xa[2], xb;
  };
  auto frag_b = [&](const uint8_t* base, int rd, int kk) -> bf16x8 {
    if constexpr (BR) return *reinterpret_cast<const bf16x8*>(base + (rd ^ (kk << 5)));
    const uint8_t* p = base + rd + kk * 8192;
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p);
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p + 2048));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  auto read_frags = [&](auto nmb_c, auto nx_c, const uint8_t* sa, const uint8_t* sb, int kk, int AX, Frags& f) {
    constexpr int NMB = decltype(nmb_c)::value;
    constexpr int NX = decltype(nx_c)::value;
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) f.b[nb] = frag_b(sb, b_rd[nb], kk);
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb) f.a[mb] = *reinterpret_cast<const bf16x8*>(sa + (a_rd[kk][mb] ^ AX));
    if constexpr (NX > 0) {
#pragma unroll
      for (int xb = 0; xb < NX; ++xb)
        f.xa[xb] = *reinterpret_cast<const bf16x8*>(sa + xb * 32 * kBK2 * 2 + (xa_rd[kk] ^ AX));
      f.xb = frag_b(sb, xb_rd, kk);
    }
  };
  auto mfmas = [&](auto nmb_c, auto nx_c, const Frags& f, f32x16* acc_x) {
    constexpr int NMB = decltype(nmb_c)::value;
    constexpr int NX = decltype(nx_c)::value;
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
        acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.b[nb], f.a[mb], acc[mb][nb], 0, 0, 0);
#pragma unroll
    for (int xb = 0; xb < NX; ++xb)
      acc_x[xb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.xb, f.xa[xb], acc_x[xb], 0, 0, 0);
  };
  // The waits at the end of a step: the DMAs of step kt + 1 must have landed. Newer than those:
  // after P = 0: B kt + 2, this step's A stage (kDmaA2 + band) and B kt + 3; after P = 1: B kt + 2
  // and B kt + 3. (A stage of step kt + 1 went out at step kt - 1 with B kt + 2 after it.)
  auto wait_p0 = [&](int band) {
    if (band)
      asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(2 * kDmaB + kDmaA2 + 1) : "memory");
    else
      asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(2 * kDmaB + kDmaA2) : "memory");
  };
  // One step kt (P = kt % 2) computing from sa / sb; `io` are the operands of the DMAs this step
  // issues: at P = 0 A stage ast into pa; B step bst into pb. LAST: the tile's last step, whose
  // end waits for nothing (its successors' DMAs belong to the next tile).
  auto step = [&](auto nmb_c, auto x_c, auto p_c, f32x16* acc_x, const Ops& io, int ast, int bst, const uint8_t* sa,
                  const uint8_t* sb, uint8_t* pa, uint8_t* pb, bool last) {
    constexpr int NMB = decltype(nmb_c)::value;
    constexpr int NX = decltype(x_c)::value;
    constexpr int P = decltype(p_c)::value;
    constexpr int AX = P * 64;
    auto issue = [&]() {
      if constexpr (P == 0) dma_a(io, ast, pa);
      dma_b(io, bst, pb);
    };
    if constexpr (NMB == 0) {
      issue();
    } else if constexpr (NX > 0) {
      Frags f;
      read_frags(nmb_c, x_c, sa, sb, 0, AX, f);
      issue();
      mfmas(nmb_c, x_c, f, acc_x);
      read_frags(nmb_c, x_c, sa, sb, 1, AX, f);
      mfmas(nmb_c, x_c, f, acc_x);
    } else {
      Frags f0, f1;
      read_frags(nmb_c, x_c, sa, sb, 0, AX, f0);
      read_frags(nmb_c, x_c, sa, sb, 1, AX, f1);
      issue();
      mfmas(nmb_c, x_c, f0, acc_x);
      mfmas(nmb_c, x_c, f1, acc_x);
    }
    if (last)
      asm volatile("s_barrier" ::: "memory");
    else if constexpr (P == 0)
      wait_p0(io.band);
    else
      asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(2 * kDmaB) : "memory");
  };

  // ---- the walk
  Tile cur;
  decode(L, cur);
  Ops ops;
  if constexpr (GATHER) {  // the first tile's slot map straight from global memory
    int* tmp = s_slot;
    for (int i = tid; i < kBMX; i += kGemmThreads) tmp[i] = i < cur.mvalid ? g.a_slot[cur.m0 + i] : 0;
    __syncthreads();
  }
  set_ops(cur, s_slot, ops);
  __syncthreads();  // every wave has read the slot map before it is overwritten
  dma_a(ops, 0, sA0);
  dma_b(ops, 0, sB0);
  dma_b(ops, 1, sB1);
  dma_b(ops, 2, sB2);
  int pending_stores = 0;  // stores of the previous tile's epilogue still counted in vmcnt
  const int KT = (K + kBK - 1) / kBK;
  const int KT4 = max(kStages, (KT + kStages - 1) / kStages * kStages);
  using P0 = std::integral_constant<int, 0>;
  using P1 = std::integral_constant<int, 1>;
  constexpr int kEpiStores = EPI == kEpiStore ? 16 : 8;  // buffer stores per wave per epilogue
  while (true) {
    const int Ln = pos(rnd + 1);
    const bool has_next = Ln >= 0;
    // A stage 0 and B step 0 of this tile have landed (B 1, B 2 and the previous epilogue's
    // stores may still be in flight)
    if (pending_stores)
      asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(2 * kDmaB + kEpiStores) : "memory");
    else
      asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(2 * kDmaB) : "memory");
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
#pragma unroll
        for (int qq = 0; qq < 16; ++qq) acc[mb][nb][qq] = 0.0f;
    f32x16 acc_x[2];
#pragma unroll
    for (int xb = 0; xb < 2; ++xb)
#pragma unroll
      for (int qq = 0; qq < 16; ++qq) acc_x[xb][qq] = 0.0f;

    // K loop of this tile; the last four steps switch the DMA operands to the next tile after
    // their first step (a tile without a successor keeps its own operands: zero-filling DMAs)
    auto run = [&](auto nmb_c, auto x_c) {
      if (GATHER && has_next) {  // older than step 0's DMAs: step 1's wait covers it
        Tile nx;
        decode(Ln, nx);
        dma_slots(nx);
      }
      for (int kt = 0; kt < KT4 - kStages; kt += kStages) {
        step(nmb_c, x_c, P0{}, acc_x, ops, kt / 2 + 1, kt + 3, sA0, sB0, sA1, sB3, false);
        step(nmb_c, x_c, P1{}, acc_x, ops, 0, kt + 4, sA0, sB1, nullptr, sB0, false);
        step(nmb_c, x_c, P0{}, acc_x, ops, kt / 2 + 2, kt + 5, sA1, sB2, sA0, sB1, false);
        step(nmb_c, x_c, P1{}, acc_x, ops, 0, kt + 6, sA1, sB3, nullptr, sB2, false);
      }
      const int kt = KT4 - kStages;
      step(nmb_c, x_c, P0{}, acc_x, ops, kt / 2 + 1, kt + 3, sA0, sB0, sA1, sB3, false);
      // the slot map DMA is only known to have landed after step 1's wait; with one group of four
      // steps (K <= 128) wait for it here
      if (GATHER && has_next && kt == 0) asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
      Tile nxt = cur;
      if (has_next) {
        decode(Ln, nxt);
        set_ops(nxt, s_slot, ops);
      }
      const int o = has_next ? KT4 : 0;  // the next tile's steps 0..2 (or zero fills past K)
      step(nmb_c, x_c, P1{}, acc_x, ops, 0, kt + 4 - o, sA0, sB1, nullptr, sB0, false);
      step(nmb_c, x_c, P0{}, acc_x, ops, kt / 2 + 2 - o / 2, kt + 5 - o, sA1, sB2, sA0, sB1, false);
      step(nmb_c, x_c, P1{}, acc_x, ops, 0, kt + 6 - o, sA1, sB3, nullptr, sB2, true);
      if constexpr (decltype(x_c)::value > 0) {
        int zx;  // (an opaque lane id: the band's store addresses are not hoisted out of the tile loop)
        asm volatile("v_mov_b32 %0, 0" : "=v"(zx));
#pragma unroll
        for (int xb = 0; xb < decltype(x_c)::value; ++xb)
          store_extra<EPI>(g, acc_x[xb], xb, cur.m0, cur.mvalid, cur.nt * kBN, cur.nt, g0, wm, wn, lane + zx);
      }
      return nxt;
    };
    using F = std::integral_constant<int, 0>;
    Tile nxt;
    if (cur.mvalid > kBM) {
      if (cur.mvalid > kBM + 32)
        nxt = run(std::integral_constant<int, 2>{}, std::integral_constant<int, 2>{});
      else
        nxt = run(std::integral_constant<int, 2>{}, std::integral_constant<int, 1>{});
    } else {
      const int wrows = cur.mvalid - wm * 64;
      const int nmb = __builtin_amdgcn_readfirstlane(wrows <= 0 ? 0 : min(2, (wrows + 31) / 32));
      switch (nmb) {
        case 2: nxt = run(std::integral_constant<int, 2>{}, F{}); break;
        case 1: nxt = run(std::integral_constant<int, 1>{}, F{}); break;
        default: nxt = run(std::integral_constant<int, 0>{}, F{}); break;
      }
    }

    // ---- epilogue: every wave writes its bf16 block (SwiGLU: 64 rows x 64 h columns; store: 64 x
    // 128) as 32 x 64 pieces, each transposed through the wave's own 4 KB of sA1 (free after the
    // last step's barrier; the prefetches went to sA0 and sB0..sB2), so that each store writes
    // whole 128-byte row segments. Lane holds row (lane & 31) of each 32-row block and, per
    // 32-column block, columns (q / 4) * 8 + (lane / 32) * 4 + q % 4 for element q; in the wave's
    // buffer, 16-byte chunk c of row r sits at chunk c ^ (r & 7). Only the wave itself reads what it
    // wrote, so no workgroup barrier is needed until the end. The lane terms are built from a value
    // the compiler cannot see through, so that they are computed here rather than hoisted out of
    // the tile loop (where they would stay live through K).
    int zv;
    asm volatile("v_mov_b32 %0, 0" : "=v"(zv));
    const int lane_e = lane + zv;
    const int lr = lane_e & 31;
    uint8_t* const wbuf = sA1 + wave * 4096;
    const __amdgpu_buffer_rsrc_t rsC = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(g.C + (int64_t)cur.m0 * g.ldc), (short)0, min(cur.mvalid, kBM) * g.ldc * 2, kBufferWord3);
    // rows row0 .. row0 + 31 of the tile, global columns col0 .. col0 + 63 (rows past the tile are
    // dropped by the descriptor, columns past N by their offset): 4 buffer stores per lane
    auto piece_out = [&](const uint2 (&v)[2][4], int row0, int col0) {
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int gq = 0; gq < 4; ++gq)
          *reinterpret_cast<uint2*>(wbuf + lr * 128 + (((nb * 4 + gq) ^ (lr & 7)) << 4) + (lane_e >> 5) * 8) =
              v[nb][gq];
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = j * 8 + (lane_e >> 3), c = lane_e & 7;
        const u32x4 w = *reinterpret_cast<const u32x4*>(wbuf + r * 128 + ((c ^ (r & 7)) << 4));
        const int col = col0 + c * 8;
        const int off = col < g.N ? ((row0 + r) * g.ldc + col) * 2 : kOutOfRange;
        __builtin_amdgcn_raw_buffer_store_b128(w, rsC, off, 0, 0);
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // read back before the buffer is rewritten
    };
    if constexpr (EPI == kEpiStore) {
      // pieces are the wave's column halves of each 32-row block, rounded to bf16 one at a time
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int nh = 0; nh < 2; ++nh) {
          uint2 pk[2][4];
#pragma unroll
          for (int nb = 0; nb < 2; ++nb)
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
              const f32x16& a = acc[mb][2 * nh + nb];
              pk[nb][gq] = make_uint2(pack_bf16x2(a[gq * 4 + 0], a[gq * 4 + 1]), pack_bf16x2(a[gq * 4 + 2], a[gq * 4 + 3]));
            }
          piece_out(pk, wm * 64 + mb * 32, cur.nt * kBN + wn * 128 + nh * 64);
        }
    } else {
      // The saved g | u (training only) go out straight from the accumulators; then h = silu(g) u
      // is rounded to bf16 (32 packed registers), one piece per 32-row block
      if (g.gu_out) {
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
          const int mloc = wm * 64 + mb * 32 + lr;
          if (mloc < cur.mvalid) {
            uint16_t* gs = g.gu_out + (int64_t)(cur.m0 + mloc) * 2 * g.N;
#pragma unroll
            for (int nb = 0; nb < 2; ++nb)
#pragma unroll
              for (int gq = 0; gq < 4; ++gq) {
                const int col = cur.nt * 128 + wn * 64 + nb * 32 + gq * 8 + (lane_e >> 5) * 4;
                if (col >= g.N) continue;
                *reinterpret_cast<uint2*>(gs + col) =
                    make_uint2(pack_bf16x2(acc[mb][nb][gq * 4 + 0], acc[mb][nb][gq * 4 + 1]),
                               pack_bf16x2(acc[mb][nb][gq * 4 + 2], acc[mb][nb][gq * 4 + 3]));
                *reinterpret_cast<uint2*>(gs + g.N + col) =
                    make_uint2(pack_bf16x2(acc[mb][nb + 2][gq * 4 + 0], acc[mb][nb + 2][gq * 4 + 1]),
                               pack_bf16x2(acc[mb][nb + 2][gq * 4 + 2], acc[mb][nb + 2][gq * 4 + 3]));
              }
          }
        }
      }
      uint2 hp[2][2][4];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
#pragma unroll
          for (int gq = 0; gq < 4; ++gq) {
            float hv[4];
#pragma unroll
            for (int qq = 0; qq < 4; ++qq) hv[qq] = silu_f(acc[mb][nb][gq * 4 + qq]) * acc[mb][nb + 2][gq * 4 + qq];
            hp[mb][nb][gq] = make_uint2(pack_bf16x2(hv[0], hv[1]), pack_bf16x2(hv[2], hv[3]));
          }
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) piece_out(hp[mb], wm * 64 + mb * 32, cur.nt * 128 + wn * 64);
    }
    // every wave is done with sA1 before the next tile's first step refills it
    asm volatile("s_barrier" ::: "memory");
    if (!has_next) break;
    cur = nxt;
    L = Ln;
    ++rnd;
    pending_stores = 1;
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the last zero-filling DMAs into LDS
}

// ---------------------------------------------------------------------------------------------
static inline int round_up8(int64_t v) { return (int)((v + 7) / 8 * 8); }

static int cu_count() {
  static int cus = 0;
  if (cus == 0) {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0)
      cus = n;
    else
      cus = 256;
  }
  return cus;
}

// persistent forward product: one workgroup per CU, a multiple of 8 (workgroups of an XCD without
// a tile exit after building the tile list)
template <int EPI, bool GATHER>
static void launch_fwd(GemmArgs g, hipStream_t s) {
  const int64_t grid = std::max(8, cu_count() / 8 * 8);
  // K a multiple of four K steps (no tail, whole groups of four steps): per-step descriptor moves
  if (g.K % (kStages * kBK) == 0)
    hipLaunchKernelGGL((grouped_gemm_fwd_kernel<EPI, GATHER, true>), dim3((unsigned)grid), dim3(kGemmThreads), 0, s,
                       g);
  else
    hipLaunchKernelGGL((grouped_gemm_fwd_kernel<EPI, GATHER, false>), dim3((unsigned)grid), dim3(kGemmThreads), 0, s,
                       g);
}

// the persistent kernel with row-tile weights (K a multiple of four K steps)
static void launch_fwd_rows(GemmArgs g, hipStream_t s) {
  const int64_t grid = std::max(8, cu_count() / 8 * 8);
  hipLaunchKernelGGL((grouped_gemm_fwd_kernel<kEpiStore, false, true, true>), dim3((unsigned)grid), dim3(kGemmThreads),
                     0, s, g);
}

template <bool A_ROWS, bool B_ROWS, int EPI>
static void launch_generic(GemmArgs g, int64_t grid, hipStream_t s) {
  hipLaunchKernelGGL((grouped_gemm_bf16_kernel<A_ROWS, B_ROWS, EPI>), dim3(round_up8(grid)), dim3(kGemmThreads), 0, s,
                     g);
}

// worst-case row tiles over any distribution of N rows among E experts
static inline int64_t row_tiles_bound(int N, int E) { return ((int64_t)N + (int64_t)E * (kBMX - 1)) / kBMX; }

// x_perm [N, H] holds the grouped rows; or, with slot_of_row, x is the token matrix [T, H] and row r
// is token slot_of_row[r] / k (the rows are gathered inside the GEMM)
hipError_t launch_gemm_gate_up(const void* x_perm, const void* gate_up, int dt, int N, int H, int I, int E,
                               const int32_t* offsets, void* h, void* gu_saved, hipStream_t s,
                               const int32_t* slot_of_row, int k, int T) {
  if (mfma_shapes_ok(dt, H, I, x_perm, gate_up, h, gu_saved)) {
    GemmArgs g{};
    g.A = (const uint16_t*)x_perm;
    g.a_slot = slot_of_row;
    g.a_div = k;
    g.M = T;
    g.B = (const uint16_t*)gate_up;
    g.C = (uint16_t*)h;
    g.gu_out = (uint16_t*)gu_saved;
    g.offsets = offsets;
    g.E = E;
    g.N = I;
    g.K = H;
    g.lda = H;
    g.ldb = 2 * I;
    g.ldc = I;
    g.b_expert = (int64_t)H * 2 * I;
    g.b_rows = H;
    g.ntiles_n = (I + 127) / 128;
    if (slot_of_row)
      launch_fwd<kEpiSwiglu, true>(g, s);
    else
      launch_fwd<kEpiSwiglu, false>(g, s);
  } else {
    return launch_gen_ffn1(x_perm, gate_up, dt, offsets, E, N, H, I, h, gu_saved, slot_of_row, k, s);
  }
  return hipGetLastError();
}

hipError_t launch_gemm_down(const void* h, const void* down, int dt, int N, int H, int I, int E, const int32_t* offsets,
                            void* y, hipStream_t s) {
  if (mfma_shapes_ok(dt, H, I, h, down, y)) {
    GemmArgs g{};
    g.A = (const uint16_t*)h;
    g.B = (const uint16_t*)down;
    g.C = (uint16_t*)y;
    g.offsets = offsets;
    g.E = E;
    g.N = H;
    g.K = I;
    g.lda = I;
    g.ldb = H;
    g.ldc = H;
    g.b_expert = (int64_t)I * H;
    g.b_rows = I;
    g.ntiles_n = (H + kBN - 1) / kBN;
    launch_fwd<kEpiStore, false>(g, s);
  } else {
    return launch_gen_ffn2(h, down, dt, offsets, E, N, H, I, y, s);
  }
  return hipGetLastError();
}

// ---- backward (bf16) --------------------------------------------------------------------------
// dGU[r] = SwiGLU'(dY[r] down_e^T, g, u): rows grouped; A = dY (K = H contiguous), B = down_e rows
// (n = i, K = H contiguous); epilogue writes dG into columns [0, I) and dU into [I, 2I).
hipError_t launch_gemm_down_bwd(const void* d_y, const void* down, const void* gu_saved, int N, int H, int I, int E,
                                const int32_t* offsets, void* d_gu, hipStream_t s) {
  GemmArgs g{};
  g.A = (const uint16_t*)d_y;
  g.B = (const uint16_t*)down;
  g.C = (uint16_t*)d_gu;
  g.gu = (const uint16_t*)gu_saved;
  g.offsets = offsets;
  g.E = E;
  g.N = I;
  g.K = H;
  g.lda = H;
  g.ldb = H;
  g.ldc = 2 * I;
  g.b_expert = (int64_t)I * H;
  g.b_rows = I;
  g.ntiles_n = (I + kBN - 1) / kBN;
  launch_generic<true, true, kEpiSwigluBwd>(g, row_tiles_bound(N, E) * g.ntiles_n, s);
  return hipGetLastError();
}

// dX[r] = dGU[r] gate_up_e^T: rows grouped; A = dGU (K = 2I contiguous), B = gate_up_e rows (n = h).
hipError_t launch_gemm_gate_up_bwd(const void* d_gu, const void* gate_up, int N, int H, int I, int E,
                                   const int32_t* offsets, void* d_x, hipStream_t s) {
  GemmArgs g{};
  g.A = (const uint16_t*)d_gu;
  g.B = (const uint16_t*)gate_up;
  g.C = (uint16_t*)d_x;
  g.offsets = offsets;
  g.E = E;
  g.N = H;
  g.K = 2 * I;
  g.lda = 2 * I;
  g.ldb = 2 * I;
  g.ldc = H;
  g.b_expert = (int64_t)H * 2 * I;
  g.b_rows = H;
  g.ntiles_n = (H + kBN - 1) / kBN;
  if ((2 * I) % (kStages * kBK) == 0)
    launch_fwd_rows(g, s);
  else
    launch_generic<true, true, kEpiStore>(g, row_tiles_bound(N, E) * g.ntiles_n, s);
  return hipGetLastError();
}

// dW_e = P_e^T Q_e over the rows of expert e: P [rows, M] and Q [rows, Nq] both row-major, so both
// are k-row tiles; the result block of expert e is [M, Nq] at dW + e * M * Nq. Every expert gets a
// block (zeros when it has no rows).
hipError_t launch_gemm_wgrad(const void* P, const void* Q, int M, int Nq, int E, const int32_t* offsets, void* d_w,
                             hipStream_t s, int max_wg) {
  GemmArgs g{};
  g.A = (const uint16_t*)P;
  g.B = (const uint16_t*)Q;
  g.C = (uint16_t*)d_w;
  g.offsets = offsets;
  g.E = E;
  g.M = M;
  g.N = Nq;
  g.lda = M;
  g.ldb = Nq;
  g.ldc = Nq;
  g.c_expert = (int64_t)M * Nq;
  g.ntiles_m = (M + kBM - 1) / kBM;
  g.ntiles_n = (Nq + kBN - 1) / kBN;
  const int64_t total = (int64_t)E * g.ntiles_m * g.ntiles_n;
  // one workgroup per CU (each holds most of the LDS and a full register file); the experts with
  // at most kResK rows go to the resident kernel, the others to the streaming one (each kernel
  // counts its own work on the device, and a workgroup without any exits at once)
  static int cus = 0;
  if (cus == 0) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) !=
                                                 hipSuccess || cus <= 0)
      cus = 256;
  }
  // a multiple of 8 (the tile lists are split over the 8 XCDs), at least 8
  const int64_t cap = max_wg > 0 ? std::max<int64_t>(8, std::min(max_wg, cus) / 8 * 8) : round_up8(cus);
  const int64_t grid_res = std::min<int64_t>(round_up8((int64_t)E * g.ntiles_m), cap);
  const int64_t grid = std::min<int64_t>(round_up8(total), cap);
  hipLaunchKernelGGL(grouped_wgrad_res_kernel, dim3((unsigned)grid_res), dim3(kGemmThreads), 0, s, g);
  hipLaunchKernelGGL(grouped_wgrad_kernel, dim3((unsigned)grid), dim3(kGemmThreads), 0, s, g);
  return hipGetLastError();
}

}  // namespace moe
