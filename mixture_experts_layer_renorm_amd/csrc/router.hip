// Router: gate logits, then softmax -> top-k -> renormalised weights.
//
// The MoE block of the MindSpeed-MM InternVL3.5 practice doc (issue 625, sections 8.2 and 8.3)
// routes each token with gate -> FP32 softmax -> top-k -> weight normalisation. Each logit is four
// fp32 fused-multiply-add chains, one per fixed block of the hidden dimension, each in ascending h,
// added in block order: a fixed order, so that the top-k decision is reproducible bit for bit by a
// sequential CPU implementation. Selection works on the logits (softmax is monotone); ties go to the
// lower expert index.
#include "common.hpp"
#include "internal.hpp"

namespace moe {

// ---------------------------------------------------------------------------------------------
// logits[t, e] = ((c0 + c1) + c2) + c3 in fp32, c_b = the chain fma(x[t,h], w_gate[h,e], acc) from
// acc = 0 over the h of block b in ascending order; block b = [b*hblk, min((b+1)*hblk, H)) with
// hblk = logit_block(H) = 128 * ceil(H / 512), a multiple of this kernel's 128-wide chunks (HB).
//
// Lanes are tokens: a workgroup of 8 waves owns 64 tokens (one per lane) and 8 * EQ experts
// (EQ per wave), so a lane runs EQ independent chains, all consuming h = 0, 1, ..., H-1 in order;
// the eight waves share each x tile the workgroup stages (one workgroup per CU, two waves per SIMD).
// The hidden dimension is walked in chunks of HB. Each chunk's x tile [64 x HB] and W_g tile
// [HB x 8*EQ] are loaded into registers DEPTH chunks ahead (the loads of x come from HBM, so
// their latency has to be covered by more than one chunk of arithmetic), widened to fp32 once and
// stored to a double-buffered LDS tile. A lane then reads four h of its own token with one 16-byte
// read (row pitch padded by 4 floats, so 16 consecutive rows cover all banks).
//
// Waves 0-3 run their chains on the vector ALUs: the wave's weights reach every lane through DPP
// row broadcasts (fmac4 below). With four chains per lane, waves 4-7 run theirs on the matrix cores: one
// v_mfma_f32_4x4x1_16b_f32 per h takes x[token][h] from each lane and W_g[h][e] for the four experts
// of a quad, and adds to each of its 16 blocks of 4 tokens x 4 experts the products, one fused
// multiply-add per element onto the accumulator (the operation fmaf performs, measured bit-identical
// to it, subnormals included). The matrix and vector pipelines of a SIMD run at the same time.
constexpr int kLogitWaves = 8;
inline int logit_block(int H) { return 128 * ((H + 511) / 512); }
constexpr int kRd = 3;  // groups of four h whose LDS reads run ahead of the arithmetic
constexpr int kLogitTok = kWave;  // tokens per workgroup

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

// 16 bytes (VEC elements) of row `row` from column `col` without a vector load (rows not 16-byte
// aligned); columns >= ncols read as zero.
template <typename TIn>
__device__ __forceinline__ uint4 load_chunk_scalar(const TIn* __restrict__ row, int col, int ncols) {
  constexpr int VEC = 16 / sizeof(TIn);
  TIn tmp[VEC];
#pragma unroll
  for (int i = 0; i < VEC; ++i) tmp[i] = col + i < ncols ? row[col + i] : TIn(0);
  uint4 v;
  __builtin_memcpy(&v, tmp, 16);
  return v;
}

typedef __attribute__((ext_vector_type(4))) unsigned int u32x4_t;
constexpr int kRawBufferWord3 = 0x00020000;  // gfx9 raw buffer descriptor: 32-bit data, offset addressing
constexpr int kPastEnd = 0x7ffffff0;         // an offset past every descriptor's end: loads return zero

__device__ __forceinline__ uint4 buffer_load16(__amdgpu_buffer_rsrc_t r, int off) {
  const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
  return make_uint4(v[0], v[1], v[2], v[3]);
}

// acc[q] = fma(w[h][q], x[h], acc[q]) for h = 0..3 in order, q = 0..EQ-1: register w[r] holds, in
// lane j of every 16-lane row, the weight of h = r * (16 / EQ) + j / EQ and expert j % EQ, and
// v_fmac_f32_dpp with row_newbcast:j hands lane j's value of its row to all 16 lanes. (The fused
// multiply-add is the same IEEE operation as fmaf; only the operand's lane changes.) The leading
// s_nop covers the wait states a DPP read needs after a vector-ALU write of its source.
template <int EQ>
__device__ __forceinline__ void fmac4(float* acc, const float* w, const float4& x);
template <>
__device__ __forceinline__ void fmac4<4>(float* acc, const float* w, const float4& x) {
  asm("s_nop 1\n\t"
               "v_fmac_f32_dpp %[a0], %[w0], %[x0] row_newbcast:0 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %[a1], %[w0], %[x0] row_newbcast:1 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %[a2], %[w0], %[x0] row_newbcast:2 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %[a3], %[w0], %[x0] row_newbcast:3 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %[a0], %[w0], %[x1] row_newbcast:4 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %[a1], %[w0], %[x1] row_newbcast:5 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %[a2], %[w0], %[x1] row_newbcast:6 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %[a3], %[w0], %[x1] row_newbcast:7 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %[a0], %[w0], %[x2] row_newbcast:8 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %[a1], %[w0], %[x2] row_newbcast:9 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %[a2], %[w0], %[x2] row_newbcast:10 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %[a3], %[w0], %[x2] row_newbcast:11 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %[a0], %[w0], %[x3] row_newbcast:12 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %[a1], %[w0], %[x3] row_newbcast:13 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %[a2], %[w0], %[x3] row_newbcast:14 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %[a3], %[w0], %[x3] row_newbcast:15 row_mask:0xf bank_mask:0xf\n\t"
               : [a0] "+v"(acc[0]), [a1] "+v"(acc[1]), [a2] "+v"(acc[2]), [a3] "+v"(acc[3])
               : [w0] "v"(w[0]), [x0] "v"(x.x), [x1] "v"(x.y), [x2] "v"(x.z), [x3] "v"(x.w));
}
template <>
__device__ __forceinline__ void fmac4<8>(float* acc, const float* w, const float4& x) {
  asm("s_nop 1\n\t"
               "v_fmac_f32_dpp %[a0], %[w0], %[x0] row_newbcast:0 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %[a1], %[w0], %[x0] row_newbcast:1 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %[a2], %[w0], %[x0] row_newbcast:2 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %[a3], %[w0], %[x0] row_newbcast:3 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %[a4], %[w0], %[x0] row_newbcast:4 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %[a5], %[w0], %[x0] row_newbcast:5 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %[a6], %[w0], %[x0] row_newbcast:6 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %[a7], %[w0], %[x0] row_newbcast:7 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %[a0], %[w0], %[x1] row_newbcast:8 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %[a1], %[w0], %[x1] row_newbcast:9 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %[a2], %[w0], %[x1] row_newbcast:10 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %[a3], %[w0], %[x1] row_newbcast:11 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %[a4], %[w0], %[x1] row_newbcast:12 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %[a5], %[w0], %[x1] row_newbcast:13 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %[a6], %[w0], %[x1] row_newbcast:14 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %[a7], %[w0], %[x1] row_newbcast:15 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %[a0], %[w1], %[x2] row_newbcast:0 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %[a1], %[w1], %[x2] row_newbcast:1 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %[a2], %[w1], %[x2] row_newbcast:2 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %[a3], %[w1], %[x2] row_newbcast:3 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %[a4], %[w1], %[x2] row_newbcast:4 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %[a5], %[w1], %[x2] row_newbcast:5 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %[a6], %[w1], %[x2] row_newbcast:6 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %[a7], %[w1], %[x2] row_newbcast:7 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %[a0], %[w1], %[x3] row_newbcast:8 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %[a1], %[w1], %[x3] row_newbcast:9 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %[a2], %[w1], %[x3] row_newbcast:10 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %[a3], %[w1], %[x3] row_newbcast:11 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %[a4], %[w1], %[x3] row_newbcast:12 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %[a5], %[w1], %[x3] row_newbcast:13 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %[a6], %[w1], %[x3] row_newbcast:14 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %[a7], %[w1], %[x3] row_newbcast:15 row_mask:0xf bank_mask:0xf\n\t"
               : [a0] "+v"(acc[0]), [a1] "+v"(acc[1]), [a2] "+v"(acc[2]), [a3] "+v"(acc[3]), [a4] "+v"(acc[4]), [a5] "+v"(acc[5]), [a6] "+v"(acc[6]), [a7] "+v"(acc[7])
               : [w0] "v"(w[0]), [w1] "v"(w[1]), [x0] "v"(x.x), [x1] "v"(x.y), [x2] "v"(x.z), [x3] "v"(x.w));
}

typedef float f32x4_t __attribute__((ext_vector_type(4)));

template <typename TIn, int EQ>
struct LogitTile {
  static constexpr int EB = kLogitWaves * EQ;                     // experts per workgroup
  static constexpr int HB = 128;                                  // hidden chunk (the largest that fits LDS at EQ = 8)
  static constexpr int PITCH = HB + 4;                            // LDS row pitch of the x tile
  static constexpr int DEPTH = 3;                                 // chunks in flight
  static constexpr int G = 32 / EQ;                               // h per software-pipelined group
  static constexpr int VEC = 16 / sizeof(TIn);                    // elements per 16-byte load
  static constexpr int XCH = kLogitTok * HB / VEC;                // 16-byte chunks of the x tile
  static constexpr int WCH = (HB * EB + VEC - 1) / VEC;           // and of the W tile
  static constexpr int XPT = (XCH + kLogitWaves * kWave - 1) / (kLogitWaves * kWave);  // per thread
  static constexpr int WPT = (WCH + kLogitWaves * kWave - 1) / (kLogitWaves * kWave);
};

template <typename TIn, int EQ>
__global__ __launch_bounds__(kLogitWaves * kWave) __attribute__((amdgpu_waves_per_eu(2, 2))) void router_logits_kernel(
    const TIn* __restrict__ x, const TIn* __restrict__ wg, int T, int H, int E, float* __restrict__ logits, int vec_x,
    int vec_w, int hblk) {
  using P = LogitTile<TIn, EQ>;
  constexpr int EB = P::EB, VEC = P::VEC, HB = P::HB, DEPTH = P::DEPTH;
  static_assert(EQ % 4 == 0, "experts per wave come in 16-byte groups");
  __shared__ __attribute__((aligned(16))) float xs[2][kLogitTok][P::PITCH];
  __shared__ __attribute__((aligned(16))) float ws[2][HB][EB];
  const int tid = threadIdx.x, lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int t0 = blockIdx.x * kLogitTok;
  const int e0 = blockIdx.y * EB;
  const int nch = (H + HB - 1) / HB;

  // Global loads. With rows a multiple of 16 bytes (vec_x / vec_w) they are 16-byte buffer loads
  // whose descriptors end at the last token of the workgroup and the last row of W_g; elements
  // past H or E get an offset past the end and read as zero, so there is no branch per element.
  const int rows = min(kLogitTok, T - t0);
  const __amdgpu_buffer_rsrc_t rsx =
      __builtin_amdgcn_make_buffer_rsrc((void*)(x + (int64_t)t0 * H), (short)0, rows * H * (int)sizeof(TIn), kRawBufferWord3);
  const __amdgpu_buffer_rsrc_t rsw =
      __builtin_amdgcn_make_buffer_rsrc((void*)wg, (short)0, H * E * (int)sizeof(TIn), kRawBufferWord3);
  // register stage r holds chunk c with c % DEPTH == r
  uint4 rx[DEPTH][P::XPT], rw[DEPTH][P::WPT];
  auto load = [&](int c, uint4* px, uint4* pw) {
    const int h0 = c * HB;
#pragma unroll
    for (int i = 0; i < P::XPT; ++i) {
      const int q = tid + kLogitWaves * kWave * i;
      if (q < P::XCH) {
        const int tt = q / (HB / VEC), hh = h0 + (q % (HB / VEC)) * VEC;
        if (vec_x)
          px[i] = buffer_load16(rsx, hh < H ? (tt * H + hh) * (int)sizeof(TIn) : kPastEnd);
        else
          px[i] = load_chunk_scalar<TIn>(x + (int64_t)min(t0 + tt, T - 1) * H, hh, H);
      }
    }
#pragma unroll
    for (int i = 0; i < P::WPT; ++i) {
      const int q = tid + kLogitWaves * kWave * i;
      if (q < P::WCH) {
        const int h = h0 + q / (EB / VEC), ee = e0 + (q % (EB / VEC)) * VEC;
        if (vec_w)
          pw[i] = buffer_load16(rsw, (h < H && ee < E) ? (h * E + ee) * (int)sizeof(TIn) : kPastEnd);
        else
          pw[i] = load_chunk_scalar<TIn>(wg + (int64_t)min(h, H - 1) * E, ee, E);
      }
    }
  };
  auto store = [&](int buf, const uint4* px, const uint4* pw) {
#pragma unroll
    for (int i = 0; i < P::XPT; ++i) {
      const int q = tid + kLogitWaves * kWave * i;
      if (q < P::XCH) {
        const int tt = q / (HB / VEC), hh = (q % (HB / VEC)) * VEC;
        float f[VEC];
        widen<TIn>(px[i], f);
#pragma unroll
        for (int v = 0; v < VEC; v += 4)
          *reinterpret_cast<float4*>(&xs[buf][tt][hh + v]) = make_float4(f[v], f[v + 1], f[v + 2], f[v + 3]);
      }
    }
#pragma unroll
    for (int i = 0; i < P::WPT; ++i) {
      const int q = tid + kLogitWaves * kWave * i;
      if (q < P::WCH) {
        const int hh = q / (EB / VEC), ee = (q % (EB / VEC)) * VEC;
        float f[VEC];
        widen<TIn>(pw[i], f);
#pragma unroll
        for (int v = 0; v < VEC; v += 4)
          *reinterpret_cast<float4*>(&ws[buf][hh][ee + v]) = make_float4(f[v], f[v + 1], f[v + 2], f[v + 3]);
      }
    }
  };

  float acc[EQ];
#pragma unroll
  for (int q = 0; q < EQ; ++q) acc[q] = 0.0f;

  // h = hh of the chunk in LDS buffer buf, for the lane's token and the wave's EQ experts
  auto fma_h = [&](int buf, int hh, float xe) {
    const float* wl = &ws[buf][hh][wave * EQ];
#pragma unroll
    for (int q = 0; q < EQ; q += 4) {
      const float4 wv = *reinterpret_cast<const float4*>(wl + q);
      acc[q + 0] = __builtin_fmaf(xe, wv.x, acc[q + 0]);
      acc[q + 1] = __builtin_fmaf(xe, wv.y, acc[q + 1]);
      acc[q + 2] = __builtin_fmaf(xe, wv.z, acc[q + 2]);
      acc[q + 3] = __builtin_fmaf(xe, wv.w, acc[q + 3]);
    }
  };
  const int wrow = (lane & 15) / EQ, wcol = (lane & 15) % EQ;  // the lane's value in a W register
  auto compute = [&](int c) {
    const int buf = c & 1;
    const int nh = min(HB, H - c * HB);
    const float* xl = &xs[buf][lane][0];
    if (nh == HB) {
      // four h at a time: the lane's x for them (one 16-byte read) and the wave's weights for them
      // (16 values per register, replicated over the four 16-lane rows), consumed by fmac with a
      // row_newbcast operand; the reads run kRd groups of four h ahead of the fmacs
      float4 xv[kRd + 1];
      float wv[kRd + 1][EQ / 4];
      auto rd = [&](int h4, int slot) {
        xv[slot] = *reinterpret_cast<const float4*>(xl + h4);
#pragma unroll
        for (int r = 0; r < EQ / 4; ++r) wv[slot][r] = ws[buf][h4 + r * (16 / EQ) + wrow][wave * EQ + wcol];
      };
#pragma unroll
      for (int i = 0; i < kRd; ++i) rd(4 * i, i);
#pragma unroll
      for (int h4 = 0; h4 < HB; h4 += 4) {
        const int cs = (h4 / 4) % (kRd + 1);
        if (h4 + 4 * kRd < HB) rd(h4 + 4 * kRd, (cs + kRd) % (kRd + 1));
        fmac4<EQ>(acc, wv[cs], xv[cs]);
      }
    } else {
      for (int hh = 0; hh < nh; ++hh) fma_h(buf, hh, xl[hh]);
    }
  };

  // matrix-core waves: quad q of the wave's experts accumulates in macc[q]; lane l holds, in element
  // m, the logit of token 4 * (l / 4) + m and expert 4 q + l % 4 of the wave
  // (with eight chains per lane the matrix-core waves would read twice the weights per h and the
  // kernel becomes bound by LDS reads: measured slower, so that launch keeps every wave on the vector ALUs)
  const bool mx = EQ == 4 && wave >= kLogitWaves / 2;
  f32x4_t macc[EQ / 4];
#pragma unroll
  for (int q = 0; q < EQ / 4; ++q) macc[q] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  const int wc = wave * EQ + (lane & 3);
  auto compute_mx = [&](int c) {
    const int buf = c & 1;
    const int nh = min(HB, H - c * HB);
    const float* xl = &xs[buf][lane][0];
    if (nh == HB) {
      // four h at a time, read kRd groups ahead
      float4 xv[kRd + 1];
      float wv[kRd + 1][4][EQ / 4];
      auto rd = [&](int h4, int slot) {
        xv[slot] = *reinterpret_cast<const float4*>(xl + h4);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int q = 0; q < EQ / 4; ++q) wv[slot][i][q] = ws[buf][h4 + i][wc + 4 * q];
      };
#pragma unroll
      for (int i = 0; i < kRd; ++i) rd(4 * i, i);
#pragma unroll
      for (int h4 = 0; h4 < HB; h4 += 4) {
        const int cs = (h4 / 4) % (kRd + 1);
        if (h4 + 4 * kRd < HB) rd(h4 + 4 * kRd, (cs + kRd) % (kRd + 1));
        const float xa[4] = {xv[cs].x, xv[cs].y, xv[cs].z, xv[cs].w};
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int q = 0; q < EQ / 4; ++q)
            macc[q] = __builtin_amdgcn_mfma_f32_4x4x1f32(xa[i], wv[cs][i][q], macc[q], 0, 0, 0);
      }
    } else {
      for (int hh = 0; hh < nh; ++hh) {
        const float xa = xl[hh];
#pragma unroll
        for (int q = 0; q < EQ / 4; ++q)
          macc[q] = __builtin_amdgcn_mfma_f32_4x4x1f32(xa, ws[buf][hh][wc + 4 * q], macc[q], 0, 0, 0);
      }
    }
  };

  // The hidden dimension is four blocks of hblk (a multiple of the chunk) units: at the end of a
  // block its chains are added to the running totals (the first block's chains are the totals)
  // and restarted from zero; blocks past H add +0.0.
  float tot[EQ];
  f32x4_t mtot[EQ / 4];
  int nfold = 0;
  auto fold = [&]() {
    if (mx) {
#pragma unroll
      for (int q = 0; q < EQ / 4; ++q) {
        mtot[q] = nfold == 0 ? macc[q] : mtot[q] + macc[q];
        macc[q] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
      }
    } else {
#pragma unroll
      for (int q = 0; q < EQ; ++q) {
        tot[q] = nfold == 0 ? acc[q] : tot[q] + acc[q];
        acc[q] = 0.0f;
      }
    }
    ++nfold;
  };
  const int cpb = hblk / HB;  // chunks per block

  // prologue: chunks 0 .. depth-1 in flight
#pragma unroll
  for (int r = 0; r < DEPTH; ++r)
    if (r < nch) load(r, rx[r], rw[r]);
  // steady state, unrolled by the register depth so that every stage index is a constant
  for (int c0 = 0; c0 < nch; c0 += DEPTH) {
#pragma unroll
    for (int r = 0; r < DEPTH; ++r) {
      const int c = c0 + r;
      if (c < nch) {
        store(c & 1, rx[r], rw[r]);
        __syncthreads();
        if (c + DEPTH < nch) load(c + DEPTH, rx[r], rw[r]);
        if (mx)
          compute_mx(c);
        else
          compute(c);
        if ((c + 1) % cpb == 0 || c == nch - 1) fold();
      }
    }
  }
  while (nfold < 4) fold();  // (H = 0 folds four zero blocks)

  if (mx) {
#pragma unroll
    for (int q = 0; q < EQ / 4; ++q)
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int t = t0 + (lane & ~3) + m, e = e0 + wave * EQ + 4 * q + (lane & 3);
        if (t < T && e < E) logits[(int64_t)t * E + e] = mtot[q][m];
      }
    return;
  }
  const int t = t0 + lane;
  if (t < T) {
    float* out = logits + (int64_t)t * E + e0 + wave * EQ;
    if (e0 + wave * EQ + EQ <= E && (E & 3) == 0) {
#pragma unroll
      for (int q = 0; q < EQ; q += 4)
        *reinterpret_cast<float4*>(out + q) = make_float4(tot[q], tot[q + 1], tot[q + 2], tot[q + 3]);
    } else {
#pragma unroll
      for (int q = 0; q < EQ; ++q)
        if (e0 + wave * EQ + q < E) out[q] = tot[q];
    }
  }
}

// ---------------------------------------------------------------------------------------------
// The same logits on the matrix cores (bf16 inputs, H % 32 == 0, E % 8 == 0, 16-byte aligned):
// v_mfma_f32_32x32x1f32 adds, to each element of two 32 x 32 blocks, the product of one A and one
// B value with a single fused multiply-add (K = 1; the operation fmaf performs), so a chain of
// them over h is the fmaf chain of every (token, expert) element. The four blocks of h make four
// times as many independent chains as there are logits, enough to keep every SIMD on its own
// chains: a workgroup of four waves owns 64 tokens x 32 experts, wave w runs block w's chains
// (lanes 0-31 feed tokens 0-31 and lanes 32-63 tokens 32-63, both against the same 32 experts),
// and the four partial chains are added in block order at the end through LDS.
// Each wave streams its block's x [64 tokens][32 h] and W_g [32 h][32 experts] in 32-h chunks
// through a 3-deep LDS ring of its own (no barrier between waves in the loop); the 16-byte pieces
// of each 64-byte x row are XOR-swizzled by row so that the 64 lanes reading one h of their own
// rows spread over 16 bank groups, and the W_g value of a lane's expert is a broadcast read.
// The operands reach the matrix cores without a conversion instruction (on this chip a vector
// instruction between two MFMAs of a wave costs as much issue time as a tenth of an MFMA): every
// operand register keeps a zero low half, and ds_read_u16_d16_hi replaces only its high half, so
// the register holds exactly the fp32 value of the bf16 number. Groups of 8 h run back to back on
// one of two register sets while the other set is loaded for the next 8 h.
constexpr int kRtTok = 64, kRtExp = 32, kRtHc = 32;

typedef __attribute__((ext_vector_type(4))) int rt_i32x4;
// raw buffer descriptor over [p, p + bytes): 32-bit offsets, loads past the end return zero
__device__ __forceinline__ rt_i32x4 rt_rsrc(const void* p, int bytes) {
  const uint64_t a = (uint64_t)p;
  rt_i32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  r[1] = __builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32) & 0xffff);
  r[2] = __builtin_amdgcn_readfirstlane(bytes);
  r[3] = kRawBufferWord3;
  return r;
}
// One wave-wide 1 KB DMA: 16 bytes per lane from rs + voff into LDS at lds + 16 * lane. Written
// as asm so that the compiler does not wait for it before every LDS read: the kernel counts the
// loads itself (s_waitcnt vmcnt).
__device__ __forceinline__ void rt_dma16(const rt_i32x4& rs, int voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff), "s"(rs),
               "s"(lds)
               : "memory", "m0");
}

// waits until at most `ahead` chunks of this wave's DMA (6 loads each) are in flight
template <int N>
__device__ __forceinline__ void rt_wait_chunks(int ahead) {
  if constexpr (N == 0) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  } else {
    if (ahead >= N)
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(6 * N) : "memory");
    else
      rt_wait_chunks<N - 1>(ahead);
  }
}

typedef __attribute__((ext_vector_type(32))) float rt_f32x32;
#define RT_MFMA(a, b) "v_mfma_f32_32x32x1_2b_f32 %0, " a ", " b ", %0\n"
#define RT_LD(d, a, off) "ds_read_u16_d16_hi " d ", " a " offset:" #off "\n"
// Loads 8 h into a register set: x[token = lane][h0 .. h0 + 7] (2-byte steps from xa) and
// W_g[h0 .. h0 + 7][expert] (64-byte steps from wa), into the high halves of nx and nw.
__device__ __forceinline__ void rt_load(uint32_t (&nx)[8], uint32_t (&nw)[8], uint32_t xa, uint32_t wa) {
  asm volatile(RT_LD("%0", "%16", 0) RT_LD("%1", "%16", 2) RT_LD("%2", "%16", 4) RT_LD("%3", "%16", 6)
               RT_LD("%4", "%16", 8) RT_LD("%5", "%16", 10) RT_LD("%6", "%16", 12) RT_LD("%7", "%16", 14)
               RT_LD("%8", "%17", 0) RT_LD("%9", "%17", 64) RT_LD("%10", "%17", 128) RT_LD("%11", "%17", 192)
               RT_LD("%12", "%17", 256) RT_LD("%13", "%17", 320) RT_LD("%14", "%17", 384) RT_LD("%15", "%17", 448)
               : "+v"(nx[0]), "+v"(nx[1]), "+v"(nx[2]), "+v"(nx[3]), "+v"(nx[4]), "+v"(nx[5]), "+v"(nx[6]),
                 "+v"(nx[7]), "+v"(nw[0]), "+v"(nw[1]), "+v"(nw[2]), "+v"(nw[3]), "+v"(nw[4]), "+v"(nw[5]),
                 "+v"(nw[6]), "+v"(nw[7])
               : "v"(xa), "v"(wa)
               : "memory");
}
// Eight chain steps on the set (cx, cw) once its loads have landed; with LOAD, the loads of the
// next 8 h into (nx, nw) are issued after the first MFMA (by then every MFMA that read that set
// has started) and land while the other seven run.
template <bool LOAD>
__device__ __forceinline__ void rt_group(rt_f32x32& acc, const uint32_t (&cx)[8], const uint32_t (&cw)[8],
                                         uint32_t (&nx)[8], uint32_t (&nw)[8], uint32_t xa, uint32_t wa) {
  if constexpr (LOAD) {
    asm volatile("s_waitcnt lgkmcnt(0)\n" RT_MFMA("%17", "%25")
                 RT_LD("%1", "%33", 0) RT_LD("%2", "%33", 2) RT_LD("%3", "%33", 4) RT_LD("%4", "%33", 6)
                 RT_LD("%5", "%33", 8) RT_LD("%6", "%33", 10) RT_LD("%7", "%33", 12) RT_LD("%8", "%33", 14)
                 RT_LD("%9", "%34", 0) RT_LD("%10", "%34", 64) RT_LD("%11", "%34", 128) RT_LD("%12", "%34", 192)
                 RT_LD("%13", "%34", 256) RT_LD("%14", "%34", 320) RT_LD("%15", "%34", 384) RT_LD("%16", "%34", 448)
                 RT_MFMA("%18", "%26") RT_MFMA("%19", "%27") RT_MFMA("%20", "%28") RT_MFMA("%21", "%29")
                 RT_MFMA("%22", "%30") RT_MFMA("%23", "%31") RT_MFMA("%24", "%32")
                 : "+a"(acc), "+v"(nx[0]), "+v"(nx[1]), "+v"(nx[2]), "+v"(nx[3]), "+v"(nx[4]), "+v"(nx[5]),
                   "+v"(nx[6]), "+v"(nx[7]), "+v"(nw[0]), "+v"(nw[1]), "+v"(nw[2]), "+v"(nw[3]), "+v"(nw[4]),
                   "+v"(nw[5]), "+v"(nw[6]), "+v"(nw[7])
                 : "v"(cx[0]), "v"(cx[1]), "v"(cx[2]), "v"(cx[3]), "v"(cx[4]), "v"(cx[5]), "v"(cx[6]), "v"(cx[7]),
                   "v"(cw[0]), "v"(cw[1]), "v"(cw[2]), "v"(cw[3]), "v"(cw[4]), "v"(cw[5]), "v"(cw[6]), "v"(cw[7]),
                   "v"(xa), "v"(wa)
                 : "memory");
  } else {
    asm volatile("s_waitcnt lgkmcnt(0)\n" RT_MFMA("%1", "%9") RT_MFMA("%2", "%10") RT_MFMA("%3", "%11")
                 RT_MFMA("%4", "%12") RT_MFMA("%5", "%13") RT_MFMA("%6", "%14") RT_MFMA("%7", "%15")
                 RT_MFMA("%8", "%16")
                 : "+a"(acc)
                 : "v"(cx[0]), "v"(cx[1]), "v"(cx[2]), "v"(cx[3]), "v"(cx[4]), "v"(cx[5]), "v"(cx[6]), "v"(cx[7]),
                   "v"(cw[0]), "v"(cw[1]), "v"(cw[2]), "v"(cw[3]), "v"(cw[4]), "v"(cw[5]), "v"(cw[6]), "v"(cw[7])
                 : "memory");
  }
}

template <int D>
__global__ __launch_bounds__(256) void router_logits_mfma_kernel(const uint16_t* __restrict__ x,
                                                                 const uint16_t* __restrict__ wg, int T, int H, int E,
                                                                 int hblk, float* __restrict__ logits) {
  __shared__ __attribute__((aligned(1024))) uint8_t sx[4][D][kRtTok * kRtHc * 2];   // 4 KB each
  __shared__ __attribute__((aligned(1024))) uint8_t sw[4][D][kRtHc * kRtExp * 2];   // 2 KB each
  const int tid = threadIdx.x, lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int t0 = blockIdx.x * kRtTok, e0 = blockIdx.y * kRtExp;
  const int hb0 = min(H, wave * hblk), hb1 = min(H, (wave + 1) * hblk);
  const int nch = (hb1 - hb0) / kRtHc;
  const int rows = min(kRtTok, T - t0);
  const rt_i32x4 rsx = rt_rsrc(x + (int64_t)t0 * H, rows * H * 2);
  const rt_i32x4 rsw = rt_rsrc(wg, H * E * 2);
  // DMA lanes: x instruction i fills rows 16 i .. 16 i + 15 (64-byte rows, 4 pieces of 8 h); the
  // lane at LDS piece p of row r fetches piece p ^ ((r >> 2) & 3). W_g instruction i fills h-rows
  // 16 i .. 16 i + 15 (64-byte rows of 32 experts).
  int xo[4], wo[2];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = i * 16 + (lane >> 2), c = (lane & 3) ^ ((r >> 2) & 3);
    xo[i] = (r * H + c * 8) * 2;
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = i * 16 + (lane >> 2);
    wo[i] = (r * E + e0 + (lane & 3) * 8) * 2;
  }
  const uint32_t sx0 = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)sx[wave][0]);
  const uint32_t sw0 = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)sw[wave][0]);
  auto issue = [&](int c, int slot) {
    const int h0 = hb0 + c * kRtHc;
    const uint32_t bx = sx0 + slot * (kRtTok * kRtHc * 2), bw = sw0 + slot * (kRtHc * kRtExp * 2);
#pragma unroll
    for (int i = 0; i < 4; ++i) rt_dma16(rsx, xo[i] + h0 * 2, bx + i * 1024);
#pragma unroll
    for (int i = 0; i < 2; ++i) rt_dma16(rsw, wo[i] + h0 * E * 2, bw + i * 1024);
  };
  rt_f32x32 acc;
#pragma unroll
  for (int i = 0; i < 32; ++i) acc[i] = 0.0f;
  // two operand register sets, low halves zero for the whole kernel
  uint32_t xA[8], wA[8], xB[8], wB[8];
  {
    uint32_t z;
    asm volatile("v_mov_b32 %0, 0" : "=v"(z));
#pragma unroll
    for (int j = 0; j < 8; ++j) xA[j] = wA[j] = xB[j] = wB[j] = z;
  }
  // this lane's x row (token t0 + lane, pieces swizzled) and W_g column (expert e0 + lane % 32)
  const uint32_t xrow = sx0 + lane * 64, xs = (lane >> 2) & 3, wcol = sw0 + (lane & 31) * 2;
  auto xaddr = [&](int slot, int q) { return xrow + slot * (kRtTok * kRtHc * 2) + ((q ^ xs) << 4); };
  auto waddr = [&](int slot, int q) { return wcol + slot * (kRtHc * kRtExp * 2) + q * 512; };
#pragma unroll
  for (int d = 0; d < D - 1; ++d)
    if (d < nch) issue(d, d);
  if (nch > 0) {
    rt_wait_chunks<D - 2>(min(nch - 1, D - 2));  // chunk 0 has landed
    rt_load(xA, wA, xaddr(0, 0), waddr(0, 0));
  }
  asm volatile("s_nop 7" : "+a"(acc));  // the accumulator's initial writes settle before the first MFMA
  // chunks 0 .. nch - 2; the last group of each loads the first 8 h of the next chunk
  for (int c = 0; c + 1 < nch; ++c) {
    const int slot = c % D, nslot = (c + 1) % D;
    rt_group<true>(acc, xA, wA, xB, wB, xaddr(slot, 1), waddr(slot, 1));
    // every LDS read of chunk c - 1 has completed (the group above began with lgkmcnt(0)): its
    // slot takes chunk c + D - 1
    if (c + D - 1 < nch) issue(c + D - 1, (c + D - 1) % D);
    rt_group<true>(acc, xB, wB, xA, wA, xaddr(slot, 2), waddr(slot, 2));
    rt_group<true>(acc, xA, wA, xB, wB, xaddr(slot, 3), waddr(slot, 3));
    rt_wait_chunks<D - 2>(min(nch - 1, c + D - 1) - (c + 1));  // chunk c + 1 has landed
    rt_group<true>(acc, xB, wB, xA, wA, xaddr(nslot, 0), waddr(nslot, 0));
  }
  if (nch > 0) {  // the last chunk
    const int slot = (nch - 1) % D;
    rt_group<true>(acc, xA, wA, xB, wB, xaddr(slot, 1), waddr(slot, 1));
    rt_group<true>(acc, xB, wB, xA, wA, xaddr(slot, 2), waddr(slot, 2));
    rt_group<true>(acc, xA, wA, xB, wB, xaddr(slot, 3), waddr(slot, 3));
    rt_group<false>(acc, xB, wB, xA, wA, 0, 0);
  }
  // the last MFMA's result is complete before the accumulator is read
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+a"(acc));
  // the four blocks' chains, added in block order: element i of the accumulator of this lane is
  // (token 32 (i / 16) + 8 ((i % 16) / 4) + 4 (lane / 32) + i % 4, expert lane % 32)
  __syncthreads();  // every wave is done with its chunks; sx becomes the partial sums
  float* part = reinterpret_cast<float*>(&sx[0][0][0]);  // [4 blocks][64 tokens][32 experts]
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const int tok = 32 * (i >> 4) + 8 * ((i & 15) >> 2) + 4 * (lane >> 5) + (i & 3);
    part[(wave * kRtTok + tok) * kRtExp + (lane & 31)] = acc[i];
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < kRtTok * kRtExp / 256; ++j) {
    const int idx = tid + 256 * j;
    const int tok = idx / kRtExp, ex = idx % kRtExp;
    float v = part[tok * kRtExp + ex];
#pragma unroll
    for (int b = 1; b < 4; ++b) v = v + part[(b * kRtTok + tok) * kRtExp + ex];
    if (t0 + tok < T && e0 + ex < E) logits[(int64_t)(t0 + tok) * E + e0 + ex] = v;
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
// The same selection and weights with L = 8 or 16 lanes per token (E <= 256): lane `sub` of a
// token's group holds experts e = q * L + sub, q = 0..VPL-1 (ascending e per lane), so a round's
// argmax is a local scan plus log2(L) exchanges inside a 16-lane row (DPP quad permutes and the
// row mirrors, a few cycles each, against the 64-lane shuffles above). Slot j is kept by lane
// j % L. A workgroup of 4 waves holds kCountTok = 16 tokens (L = 16: 4 tokens per wave), so it can
// also write those tokens' expert histogram that the permute's plan takes (permute_count_kernel's
// output), and the 256 workgroups of a 4096-token batch spread the k argmax rounds over every CU.
template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xf, 0xf, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(dpp_i<CTRL>(__float_as_int(v)));
}
constexpr int kNoExpert = 0x7fffffff;
// (value, index) order: larger value first, ties to the lower index; kNoExpert = no candidate
__device__ __forceinline__ void take_better(float& bv, int& be, float ov, int oe) {
  const bool take = (oe != kNoExpert) && (be == kNoExpert || ov > bv || (ov == bv && oe < be));
  bv = take ? ov : bv;
  be = take ? oe : be;
}
template <int CTRL>
__device__ __forceinline__ void xchg_better(float& bv, int& be) {
  const float ov = dpp_f<CTRL>(bv);
  const int oe = dpp_i<CTRL>(be);
  take_better(bv, be, ov, oe);
}
// all-reduce over groups of L lanes: quad_perm [1,0,3,2], [2,3,0,1], row_half_mirror, row_mirror
template <int L>
__device__ __forceinline__ void group_best(float& bv, int& be) {
  xchg_better<0xB1>(bv, be);
  xchg_better<0x4E>(bv, be);
  xchg_better<0x141>(bv, be);
  if constexpr (L == 16) xchg_better<0x140>(bv, be);
}
template <int CTRL>
__device__ __forceinline__ void xchg_max64(uint64_t& x) {
  const uint32_t lo = (uint32_t)dpp_i<CTRL>((int)(uint32_t)x), hi = (uint32_t)dpp_i<CTRL>((int)(uint32_t)(x >> 32));
  const uint64_t o = ((uint64_t)hi << 32) | lo;
  x = o > x ? o : x;
}
// all-reduce max of 64-bit keys over groups of L lanes (the same exchanges as group_best)
template <int L>
__device__ __forceinline__ void group_max64(uint64_t& x) {
  xchg_max64<0xB1>(x);
  xchg_max64<0x4E>(x);
  xchg_max64<0x141>(x);
  if constexpr (L == 16) xchg_max64<0x140>(x);
}
template <int L>
__device__ __forceinline__ float group_sum(float v) {
  v += dpp_f<0xB1>(v);
  v += dpp_f<0x4E>(v);
  v += dpp_f<0x141>(v);
  if constexpr (L == 16) v += dpp_f<0x140>(v);
  return v;
}

constexpr int kTopkGroupWaves = 4;
template <int L, int VPL>
__global__ __launch_bounds__(kTopkGroupWaves * kWave) void router_topk_group_kernel(
    const float* __restrict__ logits, int T, int E, int k, int renorm, int32_t* __restrict__ topk_idx,
    float* __restrict__ topk_w, int32_t* __restrict__ chunk_counts) {
  static_assert(L == 8 || L == 16, "a token's lanes stay inside one 16-lane row");
  constexpr int TPW = kWave / L;  // tokens per wave
  constexpr int KR = 32 / L;      // slots kept per lane (k <= 32)
  static_assert(kTopkGroupWaves * TPW == kCountTok, "a workgroup owns one row of the expert histogram");
  __shared__ int cnt[L * VPL];
  const int lane = lane_id(), sub = lane & (L - 1);
  const int t = blockIdx.x * kCountTok + (int)(threadIdx.x / kWave) * TPW + lane / L;
  const bool live = t < T;
  if (chunk_counts) {
    for (int e = threadIdx.x; e < E; e += kTopkGroupWaves * kWave) cnt[e] = 0;
    __syncthreads();
  }
  const float* l = logits + (int64_t)t * E;
  float v[VPL];
  uint32_t valid = 0;
#pragma unroll
  for (int q = 0; q < VPL; ++q) {
    const int e = q * L + sub;
    const bool ok = live && e < E;
    v[q] = ok ? l[e] : 0.0f;
    valid |= ok ? 1u << q : 0u;
  }
  float sv[KR];
  int se[KR];
#pragma unroll
  for (int r = 0; r < KR; ++r) {
    sv[r] = 0.0f;
    se[r] = -1;
  }
  // Order-preserving 64-bit keys: the high word maps the float's bits to an unsigned order (-0 is
  // folded into +0 first, since the two compare equal), the low word is 0xffff - e, so that equal
  // values rank the lower expert higher. A valid expert's key is > 0; absent experts have key 0.
  // Round j takes the largest key below round j-1's: no per-round bookkeeping, no branches.
  uint64_t key[VPL];
#pragma unroll
  for (int q = 0; q < VPL; ++q) {
    const uint32_t b = __float_as_uint(v[q] + 0.0f);
    const uint32_t o = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
    key[q] = ((valid >> q) & 1u) ? ((uint64_t)o << 32) | (uint32_t)(0xffff - (q * L + sub)) : 0ull;
  }
  float m = 0.0f;
  uint64_t prev = ~0ull;
  for (int j = 0; j < k; ++j) {
    uint64_t best = 0;
#pragma unroll
    for (int q = 0; q < VPL; ++q) best = (key[q] < prev && key[q] > best) ? key[q] : best;
    group_max64<L>(best);
    prev = best;
    const uint32_t o = (uint32_t)(best >> 32);
    const float bv = __uint_as_float((o & 0x80000000u) ? (o & 0x7fffffffu) : ~o);
    const int be = 0xffff - (int)(uint32_t)best;  // k <= E: every round finds a valid expert
    if (j == 0) m = bv;
#pragma unroll
    for (int r = 0; r < KR; ++r)
      if (j == r * L + sub) {
        sv[r] = bv;
        se[r] = be;
      }
  }
  float part = 0.0f;
  if (renorm) {
#pragma unroll
    for (int r = 0; r < KR; ++r)
      if (r * L + sub < k) part += expf(sv[r] - m);
  } else {
#pragma unroll
    for (int q = 0; q < VPL; ++q)
      if ((valid >> q) & 1u) part += expf(v[q] - m);
  }
  const float den = group_sum<L>(part);
  if (live) {
#pragma unroll
    for (int r = 0; r < KR; ++r) {
      const int j = r * L + sub;
      if (j < k) {
        topk_idx[(int64_t)t * k + j] = se[r];
        topk_w[(int64_t)t * k + j] = expf(sv[r] - m) / den;
      }
    }
  }
  if (chunk_counts) {
    if (live) {
#pragma unroll
      for (int r = 0; r < KR; ++r)
        if (r * L + sub < k) atomicAdd(&cnt[se[r]], 1);
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += kTopkGroupWaves * kWave) chunk_counts[(int64_t)blockIdx.x * E + e] = cnt[e];
  }
}

// ---------------------------------------------------------------------------------------------
// Router statistics for an auxiliary load-balance loss: the full softmax per token (probs), its
// sum over tokens, and the expert load (how many (token, slot) pairs chose each expert).
// Stage 1: a workgroup of 4 waves owns kStatsTok tokens, a wave a contiguous run of them in
// ascending order; lane j holds experts j, j+64, ... Each wave sums its tokens' probabilities,
// the workgroup adds the four wave sums in wave order and writes one partial row per workgroup,
// and counts its slots' experts in LDS (integers). Stage 2 adds the partial rows in workgroup
// order. No floating-point atomics, so the result is the same on every run.
constexpr int kStatsWaves = 4;
constexpr int kStatsTok = 128;
constexpr int kStatsMaxE = 1024;

size_t router_stats_workspace_bytes(int T, int E) {
  const int64_t nblk = ((int64_t)T + kStatsTok - 1) / kStatsTok;
  return (size_t)(nblk * E * (int64_t)(sizeof(float) + sizeof(int32_t)));
}

template <int VPL>
__global__ __launch_bounds__(kStatsWaves * kWave) void router_stats_kernel(
    const float* __restrict__ logits, const int32_t* __restrict__ topk_idx, int T, int E, int k,
    float* __restrict__ probs, float* __restrict__ part_p, int32_t* __restrict__ part_load) {
  __shared__ float wsum[kStatsWaves][VPL * kWave];
  __shared__ int cnt[kStatsMaxE];
  const int lane = lane_id(), wave = (int)(threadIdx.x / kWave);
  const int blk = blockIdx.x;
  const int t0 = blk * kStatsTok;
  for (int e = threadIdx.x; e < E; e += kStatsWaves * kWave) cnt[e] = 0;
  float acc[VPL];
#pragma unroll
  for (int q = 0; q < VPL; ++q) acc[q] = 0.0f;
  constexpr int TPW = kStatsTok / kStatsWaves;
  for (int i = 0; i < TPW; ++i) {
    const int t = t0 + wave * TPW + i;
    if (t >= T) break;
    const float* l = logits + (int64_t)t * E;
    float v[VPL];
    float m = -INFINITY;
#pragma unroll
    for (int q = 0; q < VPL; ++q) {
      const int e = q * kWave + lane;
      v[q] = e < E ? l[e] : -INFINITY;
      m = fmaxf(m, v[q]);
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, kWave));
    float ex[VPL], se = 0.0f;
#pragma unroll
    for (int q = 0; q < VPL; ++q) {
      ex[q] = q * kWave + lane < E ? expf(v[q] - m) : 0.0f;
      se += ex[q];
    }
    const float den = wave_sum(se);
#pragma unroll
    for (int q = 0; q < VPL; ++q) {
      const int e = q * kWave + lane;
      const float p = ex[q] / den;
      acc[q] += p;
      if (probs && e < E) probs[(int64_t)t * E + e] = p;
    }
  }
#pragma unroll
  for (int q = 0; q < VPL; ++q) wsum[wave][q * kWave + lane] = acc[q];
  __syncthreads();
  const int64_t s0 = (int64_t)t0 * k, s1 = (int64_t)min(T, t0 + kStatsTok) * k;
  for (int64_t s = s0 + threadIdx.x; s < s1; s += kStatsWaves * kWave) {
    const int e = topk_idx[s];
    if (e >= 0 && e < E) atomicAdd(&cnt[e], 1);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kStatsWaves * kWave) {
    part_p[(int64_t)blk * E + e] = ((wsum[0][e] + wsum[1][e]) + wsum[2][e]) + wsum[3][e];
    part_load[(int64_t)blk * E + e] = cnt[e];
  }
}

__global__ __launch_bounds__(256) void router_stats_reduce_kernel(const float* __restrict__ part_p,
                                                                  const int32_t* __restrict__ part_load, int nblk,
                                                                  int E, int T, float* __restrict__ mean_prob,
                                                                  int32_t* __restrict__ load) {
  const int e = blockIdx.x * 256 + (int)threadIdx.x;
  if (e >= E) return;
  float sp = 0.0f;
  int sl = 0;
  int b = 0;
  for (; b + 8 <= nblk; b += 8) {  // eight independent loads at a time, added in block order
    float vp[8];
    int vl[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      vp[u] = part_p[(int64_t)(b + u) * E + e];
      vl[u] = part_load[(int64_t)(b + u) * E + e];
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      sp += vp[u];
      sl += vl[u];
    }
  }
  for (; b < nblk; ++b) {
    sp += part_p[(int64_t)b * E + e];
    sl += part_load[(int64_t)b * E + e];
  }
  mean_prob[e] = sp / (float)T;
  load[e] = sl;
}

hipError_t launch_router_stats(const float* logits, const int32_t* topk_idx, int T, int E, int k, float* probs,
                               float* mean_prob, int32_t* load, void* workspace, hipStream_t s) {
  const int nblk = (T + kStatsTok - 1) / kStatsTok;
  float* part_p = (float*)workspace;
  int32_t* part_load = (int32_t*)(part_p + (int64_t)nblk * E);
  const int vpl = (E + kWave - 1) / kWave;
  dim3 grid(nblk), block(kStatsWaves * kWave);
#define MOE_STATS_CASE(V)                                                                                     \
  case V:                                                                                                    \
    hipLaunchKernelGGL(router_stats_kernel<V>, grid, block, 0, s, logits, topk_idx, T, E, k, probs, part_p, \
                       part_load);                                                                           \
    break;
  switch (vpl <= 1 ? 1 : vpl <= 2 ? 2 : vpl <= 4 ? 4 : vpl <= 8 ? 8 : 16) {
    MOE_STATS_CASE(1)
    MOE_STATS_CASE(2)
    MOE_STATS_CASE(4)
    MOE_STATS_CASE(8)
    MOE_STATS_CASE(16)
  }
#undef MOE_STATS_CASE
  hipLaunchKernelGGL(router_stats_reduce_kernel, dim3((E + 255) / 256), dim3(256), 0, s, part_p, part_load, nblk, E, T,
                     mean_prob, load);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------
template <typename TIn, int EQ>
static void launch_logits_t(const void* x, const void* w_gate, int T, int H, int E, float* logits, hipStream_t s) {
  constexpr int EB = kLogitWaves * EQ;
  const bool vec_x = H % (16 / sizeof(TIn)) == 0 && ((uintptr_t)x & 15) == 0;
  const bool vec_w = E % (16 / sizeof(TIn)) == 0 && ((uintptr_t)w_gate & 15) == 0;
  dim3 grid((T + kLogitTok - 1) / kLogitTok, (E + EB - 1) / EB);
  hipLaunchKernelGGL((router_logits_kernel<TIn, EQ>), grid, dim3(kLogitWaves * kWave), 0, s, (const TIn*)x,
                     (const TIn*)w_gate, T, H, E, logits, (int)vec_x, (int)vec_w, logit_block(H));
}

// Eight chains per lane when that still gives a workgroup per CU, else four (twice the
// workgroups, twice the weight broadcasts per multiply-add).
template <typename TIn>
static void launch_logits_dt(const void* x, const void* w_gate, int T, int H, int E, float* logits, hipStream_t s) {
  const int64_t blocks8 = (int64_t)((T + kLogitTok - 1) / kLogitTok) * ((E + 8 * kLogitWaves - 1) / (8 * kLogitWaves));
  if (blocks8 >= 256)
    launch_logits_t<TIn, 8>(x, w_gate, T, H, E, logits, s);
  else
    launch_logits_t<TIn, 4>(x, w_gate, T, H, E, logits, s);
}

hipError_t launch_router_logits(const void* x, const void* w_gate, int dt, int T, int H, int E, float* logits,
                                hipStream_t s) {
  const bool mfma_ok = dt == kBF16 && H % kRtHc == 0 && E % 8 == 0 && ((uintptr_t)x & 15) == 0 &&
                       ((uintptr_t)w_gate & 15) == 0 && (int64_t)T * H * 2 < (1LL << 31) &&
                       (int64_t)H * E * 2 < (1LL << 31);
  if (mfma_ok) {
    const dim3 grid((T + kRtTok - 1) / kRtTok, (E + kRtExp - 1) / kRtExp);
    hipLaunchKernelGGL(router_logits_mfma_kernel<3>, grid, dim3(256), 0, s, (const uint16_t*)x, (const uint16_t*)w_gate,
                       T, H, E, logit_block(H), logits);
    return hipGetLastError();
  }
  if (dt == kF32)
    launch_logits_dt<float>(x, w_gate, T, H, E, logits, s);
  else
    launch_logits_dt<uint16_t>(x, w_gate, T, H, E, logits, s);
  return hipGetLastError();
}

hipError_t launch_router_topk(const float* logits, int T, int E, int k, int renorm, int32_t* idx, float* w,
                              hipStream_t s, int32_t* chunk_counts, bool* counted) {
  if (E <= 256) {
    const dim3 grid(permute_ncount(T));
#define MOE_TOPK_GROUP(L, V)                                                                                     \
  hipLaunchKernelGGL((router_topk_group_kernel<L, V>), grid, dim3(kTopkGroupWaves * kWave), 0, s, logits, T, E, k, \
                     renorm, idx, w, chunk_counts)
    if (E <= 16)
      MOE_TOPK_GROUP(16, 1);
    else if (E <= 32)
      MOE_TOPK_GROUP(16, 2);
    else if (E <= 64)
      MOE_TOPK_GROUP(16, 4);
    else if (E <= 128)
      MOE_TOPK_GROUP(16, 8);
    else
      MOE_TOPK_GROUP(16, 16);
#undef MOE_TOPK_GROUP
    if (counted) *counted = chunk_counts != nullptr;
    return hipGetLastError();
  }
  if (counted) *counted = false;
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
