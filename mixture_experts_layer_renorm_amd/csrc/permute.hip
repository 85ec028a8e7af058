// Token permute: group the T*k (token, slot) rows by expert.
//
// Row order follows the VeOmni walk-through of the "DeepSeek MoE: EP and FSDP" guide (gsyq.cn):
// the permuted buffer holds expert 0's rows first, then expert 1's, and inside an expert the
// tokens stay in ascending order; per-expert counts come from summing the routing mask.
//
// Three kernels, no host synchronisation and no atomics that decide an order:
//  1. count : per kCountTok tokens, an LDS histogram of their expert choices.
//  2. plan  : per chunk of kPermuteChunk tokens, global bases = exclusive scan over experts of the
//             totals + the counts of earlier tokens; in-chunk ranks from per-expert token bitmaps (popcount of the
//             tokens before this one). Writes counts, offsets, row_of_slot, slot_of_row. A chunk
//             in which a token names one expert in two slots ranks by counting earlier slots
//             instead, so every slot gets its own row in (expert, token, slot) order.
//     (The router's top-k kernel can produce the counts of step 1 itself: launch_permute_counted.)
//  3. scatter: one wave per token copies x[t] (read once) to its k rows of x_perm.
// Slots whose expert index is outside [0, E) get no row (row_of_slot = -1).
#include <mutex>

#include "common.hpp"
#include "internal.hpp"

namespace moe {

constexpr int kPlanThreads = 256;
constexpr int kMaxE = 1024;
constexpr int kMaskWords = kPermuteChunk / 32;
constexpr int kMaxChunkSlots = kPermuteChunk * 32;  // k <= 32

__global__ __launch_bounds__(kPlanThreads) void permute_count_kernel(const int32_t* __restrict__ idx, int T, int k,
                                                                     int E, int32_t* __restrict__ chunk_counts) {
  __shared__ int cnt[kMaxE];
  const int c = blockIdx.x;
  for (int e = threadIdx.x; e < E; e += kPlanThreads) cnt[e] = 0;
  __syncthreads();
  const int64_t s0 = (int64_t)c * kCountTok * k;
  const int64_t s1 = (int64_t)min(T, (c + 1) * kCountTok) * k;
  for (int64_t s = s0 + threadIdx.x; s < s1; s += kPlanThreads) {
    const int e = idx[s];
    if (e >= 0 && e < E) atomicAdd(&cnt[e], 1);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kPlanThreads) chunk_counts[(int64_t)c * E + e] = cnt[e];
}

__global__ __launch_bounds__(kPlanThreads) void permute_plan_kernel(
    const int32_t* __restrict__ idx, int T, int k, int E, const int32_t* __restrict__ chunk_counts, int ncount,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int32_t* __restrict__ row_of_slot,
    int32_t* __restrict__ slot_of_row) {
  __shared__ int scan[kMaxE + 1];
  __shared__ int base[kMaxE];
  __shared__ uint32_t mask[kMaxE * kMaskWords];
  __shared__ int s_idx[kMaxChunkSlots];      // the chunk's expert choices, slot order
  __shared__ int p_tot[kPlanThreads], p_bef[kPlanThreads];
  __shared__ int4 p_tot4[kPlanThreads], p_bef4[kPlanThreads];
  __shared__ int wave_tot[kPlanThreads / kWave];
  __shared__ int s_dup;
  const int c = blockIdx.x;
  const int tid = threadIdx.x;
  // per expert: its total over all count rows and over the rows before this chunk's first. With
  // E < 256 the rows of an expert are split over G = 256 / E threads, each issuing its loads as one
  // batch (the loads are independent; one chain of them per expert would be a chain of L2 round
  // trips).
  const int first = c * kCountPerChunk;
  auto sum_chunks = [&](int e, int g, int G, int& tot, int& before) {
    tot = 0;
    before = 0;
    int cc = g;
    for (; cc + 15 * G < ncount; cc += 16 * G) {
      int v[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) v[u] = chunk_counts[(int64_t)(cc + u * G) * E + e];
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        tot += v[u];
        if (cc + u * G < first) before += v[u];
      }
    }
    for (; cc < ncount; cc += G) {
      const int v = chunk_counts[(int64_t)cc * E + e];
      tot += v;
      if (cc < first) before += v;
    }
  };
  // the chunk's expert choices (their loads overlap the count loads below)
  for (int i = tid; i < E * kMaskWords; i += kPlanThreads) mask[i] = 0u;
  const int t0 = c * kPermuteChunk;
  const int64_t s0 = (int64_t)t0 * k;
  const int ns = (int)((int64_t)min(T, t0 + kPermuteChunk) * k - s0);
  for (int i = tid; i < ns; i += kPlanThreads) s_idx[i] = idx[s0 + i];
  if (tid == 0) s_dup = 0;
  const bool vec = (E % 4 == 0) && ((uintptr_t)chunk_counts % 16 == 0);
  if (vec) {
    // 16-byte loads of 4 experts' counts: thread (phase ph, expert quad ev) sums the rows
    // ph, ph + P, ... with 16 loads in flight at a time (the rows were written by other XCDs, so
    // each batch is a round trip to the last-level cache), then the P phases are added in LDS
    const int EV = E / 4, P = kPlanThreads / EV;
    int4 tot = make_int4(0, 0, 0, 0), bef = make_int4(0, 0, 0, 0);
    if (tid < P * EV) {
      const int ev = tid % EV, ph = tid / EV;
      const int4* cc4 = reinterpret_cast<const int4*>(chunk_counts) + ev;
      int r = ph;
      for (; r + 15 * P < ncount; r += 16 * P) {
        int4 v[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) v[u] = cc4[(int64_t)(r + u * P) * EV];
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          tot.x += v[u].x, tot.y += v[u].y, tot.z += v[u].z, tot.w += v[u].w;
          if (r + u * P < first) bef.x += v[u].x, bef.y += v[u].y, bef.z += v[u].z, bef.w += v[u].w;
        }
      }
      for (; r < ncount; r += P) {
        const int4 v = cc4[(int64_t)r * EV];
        tot.x += v.x, tot.y += v.y, tot.z += v.z, tot.w += v.w;
        if (r < first) bef.x += v.x, bef.y += v.y, bef.z += v.z, bef.w += v.w;
      }
    }
    p_tot4[tid] = tot;
    p_bef4[tid] = bef;
    __syncthreads();
    for (int e = tid; e < E; e += kPlanThreads) {
      int a = 0, b = 0;
      for (int ph = 0; ph < P; ++ph) {
        a += reinterpret_cast<const int*>(&p_tot4[ph * EV + e / 4])[e % 4];
        b += reinterpret_cast<const int*>(&p_bef4[ph * EV + e / 4])[e % 4];
      }
      scan[e] = a;
      base[e] = b;
    }
  } else if (E >= kPlanThreads) {
    for (int e = tid; e < E; e += kPlanThreads) sum_chunks(e, 0, 1, scan[e], base[e]);
  } else {
    const int G = kPlanThreads / E;
    int tot = 0, before = 0;
    if (tid < G * E) sum_chunks(tid % E, tid / E, G, tot, before);
    p_tot[tid] = tot;
    p_bef[tid] = before;
    __syncthreads();
    if (tid < E) {
      int a = 0, b = 0;
      for (int g = 0; g < G; ++g) {
        a += p_tot[g * E + tid];
        b += p_bef[g * E + tid];
      }
      scan[tid] = a;
      base[tid] = b;
    }
  }
  __syncthreads();
  if (c == 0)
    for (int e = tid; e < E; e += kPlanThreads) counts[e] = scan[e];
  block_exclusive_scan<kPlanThreads>(scan, E, wave_tot);
  for (int e = tid; e < E; e += kPlanThreads) {
    base[e] += scan[e];
    if (c == 0) offsets[e] = scan[e];
  }
  if (c == 0 && tid == 0) offsets[E] = scan[E];

  // per-expert bitmaps of the chunk's tokens; a bit found already set means that a token names one
  // expert in two of its slots (the router never does that; routing supplied by a caller may)
  for (int i = tid; i < ns; i += kPlanThreads) {
    const int e = s_idx[i];
    if (e >= 0 && e < E) {
      const int tl = i / k;
      const uint32_t bit = 1u << (tl & 31);
      if (atomicOr(&mask[e * kMaskWords + (tl >> 5)], bit) & bit) s_dup = 1;
    }
  }
  __syncthreads();
  const bool dup = s_dup != 0;
  for (int i = tid; i < ns; i += kPlanThreads) {
    const int e = s_idx[i];
    const int64_t s = s0 + i;
    if (e >= 0 && e < E) {
      int rank = 0;
      if (!dup) {  // rank = earlier tokens of the chunk that chose e
        const int tl = i / k;
        const uint32_t* m = mask + e * kMaskWords;
        for (int w = 0; w < (tl >> 5); ++w) rank += __popc(m[w]);
        rank += __popc(m[tl >> 5] & ((1u << (tl & 31)) - 1u));
      } else {     // rank = earlier slots of the chunk that chose e: (token, slot) order
        for (int i2 = 0; i2 < i; ++i2) rank += s_idx[i2] == e;
      }
      const int row = base[e] + rank;
      row_of_slot[s] = row;
      slot_of_row[row] = (int32_t)s;
    } else {
      row_of_slot[s] = -1;
    }
  }
}

// One wave per token; 16-byte vectors when rows allow it, 2-byte units otherwise.
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;
constexpr int kScatterWaves = 4;

__global__ __launch_bounds__(kScatterWaves * kWave) void permute_scatter_kernel(
    const uint8_t* __restrict__ x, int T, int64_t row_bytes, int k, const int32_t* __restrict__ row_of_slot,
    uint8_t* __restrict__ x_perm, int vec16) {
  const int lane = lane_id();
  const int t = blockIdx.x * kScatterWaves + (int)(threadIdx.x / kWave);
  if (t >= T) return;
  const int my_row = lane < k ? row_of_slot[(int64_t)t * k + lane] : -1;
  const uint8_t* src = x + (int64_t)t * row_bytes;
  if (vec16) {
    const int64_t nvec = row_bytes >> 4;
    const uint4* s4 = reinterpret_cast<const uint4*>(src);
    for (int64_t v0 = 0; v0 < nvec; v0 += 4 * kWave) {
      uint4 buf[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int64_t v = v0 + u * kWave + lane;
        if (v < nvec) buf[u] = s4[v];
      }
      for (int j = 0; j < k; ++j) {
        const int r = __shfl(my_row, j, kWave);
        if (r < 0) continue;
        u32x4* d4 = reinterpret_cast<u32x4*>(x_perm + (int64_t)r * row_bytes);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int64_t v = v0 + u * kWave + lane;
          // non-temporal: the copies are written once and read back only by a later kernel, so
          // they need not displace the source rows from L2 (4.5 -> 5.6-6.2 TB/s measured)
          if (v < nvec) __builtin_nontemporal_store(u32x4{buf[u].x, buf[u].y, buf[u].z, buf[u].w}, &d4[v]);
        }
      }
    }
  } else {
    const int64_t n16 = row_bytes >> 1;
    const uint16_t* s2 = reinterpret_cast<const uint16_t*>(src);
    for (int64_t base = 0; base < n16; base += kWave) {   // uniform trip count: the shuffles read active lanes
      const int64_t i = base + lane;
      const bool act = i < n16;
      const uint16_t v = act ? s2[i] : 0;
      for (int j = 0; j < k; ++j) {
        const int r = __shfl(my_row, j, kWave);
        if (r >= 0 && act) reinterpret_cast<uint16_t*>(x_perm + (int64_t)r * row_bytes)[i] = v;
      }
    }
  }
}

__global__ void fill_i32_kernel(int32_t* __restrict__ p, int n, int32_t v) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

hipError_t launch_fill_i32(int32_t* p, int n, int32_t v, hipStream_t s) {
  if (n > 0) hipLaunchKernelGGL(fill_i32_kernel, dim3((n + 255) / 256), dim3(256), 0, s, p, n, v);
  return hipGetLastError();
}

// plan + row copy from chunk counts already in chunk_counts
static hipError_t plan_and_scatter(const void* x, int dt, int T, int H, const int32_t* topk_idx, int k, int E,
                                   void* x_perm, int32_t* counts, int32_t* offsets, int32_t* row_of_slot,
                                   int32_t* slot_of_row, const int32_t* chunk_counts, hipStream_t s) {
  const int nchunks = permute_nchunks(T);
  const int64_t row_bytes = (int64_t)H * (int64_t)dtype_bytes(dt);
  const int vec16 = (row_bytes % 16 == 0) && (((uintptr_t)x | (uintptr_t)x_perm) % 16 == 0);
  hipLaunchKernelGGL(permute_plan_kernel, dim3(nchunks), dim3(kPlanThreads), 0, s, topk_idx, T, k, E, chunk_counts,
                     permute_ncount(T), counts, offsets, row_of_slot, slot_of_row);
  if (x_perm)  // else the plan only: a gathering GEMM reads the rows from x itself
    hipLaunchKernelGGL(permute_scatter_kernel, dim3((T + kScatterWaves - 1) / kScatterWaves),
                       dim3(kScatterWaves * kWave), 0, s, (const uint8_t*)x, T, row_bytes, k, row_of_slot,
                       (uint8_t*)x_perm, vec16);
  return hipGetLastError();
}

hipError_t launch_permute(const void* x, int dt, int T, int H, const int32_t* topk_idx, int k, int E, void* x_perm,
                          int32_t* counts, int32_t* offsets, int32_t* row_of_slot, int32_t* slot_of_row,
                          int32_t* chunk_counts, hipStream_t s) {
  hipLaunchKernelGGL(permute_count_kernel, dim3(permute_ncount(T)), dim3(kPlanThreads), 0, s, topk_idx, T, k, E,
                     chunk_counts);
  return plan_and_scatter(x, dt, T, H, topk_idx, k, E, x_perm, counts, offsets, row_of_slot, slot_of_row,
                          chunk_counts, s);
}

hipError_t launch_permute_counted(const void* x, int dt, int T, int H, const int32_t* topk_idx, int k, int E,
                                  void* x_perm, int32_t* counts, int32_t* offsets, int32_t* row_of_slot,
                                  int32_t* slot_of_row, const int32_t* chunk_counts, hipStream_t s) {
  return plan_and_scatter(x, dt, T, H, topk_idx, k, E, x_perm, counts, offsets, row_of_slot, slot_of_row,
                          chunk_counts, s);
}

// ---- the allocation-free permute's scratch ---------------------------------------------------
// The per-chunk expert counts of moe_permute_noalloc live in this file-scope device array instead
// of a caller workspace: each GPU holds its own copy for the life of the process, and every call on
// that GPU shares it (the count kernel rewrites every entry the plan reads, so nothing needs
// clearing; calls that overlap on one GPU race on it). Host code never passes the array's name to
// a kernel: that is a host-side stand-in, not the device address. The device address is looked up
// with hipGetSymbolAddress once per device, with that device current, and kept.
static __device__ __align__(256) int32_t scratch[kPermuteScratchInts];

hipError_t permute_noalloc_scratch(int32_t** out) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static int32_t* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = (int32_t*)p;
  }
  *out = addr[dev];
  return hipSuccess;
}

}  // namespace moe
