// route.hip -- top-k MoE routing into the contiguous per-expert layout on the
// device (gfx950).
//
// The miniTE page (section Transformer Engine路径优化) names contiguous
// layouts and device-side metadata among the fixes that cut data preparation
// and dispatch around the grouped GEMMs: the layout the grouped GEMM consumes
// (offsets, row_index) is built here from the router logits without a host
// round trip, and each token is quantized once and gathered by row_index.
//
// Launches:
//  1. route_topk_kernel: L lanes per token (16 for up to 128 experts).  Each
//     round takes the group max of the order-preserving bits of the logits
//     still in play (-0 folded into +0), then the lowest expert id holding
//     it, so the experts come out largest logit first, lower id first on
//     ties.
//  2. route_expert_kernel<COUNT>, then <PLACE>: one workgroup per expert
//     walks the (token, choice) pairs in token order, 16 waves each owning
//     a contiguous run; a ballot of "chose this expert" per 64 pairs gives
//     counts, then positions (running count of the wave plus the matches of
//     earlier lanes).  The counts go to offsets[e + 1]; the placing pass
//     starts expert e at the sum of the lower experts' counts.  A stable
//     counting sort by (expert, token): deterministic, no atomics.
//  3. route_scan_kernel turns the counts into offsets.
#include "nvfp4_internal.h"

namespace nvfp4 {

constexpr int ROUTE_MAX_EXPERTS = 1024;
constexpr int ROUTE_MAX_TOPK = 64;

__device__ __forceinline__ uint32_t ordered_bits(float v) {
  uint32_t u = __float_as_uint(v);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// L lanes own one token (V logits each, expert j + L v on lane j of the
// group); a wave holds 64 / L tokens.  Per round: the group max of the
// order-preserving logit bits, then the group min of the expert ids holding
// that value (ties go to the lower id), which the owner marks as taken.
template <int L, int V>
__global__ __launch_bounds__(256) void route_topk_kernel(const float* __restrict__ logits,
                                                         int64_t T, int E, int topk,
                                                         int32_t* __restrict__ experts) {
  constexpr int TPW = 64 / L;
  const int lane = threadIdx.x & 63;
  const int j = lane % L;
  const int sub = lane / L;
  for (int64_t t0 = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * TPW; t0 < T;
       t0 += (int64_t)gridDim.x * 4 * TPW) {  // wave-uniform
    const int64_t t = t0 + sub;
    const bool ok = t < T;
    const float* lt = logits + (ok ? t : 0) * E;
    uint32_t val[V];
    uint32_t live = 0;  // bit v: expert j + L v exists and is not chosen yet
#pragma unroll
    for (int v = 0; v < V; ++v) {
      const int e = j + L * v;
      const bool in = ok && e < E;
      val[v] = in ? ordered_bits(lt[e]) : 0u;
      live |= in ? (1u << v) : 0u;
    }
    for (int r = 0; r < topk; ++r) {
      uint32_t m = 0;
#pragma unroll
      for (int v = 0; v < V; ++v)
        if ((live >> v) & 1u) m = max(m, val[v]);
      m = group_max_u32<L>(m);
      uint32_t nid = 0;  // ~(lowest expert id of this lane holding m)
#pragma unroll
      for (int v = V - 1; v >= 0; --v)
        if (((live >> v) & 1u) && val[v] == m) nid = ~(uint32_t)(j + L * v);
      const uint32_t id = ~group_max_u32<L>(nid);
      if (ok && j == 0) experts[t * topk + r] = (int32_t)id;
#pragma unroll
      for (int v = 0; v < V; ++v)
        if ((uint32_t)(j + L * v) == id) live &= ~(1u << v);
    }
  }
}

__global__ __launch_bounds__(1024) void fill_i32_kernel(int32_t* __restrict__ p, int64_t n,
                                                        int32_t v) {
  for (int64_t i = threadIdx.x; i < n; i += 1024) p[i] = v;
}

constexpr int ROUTE_WAVES = 16;
constexpr int ROUTE_BATCH = 32;  // 64-pair steps per batch of loads

// One workgroup per expert e walks all (token, choice) pairs in pair order
// (token order: a token picks an expert at most once); wave w owns the
// contiguous run [w seg, (w + 1) seg) of the pairs.
//  COUNT: offsets[e + 1] = number of pairs choosing e.
//  PLACE: reads those counts, so base = pairs of experts below e; counts
//         its waves' matches, then walks again writing each match to
//         base + (matches of earlier waves) + (earlier matches of its wave).
template <bool PLACE>
__global__ __launch_bounds__(1024) void route_expert_kernel(const int32_t* __restrict__ experts,
                                                            int64_t ne, int E, int topk,
                                                            int32_t* __restrict__ offsets,
                                                            int32_t* __restrict__ row_index,
                                                            int32_t* __restrict__ slot_of) {
  __shared__ int32_t wcnt[ROUTE_WAVES];
  __shared__ int32_t wbase[ROUTE_WAVES];
  const int e = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t seg = ((ne + ROUTE_WAVES - 1) / ROUTE_WAVES + 63) / 64 * 64;
  const int64_t w0 = wave * seg;
  const int64_t w1 = w0 + seg < ne ? w0 + seg : ne;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  // a run of at most one batch stays in registers for the placing walk
  const bool one_batch = w1 - w0 <= 64 * ROUTE_BATCH;
  int key[ROUTE_BATCH];
  int run = 0;
  for (int64_t b0 = w0; b0 < w1; b0 += 64 * ROUTE_BATCH) {
#pragma unroll
    for (int s = 0; s < ROUTE_BATCH; ++s) {
      const int64_t i = b0 + 64 * s + lane;
      key[s] = i < w1 ? experts[i] : -1;
    }
#pragma unroll
    for (int s = 0; s < ROUTE_BATCH; ++s) run += __popcll(__ballot(key[s] == e));
  }
  if (lane == 0) wcnt[wave] = run;
  __syncthreads();
  if (!PLACE) {
    if (tid == 0) {
      int tot = 0;
      for (int w = 0; w < ROUTE_WAVES; ++w) tot += wcnt[w];
      offsets[e + 1] = tot;
    }
    return;
  }
  if (wave == 0) {
    // base = sum of the counts of experts below e
    int part = 0;
    for (int x = lane; x < e; x += 64) part += offsets[x + 1];
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) part += __shfl_xor(part, d, 64);
    if (lane == 0) {
      int acc = part;
      for (int w = 0; w < ROUTE_WAVES; ++w) {
        wbase[w] = acc;
        acc += wcnt[w];
      }
    }
  }
  __syncthreads();
  int pos0 = wbase[wave];
  for (int64_t b0 = w0; b0 < w1; b0 += 64 * ROUTE_BATCH) {
    if (!one_batch) {
#pragma unroll
      for (int s = 0; s < ROUTE_BATCH; ++s) {
        const int64_t i = b0 + 64 * s + lane;
        key[s] = i < w1 ? experts[i] : -1;
      }
    }
#pragma unroll
    for (int s = 0; s < ROUTE_BATCH; ++s) {
      const uint64_t m = __ballot(key[s] == e);
      if (key[s] == e) {
        const int64_t i = b0 + 64 * s + lane;
        const int pos = pos0 + __popcll(m & below);
        row_index[pos] = (int32_t)i / topk;  // pairs < 2^31
        slot_of[i] = pos;
      }
      pos0 += __popcll(m);
    }
  }
}

// offsets[1..E] hold per-expert counts; turn them into the running offsets
// (offsets[0] = 0) with a block scan (E <= 1024).
__global__ __launch_bounds__(1024) void route_scan_kernel(int E, int32_t* __restrict__ offsets) {
  __shared__ int32_t wsum[16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = tid < E ? offsets[tid + 1] : 0;
  int incl = c;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int o = __shfl_up(incl, d, 64);
    if (lane >= d) incl += o;
  }
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  int before = 0;
  for (int w = 0; w < wave; ++w) before += wsum[w];
  if (tid < E) offsets[tid + 1] = before + incl;
  if (tid == 0) offsets[0] = 0;
}

}  // namespace nvfp4

using nvfp4host::aligned;

extern "C" int nvfp4_moe_route(const float* logits, int64_t tokens, int64_t num_experts,
                               int64_t topk, int32_t* experts, int32_t* offsets,
                               int32_t* row_index, int32_t* slot_of, void* stream) {
  if (tokens < 0 || num_experts < 1 || topk < 1) return NVFP4_ERROR_INVALID_VALUE;
  if (topk > num_experts) return NVFP4_ERROR_INVALID_VALUE;
  if (num_experts > nvfp4::ROUTE_MAX_EXPERTS || topk > nvfp4::ROUTE_MAX_TOPK)
    return NVFP4_ERROR_UNSUPPORTED_SHAPE;
  if (tokens > 0 && tokens * topk >= ((int64_t)1 << 31)) return NVFP4_ERROR_UNSUPPORTED_SHAPE;
  if (!offsets) return NVFP4_ERROR_INVALID_VALUE;
  if (tokens > 0 && (!logits || !experts || !row_index || !slot_of))
    return NVFP4_ERROR_INVALID_VALUE;
  if (!aligned(logits, 4) || !aligned(experts, 4) || !aligned(offsets, 4) ||
      !aligned(row_index, 4) || !aligned(slot_of, 4))
    return NVFP4_ERROR_MISALIGNED;
  int st = nvfp4host::check_arch();
  if (st) return st;
#if NVFP4_CHECKED
  {
    nvfp4check::Checks chk((hipStream_t)stream);
    chk.f32_finite(logits, tokens * num_experts);
    if ((st = chk.result())) return st;
  }
#endif
  hipStream_t str = (hipStream_t)stream;
  const int E = (int)num_experts, K = (int)topk;
  if (tokens > 0) {
    const int tpb = E <= 128 ? 16 : (E <= 256 ? 8 : 4);  // tokens per 256-lane block
    const int64_t need = (tokens + tpb - 1) / tpb;
    const int64_t cap = (int64_t)nvfp4host::num_cus() * 8;
    dim3 grid((unsigned)(need < cap ? need : cap));
    if (E <= 16)
      hipLaunchKernelGGL((nvfp4::route_topk_kernel<16, 1>), grid, dim3(256), 0, str, logits,
                         tokens, E, K, experts);
    else if (E <= 32)
      hipLaunchKernelGGL((nvfp4::route_topk_kernel<16, 2>), grid, dim3(256), 0, str, logits,
                         tokens, E, K, experts);
    else if (E <= 64)
      hipLaunchKernelGGL((nvfp4::route_topk_kernel<16, 4>), grid, dim3(256), 0, str, logits,
                         tokens, E, K, experts);
    else if (E <= 128)
      hipLaunchKernelGGL((nvfp4::route_topk_kernel<16, 8>), grid, dim3(256), 0, str, logits,
                         tokens, E, K, experts);
    else if (E <= 256)
      hipLaunchKernelGGL((nvfp4::route_topk_kernel<32, 8>), grid, dim3(256), 0, str, logits,
                         tokens, E, K, experts);
    else if (E <= 512)
      hipLaunchKernelGGL((nvfp4::route_topk_kernel<64, 8>), grid, dim3(256), 0, str, logits,
                         tokens, E, K, experts);
    else
      hipLaunchKernelGGL((nvfp4::route_topk_kernel<64, 16>), grid, dim3(256), 0, str, logits,
                         tokens, E, K, experts);
  }
  const int64_t ne = tokens * topk;
  if (ne > 0) {
    hipLaunchKernelGGL(nvfp4::route_expert_kernel<false>, dim3(E), dim3(1024), 0, str, experts, ne,
                       E, K, offsets, row_index, slot_of);
    hipLaunchKernelGGL(nvfp4::route_expert_kernel<true>, dim3(E), dim3(1024), 0, str, experts, ne,
                       E, K, offsets, row_index, slot_of);
  } else {
    hipLaunchKernelGGL(nvfp4::fill_i32_kernel, dim3(1), dim3(1024), 0, str, offsets + 1, (int64_t)E,
                       0);
  }
  hipLaunchKernelGGL(nvfp4::route_scan_kernel, dim3(1), dim3(1024), 0, str, E, offsets);
  return nvfp4host::launch_status();
}
