// Stream-K split of the per-rank partial attention over persistent workers,
// shared by the GQA and MLA MFMA kernels.
//
// A unit is (rank, request, KV head); its local tokens are cut into tiles of
// `tok` tokens and the tiles of all units, in unit order, are dealt out in
// equal contiguous ranges (ceil(total / workers) tiles) to the workers. A
// worker that covers a whole unit writes the unit's final partial (O, LSE)
// for the rank; a unit cut between workers leaves one unnormalised piece per
// worker in the workspace ("tail" piece of the worker where the unit starts,
// "head" piece of every later worker) and the combine kernel merges them by
// log-sum-exp. The planner builds the tile prefix over units on the device,
// so grids depend only on the device, never on the lengths.
#pragma once

#include "common.h"

namespace dcp {

constexpr int kPlanThreads = 1024;
constexpr int kCombineThreads = 256;
// Per partial head row: O[Dv] (unnormalised, value scale applied), then the
// running max m (log2 units), the sum of the bf16-rounded weights (the
// normaliser of O) and the sum of the fp32 weights (the LSE).
constexpr int kPartExtra = 3;

struct SplitWs {
  int64_t* prefix;  // [U + 1] tile prefix over units; prefix[U] = total tiles
  int32_t* wunit;   // [max_workers] unit holding each worker's first tile
  int32_t* todo;    // [1 + U + max_workers]: count, then the units that are empty or cut
  float* part;      // [max_workers][2][group][Dv + kPartExtra]
};

__host__ __device__ inline SplitWs split_ws(void* base, int64_t units, int max_workers) {
  SplitWs w;
  char* p = static_cast<char*>(base);
  w.prefix = reinterpret_cast<int64_t*>(p);
  p += align_up(static_cast<size_t>(units + 1) * sizeof(int64_t), 256);
  w.wunit = reinterpret_cast<int32_t*>(p);
  p += align_up(static_cast<size_t>(max_workers) * sizeof(int32_t), 256);
  w.todo = reinterpret_cast<int32_t*>(p);
  p += align_up(static_cast<size_t>(1 + units + max_workers) * sizeof(int32_t), 256);
  w.part = reinterpret_cast<float*>(p);
  return w;
}

static inline size_t split_ws_bytes(int64_t units, int max_workers, int group, int dv) {
  size_t b = align_up(static_cast<size_t>(units + 1) * sizeof(int64_t), 256);
  b += align_up(static_cast<size_t>(max_workers) * sizeof(int32_t), 256);
  b += align_up(static_cast<size_t>(1 + units + max_workers) * sizeof(int32_t), 256);
  b += static_cast<size_t>(max_workers) * 2 * group * (dv + kPartExtra) * sizeof(float);
  return b;
}

__device__ __forceinline__ int64_t split_units(const AttnParams& p) {
  return static_cast<int64_t>(p.rank_count) * p.batch * p.kv.num_kv_heads;
}

// Tiles of unit u = (r * batch + b) * Hkv + h (tok = 1 << tok_log2 tokens each).
__device__ __forceinline__ int64_t unit_tiles(const AttnParams& p, int64_t u, int tok_log2) {
  const int64_t rb = u / p.kv.num_kv_heads;
  const int b = static_cast<int>(rb % p.batch), r = static_cast<int>(rb / p.batch);
  const int64_t n = max(p.local_lens[static_cast<int64_t>(b) * p.dcp_size + p.rank_begin + r], 0);
  return (n + (int64_t(1) << tok_log2) - 1) >> tok_log2;
}

// ceil(a / b) for 0 <= a < 2^53, b >= 1, through fp64 (exact in that range).
__device__ __forceinline__ int64_t ceil_div_fp64(int64_t a, int64_t b) {
  int64_t q = static_cast<int64_t>(static_cast<double>(a) / static_cast<double>(b));
  while (q * b < a) ++q;            // guard against one-off rounding
  while (q > 0 && (q - 1) * b >= a) --q;
  return q;
}

// One block: tile prefix over units, the first unit of every worker and the
// list of units the combine has to touch (empty ones and ones cut between
// workers).
static __global__ void __launch_bounds__(kPlanThreads) split_plan_kernel(AttnParams p, int tok_log2, int workers,
                                                                         int max_workers) {
  __shared__ int64_t wsum[kPlanThreads / 64];
  __shared__ int64_t total_s;
  __shared__ int todo_n;
  const int64_t U = split_units(p);
  SplitWs ws = split_ws(p.workspace, U, max_workers);
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int64_t chunk = (U + kPlanThreads - 1) / kPlanThreads;
  const int64_t u0 = min(U, tid * chunk), u1 = min(U, u0 + chunk);
  int64_t s = 0;
  for (int64_t u = u0; u < u1; ++u) s += unit_tiles(p, u, tok_log2);
  // block exclusive scan: within each wavefront, then over the 16 wavefront sums
  int64_t incl = s;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int64_t v = __shfl_up(incl, off, 64);
    if (lane >= off) incl += v;
  }
  if (lane == 63) wsum[wid] = incl;
  if (tid == 0) todo_n = 0;
  __syncthreads();
  int64_t before = 0;
  for (int w = 0; w < wid; ++w) before += wsum[w];
  if (tid == kPlanThreads - 1) total_s = before + incl;
  __syncthreads();
  const int64_t T = total_s;
  const int64_t tpw = T > 0 ? (T + workers - 1) / workers : 1;
  int64_t run = before + incl - s;  // exclusive prefix of this thread's first unit
  for (int64_t u = u0; u < u1; ++u) {
    ws.prefix[u] = run;
    const int64_t nxt = run + unit_tiles(p, u, tok_log2);
    if (nxt == run) {
      ws.todo[1 + atomicAdd(&todo_n, 1)] = static_cast<int32_t>(u);       // empty
    } else {
      const int64_t wa = run / tpw, wb = (nxt - 1) / tpw;
      if (wa != wb) ws.todo[1 + atomicAdd(&todo_n, 1)] = static_cast<int32_t>(u);  // cut
      // workers whose first tile lies in [run, nxt)
      const int64_t wlo = ceil_div_fp64(run, tpw), whi = min<int64_t>(ceil_div_fp64(nxt, tpw), workers);
      for (int64_t w = wlo; w < whi; ++w) ws.wunit[w] = static_cast<int32_t>(u);
    }
    run = nxt;
  }
  if (tid == kPlanThreads - 1) ws.prefix[U] = T;
  __syncthreads();
  if (tid == 0) ws.todo[0] = todo_n;
}

// Fixed grid; one wavefront per (listed unit, query head of its group) item:
// merge the pieces of a unit cut between workers, or write O = 0 / LSE = -inf
// for an empty unit.
template <int kDv>
__global__ void __launch_bounds__(kCombineThreads) split_combine_kernel(AttnParams p, int workers, int max_workers) {
  const int G = p.group;
  const int64_t U = split_units(p);
  SplitWs ws = split_ws(p.workspace, U, max_workers);
  const int64_t T = ws.prefix[U];
  const int64_t tpw = T > 0 ? (T + workers - 1) / workers : 1;
  const int64_t items = static_cast<int64_t>(ws.todo[0]) * G;
  const int lane = threadIdx.x & 63;
  const int64_t wave0 = (static_cast<int64_t>(blockIdx.x) * kCombineThreads + threadIdx.x) >> 6;
  const int64_t nwaves = (static_cast<int64_t>(gridDim.x) * kCombineThreads) >> 6;
  constexpr int kRow = kDv + kPartExtra;
  constexpr int kPer = (kDv + 63) / 64;
  for (int64_t it = wave0; it < items; it += nwaves) {
    const int64_t u = ws.todo[1 + it / G];
    const int g = static_cast<int>(it % G);
    const int h = static_cast<int>(u % p.kv.num_kv_heads);
    const int64_t rb = u / p.kv.num_kv_heads;
    const int64_t row = rb * p.num_q_heads + static_cast<int64_t>(h) * G + g;
    const int64_t ubeg = ws.prefix[u], uend = ws.prefix[u + 1];
    float* dst = p.out_o + row * kDv;
    if (ubeg == uend) {
#pragma unroll
      for (int i = 0; i < kPer; ++i)
        if (lane + 64 * i < kDv) dst[lane + 64 * i] = 0.f;
      if (lane == 0) p.out_lse[row] = -INFINITY;
      continue;
    }
    const int64_t wa = ubeg / tpw, wb = (uend - 1) / tpw;
    float mx = -INFINITY;
    for (int64_t w = wa; w <= wb; ++w)
      mx = fmaxf(mx, ws.part[((w * 2 + (w == wa ? 1 : 0)) * G + g) * kRow + kDv]);
    float acc[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) acc[i] = 0.f;
    float lsum = 0.f, esum = 0.f;
    for (int64_t w = wa; w <= wb; ++w) {
      const float* hrow = ws.part + ((w * 2 + (w == wa ? 1 : 0)) * G + g) * kRow;
      const float sc = exp2f(hrow[kDv] - mx);
#pragma unroll
      for (int i = 0; i < kPer; ++i)
        if (lane + 64 * i < kDv) acc[i] += sc * hrow[lane + 64 * i];
      lsum += sc * hrow[kDv + 1];
      esum += sc * hrow[kDv + 2];
    }
    const float inv = 1.f / lsum;
#pragma unroll
    for (int i = 0; i < kPer; ++i)
      if (lane + 64 * i < kDv) dst[lane + 64 * i] = acc[i] * inv;
    if (lane == 0) p.out_lse[row] = (mx + __log2f(esum)) * DCP_LN2;
  }
}

static inline int log2_exact(int x) {
  int l = 0;
  while ((1 << l) < x) ++l;
  return l;
}

static inline void launch_split_plan(const AttnParams& p, int tok, int workers, int max_workers) {
  hipLaunchKernelGGL(split_plan_kernel, dim3(1), dim3(kPlanThreads), 0, p.stream, p, log2_exact(tok), workers,
                     max_workers);
}

template <int kDv>
static inline void launch_split_combine(const AttnParams& p, int workers, int max_workers) {
  hipLaunchKernelGGL(split_combine_kernel<kDv>, dim3(4 * device_cu_count()), dim3(kCombineThreads), 0, p.stream, p,
                     workers, max_workers);
}

}  // namespace dcp
