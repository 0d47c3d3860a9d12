// Stream-K split of the per-rank partial attention over persistent workers,
// shared by the GQA and MLA MFMA kernels.
//
// A unit is (rank, request, KV head, group of tpu query tokens); its local
// tokens (as many as its longest query sees) are cut into tiles of `tok`
// tokens and the tiles of all units, in unit order, are dealt out in
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
  float* part;      // [max_workers][2][rows][Dv + kPartExtra], rows = tpu * group
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

static inline size_t split_ws_bytes(int64_t units, int max_workers, int rows, int dv) {
  size_t b = align_up(static_cast<size_t>(units + 1) * sizeof(int64_t), 256);
  b += align_up(static_cast<size_t>(max_workers) * sizeof(int32_t), 256);
  b += align_up(static_cast<size_t>(1 + units + max_workers) * sizeof(int32_t), 256);
  b += static_cast<size_t>(max_workers) * 2 * rows * (dv + kPartExtra) * sizeof(float);
  return b;
}

static inline int64_t split_units_host(const AttnParams& p) {
  return static_cast<int64_t>(p.rank_count) * p.batch * p.kv.num_kv_heads * p.ntg;
}

__device__ __forceinline__ int64_t split_units(const AttnParams& p) {
  return static_cast<int64_t>(p.rank_count) * p.batch * p.kv.num_kv_heads * p.ntg;
}

// Unit u = ((r * batch + b) * Hkv + h) * ntg + tg covers rank r (counted from
// rank_begin), request b, KV head h and query tokens [i0, i1) of the request.
struct UnitRef {
  int64_t rb;  // r * batch + b
  int r, b, h, i0, i1;
};

__device__ __forceinline__ UnitRef unit_ref(const AttnParams& p, int64_t u) {
  UnitRef x;
  const int tg = static_cast<int>(u % p.ntg);
  const int64_t uh = u / p.ntg;
  x.h = static_cast<int>(uh % p.kv.num_kv_heads);
  x.rb = uh / p.kv.num_kv_heads;
  x.b = static_cast<int>(x.rb % p.batch);
  x.r = static_cast<int>(x.rb / p.batch);
  x.i0 = tg * p.tpu;
  x.i1 = min(p.q_len, x.i0 + p.tpu);
  return x;
}

// Local tokens query token i of request b sees on rank r (from rank_begin).
__device__ __forceinline__ int query_len(const AttnParams& p, int b, int i, int r) {
  return max(p.local_lens[(static_cast<int64_t>(b) * p.q_len + i) * p.dcp_size + p.rank_begin + r], 0);
}

// Local tokens of a unit: as many as its longest query sees.
__device__ __forceinline__ int unit_len(const AttnParams& p, const UnitRef& x) {
  int n = 0;
  for (int i = x.i0; i < x.i1; ++i) n = max(n, query_len(p, x.b, i, x.r));
  return n;
}

// Output row of (query token i, query head h * group + g) of unit x.
__device__ __forceinline__ int64_t out_row(const AttnParams& p, const UnitRef& x, int i, int g) {
  return (x.rb * p.q_len + i) * p.num_q_heads + static_cast<int64_t>(x.h) * p.group + g;
}

// Tiles of unit u (tok = 1 << tok_log2 tokens each).
__device__ __forceinline__ int64_t unit_tiles(const AttnParams& p, int64_t u, int tok_log2) {
  const int64_t n = unit_len(p, unit_ref(p, u));
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

// Fixed grid; one wavefront per (listed unit, row of the unit) item, a row
// being (query token, query head of the group): merge the pieces of a unit
// cut between workers, or write O = 0 / LSE = -inf for an empty unit and for
// a row that sees no token of the unit (a query earlier than every local
// token; its pieces carry m = -inf).
template <int kDv>
__global__ void __launch_bounds__(kCombineThreads) split_combine_kernel(AttnParams p, int workers, int max_workers) {
  const int G = p.group, rows = p.tpu * p.group;
  const int64_t U = split_units(p);
  SplitWs ws = split_ws(p.workspace, U, max_workers);
  const int64_t T = ws.prefix[U];
  const int64_t tpw = T > 0 ? (T + workers - 1) / workers : 1;
  const int64_t items = static_cast<int64_t>(ws.todo[0]) * rows;
  const int lane = threadIdx.x & 63;
  const int64_t wave0 = (static_cast<int64_t>(blockIdx.x) * kCombineThreads + threadIdx.x) >> 6;
  const int64_t nwaves = (static_cast<int64_t>(gridDim.x) * kCombineThreads) >> 6;
  constexpr int kRow = kDv + kPartExtra;
  constexpr int kPer = (kDv + 63) / 64;
  for (int64_t it = wave0; it < items; it += nwaves) {
    const int64_t u = ws.todo[1 + it / rows];
    const int c = static_cast<int>(it % rows);
    const UnitRef x = unit_ref(p, u);
    const int i = x.i0 + c / G;
    if (i >= x.i1) continue;  // a row past the request's last query token
    const int64_t row = out_row(p, x, i, c % G);
    const int64_t ubeg = ws.prefix[u], uend = ws.prefix[u + 1];
    float* dst = p.out_o + row * kDv;
    float mx = -INFINITY;
    int64_t wa = 0, wb = -1;
    if (ubeg != uend) {
      wa = ubeg / tpw;
      wb = (uend - 1) / tpw;
      for (int64_t w = wa; w <= wb; ++w)
        mx = fmaxf(mx, ws.part[((w * 2 + (w == wa ? 1 : 0)) * rows + c) * kRow + kDv]);
    }
    if (mx == -INFINITY) {
#pragma unroll
      for (int k = 0; k < kPer; ++k)
        if (lane + 64 * k < kDv) dst[lane + 64 * k] = 0.f;
      if (lane == 0) p.out_lse[row] = -INFINITY;
      continue;
    }
    float acc[kPer];
#pragma unroll
    for (int k = 0; k < kPer; ++k) acc[k] = 0.f;
    float lsum = 0.f, esum = 0.f;
    for (int64_t w = wa; w <= wb; ++w) {
      const float* hrow = ws.part + ((w * 2 + (w == wa ? 1 : 0)) * rows + c) * kRow;
      const float sc = exp2f(hrow[kDv] - mx);  // 0 for a piece with m = -inf
#pragma unroll
      for (int k = 0; k < kPer; ++k)
        if (lane + 64 * k < kDv) acc[k] += sc * hrow[lane + 64 * k];
      lsum += sc * hrow[kDv + 1];
      esum += sc * hrow[kDv + 2];
    }
    const float inv = 1.f / lsum;
#pragma unroll
    for (int k = 0; k < kPer; ++k)
      if (lane + 64 * k < kDv) dst[lane + 64 * k] = acc[k] * inv;
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
