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
// Per partial head row: O[Dv] (unnormalised, value scale applied), then the
// running max m (log2 units), the sum of the bf16-rounded weights (the
// normaliser of O) and the sum of the fp32 weights (the LSE).
constexpr int kPartExtra = 3;

struct SplitWs {
  int64_t* prefix;  // [U + 1] tile prefix over units; prefix[U] = total tiles
  int32_t* wunit;   // [max_workers] unit holding each worker's first tile
  float* part;      // [max_workers][2][group][Dv + kPartExtra]
};

__host__ __device__ inline SplitWs split_ws(void* base, int64_t units, int max_workers) {
  SplitWs w;
  char* p = static_cast<char*>(base);
  w.prefix = reinterpret_cast<int64_t*>(p);
  p += align_up(static_cast<size_t>(units + 1) * sizeof(int64_t), 256);
  w.wunit = reinterpret_cast<int32_t*>(p);
  p += align_up(static_cast<size_t>(max_workers) * sizeof(int32_t), 256);
  w.part = reinterpret_cast<float*>(p);
  return w;
}

static inline size_t split_ws_bytes(int64_t units, int max_workers, int group, int dv) {
  size_t b = align_up(static_cast<size_t>(units + 1) * sizeof(int64_t), 256);
  b += align_up(static_cast<size_t>(max_workers) * sizeof(int32_t), 256);
  b += static_cast<size_t>(max_workers) * 2 * group * (dv + kPartExtra) * sizeof(float);
  return b;
}

__device__ __forceinline__ int64_t split_units(const AttnParams& p) {
  return static_cast<int64_t>(p.rank_count) * p.batch * p.kv.num_kv_heads;
}

// Local length of unit u = (r * batch + b) * Hkv + h.
__device__ __forceinline__ int64_t unit_len(const AttnParams& p, int64_t u) {
  const int64_t rb = u / p.kv.num_kv_heads;
  const int b = static_cast<int>(rb % p.batch), r = static_cast<int>(rb / p.batch);
  return max(p.local_lens[static_cast<int64_t>(b) * p.dcp_size + p.rank_begin + r], 0);
}

// One block: tile prefix over units and the first unit of every worker.
static __global__ void __launch_bounds__(kPlanThreads) split_plan_kernel(AttnParams p, int tok, int workers,
                                                                  int max_workers) {
  __shared__ int64_t scan[kPlanThreads];
  __shared__ int64_t total_s;
  const int64_t U = split_units(p);
  SplitWs ws = split_ws(p.workspace, U, max_workers);
  const int tid = threadIdx.x;
  const int64_t chunk = (U + kPlanThreads - 1) / kPlanThreads;
  const int64_t u0 = min(U, tid * chunk), u1 = min(U, u0 + chunk);
  int64_t s = 0;
  for (int64_t u = u0; u < u1; ++u) s += (unit_len(p, u) + tok - 1) / tok;
  scan[tid] = s;
  __syncthreads();
  for (int off = 1; off < kPlanThreads; off <<= 1) {  // inclusive scan
    const int64_t v = tid >= off ? scan[tid - off] : 0;
    __syncthreads();
    scan[tid] += v;
    __syncthreads();
  }
  if (tid == kPlanThreads - 1) {
    ws.prefix[U] = scan[tid];
    total_s = scan[tid];
  }
  __syncthreads();
  const int64_t T = total_s;
  const int64_t tpw = T > 0 ? (T + workers - 1) / workers : 1;
  int64_t run = scan[tid] - s;  // exclusive prefix
  for (int64_t u = u0; u < u1; ++u) {
    ws.prefix[u] = run;
    const int64_t nxt = run + (unit_len(p, u) + tok - 1) / tok;
    // workers whose first tile lies in [run, nxt)
    for (int64_t w = (run + tpw - 1) / tpw; w < (nxt + tpw - 1) / tpw && w < workers; ++w)
      ws.wunit[w] = static_cast<int32_t>(u);
    run = nxt;
  }
}

// One block per unit: merge the pieces of a unit cut between workers, write
// O = 0 / LSE = -inf for an empty unit, leave whole units alone.
template <int kDv>
__global__ void __launch_bounds__(256) split_combine_kernel(AttnParams p, int workers, int max_workers) {
  const int G = p.group;
  const int64_t U = split_units(p);
  const int64_t u = blockIdx.x;
  SplitWs ws = split_ws(p.workspace, U, max_workers);
  const int64_t T = ws.prefix[U];
  const int64_t ubeg = ws.prefix[u], uend = ws.prefix[u + 1];
  const int h = static_cast<int>(u % p.kv.num_kv_heads);
  const int64_t rb = u / p.kv.num_kv_heads;
  constexpr int kRow = kDv + kPartExtra;
  if (ubeg == uend) {
    for (int i = threadIdx.x; i < G * kDv; i += blockDim.x) {
      const int g = i / kDv, d = i % kDv;
      const int64_t row = rb * p.num_q_heads + static_cast<int64_t>(h) * G + g;
      p.out_o[row * kDv + d] = 0.f;
      if (d == 0) p.out_lse[row] = -INFINITY;
    }
    return;
  }
  const int64_t tpw = (T + workers - 1) / workers;
  const int64_t wa = ubeg / tpw, wb = (uend - 1) / tpw;
  if (wa == wb) return;
  for (int i = threadIdx.x; i < G * kDv; i += blockDim.x) {
    const int g = i / kDv, d = i % kDv;
    float mx = -INFINITY;
    for (int64_t w = wa; w <= wb; ++w)
      mx = fmaxf(mx, ws.part[((w * 2 + (w == wa ? 1 : 0)) * G + g) * kRow + kDv]);
    float acc = 0.f, lsum = 0.f, esum = 0.f;
    for (int64_t w = wa; w <= wb; ++w) {
      const float* hrow = ws.part + ((w * 2 + (w == wa ? 1 : 0)) * G + g) * kRow;
      const float sc = exp2f(hrow[kDv] - mx);
      acc += sc * hrow[d];
      lsum += sc * hrow[kDv + 1];
      esum += sc * hrow[kDv + 2];
    }
    const int64_t row = rb * p.num_q_heads + static_cast<int64_t>(h) * G + g;
    p.out_o[row * kDv + d] = acc / lsum;
    if (d == 0) p.out_lse[row] = (mx + __log2f(esum)) * DCP_LN2;
  }
}

}  // namespace dcp
