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

#include <type_traits>

#include "common.h"

namespace dcp {

constexpr int kPlanThreads = 1024;
constexpr int kCombineThreads = 256;
// Per partial head row: O[Dv] (unnormalised, value scale applied), then the
// running max m (log2 units), the sum of the bf16-rounded weights (the
// normaliser of O), the sum of the fp32 weights (the LSE) and one unused
// float, so rows of a Dv divisible by 4 start on 16-byte boundaries.
constexpr int kPartExtra = 4;

struct SplitWs {
  int64_t* prefix;  // [U + 1] tile prefix over units; prefix[U] = total tiles
  int32_t* wunit;   // [workers] unit holding each worker's first tile
  int32_t* todo;    // [1 + U + workers]: count, then the units that are empty or cut
  float* part;      // [workers][2][rows][Dv + kPartExtra], rows = tpu * group
};

// The layout depends on the number of workers the launch uses (fixed per
// device), so the size query and every kernel of a call agree on it.
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

// Output row of (query token i, query head h * group + g) of unit x.
__device__ __forceinline__ int64_t out_row(const AttnParams& p, const UnitRef& x, int i, int g) {
  return (x.rb * p.q_len + i) * p.num_q_heads + static_cast<int64_t>(x.h) * p.group + g;
}

// Tiles (tok = 1 << tok_log2 tokens each) of token group tg of request b on
// rank r: as many local tokens as the group's longest query sees. Every KV
// head of the pair has the same count.
__device__ __forceinline__ int64_t group_tiles(const AttnParams& p, int b, int r, int tg, int tok_log2) {
  const int i0 = tg * p.tpu, i1 = min(p.q_len, i0 + p.tpu);
  int n = 0;
  for (int i = i0; i < i1; ++i) n = max(n, query_len(p, b, i, r));
  return (static_cast<int64_t>(n) + (int64_t(1) << tok_log2) - 1) >> tok_log2;
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
// workers). Units come in runs of Hkv * ntg per (rank, request) pair, and each
// thread takes a contiguous range of pairs, so a unit's position is a loop
// counter rather than a decomposition of its index (64-bit divisions are
// software routines, and on one CU they set the planner's time).
static __global__ void __launch_bounds__(kPlanThreads) split_plan_kernel(AttnParams p, int tok_log2, int workers) {
  __shared__ int64_t wsum[kPlanThreads / 64];
  __shared__ int64_t total_s;
  __shared__ int todo_n;
  const int64_t U = split_units(p);
  SplitWs ws = split_ws(p.workspace, U, workers);
  const int H = p.kv.num_kv_heads, ntg = p.ntg;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int RB = p.rank_count * p.batch;  // (rank, request) pairs; U < 2^31
  const int chunk = (RB + kPlanThreads - 1) / kPlanThreads;
  const int rb0 = min(RB, tid * chunk), rb1 = min(RB, rb0 + chunk);
  const int b0 = p.batch > 0 ? rb0 % p.batch : 0, r0 = p.batch > 0 ? rb0 / p.batch : 0;
  int64_t s = 0;
  for (int rb = rb0, b = b0, r = r0; rb < rb1; ++rb) {
    int64_t srb = 0;
    for (int tg = 0; tg < ntg; ++tg) srb += group_tiles(p, b, r, tg, tok_log2);
    s += srb * H;
    if (++b == p.batch) b = 0, ++r;
  }
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
  // wfirst: the first worker whose first tile (w * tpw) is at or after `run`;
  // it only moves forward, so one division per thread
  int64_t wfirst = ceil_div_fp64(run, tpw);
  for (int rb = rb0, b = b0, r = r0; rb < rb1; ++rb) {
    const int64_t t1 = ntg == 1 ? group_tiles(p, b, r, 0, tok_log2) : 0;
    for (int h = 0; h < H; ++h) {
      for (int tg = 0; tg < ntg; ++tg) {
        const int64_t u = (static_cast<int64_t>(rb) * H + h) * ntg + tg;
        ws.prefix[u] = run;
        const int64_t nxt = run + (ntg == 1 ? t1 : group_tiles(p, b, r, tg, tok_log2));
        // workers whose first tile lies in [run, nxt) start in this unit; one
        // starting after its first tile cuts it (every tile < T belongs to a
        // worker below `workers`, so the bound misses no cut)
        bool cut = false;
        for (; wfirst < workers && wfirst * tpw < nxt; ++wfirst) {
          ws.wunit[wfirst] = static_cast<int32_t>(u);
          cut |= wfirst * tpw > run;
        }
        if (nxt == run || cut) ws.todo[1 + atomicAdd(&todo_n, 1)] = static_cast<int32_t>(u);  // empty or cut
        run = nxt;
      }
    }
    if (++b == p.batch) b = 0, ++r;
  }
  if (tid == kPlanThreads - 1) ws.prefix[U] = T;
  __syncthreads();
  if (tid == 0) ws.todo[0] = todo_n;
}

// Fixed grid; one wavefront per (listed unit, row of the unit) item, a row
// being (query token, query head of the group): merge the pieces of a unit
// cut between workers, or write O = 0 / LSE = -inf for an empty unit and for
// a row that sees no token of the unit (a query earlier than every local
// token; its pieces carry m = -inf). Pieces are read four at a time (rows as
// 8- or 16-byte vectors, the statistics as one 16-byte load), all issued
// before the first is used; a unit cut into at most four pieces (the usual
// case) takes its maximum from the same loads.
template <int kDv>
__global__ void __launch_bounds__(kCombineThreads) split_combine_kernel(AttnParams p, int workers, int vec_out) {
  constexpr int kVec = kDv >= 256 ? 4 : kDv / 64;  // floats per lane per load
  constexpr int kRounds = kDv / (64 * kVec);
  static_assert(kVec == 2 || kVec == 4, "combine widths");
  static_assert(kDv % (64 * kVec) == 0 && (kDv + kPartExtra) % 4 == 0, "combine row layout");
  using VecT = typename std::conditional<kVec == 4, float4, float2>::type;
  constexpr int kRow = kDv + kPartExtra;
  constexpr int kBatch = 4;
  const int G = p.group, rows = p.tpu * p.group;
  const int64_t U = split_units(p);
  SplitWs ws = split_ws(p.workspace, U, workers);
  const int64_t T = ws.prefix[U];
  const int64_t tpw = T > 0 ? (T + workers - 1) / workers : 1;
  const int64_t items = static_cast<int64_t>(ws.todo[0]) * rows;
  const int lane = threadIdx.x & 63;
  const int64_t wave0 = (static_cast<int64_t>(blockIdx.x) * kCombineThreads + threadIdx.x) >> 6;
  const int64_t nwaves = (static_cast<int64_t>(gridDim.x) * kCombineThreads) >> 6;
  for (int64_t it = wave0; it < items; it += nwaves) {
    const int64_t u = ws.todo[1 + it / rows];
    const int c = static_cast<int>(it % rows);
    const UnitRef x = unit_ref(p, u);
    const int i = x.i0 + c / G;
    if (i >= x.i1) continue;  // a row past the request's last query token
    const int64_t row = out_row(p, x, i, c % G);
    const int64_t ubeg = ws.prefix[u], uend = ws.prefix[u + 1];
    float* dst = p.out_o + row * kDv;
    // piece w's row: the "tail" slot of the worker where the unit starts, else the "head" slot
    auto piece = [&](int64_t w, int64_t wa) {
      return ws.part + ((w * 2 + (w == wa ? 1 : 0)) * rows + c) * kRow;
    };
    float mx = -INFINITY;
    int64_t wa = 0, wb = -1;
    VecT v[kBatch][kRounds];
    float4 st[kBatch];
    auto load_batch = [&](int64_t w0) {
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        const float* hrow = piece(min(w0 + j, wb), wa);
        st[j] = *reinterpret_cast<const float4*>(hrow + kDv);
#pragma unroll
        for (int q = 0; q < kRounds; ++q) v[j][q] = reinterpret_cast<const VecT*>(hrow)[lane + 64 * q];
      }
    };
    if (ubeg != uend) {
      wa = ubeg / tpw;
      wb = (uend - 1) / tpw;
      if (wb - wa < kBatch) {
        load_batch(wa);
#pragma unroll
        for (int j = 0; j < kBatch; ++j)
          if (wa + j <= wb) mx = fmaxf(mx, st[j].x);
      } else {
        for (int64_t w0 = wa; w0 <= wb; w0 += 8) {
          float mm[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) mm[j] = piece(min(w0 + j, wb), wa)[kDv];
#pragma unroll
          for (int j = 0; j < 8; ++j) mx = fmaxf(mx, mm[j]);  // repeats of the last piece change nothing
        }
      }
    }
    if (mx == -INFINITY) {
#pragma unroll
      for (int k = 0; k < kDv / 64; ++k) dst[lane + 64 * k] = 0.f;
      if (lane == 0) p.out_lse[row] = -INFINITY;
      continue;
    }
    float acc[kRounds][kVec];
#pragma unroll
    for (int q = 0; q < kRounds; ++q)
#pragma unroll
      for (int k = 0; k < kVec; ++k) acc[q][k] = 0.f;
    float lsum = 0.f, esum = 0.f;
    for (int64_t w0 = wa; w0 <= wb; w0 += kBatch) {
      if (wb - wa >= kBatch) load_batch(w0);
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        if (w0 + j > wb) break;
        const float sc = exp2f(st[j].x - mx);  // 0 for a piece with m = -inf
#pragma unroll
        for (int q = 0; q < kRounds; ++q) {
          const float* e = reinterpret_cast<const float*>(&v[j][q]);
#pragma unroll
          for (int k = 0; k < kVec; ++k) acc[q][k] += sc * e[k];
        }
        lsum += sc * st[j].y;
        esum += sc * st[j].z;
      }
    }
    const float inv = 1.f / lsum;
    if (vec_out) {
#pragma unroll
      for (int q = 0; q < kRounds; ++q) {
        VecT o;
        float* e = reinterpret_cast<float*>(&o);
#pragma unroll
        for (int k = 0; k < kVec; ++k) e[k] = acc[q][k] * inv;
        reinterpret_cast<VecT*>(dst)[lane + 64 * q] = o;
      }
    } else {
#pragma unroll
      for (int q = 0; q < kRounds; ++q)
#pragma unroll
        for (int k = 0; k < kVec; ++k) dst[(lane + 64 * q) * kVec + k] = acc[q][k] * inv;
    }
    if (lane == 0) p.out_lse[row] = (mx + __log2f(esum)) * DCP_LN2;
  }
}

static inline int log2_exact(int x) {
  int l = 0;
  while ((1 << l) < x) ++l;
  return l;
}

static inline void launch_split_plan(const AttnParams& p, int tok, int workers) {
  hipLaunchKernelGGL(split_plan_kernel, dim3(1), dim3(kPlanThreads), 0, p.stream, p, log2_exact(tok), workers);
}

// Eight workgroups of four wavefronts per CU: every SIMD holds eight items in flight.
template <int kDv>
static inline void launch_split_combine(const AttnParams& p, int workers) {
  const int vec_out = reinterpret_cast<uintptr_t>(p.out_o) % 16 == 0;
  hipLaunchKernelGGL(split_combine_kernel<kDv>, dim3(8 * device_cu_count()), dim3(kCombineThreads), 0, p.stream, p,
                     workers, vec_out);
}

}  // namespace dcp
