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
// log-sum-exp. Grids depend only on the device, never on the lengths. Workers
// find their first unit in one of two ways:
//   * the GQA kernel's workgroups search the local lengths themselves
//     (split_locate) and walk units with their tile counts: the attention
//     kernel is the first launch of a call;
//   * for the MLA kernel, whose register budget has no room for that walk, a
//     one-block planner kernel first writes the tile prefix over units and
//     every worker's first unit to the workspace (split_plan_kernel).
// Either way the cut records (below), their count and the total reach the
// workspace for the combine.
#pragma once

#include <type_traits>

#include "common.h"
#include "halves.h"

namespace dcp {

constexpr int kCombineThreads = 256;
// Per partial head row: O[Dv] (unnormalised, value scale applied), then the
// running max m (log2 units), the sum of the bf16-rounded weights (the
// normaliser of O), the sum of the fp32 weights (the LSE) and one unused
// float, so rows of a Dv divisible by 4 start on 16-byte boundaries.
constexpr int kPartExtra = 4;
// Cut record: a unit cut between workers, as {unit or -1 (none), first tile,
// end tile, worker holding its first tile}. Either one per worker (the unit
// that starts inside the worker's range and runs past its end), or, from the
// planner, one per cut unit and no more.
constexpr int kCutRec = 4;

struct SplitWs {
  int64_t* prefix;  // planned split: [U + 1] tile prefix over units, prefix[U] = total (else unused)
  int32_t* wunit;   // planned split: [workers] unit holding each worker's first tile (else unused)
  int64_t* total;   // [2]: tiles of all units, cut records to read
  int64_t* cut;     // [up to workers][kCutRec], rewritten on every call
  float* part;      // [workers][2][rows][Dv + kPartExtra], rows = tpu * group
};

// The layout depends on the number of workers the launch uses (fixed per
// device) and, for a planned split, on the number of units U (plan_units = U,
// else 0), so the size query and every kernel of a call agree on it.
__host__ __device__ inline SplitWs split_ws(void* base, int max_workers, int64_t plan_units) {
  SplitWs w;
  char* p = static_cast<char*>(base);
  w.prefix = reinterpret_cast<int64_t*>(p);
  p += align_up(static_cast<size_t>(plan_units + 1) * sizeof(int64_t), 256);
  w.wunit = reinterpret_cast<int32_t*>(p);
  p += align_up(static_cast<size_t>(max_workers) * sizeof(int32_t), 256);
  w.total = reinterpret_cast<int64_t*>(p);
  w.cut = w.total + 2;
  p += align_up(static_cast<size_t>(2 + max_workers * kCutRec) * sizeof(int64_t), 256);
  w.part = reinterpret_cast<float*>(p);
  return w;
}

static inline size_t split_ws_bytes(int max_workers, int64_t plan_units, int rows, int dv) {
  size_t b = align_up(static_cast<size_t>(plan_units + 1) * sizeof(int64_t), 256);
  b += align_up(static_cast<size_t>(max_workers) * sizeof(int32_t), 256);
  b += align_up(static_cast<size_t>(2 + max_workers * kCutRec) * sizeof(int64_t), 256);
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

// (Unit indices fit in 32 bits: the host refuses larger splits.)
__device__ __forceinline__ UnitRef unit_ref(const AttnParams& p, int64_t u64) {
  const int u = static_cast<int>(u64);
  UnitRef x;
  const int tg = u % p.ntg;
  const int uh = u / p.ntg;
  x.h = uh % p.kv.num_kv_heads;
  const int rb = uh / p.kv.num_kv_heads;
  x.rb = rb;
  x.b = rb % p.batch;
  x.r = rb / p.batch;
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

// Tiles of one KV head's units of (rank r, request b): all its token groups.
__device__ __forceinline__ int64_t pair_tiles(const AttnParams& p, int b, int r, int tok_log2) {
  int64_t s = 0;
  for (int tg = 0; tg < p.ntg; ++tg) s += group_tiles(p, b, r, tg, tok_log2);
  return s;
}

// Tiles of unit u.
__device__ __forceinline__ int64_t unit_tiles(const AttnParams& p, int64_t u, int tok_log2) {
  const UnitRef x = unit_ref(p, u);
  return group_tiles(p, x.b, x.r, x.i0 / p.tpu, tok_log2);
}

// ceil(a / b) and floor(a / b) for 0 <= a < 2^53, b >= 1, through fp64 (exact
// in that range up to one-off rounding, which the loops correct). 64-bit
// integer divisions are software routines on the GPU.
__device__ __forceinline__ int64_t ceil_div_fp64(int64_t a, int64_t b) {
  int64_t q = static_cast<int64_t>(static_cast<double>(a) / static_cast<double>(b));
  while (q * b < a) ++q;
  while (q > 0 && (q - 1) * b >= a) --q;
  return q;
}
__device__ __forceinline__ int64_t floor_div_fp64(int64_t a, int64_t b) {
  int64_t q = static_cast<int64_t>(static_cast<double>(a) / static_cast<double>(b));
  while (q > 0 && q * b > a) --q;
  while ((q + 1) * b <= a) ++q;
  return q;
}

// Inclusive prefix sum over the 64 lanes of a wavefront.
__device__ __forceinline__ int64_t wave_incl_scan(int64_t v, int lane) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int64_t x = __shfl_up(v, off, 64);
    if (lane >= off) v += x;
  }
  return v;
}

// A wave-uniform copy of v (through the 32-bit broadcast, half by half).
__device__ __forceinline__ int64_t uniform64(int64_t v) {
  const uint64_t u = static_cast<uint64_t>(v);
  return static_cast<int64_t>(
      join_halves(__builtin_amdgcn_readfirstlane(low_half(u)), __builtin_amdgcn_readfirstlane(high_half(u))));
}

// Where a worker starts (wave-uniform values).
struct SplitStart {
  int64_t total;         // tiles of all units
  int64_t wstart, wend;  // the worker's tile range; empty when wstart >= total
  int64_t u;             // unit holding tile wstart (when the range is not empty)
  int64_t ubeg, uend;    // its tile range
};

// Called by every thread of a kThreads-thread workgroup (it synchronises the
// block); `worker` is uniform per wavefront, `lds` holds kThreads + 16 int64.
//
// Thread t sums the tiles of (rank, request) pairs [t c, t c + c), c =
// ceil(pairs / kThreads); a block scan of those sums gives the total and the
// chunk holding the worker's first tile wstart = worker * ceil(total /
// workers); the wavefront then rescans that chunk's pairs 64 at a time to
// find the pair, and within the pair the KV head (all heads of a pair have
// the same tiles) and the token group.
template <int kThreads>
__device__ SplitStart split_locate(const AttnParams& p, int tok_log2, int workers, int worker, int64_t* lds) {
  static_assert(kThreads % 64 == 0 && kThreads <= 1024, "whole wavefronts");
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int H = p.kv.num_kv_heads;
  const int RB = p.rank_count * p.batch;  // (rank, request) pairs, < 2^31
  const int c = (RB + kThreads - 1) / kThreads;
  const int rb0 = min(RB, tid * c), rb1 = min(RB, rb0 + c);
  int64_t s = 0;
  if (rb0 < rb1) {
    int b = rb0 % p.batch, r = rb0 / p.batch;
    if (p.q_len == 1) {
      // one length per pair: eight loads in flight before the first is used
      const int tok_m1 = (1 << tok_log2) - 1;
      for (int rb = rb0; rb < rb1; rb += 8) {
        int len[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          // (b, r) stays at the chunk's last pair past its end: every load is in bounds
          len[j] = query_len(p, b, 0, r);
          if (rb + j >= rb1) len[j] = 0;
          if (rb + j + 1 < rb1 && ++b == p.batch) b = 0, ++r;
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) s += (static_cast<int64_t>(len[j]) + tok_m1) >> tok_log2;
      }
    } else {
      for (int rb = rb0; rb < rb1; ++rb) {
        s += pair_tiles(p, b, r, tok_log2);
        if (++b == p.batch) b = 0, ++r;
      }
    }
    s *= H;
  }
  // block inclusive scan: within each wavefront, then over the wavefront sums
  int64_t incl = wave_incl_scan(s, lane);
  if (lane == 63) lds[kThreads + wid] = incl;
  __syncthreads();
  int64_t before = 0;
  for (int w = 0; w < wid; ++w) before += lds[kThreads + w];
  lds[tid] = before + incl;
  __syncthreads();

  SplitStart st;
  st.total = uniform64(lds[kThreads - 1]);
  const int64_t T = st.total;
  const int64_t tpw = T > 0 ? ceil_div_fp64(T, workers) : 1;
  st.wstart = static_cast<int64_t>(worker) * tpw;
  st.wend = min(T, st.wstart + tpw);
  st.u = -1;
  st.ubeg = st.uend = 0;
  if (st.wstart >= T) return st;
  const int64_t wstart = st.wstart;

  // the chunk holding tile wstart: the first thread whose inclusive sum exceeds it
  int j = -1;
  for (int k = 0; k < kThreads / 64 && j < 0; ++k) {
    const uint64_t m = __ballot(lds[64 * k + lane] > wstart);
    if (m) j = 64 * k + __builtin_ctzll(m);
  }
  j = __builtin_amdgcn_readfirstlane(j);
  if (j < 0) {  // unreachable: lds[kThreads - 1] = T > wstart
    st.wstart = st.wend = T;
    return st;
  }
  int64_t pos = j > 0 ? uniform64(lds[j - 1]) : 0;
  const int cb = min(RB, j * c), ce = min(RB, cb + c);
  int pair = -1;
  int64_t pexcl = 0;
  for (int base = cb; base < ce; base += 64) {
    const int x = base + lane;
    int64_t w = 0;
    if (x < ce) w = pair_tiles(p, x % p.batch, x / p.batch, tok_log2) * H;
    const int64_t in2 = wave_incl_scan(w, lane) + pos;
    const uint64_t m = __ballot(in2 > wstart);
    if (m) {
      const int f = __builtin_ctzll(m);
      pair = base + f;
      pexcl = uniform64(__shfl(in2 - w, f, 64));
      break;
    }
    pos = uniform64(__shfl(in2, 63, 64));
  }
  pair = __builtin_amdgcn_readfirstlane(pair);
  if (pair < 0) {  // unreachable: the chunk's tiles cover wstart
    st.wstart = st.wend = T;
    return st;
  }
  const int b = pair % p.batch, r = pair / p.batch;
  const int64_t srb = uniform64(pair_tiles(p, b, r, tok_log2));  // > 0
  const int64_t off = wstart - pexcl;                            // < H * srb
  const int64_t h = floor_div_fp64(off, srb);
  int64_t rem = off - h * srb;
  int tg = 0;
  int64_t gt = 0;
  for (; tg < p.ntg; ++tg) {  // the group holding the tile (empty groups are passed)
    gt = group_tiles(p, b, r, tg, tok_log2);
    if (rem < gt) break;
    rem -= gt;
  }
  st.u = uniform64((static_cast<int64_t>(pair) * H + h) * p.ntg + tg);
  st.ubeg = uniform64(wstart - rem);
  st.uend = uniform64(st.ubeg + gt);
  return st;
}

// A worker's record for the combine (tile range [wstart, wend)): the unit of
// its last piece when that unit starts inside the range and runs past its
// end, else none (last_u = -1 for a worker without tiles). Written by one
// lane; worker 0 also stores the header (total tiles, one record per worker).
__device__ __forceinline__ void split_record(const SplitWs& ws, int worker, int64_t wstart, int64_t wend,
                                             int64_t last_u, int64_t last_beg, int64_t last_end) {
  const bool cut = last_u >= 0 && last_beg >= wstart && last_end > wend;
  int64_t* rec = ws.cut + static_cast<int64_t>(worker) * kCutRec;
  rec[0] = cut ? last_u : -1;
  rec[1] = last_beg;
  rec[2] = last_end;
  rec[3] = worker;
}

// Planned split (one block): tile prefix over units, the first unit of every
// worker, the total and every worker's cut record. Units come in runs of
// Hkv * ntg per (rank, request) pair, and each thread takes a contiguous range
// of pairs, so a unit's position is a loop counter rather than a
// decomposition of its index (64-bit divisions are software routines, and on
// one CU they set the planner's time).
constexpr int kPlanThreads = 1024;

static __global__ void __launch_bounds__(kPlanThreads) split_plan_kernel(AttnParams p, int tok_log2, int workers) {
  __shared__ int64_t wsum[kPlanThreads / 64];
  __shared__ int64_t total_s;
  __shared__ int ncut_s;
  const int64_t U = split_units(p);
  SplitWs ws = split_ws(p.workspace, workers, U);
  const int H = p.kv.num_kv_heads, ntg = p.ntg;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int RB = p.rank_count * p.batch;  // (rank, request) pairs; U < 2^31
  const int chunk = (RB + kPlanThreads - 1) / kPlanThreads;
  const int rb0 = min(RB, tid * chunk), rb1 = min(RB, rb0 + chunk);
  const int b0 = p.batch > 0 ? rb0 % p.batch : 0, r0 = p.batch > 0 ? rb0 / p.batch : 0;
  if (tid == 0) ncut_s = 0;
  int64_t s = 0;
  for (int rb = rb0, b = b0, r = r0; rb < rb1; ++rb) {
    int64_t srb = 0;
    for (int tg = 0; tg < ntg; ++tg) srb += group_tiles(p, b, r, tg, tok_log2);
    s += srb * H;
    if (++b == p.batch) b = 0, ++r;
  }
  // block exclusive scan: within each wavefront, then over the 16 wavefront sums
  const int64_t incl = wave_incl_scan(s, lane);
  if (lane == 63) wsum[wid] = incl;
  __syncthreads();
  int64_t before = 0;
  for (int w = 0; w < wid; ++w) before += wsum[w];
  if (tid == kPlanThreads - 1) total_s = before + incl;
  __syncthreads();
  const int64_t T = total_s;
  const int64_t tpw = T > 0 ? ceil_div_fp64(T, workers) : 1;
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
        if (cut) {  // one record per cut unit, in no particular order (at most one per worker)
          int64_t* rec = ws.cut + static_cast<int64_t>(atomicAdd(&ncut_s, 1)) * kCutRec;
          rec[0] = u;
          rec[1] = run;
          rec[2] = nxt;
          rec[3] = floor_div_fp64(run, tpw);  // the worker holding its first tile
        }
        run = nxt;
      }
    }
    if (++b == p.batch) b = 0, ++r;
  }
  if (tid == kPlanThreads - 1) {
    ws.prefix[U] = T;
    ws.total[0] = T;
  }
  __syncthreads();
  if (tid == 0) ws.total[1] = ncut_s;
}

// Fixed grid; one wavefront per item. Items of the first kind are (cut
// record, row of its unit) for every record the workspace header lists, a row being (query token,
// query head of the group): merge the pieces of the unit, or write O = 0 /
// LSE = -inf for a row that sees no token of the unit (a query earlier than
// every local token; its pieces carry m = -inf). Pieces are read four at a
// time (rows as 8- or 16-byte vectors, the statistics as one 16-byte load),
// all issued before the first is used; a unit cut into at most four pieces
// (the usual case) takes its maximum from the same loads. Items of the
// second kind are (64 token groups, one output row slot of a group): lane l
// tests group 64 k + l for local tokens, and the row of every empty group
// (no worker visits it) gets O = 0 / LSE = -inf.
template <int kDv>
__global__ void __launch_bounds__(kCombineThreads)
    split_combine_kernel(AttnParams p, int tok_log2, int workers, int64_t plan_units, int vec_out) {
  constexpr int kVec = kDv >= 256 ? 4 : kDv / 64;  // floats per lane per load
  constexpr int kRounds = kDv / (64 * kVec);
  static_assert(kVec == 2 || kVec == 4, "combine widths");
  static_assert(kDv % (64 * kVec) == 0 && (kDv + kPartExtra) % 4 == 0, "combine row layout");
  using VecT = typename std::conditional<kVec == 4, float4, float2>::type;
  constexpr int kRow = kDv + kPartExtra;
  constexpr int kBatch = 4;
  const int G = p.group, rows = p.tpu * p.group;
  SplitWs ws = split_ws(p.workspace, workers, plan_units);
  const int64_t T = ws.total[0];
  const int64_t tpw = T > 0 ? ceil_div_fp64(T, workers) : 1;
  const int64_t items_cut = ws.total[1] * rows;
  const int groups = p.rank_count * p.batch * p.ntg;  // < 2^31
  const int slots = p.tpu * p.num_q_heads;            // output rows of a token group
  const int64_t items = items_cut + static_cast<int64_t>((groups + 63) / 64) * slots;
  const int lane = threadIdx.x & 63;
  const int64_t wave0 = (static_cast<int64_t>(blockIdx.x) * kCombineThreads + threadIdx.x) >> 6;
  const int64_t nwaves = (static_cast<int64_t>(gridDim.x) * kCombineThreads) >> 6;
  for (int64_t it = wave0; it < items; it += nwaves) {
    if (it >= items_cut) {  // empty token groups
      const int64_t e = it - items_cut;
      const int k = static_cast<int>(e / slots), slot = static_cast<int>(e % slots);
      const int g = 64 * k + lane;  // group (r * batch + b) * ntg + tg
      bool empty = false;
      if (g < groups) {
        const int tg = g % p.ntg, rb = g / p.ntg;
        empty = group_tiles(p, rb % p.batch, rb / p.batch, tg, tok_log2) == 0;
      }
      uint64_t m = __ballot(empty);
      while (m) {
        const int gg = 64 * k + __builtin_ctzll(m);
        m &= m - 1;
        const int tg = gg % p.ntg, rb = gg / p.ntg;
        const int i = tg * p.tpu + slot / p.num_q_heads;
        if (i >= min(p.q_len, tg * p.tpu + p.tpu)) continue;  // past the request's last query token
        const int64_t row = (static_cast<int64_t>(rb) * p.q_len + i) * p.num_q_heads + slot % p.num_q_heads;
        float* dst = p.out_o + row * kDv;
#pragma unroll
        for (int q = 0; q < kDv / 64; ++q) dst[lane + 64 * q] = 0.f;
        if (lane == 0) p.out_lse[row] = -INFINITY;
      }
      continue;
    }
    const int c = static_cast<int>(it % rows);
    const int64_t* rec = ws.cut + (it / rows) * kCutRec;
    const int64_t u = rec[0];
    if (u < 0) continue;  // no unit starts in this worker's range and runs past it
    const int64_t ubeg = rec[1], uend = rec[2], wk = rec[3];
    const UnitRef x = unit_ref(p, u);
    const int i = x.i0 + c / G;
    if (i >= x.i1) continue;  // a row past the request's last query token
    const int64_t row = out_row(p, x, i, c % G);
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
    if (ubeg != uend) {  // (always: a cut unit has tiles)
      wa = wk;           // = ubeg / tpw
      wb = floor_div_fp64(uend - 1, tpw);
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
// (plan_units: as for split_ws)
template <int kDv>
static inline void launch_split_combine(const AttnParams& p, int tok, int workers, int64_t plan_units) {
  const int vec_out = reinterpret_cast<uintptr_t>(p.out_o) % 16 == 0;
  hipLaunchKernelGGL(split_combine_kernel<kDv>, dim3(8 * device_cu_count()), dim3(kCombineThreads), 0, p.stream, p,
                     log2_exact(tok), workers, plan_units, vec_out);
}

}  // namespace dcp
