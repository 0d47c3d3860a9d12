// GQA per-rank partial decode attention on MFMA (bf16 or fp8-e4m3 KV, head
// dim 128, up to 16 (query token, query head) columns per KV head: a decode
// query's group, or the groups of several query tokens of a request).
//
// Source: "Decode Context Parallel (DCP)" (vLLM Ascend design doc), section
// "Decode" (attention of the gathered query heads against the local KV shard,
// partial output and LSE out); "Efficient Decode Context Parallelism with vLLM
// for Long Context Workloads", section 5.4 (the query heads of a group share
// one KV head).
//
// Work split: stream-K over (rank, request, KV head, query tokens) units
// (splitkv.h) with
// one persistent wavefront per worker and tiles of TOK tokens (16 KB of K and
// V per tile), streamed two tiles at a time straight into registers.
//
// Per wavefront and tile, with lane l = 16*qd + n (n = l % 16, qd = l / 16):
//   scores  S^T[token, head] = K[token, :] . Q[head, :]   (MFMA 16x16x32 bf16,
//           A = K rows loaded straight from HBM in operand layout, B = Q^T
//           held in registers, head columns >= group are zero)
//   softmax online, per head column, against a reference max that moves
//           only when a tile's max exceeds it by more than 2^8; the weights are
//           rounded to bf16 for the value product and the same rounded values
//           form the normalising sum (O is an exact convex combination of the
//           values), while an fp32 sum of the unrounded weights gives the LSE
//   values  O^T[dim, head] += V^T[dim, token] . P^T[token, head] (A = V^T,
//           read straight from HBM because V is stored transposed inside a
//           block, [block, head, dim, token]; B = P^T from the score registers)
// The token order inside a tile is permuted so that the score accumulator of
// lane l already holds exactly the weights that lane must feed to the value
// product: no LDS, no shuffles besides the max/sum reductions. fp8 codes are
// widened to bf16 in registers (exact) and the per-head scales are applied to
// the scores and to the output, outside the dot products.
#include <atomic>

#include "splitkv.h"

namespace dcp {

constexpr int kGqaDim = 128;
constexpr int kGqaMaxWorkers = 8192;
constexpr int kGqaWavesPerBlock = 4;
constexpr float kGqaRescaleLog2 = 8.f;  // largest weight kept without rescaling: 2^8

template <bool kFp8>
struct GqaTile {
  static constexpr int TOK = kFp8 ? 64 : 32;  // tokens per tile
  static constexpr int TOK_LOG2 = kFp8 ? 6 : 5;
  static constexpr int NT = TOK / 16;         // score row tiles (16 tokens each)
  static constexpr int RUN = TOK / 4;         // consecutive tokens per lane group
  static constexpr int KS = TOK / 32;         // value-product k-steps
};

// 8 fp8 codes (two dwords) -> 8 bf16, exact.
__device__ __forceinline__ bf16x8_t fp8x8_to_bf16x8(uint32_t d0, uint32_t d1) {
  const bf16x2_t a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d0, 1.0f, false);
  const bf16x2_t b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d0, 1.0f, true);
  const bf16x2_t c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d1, 1.0f, false);
  const bf16x2_t d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d1, 1.0f, true);
  return bf16x8_t{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

__device__ __forceinline__ u32x4_t ldg16(const void* p) { return *reinterpret_cast<const u32x4_t*>(p); }

// KV is streamed exactly once: non-temporal loads (measured ~14% more read
// bandwidth than cached loads on MI355X).
__device__ __forceinline__ u32x4_t ldg16_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
}

// Zero bytes [keep, 16) of a 16-byte vector.
__device__ __forceinline__ u32x4_t keep_bytes(u32x4_t v, int keep) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int k = keep - 4 * i;
    const uint32_t m = k >= 4 ? 0xffffffffu : (k <= 0 ? 0u : (0xffffffffu >> (32 - 8 * k)));
    v[i] &= m;
  }
  return v;
}

// ---------------------------------------------------------------------------
// Tile pieces. Lane l = 16*qd + n. Tiles start at multiples of TOK and the
// block size is a multiple of 16, so every aligned 16-token chunk lies in one
// KV block. A lane's K rows all lie in chunk kc, its V run in chunk vc.
// ---------------------------------------------------------------------------
template <bool kFp8>
struct GqaLane {
  using C = GqaTile<kFp8>;
  static __device__ __forceinline__ int kc(int n) { return (C::RUN * (n >> 2)) >> 4; }
  static __device__ __forceinline__ int koff(int n) { return ((C::RUN * (n >> 2)) & 15) + (n & 3); }
  static __device__ __forceinline__ int vc(int qd) { return (C::RUN * qd) >> 4; }
  static __device__ __forceinline__ int voff(int qd) { return (C::RUN * qd) & 15; }
};

// First token of a lane's chunk in tile t; a chunk past the shard's end
// (len) is replaced by the tile's first chunk, which always holds a token.
template <bool kFp8>
__device__ __forceinline__ int gqa_chunk_start(int t, int chunk, int len) {
  const int t0 = t * GqaTile<kFp8>::TOK;
  const int cs = t0 + 16 * chunk;
  return cs < len ? cs : t0;
}

struct GqaIds {
  int32_t k, v;  // physical blocks of the lane's K chunk and V chunk
};

template <bool kFp8>
__device__ __forceinline__ GqaIds gqa_load_ids(const int32_t* bt, int t, int len, int bs, int n, int qd) {
  using L = GqaLane<kFp8>;
  GqaIds r;
  r.k = bt[gqa_chunk_start<kFp8>(t, L::kc(n), len) / bs];
  r.v = bt[gqa_chunk_start<kFp8>(t, L::vc(qd), len) / bs];
  return r;
}

template <bool kFp8>
struct GqaBuf {
  u32x4_t k[GqaTile<kFp8>::NT][kFp8 ? 2 : 4];  // K rows in MFMA A-operand layout
  u32x4_t v[8];                                // V^T runs, one per 16 value dims
};

// Issue the loads of tile t (raw bytes; masking happens in gqa_tile).
template <bool kFp8>
__device__ __forceinline__ void gqa_issue(GqaBuf<kFp8>& B, GqaIds ids, int t, int len, int bs, const char* kh,
                                          int64_t ks1, int64_t ks3, const char* vh, int64_t vs1, int64_t vs4,
                                          int n, int qd) {
  using L = GqaLane<kFp8>;
  constexpr int EB = kFp8 ? 1 : 2;
  const int csk = gqa_chunk_start<kFp8>(t, L::kc(n), len);
  const char* krow = kh + (static_cast<int64_t>(ids.k) * ks1 + static_cast<int64_t>(csk % bs + L::koff(n)) * ks3) * EB +
                     16 * qd;
#pragma unroll
  for (int ut = 0; ut < GqaTile<kFp8>::NT; ++ut)
#pragma unroll
    for (int j = 0; j < (kFp8 ? 2 : 4); ++j) B.k[ut][j] = ldg16_stream(krow + (4 * ut) * ks3 * EB + 64 * j);
  const int csv = gqa_chunk_start<kFp8>(t, L::vc(qd), len);
  const char* run = vh + (static_cast<int64_t>(ids.v) * vs1 + csv % bs + L::voff(qd) + n * vs4) * EB;
#pragma unroll
  for (int nt = 0; nt < 8; ++nt) B.v[nt] = ldg16_stream(run + static_cast<int64_t>(16 * nt) * vs4 * EB);
  // nothing of the tile computed next may move above these loads: the wait
  // for that tile's data must leave this tile's loads in flight
  __builtin_amdgcn_sched_barrier(0);
}

// Scores, online softmax and value product of one tile whose loads landed.
// len: the unit's local tokens (the longest query's); col_len: tokens this
// lane's column (query token, head) sees; min_len: the fewest any column sees.
template <bool kFp8>
__device__ __forceinline__ void gqa_tile(GqaBuf<kFp8>& B, int t0, int len, int col_len, int min_len, float c2,
                                         const bf16x8_t (&qop)[4], f32x4_t (&o)[8], float& m_run, float& l_run,
                                         float& e_run, int qd) {
  using C = GqaTile<kFp8>;
  constexpr int NT = C::NT, RUN = C::RUN;
  constexpr int EB = kFp8 ? 1 : 2;
  // ---- scores ---------------------------------------------------------
  f32x4_t s[NT];
#pragma unroll
  for (int ut = 0; ut < NT; ++ut) {
    s[ut] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      bf16x8_t a;
      if constexpr (kFp8) {
        const u32x4_t& w = B.k[ut][k >> 1];
        a = (k & 1) ? fp8x8_to_bf16x8(w[2], w[3]) : fp8x8_to_bf16x8(w[0], w[1]);
      } else {
        a = __builtin_bit_cast(bf16x8_t, B.k[ut][k]);
      }
      s[ut] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qop[k], s[ut], 0, 0, 0);
    }
    // keep each row tile's widened operands next to their MFMAs (otherwise
    // the scheduler hoists every conversion and doubles the live registers)
    __builtin_amdgcn_sched_barrier(0);
  }
  // ---- online softmax (log2 domain) ----------------------------------
#pragma unroll
  for (int ut = 0; ut < NT; ++ut) s[ut] *= c2;
  if (t0 + C::TOK > min_len) {  // a tile some column sees only in part (wave-uniform test)
#pragma unroll
    for (int ut = 0; ut < NT; ++ut)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (t0 + RUN * qd + 4 * ut + i >= col_len) s[ut][i] = -INFINITY;
  }
  float mloc = -INFINITY;
#pragma unroll
  for (int ut = 0; ut < NT; ++ut)
#pragma unroll
    for (int i = 0; i < 4; ++i) mloc = fmaxf(mloc, s[ut][i]);
  mloc = fmaxf(mloc, __shfl_xor(mloc, 16, 64));
  mloc = fmaxf(mloc, __shfl_xor(mloc, 32, 64));
  // Lazy rescaling: the weights are taken relative to a reference max m_run
  // that only moves (rescaling O and the sums) when some column's tile max
  // exceeds it by more than 2^8; otherwise weights up to 2^8 are exact
  // enough in fp32 and bf16 alike. The decision is wave-uniform.
  if (__builtin_amdgcn_ballot_w64(mloc > m_run + kGqaRescaleLog2) != 0) {
    const float m_new = fmaxf(m_run, mloc);
    // 0 on a column's first tile with tokens; 1 for a column that has seen none yet
    const float alpha = m_new == -INFINITY ? 1.f : exp2f(m_run - m_new);
    m_run = m_new;
    l_run *= alpha;
    e_run *= alpha;
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] *= alpha;
  }
  const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
  __bf16 pb[NT][4];
  float psum = 0.f, esum = 0.f;
#pragma unroll
  for (int ut = 0; ut < NT; ++ut)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float e = exp2f(s[ut][i] - m_use);
      const __bf16 eb = static_cast<__bf16>(e);
      pb[ut][i] = eb;
      psum += static_cast<float>(eb);
      esum += e;
    }
  l_run += psum;
  e_run += esum;
  // ---- values: V^T runs past the shard's end are zeroed (weights there
  // are 0, but the bytes may hold anything, NaN included). Only the last
  // tile of a shard can hold such runs; the test is wave-uniform. ---------
  if (t0 + C::TOK > len) {
    const int keep = (len - (t0 + RUN * qd)) * EB;
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) B.v[nt] = keep_bytes(B.v[nt], keep);
  }
#pragma unroll
  for (int ksx = 0; ksx < C::KS; ++ksx) {
    const bf16x8_t pop = {pb[2 * ksx][0], pb[2 * ksx][1], pb[2 * ksx][2], pb[2 * ksx][3],
                          pb[2 * ksx + 1][0], pb[2 * ksx + 1][1], pb[2 * ksx + 1][2], pb[2 * ksx + 1][3]};
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) {
      bf16x8_t a;
      if constexpr (kFp8) {
        a = ksx ? fp8x8_to_bf16x8(B.v[nt][2], B.v[nt][3]) : fp8x8_to_bf16x8(B.v[nt][0], B.v[nt][1]);
      } else {
        a = __builtin_bit_cast(bf16x8_t, B.v[nt]);
      }
      o[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pop, o[nt], 0, 0, 0);
      if (nt & 1) __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// ---------------------------------------------------------------------------
// Main kernel: one persistent wavefront per worker.
// ---------------------------------------------------------------------------
// Waves per SIMD the register allocation must allow (measured best: two
// for fp8, whose tile work is heavier; one for bf16).
template <bool kFp8>
__global__ void __launch_bounds__(64 * kGqaWavesPerBlock)
    __attribute__((amdgpu_waves_per_eu(kFp8 ? 2 : 1))) gqa_attn_kernel(AttnParams p, int workers) {
  using C = GqaTile<kFp8>;
  constexpr int TOK = C::TOK;
  const int lane = threadIdx.x & 63;
  // wave-uniform (the compiler cannot tell on its own): keeps every unit and
  // tile quantity in scalar registers and the tile loop free of exec masks
  const int worker = __builtin_amdgcn_readfirstlane(blockIdx.x * kGqaWavesPerBlock + (threadIdx.x >> 6));
  const int n = lane & 15, qd = lane >> 4;
  const int G = p.group, rows = p.tpu * G;
  SplitWs ws = split_ws(p.workspace, workers, 0);
  __shared__ int64_t plan_lds[64 * kGqaWavesPerBlock + 16];
  const SplitStart st = split_locate<64 * kGqaWavesPerBlock>(p, C::TOK_LOG2, workers, worker, plan_lds);
  if (worker >= workers) return;  // (the grid's last workgroup may have spare wavefronts)
  const int64_t wstart = st.wstart, wend = st.wend;
  // the unit of the piece being computed and its tile range
  int64_t u = st.u, ubeg = st.ubeg, uend = st.uend;
  if (lane == 0 && worker == 0) {
    ws.total[0] = st.total;
    ws.total[1] = workers;  // one record per worker
  }
  if (wstart >= wend) {
    if (lane == 0) split_record(ws, worker, wstart, wend, -1, 0, 0);
    return;
  }

  const int bs = p.kv.block_size;
  const int64_t ks0 = p.kv.k_stride[0], ks1 = p.kv.k_stride[1], ks2 = p.kv.k_stride[2], ks3 = p.kv.k_stride[3];
  const int64_t vs0 = p.kv.v_stride[0], vs1 = p.kv.v_stride[1], vs2 = p.kv.v_stride[2], vs4 = p.kv.v_stride[4];
  constexpr int EB = kFp8 ? 1 : 2;
  const char* kbase = static_cast<const char*>(p.kv.k);
  const char* vbase = static_cast<const char*>(p.kv.v);

  int64_t tile = wstart;
  while (tile < wend) {
    while (uend <= tile) {  // uniform: on to the next unit with tiles
      ++u;
      ubeg = uend;
      uend = ubeg + unit_tiles(p, u, C::TOK_LOG2);
    }
    const int64_t t_lo = tile - ubeg, t_hi = min(wend, uend) - ubeg;  // unit-local tile range
    const UnitRef x = unit_ref(p, u);
    const int h = x.h, b = x.b, r = x.r;
    // column n = (query token x.i0 + n / G, head g = n % G); columns past the
    // unit's last query token have Q = 0 and the unit's length
    const int qi = x.i0 + n / G;
    const bool col = n < rows && qi < x.i1;
    int len = 0, min_len = 0x7fffffff;
    for (int i = x.i0; i < x.i1; ++i) {  // wave-uniform
      const int li = query_len(p, b, i, r);
      len = max(len, li);
      min_len = min(min_len, li);
    }
    const int col_len = col ? query_len(p, b, qi, r) : len;
    const int32_t* bt = p.block_table + static_cast<int64_t>(b) * p.bt_stride;
    const char* kh = kbase + (r * ks0 + h * ks2) * EB;
    const char* vh = vbase + (r * vs0 + h * vs2) * EB;
    const float kscale = kFp8 ? p.kv.k_scale[h] : 1.f;
    const float vscale = kFp8 ? p.kv.v_scale[h] : 1.f;
    const float c2 = p.softmax_scale * kscale * DCP_LOG2E;

    // Q^T operand for the 4 k-steps over the 128 dims (zero for unused columns).
    bf16x8_t qop[4];
    {
      const uint16_t* qrow = reinterpret_cast<const uint16_t*>(p.q) +
                             ((static_cast<int64_t>(b) * p.q_len + qi) * p.num_q_heads + h * G + n % G) * kGqaDim;
      const uint16_t* qsrc = col ? qrow : reinterpret_cast<const uint16_t*>(p.q);  // in bounds, then zeroed
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int d0 = kFp8 ? (64 * (k >> 1) + 16 * qd + 8 * (k & 1)) : (32 * k + 8 * qd);
        u32x4_t raw = ldg16(qsrc + d0);
        if (!col) raw = u32x4_t{0u, 0u, 0u, 0u};
        qop[k] = __builtin_bit_cast(bf16x8_t, raw);
      }
    }

    f32x4_t o[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    // l_run sums the bf16-rounded weights that enter the value product (so O
    // is an exact convex combination of the values); e_run sums the fp32
    // weights and gives the LSE.
    float m_run = -INFINITY, l_run = 0.f, e_run = 0.f;

    // Two tiles per iteration: the loads of both (32 KB per wave) are issued
    // before either is consumed, and the block ids of the next pair are
    // fetched meanwhile, so a wave never waits on a block-table read. Inside
    // the loop the loads are unconditional (a branch around them makes the
    // compiler's wait counts assume they may be missing, so consuming the
    // first tile would also wait for the second): rows past the shard's end
    // read the tile's first chunk instead and are masked afterwards. An odd
    // tile count leaves the piece's last tile to a step of its own after the
    // loop rather than loading it twice as the two tiles of a pair (1.0% of
    // the fp8 kernel's time and 1.8% of the bf16 one's, timed in one process
    // on one pool against the loop that re-read it).
    // (tile indices inside one unit fit in 32 bits: a shard holds < 2^31 tokens)
    const int tb = static_cast<int>(t_lo), te = static_cast<int>(t_hi), t_last = te - 1;
    GqaIds ids_a = gqa_load_ids<kFp8>(bt, tb, len, bs, n, qd);
    GqaIds ids_b = gqa_load_ids<kFp8>(bt, min(tb + 1, t_last), len, bs, n, qd);
    GqaBuf<kFp8> buf_a, buf_b;
    int t = tb;
    for (; t + 1 < te; t += 2) {
      gqa_issue<kFp8>(buf_a, ids_a, t, len, bs, kh, ks1, ks3, vh, vs1, vs4, n, qd);
      gqa_issue<kFp8>(buf_b, ids_b, t + 1, len, bs, kh, ks1, ks3, vh, vs1, vs4, n, qd);
      ids_a = gqa_load_ids<kFp8>(bt, min(t + 2, t_last), len, bs, n, qd);
      ids_b = gqa_load_ids<kFp8>(bt, min(t + 3, t_last), len, bs, n, qd);
      gqa_tile<kFp8>(buf_a, t * TOK, len, col_len, min_len, c2, qop, o, m_run, l_run, e_run, qd);
      gqa_tile<kFp8>(buf_b, (t + 1) * TOK, len, col_len, min_len, c2, qop, o, m_run, l_run, e_run, qd);
    }
    if (t < te) {  // uniform: an odd tile count leaves the last tile alone
      gqa_issue<kFp8>(buf_a, ids_a, t, len, bs, kh, ks1, ks3, vh, vs1, vs4, n, qd);
      gqa_tile<kFp8>(buf_a, t * TOK, len, col_len, min_len, c2, qop, o, m_run, l_run, e_run, qd);
    }

    // ---- piece end: full unit -> final output, else partial --------------
    float l_tot = l_run + __shfl_xor(l_run, 16, 64);
    l_tot += __shfl_xor(l_tot, 32, 64);
    float e_tot = e_run + __shfl_xor(e_run, 16, 64);
    e_tot += __shfl_xor(e_tot, 32, 64);
    const bool whole = (t_lo == 0) && (t_hi == uend - ubeg);
    if (whole) {
      const float inv = l_tot > 0.f ? vscale / l_tot : 0.f;  // l_tot = 0: the column sees no token (O = 0)
      if (col) {
        const int64_t row = out_row(p, x, qi, n % G);
        float* dst = p.out_o + row * kGqaDim;
#pragma unroll
        for (int nt = 0; nt < 8; ++nt) {
          f32x4_t v = o[nt] * inv;
          *reinterpret_cast<f32x4_t*>(dst + 16 * nt + 4 * qd) = v;
        }
        if (qd == 0) p.out_lse[row] = (m_run + __log2f(e_tot)) * DCP_LN2;
      }
    } else {
      const int which = (t_lo == 0) ? 1 : 0;  // 0: unit began before this worker
      float* dst = ws.part + ((static_cast<int64_t>(worker) * 2 + which) * rows) * (kGqaDim + kPartExtra);
      if (n < rows) {
        float* hrow = dst + static_cast<int64_t>(n) * (kGqaDim + kPartExtra);
#pragma unroll
        for (int nt = 0; nt < 8; ++nt) {
          f32x4_t v = o[nt] * vscale;
          *reinterpret_cast<f32x4_t*>(hrow + 16 * nt + 4 * qd) = v;
        }
        if (qd == 0) {
          hrow[kGqaDim] = m_run;
          hrow[kGqaDim + 1] = l_tot;
          hrow[kGqaDim + 2] = e_tot;
        }
      }
    }
    tile = ubeg + t_hi;
  }
  if (lane == 0) split_record(ws, worker, wstart, wend, u, ubeg, uend);
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
bool gqa_supported(const AttnParams& p) {
  const dcp_kv_cache_t& kv = p.kv;
  if (p.q_dtype != DCP_BF16) return false;
  if (kv.dtype != DCP_BF16 && kv.dtype != DCP_FP8_E4M3) return false;
  if (kv.head_dim_k != kGqaDim || kv.head_dim_v != kGqaDim || !kv.v) return false;
  if (p.tpu * p.group > 16) return false;  // (query token, head) columns of the 16-wide MFMA tile
  if (kv.block_size % 16 != 0) return false;
  if (kv.k_stride[4] != 1 || kv.v_stride[3] != 1) return false;
  const int eb = kv.dtype == DCP_BF16 ? 2 : 1;
  // 16-byte alignment of every row / run the kernel loads
  for (int i = 0; i < 4; ++i)
    if ((kv.k_stride[i] * eb) % 16 != 0) return false;
  for (int i : {0, 1, 2, 4})
    if ((kv.v_stride[i] * eb) % 16 != 0) return false;
  if (reinterpret_cast<uintptr_t>(kv.k) % 16 || reinterpret_cast<uintptr_t>(kv.v) % 16) return false;
  return true;
}

// Persistent wavefronts the device holds at once, cached per device (static
// storage starts zeroed; concurrent first calls store the same value).
template <bool kFp8>
static int gqa_workers() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) dev = 0;
  if (dev < 64 && cached[dev].load() > 0) return cached[dev].load();
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, gqa_attn_kernel<kFp8>, 64 * kGqaWavesPerBlock, 0) !=
          hipSuccess || per_cu < 1)
    per_cu = 2;
  const int c = min(kGqaMaxWorkers, device_cu_count() * per_cu * kGqaWavesPerBlock);
  if (dev < 64) cached[dev].store(c);
  return c;
}

// Sized for the workers this device runs (split pieces: two per worker).
size_t gqa_workspace_bytes(const AttnParams& p) {
  const int workers = p.kv.dtype == DCP_FP8_E4M3 ? gqa_workers<true>() : gqa_workers<false>();
  return split_ws_bytes(workers, 0, p.tpu * p.group, kGqaDim);
}

hipError_t launch_gqa_attn(const AttnParams& p) {
  const bool fp8 = p.kv.dtype == DCP_FP8_E4M3;
  const int workers = fp8 ? gqa_workers<true>() : gqa_workers<false>();
  const int tok = fp8 ? GqaTile<true>::TOK : GqaTile<false>::TOK;
  const dim3 grid((workers + kGqaWavesPerBlock - 1) / kGqaWavesPerBlock);
  if (p.ev_begin) (void)hipEventRecord(p.ev_begin, p.stream);
  if (fp8)
    hipLaunchKernelGGL(gqa_attn_kernel<true>, grid, dim3(64 * kGqaWavesPerBlock), 0, p.stream, p, workers);
  else
    hipLaunchKernelGGL(gqa_attn_kernel<false>, grid, dim3(64 * kGqaWavesPerBlock), 0, p.stream, p, workers);
  if (p.ev_end) (void)hipEventRecord(p.ev_end, p.stream);
  launch_split_combine<kGqaDim>(p, tok, workers, 0);
  return hipGetLastError();
}

}  // namespace dcp
