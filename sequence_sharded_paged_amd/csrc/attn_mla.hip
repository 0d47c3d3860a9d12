// MLA per-rank partial decode attention on MFMA: 128 query heads sharing one
// bf16 latent KV row of 576 (512 latent + 64 rope); the value is the first
// 512 entries of the same row.
//
// Source: "Efficient Decode Context Parallelism with vLLM for Long Context
// Workloads", section 1 (MLA keeps one low-rank latent vector per token,
// shared by all query heads: effectively one KV head); "Decode Context
// Parallel (DCP)" (vLLM Ascend design doc), section "Decode" (attention
// against the local KV shard, partial output and LSE out).
//
// At 128 heads a token costs 2 x 128 x (576 + 512) flops for 1152 bytes, so
// at the HBM rate this kernel needs most of the chip's bf16 MFMA rate: the
// design goal is to keep the matrix cores busy, and everything else (LDS
// operand reads, softmax, address arithmetic) runs in their shadow.
//
// Work split: stream-K over (rank, request, query token) units (splitkv.h;
// one query token per unit when several are decoded at once), one persistent
// 256-thread workgroup (one wavefront per SIMD) per worker, tiles of 32
// tokens. Per workgroup:
//   * a 4-stage LDS ring of 32-token tiles (36 KB each) is filled straight
//     from HBM with global_load_lds_dwordx4 (each wavefront loads 8 of the 32
//     rows); the 16-byte chunks of a row are XOR-swizzled by the row index so
//     that the MFMA operand reads spread over the LDS banks. At any time two
//     stages are read (scores of tile t, values of tile t - 1) and two are in
//     flight (the refill with tile t + 2 goes out during step t);
//   * scores: wavefront w owns query heads 32 w .. 32 w + 31, whose Q (32 x
//     576 bf16, 144 VGPRs) stays in registers for the whole piece;
//     S^T[token, head] = K[token, :] . Q[head, :] on 32x32x16 bf16 MFMA, K
//     rows read from LDS with ds_read_b128;
//   * softmax weights in log2 units relative to a per-piece reference max
//     (the first tile's): no rescaling of the accumulator and no cross-lane
//     reduction inside the loop; a piece whose scores outgrow the reference
//     by more than 2^64 is replayed with a higher reference. The weights are
//     rounded to bf16 for the value product and their sum (the normaliser) is
//     taken over the same rounded values, with an fp32 sum of the unrounded
//     weights for the LSE (as in the GQA kernel);
//   * values: the weights of all 128 heads go through an 8 KB LDS buffer, and
//     wavefront w owns latent dims 128 w .. 128 w + 127 of every head:
//     O^T[dim, head] += V^T[dim, token] . P^T[token, head], its O (128 x 128
//     fp32, 256 AGPRs) in registers for the whole piece. V^T comes from the
//     tile's LDS rows through ds_read_b64_tr_b16, whose 16-lane transpose
//     hands each lane four consecutive tokens of one dimension. Splitting the
//     value product by dimension rather than by head means each wavefront
//     reads a quarter of the V tile: the transposing reads move half the bytes
//     per instruction of ds_read_b128, and when every wavefront read the whole
//     V tile they were the largest LDS cost of the kernel;
//   * software pipeline across tiles: step t runs the score MFMAs of tile t,
//     then the value MFMAs of tile t - 1 with the softmax of tile t
//     interleaved (two weights per value step), then stores tile t's weights;
//     one barrier per step publishes them and the refill that landed.
#include <utility>

#include "splitkv.h"

namespace dcp {

constexpr int kMlaDk = 576;
constexpr int kMlaDv = 512;
constexpr int kMlaHeads = 128;
constexpr int kMlaTile = 32;                                     // tokens per tile
constexpr int kMlaStages = 4;                                    // LDS ring depth
constexpr int kMlaRowBytes = kMlaDk * 2;                         // 1152
constexpr int kMlaStageBytes = kMlaTile * kMlaRowBytes;          // 36864
constexpr int kMlaLatBytes = kMlaDv * 2;                         // 1024: latent part of a row (also V)
constexpr int kMlaRopeOff = kMlaTile * kMlaLatBytes;             // 32768: rope rows follow the latent rows
constexpr int kMlaRopeBytes = kMlaRowBytes - kMlaLatBytes;       // 128
constexpr int kMlaWaves = 4;                                     // wavefronts per workgroup
constexpr int kMlaThreads = 64 * kMlaWaves;
constexpr int kMlaHeadsPerWave = kMlaHeads / kMlaWaves;          // 32: the N side of the MFMAs
constexpr int kMlaRowsPerWave = kMlaTile / kMlaWaves;            // 8 rows of a tile loaded per wavefront
constexpr int kMlaDmaPerTile = kMlaRowsPerWave + 1;              // DMA instructions per wavefront and tile
constexpr int kMlaKSteps = kMlaDk / 16;                          // 36 score k-steps of 16 dims
constexpr int kMlaKStepsLat = kMlaDv / 16;                       // 32 latent k-steps (Q in VGPRs)
constexpr int kMlaDvTiles = kMlaDv / 32 / kMlaWaves;             // 4 value M-tiles of 32 dims per wave
constexpr int kMlaHeadTiles = kMlaHeads / 32;                    // 4 value N-tiles of 32 heads
constexpr int kMlaValSteps = 2 * kMlaDvTiles;                    // (token step, M-tile) pairs per tile
constexpr int kMlaPBytes = kMlaTile * kMlaHeads * 2;             // 8 KB of bf16 weights per tile
#ifndef DCP_MLA_KPF
#define DCP_MLA_KPF 4
#endif
#ifndef DCP_MLA_VPF
#define DCP_MLA_VPF 2
#endif
constexpr int kMlaKPf = DCP_MLA_KPF;  // score-operand read distance (k-steps)
constexpr int kMlaVPf = DCP_MLA_VPF;  // value-operand read distance (value steps)
constexpr int kMlaMaxWorkers = 512;
constexpr float kMlaRefSlack = 64.f;  // log2 units a score may exceed the piece's reference

static_assert(kMlaStages == 4, "the refill distance below assumes 4 stages");
static_assert(kMlaKStepsLat == 32 && kMlaKSteps - kMlaKStepsLat == 4, "32 latent + 4 rope k-steps");

typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

// f(std::integral_constant<int, I>{}) for I = 0 .. N-1, in order
template <typename F, int... I>
__device__ __forceinline__ void static_for_seq(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_seq(f, std::make_integer_sequence<int, N>{});
}
typedef float f32x16_t __attribute__((ext_vector_type(16)));

// Uniform read-only load through the constant address space (scalar load).
template <typename T>
__device__ __forceinline__ T ld_uniform(const T* p) {
  return *(const __attribute__((address_space(4))) T*)(p);
}

// s_waitcnt vmcnt(N) with expcnt / lgkmcnt left alone (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// 16 bytes per lane from `src` into LDS at lds_base + 16 * lane (the wave's
// M0 base). Issued through asm so that the compiler, which cannot tell the
// ring stages apart, does not make every later LDS read wait for it; the
// kernel orders these writes itself (vmcnt wait + barrier before a stage is
// read, barrier before it is refilled).
__device__ __forceinline__ void dma16(const void* src, uint32_t lds_base) {
  // one wait state between the M0 write and the LDS DMA that reads it
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(lds_base)
               : "memory", "m0");
}

// Same, from a wave-uniform base plus a 32-bit per-lane byte offset.
// (The base and M0 values are wave-uniform by construction; readfirstlane
// pins them to SGPRs where the compiler cannot prove it.) The asm only moves
// into M0: any SALU arithmetic here would overwrite SCC, which the compiler
// may hold live across the statement.
__device__ __forceinline__ void dma16_s(uint32_t voff, const void* sbase, uint32_t lds_base) {
  // (readfirstlane yields a signed int: each half is taken as uint32_t before
  // widening, or a low word with bit 31 set would smear into the high word)
  const uint64_t b = reinterpret_cast<uint64_t>(sbase);
  const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(b)));
  const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(b >> 32)));
  const uint64_t bu = static_cast<uint64_t>(lo) | (static_cast<uint64_t>(hi) << 32);
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff),
               "s"(reinterpret_cast<const void*>(bu)), "s"(__builtin_amdgcn_readfirstlane(lds_base))
               : "memory", "m0");
}

// Workgroup barrier without the memory fence of __syncthreads (which would
// wait for every tile in flight); the asm memory clobber keeps the compiler
// from moving LDS accesses across it.
__device__ __forceinline__ void block_sync() { asm volatile("s_barrier" ::: "memory"); }

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) char*)p));
}


// s_waitcnt lgkmcnt(0) with vmcnt / expcnt left alone.
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xc07f); }

// bf16 pair (round to nearest even) packed in one dword, low half first.
__device__ __forceinline__ bf16x2_t pack_bf16(float lo, float hi) {
  return bf16x2_t{static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
}

// LDS tile layout, in MFMA operand order. The tile's 32 rows x 72 chunks of
// 16 bytes form 36 blocks of 1 KB, block 2 ks + u holding chunks 4 ks .. 4 ks
// + 3 of rows 16 u .. 16 u + 15 (the score operand of k-step ks for token
// half u): chunk 4 ks + c of row 16 u + r sits at 16 (16 c + (r ^ 4 c)) in
// its block. A score-operand read (lane 16 c + r) is then one contiguous
// 1 KB block, and a transpose read of the value operand (4 rows x 2 chunks
// per 16 lanes) touches two 64-byte runs in different bank halves.
__device__ __forceinline__ int mla_slot(int r, int c) { return 16 * c + (r ^ (4 * c)); }

__global__ void __attribute__((amdgpu_flat_work_group_size(kMlaThreads, kMlaThreads), amdgpu_waves_per_eu(1, 1)))
mla_attn_kernel(AttnParams p, int workers) {
  __shared__ __attribute__((aligned(16))) char lds[kMlaStages * kMlaStageBytes];
  // bf16 weights of tile t in buffer t % 2, in value-operand order: the 1 KB
  // block 2 nt + kk holds, at 16 l, head 32 nt + l % 32, tokens 16 kk + 8 (l /
  // 32) .. +7 (lane l's part of the B operand of N-tile nt, token step kk).
  // Wave w writes blocks 2 w, 2 w + 1 (its own heads).
  __shared__ __attribute__((aligned(16))) char pbuf[2 * kMlaPBytes];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (SGPR)
  const int n = lane & 15, g = lane >> 4;
  const int worker = blockIdx.x;
  const int64_t U = split_units(p);
  SplitWs ws = split_ws(p.workspace, U, workers);
  const int64_t T = ld_uniform(ws.prefix + U);
  if (T == 0 || worker >= workers) return;
  const int64_t tpw = (T + workers - 1) / workers;
  const int64_t wstart = static_cast<int64_t>(worker) * tpw;
  if (wstart >= T) return;
  const int64_t wend = min(T, wstart + tpw);

  const int bs = p.kv.block_size;
  const int64_t ks0 = p.kv.k_stride[0], ks1 = p.kv.k_stride[1], ks3 = p.kv.k_stride[3];
  const int row_bytes = static_cast<int>(ks3 * 2);  // bytes between consecutive tokens of a block
  const char* kbase = static_cast<const char*>(p.kv.k);
  // The kernel masks a shard's tail tokens with -inf scores before scaling,
  // which needs a positive scale: a negative one is carried by Q's sign bits
  // (s c2 = (-s) (-c2), exact in bf16), a zero one by a zeroed Q and scale 1
  // (every weight is then exp2(0 - m_ref), as with scale 0).
  const float c2_in = p.softmax_scale * DCP_LOG2E;
  const float c2 = c2_in > 0.f ? c2_in : (c2_in < 0.f ? -c2_in : 1.f);
  const uint32_t q_keep = c2_in == 0.f ? 0u : 0xFFFFFFFFu, q_flip = c2_in < 0.f ? 0x80008000u : 0u;
  const uint32_t lds0 = lds_addr(lds);
  auto stage_of = [&](int64_t t) __attribute__((always_inline)) {
    return static_cast<int>((t - wstart) & (kMlaStages - 1));
  };

  // ---- tile sources -----------------------------------------------------------
  // A walker over the worker's tiles in order, yielding this wave's refill
  // (its 16-token half of the tile: tokens t0 + 16 (w % 2) .. +15, which share
  // one block, block_size % 16 == 0). Per unit it caches the length,
  // block-table row and rank base; per tile it advances the (virtual block,
  // offset) of the tile's first token. Rows past the shard's end are replaced
  // by the last valid row of the half, or of the first half if the second has
  // none (finite data, zero weight).
  //
  // Block-table entries come from a window of 64 consecutive entries of the
  // unit's row, one per lane of a VGPR, read with v_readlane: a scalar load
  // per block would stall the loop for a cache miss (the KV stream keeps the
  // table out of the caches) and, sharing a counter with the LDS reads, drain
  // them; the window is reloaded once per 64 blocks. Tile indices are kept
  // relative to the worker's first tile, in 32 bits, and the per-tile work
  // is a few scalar instructions: with one wavefront per SIMD every
  // instruction of the loop costs an issue slot.
  const int my_half = wave & 1;
  const int dma_row = n ^ (4 * g);
  const uint32_t blk_bytes = static_cast<uint32_t>(ks1 * 2);  // < 2^32 (checked on the host)
  const uint32_t voff_full = static_cast<uint32_t>(dma_row * row_bytes + 16 * g + 64 * (wave >> 1));
  const uint32_t m0_wave = lds0 + wave * 1024;
  struct Walker {
    int t;     // next tile, relative to wstart
    int u;     // its unit
    int uend;  // end of unit u, relative to wstart (clamped to the int range)
    int tok;   // first token of tile t within the unit's shard
    int len;
    int hvb, hoff;     // block and offset of token tok + 16 (w % 2), this wave's half
    bool dirty;        // hbase must be recomputed (new unit or new block)
    const char* hbase; // address of that token's row
    int win, win_lo;   // entries win_lo + lane of the row (win_lo < 0: no window)
    const int32_t* bt;
    const char* rk;
  };
  struct Refill {
    const char* base;  // this wave's token half
    uint32_t voff;     // lane offset of k-step w / 2
    uint32_t m0;       // LDS address of block w of the stage
  };
  auto rel_end = [&](int64_t e) __attribute__((always_inline)) {
    return static_cast<int>(min(e - wstart, static_cast<int64_t>(INT32_MAX)));
  };
  // (re)enter unit w.u at tile w.t, the unit starting at tile ubeg (absolute)
  auto set_unit = [&](Walker& w, int64_t ubeg) __attribute__((always_inline)) {
    // unit u = (r * batch + b) * q_len + i: rank r, request b, query token i
    const int rb = w.u / p.q_len, i = w.u - rb * p.q_len;
    const int b = rb % p.batch, r = rb / p.batch;
    w.len = ld_uniform(p.local_lens + (static_cast<int64_t>(b) * p.q_len + i) * p.dcp_size + p.rank_begin + r);
    w.bt = p.block_table + static_cast<int64_t>(b) * p.bt_stride;
    w.rk = kbase + r * ks0 * 2;
    w.tok = static_cast<int>(wstart + w.t - ubeg) * kMlaTile;
    const int ht = w.tok + 16 * my_half;
    w.hvb = ht / bs;
    w.hoff = ht - w.hvb * bs;
    w.dirty = true;
    w.win_lo = -1;
  };
  // a walker at tile t, searching forward from unit u (at or before t's unit)
  auto walker_at = [&](int64_t t, int64_t u) __attribute__((always_inline)) {
    Walker w;
    int64_t ubeg = ld_uniform(ws.prefix + u), uend = ld_uniform(ws.prefix + u + 1);
    while (uend <= t) {  // uniform
      ++u;
      ubeg = uend;
      uend = ld_uniform(ws.prefix + u + 1);
    }
    w.t = static_cast<int>(t - wstart);
    w.u = static_cast<int>(u);
    w.uend = rel_end(uend);
    w.win = 0;
    w.hbase = kbase;
    set_unit(w, ubeg);
    return w;
  };
  // block-table entry vb (< max_vblocks) of the walker's row
  auto entry = [&](Walker& w, int vb) __attribute__((always_inline)) {
    if (w.win_lo < 0 || vb < w.win_lo || vb >= w.win_lo + 64) {  // uniform
      w.win_lo = vb;
      w.win = vb + lane < p.max_vblocks ? w.bt[vb + lane] : 0;
      // wait here, on the reload path only (the compiler does not see the ring's
      // DMAs and would otherwise put a full wait where the paths join)
      wait_vmcnt<0>();
    }
    return __builtin_amdgcn_readlane(w.win, vb - w.win_lo);
  };
  auto row_at = [&](Walker& w, int vb, int off) __attribute__((always_inline)) {
    const uint32_t blk = static_cast<uint32_t>(entry(w, vb));
    return w.rk + static_cast<uint64_t>(blk) * blk_bytes + static_cast<uint32_t>(off * row_bytes);
  };
  // The refill of the DMA walker's next tile (stage t % 4); advances it. The
  // common case (same unit, same block, a whole half) adds 32 rows to the
  // half's address.
  Walker dw;
  auto prepare = [&]() __attribute__((always_inline)) {
    Walker& w = dw;
    if (w.t >= w.uend) {  // uniform, rare: the tile opens the next non-empty unit
      int64_t ubeg = wstart + w.uend, uend;
      for (;;) {
        ++w.u;
        uend = ld_uniform(ws.prefix + w.u + 1);
        if (uend > ubeg) break;
      }
      w.uend = rel_end(uend);
      set_unit(w, ubeg);
    }
    if (w.dirty) {  // uniform
      w.hbase = row_at(w, w.hvb, w.hoff);
      w.dirty = false;
    }
    Refill r;
    r.base = w.hbase;
    r.voff = voff_full;
    r.m0 = m0_wave + (w.t & (kMlaStages - 1)) * kMlaStageBytes;
    const int nv = w.len - w.tok - 16 * my_half;  // valid rows of the half (if < 16)
    if (nv < 16) {  // uniform, rare: the unit's last tile
      int rows = nv;
      if (nv <= 0) {  // no second half: take the first half's rows
        rows = min(16, w.len - w.tok);
        const int fvb = w.tok / bs;
        r.base = row_at(w, fvb, w.tok - fvb * bs);
      }
      r.voff = static_cast<uint32_t>(min(dma_row, rows - 1) * row_bytes + 16 * g + 64 * (wave >> 1));
    }
    ++w.t;
    w.tok += kMlaTile;
    w.hoff += kMlaTile;
    if (w.hoff < bs) {  // uniform
      w.hbase += kMlaTile * row_bytes;
    } else {
      do {  // once, or twice when block_size is 16
        w.hoff -= bs;
        ++w.hvb;
      } while (w.hoff >= bs);
      w.dirty = true;
    }
    return r;
  };

  // ---- DMA producer -------------------------------------------------------------
  // Wave w loads blocks w, w+4, .., w+32 of each tile: token half w % 2,
  // k-steps w / 2 + 2 k (k = 0 .. 8); DMA lane 16 c + m fetches row m ^ 4 c of
  // the half, chunk 4 ks + c. A refill (one wave's share of a tile) is
  // prepared at the end of a step and its 9 DMAs are spread over the k-steps
  // of the next score phase.
  // DMA k (0 .. 8) of this wave for the refill r: k-step w / 2 + 2 k, block w + 4 k
  auto dma = [&](const Refill& r, auto kc) __attribute__((always_inline)) {
    constexpr int k = decltype(kc)::value;
    dma16_s(r.voff + 128 * k, r.base, r.m0 + 4096 * k);
  };
  auto dma_all = [&](const Refill& r) __attribute__((always_inline)) {
    static_for<kMlaDmaPerTile>([&](auto kc) __attribute__((always_inline)) { dma(r, kc); });
  };
  // Every tile step issues exactly one refill (9 DMAs per wave): once the
  // worker's tiles run out, the last real refill is issued again (it rewrites
  // a stage with the data it already holds), so every wait count below is a
  // constant and no branch guards a DMA. The kernel drains them before exit.
  Refill next_refill;  // the refill prepared during the current tile
  Refill pending;      // the refill the next score phase issues

  // Ring schedule: step t reads stage t % 4 (scores of tile t) and stage
  // (t - 1) % 4 (values of tile t - 1), and its score phase issues the refill
  // with tile t + 2 into stage (t + 2) % 4, whose last reader (the values of
  // tile t - 2) finished before the barrier that ended step t - 1. So two
  // stages are read and two are in flight at any time.
  //
  // (Re)start the ring at tile t (unit u): load tiles t and t + 1, prepare the
  // refill with tile t + 2 and wait until tile t has landed everywhere.
  auto restart = [&](int64_t t, int64_t u) __attribute__((always_inline)) {
    dw = walker_at(t, u);
    for (int j = 0; j < 2; ++j) {
      if (t + j < wend) next_refill = prepare();  // uniform
      dma_all(next_refill);
    }
    // past the worker's last tile the step re-issues the last real refill:
    // same data into the same stage (it only makes later waits more
    // conservative)
    if (t + 2 < wend) next_refill = prepare();  // uniform
    pending = next_refill;
    wait_vmcnt<kMlaDmaPerTile>();
    block_sync();
  };
  // End of step t (every read of stages t, t - 1 and of the weights issued):
  // prepare the refill with tile t + 3, which becomes pending (issued by step
  // t + 1), and wait until tile t + 1 has landed. The refill issued by this
  // step (tile t + 2) is the only one allowed to stay in flight. The walker
  // runs here rather than among the value MFMAs: issued as one block there it
  // starves the matrix core, and here its rare scalar loads (a unit change)
  // find no LDS read in flight.
  auto end_tile = [&](int64_t t) __attribute__((always_inline)) {
    wait_lgkm0();
    if (t + 3 < wend) next_refill = prepare();  // uniform
    pending = next_refill;
    wait_vmcnt<kMlaDmaPerTile>();
    block_sync();
  };
  // DMA j of the pending refill, issued after k-step 4 j of a score phase (a
  // burst of all nine at once lands as one block of LDS writes that stalls the
  // score operand reads)
  auto pending_dma = [&](auto ksc) __attribute__((always_inline)) {
    constexpr int ks = decltype(ksc)::value;
    if constexpr ((ks & 3) == 0 && ks / 4 < kMlaDmaPerTile) dma(pending, std::integral_constant<int, ks / 4>{});
  };

  // ---- per-lane LDS operand offsets ------------------------------------------
  // Lane l = 32 h + c32 (h = l / 32), and in 16-lane groups l = 16 G + 4 i + j.
  // Score operand (A of v_mfma_f32_32x32x16_bf16) of k-step ks (dims 16 ks
  // .. +15): token row c32, dims 16 ks + 8 h .. +7, i.e. 32-dim block ks / 2,
  // token half c32 / 16, chunk 2 (ks % 2) + h of row c32 % 16:
  //   koff[ks % 2] + 2048 (ks / 2)
  int koff[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) koff[q] = ((lane >> 4) & 1) * 1024 + 16 * mla_slot(lane & 15, 2 * q + (lane >> 5));
  // Value operand (A) of M-tile mt (dims 32 mt .. +31) and token step kk
  // (tokens 16 kk .. +15), through two transpose reads rd = 0, 1: the lane
  // addresses token 8 (G / 2) + 4 rd + i of half kk and dims 32 mt + 16 (G % 2)
  // + 4 j .. +3, i.e. chunk 2 (G % 2) + j / 2, byte 8 (j % 2):
  //   voff[rd] + 2048 mt + 1024 kk
  // and receives dim 32 mt + l % 32, tokens 8 h + 4 rd .. +3 of the step.
  int voff[2];
#pragma unroll
  for (int rd = 0; rd < 2; ++rd) {
    const int G = lane >> 4, i = (lane & 15) >> 2, j = lane & 3;
    voff[rd] = 16 * mla_slot(8 * (G >> 1) + 4 * rd + i, 2 * (G & 1) + (j >> 1)) + 8 * (j & 1);
  }

  restart(wstart, ld_uniform(ws.wunit + worker));

  int64_t cur_u = ld_uniform(ws.wunit + worker);  // unit of the tile being computed
  int64_t tile = wstart;
  float m_hint = -INFINITY;  // reference for a replayed piece (this lane's head)
  bool replay = false;       // the current piece is a replay (at most one per piece)
  const int h = lane >> 5;   // token quarter-row group of the score layout, k-half of the operands

  while (tile < wend) {
    while (ld_uniform(ws.prefix + cur_u + 1) <= tile) ++cur_u;
    const int64_t ubeg = ld_uniform(ws.prefix + cur_u), uend = ld_uniform(ws.prefix + cur_u + 1);
    const int64_t lt_lo = tile - ubeg, lt_hi = min(wend, uend) - ubeg;
    const int64_t rb = cur_u / p.q_len;
    const int qi = static_cast<int>(cur_u - rb * p.q_len);
    const int b = static_cast<int>(rb % p.batch);
    const int len = ld_uniform(p.local_lens + (static_cast<int64_t>(b) * p.q_len + qi) * p.dcp_size + p.rank_begin +
                               static_cast<int>(rb / p.batch));
    const int64_t piece_tile0 = tile, piece_end = tile + (lt_hi - lt_lo);

    // Q operand (B of the score MFMA): head 32 wave + l % 32, dims 16 ks + 8 h
    // .. +7, all 36 k-steps in VGPRs
    bf16x8_t qop[kMlaKSteps];
    {
      const uint16_t* qb = reinterpret_cast<const uint16_t*>(p.q) +
                           ((static_cast<int64_t>(b) * p.q_len + qi) * kMlaHeads + kMlaHeadsPerWave * wave +
                            (lane & 31)) * kMlaDk + 8 * h;
#pragma unroll
      for (int ks = 0; ks < kMlaKSteps; ++ks) qop[ks] = *reinterpret_cast<const bf16x8_t*>(qb + 16 * ks);
      if (!(c2_in > 0.f)) {  // uniform
#pragma unroll
        for (int ks = 0; ks < kMlaKSteps; ++ks) {
          u32x4_t w = __builtin_bit_cast(u32x4_t, qop[ks]);
#pragma unroll
          for (int j = 0; j < 4; ++j) w[j] = (w[j] & q_keep) ^ q_flip;
          qop[ks] = __builtin_bit_cast(bf16x8_t, w);
        }
      }
    }
    // Q is complete here, so no wait for it lands inside the tile loop (where
    // it would also drain the tiles in flight).
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_sched_barrier(0);

    // ---- piece state ------------------------------------------------------------
    // Weights are exp2(s c2 - m_ref) with m_ref fixed for the piece (the first
    // tile's max unless a replay hands one in); mx tracks the largest exponent
    // seen, for the replay vote and the next reference. O^T[dim, head] of
    // M-tile mt, N-tile nt (o[4 mt + nt]): lane l holds head 32 nt + l % 32,
    // dims 128 wave + 32 mt + 8 (r / 4) + 4 h + r % 4.
    float m_ref = m_hint, mx = -INFINITY, lsum = 0.f, esum = 0.f;
    f32x16_t o[kMlaDvTiles * kMlaHeadTiles];
#pragma unroll
    for (int i = 0; i < kMlaDvTiles * kMlaHeadTiles; ++i) o[i] = f32x16_t{};
    bool need_ref = !replay;  // uniform

    // ---- score MFMAs of one tile: S^T[token, head], lane l holding head l % 32,
    // tokens 8 (r / 4) + 4 h + r % 4 of register r; each k-step's MFMA depends
    // on the one before it; the pending refill goes out between them --------------
    auto scores = [&](const char* st, f32x16_t& s, auto&& tail) __attribute__((always_inline)) {
      s = f32x16_t{};
      bf16x8_t ka[kMlaKPf + 1];
      auto kread = [&](int ks) __attribute__((always_inline)) {
        ka[ks % (kMlaKPf + 1)] = *reinterpret_cast<const bf16x8_t*>(st + koff[ks & 1] + 2048 * (ks >> 1));
      };
#pragma unroll
      for (int j = 0; j < kMlaKPf; ++j) kread(j);
      static_for<kMlaKSteps>([&](auto ksc) __attribute__((always_inline)) {
        constexpr int ks = decltype(ksc)::value;
        if constexpr (ks + kMlaKPf < kMlaKSteps) kread(ks + kMlaKPf);
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[ks % (kMlaKPf + 1)], qop[ks], s, 0, 0, 0);
        pending_dma(ksc);
        // the value phase's first operand reads go out once the K ring stops
        // refilling, so that their latency hides behind the last score MFMAs
        if constexpr (ks == kMlaKSteps - kMlaKPf) tail();
        __builtin_amdgcn_sched_barrier(0);
      });
    };

    // ---- softmax of one tile: weight r (0 .. 15) of this lane; pw[d] packs
    // weights 2 d, 2 d + 1 (tokens 8 (d / 2) + 4 h + 2 (d % 2) + {0, 1})
    f32x16_t s_cur;
    uint32_t pw[8];
    float pe_lo = 0.f;
    auto weight = [&](int r) __attribute__((always_inline)) {
      if (r >= 16) return;
      const float x = fmaf(s_cur[r], c2, -m_ref);
      mx = fmaxf(mx, x);
      const float pe = __builtin_amdgcn_exp2f(x);  // v_exp_f32; results below 2^-126 flush to 0
      esum += pe;
      if (r & 1) {
        const bf16x2_t pk = pack_bf16(pe_lo, pe);
        pw[r >> 1] = __builtin_bit_cast(uint32_t, pk);
        lsum = __builtin_amdgcn_fdot2_f32_bf16(pk, bf16x2_t{__bf16(1.f), __bf16(1.f)}, lsum, false);
      } else {
        pe_lo = pe;
      }
    };

    // ---- weights to LDS -------------------------------------------------------------
    // B operand of token step kk: lane l needs head l % 32, tokens 16 kk + 8 h ..
    // +7. A lane holds tokens 4 h + {0..3} + 8 q (q = 2 kk, 2 kk + 1): swapping the
    // upper half of the q = 2 kk words with the lower half of the q = 2 kk + 1
    // words (v_permlane32_swap) gives every lane its 8 tokens, in order, which
    // go to block 2 wave + kk of the weight buffer (one contiguous 1 KB store).
    auto store_weights = [&](char* pbuf) __attribute__((always_inline)) {
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        u32x4_t pb;
#pragma unroll
        for (int w2 = 0; w2 < 2; ++w2) {
          const auto sw = __builtin_amdgcn_permlane32_swap(pw[4 * kk + w2], pw[4 * kk + 2 + w2], false, false);
          pb[w2] = sw[0];
          pb[2 + w2] = sw[1];
        }
        *reinterpret_cast<u32x4_t*>(pbuf + 1024 * (2 * wave + kk) + 16 * lane) = pb;
      }
    };

    // ---- value MFMAs of one tile: dims 128 wave .. +127, all heads -----------------
    // step idx = 4 kk + mt (kk outer, so that the two MFMAs into one accumulator
    // are 16 apart): the A operand V^T of dims 128 wave + 32 mt .. +31, tokens
    // 16 kk .. +15 through two transpose reads, kept in a ring indexed by the
    // step, feeds the four N-tiles; the B operands (weights) of token step kk,
    // N-tile nt are pb[kk][nt]. vstart() issues the reads the first steps need
    // (called from the end of a score phase); values() runs the MFMAs with
    // `slice(j)` (VALU work: two softmax weights of the next tile) in their
    // shadow.
    bf16x8_t pb[2][kMlaHeadTiles];
    s16x4_t vb[kMlaVPf + 1][2];
    auto vread = [&](const char* st, int idx) __attribute__((always_inline)) {
      const int mt = idx % kMlaDvTiles, kk = idx / kMlaDvTiles;
      const char* a0 = st + 2048 * (kMlaDvTiles * wave + mt) + 1024 * kk;
      vb[idx % (kMlaVPf + 1)][0] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(a0 + voff[0]));
      vb[idx % (kMlaVPf + 1)][1] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(a0 + voff[1]));
    };
    auto bread = [&](const char* pbuf, int kk) __attribute__((always_inline)) {
#pragma unroll
      for (int nt = 0; nt < kMlaHeadTiles; ++nt)
        pb[kk][nt] = *reinterpret_cast<const bf16x8_t*>(pbuf + 1024 * (2 * nt + kk) + 16 * lane);
    };
    auto vstart = [&](const char* st, const char* pbuf) __attribute__((always_inline)) {
      bread(pbuf, 0);
#pragma unroll
      for (int j = 0; j < kMlaVPf; ++j) vread(st, j);
    };
    auto values = [&](const char* st, const char* pbuf, auto&& slice) __attribute__((always_inline)) {
#pragma unroll
      for (int idx = 0; idx < kMlaValSteps; ++idx) {
        if (idx + kMlaVPf < kMlaValSteps) vread(st, idx + kMlaVPf);
        const int mt = idx % kMlaDvTiles, kk = idx / kMlaDvTiles;
        const s16x4_t* v = vb[idx % (kMlaVPf + 1)];
        const bf16x8_t a = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(v[0], v[1], 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
        for (int nt = 0; nt < kMlaHeadTiles; ++nt)
          o[kMlaHeadTiles * mt + nt] =
              __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[kk][nt], o[kMlaHeadTiles * mt + nt], 0, 0, 0);
        if (idx == 0) bread(pbuf, 1);
        slice(idx);
        __builtin_amdgcn_sched_barrier(0);
      }
    };

    // Before the weights of tile t: mask tokens past the shard's end (last
    // tile only) and, on a piece's first tile, set the reference max.
    auto prep = [&](int64_t t) __attribute__((always_inline)) {
      const int tok0 = static_cast<int>(t - ubeg) * kMlaTile;
      if (tok0 + kMlaTile > len) {  // uniform
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (tok0 + 8 * (r >> 2) + 4 * h + (r & 3) >= len) s_cur[r] = -INFINITY;
      }
      if (need_ref) {  // uniform
        float mt = -INFINITY;
#pragma unroll
        for (int r = 0; r < 16; ++r) mt = fmaxf(mt, s_cur[r] * c2);
        m_ref = fmaxf(mt, __shfl_xor(mt, 32, 64));
        need_ref = false;
      }
    };

    // Step t: scores of tile t, then the values of tile t - 1 (weights in LDS
    // buffer (t - 1) % 2) with the softmax of tile t in their shadow, then tile
    // t's weights to buffer t % 2; the barrier that ends the step publishes
    // them. The piece's first step has no values and the last tile's values
    // follow the loop.
    auto two_weights = [&](int j) __attribute__((always_inline)) {
      weight(2 * j);
      weight(2 * j + 1);
    };
    auto no_slice = [](int) __attribute__((always_inline)) {};
    auto no_tail = []() __attribute__((always_inline)) {};
    scores(lds + stage_of(tile) * kMlaStageBytes, s_cur, no_tail);
    prep(tile);
#pragma unroll
    for (int r = 0; r < 16; ++r) weight(r);
    store_weights(pbuf + kMlaPBytes * (tile & 1));
    end_tile(tile);
    for (int64_t t = tile + 1; t < piece_end; ++t) {
      const char* vst = lds + stage_of(t - 1) * kMlaStageBytes;
      const char* vpb = pbuf + kMlaPBytes * ((t - 1) & 1);
      scores(lds + stage_of(t) * kMlaStageBytes, s_cur,
             [&]() __attribute__((always_inline)) { vstart(vst, vpb); });
      prep(t);
      values(vst, vpb, two_weights);
      store_weights(pbuf + kMlaPBytes * (t & 1));
      end_tile(t);
    }
    {
      const char* vst = lds + stage_of(piece_end - 1) * kMlaStageBytes;
      const char* vpb = pbuf + kMlaPBytes * ((piece_end - 1) & 1);
      vstart(vst, vpb);
      values(vst, vpb, no_slice);
    }
    tile = piece_end;

    // ---- replay vote (block-uniform) and normalisers ----------------------------
    // This wave's heads: normaliser (sum of the rounded weights) and fp32 weight
    // sum over both token halves of the lane pair (l, l ^ 32).
    const float lt_ = lsum + __shfl_xor(lsum, 32, 64);
    const float et = esum + __shfl_xor(esum, 32, 64);
    const int my_head = kMlaHeadsPerWave * wave + (lane & 31);
    // the replay votes of the waves and the normaliser of each head go to the
    // weight buffer of tile piece_end: its last readers (the values of tile
    // piece_end - 2) finished before the last step's barrier, and its next
    // writer (the next piece's first step) comes after the barriers below
    float* s_norm = reinterpret_cast<float*>(pbuf + kMlaPBytes * (piece_end & 1));
    int* s_vote = reinterpret_cast<int*>(s_norm + kMlaHeads);
    const int wave_bad = __any(mx > kMlaRefSlack) ? 1 : 0;  // every lane takes part in the wave vote
    if (lane == 0) s_vote[wave] = wave_bad;
    if (h == 0) s_norm[my_head] = lt_;
    wait_lgkm0();  // votes and normalisers are in LDS before the barrier
    block_sync();
    int any_bad = 0;
#pragma unroll
    for (int w = 0; w < kMlaWaves; ++w) any_bad |= s_vote[w];
    float inv[kMlaHeadTiles];  // 1 / normaliser of head 32 nt + l % 32
#pragma unroll
    for (int nt = 0; nt < kMlaHeadTiles; ++nt) inv[nt] = 1.f / s_norm[32 * nt + (lane & 31)];
    wait_lgkm0();
    block_sync();  // every wave has read votes and normalisers before they are written again
    // One replay always suffices for finite scores (its reference is the
    // largest scaled score of the piece); a second vote can only come from
    // non-finite inputs, which then simply propagate.
    if (any_bad && !replay) {
      replay = true;
      // replay the piece with the largest scaled score seen as the reference
      const float ms = mx + m_ref;
      m_hint = fmaxf(ms, __shfl_xor(ms, 32, 64));
      wait_vmcnt<0>();
      block_sync();
      tile = piece_tile0;
      cur_u = ld_uniform(ws.wunit + worker);
      restart(piece_tile0, cur_u);
      continue;
    }
    replay = false;
    m_hint = -INFINITY;

    // ---- piece end --------------------------------------------------------------
    // O rows: this wave's dims of every head; LSE / (m_ref, normaliser, weight
    // sum): this wave's heads.
    const bool whole = (lt_lo == 0) && (lt_hi == uend - ubeg);
    const int which = (lt_lo == 0) ? 1 : 0;  // 0: the unit began before this worker
    const int dim0 = kMlaDvTiles * 32 * wave + 4 * h;
    if (whole) {
      const int64_t row0 = cur_u * kMlaHeads;  // = ((r * batch + b) * q_len + i) * Hq
#pragma unroll
      for (int nt = 0; nt < kMlaHeadTiles; ++nt) {
        float* dst = p.out_o + (row0 + 32 * nt + (lane & 31)) * kMlaDv + dim0;
#pragma unroll
        for (int mt = 0; mt < kMlaDvTiles; ++mt)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const f32x16_t& a = o[kMlaHeadTiles * mt + nt];
            *reinterpret_cast<f32x4_t*>(dst + 32 * mt + 8 * q) =
                f32x4_t{a[4 * q], a[4 * q + 1], a[4 * q + 2], a[4 * q + 3]} * inv[nt];
          }
      }
      if (h == 0) p.out_lse[row0 + my_head] = (m_ref + __log2f(et)) * DCP_LN2;
    } else {
      float* part = ws.part + (static_cast<int64_t>(worker) * 2 + which) * kMlaHeads * (kMlaDv + kPartExtra);
#pragma unroll
      for (int nt = 0; nt < kMlaHeadTiles; ++nt) {
        float* dst = part + (32 * nt + (lane & 31)) * (kMlaDv + kPartExtra) + dim0;
#pragma unroll
        for (int mt = 0; mt < kMlaDvTiles; ++mt)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const f32x16_t& a = o[kMlaHeadTiles * mt + nt];
            *reinterpret_cast<f32x4_t*>(dst + 32 * mt + 8 * q) = f32x4_t{a[4 * q], a[4 * q + 1], a[4 * q + 2], a[4 * q + 3]};
          }
      }
      if (h == 0) {
        float* dst = part + my_head * (kMlaDv + kPartExtra);
        dst[kMlaDv] = m_ref;
        dst[kMlaDv + 1] = lt_;
        dst[kMlaDv + 2] = et;
      }
    }
  }
  wait_vmcnt<0>();  // refills issued past the last tile still write this workgroup's LDS
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
bool mla_supported(const AttnParams& p) {
  const dcp_kv_cache_t& kv = p.kv;
  if (p.q_dtype != DCP_BF16 || kv.dtype != DCP_BF16) return false;
  if (kv.v != nullptr || kv.num_kv_heads != 1 || p.num_q_heads != kMlaHeads) return false;
  if (kv.head_dim_k != kMlaDk || kv.head_dim_v != kMlaDv) return false;
  if (kv.block_size % 16 != 0) return false;
  if (kv.k_stride[4] != 1) return false;
  for (int i = 0; i < 4; ++i)
    if ((kv.k_stride[i] * 2) % 16 != 0) return false;
  if (reinterpret_cast<uintptr_t>(kv.k) % 16) return false;
  // block byte stride in 32 bits, offsets within a block in 31
  if (kv.k_stride[1] * 2 >= (int64_t(1) << 32)) return false;
  if (static_cast<int64_t>(kv.block_size) * kv.k_stride[3] * 2 >= (int64_t(1) << 31)) return false;
  if (static_cast<int64_t>(p.rank_count) * p.batch * p.q_len >= (int64_t(1) << 31)) return false;
  if (p.tpu != 1) return false;  // one query token per unit
  return true;
}

// One persistent workgroup per CU; the workspace is sized for that many.
static int mla_workers() { return min(kMlaMaxWorkers, device_cu_count()); }

size_t mla_workspace_bytes(const AttnParams& p) {
  return split_ws_bytes(split_units_host(p), mla_workers(), kMlaHeads, kMlaDv);
}

hipError_t launch_mla_attn(const AttnParams& p) {
  const int workers = mla_workers();
  launch_split_plan(p, kMlaTile, workers);
  if (p.ev_begin) (void)hipEventRecord(p.ev_begin, p.stream);
  hipLaunchKernelGGL(mla_attn_kernel, dim3(workers), dim3(kMlaThreads), 0, p.stream, p, workers);
  if (p.ev_end) (void)hipEventRecord(p.ev_end, p.stream);
  launch_split_combine<kMlaDv>(p, workers);
  return hipGetLastError();
}

}  // namespace dcp
