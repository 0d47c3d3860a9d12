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
//     that the MFMA operand reads spread over the LDS banks. A tile is
//     refilled four tiles ahead, right after the barrier that ends the last
//     read of its stage, so two to three tiles are always in flight;
//   * each of the 4 wavefronts owns 32 query heads: its latent Q (32 x 512
//     bf16, 128 VGPRs) and its O accumulator (32 x 512 fp32, 256 AGPRs) stay
//     in registers for the whole piece; the rope part of Q sits in LDS;
//   * scores S^T[token, head] = K[token, :] . Q[head, :] on 16x16x32 bf16
//     MFMA, K rows read from LDS with ds_read_b128 (one read feeds both head
//     tiles);
//   * softmax weights in log2 units relative to a per-piece reference max
//     (the first tile's): no rescaling of the 256-register accumulator and no
//     cross-lane reduction inside the loop; a piece whose scores outgrow the
//     reference by more than 2^64 is replayed with a higher reference. The
//     weights are rounded to bf16 for the value product and their sum (the
//     normaliser) is taken over the same rounded values, with an fp32 sum of
//     the unrounded weights for the LSE (as in the GQA kernel);
//   * values O^T[dim, head] += V^T[dim, token] . P^T[token, head]; V^T comes
//     from the same LDS rows through ds_read_b64_tr_b16, whose 16-lane
//     transpose hands each lane four consecutive tokens of one dimension;
//   * software pipeline across tiles: the softmax of tile t is interleaved,
//     one weight per k-step, with the score MFMAs of tile t+1, and the value
//     MFMAs of tile t follow, so the matrix core never waits for the softmax.
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
constexpr int kMlaQRopeWaveBytes = (kMlaKSteps - kMlaKStepsLat) * 64 * 16;  // 4 KB per wave
constexpr int kMlaDvTiles = kMlaDv / 32;                         // 16 value M-tiles of 32 dims
#ifndef DCP_MLA_KPF
#define DCP_MLA_KPF 4
#endif
#ifndef DCP_MLA_VPF
#define DCP_MLA_VPF 6
#endif
constexpr int kMlaKPf = DCP_MLA_KPF;  // score-operand read distance (k-steps)
constexpr int kMlaVPf = DCP_MLA_VPF;  // value-operand read distance (value tiles)
constexpr int kMlaMaxWorkers = 512;
constexpr float kMlaRefSlack = 64.f;  // log2 units a score may exceed the piece's reference

static_assert(kMlaStages == 4, "the refill distance below assumes 4 stages");
static_assert(kMlaKStepsLat == 32 && kMlaKSteps - kMlaKStepsLat == 4, "32 latent + 4 rope k-steps");

typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;
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
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(lds_base) : "memory");
}

// Same, from a wave-uniform base plus a 32-bit per-lane byte offset.
// (The base and M0 values are wave-uniform by construction; readfirstlane
// pins them to SGPRs where the compiler cannot prove it.)
__device__ __forceinline__ void dma16_s(uint32_t voff, const void* sbase, uint32_t lds_base) {
  // (readfirstlane yields a signed int: each half is taken as uint32_t before
  // widening, or a low word with bit 31 set would smear into the high word)
  const uint64_t b = reinterpret_cast<uint64_t>(sbase);
  const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(b)));
  const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(b >> 32)));
  const uint64_t bu = static_cast<uint64_t>(lo) | (static_cast<uint64_t>(hi) << 32);
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff),
               "s"(reinterpret_cast<const void*>(bu)), "s"(__builtin_amdgcn_readfirstlane(lds_base))
               : "memory");
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
  // rope part of Q in operand order: [wave][hh][ks - 16][lane] x 16 bytes.
  // The replay vote of wave w lives in the first 4 bytes of w's own slice: by
  // the time a wave votes it no longer reads its slice, and the slice is
  // refilled only after every wave has read the votes.
  __shared__ __attribute__((aligned(16))) char qrope[kMlaWaves * kMlaQRopeWaveBytes];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (SGPR)
  const int n = lane & 15, g = lane >> 4;
  const int worker = blockIdx.x;
  const int64_t U = split_units(p);
  SplitWs ws = split_ws(p.workspace, U, kMlaMaxWorkers);
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
  const float c2 = p.softmax_scale * DCP_LOG2E;
  const uint32_t lds0 = lds_addr(lds);
  auto stage_of = [&](int64_t t) __attribute__((always_inline)) {
    return static_cast<int>((t - wstart) & (kMlaStages - 1));
  };

  // ---- tile sources -----------------------------------------------------------
  // A walker over the worker's tiles in order: per unit it caches the length,
  // block-table row and rank base; per tile it advances the (virtual block,
  // offset) of the tile's first token and yields the two 16-token halves
  // (tokens t0 .. t0+15 share one block and so do t0+16 .. t0+31, block_size %
  // 16 == 0). Rows past the shard's end are replaced by the last valid row
  // of their half, or of the first half if the second has none (finite data,
  // zero weight): nv0 / nv1 give the rows to clamp to, and base1 = base0 when
  // the second half is empty.
  struct Walker {
    int64_t t, u, ubeg, uend;
    bool fresh;
    int len, vb, off;
    int vb_loaded, blk;  // the last block-table entry read (consecutive tiles often share it)
    const int32_t* bt;
    const char* rk;
  };
  struct TileSrc {
    const char* base0;
    const char* base1;
    int nv0, nv1;
  };
  auto walker_at = [&](int64_t t, int64_t u) __attribute__((always_inline)) {
    Walker w;
    w.t = t;
    w.u = u;
    w.ubeg = ld_uniform(ws.prefix + u);
    w.uend = ld_uniform(ws.prefix + u + 1);
    w.fresh = true;
    w.len = w.vb = w.off = 0;
    w.vb_loaded = -1;
    w.blk = 0;
    w.bt = p.block_table;
    w.rk = kbase;
    return w;
  };
  auto next_src = [&](Walker& w) __attribute__((always_inline)) {
    while (w.uend <= w.t) {
      ++w.u;
      w.ubeg = w.uend;
      w.uend = ld_uniform(ws.prefix + w.u + 1);
      w.fresh = true;
    }
    if (w.fresh) {
      // unit u = (r * batch + b) * q_len + i: rank r, request b, query token i
      const int uu = static_cast<int>(w.u), rb = uu / p.q_len, i = uu - rb * p.q_len;
      const int b = rb % p.batch, r = rb / p.batch;
      w.len = ld_uniform(p.local_lens + (static_cast<int64_t>(b) * p.q_len + i) * p.dcp_size + p.rank_begin + r);
      w.bt = p.block_table + static_cast<int64_t>(b) * p.bt_stride;
      w.rk = kbase + r * ks0 * 2;
      const int t0 = static_cast<int>(w.t - w.ubeg) * kMlaTile;
      w.vb = t0 / bs;
      w.off = t0 - w.vb * bs;
      w.vb_loaded = -1;
      w.fresh = false;
    }
    if (w.vb != w.vb_loaded) {  // uniform
      w.blk = ld_uniform(w.bt + w.vb);
      w.vb_loaded = w.vb;
    }
    const int t0 = static_cast<int>(w.t - w.ubeg) * kMlaTile;
    TileSrc src;
    src.nv0 = min(16, w.len - t0);
    const int nv1 = min(16, w.len - t0 - 16);
    src.base0 = w.rk + (static_cast<int64_t>(w.blk) * ks1 + w.off * ks3) * 2;
    src.base1 = src.base0;
    src.nv1 = src.nv0;
    if (nv1 > 0) {  // uniform
      int off_b = w.off + 16, vb_b = w.vb;
      int blk_b = w.blk;
      if (off_b >= bs) {  // uniform: the second half starts a new block
        off_b -= bs;
        ++vb_b;
        blk_b = ld_uniform(w.bt + vb_b);
      }
      src.base1 = w.rk + (static_cast<int64_t>(blk_b) * ks1 + off_b * ks3) * 2;
      src.nv1 = nv1;
    }
    ++w.t;
    w.off += kMlaTile;
    while (w.off >= bs) { w.off -= bs; ++w.vb; }
    return src;
  };

  // ---- DMA producer -------------------------------------------------------------
  // Wave w loads blocks w, w+4, .., w+32 of each tile: token half w % 2,
  // k-steps w / 2 + 2 k (k = 0 .. 8); DMA lane 16 c + m fetches row m ^ 4 c of
  // the half, chunk 4 ks + c. A refill (one wave's share of a tile) is
  // prepared while the previous tile computes, and its 9 DMAs are spread
  // over the k-steps of the next score phase.
  Walker dw = walker_at(wstart, ld_uniform(ws.wunit + worker));
  const int dma_row = n ^ (4 * g);
  const int my_half = wave & 1;
  struct Refill {
    const char* base;  // this wave's token half
    uint32_t voff;     // lane offset of k-step w / 2
    uint32_t m0;       // LDS address of block w of the stage
  };
  auto prepare = [&]() __attribute__((always_inline)) {
    const int stage = stage_of(dw.t);
    const TileSrc src = next_src(dw);
    Refill r;
    r.base = my_half ? src.base1 : src.base0;
    const int nv = my_half ? src.nv1 : src.nv0;
    r.voff = static_cast<uint32_t>(min(dma_row, nv - 1) * row_bytes + 16 * g + 64 * (wave >> 1));
    r.m0 = lds0 + stage * kMlaStageBytes + wave * 1024;
    return r;
  };
  // DMA k (0 .. 8) of this wave for the refill r: k-step w / 2 + 2 k, block w + 4 k
  auto dma = [&](const Refill& r, int k) __attribute__((always_inline)) {
    dma16_s(r.voff + 128 * k, r.base, r.m0 + 4096 * k);
  };
  // Every tile step issues exactly one refill (9 DMAs per wave): once the
  // worker's tiles run out, the last real refill is issued again (it rewrites
  // a stage with the data it already holds), so every wait count below is a
  // constant and no branch guards a DMA. The kernel drains them before exit.
  Refill next_refill;  // the refill prepared during the current tile
  Refill pending;      // the refill the next score phase issues

  // (Re)start the ring at tile t (unit u): load tiles t .. t+3 at once and
  // wait until the first two have landed everywhere.
  auto restart = [&](int64_t t, int64_t u) __attribute__((always_inline)) {
    dw = walker_at(t, u);
    for (int j = 0; j < kMlaStages; ++j) {
      if (t + j < wend) next_refill = prepare();  // uniform
#pragma unroll
      for (int k = 0; k < kMlaDmaPerTile; ++k) dma(next_refill, k);
    }
    // the next score phase re-issues the last refill: same data into the same
    // stage (a duplicate step only makes the next waits more conservative)
    pending = next_refill;
    wait_vmcnt<2 * kMlaDmaPerTile>();
    block_sync();
  };
  // During tile t's value phase: prepare the refill with tile t+4 (issued
  // after the barrier that ends tile t).
  auto begin_tile = [&](int64_t t) __attribute__((always_inline)) {
    if (t + kMlaStages < wend) next_refill = prepare();  // uniform
  };
  // End of tile t (every read of its stage issued): wait until tile t+2 has
  // landed; the refill of t's stage with tile t+4 becomes pending. The step
  // after t+2's (issued during this iteration's score phase, or by restart)
  // is the only one allowed to stay in flight.
  auto end_tile = [&](int64_t) __attribute__((always_inline)) {
    wait_lgkm0();
    wait_vmcnt<kMlaDmaPerTile>();
    block_sync();
    pending = next_refill;
  };
  // DMA j of the pending refill, issued after k-step 4 j of a score phase
  auto pending_dma = [&](int ks) __attribute__((always_inline)) {
    if ((ks & 3) == 0 && ks / 4 < kMlaDmaPerTile) dma(pending, ks / 4);
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
  char* qr = qrope + wave * kMlaQRopeWaveBytes + lane * 16;

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
    // .. +7; latent k-steps in VGPRs, rope k-steps in this wave's LDS slice
    bf16x8_t qop[kMlaKStepsLat];
    {
      const uint16_t* qb = reinterpret_cast<const uint16_t*>(p.q) +
                           ((static_cast<int64_t>(b) * p.q_len + qi) * kMlaHeads + kMlaHeadsPerWave * wave +
                            (lane & 31)) * kMlaDk + 8 * h;
#pragma unroll
      for (int ks = 0; ks < kMlaKStepsLat; ++ks) qop[ks] = *reinterpret_cast<const bf16x8_t*>(qb + 16 * ks);
#pragma unroll
      for (int ks = kMlaKStepsLat; ks < kMlaKSteps; ++ks)
        *reinterpret_cast<bf16x8_t*>(qr + (ks - kMlaKStepsLat) * 1024) =
            *reinterpret_cast<const bf16x8_t*>(qb + 16 * ks);
    }
    // Q is complete here, so no wait for it lands inside the tile loop (where
    // it would also drain the tiles in flight).
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_sched_barrier(0);

    // ---- piece state ------------------------------------------------------------
    // Weights are exp2(s c2 - m_ref) with m_ref fixed for the piece (the first
    // tile's max unless a replay hands one in); mx tracks the largest exponent
    // seen, for the replay vote and the next reference. O^T[dim, head] of M-tile
    // mt: lane l holds head l % 32, dims 32 mt + 8 (r / 4) + 4 h + r % 4.
    float m_ref = m_hint, mx = -INFINITY, lsum = 0.f, esum = 0.f;
    f32x16_t o[kMlaDvTiles];
#pragma unroll
    for (int mt = 0; mt < kMlaDvTiles; ++mt) o[mt] = f32x16_t{};
    bool need_ref = !replay;  // uniform

    // ---- score MFMAs of one tile: S^T[token, head], lane l holding head l % 32,
    // tokens 8 (r / 4) + 4 h + r % 4 of register r; `slice(ks)` (VALU work of
    // the previous tile) goes after k-step ks's MFMA, which depends on the one
    // before it ------------------------------------------------------------------
    auto scores = [&](const char* st, f32x16_t& s, auto&& slice) __attribute__((always_inline)) {
      s = f32x16_t{};
      bf16x8_t ka[kMlaKPf + 1];
      bf16x8_t qx[kMlaKSteps - kMlaKStepsLat];  // rope Q, read from LDS with the rope K rows
      auto kread = [&](int ks) __attribute__((always_inline)) {
        ka[ks % (kMlaKPf + 1)] = *reinterpret_cast<const bf16x8_t*>(st + koff[ks & 1] + 2048 * (ks >> 1));
        if (ks >= kMlaKStepsLat)
          qx[ks - kMlaKStepsLat] = *reinterpret_cast<const bf16x8_t*>(qr + (ks - kMlaKStepsLat) * 1024);
      };
#pragma unroll
      for (int j = 0; j < kMlaKPf; ++j) kread(j);
#pragma unroll
      for (int ks = 0; ks < kMlaKSteps; ++ks) {
        if (ks + kMlaKPf < kMlaKSteps) kread(ks + kMlaKPf);
        const bf16x8_t bq = ks < kMlaKStepsLat ? qop[ks < kMlaKStepsLat ? ks : 0]
                                               : qx[ks < kMlaKStepsLat ? 0 : ks - kMlaKStepsLat];
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[ks % (kMlaKPf + 1)], bq, s, 0, 0, 0);
        slice(ks);
        pending_dma(ks);
        __builtin_amdgcn_sched_barrier(0);
      }
    };

    // ---- softmax of one tile: weight r (0 .. 15) of this lane, one per slice;
    // pw[d] packs weights 2 d, 2 d + 1 (tokens 8 (d / 2) + 4 h + 2 (d % 2) + {0, 1})
    f32x16_t s_cur, s_nxt;
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
    auto no_slice = [](int) __attribute__((always_inline)) {};

    // ---- value MFMAs of one tile --------------------------------------------------
    // B operand of token step kk: lane l needs head l % 32, tokens 16 kk + 8 h ..
    // +7. A lane holds tokens 4 h + {0..3} + 8 q (q = 2 kk, 2 kk + 1): swapping the
    // upper half of the q = 2 kk words with the lower half of the q = 2 kk + 1
    // words (v_permlane32_swap) gives every lane its 8 tokens, in order.
    auto values = [&](const char* st, auto&& side) __attribute__((always_inline)) {
      u32x4_t pb[2];
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
        for (int w2 = 0; w2 < 2; ++w2) {
          const auto sw = __builtin_amdgcn_permlane32_swap(pw[4 * kk + w2], pw[4 * kk + 2 + w2], false, false);
          pb[kk][w2] = sw[0];
          pb[kk][2 + w2] = sw[1];
        }
      }
      // step idx = 16 kk + mt (kk outer, so that the two MFMAs into one
      // accumulator are 16 apart): two transpose reads, kept in a ring indexed
      // by the step
      s16x4_t vb[kMlaVPf + 1][2];
      auto vread = [&](int idx) __attribute__((always_inline)) {
        const int mt = idx & 15, kk = idx >> 4;
        const char* a0 = st + 2048 * mt + 1024 * kk;
        vb[idx % (kMlaVPf + 1)][0] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(a0 + voff[0]));
        vb[idx % (kMlaVPf + 1)][1] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(a0 + voff[1]));
      };
#pragma unroll
      for (int j = 0; j < kMlaVPf; ++j) vread(j);
#pragma unroll
      for (int idx = 0; idx < 2 * kMlaDvTiles; ++idx) {
        if (idx == 2) side();  // scalar work in the shadow of the MFMAs
        if (idx + kMlaVPf < 2 * kMlaDvTiles) vread(idx + kMlaVPf);
        const int mt = idx & 15, kk = idx >> 4;
        const s16x4_t* v = vb[idx % (kMlaVPf + 1)];
        const bf16x8_t a = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(v[0], v[1], 0, 1, 2, 3, 4, 5, 6, 7));
        o[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, __builtin_bit_cast(bf16x8_t, pb[kk]), o[mt], 0, 0, 0);
        if (idx & 1) __builtin_amdgcn_sched_barrier(0);
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

    scores(lds + stage_of(tile) * kMlaStageBytes, s_cur, no_slice);
    for (int64_t t = tile; t < piece_end; ++t) {
      prep(t);
      if (t + 1 < piece_end) {
        scores(lds + stage_of(t + 1) * kMlaStageBytes, s_nxt, weight);
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) weight(r);
        // no score phase here: the pending refill goes out now, before
        // end_tile counts on it
#pragma unroll
        for (int k = 0; k < kMlaDmaPerTile; ++k) dma(pending, k);
      }
      values(lds + stage_of(t) * kMlaStageBytes, [&]() __attribute__((always_inline)) { begin_tile(t); });
      end_tile(t);
      s_cur = s_nxt;
    }
    tile = piece_end;

    // ---- replay vote (block-uniform) ------------------------------------------
    const int wave_bad = __any(mx > kMlaRefSlack) ? 1 : 0;  // every lane takes part in the wave vote
    if (lane == 0) *reinterpret_cast<int*>(qrope + wave * kMlaQRopeWaveBytes) = wave_bad;
    wait_lgkm0();  // the vote is in LDS before the barrier
    block_sync();
    int any_bad = 0;
#pragma unroll
    for (int w = 0; w < kMlaWaves; ++w) any_bad |= *reinterpret_cast<const int*>(qrope + w * kMlaQRopeWaveBytes);
    block_sync();  // every wave has read the votes before they are written again
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
    const bool whole = (lt_lo == 0) && (lt_hi == uend - ubeg);
    const int which = (lt_lo == 0) ? 1 : 0;  // 0: the unit began before this worker
    const float lt_ = lsum + __shfl_xor(lsum, 32, 64);
    const float et = esum + __shfl_xor(esum, 32, 64);
    const int head = kMlaHeadsPerWave * wave + (lane & 31);
    if (whole) {
      const int64_t row = cur_u * kMlaHeads + head;  // = ((r * batch + b) * q_len + i) * Hq + head
      float* dst = p.out_o + row * kMlaDv + 4 * h;
      const float inv = 1.f / lt_;
#pragma unroll
      for (int mt = 0; mt < kMlaDvTiles; ++mt)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          *reinterpret_cast<f32x4_t*>(dst + 32 * mt + 8 * q) =
              f32x4_t{o[mt][4 * q], o[mt][4 * q + 1], o[mt][4 * q + 2], o[mt][4 * q + 3]} * inv;
      if (h == 0) p.out_lse[row] = (m_ref + __log2f(et)) * DCP_LN2;
    } else {
      float* dst = ws.part + ((static_cast<int64_t>(worker) * 2 + which) * kMlaHeads + head) * (kMlaDv + kPartExtra);
#pragma unroll
      for (int mt = 0; mt < kMlaDvTiles; ++mt)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          *reinterpret_cast<f32x4_t*>(dst + 32 * mt + 8 * q + 4 * h) =
              f32x4_t{o[mt][4 * q], o[mt][4 * q + 1], o[mt][4 * q + 2], o[mt][4 * q + 3]};
      if (h == 0) {
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
  if (static_cast<int64_t>(p.rank_count) * p.batch * p.q_len >= (int64_t(1) << 31)) return false;
  if (p.tpu != 1) return false;  // one query token per unit
  return true;
}

size_t mla_workspace_bytes(const AttnParams& p) {
  return split_ws_bytes(split_units_host(p), kMlaMaxWorkers, kMlaHeads, kMlaDv);
}

hipError_t launch_mla_attn(const AttnParams& p) {
  const int workers = min(kMlaMaxWorkers, device_cu_count());
  launch_split_plan(p, kMlaTile, workers, kMlaMaxWorkers);
  if (p.ev_begin) (void)hipEventRecord(p.ev_begin, p.stream);
  hipLaunchKernelGGL(mla_attn_kernel, dim3(workers), dim3(kMlaThreads), 0, p.stream, p, workers);
  if (p.ev_end) (void)hipEventRecord(p.ev_end, p.stream);
  launch_split_combine<kMlaDv>(p, workers, kMlaMaxWorkers);
  return hipGetLastError();
}

}  // namespace dcp
