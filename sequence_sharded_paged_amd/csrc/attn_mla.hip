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
// at the HBM rate this kernel needs most of the chip's bf16 MFMA rate. The
// design keeps the matrix cores fed from LDS at a rate one wavefront can
// sustain: on gfx950 the LDS serves a CU about 220 B/clk, but a single
// wavefront draws only about 29 B/clk from it, so with one wavefront per SIMD
// an MFMA that needs a fresh 1 KB LDS operand every 32 cycles (the previous
// design's score phase) waits on the LDS.
//
// Work split: stream-K over (rank, request, query token) units (splitkv.h;
// one query token per unit when several are decoded at once), one persistent
// 256-thread workgroup (one wavefront per SIMD) per CU, tiles of 16 tokens.
// Per workgroup and tile:
//   * the tile (16 rows x 1152 B) sits in a 7-stage LDS ring, filled straight
//     from HBM with global_load_lds_dwordx4, in score-operand order: the 16
//     rows' 16-byte chunk c (dims 8 c .. 8 c + 7) of the 32-dim k-step ks
//     form a 256-byte run, placed so that neither the score-operand reads nor
//     the transposing value-operand reads meet LDS bank conflicts (ring_run,
//     ring_swz). Tiles are loaded five ahead, so a tile has about three steps
//     to arrive;
//   * scores: the wavefront pair (0, 1) handles heads 0..63, the pair (2, 3)
//     heads 64..127; within a pair, wavefront dh takes key dims 288 dh ..
//     288 dh + 287. Each wavefront holds Q for its 64 heads x 288 dims (144
//     VGPRs) and computes partial scores S^T[token, head] on 16x16x32 bf16
//     MFMAs: every K operand read from LDS feeds four MFMAs (four head
//     tiles), a quarter of the LDS traffic per MFMA of a one-head-tile
//     layout;
//   * the pair exchanges partial scores through LDS (2 KB per wavefront per
//     tile): wavefront dh keeps heads 32 dh .. 32 dh + 31 of its pair's 64,
//     adds the partner's partial and owns their softmax;
//   * softmax in log2 units relative to a per-piece reference max (the first
//     tile's): no rescaling of the accumulators and no cross-lane reduction
//     inside the loop; a piece whose scores outgrow the reference by more
//     than 2^64 is replayed with a higher reference. Weights are rounded to
//     bf16 for the value product and their sum (the normaliser) is taken over
//     the same rounded values, with an fp32 sum of the unrounded weights for
//     the LSE. Tokens past the shard's end are masked after scaling, so any
//     finite softmax scale (zero and negative included) is handled;
//   * values: the bf16 weights of all 128 heads go through a 4 KB LDS buffer;
//     wavefront w owns latent dims 128 w .. 128 w + 127 of every head:
//     O^T[dim, head] += V^T[dim, token] . P^T[token, head] on 32x32x16 bf16
//     MFMAs, its O (128 x 128 fp32) in AGPRs for the whole piece. V^T comes
//     from the tile's LDS rows through ds_read_b64_tr_b16 (a 16-lane
//     transpose handing each lane four consecutive tokens of one dim);
//   * software pipeline, one workgroup barrier per tile: after the barrier
//     that publishes tile t's partial scores, step t issues the DMA of tile
//     t + 5 and runs one MFMA stream that interleaves the score MFMAs of tile
//     t + 1 with the value MFMAs of tile t - 1 (independent accumulators, so
//     neither waits on its own accumulation chain), with the softmax of tile t
//     in its shadow, and tile t's weights stored under its last MFMAs; it
//     then sends tile t + 1's partial scores.
//
// DMA sources come from a scalar walker over the worker's tiles (a few scalar
// instructions per tile); block-table entries are read through a 64-entry
// window held one per lane of a VGPR and refilled once per 64 blocks or unit.
#include <utility>

#include "splitkv.h"

namespace dcp {

constexpr int kMlaDk = 576;
constexpr int kMlaDv = 512;
constexpr int kMlaHeads = 128;
constexpr int kMlaTile = 16;                                   // tokens per tile
constexpr int kMlaStages = 7;                                  // LDS ring depth
constexpr int kMlaAhead = 5;                                   // tiles loaded ahead of the scores
constexpr int kMlaBlocks = kMlaDk / 32;                        // 18 operand blocks of 1 KB per tile
constexpr int kMlaStageBytes = kMlaBlocks * 1024;              // 18432
constexpr int kMlaWaves = 4;
constexpr int kMlaThreads = 64 * kMlaWaves;
constexpr int kMlaKSteps = kMlaBlocks / 2;                     // 9 score k-steps (32 dims) per wavefront
constexpr int kMlaDvTiles = kMlaDv / 32 / kMlaWaves;           // 4 value M-tiles of 32 dims per wavefront
constexpr int kMlaHeadTiles = kMlaHeads / 32;                  // 4 value N-tiles of 32 heads
constexpr int kMlaPBytes = kMlaTile * kMlaHeads * 2;           // 4 KB of bf16 weights per tile
constexpr int kMlaXBytes = kMlaWaves * 2048;                   // partial scores sent per tile
#ifndef DCP_MLA_KAHEAD
#define DCP_MLA_KAHEAD 1
#endif
constexpr int kMlaKAhead = DCP_MLA_KAHEAD;                    // score operand read distance (k-steps)
constexpr int kMlaMaxWorkers = 512;
constexpr float kMlaRefSlack = 64.f;  // log2 units a score may exceed the piece's reference

static_assert(kMlaStages >= kMlaAhead + 2, "the refill of tile t + ahead goes to the stage of tile t - 2");
static_assert(kMlaStages * kMlaStageBytes + 2 * kMlaPBytes + 2 * kMlaXBytes + 2048 <= 160 * 1024, "LDS");

typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// f(std::integral_constant<int, I>{}) for I = 0 .. N-1, in order
template <typename F, int... I>
__device__ __forceinline__ void static_for_seq(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_seq(f, std::make_integer_sequence<int, N>{});
}

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

// s_waitcnt lgkmcnt(0) with vmcnt / expcnt left alone.
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xc07f); }

// Workgroup barrier without the memory fence of __syncthreads (which would
// wait for every tile in flight); the asm memory clobber keeps the compiler
// from moving LDS accesses across it.
__device__ __forceinline__ void block_sync() { asm volatile("s_barrier" ::: "memory"); }

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) char*)p));
}

// 16 bytes per lane from sbase + voff + kImm into LDS at lds_base + 16 * lane.
// The instruction's immediate offset applies to both addresses (global and
// LDS), so M0 is set to lds_base - kImm.
// Issued through asm so that the compiler, which cannot tell the ring stages
// apart, does not make later LDS reads wait for it; the kernel orders these
// writes itself (vmcnt wait + barrier before a stage is read, barrier before it
// is refilled). The base and M0 values are wave-uniform by construction
// (readfirstlane pins them to SGPRs); the asm only moves into M0, since SALU
// arithmetic inside it would overwrite SCC, which the compiler may hold live.
template <int kImm>
__device__ __forceinline__ void dma16(uint32_t voff, const void* sbase, uint32_t lds_base) {
  static_assert(kImm >= 0 && kImm < 4096, "global offset immediate");
  const uint64_t b = reinterpret_cast<uint64_t>(sbase);
  const uint64_t bu = join_halves(__builtin_amdgcn_readfirstlane(low_half(b)), __builtin_amdgcn_readfirstlane(high_half(b)));
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 offset:%3" ::"v"(voff),
               "s"(reinterpret_cast<const void*>(bu)), "s"(__builtin_amdgcn_readfirstlane(lds_base - kImm)), "i"(kImm)
               : "memory", "m0");
}

// LDS offset of lane l's 16 bytes in a 4 KB buffer read or written with one
// 128-bit access per lane: 16-lane quarter q of the wave at 1 KB q. On gfx950
// a 128-bit LDS access whose four quarters share one 1 KB line costs three
// bank-conflict cycles (measured with SQ_LDS_BANK_CONFLICT); quarters 1 KB
// apart cost none. Buffers accessed this way interleave four 256-byte rows
// (selected by the caller's offset) per 1 KB line.
__device__ __forceinline__ int quad_off(int lane) { return 1024 * (lane >> 4) + 16 * (lane & 15); }

// Ring tile layout. Run (ks, c) (chunk c = 0..3 of k-step ks = 0..17, 16 rows
// x 16 bytes) starts at ring_run(ks, c); row t sits at 16 (t ^ ring_swz(c))
// in it. The runs of a score-operand read (one k-step, chunk c in 16-lane
// quarter c) pair quarters 0, 1 and 2, 3 across different 1 KB lines, and
// the row permutations 0, 12, 4, 8 keep both that read and the transposing
// value read (rows 4 i .. 4 i + 3 of chunks 2 j, 2 j + 1 per quarter) free of
// bank conflicts on gfx950 (measured per pattern with SQ_LDS_BANK_CONFLICT;
// the plain 16 c + (t ^ 4 c) order within one 1 KB block cost four cycles per
// score read). The 1 KB line 2 (ks / 2) + (c % 2) holds chunks c % 2 and
// c % 2 + 2 of k-steps ks & ~1 and ks | 1, which is what one DMA writes.
__device__ __forceinline__ constexpr int ring_run(int ks, int c) {
  return 1024 * (2 * (ks >> 1) + (c & 1)) + 256 * (2 * (ks & 1) + (c >> 1));
}
__device__ __forceinline__ constexpr int ring_swz(int c) { return (0x84C0 >> (4 * c)) & 15; }

// O += A . B on a 32x32x16 bf16 MFMA, a compiler builtin: the compiler then
// tracks the wait states of every other instruction that reads or moves O,
// including the copies it makes between code paths.
__device__ __forceinline__ void mfma_acc(f32x16_t& acc, const bf16x8_t& a, const bf16x8_t& b) {
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
}

// Score MFMA (16x16x32 bf16) with its accumulator in VGPRs, issued through
// asm: with the AGPRs full of O accumulators the compiler would give a
// builtin score MFMA an AGPR destination and move an O tile out of its way
// around every step. The first k-step starts from the constant 0, the
// following ones accumulate in place; score_settle() then provides the wait
// states (an MFMA of n passes needs about n + 3 before another instruction
// reads its destination; this one takes 4) and names the scores as operands,
// so that no read of them is scheduled above it. The first form's result is
// early-clobber: an MFMA's destination must not overlap its A or B operand.
__device__ __forceinline__ void mfma_score_first(f32x4_t& acc, const bf16x8_t& a, const bf16x8_t& b) {
  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, 0" : "=&v"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_score(f32x4_t& acc, const bf16x8_t& a, const bf16x8_t& b) {
  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void score_settle(f32x4_t (&s)[4]) {
  asm volatile("s_nop 15" : "+v"(s[0]), "+v"(s[1]), "+v"(s[2]), "+v"(s[3]));
}

struct MlaShared {
  char* ring;    // kMlaStages x kMlaStageBytes
  char* pbuf;    // 2 x kMlaPBytes: bf16 weights of tile t in buffer t % 2
  char* xbuf;    // 2 x kMlaXBytes: partial scores of tile t in buffer t % 2
  float* s_norm;  // [128]: normaliser of each head, exchanged at a piece's end
  int* s_vote;    // [4]: replay votes
};

// The tile walker that feeds the DMAs (identical and wave-uniform in every
// wavefront): tiles in order from the worker's first, each giving the address
// of its first row and how many of its 16 rows are inside the shard.
struct MlaWalker {
  int t;           // next tile, relative to the worker's first tile
  int last;        // the worker's last tile (relative): later requests repeat it
  int u;           // unit of tile t
  int uend;        // end of unit u (relative tile index, clamped to the int range)
  int tok, len;    // first token of tile t in the unit's shard, shard length
  int vb, off;     // block-table column and in-block token offset of tile t
  int win_lo;      // the window holds columns win_lo .. win_lo + 63 (-1: none)
  int win;         // this lane's column win_lo + lane
  const int32_t* bt;
  const char* rank_base;
  const char* blk_base;  // base of block vb in the unit's rank pool
  const char* addr;      // first row of the last tile produced
  int nv;                // valid rows of the last tile produced
};

template <int DH>
__device__ __forceinline__ void mla_worker(const AttnParams& p, const MlaShared& sh, int workers, const SplitWs& ws,
                                           int64_t wstart, int64_t wend) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform (SGPR)
  const int hg = wave >> 1;                                          // head group: heads 64 hg .. 64 hg + 63
  const int worker = blockIdx.x;
  const int g4 = lane >> 4, n16 = lane & 15;

  const int bs = p.kv.block_size;
  const int64_t ks0 = p.kv.k_stride[0], ks1 = p.kv.k_stride[1], ks3 = p.kv.k_stride[3];
  const int row_bytes = static_cast<int>(ks3 * 2);
  const uint64_t blk_bytes = static_cast<uint64_t>(ks1) * 2;
  const char* kbase = static_cast<const char*>(p.kv.k);
  const float c2 = p.softmax_scale * DCP_LOG2E;
  const uint32_t ring0 = lds_addr(sh.ring);
  auto stage_of = [&](int64_t t) __attribute__((always_inline)) {
    return static_cast<int>(static_cast<uint32_t>(t - wstart) % kMlaStages);  // tiles per worker < 2^31
  };

  // ---- DMA walker ------------------------------------------------------------------
  // DMA lines of this wavefront: 2 DH + hg + 4 k (k < kDma): wavefronts with
  // DH = 0 load five of the tile's 18 lines of 1 KB, DH = 1 four. Line
  // L = 2 j + hg holds the runs of chunks hg, hg + 2 of k-steps 2 j, 2 j + 1;
  // lane l = 16 s + u writes position u of the line's run s (k-step
  // 2 j + s / 2, chunk hg + 2 (s % 2)), i.e. row u ^ ring_swz(chunk). The
  // k-steps' 64-byte column offset 128 j = 64 (2 DH + 4 k) is the DMA's
  // immediate offset.
  constexpr int kDma = DH == 0 ? 5 : 4;
  const int dma_first = 2 * DH + hg;
  const int dma_row = n16 ^ ring_swz(hg + 2 * (g4 & 1));
  const uint32_t dma_col = static_cast<uint32_t>(64 * (g4 >> 1) + 32 * (g4 & 1) + 16 * hg);
  auto rel_end = [&](int64_t e) __attribute__((always_inline)) {
    return static_cast<int>(min(e - wstart, static_cast<int64_t>(INT32_MAX)));
  };
  MlaWalker dw;
  auto win_load = [&](int vb) __attribute__((always_inline)) {
    dw.win_lo = vb;
    dw.win = vb + lane < p.max_vblocks ? dw.bt[vb + lane] : 0;
    wait_vmcnt<0>();  // the window is needed now (rare: per unit or per 64 blocks)
  };
  auto set_block = [&]() __attribute__((always_inline)) {
    if (dw.vb - dw.win_lo >= 64 || dw.win_lo < 0) win_load(dw.vb);  // uniform
    const uint32_t blk = static_cast<uint32_t>(__builtin_amdgcn_readlane(dw.win, dw.vb - dw.win_lo));
    dw.blk_base = dw.rank_base + static_cast<uint64_t>(blk) * blk_bytes;
  };
  // enter unit u at relative tile dw.t (the unit spans tiles [ubeg, uend))
  auto set_unit = [&](int u, int64_t ubeg, int64_t uend) __attribute__((always_inline)) {
    dw.u = u;
    dw.uend = rel_end(uend);
    const int rb = u / p.q_len, qi = u - rb * p.q_len;
    const int b = rb % p.batch, r = rb / p.batch;
    dw.len = ld_uniform(p.local_lens + (static_cast<int64_t>(b) * p.q_len + qi) * p.dcp_size + p.rank_begin + r);
    dw.bt = p.block_table + static_cast<int64_t>(b) * p.bt_stride;
    dw.rank_base = kbase + static_cast<int64_t>(r) * ks0 * 2;
    dw.tok = static_cast<int>(wstart + dw.t - ubeg) * kMlaTile;
    dw.vb = dw.tok / bs;
    dw.off = dw.tok - dw.vb * bs;
    dw.win_lo = -1;
    set_block();
  };
  // position the walker at relative tile t, searching units forward from u
  auto walker_at = [&](int t, int64_t u) __attribute__((always_inline)) {
    int64_t ubeg = ld_uniform(ws.prefix + u), uend = ld_uniform(ws.prefix + u + 1);
    while (uend <= wstart + t) {  // uniform
      ++u;
      ubeg = uend;
      uend = ld_uniform(ws.prefix + u + 1);
    }
    dw.t = t;
    dw.last = static_cast<int>(wend - 1 - wstart);
    set_unit(static_cast<int>(u), ubeg, uend);
  };
  // The walker's next tile (the last tile again once the worker's run out).
  auto next_tile = [&]() __attribute__((always_inline)) {
    if (dw.t > dw.last) return;  // uniform: keep the last tile's addr / nv
    if (dw.t >= dw.uend) {       // uniform, rare: the next non-empty unit
      int64_t ubeg = wstart + dw.uend, uend;
      int u = dw.u;
      for (;;) {
        ++u;
        uend = ld_uniform(ws.prefix + u + 1);
        if (uend > ubeg) break;
      }
      set_unit(u, ubeg, uend);
    }
    dw.addr = dw.blk_base + static_cast<uint32_t>(dw.off * row_bytes);
    dw.nv = min(kMlaTile, dw.len - dw.tok);
    ++dw.t;
    dw.tok += kMlaTile;
    dw.off += kMlaTile;
    if (dw.off == bs && dw.t <= dw.last && dw.t < dw.uend) {  // uniform: the next tile opens a block
      dw.off = 0;
      ++dw.vb;
      set_block();
    }
  };
  // DMAs of the walker's next tile into stage s
  auto dma_tile = [&](int s) __attribute__((always_inline)) {
    next_tile();
    const uint32_t voff = static_cast<uint32_t>(min(dma_row, dw.nv - 1) * row_bytes) + dma_col;
    const uint32_t m0 = ring0 + s * kMlaStageBytes + dma_first * 1024;
    static_for<kDma>([&](auto kc) __attribute__((always_inline)) {
      constexpr int k = decltype(kc)::value;
      dma16<64 * (2 * DH + 4 * k)>(voff, dw.addr, m0 + 4096 * k);
    });
  };
  // (Re)start the ring at tile t (unit u): load tiles t .. t + ahead - 1 and
  // wait until tile t has landed everywhere.
  auto restart = [&](int64_t t, int64_t u) __attribute__((always_inline)) {
    walker_at(static_cast<int>(t - wstart), u);
    static_for<kMlaAhead>([&](auto jc) __attribute__((always_inline)) {
      dma_tile(stage_of(t + decltype(jc)::value));
    });
    wait_vmcnt<(kMlaAhead - 1) * kDma>();
    block_sync();
  };

  // ---- per-lane LDS offsets -----------------------------------------------------------
  // score operand (A of the 16x16x32 MFMA): token n16, dims 32 ks + 8 g4 .. +7,
  // at koff + ring_run(9 DH + ks, 0)
  const int koff = ring_run(0, g4) + 16 * (n16 ^ ring_swz(g4));
  // value operand (A of the 32x32x16 MFMA) of dim tile mt (k-step 4 w + mt)
  // through two transposing reads rd: lane l addresses token 8 (g4 / 2) + 4 rd
  // + n16 / 4, dims 16 (g4 % 2) + 4 (l % 4) .. +3 of the k-step, and receives
  // dim 32 mt + l % 32, tokens 8 (l / 32) + 4 rd .. +3; at voff[rd] +
  // ring_run(mt, 0) (ring_run(4 w + mt, c) = ring_run(4 w, c) + ring_run(mt, 0))
  int voff[2];
#pragma unroll
  for (int rd = 0; rd < 2; ++rd) {
    const int T = 8 * (g4 >> 1) + 4 * rd + (n16 >> 2), cc = 2 * (g4 & 1) + ((lane & 3) >> 1);
    voff[rd] = ring_run(kMlaDvTiles * wave, cc) + 16 * (T ^ ring_swz(cc)) + 8 * (lane & 1);
  }
  // Weight buffer: the B operand of N-tile nt for lane l (head 32 nt + l % 32,
  // tokens 8 (l / 32) .. +7) at 256 nt + quad_off(l). This wavefront writes
  // N-tile nt_mine = 2 hg + DH, each lane its reader's 16 bytes (after a swap
  // of 16-lane rows, see store_weights).
  const int nt_mine = 2 * hg + DH;
  const int quad = quad_off(lane);
  const int pw_off = 256 * nt_mine + quad;

  const int64_t w_unit0 = ld_uniform(ws.wunit + worker);
  restart(wstart, w_unit0);

  int64_t cur_u = w_unit0;  // unit of the tile being computed
  int64_t tile = wstart;
  float m_hint[2] = {-INFINITY, -INFINITY};  // reference for a replayed piece (this lane's two heads)
  bool replay = false;                       // the current piece is a replay (at most one per piece)

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

    // Q operand (B of the score MFMA) of k-step ks, head tile ht: head
    // 64 hg + 16 ht + n16, dims 288 DH + 32 ks + 8 g4 .. +7
    bf16x8_t qop[kMlaKSteps][4];
    {
      const uint16_t* qb = reinterpret_cast<const uint16_t*>(p.q) +
                           ((static_cast<int64_t>(b) * p.q_len + qi) * kMlaHeads + 64 * hg + n16) * kMlaDk +
                           288 * DH + 8 * g4;
#pragma unroll
      for (int ks = 0; ks < kMlaKSteps; ++ks)
#pragma unroll
        for (int ht = 0; ht < 4; ++ht)
          qop[ks][ht] = *reinterpret_cast<const bf16x8_t*>(qb + 16 * kMlaDk * ht + 32 * ks);
    }
    // Q is complete here, so no wait for it lands inside the tile loop (where
    // it would also drain the tiles in flight).
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_sched_barrier(0);

    // ---- piece state ------------------------------------------------------------------
    // This lane's two heads (i = 0, 1): 64 hg + 32 DH + 16 i + n16. Weights are
    // exp2(s c2 - m_ref[i]); mx[i] tracks the largest exponent for the replay vote.
    float m_ref[2] = {m_hint[0], m_hint[1]};
    float mx[2] = {-INFINITY, -INFINITY}, esum[2] = {0.f, 0.f}, lsum[2] = {0.f, 0.f};
    bool need_ref = !replay;  // uniform
    // O^T[dim, head] of M-tile mt, N-tile nt (o[4 mt + nt]): lane l holds head
    // 32 nt + l % 32, dims 128 wave + 32 mt + 8 (r / 4) + 4 (l / 32) + r % 4
    f32x16_t o[kMlaDvTiles * kMlaHeadTiles];
#pragma unroll
    for (int i = 0; i < kMlaDvTiles * kMlaHeadTiles; ++i) o[i] = f32x16_t{};

    // ---- pipeline ------------------------------------------------------------------------------
    f32x4_t s[4];   // partial scores: token 4 g4 + j, head 64 hg + 16 ht + n16
    bf16x8_t kf[kMlaKAhead + 1];  // K operands, read kMlaKAhead k-steps (six MFMAs each) ahead
    auto kread = [&](const char* st, int ks) __attribute__((always_inline)) {
      kf[ks % (kMlaKAhead + 1)] = *reinterpret_cast<const bf16x8_t*>(st + koff + ring_run(9 * DH + ks, 0));
    };
    // send the partner its heads' partial scores (head tiles 2 (1 - DH), +1):
    // wavefront w's part i at 4 KB (w / 2) + 256 (2 (w % 2) + i) + quad_off(l)
    auto send = [&](char* xb) __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
        *reinterpret_cast<f32x4_t*>(xb + 4096 * hg + 256 * (2 * DH + i) + quad) = s[2 * (1 - DH) + i];
    };
    f32x4_t rcv[2];
    auto receive = [&](const char* xb) __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
        rcv[i] = *reinterpret_cast<const f32x4_t*>(xb + 4096 * hg + 256 * (2 * (1 - DH) + i) + quad);
    };

    // softmax of this lane's 8 scores of the tile being normalised (sf: head i,
    // token 4 g4 + j), one element e = 4 i + j at a time in three parts so that
    // the stream can spread them between MFMAs; on the last tile of the unit
    // tokens >= len are masked after scaling (only a step without a next tile
    // can hold it)
    f32x4_t sf[2];
    uint32_t pw[2][2];
    float xe[8];
    auto soft_a = [&](int e, int tok0, bool last, auto mask_c) __attribute__((always_inline)) {
      const int i = e >> 2, j = e & 3;
      xe[e] = fmaf(sf[i][j], c2, -m_ref[i]);
      if constexpr (decltype(mask_c)::value) {
        if (last && tok0 + 4 * g4 + j >= len) xe[e] = -INFINITY;
      }
      mx[i] = fmaxf(mx[i], xe[e]);
    };
    auto soft_b = [&](int e) __attribute__((always_inline)) {
      xe[e] = __builtin_amdgcn_exp2f(xe[e]);  // v_exp_f32; results below 2^-126 flush to 0
      esum[e >> 2] += xe[e];
    };
    auto soft_c = [&](int e) __attribute__((always_inline)) {  // e odd: pack elements e - 1, e
      const int i = e >> 2, q = (e & 3) >> 1;
      const bf16x2_t pk = bf16x2_t{static_cast<__bf16>(xe[e - 1]), static_cast<__bf16>(xe[e])};
      pw[i][q] = __builtin_bit_cast(uint32_t, pk);
      lsum[i] = __builtin_amdgcn_fdot2_f32_bf16(pk, bf16x2_t{__bf16(1.f), __bf16(1.f)}, lsum[i], false);
    };
    auto set_ref = [&](int tok0, bool last) __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        float mt = -INFINITY;
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (!(last && tok0 + 4 * g4 + j >= len)) mt = fmaxf(mt, sf[i][j] * c2);
        mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
        m_ref[i] = fmaxf(mt, __shfl_xor(mt, 32, 64));
      }
    };
    // A lane holds tokens 4 g4 .. +3 of its two heads i (16 i + n16 of the
    // N-tile); the reader lane wants 8 consecutive tokens of one head. Swapping
    // 16-lane rows (odd rows of head 0's words with even rows of head 1's)
    // leaves lane l with head (l / 16) % 2, tokens 8 (l / 32) .. +7: exactly
    // reader lane l's operand, stored with one 128-bit write.
    auto store_weights = [&](char* pb) __attribute__((always_inline)) {
      u32x4_t v;
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const auto sw = __builtin_amdgcn_permlane16_swap(pw[0][q], pw[1][q], false, false);
        v[q] = sw[0];
        v[2 + q] = sw[1];
      }
      *reinterpret_cast<u32x4_t*>(pb + pw_off) = v;
    };

    // value operands: weights of every head (B, pbv[nt]) and V^T of dim tile mt
    // (A, through two transposing reads into va[mt % 2])
    s16x4_t va[2][2];
    bf16x8_t pbv[kMlaHeadTiles];
    auto vread = [&](const char* st, int mt) __attribute__((always_inline)) {
#pragma unroll
      for (int rd = 0; rd < 2; ++rd)
        va[mt & 1][rd] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(st + voff[rd] + ring_run(mt, 0)));
    };

    // One MFMA stream over the 9 score k-steps: the score MFMAs of the next
    // tile (kNext: four per k-step, one per head tile), the value MFMAs of the
    // previous tile (kPrev: two per k-step, dim tile ks / 2 with head tiles
    // 2 (ks % 2) and + 1) and the softmax of the current tile (kSoft: element ks
    // of this lane's eight). With one wavefront per SIMD the instructions issue
    // in order, so the stream is written MFMA by MFMA with a small group of
    // other instructions (operand reads, softmax parts) after each, pinned by
    // scheduling barriers: they issue while the MFMA before them runs.
    // Interleaving the two products also keeps every score accumulator's next
    // MFMA several MFMAs behind the last one.
    // The stream's first operands, issued before the step's other LDS traffic
    // (the K operand of the first score MFMA first: LDS reads return in order)
    auto stream_pre = [&](auto next_c, auto prev_c, const char* stn, const char* stp, const char* pbp)
        __attribute__((always_inline)) {
      if constexpr (decltype(next_c)::value)
#pragma unroll
        for (int j = 0; j < kMlaKAhead; ++j) kread(stn, j);
      if constexpr (decltype(prev_c)::value) {
#pragma unroll
        for (int nt = 0; nt < kMlaHeadTiles; ++nt)
          pbv[nt] = *reinterpret_cast<const bf16x8_t*>(pbp + 256 * nt + quad);
        vread(stp, 0);
      }
    };
    auto stream = [&](auto next_c, auto prev_c, auto soft_c_, const char* stn, const char* stp, const char* pbp,
                      int tok0, bool last, char* pbw) __attribute__((always_inline)) {
      constexpr bool kNext = decltype(next_c)::value, kPrev = decltype(prev_c)::value;
      constexpr bool kSoft = decltype(soft_c_)::value;
      const std::bool_constant<!kNext> mask_c{};
      auto score_mfma = [&](int ks, int ht) __attribute__((always_inline)) {
        if (ks == 0)
          mfma_score_first(s[ht], kf[0], qop[0][ht]);
        else
          mfma_score(s[ht], kf[ks % (kMlaKAhead + 1)], qop[ks][ht]);
      };
      static_for<kMlaKSteps>([&](auto ksc) __attribute__((always_inline)) {
        constexpr int ks = decltype(ksc)::value;
        constexpr bool kVal = kPrev && ks < 2 * kMlaDvTiles;
        constexpr bool kSm = kSoft && ks < 8;
        constexpr int mt = ks / 2, nt0 = 2 * (ks % 2);
        bf16x8_t a;
        if constexpr (kVal)
          a = __builtin_bit_cast(bf16x8_t,
                                 __builtin_shufflevector(va[mt & 1][0], va[mt & 1][1], 0, 1, 2, 3, 4, 5, 6, 7));
        if constexpr (kNext) score_mfma(ks, 0);
        if constexpr (kNext && ks + kMlaKAhead < kMlaKSteps) kread(stn, ks + kMlaKAhead);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (kVal) mfma_acc(o[kMlaHeadTiles * mt + nt0], a, pbv[nt0]);
        if constexpr (kVal && ks % 2 == 0 && mt + 1 < kMlaDvTiles) vread(stp, mt + 1);
        if constexpr (kSm) soft_a(ks, tok0, last, mask_c);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (kNext) score_mfma(ks, 1);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (kNext) score_mfma(ks, 2);
        if constexpr (kSm) soft_b(ks);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (kVal) mfma_acc(o[kMlaHeadTiles * mt + nt0 + 1], a, pbv[nt0 + 1]);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (kNext) score_mfma(ks, 3);
        if constexpr (kSm && (ks & 1)) soft_c(ks);
        // the weights are final after the last softmax part: stored under the last score MFMAs
        if constexpr (kSoft && ks == kMlaKSteps - 1) store_weights(pbw);
        __builtin_amdgcn_sched_barrier(0);
      });
      if constexpr (kNext) score_settle(s);
    };

    // Step t (after the barrier that ends step t - 1): the partner's partial of
    // tile t, the DMA of tile t + ahead into the stage of tile t - 2, then one
    // stream with the scores of tile t + 1 (if in the piece), the values of tile
    // t - 1 (if in the piece) and the softmax of tile t, tile t's weights to
    // buffer t % 2 (in the stream), tile t + 1's partial scores to the partner, and the barrier
    // (after this wave's DMAs of tile t + 2 have landed).
    auto step = [&](int64_t t, auto next_c, auto prev_c) __attribute__((always_inline)) {
      constexpr bool kNext = decltype(next_c)::value;
      const char* stn = sh.ring + stage_of(t + 1) * kMlaStageBytes;
      const char* stp = sh.ring + stage_of(t - 1) * kMlaStageBytes;
      const char* pbp = sh.pbuf + kMlaPBytes * ((t - 1) & 1);
      stream_pre(next_c, prev_c, stn, stp, pbp);
      receive(sh.xbuf + kMlaXBytes * (t & 1));
      dma_tile(stage_of(t + kMlaAhead));
      const int tok0 = static_cast<int>(t - ubeg) * kMlaTile;
      const bool last = tok0 + kMlaTile > len;  // uniform
#pragma unroll
      for (int i = 0; i < 2; ++i) sf[i] = s[2 * DH + i] + rcv[i];
      if (need_ref) {  // uniform: the piece's first tile
        set_ref(tok0, last);
        need_ref = false;
      }
      stream(next_c, prev_c, std::true_type{}, stn, stp, pbp, tok0, last, sh.pbuf + kMlaPBytes * (t & 1));
      if constexpr (kNext) send(sh.xbuf + kMlaXBytes * ((t + 1) & 1));
      // this wave's DMAs of tile t + 2 are done once at most those of the three
      // later tiles are in flight
      wait_vmcnt<(kMlaAhead - 2) * kDma>();
      wait_lgkm0();
      block_sync();
    };

    // prologue: the scores of the piece's first tile, sent to the partner
    stream_pre(std::true_type{}, std::false_type{}, sh.ring + stage_of(tile) * kMlaStageBytes, nullptr, nullptr);
    stream(std::true_type{}, std::false_type{}, std::false_type{}, sh.ring + stage_of(tile) * kMlaStageBytes, nullptr,
           nullptr, 0, false, nullptr);
    send(sh.xbuf + kMlaXBytes * (tile & 1));
    wait_vmcnt<(kMlaAhead - 2) * kDma>();  // tile + 1, which step `tile` reads
    wait_lgkm0();
    block_sync();
    if (piece_end - tile == 1) {  // uniform
      step(tile, std::false_type{}, std::false_type{});
    } else {
      step(tile, std::true_type{}, std::false_type{});
      for (int64_t t = tile + 1; t < piece_end - 1; ++t) step(t, std::true_type{}, std::true_type{});
      step(piece_end - 1, std::false_type{}, std::true_type{});
    }
    // the last tile's values
    {
      const char* stp = sh.ring + stage_of(piece_end - 1) * kMlaStageBytes;
      const char* pbp = sh.pbuf + kMlaPBytes * ((piece_end - 1) & 1);
      stream_pre(std::false_type{}, std::true_type{}, nullptr, stp, pbp);
      stream(std::false_type{}, std::true_type{}, std::false_type{}, nullptr, stp, pbp, 0, false, nullptr);
    }
    tile = piece_end;

    // ---- replay vote (block-uniform) and normalisers ---------------------------------------
    // Sums over the four lane groups holding the other tokens of each head.
    float lt[2], et[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      lt[i] = lsum[i] + __shfl_xor(lsum[i], 16, 64);
      lt[i] += __shfl_xor(lt[i], 32, 64);
      et[i] = esum[i] + __shfl_xor(esum[i], 16, 64);
      et[i] += __shfl_xor(et[i], 32, 64);
    }
    const int wave_bad = __any(mx[0] > kMlaRefSlack || mx[1] > kMlaRefSlack) ? 1 : 0;
    if (lane == 0) sh.s_vote[wave] = wave_bad;
    if (lane < 16) {
      sh.s_norm[32 * nt_mine + lane] = lt[0];
      sh.s_norm[32 * nt_mine + 16 + lane] = lt[1];
    }
    wait_lgkm0();
    block_sync();
    int any_bad = 0;
#pragma unroll
    for (int w = 0; w < kMlaWaves; ++w) any_bad |= sh.s_vote[w];
    float inv[kMlaHeadTiles];  // 1 / normaliser of head 32 nt + l % 32
#pragma unroll
    for (int nt = 0; nt < kMlaHeadTiles; ++nt) inv[nt] = 1.f / sh.s_norm[32 * nt + (lane & 31)];
    wait_lgkm0();
    block_sync();  // every wave has read votes and normalisers before they are written again
    // One replay always suffices for finite scores (its reference is the
    // largest scaled score of the piece); a second vote can only come from
    // non-finite inputs, which then simply propagate.
    if (any_bad && !replay) {
      replay = true;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        float ms = mx[i] + m_ref[i];
        ms = fmaxf(ms, __shfl_xor(ms, 16, 64));
        m_hint[i] = fmaxf(ms, __shfl_xor(ms, 32, 64));
      }
      wait_vmcnt<0>();
      block_sync();
      tile = piece_tile0;
      cur_u = w_unit0;
      restart(piece_tile0, cur_u);
      continue;
    }
    replay = false;
    m_hint[0] = m_hint[1] = -INFINITY;

    // ---- piece end --------------------------------------------------------------------------
    // O rows: this wave's dims of every head; LSE / (m_ref, normaliser, weight
    // sum): this wave's 32 heads (lanes 0..15, heads 16 i + lane of tile nt_mine).
    const bool whole = (lt_lo == 0) && (lt_hi == uend - ubeg);
    const int which = (lt_lo == 0) ? 1 : 0;  // 0: the unit began before this worker
    const int dim0 = kMlaDvTiles * 32 * wave + 4 * (lane >> 5);
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
      if (lane < 16) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
          p.out_lse[row0 + 32 * nt_mine + 16 * i + lane] = (m_ref[i] + __log2f(et[i])) * DCP_LN2;
      }
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
      if (lane < 16) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          float* dst = part + (32 * nt_mine + 16 * i + lane) * (kMlaDv + kPartExtra);
          dst[kMlaDv] = m_ref[i];
          dst[kMlaDv + 1] = lt[i];
          dst[kMlaDv + 2] = et[i];
        }
      }
    }
  }
  wait_vmcnt<0>();  // refills issued past the last tile still write this workgroup's LDS
}

__global__ void __attribute__((amdgpu_flat_work_group_size(kMlaThreads, kMlaThreads), amdgpu_waves_per_eu(1, 1)))
mla_attn_kernel(AttnParams p, int workers) {
  __shared__ __attribute__((aligned(16))) char ring[kMlaStages * kMlaStageBytes];
  __shared__ __attribute__((aligned(16))) char pbuf[2 * kMlaPBytes];
  __shared__ __attribute__((aligned(16))) char xbuf[2 * kMlaXBytes];
  __shared__ float s_norm[kMlaHeads];
  __shared__ int s_vote[kMlaWaves];
  const int worker = blockIdx.x;
  const int64_t U = split_units(p);
  SplitWs ws = split_ws(p.workspace, workers, U);
  const int64_t T = ld_uniform(ws.prefix + U);
  if (T == 0 || worker >= workers) return;
  const int64_t tpw = (T + workers - 1) / workers;
  const int64_t wstart = static_cast<int64_t>(worker) * tpw;
  if (wstart >= T) return;
  const int64_t wend = min(T, wstart + tpw);
  const MlaShared sh{ring, pbuf, xbuf, s_norm, s_vote};
  if ((threadIdx.x >> 6) & 1)
    mla_worker<1>(p, sh, workers, ws, wstart, wend);
  else
    mla_worker<0>(p, sh, workers, ws, wstart, wend);
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
bool mla_supported(const AttnParams& p) {
  const dcp_kv_cache_t& kv = p.kv;
  if (p.q_dtype != DCP_BF16 || kv.dtype != DCP_BF16) return false;
  if (kv.v != nullptr || kv.num_kv_heads != 1 || p.num_q_heads != kMlaHeads) return false;
  if (kv.head_dim_k != kMlaDk || kv.head_dim_v != kMlaDv) return false;
  if (kv.block_size % kMlaTile != 0) return false;
  if (kv.k_stride[4] != 1) return false;
  for (int i = 0; i < 4; ++i)
    if ((kv.k_stride[i] * 2) % 16 != 0) return false;
  if (reinterpret_cast<uintptr_t>(kv.k) % 16) return false;
  // offsets within a block in 31 bits (a row offset is a 32-bit lane offset)
  if (static_cast<int64_t>(kv.block_size) * kv.k_stride[3] * 2 >= (int64_t(1) << 31)) return false;
  if (static_cast<int64_t>(p.rank_count) * p.batch * p.q_len >= (int64_t(1) << 31)) return false;
  if (p.tpu != 1) return false;  // one query token per unit
  return true;
}

// One persistent workgroup per CU; the workspace is sized for that many.
static int mla_workers() { return min(kMlaMaxWorkers, device_cu_count()); }

size_t mla_workspace_bytes(const AttnParams& p) {
  return split_ws_bytes(mla_workers(), split_units_host(p), kMlaHeads, kMlaDv);
}

hipError_t launch_mla_attn(const AttnParams& p) {
  const int workers = mla_workers();
  launch_split_plan(p, kMlaTile, workers);
  if (p.ev_begin) (void)hipEventRecord(p.ev_begin, p.stream);
  hipLaunchKernelGGL(mla_attn_kernel, dim3(workers), dim3(kMlaThreads), 0, p.stream, p, workers);
  if (p.ev_end) (void)hipEventRecord(p.ev_end, p.stream);
  launch_split_combine<kMlaDv>(p, kMlaTile, workers, split_units_host(p));
  return hipGetLastError();
}

}  // namespace dcp
