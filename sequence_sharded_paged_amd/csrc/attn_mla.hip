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
// Work split: stream-K over (rank, request) units (splitkv.h), one persistent
// 256-thread workgroup per worker, tiles of 32 tokens. Per workgroup:
//   * a 3-stage LDS ring of 32-token tiles (36 KB each) is filled straight
//     from HBM with global_load_lds_dwordx4; the 16-byte chunks of a row are
//     XOR-swizzled by the row index so the MFMA operand reads spread over the
//     LDS banks. Waits are explicit vmcnt counts plus raw s_barrier, so two
//     tiles stay in flight while the third is consumed;
//   * each of the 4 wavefronts owns 32 query heads: its Q (32 x 576 bf16, 144
//     VGPRs) and its O accumulator (32 x 512 fp32, 256 AGPRs) stay in
//     registers for the whole piece;
//   * scores S^T[token, head] = K[token, :] . Q[head, :] on 16x16x32 bf16
//     MFMA, K rows read from LDS with ds_read_b128 (one read feeds both head
//     tiles);
//   * softmax weights in log2 units relative to a per-piece reference max
//     (no rescaling of the 256-register accumulator inside the loop; a piece
//     whose scores outgrow the reference by more than 2^64 is replayed with a
//     higher reference), rounded to bf16 for the value product, with an fp32
//     sum for the LSE (as in the GQA kernel);
//   * values O^T[dim, head] += V^T[dim, token] . P^T[token, head]; V^T comes
//     from the same LDS rows through ds_read_b64_tr_b16, whose 16-lane
//     transpose hands each lane four consecutive tokens of one dimension, so
//     no second copy of the tile is needed.
#include "splitkv.h"

namespace dcp {

constexpr int kMlaDk = 576;
constexpr int kMlaDv = 512;
constexpr int kMlaHeads = 128;
constexpr int kMlaTile = 32;                                     // tokens per tile
#ifndef DCP_MLA_STAGES
#define DCP_MLA_STAGES 4
#endif
constexpr int kMlaStages = DCP_MLA_STAGES;                       // LDS ring depth (tiles in flight + 1)
constexpr int kMlaRowBytes = kMlaDk * 2;                         // 1152
constexpr int kMlaStageBytes = kMlaTile * kMlaRowBytes;          // 36864
constexpr int kMlaLatBytes = kMlaDv * 2;                         // 1024: latent part of a row (also V)
constexpr int kMlaRopeOff = kMlaTile * kMlaLatBytes;             // 32768: rope rows follow the latent rows
constexpr int kMlaRopeBytes = kMlaRowBytes - kMlaLatBytes;       // 128
#ifndef DCP_MLA_WAVES
#define DCP_MLA_WAVES 4
#endif
constexpr int kMlaWaves = DCP_MLA_WAVES;                         // wavefronts per workgroup (4 or 8)
constexpr int kMlaThreads = 64 * kMlaWaves;
constexpr int kMlaHeadsPerWave = kMlaHeads / kMlaWaves;          // 32 or 16
constexpr int kMlaHT = kMlaHeadsPerWave / 16;                    // 16-head MFMA tiles per wavefront
constexpr int kMlaLatRowsPerWave = kMlaTile / kMlaWaves;         // latent rows loaded per wave and tile
constexpr int kMlaKSteps = kMlaDk / 32;                          // 18
#ifndef DCP_MLA_QREG
#define DCP_MLA_QREG 16
#endif
#ifndef DCP_MLA_KPF
#define DCP_MLA_KPF 1
#endif
#ifndef DCP_MLA_VPF
#define DCP_MLA_VPF 1
#endif
constexpr int kMlaKStepsReg = DCP_MLA_QREG;                      // k-steps of Q kept in VGPRs; the rest in LDS
constexpr int kMlaKPf = DCP_MLA_KPF;                             // score-operand read distance (k-steps)
constexpr int kMlaVPf = DCP_MLA_VPF;                             // value-operand read distance (tiles)
constexpr int kMlaQLdsSteps = kMlaKSteps - kMlaKStepsReg;        // k-steps of Q held in LDS
constexpr int kMlaQRopeWaveBytes = kMlaHT * kMlaQLdsSteps * 64 * 16;  // per wave
constexpr int kMlaDvTiles = kMlaDv / 16;                         // 32
constexpr int kMlaMaxWorkers = 512;
constexpr float kMlaRefSlack = 64.f;  // log2 units a tile max may exceed the piece's reference

static_assert(kMlaWaves == 4 || kMlaWaves == 8, "4 or 8 wavefronts");
static_assert(kMlaKStepsReg % 4 == 0 && kMlaKStepsReg <= 16, "latent k-steps in registers");

typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

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

// Workgroup barrier without the memory fence of __syncthreads (which would
// wait for every tile in flight); the asm memory clobber keeps the compiler
// from moving LDS accesses across it.
__device__ __forceinline__ void block_sync() { asm volatile("s_barrier" ::: "memory"); }

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) char*)p));
}

// Chunk swizzles. A latent row holds 64 16-byte chunks; chunk c of row r sits
// at slot c ^ lat_swz(r). lat_swz is a bijection of r & 15 whose bits 1..3
// carry r & 7: the 16 rows of a score-operand read (same chunk) land on 16
// distinct slots mod 16, and the 4 rows x 2 chunks of a transpose read as
// well. Rope rows (8 chunks) use chunk ^ (r & 7).
__device__ __forceinline__ int lat_swz(int row) { return ((row & 7) << 1) | ((row >> 3) & 1); }
__device__ __forceinline__ int rope_swz(int row) { return row & 7; }

__global__ void __attribute__((amdgpu_flat_work_group_size(kMlaThreads, kMlaThreads),
                               amdgpu_waves_per_eu(kMlaWaves / 4, kMlaWaves / 4)))
mla_attn_kernel(AttnParams p, int workers) {
  __shared__ __attribute__((aligned(16))) char lds[kMlaStages * kMlaStageBytes];
  // rope part of Q in operand order: [wave][ks - 16][lane] x 16 bytes
  __shared__ __attribute__((aligned(16))) char qrope[kMlaWaves * kMlaQRopeWaveBytes];
  // The replay vote of wave w lives in the first 4 bytes of w's own Q slice:
  // by the time a wave votes it no longer reads its slice, and the slice is
  // refilled only after every wave has read the votes.
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
  const char* kbase = static_cast<const char*>(p.kv.k);
  const float c2 = p.softmax_scale * DCP_LOG2E;
  const bool rope_loader = wave < 4;   // waves 0..3 also load the rope rows (8 rows each)
  (void)rope_loader;

  // ---- tile prefetch (uniform control flow) --------------------------------
  int64_t pf_u = ld_uniform(ws.wunit + worker);
  int64_t pf_t = wstart;
  auto issue = [&](int stage) {
    while (ld_uniform(ws.prefix + pf_u + 1) <= pf_t) ++pf_u;
    const int lt = static_cast<int>(pf_t - ld_uniform(ws.prefix + pf_u));
    const int uu = static_cast<int>(pf_u);
    const int b = uu % p.batch, r = uu / p.batch;
    const int len = ld_uniform(p.local_lens + static_cast<int64_t>(b) * p.dcp_size + p.rank_begin + r);
    const int t0 = lt * kMlaTile;
    const int32_t* bt = p.block_table + static_cast<int64_t>(b) * p.bt_stride;
    // tokens t0..t0+15 share one block and so do t0+16..t0+31 (block_size %
    // 16 == 0); a row past the end re-reads token t0 (finite data, zero weight)
    const int vb_a = t0 / bs, off_a = t0 - vb_a * bs;
    const bool has_b = t0 + 16 < len;
    const int vb_b = has_b ? (t0 + 16) / bs : vb_a;
    const int off_b = has_b ? t0 + 16 - vb_b * bs : off_a;
    const int64_t base_a = ld_uniform(bt + vb_a) * ks1 + static_cast<int64_t>(off_a) * ks3;
    const int64_t base_b = ld_uniform(bt + vb_b) * ks1 + static_cast<int64_t>(off_b) * ks3;
    const char* rank_k = kbase + r * ks0 * 2;
    char* dst = lds + stage * kMlaStageBytes;
    // latent rows: one row per instruction (uniform address), lane = destination slot
#pragma unroll
    for (int k = 0; k < kMlaLatRowsPerWave; ++k) {
      const int row = kMlaLatRowsPerWave * wave + k;
      const int64_t el = (t0 + row < len) ? (row < 16 ? base_a : base_b) + (row & 15) * ks3 : base_a;
      dma16(rank_k + el * 2 + 16 * (lane ^ lat_swz(row)), lds_addr(dst + row * kMlaLatBytes));
    }
    // rope rows 8*wave .. 8*wave+7 (waves 0..3), 8 chunks each
    if (rope_loader) {
      const int row = 8 * wave + (lane >> 3);
      const int64_t el = (t0 + row < len) ? (wave < 2 ? base_a : base_b) + (row & 15) * ks3 : base_a;
      dma16(rank_k + el * 2 + kMlaLatBytes + 16 * ((lane & 7) ^ rope_swz(row)),
            lds_addr(dst + kMlaRopeOff + 8 * wave * kMlaRopeBytes));
    }
    ++pf_t;
  };
  // this thread's DMA count per tile (for the vmcnt waits)
  // waits until this thread's loads of the current tile have landed; `ahead`
  // younger tiles (0 .. stages-2) may stay in flight
  auto wait_tile = [&](int ahead) {
    constexpr int a = kMlaLatRowsPerWave + 1, b = kMlaLatRowsPerWave;
    if (ahead <= 0) wait_vmcnt<0>();
    else if (ahead == 1) { if (rope_loader) wait_vmcnt<a>(); else wait_vmcnt<b>(); }
    else if (ahead == 2 || kMlaStages < 4) { if (rope_loader) wait_vmcnt<2 * a>(); else wait_vmcnt<2 * b>(); }
    else { if (rope_loader) wait_vmcnt<3 * a>(); else wait_vmcnt<3 * b>(); }
  };

  for (int j = 0; j < kMlaStages - 1 && wstart + j < wend; ++j) issue(j);

  int64_t cur_u = ld_uniform(ws.wunit + worker);  // unit of the tile being computed
  int64_t tile = wstart;
  int stage = 0;
  float m_hint[kMlaHT];  // reference for a replayed piece
#pragma unroll
  for (int hh = 0; hh < kMlaHT; ++hh) m_hint[hh] = -INFINITY;
  // per-lane LDS byte offsets (the swizzles only touch the low 4 bits of a
  // chunk index, so the rest of each address is an immediate)
  // score operand, k-step ks: row n, chunk (4ks + g) ^ lat_swz(n) =
  //   koff(ks & 3) + 256 * (ks >> 2) bytes; value operand, tile nt: row tr_row,
  //   chunk (2nt + tr_j / 2) ^ lat_swz(tr_row) = troff(nt & 7) + 256 * (nt >> 3)
  const int kroff = kMlaRopeOff + n * kMlaRopeBytes;
  const int tr_row = 4 * g + (n >> 2);             // LDS row (u = 0) of this lane's transpose read
  const int tr_j = n & 3;
  auto koff = [&](int j) { return n * kMlaLatBytes + 16 * ((4 * j + g) ^ lat_swz(n)); };
  auto troff = [&](int j) {
    return tr_row * kMlaLatBytes + 8 * (tr_j & 1) + 16 * ((2 * j + (tr_j >> 1)) ^ lat_swz(tr_row));
  };
  char* qr = qrope + wave * kMlaQRopeWaveBytes + lane * 16;

  while (tile < wend) {
    while (ld_uniform(ws.prefix + cur_u + 1) <= tile) ++cur_u;
    const int64_t ubeg = ld_uniform(ws.prefix + cur_u), uend = ld_uniform(ws.prefix + cur_u + 1);
    const int64_t lt_lo = tile - ubeg, lt_hi = min(wend, uend) - ubeg;
    const int b = static_cast<int>(cur_u % p.batch);
    const int len = ld_uniform(p.local_lens + static_cast<int64_t>(b) * p.dcp_size + p.rank_begin +
                               static_cast<int>(cur_u / p.batch));

    // Q operand (B of the score MFMA): head 16*wave + n, dims 32*ks + 8*g .. +8;
    // latent k-steps in VGPRs, rope k-steps in this wave's slice of LDS
    bf16x8_t qop[kMlaHT][kMlaKStepsReg];
    {
      const uint16_t* qb = reinterpret_cast<const uint16_t*>(p.q) +
                           (static_cast<int64_t>(b) * kMlaHeads + kMlaHeadsPerWave * wave + n) * kMlaDk + 8 * g;
#pragma unroll
      for (int hh = 0; hh < kMlaHT; ++hh) {
#pragma unroll
        for (int ks = 0; ks < kMlaKStepsReg; ++ks)
          qop[hh][ks] = *reinterpret_cast<const bf16x8_t*>(qb + 16 * hh * kMlaDk + 32 * ks);
#pragma unroll
        for (int ks = kMlaKStepsReg; ks < kMlaKSteps; ++ks)
          *reinterpret_cast<bf16x8_t*>(qr + (hh * (kMlaKSteps - kMlaKStepsReg) + ks - kMlaKStepsReg) * 1024) =
              *reinterpret_cast<const bf16x8_t*>(qb + 16 * hh * kMlaDk + 32 * ks);
      }
    }
    // Q is complete here, so no wait for it lands inside the tile loop (where
    // it would also drain the tiles in flight).
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_sched_barrier(0);

    // The weights of a piece are taken relative to a fixed reference max m_ref
    // (the first tile's max), so the accumulator is never rescaled: weights up
    // to 2^kMlaRefSlack are exact in fp32 / bf16. If any tile's max exceeds the
    // reference by more than that, the workgroup replays the piece with the
    // largest max seen as the reference (m_hint).
    const int64_t piece_tile0 = tile, piece_u0 = cur_u;
    float m_ref[kMlaHT], m_seen[kMlaHT], l[kMlaHT], e[kMlaHT];
    f32x4_t o[kMlaHT][kMlaDvTiles];
#pragma unroll
    for (int hh = 0; hh < kMlaHT; ++hh) {
      m_ref[hh] = m_hint[hh];
      m_seen[hh] = m_hint[hh];
      l[hh] = 0.f;
      e[hh] = 0.f;
#pragma unroll
      for (int nt = 0; nt < kMlaDvTiles; ++nt) o[hh][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    bool bad = false;
    for (int64_t lt = lt_lo; lt < lt_hi; ++lt, ++tile) {
      wait_tile(static_cast<int>(min<int64_t>(wend - 1 - tile, kMlaStages - 2)));
      block_sync();
      if (tile + kMlaStages - 1 < wend) issue(stage == 0 ? kMlaStages - 1 : stage - 1);
      const char* st = lds + stage * kMlaStageBytes;

      // ---- scores S^T[token 16u + 4g + i][head n] ----------------------------
      // The K operand of k-step ks+1 is read before the MFMAs of step ks.
      // per-tile operand bases; everything else of an address is an immediate
      const char* kb[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) kb[j] = st + koff(j);
      const char* krb[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) krb[j] = st + kroff + 16 * ((4 * j + g) ^ rope_swz(n));
      auto kaddr = [&](int ks, int u) -> const char* {
        return ks < kMlaDv / 32 ? kb[ks & 3] + 256 * (ks >> 2) + u * 16 * kMlaLatBytes
                                : krb[ks - kMlaDv / 32] + u * 16 * kMlaRopeBytes;
      };
      f32x4_t s[kMlaHT][2];
#pragma unroll
      for (int hh = 0; hh < kMlaHT; ++hh) s[hh][0] = s[hh][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      bf16x8_t ka[kMlaKPf + 1][2];
#pragma unroll
      for (int j = 0; j < kMlaKPf; ++j) {
        ka[j][0] = *reinterpret_cast<const bf16x8_t*>(kaddr(j, 0));
        ka[j][1] = *reinterpret_cast<const bf16x8_t*>(kaddr(j, 1));
      }
#pragma unroll
      for (int ks = 0; ks < kMlaKSteps; ++ks) {
        if (ks + kMlaKPf < kMlaKSteps) {
          ka[(ks + kMlaKPf) % (kMlaKPf + 1)][0] = *reinterpret_cast<const bf16x8_t*>(kaddr(ks + kMlaKPf, 0));
          ka[(ks + kMlaKPf) % (kMlaKPf + 1)][1] = *reinterpret_cast<const bf16x8_t*>(kaddr(ks + kMlaKPf, 1));
        }
#pragma unroll
        for (int hh = 0; hh < kMlaHT; ++hh) {
          const bf16x8_t bq = ks < kMlaKStepsReg
                                  ? qop[hh][ks < kMlaKStepsReg ? ks : 0]
                                  : *reinterpret_cast<const bf16x8_t*>(
                                        qr + (hh * (kMlaKSteps - kMlaKStepsReg) + ks - kMlaKStepsReg) * 1024);
#pragma unroll
          for (int u = 0; u < 2; ++u)
            s[hh][u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[ks % (kMlaKPf + 1)][u], bq, s[hh][u], 0, 0, 0);
        }
      }

      // ---- softmax weights (log2 units, fixed reference) ----------------------
      const int tok0 = static_cast<int>(lt) * kMlaTile + 4 * g;   // + 16u + i
      const bool partial = static_cast<int>(lt) * kMlaTile + kMlaTile > len;   // uniform
      bf16x8_t pop[kMlaHT];
#pragma unroll
      for (int hh = 0; hh < kMlaHT; ++hh) {
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int i = 0; i < 4; ++i) s[hh][u][i] *= c2;
        if (partial) {
#pragma unroll
          for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (tok0 + 16 * u + i >= len) s[hh][u][i] = -INFINITY;
        }
        float mt = fmaxf(fmaxf(fmaxf(s[hh][0][0], s[hh][0][1]), fmaxf(s[hh][0][2], s[hh][0][3])),
                         fmaxf(fmaxf(s[hh][1][0], s[hh][1][1]), fmaxf(s[hh][1][2], s[hh][1][3])));
        mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
        mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
        m_seen[hh] = fmaxf(m_seen[hh], mt);
        if (m_ref[hh] == -INFINITY) m_ref[hh] = mt;
        bad |= mt > m_ref[hh] + kMlaRefSlack;
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            // v_exp_f32: exact enough for weights, flushes results below 2^-126 to 0
            const float pe = __builtin_amdgcn_exp2f(s[hh][u][i] - m_ref[hh]);
            const __bf16 pb = static_cast<__bf16>(pe);
            pop[hh][4 * u + i] = pb;
            l[hh] += static_cast<float>(pb);
            e[hh] += pe;
          }
      }

      // ---- values O^T[dim 16nt + 4g + i][head n] -------------------------------
      // The two transpose reads of value tile nt+1 are issued before the MFMAs
      // of tile nt.
      s16x4_t vb[kMlaVPf + 1][2];
      const char* tb[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) tb[j] = st + troff(j);
      auto vread = [&](int nt, s16x4_t* dst2) {
        const char* a1 = tb[nt & 7] + 256 * (nt >> 3);
        dst2[0] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(a1));
        dst2[1] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(a1 + 16 * kMlaLatBytes));
      };
#pragma unroll
      for (int j = 0; j < kMlaVPf; ++j) vread(j, vb[j]);
#pragma unroll
      for (int nt = 0; nt < kMlaDvTiles; ++nt) {
        if (nt + kMlaVPf < kMlaDvTiles) vread(nt + kMlaVPf, vb[(nt + kMlaVPf) % (kMlaVPf + 1)]);
        const int cb = nt % (kMlaVPf + 1);
        const bf16x8_t a =
            __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(vb[cb][0], vb[cb][1], 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
        for (int hh = 0; hh < kMlaHT; ++hh)
          o[hh][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pop[hh], o[hh][nt], 0, 0, 0);
      }
      stage = stage == kMlaStages - 1 ? 0 : stage + 1;
    }

    // ---- replay vote (block-uniform) ------------------------------------------
    const int wave_bad = __any(bad) ? 1 : 0;  // every lane takes part in the wave vote
    if (lane == 0) *reinterpret_cast<int*>(qrope + wave * kMlaQRopeWaveBytes) = wave_bad;
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the vote is in LDS before the barrier
    block_sync();
    int any_bad = 0;
#pragma unroll
    for (int w = 0; w < kMlaWaves; ++w) any_bad |= *reinterpret_cast<const int*>(qrope + w * kMlaQRopeWaveBytes);
    block_sync();  // every wave has read the votes before they are written again
    if (any_bad) {
      wait_vmcnt<0>();
      block_sync();
      tile = piece_tile0;
      cur_u = piece_u0;
      pf_t = piece_tile0;
      pf_u = piece_u0;
      stage = 0;
      for (int j = 0; j < kMlaStages - 1 && tile + j < wend; ++j) issue(j);
#pragma unroll
      for (int hh = 0; hh < kMlaHT; ++hh) m_hint[hh] = m_seen[hh];
      continue;
    }
#pragma unroll
    for (int hh = 0; hh < kMlaHT; ++hh) m_hint[hh] = -INFINITY;

    // ---- piece end --------------------------------------------------------------
    const bool whole = (lt_lo == 0) && (lt_hi == uend - ubeg);
    const int which = (lt_lo == 0) ? 1 : 0;  // 0: the unit began before this worker
#pragma unroll
    for (int hh = 0; hh < kMlaHT; ++hh) {
      float lt_ = l[hh] + __shfl_xor(l[hh], 16, 64);
      lt_ += __shfl_xor(lt_, 32, 64);
      float et = e[hh] + __shfl_xor(e[hh], 16, 64);
      et += __shfl_xor(et, 32, 64);
      const int head = kMlaHeadsPerWave * wave + 16 * hh + n;
      if (whole) {
        const int64_t row = cur_u * kMlaHeads + head;
        float* dst = p.out_o + row * kMlaDv + 4 * g;
        const float inv = 1.f / lt_;
#pragma unroll
        for (int nt = 0; nt < kMlaDvTiles; ++nt) *reinterpret_cast<f32x4_t*>(dst + 16 * nt) = o[hh][nt] * inv;
        if (g == 0) p.out_lse[row] = (m_ref[hh] + __log2f(et)) * DCP_LN2;
      } else {
        float* dst =
            ws.part + ((static_cast<int64_t>(worker) * 2 + which) * kMlaHeads + head) * (kMlaDv + kPartExtra);
#pragma unroll
        for (int nt = 0; nt < kMlaDvTiles; ++nt) *reinterpret_cast<f32x4_t*>(dst + 16 * nt + 4 * g) = o[hh][nt];
        if (g == 0) {
          dst[kMlaDv] = m_ref[hh];
          dst[kMlaDv + 1] = lt_;
          dst[kMlaDv + 2] = et;
        }
      }
    }
  }
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
  if (static_cast<int64_t>(p.rank_count) * p.batch >= (int64_t(1) << 31)) return false;
  return true;
}

size_t mla_workspace_bytes(const AttnParams& p) {
  const int64_t U = static_cast<int64_t>(p.rank_count) * p.batch;
  return split_ws_bytes(U, kMlaMaxWorkers, kMlaHeads, kMlaDv);
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
