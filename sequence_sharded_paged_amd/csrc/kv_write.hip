// DCP KV-cache write: new K/V rows stored at their slots on the owning rank.
//
// Source: "Decode Context Parallel (DCP)" (vLLM Ascend design doc), section
// "KV-cache layout" (each rank stores only its local shard, at the slot the
// slot mapping gives); "DeepSeek V4.1 context parallelism" (TokenSpeed design
// note), section "Cache ownership" (a write turns the virtual slot into the
// owner's local slot; non-owners are masked).
//
// Kernels, chosen by batch size, row width and V layout (see each):
//   * kv_scatter_kernel, batches under 1024 tokens (a decode step): one
//     wavefront per (token, KV head), shortest chain of memory accesses;
//   * kv_tokrow_kernel, larger batches whose token rows are 48 .. 64 pieces
//     of 16 elements (GQA K, and V in a row layout): a wavefront per run of
//     tokens, one token at a time across its lanes, 16-byte stores;
//   * kv_rows_kernel, larger batches, other rows (MLA's 576-wide latent,
//     unaligned pools): one wavefront per few tokens (all KV heads), owners
//     found by a ballot over (token, rank) lanes, whole rows loaded and
//     stored with 8-element chunks;
//   * kv_vt_kernel, larger batches, V stored token-contiguous inside a block
//     (the layout the attention kernel reads): 64-token tiles transposed
//     through LDS so that consecutive slots of a block are stored together.
// A token kept on several ranks is written on each of them.
// Stored formats: fp32 as is; bf16 rounded to nearest even; fp8 E4M3 (no
// infinities) nearest to the fp32 quotient x / scale[h], ties to even,
// saturating at 448, NaN -> 0x7F. bf16 rounding is integer code written from
// the format's definition; the fp8 quotient is an fp64 product rounded once
// (exact, see quotient) and its code comes from the hardware conversion.
#include "common.h"

namespace dcp {

constexpr int kSlotBits = 56;          // slots below 2^56 (num_blocks * block_size is checked)

// fp32 quotient x / s, correctly rounded: the fp64 product with r = RN64(1/s)
// rounded once to fp32. The fp64 product is within 2^-52 (relative) of x / s,
// while a quotient of two 24-bit significands is never a midpoint between
// fp32 neighbours and lies at least 2^-49 (relative) away from every such
// midpoint, so both round to the same fp32 number. Zeros, infinities and
// NaNs propagate as in the quotient.
__device__ __forceinline__ float quotient(float x, double r) {
  return static_cast<float>(static_cast<double>(x) * r);
}

// fp32 -> E4M3 codes of eight values: round to nearest, ties to even
// (v_cvt_pk_fp8_f32, OCP E4M3 on gfx950), after clamping to +-448 (v_med3_f32)
// so that larger magnitudes and infinities saturate; NaN -> 0x7F (whatever the
// clamp and the conversion made of a NaN is replaced; a lane takes that branch
// only when one of its eight values is a NaN).
__device__ __forceinline__ void e4m3_codes(const float (&q)[8], uint32_t (&code)[8]) {
  bool any_nan = false;
  float c[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    any_nan |= __builtin_isnan(q[i]);
    c[i] = __builtin_amdgcn_fmed3f(q[i], -448.0f, 448.0f);
  }
#pragma unroll
  for (int i = 0; i < 8; i += 2) {
    const uint32_t w = static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(c[i], c[i + 1], 0, false));
    code[i] = w & 0xffu;
    code[i + 1] = (w >> 8) & 0xffu;
  }
  if (any_nan) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (__builtin_isnan(q[i])) code[i] = 0x7fu;
  }
}

// fp32 -> bf16 bits: round to nearest, ties to even; NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t f32_to_bf16(float x) {
  const uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// Reciprocal of a head's fp8 scale in fp64 (exact division).
__device__ __forceinline__ double scale_rcp(const float* scales, int h) {
  return 1.0 / static_cast<double>(scales[h]);
}

template <int kDst> struct Stored;
template <> struct Stored<DCP_F32> { using T = uint32_t; };
template <> struct Stored<DCP_BF16> { using T = uint16_t; };
template <> struct Stored<DCP_FP8_E4M3> { using T = uint8_t; };

// Eight source elements, raw (bf16: one 16-byte load; fp32: two).
template <bool kSrcBf16>
struct Raw8 {
  uint4 w[kSrcBf16 ? 1 : 2];
};

template <bool kSrcBf16>
__device__ __forceinline__ Raw8<kSrcBf16> load8(const void* src, int64_t elem) {
  Raw8<kSrcBf16> r;
  if constexpr (kSrcBf16) {
    r.w[0] = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(src) + elem);
  } else {
    const uint4* p = reinterpret_cast<const uint4*>(static_cast<const float*>(src) + elem);
    r.w[0] = p[0];
    r.w[1] = p[1];
  }
  return r;
}

// Stored bit patterns of 8 source values (rcp: fp8 only).
template <int kDst, bool kSrcBf16>
__device__ __forceinline__ void convert8(const Raw8<kSrcBf16>& r, double rcp, uint32_t (&q)[8]) {
  float x[8];
  if constexpr (kSrcBf16) {
    const uint32_t w[4] = {r.w[0].x, r.w[0].y, r.w[0].z, r.w[0].w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = __uint_as_float(w[i] << 16);
      x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  } else {
    const uint32_t w[8] = {r.w[0].x, r.w[0].y, r.w[0].z, r.w[0].w, r.w[1].x, r.w[1].y, r.w[1].z, r.w[1].w};
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = __uint_as_float(w[i]);
  }
  if constexpr (kDst == DCP_FP8_E4M3) {
    float y[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) y[i] = quotient(x[i], rcp);
    e4m3_codes(y, q);
  } else if constexpr (kDst == DCP_BF16) {
#pragma unroll
    for (int i = 0; i < 8; ++i) q[i] = f32_to_bf16(x[i]);
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) q[i] = __float_as_uint(x[i]);
  }
}

template <int kDst>
__device__ __forceinline__ void store8(void* pool, int64_t elem, int64_t dim_stride, bool vec,
                                       const uint32_t (&q)[8]) {
  using St = typename Stored<kDst>::T;
  St* dst = static_cast<St*>(pool) + elem;
  if (vec) {
    if constexpr (kDst == DCP_FP8_E4M3) {
      *reinterpret_cast<uint2*>(dst) = uint2{q[0] | (q[1] << 8) | (q[2] << 16) | (q[3] << 24),
                                             q[4] | (q[5] << 8) | (q[6] << 16) | (q[7] << 24)};
    } else if constexpr (kDst == DCP_BF16) {
      *reinterpret_cast<uint4*>(dst) = uint4{q[0] | (q[1] << 16), q[2] | (q[3] << 16), q[4] | (q[5] << 16),
                                             q[6] | (q[7] << 16)};
    } else {
      reinterpret_cast<uint4*>(dst)[0] = uint4{q[0], q[1], q[2], q[3]};
      reinterpret_cast<uint4*>(dst)[1] = uint4{q[4], q[5], q[6], q[7]};
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) dst[i * dim_stride] = static_cast<St>(q[i]);
  }
}

// Sixteen stored values at a 16-byte aligned, contiguous destination.
template <int kDst>
__device__ __forceinline__ void store16(void* pool, int64_t elem, const uint32_t (&q)[16]) {
  using St = typename Stored<kDst>::T;
  uint4* dst = reinterpret_cast<uint4*>(static_cast<St*>(pool) + elem);
  if constexpr (kDst == DCP_FP8_E4M3) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = q[4 * i] | (q[4 * i + 1] << 8) | (q[4 * i + 2] << 16) | (q[4 * i + 3] << 24);
    dst[0] = uint4{w[0], w[1], w[2], w[3]};
  } else if constexpr (kDst == DCP_BF16) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
      dst[i] = uint4{q[8 * i] | (q[8 * i + 1] << 16), q[8 * i + 2] | (q[8 * i + 3] << 16),
                     q[8 * i + 4] | (q[8 * i + 5] << 16), q[8 * i + 6] | (q[8 * i + 7] << 16)};
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) dst[i] = uint4{q[4 * i], q[4 * i + 1], q[4 * i + 2], q[4 * i + 3]};
  }
}

struct KvWriteParams {
  const void* k_new;
  const void* v_new;     // nullptr: no V rows (MLA)
  int64_t num_tokens;
  const int64_t* slots;  // [num_ranks, num_tokens]
  int num_ranks;
  dcp_kv_cache_t kv;
  int vec_k, vec_v;      // 1: the pool's 8-element chunks are contiguous and aligned (vector stores)
  int v_transposed;      // 1: V is token-contiguous inside a block (kv_vt_kernel)
  int vt_quads;          // kv_vt_kernel may store an aligned word of 4 slots as one vector
  int vt_vec16;          // kv_vt16_kernel: 16-byte words of slots stay aligned across heads and dims
  int rank_lanes;        // kv_rows_kernel: lanes per token, a power of two >= num_ranks
};

// One tensor (K, or V in a row layout) for kv_rows_kernel.
struct RowsArgs {
  const void* src;       // [T, H, dim], contiguous
  void* pool;
  int64_t st[5];         // pool strides (rank, block, head, token, dim)
  const float* scale;    // [H], fp8 only
  int dim;
  int vec;               // vector stores of 8-element chunks
  int tpw;               // tokens per wavefront (a power of two, tpw * rank_lanes <= 64)
  uint32_t tok_magic;    // c / (H * dim / 8) = umulhi(c, tok_magic) for the chunk numbers c used here
  uint32_t head_magic;   // c / (dim / 8) = umulhi(c, head_magic)
  int bs_shift;          // kv_tokrow_kernel: log2(block_size), or -1 when it is not a power of two
};

constexpr int kRowsRounds = 9;  // 64-chunk rounds of a wavefront's rows held in registers

// Large batches, rows: a wavefront per tpw consecutive tokens, all KV heads.
// Lane (j, r) = (lane / rank_lanes, lane % rank_lanes) reads token t0 + j's
// slot on rank r and computes the token's row offset there (head 0). The
// tokens' rows, [H, dim] each and contiguous in the source, are cut into
// 8-element chunks spread over the lanes (chunk c: token c / (H * dim / 8),
// then head and dims), all loaded before the slots are needed; each chunk
// takes its token's offset at the first owner from the owning lane (a
// wavefront shuffle). Further owners (a token kept on more than one rank)
// are written in later passes from reloaded rows.
template <int kDst, bool kSrcBf16>
__global__ void __launch_bounds__(256) kv_rows_kernel(KvWriteParams p, RowsArgs a) {
  const int lane = threadIdx.x & 63;
  const int H = p.kv.num_kv_heads;
  const int64_t T = p.num_tokens;
  const int64_t w = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  const int64_t t0 = w * a.tpw;
  if (t0 >= T) return;  // whole wavefronts leave together
  const int ntok = static_cast<int>(T - t0 < a.tpw ? T - t0 : a.tpw);
  const int RL = p.rank_lanes;
  const uint64_t segmask = RL == 64 ? ~uint64_t(0) : (uint64_t(1) << RL) - 1;
  const int cpt = a.dim / 8, cptok = H * cpt, total = ntok * cptok;
  const int64_t cap = static_cast<int64_t>(p.kv.num_blocks) * p.kv.block_size;
  const int64_t row_elems = static_cast<int64_t>(H) * a.dim;  // source elements per token

  const int j = lane / RL, r = lane - j * RL;
  const int64_t slot = (j < ntok && r < p.num_ranks) ? p.slots[r * T + t0 + j] : -1;
  // fp8: lane h holds head h's reciprocal scale (heads past 64: computed per chunk)
  double lane_rcp = 1.0;
  if constexpr (kDst == DCP_FP8_E4M3) {
    if (lane < H) lane_rcp = scale_rcp(a.scale, lane);
  }

  for (int g0 = 0; g0 < total; g0 += 64 * kRowsRounds) {
    const int rounds = (total - g0 + 63) / 64;  // wave-uniform
    Raw8<kSrcBf16> raw[kRowsRounds];
#pragma unroll
    for (int k = 0; k < kRowsRounds; ++k) {
      const int c = g0 + k * 64 + lane;
      if (k < rounds && c < total) raw[k] = load8<kSrcBf16>(a.src, t0 * row_elems + static_cast<int64_t>(c) * 8);
    }
    const bool valid = slot >= 0 && slot < cap;
    int64_t row = -1;
    if (valid) {
      const int64_t blk = slot / p.kv.block_size, off = slot - blk * p.kv.block_size;
      row = r * a.st[0] + blk * a.st[1] + off * a.st[3];
    }
    uint64_t rem = __builtin_amdgcn_ballot_w64(valid);
    for (int pass = 0; rem; ++pass) {  // wave-uniform
      uint64_t first = 0;  // lowest remaining owner of every token
      for (int jj = 0; jj < ntok; ++jj) {
        const uint64_t seg = (rem >> (jj * RL)) & segmask;
        first |= (seg & (~seg + 1)) << (jj * RL);
      }
      rem &= ~first;
#pragma unroll
      for (int k = 0; k < kRowsRounds; ++k) {
        if (k >= rounds) continue;  // wave-uniform
        const int c = g0 + k * 64 + lane;
        const int jc = c < total ? static_cast<int>(__umulhi(static_cast<uint32_t>(c), a.tok_magic)) : 0;
        const uint64_t seg = (first >> (jc * RL)) & segmask;
        const int64_t orow = __shfl(row, jc * RL + (seg ? __builtin_ctzll(seg) : 0), 64);
        double head_rcp = 1.0;  // shuffled while every lane is active
        if constexpr (kDst == DCP_FP8_E4M3) {
          const int ctk = c - jc * cptok;
          const int hk = static_cast<int>(__umulhi(static_cast<uint32_t>(ctk), a.head_magic));
          if (H <= 64) head_rcp = __shfl(lane_rcp, hk < 64 ? hk : 0, 64);
        }
        if (c >= total || !seg) continue;
        const int ct = c - jc * cptok;                                         // chunk within the token
        const int hc = static_cast<int>(__umulhi(static_cast<uint32_t>(ct), a.head_magic));
        const int d0 = (ct - hc * cpt) * 8;
        Raw8<kSrcBf16> x = raw[k];
        if (pass > 0) x = load8<kSrcBf16>(a.src, t0 * row_elems + static_cast<int64_t>(c) * 8);
        double rcp = 1.0;
        if constexpr (kDst == DCP_FP8_E4M3) rcp = H <= 64 ? head_rcp : scale_rcp(a.scale, hc);
        uint32_t q[8];
        convert8<kDst, kSrcBf16>(x, rcp, q);
        store8<kDst>(a.pool, orow + hc * a.st[2] + static_cast<int64_t>(d0) * a.st[4], a.st[4], a.vec, q);
      }
    }
  }
}

constexpr int kVtTokens = 64;   // tokens per kv_vt_kernel tile
constexpr int kXcds = 8;        // XCDs of an MI355X; workgroup i runs on XCD i % 8
constexpr int kVtDims = 128;    // V dims per tile
constexpr int kVtPitch = 136;   // LDS row pitch in elements (8-element chunks stay 16-byte aligned)

// Wave 0 of the V^T kernels, one owner pass: f[lane] = (owner << kSlotBits) |
// slot of tile token `lane` at this pass's owner (all ones: none). The tokens
// with an owner are ranked by the pool offset of their V row (head 0, dim 0)
// with per-lane counting (ties by token) and permuted into that order, then
// grouped by the aligned word of 2^log_w elements their offset falls in.
// Lane i < nvalid receives the i-th token in order: its index (tok), its
// offset (vs) and group (g, counted in order); bit i of `starts` is set when
// it opens its group.
struct VtOrder {
  int tok, g, nvalid;
  int64_t vs;
  bool in;
  uint64_t starts;
};

__device__ __forceinline__ VtOrder vt_order(const KvWriteParams& p, int lane, int ntok, uint64_t f, int log_w) {
  const bool valid = lane < ntok && f != ~uint64_t(0);
  int64_t vr = 0;
  if (valid) {
    const int rk = static_cast<int>(f >> kSlotBits);
    const int64_t s = static_cast<int64_t>(f & ((uint64_t(1) << kSlotBits) - 1));
    const int64_t blk = s / p.kv.block_size, off = s - blk * p.kv.block_size;
    vr = rk * p.kv.v_stride[0] + blk * p.kv.v_stride[1] + off * p.kv.v_stride[3];
  }
  const uint64_t vmask = __builtin_amdgcn_ballot_w64(valid);
  const int nvalid = __builtin_popcountll(vmask);
  const uint64_t below = (uint64_t(1) << lane) - 1;
  int rank;  // position in the order (valid first, by offset, ties by token)
  if (valid) {
    rank = 0;
    for (uint64_t m = vmask; m; m &= m - 1) {
      const int jl = __builtin_ctzll(m);
      const int64_t vj = __shfl(vr, jl, 64);
      rank += (vj < vr) || (vj == vr && jl < lane);
    }
  } else {
    rank = nvalid + __builtin_popcountll(~vmask & below);
  }
  // lane `rank` receives (token, offset)
  VtOrder o;
  o.tok = __builtin_amdgcn_ds_permute(rank * 4, lane);
  const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_ds_permute(rank * 4, static_cast<int>(vr)));
  const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_ds_permute(rank * 4, static_cast<int>(vr >> 32)));
  o.vs = static_cast<int64_t>((static_cast<uint64_t>(hi) << 32) | lo);
  const int64_t word = o.vs >> log_w;
  const int64_t prev = __shfl(word, lane == 0 ? 0 : lane - 1, 64);
  o.nvalid = nvalid;
  o.in = lane < nvalid;
  o.starts = __builtin_amdgcn_ballot_w64(o.in && (lane == 0 || word != prev));
  o.g = __builtin_popcountll(o.starts & ((below << 1) | 1)) - 1;
  return o;
}

// kv_vt_kernel's grouping by aligned 4-element words: group g's word starts
// at element s_gbase[g] and s_gtok[4 g + u] is the token stored at its
// element u (-1: none). Returns the number of tokens with an owner.
__device__ __forceinline__ int vt_group_pass(const KvWriteParams& p, int lane, int ntok, uint64_t f,
                                             int* s_gtok, int64_t* s_gbase, int* s_groups) {
  const VtOrder o = vt_order(p, lane, ntok, f, 2);
  const int tok = o.tok, g = o.g;
  const int64_t vs = o.vs, word = vs >> 2;
  const bool in = o.in;
  const uint64_t starts = o.starts;
#pragma unroll
  for (int u = 0; u < 4; ++u) s_gtok[4 * lane + u] = -1;
  if (in) {
    s_gtok[4 * g + static_cast<int>(vs & 3)] = tok;
    if ((starts >> lane) & 1) s_gbase[g] = word * 4;
  }
  if (lane == 0) *s_groups = __builtin_popcountll(starts);
  return o.nvalid;
}

// Large batches, V stored token-contiguous inside a block ([block, head,
// dim, token], the layout the attention kernel reads): a workgroup per tile
// of 64 consecutive tokens x 128 dims, looping over the KV heads. The owners
// are found once per tile and the tokens grouped by the aligned 4-element
// pool word they land in (vt_group_pass); per head the tile is loaded
// (coalesced rows; the next head's loads are issued before the current head
// is stored), converted into LDS as [token][dim], and stored one word per
// (group, dim): a single vector store when all four slots of the word are
// written (and the layout keeps words aligned), else one store per slot.
template <int kDst, bool kSrcBf16>
__global__ void __launch_bounds__(256) kv_vt_kernel(KvWriteParams p) {
  using St = typename Stored<kDst>::T;
  __shared__ uint64_t s_owners[kVtTokens];    // owners not yet written, per token
  __shared__ uint64_t s_first[kVtTokens];     // (first owner << kSlotBits) | its slot; all ones: none
  __shared__ __attribute__((aligned(16))) int s_gtok[4 * kVtTokens];  // token at element u of group g's word, or -1
  __shared__ int64_t s_gbase[kVtTokens];      // first element of group g's word (head 0, dim 0)
  __shared__ int s_groups;
  __shared__ St s_tile[kVtTokens * kVtPitch]; // [token][dim]

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t T = p.num_tokens;
  // Workgroups are dealt to the 8 XCDs in turn; tile L = (x % 8) * per + x / 8
  // gives each XCD a contiguous run of tiles, so the slots of a block that
  // neighbouring tiles fill land in the same L2 and leave it as whole lines.
  const int64_t tiles = (T + kVtTokens - 1) / kVtTokens;
  const int64_t per = gridDim.x / kXcds;
  const int64_t tile = (blockIdx.x % kXcds) * per + blockIdx.x / kXcds;
  if (tile >= tiles) return;
  const int64_t t0 = tile * kVtTokens;
  const int ntok = static_cast<int>(T - t0 < kVtTokens ? T - t0 : kVtTokens);
  const int H = p.kv.num_kv_heads, dv = p.kv.head_dim_v;
  const int ds = blockIdx.y * kVtDims;
  const int nd = dv - ds < kVtDims ? dv - ds : kVtDims;
  const int cpt = nd / 8, total = ntok * cpt;  // <= 1024
  const int64_t cap = static_cast<int64_t>(p.kv.num_blocks) * p.kv.block_size;
  St* vpool = static_cast<St*>(p.kv.v);
  const int64_t vdim = p.kv.v_stride[4], vhead = p.kv.v_stride[2];

  auto load_head = [&](int h, Raw8<kSrcBf16> (&raw)[4]) __attribute__((always_inline)) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int c = k * 256 + tid;
      if (c < total) {
        const int i = c / cpt;
        raw[k] = load8<kSrcBf16>(p.v_new, ((t0 + i) * H + h) * dv + ds + (c - i * cpt) * 8);
      }
    }
  };
  auto to_lds = [&](int h, const Raw8<kSrcBf16> (&raw)[4]) __attribute__((always_inline)) {
    double rcp = 1.0;
    if constexpr (kDst == DCP_FP8_E4M3) rcp = scale_rcp(p.kv.v_scale, h);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int c = k * 256 + tid;
      if (c >= total) continue;
      const int i = c / cpt, d0 = (c - i * cpt) * 8;
      uint32_t q[8];
      convert8<kDst, kSrcBf16>(raw[k], rcp, q);
      St* dst = s_tile + i * kVtPitch + d0;
#pragma unroll
      for (int e = 0; e < 8; ++e) dst[e] = static_cast<St>(q[e]);
    }
  };
  // thread = (group tid % gp, dims tid / gp + k * 256 / gp), gp = groups rounded up to a power of two
  auto store_head = [&](int h) __attribute__((always_inline)) {
    const int groups = s_groups;
    int gp = 1;
    while (gp < groups) gp *= 2;
    const int g = tid & (gp - 1);
    if (g >= groups) return;
    const int4 tk = *reinterpret_cast<const int4*>(&s_gtok[4 * g]);
    const int64_t base = s_gbase[g] + h * vhead;
    const bool full = p.vt_quads && tk.x >= 0 && tk.y >= 0 && tk.z >= 0 && tk.w >= 0;
    const int toks[4] = {tk.x, tk.y, tk.z, tk.w};
    for (int d = tid / gp; d < nd; d += 256 / gp) {
      St* dst = vpool + base + static_cast<int64_t>(ds + d) * vdim;
      if (full) {
        const uint32_t e0 = s_tile[tk.x * kVtPitch + d], e1 = s_tile[tk.y * kVtPitch + d];
        const uint32_t e2 = s_tile[tk.z * kVtPitch + d], e3 = s_tile[tk.w * kVtPitch + d];
        if constexpr (kDst == DCP_FP8_E4M3) {
          *reinterpret_cast<uint32_t*>(dst) = e0 | (e1 << 8) | (e2 << 16) | (e3 << 24);
        } else if constexpr (kDst == DCP_BF16) {
          *reinterpret_cast<uint2*>(dst) = uint2{e0 | (e1 << 16), e2 | (e3 << 16)};
        } else {
          *reinterpret_cast<uint4*>(dst) = uint4{e0, e1, e2, e3};
        }
      } else {
#pragma unroll
        for (int u = 0; u < 4; ++u)
          if (toks[u] >= 0) dst[u] = s_tile[toks[u] * kVtPitch + d];
      }
    }
  };

  Raw8<kSrcBf16> raw[4];
  load_head(0, raw);
  if (tid < kVtTokens) {
    s_owners[tid] = 0;
    s_first[tid] = ~uint64_t(0);
  }
  __syncthreads();
  for (int pr = tid; pr < kVtTokens * p.num_ranks; pr += 256) {  // (token, rank) pairs
    const int rk = pr / kVtTokens, i = pr - rk * kVtTokens;
    if (i >= ntok) continue;
    const int64_t s = p.slots[rk * T + t0 + i];
    if (s >= 0 && s < cap) {
      atomicOr(reinterpret_cast<unsigned long long*>(&s_owners[i]), 1ull << rk);
      atomicMin(reinterpret_cast<unsigned long long*>(&s_first[i]),
                (static_cast<unsigned long long>(rk) << kSlotBits) | static_cast<unsigned long long>(s));
    }
  }
  __syncthreads();
  int any = 0;
  if (wave == 0) {
    const uint64_t f = s_first[lane];
    if (f != ~uint64_t(0)) s_owners[lane] &= ~(uint64_t(1) << (f >> kSlotBits));
    any = vt_group_pass(p, lane, ntok, f, s_gtok, s_gbase, &s_groups) > 0;
  }
  if (!__syncthreads_or(any)) return;  // no token of the tile has an owner

  // first owner, all heads: convert head h, prefetch head h + 1, store head h
  for (int h = 0; h < H; ++h) {
    to_lds(h, raw);
    if (h + 1 < H) load_head(h + 1, raw);
    __syncthreads();
    store_head(h);
    __syncthreads();
  }

  // further owners (a token kept on more than one rank): reload per head
  for (;;) {
    any = 0;
    if (wave == 0) {
      const uint64_t m = s_owners[lane];
      uint64_t f = ~uint64_t(0);
      if (m) {
        const int rk = __builtin_ctzll(m);
        s_owners[lane] = m & (m - 1);
        f = (static_cast<uint64_t>(rk) << kSlotBits) | static_cast<uint64_t>(p.slots[rk * T + t0 + lane]);
      }
      any = vt_group_pass(p, lane, ntok, f, s_gtok, s_gbase, &s_groups) > 0;
    }
    if (!__syncthreads_or(any)) break;
    for (int h = 0; h < H; ++h) {
      load_head(h, raw);
      to_lds(h, raw);
      __syncthreads();
      store_head(h);
      __syncthreads();
    }
  }
}

// Large batches, V stored token-contiguous inside a block, with 16-byte
// words of slots aligned across heads and dims (the common case): as
// kv_vt_kernel, but the tokens are grouped by the 16-byte pool word their slot
// falls in (16 fp8 / 8 bf16 / 4 fp32 slots), and the converted tile sits in
// LDS as [dim][group] 16-byte cells, so a word whose slots are all written
// leaves LDS with one 16-byte read and reaches the pool with one 16-byte store
// (consecutive words of a block row by consecutive lanes). Up to kVtGroups
// groups are staged at a time; tiles with more (scattered slots) take several
// rounds per head (cells placed by vt16_cell).
constexpr int kVtGroups = 8;  // 16-byte word groups staged in LDS at a time

template <int kW>
__device__ __forceinline__ int vt16_group_pass(const KvWriteParams& p, int lane, int ntok, uint64_t f,
                                               uint32_t* s_gmask, int64_t* s_gbase, int* s_col, int* s_groups) {
  constexpr int kLog = kW == 16 ? 4 : kW == 8 ? 3 : 2;
  const VtOrder o = vt_order(p, lane, ntok, f, kLog);
  const int tok = o.tok, g = o.g;
  const int64_t vs = o.vs, word = vs >> kLog;
  const bool in = o.in;
  const uint64_t starts = o.starts;
  s_gmask[lane] = 0;
  s_col[lane] = -1;
  __builtin_amdgcn_wave_barrier();
  if (in) {
    const int u = static_cast<int>(vs & (kW - 1));
    atomicOr(&s_gmask[g], 1u << u);
    s_col[tok] = kW * g + u;
    if ((starts >> lane) & 1) s_gbase[g] = word * kW;
  }
  if (lane == 0) *s_groups = __builtin_popcountll(starts);
  return o.nvalid;
}

// The 16-byte cell of group g in dim row d of a tile's LDS cell buffer
// ([dim][group], kVtGroups groups per row): g ^ ((d / 8) % 8), so that the
// sixteen lanes converting one token's row (rows eight apart) spread over the
// banks.
__device__ __forceinline__ int vt16_cell(int d, int g) { return d * kVtGroups + (g ^ ((d >> 3) & 7)); }

// A thread's four 8-element chunks of a tile's V rows (nd dims of ntok
// tokens, nd / 8 chunks per token, 256 threads): chunk c = 256 k + thread is
// token c / (nd / 8), dims 8 (c % (nd / 8)) .. +7; ck_tok[k] = -1 past the
// tile's tokens.
__device__ __forceinline__ void vt16_chunks(int nd, int ntok, int (&ck_tok)[4], int (&ck_d0)[4]) {
  const int cpt = nd / 8, total = ntok * cpt;  // <= 1024
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int c = k * 256 + static_cast<int>(threadIdx.x);
    const int i = c / cpt;
    ck_tok[k] = c < total ? i : -1;
    ck_d0[k] = (c - i * cpt) * 8;
  }
}

// The tile's V^T words through LDS, step 1: this thread's chunks (token
// ck_tok[k] or -1, dims ck_d0[k] .. +7) of one head, converted, into the cells
// of their tokens' groups when the group is one of g0 .. g0 + kVtGroups - 1.
template <int kDst, bool kSrcBf16>
__device__ __forceinline__ void vt16_to_lds(const Raw8<kSrcBf16> (&raw)[4], const int (&ck_tok)[4],
                                            const int (&ck_d0)[4], const int* s_col, int g0, double rcp,
                                            uint4* s_cell) {
  using St = typename Stored<kDst>::T;
  constexpr int kW = 16 / static_cast<int>(sizeof(St));
  char* cells = reinterpret_cast<char*>(s_cell);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int i = ck_tok[k], d0 = ck_d0[k];
    if (i < 0) continue;
    const int col = s_col[i];
    const int gb = (col >= 0 ? col / kW : -1) - g0;
    if (col < 0 || gb < 0 || gb >= kVtGroups) continue;
    uint32_t q[8];
    convert8<kDst, kSrcBf16>(raw[k], rcp, q);
    const int u = col - (col / kW) * kW;
#pragma unroll
    for (int e = 0; e < 8; ++e)
      *reinterpret_cast<St*>(cells + vt16_cell(d0 + e, gb) * 16 + u * sizeof(St)) = static_cast<St>(q[e]);
  }
}

// Step 2: thread = (group gb of the round, dim), the round's groups rounded
// up to a power of two; each cell goes to its pool word (head offset
// head_off, dims ds .. ds + nd - 1). A word whose slots are all written is one
// 16-byte store; a partial word (the ends of a run of slots) is stored in the
// widest aligned pieces it fills: 8 bytes, 4 bytes, then single elements.
template <int kDst>
__device__ __forceinline__ void vt16_store_cells(const KvWriteParams& p, int64_t head_off, int ds, int nd, int g0,
                                                 int groups, const uint32_t* s_gmask, const int64_t* s_gbase,
                                                 const uint4* s_cell) {
  using St = typename Stored<kDst>::T;
  constexpr int kW = 16 / static_cast<int>(sizeof(St));
  const int tid = threadIdx.x;
  const int ng = min(groups - g0, kVtGroups);
  int gp = 1;
  while (gp < ng) gp *= 2;
  const int gb = tid & (gp - 1);
  if (gb >= ng) return;
  const int g = g0 + gb;
  const uint32_t mask = s_gmask[g];
  const bool full = mask == (kW == 32 ? ~0u : (1u << kW) - 1);
  const int64_t base = s_gbase[g] + head_off;
  St* vpool = static_cast<St*>(p.kv.v);
  const int64_t vdim = p.kv.v_stride[4];
  for (int d = tid / gp; d < nd; d += 256 / gp) {
    const uint4 v = s_cell[vt16_cell(d, gb)];
    St* dst = vpool + base + static_cast<int64_t>(ds + d) * vdim;
    if (full) {
      *reinterpret_cast<uint4*>(dst) = v;
      continue;
    }
    const uint32_t dw[4] = {v.x, v.y, v.z, v.w};
    const St* el = reinterpret_cast<const St*>(&v);
    constexpr int kHalf = kW / 2, kQuad = 4 / static_cast<int>(sizeof(St));
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const uint32_t hm = (mask >> (hh * kHalf)) & ((1u << kHalf) - 1);
      if (hm == (1u << kHalf) - 1) {
        *reinterpret_cast<uint2*>(dst + hh * kHalf) = uint2{dw[2 * hh], dw[2 * hh + 1]};
        continue;
      }
#pragma unroll
      for (int qq = 0; qq < 2; ++qq) {
        const int u0 = hh * kHalf + qq * kQuad;
        const uint32_t qm = (mask >> u0) & ((1u << kQuad) - 1);
        if (qm == (1u << kQuad) - 1) {
          *reinterpret_cast<uint32_t*>(dst + u0) = dw[2 * hh + qq];
        } else if (qm) {
#pragma unroll
          for (int u = u0; u < u0 + kQuad; ++u)
            if ((mask >> u) & 1u) dst[u] = el[u];
        }
      }
    }
  }
}

template <int kDst, bool kSrcBf16>
__global__ void __launch_bounds__(256) kv_vt16_kernel(KvWriteParams p) {
  constexpr int kW = 16 / static_cast<int>(sizeof(typename Stored<kDst>::T));  // slots per 16-byte word
  __shared__ uint64_t s_owners[kVtTokens];    // owners not yet written, per token
  __shared__ uint64_t s_first[kVtTokens];     // (first owner << kSlotBits) | its slot; all ones: none
  __shared__ uint32_t s_gmask[kVtTokens];     // slots of group g's word that a token of the pass writes
  __shared__ int64_t s_gbase[kVtTokens];      // first element of group g's word (head 0, dim 0)
  __shared__ int s_col[kVtTokens];            // token -> kW * group + slot, or -1
  __shared__ int s_groups;
  __shared__ uint4 s_cell[kVtDims * kVtGroups];  // [dim][group ^ swizzle], 16 KB

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t T = p.num_tokens;
  const int64_t tiles = (T + kVtTokens - 1) / kVtTokens;
  const int64_t per = gridDim.x / kXcds;
  const int64_t tile = (blockIdx.x % kXcds) * per + blockIdx.x / kXcds;
  if (tile >= tiles) return;
  const int64_t t0 = tile * kVtTokens;
  const int ntok = static_cast<int>(T - t0 < kVtTokens ? T - t0 : kVtTokens);
  const int H = p.kv.num_kv_heads, dv = p.kv.head_dim_v;
  const int ds = blockIdx.y * kVtDims;
  const int nd = dv - ds < kVtDims ? dv - ds : kVtDims;
  const int64_t cap = static_cast<int64_t>(p.kv.num_blocks) * p.kv.block_size;
  const int64_t vhead = p.kv.v_stride[2];
  int ck_tok[4], ck_d0[4];
  vt16_chunks(nd, ntok, ck_tok, ck_d0);

  // Unconditional loads (a chunk past the tile's tokens reloads token 0's):
  // with a branch around them the compiler cannot count the loads in flight
  // and waits for all of them before the first use.
  auto load_head = [&](int h, Raw8<kSrcBf16> (&raw)[4]) __attribute__((always_inline)) {
#pragma unroll
    for (int k = 0; k < 4; ++k)
      raw[k] = load8<kSrcBf16>(p.v_new, ((t0 + max(ck_tok[k], 0)) * H + h) * dv + ds + ck_d0[k]);
  };
  auto to_lds = [&](int h, const Raw8<kSrcBf16> (&raw)[4], int g0) __attribute__((always_inline)) {
    double rcp = 1.0;
    if constexpr (kDst == DCP_FP8_E4M3) rcp = scale_rcp(p.kv.v_scale, h);
    vt16_to_lds<kDst, kSrcBf16>(raw, ck_tok, ck_d0, s_col, g0, rcp, s_cell);
  };
  auto store_cells = [&](int h, int g0) __attribute__((always_inline)) {
    vt16_store_cells<kDst>(p, h * vhead, ds, nd, g0, s_groups, s_gmask, s_gbase, s_cell);
  };
  // all heads of one owner pass, one round of up to kVtGroups groups at a
  // time (one round unless the slots are scattered); within a round the next
  // head's rows load while this one is stored.
  // Two register buffers: head h + 1's rows are requested once head h is
  // converted, so their latency hides behind the barrier and the stores.
  // (Requested before the conversion they would be waited for at its start:
  // with stores of the previous head in flight, loads and stores complete out
  // of order with respect to each other, and the compiler then waits for the
  // vector memory counter to reach zero before using any load.)
  auto head_step = [&](int h, int g0, const Raw8<kSrcBf16> (&cur)[4], Raw8<kSrcBf16> (&nxt)[4])
      __attribute__((always_inline)) {
    to_lds(h, cur, g0);
    if (h + 1 < H) load_head(h + 1, nxt);
    __syncthreads();
    store_cells(h, g0);
    __syncthreads();
  };
  auto heads = [&](Raw8<kSrcBf16> (&raw)[4], bool preloaded) __attribute__((always_inline)) {
    const int groups = s_groups;
    Raw8<kSrcBf16> alt[4];
    for (int g0 = 0; g0 < groups; g0 += kVtGroups) {
      if (g0 > 0 || !preloaded) load_head(0, raw);
      for (int h = 0; h < H; h += 2) {
        head_step(h, g0, raw, alt);
        if (h + 1 < H) head_step(h + 1, g0, alt, raw);
      }
    }
  };

  Raw8<kSrcBf16> raw[4];
  load_head(0, raw);
  if (tid < kVtTokens) {
    s_owners[tid] = 0;
    s_first[tid] = ~uint64_t(0);
  }
  __syncthreads();
  for (int pr = tid; pr < kVtTokens * p.num_ranks; pr += 256) {  // (token, rank) pairs
    const int rk = pr / kVtTokens, i = pr - rk * kVtTokens;
    if (i >= ntok) continue;
    const int64_t s = p.slots[rk * T + t0 + i];
    if (s >= 0 && s < cap) {
      atomicOr(reinterpret_cast<unsigned long long*>(&s_owners[i]), 1ull << rk);
      atomicMin(reinterpret_cast<unsigned long long*>(&s_first[i]),
                (static_cast<unsigned long long>(rk) << kSlotBits) | static_cast<unsigned long long>(s));
    }
  }
  __syncthreads();
  int any = 0;
  if (wave == 0) {
    const uint64_t f = s_first[lane];
    if (f != ~uint64_t(0)) s_owners[lane] &= ~(uint64_t(1) << (f >> kSlotBits));
    any = vt16_group_pass<kW>(p, lane, ntok, f, s_gmask, s_gbase, s_col, &s_groups) > 0;
  }
  if (!__syncthreads_or(any)) return;  // no token of the tile has an owner
  heads(raw, true);

  // further owners (a token kept on more than one rank)
  for (;;) {
    any = 0;
    if (wave == 0) {
      const uint64_t m = s_owners[lane];
      uint64_t f = ~uint64_t(0);
      if (m) {
        const int rk = __builtin_ctzll(m);
        s_owners[lane] = m & (m - 1);
        f = (static_cast<uint64_t>(rk) << kSlotBits) | static_cast<uint64_t>(p.slots[rk * T + t0 + lane]);
      }
      any = vt16_group_pass<kW>(p, lane, ntok, f, s_gmask, s_gbase, s_col, &s_groups) > 0;
    }
    if (!__syncthreads_or(any)) break;
    heads(raw, false);
  }
}

// Small batches (a decode step writes one token per request): one wavefront
// per (token, KV head). Lane r < num_ranks reads the token's slot on rank r
// while the lanes' source loads are in flight; each lane then converts its
// 8-element chunks of the K row (lanes 0 .. Dk/8 - 1) and V row (the next
// Dv/8 lanes) once and stores them at every owner (normally one).
template <int kDst, bool kSrcBf16>
__global__ void __launch_bounds__(256) kv_scatter_kernel(KvWriteParams p) {
  const int lane = threadIdx.x & 63;
  const int H = p.kv.num_kv_heads;
  const int64_t T = p.num_tokens;
  const int64_t pair = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (pair >= T * H) return;  // whole wavefronts leave together
  const int64_t t = pair / H;
  const int h = static_cast<int>(pair - t * H);
  const int dk = p.kv.head_dim_k, dv = p.kv.head_dim_v;
  const int ck = dk / 8, total = ck + (p.v_new ? dv / 8 : 0);
  const int bs = p.kv.block_size;
  const int64_t cap = static_cast<int64_t>(p.kv.num_blocks) * bs;

  const int64_t my_slot = lane < p.num_ranks ? p.slots[lane * T + t] : -1;
  double ks = 1.0, vs = 1.0;
  if constexpr (kDst == DCP_FP8_E4M3) {
    ks = scale_rcp(p.kv.k_scale, h);
    if (p.v_new) vs = scale_rcp(p.kv.v_scale, h);
  }
  constexpr int kGroup = 2;
  for (int c0 = 0; c0 < total; c0 += 64 * kGroup) {
    Raw8<kSrcBf16> raw[kGroup];
#pragma unroll
    for (int j = 0; j < kGroup; ++j) {
      const int c = c0 + j * 64 + lane;
      if (c < ck) raw[j] = load8<kSrcBf16>(p.k_new, (t * H + h) * dk + c * 8);
      else if (c < total) raw[j] = load8<kSrcBf16>(p.v_new, (t * H + h) * dv + (c - ck) * 8);
    }
    uint32_t q[kGroup][8];
#pragma unroll
    for (int j = 0; j < kGroup; ++j) {
      const int c = c0 + j * 64 + lane;
      if (c < total) convert8<kDst, kSrcBf16>(raw[j], c < ck ? ks : vs, q[j]);
    }
    uint64_t owners = __builtin_amdgcn_ballot_w64(my_slot >= 0 && my_slot < cap);
    while (owners) {  // wave-uniform
      const int r = __builtin_ctzll(owners);
      owners &= owners - 1;
      const int64_t s = __shfl(my_slot, r, 64);
      const int64_t blk = s / bs, off = s - blk * bs;
#pragma unroll
      for (int j = 0; j < kGroup; ++j) {
        const int c = c0 + j * 64 + lane;
        if (c >= total) continue;
        const bool is_v = c >= ck;
        const int64_t* st = is_v ? p.kv.v_stride : p.kv.k_stride;
        const int64_t d0 = is_v ? c - ck : c;
        const int64_t e = r * st[0] + blk * st[1] + h * st[2] + off * st[3] + d0 * 8 * st[4];
        store8<kDst>(is_v ? p.kv.v : p.kv.k, e, st[4], is_v ? p.vec_v : p.vec_k, q[j]);
      }
    }
  }
}

// Large batches, rows of 48 .. 64 pieces of 16 elements (GQA: 8 KV heads x
// 128 dims = 64 pieces): a wavefront walks its tokens one at a time, lane l
// taking elements 16 l .. 16 l + 15 of the token's row. The owner's row
// address is then wave-uniform (one slot read per rank, no shuffles), a
// lane's head and fp8 scale are fixed for the whole launch, and every lane
// stores its 16 values at once. kTokUnroll tokens' sources and slots are
// loaded before the first is converted.
constexpr int kTokUnroll = 4;

template <int kDst, bool kSrcBf16>
__global__ void __launch_bounds__(256) kv_tokrow_kernel(KvWriteParams p, RowsArgs a, int tok_per_wave) {
  const int lane = threadIdx.x & 63;
  const int64_t T = p.num_tokens;
  const int64_t t_begin = (static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6)) * tok_per_wave;
  if (t_begin >= T) return;  // whole wavefronts leave together
  const int64_t t_end = T - t_begin < tok_per_wave ? T : t_begin + tok_per_wave;
  const int H = p.kv.num_kv_heads, dim = a.dim, bs = p.kv.block_size;
  const int pieces = H * dim / 16;
  const bool act = lane < pieces;
  const int e0 = 16 * (act ? lane : pieces - 1);  // idle lanes load a valid piece and store nothing
  const int h = e0 / dim, d0 = e0 - h * dim;
  const int64_t row_elems = static_cast<int64_t>(H) * dim;
  const int64_t cap = static_cast<int64_t>(p.kv.num_blocks) * bs;
  const int64_t lane_off = h * a.st[2] + d0;  // dim stride 1 (checked on the host)
  double rcp = 1.0;
  if constexpr (kDst == DCP_FP8_E4M3) rcp = scale_rcp(a.scale, h);

  for (int64_t t0 = t_begin; t0 < t_end; t0 += kTokUnroll) {
    Raw8<kSrcBf16> raw[kTokUnroll][2];
    int64_t slot[kTokUnroll];
#pragma unroll
    for (int j = 0; j < kTokUnroll; ++j) {
      const int64_t t = t0 + j < t_end ? t0 + j : t_end - 1;  // in range; repeats are skipped below
      slot[j] = lane < p.num_ranks ? p.slots[lane * T + t] : -1;
      raw[j][0] = load8<kSrcBf16>(a.src, t * row_elems + e0);
      raw[j][1] = load8<kSrcBf16>(a.src, t * row_elems + e0 + 8);
    }
#pragma unroll
    for (int j = 0; j < kTokUnroll; ++j) {
      if (t0 + j >= t_end) break;  // wave-uniform
      uint32_t q[16];
      uint32_t (&lo)[8] = *reinterpret_cast<uint32_t(*)[8]>(&q[0]);
      uint32_t (&hi)[8] = *reinterpret_cast<uint32_t(*)[8]>(&q[8]);
      convert8<kDst, kSrcBf16>(raw[j][0], rcp, lo);
      convert8<kDst, kSrcBf16>(raw[j][1], rcp, hi);
      uint64_t owners = __builtin_amdgcn_ballot_w64(slot[j] >= 0 && slot[j] < cap);
      while (owners) {  // wave-uniform: normally one owner
        const int r = __builtin_ctzll(owners);
        owners &= owners - 1;
        const uint32_t s_lo = __builtin_amdgcn_readlane(static_cast<uint32_t>(slot[j]), r);
        const uint32_t s_hi = __builtin_amdgcn_readlane(static_cast<uint32_t>(static_cast<uint64_t>(slot[j]) >> 32), r);
        const int64_t s = static_cast<int64_t>((static_cast<uint64_t>(s_hi) << 32) | s_lo);
        const int64_t blk = a.bs_shift >= 0 ? (s >> a.bs_shift) : s / bs;
        const int64_t off = s - blk * bs;
        const int64_t row = r * a.st[0] + blk * a.st[1] + off * a.st[3];
        if (act) store16<kDst>(a.pool, row + lane_off, q);
      }
    }
  }
}

// Whether every chunk of 8 elements of a pool is contiguous and aligned for a
// vector store of 8 elements (16 bytes for 2- and 4-byte elements, 8 for fp8).
static int chunks_vectorizable(const void* base, const int64_t* st, int elem_bytes) {
  if (st[4] != 1) return 0;
  for (int i = 0; i < 4; ++i)
    if (st[i] % 8 != 0) return 0;
  const uintptr_t align = elem_bytes == 1 ? 8 : 16;
  return reinterpret_cast<uintptr_t>(base) % align == 0;
}

// kv_tokrow_kernel applies when a token's row is 48 .. 64 pieces of 16
// elements that never straddle a head, every piece of the pool is contiguous
// and 16-byte aligned, the source rows are 16-byte aligned and every rank's
// slot has a lane.
static bool tokrow_fits(const KvWriteParams& p, const RowsArgs& a, int64_t pieces) {
  const int eb = p.kv.dtype == DCP_F32 ? 4 : p.kv.dtype == DCP_BF16 ? 2 : 1;
  if (a.dim % 16 != 0 || pieces < 48 || pieces > 64 || p.num_ranks > 64) return false;
  if (a.st[4] != 1 || reinterpret_cast<uintptr_t>(a.pool) % 16 != 0 || reinterpret_cast<uintptr_t>(a.src) % 16 != 0)
    return false;
  for (int i = 0; i < 4; ++i)
    if ((a.st[i] * eb) % 16 != 0) return false;
  return true;
}

// Batches below this many tokens take the one-wavefront-per-(token, head)
// kernel: its chain of dependent memory accesses is shorter, which is what
// bounds a write of a few hundred scattered tokens.
constexpr int64_t kScatterMaxTokens = 1024;

template <int kDst, bool kSrcBf16>
static void launch_typed(const KvWriteParams& p, hipStream_t stream) {
  const int64_t T = p.num_tokens, H = p.kv.num_kv_heads;
  if (T < kScatterMaxTokens) {
    hipLaunchKernelGGL((kv_scatter_kernel<kDst, kSrcBf16>), dim3(static_cast<unsigned>((T * H + 3) / 4)), dim3(256),
                       0, stream, p);
    return;
  }
  auto rows = [&](const void* src, void* pool, const int64_t* st, const float* scale, int dim, int vec) {
    RowsArgs a;
    a.src = src;
    a.pool = pool;
    for (int i = 0; i < 5; ++i) a.st[i] = st[i];
    a.scale = scale;
    a.dim = dim;
    a.vec = vec;
    const uint64_t cpt = static_cast<uint64_t>(dim / 8), cptok = static_cast<uint64_t>(H) * cpt;
    a.tpw = 64 / p.rank_lanes;
    while (a.tpw > 1 && static_cast<uint64_t>(a.tpw) * cptok > 64 * kRowsRounds) a.tpw /= 2;
    a.tok_magic = static_cast<uint32_t>(((uint64_t(1) << 32) + cptok - 1) / cptok);
    a.head_magic = static_cast<uint32_t>(((uint64_t(1) << 32) + cpt - 1) / cpt);
    a.bs_shift = -1;
    for (int sh = 0; sh < 31; ++sh)
      if ((1 << sh) == p.kv.block_size) a.bs_shift = sh;
    const int64_t pieces = H * dim / 16;
    if (tokrow_fits(p, a, pieces)) {
      // about eight wavefronts per SIMD, each a multiple of kTokUnroll tokens
      const int64_t target = static_cast<int64_t>(device_cu_count()) * 32;
      int64_t tpw = (T + target - 1) / target;
      tpw = (tpw + kTokUnroll - 1) / kTokUnroll * kTokUnroll;
      const int64_t waves = (T + tpw - 1) / tpw;
      hipLaunchKernelGGL((kv_tokrow_kernel<kDst, kSrcBf16>), dim3(static_cast<unsigned>((waves + 3) / 4)),
                         dim3(256), 0, stream, p, a, static_cast<int>(tpw));
      return;
    }
    const int64_t waves = (T + a.tpw - 1) / a.tpw;
    hipLaunchKernelGGL((kv_rows_kernel<kDst, kSrcBf16>), dim3(static_cast<unsigned>((waves + 3) / 4)), dim3(256),
                       0, stream, p, a);
  };
  rows(p.k_new, p.kv.k, p.kv.k_stride, p.kv.k_scale, p.kv.head_dim_k, p.vec_k);
  if (!p.v_new) return;
  if (!p.v_transposed) {
    rows(p.v_new, p.kv.v, p.kv.v_stride, p.kv.v_scale, p.kv.head_dim_v, p.vec_v);
    return;
  }
  const int64_t tiles = (T + kVtTokens - 1) / kVtTokens;
  const dim3 grid(static_cast<unsigned>((tiles + kXcds - 1) / kXcds * kXcds),
                  static_cast<unsigned>((p.kv.head_dim_v + kVtDims - 1) / kVtDims));
  if (p.vt_vec16) hipLaunchKernelGGL((kv_vt16_kernel<kDst, kSrcBf16>), grid, dim3(256), 0, stream, p);
  else hipLaunchKernelGGL((kv_vt_kernel<kDst, kSrcBf16>), grid, dim3(256), 0, stream, p);
}

template <int kDst>
static void launch_for(const KvWriteParams& p, bool src_bf16, hipStream_t stream) {
  if (src_bf16) launch_typed<kDst, true>(p, stream);
  else launch_typed<kDst, false>(p, stream);
}

hipError_t launch_kv_write(const void* k_new, const void* v_new, int src_bf16, int64_t num_tokens,
                           const int64_t* slots, int num_ranks, const dcp_kv_cache_t& kv, hipStream_t stream) {
  KvWriteParams p;
  p.k_new = k_new;
  p.v_new = kv.v ? v_new : nullptr;
  p.num_tokens = num_tokens;
  p.slots = slots;
  p.num_ranks = num_ranks;
  p.kv = kv;
  const int eb = kv.dtype == DCP_F32 ? 4 : kv.dtype == DCP_BF16 ? 2 : 1;
  p.vec_k = chunks_vectorizable(kv.k, kv.k_stride, eb);
  p.vec_v = kv.v ? chunks_vectorizable(kv.v, kv.v_stride, eb) : 0;
  p.v_transposed = kv.v && kv.v_stride[3] == 1 && kv.v_stride[4] != 1;
  p.vt_quads = p.v_transposed && kv.v_stride[4] % 4 == 0 && kv.v_stride[2] % 4 == 0 &&
               reinterpret_cast<uintptr_t>(kv.v) % static_cast<uintptr_t>(4 * eb) == 0;
  const int w16 = 16 / eb;  // slots per 16-byte word
  p.vt_vec16 = p.v_transposed && kv.v_stride[4] % w16 == 0 && kv.v_stride[2] % w16 == 0 &&
               reinterpret_cast<uintptr_t>(kv.v) % 16 == 0;
  p.rank_lanes = 1;
  while (p.rank_lanes < num_ranks) p.rank_lanes *= 2;
  if (kv.dtype == DCP_FP8_E4M3) launch_for<DCP_FP8_E4M3>(p, src_bf16, stream);
  else if (kv.dtype == DCP_BF16) launch_for<DCP_BF16>(p, src_bf16, stream);
  else launch_for<DCP_F32>(p, src_bf16, stream);
  return hipGetLastError();
}

}  // namespace dcp
