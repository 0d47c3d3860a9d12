// DCP KV-cache write: new K/V rows stored at their slots on the owning rank.
//
// Source: "Decode Context Parallel (DCP)" (vLLM Ascend design doc), section
// "KV-cache layout" (each rank stores only its local shard, at the slot the
// slot mapping gives); "DeepSeek V4.1 context parallelism" (TokenSpeed design
// note), section "Cache ownership" (a write turns the virtual slot into the
// owner's local slot; non-owners are masked).
//
// One wavefront per token: lane r < num_ranks reads the token's slot on rank
// r, so the (normally single) owner is found once per token, wave-uniform;
// the lanes then convert and write 8-element chunks of every KV head's K row
// (and V row), chunk c of the token's H*(Dk+Dv)/8 chunks on lane c % 64.
// Stored formats: fp32 as is; bf16 rounded to nearest even; fp8 E4M3 (no
// infinities) nearest to the fp32 quotient x / scale[h], ties to even,
// saturating at 448, NaN -> 0x7F. The conversions are integer code written
// from the formats' definitions.
#include "common.h"

namespace dcp {

// fp32 -> E4M3 code: round to nearest, ties to even, saturate, NaN -> 0x7F.
__device__ __forceinline__ uint32_t f32_to_e4m3(float x) {
  const uint32_t u = __float_as_uint(x);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7fffffffu;
  if (a > 0x7f800000u) return 0x7fu;              // NaN
  if (a >= 0x43e00000u) return sign | 0x7eu;      // |x| >= 448 (infinity included): largest finite
  if (a >= 0x3c800000u) {                         // |x| >= 2^-6: normal E4M3 range
    const uint32_t mant = a & 0x7fffffu;
    uint32_t q = (((a >> 23) - 120u) << 3) | (mant >> 20);  // biased exponent (bias 7) and 3 mantissa bits
    const uint32_t rest = mant & 0xfffffu;                  // the 20 dropped bits
    if (rest > 0x80000u || (rest == 0x80000u && (q & 1u))) ++q;  // carries into the exponent as it should
    return sign | q;                              // < 448 here, so q <= 0x7e
  }
  // subnormal E4M3: multiples of 2^-9; |x| * 512 is exact, rintf rounds half to even
  return sign | static_cast<uint32_t>(rintf(__uint_as_float(a) * 512.0f));
}

// fp32 -> bf16 bits: round to nearest, ties to even; NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t f32_to_bf16(float x) {
  const uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

struct KvWriteParams {
  const void* k_new;
  const void* v_new;     // nullptr: no V rows (MLA)
  int src_bf16;          // 1: sources are bf16, 0: fp32
  int64_t num_tokens;
  const int64_t* slots;  // [num_ranks, num_tokens]
  int num_ranks;
  dcp_kv_cache_t kv;
  int chunks_k, chunks_v;  // 8-element chunks per token: H * Dk / 8, H * Dv / 8
  int vec_k, vec_v;        // 1: the pool's 8-element chunks are contiguous and aligned (vector stores)
};

template <int kDst>  // DCP_F32, DCP_BF16, DCP_FP8_E4M3
__global__ void __launch_bounds__(256) kv_write_kernel(KvWriteParams p) {
  const int lane = threadIdx.x & 63;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (t >= p.num_tokens) return;  // whole wavefronts leave together
  const int64_t cap = static_cast<int64_t>(p.kv.num_blocks) * p.kv.block_size;
  const int64_t my_slot = lane < p.num_ranks ? p.slots[static_cast<int64_t>(lane) * p.num_tokens + t] : -1;
  const bool mine = my_slot >= 0 && my_slot < cap;
  uint64_t owners = __builtin_amdgcn_ballot_w64(mine);
  const int H = p.kv.num_kv_heads, dk = p.kv.head_dim_k, dv = p.kv.head_dim_v;
  const int chunks = p.chunks_k + p.chunks_v;
  while (owners) {  // wave-uniform loop over the ranks that own the token (normally one)
    const int r = __builtin_ctzll(owners);
    owners &= owners - 1;
    const int64_t s = __shfl(my_slot, r, 64);
    const int64_t blk = s / p.kv.block_size, off = s - blk * p.kv.block_size;
    for (int c = lane; c < chunks; c += 64) {
      const bool is_v = c >= p.chunks_k;
      const int cc = is_v ? c - p.chunks_k : c;
      const int dim = is_v ? dv : dk;
      const int h = (cc * 8) / dim, d0 = cc * 8 - h * dim;
      // 8 source elements (contiguous [T, H, D] rows)
      float x[8];
      const int64_t src_off = (t * H + h) * dim + d0;
      if (p.src_bf16) {
        const uint4 raw = *reinterpret_cast<const uint4*>(
            static_cast<const uint16_t*>(is_v ? p.v_new : p.k_new) + src_off);
        const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          x[2 * i] = __uint_as_float(w[i] << 16);
          x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
        }
      } else {
        const float4* s4 = reinterpret_cast<const float4*>(static_cast<const float*>(is_v ? p.v_new : p.k_new) + src_off);
        const float4 a = s4[0], b = s4[1];
        x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
        x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
      }
      const int64_t* st = is_v ? p.kv.v_stride : p.kv.k_stride;
      const bool vec = is_v ? p.vec_v : p.vec_k;
      char* base = static_cast<char*>(const_cast<void*>(is_v ? p.kv.v : p.kv.k));
      const int64_t e0 = r * st[0] + blk * st[1] + h * st[2] + off * st[3] + static_cast<int64_t>(d0) * st[4];
      if constexpr (kDst == DCP_FP8_E4M3) {
        const float scale = (is_v ? p.kv.v_scale : p.kv.k_scale)[h];
        uint32_t q[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) q[i] = f32_to_e4m3(x[i] / scale);
        uint8_t* dst = reinterpret_cast<uint8_t*>(base) + e0;
        if (vec) {
          *reinterpret_cast<uint2*>(dst) = uint2{q[0] | (q[1] << 8) | (q[2] << 16) | (q[3] << 24),
                                                 q[4] | (q[5] << 8) | (q[6] << 16) | (q[7] << 24)};
        } else {
#pragma unroll
          for (int i = 0; i < 8; ++i) dst[i * st[4]] = static_cast<uint8_t>(q[i]);
        }
      } else if constexpr (kDst == DCP_BF16) {
        uint32_t q[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) q[i] = f32_to_bf16(x[i]);
        uint16_t* dst = reinterpret_cast<uint16_t*>(base) + e0;
        if (vec) {
          *reinterpret_cast<uint4*>(dst) = uint4{q[0] | (q[1] << 16), q[2] | (q[3] << 16), q[4] | (q[5] << 16),
                                                 q[6] | (q[7] << 16)};
        } else {
#pragma unroll
          for (int i = 0; i < 8; ++i) dst[i * st[4]] = static_cast<uint16_t>(q[i]);
        }
      } else {
        float* dst = reinterpret_cast<float*>(base) + e0;
        if (vec) {
          reinterpret_cast<float4*>(dst)[0] = float4{x[0], x[1], x[2], x[3]};
          reinterpret_cast<float4*>(dst)[1] = float4{x[4], x[5], x[6], x[7]};
        } else {
#pragma unroll
          for (int i = 0; i < 8; ++i) dst[i * st[4]] = x[i];
        }
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

hipError_t launch_kv_write(const void* k_new, const void* v_new, int src_bf16, int64_t num_tokens,
                           const int64_t* slots, int num_ranks, const dcp_kv_cache_t& kv, hipStream_t stream) {
  KvWriteParams p;
  p.k_new = k_new;
  p.v_new = v_new;
  p.src_bf16 = src_bf16;
  p.num_tokens = num_tokens;
  p.slots = slots;
  p.num_ranks = num_ranks;
  p.kv = kv;
  p.chunks_k = kv.num_kv_heads * kv.head_dim_k / 8;
  p.chunks_v = kv.v ? kv.num_kv_heads * kv.head_dim_v / 8 : 0;
  const int eb = kv.dtype == DCP_F32 ? 4 : kv.dtype == DCP_BF16 ? 2 : 1;
  p.vec_k = chunks_vectorizable(kv.k, kv.k_stride, eb);
  p.vec_v = kv.v ? chunks_vectorizable(kv.v, kv.v_stride, eb) : 0;
  const dim3 grid(static_cast<unsigned>((num_tokens + 3) / 4));
  if (kv.dtype == DCP_FP8_E4M3)
    hipLaunchKernelGGL(kv_write_kernel<DCP_FP8_E4M3>, grid, dim3(256), 0, stream, p);
  else if (kv.dtype == DCP_BF16)
    hipLaunchKernelGGL(kv_write_kernel<DCP_BF16>, grid, dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL(kv_write_kernel<DCP_F32>, grid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace dcp
