// Internal declarations shared by the libdcp translation units (not part of
// the C ABI; the ABI is include/dcp.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include "dcp.h"

namespace dcp {

// Parameters of one dcp_partial_decode_attn call after host validation.
struct AttnParams {
  const void* q;
  int q_dtype;
  int batch, num_q_heads, group;  // group = num_q_heads / num_kv_heads
  // Query tokens per request (1: decode; more: the last q_len tokens of each
  // request at once, query i attending local_lens row (b * q_len + i)). A
  // split-KV unit covers tpu of them (ntg = ceil(q_len / tpu) units per
  // request and KV head).
  int q_len = 1, tpu = 1, ntg = 1;
  dcp_kv_cache_t kv;
  const int32_t* block_table;
  int64_t bt_stride;
  int max_vblocks;
  const int32_t* local_lens;
  int dcp_size, rank_begin, rank_count;
  float softmax_scale;
  float* out_o;
  float* out_lse;
  void* workspace;
  size_t workspace_bytes;
  hipStream_t stream;
  // Measurement hook: when set, recorded on `stream` right before and right
  // after the family's main attention kernel.
  hipEvent_t ev_begin = nullptr, ev_end = nullptr;
};

// Kernel families behind dcp_partial_decode_attn.
enum class AttnKernel { Generic, GqaMfma, MlaMfma };

// Workspace bytes each family needs (host only, device independent).
size_t generic_workspace_bytes(const AttnParams& p);
size_t gqa_workspace_bytes(const AttnParams& p);
size_t mla_workspace_bytes(const AttnParams& p);

// Whether an MFMA family supports the (validated) geometry and layout.
bool gqa_supported(const AttnParams& p);
bool mla_supported(const AttnParams& p);

hipError_t launch_generic_attn(const AttnParams& p);
hipError_t launch_gqa_attn(const AttnParams& p);
hipError_t launch_mla_attn(const AttnParams& p);

hipError_t launch_check_block_table(const int32_t* bt, int num_reqs, int64_t bt_stride, int max_vblocks,
                                    const int32_t* seq_lens, int block_size, int dcp_size, int num_blocks,
                                    int32_t* bad, hipStream_t s);
hipError_t launch_local_seq_lens(const int32_t* seq_lens, int num_reqs, int dcp_size,
                                 int interleave, int32_t* local_lens, hipStream_t s);
hipError_t launch_slot_mapping(const int64_t* positions, const int32_t* req_indices,
                               int64_t num_tokens, const int32_t* block_table, int num_reqs,
                               int64_t bt_stride, int max_vblocks, int block_size, int dcp_size,
                               int interleave, int64_t* slots, hipStream_t s);
hipError_t launch_kv_write(const void* k_new, const void* v_new, int src_bf16, int64_t num_tokens,
                           const int64_t* slots, int num_ranks, const dcp_kv_cache_t& kv, hipStream_t stream);
bool gather_supported(const dcp_kv_cache_t& kv, bool with_v);
hipError_t launch_gather_context(const dcp_kv_cache_t& kv, int dcp_size, int interleave, const int32_t* block_table,
                                 int num_reqs, int64_t bt_stride, int max_vblocks, const int64_t* cu_ctx,
                                 int64_t total, void* out_k, void* out_v, hipStream_t stream);
hipError_t launch_lse_fold(float* o, float* lse, const float* o_add, const float* lse_add, int64_t rows,
                           int head_dim_v, hipStream_t s);
hipError_t launch_lse_merge(const float* part_o, const float* part_lse, int num_parts, int batch,
                            int num_heads, int head_dim_v, const float* sink, int out_dtype,
                            void* out_o, float* out_lse, hipStream_t s);

// Streaming-read probe (probe.hip): workgroups it launches on the current
// device, and the launch (bytes a multiple of 16, buf 16-byte aligned).
int hbm_read_probe_blocks();
hipError_t launch_hbm_read_probe(const void* buf, int64_t bytes, uint32_t* digest, int blocks, hipStream_t s);

// Number of compute units of the current device (cached per device).
int device_cu_count();

__host__ __device__ inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

}  // namespace dcp

// ---------------------------------------------------------------------------
// Device helpers
// ---------------------------------------------------------------------------
#ifdef __HIPCC__

#define DCP_LOG2E 1.4426950408889634f
#define DCP_LN2 0.6931471805599453f

namespace dcp {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round-to-nearest-even float -> bf16 bits (NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// OCP E4M3 (no infinities) code -> float, from the format definition.
__device__ __forceinline__ float fp8e4m3_to_f32(uint8_t c) {
  const uint32_t sign = static_cast<uint32_t>(c & 0x80) << 24;
  const uint32_t e = (c >> 3) & 0xf, m = c & 0x7;
  if (e == 0xf && m == 0x7) return __uint_as_float(sign | 0x7fc00000u);
  if (e == 0) return __uint_as_float(sign) + (sign ? -1.f : 1.f) * (float)m * 0.001953125f;  // m * 2^-9
  return __uint_as_float(sign | ((e + 120u) << 23) | (m << 20));
}

template <typename T>
__device__ __forceinline__ T wave_max(T v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

}  // namespace dcp

#endif  // __HIPCC__
