// Log-sum-exp merge of per-rank partial attention outputs, with an attention
// sink applied once.
//
// Source: "Decode Context Parallel (DCP)" (vLLM Ascend design doc), section
// "Decode": the ranks' partial outputs and LSE values are combined across the
// DCP group. "DeepSeek V4.1 context parallelism", section "Decode
// computation": the sink is applied once, when the partials are merged by
// log-sum-exp.
//
// Each (request, head) row is handled by a group of `tpr` consecutive threads
// (a power of two up to the block size), each taking kVec consecutive outputs
// per column step. Every thread derives the merge weights from the row's
// num_parts LSE values itself (the same addresses across the group, so one
// fetch serves it), then loads the parts' slices of its columns eight at a
// time, all issued before the first is used. HBM bound: reads
// num_parts*(Dv+1) floats and writes Dv outputs per (request, head). The same
// file holds the in-place fold that adds a replicated segment's partial to
// one rank's.
#include "common.h"

namespace dcp {

constexpr int kMergeThreads = 256;
constexpr int kMergeChunk = 8;

template <int kVec>
struct MergeVec;
template <>
struct MergeVec<1> {
  using T = float;
  static __device__ __forceinline__ float at(const T& v, int) { return v; }
};
template <>
struct MergeVec<4> {
  using T = float4;
  static __device__ __forceinline__ float at(const T& v, int k) {
    return k == 0 ? v.x : k == 1 ? v.y : k == 2 ? v.z : v.w;
  }
};

template <int kVec, bool kBf16Out>
__global__ void __launch_bounds__(kMergeThreads) lse_merge_kernel(
    const float* __restrict__ part_o, const float* __restrict__ part_lse, int num_parts, int64_t rows,
    int num_heads, int head_dim_v, int tpr_log2, const float* __restrict__ sink, void* __restrict__ out_o,
    float* __restrict__ out_lse) {
  using V = typename MergeVec<kVec>::T;
  const int64_t bh = (static_cast<int64_t>(blockIdx.x) * kMergeThreads + threadIdx.x) >> tpr_log2;
  if (bh >= rows) return;
  const int tpr = 1 << tpr_log2;
  const int col0 = threadIdx.x & (tpr - 1);
  const int ncols = head_dim_v / kVec;
  const int h = static_cast<int>(bh % num_heads);
  const int last = num_parts - 1;

  // M = max(max_r LSE_r, sink); Z = sum_r exp(LSE_r - M) (+ exp(sink - M))
  const float sk = sink ? sink[h] : -INFINITY;
  float m = sk;
  for (int r0 = 0; r0 < num_parts; r0 += kMergeChunk) {
    float l[kMergeChunk];
#pragma unroll
    for (int j = 0; j < kMergeChunk; ++j) l[j] = part_lse[min(r0 + j, last) * rows + bh];
#pragma unroll
    for (int j = 0; j < kMergeChunk; ++j) m = fmaxf(m, l[j]);  // repeats of the last part change nothing
  }
  float z = 0.f;
  for (int r0 = 0; r0 < num_parts; r0 += kMergeChunk) {
    float l[kMergeChunk];
#pragma unroll
    for (int j = 0; j < kMergeChunk; ++j) l[j] = part_lse[min(r0 + j, last) * rows + bh];
#pragma unroll
    for (int j = 0; j < kMergeChunk; ++j)
      if (r0 + j < num_parts && l[j] != -INFINITY) z += __expf(l[j] - m);
  }
  if (sink && sk != -INFINITY) z += __expf(sk - m);
  const bool empty = m == -INFINITY;
  if (col0 == 0 && out_lse) out_lse[bh] = empty ? -INFINITY : m + __logf(z);

  for (int c = col0; c < ncols; c += tpr) {
    float acc[kVec];
#pragma unroll
    for (int k = 0; k < kVec; ++k) acc[k] = 0.f;
    for (int r0 = 0; r0 < num_parts; r0 += kMergeChunk) {
      V x[kMergeChunk];
      float w[kMergeChunk];
#pragma unroll
      for (int j = 0; j < kMergeChunk; ++j) {
        const int64_t r = min(r0 + j, last);
        x[j] = reinterpret_cast<const V*>(part_o + (r * rows + bh) * head_dim_v)[c];
        const float l = part_lse[r * rows + bh];
        const float e = l != -INFINITY ? __expf(l - m) : 0.f;
        w[j] = (r0 + j < num_parts && !empty) ? e / z : 0.f;
      }
#pragma unroll
      for (int j = 0; j < kMergeChunk; ++j)
        if (w[j] != 0.f) {
#pragma unroll
          for (int k = 0; k < kVec; ++k) acc[k] += w[j] * MergeVec<kVec>::at(x[j], k);
        }
    }
    const int64_t o = bh * head_dim_v + static_cast<int64_t>(c) * kVec;
    if constexpr (kBf16Out) {
      uint16_t* dst = reinterpret_cast<uint16_t*>(out_o) + o;
      if constexpr (kVec == 4) {
        uint2 pk;
        pk.x = f32_to_bf16_bits(acc[0]) | (static_cast<uint32_t>(f32_to_bf16_bits(acc[1])) << 16);
        pk.y = f32_to_bf16_bits(acc[2]) | (static_cast<uint32_t>(f32_to_bf16_bits(acc[3])) << 16);
        *reinterpret_cast<uint2*>(dst) = pk;
      } else {
        dst[0] = f32_to_bf16_bits(acc[0]);
      }
    } else {
      float* dst = reinterpret_cast<float*>(out_o) + o;
      if constexpr (kVec == 4) *reinterpret_cast<float4*>(dst) = make_float4(acc[0], acc[1], acc[2], acc[3]);
      else dst[0] = acc[0];
    }
  }
}

// In-place fold of a second partial into a first: (O, LSE) of attention over
// the union of two disjoint token sets from the two sets' partials. Used to
// add a replicated segment to the one rank that counts it. One workgroup per
// (request, head); wave 0 reads the two LSE values and shares the weights.
constexpr int kFoldThreads = 128;

__global__ void __launch_bounds__(kFoldThreads) lse_fold_kernel(float* __restrict__ o, float* __restrict__ lse,
                                                                 const float* __restrict__ o_add,
                                                                 const float* __restrict__ lse_add, int head_dim_v) {
  __shared__ float wts[2];
  const int64_t bh = blockIdx.x;
  if (threadIdx.x == 0) {
    const float l1 = lse[bh], l2 = lse_add[bh];
    const float m = fmaxf(l1, l2);
    if (m == -INFINITY) {  // both empty: O stays 0, LSE -inf
      wts[0] = 1.f;
      wts[1] = 0.f;
    } else {
      const float e1 = l1 == -INFINITY ? 0.f : __expf(l1 - m);
      const float e2 = l2 == -INFINITY ? 0.f : __expf(l2 - m);
      const float z = e1 + e2;
      wts[0] = e1 / z;
      wts[1] = e2 / z;
      lse[bh] = m + __logf(z);
    }
  }
  __syncthreads();
  const float w1 = wts[0], w2 = wts[1];
  float* dst = o + bh * head_dim_v;
  const float* add = o_add + bh * head_dim_v;
  for (int d = threadIdx.x; d < head_dim_v; d += kFoldThreads) {
    float acc = w1 != 0.f ? w1 * dst[d] : 0.f;
    if (w2 != 0.f) acc += w2 * add[d];
    dst[d] = acc;
  }
}

hipError_t launch_lse_fold(float* o, float* lse, const float* o_add, const float* lse_add, int64_t rows,
                           int head_dim_v, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  hipLaunchKernelGGL(lse_fold_kernel, dim3(static_cast<unsigned>(rows)), dim3(kFoldThreads), 0, s, o, lse, o_add,
                     lse_add, head_dim_v);
  return hipGetLastError();
}

template <int kVec>
static void launch_merge_vec(const float* part_o, const float* part_lse, int num_parts, int64_t rows,
                             int num_heads, int head_dim_v, const float* sink, bool bf16_out, void* out_o,
                             float* out_lse, unsigned grid, int tpr_log2, hipStream_t s) {
  if (bf16_out)
    hipLaunchKernelGGL((lse_merge_kernel<kVec, true>), dim3(grid), dim3(kMergeThreads), 0, s, part_o, part_lse,
                       num_parts, rows, num_heads, head_dim_v, tpr_log2, sink, out_o, out_lse);
  else
    hipLaunchKernelGGL((lse_merge_kernel<kVec, false>), dim3(grid), dim3(kMergeThreads), 0, s, part_o, part_lse,
                       num_parts, rows, num_heads, head_dim_v, tpr_log2, sink, out_o, out_lse);
}

hipError_t launch_lse_merge(const float* part_o, const float* part_lse, int num_parts, int batch,
                            int num_heads, int head_dim_v, const float* sink, int out_dtype, void* out_o,
                            float* out_lse, hipStream_t s) {
  const int64_t rows = static_cast<int64_t>(batch) * num_heads;
  if (rows == 0) return hipSuccess;
  const bool bf16_out = out_dtype == DCP_BF16;
  // float4 loads and 8/16-byte stores when every row starts on those boundaries
  const bool vec = head_dim_v % 4 == 0 && reinterpret_cast<uintptr_t>(part_o) % 16 == 0 &&
                   reinterpret_cast<uintptr_t>(out_o) % (bf16_out ? 8 : 16) == 0;
  const int ncols = vec ? head_dim_v / 4 : head_dim_v;
  int tpr_log2 = 0;
  while ((1 << tpr_log2) < ncols && (1 << tpr_log2) < kMergeThreads) ++tpr_log2;
  const int64_t rows_per_block = kMergeThreads >> tpr_log2;
  const int64_t grid = (rows + rows_per_block - 1) / rows_per_block;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  if (vec)
    launch_merge_vec<4>(part_o, part_lse, num_parts, rows, num_heads, head_dim_v, sink, bf16_out, out_o, out_lse,
                        static_cast<unsigned>(grid), tpr_log2, s);
  else
    launch_merge_vec<1>(part_o, part_lse, num_parts, rows, num_heads, head_dim_v, sink, bf16_out, out_o, out_lse,
                        static_cast<unsigned>(grid), tpr_log2, s);
  return hipGetLastError();
}

}  // namespace dcp
