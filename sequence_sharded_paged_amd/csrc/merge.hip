// Log-sum-exp merge of per-rank partial attention outputs, with an attention
// sink applied once.
//
// Source: "Decode Context Parallel (DCP)" (vLLM Ascend design doc), section
// "Decode": the ranks' partial outputs and LSE values are combined across the
// DCP group. "DeepSeek V4.1 context parallelism", section "Decode
// computation": the sink is applied once, when the partials are merged by
// log-sum-exp.
//
// One workgroup per (request, head); every thread derives the merge weights
// from the num_parts LSE values (read once into LDS) and then scales and sums
// its slice of the head's output rows. HBM bound: reads num_parts*(Dv+1)
// floats and writes Dv outputs per (request, head). The same file holds the
// in-place fold that adds a replicated segment's partial to one rank's.
#include "common.h"

namespace dcp {

constexpr int kMergeThreads = 128;
constexpr int kMaxParts = 64;

template <bool kBf16Out>
__global__ void __launch_bounds__(kMergeThreads) lse_merge_kernel(
    const float* __restrict__ part_o, const float* __restrict__ part_lse, int num_parts, int batch,
    int num_heads, int head_dim_v, const float* __restrict__ sink, void* __restrict__ out_o,
    float* __restrict__ out_lse) {
  __shared__ float w[kMaxParts];
  __shared__ float lse_s;
  const int bh = blockIdx.x;  // b * num_heads + h
  const int h = bh % num_heads;
  const int64_t part_stride = static_cast<int64_t>(batch) * num_heads;
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    float l = -INFINITY;
    if (lane < num_parts) l = part_lse[lane * part_stride + bh];
    float m = wave_max(l);
    const float sk = sink ? sink[h] : -INFINITY;
    m = fmaxf(m, sk);
    float e = (lane < num_parts && l != -INFINITY) ? __expf(l - m) : 0.f;
    float z = wave_sum(e);
    if (sink && sk != -INFINITY) z += __expf(sk - m);
    const float lse = (m == -INFINITY) ? -INFINITY : m + __logf(z);
    if (lane < num_parts) w[lane] = (m == -INFINITY) ? 0.f : e / z;
    if (lane == 0) lse_s = lse;
  }
  __syncthreads();
  if (threadIdx.x == 0 && out_lse) out_lse[bh] = lse_s;
  const float* src = part_o + static_cast<int64_t>(bh) * head_dim_v;
  const int64_t src_stride = part_stride * head_dim_v;
  for (int d = threadIdx.x; d < head_dim_v; d += kMergeThreads) {
    float acc = 0.f;
    for (int r = 0; r < num_parts; ++r) {
      const float wr = w[r];
      if (wr != 0.f) acc += wr * src[r * src_stride + d];
    }
    const int64_t o = static_cast<int64_t>(bh) * head_dim_v + d;
    if (kBf16Out) reinterpret_cast<uint16_t*>(out_o)[o] = f32_to_bf16_bits(acc);
    else reinterpret_cast<float*>(out_o)[o] = acc;
  }
}

// In-place fold of a second partial into a first: (O, LSE) of attention over
// the union of two disjoint token sets from the two sets' partials. Used to
// add a replicated segment to the one rank that counts it. One workgroup per
// (request, head); wave 0 reads the two LSE values and shares the weights.
__global__ void __launch_bounds__(kMergeThreads) lse_fold_kernel(float* __restrict__ o, float* __restrict__ lse,
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
  for (int d = threadIdx.x; d < head_dim_v; d += kMergeThreads) {
    float acc = w1 != 0.f ? w1 * dst[d] : 0.f;
    if (w2 != 0.f) acc += w2 * add[d];
    dst[d] = acc;
  }
}

hipError_t launch_lse_fold(float* o, float* lse, const float* o_add, const float* lse_add, int64_t rows,
                           int head_dim_v, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  hipLaunchKernelGGL(lse_fold_kernel, dim3(static_cast<unsigned>(rows)), dim3(kMergeThreads), 0, s, o, lse, o_add,
                     lse_add, head_dim_v);
  return hipGetLastError();
}

hipError_t launch_lse_merge(const float* part_o, const float* part_lse, int num_parts, int batch,
                            int num_heads, int head_dim_v, const float* sink, int out_dtype, void* out_o,
                            float* out_lse, hipStream_t s) {
  const int64_t n = static_cast<int64_t>(batch) * num_heads;
  if (n == 0) return hipSuccess;
  if (out_dtype == DCP_BF16)
    hipLaunchKernelGGL(lse_merge_kernel<true>, dim3(static_cast<unsigned>(n)), dim3(kMergeThreads), 0, s,
                       part_o, part_lse, num_parts, batch, num_heads, head_dim_v, sink, out_o, out_lse);
  else
    hipLaunchKernelGGL(lse_merge_kernel<false>, dim3(static_cast<unsigned>(n)), dim3(kMergeThreads), 0, s,
                       part_o, part_lse, num_parts, batch, num_heads, head_dim_v, sink, out_o, out_lse);
  return hipGetLastError();
}

}  // namespace dcp
