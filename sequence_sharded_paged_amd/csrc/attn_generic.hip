// Generic per-rank partial decode attention (fp32 arithmetic, any layout).
//
// Source: "Decode Context Parallel (DCP)" (vLLM Ascend design doc), section
// "Decode": each rank attends the gathered query heads against its local KV
// shard and emits a partial output and its LSE.
//
// This kernel serves the geometries the MFMA kernels do not (fp32 KV, other
// head dims, other layouts) and cross-checks them. One workgroup per (rank,
// request, query token, query head) walks the local tokens that query sees in
// chunks of 256: each
// thread scores one token with an fp32 dot product, the workgroup updates the
// running max and sum (online softmax), and each thread then accumulates its
// output dimensions over the chunk. Every K/V element goes through the
// caller's strides, so any layout works; it is latency- and VALU-bound and is
// not the fast path.
#include "common.h"

namespace dcp {

constexpr int kGenThreads = 256;
constexpr int kGenMaxDim = 1024;

template <int kKvDtype>
__device__ __forceinline__ float load_kv(const void* base, int64_t idx) {
  if constexpr (kKvDtype == DCP_F32) return reinterpret_cast<const float*>(base)[idx];
  else if constexpr (kKvDtype == DCP_BF16) return bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(base)[idx]);
  else return fp8e4m3_to_f32(reinterpret_cast<const uint8_t*>(base)[idx]);
}

template <int kKvDtype, int kQDtype>
__global__ void __launch_bounds__(kGenThreads) generic_attn_kernel(AttnParams p) {
  __shared__ float q_s[kGenMaxDim];
  __shared__ float p_s[kGenThreads];
  __shared__ float red[kGenThreads / 64];
  // one workgroup per (rank r, query row bq = b * q_len + i, query head h)
  const int nq = p.batch * p.q_len;
  const int h = blockIdx.x % p.num_q_heads;
  const int bq = (blockIdx.x / p.num_q_heads) % nq;
  const int r = blockIdx.x / (p.num_q_heads * nq);
  const int b = bq / p.q_len;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int g = h / p.group;
  const dcp_kv_cache_t& kv = p.kv;
  const int Dk = kv.head_dim_k, Dv = kv.head_dim_v;
  const int n = max(p.local_lens[static_cast<int64_t>(bq) * p.dcp_size + p.rank_begin + r], 0);
  const int64_t out_row = (static_cast<int64_t>(r) * nq + bq) * p.num_q_heads + h;

  for (int d = tid; d < Dk; d += kGenThreads) {
    const int64_t qi = (static_cast<int64_t>(bq) * p.num_q_heads + h) * Dk + d;
    q_s[d] = (kQDtype == DCP_F32) ? reinterpret_cast<const float*>(p.q)[qi]
                                  : bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(p.q)[qi]);
  }
  const float kscale = (kKvDtype == DCP_FP8_E4M3) ? kv.k_scale[g] : 1.f;
  const float vscale = (kKvDtype == DCP_FP8_E4M3) ? kv.v_scale[g] : 1.f;
  const void* vbase = kv.v ? kv.v : kv.k;
  const int64_t* vs = kv.v ? kv.v_stride : kv.k_stride;
  const int64_t k_head = r * kv.k_stride[0] + g * kv.k_stride[2];
  const int64_t v_head = r * vs[0] + g * vs[2];
  const int32_t* bt = p.block_table + static_cast<int64_t>(b) * p.bt_stride;
  __syncthreads();

  float m = -INFINITY, l = 0.f;
  float acc[kGenMaxDim / kGenThreads];
#pragma unroll
  for (int i = 0; i < kGenMaxDim / kGenThreads; ++i) acc[i] = 0.f;

  for (int c = 0; c < n; c += kGenThreads) {
    const int j = c + tid;
    float s = -INFINITY;
    if (j < n) {
      const int64_t phys = bt[j / kv.block_size];
      const int64_t row = k_head + phys * kv.k_stride[1] + static_cast<int64_t>(j % kv.block_size) * kv.k_stride[3];
      float dot = 0.f;
      for (int d = 0; d < Dk; ++d) dot += q_s[d] * load_kv<kKvDtype>(kv.k, row + d * kv.k_stride[4]);
      s = dot * kscale * p.softmax_scale;
    }
    float cm = wave_max(s);
    if (lane == 0) red[wid] = cm;
    __syncthreads();
    cm = red[0];
    for (int w = 1; w < kGenThreads / 64; ++w) cm = fmaxf(cm, red[w]);
    __syncthreads();
    const float m_new = fmaxf(m, cm);              // finite: chunk has >= 1 token
    const float alpha = expf(m - m_new);           // 0 on the first chunk
    const float e = (j < n) ? expf(s - m_new) : 0.f;
    p_s[tid] = e;
    float cs = wave_sum(e);
    if (lane == 0) red[wid] = cs;
    __syncthreads();
    cs = 0.f;
    for (int w = 0; w < kGenThreads / 64; ++w) cs += red[w];
    l = l * alpha + cs;
    m = m_new;
    const int cnt = min(kGenThreads, n - c);
#pragma unroll
    for (int i = 0; i < kGenMaxDim / kGenThreads; ++i) {
      const int d = tid + i * kGenThreads;
      if (d < Dv) {
        float a = acc[i] * alpha;
        for (int jj = 0; jj < cnt; ++jj) {
          const int jt = c + jj;
          const int64_t phys = bt[jt / kv.block_size];
          const int64_t idx = v_head + phys * vs[1] + static_cast<int64_t>(jt % kv.block_size) * vs[3] + d * vs[4];
          a += p_s[jj] * load_kv<kKvDtype>(vbase, idx);
        }
        acc[i] = a;
      }
    }
    __syncthreads();
  }

  const float inv = (n > 0) ? vscale / l : 0.f;
#pragma unroll
  for (int i = 0; i < kGenMaxDim / kGenThreads; ++i) {
    const int d = tid + i * kGenThreads;
    if (d < Dv) p.out_o[out_row * Dv + d] = acc[i] * inv;
  }
  if (tid == 0) p.out_lse[out_row] = (n > 0) ? m + logf(l) : -INFINITY;
}

size_t generic_workspace_bytes(const AttnParams&) { return 0; }

template <int kKv>
static hipError_t launch_generic_q(const AttnParams& p, dim3 grid) {
  if (p.q_dtype == DCP_F32)
    hipLaunchKernelGGL((generic_attn_kernel<kKv, DCP_F32>), grid, dim3(kGenThreads), 0, p.stream, p);
  else
    hipLaunchKernelGGL((generic_attn_kernel<kKv, DCP_BF16>), grid, dim3(kGenThreads), 0, p.stream, p);
  return hipGetLastError();
}

hipError_t launch_generic_attn(const AttnParams& p) {
  const int64_t n = static_cast<int64_t>(p.rank_count) * p.batch * p.q_len * p.num_q_heads;
  if (n == 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>(n));
  if (p.ev_begin) (void)hipEventRecord(p.ev_begin, p.stream);
  hipError_t e;
  switch (p.kv.dtype) {
    case DCP_F32: e = launch_generic_q<DCP_F32>(p, grid); break;
    case DCP_BF16: e = launch_generic_q<DCP_BF16>(p, grid); break;
    default: e = launch_generic_q<DCP_FP8_E4M3>(p, grid); break;
  }
  if (p.ev_end) (void)hipEventRecord(p.ev_end, p.stream);
  return e;
}

}  // namespace dcp
