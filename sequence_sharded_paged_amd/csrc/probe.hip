// Measurement aid: the device's sustained streaming-read rate, the ceiling
// the decode kernels' HBM fractions are set against next to the 8 TB/s
// specification.
//
// Every byte of the buffer is read exactly once with 16-byte non-temporal
// loads: each wavefront streams one contiguous run of the buffer, consecutive
// lanes on consecutive 16 bytes (1 KB per load), eight loads in flight per
// lane, over a grid of four 256-thread workgroups per CU. On MI355X this
// reads ≈7.06 TB/s, where a grid-stride walk (consecutive wavefronts on
// consecutive 1 KB runs) reaches 6.0–6.5 TB/s, so the contiguous runs are
// what the ceiling is taken with. Each workgroup XORs what it read into one
// 32-bit digest, so that no load is dead and a test can check the kernel
// covered the buffer exactly.
#include "common.h"

namespace dcp {

constexpr int kProbeThreads = 256;
constexpr int kProbeUnroll = 8;  // loads in flight per lane

__global__ void __launch_bounds__(kProbeThreads) hbm_read_probe_kernel(const u32x4_t* __restrict__ buf, int64_t n16,
                                                                       uint32_t* __restrict__ digest) {
  __shared__ uint32_t s_acc[kProbeThreads / 64];
  const int lane = threadIdx.x & 63;
  const int64_t waves = static_cast<int64_t>(gridDim.x) * (kProbeThreads / 64);
  const int64_t wid = static_cast<int64_t>(blockIdx.x) * (kProbeThreads / 64) + (threadIdx.x >> 6);
  const int64_t per = (n16 + waves - 1) / waves;
  const int64_t lo = wid * per, hi = lo + per < n16 ? lo + per : n16;
  uint32_t acc = 0;
  int64_t c = lo + lane;
  for (; c + 64 * (kProbeUnroll - 1) < hi; c += 64 * kProbeUnroll) {
    u32x4_t v[kProbeUnroll];
#pragma unroll
    for (int k = 0; k < kProbeUnroll; ++k) v[k] = __builtin_nontemporal_load(buf + c + 64 * k);
#pragma unroll
    for (int k = 0; k < kProbeUnroll; ++k) acc ^= v[k][0] ^ v[k][1] ^ v[k][2] ^ v[k][3];
  }
  for (; c < hi; c += 64) {
    const u32x4_t v = __builtin_nontemporal_load(buf + c);
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) acc ^= static_cast<uint32_t>(__shfl_xor(static_cast<int>(acc), o, 64));
  if ((threadIdx.x & 63) == 0) s_acc[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t a = 0;
#pragma unroll
    for (int w = 0; w < kProbeThreads / 64; ++w) a ^= s_acc[w];
    digest[blockIdx.x] = a;
  }
}

int hbm_read_probe_blocks() { return 4 * device_cu_count(); }

hipError_t launch_hbm_read_probe(const void* buf, int64_t bytes, uint32_t* digest, int blocks, hipStream_t s) {
  hipLaunchKernelGGL(hbm_read_probe_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kProbeThreads), 0, s,
                     static_cast<const u32x4_t*>(buf), bytes / 16, digest);
  return hipGetLastError();
}

}  // namespace dcp
