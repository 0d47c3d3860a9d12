// DCP token placement kernels: per-rank context lengths and slot mapping.
//
// Source: "Decode Context Parallel (DCP)" (vLLM Ascend design doc), section
// "KV-cache layout": a virtual block holds block_size * dcp_size tokens and
// token x goes to rank ((x % (block_size*dcp_size)) / interleave) % dcp_size,
// with block_size % interleave == 0. "DeepSeek V4.1 context parallelism",
// section "Cache ownership": writes map virtual slots to local slots and mask
// the ranks that do not own the token.
//
// Closed forms used here (each rank keeps the tokens it owns in ascending
// position order; block_size % interleave == 0 makes every rank own exactly
// block_size tokens of each full virtual block):
//   owner(x)     = (x / interleave) % dcp_size
//   local_pos(x) = (x / (interleave*dcp_size)) * interleave + x % interleave
//   local_pos(x) / block_size == x / (block_size*dcp_size)   (virtual block)
//   len_r(L)     = full*interleave + clamp(rem - r*interleave, 0, interleave),
//                  full = L / (interleave*dcp_size), rem = L - full*interleave*dcp_size
#include "common.h"

namespace dcp {

__global__ void __launch_bounds__(256) local_seq_lens_kernel(const int32_t* __restrict__ seq_lens,
                                                             int num_reqs, int dcp_size, int interleave,
                                                             int32_t* __restrict__ local_lens) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= static_cast<int64_t>(num_reqs) * dcp_size) return;
  const int b = static_cast<int>(i / dcp_size), r = static_cast<int>(i % dcp_size);
  const int64_t L = max(seq_lens[b], 0);
  const int64_t round = static_cast<int64_t>(interleave) * dcp_size;
  const int64_t full = L / round;
  const int64_t rem = L - full * round;
  const int64_t extra = min(max(rem - static_cast<int64_t>(r) * interleave, int64_t(0)),
                            static_cast<int64_t>(interleave));
  local_lens[i] = static_cast<int32_t>(full * interleave + extra);
}

__global__ void __launch_bounds__(256) slot_mapping_kernel(
    const int64_t* __restrict__ positions, const int32_t* __restrict__ req_indices,
    int64_t num_tokens, const int32_t* __restrict__ block_table, int num_reqs, int64_t bt_stride,
    int max_vblocks, int block_size, int dcp_size, int interleave, int64_t* __restrict__ slots) {
  const int64_t t = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (t >= num_tokens) return;
  const int64_t x = positions[t];
  const int b = req_indices[t];
  int owner = -1;
  int64_t slot = -1;
  if (x >= 0 && b >= 0 && b < num_reqs) {
    const int64_t vb = x / (static_cast<int64_t>(block_size) * dcp_size);
    if (vb < max_vblocks) {
      const int32_t phys = block_table[static_cast<int64_t>(b) * bt_stride + vb];
      if (phys >= 0) {
        owner = static_cast<int>((x / interleave) % dcp_size);
        const int64_t lp = (x / (static_cast<int64_t>(interleave) * dcp_size)) * interleave + x % interleave;
        slot = static_cast<int64_t>(phys) * block_size + lp % block_size;
      }
    }
  }
  for (int r = 0; r < dcp_size; ++r) slots[static_cast<int64_t>(r) * num_tokens + t] = (r == owner) ? slot : -1;
}

// Block-table check: one workgroup per request counts the virtual blocks its
// length needs whose entry is missing (vb >= max_vblocks) or outside the pool;
// a wavefront reduction, then one atomic add per wavefront.
__global__ void check_clear_kernel(int32_t* bad) { *bad = 0; }

__global__ void __launch_bounds__(256) check_block_table_kernel(const int32_t* __restrict__ bt, int64_t bt_stride,
                                                              int max_vblocks, const int32_t* __restrict__ seq_lens,
                                                              int64_t span, int num_blocks, int32_t* bad) {
  const int b = blockIdx.x;
  const int64_t len = seq_lens[b] > 0 ? seq_lens[b] : 0;
  const int64_t need = (len + span - 1) / span;
  const int64_t have = need < max_vblocks ? need : max_vblocks;
  int64_t n = 0;
  for (int64_t vb = threadIdx.x; vb < have; vb += blockDim.x) {
    const int32_t id = bt[b * bt_stride + vb];
    n += (id < 0 || id >= num_blocks) ? 1 : 0;
  }
  if (threadIdx.x == 0) n += need - have;  // entries the table lacks
  for (int off = 32; off > 0; off >>= 1) n += __shfl_down(n, off, 64);
  if ((threadIdx.x & 63) == 0 && n > 0) {
    // add, saturating at INT32_MAX: a compare-and-swap loop (a failed swap
    // means another wavefront's single addition landed, so it ends)
    int32_t cur = atomicAdd(bad, 0);
    for (;;) {
      const int64_t sum = static_cast<int64_t>(cur) + n;
      const int32_t next = sum > INT32_MAX ? INT32_MAX : static_cast<int32_t>(sum);
      const int32_t prev = atomicCAS(bad, cur, next);
      if (prev == cur) break;
      cur = prev;
    }
  }
}

hipError_t launch_check_block_table(const int32_t* bt, int num_reqs, int64_t bt_stride, int max_vblocks,
                                    const int32_t* seq_lens, int block_size, int dcp_size, int num_blocks,
                                    int32_t* bad, hipStream_t s) {
  hipLaunchKernelGGL(check_clear_kernel, dim3(1), dim3(1), 0, s, bad);
  if (num_reqs > 0)
    hipLaunchKernelGGL(check_block_table_kernel, dim3(static_cast<unsigned>(num_reqs)), dim3(256), 0, s, bt, bt_stride,
                       max_vblocks, seq_lens, static_cast<int64_t>(block_size) * dcp_size, num_blocks, bad);
  return hipGetLastError();
}

hipError_t launch_local_seq_lens(const int32_t* seq_lens, int num_reqs, int dcp_size, int interleave,
                                 int32_t* local_lens, hipStream_t s) {
  const int64_t n = static_cast<int64_t>(num_reqs) * dcp_size;
  if (n == 0) return hipSuccess;
  const unsigned grid = static_cast<unsigned>((n + 255) / 256);
  hipLaunchKernelGGL(local_seq_lens_kernel, dim3(grid), dim3(256), 0, s, seq_lens, num_reqs, dcp_size,
                     interleave, local_lens);
  return hipGetLastError();
}

hipError_t launch_slot_mapping(const int64_t* positions, const int32_t* req_indices, int64_t num_tokens,
                               const int32_t* block_table, int num_reqs, int64_t bt_stride, int max_vblocks,
                               int block_size, int dcp_size, int interleave, int64_t* slots, hipStream_t s) {
  if (num_tokens == 0) return hipSuccess;
  const int64_t grid = (num_tokens + 255) / 256;
  hipLaunchKernelGGL(slot_mapping_kernel, dim3(static_cast<unsigned>(grid)), dim3(256), 0, s, positions,
                     req_indices, num_tokens, block_table, num_reqs, bt_stride, max_vblocks, block_size,
                     dcp_size, interleave, slots);
  return hipGetLastError();
}

}  // namespace dcp
