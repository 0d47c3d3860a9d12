// Context gather for (chunked) prefill: the inverse of the slot mapping.
//
// Source: "Decode Context Parallel (DCP)" (vLLM Ascend design doc), section
// "Prefill and chunked prefill" (MLA gathers the context KV cache spread over
// the DCP group and restores request-contiguous order before the query chunk
// attends it); "DeepSeek V4.1 context parallelism", section "Cache
// ownership" (pages are copied as stored, quantised values included).
//
// Output row t (request-major, then position) is position x = t - cu[b] of
// request b, cu[b] <= t < cu[b + 1]. Its owner and pool row follow the
// layout of the slot mapping (layout.hip): owner (x / I) % D, block
// block_table[b][x / (bs D)], offset ((x / (I D)) I + x % I) % bs. One
// workgroup per 64 output rows: wave 0 finds each row's request (binary
// search in cu), owner and pool row; then every thread copies 16-byte chunks
// of the (token, head) rows, consecutive threads on consecutive chunks, so a
// row is one contiguous read from its owner's pool and the output is written
// front to back. Data is read and written once: non-temporal loads/stores.
// Unmapped positions (negative block id, virtual block past max_vblocks)
// produce zero rows.
#include <algorithm>

#include "common.h"

namespace dcp {

constexpr int kGatherRows = 64;
constexpr int kGatherGroup = 6;  // 16-byte chunks in flight per thread

struct GatherTensor {
  const char* pool;  // rank 0's pool
  int64_t st[5];     // element strides (rank, block, head, token, dim)
  char* out;         // [T, H, dim]
  int row_chunks;    // 16-byte chunks per (token, head) row
  uint32_t row_magic, tok_magic;  // c / row_chunks, c / (H * row_chunks) by umulhi
};

struct GatherParams {
  const int32_t* bt;
  int64_t bt_stride;
  int max_vblocks, num_reqs;
  const int64_t* cu;  // [num_reqs + 1]
  int64_t total;
  int dcp_size, interleave, block_size, heads, eb;
  GatherTensor k, v;  // v.pool == nullptr: K only
};

__device__ __forceinline__ void gather_rows(const GatherParams& p, const GatherTensor& g, int64_t t0, int n,
                                            const int64_t* s_row) {
  const int per_tok = p.heads * g.row_chunks;
  const int total = n * per_tok;
  const int tid = threadIdx.x;
  for (int c0 = 0; c0 < total; c0 += 256 * kGatherGroup) {
    u32x4_t data[kGatherGroup];
#pragma unroll
    for (int j = 0; j < kGatherGroup; ++j) {
      const int c = c0 + j * 256 + tid;
      data[j] = u32x4_t{0u, 0u, 0u, 0u};
      if (c < total) {
        const int i = static_cast<int>(__umulhi(static_cast<uint32_t>(c), g.tok_magic));
        const int rc = c - i * per_tok;
        const int h = static_cast<int>(__umulhi(static_cast<uint32_t>(rc), g.row_magic));
        const int k = rc - h * g.row_chunks;
        const int64_t row = s_row[i];
        if (row >= 0)
          data[j] = __builtin_nontemporal_load(
              reinterpret_cast<const u32x4_t*>(g.pool + (row + h * g.st[2]) * p.eb + 16 * k));
      }
    }
#pragma unroll
    for (int j = 0; j < kGatherGroup; ++j) {
      const int c = c0 + j * 256 + tid;
      if (c < total)  // output chunks are contiguous: token-major, then head, then chunk
        __builtin_nontemporal_store(data[j], reinterpret_cast<u32x4_t*>(g.out + ((t0 * per_tok) + c) * 16));
    }
  }
}

__global__ void __launch_bounds__(256) gather_context_kernel(GatherParams p) {
  __shared__ int64_t s_krow[kGatherRows];  // element offset of the row's head-0 K row, -1: unmapped
  __shared__ int64_t s_vrow[kGatherRows];
  const int tid = threadIdx.x;
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * kGatherRows;
  const int n = static_cast<int>(p.total - t0 < kGatherRows ? p.total - t0 : kGatherRows);
  if (tid < kGatherRows) {
    int64_t kr = -1, vr = -1;
    if (tid < n) {
      const int64_t t = t0 + tid;
      int lo = 0, hi = p.num_reqs - 1;  // the last request with cu[b] <= t (it holds t)
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (p.cu[mid] <= t) lo = mid;
        else hi = mid - 1;
      }
      const int b = lo;
      const int64_t x = t - p.cu[b];
      const int64_t vb = x / (static_cast<int64_t>(p.block_size) * p.dcp_size);
      if (vb < p.max_vblocks) {
        const int32_t phys = p.bt[static_cast<int64_t>(b) * p.bt_stride + vb];
        if (phys >= 0) {
          const int owner = static_cast<int>((x / p.interleave) % p.dcp_size);
          const int64_t lp = (x / (static_cast<int64_t>(p.interleave) * p.dcp_size)) * p.interleave + x % p.interleave;
          const int64_t off = lp % p.block_size;
          kr = owner * p.k.st[0] + phys * p.k.st[1] + off * p.k.st[3];
          if (p.v.pool) vr = owner * p.v.st[0] + phys * p.v.st[1] + off * p.v.st[3];
        }
      }
    }
    s_krow[tid] = kr;
    s_vrow[tid] = vr;
  }
  __syncthreads();
  gather_rows(p, p.k, t0, n, s_krow);
  if (p.v.pool) gather_rows(p, p.v, t0, n, s_vrow);
}

static GatherTensor gather_tensor(const void* pool, const int64_t* st, void* out, int heads, int dim, int eb) {
  GatherTensor g;
  g.pool = static_cast<const char*>(pool);
  for (int i = 0; i < 5; ++i) g.st[i] = st[i];
  g.out = static_cast<char*>(out);
  g.row_chunks = dim * eb / 16;
  const uint64_t rc = static_cast<uint64_t>(g.row_chunks), tc = rc * static_cast<uint64_t>(heads);
  g.row_magic = static_cast<uint32_t>(((uint64_t(1) << 32) + rc - 1) / rc);
  g.tok_magic = static_cast<uint32_t>(((uint64_t(1) << 32) + tc - 1) / tc);
  return g;
}

bool gather_supported(const dcp_kv_cache_t& kv, bool with_v) {
  const int eb = kv.dtype == DCP_F32 ? 4 : kv.dtype == DCP_BF16 ? 2 : 1;
  auto rows_ok = [&](const void* base, const int64_t* st, int dim) {
    if (st[4] != 1 || (static_cast<int64_t>(dim) * eb) % 16 != 0) return false;
    for (int i = 0; i < 4; ++i)
      if ((st[i] * eb) % 16 != 0) return false;
    return reinterpret_cast<uintptr_t>(base) % 16 == 0;
  };
  if (!rows_ok(kv.k, kv.k_stride, kv.head_dim_k)) return false;
  if (with_v && !rows_ok(kv.v, kv.v_stride, kv.head_dim_v)) return false;
  // umulhi divisions are exact while chunk number * divisor < 2^32: chunk numbers of a
  // 64-row tile below 2^20, divisors (chunks per token) below 2^12
  const int64_t per_tok = static_cast<int64_t>(kv.num_kv_heads) * std::max(kv.head_dim_k, kv.head_dim_v) * eb / 16;
  return per_tok < (1 << 12) && per_tok * kGatherRows < (1 << 20);
}

hipError_t launch_gather_context(const dcp_kv_cache_t& kv, int dcp_size, int interleave, const int32_t* block_table,
                                 int num_reqs, int64_t bt_stride, int max_vblocks, const int64_t* cu_ctx,
                                 int64_t total, void* out_k, void* out_v, hipStream_t stream) {
  if (total == 0) return hipSuccess;
  GatherParams p;
  p.bt = block_table;
  p.bt_stride = bt_stride;
  p.max_vblocks = max_vblocks;
  p.num_reqs = num_reqs;
  p.cu = cu_ctx;
  p.total = total;
  p.dcp_size = dcp_size;
  p.interleave = interleave;
  p.block_size = kv.block_size;
  p.heads = kv.num_kv_heads;
  p.eb = kv.dtype == DCP_F32 ? 4 : kv.dtype == DCP_BF16 ? 2 : 1;
  p.k = gather_tensor(kv.k, kv.k_stride, out_k, p.heads, kv.head_dim_k, p.eb);
  if (out_v) {
    p.v = gather_tensor(kv.v, kv.v_stride, out_v, p.heads, kv.head_dim_v, p.eb);
  } else {
    p.v = p.k;
    p.v.pool = nullptr;
  }
  const int64_t grid = (total + kGatherRows - 1) / kGatherRows;
  hipLaunchKernelGGL(gather_context_kernel, dim3(static_cast<unsigned>(grid)), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace dcp
