// C ABI entry points of libdcp: host-side validation, kernel selection and
// launch. The operations and their sources are documented in include/dcp.h.
#include <algorithm>
#include <climits>
#include <atomic>
#include <cmath>
#include <mutex>
#include <utility>
#include <vector>

#include "common.h"

namespace dcp {

// CU count of the current device, cached per device (static storage starts
// zeroed; concurrent first calls store the same value).
int device_cu_count() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  if (dev < 64 && cache[dev].load() > 0) return cache[dev].load();
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
  if (dev < 64) cache[dev].store(cus);
  return cus;
}

static int check_layout_args(int32_t block_size, int32_t dcp_size, int32_t interleave) {
  if (block_size < 1 || dcp_size < 1 || interleave < 1) return DCP_ERR_INVALID_ARG;
  if (block_size % interleave != 0) return DCP_ERR_INVALID_ARG;
  return DCP_OK;
}

static bool valid_dtype(int32_t t) { return t == DCP_F32 || t == DCP_BF16 || t == DCP_FP8_E4M3; }

// Validation shared by the size query and the launch. Fills p (except the
// output, workspace and stream fields) and picks the kernel family.
static int validate_attn(int32_t batch, int32_t q_len, int32_t num_q_heads, int32_t q_dtype,
                         const dcp_kv_cache_t* kv, int32_t rank_count, int32_t algo, AttnParams& p,
                         AttnKernel& kernel) {
  if (!kv) return DCP_ERR_INVALID_ARG;
  if (batch < 0 || num_q_heads < 1 || rank_count < 1) return DCP_ERR_INVALID_ARG;
  if (q_len < 1 || q_len > 64) return DCP_ERR_INVALID_ARG;
  if (static_cast<int64_t>(batch) * q_len >= (int64_t(1) << 31)) return DCP_ERR_INVALID_ARG;
  if (q_dtype != DCP_F32 && q_dtype != DCP_BF16) return DCP_ERR_UNSUPPORTED;
  if (!valid_dtype(kv->dtype)) return DCP_ERR_UNSUPPORTED;
  if (kv->num_kv_heads < 1 || num_q_heads % kv->num_kv_heads != 0) return DCP_ERR_INVALID_ARG;
  if (kv->block_size < 1 || kv->num_blocks < 1) return DCP_ERR_INVALID_ARG;
  if (kv->head_dim_k < 1 || kv->head_dim_v < 1) return DCP_ERR_INVALID_ARG;
  if (!kv->v && kv->head_dim_v > kv->head_dim_k) return DCP_ERR_INVALID_ARG;
  if (kv->head_dim_k > 1024 || kv->head_dim_v > 1024) return DCP_ERR_UNSUPPORTED;
  if (kv->dtype == DCP_FP8_E4M3 && (!kv->k_scale || !kv->v_scale)) return DCP_ERR_INVALID_ARG;
  if (algo != DCP_ALGO_AUTO && algo != DCP_ALGO_GENERIC && algo != DCP_ALGO_FAST) return DCP_ERR_INVALID_ARG;
  p.q_dtype = q_dtype;
  p.batch = batch;
  p.num_q_heads = num_q_heads;
  p.group = num_q_heads / kv->num_kv_heads;
  p.kv = *kv;
  p.rank_count = rank_count;
  p.q_len = q_len;
  // GQA MFMA: the query tokens of a request share the 16 columns of the
  // score tile (16 / group of them per unit); MLA MFMA: one per unit.
  auto tokens_per_unit = [&](int tpu) {
    p.tpu = tpu;
    p.ntg = (q_len + tpu - 1) / tpu;
  };
  // The MFMA kernels' split plan names units (rank, request, KV head, token
  // group) with 32-bit indices.
  auto units_fit = [&]() {
    return static_cast<int64_t>(rank_count) * batch * kv->num_kv_heads * p.ntg <= INT32_MAX;
  };
  tokens_per_unit(std::max(1, std::min(q_len, 16 / std::max(1, p.group))));
  if (algo != DCP_ALGO_GENERIC && units_fit() && gqa_supported(p)) {
    kernel = AttnKernel::GqaMfma;
    return DCP_OK;
  }
  tokens_per_unit(1);
  if (algo == DCP_ALGO_GENERIC) {
    kernel = AttnKernel::Generic;
  } else if (units_fit() && mla_supported(p)) {
    kernel = AttnKernel::MlaMfma;
  } else if (algo == DCP_ALGO_FAST) {
    return DCP_ERR_UNSUPPORTED;
  } else {
    kernel = AttnKernel::Generic;
  }
  // the generic kernel runs one workgroup per (rank, request, query token,
  // query head), indexed in 32 bits
  if (kernel == AttnKernel::Generic &&
      static_cast<int64_t>(rank_count) * batch * q_len * num_q_heads > INT32_MAX)
    return DCP_ERR_UNSUPPORTED;
  return DCP_OK;
}

static size_t workspace_for(const AttnParams& p, AttnKernel k) {
  switch (k) {
    case AttnKernel::GqaMfma: return gqa_workspace_bytes(p);
    case AttnKernel::MlaMfma: return mla_workspace_bytes(p);
    default: return generic_workspace_bytes(p);
  }
}

// Kernel timing for benchmarks (dcp_profile_enable / dcp_profile_collect):
// per host thread, a growing pool of event pairs, one pair per profiled call.
struct ProfileState {
  bool on = false;
  std::vector<std::pair<hipEvent_t, hipEvent_t>> events;
  size_t used = 0;
  int device = -1;
};
static thread_local ProfileState g_prof;

static void profile_release() {
  for (auto& e : g_prof.events) {
    (void)hipEventDestroy(e.first);
    (void)hipEventDestroy(e.second);
  }
  g_prof.events.clear();
  g_prof.used = 0;
}

// Event pair for the next profiled call, or {nullptr, nullptr}.
static std::pair<hipEvent_t, hipEvent_t> profile_next() {
  if (!g_prof.on) return {nullptr, nullptr};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return {nullptr, nullptr};
  if (dev != g_prof.device) {
    profile_release();
    g_prof.device = dev;
  }
  if (g_prof.used == g_prof.events.size()) {
    hipEvent_t a = nullptr, b = nullptr;
    if (hipEventCreate(&a) != hipSuccess) return {nullptr, nullptr};
    if (hipEventCreate(&b) != hipSuccess) {
      (void)hipEventDestroy(a);
      return {nullptr, nullptr};
    }
    g_prof.events.emplace_back(a, b);
  }
  return g_prof.events[g_prof.used++];
}

}  // namespace dcp

using namespace dcp;

extern "C" {

int dcp_abi_version(void) { return 1; }

const char* dcp_status_string(int status) {
  switch (status) {
    case DCP_OK: return "ok";
    case DCP_ERR_INVALID_ARG: return "invalid argument";
    case DCP_ERR_UNSUPPORTED: return "unsupported dtype, geometry or layout";
    case DCP_ERR_WORKSPACE: return "workspace too small";
    case DCP_ERR_HIP: return "HIP runtime or launch error";
    case DCP_ERR_SCRATCH: return "needs more than the library's fixed device scratch";
    default: return "unknown status";
  }
}

int dcp_local_seq_lens(const int32_t* seq_lens, int32_t num_reqs, int32_t block_size, int32_t dcp_size,
                       int32_t interleave, int32_t* local_lens, void* stream) {
  if (int st = check_layout_args(block_size, dcp_size, interleave)) return st;
  if (num_reqs < 0) return DCP_ERR_INVALID_ARG;
  if (num_reqs == 0) return DCP_OK;
  if (!seq_lens || !local_lens) return DCP_ERR_INVALID_ARG;
  return launch_local_seq_lens(seq_lens, num_reqs, dcp_size, interleave, local_lens,
                               static_cast<hipStream_t>(stream)) == hipSuccess ? DCP_OK : DCP_ERR_HIP;
}

int dcp_check_block_table(const int32_t* block_table, int32_t num_reqs, int64_t block_table_stride,
                          int32_t max_vblocks, const int32_t* seq_lens, int32_t block_size, int32_t dcp_size,
                          int32_t num_blocks, int32_t* bad_count, void* stream) {
  if (block_size < 1 || dcp_size < 1 || num_reqs < 0 || max_vblocks < 0 || num_blocks < 0 ||
      block_table_stride < max_vblocks)
    return DCP_ERR_INVALID_ARG;
  if (!bad_count) return DCP_ERR_INVALID_ARG;
  if (num_reqs > 0 && !seq_lens) return DCP_ERR_INVALID_ARG;
  if (num_reqs > 0 && max_vblocks > 0 && !block_table) return DCP_ERR_INVALID_ARG;
  return launch_check_block_table(block_table, num_reqs, block_table_stride, max_vblocks, seq_lens, block_size,
                                  dcp_size, num_blocks, bad_count, static_cast<hipStream_t>(stream)) == hipSuccess
             ? DCP_OK
             : DCP_ERR_HIP;
}

int dcp_slot_mapping(const int64_t* positions, const int32_t* req_indices, int64_t num_tokens,
                     const int32_t* block_table, int32_t num_reqs, int64_t block_table_stride,
                     int32_t max_vblocks, int32_t block_size, int32_t dcp_size, int32_t interleave,
                     int64_t* slots, void* stream) {
  if (int st = check_layout_args(block_size, dcp_size, interleave)) return st;
  if (num_tokens < 0 || num_reqs < 0 || max_vblocks < 0 || block_table_stride < max_vblocks)
    return DCP_ERR_INVALID_ARG;
  if (num_tokens == 0) return DCP_OK;
  if (!positions || !req_indices || !slots) return DCP_ERR_INVALID_ARG;
  if (num_reqs > 0 && max_vblocks > 0 && !block_table) return DCP_ERR_INVALID_ARG;
  if (num_tokens > (int64_t(1) << 40)) return DCP_ERR_INVALID_ARG;
  return launch_slot_mapping(positions, req_indices, num_tokens, block_table, num_reqs, block_table_stride,
                             max_vblocks, block_size, dcp_size, interleave, slots,
                             static_cast<hipStream_t>(stream)) == hipSuccess ? DCP_OK : DCP_ERR_HIP;
}

}  // extern "C"

namespace dcp {

static size_t attn_workspace_size(int32_t batch, int32_t q_len, int32_t num_q_heads, int32_t q_dtype,
                                  const dcp_kv_cache_t* kv, int32_t rank_count, int32_t algo, int* status) {
  AttnParams p{};
  AttnKernel k = AttnKernel::Generic;
  const int st = validate_attn(batch, q_len, num_q_heads, q_dtype, kv, rank_count, algo, p, k);
  if (status) *status = st;
  if (st != DCP_OK) return 0;
  return workspace_for(p, k);
}

// Workspace of dcp_partial_decode_attn_noalloc, held by the library: one copy
// per device, loaded with the library's code on that device. On the host the
// array's name is only a stand-in for registration; kernels and copies get
// the device address that hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) char scratch[DCP_NOALLOC_SCRATCH_BYTES];

constexpr int kScratchDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kScratchDevices];  // per device; static storage starts null

// Address of the current device's scratch, looked up once per device.
static int scratch_of_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return DCP_ERR_HIP;
  if (dev >= kScratchDevices) return DCP_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return DCP_ERR_HIP;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return DCP_OK;
}

static int partial_attn(const void* q, int32_t q_dtype, int32_t batch, int32_t q_len, int32_t num_q_heads,
                        const dcp_kv_cache_t* kv, const int32_t* block_table, int64_t block_table_stride,
                        int32_t max_vblocks, const int32_t* local_lens, int32_t dcp_size, int32_t rank_begin,
                        int32_t rank_count, float softmax_scale, int32_t algo, float* out_o, float* out_lse,
                        void* workspace, size_t workspace_bytes, void* stream, bool profiled = true,
                        bool from_scratch = false) {
  AttnParams p{};
  AttnKernel k = AttnKernel::Generic;
  if (int st = validate_attn(batch, q_len, num_q_heads, q_dtype, kv, rank_count, algo, p, k)) return st;
  if (dcp_size < 1 || rank_begin < 0 || rank_begin + rank_count > dcp_size) return DCP_ERR_INVALID_ARG;
  if (max_vblocks < 0 || block_table_stride < max_vblocks) return DCP_ERR_INVALID_ARG;
  if (!std::isfinite(softmax_scale)) return DCP_ERR_INVALID_ARG;
  if (batch == 0) return DCP_OK;
  if (!q || !kv->k || !local_lens || !out_o || !out_lse) return DCP_ERR_INVALID_ARG;
  if (max_vblocks > 0 && !block_table) return DCP_ERR_INVALID_ARG;
  const size_t need = workspace_for(p, k);
  if (from_scratch && need > 0) {  // the library's own workspace, after every other check
    if (need > DCP_NOALLOC_SCRATCH_BYTES) return DCP_ERR_SCRATCH;
    if (int st = scratch_of_current_device(&workspace)) return st;
    workspace_bytes = DCP_NOALLOC_SCRATCH_BYTES;
  }
  if (workspace_bytes < need || (need > 0 && !workspace)) return DCP_ERR_WORKSPACE;
  p.q = q;
  p.block_table = block_table;
  p.bt_stride = block_table_stride;
  p.max_vblocks = max_vblocks;
  p.local_lens = local_lens;
  p.dcp_size = dcp_size;
  p.rank_begin = rank_begin;
  p.softmax_scale = softmax_scale;
  p.out_o = out_o;
  p.out_lse = out_lse;
  p.workspace = workspace;
  p.workspace_bytes = workspace_bytes;
  p.stream = static_cast<hipStream_t>(stream);
  const auto ev = profiled ? profile_next() : std::pair<hipEvent_t, hipEvent_t>{nullptr, nullptr};
  p.ev_begin = ev.first;
  p.ev_end = ev.second;
  hipError_t e;
  switch (k) {
    case AttnKernel::GqaMfma: e = launch_gqa_attn(p); break;
    case AttnKernel::MlaMfma: e = launch_mla_attn(p); break;
    default: e = launch_generic_attn(p); break;
  }
  return e == hipSuccess ? DCP_OK : DCP_ERR_HIP;
}

// Workspace of dcp_partial_segment_attn: the segment's partial O [B, Hq, Dv]
// and LSE [B, Hq], then the attention workspace for the segment pool.
struct SegmentWs {
  size_t o_bytes, lse_bytes, attn_bytes;
  size_t total() const { return o_bytes + lse_bytes + attn_bytes; }
};

static int segment_ws(int32_t batch, int32_t num_q_heads, int32_t q_dtype, const dcp_kv_cache_t* seg_kv,
                      int32_t algo, SegmentWs& w) {
  int st = DCP_OK;
  w.attn_bytes = attn_workspace_size(batch, 1, num_q_heads, q_dtype, seg_kv, 1, algo, &st);
  if (st != DCP_OK) return st;
  w.o_bytes = align_up(static_cast<size_t>(batch) * num_q_heads * seg_kv->head_dim_v * sizeof(float), 256);
  w.lse_bytes = align_up(static_cast<size_t>(batch) * num_q_heads * sizeof(float), 256);
  return DCP_OK;
}

}  // namespace dcp

extern "C" {

size_t dcp_partial_segment_attn_workspace_size(int32_t batch, int32_t num_q_heads, int32_t q_dtype,
                                               const dcp_kv_cache_t* seg_kv, int32_t algo, int* status) {
  SegmentWs w{};
  const int st = segment_ws(batch, num_q_heads, q_dtype, seg_kv, algo, w);
  if (status) *status = st;
  return st == DCP_OK ? w.total() : 0;
}

int dcp_partial_segment_attn(const void* q, int32_t q_dtype, int32_t batch, int32_t num_q_heads,
                             const dcp_kv_cache_t* seg_kv, const int32_t* seg_block_table,
                             int64_t seg_block_table_stride, int32_t seg_max_vblocks, const int32_t* seg_lens,
                             float softmax_scale, int32_t algo, int32_t seg_rank, int32_t rank_begin,
                             int32_t rank_count, float* part_o, float* part_lse, void* workspace,
                             size_t workspace_bytes, void* stream) {
  SegmentWs w{};
  if (int st = segment_ws(batch, num_q_heads, q_dtype, seg_kv, algo, w)) return st;
  if (rank_begin < 0 || rank_count < 1 || seg_rank < 0) return DCP_ERR_INVALID_ARG;
  if (seg_rank < rank_begin || seg_rank >= rank_begin + rank_count) return DCP_OK;  // another GPU's rank counts it
  if (batch == 0) return DCP_OK;
  if (!part_o || !part_lse) return DCP_ERR_INVALID_ARG;
  if (workspace_bytes < w.total() || !workspace) return DCP_ERR_WORKSPACE;
  char* ws = static_cast<char*>(workspace);
  float* o_seg = reinterpret_cast<float*>(ws);
  float* lse_seg = reinterpret_cast<float*>(ws + w.o_bytes);
  void* attn_ws = ws + w.o_bytes + w.lse_bytes;
  // the segment as a one-rank pool: its lengths are its local lengths
  if (int st = partial_attn(q, q_dtype, batch, 1, num_q_heads, seg_kv, seg_block_table, seg_block_table_stride,
                            seg_max_vblocks, seg_lens, 1, 0, 1, softmax_scale, algo, o_seg, lse_seg, attn_ws,
                            w.attn_bytes, stream, false))
    return st;
  const int64_t rows = static_cast<int64_t>(batch) * num_q_heads;
  const int64_t r = seg_rank - rank_begin;
  return launch_lse_fold(part_o + r * rows * seg_kv->head_dim_v, part_lse + r * rows, o_seg, lse_seg, rows,
                         seg_kv->head_dim_v, static_cast<hipStream_t>(stream)) == hipSuccess
             ? DCP_OK
             : DCP_ERR_HIP;
}

size_t dcp_partial_decode_attn_workspace_size(int32_t batch, int32_t num_q_heads, int32_t q_dtype,
                                              const dcp_kv_cache_t* kv, int32_t rank_count, int32_t algo,
                                              int* status) {
  return attn_workspace_size(batch, 1, num_q_heads, q_dtype, kv, rank_count, algo, status);
}

int dcp_partial_decode_attn(const void* q, int32_t q_dtype, int32_t batch, int32_t num_q_heads,
                            const dcp_kv_cache_t* kv, const int32_t* block_table, int64_t block_table_stride,
                            int32_t max_vblocks, const int32_t* local_lens, int32_t dcp_size, int32_t rank_begin,
                            int32_t rank_count, float softmax_scale, int32_t algo, float* out_o, float* out_lse,
                            void* workspace, size_t workspace_bytes, void* stream) {
  return partial_attn(q, q_dtype, batch, 1, num_q_heads, kv, block_table, block_table_stride, max_vblocks,
                      local_lens, dcp_size, rank_begin, rank_count, softmax_scale, algo, out_o, out_lse, workspace,
                      workspace_bytes, stream);
}

int dcp_partial_decode_attn_noalloc(const void* q, int32_t q_dtype, int32_t batch, int32_t num_q_heads,
                                    const dcp_kv_cache_t* kv, const int32_t* block_table,
                                    int64_t block_table_stride, int32_t max_vblocks, const int32_t* local_lens,
                                    int32_t dcp_size, int32_t rank_begin, int32_t rank_count, float softmax_scale,
                                    int32_t algo, float* out_o, float* out_lse, void* stream) {
  return partial_attn(q, q_dtype, batch, 1, num_q_heads, kv, block_table, block_table_stride, max_vblocks,
                      local_lens, dcp_size, rank_begin, rank_count, softmax_scale, algo, out_o, out_lse, nullptr, 0,
                      stream, false, true);
}

size_t dcp_partial_verify_attn_workspace_size(int32_t batch, int32_t q_len, int32_t num_q_heads, int32_t q_dtype,
                                              const dcp_kv_cache_t* kv, int32_t rank_count, int32_t algo,
                                              int* status) {
  return attn_workspace_size(batch, q_len, num_q_heads, q_dtype, kv, rank_count, algo, status);
}

int dcp_partial_verify_attn(const void* q, int32_t q_dtype, int32_t batch, int32_t q_len, int32_t num_q_heads,
                            const dcp_kv_cache_t* kv, const int32_t* block_table, int64_t block_table_stride,
                            int32_t max_vblocks, const int32_t* local_lens, int32_t dcp_size, int32_t rank_begin,
                            int32_t rank_count, float softmax_scale, int32_t algo, float* out_o, float* out_lse,
                            void* workspace, size_t workspace_bytes, void* stream) {
  return partial_attn(q, q_dtype, batch, q_len, num_q_heads, kv, block_table, block_table_stride, max_vblocks,
                      local_lens, dcp_size, rank_begin, rank_count, softmax_scale, algo, out_o, out_lse, workspace,
                      workspace_bytes, stream);
}

int dcp_hbm_read_probe_blocks(void) {
  const int b = hbm_read_probe_blocks();
  return b > 0 ? b : DCP_ERR_HIP;
}

int dcp_hbm_read_probe(const void* buf, int64_t bytes, uint32_t* digest, int32_t digest_len, void* stream) {
  if (bytes < 0 || bytes % 16 != 0 || digest_len < 1) return DCP_ERR_INVALID_ARG;
  if (bytes == 0) return DCP_OK;
  if (!buf || !digest || reinterpret_cast<uintptr_t>(buf) % 16 != 0) return DCP_ERR_INVALID_ARG;
  const int blocks = hbm_read_probe_blocks();
  if (blocks < 1) return DCP_ERR_HIP;
  if (digest_len < blocks) return DCP_ERR_INVALID_ARG;
  return launch_hbm_read_probe(buf, bytes, digest, blocks, static_cast<hipStream_t>(stream)) == hipSuccess
             ? DCP_OK
             : DCP_ERR_HIP;
}

int dcp_profile_enable(int on) {
  g_prof.on = on != 0;
  g_prof.used = 0;
  return DCP_OK;
}

int dcp_profile_collect(double* total_ms, int32_t* launches) {
  if (!total_ms || !launches) return DCP_ERR_INVALID_ARG;
  double sum = 0.0;
  for (size_t i = 0; i < g_prof.used; ++i) {
    float ms = 0.f;
    if (hipEventSynchronize(g_prof.events[i].second) != hipSuccess ||
        hipEventElapsedTime(&ms, g_prof.events[i].first, g_prof.events[i].second) != hipSuccess)
      return DCP_ERR_HIP;
    sum += ms;
  }
  *total_ms = sum;
  *launches = static_cast<int32_t>(g_prof.used);
  g_prof.used = 0;
  return DCP_OK;
}

int dcp_gather_context(const dcp_kv_cache_t* kv, int32_t dcp_size, int32_t interleave, const int32_t* block_table,
                       int32_t num_reqs, int64_t block_table_stride, int32_t max_vblocks, const int64_t* cu_ctx,
                       int64_t total_tokens, void* out_k, void* out_v, void* stream) {
  if (!kv) return DCP_ERR_INVALID_ARG;
  if (int st = check_layout_args(kv->block_size, dcp_size, interleave)) return st;
  if (!valid_dtype(kv->dtype)) return DCP_ERR_UNSUPPORTED;
  if (num_reqs < 0 || total_tokens < 0 || max_vblocks < 0 || block_table_stride < max_vblocks)
    return DCP_ERR_INVALID_ARG;
  if (kv->num_kv_heads < 1 || kv->head_dim_k < 1 || kv->head_dim_v < 1 || kv->num_blocks < 1)
    return DCP_ERR_INVALID_ARG;
  if (out_v && !kv->v) return DCP_ERR_INVALID_ARG;  // MLA: the value is part of the gathered K row
  if (total_tokens == 0) return DCP_OK;
  if (num_reqs == 0 || !cu_ctx || !out_k || !kv->k) return DCP_ERR_INVALID_ARG;
  if (max_vblocks > 0 && !block_table) return DCP_ERR_INVALID_ARG;
  if (total_tokens >= (int64_t(1) << 37)) return DCP_ERR_INVALID_ARG;
  if (!gather_supported(*kv, out_v != nullptr)) return DCP_ERR_UNSUPPORTED;
  return launch_gather_context(*kv, dcp_size, interleave, block_table, num_reqs, block_table_stride, max_vblocks,
                               cu_ctx, total_tokens, out_k, out_v, static_cast<hipStream_t>(stream)) == hipSuccess
             ? DCP_OK
             : DCP_ERR_HIP;
}

int dcp_kv_cache_write(const void* k_new, const void* v_new, int32_t src_dtype, int64_t num_tokens,
                       const int64_t* slots, int32_t num_ranks, const dcp_kv_cache_t* kv, void* stream) {
  if (!kv || num_tokens < 0 || num_ranks < 1) return DCP_ERR_INVALID_ARG;
  if (src_dtype != DCP_F32 && src_dtype != DCP_BF16) return DCP_ERR_UNSUPPORTED;
  if (!valid_dtype(kv->dtype)) return DCP_ERR_UNSUPPORTED;
  if (num_ranks > 64) return DCP_ERR_UNSUPPORTED;
  if (kv->num_kv_heads < 1 || kv->block_size < 1 || kv->num_blocks < 1) return DCP_ERR_INVALID_ARG;
  if (kv->head_dim_k < 1 || kv->head_dim_v < 1) return DCP_ERR_INVALID_ARG;
  if ((v_new == nullptr) != (kv->v == nullptr)) return DCP_ERR_INVALID_ARG;
  if (!kv->v && kv->head_dim_v > kv->head_dim_k) return DCP_ERR_INVALID_ARG;
  if (kv->head_dim_k % 8 != 0 || (kv->v && kv->head_dim_v % 8 != 0)) return DCP_ERR_UNSUPPORTED;
  if (int64_t(kv->num_kv_heads) * (kv->head_dim_k + kv->head_dim_v) > (int64_t(1) << 24)) return DCP_ERR_UNSUPPORTED;
  if (kv->num_kv_heads > 65535) return DCP_ERR_UNSUPPORTED;  // one grid row per head
  if (kv->head_dim_k + (kv->v ? kv->head_dim_v : 0) > 8192) return DCP_ERR_UNSUPPORTED;
  if (int64_t(kv->num_blocks) * kv->block_size >= (int64_t(1) << 56)) return DCP_ERR_UNSUPPORTED;
  if (kv->dtype == DCP_FP8_E4M3 && (!kv->k_scale || (kv->v && !kv->v_scale))) return DCP_ERR_INVALID_ARG;
  if (num_tokens > (int64_t(1) << 33)) return DCP_ERR_INVALID_ARG;
  if (num_tokens * kv->num_kv_heads >= (int64_t(1) << 33)) return DCP_ERR_UNSUPPORTED;  // grid size
  if (num_tokens == 0) return DCP_OK;
  if (!k_new || !slots || !kv->k) return DCP_ERR_INVALID_ARG;
  if (reinterpret_cast<uintptr_t>(k_new) % 16 != 0 || reinterpret_cast<uintptr_t>(v_new) % 16 != 0)
    return DCP_ERR_UNSUPPORTED;
  return launch_kv_write(k_new, v_new, src_dtype == DCP_BF16, num_tokens, slots, num_ranks, *kv,
                         static_cast<hipStream_t>(stream)) == hipSuccess ? DCP_OK : DCP_ERR_HIP;
}

int dcp_lse_merge(const float* part_o, const float* part_lse, int32_t num_parts, int32_t batch, int32_t num_heads,
                  int32_t head_dim_v, const float* sink, int32_t out_dtype, void* out_o, float* out_lse,
                  void* stream) {
  if (num_parts < 1 || num_parts > 64 || batch < 0 || num_heads < 1 || head_dim_v < 1 || head_dim_v > 4096)
    return DCP_ERR_INVALID_ARG;
  if (out_dtype != DCP_F32 && out_dtype != DCP_BF16) return DCP_ERR_UNSUPPORTED;
  if (batch == 0) return DCP_OK;
  if (!part_o || !part_lse || !out_o) return DCP_ERR_INVALID_ARG;
  return launch_lse_merge(part_o, part_lse, num_parts, batch, num_heads, head_dim_v, sink, out_dtype, out_o,
                          out_lse, static_cast<hipStream_t>(stream)) == hipSuccess ? DCP_OK : DCP_ERR_HIP;
}

}  // extern "C"
