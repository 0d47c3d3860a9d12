/*
 * dcp.h - C ABI of libdcp: Decode Context Parallel (DCP) decode attention on
 * one AMD Instinct MI355X (gfx950).
 *
 * The library computes, for a paged KV cache sharded along the sequence
 * dimension over dcp_size ranks with an interleaved layout, the slot mapping
 * of tokens to ranks, the per-rank context lengths, each rank's partial decode
 * attention (O, LSE) over its local shard, and the log-sum-exp merge of the
 * partials with an optional attention sink applied once. All dcp_size virtual
 * ranks may live on the same GPU; a per-GPU deployment passes its own rank
 * through rank_begin / rank_count.
 *
 * Conventions for every entry point
 *   - Pointers named as device pointers must point to device memory of the
 *     current HIP device; the caller owns every buffer. The library
 *     allocates no device memory and keeps no state besides per-device
 *     attributes and, while profiling is enabled, a pool of HIP events.
 *   - All calls are stream-ordered on `stream` (a hipStream_t; NULL = the
 *     null stream) and never synchronize the host.
 *   - Arguments are validated on the host before anything is launched. On an
 *     error nothing is launched and a negative status is returned; nothing is
 *     printed and nothing aborts. Values that live in device memory (block
 *     ids, lengths, positions) are the caller's contract: block ids must lie
 *     in [0, num_blocks) wherever a kernel reads them.
 *   - Element strides are counted in elements of the stated type.
 */
#ifndef DCP_H
#define DCP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
enum {
  DCP_OK = 0,
  DCP_ERR_INVALID_ARG = -1, /* a size, pointer or relation between arguments is wrong */
  DCP_ERR_UNSUPPORTED = -2, /* valid but not implemented (dtype, head dims, layout) */
  DCP_ERR_WORKSPACE = -3,   /* workspace smaller than the size query returned */
  DCP_ERR_HIP = -4,         /* a HIP runtime call or kernel launch failed */
  DCP_ERR_SCRATCH = -5      /* the call needs more than the library's fixed scratch holds */
};

/* Element formats. DCP_FP8_E4M3 is the OCP 8-bit E4M3 format without
 * infinities (bias 7, max 448, S.1111.111 = NaN); fp8 values are dequantised
 * as code * scale[kv_head]. */
enum { DCP_F32 = 0, DCP_BF16 = 1, DCP_FP8_E4M3 = 2 };

/* Kernel selection for dcp_partial_decode_attn. AUTO picks the MFMA kernel
 * when the geometry is supported and the generic kernel otherwise; GENERIC
 * forces the generic fp32 kernel; FAST fails with DCP_ERR_UNSUPPORTED when no
 * MFMA kernel fits. */
enum { DCP_ALGO_AUTO = 0, DCP_ALGO_GENERIC = 1, DCP_ALGO_FAST = 2 };

/* Version of this ABI (incremented on incompatible change). */
int dcp_abi_version(void);

/* Static, human-readable text for a status code. Never NULL. */
const char* dcp_status_string(int status);

/*
 * dcp_local_seq_lens - per-rank context-length matrix.
 *
 * Source: "Decode Context Parallel (DCP)" (vLLM Ascend design doc), sections
 * "KV-cache layout" (token placement) and "Backend structure" (the per-rank
 * context-length matrix).
 *
 * local_lens[b * dcp_size + r] = number of positions x in [0, seq_lens[b])
 * whose target_rank is r, where
 *   target_rank = ((x % (block_size * dcp_size)) / interleave) % dcp_size.
 *
 * seq_lens   device, [num_reqs] int32, each >= 0 (negative is read as 0)
 * num_reqs   >= 0 (0: nothing is launched)
 * block_size >= 1; dcp_size >= 1; interleave >= 1; block_size % interleave == 0
 * local_lens device, [num_reqs, dcp_size] int32, row-major, rank fastest
 * Errors: DCP_ERR_INVALID_ARG for a bad size or relation or a NULL pointer
 * when num_reqs > 0; DCP_ERR_HIP if the launch fails.
 */
int dcp_local_seq_lens(const int32_t* seq_lens, int32_t num_reqs, int32_t block_size,
                       int32_t dcp_size, int32_t interleave, int32_t* local_lens,
                       void* stream);

/*
 * dcp_check_block_table - count the block-table entries in use that break the
 * device-data contract. A checking aid: the attention, write and gather calls
 * do not check block ids, and an id outside the pool makes them read or write
 * outside it.
 *
 * Source: "Decode Context Parallel (DCP)", section "KV-cache layout" (a
 * virtual block spans block_size * dcp_size positions; one table row per
 * request holds a physical block id per virtual block, shared by the ranks).
 *
 * Request b with length L = max(seq_lens[b], 0) uses virtual blocks vb = 0 ..
 * ceil(L / (block_size * dcp_size)) - 1. *bad_count receives the number of
 * those (b, vb) with vb >= max_vblocks (entries the table lacks) or with
 * block_table[b * block_table_stride + vb] outside [0, num_blocks), saturated
 * at INT32_MAX. 0 means the table is valid for these lengths.
 *
 * block_table        device, int32, row b at block_table + b * block_table_stride
 * num_reqs           rows, >= 0
 * block_table_stride >= max_vblocks
 * max_vblocks        >= 0, valid columns per row
 * seq_lens           device, [num_reqs] int32
 * block_size, dcp_size >= 1; num_blocks >= 0 (physical blocks per rank pool)
 * bad_count          device, one int32, overwritten (also when num_reqs == 0)
 * Two kernels (clear, count); nothing is allocated.
 * Errors: DCP_ERR_INVALID_ARG for a bad size or relation or a NULL pointer
 * (block_table may be NULL when num_reqs or max_vblocks is 0; seq_lens when
 * num_reqs is 0); DCP_ERR_HIP if a launch fails.
 */
int dcp_check_block_table(const int32_t* block_table, int32_t num_reqs, int64_t block_table_stride,
                          int32_t max_vblocks, const int32_t* seq_lens, int32_t block_size,
                          int32_t dcp_size, int32_t num_blocks, int32_t* bad_count, void* stream);

/*
 * dcp_slot_mapping - where each new token's KV goes on each rank.
 *
 * Source: "Decode Context Parallel (DCP)", section "KV-cache layout" (a
 * virtual block spans block_size * dcp_size tokens; the four formulas give the
 * owner of token x; block_size % interleave == 0); "DeepSeek V4.1 context
 * parallelism", section "Cache ownership" (writes translate virtual slots to
 * local slots and mask non-owners).
 *
 * For token t with position x = positions[t] in request b = req_indices[t]:
 *   vb    = x / (block_size * dcp_size)            (virtual block index)
 *   owner = ((x % (block_size * dcp_size)) / interleave) % dcp_size
 *   off   = offset of x among the tokens of virtual block vb that the owner
 *           holds, in ascending position order
 *         = ((x / (interleave * dcp_size)) * interleave + x % interleave) % block_size
 *   slots[owner * num_tokens + t] = block_table[b * block_table_stride + vb] * block_size + off
 *   slots[r * num_tokens + t]     = -1 for every other rank r.
 * All ranks get -1 when x < 0, b is outside [0, num_reqs), vb >= max_vblocks or
 * the block id is negative. The block table is shared by all ranks: each rank
 * has its own pool and physical block id p means block p of that rank's pool.
 *
 * positions          device, [num_tokens] int64
 * req_indices        device, [num_tokens] int32
 * num_tokens         >= 0 (0: nothing is launched)
 * block_table        device, int32, row b at block_table + b * block_table_stride
 * num_reqs           rows in block_table, >= 0
 * block_table_stride >= max_vblocks
 * max_vblocks        >= 0, valid columns per row
 * slots              device, [dcp_size, num_tokens] int64
 * Errors: DCP_ERR_INVALID_ARG, DCP_ERR_HIP.
 */
int dcp_slot_mapping(const int64_t* positions, const int32_t* req_indices, int64_t num_tokens,
                     const int32_t* block_table, int32_t num_reqs, int64_t block_table_stride,
                     int32_t max_vblocks, int32_t block_size, int32_t dcp_size,
                     int32_t interleave, int64_t* slots, void* stream);

/*
 * Paged KV pools of the ranks being computed, all with the same geometry.
 * Element (rank r, block p, kv head h, token t, dim d) of K lives at
 *   k + r*k_stride[0] + p*k_stride[1] + h*k_stride[2] + t*k_stride[3] + d*k_stride[4]
 * with r counted from rank_begin; likewise V with v_stride. v == NULL means V
 * is the first head_dim_v entries of the K row (MLA: one latent vector is both
 * key and value) and v_stride is ignored. k_scale / v_scale are device
 * [num_kv_heads] float32 and required exactly when dtype is DCP_FP8_E4M3.
 *
 * The MFMA kernels read these layouts (others use the generic kernel):
 *   GQA  bf16 / fp8, head_dim_k = head_dim_v = 128, Hq/Hkv <= 16:
 *        K dim stride 1 and V token stride 1 ("V transposed inside a block",
 *        [block, head, dim, token]); block_size a multiple of 16; 16-byte
 *        aligned rows.
 *   MLA  bf16, num_kv_heads = 1, Hq = 128, head_dim_k = 576, head_dim_v = 512,
 *        v == NULL, K dim stride 1, 16-byte aligned rows.
 */
typedef struct dcp_kv_cache {
  int32_t dtype;              /* DCP_F32 | DCP_BF16 | DCP_FP8_E4M3 */
  int32_t num_blocks;         /* physical blocks in each rank's pool */
  int32_t block_size;         /* tokens per physical block */
  int32_t num_kv_heads;
  int32_t head_dim_k;
  int32_t head_dim_v;
  void* k;                    /* device; written only by dcp_kv_cache_write */
  int64_t k_stride[5];        /* rank, block, head, token, dim (elements) */
  void* v;                    /* NULL: V aliases K[..., 0:head_dim_v] */
  int64_t v_stride[5];
  const float* k_scale;       /* [num_kv_heads], fp8 only, else NULL */
  const float* v_scale;       /* [num_kv_heads], fp8 only, else NULL */
} dcp_kv_cache_t;

/*
 * dcp_partial_decode_attn_workspace_size - bytes of device workspace that
 * dcp_partial_decode_attn needs for these arguments (0 is possible). Host
 * only: it reads no device memory, but the MFMA kernels size their split
 * pieces by the number of persistent workers the current device runs (its
 * compute-unit count), so the size holds for calls on the current device (and
 * devices of the same model). Returns 0 and sets *status (if non-NULL) to an
 * error code when the arguments are invalid.
 */
size_t dcp_partial_decode_attn_workspace_size(int32_t batch, int32_t num_q_heads,
                                              int32_t q_dtype, const dcp_kv_cache_t* kv,
                                              int32_t rank_count, int32_t algo, int* status);

/*
 * dcp_partial_decode_attn - each rank's partial decode attention over its
 * local KV shard (GQA, and MLA with v == NULL).
 *
 * Source: "Decode Context Parallel (DCP)", section "Decode" (attention of the
 * gathered query heads against the local KV-cache shard, producing partial
 * outputs and LSE values); "Efficient Decode Context Parallelism with vLLM for
 * Long Context Workloads", sections 1 and 5.4 (MLA's single latent KV head;
 * GQA query heads sharing their group's KV head).
 *
 * For rank r in [0, rank_count) (global rank rank_begin + r), request b and
 * query head h, with n = local_lens[b * dcp_size + rank_begin + r] and KV head
 * g = h / (num_q_heads / num_kv_heads), over the rank-local tokens j < n
 * (token j sits in block block_table[b * block_table_stride + j / block_size],
 * slot j % block_size of rank r's pool):
 *   s_j   = softmax_scale * <q[b,h,:], k_j[g,:]>
 *   LSE   = ln sum_j exp(s_j)                       (-inf when n == 0)
 *   O     = sum_j exp(s_j - LSE) * v_j[g,:]         (0 when n == 0)
 * fp8 K and V are dequantised as code * k_scale[g] / v_scale[g]. Accumulation
 * is fp32; the MFMA kernels round the softmax weights to bf16 before the
 * value product and use the same rounded weights in the denominator.
 *
 * q           device, [batch, num_q_heads, head_dim_k], contiguous, q_dtype
 *             DCP_F32 or DCP_BF16
 * local_lens  device, [batch, dcp_size] int32 (as from dcp_local_seq_lens);
 *             every length must be <= max_vblocks * block_size
 * rank_begin, rank_count: 0 <= rank_begin, 1 <= rank_count,
 *             rank_begin + rank_count <= dcp_size
 * out_o       device, [rank_count, batch, num_q_heads, head_dim_v] float32
 * out_lse     device, [rank_count, batch, num_q_heads] float32 (natural log)
 * workspace   device, >= the size query's bytes (may be NULL if that is 0)
 * Errors: DCP_ERR_INVALID_ARG (sizes, relations, NULL pointers,
 * num_q_heads % num_kv_heads != 0, head_dim_v > head_dim_k with v == NULL,
 * fp8 without scales), DCP_ERR_UNSUPPORTED (also when rank_count * batch *
 * num_kv_heads split units, or rank_count * batch * num_q_heads rows for the
 * generic kernel, exceed 2^31 - 1), DCP_ERR_WORKSPACE, DCP_ERR_HIP.
 */
int dcp_partial_decode_attn(const void* q, int32_t q_dtype, int32_t batch, int32_t num_q_heads,
                            const dcp_kv_cache_t* kv, const int32_t* block_table,
                            int64_t block_table_stride, int32_t max_vblocks,
                            const int32_t* local_lens, int32_t dcp_size, int32_t rank_begin,
                            int32_t rank_count, float softmax_scale, int32_t algo,
                            float* out_o, float* out_lse, void* workspace,
                            size_t workspace_bytes, void* stream);

/* Bytes of device scratch that dcp_partial_decode_attn_noalloc holds per
 * device: enough for the 128-head, 512-dim MLA decode on a 256-CU device
 * (its stream-K partials take about 129 MiB) and for the GQA kernels' far
 * smaller plans. */
#define DCP_NOALLOC_SCRATCH_BYTES ((size_t)136 << 20)

/*
 * dcp_partial_decode_attn_noalloc - dcp_partial_decode_attn for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): the same operation, arguments,
 * kernels and results, with no workspace argument.
 *
 * The workspace is a static device array of DCP_NOALLOC_SCRATCH_BYTES that
 * the library holds on every device it runs this call on, from the first
 * such call there until the process ends (with HIP's default deferred code
 * loading; with eager loading, on every device from the library's load). The call allocates no device or
 * pinned memory; it fails with DCP_ERR_SCRATCH when
 * dcp_partial_decode_attn_workspace_size for the same arguments exceeds
 * DCP_NOALLOC_SCRATCH_BYTES (nothing is launched then). The kernels write
 * every scratch word they read within a call, so nothing carries over from
 * the previous call. All calls on one device share that device's array:
 * calls that may overlap there (on different streams, or from several host
 * threads without ordering) race and must be serialised by the caller.
 * Errors: those of dcp_partial_decode_attn except DCP_ERR_WORKSPACE, plus
 * DCP_ERR_SCRATCH; DCP_ERR_HIP also when the scratch address cannot be
 * obtained on the current device.
 */
int dcp_partial_decode_attn_noalloc(const void* q, int32_t q_dtype, int32_t batch,
                                    int32_t num_q_heads, const dcp_kv_cache_t* kv,
                                    const int32_t* block_table, int64_t block_table_stride,
                                    int32_t max_vblocks, const int32_t* local_lens,
                                    int32_t dcp_size, int32_t rank_begin, int32_t rank_count,
                                    float softmax_scale, int32_t algo, float* out_o,
                                    float* out_lse, void* stream);

/*
 * dcp_partial_verify_attn - each rank's partial attention for several new
 * tokens of every request at once (multi-token decode: MTP, speculative
 * verification), causal among them.
 *
 * Source: "DeepSeek V4.1 context parallelism", section "Decode computation"
 * (decode and speculative verification share the decode path: each rank
 * attends the pages it owns); "Efficient Decode Context Parallelism with vLLM
 * for Long Context Workloads", section 6 (MTP and speculative decoding on the
 * DCP decode path); "Decode Context Parallel (DCP)", section "Decode".
 *
 * The last q_len tokens of request b (already written to the cache, e.g. by
 * dcp_kv_cache_write) are queried together: query token i sits at position
 * L_b - q_len + i and attends every cached position up to its own. Its
 * rank-local tokens are the first n(b, i, r) local tokens of rank r's shard
 * (local order is ascending position), n = local_lens[(b * q_len + i) *
 * dcp_size + rank_begin + r], which is what dcp_local_seq_lens returns for
 * the sequence length L_b - q_len + i + 1. With those lengths, for rank r,
 * query token i, query head h (KV head g = h / (num_q_heads / num_kv_heads)):
 *   s_j   = softmax_scale * <q[b,i,h,:], k_j[g,:]>, j < n(b, i, r)
 *   LSE   = ln sum_j exp(s_j)                       (-inf when n == 0)
 *   O     = sum_j exp(s_j - LSE) * v_j[g,:]         (0 when n == 0)
 * (each row is the dcp_partial_decode_attn result for that query token and
 * length; q_len = 1 is dcp_partial_decode_attn). Merging the rank partials
 * with dcp_lse_merge (batch = batch * q_len) gives causal attention.
 *
 * q           device, [batch, q_len, num_q_heads, head_dim_k], contiguous
 * q_len       1..64 query tokens per request
 * local_lens  device, [batch, q_len, dcp_size] int32, each <= max_vblocks *
 *             block_size
 * out_o       device, [rank_count, batch, q_len, num_q_heads, head_dim_v] f32
 * out_lse     device, [rank_count, batch, q_len, num_q_heads] f32
 * other arguments and errors as for dcp_partial_decode_attn. The GQA MFMA
 * kernel reads the KV once for up to 16 / (num_q_heads / num_kv_heads)
 * query tokens of a request; the MLA MFMA kernel takes each query token
 * separately.
 */
size_t dcp_partial_verify_attn_workspace_size(int32_t batch, int32_t q_len, int32_t num_q_heads,
                                              int32_t q_dtype, const dcp_kv_cache_t* kv,
                                              int32_t rank_count, int32_t algo, int* status);

int dcp_partial_verify_attn(const void* q, int32_t q_dtype, int32_t batch, int32_t q_len,
                            int32_t num_q_heads, const dcp_kv_cache_t* kv,
                            const int32_t* block_table, int64_t block_table_stride,
                            int32_t max_vblocks, const int32_t* local_lens, int32_t dcp_size,
                            int32_t rank_begin, int32_t rank_count, float softmax_scale,
                            int32_t algo, float* out_o, float* out_lse, void* workspace,
                            size_t workspace_bytes, void* stream);

/*
 * dcp_partial_segment_attn - add a replicated segment to the one rank that
 * counts it.
 *
 * Source: "DeepSeek V4.1 context parallelism", sections "Cache ownership"
 * (the sliding-window (SWA) cache stays replicated on every rank) and
 * "Decode computation" (replicated SWA contributes on one rank; the sink is
 * applied once in the log-sum-exp merge).
 *
 * A segment is a set of KV entries per request kept whole on every rank
 * (e.g. the SWA window), separate from the sharded cache; every query head of
 * the request attends it in addition to the sharded tokens. This call
 * computes each request's attention over its segment (seg_lens[b] tokens of
 * the paged pool seg_kv, read through seg_block_table as a one-rank cache:
 * token j in block seg_block_table[b * stride + j / block_size], slot
 * j % block_size of pool 0) and folds it in place into the partial of rank
 * seg_rank:
 *   LSE' = ln(exp(LSE_r) + exp(LSE_seg)),
 *   O'   = exp(LSE_r - LSE') O_r + exp(LSE_seg - LSE') O_seg
 * (an empty side contributes nothing; both empty leaves O = 0, LSE = -inf).
 * Every other rank's partial is left as it is, so dcp_lse_merge afterwards
 * counts the segment exactly once (and the sink once). Call it after
 * dcp_partial_decode_attn and before dcp_lse_merge.
 *
 * q, q_dtype, batch, num_q_heads, softmax_scale, algo: as for
 *             dcp_partial_decode_attn (one query token per request)
 * seg_kv      the segment pool (rank index 0; num_kv_heads and head dims as
 *             the sharded cache; MLA: v == NULL)
 * seg_lens    device, [batch] int32, each <= seg_max_vblocks * block_size
 * seg_rank    the rank that counts the segment, >= 0; when it lies outside
 *             [rank_begin, rank_begin + rank_count) nothing is launched (the
 *             GPU holding that rank adds it)
 * part_o, part_lse  device, the partials dcp_partial_decode_attn wrote for
 *             ranks rank_begin .. rank_begin + rank_count - 1; updated in place
 * workspace   device, >= dcp_partial_segment_attn_workspace_size bytes
 * Errors: as for dcp_partial_decode_attn.
 */
size_t dcp_partial_segment_attn_workspace_size(int32_t batch, int32_t num_q_heads, int32_t q_dtype,
                                               const dcp_kv_cache_t* seg_kv, int32_t algo,
                                               int* status);

int dcp_partial_segment_attn(const void* q, int32_t q_dtype, int32_t batch, int32_t num_q_heads,
                             const dcp_kv_cache_t* seg_kv, const int32_t* seg_block_table,
                             int64_t seg_block_table_stride, int32_t seg_max_vblocks,
                             const int32_t* seg_lens, float softmax_scale, int32_t algo,
                             int32_t seg_rank, int32_t rank_begin, int32_t rank_count,
                             float* part_o, float* part_lse, void* workspace,
                             size_t workspace_bytes, void* stream);

/*
 * dcp_lse_merge - combine per-rank partials into exact attention, applying an
 * attention sink once.
 *
 * Source: "Decode Context Parallel (DCP)", section "Decode" (partial outputs
 * and LSE values are combined across the DCP group); "DeepSeek V4.1 context
 * parallelism", section "Decode computation" (the attention sink is applied
 * once when the partial outputs are merged by log-sum-exp).
 *
 * For each (b, h), over parts r with LSE_r = part_lse[(r*batch + b)*num_heads + h]:
 *   M   = max(max_r LSE_r, sink[h])          (sink term only if sink != NULL)
 *   Z   = sum_r exp(LSE_r - M) + exp(sink[h] - M)
 *   LSE = M + ln Z
 *   O   = sum_r exp(LSE_r - LSE) * part_o[r, b, h, :]
 * Parts with LSE_r = -inf contribute nothing; when every term is -inf, O = 0
 * and LSE = -inf. The sink is a logit in the units of the scaled scores with
 * a zero value vector; the returned LSE includes it.
 *
 * part_o    device, [num_parts, batch, num_heads, head_dim_v] float32
 * part_lse  device, [num_parts, batch, num_heads] float32
 * num_parts 1..64; batch >= 0; num_heads >= 1; head_dim_v 1..4096
 * sink      device, [num_heads] float32, or NULL
 * out_dtype DCP_F32 or DCP_BF16 (round to nearest even)
 * out_o     device, [batch, num_heads, head_dim_v]
 * out_lse   device, [batch, num_heads] float32, or NULL
 * Errors: DCP_ERR_INVALID_ARG, DCP_ERR_UNSUPPORTED, DCP_ERR_HIP.
 */
int dcp_lse_merge(const float* part_o, const float* part_lse, int32_t num_parts, int32_t batch,
                  int32_t num_heads, int32_t head_dim_v, const float* sink, int32_t out_dtype,
                  void* out_o, float* out_lse, void* stream);

/*
 * dcp_kv_cache_write - store new tokens' K and V rows into the pools of the
 * ranks that own them.
 *
 * Source: "Decode Context Parallel (DCP)", section "KV-cache layout" (each
 * rank stores only the tokens of its shard, at the slot given by the slot
 * mapping); "DeepSeek V4.1 context parallelism", section "Cache ownership"
 * (a cache write turns the virtual slot into the owner's local slot; ranks
 * that do not own the token write nothing).
 *
 * For token t and rank r in [0, num_ranks), with s = slots[r * num_tokens + t]:
 * if 0 <= s < num_blocks * block_size, then for every kv head h and dim d
 *   K[r, s / block_size, h, s % block_size, d] = store(k_new[t, h, d], k_scale[h])
 *   V[r, s / block_size, h, s % block_size, d] = store(v_new[t, h, d], v_scale[h])
 * (addresses as in dcp_kv_cache_t); any other s (-1 for a rank that does not
 * own the token) writes nothing on rank r. store() by kv->dtype:
 *   DCP_F32       the fp32 value of the input;
 *   DCP_BF16      the input rounded to the nearest bf16, ties to even
 *                 (NaN stays a quiet NaN);
 *   DCP_FP8_E4M3  the E4M3 code nearest to the fp32 quotient x / scale[h]
 *                 (IEEE division), ties to the even code; magnitudes beyond
 *                 448 (infinities included) saturate to +-448; NaN gives
 *                 0x7F; zero keeps its sign.
 * A token that two ranks own is written on both. Two tokens with the same
 * valid slot on one rank race: which row lands is unspecified.
 *
 * k_new      device, [num_tokens, num_kv_heads, head_dim_k], contiguous,
 *            src_dtype (DCP_F32 or DCP_BF16), 16-byte aligned
 * v_new      device, [num_tokens, num_kv_heads, head_dim_v], like k_new;
 *            must be NULL exactly when kv->v is NULL (MLA: the value is the
 *            first head_dim_v entries of the K row, written with it)
 * num_tokens >= 0 (0: nothing is launched)
 * slots      device, [num_ranks, num_tokens] int64 (as from dcp_slot_mapping)
 * num_ranks  1..64: pools kv describes, counted from the pool kv->k points to
 * kv         the pools to write (the descriptor is not modified; the pools
 *            its k and v point to are); head_dim_k and head_dim_v multiples
 *            of 8; fp8 needs k_scale (and v_scale when v != NULL)
 * Errors: DCP_ERR_INVALID_ARG (sizes, NULL pointers, v_new / kv->v mismatch,
 * fp8 without scales), DCP_ERR_UNSUPPORTED (src_dtype, head dims not
 * multiples of 8 or head_dim_k + head_dim_v over 8192, num_ranks > 64,
 * num_kv_heads > 65535, unaligned sources), DCP_ERR_HIP.
 */
int dcp_kv_cache_write(const void* k_new, const void* v_new, int32_t src_dtype, int64_t num_tokens,
                       const int64_t* slots, int32_t num_ranks, const dcp_kv_cache_t* kv, void* stream);

/*
 * dcp_gather_context - (chunked) prefill: gather each request's cached
 * context from the ranks' shards back into request-contiguous order.
 *
 * Source: "Decode Context Parallel (DCP)", section "Prefill and chunked
 * prefill" (MLA gathers the context KV cache and restores request-contiguous
 * order before the current query chunk attends it); "DeepSeek V4.1 context
 * parallelism", section "Cache ownership" (pages are copied as stored,
 * without dequantising).
 *
 * Request b's context is its positions 0 .. cu_ctx[b+1] - cu_ctx[b] - 1.
 * Output row t = cu_ctx[b] + x holds the stored K row (and V row) of
 * position x of request b, copied bit for bit from the pool of its owner
 * ((x / interleave) % dcp_size) at the slot dcp_slot_mapping gives (block
 * block_table[b][x / (block_size * dcp_size)], shared by all ranks). A
 * position whose virtual block is >= max_vblocks or has a negative block id
 * gives a zero row.
 *
 * kv          the dcp_size pools, counted from the pool kv->k points to;
 *             rows must be contiguous (dim stride 1) and 16-byte aligned
 *             (head_dim * element size a multiple of 16)
 * block_table device, int32, row b at block_table + b * block_table_stride
 * cu_ctx      device, [num_reqs + 1] int64, cu_ctx[0] = 0, non-decreasing
 * total_tokens = cu_ctx[num_reqs] (the host knows it from the batch plan)
 * out_k       device, [total_tokens, num_kv_heads, head_dim_k], kv->dtype
 * out_v       device, [total_tokens, num_kv_heads, head_dim_v], or NULL (K
 *             only; must be NULL when kv->v is NULL: MLA gathers the latent
 *             row, which holds the value)
 * Errors: DCP_ERR_INVALID_ARG (sizes, relations, NULL pointers, out_v with
 * kv->v == NULL), DCP_ERR_UNSUPPORTED (dtype, a row layout that is not
 * contiguous and 16-byte aligned, more than 4095 16-byte chunks per token),
 * DCP_ERR_HIP.
 */
int dcp_gather_context(const dcp_kv_cache_t* kv, int32_t dcp_size, int32_t interleave,
                       const int32_t* block_table, int32_t num_reqs, int64_t block_table_stride,
                       int32_t max_vblocks, const int64_t* cu_ctx, int64_t total_tokens,
                       void* out_k, void* out_v, void* stream);

/*
 * Measurement hook for benchmarks.
 *
 * dcp_profile_enable(1) makes every following dcp_partial_decode_attn and
 * dcp_partial_verify_attn call made by this host thread record a pair of HIP
 * events on its stream, right
 * before and right after its main attention kernel (the MLA planner and the
 * split combine are outside the pair). dcp_profile_collect waits for the recorded
 * events, returns the summed elapsed milliseconds and the number of calls
 * since the last collect (or enable), and starts a new count.
 * dcp_profile_enable(0) stops recording. The events are created by the
 * library on first use and reused; nothing else changes in the calls.
 * Errors: DCP_ERR_INVALID_ARG (NULL output), DCP_ERR_HIP.
 */
int dcp_profile_enable(int on);
int dcp_profile_collect(double* total_ms, int32_t* launches);

/*
 * Measurement hook: the device's sustained streaming-read rate, the measured
 * ceiling that the decode kernels' HBM fractions are reported against next to
 * the 8 TB/s specification (time a call with events on `stream`; rate =
 * bytes / time).
 *
 * dcp_hbm_read_probe reads each of the `bytes` bytes of `buf` exactly once
 * (16-byte non-temporal loads, each wavefront one contiguous run, a fixed grid
 * of dcp_hbm_read_probe_blocks() workgroups) and writes digest[g] = the XOR of
 * the 32-bit words that workgroup g read; the XOR of all digests is the XOR
 * of every 32-bit word of the buffer.
 *   buf     device, 16-byte aligned; bytes >= 0 and a multiple of 16
 *   digest  device, uint32[digest_len], digest_len >= dcp_hbm_read_probe_blocks()
 * dcp_hbm_read_probe_blocks() returns the workgroup count for the current
 * device (4 per CU), or a negative status.
 * Errors: DCP_ERR_INVALID_ARG (NULL or misaligned buffer, bad sizes),
 * DCP_ERR_HIP. bytes == 0 launches nothing.
 */
int dcp_hbm_read_probe_blocks(void);
int dcp_hbm_read_probe(const void* buf, int64_t bytes, uint32_t* digest, int32_t digest_len, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* DCP_H */
