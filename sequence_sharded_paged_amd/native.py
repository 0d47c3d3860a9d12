"""ctypes binding of libdcp (include/dcp.h), one Python function per C entry point.

Argument marshalling only: tensors become device pointers, torch's current
stream becomes the stream argument, and a negative status raises
``DcpError``. Every computation runs in the HIP kernels of libdcp; when the
library is missing this module raises instead of falling back to anything.
"""

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("DCP_LIB", os.path.join(_HERE, "lib", "libdcp.so"))

DCP_OK, DCP_ERR_INVALID_ARG, DCP_ERR_UNSUPPORTED, DCP_ERR_WORKSPACE, DCP_ERR_HIP, DCP_ERR_SCRATCH = 0, -1, -2, -3, -4, -5
DCP_NOALLOC_SCRATCH_BYTES = 136 << 20
DCP_F32, DCP_BF16, DCP_FP8_E4M3 = 0, 1, 2
DCP_ALGO_AUTO, DCP_ALGO_GENERIC, DCP_ALGO_FAST = 0, 1, 2

TORCH_TO_DCP = {torch.float32: DCP_F32, torch.bfloat16: DCP_BF16, torch.float8_e4m3fn: DCP_FP8_E4M3}

EXPORTS = [
    "dcp_abi_version", "dcp_status_string", "dcp_local_seq_lens", "dcp_slot_mapping",
    "dcp_partial_decode_attn_workspace_size", "dcp_partial_decode_attn", "dcp_lse_merge",
    "dcp_kv_cache_write", "dcp_partial_verify_attn_workspace_size", "dcp_partial_verify_attn",
    "dcp_partial_segment_attn_workspace_size", "dcp_partial_segment_attn", "dcp_gather_context",
    "dcp_profile_enable", "dcp_profile_collect", "dcp_check_block_table", "dcp_partial_decode_attn_noalloc",
    "dcp_hbm_read_probe_blocks", "dcp_hbm_read_probe",
]


class DcpError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        super().__init__(f"{fn} failed: {status_string(status)} ({status})")


class KvCache(ctypes.Structure):
    """Mirror of ``dcp_kv_cache_t``."""
    _fields_ = [
        ("dtype", ctypes.c_int32), ("num_blocks", ctypes.c_int32), ("block_size", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32), ("head_dim_k", ctypes.c_int32), ("head_dim_v", ctypes.c_int32),
        ("k", ctypes.c_void_p), ("k_stride", ctypes.c_int64 * 5),
        ("v", ctypes.c_void_p), ("v_stride", ctypes.c_int64 * 5),
        ("k_scale", ctypes.c_void_p), ("v_scale", ctypes.c_void_p),
    ]


_lib = None


def lib():
    """Load libdcp once; raise if it is not built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"libdcp not built ({LIB_PATH} missing): run "
                               "`python -m sequence_sharded_paged_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        i32, i64, vp, f32 = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p, ctypes.c_float
        L.dcp_abi_version.restype = ctypes.c_int
        L.dcp_abi_version.argtypes = []
        L.dcp_status_string.restype = ctypes.c_char_p
        L.dcp_status_string.argtypes = [ctypes.c_int]
        L.dcp_local_seq_lens.restype = ctypes.c_int
        L.dcp_local_seq_lens.argtypes = [vp, i32, i32, i32, i32, vp, vp]
        L.dcp_slot_mapping.restype = ctypes.c_int
        L.dcp_slot_mapping.argtypes = [vp, vp, i64, vp, i32, i64, i32, i32, i32, i32, vp, vp]
        L.dcp_partial_decode_attn_workspace_size.restype = ctypes.c_size_t
        L.dcp_partial_decode_attn_workspace_size.argtypes = [i32, i32, i32, ctypes.POINTER(KvCache), i32, i32,
                                                             ctypes.POINTER(ctypes.c_int)]
        L.dcp_partial_decode_attn.restype = ctypes.c_int
        L.dcp_partial_decode_attn.argtypes = [vp, i32, i32, i32, ctypes.POINTER(KvCache), vp, i64, i32, vp, i32,
                                              i32, i32, f32, i32, vp, vp, vp, ctypes.c_size_t, vp]
        L.dcp_partial_decode_attn_noalloc.restype = ctypes.c_int
        L.dcp_partial_decode_attn_noalloc.argtypes = [vp, i32, i32, i32, ctypes.POINTER(KvCache), vp, i64, i32, vp,
                                                      i32, i32, i32, f32, i32, vp, vp, vp]
        L.dcp_lse_merge.restype = ctypes.c_int
        L.dcp_lse_merge.argtypes = [vp, vp, i32, i32, i32, i32, vp, i32, vp, vp, vp]
        L.dcp_partial_verify_attn_workspace_size.restype = ctypes.c_size_t
        L.dcp_partial_verify_attn_workspace_size.argtypes = [i32, i32, i32, i32, ctypes.POINTER(KvCache), i32, i32,
                                                             ctypes.POINTER(ctypes.c_int)]
        L.dcp_partial_verify_attn.restype = ctypes.c_int
        L.dcp_partial_verify_attn.argtypes = [vp, i32, i32, i32, i32, ctypes.POINTER(KvCache), vp, i64, i32, vp, i32,
                                              i32, i32, f32, i32, vp, vp, vp, ctypes.c_size_t, vp]
        L.dcp_partial_segment_attn_workspace_size.restype = ctypes.c_size_t
        L.dcp_partial_segment_attn_workspace_size.argtypes = [i32, i32, i32, ctypes.POINTER(KvCache), i32,
                                                              ctypes.POINTER(ctypes.c_int)]
        L.dcp_partial_segment_attn.restype = ctypes.c_int
        L.dcp_partial_segment_attn.argtypes = [vp, i32, i32, i32, ctypes.POINTER(KvCache), vp, i64, i32, vp, f32, i32,
                                               i32, i32, i32, vp, vp, vp, ctypes.c_size_t, vp]
        L.dcp_gather_context.restype = ctypes.c_int
        L.dcp_gather_context.argtypes = [ctypes.POINTER(KvCache), i32, i32, vp, i32, i64, i32, vp, i64, vp, vp, vp]
        L.dcp_kv_cache_write.restype = ctypes.c_int
        L.dcp_kv_cache_write.argtypes = [vp, vp, i32, i64, vp, i32, ctypes.POINTER(KvCache), vp]
        L.dcp_check_block_table.restype = ctypes.c_int
        L.dcp_check_block_table.argtypes = [vp, i32, i64, i32, vp, i32, i32, i32, vp, vp]
        L.dcp_profile_enable.restype = ctypes.c_int
        L.dcp_profile_enable.argtypes = [ctypes.c_int]
        L.dcp_profile_collect.restype = ctypes.c_int
        L.dcp_profile_collect.argtypes = [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int32)]
        L.dcp_hbm_read_probe_blocks.restype = ctypes.c_int
        L.dcp_hbm_read_probe_blocks.argtypes = []
        L.dcp_hbm_read_probe.restype = ctypes.c_int
        L.dcp_hbm_read_probe.argtypes = [vp, i64, vp, i32, vp]
        _lib = L
    return _lib


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check(fn, st):
    if st != DCP_OK:
        raise DcpError(fn, st)


def dcp_abi_version() -> int:
    return lib().dcp_abi_version()


def status_string(status: int) -> str:
    return lib().dcp_status_string(int(status)).decode()


dcp_status_string = status_string


def dcp_local_seq_lens(seq_lens, block_size, dcp_size, interleave, out=None, stream=None):
    """``seq_lens [B] int32`` (device) -> ``local_lens [B, dcp_size] int32``."""
    B = seq_lens.shape[0]
    assert seq_lens.dtype == torch.int32 and seq_lens.is_contiguous()
    if out is None:
        out = torch.empty((B, dcp_size), dtype=torch.int32, device=seq_lens.device)
    _check("dcp_local_seq_lens", lib().dcp_local_seq_lens(
        _ptr(seq_lens), B, block_size, dcp_size, interleave, _ptr(out), _stream(stream)))
    return out


def dcp_check_block_table(block_table, seq_lens, block_size, dcp_size, num_blocks, max_vblocks=None, out=None,
                          stream=None):
    """Count the in-use entries of ``block_table [B, >= max_vblocks] int32``
    (device) that are missing or outside ``[0, num_blocks)`` for the lengths
    ``seq_lens [B] int32``; returns a device ``int32 [1]`` tensor (0: valid)."""
    B = seq_lens.shape[0]
    assert seq_lens.dtype == torch.int32 and seq_lens.is_contiguous()
    assert block_table.dtype == torch.int32 and block_table.dim() == 2 and block_table.stride(1) == 1
    if max_vblocks is None:
        max_vblocks = block_table.shape[1]
    if out is None:
        out = torch.empty(1, dtype=torch.int32, device=seq_lens.device)
    _check("dcp_check_block_table", lib().dcp_check_block_table(
        _ptr(block_table), B, block_table.stride(0), max_vblocks, _ptr(seq_lens), block_size, dcp_size, num_blocks,
        _ptr(out), _stream(stream)))
    return out


def dcp_slot_mapping(positions, req_indices, block_table, block_size, dcp_size, interleave,
                     max_vblocks=None, out=None, stream=None):
    """``positions [T] int64``, ``req_indices [T] int32``, ``block_table [B, W] int32``
    -> ``slots [dcp_size, T] int64`` (-1 where the rank does not own the token)."""
    T = positions.shape[0]
    assert positions.dtype == torch.int64 and req_indices.dtype == torch.int32
    assert block_table.dtype == torch.int32 and block_table.stride(1) == 1
    if max_vblocks is None:
        max_vblocks = block_table.shape[1]
    if out is None:
        out = torch.empty((dcp_size, T), dtype=torch.int64, device=positions.device)
    _check("dcp_slot_mapping", lib().dcp_slot_mapping(
        _ptr(positions), _ptr(req_indices), T, _ptr(block_table), block_table.shape[0], block_table.stride(0),
        max_vblocks, block_size, dcp_size, interleave, _ptr(out), _stream(stream)))
    return out


def dcp_partial_decode_attn_workspace_size(batch, num_q_heads, q_dtype, kv: KvCache, rank_count,
                                           algo=DCP_ALGO_AUTO) -> int:
    st = ctypes.c_int(0)
    n = lib().dcp_partial_decode_attn_workspace_size(batch, num_q_heads, q_dtype, ctypes.byref(kv), rank_count,
                                                    algo, ctypes.byref(st))
    _check("dcp_partial_decode_attn_workspace_size", st.value)
    return int(n)


def dcp_partial_decode_attn(q, kv: KvCache, block_table, local_lens, dcp_size, rank_begin, rank_count,
                            softmax_scale, out_o, out_lse, workspace, algo=DCP_ALGO_AUTO,
                            max_vblocks=None, stream=None):
    """Per-rank partial decode attention; fills ``out_o [R, B, Hq, Dv]`` and
    ``out_lse [R, B, Hq]`` (float32)."""
    B, Hq, _ = q.shape
    assert q.is_contiguous() and local_lens.dtype == torch.int32 and local_lens.is_contiguous()
    assert block_table.dtype == torch.int32 and block_table.stride(1) == 1
    assert out_o.dtype == torch.float32 and out_lse.dtype == torch.float32
    if max_vblocks is None:
        max_vblocks = block_table.shape[1]
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("dcp_partial_decode_attn", lib().dcp_partial_decode_attn(
        _ptr(q), TORCH_TO_DCP[q.dtype], B, Hq, ctypes.byref(kv), _ptr(block_table), block_table.stride(0),
        max_vblocks, _ptr(local_lens), dcp_size, rank_begin, rank_count, float(softmax_scale), algo,
        _ptr(out_o), _ptr(out_lse), _ptr(workspace), ws_bytes, _stream(stream)))


def dcp_partial_decode_attn_noalloc(q, kv: KvCache, block_table, local_lens, dcp_size, rank_begin, rank_count,
                                    softmax_scale, out_o, out_lse, algo=DCP_ALGO_AUTO, max_vblocks=None, stream=None):
    """``dcp_partial_decode_attn`` with the library's fixed device scratch as
    its workspace (no workspace argument, no device allocation)."""
    B, Hq, _ = q.shape
    assert q.is_contiguous() and local_lens.dtype == torch.int32 and local_lens.is_contiguous()
    assert block_table.dtype == torch.int32 and block_table.stride(1) == 1
    assert out_o.dtype == torch.float32 and out_lse.dtype == torch.float32
    if max_vblocks is None:
        max_vblocks = block_table.shape[1]
    _check("dcp_partial_decode_attn_noalloc", lib().dcp_partial_decode_attn_noalloc(
        _ptr(q), TORCH_TO_DCP[q.dtype], B, Hq, ctypes.byref(kv), _ptr(block_table), block_table.stride(0),
        max_vblocks, _ptr(local_lens), dcp_size, rank_begin, rank_count, float(softmax_scale), algo,
        _ptr(out_o), _ptr(out_lse), _stream(stream)))


def dcp_partial_verify_attn_workspace_size(batch, q_len, num_q_heads, q_dtype, kv: KvCache, rank_count,
                                           algo=DCP_ALGO_AUTO) -> int:
    st = ctypes.c_int(0)
    n = lib().dcp_partial_verify_attn_workspace_size(batch, q_len, num_q_heads, q_dtype, ctypes.byref(kv),
                                                    rank_count, algo, ctypes.byref(st))
    _check("dcp_partial_verify_attn_workspace_size", st.value)
    return int(n)


def dcp_partial_verify_attn(q, kv: KvCache, block_table, local_lens, dcp_size, rank_begin, rank_count,
                            softmax_scale, out_o, out_lse, workspace, algo=DCP_ALGO_AUTO, max_vblocks=None,
                            stream=None):
    """Multi-token decode: ``q [B, q_len, Hq, Dk]``, ``local_lens [B, q_len, dcp_size]`` int32;
    fills ``out_o [R, B, q_len, Hq, Dv]`` and ``out_lse [R, B, q_len, Hq]`` (float32)."""
    B, q_len, Hq, _ = q.shape
    assert q.is_contiguous() and local_lens.dtype == torch.int32 and local_lens.is_contiguous()
    assert block_table.dtype == torch.int32 and block_table.stride(1) == 1
    assert out_o.dtype == torch.float32 and out_lse.dtype == torch.float32
    if max_vblocks is None:
        max_vblocks = block_table.shape[1]
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("dcp_partial_verify_attn", lib().dcp_partial_verify_attn(
        _ptr(q), TORCH_TO_DCP[q.dtype], B, q_len, Hq, ctypes.byref(kv), _ptr(block_table), block_table.stride(0),
        max_vblocks, _ptr(local_lens), dcp_size, rank_begin, rank_count, float(softmax_scale), algo,
        _ptr(out_o), _ptr(out_lse), _ptr(workspace), ws_bytes, _stream(stream)))


def dcp_partial_segment_attn_workspace_size(batch, num_q_heads, q_dtype, seg_kv: KvCache,
                                            algo=DCP_ALGO_AUTO) -> int:
    st = ctypes.c_int(0)
    n = lib().dcp_partial_segment_attn_workspace_size(batch, num_q_heads, q_dtype, ctypes.byref(seg_kv), algo,
                                                     ctypes.byref(st))
    _check("dcp_partial_segment_attn_workspace_size", st.value)
    return int(n)


def dcp_partial_segment_attn(q, seg_kv: KvCache, seg_block_table, seg_lens, softmax_scale, seg_rank, rank_begin,
                             rank_count, part_o, part_lse, workspace, algo=DCP_ALGO_AUTO, seg_max_vblocks=None,
                             stream=None):
    """Fold each request's attention over its replicated segment into rank
    ``seg_rank``'s partial (``part_o [R, B, Hq, Dv]``, ``part_lse [R, B, Hq]``, in place)."""
    B, Hq, _ = q.shape
    assert q.is_contiguous() and seg_lens.dtype == torch.int32 and seg_lens.is_contiguous()
    assert seg_block_table.dtype == torch.int32 and seg_block_table.stride(1) == 1
    assert part_o.dtype == torch.float32 and part_lse.dtype == torch.float32
    if seg_max_vblocks is None:
        seg_max_vblocks = seg_block_table.shape[1]
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("dcp_partial_segment_attn", lib().dcp_partial_segment_attn(
        _ptr(q), TORCH_TO_DCP[q.dtype], B, Hq, ctypes.byref(seg_kv), _ptr(seg_block_table),
        seg_block_table.stride(0), seg_max_vblocks, _ptr(seg_lens), float(softmax_scale), algo, seg_rank,
        rank_begin, rank_count, _ptr(part_o), _ptr(part_lse), _ptr(workspace), ws_bytes, _stream(stream)))


def dcp_lse_merge(part_o, part_lse, sink=None, out_dtype=torch.float32, out_o=None, out_lse=None,
                  want_lse=True, stream=None):
    """Merge ``part_o [R, B, H, Dv]``, ``part_lse [R, B, H]`` -> ``(O [B, H, Dv], LSE [B, H])``."""
    R, B, H, Dv = part_o.shape
    assert part_o.dtype == torch.float32 and part_lse.dtype == torch.float32
    assert part_o.is_contiguous() and part_lse.is_contiguous()
    if out_o is None:
        out_o = torch.empty((B, H, Dv), dtype=out_dtype, device=part_o.device)
    if out_lse is None and want_lse:
        out_lse = torch.empty((B, H), dtype=torch.float32, device=part_o.device)
    if sink is not None:
        assert sink.dtype == torch.float32 and sink.numel() == H
    _check("dcp_lse_merge", lib().dcp_lse_merge(
        _ptr(part_o), _ptr(part_lse), R, B, H, Dv, _ptr(sink), TORCH_TO_DCP[out_o.dtype], _ptr(out_o),
        _ptr(out_lse), _stream(stream)))
    return out_o, out_lse


def dcp_kv_cache_write(k_new, v_new, slots, kv: KvCache, stream=None):
    """Store ``k_new [T, Hkv, Dk]`` (and ``v_new [T, Hkv, Dv]``, or None for MLA)
    at ``slots [R, T]`` (int64, -1 = not on that rank) of the pools ``kv``
    describes; R pools counted from ``kv.k``."""
    assert k_new.is_contiguous() and k_new.dtype in (torch.float32, torch.bfloat16)
    assert slots.dtype == torch.int64 and slots.is_contiguous() and slots.dim() == 2
    if v_new is not None:
        assert v_new.is_contiguous() and v_new.dtype == k_new.dtype and v_new.shape[0] == k_new.shape[0]
    R, T = slots.shape
    assert k_new.shape[0] == T
    _check("dcp_kv_cache_write", lib().dcp_kv_cache_write(
        _ptr(k_new), _ptr(v_new), TORCH_TO_DCP[k_new.dtype], T, _ptr(slots), R, ctypes.byref(kv),
        _stream(stream)))


def dcp_gather_context(kv: KvCache, dcp_size, interleave, block_table, cu_ctx, total_tokens, out_k, out_v=None,
                       max_vblocks=None, stream=None):
    """Gather every request's context (``cu_ctx [B+1]`` int64 offsets) from the
    ``dcp_size`` pools ``kv`` describes into ``out_k [T, Hkv, Dk]`` (and
    ``out_v``) in request-then-position order, stored bits copied."""
    assert cu_ctx.dtype == torch.int64 and cu_ctx.is_contiguous()
    assert block_table.dtype == torch.int32 and block_table.stride(1) == 1
    assert out_k.is_contiguous() and (out_v is None or out_v.is_contiguous())
    if max_vblocks is None:
        max_vblocks = block_table.shape[1]
    _check("dcp_gather_context", lib().dcp_gather_context(
        ctypes.byref(kv), dcp_size, interleave, _ptr(block_table), block_table.shape[0], block_table.stride(0),
        max_vblocks, _ptr(cu_ctx), int(total_tokens), _ptr(out_k), _ptr(out_v), _stream(stream)))


def dcp_hbm_read_probe_blocks() -> int:
    n = lib().dcp_hbm_read_probe_blocks()
    if n < 1:
        raise DcpError("dcp_hbm_read_probe_blocks", n)
    return n


def dcp_hbm_read_probe(buf, digest, stream=None):
    """Read every byte of the device tensor ``buf`` once; ``digest`` (uint32 /
    int32, >= dcp_hbm_read_probe_blocks() entries) receives each workgroup's XOR."""
    _check("dcp_hbm_read_probe", lib().dcp_hbm_read_probe(
        _ptr(buf), buf.numel() * buf.element_size(), _ptr(digest), digest.numel(), _stream(stream)))


def dcp_profile_enable(on: bool = True):
    _check("dcp_profile_enable", lib().dcp_profile_enable(1 if on else 0))


def dcp_profile_collect():
    """``(total_ms, launches)`` of the main attention kernel since the last collect."""
    ms, n = ctypes.c_double(0.0), ctypes.c_int32(0)
    _check("dcp_profile_collect", lib().dcp_profile_collect(ctypes.byref(ms), ctypes.byref(n)))
    return ms.value, n.value
