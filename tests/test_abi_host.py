"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and rejects invalid arguments on the host before any launch
(so these calls never touch a device)."""

import ctypes
import os
import re

import pytest

from sequence_sharded_paged_amd import native

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dcp.h")

INV, UNS, WS = native.DCP_ERR_INVALID_ARG, native.DCP_ERR_UNSUPPORTED, native.DCP_ERR_WORKSPACE
NULL = None


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dcp_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(native.LIB_PATH):
        pytest.skip("libdcp.so not built")
    return native.lib()


def test_exports_every_declared_symbol(L):
    declared = _declared()
    assert declared, "no declarations found"
    for name in declared:
        assert hasattr(L, name), f"{name} declared in dcp.h but not exported"
    assert set(declared) == set(native.EXPORTS)


def test_version_and_status_strings(L):
    assert native.dcp_abi_version() == 1
    for st in (0, -1, -2, -3, -4, -5):
        assert native.status_string(st) not in ("", "unknown status")
    assert native.status_string(-99) == "unknown status"


def _fake(n=16):
    # host buffers: validation rejects the call before any pointer is read
    return ctypes.c_void_p(ctypes.addressof((ctypes.c_char * n)()))


def test_local_seq_lens_validation(L):
    p = _fake()
    assert L.dcp_local_seq_lens(p, 4, 4, 2, 3, p, NULL) == INV      # block_size % interleave
    assert L.dcp_local_seq_lens(p, 4, 4, 0, 1, p, NULL) == INV      # dcp_size
    assert L.dcp_local_seq_lens(p, 4, 4, 2, 0, p, NULL) == INV      # interleave
    assert L.dcp_local_seq_lens(p, -1, 4, 2, 1, p, NULL) == INV     # num_reqs
    assert L.dcp_local_seq_lens(NULL, 4, 4, 2, 1, p, NULL) == INV   # null
    assert L.dcp_local_seq_lens(NULL, 0, 4, 2, 1, NULL, NULL) == 0  # empty: nothing launched


def test_slot_mapping_validation(L):
    p = _fake()
    f = L.dcp_slot_mapping
    assert f(p, p, 8, p, 2, 4, 4, 16, 4, 3, p, NULL) == INV         # 16 % 3
    assert f(p, p, 8, p, 2, 2, 4, 16, 4, 1, p, NULL) == INV         # stride < max_vblocks
    assert f(p, p, -1, p, 2, 4, 4, 16, 4, 1, p, NULL) == INV        # negative tokens
    assert f(NULL, p, 8, p, 2, 4, 4, 16, 4, 1, p, NULL) == INV      # null positions
    assert f(p, p, 8, NULL, 2, 4, 4, 16, 4, 1, p, NULL) == INV      # null table
    assert f(p, p, 0, p, 2, 4, 4, 16, 4, 1, p, NULL) == 0           # empty


def _kv(**kw):
    d = native.KvCache()
    d.dtype, d.num_blocks, d.block_size, d.num_kv_heads = native.DCP_BF16, 8, 16, 2
    d.head_dim_k, d.head_dim_v = 128, 128
    d.k = 4096
    d.v = 8192
    for i, s in enumerate((8 * 2 * 16 * 128, 2 * 16 * 128, 16 * 128, 128, 1)):
        d.k_stride[i] = s
    for i, s in enumerate((8 * 2 * 16 * 128, 2 * 16 * 128, 16 * 128, 1, 16)):
        d.v_stride[i] = s
    for k, v in kw.items():
        setattr(d, k, v)
    return d


def _ws(L, kv, batch=4, hq=8, qd=native.DCP_BF16, rc=2, algo=0):
    st = ctypes.c_int(123)
    n = L.dcp_partial_decode_attn_workspace_size(batch, hq, qd, ctypes.byref(kv), rc, algo, ctypes.byref(st))
    return st.value, n


def test_workspace_size_is_host_only(L):
    st, n = _ws(L, _kv())
    assert st == 0 and n > 0                      # MFMA path needs a plan + partials
    st, n = _ws(L, _kv(), algo=native.DCP_ALGO_GENERIC)
    assert st == 0 and n == 0
    st, n = _ws(L, _kv(), hq=7)
    assert st == INV and n == 0                   # Hq % Hkv
    st, _ = _ws(L, _kv(dtype=native.DCP_FP8_E4M3))
    assert st == INV                              # fp8 without scales
    st, _ = _ws(L, _kv(dtype=7))
    assert st == UNS
    st, _ = _ws(L, _kv(v=None, head_dim_v=256))
    assert st == INV                              # aliased V longer than K
    st, _ = _ws(L, _kv(head_dim_k=2048))
    assert st == UNS
    st, _ = _ws(L, _kv(), algo=9)
    assert st == INV
    st, _ = _ws(L, _kv(head_dim_k=64, head_dim_v=64), algo=native.DCP_ALGO_FAST)
    assert st == UNS                              # no MFMA kernel for d=64
    # more split units (rank x request x KV head) than 32-bit indices hold: no
    # MFMA kernel, and the generic kernel's workgroups (rank x request x query
    # head, never fewer) do not fit either
    st, n = _ws(L, _kv(), batch=1 << 27, rc=16, hq=2, algo=native.DCP_ALGO_FAST)
    assert st == UNS
    st, n = _ws(L, _kv(), batch=1 << 27, rc=16, hq=2)
    assert st == UNS and n == 0
    st, n = _ws(L, _kv(), batch=1 << 25, rc=16, hq=2)  # 2^30 units: the MFMA plan
    assert st == 0 and n > 0


def test_partial_attn_validation(L):
    p = _fake(64)
    kv = _kv()
    f = L.dcp_partial_decode_attn

    def call(batch=4, hq=8, bt_stride=4, max_vb=4, dcp=4, rb=0, rc=2, scale=0.1, ws=p, ws_bytes=1 << 40,
             q=p, out=p):
        return f(q, native.DCP_BF16, batch, hq, ctypes.byref(kv), p, bt_stride, max_vb, p, dcp, rb, rc,
                 ctypes.c_float(scale), 0, out, p, ws, ctypes.c_size_t(ws_bytes), NULL)

    assert call(rb=3, rc=2) == INV                 # rank range past dcp_size
    assert call(rb=-1) == INV
    assert call(rc=0) == INV
    assert call(bt_stride=2) == INV
    assert call(scale=float("inf")) == INV
    assert call(q=NULL) == INV
    assert call(out=NULL) == INV
    assert call(ws_bytes=16) == WS                 # workspace too small
    assert call(batch=0) == 0                      # empty batch: nothing launched


def test_merge_validation(L):
    p = _fake()
    f = L.dcp_lse_merge
    assert f(p, p, 0, 2, 4, 8, NULL, 0, p, p, NULL) == INV      # no parts
    assert f(p, p, 65, 2, 4, 8, NULL, 0, p, p, NULL) == INV     # too many parts
    assert f(p, p, 2, 2, 0, 8, NULL, 0, p, p, NULL) == INV      # heads
    assert f(p, p, 2, 2, 4, 8, NULL, 2, p, p, NULL) == UNS      # fp8 output
    assert f(NULL, p, 2, 2, 4, 8, NULL, 0, p, p, NULL) == INV
    assert f(NULL, NULL, 2, 0, 4, 8, NULL, 0, NULL, NULL, NULL) == 0


def test_kv_cache_write_validation(L):
    p = _fake(64)
    f = L.dcp_kv_cache_write
    F32, BF16 = native.DCP_F32, native.DCP_BF16

    def call(k=p, v=p, src=BF16, T=4, slots=p, R=2, kv=None):
        return f(k, v, src, T, slots, R, ctypes.byref(kv if kv is not None else _kv()), NULL)

    assert call(T=-1) == INV
    assert call(R=0) == INV
    assert call(R=65) == UNS                                   # one lane per rank
    assert call(src=native.DCP_FP8_E4M3) == UNS                # sources are fp32 or bf16
    assert call(kv=_kv(dtype=9)) == UNS
    assert call(v=NULL) == INV                                 # GQA pools need V rows
    assert call(kv=_kv(v=None, head_dim_v=64)) == INV          # MLA pools take no V rows
    assert call(kv=_kv(head_dim_k=100, head_dim_v=100)) == UNS # not a multiple of 8
    assert call(kv=_kv(dtype=native.DCP_FP8_E4M3)) == INV      # fp8 without scales
    assert call(kv=_kv(dtype=native.DCP_FP8_E4M3, k_scale=4096)) == INV  # V scale missing
    assert call(kv=_kv(num_blocks=0)) == INV
    assert call(k=NULL) == INV
    assert call(slots=NULL) == INV
    assert call(k=ctypes.c_void_p(p.value + 2)) == UNS         # unaligned source rows
    assert call(T=0, k=NULL, slots=NULL) == 0                  # empty: nothing launched
    assert call(T=0, src=F32, kv=_kv(v=None, head_dim_v=64), v=NULL) == 0


def test_verify_validation(L):
    def ws(q_len, batch=4, hq=8, algo=0, kv=None):
        st = ctypes.c_int(123)
        n = L.dcp_partial_verify_attn_workspace_size(batch, q_len, hq, native.DCP_BF16,
                                                     ctypes.byref(kv if kv is not None else _kv()), 2, algo,
                                                     ctypes.byref(st))
        return st.value, n
    assert ws(0)[0] == INV and ws(65)[0] == INV           # 1 <= q_len <= 64
    st1, n1 = ws(1)
    st2, n2 = ws(2)
    assert st1 == 0 and st2 == 0 and n2 > n1            # two units' rows per worker piece
    _, n_dec = _ws(L, _kv())
    assert n1 == n_dec                                   # q_len = 1 is decode
    assert ws(8, algo=native.DCP_ALGO_GENERIC) == (0, 0)
    p = _fake(64)
    f = L.dcp_partial_verify_attn
    assert f(p, native.DCP_BF16, 4, 0, 8, ctypes.byref(_kv()), p, 4, 4, p, 4, 0, 2, ctypes.c_float(0.1), 0, p, p,
             p, ctypes.c_size_t(1 << 40), NULL) == INV
    assert f(p, native.DCP_BF16, 0, 3, 8, ctypes.byref(_kv()), p, 4, 4, p, 4, 0, 2, ctypes.c_float(0.1), 0, p, p,
             p, ctypes.c_size_t(1 << 40), NULL) == 0     # empty batch: nothing launched


def test_segment_validation(L):
    st = ctypes.c_int(5)
    n = L.dcp_partial_segment_attn_workspace_size(4, 8, native.DCP_BF16, ctypes.byref(_kv()), 0, ctypes.byref(st))
    assert st.value == 0 and n > 4 * 8 * 128 * 4           # segment partial + attention workspace
    p = _fake(64)
    f = L.dcp_partial_segment_attn

    def call(seg_rank=1, rb=0, rc=2, part=p, ws_bytes=1 << 40, batch=4, scale=0.1, stride=4, lens=p, algo=0):
        return f(p, native.DCP_BF16, batch, 8, ctypes.byref(_kv()), p, stride, 4, lens, ctypes.c_float(scale), algo,
                 seg_rank, rb, rc, part, p, p, ctypes.c_size_t(ws_bytes), NULL)

    assert call(seg_rank=-1) == INV
    assert call(rc=0) == INV
    assert call(seg_rank=5) == 0          # another GPU's rank counts the segment: nothing launched
    assert call(part=NULL) == INV
    assert call(ws_bytes=16) == WS
    assert call(batch=0) == 0
    # the segment's attention checks the arguments dcp_partial_decode_attn checks
    for algo in (0, 1, 2):
        assert call(scale=float("nan"), algo=algo) == INV
        assert call(stride=3, algo=algo) == INV       # stride < seg_max_vblocks
        assert call(lens=NULL, algo=algo) == INV


def test_hbm_read_probe_validation(L):
    p = _fake(64)
    aligned = ctypes.c_void_p((p.value + 15) // 16 * 16)   # (never dereferenced: every call below is refused)
    f = L.dcp_hbm_read_probe
    assert f(p, 0, p, 1, NULL) == 0                  # nothing to read: nothing launched
    assert f(p, 24, p, 8, NULL) == INV               # not a multiple of 16 bytes
    assert f(p, -16, p, 8, NULL) == INV
    assert f(p, 32, p, 0, NULL) == INV               # no digest entries
    assert f(NULL, 32, p, 8, NULL) == INV
    assert f(aligned, 32, NULL, 8, NULL) == INV
    misaligned = ctypes.c_void_p(aligned.value + 4)
    assert f(misaligned, 32, p, 8, NULL) == INV


def test_gather_validation(L):
    p = _fake(64)
    f = L.dcp_gather_context
    kv = _kv()

    def call(kv=kv, D=4, I=1, nreq=2, stride=4, maxvb=4, cu=p, total=100, out_k=p, out_v=NULL):
        return f(ctypes.byref(kv), D, I, p, nreq, stride, maxvb, cu, total, out_k, out_v, NULL)

    assert call(I=3) == INV                                # block_size 16 % 3
    assert call(stride=2) == INV                           # stride < max_vblocks
    assert call(total=-1) == INV
    assert call(cu=NULL) == INV
    assert call(out_k=NULL) == INV
    assert call(nreq=0) == INV                             # tokens but no request
    assert call(kv=_kv(v=None, head_dim_v=64), out_v=p) == INV   # MLA: no V output
    assert call(kv=_kv(dtype=9)) == UNS
    assert call(out_v=p) == UNS                            # V transposed inside a block
    assert call(kv=_kv(head_dim_k=4)) == UNS               # rows under 16 bytes
    assert call(total=0, cu=NULL, out_k=NULL) == 0         # nothing to gather


def test_check_block_table_validation(L):
    p = _fake()
    call = L.dcp_check_block_table
    assert call(p, 2, 8, 8, p, 0, 4, 10, p, NULL) == INV       # block_size
    assert call(p, 2, 8, 8, p, 16, 0, 10, p, NULL) == INV      # dcp_size
    assert call(p, -1, 8, 8, p, 16, 4, 10, p, NULL) == INV     # num_reqs
    assert call(p, 2, 4, 8, p, 16, 4, 10, p, NULL) == INV      # stride below max_vblocks
    assert call(p, 2, 8, -1, p, 16, 4, 10, p, NULL) == INV     # max_vblocks
    assert call(p, 2, 8, 8, p, 16, 4, -1, p, NULL) == INV      # num_blocks
    assert call(p, 2, 8, 8, p, 16, 4, 10, NULL, NULL) == INV   # bad_count
    assert call(p, 2, 8, 8, NULL, 16, 4, 10, p, NULL) == INV   # seq_lens
    assert call(NULL, 2, 8, 8, p, 16, 4, 10, p, NULL) == INV   # block table


def test_product_path_loads_no_oracle():
    """The package, the workload generators and the device-side set-up that
    bench.py times through load no module of the oracle (it enters only in
    the tests' checks and bench.py's cpu_baseline functions)."""
    import subprocess
    import sys
    code = ("import sys; import sequence_sharded_paged_amd, workloads, workloads.generate, workloads.device; "
            "bad = [m for m in sys.modules if m == 'oracle' or m.startswith('oracle.')]; "
            "assert not bad, bad")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, "-c", code], cwd=root, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]


def test_noalloc_validation(L):
    """The no-allocation decode entry point checks its arguments like the one
    with a workspace, then refuses (before looking up its scratch or launching
    anything) a problem whose workspace exceeds the fixed scratch."""
    p = _fake(64)
    f = L.dcp_partial_decode_attn_noalloc

    def call(kv, batch=4, hq=8, bt_stride=4, max_vb=4, dcp=4, rb=0, rc=2, scale=0.1, q=p, algo=0):
        return f(q, native.DCP_BF16, batch, hq, ctypes.byref(kv), p, bt_stride, max_vb, p, dcp, rb, rc,
                 ctypes.c_float(scale), algo, p, p, NULL)

    kv = _kv()
    assert call(kv, rb=3, rc=2) == INV
    assert call(kv, bt_stride=2) == INV
    assert call(kv, scale=float("nan")) == INV
    assert call(kv, q=NULL) == INV
    assert call(kv, hq=7) == INV
    assert call(kv, batch=0) == 0                  # empty: nothing launched, no scratch needed
    mla = _kv(num_kv_heads=1, head_dim_k=576, head_dim_v=512, v=None)
    st, n = _ws(L, mla, batch=1 << 20, hq=128, rc=8)
    assert st == 0 and n > native.DCP_NOALLOC_SCRATCH_BYTES
    assert call(mla, batch=1 << 20, hq=128, dcp=8, rc=8) == native.DCP_ERR_SCRATCH
    st, n = _ws(L, mla, batch=64, hq=128, rc=8)    # the bimodal MLA batch fits
    assert st == 0 and 0 < n <= native.DCP_NOALLOC_SCRATCH_BYTES
