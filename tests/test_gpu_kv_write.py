"""GPU parity of the KV-cache write (dcp_kv_cache_write) against the oracle.

Stored bits must match the oracle's bit for bit (fp32 values, bf16 patterns,
fp8 codes), in every pool layout the attention kernels read and in padded
layouts that force the element-wise store path. Pools start as a byte
sentinel on both sides, so a write to a wrong place, or a write where the
slot says "not on this rank", shows up as a changed byte.

Small cases compare whole pools with ``oracle.cache.cache_write``. The
full-size KV-write workloads compare every written row with the oracle's
stored rows (``oracle.cache.store_values`` at the oracle's slot mapping),
then restore those rows to the sentinel and require the whole pool to be
the sentinel again (nothing else was touched).
"""

import zlib

import numpy as np
import pytest
import torch

import sequence_sharded_paged_amd as dcp
from oracle import cache as ocache
from oracle import formats as ofmt
from oracle import layout as olay
from workloads import KV_WRITE_WORKLOADS, get_kv_write_workload, make_kv_write_case
from workloads.generate import stored_numpy

pytestmark = pytest.mark.gpu

SENTINEL = 0xA5
POOL_T = {"fp32": torch.float32, "bf16": torch.bfloat16, "fp8_e4m3": torch.float8_e4m3fn}
RAW_T = {1: torch.uint8, 2: torch.int16, 4: torch.int32}
NP_RAW = {1: np.uint8, 2: np.uint16, 4: np.uint32}
SRC_T = {"fp32": torch.float32, "bf16": torch.bfloat16}


def _raw(t):
    return t.view(RAW_T[t.element_size()])


def _host_bits(t):
    """Device tensor -> host uint array of its bytes' element patterns."""
    return _raw(t).cpu().numpy().view(NP_RAW[t.element_size()])


def _sentinel_pool(shape, fmt, device, pad_last=0):
    """Pool tensor of ``shape`` (+ ``pad_last`` unused elements on the last
    axis) filled with the byte sentinel; returns (storage, logical view)."""
    full = list(shape)
    full[-1] += pad_last
    t = torch.empty(full, dtype=POOL_T[fmt], device=device)
    t.view(torch.uint8).fill_(SENTINEL)
    return t, t[..., :shape[-1]]


def _descriptor(fmt, k_log, v_log, N, bs, H, Dk, Dv, k_scale=None, v_scale=None):
    """dcp_kv_cache_t for logical views K [R, N, H, bs, Dk] and V [R, N, H, bs, Dv]
    (any strides) or V None."""
    d = dcp.native.KvCache()
    d.dtype = dcp.native.TORCH_TO_DCP[POOL_T[fmt]]
    d.num_blocks, d.block_size, d.num_kv_heads, d.head_dim_k, d.head_dim_v = N, bs, H, Dk, Dv
    d.k = k_log.data_ptr()
    for i, s in enumerate(k_log.stride()):
        d.k_stride[i] = s
    if v_log is None:
        d.v = None
    else:
        d.v = v_log.data_ptr()
        for i, s in enumerate(v_log.stride()):
            d.v_stride[i] = s
    d.k_scale = None if k_scale is None else k_scale.data_ptr()
    d.v_scale = None if v_scale is None else v_scale.data_ptr()
    return d


def _oracle_input(src):
    """The fp32 values of a device source tensor (exact for bf16)."""
    st = stored_numpy(src)
    if src.dtype == torch.bfloat16:
        return ofmt.decode(st, ofmt.BF16).astype(np.float32)
    return st.copy()


def _oracle_pool(shape, fmt):
    a = np.empty(shape, dtype={"fp32": np.float32, "bf16": np.uint16, "fp8_e4m3": np.uint8}[fmt])
    a.view(np.uint8)[...] = SENTINEL
    return a


def _special_values(rng, n):
    """Finite normals plus the cases the formats treat specially."""
    x = (rng.standard_normal(n) * 3.0).astype(np.float32)
    e4m3 = ofmt.e4m3fn_table()[:0x7F]
    mids = ((e4m3[:-1] + e4m3[1:]) / 2).astype(np.float32)          # exact ties of the fp8 rounding
    specials = np.concatenate([
        [np.nan, np.inf, -np.inf, 0.0, -0.0, 448.0, -448.0, 464.0, 1e30, -1e30, 2.0 ** -10, 3 * 2.0 ** -10,
         1e-40, -1e-42, 3.0e38, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 2.0 ** -6, 0.9999999],
        mids, -mids,
    ]).astype(np.float32)
    idx = rng.choice(n, size=min(n, specials.size), replace=False)
    x[idx] = specials[:idx.size]
    return x


def _slots_for(rng, T, R, N, bs, I):
    """Seeded positions in a few requests, mapped by the oracle, plus extra
    cases: tokens owned by no rank, slots past the pool, negative slots, and
    tokens that a second rank also owns (at slots of an otherwise unused block)."""
    span = bs * R
    nreq = min(3, N - 1)
    per_req = (N - 1) // nreq                                        # virtual blocks per request
    lens = rng.integers(1, per_req * span + 1, size=nreq)
    perm = rng.permutation(N - 1).astype(np.int32)                  # block N-1 stays free
    table = perm[:nreq * per_req].reshape(nreq, per_req)
    reqs = rng.integers(0, nreq, size=T).astype(np.int32)
    positions = np.full(T, -1, dtype=np.int64)                       # surplus tokens: no position, no owner
    for b in range(nreq):
        sel = np.flatnonzero(reqs == b)
        n = min(sel.size, int(lens[b]))
        positions[sel[:n]] = rng.choice(int(lens[b]), size=n, replace=False)  # distinct: no shared slots
    slots = olay.slot_mapping(positions, reqs, table, bs, R, I)
    if T >= 8:
        slots[:, 0] = -1                                             # owned by nobody
        slots[0, 1] = N * bs                                         # past the pool: skipped
        slots[R - 1, 2] = -7                                         # negative: skipped
        free = (N - 1) * bs
        slots[:, 3] = -1
        slots[0, 3] = free + 0                                       # owned by two ranks
        slots[R - 1, 3] = free + (bs - 1)
    return slots


# Batches under 1024 tokens take the per-(token, head) kernel. Larger ones take
# the one-token-per-wavefront row kernel when a token's row is 48..64 pieces
# of 16 elements in aligned pools (8 x 128 with a block size that is not a
# power of two, 3 x 256 with 16 idle lanes, 8 x 128 over 8 ranks; padded pools
# fall back), else the general row kernel (4 x 128 is 32 pieces); V stored
# dim-major takes the 64-token tile kernels (whose
# last tile is ragged in every case below; the last two have 8 ranks, 16-byte
# words of fp8 slots aligned in the pool, and scattered positions that give
# tiles several rounds of word groups).
GQA_CASES = [
    # (H, Dk, Dv, bs, R, I, N, T)
    (2, 16, 16, 16, 4, 1, 6, 70),
    (8, 128, 128, 16, 4, 2, 5, 150),
    (3, 24, 40, 8, 3, 8, 7, 65),
    (1, 8, 8, 1, 2, 1, 40, 33),
    (2, 16, 16, 16, 4, 1, 80, 1100),
    (3, 24, 136, 8, 3, 8, 150, 1030),
    (8, 128, 128, 24, 4, 8, 40, 1301),
    (3, 256, 256, 16, 3, 16, 60, 1030),
    (4, 128, 128, 64, 8, 64, 40, 1100),
    (8, 128, 128, 32, 8, 1, 60, 1090),
]


@pytest.mark.parametrize("fmt", ["fp32", "bf16", "fp8_e4m3"])
@pytest.mark.parametrize("src", ["fp32", "bf16"])
@pytest.mark.parametrize("case", GQA_CASES)
@pytest.mark.parametrize("v_layout", ["dim_major", "token_major", "padded"])
def test_gqa_write_bitexact(device, fmt, src, case, v_layout):
    H, Dk, Dv, bs, R, I, N, T = case
    seed = zlib.crc32(repr((fmt, src, case, v_layout)).encode())
    rng = np.random.default_rng(seed)
    slots = _slots_for(rng, T, R, N, bs, I)
    k32 = _special_values(rng, T * H * Dk).reshape(T, H, Dk)
    v32 = _special_values(rng, T * H * Dv).reshape(T, H, Dv)
    k_src = torch.from_numpy(k32).to(device).to(SRC_T[src])
    v_src = torch.from_numpy(v32).to(device).to(SRC_T[src])
    k_scale = v_scale = None
    ks_np = vs_np = None
    if fmt == "fp8_e4m3":
        ks_np = np.array([1.0, 0.37, 2.0 ** -5, 3.5, 0.5, 1.25, 0.01, 9.0][:H], dtype=np.float32)
        vs_np = np.array([0.25, 1.0, 0.7, 2.0, 6.0, 0.03, 1.5, 1.0][:H], dtype=np.float32)
        k_scale = torch.from_numpy(ks_np).to(device)
        v_scale = torch.from_numpy(vs_np).to(device)

    pad = 3 if v_layout == "padded" else 0     # row strides off the 8-element grid: element-wise stores
    k_store, k_log = _sentinel_pool((R, N, H, bs, Dk), fmt, device, pad_last=pad)
    if v_layout == "dim_major":
        v_store, v_phys = _sentinel_pool((R, N, H, Dv, bs), fmt, device)
        v_log = v_phys.transpose(3, 4)
    else:
        v_store, v_log = _sentinel_pool((R, N, H, bs, Dv), fmt, device, pad_last=5 if pad else 0)
    d = _descriptor(fmt, k_log, v_log, N, bs, H, Dk, Dv, k_scale, v_scale)
    dcp.dcp_kv_cache_write(k_src, v_src, torch.from_numpy(slots).to(device), d)
    torch.cuda.synchronize()

    ko = _oracle_pool((R, N, H, bs, Dk + pad), fmt)
    vo_shape = (R, N, H, Dv, bs) if v_layout == "dim_major" else (R, N, H, bs, Dv + (5 if pad else 0))
    vo = _oracle_pool(vo_shape, fmt)
    vo_log = vo if v_layout == "dim_major" else np.swapaxes(vo[..., :Dv], 3, 4)  # oracle's V is [.., dim, token]
    ocache.cache_write(ko[..., :Dk], vo_log, _oracle_input(k_src), _oracle_input(v_src), slots, bs, fmt,
                       ks_np, vs_np)
    kb, vb = _host_bits(k_store), _host_bits(v_store)
    nb = {"fp32": np.uint32, "bf16": np.uint16, "fp8_e4m3": np.uint8}[fmt]
    assert np.array_equal(kb, ko.view(nb)), "K pool differs"
    assert np.array_equal(vb, vo.view(nb)), "V pool differs"


@pytest.mark.parametrize("fmt", ["fp32", "bf16", "fp8_e4m3"])
@pytest.mark.parametrize("src", ["fp32", "bf16"])
@pytest.mark.parametrize("N,T", [(4, 300), (7, 1500)])
def test_mla_write_bitexact(device, fmt, src, N, T):
    H, Dk, Dv, bs, R, I = 1, 576, 512, 64, 8, 1
    rng = np.random.default_rng(1000 + len(fmt) + len(src) + T)
    slots = _slots_for(rng, T, R, N, bs, I)
    k32 = _special_values(rng, T * H * Dk).reshape(T, H, Dk)
    k_src = torch.from_numpy(k32).to(device).to(SRC_T[src])
    ks_np = np.array([0.031], dtype=np.float32) if fmt == "fp8_e4m3" else None
    k_scale = None if ks_np is None else torch.from_numpy(ks_np).to(device)
    k_store, k_log = _sentinel_pool((R, N, H, bs, Dk), fmt, device)
    d = _descriptor(fmt, k_log, None, N, bs, H, Dk, Dv, k_scale, None)
    dcp.dcp_kv_cache_write(k_src, None, torch.from_numpy(slots).to(device), d)
    torch.cuda.synchronize()
    ko = _oracle_pool((R, N, H, bs, Dk), fmt)
    ocache.cache_write(ko, None, _oracle_input(k_src), None, slots, bs, fmt, ks_np, None)
    nb = {"fp32": np.uint32, "bf16": np.uint16, "fp8_e4m3": np.uint8}[fmt]
    assert np.array_equal(_host_bits(k_store), ko.view(nb))


@pytest.mark.parametrize("reps", [1, 400])
def test_fp8_quotients_next_to_code_midpoints(device, reps):
    """Inputs whose quotient by a non-power-of-two scale lands on, or one fp32
    step either side of, a midpoint between E4M3 codes: the cases where a
    quotient computed with an error of even one fp32 ulp rounds apart."""
    scales = np.array([0.37, 0.0134, 3.3, 1e-3, 7.77e-7, 2.0 ** 99, 1e-35, 1.0], dtype=np.float32)
    H, D, bs, R = scales.size, 256, 16, 1                                            # 2 x 126 midpoints fit in D
    e4m3 = ofmt.e4m3fn_table()[:0x7F]
    mids = ((e4m3[:-1] + e4m3[1:]) / 2).astype(np.float32)
    with np.errstate(over="ignore"):
        base = np.concatenate([mids, -mids]).astype(np.float32)[None, :] * scales[:, None]   # [H, 252]
    x = np.stack([base, np.nextafter(base, np.float32(np.inf)), np.nextafter(base, np.float32(-np.inf))])
    k32 = np.pad(x, ((0, 0), (0, 0), (0, D - x.shape[2]))).astype(np.float32)         # [3, H, D]
    k32 = np.ascontiguousarray(np.tile(k32, (reps, 1, 1)))
    T = k32.shape[0]
    N = (T + 16) // bs + 2
    slots = (np.random.default_rng(reps).permutation(N * bs)[:T]).astype(np.int64)[None, :]
    sc = torch.from_numpy(scales).to(device)
    k_store, k_log = _sentinel_pool((R, N, H, bs, D), "fp8_e4m3", device)
    d = _descriptor("fp8_e4m3", k_log, None, N, bs, H, D, D, sc, None)
    dcp.dcp_kv_cache_write(torch.from_numpy(k32).to(device), None, torch.from_numpy(slots).to(device), d)
    torch.cuda.synchronize()
    ko = _oracle_pool((R, N, H, bs, D), "fp8_e4m3")
    ocache.cache_write(ko, None, k32, None, slots, bs, "fp8_e4m3", scales, None)
    assert np.array_equal(_host_bits(k_store), ko)


@pytest.mark.parametrize("fmt,scale", [("fp8_e4m3", 1.0), ("fp8_e4m3", 0.37), ("bf16", None)])
def test_conversion_sweep_over_fp32_patterns(device, fmt, scale):
    """Every 97th fp32 bit pattern (44M values: all exponents, signs, NaN
    payloads, infinities, subnormals) through the tile kernel, each stored
    value compared with the oracle's."""
    H, D, bs = 8, 128, 64
    pats = np.arange(0, 1 << 32, 97, dtype=np.uint64).astype(np.uint32)
    T = -(-pats.size // (H * D))
    pats = np.pad(pats, (0, T * H * D - pats.size))
    k32 = pats.view(np.float32).reshape(T, H, D)
    N = -(-T // bs)
    scales = None if scale is None else np.full(H, scale, dtype=np.float32)
    sc = None if scales is None else torch.from_numpy(scales).to(device)
    k_store, k_log = _sentinel_pool((1, N, H, bs, D), fmt, device)
    d = _descriptor(fmt, k_log, None, N, bs, H, D, D, sc, None)
    slots = torch.arange(T, dtype=torch.int64, device=device)[None, :]
    dcp.dcp_kv_cache_write(torch.from_numpy(k32).to(device), None, slots, d)
    torch.cuda.synchronize()
    got = _host_bits(k_store)[0].transpose(0, 2, 1, 3).reshape(N * bs, H, D)[:T]    # token order
    exp = ocache.store_values(k32, fmt, scales)
    bad = np.flatnonzero(got.reshape(-1) != exp.reshape(-1))
    assert bad.size == 0, (f"{bad.size} mismatches, e.g. x bits {pats[bad[:4]]}: got {got.reshape(-1)[bad[:4]]}, "
                           f"oracle {exp.reshape(-1)[bad[:4]]}")


def test_empty_write_launches_nothing(device):
    k_store, k_log = _sentinel_pool((2, 2, 1, 4, 8), "bf16", device)
    d = _descriptor("bf16", k_log, None, 2, 4, 1, 8, 8)
    empty = torch.empty((0, 1, 8), dtype=torch.bfloat16, device=device)
    dcp.dcp_kv_cache_write(empty, None, torch.empty((2, 0), dtype=torch.int64, device=device), d)
    torch.cuda.synchronize()
    assert bool((k_store.view(torch.uint8) == SENTINEL).all())


def test_two_writes_in_a_row_keep_earlier_rows(device):
    """A second write (fewer tokens, other slots) leaves the first one's rows."""
    H, Dk, Dv, bs, R, I, N = 2, 16, 16, 16, 2, 1, 6
    rng = np.random.default_rng(99)
    positions = np.arange(40, dtype=np.int64)
    reqs = np.zeros(40, dtype=np.int32)
    table = np.array([[3, 1]], dtype=np.int32)
    slots = olay.slot_mapping(positions, reqs, table, bs, R, I)
    k32 = rng.standard_normal((40, H, Dk)).astype(np.float32)
    v32 = rng.standard_normal((40, H, Dv)).astype(np.float32)
    k_store, k_log = _sentinel_pool((R, N, H, bs, Dk), "bf16", device)
    v_store, v_phys = _sentinel_pool((R, N, H, Dv, bs), "bf16", device)
    d = _descriptor("bf16", k_log, v_phys.transpose(3, 4), N, bs, H, Dk, Dv)
    ko, vo = _oracle_pool((R, N, H, bs, Dk), "bf16"), _oracle_pool((R, N, H, Dv, bs), "bf16")
    for lo, hi in ((0, 32), (32, 40)):
        ks = torch.from_numpy(k32[lo:hi]).to(device)
        vs = torch.from_numpy(v32[lo:hi]).to(device)
        dcp.dcp_kv_cache_write(ks, vs, torch.from_numpy(np.ascontiguousarray(slots[:, lo:hi])).to(device), d)
        ocache.cache_write(ko, vo, k32[lo:hi], v32[lo:hi], slots[:, lo:hi], bs, "bf16")
    torch.cuda.synchronize()
    assert np.array_equal(_host_bits(k_store), ko)
    assert np.array_equal(_host_bits(v_store), vo)


@pytest.mark.parametrize("name", sorted(KV_WRITE_WORKLOADS))
def test_full_size_workload(device, name):
    """The benchmark's KV-write workloads at full size, in the launch the
    benchmark times (slot mapping on the GPU, then the write)."""
    w = get_kv_write_workload(name)
    g = w.geometry()
    case = make_kv_write_case(w, device)
    R, N, H, bs = g.dcp_size, case.num_blocks, g.num_kv_heads, g.block_size
    fmt = g.kv_format
    slots_ref = olay.slot_mapping(case.positions, case.req_indices, case.block_table, bs, R, g.interleave)
    slots = dcp.dcp_slot_mapping(torch.from_numpy(case.positions).to(device),
                                 torch.from_numpy(case.req_indices).to(device),
                                 torch.from_numpy(case.block_table).to(device), bs, R, g.interleave)
    assert np.array_equal(slots.cpu().numpy(), slots_ref)
    k_scale = None if case.k_scale is None else torch.from_numpy(case.k_scale).to(device)
    v_scale = None if case.v_scale is None else torch.from_numpy(case.v_scale).to(device)
    k_store, k_log = _sentinel_pool((R, N, H, bs, g.head_dim_k), fmt, device)
    if g.mla:
        v_store = v_log = None
    else:
        v_store, v_phys = _sentinel_pool((R, N, H, g.head_dim_v, bs), fmt, device)
        v_log = v_phys.transpose(3, 4)
    d = _descriptor(fmt, k_log, v_log, N, bs, H, g.head_dim_k, g.head_dim_v, k_scale, v_scale)
    dcp.dcp_kv_cache_write(case.k_new, case.v_new, slots, d)
    torch.cuda.synchronize()

    k_exp = ocache.store_values(_oracle_input(case.k_new), fmt, case.k_scale)
    v_exp = None if g.mla else ocache.store_values(_oracle_input(case.v_new), fmt, case.v_scale)
    kraw = _raw(k_store)
    vraw = None if v_store is None else _raw(v_store)
    sentinel = {1: SENTINEL, 2: -0x5A5B, 4: -0x5A5A5A5B}[k_store.element_size()]  # 0xA5.. as signed
    written = 0
    for r in range(R):
        tok = np.flatnonzero(slots_ref[r] >= 0)
        if tok.size == 0:
            continue
        s = torch.from_numpy(slots_ref[r][tok]).to(device)
        blk, off = s // bs, s % bs
        got_k = kraw[r][blk, :, off, :].cpu().numpy().view(k_exp.dtype)
        assert np.array_equal(got_k, k_exp[tok]), f"K rows of rank {r}"
        kraw[r][blk, :, off, :] = sentinel
        if vraw is not None:
            got_v = vraw[r][blk, :, :, off].cpu().numpy().view(v_exp.dtype)
            assert np.array_equal(got_v, v_exp[tok]), f"V rows of rank {r}"
            vraw[r][blk, :, :, off] = sentinel
        written += tok.size
    assert written == w.tokens                      # every token has exactly one owner
    assert bool((k_store.view(torch.uint8) == SENTINEL).all()), "K bytes written outside the slots"
    if v_store is not None:
        assert bool((v_store.view(torch.uint8) == SENTINEL).all()), "V bytes written outside the slots"
