"""Shared test plumbing: device inputs for the HIP path, oracle evaluation on
the host, and the parity checks (tolerances from the project's acceptance
bar: max-abs 1e-5 for fp32 and 2e-2 for bf16/fp8 inputs, plus a per-row
relative bound and an LSE bound so that long rows, whose outputs are small,
cannot pass vacuously)."""

import numpy as np
import torch

import sequence_sharded_paged_amd as dcp  # noqa: F401
from workloads.device import DeviceInputs, SegmentInputs, VerifyRun, verify_query_lens  # noqa: F401
from workloads.generate import stored_numpy, stored_format


def _oracle():
    """The oracle modules, imported only by the functions that check against
    them (the device-side set-up lives in workloads.device and never loads
    the oracle)."""
    from oracle import attention, formats, layout
    return attention, formats, layout

TOL = {
    "fp32": dict(max_abs=1e-5, row_rel=1e-4, lse=1e-5),
    "bf16": dict(max_abs=2e-2, row_rel=1e-2, lse=1e-3),
    "fp8_e4m3": dict(max_abs=2e-2, row_rel=1e-2, lse=1e-3),
}
OUT_BF16_EXTRA = 2.0 ** -8   # relative rounding of a bf16 output element


def oracle_request(case, b, dcp_size=None, interleave=None, with_partials=True):
    """Float64 oracle for request b: full attention (with the sink) and the
    per-rank partials over the brute-force ownership."""
    oatt, ofmt, olay = _oracle()
    w = case.workload
    D = dcp_size or w.dcp_size
    I = interleave or w.interleave
    q = ofmt.decode(stored_numpy(case.q[b]), stored_format(case.q))
    k = ofmt.decode_kv(stored_numpy(case.k[b]), stored_format(case.k[b]), case.k_scale)
    if case.v is None:
        v = k[:, :, :w.head_dim_v]
    else:
        v = ofmt.decode_kv(stored_numpy(case.v[b]), stored_format(case.v[b]), case.v_scale)
    full = oatt.decode_attention(q, k, v, w.softmax_scale, case.sink)
    parts = None
    if with_partials:
        own = olay.owners(int(case.seq_lens[b]), w.block_size, D, I)
        parts = oatt.rank_partials(q, k, v, w.softmax_scale, own, D)
    return full, parts


def check_rows(got, ref, tol, what, out_bf16=False):
    """Element-wise max-abs and per-row relative bounds for [H, Dv] outputs."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = np.abs(got - ref)
    max_abs = tol["max_abs"]
    assert err.max() <= max_abs, f"{what}: max-abs {err.max():.3e} > {max_abs}"
    rel_tol = tol["row_rel"] + (OUT_BF16_EXTRA if out_bf16 else 0.0)
    row_ref = np.maximum(np.abs(ref).max(axis=-1), 1e-3)
    rel = err.max(axis=-1) / row_ref
    assert rel.max() <= rel_tol, f"{what}: row-relative {rel.max():.3e} > {rel_tol}"


def check_lse(got, ref, tol, what):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    inf_ref = np.isneginf(ref)
    assert np.array_equal(np.isneginf(got), inf_ref), f"{what}: -inf pattern differs"
    d = np.abs(got[~inf_ref] - ref[~inf_ref])
    if d.size:
        assert d.max() <= tol["lse"], f"{what}: LSE err {d.max():.3e} > {tol['lse']}"


def check_against_oracle(inputs, result, requests=None, check_parts=True, rank_begin=0):
    case, w = inputs.case, inputs.w
    po, pl, o, lse = [t.float().cpu().numpy() for t in result]
    tol = TOL[w.kv_format]
    R = po.shape[0]
    for b in (range(case.batch) if requests is None else requests):
        (fo, fl), parts = oracle_request(case, b, inputs.D, inputs.I, with_partials=check_parts)
        if R == inputs.D:
            check_rows(o[b], fo, tol, f"merged O b={b}", out_bf16=(w.out_format == "bf16"))
            check_lse(lse[b], fl, tol, f"merged LSE b={b}")
        if check_parts:
            ro, rl = parts
            for r in range(R):
                check_rows(po[r, b], ro[rank_begin + r], tol, f"partial O r={rank_begin + r} b={b}")
                check_lse(pl[r, b], rl[rank_begin + r], tol, f"partial LSE r={rank_begin + r} b={b}")


# ---------------------------------------------------------------------------
# multi-token decode (speculative verification)
# ---------------------------------------------------------------------------
def oracle_verify_request(case, q, b, dcp_size, interleave, with_partials=True):
    """Float64 oracle for request b's q_len query tokens: causal attention over
    the cached sequence (with the sink) and the per-rank partials."""
    oatt, ofmt, olay = _oracle()
    w = case.workload
    qb = ofmt.decode(stored_numpy(q[b]), stored_format(q))                     # [q_len, Hq, Dk]
    k = ofmt.decode_kv(stored_numpy(case.k[b]), stored_format(case.k[b]), case.k_scale)
    v = k[:, :, :w.head_dim_v] if case.v is None else ofmt.decode_kv(stored_numpy(case.v[b]),
                                                                      stored_format(case.v[b]), case.v_scale)
    full = oatt.verify_attention(qb, k, v, w.softmax_scale, case.sink)
    if not with_partials:
        return full, None
    own = olay.owners(int(case.seq_lens[b]), w.block_size, dcp_size, interleave)
    parts = oatt.verify_rank_partials(qb, k, v, w.softmax_scale, own, dcp_size)
    return full, parts


def check_verify_against_oracle(run, result, requests=None, check_parts=True):
    inputs = run.inputs
    case, w = inputs.case, inputs.w
    po, pl, o, lse = [t.float().cpu().numpy() for t in result]
    tol = TOL[w.kv_format]
    R = po.shape[0]
    for b in (range(case.batch) if requests is None else requests):
        (fo, fl), parts = oracle_verify_request(case, run.q.cpu(), b, inputs.D, inputs.I, with_partials=check_parts)
        for i in range(run.q_len):
            if R == inputs.D:
                check_rows(o[b, i], fo[i], tol, f"merged O b={b} i={i}", out_bf16=(w.out_format == "bf16"))
                check_lse(lse[b, i], fl[i], tol, f"merged LSE b={b} i={i}")
            if check_parts:
                ro, rl = parts
                for r in range(R):
                    rr = run.rank_begin + r
                    check_rows(po[r, b, i], ro[rr, i], tol, f"partial O r={rr} b={b} i={i}")
                    check_lse(pl[r, b, i], rl[rr, i], tol, f"partial LSE r={rr} b={b} i={i}")


# ---------------------------------------------------------------------------
# replicated segment (a sliding-window cache counted by one rank)
# ---------------------------------------------------------------------------
def oracle_segment_request(case, seg, b, dcp_size, interleave, seg_rank, with_partials=True):
    """Float64 oracle for request b with its segment: attention over the
    sequence and the segment together (sink included) and the per-rank
    partials with the segment on rank seg_rank."""
    oatt, ofmt, olay = _oracle()
    w = case.workload
    q = ofmt.decode(stored_numpy(case.q[b]), stored_format(case.q))

    def kv(kt, vt):
        k = ofmt.decode_kv(stored_numpy(kt), stored_format(kt), case.k_scale)
        v = k[:, :, :w.head_dim_v] if vt is None else ofmt.decode_kv(stored_numpy(vt), stored_format(vt),
                                                                      case.v_scale)
        return k, v

    k, v = kv(case.k[b], None if case.v is None else case.v[b])
    ks, vs = kv(seg.k[b], None if seg.v is None else seg.v[b])
    full = oatt.decode_attention(q, np.concatenate([k, ks]), np.concatenate([v, vs]), w.softmax_scale, case.sink)
    if not with_partials:
        return full, None
    own = olay.owners(int(case.seq_lens[b]), w.block_size, dcp_size, interleave)
    parts = oatt.segment_rank_partials(q, k, v, w.softmax_scale, own, dcp_size, ks, vs, seg_rank)
    return full, parts


def check_segment_against_oracle(inputs, seg, seg_rank, result, requests=None, check_parts=True):
    case, w = inputs.case, inputs.w
    po, pl, o, lse = [t.float().cpu().numpy() for t in result]
    tol = TOL[w.kv_format]
    R = po.shape[0]
    for b in (range(case.batch) if requests is None else requests):
        (fo, fl), parts = oracle_segment_request(case, seg, b, inputs.D, inputs.I, seg_rank, with_partials=check_parts)
        if R == inputs.D:
            check_rows(o[b], fo, tol, f"merged O b={b}", out_bf16=(w.out_format == "bf16"))
            check_lse(lse[b], fl, tol, f"merged LSE b={b}")
        if not check_parts:
            continue
        ro, rl = parts
        for r in range(R):
            rr = inputs.rank_begin + r
            check_rows(po[r, b], ro[rr], tol, f"partial O r={rr} b={b}")
            check_lse(pl[r, b], rl[rr], tol, f"partial LSE r={rr} b={b}")
