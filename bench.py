#!/usr/bin/env python3
"""Benchmark: one DCP decode step on one MI355X.

A step is the whole hot path over one batch already resident in HBM: every
DCP rank's partial decode attention over its sequence shard (the MFMA
attention kernel and the split combine, with a planner kernel first for MLA)
followed by the log-sum-exp merge across the ranks. The batch is synthetic (seeded; lengths, geometry and value
distributions of the named workload). Prints ONE JSON line:

* ``value``   - algorithmic KV bytes of the batch / step time, in GB/s
                (KV bytes = sum of context lengths x KV bytes per token);
* ``roofline``- the main attention kernel alone, timed with HIP events that
                the library records around it on the launch stream (in a
                second loop of as many steps, so that the step time carries
                no instrumentation), against
                the 8 TB/s HBM peak; ``traffic`` comes from the committed
                rocprofv3 counter summary when it was taken on the current
                kernel source, else null;
* ``cpu_baseline`` - the float64 CPU oracle timed on a bounded sample of the
                same batch (rank 0, N = 1 only);
* ``per_config``- (default run) the same measurements for the GQA bf16, the
                two MLA and the GQA fp8 decode workloads, each with a shorter
                oracle sample, the MLA ones also against the bf16 MFMA peak;
* ``hbm_read_ceiling`` - (default run) the device's measured streaming-read
                rate (dcp_hbm_read_probe over 8 GiB); every decode roofline
                then also carries ``frac_of_read_ceiling``;
* ``layout``  - local lengths and the slot mapping (one decode step's new
                tokens, and the bulk fill of every cached token) timed apart
                from the step, with the oracle's brute-force mapper beside it.

With a multi-token decode workload (``--workload *_q<N>``) a step is every
rank's partial attention for the last N tokens of every request at once
(causal among them) plus the merge; ``value`` counts the KV bytes of the
batch once, like decode, and ``config`` adds the verified tokens per second.

With a replicated-segment workload (``--workload *_swa<W>``) a step is every
rank's partial attention, the fold of each request's W-token segment into
the designated rank's partial, and the merge (sink once); ``value`` counts
the sharded KV and the segments once.

With ``--workload gather_<decode workload>`` a step is the chunked-prefill
context gather of every request's whole cached sequence back into
request-contiguous order (``value``: bytes read + written per second).

With ``--workload kvw_*`` a step is instead the KV-cache write of a batch of
new tokens (slot mapping, then the write of every row into its owner's pool);
``value`` and ``roofline`` then count the write's algorithmic bytes (new rows
read, one slot per rank read, stored rows written once).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
"""

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "decode-attn KV GB/s (% of MI355X HBM peak) + merged queries/s at 1 GPU"
DEFAULT_WORKLOAD = "gqa_fp8_binned"
KV_WRITE_METRIC = "KV-cache write GB/s (new rows + slots read, stored rows written) at 1 GPU"
VERIFY_METRIC = "multi-token decode KV GB/s (% of MI355X HBM peak) + verified tokens/s at 1 GPU"
SEGMENT_METRIC = "decode with a replicated segment: KV GB/s (% of MI355X HBM peak) + merged queries/s at 1 GPU"
GATHER_METRIC = "context gather GB/s (stored rows read + written) at 1 GPU"
KERNEL_NAMES = {"gqa": "gqa_attn_kernel", "mla": "mla_attn_kernel", "generic": "generic_attn_kernel",
                "kv_write": "kv_write", "gather": "gather_context_kernel"}
# Sources compiled into each kernel family (the attention kernels include the
# split-KV header, which fixes their workspace layout, and through it the
# 64-bit half split and join).
KERNEL_SOURCES = {"gqa": ["attn_gqa.hip", "splitkv.h", "halves.h"], "mla": ["attn_mla.hip", "splitkv.h", "halves.h"],
                  "generic": ["attn_generic.hip"], "kv_write": ["kv_write.hip"], "gather": ["gather.hip"]}


def kernel_family(w):
    if w.mla:
        return "mla"
    if w.kv_format in ("bf16", "fp8_e4m3") and w.head_dim_k == 128:
        return "gqa"
    return "generic"


def source_hash(family):
    """sha256 prefix of the family's sources, concatenated in the listed order."""
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[family]:
        with open(os.path.join(ROOT, "sequence_sharded_paged_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(family, workload):
    """HBM bytes per launch from the committed counter summary, if it was
    taken on the current kernel source."""
    path = os.path.join(ROOT, "profiles", f"{KERNEL_NAMES[family]}_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_sha256_16") != source_hash(family):
        return None
    return rec.get("hbm_bytes_per_launch")


def timed_steps(step, steps):
    """(ms per step, ms per main attention kernel): the steps are timed first
    with nothing recorded between their launches, then as many again with the
    library's HIP events around each attention kernel (events recorded on the
    stream add a gap to every step, which would otherwise count as step time)."""
    import torch
    import sequence_sharded_paged_amd as dcp
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for _ in range(steps):
        step()
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / steps
    dcp.native.dcp_profile_enable(True)
    dcp.native.dcp_profile_collect()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    kern_ms, launches = dcp.native.dcp_profile_collect()
    dcp.native.dcp_profile_enable(False)
    return ms, kern_ms / max(launches, 1)


def blas_threads():
    """Threads NumPy's BLAS uses (the oracle's matrix products run there)."""
    try:
        from threadpoolctl import threadpool_info
        return max([d.get("num_threads", 1) for d in threadpool_info() if d.get("user_api") == "blas"] or [1])
    except Exception:  # threadpoolctl missing
        return 1


def cpu_baseline(case, budget_s):
    """Time the float64 oracle on a seeded sample of requests (~budget_s)."""
    import numpy as np
    from oracle import attention as oatt
    from oracle import formats as ofmt
    from workloads.generate import stored_format, stored_numpy
    threads = blas_threads()
    w = case.workload
    order = np.random.default_rng(12345).permutation(case.batch)
    spent, kv_bytes, done = 0.0, 0, []
    for b in order:
        q_st = stored_numpy(case.q[b])
        k_st = stored_numpy(case.k[b])
        v_st = None if case.v is None else stored_numpy(case.v[b])
        t0 = time.perf_counter()
        q = ofmt.decode(q_st, stored_format(case.q))
        k = ofmt.decode_kv(k_st, stored_format(case.k[b]), case.k_scale)
        v = k[:, :, :w.head_dim_v] if v_st is None else ofmt.decode_kv(v_st, stored_format(case.v[b]),
                                                                        case.v_scale)
        oatt.decode_attention(q, k, v, w.softmax_scale, case.sink)
        spent += time.perf_counter() - t0
        kv_bytes += int(case.seq_lens[b]) * w.kv_bytes_per_token()
        done.append(int(b))
        if spent >= budget_s:
            break
    return {
        "value": kv_bytes / spent / 1e9,
        "unit": "GB/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": (f"{len(done)} of {case.batch} requests (seeded random order, "
                   f"{sum(int(case.seq_lens[b]) for b in done)} tokens), full softmax over the unsharded "
                   f"sequence in float64 incl. decoding the stored KV; {spent:.1f} s"),
        "queries_per_s": len(done) / spent,
    }


def kv_write_kernels(w):
    """The kernels one dcp_kv_cache_write call launches for this workload."""
    if w.tokens < 1024:
        return ["kv_scatter_kernel"]
    g = w.geometry()
    if g.mla:
        return ["kv_rows_kernel"]  # 576-wide latent rows: 36 pieces of 16, the general row kernel
    return ["kv_tokrow_kernel", "kv_vt16_kernel"]  # 8 x 128 K rows; V stored dim-major


def cpu_baseline_kv_write(case, budget_s):
    """Time the oracle's slot mapping + cache write on request-sized pieces of
    the batch (~budget_s)."""
    import numpy as np
    from oracle import cache as ocache
    from oracle import formats as ofmt
    from oracle import layout as olay
    from workloads.generate import stored_numpy
    w, g = case.workload, case.workload.geometry()
    R, H, bs = g.dcp_size, g.num_kv_heads, g.block_size
    fmt = g.kv_format
    np_t = {"fp32": np.float32, "bf16": np.uint16, "fp8_e4m3": np.uint8}[fmt]
    k_all, v_all = stored_numpy(case.k_new), None if case.v_new is None else stored_numpy(case.v_new)
    spent, tokens, reqs = 0.0, 0, 0
    for b in range(w.requests):
        lo, hi = b * w.chunk, (b + 1) * w.chunk
        # a pool of just this request's blocks keeps the sample's memory bounded
        used = case.block_table[b][case.block_table[b] >= 0]
        table = np.full_like(case.block_table[b:b + 1], -1)
        table[0, :used.size] = np.arange(used.size, dtype=np.int32)
        kp = np.zeros((R, max(used.size, 1), H, bs, g.head_dim_k), dtype=np_t)
        vp = None if g.mla else np.zeros((R, max(used.size, 1), H, g.head_dim_v, bs), dtype=np_t)
        t0 = time.perf_counter()
        k = k_all[lo:hi] if w.src_format == "fp32" else ofmt.decode(k_all[lo:hi], ofmt.BF16).astype(np.float32)
        v = None
        if v_all is not None:
            v = v_all[lo:hi] if w.src_format == "fp32" else ofmt.decode(v_all[lo:hi], ofmt.BF16).astype(np.float32)
        slots = olay.slot_mapping(case.positions[lo:hi], np.zeros(hi - lo, dtype=np.int32), table, bs, R,
                                  g.interleave)
        ocache.cache_write(kp, vp, k, v, slots, bs, fmt, case.k_scale, case.v_scale)
        spent += time.perf_counter() - t0
        tokens += hi - lo
        reqs += 1
        if spent >= budget_s:
            break
    return {
        "value": tokens * w.bytes_per_token() / spent / 1e9,
        "unit": "GB/s",
        "cores": 1,
        "kind": "oracle",
        "sample": (f"{reqs} of {w.requests} requests ({tokens} of {w.tokens} tokens), slot mapping + "
                   f"quantise + placement in numpy, each request into a pool of its own blocks; {spent:.1f} s"),
    }


def bench_kv_write(args, name):
    import numpy as np
    import torch
    import sequence_sharded_paged_amd as dcp
    from workloads import get_kv_write_workload, make_kv_write_case
    from workloads.generate import TORCH_FORMAT

    w = get_kv_write_workload(name)
    g = w.geometry()
    dev = "cuda"
    t_gen = time.perf_counter()
    case = make_kv_write_case(w, dev)
    R, N, H, bs = g.dcp_size, case.num_blocks, g.num_kv_heads, g.block_size
    pool = dcp.PagedKVCache(R, N, bs, H, g.head_dim_k, g.head_dim_v, TORCH_FORMAT[g.kv_format], mla=g.mla,
                            device=dev, k_scale=case.k_scale, v_scale=case.v_scale)
    desc = pool.descriptor()
    positions = torch.from_numpy(case.positions).to(dev)
    reqs = torch.from_numpy(case.req_indices).to(dev)
    table = torch.from_numpy(case.block_table).to(dev)
    slots = torch.empty((R, w.tokens), dtype=torch.int64, device=dev)
    torch.cuda.synchronize()
    t_gen = time.perf_counter() - t_gen
    print(f"[bench] {w.name}: {w.tokens} tokens into {R} ranks x {N} blocks, "
          f"{w.tokens * w.bytes_per_token() / 1e6:.1f} MB per write, inputs ready in {t_gen:.1f} s",
          file=sys.stderr, flush=True)

    def step():
        dcp.dcp_slot_mapping(positions, reqs, table, bs, R, g.interleave, out=slots)
        dcp.dcp_kv_cache_write(case.k_new, case.v_new, slots, desc)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(args.steps):
        step()
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / args.steps
    # the write alone (its kernels back to back), on the stream they are launched on
    # (torch's current stream)
    start.record()
    for _ in range(args.steps):
        dcp.dcp_kv_cache_write(case.k_new, case.v_new, slots, desc)
    stop.record()
    torch.cuda.synchronize()
    kern_ms = start.elapsed_time(stop) / args.steps

    nbytes = w.tokens * w.bytes_per_token()
    out = {
        "metric": KV_WRITE_METRIC,
        "value": round(nbytes / (ms * 1e-3) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"fp32": "f32", "bf16": "bf16", "fp8_e4m3": "fp8_e4m3"}[g.kv_format],
        "data": "synthetic",
        "config": {
            "workload": w.name,
            "tokens": w.tokens,
            "requests": w.requests,
            "chunk": w.chunk,
            "num_kv_heads": H,
            "head_dim_k": g.head_dim_k,
            "head_dim_v": g.head_dim_v,
            "kv_format": g.kv_format,
            "src_format": w.src_format,
            "mla": g.mla,
            "block_size": bs,
            "dcp_size": R,
            "interleave": g.interleave,
            "bytes_per_token": w.bytes_per_token(),
            "tokens_per_s": round(w.tokens / (ms * 1e-3), 1),
            "kernel": "+".join(kv_write_kernels(w)),
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(nbytes / (kern_ms * 1e-3) / 1e9, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(nbytes / (kern_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "traffic": load_traffic("kv_write", w.name),
            "unit_of_launch": "one dcp_kv_cache_write call",
            "kernel_avg_ms": round(kern_ms, 5),
        },
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_kv_write(case, args.cpu_budget_s)
    print(json.dumps(out), flush=True)


def cpu_baseline_verify(case, q, q_len, budget_s):
    """Time the float64 oracle's multi-token decode on a seeded sample of requests."""
    import numpy as np
    from oracle import attention as oatt
    from oracle import formats as ofmt
    from workloads.generate import stored_format, stored_numpy
    w = case.workload
    qh = q.cpu()
    order = np.random.default_rng(12345).permutation(case.batch)
    spent, kv_bytes, done = 0.0, 0, []
    for b in order:
        q_st = stored_numpy(qh[b])
        k_st = stored_numpy(case.k[b])
        v_st = None if case.v is None else stored_numpy(case.v[b])
        t0 = time.perf_counter()
        qq = ofmt.decode(q_st, stored_format(qh))
        k = ofmt.decode_kv(k_st, stored_format(case.k[b]), case.k_scale)
        v = k[:, :, :w.head_dim_v] if v_st is None else ofmt.decode_kv(v_st, stored_format(case.v[b]), case.v_scale)
        oatt.verify_attention(qq, k, v, w.softmax_scale, case.sink)
        spent += time.perf_counter() - t0
        kv_bytes += int(case.seq_lens[b]) * w.kv_bytes_per_token()
        done.append(int(b))
        if spent >= budget_s:
            break
    return {
        "value": kv_bytes / spent / 1e9,
        "unit": "GB/s",
        "cores": int(blas_threads()),
        "kind": "oracle",
        "sample": (f"{len(done)} of {case.batch} requests ({q_len} query tokens each, seeded random order), "
                   f"causal attention per query token over the unsharded sequence in float64 incl. decoding the "
                   f"stored KV; {spent:.1f} s"),
        "verified_tokens_per_s": len(done) * q_len / spent,
    }


def bench_verify(args, vw):
    import numpy as np
    import torch
    import sequence_sharded_paged_amd as dcp
    from workloads.device import DeviceInputs, VerifyRun
    from workloads import make_case, make_verify_queries

    w = vw.geometry()
    t_gen = time.perf_counter()
    case = make_case(w, device="cuda")
    inp = DeviceInputs(case, "cuda", fill="zero")
    q = make_verify_queries(w, case.batch, vw.q_len, "cuda")
    run = VerifyRun(inp, q, algo=dcp.DCP_ALGO_AUTO)
    torch.cuda.synchronize()
    t_gen = time.perf_counter() - t_gen
    print(f"[bench] {vw.name}: batch {case.batch} x {vw.q_len} query tokens, {int(case.seq_lens.sum())} tokens, "
          f"{case.kv_bytes() / 1e9:.3f} GB KV, inputs ready in {t_gen:.1f} s", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        run.step()
    torch.cuda.synchronize()
    ms, kern_avg_ms = timed_steps(run.step, args.steps)
    kv_bytes = case.kv_bytes()
    family = kernel_family(w)
    out = {
        "metric": VERIFY_METRIC,
        "value": round(kv_bytes / (ms * 1e-3) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": DTYPE_DESC[w.kv_format],
        "data": "synthetic",
        "config": {
            "workload": vw.name,
            "base": w.name,
            "q_len": vw.q_len,
            "batch": case.batch,
            "num_q_heads": w.num_q_heads,
            "num_kv_heads": w.num_kv_heads,
            "kv_format": w.kv_format,
            "dcp_size": w.dcp_size,
            "interleave": w.interleave,
            "tokens": int(case.seq_lens.astype(np.int64).sum()),
            "kv_bytes": int(kv_bytes),
            "pct_hbm_peak": round(100.0 * kv_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
            "verified_tokens_per_s": round(case.batch * vw.q_len / (ms * 1e-3), 1),
            "kernel": KERNEL_NAMES[family],
        },
        "roofline": attn_roofline(kv_bytes, verify_flops(w, case.seq_lens, vw.q_len), kern_avg_ms,
                                  load_traffic(family, vw.name)),
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_verify(case, q, vw.q_len, args.cpu_budget_s)
    print(json.dumps(out), flush=True)


def bench_segment(args, sw):
    import numpy as np
    import torch
    import sequence_sharded_paged_amd as dcp
    from workloads.device import DeviceInputs, SegmentInputs
    from workloads import make_case, make_segment

    w = sw.geometry()
    t_gen = time.perf_counter()
    case = make_case(w, device="cuda")
    inp = DeviceInputs(case, "cuda", fill="zero")
    seg = make_segment(w, case.seq_lens, sw.window, case.k_scale, case.v_scale, "cuda")
    sgi = SegmentInputs(inp, seg, "cuda")
    inp.prepare(algo=dcp.DCP_ALGO_AUTO)
    torch.cuda.synchronize()
    t_gen = time.perf_counter() - t_gen
    seg_bytes = int(seg.lens.astype(np.int64).sum()) * w.kv_bytes_per_token()
    kv_bytes = case.kv_bytes() + seg_bytes
    print(f"[bench] {sw.name}: batch {case.batch}, {int(case.seq_lens.sum())} sharded + {int(seg.lens.sum())} "
          f"segment tokens, {kv_bytes / 1e9:.3f} GB KV, inputs ready in {t_gen:.1f} s", file=sys.stderr, flush=True)

    def step():
        inp.partial()
        sgi.fold(sw.seg_rank)
        inp.merge()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ms, kern_avg_ms = timed_steps(step, args.steps)
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    # the segment call alone (its attention over the segments and the fold)
    start.record()
    for _ in range(args.steps):
        sgi.fold(sw.seg_rank)
    stop.record()
    torch.cuda.synchronize()
    seg_ms = start.elapsed_time(stop) / args.steps
    family = kernel_family(w)
    out = {
        "metric": SEGMENT_METRIC,
        "value": round(kv_bytes / (ms * 1e-3) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": DTYPE_DESC[w.kv_format],
        "data": "synthetic",
        "config": {
            "workload": sw.name,
            "base": w.name,
            "window": sw.window,
            "seg_rank": sw.seg_rank,
            "batch": case.batch,
            "kv_format": w.kv_format,
            "dcp_size": w.dcp_size,
            "interleave": w.interleave,
            "tokens": int(case.seq_lens.astype(np.int64).sum()),
            "segment_tokens": int(seg.lens.astype(np.int64).sum()),
            "kv_bytes": int(kv_bytes),
            "pct_hbm_peak": round(100.0 * kv_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
            "merged_queries_per_s": round(case.batch / (ms * 1e-3), 1),
            "segment_call_ms": round(seg_ms, 5),
            "kernel": KERNEL_NAMES[family],
        },
        "roofline": dict(attn_roofline(case.kv_bytes(), step_flops(w, int(case.seq_lens.astype(np.int64).sum())),
                                       kern_avg_ms, None),
                         note="the sharded attention kernel (the segment call is timed separately in config)"),
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_segment(case, seg, sw, args.cpu_budget_s)
    print(json.dumps(out), flush=True)


def cpu_baseline_segment(case, seg, sw, budget_s):
    """Time the float64 oracle (attention over each request's sequence and segment) on a sample."""
    import numpy as np
    from oracle import attention as oatt
    from oracle import formats as ofmt
    from workloads.generate import stored_format, stored_numpy
    w = case.workload
    order = np.random.default_rng(12345).permutation(case.batch)
    spent, kv_bytes, done = 0.0, 0, []
    for b in order:
        q_st = stored_numpy(case.q[b])
        arrs = [(stored_numpy(t), stored_format(t)) for t in (case.k[b], seg.k[b])]
        varrs = None if case.v is None else [(stored_numpy(t), stored_format(t)) for t in (case.v[b], seg.v[b])]
        t0 = time.perf_counter()
        q = ofmt.decode(q_st, stored_format(case.q))
        k = np.concatenate([ofmt.decode_kv(a, f, case.k_scale) for a, f in arrs])
        v = k[:, :, :w.head_dim_v] if varrs is None else np.concatenate(
            [ofmt.decode_kv(a, f, case.v_scale) for a, f in varrs])
        oatt.decode_attention(q, k, v, w.softmax_scale, case.sink)
        spent += time.perf_counter() - t0
        kv_bytes += (int(case.seq_lens[b]) + int(seg.lens[b])) * w.kv_bytes_per_token()
        done.append(int(b))
        if spent >= budget_s:
            break
    return {
        "value": kv_bytes / spent / 1e9,
        "unit": "GB/s",
        "cores": int(blas_threads()),
        "kind": "oracle",
        "sample": (f"{len(done)} of {case.batch} requests (seeded random order), full softmax over the sequence "
                   f"and its {sw.window}-token segment in float64 incl. decoding the stored KV; {spent:.1f} s"),
    }


def bench_gather(args, name):
    import numpy as np
    import torch
    import sequence_sharded_paged_amd as dcp
    from workloads.device import DeviceInputs
    from workloads import get_workload, make_case

    w = get_workload(name[len("gather_"):])
    if not w.mla:
        print("the context gather is measured on MLA caches (a GQA cache keeps V transposed inside a block)",
              file=sys.stderr)
        sys.exit(2)
    case = make_case(w, device="cuda")
    inp = DeviceInputs(case, "cuda", fill="zero")
    ctx = case.seq_lens.astype(np.int64)
    cu = torch.from_numpy(np.concatenate([[0], np.cumsum(ctx)]).astype(np.int64)).cuda()
    T = int(ctx.sum())
    out = torch.empty((T, w.num_kv_heads, w.head_dim_k), dtype=inp.cache.dtype, device="cuda")
    kv = inp.cache.descriptor(0)
    torch.cuda.synchronize()
    print(f"[bench] {name}: {case.batch} requests, {T} context tokens, {case.kv_bytes() / 1e9:.3f} GB gathered",
          file=sys.stderr, flush=True)

    def step():
        dcp.dcp_gather_context(kv, inp.D, inp.I, inp.block_table, cu, T, out)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(args.steps):
        step()
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / args.steps
    nbytes = 2 * case.kv_bytes()  # every stored row read once and written once
    gbs = nbytes / (ms * 1e-3) / 1e9
    out_line = {
        "metric": GATHER_METRIC,
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": f"{w.kv_format} (stored bits copied)",
        "data": "synthetic",
        "config": {"workload": name, "base": w.name, "requests": case.batch, "tokens": T,
                   "bytes_per_token": 2 * w.kv_bytes_per_token(), "kernel": "gather_context_kernel",
                   "tokens_per_s": round(T / (ms * 1e-3), 1)},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": load_traffic("gather", name),
                     "kernel_avg_ms": round(ms, 5)},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        out_line["cpu_baseline"] = cpu_baseline_gather(inp, case, args.cpu_budget_s)
    print(json.dumps(out_line), flush=True)


def cpu_baseline_gather(inp, case, budget_s):
    """Time the oracle's gather on whole requests of the same pools (copied to the host)."""
    import numpy as np
    import torch
    from oracle import gather as ogather
    w = case.workload
    kp = inp.cache.k.view(torch.int16).cpu().numpy()
    order = np.random.default_rng(12345).permutation(case.batch)
    spent, nbytes, done = 0.0, 0, []
    for b in order:
        ctx = np.zeros(case.batch, dtype=np.int64)
        ctx[b] = int(case.seq_lens[b])
        t0 = time.perf_counter()
        ogather.gather_context(kp, None, inp.block_table_np, ctx, inp.bs, inp.D, inp.I)
        spent += time.perf_counter() - t0
        nbytes += 2 * int(ctx[b]) * w.kv_bytes_per_token()
        done.append(int(b))
        if spent >= budget_s:
            break
    return {"value": nbytes / spent / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{len(done)} of {case.batch} requests gathered one at a time by the oracle; {spent:.1f} s"}


DTYPE_DESC = {
    "fp32": "f32 KV, fp32 arithmetic",
    "bf16": "bf16 KV, bf16 MFMA, fp32 accumulate",
    "fp8_e4m3": "fp8_e4m3 KV (widened exactly to bf16 MFMA operands, per-head scales), fp32 accumulate",
}
PER_CONFIG = ["gqa_bf16_32k", "mla_bf16_bimodal", "mla_bf16_longtail_sink", "gqa_fp8_binned"]
BF16_MFMA_PEAK_TFLOPS = 2500.0


def host_cores():
    """Host cores this process may run on, and the BLAS thread count."""
    try:
        aff = len(os.sched_getaffinity(0))
    except AttributeError:
        aff = os.cpu_count() or 1
    return aff, blas_threads()


def load_counters(family, workload):
    """MFMA-busy and fetched-bytes figures from the committed counter summary
    of this kernel and workload, if it was taken on the current source."""
    path = os.path.join(ROOT, "profiles", f"{KERNEL_NAMES[family]}_{workload}_counters.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_sha256_16") != source_hash(family):
        return None
    return {k: rec[k] for k in ("mfma_busy_frac", "lds_bank_conflict_cycles", "source_sha256_16") if k in rec}


def step_flops(w, tokens):
    """Algorithmic matrix flops of one decode step: QK^T and PV over every
    cached token, for every query head."""
    return 2 * tokens * w.num_q_heads * (w.head_dim_k + w.head_dim_v)


def attn_roofline(kv_bytes, flops, kern_avg_ms, traffic):
    """Roofline of an attention kernel launch against the bound its arithmetic
    intensity selects: the bf16 matrix peak when its flops per KV byte exceed
    the ridge (2.5 PFLOP/s / 8 TB/s = 312.5, e.g. MLA with several query
    tokens), else HBM. Both fractions are reported either way."""
    s = kern_avg_ms * 1e-3
    hbm = kv_bytes / s / 1e9
    tf = flops / s / 1e12
    ridge = BF16_MFMA_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
    mfma_bound = flops / max(kv_bytes, 1) > ridge
    r = {"bound": "mfma" if mfma_bound else "hbm",
         "achieved": round(tf if mfma_bound else hbm, 2),
         "peak": BF16_MFMA_PEAK_TFLOPS if mfma_bound else HBM_PEAK_GBS,
         "unit": "TFLOP/s" if mfma_bound else "GB/s",
         "frac": round((tf / BF16_MFMA_PEAK_TFLOPS) if mfma_bound else (hbm / HBM_PEAK_GBS), 4),
         "traffic": traffic,
         "kernel_avg_ms": round(kern_avg_ms, 5),
         "flop_per_kv_byte": round(flops / max(kv_bytes, 1), 1),
         "hbm_gbs": round(hbm, 2), "hbm_frac": round(hbm / HBM_PEAK_GBS, 4),
         "mfma_tflops": round(tf, 1), "mfma_frac": round(tf / BF16_MFMA_PEAK_TFLOPS, 4)}
    return r


def verify_flops(w, seq_lens, q_len):
    """Algorithmic matrix flops of one multi-token step: query token i of a
    request of length L sees L - q_len + i + 1 positions."""
    import numpy as np
    L = np.asarray(seq_lens, dtype=np.int64)
    seen = int((q_len * L - q_len * (q_len - 1) // 2).sum())
    return 2 * seen * w.num_q_heads * (w.head_dim_k + w.head_dim_v)


def step_bytes(w, case, out_elem):
    """Algorithmic HBM bytes of one decode step: the KV once, every rank's
    read of the queries, the rank partials written and read back (O and LSE,
    float32) and the merged output (O and LSE)."""
    B, Hq, Dk, Dv, D = case.batch, w.num_q_heads, w.head_dim_k, w.head_dim_v, w.dcp_size
    q_elem = 4 if w.q_format == "fp32" else 2
    kv = case.kv_bytes()
    q = D * B * Hq * Dk * q_elem
    parts = 2 * D * B * Hq * (Dv + 1) * 4
    final = B * Hq * (Dv * out_elem + 4)
    return {"kv": int(kv), "q_reads": int(q), "partials_write_read": int(parts), "final_out": int(final),
            "total": int(kv + q + parts + final)}


def measure_decode(w, steps, warmup, cpu_budget_s):
    """One decode workload: inputs resident in HBM, `steps` timed decode steps
    (all ranks' partials + merge), the attention kernel timed alone with the
    library's HIP events on its stream, and the oracle on a bounded sample."""
    import numpy as np
    import torch
    import sequence_sharded_paged_amd as dcp
    from workloads import make_case
    from workloads.device import DeviceInputs

    t_gen = time.perf_counter()
    case = make_case(w, device="cuda")
    inp = DeviceInputs(case, "cuda", fill="zero")
    inp.prepare(algo=dcp.DCP_ALGO_AUTO)
    torch.cuda.synchronize()
    t_gen = time.perf_counter() - t_gen
    print(f"[bench] {w.name}: batch {case.batch}, {int(case.seq_lens.sum())} tokens, "
          f"{case.kv_bytes() / 1e9:.3f} GB KV, inputs ready in {t_gen:.1f} s", file=sys.stderr, flush=True)
    for _ in range(warmup):
        inp.step()
    torch.cuda.synchronize()
    ms, kern_avg_ms = timed_steps(inp.step, steps)
    tokens = int(case.seq_lens.astype(np.int64).sum())
    kv_bytes = case.kv_bytes()
    family = kernel_family(w)
    out_elem = 2 if w.out_format == "bf16" else 4
    ab = step_bytes(w, case, out_elem)
    flops = step_flops(w, tokens)
    achieved = kv_bytes / (kern_avg_ms * 1e-3) / 1e9
    traffic = load_traffic(family, w.name)
    res = {
        "workload": w.name,
        "batch": case.batch,
        "tokens": tokens,
        "kv_format": w.kv_format,
        "dtype": DTYPE_DESC[w.kv_format],
        "kernel": KERNEL_NAMES[family],
        "ms_per_step": round(ms, 5),
        "kv_gbs": round(kv_bytes / (ms * 1e-3) / 1e9, 2),
        "pct_hbm_peak": round(100.0 * kv_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
        "merged_queries_per_s": round(case.batch / (ms * 1e-3), 1),
        "algorithmic_bytes": ab,
        "algorithmic_total_gbs": round(ab["total"] / (ms * 1e-3) / 1e9, 2),
        "step_overhead_ms": round(ms - kern_avg_ms, 5),
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "fetch_gbs": None if traffic is None else round(traffic / (kern_avg_ms * 1e-3) / 1e9, 2),
            "kernel_avg_ms": round(kern_avg_ms, 5),
            "mfma_tflops": round(flops / (kern_avg_ms * 1e-3) / 1e12, 1),
            "mfma_frac": round(flops / (kern_avg_ms * 1e-3) / 1e12 / BF16_MFMA_PEAK_TFLOPS, 4),
            "counters": load_counters(family, w.name),
        },
        "cpu_baseline": None,
    }
    if cpu_budget_s > 0:
        cb = cpu_baseline(case, cpu_budget_s)
        cb["speedup_gpu_over_oracle"] = round(res["kv_gbs"] / cb["value"], 1)
        res["cpu_baseline"] = cb
    del inp, case
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


def measure_read_ceiling(nbytes=8 << 30, reps=10):
    """The device's sustained streaming-read rate: dcp_hbm_read_probe over an
    `nbytes` buffer (far past the 256 MB last-level cache), 3 untimed reads,
    then `reps` timed with events. Taken first in the run, on a fresh
    allocation: a buffer allocated where freed pools were reads up to ≈5%
    slower."""
    import torch
    import sequence_sharded_paged_amd as dcp
    buf = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")  # (written once, as the KV pools are)
    digest = torch.empty(dcp.dcp_hbm_read_probe_blocks(), dtype=torch.int32, device="cuda")
    for _ in range(3):
        dcp.dcp_hbm_read_probe(buf, digest)
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for _ in range(reps):
        dcp.dcp_hbm_read_probe(buf, digest)
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / reps
    del buf, digest
    torch.cuda.empty_cache()
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"gbs": round(gbs, 2), "pct_hbm_peak": round(100.0 * gbs / HBM_PEAK_GBS, 2), "bytes": nbytes,
            "ms_per_read": round(ms, 4), "reads": reps, "kernel": "hbm_read_probe_kernel"}


def with_ceiling(roofline, ceiling_gbs):
    """The kernel's HBM rate also as a fraction of the measured read ceiling."""
    hbm = roofline.get("hbm_gbs", roofline["achieved"] if roofline.get("unit") == "GB/s" else None)
    if hbm is not None and ceiling_gbs:
        roofline["frac_of_read_ceiling"] = round(hbm / ceiling_gbs, 4)
    return roofline


def measure_layout(w, steps, cpu_budget_s):
    """The layout steps of the path on one workload's batch, timed apart from
    the decode step: local lengths and the slot mapping of one decode step's
    new tokens (one per request), and the slot mapping of the bulk fill (every
    cached token); the oracle's brute-force mapper on a sample of the same
    tokens."""
    import numpy as np
    import torch
    import sequence_sharded_paged_amd as dcp
    from workloads.generate import make_block_table, sample_lengths

    lens = sample_lengths(w)
    table, _ = make_block_table(w, lens, extra_vblocks=1)
    dev = "cuda"
    seq = torch.from_numpy(lens.astype(np.int32)).to(dev)
    bt = torch.from_numpy(table).to(dev)
    B, D = len(lens), w.dcp_size
    local = torch.empty((B, D), dtype=torch.int32, device=dev)
    dec_pos = torch.from_numpy(lens.astype(np.int64)).to(dev)            # the next token of every request
    dec_req = torch.arange(B, dtype=torch.int32, device=dev)
    dec_slots = torch.empty((D, B), dtype=torch.int64, device=dev)
    T = int(lens.astype(np.int64).sum())
    bulk_pos = torch.cat([torch.arange(int(L), dtype=torch.int64, device=dev) for L in lens])
    bulk_req = torch.repeat_interleave(torch.arange(B, dtype=torch.int32, device=dev),
                                       torch.from_numpy(lens.astype(np.int64)).to(dev))
    bulk_slots = torch.empty((D, T), dtype=torch.int64, device=dev)

    def timed(fn, n):
        fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(n):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n

    ms_local = timed(lambda: dcp.dcp_local_seq_lens(seq, w.block_size, D, w.interleave, out=local), steps)
    ms_dec = timed(lambda: dcp.dcp_slot_mapping(dec_pos, dec_req, bt, w.block_size, D, w.interleave,
                                                out=dec_slots), steps)
    ms_bulk = timed(lambda: dcp.dcp_slot_mapping(bulk_pos, bulk_req, bt, w.block_size, D, w.interleave,
                                                 out=bulk_slots), max(1, steps // 4))
    bulk_bytes = T * (8 + 4) + D * T * 8 + T * 4   # positions + request ids read, slots written, table entries
    res = {
        "workload": w.name,
        "local_seq_lens": {"requests": B, "us": round(ms_local * 1e3, 2),
                           "requests_per_s": round(B / (ms_local * 1e-3), 1)},
        "slot_mapping_decode": {"tokens": B, "us": round(ms_dec * 1e3, 2),
                                "tokens_per_s": round(B / (ms_dec * 1e-3), 1)},
        "slot_mapping_bulk": {"tokens": T, "ms": round(ms_bulk, 4), "tokens_per_s": round(T / (ms_bulk * 1e-3), 1),
                              "gbs": round(bulk_bytes / (ms_bulk * 1e-3) / 1e9, 2)},
        "cpu_baseline": None,
    }
    if cpu_budget_s > 0:
        from oracle import layout as olay
        pos_np, req_np = bulk_pos.cpu().numpy(), bulk_req.cpu().numpy()
        spent, done, chunk = 0.0, 0, 1 << 16
        while spent < cpu_budget_s and done < T:
            hi = min(T, done + chunk)
            t0 = time.perf_counter()
            olay.slot_mapping(pos_np[done:hi], req_np[done:hi], table, w.block_size, D, w.interleave)
            spent += time.perf_counter() - t0
            done = hi
        cores, blas = host_cores()
        res["cpu_baseline"] = {"value": round(done / spent, 1), "unit": "tokens/s", "cores": 1, "kind": "oracle",
                               "sample": f"brute-force mapper over the first {done} of the bulk fill's {T} tokens; "
                                         f"{spent:.1f} s", "host_cores": cores}
        res["slot_mapping_bulk"]["speedup_gpu_over_oracle"] = round(res["slot_mapping_bulk"]["tokens_per_s"] /
                                                                   res["cpu_baseline"]["value"], 1)
    del bulk_pos, bulk_req, bulk_slots
    torch.cuda.empty_cache()
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    # untimed steps before the timed ones: the first ~25 ms of sustained load
    # run at changing clocks (an MLA step settles from 2.9 ms to 1.8 ms over
    # its first 12 steps), so the default warms up past that
    ap.add_argument("--warmup", type=int, default=25)
    ap.add_argument("--workload", default=None,
                    help=f"one workload only (default: {DEFAULT_WORKLOAD} as the headline, plus the per-config block)")
    ap.add_argument("--cpu-budget-s", type=float, default=15.0)
    ap.add_argument("--per-config-cpu-budget-s", type=float, default=4.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-per-config", action="store_true")
    ap.add_argument("--calibrate-hbm", type=int, default=0, metavar="BYTES",
                    help="only run reference kernels for the HBM counters: a plain read (sum) of BYTES bytes "
                         "and a plain device copy of BYTES bytes, 5 times each")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus > 1 or world > 1:
        print("bench.py measures one GPU: the DCP ranks are virtual and all resident in one GPU's HBM; "
              "runs on more than one GPU are not part of this build.", file=sys.stderr)
        sys.exit(2)

    import torch
    from workloads import get_workload

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    if args.calibrate_hbm:
        src = torch.ones(args.calibrate_hbm // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        acc = torch.zeros((), dtype=torch.float32, device="cuda")
        for _ in range(5):
            acc += src.sum()        # reads BYTES, writes a scalar: reference for FETCH_SIZE
        for _ in range(5):
            dst.copy_(src)          # reads and writes BYTES: reference for WRITE_SIZE
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_hbm_bytes": args.calibrate_hbm, "reads": 5, "copies": 5,
                          "check": float(acc) / 5 / src.numel()}))
        return
    name = args.workload or DEFAULT_WORKLOAD
    if name.startswith("kvw_"):
        bench_kv_write(args, name)
        return
    if name.startswith("gather_"):
        bench_gather(args, name)
        return
    from workloads import SEGMENT_WORKLOADS, VERIFY_WORKLOADS
    if name in VERIFY_WORKLOADS:
        bench_verify(args, VERIFY_WORKLOADS[name])
        return
    if name in SEGMENT_WORKLOADS:
        bench_segment(args, SEGMENT_WORKLOADS[name])
        return
    w = get_workload(name)
    cpu = 0.0 if args.no_cpu_baseline else args.cpu_budget_s
    full_run = args.workload is None and not args.no_per_config
    ceiling = measure_read_ceiling() if full_run else None
    head = measure_decode(w, args.steps, args.warmup, cpu)
    cores, blas = host_cores()
    out = {
        "metric": METRIC,
        "value": head["kv_gbs"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": head["dtype"],
        "data": "synthetic",
        "config": {
            "workload": w.name,
            "batch": head["batch"],
            "num_q_heads": w.num_q_heads,
            "num_kv_heads": w.num_kv_heads,
            "head_dim_k": w.head_dim_k,
            "head_dim_v": w.head_dim_v,
            "kv_format": w.kv_format,
            "block_size": w.block_size,
            "dcp_size": w.dcp_size,
            "interleave": w.interleave,
            "tokens": head["tokens"],
            "kv_bytes": head["algorithmic_bytes"]["kv"],
            "pct_hbm_peak": head["pct_hbm_peak"],
            "merged_queries_per_s": head["merged_queries_per_s"],
            "algorithmic_bytes": head["algorithmic_bytes"],
            "algorithmic_total_gbs": head["algorithmic_total_gbs"],
            "step_overhead_ms": head["step_overhead_ms"],
            "kernel": head["kernel"],
        },
        "roofline": head["roofline"],
        "cpu_baseline": None,
    }
    if head["cpu_baseline"] is not None:
        cb = dict(head["cpu_baseline"])
        cb["cores"] = blas
        cb["host_cores"] = cores
        cb["blas_threads"] = blas
        out["cpu_baseline"] = cb
    if full_run:
        pc_cpu = 0.0 if args.no_cpu_baseline else args.per_config_cpu_budget_s
        per = {}
        for pname in PER_CONFIG:
            if pname == w.name:
                per[pname] = {k: v for k, v in head.items() if k != "cpu_baseline"}
                per[pname]["cpu_baseline"] = out["cpu_baseline"]
                continue
            pw = get_workload(pname)
            r = measure_decode(pw, max(5, args.steps // 2), args.warmup, pc_cpu)
            if r["cpu_baseline"] is not None:
                r["cpu_baseline"]["host_cores"] = cores
                r["cpu_baseline"]["blas_threads"] = blas
            per[pname] = r
            print(f"[bench] {pname}: step {r['ms_per_step']:.3f} ms, {r['kv_gbs']:.0f} GB/s "
                  f"({r['pct_hbm_peak']:.1f}%), kernel frac {r['roofline']['frac']:.3f}", file=sys.stderr, flush=True)
        out["per_config"] = per
        out["layout"] = measure_layout(w, 50, pc_cpu)
        out["hbm_read_ceiling"] = ceiling
        with_ceiling(out["roofline"], ceiling["gbs"])
        for r in per.values():
            with_ceiling(r["roofline"], ceiling["gbs"])
        print(f"[bench] streaming-read ceiling {ceiling['gbs']:.0f} GB/s ({ceiling['pct_hbm_peak']:.1f}% of the "
              f"8 TB/s peak); {w.name} kernel at {out['roofline'].get('frac_of_read_ceiling', 0) * 100:.1f}% of it",
              file=sys.stderr, flush=True)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
