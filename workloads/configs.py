"""The five synthetic decode workloads, the multi-token decode (speculative
verification) and replicated-segment workloads built on them, and the
KV-cache write workloads, named by what they are.

Length laws ("k" = 1024 tokens):
* ``loguniform(a, b)``: L = floor(exp(U(ln a, ln b))), clipped to [a, b];
* ``uniform(a, b)``: integer uniform on [a, b];
* mixtures: bin counts by largest remainder, then a seeded shuffle.
"""

from dataclasses import dataclass, field
import math

K = 1024


@dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim_k: int
    head_dim_v: int
    kv_format: str            # "fp32" | "bf16" | "fp8_e4m3"
    q_format: str             # "fp32" | "bf16"
    block_size: int
    dcp_size: int
    interleave: int
    # list of (count, law, a, b); law in {"fixed", "loguniform", "uniform"}
    lengths: tuple = ()
    mla: bool = False         # value = first head_dim_v entries of the key row
    sink: bool = False        # per-query-head sink logit ~ N(0, 1)
    out_format: str = "fp32"  # merged output format
    description: str = ""
    scale_override: float | None = None  # a test's softmax scale in place of 1 / sqrt(head_dim_k)

    @property
    def softmax_scale(self) -> float:
        if self.scale_override is not None:
            return self.scale_override
        return 1.0 / math.sqrt(self.head_dim_k)

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    def kv_bytes_per_token(self) -> int:
        elem = {"fp32": 4, "bf16": 2, "fp8_e4m3": 1}[self.kv_format]
        if self.mla:
            return self.num_kv_heads * self.head_dim_k * elem
        return self.num_kv_heads * (self.head_dim_k + self.head_dim_v) * elem


WORKLOADS = {
    w.name: w
    for w in [
        Workload(
            name="gqa_fp32_tiny", seed=1, batch=2, num_q_heads=8, num_kv_heads=2,
            head_dim_k=64, head_dim_v=64, kv_format="fp32", q_format="fp32",
            block_size=16, dcp_size=2, interleave=1,
            lengths=((1, "fixed", 37, 37), (1, "fixed", 100, 100)),
            description="tiny GQA decode, fp32, 2 requests of 37 and 100 tokens"),
        Workload(
            name="gqa_bf16_32k", seed=2, batch=32, num_q_heads=32, num_kv_heads=8,
            head_dim_k=128, head_dim_v=128, kv_format="bf16", q_format="bf16",
            block_size=16, dcp_size=4, interleave=1,
            lengths=((32, "loguniform", 1 * K, 32 * K),),
            out_format="bf16",
            description="GQA decode, bf16 KV, 32 requests log-uniform 1k-32k"),
        Workload(
            name="mla_bf16_bimodal", seed=3, batch=64, num_q_heads=128, num_kv_heads=1,
            head_dim_k=576, head_dim_v=512, kv_format="bf16", q_format="bf16",
            block_size=64, dcp_size=8, interleave=1,
            lengths=((30, "loguniform", 1 * K, 64 * K), (34, "loguniform", 64 * K, 256 * K)),
            mla=True, out_format="bf16",
            description="MLA latent decode, bf16, 64 requests, 47% 1k-64k / 53% 64k-256k"),
        Workload(
            name="mla_bf16_longtail_sink", seed=4, batch=4, num_q_heads=128, num_kv_heads=1,
            head_dim_k=576, head_dim_v=512, kv_format="bf16", q_format="bf16",
            block_size=64, dcp_size=8, interleave=64,
            lengths=((4, "uniform", 512 * K, 1024 * K),),
            mla=True, sink=True, out_format="bf16",
            description="MLA long-tail decode, bf16, 4 requests 512k-1M, attention sink"),
        Workload(
            name="gqa_fp8_binned", seed=5, batch=256, num_q_heads=64, num_kv_heads=8,
            head_dim_k=128, head_dim_v=128, kv_format="fp8_e4m3", q_format="bf16",
            block_size=64, dcp_size=8, interleave=64,
            lengths=((46, "loguniform", 1 * K, 8 * K), (74, "loguniform", 8 * K, 64 * K),
                     (115, "loguniform", 64 * K, 128 * K), (21, "loguniform", 128 * K, 256 * K)),
            out_format="bf16",
            description="GQA decode, fp8 e4m3 KV with per-head scales, 256 requests, binned 1k-256k"),
    ]
}


def get_workload(name: str) -> Workload:
    if name not in WORKLOADS:
        raise KeyError(f"unknown workload {name!r}; known: {sorted(WORKLOADS)}")
    return WORKLOADS[name]


@dataclass(frozen=True)
class KvWriteWorkload:
    """New tokens written into the pools of a decode workload's geometry:
    ``requests`` requests each append ``chunk`` consecutive tokens after an
    existing context of ``uniform(0, max_context)`` tokens (a chunked-prefill
    step; ``chunk = 1`` is a decode step)."""
    name: str
    seed: int
    base: str                 # decode workload giving format, heads, dims, block size, DCP layout
    requests: int
    chunk: int
    max_context: int
    src_format: str           # "fp32" | "bf16": format of the new rows
    description: str = ""

    @property
    def tokens(self) -> int:
        return self.requests * self.chunk

    def geometry(self) -> Workload:
        return WORKLOADS[self.base]

    def bytes_per_token(self) -> int:
        """Algorithmic HBM bytes per token: new rows read, one slot per rank
        read, stored rows written once (one owner)."""
        g = self.geometry()
        dims = g.head_dim_k if g.mla else g.head_dim_k + g.head_dim_v
        src = {"fp32": 4, "bf16": 2}[self.src_format]
        dst = {"fp32": 4, "bf16": 2, "fp8_e4m3": 1}[g.kv_format]
        return g.num_kv_heads * dims * (src + dst) + 8 * g.dcp_size


KV_WRITE_WORKLOADS = {
    w.name: w
    for w in [
        KvWriteWorkload(
            name="kvw_gqa_fp8_chunk", seed=11, base="gqa_fp8_binned", requests=32, chunk=2048,
            max_context=16 * K, src_format="bf16",
            description="GQA fp8 pools (8 KV heads x 128, per-head scales), 32 requests x 2048-token "
                        "prefill chunks, bf16 rows"),
        KvWriteWorkload(
            name="kvw_mla_bf16_chunk", seed=12, base="mla_bf16_bimodal", requests=32, chunk=2048,
            max_context=16 * K, src_format="bf16",
            description="MLA bf16 latent pools (1 x 576), 32 requests x 2048-token prefill chunks, bf16 rows"),
        KvWriteWorkload(
            name="kvw_gqa_fp8_decode", seed=13, base="gqa_fp8_binned", requests=256, chunk=1,
            max_context=256 * K, src_format="bf16",
            description="one decode step's writes: 256 requests x 1 new token into GQA fp8 pools"),
    ]
}


def get_kv_write_workload(name: str) -> KvWriteWorkload:
    if name not in KV_WRITE_WORKLOADS:
        raise KeyError(f"unknown KV-write workload {name!r}; known: {sorted(KV_WRITE_WORKLOADS)}")
    return KV_WRITE_WORKLOADS[name]


@dataclass(frozen=True)
class VerifyWorkload:
    """Multi-token decode on a decode workload's batch: the last ``q_len``
    tokens of every request are queried at once, causal among them (MTP /
    speculative verification of q_len - 1 draft tokens)."""
    name: str
    base: str
    q_len: int
    description: str = ""

    def geometry(self) -> Workload:
        return WORKLOADS[self.base]


VERIFY_WORKLOADS = {
    w.name: w
    for w in [
        VerifyWorkload(name="gqa_fp8_binned_q2", base="gqa_fp8_binned", q_len=2,
                       description="gqa_fp8_binned batch, 2 query tokens per request (one draft token)"),
        VerifyWorkload(name="gqa_bf16_32k_q4", base="gqa_bf16_32k", q_len=4,
                       description="gqa_bf16_32k batch, 4 query tokens per request (three draft tokens)"),
        VerifyWorkload(name="mla_bf16_bimodal_q2", base="mla_bf16_bimodal", q_len=2,
                       description="mla_bf16_bimodal batch, 2 query tokens per request (one draft token)"),
    ]
}


def get_verify_workload(name: str) -> VerifyWorkload:
    if name not in VERIFY_WORKLOADS:
        raise KeyError(f"unknown verify workload {name!r}; known: {sorted(VERIFY_WORKLOADS)}")
    return VERIFY_WORKLOADS[name]


@dataclass(frozen=True)
class SegmentWorkload:
    """Decode with a replicated segment: each request also attends a window of
    its last ``window`` tokens kept whole on every rank (a sliding-window
    cache, new rows drawn independently), counted by rank ``seg_rank``."""
    name: str
    base: str
    window: int
    seg_rank: int = 0
    description: str = ""

    def geometry(self) -> Workload:
        return WORKLOADS[self.base]


SEGMENT_WORKLOADS = {
    w.name: w
    for w in [
        SegmentWorkload(name="mla_bf16_longtail_sink_swa128", base="mla_bf16_longtail_sink", window=128,
                        description="mla_bf16_longtail_sink batch (attention sink) plus a replicated 128-token "
                                    "sliding window per request, counted on rank 0"),
        SegmentWorkload(name="gqa_fp8_binned_swa128", base="gqa_fp8_binned", window=128, seg_rank=7,
                        description="gqa_fp8_binned batch plus a replicated 128-token sliding window per request, "
                                    "counted on rank 7"),
    ]
}


def get_segment_workload(name: str) -> SegmentWorkload:
    if name not in SEGMENT_WORKLOADS:
        raise KeyError(f"unknown segment workload {name!r}; known: {sorted(SEGMENT_WORKLOADS)}")
    return SEGMENT_WORKLOADS[name]
