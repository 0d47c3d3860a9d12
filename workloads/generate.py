"""Seeded generation of one decode batch in its stored formats.

Streams: ``numpy.random.SeedSequence(entropy=seed, spawn_key=(stream, i))``
with stream 0 = lengths, 1 = block permutation, 2 = q, 3 = K, 4 = V,
5 = fp8 scales and sinks, 6 = needles, 7 = KV-write contexts, 8 = the
queries of multi-token decode, 9 = replicated segments. K and V are drawn per request, in
canonical (request-contiguous) token order, with a torch generator on the
requested device, so large batches are produced in device memory; the stored
values are what both the oracle (after a copy to the host) and the GPU path
read.

Values: q, K, V ~ N(0, 1). bf16 is round-to-nearest-even from the float32
sample. fp8 e4m3 stores ``clamp(x / scale[h], -448, 448)`` rounded to nearest
even, with ``scale[h] = (6 / 448) * 2**U(0, 2)`` drawn per KV head for K and,
independently, for V (6 stands for the largest |x| expected from N(0, 1) at
these sizes; the random power of two makes every head's scale different).
Sinks ~ N(0, 1) per query head.

Block table: request b needs ``ceil(L_b / (block_size * dcp_size))`` virtual
blocks; physical block ids are a seeded random permutation of
``0..num_blocks-1`` handed out to (request, virtual block) in order; unused
entries hold -1.
"""

from dataclasses import dataclass
import math

import numpy as np
import torch

from .configs import KvWriteWorkload, Workload

LENGTHS, BLOCKPERM, QSTREAM, KSTREAM, VSTREAM, SCALES, NEEDLES, CONTEXT, VERIFYQ, SEGMENT = range(10)

TORCH_FORMAT = {"fp32": torch.float32, "bf16": torch.bfloat16, "fp8_e4m3": torch.float8_e4m3fn}


def _seed(seed: int, stream: int, index: int = 0) -> int:
    ss = np.random.SeedSequence(entropy=seed, spawn_key=(stream, index))
    return int(ss.generate_state(1, dtype=np.uint64)[0] & ((1 << 63) - 1))


def _rng(seed: int, stream: int, index: int = 0) -> np.random.Generator:
    return np.random.default_rng(_seed(seed, stream, index))


def sample_lengths(w: Workload) -> np.ndarray:
    rng = _rng(w.seed, LENGTHS)
    out = []
    for count, law, a, b in w.lengths:
        if law == "fixed":
            out += [a] * count
        elif law == "uniform":
            out += list(rng.integers(a, b + 1, size=count))
        elif law == "loguniform":
            x = np.exp(rng.uniform(math.log(a), math.log(b), size=count))
            out += list(np.clip(np.floor(x), a, b).astype(np.int64))
        else:
            raise ValueError(law)
    lens = np.asarray(out, dtype=np.int64)
    if len(w.lengths) > 1 and any(law != "fixed" for _, law, _, _ in w.lengths):
        lens = lens[rng.permutation(lens.shape[0])]
    return lens.astype(np.int32)


def make_block_table(w: Workload, seq_lens: np.ndarray, extra_vblocks: int = 0):
    span = w.block_size * w.dcp_size
    nvb = [(int(L) + span - 1) // span for L in seq_lens]
    num_blocks = int(sum(nvb))
    max_vb = max(nvb + [1]) + extra_vblocks
    perm = _rng(w.seed, BLOCKPERM).permutation(num_blocks).astype(np.int32)
    table = np.full((len(seq_lens), max_vb), -1, dtype=np.int32)
    pos = 0
    for b, n in enumerate(nvb):
        table[b, :n] = perm[pos:pos + n]
        pos += n
    return table, max(num_blocks, 1)


def _randn(shape, seed: int, device) -> torch.Tensor:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32)


def _scales(w: Workload, which: int) -> np.ndarray:
    rng = _rng(w.seed, SCALES, which)
    return ((6.0 / 448.0) * np.exp2(rng.uniform(0.0, 2.0, size=w.num_kv_heads))).astype(np.float32)


def _store(x: torch.Tensor, fmt: str, scale=None) -> torch.Tensor:
    if fmt == "fp8_e4m3":
        s = torch.as_tensor(scale, device=x.device).view(1, -1, 1)
        return (x / s).clamp_(-448.0, 448.0).to(torch.float8_e4m3fn)
    return x.to(TORCH_FORMAT[fmt])


@dataclass
class Case:
    workload: Workload
    seq_lens: np.ndarray          # [B] int32
    block_table: np.ndarray       # [B, max_vblocks] int32, -1 = unused
    num_blocks: int               # physical blocks per rank pool
    q: torch.Tensor               # [B, Hq, Dk] in q_format
    k: list                       # per request [L, Hkv, Dk] in kv_format
    v: list                       # per request [L, Hkv, Dv] in kv_format, or None (MLA)
    k_scale: np.ndarray           # [Hkv] float32 (fp8) or None
    v_scale: np.ndarray           # [Hkv] float32 (fp8) or None
    sink: np.ndarray              # [Hq] float32 or None

    @property
    def batch(self) -> int:
        return int(self.seq_lens.shape[0])

    def kv_bytes(self) -> int:
        return int(self.seq_lens.astype(np.int64).sum()) * self.workload.kv_bytes_per_token()


def make_case(w: Workload, device="cpu", seq_lens=None, extra_vblocks: int = 0,
              needles: int = 0, needle_logit: float = 20.0) -> Case:
    """Generate one batch. ``seq_lens`` overrides the workload's length law
    (used for reduced-size parity cases with the workload's geometry)."""
    lens = sample_lengths(w) if seq_lens is None else np.asarray(seq_lens, dtype=np.int32)
    B = lens.shape[0]
    table, num_blocks = make_block_table(w, lens, extra_vblocks)
    q32 = _randn((B, w.num_q_heads, w.head_dim_k), _seed(w.seed, QSTREAM), device)
    q = q32.to(TORCH_FORMAT[w.q_format])
    k_scale = _scales(w, 0) if w.kv_format == "fp8_e4m3" else None
    v_scale = _scales(w, 1) if w.kv_format == "fp8_e4m3" else None
    sink = _rng(w.seed, SCALES, 2).standard_normal(w.num_q_heads).astype(np.float32) if w.sink else None
    ks, vs = [], []
    for b in range(B):
        L = int(lens[b])
        kb = _randn((L, w.num_kv_heads, w.head_dim_k), _seed(w.seed, KSTREAM, b), device)
        vb = None
        if not w.mla:
            vb = _randn((L, w.num_kv_heads, w.head_dim_v), _seed(w.seed, VSTREAM, b), device)
        if needles and L > 0:
            _plant_needles(w, b, L, kb, q32[b], needles, needle_logit, lens)
        ks.append(_store(kb, w.kv_format, k_scale))
        vs.append(None if vb is None else _store(vb, w.kv_format, v_scale))
        del kb, vb
    return Case(w, lens, table, num_blocks, q, ks, None if w.mla else vs, k_scale, v_scale, sink)


def needle_positions(w: Workload, b: int, L: int, count: int) -> np.ndarray:
    """Seeded needle positions: ``count`` random ones plus the last token and
    the first token of the last (possibly partial) block-sized chunk."""
    rng = _rng(w.seed, NEEDLES, b)
    pos = list(rng.integers(0, L, size=count))
    pos += [L - 1, (L - 1) - ((L - 1) % w.block_size)]
    return np.unique(np.asarray(pos, dtype=np.int64))


def _plant_needles(w, b, L, kb, qb, count, logit, lens):
    """Overwrite a few key rows so one query head of the group scores them at
    about ``logit`` (before the fp8 scale), making the output of that head
    close to the needle's value row. For MLA, whose value is the latent part
    of the key, only the rope part of the key is set, so the value row keeps
    its N(0, 1) entries."""
    rng = _rng(w.seed, NEEDLES, 100000 + b)
    lo = w.head_dim_v if w.mla else 0
    for x in needle_positions(w, b, L, count):
        kv = int(rng.integers(0, w.num_kv_heads))
        h = kv * w.group + int(rng.integers(0, w.group))
        qh = qb[h, lo:].float()
        kb[int(x), kv, lo:] = qh * (logit / (w.softmax_scale * float(qh.norm()) ** 2))


def stored_numpy(t: torch.Tensor) -> np.ndarray:
    """Raw stored representation on the host: float32, uint16 (bf16 bits) or
    uint8 (fp8 codes)."""
    t = t.detach().cpu()
    if t.dtype == torch.float32:
        return t.numpy()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8).numpy()
    raise TypeError(t.dtype)


def stored_format(t: torch.Tensor) -> str:
    return {torch.float32: "fp32", torch.bfloat16: "bf16", torch.float8_e4m3fn: "fp8_e4m3"}[t.dtype]


@dataclass
class KvWriteCase:
    workload: KvWriteWorkload
    context: np.ndarray           # [requests] int64: tokens already in each request's cache
    positions: np.ndarray         # [T] int64, request-major: context[b] .. context[b] + chunk - 1
    req_indices: np.ndarray       # [T] int32
    block_table: np.ndarray       # [requests, max_vblocks] int32 covering context + chunk
    num_blocks: int               # physical blocks per rank pool
    k_new: torch.Tensor           # [T, Hkv, Dk] in src_format
    v_new: torch.Tensor           # [T, Hkv, Dv] in src_format, or None (MLA)
    k_scale: np.ndarray           # [Hkv] float32 (fp8 pools) or None
    v_scale: np.ndarray           # [Hkv] float32 (fp8 pools, GQA) or None


def make_kv_write_case(w: KvWriteWorkload, device="cpu") -> KvWriteCase:
    """Seeded new rows ~ N(0, 1) (rounded to ``src_format``) at the positions
    right after each request's context; the block table, scales and pool
    geometry follow the base decode workload's laws (stream 7 = contexts)."""
    g = w.geometry()
    ctx = _rng(w.seed, CONTEXT).integers(0, w.max_context + 1, size=w.requests).astype(np.int64)
    table, num_blocks = make_block_table(g, (ctx + w.chunk).astype(np.int64))
    positions = (ctx[:, None] + np.arange(w.chunk, dtype=np.int64)[None, :]).reshape(-1)
    reqs = np.repeat(np.arange(w.requests, dtype=np.int32), w.chunk)
    T = w.tokens
    src = TORCH_FORMAT[w.src_format]
    k_new = _randn((T, g.num_kv_heads, g.head_dim_k), _seed(w.seed, KSTREAM), device).to(src)
    v_new = None
    if not g.mla:
        v_new = _randn((T, g.num_kv_heads, g.head_dim_v), _seed(w.seed, VSTREAM), device).to(src)
    fp8 = g.kv_format == "fp8_e4m3"
    k_scale = _scales(g, 0) if fp8 else None
    v_scale = _scales(g, 1) if fp8 and not g.mla else None
    return KvWriteCase(w, ctx, positions, reqs, table, num_blocks, k_new, v_new, k_scale, v_scale)


def make_verify_queries(w: Workload, batch: int, q_len: int, device="cpu") -> torch.Tensor:
    """Seeded queries ``[batch, q_len, Hq, Dk]`` ~ N(0, 1) in ``q_format`` for
    multi-token decode of the last ``q_len`` tokens of each request."""
    q32 = _randn((batch, q_len, w.num_q_heads, w.head_dim_k), _seed(w.seed, VERIFYQ, q_len), device)
    return q32.to(TORCH_FORMAT[w.q_format])


@dataclass
class Segment:
    """A replicated segment per request (e.g. the sliding-window cache): its
    own tokens, stored in a one-rank paged pool of the workload's geometry."""
    lens: np.ndarray              # [B] int32: min(L_b, window)
    block_table: np.ndarray       # [B, max_vblocks] int32, -1 = unused
    num_blocks: int
    k: list                       # per request [lens_b, Hkv, Dk] in kv_format
    v: list                       # per request [lens_b, Hkv, Dv], or None (MLA)


def make_segment(w: Workload, seq_lens, window: int, k_scale=None, v_scale=None, device="cpu") -> Segment:
    """Seeded segment rows ~ N(0, 1) (stream 9), ``min(L_b, window)`` tokens per
    request, stored like the cache (same fp8 scales); block ids a seeded
    permutation handed out in request order."""
    lens = np.minimum(np.asarray(seq_lens, dtype=np.int64), window).astype(np.int32)
    nvb = [(int(L) + w.block_size - 1) // w.block_size for L in lens]
    nblk = max(1, int(sum(nvb)))
    perm = _rng(w.seed, SEGMENT).permutation(nblk).astype(np.int32)
    table = np.full((len(lens), max(nvb + [1])), -1, dtype=np.int32)
    pos = 0
    for b, n in enumerate(nvb):
        table[b, :n] = perm[pos:pos + n]
        pos += n
    ks, vs = [], []
    for b, L in enumerate(lens):
        kb = _randn((int(L), w.num_kv_heads, w.head_dim_k), _seed(w.seed, SEGMENT, 1 + 2 * b), device)
        ks.append(_store(kb, w.kv_format, k_scale))
        if not w.mla:
            vb = _randn((int(L), w.num_kv_heads, w.head_dim_v), _seed(w.seed, SEGMENT, 2 + 2 * b), device)
            vs.append(_store(vb, w.kv_format, v_scale))
    return Segment(lens, table, nblk, ks, None if w.mla else vs)
