"""Float64 decode attention: full softmax, per-rank partials, LSE merge, and
multi-token decode (speculative verification).

Test infrastructure: see the package docstring.

Sources:

* "Decode Context Parallel (DCP)" (vLLM Ascend design doc), section "Decode":
  each rank computes attention of the gathered query heads against its local
  KV shard and the partial outputs and LSE values are combined across the DCP
  group.
* "Efficient Decode Context Parallelism with vLLM for Long Context Workloads",
  section 1 (MLA keeps one latent KV vector shared by all query heads) and
  section 5.4 (GQA: query heads share their group's KV head).
* "DeepSeek V4.1 context parallelism", section "Decode computation": the
  attention sink is applied once, when the partial outputs are merged by
  log-sum-exp; decode and speculative (DSpark) verification share the decode
  path, each rank attending the pages it owns; a replicated segment (the
  sliding-window cache, section "Cache ownership": kept on every rank)
  contributes on one rank only.
* "Efficient Decode Context Parallelism with vLLM for Long Context Workloads",
  section 6 (MTP and speculative decoding on the DCP decode path).

Because sharding plus a log-sum-exp merge is an exact identity, the reference
result is plain softmax attention over the unsharded sequence. Readings where
the pages are silent:

* query head ``h`` uses KV head ``h // (Hq // Hkv)`` (contiguous groups);
* the softmax scale is an argument; LSE is a natural logarithm;
* the sink is a per-query-head logit in the same units as the scaled scores
  that joins the softmax denominator with a zero value vector;
* an empty token set gives O = 0 and LSE = -inf (LSE = sink with a sink);
* for MLA the value of a token is the first ``Dv`` entries of its stored key
  row (latent part), so the caller passes ``v = k[..., :Dv]``;
* multi-token decode: the ``q_len`` queried tokens are the last ``q_len``
  positions, already in the cache, and query ``i`` attends every position up
  to its own (``verify_attention``);
* a replicated segment is a separate set of KV entries that joins the
  attention of every query of its request (the reference is plain attention
  over the sharded sequence and the segment together); one designated rank
  adds it to its partial (``segment_rank_partials``).
"""

import numpy as np

NEG_INF = -np.inf


def decode_attention(q, k, v, scale: float, sink=None):
    """Full-softmax attention of one decode query per head, float64.

    q: ``[Hq, Dk]``; k: ``[L, Hkv, Dk]``; v: ``[L, Hkv, Dv]``; sink: ``[Hq]`` or
    None. Returns ``(O [Hq, Dv], LSE [Hq])``.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    Hq, Dk = q.shape
    L, Hkv, _ = k.shape
    Dv = v.shape[2]
    if Hq % Hkv != 0:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")
    G = Hq // Hkv
    out = np.zeros((Hq, Dv), dtype=np.float64)
    lse = np.full((Hq,), NEG_INF, dtype=np.float64)
    if L == 0 and sink is None:
        return out, lse
    for kv in range(Hkv):
        heads = slice(kv * G, (kv + 1) * G)
        kh = np.ascontiguousarray(k[:, kv, :])              # [L, Dk]
        vh = np.ascontiguousarray(v[:, kv, :])              # [L, Dv]
        s = (q[heads] @ kh.T) * scale                      # [G, L] scores
        m = s.max(axis=1) if L > 0 else np.full((G,), NEG_INF)
        if sink is not None:
            sk = np.asarray(sink, dtype=np.float64)[heads]
            m = np.maximum(m, sk)
        e = np.exp(s - m[:, None])                         # [G, L]
        z = e.sum(axis=1)
        if sink is not None:
            z = z + np.exp(sk - m)
        out[heads] = (e @ vh) / z[:, None]
        lse[heads] = m + np.log(z)
    return out, lse


def rank_partials(q, k, v, scale: float, owner, dcp_size: int):
    """Per-rank partial ``(O_r, LSE_r)`` over the tokens each rank owns.

    ``owner[L]`` is the owning rank of every token (from the brute-force
    mapper). No sink: the sink belongs to the merge only.
    Returns ``(O [D, Hq, Dv], LSE [D, Hq])``.
    """
    owner = np.asarray(owner)
    parts = [decode_attention(q, k[owner == r], v[owner == r], scale) for r in range(dcp_size)]
    return np.stack([p[0] for p in parts]), np.stack([p[1] for p in parts])


def verify_attention(q, k, v, scale: float, sink=None):
    """Multi-token decode (MTP / speculative verification), float64.

    The last ``q_len`` tokens of a sequence are queried at once; their keys
    and values are already in ``k [L, Hkv, Dk]`` / ``v [L, Hkv, Dv]``.
    Query ``i`` (``q[i]``, ``[Hq, Dk]``) sits at position ``L - q_len + i``
    and attends positions ``0 .. L - q_len + i`` (causal among the new
    tokens; the earlier context is seen in full). Returns
    ``(O [q_len, Hq, Dv], LSE [q_len, Hq])``.
    """
    q = np.asarray(q, dtype=np.float64)
    q_len, L = q.shape[0], k.shape[0]
    if q_len > L:
        raise ValueError("the queried tokens must be in the cache (q_len <= L)")
    res = [decode_attention(q[i], k[:L - q_len + i + 1], v[:L - q_len + i + 1], scale, sink) for i in range(q_len)]
    return np.stack([r[0] for r in res]), np.stack([r[1] for r in res])


def verify_rank_partials(q, k, v, scale: float, owner, dcp_size: int):
    """Per-rank partials of multi-token decode: for query ``i``, rank ``r``
    attends the tokens it owns at positions ``<= L - q_len + i``.
    Returns ``(O [D, q_len, Hq, Dv], LSE [D, q_len, Hq])``."""
    q = np.asarray(q, dtype=np.float64)
    owner = np.asarray(owner)
    q_len, L = q.shape[0], k.shape[0]
    os_, ls_ = [], []
    for i in range(q_len):
        seen = slice(0, L - q_len + i + 1)
        o, lse = rank_partials(q[i], k[seen], v[seen], scale, owner[seen], dcp_size)
        os_.append(o)
        ls_.append(lse)
    return np.stack(os_, axis=1), np.stack(ls_, axis=1)


def segment_rank_partials(q, k, v, scale: float, owner, dcp_size: int, k_seg, v_seg, seg_rank: int):
    """Per-rank partials when a replicated segment (its own tokens ``k_seg``,
    ``v_seg``, e.g. a sliding-window cache kept on every rank) joins the
    attention: rank ``seg_rank`` attends its owned tokens and the segment,
    every other rank only its owned tokens, so the merge counts the segment
    once. Returns ``(O [D, Hq, Dv], LSE [D, Hq])``."""
    owner = np.asarray(owner)
    out = []
    for r in range(dcp_size):
        kr, vr = k[owner == r], v[owner == r]
        if r == seg_rank:
            kr = np.concatenate([kr, k_seg], axis=0)
            vr = np.concatenate([vr, v_seg], axis=0)
        out.append(decode_attention(q, kr, vr, scale))
    return np.stack([o for o, _ in out]), np.stack([l for _, l in out])


def lse_merge(part_o, part_lse, sink=None):
    """Merge partials ``(O_r [R, H, Dv], LSE_r [R, H])`` into ``(O [H, Dv], LSE [H])``.

    M = max(max_r LSE_r, sink); Z = sum_r exp(LSE_r - M) + exp(sink - M);
    LSE = M + ln Z; O = sum_r exp(LSE_r - LSE) O_r. The sink enters once.
    All parts empty and no sink: O = 0, LSE = -inf.
    """
    part_o = np.asarray(part_o, dtype=np.float64)
    part_lse = np.asarray(part_lse, dtype=np.float64)
    R, H, Dv = part_o.shape
    out = np.zeros((H, Dv), dtype=np.float64)
    lse = np.full((H,), NEG_INF, dtype=np.float64)
    for h in range(H):
        terms = [float(x) for x in part_lse[:, h]]
        if sink is not None:
            terms.append(float(sink[h]))
        m = max(terms)
        if m == NEG_INF:
            continue
        z = sum(np.exp(t - m) for t in terms)
        lse[h] = m + np.log(z)
        for r in range(R):
            if part_lse[r, h] != NEG_INF:
                out[h] += np.exp(part_lse[r, h] - lse[h]) * part_o[r, h]
    return out, lse
