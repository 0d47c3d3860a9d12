"""Float64 decode attention: full softmax, per-rank partials, LSE merge.

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
  log-sum-exp.

Because sharding plus a log-sum-exp merge is an exact identity, the reference
result is plain softmax attention over the unsharded sequence. Readings where
the pages are silent:

* query head ``h`` uses KV head ``h // (Hq // Hkv)`` (contiguous groups);
* the softmax scale is an argument; LSE is a natural logarithm;
* the sink is a per-query-head logit in the same units as the scaled scores
  that joins the softmax denominator with a zero value vector;
* an empty token set gives O = 0 and LSE = -inf (LSE = sink with a sink);
* for MLA the value of a token is the first ``Dv`` entries of its stored key
  row (latent part), so the caller passes ``v = k[..., :Dv]``.
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
